// C ABI of the GenRank hot path: host-side argument checks, workspace layout, and the
// composition of kernels into a block forward / backward.  Every entry point validates
// its arguments before enqueuing anything and returns a genrank_status.
#include <hip/hip_runtime.h>
#include <algorithm>
#include <math.h>
#include <string.h>

#include "genrank.h"
#include "internal.hpp"

namespace genrank {

genrank_status check_batch(const genrank_batch* b) {
  if (!b) return GENRANK_E_ARG;
  if (b->B < 1 || b->m < 0 || b->d < 1 || b->H < 1 || b->dh < 1 || b->max_hist < 0 ||
      b->total_hist < 0)
    return GENRANK_E_ARG;
  if (b->H > GENRANK_MAX_HEADS) return GENRANK_E_SHAPE;
  if (static_cast<int64_t>(b->H) * b->dh != b->d) return GENRANK_E_SHAPE;
  if (b->dtype != GENRANK_F32 && b->dtype != GENRANK_BF16) return GENRANK_E_DTYPE;
  if (b->resid != GENRANK_RESID_ACT && b->resid != GENRANK_RESID_F32) return GENRANK_E_DTYPE;
  if (b->total_hist > static_cast<int64_t>(b->max_hist) * b->B) return GENRANK_E_SHAPE;
  const int64_t T = b->total_hist + static_cast<int64_t>(b->B) * b->m;
  if (T >= (int64_t(1) << 31)) return GENRANK_E_SHAPE;
  return GENRANK_OK;
}

size_t dtype_size(int dtype) { return dtype == GENRANK_BF16 ? 2 : 4; }

int resid_dtype(const genrank_batch* b) { return b->resid == GENRANK_RESID_F32 ? GENRANK_F32 : b->dtype; }

namespace {

inline hipStream_t S(genrank_stream_t s) { return reinterpret_cast<hipStream_t>(s); }

inline size_t align_up(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

inline int64_t rows_of(const genrank_batch* b) {
  return b->total_hist + static_cast<int64_t>(b->B) * b->m;
}

// Activations kept by the block forward, in this order, each 256-byte aligned.
struct LayerFwdWs {
  char* z;    // [T, d]   rmsnorm(x) g1          (PRENORM)
  char* qkv;  // [T, 3d]
  char* o;    // [T, d]   attention output
  float* lse; // [T, H]
  char* x1;   // [T, d]   x + attention branch   (PRENORM; in the residual stream's type)
  char* z2;   // [T, d]   rmsnorm(x1) g2         (PRENORM)
  char* a;    // [T, f]   FFN pre-activation     (PRENORM)
  char* hdn;  // [T, f]   silu(a)                (PRENORM)
  char* wg;   // [max(3d, f), d] a weight with the RMSNorm gain folded in (PRENORM, fused path)
  size_t bytes;
};

LayerFwdWs layer_fwd_layout(const genrank_batch* b, int block, int ffn, char* base) {
  const size_t T = static_cast<size_t>(rows_of(b));
  const size_t es = dtype_size(b->dtype);
  const size_t d = b->d;
  const bool pre = block == GENRANK_BLOCK_PRENORM;
  LayerFwdWs w{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off += align_up(bytes);
    return p;
  };
  w.z = pre ? take(T * d * es) : nullptr;
  w.qkv = take(T * 3 * d * es);
  w.o = take(T * d * es);
  w.lse = reinterpret_cast<float*>(take(T * b->H * sizeof(float)));
  w.x1 = pre ? take(T * d * dtype_size(resid_dtype(b))) : nullptr;
  w.z2 = pre ? take(T * d * es) : nullptr;
  w.a = pre ? take(T * static_cast<size_t>(ffn) * es) : nullptr;
  w.hdn = pre ? take(T * static_cast<size_t>(ffn) * es) : nullptr;
  w.wg = pre ? take(std::max(3 * d, static_cast<size_t>(ffn)) * d * es) : nullptr;
  w.bytes = off;
  return w;
}

// The pre-norm block's RMSNorm goes into the GEMMs that read its output (the norm's scale
// applied to the GEMM rows, its gain folded into the weight) when every such GEMM fits the
// fused kernel.  The choice depends on the widths only, so the full forward, the history
// key/value projection and the candidate-only forward take the same arithmetic for a row.
// A forward that saves activations for the backward keeps the normalised rows.
bool rms_fused(const genrank_batch* b, const genrank_layer_weights* w) {
  const int d = b->d;
  return w->block == GENRANK_BLOCK_PRENORM && b->dtype == GENRANK_BF16 && b->resid == GENRANK_RESID_ACT &&
         gemm_rms_ok(3 * d, d) &&
         gemm_rms_ok(2 * d, d) && gemm_rms_ok(w->ffn_dim, d);
}

struct LayerBwdWs {
  char* dqkv;   // [T, 3d]
  char* dout;   // [T, d]  gradient of the attention output
  char* dz;     // [T, d]  gradient of the QKV input
  char* dx1;    // [T, d]  (PRENORM)
  char* dh;     // [T, f]  (PRENORM) gradient of silu(a), then of a
  char* dz2;    // [T, d]  (PRENORM)
  char* attn;   // attention backward scratch
  char* rms;    // RMSNorm backward partial rows
  char* wt;     // one transposed weight (bf16 data gradients)
  char* tn;     // split partial tiles of the weight gradients
  size_t tn_bytes;
  size_t bytes;
};

LayerBwdWs layer_bwd_layout(const genrank_batch* b, int block, int ffn, char* base) {
  const size_t T = static_cast<size_t>(rows_of(b));
  const size_t es = dtype_size(b->dtype);
  const size_t d = b->d;
  const bool pre = block == GENRANK_BLOCK_PRENORM;
  LayerBwdWs w{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off += align_up(bytes);
    return p;
  };
  w.dqkv = take(T * 3 * d * es);
  w.dout = take(T * d * es);
  w.dz = take(T * d * es);
  w.dx1 = pre ? take(T * d * es) : nullptr;
  w.dh = pre ? take(T * static_cast<size_t>(ffn) * es) : nullptr;
  w.dz2 = pre ? take(T * d * es) : nullptr;
  w.attn = take(attn_bwd_workspace(b));
  const int64_t Ti = static_cast<int64_t>(T);
  const int di = static_cast<int>(d);
  size_t wt = 3 * d * d, tn = std::max(gemm_tn_workspace(3 * di, di, Ti), gemm_tn_workspace(di, di, Ti));
  if (pre) {
    wt = std::max(wt, d * static_cast<size_t>(ffn));
    tn = std::max({tn, gemm_tn_workspace(di, ffn, Ti), gemm_tn_workspace(ffn, di, Ti)});
  }
  w.rms = take(rmsnorm_bwd_workspace(di));
  w.wt = take(wt * es);
  w.tn = take(tn);
  w.tn_bytes = tn;
  w.bytes = off;
  return w;
}

genrank_status check_layer_weights(const genrank_batch* b, const genrank_layer_weights* w) {
  if (!w || !w->wqkv || !w->wo || !w->alibi.slopes_pos || !w->alibi.slopes_time)
    return GENRANK_E_ARG;
  if (w->block == GENRANK_BLOCK_PRENORM) {
    if (!w->w1 || !w->w2 || !w->g1 || !w->g2) return GENRANK_E_ARG;
    if (w->ffn_dim < 1 || w->ffn_dim % 64 != 0) return GENRANK_E_SHAPE;
  } else if (w->block != GENRANK_BLOCK_ATTN_ONLY) {
    return GENRANK_E_ARG;
  }
  if (b->d % 64 != 0 && b->dtype == GENRANK_BF16) return GENRANK_E_SHAPE;
  if (resid_dtype(b) != b->dtype && w->block != GENRANK_BLOCK_PRENORM) return GENRANK_E_DTYPE;
  return check_alibi_variant(w->alibi, b->H);
}

#define GR_TRY(expr)                         \
  do {                                       \
    genrank_status _s = (expr);              \
    if (_s != GENRANK_OK) return _s;         \
  } while (0)

}  // namespace
}  // namespace genrank

using namespace genrank;

extern "C" {

const char* genrank_status_string(int s) {
  switch (s) {
    case GENRANK_OK: return "GENRANK_OK";
    case GENRANK_E_ARG: return "GENRANK_E_ARG: invalid argument";
    case GENRANK_E_SHAPE: return "GENRANK_E_SHAPE: unsupported or inconsistent shape";
    case GENRANK_E_DTYPE: return "GENRANK_E_DTYPE: unsupported dtype";
    case GENRANK_E_UNSORTED: return "GENRANK_E_UNSORTED: offsets or timestamps out of order";
    case GENRANK_E_RANGE: return "GENRANK_E_RANGE: id or time difference out of range";
    case GENRANK_E_WORKSPACE: return "GENRANK_E_WORKSPACE: workspace missing or too small";
    case GENRANK_E_HIP: return "GENRANK_E_HIP: HIP runtime or launch failure";
    default: return "GENRANK: unknown status";
  }
}

int32_t genrank_version(void) { return (GENRANK_VERSION_MAJOR << 16) | GENRANK_VERSION_MINOR; }

// ---------------------------------------------------------------- serving with cached history
namespace genrank {
namespace {
// the candidate rows of a batch as a batch of their own (no history rows)
genrank_batch cand_rows_batch(const genrank_batch* b) {
  genrank_batch c = *b;
  c.total_hist = 0;
  c.max_hist = 0;
  return c;
}
genrank_status check_cached_attn(const genrank_batch* b, const void* q, const void* k, const void* v,
                                 int64_t ld_c, const void* kh, const void* vh, int64_t ld_h, const void* o,
                                 int64_t ld_o) {
  if (b->dtype != GENRANK_BF16) return GENRANK_E_DTYPE;
  if (b->dh != 64) return GENRANK_E_SHAPE;
  if (ld_c < b->d || ld_h < b->d || ld_o < b->d || ld_c % 8 || ld_h % 8 || ld_o % 4) return GENRANK_E_SHAPE;
  if ((static_cast<int64_t>(b->max_hist) + 64) * ld_h * 2 >= (int64_t{1} << 31)) return GENRANK_E_SHAPE;
  auto al = [](const void* p, uintptr_t n) { return reinterpret_cast<uintptr_t>(p) % n == 0; };
  if (!al(q, 16) || !al(k, 16) || !al(v, 16) || !al(kh, 16) || !al(vh, 16) || !al(o, 8)) return GENRANK_E_ARG;
  return GENRANK_OK;
}
size_t layer_kv_bytes(const genrank_batch* b, const genrank_layer_weights* w) {
  const size_t es = dtype_size(b->dtype), d = b->d;
  return w->block == GENRANK_BLOCK_PRENORM
             ? align_up(static_cast<size_t>(b->total_hist) * d * es) + align_up(2 * d * d * es)
             : 0;
}
size_t layer_fwd_cached_bytes(const genrank_batch* b, const genrank_layer_weights* w) {
  const genrank_batch c = cand_rows_batch(b);
  return layer_fwd_layout(&c, w->block, w->block == GENRANK_BLOCK_PRENORM ? w->ffn_dim : 0, nullptr).bytes;
}
}  // namespace
}  // namespace genrank

genrank_status genrank_workspace_size(int32_t op, const genrank_batch* b,
                                      const genrank_layer_weights* w, size_t* bytes) {
  if (!b || !bytes) return GENRANK_E_ARG;
  GR_TRY(check_batch(b));
  switch (op) {
    case GENRANK_OP_EMBED_SUM:
    case GENRANK_OP_ATTN_FWD:
      *bytes = 0;
      return GENRANK_OK;
    case GENRANK_OP_ATTN_BWD:
      *bytes = attn_bwd_workspace(b);
      return GENRANK_OK;
    case GENRANK_OP_EMBED_BWD:
      *bytes = embed_bwd_workspace(b);
      return GENRANK_OK;
    case GENRANK_OP_HEAD_BWD:
      *bytes = head_bwd_workspace(b->d, 4);
      return GENRANK_OK;
    case GENRANK_OP_LAYER_KV:
    case GENRANK_OP_LAYER_FWD_CACHED:
      if (!w) return GENRANK_E_ARG;
      *bytes = op == GENRANK_OP_LAYER_KV ? layer_kv_bytes(b, w) : layer_fwd_cached_bytes(b, w);
      return GENRANK_OK;
    case GENRANK_OP_LAYER_FWD:
    case GENRANK_OP_LAYER_BWD: {
      if (!w) return GENRANK_E_ARG;
      const int block = w->block;
      const int ffn = block == GENRANK_BLOCK_PRENORM ? w->ffn_dim : 0;
      *bytes = (op == GENRANK_OP_LAYER_FWD) ? layer_fwd_layout(b, block, ffn, nullptr).bytes
                                            : layer_bwd_layout(b, block, ffn, nullptr).bytes;
      return GENRANK_OK;
    }
    default:
      return GENRANK_E_ARG;
  }
}

genrank_status genrank_error_word(uint32_t* word, int32_t clear, genrank_stream_t stream) {
  if (!word) return GENRANK_E_ARG;
  uint32_t* dev = device_error_word();
  if (!dev) return GENRANK_E_HIP;
  if (hipStreamSynchronize(S(stream)) != hipSuccess) return GENRANK_E_HIP;
  if (hipMemcpy(word, dev, sizeof(uint32_t), hipMemcpyDeviceToHost) != hipSuccess) return GENRANK_E_HIP;
  if (clear) {
    const uint32_t zero = 0;
    if (hipMemcpy(dev, &zero, sizeof(uint32_t), hipMemcpyHostToDevice) != hipSuccess) return GENRANK_E_HIP;
  }
  return GENRANK_OK;
}

genrank_status genrank_validate_host(const genrank_batch* b, const genrank_inputs* in,
                                     const genrank_tables* t, int64_t* bad_row) {
  if (bad_row) *bad_row = -1;
  if (!b || !in || !t) return GENRANK_E_ARG;
  GR_TRY(check_batch(b));
  if (!in->hist_offsets || !in->req_ts) return GENRANK_E_ARG;
  const int32_t* off = in->hist_offsets;
  auto bad = [&](int64_t r, genrank_status s) {
    if (bad_row) *bad_row = r;
    return s;
  };
  if (off[0] != 0) return bad(0, GENRANK_E_UNSORTED);
  int32_t mx = 0;
  for (int u = 0; u < b->B; ++u) {
    if (off[u + 1] < off[u]) return bad(u, GENRANK_E_UNSORTED);
    mx = off[u + 1] - off[u] > mx ? off[u + 1] - off[u] : mx;
  }
  if (off[b->B] != b->total_hist || mx > b->max_hist) return bad(-1, GENRANK_E_SHAPE);
  if (b->total_hist > 0 && (!in->hist_items || !in->hist_actions || !in->hist_ts))
    return GENRANK_E_ARG;
  if (b->m > 0 && !in->cand_items) return GENRANK_E_ARG;
  for (int k = 1; k + 1 < t->n_rt; ++k)
    if (t->rt_bounds[k] < t->rt_bounds[k - 1]) return bad(k, GENRANK_E_UNSORTED);
  for (int u = 0; u < b->B; ++u) {
    const int64_t a = off[u], e = off[u + 1];
    for (int64_t r = a; r < e; ++r) {
      if (r > a && in->hist_ts[r] < in->hist_ts[r - 1]) return bad(r, GENRANK_E_UNSORTED);
      if (in->hist_items[r] < 0 || in->hist_items[r] >= t->n_item) return bad(r, GENRANK_E_RANGE);
      if (in->hist_actions[r] < 0 || in->hist_actions[r] >= t->n_action)
        return bad(r, GENRANK_E_RANGE);
    }
    if (e > a) {
      if (in->req_ts[u] <= in->hist_ts[e - 1]) return bad(e - 1, GENRANK_E_UNSORTED);
      if (in->req_ts[u] - in->hist_ts[a] >= (int64_t(1) << 24)) return bad(a, GENRANK_E_RANGE);
    }
    for (int k = 0; k < b->m; ++k) {
      const int32_t it = in->cand_items[static_cast<int64_t>(u) * b->m + k];
      if (it < 0 || it >= t->n_item) return bad(b->total_hist + static_cast<int64_t>(u) * b->m + k, GENRANK_E_RANGE);
    }
  }
  return GENRANK_OK;
}

genrank_status genrank_embed_sum(const genrank_batch* b, const genrank_inputs* in,
                                 const genrank_tables* t, void* x_out, genrank_stream_t stream) {
  GR_TRY(check_embed_args(b, in, t));
  if (!x_out) return GENRANK_E_ARG;
  return launch_embed_sum(b, in, t, x_out, S(stream));
}

genrank_status genrank_debug_indices(const genrank_batch* b, const genrank_inputs* in,
                                     const genrank_tables* t, int32_t* out,
                                     genrank_stream_t stream) {
  GR_TRY(check_embed_args(b, in, t));
  if (!out) return GENRANK_E_ARG;
  return launch_debug_indices(b, in, t, out, S(stream));
}

genrank_status genrank_embed_bwd(const genrank_batch* b, const genrank_inputs* in,
                                 const genrank_tables* t, const void* dx, int32_t* item_ids,
                                 float* item_rows, int32_t* n_items, float* d_action, float* d_pos,
                                 float* d_ri, float* d_rt, void* ws, size_t ws_bytes,
                                 genrank_stream_t stream) {
  GR_TRY(check_embed_args(b, in, t));
  if (!dx || !item_ids || !item_rows || !n_items || !d_action || !d_pos || !d_ri || !d_rt)
    return GENRANK_E_ARG;
  if (5 * static_cast<int64_t>(rows_of(b)) >= (int64_t(1) << 31)) return GENRANK_E_SHAPE;
  if (!ws || ws_bytes < embed_bwd_workspace(b)) return GENRANK_E_WORKSPACE;
  return launch_embed_bwd(b, in, t, dx, item_ids, item_rows, n_items, d_action, d_pos, d_ri, d_rt, ws,
                          S(stream));
}

genrank_status genrank_attn_fwd(const genrank_batch* b, const int32_t* offsets,
                                const int64_t* ts, const int64_t* req, genrank_alibi alibi,
                                const void* q, const void* k, const void* v, int64_t ld_qkv,
                                void* o, int64_t ld_o, float* lse, genrank_stream_t stream) {
  GR_TRY(check_attn_args(b, offsets, ts, req, alibi, q, k, v, ld_qkv, o, ld_o));
  return launch_attn_fwd(b, offsets, ts, req, alibi, q, k, v, ld_qkv, o, ld_o, lse, S(stream));
}

genrank_status genrank_hstu_rab_layout(const genrank_batch* b, const int32_t* offsets,
                                       int64_t* rab_offsets, genrank_stream_t stream) {
  GR_TRY(check_batch(b));
  if (!offsets || !rab_offsets) return GENRANK_E_ARG;
  return launch_hstu_rab_layout(b, offsets, rab_offsets, S(stream));
}

genrank_status genrank_hstu_rab(const genrank_batch* b, const int32_t* offsets, const int64_t* ts,
                                const int64_t* req, const float* pos_table, int32_t n_pos,
                                const float* time_table, const int64_t* time_bounds, int32_t n_time,
                                const int64_t* rab_offsets, void* rab, genrank_stream_t stream) {
  GR_TRY(check_batch(b));
  if (!offsets || !req || !pos_table || !time_table || !rab_offsets || !rab) return GENRANK_E_ARG;
  if (b->total_hist > 0 && !ts) return GENRANK_E_ARG;
  if (n_pos < 1 || n_time < 1 || (n_time > 1 && !time_bounds)) return GENRANK_E_ARG;
  return launch_hstu_rab(b, offsets, ts, req, pos_table, n_pos, time_table, time_bounds, n_time,
                         rab_offsets, rab, S(stream));
}

genrank_status genrank_hstu_attn_fwd(const genrank_batch* b, const int32_t* offsets, const void* rab,
                                     const int64_t* rab_offsets, const void* q, const void* k,
                                     const void* v, int64_t ld_qkv, void* o, int64_t ld_o, float* lse,
                                     genrank_stream_t stream) {
  GR_TRY(check_batch(b));
  if (!offsets || !rab || !rab_offsets || !q || !k || !v || !o) return GENRANK_E_ARG;
  return launch_hstu_attn_fwd(b, offsets, rab, rab_offsets, q, k, v, ld_qkv, o, ld_o, lse, S(stream));
}

genrank_status genrank_attn_bwd(const genrank_batch* b, const int32_t* offsets,
                                const int64_t* ts, const int64_t* req, genrank_alibi alibi,
                                const void* q, const void* k, const void* v, int64_t ld_qkv,
                                const void* o, const void* dout, int64_t ld_o, const float* lse,
                                void* dq, void* dk, void* dv, int64_t ld_dqkv,
                                int32_t cand_only, void* ws, size_t ws_bytes,
                                genrank_stream_t stream) {
  GR_TRY(check_attn_args(b, offsets, ts, req, alibi, q, k, v, ld_qkv, o, ld_o));
  if (!dout || !lse || !dq || !dk || !dv) return GENRANK_E_ARG;
  if (ld_dqkv < b->d) return GENRANK_E_SHAPE;
  if (b->dh > 64) return GENRANK_E_SHAPE;
  if (b->dtype == GENRANK_BF16) {  // 16-byte fragments of dout, 8-byte ones of dq, dk, dv
    if (ld_o % 8 || ld_dqkv % 4) return GENRANK_E_SHAPE;
    if (reinterpret_cast<uintptr_t>(dout) % 16 || reinterpret_cast<uintptr_t>(o) % 16 ||
        (reinterpret_cast<uintptr_t>(dq) | reinterpret_cast<uintptr_t>(dk) | reinterpret_cast<uintptr_t>(dv)) % 8)
      return GENRANK_E_ARG;
  }
  if (!ws || ws_bytes < attn_bwd_workspace(b)) return GENRANK_E_WORKSPACE;
  return launch_attn_bwd(b, offsets, ts, req, alibi, q, k, v, ld_qkv, o, dout, ld_o, lse, dq, dk,
                         dv, ld_dqkv, cand_only, ws, S(stream));
}

genrank_status genrank_attn_bwd_noalloc(const genrank_batch* b, const int32_t* offsets, const int64_t* ts,
                                        const int64_t* req, genrank_alibi alibi, const void* q, const void* k,
                                        const void* v, int64_t ld_qkv, const void* o, const void* dout,
                                        int64_t ld_o, const float* lse, void* dq, void* dk, void* dv,
                                        int64_t ld_dqkv, int32_t cand_only, genrank_stream_t stream) {
  GR_TRY(check_attn_args(b, offsets, ts, req, alibi, q, k, v, ld_qkv, o, ld_o));
  if (!dout || !lse || !dq || !dk || !dv) return GENRANK_E_ARG;
  if (ld_dqkv < b->d) return GENRANK_E_SHAPE;
  if (b->dh > 64) return GENRANK_E_SHAPE;
  if (b->dtype == GENRANK_BF16) {
    if (ld_o % 8 || ld_dqkv % 4) return GENRANK_E_SHAPE;
    if (reinterpret_cast<uintptr_t>(dout) % 16 || reinterpret_cast<uintptr_t>(o) % 16 ||
        (reinterpret_cast<uintptr_t>(dq) | reinterpret_cast<uintptr_t>(dk) | reinterpret_cast<uintptr_t>(dv)) % 8)
      return GENRANK_E_ARG;
  }
  if (attn_bwd_workspace(b) > attn_bwd_scratch_bytes()) return GENRANK_E_WORKSPACE;
  void* ws = nullptr;
  GR_TRY(attn_bwd_scratch(&ws));
  return launch_attn_bwd(b, offsets, ts, req, alibi, q, k, v, ld_qkv, o, dout, ld_o, lse, dq, dk,
                         dv, ld_dqkv, cand_only, ws, S(stream));
}

genrank_status genrank_layer_fwd(const genrank_batch* b, const genrank_layer_weights* w,
                                 const int32_t* offsets, const int64_t* ts, const int64_t* req,
                                 const void* x_in, void* y_out, int32_t flags, void* ws,
                                 size_t ws_bytes, genrank_stream_t stream) {
  GR_TRY(check_batch(b));
  GR_TRY(check_layer_weights(b, w));
  if (!x_in || !y_out || !offsets || !req || (b->total_hist > 0 && !ts)) return GENRANK_E_ARG;
  const bool pre = w->block == GENRANK_BLOCK_PRENORM;
  const int ffn = pre ? w->ffn_dim : 0;
  const LayerFwdWs L = layer_fwd_layout(b, w->block, ffn, static_cast<char*>(ws));
  if (!ws || ws_bytes < L.bytes) return GENRANK_E_WORKSPACE;
  if (!pre && x_in == y_out) return GENRANK_E_ARG;
  const hipStream_t s = S(stream);
  const int dt = b->dtype;
  const int T = static_cast<int>(rows_of(b));
  const int d = b->d;
  const size_t es = dtype_size(dt);
  if (T == 0) return GENRANK_OK;
  GR_TRY(check_attn_args(b, offsets, ts, req, w->alibi, L.qkv, L.qkv + d * es, L.qkv + 2 * d * es,
                         3 * d, L.o, d));
  const bool fuse = pre && rms_fused(b, w) && !(flags & GENRANK_FWD_SAVE);
  const int rt = resid_dtype(b);
  // the residual sums: bf16 (EPI_RESID) or f32 (EPI_RESID_F32) rows
  const int epi_res = rt == dt ? GEMM_EPI_RESID : GEMM_EPI_RESID_F32;
  if (fuse) {
    GR_TRY(launch_scale_cols(w->wqkv, d, w->g1, L.wg, d, 3 * d, d, s));
    GR_TRY(launch_gemm_nt_rms(x_in, d, L.wg, d, L.qkv, 3 * d, T, 3 * d, d, GEMM_EPI_STORE, s));
  } else {
    const void* zin = x_in;
    if (pre) {
      GR_TRY(launch_rmsnorm(rt, dt, x_in, w->g1, L.z, T, d, s));
      zin = L.z;
    }
    GR_TRY(launch_gemm_nt(dt, zin, d, w->wqkv, d, L.qkv, 3 * d, T, 3 * d, d, GEMM_EPI_STORE,
                          nullptr, 0, nullptr, 0, s));
  }
  // the softmax statistics only serve the backward
  GR_TRY(launch_attn_fwd(b, offsets, ts, req, w->alibi, L.qkv, L.qkv + d * es, L.qkv + 2 * d * es,
                         3 * d, L.o, d, (flags & GENRANK_FWD_SAVE) ? L.lse : nullptr, s));
  if (!pre) {
    return launch_gemm_nt(dt, L.o, d, w->wo, d, y_out, d, T, d, d, GEMM_EPI_STORE, nullptr, 0,
                          nullptr, 0, s);
  }
  GR_TRY(launch_gemm_nt(dt, L.o, d, w->wo, d, L.x1, d, T, d, d, epi_res, x_in, d, nullptr, 0, s));
  if (fuse) {
    GR_TRY(launch_scale_cols(w->w1, d, w->g2, L.wg, d, ffn, d, s));
    GR_TRY(launch_gemm_nt_rms(L.x1, d, L.wg, d, L.hdn, ffn, T, ffn, d, GEMM_EPI_SILU, s));
  } else {
    GR_TRY(launch_rmsnorm(rt, dt, L.x1, w->g2, L.z2, T, d, s));
    GR_TRY(launch_gemm_nt(dt, L.z2, d, w->w1, d, L.hdn, ffn, T, ffn, d, GEMM_EPI_SILU, nullptr, 0,
                          (flags & GENRANK_FWD_SAVE) ? L.a : nullptr, ffn, s));
  }
  return launch_gemm_nt(dt, L.hdn, ffn, w->w2, ffn, y_out, d, T, d, ffn, epi_res, L.x1, d, nullptr, 0, s);
}

genrank_status genrank_embed_sum_cand(const genrank_batch* b, const genrank_inputs* in, const genrank_tables* t,
                                      void* x_cand, genrank_stream_t stream) {
  GR_TRY(check_embed_args(b, in, t));
  if (!x_cand) return GENRANK_E_ARG;
  return launch_embed_sum_cand(b, in, t, x_cand, S(stream));
}

genrank_status genrank_attn_fwd_cached(const genrank_batch* b, const int32_t* offsets, const int64_t* ts,
                                       const int64_t* req, genrank_alibi alibi, const void* q, const void* k,
                                       const void* v, int64_t ld_qkv, const void* k_hist, const void* v_hist,
                                       int64_t ld_hist, void* o, int64_t ld_o, float* lse, genrank_stream_t stream) {
  if (!b) return GENRANK_E_ARG;
  GR_TRY(check_batch(b));
  if (!offsets || !req || !alibi.slopes_pos || !alibi.slopes_time) return GENRANK_E_ARG;
  if ((b->total_hist > 0 && (!ts || !k_hist || !v_hist)) || !q || !k || !v || !o) return GENRANK_E_ARG;
  GR_TRY(check_alibi_variant(alibi, b->H));
  GR_TRY(check_cached_attn(b, q, k, v, ld_qkv, k_hist, v_hist, ld_hist, o, ld_o));
  return launch_attn_fwd_cached(b, offsets, ts, req, alibi, q, k, v, ld_qkv, k_hist, v_hist, ld_hist, o, ld_o,
                                lse, S(stream));
}

genrank_status genrank_layer_kv(const genrank_batch* b, const genrank_layer_weights* w, const void* x_hist,
                                void* kv, int64_t ld_kv, void* ws, size_t ws_bytes, genrank_stream_t stream) {
  GR_TRY(check_batch(b));
  GR_TRY(check_layer_weights(b, w));
  if (!x_hist || !kv) return GENRANK_E_ARG;
  if (ld_kv < 2 * b->d) return GENRANK_E_SHAPE;
  if (ws_bytes < layer_kv_bytes(b, w) || (layer_kv_bytes(b, w) > 0 && !ws)) return GENRANK_E_WORKSPACE;
  const int64_t Th = b->total_hist;
  if (Th == 0) return GENRANK_OK;
  const hipStream_t s = S(stream);
  const int dt = b->dtype;
  const int d = b->d;
  // rows [d, 3d) of wqkv: the key and value projections
  const char* wkv = static_cast<const char*>(w->wqkv) + static_cast<size_t>(d) * d * dtype_size(dt);
  if (rms_fused(b, w)) {
    char* wg = static_cast<char*>(ws) + align_up(static_cast<size_t>(Th) * d * dtype_size(dt));
    GR_TRY(launch_scale_cols(wkv, d, w->g1, wg, d, 2 * d, d, s));
    return launch_gemm_nt_rms(x_hist, d, wg, d, kv, ld_kv, static_cast<int>(Th), 2 * d, d, GEMM_EPI_STORE, s);
  }
  const void* z = x_hist;
  if (w->block == GENRANK_BLOCK_PRENORM) {
    GR_TRY(launch_rmsnorm(resid_dtype(b), dt, x_hist, w->g1, ws, Th, d, s));
    z = ws;
  }
  return launch_gemm_nt(dt, z, d, wkv, d, kv, ld_kv, static_cast<int>(Th), 2 * d, d, GEMM_EPI_STORE, nullptr, 0,
                        nullptr, 0, s);
}

genrank_status genrank_layer_fwd_cached(const genrank_batch* b, const genrank_layer_weights* w,
                                        const int32_t* offsets, const int64_t* ts, const int64_t* req,
                                        const void* kv_hist, int64_t ld_kv, const void* x_cand, void* y_cand,
                                        void* ws, size_t ws_bytes, genrank_stream_t stream) {
  GR_TRY(check_batch(b));
  GR_TRY(check_layer_weights(b, w));
  if (!x_cand || !y_cand || !offsets || !req || (b->total_hist > 0 && (!ts || !kv_hist))) return GENRANK_E_ARG;
  const bool pre = w->block == GENRANK_BLOCK_PRENORM;
  if (!pre && x_cand == y_cand) return GENRANK_E_ARG;
  const genrank_batch c = cand_rows_batch(b);
  const int ffn = pre ? w->ffn_dim : 0;
  const LayerFwdWs L = layer_fwd_layout(&c, w->block, ffn, static_cast<char*>(ws));
  if (!ws || ws_bytes < L.bytes) return GENRANK_E_WORKSPACE;
  const int dt = b->dtype;
  const int d = b->d;
  const size_t es = dtype_size(dt);
  const int Tc = static_cast<int>(static_cast<int64_t>(b->B) * b->m);
  const char* kh = static_cast<const char*>(kv_hist);
  GR_TRY(check_cached_attn(b, L.qkv, L.qkv + d * es, L.qkv + 2 * d * es, 3 * d, kh ? kh : L.qkv,
                           kh ? kh + d * es : L.qkv, ld_kv, L.o, d));
  if (Tc == 0) return GENRANK_OK;
  const hipStream_t s = S(stream);
  const bool fuse = pre && rms_fused(b, w);
  const int rt = resid_dtype(b);
  const int epi_res = rt == dt ? GEMM_EPI_RESID : GEMM_EPI_RESID_F32;
  if (fuse) {
    GR_TRY(launch_scale_cols(w->wqkv, d, w->g1, L.wg, d, 3 * d, d, s));
    GR_TRY(launch_gemm_nt_rms(x_cand, d, L.wg, d, L.qkv, 3 * d, Tc, 3 * d, d, GEMM_EPI_STORE, s));
  } else {
    const void* zin = x_cand;
    if (pre) {
      GR_TRY(launch_rmsnorm(rt, dt, x_cand, w->g1, L.z, Tc, d, s));
      zin = L.z;
    }
    GR_TRY(launch_gemm_nt(dt, zin, d, w->wqkv, d, L.qkv, 3 * d, Tc, 3 * d, d, GEMM_EPI_STORE, nullptr, 0, nullptr,
                          0, s));
  }
  GR_TRY(launch_attn_fwd_cached(b, offsets, ts, req, w->alibi, L.qkv, L.qkv + d * es, L.qkv + 2 * d * es, 3 * d,
                                kh ? kh : L.qkv, kh ? kh + d * es : L.qkv, ld_kv, L.o, d, nullptr, s));
  if (!pre)
    return launch_gemm_nt(dt, L.o, d, w->wo, d, y_cand, d, Tc, d, d, GEMM_EPI_STORE, nullptr, 0, nullptr, 0, s);
  GR_TRY(launch_gemm_nt(dt, L.o, d, w->wo, d, L.x1, d, Tc, d, d, epi_res, x_cand, d, nullptr, 0, s));
  if (fuse) {
    GR_TRY(launch_scale_cols(w->w1, d, w->g2, L.wg, d, ffn, d, s));
    GR_TRY(launch_gemm_nt_rms(L.x1, d, L.wg, d, L.hdn, ffn, Tc, ffn, d, GEMM_EPI_SILU, s));
  } else {
    GR_TRY(launch_rmsnorm(rt, dt, L.x1, w->g2, L.z2, Tc, d, s));
    GR_TRY(launch_gemm_nt(dt, L.z2, d, w->w1, d, L.hdn, ffn, Tc, ffn, d, GEMM_EPI_SILU, nullptr, 0, nullptr, ffn,
                          s));
  }
  return launch_gemm_nt(dt, L.hdn, ffn, w->w2, ffn, y_cand, d, Tc, d, ffn, epi_res, L.x1, d, nullptr, 0, s);
}

genrank_status genrank_layer_bwd(const genrank_batch* b, const genrank_layer_weights* w,
                                 const int32_t* offsets, const int64_t* ts, const int64_t* req,
                                 const void* x_in, const void* ws, const void* dy, void* dx,
                                 genrank_layer_grads g, int32_t cand_only, void* ws_bwd,
                                 size_t ws_bwd_bytes, genrank_stream_t stream) {
  GR_TRY(check_batch(b));
  GR_TRY(check_layer_weights(b, w));
  if (!x_in || !ws || !dy || !dx || !offsets || !req || (b->total_hist > 0 && !ts))
    return GENRANK_E_ARG;
  const bool pre = w->block == GENRANK_BLOCK_PRENORM;
  const int ffn = pre ? w->ffn_dim : 0;
  if (!g.wqkv || !g.wo || (pre && (!g.w1 || !g.w2 || !g.g1 || !g.g2))) return GENRANK_E_ARG;
  if (b->dh > 64) return GENRANK_E_SHAPE;
  const LayerFwdWs F = layer_fwd_layout(b, w->block, ffn, static_cast<char*>(const_cast<void*>(ws)));
  const LayerBwdWs L = layer_bwd_layout(b, w->block, ffn, static_cast<char*>(ws_bwd));
  if (!ws_bwd || ws_bwd_bytes < L.bytes) return GENRANK_E_WORKSPACE;
  const hipStream_t s = S(stream);
  const int dt = b->dtype;
  const int T = static_cast<int>(rows_of(b));
  const int d = b->d;
  const size_t es = dtype_size(dt);
  const void* att_grad = dy;  // gradient reaching the attention branch output
  const int64_t Tl = T;
  if (pre) {
    // FFN branch: y = x1 + W2 silu(W1 z2)
    GR_TRY(launch_gemm_tn(dt, dy, d, F.hdn, ffn, g.w2, ffn, d, ffn, Tl, L.tn, L.tn_bytes, s));
    // d a = (dy W2) * silu'(a), the SiLU backward fused into the product's epilogue
    GR_TRY(launch_gemm_nn(dt, dy, d, w->w2, ffn, L.dh, ffn, T, ffn, d, L.wt, s, GEMM_EPI_DSILU, F.a, ffn));
    GR_TRY(launch_gemm_tn(dt, L.dh, ffn, F.z2, d, g.w1, d, ffn, d, Tl, L.tn, L.tn_bytes, s));
    GR_TRY(launch_gemm_nn(dt, L.dh, ffn, w->w1, d, L.dz2, d, T, d, ffn, L.wt, s));
    GR_TRY(launch_rmsnorm_bwd(resid_dtype(b), dt, F.x1, w->g2, L.dz2, dy, L.dx1, g.g2, T, d, L.rms, s));
    att_grad = L.dx1;
  }
  // attention branch: out = Wo o
  GR_TRY(launch_gemm_tn(dt, att_grad, d, F.o, d, g.wo, d, d, d, Tl, L.tn, L.tn_bytes, s));
  GR_TRY(launch_gemm_nn(dt, att_grad, d, w->wo, d, L.dout, d, T, d, d, L.wt, s));
  GR_TRY(launch_attn_bwd(b, offsets, ts, req, w->alibi, F.qkv, F.qkv + d * es, F.qkv + 2 * d * es,
                         3 * d, F.o, L.dout, d, F.lse, L.dqkv, L.dqkv + d * es,
                         L.dqkv + 2 * d * es, 3 * d, cand_only, L.attn, s));
  const void* zin = pre ? static_cast<const void*>(F.z) : x_in;
  GR_TRY(launch_gemm_tn(dt, L.dqkv, 3 * d, zin, d, g.wqkv, d, 3 * d, d, Tl, L.tn, L.tn_bytes, s));
  if (!pre) return launch_gemm_nn(dt, L.dqkv, 3 * d, w->wqkv, d, dx, d, T, d, 3 * d, L.wt, s);
  GR_TRY(launch_gemm_nn(dt, L.dqkv, 3 * d, w->wqkv, d, L.dz, d, T, d, 3 * d, L.wt, s));
  return launch_rmsnorm_bwd(resid_dtype(b), dt, x_in, w->g1, L.dz, L.dx1, dx, g.g1, T, d, L.rms, s);
}

genrank_status genrank_linear(int32_t dtype, const void* x, int64_t ldx, const void* w,
                              int64_t ldw, void* y, int64_t ldy, int64_t M, int32_t N, int32_t K,
                              int32_t epilogue, const void* residual, int64_t ldr, void* pre,
                              int64_t ldpre, genrank_stream_t stream) {
  if (dtype != GENRANK_F32 && dtype != GENRANK_BF16) return GENRANK_E_DTYPE;
  if (!x || !w || !y) return GENRANK_E_ARG;
  if (M < 0 || N < 1 || K < 1 || M >= (int64_t(1) << 31)) return GENRANK_E_SHAPE;
  if (ldx < K || ldw < K || ldy < N) return GENRANK_E_SHAPE;
  int epi;
  switch (epilogue) {
    case GENRANK_EPI_NONE: epi = GEMM_EPI_STORE; break;
    case GENRANK_EPI_RESIDUAL:
      if (!residual || ldr < N) return GENRANK_E_ARG;
      epi = GEMM_EPI_RESID;
      break;
    case GENRANK_EPI_SILU:
      if (pre && ldpre < N) return GENRANK_E_SHAPE;
      epi = GEMM_EPI_SILU;
      break;
    case GENRANK_EPI_RESIDUAL_F32:
      if (!residual || ldr < N) return GENRANK_E_ARG;
      if (ldy % 4 || ldr % 4) return GENRANK_E_SHAPE;
      if ((reinterpret_cast<uintptr_t>(y) | reinterpret_cast<uintptr_t>(residual)) % 16) return GENRANK_E_ARG;
      epi = GEMM_EPI_RESID_F32;
      break;
    default: return GENRANK_E_ARG;
  }
  return launch_gemm_nt(dtype, x, ldx, w, ldw, y, ldy, static_cast<int>(M), N, K, epi, residual, ldr,
                        pre, ldpre, S(stream));
}

namespace genrank {
namespace {
size_t linear_bwd_bytes(int32_t dtype, int64_t M, int32_t N, int32_t K) {
  if (dtype != GENRANK_BF16) return 0;
  return align_up(static_cast<size_t>(N) * K * 2) + gemm_tn_workspace(N, K, M);
}
}  // namespace
}  // namespace genrank

genrank_status genrank_linear_bwd_workspace(int32_t dtype, int64_t M, int32_t N, int32_t K, size_t* bytes) {
  if (!bytes) return GENRANK_E_ARG;
  if (dtype != GENRANK_F32 && dtype != GENRANK_BF16) return GENRANK_E_DTYPE;
  if (M < 0 || N < 1 || K < 1 || M >= (int64_t(1) << 31)) return GENRANK_E_SHAPE;
  *bytes = linear_bwd_bytes(dtype, M, N, K);
  return GENRANK_OK;
}

genrank_status genrank_linear_bwd(int32_t dtype, const void* x, int64_t ldx, const void* w, int64_t ldw,
                                  const void* dy, int64_t ldy, void* dx, int64_t lddx, float* dw,
                                  int64_t lddw, int64_t M, int32_t N, int32_t K, void* ws,
                                  size_t ws_bytes, genrank_stream_t stream) {
  if (dtype != GENRANK_F32 && dtype != GENRANK_BF16) return GENRANK_E_DTYPE;
  if (!dy || (dx && !w) || (dw && !x)) return GENRANK_E_ARG;
  if (M < 0 || N < 1 || K < 1 || M >= (int64_t(1) << 31)) return GENRANK_E_SHAPE;
  if (ldy < N || (dx && (ldw < K || lddx < K)) || (dw && (ldx < K || lddw < K))) return GENRANK_E_SHAPE;
  const size_t need = linear_bwd_bytes(dtype, M, N, K);
  if (need > 0 && (!ws || ws_bytes < need || reinterpret_cast<uintptr_t>(ws) % 16)) return GENRANK_E_WORKSPACE;
  const hipStream_t s = S(stream);
  char* wt = static_cast<char*>(ws);
  char* tn = need > 0 ? wt + align_up(static_cast<size_t>(N) * K * 2) : nullptr;
  const size_t tn_bytes = need > 0 ? need - align_up(static_cast<size_t>(N) * K * 2) : 0;
  if (dx) GR_TRY(launch_gemm_nn(dtype, dy, ldy, w, ldw, dx, lddx, static_cast<int>(M), K, N, wt, s));
  if (dw) GR_TRY(launch_gemm_tn(dtype, dy, ldy, x, ldx, dw, lddw, N, K, M, tn, tn_bytes, s));
  return GENRANK_OK;
}

genrank_status genrank_rmsnorm(int32_t x_dtype, int32_t y_dtype, const void* x, const float* g, void* y,
                               int64_t rows, int32_t d, genrank_stream_t stream) {
  if (!x || !g || !y) return GENRANK_E_ARG;
  if (rows < 0 || d < 1) return GENRANK_E_SHAPE;
  const bool ok = (x_dtype == GENRANK_BF16 && y_dtype == GENRANK_BF16) ||
                  (x_dtype == GENRANK_F32 && (y_dtype == GENRANK_BF16 || y_dtype == GENRANK_F32));
  if (!ok) return GENRANK_E_DTYPE;
  return launch_rmsnorm(x_dtype, y_dtype, x, g, y, rows, d, S(stream));
}

genrank_status genrank_head_fwd(const genrank_batch* b, const void* x, const float* g_final,
                                const float* w_head, const float* b_head, int32_t n_tasks,
                                float* logits, genrank_stream_t stream) {
  GR_TRY(check_batch(b));
  if (!x || !g_final || !w_head || !b_head || !logits) return GENRANK_E_ARG;
  if (n_tasks < 1 || n_tasks > 8) return GENRANK_E_SHAPE;
  return launch_head_fwd(resid_dtype(b), x, b->total_hist, static_cast<int64_t>(b->B) * b->m, nullptr, b->d,
                         g_final, w_head, b_head, n_tasks, logits, S(stream));
}

genrank_status genrank_head_fwd_rows(int32_t dtype, int32_t d, const void* x, int64_t n_rows,
                                     const int32_t* rows, const float* g_final, const float* w_head,
                                     const float* b_head, int32_t n_tasks, float* logits,
                                     genrank_stream_t stream) {
  if (dtype != GENRANK_BF16 && dtype != GENRANK_F32) return GENRANK_E_DTYPE;
  if (!x || !g_final || !w_head || !b_head || !logits || (n_rows > 0 && !rows)) return GENRANK_E_ARG;
  if (n_rows < 0 || d < 1) return GENRANK_E_SHAPE;
  if (n_tasks < 1 || n_tasks > 8) return GENRANK_E_SHAPE;
  return launch_head_fwd(dtype, x, 0, n_rows, rows, d, g_final, w_head, b_head, n_tasks, logits, S(stream));
}

genrank_status genrank_head_bwd(const genrank_batch* b, const void* x, const float* g_final,
                                const float* w_head, int32_t n_tasks, const float* dlogits,
                                void* dx, float* dg_final, float* dw_head, float* db_head, void* ws,
                                size_t ws_bytes, genrank_stream_t stream) {
  GR_TRY(check_batch(b));
  if (!x || !g_final || !w_head || !dlogits || !dx || !dg_final || !dw_head || !db_head)
    return GENRANK_E_ARG;
  if (n_tasks < 1 || n_tasks > 4) return GENRANK_E_SHAPE;
  if (b->d > 1024 || b->d % 4) return GENRANK_E_SHAPE;
  if (!ws || ws_bytes < head_bwd_workspace(b->d, n_tasks)) return GENRANK_E_WORKSPACE;
  const hipStream_t s = S(stream);
  GR_TRY(launch_fill_zero(b->dtype, dx, b->total_hist * b->d, s));
  return launch_head_bwd(resid_dtype(b), b->dtype, x, b->total_hist, static_cast<int64_t>(b->B) * b->m, nullptr, b->d,
                         g_final, w_head, n_tasks, dlogits, dx, dg_final, dw_head, db_head, ws, s);
}

genrank_status genrank_head_bwd_rows(int32_t x_dtype, int32_t dtype, int32_t d, int64_t n_x_rows, const void* x,
                                     int64_t n_rows, const int32_t* rows, const float* g_final,
                                     const float* w_head, int32_t n_tasks, const float* dlogits, void* dx,
                                     float* dg_final, float* dw_head, float* db_head, void* ws,
                                     size_t ws_bytes, genrank_stream_t stream) {
  if (dtype != GENRANK_BF16 && dtype != GENRANK_F32) return GENRANK_E_DTYPE;
  if (x_dtype != dtype && x_dtype != GENRANK_F32) return GENRANK_E_DTYPE;
  if (!x || !g_final || !w_head || !dlogits || !dx || !dg_final || !dw_head || !db_head ||
      (n_rows > 0 && !rows))
    return GENRANK_E_ARG;
  if (n_rows < 0 || n_x_rows < 0 || d < 1) return GENRANK_E_SHAPE;
  if (n_tasks < 1 || n_tasks > 4) return GENRANK_E_SHAPE;
  if (d > 1024 || d % 4) return GENRANK_E_SHAPE;
  if (!ws || ws_bytes < head_bwd_workspace(d, n_tasks)) return GENRANK_E_WORKSPACE;
  const hipStream_t s = S(stream);
  GR_TRY(launch_fill_zero(dtype, dx, n_x_rows * d, s));
  return launch_head_bwd(x_dtype, dtype, x, 0, n_rows, rows, d, g_final, w_head, n_tasks, dlogits, dx, dg_final, dw_head,
                         db_head, ws, s);
}

genrank_status genrank_bce_loss(int64_t n, int32_t n_tasks, const float* logits,
                                const float* labels, float* loss, float* dlogits,
                                genrank_stream_t stream) {
  if (!logits || !labels || !loss || !dlogits) return GENRANK_E_ARG;
  if (n < 1 || n_tasks < 1) return GENRANK_E_ARG;
  return launch_bce(n, n_tasks, logits, labels, loss, dlogits, S(stream));
}

genrank_status genrank_debug_mask(const genrank_batch* b, const int32_t* offsets, int32_t user,
                                  int32_t L_cap, uint8_t* out, genrank_stream_t stream) {
  GR_TRY(check_batch(b));
  if (!offsets || !out) return GENRANK_E_ARG;
  if (user < 0 || user >= b->B || L_cap < 1) return GENRANK_E_ARG;
  return launch_debug_mask(offsets, b->m, user, L_cap, out, S(stream));
}

}  // extern "C"
