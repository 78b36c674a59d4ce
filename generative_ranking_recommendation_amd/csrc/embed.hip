// Fused index derivation + five-table embedding gather-sum (and its adjoint).
//
// Token embedding of GenRank ("一、 GenRank [2025]", section 1.4.2, five-term input
// representation; section 1.4.1 for the item + action token and the mask-action row):
//   e = psi(item) + phi(action) + Omega_pe(position) + Omega_ri(request index)
//       + Omega_rt(bucket(gap to the previous request)).
//
// Work decomposition: one workgroup per (user, chunk of ROWS rows).  Wave 0 derives the
// chunk's indices: the request index is 1 + the number of timestamp changes in the
// user's prefix (timestamps are non-decreasing, so distinct values == runs); a block
// reduction counts the changes before the chunk and a 64-lane ballot scans the chunk.
// The previous distinct timestamp of a row is the one just before its run.  The five
// rows are then gathered with 16-byte loads (d/8 lanes per bf16 row), summed in f32 and
// written once.  The small tables stay L2-resident across the grid.
#include "common.hpp"
#include "internal.hpp"

namespace genrank {

namespace {

constexpr int EMB_THREADS = 256;
constexpr int EMB_ROWS = 64;  // rows per workgroup (one wave derives 64 rows' indices)
constexpr int MAX_BOUNDS = 1024;

struct EmbedArgs {
  const int32_t* offsets;
  const int32_t* hist_items;
  const int32_t* hist_actions;
  const int64_t* hist_ts;
  const int32_t* cand_items;
  const int64_t* req_ts;
  const void* t_item;
  const void* t_action;
  const void* t_pos;
  const void* t_ri;
  const void* t_rt;
  const int64_t* rt_bounds;
  int B, m, d, hist_chunks, cand_chunks;
  int n_action, n_pos, n_ri, n_bounds;
  int64_t T_h;
  void* out;            // gather: [T, d]; debug: int32 [6, T]
  const void* dx;       // backward: [T, d]
  float* g_item; float* g_action; float* g_pos; float* g_ri; float* g_rt;
};

template <typename T> struct Vec;
template <> struct Vec<bf16_t> { static constexpr int N = 8; };
template <> struct Vec<float> { static constexpr int N = 4; };

__device__ __forceinline__ void load_vec(const bf16_t* p, float* f) {
  uint4 v = *reinterpret_cast<const uint4*>(p);
  unpack8(v, f);
}
__device__ __forceinline__ void load_vec(const float* p, float* f) {
  float4 v = *reinterpret_cast<const float4*>(p);
  f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w;
}
__device__ __forceinline__ void store_vec(bf16_t* p, const float* f) {
  *reinterpret_cast<uint4*>(p) = pack8(f);
}
__device__ __forceinline__ void store_vec(float* p, const float* f) {
  *reinterpret_cast<float4*>(p) = make_float4(f[0], f[1], f[2], f[3]);
}

// Count k in [lo, hi) with ts[k] != ts[k-1] (block-wide; every thread gets the result).
__device__ int block_count_changes(const int64_t* __restrict__ ts, int64_t lo, int64_t hi,
                                   int* red) {
  int c = 0;
  for (int64_t k = lo + threadIdx.x; k < hi; k += EMB_THREADS) c += (ts[k] != ts[k - 1]);
  for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off);
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wave] = c;
  __syncthreads();
  int total = 0;
#pragma unroll
  for (int w = 0; w < EMB_THREADS / 64; ++w) total += red[w];
  return total;
}

// #{k : bounds[k] <= gap} over non-decreasing bounds (upper bound).
__device__ __forceinline__ int bucket_of(const int64_t* bounds, int n, int64_t gap) {
  int lo = 0, hi = n;
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if (bounds[mid] <= gap) lo = mid + 1; else hi = mid;
  }
  return lo;
}

struct RowIdx {
  int item, act, pos, pe, ri, ri_slot, rt;
};

// Derives the indices of the workgroup's rows into shared memory.  Returns the number of
// valid rows and the global row of the first one (via *row0).
__device__ int derive_chunk(const EmbedArgs& a, RowIdx* sidx, int64_t* sbounds, int* red,
                            int64_t* row0_out) {
  const int u = blockIdx.y;
  const int chunk = blockIdx.x;
  const int64_t off = a.offsets[u];
  const int N = a.offsets[u + 1] - a.offsets[u];
  const int lane = threadIdx.x & 63;
  const bool is_hist = chunk < a.hist_chunks;

  for (int k = threadIdx.x; k < a.n_bounds; k += EMB_THREADS) sbounds[k] = a.rt_bounds[k];

  if (is_hist) {
    const int s0 = chunk * EMB_ROWS;  // first sequence slot of the chunk
    if (s0 >= N) return 0;            // uniform across the block
    const int rows = min(EMB_ROWS, N - s0);
    const int64_t r0 = off + s0;
    // changes at k in [off+1, r0): each one starts a new request before the chunk
    const int before = block_count_changes(a.hist_ts, off + 1, r0, red);
    if (threadIdx.x < 64) {
      const int i = lane;
      const bool valid = i < rows;
      const int64_t r = r0 + i;
      const int64_t t = valid ? a.hist_ts[r] : 0;
      const bool change = valid && r > off && t != a.hist_ts[r - 1];
      const uint64_t mask = __ballot(change);
      // start of the run that holds r0: lower bound of ts[r0] in ts[off .. r0]
      int64_t run0;
      {
        const int64_t key = a.hist_ts[r0];
        int64_t lo = off, hi = r0;
        while (lo < hi) {
          int64_t mid = (lo + hi) >> 1;
          if (a.hist_ts[mid] < key) lo = mid + 1; else hi = mid;
        }
        run0 = lo;
      }
      if (valid) {
        const uint64_t upto = (i == 63) ? ~0ull : ((2ull << i) - 1ull);
        const uint64_t c = mask & upto;
        const int64_t run_start = c ? (r0 + 63 - __clzll(static_cast<long long>(c))) : run0;
        int rt = 0;
        if (run_start > off) {
          const int64_t gap = t - a.hist_ts[run_start - 1];
          rt = bucket_of(sbounds, a.n_bounds, gap);
        }
        RowIdx ix;
        ix.item = a.hist_items[r];
        ix.act = a.hist_actions[r];
        ix.pos = s0 + i;
        ix.pe = min(ix.pos, a.n_pos - 1);
        ix.ri = 1 + before + __popcll(c);
        ix.ri_slot = min(ix.ri - 1, a.n_ri - 1);
        ix.rt = rt;
        sidx[i] = ix;
      }
    }
    __syncthreads();
    *row0_out = r0;
    return rows;
  }
  // candidate chunk
  const int c0 = (chunk - a.hist_chunks) * EMB_ROWS;
  if (c0 >= a.m) return 0;
  const int rows = min(EMB_ROWS, a.m - c0);
  const int changes = block_count_changes(a.hist_ts, off + 1, off + N, red);
  const int distinct_hist = (N > 0) ? 1 + changes : 0;
  int rt = 0;
  if (N > 0) rt = bucket_of(sbounds, a.n_bounds, a.req_ts[u] - a.hist_ts[off + N - 1]);
  const int64_t r0 = a.T_h + static_cast<int64_t>(u) * a.m + c0;
  if (threadIdx.x < rows) {
    RowIdx ix;
    ix.item = a.cand_items[static_cast<int64_t>(u) * a.m + c0 + threadIdx.x];
    ix.act = a.n_action;
    ix.pos = N;
    ix.pe = min(N, a.n_pos - 1);
    ix.ri = distinct_hist + 1;
    ix.ri_slot = min(ix.ri - 1, a.n_ri - 1);
    ix.rt = rt;
    sidx[threadIdx.x] = ix;
  }
  __syncthreads();
  *row0_out = r0;
  return rows;
}

template <typename T>
__global__ void __launch_bounds__(EMB_THREADS) embed_sum_kernel(EmbedArgs a) {
  __shared__ RowIdx sidx[EMB_ROWS];
  __shared__ int64_t sbounds[MAX_BOUNDS];
  __shared__ int red[EMB_THREADS / 64];
  int64_t row0;
  const int rows = derive_chunk(a, sidx, sbounds, red, &row0);
  if (rows == 0) return;
  constexpr int V = Vec<T>::N;
  const int cpr = a.d / V;  // 16-byte chunks per row
  const int total = rows * cpr;
  const T* ti = static_cast<const T*>(a.t_item);
  const T* ta = static_cast<const T*>(a.t_action);
  const T* tp = static_cast<const T*>(a.t_pos);
  const T* tr = static_cast<const T*>(a.t_ri);
  const T* tt = static_cast<const T*>(a.t_rt);
  T* out = static_cast<T*>(a.out);
  const int64_t d = a.d;
  constexpr int U = 2;  // items per thread in flight
  for (int base = threadIdx.x; base < total; base += EMB_THREADS * U) {
    float acc[U][V];
    float tmp[V];
#pragma unroll
    for (int uu = 0; uu < U; ++uu) {
      const int idx = base + uu * EMB_THREADS;
      if (idx < total) {
        const int r = idx / cpr;
        const int col = (idx - r * cpr) * V;
        const RowIdx ix = sidx[r];
        load_vec(ti + ix.item * d + col, acc[uu]);
        load_vec(ta + ix.act * d + col, tmp);
#pragma unroll
        for (int e = 0; e < V; ++e) acc[uu][e] += tmp[e];
        load_vec(tp + ix.pe * d + col, tmp);
#pragma unroll
        for (int e = 0; e < V; ++e) acc[uu][e] += tmp[e];
        load_vec(tr + ix.ri_slot * d + col, tmp);
#pragma unroll
        for (int e = 0; e < V; ++e) acc[uu][e] += tmp[e];
        load_vec(tt + ix.rt * d + col, tmp);
#pragma unroll
        for (int e = 0; e < V; ++e) acc[uu][e] += tmp[e];
      }
    }
#pragma unroll
    for (int uu = 0; uu < U; ++uu) {
      const int idx = base + uu * EMB_THREADS;
      if (idx < total) {
        const int r = idx / cpr;
        const int col = (idx - r * cpr) * V;
        store_vec(out + (row0 + r) * d + col, acc[uu]);
      }
    }
  }
}

__global__ void __launch_bounds__(EMB_THREADS) debug_indices_kernel(EmbedArgs a, int64_t T) {
  __shared__ RowIdx sidx[EMB_ROWS];
  __shared__ int64_t sbounds[MAX_BOUNDS];
  __shared__ int red[EMB_THREADS / 64];
  int64_t row0;
  const int rows = derive_chunk(a, sidx, sbounds, red, &row0);
  if (static_cast<int>(threadIdx.x) < rows) {
    int32_t* out = static_cast<int32_t*>(a.out);
    const RowIdx ix = sidx[threadIdx.x];
    const int64_t r = row0 + threadIdx.x;
    out[0 * T + r] = ix.act;
    out[1 * T + r] = ix.pos;
    out[2 * T + r] = ix.pe;
    out[3 * T + r] = ix.ri;
    out[4 * T + r] = ix.ri_slot;
    out[5 * T + r] = ix.rt;
  }
}

// Adjoint: scatter-add dx rows into the five f32 table gradients.
template <typename T>
__global__ void __launch_bounds__(EMB_THREADS) embed_bwd_kernel(EmbedArgs a) {
  __shared__ RowIdx sidx[EMB_ROWS];
  __shared__ int64_t sbounds[MAX_BOUNDS];
  __shared__ int red[EMB_THREADS / 64];
  int64_t row0;
  const int rows = derive_chunk(a, sidx, sbounds, red, &row0);
  if (rows == 0) return;
  constexpr int V = Vec<T>::N;
  const int cpr = a.d / V;
  const int total = rows * cpr;
  const T* dx = static_cast<const T*>(a.dx);
  const int64_t d = a.d;
  for (int idx = threadIdx.x; idx < total; idx += EMB_THREADS) {
    const int r = idx / cpr;
    const int col = (idx - r * cpr) * V;
    const RowIdx ix = sidx[r];
    float g[V];
    load_vec(dx + (row0 + r) * d + col, g);
#pragma unroll
    for (int e = 0; e < V; ++e) {
      atomicAdd(a.g_item + ix.item * d + col + e, g[e]);
      atomicAdd(a.g_action + ix.act * d + col + e, g[e]);
      atomicAdd(a.g_pos + ix.pe * d + col + e, g[e]);
      atomicAdd(a.g_ri + ix.ri_slot * d + col + e, g[e]);
      atomicAdd(a.g_rt + ix.rt * d + col + e, g[e]);
    }
  }
}

EmbedArgs make_args(const genrank_batch* b, const genrank_inputs* in, const genrank_tables* t) {
  EmbedArgs a{};
  a.offsets = in->hist_offsets;
  a.hist_items = in->hist_items;
  a.hist_actions = in->hist_actions;
  a.hist_ts = in->hist_ts;
  a.cand_items = in->cand_items;
  a.req_ts = in->req_ts;
  a.t_item = t->item;
  a.t_action = t->action;
  a.t_pos = t->pos;
  a.t_ri = t->ri;
  a.t_rt = t->rt;
  a.rt_bounds = t->rt_bounds;
  a.B = b->B;
  a.m = b->m;
  a.d = b->d;
  a.hist_chunks = (b->max_hist + EMB_ROWS - 1) / EMB_ROWS;
  a.cand_chunks = (b->m + EMB_ROWS - 1) / EMB_ROWS;
  a.n_action = t->n_action;
  a.n_pos = t->n_pos;
  a.n_ri = t->n_ri;
  a.n_bounds = t->n_rt - 1;
  a.T_h = b->total_hist;
  return a;
}

dim3 grid_of(const EmbedArgs& a) {
  return dim3(static_cast<unsigned>(a.hist_chunks + a.cand_chunks), static_cast<unsigned>(a.B));
}

}  // namespace

genrank_status check_embed_args(const genrank_batch* b, const genrank_inputs* in,
                                const genrank_tables* t) {
  if (!b || !in || !t) return GENRANK_E_ARG;
  genrank_status s = check_batch(b);
  if (s != GENRANK_OK) return s;
  if (!in->hist_offsets || !in->req_ts) return GENRANK_E_ARG;
  if (b->total_hist > 0 && (!in->hist_items || !in->hist_actions || !in->hist_ts))
    return GENRANK_E_ARG;
  if (b->m > 0 && !in->cand_items) return GENRANK_E_ARG;
  if (!t->item || !t->action || !t->pos || !t->ri || !t->rt) return GENRANK_E_ARG;
  if (t->n_item < 1 || t->n_action < 1 || t->n_pos < 1 || t->n_ri < 1 || t->n_rt < 1)
    return GENRANK_E_ARG;
  if (t->n_rt - 1 > MAX_BOUNDS) return GENRANK_E_SHAPE;
  if (t->n_rt > 1 && !t->rt_bounds) return GENRANK_E_ARG;
  const int vec = (b->dtype == GENRANK_BF16) ? 8 : 4;
  if (b->d % vec != 0) return GENRANK_E_SHAPE;
  return GENRANK_OK;
}

genrank_status launch_embed_sum(const genrank_batch* b, const genrank_inputs* in,
                                const genrank_tables* t, void* out, hipStream_t stream) {
  EmbedArgs a = make_args(b, in, t);
  a.out = out;
  if (b->dtype == GENRANK_BF16)
    hipLaunchKernelGGL(embed_sum_kernel<bf16_t>, grid_of(a), dim3(EMB_THREADS), 0, stream, a);
  else
    hipLaunchKernelGGL(embed_sum_kernel<float>, grid_of(a), dim3(EMB_THREADS), 0, stream, a);
  GR_CHECK_LAUNCH();
  return GENRANK_OK;
}

genrank_status launch_debug_indices(const genrank_batch* b, const genrank_inputs* in,
                                    const genrank_tables* t, int32_t* out, hipStream_t stream) {
  EmbedArgs a = make_args(b, in, t);
  a.out = out;
  const int64_t T = b->total_hist + static_cast<int64_t>(b->B) * b->m;
  hipLaunchKernelGGL(debug_indices_kernel, grid_of(a), dim3(EMB_THREADS), 0, stream, a, T);
  GR_CHECK_LAUNCH();
  return GENRANK_OK;
}

genrank_status launch_embed_bwd(const genrank_batch* b, const genrank_inputs* in,
                                const genrank_tables* t, const void* dx, float* g_item,
                                float* g_action, float* g_pos, float* g_ri, float* g_rt,
                                hipStream_t stream) {
  EmbedArgs a = make_args(b, in, t);
  a.dx = dx;
  a.g_item = g_item;
  a.g_action = g_action;
  a.g_pos = g_pos;
  a.g_ri = g_ri;
  a.g_rt = g_rt;
  if (b->dtype == GENRANK_BF16)
    hipLaunchKernelGGL(embed_bwd_kernel<bf16_t>, grid_of(a), dim3(EMB_THREADS), 0, stream, a);
  else
    hipLaunchKernelGGL(embed_bwd_kernel<float>, grid_of(a), dim3(EMB_THREADS), 0, stream, a);
  GR_CHECK_LAUNCH();
  return GENRANK_OK;
}

}  // namespace genrank
