// Backward of the masked ALiBi attention ("一、 GenRank [2025]" section 1.4.2: ALiBi is
// parameter-free, so only q, k, v receive gradients; section 1.3.1: the loss sits at
// candidate positions only).
//
// With P recomputed from the forward's log-sum-exp:
//   D_i = sum_d dO_i O_i;  dP_ij = dO_i . v_j;  dS_ij = P_ij (dP_ij - D_i)
//   dQ_i = sum_j dS_ij k_j / sqrt(dh);  dK_j = sum_i dS_ij q_i / sqrt(dh);
//   dV_j = sum_i P_ij dO_i.
// Three kernels: D (one wave per row and head), dQ (one wave per query row: loop over the
// keys it attends) and dK/dV (one wave per key row: loop over the queries that attend it
// -- later history queries and every candidate for a history key, the candidate itself
// for a candidate key).  Lane d owns head dimension d; dot products are wave reductions.
// With cand_only set, history query rows carry dO = 0 and are skipped.
#include <math.h>

#include "common.hpp"
#include "internal.hpp"

namespace genrank {

namespace {

struct BwdArgs {
  const int32_t* offsets;
  const int64_t* ts;
  const int64_t* req;
  const void* q; const void* k; const void* v; int64_t ld_qkv;
  const void* o; const void* dout; int64_t ld_o;
  const float* lse;
  void* dq; void* dk; void* dv; int64_t ld_d;
  float* delta;   // [T, H]
  float sp[GENRANK_MAX_HEADS];
  float st[GENRANK_MAX_HEADS];
  float scale;
  int B, m, H, dh, cand_only;
  int64_t T_h;
};

__device__ __forceinline__ float wsum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

struct Slots {
  int u, i, N;
  int64_t off, t0;
};

__device__ __forceinline__ Slots locate(const BwdArgs& a, int64_t row) {
  Slots s;
  if (row < a.T_h) {
    s.u = find_user(a.offsets, a.B, row);
    s.i = static_cast<int>(row - a.offsets[s.u]);
  } else {
    const int64_t c = row - a.T_h;
    s.u = static_cast<int>(c / a.m);
    s.i = static_cast<int>(c - static_cast<int64_t>(s.u) * a.m);
  }
  s.off = a.offsets[s.u];
  s.N = a.offsets[s.u + 1] - a.offsets[s.u];
  if (row >= a.T_h) s.i += s.N;
  s.t0 = (s.N > 0) ? a.ts[s.off] : a.req[s.u];
  return s;
}

__device__ __forceinline__ int64_t slot_row(const BwdArgs& a, const Slots& s, int j) {
  return (j < s.N) ? s.off + j : a.T_h + static_cast<int64_t>(s.u) * a.m + (j - s.N);
}
__device__ __forceinline__ float slot_bias(const BwdArgs& a, const Slots& s, int h, int i, int j) {
  const int pi = (i < s.N) ? i : s.N, pj = (j < s.N) ? j : s.N;
  const int64_t ti = ((i < s.N) ? a.ts[s.off + i] : a.req[s.u]) - s.t0;
  const int64_t tj = ((j < s.N) ? a.ts[s.off + j] : a.req[s.u]) - s.t0;
  return -a.sp[h] * fabsf(static_cast<float>(pi - pj)) - a.st[h] * fabsf(static_cast<float>(ti - tj));
}

template <typename T>
__global__ void __launch_bounds__(64) delta_kernel(BwdArgs a) {
  const int64_t row = blockIdx.x;
  const int h = blockIdx.y;
  const int lane = threadIdx.x;
  const T* o = static_cast<const T*>(a.o);
  const T* dO = static_cast<const T*>(a.dout);
  float v = 0.f;
  if (lane < a.dh) v = to_f32(o[row * a.ld_o + h * a.dh + lane]) * to_f32(dO[row * a.ld_o + h * a.dh + lane]);
  v = wsum(v);
  if (lane == 0) a.delta[row * a.H + h] = v;
}

template <typename T>
__global__ void __launch_bounds__(64) dq_kernel(BwdArgs a) {
  const int64_t row = blockIdx.x;
  const int h = blockIdx.y;
  const int lane = threadIdx.x;
  const bool act = lane < a.dh;
  T* dq = static_cast<T*>(a.dq);
  if (a.cand_only && row < a.T_h) {
    if (act) dq[row * a.ld_d + h * a.dh + lane] = from_f32<T>(0.f);
    return;
  }
  const T* q = static_cast<const T*>(a.q);
  const T* k = static_cast<const T*>(a.k);
  const T* v = static_cast<const T*>(a.v);
  const T* dO = static_cast<const T*>(a.dout);
  const Slots s = locate(a, row);
  const int L = s.N + a.m;
  const float qd = act ? to_f32(q[row * a.ld_qkv + h * a.dh + lane]) : 0.f;
  const float dod = act ? to_f32(dO[row * a.ld_o + h * a.dh + lane]) : 0.f;
  const float lse = a.lse[row * a.H + h];
  const float Di = a.delta[row * a.H + h];
  float acc = 0.f;
  for (int j = 0; j < L; ++j) {
    if (!attn_allowed(s.i, j, s.N)) continue;
    const int64_t kr = slot_row(a, s, j);
    const float kd = act ? to_f32(k[kr * a.ld_qkv + h * a.dh + lane]) : 0.f;
    const float vd = act ? to_f32(v[kr * a.ld_qkv + h * a.dh + lane]) : 0.f;
    const float sc = wsum(qd * kd) * a.scale + slot_bias(a, s, h, s.i, j);
    const float p = expf(sc - lse);
    const float dp = wsum(dod * vd);
    acc += p * (dp - Di) * kd;
  }
  if (act) dq[row * a.ld_d + h * a.dh + lane] = from_f32<T>(acc * a.scale);
}

template <typename T>
__global__ void __launch_bounds__(64) dkv_kernel(BwdArgs a) {
  const int64_t row = blockIdx.x;  // key row
  const int h = blockIdx.y;
  const int lane = threadIdx.x;
  const bool act = lane < a.dh;
  const T* q = static_cast<const T*>(a.q);
  const T* k = static_cast<const T*>(a.k);
  const T* v = static_cast<const T*>(a.v);
  const T* dO = static_cast<const T*>(a.dout);
  const Slots s = locate(a, row);
  const int j = s.i;
  const int L = s.N + a.m;
  const float kd = act ? to_f32(k[row * a.ld_qkv + h * a.dh + lane]) : 0.f;
  const float vd = act ? to_f32(v[row * a.ld_qkv + h * a.dh + lane]) : 0.f;
  float ak = 0.f, av = 0.f;
  const int i_begin = (a.cand_only && j < s.N) ? s.N : j;
  for (int i = i_begin; i < L; ++i) {
    if (!attn_allowed(i, j, s.N)) continue;
    if (a.cand_only && i < s.N) continue;
    const int64_t qr = slot_row(a, s, i);
    const float qd = act ? to_f32(q[qr * a.ld_qkv + h * a.dh + lane]) : 0.f;
    const float dod = act ? to_f32(dO[qr * a.ld_o + h * a.dh + lane]) : 0.f;
    const float sc = wsum(qd * kd) * a.scale + slot_bias(a, s, h, i, j);
    const float p = expf(sc - a.lse[qr * a.H + h]);
    const float dp = wsum(dod * vd);
    const float ds = p * (dp - a.delta[qr * a.H + h]);
    av += p * dod;
    ak += ds * qd;
  }
  if (act) {
    static_cast<T*>(a.dk)[row * a.ld_d + h * a.dh + lane] = from_f32<T>(ak * a.scale);
    static_cast<T*>(a.dv)[row * a.ld_d + h * a.dh + lane] = from_f32<T>(av);
  }
}

}  // namespace

size_t attn_bwd_workspace(const genrank_batch* b) {
  const int64_t T = b->total_hist + static_cast<int64_t>(b->B) * b->m;
  return static_cast<size_t>(T) * b->H * sizeof(float) + 256;
}

genrank_status launch_attn_bwd(const genrank_batch* b, const int32_t* offsets, const int64_t* ts,
                               const int64_t* req, genrank_alibi alibi, const void* q,
                               const void* k, const void* v, int64_t ld_qkv, const void* o,
                               const void* dout, int64_t ld_o, const float* lse, void* dq,
                               void* dk, void* dv, int64_t ld_dqkv, int cand_only, void* ws,
                               hipStream_t stream) {
  const int64_t T = b->total_hist + static_cast<int64_t>(b->B) * b->m;
  if (T == 0) return GENRANK_OK;
  BwdArgs a{};
  a.offsets = offsets; a.ts = ts; a.req = req;
  a.q = q; a.k = k; a.v = v; a.ld_qkv = ld_qkv;
  a.o = o; a.dout = dout; a.ld_o = ld_o; a.lse = lse;
  a.dq = dq; a.dk = dk; a.dv = dv; a.ld_d = ld_dqkv;
  a.delta = static_cast<float*>(ws);
  for (int h = 0; h < b->H; ++h) {
    a.sp[h] = alibi.slopes_pos[h];
    a.st[h] = alibi.slopes_time[h];
  }
  a.scale = 1.f / sqrtf(static_cast<float>(b->dh));
  a.B = b->B; a.m = b->m; a.H = b->H; a.dh = b->dh; a.cand_only = cand_only;
  a.T_h = b->total_hist;
  dim3 grid(static_cast<unsigned>(T), b->H);
  if (b->dtype == GENRANK_BF16) {
    hipLaunchKernelGGL(delta_kernel<bf16_t>, grid, dim3(64), 0, stream, a);
    hipLaunchKernelGGL(dq_kernel<bf16_t>, grid, dim3(64), 0, stream, a);
    hipLaunchKernelGGL(dkv_kernel<bf16_t>, grid, dim3(64), 0, stream, a);
  } else {
    hipLaunchKernelGGL(delta_kernel<float>, grid, dim3(64), 0, stream, a);
    hipLaunchKernelGGL(dq_kernel<float>, grid, dim3(64), 0, stream, a);
    hipLaunchKernelGGL(dkv_kernel<float>, grid, dim3(64), 0, stream, a);
  }
  GR_CHECK_LAUNCH();
  return GENRANK_OK;
}

}  // namespace genrank
