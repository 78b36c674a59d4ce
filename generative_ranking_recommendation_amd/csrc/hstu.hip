// HSTU-style comparison path: the interleaved item/action sequence with a learned relative
// attention bias materialised in memory, against which the action-oriented ALiBi path is
// measured ("一、 GenRank [2025]", section 1.4.1 on the interleaved organisation and its
// cost; "The Overall Generative Ranking Paradigm", section 7.2.2 on the learned relative
// bias).  User u's sequence: slots 0 .. 2N-1 alternate the item and the action token of
// history action i (both at time t_i, position = slot), then the m candidates (position 2N,
// the request time); L = 2N + m.  The bias matrix of user u is [L, P] bf16 (row pitch P = L
// rounded up to 8, pad columns 0) at element offset rab_off[u]:
//   rab[i][j] = pos_table[min(|p_i - p_j|, n_pos - 1)] + time_table[#{k : b_k <= |t_i - t_j|}].
#include "common.hpp"
#include "internal.hpp"

namespace genrank {

namespace {

constexpr int HT = 256;
constexpr int HSTU_MAX_L = 2048;     // longest sequence the bias kernel stages in LDS
constexpr int HSTU_MAX_BOUNDS = 1024;
constexpr int RAB_ROWS = 64;         // bias rows per workgroup
constexpr int HSTU_MAX_POS = 1024;   // position-difference table rows staged in LDS
constexpr int DIRECT_LOG2 = 10;
constexpr int DIRECT = 1 << DIRECT_LOG2;  // gaps below this many seconds: direct bucket table

__device__ __forceinline__ int64_t rab_elems(int n_hist, int m) {
  const int64_t L = 2 * static_cast<int64_t>(n_hist) + m;
  return L * ((L + 7) & ~int64_t{7});
}

// One workgroup: exclusive scan of L_u * P_u over the users.
__global__ void __launch_bounds__(HT) hstu_layout_kernel(const int32_t* offsets, int B, int m, int64_t* rab_off) {
  __shared__ int64_t part[HT];
  int64_t carry = 0;
  for (int base = 0; base < B; base += HT) {
    const int u = base + static_cast<int>(threadIdx.x);
    const int64_t v = u < B ? rab_elems(offsets[u + 1] - offsets[u], m) : 0;
    part[threadIdx.x] = v;
    __syncthreads();
    for (int d = 1; d < HT; d <<= 1) {  // inclusive scan (Hillis-Steele)
      const int64_t t = static_cast<int>(threadIdx.x) >= d ? part[threadIdx.x - d] : 0;
      __syncthreads();
      part[threadIdx.x] += t;
      __syncthreads();
    }
    if (u < B) rab_off[u] = carry + part[threadIdx.x] - v;
    carry += part[HT - 1];
    __syncthreads();
  }
  if (threadIdx.x == 0) rab_off[B] = carry;
}

struct RabArgs {
  const int32_t* offsets;
  const int64_t* ts;
  const int64_t* req;
  const float* pos_table;
  const float* time_table;
  const int64_t* bounds;
  const int64_t* rab_off;
  bf16_t* rab;
  int m, n_pos, n_bounds;
};

// Workgroup (row block, user): RAB_ROWS rows of user u's matrix.  Both tables, the slot
// times and the edges sit in LDS.
__global__ void __launch_bounds__(HT) hstu_rab_kernel(RabArgs a) {
  __shared__ int32_t st[HSTU_MAX_L];          // slot times relative to the user's first
  __shared__ int32_t sb[HSTU_MAX_BOUNDS];     // edges, clamped to int32
  __shared__ float spos[HSTU_MAX_POS];
  __shared__ float stime[HSTU_MAX_BOUNDS + 1];
  __shared__ int socts[34];
  __shared__ uint16_t sdir[DIRECT];            // bucket of every gap below DIRECT seconds
  __shared__ int sspan;
  const int u = blockIdx.y;
  const int64_t off = a.offsets[u];
  const int N = a.offsets[u + 1] - a.offsets[u];
  const int L = 2 * N + a.m;
  const int P = (L + 7) & ~7;
  const int i0 = blockIdx.x * RAB_ROWS;
  if (i0 >= L) return;
  const int64_t req = a.req[u];
  const int64_t t0 = N > 0 ? a.ts[off] : req;
  // relative times are below 2^24 s (a checked precondition of the inputs), so int32 holds them
  for (int j = threadIdx.x; j < L; j += HT)
    st[j] = static_cast<int32_t>((j < 2 * N ? a.ts[off + j / 2] : req) - t0);
  for (int k = threadIdx.x; k < a.n_bounds; k += HT) {
    const int64_t b = a.bounds[k];
    sb[k] = b > INT32_MAX ? INT32_MAX : (b < INT32_MIN ? INT32_MIN : static_cast<int32_t>(b));
  }
  for (int k = threadIdx.x; k < a.n_pos; k += HT) spos[k] = a.pos_table[k];
  for (int k = threadIdx.x; k <= a.n_bounds; k += HT) stime[k] = a.time_table[k];
  __syncthreads();
  if (threadIdx.x <= 32) {  // lo_e = #{k : b_k < 2^e}, e = 0 .. 32
    const int e = threadIdx.x;
    int lo = 0;
    while (lo < a.n_bounds && (e >= 31 || sb[lo] < (1 << e))) ++lo;
    socts[e] = lo;
  }
  __syncthreads();
  for (int x = threadIdx.x; x < DIRECT; x += HT) {  // #{k : b_k <= x}
    int lo = 0, hi = a.n_bounds;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (sb[mid] <= x) lo = mid + 1; else hi = mid;
    }
    sdir[x] = static_cast<uint16_t>(lo);
  }
  if (threadIdx.x == 0) {  // the most edges inside one octave at or above DIRECT: the scan length
    int mx = 0;
    for (int e = DIRECT_LOG2; e < 32; ++e) mx = max(mx, socts[e + 1] - socts[e]);
    sspan = mx;
  }
  __syncthreads();
  const int span = sspan;
  // Each wave takes rows i0 + wave, i0 + wave + 4, ...; lane l computes column j = 64 c + l,
  // so the per-column LDS reads of a wave are consecutive (no bank conflicts) and each store
  // writes 128 contiguous bytes.  The time bucket #{k : b_k <= dt}: gaps below DIRECT
  // seconds (where the edges are dense) read a direct table; above, it lies in
  // [lo_e, lo_(e+1)] for dt in [2^e, 2^(e+1)), lo_e = #{k : b_k < 2^e}, and a scan of at most
  // `span` edges from lo_e finishes it (exact for any non-decreasing edges).
  bf16_t* base = a.rab + a.rab_off[u];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int i1 = min(i0 + RAB_ROWS, L);
  for (int i = i0 + wave; i < i1; i += HT / 64) {
    const int pi = i < 2 * N ? i : 2 * N;
    const int32_t ti = st[i];
    bf16_t* row = base + static_cast<int64_t>(i) * P;
    for (int j = lane; j < P; j += 64) {
      const int jj = min(j, L - 1);
      const int pj = jj < 2 * N ? jj : 2 * N;
      const int dp = min(abs(pi - pj), a.n_pos - 1);
      const int32_t dt = abs(ti - st[jj]);
      int bk;
      if (dt < DIRECT) {
        bk = sdir[dt];
      } else {
        const int e = 31 - __clz(dt);
        bk = socts[e];
        const int hi = socts[e + 1];
        for (int q = 0; q < span; ++q) bk += (bk < hi && sb[min(bk, a.n_bounds - 1)] <= dt) ? 1 : 0;
      }
      const float v = spos[dp] + stime[bk];
      row[j] = f32_to_bf16(j < L ? v : 0.f);
    }
  }
}

}  // namespace

genrank_status launch_hstu_rab_layout(const genrank_batch* b, const int32_t* offsets, int64_t* rab_off,
                                      hipStream_t stream) {
  hipLaunchKernelGGL(hstu_layout_kernel, dim3(1), dim3(HT), 0, stream, offsets, b->B, b->m, rab_off);
  GR_CHECK_LAUNCH();
  return GENRANK_OK;
}

genrank_status launch_hstu_rab(const genrank_batch* b, const int32_t* offsets, const int64_t* ts,
                               const int64_t* req, const float* pos_table, int n_pos,
                               const float* time_table, const int64_t* bounds, int n_time,
                               const int64_t* rab_off, void* rab, hipStream_t stream) {
  if (2 * static_cast<int64_t>(b->max_hist) + b->m > HSTU_MAX_L || n_time - 1 > HSTU_MAX_BOUNDS ||
      n_pos > HSTU_MAX_POS)
    return GENRANK_E_SHAPE;
  RabArgs a{offsets, ts, req, pos_table, time_table, bounds, rab_off, static_cast<bf16_t*>(rab),
            b->m, n_pos, n_time - 1};
  const int Lmax = 2 * b->max_hist + b->m;
  if (Lmax == 0 || b->B == 0) return GENRANK_OK;
  dim3 grid((Lmax + RAB_ROWS - 1) / RAB_ROWS, b->B);
  hipLaunchKernelGGL(hstu_rab_kernel, grid, dim3(HT), 0, stream, a);
  GR_CHECK_LAUNCH();
  return GENRANK_OK;
}

}  // namespace genrank
