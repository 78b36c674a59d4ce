// Stable LSD radix sort of (key, value) pairs with 32-bit unsigned keys.  The embedding
// backward uses it to group rows by the table row they read (one slice per table).
//
// `slices` independent arrays of n pairs (slice s at [s n, (s + 1) n)) are sorted in the
// same launches by the low `bits` bits of the key, 8 bits per pass.  A pass has three
// kernels:
//   1. per tile of 2048 keys, a histogram of the digit;
//   2. per slice, an exclusive scan over (digit, tile): the first output slot of each
//      tile's keys of each digit;
//   3. per tile, a stable sort of its keys by the digit in LDS (eight 1-bit splits, each a
//      block-wide prefix count), after which a key's output slot is its digit's slot for
//      the tile plus its rank among the tile's keys of that digit.
// Keys of equal digit keep their input order, so the passes compose into a stable sort.
#include <utility>

#include "common.hpp"
#include "internal.hpp"

namespace genrank {

namespace {

constexpr int RT = 256;        // threads per tile
constexpr int RK = 8;          // keys per thread
constexpr int TILE = RT * RK;  // keys per tile
constexpr int RADIX = 256;
constexpr int SCAN_T = 1024;   // threads of the scan kernel

// Exclusive prefix sum over the block (RT threads); *total gets the block's sum.
__device__ __forceinline__ uint32_t excl_scan_block(uint32_t x, uint32_t* sw, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t inc = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(inc, o);
    if (lane >= o) inc += y;
  }
  if (lane == 63) sw[wave] = inc;
  __syncthreads();
  uint32_t pre = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < RT / 64; ++w) {
    pre += w < wave ? sw[w] : 0u;
    tot += sw[w];
  }
  __syncthreads();  // sw may be reused by the next call
  *total = tot;
  return pre + inc - x;
}

__global__ void __launch_bounds__(RT) radix_hist_kernel(const uint32_t* keys, int64_t n, int shift, int ntiles,
                                                        uint32_t* hist) {
  __shared__ uint32_t cnt[RADIX];
  const int s = blockIdx.y, tile = blockIdx.x;
  cnt[threadIdx.x] = 0;
  __syncthreads();
  const uint32_t* k = keys + s * n;
  const int64_t base = static_cast<int64_t>(tile) * TILE;
#pragma unroll
  for (int i = 0; i < RK; ++i) {
    const int64_t p = base + i * RT + threadIdx.x;
    if (p < n) atomicAdd(&cnt[(k[p] >> shift) & (RADIX - 1)], 1u);
  }
  __syncthreads();
  hist[(static_cast<int64_t>(s) * RADIX + threadIdx.x) * ntiles + tile] = cnt[threadIdx.x];
}

// In-place exclusive scan of slice s's RADIX * ntiles counts (digit-major), one workgroup
// per slice.
__global__ void __launch_bounds__(SCAN_T) radix_scan_kernel(uint32_t* hist, int ntiles) {
  __shared__ uint32_t sw[SCAN_T / 64];
  uint32_t* h = hist + static_cast<int64_t>(blockIdx.x) * RADIX * ntiles;
  const int64_t L = static_cast<int64_t>(RADIX) * ntiles;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t carry = 0;
  for (int64_t base = 0; base < L; base += SCAN_T * 4) {
    const int64_t p = base + threadIdx.x * 4;
    uint32_t v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = p + j < L ? h[p + j] : 0u;
    const uint32_t x = v[0] + v[1] + v[2] + v[3];
    uint32_t inc = x;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_up(inc, o);
      if (lane >= o) inc += y;
    }
    if (lane == 63) sw[wave] = inc;
    __syncthreads();
    uint32_t pre = carry, tot = 0;
#pragma unroll
    for (int w = 0; w < SCAN_T / 64; ++w) {
      pre += w < wave ? sw[w] : 0u;
      tot += sw[w];
    }
    uint32_t run = pre + inc - x;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (p + j < L) h[p + j] = run;
      run += v[j];
    }
    carry += tot;
    __syncthreads();
  }
}

__global__ void __launch_bounds__(RT) radix_scatter_kernel(const uint32_t* kin, const uint32_t* vin, uint32_t* kout,
                                                           uint32_t* vout, int64_t n, int shift, int ntiles,
                                                           const uint32_t* hist) {
  __shared__ uint32_t sk[2][TILE];
  __shared__ uint32_t sv[2][TILE];
  __shared__ uint32_t dcnt[RADIX];
  __shared__ uint32_t dstart[RADIX];
  __shared__ uint32_t sw[RT / 64];
  const int s = blockIdx.y, tile = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t base = static_cast<int64_t>(tile) * TILE;
  const int nvalid = static_cast<int>(min<int64_t>(TILE, n - base));
  const uint32_t* ki = kin + s * n + base;
  const uint32_t* vi = vin + s * n + base;

  // thread t holds the tile's keys t*RK .. t*RK + RK - 1 (input order); positions past n
  // get an all-ones key, which has the largest digit and, the sort being stable, stays
  // behind every real key of that digit
  uint32_t k[RK], v[RK];
#pragma unroll
  for (int j = 0; j < RK; ++j) {
    const int i = tid * RK + j;
    k[j] = i < nvalid ? ki[i] : 0xFFFFFFFFu;
    v[j] = i < nvalid ? vi[i] : 0u;
  }
  dcnt[tid] = 0;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < RK; ++j)
    if (tid * RK + j < nvalid) atomicAdd(&dcnt[(k[j] >> shift) & (RADIX - 1)], 1u);
  __syncthreads();
  uint32_t total;
  dstart[tid] = excl_scan_block(dcnt[tid], sw, &total);

  // stable split on each bit of the digit, lowest first
  int buf = 0;
#pragma unroll 1
  for (int b = 0; b < 8; ++b) {
    uint32_t f[RK], zeros = 0;
#pragma unroll
    for (int j = 0; j < RK; ++j) {
      f[j] = (k[j] >> (shift + b)) & 1u;
      zeros += 1u - f[j];
    }
    uint32_t Z;
    uint32_t zr = excl_scan_block(zeros, sw, &Z);
#pragma unroll
    for (int j = 0; j < RK; ++j) {
      const uint32_t i = tid * RK + j;
      const uint32_t pos = f[j] ? Z + (i - zr) : zr;
      zr += 1u - f[j];
      sk[buf][pos] = k[j];
      sv[buf][pos] = v[j];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < RK; ++j) {
      k[j] = sk[buf][tid * RK + j];
      v[j] = sv[buf][tid * RK + j];
    }
    buf ^= 1;
  }
  // sorted tile in sk[buf ^ 1]; write with consecutive threads on consecutive slots
  const uint32_t* hs = hist + static_cast<int64_t>(s) * RADIX * ntiles + tile;
  uint32_t* ko = kout + s * n;
  uint32_t* vo = vout + s * n;
#pragma unroll
  for (int j = 0; j < RK; ++j) {
    const int i = j * RT + tid;
    if (i < nvalid) {
      const uint32_t key = sk[buf ^ 1][i];
      const uint32_t dg = (key >> shift) & (RADIX - 1);
      const uint32_t out = hs[static_cast<int64_t>(dg) * ntiles] + (i - dstart[dg]);
      ko[out] = key;
      vo[out] = sv[buf ^ 1][i];
    }
  }
}

}  // namespace

size_t radix_sort_workspace(int64_t n, int slices) {
  const int64_t ntiles = (n + TILE - 1) / TILE;
  return static_cast<size_t>(slices) * RADIX * static_cast<size_t>(ntiles > 0 ? ntiles : 1) * sizeof(uint32_t);
}

genrank_status launch_radix_sort(uint32_t* keys, uint32_t* vals, uint32_t* tmp_keys, uint32_t* tmp_vals,
                                 int64_t n, int slices, int bits, uint32_t* hist, int* result_in_tmp,
                                 hipStream_t stream) {
  *result_in_tmp = 0;
  if (n <= 0 || slices <= 0) return GENRANK_OK;
  if (n * slices >= (int64_t(1) << 32)) return GENRANK_E_SHAPE;
  const int ntiles = static_cast<int>((n + TILE - 1) / TILE);
  const int passes = bits <= 8 ? 1 : (bits + 7) / 8;
  uint32_t *ki = keys, *vi = vals, *ko = tmp_keys, *vo = tmp_vals;
  for (int p = 0; p < passes; ++p) {
    const int shift = 8 * p;
    hipLaunchKernelGGL(radix_hist_kernel, dim3(ntiles, slices), dim3(RT), 0, stream, ki, n, shift, ntiles, hist);
    hipLaunchKernelGGL(radix_scan_kernel, dim3(slices), dim3(SCAN_T), 0, stream, hist, ntiles);
    hipLaunchKernelGGL(radix_scatter_kernel, dim3(ntiles, slices), dim3(RT), 0, stream, ki, vi, ko, vo, n, shift,
                       ntiles, hist);
    std::swap(ki, ko);
    std::swap(vi, vo);
  }
  *result_in_tmp = passes & 1;
  GR_CHECK_LAUNCH();
  return GENRANK_OK;
}

}  // namespace genrank
