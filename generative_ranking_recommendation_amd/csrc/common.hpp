// Shared device helpers for the GenRank gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "genrank.h"

namespace genrank {

typedef uint16_t bf16_t;  // bf16 storage (bit pattern)

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2_t;

// Two floats to packed bf16 with one v_cvt_pk_bf16_f32 (round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return static_cast<bf16_t>(pack_bf16x2(f, 0.f) & 0xFFFFu);
}

// Unpack 8 bf16 held in a uint4 to floats.
__device__ __forceinline__ void unpack8(const uint4& v, float* f) {
  f[0] = __uint_as_float(v.x << 16); f[1] = __uint_as_float(v.x & 0xFFFF0000u);
  f[2] = __uint_as_float(v.y << 16); f[3] = __uint_as_float(v.y & 0xFFFF0000u);
  f[4] = __uint_as_float(v.z << 16); f[5] = __uint_as_float(v.z & 0xFFFF0000u);
  f[6] = __uint_as_float(v.w << 16); f[7] = __uint_as_float(v.w & 0xFFFF0000u);
}

__device__ __forceinline__ uint4 pack8(const float* f) {
  uint4 v;
  v.x = pack_bf16x2(f[0], f[1]);
  v.y = pack_bf16x2(f[2], f[3]);
  v.z = pack_bf16x2(f[4], f[5]);
  v.w = pack_bf16x2(f[6], f[7]);
  return v;
}

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return bf16_to_f32(x); }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) { return f32_to_bf16(x); }

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

// Which user a row belongs to, for rows in the history block: the largest u with
// offsets[u] <= row (binary search over B+1 non-decreasing offsets).
__device__ __forceinline__ int find_user(const int32_t* __restrict__ offsets, int B, int64_t row) {
  int lo = 0, hi = B;  // invariant: offsets[lo] <= row < offsets[hi]
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (static_cast<int64_t>(offsets[mid]) <= row) lo = mid; else hi = mid;
  }
  return lo;
}

// The chip hands workgroup w of a launch to XCD w % 8, and each XCD runs its share in order
// of w / 8.  This maps w to a logical id so that every XCD owns one contiguous range of
// logical ids (the first G % 8 XCDs one id more), walked in order: work items with
// neighbouring logical ids then run on the same XCD at about the same time and share its L2.
// A bijection on [0, G) for every G.
__device__ __forceinline__ int xcd_local_id(int w, int G) {
  const int q = G >> 3, r = G & 7;
  const int x = w & 7, k = w >> 3;
  return x * q + (x < r ? x : r) + k;
}

// The attention mask on one user's sequence slots: 0..N-1 history, N.. candidates.
// History queries see history keys at or before them (every history key with the fully
// visible history variant); a candidate sees all history and itself.  The f32 kernels and
// genrank_debug_mask evaluate this predicate per pair.  The bf16 kernels enforce the same
// rule without it: a history query's key limit (its own slot, or the history's end), keys
// past the history's end given probability 0, and a candidate's own key merged on its own;
// their mask is checked bit for bit by reading it out of their outputs.
__device__ __forceinline__ bool attn_allowed(int i, int j, int N, bool full_history = false) {
  return (i < N) ? (full_history ? j < N : j <= i) : (j < N || j == i);
}

// Bias terms of large magnitude.  The bf16 attention kernels form a pair's ALiBi bias as
// w_j - w_i, the key's and the query's terms relative to one reference point per query block
// (w = s p + s' tau), or seed the scores with w_j alone.  In f32 that is exact to about
// 2^-24 |w|: harmless while |w| stays small, but a history that spans millions of seconds
// puts w_i and w_j both near s' 2^23 while their difference is a few units, and the rounding
// then swamps it.  A query block whose row terms exceed this bound (log2 units) forms every
// bias exactly instead, from the integer position and time differences of the pair; below
// it the error of the separable form is at most 2^-24 * 2^12 = 2^-12 in the exponent.
constexpr float BIAS_FAR_LOG2 = 4096.f;

// #{k : b[k] <= g} for b sorted ascending in p2 entries (a power of two >= the edge count,
// at least 1), the entries past the real edges being INT32_MAX (g < INT32_MAX): a branchless
// binary search over the first p2 - 1 entries, then one compare with the entry it stops at
// (index <= p2 - 1), so that p2 entries count
__device__ __forceinline__ int bucket_search(const int32_t* b, int p2, int32_t g) {
  int pos = 0;
  for (int step = p2 >> 1; step > 0; step >>= 1) pos += (b[pos + step - 1] <= g) ? step : 0;
  return pos + (b[pos] <= g ? 1 : 0);
}
// Bucket table over gaps g in [0, 2^24): one cell per integer below 2^BK_M, then 2^BK_M
// cells per octave [2^e, 2^(e+1)) (the top BK_M bits after the leading one; cell width
// 2^(e - BK_M)).  A cell is one 32-bit word: bits 0-10 lo = #{k : b_k < start}, bit 11 set
// when the cell holds two or more edges, bits 12-30 the offset from the cell's start of
// the one edge inside it (2^19 - 1 if none), so that bucket(g) = lo + (g - start >= offset).
// Dense cells and gaps of 2^24 s or more fall back to bucket_search: exact for any edges.
constexpr int BK_M = 5;
constexpr int BK_CELLS = (25 - BK_M) << BK_M;  // 640
constexpr uint32_t BK_DENSE = 1u << 11, BK_NONE = (1u << 19) - 1;
// fill the table from the padded edges b (p2 entries, visible to every thread; at most 1024
// edges); thread t of nt; the caller synchronises before the first lookup
__device__ __forceinline__ void bucket_table_build(uint32_t* lut, const int32_t* b, int p2, int t, int nt) {
  for (int c = t; c < BK_CELLS; c += nt) {
    int32_t start, width;
    if (c < (1 << BK_M)) {
      start = c;
      width = 1;
    } else {
      const int q = c >> BK_M, r = c & ((1 << BK_M) - 1);
      start = ((1 << BK_M) + r) << (q - 1);
      width = 1 << (q - 1);
    }
    const int lo = bucket_search(b, p2, start - 1);          // #{k : b_k < start}
    const int hi = bucket_search(b, p2, start + width - 1);  // #{k : b_k < end}, end <= 2^24
    const uint32_t off = hi == lo ? BK_NONE : static_cast<uint32_t>(b[lo] - start);  // < 2^18
    lut[c] = static_cast<uint32_t>(lo) | (hi > lo + 1 ? BK_DENSE : 0u) | (off << 12);
  }
}
__device__ __forceinline__ int bucket_lookup(const uint32_t* lut, const int32_t* b, int p2, int32_t g) {
  const uint32_t fb = __float_as_uint(static_cast<float>(g));  // exact below 2^24
  const bool big = g >= (1 << 24);
  const int sh = max(static_cast<int>(fb >> 23) - (127 + BK_M), 0);  // log2 of the cell width
  const int c = g < (1 << BK_M) ? g : static_cast<int>(fb >> (23 - BK_M)) - ((126 + BK_M) << BK_M);
  const uint32_t e = lut[big ? 0 : c];
  const uint32_t low = static_cast<uint32_t>(g) & ((1u << sh) - 1u);  // g - start
  int bk = static_cast<int>(e & 0x7FFu) + (low >= (e >> 12) ? 1 : 0);
  if (big || (e & BK_DENSE)) bk = bucket_search(b, p2, g);
  return bk;
}
// the power of two that bucket_search takes for n edges (n <= ATTN_MAX_TIME_BOUNDS)
inline int bucket_p2(int n) {
  int p2 = 1;
  while (p2 < n) p2 <<= 1;
  return p2;
}
// the same count over int64 edges in global memory (n edges, upper bound search)
__device__ __forceinline__ int bucket_search_global(const int64_t* b, int n, int64_t g) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (b[mid] <= g) lo = mid + 1; else hi = mid;
  }
  return lo;
}
constexpr int ATTN_MAX_TIME_BOUNDS = 1024;

// ---- direct global -> LDS loads and explicit waits (operand rings)
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// vmcnt(n) with every other counter left alone (gfx9 encoding: vmcnt in bits 3:0 and
// 15:14, expcnt 6:4, lgkmcnt 11:8).  On gfx9 vector loads and stores share this counter
// and retire in issue order.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}
// Barrier for LDS filled by direct loads: each wave first waits (vmcnt) for its own loads,
// then all waves meet; the empty asm keeps the compiler from moving memory accesses across.
// It does not wait for the wave's own ds_write instructions: use lds_sync for those.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
// Sets a bit of the device error word (GENRANK_ERR_*); err may be NULL
__device__ __forceinline__ void report_error(uint32_t* err, uint32_t bit) {
  if (err) atomicOr(err, bit);
}
// lgkmcnt(0) with vmcnt and expcnt left alone: the wave's LDS reads and writes are done
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }
// Barrier for ordinary LDS writes and reads (without the vmcnt wait __syncthreads implies)
__device__ __forceinline__ void lds_sync() {
  asm volatile("" ::: "memory");
  wait_lgkm0();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace genrank

#define GR_CHECK_LAUNCH()                                   \
  do {                                                      \
    if (hipGetLastError() != hipSuccess) return GENRANK_E_HIP; \
  } while (0)
