// Dense projections of the GenRank block (QKV, output, FFN): bf16 MFMA GEMM on gfx950.
//
//   C[M, N] = A[M, K] . W[N, K]^T  (+ epilogue), f32 accumulation.
//
// Every bf16 kernel issues v_mfma_f32_16x16x32_bf16 with W rows as the MFMA row operand and
// A rows as the column operand, so each lane ends with 4 consecutive N values of one A row.
// Both operands are K-contiguous and XOR-swizzled in LDS (conflict-free 16-byte fragment
// reads).  C tiles leave through LDS, so that every global store writes whole 16-byte pieces
// of long row runs (measured faster than 16-byte stores straight from the registers, whose
// runs are 64 bytes).  Workgroups are renumbered so that the N tiles of one M tile run on the
// same XCD and share its L2.  The kernels, by shape (launch_gemm_nt picks):
//   gemm_nt_bf16_kernel       128 x 128, 4 waves, operands staged through registers
//   gemm_nt_bf16_dma_kernel   128 x 128, 4 waves, operands loaded straight into LDS
//   gemm_nt_bf16_big_kernel   256 x 256, 8 waves, one workgroup per CU (K >= 512)
//   gemm_nt_bf16_half_kernel  256 x 128, 4 waves, two workgroups per CU (K = 512)
// plus an LDS-tiled FMA kernel for f32 and general strides, and the transposed products of
// the backward pass.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

namespace genrank {

namespace {

constexpr int GBM = 128, GBN = 128, GBK = 32;
constexpr int GTHREADS = 256;
constexpr int BUF_DWORD3 = 0x00020000;  // raw buffer descriptor word 3 (gfx9 family)

struct GemmArgs {
  const bf16_t* A; int64_t lda;
  const bf16_t* W; int64_t ldw;
  void* C; int64_t ldc;
  const void* R; int64_t ldr;     // residual (EPI_RESID: bf16; EPI_RESID_F32: f32), may alias C
  bf16_t* Cpre; int64_t ldpre;    // pre-activation copy (EPI_SILU, optional)
  int M, N, K;
  int nt;                          // outputs far beyond the last-level cache: streaming stores
};

// Outputs larger than the last-level cache (256 MiB) are written with non-temporal stores:
// the next kernel finds them in memory either way, and they leave no dirty cache lines
// behind for later kernels to evict.
constexpr int64_t STREAM_OUT_BYTES = int64_t(256) << 20;

// one 16-byte piece of an output row (wave-uniform choice of the store kind)
__device__ __forceinline__ void store16(void* p, const uint4& v, bool nt) {
  if (nt)
    __builtin_nontemporal_store(__builtin_bit_cast(f32x4_t, v), reinterpret_cast<f32x4_t*>(p));
  else
    *reinterpret_cast<uint4*>(p) = v;
}

// sigmoid through the hardware reciprocal (about 1 ulp) rather than a full-precision
// division; exp(-a) = inf for very negative a gives 1 / inf = 0, the right limit
__device__ __forceinline__ float sigmoid_f(float a) { return __builtin_amdgcn_rcpf(1.0f + __expf(-a)); }
__device__ __forceinline__ float silu_f(float x) { return x * sigmoid_f(x); }
// d silu(a) / da = s (1 + a (1 - s)), s = sigmoid(a)
__device__ __forceinline__ float dsilu_f(float a) {
  const float sg = sigmoid_f(a);
  return sg * (1.0f + a * (1.0f - sg));
}

// LDS operand tile: [rows][32 bf16] = 64 B per row, four 16-byte chunks.  Chunk c of row r
// is stored at slot c ^ swz_row(r), swz_row(r) = (r >> 2) & 3: the 16-byte reads of 16
// consecutive rows at one chunk (an MFMA operand fragment) fall on 16 distinct 16-byte slots
// of the 64-bank LDS (4 rows of 64 B span its 256 bytes; the XOR spreads the 4 row groups
// over the 4 chunks), and so do the 16-byte writes of the staging pattern.  A 16-row block
// keeps its swizzle under any offset that is a multiple of 16.
__device__ __forceinline__ int swz_row(int r) { return (r >> 2) & 3; }
__device__ __forceinline__ int swz(int r, int c) { return r * GBK + ((c ^ swz_row(r)) << 3); }

constexpr int CP = GBN + 8;                           // staged C row pitch (bf16)
constexpr int SMEM_OPS = 2 * 2 * GBM * GBK;           // [stage][A|W] operand tiles
constexpr int SMEM = SMEM_OPS > GBM * CP ? SMEM_OPS : GBM * CP;

// ---- element-wise epilogue math on C[m][n .. n+3] (in f32, before the bf16 store)
template <int EPI>
__device__ __forceinline__ void epi_math(const GemmArgs& g, int m, int n, float (&v)[4]) {
  if constexpr (EPI == GEMM_EPI_RESID) {
    if (m < g.M) {
      const uint2 r = *reinterpret_cast<const uint2*>(static_cast<const bf16_t*>(g.R) + static_cast<int64_t>(m) * g.ldr + n);
      v[0] += __uint_as_float(r.x << 16); v[1] += __uint_as_float(r.x & 0xFFFF0000u);
      v[2] += __uint_as_float(r.y << 16); v[3] += __uint_as_float(r.y & 0xFFFF0000u);
    }
  }
  if constexpr (EPI == GEMM_EPI_DSILU) {
    if (m < g.M) {
      const uint2 r = *reinterpret_cast<const uint2*>(static_cast<const bf16_t*>(g.R) + static_cast<int64_t>(m) * g.ldr + n);
      v[0] *= dsilu_f(__uint_as_float(r.x << 16)); v[1] *= dsilu_f(__uint_as_float(r.x & 0xFFFF0000u));
      v[2] *= dsilu_f(__uint_as_float(r.y << 16)); v[3] *= dsilu_f(__uint_as_float(r.y & 0xFFFF0000u));
    }
  }
  if constexpr (EPI == GEMM_EPI_SILU) {
    if (g.Cpre && m < g.M) {
      uint2 p;
      p.x = pack_bf16x2(v[0], v[1]);
      p.y = pack_bf16x2(v[2], v[3]);
      *reinterpret_cast<uint2*>(g.Cpre + static_cast<int64_t>(m) * g.ldpre + n) = p;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = silu_f(v[i]);
  }
}

// f32 output rows straight from the MFMA layout (a lane's 4 consecutive columns of one row are
// one 16-byte store; four lanes cover 64 contiguous bytes of a row): EPI_F32 stores the
// accumulator, EPI_RESID_F32 adds the f32 residual first (read by the same lane before its store,
// so R may alias C).
template <int EPI>
__device__ __forceinline__ void store_f32(const GemmArgs& g, int m, int n, const float (&v)[4]) {
  float4 o = make_float4(v[0], v[1], v[2], v[3]);
  if constexpr (EPI == GEMM_EPI_RESID_F32) {
    const float4 r = *reinterpret_cast<const float4*>(static_cast<const float*>(g.R) + static_cast<int64_t>(m) * g.ldr + n);
    o.x += r.x; o.y += r.y; o.z += r.z; o.w += r.w;
  }
  *reinterpret_cast<float4*>(static_cast<float*>(g.C) + static_cast<int64_t>(m) * g.ldc + n) = o;
}

// ---- epilogue shared by the MFMA kernels: lane holds C[m][n .. n+3] for each (nb, mb).
// The 128 x 128 tile (after the epilogue math, in the output dtype) is staged through LDS,
// rows 0-63 at sC_lo and rows 64-127 at sC_hi (pitch CP), so that every global store is a
// 16-byte piece of a row.  The caller guarantees that no wave still reads those buffers.
template <int EPI>
__device__ __forceinline__ void epilogue(const GemmArgs& g, const f32x4_t (&acc)[4][4], bf16_t* sC_lo,
                                         bf16_t* sC_hi, int m0, int n0, int wm, int wn, int l16, int g4,
                                         int tid) {
  if constexpr (EPI == GEMM_EPI_F32 || EPI == GEMM_EPI_RESID_F32) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int m = m0 + wm * 64 + mb * 16 + l16;
      if (m >= g.M) continue;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const float v[4] = {acc[nb][mb][0], acc[nb][mb][1], acc[nb][mb][2], acc[nb][mb][3]};
        store_f32<EPI>(g, m, n0 + wn * 64 + nb * 16 + g4 * 4, v);
      }
    }
    return;
  }
  bf16_t* sCw = wm ? sC_hi : sC_lo;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const int ml = wm * 64 + mb * 16 + l16;
    const int m = m0 + ml;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int nl = wn * 64 + nb * 16 + g4 * 4;
      const int n = n0 + nl;
      float v[4] = {acc[nb][mb][0], acc[nb][mb][1], acc[nb][mb][2], acc[nb][mb][3]};
      epi_math<EPI>(g, m, n, v);
      uint2 o;
      o.x = pack_bf16x2(v[0], v[1]);
      o.y = pack_bf16x2(v[2], v[3]);
      *reinterpret_cast<uint2*>(sCw + (mb * 16 + l16) * CP + nl) = o;
    }
  }
  __syncthreads();
  // 128 rows x 256 B: 16 threads per row, 16 rows per pass
  bf16_t* C = static_cast<bf16_t*>(g.C);
#pragma unroll
  for (int pass = 0; pass < GBM / 16; ++pass) {
    const int ml = pass * 16 + (tid >> 4);
    const int m = m0 + ml;
    if (m >= g.M) continue;
    const int nl = (tid & 15) * 8;
    const bf16_t* src = (ml < 64 ? sC_lo : sC_hi) + (ml & 63) * CP + nl;
    store16(C + static_cast<int64_t>(m) * g.ldc + n0 + nl, *reinterpret_cast<const uint4*>(src), g.nt);
  }
}

template <int EPI>
__global__ void __launch_bounds__(GTHREADS) gemm_nt_bf16_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) bf16_t smem[SMEM];  // operands, then the C tile
  // stage st: A tile at smem + st * 2 * GBM * GBK, W tile right after it
  auto sA = [&](int st) { return smem + st * (2 * GBM * GBK); };
  auto sW = [&](int st) { return smem + st * (2 * GBM * GBK) + GBM * GBK; };

  // XCD-aware renumbering: hardware hands workgroup w to XCD w % 8; give the tiles of
  // one M row-block consecutive logical ids on the same XCD.
  const int nN = g.N / GBN;
  const int nM = (g.M + GBM - 1) / GBM;
  const int G = nN * nM;
  const int L = xcd_local_id(blockIdx.x, G);
  const int mblk = L / nN;
  const int nblk = L - mblk * nN;
  const int m0 = mblk * GBM;
  const int n0 = nblk * GBN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int l16 = lane & 15, g4 = lane >> 4;

  // Buffer descriptors over this tile's rows: rows past M read as zero.
  const uint64_t a_rows = static_cast<uint64_t>(g.M - m0);
  const uint32_t a_bytes = static_cast<uint32_t>(min<uint64_t>(a_rows * g.lda * 2u, 0xFFFFFFF0ull));
  const __amdgpu_buffer_rsrc_t rsA = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t*>(g.A + static_cast<int64_t>(m0) * g.lda), static_cast<short>(0), a_bytes, BUF_DWORD3);
  const __amdgpu_buffer_rsrc_t rsW = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t*>(g.W + static_cast<int64_t>(n0) * g.ldw), static_cast<short>(0),
      static_cast<uint32_t>(GBN * g.ldw * 2), BUF_DWORD3);
  // staging: thread moves rows srow and srow + 64, chunk sc (16 B) of A and of W
  const int srow = tid >> 2, sc = tid & 3;
  const uint32_t voA0 = static_cast<uint32_t>(srow * g.lda + sc * 8) * 2u;
  const uint32_t voA1 = voA0 + static_cast<uint32_t>(64 * g.lda * 2);
  const uint32_t voW0 = static_cast<uint32_t>(srow * g.ldw + sc * 8) * 2u;
  const uint32_t voW1 = voW0 + static_cast<uint32_t>(64 * g.ldw * 2);
  uint4 ra0, ra1, rw0, rw1;
  auto fetch = [&](int k0) {
    const uint32_t so = static_cast<uint32_t>(k0) * 2u;
    ra0 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsA, voA0, so, 0));
    ra1 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsA, voA1, so, 0));
    rw0 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsW, voW0, so, 0));
    rw1 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsW, voW1, so, 0));
  };
  auto stash = [&](int st) {
    *reinterpret_cast<uint4*>(sA(st) + swz(srow, sc)) = ra0;
    *reinterpret_cast<uint4*>(sA(st) + swz(srow + 64, sc)) = ra1;
    *reinterpret_cast<uint4*>(sW(st) + swz(srow, sc)) = rw0;
    *reinterpret_cast<uint4*>(sW(st) + swz(srow + 64, sc)) = rw1;
  };

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nk = g.K / GBK;
  fetch(0);
  stash(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < nk) fetch((kt + 1) * GBK);
    bf16x8_t fw[4], fa[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
      fw[nb] = as_bf16x8(*reinterpret_cast<const uint4*>(sW(st) + swz(wn * 64 + nb * 16 + l16, g4)));
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
      fa[mb] = as_bf16x8(*reinterpret_cast<const uint4*>(sA(st) + swz(wm * 64 + mb * 16 + l16, g4)));
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        acc[nb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fw[nb], fa[mb], acc[nb][mb], 0, 0, 0);
    if (kt + 1 < nk) stash(st ^ 1);
    __syncthreads();
  }

  epilogue<EPI>(g, acc, smem, smem + 64 * CP, m0, n0, wm, wn, l16, g4, tid);
}

// ------------------------------------------------------------------ pipelined MFMA GEMM
// Same tile, waves and epilogue as gemm_nt_bf16_kernel, for K a multiple of 4 * GBK.  The
// operand tiles go from global memory straight into LDS (one 16-byte direct load per lane:
// lane l of a wave fills bytes 16 l .. 16 l + 15 of a 1 KB block, so the XOR swizzle is
// applied by choosing which 16-byte chunk each lane fetches), through a ring of four stage
// buffers with three stages in flight.  No registers are spent on staging and each
// workgroup waits for memory about once instead of once per K tile.  Each stage buffer is
// its own LDS array and the ring is unrolled, so the compiler can tell the stage being read
// from the stages in flight and keeps the waits partial; the waits and barriers are
// explicit.  Two stage buffers (each sized for 64 rows of the C tile) hold the C tile in
// the epilogue.
constexpr int DSTAGE_ELEMS = 64 * CP;  // bf16 per stage buffer: A and W tiles, or half of C
static_assert(2 * GBM * GBK <= DSTAGE_ELEMS, "stage buffer holds an A and a W tile");


template <int EPI>
__global__ void __launch_bounds__(GTHREADS) gemm_nt_bf16_dma_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) bf16_t st0[DSTAGE_ELEMS];
  __shared__ __attribute__((aligned(16))) bf16_t st1[DSTAGE_ELEMS];
  __shared__ __attribute__((aligned(16))) bf16_t st2[DSTAGE_ELEMS];
  __shared__ __attribute__((aligned(16))) bf16_t st3[DSTAGE_ELEMS];

  const int nN = g.N / GBN;
  const int nM = (g.M + GBM - 1) / GBM;
  const int L = xcd_local_id(blockIdx.x, nN * nM);
  const int mblk = L / nN;
  const int m0 = mblk * GBM;
  const int n0 = (L - mblk * nN) * GBN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int l16 = lane & 15, g4 = lane >> 4;

  // direct loads: wave w fills rows 32 w .. 32 w + 31 of the A tile and of the W tile, 16
  // rows (1 KB) per load; lane -> row r = r0 + lane / 4, LDS chunk lane % 4, which holds
  // global chunk (lane % 4) ^ swz_row(r).  A rows past M re-read row M - 1 (never stored).
  const int lr = lane >> 2, ls = lane & 3;
  const int r0 = wave * 32 + lr, r1 = r0 + 16;
  const int c0 = ls ^ swz_row(r0), c1 = ls ^ swz_row(r1);
  const bf16_t* gA0 = g.A + static_cast<int64_t>(min(m0 + r0, g.M - 1)) * g.lda + c0 * 8;
  const bf16_t* gA1 = g.A + static_cast<int64_t>(min(m0 + r1, g.M - 1)) * g.lda + c1 * 8;
  const bf16_t* gW0 = g.W + static_cast<int64_t>(n0 + r0) * g.ldw + c0 * 8;
  const bf16_t* gW1 = g.W + static_cast<int64_t>(n0 + r1) * g.ldw + c1 * 8;
  const int dA0 = wave * 32 * GBK, dA1 = dA0 + 16 * GBK;  // LDS block offsets (elements)
  auto load = [&](int kt, bf16_t* stg) {
    const int k0 = kt * GBK;
    __builtin_amdgcn_global_load_lds((glb_void_t*)(gA0 + k0), (lds_void_t*)(stg + dA0), 16, 0, 0);
    __builtin_amdgcn_global_load_lds((glb_void_t*)(gA1 + k0), (lds_void_t*)(stg + dA1), 16, 0, 0);
    __builtin_amdgcn_global_load_lds((glb_void_t*)(gW0 + k0), (lds_void_t*)(stg + GBM * GBK + dA0), 16, 0, 0);
    __builtin_amdgcn_global_load_lds((glb_void_t*)(gW1 + k0), (lds_void_t*)(stg + GBM * GBK + dA1), 16, 0, 0);
  };

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const bf16_t* stg) {
    bf16x8_t fw[4], fa[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
      fw[nb] = as_bf16x8(*reinterpret_cast<const uint4*>(stg + GBM * GBK + swz(wn * 64 + nb * 16 + l16, g4)));
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
      fa[mb] = as_bf16x8(*reinterpret_cast<const uint4*>(stg + swz(wm * 64 + mb * 16 + l16, g4)));
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        acc[nb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fw[nb], fa[mb], acc[nb][mb], 0, 0, 0);
  };

  // K tile kt sits in stage buffer kt % 4.  A step waits until its own tile has landed (the
  // two newer tiles may stay in flight: 4 loads each), synchronises, refills the buffer the
  // previous step read with tile kt + 3, and multiplies.
  const int nk = g.K / GBK;  // a multiple of 4
  load(0, st0);
  load(1, st1);
  load(2, st2);
  int kt = 0;
  for (; kt + 4 < nk; kt += 4) {
    wait_vmcnt<8>(); lds_barrier(); load(kt + 3, st3); compute(st0);
    wait_vmcnt<8>(); lds_barrier(); load(kt + 4, st0); compute(st1);
    wait_vmcnt<8>(); lds_barrier(); load(kt + 5, st1); compute(st2);
    wait_vmcnt<8>(); lds_barrier(); load(kt + 6, st2); compute(st3);
  }
  // the last four tiles: only tile nk - 1 is still to be requested
  wait_vmcnt<8>(); lds_barrier(); load(kt + 3, st3); compute(st0);
  wait_vmcnt<8>(); lds_barrier(); compute(st1);
  wait_vmcnt<4>(); lds_barrier(); compute(st2);
  wait_vmcnt<0>(); lds_barrier(); compute(st3);
  lds_barrier();  // every wave is done with the stage buffers before C goes into st0 / st1

  epilogue<EPI>(g, acc, st0, st1, m0, n0, wm, wn, l16, g4, tid);
}

// ------------------------------------------------------------------ 256 x 256 tiles
// For the MFMA-bound shapes (K >= 512): the same direct-load ring with 256 x 256 tiles and
// 8 waves in a 2 (M) x 4 (N) grid, each wave 128 x 64 (32 MFMAs per K tile).  Per K tile a
// wave reads 12 KB of operands from LDS for 32 MFMAs, against 8 KB for 16 with 64 x 64
// waves, so LDS traffic no longer matches the MFMA time.  One workgroup per CU (four
// 33 KB stage buffers); the C tile is staged through all four buffers, 64 rows each.
constexpr int BBM = 256, BBN = 256, BTHREADS = 512;
constexpr int BCP = BBN + 8;  // staged C row pitch (bf16)
constexpr int BSTAGE_ELEMS = (2 * BBM * GBK > 64 * BCP) ? 2 * BBM * GBK : 64 * BCP;

// RMS: the A rows are raw inputs x and W is the weight with the RMSNorm gain folded into its
// columns (W g); the kernel forms each row's r = 1 / sqrt(mean(x^2) + eps) from the A tiles
// it already holds in LDS (thread t sums the squares of half of row t / 2 of every K tile,
// in K order, and a lane pair adds its halves) and scales the row by r before the
// epilogue: rmsnorm(x) g . W^T = r (x . (W g)^T).  A row's r depends only on that row.
template <int EPI, bool RMS>
__global__ void __launch_bounds__(BTHREADS) gemm_nt_bf16_big_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) bf16_t st0[BSTAGE_ELEMS];
  __shared__ __attribute__((aligned(16))) bf16_t st1[BSTAGE_ELEMS];
  __shared__ __attribute__((aligned(16))) bf16_t st2[BSTAGE_ELEMS];
  __shared__ __attribute__((aligned(16))) bf16_t st3[BSTAGE_ELEMS];
  __shared__ float sR[RMS ? BBM : 1];

  const int nN = g.N / BBN;
  const int nM = (g.M + BBM - 1) / BBM;
  const int L = xcd_local_id(blockIdx.x, nN * nM);
  const int mblk = L / nN;
  const int m0 = mblk * BBM;
  const int n0 = (L - mblk * nN) * BBN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int l16 = lane & 15, g4 = lane >> 4;

  // direct loads as in gemm_nt_bf16_dma_kernel: wave w fills rows 32 w .. 32 w + 31 of the
  // A tile and of the W tile (256 rows each), 16 rows (1 KB) per load
  const int lr = lane >> 2, ls = lane & 3;
  const int r0 = wave * 32 + lr, r1 = r0 + 16;
  const int c0 = ls ^ swz_row(r0), c1 = ls ^ swz_row(r1);
  const bf16_t* gA0 = g.A + static_cast<int64_t>(min(m0 + r0, g.M - 1)) * g.lda + c0 * 8;
  const bf16_t* gA1 = g.A + static_cast<int64_t>(min(m0 + r1, g.M - 1)) * g.lda + c1 * 8;
  const bf16_t* gW0 = g.W + static_cast<int64_t>(n0 + r0) * g.ldw + c0 * 8;
  const bf16_t* gW1 = g.W + static_cast<int64_t>(n0 + r1) * g.ldw + c1 * 8;
  const int dA0 = wave * 32 * GBK, dA1 = dA0 + 16 * GBK;
  auto load = [&](int kt, bf16_t* stg) {
    const int k0 = kt * GBK;
    __builtin_amdgcn_global_load_lds((glb_void_t*)(gA0 + k0), (lds_void_t*)(stg + dA0), 16, 0, 0);
    __builtin_amdgcn_global_load_lds((glb_void_t*)(gA1 + k0), (lds_void_t*)(stg + dA1), 16, 0, 0);
    __builtin_amdgcn_global_load_lds((glb_void_t*)(gW0 + k0), (lds_void_t*)(stg + BBM * GBK + dA0), 16, 0, 0);
    __builtin_amdgcn_global_load_lds((glb_void_t*)(gW1 + k0), (lds_void_t*)(stg + BBM * GBK + dA1), 16, 0, 0);
  };

  f32x4_t acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int rr = tid >> 1, rc = (tid & 1) * 2;  // RMS: this thread's row and first chunk
  float ss = 0.f;
  // a wave's operand fragments of one K tile: 4 W blocks and 8 A blocks of 16 rows
  auto read_w = [&](const bf16_t* stg, int nb) {
    return as_bf16x8(*reinterpret_cast<const uint4*>(stg + BBM * GBK + swz(wn * 64 + nb * 16 + l16, g4)));
  };
  auto read_a = [&](const bf16_t* stg, int mb) {
    return as_bf16x8(*reinterpret_cast<const uint4*>(stg + swz(wm * 128 + mb * 16 + l16, g4)));
  };

  const int nk = g.K / GBK;  // a multiple of 4, at least 16
  if constexpr (RMS) {
    // the row sums of squares need registers the pipelined schedule below does not leave:
    // stage s is read and multiplied in step s, three stages in flight
    auto compute = [&](const bf16_t* stg) {
      float x[8];
      unpack8(*reinterpret_cast<const uint4*>(stg + swz(rr, rc)), x);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
      unpack8(*reinterpret_cast<const uint4*>(stg + swz(rr, rc + 1)), x);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
      bf16x8_t fw[4], fa[8];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) fw[nb] = read_w(stg, nb);
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) fa[mb] = read_a(stg, mb);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int mb = 0; mb < 8; ++mb)
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fw[nb], fa[mb], acc[nb][mb], 0, 0, 0);
    };
    load(0, st0);
    load(1, st1);
    load(2, st2);
    int kt = 0;
    for (; kt + 4 < nk; kt += 4) {
      wait_vmcnt<8>(); lds_barrier(); load(kt + 3, st3); compute(st0);
      wait_vmcnt<8>(); lds_barrier(); load(kt + 4, st0); compute(st1);
      wait_vmcnt<8>(); lds_barrier(); load(kt + 5, st1); compute(st2);
      wait_vmcnt<8>(); lds_barrier(); load(kt + 6, st2); compute(st3);
    }
    wait_vmcnt<8>(); lds_barrier(); load(kt + 3, st3); compute(st0);
    wait_vmcnt<8>(); lds_barrier(); compute(st1);
    wait_vmcnt<4>(); lds_barrier(); compute(st2);
    wait_vmcnt<0>(); lds_barrier(); compute(st3);
  } else {
    // Stage s of the K loop lives in buffer s % 4.  Step s multiplies the fragments of
    // stage s, already in registers, and refills those registers with stage s + 1 as they
    // free up: the W blocks into spare registers first, then A block mb right after the
    // four MFMAs that read A block mb.  So each wave's LDS reads run under its own MFMAs and
    // are spread over the step.  At the start of step s every wave has waited for its
    // loads of stage s + 1 and for its reads of stage s (lds_sync): after the barrier stage
    // s + 1 is complete in LDS and buffer s % 4 is free for stage s + 4.
    bf16x8_t fw[4], fa[8];
    using Yes = std::true_type;
    using No = std::false_type;
    auto step = [&](auto vm, auto do_load, auto do_read, bf16_t* ld_buf, int ld_kt, const bf16_t* rd_buf) {
      constexpr bool LOAD = decltype(do_load)::value, READ = decltype(do_read)::value;
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (READ) {
        wait_vmcnt<decltype(vm)::value>();
        if constexpr (LOAD) lds_sync(); else lds_barrier();
      }
      if constexpr (LOAD) load(ld_kt, ld_buf);
      bf16x8_t wnx[4];
      if constexpr (READ) {
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) wnx[nb] = read_w(rd_buf, nb);
      }
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) {
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fw[nb], fa[mb], acc[nb][mb], 0, 0, 0);
        if constexpr (READ) fa[mb] = read_a(rd_buf, mb);
      }
      if constexpr (READ) {
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) fw[nb] = wnx[nb];
        // 4 W reads, then 8 x (4 MFMAs, 1 A read)
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) {
          __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      }
    };
    load(0, st0);
    load(1, st1);
    load(2, st2);
    load(3, st3);
    wait_vmcnt<12>();
    lds_barrier();
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) fw[nb] = read_w(st0, nb);
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) fa[mb] = read_a(st0, mb);
    using V8 = std::integral_constant<int, 8>;
    using V4 = std::integral_constant<int, 4>;
    using V0 = std::integral_constant<int, 0>;
    int kt = 0;
    for (; kt + 4 < nk; kt += 4) {
      step(V8{}, Yes{}, Yes{}, st0, kt + 4, st1);
      step(V8{}, Yes{}, Yes{}, st1, kt + 5, st2);
      step(V8{}, Yes{}, Yes{}, st2, kt + 6, st3);
      step(V8{}, Yes{}, Yes{}, st3, kt + 7, st0);
    }
    step(V8{}, No{}, Yes{}, st0, 0, st1);
    step(V4{}, No{}, Yes{}, st0, 0, st2);
    step(V0{}, No{}, Yes{}, st0, 0, st3);
    step(V0{}, No{}, No{}, st0, 0, st0);
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (RMS) {
    ss += __shfl_xor(ss, 1);
    if ((tid & 1) == 0) sR[rr] = rsqrtf(ss / static_cast<float>(g.K) + RMS_EPS);
    lds_sync();  // sR written; every wave is done with the stage buffers
  } else {
    lds_barrier();  // every wave is done with the stage buffers before C goes into them
  }

  if constexpr (EPI == GEMM_EPI_RESID_F32) {
    // f32 rows through LDS, one half of the tile (128 rows, the waves with wm = half) at a
    // time: those waves write their 128 x 64 blocks (stage buffer q holds rows 32 q ..
    // 32 q + 31 of the half, pitch FCP floats), then every wave adds the residual to whole
    // rows and stores them, lane l on columns 4 l .. 4 l + 3, so that each access of a wave
    // is one contiguous 1 KB span.  A residual element is read by the lane that stores its
    // sum, so R may alias C.
    static_assert(!RMS, "the RMSNorm-folded kernel has no f32 residual epilogue");
    constexpr int FCP = BBN + 4;
    static_assert(32 * FCP * 4 <= BSTAGE_ELEMS * 2, "32 f32 rows per stage buffer");
    auto fb = [&](int q) -> float* {
      return reinterpret_cast<float*>(q == 0 ? st0 : (q == 1 ? st1 : (q == 2 ? st2 : st3)));
    };
    const float* Rp = static_cast<const float*>(g.R);
    float* Cp = static_cast<float*>(g.C);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      // the residual rows this wave adds (rows wave, wave + 8, ... of the half): the first
      // eight in flight before the tile half goes through LDS, each later one issued as an
      // earlier one is consumed (rows past M re-read row M - 1)
      auto rrow = [&](int i) {
        const int m = min(m0 + half * 128 + wave + 8 * i, g.M - 1);
        return *reinterpret_cast<const f32x4_t*>(Rp + static_cast<int64_t>(m) * g.ldr + n0 + lane * 4);
      };
      f32x4_t rv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) rv[i] = rrow(i);
      if (wm == half) {
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) {
          float* rowp = fb(mb >> 1) + ((mb & 1) * 16 + l16) * FCP + wn * 64 + g4 * 4;
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) *reinterpret_cast<f32x4_t*>(rowp + nb * 16) = acc[nb][mb];
        }
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int rr = wave + 8 * i;
        const int m = m0 + half * 128 + rr;
        const f32x4_t r = rv[i & 7];
        if (i < 8) rv[i] = rrow(i + 8);
        if (m < g.M) {
          const f32x4_t v = *reinterpret_cast<const f32x4_t*>(fb(rr >> 5) + (rr & 31) * FCP + lane * 4) + r;
          store16(Cp + static_cast<int64_t>(m) * g.ldc + n0 + lane * 4, __builtin_bit_cast(uint4, v), g.nt);
        }
      }
      __syncthreads();
    }
    return;
  }
  // epilogue: rows 64 q .. 64 q + 63 of the C tile in buffer q; a wave's rows
  // wm * 128 + mb * 16 + l16 fall in buffers 2 wm (mb < 4) and 2 wm + 1
  bf16_t* cb_lo = wm ? st2 : st0;
  bf16_t* cb_hi = wm ? st3 : st1;
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) {
    const int ml = wm * 128 + mb * 16 + l16;
    const int m = m0 + ml;
    bf16_t* cb = mb < 4 ? cb_lo : cb_hi;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int nl = wn * 64 + nb * 16 + g4 * 4;
      float v[4] = {acc[nb][mb][0], acc[nb][mb][1], acc[nb][mb][2], acc[nb][mb][3]};
      if constexpr (RMS) {
        const float r = sR[ml];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] *= r;
      }
      epi_math<EPI>(g, m, n0 + nl, v);
      uint2 o;
      o.x = pack_bf16x2(v[0], v[1]);
      o.y = pack_bf16x2(v[2], v[3]);
      *reinterpret_cast<uint2*>(cb + (ml & 63) * BCP + nl) = o;
    }
  }
  __syncthreads();
  // 256 rows x 512 B: 32 threads per row, 16 rows per pass
  bf16_t* C = static_cast<bf16_t*>(g.C);
#pragma unroll
  for (int pass = 0; pass < BBM / 16; ++pass) {
    const int ml = pass * 16 + (tid >> 5);
    const int m = m0 + ml;
    if (m >= g.M) continue;
    const int nl = (tid & 31) * 8;
    const bf16_t* cb = pass < 4 ? st0 : (pass < 8 ? st1 : (pass < 12 ? st2 : st3));
    store16(C + static_cast<int64_t>(m) * g.ldc + n0 + nl, *reinterpret_cast<const uint4*>(cb + (ml & 63) * BCP + nl),
            g.nt);
  }
}

// ------------------------------------------------------------------ 256 x 128 tiles, two per CU
// The 256 x 256 kernel's operand path with half the tile width: 4 waves in a 2 (M) x 2 (N)
// grid, each 128 x 64, and a three-stage ring of 24 KB stages (72 KB of LDS), so that two
// workgroups share each CU.  With one workgroup per CU every CU runs its K loop, then its
// epilogue, in step with the others, so the MFMAs idle while the whole chip stores C and
// HBM idles while it multiplies; with two, one workgroup's epilogue, prologue and barrier
// waits run under the other's MFMAs.
constexpr int HBM = 256, HBN = 128, HTHREADS = 256;
constexpr int HSTAGE = (HBM + HBN) * GBK;  // bf16 per stage: the A tile, then the W tile
constexpr int HCP = HBN + 8;               // staged bf16 C row pitch
constexpr int HFCP = HBN + 4;              // staged f32 C row pitch (half a tile at a time)
static_assert(3 * HSTAGE >= HBM * HCP, "the bf16 C tile fits the stage buffers");
static_assert(3 * HSTAGE * 2 >= (HBM / 2) * HFCP * 4, "half the f32 C tile fits the stage buffers");

template <int EPI>
__global__ void __launch_bounds__(HTHREADS, 2) gemm_nt_bf16_half_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) bf16_t sm[3 * HSTAGE];

  const int nN = g.N / HBN;
  const int nM = (g.M + HBM - 1) / HBM;
  const int L = xcd_local_id(blockIdx.x, nN * nM);
  const int mblk = L / nN;
  const int m0 = mblk * HBM;
  const int n0 = (L - mblk * nN) * HBN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int l16 = lane & 15, g4 = lane >> 4;

  // direct loads: wave w fills A rows 64 w .. 64 w + 63 and W rows 32 w .. 32 w + 31 of a
  // stage, 16 rows (1 KB) per load; lane (lr, ls) loads chunk ls ^ swz_row(lr) of its row,
  // which lands in slot ls (the swizzle of swz(); the row's bits from 4 up do not enter)
  const int lr = lane >> 2, ls = lane & 3;
  const int ck = (ls ^ swz_row(lr)) * 8;
  const bf16_t* gA[4];
  const bf16_t* gW[2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    gA[i] = g.A + static_cast<int64_t>(min(m0 + wave * 64 + i * 16 + lr, g.M - 1)) * g.lda + ck;
#pragma unroll
  for (int i = 0; i < 2; ++i) gW[i] = g.W + static_cast<int64_t>(n0 + wave * 32 + i * 16 + lr) * g.ldw + ck;
  auto load = [&](int kt, bf16_t* stg) {
    const int k0 = kt * GBK;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_global_load_lds((glb_void_t*)(gA[i] + k0), (lds_void_t*)(stg + (wave * 64 + i * 16) * GBK), 16,
                                       0, 0);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      __builtin_amdgcn_global_load_lds((glb_void_t*)(gW[i] + k0),
                                       (lds_void_t*)(stg + HBM * GBK + (wave * 32 + i * 16) * GBK), 16, 0, 0);
  };
  auto read_w = [&](const bf16_t* stg, int nb) {
    return as_bf16x8(*reinterpret_cast<const uint4*>(stg + HBM * GBK + swz(wn * 64 + nb * 16 + l16, g4)));
  };
  auto read_a = [&](const bf16_t* stg, int mb) {
    return as_bf16x8(*reinterpret_cast<const uint4*>(stg + swz(wm * 128 + mb * 16 + l16, g4)));
  };

  f32x4_t acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Stage s lives in buffer s % 3.  Step s multiplies the fragments of stage s, already in
  // registers, and refills those registers with stage s + 1 as they free up (the W blocks
  // into spare registers, A block mb right after its four MFMAs).  At the start of step s
  // every wave has waited for its loads of stage s + 1 and its reads of stage s (lds_sync),
  // so after the barrier stage s + 1 is complete and buffer s % 3 is free for stage s + 3.
  bf16x8_t fw[4], fa[8];
  auto mma_read = [&](const bf16_t* rd, auto do_read) {
    constexpr bool READ = decltype(do_read)::value;
    bf16x8_t wnx[4];
    if constexpr (READ) {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) wnx[nb] = read_w(rd, nb);
    }
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        acc[nb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fw[nb], fa[mb], acc[nb][mb], 0, 0, 0);
      if constexpr (READ) fa[mb] = read_a(rd, mb);
    }
    if constexpr (READ) {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) fw[nb] = wnx[nb];
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) {
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
  };
  const int nk = g.K / GBK;  // at least 4
  load(0, sm);
  load(1, sm + HSTAGE);
  load(2, sm + 2 * HSTAGE);
  wait_vmcnt<12>();
  lds_barrier();
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) fw[nb] = read_w(sm, nb);
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) fa[mb] = read_a(sm, mb);
  int bl = 0;  // buffer of stage s
  for (int kt = 0; kt + 3 < nk; ++kt) {
    const int br = bl == 2 ? 0 : bl + 1;
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<6>();
    lds_sync();
    load(kt + 3, sm + bl * HSTAGE);
    mma_read(sm + br * HSTAGE, std::true_type{});
    __builtin_amdgcn_sched_barrier(0);
    bl = br;
  }
  // the last three stages: nothing more to load
  {
    const int b1 = bl == 2 ? 0 : bl + 1, b2 = b1 == 2 ? 0 : b1 + 1;
    wait_vmcnt<6>();
    lds_barrier();
    mma_read(sm + b1 * HSTAGE, std::true_type{});
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<0>();
    lds_barrier();
    mma_read(sm + b2 * HSTAGE, std::true_type{});
    __builtin_amdgcn_sched_barrier(0);
    mma_read(sm, std::false_type{});
  }
  lds_sync();  // every wave is done with the stage buffers before C goes into them

  if constexpr (EPI == GEMM_EPI_RESID_F32) {
    // f32 rows through LDS, half the tile (128 rows, the waves with wm = half) at a time,
    // then whole rows: lane l of a wave on columns 4 l .. 4 l + 3 of every other row pair,
    // each access of a half wave one contiguous 512-byte row.  A residual element is read
    // by the lane that stores its sum, so R may alias C.
    float* fb = reinterpret_cast<float*>(sm);
    const float* Rp = static_cast<const float*>(g.R);
    float* Cp = static_cast<float*>(g.C);
    const int hr = lane >> 5, hc = (lane & 31) * 4;  // a wave stores two rows per access
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      // rows 2 (wave + 4 i) + hr of the half, i = 0 .. 15; the first eight residual rows in
      // flight before the tile half goes through LDS (rows past M re-read row M - 1)
      auto rrow = [&](int i) {
        const int m = min(m0 + half * 128 + 2 * (wave + 4 * i) + hr, g.M - 1);
        return *reinterpret_cast<const f32x4_t*>(Rp + static_cast<int64_t>(m) * g.ldr + n0 + hc);
      };
      f32x4_t rv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) rv[i] = rrow(i);
      if (wm == half) {
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) {
          float* rowp = fb + (mb * 16 + l16) * HFCP + wn * 64 + g4 * 4;
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) *reinterpret_cast<f32x4_t*>(rowp + nb * 16) = acc[nb][mb];
        }
      }
      lds_sync();
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int rl = 2 * (wave + 4 * i) + hr;
        const int m = m0 + half * 128 + rl;
        const f32x4_t r = rv[i & 7];
        if (i < 8) rv[i] = rrow(i + 8);
        if (m < g.M) {
          const f32x4_t v = *reinterpret_cast<const f32x4_t*>(fb + rl * HFCP + hc) + r;
          store16(Cp + static_cast<int64_t>(m) * g.ldc + n0 + hc, __builtin_bit_cast(uint4, v), g.nt);
        }
      }
      lds_sync();
    }
    return;
  }
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) {
    const int ml = wm * 128 + mb * 16 + l16;
    const int m = m0 + ml;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int nl = wn * 64 + nb * 16 + g4 * 4;
      float v[4] = {acc[nb][mb][0], acc[nb][mb][1], acc[nb][mb][2], acc[nb][mb][3]};
      epi_math<EPI>(g, m, n0 + nl, v);
      uint2 o;
      o.x = pack_bf16x2(v[0], v[1]);
      o.y = pack_bf16x2(v[2], v[3]);
      *reinterpret_cast<uint2*>(sm + ml * HCP + nl) = o;
    }
  }
  lds_sync();
  // 256 rows x 256 B: 16 threads per row, 16 rows per pass
  bf16_t* C = static_cast<bf16_t*>(g.C);
#pragma unroll
  for (int pass = 0; pass < HBM / 16; ++pass) {
    const int ml = pass * 16 + (tid >> 4);
    const int m = m0 + ml;
    if (m >= g.M) continue;
    const int nl = (tid & 15) * 8;
    store16(C + static_cast<int64_t>(m) * g.ldc + n0 + nl, *reinterpret_cast<const uint4*>(sm + ml * HCP + nl), g.nt);
  }
}

// W'[n, k] = bf16(W[n, k] g[k]): the RMSNorm gain folded into a weight's input columns
__global__ void scale_cols_bf16_kernel(const bf16_t* __restrict__ W, int64_t ldw, const float* __restrict__ gain,
                                       bf16_t* __restrict__ out, int64_t ldo, int N, int K) {
  const int kc = K / 8;
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < static_cast<int64_t>(N) * kc;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t n = i / kc;
    const int k = static_cast<int>(i - n * kc) * 8;
    float f[8];
    unpack8(*reinterpret_cast<const uint4*>(W + n * ldw + k), f);
    const float4 g0 = *reinterpret_cast<const float4*>(gain + k);
    const float4 g1 = *reinterpret_cast<const float4*>(gain + k + 4);
    f[0] *= g0.x; f[1] *= g0.y; f[2] *= g0.z; f[3] *= g0.w;
    f[4] *= g1.x; f[5] *= g1.y; f[6] *= g1.z; f[7] *= g1.w;
    *reinterpret_cast<uint4*>(out + n * ldo + k) = pack8(f);
  }
}

// ------------------------------------------------------------------ general GEMM
// C[m, n] = sum_k A[m*sam + k*sak] * B[k*sbk + n*sbn]  (+ epilogue), f32 accumulation.
constexpr int ST = 16;

template <typename TI, typename TO, int EPI, bool ACCUM>
__global__ void __launch_bounds__(ST * ST) gemm_general_kernel(
    const TI* __restrict__ A, int64_t sam, int64_t sak, const TI* __restrict__ Bm, int64_t sbk,
    int64_t sbn, TO* C, int64_t ldc, const TO* R, int64_t ldr, TO* Cpre, int64_t ldpre,
    int M, int N, int K) {
  __shared__ float sa[ST][ST + 1];
  __shared__ float sb[ST][ST + 1];
  const int tx = threadIdx.x % ST, ty = threadIdx.x / ST;
  const int m = blockIdx.y * ST + ty;
  const int n = blockIdx.x * ST + tx;
  float acc = 0.f;
  for (int k0 = 0; k0 < K; k0 += ST) {
    const int ka = k0 + tx, kb = k0 + ty;
    const int am = blockIdx.y * ST + ty;
    const int bn = blockIdx.x * ST + tx;
    sa[ty][tx] = (am < M && ka < K) ? to_f32(A[am * sam + ka * sak]) : 0.f;
    sb[ty][tx] = (kb < K && bn < N) ? to_f32(Bm[kb * sbk + bn * sbn]) : 0.f;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < ST; ++kk) acc += sa[ty][kk] * sb[kk][tx];
    __syncthreads();
  }
  if (m >= M || n >= N) return;
  const int64_t ci = static_cast<int64_t>(m) * ldc + n;
  float v = acc;
  if constexpr (ACCUM) v += to_f32(C[ci]);
  if constexpr (EPI == GEMM_EPI_RESID) v += to_f32(R[static_cast<int64_t>(m) * ldr + n]);
  if constexpr (EPI == GEMM_EPI_DSILU) v *= dsilu_f(to_f32(R[static_cast<int64_t>(m) * ldr + n]));
  if constexpr (EPI == GEMM_EPI_SILU) {
    if (Cpre) Cpre[static_cast<int64_t>(m) * ldpre + n] = from_f32<TO>(v);
    v = silu_f(v);
  }
  C[ci] = from_f32<TO>(v);
}

// ------------------------------------------------------------------ weight-gradient GEMM
// C[m, n] = sum_t A[t, m] B[t, n] over T rows: the weight gradient dW = dY^T X of a
// projection Y = X W^T.  Both operands are row-major with the reduction running down their
// rows, so the MFMA fragments (8 consecutive t per lane) come from tiles transposed on the
// way into LDS: a thread loads 4 rows x 8 columns of each operand (four 16-byte loads),
// packs each column's 4 values into 8 bytes and writes them to the tile [column][t].
// Tile 128 x 128 x 64 rows of T, 2 x 2 waves of 64 x 64 as in the NT kernel.  The T rows
// are split over S workgroups per output tile: each writes an f32 partial tile and a second
// kernel sums the S partials in a fixed order (deterministic), so the grid fills the chip
// even for a 256 x 256 gradient.
constexpr int TBT = 64;          // rows of T per step
constexpr int TP = TBT + 8;      // transposed tile pitch (bf16)
constexpr int TTILE = 128 * TP;  // elements of one transposed operand tile

struct TnArgs {
  const bf16_t* A; int64_t lda;
  const bf16_t* B; int64_t ldb;
  float* C; int64_t ldc;   // the output (S == 1) or the partial tiles (pitch N)
  int64_t split_stride;    // elements between the partial results of two splits
  int M, N, T, chunk;      // chunk: rows of T per split, a multiple of TBT
};

__device__ __forceinline__ uint32_t word_of(const uint4& v, int j) {
  return j == 0 ? v.x : (j == 1 ? v.y : (j == 2 ? v.z : v.w));
}

__global__ void __launch_bounds__(GTHREADS) gemm_tn_bf16_kernel(TnArgs g) {
  __shared__ __attribute__((aligned(16))) bf16_t sA[2][TTILE];
  __shared__ __attribute__((aligned(16))) bf16_t sB[2][TTILE];
  const int nN = (g.N + 127) / 128;
  const int mblk = static_cast<int>(blockIdx.x) / nN;
  const int m0 = mblk * 128, n0 = (static_cast<int>(blockIdx.x) - mblk * nN) * 128;
  const int t_begin = static_cast<int>(blockIdx.y) * g.chunk;
  const int rows = min(g.chunk, g.T - t_begin);  // >= 1: the host sizes the grid to T

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int l16 = lane & 15, g4 = lane >> 4;

  // staging: rows 4 rq .. 4 rq + 3 of the step, columns 8 ch .. 8 ch + 7 of the tile; the
  // descriptors cover this split's rows (later rows read as zero: the whole offset sits in
  // the vector operand, which the range check covers); columns past M (N) re-read valid
  // ones, whose results are never stored
  const int rq = tid & 15, ch = tid >> 4;
  const __amdgpu_buffer_rsrc_t rsA = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t*>(g.A + static_cast<int64_t>(t_begin) * g.lda), static_cast<short>(0),
      static_cast<uint32_t>(rows * g.lda * 2), BUF_DWORD3);
  const __amdgpu_buffer_rsrc_t rsB = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t*>(g.B + static_cast<int64_t>(t_begin) * g.ldb), static_cast<short>(0),
      static_cast<uint32_t>(rows * g.ldb * 2), BUF_DWORD3);
  const uint32_t voA = static_cast<uint32_t>(4 * rq * g.lda + min(m0 + 8 * ch, g.M - 8)) * 2u;
  const uint32_t voB = static_cast<uint32_t>(4 * rq * g.ldb + min(n0 + 8 * ch, g.N - 8)) * 2u;
  const uint32_t rowA = static_cast<uint32_t>(g.lda) * 2u, rowB = static_cast<uint32_t>(g.ldb) * 2u;
  uint4 ra[4], rb[4];
  auto fetch = [&](int t0) {
    const uint32_t soA = static_cast<uint32_t>(t0) * rowA, soB = static_cast<uint32_t>(t0) * rowB;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      ra[r] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsA, voA + r * rowA + soA, 0, 0));
      rb[r] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsB, voB + r * rowB + soB, 0, 0));
    }
  };
  // column 2j (2j + 1) of the 8: the low (high) halves of word j of the four rows
  auto put = [&](bf16_t* dst, const uint4 (&v)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t w0 = word_of(v[0], j), w1 = word_of(v[1], j), w2 = word_of(v[2], j), w3 = word_of(v[3], j);
      *reinterpret_cast<uint2*>(dst + (8 * ch + 2 * j) * TP + 4 * rq) =
          make_uint2(__builtin_amdgcn_perm(w1, w0, 0x05040100u), __builtin_amdgcn_perm(w3, w2, 0x05040100u));
      *reinterpret_cast<uint2*>(dst + (8 * ch + 2 * j + 1) * TP + 4 * rq) =
          make_uint2(__builtin_amdgcn_perm(w1, w0, 0x07060302u), __builtin_amdgcn_perm(w3, w2, 0x07060302u));
    }
  };

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nsteps = (rows + TBT - 1) / TBT;
  fetch(0);
  put(sA[0], ra);
  put(sB[0], rb);
  __syncthreads();
  for (int it = 0; it < nsteps; ++it) {
    const int buf = it & 1;
    if (it + 1 < nsteps) fetch((it + 1) * TBT);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8_t fb[4], fa[4];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        fb[nb] = as_bf16x8(*reinterpret_cast<const uint4*>(&sB[buf][(wn * 64 + nb * 16 + l16) * TP + ks * 32 + g4 * 8]));
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        fa[mb] = as_bf16x8(*reinterpret_cast<const uint4*>(&sA[buf][(wm * 64 + mb * 16 + l16) * TP + ks * 32 + g4 * 8]));
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[nb], fa[mb], acc[nb][mb], 0, 0, 0);
    }
    if (it + 1 < nsteps) {
      put(sA[buf ^ 1], ra);
      put(sB[buf ^ 1], rb);
    }
    __syncthreads();
  }

  // lane holds C[m][n .. n + 3] for each (nb, mb)
  float* C = g.C + static_cast<int64_t>(blockIdx.y) * g.split_stride;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const int m = m0 + wm * 64 + mb * 16 + l16;
    if (m >= g.M) continue;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int n = n0 + wn * 64 + nb * 16 + g4 * 4;
      if (n < g.N)
        *reinterpret_cast<float4*>(C + static_cast<int64_t>(m) * g.ldc + n) =
            make_float4(acc[nb][mb][0], acc[nb][mb][1], acc[nb][mb][2], acc[nb][mb][3]);
    }
  }
}

// C[m, n] = sum over s of P[s][m, n] (partials of pitch N), s in increasing order
__global__ void __launch_bounds__(256) splitk_reduce_kernel(const float* P, int64_t split_stride, int S,
                                                            float* C, int64_t ldc, int M, int N) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int n4 = N / 4;
  if (e >= static_cast<int64_t>(M) * n4) return;
  const int m = static_cast<int>(e / n4), n = static_cast<int>(e - static_cast<int64_t>(m) * n4) * 4;
  const float* p = P + static_cast<int64_t>(m) * N + n;
  float4 a = *reinterpret_cast<const float4*>(p);
  int s = 1;
  for (; s + 4 <= S; s += 4) {  // four loads in flight, added in split order
    float4 b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) b[i] = *reinterpret_cast<const float4*>(p + (s + i) * split_stride);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a.x += b[i].x; a.y += b[i].y; a.z += b[i].z; a.w += b[i].w;
    }
  }
  for (; s < S; ++s) {
    const float4 b = *reinterpret_cast<const float4*>(p + s * split_stride);
    a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
  }
  *reinterpret_cast<float4*>(C + static_cast<int64_t>(m) * ldc + n) = a;
}

// dst[c, r] = src[r, c] for an R x C bf16 matrix, 32 x 32 tiles through LDS
__global__ void __launch_bounds__(256) transpose_bf16_kernel(const bf16_t* src, int64_t lds, bf16_t* dst,
                                                             int64_t ldd, int R, int C) {
  __shared__ bf16_t t[32][33];
  const int c0 = blockIdx.x * 32, r0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
#pragma unroll
  for (int i = 0; i < 32; i += 8) {
    const int r = r0 + ty + i, c = c0 + tx;
    if (r < R && c < C) t[ty + i][tx] = src[static_cast<int64_t>(r) * lds + c];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 32; i += 8) {
    const int c = c0 + ty + i, r = r0 + tx;
    if (r < R && c < C) dst[static_cast<int64_t>(c) * ldd + r] = t[tx][ty + i];
  }
}

struct TnPlan {
  int S, chunk;
};
// enough splits for ~512 workgroups, at least 256 rows each
TnPlan tn_plan(int M, int N, int64_t T) {
  const int tiles = ((M + 127) / 128) * ((N + 127) / 128);
  int64_t S = (512 + tiles - 1) / tiles;
  S = std::min<int64_t>(S, std::max<int64_t>(1, (T + 255) / 256));
  int64_t chunk = (T + S - 1) / S;
  chunk = (chunk + TBT - 1) / TBT * TBT;
  S = (T + chunk - 1) / chunk;
  return {static_cast<int>(S), static_cast<int>(chunk)};
}

}  // namespace

genrank_status launch_gemm_nt(int dtype, const void* A, int64_t lda, const void* W, int64_t ldw,
                              void* C, int64_t ldc, int M, int N, int K, int epi, const void* R,
                              int64_t ldr, void* Cpre, int64_t ldpre, hipStream_t stream) {
  if (M <= 0) return GENRANK_OK;
  if (dtype == GENRANK_BF16 && N % GBN == 0 && K % GBK == 0 && lda % 8 == 0 && ldw % 8 == 0 &&
      ldc % 8 == 0 && (epi == GEMM_EPI_STORE || epi == GEMM_EPI_SILU || ldr % 4 == 0) && (!Cpre || ldpre % 4 == 0) &&
      static_cast<int64_t>(GBN) * ldw * 2 < (int64_t(1) << 32)) {
    GemmArgs g{static_cast<const bf16_t*>(A), lda, static_cast<const bf16_t*>(W), ldw, C, ldc,
               R, ldr, static_cast<bf16_t*>(Cpre), ldpre, M, N, K};
    g.nt = static_cast<int64_t>(M) * N * (epi == GEMM_EPI_RESID_F32 ? 4 : 2) > STREAM_OUT_BYTES;
    const int grid = (N / GBN) * ((M + GBM - 1) / GBM);
    // 256 x 128 tiles two per CU, or 256 x 256 tiles one per CU: measured on the pre-norm
    // block's projections at d = 512 (K = 512), the former wins for N = 512 and N = 2048 (by
    // 30-50 us at 377K rows), the latter for N = 1536 (by 40-60 us) and for K = 2048.  At
    // d = 256 (K = 256, where the 256 x 256 kernel does not apply) the 256 x 128 tiles beat the
    // 128 x 128 kernel: 54.0 against 60.1 us for QKV and 24.5 against 25.5 us for Wo at 96K rows
    const bool half_tiles = (K == 512 && (N <= 512 || N >= 2048)) || K == 256;
    if (half_tiles && N % HBN == 0 && M >= 8 * HBM &&
        static_cast<int64_t>(HBN) * ldw * 2 < (int64_t(1) << 32)) {
      const int hgrid = (N / HBN) * ((M + HBM - 1) / HBM);
      switch (epi) {
        case GEMM_EPI_STORE:
          hipLaunchKernelGGL(gemm_nt_bf16_half_kernel<GEMM_EPI_STORE>, dim3(hgrid), dim3(HTHREADS), 0, stream, g);
          break;
        case GEMM_EPI_RESID:
          hipLaunchKernelGGL(gemm_nt_bf16_half_kernel<GEMM_EPI_RESID>, dim3(hgrid), dim3(HTHREADS), 0, stream, g);
          break;
        case GEMM_EPI_SILU:
          hipLaunchKernelGGL(gemm_nt_bf16_half_kernel<GEMM_EPI_SILU>, dim3(hgrid), dim3(HTHREADS), 0, stream, g);
          break;
        case GEMM_EPI_DSILU:
          hipLaunchKernelGGL(gemm_nt_bf16_half_kernel<GEMM_EPI_DSILU>, dim3(hgrid), dim3(HTHREADS), 0, stream, g);
          break;
        case GEMM_EPI_RESID_F32:
          hipLaunchKernelGGL(gemm_nt_bf16_half_kernel<GEMM_EPI_RESID_F32>, dim3(hgrid), dim3(HTHREADS), 0, stream, g);
          break;
        default:
          return GENRANK_E_ARG;
      }
      GR_CHECK_LAUNCH();
      return GENRANK_OK;
    }
    if (K % (4 * GBK) == 0 && K >= 512 && N % BBN == 0 && M >= 4 * BBM &&
        static_cast<int64_t>(BBN) * ldw * 2 < (int64_t(1) << 32)) {
      const int bgrid = (N / BBN) * ((M + BBM - 1) / BBM);
      switch (epi) {
        case GEMM_EPI_STORE:
          hipLaunchKernelGGL((gemm_nt_bf16_big_kernel<GEMM_EPI_STORE, false>), dim3(bgrid), dim3(BTHREADS), 0, stream, g);
          break;
        case GEMM_EPI_RESID:
          hipLaunchKernelGGL((gemm_nt_bf16_big_kernel<GEMM_EPI_RESID, false>), dim3(bgrid), dim3(BTHREADS), 0, stream, g);
          break;
        case GEMM_EPI_SILU:
          hipLaunchKernelGGL((gemm_nt_bf16_big_kernel<GEMM_EPI_SILU, false>), dim3(bgrid), dim3(BTHREADS), 0, stream, g);
          break;
        case GEMM_EPI_DSILU:
          hipLaunchKernelGGL((gemm_nt_bf16_big_kernel<GEMM_EPI_DSILU, false>), dim3(bgrid), dim3(BTHREADS), 0, stream, g);
          break;
        case GEMM_EPI_RESID_F32:
          hipLaunchKernelGGL((gemm_nt_bf16_big_kernel<GEMM_EPI_RESID_F32, false>), dim3(bgrid), dim3(BTHREADS), 0, stream, g);
          break;
        default:
          return GENRANK_E_ARG;
      }
      GR_CHECK_LAUNCH();
      return GENRANK_OK;
    }
    if (K % (4 * GBK) == 0) {
      switch (epi) {
        case GEMM_EPI_STORE:
          hipLaunchKernelGGL(gemm_nt_bf16_dma_kernel<GEMM_EPI_STORE>, dim3(grid), dim3(GTHREADS), 0, stream, g);
          break;
        case GEMM_EPI_RESID:
          hipLaunchKernelGGL(gemm_nt_bf16_dma_kernel<GEMM_EPI_RESID>, dim3(grid), dim3(GTHREADS), 0, stream, g);
          break;
        case GEMM_EPI_SILU:
          hipLaunchKernelGGL(gemm_nt_bf16_dma_kernel<GEMM_EPI_SILU>, dim3(grid), dim3(GTHREADS), 0, stream, g);
          break;
        case GEMM_EPI_DSILU:
          hipLaunchKernelGGL(gemm_nt_bf16_dma_kernel<GEMM_EPI_DSILU>, dim3(grid), dim3(GTHREADS), 0, stream, g);
          break;
        case GEMM_EPI_RESID_F32:
          hipLaunchKernelGGL(gemm_nt_bf16_dma_kernel<GEMM_EPI_RESID_F32>, dim3(grid), dim3(GTHREADS), 0, stream, g);
          break;
        default:
          return GENRANK_E_ARG;
      }
      GR_CHECK_LAUNCH();
      return GENRANK_OK;
    }
    switch (epi) {
      case GEMM_EPI_STORE:
        hipLaunchKernelGGL(gemm_nt_bf16_kernel<GEMM_EPI_STORE>, dim3(grid), dim3(GTHREADS), 0, stream, g);
        break;
      case GEMM_EPI_RESID:
        hipLaunchKernelGGL(gemm_nt_bf16_kernel<GEMM_EPI_RESID>, dim3(grid), dim3(GTHREADS), 0, stream, g);
        break;
      case GEMM_EPI_SILU:
        hipLaunchKernelGGL(gemm_nt_bf16_kernel<GEMM_EPI_SILU>, dim3(grid), dim3(GTHREADS), 0, stream, g);
        break;
      case GEMM_EPI_DSILU:
        hipLaunchKernelGGL(gemm_nt_bf16_kernel<GEMM_EPI_DSILU>, dim3(grid), dim3(GTHREADS), 0, stream, g);
        break;
      case GEMM_EPI_RESID_F32:
        hipLaunchKernelGGL(gemm_nt_bf16_kernel<GEMM_EPI_RESID_F32>, dim3(grid), dim3(GTHREADS), 0, stream, g);
        break;
      default:
        return GENRANK_E_ARG;
    }
    GR_CHECK_LAUNCH();
    return GENRANK_OK;
  }
  // C = A W^T : B[k, n] = W[n, k]
  if (epi == GEMM_EPI_RESID_F32)  // f32 output and residual
    return launch_gemm_general(dtype, GENRANK_F32, A, lda, 1, W, 1, ldw, C, ldc, M, N, K, GEMM_EPI_RESID, false, R,
                               ldr, Cpre, ldpre, stream);
  return launch_gemm_general(dtype, dtype, A, lda, 1, W, 1, ldw, C, ldc, M, N, K, epi, false, R,
                             ldr, Cpre, ldpre, stream);
}

bool gemm_rms_ok(int N, int K) { return N > 0 && N % BBN == 0 && K >= 512 && K % (4 * GBK) == 0; }

genrank_status launch_gemm_nt_rms(const void* A, int64_t lda, const void* Wg, int64_t ldw, void* C, int64_t ldc,
                                  int M, int N, int K, int epi, hipStream_t stream) {
  if (M <= 0) return GENRANK_OK;
  if (!gemm_rms_ok(N, K) || lda % 8 || ldw % 8 || ldc % 8 || static_cast<int64_t>(BBN) * ldw * 2 >= (int64_t(1) << 32))
    return GENRANK_E_SHAPE;
  GemmArgs g{static_cast<const bf16_t*>(A), lda, static_cast<const bf16_t*>(Wg), ldw, C, ldc, nullptr, 0, nullptr, 0,
             M, N, K};
  g.nt = static_cast<int64_t>(M) * N * 2 > STREAM_OUT_BYTES;
  const int bgrid = (N / BBN) * ((M + BBM - 1) / BBM);
  if (epi == GEMM_EPI_STORE)
    hipLaunchKernelGGL((gemm_nt_bf16_big_kernel<GEMM_EPI_STORE, true>), dim3(bgrid), dim3(BTHREADS), 0, stream, g);
  else if (epi == GEMM_EPI_SILU)
    hipLaunchKernelGGL((gemm_nt_bf16_big_kernel<GEMM_EPI_SILU, true>), dim3(bgrid), dim3(BTHREADS), 0, stream, g);
  else
    return GENRANK_E_ARG;
  GR_CHECK_LAUNCH();
  return GENRANK_OK;
}

genrank_status launch_scale_cols(const void* W, int64_t ldw, const float* gain, void* out, int64_t ldo, int N, int K,
                                 hipStream_t stream) {
  if (N <= 0) return GENRANK_OK;
  if (K % 8 || ldw % 8 || ldo % 8) return GENRANK_E_SHAPE;
  const int64_t n = static_cast<int64_t>(N) * (K / 8);
  const unsigned grid = static_cast<unsigned>(std::min<int64_t>((n + 255) / 256, 2048));
  hipLaunchKernelGGL(scale_cols_bf16_kernel, dim3(grid), dim3(256), 0, stream, static_cast<const bf16_t*>(W), ldw, gain,
                     static_cast<bf16_t*>(out), ldo, N, K);
  GR_CHECK_LAUNCH();
  return GENRANK_OK;
}

genrank_status launch_gemm_general(int in_dtype, int out_dtype, const void* A, int64_t sam,
                                   int64_t sak, const void* Bm, int64_t sbk, int64_t sbn, void* C,
                                   int64_t ldc, int M, int N, int K, int epi, bool accumulate,
                                   const void* R, int64_t ldr, void* Cpre, int64_t ldpre,
                                   hipStream_t stream) {
  if (M <= 0 || N <= 0) return GENRANK_OK;
  dim3 grid((N + ST - 1) / ST, (M + ST - 1) / ST);
  dim3 block(ST * ST);
#define GR_GEN(TI, TO, E, ACC)                                                                  \
  hipLaunchKernelGGL((gemm_general_kernel<TI, TO, E, ACC>), grid, block, 0, stream,            \
                     static_cast<const TI*>(A), sam, sak, static_cast<const TI*>(Bm), sbk, sbn, \
                     static_cast<TO*>(C), ldc, static_cast<const TO*>(R), ldr,                  \
                     static_cast<TO*>(Cpre), ldpre, M, N, K)
#define GR_GEN_EPI(TI, TO, ACC)                         \
  switch (epi) {                                        \
    case GEMM_EPI_STORE: GR_GEN(TI, TO, GEMM_EPI_STORE, ACC); break; \
    case GEMM_EPI_RESID: GR_GEN(TI, TO, GEMM_EPI_RESID, ACC); break; \
    case GEMM_EPI_SILU: GR_GEN(TI, TO, GEMM_EPI_SILU, ACC); break;   \
    case GEMM_EPI_DSILU: GR_GEN(TI, TO, GEMM_EPI_DSILU, ACC); break; \
    default: return GENRANK_E_ARG;                      \
  }
  if (in_dtype == GENRANK_F32 && out_dtype == GENRANK_F32) {
    if (accumulate) { GR_GEN_EPI(float, float, true) } else { GR_GEN_EPI(float, float, false) }
  } else if (in_dtype == GENRANK_BF16 && out_dtype == GENRANK_BF16) {
    if (accumulate) { GR_GEN_EPI(bf16_t, bf16_t, true) } else { GR_GEN_EPI(bf16_t, bf16_t, false) }
  } else if (in_dtype == GENRANK_BF16 && out_dtype == GENRANK_F32) {
    if (accumulate) { GR_GEN_EPI(bf16_t, float, true) } else { GR_GEN_EPI(bf16_t, float, false) }
  } else {
    return GENRANK_E_DTYPE;
  }
#undef GR_GEN_EPI
#undef GR_GEN
  GR_CHECK_LAUNCH();
  return GENRANK_OK;
}

}  // namespace genrank

namespace genrank {

size_t gemm_tn_workspace(int M, int N, int64_t T) {
  if (T <= 0) return 0;
  const TnPlan p = tn_plan(M, N, T);
  return p.S > 1 ? static_cast<size_t>(p.S) * M * N * sizeof(float) : 0;
}

genrank_status launch_gemm_tn(int dtype, const void* A, int64_t lda, const void* Bm, int64_t ldb, float* C,
                              int64_t ldc, int M, int N, int64_t T, void* ws, size_t ws_bytes,
                              hipStream_t stream) {
  if (M <= 0 || N <= 0) return GENRANK_OK;
  auto al = [](const void* p, uintptr_t n) { return reinterpret_cast<uintptr_t>(p) % n == 0; };
  const TnPlan p = T > 0 ? tn_plan(M, N, T) : TnPlan{0, 0};
  if (dtype == GENRANK_BF16 && T > 0 && M % 8 == 0 && N % 8 == 0 && lda % 8 == 0 && ldb % 8 == 0 &&
      ldc % 4 == 0 && al(A, 16) && al(Bm, 16) && al(C, 16) &&
      static_cast<int64_t>(p.chunk) * std::max(lda, ldb) * 2 < (int64_t(1) << 31)) {
    const size_t need = gemm_tn_workspace(M, N, T);
    if (need > 0 && (!ws || ws_bytes < need || !al(ws, 16))) return GENRANK_E_WORKSPACE;
    TnArgs g{static_cast<const bf16_t*>(A), lda, static_cast<const bf16_t*>(Bm), ldb,
             p.S > 1 ? static_cast<float*>(ws) : C, p.S > 1 ? N : ldc,
             p.S > 1 ? static_cast<int64_t>(M) * N : 0, M, N, static_cast<int>(T), p.chunk};
    const dim3 grid(((M + 127) / 128) * ((N + 127) / 128), p.S);
    hipLaunchKernelGGL(gemm_tn_bf16_kernel, grid, dim3(GTHREADS), 0, stream, g);
    if (p.S > 1) {
      const int64_t n = static_cast<int64_t>(M) * (N / 4);
      hipLaunchKernelGGL(splitk_reduce_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, stream,
                         static_cast<const float*>(ws), static_cast<int64_t>(M) * N, p.S, C, ldc, M, N);
    }
    GR_CHECK_LAUNCH();
    return GENRANK_OK;
  }
  // C[m, n] = sum_t A[t * lda + m] B[t * ldb + n]
  return launch_gemm_general(dtype, GENRANK_F32, A, 1, lda, Bm, ldb, 1, C, ldc, M, N, static_cast<int>(T),
                             GEMM_EPI_STORE, false, nullptr, 0, nullptr, 0, stream);
}

genrank_status launch_gemm_nn(int dtype, const void* A, int64_t lda, const void* W, int64_t ldw, void* C,
                              int64_t ldc, int M, int N, int K, void* wt, hipStream_t stream, int epi,
                              const void* R, int64_t ldr) {
  if (M <= 0 || N <= 0) return GENRANK_OK;
  if (dtype == GENRANK_BF16 && wt && K > 0) {
    // W [K, N] -> W^T [N, K] (pitch K), then C = A (W^T)^T on the NT kernels
    const dim3 grid((N + 31) / 32, (K + 31) / 32);
    hipLaunchKernelGGL(transpose_bf16_kernel, grid, dim3(256), 0, stream, static_cast<const bf16_t*>(W), ldw,
                       static_cast<bf16_t*>(wt), static_cast<int64_t>(K), K, N);
    GR_CHECK_LAUNCH();
    return launch_gemm_nt(dtype, A, lda, wt, K, C, ldc, M, N, K, epi, R, ldr, nullptr, 0, stream);
  }
  return launch_gemm_general(dtype, dtype, A, lda, 1, W, ldw, 1, C, ldc, M, N, K, epi, false, R, ldr, nullptr, 0,
                             stream);
}

}  // namespace genrank
