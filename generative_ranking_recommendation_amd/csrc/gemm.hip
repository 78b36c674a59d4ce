// Dense projections of the GenRank block (QKV, output, FFN): bf16 MFMA GEMM on gfx950.
//
//   C[M, N] = A[M, K] . W[N, K]^T  (+ epilogue), f32 accumulation.
//
// Tile: 128 (M) x 128 (N) x 64 (K) per 256-thread workgroup; 2 x 2 waves of 64 x 64.
// Each wave issues v_mfma_f32_16x16x32_bf16 with W rows as the MFMA row operand and A
// rows as the column operand, so each lane ends with 4 consecutive N values of one A row
// and stores them as one 8-byte write.  Both operands are K-contiguous and staged through
// LDS with a 16-byte row pad (conflict-free 16-byte reads).  The next K tile is fetched
// into registers while the current one is multiplied.  Workgroups are renumbered so that
// the N tiles of one M tile run on the same XCD and share its L2.
//
// A second, simple kernel handles f32 data and the transposed products of the backward
// pass (general strides, LDS-tiled FMA).
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
  const bf16_t* R; int64_t ldr;   // residual (EPI_RESID), may alias C
  bf16_t* Cpre; int64_t ldpre;    // pre-activation copy (EPI_SILU, optional)
  int M, N, K;
};

__device__ __forceinline__ float silu_f(float x) { return x / (1.0f + __expf(-x)); }

// LDS operand tile: [128 rows][32 bf16] = 64 B per row, four 16-byte chunks.  Chunk c of
// row r is stored at chunk c ^ ((r >> 1) & 3): the 16-byte reads of 16 consecutive rows at
// one chunk (an MFMA operand fragment) and the 16-byte writes of the staging pattern both
// hit distinct banks.
__device__ __forceinline__ int swz(int r, int c) { return r * GBK + ((c ^ ((r >> 1) & 3)) << 3); }

constexpr int CP = GBN + 8;                           // staged C row pitch (bf16)
constexpr int SMEM_OPS = 2 * 2 * GBM * GBK;           // [stage][A|W] operand tiles
constexpr int SMEM = SMEM_OPS > GBM * CP ? SMEM_OPS : GBM * CP;

// ---- epilogue shared by the MFMA kernels: lane holds C[m][n .. n+3] for each (nb, mb).
// The 128 x 128 tile (after the epilogue math, in the output dtype) is staged through LDS,
// rows 0-63 at sC_lo and rows 64-127 at sC_hi (pitch CP), so that every global store is a
// 16-byte piece of a row.  The caller guarantees that no wave still reads those buffers.
template <int EPI>
__device__ __forceinline__ void epilogue(const GemmArgs& g, const f32x4_t (&acc)[4][4], bf16_t* sC_lo,
                                         bf16_t* sC_hi, int m0, int n0, int wm, int wn, int l16, int g4,
                                         int tid) {
  if constexpr (EPI == GEMM_EPI_F32) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int m = m0 + wm * 64 + mb * 16 + l16;
      if (m >= g.M) continue;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int n = n0 + wn * 64 + nb * 16 + g4 * 4;
        float* c = static_cast<float*>(g.C) + static_cast<int64_t>(m) * g.ldc + n;
        *reinterpret_cast<float4*>(c) = make_float4(acc[nb][mb][0], acc[nb][mb][1], acc[nb][mb][2], acc[nb][mb][3]);
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
      if constexpr (EPI == GEMM_EPI_RESID) {
        if (m < g.M) {
          const uint2 r = *reinterpret_cast<const uint2*>(g.R + static_cast<int64_t>(m) * g.ldr + n);
          v[0] += __uint_as_float(r.x << 16); v[1] += __uint_as_float(r.x & 0xFFFF0000u);
          v[2] += __uint_as_float(r.y << 16); v[3] += __uint_as_float(r.y & 0xFFFF0000u);
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
    *reinterpret_cast<uint4*>(C + static_cast<int64_t>(m) * g.ldc + n0 + nl) = *reinterpret_cast<const uint4*>(src);
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

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// vmcnt(n) with every other counter left alone (gfx9 encoding: vmcnt in bits 3:0 and
// 15:14, expcnt 6:4, lgkmcnt 11:8)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 16, "");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}
// all waves past this point see every LDS write made before it; the empty asm keeps the
// compiler from moving memory accesses across
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

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
  // global chunk (lane % 4) ^ ((r >> 1) & 3).  A rows past M re-read row M - 1 (never stored).
  const int lr = lane >> 2, ls = lane & 3;
  const int r0 = wave * 32 + lr, r1 = r0 + 16;
  const int c0 = ls ^ ((r0 >> 1) & 3), c1 = ls ^ ((r1 >> 1) & 3);
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
  if constexpr (EPI == GEMM_EPI_SILU) {
    if (Cpre) Cpre[static_cast<int64_t>(m) * ldpre + n] = from_f32<TO>(v);
    v = silu_f(v);
  }
  C[ci] = from_f32<TO>(v);
}

}  // namespace

genrank_status launch_gemm_nt(int dtype, const void* A, int64_t lda, const void* W, int64_t ldw,
                              void* C, int64_t ldc, int M, int N, int K, int epi, const void* R,
                              int64_t ldr, void* Cpre, int64_t ldpre, hipStream_t stream) {
  if (M <= 0) return GENRANK_OK;
  if (dtype == GENRANK_BF16 && N % GBN == 0 && K % GBK == 0 && lda % 8 == 0 && ldw % 8 == 0 &&
      ldc % 8 == 0 && (epi != GEMM_EPI_RESID || ldr % 4 == 0) && (!Cpre || ldpre % 4 == 0) &&
      static_cast<int64_t>(GBN) * ldw * 2 < (int64_t(1) << 32)) {
    GemmArgs g{static_cast<const bf16_t*>(A), lda, static_cast<const bf16_t*>(W), ldw, C, ldc,
               static_cast<const bf16_t*>(R), ldr, static_cast<bf16_t*>(Cpre), ldpre, M, N, K};
    const int grid = (N / GBN) * ((M + GBM - 1) / GBM);
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
      default:
        return GENRANK_E_ARG;
    }
    GR_CHECK_LAUNCH();
    return GENRANK_OK;
  }
  // C = A W^T : B[k, n] = W[n, k]
  return launch_gemm_general(dtype, dtype, A, lda, 1, W, 1, ldw, C, ldc, M, N, K, epi, false, R,
                             ldr, Cpre, ldpre, stream);
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
