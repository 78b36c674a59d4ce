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

constexpr int GBM = 128, GBN = 128, GBK = 64;
constexpr int GPAD = 8;              // bf16 elements of padding per LDS row
constexpr int GLD = GBK + GPAD;      // LDS row pitch (elements)
constexpr int GTHREADS = 256;

struct GemmArgs {
  const bf16_t* A; int64_t lda;
  const bf16_t* W; int64_t ldw;
  void* C; int64_t ldc;
  const bf16_t* R; int64_t ldr;   // residual (EPI_RESID), may alias C
  bf16_t* Cpre; int64_t ldpre;    // pre-activation copy (EPI_SILU, optional)
  int M, N, K;
};

__device__ __forceinline__ float silu_f(float x) { return x / (1.0f + __expf(-x)); }

template <int EPI>
__global__ void __launch_bounds__(GTHREADS) gemm_nt_bf16_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) bf16_t sA[GBM * GLD];
  __shared__ __attribute__((aligned(16))) bf16_t sW[GBN * GLD];

  // XCD-aware renumbering: hardware hands workgroup w to XCD w % 8; give the tiles of
  // one M row-block consecutive logical ids on the same XCD.
  const int nN = g.N / GBN;
  const int nM = (g.M + GBM - 1) / GBM;
  const int G = nN * nM;
  const int w = blockIdx.x;
  int L = w;
  if (G % 8 == 0) L = (w % 8) * (G / 8) + (w / 8);
  const int mblk = L / nN;
  const int nblk = L - mblk * nN;
  const int m0 = mblk * GBM;
  const int n0 = nblk * GBN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int l16 = lane & 15, g4 = lane >> 4;

  // global -> register staging: 4 chunks of 16 B per operand per thread (named
  // registers: an indexed array here ends up in scratch memory)
  uint4 ra0, ra1, ra2, ra3, rw0, rw1, rw2, rw3;
  const int srow = tid >> 3;          // + 32 * i for chunk i
  const int skc = (tid & 7) * 8;
  const bf16_t* a_row[4];
  const bf16_t* w_row[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // rows past M are clamped to M-1: their results are never stored
    const int gm = min(m0 + srow + 32 * i, g.M - 1);
    a_row[i] = g.A + static_cast<int64_t>(gm) * g.lda + skc;
    w_row[i] = g.W + static_cast<int64_t>(n0 + srow + 32 * i) * g.ldw + skc;
  }
#define GR_FETCH(k0)                                                     \
  do {                                                                   \
    ra0 = *reinterpret_cast<const uint4*>(a_row[0] + (k0));              \
    ra1 = *reinterpret_cast<const uint4*>(a_row[1] + (k0));              \
    ra2 = *reinterpret_cast<const uint4*>(a_row[2] + (k0));              \
    ra3 = *reinterpret_cast<const uint4*>(a_row[3] + (k0));              \
    rw0 = *reinterpret_cast<const uint4*>(w_row[0] + (k0));              \
    rw1 = *reinterpret_cast<const uint4*>(w_row[1] + (k0));              \
    rw2 = *reinterpret_cast<const uint4*>(w_row[2] + (k0));              \
    rw3 = *reinterpret_cast<const uint4*>(w_row[3] + (k0));              \
  } while (0)
#define GR_STASH()                                                        \
  do {                                                                    \
    *reinterpret_cast<uint4*>(sA + (srow + 0) * GLD + skc) = ra0;         \
    *reinterpret_cast<uint4*>(sA + (srow + 32) * GLD + skc) = ra1;        \
    *reinterpret_cast<uint4*>(sA + (srow + 64) * GLD + skc) = ra2;        \
    *reinterpret_cast<uint4*>(sA + (srow + 96) * GLD + skc) = ra3;        \
    *reinterpret_cast<uint4*>(sW + (srow + 0) * GLD + skc) = rw0;         \
    *reinterpret_cast<uint4*>(sW + (srow + 32) * GLD + skc) = rw1;        \
    *reinterpret_cast<uint4*>(sW + (srow + 64) * GLD + skc) = rw2;        \
    *reinterpret_cast<uint4*>(sW + (srow + 96) * GLD + skc) = rw3;        \
  } while (0)

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nk = g.K / GBK;
  GR_FETCH(0);
  for (int kt = 0; kt < nk; ++kt) {
    __syncthreads();
    GR_STASH();
    __syncthreads();
    if (kt + 1 < nk) GR_FETCH((kt + 1) * GBK);
#pragma unroll
    for (int ks = 0; ks < GBK / 32; ++ks) {
      bf16x8_t fw[4], fa[4];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        fw[nb] = as_bf16x8(*reinterpret_cast<const uint4*>(
            sW + (wn * 64 + nb * 16 + l16) * GLD + ks * 32 + g4 * 8));
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        fa[mb] = as_bf16x8(*reinterpret_cast<const uint4*>(
            sA + (wm * 64 + mb * 16 + l16) * GLD + ks * 32 + g4 * 8));
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fw[nb], fa[mb], acc[nb][mb], 0, 0, 0);
    }
  }

#undef GR_FETCH
#undef GR_STASH

  // epilogue: lane holds C[m][n .. n+3] for each (nb, mb)
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const int m = m0 + wm * 64 + mb * 16 + l16;
    if (m >= g.M) continue;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int n = n0 + wn * 64 + nb * 16 + g4 * 4;
      float v[4] = {acc[nb][mb][0], acc[nb][mb][1], acc[nb][mb][2], acc[nb][mb][3]};
      if constexpr (EPI == GEMM_EPI_F32) {
        float* c = static_cast<float*>(g.C) + static_cast<int64_t>(m) * g.ldc + n;
        *reinterpret_cast<float4*>(c) = make_float4(v[0], v[1], v[2], v[3]);
      } else {
        if constexpr (EPI == GEMM_EPI_RESID) {
          const uint2 r = *reinterpret_cast<const uint2*>(g.R + static_cast<int64_t>(m) * g.ldr + n);
          v[0] += __uint_as_float(r.x << 16); v[1] += __uint_as_float(r.x & 0xFFFF0000u);
          v[2] += __uint_as_float(r.y << 16); v[3] += __uint_as_float(r.y & 0xFFFF0000u);
        }
        if constexpr (EPI == GEMM_EPI_SILU) {
          if (g.Cpre) {
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
        *reinterpret_cast<uint2*>(static_cast<bf16_t*>(g.C) + static_cast<int64_t>(m) * g.ldc + n) = o;
      }
    }
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
      ldc % 4 == 0 && (epi != GEMM_EPI_RESID || ldr % 4 == 0) && (!Cpre || ldpre % 4 == 0)) {
    GemmArgs g{static_cast<const bf16_t*>(A), lda, static_cast<const bf16_t*>(W), ldw, C, ldc,
               static_cast<const bf16_t*>(R), ldr, static_cast<bf16_t*>(Cpre), ldpre, M, N, K};
    const int grid = (N / GBN) * ((M + GBM - 1) / GBM);
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
