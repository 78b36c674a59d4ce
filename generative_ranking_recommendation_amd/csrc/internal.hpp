// Launchers shared between the kernel files and the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "genrank.h"

namespace genrank {

// epilogues: STORE C = acc; RESID C = acc + R; SILU C = silu(acc) (Cpre = acc);
// F32 C = acc in f32; DSILU C = acc * silu'(R) (R the pre-activation: the SiLU backward)
// RESID_F32 C = acc + R with R and C f32 (the f32 residual stream)
enum { GEMM_EPI_STORE = 0, GEMM_EPI_RESID = 1, GEMM_EPI_SILU = 2, GEMM_EPI_F32 = 3, GEMM_EPI_DSILU = 4,
       GEMM_EPI_RESID_F32 = 5 };

constexpr float RMS_EPS = 1e-6f;

genrank_status check_batch(const genrank_batch* b);
size_t dtype_size(int dtype);
// the element type of the batch's residual stream (genrank_batch.resid)
int resid_dtype(const genrank_batch* b);

// embedding
genrank_status check_embed_args(const genrank_batch* b, const genrank_inputs* in,
                                const genrank_tables* t);
genrank_status launch_embed_sum(const genrank_batch* b, const genrank_inputs* in,
                                const genrank_tables* t, void* out, hipStream_t stream);
genrank_status launch_debug_indices(const genrank_batch* b, const genrank_inputs* in,
                                    const genrank_tables* t, int32_t* out, hipStream_t stream);
// candidate rows only: [B*m, d] written from row 0
genrank_status launch_embed_sum_cand(const genrank_batch* b, const genrank_inputs* in, const genrank_tables* t,
                                     void* out, hipStream_t stream);
// candidate queries ([B*m] rows of q / k / v / o / lse) against history keys and values
// held elsewhere (rows [off_u, off_u + N_u) of kh / vh); bf16, dh = 64
genrank_status launch_attn_fwd_cached(const genrank_batch* b, const int32_t* offsets, const int64_t* ts,
                                      const int64_t* req, genrank_alibi alibi, const void* q, const void* k,
                                      const void* v, int64_t ld_c, const void* kh, const void* vh, int64_t ld_h,
                                      void* o, int64_t ld_o, float* lse, hipStream_t stream);
size_t embed_bwd_workspace(const genrank_batch* b);
genrank_status launch_embed_bwd(const genrank_batch* b, const genrank_inputs* in, const genrank_tables* t,
                                const void* dx, int32_t* item_ids, float* item_rows, int32_t* n_items,
                                float* g_action, float* g_pos, float* g_ri, float* g_rt, void* ws,
                                hipStream_t stream);
// Stable radix sort of `slices` arrays of n (key, value) pairs by the low `bits` key bits;
// *result_in_tmp tells whether the result ended in (tmp_keys, tmp_vals).
size_t radix_sort_workspace(int64_t n, int slices);
genrank_status launch_radix_sort(uint32_t* keys, uint32_t* vals, uint32_t* tmp_keys, uint32_t* tmp_vals,
                                 int64_t n, int slices, int bits, uint32_t* hist, int* result_in_tmp,
                                 hipStream_t stream);

// attention
genrank_status check_attn_args(const genrank_batch* b, const int32_t* offsets, const int64_t* ts,
                               const int64_t* req, genrank_alibi alibi, const void* q,
                               const void* k, const void* v, int64_t ld_qkv, const void* o,
                               int64_t ld_o);
genrank_status launch_attn_fwd(const genrank_batch* b, const int32_t* offsets, const int64_t* ts,
                               const int64_t* req, genrank_alibi alibi, const void* q,
                               const void* k, const void* v, int64_t ld_qkv, void* o,
                               int64_t ld_o, float* lse, hipStream_t stream);
genrank_status launch_debug_mask(const int32_t* offsets, int m, int user, int L_cap, uint8_t* out,
                                 hipStream_t stream);
size_t attn_bwd_workspace(const genrank_batch* b);
// the allocation-free backward: the size of its library-owned scratch array, and the current
// device's copy of it (looked up on the first call on each device)
size_t attn_bwd_scratch_bytes();
genrank_status attn_bwd_scratch(void** ptr);
genrank_status launch_attn_bwd(const genrank_batch* b, const int32_t* offsets, const int64_t* ts,
                               const int64_t* req, genrank_alibi alibi, const void* q,
                               const void* k, const void* v, int64_t ld_qkv, const void* o,
                               const void* dout, int64_t ld_o, const float* lse, void* dq,
                               void* dk, void* dv, int64_t ld_dqkv, int cand_only, void* ws,
                               hipStream_t stream);

// HSTU-style comparison (interleaved sequence, learned bias in memory)
genrank_status launch_hstu_rab_layout(const genrank_batch* b, const int32_t* offsets, int64_t* rab_off,
                                      hipStream_t stream);
genrank_status launch_hstu_rab(const genrank_batch* b, const int32_t* offsets, const int64_t* ts,
                               const int64_t* req, const float* pos_table, int n_pos,
                               const float* time_table, const int64_t* bounds, int n_time,
                               const int64_t* rab_off, void* rab, hipStream_t stream);
genrank_status launch_hstu_attn_fwd(const genrank_batch* b, const int32_t* offsets, const void* rab,
                                    const int64_t* rab_off, const void* q, const void* k,
                                    const void* v, int64_t ld_qkv, void* o, int64_t ld_o, float* lse,
                                    hipStream_t stream);

// the ALiBi variant flags: known bits only; bucket edges present and at most 1024; under the
// fully visible mask the kernels form the bias as -|w_j - w_i| (w = s p + s' tau), which is
// the per-term form only when the H slopes are non-negative (positions and times are sorted)
inline genrank_status check_alibi_variant(const genrank_alibi& a, int H) {
  if (a.flags & ~(GENRANK_ATTN_FULL_HISTORY | GENRANK_ATTN_TIME_BUCKET)) return GENRANK_E_ARG;
  if (a.flags & GENRANK_ATTN_FULL_HISTORY)
    for (int h = 0; h < H; ++h)
      if (!(a.slopes_pos[h] >= 0.f) || !(a.slopes_time[h] >= 0.f)) return GENRANK_E_ARG;
  if (a.flags & GENRANK_ATTN_TIME_BUCKET) {
    if (a.n_time_bounds < 0 || a.n_time_bounds > 1024) return GENRANK_E_SHAPE;
    if (a.n_time_bounds > 0 && !a.time_bounds) return GENRANK_E_ARG;
  }
  return GENRANK_OK;
}

// GEMM: C = A W^T (A [M, K], W [N, K]) with an epilogue
genrank_status launch_gemm_nt(int dtype, const void* A, int64_t lda, const void* W, int64_t ldw,
                              void* C, int64_t ldc, int M, int N, int K, int epi, const void* R,
                              int64_t ldr, void* Cpre, int64_t ldpre, hipStream_t stream);
// The bf16 GEMM with the RMSNorm of A's rows fused (A raw, Wg = W with the gain folded into
// its columns, see launch_scale_cols); epi STORE or SILU; requires gemm_rms_ok(N, K)
bool gemm_rms_ok(int N, int K);
// The current device's error word (GENRANK_ERR_* bits), or NULL if it cannot be located
uint32_t* device_error_word();
genrank_status launch_gemm_nt_rms(const void* A, int64_t lda, const void* Wg, int64_t ldw, void* C, int64_t ldc,
                                  int M, int N, int K, int epi, hipStream_t stream);
// out[n, k] = bf16(W[n, k] gain[k]) (bf16 W and out)
genrank_status launch_scale_cols(const void* W, int64_t ldw, const float* gain, void* out, int64_t ldo, int N, int K,
                                 hipStream_t stream);
// General strided GEMM: C[m, n] (+)= sum_k A[m*sam + k*sak] B[k*sbk + n*sbn]
genrank_status launch_gemm_general(int in_dtype, int out_dtype, const void* A, int64_t sam,
                                   int64_t sak, const void* Bm, int64_t sbk, int64_t sbn, void* C,
                                   int64_t ldc, int M, int N, int K, int epi, bool accumulate,
                                   const void* R, int64_t ldr, void* Cpre, int64_t ldpre,
                                   hipStream_t stream);

// Weight gradient: C[m, n] = sum_t A[t, m] B[t, n] (f32 out), split over T with f32 partial
// tiles in ws (gemm_tn_workspace bytes) when the bf16 MFMA kernel takes it
size_t gemm_tn_workspace(int M, int N, int64_t T);
genrank_status launch_gemm_tn(int dtype, const void* A, int64_t lda, const void* Bm, int64_t ldb, float* C,
                              int64_t ldc, int M, int N, int64_t T, void* ws, size_t ws_bytes,
                              hipStream_t stream);
// Data gradient: C[M, N] = A[M, K] W[K, N]; bf16 transposes W into wt ([N, K], N * K elements)
// and runs the NT kernels
genrank_status launch_gemm_nn(int dtype, const void* A, int64_t lda, const void* W, int64_t ldw, void* C,
                              int64_t ldc, int M, int N, int K, void* wt, hipStream_t stream,
                              int epi = GEMM_EPI_STORE, const void* R = nullptr, int64_t ldr = 0);

// row-wise ops
// y = rmsnorm(x) g with x in in_dtype and y in out_dtype (bf16 -> bf16, f32 -> bf16, f32 -> f32)
genrank_status launch_rmsnorm(int in_dtype, int out_dtype, const void* x, const float* g, void* y, int64_t rows,
                              int d, hipStream_t stream);
size_t rmsnorm_bwd_workspace(int d);  // per-block partial rows of dg
// x in x_dtype (the residual stream), dy, add, dx in dtype
genrank_status launch_rmsnorm_bwd(int x_dtype, int dtype, const void* x, const float* g, const void* dy,
                                  const void* add, void* dx, float* dg, int64_t rows, int d, void* ws,
                                  hipStream_t stream);
genrank_status launch_fill_f32(float* p, int64_t n, float v, hipStream_t stream);
genrank_status launch_fill_zero(int dtype, void* p, int64_t n, hipStream_t stream);
// the head at rows row0 .. row0 + rows - 1 of x, or at rows idx[0 .. rows) when idx is given
genrank_status launch_head_fwd(int dtype, const void* x, int64_t row0, int64_t rows, const int32_t* idx,
                               int d, const float* g, const float* w, const float* bias, int nt,
                               float* logits, hipStream_t stream);
size_t head_bwd_workspace(int d, int nt);  // per-block partial rows of dg, dw, db
// x in x_dtype (the residual stream), dx in dtype
genrank_status launch_head_bwd(int x_dtype, int dtype, const void* x, int64_t row0, int64_t rows,
                               const int32_t* idx, int d, const float* g, const float* w, int nt,
                               const float* dlogits, void* dx, float* dg, float* dw, float* db, void* ws,
                               hipStream_t stream);
genrank_status launch_bce(int64_t n, int nt, const float* logits, const float* labels,
                          float* loss, float* dlogits, hipStream_t stream);

}  // namespace genrank
