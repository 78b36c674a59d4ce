/*
 * genrank.h -- C ABI of the MI355X (gfx950) GenRank ranking hot path.
 *
 * GenRank ("Towards Large-scale Generative Ranking") scores a request's candidates
 * against a user's chronological action history.  One token per history action is the
 * sum of five embeddings (item, action, position, request index, pre-request time gap);
 * each candidate token uses the mask-action embedding and shares one position with the
 * other candidates of its request.  Tokens feed causal attention with ALiBi position and
 * time biases and a candidate mask: history tokens attend causally, each candidate sees
 * the whole history and itself, never another candidate.
 *
 * Page titles cited below:
 *   [GR-zh]   "一、 GenRank [2025]" (huaxiaozhuan.com)
 *   [GR-note] "生成式排序 —— 小红书 GenRank 精读笔记" (wln20.github.io)
 *   [FR-en]   "The Overall Generative Ranking Paradigm" (fun-rec mdbook, chapter 7.2)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Row layout.  B users; user u has N_u = hist_offsets[u+1] - hist_offsets[u] history
 *    actions and m candidates.  Rows [0, T_h) are history rows, user after user
 *    (T_h = hist_offsets[B]); row T_h + u*m + k is candidate k of user u.  T = T_h + B*m.
 *  - Pointers.  Unless a parameter says "host", every array pointer is DEVICE memory
 *    owned by the caller.  The library allocates nothing and keeps no pointer after a
 *    call returns.  Scratch memory comes from a caller-supplied workspace whose size
 *    genrank_workspace_size() reports.
 *  - Streams.  Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *    is asynchronous; nothing synchronises except genrank_validate_host (host only) and
 *    genrank_error_word (it waits for `stream` before reading the word).
 *  - Graph capture.  The compute entry points only launch kernels on `stream`: none
 *    allocates, synchronises or clears memory with a memset, so a caller may capture them
 *    in a HIP graph (stream capture) and replay it; kernel arguments, including the
 *    host-side ALiBi slopes, are taken at capture.  genrank_error_word cannot be captured.
 *  - Errors.  Host-side argument checks run before anything is enqueued; on error the
 *    call returns a negative genrank_status, enqueues nothing and leaves outputs
 *    untouched.  A failed kernel launch returns GENRANK_E_HIP.  Data-dependent
 *    preconditions (sorted timestamps, ids in range) are NOT checked on the hot path:
 *    genrank_validate_host checks host copies of the inputs.
 *  - Dtypes.  Activations and tables are f32 or bf16 (genrank_dtype); accumulation is
 *    always f32; softmax statistics (LSE) are f32; timestamps are int64 seconds.
 *  - Matrices are row-major.  A weight W of shape [out, in] is applied as y = x W^T.
 *  - Reentrancy.  Stateless; calls on different streams may overlap.
 */
#ifndef GENRANK_H
#define GENRANK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#define GENRANK_API __attribute__((visibility("default")))
#else
#define GENRANK_API
#endif

#define GENRANK_VERSION_MAJOR 0
#define GENRANK_VERSION_MINOR 1
#define GENRANK_MAX_HEADS 16

typedef void* genrank_stream_t; /* hipStream_t */

typedef enum {
  GENRANK_OK = 0,
  GENRANK_E_ARG = -1,       /* null pointer or invalid scalar argument */
  GENRANK_E_SHAPE = -2,     /* inconsistent sizes (H*dh != d, unsupported d/dh, ...) */
  GENRANK_E_DTYPE = -3,     /* unsupported dtype for this entry point */
  GENRANK_E_UNSORTED = -4,  /* offsets or timestamps out of order (validate only) */
  GENRANK_E_RANGE = -5,     /* an id or time difference out of range (validate only) */
  GENRANK_E_WORKSPACE = -6, /* workspace missing or smaller than required */
  GENRANK_E_HIP = -7        /* a HIP runtime call or kernel launch failed */
} genrank_status;

typedef enum { GENRANK_F32 = 0, GENRANK_BF16 = 1 } genrank_dtype;

typedef enum { GENRANK_BLOCK_ATTN_ONLY = 0, GENRANK_BLOCK_PRENORM = 1 } genrank_block;

typedef enum {
  GENRANK_OP_EMBED_SUM = 0,
  GENRANK_OP_ATTN_FWD = 1,
  GENRANK_OP_ATTN_BWD = 2,
  GENRANK_OP_LAYER_FWD = 3,
  GENRANK_OP_LAYER_BWD = 4,
  GENRANK_OP_EMBED_BWD = 5,
  GENRANK_OP_HEAD_BWD = 6,
  GENRANK_OP_LAYER_KV = 7,
  GENRANK_OP_LAYER_FWD_CACHED = 8
} genrank_op;

/* Batch geometry.  total_hist and max_hist are host copies of hist_offsets[B] and
 * max_u N_u so that no device-to-host copy is needed; they must match the device data.
 *
 * resid chooses the element type of the residual stream: the rows genrank_embed_sum /
 * genrank_embed_sum_cand write, the block inputs and outputs of genrank_layer_fwd,
 * genrank_layer_kv and genrank_layer_fwd_cached, the block input genrank_layer_bwd reads,
 * and the rows genrank_head_fwd / genrank_head_bwd read.
 *   GENRANK_RESID_ACT (0): the residual stream is in `dtype`;
 *   GENRANK_RESID_F32 (1): it is f32 while the projections' operands (normalised rows, Q/K/V,
 *     attention output, FFN hidden) stay in `dtype`.  This is mixed precision in the sense
 *     of "一、 GenRank [2025]" section 1.3 (training setup): bf16 products with f32
 *     accumulation, and each residual sum kept in f32 instead of being rounded to bf16 after
 *     every block.  Pre-norm blocks only (an attention-only block's input is its QKV
 *     operand): genrank_layer_* return GENRANK_E_DTYPE for it.
 * Gradients of the residual stream (dy, dx of genrank_layer_bwd, genrank_head_bwd's dx and
 * genrank_embed_bwd's dx) are in `dtype` either way. */
#define GENRANK_RESID_ACT 0
#define GENRANK_RESID_F32 1
typedef struct {
  int32_t B;          /* users, >= 1 */
  int32_t m;          /* candidates per user, >= 0 */
  int32_t d;          /* model dim */
  int32_t H;          /* heads, 1..GENRANK_MAX_HEADS */
  int32_t dh;         /* head dim; H*dh == d */
  int32_t max_hist;   /* max_u N_u */
  int64_t total_hist; /* T_h = sum_u N_u */
  int32_t dtype;      /* genrank_dtype of activations and embedding tables */
  int32_t resid;      /* GENRANK_RESID_ACT or GENRANK_RESID_F32 (see above) */
} genrank_batch;

/* Per-user chronological histories and the candidates of one request
 * ([GR-zh] section 1.4.1: items x_i with actions a_i at timestamps t_i). */
typedef struct {
  const int32_t* hist_offsets; /* [B+1], hist_offsets[0] = 0, non-decreasing */
  const int32_t* hist_items;   /* [T_h] item ids in [0, n_item) */
  const int32_t* hist_actions; /* [T_h] action ids in [0, n_action) */
  const int64_t* hist_ts;      /* [T_h] seconds, non-decreasing within a user */
  const int32_t* cand_items;   /* [B*m] candidate item ids */
  const int64_t* req_ts;       /* [B] request time of the candidates, > the user's last ts */
} genrank_inputs;

/* The five embedding tables ([GR-zh] section 1.4.2, five-term input representation),
 * each row-major [rows, d] in batch.dtype. */
typedef struct {
  const void* item;   /* psi     [n_item, d] */
  const void* action; /* phi     [n_action + 1, d]; row n_action is the mask-action row M */
  const void* pos;    /* Omega_pe [n_pos, d]; slot = min(position, n_pos - 1) */
  const void* ri;     /* Omega_ri [n_ri, d]; slot = min(request index - 1, n_ri - 1) */
  const void* rt;     /* Omega_rt [n_rt, d]; slot = time-gap bucket */
  const int64_t* rt_bounds; /* [n_rt - 1] non-decreasing integer bucket edges (seconds):
                               bucket = #{k : rt_bounds[k] <= gap}; 0 = no earlier request */
  int64_t n_item;
  int32_t n_action;
  int32_t n_pos;
  int32_t n_ri;
  int32_t n_rt;
} genrank_tables;

/* ALiBi slopes, HOST arrays of H floats: the score of query i and key j in head h gets
 * -slopes_pos[h]*|p_i - p_j| - slopes_time[h]*|tau_i - tau_j|, p the position id (all
 * candidates of a request share p = N_u) and tau the timestamp in seconds relative to
 * the user's first history timestamp ([GR-zh] section 1.4.2, ALiBi score; [FR-en]
 * section 7.2.2, position-and-time bias).
 * flags (0 = the default above and the causal history mask):
 *   GENRANK_ATTN_FULL_HISTORY: history queries see every history key (the fully visible
 *     mask over the historical positions, [GR-zh] section 1.3.1); candidates unchanged.
 *     Requires slopes_pos, slopes_time >= 0 (else GENRANK_E_ARG).
 *   GENRANK_ATTN_TIME_BUCKET: the time term is -slopes_time[h]*bucket(|tau_i - tau_j|),
 *     bucket(g) = #{k : time_bounds[k] <= g} ([GR-zh] section 1.4.2, -m_t bucket(t_i - t_j);
 *     the request-gap bucketing of the time embedding).  time_bounds: DEVICE int64
 *     [n_time_bounds], non-decreasing, n_time_bounds <= 1024. */
#define GENRANK_ATTN_FULL_HISTORY 1
#define GENRANK_ATTN_TIME_BUCKET 2
typedef struct {
  const float* slopes_pos;    /* host [H] */
  const float* slopes_time;   /* host [H] */
  int32_t flags;              /* GENRANK_ATTN_* */
  int32_t n_time_bounds;      /* GENRANK_ATTN_TIME_BUCKET only */
  const int64_t* time_bounds; /* device, GENRANK_ATTN_TIME_BUCKET only */
} genrank_alibi;

/* Weights of one block.  GENRANK_BLOCK_ATTN_ONLY: y = Wo . attn(Wqkv . x).
 * GENRANK_BLOCK_PRENORM: x1 = x + Wo . attn(Wqkv . rmsnorm(x)*g1);
 *                         y = x1 + W2 . silu(W1 . rmsnorm(x1)*g2).
 * The pages fix the attention ([GR-zh] section 1.4.2, [FR-en] section 7.2) but not what
 * surrounds it in a block.  This library takes the plain pre-norm reading: RMSNorm
 * (eps 1e-6, learned gain) before the attention and before the FFN, bias-free projections,
 * residual adds, a non-gated SiLU FFN of ffn_dim, and (genrank_head_fwd) a final RMSNorm
 * and a 4-logit head with bias.  The attention-only block is the single-layer form of the
 * pages' inference description: QKV, attention, output projection, no norm or residual.
 * genrank_layer_fwd, genrank_layer_bwd and genrank_linear compute exactly these.
 * Matrices are in batch.dtype; gains are f32. */
typedef struct {
  const void* wqkv;  /* [3d, d]: rows [0,d) -> Q, [d,2d) -> K, [2d,3d) -> V; head h at h*dh */
  const void* wo;    /* [d, d] */
  const void* w1;    /* [ffn_dim, d] (PRENORM) */
  const void* w2;    /* [d, ffn_dim] (PRENORM) */
  const float* g1;   /* [d] (PRENORM) */
  const float* g2;   /* [d] (PRENORM) */
  int32_t ffn_dim;   /* PRENORM: hidden size of the FFN, multiple of 64 */
  int32_t block;     /* genrank_block */
  genrank_alibi alibi;
} genrank_layer_weights;

/* Gradients of one block, f32, same shapes as the weights.  Overwritten (not added). */
typedef struct {
  float* wqkv;
  float* wo;
  float* w1;
  float* w2;
  float* g1;
  float* g2;
} genrank_layer_grads;

/* ------------------------------------------------------------------ informational */

/* Human-readable name of a status code (static storage). */
GENRANK_API const char* genrank_status_string(int status);
/* (major << 16) | minor */
GENRANK_API int32_t genrank_version(void);

/* Bytes of workspace `op` needs for this batch (and, for the layer ops, this block:
 * `w` may be NULL for the other ops).  Writes *bytes; returns E_ARG on null pointers. */
GENRANK_API genrank_status genrank_workspace_size(int32_t op, const genrank_batch* batch,
                                      const genrank_layer_weights* w, size_t* bytes);

/* Checks HOST copies of the inputs against the preconditions the kernels assume:
 * hist_offsets[0] == 0 and non-decreasing (E_UNSORTED), timestamps non-decreasing per
 * user and req_ts[u] > the user's last timestamp (E_UNSORTED), ids in range and
 * req_ts[u] - first timestamp < 2^24 s so that relative times are exact in f32
 * (E_RANGE), rt_bounds non-decreasing (E_UNSORTED).  All pointers are HOST memory here.
 * Writes the first offending row (or -1) to *bad_row when bad_row is not NULL. */
GENRANK_API genrank_status genrank_validate_host(const genrank_batch* batch, const genrank_inputs* in,
                                     const genrank_tables* tables, int64_t* bad_row);

/* Device error word: one per GPU, sticky.  Kernels that meet an input genrank_validate_host
 * would have rejected (a caller that skipped it) neither fault nor stop: they go on as
 * stated below and set a bit of this word, which stays set until read with clear != 0.
 *   GENRANK_ERR_ID_RANGE   an item id outside [0, n_item) or an action id outside
 *                          [0, n_action) reached the embedding kernels (forward, backward,
 *                          genrank_debug_indices): the nearest valid row is used.
 *   GENRANK_ERR_HIST_LONG  a history longer than batch.max_hist reached the embedding
 *                          kernels (rows past max_hist are not written), or a history longer
 *                          than 576 actions reached the bf16 attention kernel that holds a
 *                          user's keys in LDS (chosen when batch.max_hist <= 576): keys and
 *                          queries past the 576th are ignored.
 * genrank_error_word waits for `stream`, then copies the current device's word to *word
 * (E_ARG if word is NULL, E_HIP if the word cannot be read). */
#define GENRANK_ERR_ID_RANGE 1u
#define GENRANK_ERR_HIST_LONG 2u
GENRANK_API genrank_status genrank_error_word(uint32_t* word, int32_t clear, genrank_stream_t stream);

/* ------------------------------------------------------------------ hot path */

/* Fused index derivation + five-table gather-sum ([GR-zh] section 1.4.2, the input
 * representation e = psi(x) + phi(a) + E_pe + E_ri + E_rt; section 1.4.1 for the
 * mask-action row of candidates).  Per row, in one kernel:
 *   action slot a_i (history) or n_action (candidates);
 *   position p = i - hist_offsets[u] (history) or N_u (candidates), slot min(p, n_pos-1);
 *   request index = number of distinct timestamps in the user's prefix (a candidate's
 *   prefix is the whole history plus its request), slot min(ri-1, n_ri-1);
 *   gap = t - (largest earlier distinct timestamp), bucket #{k: rt_bounds[k] <= gap},
 *   0 when there is no earlier request.
 * The five rows are summed in f32 and stored once in the residual stream's type.
 * x_out: [T, d] in batch.dtype, or f32 with batch.resid == GENRANK_RESID_F32.  d must be a
 * multiple of 8 (bf16) / 4 (f32). */
GENRANK_API genrank_status genrank_embed_sum(const genrank_batch* batch, const genrank_inputs* in,
                                 const genrank_tables* tables, void* x_out,
                                 genrank_stream_t stream);

/* Masked ALiBi flash attention forward ([GR-zh] section 1.4.2, ALiBi score with the
 * 1/sqrt(head dim) scale; [FR-en] sections 7.2.1-7.2.2, causal history mask, candidate
 * mask, position and time bias).  For each user and head:
 *   score_ij = q_i.k_j/sqrt(dh) - sp_h|p_i-p_j| - st_h|tau_i-tau_j| on allowed pairs,
 *   allowed = (i history and j <= i) or (i candidate and (j history or j == i)),
 *   o_i = softmax_j(score_ij) v_j, lse_i = log sum_j exp(score_ij)  (natural log).
 * Positions, times and the mask are derived in-kernel from hist_offsets, hist_ts and
 * req_ts; the bias is computed in registers and no T x T array is formed.
 * q, k, v: [T, ld_qkv] rows, head h at columns [h*dh, (h+1)*dh) of each (they may be
 * three views into one [T, 3d] buffer).  o: [T, ld_o], head h at h*dh.
 * lse: [T, H] f32 or NULL.  bf16 requires dh == 64; f32 requires dh <= 64.
 * bf16 kernels: when batch.max_hist <= 576 and o is 16-byte aligned with ld_o a multiple
 * of 8, one workgroup per (user, head) holds that user's whole K/V history in LDS (users
 * taken longest history first); otherwise a tiled kernel streams K/V per 128-query tile.
 * Both give the same bits.  batch.max_hist selects between them and must
 * not be below any user's history length (a longer history would be cut to 576 keys:
 * wrong results for that user, no out-of-bounds access). */
GENRANK_API genrank_status genrank_attn_fwd(const genrank_batch* batch, const int32_t* hist_offsets,
                                const int64_t* hist_ts, const int64_t* req_ts,
                                genrank_alibi alibi, const void* q, const void* k,
                                const void* v, int64_t ld_qkv, void* o, int64_t ld_o,
                                float* lse, genrank_stream_t stream);

/* Backward of genrank_attn_fwd (ALiBi is parameter-free, so it has no gradient,
 * [GR-zh] section 1.4.2).  Inputs are the forward's q, k, v, o, its lse (required) and
 * dout = dL/do ([T, ld_o]).  Writes dq, dk, dv ([T, ld_dqkv], head h at h*dh; they may
 * be views into one [T, 3d] buffer) in batch.dtype.  When cand_only_dout != 0 the
 * caller asserts that dout is zero on every history row (loss at candidate positions
 * only, [GR-zh] section 1.3.1, at the last block) and the history query rows are
 * skipped (their dq rows are written as zero).  bf16 (dh == 64): tiled MFMA kernels
 * that take P and dS as bf16 operands with f32 accumulation; ld_o must be a multiple of 8
 * and ld_dqkv of 4 (else GENRANK_E_SHAPE), o and dout 16-byte and dq, dk, dv 8-byte aligned
 * (else GENRANK_E_ARG).  f32: per-row kernels, f32 throughout.
 * ws: workspace of genrank_workspace_size(GENRANK_OP_ATTN_BWD) bytes. */
GENRANK_API genrank_status genrank_attn_bwd(const genrank_batch* batch, const int32_t* hist_offsets,
                                const int64_t* hist_ts, const int64_t* req_ts,
                                genrank_alibi alibi, const void* q, const void* k,
                                const void* v, int64_t ld_qkv, const void* o,
                                const void* dout, int64_t ld_o, const float* lse, void* dq,
                                void* dk, void* dv, int64_t ld_dqkv, int32_t cand_only_dout,
                                void* ws, size_t ws_bytes, genrank_stream_t stream);

/* genrank_attn_bwd without the workspace argument, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving or training loops, harnesses that
 * forbid allocation.  Same arguments (minus ws, ws_bytes), results and errors as
 * genrank_attn_bwd.  Its scratch (the per-row D = rowsum(dout * o), T * H f32) is a
 * library-owned 16 MiB device array, one copy per GPU, found on the first call on each
 * device and held until the process ends; this call allocates nothing.  Limit: a batch with
 * T * H * 4 + 256 > 16 MiB (T * H > 4,194,240) returns GENRANK_E_WORKSPACE.  Every call on a
 * GPU shares that GPU's array: calls that overlap on one GPU (different streams, or threads)
 * race and must be serialised by the caller.  The current device must be the one `stream`
 * and the pointers belong to.  GENRANK_E_HIP if the array cannot be located. */
GENRANK_API genrank_status genrank_attn_bwd_noalloc(const genrank_batch* batch, const int32_t* hist_offsets,
                                                    const int64_t* hist_ts, const int64_t* req_ts,
                                                    genrank_alibi alibi, const void* q, const void* k,
                                                    const void* v, int64_t ld_qkv, const void* o,
                                                    const void* dout, int64_t ld_o, const float* lse, void* dq,
                                                    void* dk, void* dv, int64_t ld_dqkv, int32_t cand_only,
                                                    genrank_stream_t stream);

/* One block forward (see genrank_layer_weights for the two block forms): the dense
 * projections (QKV, output, FFN) as bf16 MFMA GEMMs with fused residual / SiLU
 * epilogues, RMSNorm, and genrank_attn_fwd between them.
 * x_in, y_out: [T, d] residual-stream rows (batch.dtype, or f32 with GENRANK_RESID_F32: the
 * residual sums are then formed and stored in f32 and only the projections' operands are
 * rounded to batch.dtype); y_out may equal x_in (inference only: the backward needs the block
 * input).  ws: genrank_workspace_size(GENRANK_OP_LAYER_FWD) bytes.
 * flags: GENRANK_FWD_SAVE makes the workspace keep every activation genrank_layer_bwd
 * needs (keep it untouched until then); without it the FFN pre-activation is not stored.
 * Without GENRANK_FWD_SAVE, a bf16 pre-norm block with a bf16 residual stream, d >= 512,
 * d % 256 == 0 and ffn_dim % 256 == 0 fuses each RMSNorm into the GEMM that reads it: rows are scaled by
 * their 1/rms after the product with the gain-scaled weight, so the normalised rows are
 * never stored and the result differs from the saving forward by bf16 rounding only.
 * genrank_layer_kv and genrank_layer_fwd_cached take the same path under the same
 * conditions (their rows equal this forward's bit for bit). */
#define GENRANK_FWD_SAVE 1
GENRANK_API genrank_status genrank_layer_fwd(const genrank_batch* batch, const genrank_layer_weights* w,
                                 const int32_t* hist_offsets, const int64_t* hist_ts,
                                 const int64_t* req_ts, const void* x_in, void* y_out,
                                 int32_t flags, void* ws, size_t ws_bytes,
                                 genrank_stream_t stream);

/* Backward of one block.  x_in is the block's forward input (residual-stream rows), ws the
 * workspace the forward filled; dy: [T, d] gradient of the block output in batch.dtype; dx:
 * [T, d] in batch.dtype (may equal dy).
 * ws_bwd: genrank_workspace_size(GENRANK_OP_LAYER_BWD) bytes.  Gradients are f32. */
GENRANK_API genrank_status genrank_layer_bwd(const genrank_batch* batch, const genrank_layer_weights* w,
                                 const int32_t* hist_offsets, const int64_t* hist_ts,
                                 const int64_t* req_ts, const void* x_in, const void* ws,
                                 const void* dy, void* dx, genrank_layer_grads grads,
                                 int32_t cand_only_dout, void* ws_bwd, size_t ws_bwd_bytes,
                                 genrank_stream_t stream);

/* Dense projection of the block (the QKV, output and FFN layers of
 * genrank_layer_weights): y[M, N] = x[M, K] . w[N, K]^T, f32 accumulation, then
 *   GENRANK_EPI_NONE:     y = acc
 *   GENRANK_EPI_RESIDUAL: y = acc + residual   (residual [M, ldr], may equal y)
 *   GENRANK_EPI_SILU:     y = silu(acc), and pre = acc when pre is not NULL.
 *   GENRANK_EPI_RESIDUAL_F32: y = acc + residual with y and residual f32 (an f32 residual
 *                         stream, see genrank_batch.resid; ldy and ldr multiples of 4, y and
 *                         residual 16-byte aligned on the MFMA path).
 * bf16 runs on MFMA when N % 128 == 0, K % 32 == 0 and the leading dimensions are
 * multiples of 8 (K % 128 == 0 takes the kernel that streams operands straight into LDS);
 * other shapes and f32 use a plain tiled kernel.  Rows of y past M are not written. */
#define GENRANK_EPI_NONE 0
#define GENRANK_EPI_RESIDUAL 1
#define GENRANK_EPI_SILU 2
#define GENRANK_EPI_RESIDUAL_F32 3
GENRANK_API genrank_status genrank_linear(int32_t dtype, const void* x, int64_t ldx, const void* w,
                                          int64_t ldw, void* y, int64_t ldy, int64_t M, int32_t N,
                                          int32_t K, int32_t epilogue, const void* residual,
                                          int64_t ldr, void* pre, int64_t ldpre,
                                          genrank_stream_t stream);

/* Backward of genrank_linear without an epilogue (y = x w^T; a residual or SiLU epilogue
 * is differentiated by the caller first):
 *   dx[M, K] = dy[M, N] . w[N, K]   in dtype ([M, lddx]),
 *   dw[N, K] = dy^T . x             f32 ([N, lddw]), overwritten.
 * Either dx or dw may be NULL to skip it.  bf16: dx transposes w into the workspace and
 * runs on the genrank_linear kernels; dw runs on an MFMA kernel that transposes tiles of
 * dy and x on their way into LDS and splits the M rows over several workgroups per output
 * tile (f32 partial tiles in the workspace, summed in a fixed order, so the result does
 * not depend on scheduling).  Its MFMA path needs N and K multiples of 8, ldx and ldy
 * multiples of 8 and lddw of 4 with 16-byte aligned x, dy, dw; other layouts and f32 take a
 * plain tiled kernel.  ws: genrank_linear_bwd_workspace() bytes, 16-byte aligned
 * (GENRANK_E_WORKSPACE if short). */
GENRANK_API genrank_status genrank_linear_bwd_workspace(int32_t dtype, int64_t M, int32_t N, int32_t K,
                                                        size_t* bytes);
GENRANK_API genrank_status genrank_linear_bwd(int32_t dtype, const void* x, int64_t ldx, const void* w,
                                              int64_t ldw, const void* dy, int64_t ldy, void* dx,
                                              int64_t lddx, float* dw, int64_t lddw, int64_t M,
                                              int32_t N, int32_t K, void* ws, size_t ws_bytes,
                                              genrank_stream_t stream);

/* The pre-norm block's RMSNorm on its own (the pages are silent on the block's internals;
 * reading: pre-RMSNorm blocks, eps 1e-6): y[r] = x[r] / sqrt(mean(x[r]^2) + 1e-6) * g, per
 * row.  x: [rows, d] in x_dtype (the residual stream); y: [rows, d] in y_dtype (the next
 * projection's operand); g: [d] f32.  Supported (x_dtype, y_dtype): (BF16, BF16), (F32, BF16),
 * (F32, F32) (else GENRANK_E_DTYPE).  This is the normalisation genrank_layer_fwd runs
 * without GENRANK_FWD_SAVE on an f32 residual stream (and with it on any stream). */
GENRANK_API genrank_status genrank_rmsnorm(int32_t x_dtype, int32_t y_dtype, const void* x, const float* g, void* y,
                                           int64_t rows, int32_t d, genrank_stream_t stream);

/* Per-candidate action logits ([GR-zh] section 1.2: predictions for a set of predefined
 * tasks): logits[c, t] = (rmsnorm(x[T_h + c]) * g_final) . w_head[t] + b_head[t].
 * x: [T, d] residual-stream rows (batch.dtype, or f32 with GENRANK_RESID_F32); g_final [d],
 * w_head [n_tasks, d], b_head [n_tasks] f32;
 * logits: [B*m, n_tasks] f32.  n_tasks in 1..8. */
GENRANK_API genrank_status genrank_head_fwd(const genrank_batch* batch, const void* x, const float* g_final,
                                const float* w_head, const float* b_head, int32_t n_tasks,
                                float* logits, genrank_stream_t stream);

/* Backward of genrank_head_fwd.  x as genrank_head_fwd; dx: [T, d] in batch.dtype; history rows
 * are set to zero (the loss is taken at candidate positions only, [GR-zh] section 1.3.1).
 * dg_final [d], dw_head [n_tasks, d], db_head [n_tasks]: f32, overwritten; they are sums over
 * the candidate rows formed in a fixed order (per-block partials in ws, then summed), so
 * the result does not depend on scheduling.  ws: genrank_workspace_size(GENRANK_OP_HEAD_BWD)
 * bytes (sized for n_tasks <= 4). */
GENRANK_API genrank_status genrank_head_bwd(const genrank_batch* batch, const void* x, const float* g_final,
                                const float* w_head, int32_t n_tasks, const float* dlogits,
                                void* dx, float* dg_final, float* dw_head, float* db_head,
                                void* ws, size_t ws_bytes, genrank_stream_t stream);

/* The head of genrank_head_fwd at a list of rows, for a loss taken at candidate and some
 * history positions (the ablation of [GR-zh] section 1.3.1; the default training loss is
 * at candidate positions only).  x: [n_x_rows, d] in dtype (GENRANK_BF16 or GENRANK_F32),
 * row-major; rows: DEVICE int32 [n_rows], each in [0, n_x_rows) (not checked on the
 * device: an index outside reads outside x); logits: [n_rows, n_tasks] f32, row r for
 * x row rows[r].  Errors: GENRANK_E_DTYPE, GENRANK_E_ARG (null pointer), GENRANK_E_SHAPE
 * (n_rows < 0, d < 1, n_tasks outside 1..8). */
GENRANK_API genrank_status genrank_head_fwd_rows(int32_t dtype, int32_t d, const void* x, int64_t n_rows,
                                     const int32_t* rows, const float* g_final, const float* w_head,
                                     const float* b_head, int32_t n_tasks, float* logits,
                                     genrank_stream_t stream);

/* Backward of genrank_head_fwd_rows.  x: [n_x_rows, d] in x_dtype (dtype, or GENRANK_F32 for an
 * f32 residual stream); dx: [n_x_rows, d] in dtype, overwritten: each listed
 * row gets the head's gradient, every other row zero.  The rows must be distinct (a
 * repeated row gets one of its gradients, not their sum).  dg_final, dw_head, db_head: as
 * genrank_head_bwd (f32, overwritten, fixed summation order).  ws: at least
 * genrank_workspace_size(GENRANK_OP_HEAD_BWD) of a batch with the same d.  Errors as
 * genrank_head_fwd_rows, plus n_tasks > 4 or d > 1024 or d % 4 != 0 -> GENRANK_E_SHAPE and
 * GENRANK_E_WORKSPACE. */
GENRANK_API genrank_status genrank_head_bwd_rows(int32_t x_dtype, int32_t dtype, int32_t d, int64_t n_x_rows,
                                     const void* x,
                                     int64_t n_rows, const int32_t* rows, const float* g_final,
                                     const float* w_head, int32_t n_tasks, const float* dlogits, void* dx,
                                     float* dg_final, float* dw_head, float* db_head, void* ws,
                                     size_t ws_bytes, genrank_stream_t stream);

/* Mean sigmoid binary cross-entropy over n rows x n_tasks logits and its gradient:
 * loss[0] = mean(softplus(z) - y z); dlogits = (sigmoid(z) - y) / (n * n_tasks).
 * logits, labels, dlogits: [n, n_tasks] f32; loss: [1] f32 (device). */
GENRANK_API genrank_status genrank_bce_loss(int64_t n, int32_t n_tasks, const float* logits,
                                const float* labels, float* loss, float* dlogits,
                                genrank_stream_t stream);

/* Adjoint of genrank_embed_sum: row r of a table's gradient is the sum of dx over the
 * batch rows whose slot in that table is r.  dx: [T, d] in batch.dtype.  Outputs, f32,
 * overwritten:
 *   item gradient, sparse: *n_items (device int32) distinct item ids in ascending order
 *     in item_ids[0 .. n_items) ([T] capacity), their gradient rows in item_rows
 *     ([T, d] capacity; rows past n_items untouched);
 *   d_action [n_action + 1, d], d_pos [n_pos, d], d_ri [n_ri, d], d_rt [n_rt, d]: dense,
 *     zero where no row maps.
 * The rows are grouped by slot with a radix sort and each group is summed in ascending row
 * order (no atomics): the result does not depend on scheduling.  5 T must be below 2^31.
 * dx is in batch.dtype whatever batch.resid says.
 * ws: genrank_workspace_size(GENRANK_OP_EMBED_BWD) bytes. */
GENRANK_API genrank_status genrank_embed_bwd(const genrank_batch* batch, const genrank_inputs* in,
                                             const genrank_tables* tables, const void* dx,
                                             int32_t* item_ids, float* item_rows, int32_t* n_items,
                                             float* d_action, float* d_pos, float* d_ri, float* d_rt,
                                             void* ws, size_t ws_bytes, genrank_stream_t stream);

/* ------------------------------------------------------------------ serving with cached history
 *
 * History rows never depend on candidates (history queries only see earlier history keys,
 * [GR-zh] 1.4.2 mask; [FR-en] 7.2.1), so a user's per-block history keys and values can be
 * computed once and reused for every later request: a request then runs its m candidate
 * rows only, each candidate attending to the cached history and to itself.  The results
 * equal the candidate rows of the full forward (bit for bit on this library's kernels).
 * Layout of a cache for one block: kv [T_h, ld_kv] with the keys in columns [0, d) and the
 * values in [d, 2d), head h at h * dh in each; rows in the batch's history order.
 * bf16 with dh == 64 for the attention. */

/* genrank_embed_sum for the candidate rows only: x_cand [B*m, d] (residual-stream type), row
 * u*m + k. */
GENRANK_API genrank_status genrank_embed_sum_cand(const genrank_batch* batch, const genrank_inputs* in,
                                                  const genrank_tables* tables, void* x_cand,
                                                  genrank_stream_t stream);

/* The attention of genrank_attn_fwd for the candidate rows only: q, k, v, o: [B*m] rows
 * (row stride ld_qkv, ld_o; lse [B*m, H] or NULL); the history keys and values come from
 * k_hist, v_hist ([T_h] rows, stride ld_hist).  ld_qkv, ld_hist multiples of 8, ld_o of 4;
 * q, k, v, k_hist, v_hist 16-byte and o 8-byte aligned (else GENRANK_E_SHAPE / E_ARG).
 * The tiled kernel of genrank_attn_fwd, which reads a user's history once per 128-candidate
 * tile; candidate rows get the same bits as from genrank_attn_fwd. */
GENRANK_API genrank_status genrank_attn_fwd_cached(const genrank_batch* batch, const int32_t* hist_offsets,
                                                   const int64_t* hist_ts, const int64_t* req_ts,
                                                   genrank_alibi alibi, const void* q, const void* k,
                                                   const void* v, int64_t ld_qkv, const void* k_hist,
                                                   const void* v_hist, int64_t ld_hist, void* o, int64_t ld_o,
                                                   float* lse, genrank_stream_t stream);

/* A block's history keys and values: kv [T_h, ld_kv] (see above) from the block's input on
 * the history rows, x_hist [T_h, d] residual-stream rows (the top block needs nothing else of the history: its
 * history outputs are never read).  ws: genrank_workspace_size(GENRANK_OP_LAYER_KV). */
GENRANK_API genrank_status genrank_layer_kv(const genrank_batch* batch, const genrank_layer_weights* w,
                                            const void* x_hist, void* kv, int64_t ld_kv, void* ws,
                                            size_t ws_bytes, genrank_stream_t stream);

/* genrank_layer_fwd on the candidate rows only: x_cand, y_cand [B*m, d] residual-stream rows
 * (equal only for GENRANK_BLOCK_PRENORM), history keys and values from kv_hist ([T_h, ld_kv]).
 * ws: genrank_workspace_size(GENRANK_OP_LAYER_FWD_CACHED). */
GENRANK_API genrank_status genrank_layer_fwd_cached(const genrank_batch* batch, const genrank_layer_weights* w,
                                                    const int32_t* hist_offsets, const int64_t* hist_ts,
                                                    const int64_t* req_ts, const void* kv_hist, int64_t ld_kv,
                                                    const void* x_cand, void* y_cand, void* ws, size_t ws_bytes,
                                                    genrank_stream_t stream);

/* ------------------------------------------------------------------ debug exports */

/* The per-row indices genrank_embed_sum derives, written as int32 out[6][T]:
 * out[0] action slot, out[1] position id (unclamped), out[2] position slot,
 * out[3] request index (unclamped), out[4] request-index slot, out[5] time-gap bucket. */
GENRANK_API genrank_status genrank_debug_indices(const genrank_batch* batch, const genrank_inputs* in,
                                     const genrank_tables* tables, int32_t* out,
                                     genrank_stream_t stream);

/* The attention mask of user `user` as the f32 attention kernels evaluate it, on sequence
 * slots (0..N_u-1 history, N_u..N_u+m-1 candidates): out[i*L_cap + j] = 1 if i and j are
 * below L = N_u + m and slot i may attend slot j, else 0.  out: [L_cap * L_cap] uint8;
 * L_cap >= 1 (pass max_hist + m to see every user whole). */
GENRANK_API genrank_status genrank_debug_mask(const genrank_batch* batch, const int32_t* hist_offsets,
                                  int32_t user, int32_t L_cap, uint8_t* out,
                                  genrank_stream_t stream);

/* ---- HSTU-style comparison path ("一、 GenRank [2025]" section 1.4.1: the interleaved
 * item/action organisation the action-oriented sequence replaces; "The Overall Generative
 * Ranking Paradigm" section 7.2.2: a learned relative bias).  Measured against the ALiBi path;
 * not part of the ranking forward.
 * User u's sequence: slots 0 .. 2N_u-1 alternate the item and the action token of history
 * action i (both at time hist_ts[i], position = slot), then the m candidates (position 2N_u,
 * time req_ts[u]); L_u = 2N_u + m.  Its bias matrix is [L_u, P_u] bf16 (row pitch
 * P_u = L_u rounded up to a multiple of 8) at element offset rab_offsets[u]:
 *   rab[i][j] = pos_table[min(|p_i - p_j|, n_pos - 1)] + time_table[#{k : time_bounds[k] <= |t_i - t_j|}]
 * summed in f32, rounded to bf16 (round to nearest even); pad columns are 0.
 * q/k/v/o rows: [0, 2 T_h) the interleaved history, user after user (user u at rows
 * 2 hist_offsets[u] ..), then candidate c of user u at row 2 T_h + u m + c. */

/* rab_offsets (device int64 [B + 1]): exclusive prefix sums of L_u * P_u; rab_offsets[B] is
 * the element count of the whole bias buffer. */
GENRANK_API genrank_status genrank_hstu_rab_layout(const genrank_batch* batch, const int32_t* hist_offsets,
                                       int64_t* rab_offsets, genrank_stream_t stream);
/* Materialises every user's bias matrix into rab (device, rab_offsets[B] bf16 elements).
 * pos_table: f32 [n_pos] (n_pos >= 1); time_table: f32 [n_time]; time_bounds: int64
 * [n_time - 1], non-decreasing.  E_SHAPE if 2 * max_hist + m > 2048, n_pos > 1024 or
 * n_time - 1 > 1024. */
GENRANK_API genrank_status genrank_hstu_rab(const genrank_batch* batch, const int32_t* hist_offsets,
                                const int64_t* hist_ts, const int64_t* req_ts,
                                const float* pos_table, int32_t n_pos, const float* time_table,
                                const int64_t* time_bounds, int32_t n_time,
                                const int64_t* rab_offsets, void* rab, genrank_stream_t stream);
/* Attention over the interleaved sequences: softmax(q k^T / sqrt(dh) + rab) over the mask
 * of genrank_attn_fwd with 2N_u history slots (history causal, candidates see every history
 * slot and themselves), o = P v, lse (f32 [rows, H], natural log, or NULL).  bf16 only,
 * dh = 64, same strides and errors as genrank_attn_fwd. */
GENRANK_API genrank_status genrank_hstu_attn_fwd(const genrank_batch* batch, const int32_t* hist_offsets,
                                     const void* rab, const int64_t* rab_offsets, const void* q,
                                     const void* k, const void* v, int64_t ld_qkv, void* o,
                                     int64_t ld_o, float* lse, genrank_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* GENRANK_H */
