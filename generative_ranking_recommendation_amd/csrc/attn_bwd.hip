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

#include <mutex>
#include <type_traits>

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
  int flags;              // GENRANK_ATTN_* variants
  const int64_t* tb;      // bucket edges (time-bucket variant)
  int n_tb;
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
  const int64_t gap = ti > tj ? ti - tj : tj - ti;
  const float dt = (a.flags & GENRANK_ATTN_TIME_BUCKET) ? static_cast<float>(bucket_search_global(a.tb, a.n_tb, gap))
                                                        : static_cast<float>(gap);
  return -a.sp[h] * fabsf(static_cast<float>(pi - pj)) - a.st[h] * dt;
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
  const bool full = (a.flags & GENRANK_ATTN_FULL_HISTORY) != 0;
  for (int j = 0; j < L; ++j) {
    if (!attn_allowed(s.i, j, s.N, full)) continue;
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
  const bool full = (a.flags & GENRANK_ATTN_FULL_HISTORY) != 0;
  const int i_begin = (a.cand_only && j < s.N) ? s.N : (full && j < s.N ? 0 : j);
  for (int i = i_begin; i < L; ++i) {
    if (!attn_allowed(i, j, s.N, full)) continue;
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

// ------------------------------------------------------------------ MFMA kernels (bf16, dh = 64)
// The same products as above, on 64 x 64 tiles with v_mfma_f32_16x16x32_bf16 and the
// forward's conventions: scores in log2 units, the bias as w_j - w_i against a reference
// point of the query tile (its first query, or the candidates' shared (N, request time)), so
//   P_ij = exp2(q_i.k_j scale2 + w_j - c_i),  c_i = w_i + lse_i log2(e).
// dQ kernel: one 256-thread workgroup per 64-query tile (4 waves x 16 queries, one query per
//   lane as in the forward): per key tile S^T = K Q^T and dP^T = V dO^T (K, V rows in LDS,
//   Q, dO fragments in registers), dS^T = P^T (dP^T - D), dQ^T += K^T dS^T (K^T in LDS with
//   its keys permuted to match the registers).  Candidate tiles also take the candidate's
//   own key, which gives the candidate rows their whole dK and dV.  Its prologue forms
//   D_i = dO_i . O_i of its queries and stores it for the dK/dV kernel.
// dK/dV kernel: one workgroup per KT = 4 KW history keys (4 waves x KW keys, KW = 16; with
//   KW = 32 two 16-key blocks per wave would share every Q and dO fragment read, but need
//   250 VGPRs, two waves per SIMD, and 16 keys at 165 VGPRs and three waves per SIMD
//   measured faster): per 64-query tile that sees the keys (every later history tile unless
//   the loss sits at the candidates only, then every candidate tile) S = Q K^T and
//   dP = dO V^T (Q, dO rows in LDS, K, V fragments in registers), dV^T += dO^T P and
//   dK^T += Q^T dS (Q^T, dO^T read transposed out of LDS).
constexpr int TB = 64;      // rows per tile (queries or keys)
constexpr int KW = 16;      // keys per wave in the dK/dV kernel
constexpr int KB = KW / 16; // its 16-key blocks
constexpr int KT = 4 * KW;  // keys per dK/dV workgroup
constexpr int DHB = 64;     // head dim
constexpr int PLD = 72;     // LDS row pitch (bf16)
constexpr int BWCH = 512;   // keys whose bias terms sit in LDS at a time
constexpr int BUF_DWORD3_B = 0x00020000;
constexpr float LOG2E_B = 1.4426950408889634f;

struct BwdMArgs {
  const int32_t* offsets;
  const int64_t* ts;
  const int64_t* req;
  const bf16_t* q; const bf16_t* k; const bf16_t* v; int64_t ld_qkv;
  const bf16_t* o; const bf16_t* dout; int64_t ld_o;
  const float* lse;
  float* delta;  // D per (row, head): written by the dQ kernel, read by the dK/dV kernel
  bf16_t* dq; bf16_t* dk; bf16_t* dv; int64_t ld_d;
  float sp2[GENRANK_MAX_HEADS];
  float st2[GENRANK_MAX_HEADS];
  float scale2, scale;
  int B, m, H, hist_tiles, cand_tiles, cand_only;
  int64_t T_h;
  const int64_t* tb;  // bucket edges (time-bucket variant), their count, pow2 >= count + 1
  int n_tb, tb_p2;
};
constexpr int BVAR_FULL = 1, BVAR_TBUCKET = 2;  // the ALiBi variants, as template bits

__device__ __forceinline__ float bxor16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float bxor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float dot16(const uint4& a0, const uint4& a1, const uint4& b0, const uint4& b1) {
  float fa[8], fb[8], s = 0.f;
  unpack8(a0, fa); unpack8(b0, fb);
#pragma unroll
  for (int e = 0; e < 8; ++e) s += fa[e] * fb[e];
  unpack8(a1, fa); unpack8(b1, fb);
#pragma unroll
  for (int e = 0; e < 8; ++e) s += fa[e] * fb[e];
  return s;
}
// tile staging: a thread moves rows pr and pr + 32, columns 8ch..8ch+7 of a 64 x 64 tile
// into its row-major LDS copy (pr = tid / 8, ch = tid % 8: eight lanes cover a row's 128
// bytes, so global loads read whole rows, and the two rows a 16-lane group writes together
// are neighbours, which meet on at most one 16-byte bank group at this pitch)
__device__ __forceinline__ void stash_rows(bf16_t* rows, int pr, int ch, const uint4& ra, const uint4& rb) {
  *reinterpret_cast<uint4*>(rows + pr * PLD + ch * 8) = ra;
  *reinterpret_cast<uint4*>(rows + (pr + 32) * PLD + ch * 8) = rb;
}
typedef short bv4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bv4i16_t lds_bv4i16_t;
// The transposed operand X^T (columns nb*16 .. nb*16+15 of a row-major 64 x 64 LDS tile as
// rows, 32 of its rows as the k axis) of a product whose other operand packs two 16-row
// result blocks (pack_blocks): lane (l16, g4) gets column nb*16 + l16 at rows
// 32 ks + 4 g4 + e and 32 ks + 16 + 4 g4 + e (e = 0..3), the order of those packed values.
// gfx950's transposing read gives within each 16-lane group lane j, element e, the element
// j % 4 of what lane 4 e + j / 4 addressed: lane 4 e + r addresses row 4 g4 + e, columns
// nb*16 + 4 r .. + 3.
__device__ __forceinline__ bf16x8_t tr_operand(const bf16_t* tile, int nb, int ks, int l16, int g4) {
  const bf16_t* p = tile + (ks * 32 + 4 * g4 + (l16 >> 2)) * PLD + nb * 16 + (l16 & 3) * 4;
  const bv4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_bv4i16_t*)p);
  const bv4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_bv4i16_t*)(p + 16 * PLD));
  const bv4i16_t both[2] = {lo, hi};
  return __builtin_bit_cast(bf16x8_t, both);
}
// pack the 8 values a lane holds for two 16-row result blocks into an MFMA operand
__device__ __forceinline__ bf16x8_t pack_blocks(const f32x4_t& lo, const f32x4_t& hi) {
  uint4 p;
  p.x = pack_bf16x2(lo[0], lo[1]);
  p.y = pack_bf16x2(lo[2], lo[3]);
  p.z = pack_bf16x2(hi[0], hi[1]);
  p.w = pack_bf16x2(hi[2], hi[3]);
  return as_bf16x8(p);
}

template <int VAR>
__global__ void __launch_bounds__(256) attn_bwd_dq_kernel(BwdMArgs a) {
  constexpr bool FULL = (VAR & BVAR_FULL) != 0, TBK = (VAR & BVAR_TBUCKET) != 0;
  constexpr bool CAN_FAR = !TBK;  // the bucketed variants' key terms hold the position part only
  __shared__ __attribute__((aligned(16))) bf16_t sK[2][TB * PLD];
  __shared__ __attribute__((aligned(16))) bf16_t sV[2][TB * PLD];
  __shared__ __attribute__((aligned(16))) float sW[BWCH];
  __shared__ __attribute__((aligned(16))) int32_t sT[BWCH];  // key times relative to the reference
  __shared__ int32_t sTB[TBK ? ATTN_MAX_TIME_BOUNDS : 1];
  __shared__ uint32_t sLUT[TBK ? BK_CELLS : 1];  // bucket table over the gap

  const int u = blockIdx.x / a.H;
  const int h = blockIdx.x - u * a.H;
  const int y = blockIdx.y;
  const int64_t off = a.offsets[u];
  const int N = a.offsets[u + 1] - a.offsets[u];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;

  bool is_cand;
  int q0, nq, n_tiles;
  int64_t qrow0;
  if (y < a.cand_tiles) {
    is_cand = true;
    q0 = y * TB;
    if (q0 >= a.m) return;
    nq = min(TB, a.m - q0);
    qrow0 = a.T_h + static_cast<int64_t>(u) * a.m + q0;
    n_tiles = (N + TB - 1) / TB;
  } else {
    is_cand = false;
    q0 = (a.hist_tiles - 1 - (y - a.cand_tiles)) * TB;  // the latest (longest) query tiles first
    if (q0 >= N) return;
    nq = min(TB, N - q0);
    qrow0 = off + q0;
    n_tiles = FULL ? (N + TB - 1) / TB : (q0 + nq + TB - 1) / TB;
    if (a.cand_only) {  // the history rows carry no gradient: dQ = 0
      for (int e = tid; e < nq * (DHB / 4); e += 256) {
        const int r = e / (DHB / 4), c = (e - r * (DHB / 4)) * 4;
        *reinterpret_cast<uint2*>(a.dq + (qrow0 + r) * a.ld_d + h * DHB + c) = make_uint2(0u, 0u);
      }
      return;
    }
  }

  const float sp2 = a.sp2[h], st2 = a.st2[h];
  const int p_ref = is_cand ? N : q0;
  const int64_t ts_ref = is_cand ? a.req[u] : a.ts[off + q0];
  // with the bucketed time term, w holds the position term and sT the key time
  auto load_w = [&](int wbase) {
    for (int j = tid; j < BWCH; j += 256) {
      const int key = wbase + j;
      const int32_t tk = key < N ? static_cast<int32_t>(a.ts[off + key] - ts_ref) : 0;
      sW[j] = key < N ? (TBK ? sp2 * static_cast<float>(key - p_ref)
                             : sp2 * static_cast<float>(key - p_ref) + st2 * static_cast<float>(tk))
                      : 0.f;
      sT[j] = tk;
    }
  };
  if constexpr (TBK)
    for (int k = tid; k < a.tb_p2; k += 256) {
      const int64_t b = k < a.n_tb ? a.tb[k] : INT64_MAX;
      sTB[k] = b > INT32_MAX ? INT32_MAX : (b < INT32_MIN ? INT32_MIN : static_cast<int32_t>(b));
    }
  const int kt_first = n_tiles - 1;
  int wbase = n_tiles > 0 ? (kt_first * TB / BWCH) * BWCH : 0;

  // this lane's query
  const int q_local = wave * 16 + l16;
  const bool q_valid = q_local < nq;
  const int64_t qrow = qrow0 + min(q_local, nq - 1);
  const int q_slot = is_cand ? N + q0 + q_local : q0 + q_local;
  const int k_lim = (is_cand || FULL) ? N - 1 : min(q_slot, N - 1);
  const int64_t ro = qrow * a.ld_qkv + h * DHB;
  const int64_t rdo = qrow * a.ld_o + h * DHB;
  const uint4 qa = *reinterpret_cast<const uint4*>(a.q + ro + g4 * 8);
  const uint4 qb = *reinterpret_cast<const uint4*>(a.q + ro + g4 * 8 + 32);
  const uint4 da = *reinterpret_cast<const uint4*>(a.dout + rdo + g4 * 8);
  const uint4 db = *reinterpret_cast<const uint4*>(a.dout + rdo + g4 * 8 + 32);
  bf16x8_t qf[2] = {as_bf16x8(qa), as_bf16x8(qb)};
  bf16x8_t dof[2] = {as_bf16x8(da), as_bf16x8(db)};
  const float lse2 = a.lse[qrow * a.H + h] * LOG2E_B;
  // D_i = dO_i . O_i over the head's 64 dimensions (16 per lane of the query's lane group);
  // stored for the dK/dV kernel, which runs after this one
  const uint4 oa = *reinterpret_cast<const uint4*>(a.o + rdo + g4 * 8);
  const uint4 ob = *reinterpret_cast<const uint4*>(a.o + rdo + g4 * 8 + 32);
  const float Di = bxor32_sum(bxor16_sum(dot16(da, db, oa, ob)));
  if (q_valid && g4 == 0) a.delta[qrow * a.H + h] = Di;
  float w_i = 0.f;
  int32_t tq = 0;  // the query's time relative to ts_ref
  if (!is_cand) {
    tq = static_cast<int32_t>(a.ts[off + min(q_slot, N - 1)] - ts_ref);
    w_i = TBK ? sp2 * static_cast<float>(q_slot - p_ref)
              : sp2 * static_cast<float>(q_slot - p_ref) + st2 * static_cast<float>(tq);
  }
  // a wave whose queries lie far from the tile's reference point forms each bias exactly from
  // the pair's own position and time differences (its row term is then 0)
  const bool far = CAN_FAR && __builtin_amdgcn_ballot_w64(q_valid && fabsf(w_i) > BIAS_FAR_LOG2) != 0;
  const float c_i = far ? lse2 : w_i + lse2;

  f32x4_t accQ[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) accQ[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // a candidate's own key: P_ii, dS_ii from dot products over the lane group's 16 dims, then
  // dQ_i += dS_ii k_i, dK_i = dS_ii q_i scale, dV_i = P_ii dO_i (the candidate key's only terms)
  if (is_cand) {
    const uint4 ka = *reinterpret_cast<const uint4*>(a.k + ro + g4 * 8);
    const uint4 kb = *reinterpret_cast<const uint4*>(a.k + ro + g4 * 8 + 32);
    const uint4 va = *reinterpret_cast<const uint4*>(a.v + ro + g4 * 8);
    const uint4 vb = *reinterpret_cast<const uint4*>(a.v + ro + g4 * 8 + 32);
    const float sqk = bxor32_sum(bxor16_sum(dot16(qa, qb, ka, kb)));
    const float sdv = bxor32_sum(bxor16_sum(dot16(da, db, va, vb)));
    float self_bias = 0.f;  // the bucketed time term of the gap 0
    if constexpr (TBK) self_bias = -st2 * static_cast<float>(bucket_search_global(a.tb, a.n_tb, 0));
    const float p = __builtin_amdgcn_exp2f(sqk * a.scale2 + self_bias - c_i);
    const float ds = p * (sdv - Di);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int dcol = nb * 16 + g4 * 4;
      const uint2 kk = *reinterpret_cast<const uint2*>(a.k + ro + dcol);
      const uint2 qq = *reinterpret_cast<const uint2*>(a.q + ro + dcol);
      const uint2 dd = *reinterpret_cast<const uint2*>(a.dout + rdo + dcol);
      const float kf[4] = {__uint_as_float(kk.x << 16), __uint_as_float(kk.x & 0xFFFF0000u),
                           __uint_as_float(kk.y << 16), __uint_as_float(kk.y & 0xFFFF0000u)};
      const float qv[4] = {__uint_as_float(qq.x << 16), __uint_as_float(qq.x & 0xFFFF0000u),
                           __uint_as_float(qq.y << 16), __uint_as_float(qq.y & 0xFFFF0000u)};
      const float dv[4] = {__uint_as_float(dd.x << 16), __uint_as_float(dd.x & 0xFFFF0000u),
                           __uint_as_float(dd.y << 16), __uint_as_float(dd.y & 0xFFFF0000u)};
#pragma unroll
      for (int i = 0; i < 4; ++i) accQ[nb][i] += ds * kf[i];
      if (q_valid) {
        const int64_t dro = qrow * a.ld_d + h * DHB + dcol;
        uint2 o;
        o.x = pack_bf16x2(ds * qv[0] * a.scale, ds * qv[1] * a.scale);
        o.y = pack_bf16x2(ds * qv[2] * a.scale, ds * qv[3] * a.scale);
        *reinterpret_cast<uint2*>(a.dk + dro) = o;
        o.x = pack_bf16x2(p * dv[0], p * dv[1]);
        o.y = pack_bf16x2(p * dv[2], p * dv[3]);
        *reinterpret_cast<uint2*>(a.dv + dro) = o;
      }
    }
  }

  // K/V staging (rows pr, pr + 32, columns 8ch..8ch+7), one tile ahead, buffer loads over the
  // user's history rows (rows past it read as zero; the whole offset sits in the vector
  // operand, which the range check covers)
  const int pr = tid >> 3, ch = tid & 7;
  const uint32_t row_bytes = static_cast<uint32_t>(a.ld_qkv) * 2u;
  const uint32_t hist_bytes = static_cast<uint32_t>(N) * row_bytes;
  const __amdgpu_buffer_rsrc_t rsK = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t*>(a.k + off * a.ld_qkv), static_cast<short>(0), hist_bytes, BUF_DWORD3_B);
  const __amdgpu_buffer_rsrc_t rsV = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t*>(a.v + off * a.ld_qkv), static_cast<short>(0), hist_bytes, BUF_DWORD3_B);
  const uint32_t voA = static_cast<uint32_t>(pr) * row_bytes + (h * DHB + ch * 8) * 2u;
  const uint32_t voB = voA + 32u * row_bytes;
  uint4 rka, rkb, rva, rvb;
  auto fetch = [&](int kt) {
    const uint32_t so = static_cast<uint32_t>(kt * TB) * row_bytes;
    rka = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsK, voA + so, 0, 0));
    rkb = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsK, voB + so, 0, 0));
    rva = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsV, voA + so, 0, 0));
    rvb = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsV, voB + so, 0, 0));
  };
  auto stash = [&](int buf) {
    stash_rows(sK[buf], pr, ch, rka, rkb);
    stash_rows(sV[buf], pr, ch, rva, rvb);
  };
  if (n_tiles > 0) {
    load_w(wbase);
    fetch(kt_first);
    stash(0);
  }
  asm volatile("" : "+v"(qf[0]), "+v"(qf[1]), "+v"(dof[0]), "+v"(dof[1]));
  __syncthreads();
  if constexpr (TBK) {
    bucket_table_build(sLUT, sTB, a.tb_p2, tid, 256);
    __syncthreads();
  }

  const int klim_min = (is_cand || FULL) ? N - 1 : q0;
  for (int it = 0; it < n_tiles; ++it) {
    const int kt = kt_first - it;
    const int buf = it & 1;
    const int base = kt * TB;
    if (base < wbase) {
      __syncthreads();
      wbase -= BWCH;
      load_w(wbase);
      __syncthreads();
    }
    if (kt > 0) fetch(kt - 1);
    const bool masked = base + TB - 1 > klim_min;
    f32x4_t s[4], dp[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      s[kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      dp[kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8_t kf = as_bf16x8(*reinterpret_cast<const uint4*>(&sK[buf][(kb * 16 + l16) * PLD + ks * 32 + g4 * 8]));
        const bf16x8_t vf = as_bf16x8(*reinterpret_cast<const uint4*>(&sV[buf][(kb * 16 + l16) * PLD + ks * 32 + g4 * 8]));
        s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[ks], s[kb], 0, 0, 0);
        dp[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, dof[ks], dp[kb], 0, 0, 0);
      }
    }
    // P^T and dS^T for keys base + kb*16 + 4*g4 + i of this lane's query.  F: the exact bias
    // of each pair (rare).  MASK 0: no key limit, 1: the key limit, 2: the key limit on masked
    // tiles, decided at run time (one instance for both).
    auto pds = [&](auto FARC, auto MASKC) {
      constexpr bool F = decltype(FARC)::value;
      constexpr int MASK = decltype(MASKC)::value;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const float4 w = reinterpret_cast<const float4*>(sW)[((base - wbase) >> 2) + kb * 4 + g4];
        const float wv[4] = {w.x, w.y, w.z, w.w};
        int32_t tkv[4] = {0, 0, 0, 0};
        if constexpr (F || TBK) {
          const int4 t4 = reinterpret_cast<const int4*>(sT)[((base - wbase) >> 2) + kb * 4 + g4];
          tkv[0] = t4.x; tkv[1] = t4.y; tkv[2] = t4.z; tkv[3] = t4.w;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float arg;
          if constexpr (F) {  // the exact bias of the pair, log2 units
            const float b = sp2 * static_cast<float>(base + kb * 16 + g4 * 4 + i - q_slot) +
                            st2 * static_cast<float>(tkv[i] - tq);
            arg = s[kb][i] * a.scale2 + (FULL ? -fabsf(b) : b) - c_i;
          } else if constexpr (!FULL && !TBK) {
            arg = __builtin_fmaf(s[kb][i], a.scale2, wv[i] - c_i);
          } else {
            // fully visible: -|w_j - w_i|; bucketed time: - s' bucket(|t_i - t_j|)
            arg = s[kb][i] * a.scale2 + (FULL ? -fabsf(wv[i] - w_i) : wv[i] - w_i) - lse2;
            if constexpr (TBK) arg -= st2 * static_cast<float>(bucket_lookup(sLUT, sTB, a.tb_p2, abs(tq - tkv[i])));
          }
          float p = __builtin_amdgcn_exp2f(arg);
          if constexpr (MASK == 1) {
            if (base + kb * 16 + g4 * 4 + i > k_lim) p = 0.f;
          } else if constexpr (MASK == 2) {
            if (masked && base + kb * 16 + g4 * 4 + i > k_lim) p = 0.f;
          }
          s[kb][i] = p * (dp[kb][i] - Di);
        }
      }
    };
    using FT = std::integral_constant<bool, true>;
    using FF = std::integral_constant<bool, false>;
    if constexpr (CAN_FAR) {
      if (far) pds(FT{}, std::integral_constant<int, 2>{});
      else if (masked) pds(FF{}, std::integral_constant<int, 1>{});
      else pds(FF{}, std::integral_constant<int, 0>{});
    } else {  // the bucketed variants: one instance
      pds(FF{}, std::integral_constant<int, 2>{});
    }
    // dQ^T += K^T dS^T
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8_t dsf = pack_blocks(s[2 * ks], s[2 * ks + 1]);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const bf16x8_t ktf = tr_operand(sK[buf], nb, ks, l16, g4);
        accQ[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ktf, dsf, accQ[nb], 0, 0, 0);
      }
    }
    if (kt > 0) stash(buf ^ 1);
    __syncthreads();
  }

  if (q_valid) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      uint2 o;
      o.x = pack_bf16x2(accQ[nb][0] * a.scale, accQ[nb][1] * a.scale);
      o.y = pack_bf16x2(accQ[nb][2] * a.scale, accQ[nb][3] * a.scale);
      *reinterpret_cast<uint2*>(a.dq + qrow * a.ld_d + h * DHB + nb * 16 + g4 * 4) = o;
    }
  }
}

template <int VAR>
__global__ void __launch_bounds__(256) attn_bwd_dkv_kernel(BwdMArgs a) {
  constexpr bool FULL = (VAR & BVAR_FULL) != 0, TBK = (VAR & BVAR_TBUCKET) != 0;
  constexpr bool CAN_FAR = !TBK;  // the bucketed variants' key terms hold the position part only
  __shared__ __attribute__((aligned(16))) bf16_t sQ[2][TB * PLD];
  __shared__ __attribute__((aligned(16))) bf16_t sO[2][TB * PLD];
  __shared__ __attribute__((aligned(16))) float sC[2][TB];
  __shared__ __attribute__((aligned(16))) float sD[2][TB];
  // variants: with the fully visible history sC holds w_i alone and sL the query's lse (with
  // the bucketed time term as well, w_i is the position term, formed in registers, and sC
  // holds the lse); sTq the query's time relative to the tile's reference (bucketed time);
  // sTB the bucket edges
  constexpr bool SPLIT_L = FULL && !TBK;
  __shared__ __attribute__((aligned(16))) float sL[SPLIT_L ? 2 : 1][SPLIT_L ? TB : 4];
  __shared__ __attribute__((aligned(16))) int32_t sTq[2][TB];
  // a query tile far from its reference point (a query's row term above BIAS_FAR_LOG2): its
  // pairs' biases are formed exactly from their position and time differences, and sC holds
  // the queries' lse alone
  __shared__ int sFar[2];
  __shared__ int32_t sTB[TBK ? ATTN_MAX_TIME_BOUNDS : 1];
  __shared__ uint32_t sLUT[TBK ? BK_CELLS : 1];  // bucket table over the gap

  const int u = blockIdx.x / a.H;
  const int h = blockIdx.x - u * a.H;
  const int64_t off = a.offsets[u];
  const int N = a.offsets[u + 1] - a.offsets[u];
  const int k0 = blockIdx.y * KT;
  if (k0 >= N) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;
  const float sp2 = a.sp2[h], st2 = a.st2[h];

  // this lane's keys: kw0 + 16 kb + l16 (kb < KB), kw0 the wave's first key; the blocks
  // share every Q and dO fragment the wave reads
  const int kw0 = k0 + wave * KW;
  const bool wave_live = kw0 < N;
  int j[KB];
  bool key_valid[KB];
  int64_t krow[KB], ts_j[KB];
  bf16x8_t kf[KB][2], vf[KB][2];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    j[kb] = kw0 + kb * 16 + l16;
    key_valid[kb] = j[kb] < N;
    krow[kb] = off + min(j[kb], N - 1);
    const int64_t rk = krow[kb] * a.ld_qkv + h * DHB;
    kf[kb][0] = as_bf16x8(*reinterpret_cast<const uint4*>(a.k + rk + g4 * 8));
    kf[kb][1] = as_bf16x8(*reinterpret_cast<const uint4*>(a.k + rk + g4 * 8 + 32));
    vf[kb][0] = as_bf16x8(*reinterpret_cast<const uint4*>(a.v + rk + g4 * 8));
    vf[kb][1] = as_bf16x8(*reinterpret_cast<const uint4*>(a.v + rk + g4 * 8 + 32));
    ts_j[kb] = a.ts[krow[kb]];
  }

  // query tiles that see these keys: history tiles from the one holding key k0 (unless only
  // candidates carry a gradient), then every candidate tile
  const int n_ht = (N + TB - 1) / TB;
  const int n_ct = (a.m + TB - 1) / TB;
  const int h_first = a.cand_only ? n_ht : (FULL ? 0 : k0 / TB);
  const int n_qt = (n_ht - h_first) + n_ct;
  struct QT { bool cand; int q0, nq; int64_t row0; };
  auto qtile = [&](int qi) {
    QT t;
    const int ht = h_first + qi;
    t.cand = ht >= n_ht;
    if (t.cand) {
      t.q0 = (ht - n_ht) * TB;
      t.nq = min(TB, a.m - t.q0);
      t.row0 = a.T_h + static_cast<int64_t>(u) * a.m + t.q0;
    } else {
      t.q0 = ht * TB;
      t.nq = min(TB, N - t.q0);
      t.row0 = off + t.q0;
    }
    return t;
  };

  // staging of a query tile: Q and dO rows pr, pr + 32 (clamped to the tile), columns
  // 8ch..8ch+7; threads 0..63 also load the time, lse and D of query tid.  What depends on
  // those loads (the row terms, the far test) is formed at the stash, a tile later, so no
  // wave waits on its loads at the fetch.
  const int pr = tid >> 3, ch = tid & 7;
  uint4 rqa, rqb, roa, rob;
  int64_t rtsq = 0, rts0 = 0;
  float rlse = 0.f, rd = 0.f;
  auto fetch = [&](const QT& t) {
    const int64_t ra = t.row0 + min(pr, t.nq - 1), rb = t.row0 + min(pr + 32, t.nq - 1);
    rqa = *reinterpret_cast<const uint4*>(a.q + ra * a.ld_qkv + h * DHB + ch * 8);
    rqb = *reinterpret_cast<const uint4*>(a.q + rb * a.ld_qkv + h * DHB + ch * 8);
    roa = *reinterpret_cast<const uint4*>(a.dout + ra * a.ld_o + h * DHB + ch * 8);
    rob = *reinterpret_cast<const uint4*>(a.dout + rb * a.ld_o + h * DHB + ch * 8);
    if (tid < TB) {
      const int ql = min(tid, t.nq - 1);
      const int64_t r = t.row0 + ql;
      if (!t.cand) {
        rtsq = a.ts[off + t.q0 + ql];
        rts0 = a.ts[off + t.q0];
      }
      rlse = a.lse[r * a.H + h];
      rd = a.delta[r * a.H + h];
    }
  };
  auto stash = [&](const QT& t, int buf) {
    stash_rows(sQ[buf], pr, ch, rqa, rqb);
    stash_rows(sO[buf], pr, ch, roa, rob);
    if (tid < TB) {
      const int ql = min(tid, t.nq - 1);
      float w_i = 0.f;
      int32_t tq = 0;
      if (!t.cand) {
        tq = static_cast<int32_t>(rtsq - rts0);
        w_i = TBK ? sp2 * static_cast<float>(ql) : sp2 * static_cast<float>(ql) + st2 * static_cast<float>(tq);
      }
      const float lse2 = rlse * LOG2E_B;
      const bool rfar = CAN_FAR && __builtin_amdgcn_ballot_w64(fabsf(w_i) > BIAS_FAR_LOG2) != 0;  // wave 0 alone
      // rows past the tile's last query: +inf row terms, so every exponent of theirs is 0
      const bool q_in = tid < t.nq;
      sC[buf][tid] = q_in ? (rfar ? lse2 : (FULL ? (TBK ? lse2 : w_i) : w_i + lse2)) : INFINITY;
      sD[buf][tid] = rd;
      if constexpr (SPLIT_L) sL[buf][tid] = q_in ? lse2 : INFINITY;
      sTq[buf][tid] = tq;
      if (tid == 0) sFar[buf] = rfar ? 1 : 0;
    }
  };
  if constexpr (TBK)
    for (int k = tid; k < a.tb_p2; k += 256) {
      const int64_t b = k < a.n_tb ? a.tb[k] : INT64_MAX;
      sTB[k] = b > INT32_MAX ? INT32_MAX : (b < INT32_MIN ? INT32_MIN : static_cast<int32_t>(b));
    }

  f32x4_t accK[KB][4], accV[KB][4];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      accK[kb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      accV[kb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  if (n_qt > 0) {
    const QT t0 = qtile(0);
    fetch(t0);
    stash(t0, 0);
  }
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) asm volatile("" : "+v"(kf[kb][0]), "+v"(kf[kb][1]), "+v"(vf[kb][0]), "+v"(vf[kb][1]));
  __syncthreads();
  if constexpr (TBK) {
    bucket_table_build(sLUT, sTB, a.tb_p2, tid, 256);
    __syncthreads();
  }

  for (int qi = 0; qi < n_qt; ++qi) {
    const int buf = qi & 1;
    const QT t = qtile(qi);
    if (qi + 1 < n_qt) fetch(qtile(qi + 1));
    // a wave whose keys no query of this tile sees (past the history, or after the tile's
    // last query) skips the products; it still stages and meets the barrier
    const bool live = wave_live && (t.cand || FULL || kw0 <= t.q0 + t.nq - 1);
    if (live) {
      // this tile's bias reference: its first query, or the candidates' (N, request time)
      const int p_ref = t.cand ? N : t.q0;
      const int64_t ts_ref = t.cand ? a.req[u] : a.ts[off + t.q0];
      // key terms; keys past the history get -inf, so every exponent of theirs is 0
      int32_t tk[KB];
      float w_j[KB], kneg[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        tk[kb] = static_cast<int32_t>(ts_j[kb] - ts_ref);
        kneg[kb] = key_valid[kb] ? 0.f : -INFINITY;
        w_j[kb] = (TBK ? sp2 * static_cast<float>(j[kb] - p_ref)
                       : sp2 * static_cast<float>(j[kb] - p_ref) + st2 * static_cast<float>(tk[kb])) + kneg[kb];
      }
      const bool far = CAN_FAR && __builtin_amdgcn_readfirstlane(sFar[buf]) != 0;
      // a history tile on the diagonal (some key after some query) needs the causal test
      const bool diag = !t.cand && !FULL && kw0 + KW - 1 > t.q0;
      // two halves of 32 queries each (query blocks 2 hq, 2 hq + 1): the k axis of the dV and
      // dK products
#pragma unroll
      for (int hq = 0; hq < 2; ++hq) {
        f32x4_t s[KB][2], dp[KB][2];  // [key block][query block of the half]
#pragma unroll
        for (int qq = 0; qq < 2; ++qq) {
          const int qb = 2 * hq + qq;
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
            s[kb][qq] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            dp[kb][qq] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          }
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const bf16x8_t qf = as_bf16x8(*reinterpret_cast<const uint4*>(&sQ[buf][(qb * 16 + l16) * PLD + ks * 32 + g4 * 8]));
            const bf16x8_t of = as_bf16x8(*reinterpret_cast<const uint4*>(&sO[buf][(qb * 16 + l16) * PLD + ks * 32 + g4 * 8]));
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
              s[kb][qq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf, kf[kb][ks], s[kb][qq], 0, 0, 0);
              dp[kb][qq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(of, vf[kb][ks], dp[kb][qq], 0, 0, 0);
            }
          }
        }
        // P and dS for queries qb*16 + 4*g4 + i of the tile and this lane's keys.  F: the
        // exact bias of each pair (rare).  MASK 0: no causal test, 1: the causal test, 2: the
        // causal test on diagonal tiles, decided at run time (one instance for both).
        auto pds = [&](auto FARC, auto MASKC) {
          constexpr bool F = decltype(FARC)::value;
          constexpr int MASK = decltype(MASKC)::value;
#pragma unroll
          for (int qq = 0; qq < 2; ++qq) {
            const int qb = 2 * hq + qq;
            const float4 c4 = reinterpret_cast<const float4*>(sC[buf])[qb * 4 + g4];
            const float4 d4 = reinterpret_cast<const float4*>(sD[buf])[qb * 4 + g4];
            const float cv[4] = {c4.x, c4.y, c4.z, c4.w};
            const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
            float lv[4] = {0.f, 0.f, 0.f, 0.f};
            if constexpr (SPLIT_L) {
              const float4 l4 = reinterpret_cast<const float4*>(sL[buf])[qb * 4 + g4];
              lv[0] = l4.x; lv[1] = l4.y; lv[2] = l4.z; lv[3] = l4.w;
            }
            int32_t tv[4] = {0, 0, 0, 0};
            if constexpr (F || TBK) {
              const int4 t4 = reinterpret_cast<const int4*>(sTq[buf])[qb * 4 + g4];
              tv[0] = t4.x; tv[1] = t4.y; tv[2] = t4.z; tv[3] = t4.w;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int ql = qb * 16 + g4 * 4 + i;
              const int slot = t.cand ? N + t.q0 + ql : t.q0 + ql;
#pragma unroll
              for (int kb = 0; kb < KB; ++kb) {
                const float sv = s[kb][qq][i];
                float arg;
                if constexpr (F) {  // log2 units; sC holds the lse
                  const float b = sp2 * static_cast<float>(j[kb] - slot) + st2 * static_cast<float>(tk[kb] - tv[i]);
                  arg = sv * a.scale2 + (FULL ? -fabsf(b) : b) - cv[i] + kneg[kb];
                } else if constexpr (!FULL && !TBK) {
                  arg = __builtin_fmaf(sv, a.scale2, w_j[kb] - cv[i]);
                } else {
                  // fully visible: -|w_j - w_i|; bucketed time: - s' bucket(|t_i - t_j|)
                  if constexpr (SPLIT_L) {
                    arg = sv * a.scale2 - fabsf(w_j[kb] - cv[i]) - lv[i];
                  } else if constexpr (FULL) {  // and TBK: w_i = s (p_i - p_ref) = s ql on history tiles
                    const float w_i = t.cand ? 0.f : sp2 * static_cast<float>(ql);
                    arg = sv * a.scale2 - fabsf(w_j[kb] - w_i) - cv[i];
                  } else {
                    arg = sv * a.scale2 + w_j[kb] - cv[i];
                  }
                  if constexpr (TBK) arg -= st2 * static_cast<float>(bucket_lookup(sLUT, sTB, a.tb_p2, abs(tv[i] - tk[kb])));
                }
                float p = __builtin_amdgcn_exp2f(arg);
                if constexpr (MASK == 1) {
                  if (j[kb] > slot) p = 0.f;
                } else if constexpr (MASK == 2) {
                  if (diag && j[kb] > slot) p = 0.f;
                }
                s[kb][qq][i] = p;
                dp[kb][qq][i] = p * (dp[kb][qq][i] - dv[i]);
              }
            }
          }
        };
        using FT = std::integral_constant<bool, true>;
        using FF = std::integral_constant<bool, false>;
        if constexpr (CAN_FAR) {
          if (far) pds(FT{}, std::integral_constant<int, 2>{});
          else if (diag) pds(FF{}, std::integral_constant<int, 1>{});
          else pds(FF{}, std::integral_constant<int, 0>{});
        } else {  // the bucketed variants: one instance
          pds(FF{}, std::integral_constant<int, 2>{});
        }
        // dV^T += dO^T P,  dK^T += Q^T dS over this half's 32 queries
        bf16x8_t pf[KB], dsf[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          pf[kb] = pack_blocks(s[kb][0], s[kb][1]);
          dsf[kb] = pack_blocks(dp[kb][0], dp[kb][1]);
        }
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const bf16x8_t otf = tr_operand(sO[buf], nb, hq, l16, g4);
          const bf16x8_t qtf = tr_operand(sQ[buf], nb, hq, l16, g4);
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
            accV[kb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(otf, pf[kb], accV[kb][nb], 0, 0, 0);
            accK[kb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qtf, dsf[kb], accK[kb][nb], 0, 0, 0);
          }
        }
      }
    }
    if (qi + 1 < n_qt) stash(qtile(qi + 1), buf ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    if (!key_valid[kb]) continue;
    const int64_t dro = krow[kb] * a.ld_d + h * DHB;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      uint2 o;
      o.x = pack_bf16x2(accK[kb][nb][0] * a.scale, accK[kb][nb][1] * a.scale);
      o.y = pack_bf16x2(accK[kb][nb][2] * a.scale, accK[kb][nb][3] * a.scale);
      *reinterpret_cast<uint2*>(a.dk + dro + nb * 16 + g4 * 4) = o;
      o.x = pack_bf16x2(accV[kb][nb][0], accV[kb][nb][1]);
      o.y = pack_bf16x2(accV[kb][nb][2], accV[kb][nb][3]);
      *reinterpret_cast<uint2*>(a.dv + dro + nb * 16 + g4 * 4) = o;
    }
  }
}

}  // namespace

// ---- the allocation-free entry point's scratch: the per-row D of the backward, in a
// file-scope device array (one copy per GPU, held until the process ends).  In host code
// `scratch` names a host-side stand-in, not device memory: every use goes through the
// per-device address hipGetSymbolAddress returns.
constexpr size_t ATTN_BWD_SCRATCH_BYTES = size_t(16) << 20;
static __device__ __align__(256) float scratch[ATTN_BWD_SCRATCH_BYTES / sizeof(float)];

namespace {
constexpr int SCRATCH_MAX_DEVICES = 64;
std::once_flag scratch_once[SCRATCH_MAX_DEVICES];
void* scratch_ptr[SCRATCH_MAX_DEVICES];
hipError_t scratch_err[SCRATCH_MAX_DEVICES];
}  // namespace

size_t attn_bwd_scratch_bytes() { return ATTN_BWD_SCRATCH_BYTES; }

// The current device's copy of the scratch array, looked up once per device.
genrank_status attn_bwd_scratch(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= SCRATCH_MAX_DEVICES) return GENRANK_E_HIP;
  std::call_once(scratch_once[dev], [dev] {
    scratch_err[dev] = hipGetSymbolAddress(&scratch_ptr[dev], HIP_SYMBOL(scratch));
  });
  if (scratch_err[dev] != hipSuccess || !scratch_ptr[dev]) return GENRANK_E_HIP;
  *ptr = scratch_ptr[dev];
  return GENRANK_OK;
}

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
  a.flags = alibi.flags;
  a.tb = alibi.time_bounds;
  a.n_tb = alibi.n_time_bounds;
  dim3 grid(static_cast<unsigned>(T), b->H);
  if (b->dtype == GENRANK_BF16) {  // dh == 64 and the alignments are checked by the caller
    BwdMArgs m{};
    m.offsets = offsets; m.ts = ts; m.req = req;
    m.q = static_cast<const bf16_t*>(q); m.k = static_cast<const bf16_t*>(k); m.v = static_cast<const bf16_t*>(v);
    m.ld_qkv = ld_qkv;
    m.o = static_cast<const bf16_t*>(o); m.dout = static_cast<const bf16_t*>(dout); m.ld_o = ld_o;
    m.lse = lse; m.delta = a.delta;
    m.dq = static_cast<bf16_t*>(dq); m.dk = static_cast<bf16_t*>(dk); m.dv = static_cast<bf16_t*>(dv);
    m.ld_d = ld_dqkv;
    for (int h = 0; h < b->H; ++h) {
      m.sp2[h] = alibi.slopes_pos[h] * LOG2E_B;
      m.st2[h] = alibi.slopes_time[h] * LOG2E_B;
    }
    m.scale = 1.f / sqrtf(static_cast<float>(b->dh));
    m.scale2 = m.scale * LOG2E_B;
    m.B = b->B; m.m = b->m; m.H = b->H; m.cand_only = cand_only;
    m.hist_tiles = (b->max_hist + TB - 1) / TB;
    m.cand_tiles = (b->m + TB - 1) / TB;
    m.T_h = b->total_hist;
    if (alibi.flags & GENRANK_ATTN_TIME_BUCKET) {
      m.tb = alibi.time_bounds;
      m.n_tb = alibi.n_time_bounds;
      m.tb_p2 = bucket_p2(m.n_tb);
    }
    const int key_tiles = (b->max_hist + KT - 1) / KT;
    const dim3 gq(b->B * b->H, m.cand_tiles + m.hist_tiles), gk(b->B * b->H, key_tiles);
    const int var = ((alibi.flags & GENRANK_ATTN_FULL_HISTORY) ? BVAR_FULL : 0) |
                    ((alibi.flags & GENRANK_ATTN_TIME_BUCKET) ? BVAR_TBUCKET : 0);
    auto launch = [&](auto dq_kernel, auto dkv_kernel) {
      if (m.hist_tiles + m.cand_tiles > 0) hipLaunchKernelGGL(dq_kernel, gq, dim3(256), 0, stream, m);
      if (key_tiles > 0) hipLaunchKernelGGL(dkv_kernel, gk, dim3(256), 0, stream, m);
    };
    switch (var) {
      case 0: launch(attn_bwd_dq_kernel<0>, attn_bwd_dkv_kernel<0>); break;
      case BVAR_FULL: launch(attn_bwd_dq_kernel<BVAR_FULL>, attn_bwd_dkv_kernel<BVAR_FULL>); break;
      case BVAR_TBUCKET: launch(attn_bwd_dq_kernel<BVAR_TBUCKET>, attn_bwd_dkv_kernel<BVAR_TBUCKET>); break;
      default:
        launch(attn_bwd_dq_kernel<BVAR_FULL | BVAR_TBUCKET>, attn_bwd_dkv_kernel<BVAR_FULL | BVAR_TBUCKET>);
        break;
    }
  } else {
    hipLaunchKernelGGL(delta_kernel<float>, grid, dim3(64), 0, stream, a);
    hipLaunchKernelGGL(dq_kernel<float>, grid, dim3(64), 0, stream, a);
    hipLaunchKernelGGL(dkv_kernel<float>, grid, dim3(64), 0, stream, a);
  }
  GR_CHECK_LAUNCH();
  return GENRANK_OK;
}

}  // namespace genrank
