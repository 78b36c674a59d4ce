// Masked ALiBi flash attention forward for GenRank on gfx950.
//
// Per user u and head h ("一、 GenRank [2025]" section 1.4.2, ALiBi score;
// "The Overall Generative Ranking Paradigm" sections 7.2.1-7.2.2, masks and the
// position + time bias):
//   score_ij = q_i.k_j / sqrt(dh) - sp_h |p_i - p_j| - st_h |tau_i - tau_j|
// over allowed pairs (history i sees history j <= i; candidate i sees all history and
// itself).  On allowed pairs p_i >= p_j and tau_i >= tau_j (timestamps are sorted and the
// request comes after the history), so the bias is w_j - w_i with
// w = sp*(p - p_ref) + st*(tau - tau_ref); the row term w_i cancels in the softmax and is
// only added back into the saved log-sum-exp.  The bias therefore costs one FMA per score
// and no T x T array exists anywhere.
//
// bf16 kernels (dh = 64), all with S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (each lane
// holds 16 scores of ONE query, so row max / row sum need only two cross-lane steps) and
// O^T = V^T P^T with P^T taken straight from the score registers; a candidate never
// forms the m x m candidate block (its own key is handled on its own):
//   attn_fwd_pair_kernel   one workgroup per (user, head), the user's K/V resident in LDS
//                          (histories up to PAIR_MAXK keys: the full forward);
//   attn_fwd_ring_kernel   one workgroup per 128-query tile, K/V streamed through an LDS
//                          ring (longer histories; candidates-only scoring);
//   attn_fwd_rab_kernel    the tile grid with a learned bias read from memory instead of
//                          ALiBi (the HSTU-style comparison).
// f32 kernel: one wave per (row, head), the literal definition (reference-precision path).
#include <math.h>

#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

namespace genrank {

namespace {

constexpr int GROUP = 32;       // (user, head) pairs per XCD scheduling group
constexpr int QW = 16;          // queries per wave (16-column MFMA blocks)
constexpr int QB = QW / 16;     // column blocks per wave
constexpr int NW = 8;           // waves per workgroup
constexpr int NT = 64 * NW;     // threads per workgroup
constexpr int AQ = NW * QW;     // queries per workgroup
constexpr int AK = 64;          // keys per tile
constexpr int DH = 64;          // head dim of the bf16 kernels
constexpr int KLD = DH + 8;     // sK row pitch (bf16)
constexpr int VLD = AK + 8;     // sVt row pitch (bf16)
constexpr int WCHUNK = 512;     // keys whose bias terms sit in LDS at a time
constexpr int BUF_DWORD3 = 0x00020000;  // raw buffer descriptor word 3 (gfx9 family)
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

struct AttnArgs {
  const int32_t* offsets;
  const int64_t* ts;
  const int64_t* req;
  const bf16_t* q;
  const bf16_t* k;
  const bf16_t* v;
  int64_t ld_qkv;
  bf16_t* o;
  int64_t ld_o;
  float* lse;
  float sp2[GENRANK_MAX_HEADS];  // slopes * log2(e)
  float st2[GENRANK_MAX_HEADS];
  float scale2;                  // log2(e) / sqrt(dh)
  float rscale2;                 // 1 / scale2
  int B, m, H, hist_tiles, cand_tiles;
  int64_t T_h;
  const bf16_t* rab;       // learned-bias variant: per-user [L, P] bf16 matrices
  const int64_t* rab_off;  // element offset of user u's matrix, [B + 1]
  // history keys and values: rows [off_u, off_u + N_u) of kh / vh (row stride ld_h); the
  // q / k / v rows above in the batch layout, or a cache of earlier requests' history
  const bf16_t* kh;
  const bf16_t* vh;
  int64_t ld_h;
  int64_t crow0;           // row of candidate (u, 0) in q / k / v / o / lse: T_h, or 0
  // bucketed time term: edges (int64, device), their count, and the power of two >= count + 1
  const int64_t* tb;
  int n_tb, tb_p2;
  int nt_o;  // o far larger than the last-level cache: streaming stores (pair kernel)
  uint32_t* err;  // the device error word (GENRANK_ERR_*)
  int order;      // pair kernel: take the users heaviest first (0: every history has one length)
};

// variant bits of the ALiBi kernels: the fully visible history mask, the bucketed time term
constexpr int VAR_FULL = 1, VAR_TBUCKET = 2;

// slot of key j (0..63 in a tile) in the permuted key axis of sVt
__device__ __forceinline__ int vt_slot(int j) {
  const int ks = j >> 5, r = j & 31;
  const int hi = r >> 4, rr = r & 15;
  return ks * 32 + (rr >> 2) * 8 + hi * 4 + (rr & 3);
}

// max / sum with lane l ^ 16 and lane l ^ 32 via the gfx950 lane-swap instructions
__device__ __forceinline__ float xor16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// the largest of a lane's 16 scores (as a chain of three-way maxima)
__device__ __forceinline__ float max16(const f32x4_t (&sc)[4]) {
  float m = fmaxf(fmaxf(sc[0][0], sc[0][1]), sc[0][2]);
  m = fmaxf(fmaxf(m, sc[0][3]), sc[1][0]);
  m = fmaxf(fmaxf(m, sc[1][1]), sc[1][2]);
  m = fmaxf(fmaxf(m, sc[1][3]), sc[2][0]);
  m = fmaxf(fmaxf(m, sc[2][1]), sc[2][2]);
  m = fmaxf(fmaxf(m, sc[2][3]), sc[3][0]);
  m = fmaxf(fmaxf(m, sc[3][1]), sc[3][2]);
  return fmaxf(m, sc[3][3]);
}
__device__ __forceinline__ float xor16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The HSTU-style comparison kernel: each user's history is the interleaved item/action
// sequence (2 N slots, rows 2 off .. 2 off + 2N of q / k / v) and the bias is a learned
// matrix read from memory (user u's [L, P] bf16 block, L = 2N + m, row pitch P = L rounded
// up to 8).  One workgroup = 8 waves x 16 query rows of one (user, head): a 128-row history
// tile (keys up to and including the diagonal) or a 128-row candidate tile (every history
// key, plus each candidate's own key, which seeds the online softmax).
//   S^T = K Q^T with v_mfma_f32_16x16x32_bf16: K rows from LDS are the row operand, the
//         wave's 16 queries (registers) the column operand, so each lane holds 16 scores
//         of ONE query.
//   O^T = V^T P^T: P^T goes from the score registers straight into the column operand; V
//         is stored transposed in LDS with its keys permuted to match that register order.
// K/V tiles are double-buffered in LDS and the next tile is fetched into registers while
// the current one is multiplied; the lane's 16 bias values of a tile are loaded one tile
// ahead.  The pairs' tiles run next to each other on one XCD (the flat-grid order of the
// ring kernel).
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(4, 8))) attn_fwd_rab_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) bf16_t sK[2][AK * KLD];
  __shared__ __attribute__((aligned(16))) bf16_t sVt[2][DH * VLD];

  const int TY = a.cand_tiles + a.hist_tiles;
  const int x8 = blockIdx.x & 7;
  const int kx = blockIdx.x >> 3;
  const int grp = kx / (TY * GROUP);
  const int rem = kx - grp * (TY * GROUP);
  const int y = rem / GROUP;
  const int bh = (grp * GROUP + (rem - y * GROUP)) * 8 + x8;
  if (bh >= a.B * a.H) return;
  const int u = bh / a.H;
  const int h = bh - u * a.H;
  const int64_t off = 2 * static_cast<int64_t>(a.offsets[u]);
  const int N = 2 * (a.offsets[u + 1] - a.offsets[u]);  // interleaved history slots

  bool is_cand;
  int q0, nq, n_tiles;
  int64_t qrow0;
  if (y < a.cand_tiles) {
    is_cand = true;
    q0 = y * AQ;
    if (q0 >= a.m) return;
    nq = min(AQ, a.m - q0);
    qrow0 = a.crow0 + static_cast<int64_t>(u) * a.m + q0;
    n_tiles = (N + AK - 1) / AK;
  } else {
    is_cand = false;
    const int t = a.hist_tiles - 1 - (y - a.cand_tiles);  // largest tiles first
    q0 = t * AQ;
    if (q0 >= N) return;
    nq = min(AQ, N - q0);
    qrow0 = off + q0;
    n_tiles = (q0 + nq + AK - 1) / AK;
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;
  const int kt_first = n_tiles - 1;

  // this lane's query
  const int q_local = wave * QW + l16;
  const bool q_valid = q_local < nq;
  const int64_t qrow = qrow0 + q_local;
  const int q_slot = is_cand ? (N + q0 + q_local) : (q0 + q_local);
  // keys with a slot above k_lim are masked (a candidate's own key is the seed below)
  const int k_lim = is_cand ? (N - 1) : min(q_slot, N - 1);
  const int kmax_blk = is_cand ? (N - 1) : min(q0 + wave * QW + 15, N - 1);
  const int64_t rowoff = (qrow0 + min(q_local, nq - 1)) * a.ld_qkv + h * DH;
  bf16x8_t qf[2];
  qf[0] = as_bf16x8(*reinterpret_cast<const uint4*>(a.q + rowoff + g4 * 8));
  qf[1] = as_bf16x8(*reinterpret_cast<const uint4*>(a.q + rowoff + g4 * 8 + 32));
  uint4 kself[2] = {};
  uint2 vself[4] = {};
  if (is_cand) {
    kself[0] = *reinterpret_cast<const uint4*>(a.k + rowoff + g4 * 8);
    kself[1] = *reinterpret_cast<const uint4*>(a.k + rowoff + g4 * 8 + 32);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) vself[nb] = *reinterpret_cast<const uint2*>(a.v + rowoff + nb * 16 + g4 * 4);
  }

  // ---- K/V tile staging: waves 0-3 move K, waves 4-7 move V, two 16-byte loads per lane
  // per tile.  K: rows krow and krow+32, columns kcol..kcol+7 (conflict-free 16-byte LDS
  // writes).  V: the key pair 2pr, 2pr+1, columns 8ch..8ch+7, into sVt transposed; each
  // 32-bit write holds the two keys' values of one column.  Buffer loads over the user's
  // history rows; rows past the history end read as zero (the mask gives those keys
  // probability 0), and a tile index below 0 gets an offset at the record count (zeros, no
  // memory access; such a stage is never written to LDS).  Every fetch is issued, so the
  // wait before a stash covers only that stage's own two loads.
  const bool stage_k = wave < NW / 2;
  const int st = tid & (NT / 2 - 1);
  const int pr = st & 31;
  const int ch = st >> 5;
  const int kA = 2 * pr;
  const int krow = st >> 3;
  const int kcol = (st & 7) * 8;
  const uint32_t row_bytes = static_cast<uint32_t>(a.ld_h) * 2u;
  const uint32_t hist_bytes = static_cast<uint32_t>(N) * row_bytes;
  const __amdgpu_buffer_rsrc_t rsKV = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t*>((stage_k ? a.kh : a.vh) + off * a.ld_h), static_cast<short>(0), hist_bytes,
      BUF_DWORD3);
  const uint32_t vo0 = stage_k ? static_cast<uint32_t>(krow) * row_bytes + (h * DH + kcol) * 2u
                               : static_cast<uint32_t>(kA) * row_bytes + (h * DH + ch * 8) * 2u;
  const uint32_t vo1 = vo0 + (stage_k ? 32u : 1u) * row_bytes;
  struct Stage { uint4 r0, r1; };
  Stage S0, S1;
  auto fetch = [&](int kt, Stage& S) {
    const uint32_t so = kt >= 0 ? static_cast<uint32_t>(kt * AK) * row_bytes : hist_bytes;
    S.r0 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsKV, vo0 + so, 0, 0));
    S.r1 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsKV, vo1 + so, 0, 0));
  };
  const int slotA = vt_slot(kA);  // the pair's second key sits at slotA + 1
  auto stash = [&](int buf, const Stage& S) {
    if (stage_k) {
      *reinterpret_cast<uint4*>(&sK[buf][krow * KLD + kcol]) = S.r0;
      *reinterpret_cast<uint4*>(&sK[buf][(krow + 32) * KLD + kcol]) = S.r1;
    } else {
      uint32_t* col = reinterpret_cast<uint32_t*>(&sVt[buf][ch * 8 * VLD + slotA]);
      constexpr int P = VLD / 2;  // row pitch in 32-bit words
      col[0 * P] = __builtin_amdgcn_perm(S.r1.x, S.r0.x, 0x05040100u);
      col[1 * P] = __builtin_amdgcn_perm(S.r1.x, S.r0.x, 0x07060302u);
      col[2 * P] = __builtin_amdgcn_perm(S.r1.y, S.r0.y, 0x05040100u);
      col[3 * P] = __builtin_amdgcn_perm(S.r1.y, S.r0.y, 0x07060302u);
      col[4 * P] = __builtin_amdgcn_perm(S.r1.z, S.r0.z, 0x05040100u);
      col[5 * P] = __builtin_amdgcn_perm(S.r1.z, S.r0.z, 0x07060302u);
      col[6 * P] = __builtin_amdgcn_perm(S.r1.w, S.r0.w, 0x05040100u);
      col[7 * P] = __builtin_amdgcn_perm(S.r1.w, S.r0.w, 0x07060302u);
    }
  };
  fetch(kt_first, S0);
  fetch(kt_first - 1, S1);

  // ---- the learned bias: the lane's 16 bias values of a key tile are four 8-byte pieces
  // of its query's row, loaded one tile ahead.  A buffer descriptor over the user's matrix:
  // rows past it and tile indices below 0 read zeros without a memory access.
  struct RabRegs { uint2 v[4]; };
  RabRegs R0, R1;
  const uint32_t rab_P = static_cast<uint32_t>((N + a.m + 7) & ~7);
  const uint32_t rab_bytes = static_cast<uint32_t>(N + a.m) * rab_P * 2u;
  const uint32_t rab_row = static_cast<uint32_t>(q_slot) * rab_P * 2u + g4 * 8u;
  const __amdgpu_buffer_rsrc_t rsR = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t*>(a.rab + a.rab_off[u]), static_cast<short>(0), rab_bytes, BUF_DWORD3);
  const uint16_t rab_self_b = __builtin_amdgcn_raw_buffer_load_b16(
      rsR, static_cast<uint32_t>(q_slot) * (rab_P + 1u) * 2u, 0, 0);  // the bias of (i, i)
  auto rab_load = [&](int kt, RabRegs& R) {
    const uint32_t so = kt >= 0 ? static_cast<uint32_t>(kt * AK) * 2u : rab_bytes;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      R.v[kb] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rsR, rab_row + kb * 32u + so, 0, 0));
  };
  rab_load(kt_first, R0);

  // ---- softmax state (log2 units); a candidate starts from its own key
  f32x4_t accO[4];
  float m2, lsum;
  if (is_cand) {
    float dot = 0.f, kf[8], qv[8];
#pragma unroll
    for (int hlf = 0; hlf < 2; ++hlf) {
      unpack8(kself[hlf], kf);
      unpack8(__builtin_bit_cast(uint4, qf[hlf]), qv);
#pragma unroll
      for (int e = 0; e < 8; ++e) dot += qv[e] * kf[e];
    }
    dot = xor32_sum(xor16_sum(dot));
    m2 = dot * a.scale2 + __uint_as_float(static_cast<uint32_t>(rab_self_b) << 16) * LOG2E;
    lsum = (g4 == 0) ? 1.f : 0.f;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const uint2 vv = vself[nb];
      accO[nb] = f32x4_t{__uint_as_float(vv.x << 16), __uint_as_float(vv.x & 0xFFFF0000u),
                         __uint_as_float(vv.y << 16), __uint_as_float(vv.y & 0xFFFF0000u)};
    }
  } else {
    m2 = -1e30f;
    lsum = 0.f;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) accO[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  stash(0, S0);
  // The query fragments come straight from a global load.  Without this the compiler's
  // wait-count analysis cannot prove at the loop head that the load has landed and makes
  // every iteration wait for that iteration's K/V prefetch before its first MFMA.  An empty
  // asm that reads and redefines the registers makes it wait here, once.
  asm volatile("" : "+v"(qf[0]), "+v"(qf[1]));
  __syncthreads();

  // One key tile, newest first.  Tiles that reach past some query's limit (the causal
  // diagonal, the ragged end of the history) take the masked instantiation.  Waves whose
  // 16 queries all lie past the tile's end only stage and synchronise, in their own copy
  // of the loop (same barriers in the same order).
  const bool wave_on = wave * QW < nq;
  auto tile = [&](auto active_tag, auto masked_tag, int it, Stage& ld, const Stage& nxt, const RabRegs& rc,
                  RabRegs& rn) {
    constexpr bool ACTIVE = decltype(active_tag)::value;
    constexpr bool MASKED = decltype(masked_tag)::value;
    const int kt = kt_first - it;
    const int buf = it & 1;
    const int base = kt * AK;
    fetch(kt - 2, ld);
    rab_load(kt - 1, rn);
    if constexpr (ACTIVE) {
      f32x4_t s[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        s[kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (!MASKED || base + kb * 16 <= kmax_blk) {
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const bf16x8_t kf = as_bf16x8(*reinterpret_cast<const uint4*>(
                &sK[buf][(kb * 16 + l16) * KLD + ks * 32 + g4 * 8]));
            s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[ks], s[kb], 0, 0, 0);
          }
        }
      }
      // scale + the learned bias (natural-log units -> log2 units), mask, row max
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const uint2 r = rc.v[kb];
        s[kb][0] = s[kb][0] * a.scale2 + __uint_as_float(r.x << 16) * LOG2E;
        s[kb][1] = s[kb][1] * a.scale2 + __uint_as_float(r.x & 0xFFFF0000u) * LOG2E;
        s[kb][2] = s[kb][2] * a.scale2 + __uint_as_float(r.y << 16) * LOG2E;
        s[kb][3] = s[kb][3] * a.scale2 + __uint_as_float(r.y & 0xFFFF0000u) * LOG2E;
      }
      if constexpr (MASKED) {
        const int lim = k_lim - base - g4 * 4;  // local key kb*16 + i must be <= lim
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (kb * 16 + i > lim) s[kb][i] = -INFINITY;
      }
      float m = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), s[0][2]), fmaxf(fmaxf(s[0][3], s[1][0]), s[1][1]));
      m = fmaxf(fmaxf(m, s[1][2]), fmaxf(fmaxf(s[1][3], s[2][0]), s[2][1]));
      m = fmaxf(fmaxf(m, s[2][2]), fmaxf(fmaxf(s[2][3], s[3][0]), s[3][1]));
      m = fmaxf(fmaxf(m, s[3][2]), s[3][3]);
      const float mx = xor32_max(xor16_max(m));
      // online softmax: raise the running maximum and rescale O and l by 2^(m_old - m_new)
      const float m_new = fmaxf(m2, mx);
      const float alpha = __builtin_amdgcn_exp2f(m2 - m_new);
      m2 = m_new;
      lsum *= alpha;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) accO[nb] = accO[nb] * alpha;
      float psum = 0.f;
      bf16x8_t pf[2];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = __builtin_amdgcn_exp2f(s[kb][i] - m2);
          s[kb][i] = p;
          psum += p;
        }
      lsum += psum;
      // P^T as the column operand: keys {4g..4g+3} of blocks 2ks and 2ks+1
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        uint4 pk;
        pk.x = pack_bf16x2(s[2 * ks][0], s[2 * ks][1]);
        pk.y = pack_bf16x2(s[2 * ks][2], s[2 * ks][3]);
        pk.z = pack_bf16x2(s[2 * ks + 1][0], s[2 * ks + 1][1]);
        pk.w = pack_bf16x2(s[2 * ks + 1][2], s[2 * ks + 1][3]);
        pf[ks] = as_bf16x8(pk);
      }
      // O^T += V^T P^T
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        if (MASKED && base + ks * 32 > kmax_blk) continue;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const bf16x8_t vf = as_bf16x8(*reinterpret_cast<const uint4*>(
              &sVt[buf][(nb * 16 + l16) * VLD + ks * 32 + g4 * 8]));
          accO[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[ks], accO[nb], 0, 0, 0);
        }
      }
    }  // ACTIVE
    if (kt > 0) stash(buf ^ 1, nxt);
    __syncthreads();
  };

  // a tile needs the mask when its last key lies past some query's limit
  const int klim_min = is_cand ? (N - 1) : q0;
  auto loop = [&](auto active_tag) {
    auto step = [&](int it, Stage& ld, const Stage& nxt, const RabRegs& rc, RabRegs& rn) {
      if ((kt_first - it) * AK + AK - 1 > klim_min)
        tile(active_tag, std::true_type{}, it, ld, nxt, rc, rn);
      else
        tile(active_tag, std::false_type{}, it, ld, nxt, rc, rn);
    };
    // unrolled by two so that the two staging register sets keep fixed names
    for (int it = 0; it < n_tiles; it += 2) {
      step(it, S0, S1, R0, R1);
      if (it + 1 < n_tiles) step(it + 1, S1, S0, R1, R0);
    }
  };
  if (wave_on)
    loop(std::true_type{});
  else
    loop(std::false_type{});

  // ---- epilogue
  const float ltot = xor32_sum(xor16_sum(lsum));
  if (!q_valid) return;
  const float inv = 1.f / ltot;
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    uint2 o;
    o.x = pack_bf16x2(accO[nb][0] * inv, accO[nb][1] * inv);
    o.y = pack_bf16x2(accO[nb][2] * inv, accO[nb][3] * inv);
    *reinterpret_cast<uint2*>(a.o + qrow * a.ld_o + h * DH + nb * 16 + g4 * 4) = o;
  }
  if (a.lse && g4 == 0) a.lse[qrow * a.H + h] = LN2 * (m2 + log2f(ltot));
}

// ------------------------------------------------------------------ bf16 ring kernel
// ALiBi (and its variants) over the tile grid of attn_fwd_rab_kernel above: one workgroup
// = 8 waves x 16 query rows of one (user, head), a history tile (keys up to the diagonal)
// or a candidate tile (every history key, then the candidate's own key); same XCD order.
// What differs from that kernel is how K and V reach LDS and how much vector work a tile
// costs:
//  - K and V tiles go from global memory straight into LDS (one 16-byte direct load per
//    lane and tile for each), through a ring of NS stage buffers with NS - 1 tiles in
//    flight.  No registers hold staged data and each workgroup waits for memory about
//    once, not once per tile.  Both tiles are stored row-major with an XOR swizzle of
//    their 16-byte chunks (chosen through which chunk each lane fetches).
//  - The O^T = V^T P^T row operand comes from the row-major V tile through the gfx950
//    transposing LDS read (ds_read_b64_tr_b16): within each 16-lane group, output lane j
//    element e is element j % 4 of what lane 4 e + j / 4 addressed.  Two such reads give
//    one lane 8 keys of one head dimension.
//  - With the plain separable bias the key term w_j seeds the score accumulator, so the
//    MFMA leaves q.k + w_j / c (c = log2(e) / sqrt(dh)) and the softmax scales once, inside
//    the exponent's FMA.
//  - The running maximum is raised only when some score exceeds it by more than 2^8 (a
//    wave-uniform branch); until then probabilities up to 2^8 are accumulated against the
//    stale maximum, which changes nothing in exact arithmetic and stays far inside fp32
//    and bf16 range.
//  - Row sums come from the bf16 probabilities the P V product uses, on the matrix cores:
//    one more product per 32-key half, ones^T P^T, leaves every lane its query's whole sum
//    (no vector instruction per probability, no cross-lane sum at the end).
constexpr int NS = 4;               // stage buffers in the K/V ring
constexpr int STAGE = 2 * AK * DH;  // bf16 per stage buffer: the K tile, then the V tile
constexpr float RESCALE_LOG2 = 8.f; // headroom of the stale running maximum (log2 units)
static_assert(QB == 1 && NW * 8 == AK, "one 16-query block per wave; 8 tile rows per wave");

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// The ring and pair kernels give candidate rows the same bits (cached scoring runs the ring
// kernel, the full forward the pair kernel), so the steps whose rounding could differ are
// written once, here, with explicit FMAs.
// Bias term of a key in score units: position part, plus the time part unless bucketed.
__device__ __forceinline__ float key_term(bool tbk, float spr, float str, int dp, int32_t dt) {
  return tbk ? spr * static_cast<float>(dp) : __builtin_fmaf(spr, static_cast<float>(dp), str * static_cast<float>(dt));
}
// Scaled score plus bias (the non-separable variants, log2 units).
__device__ __forceinline__ float biased(float s, float scale2, float bias) { return __builtin_fmaf(s, scale2, bias); }
// Merge a candidate's own key (score m_self in score units, value row vself) into its
// softmax state after the history keys.
__device__ __forceinline__ void merge_self(const u32x4_t (&kself)[2], const u32x2_t (&vself)[4], const bf16x8_t (&qf)[2],
                                           bool sep, float scale2, float self_bias, float SC, float th, int g4,
                                           float& m_run, float& lsum, f32x4_t (&accO)[4]) {
  // q . k over this lane's 16 dimensions, two products per step (exact bf16 products)
  float dot = 0.f;
#pragma unroll
  for (int hlf = 0; hlf < 2; ++hlf) {
    const uint4 kw = __builtin_bit_cast(uint4, kself[hlf]);
    const uint4 qw = __builtin_bit_cast(uint4, qf[hlf]);
    const uint32_t kk[4] = {kw.x, kw.y, kw.z, kw.w}, qq[4] = {qw.x, qw.y, qw.z, qw.w};
#pragma unroll
    for (int e = 0; e < 4; ++e)
      dot = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qq[e]), __builtin_bit_cast(bf16x2_t, kk[e]), dot,
                                            false);
  }
  dot = xor32_sum(xor16_sum(dot));
  const float m_self = sep ? dot : __builtin_fmaf(dot, scale2, -self_bias);
  // as for the key tiles, the running maximum moves only when the own-key score exceeds
  // it by more than th; decided per query (lane), so that a candidate's result does not
  // depend on the other candidates of its block (the branch is skipped when no lane needs
  // it)
  if (m_self > m_run + th) {
    const float alpha = __builtin_amdgcn_exp2f((m_run - m_self) * SC);
    m_run = m_self;
    lsum *= alpha;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) accO[nb] = accO[nb] * alpha;
  }
  const float p_self = __builtin_amdgcn_exp2f((m_self - m_run) * SC);
  lsum += p_self;  // (every lane holds its query's whole row sum)
  uint32_t hi = 0xFFFF0000u;  // kept in a scalar register
  asm volatile("" : "+s"(hi));
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const u32x2_t vv = vself[nb];
    const float v4[4] = {__uint_as_float(vv.x << 16), __uint_as_float(vv.x & hi), __uint_as_float(vv.y << 16),
                         __uint_as_float(vv.y & hi)};
#pragma unroll
    for (int i = 0; i < 4; ++i) accO[nb][i] = __builtin_fmaf(p_self, v4[i], accO[nb][i]);
  }
}

template <int VAR>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(4, 8))) attn_fwd_ring_kernel(AttnArgs a) {
  constexpr bool FULL = (VAR & VAR_FULL) != 0;
  constexpr bool TBK = (VAR & VAR_TBUCKET) != 0;
  constexpr bool SEP = VAR == 0;  // bias term of the key only: it seeds the accumulator
  constexpr bool CAN_FAR = !TBK;  // the bucketed variants' key terms hold the position part only
  __shared__ __attribute__((aligned(16))) bf16_t sg0[STAGE];
  __shared__ __attribute__((aligned(16))) bf16_t sg1[STAGE];
  __shared__ __attribute__((aligned(16))) bf16_t sg2[STAGE];
  __shared__ __attribute__((aligned(16))) bf16_t sg3[STAGE];
  __shared__ __attribute__((aligned(16))) float sW[WCHUNK];
  __shared__ __attribute__((aligned(16))) int32_t sT[WCHUNK];  // key times relative to the reference
  __shared__ int32_t sTB[TBK ? ATTN_MAX_TIME_BOUNDS : 1];
  __shared__ uint32_t sLUT[TBK ? BK_CELLS : 1];

  // flat grid over (user, head, tile), walked per XCD as in attn_fwd_rab_kernel
  const int TY = a.cand_tiles + a.hist_tiles;
  const int x8 = blockIdx.x & 7;
  const int kx = blockIdx.x >> 3;
  const int grp = kx / (TY * GROUP);
  const int rem = kx - grp * (TY * GROUP);
  const int y = rem / GROUP;
  const int bh = (grp * GROUP + (rem - y * GROUP)) * 8 + x8;
  if (bh >= a.B * a.H) return;
  const int u = bh / a.H;
  const int h = bh - u * a.H;
  const int64_t off = a.offsets[u];
  const int N = a.offsets[u + 1] - a.offsets[u];

  bool is_cand;
  int q0, nq, n_tiles;
  int64_t qrow0;
  if (y < a.cand_tiles) {
    is_cand = true;
    q0 = y * AQ;
    if (q0 >= a.m) return;
    nq = min(AQ, a.m - q0);
    qrow0 = a.crow0 + static_cast<int64_t>(u) * a.m + q0;
    n_tiles = (N + AK - 1) / AK;
  } else {
    is_cand = false;
    const int t = a.hist_tiles - 1 - (y - a.cand_tiles);  // largest tiles first
    q0 = t * AQ;
    if (q0 >= N) return;
    nq = min(AQ, N - q0);
    qrow0 = off + q0;
    n_tiles = FULL ? (N + AK - 1) / AK : (q0 + nq + AK - 1) / AK;
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;
  const float sp2 = a.sp2[h], st2 = a.st2[h];
  // Score units.  Separable bias: raw = q.k + w_j / c, log2 units = raw * c.  Otherwise the
  // scores are formed in log2 units (SC = 1).
  const float SC = SEP ? a.scale2 : 1.f;
  const float spr = SEP ? sp2 * a.rscale2 : sp2;
  const float str = SEP ? st2 * a.rscale2 : st2;
  const int p_ref = is_cand ? N : q0;

  // ---- register loads, all unconditional from valid addresses (a load behind a branch
  // makes the compiler wait for it at the join, before the ring below is issued)
  const int64_t ts_ref = is_cand ? a.req[u] : a.ts[off + q0];
  const int kt_first = n_tiles - 1;
  int wbase = n_tiles > 0 ? (kt_first * AK / WCHUNK) * WCHUNK : 0;
  static_assert(WCHUNK == NT, "one bias key per thread in the first chunk");
  const int wkey = wbase + tid;
  const bool wkey_in = wkey < N;
  int64_t ts_key = *(wkey_in ? a.ts + off + wkey : a.req + u);

  const int q_local = wave * QW + l16;
  const bool q_valid = q_local < nq;
  const int64_t qrow = qrow0 + q_local;
  const int q_slot = is_cand ? (N + q0 + q_local) : (q0 + q_local);
  const int k_lim = (is_cand || FULL) ? (N - 1) : min(q_slot, N - 1);
  const int kmax_blk = (is_cand || FULL) ? (N - 1) : min(q0 + wave * QW + 15, N - 1);
  const int64_t rowoff = (qrow0 + min(q_local, nq - 1)) * a.ld_qkv + h * DH;
  bf16x8_t qf[2];
  qf[0] = as_bf16x8(*reinterpret_cast<const uint4*>(a.q + rowoff + g4 * 8));
  qf[1] = as_bf16x8(*reinterpret_cast<const uint4*>(a.q + rowoff + g4 * 8 + 32));
  // a candidate's own key and value (merged after the history keys; history tiles read
  // and drop them)
  u32x4_t kself[2];
  u32x2_t vself[4];
  kself[0] = *reinterpret_cast<const u32x4_t*>(a.k + rowoff + g4 * 8);
  kself[1] = *reinterpret_cast<const u32x4_t*>(a.k + rowoff + g4 * 8 + 32);
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) vself[nb] = *reinterpret_cast<const u32x2_t*>(a.v + rowoff + nb * 16 + g4 * 4);
  // a history query's own time
  int64_t tq_raw = *(N > 0 ? a.ts + off + min(q_slot, N - 1) : a.req + u);

  // ---- the K/V ring.  Wave w loads rows 8 w .. 8 w + 7 of each tile: lane l takes row
  // 8 w + l / 8 and fills LDS chunk l % 8 of it, which holds the row's global chunk
  // (l % 8) ^ ((row >> 1) & 7) for K and (l % 8) ^ 2 ((row >> 1) & 3) for V (LDS has
  // 64 banks: the 16 rows of a K fragment read, and the 8 rows that two 16-lane groups of
  // a transposing V read cover, then fall on distinct banks).  Rows past the history end
  // re-read its last row (finite values; the mask gives those keys probability 0).
  // The prologue always issues NS - 1 tiles, so the compiler's waits for the register
  // loads above see one fixed count of loads behind them and leave the ring in flight;
  // tiles past the last read row 0 (with no history at all: the query row) into stage
  // buffers nothing reads.  Row offsets fit 32 bits (checked on the host).
  const int lr = wave * 8 + (lane >> 3);
  const int lc = lane & 7;
  const uint32_t row_bytes = static_cast<uint32_t>(a.ld_h) * 2u;
  const char* gk = reinterpret_cast<const char*>(N > 0 ? a.kh + off * a.ld_h + h * DH + ((lc ^ ((lr >> 1) & 7)) * 8) : a.q + rowoff);
  const char* gv = reinterpret_cast<const char*>(N > 0 ? a.vh + off * a.ld_h + h * DH + ((lc ^ (2 * ((lr >> 1) & 3))) * 8) : a.q + rowoff);
  auto issue = [&](int it, bf16_t* stg) {
    const int r = max(min((kt_first - it) * AK + lr, N - 1), 0);
    const uint32_t ro = static_cast<uint32_t>(r) * row_bytes;
    __builtin_amdgcn_global_load_lds((glb_void_t*)(gk + ro), (lds_void_t*)(stg + wave * 8 * DH), 16, 0, 0);
    __builtin_amdgcn_global_load_lds((glb_void_t*)(gv + ro), (lds_void_t*)(stg + AK * DH + wave * 8 * DH), 16, 0, 0);
  };
  issue(0, sg0);
  issue(1, sg1);
  issue(2, sg2);
  static_assert(NS == 4, "the prologue fills NS - 1 stages");
  // Direct loads and register loads in flight together leave the compiler unable to
  // order them, so its first wait for a register load waits for everything.  This empty
  // asm (which reads and redefines registers the loads above wrote) makes that one wait
  // come after the whole ring has been issued; the query fragments are covered too (see
  // attn_fwd_rab_kernel).
  asm volatile("" : "+v"(ts_key), "+v"(tq_raw), "+v"(qf[0]), "+v"(qf[1]), "+v"(kself[0]), "+v"(kself[1]),
               "+v"(vself[0]), "+v"(vself[1]), "+v"(vself[2]), "+v"(vself[3])::"memory");
  const int32_t tq = !is_cand && N > 0 ? static_cast<int32_t>(tq_raw - ts_ref) : 0;
  if constexpr (TBK)
    for (int k = tid; k < a.tb_p2; k += NT) {
      const int64_t b = k < a.n_tb ? a.tb[k] : INT64_MAX;
      sTB[k] = b > INT32_MAX ? INT32_MAX : (b < INT32_MIN ? INT32_MIN : static_cast<int32_t>(b));
    }

  // ---- bias terms of the first chunk, in the score units above
  sW[tid] = wkey_in ? key_term(TBK, spr, str, wkey - p_ref, static_cast<int32_t>(ts_key - ts_ref)) : 0.f;
  sT[tid] = wkey_in ? static_cast<int32_t>(ts_key - ts_ref) : 0;
  auto load_w = [&](int wb) {
    for (int j = tid; j < WCHUNK; j += NT) {
      const int key = wb + j;
      float w = 0.f;
      int32_t tk = 0;
      if (key < N) {
        tk = static_cast<int32_t>(a.ts[off + key] - ts_ref);
        w = key_term(TBK, spr, str, key - p_ref, tk);
      }
      sW[j] = w;
      sT[j] = tk;
    }
  };

  // ---- softmax state in score units
  f32x4_t accO[4];
  // row sums on the matrix cores: ones^T P^T adds a query's probabilities over all 32 keys
  // of a half tile into every element of its column, so each lane holds its query's sum
  f32x4_t lacc = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const bf16x8_t ones8 = as_bf16x8(make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));
  float m_run = -1e30f;
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) accO[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  lds_sync();  // sW, sT, sTB written
  float tbk_self = 0.f;  // bucketed time term of a candidate's own key (gap 0)
  if constexpr (TBK) {
    tbk_self = st2 * static_cast<float>(bucket_search(sTB, a.tb_p2, 0));
    bucket_table_build(sLUT, sTB, a.tb_p2, tid, NT);
    lds_sync();
  }
  // the row term of the bias in log2 units, added back into the log-sum-exp
  float w_i = 0.f;
  if constexpr (FULL) {
    w_i = (!is_cand && q_valid) ? (TBK ? sp2 * static_cast<float>(q_slot - p_ref)
                                       : sp2 * static_cast<float>(q_slot - p_ref) + st2 * static_cast<float>(tq))
                                : 0.f;
  } else {
    w_i = (!is_cand && q_valid) ? sW[q_slot - wbase] * SC : 0.f;
  }
  const float w_i_u = w_i / SC;  // the same in score units (FULL only)
  // a wave whose queries lie far from the tile's reference point forms each bias exactly
  // from the pair's own position and time differences (its row term is then 0)
  const bool far = CAN_FAR && __builtin_amdgcn_ballot_w64(fabsf(w_i) > BIAS_FAR_LOG2) != 0;
  if (far) w_i = 0.f;
  // the exact bias of key slot j for this lane's query, in score units (far waves)
  auto exact_bias = [&](int j, int32_t tk) __attribute__((always_inline)) {
    return key_term(false, spr, str, j - q_slot, tk - tq);
  };

  // LDS offsets (bf16 elements) of this lane's fragments inside a stage buffer
  const int k_off0 = l16 * DH + (((0 + g4) ^ ((l16 >> 1) & 7)) * 8);
  const int k_off1 = l16 * DH + (((4 + g4) ^ ((l16 >> 1) & 7)) * 8);
  int v_off[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
    v_off[nb] = AK * DH + (4 * g4 + (l16 >> 2)) * DH +
                (((2 * nb + ((l16 & 3) >> 1)) ^ (2 * (((4 * g4 + (l16 >> 2)) >> 1) & 3))) * 8) + (l16 & 1) * 4;
  const float th = RESCALE_LOG2 / SC;
  const bool wave_on = wave * QW < nq;

  auto compute = [&](auto masked_tag, auto far_tag, const bf16_t* stg, int it) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    constexpr bool FAR = decltype(far_tag)::value;
    const int base = (kt_first - it) * AK;
    f32x4_t s[4];
    float4 wv[4];
    int4 tv[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      wv[kb] = reinterpret_cast<const float4*>(sW)[((base - wbase) >> 2) + kb * 4 + g4];
      tv[kb] = (TBK || FAR) ? reinterpret_cast<const int4*>(sT)[((base - wbase) >> 2) + kb * 4 + g4]
                            : make_int4(0, 0, 0, 0);
      const int j0 = base + kb * 16 + g4 * 4;
      if constexpr (SEP && FAR)
        s[kb] = f32x4_t{exact_bias(j0, tv[kb].x), exact_bias(j0 + 1, tv[kb].y), exact_bias(j0 + 2, tv[kb].z),
                        exact_bias(j0 + 3, tv[kb].w)};
      else
        s[kb] = SEP ? f32x4_t{wv[kb].x, wv[kb].y, wv[kb].z, wv[kb].w} : f32x4_t{0.f, 0.f, 0.f, 0.f};
      if (!MASKED || base + kb * 16 <= kmax_blk) {
        const bf16x8_t k0 = as_bf16x8(*reinterpret_cast<const uint4*>(stg + kb * 16 * DH + k_off0));
        const bf16x8_t k1 = as_bf16x8(*reinterpret_cast<const uint4*>(stg + kb * 16 * DH + k_off1));
        s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qf[0], s[kb], 0, 0, 0);
        s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qf[1], s[kb], 0, 0, 0);
      }
    }
    if constexpr (!SEP) {
      // fully visible: -|w_j - w_i|; bucketed time: - s' bucket(|t_i - t_j|)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const float wk[4] = {wv[kb].x, wv[kb].y, wv[kb].z, wv[kb].w};
        const int32_t tk[4] = {tv[kb].x, tv[kb].y, tv[kb].z, tv[kb].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float fb = FAR ? -fabsf(exact_bias(base + kb * 16 + g4 * 4 + i, tk[i])) : -fabsf(wk[i] - w_i_u);
          float x = biased(s[kb][i], a.scale2, FULL ? fb : wk[i]);
          if constexpr (TBK) x -= st2 * static_cast<float>(bucket_lookup(sLUT, sTB, a.tb_p2, abs(tq - tk[i])));
          s[kb][i] = x;
        }
      }
    }
    if constexpr (MASKED) {
      const int lim = k_lim - base - g4 * 4;  // local key kb*16 + i must be <= lim
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (kb * 16 + i > lim) s[kb][i] = -INFINITY;
    }
    float mx = max16(s);
    // Some query's maximum exceeds its threshold exactly when some lane's share of it does,
    // so the lane-local maximum decides, and the four lane groups of a query combine their
    // shares only on the rare raise.
    if (__builtin_amdgcn_ballot_w64(mx > m_run + th) != 0) {  // rare: raise the maximum
      mx = xor32_max(xor16_max(mx));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * SC);
      m_run = m_new;
      lacc = lacc * alpha;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) accO[nb] = accO[nb] * alpha;
    }
    const float mb = -m_run * SC;
    bf16x8_t pf[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      uint4 pk;
      uint32_t* pw = reinterpret_cast<uint32_t*>(&pk);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4_t& sb = s[2 * ks + (j >> 1)];
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sb[(j & 1) * 2], SC, mb));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sb[(j & 1) * 2 + 1], SC, mb));
        pw[j] = pack_bf16x2(p0, p1);
      }
      pf[ks] = as_bf16x8(pk);
    }
    // O^T += V^T P^T; the V^T fragment: two transposing reads of 4 keys each
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      if (MASKED && base + ks * 32 > kmax_blk) continue;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16_t*)(stg + v_off[nb] + (ks * 32) * DH));
        const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16_t*)(stg + v_off[nb] + (ks * 32 + 16) * DH));
        const v4i16_t both[2] = {lo, hi};
        accO[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, both), pf[ks], accO[nb], 0, 0, 0);
      }
      lacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones8, pf[ks], lacc, 0, 0, 0);
    }
  };

  // Tile it (key tile kt_first - it, newest first) sits in stage buffer it % NS.  A step
  // reloads the bias chunk when the tile leaves it (histories longer than WCHUNK keys),
  // waits for its own tile (the newer tiles may stay in flight: two loads each), meets the
  // other waves, refills the buffer the previous step read with tile it + NS - 1, and
  // computes.  Masks are needed only in the first two tiles (the ragged history end and
  // the causal diagonal); every later tile lies wholly below every query's limit.
  auto step = [&](auto masked_tag, auto far_tag, auto stage_tag, int it) __attribute__((always_inline)) {
    constexpr int S = decltype(stage_tag)::value;
    bf16_t* const cur = S == 0 ? sg0 : S == 1 ? sg1 : S == 2 ? sg2 : sg3;
    bf16_t* const nxt = S == 0 ? sg3 : S == 1 ? sg0 : S == 2 ? sg1 : sg2;  // stage (it - 1) % NS
    if ((kt_first - it) * AK < wbase) {
      lds_sync();
      wbase -= WCHUNK;
      load_w(wbase);
      lds_sync();
    }
    const int left = kt_first - it;  // tiles after this one
    if (left >= 2) wait_vmcnt<4>(); else if (left == 1) wait_vmcnt<2>(); else wait_vmcnt<0>();
    lds_barrier();
    if (it + NS - 1 < n_tiles) issue(it + NS - 1, nxt);
    if (wave_on) compute(masked_tag, far_tag, cur, it);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  // (a far wave runs its own copy of the loop, with the same waits and barriers in the same
  // order as the other waves)
  auto loop = [&](auto far_tag) __attribute__((always_inline)) {
    if (n_tiles > 0) step(std::true_type{}, far_tag, I0{}, 0);
    if (n_tiles > 1) step(std::true_type{}, far_tag, I1{}, 1);
    for (int it = 2; it < n_tiles; it += NS) {
      step(std::false_type{}, far_tag, I2{}, it);
      if (it + 1 < n_tiles) step(std::false_type{}, far_tag, I3{}, it + 1);
      if (it + 2 < n_tiles) step(std::false_type{}, far_tag, I0{}, it + 2);
      if (it + 3 < n_tiles) step(std::false_type{}, far_tag, I1{}, it + 3);
    }
  };
  if constexpr (CAN_FAR) {
    if (far)
      loop(std::true_type{});
    else
      loop(std::false_type{});
  } else {
    loop(std::false_type{});
  }
  wait_vmcnt<0>();  // no direct load may still be writing LDS when the workgroup ends
  float lsum = lacc[0];
  if (is_cand) merge_self(kself, vself, qf, SEP, a.scale2, tbk_self, SC, th, g4, m_run, lsum, accO);

  // ---- epilogue
  const float ltot = lsum;
  if (!q_valid) return;
  // (a row's sum is at least 1: the hardware reciprocal and log2 need no range fix-up)
  const float inv = __builtin_amdgcn_rcpf(ltot);
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    uint2 o;
    o.x = pack_bf16x2(accO[nb][0] * inv, accO[nb][1] * inv);
    o.y = pack_bf16x2(accO[nb][2] * inv, accO[nb][3] * inv);
    *reinterpret_cast<uint2*>(a.o + qrow * a.ld_o + h * DH + nb * 16 + g4 * 4) = o;
  }
  if (a.lse && g4 == 0)
    a.lse[qrow * a.H + h] = LN2 * (m_run * SC + __builtin_amdgcn_logf(ltot) - (FULL ? 0.f : w_i));
}

// ------------------------------------------------------------------ bf16 pair kernel
// One workgroup per (user, head) pair, for batches whose longest history fits in LDS
// (PAIR_MAXK keys).  The pair's whole K and V history goes into LDS once, in 64-key tiles
// (direct loads with the ring kernel's swizzles; V^T operands through transposing reads),
// together with every key's bias term.  The 12 waves then work through the pair's 32-query units
// (candidate units first, then history units newest first) with no further barrier:
// each wave runs its units' key tiles from LDS on its own.  Against the tile grid this
// loads every K/V byte of a pair once instead of once per query tile, and pays one
// workgroup prologue per pair instead of one per query tile.  Workgroups take the users
// heaviest first (see below), so the light pairs fill the end of the launch.
// A unit is two 16-query blocks, A and B, that share every K and V fragment read (half
// the LDS traffic per query of one block per wave).  Per key tile the wave issues both
// blocks' score products, runs A's softmax while B's products finish, then B's, then the
// PV products of each 32-key half right after that half's V^T fragments are read.  The
// fragments of one half only are held, the next unit's queries and a candidate's own
// key and value are fetched after the key tiles, so a wave fits 168 registers and three
// waves share each SIMD (with two per SIMD at 256 registers: 553 us against 520 us per
// launch of the four-layer batch; one 16-query block per wave, 16 waves: 535 us, as the
// K/V fragment reads per query double).  Each block's
// arithmetic is that of one 16-query wave of the ring kernel: the same bias terms, the
// same lazy-rescaling decisions over its 16 queries, the same row-sum order, so candidate
// rows come out of both kernels bit for bit alike.
// The bias reference point of the whole pair is the candidates' shared (p, tau) = (N,
// request time), so candidate rows carry no row term.  A candidate's own key is merged
// into its softmax state after the history keys (same result as seeding with it).
constexpr int PAIR_WAVES = 12;
constexpr int PAIR_NT = 64 * PAIR_WAVES;
constexpr int PAIR_MAXT = 9;                 // key tiles held in LDS
constexpr int PAIR_MAXK = PAIR_MAXT * AK;    // longest history this kernel takes
constexpr int PB = 2;                        // 16-query blocks per unit
constexpr int PQ = PB * QW;                  // queries per unit
constexpr int PAIR_RG = 2 * AK / 8;          // 8-row groups of a K tile and its V tile
static_assert(PAIR_WAVES <= PAIR_RG && 2 * PAIR_WAVES >= PAIR_RG, "each wave loads one or two row groups");

template <int VAR>
__global__ void __launch_bounds__(PAIR_NT) attn_fwd_pair_kernel(AttnArgs a) {
  constexpr bool FULL = (VAR & VAR_FULL) != 0;
  constexpr bool TBK = (VAR & VAR_TBUCKET) != 0;
  constexpr bool SEP = VAR == 0;
  constexpr bool CAN_FAR = !TBK;  // the bucketed variants' key terms hold the position part only
  __shared__ __attribute__((aligned(16))) bf16_t sKV[PAIR_MAXT * STAGE];
  __shared__ __attribute__((aligned(16))) float sW[PAIR_MAXK];
  __shared__ __attribute__((aligned(16))) int32_t sT[PAIR_MAXK];  // key times relative to the request
  __shared__ int32_t sTB[TBK ? ATTN_MAX_TIME_BOUNDS : 1];
  __shared__ uint32_t sLUT[TBK ? BK_CELLS : 1];
  __shared__ int sCnt[PAIR_MAXT + 1];
  __shared__ int sWave[PAIR_WAVES];
  __shared__ int sUser, sLen;
  __shared__ int64_t sOff, sReq;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // Which pair: workgroups run in launch order, so the pairs go heaviest first (users
  // ordered by key-tile count, descending, ties by index) and the light ones fill the end
  // of the launch.  Every workgroup derives the same order from the offsets.  With more
  // users than threads, or when every history has the same length (the host knows it:
  // total_hist = B max_hist), the order is the plain one.  The thread that finds the pair
  // passes on its user's offset, length and request time (no second round trip).
  const int ur = blockIdx.x / a.H;
  const int h = blockIdx.x - ur * a.H;
  int u = ur, len;
  int64_t off, ts_ref;
  if (a.order && a.B <= PAIR_NT) {
    if (tid <= PAIR_MAXT) sCnt[tid] = 0;
    int ntl = -1, o0 = 0, o1 = 0;
    int64_t rq = 0;
    if (tid < a.B) {
      o0 = a.offsets[tid];
      o1 = a.offsets[tid + 1];
      rq = a.req[tid];
      ntl = (min(o1 - o0, PAIR_MAXK) + AK - 1) / AK;
    }
    lds_sync();
    if (ntl >= 0) atomicAdd(&sCnt[ntl], 1);
    lds_sync();
    int bk = PAIR_MAXT, before = 0;  // the tile-count class holding rank ur
    while (bk > 0 && before + sCnt[bk] <= ur) before += sCnt[bk--];
    const bool mine = ntl == bk;
    const uint64_t bal = __builtin_amdgcn_ballot_w64(mine);
    const int below = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(bal >> 32), __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bal), 0));
    if (lane == 0) sWave[wave] = __builtin_popcountll(bal);
    lds_sync();
    int rank = below;
    for (int w = 0; w < wave; ++w) rank += sWave[w];
    if (mine && rank == ur - before) {
      sUser = tid;
      sOff = o0;
      sLen = o1 - o0;
      sReq = rq;
    }
    lds_sync();
    u = sUser;
    off = sOff;
    len = sLen;
    ts_ref = sReq;
  } else {
    off = a.offsets[u];
    len = a.offsets[u + 1] - a.offsets[u];
    ts_ref = a.req[u];
  }
  // (a history longer than the batch's declared maximum is cut, so that LDS is never
  // overrun, and flagged in the device error word; the declared maximum is the caller's
  // promise)
  if (len > PAIR_MAXK && tid == 0) report_error(a.err, GENRANK_ERR_HIST_LONG);
  const int N = min(len, PAIR_MAXK);
  const int n_tiles = (N + AK - 1) / AK;
  const int l16 = lane & 15, g4 = lane >> 4;
  const float sp2 = a.sp2[h], st2 = a.st2[h];
  const float SC = SEP ? a.scale2 : 1.f;
  const float spr = SEP ? sp2 * a.rscale2 : sp2;
  const float str = SEP ? st2 * a.rscale2 : st2;

  // ---- units: PQ-query blocks, candidates first (each sees every key), then history
  // blocks newest first, so in order of non-increasing key-tile count.  Wave w takes one
  // unit per round, in snake order: w in even rounds, PAIR_WAVES - 1 - w in odd ones, which
  // evens out the waves' key tiles.
  const int nu_c = (a.m + PQ - 1) / PQ;
  const int nu_h = a.hist_tiles > 0 ? (N + PQ - 1) / PQ : 0;
  const int n_units = nu_c + nu_h;
  // unit k's first row in q / k / v / o (wave-uniform) and its number of queries; a
  // lane's rows are that row plus a small offset, so addresses are a scalar base plus a
  // 32-bit lane offset (row strides fit 32 bits: checked on the host)
  auto unit_row0 = [&](int k) -> int64_t {
    return k < nu_c ? a.crow0 + static_cast<int64_t>(u) * a.m + k * PQ : off + (nu_h - 1 - (k - nu_c)) * PQ;
  };
  auto unit_nq = [&](int k) -> int { return min(PQ, k < nu_c ? a.m - k * PQ : N - (nu_h - 1 - (k - nu_c)) * PQ); };
  const uint32_t ldq = static_cast<uint32_t>(a.ld_qkv);
  u32x4_t qn[PB][2] = {};
  auto fetch_q = [&](int k) __attribute__((always_inline)) {
    const char* qb = reinterpret_cast<const char*>(a.q + unit_row0(k) * a.ld_qkv + h * DH);
    const int nq = unit_nq(k);
#pragma unroll
    for (int hb = 0; hb < PB; ++hb) {  // rows past the unit's last query re-read it
      const uint32_t lo = (static_cast<uint32_t>(min(hb * QW + l16, nq - 1)) * ldq + g4 * 8) * 2u;
      qn[hb][0] = *reinterpret_cast<const u32x4_t*>(qb + lo);
      qn[hb][1] = *reinterpret_cast<const u32x4_t*>(qb + lo + 64);
    }
  };
  auto unit_of = [&](int r) -> int { return r * PAIR_WAVES + ((r & 1) ? PAIR_WAVES - 1 - wave : wave); };
  // the first unit's query fragments travel with the K/V tiles
  if (wave < n_units) fetch_q(wave);

  // ---- the pair's K/V tiles, row-major (key, dim), straight into LDS, in 8-row groups:
  // groups 0-7 are rows 8 g .. 8 g + 7 of every K tile, groups 8-15 the same rows of every V
  // tile; wave w loads groups w and w + PAIR_WAVES (lane l: row 8 (g % 8) + l / 8, LDS chunk
  // l % 8 <- global chunk (l % 8) ^ ((row >> 1) & 7) for K, (l % 8) ^ 2 ((row >> 1) & 3) for
  // V).  Rows past the history end re-read its last row.
  const int lc = lane & 7;
  for (int rg = wave; rg < PAIR_RG; rg += PAIR_WAVES) {
    const int kv_half = rg >> 3;  // 0: K, 1: V (wave-uniform)
    const int lr = (rg & 7) * 8 + (lane >> 3);
    const uint32_t row_bytes = static_cast<uint32_t>(a.ld_h) * 2u;
    const char* g = kv_half == 0
                        ? reinterpret_cast<const char*>(a.kh + off * a.ld_h + h * DH + ((lc ^ ((lr >> 1) & 7)) * 8))
                        : reinterpret_cast<const char*>(a.vh + off * a.ld_h + h * DH + ((lc ^ (2 * ((lr >> 1) & 3))) * 8));
    bf16_t* dst = sKV + kv_half * AK * DH + (rg & 7) * 8 * DH;
#pragma unroll
    for (int t = 0; t < PAIR_MAXT; ++t) {
      if (t < n_tiles) {
        const uint32_t ro = static_cast<uint32_t>(min(t * AK + lr, N - 1)) * row_bytes;
        __builtin_amdgcn_global_load_lds((glb_void_t*)(g + ro), (lds_void_t*)(dst + t * STAGE), 16, 0, 0);
      }
    }
  }

  // ---- every key's bias term relative to the candidates; -inf past the history end, so
  // that those keys' scores come out -inf (probability 0) without a mask
  for (int j = tid; j < n_tiles * AK; j += PAIR_NT) {
    float w = -INFINITY;
    int32_t tk = 0;
    if (j < N) {
      tk = static_cast<int32_t>(a.ts[off + j] - ts_ref);
      w = key_term(TBK, spr, str, j - N, tk);
    }
    sW[j] = w;
    sT[j] = tk;
  }
  if constexpr (TBK)
    for (int k = tid; k < a.tb_p2; k += PAIR_NT) {
      const int64_t b = k < a.n_tb ? a.tb[k] : INT64_MAX;
      sTB[k] = b > INT32_MAX ? INT32_MAX : (b < INT32_MIN ? INT32_MIN : static_cast<int32_t>(b));
    }
  wait_vmcnt<0>();
  lds_sync();
  float tbk_self = 0.f;  // bucketed time term of a candidate's own key (gap 0)
  if constexpr (TBK) {
    tbk_self = st2 * static_cast<float>(bucket_search(sTB, a.tb_p2, 0));
    bucket_table_build(sLUT, sTB, a.tb_p2, tid, PAIR_NT);
    lds_sync();
  }

  const float th = RESCALE_LOG2 / SC;
  // LDS offsets (bf16 elements) of this lane's fragments inside a tile
  const int k_off0 = l16 * DH + (((0 + g4) ^ ((l16 >> 1) & 7)) * 8);
  const int k_off1 = l16 * DH + (((4 + g4) ^ ((l16 >> 1) & 7)) * 8);
  // V^T operand of dim block nb through transposing reads of the row-major V tile: within
  // each 16-lane group, output lane j element e of ds_read_b64_tr_b16 is element j % 4 of
  // the 8 bytes lane 4 e + j / 4 addressed.  Lane (l16, g4) addresses key row 4 g4 + l16 / 4
  // (and + 16, in the 32-key half), dims 16 nb + 4 (l16 % 4) .., through V's swizzle; so
  // lane group g4 receives dim 16 nb + l16 of keys 4 g4 .. 4 g4 + 3 and 16 + 4 g4 .., the
  // keys its P^T fragment holds.
  int v_off[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
    v_off[nb] = AK * DH + (4 * g4 + (l16 >> 2)) * DH +
                (((2 * nb + ((l16 & 3) >> 1)) ^ (2 * (((4 * g4 + (l16 >> 2)) >> 1) & 3))) * 8) + (l16 & 1) * 4;
  // a tile's start as a wave-uniform value: every fragment read is then one address
  // register plus a constant offset
  auto tile_at = [&](int kt) __attribute__((always_inline)) {
    return sKV + __builtin_amdgcn_readfirstlane(kt * STAGE);
  };

  for (int r = 0, k = wave; k < n_units; k = unit_of(++r)) {
    const bool is_cand = k < nu_c;
    const int b = is_cand ? k : nu_h - 1 - (k - nu_c);
    const int qf0 = b * PQ;                               // first query of the unit
    const int nq = min(PQ, (is_cand ? a.m : N) - qf0);
    const int n_t = (is_cand || FULL) ? n_tiles : (qf0 + nq - 1) / AK + 1;
    // causal history units: the 16-key block of the first (newest) tile that holds the
    // unit's (first) block's diagonal; a second block's would be the next one (query blocks
    // are 16-aligned, a unit's queries lie in one tile)
    const int kd0 = (qf0 - (n_t - 1) * AK) >> 4;
    const int64_t row0 = unit_row0(k);
    bf16x8_t qf[PB][2];
    bool q_valid[PB];
    int q_slot[PB];
    int32_t tq[PB];
    float w_i_ref[PB];
#pragma unroll
    for (int hb = 0; hb < PB; ++hb) {
      qf[hb][0] = __builtin_bit_cast(bf16x8_t, qn[hb][0]);
      qf[hb][1] = __builtin_bit_cast(bf16x8_t, qn[hb][1]);
      q_valid[hb] = hb * QW + l16 < nq;
      q_slot[hb] = (is_cand ? N : 0) + qf0 + hb * QW + l16;
      // the row term (log2 units) and the query's own time
      w_i_ref[hb] = (!is_cand && q_valid[hb]) ? sW[min(q_slot[hb], N - 1)] * SC : 0.f;
      tq[hb] = (!is_cand && N > 0) ? sT[min(q_slot[hb], N - 1)] : 0;
    }
    // a history unit far from the candidates' reference point forms each bias exactly
    // from the pair's own position and time differences (the row terms are then 0)
    bool far_lane = false;
#pragma unroll
    for (int hb = 0; hb < PB; ++hb) far_lane = far_lane || fabsf(w_i_ref[hb]) > BIAS_FAR_LOG2;
    const bool far = CAN_FAR && __builtin_amdgcn_ballot_w64(far_lane) != 0;
    float w_i[PB], w_i_u[PB];
#pragma unroll
    for (int hb = 0; hb < PB; ++hb) {
      w_i[hb] = far ? 0.f : w_i_ref[hb];
      w_i_u[hb] = w_i_ref[hb] / SC;
    }

    f32x4_t accO[PB][4];
#pragma unroll
    for (int hb = 0; hb < PB; ++hb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) accO[hb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m_run[PB];
    f32x4_t lacc[PB];  // row sums on the matrix cores, as in the ring kernel
    // the raise threshold and the exponent's offset follow the maximum (set where it moves)
    float m_thr[PB], m_bias[PB];
#pragma unroll
    for (int hb = 0; hb < PB; ++hb) {
      m_run[hb] = -1e30f;
      lacc[hb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      m_thr[hb] = -1e30f + th;
      m_bias[hb] = 1e30f * SC;
    }
    f32x4_t s[PB][4];
    const bf16x8_t ones8 = as_bf16x8(make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));

    // the exact bias of key slot j for this lane's query of block hb, in score units (far
    // units): from the integer position and time differences, each product rounded once
    auto exact_bias = [&](int hb, int j, int32_t tk) __attribute__((always_inline)) {
      return key_term(false, spr, str, j - q_slot[hb], tk - tq[hb]);
    };
    // S^T of key tile kt for both blocks (with the separable bias: seeded with the key
    // terms); each K fragment read feeds both blocks
    auto scores = [&](auto masked_tag, auto far_tag, int kt) __attribute__((always_inline)) {
      constexpr bool MASKED = decltype(masked_tag)::value;
      constexpr bool FAR = decltype(far_tag)::value;
      const bf16_t* stg = tile_at(kt);
      const int base = kt * AK;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        if constexpr (SEP && FAR) {
          const int4 t4 = reinterpret_cast<const int4*>(sT)[(base >> 2) + kb * 4 + g4];
          const int j0 = base + kb * 16 + g4 * 4;
#pragma unroll
          for (int hb = 0; hb < PB; ++hb)
            s[hb][kb] = f32x4_t{exact_bias(hb, j0, t4.x), exact_bias(hb, j0 + 1, t4.y),
                                exact_bias(hb, j0 + 2, t4.z), exact_bias(hb, j0 + 3, t4.w)};
        } else if constexpr (SEP) {
          const float4 w = reinterpret_cast<const float4*>(sW)[(base >> 2) + kb * 4 + g4];
          s[0][kb] = f32x4_t{w.x, w.y, w.z, w.w};
          if constexpr (PB == 2) s[PB - 1][kb] = s[0][kb];
        } else {
          s[0][kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          if constexpr (PB == 2) s[PB - 1][kb] = s[0][kb];
        }
        if (MASKED && kb > kd0) {  // the first block lies wholly above its diagonal here
          s[0][kb] = f32x4_t{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
          if (PB == 1 || kb > kd0 + 1) {
            if constexpr (PB == 2) s[PB - 1][kb] = s[0][kb];
            continue;
          }
        }
        const bf16x8_t k0 = as_bf16x8(*reinterpret_cast<const uint4*>(stg + kb * 16 * DH + k_off0));
        const bf16x8_t k1 = as_bf16x8(*reinterpret_cast<const uint4*>(stg + kb * 16 * DH + k_off1));
        if constexpr (PB == 1) {
          s[0][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qf[0][0], s[0][kb], 0, 0, 0);
          s[0][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qf[0][1], s[0][kb], 0, 0, 0);
        } else if (!MASKED || kb <= kd0) {
          s[0][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qf[0][0], s[0][kb], 0, 0, 0);
          s[PB - 1][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qf[PB - 1][0], s[PB - 1][kb], 0, 0, 0);
          s[0][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qf[0][1], s[0][kb], 0, 0, 0);
          s[PB - 1][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qf[PB - 1][1], s[PB - 1][kb], 0, 0, 0);
        } else {
          s[PB - 1][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qf[PB - 1][0], s[PB - 1][kb], 0, 0, 0);
          s[PB - 1][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qf[PB - 1][1], s[PB - 1][kb], 0, 0, 0);
        }
      }
    };
    // block hb on key tile kt: bias (variants), mask, online softmax; P^T as two bf16
    // fragments
    auto softmax = [&](auto masked_tag, auto far_tag, int kt, auto hb_tag, bf16x8_t(&pf)[2]) __attribute__((always_inline)) {
      constexpr bool MASKED = decltype(masked_tag)::value;
      constexpr bool FAR = decltype(far_tag)::value;
      constexpr int hb = decltype(hb_tag)::value;
      const int base = kt * AK;
      f32x4_t(&sc)[4] = s[hb];
      if constexpr (!SEP) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const float4 wq = reinterpret_cast<const float4*>(sW)[(base >> 2) + kb * 4 + g4];
          const float wk[4] = {wq.x, wq.y, wq.z, wq.w};
          int4 t4 = make_int4(0, 0, 0, 0);
          if constexpr (TBK || FAR) t4 = reinterpret_cast<const int4*>(sT)[(base >> 2) + kb * 4 + g4];
          const int32_t tk[4] = {t4.x, t4.y, t4.z, t4.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            // fully visible: -|w_j - w_i|, or the exact -|bias| of the pair in far units (keys
            // past the history end, whose key terms are -inf, stay -inf)
            const float fb = FAR ? (wk[i] == -INFINITY ? -INFINITY : -fabsf(exact_bias(hb, base + kb * 16 + g4 * 4 + i, tk[i])))
                                 : -fabsf(wk[i] - w_i_u[hb]);
            float x = biased(sc[kb][i], a.scale2, FULL ? fb : wk[i]);
            if constexpr (TBK) x -= st2 * static_cast<float>(bucket_lookup(sLUT, sTB, a.tb_p2, abs(tq[hb] - tk[i])));
            sc[kb][i] = x;
          }
        }
      }
      if constexpr (MASKED) {  // the diagonal block: key g4 * 4 + i against query l16
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
          if (kb == kd0 + hb) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (g4 * 4 + i > l16) sc[kb][i] = -INFINITY;
          }
      }
      float mx = max16(sc);
      // (the lane-local maximum decides, as in the ring kernel; a query's four lane groups
      // combine their shares only on the rare raise)
      if (__builtin_amdgcn_ballot_w64(mx > m_thr[hb]) != 0) {
        mx = xor32_max(xor16_max(mx));
        const float m_new = fmaxf(m_run[hb], mx);
        const float alpha = __builtin_amdgcn_exp2f((m_run[hb] - m_new) * SC);
        m_run[hb] = m_new;
        m_thr[hb] = m_new + th;
        m_bias[hb] = -m_new * SC;
        lacc[hb] = lacc[hb] * alpha;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) accO[hb][nb] = accO[hb][nb] * alpha;
      }
      const float mb = m_bias[hb];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        uint4 pk;
        uint32_t* pw = reinterpret_cast<uint32_t*>(&pk);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4_t& sb = sc[2 * ks + (j >> 1)];
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sb[(j & 1) * 2], SC, mb));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sb[(j & 1) * 2 + 1], SC, mb));
          pw[j] = pack_bf16x2(p0, p1);
        }
        pf[ks] = as_bf16x8(pk);
      }
    };
    // O^T += V^T P^T for every block, the V^T fragments of each 32-key half read right
    // before its products (16 registers of fragments held instead of 32)
    auto pv_direct = [&](auto masked_tag, int kt, const bf16x8_t(&pa)[2], const bf16x8_t(&pb)[2]) __attribute__((always_inline)) {
      constexpr bool MASKED = decltype(masked_tag)::value;
      const bf16_t* stg = tile_at(kt);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        if (MASKED && 2 * ks > kd0 + PB - 1) continue;  // past every block's diagonal
        bf16x8_t vh[4];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(stg + v_off[nb] + (ks * 32) * DH));
          const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(stg + v_off[nb] + (ks * 32 + 16) * DH));
          const v4i16_t both[2] = {lo, hi};
          vh[nb] = __builtin_bit_cast(bf16x8_t, both);
        }
        if (!(MASKED && 2 * ks > kd0)) {  // (the first block's diagonal)
#pragma unroll
          for (int nb = 0; nb < 4; ++nb)
            accO[0][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vh[nb], pa[ks], accO[0][nb], 0, 0, 0);
          lacc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones8, pa[ks], lacc[0], 0, 0, 0);
        }
        if constexpr (PB == 2) {
#pragma unroll
          for (int nb = 0; nb < 4; ++nb)
            accO[PB - 1][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vh[nb], pb[ks], accO[PB - 1][nb], 0, 0, 0);
          lacc[PB - 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones8, pb[ks], lacc[PB - 1], 0, 0, 0);
        }
      }
    };
    // one key tile: the blocks' scores, their softmaxes, then the PV products
    auto tile = [&](auto masked_tag, auto far_tag, int kt) __attribute__((always_inline)) {
      using HA = std::integral_constant<int, 0>;
      using HB = std::integral_constant<int, PB - 1>;
      bf16x8_t pa[2], pb[2];
      scores(masked_tag, far_tag, kt);
      softmax(masked_tag, far_tag, kt, HA{}, pa);
      if constexpr (PB == 2) softmax(masked_tag, far_tag, kt, HB{}, pb);
      pv_direct(masked_tag, kt, pa, pb);
    };
    // Key tiles newest first; only the first can cross a causal query's limit.  A
    // candidate's limit is the history end, which the -inf bias terms already enforce, and
    // so is every key's limit under the fully visible history (candidate units are never
    // far: their reference point is their own).
    auto run_tiles = [&](auto far_tag) __attribute__((always_inline)) {
      if (is_cand || FULL)
        tile(std::false_type{}, far_tag, n_t - 1);
      else
        tile(std::true_type{}, far_tag, n_t - 1);
      for (int kt = n_t - 2; kt >= 0; --kt) tile(std::false_type{}, far_tag, kt);
    };
    if (n_t > 0) {
      if constexpr (CAN_FAR) {
        if (far)
          run_tiles(std::true_type{});
        else
          run_tiles(std::false_type{});
      } else {
        run_tiles(std::false_type{});
      }
    }

    // the next unit's query fragments, and a candidate's own key and value (merged after
    // the history keys), fetched only now so that they hold no registers in the tile loop
    if (unit_of(r + 1) < n_units) fetch_q(unit_of(r + 1));
    u32x4_t kself[PB][2] = {};
    u32x2_t vself[PB][4] = {};
    if (is_cand) {
      const char* kb0 = reinterpret_cast<const char*>(a.k + row0 * a.ld_qkv + h * DH);
      const char* vb0 = reinterpret_cast<const char*>(a.v + row0 * a.ld_qkv + h * DH);
#pragma unroll
      for (int hb = 0; hb < PB; ++hb) {
        const uint32_t lo = static_cast<uint32_t>(min(hb * QW + l16, nq - 1)) * ldq * 2u;
        kself[hb][0] = *reinterpret_cast<const u32x4_t*>(kb0 + lo + g4 * 16);
        kself[hb][1] = *reinterpret_cast<const u32x4_t*>(kb0 + lo + g4 * 16 + 64);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) vself[hb][nb] = *reinterpret_cast<const u32x2_t*>(vb0 + lo + nb * 32 + g4 * 8);
      }
    }
    // Waiting for these loads here, ahead of the stores, leaves the stores in flight into
    // the next unit instead of a wait for everything at its start.
    wait_vmcnt<0>();
#pragma unroll
    for (int hb = 0; hb < PB; ++hb) {
      // the candidate's own key: bias 0 (it is the reference point)
      float lsum = lacc[hb][0];
      if (is_cand)
        merge_self(kself[hb], vself[hb], qf[hb], SEP, a.scale2, tbk_self, SC, th, g4, m_run[hb], lsum, accO[hb]);
      const float ltot = lsum;
      const float inv = __builtin_amdgcn_rcpf(ltot);  // (as in the ring kernel)
      // Lane groups g4 and g4 ^ 1 (same query) trade halves: lane group g4 then holds the 8
      // consecutive dimensions 8 (g4 / 2) + 16 (g4 % 2) .. + 7 of blocks nb = 0, 1, and the
      // same + 32 of nb = 2, 3, so a row leaves in two 16-byte stores per lane, each wave store
      // covering 64 contiguous bytes of a row.  (The lane-swap puts odd 16-lane rows of its
      // first operand in the even rows of its second.)
      uint4 ow[2];
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        float xs[4], ys[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(accO[hb][2 * pp][i] * inv),
                                                          __float_as_uint(accO[hb][2 * pp + 1][i] * inv), false, false);
          xs[i] = __uint_as_float(r[0]);
          ys[i] = __uint_as_float(r[1]);
        }
        ow[pp] = make_uint4(pack_bf16x2(xs[0], xs[1]), pack_bf16x2(xs[2], xs[3]), pack_bf16x2(ys[0], ys[1]),
                            pack_bf16x2(ys[2], ys[3]));
      }
      if (q_valid[hb]) {
        char* ob = reinterpret_cast<char*>(a.o + row0 * a.ld_o + h * DH);
        const uint32_t dbase = 8 * (g4 >> 1) + 16 * (g4 & 1);
        const uint32_t lo = (static_cast<uint32_t>(hb * QW + l16) * static_cast<uint32_t>(a.ld_o) + dbase) * 2u;
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          char* dst = ob + lo + pp * 64;
          if (a.nt_o)
            __builtin_nontemporal_store(__builtin_bit_cast(f32x4_t, ow[pp]), reinterpret_cast<f32x4_t*>(dst));
          else
            *reinterpret_cast<uint4*>(dst) = ow[pp];
        }
        if (a.lse && g4 == 0)
          a.lse[(row0 + hb * QW + l16) * a.H + h] = LN2 * (m_run[hb] * SC + __builtin_amdgcn_logf(ltot) - (FULL ? 0.f : w_i[hb]));
      }
    }
  }
}

// ------------------------------------------------------------------ f32 kernel
// One wave per (row, head); lane d owns output dimension d (dh <= 64).  The bias is the
// literal -sp|p_i - p_j| - st|tau_i - tau_j| and the mask the literal predicate.
struct AttnF32Args {
  const int32_t* offsets;
  const int64_t* ts;
  const int64_t* req;
  const float* q;
  const float* k;
  const float* v;
  int64_t ld_qkv;
  float* o;
  int64_t ld_o;
  float* lse;
  float sp[GENRANK_MAX_HEADS];
  float st[GENRANK_MAX_HEADS];
  float scale;
  int B, m, H, dh;
  int64_t T_h;
  int flags;
  const int64_t* tb;
  int n_tb;
};

__global__ void __launch_bounds__(64) attn_fwd_f32_kernel(AttnF32Args a) {
  const int64_t row = blockIdx.x;
  const int h = blockIdx.y;
  const int lane = threadIdx.x;
  int u, i;
  if (row < a.T_h) {
    u = find_user(a.offsets, a.B, row);
    i = static_cast<int>(row - a.offsets[u]);
  } else {
    const int64_t c = row - a.T_h;
    u = static_cast<int>(c / a.m);
    i = static_cast<int>(c - static_cast<int64_t>(u) * a.m);
  }
  const int64_t off = a.offsets[u];
  const int N = a.offsets[u + 1] - a.offsets[u];
  if (row >= a.T_h) i += N;  // candidate sequence slot
  const int L = N + a.m;
  const int64_t t0 = (N > 0) ? a.ts[off] : a.req[u];
  auto slot_row = [&](int j) -> int64_t {
    return (j < N) ? off + j : a.T_h + static_cast<int64_t>(u) * a.m + (j - N);
  };
  auto slot_pos = [&](int j) -> int { return (j < N) ? j : N; };
  auto slot_tau = [&](int j) -> int64_t { return ((j < N) ? a.ts[off + j] : a.req[u]) - t0; };

  const bool act = lane < a.dh;
  const float qd = act ? a.q[row * a.ld_qkv + h * a.dh + lane] : 0.f;
  const int pi = slot_pos(i);
  const int64_t ti = slot_tau(i);
  float mx = -INFINITY, l = 0.f, acc = 0.f;
  const bool full = (a.flags & GENRANK_ATTN_FULL_HISTORY) != 0;
  const bool tbk = (a.flags & GENRANK_ATTN_TIME_BUCKET) != 0;
  for (int j = 0; j < L; ++j) {
    if (!attn_allowed(i, j, N, full)) continue;
    const int64_t kr = slot_row(j);
    float dot = act ? qd * a.k[kr * a.ld_qkv + h * a.dh + lane] : 0.f;
    for (int off2 = 32; off2 > 0; off2 >>= 1) dot += __shfl_xor(dot, off2);
    const int64_t gap = ti > slot_tau(j) ? ti - slot_tau(j) : slot_tau(j) - ti;
    const float dt = tbk ? static_cast<float>(bucket_search_global(a.tb, a.n_tb, gap)) : static_cast<float>(gap);
    const float s = dot * a.scale - a.sp[h] * fabsf(static_cast<float>(pi - slot_pos(j))) - a.st[h] * dt;
    const float m_new = fmaxf(mx, s);
    const float c = expf(mx - m_new);
    const float p = expf(s - m_new);
    l = l * c + p;
    acc = acc * c + p * (act ? a.v[kr * a.ld_qkv + h * a.dh + lane] : 0.f);
    mx = m_new;
  }
  if (act) a.o[row * a.ld_o + h * a.dh + lane] = acc / l;
  if (a.lse && lane == 0) a.lse[row * a.H + h] = mx + logf(l);
}

__global__ void debug_mask_kernel(const int32_t* offsets, int m, int user, int L_cap, uint8_t* out) {
  const int N = offsets[user + 1] - offsets[user];
  const int L = N + m;
  const int64_t n = static_cast<int64_t>(L_cap) * L_cap;
  for (int64_t e = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; e < n;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int i = static_cast<int>(e / L_cap), j = static_cast<int>(e % L_cap);
    out[e] = (i < L && j < L && attn_allowed(i, j, N)) ? 1 : 0;
  }
}

}  // namespace

genrank_status check_attn_args(const genrank_batch* b, const int32_t* offsets, const int64_t* ts,
                               const int64_t* req, genrank_alibi alibi, const void* q,
                               const void* k, const void* v, int64_t ld_qkv, const void* o,
                               int64_t ld_o) {
  if (!b) return GENRANK_E_ARG;
  genrank_status s = check_batch(b);
  if (s != GENRANK_OK) return s;
  if (!offsets || !req || !alibi.slopes_pos || !alibi.slopes_time) return GENRANK_E_ARG;
  {
    const genrank_status vs = check_alibi_variant(alibi, b->H);
    if (vs != GENRANK_OK) return vs;
  }
  if (b->total_hist > 0 && !ts) return GENRANK_E_ARG;
  if (!q || !k || !v || !o) return GENRANK_E_ARG;
  if (ld_qkv < b->d || ld_o < b->d) return GENRANK_E_SHAPE;
  if (b->dtype == GENRANK_BF16) {
    if (b->dh != DH) return GENRANK_E_SHAPE;
    if (ld_qkv % 8 || ld_o % 4) return GENRANK_E_SHAPE;
    // the kernel addresses one user's K/V rows with 32-bit buffer offsets
    if ((static_cast<int64_t>(b->max_hist) + AK) * ld_qkv * 2 >= (int64_t{1} << 31)) return GENRANK_E_SHAPE;
    if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
         reinterpret_cast<uintptr_t>(v)) % 16 || reinterpret_cast<uintptr_t>(o) % 8)
      return GENRANK_E_ARG;
  } else if (b->dh > 64) {
    return GENRANK_E_SHAPE;
  }
  return GENRANK_OK;
}

genrank_status launch_hstu_attn_fwd(const genrank_batch* b, const int32_t* offsets, const void* rab,
                                    const int64_t* rab_off, const void* q, const void* k,
                                    const void* v, int64_t ld_qkv, void* o, int64_t ld_o, float* lse,
                                    hipStream_t stream) {
  if (b->dtype != GENRANK_BF16) return GENRANK_E_DTYPE;
  if (b->dh != DH || ld_qkv < b->d || ld_o < b->d || ld_qkv % 8 || ld_o % 4) return GENRANK_E_SHAPE;
  if ((2 * static_cast<int64_t>(b->max_hist) + AK) * ld_qkv * 2 >= (int64_t{1} << 31)) return GENRANK_E_SHAPE;
  const int64_t Lmax = 2 * static_cast<int64_t>(b->max_hist) + b->m;
  if (Lmax * ((Lmax + 7) & ~int64_t{7}) * 2 >= (int64_t{1} << 32)) return GENRANK_E_SHAPE;
  const int64_t T = 2 * b->total_hist + static_cast<int64_t>(b->B) * b->m;
  if (T == 0) return GENRANK_OK;
  AttnArgs a{};
  a.offsets = offsets;
  a.q = static_cast<const bf16_t*>(q);
  a.k = static_cast<const bf16_t*>(k);
  a.v = static_cast<const bf16_t*>(v);
  a.ld_qkv = ld_qkv;
  a.o = static_cast<bf16_t*>(o);
  a.ld_o = ld_o;
  a.lse = lse;
  a.scale2 = LOG2E / sqrtf(static_cast<float>(b->dh));
  a.B = b->B; a.m = b->m; a.H = b->H;
  a.hist_tiles = static_cast<int>((2 * static_cast<int64_t>(b->max_hist) + AQ - 1) / AQ);
  a.cand_tiles = (b->m + AQ - 1) / AQ;
  a.T_h = 2 * b->total_hist;
  a.kh = a.k; a.vh = a.v; a.ld_h = ld_qkv; a.crow0 = a.T_h;
  a.rab = static_cast<const bf16_t*>(rab);
  a.rab_off = rab_off;
  if (a.hist_tiles + a.cand_tiles == 0) return GENRANK_OK;
  const int64_t pairs = (static_cast<int64_t>(b->B) * b->H + 8 * GROUP - 1) / (8 * GROUP) * (8 * GROUP);
  const int64_t G = pairs * (a.hist_tiles + a.cand_tiles);
  if (G > INT32_MAX) return GENRANK_E_SHAPE;
  hipLaunchKernelGGL(attn_fwd_rab_kernel, dim3(static_cast<unsigned>(G)), dim3(NT), 0, stream, a);
  GR_CHECK_LAUNCH();
  return GENRANK_OK;
}

// the instantiation for the ALiBi variant flags, and the bucket edges' fields
void set_variant(AttnArgs& a, const genrank_alibi& alibi) {
  a.tb = alibi.time_bounds;
  a.n_tb = (alibi.flags & GENRANK_ATTN_TIME_BUCKET) ? alibi.n_time_bounds : 0;
  a.tb_p2 = bucket_p2(a.n_tb);
}
// Batches whose longest history fits in LDS take the pair kernel (one workgroup per
// (user, head)); longer histories, and outputs not 16-byte aligned row by row, the ring
// kernel over the tile grid.
void launch_bf16_variant(int flags, int max_hist, dim3 grid, hipStream_t stream, const AttnArgs& a) {
  const int var = ((flags & GENRANK_ATTN_FULL_HISTORY) ? VAR_FULL : 0) |
                  ((flags & GENRANK_ATTN_TIME_BUCKET) ? VAR_TBUCKET : 0);
  // the pair kernel's epilogue stores 16-byte runs of an output row: o and its rows 16-byte aligned
  const bool o16 = reinterpret_cast<uintptr_t>(a.o) % 16 == 0 && a.ld_o % 8 == 0;
  if (max_hist <= PAIR_MAXK && o16) {
    const dim3 pg(static_cast<unsigned>(a.B * a.H));
    switch (var) {
      case 0: hipLaunchKernelGGL((attn_fwd_pair_kernel<0>), pg, dim3(PAIR_NT), 0, stream, a); break;
      case 1: hipLaunchKernelGGL((attn_fwd_pair_kernel<1>), pg, dim3(PAIR_NT), 0, stream, a); break;
      case 2: hipLaunchKernelGGL((attn_fwd_pair_kernel<2>), pg, dim3(PAIR_NT), 0, stream, a); break;
      default: hipLaunchKernelGGL((attn_fwd_pair_kernel<3>), pg, dim3(PAIR_NT), 0, stream, a); break;
    }
    return;
  }
  switch (var) {
    case 0: hipLaunchKernelGGL((attn_fwd_ring_kernel<0>), grid, dim3(NT), 0, stream, a); break;
    case 1: hipLaunchKernelGGL((attn_fwd_ring_kernel<1>), grid, dim3(NT), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((attn_fwd_ring_kernel<2>), grid, dim3(NT), 0, stream, a); break;
    default: hipLaunchKernelGGL((attn_fwd_ring_kernel<3>), grid, dim3(NT), 0, stream, a); break;
  }
}

genrank_status launch_attn_fwd(const genrank_batch* b, const int32_t* offsets, const int64_t* ts,
                               const int64_t* req, genrank_alibi alibi, const void* q,
                               const void* k, const void* v, int64_t ld_qkv, void* o,
                               int64_t ld_o, float* lse, hipStream_t stream) {
  const int64_t T = b->total_hist + static_cast<int64_t>(b->B) * b->m;
  if (T == 0) return GENRANK_OK;
  if (b->dtype == GENRANK_BF16) {
    AttnArgs a{};
    a.offsets = offsets; a.ts = ts; a.req = req;
    a.q = static_cast<const bf16_t*>(q);
    a.k = static_cast<const bf16_t*>(k);
    a.v = static_cast<const bf16_t*>(v);
    a.ld_qkv = ld_qkv;
    a.o = static_cast<bf16_t*>(o);
    a.ld_o = ld_o;
    a.nt_o = T * b->d * 2 > (int64_t(256) << 20);  // streaming stores for o beyond the last-level cache
    a.err = device_error_word();
    a.order = b->total_hist != static_cast<int64_t>(b->B) * b->max_hist;
    a.lse = lse;
    for (int h = 0; h < b->H; ++h) {
      a.sp2[h] = alibi.slopes_pos[h] * LOG2E;
      a.st2[h] = alibi.slopes_time[h] * LOG2E;
    }
    a.scale2 = LOG2E / sqrtf(static_cast<float>(b->dh));
    a.rscale2 = sqrtf(static_cast<float>(b->dh)) / LOG2E;
    a.B = b->B; a.m = b->m; a.H = b->H;
    a.hist_tiles = (b->max_hist + AQ - 1) / AQ;
    a.cand_tiles = (b->m + AQ - 1) / AQ;
    a.T_h = b->total_hist;
    a.kh = a.k; a.vh = a.v; a.ld_h = ld_qkv; a.crow0 = a.T_h;
    if (a.hist_tiles + a.cand_tiles == 0) return GENRANK_OK;
    const int64_t pairs = (static_cast<int64_t>(b->B) * b->H + 8 * GROUP - 1) / (8 * GROUP) * (8 * GROUP);
    const int64_t G = pairs * (a.hist_tiles + a.cand_tiles);
    if (G > INT32_MAX) return GENRANK_E_SHAPE;
    set_variant(a, alibi);
    launch_bf16_variant(alibi.flags, b->max_hist, dim3(static_cast<unsigned>(G)), stream, a);
  } else {
    AttnF32Args a{};
    a.offsets = offsets; a.ts = ts; a.req = req;
    a.q = static_cast<const float*>(q);
    a.k = static_cast<const float*>(k);
    a.v = static_cast<const float*>(v);
    a.ld_qkv = ld_qkv;
    a.o = static_cast<float*>(o);
    a.ld_o = ld_o;
    a.lse = lse;
    for (int h = 0; h < b->H; ++h) {
      a.sp[h] = alibi.slopes_pos[h];
      a.st[h] = alibi.slopes_time[h];
    }
    a.scale = 1.f / sqrtf(static_cast<float>(b->dh));
    a.B = b->B; a.m = b->m; a.H = b->H; a.dh = b->dh;
    a.T_h = b->total_hist;
    a.flags = alibi.flags;
    a.tb = alibi.time_bounds;
    a.n_tb = (alibi.flags & GENRANK_ATTN_TIME_BUCKET) ? alibi.n_time_bounds : 0;
    hipLaunchKernelGGL(attn_fwd_f32_kernel, dim3(static_cast<unsigned>(T), b->H), dim3(64), 0,
                       stream, a);
  }
  GR_CHECK_LAUNCH();
  return GENRANK_OK;
}

genrank_status launch_attn_fwd_cached(const genrank_batch* b, const int32_t* offsets, const int64_t* ts,
                                      const int64_t* req, genrank_alibi alibi, const void* q, const void* k,
                                      const void* v, int64_t ld_c, const void* kh, const void* vh, int64_t ld_h,
                                      void* o, int64_t ld_o, float* lse, hipStream_t stream) {
  if (b->m == 0) return GENRANK_OK;
  AttnArgs a{};
  a.offsets = offsets; a.ts = ts; a.req = req;
  a.q = static_cast<const bf16_t*>(q);
  a.k = static_cast<const bf16_t*>(k);
  a.v = static_cast<const bf16_t*>(v);
  a.ld_qkv = ld_c;
  a.o = static_cast<bf16_t*>(o);
  a.ld_o = ld_o;
  a.lse = lse;
  for (int h = 0; h < b->H; ++h) {
    a.sp2[h] = alibi.slopes_pos[h] * LOG2E;
    a.st2[h] = alibi.slopes_time[h] * LOG2E;
  }
  a.scale2 = LOG2E / sqrtf(static_cast<float>(b->dh));
  a.rscale2 = sqrtf(static_cast<float>(b->dh)) / LOG2E;
  a.B = b->B; a.m = b->m; a.H = b->H;
  a.hist_tiles = 0;  // candidate tiles only: history queries were answered earlier
  a.cand_tiles = (b->m + AQ - 1) / AQ;
  a.T_h = b->total_hist;
  a.kh = static_cast<const bf16_t*>(kh); a.vh = static_cast<const bf16_t*>(vh); a.ld_h = ld_h;
  a.crow0 = 0;
  const int64_t pairs = (static_cast<int64_t>(b->B) * b->H + 8 * GROUP - 1) / (8 * GROUP) * (8 * GROUP);
  const int64_t G = pairs * a.cand_tiles;
  if (G > INT32_MAX) return GENRANK_E_SHAPE;
  set_variant(a, alibi);
  a.err = device_error_word();
  // The ring kernel: each 128-candidate tile streams its user's history.  The pair kernel,
  // which loads a history once for all of a user's candidates, measured slower here (342
  // against 329 us at 512 users x 256 candidates x 480 keys, d = 512): with no history
  // queries to share the load, its one workgroup per CU waits on it.  The variant instance
  // matches the full forward's, and candidate rows get the same bits from both kernels.
  launch_bf16_variant(alibi.flags, INT32_MAX, dim3(static_cast<unsigned>(G)), stream, a);
  GR_CHECK_LAUNCH();
  return GENRANK_OK;
}

genrank_status launch_debug_mask(const int32_t* offsets, int m, int user, int L_cap, uint8_t* out,
                                 hipStream_t stream) {
  hipLaunchKernelGGL(debug_mask_kernel, dim3(256), dim3(256), 0, stream, offsets, m, user, L_cap, out);
  GR_CHECK_LAUNCH();
  return GENRANK_OK;
}

}  // namespace genrank
