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
// bf16 kernel (dh = 64).  One workgroup = 4 waves = 64 query rows of one (user, head):
// either a 64-row history tile (keys: history tiles up to and including the diagonal) or
// a 64-row candidate tile (keys: every history tile, plus each candidate's own key, which
// seeds the online softmax so the m x m candidate block is never formed).
//   S^T = K Q^T with v_mfma_f32_16x16x32_bf16: K rows from LDS are the row operand, the
//         wave's 16 queries (registers) the column operand.  Each lane then holds 16
//         scores of ONE query, so row max / row sum need only two cross-lane steps.
//   O^T = V^T P^T: P^T goes from the score registers straight into the column operand;
//         V is stored transposed in LDS with its keys permuted to match that register
//         order, so each lane's row-operand fragment is one 16-byte LDS read.
// K/V tiles are double-buffered in LDS and the next tile is fetched into registers while
// the current one is multiplied.  Workgroups of one (user, head) share an XCD (the grid's
// x dimension is a multiple of 8), so their K/V reuse hits one L2.
#include <math.h>

#include "common.hpp"
#include "internal.hpp"

namespace genrank {

namespace {

constexpr int AQ = 64;          // queries per workgroup
constexpr int AK = 64;          // keys per tile
constexpr int DH = 64;          // head dim of the bf16 kernel
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
  int B, m, H, hist_tiles, cand_tiles;
  int64_t T_h;
};

// slot of key j (0..63 in a tile) in the permuted key axis of sVt
__device__ __forceinline__ int vt_slot(int j) {
  const int ks = j >> 5, r = j & 31;
  const int hi = r >> 4, rr = r & 15;
  return ks * 32 + (rr >> 2) * 8 + hi * 4 + (rr & 3);
}

__global__ void __launch_bounds__(256) attn_fwd_bf16_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) bf16_t sK[2][AK * KLD];
  __shared__ __attribute__((aligned(16))) bf16_t sVt[2][DH * VLD];
  __shared__ __attribute__((aligned(16))) float sW[WCHUNK];

  const int u = blockIdx.x / a.H;
  const int h = blockIdx.x - u * a.H;
  const int y = blockIdx.y;
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
    qrow0 = a.T_h + static_cast<int64_t>(u) * a.m + q0;
    n_tiles = (N + AK - 1) / AK;
  } else {
    is_cand = false;
    const int t = a.hist_tiles - 1 - (y - a.cand_tiles);  // largest tiles first
    q0 = t * AQ;
    if (q0 >= N) return;
    nq = min(AQ, N - q0);
    qrow0 = off + q0;
    n_tiles = t + 1;
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int l16 = lane & 15, g4 = lane >> 4;
  const float sp2 = a.sp2[h], st2 = a.st2[h];
  // bias reference point: the candidates' shared (p, tau), or the tile's first query
  const int p_ref = is_cand ? N : q0;
  const int64_t ts_ref = is_cand ? a.req[u] : a.ts[off + q0];

  // ---- per-key bias terms w_j = sp (p_j - p_ref) + st (tau_j - tau_ref) for keys
  // [wbase, wbase + WCHUNK); keys past the history end get 0 (they are masked).  The time
  // difference is below 2^24 s, so it converts exactly through int32.
  auto load_w = [&](int wbase) {
    for (int j = tid; j < WCHUNK; j += 256) {
      const int key = wbase + j;
      float w = 0.f;
      if (key < N) {
        w = sp2 * static_cast<float>(key - p_ref) +
            st2 * static_cast<float>(static_cast<int32_t>(a.ts[off + key] - ts_ref));
      }
      sW[j] = w;
    }
  };
  if (n_tiles > 0) load_w(0);

  // ---- this lane's query (column of S^T / O^T)
  const int qi_local = wave * 16 + l16;       // 0..63 within the tile
  const bool q_valid = qi_local < nq;
  const int64_t qrow = qrow0 + qi_local;
  const int q_slot = is_cand ? (N + q0 + qi_local) : (q0 + qi_local);  // sequence slot
  // lanes past the tile's last query read that query's row (never stored)
  const int64_t qrow_ld = qrow0 + min(qi_local, nq - 1);
  bf16x8_t qf[2];
  {
    const bf16_t* qp = a.q + qrow_ld * a.ld_qkv + h * DH + g4 * 8;
    qf[0] = as_bf16x8(*reinterpret_cast<const uint4*>(qp));
    qf[1] = as_bf16x8(*reinterpret_cast<const uint4*>(qp + 32));
  }

  f32x4_t accO[4];
  float m2, lsum;
  if (is_cand) {
    // seed with the candidate's own key: bias 0 (same position and time as p_ref)
    float dot = 0.f;
    {
      const bf16_t* kp = a.k + qrow_ld * a.ld_qkv + h * DH + g4 * 8;
      float kf[8], qv[8];
      uint4 kk = *reinterpret_cast<const uint4*>(kp);
      unpack8(kk, kf);
      unpack8(__builtin_bit_cast(uint4, qf[0]), qv);
#pragma unroll
      for (int e = 0; e < 8; ++e) dot += qv[e] * kf[e];
      kk = *reinterpret_cast<const uint4*>(kp + 32);
      unpack8(kk, kf);
      unpack8(__builtin_bit_cast(uint4, qf[1]), qv);
#pragma unroll
      for (int e = 0; e < 8; ++e) dot += qv[e] * kf[e];
    }
    dot += __shfl_xor(dot, 16);
    dot += __shfl_xor(dot, 32);
    m2 = dot * a.scale2;
    lsum = (g4 == 0) ? 1.f : 0.f;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const uint2 vv = *reinterpret_cast<const uint2*>(a.v + qrow_ld * a.ld_qkv + h * DH + nb * 16 + g4 * 4);
      accO[nb] = f32x4_t{__uint_as_float(vv.x << 16), __uint_as_float(vv.x & 0xFFFF0000u),
                         __uint_as_float(vv.y << 16), __uint_as_float(vv.y & 0xFFFF0000u)};
    }
  } else {
    m2 = -1e30f;
    lsum = 0.f;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) accO[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // ---- K/V tile staging.  Thread (pair p, chunk c) moves rows 2p and 2p+1, columns
  // 8c..8c+7, of both K and V: K rows go to sK as 16-byte writes; V goes to sVt
  // transposed, each 32-bit write holding the two keys' values of one column (adjacent
  // in the permuted key order).  Loads are buffer loads over the user's history rows:
  // the descriptor sits in scalar registers, the lane offset is loop-invariant and the
  // tile offset is scalar, and rows past the history end read as zero (the mask gives
  // those keys probability 0).
  const int pr = tid & 31;
  const int ch = tid >> 5;
  const int kA = 2 * pr, kB = 2 * pr + 1;
  const int d0 = ch * 8;
  const uint32_t row_bytes = static_cast<uint32_t>(a.ld_qkv) * 2u;
  const uint32_t hist_bytes = static_cast<uint32_t>(N) * row_bytes;
  const __amdgpu_buffer_rsrc_t rsK = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t*>(a.k + off * a.ld_qkv), static_cast<short>(0), hist_bytes, BUF_DWORD3);
  const __amdgpu_buffer_rsrc_t rsV = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t*>(a.v + off * a.ld_qkv), static_cast<short>(0), hist_bytes, BUF_DWORD3);
  const uint32_t voA = static_cast<uint32_t>(kA) * row_bytes + (h * DH + d0) * 2u;
  const uint32_t voB = voA + row_bytes;
  uint4 rka, rkb, rva, rvb;
  auto fetch = [&](int kt) {
    const uint32_t so = static_cast<uint32_t>(kt * AK) * row_bytes;
    rka = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsK, voA, so, 0));
    rkb = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsK, voB, so, 0));
    rva = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsV, voA, so, 0));
    rvb = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsV, voB, so, 0));
  };
  const int slotA = vt_slot(kA);  // slot(kB) == slotA + 1
  auto stash = [&](int buf) {
    *reinterpret_cast<uint4*>(&sK[buf][kA * KLD + d0]) = rka;
    *reinterpret_cast<uint4*>(&sK[buf][kB * KLD + d0]) = rkb;
    uint32_t* col = reinterpret_cast<uint32_t*>(&sVt[buf][d0 * VLD + slotA]);
    constexpr int P = VLD / 2;  // row pitch in 32-bit words
    col[0 * P] = __builtin_amdgcn_perm(rvb.x, rva.x, 0x05040100u);
    col[1 * P] = __builtin_amdgcn_perm(rvb.x, rva.x, 0x07060302u);
    col[2 * P] = __builtin_amdgcn_perm(rvb.y, rva.y, 0x05040100u);
    col[3 * P] = __builtin_amdgcn_perm(rvb.y, rva.y, 0x07060302u);
    col[4 * P] = __builtin_amdgcn_perm(rvb.z, rva.z, 0x05040100u);
    col[5 * P] = __builtin_amdgcn_perm(rvb.z, rva.z, 0x07060302u);
    col[6 * P] = __builtin_amdgcn_perm(rvb.w, rva.w, 0x05040100u);
    col[7 * P] = __builtin_amdgcn_perm(rvb.w, rva.w, 0x07060302u);
  };

  if (n_tiles > 0) {
    fetch(0);
    stash(0);
  }
  // The query fragments come straight from a global load.  Without this the compiler's
  // wait-count analysis cannot prove at the loop head that the load has landed and makes
  // every iteration wait for that iteration's K/V prefetch before its first MFMA.  An
  // empty asm that reads and redefines the registers makes it wait here, once.
  asm volatile("" : "+v"(qf[0]), "+v"(qf[1]));
  __syncthreads();

  int wbase = 0;
  for (int kt = 0; kt < n_tiles; ++kt) {
    const int buf = kt & 1;
    const int base = kt * AK;
    if (base >= wbase + WCHUNK) {  // histories longer than WCHUNK keys: next bias chunk
      __syncthreads();
      wbase += WCHUNK;
      load_w(wbase);
      __syncthreads();
    }
    if (kt + 1 < n_tiles) fetch(kt + 1);
    const bool diag = !is_cand && kt == n_tiles - 1;   // causal diagonal tile
    const bool ragged = base + AK > N;                  // keys past the history end
    const int kb_end = diag ? (wave + 1) : 4;           // key blocks this wave needs

    // S^T = K Q^T
    f32x4_t s[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      s[kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if (kb < kb_end) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const bf16x8_t kf = as_bf16x8(*reinterpret_cast<const uint4*>(
              &sK[buf][(kb * 16 + l16) * KLD + ks * 32 + g4 * 8]));
          s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[ks], s[kb], 0, 0, 0);
        }
      }
    }
    // scale + separable bias, mask, tile max
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const float4 w = *reinterpret_cast<const float4*>(&sW[base - wbase + kb * 16 + g4 * 4]);
      const float wv[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = s[kb][i] * a.scale2 + wv[i];
        if (kb >= kb_end) {
          v = -INFINITY;
        } else if (diag || ragged) {
          const int k_slot = base + kb * 16 + g4 * 4 + i;
          if (!(k_slot < N && attn_allowed(q_slot, k_slot, N))) v = -INFINITY;
        }
        s[kb][i] = v;
        mx = fmaxf(mx, v);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m2, mx);
    const float alpha = __builtin_amdgcn_exp2f(m2 - m_new);
    m2 = m_new;
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = __builtin_amdgcn_exp2f(s[kb][i] - m_new);
        s[kb][i] = p;
        psum += p;
      }
    lsum = lsum * alpha + psum;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) accO[nb][i] *= alpha;

    // P^T as the column operand: keys {4g..4g+3} of blocks 2ks and 2ks+1
    bf16x8_t pf[2];
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
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        if (ks * 2 >= kb_end) continue;
        const bf16x8_t vf = as_bf16x8(*reinterpret_cast<const uint4*>(
            &sVt[buf][(nb * 16 + l16) * VLD + ks * 32 + g4 * 8]));
        accO[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[ks], accO[nb], 0, 0, 0);
      }

    if (kt + 1 < n_tiles) stash(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue
  float ltot = lsum + __shfl_xor(lsum, 16);
  ltot += __shfl_xor(ltot, 32);
  if (!q_valid) return;
  const float inv = 1.f / ltot;
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    uint2 o;
    o.x = pack_bf16x2(accO[nb][0] * inv, accO[nb][1] * inv);
    o.y = pack_bf16x2(accO[nb][2] * inv, accO[nb][3] * inv);
    *reinterpret_cast<uint2*>(a.o + qrow * a.ld_o + h * DH + nb * 16 + g4 * 4) = o;
  }
  if (a.lse && g4 == 0) {
    float w_i = 0.f;
    if (!is_cand) {
      w_i = sp2 * static_cast<float>(q_slot - p_ref) +
            st2 * static_cast<float>(static_cast<int32_t>(a.ts[off + q_slot] - ts_ref));
    }
    a.lse[qrow * a.H + h] = LN2 * (m2 + log2f(ltot) - w_i);
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
  for (int j = 0; j < L; ++j) {
    if (!attn_allowed(i, j, N)) continue;
    const int64_t kr = slot_row(j);
    float dot = act ? qd * a.k[kr * a.ld_qkv + h * a.dh + lane] : 0.f;
    for (int off2 = 32; off2 > 0; off2 >>= 1) dot += __shfl_xor(dot, off2);
    const float s = dot * a.scale - a.sp[h] * fabsf(static_cast<float>(pi - slot_pos(j))) -
                    a.st[h] * fabsf(static_cast<float>(ti - slot_tau(j)));
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
  if (b->total_hist > 0 && !ts) return GENRANK_E_ARG;
  if (!q || !k || !v || !o) return GENRANK_E_ARG;
  if (ld_qkv < b->d || ld_o < b->d) return GENRANK_E_SHAPE;
  if (b->dtype == GENRANK_BF16) {
    if (b->dh != DH) return GENRANK_E_SHAPE;
    if (ld_qkv % 8 || ld_o % 4) return GENRANK_E_SHAPE;
    if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
         reinterpret_cast<uintptr_t>(v)) % 16 || reinterpret_cast<uintptr_t>(o) % 8)
      return GENRANK_E_ARG;
  } else if (b->dh > 64) {
    return GENRANK_E_SHAPE;
  }
  return GENRANK_OK;
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
    a.lse = lse;
    for (int h = 0; h < b->H; ++h) {
      a.sp2[h] = alibi.slopes_pos[h] * LOG2E;
      a.st2[h] = alibi.slopes_time[h] * LOG2E;
    }
    a.scale2 = LOG2E / sqrtf(static_cast<float>(b->dh));
    a.B = b->B; a.m = b->m; a.H = b->H;
    a.hist_tiles = (b->max_hist + AQ - 1) / AQ;
    a.cand_tiles = (b->m + AQ - 1) / AQ;
    a.T_h = b->total_hist;
    if (a.hist_tiles + a.cand_tiles == 0) return GENRANK_OK;
    dim3 grid(b->B * b->H, a.hist_tiles + a.cand_tiles);
    hipLaunchKernelGGL(attn_fwd_bf16_kernel, grid, dim3(256), 0, stream, a);
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
    hipLaunchKernelGGL(attn_fwd_f32_kernel, dim3(static_cast<unsigned>(T), b->H), dim3(64), 0,
                       stream, a);
  }
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
