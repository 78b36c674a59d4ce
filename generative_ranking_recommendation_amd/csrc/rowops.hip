// Row-wise pieces of the GenRank block and head: RMSNorm (+ backward),
// the per-candidate action head (+ backward), sigmoid BCE at candidate rows, fills.
// One wave per row; rows are read with 16-byte vector loads where the width allows.
#include <algorithm>

#include "common.hpp"
#include "internal.hpp"

namespace genrank {

namespace {

constexpr int RW = 256;  // threads per block (4 rows per block, one wave each)

__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

template <typename TI, typename TO>
__global__ void __launch_bounds__(RW) rmsnorm_kernel(const TI* __restrict__ x, const float* __restrict__ g,
                                                     TO* __restrict__ y, int64_t rows, int d) {
  const int64_t r = static_cast<int64_t>(blockIdx.x) * (RW / 64) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= rows) return;
  const TI* xr = x + r * d;
  float ss = 0.f;
  for (int c = lane; c < d; c += 64) {
    const float v = to_f32(xr[c]);
    ss += v * v;
  }
  ss = wave_sum(ss);
  const float inv = rsqrtf(ss / d + RMS_EPS);
  TO* yr = y + r * d;
  for (int c = lane; c < d; c += 64) yr[c] = from_f32<TO>(to_f32(xr[c]) * inv * g[c]);
}

// The same normalisation with x read once through 16-byte loads: a group of LPR lanes owns
// one row, each lane Q 16-byte chunks of it (chunk q of lane l at elements
// (q LPR + l) VEC ..), kept in registers between the sum of squares and the store; a wave
// takes 64 / LPR rows.  Each row's result depends only on its own elements.  TO may be
// narrower than TI (f32 rows normalised into bf16 operands): then each store is 8 bytes.
template <typename TI, typename TO, int LPR, int Q>
__global__ void __launch_bounds__(RW) rmsnorm_vec_kernel(const TI* __restrict__ x, const float* __restrict__ g,
                                                         TO* __restrict__ y, int64_t rows, int d) {
  constexpr int VEC = 16 / static_cast<int>(sizeof(TI));
  constexpr int RPW = 64 / LPR;
  const int lane = threadIdx.x & 63;
  const int li = lane % LPR;
  const int64_t r = (static_cast<int64_t>(blockIdx.x) * (RW / 64) + (threadIdx.x >> 6)) * RPW + lane / LPR;
  const int64_t rc = r < rows ? r : rows - 1;  // every lane takes part in the shuffles
  float v[Q][VEC];
  float ss = 0.f;
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const uint4 u = *reinterpret_cast<const uint4*>(x + rc * d + (q * LPR + li) * VEC);
    if constexpr (VEC == 8) {
      unpack8(u, v[q]);
    } else {
      v[q][0] = __uint_as_float(u.x); v[q][1] = __uint_as_float(u.y);
      v[q][2] = __uint_as_float(u.z); v[q][3] = __uint_as_float(u.w);
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) ss += v[q][e] * v[q][e];
  }
#pragma unroll
  for (int o = LPR / 2; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  const float inv = rsqrtf(ss / d + RMS_EPS);
  if (r >= rows) return;
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int c = (q * LPR + li) * VEC;
    float o[VEC];
#pragma unroll
    for (int e = 0; e < VEC; e += 4) {
      const float4 g4 = *reinterpret_cast<const float4*>(g + c + e);
      o[e] = v[q][e] * inv * g4.x;
      o[e + 1] = v[q][e + 1] * inv * g4.y;
      o[e + 2] = v[q][e + 2] * inv * g4.z;
      o[e + 3] = v[q][e + 3] * inv * g4.w;
    }
    if constexpr (VEC == 8) {
      *reinterpret_cast<uint4*>(y + r * d + c) = pack8(o);
    } else if constexpr (sizeof(TO) == 2) {
      *reinterpret_cast<uint2*>(y + r * d + c) = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
    } else {
      *reinterpret_cast<uint4*>(y + r * d + c) =
          make_uint4(__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]), __float_as_uint(o[3]));
    }
  }
}

// 4 consecutive elements as f32 (8-byte bf16 / 16-byte f32 accesses)
__device__ __forceinline__ void ld4(const bf16_t* p, float* f) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  f[0] = __uint_as_float(v.x << 16); f[1] = __uint_as_float(v.x & 0xFFFF0000u);
  f[2] = __uint_as_float(v.y << 16); f[3] = __uint_as_float(v.y & 0xFFFF0000u);
}
__device__ __forceinline__ void ld4(const float* p, float* f) {
  const float4 v = *reinterpret_cast<const float4*>(p);
  f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w;
}
__device__ __forceinline__ void st4(bf16_t* p, const float* f) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]));
}
__device__ __forceinline__ void st4(float* p, const float* f) {
  *reinterpret_cast<float4*>(p) = make_float4(f[0], f[1], f[2], f[3]);
}

// Parameter gradients (sums over rows) are formed without atomics: each wave keeps its
// partial in registers, the block adds its waves' partials in order through LDS and
// writes one partial row, and column_sum_kernel adds the blocks' rows in order.
constexpr int MAXQ = 4;           // 4-column groups per lane: d <= 64 * 4 * MAXQ = 1024
constexpr int PART_BLOCKS = 1024;  // rmsnorm backward blocks (partial rows)

// dx = r g dy - r^3 x sum(g dy x) / d  (+ add);  dg = sum over rows of dy x r.
// Lane l owns columns 4 l + 256 q; a wave takes two rows per step.
template <typename TX, typename T>
__global__ void __launch_bounds__(RW) rmsnorm_bwd_kernel(const TX* __restrict__ x, const float* __restrict__ g,
                                                         const T* dy, const T* add, T* dx,
                                                         float* __restrict__ part, int64_t rows, int d) {
  __shared__ float sp[RW / 64][64 * 4 * MAXQ];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t nw = static_cast<int64_t>(gridDim.x) * (RW / 64);
  float pg[MAXQ][4];
#pragma unroll
  for (int q = 0; q < MAXQ; ++q)
#pragma unroll
    for (int e = 0; e < 4; ++e) pg[q][e] = 0.f;
  for (int64_t r0 = static_cast<int64_t>(blockIdx.x) * (RW / 64) + wave; r0 < rows; r0 += 2 * nw) {
    float xv[2][MAXQ][4], gv[2][MAXQ][4], ss[2] = {0.f, 0.f}, dot[2] = {0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int64_t r = r0 + k * nw;
#pragma unroll
      for (int q = 0; q < MAXQ; ++q) {
        const int c = 4 * lane + 256 * q;
        if (r < rows && c < d) {
          ld4(x + r * d + c, xv[k][q]);
          ld4(dy + r * d + c, gv[k][q]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) xv[k][q][e] = gv[k][q][e] = 0.f;
        }
      }
    }
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int q = 0; q < MAXQ; ++q) {
        const int c = 4 * lane + 256 * q;
        if (c >= d) break;
        const float4 g4 = *reinterpret_cast<const float4*>(g + c);
        const float gg[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ss[k] += xv[k][q][e] * xv[k][q][e];
          dot[k] += gg[e] * gv[k][q][e] * xv[k][q][e];
        }
      }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int64_t r = r0 + k * nw;
      const float s2 = wave_sum(ss[k]), dt = wave_sum(dot[k]);
      if (r >= rows) continue;
      const float rr = rsqrtf(s2 / d + RMS_EPS);
      const float c3 = rr * rr * rr * dt / d;
#pragma unroll
      for (int q = 0; q < MAXQ; ++q) {
        const int c = 4 * lane + 256 * q;
        if (c >= d) break;
        const float4 g4 = *reinterpret_cast<const float4*>(g + c);
        const float gg[4] = {g4.x, g4.y, g4.z, g4.w};
        float o[4], ad[4] = {0.f, 0.f, 0.f, 0.f};
        if (add) ld4(add + r * d + c, ad);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o[e] = rr * gg[e] * gv[k][q][e] - c3 * xv[k][q][e] + ad[e];
          pg[q][e] += gv[k][q][e] * xv[k][q][e] * rr;
        }
        st4(dx + r * d + c, o);
      }
    }
  }
#pragma unroll
  for (int q = 0; q < MAXQ; ++q) {
    const int c = 4 * lane + 256 * q;
    if (c < d)
#pragma unroll
      for (int e = 0; e < 4; ++e) sp[wave][c + e] = pg[q][e];
  }
  __syncthreads();
  for (int c = threadIdx.x; c < d; c += RW)
    part[static_cast<int64_t>(blockIdx.x) * d + c] = ((sp[0][c] + sp[1][c]) + sp[2][c]) + sp[3][c];
}

// Column c's sum over b < nparts of part[b * width + c], b ascending, goes to out0[c] for
// c < n0, out1[c - n0] for c < n0 + n1, out2[c - n0 - n1] beyond.  Block: 16 columns x 16
// groups of partial rows; the groups' sums are added in order.
__global__ void __launch_bounds__(256) column_sum_kernel(const float* __restrict__ part, int nparts, int width,
                                                         float* __restrict__ out0, int n0,
                                                         float* __restrict__ out1, int n1,
                                                         float* __restrict__ out2) {
  __shared__ float sg[16][17];
  const int cl = threadIdx.x & 15, grp = threadIdx.x >> 4;
  const int c = blockIdx.x * 16 + cl;
  float acc = 0.f;
  if (c < width) {
    const int per = (nparts + 15) / 16;
    const int b0 = grp * per, b1 = min(nparts, b0 + per);
    int b = b0;
    for (; b + 4 <= b1; b += 4) {
      const float v0 = part[static_cast<int64_t>(b) * width + c];
      const float v1 = part[static_cast<int64_t>(b + 1) * width + c];
      const float v2 = part[static_cast<int64_t>(b + 2) * width + c];
      const float v3 = part[static_cast<int64_t>(b + 3) * width + c];
      acc = (((acc + v0) + v1) + v2) + v3;
    }
    for (; b < b1; ++b) acc += part[static_cast<int64_t>(b) * width + c];
  }
  sg[grp][cl] = acc;
  __syncthreads();
  if (grp == 0 && c < width) {
    float t = 0.f;
    for (int k = 0; k < 16; ++k) t += sg[k][cl];
    if (c < n0)
      out0[c] = t;
    else if (c < n0 + n1)
      out1[c - n0] = t;
    else
      out2[c - n0 - n1] = t;
  }
}

__global__ void fill_f32_kernel(float* p, int64_t n, float v) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = v;
}

__global__ void fill_u16_kernel(uint16_t* p, int64_t n) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = 0;
}

// logits[c, t] = rmsnorm(x_c) g . w[t] + b[t] for row c = row0 + r, or idx[r] when a row
// list is given
template <typename T>
__global__ void __launch_bounds__(RW) head_fwd_kernel(const T* __restrict__ x, int64_t row0, int64_t rows,
                                                      const int32_t* __restrict__ idx, int d,
                                                      const float* __restrict__ g,
                                                      const float* __restrict__ w,
                                                      const float* __restrict__ b, int nt,
                                                      float* __restrict__ logits) {
  const int64_t r = static_cast<int64_t>(blockIdx.x) * (RW / 64) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= rows) return;
  const T* xr = x + (idx ? static_cast<int64_t>(idx[r]) : row0 + r) * d;
  float ss = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int c = lane; c < d; c += 64) {
    const float v = to_f32(xr[c]);
    ss += v * v;
    const float vg = v * g[c];
#pragma unroll
    for (int t = 0; t < 8; ++t)
      if (t < nt) acc[t] += vg * w[t * d + c];
  }
  ss = wave_sum(ss);
  const float inv = rsqrtf(ss / d + RMS_EPS);
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    if (t >= nt) break;
    const float s = wave_sum(acc[t]);
    if (lane == 0) logits[r * nt + t] = s * inv + b[t];
  }
}

// RMSNorm backward with rows read through 16-byte loads (lane groups as rmsnorm_vec_kernel,
// two rows per group in flight): dx = r g dy - r^3 x sum(g dy x) / d (+ add), and the
// block's partial row of dg = sum over rows of dy x r.  The groups of a wave add their dg
// partials by xor-shuffles, the block's waves in order through LDS: a fixed order.  x may be
// wider than the gradients (f32 residual rows, bf16 gradients): it is then read in two pieces.
template <typename TX, typename T, int LPR, int Q>
__global__ void __launch_bounds__(RW) rmsnorm_bwd_vec_kernel(const TX* __restrict__ x, const float* __restrict__ g,
                                                             const T* dy, const T* add, T* dx,
                                                             float* __restrict__ part, int64_t rows, int d) {
  constexpr int VEC = 16 / static_cast<int>(sizeof(T));
  constexpr int RPW = 64 / LPR;
  constexpr int UR = 2;
  __shared__ float sp[RW / 64][64 * Q * VEC];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane % LPR;
  const int64_t ngroups = static_cast<int64_t>(gridDim.x) * (RW / 64) * RPW;
  const int64_t gid = (static_cast<int64_t>(blockIdx.x) * (RW / 64) + wave) * RPW + lane / LPR;
  auto load = [](const T* p, float* f) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    if constexpr (VEC == 8) {
      unpack8(u, f);
    } else {
      f[0] = __uint_as_float(u.x); f[1] = __uint_as_float(u.y);
      f[2] = __uint_as_float(u.z); f[3] = __uint_as_float(u.w);
    }
  };
  float pg[Q][VEC];
#pragma unroll
  for (int q = 0; q < Q; ++q)
#pragma unroll
    for (int e = 0; e < VEC; ++e) pg[q][e] = 0.f;
  for (int64_t r0 = gid; r0 < rows; r0 += UR * ngroups) {
    float xv[UR][Q][VEC], gv[UR][Q][VEC], ss[UR], dot[UR];
#pragma unroll
    for (int k = 0; k < UR; ++k) {
      const int64_t r = min(r0 + k * ngroups, rows - 1);  // every lane takes part in the shuffles
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const int c = (q * LPR + li) * VEC;
        if constexpr (sizeof(TX) == sizeof(T)) {
          load(x + r * d + c, xv[k][q]);
        } else {  // VEC = 8 f32 values: two 16-byte loads
          const float4 a0 = *reinterpret_cast<const float4*>(x + r * d + c);
          const float4 a1 = *reinterpret_cast<const float4*>(x + r * d + c + 4);
          xv[k][q][0] = a0.x; xv[k][q][1] = a0.y; xv[k][q][2] = a0.z; xv[k][q][3] = a0.w;
          xv[k][q][4] = a1.x; xv[k][q][5] = a1.y; xv[k][q][6] = a1.z; xv[k][q][7] = a1.w;
        }
        load(dy + r * d + c, gv[k][q]);
      }
    }
#pragma unroll
    for (int k = 0; k < UR; ++k) {
      ss[k] = 0.f;
      dot[k] = 0.f;
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const int c = (q * LPR + li) * VEC;
#pragma unroll
        for (int e = 0; e < VEC; e += 4) {
          const float4 g4 = *reinterpret_cast<const float4*>(g + c + e);
          const float gg[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            ss[k] += xv[k][q][e + i] * xv[k][q][e + i];
            dot[k] += gg[i] * gv[k][q][e + i] * xv[k][q][e + i];
          }
        }
      }
#pragma unroll
      for (int o = LPR / 2; o > 0; o >>= 1) {
        ss[k] += __shfl_xor(ss[k], o);
        dot[k] += __shfl_xor(dot[k], o);
      }
    }
#pragma unroll
    for (int k = 0; k < UR; ++k) {
      const int64_t r = r0 + k * ngroups;
      if (r >= rows) continue;
      const float rr = rsqrtf(ss[k] / d + RMS_EPS);
      const float c3 = rr * rr * rr * dot[k] / d;
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const int c = (q * LPR + li) * VEC;
        float ad[VEC], o[VEC];
        if (add) {
          load(add + r * d + c, ad);
        } else {
#pragma unroll
          for (int e = 0; e < VEC; ++e) ad[e] = 0.f;
        }
#pragma unroll
        for (int e = 0; e < VEC; e += 4) {
          const float4 g4 = *reinterpret_cast<const float4*>(g + c + e);
          const float gg[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            o[e + i] = rr * gg[i] * gv[k][q][e + i] - c3 * xv[k][q][e + i] + ad[e + i];
            pg[q][e + i] += gv[k][q][e + i] * xv[k][q][e + i] * rr;
          }
        }
        uint4 u;
        if constexpr (VEC == 8) {
          u = pack8(o);
        } else {
          u = make_uint4(__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]), __float_as_uint(o[3]));
        }
        *reinterpret_cast<uint4*>(dx + r * d + c) = u;
      }
    }
  }
  // the wave's groups hold the same columns: add them, then the waves in order
#pragma unroll
  for (int q = 0; q < Q; ++q)
#pragma unroll
    for (int e = 0; e < VEC; ++e)
#pragma unroll
      for (int o = LPR; o < 64; o <<= 1) pg[q][e] += __shfl_xor(pg[q][e], o);
  if (lane < LPR) {
#pragma unroll
    for (int q = 0; q < Q; ++q)
#pragma unroll
      for (int e = 0; e < VEC; ++e) sp[wave][(q * LPR + li) * VEC + e] = pg[q][e];
  }
  __syncthreads();
  for (int c = threadIdx.x; c < d; c += RW)
    part[static_cast<int64_t>(blockIdx.x) * d + c] = ((sp[0][c] + sp[1][c]) + sp[2][c]) + sp[3][c];
}

// The head with rows read once through 16-byte loads, laid out as rmsnorm_vec_kernel: a
// group of LPR lanes per row, Q 16-byte chunks per lane; the sum of squares and the nt
// dot products are reduced within the group.
template <typename T, int LPR, int Q>
__global__ void __launch_bounds__(RW) head_fwd_vec_kernel(const T* __restrict__ x, int64_t row0, int64_t rows,
                                                          const int32_t* __restrict__ idx, int d,
                                                          const float* __restrict__ g,
                                                          const float* __restrict__ w,
                                                          const float* __restrict__ b, int nt,
                                                          float* __restrict__ logits) {
  constexpr int VEC = 16 / static_cast<int>(sizeof(T));
  constexpr int RPW = 64 / LPR;
  const int lane = threadIdx.x & 63;
  const int li = lane % LPR;
  const int64_t r = (static_cast<int64_t>(blockIdx.x) * (RW / 64) + (threadIdx.x >> 6)) * RPW + lane / LPR;
  const int64_t rc = r < rows ? r : rows - 1;  // every lane takes part in the shuffles
  const T* xr = x + (idx ? static_cast<int64_t>(idx[rc]) : row0 + rc) * d;
  float ss = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int c = (q * LPR + li) * VEC;
    const uint4 u = *reinterpret_cast<const uint4*>(xr + c);
    float v[VEC];
    if constexpr (VEC == 8) {
      unpack8(u, v);
    } else {
      v[0] = __uint_as_float(u.x); v[1] = __uint_as_float(u.y);
      v[2] = __uint_as_float(u.z); v[3] = __uint_as_float(u.w);
    }
#pragma unroll
    for (int e = 0; e < VEC; e += 4) {
      const float4 g4 = *reinterpret_cast<const float4*>(g + c + e);
      const float vg[4] = {v[e] * g4.x, v[e + 1] * g4.y, v[e + 2] * g4.z, v[e + 3] * g4.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) ss += v[e + k] * v[e + k];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        if (t >= nt) break;
        const float4 w4 = *reinterpret_cast<const float4*>(w + t * d + c + e);
        acc[t] += vg[0] * w4.x + vg[1] * w4.y + vg[2] * w4.z + vg[3] * w4.w;
      }
    }
  }
#pragma unroll
  for (int o = LPR / 2; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    if (t >= nt) break;
#pragma unroll
    for (int o = LPR / 2; o > 0; o >>= 1) acc[t] += __shfl_xor(acc[t], o);
  }
  const float inv = rsqrtf(ss / d + RMS_EPS);
  if (r >= rows || li != 0) return;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    if (t >= nt) break;
    logits[r * nt + t] = acc[t] * inv + b[t];
  }
}

// z = rmsnorm(x) g; dz = dlogits . w; dx by the RMSNorm backward with dz as the output
// gradient; dw[t] = sum dlogits[t] z; db[t] = sum dlogits[t]; dg = sum dz x r.  One wave per
// row (grid stride), lane l owning columns 4 l + 256 q; the block's waves add their
// parameter partials in order through LDS into one partial row
// [dg (d) | dw (nt d) | db (nt)], summed over blocks by column_sum_kernel.
constexpr int HEAD_BLOCKS = 64;

template <typename TX, typename T>
__global__ void __launch_bounds__(RW) head_bwd_kernel(const TX* __restrict__ x, int64_t row0, int64_t rows,
                                                      const int32_t* __restrict__ idx, int d,
                                                      const float* __restrict__ g,
                                                      const float* __restrict__ w, int nt,
                                                      const float* __restrict__ dl, T* __restrict__ dx,
                                                      float* __restrict__ part) {
  __shared__ float sp[64 * 4 * MAXQ * 5 + 4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t nw = static_cast<int64_t>(gridDim.x) * (RW / 64);
  const int width = d * (1 + nt) + nt;
  float pg[MAXQ][4], pw[4][MAXQ][4], pb[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int q = 0; q < MAXQ; ++q)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      pg[q][e] = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t) pw[t][q][e] = 0.f;
    }
  for (int64_t r = static_cast<int64_t>(blockIdx.x) * (RW / 64) + wave; r < rows; r += nw) {
    const int64_t xrow = idx ? static_cast<int64_t>(idx[r]) : row0 + r;
    const TX* xr = x + xrow * d;
    float dlr[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) dlr[t] = (t < nt) ? dl[r * nt + t] : 0.f;
    float xv[MAXQ][4], dz[MAXQ][4], ss = 0.f, dot = 0.f;
#pragma unroll
    for (int q = 0; q < MAXQ; ++q) {
      const int c = 4 * lane + 256 * q;
#pragma unroll
      for (int e = 0; e < 4; ++e) xv[q][e] = dz[q][e] = 0.f;
      if (c >= d) continue;
      ld4(xr + c, xv[q]);
      const float4 g4 = *reinterpret_cast<const float4*>(g + c);
      const float gg[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if (t >= nt) break;
        const float4 w4 = *reinterpret_cast<const float4*>(w + t * d + c);
        dz[q][0] += dlr[t] * w4.x; dz[q][1] += dlr[t] * w4.y;
        dz[q][2] += dlr[t] * w4.z; dz[q][3] += dlr[t] * w4.w;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ss += xv[q][e] * xv[q][e];
        dot += gg[e] * dz[q][e] * xv[q][e];
      }
    }
    ss = wave_sum(ss);
    dot = wave_sum(dot);
    const float rr = rsqrtf(ss / d + RMS_EPS);
    const float c3 = rr * rr * rr * dot / d;
#pragma unroll
    for (int q = 0; q < MAXQ; ++q) {
      const int c = 4 * lane + 256 * q;
      if (c >= d) break;
      const float4 g4 = *reinterpret_cast<const float4*>(g + c);
      const float gg[4] = {g4.x, g4.y, g4.z, g4.w};
      float o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[e] = rr * gg[e] * dz[q][e] - c3 * xv[q][e];
        pg[q][e] += dz[q][e] * xv[q][e] * rr;
        const float z = xv[q][e] * rr * gg[e];
#pragma unroll
        for (int t = 0; t < 4; ++t) pw[t][q][e] += dlr[t] * z;
      }
      st4(dx + xrow * d + c, o);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) pb[t] += dlr[t];
  }
  // waves in order: wave 0 writes, waves 1..3 add
  for (int wv = 0; wv < RW / 64; ++wv) {
    if (wave == wv) {
#pragma unroll
      for (int q = 0; q < MAXQ; ++q) {
        const int c = 4 * lane + 256 * q;
        if (c >= d) break;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sp[c + e] = wv ? sp[c + e] + pg[q][e] : pg[q][e];
#pragma unroll
          for (int t = 0; t < 4; ++t)
            if (t < nt) sp[d * (1 + t) + c + e] = wv ? sp[d * (1 + t) + c + e] + pw[t][q][e] : pw[t][q][e];
        }
      }
      if (lane < nt) sp[d * (1 + nt) + lane] = wv ? sp[d * (1 + nt) + lane] + pb[lane] : pb[lane];
    }
    __syncthreads();
  }
  for (int c = threadIdx.x; c < width; c += RW) part[static_cast<int64_t>(blockIdx.x) * width + c] = sp[c];
}

// one block: mean BCE over n*nt logits (deterministic order) and its gradient
__global__ void __launch_bounds__(1024) bce_kernel(int64_t n, const float* __restrict__ z,
                                                   const float* __restrict__ y,
                                                   float* __restrict__ loss,
                                                   float* __restrict__ dz) {
  __shared__ float red[16];
  const float inv_n = 1.f / static_cast<float>(n);
  float s = 0.f;
  constexpr int U = 4;  // four elements' loads in flight per thread
  for (int64_t base = threadIdx.x; base < n; base += U * static_cast<int64_t>(blockDim.x)) {
    float zv[U], yv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + u * static_cast<int64_t>(blockDim.x);
      zv[u] = i < n ? z[i] : 0.f;
      yv[u] = i < n ? y[i] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + u * static_cast<int64_t>(blockDim.x);
      if (i >= n) break;
      const float zi = zv[u], yi = yv[u];
      s += fmaxf(zi, 0.f) + log1pf(__expf(-fabsf(zi))) - yi * zi;
      dz[i] = (1.f / (1.f + __expf(-zi)) - yi) * inv_n;
    }
  }
  s = wave_sum(s);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.f;
    for (int w = 0; w < static_cast<int>(blockDim.x >> 6); ++w) t += red[w];
    loss[0] = t * inv_n;
  }
}

unsigned blocks_for(int64_t n, int per_block) {
  int64_t b = (n + per_block - 1) / per_block;
  return static_cast<unsigned>(b < 1 ? 1 : (b > 65535 * 16 ? 65535 * 16 : b));
}

}  // namespace

template <typename TI, typename TO>
static bool launch_rmsnorm_vec(const TI* x, const float* g, TO* y, int64_t rows, int d, hipStream_t stream) {
  constexpr int VEC = 16 / static_cast<int>(sizeof(TI));
  if (d % VEC != 0 || ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(y) |
                        reinterpret_cast<uintptr_t>(g)) & 15u))
    return false;
  const int chunks = d / VEC;
  auto go = [&](auto kernel, int lpr) {
    const int64_t per_block = (RW / 64) * (64 / lpr);
    hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>((rows + per_block - 1) / per_block)), dim3(RW), 0,
                       stream, x, g, y, rows, d);
    return true;
  };
  switch (chunks) {
    case 2: return go(rmsnorm_vec_kernel<TI, TO, 2, 1>, 2);
    case 4: return go(rmsnorm_vec_kernel<TI, TO, 4, 1>, 4);
    case 8: return go(rmsnorm_vec_kernel<TI, TO, 8, 1>, 8);
    case 16: return go(rmsnorm_vec_kernel<TI, TO, 16, 1>, 16);
    case 32: return go(rmsnorm_vec_kernel<TI, TO, 32, 1>, 32);
    case 64: return go(rmsnorm_vec_kernel<TI, TO, 64, 1>, 64);
    case 128: return go(rmsnorm_vec_kernel<TI, TO, 64, 2>, 64);
    case 192: return go(rmsnorm_vec_kernel<TI, TO, 64, 3>, 64);
    case 256: return go(rmsnorm_vec_kernel<TI, TO, 64, 4>, 64);
    default: return false;
  }
}

template <typename TI, typename TO>
static void launch_rmsnorm_typed(const void* x, const float* g, void* y, int64_t rows, int d, hipStream_t stream) {
  if (launch_rmsnorm_vec(static_cast<const TI*>(x), g, static_cast<TO*>(y), rows, d, stream)) return;
  hipLaunchKernelGGL((rmsnorm_kernel<TI, TO>), dim3(static_cast<unsigned>((rows + 3) / 4)), dim3(RW), 0, stream,
                     static_cast<const TI*>(x), g, static_cast<TO*>(y), rows, d);
}

genrank_status launch_rmsnorm(int in_dtype, int out_dtype, const void* x, const float* g, void* y, int64_t rows,
                              int d, hipStream_t stream) {
  if (rows <= 0) return GENRANK_OK;
  if (in_dtype == GENRANK_BF16 && out_dtype == GENRANK_BF16)
    launch_rmsnorm_typed<bf16_t, bf16_t>(x, g, y, rows, d, stream);
  else if (in_dtype == GENRANK_F32 && out_dtype == GENRANK_BF16)
    launch_rmsnorm_typed<float, bf16_t>(x, g, y, rows, d, stream);
  else if (in_dtype == GENRANK_F32 && out_dtype == GENRANK_F32)
    launch_rmsnorm_typed<float, float>(x, g, y, rows, d, stream);
  else
    return GENRANK_E_DTYPE;
  GR_CHECK_LAUNCH();
  return GENRANK_OK;
}

size_t rmsnorm_bwd_workspace(int d) { return static_cast<size_t>(PART_BLOCKS) * d * sizeof(float); }

template <typename TX, typename T>
static int launch_rmsnorm_bwd_vec(const TX* x, const float* g, const T* dy, const T* add, T* dx, float* part,
                                  int64_t rows, int d, hipStream_t stream) {
  constexpr int VEC = 16 / static_cast<int>(sizeof(T));
  if (d % VEC != 0 || ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(dy) |
                        reinterpret_cast<uintptr_t>(add) | reinterpret_cast<uintptr_t>(dx) |
                        reinterpret_cast<uintptr_t>(g)) & 15u))
    return 0;
  auto go = [&](auto kernel, int lpr) {
    const int64_t per_block = (RW / 64) * (64 / lpr) * 2;
    const int grid = static_cast<int>(std::min<int64_t>(PART_BLOCKS, (rows + per_block - 1) / per_block));
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(RW), 0, stream, x, g, dy, add, dx, part, rows, d);
    return grid;
  };
  switch (d / VEC) {
    case 4: return go(rmsnorm_bwd_vec_kernel<TX, T, 4, 1>, 4);
    case 8: return go(rmsnorm_bwd_vec_kernel<TX, T, 8, 1>, 8);
    case 16: return go(rmsnorm_bwd_vec_kernel<TX, T, 16, 1>, 16);
    case 32: return go(rmsnorm_bwd_vec_kernel<TX, T, 32, 1>, 32);
    case 64: return go(rmsnorm_bwd_vec_kernel<TX, T, 64, 1>, 64);
    case 128: return go(rmsnorm_bwd_vec_kernel<TX, T, 64, 2>, 64);
    default: return 0;
  }
}

template <typename TX, typename T>
static int launch_rmsnorm_bwd_typed(const void* x, const float* g, const void* dy, const void* add, void* dx,
                                    float* part, int64_t rows, int d, hipStream_t stream) {
  const int vgrid = launch_rmsnorm_bwd_vec(static_cast<const TX*>(x), g, static_cast<const T*>(dy),
                                           static_cast<const T*>(add), static_cast<T*>(dx), part, rows, d, stream);
  if (vgrid > 0) return vgrid;
  const unsigned grid = static_cast<unsigned>(std::min<int64_t>(PART_BLOCKS, (rows + 7) / 8));
  hipLaunchKernelGGL((rmsnorm_bwd_kernel<TX, T>), dim3(grid), dim3(RW), 0, stream, static_cast<const TX*>(x), g,
                     static_cast<const T*>(dy), static_cast<const T*>(add), static_cast<T*>(dx), part, rows, d);
  return static_cast<int>(grid);
}

genrank_status launch_rmsnorm_bwd(int x_dtype, int dtype, const void* x, const float* g, const void* dy,
                                  const void* add, void* dx, float* dg, int64_t rows, int d, void* ws,
                                  hipStream_t stream) {
  if (d > 256 * MAXQ || d % 4) return GENRANK_E_SHAPE;
  float* part = static_cast<float*>(ws);
  if (rows <= 0) return launch_fill_f32(dg, d, 0.f, stream);
  int grid;
  if (x_dtype == GENRANK_BF16 && dtype == GENRANK_BF16)
    grid = launch_rmsnorm_bwd_typed<bf16_t, bf16_t>(x, g, dy, add, dx, part, rows, d, stream);
  else if (x_dtype == GENRANK_F32 && dtype == GENRANK_BF16)
    grid = launch_rmsnorm_bwd_typed<float, bf16_t>(x, g, dy, add, dx, part, rows, d, stream);
  else if (x_dtype == GENRANK_F32 && dtype == GENRANK_F32)
    grid = launch_rmsnorm_bwd_typed<float, float>(x, g, dy, add, dx, part, rows, d, stream);
  else
    return GENRANK_E_DTYPE;
  hipLaunchKernelGGL(column_sum_kernel, dim3((d + 15) / 16), dim3(256), 0, stream, part, grid, d, dg, d,
                     nullptr, 0, nullptr);
  GR_CHECK_LAUNCH();
  return GENRANK_OK;
}

genrank_status launch_fill_f32(float* p, int64_t n, float v, hipStream_t stream) {
  if (n <= 0) return GENRANK_OK;
  hipLaunchKernelGGL(fill_f32_kernel, dim3(blocks_for(n, 1024)), dim3(256), 0, stream, p, n, v);
  GR_CHECK_LAUNCH();
  return GENRANK_OK;
}

genrank_status launch_fill_zero(int dtype, void* p, int64_t n, hipStream_t stream) {
  if (dtype == GENRANK_F32) return launch_fill_f32(static_cast<float*>(p), n, 0.f, stream);
  if (n <= 0) return GENRANK_OK;
  hipLaunchKernelGGL(fill_u16_kernel, dim3(blocks_for(n, 1024)), dim3(256), 0, stream,
                     static_cast<uint16_t*>(p), n);
  GR_CHECK_LAUNCH();
  return GENRANK_OK;
}

template <typename T>
static bool launch_head_fwd_vec(const T* x, int64_t row0, int64_t rows, const int32_t* idx, int d,
                                const float* g, const float* w, const float* bias, int nt, float* logits,
                                hipStream_t stream) {
  constexpr int VEC = 16 / static_cast<int>(sizeof(T));
  if (d % VEC != 0 || ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(g) |
                        reinterpret_cast<uintptr_t>(w)) & 15u))
    return false;
  auto go = [&](auto kernel, int lpr) {
    const int64_t per_block = (RW / 64) * (64 / lpr);
    hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>((rows + per_block - 1) / per_block)), dim3(RW), 0,
                       stream, x, row0, rows, idx, d, g, w, bias, nt, logits);
    return true;
  };
  switch (d / VEC) {
    case 4: return go(head_fwd_vec_kernel<T, 4, 1>, 4);
    case 8: return go(head_fwd_vec_kernel<T, 8, 1>, 8);
    case 16: return go(head_fwd_vec_kernel<T, 16, 1>, 16);
    case 32: return go(head_fwd_vec_kernel<T, 32, 1>, 32);
    case 64: return go(head_fwd_vec_kernel<T, 64, 1>, 64);
    case 128: return go(head_fwd_vec_kernel<T, 64, 2>, 64);
    default: return false;
  }
}

genrank_status launch_head_fwd(int dtype, const void* x, int64_t row0, int64_t rows, const int32_t* idx,
                               int d, const float* g, const float* w, const float* bias, int nt,
                               float* logits, hipStream_t stream) {
  if (rows <= 0) return GENRANK_OK;
  const bool vec = dtype == GENRANK_BF16
                       ? launch_head_fwd_vec(static_cast<const bf16_t*>(x), row0, rows, idx, d, g, w, bias, nt,
                                             logits, stream)
                       : launch_head_fwd_vec(static_cast<const float*>(x), row0, rows, idx, d, g, w, bias, nt,
                                             logits, stream);
  if (vec) {
    GR_CHECK_LAUNCH();
    return GENRANK_OK;
  }
  const unsigned grid = static_cast<unsigned>((rows + 3) / 4);
  if (dtype == GENRANK_BF16)
    hipLaunchKernelGGL(head_fwd_kernel<bf16_t>, dim3(grid), dim3(RW), 0, stream,
                       static_cast<const bf16_t*>(x), row0, rows, idx, d, g, w, bias, nt, logits);
  else
    hipLaunchKernelGGL(head_fwd_kernel<float>, dim3(grid), dim3(RW), 0, stream,
                       static_cast<const float*>(x), row0, rows, idx, d, g, w, bias, nt, logits);
  GR_CHECK_LAUNCH();
  return GENRANK_OK;
}

size_t head_bwd_workspace(int d, int nt) {
  return static_cast<size_t>(HEAD_BLOCKS) * (static_cast<size_t>(d) * (1 + nt) + nt) * sizeof(float);
}

genrank_status launch_head_bwd(int x_dtype, int dtype, const void* x, int64_t row0, int64_t rows,
                               const int32_t* idx, int d, const float* g, const float* w, int nt,
                               const float* dlogits, void* dx, float* dg, float* dw, float* db, void* ws,
                               hipStream_t stream) {
  if (d > 256 * MAXQ || d % 4 || nt > 4) return GENRANK_E_SHAPE;
  if (rows <= 0) {
    genrank_status st = launch_fill_f32(dg, d, 0.f, stream);
    if (st == GENRANK_OK) st = launch_fill_f32(dw, static_cast<int64_t>(nt) * d, 0.f, stream);
    return st == GENRANK_OK ? launch_fill_f32(db, nt, 0.f, stream) : st;
  }
  float* part = static_cast<float*>(ws);
  const int width = d * (1 + nt) + nt;
  const unsigned grid = static_cast<unsigned>(std::min<int64_t>(HEAD_BLOCKS, (rows + 3) / 4));
  if (x_dtype == GENRANK_BF16 && dtype == GENRANK_BF16)
    hipLaunchKernelGGL((head_bwd_kernel<bf16_t, bf16_t>), dim3(grid), dim3(RW), 0, stream,
                       static_cast<const bf16_t*>(x), row0, rows, idx, d, g, w, nt, dlogits,
                       static_cast<bf16_t*>(dx), part);
  else if (x_dtype == GENRANK_F32 && dtype == GENRANK_BF16)
    hipLaunchKernelGGL((head_bwd_kernel<float, bf16_t>), dim3(grid), dim3(RW), 0, stream,
                       static_cast<const float*>(x), row0, rows, idx, d, g, w, nt, dlogits,
                       static_cast<bf16_t*>(dx), part);
  else if (x_dtype == GENRANK_F32 && dtype == GENRANK_F32)
    hipLaunchKernelGGL((head_bwd_kernel<float, float>), dim3(grid), dim3(RW), 0, stream,
                       static_cast<const float*>(x), row0, rows, idx, d, g, w, nt, dlogits,
                       static_cast<float*>(dx), part);
  else
    return GENRANK_E_DTYPE;
  hipLaunchKernelGGL(column_sum_kernel, dim3((width + 15) / 16), dim3(256), 0, stream, part,
                     static_cast<int>(grid), width, dg, d, dw, nt * d, db);
  GR_CHECK_LAUNCH();
  return GENRANK_OK;
}


genrank_status launch_bce(int64_t n, int nt, const float* logits, const float* labels,
                          float* loss, float* dlogits, hipStream_t stream) {
  hipLaunchKernelGGL(bce_kernel, dim3(1), dim3(1024), 0, stream, n * nt, logits, labels, loss,
                     dlogits);
  GR_CHECK_LAUNCH();
  return GENRANK_OK;
}

}  // namespace genrank
