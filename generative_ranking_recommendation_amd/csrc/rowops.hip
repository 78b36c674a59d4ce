// Row-wise pieces of the GenRank block and head: RMSNorm (+ backward), SiLU backward,
// the per-candidate action head (+ backward), sigmoid BCE at candidate rows, fills.
// One wave per row; rows are read with 16-byte vector loads where the width allows.
#include "common.hpp"
#include "internal.hpp"

namespace genrank {

namespace {

constexpr int RW = 256;  // threads per block (4 rows per block, one wave each)

__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

template <typename T>
__global__ void __launch_bounds__(RW) rmsnorm_kernel(const T* __restrict__ x, const float* __restrict__ g,
                                                     T* __restrict__ y, int64_t rows, int d) {
  const int64_t r = static_cast<int64_t>(blockIdx.x) * (RW / 64) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= rows) return;
  const T* xr = x + r * d;
  float ss = 0.f;
  for (int c = lane; c < d; c += 64) {
    const float v = to_f32(xr[c]);
    ss += v * v;
  }
  ss = wave_sum(ss);
  const float inv = rsqrtf(ss / d + RMS_EPS);
  T* yr = y + r * d;
  for (int c = lane; c < d; c += 64) yr[c] = from_f32<T>(to_f32(xr[c]) * inv * g[c]);
}

// dx = r g dy - r^3 x sum(g dy x) / d  (+ add);  dg += sum_rows dy x r.
// Each wave walks rows with a grid stride and keeps its dg partial in registers (lane c
// owns columns c, c+64, ...), so dg takes one atomic per column per wave.
constexpr int MAXC = 16;  // d <= 1024

template <typename T>
__global__ void __launch_bounds__(RW) rmsnorm_bwd_kernel(const T* __restrict__ x, const float* __restrict__ g,
                                                         const T* __restrict__ dy, const T* add,
                                                         T* dx, float* __restrict__ dg,
                                                         int64_t rows, int d) {
  const int lane = threadIdx.x & 63;
  const int64_t nw = static_cast<int64_t>(gridDim.x) * (RW / 64);
  float part[MAXC];
#pragma unroll
  for (int i = 0; i < MAXC; ++i) part[i] = 0.f;
  for (int64_t r = static_cast<int64_t>(blockIdx.x) * (RW / 64) + (threadIdx.x >> 6); r < rows; r += nw) {
    const T* xr = x + r * d;
    const T* dyr = dy + r * d;
    float ss = 0.f, dot = 0.f;
    for (int c = lane; c < d; c += 64) {
      const float v = to_f32(xr[c]);
      ss += v * v;
      dot += g[c] * to_f32(dyr[c]) * v;
    }
    ss = wave_sum(ss);
    dot = wave_sum(dot);
    const float rr = rsqrtf(ss / d + RMS_EPS);
    const float c3 = rr * rr * rr * dot / d;
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      const int c = lane + 64 * i;
      if (c >= d) break;
      const float v = to_f32(xr[c]);
      const float gy = to_f32(dyr[c]);
      float o = rr * g[c] * gy - c3 * v;
      if (add) o += to_f32(add[r * d + c]);
      dx[r * d + c] = from_f32<T>(o);
      part[i] += gy * v * rr;
    }
  }
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = lane + 64 * i;
    if (c >= d) break;
    atomicAdd(dg + c, part[i]);
  }
}

template <typename T>
__global__ void silu_bwd_kernel(const T* __restrict__ a, const T* __restrict__ dy, T* __restrict__ da, int64_t n) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const float av = to_f32(a[i]);
    const float sg = 1.f / (1.f + __expf(-av));
    da[i] = from_f32<T>(to_f32(dy[i]) * sg * (1.f + av * (1.f - sg)));
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

// logits[c, t] = rmsnorm(x_c) g . w[t] + b[t]
template <typename T>
__global__ void __launch_bounds__(RW) head_fwd_kernel(const T* __restrict__ x, int64_t row0, int64_t rows,
                                                      int d, const float* __restrict__ g,
                                                      const float* __restrict__ w,
                                                      const float* __restrict__ b, int nt,
                                                      float* __restrict__ logits) {
  const int64_t r = static_cast<int64_t>(blockIdx.x) * (RW / 64) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= rows) return;
  const T* xr = x + (row0 + r) * d;
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

// z = rmsnorm(x) g; dz = dlogits . w; dx by the RMSNorm backward with dz as the output
// gradient; dw[t] += dlogits[t] z; db[t] += dlogits[t]; dg += dz x r.  Parameter
// gradients are summed per wave in registers, then added with one atomic per element.
template <typename T>
__global__ void __launch_bounds__(RW) head_bwd_kernel(const T* __restrict__ x, int64_t row0, int64_t rows,
                                                      int d, const float* __restrict__ g,
                                                      const float* __restrict__ w, int nt,
                                                      const float* __restrict__ dl, T* __restrict__ dx,
                                                      float* __restrict__ dg, float* __restrict__ dw,
                                                      float* __restrict__ db) {
  const int lane = threadIdx.x & 63;
  const int64_t nw = static_cast<int64_t>(gridDim.x) * (RW / 64);
  float pg[MAXC], pw[4][MAXC], pb[4];
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    pg[i] = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t) pw[t][i] = 0.f;
  }
#pragma unroll
  for (int t = 0; t < 4; ++t) pb[t] = 0.f;
  for (int64_t r = static_cast<int64_t>(blockIdx.x) * (RW / 64) + (threadIdx.x >> 6); r < rows; r += nw) {
    const T* xr = x + (row0 + r) * d;
    float dlr[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) dlr[t] = (t < nt) ? dl[r * nt + t] : 0.f;
    float ss = 0.f, dot = 0.f;
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      const int c = lane + 64 * i;
      if (c >= d) break;
      const float v = to_f32(xr[c]);
      ss += v * v;
      float dz = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if (t < nt) dz += dlr[t] * w[t * d + c];
      dot += g[c] * dz * v;
    }
    ss = wave_sum(ss);
    dot = wave_sum(dot);
    const float rr = rsqrtf(ss / d + RMS_EPS);
    const float c3 = rr * rr * rr * dot / d;
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      const int c = lane + 64 * i;
      if (c >= d) break;
      const float v = to_f32(xr[c]);
      float dz = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if (t < nt) dz += dlr[t] * w[t * d + c];
      dx[(row0 + r) * d + c] = from_f32<T>(rr * g[c] * dz - c3 * v);
      pg[i] += dz * v * rr;
      const float z = v * rr * g[c];
#pragma unroll
      for (int t = 0; t < 4; ++t) pw[t][i] += dlr[t] * z;
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) pb[t] += dlr[t];
  }
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = lane + 64 * i;
    if (c >= d) break;
    atomicAdd(dg + c, pg[i]);
#pragma unroll
    for (int t = 0; t < 4; ++t)
      if (t < nt) atomicAdd(dw + t * d + c, pw[t][i]);
  }
  if (lane == 0) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
      if (t < nt) atomicAdd(db + t, pb[t]);
  }
}

// one block: mean BCE over n*nt logits (deterministic order) and its gradient
__global__ void __launch_bounds__(1024) bce_kernel(int64_t n, const float* __restrict__ z,
                                                   const float* __restrict__ y,
                                                   float* __restrict__ loss,
                                                   float* __restrict__ dz) {
  __shared__ float red[16];
  const float inv_n = 1.f / static_cast<float>(n);
  float s = 0.f;
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
    const float zi = z[i], yi = y[i];
    s += fmaxf(zi, 0.f) + log1pf(__expf(-fabsf(zi))) - yi * zi;
    dz[i] = (1.f / (1.f + __expf(-zi)) - yi) * inv_n;
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

genrank_status launch_rmsnorm(int dtype, const void* x, const float* g, void* y, int64_t rows,
                              int d, hipStream_t stream) {
  if (rows <= 0) return GENRANK_OK;
  const unsigned grid = static_cast<unsigned>((rows + 3) / 4);
  if (dtype == GENRANK_BF16)
    hipLaunchKernelGGL(rmsnorm_kernel<bf16_t>, dim3(grid), dim3(RW), 0, stream,
                       static_cast<const bf16_t*>(x), g, static_cast<bf16_t*>(y), rows, d);
  else
    hipLaunchKernelGGL(rmsnorm_kernel<float>, dim3(grid), dim3(RW), 0, stream,
                       static_cast<const float*>(x), g, static_cast<float*>(y), rows, d);
  GR_CHECK_LAUNCH();
  return GENRANK_OK;
}

genrank_status launch_rmsnorm_bwd(int dtype, const void* x, const float* g, const void* dy,
                                  const void* add, void* dx, float* dg, int64_t rows, int d,
                                  hipStream_t stream) {
  if (rows <= 0) return GENRANK_OK;
  if (d > 64 * MAXC) return GENRANK_E_SHAPE;
  const unsigned grid = static_cast<unsigned>(rows < 4096 ? (rows + 3) / 4 : 1024);
  if (dtype == GENRANK_BF16)
    hipLaunchKernelGGL(rmsnorm_bwd_kernel<bf16_t>, dim3(grid), dim3(RW), 0, stream,
                       static_cast<const bf16_t*>(x), g, static_cast<const bf16_t*>(dy),
                       static_cast<const bf16_t*>(add), static_cast<bf16_t*>(dx), dg, rows, d);
  else
    hipLaunchKernelGGL(rmsnorm_bwd_kernel<float>, dim3(grid), dim3(RW), 0, stream,
                       static_cast<const float*>(x), g, static_cast<const float*>(dy),
                       static_cast<const float*>(add), static_cast<float*>(dx), dg, rows, d);
  GR_CHECK_LAUNCH();
  return GENRANK_OK;
}

genrank_status launch_silu_bwd(int dtype, const void* a, const void* dy, void* da, int64_t n,
                               hipStream_t stream) {
  if (n <= 0) return GENRANK_OK;
  if (dtype == GENRANK_BF16)
    hipLaunchKernelGGL(silu_bwd_kernel<bf16_t>, dim3(blocks_for(n, 256)), dim3(256), 0, stream,
                       static_cast<const bf16_t*>(a), static_cast<const bf16_t*>(dy),
                       static_cast<bf16_t*>(da), n);
  else
    hipLaunchKernelGGL(silu_bwd_kernel<float>, dim3(blocks_for(n, 256)), dim3(256), 0, stream,
                       static_cast<const float*>(a), static_cast<const float*>(dy),
                       static_cast<float*>(da), n);
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

genrank_status launch_head_fwd(int dtype, const void* x, int64_t row0, int64_t rows, int d,
                               const float* g, const float* w, const float* bias, int nt,
                               float* logits, hipStream_t stream) {
  if (rows <= 0) return GENRANK_OK;
  const unsigned grid = static_cast<unsigned>((rows + 3) / 4);
  if (dtype == GENRANK_BF16)
    hipLaunchKernelGGL(head_fwd_kernel<bf16_t>, dim3(grid), dim3(RW), 0, stream,
                       static_cast<const bf16_t*>(x), row0, rows, d, g, w, bias, nt, logits);
  else
    hipLaunchKernelGGL(head_fwd_kernel<float>, dim3(grid), dim3(RW), 0, stream,
                       static_cast<const float*>(x), row0, rows, d, g, w, bias, nt, logits);
  GR_CHECK_LAUNCH();
  return GENRANK_OK;
}

genrank_status launch_head_bwd(int dtype, const void* x, int64_t row0, int64_t rows, int d,
                               const float* g, const float* w, int nt, const float* dlogits,
                               void* dx, float* dg, float* dw, float* db, hipStream_t stream) {
  if (rows <= 0) return GENRANK_OK;
  if (d > 64 * MAXC || nt > 4) return GENRANK_E_SHAPE;
  const unsigned grid = static_cast<unsigned>(rows < 4096 ? (rows + 3) / 4 : 1024);
  if (dtype == GENRANK_BF16)
    hipLaunchKernelGGL(head_bwd_kernel<bf16_t>, dim3(grid), dim3(RW), 0, stream,
                       static_cast<const bf16_t*>(x), row0, rows, d, g, w, nt, dlogits,
                       static_cast<bf16_t*>(dx), dg, dw, db);
  else
    hipLaunchKernelGGL(head_bwd_kernel<float>, dim3(grid), dim3(RW), 0, stream,
                       static_cast<const float*>(x), row0, rows, d, g, w, nt, dlogits,
                       static_cast<float*>(dx), dg, dw, db);
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
