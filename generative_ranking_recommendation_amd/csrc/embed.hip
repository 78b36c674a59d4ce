// Fused index derivation + five-table embedding gather-sum (and its adjoint).
//
// Token embedding of GenRank ("一、 GenRank [2025]", section 1.4.2, five-term input
// representation; section 1.4.1 for the item + action token and the mask-action row):
//   e = psi(item) + phi(action) + Omega_pe(position) + Omega_ri(request index)
//       + Omega_rt(bucket(gap to the previous request)).
//
// Work decomposition: one workgroup per (user, chunk of ROWS rows).  Wave 0 derives the
// chunk's indices: the request index is 1 + the number of timestamp changes in the
// user's prefix (timestamps are non-decreasing, so distinct values == runs); a block
// reduction counts the changes before the chunk and a 64-lane ballot scans the chunk.
// The previous distinct timestamp of a row is the one just before its run.  The five
// rows are then gathered with 16-byte loads (d/8 lanes per bf16 row), summed in f32 and
// written once.  The small tables stay L2-resident across the grid.
#include <algorithm>
#include <mutex>

#include "common.hpp"
#include "internal.hpp"

namespace genrank {

namespace {

constexpr int EMB_THREADS = 256;
constexpr int EMB_ROWS = 64;  // rows per workgroup (one wave derives 64 rows' indices)
constexpr int MAX_BOUNDS = 1024;

struct EmbedArgs {
  const int32_t* offsets;
  const int32_t* hist_items;
  const int32_t* hist_actions;
  const int64_t* hist_ts;
  const int32_t* cand_items;
  const int64_t* req_ts;
  const void* t_item;
  const void* t_action;
  const void* t_pos;
  const void* t_ri;
  const void* t_rt;
  const int64_t* rt_bounds;
  int B, m, d, hist_chunks, cand_chunks;
  int n_action, n_pos, n_ri, n_bounds;
  int64_t T_h;
  uint32_t bytes_item, bytes_action, bytes_pos, bytes_ri, bytes_rt;  // table sizes (< 4 GB)
  int64_t n_item;
  uint32_t* err;        // the device error word (GENRANK_ERR_*)
  void* out;            // gather: [T, d]; debug: int32 [6, T]
  const void* dx;       // backward: [T, d]
  float* g_item; float* g_action; float* g_pos; float* g_ri; float* g_rt;
};

template <typename T> struct Vec;
template <> struct Vec<bf16_t> { static constexpr int N = 8; };
template <> struct Vec<float> { static constexpr int N = 4; };

__device__ __forceinline__ void load_vec(const bf16_t* p, float* f) {
  uint4 v = *reinterpret_cast<const uint4*>(p);
  unpack8(v, f);
}
__device__ __forceinline__ void load_vec(const float* p, float* f) {
  float4 v = *reinterpret_cast<const float4*>(p);
  f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w;
}
__device__ __forceinline__ void store_vec(bf16_t* p, const float* f) {
  *reinterpret_cast<uint4*>(p) = pack8(f);
}
__device__ __forceinline__ void store_vec(float* p, const float* f) {
  *reinterpret_cast<float4*>(p) = make_float4(f[0], f[1], f[2], f[3]);
}

// #{k : bounds[k] <= gap} over non-decreasing bounds (upper bound).
__device__ __forceinline__ int bucket_of(const int64_t* bounds, int n, int64_t gap) {
  int lo = 0, hi = n;
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if (bounds[mid] <= gap) lo = mid + 1; else hi = mid;
  }
  return lo;
}

struct RowIdx {
  int item, act, pos, pe, ri, ri_slot, rt;
};

// Block-wide sum (int) and max (int64) of per-thread values; every thread gets both.
__device__ __forceinline__ void block_sum_max(int& c, int64_t& mx, int* red_c, int64_t* red_m) {
  for (int off = 32; off > 0; off >>= 1) {
    c += __shfl_xor(c, off);
    const int64_t o = __shfl_xor(mx, off);
    mx = o > mx ? o : mx;
  }
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    red_c[wave] = c;
    red_m[wave] = mx;
  }
  __syncthreads();
  c = 0;
  mx = INT64_MIN;
#pragma unroll
  for (int w = 0; w < EMB_THREADS / 64; ++w) {
    c += red_c[w];
    mx = red_m[w] > mx ? red_m[w] : mx;
  }
}

// Derives the indices of the workgroup's rows into shared memory.  Returns the number of
// valid rows and the global row of the first one (via *row0).  Every load that depends
// only on the user's offsets is issued before the first wait, so a chunk costs about two
// memory round trips before its gathers:
//   * request index: 1 + number of timestamp changes up to the row (timestamps are
//     non-decreasing, so distinct values are runs); changes before the chunk come from a
//     block reduction over the user's prefix, changes inside it from a 64-lane ballot;
//   * gap to the previous request: the row's time minus the time just before its run.
//     Inside the chunk that is a neighbouring lane's value; for a run that began before
//     the chunk it is the largest prefix timestamp below ts[r0], reduced alongside.
__device__ int derive_chunk(const EmbedArgs& a, RowIdx* sidx, int64_t* sbounds, int* red_c,
                            int64_t* red_m, int64_t* row0_out) {
  const int u = blockIdx.y;
  const int chunk = blockIdx.x;
  const int64_t off = a.offsets[u];
  const int N = a.offsets[u + 1] - a.offsets[u];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const bool is_hist = chunk < a.hist_chunks;

  if (is_hist) {
    const int s0 = chunk * EMB_ROWS;  // first sequence slot of the chunk
    if (s0 >= N) return 0;            // uniform across the block
    // the grid covers batch.max_hist rows per user: a longer history is cut here
    if (tid == 0 && chunk == a.hist_chunks - 1 && N > s0 + EMB_ROWS) report_error(a.err, GENRANK_ERR_HIST_LONG);
    const int rows = min(EMB_ROWS, N - s0);
    const int64_t r0 = off + s0;
    // the chunk's own rows (wave 0), the bucket bounds and the prefix, all in flight
    const bool valid = tid < rows;
    const int64_t r = r0 + lane;
    int64_t t = 0;
    int item = 0, act = 0;
    if (tid < 64 && valid) {
      t = a.hist_ts[r];
      item = a.hist_items[r];
      act = a.hist_actions[r];
      // ids outside their tables: flagged, and the nearest valid row used
      if (item < 0 || item >= a.n_item || act < 0 || act >= a.n_action) {
        report_error(a.err, GENRANK_ERR_ID_RANGE);
        item = static_cast<int>(min<int64_t>(max(item, 0), a.n_item - 1));
        act = min(max(act, 0), a.n_action - 1);
      }
    }
    for (int k = tid; k < a.n_bounds; k += EMB_THREADS) sbounds[k] = a.rt_bounds[k];
    const int64_t t_r0 = a.hist_ts[r0];
    const int64_t t_rm1 = r0 > off ? a.hist_ts[r0 - 1] : t_r0;
    int c = 0;
    int64_t mx = INT64_MIN;
    for (int64_t k = off + tid; k < r0; k += EMB_THREADS) {
      const int64_t v = a.hist_ts[k];
      if (k > off) c += (v != a.hist_ts[k - 1]);
      if (v < t_r0 && v > mx) mx = v;
    }
    block_sum_max(c, mx, red_c, red_m);  // also orders the sbounds writes
    const int before = c;                // changes at k in [off + 1, r0)
    const int64_t prev_head = mx;        // time before the run holding r0 (INT64_MIN: none)
    if (tid < 64) {
      const int64_t tl = __shfl_up(t, 1);  // lane i - 1's time
      const bool change = valid && (lane == 0 ? t != t_rm1 : t != tl);
      const uint64_t mask = __ballot(change);
      const uint64_t upto = (lane == 63) ? ~0ull : ((2ull << lane) - 1ull);
      const uint64_t cm = mask & upto;
      // the run of row r starts at lane j = highest change at or below r, or before the
      // chunk (j = -1); a change at lane 0 means ts[r0 - 1] < ts[r0], which is then the
      // largest prefix time below ts[r0], i.e. prev_head
      const int j = cm ? 63 - __clzll(static_cast<long long>(cm)) : -1;
      const int64_t tj = __shfl(t, j > 0 ? j - 1 : 0);
      const int64_t prev = j > 0 ? tj : prev_head;
      if (valid) {
        RowIdx ix;
        ix.item = item;
        ix.act = act;
        ix.pos = s0 + lane;
        ix.pe = min(ix.pos, a.n_pos - 1);
        ix.ri = 1 + before + __popcll(cm);
        ix.ri_slot = min(ix.ri - 1, a.n_ri - 1);
        ix.rt = prev != INT64_MIN ? bucket_of(sbounds, a.n_bounds, t - prev) : 0;
        sidx[lane] = ix;
      }
    }
    __syncthreads();
    *row0_out = r0;
    return rows;
  }
  // candidate chunk
  const int c0 = (chunk - a.hist_chunks) * EMB_ROWS;
  if (c0 >= a.m) return 0;
  const int rows = min(EMB_ROWS, a.m - c0);
  const int64_t r0 = a.T_h + static_cast<int64_t>(u) * a.m + c0;
  int item = 0;
  if (tid < rows) {
    item = a.cand_items[static_cast<int64_t>(u) * a.m + c0 + tid];
    if (item < 0 || item >= a.n_item) {
      report_error(a.err, GENRANK_ERR_ID_RANGE);
      item = static_cast<int>(min<int64_t>(max(item, 0), a.n_item - 1));
    }
  }
  for (int k = tid; k < a.n_bounds; k += EMB_THREADS) sbounds[k] = a.rt_bounds[k];
  const int64_t req = a.req_ts[u];
  const int64_t t_last = N > 0 ? a.hist_ts[off + N - 1] : 0;
  int c = 0;
  int64_t mx = INT64_MIN;
  for (int64_t k = off + 1 + tid; k < off + N; k += EMB_THREADS) c += (a.hist_ts[k] != a.hist_ts[k - 1]);
  block_sum_max(c, mx, red_c, red_m);
  const int distinct_hist = (N > 0) ? 1 + c : 0;
  if (tid < rows) {
    RowIdx ix;
    ix.item = item;
    ix.act = a.n_action;
    ix.pos = N;
    ix.pe = min(N, a.n_pos - 1);
    ix.ri = distinct_hist + 1;
    ix.ri_slot = min(ix.ri - 1, a.n_ri - 1);
    ix.rt = N > 0 ? bucket_of(sbounds, a.n_bounds, req - t_last) : 0;
    sidx[tid] = ix;
  }
  __syncthreads();
  *row0_out = r0;
  return rows;
}

template <typename T, typename TO>
__global__ void __launch_bounds__(EMB_THREADS) embed_sum_kernel(EmbedArgs a) {
  __shared__ RowIdx sidx[EMB_ROWS];
  __shared__ int64_t sbounds[MAX_BOUNDS];
  __shared__ int red_c[EMB_THREADS / 64];
  __shared__ int64_t red_m[EMB_THREADS / 64];
  int64_t row0;
  const int rows = derive_chunk(a, sidx, sbounds, red_c, red_m, &row0);
  if (rows == 0) return;
  constexpr int V = Vec<T>::N;
  const int cpr = a.d / V;  // 16-byte chunks per row
  const int total = rows * cpr;
  const T* ti = static_cast<const T*>(a.t_item);
  const T* ta = static_cast<const T*>(a.t_action);
  const T* tp = static_cast<const T*>(a.t_pos);
  const T* tr = static_cast<const T*>(a.t_ri);
  const T* tt = static_cast<const T*>(a.t_rt);
  TO* out = static_cast<TO*>(a.out);
  const int64_t d = a.d;
  constexpr int U = 2;  // items per thread in flight
  for (int base = threadIdx.x; base < total; base += EMB_THREADS * U) {
    float acc[U][V];
    float tmp[V];
#pragma unroll
    for (int uu = 0; uu < U; ++uu) {
      const int idx = base + uu * EMB_THREADS;
      if (idx < total) {
        const int r = idx / cpr;
        const int col = (idx - r * cpr) * V;
        const RowIdx ix = sidx[r];
        load_vec(ti + ix.item * d + col, acc[uu]);
        load_vec(ta + ix.act * d + col, tmp);
#pragma unroll
        for (int e = 0; e < V; ++e) acc[uu][e] += tmp[e];
        load_vec(tp + ix.pe * d + col, tmp);
#pragma unroll
        for (int e = 0; e < V; ++e) acc[uu][e] += tmp[e];
        load_vec(tr + ix.ri_slot * d + col, tmp);
#pragma unroll
        for (int e = 0; e < V; ++e) acc[uu][e] += tmp[e];
        load_vec(tt + ix.rt * d + col, tmp);
#pragma unroll
        for (int e = 0; e < V; ++e) acc[uu][e] += tmp[e];
      }
    }
#pragma unroll
    for (int uu = 0; uu < U; ++uu) {
      const int idx = base + uu * EMB_THREADS;
      if (idx < total) {
        const int r = idx / cpr;
        const int col = (idx - r * cpr) * V;
        if constexpr (sizeof(TO) == sizeof(T)) {
          store_vec(out + (row0 + r) * d + col, acc[uu]);
        } else {  // bf16 tables, f32 rows: two 4-column stores
          store_vec(out + (row0 + r) * d + col, acc[uu]);
          store_vec(out + (row0 + r) * d + col + 4, acc[uu] + 4);
        }
      }
    }
  }
}

// Gather phase with a fixed column per thread: thread t handles column piece t % cpr of
// rows t / cpr, t / cpr + rpp, ... (cpr = d / 8 threads per row, rpp = threads / cpr),
// four rows in flight.  A piece is 16 bytes of each table row (8 bf16 or 4 f32 columns),
// except for f32 rows summed from bf16 tables: there thread c of a row takes the 4-column
// groups c and c + cpr (two 8-byte reads per table), so that each of its two 16-byte
// output stores lands next to its neighbours' (a wave's store covers one contiguous span).
// Table reads and output writes are buffer accesses with 32-bit byte offsets (every table
// is below 4 GB); rows past the chunk write nothing.  NT: outputs far larger than the
// last-level cache (256 MiB) go out as streaming (non-temporal) stores, so that they leave no dirty
// lines behind for the next kernels to evict; smaller ones stay cached for the next kernel.
constexpr int BUF_DWORD3 = 0x00020000;  // raw buffer descriptor word 3 (gfx9 family)
constexpr int CPOL_NT = 2;              // buffer cache policy: non-temporal
constexpr int64_t STREAM_OUT_BYTES = int64_t(256) << 20;  // outputs above this use NT stores

template <typename T>
__device__ __forceinline__ void add_vec(const uint4& v, float* acc) {
  if constexpr (sizeof(T) == 2) {
    acc[0] += __uint_as_float(v.x << 16); acc[1] += __uint_as_float(v.x & 0xFFFF0000u);
    acc[2] += __uint_as_float(v.y << 16); acc[3] += __uint_as_float(v.y & 0xFFFF0000u);
    acc[4] += __uint_as_float(v.z << 16); acc[5] += __uint_as_float(v.z & 0xFFFF0000u);
    acc[6] += __uint_as_float(v.w << 16); acc[7] += __uint_as_float(v.w & 0xFFFF0000u);
  } else {
    acc[0] += __uint_as_float(v.x); acc[1] += __uint_as_float(v.y);
    acc[2] += __uint_as_float(v.z); acc[3] += __uint_as_float(v.w);
  }
}

// SACT: the action table (n_action + 1 rows, at most SACT_MAX bytes) is staged in dynamic
// LDS: every workgroup reads its few rows for every token, so they are copied once per
// workgroup rather than fetched from the same L2 lines by every row.
constexpr int SACT_MAX = 32768;

// TO: the element type of the output rows (the tables' type, or f32 rows from bf16 tables).
template <typename T, typename TO, bool SACT, bool NT>
__global__ void __launch_bounds__(EMB_THREADS) embed_sum_rows_kernel(EmbedArgs a) {
  constexpr int CPOL = NT ? CPOL_NT : 0;
  __shared__ RowIdx sidx[EMB_ROWS];
  __shared__ int64_t sbounds[MAX_BOUNDS];
  __shared__ int red_c[EMB_THREADS / 64];
  __shared__ int64_t red_m[EMB_THREADS / 64];
  extern __shared__ __attribute__((aligned(16))) uint4 s_act[];
  int64_t row0;
  const int rows = derive_chunk(a, sidx, sbounds, red_c, red_m, &row0);
  if (rows == 0) return;
  if constexpr (SACT) {
    const int n16 = static_cast<int>(a.bytes_action / 16);
    const uint4* src = static_cast<const uint4*>(a.t_action);
    for (int i = threadIdx.x; i < n16; i += EMB_THREADS) s_act[i] = src[i];
    __syncthreads();
  }
  constexpr bool SPLIT = sizeof(TO) > sizeof(T);  // bf16 tables, f32 rows
  constexpr int V = Vec<T>::N;
  constexpr int UR = 4;
  const int cpr = a.d / V;
  const int rpp = EMB_THREADS / cpr;
  const int rp = threadIdx.x / cpr;
  const int c = threadIdx.x - rp * cpr;
  const uint32_t rowb = static_cast<uint32_t>(a.d * sizeof(T));
  // byte offsets of this thread's piece(s) in a table row and in an output row
  const uint32_t colb = SPLIT ? 8u * c : static_cast<uint32_t>(c * V * sizeof(T));
  const uint32_t colb2 = 8u * (c + cpr);  // SPLIT: the second 4-column group
  auto rsrc = [](const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), static_cast<short>(0), bytes, BUF_DWORD3);
  };
  const __amdgpu_buffer_rsrc_t rs_item = rsrc(a.t_item, a.bytes_item);
  const __amdgpu_buffer_rsrc_t rs_act = rsrc(a.t_action, a.bytes_action);
  const __amdgpu_buffer_rsrc_t rs_pos = rsrc(a.t_pos, a.bytes_pos);
  const __amdgpu_buffer_rsrc_t rs_ri = rsrc(a.t_ri, a.bytes_ri);
  const __amdgpu_buffer_rsrc_t rs_rt = rsrc(a.t_rt, a.bytes_rt);
  constexpr uint32_t OW = sizeof(TO) / sizeof(T);  // output bytes per table byte
  const uint32_t orowb = rowb * OW;
  const uint32_t out_bytes = static_cast<uint32_t>(rows) * orowb;
  const __amdgpu_buffer_rsrc_t rs_out = rsrc(static_cast<TO*>(a.out) + row0 * a.d, out_bytes);
  typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
  // one table piece at byte offset `o` of a row: 16 bytes, or (SPLIT) two 8-byte groups
  auto load = [&](const __amdgpu_buffer_rsrc_t& rs, uint32_t rowoff) -> uint4 {
    if constexpr (SPLIT) {
      const uint2 lo = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs, rowoff + colb, 0, 0));
      const uint2 hi = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs, rowoff + colb2, 0, 0));
      return make_uint4(lo.x, lo.y, hi.x, hi.y);
    } else {
      return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, rowoff + colb, 0, 0));
    }
  };
  auto load_act = [&](int act) -> uint4 {
    const char* base = reinterpret_cast<const char*>(s_act) + min(act, a.n_action) * rowb;
    if constexpr (SPLIT) {
      const uint2 lo = *reinterpret_cast<const uint2*>(base + colb);
      const uint2 hi = *reinterpret_cast<const uint2*>(base + colb2);
      return make_uint4(lo.x, lo.y, hi.x, hi.y);
    } else {
      return *reinterpret_cast<const uint4*>(base + colb);
    }
  };
  for (int r = rp; r < rows; r += rpp * UR) {
    uint4 v[UR][5];
#pragma unroll
    for (int u = 0; u < UR; ++u) {
      const RowIdx ix = sidx[min(r + u * rpp, rows - 1)];
      v[u][0] = load(rs_item, ix.item * rowb);
      if constexpr (SACT)
        v[u][1] = load_act(ix.act);
      else
        v[u][1] = load(rs_act, ix.act * rowb);
      v[u][2] = load(rs_pos, ix.pe * rowb);
      v[u][3] = load(rs_ri, ix.ri_slot * rowb);
      v[u][4] = load(rs_rt, ix.rt * rowb);
    }
#pragma unroll
    for (int u = 0; u < UR; ++u) {
      float acc[V];
#pragma unroll
      for (int e = 0; e < V; ++e) acc[e] = 0.f;
#pragma unroll
      for (int t = 0; t < 5; ++t) add_vec<T>(v[u][t], acc);
      const int rr = r + u * rpp;
      const bool ok = rr < rows;
      const uint32_t ro = static_cast<uint32_t>(rr) * orowb;
      if constexpr (sizeof(TO) == 2) {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, pack8(acc)), rs_out,
                                               ok ? ro + colb : out_bytes, 0, CPOL);
      } else if constexpr (SPLIT) {  // groups c and c + cpr: 16 bytes each at 16 c and 16 (c + cpr)
        const uint4 o0 = make_uint4(__float_as_uint(acc[0]), __float_as_uint(acc[1]), __float_as_uint(acc[2]),
                                    __float_as_uint(acc[3]));
        const uint4 o1 = make_uint4(__float_as_uint(acc[4]), __float_as_uint(acc[5]), __float_as_uint(acc[6]),
                                    __float_as_uint(acc[7]));
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o0), rs_out, ok ? ro + 2u * colb : out_bytes,
                                               0, CPOL);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o1), rs_out, ok ? ro + 2u * colb2 : out_bytes,
                                               0, CPOL);
      } else {
        const uint4 o = make_uint4(__float_as_uint(acc[0]), __float_as_uint(acc[1]), __float_as_uint(acc[2]),
                                   __float_as_uint(acc[3]));
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o), rs_out, ok ? ro + colb : out_bytes, 0,
                                               CPOL);
      }
    }
  }
}

__global__ void __launch_bounds__(EMB_THREADS) debug_indices_kernel(EmbedArgs a, int64_t T) {
  __shared__ RowIdx sidx[EMB_ROWS];
  __shared__ int64_t sbounds[MAX_BOUNDS];
  __shared__ int red_c[EMB_THREADS / 64];
  __shared__ int64_t red_m[EMB_THREADS / 64];
  int64_t row0;
  const int rows = derive_chunk(a, sidx, sbounds, red_c, red_m, &row0);
  if (static_cast<int>(threadIdx.x) < rows) {
    int32_t* out = static_cast<int32_t*>(a.out);
    const RowIdx ix = sidx[threadIdx.x];
    const int64_t r = row0 + threadIdx.x;
    out[0 * T + r] = ix.act;
    out[1 * T + r] = ix.pos;
    out[2 * T + r] = ix.pe;
    out[3 * T + r] = ix.ri;
    out[4 * T + r] = ix.ri_slot;
    out[5 * T + r] = ix.rt;
  }
}

// ---------------------------------------------------------------- backward (adjoint)
// Row r of table t's gradient is the sum of dx over the batch rows whose slot in table t is
// r.  The rows are grouped by slot rather than scattered with atomics:
//   1. keys: every batch row writes its five slots, table t into slice t of T (key, row)
//      pairs;
//   2. the five slices are radix-sorted by key, stably, so a group keeps its rows in
//      ascending order;
//   3. the sorted pairs are cut into chunks of SEG; a run of equal keys that lies inside a
//      chunk is summed there column by column in row order and written out; a run that
//      crosses chunk borders leaves one partial sum per chunk, and the chunk holding its
//      first row adds those up in chunk order.
// The summation order is fixed (deterministic results) and there are no atomics.  The item
// gradient comes out sparse (one row per distinct item, ascending ids); the four small
// tables dense, every row written.
constexpr int SEG = 64;  // sorted pairs per chunk (one wave classifies a chunk)

__global__ void __launch_bounds__(EMB_THREADS) embed_keys_kernel(EmbedArgs a, uint32_t* keys, uint32_t* vals,
                                                                 int64_t T) {
  __shared__ RowIdx sidx[EMB_ROWS];
  __shared__ int64_t sbounds[MAX_BOUNDS];
  __shared__ int red_c[EMB_THREADS / 64];
  __shared__ int64_t red_m[EMB_THREADS / 64];
  int64_t row0;
  const int rows = derive_chunk(a, sidx, sbounds, red_c, red_m, &row0);
  if (static_cast<int>(threadIdx.x) >= rows) return;
  const RowIdx ix = sidx[threadIdx.x];
  const int64_t r = row0 + threadIdx.x;
  const uint32_t k[5] = {static_cast<uint32_t>(ix.item), static_cast<uint32_t>(ix.act),
                         static_cast<uint32_t>(ix.pe), static_cast<uint32_t>(ix.ri_slot),
                         static_cast<uint32_t>(ix.rt)};
#pragma unroll
  for (int t = 0; t < 5; ++t) {
    keys[t * T + r] = k[t];
    vals[t * T + r] = static_cast<uint32_t>(r);
  }
}

struct SegArgs {
  const uint32_t* keys;   // sorted, 5 slices of T
  const uint32_t* vals;   // batch row of each sorted pair
  int64_t T, total;       // total = 5 T
  int nch;                // chunks of SEG pairs
  uint32_t* cnt;          // [nch] run heads per chunk, then their exclusive scan
  uint32_t* cnt_item;     // [nch] run heads in the item slice
  int32_t* n_items;       // [1] distinct items
  const void* dx;
  int d;
  int32_t* item_ids;      // [T] sparse item gradient: ids
  float* item_rows;       // [T, d] and rows
  float* dense[4];        // action, pos, ri, rt gradients
  int64_t dense_elems[4];
  float* carry_in;        // [nch, d] partial sum of a run that began in an earlier chunk
  float* carry_out;       // [nch, d] partial sum of a run that begins here and goes on
  int32_t* meta;          // [nch, 4]: flags, table, key, sparse slot of the carry_out run
};
constexpr int META_CONT_IN = 1;   // the chunk's first pair continues a run
constexpr int META_NO_HEAD = 2;   // no run starts in the chunk
constexpr int META_CARRY_OUT = 4; // the chunk's last run starts here and goes on

__device__ __forceinline__ bool seg_head(const SegArgs& g, int64_t p) {
  return p % g.T == 0 || g.keys[p] != g.keys[p - 1];
}

// One wave per chunk: count run heads (all, and in the item slice); the first waves also
// clear the dense gradients.
__global__ void __launch_bounds__(256) seg_count_kernel(SegArgs g) {
  const int64_t gt = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t nthreads = static_cast<int64_t>(gridDim.x) * 256;
  for (int t = 0; t < 4; ++t)
    for (int64_t e = gt; e < g.dense_elems[t]; e += nthreads) g.dense[t][e] = 0.f;
  const int c = static_cast<int>(gt >> 6);
  const int lane = threadIdx.x & 63;
  if (c >= g.nch) return;
  const int64_t p = static_cast<int64_t>(c) * SEG + lane;
  const bool head = p < g.total && seg_head(g, p);
  const uint64_t m = __ballot(head);
  const uint64_t mi = __ballot(head && p < g.T);
  if (lane == 0) {
    g.cnt[c] = static_cast<uint32_t>(__popcll(m));
    g.cnt_item[c] = static_cast<uint32_t>(__popcll(mi));
  }
}

// One workgroup: exclusive scan of the head counts; the number of distinct items.
__global__ void __launch_bounds__(1024) seg_scan_kernel(SegArgs g) {
  __shared__ uint32_t sw[16];
  __shared__ uint32_t si[16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t carry = 0, items = 0;
  for (int base = 0; base < g.nch; base += 1024) {
    const int c = base + static_cast<int>(threadIdx.x);
    const uint32_t x = c < g.nch ? g.cnt[c] : 0u;
    uint32_t xi = c < g.nch ? g.cnt_item[c] : 0u;
    uint32_t inc = x;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_up(inc, o);
      if (lane >= o) inc += y;
      xi += __shfl_xor(xi, o);
    }
    if (lane == 63) sw[wave] = inc;
    if (lane == 0) si[wave] = xi;
    __syncthreads();
    uint32_t pre = carry, tot = 0;
    for (int w = 0; w < 16; ++w) {
      pre += w < wave ? sw[w] : 0u;
      tot += sw[w];
      items += (threadIdx.x == 0) ? si[w] : 0u;
    }
    if (c < g.nch) g.cnt[c] = pre + inc - x;
    carry += tot;
    __syncthreads();
  }
  if (threadIdx.x == 0) *g.n_items = static_cast<int32_t>(items);
}

template <typename T>
__device__ __forceinline__ float ld_elem(const T* p);
template <>
__device__ __forceinline__ float ld_elem<bf16_t>(const bf16_t* p) {
  return __uint_as_float(static_cast<uint32_t>(*reinterpret_cast<const uint16_t*>(p)) << 16);
}
template <>
__device__ __forceinline__ float ld_elem<float>(const float* p) { return *p; }

// destination of a finished run: the sparse item row, or the dense small-table row (null
// for a slot past the table, which only ids out of range can produce)
__device__ __forceinline__ float* seg_dest(const SegArgs& g, int table, uint32_t key, uint32_t slot) {
  if (table == 0) return g.item_rows + static_cast<int64_t>(slot) * g.d;
  const int64_t off = static_cast<int64_t>(key) * g.d;
  return off < g.dense_elems[table - 1] ? g.dense[table - 1] + off : nullptr;
}

// One workgroup per chunk; thread j owns columns j, j + 256, ...  and walks the chunk's
// pairs in order, loading eight rows ahead.
template <typename T>
__global__ void __launch_bounds__(256) seg_sum_kernel(SegArgs g) {
  __shared__ uint32_t sk[SEG], sv[SEG], sslot[SEG];
  __shared__ int shead[SEG + 1];
  __shared__ int stab[SEG];
  __shared__ int sinfo[2];
  const int c = blockIdx.x;
  const int64_t p0 = static_cast<int64_t>(c) * SEG;
  const int cnt = static_cast<int>(min<int64_t>(SEG, g.total - p0));
  const int tid = threadIdx.x;
  if (tid < 64) {
    const int64_t p = p0 + tid;
    const bool valid = tid < cnt;
    const bool head = valid && seg_head(g, p);
    const uint64_t m = __ballot(head);
    if (valid) {
      const uint32_t key = g.keys[p];
      const uint32_t slot = g.cnt[c] + static_cast<uint32_t>(__popcll(m & ((1ull << tid) - 1ull)));
      sk[tid] = key;
      sv[tid] = g.vals[p];
      sslot[tid] = slot;
      shead[tid] = head ? 1 : 0;
      stab[tid] = static_cast<int>(p / g.T);
      if (head && p < g.T) g.item_ids[slot] = static_cast<int32_t>(key);
    }
    if (tid == 0) {
      const int64_t pn = p0 + SEG;
      const bool next_cont = pn < g.total && !seg_head(g, pn);
      shead[cnt] = next_cont ? 0 : 1;  // a run ending at the chunk's end goes on iff 0
      sinfo[0] = next_cont ? 1 : 0;
      sinfo[1] = (m & 1ull) ? 0 : 1;   // the first pair continues a run
    }
  }
  __syncthreads();
  const bool next_cont = sinfo[0] != 0;
  const bool cont_in = sinfo[1] != 0;
  // the last run: its first pair (or -1 for the continued run) and whether it goes on
  int last_head = -1;
  for (int i = cnt - 1; i >= 0; --i)
    if (shead[i]) { last_head = i; break; }
  if (tid == 0) {
    int32_t* mt = g.meta + 4 * c;
    int flags = (cont_in ? META_CONT_IN : 0) | (last_head < 0 ? META_NO_HEAD : 0);
    if (next_cont && last_head >= 0) {
      flags |= META_CARRY_OUT;
      mt[1] = stab[last_head];
      mt[2] = static_cast<int32_t>(sk[last_head]);
      mt[3] = static_cast<int32_t>(sslot[last_head]);
    }
    mt[0] = flags;
  }
  const T* dx = static_cast<const T*>(g.dx);
  const int64_t d = g.d;
  for (int col = tid; col < g.d; col += 256) {
    float acc = 0.f;
    int run = shead[0] ? 0 : -1;
    for (int i0 = 0; i0 < cnt; i0 += 8) {
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = i0 + j < cnt ? ld_elem<T>(dx + static_cast<int64_t>(sv[i0 + j]) * d + col) : 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int i = i0 + j;
        if (i >= cnt) break;
        acc += v[j];
        if (i + 1 == cnt || shead[i + 1]) {  // the run ends at pair i (in this chunk)
          float* dst;
          if (run < 0)
            dst = g.carry_in + static_cast<int64_t>(c) * d;
          else if (i + 1 == cnt && next_cont)
            dst = g.carry_out + static_cast<int64_t>(c) * d;
          else
            dst = seg_dest(g, stab[run], sk[run], sslot[run]);
          if (dst) dst[col] = acc;
          acc = 0.f;
          run = i + 1;
        }
      }
    }
  }
}

// One workgroup per chunk whose last run goes on: its partial plus the continuing chunks'
// partials, in chunk order.  The run's last chunk is found first (the threads test 256
// chunks at a time), then each column adds the partials with several loads in flight.
__global__ void __launch_bounds__(256) seg_fix_kernel(SegArgs g) {
  __shared__ int s_end;
  const int c = blockIdx.x;
  const int32_t* mt = g.meta + 4 * c;
  if (!(mt[0] & META_CARRY_OUT)) return;
  const int table = mt[1];
  const uint32_t key = static_cast<uint32_t>(mt[2]), slot = static_cast<uint32_t>(mt[3]);
  float* dst = seg_dest(g, table, key, slot);
  if (!dst) return;
  // chunk j (> c) holds the run's last piece unless no run starts in it and chunk j + 1
  // continues it
  if (threadIdx.x == 0) s_end = g.nch - 1;
  __syncthreads();
  for (int base = c + 1; base < g.nch; base += 256) {
    const int j = base + static_cast<int>(threadIdx.x);
    const bool ends = j < g.nch && !((g.meta[4 * j] & META_NO_HEAD) && j + 1 < g.nch &&
                                     (g.meta[4 * (j + 1)] & META_CONT_IN));
    if (ends) atomicMin(&s_end, j);
    __syncthreads();
    if (s_end < base + 256) break;  // uniform: read after the barrier
    __syncthreads();
  }
  const int j1 = s_end;
  const int64_t d = g.d;
  for (int col = threadIdx.x; col < g.d; col += 256) {
    float acc = g.carry_out[c * d + col];
    int j = c + 1;
    for (; j + 4 <= j1 + 1; j += 4) {
      const float v0 = g.carry_in[j * d + col], v1 = g.carry_in[(j + 1) * d + col];
      const float v2 = g.carry_in[(j + 2) * d + col], v3 = g.carry_in[(j + 3) * d + col];
      acc = (((acc + v0) + v1) + v2) + v3;
    }
    for (; j <= j1; ++j) acc += g.carry_in[j * d + col];
    dst[col] = acc;
  }
}

// ---- the device error word: one per GPU (file-scope device memory, located once per device
// with hipGetSymbolAddress; `error_words` names a host-side stand-in, never device memory)
static __device__ __align__(16) uint32_t error_words[4];
constexpr int ERR_MAX_DEVICES = 64;
std::once_flag err_once[ERR_MAX_DEVICES];
uint32_t* err_ptr[ERR_MAX_DEVICES];

EmbedArgs make_args(const genrank_batch* b, const genrank_inputs* in, const genrank_tables* t) {
  EmbedArgs a{};
  a.offsets = in->hist_offsets;
  a.hist_items = in->hist_items;
  a.hist_actions = in->hist_actions;
  a.hist_ts = in->hist_ts;
  a.cand_items = in->cand_items;
  a.req_ts = in->req_ts;
  a.t_item = t->item;
  a.t_action = t->action;
  a.t_pos = t->pos;
  a.t_ri = t->ri;
  a.t_rt = t->rt;
  a.rt_bounds = t->rt_bounds;
  a.B = b->B;
  a.m = b->m;
  a.d = b->d;
  a.hist_chunks = (b->max_hist + EMB_ROWS - 1) / EMB_ROWS;
  a.cand_chunks = (b->m + EMB_ROWS - 1) / EMB_ROWS;
  a.n_action = t->n_action;
  a.n_pos = t->n_pos;
  a.n_ri = t->n_ri;
  a.n_bounds = t->n_rt - 1;
  a.T_h = b->total_hist;
  const int64_t es = b->dtype == GENRANK_BF16 ? 2 : 4;
  const int64_t rb = static_cast<int64_t>(b->d) * es;
  auto clamp32 = [](int64_t v) { return static_cast<uint32_t>(v < 0xFFFFFFFFll ? v : 0xFFFFFFFFll); };
  a.bytes_item = clamp32(t->n_item * rb);
  a.bytes_action = clamp32((static_cast<int64_t>(t->n_action) + 1) * rb);
  a.bytes_pos = clamp32(static_cast<int64_t>(t->n_pos) * rb);
  a.bytes_ri = clamp32(static_cast<int64_t>(t->n_ri) * rb);
  a.bytes_rt = clamp32(static_cast<int64_t>(t->n_rt) * rb);
  a.n_item = t->n_item;
  a.err = device_error_word();
  return a;
}

dim3 grid_of(const EmbedArgs& a) {
  return dim3(static_cast<unsigned>(a.hist_chunks + a.cand_chunks), static_cast<unsigned>(a.B));
}

// the row kernel, with the action table in LDS when it is small enough; f32_out: f32 rows
// from bf16 tables (the f32 residual stream); out_bytes: the size of the output rows
template <typename T, typename TO>
void launch_rows_t(const EmbedArgs& a, bool sact, bool nt, hipStream_t stream) {
  const size_t lds = sact ? a.bytes_action : 0;
  if (sact && nt)
    hipLaunchKernelGGL((embed_sum_rows_kernel<T, TO, true, true>), grid_of(a), dim3(EMB_THREADS), lds, stream, a);
  else if (sact)
    hipLaunchKernelGGL((embed_sum_rows_kernel<T, TO, true, false>), grid_of(a), dim3(EMB_THREADS), lds, stream, a);
  else if (nt)
    hipLaunchKernelGGL((embed_sum_rows_kernel<T, TO, false, true>), grid_of(a), dim3(EMB_THREADS), 0, stream, a);
  else
    hipLaunchKernelGGL((embed_sum_rows_kernel<T, TO, false, false>), grid_of(a), dim3(EMB_THREADS), 0, stream, a);
}
void launch_rows(const EmbedArgs& a, int dtype, bool f32_out, int64_t out_bytes, hipStream_t stream) {
  const bool sact = a.bytes_action % 16 == 0 && a.bytes_action <= static_cast<uint32_t>(SACT_MAX);
  const bool nt = out_bytes > STREAM_OUT_BYTES;
  if (dtype == GENRANK_BF16 && f32_out)
    launch_rows_t<bf16_t, float>(a, sact, nt, stream);
  else if (dtype == GENRANK_BF16)
    launch_rows_t<bf16_t, bf16_t>(a, sact, nt, stream);
  else
    launch_rows_t<float, float>(a, sact, nt, stream);
}
// either gather kernel for the batch's dtype and residual-stream type
void launch_gather(const genrank_batch* b, const genrank_tables* t, const EmbedArgs& a, hipStream_t stream) {
  const int es = b->dtype == GENRANK_BF16 ? 2 : 4;
  const bool f32_out = b->dtype == GENRANK_BF16 && b->resid == GENRANK_RESID_F32;
  const int cpr = b->d * es / 16;
  // the row kernel needs whole 16-byte columns that divide the workgroup, and every table
  // and the chunk's output addressable with 32-bit offsets
  const int64_t rb = static_cast<int64_t>(b->d) * es;
  const bool rows_ok = b->d * es % 16 == 0 && cpr <= EMB_THREADS && EMB_THREADS % cpr == 0 &&
                       t->n_item * rb < 0xFFFFFFFFll && EMB_ROWS * rb * 2 < 0xFFFFFFFFll;
  const int64_t out_bytes = (a.T_h + static_cast<int64_t>(a.B) * a.m) * b->d * (f32_out ? 4 : es);
  if (rows_ok)
    launch_rows(a, b->dtype, f32_out, out_bytes, stream);
  else if (f32_out)
    hipLaunchKernelGGL((embed_sum_kernel<bf16_t, float>), grid_of(a), dim3(EMB_THREADS), 0, stream, a);
  else if (b->dtype == GENRANK_BF16)
    hipLaunchKernelGGL((embed_sum_kernel<bf16_t, bf16_t>), grid_of(a), dim3(EMB_THREADS), 0, stream, a);
  else
    hipLaunchKernelGGL((embed_sum_kernel<float, float>), grid_of(a), dim3(EMB_THREADS), 0, stream, a);
}

}  // namespace

uint32_t* device_error_word() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= ERR_MAX_DEVICES) return nullptr;
  std::call_once(err_once[dev], [dev] {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(error_words)) == hipSuccess) err_ptr[dev] = static_cast<uint32_t*>(p);
  });
  return err_ptr[dev];
}

genrank_status check_embed_args(const genrank_batch* b, const genrank_inputs* in,
                                const genrank_tables* t) {
  if (!b || !in || !t) return GENRANK_E_ARG;
  genrank_status s = check_batch(b);
  if (s != GENRANK_OK) return s;
  if (!in->hist_offsets || !in->req_ts) return GENRANK_E_ARG;
  if (b->total_hist > 0 && (!in->hist_items || !in->hist_actions || !in->hist_ts))
    return GENRANK_E_ARG;
  if (b->m > 0 && !in->cand_items) return GENRANK_E_ARG;
  if (!t->item || !t->action || !t->pos || !t->ri || !t->rt) return GENRANK_E_ARG;
  if (t->n_item < 1 || t->n_action < 1 || t->n_pos < 1 || t->n_ri < 1 || t->n_rt < 1)
    return GENRANK_E_ARG;
  if (t->n_rt - 1 > MAX_BOUNDS) return GENRANK_E_SHAPE;
  if (t->n_rt > 1 && !t->rt_bounds) return GENRANK_E_ARG;
  const int vec = (b->dtype == GENRANK_BF16) ? 8 : 4;
  if (b->d % vec != 0) return GENRANK_E_SHAPE;
  return GENRANK_OK;
}

genrank_status launch_embed_sum(const genrank_batch* b, const genrank_inputs* in,
                                const genrank_tables* t, void* out, hipStream_t stream) {
  EmbedArgs a = make_args(b, in, t);
  a.out = out;
  launch_gather(b, t, a, stream);
  GR_CHECK_LAUNCH();
  return GENRANK_OK;
}

genrank_status launch_embed_sum_cand(const genrank_batch* b, const genrank_inputs* in, const genrank_tables* t,
                                     void* out, hipStream_t stream) {
  // candidate chunks only (no history chunk in the grid), rows written from 0
  EmbedArgs a = make_args(b, in, t);
  a.hist_chunks = 0;
  a.T_h = 0;
  a.out = out;
  if (a.cand_chunks == 0) return GENRANK_OK;
  launch_gather(b, t, a, stream);
  GR_CHECK_LAUNCH();
  return GENRANK_OK;
}

genrank_status launch_debug_indices(const genrank_batch* b, const genrank_inputs* in,
                                    const genrank_tables* t, int32_t* out, hipStream_t stream) {
  EmbedArgs a = make_args(b, in, t);
  a.out = out;
  const int64_t T = b->total_hist + static_cast<int64_t>(b->B) * b->m;
  hipLaunchKernelGGL(debug_indices_kernel, grid_of(a), dim3(EMB_THREADS), 0, stream, a, T);
  GR_CHECK_LAUNCH();
  return GENRANK_OK;
}

struct EmbedBwdWs {
  uint32_t *keys, *vals, *tkeys, *tvals, *hist, *cnt, *cnt_item;
  float *carry_in, *carry_out;
  int32_t* meta;
  size_t bytes;
};

EmbedBwdWs embed_bwd_layout(const genrank_batch* b, char* base) {
  const int64_t T = b->total_hist + static_cast<int64_t>(b->B) * b->m;
  const int64_t total = 5 * T;
  const int64_t nch = (total + SEG - 1) / SEG;
  EmbedBwdWs w{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off += (bytes + 255) & ~static_cast<size_t>(255);
    return p;
  };
  w.keys = reinterpret_cast<uint32_t*>(take(total * 4));
  w.vals = reinterpret_cast<uint32_t*>(take(total * 4));
  w.tkeys = reinterpret_cast<uint32_t*>(take(total * 4));
  w.tvals = reinterpret_cast<uint32_t*>(take(total * 4));
  w.hist = reinterpret_cast<uint32_t*>(take(radix_sort_workspace(T, 5)));
  w.cnt = reinterpret_cast<uint32_t*>(take(nch * 4));
  w.cnt_item = reinterpret_cast<uint32_t*>(take(nch * 4));
  w.carry_in = reinterpret_cast<float*>(take(nch * b->d * 4));
  w.carry_out = reinterpret_cast<float*>(take(nch * b->d * 4));
  w.meta = reinterpret_cast<int32_t*>(take(nch * 16));
  w.bytes = off;
  return w;
}

size_t embed_bwd_workspace(const genrank_batch* b) { return embed_bwd_layout(b, nullptr).bytes; }

genrank_status launch_embed_bwd(const genrank_batch* b, const genrank_inputs* in, const genrank_tables* t,
                                const void* dx, int32_t* item_ids, float* item_rows, int32_t* n_items,
                                float* g_action, float* g_pos, float* g_ri, float* g_rt, void* ws,
                                hipStream_t stream) {
  const int64_t T = b->total_hist + static_cast<int64_t>(b->B) * b->m;
  EmbedBwdWs w = embed_bwd_layout(b, static_cast<char*>(ws));
  SegArgs g{};
  g.T = T;
  g.total = 5 * T;
  g.nch = static_cast<int>((g.total + SEG - 1) / SEG);
  g.n_items = n_items;
  g.dx = dx;
  g.d = b->d;
  g.item_ids = item_ids;
  g.item_rows = item_rows;
  g.dense[0] = g_action; g.dense[1] = g_pos; g.dense[2] = g_ri; g.dense[3] = g_rt;
  g.dense_elems[0] = (static_cast<int64_t>(t->n_action) + 1) * b->d;
  g.dense_elems[1] = static_cast<int64_t>(t->n_pos) * b->d;
  g.dense_elems[2] = static_cast<int64_t>(t->n_ri) * b->d;
  g.dense_elems[3] = static_cast<int64_t>(t->n_rt) * b->d;
  g.cnt = w.cnt;
  g.cnt_item = w.cnt_item;
  g.carry_in = w.carry_in;
  g.carry_out = w.carry_out;
  g.meta = w.meta;
  if (T > 0) {
    EmbedArgs a = make_args(b, in, t);
    hipLaunchKernelGGL(embed_keys_kernel, grid_of(a), dim3(EMB_THREADS), 0, stream, a, w.keys, w.vals, T);
    // key bits: the largest slot of any table
    const int64_t top = std::max<int64_t>({t->n_item - 1, t->n_action, t->n_pos - 1, t->n_ri - 1, t->n_rt - 1, 1});
    int bits = 0;
    while (bits < 32 && (top >> bits) != 0) ++bits;
    int in_tmp = 0;
    const genrank_status st = launch_radix_sort(w.keys, w.vals, w.tkeys, w.tvals, T, 5, bits, w.hist, &in_tmp, stream);
    if (st != GENRANK_OK) return st;
    g.keys = in_tmp ? w.tkeys : w.keys;
    g.vals = in_tmp ? w.tvals : w.vals;
  }
  // the count kernel also clears the dense gradients: enough threads for both jobs
  int64_t need = std::max<int64_t>(static_cast<int64_t>(g.nch) * 64, 1);
  need = std::max<int64_t>(need, std::min<int64_t>(g.dense_elems[1], int64_t(1) << 20));
  const unsigned cgrid = static_cast<unsigned>((need + 255) / 256);
  hipLaunchKernelGGL(seg_count_kernel, dim3(cgrid), dim3(256), 0, stream, g);
  hipLaunchKernelGGL(seg_scan_kernel, dim3(1), dim3(1024), 0, stream, g);
  if (T > 0) {
    if (b->dtype == GENRANK_BF16)
      hipLaunchKernelGGL(seg_sum_kernel<bf16_t>, dim3(g.nch), dim3(256), 0, stream, g);
    else
      hipLaunchKernelGGL(seg_sum_kernel<float>, dim3(g.nch), dim3(256), 0, stream, g);
    hipLaunchKernelGGL(seg_fix_kernel, dim3(g.nch), dim3(256), 0, stream, g);
  }
  GR_CHECK_LAUNCH();
  return GENRANK_OK;
}

}  // namespace genrank
