// The steps on either side of the MoE chain on one GPU ("DeepSeek-V4 W8A8 执行链
// 从量化权重到 Ascend INT8 算子", §三: the INT8 dispatch moves INT8 hidden states
// with one scale per token, plus topk_ids, topk_weights and the per-expert
// token counts, and the runner feeds them to W13 without quantizing again).
//
//   route:   (token, slot) expert ids -> per-expert counts (group_list), the
//            token of every expert-major row, and the row of every pair; rows
//            of one expert keep the order of their pair index t * top_k + j;
//            ids outside [0, E) are dropped (pair row -1).
//   gather:  INT8 codes and scales of the tokens (quantized once) -> rows.
//   combine: out[t] = BF16(sum over slots j in order of fl32(w[t, j] * y_row)),
//            one fp32 rounding per product and per sum, from +0.0.
#include <algorithm>

#include "device_common.hpp"
#include "launch.hpp"

namespace w8a8 {

constexpr int kRouteThreads = 1024, kRouteWaves = kRouteThreads / kWave;
constexpr int kMaxExpertsDev = 1024;  // one scan value per thread; ids need 10 bits

// Lanes of the wavefront whose key (0 .. 2^11 - 1) equals this lane's: one
// ballot per bit. Every lane of the wavefront must take part.
__device__ __forceinline__ uint64_t match_lanes(int key) {
  uint64_t same = ~0ull;
#pragma unroll
  for (int bit = 0; bit < 11; ++bit) {
    const int mine = (key >> bit) & 1;
    const uint64_t b = __ballot(mine);
    same &= mine ? b : ~b;
  }
  return same;
}

// Exclusive scan over the workgroup of one value per thread: off[t] for
// threads t < E. Every thread of the workgroup must take part.
__device__ __forceinline__ void route_scan_block(int c, int E, int* off, int* wsum, int tid, int lane,
                                                 int wave) {
  int incl = c;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int o = __shfl_up(incl, d, kWave);
    if (lane >= d) incl += o;
  }
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  for (int w = 0; w < wave; ++w) incl += wsum[w];
  if (tid < E) off[tid] = incl - c;
}

// Places the pairs of the chunk that starts at pair c0: a pair's row is its
// expert's offset off[e], plus base[e] (that expert's pairs in earlier
// chunks), plus its pairs in earlier wavefronts of this chunk and in earlier
// lanes of its wavefront. Lanes with the same expert are found with one
// ballot per bit of the id, so the order is the pair order. wcnt must be
// zero; off and base are read after this function's barrier.
__device__ __forceinline__ void route_place_chunk(const int32_t* __restrict__ ids, int64_t P, int k, int E,
                                                  int64_t c0, const int* off, const int* base,
                                                  unsigned char (*wcnt)[kMaxExpertsDev],
                                                  int32_t* __restrict__ row_token,
                                                  int32_t* __restrict__ pair_row, int tid, int lane,
                                                  int wave) {
  const int64_t i = c0 + tid;
  const int e = i < P ? ids[i] : -1;
  const bool valid = e >= 0 && e < E;
  const uint64_t same = match_lanes(valid ? e : kMaxExpertsDev);
  const int before = __popcll(same & ((1ull << lane) - 1ull));
  if (valid && before == 0) wcnt[wave][e] = (unsigned char)__popcll(same);
  __syncthreads();
  if (valid) {
    int pos = off[e] + base[e] + before;
    for (int w = 0; w < wave; ++w) pos += wcnt[w][e];
    row_token[pos] = (int32_t)(i / k);
    pair_row[i] = pos;
  } else if (i < P) {
    pair_row[i] = -1;
  }
}

// Few chunks (at most kRouteDirectChunks of 1024 pairs, E <= 1024): one
// launch, one workgroup per chunk, and every workgroup counts all pairs itself
// in LDS (per-expert totals, and the counts of the pairs before its chunk),
// scans the totals into expert offsets and places its chunk. Row slots past
// the number of routed pairs get token 0 (a valid index for a gather over all
// T * top_k rows).
constexpr int kRouteDirectChunks = 32;

__global__ __launch_bounds__(kRouteThreads) void route_kernel(const int32_t* __restrict__ ids,
                                                              int64_t P, int k, int E,
                                                              int64_t* __restrict__ group_list,
                                                              int32_t* __restrict__ row_token,
                                                              int32_t* __restrict__ pair_row) {
  __shared__ int tot[kMaxExpertsDev];
  __shared__ int pre[kMaxExpertsDev];
  __shared__ int off[kMaxExpertsDev];
  __shared__ __align__(16) unsigned char wcnt[kRouteWaves][kMaxExpertsDev];
  __shared__ int wsum[kRouteWaves];
  static_assert(kRouteWaves * kMaxExpertsDev == 16 * kRouteThreads, "one 16-byte clear per thread");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t c0 = (int64_t)blockIdx.x * kRouteThreads;
  for (int e = tid; e < E; e += kRouteThreads) {
    tot[e] = 0;
    pre[e] = 0;
  }
  reinterpret_cast<uint4*>(&wcnt[0][0])[tid] = uint4{0u, 0u, 0u, 0u};
  __syncthreads();
  auto count = [&](int e, int64_t i) {
    if (e >= 0 && e < E) {
      atomicAdd(&tot[e], 1);
      if (i < c0) atomicAdd(&pre[e], 1);
    }
  };
  // four ids per 16-byte load when the array allows it (a thread's loads of one
  // step issued before its atomics), the rest one by one
  const int64_t P4 = (reinterpret_cast<uintptr_t>(ids) & 15) == 0 ? P / 4 : 0;
  constexpr int kBatch = 4;
  for (int64_t v0 = tid; v0 < P4; v0 += kBatch * kRouteThreads) {
    int4 q[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int64_t v = v0 + (int64_t)u * kRouteThreads;
      q[u] = v < P4 ? reinterpret_cast<const int4*>(ids)[v] : int4{-1, -1, -1, -1};
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int64_t v = v0 + (int64_t)u * kRouteThreads;
      count(q[u].x, 4 * v);
      count(q[u].y, 4 * v + 1);
      count(q[u].z, 4 * v + 2);
      count(q[u].w, 4 * v + 3);
    }
  }
  for (int64_t i = 4 * P4 + tid; i < P; i += kRouteThreads) count(ids[i], i);
  __syncthreads();
  const int c = tid < E ? tot[tid] : 0;
  route_scan_block(c, E, off, wsum, tid, lane, wave);
  if (blockIdx.x == 0 && tid < E) group_list[tid] = c;
  route_place_chunk(ids, P, k, E, c0, off, pre, wcnt, row_token, pair_row, tid, lane, wave);
  const int routed = off[E - 1] + tot[E - 1];
  for (int64_t p = routed + c0 + tid; p < P; p += (int64_t)gridDim.x * kRouteThreads)
    row_token[p] = 0;
}

// Many chunks: three launches whose work grows linearly with the pairs, and
// no workspace. The per-chunk expert counts of the C - 1 full chunks live in
// pair_row, chunk c's E counts in pair_row[1024 c .. 1024 c + E) (its own
// pairs' slots, E <= 1024), until the place step of that chunk overwrites
// them with the pairs' rows.
//   count: chunk c < C - 1 counts its pairs per expert into its slots.
//   scan:  per expert, the counts are replaced by their exclusive prefix over
//          the chunks, and group_list gets the expert's total (the last,
//          possibly partial, chunk counted directly).
//   place: chunk c reads its prefixes (the last chunk: total minus its own
//          counts), scans group_list into expert offsets and places its pairs.
__global__ __launch_bounds__(kRouteThreads) void route_count_kernel(const int32_t* __restrict__ ids, int E,
                                                                    int32_t* __restrict__ table) {
  __shared__ int cnt[kMaxExpertsDev];
  const int tid = threadIdx.x;
  const int64_t c0 = (int64_t)blockIdx.x * kRouteThreads;  // a full chunk: every id is in range
  if (tid < E) cnt[tid] = 0;
  __syncthreads();
  const int e = ids[c0 + tid];
  if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  __syncthreads();
  if (tid < E) table[c0 + tid] = cnt[tid];
}

// kWave experts per workgroup: lane = expert, wavefront = a contiguous slice
// of the full chunks.
__global__ __launch_bounds__(kRouteThreads) void route_scan_kernel(const int32_t* __restrict__ ids, int64_t P,
                                                                   int E, int nfull,
                                                                   int64_t* __restrict__ group_list,
                                                                   int32_t* __restrict__ table) {
  __shared__ int ssum[kRouteWaves][kWave];
  __shared__ int last[kWave];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int e0 = blockIdx.x * kWave, e = e0 + lane;
  if (tid < kWave) last[tid] = 0;
  const int per = (nfull + kRouteWaves - 1) / kRouteWaves;
  const int cb = min(wave * per, nfull), ce = min(cb + per, nfull);
  int s = 0;
  if (e < E) {
#pragma unroll 8
    for (int c = cb; c < ce; ++c) s += table[(int64_t)c * kRouteThreads + e];
  }
  ssum[wave][lane] = s;
  __syncthreads();
  // the last chunk's pairs of this workgroup's experts
  const int64_t i = (int64_t)nfull * kRouteThreads + tid;
  if (i < P) {
    const int id = ids[i];
    if (id >= e0 && id < e0 + kWave && id < E) atomicAdd(&last[id - e0], 1);
  }
  int run = 0;
  for (int w = 0; w < wave; ++w) run += ssum[w][lane];
  if (e < E) {
#pragma unroll 8
    for (int c = cb; c < ce; ++c) {
      const int64_t o = (int64_t)c * kRouteThreads + e;
      const int v = table[o];
      table[o] = run;
      run += v;
    }
  }
  __syncthreads();
  // the last wavefront's running sum is the total over all full chunks
  if (wave == kRouteWaves - 1 && e < E) group_list[e] = (int64_t)run + last[lane];
}

__global__ __launch_bounds__(kRouteThreads) void route_place_kernel(const int32_t* __restrict__ ids,
                                                                    int64_t P, int k, int E, int nfull,
                                                                    const int64_t* __restrict__ group_list,
                                                                    int32_t* __restrict__ row_token,
                                                                    int32_t* __restrict__ pair_row) {
  __shared__ int tot[kMaxExpertsDev];
  __shared__ int base[kMaxExpertsDev];
  __shared__ int off[kMaxExpertsDev];
  __shared__ __align__(16) unsigned char wcnt[kRouteWaves][kMaxExpertsDev];
  __shared__ int wsum[kRouteWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t c0 = (int64_t)blockIdx.x * kRouteThreads;
  const bool is_last = (int)blockIdx.x == nfull;
  reinterpret_cast<uint4*>(&wcnt[0][0])[tid] = uint4{0u, 0u, 0u, 0u};
  const int g = tid < E ? (int)group_list[tid] : 0;
  if (tid < E) {
    tot[tid] = g;
    // a full chunk's prefixes, read before the barrier below: the place
    // step then overwrites these slots
    base[tid] = is_last ? 0 : pair_row[c0 + tid];
  }
  __syncthreads();
  if (is_last) {
    const int64_t i = c0 + tid;
    const int e = i < P ? ids[i] : -1;
    if (e >= 0 && e < E) atomicAdd(&base[e], 1);
    __syncthreads();
    if (tid < E) base[tid] = g - base[tid];
  }
  route_scan_block(g, E, off, wsum, tid, lane, wave);
  route_place_chunk(ids, P, k, E, c0, off, base, wcnt, row_token, pair_row, tid, lane, wave);
  const int routed = off[E - 1] + tot[E - 1];
  for (int64_t p = routed + c0 + tid; p < P; p += (int64_t)gridDim.x * kRouteThreads)
    row_token[p] = 0;
}

// rows[p] = src[row_token[p]] (H bytes per row) and their scales; a token
// outside [0, T) gives a zero row with scale 0. kGatherRows rows per
// workgroup, every thread loading its piece of each row before storing any,
// 16-byte pieces when H % 16 == 0 and the buffers allow it.
constexpr int kGatherRows = 4;

__global__ __launch_bounds__(256) void gather_rows_kernel(const int8_t* __restrict__ q,
                                                          const float* __restrict__ scale,
                                                          const int32_t* __restrict__ row_token,
                                                          int64_t T, int64_t R, int64_t H, bool vec,
                                                          int8_t* __restrict__ q_rows,
                                                          float* __restrict__ s_rows) {
  const int64_t p0 = (int64_t)blockIdx.x * kGatherRows;
  int64_t t[kGatherRows];
  bool in[kGatherRows];
#pragma unroll
  for (int r = 0; r < kGatherRows; ++r) {
    const bool live = p0 + r < R;
    t[r] = live ? row_token[p0 + r] : 0;
    in[r] = live && t[r] >= 0 && t[r] < T;
    if (live && threadIdx.x == 0) s_rows[p0 + r] = in[r] ? scale[t[r]] : 0.f;
  }
  if (vec) {
    const int64_t per = H / 16;
    for (int64_t c = threadIdx.x; c < per; c += 256) {
      uint4 v[kGatherRows];
#pragma unroll
      for (int r = 0; r < kGatherRows; ++r)
        v[r] = in[r] ? reinterpret_cast<const uint4*>(q + t[r] * H)[c] : uint4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int r = 0; r < kGatherRows; ++r)
        if (p0 + r < R) reinterpret_cast<uint4*>(q_rows + (p0 + r) * H)[c] = v[r];
    }
  } else {
    for (int64_t c = threadIdx.x; c < H; c += 256) {
#pragma unroll
      for (int r = 0; r < kGatherRows; ++r)
        if (p0 + r < R) q_rows[(p0 + r) * H + c] = in[r] ? q[t[r] * H + c] : (int8_t)0;
    }
  }
}

// One 256-thread workgroup per token, 8 BF16 values per thread and step. The
// rows of up to kCombineSlots slots are loaded before the sum, which then
// runs in slot order; pair rows outside [0, R) contribute nothing.
constexpr int kCombineSlots = 8;

__device__ __forceinline__ void combine_add(float (&acc)[8], float w, const uint4& v) {
  const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const float a = w * bf16_to_f32(u[h] & 0xFFFFu);
    const float b = w * bf16_to_f32(u[h] >> 16);
    acc[2 * h] = acc[2 * h] + a;
    acc[2 * h + 1] = acc[2 * h + 1] + b;
  }
}

__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ y,
                                                      const int32_t* __restrict__ pair_row,
                                                      const float* __restrict__ wts, int64_t T,
                                                      int k, int64_t R, int64_t H, bool vec,
                                                      uint16_t* __restrict__ out) {
  const int64_t t = blockIdx.x;
  if (t >= T) return;
  if (vec) {
    for (int64_t c = threadIdx.x; c < H / 8; c += 256) {
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      for (int j0 = 0; j0 < k; j0 += kCombineSlots) {
        uint4 v[kCombineSlots];
        float w[kCombineSlots];
        bool use[kCombineSlots];
#pragma unroll
        for (int j = 0; j < kCombineSlots; ++j) {
          const int32_t p = j0 + j < k ? pair_row[t * k + j0 + j] : -1;
          use[j] = p >= 0 && p < R;
          w[j] = use[j] ? wts[t * k + j0 + j] : 0.f;
          v[j] = use[j] ? reinterpret_cast<const uint4*>(y + (int64_t)p * H)[c]
                        : uint4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int j = 0; j < kCombineSlots; ++j)
          if (use[j]) combine_add(acc, w[j], v[j]);
      }
      uint4 o;
      o.x = f32_to_bf16(acc[0]) | (f32_to_bf16(acc[1]) << 16);
      o.y = f32_to_bf16(acc[2]) | (f32_to_bf16(acc[3]) << 16);
      o.z = f32_to_bf16(acc[4]) | (f32_to_bf16(acc[5]) << 16);
      o.w = f32_to_bf16(acc[6]) | (f32_to_bf16(acc[7]) << 16);
      reinterpret_cast<uint4*>(out + t * H)[c] = o;
    }
  } else {
    for (int64_t h = threadIdx.x; h < H; h += 256) {
      float acc = 0.f;
      for (int j = 0; j < k; ++j) {
        const int32_t p = pair_row[t * k + j];
        if (p < 0 || p >= R) continue;
        const float a = wts[t * k + j] * bf16_to_f32(y[(int64_t)p * H + h]);
        acc = acc + a;
      }
      out[t * H + h] = (uint16_t)f32_to_bf16(acc);
    }
  }
}

static inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

hipError_t launch_route(const int32_t* ids, int64_t T, int64_t k, int64_t E, int64_t* group_list,
                        int32_t* row_token, int32_t* pair_row, hipStream_t stream) {
  // T == 0 still runs one workgroup: it writes the zero counts
  const int64_t P = T * k;
  const int64_t chunks = std::max<int64_t>(1, (P + kRouteThreads - 1) / kRouteThreads);
  if (chunks <= kRouteDirectChunks) {
    hipLaunchKernelGGL(route_kernel, dim3((unsigned)chunks), dim3(kRouteThreads), 0, stream, ids, P,
                       (int)k, (int)E, group_list, row_token, pair_row);
    return hipGetLastError();
  }
  const int nfull = (int)(chunks - 1);
  hipLaunchKernelGGL(route_count_kernel, dim3((unsigned)nfull), dim3(kRouteThreads), 0, stream, ids, (int)E,
                     pair_row);
  hipLaunchKernelGGL(route_scan_kernel, dim3((unsigned)((E + kWave - 1) / kWave)), dim3(kRouteThreads), 0,
                     stream, ids, P, (int)E, nfull, group_list, pair_row);
  hipLaunchKernelGGL(route_place_kernel, dim3((unsigned)chunks), dim3(kRouteThreads), 0, stream, ids, P,
                     (int)k, (int)E, nfull, group_list, row_token, pair_row);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const int8_t* q, const float* scale, const int32_t* row_token,
                              int64_t T, int64_t R, int64_t H, int8_t* q_rows, float* s_rows,
                              hipStream_t stream) {
  if (R == 0) return hipSuccess;
  const bool vec = H % 16 == 0 && aligned(q, 16) && aligned(q_rows, 16);
  const int64_t grid = (R + kGatherRows - 1) / kGatherRows;
  hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)grid), dim3(256), 0, stream, q, scale,
                     row_token, T, R, H, vec, q_rows, s_rows);
  return hipGetLastError();
}

hipError_t launch_combine(const uint16_t* y, const int32_t* pair_row, const float* wts, int64_t T,
                          int64_t k, int64_t R, int64_t H, uint16_t* out, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const bool vec = H % 8 == 0 && aligned(y, 16) && aligned(out, 16);
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)T), dim3(256), 0, stream, y, pair_row, wts, T,
                     (int)k, R, H, vec, out);
  return hipGetLastError();
}

}  // namespace w8a8
