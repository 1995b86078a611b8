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
constexpr int kMaxExpertsDev = 1024;  // one scan value per thread

// One 1024-thread workgroup (E <= 1024). Counts with LDS atomics, exclusive
// scan, then the pairs in chunks of 1024: a pair's place within its expert is
// the expert's count from earlier chunks, plus those of earlier wavefronts in
// the chunk, plus those of earlier lanes in its wavefront (shuffles), so the
// order is the pair order. Row slots past the number of routed pairs get
// token 0 (a valid index for a gather over all T * top_k rows).
__global__ __launch_bounds__(kRouteThreads) void route_kernel(const int32_t* __restrict__ ids,
                                                              int64_t P, int k, int E,
                                                              int64_t* __restrict__ group_list,
                                                              int32_t* __restrict__ row_token,
                                                              int32_t* __restrict__ pair_row) {
  __shared__ int cnt[kMaxExpertsDev];
  __shared__ int off[kMaxExpertsDev];
  __shared__ int base[kMaxExpertsDev];
  __shared__ unsigned char wcnt[kRouteWaves][kMaxExpertsDev];
  __shared__ int wsum[kRouteWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < E; e += kRouteThreads) {
    cnt[e] = 0;
    base[e] = 0;
  }
  for (int i = tid; i < kRouteWaves * kMaxExpertsDev; i += kRouteThreads) (&wcnt[0][0])[i] = 0;
  __syncthreads();
  for (int64_t i = tid; i < P; i += kRouteThreads) {
    const int e = ids[i];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  // exclusive scan of cnt[0 .. E) (one value per thread)
  const int c = tid < E ? cnt[tid] : 0;
  int incl = c;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int o = __shfl_up(incl, d, kWave);
    if (lane >= d) incl += o;
  }
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  for (int w = 0; w < wave; ++w) incl += wsum[w];
  if (tid < E) {
    off[tid] = incl - c;
    group_list[tid] = c;
  }
  __syncthreads();
  const int routed = off[E - 1] + cnt[E - 1];
  for (int64_t c0 = 0; c0 < P; c0 += kRouteThreads) {
    const int64_t i = c0 + tid;
    int e = -1;
    if (i < P) {
      e = ids[i];
      if (e < 0 || e >= E) e = -1;
    }
    int before = 0, total = 0;
    for (int d = 0; d < kWave; ++d) {
      const int ed = __shfl(e, d, kWave);
      const int same = (ed == e) ? 1 : 0;
      before += (d < lane) ? same : 0;
      total += same;
    }
    if (e >= 0 && before == 0) wcnt[wave][e] = (unsigned char)total;
    __syncthreads();
    if (e >= 0) {
      int pos = off[e] + base[e] + before;
      for (int w = 0; w < wave; ++w) pos += wcnt[w][e];
      row_token[pos] = (int32_t)(i / k);
      pair_row[i] = pos;
    } else if (i < P) {
      pair_row[i] = -1;
    }
    __syncthreads();
    for (int ee = tid; ee < E; ee += kRouteThreads) {
      int s = 0;
#pragma unroll
      for (int w = 0; w < kRouteWaves; ++w) {
        s += wcnt[w][ee];
        wcnt[w][ee] = 0;
      }
      base[ee] += s;
    }
    __syncthreads();
  }
  for (int64_t p = routed + tid; p < P; p += kRouteThreads) row_token[p] = 0;
}

// rows[p] = src[row_token[p]] (H bytes per row) and their scales; 16-byte
// pieces when H % 16 == 0 and the buffers allow it. A token outside [0, T)
// gives a zero row with scale 0.
__global__ __launch_bounds__(256) void gather_rows_kernel(const int8_t* __restrict__ q,
                                                          const float* __restrict__ scale,
                                                          const int32_t* __restrict__ row_token,
                                                          int64_t T, int64_t R, int64_t H, bool vec,
                                                          int8_t* __restrict__ q_rows,
                                                          float* __restrict__ s_rows) {
  const int64_t per = vec ? H / 16 : H;
  const int64_t total = R * per;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x; g < total; g += stride) {
    const int64_t p = g / per, c = g % per;
    const int64_t t = row_token[p];
    const bool in = t >= 0 && t < T;
    if (vec) {
      reinterpret_cast<uint4*>(q_rows + p * H)[c] =
          in ? reinterpret_cast<const uint4*>(q + t * H)[c] : uint4{0u, 0u, 0u, 0u};
    } else {
      q_rows[p * H + c] = in ? q[t * H + c] : (int8_t)0;
    }
    if (c == 0) s_rows[p] = in ? scale[t] : 0.f;
  }
}

// One 256-thread workgroup per token, 8 BF16 values per thread and step. Pair
// rows outside [0, R) contribute nothing.
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
      for (int j = 0; j < k; ++j) {
        const int32_t p = pair_row[t * k + j];
        if (p < 0 || p >= R) continue;
        const float w = wts[t * k + j];
        const uint4 v = reinterpret_cast<const uint4*>(y + (int64_t)p * H)[c];
        const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const float a = w * bf16_to_f32(u[h] & 0xFFFFu);
          const float b = w * bf16_to_f32(u[h] >> 16);
          acc[2 * h] = acc[2 * h] + a;
          acc[2 * h + 1] = acc[2 * h + 1] + b;
        }
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
  // T == 0 still runs: it writes the zero counts
  hipLaunchKernelGGL(route_kernel, dim3(1), dim3(kRouteThreads), 0, stream, ids, T * k, (int)k,
                     (int)E, group_list, row_token, pair_row);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const int8_t* q, const float* scale, const int32_t* row_token,
                              int64_t T, int64_t R, int64_t H, int8_t* q_rows, float* s_rows,
                              hipStream_t stream) {
  if (R == 0) return hipSuccess;
  const bool vec = H % 16 == 0 && aligned(q, 16) && aligned(q_rows, 16);
  const int64_t total = R * (vec ? H / 16 : H);
  const int64_t grid = std::min<int64_t>((total + 255) / 256, 256 * 32);
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
