// Per-token INT8 quantization kernels for gfx950.
//
//  * dynamic quant: BF16 [M, K] -> INT8 [M, K] + fp32 scale [M]
//    ("DeepSeek-V4 W8A8 执行链从量化权重到 Ascend INT8 算子", §一 recipe
//    per_token / int8 / symmetric, §二 npu_dynamic_quant).
//  * SwiGLU + requant: BF16 h [R, 2I] -> INT8 [R, I] + fp32 scale [R]
//    (same page, §三 and §五: the fused "SwiGLU + Requant" step between the W13
//    and W2 grouped matmuls; §一: W13 = gate_proj + up_proj).
//
// One wavefront owns one row. The fast kernels keep the whole row in registers
// (CPL chunks of 8 elements per lane, 16-byte loads), reduce the row amax with
// DPP row reductions plus four readlanes, then divide every element by the
// scale and store 8 codes per chunk. Rows are independent, so four rows share a
// 256-thread workgroup and the grid is ceil(M / 4) workgroups. HBM traffic is
// one read of the input and one write of the codes.
//
// Shapes outside the fast kernels' limits (K not a multiple of 8, K > 8192,
// unaligned pointers) take a two-pass kernel with one element per lane per step.
#include "device_common.hpp"
#include "launch.hpp"

namespace w8a8 {

constexpr int kRowsPerBlock = 4;

// |BF16| bit patterns of the two halves of a 32-bit word, max-reduced.
__device__ __forceinline__ uint32_t abs_bf16_pair_max(uint32_t w) {
  return max(w & 0x7FFFu, (w >> 16) & 0x7FFFu);
}

// Store of 8 codes (row, k = 8 c .. 8 c + 7): row-major q (row stride ldq)
// when kb == 0, else the packed block layout of the weights with kb k-blocks
// per 16 rows: block (row / 16, k / 64), byte (row % 16 + 16 (k % 64 / 16)) *
// 16 + k % 16.
__device__ __forceinline__ void store_codes8(int8_t* q, int64_t row, int c, int64_t ldq, int64_t kb,
                                             uint2 o) {
  if (kb == 0) {
    reinterpret_cast<uint2*>(q + row * ldq)[c] = o;
  } else {
    const int64_t k = (int64_t)c * 8;
    const int64_t at = ((row >> 4) * kb + (k >> 6)) * 1024 + ((row & 15) + 16 * ((k & 63) >> 4)) * 16 +
                       (k & 15);
    *reinterpret_cast<uint2*>(q + at) = o;
  }
}

template <int CPL>
__global__ __launch_bounds__(256) void quant_rows_vec(const uint16_t* __restrict__ x, int64_t M,
                                                      int64_t K, int8_t* __restrict__ q,
                                                      float* __restrict__ scale, int64_t kb, int64_t ldx,
                                                      int64_t ldq) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= M) return;  // whole wave leaves together
  const int nchunk = (int)(K >> 3);
  const uint4* xr = reinterpret_cast<const uint4*>(x + row * ldx);
  uint4 v[CPL];
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = lane + i * kWave;
    if (c < nchunk) {
      v[i] = xr[c];
      amax = max(amax, max(max(abs_bf16_pair_max(v[i].x), abs_bf16_pair_max(v[i].y)),
                           max(abs_bf16_pair_max(v[i].z), abs_bf16_pair_max(v[i].w))));
    }
  }
  amax = wave_max_u32(amax);
  const float s = bf16_to_f32(amax) / 127.0f;
  if (lane == 0) scale[row] = s;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = lane + i * kWave;
    if (c < nchunk) {
      const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
      store_codes8(q, row, c, ldq, kb, quant8_bf16(w, s));
    }
  }
}

// Few rows (decode-sized M): one 1024-thread workgroup per row, so the row's
// divisions spread over 16 wavefronts instead of one. The amax is reduced per
// wavefront with DPP, then across the 16 wavefronts through LDS.
constexpr int kRowBlock = 1024;

template <int CPL>
__global__ __launch_bounds__(kRowBlock) void quant_rows_block(const uint16_t* __restrict__ x,
                                                              int64_t M, int64_t K,
                                                              int8_t* __restrict__ q,
                                                              float* __restrict__ scale, int64_t kb,
                                                              int64_t ldx, int64_t ldq) {
  __shared__ uint32_t wave_max[kRowBlock / kWave];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.x;
  const int nchunk = (int)(K >> 3);
  const uint4* xr = reinterpret_cast<const uint4*>(x + row * ldx);
  uint4 v[CPL];
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = tid + i * kRowBlock;
    if (c < nchunk) {
      v[i] = xr[c];
      amax = max(amax, max(max(abs_bf16_pair_max(v[i].x), abs_bf16_pair_max(v[i].y)),
                           max(abs_bf16_pair_max(v[i].z), abs_bf16_pair_max(v[i].w))));
    }
  }
  amax = wave_max_u32(amax);
  if (lane == 0) wave_max[wave] = amax;
  __syncthreads();
  amax = wave_max[0];
#pragma unroll
  for (int w = 1; w < kRowBlock / kWave; ++w) amax = max(amax, wave_max[w]);
  const float s = bf16_to_f32(amax) / 127.0f;
  if (tid == 0) scale[row] = s;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = tid + i * kRowBlock;
    if (c < nchunk) {
      const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
      store_codes8(q, row, c, ldq, kb, quant8_bf16(w, s));
    }
  }
}

// Packed codes for many rows: one 1024-thread workgroup per 16-row block.
// Phase 1: wavefront w takes the amax (and scale) of row 16 b + w. Phase 2:
// the workgroup walks the block's 1 KB pieces in order, thread t writing the
// 16 codes of byte range [16 t, 16 t + 16) of the row-block's blocks — a
// whole 1 KB block per wavefront store — from 16 BF16 values it re-reads (L2
// hot after phase 1). Rows past M get zero codes. K % 8 == 0.
__global__ __launch_bounds__(kRowBlock) void quant_rows16_packed(const uint16_t* __restrict__ x,
                                                                 int64_t M, int64_t K,
                                                                 int8_t* __restrict__ q,
                                                                 float* __restrict__ scale) {
  __shared__ float row_scale[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t b = blockIdx.x;
  const int64_t kb = (K + 63) / 64;
  {
    const int64_t row = b * 16 + wave;
    uint32_t amax = 0;
    if (row < M) {
      const uint4* xr = reinterpret_cast<const uint4*>(x + row * K);
      for (int64_t c = lane; c < K / 8; c += kWave) {
        const uint4 v = xr[c];
        amax = max(amax, max(max(abs_bf16_pair_max(v.x), abs_bf16_pair_max(v.y)),
                             max(abs_bf16_pair_max(v.z), abs_bf16_pair_max(v.w))));
      }
    }
    amax = wave_max_u32(amax);
    const float s = bf16_to_f32(amax) / 127.0f;
    if (lane == 0) {
      row_scale[wave] = s;
      if (row < M) scale[row] = s;
    }
  }
  __syncthreads();
  int8_t* qb = q + b * kb * 1024;
  for (int64_t t = tid; t < kb * 64; t += kRowBlock) {
    const int l = (int)(t & 63);
    const int r = l & 15;
    const int64_t row = b * 16 + r;
    const int64_t k0 = (t >> 6) * 64 + (l >> 4) * 16;
    uint4 o = uint4{0u, 0u, 0u, 0u};
    if (row < M && k0 < K) {
      const uint16_t* xr = x + row * K + k0;
      const uint4 v0 = *reinterpret_cast<const uint4*>(xr);
      const uint4 v1 = k0 + 16 <= K ? *reinterpret_cast<const uint4*>(xr + 8) : uint4{0u, 0u, 0u, 0u};
      const float s = row_scale[r];
      const uint32_t w0[4] = {v0.x, v0.y, v0.z, v0.w};
      const uint32_t w1[4] = {v1.x, v1.y, v1.z, v1.w};
      const uint2 lo = quant8_bf16(w0, s), hi = quant8_bf16(w1, s);
      o = uint4{lo.x, lo.y, hi.x, hi.y};
    }
    *reinterpret_cast<uint4*>(qb + t * 16) = o;
  }
}

// The same packed codes in one pass over x, one wavefront per row (four rows
// per 256-thread workgroup), for K <= 64 * 16 * P: lane l holds the 16-value
// pieces j = l, l + 64, ... of its row (two contiguous 16-byte loads each) in
// registers, the row amax is a wavefront reduction (no LDS, no barrier), and
// each piece's 16 codes go to their place in the row-block's 1 KB blocks
// (block j / 4, byte (r + 16 (j % 4)) * 16 for row r of the block). The
// wavefronts of rows M .. the end of the last 16-row block, and the pieces
// past K, write zero codes, so every block is written whole.
template <int P>
__global__ __launch_bounds__(256) void quant_rows_packed_wave(const uint16_t* __restrict__ x, int64_t M,
                                                              int64_t K, int8_t* __restrict__ q,
                                                              float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  // The four workgroups of a 16-row block write into the same 1 KB code
  // blocks; workgroup b runs on XCD b % 8, so when the grid allows, row block
  // indices are laid out so that those four share one XCD (and its L2)
  // instead of leaving four partial copies of each line in four L2s.
  int64_t bidx = blockIdx.x;
  if (gridDim.x % (8 * 16 / kRowsPerBlock) == 0) {
    const int64_t per = gridDim.x / 8;
    bidx = (int64_t)(blockIdx.x % 8) * per + blockIdx.x / 8;
  }
  const int64_t row = bidx * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= (M + 15) / 16 * 16) return;  // whole wave leaves together
  const int64_t kb = (K + 63) / 64, npc = kb * 4;  // 16-value pieces of a row, padding included
  const bool live = row < M;
  const uint16_t* xr = x + row * K;
  uint4 v[P][2];
  uint32_t am = 0;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int64_t k0 = (int64_t)(lane + p * kWave) * 16;
    const bool in = live && k0 < K;
    v[p][0] = in ? *reinterpret_cast<const uint4*>(xr + k0) : uint4{0u, 0u, 0u, 0u};
    v[p][1] = in && k0 + 16 <= K ? *reinterpret_cast<const uint4*>(xr + k0 + 8) : uint4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int h = 0; h < 2; ++h)
      am = max(am, max(max(abs_bf16_pair_max(v[p][h].x), abs_bf16_pair_max(v[p][h].y)),
                       max(abs_bf16_pair_max(v[p][h].z), abs_bf16_pair_max(v[p][h].w))));
  }
  am = wave_max_u32(am);
  const float s = bf16_to_f32(am) / 127.0f;
  if (lane == 0 && live) scale[row] = s;
  int8_t* qb = q + (row >> 4) * kb * 1024 + (row & 15) * 16;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int64_t j = lane + p * kWave;
    if (j >= npc) break;
    uint4 o = uint4{0u, 0u, 0u, 0u};
    if (live && j * 16 < K) {
      const uint32_t w0[4] = {v[p][0].x, v[p][0].y, v[p][0].z, v[p][0].w};
      const uint32_t w1[4] = {v[p][1].x, v[p][1].y, v[p][1].z, v[p][1].w};
      const uint2 lo = quant8_bf16(w0, s), hi = quant8_bf16(w1, s);
      o = uint4{lo.x, lo.y, hi.x, hi.y};
    }
    *reinterpret_cast<uint4*>(qb + ((j >> 2) * 64 + 16 * (j & 3)) * 16) = o;
  }
}

__global__ __launch_bounds__(256) void quant_rows_generic(const uint16_t* __restrict__ x, int64_t M,
                                                          int64_t K, int8_t* __restrict__ q,
                                                          float* __restrict__ scale, int64_t ldx, int64_t ldq) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= M) return;
  const uint16_t* xr = x + row * ldx;
  uint32_t amax = 0;
  for (int64_t k = lane; k < K; k += kWave) amax = max(amax, (uint32_t)xr[k] & 0x7FFFu);
  amax = wave_max_u32(amax);
  const float s = bf16_to_f32(amax) / 127.0f;
  if (lane == 0) scale[row] = s;
  int8_t* qr = q + row * ldq;
  for (int64_t k = lane; k < K; k += kWave) qr[k] = (int8_t)quant_code(bf16_to_f32(xr[k]), s);
}

// ---------------------------------------------------------------------------
// SwiGLU + requant
// ---------------------------------------------------------------------------
template <int CPL>
__global__ __launch_bounds__(256) void swiglu_quant_vec(const uint16_t* __restrict__ h, int64_t R,
                                                        int64_t I, int8_t* __restrict__ q,
                                                        float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= R) return;
  const int nchunk = (int)(I >> 3);
  const uint4* gr = reinterpret_cast<const uint4*>(h + row * 2 * I);
  const uint4* ur = reinterpret_cast<const uint4*>(h + row * 2 * I + I);
  float a[CPL][8];
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = lane + i * kWave;
    if (c < nchunk) {
      const uint4 g4 = gr[c];
      const uint4 u4 = ur[c];
      const uint32_t gw[4] = {g4.x, g4.y, g4.z, g4.w};
      const uint32_t uw[4] = {u4.x, u4.y, u4.z, u4.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        a[i][2 * j] = swiglu_fixed(bf16_to_f32(gw[j] & 0xFFFFu), bf16_to_f32(uw[j] & 0xFFFFu));
        a[i][2 * j + 1] = swiglu_fixed(bf16_to_f32(gw[j] >> 16), bf16_to_f32(uw[j] >> 16));
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) amax = max(amax, __float_as_uint(a[i][j]) & 0x7FFFFFFFu);
    }
  }
  amax = wave_max_u32(amax);
  const float s = __uint_as_float(amax) / 127.0f;
  if (lane == 0) scale[row] = s;
  uint2* qr = reinterpret_cast<uint2*>(q + row * I);
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = lane + i * kWave;
    if (c < nchunk) {
      qr[c] = quant8(a[i], s);
    }
  }
}

__global__ __launch_bounds__(256) void swiglu_quant_generic(const uint16_t* __restrict__ h, int64_t R,
                                                            int64_t I, int8_t* __restrict__ q,
                                                            float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= R) return;
  const uint16_t* gr = h + row * 2 * I;
  const uint16_t* ur = gr + I;
  uint32_t amax = 0;
  for (int64_t j = lane; j < I; j += kWave) {
    const float a = swiglu_fixed(bf16_to_f32(gr[j]), bf16_to_f32(ur[j]));
    amax = max(amax, __float_as_uint(a) & 0x7FFFFFFFu);
  }
  amax = wave_max_u32(amax);
  const float s = __uint_as_float(amax) / 127.0f;
  if (lane == 0) scale[row] = s;
  int8_t* qr = q + row * I;
  for (int64_t j = lane; j < I; j += kWave) {
    // recomputed: the same fp32 steps give the same bits as in the amax pass
    const float a = swiglu_fixed(bf16_to_f32(gr[j]), bf16_to_f32(ur[j]));
    qr[j] = (int8_t)quant_code(a, s);
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
static inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

hipError_t launch_dynamic_quant(const uint16_t* x, int64_t M, int64_t K, int8_t* q, float* scale,
                                bool packed, hipStream_t stream, int64_t ldx, int64_t ldq) {
  if (M == 0) return hipSuccess;
  if (ldx == 0) ldx = K;
  if (ldq == 0) ldq = K;
  const dim3 grid((unsigned)((M + kRowsPerBlock - 1) / kRowsPerBlock)), block(256);
  // 16-byte loads and 8-byte code stores need aligned rows
  const bool vec = (K % 8 == 0) && (ldx % 8 == 0) && (packed || ldq % 8 == 0) && aligned(x, 16) &&
                   aligned(q, 8);
  // packed codes need the vector kernels (the caller checks K % 16 == 0 and alignment)
  if (packed && !vec) return hipErrorInvalidValue;
  // the packed kernels read x with row stride K
  if (packed && ldx != K) return hipErrorInvalidValue;
  const int64_t kb = packed ? (K + 63) / 64 : 0;
  if (packed && M > 512) {
    // many rows: one pass over x, a wavefront per row, while a lane's pieces
    // fit in registers (K <= 8192); else the two-pass 16-row kernel
    const dim3 gw((unsigned)(((M + 15) / 16 * 16 + kRowsPerBlock - 1) / kRowsPerBlock));
    switch ((kb * 4 + kWave - 1) / kWave) {
#define W8A8_QPW(P)                                                                                  \
  case P:                                                                                            \
    hipLaunchKernelGGL(quant_rows_packed_wave<P>, gw, dim3(256), 0, stream, x, M, K, q, scale);      \
    break;
      W8A8_QPW(1) W8A8_QPW(2) W8A8_QPW(3) W8A8_QPW(4) W8A8_QPW(5) W8A8_QPW(6) W8A8_QPW(7) W8A8_QPW(8)
#undef W8A8_QPW
      default:
        hipLaunchKernelGGL(quant_rows16_packed, dim3((unsigned)((M + 15) / 16)), dim3(kRowBlock), 0, stream, x,
                           M, K, q, scale);
    }
    return hipGetLastError();
  }
  const int64_t chunks = K / 8;
  if (vec && M <= 512 && chunks <= 2 * kRowBlock) {
    // few rows: a whole workgroup per row
    if (chunks <= kRowBlock)
      hipLaunchKernelGGL(quant_rows_block<1>, dim3((unsigned)M), dim3(kRowBlock), 0, stream, x, M,
                         K, q, scale, kb, ldx, ldq);
    else
      hipLaunchKernelGGL(quant_rows_block<2>, dim3((unsigned)M), dim3(kRowBlock), 0, stream, x, M,
                         K, q, scale, kb, ldx, ldq);
  } else if (vec && chunks <= 64 * 1)
    hipLaunchKernelGGL(quant_rows_vec<1>, grid, block, 0, stream, x, M, K, q, scale, kb, ldx, ldq);
  else if (vec && chunks <= 64 * 2)
    hipLaunchKernelGGL(quant_rows_vec<2>, grid, block, 0, stream, x, M, K, q, scale, kb, ldx, ldq);
  else if (vec && chunks <= 64 * 4)
    hipLaunchKernelGGL(quant_rows_vec<4>, grid, block, 0, stream, x, M, K, q, scale, kb, ldx, ldq);
  else if (vec && chunks <= 64 * 8)
    hipLaunchKernelGGL(quant_rows_vec<8>, grid, block, 0, stream, x, M, K, q, scale, kb, ldx, ldq);
  else if (vec && chunks <= 64 * 16)
    hipLaunchKernelGGL(quant_rows_vec<16>, grid, block, 0, stream, x, M, K, q, scale, kb, ldx, ldq);
  else
    hipLaunchKernelGGL(quant_rows_generic, grid, block, 0, stream, x, M, K, q, scale, ldx, ldq);
  return hipGetLastError();
}

hipError_t launch_swiglu_quant(const uint16_t* h, int64_t R, int64_t I, int8_t* q, float* scale,
                               hipStream_t stream) {
  if (R == 0) return hipSuccess;
  const dim3 grid((unsigned)((R + kRowsPerBlock - 1) / kRowsPerBlock)), block(256);
  const bool vec = (I % 8 == 0) && aligned(h, 16) && aligned(q, 8);
  const int64_t chunks = I / 8;
  if (vec && chunks <= 64 * 1)
    hipLaunchKernelGGL(swiglu_quant_vec<1>, grid, block, 0, stream, h, R, I, q, scale);
  else if (vec && chunks <= 64 * 2)
    hipLaunchKernelGGL(swiglu_quant_vec<2>, grid, block, 0, stream, h, R, I, q, scale);
  else if (vec && chunks <= 64 * 4)
    hipLaunchKernelGGL(swiglu_quant_vec<4>, grid, block, 0, stream, h, R, I, q, scale);
  else if (vec && chunks <= 64 * 8)
    hipLaunchKernelGGL(swiglu_quant_vec<8>, grid, block, 0, stream, h, R, I, q, scale);
  else
    hipLaunchKernelGGL(swiglu_quant_generic, grid, block, 0, stream, h, R, I, q, scale);
  return hipGetLastError();
}

}  // namespace w8a8
