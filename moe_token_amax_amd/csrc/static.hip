// Static W8A8 ("DeepSeek-V4 W8A8 执行链从量化权重到 Ascend INT8 算子", the
// static W8A8 comparison at the end of the page): the activation is quantized
// with a fixed per-tensor scale and offset, and the matmul takes a per-channel
// dequant scale (input_scale * weight_scale) and an integer bias that folds in
// both the floating bias and the offset's correction,
//   quant_bias = round(fp_bias / deq_scale - (sum_k Qw[n, k]) * input_offset).
// The product itself is the dense GEMM of gemm.hip with its static epilogue
// (fp32(acc + quant_bias) * deq_scale -> BF16).
//
// Readings of the steps the page leaves open (one IEEE fp32 rounding per
// operation, round half to even, no fused multiply-add):
//   code = clamp(rint(fl32(fl32(x / input_scale) + input_offset)), -128, 127);
//   deq_scale = fl32(input_scale * w_scale[n]);
//   correction = fl32(fp32(S_n) * input_offset), S_n the exact row sum;
//   quant_bias = saturate_int32(rint(fl32(fl32(fp_bias / deq_scale) - correction))).
#include <algorithm>

#include "device_common.hpp"
#include "launch.hpp"

namespace w8a8 {

__device__ __forceinline__ int static_code(float x, float s, float o) {
  float t = x / s;  // IEEE division
  t = t + o;
  t = __builtin_rintf(t);
  t = fminf(fmaxf(t, -128.0f), 127.0f);
  return (int)t;
}

// 8 elements per thread (16-byte BF16 loads, 8-byte code stores), grid-stride.
__global__ __launch_bounds__(256) void static_quant_vec(const uint16_t* __restrict__ x, int64_t n8,
                                                        float s, float o, int8_t* __restrict__ q) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < n8; c += stride) {
    const uint4 v = reinterpret_cast<const uint4*>(x)[c];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    int code[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      code[2 * j] = static_code(bf16_to_f32(w[j] & 0xFFFFu), s, o);
      code[2 * j + 1] = static_code(bf16_to_f32(w[j] >> 16), s, o);
    }
    reinterpret_cast<uint2*>(q)[c] =
        uint2{pack4(code[0], code[1], code[2], code[3]), pack4(code[4], code[5], code[6], code[7])};
  }
}

// Any size or alignment: one element per thread, grid-stride.
__global__ __launch_bounds__(256) void static_quant_generic(const uint16_t* __restrict__ x, int64_t n,
                                                            float s, float o, int8_t* __restrict__ q) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride)
    q[i] = (int8_t)static_code(bf16_to_f32(x[i]), s, o);
}

// Codes in the packed block layout of the weight (1 KB blocks [ceil(M/16)][KB],
// byte 16 l + j of a block = row 16 b + l % 16, column 64 kb + 16 (l / 16) + j;
// rows past M and columns past K are zero), which the GEMM kernels read as
// whole blocks. One thread per 16-byte piece; 16-byte BF16 loads when K % 8 == 0
// and x is 16-byte aligned.
__global__ __launch_bounds__(256) void static_quant_packed_kernel(const uint16_t* __restrict__ x,
                                                                  int64_t M, int64_t K, int KB,
                                                                  float s, float o, bool vec,
                                                                  int8_t* __restrict__ q) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (M + 15) / 16 * KB * 64;
  if (gid >= total) return;
  const int l = (int)(gid & 63);
  const int64_t blk = gid >> 6;
  const int64_t row = (blk / KB) * 16 + (l & 15);
  const int64_t k0 = (blk % KB) * 64 + (l >> 4) * 16;
  uint32_t w[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};  // 16 BF16 values, zero past K
  if (row < M && k0 < K) {
    const uint16_t* src = x + row * K + k0;
    if (vec) {
      const uint4 v0 = *reinterpret_cast<const uint4*>(src);
      w[0] = v0.x, w[1] = v0.y, w[2] = v0.z, w[3] = v0.w;
      if (k0 + 8 < K) {
        const uint4 v1 = *reinterpret_cast<const uint4*>(src + 8);
        w[4] = v1.x, w[5] = v1.y, w[6] = v1.z, w[7] = v1.w;
      }
    } else {
      for (int j = 0; j < 16 && k0 + j < K; ++j) w[j >> 1] |= (uint32_t)src[j] << (16 * (j & 1));
    }
  }
  int code[16];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    code[2 * j] = static_code(bf16_to_f32(w[j] & 0xFFFFu), s, o);
    code[2 * j + 1] = static_code(bf16_to_f32(w[j] >> 16), s, o);
  }
  // pieces past M or K hold zero codes (their values feed only unstored rows
  // or meet the weight's zero padding)
  const int64_t valid = (row < M) ? min((int64_t)16, K - k0) : 0;
#pragma unroll
  for (int j = 0; j < 16; ++j)
    if (j >= valid) code[j] = 0;
  *reinterpret_cast<uint4*>(q + gid * 16) =
      uint4{pack4(code[0], code[1], code[2], code[3]), pack4(code[4], code[5], code[6], code[7]),
            pack4(code[8], code[9], code[10], code[11]), pack4(code[12], code[13], code[14], code[15])};
}

// One wavefront per weight row: exact integer row sum, then the row's dequant
// scale and integer bias.
__global__ __launch_bounds__(256) void static_prepare_kernel(const int8_t* __restrict__ w, int64_t N,
                                                             int64_t K, const float* __restrict__ w_scale,
                                                             const uint16_t* __restrict__ bias, float s,
                                                             float o, float* __restrict__ deq_scale,
                                                             int32_t* __restrict__ quant_bias) {
  const int lane = threadIdx.x & 63;
  const int64_t n = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= N) return;
  const int8_t* wr = w + n * K;
  int sum = 0;  // |sum| <= 128 * K < 2^31
  for (int64_t k = lane; k < K; k += kWave) sum += wr[k];
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) sum += __shfl_xor(sum, d, kWave);
  if (lane != 0) return;
  const float deq = s * w_scale[n];
  const float corr = (float)sum * o;
  const float fb = bias ? bf16_to_f32(bias[n]) : 0.0f;
  float t = fb / deq;  // IEEE division
  t = t - corr;
  t = __builtin_rintf(t);
  int32_t qb;
  if (t >= 2147483648.0f) qb = 2147483647;
  else if (t <= -2147483648.0f) qb = (int32_t)(-2147483647 - 1);
  else qb = (int32_t)t;
  deq_scale[n] = deq;
  quant_bias[n] = qb;
}

static inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

hipError_t launch_static_quant(const uint16_t* x, int64_t n, float input_scale, float input_offset,
                               int8_t* q, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  if (n % 8 == 0 && aligned(x, 16) && aligned(q, 8)) {
    const int64_t n8 = n / 8;
    const int64_t grid = std::min<int64_t>((n8 + 255) / 256, 256 * 16);
    hipLaunchKernelGGL(static_quant_vec, dim3((unsigned)grid), dim3(256), 0, stream, x, n8,
                       input_scale, input_offset, q);
  } else {
    const int64_t grid = std::min<int64_t>((n + 255) / 256, 256 * 16);
    hipLaunchKernelGGL(static_quant_generic, dim3((unsigned)grid), dim3(256), 0, stream, x, n,
                       input_scale, input_offset, q);
  }
  return hipGetLastError();
}

hipError_t launch_static_quant_packed(const uint16_t* x, int64_t M, int64_t K, float input_scale,
                                      float input_offset, void* q, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const int KB = (int)((K + 63) / 64);
  const int64_t total = (M + 15) / 16 * KB * 64;
  const bool vec = K % 8 == 0 && aligned(x, 16);
  hipLaunchKernelGGL(static_quant_packed_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                     stream, x, M, K, KB, input_scale, input_offset, vec, reinterpret_cast<int8_t*>(q));
  return hipGetLastError();
}

hipError_t launch_static_prepare(const int8_t* w, int64_t N, int64_t K, const float* w_scale,
                                 const uint16_t* bias, float input_scale, float input_offset,
                                 float* deq_scale, int32_t* quant_bias, hipStream_t stream) {
  if (N == 0) return hipSuccess;
  hipLaunchKernelGGL(static_prepare_kernel, dim3((unsigned)((N + 3) / 4)), dim3(256), 0, stream, w,
                     N, K, w_scale, bias, input_scale, input_offset, deq_scale, quant_bias);
  return hipGetLastError();
}

}  // namespace w8a8
