// Load-time weight prepack for gfx950.
//
// ("DeepSeek-V4 W8A8 执行链从量化权重到 Ascend INT8 算子", §二: the offline
// INT8 [N, K] weight is transposed and format-cast once at load, then reused by
// every forward; §四: that layout is what the matmul kernel reads.)
//
// Layout written ("P16x64"): 1 KB blocks ordered [e][n/16][k/64]; inside a block
// byte l*16 + j (lane l of a wavefront, j < 16) holds
// w[e][16*(n/16) + l%16][64*(k/64) + 16*(l/16) + j]. That is the operand order
// of v_mfma_i32_16x16x64_i8 for a 16-column slice, so a GEMM copies each block
// with one 16-byte load per lane and feeds it to the MFMA unchanged. K is
// zero-padded to a multiple of 64 and N to a multiple of 16, so the GEMM needs
// no K tail handling on the weight side.
#include "device_common.hpp"
#include "launch.hpp"

namespace w8a8 {

// One thread writes one 16-byte lane slot of one block.
__global__ __launch_bounds__(256) void prepack_kernel(const int8_t* __restrict__ w, int64_t E,
                                                      int64_t N, int64_t K, int NB, int KB,
                                                      bool vec, uint8_t* __restrict__ out) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = E * NB * KB * 64;
  if (gid >= total) return;
  const int l = (int)(gid & 63);
  const int64_t blk = gid >> 6;
  const int kb = (int)(blk % KB);
  const int64_t nb = (blk / KB) % NB;
  const int64_t e = blk / ((int64_t)KB * NB);
  const int64_t n = nb * 16 + (l & 15);
  const int64_t k0 = (int64_t)kb * 64 + (l >> 4) * 16;
  uint4 v = {0u, 0u, 0u, 0u};
  if (n < N && k0 < K) {
    const int8_t* src = w + (e * N + n) * K + k0;
    if (vec) {
      v = *reinterpret_cast<const uint4*>(src);
    } else {
      uint32_t wd[4] = {0u, 0u, 0u, 0u};
      const int64_t cnt = min((int64_t)16, K - k0);
      for (int j = 0; j < cnt; ++j) wd[j >> 2] |= (uint32_t)(uint8_t)src[j] << (8 * (j & 3));
      v = uint4{wd[0], wd[1], wd[2], wd[3]};
    }
  }
  *reinterpret_cast<uint4*>(out + gid * 16) = v;
}

hipError_t launch_prepack(const int8_t* w, int64_t E, int64_t N, int64_t K, void* packed,
                          hipStream_t stream) {
  const int NB = (int)ceil_div(N, 16), KB = (int)ceil_div(K, 64);
  const int64_t total = E * NB * KB * 64;
  if (total == 0) return hipSuccess;
  const bool vec = (K % 16 == 0) && (((uintptr_t)w & 15) == 0);
  hipLaunchKernelGGL(prepack_kernel, dim3((unsigned)ceil_div(total, 256)), dim3(256), 0, stream, w,
                     E, N, K, NB, KB, vec, reinterpret_cast<uint8_t*>(packed));
  return hipGetLastError();
}

}  // namespace w8a8
