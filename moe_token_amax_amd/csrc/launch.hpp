// Internal launchers of the gfx950 kernels (host side). Arguments are checked
// by the C ABI layer before these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w8a8 {

// codes row-major [M, K], or (packed) in the weight's 1 KB block layout
// [ceil(M/16)][ceil(K/64)]; packed needs K % 8 == 0 and 16-byte aligned rows
// ldx / ldq: row strides of x and of the row-major codes (0: K; packed codes
// need ldx == K)
hipError_t launch_dynamic_quant(const uint16_t* x, int64_t M, int64_t K, int8_t* q, float* scale,
                                bool packed, hipStream_t stream, int64_t ldx = 0, int64_t ldq = 0);
hipError_t launch_swiglu_quant(const uint16_t* h, int64_t R, int64_t I, int8_t* q, float* scale,
                               hipStream_t stream);
hipError_t launch_prepack(const int8_t* w, int64_t E, int64_t N, int64_t K, void* packed,
                          hipStream_t stream);

// Output kinds of the GEMM kernels.
enum OutKind { kOutBf16 = 0, kOutI32 = 1 };

// Dense GEMM plan: kernel variant chosen from the shape.
struct DensePlan {
  int variant;       // index into the dense kernel table
  int64_t ws_bytes;  // device workspace the variant needs (0 for every variant today)
};
DensePlan plan_dense(int64_t M, int64_t N, int64_t K);
// quant fused into the decode GEMM (BF16 input, M <= 2 or M <= 16 with
// M * K <= kFusedElems, K <= 16384, K % 8 == 0, 16-byte aligned x, the codes
// of all rows within kFusedLdsBytes of LDS)
constexpr int64_t kFusedLdsBytes = 65536;
constexpr int64_t kFusedElems = 16384;
bool decode_fused_ok(int64_t M, int64_t K, const void* x);
hipError_t launch_decode_fused(const uint16_t* x, int64_t M, int64_t K, const void* w_packed,
                               const float* w_scale, int64_t N, const uint16_t* bias, void* y, int out,
                               hipStream_t stream);
// lda / ldy: row strides of row-major codes and of y (0: K and N)
hipError_t launch_dense_gemm(const DensePlan& plan, const int8_t* q, const float* x_scale, int64_t M,
                             int64_t K, const void* w_packed, const float* w_scale, int64_t N,
                             const uint16_t* bias, void* y, int out, bool a_packed, void* ws,
                             hipStream_t stream, const int32_t* qbias = nullptr, int64_t lda = 0,
                             int64_t ldy = 0);
// static W8A8: the GEMM above with qbias set (w_scale = the dequant scale,
// x_scale = bias = null); the static activation quant and the load-time
// dequant scale / integer bias
hipError_t launch_static_quant(const uint16_t* x, int64_t n, float input_scale, float input_offset,
                               int8_t* q, hipStream_t stream);
hipError_t launch_static_quant_packed(const uint16_t* x, int64_t M, int64_t K, float input_scale,
                                      float input_offset, void* q, hipStream_t stream);
hipError_t launch_static_prepare(const int8_t* w, int64_t N, int64_t K, const float* w_scale,
                                 const uint16_t* bias, float input_scale, float input_offset,
                                 float* deq_scale, int32_t* quant_bias, hipStream_t stream);

int64_t grouped_ws_bytes(int64_t R, int64_t E, int64_t N, int64_t K);
// the grouped GEMM's schedule for E experts: row offsets int64 [E + 1], large-
// expert tile offsets int32 [E + 1], small-expert ids int32 [E + 1] and kQueues
// work-queue counters, each part 256-byte aligned (grouped_ws_bytes returns it)
constexpr int kQueues = 8;
__host__ __device__ constexpr int64_t sched_align(int64_t b) { return (b + 255) / 256 * 256; }
__host__ __device__ constexpr int64_t group_sched_bytes(int64_t E) {
  return sched_align((E + 1) * 8) + 2 * sched_align((E + 1) * 4) + sched_align(kQueues * 4);
}

// around the MoE chain: routing of (token, slot) expert ids, gather of the INT8
// rows, and the weighted combine (moe_io.hip)
hipError_t launch_route(const int32_t* ids, int64_t T, int64_t k, int64_t E, int64_t* group_list,
                        int32_t* row_token, int32_t* pair_row, hipStream_t stream);
hipError_t launch_gather_rows(const int8_t* q, const float* scale, const int32_t* row_token,
                              int64_t T, int64_t R, int64_t H, int8_t* q_rows, float* s_rows,
                              hipStream_t stream);
hipError_t launch_combine(const uint16_t* y, const int32_t* pair_row, const float* wts, int64_t T,
                          int64_t k, int64_t R, int64_t H, uint16_t* out, hipStream_t stream);
hipError_t launch_grouped_gemm(const int8_t* a, const float* a_scale, const int64_t* group_list,
                               int64_t R, int64_t E, int64_t N, int64_t K, const void* w_packed,
                               const float* w_scale, void* y, int out, void* ws,
                               hipStream_t stream);

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

}  // namespace w8a8
