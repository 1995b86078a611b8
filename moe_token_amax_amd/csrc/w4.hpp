// Internal launchers of the W4A16 kernels (host side).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w8a8 {

// 128-deep k-chunks of the packed INT4 weight, and its bytes (1152 per
// 16-column block and chunk)
int64_t w4_chunks(int64_t K);
int64_t w4_packed_bytes(int64_t N, int64_t K);
// FP4: 1088 bytes per 16-column block and chunk (1 KB of codes, 64 E8M0 bytes)
int64_t fp4_packed_bytes(int64_t N, int64_t K);
// BF16 w [N, K] -> codes (int8, may be null), BF16 scales [N, K/32] (may be
// null) and the packed layout (may be null)
hipError_t launch_w4_quant_pack(const uint16_t* w, int64_t N, int64_t K, int8_t* q, uint16_t* s,
                                uint8_t* packed, hipStream_t stream);
hipError_t launch_w4_pack(const int8_t* q, const uint16_t* s, int64_t N, int64_t K, uint8_t* packed,
                          hipStream_t stream);
// workspace of the linears: none (0 bytes for every shape)
int64_t w4_linear_ws_bytes(int64_t M, int64_t K);
// y BF16 [M, N] = x BF16 [M, K] times the dequantized packed weight
hipError_t launch_w4a16_linear(const uint16_t* x, int64_t M, int64_t K, const uint8_t* wp, int64_t N,
                               uint16_t* y, void* ws, hipStream_t stream);
// FP4 (E2M1 + E8M0 per 32) weights in the same packed layout: codes (uint8,
// may be null), E8M0 bytes [N, K/32] (may be null), packed (may be null)
hipError_t launch_fp4_quant_pack(const uint16_t* w, int64_t N, int64_t K, uint8_t* c, uint8_t* s,
                                 uint8_t* packed, hipStream_t stream);
hipError_t launch_fp4_linear(const uint16_t* x, int64_t M, int64_t K, const uint8_t* wp, int64_t N,
                             uint16_t* y, void* ws, hipStream_t stream);

// grouped form: rows grouped by expert (group_list = rows per expert, E <=
// 1024), expert e's packed weight (fmt 0 INT4, 1 FP4) at wp + e * the packed
// bytes of one [N, K] weight; y BF16 [R, N]; no workspace
hipError_t launch_lowbit_grouped(int fmt, const uint16_t* x, const int64_t* group_list, int64_t R, int64_t E,
                                 int64_t N, int64_t K, const uint8_t* wp, uint16_t* y, hipStream_t stream);
// a BF16 [R, I] = BF16(silu(gate) * up) of h BF16 [R, 2I] (gate first)
hipError_t launch_lowbit_swiglu(const uint16_t* h, int64_t R, int64_t I, uint16_t* a, hipStream_t stream);

}  // namespace w8a8
