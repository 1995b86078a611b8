// Internal launchers of the MXFP8 kernels (host side).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w8a8 {

// bytes of k-block-major scales [ceil(K/64)][rows_padded][2]
int64_t mx_scale_kb_bytes(int64_t rows_padded, int64_t K);
hipError_t launch_mx_resolve(const uint8_t* w, const float* s, int64_t N, int64_t K, int64_t BN,
                             int64_t BK, uint16_t* out, hipStream_t stream);
// payload: row-major [M, K], or (blocked) the P16x64 blocks [ceil(M/16)][ceil(K/64)]
// with a zeroed ragged K tail; scale_rm: [M, K/32] (or null);
// scale_kb: [ceil(K/64)][Mp][2] (or null)
hipError_t launch_mx_quant(const uint16_t* x, int64_t M, int64_t K, int scale_alg, uint8_t* payload,
                           bool blocked, uint8_t* scale_rm, uint8_t* scale_kb, int64_t Mp,
                           hipStream_t stream);
hipError_t launch_mx_scale_relayout(const uint8_t* src, int64_t R, int64_t K, int64_t Rp,
                                    uint8_t* dst, hipStream_t stream);
// a: E4M3 activations in P16x64 blocks (as launch_mx_quant with blocked = true)
hipError_t launch_mx_gemm(const uint8_t* a, const uint8_t* a_scale_kb, int64_t Mp, int64_t M,
                          int64_t K, const uint8_t* w_packed, const uint8_t* w_scale_kb, int64_t N,
                          uint16_t* y, hipStream_t stream);

// SwiGLU of h [R, 2I] (gate | up) rounded to BF16, then MX-quantized:
// row-major payload [R, I] and scales [R, I/32]
hipError_t launch_mx_swiglu_quant(const uint16_t* h, int64_t R, int64_t I, int scale_alg,
                                  uint8_t* payload, uint8_t* scale_rm, hipStream_t stream);

// Grouped (MoE) form. Tile records int4 {expert, first source row, first
// padded row, rows} in mx_max_tiles(R, E) slots (192-row tiles first, then
// one 64-row slot per expert), counts int[2]; the MX activation lives in
// mx_padded_rows(R, E) padded rows (P16x64 blocks, k-block-major scales).
int64_t mx_max_tiles(int64_t R, int64_t E);
int64_t mx_padded_rows(int64_t R, int64_t E);
hipError_t launch_mx_group_schedule(const int64_t* group_list, int64_t E, int64_t R, int4* tiles,
                                    int* counts, hipStream_t stream);
// act 0: the rows of x [R, K] (row stride ldx); act 1: SwiGLU of x = h [R, 2K]
hipError_t launch_mx_quant_tiles(const uint16_t* x, int64_t ldx, int64_t K, int act, const int4* tiles,
                                 const int* counts, int64_t R, int64_t E, int scale_alg,
                                 uint8_t* payload, uint8_t* scale_kb, hipStream_t stream);
// expert e's packed weight at w_packed + e * w_stride, its scales w_scale_off further
hipError_t launch_mx_grouped_gemm(const uint8_t* payload, const uint8_t* scale_kb, int64_t R,
                                  int64_t E, int64_t K, const int4* tiles, const int* counts,
                                  const uint8_t* w_packed, int64_t w_stride, int64_t w_scale_off,
                                  int64_t N, uint16_t* y, hipStream_t stream);

}  // namespace w8a8
