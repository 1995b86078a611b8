// MXFP8 variant for gfx950: block-FP8 resolve, MX quantization and the
// block-scaled GEMM, whose operands are dequantized exactly to BF16 in
// registers (E4M3 x 2^E by v_cvt_scalef32_pk_bf16_fp8) and multiplied on the
// BF16 MFMAs with fp32 accumulation (every product exact).
//
// ("Qwen3.8-FP8 on Ascend 950: Why Weights Become MXFP8 at Load Time":
// Deep Dive 2 resolve equation, Deep Dive 3 E4M3 payload + E8M0 scale per 32
// values along K, Deep Dive 5 runtime activation MX quant + block-scaled
// matmul to the model dtype.)
//
// Formats: E4M3 = OCP E4M3FN (bias 7, largest finite 448, no infinities);
// E8M0 byte b = 2^(b - 127). Encoding rounds to nearest, ties to the even
// code, keeps subnormals, saturates to 448 and keeps the sign of zero (a clamp
// to +-448, then the hardware conversion v_cvt_pk_fp8_f32). The
// shared exponent of a group of 32 is floor(log2(amax)) - 8 (scale rule 0) or
// the smallest E with amax / 2^E <= 448 (scale rule 1), clamped to
// [-127, 127]; amax == 0 gives byte 0.
//
// Layouts: payloads are row-major [rows, K] at the C ABI; the GEMM reads both
// operands in the P16x64 blocks of the INT8 path (the weight prepacked at
// load time, the activation written that way by the MX quant of the linear). Scales at the C ABI are
// row-major [rows, K/32]; the GEMM reads them "k-block major",
// [K/64][rows_p][2] (the two 32-groups of one 64-deep k-block of a row are
// adjacent; rows_p = rows rounded up to even for activations, to 16 for
// weights), so the scales of one stage are a contiguous, dword-aligned run
// per operand.
#include <algorithm>

#include "device_common.hpp"
#include "launch.hpp"
#include "mx.hpp"

namespace w8a8 {

#define W8A8_LDS_MX __attribute__((address_space(3)))

// ---------------------------------------------------------------------------
// E4M3 / E8M0 helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  float v = e ? __builtin_ldexpf((float)(8u + m), (int)e - 10) : __builtin_ldexpf((float)m, -9);
  return (b & 0x80u) ? -v : v;
}

// shared exponent of a group (without the +127 bias)
__device__ __forceinline__ int mx_exponent(float amax, int scale_alg) {
  if (!(amax > 0.0f)) return -127;
  int e = __builtin_amdgcn_frexp_expf(amax) - 1 - 8;
  if (scale_alg == 1 && __builtin_ldexpf(amax, -e) > 448.0f) e += 1;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// ---------------------------------------------------------------------------
// resolve: BF16(fl32(fp32(e4m3) * S[i / BN, j / BK]))
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void mx_resolve_kernel(const uint8_t* __restrict__ w,
                                                         const float* __restrict__ s, int64_t N,
                                                         int64_t K, int64_t BN, int64_t BK,
                                                         uint16_t* __restrict__ out, int vec) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;  // one thread, 8 elements
  const int64_t per_row = (K + 7) / 8;
  if (idx >= N * per_row) return;
  const int64_t i = idx / per_row, j0 = (idx % per_row) * 8;
  const int64_t scols = (K + BK - 1) / BK;
  const float* srow = s + (i / BN) * scols;
  if (vec) {  // K % 8 == 0, w 8-byte and out 16-byte aligned: one load, one store
    const uint2 v = *reinterpret_cast<const uint2*>(w + i * K + j0);
    const uint32_t b[2] = {v.x, v.y};
    uint32_t o[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t j = j0 + 2 * u;
      const float f0 = e4m3_to_f32((b[u / 2] >> (16 * (u & 1))) & 0xFFu) * srow[j / BK];
      const float f1 = e4m3_to_f32((b[u / 2] >> (16 * (u & 1) + 8)) & 0xFFu) * srow[(j + 1) / BK];
      o[u] = f32_to_bf16(f0) | (f32_to_bf16(f1) << 16);
    }
    *reinterpret_cast<uint4*>(out + i * K + j0) = uint4{o[0], o[1], o[2], o[3]};
    return;
  }
  for (int u = 0; u < 8; ++u) {
    const int64_t j = j0 + u;
    if (j >= K) break;
    const float f = e4m3_to_f32(w[i * K + j]) * srow[j / BK];
    out[i * K + j] = (uint16_t)f32_to_bf16(f);
  }
}

// ---------------------------------------------------------------------------
// MX quant: BF16 [M, K] -> E4M3 [M, K] + E8M0. Four consecutive lanes own one
// 32-group (8 values each); the group amax is two DPP steps inside the quad.
// ACT 0 quantizes the rows of x (row stride ldx); ACT 1 quantizes the SwiGLU
// of h = [gate | up] (row stride ldx = 2K): a = BF16(silu(gate) * up), the
// fixed fp32 sequence, rounded once to BF16 before the MX quant.
// ---------------------------------------------------------------------------

// 8 BF16 values (as 4 packed pairs) of chunk c of row `row`
template <int ACT>
__device__ __forceinline__ void mx_load8(const uint16_t* __restrict__ x, int64_t ldx, int64_t K,
                                         int64_t row, int64_t c, uint32_t (&w)[4]) {
  const uint4 v = *reinterpret_cast<const uint4*>(x + row * ldx + c * 8);
  if (ACT == 0) {
    w[0] = v.x;
    w[1] = v.y;
    w[2] = v.z;
    w[3] = v.w;
  } else {
    const uint4 u = *reinterpret_cast<const uint4*>(x + row * ldx + K + c * 8);
    const uint32_t g[4] = {v.x, v.y, v.z, v.w}, up[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a0 = swiglu_fixed(bf16_to_f32(g[j] & 0xFFFFu), bf16_to_f32(up[j] & 0xFFFFu));
      const float a1 = swiglu_fixed(bf16_to_f32(g[j] >> 16), bf16_to_f32(up[j] >> 16));
      w[j] = f32_to_bf16(a0) | (f32_to_bf16(a1) << 16);
    }
  }
}

// group amax of 4 lanes (every lane of the quad must take part)
__device__ __forceinline__ uint32_t mx_quad_amax(const uint32_t (&w)[4]) {
  uint32_t amax = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) amax = max(amax, max(w[j] & 0x7FFFu, (w[j] >> 16) & 0x7FFFu));
  amax = max(amax, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)amax, 0xB1, 0xF, 0xF, false));
  amax = max(amax, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)amax, 0x4E, 0xF, 0xF, false));
  return amax;
}

// 8 E4M3 codes of the BF16 values w scaled by 2^-e: the exact power-of-two
// scaling, a clamp to [-448, 448] (the saturation rule: an encoder input is
// then never past the largest finite code) and the hardware's round-to-
// nearest-even conversion, two values per instruction (subnormals and the sign
// of zero kept; the bit-exact MX tests pin it against the encoding rules).
__device__ __forceinline__ float mx_scaled(uint32_t bf16_bits, int e) {
  return fminf(fmaxf(__builtin_ldexpf(bf16_to_f32(bf16_bits), -e), -448.0f), 448.0f);
}

__device__ __forceinline__ uint2 mx_codes8(const uint32_t (&w)[4], int e) {
  uint32_t o[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t a = w[2 * h], b = w[2 * h + 1];
    int v = __builtin_amdgcn_cvt_pk_fp8_f32(mx_scaled(a & 0xFFFFu, e), mx_scaled(a >> 16, e), 0, false);
    v = __builtin_amdgcn_cvt_pk_fp8_f32(mx_scaled(b & 0xFFFFu, e), mx_scaled(b >> 16, e), v, true);
    o[h] = (uint32_t)v;
  }
  return uint2{o[0], o[1]};
}

// stores of chunk c (8 codes) of row `row` and, on the first lane of the
// quad, the group's scale byte: payload row-major [.., K] or P16x64 blocks,
// scales row-major [.., K/32] and/or k-block-major [KB][Mp][2]
__device__ __forceinline__ void mx_store8(uint2 o, uint8_t sb, int64_t row, int64_t c, int64_t K,
                                          uint8_t* __restrict__ payload, int blocked,
                                          uint8_t* __restrict__ scale_rm,
                                          uint8_t* __restrict__ scale_kb, int64_t Mp) {
  if (!blocked) {
    *reinterpret_cast<uint2*>(payload + row * K + c * 8) = o;
  } else {
    // P16x64 blocks [row / 16][k / 64], byte (row % 16 + 16 * (k % 64 / 16)) * 16 + k % 16
    const int64_t KB = (K + 63) / 64;
    const int64_t k = c * 8;
    const int64_t blk = (row / 16) * KB + k / 64;
    const int64_t at = blk * 1024 + ((row & 15) + 16 * ((k & 63) >> 4)) * 16 + (k & 15);
    *reinterpret_cast<uint2*>(payload + at) = o;
    // a ragged last k-block (K % 64 == 32): its upper 32 bytes per row are
    // zero, the partners of the weight's zero padding
    if ((K & 63) && k >= K - 32) *reinterpret_cast<uint2*>(payload + at + 32 * 16) = uint2{0u, 0u};
  }
  if ((c & 3) == 0) {
    const int64_t g = c / 4;                 // 32-group index along K
    if (scale_rm) scale_rm[row * (K / 32) + g] = sb;
    if (scale_kb) {
      scale_kb[((g / 2) * Mp + row) * 2 + (g & 1)] = sb;
      // odd group count: the last k-block's second slot covers no data; give it
      // byte 0 so that the padded half of that k-block multiplies out to zero
      if (g == K / 32 - 1 && (g & 1) == 0) scale_kb[((g / 2) * Mp + row) * 2 + 1] = 0;
    }
  }
}

template <int ACT>
__global__ __launch_bounds__(256) void mx_quant_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                       int64_t M, int64_t K, int scale_alg,
                                                       uint8_t* __restrict__ payload, int blocked,
                                                       uint8_t* __restrict__ scale_rm,
                                                       uint8_t* __restrict__ scale_kb,
                                                       int64_t Mp) {
  const int64_t chunks = K / 8;             // K % 32 == 0, so quads never straddle rows
  int64_t row, c;
  bool live;
  if (blocked) {
    // a workgroup per 16 rows x 128 k: it writes whole P16x64 blocks (full
    // cache lines), instead of 16 rows' pieces from 16 workgroups
    const int64_t KT = (chunks + 15) / 16;
    row = (int64_t)(blockIdx.x / KT) * 16 + (threadIdx.x >> 4);
    c = (int64_t)(blockIdx.x % KT) * 16 + (threadIdx.x & 15);
    live = row < M && c < chunks;
  } else {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    live = t < M * chunks;
    const int64_t tc = live ? t : 0;
    row = tc / chunks;
    c = tc % chunks;
  }
  uint32_t w[4] = {0u, 0u, 0u, 0u};
  if (live) mx_load8<ACT>(x, ldx, K, row, c, w);
  const uint32_t amax = mx_quad_amax(w);
  if (!live) return;
  const int e = mx_exponent(bf16_to_f32(amax), scale_alg);
  mx_store8(mx_codes8(w, e), (uint8_t)(e + 127), row, c, K, payload, blocked, scale_rm, scale_kb,
            Mp);
}

// row-major [R, K/32] scales -> k-block-major [ceil(K/64)][Rp][2]; pads with 0
__global__ __launch_bounds__(256) void mx_scale_relayout_kernel(const uint8_t* __restrict__ src,
                                                                int64_t R, int64_t G, int64_t Rp,
                                                                uint8_t* __restrict__ dst) {
  const int64_t KB = (G + 1) / 2;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= KB * Rp * 2) return;
  const int64_t g2 = t & 1, r = (t >> 1) % Rp, kb = (t >> 1) / Rp;
  const int64_t g = kb * 2 + g2;
  dst[t] = (r < R && g < G) ? src[r * G + g] : (uint8_t)0;
}

// ---------------------------------------------------------------------------
// Block-scaled GEMM tile: 192 x 256 (M x N), 8 wavefronts (2 x 4) of 96 x 64,
// each a 3 x 2 grid of 32 x 32 fp32 accumulator blocks, one 64-deep k-block
// per stage. A stage holds 12 A blocks + 16 B blocks (1 KB each, MFMA operand
// order) + 1 KB of scales (192 A rows x 2 at byte 0, 256 B columns x 2 at
// byte 512). 192-row tiles give 220 tiles for a 2048 x 5120 output, one round
// on 256 CUs (256-row tiles would give 160). Every wavefront issues 5 LDS-DMA
// loads per stage: wavefronts 0..3 four payload blocks and one scale slice,
// 4..7 three payload blocks and two scale slices (the seven 128-byte slices
// of a stage, the spare ones repeating the last slice: identical bytes to the
// same place), so the per-wavefront vmcnt bookkeeping is uniform.
// ---------------------------------------------------------------------------
struct MxArgs {
  const uint8_t* a;        // E4M3, P16x64 blocks [ceil(M/16)][KB] (K zero-padded to 64)
  const uint8_t* a_scale;  // k-block-major [KB][Mp][2], Mp even
  int64_t Mp;              // row stride of a_scale
  int64_t Mclamp;          // a_scale rows readable from a_scale (even)
  const uint8_t* w;        // packed E4M3 (P16x64), NB x KB blocks
  const uint8_t* w_scale;  // k-block-major [KB][Np][2], Np = NB * 16
  int64_t M, N, K;
  int KB, NB;
  uint16_t* y;             // BF16 [M, N]
};

template <int VM>
__device__ __forceinline__ void mx_wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(VM) : "memory");
}

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// 2^(b - 127) for an E8M0 byte b (b = 0 gives the fp32 subnormal 2^-127)
__device__ __forceinline__ float e8m0_scale(uint32_t b) { return __builtin_ldexpf(1.0f, (int)b - 127); }

// Eight E4M3 codes (bytes of lo, then hi) times sc = 2^E as BF16, two per
// instruction with gfx950's MX conversion v_cvt_scalef32_pk_bf16_fp8. The
// product is exact: an E4M3 value has at most 4 significant bits, and for a
// group scale of a BF16 source (E <= 119) code * 2^E stays inside the BF16
// range. So the BF16 MFMA below multiplies the exact dequantized operands and
// its products (at most 8 x 8 significant bits) are exact in fp32.
__device__ __forceinline__ bf16x8 mx_dequant8(uint32_t lo, uint32_t hi, float sc) {
  const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, sc, false);
  const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, sc, true);
  const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, sc, false);
  const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, sc, true);
  return __builtin_bit_cast(bf16x8, uint4{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                                          __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3)});
}

template <int BM_>
struct MxTile {
  static constexpr int BM = BM_, BN = 256, WM = 2, WN = 4, kWaves = 8, RING = 5;
  static constexpr int TM = BM / WM / 32;  // 3 (BM 192) or 1 (BM 64)
  static constexpr int TN = BN / WN / 32;  // 2
  static constexpr int kABlocks = BM / 16, kBBlocks = BN / 16;  // 12 or 4, and 16
  // payload blocks per wavefront: kPayHi on wavefronts 0..3, one fewer on 4..7
  static constexpr int kPayHi = (kABlocks + kBBlocks + 7) / 8;  // 4 or 3
  static constexpr int kASlices = BM / 64, kSlices = kASlices + 4;  // 128-byte scale slices
  static constexpr int kLoads = kPayHi + 1;                     // DMA per wavefront per stage
  static constexpr int kScaleOfs = (kABlocks + kBBlocks) * 1024;
  static constexpr int kStageBytes = kScaleOfs + 1024;
  static constexpr int kLdsBytes = RING * kStageBytes;
  static_assert(BM % 64 == 0 && TM >= 1, "tile height");
  static_assert(kABlocks + kBBlocks == 4 * kPayHi + 4 * (kPayHi - 1), "payload split over the wavefronts");
  static_assert(kPayHi <= 4 && kSlices >= 5, "DMA source slots");
  static_assert(kLdsBytes <= 163840, "LDS");

  // DMA sources of one wavefront: payload blocks (16 bytes per lane) and scale
  // slices (4 bytes per lane on lanes 0..31), k-block 0 address + step.
  struct Src {
    const uint8_t* pbase[4];
    int64_t pstep[4];
    int pdst[4];            // LDS offset inside a stage
    const uint8_t* sbase[2];
    int64_t sstep[2];
    int sdst[2];
  };

  __device__ __forceinline__ static void payload_src(const MxArgs& p, int bi, int lane, int64_t row0,
                                                     int64_t row_last, int nb0, const uint8_t*& base,
                                                     int64_t& step) {
    if (bi < kABlocks) {
      // A in the P16x64 block layout: 16-row block mb, k-block kb at
      // (mb * KB + kb) KB; blocks past the last one are read clamped
      int64_t mb = row0 / 16 + bi;
      mb = mb < row_last / 16 ? mb : row_last / 16;
      base = p.a + mb * p.KB * 1024 + lane * 16;
      step = 1024;
    } else {
      int nb = nb0 + (bi - kABlocks);
      nb = nb < p.NB ? nb : p.NB - 1;
      base = p.w + (int64_t)nb * p.KB * 1024 + lane * 16;
      step = 1024;
    }
  }

  // scale slice q: A rows [64q, 64q + 64) for q < kASlices, else B columns
  // [64(q - kASlices), + 64); lanes 0..31 bring two rows (columns) each
  __device__ __forceinline__ static void scale_src(const MxArgs& p, int q, int lane, int64_t row0,
                                                   int nb0, const uint8_t*& base, int64_t& step,
                                                   int& dst) {
    if (q < kASlices) {
      int64_t r = row0 + q * 64 + 2 * (lane & 31);
      r = r < p.Mclamp - 2 ? r : p.Mclamp - 2;
      base = p.a_scale + r * 2;
      step = p.Mp * 2;
      dst = kScaleOfs + q * 128;
    } else {
      const int64_t np = (int64_t)p.NB * 16;
      int64_t c = (int64_t)nb0 * 16 + (q - kASlices) * 64 + 2 * (lane & 31);
      c = c < np - 2 ? c : np - 2;
      base = p.w_scale + c * 2;
      step = np * 2;
      dst = kScaleOfs + 512 + (q - kASlices) * 128;
    }
  }

  __device__ __forceinline__ static void sources(const MxArgs& p, Src& s, int wave, int lane,
                                                 int64_t row0, int64_t row_last, int nb0) {
    // payload: wavefronts 0..3 kPayHi blocks each, 4..7 one fewer
    const int first = wave < 4 ? kPayHi * wave : 4 * kPayHi + (kPayHi - 1) * (wave - 4);
    const int count = wave < 4 ? kPayHi : kPayHi - 1;
#pragma unroll
    for (int i = 0; i < kPayHi; ++i) {
      const int bi = first + (i < count ? i : count - 1);
      payload_src(p, bi, lane, row0, row_last, nb0, s.pbase[i], s.pstep[i]);
      s.pdst[i] = bi * 1024;
    }
    // scale slices: wavefronts 0..3 slice w; 4: slices 4 and 5; 5..7 the last
    // slice twice (spares repeat it: identical bytes to the same place)
    const int q0 = wave < 4 ? wave : (wave == 4 ? 4 : kSlices - 1);
    const int q1 = wave == 4 ? (5 < kSlices ? 5 : kSlices - 1) : kSlices - 1;
    scale_src(p, q0, lane, row0, nb0, s.sbase[0], s.sstep[0], s.sdst[0]);
    scale_src(p, q1, lane, row0, nb0, s.sbase[1], s.sstep[1], s.sdst[1]);
  }

  // the 5 loads of k-block kb into ring buffer buf
  __device__ __forceinline__ static void issue(const MxArgs& p, const Src& s, uint8_t* smem, int buf,
                                               int kb, int wave, int lane) {
    uint8_t* st = smem + buf * kStageBytes;
    const bool four = wave < 4;
#pragma unroll
    for (int i = 0; i < kPayHi; ++i) {
      if (i == kPayHi - 1 && !four) break;
      const uint8_t* src = s.pbase[i] + kb * s.pstep[i];
      __builtin_amdgcn_global_load_lds(src, (W8A8_LDS_MX void*)((W8A8_LDS_MX uint8_t*)st + s.pdst[i]),
                                       16, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      if (q == 1 && four) break;
      if (lane < 32)  // 32 lanes x 4 bytes: lane l lands at slice + 4 l
        __builtin_amdgcn_global_load_lds(s.sbase[q] + kb * s.sstep[q],
                                         (W8A8_LDS_MX void*)((W8A8_LDS_MX uint8_t*)st + s.sdst[q]), 4,
                                         0, 0);
    }
  }

  struct Frags {
    i32x8 a[TM];
    i32x8 b[TN];
    uint32_t sa[TM];  // E8M0 bytes of the lane's row: group 0 | group 1 << 8
    uint32_t sb[TN];
  };

  // Operand of 32 rows (columns) starting at 16-row block 2i. Lane l (row
  // l & 31, h = l >> 5) reads block 2i + (l>>4 & 1), row l & 15, 16-byte
  // k-chunks h and h + 2: bytes 0..15 hold k [16h, 16h + 16) of the
  // k-block's first 32-group, bytes 16..31 hold k [32 + 16h, 48 + 16h) of
  // the second. A and B fragments use the same lane -> k mapping, so every
  // MFMA below pairs equal k.
  __device__ __forceinline__ static i32x8 read_operand(const uint8_t* blk, int lane) {
    const uint8_t* q = blk + (((lane >> 4) & 1) * 1024) + ((lane >> 5) * 16 + (lane & 15)) * 16;
    const i32x4 lo = *reinterpret_cast<const i32x4*>(q);
    const i32x4 hi = *reinterpret_cast<const i32x4*>(q + 512);
    return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }

  __device__ __forceinline__ static void read_frags(const uint8_t* st, Frags& f, int wm, int wn,
                                                    int lane) {
    const int r = lane & 31;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int c32 = wn * TN + j;
      f.b[j] = read_operand(st + (kABlocks + c32 * 2) * 1024, lane);
      f.sb[j] = *reinterpret_cast<const uint16_t*>(st + kScaleOfs + 512 + (c32 * 32 + r) * 2);
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int r32 = wm * TM + i;
      f.a[i] = read_operand(st + r32 * 2 * 1024, lane);
      f.sa[i] = *reinterpret_cast<const uint16_t*>(st + kScaleOfs + (r32 * 32 + r) * 2);
    }
  }

  // The 32 codes of a fragment times their group's 2^E as BF16 (exact:
  // mx_dequant8), four MFMA operands of 8 values (k-steps t = 0..3; t < 2 in
  // group 0, t >= 2 in group 1).
  __device__ __forceinline__ static void dequant_frag(const i32x8& v, uint32_t sc, bf16x8 (&o)[4]) {
    const float s0 = e8m0_scale(sc & 0xFFu), s1 = e8m0_scale((sc >> 8) & 0xFFu);
    o[0] = mx_dequant8((uint32_t)v[0], (uint32_t)v[1], s0);
    o[1] = mx_dequant8((uint32_t)v[2], (uint32_t)v[3], s0);
    o[2] = mx_dequant8((uint32_t)v[4], (uint32_t)v[5], s1);
    o[3] = mx_dequant8((uint32_t)v[6], (uint32_t)v[7], s1);
  }

  // One k-block: B fragments dequantized once, then per accumulator row the A
  // fragment and 4 x TN MFMAs of 32 x 32 x 16 (exact BF16 products, fp32 sums).
  __device__ __forceinline__ static void mfma_rows(const Frags& f, f32x16 (&acc)[TM][TN], int lo,
                                                   int hi) {
    bf16x8 bq[TN][4];
#pragma unroll
    for (int j = 0; j < TN; ++j) dequant_frag(f.b[j], f.sb[j], bq[j]);
#pragma unroll
    for (int i = lo; i < hi; ++i) {
      bf16x8 aq[4];
      dequant_frag(f.a[i], f.sa[i], aq);
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq[t], bq[j][t], acc[i][j], 0, 0, 0);
    }
  }

  // K loop in pairs of k-blocks over a five-buffer ring: one wait + barrier
  // per pair, two to three k-blocks of DMA always in flight (the same ring as
  // the INT8 tile). One fragment set F: the MFMAs of a k-block are issued,
  // then F is refilled for the next one; with one barrier per pair the two
  // wavefronts of a SIMD drift apart, so one's LDS reads run under the other's
  // MFMAs (two sets of the 8-register MFMA operands do not fit next to the
  // accumulators).
  __device__ static void mainloop(const MxArgs& p, uint8_t* smem, f32x16 (&acc)[TM][TN],
                                  int64_t row0, int64_t row_end, int nb0) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int KB = p.KB;
    Src src;
    sources(p, src, wave, lane, row0, row_end - 1, nb0);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};
#pragma unroll
    for (int s = 0; s < RING; ++s)
      if (s < KB) issue(p, src, smem, s, s, wave, lane);
    if (KB >= 5) mx_wait_barrier<3 * kLoads>();
    else if (KB == 4) mx_wait_barrier<2 * kLoads>();
    else if (KB == 3) mx_wait_barrier<kLoads>();
    else mx_wait_barrier<0>();
    Frags F;
    read_frags(smem, F, wm, wn, lane);
    int buf = 0;
    for (int kb = 0; kb < KB; kb += 2) {
      const int buf1 = buf == RING - 1 ? 0 : buf + 1;
      const int buf2 = buf1 == RING - 1 ? 0 : buf1 + 1;
      __builtin_amdgcn_sched_barrier(0);
      mfma_rows(F, acc, 0, TM);
      __builtin_amdgcn_sched_barrier(0);
      if (kb + 1 < KB) {
        read_frags(smem + buf1 * kStageBytes, F, wm, wn, lane);
        __builtin_amdgcn_sched_barrier(0);
        mfma_rows(F, acc, 0, TM);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (kb + 2 < KB) {
        if (kb + 4 < KB) mx_wait_barrier<kLoads>();
        else mx_wait_barrier<0>();
        if (kb + 5 < KB) issue(p, src, smem, buf, kb + 5, wave, lane);
        if (kb + 6 < KB) issue(p, src, smem, buf1, kb + 6, wave, lane);
        read_frags(smem + buf2 * kStageBytes, F, wm, wn, lane);
      }
      buf = buf2;
    }
    mx_wait_barrier<0>();
  }

  // register v of block (i, j): row 8*(v/4) + 4*(l/32) + v%4, column l%32
  __device__ static void epilogue(const MxArgs& p, const f32x16 (&acc)[TM][TN], int64_t row0,
                                  int64_t row_end, int64_t n0) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave / WN, wn = wave % WN;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int64_t n = n0 + (wn * TN + j) * 32 + (lane & 31);
      if (n >= p.N) continue;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t m = row0 + (wm * TM + i) * 32 + 8 * (v / 4) + 4 * (lane >> 5) + (v & 3);
          if (m < row_end) p.y[m * p.N + n] = (uint16_t)f32_to_bf16(acc[i][j][v]);
        }
      }
    }
  }
};

using MxBig = MxTile<192>;
using MxSmall = MxTile<64>;

// ---------------------------------------------------------------------------
// Dense block-scaled GEMM tile: BM x BN = (WM TM 16) x (WN TN 16), WM x WN
// wavefronts, each a TM x TN grid of 16 x 16 fp32 accumulator blocks fed by
// v_mfma_f32_16x16x32_bf16. The default 256 x 160 tile with 4 x 2 wavefronts
// (two per SIMD) gives 8 x 32 = 256 equal tiles for a 2048 x 5120 output: one
// per CU, none idle. A stage holds BM/16 A blocks and BN/16 B blocks (1 KB
// P16x64 each) and 1 KB of scales (BM A rows x 2 at byte 0, BN B columns x 2
// at byte 512). In a P16x64 block lane l's 16 bytes (bytes 16 l ..) are row
// l % 16 and k = 16 (l / 16) .. + 15, all in 32-group l / 32: one
// ds_read_b128 per lane per block, dequantized to two MFMA operands (k-steps
// t = 0, 1: bytes 8t .. 8t + 7). The BF16 MFMA's lane l supplies k' = 8 (l /
// 16) + e of its k-step, here original k = 16 (l / 16) + 8 t + e for A and B
// alike, so every product pairs equal k and each k of the k-block is used
// once. The FP8 -> BF16 conversion is a half-rate VALU instruction (two values
// each): with two wavefronts per SIMD, one's conversions issue while the
// other's MFMAs run.
// ---------------------------------------------------------------------------
#ifndef W8A8_MXW_WM
#define W8A8_MXW_WM 4
#endif
#ifndef W8A8_MXW_WN
#define W8A8_MXW_WN 2
#endif
#ifndef W8A8_MXW_TM
#define W8A8_MXW_TM 4
#endif
#ifndef W8A8_MXW_TN
#define W8A8_MXW_TN 5
#endif

typedef float f32x4v __attribute__((ext_vector_type(4)));

template <int WM_, int WN_, int TM_, int TN_>
struct MxWide {
  static constexpr int WM = WM_, WN = WN_, TM = TM_, TN = TN_;
  static constexpr int BM = WM * TM * 16, BN = WN * TN * 16, kWaves = WM * WN, RING = 5;
  static constexpr int kABlocks = BM / 16, kBBlocks = BN / 16;
  static constexpr int kScaleOfs = (kABlocks + kBBlocks) * 1024;
  static constexpr int kStageBytes = kScaleOfs + 1024;
  static constexpr int kLdsBytes = RING * kStageBytes;
  // DMA per stage and wavefront: kPay payload blocks (16 bytes per lane) and
  // one 256-byte scale piece (4 bytes per lane). The pieces are A rows
  // [128 q, 128 q + 128) for q < kAPieces, then B columns likewise; slots
  // past the last block or piece repeat it (identical bytes to the same place).
  static constexpr int kAPieces = (BM + 127) / 128, kBPieces = (BN + 127) / 128;
  static constexpr int kPay = (kABlocks + kBBlocks + kWaves - 1) / kWaves;
  static constexpr int kLoads = kPay + 1;
  static_assert(kAPieces <= 2 && kBPieces <= 2 && kAPieces + kBPieces <= kWaves, "scale pieces");
  static_assert(kLdsBytes <= 163840, "LDS");
  // A fragments are read this many accumulator rows ahead of their use
  static constexpr int kAhead = 2;

  struct Src {
    const uint8_t* pay[kPay];
    int pdst[kPay];
    const uint8_t* sc;
    int64_t sc_step;
    int sdst;
  };

  __device__ __forceinline__ static void sources(const MxArgs& p, Src& s, int wave, int lane, int64_t row0,
                                                 int64_t row_last, int nb0) {
#pragma unroll
    for (int i = 0; i < kPay; ++i) {
      int L = wave * kPay + i;
      L = L < kABlocks + kBBlocks ? L : kABlocks + kBBlocks - 1;
      if (L < kABlocks) {  // A: 16-row block mb, k-block kb at (mb * KB + kb) KB
        int64_t mb = row0 / 16 + L;
        mb = mb < row_last / 16 ? mb : row_last / 16;
        s.pay[i] = p.a + mb * p.KB * 1024 + lane * 16;
      } else {
        int nb = nb0 + (L - kABlocks);
        nb = nb < p.NB ? nb : p.NB - 1;
        s.pay[i] = p.w + (int64_t)nb * p.KB * 1024 + lane * 16;
      }
      s.pdst[i] = L * 1024;
    }
    const int q = wave < kAPieces + kBPieces ? wave : kAPieces + kBPieces - 1;
    if (q < kAPieces) {  // lane l: rows 2 l, 2 l + 1 of the piece
      int64_t r = row0 + 128 * q + 2 * lane;
      r = r < p.Mclamp - 2 ? r : p.Mclamp - 2;
      s.sc = p.a_scale + r * 2;
      s.sc_step = p.Mp * 2;
      s.sdst = kScaleOfs + q * 256;
    } else {
      const int64_t np = (int64_t)p.NB * 16;
      int64_t c = (int64_t)nb0 * 16 + 128 * (q - kAPieces) + 2 * lane;
      c = c < np - 2 ? c : np - 2;
      s.sc = p.w_scale + c * 2;
      s.sc_step = np * 2;
      s.sdst = kScaleOfs + 512 + (q - kAPieces) * 256;
    }
  }

  // load i (< kLoads) of stage kb into ring buffer buf: payload slots first,
  // the scale piece last
  __device__ __forceinline__ static void issue_one(const Src& s, uint8_t* smem, int buf, int kb, int i) {
    W8A8_LDS_MX uint8_t* st = (W8A8_LDS_MX uint8_t*)(smem + buf * kStageBytes);
    if (i < kPay)
      __builtin_amdgcn_global_load_lds(s.pay[i] + (int64_t)kb * 1024, (W8A8_LDS_MX void*)(st + s.pdst[i]), 16,
                                       0, 0);
    else
      __builtin_amdgcn_global_load_lds(s.sc + kb * s.sc_step, (W8A8_LDS_MX void*)(st + s.sdst), 4, 0, 0);
  }

  __device__ __forceinline__ static void issue(const Src& s, uint8_t* smem, int buf, int kb) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) issue_one(s, smem, buf, kb, i);
  }

  // the 16 codes of a lane's block piece times 2^E: the operands of k-steps 0, 1
  __device__ __forceinline__ static void deq(const i32x4& v, uint32_t sbyte, bf16x8 (&o)[2]) {
    const float sc = e8m0_scale(sbyte);
    o[0] = mx_dequant8((uint32_t)v[0], (uint32_t)v[1], sc);
    o[1] = mx_dequant8((uint32_t)v[2], (uint32_t)v[3], sc);
  }

  __device__ __forceinline__ static i32x4 ld_a(const uint8_t* st, int wm, int i, int lane) {
    return *reinterpret_cast<const i32x4*>(st + (wm * TM + i) * 1024 + lane * 16);
  }
  __device__ __forceinline__ static uint32_t ls_a(const uint8_t* st, int wm, int i, int lane) {
    return st[kScaleOfs + ((wm * TM + i) * 16 + (lane & 15)) * 2 + (lane >> 5)];
  }
  __device__ __forceinline__ static i32x4 ld_b(const uint8_t* st, int wn, int j, int lane) {
    return *reinterpret_cast<const i32x4*>(st + (kABlocks + wn * TN + j) * 1024 + lane * 16);
  }
  __device__ __forceinline__ static uint32_t ls_b(const uint8_t* st, int wn, int j, int lane) {
    return st[kScaleOfs + 512 + ((wn * TN + j) * 16 + (lane & 15)) * 2 + (lane >> 5)];
  }

  // The MFMAs of one k-block (operands A, B), accumulator row by row. With a
  // next stage (nx != null) its fragments are read and dequantized in between:
  // B read at the start and dequantized into Bn (the other operand set) spread
  // over the rows, A row i in place right after row i's MFMAs, its LDS read
  // kAhead rows earlier.
  // The DMA of a later stage (dkb >= 0) is issued between the rows, a few
  // loads after each (an issue that waits for room in the memory queue then
  // stalls behind MFMAs already in the matrix pipe, not ahead of them).
  template <bool NEXT, bool DMA>
  __device__ __forceinline__ static void kblock(f32x4v (&acc)[TM][TN], bf16x8 (&A)[TM][2],
                                                const bf16x8 (&B)[TN][2], bf16x8 (&Bn)[TN][2],
                                                const uint8_t* nx, int wm, int wn, int lane,
                                                const Src* src = nullptr, uint8_t* smem = nullptr,
                                                int dbuf = 0, int dkb = 0) {
    i32x4 rb[TN], ra[TM];
    uint32_t sb[TN], sa[TM];
    if (NEXT) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        rb[j] = ld_b(nx, wn, j, lane);
        sb[j] = ls_b(nx, wn, j, lane);
      }
#pragma unroll
      for (int i = 0; i < kAhead; ++i) {
        ra[i] = ld_a(nx, wm, i, lane);
        sa[i] = ls_a(nx, wm, i, lane);
      }
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      if (NEXT && i + kAhead < TM) {
        ra[i + kAhead] = ld_a(nx, wm, i + kAhead, lane);
        sa[i + kAhead] = ls_a(nx, wm, i + kAhead, lane);
      }
      // k-step outer: consecutive MFMAs write different accumulators
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[i][t], B[j][t], acc[i][j], 0, 0, 0);
      if (DMA) {
#pragma unroll
        for (int l = i * kLoads / TM; l < (i + 1) * kLoads / TM; ++l) issue_one(*src, smem, dbuf, dkb, l);
      }
      if (NEXT) {
        deq(ra[i], sa[i], A[i]);
#pragma unroll
        for (int j = 0; j < TN; ++j)  // B block j refilled after row j TM / TN
          if (j * TM / TN == i) deq(rb[j], sb[j], Bn[j]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  template <int VM>
  __device__ __forceinline__ static void wait_barrier() {
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(VM) : "memory");
  }

  // Phase kb (< KB - 1): stage kb + 1 must have landed (own DMA waited, then
  // a barrier for everyone's); the barrier also means every wavefront has
  // dequantized stage kb, so its buffer takes stage kb + RING (with DMA,
  // issued between the rows of kb). Stage kb + 1 is read and dequantized
  // under the MFMAs of kb. Each phase body is straight-line code: a branch
  // inside it would split the scheduling regions and the conversions would
  // no longer issue between the MFMAs.
  template <bool DMA>
  __device__ __forceinline__ static void phase(const Src& src, uint8_t* smem, int kb, int KB, int wm, int wn,
                                               int lane, f32x4v (&acc)[TM][TN], bf16x8 (&A)[TM][2],
                                               const bf16x8 (&B)[TN][2], bf16x8 (&Bn)[TN][2]) {
    if (DMA) {
      wait_barrier<(RING - 2) * kLoads>();  // stages kb + 2 .. kb + RING - 1 in flight
    } else {
      const int n = KB - 2 - kb;  // stages issued after kb + 1
      if (n >= 3) wait_barrier<3 * kLoads>();
      else if (n == 2) wait_barrier<2 * kLoads>();
      else if (n == 1) wait_barrier<kLoads>();
      else wait_barrier<0>();
    }
    kblock<true, DMA>(acc, A, B, Bn, smem + ((kb + 1) % RING) * kStageBytes, wm, wn, lane, &src, smem,
                      kb % RING, kb + RING);
  }

  __device__ static void mainloop(const MxArgs& p, uint8_t* smem, f32x4v (&acc)[TM][TN], int64_t row0,
                                  int64_t row_end, int nb0) {
    static_assert(RING == 5, "wait cases");
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int KB = p.KB;
    Src src;
    sources(p, src, wave, lane, row0, row_end - 1, nb0);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = f32x4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < RING; ++s)
      if (s < KB) issue(src, smem, s, s);
    if (KB >= 5) wait_barrier<4 * kLoads>();
    else if (KB == 4) wait_barrier<3 * kLoads>();
    else if (KB == 3) wait_barrier<2 * kLoads>();
    else if (KB == 2) wait_barrier<kLoads>();
    else wait_barrier<0>();
    bf16x8 A[TM][2], B0[TN][2], B1[TN][2];
#pragma unroll
    for (int i = 0; i < TM; ++i) deq(ld_a(smem, wm, i, lane), ls_a(smem, wm, i, lane), A[i]);
#pragma unroll
    for (int j = 0; j < TN; ++j) deq(ld_b(smem, wn, j, lane), ls_b(smem, wn, j, lane), B0[j]);
    // k-blocks in pairs (the two B operand sets trade roles): the steady
    // state, where both phases issue a stage; the pair where only the first
    // does; the pairs with nothing left to load; the last one or two
    int kb = 0;
    for (; kb + RING + 1 < KB; kb += 2) {
      phase<true>(src, smem, kb, KB, wm, wn, lane, acc, A, B0, B1);
      phase<true>(src, smem, kb + 1, KB, wm, wn, lane, acc, A, B1, B0);
    }
    if (kb + RING < KB) {
      phase<true>(src, smem, kb, KB, wm, wn, lane, acc, A, B0, B1);
      phase<false>(src, smem, kb + 1, KB, wm, wn, lane, acc, A, B1, B0);
      kb += 2;
    }
    for (; kb + 2 < KB; kb += 2) {
      phase<false>(src, smem, kb, KB, wm, wn, lane, acc, A, B0, B1);
      phase<false>(src, smem, kb + 1, KB, wm, wn, lane, acc, A, B1, B0);
    }
    if (kb + 2 == KB) {
      phase<false>(src, smem, kb, KB, wm, wn, lane, acc, A, B0, B1);
      kblock<false, false>(acc, A, B1, B0, nullptr, wm, wn, lane);
    } else {
      kblock<false, false>(acc, A, B0, B1, nullptr, wm, wn, lane);
    }
  }

  // register v of block (i, j): row 4 (l / 16) + v, column l % 16
  __device__ static void epilogue(const MxArgs& p, const f32x4v (&acc)[TM][TN], int64_t row0,
                                  int64_t row_end, int64_t n0) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave / WN, wn = wave % WN;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int64_t n = n0 + (wn * TN + j) * 16 + (lane & 15);
      if (n >= p.N) continue;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int64_t m = row0 + (wm * TM + i) * 16 + 4 * (lane >> 4) + v;
          if (m < row_end) p.y[m * p.N + n] = (uint16_t)f32_to_bf16(acc[i][j][v]);
        }
      }
    }
  }
};

using MxDense = MxWide<W8A8_MXW_WM, W8A8_MXW_WN, W8A8_MXW_TM, W8A8_MXW_TN>;

__global__ __launch_bounds__(64 * MxDense::kWaves) void mx_gemm_kernel(MxArgs p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[MxDense::kLdsBytes];
  const int64_t MT = (p.M + MxDense::BM - 1) / MxDense::BM, NT = (p.N + MxDense::BN - 1) / MxDense::BN;
  const int64_t T = MT * NT;
  // XCD-chunked tile order, m fastest inside an XCD's range
  const int64_t per = (T + 7) / 8;
  const int64_t t = (blockIdx.x % 8) * per + blockIdx.x / 8;
  if (t >= T) return;
  const int64_t tm = t % MT, tn = t / MT;
  const int64_t row0 = tm * MxDense::BM;
  const int64_t row_end = min(row0 + MxDense::BM, p.M);
  f32x4v acc[MxDense::TM][MxDense::TN];
  MxDense::mainloop(p, smem, acc, row0, row_end, (int)(tn * MxDense::BN / 16));
  MxDense::epilogue(p, acc, row0, row_end, tn * MxDense::BN);
}

// ---------------------------------------------------------------------------
// Grouped (MoE) form. The routed rows of expert e are R rows grouped by expert
// (group_list, as the INT8 grouped path); the MX activation of a grouped
// matmul is written in the P16x64 block layout with every expert starting on
// a 16-row boundary ("padded rows"), so that a tile of one expert is a run of
// whole blocks. The schedule cuts each expert into 192-row tiles; a last
// piece of at most 64 rows gets a 64-row tile instead (most experts of a
// skewed routing are that small). Records int4 {expert, first source row,
// first padded row, rows}: 192-row tiles in slots [0, max_big), 64-row tiles
// in slots [max_big, max_big + E); counts[0] and counts[1] say how many.
// ---------------------------------------------------------------------------
constexpr int kMxSub = MxBig::BM / 16;  // 16-row groups per record slot

// exclusive scan over the 1024 threads of the block (one value each)
__device__ __forceinline__ int block_scan_1024(int v, int* wsum, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int o = __shfl_up(incl, d, kWave);
    if (lane >= d) incl += o;
  }
  __syncthreads();  // wsum free from an earlier scan
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  int before = 0;
  total = 0;
  for (int w = 0; w < 16; ++w) {
    before += w < wave ? wsum[w] : 0;
    total += wsum[w];
  }
  return before + incl - v;
}

// One 1024-thread workgroup, thread e = expert e (E <= 1024). Counts are cut
// to what fits in R rows (a group_list summing past R writes nothing out of
// bounds), so sum(padded rows) <= R + 15 E, 192-row records <= ceil(R/192) +
// E = max_big and 64-row records <= E.
__global__ __launch_bounds__(1024) void mx_group_schedule_kernel(const int64_t* __restrict__ group_list,
                                                                 int E, int64_t R, int64_t max_big,
                                                                 int4* __restrict__ tiles,
                                                                 int* __restrict__ counts) {
  __shared__ int wsum[16];
  const int e = threadIdx.x;
  int64_t n = e < E ? group_list[e] : 0;
  n = n < 0 ? 0 : (n > R ? R : n);
  int total;
  const int roff = block_scan_1024((int)n, wsum, total);
  const int64_t left = R - roff;
  const int rows = (int)(left <= 0 ? 0 : (n < left ? n : left));
  const int poff = block_scan_1024((rows + 15) & ~15, wsum, total);
  const int full = rows / MxBig::BM, rem = rows % MxBig::BM;
  const int nb = full + (rem > MxSmall::BM ? 1 : 0);
  const int ns = (rem > 0 && rem <= MxSmall::BM) ? 1 : 0;
  int nb_total, ns_total;
  const int boff = block_scan_1024(nb, wsum, nb_total);
  const int soff = block_scan_1024(ns, wsum, ns_total);
  for (int j = 0; j < nb; ++j) {
    if (boff + j >= max_big) break;
    const int r = j * MxBig::BM;
    tiles[boff + j] = int4{e, roff + r, poff + r, min(MxBig::BM, rows - r)};
  }
  if (ns) {
    const int r = full * MxBig::BM;
    tiles[max_big + soff] = int4{e, roff + r, poff + r, rem};
  }
  if (threadIdx.x == 0) {
    counts[0] = (int)(nb_total < max_big ? nb_total : max_big);
    counts[1] = ns_total;
  }
}

// record slot m holds a scheduled tile
__device__ __forceinline__ bool mx_slot_live(int64_t m, int64_t max_big, const int* counts) {
  return m < max_big ? m < counts[0] : m - max_big < counts[1];
}

// MX quant straight into the P16x64 block layout: one wavefront per output
// block (16 rows x one 64-deep k-block). Lane l takes row l / 4 and the 16
// values k = 64 kb + 16 (l % 4) .. + 15 (four consecutive lanes read a row's
// 128 contiguous bytes); its 16 codes are bytes (l / 4 + 16 (l % 4)) * 16 ..
// of the block, so the wavefront's stores cover the 1 KB block. A 32-group is
// lanes l and l ^ 1; lane 4 r stores row r's two scale bytes of the k-block
// ([KB][scale_rows][2]) as one 16-bit word. Rows past the real ones
// and the ragged upper half of a last k-block (K % 64 == 32) get zero codes
// and scale byte 0.
// Workgroup (x, y): x = (tile record, 16-row group) of the grouped schedule
// (source row rec.y + lr, padded row rec.z + lr, rec.w real rows), k-blocks
// y * 4 + wave, stepping by 4 * gridDim.y (a few k-blocks per wavefront, so
// that enough wavefronts run).
template <int ACT>
__device__ __forceinline__ void mx_load16(const uint16_t* __restrict__ x, int64_t ldx, int64_t K,
                                          int64_t row, int64_t k, uint32_t (&w)[8]) {
  const uint4* src = reinterpret_cast<const uint4*>(x + row * ldx + k);
  const uint4 v0 = src[0], v1 = src[1];
  const uint32_t g[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
  if (ACT == 0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) w[j] = g[j];
  } else {
    const uint4* usrc = reinterpret_cast<const uint4*>(x + row * ldx + K + k);
    const uint4 u0 = usrc[0], u1 = usrc[1];
    const uint32_t up[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float a0 = swiglu_fixed(bf16_to_f32(g[j] & 0xFFFFu), bf16_to_f32(up[j] & 0xFFFFu));
      const float a1 = swiglu_fixed(bf16_to_f32(g[j] >> 16), bf16_to_f32(up[j] >> 16));
      w[j] = f32_to_bf16(a0) | (f32_to_bf16(a1) << 16);
    }
  }
}

template <int ACT>
__global__ __launch_bounds__(256) void mx_quant_tiles_kernel(const uint16_t* __restrict__ x,
                                                              int64_t ldx, int64_t K,
                                                              const int4* __restrict__ tiles,
                                                              const int* __restrict__ counts,
                                                              int64_t max_big, int scale_alg,
                                                              uint8_t* __restrict__ payload,
                                                              uint8_t* __restrict__ scale_kb,
                                                              int64_t scale_rows) {
  const int tm = blockIdx.x / kMxSub, sub = blockIdx.x % kMxSub;
  if (!mx_slot_live(tm, max_big, counts)) return;
  const int4 rec = tiles[tm];
  if (16 * sub >= rec.w) return;
  const int64_t src0 = (int64_t)rec.y + 16 * sub;
  const int64_t prow0 = (int64_t)rec.z + 16 * sub;
  const int64_t nreal = rec.w - 16 * sub;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane >> 2, ch = lane & 3;
  const bool real = r < nreal;
  const int64_t prow = prow0 + r;
  const int KB = (int)((K + 63) / 64);
  uint8_t* blocks = payload + (prow0 >> 4) * (int64_t)KB * 1024;
  // k-blocks split over blockIdx.y and the 4 wavefronts
  for (int kb = (int)blockIdx.y * 4 + wave; kb < KB; kb += 4 * (int)gridDim.y) {
    const int64_t k = (int64_t)kb * 64 + 16 * ch;
    uint32_t w[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
    if (real && k < K) mx_load16<ACT>(x, ldx, K, src0 + r, k, w);
    uint32_t amax = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = max(amax, max(w[j] & 0x7FFFu, (w[j] >> 16) & 0x7FFFu));
    amax = max(amax, (uint32_t)__shfl_xor((int)amax, 1, kWave));
    const int e = mx_exponent(bf16_to_f32(amax), scale_alg);
    const uint2 lo = mx_codes8(*reinterpret_cast<const uint32_t(*)[4]>(&w[0]), e);
    const uint2 hi = mx_codes8(*reinterpret_cast<const uint32_t(*)[4]>(&w[4]), e);
    *reinterpret_cast<uint4*>(blocks + (int64_t)kb * 1024 + (r + 16 * ch) * 16) =
        uint4{lo.x, lo.y, hi.x, hi.y};
    const int e_g1 = __shfl_xor(e, 2, kWave);  // group 1 of the row: chunk 2
    if (ch == 0 && prow < scale_rows) {
      const uint32_t b0 = (uint32_t)(e + 127);
      const uint32_t b1 = (int64_t)kb * 64 + 32 < K ? (uint32_t)(e_g1 + 127) : 0u;
      *reinterpret_cast<uint16_t*>(scale_kb + ((int64_t)kb * scale_rows + prow) * 2) =
          (uint16_t)(b0 | (b1 << 8));
    }
  }
}

// Grouped block-scaled matmul: one tile per workgroup (a 192 x 256 or a
// 64 x 256 one, by record slot), slots x n-tiles, XCD-chunked with m fastest;
// workgroups of unused slots leave at once.
__global__ __launch_bounds__(512) void mx_grouped_kernel(MxArgs base, const int4* __restrict__ tiles,
                                                         const int* __restrict__ counts,
                                                         int64_t max_big, int64_t max_small,
                                                         int64_t NT, int64_t w_stride,
                                                         int64_t w_scale_off) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[MxBig::kLdsBytes];
  static_assert(MxSmall::kLdsBytes <= MxBig::kLdsBytes, "LDS shared by both tiles");
  const int64_t MT = max_big + max_small;
  const int64_t T = MT * NT;
  const int64_t per = (T + 7) / 8;
  const int64_t t = (blockIdx.x % 8) * per + blockIdx.x / 8;
  if (t >= T) return;
  const int64_t tm = t % MT, tn = t / MT;
  if (!mx_slot_live(tm, max_big, counts)) return;
  const int4 rec = tiles[tm];
  MxArgs p = base;
  p.a = base.a + (int64_t)(rec.z / 16) * p.KB * 1024;
  p.a_scale = base.a_scale + (int64_t)rec.z * 2;
  p.Mclamp = (rec.w + 1) & ~1;
  p.w = base.w + (int64_t)rec.x * w_stride;
  p.w_scale = p.w + w_scale_off;
  p.y = base.y + (int64_t)rec.y * p.N;
  const int nb0 = (int)(tn * MxBig::BN / 16);
  if (tm < max_big) {
    f32x16 acc[MxBig::TM][MxBig::TN];
    MxBig::mainloop(p, smem, acc, 0, rec.w, nb0);
    MxBig::epilogue(p, acc, 0, rec.w, tn * MxBig::BN);
  } else {
    f32x16 acc[MxSmall::TM][MxSmall::TN];
    MxSmall::mainloop(p, smem, acc, 0, rec.w, nb0);
    MxSmall::epilogue(p, acc, 0, rec.w, tn * MxSmall::BN);
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
// k-split of mx_quant_blocks_kernel: about 4 k-blocks per wavefront
static int64_t mx_quant_ksplit(int64_t K) { return std::max<int64_t>(1, ceil_div(K, 64) / 16); }
int64_t mx_scale_kb_bytes(int64_t rows_padded, int64_t K) { return ceil_div(K, 64) * rows_padded * 2; }

hipError_t launch_mx_resolve(const uint8_t* w, const float* s, int64_t N, int64_t K, int64_t BN,
                             int64_t BK, uint16_t* out, hipStream_t stream) {
  const int64_t n = N * ceil_div(K, 8);
  if (n == 0) return hipSuccess;
  const int vec = (K % 8 == 0) && ((uintptr_t)w % 8 == 0) && ((uintptr_t)out % 16 == 0);
  hipLaunchKernelGGL(mx_resolve_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, stream, w, s,
                     N, K, BN, BK, out, vec);
  return hipGetLastError();
}

hipError_t launch_mx_quant(const uint16_t* x, int64_t M, int64_t K, int scale_alg, uint8_t* payload,
                           bool blocked, uint8_t* scale_rm, uint8_t* scale_kb, int64_t Mp,
                           hipStream_t stream) {
  const int64_t n = M * (K / 8);
  if (n == 0) return hipSuccess;
  const int64_t grid = blocked ? ceil_div(M, 16) * ceil_div(K / 8, 16) : ceil_div(n, 256);
  hipLaunchKernelGGL(mx_quant_kernel<0>, dim3((unsigned)grid), dim3(256), 0, stream, x, K,
                     M, K, scale_alg, payload, blocked ? 1 : 0, scale_rm, scale_kb, Mp);
  return hipGetLastError();
}

hipError_t launch_mx_scale_relayout(const uint8_t* src, int64_t R, int64_t K, int64_t Rp,
                                    uint8_t* dst, hipStream_t stream) {
  const int64_t n = ceil_div(K, 64) * Rp * 2;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(mx_scale_relayout_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, stream,
                     src, R, K / 32, Rp, dst);
  return hipGetLastError();
}

hipError_t launch_mx_gemm(const uint8_t* a, const uint8_t* a_scale_kb, int64_t Mp, int64_t M,
                          int64_t K, const uint8_t* w_packed, const uint8_t* w_scale_kb, int64_t N,
                          uint16_t* y, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  MxArgs p{};
  p.a = a;
  p.a_scale = a_scale_kb;
  p.Mp = Mp;
  p.Mclamp = Mp;
  p.w = w_packed;
  p.w_scale = w_scale_kb;
  p.M = M;
  p.N = N;
  p.K = K;
  p.KB = (int)ceil_div(K, 64);
  p.NB = (int)ceil_div(N, 16);
  p.y = y;
  const int64_t T = ceil_div(M, MxDense::BM) * ceil_div(N, MxDense::BN);
  hipLaunchKernelGGL(mx_gemm_kernel, dim3((unsigned)round_up(T, 8)), dim3(64 * MxDense::kWaves), 0, stream,
                     p);
  return hipGetLastError();
}

static int64_t mx_max_big(int64_t R, int64_t E) { return ceil_div(R, MxBig::BM) + E; }
int64_t mx_max_tiles(int64_t R, int64_t E) { return mx_max_big(R, E) + E; }
int64_t mx_padded_rows(int64_t R, int64_t E) { return round_up(R + 15 * E, 16); }

hipError_t launch_mx_swiglu_quant(const uint16_t* h, int64_t R, int64_t I, int scale_alg,
                                  uint8_t* payload, uint8_t* scale_rm, hipStream_t stream) {
  const int64_t n = R * (I / 8);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(mx_quant_kernel<1>, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, stream, h,
                     2 * I, R, I, scale_alg, payload, 0, scale_rm, nullptr, (int64_t)0);
  return hipGetLastError();
}

hipError_t launch_mx_group_schedule(const int64_t* group_list, int64_t E, int64_t R, int4* tiles,
                                    int* counts, hipStream_t stream) {
  hipLaunchKernelGGL(mx_group_schedule_kernel, dim3(1), dim3(1024), 0, stream, group_list, (int)E, R,
                     mx_max_big(R, E), tiles, counts);
  return hipGetLastError();
}

hipError_t launch_mx_quant_tiles(const uint16_t* x, int64_t ldx, int64_t K, int act, const int4* tiles,
                                 const int* counts, int64_t R, int64_t E, int scale_alg,
                                 uint8_t* payload, uint8_t* scale_kb, hipStream_t stream) {
  const dim3 grid((unsigned)(mx_max_tiles(R, E) * kMxSub), (unsigned)mx_quant_ksplit(K));
  const int64_t Rs = mx_padded_rows(R, E);
  if (act)
    hipLaunchKernelGGL(mx_quant_tiles_kernel<1>, grid, dim3(256), 0, stream, x, ldx, K, tiles,
                       counts, mx_max_big(R, E), scale_alg, payload, scale_kb, Rs);
  else
    hipLaunchKernelGGL(mx_quant_tiles_kernel<0>, grid, dim3(256), 0, stream, x, ldx, K, tiles,
                       counts, mx_max_big(R, E), scale_alg, payload, scale_kb, Rs);
  return hipGetLastError();
}

hipError_t launch_mx_grouped_gemm(const uint8_t* payload, const uint8_t* scale_kb, int64_t R,
                                  int64_t E, int64_t K, const int4* tiles, const int* counts,
                                  const uint8_t* w_packed, int64_t w_stride, int64_t w_scale_off,
                                  int64_t N, uint16_t* y, hipStream_t stream) {
  MxArgs p{};
  p.a = payload;
  p.a_scale = scale_kb;
  p.Mp = mx_padded_rows(R, E);
  p.Mclamp = p.Mp;
  p.w = w_packed;
  p.w_scale = nullptr;
  p.M = R;
  p.N = N;
  p.K = K;
  p.KB = (int)ceil_div(K, 64);
  p.NB = (int)ceil_div(N, 16);
  p.y = y;
  const int64_t NT = ceil_div(N, MxBig::BN);
  hipLaunchKernelGGL(mx_grouped_kernel, dim3((unsigned)round_up(mx_max_tiles(R, E) * NT, 8)), dim3(512), 0,
                     stream, p, tiles, counts, mx_max_big(R, E), E, NT, w_stride, w_scale_off);
  return hipGetLastError();
}

}  // namespace w8a8
