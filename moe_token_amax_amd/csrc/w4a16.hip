// W4A16 weight variant for gfx950 ("超大 MoE 的低比特推理：INT4、FP4 与量化感知训练":
// the INT4 format with one BF16 scale per 32 weights; the quantizer of its QAT
// section, symmetric, scale = group amax / 7, codes rounded and clamped to
// [-8, 7]; the W4A16 kernel row of its kernel table: weights dequantized to
// BF16 in registers, BF16 matrix units, a decode-bound use).
//
//  * quant (load time): per row, per 32 input channels: s = BF16(amax / 7),
//    q = clamp(rint(w / s), -8, 7) against the stored scale (IEEE fp32
//    division, ties to even); amax 0 gives s = 0, q = 0.
//  * packed layout: per 16-column block and 128-deep k-chunk, 1152 bytes:
//    1 KB of codes, lane l's 16 bytes holding column l % 16 and, for each of
//    the chunk's four 32-deep steps j, k = 32 j + 8 (l / 16) + i (i = 0..7) as
//    the nibbles of 32-bit word j (nibble i = bits 4i..4i+3, code + 8), then
//    128 bytes of scales, BF16 [16 columns][4 groups]. K is padded to 128 with
//    code 0 and scale 0; N to 16.
//  * linear: y = BF16(sum_k x[m, k] * BF16(q * s)[n, k]) with the dequantized
//    weight fed to v_mfma_f32_16x16x32_bf16 and fp32 accumulation.
//  * FP4 weights (the same kernel row lists INT4 / FP4; MXFP4 = E2M1 values
//    with one E8M0 scale per 32): E = floor(log2 amax) - 2 per group (2 is
//    E2M1's largest exponent), each w / 2^E encoded to the nearest of 0, 0.5,
//    1, 1.5, 2, 3, 4, 6 (ties to the even code, saturating at 6, sign bit 8);
//    same packed layout with the codes as nibbles and E8M0 bytes [16][4] in
//    the scale area; dequantization 2^E * value is exact in BF16.
#include <algorithm>

#include "device_common.hpp"
#include "w4.hpp"

namespace w8a8 {

constexpr int kW4Group = 32, kW4Chunk = 128, kW4ChunkBytes = 1152;
// FP4 chunks: the 1 KB of codes, then the 16 x 4 E8M0 bytes
constexpr int kFp4ChunkBytes = 1088;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// quant + pack: one thread per (16-column block, k-chunk, lane): the lane's
// column and 8 k per step, the group amax of its (column, step) over the 4
// lanes l, l + 16, l + 32, l + 48 that share it
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void w4_quant_pack_kernel(const uint16_t* __restrict__ w, int64_t N,
                                                            int64_t K, int64_t KC,
                                                            int8_t* __restrict__ q_out,
                                                            uint16_t* __restrict__ s_out,
                                                            uint8_t* __restrict__ packed) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t NB = (N + 15) / 16;
  const int lane = threadIdx.x & 63;
  const int64_t unit = t >> 6;             // one wavefront per (block, chunk)
  if (unit >= NB * KC) return;             // whole wavefront leaves together
  const int64_t nb = unit / KC, kc = unit % KC;
  const int64_t n = nb * 16 + (lane & 15);
  uint32_t words[4];
  uint16_t scales[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t k0 = kc * kW4Chunk + 32 * j + 8 * (lane >> 4);
    const bool live = n < N && k0 < K;
    float v[8];
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[i] = live ? bf16_to_f32(w[n * K + k0 + i]) : 0.f;
      amax = fmaxf(amax, fabsf(v[i]));
    }
    // group of 32 = the 4 lanes of this column in this step (l, l^16, l^32, l^48)
    amax = fmaxf(amax, __shfl_xor(amax, 16, kWave));
    amax = fmaxf(amax, __shfl_xor(amax, 32, kWave));
    const uint32_t sb = f32_to_bf16(amax / 7.0f);
    const float s = bf16_to_f32(sb);
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int code = 0;
      if (s > 0.f) code = (int)fminf(fmaxf(__builtin_rintf(v[i] / s), -8.f), 7.f);
      if (q_out && live) q_out[n * K + k0 + i] = (int8_t)code;
      word |= (uint32_t)(code + 8) << (4 * i);
    }
    words[j] = word;
    scales[j] = (uint16_t)sb;
    if (s_out && live && (lane >> 4) == 0) s_out[n * (K / kW4Group) + (k0 / kW4Group)] = (uint16_t)sb;
  }
  if (packed) {
    uint8_t* base = packed + unit * kW4ChunkBytes;
    reinterpret_cast<uint4*>(base)[lane] = uint4{words[0], words[1], words[2], words[3]};
    if (lane < 16)
      reinterpret_cast<uint2*>(base + 1024)[lane] =
          uint2{scales[0] | ((uint32_t)scales[1] << 16), scales[2] | ((uint32_t)scales[3] << 16)};
  }
}

// pack pre-quantized codes (int8 in [-8, 7]) and BF16 scales
__global__ __launch_bounds__(256) void w4_pack_kernel(const int8_t* __restrict__ q,
                                                      const uint16_t* __restrict__ s, int64_t N,
                                                      int64_t K, int64_t KC,
                                                      uint8_t* __restrict__ packed) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t NB = (N + 15) / 16;
  const int lane = threadIdx.x & 63;
  const int64_t unit = t >> 6;
  if (unit >= NB * KC) return;
  const int64_t nb = unit / KC, kc = unit % KC;
  const int64_t n = nb * 16 + (lane & 15);
  uint32_t words[4];
  uint16_t scales[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t k0 = kc * kW4Chunk + 32 * j + 8 * (lane >> 4);
    const bool live = n < N && k0 < K;
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int code = live ? (int)q[n * K + k0 + i] : 0;
      code = code < -8 ? -8 : (code > 7 ? 7 : code);
      word |= (uint32_t)(code + 8) << (4 * i);
    }
    words[j] = word;
    scales[j] = live ? s[n * (K / kW4Group) + k0 / kW4Group] : (uint16_t)0;
  }
  uint8_t* base = packed + unit * kW4ChunkBytes;
  reinterpret_cast<uint4*>(base)[lane] = uint4{words[0], words[1], words[2], words[3]};
  if (lane < 16)
    reinterpret_cast<uint2*>(base + 1024)[lane] =
        uint2{scales[0] | ((uint32_t)scales[1] << 16), scales[2] | ((uint32_t)scales[3] << 16)};
}

// E2M1 code (0..15) of t = w / 2^E, exact comparisons: each count is a
// half-way point, with the tie going to the even code
__device__ __forceinline__ uint32_t e2m1_code(float t) {
  const float a = fabsf(t);
  uint32_t c = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) + (a >= 3.5f) +
               (a > 5.0f);
  return c | (__float_as_uint(t) >> 31 << 3);
}

// FP4 quant + pack: as w4_quant_pack_kernel, one wavefront per (block, chunk)
__global__ __launch_bounds__(256) void fp4_quant_pack_kernel(const uint16_t* __restrict__ w, int64_t N,
                                                             int64_t K, int64_t KC,
                                                             uint8_t* __restrict__ c_out,
                                                             uint8_t* __restrict__ s_out,
                                                             uint8_t* __restrict__ packed) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t NB = (N + 15) / 16;
  const int lane = threadIdx.x & 63;
  const int64_t unit = t >> 6;
  if (unit >= NB * KC) return;
  const int64_t nb = unit / KC, kc = unit % KC;
  const int64_t n = nb * 16 + (lane & 15);
  uint32_t words[4], sbytes = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t k0 = kc * kW4Chunk + 32 * j + 8 * (lane >> 4);
    const bool live = n < N && k0 < K;
    float v[8];
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[i] = live ? bf16_to_f32(w[n * K + k0 + i]) : 0.f;
      amax = fmaxf(amax, fabsf(v[i]));
    }
    amax = fmaxf(amax, __shfl_xor(amax, 16, kWave));
    amax = fmaxf(amax, __shfl_xor(amax, 32, kWave));
    int e = __builtin_amdgcn_frexp_expf(amax) - 1 - 2;  // floor(log2 amax) - 2
    e = e < -127 ? -127 : (e > 127 ? 127 : e);
    const uint32_t sb = amax > 0.f ? (uint32_t)(e + 127) : 0u;
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // a zero group: codes keep only the sign
      const uint32_t code = amax > 0.f ? e2m1_code(__builtin_ldexpf(v[i], -e))
                                       : (__float_as_uint(v[i]) >> 31 << 3);
      if (c_out && live) c_out[n * K + k0 + i] = (uint8_t)code;
      word |= code << (4 * i);
    }
    words[j] = word;
    sbytes |= sb << (8 * j);
    if (s_out && live && (lane >> 4) == 0) s_out[n * (K / kW4Group) + k0 / kW4Group] = (uint8_t)sb;
  }
  if (packed) {
    uint8_t* base = packed + unit * kFp4ChunkBytes;
    reinterpret_cast<uint4*>(base)[lane] = uint4{words[0], words[1], words[2], words[3]};
    if (lane < 16) reinterpret_cast<uint32_t*>(base + 1024)[lane] = sbytes;
  }
}

// ---------------------------------------------------------------------------
// decode linear: one workgroup per 16-column block and 16 MB rows, WAVES
// wavefronts over interleaved k-chunks (UNR chunks of codes, scales and
// activation fragments loaded before any of them is used), partial sums met
// in LDS
// ---------------------------------------------------------------------------

// 8 BF16 weights of one step from a packed word and the group scale. The
// nibbles are split into the bytes of two words (even and odd nibbles). A
// byte n <= 15 read as OCP E4M3 is n * 2^-9 exactly, so the MX conversion
// v_cvt_scalef32_pk_f32_fp8 with the power-of-two scale 2^9 turns two bytes
// into the floats n0, n1 in one instruction. fma(n, s, -8 s) is then the
// exact q * s (at most 12 significant bits: the fused operation does not
// round), and one RNE to BF16 per value follows.
__device__ __forceinline__ bf16x8 w4_dequant8(uint32_t word, float s) {
  const uint32_t ev = word & 0x0F0F0F0Fu, od = (word >> 4) & 0x0F0F0F0Fu;
  const f32x2 e0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(ev, 512.0f, false);  // nibbles 0, 2
  const f32x2 e1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(ev, 512.0f, true);   // nibbles 4, 6
  const f32x2 o0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(od, 512.0f, false);  // nibbles 1, 3
  const f32x2 o1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(od, 512.0f, true);   // nibbles 5, 7
  const float ms = -8.0f * s;  // exact
  const f32x2 v[4] = {{fmaf(e0.x, s, ms), fmaf(o0.x, s, ms)}, {fmaf(e0.y, s, ms), fmaf(o0.y, s, ms)},
                      {fmaf(e1.x, s, ms), fmaf(o1.x, s, ms)}, {fmaf(e1.y, s, ms), fmaf(o1.y, s, ms)}};
  uint32_t pk[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) pk[b] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v[b], bf16x2));
  return __builtin_bit_cast(bf16x8, uint4{pk[0], pk[1], pk[2], pk[3]});
}

// BF16 activation x [M, K] -> 1 KB blocks [ceil(M/16)][K/32] in the BF16 MFMA's
// A operand order: byte l * 16 of block (mb, kb) holds x[16 mb + l % 16][32 kb
// + 8 (l / 16) .. + 7]; rows past M repeat row M - 1 (their outputs are not
// stored). One thread per 16-byte piece.
__global__ __launch_bounds__(256) void w4_pack_a_kernel(const uint16_t* __restrict__ x, int64_t M,
                                                        int64_t K, uint8_t* __restrict__ out) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t KB = K / 32, MB = (M + 15) / 16;
  if (t >= MB * KB * 64) return;
  const int lane = (int)(t & 63);
  const int64_t blk = t >> 6, mb = blk / KB, kb = blk % KB;
  int64_t row = mb * 16 + (lane & 15);
  row = row < M ? row : M - 1;
  reinterpret_cast<uint4*>(out)[t] =
      *reinterpret_cast<const uint4*>(x + row * K + kb * 32 + 8 * (lane >> 4));
}

// 8 BF16 weights of one step from 8 E2M1 codes (weight 2b in the low nibble
// of byte b, 2b + 1 in the high one) and the group's scale sc = 2^E: gfx950's
// MX conversion v_cvt_scalef32_pk_bf16_fp4 decodes the two codes of one byte
// and multiplies them by sc, so one instruction yields two weights. Every
// value * 2^E is exact in BF16 (at most 2 significant bits; E in [-127, 125]
// for any BF16 group, subnormal results included), so no rounding happens.
__device__ __forceinline__ bf16x8 fp4_dequant8(uint32_t word, float sc) {
  const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, sc, 0);
  const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, sc, 1);
  const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, sc, 2);
  const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, sc, 3);
  return __builtin_bit_cast(bf16x8, uint4{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                                          __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3)});
}

template <int MB, int UNR, int WAVES, int FMT, bool ABLK>
__global__ __launch_bounds__(64 * WAVES) void w4a16_decode_kernel(const uint16_t* __restrict__ x,
                                                                  int64_t M, int64_t K,
                                                                  const uint8_t* __restrict__ wp,
                                                                  int64_t KC, int64_t N,
                                                                  uint16_t* __restrict__ y) {
  // ABLK: x is the packed activation of w4_pack_a_kernel (1 KB blocks)
  __shared__ f32x4 part[WAVES][MB][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t nb = blockIdx.x;
  const int64_t row0 = (int64_t)blockIdx.y * 16 * MB;
  constexpr int64_t kChunkBytes = FMT == 0 ? kW4ChunkBytes : kFp4ChunkBytes;
  const uint8_t* wblk = wp + nb * KC * kChunkBytes;
  // A rows of this lane (row l % 16 of each 16-row block). Rows past M read
  // row M - 1 instead: an MFMA output row depends on its own A row only, and
  // those output rows are not stored.
  const uint16_t* arow[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int64_t r = row0 + 16 * mb + (lane & 15);
    arow[mb] = x + (r < M ? r : M - 1) * K + 8 * (lane >> 4);
  }
  f32x4 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // one chunk per round (UNR 1): the next round's codes and scales are loaded
  // before this round's dequantization, so their HBM latency overlaps it
  constexpr bool PF = UNR == 1;
  auto load_w = [&](int64_t kc, uint4& c, uint2& sv) {
    const uint8_t* ch = wblk + kc * kChunkBytes;
    c = reinterpret_cast<const uint4*>(ch)[lane];
    if (FMT == 0) sv = reinterpret_cast<const uint2*>(ch + 1024)[lane & 15];
    else sv.x = reinterpret_cast<const uint32_t*>(ch + 1024)[lane & 15];
  };
  uint4 codes_n = uint4{0u, 0u, 0u, 0u};
  uint2 sc_n = uint2{0u, 0u};
  if (PF && wave < KC) load_w(wave, codes_n, sc_n);
  for (int64_t c0 = wave; c0 < KC; c0 += WAVES * UNR) {
    // all loads of UNR chunks first (codes, scales and the activation
    // fragments), then the dequantization and the MFMAs
    uint4 codes[UNR];
    uint2 sc[UNR];  // FMT 0: 4 BF16 scales; FMT 1: 4 E8M0 bytes in .x
    bf16x8 a[UNR][4][MB];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int64_t kc = c0 + WAVES * u;
      if (kc >= KC) continue;  // wavefront-uniform; a chunk past KC is never used
      if (PF) {
        codes[u] = codes_n;
        sc[u] = sc_n;
      } else {
        load_w(kc, codes[u], sc[u]);
      }
      // the activation fragment of step j, 16-row block mb (k = 128 kc + 32 j)
      auto afrag = [&](int j, int mb) -> bf16x8 {
        const int64_t k = kc * kW4Chunk + 32 * j;
        if (ABLK) {
          // 16-row blocks past the last packed one read the last (rows >= M: not stored)
          int64_t rb = row0 / 16 + mb;
          rb = rb < (M + 15) / 16 ? rb : (M + 15) / 16 - 1;
          const int64_t blk = rb * (K / 32) + k / 32;
          return reinterpret_cast<const bf16x8*>(reinterpret_cast<const uint8_t*>(x) + blk * 1024)[lane];
        }
        return *reinterpret_cast<const bf16x8*>(arow[mb] + k);
      };
      if ((kc + 1) * kW4Chunk <= K) {  // the whole chunk inside K (wavefront-uniform)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) a[u][j][mb] = afrag(j, mb);
      } else {
        // the last chunk when K % 128 != 0: steps past K (zero-weight padding)
        // take zeros instead of reads past the row
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
            a[u][j][mb] = kc * kW4Chunk + 32 * j < K ? afrag(j, mb) : bf16x8{};
      }
    }
    if (PF && c0 + WAVES < KC) load_w(c0 + WAVES, codes_n, sc_n);  // wavefront-uniform
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int64_t kc = c0 + WAVES * u;
      if (kc >= KC) break;
      const uint32_t cw[4] = {codes[u].x, codes[u].y, codes[u].z, codes[u].w};
      float s[4];
      if (FMT == 0) {
        s[0] = __uint_as_float(sc[u].x << 16);
        s[1] = __uint_as_float(sc[u].x & 0xFFFF0000u);
        s[2] = __uint_as_float(sc[u].y << 16);
        s[3] = __uint_as_float(sc[u].y & 0xFFFF0000u);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)  // 2^E = 2^(byte - 127), byte 0 the subnormal 2^-127
          s[j] = __builtin_ldexpf(1.0f, (int)((sc[u].x >> (8 * j)) & 0xFFu) - 127);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x8 b = FMT == 0 ? w4_dequant8(cw[j], s[j]) : fp4_dequant8(cw[j], s[j]);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u][j][mb], b, acc[mb], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) part[wave][mb][lane] = acc[mb];
  __syncthreads();
  // lane l holds rows 4 (l / 16) .. + 3 of column l % 16 in each 16-row block;
  // wavefronts 0 .. MB - 1 sum the WAVES partials of block mb = wave in order
  if (wave < MB) {
    f32x4 s = part[0][wave][lane];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) s = s + part[w][wave][lane];
    const int64_t n = nb * 16 + (lane & 15);
    if (n < N) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t m = row0 + 16 * wave + 4 * (lane >> 4) + i;
        if (m < M) y[m * N + n] = (uint16_t)f32_to_bf16(s[i]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
int64_t w4_chunks(int64_t K) { return (K + kW4Chunk - 1) / kW4Chunk; }
int64_t w4_packed_bytes(int64_t N, int64_t K) { return (N + 15) / 16 * w4_chunks(K) * kW4ChunkBytes; }
int64_t fp4_packed_bytes(int64_t N, int64_t K) { return (N + 15) / 16 * w4_chunks(K) * kFp4ChunkBytes; }

hipError_t launch_w4_quant_pack(const uint16_t* w, int64_t N, int64_t K, int8_t* q, uint16_t* s,
                                uint8_t* packed, hipStream_t stream) {
  const int64_t units = (N + 15) / 16 * w4_chunks(K);
  if (units == 0) return hipSuccess;
  hipLaunchKernelGGL(w4_quant_pack_kernel, dim3((unsigned)((units + 3) / 4)), dim3(256), 0, stream, w,
                     N, K, w4_chunks(K), q, s, packed);
  return hipGetLastError();
}

hipError_t launch_w4_pack(const int8_t* q, const uint16_t* s, int64_t N, int64_t K, uint8_t* packed,
                          hipStream_t stream) {
  const int64_t units = (N + 15) / 16 * w4_chunks(K);
  if (units == 0) return hipSuccess;
  hipLaunchKernelGGL(w4_pack_kernel, dim3((unsigned)((units + 3) / 4)), dim3(256), 0, stream, q, s, N,
                     K, w4_chunks(K), packed);
  return hipGetLastError();
}

hipError_t launch_fp4_quant_pack(const uint16_t* w, int64_t N, int64_t K, uint8_t* c, uint8_t* s,
                                 uint8_t* packed, hipStream_t stream) {
  const int64_t units = (N + 15) / 16 * w4_chunks(K);
  if (units == 0) return hipSuccess;
  hipLaunchKernelGGL(fp4_quant_pack_kernel, dim3((unsigned)((units + 3) / 4)), dim3(256), 0, stream, w,
                     N, K, w4_chunks(K), c, s, packed);
  return hipGetLastError();
}

int64_t w4_linear_ws_bytes(int64_t M, int64_t K) { return M > 16 ? (M + 15) / 16 * (K / 32) * 1024 : 0; }

template <int FMT>
static hipError_t launch_decode(const uint16_t* x, int64_t M, int64_t K, const uint8_t* wp, int64_t N,
                                uint16_t* y, void* ws, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const int64_t NB = (N + 15) / 16, KC = w4_chunks(K);
  if (M <= 16) {
    hipLaunchKernelGGL((w4a16_decode_kernel<1, 4, 16, FMT, false>), dim3((unsigned)NB, 1), dim3(1024), 0,
                       stream, x, M, K, wp, KC, N, y);
    return hipGetLastError();
  }
  // more rows: the activation is packed into contiguous 1 KB operand blocks
  // first, so that each fragment load of the linear is one contiguous block
  const int64_t pieces = (M + 15) / 16 * (K / 32) * 64;
  hipLaunchKernelGGL(w4_pack_a_kernel, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, stream, x, M,
                     K, reinterpret_cast<uint8_t*>(ws));
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((w4a16_decode_kernel<4, 1, 16, FMT, true>), dim3((unsigned)NB, (unsigned)((M + 63) / 64)),
                     dim3(1024), 0, stream, reinterpret_cast<const uint16_t*>(ws), M, K, wp, KC, N, y);
  return hipGetLastError();
}

hipError_t launch_w4a16_linear(const uint16_t* x, int64_t M, int64_t K, const uint8_t* wp, int64_t N,
                               uint16_t* y, void* ws, hipStream_t stream) {
  return launch_decode<0>(x, M, K, wp, N, y, ws, stream);
}

hipError_t launch_fp4_linear(const uint16_t* x, int64_t M, int64_t K, const uint8_t* wp, int64_t N,
                             uint16_t* y, void* ws, hipStream_t stream) {
  return launch_decode<1>(x, M, K, wp, N, y, ws, stream);
}

}  // namespace w8a8
