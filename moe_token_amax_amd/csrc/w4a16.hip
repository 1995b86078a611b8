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


// ---------------------------------------------------------------------------
// Grouped form: the MoE experts' matmul with low-bit weights. Rows are grouped
// by expert (group_list = rows per expert, as on the INT8 path); expert e's
// packed weight starts at wp + e * w_stride.
//
// Work item = (expert e, 256-column group g, m-tile of up to 64 rows). Items
// are ordered expert, column group, m-tile, and XCD x (workgroups b with
// b % 8 == x) walks its own contiguous eighth of the list, so the m-tiles that
// read the same weight columns run side by side on one XCD and share its L2.
// Every workgroup derives the list from group_list itself (expert scan in
// LDS): no workspace, no host sync.
//
// Workgroup = 4 wavefronts. Wavefront w owns the 16-column n-blocks 4w..4w+3
// of the column group, so each weight is dequantized by exactly one wavefront,
// and all rows of the tile. Per 128-deep k-chunk the tile's activations (MBr
// 16-row blocks x 4 steps of 32, BF16, one 1 KB block per (step, m-block) in
// the MFMA operand order) are loaded into registers 2 chunks ahead, each
// wavefront loading a quarter of the blocks, and written to a ring of 3 LDS
// slots one chunk ahead; each lane's packed codes and scales go to registers,
// also 2 chunks ahead. All global traffic is ordinary loads, so the waits on
// them are the compiler's, by register. One barrier per chunk.
// The MFMA operands are swapped with respect to the linear above: A is the
// dequantized weight (row = n), B the activation (column = m), so result lane
// l holds the 4 adjacent columns n = 4 (l / 16) + {0..3} of row m = l % 16 and
// stores them in one 8-byte write.
//
// Out-of-range reads are clamped, not masked: a row past the expert's last
// reads that last row (its outputs are not stored), a step of the last chunk
// past K reads the chunk's first step (it meets the zero padding of the
// weight: a finite value times +0 adds nothing to the sum), and the loads "2
// chunks ahead" of the last two chunks reload the last chunk (never used).
// ---------------------------------------------------------------------------
constexpr int kLbWaves = 4, kLbNBW = 4, kLbCols = 16 * kLbNBW * kLbWaves, kLbRows = 64, kLbRing = 3;
constexpr int kLbStageMax = 4 * (kLbRows / 16) * 1024;

struct LbArgs {
  const uint16_t* x;     // BF16 rows [R, K]
  const int64_t* gl;     // rows per expert [E]
  const uint8_t* wp;     // packed expert weights, w_stride bytes apart
  uint16_t* y;           // BF16 [R, N]
  int64_t R, K, N, KC, NB, w_stride;
  int E;
};

// codes (16 bytes) and scales (FMT 0: 4 BF16; FMT 1: 4 E8M0 bytes in .x) of the
// wavefront's 4 n-blocks for one chunk
struct LbW {
  uint4 c[kLbNBW];
  uint2 s[kLbNBW];
};

// the LDS writes of this wavefront are done and every wavefront got here (no
// wait on global loads, unlike __syncthreads)
__device__ __forceinline__ void lb_lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int FMT, int MBr>
struct LbItem {
  static constexpr int64_t kChunkBytes = FMT == 0 ? kW4ChunkBytes : kFp4ChunkBytes;
  static constexpr int kStage = 4 * MBr * 1024;

  const uint8_t* wb[kLbNBW];      // n-block bases of this wavefront
  int coff, soff;                 // lane offsets in a chunk: its 16 code bytes, its column's scales
  const uint16_t* ab[MBr];        // activation row of this lane in each of this wavefront's blocks
  int aj[MBr];                    // their step within the chunk, in elements (32 j)
  int ablk[MBr];                  // their block index within a stage

  __device__ __forceinline__ void load_w(LbW& w, int64_t kc) const {
#pragma unroll
    for (int q = 0; q < kLbNBW; ++q) {
      const uint8_t* ch = wb[q] + kc * kChunkBytes;
      w.c[q] = *reinterpret_cast<const uint4*>(ch + coff);
      if (FMT == 0) w.s[q] = *reinterpret_cast<const uint2*>(ch + soff);
      // FP4: .y set too (an undefined half keeps the register sets in memory)
      else w.s[q] = uint2{*reinterpret_cast<const uint32_t*>(ch + soff), 0u};
    }
  }

  __device__ __forceinline__ void load_a(uint4 (&a)[MBr], int64_t kc, int64_t K) const {
#pragma unroll
    for (int i = 0; i < MBr; ++i) {
      const int64_t k0 = kc * kW4Chunk;
      const int64_t col = k0 + aj[i] < K ? k0 + aj[i] : k0;  // wavefront-uniform
      a[i] = *reinterpret_cast<const uint4*>(ab[i] + col);
    }
  }

  __device__ __forceinline__ void store_a(uint8_t* stage, const uint4 (&a)[MBr], int lane) const {
#pragma unroll
    for (int i = 0; i < MBr; ++i) *reinterpret_cast<uint4*>(stage + ablk[i] * 1024 + lane * 16) = a[i];
  }

  __device__ __forceinline__ static void compute(const uint8_t* stage, const LbW& w, f32x4 (&acc)[kLbNBW][MBr],
                                                 int lane) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x8 bw[kLbNBW];
#pragma unroll
      for (int q = 0; q < kLbNBW; ++q) {
        const uint32_t word = j == 0 ? w.c[q].x : j == 1 ? w.c[q].y : j == 2 ? w.c[q].z : w.c[q].w;
        if (FMT == 0) {
          const uint32_t h = j < 2 ? w.s[q].x : w.s[q].y;
          const float sc = __uint_as_float((j & 1) ? (h & 0xFFFF0000u) : (h << 16));
          bw[q] = w4_dequant8(word, sc);
        } else {
          const float sc = __builtin_ldexpf(1.0f, (int)((w.s[q].x >> (8 * j)) & 0xFFu) - 127);
          bw[q] = fp4_dequant8(word, sc);
        }
      }
      bf16x8 ba[MBr];
#pragma unroll
      for (int mb = 0; mb < MBr; ++mb)
        ba[mb] = *reinterpret_cast<const bf16x8*>(stage + (j * MBr + mb) * 1024 + lane * 16);
#pragma unroll
      for (int q = 0; q < kLbNBW; ++q)
#pragma unroll
        for (int mb = 0; mb < MBr; ++mb)
          acc[q][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bw[q], ba[mb], acc[q][mb], 0, 0, 0);
    }
  }

  // register sets of 3 chunks in flight: set c % 3 holds chunk c
  struct Regs {
    LbW w[kLbRing];
    uint4 a[kLbRing][MBr];
  };

  // chunk kc (ring slot and register set S = kc % 3): loads chunk kc + 2 into
  // set (S + 2) % 3, computes chunk kc and writes the activations of chunk
  // kc + 1 to its slot
  template <int S>
  __device__ __forceinline__ void chunk(const LbArgs& p, uint8_t* ring, int64_t kc, Regs& r,
                                        f32x4 (&acc)[kLbNBW][MBr], int lane) const {
    // slot S (written during chunk kc - 1) complete; slot (S + 1) % 3 (chunk
    // kc - 2) no longer read by anyone
    lb_lds_barrier();
    const int64_t kn = kc + 2 < p.KC ? kc + 2 : p.KC - 1;
    load_w(r.w[(S + 2) % kLbRing], kn);
    load_a(r.a[(S + 2) % kLbRing], kn, p.K);
    compute(ring + S * kStage, r.w[S], acc, lane);
    store_a(ring + ((S + 1) % kLbRing) * kStage, r.a[(S + 1) % kLbRing], lane);
  }

  __device__ __forceinline__ void run(const LbArgs& p, uint8_t* ring, int e, int64_t row0, int64_t row_end,
                                      int64_t nb0, int lane, int wave) {
#pragma unroll
    for (int q = 0; q < kLbNBW; ++q) {
      const int64_t nb = nb0 + q < p.NB ? nb0 + q : p.NB - 1;
      wb[q] = p.wp + e * p.w_stride + nb * p.KC * kChunkBytes;
    }
    coff = lane * 16;
    soff = 1024 + (lane & 15) * (FMT == 0 ? 8 : 4);
#pragma unroll
    for (int i = 0; i < MBr; ++i) {
      const int b = wave + kLbWaves * i;  // block b = step j * MBr + m-block mb
      const int j = b / MBr, mb = b % MBr;
      int64_t r = row0 + 16 * mb + (lane & 15);
      r = r < row_end ? r : row_end - 1;
      ab[i] = p.x + r * p.K + 8 * (lane >> 4);
      aj[i] = 32 * j;
      ablk[i] = b;
    }
    f32x4 acc[kLbNBW][MBr];
#pragma unroll
    for (int q = 0; q < kLbNBW; ++q)
#pragma unroll
      for (int mb = 0; mb < MBr; ++mb) acc[q][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
    Regs r;
    const int64_t k1 = p.KC > 1 ? 1 : 0;
    load_a(r.a[0], 0, p.K);
    load_w(r.w[0], 0);
    load_a(r.a[1], k1, p.K);
    load_w(r.w[1], k1);
    store_a(ring, r.a[0], lane);
    // one call site per register set (a second one, for a remainder after
    // the loop, lets the compiler merge them and index the sets at run time)
    for (int64_t kc = 0; kc < p.KC; kc += 3) {
      chunk<0>(p, ring, kc, r, acc, lane);
      if (kc + 1 < p.KC) chunk<1>(p, ring, kc + 1, r, acc, lane);
      if (kc + 2 < p.KC) chunk<2>(p, ring, kc + 2, r, acc, lane);
    }
    // result lane l: columns 4 (l / 16) + {0..3} of n-block q, row l % 16 of m-block mb
#pragma unroll
    for (int q = 0; q < kLbNBW; ++q) {
      if (nb0 + q >= p.NB) continue;  // wavefront-uniform
      const int64_t n = (nb0 + q) * 16 + 4 * (lane >> 4);
#pragma unroll
      for (int mb = 0; mb < MBr; ++mb) {
        const int64_t m = row0 + 16 * mb + (lane & 15);
        if (m < row_end) {
          const f32x4 v = acc[q][mb];
          *reinterpret_cast<uint2*>(p.y + m * p.N + n) =
              uint2{f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16), f32_to_bf16(v[2]) | (f32_to_bf16(v[3]) << 16)};
        }
      }
    }
    lb_lds_barrier();  // every wavefront done with the ring before the next item writes it
  }
};

template <int FMT>
__global__ __launch_bounds__(64 * kLbWaves, 2) void lowbit_grouped_kernel(LbArgs p) {
  static_assert(kLbWaves * kWave == 256, "the expert scan assumes 256 threads");
  __shared__ __attribute__((aligned(1024))) uint8_t ring[kLbRing * kLbStageMax];
  __shared__ int64_t row_off[kMaxExperts + 1];
  __shared__ int tile_off[kMaxExperts + 1];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int E = p.E;
  build_schedule<kLbRows>(p.gl, E, row_off, tile_off);
  const int64_t NG = (p.N + kLbCols - 1) / kLbCols;
  const int64_t total = (int64_t)tile_off[E] * NG;
  const int64_t per = (total + 7) / 8;
  const int64_t first = (int64_t)(blockIdx.x % 8) * per;
  const int64_t end = min(first + per, total);
  const int64_t slots = gridDim.x / 8;  // the grid is a multiple of 8
  for (int64_t i = first + blockIdx.x / 8; i < end; i += slots) {
    // expert of item i: last e with tile_off[e] * NG <= i
    int lo = 0, hi = E - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if ((int64_t)tile_off[mid] * NG <= i) lo = mid; else hi = mid - 1;
    }
    const int e = lo;
    const int64_t mtiles = tile_off[e + 1] - tile_off[e];
    const int64_t local = i - (int64_t)tile_off[e] * NG;
    const int64_t g = local / mtiles, mt = local % mtiles;
    const int64_t row0 = row_off[e] + mt * kLbRows;
    // counts that sum past R are a caller error; rows at or past R are never touched
    const int64_t row_end = min(min(row_off[e + 1], row0 + kLbRows), p.R);
    if (row0 >= row_end) continue;
    const int64_t nb0 = g * (kLbCols / 16) + kLbNBW * wave;
    const int64_t rows = row_end - row0;
    // tiles of 1, 2 or 4 16-row blocks (a third variant of 3 blocks makes the
    // compiler keep a register array in scratch memory)
    if (rows > 32) LbItem<FMT, 4>().run(p, ring, e, row0, row_end, nb0, lane, wave);
    else if (rows > 16) LbItem<FMT, 2>().run(p, ring, e, row0, row_end, nb0, lane, wave);
    else LbItem<FMT, 1>().run(p, ring, e, row0, row_end, nb0, lane, wave);
  }
}

// a = BF16(silu(gate) * up) of h = [gate | up] [R, 2I], the fixed fp32 sequence
// of swiglu_fixed; 8 outputs per thread with 16-byte accesses (VEC) or one
__global__ __launch_bounds__(256) void lowbit_swiglu_vec(const uint16_t* __restrict__ h, int64_t R, int64_t I,
                                                         uint16_t* __restrict__ a) {
  const int64_t per_row = I / 8;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= R * per_row) return;
  const int64_t r = t / per_row, j = (t % per_row) * 8;
  const uint4 g = *reinterpret_cast<const uint4*>(h + r * 2 * I + j);
  const uint4 u = *reinterpret_cast<const uint4*>(h + r * 2 * I + I + j);
  const uint32_t gw[4] = {g.x, g.y, g.z, g.w}, uw[4] = {u.x, u.y, u.z, u.w};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = swiglu_fixed(bf16_to_f32(gw[i] & 0xFFFFu), bf16_to_f32(uw[i] & 0xFFFFu));
    const float hi = swiglu_fixed(bf16_to_f32(gw[i] >> 16), bf16_to_f32(uw[i] >> 16));
    o[i] = f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
  }
  *reinterpret_cast<uint4*>(a + r * I + j) = uint4{o[0], o[1], o[2], o[3]};
}

__global__ __launch_bounds__(256) void lowbit_swiglu_generic(const uint16_t* __restrict__ h, int64_t R,
                                                             int64_t I, uint16_t* __restrict__ a) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= R * I) return;
  const int64_t r = t / I, j = t % I;
  a[t] = (uint16_t)f32_to_bf16(swiglu_fixed(bf16_to_f32(h[r * 2 * I + j]), bf16_to_f32(h[r * 2 * I + I + j])));
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

// ---------------------------------------------------------------------------
// Linear: one workgroup per 16 MB rows x 16 NBW columns, 16 wavefronts over
// interleaved k-chunks. The row-major activation is staged through LDS, one
// region per wavefront. For each chunk (128 k) the wavefront loads its 16 MB
// rows with whole-row 16-byte loads (lane l: row 4 i + l / 16, bytes
// 16 (l % 16) of the chunk's 256), writes them to its region (row pitch 272
// bytes, so that both the writes and the fragment reads below are free of
// bank conflicts), and reads the MFMA fragments back (lane l: row l % 16,
// k 32 j + 8 (l / 16)). Only the wavefront itself touches its region, and its
// LDS operations complete in order, so no barrier is needed. The next chunk's
// codes, scales and activation rows are loaded before this chunk's
// dequantization. A workgroup covers 16 MB rows x 16 NBW columns (grid.y:
// row groups). SKIP (few rows): groups of 4 rows wholly past M are not
// written to LDS either (the fragments then read stale rows, whose outputs
// are never stored). After the loop each wavefront's partial sums go into
// its own region for the reduction.
// ---------------------------------------------------------------------------
template <int MB, int NBW, int FMT, bool SKIP>
__global__ __launch_bounds__(1024) void w4a16_rows_kernel(const uint16_t* __restrict__ x, int64_t M,
                                                          int64_t K, const uint8_t* __restrict__ wp,
                                                          int64_t KC, int64_t N, uint16_t* __restrict__ y) {
  constexpr int WAVES = 16;
  constexpr int R = 16 * MB;                  // rows of the workgroup
  constexpr int kPitch = 2 * kW4Chunk + 16;   // LDS bytes per staged row
  constexpr int kStage = R * kPitch;          // LDS bytes per wavefront
  constexpr int kLoads = R / 4;               // 16-byte row loads per lane and chunk
  static_assert(MB * NBW <= WAVES && MB * NBW * 64 * 16 <= kStage, "partials fit in a region");
  __shared__ __attribute__((aligned(16))) uint8_t lds[WAVES * kStage];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t NB = (N + 15) / 16;
  const int64_t row0 = (int64_t)blockIdx.y * R;
  constexpr int64_t kChunkBytes = FMT == 0 ? kW4ChunkBytes : kFp4ChunkBytes;
  const uint8_t* wblk[NBW];
#pragma unroll
  for (int q = 0; q < NBW; ++q) {
    const int64_t nb = (int64_t)blockIdx.x * NBW + q;
    wblk[q] = wp + (nb < NB ? nb : NB - 1) * KC * kChunkBytes;  // past the last: not stored
  }
  // this lane's staged rows row0 + 4 i + lane / 16 (rows past M load nothing:
  // their outputs are not stored)
  const int64_t r_lane = row0 + (lane >> 4);
  const uint16_t* xr = x + (r_lane < M ? r_lane : 0) * K + 8 * (lane & 15);
  uint8_t* st = lds + wave * kStage;
  auto load_w = [&](int64_t kc, uint4 (&c)[NBW], uint2 (&sv)[NBW]) {
#pragma unroll
    for (int q = 0; q < NBW; ++q) {
      const uint8_t* ch = wblk[q] + kc * kChunkBytes;
      c[q] = reinterpret_cast<const uint4*>(ch)[lane];
      if (FMT == 0) sv[q] = reinterpret_cast<const uint2*>(ch + 1024)[lane & 15];
      else sv[q] = uint2{reinterpret_cast<const uint32_t*>(ch + 1024)[lane & 15], 0u};
    }
  };
  auto load_x = [&](int64_t kc, uint4 (&v)[kLoads]) {
    const bool in = kc * kW4Chunk + 8 * (lane & 15) < K;  // past K: zeros (zero-weight padding)
#pragma unroll
    for (int i = 0; i < kLoads; ++i)
      v[i] = r_lane + 4 * i < M && in ? *reinterpret_cast<const uint4*>(xr + (4 * i) * K + kc * kW4Chunk)
                                      : uint4{0u, 0u, 0u, 0u};
  };
  f32x4 acc[MB][NBW];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int q = 0; q < NBW; ++q) acc[mb][q] = f32x4{0.f, 0.f, 0.f, 0.f};
  uint4 codes_n[NBW], xn[kLoads];
  uint2 sc_n[NBW];
#pragma unroll
  for (int q = 0; q < NBW; ++q) {
    codes_n[q] = uint4{0u, 0u, 0u, 0u};
    sc_n[q] = uint2{0u, 0u};
  }
#pragma unroll
  for (int i = 0; i < kLoads; ++i) xn[i] = uint4{0u, 0u, 0u, 0u};
  if (wave < KC) {
    load_w(wave, codes_n, sc_n);
    load_x(wave, xn);
  }
  for (int64_t kc = wave; kc < KC; kc += WAVES) {
    uint4 codes[NBW];
    uint2 sc[NBW];
#pragma unroll
    for (int q = 0; q < NBW; ++q) {
      codes[q] = codes_n[q];
      sc[q] = sc_n[q];
    }
#pragma unroll
    for (int i = 0; i < kLoads; ++i)
      if (!SKIP || row0 + 4 * i < M)  // wavefront-uniform
        *reinterpret_cast<uint4*>(st + (4 * i + (lane >> 4)) * kPitch + (lane & 15) * 16) = xn[i];
    if (kc + WAVES < KC) {  // wavefront-uniform
      load_w(kc + WAVES, codes_n, sc_n);
      load_x(kc + WAVES, xn);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x8 a[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        a[mb] = *reinterpret_cast<const bf16x8*>(st + (16 * mb + (lane & 15)) * kPitch +
                                                 (4 * j + (lane >> 4)) * 16);
#pragma unroll
      for (int q = 0; q < NBW; ++q) {
        const uint32_t cw = j == 0 ? codes[q].x : j == 1 ? codes[q].y : j == 2 ? codes[q].z : codes[q].w;
        float s;
        if (FMT == 0) {
          const uint32_t sw = j < 2 ? sc[q].x : sc[q].y;
          s = __uint_as_float((j & 1) ? (sw & 0xFFFF0000u) : (sw << 16));
        } else {  // 2^E = 2^(byte - 127), byte 0 the subnormal 2^-127
          s = __builtin_ldexpf(1.0f, (int)((sc[q].x >> (8 * j)) & 0xFFu) - 127);
        }
        const bf16x8 b = FMT == 0 ? w4_dequant8(cw, s) : fp4_dequant8(cw, s);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          acc[mb][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mb], b, acc[mb][q], 0, 0, 0);
      }
    }
  }
  // partials into this wavefront's own region (its last reads are done: LDS
  // operations of a wavefront complete in order)
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int q = 0; q < NBW; ++q)
      *reinterpret_cast<f32x4*>(st + ((mb * NBW + q) * 64 + lane) * 16) = acc[mb][q];
  __syncthreads();
  if (wave < MB * NBW) {
    f32x4 s = *reinterpret_cast<const f32x4*>(lds + (wave * 64 + lane) * 16);
#pragma unroll
    for (int w = 1; w < WAVES; ++w)
      s = s + *reinterpret_cast<const f32x4*>(lds + w * kStage + (wave * 64 + lane) * 16);
    const int mb = wave / NBW, q = wave % NBW;
    const int64_t n = ((int64_t)blockIdx.x * NBW + q) * 16 + (lane & 15);
    if (n < N) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t m = row0 + 16 * mb + 4 * (lane >> 4) + i;
        if (m < M) y[m * N + n] = (uint16_t)f32_to_bf16(s[i]);
      }
    }
  }
}

int64_t w4_linear_ws_bytes(int64_t, int64_t) { return 0; }

template <int FMT>
static hipError_t launch_decode(const uint16_t* x, int64_t M, int64_t K, const uint8_t* wp, int64_t N,
                                uint16_t* y, void* ws, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const int64_t NB = (N + 15) / 16, KC = w4_chunks(K);
  (void)ws;  // no workspace: the activation rows are staged in LDS
  if (M <= 16) {  // one 16-column block per workgroup: 256 workgroups at N = 4096
    hipLaunchKernelGGL((w4a16_rows_kernel<1, 1, FMT, true>), dim3((unsigned)NB, 1), dim3(1024), 0, stream, x, M,
                       K, wp, KC, N, y);
    return hipGetLastError();
  }
  // more rows: a workgroup covers 16 MB rows x 16 NBW columns: INT4 32 x 32,
  // FP4 (whose dequantization is 4 instructions per 8 weights against INT4's
  // 19) 16 x 64, so a workgroup reads 458 / 229 KB of the 64-row activation
  // instead of 917
  constexpr int MB = FMT == 0 ? 2 : 1, NBW = FMT == 0 ? 2 : 4;
  hipLaunchKernelGGL((w4a16_rows_kernel<MB, NBW, FMT, false>),
                     dim3((unsigned)((NB + NBW - 1) / NBW), (unsigned)((M + 16 * MB - 1) / (16 * MB))), dim3(1024),
                     0, stream, x, M, K, wp, KC, N, y);
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

hipError_t launch_lowbit_grouped(int fmt, const uint16_t* x, const int64_t* group_list, int64_t R, int64_t E,
                                 int64_t N, int64_t K, const uint8_t* wp, uint16_t* y, hipStream_t stream) {
  if (R == 0 || N == 0) return hipSuccess;
  LbArgs p;
  p.x = x;
  p.gl = group_list;
  p.wp = wp;
  p.y = y;
  p.R = R;
  p.K = K;
  p.N = N;
  p.KC = w4_chunks(K);
  p.NB = (N + 15) / 16;
  p.w_stride = fmt == 0 ? w4_packed_bytes(N, K) : fp4_packed_bytes(N, K);
  p.E = (int)E;
  // two workgroups per CU, 256 CUs
  constexpr unsigned kGrid = 512;
  if (fmt == 0) hipLaunchKernelGGL(lowbit_grouped_kernel<0>, dim3(kGrid), dim3(64 * kLbWaves), 0, stream, p);
  else hipLaunchKernelGGL(lowbit_grouped_kernel<1>, dim3(kGrid), dim3(64 * kLbWaves), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_lowbit_swiglu(const uint16_t* h, int64_t R, int64_t I, uint16_t* a, hipStream_t stream) {
  if (R == 0) return hipSuccess;
  const bool vec = I % 8 == 0 && ((uintptr_t)h & 15) == 0 && ((uintptr_t)a & 15) == 0;
  const int64_t threads = vec ? R * (I / 8) : R * I;
  const dim3 grid((unsigned)((threads + 255) / 256));
  if (vec) hipLaunchKernelGGL(lowbit_swiglu_vec, grid, dim3(256), 0, stream, h, R, I, a);
  else hipLaunchKernelGGL(lowbit_swiglu_generic, grid, dim3(256), 0, stream, h, R, I, a);
  return hipGetLastError();
}

}  // namespace w8a8
