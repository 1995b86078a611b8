// Device helpers shared by the gfx950 kernels of the W8A8_DYNAMIC path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Every fp32 expression in these kernels is evaluated one IEEE operation at a
// time: no multiply is fused into an add (the build also passes
// -ffp-contract=off). Bit-exact INT8 codes depend on this.
#pragma clang fp contract(off)

namespace w8a8 {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// BF16
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// fp32 -> BF16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// ---------------------------------------------------------------------------
// Wave-wide max of a non-negative quantity held as uint32 bit patterns.
// Non-negative IEEE floats (and |BF16| bit patterns) order like unsigned ints,
// so the amax of a row is an integer max. DPP steps reduce each 16-lane row
// (xor 1, xor 2, half-row mirror, row mirror); the four row results are read
// into scalars and combined. Every lane returns the wave result.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // row_half_mirror
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));  // row_mirror
  uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return max(max(a, b), max(c, d));
}

// ---------------------------------------------------------------------------
// Symmetric INT8 code of one value: round-half-even(x / s) clamped to
// [-127, 127], x / s one IEEE division; s == 0 (all-zero row) gives 0.
//
// Fast path with the same result: t = x * rcp(s) (v_rcp_f32, within 1 ulp,
// for a normal s) is within |q| * 2^-22 of q = x / s, i.e. within 2^-15 where
// it matters (|q| <= 128: beyond, both roundings clamp to 127); fl32(q) moves
// q by at most 2^-18 there. So |t - fl32(q)| < 2^-14, and when t lies at least
// 2^-14 away from every half-integer, fl32(q) lies on the same side of it and
// rint(fl32(q)) = rint(t). Otherwise (near a tie, or s outside [2^-120,
// 2^120]) the IEEE division decides. |t - rint(t)| is exact (Sterbenz).
// ---------------------------------------------------------------------------
constexpr float kQuantMargin = 0.5f - 0x1p-14f;

__device__ __forceinline__ int quant_code(float x, float s) {
  if (!(s > 0.0f)) return 0;
  if (s >= 0x1p-120f && s <= 0x1p+120f) {
    const float t = x * __builtin_amdgcn_rcpf(s);
    const float n = __builtin_rintf(t);
    if (fabsf(t - n) <= kQuantMargin) return (int)fminf(fmaxf(n, -127.0f), 127.0f);
  }
  float v = __builtin_rintf(x / s);
  v = fminf(fmaxf(v, -127.0f), 127.0f);
  return (int)v;
}

// Pack 4 codes (low byte first) into a uint32.
__device__ __forceinline__ uint32_t pack4(int a, int b, int c, int d) {
  return (uint32_t)(a & 0xFF) | ((uint32_t)(b & 0xFF) << 8) |
         ((uint32_t)(c & 0xFF) << 16) | ((uint32_t)(d & 0xFF) << 24);
}

// quant_code of 8 values with one scale per lane, packed (value 0 in the low
// byte of .x). The fast path of all 8 runs without branches; one wavefront
// vote follows (about 6% of votes over 8 x 64 values find a value within
// 2^-14 of a tie), and only then are the flagged values of the flagged lanes
// done by the division. quant_code one value at a time costs about twice the
// instructions (a branch per value).
__device__ __forceinline__ uint2 quant8(const float (&x)[8], float s) {
  const bool fast = s >= 0x1p-120f && s <= 0x1p+120f;  // false for 0, NaN, extreme scales
  const float r = __builtin_amdgcn_rcpf(s);
  int code[8];
  bool near = !fast;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float t = x[j] * r;
    const float n = __builtin_rintf(t);
    near = near || !(fabsf(t - n) <= kQuantMargin);
    code[j] = (int)fminf(fmaxf(n, -127.0f), 127.0f);
  }
  if (__builtin_amdgcn_ballot_w64(near) != 0) {
    if (near) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float t = x[j] * r;
        if (!fast || !(fabsf(t - __builtin_rintf(t)) <= kQuantMargin)) {
          float v = s > 0.0f ? __builtin_rintf(x[j] / s) : 0.0f;
          code[j] = (int)fminf(fmaxf(v, -127.0f), 127.0f);
        }
      }
    }
  }
  return uint2{pack4(code[0], code[1], code[2], code[3]), pack4(code[4], code[5], code[6], code[7])};
}

// quant8 of 8 BF16 values held as 4 pairs (low half first)
__device__ __forceinline__ uint2 quant8_bf16(const uint32_t (&w)[4], float s) {
  float x[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[2 * j] = __uint_as_float(w[j] << 16);
    x[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
  }
  return quant8(x, s);
}

// ---------------------------------------------------------------------------
// exp(t) by a fixed fp32 sequence (Cody-Waite range reduction with ln2 split
// into a 16-bit head and a tail, then the degree-7 Taylor polynomial of e^r by
// Horner's rule, then one exact scaling by 2^k). Every step is one fp32
// rounding, so any IEEE binary32 implementation of the same steps returns the
// same bits. Accuracy about 1.2 ulp on [-87, 88].
// ---------------------------------------------------------------------------
__device__ __forceinline__ float exp_fixed(float t) {
  const float kLog2e = __uint_as_float(0x3FB8AA3Bu);  // 1/ln2
  const float kLn2Hi = __uint_as_float(0x3F317200u);  // ln2 rounded to 16 bits
  const float kLn2Lo = __uint_as_float(0x35BFBE8Eu);  // ln2 - kLn2Hi
  const float c7 = __uint_as_float(0x39500D01u);      // 1/7!
  const float c6 = __uint_as_float(0x3AB60B61u);      // 1/6!
  const float c5 = __uint_as_float(0x3C088889u);      // 1/5!
  const float c4 = __uint_as_float(0x3D2AAAABu);      // 1/4!
  const float c3 = __uint_as_float(0x3E2AAAABu);      // 1/3!
  const float c2 = 0.5f, c1 = 1.0f, c0 = 1.0f;
  t = fminf(fmaxf(t, -127.0f), 127.0f);
  float k = __builtin_rintf(t * kLog2e);
  float hi = k * kLn2Hi;   // exact: |k| < 2^8 and kLn2Hi has 16 significant bits
  float lo = k * kLn2Lo;
  float r = (t - hi) - lo;
  float p = c7;
  p = p * r + c6;
  p = p * r + c5;
  p = p * r + c4;
  p = p * r + c3;
  p = p * r + c2;
  p = p * r + c1;
  p = p * r + c0;
  return __builtin_ldexpf(p, (int)k);
}

// silu(g) * u with one fp32 rounding per step.
__device__ __forceinline__ float swiglu_fixed(float g, float u) {
  float d = 1.0f + exp_fixed(-g);
  float s = g / d;
  return s * u;
}

// ---------------------------------------------------------------------------
// Expert schedule of the grouped kernels
// ---------------------------------------------------------------------------
constexpr int kMaxExperts = 1024;

// Exclusive prefix sums of the per-expert row counts and m-tile counts, for
// E <= 1024 experts, by a 256-thread workgroup: each thread owns 4 consecutive
// experts, a wavefront scans with shfl_up, and the 4 wave totals are combined
// through LDS. row_off[E] / tile_off[E] receive the totals.
template <int BM>
__device__ void build_schedule(const int64_t* __restrict__ gl, int E, int64_t* row_off,
                               int* tile_off) {
  __shared__ int64_t wave_rows[4];
  __shared__ int wave_tiles[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int64_t n[4];
  int64_t rs = 0;
  int ts = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = 4 * tid + j;
    n[j] = e < E ? max(gl[e], (int64_t)0) : 0;  // a negative count owns no rows
    rs += n[j];
    ts += (int)((n[j] + BM - 1) / BM);
  }
  int64_t ri = rs;
  int ti = ts;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int64_t ro = __shfl_up(ri, d, 64);
    const int to = __shfl_up(ti, d, 64);
    if (lane >= d) {
      ri += ro;
      ti += to;
    }
  }
  if (lane == 63) {
    wave_rows[wave] = ri;
    wave_tiles[wave] = ti;
  }
  __syncthreads();
  int64_t r = ri - rs;
  int t = ti - ts;
  for (int w = 0; w < wave; ++w) {
    r += wave_rows[w];
    t += wave_tiles[w];
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = 4 * tid + j;
    if (e < E) {
      row_off[e] = r;
      tile_off[e] = t;
    }
    r += n[j];
    t += (int)((n[j] + BM - 1) / BM);
  }
  if (tid == 255) {
    row_off[E] = r;
    tile_off[E] = t;
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// MFMA: 16x16x64 INT8 -> INT32. Operand lane l holds 16 bytes: row (A) or
// column (B) l % 16, reduction chunk l / 16. Result lane l holds column l % 16,
// rows 4 * (l / 16) + {0,1,2,3}.
// ---------------------------------------------------------------------------
__device__ __forceinline__ i32x4 mfma16x16x64(const i32x4& a, const i32x4& b, const i32x4& c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

}  // namespace w8a8
