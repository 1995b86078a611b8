// INT8 x INT8 -> INT32 GEMM kernels for gfx950 with the fused dequant epilogue.
//
// ("DeepSeek-V4 W8A8 执行链从量化权重到 Ascend INT8 算子": §二 npu_quant_matmul
// with a per-token and a per-channel scale, optional bias, BF16 output;
// §三 npu_grouped_matmul driven by group_list; §四 the kernel variant depends
// on M, so prefill-sized and decode-sized calls take different tilings.)
//
// Data path of one workgroup tile (BM x BN, K in stages of BKB*64):
//   * A (activations, int8 row-major) and B (weights prepacked in 1 KB blocks
//     of 16 columns x 64 k, already in MFMA operand order) are copied
//     global -> VGPR -> LDS by whole 1 KB blocks: one wavefront instruction
//     moves one block, lane l carrying bytes [16l, 16l+16). For A the lane
//     reads row l%16, k-chunk l/16 of the block, so LDS receives A in the same
//     MFMA operand order as B and every LDS write and read is a linear 16 B per
//     lane (no bank conflicts).
//   * Two LDS stages: the global loads of stage s+1 are in flight while the
//     MFMAs of stage s run.
//   * Each wavefront owns a (BM/WM) x (BN/WN) sub-tile of 16x16 INT32
//     accumulators and issues v_mfma_i32_16x16x64_i8.
//   * Epilogue in registers: y = BF16(((float(acc) * xs[m]) * ws[n]) + b[n]),
//     or the raw INT32 sums.
#include "device_common.hpp"
#include "launch.hpp"

namespace w8a8 {

constexpr int kBlockBytes = 1024;  // 16 rows/cols x 64 k of int8

struct GemmArgs {
  const int8_t* a;          // [rows, K] row-major, row stride lda
  const float* a_scale;     // [rows]
  int64_t M;                // rows (dense) / R (grouped)
  int64_t K;
  int KB;                   // packed k-blocks: ceil(K / 64)
  const uint8_t* w;         // packed weight
  int NB;                   // packed n-blocks per expert: ceil(N / 16)
  const float* w_scale;     // [E, N]
  int64_t N;
  const uint16_t* bias;     // [N] or null
  void* y;                  // [rows, N], row stride ldy
  int out;                  // OutKind
  int a_blk;                // A in 1 KB blocks [ceil(M/16)][KB] (dense kernels only)
  bool a_vec;               // K % 16 == 0 and a 16-byte aligned
  const int64_t* group_list;  // grouped only
  int E;
  // static W8A8 (dense kernels): the integer bias added to the accumulator,
  // with w_scale holding the dequant scale and a_scale / bias unused; null
  // for the dynamic scheme
  const int32_t* qbias;
  int64_t lda, ldy;         // row strides of row-major A and of y (K and N unless given)
};

// fp32 value of one output before the BF16 rounding. Dynamic scheme:
// ((fp32(acc) * xs) * ws) + bias. Static scheme: fp32(acc + qb) * ws, ws the
// dequant scale. One IEEE rounding per operation, no fused multiply-add.
__device__ __forceinline__ float out_value(const GemmArgs& p, int32_t acc, float xs, float ws,
                                           float b, int32_t qb) {
  if (p.qbias) return (float)(acc + qb) * ws;
  float f = (float)acc;
  f = f * xs;
  f = f * ws;
  if (p.bias) f = f + b;
  return f;
}

// threadIdx.x through an empty asm statement: values derived from it are
// computed where they are used instead of being hoisted out of a persistent
// loop and kept live across all of its work items (which ran the grouped
// kernel out of registers).
__device__ __forceinline__ int opaque_tid() {
  int t = (int)threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// 16 bytes of A: row `row`, columns [kcol, kcol + 16). Rows outside
// [.., row_end) and columns at or past K read as zero.
__device__ __forceinline__ i32x4 load_a16(const GemmArgs& p, int64_t row, int64_t row_end,
                                          int64_t kcol) {
  i32x4 v = {0, 0, 0, 0};
  if (row >= row_end || kcol >= p.K) return v;
  const int8_t* src = p.a + row * p.lda + kcol;
  if (p.a_vec) return *reinterpret_cast<const i32x4*>(src);
  uint32_t w[4] = {0, 0, 0, 0};
  const int64_t n = min((int64_t)16, p.K - kcol);
  for (int j = 0; j < n; ++j) w[j >> 2] |= (uint32_t)(uint8_t)src[j] << (8 * (j & 3));
  v[0] = (int)w[0];
  v[1] = (int)w[1];
  v[2] = (int)w[2];
  v[3] = (int)w[3];
  return v;
}

template <int BM, int BN, int WM, int WN, int BKB>
struct Tile {
  static constexpr int kThreads = WM * WN * kWave;
  static constexpr int kWaves = WM * WN;
  static constexpr int TM = BM / WM / 16;
  static constexpr int TN = BN / WN / 16;
  static constexpr int kABlocks = (BM / 16) * BKB;
  static constexpr int kBBlocks = (BN / 16) * BKB;
  static constexpr int kBlocks = kABlocks + kBBlocks;
  static constexpr int kPerWave = (kBlocks + kWaves - 1) / kWaves;
  static constexpr int kStageBytes = kBlocks * kBlockBytes;
  static_assert(BM % (16 * WM) == 0 && BN % (16 * WN) == 0, "tile shape");
  static_assert(kBlocks % kWaves == 0, "blocks must split evenly over waves");

  // Copies the blocks of one K stage owned by this wave into registers.
  __device__ __forceinline__ static void load_stage(const GemmArgs& p, i32x4 (&r)[kPerWave],
                                                    int wave, int lane, int64_t row0,
                                                    int64_t row_end, int64_t wblk0, int nb0,
                                                    int kb_stage, int kb_end) {
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int bi = wave + i * kWaves;
      i32x4 v = {0, 0, 0, 0};
      if (bi < kABlocks) {
        const int mb = bi / BKB, kbl = bi % BKB;
        const int kb = kb_stage + kbl;
        if (kb < kb_end)
          v = load_a16(p, row0 + mb * 16 + (lane & 15), row_end,
                       (int64_t)kb * 64 + (lane >> 4) * 16);
      } else {
        const int bj = bi - kABlocks;
        const int nb = bj / BKB, kbl = bj % BKB;
        const int kb = kb_stage + kbl;
        if (kb < kb_end && nb0 + nb < p.NB)
          v = *reinterpret_cast<const i32x4*>(p.w + (wblk0 + (int64_t)(nb0 + nb) * p.KB + kb) *
                                                        kBlockBytes + lane * 16);
      }
      r[i] = v;
    }
  }

  __device__ __forceinline__ static void store_stage(uint8_t* stage, const i32x4 (&r)[kPerWave],
                                                     int wave, int lane) {
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int bi = wave + i * kWaves;
      *reinterpret_cast<i32x4*>(stage + bi * kBlockBytes + lane * 16) = r[i];
    }
  }

  __device__ __forceinline__ static void compute_stage(const uint8_t* stage,
                                                       i32x4 (&acc)[TM][TN], int wm, int wn,
                                                       int lane) {
#pragma unroll
    for (int kbl = 0; kbl < BKB; ++kbl) {
      i32x4 af[TM], bf[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *reinterpret_cast<const i32x4*>(stage + ((wm * TM + i) * BKB + kbl) * kBlockBytes +
                                                lane * 16);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bf[j] = *reinterpret_cast<const i32x4*>(
            stage + (kABlocks + (wn * TN + j) * BKB + kbl) * kBlockBytes + lane * 16);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma16x16x64(af[i], bf[j], acc[i][j]);
    }
  }

  // Full K loop of one tile: rows [row0, row_end) of A (row0 is the tile's
  // first row), weight blocks of expert `e` starting at n-block nb0,
  // k-blocks [kb_begin, kb_end).
  __device__ __forceinline__ static void mainloop(const GemmArgs& p, uint8_t* smem,
                                                  i32x4 (&acc)[TM][TN], int64_t row0,
                                                  int64_t row_end, int e, int nb0, int kb_begin,
                                                  int kb_end) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int64_t wblk0 = (int64_t)e * p.NB * p.KB;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = i32x4{0, 0, 0, 0};
    const int nst = (kb_end - kb_begin + BKB - 1) / BKB;
    if (nst <= 0) return;
    i32x4 r[kPerWave];
    load_stage(p, r, wave, lane, row0, row_end, wblk0, nb0, kb_begin, kb_end);
    store_stage(smem, r, wave, lane);
    __syncthreads();
    for (int s = 0; s < nst; ++s) {
      uint8_t* cur = smem + (s & 1) * kStageBytes;
      uint8_t* nxt = smem + ((s + 1) & 1) * kStageBytes;
      const bool more = s + 1 < nst;
      if (more)
        load_stage(p, r, wave, lane, row0, row_end, wblk0, nb0, kb_begin + (s + 1) * BKB, kb_end);
      __builtin_amdgcn_sched_barrier(0);  // next stage's loads issue before this stage's MFMAs
      compute_stage(cur, acc, wm, wn, lane);
      if (more) store_stage(nxt, r, wave, lane);
      __syncthreads();
    }
  }

  // Writes the tile. Local row i of the tile is global row row0 + i; rows at or
  // past row_end and columns at or past N are skipped. `e` selects the w_scale
  // row.
  __device__ __forceinline__ static void epilogue(const GemmArgs& p, const i32x4 (&acc)[TM][TN],
                                                  int64_t row0, int64_t row_end, int e, int64_t n0) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const float* wsc = p.w_scale + (int64_t)e * p.N;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int64_t n = n0 + (wn * TN + j) * 16 + (lane & 15);
      if (n >= p.N) continue;
      const float ws = wsc[n];
      const float b = p.bias ? bf16_to_f32(p.bias[n]) : 0.0f;
      const int32_t qb = p.qbias ? p.qbias[n] : 0;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int64_t m = row0 + (wm * TM + i) * 16 + (lane >> 4) * 4 + t;
          if (m >= row_end) continue;
          const int32_t v = acc[i][j][t];
          if (p.out == kOutI32) {
            reinterpret_cast<int32_t*>(p.y)[m * p.ldy + n] = v;
          } else {
            const float f = out_value(p, v, p.a_scale ? p.a_scale[m] : 0.0f, ws, b, qb);
            reinterpret_cast<uint16_t*>(p.y)[m * p.ldy + n] = (uint16_t)f32_to_bf16(f);
          }
        }
      }
    }
  }
};

// ---------------------------------------------------------------------------
// LDS-DMA pipelined tile (K % 16 == 0 and 16-byte aligned activations).
//
// Four wavefronts (2 x 2), each owning a (BM/2) x (BN/2) block of 16x16 INT32
// accumulators. K advances one 64-deep k-block per stage through a ring of
// STAGES LDS buffers filled by global_load_lds_dwordx4: the data goes from
// L2 straight into LDS with no VGPR staging, and lane l of the instruction
// lands at byte 16*l of a 1 KB block, i.e. already in MFMA operand order (A:
// row l%16, k-chunk l/16; B: the prepacked block). STAGES-1 k-blocks are in
// flight while one is consumed. Every stage ends with
// "s_waitcnt vmcnt(<loads of later stages>) lgkmcnt(0); s_barrier": the
// wavefront's own loads of the stage it is about to read have landed, its
// LDS reads of the previous stage are done, and every other wavefront got
// that far too, so the buffer refilled next is free.
//
// Reads that would leave the operands are clamped to valid addresses instead
// of being masked: an A row past the tile's last row reads that last row (it
// only feeds output rows that are never stored), an A column past K reads the
// last 16 bytes of the row (multiplied by the zero padding of the weight), and
// an n-block past the weight's last one reads the last block (it only feeds
// columns >= N, never stored).
// ---------------------------------------------------------------------------
#define W8A8_LDS __attribute__((address_space(3)))

template <int VM>
__device__ __forceinline__ void wait_vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(VM) : "memory");
}

#ifndef W8A8_DMA_STAGES
#define W8A8_DMA_STAGES 5
#endif
#ifndef W8A8_DMA_GROUP_M
#define W8A8_DMA_GROUP_M 8
#endif
#ifndef W8A8_DMA_WM
#define W8A8_DMA_WM 2
#endif
#ifndef W8A8_DMA_WN
#define W8A8_DMA_WN 4
#endif

template <int BM, int BN, int STAGES, int WM, int WN>
struct DmaTile {
  static constexpr int kWaves = WM * WN;
  static constexpr int kThreads = kWaves * kWave;
  static constexpr int TM = BM / WM / 16;  // 16x16 accumulator blocks per wavefront
  static constexpr int TN = BN / WN / 16;
  static constexpr int kABlocks = BM / 16;
  static constexpr int kBBlocks = BN / 16;
  static constexpr int kBlocks = kABlocks + kBBlocks;
  static constexpr int kPerWave = kBlocks / kWaves;
  static constexpr int kStageBytes = kBlocks * kBlockBytes;
  static constexpr int kLdsBytes = STAGES * kStageBytes;
  static_assert(kBlocks % kWaves == 0 && TM >= 2 && TM % 2 == 0 && TN >= 1, "tile shape");
  static_assert(STAGES == 5, "stages");
  static_assert(3 * kPerWave <= 63, "vmcnt range");

  // Per-tile DMA sources of this wavefront's kPerWave blocks: a wave-uniform
  // base (the activation, or this expert's packed weight), a per-lane 32-bit
  // byte offset of k-block 0 and the step per k-block (64 bytes along an A
  // row, 1 KB through the packed weight). Block bi < kABlocks is A rows
  // [16*bi, 16*bi + 16). The host keeps M * K and N * K below 2^32 here.
  struct Src {
    const uint8_t* base[kPerWave];
    uint32_t off[kPerWave];
    int step[kPerWave];
    uint32_t adj;  // pull-back of this lane's A chunk in the last k-block of a ragged K
  };

  // The LDS fragments one wavefront reads from a stage: TN B blocks, TM A blocks.
  struct Frags {
    i32x4 b[TN];
    i32x4 a[TM];
  };

  __device__ __forceinline__ static void sources(const GemmArgs& p, Src& s, int wave, int lane,
                                                 int64_t row0, int64_t row_last, int64_t wblk0,
                                                 int nb0) {
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int bi = wave * kPerWave + i;  // wave-uniform
      if (bi < kABlocks && p.a_blk) {
        // packed A: 16-row block mb, k-block kb at (mb * KB + kb) KB; blocks
        // past the last one are read clamped
        int64_t mb = row0 / 16 + bi;
        mb = mb < row_last / 16 ? mb : row_last / 16;
        s.base[i] = reinterpret_cast<const uint8_t*>(p.a);
        s.off[i] = (uint32_t)(mb * p.KB * kBlockBytes + lane * 16);
        s.step[i] = kBlockBytes;
      } else if (bi < kABlocks) {
        int64_t row = row0 + bi * 16 + (lane & 15);
        row = row < row_last ? row : row_last;
        s.base[i] = reinterpret_cast<const uint8_t*>(p.a);
        s.off[i] = (uint32_t)(row * p.lda + (lane >> 4) * 16);
        s.step[i] = 64;
      } else {
        int nb = nb0 + (bi - kABlocks);
        nb = nb < p.NB ? nb : p.NB - 1;
        s.base[i] = p.w + wblk0 * kBlockBytes;
        s.off[i] = (uint32_t)((int64_t)nb * p.KB * kBlockBytes + lane * 16);
        s.step[i] = kBlockBytes;
      }
    }
    // last k-block of a ragged K: a 16-byte A chunk that would run past the
    // row end is read from K - 16 instead (its values meet zero weights)
    const int64_t col = (int64_t)(p.KB - 1) * 64 + (lane >> 4) * 16;
    s.adj = (!p.a_blk && col > p.K - 16) ? (uint32_t)(col - (p.K - 16)) : 0u;
  }

  // DMA of block i (of this wavefront) of k-block kb into ring buffer buf.
  __device__ __forceinline__ static void issue_one(const GemmArgs& p, const Src& s, uint8_t* smem,
                                                   int buf, int kb, int wave, int lane, int i) {
    const int bi = wave * kPerWave + i;
    uint32_t off = s.off[i] + (uint32_t)(kb * s.step[i]);
    if (bi < kABlocks && kb == p.KB - 1) off -= s.adj;  // wave-uniform condition
    W8A8_LDS void* dst =
        (W8A8_LDS void*)((W8A8_LDS uint8_t*)smem + buf * kStageBytes + bi * kBlockBytes);
    __builtin_amdgcn_global_load_lds(s.base[i] + off, dst, 16, 0, 0);
  }

  __device__ __forceinline__ static void read_frags(const uint8_t* st, Frags& f, int wm, int wn,
                                                    int lane) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
      f.b[j] = *reinterpret_cast<const i32x4*>(st + (kABlocks + wn * TN + j) * kBlockBytes +
                                               lane * 16);
#pragma unroll
    for (int i = 0; i < TM; ++i)
      f.a[i] = *reinterpret_cast<const i32x4*>(st + (wm * TM + i) * kBlockBytes + lane * 16);
  }

  __device__ __forceinline__ static void mfma_row(const Frags& f, i32x4 (&acc)[TM][TN], int i) {
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = mfma16x16x64(f.a[i], f.b[j], acc[i][j]);
  }

  __device__ __forceinline__ static void mfma_rows(const Frags& f, i32x4 (&acc)[TM][TN], int lo,
                                                   int hi) {
#pragma unroll
    for (int i = lo; i < hi; ++i) mfma_row(f, acc, i);
  }

  // Full K loop over rows [row0, row_end) (row_end > row0), weights of expert
  // e from n-block nb0. Rows past row_end are read clamped and computed; only
  // the epilogue drops them. Ends with every wavefront past its last LDS read.
  //
  // The ring holds five k-blocks (the whole 160 KB of LDS) and advances two at
  // a time, with one wait + barrier per pair of k-blocks (kb, kb + 1) whose
  // fragments are F and G:
  //   DMA of kb + 4 into the buffer of kb - 1 | F rows 0..H-1 | LDS reads of
  //   G | F rows H..TM-1 | G rows 0..H-1 | wait for the DMA of kb + 2, kb + 3
  //   (kb + 4 stays in flight), s_barrier | LDS reads of the next F (kb + 2) |
  //   DMA of kb + 5 into the buffer of kb | G rows H..TM-1.
  // The DMA of each pair is split over two points, after the next fragment
  // reads and before the next pair's first rows, rather than issued all at
  // once after the barrier (that burst cost about 6% of the prefill GEMM).
  // So two to three k-blocks of DMA are always in flight (a wait for every
  // load at each barrier would drain the DMA queue and expose its latency once
  // per pair), one barrier per two k-blocks keeps the two wavefronts of a SIMD
  // out of lockstep (a barrier per k-block cost about a fifth of the loop),
  // the LDS reads run under MFMAs, and F / G are distinct register sets, so no
  // fragment or accumulator is copied.
  __device__ __forceinline__ static void mainloop(const GemmArgs& p, uint8_t* smem,
                                                  i32x4 (&acc)[TM][TN], int64_t row0,
                                                  int64_t row_end, int e, int nb0) {
    static_assert(STAGES == 5, "the pairwise ring needs five k-block buffers");
    const int lane = opaque_tid() & 63;
    // wave index as a scalar: per-wave choices are uniform branches and the
    // LDS destination of every DMA is an SGPR (M0)
    const int wave = __builtin_amdgcn_readfirstlane(opaque_tid() >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int64_t wblk0 = (int64_t)e * p.NB * p.KB;
    const int KB = p.KB;
    constexpr int H = TM / 2;
    Src src;
    sources(p, src, wave, lane, row0, row_end - 1, wblk0, nb0);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = i32x4{0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < 5; ++s)
      if (s < KB) {
#pragma unroll
        for (int i = 0; i < kPerWave; ++i) issue_one(p, src, smem, s, s, wave, lane, i);
      }
    // k-blocks 0 and 1 landed; 2, 3 and 4 may still be in flight
    if (KB >= 5) wait_vm_barrier<3 * kPerWave>();
    else if (KB == 4) wait_vm_barrier<2 * kPerWave>();
    else if (KB == 3) wait_vm_barrier<kPerWave>();
    else wait_vm_barrier<0>();
    Frags F, G;
    read_frags(smem, F, wm, wn, lane);
    int buf = 0;  // ring buffer of k-block kb (kb % 5)
    int pend_buf = -1, pend_kb = 0;  // the DMA deferred to the next pair (kb + 4 there)
    for (int kb = 0; kb < KB; kb += 2) {
      const int buf1 = buf == 4 ? 0 : buf + 1;
      const int buf2 = buf1 == 4 ? 0 : buf1 + 1;
      const bool has1 = kb + 1 < KB;
      const bool more = kb + 2 < KB;
      __builtin_amdgcn_sched_barrier(0);
      if (pend_buf >= 0) {  // wave-uniform
#pragma unroll
        for (int i = 0; i < kPerWave; ++i) issue_one(p, src, smem, pend_buf, pend_kb, wave, lane, i);
        pend_buf = -1;
      }
      __builtin_amdgcn_sched_barrier(0);
      mfma_rows(F, acc, 0, H);
      __builtin_amdgcn_sched_barrier(0);
      if (has1) read_frags(smem + buf1 * kStageBytes, G, wm, wn, lane);
      __builtin_amdgcn_sched_barrier(0);
      mfma_rows(F, acc, H, TM);
      __builtin_amdgcn_sched_barrier(0);
      if (has1) mfma_rows(G, acc, 0, H);
      __builtin_amdgcn_sched_barrier(0);
      if (more) {
        // every wavefront's DMA of kb + 2 and kb + 3 landed (kb + 4 may still
        // be in flight: it is the last one issued), every read of the
        // buffers of kb and kb + 1 done; refill those with kb + 5 now and
        // kb + 6 at the start of the next pair (the vmcnt order stays the
        // issue order: kb + 6 is again the last one in flight at the next wait)
        if (kb + 4 < KB) wait_vm_barrier<kPerWave>();
        else wait_vm_barrier<0>();
        if (kb + 6 < KB) {
          pend_buf = buf1;
          pend_kb = kb + 6;
        }
        read_frags(smem + buf2 * kStageBytes, F, wm, wn, lane);
        if (kb + 5 < KB) {
#pragma unroll
          for (int i = 0; i < kPerWave; ++i) issue_one(p, src, smem, buf, kb + 5, wave, lane, i);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if (has1) mfma_rows(G, acc, H, TM);
      buf = buf2;
    }
    // all LDS reads of this tile done in every wavefront before smem is reused
    wait_vm_barrier<0>();
  }

  // Output element of accumulator register v of block (i, j) for this lane:
  // row 4*(l/16) + v, column l%16 of the 16x16 block.
  __device__ __forceinline__ static void epilogue(const GemmArgs& p, const i32x4 (&acc)[TM][TN],
                                                  int64_t row0, int64_t row_end, int e,
                                                  int64_t n0) {
    const int lane = opaque_tid() & 63;
    const int wave = opaque_tid() >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const float* wsc = p.w_scale + (int64_t)e * p.N;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int64_t n = n0 + (wn * TN + j) * 16 + (lane & 15);
      if (n >= p.N) continue;
      const float ws = wsc[n];
      const float b = p.bias ? bf16_to_f32(p.bias[n]) : 0.0f;
      const int32_t qb = p.qbias ? p.qbias[n] : 0;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int64_t m = row0 + (wm * TM + i) * 16 + (lane >> 4) * 4 + v;
          if (m >= row_end) continue;
          const int32_t val = acc[i][j][v];
          if (p.out == kOutI32) {
            reinterpret_cast<int32_t*>(p.y)[m * p.ldy + n] = val;
          } else {
            const float f = out_value(p, val, p.a_scale ? p.a_scale[m] : 0.0f, ws, b, qb);
            reinterpret_cast<uint16_t*>(p.y)[m * p.ldy + n] = (uint16_t)f32_to_bf16(f);
          }
        }
      }
    }
  }

  // BF16 epilogue through LDS (the ring is idle after the K loop): every
  // wavefront writes its BF16 results into a row-major BM x BN tile (row pitch
  // BN * 2 + 16 bytes, so the four row groups of a 16x16 block land in
  // different banks), then the workgroup writes whole rows with 16-byte
  // stores. The values are the direct epilogue's, bit for bit; only the store
  // pattern changes (each 128-byte line of y is written by one instruction
  // instead of four 32-byte pieces spread over the epilogue).
  static constexpr int kPitch = BN * 2 + 16;
  static_assert(BM * kPitch <= kLdsBytes, "staged tile fits the LDS ring");

  __device__ __forceinline__ static void epilogue_staged(const GemmArgs& p, const i32x4 (&acc)[TM][TN],
                                                         uint8_t* smem, int64_t row0, int64_t row_end,
                                                         int e, int64_t n0) {
    const int lane = opaque_tid() & 63;
    const int wave = opaque_tid() >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const float* wsc = p.w_scale + (int64_t)e * p.N;
    // this lane's element (i, j, v) sits at lbase + i * 16 * kPitch + v * kPitch + j * 32
    const int r0 = wm * TM * 16 + (lane >> 4) * 4;
    const int c0 = wn * TN * 16 + (lane & 15);
    uint8_t* lbase = smem + r0 * kPitch + c0 * 2;
    float xs[TM][4];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t m = row0 + r0 + i * 16 + v;
        xs[i][v] = p.a_scale ? p.a_scale[m < row_end ? m : row_end - 1] : 0.0f;
      }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int64_t n = n0 + c0 + j * 16;
      const int64_t nc = n < p.N ? n : p.N - 1;  // columns past N: computed, never stored
      const float ws = wsc[nc];
      const float b = p.bias ? bf16_to_f32(p.bias[nc]) : 0.0f;
      const int32_t qb = p.qbias ? p.qbias[nc] : 0;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float f = out_value(p, acc[i][j][v], xs[i][v], ws, b, qb);
          *reinterpret_cast<uint16_t*>(lbase + (i * 16 + v) * kPitch + j * 32) =
              (uint16_t)f32_to_bf16(f);
        }
      }
    }
    __syncthreads();
    constexpr int kChunks = BN * 2 / 16;  // 16-byte pieces per staged row
    const bool vec = (p.N % 8 == 0) && (p.ldy % 8 == 0) && (((uintptr_t)p.y & 15) == 0);
    for (int c = opaque_tid(); c < BM * kChunks; c += kThreads) {
      const int r = c / kChunks, cc = c % kChunks;
      const int64_t m = row0 + r;
      if (m >= row_end) continue;
      const int64_t n = n0 + cc * 8;
      if (n >= p.N) continue;
      const uint8_t* src = smem + r * kPitch + cc * 16;
      uint16_t* dst = reinterpret_cast<uint16_t*>(p.y) + m * p.ldy + n;
      if (vec && n + 8 <= p.N) {
        *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
      } else {
        for (int t = 0; t < 8 && n + t < p.N; ++t) dst[t] = reinterpret_cast<const uint16_t*>(src)[t];
      }
    }
    // the LDS is the next tile's ring: every read of the staged tile done first
    __syncthreads();
  }
};

// Tile index -> (tm, tn). Workgroup w runs on XCD w % 8 (round-robin
// dispatch), so each XCD is given a contiguous range of tile indices, and
// inside a range tiles go GROUP_M m-rows at a time: the tiles an XCD runs
// together share A rows and weight columns in that XCD's L2.
template <int GROUP_M>
__device__ __forceinline__ bool xcd_tile(int64_t w, int64_t MT, int64_t NT, int64_t& tm,
                                         int64_t& tn) {
  const int64_t T = MT * NT;
  const int64_t per = (T + 7) / 8;
  const int64_t t = (w % 8) * per + w / 8;
  if (t >= T) return false;
  const int64_t in_group = (int64_t)GROUP_M * NT;
  const int64_t g = t / in_group;
  const int64_t first_m = g * GROUP_M;
  const int64_t gm = MT - first_m < GROUP_M ? MT - first_m : GROUP_M;
  const int64_t r = t % in_group;
  tm = first_m + r % gm;
  tn = r / gm;
  return true;
}

template <int BM, int BN, int STAGES, int GROUP_M, int WM, int WN>
__global__ __launch_bounds__(WM* WN* kWave) void dense_dma_kernel(GemmArgs p) {
  using T = DmaTile<BM, BN, STAGES, WM, WN>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[T::kLdsBytes];
  const int64_t MT = (p.M + BM - 1) / BM, NT = (p.N + BN - 1) / BN;
  // grid = 8 * ceil(MT*NT / 8): a few workgroups of the last XCD range may be idle
  int64_t tm, tn;
  if (!xcd_tile<GROUP_M>(blockIdx.x, MT, NT, tm, tn)) return;
  const int64_t row0 = tm * BM;
  const int64_t row_end = min(row0 + BM, p.M);
  i32x4 acc[T::TM][T::TN];
  T::mainloop(p, smem, acc, row0, row_end, 0, (int)(tn * BN / 16));
  if (p.out == kOutI32) T::epilogue(p, acc, row0, row_end, 0, tn * BN);
  else T::epilogue_staged(p, acc, smem, row0, row_end, 0, tn * BN);
}

// ---------------------------------------------------------------------------
// dense kernel (M > 64): grid.x = tiles, n fastest
// ---------------------------------------------------------------------------
template <int BM, int BN, int WM, int WN, int BKB>
__global__ __launch_bounds__(WM* WN* kWave) void dense_gemm_kernel(GemmArgs p) {
  using T = Tile<BM, BN, WM, WN, BKB>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * T::kStageBytes];
  const int64_t nt = (p.N + BN - 1) / BN;
  const int64_t tm = blockIdx.x / nt, tn = blockIdx.x % nt;
  const int64_t row0 = tm * BM;
  i32x4 acc[T::TM][T::TN];
  T::mainloop(p, smem, acc, row0, p.M, 0, (int)(tn * BN / 16), 0, p.KB);
  T::epilogue(p, acc, row0, p.M, 0, tn * BN);
}

// ---------------------------------------------------------------------------
// grouped kernel: persistent walk over the (expert, m-tile, n-tile) list.
// Every workgroup derives the list itself from group_list (prefix sums of the
// per-expert row counts and m-tile counts, in LDS), so there is no host sync
// and no extra launch. Experts with 0 rows own no tiles.
// ---------------------------------------------------------------------------
template <int BM, int BN, int WM, int WN, int BKB>
__global__ __launch_bounds__(WM* WN* kWave) void grouped_gemm_kernel(GemmArgs p) {
  static_assert(WM * WN * kWave == 256, "schedule scan assumes 256 threads");
  using T = Tile<BM, BN, WM, WN, BKB>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * T::kStageBytes];
  __shared__ int64_t row_off[kMaxExperts + 1];   // first row of each expert
  __shared__ int tile_off[kMaxExperts + 1];      // first m-tile of each expert
  const int E = p.E;
  build_schedule<BM>(p.group_list, E, row_off, tile_off);
  const int64_t nt = (p.N + BN - 1) / BN;
  const int64_t total = (int64_t)tile_off[E] * nt;
  for (int64_t t = blockIdx.x; t < total; t += gridDim.x) {
    const int mt = (int)(t / nt);
    const int64_t tn = t % nt;
    // expert owning m-tile mt: last e with tile_off[e] <= mt (binary search)
    int lo = 0, hi = E - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (tile_off[mid] <= mt) lo = mid; else hi = mid - 1;
    }
    const int e = lo;
    const int64_t row0 = row_off[e] + (int64_t)(mt - tile_off[e]) * BM;
    // counts that sum past R are a caller error; rows at or past R are skipped
    // so that such a list cannot make the kernel touch memory outside [0, R)
    const int64_t row_end = min(row_off[e + 1], p.M);
    if (row0 >= row_end) continue;
    i32x4 acc[T::TM][T::TN];
    T::mainloop(p, smem, acc, row0, row_end, e, (int)(tn * BN / 16), 0, p.KB);
    T::epilogue(p, acc, row0, row_end, e, tn * BN);
  }
}

// ---------------------------------------------------------------------------
// Grouped GEMM, fast path (K % 16 == 0, 16-byte aligned rows).
//
// The row counts are skewed: with top-8 routing over 256 experts most
// non-empty experts own a handful of rows while a few own thousands. The two
// kinds are served by one persistent kernel that reads a schedule:
//   * experts with at most kSmallRows rows: weight streaming; each weight
//     byte is read once and no MFMA tile is padded to 256 rows;
//   * larger experts: 256 x 256 LDS-DMA tiles.
// ---------------------------------------------------------------------------
constexpr int kSmallRows = 64;
constexpr int kGroupBM = 256, kGroupBN = 256;

// Schedule in the workspace (its size is group_sched_bytes in launch.hpp):
// row_off[E + 1] (first row of each expert), tile_off[E + 1] (first m-tile of
// each large expert; small and empty experts own none), small[E + 1] (the ids
// of the non-empty small experts, their count in small[E]) and the kQueues
// work-queue counters of the mixed kernel (one per XCD).
struct GroupSched {
  int64_t* row_off;
  int* tile_off;
  int* small;
  unsigned* queue;
};

__host__ __device__ inline GroupSched group_sched(void* ws, int64_t E) {
  GroupSched g;
  char* b = reinterpret_cast<char*>(ws);
  g.row_off = reinterpret_cast<int64_t*>(b);
  b += sched_align((E + 1) * 8);
  g.tile_off = reinterpret_cast<int*>(b);
  b += sched_align((E + 1) * 4);
  g.small = reinterpret_cast<int*>(b);
  b += sched_align((E + 1) * 4);
  g.queue = reinterpret_cast<unsigned*>(b);
  return g;
}

// One 1024-thread workgroup: each thread owns one expert (E <= 1024); the
// exclusive scans of the row counts and of the large experts' m-tile counts
// run as wavefront shfl_up scans combined through LDS.
__global__ __launch_bounds__(1024) void group_schedule_kernel(const int64_t* __restrict__ gl, int E,
                                                              GroupSched out) {
  __shared__ int64_t wrows[16];
  __shared__ int wtiles[16];
  __shared__ int wsmall[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t n = tid < E ? max(gl[tid], (int64_t)0) : 0;  // a negative count owns no rows
  const int t = n > kSmallRows ? (int)((n + kGroupBM - 1) / kGroupBM) : 0;
  const int sm = (n > 0 && n <= kSmallRows) ? 1 : 0;
  int64_t ri = n;
  int ti = t, si = sm;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int64_t ro = __shfl_up(ri, d, 64);
    const int to = __shfl_up(ti, d, 64);
    const int so = __shfl_up(si, d, 64);
    if (lane >= d) {
      ri += ro;
      ti += to;
      si += so;
    }
  }
  if (lane == 63) {
    wrows[wave] = ri;
    wtiles[wave] = ti;
    wsmall[wave] = si;
  }
  __syncthreads();
  for (int w = 0; w < wave; ++w) {
    ri += wrows[w];
    ti += wtiles[w];
    si += wsmall[w];
  }
  if (tid < E) {
    out.row_off[tid] = ri - n;
    out.tile_off[tid] = ti - t;
    if (sm) out.small[si - 1] = tid;
  }
  if (tid == E - 1) {
    out.row_off[E] = ri;
    out.tile_off[E] = ti;
    out.small[E] = si;
  }
  if (tid < kQueues) out.queue[tid] = 0u;
}

// Small-expert items. An item is the rows of one expert (at most 16 * MB)
// against kSmallNB consecutive n-blocks over the full K; wavefront w owns
// n-blocks nb0 + kSmallNBW * w + j. The expert's A rows go through LDS once
// per workgroup, in chunks of kSmallCK k-blocks stored in MFMA operand order
// (wavefront w stages k-block w of each chunk, all m-blocks) into two
// buffers; the weight blocks go straight from HBM into registers, one chunk
// ahead of the MFMAs, in two register sets used for alternate chunks (no
// operand is ever copied). Registers thus hold weights in flight rather than
// A fragments re-read by every wavefront, which keeps enough weight bytes in
// flight per CU to stream at HBM rate. Step c: load chunk c + 1 (A pieces
// and weights), run the MFMAs of chunk c from buffer c % 2, store the A
// pieces of chunk c + 1 into buffer (c + 1) % 2 (last read by chunk c - 1,
// whose readers all passed the barrier of step c - 1), barrier on LDS. A is
// staged through VGPRs rather than by LDS DMA: the compiler then tracks the
// LDS contents and keeps the next chunk's weight loads in flight across the
// MFMAs instead of draining them.
constexpr int kSmallCK = 8, kSmallNBW = 2;
constexpr int kSmallNB = 8 * kSmallNBW;

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int MB>
struct SmallItem {
  static constexpr int CK = kSmallCK, NBW = kSmallNBW;
  static constexpr int kChunkBytes = MB * CK * kBlockBytes;
  using Regs = i32x4[CK][NBW];

  struct Src {
    const uint8_t* a;     // activation base (wave-uniform)
    const uint8_t* w;     // this expert's packed weight (wave-uniform)
    uint32_t aoff[MB];    // lane's A chunk of k-block 0, per m-block
    uint32_t woff[NBW];   // lane's 16 bytes of k-block 0, per owned n-block
    uint32_t adj;         // pull-back of the lane's A chunk in a ragged last k-block
  };

  // Loads of chunk c: the A pieces of k-block c * CK + wave (clamped to the
  // last one; the MFMAs skip k-blocks past it) and the chunk's weight blocks
  // (clamped the same way). A first: the store of the pieces then waits for
  // them only, not for the weights behind them.
  __device__ __forceinline__ static void load(const GemmArgs& p, const Src& s, i32x4 (&ar)[MB],
                                              Regs& wr, int c, int wave) {
    const int KB = p.KB;
    int kb = c * CK + wave;
    kb = kb < KB ? kb : KB - 1;  // wave-uniform
    const uint32_t pull = kb == KB - 1 ? s.adj : 0u;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      ar[mb] = *reinterpret_cast<const i32x4*>(s.a + (s.aoff[mb] + (uint32_t)kb * 64u - pull));
#pragma unroll
    for (int u = 0; u < CK; ++u) {
      int k = c * CK + u;
      k = k < KB ? k : KB - 1;
#pragma unroll
      for (int j = 0; j < NBW; ++j)
        wr[u][j] = *reinterpret_cast<const i32x4*>(s.w + (s.woff[j] + (uint32_t)k * kBlockBytes));
    }
  }

  template <int BUF>
  __device__ __forceinline__ static void stage(uint8_t* smem, const i32x4 (&ar)[MB], int wave,
                                               int lane) {
    uint8_t* dst = smem + BUF * kChunkBytes + wave * kBlockBytes + lane * 16;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      *reinterpret_cast<i32x4*>(dst + mb * CK * kBlockBytes) = ar[mb];
  }

  // FULL: every k-block of chunk c lies below KB (all chunks but the last)
  template <bool FULL, int BUF>
  __device__ __forceinline__ static void compute(const GemmArgs& p, const uint8_t* smem,
                                                 const Regs& wr, i32x4 (&acc)[MB][NBW], int c,
                                                 int lane) {
    const uint8_t* buf = smem + BUF * kChunkBytes + lane * 16;
#pragma unroll
    for (int u = 0; u < CK; ++u) {
      if (FULL || c * CK + u < p.KB) {  // wave-uniform: clamped duplicate k-blocks add nothing
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const i32x4 a = *reinterpret_cast<const i32x4*>(buf + (mb * CK + u) * kBlockBytes);
#pragma unroll
          for (int j = 0; j < NBW; ++j) acc[mb][j] = mfma16x16x64(a, wr[u][j], acc[mb][j]);
        }
      }
    }
  }

  __device__ __forceinline__ static void run(const GemmArgs& p, uint8_t* smem, int e, int64_t row0,
                                             int64_t rows, int nb0) {
    const int tid = opaque_tid();
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int KB = p.KB;
    Src s;
    s.a = reinterpret_cast<const uint8_t*>(p.a);
    s.w = p.w + (int64_t)e * p.NB * KB * kBlockBytes;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      // rows past the expert's last read that last row: they only feed
      // output rows that are never stored
      int64_t r = mb * 16 + (lane & 15);
      r = r < rows ? r : rows - 1;
      s.aoff[mb] = (uint32_t)((row0 + r) * p.lda + (lane >> 4) * 16);
    }
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
      int nb = nb0 + wave * NBW + j;
      nb = nb < p.NB ? nb : p.NB - 1;  // past the last n-block: never stored
      s.woff[j] = (uint32_t)((int64_t)nb * KB * kBlockBytes + lane * 16);
    }
    // last k-block of a ragged K: a 16-byte A chunk that would run past the
    // row end is read from K - 16 instead (its values meet zero weights)
    const int64_t col = (int64_t)(KB - 1) * 64 + (lane >> 4) * 16;
    s.adj = col > p.K - 16 ? (uint32_t)(col - (p.K - 16)) : 0u;

    i32x4 acc[MB][NBW];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < NBW; ++j) acc[mb][j] = i32x4{0, 0, 0, 0};
    // chunk c lives in buffer c % 2 and register set c % 2 (c starts even)
    const int nchunk = (KB + CK - 1) / CK;
    i32x4 ar[MB];
    Regs wa, wb;
    load(p, s, ar, wa, 0, wave);
    stage<0>(smem, ar, wave, lane);
    lds_barrier();
    int c = 0;
    for (; c + 2 < nchunk; c += 2) {
      load(p, s, ar, wb, c + 1, wave);
      compute<true, 0>(p, smem, wa, acc, c, lane);
      stage<1>(smem, ar, wave, lane);
      lds_barrier();
      load(p, s, ar, wa, c + 2, wave);
      compute<true, 1>(p, smem, wb, acc, c + 1, lane);
      stage<0>(smem, ar, wave, lane);
      lds_barrier();
    }
    if (c + 1 < nchunk) {
      load(p, s, ar, wb, c + 1, wave);
      compute<true, 0>(p, smem, wa, acc, c, lane);
      stage<1>(smem, ar, wave, lane);
      lds_barrier();
      compute<false, 1>(p, smem, wb, acc, c + 1, lane);
    } else {
      compute<false, 0>(p, smem, wa, acc, c, lane);
    }

#pragma unroll
    for (int j = 0; j < NBW; ++j) {
      const int64_t n = (int64_t)(nb0 + wave * NBW + j) * 16 + (lane & 15);
      if (n >= p.N) continue;
      const float ws = p.w_scale[(int64_t)e * p.N + n];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int64_t m = mb * 16 + (lane >> 4) * 4 + t;
          if (m >= rows) continue;
          const int64_t row = row0 + m;
          if (p.out == kOutI32) {
            reinterpret_cast<int32_t*>(p.y)[row * p.ldy + n] = acc[mb][j][t];
          } else {
            float f = (float)acc[mb][j][t];
            f = f * p.a_scale[row];
            f = f * ws;
            reinterpret_cast<uint16_t*>(p.y)[row * p.ldy + n] = (uint16_t)f32_to_bf16(f);
          }
        }
      }
    }
  }
};

// Small-expert item g of expert e: n-blocks [g * kSmallNB, (g + 1) * kSmallNB).
// Every wavefront of the workgroup takes part (the A DMA and the barriers are
// shared), also one whose n-blocks lie past the last.
__device__ __forceinline__ void small_item(const GemmArgs& p, const GroupSched& sc, uint8_t* smem,
                                           int e, int g) {
  const int64_t row0 = sc.row_off[e];
  // counts that sum past R are a caller error: rows at or past R are never
  // touched
  const int64_t rows = min(sc.row_off[e + 1], p.M) - row0;
  if (rows <= 0) return;  // uniform
  const int nb0 = g * kSmallNB;
  if (rows <= 16) SmallItem<1>::run(p, smem, e, row0, rows, nb0);
  else if (rows <= 32) SmallItem<2>::run(p, smem, e, row0, rows, nb0);
  else SmallItem<4>::run(p, smem, e, row0, rows, nb0);
}

// Grouped GEMM over both kinds of expert in one persistent launch (one
// workgroup per CU). Work items: the 256x256 tiles of the large experts
// (MFMA-bound, ordered expert, n-tile, m-tile) and the kSmallNB-n-block
// groups of the small experts (weight streaming, HBM-bound), merged in proportion
// (item i is a tile when floor((i + 1) T / I) > floor(i T / I)) so that at
// any time some CUs compute while others stream. XCD x (workgroups b with
// b % 8 == x) works through its own contiguous eighth of the item list,
// taking items from its queue counter (zeroed by the schedule kernel); every
// workgroup leaves when its XCD's range is exhausted.
template <int STAGES, int WM, int WN>
__global__ __launch_bounds__(WM* WN* kWave) void grouped_mixed_kernel(GemmArgs p, GroupSched sc) {
  using T = DmaTile<kGroupBM, kGroupBN, STAGES, WM, WN>;
  static_assert(WM * WN == kSmallCK, "one wavefront per k-block of a small-item chunk");
  static_assert(2 * SmallItem<4>::kChunkBytes <= T::kLdsBytes, "small items fit the ring");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[T::kLdsBytes];
  // the item index is passed through the first bytes of the ring, which is
  // idle between items (a second barrier keeps the next DMA off it until
  // every wavefront has read it)
  int64_t* item_slot = reinterpret_cast<int64_t*>(smem);
  const int E = p.E;
  const int64_t NT = (p.N + kGroupBN - 1) / kGroupBN;
  const int64_t groups = (p.NB + kSmallNB - 1) / kSmallNB;
  const int64_t n_tile = (int64_t)sc.tile_off[E] * NT;
  const int64_t n_small = (int64_t)sc.small[E] * groups;
  const int64_t total = n_tile + n_small;
  const int64_t per = (total + kQueues - 1) / kQueues;
  const int xcd = blockIdx.x % kQueues;
  const int64_t first = xcd * per, end = min(first + per, total);
  for (;;) {
    if (threadIdx.x == 0) *item_slot = first + (int64_t)atomicAdd(&sc.queue[xcd], 1u);
    __syncthreads();
    const int64_t i = *item_slot;
    __syncthreads();
    if (i >= end) break;  // uniform: every wavefront leaves together
    const int64_t tiles_before = total ? i * n_tile / total : 0;
    const bool is_tile = (i + 1) * n_tile / total > tiles_before;
    if (is_tile) {
      const int64_t t = tiles_before;
      // expert owning tile t: last e with tile_off[e] * NT <= t
      int lo = 0, hi = E - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if ((int64_t)sc.tile_off[mid] * NT <= t) lo = mid; else hi = mid - 1;
      }
      const int e = lo;
      const int64_t mtiles = sc.tile_off[e + 1] - sc.tile_off[e];
      const int64_t local = t - (int64_t)sc.tile_off[e] * NT;
      const int64_t tn = local / mtiles, mt = local % mtiles;
      const int64_t row0 = sc.row_off[e] + mt * kGroupBM;
      const int64_t row_end = min(sc.row_off[e + 1], p.M);
      if (row0 < row_end) {
        i32x4 acc[T::TM][T::TN];
        T::mainloop(p, smem, acc, row0, row_end, e, (int)(tn * kGroupBN / 16));
        if (p.out == kOutI32) T::epilogue(p, acc, row0, row_end, e, tn * kGroupBN);
        else T::epilogue_staged(p, acc, smem, row0, row_end, e, tn * kGroupBN);
      }
    } else {
      const int64_t si = i - tiles_before;
      small_item(p, sc, smem, sc.small[si / groups], (int)(si % groups));
    }
    __syncthreads();  // the item's last LDS use done before the slot is rewritten
  }
}

// ---------------------------------------------------------------------------
// decode kernel (M <= 64): weight-streaming GEMV-like path.
// One workgroup owns one 16-column n-block over the full K; its WAVES
// wavefronts take interleaved k-blocks (wave w: w, w + WAVES, ...) so that the
// workgroup streams contiguous 1 KB weight blocks. Weights go straight from
// HBM into MFMA operand registers (the packed layout is the operand layout),
// UNR blocks per wave in flight at once; the MB m-blocks of A (<= 64 rows,
// shared by all workgroups and served from L2) are loaded the same way. The
// per-wave INT32 partial sums are added in LDS and the epilogue runs on the
// full sums: one kernel, no workspace, no second pass. Grid = ceil(N / 16 /
// NBW) x ceil(M / (16 MB)): blockIdx.y selects the workgroup's 16 MB rows.
// ---------------------------------------------------------------------------
template <int MB, int NBW, int WAVES, int UNR, bool AVEC, bool ABLK = false, bool PF = false>
__global__ __launch_bounds__(WAVES* kWave) void decode_gemm_kernel(GemmArgs p) {
  static_assert(MB * NBW <= WAVES, "one wavefront per output block in the epilogue");
  __shared__ i32x4 red[WAVES][MB * NBW][kWave];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nb0 = blockIdx.x * NBW;
  const int64_t mrow0 = (int64_t)blockIdx.y * MB * 16;  // this workgroup's first row
  const uint8_t* wcol[NBW];
#pragma unroll
  for (int j = 0; j < NBW; ++j) {
    // n-blocks past the last one read the last (their outputs are not stored)
    const int nb = nb0 + j < p.NB ? nb0 + j : p.NB - 1;
    wcol[j] = p.w + (int64_t)nb * p.KB * kBlockBytes + lane * 16;
  }
  const int64_t mlast = p.M - 1;
  // 16-byte A rows (AVEC): this lane's chunk of k-block 0 per m-block, and
  // its pull-back in a ragged last k-block (a chunk that would run past the
  // row end is read from K - 16; its values meet zero weights)
  const int8_t* arow[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int64_t row = mrow0 + mb * 16 + (lane & 15);
    arow[mb] = p.a + (row < p.M ? row : mlast) * p.lda + (lane >> 4) * 16;
  }
  const int64_t col_last = (int64_t)(p.KB - 1) * 64 + (lane >> 4) * 16;
  const int64_t pull = col_last > p.K - 16 ? col_last - (p.K - 16) : 0;
  i32x4 acc[MB][NBW];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int j = 0; j < NBW; ++j) acc[mb][j] = i32x4{0, 0, 0, 0};
  // PF: the weights of the next round are loaded before this round's MFMAs
  // (after its activation loads), so that their HBM latency overlaps them
  i32x4 bn[PF ? UNR : 1][NBW];
  if (PF) {
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int kb = wave + u * WAVES;
      const int kbc = kb < p.KB ? kb : p.KB - 1;
#pragma unroll
      for (int j = 0; j < NBW; ++j)
        bn[u][j] = *reinterpret_cast<const i32x4*>(wcol[j] + (int64_t)kbc * kBlockBytes);
    }
  }
  for (int kb0 = wave; kb0 < p.KB; kb0 += WAVES * UNR) {
    i32x4 b[UNR][NBW];
    i32x4 a[UNR][MB];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int kb = kb0 + u * WAVES;
      const int kbc = kb < p.KB ? kb : p.KB - 1;    // clamped: loads stay in bounds
#pragma unroll
      for (int j = 0; j < NBW; ++j)
        b[u][j] = PF ? bn[u][j] : *reinterpret_cast<const i32x4*>(wcol[j] + (int64_t)kbc * kBlockBytes);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int64_t row = mrow0 + mb * 16 + (lane & 15);
        const int64_t kcol = (int64_t)kbc * 64 + (lane >> 4) * 16;
        if (ABLK) {
          // packed A: one contiguous 1 KB block per (m-block, k-block); m-blocks
          // past the last one are read clamped (their rows are never stored)
          const int64_t mbg = mrow0 / 16 + mb;
          const int64_t mbc = mbg <= mlast / 16 ? mbg : mlast / 16;
          a[u][mb] = *reinterpret_cast<const i32x4*>(p.a + (mbc * p.KB + kbc) * kBlockBytes +
                                                     lane * 16);
        } else if (AVEC) {
          // lanes of rows past M load nothing: their products only feed
          // output rows >= M, which are never stored
          const int8_t* src = arow[mb] + (int64_t)kbc * 64 - (kbc == p.KB - 1 ? pull : 0);
          a[u][mb] = row < p.M ? *reinterpret_cast<const i32x4*>(src) : i32x4{0, 0, 0, 0};
        } else {
          a[u][mb] = load_a16(p, row, p.M, kcol);
        }
      }
    }
    if (PF && kb0 + WAVES * UNR < p.KB) {  // wave-uniform
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int kb = kb0 + WAVES * UNR + u * WAVES;
        const int kbc = kb < p.KB ? kb : p.KB - 1;
#pragma unroll
        for (int j = 0; j < NBW; ++j)
          bn[u][j] = *reinterpret_cast<const i32x4*>(wcol[j] + (int64_t)kbc * kBlockBytes);
      }
    }
    // keep every load of this round ahead of the first MFMA: without the
    // barrier the scheduler interleaves load / wait / MFMA and only a couple of
    // blocks are in flight per wavefront
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      if (kb0 + u * WAVES >= p.KB) break;  // wave-uniform: clamped duplicate blocks add nothing
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int j = 0; j < NBW; ++j) acc[mb][j] = mfma16x16x64(a[u][mb], b[u][j], acc[mb][j]);
    }
  }
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int j = 0; j < NBW; ++j) red[wave][mb * NBW + j][lane] = acc[mb][j];
  __syncthreads();
  if (wave >= MB * NBW) return;
  // wavefront w finishes output block (m-block w / NBW, n-block w % NBW)
  i32x4 sum = red[0][wave][lane];
#pragma unroll
  for (int w = 1; w < WAVES; ++w) sum += red[w][wave][lane];
  const int mbk = wave / NBW, jn = wave % NBW;
  const int64_t n = (int64_t)(nb0 + jn) * 16 + (lane & 15);
  if (n >= p.N) return;
  const float ws = p.w_scale[n];
  const float bsv = p.bias ? bf16_to_f32(p.bias[n]) : 0.0f;
  const int32_t qb = p.qbias ? p.qbias[n] : 0;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int64_t m = mrow0 + mbk * 16 + (lane >> 4) * 4 + t;
    if (m >= p.M) continue;
    if (p.out == kOutI32) {
      reinterpret_cast<int32_t*>(p.y)[m * p.ldy + n] = sum[t];
    } else {
      const float f = out_value(p, sum[t], p.a_scale ? p.a_scale[m] : 0.0f, ws, bsv, qb);
      reinterpret_cast<uint16_t*>(p.y)[m * p.ldy + n] = (uint16_t)f32_to_bf16(f);
    }
  }
}

// ---------------------------------------------------------------------------
// Dynamic quant fused into the decode GEMM, for a few values (M * K <=
// kFusedElems): every workgroup quantizes the M BF16 rows itself (they are
// L2-resident after the first reads) into LDS — row amax over the workgroup,
// one IEEE division for the scale and one per element, exactly as the
// standalone quant — and then runs the decode K loop with the A fragments
// from LDS (rows >= M read as zero). Saves the quant launch; the results are
// bit-identical to quant + linear. ROWS <= 4: each thread holds CPT 8-value
// chunks of every row (K <= CPT * 8 * threads), amax by wavefront reductions.
// More rows: the M x ceil(K/64)*64 codes are numbered flat and each thread
// takes up to kFlat chunks of them, wherever the row boundaries fall; the row
// amax is an LDS atomic max over the chunks' amaxes. Dynamic LDS:
// M * ceil(K/64) * 64 code bytes.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t bf16_pair_absmax(uint32_t w) {
  return max(w & 0x7FFFu, (w >> 16) & 0x7FFFu);
}

template <int UNR, int WAVES, int ROWS, int CPT>
__global__ __launch_bounds__(WAVES * kWave) void decode_fused_kernel(GemmArgs p) {
  constexpr int kThreadsF = WAVES * kWave;
  constexpr int kRows = ROWS, kCpt = CPT;
  constexpr bool kFlatRows = ROWS > 4;
  constexpr int kFlat = 3;  // chunks per thread, flat numbering (M * Kp / 8 <= kFlat * threads)
  __shared__ i32x4 red[WAVES][kWave];
  __shared__ uint32_t wmax[kFlatRows ? 1 : WAVES][kRows];
  __shared__ uint32_t ramax[kRows];
  __shared__ float srow[kRows];
  extern __shared__ __attribute__((aligned(16))) int8_t qlds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint16_t* x = reinterpret_cast<const uint16_t*>(p.a);
  const int64_t K = p.K, Kp = (int64_t)p.KB * 64;
  const int M = (int)p.M;
  const int nchunk = (int)(K / 8), nchunk_p = (int)(Kp / 8);
  // The activation rows are loaded first and the first round of weights right
  // after: the wait for the activations (loads retire in issue order) then
  // leaves every weight load in flight while the rows are quantized.
  uint4 v[kFlatRows ? 1 : kRows][kCpt];
  uint4 vf[kFlatRows ? kFlat : 1];
  if constexpr (kFlatRows) {
    if (tid < kRows) ramax[tid] = 0u;
#pragma unroll
    for (int i = 0; i < kFlat; ++i) {
      const int f = tid + i * kThreadsF, r = f / nchunk_p, c = f % nchunk_p;
      vf[i] = (r < M && c < nchunk) ? reinterpret_cast<const uint4*>(x + (int64_t)r * K)[c]
                                    : uint4{0u, 0u, 0u, 0u};
    }
  } else {
#pragma unroll
    for (int r = 0; r < kRows; ++r)
#pragma unroll
      for (int i = 0; i < kCpt; ++i) {
        const int c = tid + i * kThreadsF;
        v[r][i] = (r < M && c < nchunk) ? reinterpret_cast<const uint4*>(x + (int64_t)r * K)[c]
                                        : uint4{0u, 0u, 0u, 0u};
      }
  }
  __builtin_amdgcn_sched_barrier(0);
  const int nb = blockIdx.x;
  const uint8_t* wcol = p.w + (int64_t)nb * p.KB * kBlockBytes + lane * 16;
  i32x4 b[UNR];
#pragma unroll
  for (int u = 0; u < UNR; ++u) {
    const int kb = wave + u * WAVES;
    const int kbc = kb < p.KB ? kb : p.KB - 1;    // clamped: loads stay in bounds
    b[u] = *reinterpret_cast<const i32x4*>(wcol + (int64_t)kbc * kBlockBytes);
  }
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (kFlatRows) {
    // amax: LDS atomic max of every chunk's |BF16| bit patterns into its row
    __syncthreads();  // ramax zeroed
#pragma unroll
    for (int i = 0; i < kFlat; ++i) {
      const int f = tid + i * kThreadsF, r = f / nchunk_p;
      if (r < M)
        atomicMax(&ramax[r], max(max(bf16_pair_absmax(vf[i].x), bf16_pair_absmax(vf[i].y)),
                                 max(bf16_pair_absmax(vf[i].z), bf16_pair_absmax(vf[i].w))));
    }
    __syncthreads();
    if (tid < M) srow[tid] = bf16_to_f32(ramax[tid]) / 127.0f;
#pragma unroll
    for (int i = 0; i < kFlat; ++i) {
      const int f = tid + i * kThreadsF, r = f / nchunk_p, c = f % nchunk_p;
      if (r >= M) break;
      uint2 o = uint2{0u, 0u};  // past K: zero codes
      if (c < nchunk) {
        const uint32_t w4[4] = {vf[i].x, vf[i].y, vf[i].z, vf[i].w};
        o = quant8_bf16(w4, bf16_to_f32(ramax[r]) / 127.0f);
      }
      *reinterpret_cast<uint2*>(qlds + r * Kp + (int64_t)c * 8) = o;
    }
  } else {
  // quant of the M rows: one barrier for the amax, one for the codes
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    uint32_t am = 0;
#pragma unroll
    for (int i = 0; i < kCpt; ++i)
      am = max(am, max(max(bf16_pair_absmax(v[r][i].x), bf16_pair_absmax(v[r][i].y)),
                       max(bf16_pair_absmax(v[r][i].z), bf16_pair_absmax(v[r][i].w))));
    am = wave_max_u32(am);
    if (lane == 0) wmax[wave][r] = am;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    if (r >= M) break;
    uint32_t amax = wmax[0][r];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) amax = max(amax, wmax[w][r]);
    const float sc = bf16_to_f32(amax) / 127.0f;
    if (tid == 0) srow[r] = sc;
#pragma unroll
    for (int i = 0; i < kCpt; ++i) {
      const int c = tid + i * kThreadsF;
      if (c >= nchunk_p) break;
      uint2 o = uint2{0u, 0u};
      if (c < nchunk) {
        const uint32_t w4[4] = {v[r][i].x, v[r][i].y, v[r][i].z, v[r][i].w};
        o = quant8_bf16(w4, sc);
      }
      *reinterpret_cast<uint2*>(qlds + r * Kp + (int64_t)c * 8) = o;
    }
  }
  }
  __syncthreads();
  const int arow = lane & 15;
  i32x4 acc = i32x4{0, 0, 0, 0};
  for (int kb0 = wave; kb0 < p.KB; kb0 += WAVES * UNR) {
    if (kb0 != wave) {
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int kb = kb0 + u * WAVES;
        const int kbc = kb < p.KB ? kb : p.KB - 1;
        b[u] = *reinterpret_cast<const i32x4*>(wcol + (int64_t)kbc * kBlockBytes);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int kb = kb0 + u * WAVES;
      if (kb >= p.KB) break;  // wave-uniform
      const i32x4 a = arow < M ? *reinterpret_cast<const i32x4*>(qlds + arow * Kp + kb * 64 +
                                                                  (lane >> 4) * 16)
                               : i32x4{0, 0, 0, 0};
      acc = mfma16x16x64(a, b[u], acc);
    }
  }
  red[wave][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  i32x4 sum = red[0][lane];
#pragma unroll
  for (int w = 1; w < WAVES; ++w) sum += red[w][lane];
  const int64_t n = (int64_t)nb * 16 + (lane & 15);
  if (n >= p.N) return;
  const float ws = p.w_scale[n];
  const float bsv = p.bias ? bf16_to_f32(p.bias[n]) : 0.0f;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int m = (lane >> 4) * 4 + t;
    if (m >= M) continue;
    if (p.out == kOutI32) {
      reinterpret_cast<int32_t*>(p.y)[m * p.ldy + n] = sum[t];
    } else {
      float f = (float)sum[t];
      f = f * srow[m];
      f = f * ws;
      if (p.bias) f = f + bsv;
      reinterpret_cast<uint16_t*>(p.y)[m * p.ldy + n] = (uint16_t)f32_to_bf16(f);
    }
  }
}

// ---------------------------------------------------------------------------
// host side: variants and plans
// ---------------------------------------------------------------------------
namespace {

struct DenseVariant {
  int BM, BN;
  void (*fn)(GemmArgs);
  int threads;
  bool decode;   // grid = n-blocks / nbw, one workgroup per nbw 16-column blocks
  int nbw;
  int mrows;     // decode: rows per workgroup (grid.y = ceil(M / mrows))
};

constexpr int kDecodeWaves = 8;

// 0: M > 64 fallback (K % 16 != 0 or unaligned A): 128x128 tiles, VGPR-staged
// 1..3: M <= 16 / 32 / 64: decode kernel with 1 / 2 m-blocks of one n-block;
// M <= 64 as two row groups of 32 (grid.y) with 2 m-blocks x 2 n-blocks per
// workgroup: a workgroup reads half the activation rows for twice the
// columns (458 instead of 573 KB per workgroup at K = 7168), and the weights
// of a column pair twice, by two workgroups on the same XCD
// 4..6: the same for K % 16 != 0 or an unaligned activation pointer
const DenseVariant kDense[] = {
    {128, 128, dense_gemm_kernel<128, 128, 2, 2, 2>, 256, false, 1, 0},
    {16, 16, decode_gemm_kernel<1, 1, kDecodeWaves, 14, true>, kDecodeWaves * 64, true, 1, 16},
    {32, 16, decode_gemm_kernel<2, 1, kDecodeWaves, 14, true>, kDecodeWaves * 64, true, 1, 32},
    {64, 16, decode_gemm_kernel<2, 2, kDecodeWaves, 7, true, false, true>, kDecodeWaves * 64, true, 2, 32},
    {16, 16, decode_gemm_kernel<1, 1, kDecodeWaves, 14, false>, kDecodeWaves * 64, true, 1, 16},
    {32, 16, decode_gemm_kernel<2, 1, kDecodeWaves, 14, false>, kDecodeWaves * 64, true, 1, 32},
    {64, 16, decode_gemm_kernel<2, 2, kDecodeWaves, 7, false, false, true>, kDecodeWaves * 64, true, 2, 32},
    // 7..9: M <= 16 / 32 / 64 with packed A (1 KB blocks)
    {16, 16, decode_gemm_kernel<1, 1, kDecodeWaves, 14, true, true>, kDecodeWaves * 64, true, 1, 16},
    {32, 16, decode_gemm_kernel<2, 1, kDecodeWaves, 14, true, true>, kDecodeWaves * 64, true, 1, 32},
    {64, 16, decode_gemm_kernel<2, 2, kDecodeWaves, 7, true, true, true>, kDecodeWaves * 64, true, 2, 32},
};

}  // namespace

DensePlan plan_dense(int64_t M, int64_t N, int64_t K) {
  (void)N;
  DensePlan pl{};
  if (M > 64) {
    pl.variant = 0;
  } else {
    pl.variant = M <= 16 ? 1 : (M <= 32 ? 2 : 3);
    if (K % 16 != 0) pl.variant += 3;
  }
  pl.ws_bytes = 0;
  return pl;
}

static GemmArgs make_args(const int8_t* a, const float* a_scale, int64_t M, int64_t K,
                          const void* w_packed, const float* w_scale, int64_t N,
                          const uint16_t* bias, void* y, int out) {
  GemmArgs p{};
  p.a = a;
  p.a_scale = a_scale;
  p.M = M;
  p.K = K;
  p.KB = (int)ceil_div(K, 64);
  p.w = reinterpret_cast<const uint8_t*>(w_packed);
  p.NB = (int)ceil_div(N, 16);
  p.w_scale = w_scale;
  p.N = N;
  p.bias = bias;
  p.y = y;
  p.out = out;
  p.a_vec = (K % 16 == 0) && (((uintptr_t)a & 15) == 0);
  p.lda = K;
  p.ldy = N;
  return p;
}

// The LDS-DMA tile kernels address A and one expert's packed weight with
// 32-bit per-lane byte offsets.
static bool offsets32_ok(const GemmArgs& p) {
  const int64_t lim = (int64_t)1 << 32;
  return p.M * p.lda + 64 < lim && (int64_t)p.NB * p.KB * kBlockBytes < lim;
}

hipError_t launch_dense_gemm(const DensePlan& plan, const int8_t* q, const float* x_scale, int64_t M,
                             int64_t K, const void* w_packed, const float* w_scale, int64_t N,
                             const uint16_t* bias, void* y, int out, bool a_packed, void* ws,
                             hipStream_t stream, const int32_t* qbias, int64_t lda, int64_t ldy) {
  (void)ws;
  if (M == 0 || N == 0) return hipSuccess;
  GemmArgs p = make_args(q, x_scale, M, K, w_packed, w_scale, N, bias, y, out);
  p.qbias = qbias;
  if (lda) p.lda = lda;
  if (ldy) p.ldy = ldy;
  // 16-byte row loads of A need every row aligned
  p.a_vec = p.a_vec && (p.lda % 16 == 0);
  int variant = plan.variant;
  if (a_packed) {
    // packed A (1 KB blocks): the decode kernels' block variants, or the tiles
    p.a_blk = 1;
    p.a_vec = true;
    if (variant != 0) {
      const DenseVariant& v = kDense[6 + (M <= 16 ? 1 : (M <= 32 ? 2 : 3))];
      hipLaunchKernelGGL(v.fn, dim3((unsigned)ceil_div(ceil_div(N, 16), v.nbw), (unsigned)ceil_div(M, v.mrows)),
                         dim3(v.threads), 0, stream, p);
      return hipGetLastError();
    }
    if (!offsets32_ok(p)) return hipErrorInvalidValue;
    constexpr int BM = 256, BN = 256;
    const int64_t grid = round_up(ceil_div(M, BM) * ceil_div(N, BN), 8);
    hipLaunchKernelGGL(
        (dense_dma_kernel<BM, BN, W8A8_DMA_STAGES, W8A8_DMA_GROUP_M, W8A8_DMA_WM, W8A8_DMA_WN>),
        dim3((unsigned)grid), dim3(64 * W8A8_DMA_WM * W8A8_DMA_WN), 0, stream, p);
    return hipGetLastError();
  }
  // the decode kernels load A rows with 16-byte loads when the pointer allows it
  if (kDense[variant].decode && variant <= 3 && !p.a_vec) variant += 3;
  if (variant == 0 && p.a_vec && offsets32_ok(p)) {
    // prefill-sized M: 256x256 tiles through the LDS-DMA ring
    constexpr int BM = 256, BN = 256;
    const int64_t tiles = ceil_div(M, BM) * ceil_div(N, BN);
    const int64_t grid = round_up(tiles, 8);
    hipLaunchKernelGGL(
        (dense_dma_kernel<BM, BN, W8A8_DMA_STAGES, W8A8_DMA_GROUP_M, W8A8_DMA_WM, W8A8_DMA_WN>),
        dim3((unsigned)grid), dim3(64 * W8A8_DMA_WM * W8A8_DMA_WN), 0, stream, p);
    return hipGetLastError();
  }
  const DenseVariant& v = kDense[variant];
  const int64_t tiles = v.decode ? ceil_div(ceil_div(N, 16), v.nbw) : ceil_div(M, v.BM) * ceil_div(N, v.BN);
  const int64_t gy = v.decode ? ceil_div(M, v.mrows) : 1;
  hipLaunchKernelGGL(v.fn, dim3((unsigned)tiles, (unsigned)gy), dim3(v.threads), 0, stream, p);
  return hipGetLastError();
}

bool decode_fused_ok(int64_t M, int64_t K, const void* x) {
  // every workgroup quantizes the M x K values again: past kFusedElems (four
  // rows of K = 7168 measured slower than the separate quant launch) the
  // saved launch does not pay for it, except for 1 or 2 rows (K <= 16384: two
  // 8-value chunks per thread and row). 3 to 16 rows take the flat numbering
  // (3 chunks per thread: M * Kp / 8 <= 3072 for M * K <= 16384, M <= 16)
  return M >= 1 && (M <= 2 || (M <= 16 && M * K <= kFusedElems)) && K % 8 == 0 && K <= 16384 &&
         ((uintptr_t)x & 15) == 0 && M * round_up(K, 64) <= kFusedLdsBytes;
}

hipError_t launch_decode_fused(const uint16_t* x, int64_t M, int64_t K, const void* w_packed,
                               const float* w_scale, int64_t N, const uint16_t* bias, void* y, int out,
                               hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  if (!decode_fused_ok(M, K, x)) return hipErrorInvalidValue;
  GemmArgs p = make_args(reinterpret_cast<const int8_t*>(x), nullptr, M, K, w_packed, w_scale, N, bias,
                         y, out);
  const size_t lds = (size_t)(M * round_up(K, 64));
  if (M <= 2)
    hipLaunchKernelGGL((decode_fused_kernel<7, 16, 2, 2>), dim3((unsigned)ceil_div(N, 16)), dim3(16 * 64), lds,
                       stream, p);
  else
    hipLaunchKernelGGL((decode_fused_kernel<7, 16, 16, 1>), dim3((unsigned)ceil_div(N, 16)), dim3(16 * 64), lds,
                       stream, p);  // CPT unused: flat chunks
  return hipGetLastError();
}

int64_t grouped_ws_bytes(int64_t, int64_t E, int64_t, int64_t) { return group_sched_bytes(E); }

hipError_t launch_grouped_gemm(const int8_t* a, const float* a_scale, const int64_t* group_list,
                               int64_t R, int64_t E, int64_t N, int64_t K, const void* w_packed,
                               const float* w_scale, void* y, int out, void* ws,
                               hipStream_t stream) {
  if (R == 0 || N == 0) return hipSuccess;
  GemmArgs p = make_args(a, a_scale, R, K, w_packed, w_scale, N, nullptr, y, out);
  p.group_list = group_list;
  p.E = (int)E;
  if (!p.a_vec || !offsets32_ok(p)) {
    // K % 16 != 0, unaligned rows or operands past 4 GB: VGPR-staged tiles,
    // schedule built in LDS
    constexpr int BM = 128, BN = 128;
    // upper bound on tiles: sum_e ceil(n_e / BM) <= R / BM + E
    const int64_t max_tiles = (ceil_div(R, BM) + E) * ceil_div(N, BN);
    const int64_t grid = std::min<int64_t>(max_tiles, 256 * 4);
    hipLaunchKernelGGL((grouped_gemm_kernel<BM, BN, 2, 2, 2>), dim3((unsigned)grid), dim3(256), 0,
                       stream, p);
    return hipGetLastError();
  }
  const GroupSched sc = group_sched(ws, E);
  hipLaunchKernelGGL(group_schedule_kernel, dim3(1), dim3(1024), 0, stream, group_list, (int)E, sc);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((grouped_mixed_kernel<W8A8_DMA_STAGES, W8A8_DMA_WM, W8A8_DMA_WN>), dim3(256),
                     dim3(64 * W8A8_DMA_WM * W8A8_DMA_WN), 0, stream, p, sc);
  return hipGetLastError();
}

}  // namespace w8a8
