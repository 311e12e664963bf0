// gemm_tile.h -- gfx950 (CDNA4) MFMA GEMM with an alpha/beta epilogue: the per-step GEMM of
// the TP schedules (the dense GEMM that the Distributed GEMM pull-request
// page runs at every step, written here for MI355X).
//
// Tiling.  A workgroup of 256 threads (4 wave64s, one per SIMD) owns a
// 256 x 256 tile of D; the waves form a 2 x 2 grid and each holds a
// 128 x 128 fp32 accumulator in 256 AGPRs.  K is walked in slabs of 64
// bytes per operand row (32 bf16, 64 e4m3 or 16 fp32 values), so one LDS
// geometry serves every input type and only the MFMA differs:
//   bf16 : v_mfma_f32_16x16x32_bf16         (8 x 8 blocks of 16 x 16)
//   fp32 : v_mfma_f32_16x16x4_f32           (8 x 8 blocks of 16 x 16)
//   e4m3 : v_mfma_scale_f32_32x32x64_f8f6f4 (4 x 4 blocks of 32 x 32,
//          neutral E8M0 block scales; per-tensor scales go to the epilogue)
//
// Data movement.  Both operands are K-contiguous ("TN"), so a lane's MFMA
// fragment is 16 contiguous bytes of one row (ds_read_b128).  K is walked in
// slabs of 128 bytes per row (one cache line), moved from global memory
// straight into LDS with buffer_load_dwordx4 ... lds: each wave instruction
// fills 1 KiB of LDS (lane l -> bytes 16l..16l+15), eight whole rows, so the
// L1 asks L2 for full 128-byte lines (64-byte requests halve the bytes per
// outstanding request and measured about half the L2 -> LDS rate).  Within a
// 64-byte half row the four 16-byte chunks of row r are stored XOR-permuted
// by f(r) = ((r>>1) ^ (r>>2)) & 3, which puts the 16 rows that 16 lanes read
// in one LDS cycle on distinct banks (zero bank conflicts measured).  The
// buffer descriptor of each operand covers only the tile's valid rows, so
// rows past M or N load as zeros (out-of-range lanes of an LDS load write
// zeros), and chunks past K are pushed out of range by the offset's top bit.
//
// Pipeline.  Two LDS stages of 64 KiB (A and B slabs).  MFMAs walk half
// slabs; fragments of the next half slab are read while the current one is
// multiplied.  At the end of each slab one barrier certifies that every
// wave holds the slab in registers and that the next slab has landed; the
// slab after next is then loaded into the stage just vacated, so loads run
// one slab (about 2000 MFMA cycles) ahead.
//
// Workgroup -> tile mapping is XCD-aware: MI355X places workgroup b on XCD
// b mod 8, so each XCD gets one contiguous range of the tile order, and
// that order walks groups of 8 tile rows column by column, so the tiles an
// XCD runs together share A rows and B columns in its own L2.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_launch.h"

namespace dg {
namespace tile {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) int i32x4;

constexpr int kThreads = 256;
constexpr int kSlab = 128;                        // bytes of K per operand row per stage
constexpr int kHalf = 64;                         // fragment reads walk half slabs
constexpr int kOperandStage = kBM * kSlab;        // 32 KiB
constexpr int kStageBytes = 2 * kOperandStage;    // A + B = 64 KiB
constexpr int kStages = 2;
constexpr int kLoadsPerOperand = kOperandStage / 1024 / 4;  // per wave: 8
constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int kGroupM = 8;
constexpr int kNumXcd = 8;

static_assert(kBM == 256 && kBN == 256, "tile geometry");

template <int IN>
constexpr int elem_size() {
  return IN == IN_F32 ? 4 : (IN == IN_BF16 ? 2 : 1);
}

__device__ __forceinline__ int chunk_perm(int row) { return ((row >> 1) ^ (row >> 2)) & 3; }

// Buffer descriptor of a wave-uniform base and size.  The values are
// uniform by construction (they derive from blockIdx and kernel arguments);
// readfirstlane states it, so the descriptor lives in SGPRs -- otherwise the
// compiler may keep it in VGPRs and wrap every load in a waterfall loop.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b >> 32));
  const uint64_t ub = (static_cast<uint64_t>(hi) << 32) | lo;
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(ub), (short)0,
                                           (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ void map_tile(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int T = tiles_m * tiles_n;
  const int x = bid % kNumXcd, i = bid / kNumXcd;
  const int q = T / kNumXcd, r = T % kNumXcd;
  const int t = x * q + min(x, r) + i;
  const int per_group = kGroupM * tiles_n;
  const int g = t / per_group;
  const int first_m = g * kGroupM;
  const int gm = min(kGroupM, tiles_m - first_m);
  const int w = t - g * per_group;
  tm = first_m + w % gm;
  tn = w / gm;
}

// s_waitcnt immediates (gfx9 encoding): vmcnt in bits [3:0] and [15:14],
// expcnt [6:4], lgkmcnt [11:8]; a field at its maximum means "don't wait".
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <int OUT>
__device__ __forceinline__ float load_out(const void* C, int64_t idx) {
  if constexpr (OUT == OUT_F32) {
    return static_cast<const float*>(C)[idx];
  } else {
    const uint32_t h = static_cast<const uint16_t*>(C)[idx];
    return __builtin_bit_cast(float, h << 16);
  }
}

template <int OUT>
__device__ __forceinline__ void store_out(void* D, int64_t idx, float v) {
  if constexpr (OUT == OUT_F32) {
    static_cast<float*>(D)[idx] = v;
  } else {
    static_cast<uint16_t*>(D)[idx] = f32_to_bf16_rne(v);
  }
}

// Per-input-type MFMA shape.  The wave's 128 x 128 accumulator is NB x NB
// blocks of BLK x BLK.  A wave reads 16 fragments of 16 bytes per half
// slab (8 of A, 8 of B), all at immediate offsets from at most two base
// registers per operand.
template <int IN>
struct Mma;

// 16 x 16 shapes (bf16, fp32): read r of an operand covers rows 16r +
// lane%16 of the wave's 128 rows and chunk lane/16 of the half slab.
struct Mma16Base {
  static constexpr int BLK = 16, NB = 8, R = 4;
  static constexpr bool kSplitDma = true;   // A and B bursts half a slab apart
  typedef f32x4 Acc;
  typedef i32x4 Frags[16];  // 0..7: A blocks, 8..15: B blocks
  // reads r and r+1 are 16 rows (two 8-row LDS blocks) apart
  static constexpr int kReadStride = 2 * 1024;
  __device__ static int base_row(int lane, int odd) { return lane & 15; }
  __device__ static int base_chunk(int lane, int odd) { return lane >> 4; }
  __device__ static void read(const uint8_t* half_base, const int (&fb)[4], Frags& F) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      F[r] = *reinterpret_cast<const i32x4*>(half_base + fb[0] + kReadStride * r);
      F[8 + r] = *reinterpret_cast<const i32x4*>(half_base + fb[2] + kReadStride * r);
    }
  }
  // MFMA 16 x 16 result: lane holds column lane%16, rows 4*(lane/16) + r
  __device__ static int out_row(int i, int r, int lane) { return 16 * i + 4 * (lane >> 4) + r; }
  __device__ static int out_col(int j, int lane) { return 16 * j + (lane & 15); }
};

template <>
struct Mma<IN_BF16> : Mma16Base {
  __device__ static void mma(const Frags& F, Acc (&acc)[NB][NB]) {
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, F[i]), __builtin_bit_cast(bf16x8, F[8 + j]), acc[i][j], 0,
            0, 0);
  }
};

template <>
struct Mma<IN_F32> : Mma16Base {
  // The lane's 4 floats of a block are K values 4*(lane/16) + t; MFMA t
  // takes lane group lane/16 as its K index 0..3, identically for A and B.
  __device__ static void mma(const Frags& F, Acc (&acc)[NB][NB]) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const f32x4 a = __builtin_bit_cast(f32x4, F[i]);
          const f32x4 b = __builtin_bit_cast(f32x4, F[8 + j]);
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[t], b[t], acc[i][j], 0, 0, 0);
        }
  }
};

// 32 x 32 shapes: read r of an operand covers block r/2 (rows 32*(r/2) +
// lane%32) and chunk 2*(lane/32) + r%2: 32 contiguous bytes per lane per block.
struct Mma32Base {
  static constexpr int BLK = 32, NB = 4, R = 16;
  // one DMA burst per slab: the split measured 9% slower for e4m3 (1638 vs
  // 1795 TFLOP/s at 8192 x 13312 x 16384), 21% faster for bf16
  static constexpr bool kSplitDma = false;
  typedef f32x16 Acc;
  typedef i32x8 Frags[8];  // 0..3: A blocks, 4..7: B blocks (32 bytes per lane)
  // block r/2 is 32 rows (four 8-row LDS blocks) further on
  static constexpr int kReadStride = 4 * 1024;
  __device__ static int base_row(int lane, int odd) { return lane & 31; }
  __device__ static int base_chunk(int lane, int odd) { return 2 * (lane >> 5) + odd; }
  __device__ static void read(const uint8_t* half_base, const int (&fb)[4], Frags& F) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const i32x4 a0 = *reinterpret_cast<const i32x4*>(half_base + fb[0] + kReadStride * b);
      const i32x4 a1 = *reinterpret_cast<const i32x4*>(half_base + fb[1] + kReadStride * b);
      const i32x4 b0 = *reinterpret_cast<const i32x4*>(half_base + fb[2] + kReadStride * b);
      const i32x4 b1 = *reinterpret_cast<const i32x4*>(half_base + fb[3] + kReadStride * b);
      F[b] = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
      F[4 + b] = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  }
  // MFMA 32 x 32 result: lane holds column lane%32, rows 8*(r/4) + 4*(lane/32) + r%4
  __device__ static int out_row(int i, int r, int lane) {
    return 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
  }
  __device__ static int out_col(int j, int lane) { return 32 * j + (lane & 31); }
};

template <>
struct Mma<IN_E4M3> : Mma32Base {
  __device__ static void mma(const Frags& F, Acc (&acc)[NB][NB]) {
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
        // formats 0/0 = e4m3 for A and B; E8M0 scale 127 = 2^0
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(F[i], F[NB + j], acc[i][j], 0,
                                                                    0, 0, 127, 0, 127);
  }
};

// Tile-invariant addressing of one workgroup.
//
// LDS layout of one operand in a stage: 32 blocks of 8 rows x 128 bytes,
// block b at b * 1 KiB; inside a block, half h (bytes 64h..64h+63 of each
// row) at + 512 h, row r % 8 at + 64 (r % 8), and logical 16-byte chunk q
// of the half at + 16 (q ^ f(r)).  One DMA instruction fills one block:
// lane l takes half l/32, row (l/4) % 8 and stored chunk l % 4, so every
// row's whole 128-byte line is read by one instruction.
struct TileCtx {
  const uint8_t* Ab;
  const uint8_t* Bb;
  uint32_t a_bytes, b_bytes;  // valid rows * row bytes
  uint32_t ga[2], gb[2];      // per-lane global offsets for even / odd blocks
  uint32_t lda16, ldb16;      // 16 rows of A / B in bytes (block pair stride)
  uint32_t gk[2];             // lane's K byte offset within a slab, even / odd blocks
  int kbytes;
  int fill;                   // wave's first LDS block within an operand stage
  int KT;
};

// Issue the DMA of one operand (OP 0: A, 1: B, 2: both) of slab kt into `stage`.
template <int OP>
__device__ __forceinline__ void issue_slab(const TileCtx& c, uint8_t* smem, int kt, int stage) {
  const uint32_t k0b = static_cast<uint32_t>(kt) * kSlab;
  // chunks past K: top offset bit set, so the load is out of range (zeros)
  uint32_t kinv[2];
#pragma unroll
  for (int odd = 0; odd < 2; ++odd)
    kinv[odd] = (static_cast<int>(k0b + c.gk[odd]) < c.kbytes) ? 0u : kOutOfRange;
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(c.Ab + k0b, c.a_bytes - k0b);
  const __amdgpu_buffer_rsrc_t rB = make_rsrc(c.Bb + k0b, c.b_bytes - k0b);
  uint8_t* sA = smem + stage * kStageBytes + c.fill;
  uint8_t* sB = sA + kOperandStage;
  if constexpr (OP != 1) {
#pragma unroll
    for (int i = 0; i < kLoadsPerOperand; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (lds_ptr_t)(sA + 1024 * i), 16,
                                               (c.ga[i & 1] + (i >> 1) * c.lda16) | kinv[i & 1], 0,
                                               0, 0);
  }
  if constexpr (OP != 0) {
#pragma unroll
    for (int i = 0; i < kLoadsPerOperand; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, (lds_ptr_t)(sB + 1024 * i), 16,
                                               (c.gb[i & 1] + (i >> 1) * c.ldb16) | kinv[i & 1], 0,
                                               0, 0);
  }
}

// Main loop.  Slab kt lives in LDS stage kt % 2 and is multiplied in two
// half steps.  Fragments of the next half slab are read while the current
// one is multiplied (F0 holds half 0, F1 half 1).  At the end of each slab
// one barrier certifies that every wave holds the slab in registers and that
// the next slab has landed; the slab after next is then loaded into the
// stage just vacated, so loads run one slab (about 2000 MFMA cycles) ahead.
// In the 16 x 16 family a slab's DMA goes out in two bursts -- its A rows
// right after that barrier, its B rows one half step later: issuing all 16
// loads of every wave at the barrier made each CU ask L2 for 64 KiB at once
// and measured about 20% slower.  The steady-state body has no branches, so
// the fragment buffers keep fixed registers; the last two slabs are peeled.
template <int IN>
__device__ __forceinline__ void half0(const TileCtx& c, uint8_t* smem, const int (&fb)[4], int kt,
                                      bool issue_b, typename Mma<IN>::Frags& F0,
                                      typename Mma<IN>::Frags& F1,
                                      typename Mma<IN>::Acc (&acc)[Mma<IN>::NB][Mma<IN>::NB]) {
  wait_lgkmcnt0();
  if constexpr (Mma<IN>::kSplitDma)
    if (issue_b) issue_slab<1>(c, smem, kt + 1, (kt + 1) & 1);
  Mma<IN>::read(smem + (kt & 1) * kStageBytes + 512, fb, F1);
  Mma<IN>::mma(F0, acc);
}

template <int IN>
__device__ __forceinline__ void half1(const TileCtx& c, uint8_t* smem, const int (&fb)[4], int kt,
                                      bool more, bool issue_next, typename Mma<IN>::Frags& F0,
                                      typename Mma<IN>::Frags& F1,
                                      typename Mma<IN>::Acc (&acc)[Mma<IN>::NB][Mma<IN>::NB]) {
  wait_lgkmcnt0();
  if (more) {
    wait_vmcnt<0>();  // slab kt+1, the only one in flight, has landed
    __syncthreads();
    if (issue_next) issue_slab<Mma<IN>::kSplitDma ? 0 : 2>(c, smem, kt + 2, kt & 1);
    Mma<IN>::read(smem + ((kt + 1) & 1) * kStageBytes, fb, F0);
  }
  Mma<IN>::mma(F1, acc);
}

template <int IN, int OUT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void
gemm_tn_kernel(GemmParams p) {
  using M = Mma<IN>;
  constexpr int ES = elem_size<IN>();
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * kStageBytes];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int l = blockIdx.y;

  const int tiles_m = (p.M + kBM - 1) / kBM;
  const int tiles_n = (p.N + kBN - 1) / kBN;
  int tm, tn;
  map_tile(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * kBM, n0 = tn * kBN;

  TileCtx c;
  c.Ab = static_cast<const uint8_t*>(p.A) + (l * p.sA + static_cast<int64_t>(m0) * p.lda) * ES;
  c.Bb = static_cast<const uint8_t*>(p.B) + (l * p.sB + static_cast<int64_t>(n0) * p.ldb) * ES;
  const uint32_t lda_b = static_cast<uint32_t>(p.lda * ES);
  const uint32_t ldb_b = static_cast<uint32_t>(p.ldb * ES);
  c.a_bytes = static_cast<uint32_t>(min(kBM, p.M - m0)) * lda_b;
  c.b_bytes = static_cast<uint32_t>(min(kBN, p.N - n0)) * ldb_b;
  c.kbytes = p.K * ES;
  c.lda16 = 16 * lda_b;
  c.ldb16 = 16 * ldb_b;
  const int KT = (c.kbytes + kSlab - 1) / kSlab;
  c.KT = KT;

  // DMA lane mapping.  Wave w fills blocks 8w .. 8w+7 of each operand
  // stage; block b holds rows 8b .. 8b+7, so f(row) depends on b % 2 and
  // on the lane's row within the block.
  const int half = lane >> 5, brow = (lane >> 2) & 7, schunk = lane & 3;
#pragma unroll
  for (int odd = 0; odd < 2; ++odd) {
    const int row = 64 * wave + 8 * odd + brow;          // row of block 8w + odd
    const int gch = half * 4 + (schunk ^ chunk_perm(row));
    c.ga[odd] = row * lda_b + gch * 16;
    c.gb[odd] = row * ldb_b + gch * 16;
    c.gk[odd] = gch * 16;
  }
  c.fill = wave * 8 * 1024;

  // Fragment base offsets within a stage: [A even, A odd, B even, B odd].
  // Rows of every read of a lane agree mod 16 with the lane's base row.
  int fb[4];
#pragma unroll
  for (int odd = 0; odd < 2; ++odd) {
    const int ra = wm * 128 + M::base_row(lane, odd);
    const int rb = wn * 128 + M::base_row(lane, odd);
    const int q = M::base_chunk(lane, odd);
    fb[odd] = (ra >> 3) * 1024 + (ra & 7) * 64 + ((q ^ chunk_perm(ra)) << 4);
    fb[2 + odd] = kOperandStage + (rb >> 3) * 1024 + (rb & 7) * 64 + ((q ^ chunk_perm(rb)) << 4);
  }

  typename M::Acc acc[M::NB][M::NB];
#pragma unroll
  for (int i = 0; i < M::NB; ++i)
#pragma unroll
    for (int j = 0; j < M::NB; ++j) acc[i][j] = typename M::Acc{};

  typename M::Frags F0, F1;

  // Prologue: slab 0 and slab 1 in flight (slab 1's B rows are issued in
  // slab 0's first half step when the DMA is split), slab 0 complete, its
  // half 0 requested.
  issue_slab<2>(c, smem, 0, 0);
  if constexpr (M::kSplitDma) {
    if (KT > 1) issue_slab<0>(c, smem, 1, 1);
    if (KT > 1) wait_vmcnt<kLoadsPerOperand>();
    else wait_vmcnt<0>();
  } else {
    if (KT > 1) issue_slab<2>(c, smem, 1, 1);
    if (KT > 1) wait_vmcnt<2 * kLoadsPerOperand>();
    else wait_vmcnt<0>();
  }
  __syncthreads();
  M::read(smem, fb, F0);

  int kt = 0;
  for (; kt + 2 < KT; ++kt) {
    half0<IN>(c, smem, fb, kt, true, F0, F1, acc);
    half1<IN>(c, smem, fb, kt, true, true, F0, F1, acc);
  }
  if (kt + 1 < KT) {  // second to last slab: no slab after next
    half0<IN>(c, smem, fb, kt, true, F0, F1, acc);
    half1<IN>(c, smem, fb, kt, true, false, F0, F1, acc);
    ++kt;
  }
  half0<IN>(c, smem, fb, kt, false, F0, F1, acc);  // last slab
  half1<IN>(c, smem, fb, kt, false, false, F0, F1, acc);

  // Epilogue: D = alpha * acc + beta * C, through a per-wave base pointer.
  const int wrow0 = m0 + wm * 128, wcol0 = n0 + wn * 128;
  const int rows_left = p.M - wrow0, cols_left = p.N - wcol0;
  constexpr int OES = OUT == OUT_F32 ? 4 : 2;
  uint8_t* Dw = static_cast<uint8_t*>(p.D) + (l * p.sD + static_cast<int64_t>(wrow0) * p.ldd +
                                               wcol0) * OES;
  const uint8_t* Cw =
      p.beta != 0.0f ? static_cast<const uint8_t*>(p.C) +
                           (l * p.sC + static_cast<int64_t>(wrow0) * p.ldc + wcol0) * OES
                     : nullptr;
  const bool use_c = p.beta != 0.0f;
#pragma unroll
  for (int i = 0; i < M::NB; ++i) {
#pragma unroll
    for (int r = 0; r < M::R; ++r) {
      const int row = M::out_row(i, r, lane);
      if (row >= rows_left) continue;
      uint8_t* drow = Dw + static_cast<int64_t>(row) * p.ldd * OES;
      const uint8_t* crow = use_c ? Cw + static_cast<int64_t>(row) * p.ldc * OES : nullptr;
#pragma unroll
      for (int j = 0; j < M::NB; ++j) {
        const int col = M::out_col(j, lane);
        if (col < cols_left) {
          float v = p.alpha * acc[i][j][r];
          if (use_c) v = __builtin_fmaf(p.beta, load_out<OUT>(crow, col), v);
          store_out<OUT>(drow, col, v);
        }
      }
    }
  }
}

template <int IN, int OUT>
inline hipError_t launch_t(const GemmParams& p, hipStream_t stream) {
  const int tiles_m = (p.M + kBM - 1) / kBM;
  const int tiles_n = (p.N + kBN - 1) / kBN;
  const dim3 grid(static_cast<unsigned>(tiles_m) * static_cast<unsigned>(tiles_n),
                  static_cast<unsigned>(p.L));
  hipLaunchKernelGGL((gemm_tn_kernel<IN, OUT>), grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace tile
}  // namespace dg
