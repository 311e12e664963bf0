// gemm_tile.h -- gfx950 (CDNA4) MFMA GEMM with an alpha/beta epilogue: the per-step GEMM of
// the TP schedules (the dense GEMM that the Distributed GEMM pull-request
// page runs at every step, written here for MI355X).
//
// Tiling.  A workgroup of 256 threads (4 wave64s, one per SIMD) owns a
// 256 x 256 tile of D; the waves form a 2 x 2 grid and each holds a
// 128 x 128 fp32 accumulator in all 256 of its AGPRs.  K is walked in slabs
// of 128 bytes per operand row (64 bf16, 128 e4m3 or 32 fp32 values), each
// multiplied in two half slabs of 64 bytes, so one LDS geometry serves every
// input type and only the MFMA differs:
//   bf16 : v_mfma_f32_16x16x32_bf16    (8 x 8 blocks of 16 x 16,   64 per half slab)
//   fp32 : v_mfma_f32_16x16x4_f32      (8 x 8 blocks x 4 K steps, 256 per half slab)
//   e4m3 : v_mfma_f32_32x32x64_f8f6f4  (4 x 4 blocks of 32 x 32,   16 per half slab;
//          per-tensor scales are applied in the epilogue)
//
// Data movement.  Both operands are K-contiguous ("TN"), so a lane's MFMA
// fragment is 16 contiguous bytes of one row (ds_read_b128).  Operand slabs
// go from global memory straight into LDS with buffer_load_dwordx4 ... lds:
// each wave instruction fills 1 KiB of LDS (lane l -> bytes 16l..16l+15),
// eight whole 128-byte rows, so the L1 asks L2 for full lines.  Within a
// 64-byte half row the four 16-byte chunks of row r are stored XOR-permuted
// by f(r) = ((r>>1) ^ (r>>2)) & 3, which puts the rows that one LDS cycle
// serves on distinct banks (zero bank conflicts measured).  The buffer
// descriptor of each operand covers only the tile's valid rows, so rows past
// M or N load as zeros (out-of-range lanes of an LDS load write zeros), and
// chunks past K are pushed out of range by the offset's top bit.
//
// Pipeline.  LDS holds a ring of five 32 KiB operand slabs (160 KiB): A(kt)
// in slot 2kt mod 5, B(kt) in slot 2kt+1 mod 5.  While slab kt is being
// multiplied, slab kt+1 is resident and A(kt+2) is in flight.  One barrier
// per slab (at the start of its second half) certifies that every wave holds
// slab kt in registers and that slab kt+1 has landed; it is a bare s_barrier
// after an explicit s_waitcnt, because the fence of __syncthreads() would
// wait for every outstanding LDS load, A(kt+2) included.
//
// Issue order.  With one wave per SIMD, any instruction the wave issues
// between MFMAs that the MFMA pipe has not covered is idle matrix time, so
// each half slab is written as a fixed sequence: its MFMAs, with the
// fragment reads of the next half slab and the DMA loads of the slab being
// prefetched placed after given MFMAs (scheduling barriers keep that order).
// The MFMAs are inline asm with the accumulator tied to an AGPR, which keeps
// all 64 accumulator blocks in place across the loop; with the builtin the
// compiler copied accumulators between MFMAs (about 100 to 400 moves per
// slab) and the kernel ran at about half the MFMA rate.
//
// Workgroup -> tile mapping is XCD-aware: MI355X places workgroup b on XCD
// b mod 8, so each XCD gets one contiguous range of the tile order, and
// that order walks groups of kGroupM tile rows column by column, so the tiles an
// XCD runs together share A rows and B columns in its own L2.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <algorithm>
#include <type_traits>

#include "gemm_launch.h"

namespace dg {
namespace tile {

typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

constexpr int kThreads = 256;
constexpr int kSlab = 128;                        // bytes of K per operand row per slab
constexpr int kOperandSlab = kBM * kSlab;         // 32 KiB
constexpr int kSlots = 5;                         // LDS ring of operand slabs: 160 KiB
// The operand loaded three half slabs ahead of its use (the other, two):
// 0 = A, 1 = B.  B: the 32 tiles an XCD runs at a time span 8 tile columns
// and 4 tile rows, so a B slab is shared by fewer of them and misses the
// L2 more often; the longer lead measured 0.5-1% faster on the bf16 and
// e4m3 TP=8 shapes.
constexpr int kLead = 1;
constexpr int kLoadsPerOperand = kOperandSlab / 1024 / 4;  // per wave: 8
constexpr uint32_t kOutOfRange = 0x80000000u;
// Height, in tiles, of a group of output rows walked column by column.  Four
// rows of 256 keep each XCD's A panel small enough that the eight XCDs' panels
// stay resident in the last-level cache together (measured: 4 beats 2, 6, 8,
// 16 and 32 at 4096-16384 rows).
constexpr int kGroupM = 4;

static_assert(kBM == 256 && kBN == 256, "tile geometry");
static_assert(kRowBytes == kSlab, "slab width");

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

// Position t of the tile order -> tile (tm, tn): groups of kGroupM tile rows,
// each walked column by column.
__device__ __forceinline__ void order_tile(int t, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int per_group = kGroupM * tiles_n;
  const int g = t / per_group;
  const int first_m = g * kGroupM;
  const int gm = min(kGroupM, tiles_m - first_m);
  const int w = t - g * per_group;
  tm = first_m + w % gm;
  tn = w / gm;
}

// Workgroup bid -> tile: XCD bid mod 8 takes one contiguous range of the order.
__device__ __forceinline__ void map_tile(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int T = tiles_m * tiles_n;
  const int x = bid % kNumXcd, i = bid / kNumXcd;
  const int q = T / kNumXcd, r = T % kNumXcd;
  order_tile(x * q + min(x, r) + i, tiles_m, tiles_n, tm, tn);
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
// Workgroup barrier without a memory fence: the caller has already waited
// for what the other waves must see (its LDS loads, its fragment reads).
// gfx950 does not drain memory counters at s_barrier; the "memory" clobber
// keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// OCP e4m3fn (sign, 4 exponent bits with bias 7, 3 mantissa bits; no
// infinities; S.1111.111 is NaN; largest finite 448; subnormals m * 2^-9),
// from the format's definition.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  const uint32_t sign = (b & 0x80u) << 24, e = (b >> 3) & 15u, m = b & 7u;
  if (e == 15u && m == 7u) return __builtin_bit_cast(float, sign | 0x7fc00000u);
  if (e == 0u) return __builtin_bit_cast(float, sign | __builtin_bit_cast(uint32_t, static_cast<float>(m) * 0.001953125f));
  return __builtin_bit_cast(float, sign | ((e + 120u) << 23) | (m << 20));
}

// fp32 -> e4m3fn, round to nearest even, saturating at +-448 (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_e4m3_rne_sat(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  const uint32_t sign = (u >> 24) & 0x80u, a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return sign | 0x7fu;
  if (a >= 0x43e00000u) return sign | 0x7eu;  // |f| >= 448 (infinities too)
  if (a < 0x3c800000u) {
    // below 2^-6: multiples of 2^-9; 8 * 2^-9 is the smallest normal (code 8)
    const float q = __builtin_rintf(__builtin_bit_cast(float, a) * 512.0f);
    return sign | static_cast<uint32_t>(q);
  }
  // normal: keep three mantissa bits, ties to even; the carry may raise the exponent
  const uint32_t r = (a + 0x7ffffu + ((a >> 20) & 1u)) >> 20;
  const uint32_t code = r - ((127u - 7u) << 3);
  return sign | (code > 0x7eu ? 0x7eu : code);
}

template <int OUT>
constexpr int out_size() {
  return OUT == OUT_F32 ? 4 : (OUT == OUT_BF16 ? 2 : 1);
}

template <int OUT>
__device__ __forceinline__ float load_out(const void* C, int64_t idx) {
  if constexpr (OUT == OUT_F32) {
    return static_cast<const float*>(C)[idx];
  } else if constexpr (OUT == OUT_BF16) {
    const uint32_t h = static_cast<const uint16_t*>(C)[idx];
    return __builtin_bit_cast(float, h << 16);
  } else {
    return e4m3_to_f32(static_cast<const uint8_t*>(C)[idx]);
  }
}

template <int OUT>
__device__ __forceinline__ void store_out(void* D, int64_t idx, float v) {
  if constexpr (OUT == OUT_F32) {
    static_cast<float*>(D)[idx] = v;
  } else if constexpr (OUT == OUT_BF16) {
    static_cast<uint16_t*>(D)[idx] = f32_to_bf16_rne(v);
  } else {
    static_cast<uint8_t*>(D)[idx] = static_cast<uint8_t>(f32_to_e4m3_rne_sat(v));
  }
}

// Per-input-type MFMA shape and issue schedule.  The wave's 128 x 128
// accumulator is NB x NB blocks of BLK x BLK.  A half slab takes kMfma
// MFMAs and kReads fragment reads of 16 bytes per lane.  Within a half slab,
// fragment read q follows MFMA kReadAt + (q / kReadsPer) * kReadEvery and
// DMA load d follows MFMA kDmaAt + d * kDmaEvery; both end early enough for
// the reads to land before the next half slab and for the loads to keep
// their lead.  The persistent kernel's in-loop copy issues its four stores
// after MFMA kCopyAt of the second half slab and its four loads after MFMA
// kCopyAt + kCopyEvery, behind the operand DMA.
template <int IN>
struct Mma;

// 16 x 16 shapes (bf16, fp32): read r of an operand covers rows 16r +
// lane%16 of the wave's 128 rows and chunk lane/16 of the half slab.
struct Mma16Base {
  static constexpr int BLK = 16, NB = 8, R = 4;
  static constexpr int NBM = NB;  // block rows of the wave's accumulator
  static constexpr int kLoadsA = kLoadsPerOperand, kLoadsB = kLoadsPerOperand;  // DMA loads per wave per slab
  static constexpr int kReads = 16;
  typedef f32x4 Acc;
  typedef i32x4 Frags[16];  // 0..7: A blocks, 8..15: B blocks
  // reads r and r+1 are 16 rows (two 8-row LDS blocks) apart
  static constexpr int kReadStride = 2 * 1024;
  __device__ __forceinline__ static int base_row(int lane, int odd) { return lane & 15; }
  __device__ __forceinline__ static int base_chunk(int lane, int odd) { return lane >> 4; }
  // read q: A block q/2 (q even) or B block q/2 (q odd)
  __device__ __forceinline__ static void read(int q, const uint8_t* a, const uint8_t* b, const int (&fb)[4],
                              Frags& F) {
    const int r = q >> 1;
    if ((q & 1) == 0)
      F[r] = *reinterpret_cast<const i32x4*>(a + fb[0] + kReadStride * r);
    else
      F[8 + r] = *reinterpret_cast<const i32x4*>(b + fb[2] + kReadStride * r);
  }
  // MFMA 16 x 16 result: lane holds column lane%16, rows 4*(lane/16) + r
  __device__ __forceinline__ static int out_row(int i, int r, int lane) { return 16 * i + 4 * (lane >> 4) + r; }
  // 16-row part of the wave block that holds result register r of block row i
  static constexpr int part_of(int i, int r) { return i; }
  __device__ __forceinline__ static int out_col(int j, int lane) { return 16 * j + (lane & 15); }
};

template <>
struct Mma<IN_BF16> : Mma16Base {
  static constexpr int kMfma = 64;
  // reads after MFMAs 0, 3, .., 45 and DMA loads after 2, 8, .., 44: spread
  // over three quarters of the half slab rather than packed into its first
  // half (one read after every other MFMA waited for LDS issue slots);
  // measured +1.4% on a 16384 x 13312 x 16384 TP=8 schedule
  static constexpr int kReadAt = 0, kReadEvery = 3, kReadsPer = 1;
  static constexpr int kDmaAt = 2, kDmaEvery = 6;
  static constexpr int kCopyAt = 48, kCopyEvery = 8;
  // MFMA m: block (m / 8, m % 8)
  __device__ __forceinline__ static void mma(int m, const Frags& F, Acc (&acc)[NB][NB]) {
    const int i = m >> 3, j = m & 7;
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0"
                 : "+a"(acc[i][j])
                 : "v"(F[i]), "v"(F[8 + j]));
  }
};

template <>
struct Mma<IN_F32> : Mma16Base {
  static constexpr int kMfma = 256;
  static constexpr int kReadAt = 1, kReadEvery = 4, kReadsPer = 1;
  static constexpr int kDmaAt = 2, kDmaEvery = 8;
  static constexpr int kCopyAt = 96, kCopyEvery = 32;
  // MFMA m: K step t = m / 64 of block ((m / 8) % 8, m % 8).  The lane's 4
  // floats of a block are K values 4*(lane/16) + t; the 16x16x4 MFMA takes
  // lane group lane/16 as its K index, identically for A and B.
  __device__ __forceinline__ static void mma(int m, const Frags& F, Acc (&acc)[NB][NB]) {
    const int t = m >> 6, i = (m >> 3) & 7, j = m & 7;
    const float a = __builtin_bit_cast(f32x4, F[i])[t];
    const float b = __builtin_bit_cast(f32x4, F[8 + j])[t];
    asm volatile("v_mfma_f32_16x16x4_f32 %0, %1, %2, %0" : "+a"(acc[i][j]) : "v"(a), "v"(b));
  }
};

// 32 x 32 shape (e4m3): read r of an operand covers block r/2 (rows 32*(r/2)
// + lane%32) and chunk 2*(lane/32) + r%2: 32 contiguous bytes per lane per
// block, read as two 16-byte halves.
struct Mma32Base {
  static constexpr int BLK = 32, NB = 4, R = 16;
  static constexpr int NBM = NB;
  static constexpr int kLoadsA = kLoadsPerOperand, kLoadsB = kLoadsPerOperand;
  static constexpr int kReads = 16;
  typedef f32x16 Acc;
  typedef i32x8 Frags[8];  // 0..3: A blocks, 4..7: B blocks (32 bytes per lane)
  // block b is 32 rows (four 8-row LDS blocks) further on
  static constexpr int kReadStride = 4 * 1024;
  __device__ __forceinline__ static int base_row(int lane, int odd) { return lane & 31; }
  __device__ __forceinline__ static int base_chunk(int lane, int odd) { return 2 * (lane >> 5) + odd; }
  // read q: block q/4 of A (q%4 < 2) or B, half q%2 of its 32 bytes
  __device__ __forceinline__ static void read(int q, const uint8_t* a, const uint8_t* b, const int (&fb)[4],
                              Frags& F) {
    const int blk = q >> 2, op = (q >> 1) & 1, h = q & 1;
    const i32x4 v = *reinterpret_cast<const i32x4*>((op ? b : a) + fb[2 * op + h] +
                                                    kReadStride * blk);
    if (h == 0)
      F[4 * op + blk].lo = v;
    else
      F[4 * op + blk].hi = v;
  }
  // MFMA 32 x 32 result: lane holds column lane%32, rows 8*(r/4) + 4*(lane/32) + r%4
  __device__ __forceinline__ static int out_row(int i, int r, int lane) {
    return 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
  }
  // 16-row part of the wave block that holds result register r of block row i
  static constexpr int part_of(int i, int r) { return 2 * i + (r >> 3); }
  __device__ __forceinline__ static int out_col(int j, int lane) { return 32 * j + (lane & 31); }
};

template <>
struct Mma<IN_E4M3> : Mma32Base {
  static constexpr int kMfma = 16;
  static constexpr int kReadAt = 0, kReadEvery = 1, kReadsPer = 2;
  static constexpr int kDmaAt = 0, kDmaEvery = 1;
  static constexpr int kCopyAt = 9, kCopyEvery = 3;
  // MFMA m: block (m / 4, m % 4); format fields 0/0 select e4m3 for A and B
  __device__ __forceinline__ static void mma(int m, const Frags& F, Acc (&acc)[NB][NB]) {
    const int i = m >> 2, j = m & 3;
    asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0"
                 : "+a"(acc[i][j])
                 : "v"(F[i]), "v"(F[NB + j]));
  }
};

// Half-height tile (128 x 256, for a last round of tiles that would leave at
// least half of the CUs idle): each wave's accumulator is NBM = NB / 2 block
// rows by NB block columns (64 x 128), A slabs hold 128 rows (4 DMA loads
// per wave instead of 8), and a half slab takes half the MFMAs and the reads
// of NBM A blocks and NB B blocks (the A blocks and the first B blocks in the
// full tile's order, then the other B blocks).  Every output element is
// computed by the same MFMA instruction in the same K order as in a full
// tile, so results are bitwise the same.
template <int IN>
struct MmaHalf;

template <>
struct MmaHalf<IN_BF16> : Mma16Base {
  static constexpr int NBM = 4;
  static constexpr int kLoadsA = 4;
  static constexpr int kMfma = 32, kReads = 12;
  static constexpr int kReadAt = 0, kReadEvery = 2, kReadsPer = 1;
  static constexpr int kDmaAt = 1, kDmaEvery = 3;
  static constexpr int kCopyAt = 25, kCopyEvery = 3;
  // read q < 8: A block q/2 (q even) or B block q/2; q >= 8: B block q - 4
  __device__ __forceinline__ static void read(int q, const uint8_t* a, const uint8_t* b, const int (&fb)[4],
                                              Frags& F) {
    if (q < 2 * NBM)
      Mma16Base::read(q, a, b, fb, F);
    else
      F[8 + q - NBM] = *reinterpret_cast<const i32x4*>(b + fb[2] + kReadStride * (q - NBM));
  }
  __device__ __forceinline__ static void mma(int m, const Frags& F, Acc (&acc)[NBM][NB]) {
    const int i = m >> 3, j = m & 7;
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0"
                 : "+a"(acc[i][j])
                 : "v"(F[i]), "v"(F[8 + j]));
  }
};

template <>
struct MmaHalf<IN_F32> : Mma16Base {
  static constexpr int NBM = 4;
  static constexpr int kLoadsA = 4;
  static constexpr int kMfma = 128, kReads = 12;
  static constexpr int kReadAt = 1, kReadEvery = 4, kReadsPer = 1;
  static constexpr int kDmaAt = 2, kDmaEvery = 8;
  static constexpr int kCopyAt = 96, kCopyEvery = 16;
  __device__ __forceinline__ static void read(int q, const uint8_t* a, const uint8_t* b, const int (&fb)[4],
                                              Frags& F) {
    if (q < 2 * NBM)
      Mma16Base::read(q, a, b, fb, F);
    else
      F[8 + q - NBM] = *reinterpret_cast<const i32x4*>(b + fb[2] + kReadStride * (q - NBM));
  }
  // MFMA m: K step t = m / 32 of block ((m / 8) % 4, m % 8)
  __device__ __forceinline__ static void mma(int m, const Frags& F, Acc (&acc)[NBM][NB]) {
    const int t = m >> 5, i = (m >> 3) & 3, j = m & 7;
    const float a = __builtin_bit_cast(f32x4, F[i])[t];
    const float b = __builtin_bit_cast(f32x4, F[8 + j])[t];
    asm volatile("v_mfma_f32_16x16x4_f32 %0, %1, %2, %0" : "+a"(acc[i][j]) : "v"(a), "v"(b));
  }
};

template <>
struct MmaHalf<IN_E4M3> : Mma32Base {
  static constexpr int NBM = 2;
  static constexpr int kLoadsA = 4;
  static constexpr int kMfma = 8, kReads = 12;
  static constexpr int kReadAt = 0, kReadEvery = 1, kReadsPer = 2;
  static constexpr int kDmaAt = 0, kDmaEvery = 1;
  static constexpr int kCopyAt = 6, kCopyEvery = 1;
  // read q < 8: as the full tile's (blocks 0, 1 of A and B); q >= 8: B
  // blocks 2, 3, half q % 2
  __device__ __forceinline__ static void read(int q, const uint8_t* a, const uint8_t* b, const int (&fb)[4],
                                              Frags& F) {
    if (q < 8) {
      Mma32Base::read(q, a, b, fb, F);
    } else {
      const int blk = 2 + ((q - 8) >> 1), h = q & 1;
      const i32x4 v = *reinterpret_cast<const i32x4*>(b + fb[2 + h] + kReadStride * blk);
      if (h == 0)
        F[4 + blk].lo = v;
      else
        F[4 + blk].hi = v;
    }
  }
  __device__ __forceinline__ static void mma(int m, const Frags& F, Acc (&acc)[NBM][NB]) {
    const int i = m >> 2, j = m & 3;
    asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0"
                 : "+a"(acc[i][j])
                 : "v"(F[i]), "v"(F[NB + j]));
  }
};

// Tile-invariant addressing of one workgroup.
//
// LDS layout of one operand slab: 32 blocks of 8 rows x 128 bytes, block b
// at b * 1 KiB; inside a block, half h (bytes 64h..64h+63 of each row) at
// + 512 h, row r % 8 at + 64 (r % 8), and logical 16-byte chunk q of the half
// at + 16 (q ^ f(r)).  One DMA instruction fills one block: lane l takes half
// l/32, row (l/4) % 8 and stored chunk l % 4, so every row's whole 128-byte
// line is read by one instruction.
struct TileCtx {
  const uint8_t* Ab;
  const uint8_t* Bb;
  uint32_t a_bytes, b_bytes;  // valid rows * row bytes
  uint32_t ga[2], gb[2];      // per-lane global offsets for even / odd blocks
  uint32_t lda16, ldb16;      // 16 rows of A / B in bytes (block pair stride)
  uint32_t gk[2];             // lane's K byte offset within a slab, even / odd blocks
  int kshift;                 // bytes slab 0 starts before K = 0 (see SlabLoad)
  __amdgpu_buffer_rsrc_t rA, rB;  // the tile's valid rows of A / B from K = 0
  int fillA, fillB;           // wave's first LDS block within an A / B slab (bytes)
};

__device__ __forceinline__ int slot_add(int s, int d) {
  s += d;
  return s >= kSlots ? s - kSlots : s;
}

// DMA state of one operand slab (OP 0: A, 1: B) of slab kt bound for a ring
// slot.  Slab kt covers K bytes kt * 128 - kshift .. + 127: when K is not a
// multiple of the slab, slab 0 is the partial one and starts before K = 0,
// so every later slab lies wholly inside K and its loads need no per-lane
// mask (an OR per load cost 1.3-1.9% of the TP=8 runs).  kMask (slab
// 0 only): chunks before K = 0 get the top offset bit, so the load is out of
// range and fills zeros.
//
// Slabs kt >= 1 use the tile's descriptor (its valid rows from K = 0) with
// the slab's K offset as the scalar offset, so a slab costs no descriptor
// arithmetic: a lane of a valid row reads below the row's end (the slab lies
// inside K, and K <= the leading dimension), a lane of a row past the valid
// ones is out of range by its vector offset alone, with or without the
// scalar offset in the range check.  (A half-height tile whose rows all lie
// past M has no valid rows: every load is out of range.)
template <int OP, bool kMask = false>
struct SlabLoad {
  __amdgpu_buffer_rsrc_t r;
  uint32_t kinv[2];
  uint32_t soff;
  uint8_t* dst;
  __device__ __forceinline__ SlabLoad(const TileCtx& c, uint8_t* smem, int kt, int slot) {
    if constexpr (kMask) {
      // slab 0 (kt = 0): from -kshift
#pragma unroll
      for (int odd = 0; odd < 2; ++odd)
        kinv[odd] = (c.gk[odd] >= static_cast<uint32_t>(c.kshift)) ? 0u : kOutOfRange;
      r = make_rsrc((OP == 0 ? c.Ab : c.Bb) - c.kshift,
                    (OP == 0 ? c.a_bytes : c.b_bytes) + static_cast<uint32_t>(c.kshift));
      soff = 0;
    } else {
      r = OP == 0 ? c.rA : c.rB;
      soff = static_cast<uint32_t>(kt) * kSlab - static_cast<uint32_t>(c.kshift);
    }
    dst = smem + slot * kOperandSlab + (OP == 0 ? c.fillA : c.fillB);
  }
  // load d of the wave's: LDS block fill/1K + d, rows 8d.. of the wave's rows
  __device__ __forceinline__ void issue(const TileCtx& c, int d) const {
    const uint32_t* g = OP == 0 ? c.ga : c.gb;
    const uint32_t ld16 = OP == 0 ? c.lda16 : c.ldb16;
    uint32_t off = g[d & 1] + (d >> 1) * ld16;
    if constexpr (kMask) off |= kinv[d & 1];
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(dst + 1024 * d), 16, off, soff, 0, 0);
  }
};

template <typename M, int OP, bool kMask = false>
__device__ __forceinline__ void issue_operand(const TileCtx& c, uint8_t* smem, int kt, int slot) {
  const SlabLoad<OP, kMask> L(c, smem, kt, slot);
#pragma unroll
  for (int d = 0; d < (OP == 0 ? M::kLoadsA : M::kLoadsB); ++d) L.issue(c, d);
}

// One half slab: the MFMAs on Fm, with (kRead) the reads of the next half
// slab into Fr from LDS bases ra / rb and (kIssue) the DMA of operand kOp of
// slab kt_issue into ring slot slot_issue, in the type's fixed order.
template <typename M, bool kIssue, bool kRead, int kOp, typename X>
__device__ __forceinline__ void half_step(const TileCtx& c, uint8_t* smem, int kt_issue,
                                          int slot_issue, const uint8_t* ra, const uint8_t* rb,
                                          const int (&fb)[4], const typename M::Frags& Fm,
                                          typename M::Frags& Fr, typename M::Acc (&acc)[M::NBM][M::NB],
                                          const X& extra) {
  constexpr int kLoads = kOp == 0 ? M::kLoadsA : M::kLoadsB;
  const SlabLoad<kOp> L(c, smem, kt_issue, slot_issue);
#pragma unroll
  for (int m = 0; m < M::kMfma; ++m) {
    M::mma(m, Fm, acc);
    if constexpr (kIssue) {
      const int d = (m - M::kDmaAt) / M::kDmaEvery;
      if (m >= M::kDmaAt && (m - M::kDmaAt) % M::kDmaEvery == 0 && d < kLoads)
        L.issue(c, d);
    }
    if constexpr (kRead) {
      const int g = (m - M::kReadAt) / M::kReadEvery;
      if (m >= M::kReadAt && (m - M::kReadAt) % M::kReadEvery == 0) {
#pragma unroll
        for (int u = 0; u < M::kReadsPer; ++u)
          if (g * M::kReadsPer + u < M::kReads) M::read(g * M::kReadsPer + u, ra, rb, fb, Fr);
      }
    }
    extra(m);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Element-by-element epilogue of a wave's block (128 x 128, or 64 x 128 in a
// half-height tile; any alignment).
template <typename M, int OUT>
__device__ __forceinline__ void epilogue_direct(int lane, const typename M::Acc (&acc)[M::NBM][M::NB],
                                                const GemmParams& p, uint8_t* Dw, const uint8_t* Cw,
                                                const uint8_t* Bw, int rows_left, int cols_left) {
  constexpr int OES = out_size<OUT>();
  // the lane's bias values, one per column block (Bw: the wave's first column)
  float bv[M::NB];
#pragma unroll
  for (int j = 0; j < M::NB; ++j) {
    const int col = M::out_col(j, lane);
    bv[j] = (Bw && col < cols_left) ? load_out<OUT>(Bw, col) : 0.0f;
  }
#pragma unroll
  for (int i = 0; i < M::NBM; ++i) {
#pragma unroll
    for (int r = 0; r < M::R; ++r) {
      const int row = M::out_row(i, r, lane);
      if (row >= rows_left) continue;
      uint8_t* drow = Dw + static_cast<int64_t>(row) * p.ldd * OES;
      const uint8_t* crow = Cw ? Cw + static_cast<int64_t>(row) * p.ldc * OES : nullptr;
#pragma unroll
      for (int j = 0; j < M::NB; ++j) {
        const int col = M::out_col(j, lane);
        if (col < cols_left) {
          float v = p.alpha * acc[i][j][r];
          if (crow) v = __builtin_fmaf(p.beta, load_out<OUT>(crow, col), v);
          if (Bw) v += bv[j];
          if constexpr (OUT == OUT_E4M3) v *= p.post;
          store_out<OUT>(drow, col, v);
        }
      }
    }
  }
}

// LDS-staged epilogue (fp32 output): each 32-row quarter of the wave's block
// is written to the wave's 32 x 132-float LDS area in the MFMA layout and read
// back by rows, 4 consecutive values per lane (one 16-byte LDS read), so a
// lane stores 16 contiguous bytes with one instruction.  Measured: +10% on a
// 2048 x 13312 x 16384 bf16 GEMM, +2% on e4m3 with fp32 output.  For bf16
// output the element-wise stores are kept: the staged form measured equal for
// bf16 inputs and 17% slower for e4m3 inputs.  The LDS ring is free by now; the
// barrier makes sure no wave still reads it.
//
// C (beta != 0) of a wave block with all 128 x 128 elements in range is read
// one quarter ahead into a second register buffer: the 16 loads of quarter
// q + 1 are in flight while quarter q goes through LDS and is stored, so the
// C reads of a tile overlap one another instead of costing one memory round
// trip per 16 bytes.  Blocks at the edge of D keep the checked path.
constexpr int kEpiRow = 128 + 4;             // floats per staged row (padded)
constexpr int kEpiWave = 32 * kEpiRow;       // floats per wave: 16.5 KiB

// The lane's 16 C vectors of quarter q: rows 32q + 2t + lane/32, columns
// 4*(lane%32) .. +3 of the wave block.
__device__ __forceinline__ void load_c_quarter(const float* Cf, int64_t ldc, int lane, int q,
                                               f32x4 (&cq)[16]) {
  const float* c0 = Cf + static_cast<int64_t>(32 * q + (lane >> 5)) * ldc + 4 * (lane & 31);
#pragma unroll
  for (int t = 0; t < 16; ++t) cq[t] = *reinterpret_cast<const f32x4*>(c0 + 2 * t * ldc);
}

// Full 128 x 128 wave block without C: no bounds checks.
template <typename M>
__device__ __forceinline__ void epilogue_staged_full(float* lds, int lane,
                                                     const typename M::Acc (&acc)[M::NB][M::NB],
                                                     const GemmParams& p, uint8_t* Dw, bool has_bias,
                                                     f32x4 bb) {
  constexpr int kBlocksPerQuarter = 32 / M::BLK;
  const int bc = 4 * (lane & 31);
  barrier_only();
#pragma unroll
  for (int q = 0; q < 4; ++q) {
#pragma unroll
    for (int ib = 0; ib < kBlocksPerQuarter; ++ib) {
      const int i = q * kBlocksPerQuarter + ib;
#pragma unroll
      for (int r = 0; r < M::R; ++r)
#pragma unroll
        for (int j = 0; j < M::NB; ++j)
          lds[(M::out_row(i, r, lane) - 32 * q) * kEpiRow + M::out_col(j, lane)] = acc[i][j][r];
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    // 32 lanes per row, 4 floats each; two rows per instruction
    float* d0 = reinterpret_cast<float*>(Dw) + static_cast<int64_t>(32 * q + (lane >> 5)) * p.ldd + bc;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(&lds[(2 * t + (lane >> 5)) * kEpiRow + bc]);
      f32x4 v = a * p.alpha;
      if (has_bias) v += bb;
      *reinterpret_cast<f32x4*>(d0 + 2 * t * p.ldd) = v;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads done before the next writes
  }
}

// Full 128 x 128 wave block with C (fp32), in eight parts of 16 rows.  The
// C rows of part p + 2 go from memory straight into LDS (buffer_load ...
// lds: 8 instructions per wave, each two 512-byte rows; lane l receives the
// 16 bytes of row 2t + l/32, columns 4 (l % 32) ..) while part p is formed:
// alpha * acc staged in the MFMA layout (16 x 132 floats per wave) and read
// back by rows, and the lane adds beta times the very C bytes it loaded.  No
// registers hold C (the persistent kernel has none to spare), and 16 KiB of
// C per wave stay in flight, so the C reads of a tile overlap one another.
// LDS per wave: 8.25 KiB staging + three 8 KiB C buffers.
constexpr int kEpiCParts = 8;      // 16-row parts of a wave block
constexpr int kEpiCAhead = 2;      // parts of C in flight ahead of the one in use
constexpr int kEpiCBufs = kEpiCAhead + 1;
constexpr int kEpiStage = 16 * kEpiRow * 4;  // bytes of staging per wave
constexpr int kEpiPartWave = kEpiStage + kEpiCBufs * 8192;
// Every epilogue form places wave w's LDS area at w * kEpiWaveStride: the
// waves of one workgroup may take different forms (a wave block past the
// last row or column of D takes the checked one), and their areas must not
// overlap.  The last 256 bytes of LDS stay free for the persistent kernel's
// work-item broadcast.
constexpr int kEpiWaveStride = kEpiPartWave > kEpiWave * 4 ? kEpiPartWave : kEpiWave * 4;
static_assert(4 * kEpiWaveStride <= kSlots * kOperandSlab - 256, "epilogue LDS");

// Memory operations of one wave in the C epilogue, in issue order: C parts
// 0 .. kEpiCAhead - 1, then for each part p the C load of part p +
// kEpiCAhead (if any) followed, after the wait, by the 8 stores of part p.
// epi_c_wait(p) = instructions issued after part p's C load when part p
// waits for it (the s_waitcnt vmcnt immediate; loads and stores share the
// counter and retire in order).
constexpr int epi_c_wait(int p) {
  int after = 0;
  for (int c = p + 1; c < kEpiCParts && c <= p + kEpiCAhead; ++c) after += 8;  // later C loads
  for (int d = p - kEpiCAhead > 0 ? p - kEpiCAhead : 0; d < p; ++d) after += 8;  // stores since
  return after;
}

__device__ __forceinline__ void issue_c_part(const float* Cf, uint32_t ldc_b, int lane, int part,
                                             uint8_t* buf) {
  const __amdgpu_buffer_rsrc_t r =
      make_rsrc(reinterpret_cast<const uint8_t*>(Cf) + static_cast<int64_t>(16 * part) * ldc_b, 16 * ldc_b);
  const uint32_t off = static_cast<uint32_t>(lane >> 5) * ldc_b + 16 * (lane & 31);
#pragma unroll
  for (int t = 0; t < 8; ++t)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(buf + 1024 * t), 16, off + 2 * t * ldc_b, 0, 0, 0);
}

template <typename M, int P>
__device__ __forceinline__ void epilogue_c_part(uint8_t* base, int lane,
                                                const typename M::Acc (&acc)[M::NB][M::NB],
                                                const GemmParams& p, uint8_t* Dw, const float* Cf,
                                                uint32_t ldc_b, bool has_bias, f32x4 bb) {
  float* const stage = reinterpret_cast<float*>(base);
  if constexpr (P + kEpiCAhead < kEpiCParts)
    issue_c_part(Cf, ldc_b, lane, P + kEpiCAhead, base + kEpiStage + 8192 * ((P + kEpiCAhead) % kEpiCBufs));
  wait_vmcnt<epi_c_wait(P)>();  // C of this part has landed
#pragma unroll
  for (int i = 0; i < M::NB; ++i)
#pragma unroll
    for (int r = 0; r < M::R; ++r)
      if (M::part_of(i, r) == P)
#pragma unroll
        for (int j = 0; j < M::NB; ++j)
          stage[(M::out_row(i, r, lane) - 16 * P) * kEpiRow + M::out_col(j, lane)] = p.alpha * acc[i][j][r];
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  const uint8_t* const cb = base + kEpiStage + 8192 * (P % kEpiCBufs);
  const int bc = 4 * (lane & 31);
  f32x4 a[8], c[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    a[t] = *reinterpret_cast<const f32x4*>(&stage[(2 * t + (lane >> 5)) * kEpiRow + bc]);
    c[t] = *reinterpret_cast<const f32x4*>(cb + 1024 * t + 16 * lane);
  }
  float* d0 = reinterpret_cast<float*>(Dw) + static_cast<int64_t>(16 * P + (lane >> 5)) * p.ldd + bc;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    f32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = __builtin_fmaf(p.beta, c[t][e], a[t][e]);
    if (has_bias) v += bb;
    *reinterpret_cast<f32x4*>(d0 + 2 * t * p.ldd) = v;
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads done before the buffers are reused
  if constexpr (P + 1 < kEpiCParts) epilogue_c_part<M, P + 1>(base, lane, acc, p, Dw, Cf, ldc_b, has_bias, bb);
}

template <typename M>
__device__ __forceinline__ void epilogue_staged_c(uint8_t* smem, int wave, int lane,
                                                  const typename M::Acc (&acc)[M::NB][M::NB],
                                                  const GemmParams& p, uint8_t* Dw, const float* Cf,
                                                  bool has_bias, f32x4 bb) {
  const uint32_t ldc_b = static_cast<uint32_t>(p.ldc) * 4;
  uint8_t* const base = smem + wave * kEpiWaveStride;
  barrier_only();  // no wave reads the operand ring any more
#pragma unroll
  for (int c = 0; c < kEpiCAhead; ++c) issue_c_part(Cf, ldc_b, lane, c, base + kEpiStage + 8192 * c);
  epilogue_c_part<M, 0>(base, lane, acc, p, Dw, Cf, ldc_b, has_bias, bb);
}

// bf16 output without C, whole wave block (128 x 128, or 64 x 128 in a
// half-height tile), D rows 8-byte aligned:
// the same fp32 staging as above, read back 4 consecutive values per lane,
// rounded to bf16 (RNE, as the element-wise form) and stored as 8 bytes, so
// a wave writes two 256-byte row pieces per store instead of 2 bytes per lane.
// Element-wise 2-byte stores measured about 5% of the e4m3 8192 x 13312 x
// 16384 GEMM.  The caller has passed the workgroup barrier.
template <typename M>
__device__ __forceinline__ void epilogue_staged_bf16(uint8_t* smem, int wave, int lane,
                                                     const typename M::Acc (&acc)[M::NBM][M::NB],
                                                     const GemmParams& p, uint8_t* Dw, const uint8_t* Bw) {
  constexpr int kBlocksPerQuarter = 32 / M::BLK;
  constexpr int kQuarters = M::NBM / kBlocksPerQuarter;  // 32-row parts of the wave block
  float* const lds = reinterpret_cast<float*>(smem + wave * kEpiWaveStride);
  const int bc = 4 * (lane & 31);
  // the lane's four bias values (its columns are the same in every row)
  float bv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (Bw) {
#pragma unroll
    for (int e = 0; e < 4; ++e) bv[e] = load_out<OUT_BF16>(Bw, bc + e);
  }
#pragma unroll
  for (int q = 0; q < kQuarters; ++q) {
#pragma unroll
    for (int ib = 0; ib < kBlocksPerQuarter; ++ib) {
      const int i = q * kBlocksPerQuarter + ib;
#pragma unroll
      for (int r = 0; r < M::R; ++r)
#pragma unroll
        for (int j = 0; j < M::NB; ++j)
          lds[(M::out_row(i, r, lane) - 32 * q) * kEpiRow + M::out_col(j, lane)] = acc[i][j][r];
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    uint16_t* d0 = reinterpret_cast<uint16_t*>(Dw) + static_cast<int64_t>(32 * q + (lane >> 5)) * p.ldd + bc;
    // eight rows pairs at a time: their LDS reads are issued together
#pragma unroll
    for (int t0 = 0; t0 < 16; t0 += 8) {
      f32x4 a[8];
#pragma unroll
      for (int t = 0; t < 8; ++t)
        a[t] = *reinterpret_cast<const f32x4*>(&lds[(2 * (t0 + t) + (lane >> 5)) * kEpiRow + bc]);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        uint32_t h[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float v = p.alpha * a[t][e];
          if (Bw) v += bv[e];
          h[e] = f32_to_bf16_rne(v);
        }
        typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
        const u32x2 w = {h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
        *reinterpret_cast<u32x2*>(d0 + 2 * (t0 + t) * p.ldd) = w;
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads done before the next writes
  }
}

template <typename M>
__device__ __forceinline__ void epilogue_staged(uint8_t* smem, int wave, int lane,
                                                const typename M::Acc (&acc)[M::NB][M::NB],
                                                const GemmParams& p, uint8_t* Dw, const uint8_t* Cw,
                                                const uint8_t* Bw, int rows_left, int cols_left) {
  // the lane's four bias values (its columns are the same in every row)
  const int bc = 4 * (lane & 31);
  f32x4 bb = {0.0f, 0.0f, 0.0f, 0.0f};
  if (Bw) {
    const float* bf = reinterpret_cast<const float*>(Bw);
    if (bc + 4 <= cols_left) {
      bb = *reinterpret_cast<const f32x4*>(bf + bc);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (bc + e < cols_left) bb[e] = bf[bc + e];
    }
    // complete the bias load here, so that no later wait counts it
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  float* lds = reinterpret_cast<float*>(smem + wave * kEpiWaveStride);
  // wave-uniform: the whole 128 x 128 block is inside D
  if (rows_left >= 128 && cols_left >= 128 && p.ldc < (1 << 24)) {
    if (Cw)
      epilogue_staged_c<M>(smem, wave, lane, acc, p, Dw, reinterpret_cast<const float*>(Cw), Bw != nullptr, bb);
    else
      epilogue_staged_full<M>(lds, lane, acc, p, Dw, Bw != nullptr, bb);
    return;
  }
  barrier_only();
  constexpr int kBlocksPerQuarter = 32 / M::BLK;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
#pragma unroll
    for (int ib = 0; ib < kBlocksPerQuarter; ++ib) {
      const int i = q * kBlocksPerQuarter + ib;
#pragma unroll
      for (int r = 0; r < M::R; ++r)
#pragma unroll
        for (int j = 0; j < M::NB; ++j)
          lds[(M::out_row(i, r, lane) - 32 * q) * kEpiRow + M::out_col(j, lane)] = acc[i][j][r];
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    {
      // 32 lanes per row, 4 floats each; two rows per instruction
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const int rr = 2 * t + (lane >> 5), cc = 4 * (lane & 31), row = 32 * q + rr;
        const f32x4 a = *reinterpret_cast<const f32x4*>(&lds[rr * kEpiRow + cc]);
        if (row >= rows_left) continue;
        float* drow = reinterpret_cast<float*>(Dw) + static_cast<int64_t>(row) * p.ldd;
        const float* crow = Cw ? reinterpret_cast<const float*>(Cw) + static_cast<int64_t>(row) * p.ldc : nullptr;
        if (cc + 4 <= cols_left) {
          f32x4 v = a * p.alpha;
          if (crow) {
            const f32x4 c = *reinterpret_cast<const f32x4*>(crow + cc);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = __builtin_fmaf(p.beta, c[e], v[e]);
          }
          if (Bw) v += bb;
          *reinterpret_cast<f32x4*>(drow + cc) = v;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (cc + e < cols_left) {
              float v = p.alpha * a[e];
              if (crow) v = __builtin_fmaf(p.beta, crow[cc + e], v);
              if (Bw) v += bb[e];
              drow[cc + e] = v;
            }
        }
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads done before the next writes
  }
}

// A contiguous copy that a tile of the persistent kernel performs inside its
// K loop, so that moving a shard costs memory operations in the shadow of
// the MFMAs rather than CU time of its own: in steady-state slab kt every
// wave stores the four 1 KiB it loaded in slab kt - 1 and loads chunk kt
// (16 KiB per workgroup per slab), behind the slab's operand DMA.  The
// loads land before the next slab's operand wait, which counts them with
// the DMA loads they follow (vector-memory operations retire in order), and
// the stores of slab kt retire before the wait of slab kt + 1 in the same
// way.  A tile of KT slabs copies at most KT - 2 chunks; the descriptors
// cover exactly the piece's bytes (a multiple of 16), so the last chunk's
// lanes past its end neither read nor write.  Non-temporal (the bytes are
// not reused by this tile), and the stores agent-coherent (sc1: written
// through to where every XCD reads), so publishing the piece needs no L2
// write-back.
struct LoopCopy {
  const uint8_t* src;
  uint8_t* dst;
  uint32_t bytes;
  int chunks;  // 16 KiB chunks; 0: nothing to copy
};
constexpr int kLoopCopyOps = 4;                                    // 1 KiB loads per wave per slab
constexpr int kLoopCopyChunk = kThreads / 64 * kLoopCopyOps * 1024;  // 16 KiB per workgroup per slab
static_assert(kLoopCopyChunk == kLoopCopyBytes, "in-loop copy chunk");
struct NoAfterLoop {
  __device__ __forceinline__ void operator()() const {}
};

// One 256 x 256 tile (tm, tn) of batch l of the GEMM p, computed by the
// whole workgroup with the LDS ring smem.  Every argument is workgroup-uniform.
// kCopy: the tile also performs the copy *lc inside its K loop and calls
// after_loop() (with every wave) once the loop is done.  kHalf: only rows
// 128 hrow .. 128 hrow + 127 of the tile (a half-height tile).
template <int IN, int OUT, bool kCopy = false, bool kHalf = false, typename AfterLoop = NoAfterLoop>
__device__ __forceinline__ void gemm_tile(const GemmParams& p, int l, int tm, int tn, uint8_t* smem,
                                          const LoopCopy* lc = nullptr, const AfterLoop& after_loop = {},
                                          int hrow = 0) {
  using M = std::conditional_t<kHalf, MmaHalf<IN>, Mma<IN>>;
  constexpr int ES = elem_size<IN>();
  constexpr int kRows = kHalf ? kBM / 2 : kBM;  // rows of the tile
  constexpr int kWaveRows = kRows / 2;          // rows of a wave's block

  // the lane index, redefined per tile: in the persistent kernel, nothing
  // derived from it is hoisted out of the tile loop (where it would hold
  // VGPRs across every K loop)
  int lane = threadIdx.x & 63;
  asm volatile("" : "+v"(lane));
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = tm * kBM + (kHalf ? hrow * kRows : 0), n0 = tn * kBN;

  TileCtx c;
  c.Ab = static_cast<const uint8_t*>(p.A) + (l * p.sA + static_cast<int64_t>(m0) * p.lda) * ES;
  c.Bb = static_cast<const uint8_t*>(p.B) + (l * p.sB + static_cast<int64_t>(n0) * p.ldb) * ES;
  const uint32_t lda_b = static_cast<uint32_t>(p.lda * ES);
  const uint32_t ldb_b = static_cast<uint32_t>(p.ldb * ES);
  c.a_bytes = static_cast<uint32_t>(max(0, min(kRows, p.M - m0))) * lda_b;
  c.b_bytes = static_cast<uint32_t>(min(kBN, p.N - n0)) * ldb_b;
  const int kbytes = p.K * ES;
  c.lda16 = 16 * lda_b;
  c.ldb16 = 16 * ldb_b;
  const int KT = (kbytes + kSlab - 1) / kSlab;
  c.kshift = KT * kSlab - kbytes;
  c.rA = make_rsrc(c.Ab, c.a_bytes);
  c.rB = make_rsrc(c.Bb, c.b_bytes);

  // DMA lane mapping.  Wave w fills blocks 8w .. 8w+7 of each operand
  // slab (of an A slab of a half-height tile, blocks 4w .. 4w+3); block b
  // holds rows 8b .. 8b+7, so f(row) depends on b % 2 and on the lane's row
  // within the block, identically for A and B (the K chunk of a row's
  // lanes does not depend on which of the two slabs the row is in).
  const int half = lane >> 5, brow = (lane >> 2) & 7, schunk = lane & 3;
#pragma unroll
  for (int odd = 0; odd < 2; ++odd) {
    const int r16 = 8 * odd + brow;  // the row mod 16 (the wave's first row is a multiple of 16)
    const int gch = half * 4 + (schunk ^ chunk_perm(r16));
    c.ga[odd] = (M::kLoadsA * 8 * wave + r16) * lda_b + gch * 16;  // A block kLoadsA w + odd
    c.gb[odd] = (M::kLoadsB * 8 * wave + r16) * ldb_b + gch * 16;  // B block 8w + odd
    c.gk[odd] = gch * 16;
  }
  c.fillA = wave * M::kLoadsA * 1024;
  c.fillB = wave * M::kLoadsB * 1024;

  // Fragment base offsets within an operand slab: [A even, A odd, B even,
  // B odd].  Rows of every read of a lane agree mod 16 with its base row.
  int fb[4];
#pragma unroll
  for (int odd = 0; odd < 2; ++odd) {
    const int ra = wm * kWaveRows + M::base_row(lane, odd);
    const int rb = wn * 128 + M::base_row(lane, odd);
    const int q = M::base_chunk(lane, odd);
    fb[odd] = (ra >> 3) * 1024 + (ra & 7) * 64 + ((q ^ chunk_perm(ra)) << 4);
    fb[2 + odd] = (rb >> 3) * 1024 + (rb & 7) * 64 + ((q ^ chunk_perm(rb)) << 4);
  }

  typename M::Acc acc[M::NBM][M::NB];
#pragma unroll
  for (int i = 0; i < M::NBM; ++i)
#pragma unroll
    for (int j = 0; j < M::NB; ++j) acc[i][j] = typename M::Acc{};

  typename M::Frags F0, F1;

  // in-loop copy: a chunk's loads (stored one slab later) in cb; the
  // descriptors cover the whole piece, lane offset cvoff within a chunk.
  // Chunk j is loaded at slab j * stride and stored at the next slab, the
  // stride spreading the piece's traffic over the loop.
  u32x4 cb[kLoopCopyOps];
  const uint32_t cvoff = static_cast<uint32_t>(wave) * (kLoopCopyOps * 1024) + static_cast<uint32_t>(lane) * 16;
  const int n_chunks = kCopy ? __builtin_amdgcn_readfirstlane(lc->chunks) : 0;
  const int stride = n_chunks > 0 ? max(1, (KT - 2) / max(n_chunks, 1)) : 1;
  const __amdgpu_buffer_rsrc_t csrc = make_rsrc(kCopy ? lc->src : nullptr, kCopy ? lc->bytes : 0);
  const __amdgpu_buffer_rsrc_t cdst = make_rsrc(kCopy ? lc->dst : nullptr, kCopy ? lc->bytes : 0);
  int ld_j = 0, ld_at = 0;  // the next chunk to load and its slab
  // after MFMA kCopyAt of a second half slab at slab kt: store the chunk
  // loaded at slab kt - 1; after MFMA kCopyAt + kCopyEvery: load the next
  // chunk if this is its slab
  auto copy_ops = [&](int m, int kt_cur, bool loads) {
    if constexpr (kCopy) {
      if (m == M::kCopyAt && ld_j > 0 && kt_cur == ld_at - stride + 1) {
        const uint32_t o = cvoff + static_cast<uint32_t>(ld_j - 1) * kLoopCopyChunk;
#pragma unroll
        for (int op = 0; op < kLoopCopyOps; ++op)
          __builtin_amdgcn_raw_buffer_store_b128(cb[op], cdst, o + op * 1024, 0, 18);  // nt sc1
      }
      if (m == M::kCopyAt + M::kCopyEvery && loads && ld_j < n_chunks && kt_cur == ld_at) {
        const uint32_t o = cvoff + static_cast<uint32_t>(ld_j) * kLoopCopyChunk;
#pragma unroll
        for (int op = 0; op < kLoopCopyOps; ++op) cb[op] = __builtin_amdgcn_raw_buffer_load_b128(csrc, o + op * 1024, 0, 2);
        ++ld_j;
        ld_at += stride;
      }
    }
  };
  const auto none = [](int) {};

  // The ring holds slab kt's lead operand in slot s and its other operand in
  // slot s + 1; the lead operand is loaded three half slabs ahead of its use,
  // the other two.
  constexpr int kTrail = 1 - kLead;
  auto abase = [&](int slab_slot) {
    return smem + (kLead == 0 ? slab_slot : slot_add(slab_slot, 1)) * kOperandSlab;
  };
  auto bbase = [&](int slab_slot) {
    return smem + (kLead == 1 ? slab_slot : slot_add(slab_slot, 1)) * kOperandSlab;
  };

  // Prologue: slabs 0 and 1 into slots 0..3; slab 0 landed; its half 0 read.
  constexpr int kLeadLoads = kLead == 0 ? M::kLoadsA : M::kLoadsB;
  issue_operand<M, kLead, true>(c, smem, 0, 0);
  issue_operand<M, kTrail, true>(c, smem, 0, 1);
  if (KT > 1) {
    issue_operand<M, kLead>(c, smem, 1, 2);
    issue_operand<M, kTrail>(c, smem, 1, 3);
    wait_vmcnt<M::kLoadsA + M::kLoadsB>();
  } else {
    wait_vmcnt<0>();
  }
  barrier_only();
#pragma unroll
  for (int q = 0; q < M::kReads; ++q) M::read(q, abase(0), bbase(0), fb, F0);

  // Main loop, slab kt at ring position s:
  //   half 0: MFMAs on F0 (half 0 of slab kt); read F1 = half 1 of slab kt;
  //           prefetch the lead operand of slab kt+2 into slot s+4 (vacated
  //           by slab kt-1's other operand).
  //   half 1: wait until slab kt+1 has landed (the lead operand of kt+2 may
  //           still be in flight) and F1 is in registers; barrier; MFMAs on
  //           F1; read F0 = half 0 of slab kt+1; prefetch the other operand
  //           of kt+2 into slot s (vacated by slab kt's lead operand).
  // The last two slabs are peeled so the steady-state body has no branches.
  int kt = 0, s = 0;
  for (; kt + 2 < KT; ++kt) {
    wait_lgkmcnt0();
    half_step<M, true, true, kLead>(c, smem, kt + 2, slot_add(s, 4), abase(s) + 512, bbase(s) + 512, fb, F0, F1,
                                     acc, none);
    wait_lgkmcnt0();
    wait_vmcnt<kLeadLoads>();
    barrier_only();
    half_step<M, true, true, kTrail>(c, smem, kt + 2, s, abase(slot_add(s, 2)), bbase(slot_add(s, 2)), fb, F1,
                                      F0, acc, [&](int m) { copy_ops(m, kt, true); });
    s = slot_add(s, 2);
  }
  if (kt + 1 < KT) {  // second to last slab: nothing left to prefetch
    wait_lgkmcnt0();
    half_step<M, false, true, kLead>(c, smem, kt, s, abase(s) + 512, bbase(s) + 512, fb, F0, F1, acc, none);
    wait_lgkmcnt0();
    wait_vmcnt<0>();
    barrier_only();
    half_step<M, false, true, kTrail>(c, smem, kt, s, abase(slot_add(s, 2)), bbase(slot_add(s, 2)), fb, F1, F0,
                                       acc, [&](int m) { copy_ops(m, kt, false); });
    s = slot_add(s, 2);
    ++kt;
  }
  wait_lgkmcnt0();  // last slab
  half_step<M, false, true, kLead>(c, smem, kt, s, abase(s) + 512, bbase(s) + 512, fb, F0, F1, acc, none);
  wait_lgkmcnt0();
  half_step<M, false, false, kTrail>(c, smem, kt, s, smem, smem, fb, F1, F0, acc, none);
  if constexpr (kCopy) after_loop();
  // The MFMAs are opaque to the compiler's hazard tracking: give the last
  // ones their result latency, then redefine every accumulator after that
  // wait, so that no AGPR read of the epilogue can be scheduled above it (a
  // read of a block finished early in the last half slab otherwise may be,
  // and returns the value without that half slab).
  asm volatile("s_nop 7\n s_nop 7\n s_nop 7\n s_nop 7" ::: "memory");
#pragma unroll
  for (int i = 0; i < M::NBM; ++i)
#pragma unroll
    for (int j = 0; j < M::NB; ++j) asm volatile("" : "+a"(acc[i][j]));

  // Epilogue: D = alpha * acc + beta * C (+ bias).  For fp32 output with D
  // (and C, bias) rows 16-byte aligned, each 32-row quarter of the wave's block goes through
  // LDS so that every lane stores 16 contiguous bytes; otherwise element by
  // element.
  constexpr int OES = out_size<OUT>();
  const bool use_c = p.beta != 0.0f;
  const uint8_t* Dl = static_cast<const uint8_t*>(p.D) + l * p.sD * OES;
  const uint8_t* Cl = use_c ? static_cast<const uint8_t*>(p.C) + l * p.sC * OES : nullptr;
  [[maybe_unused]] const uint64_t align = reinterpret_cast<uint64_t>(Dl) | static_cast<uint64_t>(p.ldd * OES) |
                         (use_c ? reinterpret_cast<uint64_t>(Cl) | static_cast<uint64_t>(p.ldc * OES) : 0) |
                         reinterpret_cast<uint64_t>(p.bias);
  const int wrow0 = m0 + wm * kWaveRows, wcol0 = n0 + wn * 128;
  const int rows_left = p.M - wrow0, cols_left = p.N - wcol0;
  uint8_t* Dw = const_cast<uint8_t*>(Dl) + (static_cast<int64_t>(wrow0) * p.ldd + wcol0) * OES;
  const uint8_t* Cw = use_c ? Cl + (static_cast<int64_t>(wrow0) * p.ldc + wcol0) * OES : nullptr;
  const uint8_t* Bw = p.bias ? static_cast<const uint8_t*>(p.bias) + static_cast<int64_t>(wcol0) * OES : nullptr;
  // lane index redefined here, so that the epilogue's per-lane address
  // arithmetic is not hoisted above the main loop (where it would hold VGPRs
  // the fragment buffers need)
  int elane = lane;
  asm volatile("" : "+v"(elane));
  // the condition is uniform over the workgroup (the barrier inside needs that)
  if constexpr (OUT == OUT_E4M3) {
    // e4m3 output: element by element (one byte per value)
  } else if constexpr (OUT == OUT_F32) {
    // (a half-height tile: element by element; no workload here ends in one)
    if constexpr (!kHalf) {
      if ((align & 15) == 0) {
        epilogue_staged<M>(smem, wave, elane, acc, p, Dw, Cw, Bw, rows_left, cols_left);
        return;
      }
    }
  } else {
    if ((align & 7) == 0 && !use_c) {
      barrier_only();  // every wave is done with the operand ring (uniform branch)
      if (rows_left >= kWaveRows && cols_left >= 128) {
        epilogue_staged_bf16<M>(smem, wave, elane, acc, p, Dw, Bw);
        return;
      }
    }
  }
  epilogue_direct<M, OUT>(elane, acc, p, Dw, Cw, Bw, rows_left, cols_left);
}

template <int IN, int OUT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void
gemm_tn_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kSlots * kOperandSlab];
  const int tiles_m = (p.M + kBM - 1) / kBM;
  const int tiles_n = (p.N + kBN - 1) / kBN;
  int tm, tn;
  if (p.tail_cus > 0) {
    // XCD x runs workgroups x, x + 8, .. in order: its item i is tile i of
    // its range, except that the last partial round's tiles come as two
    // half-height items each
    const int T = tiles_m * tiles_n;
    const int x = blockIdx.x % kNumXcd, i = blockIdx.x / kNumXcd;
    const int q = T / kNumXcd, r = T % kNumXcd;
    const int n = q + (x < r ? 1 : 0);
    const int split = half_tail_tiles(n, p.tail_cus), whole = n - split;
    if (i >= whole + 2 * split) return;  // padding of the grid (uniform)
    if (i >= whole) {
      order_tile(x * q + min(x, r) + whole + (i - whole) / 2, tiles_m, tiles_n, tm, tn);
      gemm_tile<IN, OUT, false, true>(p, 0, tm, tn, smem, nullptr, NoAfterLoop{}, (i - whole) & 1);
      return;
    }
    order_tile(x * q + min(x, r) + i, tiles_m, tiles_n, tm, tn);
    gemm_tile<IN, OUT>(p, 0, tm, tn, smem);
    return;
  }
  map_tile(blockIdx.x, tiles_m, tiles_n, tm, tn);
  gemm_tile<IN, OUT>(p, blockIdx.y, tm, tn, smem);
}

template <int IN, int OUT>
inline hipError_t launch_t(GemmParams p, hipStream_t stream) {
  const int tiles_m = (p.M + kBM - 1) / kBM;
  const int tiles_n = (p.N + kBN - 1) / kBN;
  const int T = tiles_m * tiles_n;
  if (p.L != 1) p.tail_cus = 0;
  unsigned gx = static_cast<unsigned>(T);
  if (p.tail_cus > 0) {
    // items of the XCD with the most: the first XCD's
    const int n = T / kNumXcd + (T % kNumXcd ? 1 : 0);
    const int split = half_tail_tiles(n, p.tail_cus);
    const int n_other = T / kNumXcd;
    const int most = std::max(n + split, n_other + half_tail_tiles(n_other, p.tail_cus));
    if (split == 0 && half_tail_tiles(n_other, p.tail_cus) == 0)
      p.tail_cus = 0;  // nothing to split: the plain mapping
    else
      gx = static_cast<unsigned>(most) * kNumXcd;
  }
  const dim3 grid(gx, static_cast<unsigned>(p.L));
  hipLaunchKernelGGL((gemm_tn_kernel<IN, OUT>), grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace tile
}  // namespace dg
