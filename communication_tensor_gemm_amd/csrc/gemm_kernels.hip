// gfx950 (CDNA4) MFMA GEMM with an alpha/beta epilogue: the per-step GEMM of
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
// fragment is 16 contiguous bytes of one row (ds_read_b128).  Slabs move
// from global memory straight into LDS with buffer_load_dwordx4 ... lds:
// each wave instruction fills 1 KiB of LDS (lane l -> bytes 16l..16l+15),
// so the LDS layout is chosen by which global chunk each lane fetches.
// Rows are 64 bytes; the four 16-byte chunks of row r are stored XOR-
// permuted by f(r) = ((r>>1) ^ (r>>2)) & 3, which puts the 16 rows that 16
// lanes read in one LDS cycle on distinct banks.  The buffer descriptor of
// each operand covers only the tile's valid rows, so rows past M or N load
// as zeros (out-of-range lanes of an LDS load write zeros), and slabs past K
// are pushed out of range by setting the offset's top bit.
//
// Pipeline.  Four LDS stages of 32 KiB (A and B slabs) form a ring.  Each
// iteration: wait for this wave's fragment reads of slab k and its loads of
// slab k+1, one barrier (every wave now holds slab k in registers, and slab
// k+1 is complete in LDS), issue the loads of slab k+4 into the stage slab
// k just vacated, issue the fragment reads of slab k+1, then run slab k's
// MFMAs.  Loads therefore run four slabs (about 4000 MFMA cycles) ahead,
// and fragment reads one slab ahead of the MFMAs that consume them.
//
// Workgroup -> tile mapping is XCD-aware: MI355X places workgroup b on XCD
// b mod 8, so each XCD gets one contiguous range of the tile order, and
// that order walks groups of 8 tile rows column by column, so the tiles an
// XCD runs together share A rows and B columns in its own L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_launch.h"

namespace dg {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) int i32x4;

constexpr int kThreads = 256;
constexpr int kSlab = 64;                         // bytes of K per operand row per stage
constexpr int kOperandStage = kBM * kSlab;        // 16 KiB
constexpr int kStageBytes = 2 * kOperandStage;    // A + B = 32 KiB
constexpr int kStages = 4;
constexpr int kLoadsPerOperand = kOperandStage / 1024 / 4;  // per wave: 4
constexpr int kLoadsPerSlab = 2 * kLoadsPerOperand;         // per wave: 8
constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int kGroupM = 8;
constexpr int kNumXcd = 8;

static_assert(kBM == 256 && kBN == 256, "tile geometry");

template <int IN>
constexpr int elem_size() {
  return IN == IN_F32 ? 4 : (IN == IN_BF16 ? 2 : 1);
}

__device__ __forceinline__ int chunk_perm(int row) { return ((row >> 1) ^ (row >> 2)) & 3; }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
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
// blocks of BLK x BLK.  A wave reads 16 fragments of 16 bytes per slab,
// 0..7 for A and 8..15 for B.  Fragment r of an operand sits at
//   base[r & 1] + r_stride * (r >> 1)        (base: lane-dependent VGPR)
// so all reads use immediate offsets from at most two base registers.
template <int IN>
struct Mma;

// 16 x 16 shapes (bf16, fp32): read r of an operand covers rows 16r +
// lane%16 of the wave's 128 rows and chunk lane/16.
struct Mma16Base {
  static constexpr int BLK = 16, NB = 8, R = 4;
  typedef f32x4 Acc;
  static constexpr int kPairStride = 2 * 16 * kSlab;  // reads r and r+2 are 32 rows apart
  __device__ static int base_row(int lane, int odd) { return 16 * odd + (lane & 15); }
  __device__ static int base_chunk(int lane, int odd) { return lane >> 4; }
  // MFMA 16 x 16 result: lane holds column lane%16, rows 4*(lane/16) + r
  __device__ static int out_row(int i, int r, int lane) { return 16 * i + 4 * (lane >> 4) + r; }
  __device__ static int out_col(int j, int lane) { return 16 * j + (lane & 15); }
};

template <>
struct Mma<IN_BF16> : Mma16Base {
  __device__ static void mma(const i32x4 (&F)[16], Acc (&acc)[NB][NB]) {
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
  __device__ static void mma(const i32x4 (&F)[16], Acc (&acc)[NB][NB]) {
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
  typedef f32x16 Acc;
  static constexpr int kPairStride = 32 * kSlab;
  __device__ static int base_row(int lane, int odd) { return lane & 31; }
  __device__ static int base_chunk(int lane, int odd) { return 2 * (lane >> 5) + odd; }
  // MFMA 32 x 32 result: lane holds column lane%32, rows 8*(r/4) + 4*(lane/32) + r%4
  __device__ static int out_row(int i, int r, int lane) {
    return 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
  }
  __device__ static int out_col(int j, int lane) { return 32 * j + (lane & 31); }
};

template <>
struct Mma<IN_E4M3> : Mma32Base {
  __device__ static void mma(const i32x4 (&F)[16], Acc (&acc)[NB][NB]) {
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const i32x8 a = __builtin_shufflevector(F[2 * i], F[2 * i + 1], 0, 1, 2, 3, 4, 5, 6, 7);
        const i32x8 b =
            __builtin_shufflevector(F[8 + 2 * j], F[8 + 2 * j + 1], 0, 1, 2, 3, 4, 5, 6, 7);
        // formats 0/0 = e4m3 for A and B; E8M0 scale 127 = 2^0
        acc[i][j] =
            __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[i][j], 0, 0, 0, 127, 0, 127);
      }
  }
};

// Tile-invariant addressing of one workgroup.
struct TileCtx {
  const uint8_t* Ab;
  const uint8_t* Bb;
  uint32_t a_bytes, b_bytes;  // valid rows * row bytes
  uint32_t ga[kLoadsPerOperand], gb[kLoadsPerOperand];  // per-lane global offsets
  uint32_t gk;                // lane's K byte offset within a slab
  int kbytes;
  int fill;                   // wave's LDS fill offset within a stage (uniform)
};

__device__ __forceinline__ void issue_slab(const TileCtx& c, uint8_t* smem, int kt, int stage) {
  const uint32_t k0b = static_cast<uint32_t>(kt) * kSlab;
  const uint32_t kinv = (static_cast<int>(k0b + c.gk) < c.kbytes) ? 0u : kOutOfRange;
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(c.Ab + k0b, c.a_bytes - k0b);
  const __amdgpu_buffer_rsrc_t rB = make_rsrc(c.Bb + k0b, c.b_bytes - k0b);
  uint8_t* sA = smem + stage * kStageBytes + c.fill;
  uint8_t* sB = sA + kOperandStage;
#pragma unroll
  for (int i = 0; i < kLoadsPerOperand; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (lds_ptr_t)(sA + 1024 * i), 16, c.ga[i] | kinv,
                                             0, 0, 0);
#pragma unroll
  for (int i = 0; i < kLoadsPerOperand; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, (lds_ptr_t)(sB + 1024 * i), 16, c.gb[i] | kinv,
                                             0, 0, 0);
}

template <int IN>
__device__ __forceinline__ void read_frags(const uint8_t* stage_base, const int (&fb)[4],
                                           i32x4 (&F)[16]) {
  using M = Mma<IN>;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    F[r] = *reinterpret_cast<const i32x4*>(stage_base + fb[r & 1] + M::kPairStride * (r >> 1));
    F[8 + r] =
        *reinterpret_cast<const i32x4*>(stage_base + fb[2 + (r & 1)] + M::kPairStride * (r >> 1));
  }
}

// Wait until this wave's loads of a slab are complete when `after` more
// slabs were issued behind it.
__device__ __forceinline__ void wait_slab(int after) {
  if (after >= 3) wait_vmcnt<3 * kLoadsPerSlab>();
  else if (after == 2) wait_vmcnt<2 * kLoadsPerSlab>();
  else if (after == 1) wait_vmcnt<kLoadsPerSlab>();
  else wait_vmcnt<0>();
}

// One pipeline step: slab kt's fragments are being read into Fcur; slabs
// kt+1 .. min(KT-1, kt+3) are in flight to LDS.
template <int IN>
__device__ __forceinline__ void pipeline_step(const TileCtx& c, uint8_t* smem, const int (&fb)[4],
                                              int kt, int KT, i32x4 (&Fcur)[16],
                                              i32x4 (&Fnext)[16],
                                              typename Mma<IN>::Acc (&acc)[Mma<IN>::NB][Mma<IN>::NB]) {
  wait_lgkmcnt0();
  if (kt + 1 < KT) wait_slab(min(KT - 1, kt + kStages - 1) - (kt + 1));
  __syncthreads();
  if (kt + kStages < KT) issue_slab(c, smem, kt + kStages, kt % kStages);
  if (kt + 1 < KT) read_frags<IN>(smem + ((kt + 1) % kStages) * kStageBytes, fb, Fnext);
  Mma<IN>::mma(Fcur, acc);
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
  const int KT = (c.kbytes + kSlab - 1) / kSlab;

  // Load mapping: wave instruction i fills LDS rows 16*(4*wave + i) .. +15;
  // lane l writes row +l/4, stored chunk l%4, which holds global chunk
  // (l%4) ^ f(row); f depends on row%16 = l/4 only.
  const int lrow = lane >> 2;
  const int gchunk = (lane & 3) ^ chunk_perm(lrow);
  c.gk = gchunk * 16;
#pragma unroll
  for (int i = 0; i < kLoadsPerOperand; ++i) {
    c.ga[i] = (16 * (4 * wave + i) + lrow) * lda_b + c.gk;
    c.gb[i] = (16 * (4 * wave + i) + lrow) * ldb_b + c.gk;
  }
  c.fill = wave * 4 * 1024;

  // Fragment base offsets within a stage: [A even, A odd, B even, B odd].
  // f(row) depends on row % 16 = lane % 16 for every read of the lane.
  const int perm = chunk_perm(lane & 15);
  int fb[4];
#pragma unroll
  for (int odd = 0; odd < 2; ++odd) {
    const int chunk = (M::base_chunk(lane, odd) ^ perm) << 4;
    fb[odd] = (wm * 128 + M::base_row(lane, odd)) * kSlab + chunk;
    fb[2 + odd] = kOperandStage + (wn * 128 + M::base_row(lane, odd)) * kSlab + chunk;
  }

  typename M::Acc acc[M::NB][M::NB];
#pragma unroll
  for (int i = 0; i < M::NB; ++i)
#pragma unroll
    for (int j = 0; j < M::NB; ++j) acc[i][j] = typename M::Acc{};

  i32x4 F0[16], F1[16];

  // Prologue: slabs 0..3 in flight, slab 0's fragments requested.
  for (int t = 0; t < kStages && t < KT; ++t) issue_slab(c, smem, t, t);
  wait_slab(min(KT - 1, kStages - 1));
  __syncthreads();
  read_frags<IN>(smem, fb, F0);

  for (int kt = 0; kt < KT; kt += 2) {
    pipeline_step<IN>(c, smem, fb, kt, KT, F0, F1, acc);
    if (kt + 1 < KT) pipeline_step<IN>(c, smem, fb, kt + 1, KT, F1, F0, acc);
  }

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
hipError_t launch_t(const GemmParams& p, hipStream_t stream) {
  const int tiles_m = (p.M + kBM - 1) / kBM;
  const int tiles_n = (p.N + kBN - 1) / kBN;
  const dim3 grid(static_cast<unsigned>(tiles_m) * static_cast<unsigned>(tiles_n),
                  static_cast<unsigned>(p.L));
  hipLaunchKernelGGL((gemm_tn_kernel<IN, OUT>), grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(int in_kind, int out_kind, const GemmParams& p, hipStream_t stream) {
  if (p.M <= 0 || p.N <= 0 || p.L <= 0) return hipSuccess;
  if (in_kind == IN_F32 && out_kind == OUT_F32) return launch_t<IN_F32, OUT_F32>(p, stream);
  if (in_kind == IN_BF16 && out_kind == OUT_F32) return launch_t<IN_BF16, OUT_F32>(p, stream);
  if (in_kind == IN_BF16 && out_kind == OUT_BF16) return launch_t<IN_BF16, OUT_BF16>(p, stream);
  if (in_kind == IN_E4M3 && out_kind == OUT_BF16) return launch_t<IN_E4M3, OUT_BF16>(p, stream);
  if (in_kind == IN_E4M3 && out_kind == OUT_F32) return launch_t<IN_E4M3, OUT_F32>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace dg
