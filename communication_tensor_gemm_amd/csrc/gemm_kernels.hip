// gfx950 (CDNA4) MFMA GEMM with an alpha/beta epilogue: the per-step GEMM of
// the TP schedules (the "any dense GEMM" that the Distributed GEMM
// pull-request page runs at every step, here written for MI355X).
//
// Tiling.  A workgroup of 256 threads (4 wave64s, one per SIMD) owns a
// 256 x 256 tile of D.  The waves form a 2 x 2 grid, each holding a
// 128 x 128 fp32 accumulator as 4 x 4 blocks of 32 x 32 MFMA outputs
// (256 accumulator registers per lane).  Every K tile stages 128 bytes of
// each operand row in LDS, i.e. 32 fp32, 64 bf16 or 128 e4m3 values, so one
// LDS geometry (2 stages x (A 32 KiB + B 32 KiB) = 128 KiB of the 160 KiB)
// serves all three input types and only the MFMA differs:
//   fp32 : v_mfma_f32_32x32x2_f32          (1 value / lane / operand)
//   bf16 : v_mfma_f32_32x32x16_bf16        (8 values)
//   e4m3 : v_mfma_scale_f32_32x32x64_f8f6f4 (32 values, neutral E8M0 scales)
//
// Both operands are K-contiguous ("TN"), which is the layout MFMA fragments
// want: a lane's fragment is 16 contiguous bytes of one row, read with
// ds_read_b128.  Rows are XOR-swizzled in 16-byte units so the 16 lanes of
// one LDS cycle hit distinct banks for both the fragment reads and the
// tile writes.
//
// Global loads are 16-byte buffer loads whose descriptor covers only the
// valid rows of the tile, so rows past M or N read as zero with no branch;
// a K tail past the last 16-byte chunk is redirected out of range the same
// way.  One K tile is loaded into registers while the previous one is
// multiplied from LDS (double buffering, one barrier per K tile).
//
// Workgroup -> tile mapping is XCD-aware: MI355X places workgroup b on XCD
// b mod 8, so each XCD is given one contiguous range of the tile order, and
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
constexpr int kTileBytes = kBM * kRowBytes;  // one operand, one stage
constexpr int kChunksPerThread = kTileBytes / 16 / kThreads;  // 8
constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int kGroupM = 8;
constexpr int kNumXcd = 8;

template <int IN>
struct InT;
template <>
struct InT<IN_F32> {
  static constexpr int kSize = 4;
};
template <>
struct InT<IN_BF16> {
  static constexpr int kSize = 2;
};
template <>
struct InT<IN_E4M3> {
  static constexpr int kSize = 1;
};

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // Raw buffer (stride 0), range check against `bytes`.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

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

// One K tile from LDS: acc[i][j] += A_frag[i] * B_frag[j] for the wave's
// 4 x 4 blocks.  `a_off[i]` / `b_off[j]` are the byte offsets of the lane's
// row in the stage; `key` its swizzle; `h` the lane's K half (lane / 32).
template <int IN>
__device__ __forceinline__ void mma_tile(const uint8_t* sa, const uint8_t* sb, const int* a_off,
                                         const int* b_off, int key, int h, f32x16 (&acc)[4][4]) {
  if constexpr (IN == IN_BF16) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int c = (((2 * g + h) ^ key) << 4);
      bf16x8 a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const bf16x8*>(sa + a_off[i] + c);
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = *reinterpret_cast<const bf16x8*>(sb + b_off[j] + c);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  } else if constexpr (IN == IN_F32) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int c = (((2 * g + h) ^ key) << 4);
      f32x4 a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const f32x4*>(sa + a_off[i] + c);
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = *reinterpret_cast<const f32x4*>(sb + b_off[j] + c);
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i][t], b[j][t], acc[i][j], 0, 0, 0);
    }
  } else {
#pragma unroll
    for (int g2 = 0; g2 < 2; ++g2) {
      // 32 bytes per lane per operand: chunks (4*g2 + h) and (4*g2 + 2 + h).
      const int c0 = (((4 * g2 + h) ^ key) << 4);
      const int c1 = (((4 * g2 + 2 + h) ^ key) << 4);
      i32x8 a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const i32x4 lo = *reinterpret_cast<const i32x4*>(sa + a_off[i] + c0);
        const i32x4 hi = *reinterpret_cast<const i32x4*>(sa + a_off[i] + c1);
        a[i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const i32x4 lo = *reinterpret_cast<const i32x4*>(sb + b_off[j] + c0);
        const i32x4 hi = *reinterpret_cast<const i32x4*>(sb + b_off[j] + c1);
        b[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          // formats 0/0 = e4m3 for A and B; E8M0 scale 127 = 2^0 for both
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], acc[i][j], 0, 0,
                                                                      0, 127, 0, 127);
    }
  }
}

template <int IN, int OUT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void
gemm_tn_kernel(GemmParams p) {
  constexpr int ES = InT<IN>::kSize;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * 2 * kTileBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5;
  const int l = blockIdx.y;

  const int tiles_m = (p.M + kBM - 1) / kBM;
  const int tiles_n = (p.N + kBN - 1) / kBN;
  int tm, tn;
  map_tile(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * kBM, n0 = tn * kBN;

  const uint8_t* Ab =
      static_cast<const uint8_t*>(p.A) + (l * p.sA + static_cast<int64_t>(m0) * p.lda) * ES;
  const uint8_t* Bb =
      static_cast<const uint8_t*>(p.B) + (l * p.sB + static_cast<int64_t>(n0) * p.ldb) * ES;
  const uint32_t lda_b = static_cast<uint32_t>(p.lda * ES);
  const uint32_t ldb_b = static_cast<uint32_t>(p.ldb * ES);
  const uint32_t rows_a = static_cast<uint32_t>(min(kBM, p.M - m0));
  const uint32_t rows_b = static_cast<uint32_t>(min(kBN, p.N - n0));
  const int kbytes = p.K * ES;
  const int KT = (kbytes + kRowBytes - 1) / kRowBytes;

  // Tile load mapping: 8 consecutive threads read one 128-byte row.
  const int lrow = tid >> 3, lcol = tid & 7;
  const uint32_t ga = lrow * lda_b + lcol * 16;
  const uint32_t gb = lrow * ldb_b + lcol * 16;
  const int st_off = lrow * kRowBytes + ((lcol ^ swz(lrow)) << 4);  // + 4096 per chunk i

  // Fragment read mapping.
  const int frow = lane & 31;
  const int key = swz(frow);
  int a_off[4], b_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a_off[i] = (wm * 128 + 32 * i + frow) * kRowBytes;
    b_off[i] = (wn * 128 + 32 * i + frow) * kRowBytes;
  }

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  i32x4 ra[kChunksPerThread], rb[kChunksPerThread];

  auto gload = [&](int kt) {
    const uint32_t k0b = static_cast<uint32_t>(kt) * kRowBytes;
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(Ab + k0b, rows_a * lda_b - k0b);
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(Bb + k0b, rows_b * ldb_b - k0b);
    const bool kval = static_cast<int>(k0b) + lcol * 16 < kbytes;
#pragma unroll
    for (int i = 0; i < kChunksPerThread; ++i) {
      const uint32_t oa = kval ? ga + i * 32 * lda_b : kOutOfRange;
      ra[i] = __builtin_amdgcn_raw_buffer_load_b128(rA, oa, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < kChunksPerThread; ++i) {
      const uint32_t ob = kval ? gb + i * 32 * ldb_b : kOutOfRange;
      rb[i] = __builtin_amdgcn_raw_buffer_load_b128(rB, ob, 0, 0);
    }
  };
  auto lstore = [&](int stage) {
    uint8_t* sa = smem + stage * 2 * kTileBytes;
    uint8_t* sb = sa + kTileBytes;
#pragma unroll
    for (int i = 0; i < kChunksPerThread; ++i)
      *reinterpret_cast<i32x4*>(sa + st_off + i * 32 * kRowBytes) = ra[i];
#pragma unroll
    for (int i = 0; i < kChunksPerThread; ++i)
      *reinterpret_cast<i32x4*>(sb + st_off + i * 32 * kRowBytes) = rb[i];
  };

  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const bool more = kt + 1 < KT;
    if (more) gload(kt + 1);
    const uint8_t* sa = smem + (kt & 1) * 2 * kTileBytes;
    mma_tile<IN>(sa, sa + kTileBytes, a_off, b_off, key, h, acc);
    if (more) lstore((kt + 1) & 1);
    __syncthreads();
  }

  // Epilogue: D = alpha * acc + beta * C.  32 x 32 block layout of an MFMA
  // result: lane holds column (lane % 32) and rows 8*(r/4) + 4*(lane/32) + r%4.
  const int64_t cbase = l * p.sC;
  const int64_t dbase = l * p.sD;
  const bool use_c = p.beta != 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + wn * 128 + 32 * j + frow;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * 128 + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
        if (row < p.M && col < p.N) {
          float v = p.alpha * acc[i][j][r];
          if (use_c) v = __builtin_fmaf(p.beta, load_out<OUT>(p.C, cbase + row * p.ldc + col), v);
          store_out<OUT>(p.D, dbase + row * p.ldd + col, v);
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
