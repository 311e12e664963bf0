// Internal interface between the step scheduler and the gfx950 GEMM kernel.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

// Element type of A/B, and of C/D.
enum InKind { IN_F32 = 0, IN_BF16 = 1, IN_E4M3 = 2 };
enum OutKind { OUT_F32 = 0, OUT_BF16 = 1 };

// One GEMM over an (M x N) block of D, full K:
//   D[i][j] = alpha * sum_k A[i][k] * B[j][k] + beta * C[i][j] (+ bias[j])
// A rows are lda apart, B rows (the N index) ldb apart, both K-contiguous.
// Strides and leading dimensions are in elements of the operand's type.
struct GemmParams {
  const void* A;
  const void* B;
  const void* C;  // read only when beta != 0
  void* D;
  const void* bias;  // NULL, or the block's first column of a bias vector (output type)
  int64_t lda, ldb, ldc, ldd;
  int64_t sA, sB, sC, sD;  // batch strides
  int32_t M, N, K, L;
  float alpha, beta;
};

// Macro tile of one workgroup, and the bytes of one operand row per K tile.
constexpr int kBM = 256;
constexpr int kBN = 256;
constexpr int kRowBytes = 128;

inline int in_elem_size(int in_kind) { return in_kind == IN_F32 ? 4 : (in_kind == IN_BF16 ? 2 : 1); }
inline int out_elem_size(int out_kind) { return out_kind == OUT_F32 ? 4 : 2; }

// ---- Single-launch run: device-side step flags --------------------------
//
// One persistent launch computes every step of a run and performs the shard
// rotation itself.  Its work items are tiles; workgroup b takes them from
// queue b mod nq, in queue order (queue q: its tiles of launch group 0, then
// of group 1, ...), by an atomic counter.  The copy of group h is cut into
// chunks carried by the tiles of group max(0, h - ahead), which copy them
// before their own GEMM; a tile of a staged group waits until every chunk of
// its group's copy is done.  Pointers are not stored: offsets are relative
// to the run's operands.

// One launch group of steps (consecutive steps on adjacent shards, computed
// as one GEMM over their union), pointer-free: its GemmParams without the
// base pointers, and its copy: count consecutive shards, chunks_per_step
// chunks each (shard m of the group at + m * cp_width bytes in both the
// rotating operand and the staging rows); a chunk is chunk_rows rows x
// chunk_cols bytes of the shard region, chunks_per_row pieces per row block.
struct FusedStep {
  int64_t offA, offB, offC, offD;  // bytes from the operand base (A / B / C / D or staging)
  int64_t lda, ldb, ldc, ldd;      // elements
  int64_t sA, sB, sC, sD;          // batch strides, elements
  int64_t offBias;                 // bytes: the group's first column in the bias vector
  int64_t copy_src_off;            // bytes: the group's first shard in the rotating operand
  int64_t copy_dst_off;            // bytes: its staging slot
  int64_t chunk_cols, chunk_rows;
  int32_t chunks_per_row, chunks_per_step;
  int32_t M, N, tiles_m, tiles_n;
  int32_t stagedA, stagedB, stagedC;  // operand read from the staging buffer
  int32_t n_chunks;                   // chunks of the group's copy (0: not staged)
};

// Synchronisation words (int32, one 128-byte line each), zero between runs
// except the error count:
//   [q] queue counters, q < nq;  [kSyncExit] workgroups finished;
//   [kSyncErr] timed-out waits (never reset by a run);
//   [kSyncDone + g] chunks done of launch group g.
constexpr int kSyncStride = 32;
constexpr int kMaxQueues = 8;
constexpr int kSyncExit = kMaxQueues;
constexpr int kSyncErr = kMaxQueues + 1;
constexpr int kSyncDone = kMaxQueues + 2;

struct FusedArgs {
  const void* A;
  const void* B;
  const void* C;           // NULL when beta == 0 (unless it is the rotating operand)
  void* D;
  const void* bias;        // NULL or N values of the output type
  uint8_t* staging;
  const void* copy_src;    // the rotating operand (A, B or C)
  const FusedStep* steps;  // [S] launch groups
  const int32_t* seg;      // [nq][S + 1]: first tile of group g in queue q; [q][S] = tiles
  int32_t* sync;
  int64_t cp_width, cp_height;         // shard region: height rows of cp_width bytes
  int64_t cp_src_pitch, cp_dst_pitch;  // bytes between rows
  int64_t spin_limit;                  // wall-clock ticks a wait may last
  int32_t unit;                        // copy unit: 16, 4 or 1 bytes
  int32_t S, K, L, nq;  // S: number of launch groups
  int32_t ahead;        // copy lookahead D >= 1 (in launch groups)
  float alpha, beta;
};

// Enqueue the single-launch run on `stream` with `grid` workgroups (a
// multiple of nq).
hipError_t launch_fused(int in_kind, int out_kind, const FusedArgs& a, int grid, hipStream_t stream);

// Enqueue one GEMM on `stream`.  The caller has validated the shapes:
// K * elem_size % 16 == 0, 256 * lda * elem_size < 2^31 (same for ldb).
hipError_t launch_gemm(int in_kind, int out_kind, const GemmParams& p, hipStream_t stream);

}  // namespace dg
