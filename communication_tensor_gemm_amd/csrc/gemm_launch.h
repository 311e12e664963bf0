// Internal interface between the step scheduler and the gfx950 GEMM kernel.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

// Element type of A/B, and of C/D.
enum InKind { IN_F32 = 0, IN_BF16 = 1, IN_E4M3 = 2 };
enum OutKind { OUT_F32 = 0, OUT_BF16 = 1, OUT_E4M3 = 2 };

// One GEMM over an (M x N) block of D, full K:
//   D[i][j] = alpha * sum_k A[i][k] * B[j][k] + beta * C[i][j] (+ bias[j])
// (with an e4m3 output, the sum times `post` before the cast)
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
  float post;  // e4m3 output: the result scale, applied before the cast
  // 0: whole tiles only.  Otherwise the CUs of one XCD: the workgroups of an
  // XCD's last round of tiles, when that round fills at most half of them,
  // each compute half a tile (128 x 256), so the round takes about half as
  // long (L = 1 only).
  int32_t tail_cus;
};

// Tiles of a last partial round that run as two half-height tiles each:
// n tiles over `slots` concurrent workgroups.
__host__ __device__ inline int half_tail_tiles(int n, int slots) {
  if (slots <= 0) return 0;
  const int rem = n % slots;
  return (rem > 0 && 2 * rem <= slots) ? rem : 0;
}

// Macro tile of one workgroup, and the bytes of one operand row per K tile.
constexpr int kBM = 256;
constexpr int kBN = 256;
constexpr int kRowBytes = 128;
// XCDs of the chip: workgroup b of a launch runs on XCD b mod 8.
constexpr int kNumXcd = 8;
// Bytes a workgroup of the persistent kernel copies per K slab inside its K
// loop (four waves, four 1 KiB loads each); a tile of KT slabs copies at
// most KT - 2 such chunks.
constexpr int kLoopCopyBytes = 16384;

inline int in_elem_size(int in_kind) { return in_kind == IN_F32 ? 4 : (in_kind == IN_BF16 ? 2 : 1); }
inline int out_elem_size(int out_kind) { return out_kind == OUT_F32 ? 4 : (out_kind == OUT_BF16 ? 2 : 1); }

// ---- Single-launch run: device-side strip readiness -----------------------
//
// One persistent launch computes every step of a run on the monolithic tile
// grid and performs the shard rotation itself.  The rotating operand (A, B
// or the partial C) is gathered into an image G with the operand's own
// layout; a tile that reads a staged shard reads G.  Readiness is kept per
// strip: the 256 rows (row schedules) or 256 columns (column schedules) of
// the rotating operand that one tile row / column reads.  A strip's step is
// the latest step (in rotation order) of the shards it overlaps; the strips
// of step 0 lie inside the local shard and are read in place.
//
// Work items are the tiles.  Workgroup b takes them from queue b mod nq, in
// queue order, by an atomic counter; the queue order is by segment (step 0,
// then groups of consecutive staged steps), each segment's tiles split into
// nq contiguous ranges of its tile order.  The copies are pieces of the
// staged strips, numbered in step order (steps 1 .. S-1, then step 0, whose
// strips are copied only when the gathered image is returned) and handed out
// by two atomic claim counters over two consecutive ranges of that order:
// list 0, the steps the launch's first round of tiles reads, and list 1, the
// later steps.  A tile of a staged strip claims and copies pieces (list 0,
// then list 1) while its strip is incomplete; a tile that starts its GEMM
// claims one piece of list 1 and copies it inside its K loop; in the quota
// form (no in-loop copy), list 1 is empty and the tiles of the first
// segments claim a quota of list 0 before their GEMM.  Pointers are not
// stored in the tables; per-run pointers travel in FusedArgs.

// One queue segment: consecutive steps whose tiles are ordered together.
struct FusedSeg {
  int32_t strip0, nst;  // its strips: positions strip0 .. strip0 + nst - 1
  int32_t tiles;        // tiles of one batch: nst * other_tiles
  int32_t quota;        // pieces each of its tiles claims before its GEMM (0: none)
};

// The copy of one step: its strips and their pieces.
struct FusedStepCopy {
  int64_t piece;        // bytes (row strips) or rows (column strips) per piece
  int32_t strip0, nst;  // its strips: positions in the strip list
  int32_t P;            // pieces per strip (the target of each strip's counter)
  int32_t n_chunks;     // nst * LG * P (its pieces)
  int32_t wait;         // its tiles wait for their strip and read the gathered image
  int32_t base;         // index of its first piece in the claim order
};

// Synchronisation words (int32, one 128-byte line each), zero between runs
// except the error count:
//   [q] queue counters, q < nq;  [kSyncExit] workgroups finished;
//   [kSyncErr] timed-out waits (never reset by a run);
//   [kSyncClaim + i] pieces claimed from list i.
constexpr int kSyncStride = 32;
constexpr int kMaxQueues = 8;
constexpr int kSyncExit = kMaxQueues;
constexpr int kSyncErr = kMaxQueues + 1;
constexpr int kSyncClaim = kMaxQueues + 2;
__host__ __device__ inline int sync_words(int /*S*/) { return (kSyncClaim + 2) * kSyncStride; }

// Device timeline of one run (unsigned 64-bit wall-clock ticks), written
// with atomic max only: [0] = ~(first workgroup start); per step s,
// [1 + 3s] = last piece of the step's copy counted, [2 + 3s] = ~(first
// tile of the step begins), [3 + 3s] = last tile of the step ends.  Zero
// at the start of the run (the previous launch zeroes it at its end).
__host__ __device__ inline int timeline_words(int S) { return 1 + 3 * S; }

struct FusedArgs {
  GemmParams g;                  // the whole problem on the monolithic tile grid
  const uint8_t* gath;           // G: the gathered image of the rotating operand
  const uint8_t* src;            // the rotating operand (source of the copies)
  const FusedSeg* segs;          // [n_seg]
  const FusedStepCopy* steps;    // [S]
  const int32_t* strip_list;     // strips, step by step
  const int32_t* strip_step;     // step of each strip-list position
  const int32_t* claim_steps;    // the steps in claim order
  const int32_t* seg;            // [nq][n_seg + 1]: first item of segment g in queue q
  int32_t* sync;
  uint32_t* ctr;                 // [LG][n_strips] pieces done per strip, then [LG][S] per
                                 // step; zero between runs
  uint64_t* times;               // NULL, or this run's timeline (zero at the start)
  uint64_t* times_next;          // NULL, or the next run's timeline, zeroed at the end
  int64_t row_bytes;             // contiguous strips: bytes per row of the operand; strided: element bytes
  int64_t ext;                   // rows or columns of the operand along the strip dimension
  int64_t gbatch;                // bytes between batches of the operand and of G
  int64_t pitch;                 // strided strips: bytes between rows
  int64_t height;                // strided strips: rows per batch
  int64_t spin_limit;            // wall-clock ticks a wait may last
  int64_t delay;                 // ticks a workgroup waits before its first copy (0: none)
  int32_t rot;                   // rotating operand: 0 A, 1 B, 2 C
  int32_t cols;                  // 1: strips are tile columns
  int32_t strided;               // 1: a strip is 256 columns of every row (else contiguous rows)
  int32_t n_strips;              // strips per batch
  int32_t LG;                    // batches of G (1 when A is shared)
  int32_t unit;                  // copy unit: 16, 4 or 1 bytes
  int32_t n_seg, nq, S;
  int32_t copy_on;               // 0: nothing rotates (a reduce-scatter with beta = 0)
  int32_t list_begin[2];         // claim lists this run: pieces [begin, end) of the claim order
  int32_t list_end[2];           // (step 0's pieces close the last list when G is returned)
  int32_t loop_copy;             // 1: starting tiles copy a list-1 piece in their K loop
  int32_t half_tail;             // 1: a queue's last partial round of tiles, when it fills at
                                 // most half of the queue's workgroups, runs as half-height tiles
};

// Enqueue the single-launch run on `stream` with `grid` workgroups (a
// multiple of nq).
hipError_t launch_fused(int in_kind, int out_kind, const FusedArgs& a, int grid, hipStream_t stream);

// Enqueue one GEMM on `stream`.  The caller has validated the shapes:
// K * elem_size % 16 == 0, 256 * lda * elem_size < 2^31 (same for ldb).
hipError_t launch_gemm(int in_kind, int out_kind, const GemmParams& p, hipStream_t stream);

}  // namespace dg
