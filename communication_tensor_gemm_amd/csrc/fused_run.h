// fused_run.h -- the whole TP-step schedule of one run as a single persistent
// launch on gfx950: the workgroups perform the shard rotation (copy chunks)
// and every tile of the problem's monolithic 256 x 256 tile grid, and a tile
// that reads a staged shard starts only once the part of the gathered
// operand it reads is complete.
//
// This is the per-step readiness of the Distributed GEMM pull-request page
// (each step's GEMM waits, at its start, for the operand its peer sent;
// described there as a few barriers at the beginning of every GEMM kernel),
// made tile-granular as in the TransformerEngine issue on overlapping
// tensor-parallel collectives with matmuls (a GEMM that reports finished
// tiles through atomic switches): one counter per strip -- the 256 rows (or
// columns) of the rotating operand that one tile row (or column) reads --
// raised once per finished copy piece, so a tile waits only for the rows it
// reads.  The copy is done by the CUs because the SDMA engines slow
// several-fold under the GEMM's memory traffic on this part.
//
// Tiles.  The launch computes the monolithic tile grid.  The rotating
// operand (A, B, or the partial C) is gathered into an image G with the
// operand's own layout; a strip's step is the latest step, in rotation
// order, of the shards it overlaps.  Strips of step 0 lie inside the local
// shard and are read in place; every other strip is copied whole into G
// (the local-shard rows of a strip that straddles a shard boundary too) and
// read from there.  Every output element is computed by the same tile code
// with the same K order as the monolithic GEMM, so the result is bitwise the
// monolithic one.
//
// Work distribution.  Workgroup b takes tiles from queue b mod nq (nq = 8:
// MI355X places workgroup b on XCD b mod 8, so every XCD runs one
// contiguous range of each segment's tile order, walked in groups of four
// strips; nq = 1: one queue for the chip), in queue order, by an atomic
// counter: queue q lists its tiles of segment 0 (step 0), then of segment
// 1 (the next steps), and so on; when the queue's last round of tiles
// would fill at most half of its workgroups, those tiles come as two
// half-height items each.
//
// Copies.  The staged strips are cut into pieces, numbered in step order
// (steps 1 .. S-1, then the local step when the gathered image is
// returned), and handed out by two atomic claim counters over consecutive
// ranges of that order: list 0 holds the steps that tiles of the launch's
// first round read, list 1 the later steps.  List 0 goes first, in small
// pieces copied through LDS by the workgroups of the first round: a tile of
// a staged strip that is not yet complete claims pieces one at a time while
// it waits (list 0, then, for a strip of list 1, list 1) instead of
// spinning, and the tiles of the first COPY_AHEAD segments (default none;
// those read the local shard) first claim a quota before their GEMM.  A
// tile that starts its GEMM claims one piece of list 1 and copies it inside
// its K loop, where the copy's loads and stores ride in the shadow of the
// MFMAs; list-1 pieces are sized so that the tiles starting before a
// step's segment carry all of its pieces.  (Where a piece cannot be copied
// inside the loop -- column strips, unaligned rows, too few slabs -- list 1
// is empty and list 0 holds every staged step.)  Workgroups whose queue is
// empty claim whatever is left.
//
// Progress.  A workgroup copies what it claims before it waits on
// anything (an in-loop piece is claimed only once the tile's own wait is
// over), and a workgroup waiting for a strip claims from the strip's list
// while pieces are left; once none are left, every piece of that list is
// held by a running workgroup that finishes it without waiting.  So every
// wait ends, given that every queue keeps at least one running workgroup
// (the host orders single-launch runs on a device one after another).
// Should a wait nevertheless outlast its limit (another kernel holding CUs,
// say), the workgroup copies its strip itself -- the same bytes the
// claimers write, so the duplicate is harmless, and the strip's region of G
// is read by no tile that has already finished -- counts the event, and
// goes on with a correct result.
//
// Visibility.  The LDS copy and the in-loop copy store with agent scope
// (written through to where every XCD reads); every wave of a claimer waits
// until its stores are complete, and after a barrier thread 0 adds the
// pieces to their strips' counters.  (The register copy loop, used for
// column strips and units under 16 bytes, stores normally: thread 0 then
// releases at agent scope first, an L2 write-back without the invalidate
// that would cost every tile on the XCD its cached operand lines.)  A
// waiting thread polls the counter with agent-scope loads and then performs
// an agent-scope acquire (cache invalidate) before the barrier that releases
// its workgroup into the tile.  Every piece also counts towards its step,
// so to keep acquires rare thread 0 reads, after its strip, the step's
// count once: when the whole step is complete (the usual case, the copies
// run ahead), the acquire covers every strip of the step and later tiles of
// the step wait no more; otherwise only the strip is remembered.  The
// counts are added without waiting for the atomics' return.  All counters
// are reset by the last workgroup to finish, so every launch starts from
// zero (also when replayed from a graph).
#pragma once
#include "gemm_tile.h"

namespace dg {
namespace tile {

// Copy `rows` rows of `bytes` bytes (a multiple of sizeof(T)) from src to dst,
// rows spitch / dpitch bytes apart, with the workgroup's 256 threads: batches
// of eight units per thread, all eight loads in flight before the stores (the
// last batch predicated, so a ragged end costs one memory round trip, not
// one per unit).  Non-temporal: the copied bytes are not reused by this
// workgroup, and they should not evict the GEMM's operand lines.
template <typename T>
__device__ __forceinline__ void copy_rows(const uint8_t* src, int64_t spitch, uint8_t* dst,
                                          int64_t dpitch, int64_t rows, int64_t bytes) {
  constexpr int U = 8;
  const int tid = threadIdx.x;
  const int64_t upr = bytes / static_cast<int64_t>(sizeof(T));
  if (rows == 1) {
    const T* s = reinterpret_cast<const T*>(src);
    T* d = reinterpret_cast<T*>(dst);
    for (int64_t u = tid; u < upr; u += U * kThreads) {
      T v[U];
#pragma unroll
      for (int j = 0; j < U; ++j)
        if (u + j * kThreads < upr) v[j] = __builtin_nontemporal_load(s + u + j * kThreads);
#pragma unroll
      for (int j = 0; j < U; ++j)
        if (u + j * kThreads < upr) __builtin_nontemporal_store(v[j], d + u + j * kThreads);
    }
    return;
  }
  // several rows: one flat index over rows x units (a piece holds < 2^32 units)
  const uint32_t total = static_cast<uint32_t>(rows * upr);
  const uint32_t up = static_cast<uint32_t>(upr);
  for (uint32_t f = tid; f < total; f += U * kThreads) {
    T v[U];
    int64_t dof[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const uint32_t idx = f + j * kThreads;
      const uint32_t r = idx / up, c = idx - r * up;
      dof[j] = r * dpitch + static_cast<int64_t>(c) * sizeof(T);
      if (idx < total)
        v[j] = __builtin_nontemporal_load(
            reinterpret_cast<const T*>(src + r * spitch + static_cast<int64_t>(c) * sizeof(T)));
    }
#pragma unroll
    for (int j = 0; j < U; ++j)
      if (f + j * kThreads < total) __builtin_nontemporal_store(v[j], reinterpret_cast<T*>(dst + dof[j]));
  }
}

// Contiguous copy of `bytes` (a multiple of 16) from src to dst through the
// workgroup's LDS, which is idle between tiles: each wave streams rounds of
// 32 KiB straight into its own 32 KiB of LDS (buffer_load ... lds, 32
// loads of 1 KiB in flight, no registers held while they fly), waits for
// them, reads them back and stores them.  128 KiB per workgroup in flight:
// the register-bounded loop above keeps 32 KiB, and at HBM latency that
// bounds one CU's copy rate.  The buffer descriptors cover `bytes`: loads
// past the end read zeros and stores past it are dropped.  The stores are
// non-temporal and agent-coherent (cache policy nt sc1: written through to
// where every XCD reads), so a release needs no L2 write-back for them.
// The caller passes a barrier before the LDS is used for anything else.
constexpr int kStoreAgentNT = 18;  // buffer store cache policy: sc1 (agent scope) | nt
constexpr int kCopyWaveBytes = 32768;
__device__ __forceinline__ void copy_lds(const uint8_t* src, uint8_t* dst, int64_t bytes, uint8_t* smem) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  uint8_t* const lbase = smem + wave * kCopyWaveBytes;
  const __amdgpu_buffer_rsrc_t r = make_rsrc(src, static_cast<uint32_t>(bytes));
  const __amdgpu_buffer_rsrc_t w = make_rsrc(dst, static_cast<uint32_t>(bytes));
  for (int64_t b0 = 0; b0 < bytes; b0 += 4 * kCopyWaveBytes) {
    const uint32_t wo = static_cast<uint32_t>(b0) + wave * kCopyWaveBytes + lane * 16;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the last round's reads are done
#pragma unroll
    for (int d = 0; d < kCopyWaveBytes / 1024; ++d)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(lbase + 1024 * d), 16, wo + 1024 * d, 0, 0, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int d0 = 0; d0 < kCopyWaveBytes / 1024; d0 += 8) {
      u32x4 v[8];
#pragma unroll
      for (int d = 0; d < 8; ++d)
        v[d] = *reinterpret_cast<const u32x4*>(lbase + 1024 * (d0 + d) + 16 * lane);
#pragma unroll
      for (int d = 0; d < 8; ++d)
        __builtin_amdgcn_raw_buffer_store_b128(v[d], w, wo + 1024 * (d0 + d), 0, kStoreAgentNT);
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// Where chunk c of step h lies: strip-list position, batch of G and piece.
struct ChunkAt {
  int pos, lg, piece;
};
__device__ __forceinline__ ChunkAt chunk_at(const FusedArgs& a, const FusedStepCopy& sh, int c) {
  const int per_strip = a.LG * sh.P;
  ChunkAt at;
  const int sp = c / per_strip;
  const int rem = c - sp * per_strip;
  at.pos = sh.strip0 + sp;
  at.lg = rem / sh.P;
  at.piece = rem - at.lg * sh.P;
  return at;
}

// Copy one piece of strip `strip` of batch lg from the operand into G.
// Contiguous strips are 256 rows of the operand's storage (A, the N x K
// storage of B, or C for row chunks); a piece is `piece` bytes of one.
// Strided strips (C's column chunks) are 256 columns of every row; a piece
// is `piece` rows of one.  Pieces past the end of a ragged last strip are
// empty.
__device__ __forceinline__ void copy_piece(const FusedArgs& a, int64_t piece, int strip, int lg, int pc,
                                           uint8_t* smem) {
  const uint8_t* src;
  uint8_t* dst;
  int64_t rows, bytes, pitch;
  const int64_t batch = static_cast<int64_t>(lg) * a.gbatch;
  if (!a.strided) {
    const int64_t r0 = static_cast<int64_t>(strip) * kBM;
    const int64_t r1 = min(r0 + kBM, a.ext);
    const int64_t off = r0 * a.row_bytes + static_cast<int64_t>(pc) * piece;
    const int64_t end = r1 * a.row_bytes;
    if (off >= end) return;
    bytes = min(piece, end - off);
    rows = 1;
    pitch = 0;
    src = a.src + batch + off;
    dst = const_cast<uint8_t*>(a.gath) + batch + off;
    if (a.unit == 16) {
      copy_lds(src, dst, bytes, smem);
      return;
    }
  } else {
    const int64_t c0 = static_cast<int64_t>(strip) * kBN;
    const int64_t c1 = min(c0 + kBN, a.ext);
    const int64_t rw0 = static_cast<int64_t>(pc) * piece;
    if (rw0 >= a.height) return;
    rows = min(piece, a.height - rw0);
    bytes = (c1 - c0) * a.row_bytes;
    pitch = a.pitch;
    const int64_t off = batch + rw0 * a.pitch + c0 * a.row_bytes;
    src = a.src + off;
    dst = const_cast<uint8_t*>(a.gath) + off;
  }
  if (a.unit == 16)
    copy_rows<u32x4>(src, pitch, dst, pitch, rows, bytes);
  else if (a.unit == 4)
    copy_rows<uint32_t>(src, pitch, dst, pitch, rows, bytes);
  else
    copy_rows<uint8_t>(src, pitch, dst, pitch, rows, bytes);
}

__device__ __forceinline__ uint32_t* strip_counter(const FusedArgs& a, int lg, int strip) {
  return a.ctr + static_cast<int64_t>(lg) * a.n_strips + strip;
}
// pieces done of step h in batch lg (after the strip counters)
__device__ __forceinline__ uint32_t* step_counter(const FusedArgs& a, int lg, int h) {
  return a.ctr + static_cast<int64_t>(a.LG) * a.n_strips + static_cast<int64_t>(lg) * a.S + h;
}

// Release at agent scope: write back this XCD's L2 so that the stores made
// before it are visible to every XCD.  (A full __threadfence() would also
// invalidate the L2, throwing away the operand lines every tile on the XCD
// is reusing.)
__device__ __forceinline__ void release_agent() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent"); }

// Thread 0: the finished chunks of this workgroup are in L2 (every wave
// waited for its stores and passed a barrier): count them, towards their
// strip and their step (no atomic's return is waited for).
__device__ __forceinline__ void count_chunk(const FusedArgs& a, int h, int c) {
  const FusedStepCopy& sh = a.steps[h];
  const ChunkAt at = chunk_at(a, sh, c);
  const int strip = a.strip_list[at.pos];
  __hip_atomic_fetch_add(strip_counter(a, at.lg, strip), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_fetch_add(step_counter(a, at.lg, h), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // the step's copy time: the latest stamp of any of its pieces
  if (a.times)
    __hip_atomic_fetch_max(a.times + 1 + 3 * h, wall_clock64(), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The step whose pieces [base, base + n_chunks) of the claim order hold
// piece p (claim_steps lists the steps in that order).
__device__ __forceinline__ int piece_step(const FusedArgs& a, int p) {
  int k = 0;
  while (p >= a.steps[a.claim_steps[k]].base + a.steps[a.claim_steps[k]].n_chunks) ++k;
  return a.claim_steps[k];
}

// Copy pieces [p0, p1) of the claim order with the whole workgroup, then
// (thread 0) count them.  The first copy of a workgroup waits for the delay
// test hook.
__device__ __forceinline__ void copy_claimed(const FusedArgs& a, int p0, int p1, uint8_t* smem,
                                             bool& delayed, uint64_t t_start) {
  if (!delayed) {
    if (threadIdx.x == 0)
      while (wall_clock64() - t_start < static_cast<uint64_t>(a.delay)) __builtin_amdgcn_s_sleep(8);
    delayed = true;
    barrier_only();
  }
  int k = 0;
  for (int p = p0; p < p1; ++p) {
    while (p >= a.steps[a.claim_steps[k]].base + a.steps[a.claim_steps[k]].n_chunks) ++k;
    const FusedStepCopy& sh = a.steps[a.claim_steps[k]];
    const ChunkAt at = chunk_at(a, sh, p - sh.base);
    copy_piece(a, sh.piece, a.strip_list[at.pos], at.lg, at.piece, smem);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's stores are complete
  barrier_only();
  if (threadIdx.x == 0) {
    // pieces copied by the register loop (column strips, units under 16
    // bytes) sit in L2: write them back before they are counted
    if (a.unit != 16 || a.strided) release_agent();
    k = 0;
    for (int p = p0; p < p1; ++p) {
      while (p >= a.steps[a.claim_steps[k]].base + a.steps[a.claim_steps[k]].n_chunks) ++k;
      const int h = a.claim_steps[k];
      count_chunk(a, h, p - a.steps[h].base);
    }
  }
}

template <int IN, int OUT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void
fused_run_kernel(FusedArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kSlots * kOperandSlab];
  // broadcast words: at the end of the last ring slot, which a tile first
  // fills only after its prologue barrier (by then every wave has read them)
  // and which the epilogue leaves alone
  volatile int32_t* bcast = reinterpret_cast<volatile int32_t*>(smem + kSlots * kOperandSlab - 256);
  const int tid = threadIdx.x;
  const int q = static_cast<int>(blockIdx.x) % a.nq;
  int32_t* const qctr = a.sync + q * kSyncStride;
  int32_t* const nexit = a.sync + kSyncExit * kSyncStride;
  int32_t* const nerr = a.sync + kSyncErr * kSyncStride;
  int32_t* const claim0 = a.sync + kSyncClaim * kSyncStride;
  int32_t* const claim1 = a.sync + (kSyncClaim + 1) * kSyncStride;
  const int32_t* const seg = a.seg + q * (a.n_seg + 1);
  // the queue's items: its tiles, except that the tiles of a last round
  // that fills at most half of the queue's workgroups come as two
  // half-height items each (consecutive, so a tile's halves wait alike)
  const int n_tiles = seg[a.n_seg];
  const int split = a.half_tail ? half_tail_tiles(n_tiles, static_cast<int>(gridDim.x) / a.nq) : 0;
  const int whole = n_tiles - split, n_items = n_tiles + split;
  const uint64_t t_start = wall_clock64();
  if (a.times && tid == 0)
    __hip_atomic_fetch_max(a.times, ~t_start, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // thread 0, for batch acq_l: the steps (bit h, h < 64) and the strips of
  // segment acq_g (bit p: segment position p < 64) seen complete before an
  // acquire
  int acq_g = -1, acq_l = -1;
  uint64_t acq_steps = 0, acq_strips = 0;
  bool delayed = a.delay == 0;
  // lists whose pieces are all handed out (uniform)
  bool done0 = !a.copy_on || a.list_begin[0] >= a.list_end[0];
  bool done1 = !a.copy_on || a.list_begin[1] >= a.list_end[1];
  int g = 0;  // segment of the last tile (tiles come in increasing order)
  for (;;) {
    barrier_only();  // every wave is done with the previous tile and its broadcast words
    if (tid == 0) bcast[0] = __hip_atomic_fetch_add(qctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    barrier_only();
    const int item = __builtin_amdgcn_readfirstlane(bcast[0]);
    if (item >= n_items) break;
    const int k = item < whole ? item : whole + (item - whole) / 2;  // the queue's tile
    const int hrow = item < whole ? -1 : (item - whole) & 1;           // half of a half-height item
    while (k >= seg[g + 1]) ++g;
    const FusedSeg& sg = a.segs[g];
    // the tile: position i of this queue's share of segment g
    const int i = k - seg[g];
    const int T2 = sg.tiles;
    const int qq = T2 / a.nq, r = T2 - qq * a.nq;
    const int share = qq + (q < r ? 1 : 0), first = q * qq + min(q, r);
    const int l = i / share, j = i - l * share;
    // the segment's tile order: groups of four tile rows walked column by
    // column, as the monolithic kernel walks (row strips: the rows are the
    // strips; column strips: the strips are the columns)
    int sp, ob;
    if (a.cols)
      order_tile(first + j, T2 / sg.nst, sg.nst, ob, sp);
    else
      order_tile(first + j, sg.nst, T2 / sg.nst, sp, ob);
    const int pos = sg.strip0 + sp;
    const int strip = a.strip_list[pos];
    const int h_own = a.strip_step[pos];
    const FusedStepCopy& own = a.steps[h_own];
    const bool wait = a.copy_on && own.wait;
    const int lg = a.LG == 1 ? 0 : l;

    // 1. the tiles of the first segments claim a quota of pieces before their
    //    GEMM (the claim list is in step order, so the first claims copy the
    //    first staged step)
    if (sg.quota > 0 && !done0) {
      if (tid == 0) bcast[1] = __hip_atomic_fetch_add(claim0, sg.quota, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      barrier_only();
      const int p0 = a.list_begin[0] + __builtin_amdgcn_readfirstlane(bcast[1]);
      if (p0 >= a.list_end[0]) {
        done0 = true;
      } else {
        copy_claimed(a, p0, min(p0 + sg.quota, a.list_end[0]), smem, delayed, t_start);
        if (p0 + sg.quota >= a.list_end[0]) done0 = true;
      }
    }

    // 2. a tile of a staged strip waits until the strip is complete; while it
    //    is not and pieces are left, the workgroup claims and copies them one
    //    at a time (a claimer copies before it waits on anything, so every
    //    wait ends)
    if (wait) {
      for (;;) {
        barrier_only();  // the broadcast words are free
        if (tid == 0) {
          // 0: go on; 1: copy claimed piece bcast[1]; 2: the wait ran out
          int state = 0;
          if (acq_l != lg) {
            acq_l = lg;
            acq_steps = 0;
            acq_g = -1;
          }
          if (acq_g != g) {
            acq_g = g;
            acq_strips = 0;
          }
          const bool known = (h_own < 64 && ((acq_steps >> h_own) & 1)) || (sp < 64 && ((acq_strips >> sp) & 1));
          if (!known) {
            const uint32_t P = static_cast<uint32_t>(own.P);
            uint32_t* const ctr = strip_counter(a, lg, strip);
            bool ready = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= P;
            if (!ready && !done0) {
              const int pc = a.list_begin[0] +
                             __hip_atomic_fetch_add(claim0, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              if (pc < a.list_end[0]) {
                state = 1;
                bcast[1] = pc;
              }
              if (pc + 1 >= a.list_end[0]) done0 = true;
            }
            // list 1 only for a strip of list 1: a tile of the first round waits
            // for list 0 alone, and a big in-loop piece would hold it back
            if (!ready && state == 0 && !done1 && own.base >= a.list_begin[1]) {
              const int pc = a.list_begin[1] +
                             __hip_atomic_fetch_add(claim1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              if (pc < a.list_end[1]) {
                state = 1;
                bcast[1] = pc;
              }
              if (pc + 1 >= a.list_end[1]) done1 = true;
            }
            if (state == 0 && !ready) {
              const uint64_t t0 = wall_clock64();
              while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < P) {
                if (wall_clock64() - t0 > static_cast<uint64_t>(a.spin_limit)) {
                  __hip_atomic_fetch_add(nerr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                  state = 2;
                  break;
                }
                __builtin_amdgcn_s_sleep(1);
              }
            }
            if (state == 0) {
              // the whole step complete?  then the acquire covers all of it
              const uint32_t v = __hip_atomic_load(step_counter(a, lg, h_own), __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
              if (h_own < 64 && v >= P * static_cast<uint32_t>(own.nst))
                acq_steps |= 1ull << h_own;
              else if (sp < 64)
                acq_strips |= 1ull << sp;
            }
            if (state != 1) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
          }
          bcast[2] = state;
          bcast[3] = (done0 ? 1 : 0) | (done1 ? 2 : 0);
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        barrier_only();
        const int state = __builtin_amdgcn_readfirstlane(bcast[2]);
        const int dn = __builtin_amdgcn_readfirstlane(bcast[3]);
        done0 = (dn & 1) != 0;
        done1 = (dn & 2) != 0;
        if (state == 1) {
          const int pc = __builtin_amdgcn_readfirstlane(bcast[1]);
          copy_claimed(a, pc, pc + 1, smem, delayed, t_start);
          continue;
        }
        if (state == 2) {
          // the wait ran out: copy the strip here (the claimers' bytes exactly)
          const int per = own.P;
          for (int pc = 0; pc < per; ++pc) copy_piece(a, own.piece, strip, lg, pc, smem);
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          barrier_only();
          if (tid == 0) {
            release_agent();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
          }
          barrier_only();
        }
        break;
      }
    }

    // 3. the GEMM tile, the rotating operand read from G for a staged strip
    if (a.times && tid == 0)
      __hip_atomic_fetch_max(a.times + 2 + 3 * h_own, ~wall_clock64(), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    GemmParams gp = a.g;
    if (wait) {
      if (a.rot == 0) gp.A = a.gath;
      else if (a.rot == 1) gp.B = a.gath;
      else gp.C = a.gath;
    }
    const int tm = a.cols ? ob : strip;
    const int tn = a.cols ? strip : ob;
    // the tile's in-loop piece (list 1), claimed now that its wait is over
    LoopCopy lc;
    lc.chunks = 0;
    int lp_step = 0, lp_chunk = 0;
    if (a.loop_copy && !done1) {
      if (tid == 0) bcast[5] = __hip_atomic_fetch_add(claim1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      barrier_only();
      const int pc = a.list_begin[1] + __builtin_amdgcn_readfirstlane(bcast[5]);
      if (pc + 1 >= a.list_end[1]) done1 = true;
      if (pc < a.list_end[1]) {
        lp_step = piece_step(a, pc);
        const FusedStepCopy& sh = a.steps[lp_step];
        lp_chunk = pc - sh.base;
        const ChunkAt at = chunk_at(a, sh, lp_chunk);
        const int64_t r0 = static_cast<int64_t>(a.strip_list[at.pos]) * kBM;
        const int64_t off = r0 * a.row_bytes + static_cast<int64_t>(at.piece) * sh.piece;
        const int64_t end = min(r0 + kBM, a.ext) * a.row_bytes;
        if (off < end) {
          const int64_t bytes = min(sh.piece, end - off);
          const int64_t o = static_cast<int64_t>(at.lg) * a.gbatch + off;
          lc.src = a.src + o;
          lc.dst = const_cast<uint8_t*>(a.gath) + o;
          lc.bytes = static_cast<uint32_t>(bytes);
          lc.chunks = static_cast<int>((bytes + kLoopCopyChunk - 1) / kLoopCopyChunk);
        }
        if (!delayed) {
          if (tid == 0)
            while (wall_clock64() - t_start < static_cast<uint64_t>(a.delay)) __builtin_amdgcn_s_sleep(8);
          delayed = true;
          barrier_only();
        }
        if (lc.chunks == 0 && tid == 0) count_chunk(a, lp_step, lp_chunk);  // an empty piece
      }
    }
    // the piece's stores (agent-coherent) are complete in every wave: count the piece
    const auto after_loop = [&]() {
      if (lc.chunks > 0) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        barrier_only();
        if (tid == 0) count_chunk(a, lp_step, lp_chunk);
      }
    };
    if (hrow < 0)
      gemm_tile<IN, OUT, true>(gp, l, tm, tn, smem, &lc, after_loop);
    else
      gemm_tile<IN, OUT, true, true>(gp, l, tm, tn, smem, &lc, after_loop, hrow);
    if (a.times && tid == 0)
      __hip_atomic_fetch_max(a.times + 3 + 3 * h_own, wall_clock64(), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // Pieces nobody has claimed yet (the local shard's pieces of a returned
  // gathered image, which no tile waits for): the workgroups whose queue is
  // empty take them, a few at a time.
  for (int li = 0; li < 2; ++li) {
    bool done = li == 0 ? done0 : done1;
    int32_t* const ctr = li == 0 ? claim0 : claim1;
    while (!done) {
      constexpr int kSweep = 4;
      barrier_only();  // every wave has read the broadcast words
      if (tid == 0) bcast[1] = __hip_atomic_fetch_add(ctr, kSweep, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      barrier_only();
      const int p0 = a.list_begin[li] + __builtin_amdgcn_readfirstlane(bcast[1]);
      if (p0 >= a.list_end[li]) break;
      copy_claimed(a, p0, min(p0 + kSweep, a.list_end[li]), smem, delayed, t_start);
      done = p0 + kSweep >= a.list_end[li];
    }
  }
  // Last workgroup out resets the counters for the next launch.
  if (tid == 0) {
    release_agent();
    const int old = __hip_atomic_fetch_add(nexit, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = old == static_cast<int>(gridDim.x) - 1;
    if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    bcast[4] = last;
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  barrier_only();
  if (bcast[4]) {
    const int n = a.LG * (a.n_strips + a.S);
    for (int x = tid; x < n; x += kThreads)
      __hip_atomic_store(a.ctr + x, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (tid == 0) {
      for (int x = 0; x < a.nq; ++x)
        __hip_atomic_store(a.sync + x * kSyncStride, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(claim0, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(claim1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(nexit, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (a.times_next)
      for (int x = tid; x < 1 + 3 * a.S; x += kThreads) a.times_next[x] = 0;
    release_agent();
  }
}

template <int IN, int OUT>
inline hipError_t launch_fused_t(const FusedArgs& a, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((fused_run_kernel<IN, OUT>), dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace tile
}  // namespace dg
