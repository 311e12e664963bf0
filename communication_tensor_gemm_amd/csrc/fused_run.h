// fused_run.h -- the whole TP-step schedule of one run as a single persistent
// launch on gfx950: the workgroups perform the shard rotation (copy chunks)
// and the step GEMMs (256 x 256 tiles), and a tile of a staged step starts
// only once its step's shard is complete.
//
// This is the per-step readiness of the Distributed GEMM pull-request page
// (each step's GEMM waits, at its start, for the operand its peer sent;
// described there as a few barriers at the beginning of every GEMM kernel),
// kept on the device: one counter per step, raised once per finished chunk,
// so the steps run back to back inside one launch with no partly filled wave
// between them.  The copy is done by the CUs because the SDMA engines slow
// several-fold under the GEMM's memory traffic on this part.
//
// Steps.  The unit of the launch is a launch group: consecutive steps on
// adjacent shards, computed as one GEMM over their union (as the step-launch
// execution merges them), which keeps steps narrower than a tile from
// leaving partly empty tiles; "group" below means such a group.
//
// Work distribution.  The work items are the tiles.  Workgroup b takes them
// from queue b mod nq (nq = 8: MI355X places workgroup b on XCD b mod 8, so
// every XCD has its own queue and runs one contiguous range of each group's
// tile order, as the per-launch kernel does; nq = 1: one queue for the
// chip), in queue order, by an atomic counter: queue q lists its tiles of
// group 0, then of group 1, and so on.  The shard copies ride on the tiles:
// the copy of group h is cut into chunks of about equal size, one or a few
// per tile of group max(0, h - D) (D = a.ahead >= 1, the copy lookahead),
// and a tile performs the chunks it carries before it waits for anything
// and before its own GEMM.  Separate copy items would make the workgroups
// of an XCD start their tiles out of phase, and tiles that run in phase
// share each K slab of A and B in the XCD's L2: measured, copy items nearly
// doubled the launch's HBM reads, while equal chunks on every tile keep the
// tiles in phase.
//
// Progress.  A carrier does its chunks without waiting, and a tile of group
// h waits only for chunks carried by tiles of earlier groups, which precede
// it in every queue.  Take the lowest group h that any waiting workgroup
// waits for; every queue that has a waiting workgroup has handed out all its
// tiles of group h - 1 or earlier (they precede the waiter's tile), and
// every other queue hands tiles out until it passes them; all of them carry
// out their chunks.  So every wait ends, given that every queue keeps at
// least one running workgroup -- two single-launch runs are therefore never
// in flight together on one device (the host orders them).  A wait is also
// bounded in time: after the limit it is counted as an error (the run's
// result is then undefined) and the workgroup goes on without waiting
// again, so a launch ends within about one limit in any case.
//
// Visibility.  Every wave of a carrier waits until its chunk stores have
// reached L2; after a barrier thread 0 fences at agent scope (L2
// write-back) and adds the chunks to the group's counter; a waiting thread
// polls the counter with agent-scope loads and then performs an agent-scope
// acquire (L1 / L2 invalidate) before the barrier that releases its
// workgroup into the tile.  All counters are reset by the last workgroup to
// finish, so every launch starts from zero (also when replayed from a graph).
#pragma once
#include "gemm_tile.h"

namespace dg {
namespace tile {

typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

// Copy `rows` rows of `bytes` bytes (a multiple of sizeof(T)) from src to dst,
// rows spitch / dpitch bytes apart, with the workgroup's 256 threads; eight
// units in flight per thread.  Non-temporal: the copied bytes are not reused
// by this workgroup, and they should not evict the GEMM's operand lines.
template <typename T>
__device__ __forceinline__ void copy_rows(const uint8_t* src, int64_t spitch, uint8_t* dst,
                                          int64_t dpitch, int64_t rows, int64_t bytes) {
  constexpr int U = 8;
  const int tid = threadIdx.x;
  const int64_t upr = bytes / static_cast<int64_t>(sizeof(T));
  if (rows == 1) {
    const T* s = reinterpret_cast<const T*>(src);
    T* d = reinterpret_cast<T*>(dst);
    int64_t u = tid;
    for (; u + (U - 1) * kThreads < upr; u += U * kThreads) {
      T v[U];
#pragma unroll
      for (int j = 0; j < U; ++j) v[j] = __builtin_nontemporal_load(s + u + j * kThreads);
#pragma unroll
      for (int j = 0; j < U; ++j) __builtin_nontemporal_store(v[j], d + u + j * kThreads);
    }
    for (; u < upr; u += kThreads) __builtin_nontemporal_store(__builtin_nontemporal_load(s + u), d + u);
    return;
  }
  // several rows: one flat index over rows x units (a chunk holds < 2^32 units)
  const uint32_t total = static_cast<uint32_t>(rows * upr);
  const uint32_t up = static_cast<uint32_t>(upr);
  uint32_t f = tid;
  for (; f + (U - 1) * kThreads < total; f += U * kThreads) {
    T v[U];
    int64_t so[U], dof[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const uint32_t idx = f + j * kThreads;
      const uint32_t r = idx / up, c = idx - r * up;
      so[j] = r * spitch + static_cast<int64_t>(c) * sizeof(T);
      dof[j] = r * dpitch + static_cast<int64_t>(c) * sizeof(T);
      v[j] = __builtin_nontemporal_load(reinterpret_cast<const T*>(src + so[j]));
    }
#pragma unroll
    for (int j = 0; j < U; ++j) __builtin_nontemporal_store(v[j], reinterpret_cast<T*>(dst + dof[j]));
  }
  for (; f < total; f += kThreads) {
    const uint32_t r = f / up, c = f - r * up;
    const T v = __builtin_nontemporal_load(
        reinterpret_cast<const T*>(src + r * spitch + static_cast<int64_t>(c) * sizeof(T)));
    __builtin_nontemporal_store(v, reinterpret_cast<T*>(dst + r * dpitch + static_cast<int64_t>(c) * sizeof(T)));
  }
}

// Chunk c of the copy of group st: shard c / chunks_per_step of the group,
// and in it row block c' / chunks_per_row, column piece c' mod chunks_per_row
// (c' = c mod chunks_per_step) of the shard region.
__device__ __forceinline__ void copy_chunk(const FusedArgs& a, const FusedStep& st, int c) {
  const int m = c / st.chunks_per_step;  // shard of the group
  c -= m * st.chunks_per_step;
  const int64_t pr = c / st.chunks_per_row, pc = c - pr * st.chunks_per_row;
  const int64_t r0 = pr * st.chunk_rows, c0 = pc * st.chunk_cols;
  const int64_t rows = min(st.chunk_rows, a.cp_height - r0);
  const int64_t bytes = min(st.chunk_cols, a.cp_width - c0);
  const int64_t shard = m * a.cp_width;
  const uint8_t* src =
      static_cast<const uint8_t*>(a.copy_src) + st.copy_src_off + shard + r0 * a.cp_src_pitch + c0;
  uint8_t* dst = a.staging + st.copy_dst_off + shard + r0 * a.cp_dst_pitch + c0;
  if (a.unit == 16)
    copy_rows<u32x4>(src, a.cp_src_pitch, dst, a.cp_dst_pitch, rows, bytes);
  else if (a.unit == 4)
    copy_rows<uint32_t>(src, a.cp_src_pitch, dst, a.cp_dst_pitch, rows, bytes);
  else
    copy_rows<uint8_t>(src, a.cp_src_pitch, dst, a.cp_dst_pitch, rows, bytes);
}

// GemmParams of step st for this run's operands.
__device__ __forceinline__ GemmParams fused_step_params(const FusedArgs& a, const FusedStep& st) {
  GemmParams g;
  const uint8_t* stg = a.staging;
  g.A = (st.stagedA ? stg : static_cast<const uint8_t*>(a.A)) + st.offA;
  g.B = (st.stagedB ? stg : static_cast<const uint8_t*>(a.B)) + st.offB;
  g.C = a.beta != 0.0f ? (st.stagedC ? stg : static_cast<const uint8_t*>(a.C)) + st.offC : nullptr;
  g.D = static_cast<uint8_t*>(a.D) + st.offD;
  g.bias = a.bias ? static_cast<const uint8_t*>(a.bias) + st.offBias : nullptr;
  g.lda = st.lda; g.ldb = st.ldb; g.ldc = st.ldc; g.ldd = st.ldd;
  g.sA = st.sA; g.sB = st.sB; g.sC = st.sC; g.sD = st.sD;
  g.M = st.M; g.N = st.N; g.K = a.K; g.L = a.L;
  g.alpha = a.alpha; g.beta = a.beta;
  return g;
}

template <int IN, int OUT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void
fused_run_kernel(FusedArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kSlots * kOperandSlab];
  // item broadcast word: at the end of the last ring slot, which a tile first
  // fills only after its prologue barrier (by then every wave has read the
  // word) and which the epilogue leaves alone
  volatile int32_t* bcast = reinterpret_cast<volatile int32_t*>(smem + kSlots * kOperandSlab - 256);
  const int tid = threadIdx.x;
  const int S = a.S;
  const int q = static_cast<int>(blockIdx.x) % a.nq;
  int32_t* const qctr = a.sync + q * kSyncStride;
  int32_t* const done = a.sync + kSyncDone * kSyncStride;
  int32_t* const nexit = a.sync + kSyncExit * kSyncStride;
  int32_t* const nerr = a.sync + kSyncErr * kSyncStride;
  const int32_t* const seg = a.seg + q * (S + 1);
  const int n_items = seg[S];

  uint64_t ready = 0;     // thread 0: groups < 64 seen complete
  bool gave_up = false;   // thread 0: a wait ran out; wait no more in this launch
  int g = 0;              // group of the last tile (tiles come in increasing order)
  for (;;) {
    barrier_only();  // every wave is done with the previous tile
    if (tid == 0) bcast[0] = __hip_atomic_fetch_add(qctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    barrier_only();
    const int k = __builtin_amdgcn_readfirstlane(bcast[0]);
    if (k >= n_items) break;
    while (k >= seg[g + 1]) ++g;
    const FusedStep& st = a.steps[g];
    // the tile: position i of this queue's share of group g
    const int i = k - seg[g];
    const int T2 = st.tiles_m * st.tiles_n;
    const int qq = T2 / a.nq, r = T2 - qq * a.nq;
    const int share = qq + (q < r ? 1 : 0), first = q * qq + min(q, r);
    const int l = i / share, j = i - l * share;
    const int gidx = l * T2 + first + j;  // index among all tiles of the group
    const int gtiles = T2 * a.L;

    // 1. the chunks this tile carries: chunk gidx, gidx + gtiles, ... of the
    //    copy of every group the tiles of group g carry
    const int h0 = g == 0 ? 1 : g + a.ahead;
    const int h1 = min(S - 1, g == 0 ? a.ahead : g + a.ahead);
    bool copied = false;
    for (int h = h0; h <= h1; ++h) {
      const FusedStep& sh = a.steps[h];
      for (int c = gidx; c < sh.n_chunks; c += gtiles) {
        copy_chunk(a, sh, c);
        copied = true;
      }
    }
    if (copied) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's stores are in L2
      barrier_only();
      if (tid == 0) {
        __threadfence();  // write back the chunks, then count them
        for (int h = h0; h <= h1; ++h) {
          const int n = a.steps[h].n_chunks;
          const int cnt = gidx < n ? (n - gidx + gtiles - 1) / gtiles : 0;
          if (cnt > 0)
            __hip_atomic_fetch_add(done + h * kSyncStride, cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }

    // 2. a staged group's tile waits until the group's copy is complete
    if (st.n_chunks > 0) {
      if (tid == 0) {
        const bool known = g < 64 && ((ready >> g) & 1);
        if (!known && !gave_up) {
          const uint64_t t0 = wall_clock64();
          while (__hip_atomic_load(done + g * kSyncStride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
                 st.n_chunks) {
            if (wall_clock64() - t0 > static_cast<uint64_t>(a.spin_limit)) {
              __hip_atomic_fetch_add(nerr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              gave_up = true;
              break;
            }
            __builtin_amdgcn_s_sleep(1);
          }
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
          if (g < 64) ready |= 1ull << g;
        }
      }
      barrier_only();
    }

    // 3. the GEMM tile
    int tm, tn;
    order_tile(first + j, st.tiles_m, st.tiles_n, tm, tn);
    const GemmParams gp = fused_step_params(a, st);
    gemm_tile<IN, OUT>(gp, l, tm, tn, smem);
  }
  // Last workgroup out resets the counters for the next launch.
  if (tid == 0) {
    __threadfence();
    const int old = __hip_atomic_fetch_add(nexit, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old == static_cast<int>(gridDim.x) - 1) {
      for (int x = 0; x < a.nq; ++x)
        __hip_atomic_store(a.sync + x * kSyncStride, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (int s = 0; s < S; ++s)
        __hip_atomic_store(done + s * kSyncStride, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(nexit, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __threadfence();
    }
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
