// Host side of the TP-step GEMM library: validation, the step table, the
// plan (gathered staging image, streams, events, device tables), the
// side-stream shard-copy engine, the single-launch tables and the C ABI
// declared in include/distgemm.h.
//
// Mechanism (Distributed GEMM pull-request page, description): the operand
// that arrives from a peer at every step is moved while the GEMM of the
// current step runs, and each step's GEMM starts only after its operand is
// in place.  On one GPU the peer's shard is a region of the caller's
// operand, copied device to device into the same region of a gathered image
// G of that operand (plan-owned, or the caller's gathered output).  By
// default one persistent launch per run does everything (fused_run.h).  The
// alternative execution launches the step GEMMs separately, with one copy
// per staged step on side streams, each followed by an event that the launch
// computing the step waits on.  Copies go round-robin to up to eight side
// streams, one per peer link that the transfer stands in for; the copy is
// the library's streaming copy kernel by default (it runs between GEMM
// workgroups); the runtime's device copy and the SDMA engine (NoCU) are
// options -- measured, SDMA slows several-fold while the GEMMs load memory.
// Consecutive staged steps whose shards are adjacent may run as one GEMM
// launch; launches alternate between the caller's stream and a second
// compute stream (the stream alternation of the PyTorch symmetric-memory
// page's all-gather consumer), so the last, partly filled wave of one
// launch overlaps the next.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <algorithm>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/distgemm.h"
#include "gemm_launch.h"

namespace {

thread_local std::string g_last_error = "no error";

struct Problem {
  int64_t M = 0, N = 0, K = 0, L = 0;
  int S = 1;  // number of steps
  int schedule = 0, dtype = 0;
  int in_kind = 0, out_kind = 0;
  int es_in = 0, es_out = 0;
  bool shared_a = false;  // one A (M x K) for all L batches
};

int fail(std::string* where, int code, const std::string& msg) {
  (where ? *where : g_last_error) = std::string(dist_gemm_status_string(code)) + ": " + msg;
  return code;
}

int dtype_kinds(int dtype, int* in_kind, int* out_kind) {
  switch (dtype) {
    case DIST_GEMM_F32: *in_kind = dg::IN_F32; *out_kind = dg::OUT_F32; return 0;
    case DIST_GEMM_BF16_F32: *in_kind = dg::IN_BF16; *out_kind = dg::OUT_F32; return 0;
    case DIST_GEMM_BF16_BF16: *in_kind = dg::IN_BF16; *out_kind = dg::OUT_BF16; return 0;
    case DIST_GEMM_E4M3_BF16: *in_kind = dg::IN_E4M3; *out_kind = dg::OUT_BF16; return 0;
    case DIST_GEMM_E4M3_F32: *in_kind = dg::IN_E4M3; *out_kind = dg::OUT_F32; return 0;
    case DIST_GEMM_E4M3_E4M3: *in_kind = dg::IN_E4M3; *out_kind = dg::OUT_E4M3; return 0;
    default: return -1;
  }
}

bool rows_schedule(int schedule) {
  return schedule == DIST_GEMM_AG_ROT_A || schedule == DIST_GEMM_RS_TILE_A_ROT_C;
}

int validate(int64_t M, int64_t N, int64_t K, int64_t L, int TP, int schedule, int dtype,
             Problem* pr, std::string* err) {
  if (M < 1 || N < 1 || K < 1 || L < 1) return fail(err, DIST_GEMM_ERR_INVALID_ARG, "M, N, K, L must be >= 1");
  if (TP < 1) return fail(err, DIST_GEMM_ERR_INVALID_ARG, "TP must be >= 1");
  if (schedule < DIST_GEMM_AG_ROT_A || schedule > DIST_GEMM_MONOLITHIC)
    return fail(err, DIST_GEMM_ERR_INVALID_ARG, "unknown schedule " + std::to_string(schedule));
  Problem p;
  if (dtype_kinds(dtype, &p.in_kind, &p.out_kind) != 0)
    return fail(err, DIST_GEMM_ERR_INVALID_ARG, "unknown dtype " + std::to_string(dtype));
  if (TP > 1024) return fail(err, DIST_GEMM_ERR_SHAPE, "TP must be <= 1024");
  if (M > INT32_MAX || N > INT32_MAX) return fail(err, DIST_GEMM_ERR_SHAPE, "M and N must be < 2^31");
  if (L > 65535) return fail(err, DIST_GEMM_ERR_SHAPE, "L must be <= 65535");
  p.es_in = dg::in_elem_size(p.in_kind);
  p.es_out = dg::out_elem_size(p.out_kind);
  if ((K * p.es_in) % 16 != 0)
    return fail(err, DIST_GEMM_ERR_SHAPE,
                "K * element size must be a multiple of 16 bytes (K=" + std::to_string(K) + ")");
  if (static_cast<double>(K) * p.es_in * dg::kBM >= 2147483648.0)
    return fail(err, DIST_GEMM_ERR_SHAPE, "K too large: 256 rows of K must span < 2 GiB");
  p.M = M; p.N = N; p.K = K; p.L = L;
  p.schedule = schedule; p.dtype = dtype;
  p.S = schedule == DIST_GEMM_MONOLITHIC ? 1 : TP;
  if (schedule != DIST_GEMM_MONOLITHIC) {
    const int64_t ext = rows_schedule(schedule) ? M : N;
    if (ext % TP != 0)
      return fail(err, DIST_GEMM_ERR_SHAPE,
                  std::string(rows_schedule(schedule) ? "M" : "N") + "=" + std::to_string(ext) +
                      " is not divisible by TP=" + std::to_string(TP));
  }
  *pr = p;
  return DIST_GEMM_OK;
}

// Step s of rank 0: the all-gather schedules consume their own shard first
// and then shard (s + rank) mod S; the reduce-scatter schedules produce
// chunk (rank + s + 1) mod S so that the own chunk comes last.
std::vector<dist_gemm_step> build_steps(const Problem& p) {
  std::vector<dist_gemm_step> v;
  if (p.schedule == DIST_GEMM_MONOLITHIC) {
    v.push_back({0, 0, 0, -1, 0, p.M, 0, p.N});
    return v;
  }
  const int S = p.S;
  const bool ag = p.schedule == DIST_GEMM_AG_ROT_A || p.schedule == DIST_GEMM_AG_ROT_B;
  const bool rows = rows_schedule(p.schedule);
  const int64_t w = (rows ? p.M : p.N) / S;
  for (int s = 0; s < S; ++s) {
    const int j = ag ? (s % S) : ((s + 1) % S);
    dist_gemm_step st{};
    st.step = s;
    st.shard = j;
    st.staged = s > 0 ? 1 : 0;
    st.slot = s > 0 ? j : -1;  // shard position in the gathered image
    if (rows) {
      st.m0 = j * w; st.m1 = (j + 1) * w; st.n0 = 0; st.n1 = p.N;
    } else {
      st.m0 = 0; st.m1 = p.M; st.n0 = j * w; st.n1 = (j + 1) * w;
    }
    v.push_back(st);
  }
  return v;
}

// The gathered image G of the rotating operand has the operand's own layout:
// shard j occupies, in G, the bytes it occupies in the operand -- `height`
// rows of `width` bytes at offset j * width, rows `pitch` apart (one row per
// batch for the row-contiguous shards; one row per row of C for the column
// chunks of RS_TILE_B_ROT_C).  So a staged step reads G exactly where it
// would read the operand, and the shards of consecutive steps are adjacent
// in G as in the operand.
struct CopyGeom {
  size_t width = 0, height = 0, pitch = 0;
  size_t alloc = 0;  // bytes of the plan's G (sized for L batches also when A is shared)
};

CopyGeom copy_geom(const Problem& p) {
  CopyGeom g;
  const size_t S = static_cast<size_t>(p.S);
  const size_t L = static_cast<size_t>(p.L);
  switch (p.schedule) {
    case DIST_GEMM_AG_ROT_A:  // A row shard, per batch contiguous (one batch if A is shared)
      g.width = static_cast<size_t>(p.M / S) * p.K * p.es_in;
      g.height = p.shared_a ? 1 : L;
      g.pitch = static_cast<size_t>(p.M) * p.K * p.es_in;
      g.alloc = L * g.pitch;
      break;
    case DIST_GEMM_AG_ROT_B:  // B column shard = rows of the N x K storage
      g.width = static_cast<size_t>(p.N / S) * p.K * p.es_in;
      g.height = L;
      g.pitch = static_cast<size_t>(p.N) * p.K * p.es_in;
      g.alloc = L * g.pitch;
      break;
    case DIST_GEMM_RS_TILE_A_ROT_C:  // C row chunk
      g.width = static_cast<size_t>(p.M / S) * p.N * p.es_out;
      g.height = L;
      g.pitch = static_cast<size_t>(p.M) * p.N * p.es_out;
      g.alloc = L * g.pitch;
      break;
    case DIST_GEMM_RS_TILE_B_ROT_C:  // C column chunk: one strip per row
      g.width = static_cast<size_t>(p.N / S) * p.es_out;
      g.height = L * static_cast<size_t>(p.M);
      g.pitch = static_cast<size_t>(p.N) * p.es_out;
      g.alloc = g.height * g.pitch;
      break;
    default:
      break;
  }
  return g;
}

bool reduce_scatter(int schedule) {
  return schedule == DIST_GEMM_RS_TILE_A_ROT_C || schedule == DIST_GEMM_RS_TILE_B_ROT_C;
}

}  // namespace

struct dist_gemm_plan_s {
  Problem pr;
  std::vector<dist_gemm_step> steps;
  CopyGeom geom;
  int device = 0;
  uint8_t* staging = nullptr;  // the plan's gathered image G (geom.alloc bytes)
  std::vector<hipStream_t> sides;     // copy engine streams (created on demand)
  std::vector<hipEvent_t> ev_side_done;  // one per side stream
  hipStream_t cs2 = nullptr;   // second compute stream
  hipEvent_t ev_start = nullptr, ev_cs2_done = nullptr, ev_done = nullptr;
  std::vector<hipEvent_t> ev_copy;
  // Per-step timing ring: event pairs for the last `step_timing` runs,
  // indexed [run % step_timing][step].
  std::vector<hipEvent_t> t_begin, t_end;
  // Timeline of the same runs: run start, and copy completion per step.
  std::vector<hipEvent_t> t_run0, t_copy;
  // [run % step_timing][step] = first step of the launch that computed it
  // (launch events are recorded at that step's index).
  std::vector<int> t_first;
  // Single-launch execution: device tables and counters (rotating plans
  // only), allocated once at their largest size and never freed before the
  // plan, so a captured run's kernel arguments stay valid.
  int execution = 1;
  int queues = dg::kMaxQueues;
  int64_t copy_chunk = 2 << 20;
  int64_t wait_limit_us = 1000000;
  int64_t copy_delay_us = 0;   // test hook: copies start this late
  int64_t clock_khz = 100000;  // device wall clock rate
  int n_cu = 256;
  int n_strips = 0;            // strips per batch of the rotating operand
  dg::FusedSeg* d_segs = nullptr;        // [S]
  dg::FusedStepCopy* d_copies = nullptr; // [S]
  int32_t* d_strips = nullptr;           // [2][n_strips]: strip list, step of each position
  int32_t* d_seg = nullptr;              // [kMaxQueues][S + 1]
  uint32_t* d_ctr = nullptr;             // [L][n_strips] strip counters, [L][S] step counters
  int32_t* d_sync = nullptr;
  uint64_t* d_times = nullptr;           // [step_timing][timeline_words(S)]
  uint64_t fused_align = 0;   // OR of the piece sizes (copy unit choice)
  int n_segs = 0;             // segments in the device tables
  int n_list0 = 0, n_list1 = 0, n_local = 0;  // copy pieces: of claim lists 0 and 1; of step 0
  bool fused_loop = false;                    // list-1 pieces are copied inside K loops
  int copy_ahead = 0;         // segments whose tiles claim a copy quota before their GEMM
  bool captured = false;      // a run was captured into a graph: tables are fixed
  std::vector<char> t_fused;  // [run % step_timing]: the run was one launch
  float scale_a = 1.0f, scale_b = 1.0f;
  float result_scale = 1.0f;   // e4m3 output only
  int fast_accum = 0;          // accepted; gfx950 MFMAs accumulate in fp32 either way
  int half_tiles = 1;          // a last partial round of tiles runs as half-height tiles
  const void* bias = nullptr;  // device, N values of the output type, or NULL
  int compute_streams = 2;
  int copy_engine = 2;  // library streaming copy kernel
  int copy_streams = 2;
  int max_group = 2;  // consecutive staged steps per launch / queue segment
  int step_timing = 0;
  int64_t timed_runs = 0;  // runs recorded since timing was (re)enabled
  bool has_prev = false;
  hipStream_t prev_stream = nullptr;
  std::string err = "no error";
};

namespace {

int hip_fail(std::string* err, hipError_t e, const char* what) {
  return fail(err, DIST_GEMM_ERR_HIP, std::string(what) + ": " + hipGetErrorName(e) + " (" +
                                          hipGetErrorString(e) + ")");
}

#define DG_HIP(plan_err, call)                                  \
  do {                                                          \
    hipError_t e_ = (call);                                     \
    if (e_ != hipSuccess) return hip_fail(plan_err, e_, #call); \
  } while (0)

void release(dist_gemm_plan_s* p) {
  if (!p) return;
  for (hipStream_t s : p->sides) if (s) (void)hipStreamSynchronize(s);
  if (p->cs2) (void)hipStreamSynchronize(p->cs2);
  if (p->ev_done) (void)hipEventSynchronize(p->ev_done);
  for (hipEvent_t e : p->ev_copy) if (e) (void)hipEventDestroy(e);
  for (hipEvent_t e : p->t_begin) if (e) (void)hipEventDestroy(e);
  for (hipEvent_t e : p->t_end) if (e) (void)hipEventDestroy(e);
  for (hipEvent_t e : p->t_run0) if (e) (void)hipEventDestroy(e);
  for (hipEvent_t e : p->t_copy) if (e) (void)hipEventDestroy(e);
  for (hipEvent_t e : p->ev_side_done) if (e) (void)hipEventDestroy(e);
  for (hipEvent_t e : {p->ev_start, p->ev_cs2_done, p->ev_done})
    if (e) (void)hipEventDestroy(e);
  for (hipStream_t s : p->sides) if (s) (void)hipStreamDestroy(s);
  if (p->cs2) (void)hipStreamDestroy(p->cs2);
  if (p->staging) (void)hipFree(p->staging);
  for (void* d : {static_cast<void*>(p->d_segs), static_cast<void*>(p->d_copies),
                  static_cast<void*>(p->d_strips), static_cast<void*>(p->d_seg),
                  static_cast<void*>(p->d_ctr), static_cast<void*>(p->d_sync),
                  static_cast<void*>(p->d_times)})
    if (d) (void)hipFree(d);
  delete p;
}

struct DeviceGuard {
  int prev = -1;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) == hipSuccess && prev != dev) (void)hipSetDevice(dev);
    else prev = -1;
  }
  ~DeviceGuard() {
    if (prev >= 0) (void)hipSetDevice(prev);
  }
};

// Make sure the plan owns at least n side streams (and their join events).
int ensure_sides(dist_gemm_plan_s* P, int n, std::string* err) {
  while (static_cast<int>(P->sides.size()) < n) {
    hipStream_t s = nullptr;
    hipEvent_t ev = nullptr;
    hipError_t e = hipStreamCreateWithFlags(&s, hipStreamNonBlocking);
    if (e != hipSuccess) return hip_fail(err, e, "side stream creation");
    e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
    if (e != hipSuccess) {
      (void)hipStreamDestroy(s);
      return hip_fail(err, e, "side stream event creation");
    }
    P->sides.push_back(s);
    P->ev_side_done.push_back(ev);
  }
  return DIST_GEMM_OK;
}

// Streaming 2-D copy for the shard rotation: `height` rows of `width` bytes,
// source rows `spitch` apart, destination rows `dpitch` apart.  Rows spread
// over gridDim.y, units of T (16, 4 or 1 bytes) of a row over gridDim.x x
// 256 threads.  Non-temporal loads and stores keep the copied bytes from
// evicting the operand lines the concurrently running GEMM reuses in L2.
typedef __attribute__((ext_vector_type(4))) unsigned int copy_u32x4;

template <typename T>
__global__ __launch_bounds__(256) void shard_copy_kernel(uint8_t* __restrict__ dst, size_t dpitch,
                                                       const uint8_t* __restrict__ src, size_t spitch,
                                                       size_t width, size_t height) {
  const size_t units = width / sizeof(T);
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (size_t r = blockIdx.y; r < height; r += gridDim.y) {
    const T* s = reinterpret_cast<const T*>(src + r * spitch);
    T* d = reinterpret_cast<T*>(dst + r * dpitch);
    for (size_t c = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; c < units; c += stride)
      __builtin_nontemporal_store(__builtin_nontemporal_load(s + c), d + c);
  }
}

hipError_t launch_shard_copy(uint8_t* dst, size_t dpitch, const uint8_t* src, size_t spitch,
                             size_t width, size_t height, hipStream_t stream) {
  const uint64_t align = reinterpret_cast<uint64_t>(dst) | reinterpret_cast<uint64_t>(src) |
                         dpitch | spitch | width;
  const size_t unit = (align % 16 == 0) ? 16 : (align % 4 == 0) ? 4 : 1;
  const size_t units = width / unit;
  // about 2048 workgroups of 256 threads in all, at least one row per grid row
  const size_t gx = std::max<size_t>(1, std::min<size_t>((units + 1023) / 1024, 2048));
  const size_t gy = std::max<size_t>(1, std::min<size_t>(height, 2048 / gx));
  const dim3 grid(static_cast<unsigned>(gx), static_cast<unsigned>(gy));
  if (unit == 16)
    hipLaunchKernelGGL(shard_copy_kernel<copy_u32x4>, grid, dim3(256), 0, stream, dst, dpitch, src,
                       spitch, width, height);
  else if (unit == 4)
    hipLaunchKernelGGL(shard_copy_kernel<uint32_t>, grid, dim3(256), 0, stream, dst, dpitch, src,
                       spitch, width, height);
  else
    hipLaunchKernelGGL(shard_copy_kernel<uint8_t>, grid, dim3(256), 0, stream, dst, dpitch, src,
                       spitch, width, height);
  return hipGetLastError();
}

// Copy shard `shard` of the rotating operand into the same region of the
// gathered image G on `side`.
int enqueue_copy(dist_gemm_plan_s* P, hipStream_t side, const void* src_base, uint8_t* G, int shard) {
  const CopyGeom& g = P->geom;
  const size_t off = static_cast<size_t>(shard) * g.width;
  const uint8_t* src = static_cast<const uint8_t*>(src_base) + off;
  uint8_t* dst = G + off;
  hipError_t e;
  if (P->copy_engine == 2) {
    e = launch_shard_copy(dst, g.pitch, src, g.pitch, g.width, g.height, side);
    if (e != hipSuccess) return hip_fail(&P->err, e, "shard copy kernel");
    return DIST_GEMM_OK;
  }
  const hipMemcpyKind kind =
      P->copy_engine == 0 ? hipMemcpyDeviceToDeviceNoCU : hipMemcpyDeviceToDevice;
  if (g.height == 1)
    e = hipMemcpyAsync(dst, src, g.width, kind, side);
  else
    e = hipMemcpy2DAsync(dst, g.pitch, src, g.pitch, g.width, g.height, kind, side);
  if (e != hipSuccess) return hip_fail(&P->err, e, "shard copy");
  return DIST_GEMM_OK;
}

// Test hook of the step-launch execution: holds a side stream for `ticks`
// of the device wall clock before its copies (one thread, bounded).
__global__ void copy_delay_kernel(uint64_t ticks) {
  const uint64_t t0 = wall_clock64();
  while (wall_clock64() - t0 < ticks) __builtin_amdgcn_s_sleep(8);
}

// Launches of one run: consecutive staged steps whose shards are adjacent
// (shard index one higher, so adjacent in G as in the operand) merge, up to
// max_group steps per launch; the unstaged step launches alone.
struct LaunchGroup {
  int first, count;
};

std::vector<LaunchGroup> group_steps(const dist_gemm_plan_s* P) {
  std::vector<LaunchGroup> v;
  for (int i = 0; i < static_cast<int>(P->steps.size()); ++i) {
    const dist_gemm_step& s = P->steps[i];
    if (!v.empty() && P->pr.schedule != DIST_GEMM_MONOLITHIC) {
      LaunchGroup& b = v.back();
      const dist_gemm_step& prev = P->steps[b.first + b.count - 1];
      const bool adjacent = s.staged && prev.staged && s.shard == prev.shard + 1;
      if (adjacent && b.count < P->max_group) {
        ++b.count;
        continue;
      }
    }
    v.push_back({i, 1});
  }
  return v;
}

// Where step st's operands live: byte offsets from the caller's operands
// (G has the rotating operand's layout, so a staged operand is read at the
// same offsets from G), with leading dimensions and batch strides in
// elements.
struct StepLayout {
  int64_t offA, offB, offC, offD, offBias;
  int64_t lda, ldb, ldc, ldd, sA, sB, sC, sD;
  int32_t M, N;
  bool stagedA, stagedB, stagedC;
};

StepLayout step_layout(const dist_gemm_plan_s* P, const dist_gemm_step& st) {
  const Problem& pr = P->pr;
  const int64_t M = pr.M, N = pr.N, K = pr.K;
  const int ei = pr.es_in, eo = pr.es_out;
  StepLayout y{};
  y.M = static_cast<int32_t>(st.m1 - st.m0);
  y.N = static_cast<int32_t>(st.n1 - st.n0);
  y.offA = st.m0 * K * ei;  y.lda = K; y.sA = pr.shared_a ? 0 : M * K;
  y.offB = st.n0 * K * ei;  y.ldb = K; y.sB = N * K;
  y.offC = (st.m0 * N + st.n0) * eo; y.ldc = N; y.sC = M * N;
  y.offD = (st.m0 * N + st.n0) * eo; y.ldd = N; y.sD = M * N;
  y.offBias = st.n0 * eo;
  if (st.staged) {
    switch (pr.schedule) {
      case DIST_GEMM_AG_ROT_A: y.stagedA = true; break;
      case DIST_GEMM_AG_ROT_B: y.stagedB = true; break;
      case DIST_GEMM_RS_TILE_A_ROT_C:
      case DIST_GEMM_RS_TILE_B_ROT_C: y.stagedC = true; break;
      default: break;
    }
  }
  return y;
}

// GEMM parameters of one step.
dg::GemmParams step_params(const dist_gemm_plan_s* P, const dist_gemm_step& st, const void* A,
                           const void* B, const void* C, void* D, const uint8_t* G, float alpha,
                           float beta) {
  const StepLayout y = step_layout(P, st);
  const uint8_t* stg = G;
  dg::GemmParams g{};
  g.K = static_cast<int32_t>(P->pr.K);
  g.L = static_cast<int32_t>(P->pr.L);
  g.alpha = alpha;
  g.beta = beta;
  g.post = P->result_scale;
  g.tail_cus = P->half_tiles ? P->n_cu / dg::kNumXcd : 0;
  g.M = y.M;
  g.N = y.N;
  g.A = (y.stagedA ? stg : static_cast<const uint8_t*>(A)) + y.offA;
  g.B = (y.stagedB ? stg : static_cast<const uint8_t*>(B)) + y.offB;
  g.C = (beta == 0.0f || (!y.stagedC && !C)) ? nullptr
                                             : (y.stagedC ? stg : static_cast<const uint8_t*>(C)) + y.offC;
  g.D = static_cast<uint8_t*>(D) + y.offD;
  g.bias = P->bias ? static_cast<const uint8_t*>(P->bias) + y.offBias : nullptr;
  g.lda = y.lda; g.ldb = y.ldb; g.ldc = y.ldc; g.ldd = y.ldd;
  g.sA = y.sA; g.sB = y.sB; g.sC = y.sC; g.sD = y.sD;
  return g;
}

// GEMM parameters of a launch group: the first step's operands, extended
// over the group's rows (row schedules) or columns.  The group's shards are
// adjacent in the source operand, in G and in D, so the
// extended views address exactly the member steps' data.
dg::GemmParams group_params(const dist_gemm_plan_s* P, const LaunchGroup& grp, const void* A,
                            const void* B, const void* C, void* D, const uint8_t* G, float alpha,
                            float beta) {
  const dist_gemm_step& f = P->steps[grp.first];
  const dist_gemm_step& l = P->steps[grp.first + grp.count - 1];
  dg::GemmParams g = step_params(P, f, A, B, C, D, G, alpha, beta);
  g.M = static_cast<int32_t>(std::max(f.m1, l.m1) - f.m0);
  g.N = static_cast<int32_t>(std::max(f.n1, l.n1) - f.n0);
  return g;
}

// ---- Single-launch execution ----------------------------------------------

// The rotating operand seen as strips of the monolithic tile grid.
struct StripGeom {
  int rot = 0, cols = 0, strided = 0;
  int64_t ext = 0;        // rows (row strips) or columns (column strips)
  int64_t row_bytes = 0;  // row strips: bytes per row; column strips: element bytes
  int64_t gbatch = 0;     // bytes between batches
  int64_t pitch = 0, height = 0;  // column strips: bytes between rows, rows per batch
  int LG = 1;             // batches of G
  int64_t strip_bytes = 0;  // bytes of one full strip of one batch
};

StripGeom strip_geom(const Problem& pr) {
  StripGeom g;
  const int64_t ei = pr.es_in, eo = pr.es_out;
  switch (pr.schedule) {
    case DIST_GEMM_AG_ROT_A:
      g.rot = 0; g.ext = pr.M; g.row_bytes = pr.K * ei;
      g.LG = pr.shared_a ? 1 : static_cast<int>(pr.L);
      g.gbatch = pr.shared_a ? 0 : pr.M * pr.K * ei;
      break;
    case DIST_GEMM_AG_ROT_B:
      g.rot = 1; g.cols = 1; g.ext = pr.N; g.row_bytes = pr.K * ei;
      g.LG = static_cast<int>(pr.L); g.gbatch = pr.N * pr.K * ei;
      break;
    case DIST_GEMM_RS_TILE_A_ROT_C:
      g.rot = 2; g.ext = pr.M; g.row_bytes = pr.N * eo;
      g.LG = static_cast<int>(pr.L); g.gbatch = pr.M * pr.N * eo;
      break;
    case DIST_GEMM_RS_TILE_B_ROT_C:
      g.rot = 2; g.cols = 1; g.ext = pr.N; g.row_bytes = eo;
      g.LG = static_cast<int>(pr.L); g.gbatch = pr.M * pr.N * eo;
      g.pitch = pr.N * eo; g.height = pr.M;
      break;
    default:
      break;
  }
  // AG_ROT_B's strips are tile columns but 256 rows of the N x K storage:
  // contiguous like A's; only RS_TILE_B_ROT_C's strips are strided
  g.strided = pr.schedule == DIST_GEMM_RS_TILE_B_ROT_C ? 1 : 0;
  g.strip_bytes = g.strided ? g.height * dg::kBN * g.row_bytes
                                                           : static_cast<int64_t>(dg::kBM) * g.row_bytes;
  return g;
}

// Allocate the single-launch tables at their largest size (once per plan).
int alloc_fused(dist_gemm_plan_s* P, std::string* err) {
  const Problem& pr = P->pr;
  const int S = pr.S;
  const StripGeom sg = strip_geom(pr);
  P->n_strips = static_cast<int>((sg.ext + dg::kBM - 1) / dg::kBM);
  const size_t n_ctr = static_cast<size_t>(pr.L) * (P->n_strips + S);
  const size_t n_sync = static_cast<size_t>(dg::sync_words(S));
  DG_HIP(err, hipMalloc(&P->d_segs, sizeof(dg::FusedSeg) * S));
  DG_HIP(err, hipMalloc(&P->d_copies, sizeof(dg::FusedStepCopy) * S));
  DG_HIP(err, hipMalloc(&P->d_strips, sizeof(int32_t) * (2 * P->n_strips + S)));
  DG_HIP(err, hipMalloc(&P->d_seg, sizeof(int32_t) * dg::kMaxQueues * (S + 1)));
  DG_HIP(err, hipMalloc(&P->d_ctr, sizeof(uint32_t) * n_ctr));
  DG_HIP(err, hipMalloc(&P->d_sync, sizeof(int32_t) * n_sync));
  DG_HIP(err, hipMemset(P->d_ctr, 0, sizeof(uint32_t) * n_ctr));
  DG_HIP(err, hipMemset(P->d_sync, 0, sizeof(int32_t) * n_sync));
  return DIST_GEMM_OK;
}

// Build the single-launch tables: each strip's step (the latest step of the
// shards it overlaps), the strip list by step, the queue segments (step 0,
// then groups of max_group consecutive steps), which segment carries (or
// claims) each step's copy, the piece size of each step, and each queue's
// item ranges.  Synchronous (plan creation and option changes only).
// Host tables of one single-launch configuration.
struct FusedTables {
  std::vector<dg::FusedSeg> segs;
  std::vector<dg::FusedStepCopy> copies;
  std::vector<int32_t> strips;  // strip list, the step of each position, the steps in claim order
  int32_t n_list0 = 0, n_list1 = 0, n_local = 0;  // pieces: of lists 0 and 1; of step 0
  bool loop = false;                               // list-1 pieces are copied inside K loops
  std::vector<int32_t> seg;     // [nq][n_segs + 1]
  uint64_t align = 0;           // OR of the contiguous piece sizes
};

struct FusedOpts {
  int queues = dg::kMaxQueues;
  int64_t copy_chunk = 2 << 20;
  int copy_ahead = 0;
  int max_group = 2;
  int n_wg = 256;  // workgroups of the launch
};

int compute_fused(const Problem& pr, const std::vector<dist_gemm_step>& steps, const FusedOpts& o,
                  FusedTables* out, std::string* err) {
  const int S = pr.S;
  const int nq = o.queues;
  const StripGeom sg = strip_geom(pr);
  const int ns = static_cast<int>((sg.ext + dg::kBM - 1) / dg::kBM);
  const int64_t w = sg.ext / S;  // shard width along the strip dimension
  const int64_t L = pr.L;
  const int64_t other = sg.cols ? (pr.M + dg::kBM - 1) / dg::kBM : (pr.N + dg::kBN - 1) / dg::kBN;

  std::vector<int> step_of_shard(S, 0);
  for (const dist_gemm_step& st : steps) step_of_shard[st.shard] = st.step;
  std::vector<int> sstep(ns, 0);
  for (int k = 0; k < ns; ++k) {
    const int64_t r0 = static_cast<int64_t>(k) * dg::kBM;
    const int64_t r1 = std::min<int64_t>(r0 + dg::kBM, sg.ext);
    for (int64_t j = r0 / w; j <= (r1 - 1) / w; ++j) sstep[k] = std::max(sstep[k], step_of_shard[j]);
  }
  std::vector<int32_t> list, lstep;
  std::vector<int> sfirst(S + 1, 0);
  for (int h = 0; h < S; ++h) {
    sfirst[h] = static_cast<int>(list.size());
    for (int k = 0; k < ns; ++k)
      if (sstep[k] == h) {
        list.push_back(k);
        lstep.push_back(h);
      }
  }
  sfirst[S] = ns;

  // segments
  std::vector<std::pair<int, int>> segr;  // first and last step
  segr.push_back({0, 0});
  // step 1 alone: the launch's first round then waits for as little as it can
  if (S > 1) segr.push_back({1, 1});
  for (int h = 2; h < S; h += o.max_group) segr.push_back({h, std::min(S - 1, h + o.max_group - 1)});
  const int G = static_cast<int>(segr.size());
  std::vector<int> seg_of(S, 0);
  std::vector<dg::FusedSeg> segs(G);
  for (int g = 0; g < G; ++g) {
    dg::FusedSeg& f = segs[g];
    f.strip0 = sfirst[segr[g].first];
    f.nst = sfirst[segr[g].second + 1] - f.strip0;
    f.tiles = static_cast<int32_t>(f.nst * other);
    f.quota = 0;
    for (int h = segr[g].first; h <= segr[g].second; ++h) seg_of[h] = g;
    if (static_cast<int64_t>(f.nst) * other * L >= INT32_MAX)
      return fail(err, DIST_GEMM_ERR_SHAPE, "too many tiles for one launch");
  }
  // Copies.  Every staged strip (and, for a returned gathered image, every
  // strip of step 0) is cut into pieces, numbered in claim order: list 0
  // (steps 1 .. h1, which the first round of tiles reads), list 1 (steps
  // h1+1 .. S-1), then step 0.  List 0 is claimed before any GEMM: a quota
  // by every tile of the first COPY_AHEAD segments, the rest by the first
  // round's waiting tiles.  In-loop form: list 0 in pieces of 128 KiB; a
  // tile that starts its GEMM copies one piece of list 1 inside its K loop
  // (16 KiB per slab over at most its KT - 2 steady-state slabs), pieces
  // being a strip's equal share, no larger than that and as small as the
  // deadlines allow (the pieces of steps up to h are claimed by tiles that
  // start before step h's segment can: n_wg per round), down to 64 KiB.
  // Quota form (column strips, rows not 16-byte multiples, fewer than 6
  // slabs, or no step after h1): list 1 is empty, pieces of about a quarter
  // of the copy bytes per claimer (whole 32 KiB above that, at least 4 KiB,
  // at most COPY_CHUNK bytes).
  const int64_t per_q = std::max(1, o.n_wg / nq);  // the first round: the first per_q items of every queue
  auto items_of = [&](int g, int q) -> int64_t {
    return (segs[g].tiles / nq + (q < segs[g].tiles % nq ? 1 : 0)) * L;
  };
  std::vector<int64_t> seg_round(G, INT64_MAX);  // the earliest round a tile of segment g starts in
  int g_first = 0;                               // the last segment the first round reaches
  int64_t carriers = 0, waiters = 0;             // claimers of list 0
  for (int q = 0; q < nq; ++q) {
    int64_t at = 0;
    for (int g = 0; g < G; ++g) {
      const int64_t items = items_of(g, q);
      if (items == 0) continue;
      seg_round[g] = std::min(seg_round[g], at / per_q);
      if (at < per_q) {
        g_first = std::max(g_first, g);
        if (g >= o.copy_ahead) waiters += std::min(items, per_q - at);
      }
      at += items;
    }
  }
  for (int g = 0; g < G && g < o.copy_ahead; ++g) carriers += static_cast<int64_t>(segs[g].tiles) * L;
  const int64_t claimers = std::max<int64_t>(1, carriers + waiters);
  const int h1 = segr[g_first].second;
  const int64_t KT = (pr.K * pr.es_in + dg::kRowBytes - 1) / dg::kRowBytes;
  const int64_t cap = std::max<int64_t>(0, KT - 2) * dg::kLoopCopyBytes;
  const bool loop = !sg.strided && sg.row_bytes % 16 == 0 && cap >= 4 * dg::kLoopCopyBytes && h1 < S - 1;
  int64_t piece0, piece1;
  if (loop) {
    piece0 = std::min<int64_t>(sg.strip_bytes, 131072);
    const int64_t n_min = (sg.strip_bytes + cap - 1) / cap;
    const int64_t n_small = (sg.strip_bytes + 65535) / 65536;
    int64_t n_dead = n_small, cum = 0;
    for (int h = h1 + 1; h < S; ++h) {
      cum += static_cast<int64_t>(sfirst[h + 1] - sfirst[h]) * sg.LG;
      const int64_t r = seg_round[seg_of[h]];
      if (cum > 0 && r != INT64_MAX) n_dead = std::min(n_dead, o.n_wg * r / cum);
    }
    const int64_t n = std::max(n_min, std::min(n_dead, n_small));
    piece1 = std::min(cap, ((sg.strip_bytes + n - 1) / n + 4095) / 4096 * 4096);
  } else {
    int64_t staged_strips = 0;
    for (int h = 1; h < S; ++h) staged_strips += sfirst[h + 1] - sfirst[h];
    const int64_t copy_bytes = std::max<int64_t>(1, staged_strips) * sg.LG * sg.strip_bytes;
    int64_t piece = (copy_bytes + 4 * claimers - 1) / (4 * claimers);
    piece = std::max<int64_t>(4096, (piece + 15) / 16 * 16);
    if (piece > 32768) piece = (piece + 32767) / 32768 * 32768;
    piece0 = piece1 = std::min<int64_t>(o.copy_chunk, piece);
  }
  std::vector<dg::FusedStepCopy> cps(S);
  std::vector<int32_t> order;  // steps in claim order
  for (int h = 1; h < S; ++h) order.push_back(h);
  order.push_back(0);
  int64_t n_list0 = 0, n_list1 = 0, base = 0;
  for (int h : order) {
    dg::FusedStepCopy& c = cps[h];
    c.strip0 = sfirst[h];
    c.nst = sfirst[h + 1] - sfirst[h];
    c.wait = h >= 1 ? 1 : 0;
    const int64_t piece = (loop && (h > h1 || h == 0)) ? piece1 : piece0;
    int64_t per;
    if (!sg.strided) {
      c.piece = piece;
      per = (sg.strip_bytes + piece - 1) / piece;
    } else {
      c.piece = std::max<int64_t>(1, piece / (dg::kBN * sg.row_bytes));
      per = (sg.height + c.piece - 1) / c.piece;
    }
    const int64_t n = per * c.nst * sg.LG;
    if (base + n > (int64_t{1} << 30))
      return fail(err, DIST_GEMM_ERR_UNSUPPORTED, "too many copy pieces; raise DIST_GEMM_OPT_COPY_CHUNK");
    c.P = static_cast<int32_t>(per);
    c.n_chunks = static_cast<int32_t>(n);
    c.base = static_cast<int32_t>(base);
    base += n;
    if (h != 0) ((loop && h > h1) ? n_list1 : n_list0) += n;
  }
  const int64_t quota = (n_list0 + claimers - 1) / claimers;
  for (int g = 0; g < G && g < o.copy_ahead; ++g) segs[g].quota = static_cast<int32_t>(quota);
  // queue q: its share of every segment's tiles (a contiguous range of the
  // segment's tile order per batch), segment after segment
  std::vector<int32_t> seg(static_cast<size_t>(nq) * (G + 1), 0);
  for (int q = 0; q < nq; ++q) {
    int64_t at = 0;
    for (int g = 0; g < G; ++g) {
      seg[static_cast<size_t>(q) * (G + 1) + g] = static_cast<int32_t>(at);
      const int64_t T2 = segs[g].tiles;
      at += (T2 / nq + (q < T2 % nq ? 1 : 0)) * L;
      if (at >= INT32_MAX) return fail(err, DIST_GEMM_ERR_SHAPE, "too many tiles for one launch");
    }
    seg[static_cast<size_t>(q) * (G + 1) + G] = static_cast<int32_t>(at);
  }
  out->strips = list;
  out->strips.insert(out->strips.end(), lstep.begin(), lstep.end());
  out->strips.insert(out->strips.end(), order.begin(), order.end());
  out->n_list0 = static_cast<int32_t>(n_list0);
  out->n_list1 = static_cast<int32_t>(n_list1);
  out->n_local = static_cast<int32_t>(base - n_list0 - n_list1);
  out->loop = loop;
  out->segs = std::move(segs);
  out->copies = std::move(cps);
  out->seg = std::move(seg);
  out->align = 0;
  for (const dg::FusedStepCopy& c : out->copies)
    if (!sg.strided) out->align |= static_cast<uint64_t>(c.piece);
  return DIST_GEMM_OK;
}

FusedOpts plan_opts(const dist_gemm_plan_s* P) {
  FusedOpts o;
  o.queues = P->queues;
  o.copy_chunk = P->copy_chunk;
  o.copy_ahead = P->copy_ahead;
  o.max_group = P->max_group;
  o.n_wg = std::max(P->queues, P->n_cu / P->queues * P->queues);
  return o;
}

// Compute the plan's tables and copy them to its device tables.
int build_fused(dist_gemm_plan_s* P, std::string* err) {
  FusedTables t;
  const int rc = compute_fused(P->pr, P->steps, plan_opts(P), &t, err);
  if (rc != DIST_GEMM_OK) return rc;
  DG_HIP(err, hipMemcpy(P->d_segs, t.segs.data(), sizeof(dg::FusedSeg) * t.segs.size(), hipMemcpyHostToDevice));
  DG_HIP(err, hipMemcpy(P->d_copies, t.copies.data(), sizeof(dg::FusedStepCopy) * t.copies.size(),
                        hipMemcpyHostToDevice));
  DG_HIP(err, hipMemcpy(P->d_strips, t.strips.data(), sizeof(int32_t) * t.strips.size(), hipMemcpyHostToDevice));
  DG_HIP(err, hipMemcpy(P->d_seg, t.seg.data(), t.seg.size() * sizeof(int32_t), hipMemcpyHostToDevice));
  P->n_segs = static_cast<int>(t.segs.size());
  P->fused_align = t.align;
  P->n_list0 = t.n_list0;
  P->n_list1 = t.n_list1;
  P->n_local = t.n_local;
  P->fused_loop = t.loop;
  return DIST_GEMM_OK;
}

// Single-launch runs on one device are ordered one after another, across
// plans: the last one's completion event per device.
struct FusedOrder {
  std::mutex mu;
  std::vector<hipEvent_t> tail;  // per device, created on first use
  std::vector<char> live;
};
FusedOrder& fused_order() {
  static FusedOrder* o = new FusedOrder();  // never destroyed: outlives every plan
  return *o;
}

// Device tables and counters of a single-launch run.
struct FusedDevice {
  const dg::FusedSeg* segs;
  const dg::FusedStepCopy* copies;
  const int32_t* strips;  // list, steps of the positions, steps in claim order
  const int32_t* seg;
  uint32_t* ctr;
  int32_t* sync;
  int n_strips, n_segs;
  uint64_t piece_align;
  int n_list0, n_list1, n_local;  // pieces: of claim lists 0 and 1; of step 0
  bool loop;                      // list-1 pieces are copied inside K loops
};

// Arguments of one single-launch run of the problem pr.
dg::FusedArgs fused_args(const Problem& pr, const FusedDevice& dv, int queues, const void* A, const void* B,
                         const void* C, void* D, const void* bias, uint8_t* G, float alpha, float beta,
                         float post, const void* copy_src, bool copy_on, bool copy_local, int64_t spin_ticks,
                         int64_t delay_ticks) {
  const StripGeom sg = strip_geom(pr);
  dg::FusedArgs a{};
  dg::GemmParams& g = a.g;
  g.A = A; g.B = B; g.C = beta != 0.0f ? C : nullptr; g.D = D;
  g.bias = bias;
  g.lda = pr.K; g.ldb = pr.K; g.ldc = pr.N; g.ldd = pr.N;
  g.sA = pr.shared_a ? 0 : pr.M * pr.K; g.sB = pr.N * pr.K; g.sC = pr.M * pr.N; g.sD = pr.M * pr.N;
  g.M = static_cast<int32_t>(pr.M); g.N = static_cast<int32_t>(pr.N);
  g.K = static_cast<int32_t>(pr.K); g.L = static_cast<int32_t>(pr.L);
  g.alpha = alpha; g.beta = beta; g.post = post;
  a.gath = G;
  a.src = static_cast<const uint8_t*>(copy_src);
  a.segs = dv.segs;
  a.steps = dv.copies;
  a.strip_list = dv.strips;
  a.strip_step = dv.strips + dv.n_strips;
  a.claim_steps = dv.strips + 2 * dv.n_strips;
  a.seg = dv.seg;
  a.sync = dv.sync;
  a.ctr = dv.ctr;
  a.row_bytes = sg.row_bytes;
  a.ext = sg.ext;
  a.gbatch = sg.gbatch;
  a.pitch = sg.pitch;
  a.height = sg.height;
  a.spin_limit = spin_ticks;
  a.delay = delay_ticks;
  a.rot = sg.rot;
  a.cols = sg.cols;
  a.strided = sg.strided;
  a.n_strips = dv.n_strips;
  a.LG = sg.LG;
  uint64_t align = reinterpret_cast<uint64_t>(copy_src) | reinterpret_cast<uint64_t>(G) |
                   static_cast<uint64_t>(sg.row_bytes) | static_cast<uint64_t>(sg.gbatch) | dv.piece_align;
  if (sg.strided)
    align |= static_cast<uint64_t>(sg.pitch) | static_cast<uint64_t>(dg::kBN * sg.row_bytes) |
             static_cast<uint64_t>(sg.ext * sg.row_bytes);
  a.unit = (align % 16 == 0) ? 16 : (align % 4 == 0) ? 4 : 1;
  a.n_seg = dv.n_segs;
  a.nq = queues;
  a.S = pr.S;
  a.copy_on = copy_on ? 1 : 0;
  // step 0's pieces (copied when G is returned) close the last list in use
  const int nz = copy_local ? dv.n_local : 0;
  if (!copy_on) {
    a.list_begin[0] = a.list_end[0] = a.list_begin[1] = a.list_end[1] = 0;
  } else if (dv.n_list1 > 0) {
    a.list_begin[0] = 0;
    a.list_end[0] = dv.n_list0;
    a.list_begin[1] = dv.n_list0;
    a.list_end[1] = dv.n_list0 + dv.n_list1 + nz;
  } else {
    a.list_begin[0] = 0;
    a.list_end[0] = dv.n_list0 + nz;
    a.list_begin[1] = a.list_end[1] = a.list_end[0];
  }
  // the in-loop copy moves whole 16-byte units (else the list-1 pieces go to
  // waiting and finished workgroups)
  a.loop_copy = copy_on && dv.loop && dv.n_list1 > 0 && a.unit == 16 ? 1 : 0;
  a.half_tail = 1;
  return a;
}

// Enqueue a single-launch run on st, ordered after the device's previous one
// unless st is capturing; `before` (if any) is enqueued between the wait and
// the launch.
template <typename Before>
int launch_ordered(int device, int in_kind, int out_kind, const dg::FusedArgs& a, int grid, hipStream_t st,
                   std::string* err, Before before) {
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  DG_HIP(err, hipStreamIsCapturing(st, &cap));
  const bool ordered = cap == hipStreamCaptureStatusNone;
  FusedOrder& o = fused_order();
  std::unique_lock<std::mutex> lock(o.mu);
  if (ordered) {
    if (static_cast<int>(o.tail.size()) <= device) {
      o.tail.resize(device + 1, nullptr);
      o.live.resize(device + 1, 0);
    }
    if (!o.tail[device]) DG_HIP(err, hipEventCreateWithFlags(&o.tail[device], hipEventDisableTiming));
    if (o.live[device]) DG_HIP(err, hipStreamWaitEvent(st, o.tail[device], 0));
  }
  const int rc = before();
  if (rc != DIST_GEMM_OK) return rc;
  DG_HIP(err, dg::launch_fused(in_kind, out_kind, a, grid, st));
  if (ordered) {
    DG_HIP(err, hipEventRecord(o.tail[device], st));
    o.live[device] = 1;
  }
  return DIST_GEMM_OK;
}

int run_fused(dist_gemm_plan_s* P, hipStream_t st, const void* A, const void* B, const void* C,
              void* D, uint8_t* G, float alpha, float beta, const void* copy_src, bool copy_on,
              bool copy_local, uint64_t* times, uint64_t* times_next) {
  const Problem& pr = P->pr;
  FusedDevice dv{P->d_segs, P->d_copies, P->d_strips, P->d_seg, P->d_ctr, P->d_sync,
                 P->n_strips, P->n_segs, P->fused_align, P->n_list0, P->n_list1, P->n_local, P->fused_loop};
  dg::FusedArgs a = fused_args(pr, dv, P->queues, A, B, C, D, P->bias, G, alpha, beta, P->result_scale,
                               copy_src, copy_on, copy_local, P->wait_limit_us * P->clock_khz / 1000,
                               P->copy_delay_us * P->clock_khz / 1000);
  a.times = times;
  a.times_next = times_next;
  a.half_tail = P->half_tiles;
  const int grid = std::max(P->queues, P->n_cu / P->queues * P->queues);
  return launch_ordered(P->device, pr.in_kind, pr.out_kind, a, grid, st, &P->err, [] { return DIST_GEMM_OK; });
}

// Change a plan setting that the single-launch tables depend on: wait for
// the plan's last run, apply, rebuild; on failure restore and rebuild.  A
// plan whose run has been captured into a graph keeps its tables (the graph
// holds their addresses and sizes in its kernel arguments).
template <typename Apply, typename Undo>
int change_tables(dist_gemm_plan_t plan, Apply apply, Undo undo) {
  if (plan->captured)
    return fail(&plan->err, DIST_GEMM_ERR_UNSUPPORTED,
                "a run of this plan was captured into a graph: options that rebuild its device "
                "tables (queues, copy chunk, copy lookahead, step group, shared A) are fixed");
  DeviceGuard guard(plan->device);
  if (plan->has_prev) DG_HIP(&plan->err, hipEventSynchronize(plan->ev_done));
  apply();
  if (!plan->d_segs) return DIST_GEMM_OK;  // no staged steps: nothing to rebuild
  const int rc = build_fused(plan, &plan->err);
  if (rc != DIST_GEMM_OK) {
    undo();
    (void)build_fused(plan, nullptr);
  }
  return rc;
}

// ---- Allocation-free runs -------------------------------------------------
//
// dist_gemm_run_noalloc keeps what a plan allocates -- the gathered image,
// the single-launch tables and the counters -- in one file-scope device
// array, `scratch`, of fixed size: every GPU that runs it holds its own copy
// until the process ends.  Host code never passes the array's name to a
// kernel (in host code that name is a host-side stand-in, not a device
// address): each device's address comes from hipGetSymbolAddress on that
// device at its first call.  A small kernel writes each call's tables
// (passed by value) and zeroes the counters, so nothing is copied from host
// memory at run time and a call can be captured into a graph.

constexpr size_t kNoAllocGatherBytes = size_t{32} << 20;  // largest gathered image
constexpr size_t kNoAllocTableBytes = size_t{256} << 10;  // tables and counters
constexpr int kNoAllocMaxSteps = 16;
constexpr int kNoAllocMaxStrips = 128;
// table region: segments, step copies, strips, queue items, sync words, counters
constexpr size_t kNaSegs = 0, kNaCopies = 1024, kNaStrips = 2048, kNaSeg = 4096, kNaSync = 8192,
                 kNaCtr = 16384;
static_assert(sizeof(dg::FusedSeg) * kNoAllocMaxSteps <= kNaCopies - kNaSegs, "no-alloc layout");
static_assert(sizeof(dg::FusedStepCopy) * kNoAllocMaxSteps <= kNaStrips - kNaCopies, "no-alloc layout");
static_assert(sizeof(int32_t) * (2 * kNoAllocMaxStrips + kNoAllocMaxSteps) <= kNaSeg - kNaStrips,
              "no-alloc layout");
static_assert(sizeof(int32_t) * dg::kMaxQueues * (kNoAllocMaxSteps + 1) <= kNaSync - kNaSeg, "no-alloc layout");
static_assert(sizeof(int32_t) * (dg::kSyncClaim + 1) * dg::kSyncStride <= kNaCtr - kNaSync, "no-alloc layout");

struct NoAllocPack {
  dg::FusedSeg segs[kNoAllocMaxSteps];
  dg::FusedStepCopy copies[kNoAllocMaxSteps];
  int32_t strips[2 * kNoAllocMaxStrips + kNoAllocMaxSteps];
  int32_t seg[dg::kMaxQueues * (kNoAllocMaxSteps + 1)];
  int32_t n_segs, n_strips, S, n_ctr;
};

}  // namespace

static __device__ __align__(256) uint8_t scratch[kNoAllocGatherBytes + kNoAllocTableBytes];

namespace {

// Write one call's tables into the table region and zero its counters.
__global__ __launch_bounds__(256) void noalloc_setup_kernel(NoAllocPack pk, uint8_t* tables) {
  const int t = threadIdx.x;
  for (int i = t; i < pk.n_segs; i += 256)
    reinterpret_cast<dg::FusedSeg*>(tables + kNaSegs)[i] = pk.segs[i];
  for (int i = t; i < pk.S; i += 256)
    reinterpret_cast<dg::FusedStepCopy*>(tables + kNaCopies)[i] = pk.copies[i];
  for (int i = t; i < 2 * pk.n_strips + pk.S; i += 256)
    reinterpret_cast<int32_t*>(tables + kNaStrips)[i] = pk.strips[i];
  for (int i = t; i < dg::kMaxQueues * (pk.n_segs + 1); i += 256)
    reinterpret_cast<int32_t*>(tables + kNaSeg)[i] = pk.seg[i];
  for (int i = t; i < dg::sync_words(pk.S); i += 256) reinterpret_cast<int32_t*>(tables + kNaSync)[i] = 0;
  for (int i = t; i < pk.n_ctr; i += 256) reinterpret_cast<uint32_t*>(tables + kNaCtr)[i] = 0;
}

// Per device: the address of `scratch`, and the device properties a run needs.
struct NoAllocDevice {
  uint8_t* ptr = nullptr;
  int n_cu = 256;
  int64_t clock_khz = 100000;
};
std::mutex g_noalloc_mu;
std::vector<NoAllocDevice> g_noalloc_dev;

int noalloc_device(int dev, NoAllocDevice* out) {
  std::lock_guard<std::mutex> lock(g_noalloc_mu);
  if (static_cast<int>(g_noalloc_dev.size()) <= dev) g_noalloc_dev.resize(dev + 1);
  NoAllocDevice& d = g_noalloc_dev[dev];
  if (!d.ptr) {
    hipDeviceProp_t prop;
    DG_HIP(nullptr, hipGetDeviceProperties(&prop, dev));
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
      return fail(nullptr, DIST_GEMM_ERR_UNSUPPORTED,
                  std::string("this library is built for gfx950 only; device is ") + prop.gcnArchName);
    void* p = nullptr;
    DG_HIP(nullptr, hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return fail(nullptr, DIST_GEMM_ERR_HIP, "hipGetSymbolAddress returned NULL for the scratch array");
    d.n_cu = std::max(1, prop.multiProcessorCount);
    int khz = 0;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) == hipSuccess && khz > 0)
      d.clock_khz = khz;
    {
      // the event that orders single-launch runs on the device, made now so
      // that no later call creates anything
      FusedOrder& o = fused_order();
      std::lock_guard<std::mutex> olock(o.mu);
      if (static_cast<int>(o.tail.size()) <= dev) {
        o.tail.resize(dev + 1, nullptr);
        o.live.resize(dev + 1, 0);
      }
      if (!o.tail[dev]) DG_HIP(nullptr, hipEventCreateWithFlags(&o.tail[dev], hipEventDisableTiming));
    }
    d.ptr = static_cast<uint8_t*>(p);
  }
  *out = d;
  return DIST_GEMM_OK;
}

}  // namespace

extern "C" {

const char* dist_gemm_status_string(int status) {
  switch (status) {
    case DIST_GEMM_OK: return "DIST_GEMM_OK";
    case DIST_GEMM_ERR_INVALID_ARG: return "DIST_GEMM_ERR_INVALID_ARG";
    case DIST_GEMM_ERR_SHAPE: return "DIST_GEMM_ERR_SHAPE";
    case DIST_GEMM_ERR_UNSUPPORTED: return "DIST_GEMM_ERR_UNSUPPORTED";
    case DIST_GEMM_ERR_OOM: return "DIST_GEMM_ERR_OOM";
    case DIST_GEMM_ERR_HIP: return "DIST_GEMM_ERR_HIP";
    default: return "DIST_GEMM_ERR_UNKNOWN";
  }
}

const char* dist_gemm_last_error(dist_gemm_plan_t plan) {
  return plan ? plan->err.c_str() : g_last_error.c_str();
}

int dist_gemm_step_table(int64_t M, int64_t N, int64_t K, int64_t L, int TP, int schedule,
                         int dtype, dist_gemm_step* out, int* n_steps) {
  if (!n_steps) return fail(nullptr, DIST_GEMM_ERR_INVALID_ARG, "n_steps is NULL");
  Problem pr;
  const int rc = validate(M, N, K, L, TP, schedule, dtype, &pr, nullptr);
  if (rc != DIST_GEMM_OK) return rc;
  const std::vector<dist_gemm_step> st = build_steps(pr);
  const int cap = *n_steps;
  if (cap > 0 && !out) return fail(nullptr, DIST_GEMM_ERR_INVALID_ARG, "out is NULL");
  for (int i = 0; i < cap && i < static_cast<int>(st.size()); ++i) out[i] = st[i];
  *n_steps = static_cast<int>(st.size());
  return DIST_GEMM_OK;
}

int dist_gemm_fused_tables(int64_t M, int64_t N, int64_t K, int64_t L, int TP, int schedule, int dtype,
                           int shared_a, int queues, int step_group, int copy_ahead, int64_t copy_chunk,
                           int n_wg, dist_gemm_fused_info* info, int32_t* segs, int64_t* steps,
                           int32_t* strips, int32_t* seg) {
  if (!info) return fail(nullptr, DIST_GEMM_ERR_INVALID_ARG, "info is NULL");
  Problem pr;
  const int rc = validate(M, N, K, L, TP, schedule, dtype, &pr, nullptr);
  if (rc != DIST_GEMM_OK) return rc;
  if (shared_a != 0 && shared_a != 1) return fail(nullptr, DIST_GEMM_ERR_INVALID_ARG, "shared A must be 0 or 1");
  if (queues != 1 && queues != dg::kMaxQueues) return fail(nullptr, DIST_GEMM_ERR_INVALID_ARG, "queues must be 1 or 8");
  if (step_group < 1 || step_group > 1024) return fail(nullptr, DIST_GEMM_ERR_INVALID_ARG, "step group must be 1..1024");
  if (copy_ahead < 0 || copy_ahead > 64) return fail(nullptr, DIST_GEMM_ERR_INVALID_ARG, "copy-ahead segments must be 0..64");
  if (copy_chunk < 4096 || copy_chunk > (int64_t{1} << 28) || copy_chunk % 16 != 0)
    return fail(nullptr, DIST_GEMM_ERR_INVALID_ARG, "copy chunk must be a multiple of 16 in [4096, 2^28]");
  if (n_wg < queues || n_wg % queues != 0)
    return fail(nullptr, DIST_GEMM_ERR_INVALID_ARG, "workgroups must be a positive multiple of the queues");
  if (pr.S < 2 || pr.schedule == DIST_GEMM_MONOLITHIC)
    return fail(nullptr, DIST_GEMM_ERR_UNSUPPORTED, "the single launch needs at least two steps");
  pr.shared_a = shared_a != 0;
  FusedOpts o;
  o.queues = queues;
  o.copy_chunk = copy_chunk;
  o.copy_ahead = copy_ahead;
  o.max_group = step_group;
  o.n_wg = n_wg;
  FusedTables t;
  std::string err;
  const int rc2 = compute_fused(pr, build_steps(pr), o, &t, &err);
  if (rc2 != DIST_GEMM_OK) {
    g_last_error = err;
    return rc2;
  }
  const StripGeom sg = strip_geom(pr);
  const int S = pr.S;
  const int n_strips = static_cast<int>((sg.ext + dg::kBM - 1) / dg::kBM);
  const int G = static_cast<int>(t.segs.size());
  info->n_strips = n_strips;
  info->n_segs = G;
  info->LG = sg.LG;
  info->cols = sg.cols;
  info->strided = sg.strided;
  info->loop = t.loop ? 1 : 0;
  info->n_list0 = t.n_list0;
  info->n_list1 = t.n_list1;
  info->n_local = t.n_local;
  info->strip_bytes = sg.strip_bytes;
  info->ext = sg.ext;
  info->row_bytes = sg.row_bytes;
  info->height = sg.height;
  const int64_t KT = (pr.K * pr.es_in + dg::kRowBytes - 1) / dg::kRowBytes;
  info->loop_capacity = std::max<int64_t>(0, KT - 2) * dg::kLoopCopyBytes;
  if (segs)
    for (int g = 0; g < G; ++g) {
      segs[4 * g + 0] = t.segs[g].strip0;
      segs[4 * g + 1] = t.segs[g].nst;
      segs[4 * g + 2] = t.segs[g].tiles;
      segs[4 * g + 3] = t.segs[g].quota;
    }
  if (steps)
    for (int h = 0; h < S; ++h) {
      const dg::FusedStepCopy& c = t.copies[h];
      int64_t* r = steps + 7 * h;
      r[0] = c.piece; r[1] = c.strip0; r[2] = c.nst; r[3] = c.P; r[4] = c.n_chunks; r[5] = c.wait; r[6] = c.base;
    }
  if (strips) std::copy(t.strips.begin(), t.strips.end(), strips);
  if (seg) std::copy(t.seg.begin(), t.seg.end(), seg);
  return DIST_GEMM_OK;
}

int dist_gemm_plan(int64_t M, int64_t N, int64_t K, int64_t L, int TP, int schedule, int dtype,
                   dist_gemm_plan_t* out) {
  if (!out) return fail(nullptr, DIST_GEMM_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  Problem pr;
  int rc = validate(M, N, K, L, TP, schedule, dtype, &pr, nullptr);
  if (rc != DIST_GEMM_OK) return rc;

  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(nullptr, e, "hipGetDevice");
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return hip_fail(nullptr, e, "hipGetDeviceProperties");
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(nullptr, DIST_GEMM_ERR_UNSUPPORTED,
                std::string("this library is built for gfx950 only; device is ") + prop.gcnArchName);

  auto* P = new dist_gemm_plan_s();
  P->pr = pr;
  P->device = dev;
  P->steps = build_steps(pr);
  P->geom = copy_geom(pr);
  std::string* perr = nullptr;  // errors before the handle is returned go to the thread slot
  const bool rotating = pr.schedule != DIST_GEMM_MONOLITHIC && pr.S > 1;
  if (rotating) {
    e = hipMalloc(&P->staging, P->geom.alloc);
    if (e != hipSuccess) {
      release(P);
      (void)hipGetLastError();
      return fail(perr, DIST_GEMM_ERR_OOM, "staging allocation of " + std::to_string(P->geom.alloc) + " bytes");
    }
  }
  auto mk = [&](hipEvent_t* ev, unsigned flags) { return hipEventCreateWithFlags(ev, flags); };
  e = hipStreamCreateWithFlags(&P->cs2, hipStreamNonBlocking);
  if (e == hipSuccess) e = mk(&P->ev_start, hipEventDisableTiming);
  if (e == hipSuccess) e = mk(&P->ev_cs2_done, hipEventDisableTiming);
  if (e == hipSuccess) e = mk(&P->ev_done, hipEventDisableTiming);
  P->ev_copy.assign(pr.S, nullptr);
  for (int s = 0; s < pr.S && e == hipSuccess; ++s) e = mk(&P->ev_copy[s], hipEventDisableTiming);
  if (e != hipSuccess) {
    release(P);
    return hip_fail(perr, e, "stream/event creation");
  }
  rc = ensure_sides(P, std::min(P->copy_streams, std::max(pr.S - 1, 1)), perr);
  if (rc != DIST_GEMM_OK) {
    release(P);
    return rc;
  }
  P->n_cu = std::max(1, prop.multiProcessorCount);
  int khz = 0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) == hipSuccess && khz > 0)
    P->clock_khz = khz;
  if (rotating) {
    rc = alloc_fused(P, perr);
    if (rc == DIST_GEMM_OK) rc = build_fused(P, perr);
    if (rc != DIST_GEMM_OK) {
      release(P);
      (void)hipGetLastError();
      return rc;
    }
  }
  *out = P;
  return DIST_GEMM_OK;
}

int dist_gemm_set_scales(dist_gemm_plan_t plan, float scale_a, float scale_b) {
  if (!plan) return fail(nullptr, DIST_GEMM_ERR_INVALID_ARG, "plan is NULL");
  if (!std::isfinite(scale_a) || !std::isfinite(scale_b))
    return fail(&plan->err, DIST_GEMM_ERR_INVALID_ARG, "scales must be finite");
  plan->scale_a = scale_a;
  plan->scale_b = scale_b;
  return DIST_GEMM_OK;
}

int dist_gemm_set_result_scale(dist_gemm_plan_t plan, float scale_result) {
  if (!plan) return fail(nullptr, DIST_GEMM_ERR_INVALID_ARG, "plan is NULL");
  if (!std::isfinite(scale_result))
    return fail(&plan->err, DIST_GEMM_ERR_INVALID_ARG, "the result scale must be finite");
  if (plan->pr.out_kind != dg::OUT_E4M3 && scale_result != 1.0f)
    return fail(&plan->err, DIST_GEMM_ERR_UNSUPPORTED,
                "a result scale applies to an fp8 (E4M3) output; this plan's output is not fp8");
  plan->result_scale = scale_result;
  return DIST_GEMM_OK;
}

int dist_gemm_set_bias(dist_gemm_plan_t plan, const void* bias) {
  if (!plan) return fail(nullptr, DIST_GEMM_ERR_INVALID_ARG, "plan is NULL");
  plan->bias = bias;
  return DIST_GEMM_OK;
}

int dist_gemm_set_option(dist_gemm_plan_t plan, int option, int64_t value) {
  if (!plan) return fail(nullptr, DIST_GEMM_ERR_INVALID_ARG, "plan is NULL");
  switch (option) {
    case DIST_GEMM_OPT_COMPUTE_STREAMS:
      if (value != 1 && value != 2)
        return fail(&plan->err, DIST_GEMM_ERR_INVALID_ARG, "compute streams must be 1 or 2");
      plan->compute_streams = static_cast<int>(value);
      return DIST_GEMM_OK;
    case DIST_GEMM_OPT_COPY_ENGINE:
      if (value < 0 || value > 2)
        return fail(&plan->err, DIST_GEMM_ERR_INVALID_ARG, "copy engine must be 0, 1 or 2");
      plan->copy_engine = static_cast<int>(value);
      return DIST_GEMM_OK;
    case DIST_GEMM_OPT_COPY_STREAMS: {
      if (value < 1 || value > 8)
        return fail(&plan->err, DIST_GEMM_ERR_INVALID_ARG, "copy streams must be 1..8");
      DeviceGuard guard(plan->device);
      const int rc = ensure_sides(plan, std::min<int>(static_cast<int>(value),
                                                      std::max(plan->pr.S - 1, 1)), &plan->err);
      if (rc != DIST_GEMM_OK) return rc;
      plan->copy_streams = static_cast<int>(value);
      return DIST_GEMM_OK;
    }
    case DIST_GEMM_OPT_STEP_GROUP: {
      if (value < 1 || value > 1024)
        return fail(&plan->err, DIST_GEMM_ERR_INVALID_ARG, "step group must be 1..1024");
      if (plan->max_group == value) return DIST_GEMM_OK;
      const int old = plan->max_group;
      return change_tables(plan, [&] { plan->max_group = static_cast<int>(value); },
                           [&] { plan->max_group = old; });
    }
    case DIST_GEMM_OPT_EXECUTION:
      if (value != 0 && value != 1)
        return fail(&plan->err, DIST_GEMM_ERR_INVALID_ARG, "execution must be 0 or 1");
      plan->execution = static_cast<int>(value);
      return DIST_GEMM_OK;
    case DIST_GEMM_OPT_QUEUES: {
      if (value != 1 && value != dg::kMaxQueues)
        return fail(&plan->err, DIST_GEMM_ERR_INVALID_ARG, "queues must be 1 or 8");
      if (plan->queues == value) return DIST_GEMM_OK;
      const int old = plan->queues;
      return change_tables(plan, [&] { plan->queues = static_cast<int>(value); },
                           [&] { plan->queues = old; });
    }
    case DIST_GEMM_OPT_COPY_CHUNK: {
      if (value < 4096 || value > (int64_t{1} << 28) || value % 16 != 0)
        return fail(&plan->err, DIST_GEMM_ERR_INVALID_ARG,
                    "copy chunk must be a multiple of 16 in [4096, 2^28]");
      if (plan->copy_chunk == value) return DIST_GEMM_OK;
      const int64_t old = plan->copy_chunk;
      return change_tables(plan, [&] { plan->copy_chunk = value; }, [&] { plan->copy_chunk = old; });
    }
    case DIST_GEMM_OPT_COPY_AHEAD: {
      if (value < 0 || value > 64)
        return fail(&plan->err, DIST_GEMM_ERR_INVALID_ARG, "copy-ahead segments must be 0..64");
      if (plan->copy_ahead == value) return DIST_GEMM_OK;
      const int old = plan->copy_ahead;
      return change_tables(plan, [&] { plan->copy_ahead = static_cast<int>(value); },
                           [&] { plan->copy_ahead = old; });
    }
    case DIST_GEMM_OPT_SHARED_A: {
      if (value != 0 && value != 1)
        return fail(&plan->err, DIST_GEMM_ERR_INVALID_ARG, "shared A must be 0 or 1");
      if (plan->pr.shared_a == (value != 0)) return DIST_GEMM_OK;
      auto flip = [&] {
        plan->pr.shared_a = !plan->pr.shared_a;
        plan->geom = copy_geom(plan->pr);
      };
      return change_tables(plan, flip, flip);
    }
    case DIST_GEMM_OPT_WAIT_LIMIT_US:
      if (value < 0 || value > 100000000)
        return fail(&plan->err, DIST_GEMM_ERR_INVALID_ARG, "wait limit must be in [0, 1e8] us");
      plan->wait_limit_us = value;
      return DIST_GEMM_OK;
    case DIST_GEMM_OPT_FAST_ACCUM:
      if (value != 0 && value != 1)
        return fail(&plan->err, DIST_GEMM_ERR_INVALID_ARG, "fast accumulate must be 0 or 1");
      plan->fast_accum = static_cast<int>(value);
      return DIST_GEMM_OK;
    case DIST_GEMM_OPT_HALF_TILES:
      if (value != 0 && value != 1)
        return fail(&plan->err, DIST_GEMM_ERR_INVALID_ARG, "half tiles must be 0 or 1");
      plan->half_tiles = static_cast<int>(value);
      return DIST_GEMM_OK;
    case DIST_GEMM_OPT_COPY_DELAY_US:
      if (value < 0 || value > 1000000)
        return fail(&plan->err, DIST_GEMM_ERR_INVALID_ARG, "copy delay must be in [0, 1e6] us");
      plan->copy_delay_us = value;
      return DIST_GEMM_OK;
    case DIST_GEMM_OPT_STEP_TIMING: {
      if (value < 0 || value > 4096)
        return fail(&plan->err, DIST_GEMM_ERR_INVALID_ARG, "step timing keeps 0..4096 runs");
      DeviceGuard guard(plan->device);
      if (plan->ev_done && plan->has_prev) (void)hipEventSynchronize(plan->ev_done);
      for (hipEvent_t ev : plan->t_begin) if (ev) (void)hipEventDestroy(ev);
      for (hipEvent_t ev : plan->t_end) if (ev) (void)hipEventDestroy(ev);
      for (hipEvent_t ev : plan->t_run0) if (ev) (void)hipEventDestroy(ev);
      for (hipEvent_t ev : plan->t_copy) if (ev) (void)hipEventDestroy(ev);
      if (plan->d_times) (void)hipFree(plan->d_times);
      plan->d_times = nullptr;
      plan->t_first.clear();
      plan->t_fused.clear();
      plan->t_begin.clear();
      plan->t_end.clear();
      plan->t_run0.clear();
      plan->t_copy.clear();
      plan->step_timing = 0;
      plan->timed_runs = 0;
      if (value == 0) return DIST_GEMM_OK;
      const size_t n = static_cast<size_t>(value) * plan->steps.size();
      plan->t_begin.assign(n, nullptr);
      plan->t_end.assign(n, nullptr);
      plan->t_copy.assign(n, nullptr);
      plan->t_first.assign(n, 0);
      plan->t_fused.assign(static_cast<size_t>(value), 0);
      plan->t_run0.assign(static_cast<size_t>(value), nullptr);
      for (size_t i = 0; i < n; ++i) {
        hipError_t e = hipEventCreate(&plan->t_begin[i]);
        if (e == hipSuccess) e = hipEventCreate(&plan->t_end[i]);
        if (e == hipSuccess) e = hipEventCreate(&plan->t_copy[i]);
        if (e != hipSuccess) return hip_fail(&plan->err, e, "timing event creation");
      }
      for (hipEvent_t& ev : plan->t_run0) {
        const hipError_t e = hipEventCreate(&ev);
        if (e != hipSuccess) return hip_fail(&plan->err, e, "timing event creation");
      }
      if (plan->d_segs) {
        const size_t words = static_cast<size_t>(value) * dg::timeline_words(plan->pr.S);
        DG_HIP(&plan->err, hipMalloc(&plan->d_times, words * sizeof(uint64_t)));
        DG_HIP(&plan->err, hipMemset(plan->d_times, 0, words * sizeof(uint64_t)));
      }
      plan->step_timing = static_cast<int>(value);
      return DIST_GEMM_OK;
    }
    default:
      return fail(&plan->err, DIST_GEMM_ERR_INVALID_ARG, "unknown option " + std::to_string(option));
  }
}

namespace {

int run_impl(dist_gemm_plan_t plan, const void* A, const void* B, const void* C, void* D, void* ag_out,
             float alpha, float beta, void* stream) {
  if (!plan) return fail(nullptr, DIST_GEMM_ERR_INVALID_ARG, "plan is NULL");
  dist_gemm_plan_s* P = plan;
  const Problem& pr = P->pr;
  if (!A || !B || !D) return fail(&P->err, DIST_GEMM_ERR_INVALID_ARG, "A, B and D must be non-NULL");
  if (beta != 0.0f && !C) return fail(&P->err, DIST_GEMM_ERR_INVALID_ARG, "C is NULL but beta != 0");
  if (!std::isfinite(alpha) || !std::isfinite(beta))
    return fail(&P->err, DIST_GEMM_ERR_INVALID_ARG, "alpha and beta must be finite");
  if (D == A || D == B) return fail(&P->err, DIST_GEMM_ERR_INVALID_ARG, "D must not alias A or B");
  const bool ag = pr.schedule == DIST_GEMM_AG_ROT_A || pr.schedule == DIST_GEMM_AG_ROT_B;
  if (ag_out) {
    if (!ag)
      return fail(&P->err, DIST_GEMM_ERR_INVALID_ARG,
                  "a gathered output exists only for the all-gather schedules");
    if (ag_out == A || ag_out == B || ag_out == C || ag_out == D)
      return fail(&P->err, DIST_GEMM_ERR_INVALID_ARG, "ag_out must not alias A, B, C or D");
  }

  DeviceGuard guard(P->device);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  DG_HIP(&P->err, hipStreamIsCapturing(st, &cap));
  if (cap != hipStreamCaptureStatusNone) P->captured = true;
  const bool rotating = pr.schedule != DIST_GEMM_MONOLITHIC && pr.S > 1;
  // a reduce-scatter with beta = 0 reads no partial: nothing rotates
  const bool copy_on = rotating && !(reduce_scatter(pr.schedule) && beta == 0.0f);
  const bool two = P->compute_streams == 2 && pr.S > 1;
  const float alpha_eff =
      (pr.in_kind == dg::IN_E4M3) ? alpha * P->scale_a * P->scale_b : alpha;
  const void* copy_src = pr.schedule == DIST_GEMM_AG_ROT_A ? A : pr.schedule == DIST_GEMM_AG_ROT_B ? B : C;
  uint8_t* G = ag_out ? static_cast<uint8_t*>(ag_out) : P->staging;

  if (rotating && P->execution == 1) {
    if (P->has_prev && P->prev_stream != st) DG_HIP(&P->err, hipStreamWaitEvent(st, P->ev_done, 0));
    const size_t trun = P->step_timing ? static_cast<size_t>(P->timed_runs % P->step_timing) : 0;
    const size_t tbase = trun * P->steps.size();
    uint64_t* times = nullptr;
    uint64_t* times_next = nullptr;
    if (P->step_timing) {
      // every slot starts zeroed (at allocation); a launch zeroes the next
      // slot of the ring at its end (one slot: zeroed before the launch)
      const size_t words = dg::timeline_words(pr.S);
      times = P->d_times + trun * words;
      DG_HIP(&P->err, hipEventRecord(P->t_run0[trun], st));
      if (P->step_timing > 1)
        times_next = P->d_times + ((trun + 1) % P->step_timing) * words;
      else
        DG_HIP(&P->err, hipMemsetAsync(times, 0, words * sizeof(uint64_t), st));
      for (size_t k = 0; k < P->steps.size(); ++k) P->t_first[tbase + k] = 0;
      P->t_fused[trun] = 1;
      DG_HIP(&P->err, hipEventRecord(P->t_begin[tbase], st));
    }
    const int rc = run_fused(P, st, A, B, C, D, G, alpha_eff, beta, copy_src, copy_on, ag_out != nullptr, times,
                             times_next);
    if (rc != DIST_GEMM_OK) return rc;
    if (P->step_timing) DG_HIP(&P->err, hipEventRecord(P->t_end[tbase], st));
    DG_HIP(&P->err, hipEventRecord(P->ev_done, st));
    P->has_prev = true;
    P->prev_stream = st;
    if (P->step_timing) ++P->timed_runs;
    return DIST_GEMM_OK;
  }

  // side streams in use: the first n, n = min(copy streams, staged copies)
  const int n_copies = (copy_on ? pr.S - 1 : 0) + (ag_out ? 1 : 0);
  const int n_side = n_copies > 0 ? std::max(1, std::min(P->copy_streams, std::max(pr.S - 1, 1))) : 0;
  if (n_side > 0) {
    const int rc = ensure_sides(P, n_side, &P->err);
    if (rc != DIST_GEMM_OK) return rc;
  }

  if (P->has_prev && P->prev_stream != st) DG_HIP(&P->err, hipStreamWaitEvent(st, P->ev_done, 0));
  DG_HIP(&P->err, hipEventRecord(P->ev_start, st));
  const size_t trun = P->step_timing ? static_cast<size_t>(P->timed_runs % P->step_timing) : 0;
  const size_t tbase = trun * P->steps.size();
  if (P->step_timing) {
    DG_HIP(&P->err, hipEventRecord(P->t_run0[trun], st));
    P->t_fused[trun] = copy_on ? 0 : 2;  // 2: step launches, nothing copied
  }
  for (int k = 0; k < n_side; ++k) DG_HIP(&P->err, hipStreamWaitEvent(P->sides[k], P->ev_start, 0));
  if (two) DG_HIP(&P->err, hipStreamWaitEvent(P->cs2, P->ev_start, 0));
  if (P->copy_delay_us > 0)
    for (int k = 0; k < n_side; ++k) {
      hipLaunchKernelGGL(copy_delay_kernel, dim3(1), dim3(1), 0, P->sides[k],
                         static_cast<uint64_t>(P->copy_delay_us * P->clock_khz / 1000));
      DG_HIP(&P->err, hipGetLastError());
    }

  // Copy engine: every staged operand, in step order, round-robin over the
  // side streams, one event per copy; with a gathered output, the local
  // shard last.
  if (copy_on) {
    for (const dist_gemm_step& s : P->steps) {
      if (!s.staged) continue;
      hipStream_t side = P->sides[(s.step - 1) % n_side];
      int rc = enqueue_copy(P, side, copy_src, G, s.shard);
      if (rc != DIST_GEMM_OK) return rc;
      DG_HIP(&P->err, hipEventRecord(P->ev_copy[s.step], side));
      if (P->step_timing) DG_HIP(&P->err, hipEventRecord(P->t_copy[tbase + s.step], side));
    }
  }
  if (ag_out) {
    const int rc = enqueue_copy(P, P->sides[0], copy_src, G, P->steps[0].shard);
    if (rc != DIST_GEMM_OK) return rc;
  }
  // Step GEMMs: one launch per group, alternating compute streams by launch.
  const std::vector<LaunchGroup> groups = group_steps(P);
  for (size_t gi = 0; gi < groups.size(); ++gi) {
    const LaunchGroup& grp = groups[gi];
    hipStream_t cs = (two && (gi & 1)) ? P->cs2 : st;
    for (int k = grp.first; k < grp.first + grp.count; ++k) {
      if (copy_on && P->steps[k].staged) DG_HIP(&P->err, hipStreamWaitEvent(cs, P->ev_copy[k], 0));
      if (P->step_timing) P->t_first[tbase + k] = grp.first;
    }
    if (P->step_timing) DG_HIP(&P->err, hipEventRecord(P->t_begin[tbase + grp.first], cs));
    const dg::GemmParams g = group_params(P, grp, A, B, C, D, copy_on ? G : nullptr, alpha_eff, beta);
    DG_HIP(&P->err, dg::launch_gemm(pr.in_kind, pr.out_kind, g, cs));
    if (P->step_timing) DG_HIP(&P->err, hipEventRecord(P->t_end[tbase + grp.first], cs));
  }
  // Join the side streams back into the caller's stream.
  for (int k = 0; k < n_side; ++k) {
    DG_HIP(&P->err, hipEventRecord(P->ev_side_done[k], P->sides[k]));
    DG_HIP(&P->err, hipStreamWaitEvent(st, P->ev_side_done[k], 0));
  }
  if (two) {
    DG_HIP(&P->err, hipEventRecord(P->ev_cs2_done, P->cs2));
    DG_HIP(&P->err, hipStreamWaitEvent(st, P->ev_cs2_done, 0));
  }
  DG_HIP(&P->err, hipEventRecord(P->ev_done, st));
  P->has_prev = true;
  P->prev_stream = st;
  if (P->step_timing) ++P->timed_runs;
  return DIST_GEMM_OK;
}

}  // namespace

int dist_gemm_run(dist_gemm_plan_t plan, const void* A, const void* B, const void* C, void* D,
                  float alpha, float beta, void* stream) {
  return run_impl(plan, A, B, C, D, nullptr, alpha, beta, stream);
}

int dist_gemm_run_ag(dist_gemm_plan_t plan, const void* A, const void* B, const void* C, void* D,
                     void* ag_out, float alpha, float beta, void* stream) {
  if (!ag_out) return fail(plan ? &plan->err : nullptr, DIST_GEMM_ERR_INVALID_ARG, "ag_out is NULL");
  return run_impl(plan, A, B, C, D, ag_out, alpha, beta, stream);
}

int dist_gemm_plan_steps(dist_gemm_plan_t plan, dist_gemm_step* out, int* n_steps) {
  if (!plan || !n_steps) return fail(nullptr, DIST_GEMM_ERR_INVALID_ARG, "plan or n_steps is NULL");
  const int cap = *n_steps;
  if (cap > 0 && !out) return fail(&plan->err, DIST_GEMM_ERR_INVALID_ARG, "out is NULL");
  for (int i = 0; i < cap && i < static_cast<int>(plan->steps.size()); ++i) out[i] = plan->steps[i];
  *n_steps = static_cast<int>(plan->steps.size());
  return DIST_GEMM_OK;
}

int dist_gemm_step_times(dist_gemm_plan_t plan, float* ms, int* n) {
  if (!plan || !n) return fail(nullptr, DIST_GEMM_ERR_INVALID_ARG, "plan or n is NULL");
  if (!plan->step_timing || plan->timed_runs == 0)
    return fail(&plan->err, DIST_GEMM_ERR_UNSUPPORTED, "no timed run recorded");
  DeviceGuard guard(plan->device);
  const int64_t S = static_cast<int64_t>(plan->steps.size());
  const int64_t R = std::min<int64_t>(plan->timed_runs, plan->step_timing);
  const int64_t cap = *n;
  if (cap > 0 && !ms) return fail(&plan->err, DIST_GEMM_ERR_INVALID_ARG, "ms is NULL");
  DG_HIP(&plan->err, hipEventSynchronize(plan->ev_done));
  int64_t w = 0;
  for (int64_t r = plan->timed_runs - R; r < plan->timed_runs; ++r) {
    const size_t base = static_cast<size_t>(r % plan->step_timing) * S;
    for (int64_t s = 0; s < S; ++s, ++w) {
      if (w >= cap) continue;
      const int f = plan->t_first[base + s];
      int members = 0;
      for (int64_t k = 0; k < S; ++k) members += plan->t_first[base + k] == f;
      float t = 0.0f;
      DG_HIP(&plan->err, hipEventElapsedTime(&t, plan->t_begin[base + f], plan->t_end[base + f]));
      ms[w] = t / static_cast<float>(members);
    }
  }
  *n = static_cast<int>(R * S);
  return DIST_GEMM_OK;
}

int dist_gemm_step_timeline(dist_gemm_plan_t plan, float* ms, int* n) {
  if (!plan || !n) return fail(nullptr, DIST_GEMM_ERR_INVALID_ARG, "plan or n is NULL");
  if (!plan->step_timing || plan->timed_runs == 0)
    return fail(&plan->err, DIST_GEMM_ERR_UNSUPPORTED, "no timed run recorded");
  DeviceGuard guard(plan->device);
  const int64_t S = static_cast<int64_t>(plan->steps.size());
  const int64_t cap = *n;
  if (cap > 0 && !ms) return fail(&plan->err, DIST_GEMM_ERR_INVALID_ARG, "ms is NULL");
  DG_HIP(&plan->err, hipEventSynchronize(plan->ev_done));
  const size_t run = static_cast<size_t>((plan->timed_runs - 1) % plan->step_timing);
  const size_t base = run * static_cast<size_t>(S);
  hipEvent_t t0 = plan->t_run0[run];
  std::vector<float> v(3 * S, -1.0f);
  if (plan->t_fused[run] == 1 && plan->d_times) {
    // one launch: the device's own stamps (wall-clock ticks), placed on the
    // run's time line by the launch's start event
    const size_t words = dg::timeline_words(plan->pr.S);
    std::vector<uint64_t> t(words);
    DG_HIP(&plan->err, hipMemcpy(t.data(), plan->d_times + run * words, words * sizeof(uint64_t),
                                 hipMemcpyDeviceToHost));
    float launch0 = 0.0f;
    DG_HIP(&plan->err, hipEventElapsedTime(&launch0, t0, plan->t_begin[base]));
    const uint64_t start = ~t[0];
    const double per_ms = static_cast<double>(plan->clock_khz);
    auto at = [&](uint64_t tick) {
      return static_cast<float>(launch0 + static_cast<double>(static_cast<int64_t>(tick - start)) / per_ms);
    };
    for (int64_t s = 0; s < S; ++s) {
      if (t[1 + 3 * s]) v[3 * s] = at(t[1 + 3 * s]);
      if (t[2 + 3 * s]) v[3 * s + 1] = at(~t[2 + 3 * s]);
      if (t[3 + 3 * s]) v[3 * s + 2] = at(t[3 + 3 * s]);
    }
  } else {
    for (int64_t s = 0; s < S; ++s) {
      const bool staged = plan->steps[s].staged && plan->pr.schedule != DIST_GEMM_MONOLITHIC &&
                          plan->t_fused[run] == 0;
      if (staged) DG_HIP(&plan->err, hipEventElapsedTime(&v[3 * s], t0, plan->t_copy[base + s]));
      const int f = plan->t_first[base + s];
      DG_HIP(&plan->err, hipEventElapsedTime(&v[3 * s + 1], t0, plan->t_begin[base + f]));
      DG_HIP(&plan->err, hipEventElapsedTime(&v[3 * s + 2], t0, plan->t_end[base + f]));
    }
  }
  for (int64_t k = 0; k < 3 * S && k < cap; ++k) ms[k] = v[k];
  *n = static_cast<int>(3 * S);
  return DIST_GEMM_OK;
}

int dist_gemm_device_errors(dist_gemm_plan_t plan, int64_t* count) {
  if (!plan || !count) return fail(nullptr, DIST_GEMM_ERR_INVALID_ARG, "plan or count is NULL");
  *count = 0;
  if (!plan->d_sync) return DIST_GEMM_OK;
  DeviceGuard guard(plan->device);
  if (plan->has_prev) DG_HIP(&plan->err, hipEventSynchronize(plan->ev_done));
  int32_t v = 0;
  const size_t at = static_cast<size_t>(dg::kSyncErr) * dg::kSyncStride;
  DG_HIP(&plan->err, hipMemcpy(&v, plan->d_sync + at, sizeof(v), hipMemcpyDeviceToHost));
  *count = v;
  return DIST_GEMM_OK;
}

int dist_gemm_destroy(dist_gemm_plan_t plan) {
  if (!plan) return DIST_GEMM_OK;
  DeviceGuard guard(plan->device);
  release(plan);
  return DIST_GEMM_OK;
}

int dist_gemm_run_noalloc(int64_t M, int64_t N, int64_t K, int64_t L, int TP, int schedule, int dtype,
                          const void* A, const void* B, const void* C, void* D, float alpha, float beta,
                          float scale_a, float scale_b, void* stream) {
  Problem pr;
  int rc = validate(M, N, K, L, TP, schedule, dtype, &pr, nullptr);
  if (rc != DIST_GEMM_OK) return rc;
  if (!A || !B || !D) return fail(nullptr, DIST_GEMM_ERR_INVALID_ARG, "A, B and D must be non-NULL");
  if (beta != 0.0f && !C) return fail(nullptr, DIST_GEMM_ERR_INVALID_ARG, "C is NULL but beta != 0");
  if (!std::isfinite(alpha) || !std::isfinite(beta) || !std::isfinite(scale_a) || !std::isfinite(scale_b))
    return fail(nullptr, DIST_GEMM_ERR_INVALID_ARG, "alpha, beta and the scales must be finite");
  if (D == A || D == B) return fail(nullptr, DIST_GEMM_ERR_INVALID_ARG, "D must not alias A or B");
  const std::vector<dist_gemm_step> steps = build_steps(pr);
  const bool rotating = pr.schedule != DIST_GEMM_MONOLITHIC && pr.S > 1;
  const CopyGeom cg = copy_geom(pr);
  const StripGeom sgeo = strip_geom(pr);
  const int n_strips = rotating ? static_cast<int>((sgeo.ext + dg::kBM - 1) / dg::kBM) : 0;
  const int64_t n_ctr = rotating ? static_cast<int64_t>(pr.L) * (n_strips + pr.S) : 0;
  if (rotating && (pr.S > kNoAllocMaxSteps || n_strips > kNoAllocMaxStrips || cg.alloc > kNoAllocGatherBytes ||
                   kNaCtr + static_cast<size_t>(n_ctr) * sizeof(uint32_t) > kNoAllocTableBytes))
    return fail(nullptr, DIST_GEMM_ERR_UNSUPPORTED,
                "dist_gemm_run_noalloc handles at most " + std::to_string(kNoAllocMaxSteps) + " steps, " +
                    std::to_string(kNoAllocMaxStrips) + " strips of 256 along the rotated dimension, a " +
                    std::to_string(kNoAllocGatherBytes >> 20) + " MiB gathered operand and " +
                    std::to_string((kNoAllocTableBytes - kNaCtr) / 4) + " strip counters; this problem needs " +
                    std::to_string(pr.S) + " steps, " + std::to_string(n_strips) + " strips, " +
                    std::to_string(cg.alloc) + " bytes and " + std::to_string(n_ctr) + " counters");
  int dev = 0;
  DG_HIP(nullptr, hipGetDevice(&dev));
  NoAllocDevice nd;
  rc = noalloc_device(dev, &nd);
  if (rc != DIST_GEMM_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const float alpha_eff = (pr.in_kind == dg::IN_E4M3) ? alpha * scale_a * scale_b : alpha;
  if (!rotating) {
    // one GEMM over the whole problem: no scratch
    dg::GemmParams g{};
    g.A = A; g.B = B; g.C = beta != 0.0f ? C : nullptr; g.D = D; g.bias = nullptr;
    g.lda = pr.K; g.ldb = pr.K; g.ldc = pr.N; g.ldd = pr.N;
    g.sA = pr.M * pr.K; g.sB = pr.N * pr.K; g.sC = pr.M * pr.N; g.sD = pr.M * pr.N;
    g.M = static_cast<int32_t>(pr.M); g.N = static_cast<int32_t>(pr.N);
    g.K = static_cast<int32_t>(pr.K); g.L = static_cast<int32_t>(pr.L);
    g.alpha = alpha_eff; g.beta = beta; g.post = 1.0f;
    g.tail_cus = nd.n_cu / dg::kNumXcd;
    DG_HIP(nullptr, dg::launch_gemm(pr.in_kind, pr.out_kind, g, st));
    return DIST_GEMM_OK;
  }
  FusedTables t;
  FusedOpts fo;
  fo.n_wg = std::max(dg::kMaxQueues, nd.n_cu / dg::kMaxQueues * dg::kMaxQueues);
  rc = compute_fused(pr, steps, fo, &t, nullptr);
  if (rc != DIST_GEMM_OK) return rc;
  NoAllocPack pk{};
  for (size_t i = 0; i < t.segs.size(); ++i) pk.segs[i] = t.segs[i];
  for (size_t i = 0; i < t.copies.size(); ++i) pk.copies[i] = t.copies[i];
  for (size_t i = 0; i < t.strips.size(); ++i) pk.strips[i] = t.strips[i];
  for (size_t i = 0; i < t.seg.size(); ++i) pk.seg[i] = t.seg[i];
  pk.n_segs = static_cast<int32_t>(t.segs.size());
  pk.n_strips = n_strips;
  pk.S = pr.S;
  pk.n_ctr = static_cast<int32_t>(n_ctr);
  uint8_t* const tables = nd.ptr + kNoAllocGatherBytes;
  FusedDevice dv{reinterpret_cast<const dg::FusedSeg*>(tables + kNaSegs),
                 reinterpret_cast<const dg::FusedStepCopy*>(tables + kNaCopies),
                 reinterpret_cast<const int32_t*>(tables + kNaStrips), reinterpret_cast<const int32_t*>(tables + kNaSeg),
                 reinterpret_cast<uint32_t*>(tables + kNaCtr), reinterpret_cast<int32_t*>(tables + kNaSync),
                 n_strips, pk.n_segs, t.align, t.n_list0, t.n_list1, t.n_local, t.loop};
  const bool copy_on = !(reduce_scatter(pr.schedule) && beta == 0.0f);
  const void* copy_src = pr.schedule == DIST_GEMM_AG_ROT_A ? A : pr.schedule == DIST_GEMM_AG_ROT_B ? B : C;
  const int64_t spin = int64_t{1000000} * nd.clock_khz / 1000;  // 1 s, as the plans' default
  const dg::FusedArgs a = fused_args(pr, dv, dg::kMaxQueues, A, B, C, D, nullptr, nd.ptr, alpha_eff, beta,
                                     1.0f, copy_src, copy_on, false, spin, 0);
  const int grid = std::max(dg::kMaxQueues, nd.n_cu / dg::kMaxQueues * dg::kMaxQueues);
  std::string err;
  rc = launch_ordered(dev, pr.in_kind, pr.out_kind, a, grid, st, &err, [&]() -> int {
    hipLaunchKernelGGL(noalloc_setup_kernel, dim3(1), dim3(256), 0, st, pk, tables);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? DIST_GEMM_OK : hip_fail(&err, e, "no-alloc table setup");
  });
  if (rc != DIST_GEMM_OK) g_last_error = err;
  return rc;
}

}  // extern "C"
