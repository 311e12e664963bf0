// Host side of the TP-step GEMM library: validation, the step table, the
// plan (staging slots, streams, events), the side-stream shard-copy engine
// and the C ABI declared in include/distgemm.h.
//
// Mechanism (Distributed GEMM pull-request page, description): the operand
// that arrives from a peer at every step is moved while the GEMM of the
// current step runs, and each step's GEMM starts only after its operand is
// in place.  On one GPU the peer's shard is a region of the caller's
// operand, moved by a device-to-device hipMemcpyAsync into a staging slot on
// a side stream, one copy per staged step, each followed by an event that
// the launch computing the step waits on.  Copies go round-robin to up to
// eight side streams, one per peer link that the transfer stands in for.
// The copy is the library's streaming copy kernel by default (it runs
// between GEMM workgroups); the runtime's device copy and the SDMA engine
// (NoCU) are options -- measured, SDMA slows several-fold while the GEMMs
// load memory.
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
    st.slot = s > 0 ? s - 1 : -1;
    if (rows) {
      st.m0 = j * w; st.m1 = (j + 1) * w; st.n0 = 0; st.n1 = p.N;
    } else {
      st.m0 = 0; st.m1 = p.M; st.n0 = j * w; st.n1 = (j + 1) * w;
    }
    v.push_back(st);
  }
  return v;
}

// Geometry of one staged shard: a 2-D region (height rows of width bytes,
// src_pitch apart) of the source operand.  The staging buffer is height rows
// of S-1 slots side by side: slot k occupies bytes [k*width, (k+1)*width) of
// every staging row, and staging rows are (S-1)*width apart.  Consecutive
// slots are therefore one contiguous region of every row, so the shards of
// consecutive steps form one operand (or partial) matrix and their GEMMs can
// run as one launch.
struct CopyGeom {
  size_t width = 0, height = 0, src_pitch = 0;
  size_t staging_pitch(int slots) const { return width * static_cast<size_t>(slots); }
};

CopyGeom copy_geom(const Problem& p) {
  CopyGeom g;
  const size_t S = static_cast<size_t>(p.S);
  switch (p.schedule) {
    case DIST_GEMM_AG_ROT_A:  // A row shard, per batch contiguous (one batch if A is shared)
      g.width = static_cast<size_t>(p.M / S) * p.K * p.es_in;
      g.height = p.shared_a ? 1 : p.L;
      g.src_pitch = static_cast<size_t>(p.M) * p.K * p.es_in;
      break;
    case DIST_GEMM_AG_ROT_B:  // B column shard = rows of the N x K storage
      g.width = static_cast<size_t>(p.N / S) * p.K * p.es_in;
      g.height = p.L;
      g.src_pitch = static_cast<size_t>(p.N) * p.K * p.es_in;
      break;
    case DIST_GEMM_RS_TILE_A_ROT_C:  // C row chunk
      g.width = static_cast<size_t>(p.M / S) * p.N * p.es_out;
      g.height = p.L;
      g.src_pitch = static_cast<size_t>(p.M) * p.N * p.es_out;
      break;
    case DIST_GEMM_RS_TILE_B_ROT_C:  // C column chunk: one strip per row
      g.width = static_cast<size_t>(p.N / S) * p.es_out;
      g.height = static_cast<size_t>(p.L) * p.M;
      g.src_pitch = static_cast<size_t>(p.N) * p.es_out;
      break;
    default:
      break;
  }
  return g;
}

}  // namespace

struct dist_gemm_plan_s {
  Problem pr;
  std::vector<dist_gemm_step> steps;
  CopyGeom geom;
  int device = 0;
  uint8_t* staging = nullptr;
  size_t staging_pitch = 0;  // bytes between staging rows: (S-1) slots of geom.width
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
  // Single-launch execution: device tables and counters (rotating plans only).
  int execution = 1;
  int queues = dg::kMaxQueues;
  int64_t copy_chunk = 2 << 20;
  int64_t wait_limit_us = 1000000;
  int64_t clock_khz = 100000;  // device wall clock rate
  int n_cu = 256;
  dg::FusedStep* d_steps = nullptr;
  int32_t* d_seg = nullptr;   // [queues][S + 1] then [queues][S] copy counts
  int32_t* d_sync = nullptr;
  uint64_t fused_align = 0;   // OR of the chunk widths (copy unit choice)
  int fused_groups = 0;       // launch groups in the device tables
  int copy_ahead = 4;         // copy lookahead, launch groups
  std::vector<char> t_fused;  // [run % step_timing]: the run was one launch
  float scale_a = 1.0f, scale_b = 1.0f;
  const void* bias = nullptr;  // device, N values of the output type, or NULL
  int compute_streams = 2;
  int copy_engine = 2;  // library streaming copy kernel
  int copy_streams = 2;
  int max_group = 2;  // consecutive staged steps per launch
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
  if (p->d_steps) (void)hipFree(p->d_steps);
  if (p->d_seg) (void)hipFree(p->d_seg);
  if (p->d_sync) (void)hipFree(p->d_sync);
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

int enqueue_copy(dist_gemm_plan_s* P, hipStream_t side, const void* src_base, int shard, int slot) {
  const CopyGeom& g = P->geom;
  const Problem& pr = P->pr;
  const uint8_t* src = static_cast<const uint8_t*>(src_base);
  switch (pr.schedule) {
    case DIST_GEMM_AG_ROT_A:
    case DIST_GEMM_AG_ROT_B:
    case DIST_GEMM_RS_TILE_A_ROT_C:
      src += static_cast<size_t>(shard) * g.width;
      break;
    case DIST_GEMM_RS_TILE_B_ROT_C:
      src += static_cast<size_t>(shard) * g.width;  // column offset within each row
      break;
    default:
      return DIST_GEMM_OK;
  }
  uint8_t* dst = P->staging + static_cast<size_t>(slot) * g.width;
  hipError_t e;
  if (P->copy_engine == 2) {
    e = launch_shard_copy(dst, P->staging_pitch, src, g.src_pitch, g.width, g.height, side);
    if (e != hipSuccess) return hip_fail(&P->err, e, "shard copy kernel");
    return DIST_GEMM_OK;
  }
  const hipMemcpyKind kind =
      P->copy_engine == 0 ? hipMemcpyDeviceToDeviceNoCU : hipMemcpyDeviceToDevice;
  if (g.height == 1)
    e = hipMemcpyAsync(dst, src, g.width, kind, side);
  else
    e = hipMemcpy2DAsync(dst, P->staging_pitch, src, g.src_pitch, g.width, g.height, kind, side);
  if (e != hipSuccess) return hip_fail(&P->err, e, "shard copy");
  return DIST_GEMM_OK;
}

// Launches of one run: consecutive staged steps whose shards are adjacent
// (shard index and staging slot both one higher) merge, up to max_group
// steps per launch; the unstaged step launches alone.
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
      const bool adjacent = s.staged && prev.staged && s.slot == prev.slot + 1 &&
                            s.shard == prev.shard + 1;
      if (adjacent && b.count < P->max_group) {
        ++b.count;
        continue;
      }
    }
    v.push_back({i, 1});
  }
  return v;
}

// Where step st's operands live: byte offsets from the caller's operands,
// or (staged*) from the staging buffer, with leading dimensions and batch
// strides in elements.
struct StepLayout {
  int64_t offA, offB, offC, offD, offBias;
  int64_t lda, ldb, ldc, ldd, sA, sB, sC, sD;
  int32_t M, N;
  bool stagedA, stagedB, stagedC;
};

StepLayout step_layout(const dist_gemm_plan_s* P, const dist_gemm_step& st) {
  const Problem& pr = P->pr;
  const int64_t M = pr.M, N = pr.N, K = pr.K;
  const int64_t S = pr.S;
  const int ei = pr.es_in, eo = pr.es_out;
  const int64_t slot = st.staged ? static_cast<int64_t>(st.slot) * P->geom.width : 0;
  const int64_t slots = S - 1;
  StepLayout y{};
  y.M = static_cast<int32_t>(st.m1 - st.m0);
  y.N = static_cast<int32_t>(st.n1 - st.n0);
  // defaults: operands in place
  y.offA = st.m0 * K * ei;  y.lda = K; y.sA = pr.shared_a ? 0 : M * K;
  y.offB = st.n0 * K * ei;  y.ldb = K; y.sB = N * K;
  y.offC = (st.m0 * N + st.n0) * eo; y.ldc = N; y.sC = M * N;
  y.offD = (st.m0 * N + st.n0) * eo; y.ldd = N; y.sD = M * N;
  y.offBias = st.n0 * eo;
  if (st.staged) {
    switch (pr.schedule) {
      case DIST_GEMM_AG_ROT_A:
        y.stagedA = true; y.offA = slot; y.sA = pr.shared_a ? 0 : slots * (M / S) * K; break;
      case DIST_GEMM_AG_ROT_B: y.stagedB = true; y.offB = slot; y.sB = slots * (N / S) * K; break;
      case DIST_GEMM_RS_TILE_A_ROT_C:
        y.stagedC = true; y.offC = slot; y.ldc = N; y.sC = slots * (M / S) * N; break;
      case DIST_GEMM_RS_TILE_B_ROT_C:
        y.stagedC = true; y.offC = slot; y.ldc = slots * (N / S); y.sC = M * slots * (N / S); break;
      default: break;
    }
  }
  return y;
}

// GEMM parameters of one step.
dg::GemmParams step_params(const dist_gemm_plan_s* P, const dist_gemm_step& st, const void* A,
                           const void* B, const void* C, void* D, float alpha, float beta) {
  const StepLayout y = step_layout(P, st);
  const uint8_t* stg = P->staging;
  dg::GemmParams g{};
  g.K = static_cast<int32_t>(P->pr.K);
  g.L = static_cast<int32_t>(P->pr.L);
  g.alpha = alpha;
  g.beta = beta;
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
// adjacent in the source operand, in the staging buffer and in D, so the
// extended views address exactly the member steps' data.
dg::GemmParams group_params(const dist_gemm_plan_s* P, const LaunchGroup& grp, const void* A,
                            const void* B, const void* C, void* D, float alpha, float beta) {
  const dist_gemm_step& f = P->steps[grp.first];
  const dist_gemm_step& l = P->steps[grp.first + grp.count - 1];
  dg::GemmParams g = step_params(P, f, A, B, C, D, alpha, beta);
  g.M = static_cast<int32_t>(std::max(f.m1, l.m1) - f.m0);
  g.N = static_cast<int32_t>(std::max(f.n1, l.n1) - f.n0);
  return g;
}

// ---- Single-launch execution ----------------------------------------------

// Build the device tables of the single-launch run: the pointer-free table of
// launch groups with their copy chunking, each queue's tile segments, and
// zeroed counters.  Synchronous (plan creation and option changes only).
int build_fused(dist_gemm_plan_s* P, std::string* err) {
  const Problem& pr = P->pr;
  const int S = pr.S;
  const int nq = P->queues;
  const CopyGeom& cg = P->geom;
  const int64_t width = static_cast<int64_t>(cg.width), height = static_cast<int64_t>(cg.height);

  // one table entry per launch group (the step-launch execution's grouping)
  const std::vector<LaunchGroup> groups = group_steps(P);
  const int G = static_cast<int>(groups.size());
  std::vector<dg::FusedStep> fs(G);
  for (int gi = 0; gi < G; ++gi) {
    const LaunchGroup& grp = groups[gi];
    const dist_gemm_step& st = P->steps[grp.first];
    const dist_gemm_step& last = P->steps[grp.first + grp.count - 1];
    const StepLayout y = step_layout(P, st);
    dg::FusedStep& f = fs[gi];
    f.offA = y.offA; f.offB = y.offB; f.offC = y.offC; f.offD = y.offD; f.offBias = y.offBias;
    f.lda = y.lda; f.ldb = y.ldb; f.ldc = y.ldc; f.ldd = y.ldd;
    f.sA = y.sA; f.sB = y.sB; f.sC = y.sC; f.sD = y.sD;
    f.M = static_cast<int32_t>(std::max(st.m1, last.m1) - st.m0);
    f.N = static_cast<int32_t>(std::max(st.n1, last.n1) - st.n0);
    f.tiles_m = (f.M + dg::kBM - 1) / dg::kBM;
    f.tiles_n = (f.N + dg::kBN - 1) / dg::kBN;
    f.stagedA = y.stagedA; f.stagedB = y.stagedB; f.stagedC = y.stagedC;
    f.copy_src_off = st.staged ? static_cast<int64_t>(st.shard) * width : 0;
    f.copy_dst_off = st.staged ? static_cast<int64_t>(st.slot) * width : 0;
  }
  // Copy chunking of group h: its bytes spread over the tiles of its carrier
  // group max(0, h - D), about one chunk per tile (at most COPY_CHUNK bytes,
  // at least 4 KiB, a multiple of 16), so that every carrier does about the
  // same copy work.
  for (int h = 0; h < G; ++h) {
    dg::FusedStep& f = fs[h];
    f.chunk_cols = width; f.chunk_rows = 1; f.chunks_per_row = 1; f.chunks_per_step = 0;
    f.n_chunks = 0;
    if (!P->steps[groups[h].first].staged) continue;
    const dg::FusedStep& carrier = fs[std::max(0, h - P->copy_ahead)];
    const int64_t ctiles = static_cast<int64_t>(carrier.tiles_m) * carrier.tiles_n * pr.L;
    const int64_t bytes = width * height * groups[h].count;
    int64_t chunk = (bytes + ctiles - 1) / ctiles;
    chunk = std::min<int64_t>(P->copy_chunk, std::max<int64_t>(4096, (chunk + 15) / 16 * 16));
    if (width >= chunk) {
      f.chunk_cols = chunk;
      f.chunks_per_row = static_cast<int32_t>((width + chunk - 1) / chunk);
      f.chunk_rows = 1;
    } else {
      f.chunk_cols = width;
      f.chunks_per_row = 1;
      f.chunk_rows = std::max<int64_t>(1, chunk / width);
    }
    const int64_t per_step = (height + f.chunk_rows - 1) / f.chunk_rows * f.chunks_per_row;
    if (per_step * groups[h].count > (int64_t{1} << 30))
      return fail(err, DIST_GEMM_ERR_UNSUPPORTED, "too many copy chunks; raise DIST_GEMM_OPT_COPY_CHUNK");
    f.chunks_per_step = static_cast<int32_t>(per_step);
    f.n_chunks = static_cast<int32_t>(per_step * groups[h].count);
  }
  P->fused_groups = G;
  // queue q: its share of every group's tiles (a contiguous range of the
  // group's tile order per batch), group after group
  std::vector<int32_t> seg(static_cast<size_t>(nq) * (G + 1), 0);
  for (int q = 0; q < nq; ++q) {
    int64_t at = 0;
    for (int s = 0; s < G; ++s) {
      seg[static_cast<size_t>(q) * (G + 1) + s] = static_cast<int32_t>(at);
      const int64_t T2 = static_cast<int64_t>(fs[s].tiles_m) * fs[s].tiles_n;
      at += (T2 / nq + (q < T2 % nq ? 1 : 0)) * pr.L;
      if (at >= INT32_MAX || T2 * pr.L >= INT32_MAX)
        return fail(err, DIST_GEMM_ERR_SHAPE, "too many tiles for one launch");
    }
    seg[static_cast<size_t>(q) * (G + 1) + G] = static_cast<int32_t>(at);
  }
  const size_t sync_words = static_cast<size_t>(dg::kSyncDone + S) * dg::kSyncStride;
  if (!P->d_steps) DG_HIP(err, hipMalloc(&P->d_steps, sizeof(dg::FusedStep) * S));
  if (P->d_seg) {
    DG_HIP(err, hipFree(P->d_seg));
    P->d_seg = nullptr;
  }
  DG_HIP(err, hipMalloc(&P->d_seg, seg.size() * sizeof(int32_t)));
  if (!P->d_sync) {
    DG_HIP(err, hipMalloc(&P->d_sync, sync_words * sizeof(int32_t)));
    DG_HIP(err, hipMemset(P->d_sync, 0, sync_words * sizeof(int32_t)));
  }
  DG_HIP(err, hipMemcpy(P->d_steps, fs.data(), sizeof(dg::FusedStep) * G, hipMemcpyHostToDevice));
  DG_HIP(err, hipMemcpy(P->d_seg, seg.data(), seg.size() * sizeof(int32_t), hipMemcpyHostToDevice));
  P->fused_align = 0;
  for (const dg::FusedStep& f : fs) P->fused_align |= static_cast<uint64_t>(f.chunk_cols);
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

int run_fused(dist_gemm_plan_s* P, hipStream_t st, const void* A, const void* B, const void* C,
              void* D, float alpha, float beta, const void* copy_src) {
  const Problem& pr = P->pr;
  const CopyGeom& g = P->geom;
  dg::FusedArgs a{};
  a.A = A; a.B = B; a.C = beta != 0.0f ? C : nullptr; a.D = D;
  a.bias = P->bias;
  a.staging = P->staging;
  a.copy_src = copy_src;
  a.steps = P->d_steps;
  a.seg = P->d_seg;
  a.sync = P->d_sync;
  a.cp_width = static_cast<int64_t>(g.width);
  a.cp_height = static_cast<int64_t>(g.height);
  a.cp_src_pitch = static_cast<int64_t>(g.src_pitch);
  a.cp_dst_pitch = static_cast<int64_t>(P->staging_pitch);
  a.spin_limit = P->wait_limit_us * P->clock_khz / 1000;
  const uint64_t align = reinterpret_cast<uint64_t>(copy_src) | reinterpret_cast<uint64_t>(P->staging) |
                         g.src_pitch | P->staging_pitch | g.width | P->fused_align;
  a.unit = (align % 16 == 0) ? 16 : (align % 4 == 0) ? 4 : 1;
  a.S = P->fused_groups;
  a.K = static_cast<int32_t>(pr.K);
  a.L = static_cast<int32_t>(pr.L);
  a.nq = P->queues;
  a.ahead = P->copy_ahead;
  a.alpha = alpha;
  a.beta = beta;
  const int grid = std::max(P->queues, P->n_cu / P->queues * P->queues);

  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  DG_HIP(&P->err, hipStreamIsCapturing(st, &cap));
  const bool ordered = cap == hipStreamCaptureStatusNone;
  FusedOrder& o = fused_order();
  std::unique_lock<std::mutex> lock(o.mu);
  if (ordered) {
    if (static_cast<int>(o.tail.size()) <= P->device) {
      o.tail.resize(P->device + 1, nullptr);
      o.live.resize(P->device + 1, 0);
    }
    if (!o.tail[P->device]) DG_HIP(&P->err, hipEventCreateWithFlags(&o.tail[P->device], hipEventDisableTiming));
    if (o.live[P->device]) DG_HIP(&P->err, hipStreamWaitEvent(st, o.tail[P->device], 0));
  }
  DG_HIP(&P->err, dg::launch_fused(pr.in_kind, pr.out_kind, a, grid, st));
  if (ordered) {
    DG_HIP(&P->err, hipEventRecord(o.tail[P->device], st));
    o.live[P->device] = 1;
  }
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
  const int n_slots = pr.S - 1;
  if (pr.schedule != DIST_GEMM_MONOLITHIC && n_slots > 0) {
    P->staging_pitch = P->geom.staging_pitch(n_slots);
    e = hipMalloc(&P->staging, P->staging_pitch * P->geom.height);
    if (e != hipSuccess) {
      release(P);
      (void)hipGetLastError();
      return fail(perr, DIST_GEMM_ERR_OOM, "staging allocation of " +
                                               std::to_string(P->staging_pitch * P->geom.height) + " bytes");
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
  if (pr.schedule != DIST_GEMM_MONOLITHIC && n_slots > 0) {
    rc = build_fused(P, perr);
    if (rc != DIST_GEMM_OK) {
      release(P);
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
      const int old_g = plan->max_group;
      plan->max_group = static_cast<int>(value);
      if (!plan->d_steps) return DIST_GEMM_OK;
      DeviceGuard guard(plan->device);
      if (plan->has_prev) DG_HIP(&plan->err, hipEventSynchronize(plan->ev_done));
      const int rc = build_fused(plan, &plan->err);
      if (rc != DIST_GEMM_OK) {
        plan->max_group = old_g;
        (void)build_fused(plan, nullptr);
      }
      return rc;
    }
    case DIST_GEMM_OPT_EXECUTION:
      if (value != 0 && value != 1)
        return fail(&plan->err, DIST_GEMM_ERR_INVALID_ARG, "execution must be 0 or 1");
      plan->execution = static_cast<int>(value);
      return DIST_GEMM_OK;
    case DIST_GEMM_OPT_QUEUES:
    case DIST_GEMM_OPT_COPY_CHUNK: {
      const bool queues = option == DIST_GEMM_OPT_QUEUES;
      if (queues && value != 1 && value != dg::kMaxQueues)
        return fail(&plan->err, DIST_GEMM_ERR_INVALID_ARG, "queues must be 1 or 8");
      if (!queues && (value < 4096 || value > (int64_t{1} << 28) || value % 16 != 0))
        return fail(&plan->err, DIST_GEMM_ERR_INVALID_ARG,
                    "copy chunk must be a multiple of 16 in [4096, 2^28]");
      if ((queues ? plan->queues : plan->copy_chunk) == value) return DIST_GEMM_OK;
      const int old_q = plan->queues;
      const int64_t old_c = plan->copy_chunk;
      if (queues)
        plan->queues = static_cast<int>(value);
      else
        plan->copy_chunk = value;
      if (!plan->d_steps) return DIST_GEMM_OK;  // no staged steps: nothing to rebuild
      DeviceGuard guard(plan->device);
      if (plan->has_prev) DG_HIP(&plan->err, hipEventSynchronize(plan->ev_done));
      const int rc = build_fused(plan, &plan->err);
      if (rc != DIST_GEMM_OK) {
        plan->queues = old_q;
        plan->copy_chunk = old_c;
        (void)build_fused(plan, nullptr);
      }
      return rc;
    }
    case DIST_GEMM_OPT_COPY_AHEAD: {
      if (value < 1 || value > 64)
        return fail(&plan->err, DIST_GEMM_ERR_INVALID_ARG, "copy lookahead must be 1..64");
      if (plan->copy_ahead == value) return DIST_GEMM_OK;
      const int old_a = plan->copy_ahead;
      plan->copy_ahead = static_cast<int>(value);
      if (!plan->d_steps) return DIST_GEMM_OK;
      DeviceGuard guard(plan->device);
      if (plan->has_prev) DG_HIP(&plan->err, hipEventSynchronize(plan->ev_done));
      const int rc = build_fused(plan, &plan->err);
      if (rc != DIST_GEMM_OK) {
        plan->copy_ahead = old_a;
        (void)build_fused(plan, nullptr);
      }
      return rc;
    }
    case DIST_GEMM_OPT_SHARED_A: {
      if (value != 0 && value != 1)
        return fail(&plan->err, DIST_GEMM_ERR_INVALID_ARG, "shared A must be 0 or 1");
      if (plan->pr.shared_a == (value != 0)) return DIST_GEMM_OK;
      DeviceGuard guard(plan->device);
      if (plan->has_prev) DG_HIP(&plan->err, hipEventSynchronize(plan->ev_done));
      // the staging buffer was sized for L batches: a shared A needs one
      plan->pr.shared_a = value != 0;
      plan->geom = copy_geom(plan->pr);
      if (!plan->d_steps) return DIST_GEMM_OK;
      const int rc = build_fused(plan, &plan->err);
      if (rc != DIST_GEMM_OK) {
        plan->pr.shared_a = !plan->pr.shared_a;
        plan->geom = copy_geom(plan->pr);
        (void)build_fused(plan, nullptr);
      }
      return rc;
    }
    case DIST_GEMM_OPT_WAIT_LIMIT_US:
      if (value < 0 || value > 100000000)
        return fail(&plan->err, DIST_GEMM_ERR_INVALID_ARG, "wait limit must be in [0, 1e8] us");
      plan->wait_limit_us = value;
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
      plan->t_first.clear();
      plan->t_fused.clear();
      plan->t_begin.clear();
      plan->t_end.clear();
      plan->t_run0.clear();
      plan->t_copy.clear();
      plan->step_timing = 0;
      plan->timed_runs = 0;
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
      plan->step_timing = static_cast<int>(value);
      return DIST_GEMM_OK;
    }
    default:
      return fail(&plan->err, DIST_GEMM_ERR_INVALID_ARG, "unknown option " + std::to_string(option));
  }
}

int dist_gemm_run(dist_gemm_plan_t plan, const void* A, const void* B, const void* C, void* D,
                  float alpha, float beta, void* stream) {
  if (!plan) return fail(nullptr, DIST_GEMM_ERR_INVALID_ARG, "plan is NULL");
  dist_gemm_plan_s* P = plan;
  if (!A || !B || !D) return fail(&P->err, DIST_GEMM_ERR_INVALID_ARG, "A, B and D must be non-NULL");
  if (beta != 0.0f && !C) return fail(&P->err, DIST_GEMM_ERR_INVALID_ARG, "C is NULL but beta != 0");
  if (!std::isfinite(alpha) || !std::isfinite(beta))
    return fail(&P->err, DIST_GEMM_ERR_INVALID_ARG, "alpha and beta must be finite");
  if (D == A || D == B) return fail(&P->err, DIST_GEMM_ERR_INVALID_ARG, "D must not alias A or B");

  DeviceGuard guard(P->device);
  const Problem& pr = P->pr;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool rotating = pr.schedule != DIST_GEMM_MONOLITHIC && pr.S > 1;
  const bool two = P->compute_streams == 2 && pr.S > 1;
  const float alpha_eff =
      (pr.in_kind == dg::IN_E4M3) ? alpha * P->scale_a * P->scale_b : alpha;
  const void* copy_src = nullptr;
  switch (pr.schedule) {
    case DIST_GEMM_AG_ROT_A: copy_src = A; break;
    case DIST_GEMM_AG_ROT_B: copy_src = B; break;
    default: copy_src = C; break;  // RS: the rotating partial
  }
  if (rotating && !copy_src) {
    return fail(&P->err, DIST_GEMM_ERR_INVALID_ARG,
                "the reduce-scatter schedules rotate C: C must be non-NULL");
  }

  if (rotating && P->execution == 1) {
    if (P->has_prev && P->prev_stream != st) DG_HIP(&P->err, hipStreamWaitEvent(st, P->ev_done, 0));
    const size_t trun = P->step_timing ? static_cast<size_t>(P->timed_runs % P->step_timing) : 0;
    const size_t tbase = trun * P->steps.size();
    if (P->step_timing) {
      DG_HIP(&P->err, hipEventRecord(P->t_run0[trun], st));
      for (size_t k = 0; k < P->steps.size(); ++k) P->t_first[tbase + k] = 0;
      P->t_fused[trun] = 1;
      DG_HIP(&P->err, hipEventRecord(P->t_begin[tbase], st));
    }
    const int rc = run_fused(P, st, A, B, C, D, alpha_eff, beta, copy_src);
    if (rc != DIST_GEMM_OK) return rc;
    if (P->step_timing) DG_HIP(&P->err, hipEventRecord(P->t_end[tbase], st));
    DG_HIP(&P->err, hipEventRecord(P->ev_done, st));
    P->has_prev = true;
    P->prev_stream = st;
    if (P->step_timing) ++P->timed_runs;
    return DIST_GEMM_OK;
  }

  // side streams in use: the first n, n = min(copy streams, staged copies)
  const int n_side = rotating ? std::min(P->copy_streams, pr.S - 1) : 0;
  if (n_side > static_cast<int>(P->sides.size()))
    return fail(&P->err, DIST_GEMM_ERR_INVALID_ARG, "copy streams not created");

  if (P->has_prev && P->prev_stream != st) DG_HIP(&P->err, hipStreamWaitEvent(st, P->ev_done, 0));
  DG_HIP(&P->err, hipEventRecord(P->ev_start, st));
  const size_t trun = P->step_timing ? static_cast<size_t>(P->timed_runs % P->step_timing) : 0;
  const size_t tbase = trun * P->steps.size();
  if (P->step_timing) {
    DG_HIP(&P->err, hipEventRecord(P->t_run0[trun], st));
    P->t_fused[trun] = 0;
  }
  for (int k = 0; k < n_side; ++k) DG_HIP(&P->err, hipStreamWaitEvent(P->sides[k], P->ev_start, 0));
  if (two) DG_HIP(&P->err, hipStreamWaitEvent(P->cs2, P->ev_start, 0));

  // Copy engine: every staged operand, in step order, round-robin over the
  // side streams, one event per copy.
  if (rotating) {
    for (const dist_gemm_step& s : P->steps) {
      if (!s.staged) continue;
      hipStream_t side = P->sides[s.slot % n_side];
      int rc = enqueue_copy(P, side, copy_src, s.shard, s.slot);
      if (rc != DIST_GEMM_OK) return rc;
      DG_HIP(&P->err, hipEventRecord(P->ev_copy[s.step], side));
      if (P->step_timing) DG_HIP(&P->err, hipEventRecord(P->t_copy[tbase + s.step], side));
    }
  }
  // Step GEMMs: one launch per group, alternating compute streams by launch.
  const std::vector<LaunchGroup> groups = group_steps(P);
  for (size_t gi = 0; gi < groups.size(); ++gi) {
    const LaunchGroup& grp = groups[gi];
    hipStream_t cs = (two && (gi & 1)) ? P->cs2 : st;
    for (int k = grp.first; k < grp.first + grp.count; ++k) {
      if (P->steps[k].staged) DG_HIP(&P->err, hipStreamWaitEvent(cs, P->ev_copy[k], 0));
      if (P->step_timing) P->t_first[tbase + k] = grp.first;
    }
    if (P->step_timing) DG_HIP(&P->err, hipEventRecord(P->t_begin[tbase + grp.first], cs));
    const dg::GemmParams g = group_params(P, grp, A, B, C, D, alpha_eff, beta);
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
  for (int64_t s = 0; s < S; ++s) {
    float v[3] = {-1.0f, 0.0f, 0.0f};
    const bool staged = plan->steps[s].staged && plan->pr.schedule != DIST_GEMM_MONOLITHIC &&
                        !plan->t_fused[run];
    if (staged) DG_HIP(&plan->err, hipEventElapsedTime(&v[0], t0, plan->t_copy[base + s]));
    const int f = plan->t_first[base + s];
    DG_HIP(&plan->err, hipEventElapsedTime(&v[1], t0, plan->t_begin[base + f]));
    DG_HIP(&plan->err, hipEventElapsedTime(&v[2], t0, plan->t_end[base + f]));
    for (int k = 0; k < 3; ++k)
      if (3 * s + k < cap) ms[3 * s + k] = v[k];
  }
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

}  // extern "C"
