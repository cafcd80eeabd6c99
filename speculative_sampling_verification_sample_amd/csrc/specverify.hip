// C ABI of the verify step: argument validation, workspace layout and the
// launch sequence of the kernels on the caller's stream.
//
//   sample : K1 row pass -> [truncation: K2 row finalisation, with the
//            exact path inside] -> K3 acceptance + list draws -> K4
//            full-row draws (chunk totals, then the per-request search)
//   greedy : K1 row pass (argmax) -> greedy scan
//   stats  : K1 -> K2 -> per-chunk sums -> per-row finish
//
// Nothing here allocates or frees device memory: every scratch buffer is a
// slice of the caller's workspace.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <map>
#include <mutex>
#include <utility>

#include "specverify.h"
#include "sv_device.h"
#include "sv_rowfinal.h"
#include "sv_rowpass.h"
#include "sv_verify.h"

namespace {

using namespace sv;

constexpr int64_t kChunkBytes = 28672;  // bytes of one row a streaming row-pass workgroup reads
constexpr int kKMax = 2048;       // longest kept set stored as a list
constexpr int kFastTopK = 256;    // top-k above this always takes the exact path
constexpr int kNwTopP = 128;      // chunk elements a top-p candidate threshold certifies
// ... for the draft's own rows (q formed in the library): drafts tend to be
// flatter, with nuclei reaching below 128 certified elements per chunk
constexpr int kNwTopPDraft = 256;
// Candidate list capacity of one chunk: a multiple of the certified count
// (lists measure about 1.5-3x nw on the workloads' rows); a longer list sends
// the row to the exact path.  It also sizes the row finisher's LDS union.
constexpr int kCapPerNw = 4;
constexpr int kCapMin = 256;
constexpr int kCapMax = 1280;
constexpr int kTruncMinWG = 2048; // truncated pass: shorter chunks until this many workgroups
constexpr int kUnionMax = 2048;   // LDS entries of the row finisher's candidate union
// Below this many requests the sampled rows are weighed by many workgroups
// per request (two launches); above it one workgroup per request already
// fills the GPU and the single launch wins.
constexpr int kOneLaunchMinB = 256;

// CALL_DRAFT: the row passes over a draft's logits [B, gamma, V] (q formed
// in the library): statistics and kept lists only.  CALL_SAMPLE_STATS: the
// sampling call whose row results also serve the statistics.
enum CallKind { CALL_SAMPLE, CALL_GREEDY, CALL_STATS, CALL_DRAFT, CALL_SAMPLE_STATS };

struct Plan {
  int64_t rows = 0;
  int rows_per_req = 0;
  int mode = M_SOFTMAX;
  bool trunc = false, need_s = false, fast = true;
  int nchunks = 1;
  int64_t chunk = 8;
  int nw = 0, cap_out = 0, um = 0;
  int nu = 16;  // truncated pass: 16-byte units per thread
  int nch4 = 1;
  int scale_bits = 40;
  size_t off_cout = 0, off_cand = 0, off_info = 0, off_kept = 0, off_jobs = 0, off_part = 0, off_gath = 0;
  size_t off_spart = 0;  // statistics partials [B * gamma][nchunks][kStatSums] (CALL_STATS, CALL_SAMPLE_STATS)
  size_t off_qsum = 0;   // a dense q's row sums by chunk [B * gamma][nchq] (the same calls)
  size_t off_s64 = 0;    // untruncated rows' S64 by chunk [2][B * gamma][nchunks]: the target's, the draft's (the same calls)
  size_t off_zqp = 0;    // listed rows' two list sums for Z' [B * gamma][2] (the same calls, truncated rows)
  int nchq = 1;
  size_t total = 0;
};

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

Plan make_plan(CallKind kind, int32_t B, int32_t gamma, int64_t V, sv_dtype dt, sv_sampling_params prm) {
  Plan p;
  const bool topk = prm.top_k > 0 && (int64_t)prm.top_k < V;
  const bool topp = prm.top_p < 1.0f;
  p.rows_per_req = (kind == CALL_STATS || kind == CALL_DRAFT) ? gamma : gamma + 1;
  p.rows = (int64_t)B * p.rows_per_req;
  p.trunc = (kind != CALL_GREEDY) && (topk || topp);
  const bool sampling = kind == CALL_SAMPLE || kind == CALL_SAMPLE_STATS;
  p.mode = (kind == CALL_GREEDY) ? M_ARGMAX : (p.trunc ? M_TRUNC : M_SOFTMAX);
  p.need_s = p.trunc && topp && !topk;
  p.fast = !topk || prm.top_k <= kFastTopK;
  if (p.trunc) {
    p.nw = topk ? std::min<int>(prm.top_k, kFastTopK) : (kind == CALL_DRAFT ? kNwTopPDraft : kNwTopP);
    p.cap_out = std::min(kCapMax, std::max(kCapMin, kCapPerNw * p.nw));
  }
  int64_t nch, chunk;
  if (p.trunc) {
    // A chunk is held in registers: at most nu * kTruncBS units of 16 bytes,
    // two of them possibly straddling the chunk ends.  Shorter chunks (fewer
    // units per thread) only when the rows alone do not fill the GPU, and
    // only while the chunks' candidates (about nw each) stay well inside the
    // row finisher's union: past it a row takes the exact path, which on a
    // few rows costs far more than the idle CUs (2 x 5 rows of 256000 bf16,
    // top-p: 16 chunks per row put the finisher at 315 us, 8 chunks keep
    // the whole step at 46 us).
    const int64_t epv = (dt == SV_BF16) ? 8 : 4;
    auto chunks_at = [&](int nu) {
      const int64_t cap = ((int64_t)nu * kTruncBS - 2) * epv / 8 * 8;
      return (V + cap - 1) / cap;
    };
    for (p.nu = 16;; p.nu /= 2) {
      nch = chunks_at(p.nu);
      if (p.nu == 4 || p.rows * nch >= kTruncMinWG) break;
      if (chunks_at(p.nu / 2) * p.nw > kUnionMax / 2) break;
    }
  } else {
    // Chunks of about kChunkBytes: shorter ones pay a workgroup's fixed cost
    // (launch, the first loads' latency, the reductions) on too few bytes,
    // longer ones leave a long launch tail.  Measured on 64 x 5 rows of 32000
    // fp32 and 512 x 9 rows of 152064 bf16.
    const int64_t esz = (dt == SV_BF16) ? 2 : 4;
    nch = std::max<int64_t>(1, (V * esz + kChunkBytes - 1) / kChunkBytes);
  }
  chunk = (V + nch - 1) / nch;
  chunk = (chunk + 7) / 8 * 8;
  nch = (V + chunk - 1) / chunk;
  p.nchunks = (int)nch;
  p.chunk = chunk;
  if (p.trunc) {
    int64_t u = nch * p.cap_out;
    int um = 1;
    while (um < u && um < kUnionMax) um <<= 1;
    p.um = um;
  }
  p.nch4 = (int)((V + kChunk4 - 1) / kChunk4);
  int lg = 0;
  while (((int64_t)1 << lg) < V) ++lg;
  p.scale_bits = std::min(40, 62 - lg);

  const size_t rows = (size_t)p.rows;
  size_t off = 0;
  p.off_cout = off;
  off = align_up(off + rows * nch * sizeof(ChunkOut), 256);
  p.off_cand = off;
  if (p.trunc) off = align_up(off + rows * nch * (size_t)p.cap_out * sizeof(Cand), 256);
  p.off_info = off;
  if (kind != CALL_GREEDY) off = align_up(off + rows * sizeof(RowInfo), 256);
  p.off_kept = off;
  if (p.trunc) off = align_up(off + rows * (size_t)kKMax * sizeof(Cand), 256);
  p.off_jobs = off;
  if (sampling) off = align_up(off + (size_t)B * sizeof(BigJob), 256);
  p.off_gath = off;
  if (sampling) off = align_up(off + rows * sizeof(float2), 256);
  p.off_part = off;
  if (sampling) off = align_up(off + (size_t)B * p.nch4 * 4 * sizeof(double), 256);
  p.off_spart = off;
  if (kind == CALL_STATS || kind == CALL_SAMPLE_STATS)
    off = align_up(off + (size_t)B * gamma * nch * kStatSums * sizeof(double), 256);
  p.nchq = (int)((V + kQSumChunk - 1) / kQSumChunk);
  p.off_qsum = off;
  if (kind == CALL_STATS || kind == CALL_SAMPLE_STATS)
    off = align_up(off + (size_t)B * gamma * p.nchq * sizeof(double), 256);
  p.off_s64 = off;
  if (!p.trunc && (kind == CALL_STATS || kind == CALL_SAMPLE_STATS))
    off = align_up(off + 2 * (size_t)B * gamma * nch * sizeof(double), 256);
  p.off_zqp = off;
  if (p.trunc && (kind == CALL_STATS || kind == CALL_SAMPLE_STATS))
    off = align_up(off + 2 * (size_t)B * gamma * sizeof(double), 256);
  p.total = std::max<size_t>(off, 256);
  return p;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

sv_status check_sizes(int32_t B, int32_t gamma, int32_t V, sv_dtype dt) {
  if (B < 0 || gamma < 0 || V < 1) return SV_ERR_INVALID_ARG;
  if (dt != SV_F32 && dt != SV_BF16) return SV_ERR_INVALID_ARG;
  if (gamma > 4096) return SV_ERR_UNSUPPORTED;
  // element offsets are 64-bit; rows are addressed with 32-bit indices
  if ((int64_t)B * (gamma + 1) > (int64_t)INT32_MAX) return SV_ERR_UNSUPPORTED;
  return SV_OK;
}

// log2(e) / T in the forms the kernels use: the double c64; c, c64 rounded
// to the nearest float (the one-part e); and the two-part split c2 + cl of
// e2, with c2 the float just below c64 and cl the (positive, at least
// FLT_MIN) float of the remainder, so that a -inf logit never meets a
// negative low part (-inf * cl would be +inf, and +inf - inf a NaN).
struct Expo {
  float c, c2, cl;
  double c64;
};
constexpr Expo kExpoGreedy = {1.0f, 1.0f, 0.0f, 1.0};  // greedy passes take no exponentials

sv_status check_params(sv_sampling_params prm, Expo* c_out) {
  const float T = prm.temperature;
  if (!(T > 0.0f) || !std::isfinite(T)) return SV_ERR_INVALID_ARG;
  if (prm.top_k < 0) return SV_ERR_INVALID_ARG;
  if (!(prm.top_p > 0.0f && prm.top_p <= 1.0f)) return SV_ERR_INVALID_ARG;
  const double c = 1.4426950408889634 / (double)T;
  if (!std::isfinite(c) || c > 1e30) return SV_ERR_INVALID_ARG;
  c_out->c64 = c;
  c_out->c = (float)c;
  float c2 = (float)c;
  if ((double)c2 >= c) c2 = std::nextafter(c2, 0.0f);
  c_out->c2 = c2;
  c_out->cl = std::max((float)(c - (double)c2), std::numeric_limits<float>::min());
  return SV_OK;
}

template <typename T>
T* ws_at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<unsigned char*>(ws) + off);
}

sv_status launched() { return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP; }

// Profiling hook: per stage, two caller events attached to that stage's
// kernel dispatch (spec_set_stage_timer).
hipEvent_t g_timer_start[SV_STAGE_COUNT] = {}, g_timer_stop[SV_STAGE_COUNT] = {};

// Launches a kernel of stage `stage` (< 0: never timed).  With the stage's
// events set, they are attached to the kernel's own dispatch, so they take
// its start and end times.
template <typename... KArgs, typename... Args>
void launch_stage(int stage, void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t shmem, hipStream_t st,
                  Args... args) {
  if (stage >= 0 && g_timer_start[stage] && g_timer_stop[stage])
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, st, g_timer_start[stage], g_timer_stop[stage], 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, shmem, st, args...);
}

void launch_row_kernel(void (*kernel)(RowPassArgs), dim3 grid, dim3 block, hipStream_t st, const RowPassArgs& a,
                       bool timed) {
  launch_stage(timed ? SV_STAGE_ROWPASS : -1, kernel, grid, block, 0, st, a);
}

template <int MODE, bool BF16>
void launch_rowpass(const Plan& p, const RowPassArgs& a, hipStream_t st, bool timed) {
  dim3 grid((unsigned)(p.nchunks * p.rows));
  // V a multiple of the unit width: every chunk's units are whole (see
  // launch_trunc)
  if (a.V % (BF16 ? 8 : 4) == 0) launch_row_kernel(rowpass_kernel<MODE, BF16, 256, true>, grid, dim3(256), st, a, timed);
  else launch_row_kernel(rowpass_kernel<MODE, BF16, 256, false>, grid, dim3(256), st, a, timed);
}

template <bool BF16, bool NEED_S, bool ALIGNED>
void launch_trunc_nu(const Plan& p, const RowPassArgs& a, hipStream_t st, bool timed) {
  dim3 grid((unsigned)(p.nchunks * p.rows));
  if (p.nu == 16) launch_row_kernel(trunc_pass_kernel<BF16, NEED_S, 16, ALIGNED>, grid, dim3(kTruncBS), st, a, timed);
  else if (p.nu == 8) launch_row_kernel(trunc_pass_kernel<BF16, NEED_S, 8, ALIGNED>, grid, dim3(kTruncBS), st, a, timed);
  else launch_row_kernel(trunc_pass_kernel<BF16, NEED_S, 4, ALIGNED>, grid, dim3(kTruncBS), st, a, timed);
}

template <bool BF16, bool NEED_S>
void launch_trunc(const Plan& p, const RowPassArgs& a, hipStream_t st, bool timed) {
  // rows start at multiples of V and chunks at multiples of 8 elements, so
  // V a multiple of the elements per 16-byte unit makes every chunk's units
  // whole (and every unit lies inside the tensor)
  const int64_t epv = BF16 ? 8 : 4;
  if (a.V % epv == 0) launch_trunc_nu<BF16, NEED_S, true>(p, a, st, timed);
  else launch_trunc_nu<BF16, NEED_S, false>(p, a, st, timed);
}

QSrc q_src_dense(const float* q, int64_t V) {
  QSrc s;
  s.dense = q;
  s.z = nullptr;
  s.info = nullptr;
  s.V = V;
  s.c = 0.0f;
  s.c2 = 0.0f;
  s.cl = 0.0f;
  s.c64 = 0.0;
  s.zbf16 = 0;
  return s;
}

QSrc q_src_none(int64_t V) { return q_src_dense(nullptr, V); }

// `timed`: this launch carries the profiling hook's events (the target rows'
// pass; not the draft rows').
// `cu`, `n_live`: a ragged batch's draft offsets and its packed rows
// (n_draft + B); cu = null: uniform.
template <bool BF16>
sv_status run_rowpass(const Plan& p, const void* logits, int64_t V, int G1, const Expo& c, void* ws, hipStream_t st,
                      const int32_t* ids = nullptr, QSrc q = QSrc{}, int gamma = 0, float2* gath = nullptr,
                      bool timed = true, const int32_t* cu = nullptr, int32_t n_live = 0) {
  RowPassArgs a;
  a.ids = ids;
  a.q = q;
  a.gamma = gamma;
  a.gath = gath;
  a.cu = cu;
  a.n_live = n_live;
  a.logits = logits;
  a.V = V;
  a.chunk = p.chunk;
  a.rows_per_req = p.rows_per_req;
  a.G1 = G1;
  a.nchunks = p.nchunks;
  a.c = c.c;
  a.c2 = c.c2;
  a.cl = c.cl;
  a.nw = p.nw;
  a.cap_out = p.cap_out;
  a.out = ws_at<ChunkOut>(ws, p.off_cout);
  a.cand = p.trunc ? ws_at<Cand>(ws, p.off_cand) : nullptr;
  if (p.mode == M_TRUNC) {
    // every chunk's units must fit the registers of one workgroup
    const int64_t epv = BF16 ? 8 : 4;
    if (p.chunk / epv + 2 > (int64_t)p.nu * kTruncBS) return SV_ERR_UNSUPPORTED;
    if (p.need_s) launch_trunc<BF16, true>(p, a, st, timed);
    else launch_trunc<BF16, false>(p, a, st, timed);
  } else if (p.mode == M_SOFTMAX) {
    launch_rowpass<M_SOFTMAX, BF16>(p, a, st, timed);
  } else {
    launch_rowpass<M_ARGMAX, BF16>(p, a, st, timed);
  }
  return launched();
}

std::once_flag g_attr_once;

void set_kernel_attrs() {
  std::call_once(g_attr_once, [] {
    const int kMaxDyn = 160 * 1024;
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&rowfinal_kernel<true>),
                        hipFuncAttributeMaxDynamicSharedMemorySize, kMaxDyn);
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&rowfinal_kernel<false>),
                        hipFuncAttributeMaxDynamicSharedMemorySize, kMaxDyn);
    (void)hipGetLastError();
  });
}

template <bool BF16>
sv_status run_rowfinal(const Plan& p, const void* logits, const QSrc& q, const int32_t* ids, int64_t V, int G1,
                       int gamma, const Expo& c, sv_sampling_params prm, void* ws, hipStream_t st,
                       const int32_t* cu = nullptr, int32_t n_live = 0, bool timed = true) {
  RowFinalArgs a;
  a.cu = cu;
  a.n_live = n_live;
  a.logits = logits;
  a.q = q;
  a.ids = ids;
  a.V = V;
  a.rows_per_req = p.rows_per_req;
  a.G1 = G1;
  a.gamma = gamma;
  a.nchunks = p.nchunks;
  a.cap_out = p.cap_out;
  a.trunc = p.trunc ? 1 : 0;
  a.fast = p.fast ? 1 : 0;
  a.top_k = prm.top_k;
  a.top_p = prm.top_p;
  a.c = c.c;
  a.c2 = c.c2;
  a.cl = c.cl;
  a.c64 = c.c64;
  a.um = p.um;
  a.kmax = kKMax;
  a.scale_bits = p.scale_bits;
  a.cout = ws_at<ChunkOut>(ws, p.off_cout);
  a.cand = p.trunc ? ws_at<Cand>(ws, p.off_cand) : nullptr;
  a.info = ws_at<RowInfo>(ws, p.off_info);
  a.kept = p.trunc ? ws_at<Cand>(ws, p.off_kept) : nullptr;
  set_kernel_attrs();
  size_t dyn = p.trunc ? (size_t)p.um * 8 : 0;  // key and token id per union entry
  launch_stage(timed ? SV_STAGE_ROWFINAL : -1, rowfinal_kernel<BF16>, dim3((unsigned)p.rows), dim3(256), dyn, st, a);
  return launched();
}

sv_status common_checks(const void* logits, sv_dtype dt, int32_t B, int32_t gamma, int32_t V) {
  sv_status s = check_sizes(B, gamma, V, dt);
  if (s != SV_OK) return s;
  if (B > 0 && (logits == nullptr || !aligned16(logits))) return SV_ERR_INVALID_ARG;
  return SV_OK;
}

// ---- a second stream for work that does not depend on the target's passes
// A call's dense-q row sums (only Z' needs them) read nothing the row passes
// write, and the draft rows' passes of a draft-logits call under top-k or
// top-p write nothing the target's row pass reads, so they run on a stream
// of the library's beside the caller's: the call records `fork` on its
// stream, the side stream waits for it, runs the work and records `join`,
// and the caller's stream waits for `join` before the first kernel that
// reads the results (the statistics finish; the target's row finisher).  One side stream (non-blocking, default priority)
// and its two events per (device, caller stream), made on first use; under
// graph capture the fork and join make the side work part of the graph.
// Without them (creation failed, or kMaxSideStreams pairs already made:
// the library keeps what it makes until the process ends, so a caller that
// cycles through many streams cannot make it grow without bound) the sums
// run on the caller's stream.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
std::mutex g_side_mu;
std::map<std::pair<int, hipStream_t>, SideStream> g_side;
constexpr size_t kMaxSideStreams = 64;

const SideStream* side_stream(hipStream_t st) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_side_mu);
  auto it = g_side.find({dev, st});
  if (it != g_side.end()) return it->second.s ? &it->second : nullptr;
  if (g_side.size() >= kMaxSideStreams) return nullptr;
  SideStream ss;
  bool ok = hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking) == hipSuccess;
  ok = ok && hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming) == hipSuccess;
  ok = ok && hipEventCreateWithFlags(&ss.join, hipEventDisableTiming) == hipSuccess;
  if (!ok) {
    (void)hipGetLastError();
    if (ss.fork) (void)hipEventDestroy(ss.fork);
    if (ss.join) (void)hipEventDestroy(ss.join);
    if (ss.s) (void)hipStreamDestroy(ss.s);
    ss = SideStream{};
  }
  auto& slot = g_side[{dev, st}];
  slot = ss;
  return slot.s ? &slot : nullptr;
}

// A dense q's row sums (rows b * gamma + j, j < gamma) for Z', in two
// steps.  qsum_fork_point records `fork` on the caller's stream right after
// the target's row pass (running beside that pass, the sums slow it more
// than they gain).  launch_qsum, called once the kernels that follow on the
// caller's stream are launched, starts the sums on the side stream behind
// `fork`: launched in that order (also as graph nodes), the latency-bound
// row finisher and acceptance kernels are dispatched before the sums' many
// short workgroups, which would otherwise take every free CU slot and hold
// them back until the sums are done.  launch_qsum returns the event the
// statistics finish must wait for (null: nothing to wait for, the sums went
// on the caller's stream).
const SideStream* qsum_fork_point(hipStream_t st, sv_status* status) {
  *status = SV_OK;
  const SideStream* ss = side_stream(st);
  if (ss != nullptr && hipEventRecord(ss->fork, st) != hipSuccess) *status = SV_ERR_HIP;
  return ss;
}

hipEvent_t launch_qsum(const SideStream* ss, const Plan& p, const float* q, int32_t B, int32_t gamma, int32_t V,
                       void* ws, hipStream_t st, sv_status* status) {
  *status = SV_OK;
  QSumArgs a;
  a.q = q;
  a.V = V;
  a.rows = (int64_t)B * gamma;
  a.nchq = p.nchq;
  a.out = ws_at<double>(ws, p.off_qsum);
  if (a.rows == 0) return nullptr;
  const dim3 grid((unsigned)(a.rows * p.nchq));
  if (ss == nullptr) {
    launch_stage(SV_STAGE_QSUM, qsum_kernel, grid, dim3(256), 0, st, a);
    *status = launched();
    return nullptr;
  }
  if (hipStreamWaitEvent(ss->s, ss->fork, 0) != hipSuccess) {
    *status = SV_ERR_HIP;
    return nullptr;
  }
  launch_stage(SV_STAGE_QSUM, qsum_kernel, grid, dim3(256), 0, ss->s, a);
  *status = launched();
  if (*status != SV_OK) return nullptr;
  if (hipEventRecord(ss->join, ss->s) != hipSuccess) {
    *status = SV_ERR_HIP;
    return nullptr;
  }
  return ss->join;
}

// The sampling verify once q's source is known (dense, or the draft's
// logits after their row passes).  `workspace` holds plan p's regions.
// Ragged batches pass their draft offsets `cu` (gamma is then the maximum
// gamma_b); `eos` < 0 disables the end-of-sequence cut; `beta` < 1 is the
// lenient acceptance (the draft compared as beta * q).
sv_status verify_sample_impl(const Plan& p, const void* target_logits, sv_dtype dt, const QSrc& q,
                             const int32_t* draft_ids, const float* u_accept, const float* u_resample, int32_t B,
                             int32_t gamma, int32_t V, sv_sampling_params prm, const Expo& c, int32_t* out_tokens,
                             int32_t* out_num_accepted, uint32_t* out_row_flags, void* workspace, hipStream_t st,
                             const int32_t* cu = nullptr, int32_t n_draft = 0, int32_t eos = -1,
                             double beta = 1.0, bool force_rowfinal = false,
                             const SideStream** qsum_fork = nullptr, hipEvent_t q_ready = nullptr) {
  const int G1 = gamma + 1;
  const bool bf = dt == SV_BF16;

  // untruncated rows: the row pass also gathers each draft's logit and q(d)
  float2* gath = p.trunc ? nullptr : ws_at<float2>(workspace, p.off_gath);
  const int32_t n_live = n_draft + B;  // ragged: packed target rows
  sv_status s =
      bf ? run_rowpass<true>(p, target_logits, V, G1, c, workspace, st, draft_ids, q, gamma, gath, true, cu, n_live)
         : run_rowpass<false>(p, target_logits, V, G1, c, workspace, st, draft_ids, q, gamma, gath, true, cu, n_live);
  if (s != SV_OK) return s;
  if (qsum_fork != nullptr) {
    // the statistics' dense-q row sums may start here (the caller launches
    // them after this call's kernels)
    *qsum_fork = qsum_fork_point(st, &s);
    if (s != SV_OK) return s;
  }
  // q's row results made on another stream (truncated rows only: their row
  // pass reads nothing of q); the row finisher is their first reader
  if (q_ready != nullptr && hipStreamWaitEvent(st, q_ready, 0) != hipSuccess) return SV_ERR_HIP;
  if (p.trunc || force_rowfinal) {
    s = bf ? run_rowfinal<true>(p, target_logits, q, draft_ids, V, G1, gamma, c, prm, workspace, st, cu, n_live)
           : run_rowfinal<false>(p, target_logits, q, draft_ids, V, G1, gamma, c, prm, workspace, st, cu, n_live);
    if (s != SV_OK) return s;
  }

  AcceptArgs ac;
  ac.info = ws_at<RowInfo>(workspace, p.off_info);
  ac.cout = ws_at<ChunkOut>(workspace, p.off_cout);
  ac.nchunks = p.nchunks;
  ac.logits = target_logits;
  ac.c = c.c;
  ac.c2 = c.c2;
  ac.cl = c.cl;
  ac.c64 = c.c64;
  ac.gath = gath;
  ac.kept = p.trunc ? ws_at<Cand>(workspace, p.off_kept) : nullptr;
  ac.kmax = kKMax;
  ac.q = q;
  ac.ids = draft_ids;
  ac.ua = u_accept;
  ac.ur = u_resample;
  ac.B = B;
  ac.gamma = gamma;
  ac.V = V;
  ac.out_tokens = out_tokens;
  ac.out_nacc = out_num_accepted;
  ac.out_flags = out_row_flags;
  ac.jobs = ws_at<BigJob>(workspace, p.off_jobs);
  ac.cu = cu;
  ac.n_draft = n_draft;
  ac.eos = eos;
  ac.beta = beta;
  const dim3 agrid((unsigned)((B + 3) / 4));
  if (p.trunc) {
    // kept lists (stored in token-id order) and oversized kept sets are
    // drawn inside K3, one workgroup per request
    if (bf) launch_stage(SV_STAGE_ACCEPT, accept_trunc_kernel<true>, dim3((unsigned)B), dim3(256), 0, st, ac);
    else launch_stage(SV_STAGE_ACCEPT, accept_trunc_kernel<false>, dim3((unsigned)B), dim3(256), 0, st, ac);
    return launched();
  }

  BigArgs bg;
  bg.logits = target_logits;
  bg.q = q;
  bg.V = V;
  bg.G1 = G1;
  bg.nch4 = p.nch4;
  bg.c64 = c.c64;
  bg.jobs = ac.jobs;
  bg.partials = ws_at<double>(workspace, p.off_part);
  bg.out_tokens = out_tokens;
  bg.out_flags = out_row_flags;
  bg.eos = eos;
  bg.beta = beta;
  const int64_t tiles_big = (V + 1024 * kSeg - 1) / (1024 * kSeg);  // tiles of the 1024-thread sampler
  if (G1 <= kWave && tiles_big <= kMaxTiles && B >= kOneLaunchMinB) {
    // one workgroup per request: decision, row weights and the draw
    if (V >= 16384) {
      if (bf) launch_stage(SV_STAGE_ACCEPT, sample_full_kernel<true, 1024>, dim3((unsigned)B), dim3(1024), 0, st, bg, ac);
      else launch_stage(SV_STAGE_ACCEPT, sample_full_kernel<false, 1024>, dim3((unsigned)B), dim3(1024), 0, st, bg, ac);
    } else {
      if (bf) launch_stage(SV_STAGE_ACCEPT, sample_full_kernel<true, 256>, dim3((unsigned)B), dim3(256), 0, st, bg, ac);
      else launch_stage(SV_STAGE_ACCEPT, sample_full_kernel<false, 256>, dim3((unsigned)B), dim3(256), 0, st, bg, ac);
    }
    return launched();
  }
  dim3 grid((unsigned)((int64_t)p.nch4 * B));
  if (G1 <= kWave) {
    // acceptance fused into the chunk weighing
    if (bf) launch_stage(SV_STAGE_ACCEPT, big_partial_kernel<true, true>, grid, dim3(256), 0, st, bg, ac);
    else launch_stage(SV_STAGE_ACCEPT, big_partial_kernel<false, true>, grid, dim3(256), 0, st, bg, ac);
  } else {
    if (bf) launch_stage(SV_STAGE_ACCEPT, accept_kernel<true>, agrid, dim3(256), 0, st, ac);
    else launch_stage(SV_STAGE_ACCEPT, accept_kernel<false>, agrid, dim3(256), 0, st, ac);
    s = launched();
    if (s != SV_OK) return s;
    if (bf) launch_stage(SV_STAGE_DRAW_PARTIAL, big_partial_kernel<true, false>, grid, dim3(256), 0, st, bg, ac);
    else launch_stage(SV_STAGE_DRAW_PARTIAL, big_partial_kernel<false, false>, grid, dim3(256), 0, st, bg, ac);
  }
  s = launched();
  if (s != SV_OK) return s;
  if (bf) launch_stage(SV_STAGE_DRAW_FINISH, big_finish_kernel<true>, dim3((unsigned)B), dim3(256), 0, st, bg);
  else launch_stage(SV_STAGE_DRAW_FINISH, big_finish_kernel<false>, dim3((unsigned)B), dim3(256), 0, st, bg);
  return launched();
}

// Outputs of the acceptance statistics (each [B, gamma] float32), and q's
// kept lists when q comes from truncated draft logits.
struct StatsOut {
  float* alpha;
  float* z_pq;
  float* z_qp;
  float* accept_prob;
  const Cand* qkept;
};

// The statistics kernels over target rows 0..gamma-1 whose row results sit
// in plan p's info / kept regions at rows b * info_rpr + j.
sv_status launch_stats(const Plan& p, const void* target_logits, bool bf, const QSrc& q, const StatsOut& so,
                       const int32_t* draft_ids, int32_t B, int32_t gamma, int32_t V, const Expo& c, int info_rpr,
                       void* workspace, hipStream_t st, hipEvent_t qsum_join) {
  StatsArgs a;
  a.logits = target_logits;
  a.q = q;
  a.qkept = so.qkept;
  a.ids = draft_ids;
  a.V = V;
  a.gamma = gamma;
  // Truncated rows whose statistics come from their kept lists need no
  // pass (a dense q's sum for Z' comes from qsum_kernel); only rows without
  // a list (rare) stream, one workgroup per row, so the launch is B * gamma
  // workgroups that mostly return at once.
  const bool lists = p.trunc;
  a.nchunks = lists ? 1 : p.nchunks;
  a.chunk = lists ? (int64_t)V : p.chunk;
  a.c64 = c.c64;
  a.info = ws_at<RowInfo>(workspace, p.off_info);
  a.kept = p.trunc ? ws_at<Cand>(workspace, p.off_kept) : nullptr;
  a.info_rpr = info_rpr;
  a.kmax = kKMax;
  a.partials = ws_at<double>(workspace, p.off_spart);
  a.p_s64 = nullptr;
  a.q_s64 = nullptr;
  a.s64_nch = p.nchunks;
  a.qsum = ws_at<double>(workspace, p.off_qsum);
  a.nchq = p.nchq;
  // listed rows with a dense q: Z' is completed after the q sums, so that
  // the rest of the finish runs beside them
  const bool defer_zqp = p.trunc && q.dense != nullptr && so.z_qp != nullptr;
  a.zqp_part = defer_zqp ? ws_at<double>(workspace, p.off_zqp) : nullptr;
  a.out_alpha = so.alpha;
  a.out_zpq = so.z_pq;
  a.out_zqp = so.z_qp;
  a.out_acc = so.accept_prob;
  a.rows = (int64_t)B * gamma;
  if (a.rows == 0) return SV_OK;
  dim3 grid((unsigned)(a.rows * a.nchunks));
  const bool qlog = q.dense == nullptr;
  if (!p.trunc) {
    // untruncated rows: their S64 first (the target's, then the draft's
    // when q comes from its logits), chunk by chunk
    double* s64 = ws_at<double>(workspace, p.off_s64);
    S64Args sa;
    sa.logits = target_logits;
    sa.info = a.info;
    sa.V = V;
    sa.gamma = gamma;
    sa.lrpr = gamma + 1;
    sa.info_rpr = info_rpr;
    sa.nchunks = p.nchunks;
    sa.chunk = p.chunk;
    sa.c64 = c.c64;
    sa.out = s64;
    const dim3 sgrid((unsigned)(a.rows * p.nchunks));
    if (bf) launch_stage(-1, s64_chunk_kernel<true>, sgrid, dim3(256), 0, st, sa);
    else launch_stage(-1, s64_chunk_kernel<false>, sgrid, dim3(256), 0, st, sa);
    sv_status s = launched();
    if (s != SV_OK) return s;
    a.p_s64 = s64;
    if (qlog) {
      sa.logits = q.z;
      sa.info = q.info;
      sa.lrpr = gamma;
      sa.info_rpr = gamma;
      sa.out = s64 + (size_t)a.rows * p.nchunks;
      if (q.zbf16) launch_stage(-1, s64_chunk_kernel<true>, sgrid, dim3(256), 0, st, sa);
      else launch_stage(-1, s64_chunk_kernel<false>, sgrid, dim3(256), 0, st, sa);
      s = launched();
      if (s != SV_OK) return s;
      a.q_s64 = sa.out;
    }
  }
  if (bf) {
    if (qlog) launch_stage(SV_STAGE_STATS_PASS, stats_chunk_kernel<true, true>, grid, dim3(256), 0, st, a);
    else launch_stage(SV_STAGE_STATS_PASS, stats_chunk_kernel<true, false>, grid, dim3(256), 0, st, a);
  } else {
    if (qlog) launch_stage(SV_STAGE_STATS_PASS, stats_chunk_kernel<false, true>, grid, dim3(256), 0, st, a);
    else launch_stage(SV_STAGE_STATS_PASS, stats_chunk_kernel<false, false>, grid, dim3(256), 0, st, a);
  }
  sv_status s = launched();
  if (s != SV_OK) return s;
  const dim3 fgrid((unsigned)((a.rows + 3) / 4));
  if (defer_zqp) {
    // the finish beside the q sums, then Z' once they are in
    if (bf) launch_stage(SV_STAGE_STATS_FINISH, stats_final_kernel<true>, fgrid, dim3(256), 0, st, a);
    else launch_stage(SV_STAGE_STATS_FINISH, stats_final_kernel<false>, fgrid, dim3(256), 0, st, a);
    s = launched();
    if (s != SV_OK) return s;
    if (qsum_join != nullptr && hipStreamWaitEvent(st, qsum_join, 0) != hipSuccess) return SV_ERR_HIP;
    launch_stage(SV_STAGE_STATS_ZQP, stats_zqp_kernel, fgrid, dim3(256), 0, st, a);
    return launched();
  }
  if (qsum_join != nullptr && hipStreamWaitEvent(st, qsum_join, 0) != hipSuccess) return SV_ERR_HIP;
  if (bf) launch_stage(SV_STAGE_STATS_FINISH, stats_final_kernel<true>, fgrid, dim3(256), 0, st, a);
  else launch_stage(SV_STAGE_STATS_FINISH, stats_final_kernel<false>, fgrid, dim3(256), 0, st, a);
  return launched();
}

// The statistics call once q's source is known (its own row passes over the
// target's rows 0..gamma-1, plan CALL_STATS).
sv_status accept_stats_impl(const Plan& p, const void* target_logits, sv_dtype dt, const QSrc& q, const StatsOut& so,
                            const int32_t* draft_ids, int32_t B, int32_t gamma, int32_t V, sv_sampling_params prm,
                            const Expo& c, void* workspace, hipStream_t st, hipEvent_t q_ready = nullptr) {
  const bool bf = dt == SV_BF16;
  const int G1 = gamma + 1;
  hipEvent_t join = nullptr;
  const SideStream* fork = nullptr;
  const bool qsum = q.dense != nullptr && so.z_qp != nullptr && p.trunc;
  sv_status s = bf ? run_rowpass<true>(p, target_logits, V, G1, c, workspace, st)
                   : run_rowpass<false>(p, target_logits, V, G1, c, workspace, st);
  if (s != SV_OK) return s;
  if (qsum) {
    // the dense-q row sums, beside the row finisher and the statistics pass
    fork = qsum_fork_point(st, &s);
    if (s != SV_OK) return s;
  }
  if (q_ready != nullptr && hipStreamWaitEvent(st, q_ready, 0) != hipSuccess) return SV_ERR_HIP;
  s = bf ? run_rowfinal<true>(p, target_logits, q, draft_ids, V, G1, gamma, c, prm, workspace, st)
         : run_rowfinal<false>(p, target_logits, q, draft_ids, V, G1, gamma, c, prm, workspace, st);
  if (s != SV_OK) return s;
  if (qsum) {
    join = launch_qsum(fork, p, q.dense, B, gamma, V, workspace, st, &s);
    if (s != SV_OK) return s;
  }
  return launch_stats(p, target_logits, bf, q, so, draft_ids, B, gamma, V, c, gamma, workspace, st, join);
}

// Row passes over the draft's logits [B, gamma, V] (plan CALL_DRAFT, in its
// own workspace region): their statistics and kept lists define q, which
// the target's passes then read through the returned source.
// A ragged batch (cu != null) packs its n_draft draft rows: plan row r is
// packed row r, the draft position the target's kernels read q at.
sv_status run_draft_rows(const void* draft_logits, sv_dtype ddt, const int32_t* draft_ids, int32_t B, int32_t gamma,
                         int32_t V, sv_sampling_params prm, const Expo& c, void* ws, hipStream_t st, QSrc* q_out,
                         const Cand** qkept_out, const int32_t* cu = nullptr, int32_t n_draft = 0) {
  const Plan pq = make_plan(CALL_DRAFT, B, gamma, V, ddt, prm);
  const bool bf = ddt == SV_BF16;
  sv_status s =
      bf ? run_rowpass<true>(pq, draft_logits, V, gamma, c, ws, st, nullptr, q_src_none(V), 0, nullptr, false, cu,
                             n_draft)
         : run_rowpass<false>(pq, draft_logits, V, gamma, c, ws, st, nullptr, q_src_none(V), 0, nullptr, false, cu,
                              n_draft);
  if (s != SV_OK) return s;
  s = bf ? run_rowfinal<true>(pq, draft_logits, q_src_none(V), draft_ids, V, gamma, gamma, c, prm, ws, st, cu, n_draft,
                              false)
         : run_rowfinal<false>(pq, draft_logits, q_src_none(V), draft_ids, V, gamma, gamma, c, prm, ws, st, cu,
                               n_draft, false);
  if (s != SV_OK) return s;
  QSrc q;
  q.dense = nullptr;
  q.z = draft_logits;
  q.info = ws_at<RowInfo>(ws, pq.off_info);
  q.V = V;
  q.c = c.c;
  q.c2 = c.c2;
  q.cl = c.cl;
  q.c64 = c.c64;
  q.zbf16 = bf ? 1 : 0;
  *q_out = q;
  *qkept_out = pq.trunc ? ws_at<Cand>(ws, pq.off_kept) : nullptr;
  return SV_OK;
}

// The draft rows' passes for a call whose target plan is p.  With truncated
// rows the target's row pass reads nothing of q, so the draft's passes run
// on the library's side stream (after the work already on the caller's
// stream), beside the target's row pass, and *q_ready is the event the
// caller's stream waits for before the target's row finisher, the first
// reader of q.  Otherwise (untruncated rows, whose row pass gathers q(d); no
// side stream) they run on the caller's stream and *q_ready is null.
sv_status draft_rows_beside(const Plan& p, const void* draft_logits, sv_dtype ddt, const int32_t* draft_ids,
                            int32_t B, int32_t gamma, int32_t V, sv_sampling_params prm, const Expo& c, void* ws,
                            hipStream_t st, QSrc* q_out, const Cand** qkept_out, hipEvent_t* q_ready,
                            const int32_t* cu = nullptr, int32_t n_draft = 0) {
  *q_ready = nullptr;
  const SideStream* ss = p.trunc ? side_stream(st) : nullptr;
  if (ss == nullptr) return run_draft_rows(draft_logits, ddt, draft_ids, B, gamma, V, prm, c, ws, st, q_out, qkept_out,
                                           cu, n_draft);
  if (hipEventRecord(ss->fork, st) != hipSuccess || hipStreamWaitEvent(ss->s, ss->fork, 0) != hipSuccess)
    return SV_ERR_HIP;
  sv_status s = run_draft_rows(draft_logits, ddt, draft_ids, B, gamma, V, prm, c, ws, ss->s, q_out, qkept_out, cu,
                               n_draft);
  if (s != SV_OK) return s;
  if (hipEventRecord(ss->join, ss->s) != hipSuccess) return SV_ERR_HIP;
  *q_ready = ss->join;
  return SV_OK;
}

// Workspace of the draft-logits calls: the target call's regions, then the
// draft rows' (at draft_ws_offset).
size_t draft_ws_offset(CallKind kind, int32_t B, int32_t gamma, int32_t V, sv_dtype dt, sv_sampling_params prm) {
  return align_up(make_plan(kind, B, gamma, V, dt, prm).total, 256);
}

// The sampling call and the statistics of its rows 0..gamma-1 from one pass
// over the target logits (plan CALL_SAMPLE_STATS): the statistics kernels
// read the sampling call's row results instead of recomputing them.
sv_status verify_sample_stats_impl(const Plan& p, const void* target_logits, sv_dtype dt, const QSrc& q,
                                   const StatsOut& so, const int32_t* draft_ids, const float* u_accept,
                                   const float* u_resample, int32_t B, int32_t gamma, int32_t V,
                                   sv_sampling_params prm, const Expo& c, int32_t* out_tokens, int32_t* out_num_accepted,
                                   uint32_t* out_row_flags, void* workspace, hipStream_t st,
                                   hipEvent_t q_ready = nullptr) {
  hipEvent_t join = nullptr;
  const SideStream* fork = nullptr;
  const bool qsum = q.dense != nullptr && so.z_qp != nullptr && p.trunc;
  sv_status s = verify_sample_impl(p, target_logits, dt, q, draft_ids, u_accept, u_resample, B, gamma, V, prm, c,
                                   out_tokens, out_num_accepted, out_row_flags, workspace, st, nullptr, 0, -1, 1.0,
                                   /*force_rowfinal=*/true, qsum ? &fork : nullptr, q_ready);
  if (s != SV_OK) return s;
  if (qsum) {
    // the dense-q row sums, behind the fork point after the row pass
    join = launch_qsum(fork, p, q.dense, B, gamma, V, workspace, st, &s);
    if (s != SV_OK) return s;
  }
  return launch_stats(p, target_logits, dt == SV_BF16, q, so, draft_ids, B, gamma, V, c, gamma + 1, workspace, st,
                      join);
}

// Greedy verify (uniform, or ragged with draft offsets `cu`).
sv_status verify_greedy_impl(const void* target_logits, sv_dtype dt, const int32_t* draft_ids, int32_t B,
                             int32_t gamma, int32_t V, int32_t* out_tokens, int32_t* out_num_accepted,
                             uint32_t* out_row_flags, void* workspace, size_t workspace_bytes, hipStream_t st,
                             const int32_t* cu = nullptr, int32_t n_draft = 0, int32_t eos = -1) {
  sv_sampling_params prm = {1.0f, 0, 1.0f};
  const Plan p = make_plan(CALL_GREEDY, B, gamma, V, dt, prm);
  if (workspace == nullptr || workspace_bytes < p.total || !aligned16(workspace)) return SV_ERR_WORKSPACE;
  const bool bf = dt == SV_BF16;
  sv_status s =
      bf ? run_rowpass<true>(p, target_logits, V, gamma + 1, kExpoGreedy, workspace, st, nullptr, QSrc{}, gamma,
                             nullptr, true, cu, n_draft + B)
         : run_rowpass<false>(p, target_logits, V, gamma + 1, kExpoGreedy, workspace, st, nullptr, QSrc{}, gamma,
                              nullptr, true, cu, n_draft + B);
  if (s != SV_OK) return s;
  GreedyArgs g;
  g.cout = ws_at<ChunkOut>(workspace, p.off_cout);
  g.nchunks = p.nchunks;
  g.ids = draft_ids;
  g.B = B;
  g.gamma = gamma;
  g.V = V;
  g.out_tokens = out_tokens;
  g.out_nacc = out_num_accepted;
  g.out_flags = out_row_flags;
  g.cu = cu;
  g.n_draft = n_draft;
  g.eos = eos;
  launch_stage(SV_STAGE_GREEDY, greedy_kernel, dim3((unsigned)((B + 3) / 4)), dim3(256), 0, st, g);
  return launched();
}

// Host checks of a ragged call's scalar arguments (the offsets themselves
// are device data, checked per request by the kernels).
sv_status ragged_checks(const int32_t* cu, int32_t n_draft, int32_t B, int32_t gamma_max, int32_t V, int32_t eos) {
  if (n_draft < 0 || (int64_t)n_draft > (int64_t)B * gamma_max) return SV_ERR_INVALID_ARG;
  if (B > 0 && cu == nullptr) return SV_ERR_INVALID_ARG;
  if (eos >= V) return SV_ERR_INVALID_ARG;
  return SV_OK;
}

}  // namespace

// ---- the allocation-free variant's scratch ------------------------------------
// One file-scope device array per GPU, used as the workspace of
// spec_verify_sample_noalloc.  Host code never passes the array's name to a
// kernel: its device address, per device, comes from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[SV_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch` (looked up once per device), or
// null when the device cannot be queried.
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

size_t spec_verify_workspace_size(int32_t B, int32_t gamma, int32_t V, sv_dtype dt, sv_sampling_params prm) {
  Expo c;
  if (check_sizes(B, gamma, V, dt) != SV_OK || check_params(prm, &c) != SV_OK) return 0;
  size_t a = make_plan(CALL_SAMPLE_STATS, B, gamma, V, dt, prm).total;  // covers CALL_SAMPLE
  size_t g = make_plan(CALL_GREEDY, B, gamma, V, dt, prm).total;
  size_t s = make_plan(CALL_STATS, B, gamma, V, dt, prm).total;
  return std::max(a, std::max(g, s));
}

sv_status spec_verify_sample(const void* target_logits, sv_dtype dt, const float* draft_probs,
                             const int32_t* draft_ids, const float* u_accept, const float* u_resample,
                             int32_t B, int32_t gamma, int32_t V, sv_sampling_params prm, int32_t* out_tokens,
                             int32_t* out_num_accepted, uint32_t* out_row_flags, void* workspace,
                             size_t workspace_bytes, void* stream) {
  sv_status s = common_checks(target_logits, dt, B, gamma, V);
  if (s != SV_OK) return s;
  Expo c;
  s = check_params(prm, &c);
  if (s != SV_OK) return s;
  if (B == 0) return SV_OK;
  if (u_resample == nullptr || out_tokens == nullptr || out_num_accepted == nullptr) return SV_ERR_INVALID_ARG;
  if (gamma > 0 && (draft_probs == nullptr || draft_ids == nullptr || u_accept == nullptr || !aligned16(draft_probs)))
    return SV_ERR_INVALID_ARG;
  const Plan p = make_plan(CALL_SAMPLE, B, gamma, V, dt, prm);
  if (workspace == nullptr || workspace_bytes < p.total || !aligned16(workspace)) return SV_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  return verify_sample_impl(p, target_logits, dt, q_src_dense(draft_probs, V), draft_ids, u_accept, u_resample, B,
                            gamma, V, prm, c, out_tokens, out_num_accepted, out_row_flags, workspace, st);
}

sv_status spec_verify_sample_noalloc(const void* target_logits, sv_dtype dt, const float* draft_probs,
                                     const int32_t* draft_ids, const float* u_accept, const float* u_resample,
                                     int32_t B, int32_t gamma, int32_t V, sv_sampling_params prm,
                                     int32_t* out_tokens, int32_t* out_num_accepted, uint32_t* out_row_flags,
                                     void* stream) {
  sv_status s = common_checks(target_logits, dt, B, gamma, V);
  if (s != SV_OK) return s;
  Expo c;
  s = check_params(prm, &c);
  if (s != SV_OK) return s;
  if (B == 0) return SV_OK;
  if (u_resample == nullptr || out_tokens == nullptr || out_num_accepted == nullptr) return SV_ERR_INVALID_ARG;
  if (gamma > 0 && (draft_probs == nullptr || draft_ids == nullptr || u_accept == nullptr || !aligned16(draft_probs)))
    return SV_ERR_INVALID_ARG;
  const Plan p = make_plan(CALL_SAMPLE, B, gamma, V, dt, prm);
  if (p.total > (size_t)SV_NOALLOC_SCRATCH_BYTES) return SV_ERR_UNSUPPORTED;  // beyond the static scratch
  void* ws = scratch_on_current_device();
  if (ws == nullptr) return SV_ERR_HIP;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  return verify_sample_impl(p, target_logits, dt, q_src_dense(draft_probs, V), draft_ids, u_accept, u_resample, B,
                            gamma, V, prm, c, out_tokens, out_num_accepted, out_row_flags, ws, st);
}

sv_status spec_verify_sample_stats(const void* target_logits, sv_dtype dt, const float* draft_probs,
                                   const int32_t* draft_ids, const float* u_accept, const float* u_resample,
                                   int32_t B, int32_t gamma, int32_t V, sv_sampling_params prm, int32_t* out_tokens,
                                   int32_t* out_num_accepted, uint32_t* out_row_flags, float* out_alpha,
                                   float* out_z_pq, float* out_z_qp, float* out_accept_prob, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  sv_status s = common_checks(target_logits, dt, B, gamma, V);
  if (s != SV_OK) return s;
  Expo c;
  s = check_params(prm, &c);
  if (s != SV_OK) return s;
  if (B == 0) return SV_OK;
  if (u_resample == nullptr || out_tokens == nullptr || out_num_accepted == nullptr) return SV_ERR_INVALID_ARG;
  if (gamma > 0 && (draft_probs == nullptr || draft_ids == nullptr || u_accept == nullptr || !aligned16(draft_probs)))
    return SV_ERR_INVALID_ARG;
  const Plan p = make_plan(CALL_SAMPLE_STATS, B, gamma, V, dt, prm);
  if (workspace == nullptr || workspace_bytes < p.total || !aligned16(workspace)) return SV_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const StatsOut so{out_alpha, out_z_pq, out_z_qp, out_accept_prob, nullptr};
  return verify_sample_stats_impl(p, target_logits, dt, q_src_dense(draft_probs, V), so, draft_ids, u_accept,
                                  u_resample, B, gamma, V, prm, c, out_tokens, out_num_accepted, out_row_flags,
                                  workspace, st);
}

sv_status spec_verify_greedy(const void* target_logits, sv_dtype dt, const int32_t* draft_ids, int32_t B,
                             int32_t gamma, int32_t V, int32_t* out_tokens, int32_t* out_num_accepted,
                             uint32_t* out_row_flags, void* workspace, size_t workspace_bytes, void* stream) {
  sv_status s = common_checks(target_logits, dt, B, gamma, V);
  if (s != SV_OK) return s;
  if (B == 0) return SV_OK;
  if (out_tokens == nullptr || out_num_accepted == nullptr) return SV_ERR_INVALID_ARG;
  if (gamma > 0 && draft_ids == nullptr) return SV_ERR_INVALID_ARG;
  return verify_greedy_impl(target_logits, dt, draft_ids, B, gamma, V, out_tokens, out_num_accepted, out_row_flags,
                            workspace, workspace_bytes, reinterpret_cast<hipStream_t>(stream));
}

sv_status spec_accept_stats(const void* target_logits, sv_dtype dt, const float* draft_probs,
                            const int32_t* draft_ids, int32_t B, int32_t gamma, int32_t V,
                            sv_sampling_params prm, float* out_alpha, float* out_z_pq, float* out_z_qp,
                            float* out_accept_prob, void* workspace, size_t workspace_bytes, void* stream) {
  sv_status s = common_checks(target_logits, dt, B, gamma, V);
  if (s != SV_OK) return s;
  Expo c;
  s = check_params(prm, &c);
  if (s != SV_OK) return s;
  if (B == 0 || gamma == 0) return SV_OK;
  if (draft_probs == nullptr || draft_ids == nullptr || !aligned16(draft_probs)) return SV_ERR_INVALID_ARG;
  const Plan p = make_plan(CALL_STATS, B, gamma, V, dt, prm);
  if (workspace == nullptr || workspace_bytes < p.total || !aligned16(workspace)) return SV_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const StatsOut so{out_alpha, out_z_pq, out_z_qp, out_accept_prob, nullptr};
  return accept_stats_impl(p, target_logits, dt, q_src_dense(draft_probs, V), so, draft_ids, B, gamma, V, prm, c,
                           workspace, st);
}

size_t spec_verify_draft_logits_workspace_size(int32_t B, int32_t gamma, int32_t V, sv_dtype dt, sv_dtype draft_dt,
                                               sv_sampling_params prm) {
  Expo c;
  if (check_sizes(B, gamma, V, dt) != SV_OK || check_sizes(B, gamma, V, draft_dt) != SV_OK ||
      check_params(prm, &c) != SV_OK)
    return 0;
  const size_t d = make_plan(CALL_DRAFT, B, gamma, V, draft_dt, prm).total;
  const size_t a = draft_ws_offset(CALL_SAMPLE_STATS, B, gamma, V, dt, prm) + d;  // covers CALL_SAMPLE
  const size_t s = draft_ws_offset(CALL_STATS, B, gamma, V, dt, prm) + d;
  return std::max(a, s);
}

sv_status spec_verify_sample_draft_logits(const void* target_logits, sv_dtype dt, const void* draft_logits,
                                          sv_dtype draft_dt, const int32_t* draft_ids, const float* u_accept,
                                          const float* u_resample, int32_t B, int32_t gamma, int32_t V,
                                          sv_sampling_params prm, int32_t* out_tokens, int32_t* out_num_accepted,
                                          uint32_t* out_row_flags, void* workspace, size_t workspace_bytes,
                                          void* stream) {
  sv_status s = common_checks(target_logits, dt, B, gamma, V);
  if (s != SV_OK) return s;
  if (draft_dt != SV_F32 && draft_dt != SV_BF16) return SV_ERR_INVALID_ARG;
  Expo c;
  s = check_params(prm, &c);
  if (s != SV_OK) return s;
  if (B == 0) return SV_OK;
  if (u_resample == nullptr || out_tokens == nullptr || out_num_accepted == nullptr) return SV_ERR_INVALID_ARG;
  if (gamma > 0 && (draft_logits == nullptr || draft_ids == nullptr || u_accept == nullptr || !aligned16(draft_logits)))
    return SV_ERR_INVALID_ARG;
  const Plan p = make_plan(CALL_SAMPLE, B, gamma, V, dt, prm);
  const size_t qoff = draft_ws_offset(CALL_SAMPLE, B, gamma, V, dt, prm);
  const size_t need = qoff + make_plan(CALL_DRAFT, B, gamma, V, draft_dt, prm).total;
  if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)) return SV_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  QSrc q = q_src_none(V);
  const Cand* qkept = nullptr;
  hipEvent_t q_ready = nullptr;
  if (gamma > 0) {
    s = draft_rows_beside(p, draft_logits, draft_dt, draft_ids, B, gamma, V, prm, c,
                          static_cast<unsigned char*>(workspace) + qoff, st, &q, &qkept, &q_ready);
    if (s != SV_OK) return s;
  }
  return verify_sample_impl(p, target_logits, dt, q, draft_ids, u_accept, u_resample, B, gamma, V, prm, c, out_tokens,
                            out_num_accepted, out_row_flags, workspace, st, nullptr, 0, -1, 1.0, false, nullptr,
                            q_ready);
}

sv_status spec_accept_stats_draft_logits(const void* target_logits, sv_dtype dt, const void* draft_logits,
                                         sv_dtype draft_dt, const int32_t* draft_ids, int32_t B, int32_t gamma,
                                         int32_t V, sv_sampling_params prm, float* out_alpha, float* out_z_pq,
                                         float* out_z_qp, float* out_accept_prob, void* workspace,
                                         size_t workspace_bytes, void* stream) {
  sv_status s = common_checks(target_logits, dt, B, gamma, V);
  if (s != SV_OK) return s;
  if (draft_dt != SV_F32 && draft_dt != SV_BF16) return SV_ERR_INVALID_ARG;
  Expo c;
  s = check_params(prm, &c);
  if (s != SV_OK) return s;
  if (B == 0 || gamma == 0) return SV_OK;
  if (draft_logits == nullptr || draft_ids == nullptr || !aligned16(draft_logits)) return SV_ERR_INVALID_ARG;
  const Plan p = make_plan(CALL_STATS, B, gamma, V, dt, prm);
  const size_t qoff = draft_ws_offset(CALL_STATS, B, gamma, V, dt, prm);
  const size_t need = qoff + make_plan(CALL_DRAFT, B, gamma, V, draft_dt, prm).total;
  if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)) return SV_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  QSrc q;
  const Cand* qkept = nullptr;
  hipEvent_t q_ready = nullptr;
  s = draft_rows_beside(p, draft_logits, draft_dt, draft_ids, B, gamma, V, prm, c,
                        static_cast<unsigned char*>(workspace) + qoff, st, &q, &qkept, &q_ready);
  if (s != SV_OK) return s;
  const StatsOut so{out_alpha, out_z_pq, out_z_qp, out_accept_prob, qkept};
  return accept_stats_impl(p, target_logits, dt, q, so, draft_ids, B, gamma, V, prm, c, workspace, st, q_ready);
}

sv_status spec_verify_sample_stats_draft_logits(const void* target_logits, sv_dtype dt, const void* draft_logits,
                                               sv_dtype draft_dt, const int32_t* draft_ids, const float* u_accept,
                                               const float* u_resample, int32_t B, int32_t gamma, int32_t V,
                                               sv_sampling_params prm, int32_t* out_tokens, int32_t* out_num_accepted,
                                               uint32_t* out_row_flags, float* out_alpha, float* out_z_pq,
                                               float* out_z_qp, float* out_accept_prob, void* workspace,
                                               size_t workspace_bytes, void* stream) {
  sv_status s = common_checks(target_logits, dt, B, gamma, V);
  if (s != SV_OK) return s;
  if (draft_dt != SV_F32 && draft_dt != SV_BF16) return SV_ERR_INVALID_ARG;
  Expo c;
  s = check_params(prm, &c);
  if (s != SV_OK) return s;
  if (B == 0) return SV_OK;
  if (u_resample == nullptr || out_tokens == nullptr || out_num_accepted == nullptr) return SV_ERR_INVALID_ARG;
  if (gamma > 0 && (draft_logits == nullptr || draft_ids == nullptr || u_accept == nullptr || !aligned16(draft_logits)))
    return SV_ERR_INVALID_ARG;
  const Plan p = make_plan(CALL_SAMPLE_STATS, B, gamma, V, dt, prm);
  const size_t qoff = draft_ws_offset(CALL_SAMPLE_STATS, B, gamma, V, dt, prm);
  const size_t need = qoff + make_plan(CALL_DRAFT, B, gamma, V, draft_dt, prm).total;
  if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)) return SV_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  QSrc q = q_src_none(V);
  const Cand* qkept = nullptr;
  hipEvent_t q_ready = nullptr;
  if (gamma > 0) {
    s = draft_rows_beside(p, draft_logits, draft_dt, draft_ids, B, gamma, V, prm, c,
                          static_cast<unsigned char*>(workspace) + qoff, st, &q, &qkept, &q_ready);
    if (s != SV_OK) return s;
  }
  const StatsOut so{out_alpha, out_z_pq, out_z_qp, out_accept_prob, qkept};
  return verify_sample_stats_impl(p, target_logits, dt, q, so, draft_ids, u_accept, u_resample, B, gamma, V, prm, c,
                                  out_tokens, out_num_accepted, out_row_flags, workspace, st, q_ready);
}

sv_status spec_verify_sample_lenient(const void* target_logits, sv_dtype dt, const float* draft_probs,
                                     const int32_t* draft_ids, const float* u_accept, const float* u_resample,
                                     int32_t B, int32_t gamma, int32_t V, sv_sampling_params prm, float lenience,
                                     int32_t* out_tokens, int32_t* out_num_accepted, uint32_t* out_row_flags,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  if (!(lenience > 0.0f && lenience <= 1.0f)) return SV_ERR_INVALID_ARG;
  sv_status s = common_checks(target_logits, dt, B, gamma, V);
  if (s != SV_OK) return s;
  Expo c;
  s = check_params(prm, &c);
  if (s != SV_OK) return s;
  if (B == 0) return SV_OK;
  if (u_resample == nullptr || out_tokens == nullptr || out_num_accepted == nullptr) return SV_ERR_INVALID_ARG;
  if (gamma > 0 && (draft_probs == nullptr || draft_ids == nullptr || u_accept == nullptr || !aligned16(draft_probs)))
    return SV_ERR_INVALID_ARG;
  const Plan p = make_plan(CALL_SAMPLE, B, gamma, V, dt, prm);
  if (workspace == nullptr || workspace_bytes < p.total || !aligned16(workspace)) return SV_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  return verify_sample_impl(p, target_logits, dt, q_src_dense(draft_probs, V), draft_ids, u_accept, u_resample, B,
                            gamma, V, prm, c, out_tokens, out_num_accepted, out_row_flags, workspace, st, nullptr, 0,
                            -1, (double)lenience);
}

sv_status spec_verify_sample_ragged(const void* target_logits, sv_dtype dt, const float* draft_probs,
                                    const int32_t* draft_ids, const int32_t* cu_draft, int32_t n_draft,
                                    const float* u_accept, const float* u_resample, int32_t B, int32_t gamma_max,
                                    int32_t V, sv_sampling_params prm, int32_t eos_id, int32_t* out_tokens,
                                    int32_t* out_num_accepted, uint32_t* out_row_flags, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  sv_status s = common_checks(target_logits, dt, B, gamma_max, V);
  if (s != SV_OK) return s;
  s = ragged_checks(cu_draft, n_draft, B, gamma_max, V, eos_id);
  if (s != SV_OK) return s;
  Expo c;
  s = check_params(prm, &c);
  if (s != SV_OK) return s;
  if (B == 0) return SV_OK;
  if (u_resample == nullptr || out_tokens == nullptr || out_num_accepted == nullptr) return SV_ERR_INVALID_ARG;
  if (n_draft > 0 &&
      (draft_probs == nullptr || draft_ids == nullptr || u_accept == nullptr || !aligned16(draft_probs)))
    return SV_ERR_INVALID_ARG;
  const Plan p = make_plan(CALL_SAMPLE, B, gamma_max, V, dt, prm);
  if (workspace == nullptr || workspace_bytes < p.total || !aligned16(workspace)) return SV_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  return verify_sample_impl(p, target_logits, dt, q_src_dense(draft_probs, V), draft_ids, u_accept, u_resample, B,
                            gamma_max, V, prm, c, out_tokens, out_num_accepted, out_row_flags, workspace, st, cu_draft,
                            n_draft, eos_id < 0 ? -1 : eos_id);
}

sv_status spec_verify_sample_ragged_draft_logits(const void* target_logits, sv_dtype dt, const void* draft_logits,
                                                sv_dtype draft_dt, const int32_t* draft_ids, const int32_t* cu_draft,
                                                int32_t n_draft, const float* u_accept, const float* u_resample,
                                                int32_t B, int32_t gamma_max, int32_t V, sv_sampling_params prm,
                                                int32_t eos_id, int32_t* out_tokens, int32_t* out_num_accepted,
                                                uint32_t* out_row_flags, void* workspace, size_t workspace_bytes,
                                                void* stream) {
  sv_status s = common_checks(target_logits, dt, B, gamma_max, V);
  if (s != SV_OK) return s;
  if (draft_dt != SV_F32 && draft_dt != SV_BF16) return SV_ERR_INVALID_ARG;
  s = ragged_checks(cu_draft, n_draft, B, gamma_max, V, eos_id);
  if (s != SV_OK) return s;
  Expo c;
  s = check_params(prm, &c);
  if (s != SV_OK) return s;
  if (B == 0) return SV_OK;
  if (u_resample == nullptr || out_tokens == nullptr || out_num_accepted == nullptr) return SV_ERR_INVALID_ARG;
  if (n_draft > 0 &&
      (draft_logits == nullptr || draft_ids == nullptr || u_accept == nullptr || !aligned16(draft_logits)))
    return SV_ERR_INVALID_ARG;
  const Plan p = make_plan(CALL_SAMPLE, B, gamma_max, V, dt, prm);
  const size_t qoff = draft_ws_offset(CALL_SAMPLE, B, gamma_max, V, dt, prm);
  const size_t need = qoff + make_plan(CALL_DRAFT, B, gamma_max, V, draft_dt, prm).total;
  if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)) return SV_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  QSrc q = q_src_none(V);
  const Cand* qkept = nullptr;
  hipEvent_t q_ready = nullptr;
  if (n_draft > 0) {
    s = draft_rows_beside(p, draft_logits, draft_dt, draft_ids, B, gamma_max, V, prm, c,
                          static_cast<unsigned char*>(workspace) + qoff, st, &q, &qkept, &q_ready, cu_draft, n_draft);
    if (s != SV_OK) return s;
  }
  return verify_sample_impl(p, target_logits, dt, q, draft_ids, u_accept, u_resample, B, gamma_max, V, prm, c,
                            out_tokens, out_num_accepted, out_row_flags, workspace, st, cu_draft, n_draft,
                            eos_id < 0 ? -1 : eos_id, 1.0, false, nullptr, q_ready);
}

sv_status spec_verify_greedy_ragged(const void* target_logits, sv_dtype dt, const int32_t* draft_ids,
                                    const int32_t* cu_draft, int32_t n_draft, int32_t B, int32_t gamma_max,
                                    int32_t V, int32_t eos_id, int32_t* out_tokens, int32_t* out_num_accepted,
                                    uint32_t* out_row_flags, void* workspace, size_t workspace_bytes, void* stream) {
  sv_status s = common_checks(target_logits, dt, B, gamma_max, V);
  if (s != SV_OK) return s;
  s = ragged_checks(cu_draft, n_draft, B, gamma_max, V, eos_id);
  if (s != SV_OK) return s;
  if (B == 0) return SV_OK;
  if (out_tokens == nullptr || out_num_accepted == nullptr) return SV_ERR_INVALID_ARG;
  if (n_draft > 0 && draft_ids == nullptr) return SV_ERR_INVALID_ARG;
  return verify_greedy_impl(target_logits, dt, draft_ids, B, gamma_max, V, out_tokens, out_num_accepted,
                            out_row_flags, workspace, workspace_bytes, reinterpret_cast<hipStream_t>(stream),
                            cu_draft, n_draft, eos_id < 0 ? -1 : eos_id);
}

sv_status spec_set_stage_timer(int32_t stage, void* start_event, void* stop_event) {
  if (stage < 0 || stage >= SV_STAGE_COUNT) return SV_ERR_INVALID_ARG;
  if (start_event == nullptr || stop_event == nullptr) {
    g_timer_start[stage] = nullptr;
    g_timer_stop[stage] = nullptr;
  } else {
    g_timer_start[stage] = reinterpret_cast<hipEvent_t>(start_event);
    g_timer_stop[stage] = reinterpret_cast<hipEvent_t>(stop_event);
  }
  return SV_OK;
}

sv_status spec_set_rowpass_timer(void* start_event, void* stop_event) {
  return spec_set_stage_timer(SV_STAGE_ROWPASS, start_event, stop_event);
}

const char* spec_status_string(sv_status status) {
  switch (status) {
    case SV_OK: return "ok";
    case SV_ERR_INVALID_ARG: return "invalid argument";
    case SV_ERR_UNSUPPORTED: return "unsupported size";
    case SV_ERR_WORKSPACE: return "workspace missing or too small";
    case SV_ERR_HIP: return "HIP launch error";
  }
  return "unknown status";
}

}  // extern "C"
