// C ABI of the GSPN propagation: host-side validation (no HIP call before an
// argument is known to be good), plan choice, workspace handling and launch.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "gspn.h"
#include "gspn_device.hpp"
#include "gspn_launch.hpp"

namespace {

thread_local std::string g_last_error;
thread_local hipEvent_t* g_trace_events = nullptr;
thread_local int g_trace_pairs = 0;
thread_local int g_trace_count = 0;
thread_local const char* g_trace_names[gspn::kTraceMax] = {};
thread_local int64_t g_trace_planes[gspn::kTraceMax] = {};

gspn_status fail(gspn_status s, const std::string& detail) {
  g_last_error = detail;
  return s;
}

size_t elem_size(gspn_dtype dt) { return dt == GSPN_F32 ? 4 : 2; }
size_t al256_(size_t v) { return (v + 255) & ~size_t(255); }

// Scratch memory of gspn_propagate_noalloc: one statically sized array per
// device, held from the library's load until the process ends. Host code never
// passes the array's name to a kernel (on the host it is only a stand-in for
// the symbol); it uses the device address that hipGetSymbolAddress returns,
// looked up once per device with that device current.
constexpr size_t kNoallocScratchBytes = size_t(64) << 20;
__device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

enum class Plan { kInvalid, kPlane16, kPlane64, kBand, kTpipe, kTpipeT, kLarge, kStream, kDirs };

// Planes at least this large that no pipeline takes go through transposed
// copies (kLarge) rather than the streaming path, whose horizontal passes
// read with a stride.
constexpr int64_t kLargePlane = 256 * 256;

// workspace of the transposed pipeline: the six inputs and out transposed,
// then the pipeline's own workspace for the transposed shape
size_t tpipe_t_workspace_bytes(int64_t planes, int64_t H, int64_t W, gspn_dtype dt) {
  const size_t t = al256_(static_cast<size_t>(planes * H * W) * (dt == GSPN_F32 ? 4 : 2));
  return 7 * t + gspn::tpipe_workspace_bytes(planes, W, H, dt);
}

struct Checked {
  gspn_status status;
  Plan plan;
  size_t ws_bytes;
};

// Pure host logic: shape, mask, group, dtype limits and the plan they lead to.
Checked check_shape(int64_t B, int64_t C, int64_t H, int64_t W, uint32_t mask,
                    int64_t G, int dtype) {
  Checked r{GSPN_OK, Plan::kInvalid, 0};
  if (dtype != GSPN_F32 && dtype != GSPN_BF16) {
    r.status = fail(GSPN_E_DTYPE, "dtype must be GSPN_F32 or GSPN_BF16");
    return r;
  }
  if (B < 0 || C < 0 || H < 1 || W < 1) {
    r.status = fail(GSPN_E_SHAPE, "need B >= 0, C >= 0, H >= 1, W >= 1");
    return r;
  }
  const int64_t kMax = int64_t(1) << 31;
  if (H >= kMax || W >= kMax || (B > 0 && C > INT64_MAX / B)) {
    r.status = fail(GSPN_E_SHAPE, "dimension too large");
    return r;
  }
  const int64_t planes = B * C;
  if (H > INT64_MAX / W || (planes > 0 && H * W > INT64_MAX / 8 / planes)) {
    r.status = fail(GSPN_E_SHAPE, "tensor size overflows");
    return r;
  }
  if (planes >= kMax) {
    r.status = fail(GSPN_E_SHAPE, "B * C must be below 2^31");
    return r;
  }
  if (mask == 0 || mask > GSPN_ALL) {
    r.status = fail(GSPN_E_DIRMASK, "dir_mask must be a non-empty subset of GSPN_ALL");
    return r;
  }
  if (G < 0) {
    r.status = fail(GSPN_E_GROUP, "group_rows must be >= 0");
    return r;
  }
  // GSPN_FORCE_PLAN=plane|band|tpipe|tpipe_t|large|stream picks a path for testing when
  // the shape allows it; otherwise the first path that fits, in that order.
  const char* force = std::getenv("GSPN_FORCE_PLAN");
  const bool f_plane = force && !std::strcmp(force, "plane");
  const bool f_band = force && !std::strcmp(force, "band");
  const bool f_tpipe = force && !std::strcmp(force, "tpipe");
  const bool f_stream = force && !std::strcmp(force, "stream");
  const bool f_tpipe_t = force && !std::strcmp(force, "tpipe_t");
  const bool f_large = force && !std::strcmp(force, "large");
  const bool any = !f_plane && !f_band && !f_tpipe && !f_stream && !f_tpipe_t && !f_large;
  const bool stream_ok = H <= gspn::stream_max_orth() && W <= gspn::stream_max_orth();
  const gspn_dtype dt = static_cast<gspn_dtype>(dtype);
  if ((any || f_plane) && gspn::plane_fits(H, W)) {
    r.plan = gspn::plane_seg(H, W) == 16 ? Plan::kPlane16 : Plan::kPlane64;
  } else if ((any || f_band) && gspn::band_fits(H, W, G)) {
    r.plan = Plan::kBand;
  } else if ((any || f_tpipe) && gspn::tpipe_fits(H, W)) {
    r.plan = Plan::kTpipe;
    r.ws_bytes = gspn::tpipe_workspace_bytes(planes, H, W, dt);
  } else if ((any || f_tpipe_t) && gspn::tpipe_fits(W, H)) {
    // the pipeline on transposed copies; the pipeline's limits are symmetric,
    // so this is reached only when forced (kept for comparison)
    r.plan = Plan::kTpipeT;
    r.ws_bytes = tpipe_t_workspace_bytes(planes, H, W, dt);
  } else if ((any || f_large) && !gspn::plane_fits(H, W) && H <= gspn::dirs_max_orth() &&
             W <= gspn::dirs_max_orth() && (f_large || H * W >= kLargePlane)) {
    // horizontal directions over transposed copies; the streaming path's
    // fp32 accumulator (taken instead for channel-shared logits) fits in
    // the same workspace
    r.plan = Plan::kLarge;
    r.ws_bytes = gspn::dirs_workspace_bytes(planes, H, W, mask, dt);
    const int nd = __builtin_popcount(mask);
    if (nd > 1) r.ws_bytes = std::max(r.ws_bytes, static_cast<size_t>(planes * H * W) * sizeof(float));
  } else if (stream_ok && (any || f_stream || !gspn::plane_fits(H, W))) {
    r.plan = Plan::kStream;
    const int nd = __builtin_popcount(mask);
    if (nd > 1) r.ws_bytes = static_cast<size_t>(planes * H * W) * sizeof(float);
  } else if (gspn::plane_fits(H, W)) {
    r.plan = gspn::plane_seg(H, W) == 16 ? Plan::kPlane16 : Plan::kPlane64;
  } else {
    r.status = fail(GSPN_E_SHAPE, "H and W must be <= 16384 for planes above 64x64");
    return r;
  }
  return r;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return na > 0 && nb > 0 && pa < pb + nb && pb < pa + na;
}

// logit_channels must divide C (channel c reads logit channel c / (C / Cl))
gspn_status check_logit_channels(int64_t C, int64_t Cl) {
  if (Cl < 1 || (C > 0 && C % Cl != 0))
    return fail(GSPN_E_SHAPE, "logit_channels must be >= 1 and divide C");
  return GSPN_OK;
}

gspn_status check_all(const void* x, const void* const w_logits[3], const void* lambda,
                      const void* u, int64_t B, int64_t C, int64_t H, int64_t W,
                      uint32_t mask, int64_t G, gspn_dtype dtype, void* out,
                      Checked* chk, gspn::Problem* pr, int64_t Cl) {
  g_last_error.clear();
  if (!x || !w_logits || !lambda || !u || !out)
    return fail(GSPN_E_NULL, "x, w_logits, lambda, u and out must be non-null");
  if (!w_logits[0] || !w_logits[1] || !w_logits[2])
    return fail(GSPN_E_NULL, "w_logits[0..2] must be non-null");
  *chk = check_shape(B, C, H, W, mask, G, static_cast<int>(dtype));
  if (chk->status != GSPN_OK) return chk->status;
  if (check_logit_channels(C, Cl) != GSPN_OK) {
    chk->status = GSPN_E_SHAPE;
    return GSPN_E_SHAPE;
  }
  const size_t es = elem_size(dtype);
  const void* ins[6] = {x, w_logits[0], w_logits[1], w_logits[2], lambda, u};
  bool vec4 = true, pair = true;
  for (const void* p : ins) {
    const uintptr_t v = reinterpret_cast<uintptr_t>(p);
    if (v % es) return fail(GSPN_E_ALIGN, "input pointer not aligned to its element size");
    if (v % (4 * es)) vec4 = false;
    if (v % (2 * es)) pair = false;
  }
  const uintptr_t vo = reinterpret_cast<uintptr_t>(out);
  if (vo % es) return fail(GSPN_E_ALIGN, "out not aligned to its element size");
  if (vo % (4 * es)) vec4 = false;
  if (vo % (2 * es)) pair = false;
  const size_t bytes = static_cast<size_t>(B * C * H * W) * es;
  const size_t lbytes = static_cast<size_t>(B * Cl * H * W) * es;
  for (int i = 0; i < 6; ++i)
    if (overlaps(out, bytes, ins[i], i >= 1 && i <= 3 ? lbytes : bytes))
      return fail(GSPN_E_ALIAS, "out overlaps an input");
  pr->x = x;
  pr->l[0] = w_logits[0];
  pr->l[1] = w_logits[1];
  pr->l[2] = w_logits[2];
  pr->lam = lambda;
  pr->u = u;
  pr->out = out;
  pr->B = B; pr->C = C; pr->H = H; pr->W = W;
  pr->mask = mask;
  pr->G = G;
  pr->dtype = dtype;
  pr->aligned_vec4 = vec4;
  pr->aligned_pair = pair;
  pr->Cl = Cl;
  return GSPN_OK;
}

// The pipeline on the transposed planes. Transposing a plane swaps the
// axes: top->bottom on the transpose is left->right on the plane (the
// neighbour at orthogonal offset k - 1 keeps its logit), bottom->top is
// right->left, and the reverse; local groups are the same blocks on both
// axes. So the six inputs are transposed, the pipeline runs with the
// direction mask swapped between the axes, and its output is transposed
// back.
template <typename T>
hipError_t run_tpipe_t_dt(const gspn::Problem& pr, void* ws, hipStream_t stream,
                          gspn::Tracer* tr) {
  const int64_t planes = pr.B * pr.C, lplanes = pr.B * pr.Cl;
  const int H = static_cast<int>(pr.H), W = static_cast<int>(pr.W);
  const size_t t = al256_(static_cast<size_t>(planes * H * W) * sizeof(T));
  char* w = static_cast<char*>(ws);
  T* xt = reinterpret_cast<T*>(w);
  T* lamt = reinterpret_cast<T*>(w + t);
  T* ut = reinterpret_cast<T*>(w + 2 * t);
  T* lt[3] = {reinterpret_cast<T*>(w + 3 * t), reinterpret_cast<T*>(w + 4 * t),
              reinterpret_cast<T*>(w + 5 * t)};
  T* outt = reinterpret_cast<T*>(w + 6 * t);
  const T* s1[3] = {static_cast<const T*>(pr.x), static_cast<const T*>(pr.lam),
                    static_cast<const T*>(pr.u)};
  T* d1[3] = {xt, lamt, ut};
  hipError_t e = gspn::transpose_planes<T>(s1, d1, 3, planes, H, W, "tp_t_in", stream, tr);
  if (e != hipSuccess) return e;
  const T* s2[3] = {static_cast<const T*>(pr.l[0]), static_cast<const T*>(pr.l[1]),
                    static_cast<const T*>(pr.l[2])};
  if ((e = gspn::transpose_planes<T>(s2, lt, 3, lplanes, H, W, "tp_t_in", stream, tr)) !=
      hipSuccess)
    return e;
  gspn::Problem pt = pr;
  pt.x = xt;
  pt.lam = lamt;
  pt.u = ut;
  for (int k = 0; k < 3; ++k) pt.l[k] = lt[k];
  pt.out = outt;
  pt.H = pr.W;
  pt.W = pr.H;
  pt.mask = ((pr.mask & 3u) << 2) | ((pr.mask >> 2) & 3u);
  pt.aligned_vec4 = false;
  pt.aligned_pair = true;
  if ((e = gspn::launch_tpipe(pt, w + 7 * t, stream, tr)) != hipSuccess) return e;
  const T* s3[1] = {outt};
  T* d3[1] = {static_cast<T*>(pr.out)};
  return gspn::transpose_planes<T>(s3, d3, 1, planes, W, H, "tp_t_out", stream, tr);
}

hipError_t run_tpipe_t(const gspn::Problem& pr, void* ws, hipStream_t stream, gspn::Tracer* tr) {
  if (pr.dtype == GSPN_F32) return run_tpipe_t_dt<float>(pr, ws, stream, tr);
  return run_tpipe_t_dt<gspn::bf16_t>(pr, ws, stream, tr);
}

// `cont`: a tracer that already holds earlier launches of the same call
gspn_status run(const gspn::Problem& pr, Plan plan, void* ws, hipStream_t stream,
                gspn::Tracer* cont = nullptr) {
  hipError_t e = hipSuccess;
  gspn::Tracer local;
  gspn::Tracer& tr = cont ? *cont : local;
  if (!cont) {
    tr.events = g_trace_events;
    tr.pairs = g_trace_pairs;
  }
  switch (plan) {
    case Plan::kPlane16:
    case Plan::kPlane64:
      e = gspn::launch_plane(pr, stream, &tr);
      break;
    case Plan::kBand:
      e = gspn::launch_band(pr, stream, &tr);
      break;
    case Plan::kTpipe:
      // the pipeline moves adjacent column pairs as one access; tensors that
      // start at an odd element take the streaming path, whose fp32
      // accumulator fits in the front of the pipeline's larger workspace
      e = pr.aligned_pair ? gspn::launch_tpipe(pr, ws, stream, &tr)
                          : gspn::launch_stream(pr, static_cast<float*>(ws), stream, &tr);
      break;
    case Plan::kTpipeT:
      e = pr.aligned_pair ? run_tpipe_t(pr, ws, stream, &tr)
                          : gspn::launch_stream(pr, static_cast<float*>(ws), stream, &tr);
      break;
    case Plan::kLarge:
      // the transposed-copy passes take one set of logits per plane
      e = pr.Cl == pr.C ? gspn::launch_dirs(pr, ws, stream, &tr)
                        : gspn::launch_stream(pr, static_cast<float*>(ws), stream, &tr);
      break;
    case Plan::kStream:
      e = gspn::launch_stream(pr, static_cast<float*>(ws), stream, &tr);
      break;
    case Plan::kDirs:
      e = gspn::launch_dirs(pr, ws, stream, &tr);
      break;
    default:
      return fail(GSPN_E_SHAPE, "no plan");
  }
  if (g_trace_events) {
    g_trace_count = tr.count;
    for (int i = 0; i < gspn::kTraceMax; ++i) {
      g_trace_names[i] = tr.names[i];
      g_trace_planes[i] = tr.planes[i];
    }
  }
  if (e != hipSuccess) return fail(GSPN_E_HIP, hipGetErrorString(e));
  return GSPN_OK;
}

const char* plan_str(Plan p) {
  switch (p) {
    case Plan::kPlane16: return "plane16";
    case Plan::kPlane64: return "plane64";
    case Plan::kBand: return "band";
    case Plan::kTpipe: return "tpipe";
    case Plan::kTpipeT: return "tpipe_t";
    case Plan::kLarge: return "large";
    case Plan::kStream: return "stream";
    case Plan::kDirs: return "dirs";
    default: return "invalid";
  }
}

// ---- per-direction parameters -----------------------------------------------
// Shape limits of the per-direction path and its workspace (an fp32
// accumulator, and transposed copies for the horizontal directions).
Checked check_dirs_shape(int64_t B, int64_t C, int64_t H, int64_t W, uint32_t mask, int64_t G,
                         int dtype, int64_t dir_stride) {
  Checked r = check_shape(B, C, H, W, mask, G, dtype);
  if (r.status != GSPN_OK) return r;
  r.plan = Plan::kDirs;
  r.ws_bytes = 0;
  if (H > gspn::dirs_max_orth() || W > gspn::dirs_max_orth()) {
    r.status = fail(GSPN_E_SHAPE, "per-direction parameters: H and W must be <= 8192");
    return r;
  }
  const int64_t P = B * C * H * W;
  if (dir_stride < 0 || (dir_stride > 0 && dir_stride < P)) {
    r.status = fail(GSPN_E_SHAPE, "dir_stride must be 0 or at least B * C * H * W");
    return r;
  }
  if (dir_stride > (INT64_MAX / 8 - P) / 3) {
    r.status = fail(GSPN_E_SHAPE, "dir_stride too large");
    return r;
  }
  r.ws_bytes = gspn::dirs_workspace_bytes(B * C, H, W, mask, static_cast<gspn_dtype>(dtype));
  return r;
}

// ---- module prologue --------------------------------------------------------
gspn_status check_prologue(const void* x_in, int64_t Cin, const void* w_r, const void* b_r,
                           const void* w_p, const void* b_p, int64_t B, int64_t C, int64_t H,
                           int64_t W, gspn_dtype dtype, void* x_out, void* const p_out[5],
                           gspn::PrologueProblem* pr) {
  if (!x_in || !w_r || !w_p || !x_out || !p_out)
    return fail(GSPN_E_NULL, "x_in, w_reduce, w_params, x_out and params_out must be non-null");
  for (int t = 0; t < 5; ++t)
    if (!p_out[t]) return fail(GSPN_E_NULL, "params_out[0..4] must be non-null");
  if (dtype != GSPN_F32 && dtype != GSPN_BF16)
    return fail(GSPN_E_DTYPE, "dtype must be GSPN_F32 or GSPN_BF16");
  if (B < 0 || Cin < 1 || C < 1 || H < 1 || W < 1)
    return fail(GSPN_E_SHAPE, "need B >= 0, Cin >= 1, C >= 1, H >= 1, W >= 1");
  const int64_t k31 = int64_t(1) << 31;
  if (B > 65535 || H >= k31 || W >= k31 || H * W >= k31 || Cin >= k31 || C >= k31 / 5)
    return fail(GSPN_E_SHAPE, "prologue limits: B <= 65535, H * W < 2^31, 5C < 2^31");
  if (B > 0 && (C * H * W > INT64_MAX / 16 / B || Cin * H * W > INT64_MAX / 16 / B))
    return fail(GSPN_E_SHAPE, "tensor size overflows");
  const size_t es = elem_size(dtype);
  const void* ins[5] = {x_in, w_r, b_r, w_p, b_p};
  const size_t in_n[5] = {static_cast<size_t>(B * Cin * H * W), static_cast<size_t>(C * Cin),
                          static_cast<size_t>(C), static_cast<size_t>(5 * C * C),
                          static_cast<size_t>(5 * C)};
  const void* outs[6] = {x_out, p_out[0], p_out[1], p_out[2], p_out[3], p_out[4]};
  for (const void* p : ins)
    if (reinterpret_cast<uintptr_t>(p) % es)
      return fail(GSPN_E_ALIGN, "input pointer not aligned to its element size");
  for (const void* p : outs)
    if (reinterpret_cast<uintptr_t>(p) % es)
      return fail(GSPN_E_ALIGN, "output pointer not aligned to its element size");
  const size_t ob = static_cast<size_t>(B * C * H * W) * es;
  for (int i = 0; i < 6; ++i) {
    for (int k = 0; k < 5; ++k)
      if (ins[k] && overlaps(outs[i], ob, ins[k], in_n[k] * es))
        return fail(GSPN_E_ALIAS, "a prologue output overlaps an input");
    for (int j = i + 1; j < 6; ++j)
      if (overlaps(outs[i], ob, outs[j], ob))
        return fail(GSPN_E_ALIAS, "two prologue outputs overlap");
  }
  pr->x_in = x_in;
  pr->w_r = w_r;
  pr->b_r = b_r;
  pr->w_p = w_p;
  pr->b_p = b_p;
  pr->x_out = x_out;
  for (int t = 0; t < 5; ++t) pr->p_out[t] = p_out[t];
  pr->B = B; pr->Cin = Cin; pr->C = C; pr->H = H; pr->W = W;
  pr->dtype = dtype;
  return GSPN_OK;
}

gspn_status run_prologue(const gspn::PrologueProblem& pr, hipStream_t stream,
                         gspn::Tracer* tr) {
  const hipError_t e = gspn::launch_prologue(pr, stream, tr);
  if (e != hipSuccess) return fail(GSPN_E_HIP, hipGetErrorString(e));
  return GSPN_OK;
}

void keep_trace(const gspn::Tracer& tr) {
  if (!g_trace_events) return;
  g_trace_count = tr.count;
  for (int i = 0; i < gspn::kTraceMax; ++i) {
    g_trace_names[i] = tr.names[i];
    g_trace_planes[i] = tr.planes[i];
  }
}

// ---- backward pass ---------------------------------------------------------
enum class BPlan { kInvalid, kPlane16, kPlane64, kBand, kTpipe, kTpipeT, kStream };
struct BChecked;
BChecked check_bwd_plan(int64_t B, int64_t C, int64_t H, int64_t W, uint32_t mask, int64_t G,
                        int dtype);

struct BChecked {
  gspn_status status;
  BPlan plan;
  size_t ws_bytes;     // total workspace
  size_t plan_bytes;   // the plan's part; shared logits add their fp32
                       // per-plane gradients after it (256-byte aligned)
};

size_t al256(size_t v) { return (v + 255) & ~size_t(255); }

// the backward pipeline on transposed planes (as run_tpipe_t for the forward
// pass): the seven inputs and six gradients transposed, then the pipeline's
// own workspace for the transposed shape and mask
uint32_t swap_axes(uint32_t mask) { return ((mask & 3u) << 2) | ((mask >> 2) & 3u); }
size_t bwd_tpipe_t_workspace_bytes(int64_t planes, int64_t H, int64_t W, uint32_t mask,
                                   gspn_dtype dt) {
  const size_t t = al256(static_cast<size_t>(planes * H * W) * (dt == GSPN_F32 ? 4 : 2));
  return 13 * t + gspn::bwd_tpipe_workspace_bytes(planes, W, H, swap_axes(mask), dt);
}

template <typename T>
hipError_t run_bwd_tpipe_t_dt(const gspn::BwdProblem& pr, void* ws, hipStream_t stream,
                              gspn::Tracer* tr) {
  const int64_t planes = pr.B * pr.C;
  const int H = static_cast<int>(pr.H), W = static_cast<int>(pr.W);
  const size_t t = al256(static_cast<size_t>(planes * H * W) * sizeof(T));
  char* w = static_cast<char*>(ws);
  auto buf = [&](int i) { return reinterpret_cast<T*>(w + i * t); };
  // inputs: x, lambda, u, grad_out, l0, l1, l2; gradients: x, l0, l1, l2, lambda, u
  const T* si[7] = {static_cast<const T*>(pr.x), static_cast<const T*>(pr.lam),
                    static_cast<const T*>(pr.u), static_cast<const T*>(pr.gy),
                    static_cast<const T*>(pr.l[0]), static_cast<const T*>(pr.l[1]),
                    static_cast<const T*>(pr.l[2])};
  T* di[7] = {buf(0), buf(1), buf(2), buf(3), buf(4), buf(5), buf(6)};
  hipError_t e = gspn::transpose_planes<T>(si, di, 7, planes, H, W, "btp_t_in", stream, tr);
  if (e != hipSuccess) return e;
  gspn::BwdProblem pt = pr;
  pt.x = di[0];
  pt.lam = di[1];
  pt.u = di[2];
  pt.gy = di[3];
  for (int k = 0; k < 3; ++k) pt.l[k] = di[4 + k];
  T* go[6] = {buf(7), buf(8), buf(9), buf(10), buf(11), buf(12)};
  pt.dx = go[0];
  for (int k = 0; k < 3; ++k) pt.dl[k] = go[1 + k];
  pt.dlam = go[4];
  pt.du = go[5];
  pt.H = pr.W;
  pt.W = pr.H;
  pt.mask = swap_axes(pr.mask);
  pt.aligned_vec4 = false;
  pt.aligned_pair = true;
  pt.dlw = nullptr;
  if ((e = gspn::launch_bwd_tpipe(pt, w + 13 * t, stream, tr)) != hipSuccess) return e;
  const T* so[6] = {go[0], go[1], go[2], go[3], go[4], go[5]};
  T* dd[6] = {static_cast<T*>(pr.dx), static_cast<T*>(pr.dl[0]), static_cast<T*>(pr.dl[1]),
              static_cast<T*>(pr.dl[2]), static_cast<T*>(pr.dlam), static_cast<T*>(pr.du)};
  return gspn::transpose_planes<T>(so, dd, 6, planes, W, H, "btp_t_out", stream, tr);
}

BChecked check_bwd_shape(int64_t B, int64_t C, int64_t H, int64_t W, uint32_t mask, int64_t G,
                         int dtype, int64_t Cl) {
  BChecked r = check_bwd_plan(B, C, H, W, mask, G, dtype);
  if (r.status != GSPN_OK) return r;
  if (r.plan == BPlan::kTpipeT && Cl < C) {
    // the transposed pipeline takes unshared logits only
    r.plan = BPlan::kStream;
    r.ws_bytes = gspn::bwd_stream_workspace_bytes(B * C, H, W, mask, static_cast<gspn_dtype>(dtype));
  }
  if (check_logit_channels(C, Cl) != GSPN_OK) {
    r.status = GSPN_E_SHAPE;
    return r;
  }
  r.plan_bytes = r.ws_bytes;
  if (Cl < C) r.ws_bytes = al256(r.plan_bytes) + static_cast<size_t>(3 * B * C * H * W) * sizeof(float);
  return r;
}
BChecked check_bwd_plan(int64_t B, int64_t C, int64_t H, int64_t W, uint32_t mask, int64_t G,
                        int dtype) {
  BChecked r{GSPN_OK, BPlan::kInvalid, 0, 0};
  const Checked f = check_shape(B, C, H, W, mask, G, dtype);
  if (f.status != GSPN_OK) {
    r.status = f.status;
    return r;
  }
  // GSPN_FORCE_BWD_PLAN=plane|band|tpipe|tpipe_t|stream picks a path for
  // testing when the shape allows it; otherwise the first path that fits, in
  // that order
  const char* force = std::getenv("GSPN_FORCE_BWD_PLAN");
  const bool f_plane = force && !std::strcmp(force, "plane");
  const bool f_band = force && !std::strcmp(force, "band");
  const bool f_tpipe = force && !std::strcmp(force, "tpipe");
  const bool f_tpipe_t = force && !std::strcmp(force, "tpipe_t");
  const bool f_stream = force && !std::strcmp(force, "stream");
  const bool any = !f_plane && !f_band && !f_tpipe && !f_tpipe_t && !f_stream;
  if ((any || f_plane) && gspn::plane_fits(H, W)) {
    r.plan = gspn::plane_seg(H, W) == 16 ? BPlan::kPlane16 : BPlan::kPlane64;
    return r;
  }
  if ((any || f_band) && gspn::bband_fits(H, W, G)) {
    r.plan = BPlan::kBand;
    r.ws_bytes = gspn::bband_workspace_bytes(B * C, H, W, mask);
    return r;
  }
  if ((any || f_tpipe) && gspn::btpipe_fits(H, W)) {
    r.plan = BPlan::kTpipe;
    r.ws_bytes = gspn::bwd_tpipe_workspace_bytes(B * C, H, W, mask, static_cast<gspn_dtype>(dtype));
    return r;
  }
  if ((any || f_tpipe_t) && gspn::btpipe_fits(W, H)) {
    // planes wider than the pipeline's row sweeps take, whose transpose it
    // takes: the pipeline on transposed copies
    r.plan = BPlan::kTpipeT;
    r.ws_bytes = bwd_tpipe_t_workspace_bytes(B * C, H, W, mask, static_cast<gspn_dtype>(dtype));
    return r;
  }
  if (f_plane && gspn::plane_fits(H, W)) {
    r.plan = gspn::plane_seg(H, W) == 16 ? BPlan::kPlane16 : BPlan::kPlane64;
    return r;
  }
  r.plan = BPlan::kStream;
  r.ws_bytes = gspn::bwd_stream_workspace_bytes(B * C, H, W, mask, static_cast<gspn_dtype>(dtype));
  return r;
}

const char* bplan_str(BPlan p) {
  switch (p) {
    case BPlan::kPlane16: return "bwd_plane16";
    case BPlan::kPlane64: return "bwd_plane64";
    case BPlan::kBand: return "bwd_band";
    case BPlan::kTpipe: return "bwd_tpipe";
    case BPlan::kTpipeT: return "bwd_tpipe_t";
    case BPlan::kStream: return "bwd_stream";
    default: return "invalid";
  }
}

gspn_status check_all_bwd(const void* x, const void* const w_logits[3], const void* lambda,
                          const void* u, const void* gy, int64_t B, int64_t C, int64_t H,
                          int64_t W, uint32_t mask, int64_t G, gspn_dtype dtype, void* dx,
                          void* const dlogits[3], void* dlam, void* du, BChecked* chk,
                          gspn::BwdProblem* pr, int64_t Cl) {
  if (!x || !w_logits || !lambda || !u || !gy || !dx || !dlogits || !dlam || !du)
    return fail(GSPN_E_NULL, "inputs, grad_out and the gradient outputs must be non-null");
  if (!w_logits[0] || !w_logits[1] || !w_logits[2] || !dlogits[0] || !dlogits[1] || !dlogits[2])
    return fail(GSPN_E_NULL, "w_logits[0..2] and grad_logits[0..2] must be non-null");
  *chk = check_bwd_shape(B, C, H, W, mask, G, static_cast<int>(dtype), Cl);
  if (chk->status != GSPN_OK) {
    if (chk->status == GSPN_E_SHAPE && g_last_error.empty())
      fail(GSPN_E_SHAPE, "logit_channels must be >= 1 and divide C");
    return chk->status;
  }
  const size_t es = elem_size(dtype);
  const void* ins[7] = {x, w_logits[0], w_logits[1], w_logits[2], lambda, u, gy};
  const void* outs[6] = {dx, dlogits[0], dlogits[1], dlogits[2], dlam, du};
  bool vec4 = true, pair = true;
  for (const void* p : ins) {
    if (reinterpret_cast<uintptr_t>(p) % es)
      return fail(GSPN_E_ALIGN, "input pointer not aligned to its element size");
    if (reinterpret_cast<uintptr_t>(p) % (4 * es)) vec4 = false;
    if (reinterpret_cast<uintptr_t>(p) % (2 * es)) pair = false;
  }
  for (const void* p : outs) {
    if (reinterpret_cast<uintptr_t>(p) % es)
      return fail(GSPN_E_ALIGN, "gradient pointer not aligned to its element size");
    if (reinterpret_cast<uintptr_t>(p) % (4 * es)) vec4 = false;
    if (reinterpret_cast<uintptr_t>(p) % (2 * es)) pair = false;
  }
  // the three logits and their gradients have Cl channels, the rest C
  const size_t bytes = static_cast<size_t>(B * C * H * W) * es;
  const size_t lbytes = static_cast<size_t>(B * Cl * H * W) * es;
  auto in_bytes = [&](int i) { return i >= 1 && i <= 3 ? lbytes : bytes; };
  for (int i = 0; i < 6; ++i) {
    const size_t ob = in_bytes(i);   // outs[] has the same order for indices 0..3
    for (int k = 0; k < 7; ++k)
      if (overlaps(outs[i], ob, ins[k], in_bytes(k)))
        return fail(GSPN_E_ALIAS, "a gradient overlaps an input");
    for (int j = i + 1; j < 6; ++j)
      if (overlaps(outs[i], ob, outs[j], in_bytes(j)))
        return fail(GSPN_E_ALIAS, "two gradient outputs overlap");
  }
  pr->x = x;
  for (int k = 0; k < 3; ++k) {
    pr->l[k] = w_logits[k];
    pr->dl[k] = dlogits[k];
  }
  pr->lam = lambda;
  pr->u = u;
  pr->gy = gy;
  pr->dx = dx;
  pr->dlam = dlam;
  pr->du = du;
  pr->B = B; pr->C = C; pr->H = H; pr->W = W;
  pr->mask = mask;
  pr->G = G;
  pr->dtype = dtype;
  pr->aligned_vec4 = vec4;
  pr->aligned_pair = pair;
  pr->Cl = Cl;
  pr->dlw = nullptr;
  return GSPN_OK;
}

gspn_status run_bwd(gspn::BwdProblem pr, const BChecked& chk, void* ws, hipStream_t stream) {
  hipError_t e = hipSuccess;
  gspn::Tracer tr;
  tr.events = g_trace_events;
  tr.pairs = g_trace_pairs;
  if (pr.Cl < pr.C) pr.dlw = reinterpret_cast<float*>(static_cast<char*>(ws) + al256(chk.plan_bytes));
  switch (chk.plan) {
    case BPlan::kPlane16:
    case BPlan::kPlane64:
      e = gspn::launch_bplane(pr, stream, &tr);
      break;
    case BPlan::kBand:
      e = gspn::launch_bband(pr, ws, stream, &tr);
      break;
    case BPlan::kTpipe:
      // the pipeline moves element pairs; tensors at odd element offsets
      // take the streaming path, whose workspace fits in the pipeline's
      e = pr.aligned_pair ? gspn::launch_bwd_tpipe(pr, ws, stream, &tr)
                          : gspn::launch_bwd_stream(pr, ws, stream, &tr);
      break;
    case BPlan::kTpipeT:
      // the transposes take any alignment; the pipeline then works on
      // aligned workspace copies
      e = pr.dtype == GSPN_F32 ? run_bwd_tpipe_t_dt<float>(pr, ws, stream, &tr)
                               : run_bwd_tpipe_t_dt<gspn::bf16_t>(pr, ws, stream, &tr);
      break;
    case BPlan::kStream:
      e = gspn::launch_bwd_stream(pr, ws, stream, &tr);
      break;
    default:
      return fail(GSPN_E_SHAPE, "no backward plan");
  }
  if (e == hipSuccess && pr.dlw) e = gspn::launch_bwd_reduce_logits(pr, stream, &tr);
  if (g_trace_events) {
    g_trace_count = tr.count;
    for (int i = 0; i < gspn::kTraceMax; ++i) {
      g_trace_names[i] = tr.names[i];
      g_trace_planes[i] = tr.planes[i];
    }
  }
  if (e != hipSuccess) return fail(GSPN_E_HIP, hipGetErrorString(e));
  return GSPN_OK;
}

}  // namespace

extern "C" {

gspn_status gspn_propagate(const void* x, const void* const w_logits[3], const void* lambda,
                           const void* u, int64_t B, int64_t C, int64_t H, int64_t W,
                           uint32_t dir_mask, int64_t group_rows, gspn_dtype dtype,
                           void* out, hipStream_t stream) {
  Checked chk;
  gspn::Problem pr;
  gspn_status s = check_all(x, w_logits, lambda, u, B, C, H, W, dir_mask, group_rows,
                            dtype, out, &chk, &pr, C > 0 ? C : 1);
  if (s != GSPN_OK) return s;
  if (B * C == 0) return GSPN_OK;
  void* ws = nullptr;
  if (chk.ws_bytes > 0) {
    hipError_t e = hipMallocAsync(&ws, chk.ws_bytes, stream);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return fail(GSPN_E_NOMEM, hipGetErrorString(e));
    }
  }
  s = run(pr, chk.plan, ws, stream);
  if (ws) {
    hipError_t e = hipFreeAsync(ws, stream);
    if (e != hipSuccess && s == GSPN_OK) s = fail(GSPN_E_HIP, hipGetErrorString(e));
  }
  return s;
}

size_t gspn_noalloc_scratch_bytes(void) { return kNoallocScratchBytes; }

gspn_status gspn_propagate_noalloc(const void* x, const void* const w_logits[3],
                                   const void* lambda, const void* u, int64_t B, int64_t C,
                                   int64_t H, int64_t W, uint32_t dir_mask, int64_t group_rows,
                                   gspn_dtype dtype, void* out, hipStream_t stream) {
  Checked chk;
  gspn::Problem pr;
  gspn_status s = check_all(x, w_logits, lambda, u, B, C, H, W, dir_mask, group_rows,
                            dtype, out, &chk, &pr, C > 0 ? C : 1);
  if (s != GSPN_OK) return s;
  if (chk.ws_bytes > kNoallocScratchBytes)
    return fail(GSPN_E_WORKSPACE,
                "this problem needs " + std::to_string(chk.ws_bytes) +
                    " bytes of scratch; gspn_propagate_noalloc holds " +
                    std::to_string(kNoallocScratchBytes) + " (use gspn_propagate_ws)");
  if (B * C == 0) return GSPN_OK;
  void* ws = nullptr;
  if (chk.ws_bytes > 0) {
    // the device the work runs on is the stream's; look its scratch up with
    // that device current
    int cur = 0, dev = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e == hipSuccess) {
      dev = cur;
      if (stream) e = hipStreamGetDevice(stream, &dev);
    }
    if (e != hipSuccess) return fail(GSPN_E_HIP, hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(GSPN_E_HIP, "device index out of range");
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
      if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess)
        return fail(GSPN_E_HIP, hipGetErrorString(e));
      void* p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (dev != cur) (void)hipSetDevice(cur);
      if (e != hipSuccess || !p)
        return fail(GSPN_E_HIP, std::string("hipGetSymbolAddress(scratch): ") +
                                    hipGetErrorString(e));
      g_scratch_ptr[dev] = p;
    }
    ws = g_scratch_ptr[dev];
  }
  pr.one_stream = true;
  return run(pr, chk.plan, ws, stream);
}

size_t gspn_workspace_bytes(int64_t B, int64_t C, int64_t H, int64_t W, uint32_t dir_mask,
                            int64_t group_rows, gspn_dtype dtype) {
  const std::string keep = g_last_error;
  Checked chk = check_shape(B, C, H, W, dir_mask, group_rows, static_cast<int>(dtype));
  g_last_error = keep;
  return chk.status == GSPN_OK ? chk.ws_bytes : 0;
}

gspn_status gspn_propagate_ws(const void* x, const void* const w_logits[3], const void* lambda,
                              const void* u, int64_t B, int64_t C, int64_t H, int64_t W,
                              uint32_t dir_mask, int64_t group_rows, gspn_dtype dtype,
                              void* out, void* workspace, size_t ws_bytes,
                              hipStream_t stream) {
  return gspn_propagate_shared_ws(x, w_logits, C > 0 ? C : 1, lambda, u, B, C, H, W, dir_mask,
                                  group_rows, dtype, out, workspace, ws_bytes, stream);
}

const char* gspn_plan_name(int64_t B, int64_t C, int64_t H, int64_t W, uint32_t dir_mask,
                           int64_t group_rows, gspn_dtype dtype) {
  const std::string keep = g_last_error;
  Checked chk = check_shape(B, C, H, W, dir_mask, group_rows, static_cast<int>(dtype));
  g_last_error = keep;
  return chk.status == GSPN_OK ? plan_str(chk.plan) : "invalid";
}

void gspn_trace_events(hipEvent_t* events, int n_pairs) {
  // the record of the last traced call stays readable after tracing stops
  g_trace_events = n_pairs > 0 ? events : nullptr;
  g_trace_pairs = n_pairs > 0 ? n_pairs : 0;
}

int gspn_trace_count(void) { return g_trace_count; }

const char* gspn_trace_kernel(int i, int64_t* planes) {
  if (i < 0 || i >= g_trace_count || i >= gspn::kTraceMax || !g_trace_names[i]) return nullptr;
  if (planes) *planes = g_trace_planes[i];
  return g_trace_names[i];
}

const char* gspn_status_str(gspn_status s) {
  switch (s) {
    case GSPN_OK: return "GSPN_OK";
    case GSPN_E_NULL: return "GSPN_E_NULL: null pointer";
    case GSPN_E_SHAPE: return "GSPN_E_SHAPE: bad or unsupported shape";
    case GSPN_E_DIRMASK: return "GSPN_E_DIRMASK: bad direction mask";
    case GSPN_E_GROUP: return "GSPN_E_GROUP: negative group_rows";
    case GSPN_E_DTYPE: return "GSPN_E_DTYPE: bad dtype";
    case GSPN_E_ALIGN: return "GSPN_E_ALIGN: misaligned pointer";
    case GSPN_E_ALIAS: return "GSPN_E_ALIAS: output overlaps an input";
    case GSPN_E_NOMEM: return "GSPN_E_NOMEM: workspace allocation failed";
    case GSPN_E_HIP: return "GSPN_E_HIP: HIP error";
    case GSPN_E_WORKSPACE: return "GSPN_E_WORKSPACE: workspace too small";
  }
  return "unknown gspn_status";
}

const char* gspn_last_error(void) { return g_last_error.c_str(); }

int gspn_abi_version(void) { return 1; }

gspn_status gspn_propagate_backward(const void* x, const void* const w_logits[3],
                                    const void* lambda, const void* u, const void* grad_out,
                                    int64_t B, int64_t C, int64_t H, int64_t W,
                                    uint32_t dir_mask, int64_t group_rows, gspn_dtype dtype,
                                    void* grad_x, void* const grad_logits[3], void* grad_lambda,
                                    void* grad_u, hipStream_t stream) {
  BChecked chk;
  gspn::BwdProblem pr;
  gspn_status s = check_all_bwd(x, w_logits, lambda, u, grad_out, B, C, H, W, dir_mask,
                                group_rows, dtype, grad_x, grad_logits, grad_lambda, grad_u,
                                &chk, &pr, C > 0 ? C : 1);
  if (s != GSPN_OK) return s;
  if (B * C == 0) return GSPN_OK;
  void* ws = nullptr;
  if (chk.ws_bytes > 0) {
    hipError_t e = hipMallocAsync(&ws, chk.ws_bytes, stream);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return fail(GSPN_E_NOMEM, hipGetErrorString(e));
    }
  }
  s = run_bwd(pr, chk, ws, stream);
  if (ws) {
    hipError_t e = hipFreeAsync(ws, stream);
    if (e != hipSuccess && s == GSPN_OK) s = fail(GSPN_E_HIP, hipGetErrorString(e));
  }
  return s;
}

size_t gspn_backward_workspace_bytes(int64_t B, int64_t C, int64_t H, int64_t W,
                                     uint32_t dir_mask, int64_t group_rows, gspn_dtype dtype) {
  return gspn_backward_workspace_bytes_shared(B, C, H, W, C > 0 ? C : 1, dir_mask, group_rows,
                                              dtype);
}

size_t gspn_backward_workspace_bytes_shared(int64_t B, int64_t C, int64_t H, int64_t W,
                                            int64_t logit_channels, uint32_t dir_mask,
                                            int64_t group_rows, gspn_dtype dtype) {
  const std::string keep = g_last_error;
  BChecked chk = check_bwd_shape(B, C, H, W, dir_mask, group_rows, static_cast<int>(dtype),
                                 logit_channels);
  g_last_error = keep;
  return chk.status == GSPN_OK ? chk.ws_bytes : 0;
}

namespace {
gspn_status backward_ws(const void* x, const void* const w_logits[3], int64_t Cl,
                        const void* lambda, const void* u, const void* grad_out, int64_t B,
                        int64_t C, int64_t H, int64_t W, uint32_t dir_mask, int64_t group_rows,
                        gspn_dtype dtype, void* grad_x, void* const grad_logits[3],
                        void* grad_lambda, void* grad_u, void* workspace, size_t ws_bytes,
                        hipStream_t stream) {
  BChecked chk;
  gspn::BwdProblem pr;
  gspn_status s = check_all_bwd(x, w_logits, lambda, u, grad_out, B, C, H, W, dir_mask,
                                group_rows, dtype, grad_x, grad_logits, grad_lambda, grad_u,
                                &chk, &pr, Cl);
  if (s != GSPN_OK) return s;
  if (chk.ws_bytes > 0) {
    if (!workspace || ws_bytes < chk.ws_bytes)
      return fail(GSPN_E_WORKSPACE,
                  "workspace missing or smaller than gspn_backward_workspace_bytes()");
    if (reinterpret_cast<uintptr_t>(workspace) % 256)
      return fail(GSPN_E_ALIGN, "workspace must be 256-byte aligned");
    const size_t es = elem_size(dtype);
    const size_t bytes = static_cast<size_t>(B * C * H * W) * es;
    const size_t lbytes = static_cast<size_t>(B * Cl * H * W) * es;
    const void* all[13] = {x, lambda, u, grad_out, grad_x, grad_lambda, grad_u,
                           w_logits[0], w_logits[1], w_logits[2],
                           grad_logits[0], grad_logits[1], grad_logits[2]};
    for (int i = 0; i < 13; ++i)
      if (overlaps(workspace, chk.ws_bytes, all[i], i < 7 ? bytes : lbytes))
        return fail(GSPN_E_ALIAS, "workspace overlaps a tensor");
  }
  if (B * C == 0) return GSPN_OK;
  return run_bwd(pr, chk, workspace, stream);
}
}  // namespace

gspn_status gspn_propagate_backward_ws(const void* x, const void* const w_logits[3],
                                       const void* lambda, const void* u, const void* grad_out,
                                       int64_t B, int64_t C, int64_t H, int64_t W,
                                       uint32_t dir_mask, int64_t group_rows, gspn_dtype dtype,
                                       void* grad_x, void* const grad_logits[3],
                                       void* grad_lambda, void* grad_u, void* workspace,
                                       size_t ws_bytes, hipStream_t stream) {
  return backward_ws(x, w_logits, C > 0 ? C : 1, lambda, u, grad_out, B, C, H, W, dir_mask, group_rows,
                     dtype, grad_x, grad_logits, grad_lambda, grad_u, workspace, ws_bytes,
                     stream);
}

gspn_status gspn_propagate_backward_shared_ws(
    const void* x, const void* const w_logits[3], int64_t logit_channels, const void* lambda,
    const void* u, const void* grad_out, int64_t B, int64_t C, int64_t H, int64_t W,
    uint32_t dir_mask, int64_t group_rows, gspn_dtype dtype, void* grad_x,
    void* const grad_logits[3], void* grad_lambda, void* grad_u, void* workspace,
    size_t ws_bytes, hipStream_t stream) {
  return backward_ws(x, w_logits, logit_channels, lambda, u, grad_out, B, C, H, W, dir_mask,
                     group_rows, dtype, grad_x, grad_logits, grad_lambda, grad_u, workspace,
                     ws_bytes, stream);
}

const char* gspn_backward_plan_name(int64_t B, int64_t C, int64_t H, int64_t W,
                                    uint32_t dir_mask, int64_t group_rows, gspn_dtype dtype) {
  const std::string keep = g_last_error;
  BChecked chk = check_bwd_shape(B, C, H, W, dir_mask, group_rows, static_cast<int>(dtype),
                                 C > 0 ? C : 1);
  g_last_error = keep;
  return chk.status == GSPN_OK ? bplan_str(chk.plan) : "invalid";
}

gspn_status gspn_propagate_shared_ws(const void* x, const void* const w_logits[3],
                                     int64_t logit_channels, const void* lambda, const void* u,
                                     int64_t B, int64_t C, int64_t H, int64_t W,
                                     uint32_t dir_mask, int64_t group_rows, gspn_dtype dtype,
                                     void* out, void* workspace, size_t ws_bytes,
                                     hipStream_t stream) {
  Checked chk;
  gspn::Problem pr;
  gspn_status s = check_all(x, w_logits, lambda, u, B, C, H, W, dir_mask, group_rows,
                            dtype, out, &chk, &pr, logit_channels);
  if (s != GSPN_OK) return s;
  if (chk.ws_bytes > 0) {
    if (!workspace || ws_bytes < chk.ws_bytes)
      return fail(GSPN_E_WORKSPACE, "workspace missing or smaller than gspn_workspace_bytes()");
    if (reinterpret_cast<uintptr_t>(workspace) % 256)
      return fail(GSPN_E_ALIGN, "workspace must be 256-byte aligned");
    const size_t es = elem_size(dtype);
    const size_t bytes = static_cast<size_t>(B * C * H * W) * es;
    const size_t lbytes = static_cast<size_t>(B * logit_channels * H * W) * es;
    const void* all[7] = {x, lambda, u, out, w_logits[0], w_logits[1], w_logits[2]};
    for (int i = 0; i < 7; ++i)
      if (overlaps(workspace, chk.ws_bytes, all[i], i < 4 ? bytes : lbytes))
        return fail(GSPN_E_ALIAS, "workspace overlaps a tensor");
  }
  if (B * C == 0) return GSPN_OK;
  return run(pr, chk.plan, workspace, stream);
}

gspn_status gspn_prologue(const void* x_in, int64_t Cin, const void* w_reduce,
                          const void* b_reduce, const void* w_params, const void* b_params,
                          int64_t B, int64_t C, int64_t H, int64_t W, gspn_dtype dtype,
                          void* x_out, void* const params_out[5], hipStream_t stream) {
  g_last_error.clear();
  gspn::PrologueProblem pr;
  gspn_status s = check_prologue(x_in, Cin, w_reduce, b_reduce, w_params, b_params, B, C, H, W,
                                 dtype, x_out, params_out, &pr);
  if (s != GSPN_OK || B == 0) return s;
  gspn::Tracer tr;
  tr.events = g_trace_events;
  tr.pairs = g_trace_pairs;
  s = run_prologue(pr, stream, &tr);
  keep_trace(tr);
  return s;
}

size_t gspn_module_workspace_bytes(int64_t B, int64_t C, int64_t H, int64_t W, uint32_t dir_mask,
                                   int64_t group_rows, gspn_dtype dtype) {
  const std::string keep = g_last_error;
  const Checked chk = check_shape(B, C, H, W, dir_mask, group_rows, static_cast<int>(dtype));
  g_last_error = keep;
  if (chk.status != GSPN_OK || C < 1) return 0;
  return 6 * al256(static_cast<size_t>(B * C * H * W) * elem_size(dtype)) + chk.ws_bytes;
}

gspn_status gspn_module_ws(const void* x_in, int64_t Cin, const void* w_reduce,
                           const void* b_reduce, const void* w_params, const void* b_params,
                           int64_t B, int64_t C, int64_t H, int64_t W, uint32_t dir_mask,
                           int64_t group_rows, gspn_dtype dtype, void* out, void* workspace,
                           size_t ws_bytes, hipStream_t stream) {
  g_last_error.clear();
  if (!out) return fail(GSPN_E_NULL, "out must be non-null");
  const Checked chk = check_shape(B, C, H, W, dir_mask, group_rows, static_cast<int>(dtype));
  if (chk.status != GSPN_OK) return chk.status;
  if (C < 1) return fail(GSPN_E_SHAPE, "need C >= 1");
  const size_t es = elem_size(dtype);
  const size_t tb = al256(static_cast<size_t>(B * C * H * W) * es);
  const size_t need = 6 * tb + chk.ws_bytes;
  if (!workspace || ws_bytes < need)
    return fail(GSPN_E_WORKSPACE, "workspace missing or smaller than gspn_module_workspace_bytes()");
  if (reinterpret_cast<uintptr_t>(workspace) % 256)
    return fail(GSPN_E_ALIGN, "workspace must be 256-byte aligned");
  char* ws = static_cast<char*>(workspace);
  void* params[5];
  for (int t = 0; t < 5; ++t) params[t] = ws + (1 + t) * tb;
  gspn::PrologueProblem pp;
  gspn_status s = check_prologue(x_in, Cin, w_reduce, b_reduce, w_params, b_params, B, C, H, W,
                                 dtype, ws, params, &pp);
  if (s != GSPN_OK) return s;
  // out against the inputs and the workspace
  const void* ins[5] = {x_in, w_reduce, b_reduce, w_params, b_params};
  const size_t in_n[5] = {static_cast<size_t>(B * Cin * H * W), static_cast<size_t>(C * Cin),
                          static_cast<size_t>(C), static_cast<size_t>(5 * C * C),
                          static_cast<size_t>(5 * C)};
  const size_t ob = static_cast<size_t>(B * C * H * W) * es;
  if (reinterpret_cast<uintptr_t>(out) % es)
    return fail(GSPN_E_ALIGN, "out not aligned to its element size");
  for (int k = 0; k < 5; ++k)
    if (ins[k] && overlaps(out, ob, ins[k], in_n[k] * es))
      return fail(GSPN_E_ALIAS, "out overlaps an input");
  if (overlaps(out, ob, workspace, need)) return fail(GSPN_E_ALIAS, "out overlaps the workspace");
  for (int k = 0; k < 5; ++k)
    if (ins[k] && overlaps(workspace, need, ins[k], in_n[k] * es))
      return fail(GSPN_E_ALIAS, "workspace overlaps an input");
  if (B == 0) return GSPN_OK;
  const void* logits[3] = {params[0], params[1], params[2]};
  Checked pchk;
  gspn::Problem pr;
  s = check_all(ws, logits, params[3], params[4], B, C, H, W, dir_mask, group_rows, dtype, out,
                &pchk, &pr, C);
  if (s != GSPN_OK) return s;
  gspn::Tracer tr;
  tr.events = g_trace_events;
  tr.pairs = g_trace_pairs;
  // small bf16 planes: the parameter product runs fused with the scan and
  // the parameter tensors are never stored (GSPN_FORCE_MODULE=unfused keeps
  // the two-step path, for comparisons)
  const char* force = std::getenv("GSPN_FORCE_MODULE");
  const bool unfused = force && !std::strcmp(force, "unfused");
  if (!unfused && gspn::fused_unit_fits(pp) && reinterpret_cast<uintptr_t>(out) % 16 == 0) {
    hipError_t e = gspn::launch_prologue_reduce(pp, stream, &tr);
    if (e == hipSuccess) e = gspn::launch_fused_unit(pp, ws, out, dir_mask, group_rows, stream, &tr);
    keep_trace(tr);
    return e == hipSuccess ? GSPN_OK : fail(GSPN_E_HIP, hipGetErrorString(e));
  }
  s = run_prologue(pp, stream, &tr);
  if (s != GSPN_OK) {
    keep_trace(tr);
    return s;
  }
  return run(pr, pchk.plan, ws + 6 * tb, stream, &tr);
}

size_t gspn_workspace_bytes_dirs(int64_t B, int64_t C, int64_t H, int64_t W, uint32_t dir_mask,
                                 int64_t group_rows, gspn_dtype dtype) {
  const std::string keep = g_last_error;
  Checked chk = check_dirs_shape(B, C, H, W, dir_mask, group_rows, static_cast<int>(dtype), 0);
  g_last_error = keep;
  return chk.status == GSPN_OK ? chk.ws_bytes : 0;
}

size_t gspn_backward_workspace_bytes_dirs(int64_t B, int64_t C, int64_t H, int64_t W,
                                          uint32_t dir_mask, int64_t group_rows,
                                          gspn_dtype dtype) {
  const std::string keep = g_last_error;
  const Checked chk = check_dirs_shape(B, C, H, W, dir_mask, group_rows, static_cast<int>(dtype), 0);
  g_last_error = keep;
  return chk.status == GSPN_OK
             ? gspn::bwd_dirs_workspace_bytes(B * C, H, W, dir_mask, dtype)
             : 0;
}

gspn_status gspn_propagate_backward_dirs_ws(
    const void* x, const void* const w_logits[3], const void* lambda, const void* u,
    int64_t dir_stride, const float* merge, const void* grad_out, int64_t B, int64_t C,
    int64_t H, int64_t W, uint32_t dir_mask, int64_t group_rows, gspn_dtype dtype, void* grad_x,
    void* const grad_logits[3], void* grad_lambda, void* grad_u, float* grad_merge,
    void* workspace, size_t ws_bytes, hipStream_t stream) {
  g_last_error.clear();
  if (!x || !w_logits || !lambda || !u || !grad_out || !grad_x || !grad_logits ||
      !grad_lambda || !grad_u)
    return fail(GSPN_E_NULL, "inputs, grad_out and the gradient outputs must be non-null");
  if (!w_logits[0] || !w_logits[1] || !w_logits[2] || !grad_logits[0] || !grad_logits[1] ||
      !grad_logits[2])
    return fail(GSPN_E_NULL, "w_logits[0..2] and grad_logits[0..2] must be non-null");
  const Checked chk = check_dirs_shape(B, C, H, W, dir_mask, group_rows, static_cast<int>(dtype),
                                       dir_stride);
  if (chk.status != GSPN_OK) return chk.status;
  const size_t es = elem_size(dtype);
  const void* ins[7] = {x, w_logits[0], w_logits[1], w_logits[2], lambda, u, grad_out};
  const void* outs[6] = {grad_x, grad_logits[0], grad_logits[1], grad_logits[2], grad_lambda,
                         grad_u};
  for (const void* p : ins)
    if (reinterpret_cast<uintptr_t>(p) % es)
      return fail(GSPN_E_ALIGN, "input pointer not aligned to its element size");
  for (const void* p : outs)
    if (reinterpret_cast<uintptr_t>(p) % es)
      return fail(GSPN_E_ALIGN, "gradient pointer not aligned to its element size");
  if (reinterpret_cast<uintptr_t>(merge) % sizeof(float) ||
      reinterpret_cast<uintptr_t>(grad_merge) % sizeof(float))
    return fail(GSPN_E_ALIGN, "merge and grad_merge must be aligned to 4 bytes");
  // byte ranges read: x, grad_out, each selected direction's five tensors,
  // the merge weights; written: grad_x, the four-slice gradients, grad_merge
  const size_t bytes = static_cast<size_t>(B * C * H * W) * es;
  const size_t mbytes = static_cast<size_t>(4 * C) * sizeof(float);
  const void* rd[23];
  size_t rn[23];
  int nr = 0;
  rd[nr] = x; rn[nr++] = bytes;
  rd[nr] = grad_out; rn[nr++] = bytes;
  if (merge) { rd[nr] = merge; rn[nr++] = mbytes; }
  for (int d = 0; d < 4; ++d) {
    if (!((dir_mask >> d) & 1u)) continue;
    const size_t off = static_cast<size_t>(d * dir_stride) * es;
    for (int k = 1; k < 6; ++k) {
      rd[nr] = static_cast<const char*>(ins[k]) + off;
      rn[nr++] = bytes;
    }
  }
  const void* wr[7] = {grad_x, grad_logits[0], grad_logits[1], grad_logits[2], grad_lambda,
                       grad_u, grad_merge};
  const size_t wn[7] = {bytes, 4 * bytes, 4 * bytes, 4 * bytes, 4 * bytes, 4 * bytes,
                        grad_merge ? mbytes : 0};
  for (int i = 0; i < 7; ++i) {
    for (int k = 0; k < nr; ++k)
      if (overlaps(wr[i], wn[i], rd[k], rn[k]))
        return fail(GSPN_E_ALIAS, "a gradient overlaps an input");
    for (int k = i + 1; k < 7; ++k)
      if (overlaps(wr[i], wn[i], wr[k], wn[k]))
        return fail(GSPN_E_ALIAS, "two gradient outputs overlap");
  }
  const size_t need = gspn::bwd_dirs_workspace_bytes(B * C, H, W, dir_mask, dtype);
  if (need > 0) {
    if (!workspace || ws_bytes < need)
      return fail(GSPN_E_WORKSPACE,
                  "workspace missing or smaller than gspn_backward_workspace_bytes_dirs()");
    if (reinterpret_cast<uintptr_t>(workspace) % 256)
      return fail(GSPN_E_ALIGN, "workspace must be 256-byte aligned");
    for (int k = 0; k < nr; ++k)
      if (overlaps(workspace, need, rd[k], rn[k]))
        return fail(GSPN_E_ALIAS, "workspace overlaps a tensor");
    for (int i = 0; i < 7; ++i)
      if (overlaps(workspace, need, wr[i], wn[i]))
        return fail(GSPN_E_ALIAS, "workspace overlaps a tensor");
  }
  gspn::BwdProblem pr;
  pr.x = x;
  for (int k = 0; k < 3; ++k) {
    pr.l[k] = w_logits[k];
    pr.dl[k] = grad_logits[k];
  }
  pr.lam = lambda;
  pr.u = u;
  pr.gy = grad_out;
  pr.dx = grad_x;
  pr.dlam = grad_lambda;
  pr.du = grad_u;
  pr.B = B; pr.C = C; pr.H = H; pr.W = W;
  pr.mask = dir_mask;
  pr.G = group_rows >= H && group_rows >= W ? 0 : group_rows;
  pr.dtype = dtype;
  pr.aligned_vec4 = false;
  pr.aligned_pair = false;
  pr.Cl = C;
  pr.dlw = nullptr;
  gspn::BwdDirsExtra ex{dir_stride, merge, grad_merge};
  gspn::Tracer tr;
  tr.events = g_trace_events;
  tr.pairs = g_trace_pairs;
  const hipError_t e = gspn::launch_bwd_dirs(pr, ex, workspace, stream, &tr);
  keep_trace(tr);
  if (e != hipSuccess) return fail(GSPN_E_HIP, hipGetErrorString(e));
  return GSPN_OK;
}

gspn_status gspn_propagate_dirs_ws(const void* x, const void* const w_logits[3],
                                   const void* lambda, const void* u, int64_t dir_stride,
                                   const float* merge, int64_t B, int64_t C, int64_t H,
                                   int64_t W, uint32_t dir_mask, int64_t group_rows,
                                   gspn_dtype dtype, void* out, void* workspace,
                                   size_t ws_bytes, hipStream_t stream) {
  g_last_error.clear();
  if (!x || !w_logits || !lambda || !u || !out)
    return fail(GSPN_E_NULL, "x, w_logits, lambda, u and out must be non-null");
  if (!w_logits[0] || !w_logits[1] || !w_logits[2])
    return fail(GSPN_E_NULL, "w_logits[0..2] must be non-null");
  const Checked chk = check_dirs_shape(B, C, H, W, dir_mask, group_rows, static_cast<int>(dtype),
                                       dir_stride);
  if (chk.status != GSPN_OK) return chk.status;
  const size_t es = elem_size(dtype);
  const void* ins[6] = {x, w_logits[0], w_logits[1], w_logits[2], lambda, u};
  for (const void* p : ins)
    if (reinterpret_cast<uintptr_t>(p) % es)
      return fail(GSPN_E_ALIGN, "input pointer not aligned to its element size");
  if (reinterpret_cast<uintptr_t>(out) % es)
    return fail(GSPN_E_ALIGN, "out not aligned to its element size");
  if (reinterpret_cast<uintptr_t>(merge) % sizeof(float))
    return fail(GSPN_E_ALIGN, "merge not aligned to 4 bytes");
  // every byte range the call reads: x, each selected direction's five
  // tensors, the merge weights
  const size_t bytes = static_cast<size_t>(B * C * H * W) * es;
  const size_t mbytes = merge ? static_cast<size_t>(4 * C) * sizeof(float) : 0;
  const void* rd[22];
  size_t rn[22];
  int nr = 0;
  rd[nr] = x; rn[nr++] = bytes;
  if (merge) { rd[nr] = merge; rn[nr++] = mbytes; }
  for (int d = 0; d < 4; ++d) {
    if (!((dir_mask >> d) & 1u)) continue;
    const size_t off = static_cast<size_t>(d * dir_stride) * es;
    for (int k = 1; k < 6; ++k) {
      rd[nr] = static_cast<const char*>(ins[k]) + off;
      rn[nr++] = bytes;
    }
  }
  for (int i = 0; i < nr; ++i)
    if (overlaps(out, bytes, rd[i], rn[i])) return fail(GSPN_E_ALIAS, "out overlaps an input");
  if (chk.ws_bytes > 0) {
    if (!workspace || ws_bytes < chk.ws_bytes)
      return fail(GSPN_E_WORKSPACE,
                  "workspace missing or smaller than gspn_workspace_bytes_dirs()");
    if (reinterpret_cast<uintptr_t>(workspace) % 256)
      return fail(GSPN_E_ALIGN, "workspace must be 256-byte aligned");
    if (overlaps(workspace, chk.ws_bytes, out, bytes))
      return fail(GSPN_E_ALIAS, "workspace overlaps a tensor");
    for (int i = 0; i < nr; ++i)
      if (overlaps(workspace, chk.ws_bytes, rd[i], rn[i]))
        return fail(GSPN_E_ALIAS, "workspace overlaps a tensor");
  }
  if (B * C == 0) return GSPN_OK;
  gspn::Problem pr;
  pr.x = x;
  for (int k = 0; k < 3; ++k) pr.l[k] = w_logits[k];
  pr.lam = lambda;
  pr.u = u;
  pr.out = out;
  pr.B = B; pr.C = C; pr.H = H; pr.W = W;
  pr.mask = dir_mask;
  pr.G = group_rows;
  pr.dtype = dtype;
  pr.aligned_vec4 = false;   // the per-direction kernels check alignment per pass
  pr.aligned_pair = false;
  pr.Cl = C;
  pr.dir_stride = dir_stride;
  pr.merge = merge;
  return run(pr, chk.plan, workspace, stream);
}

}  // extern "C"
