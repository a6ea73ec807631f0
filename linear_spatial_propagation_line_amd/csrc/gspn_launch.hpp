// Internal interface between the C ABI (gspn_api.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <functional>
#include <stdint.h>

#include "gspn.h"

namespace gspn {

// A validated problem: every pointer non-null and aligned, shapes positive.
struct Problem {
  const void* x;
  const void* l[3];
  const void* lam;
  const void* u;
  void* out;
  int64_t B, C, H, W;
  uint32_t mask;
  int64_t G;
  gspn_dtype dtype;
  bool aligned_vec4;   // every pointer aligned to 4 elements
  bool aligned_pair;   // every pointer aligned to 2 elements
  int64_t Cl;          // logit channels (Cl divides C; Cl == C: unshared)
  // per-direction parameters: direction d reads lambda, logits and u at
  // element offset d * dir_stride, merged with merge[d * C + c] (null: 1)
  int64_t dir_stride = 0;
  const float* merge = nullptr;
  // run every launch on the caller's stream (no helper streams or events)
  bool one_stream = false;
};

// A validated backward problem: the forward inputs, grad_out (gy) and the six
// gradient outputs, all of one dtype and layout.
struct BwdProblem {
  const void* x;
  const void* l[3];
  const void* lam;
  const void* u;
  const void* gy;
  void* dx;
  void* dl[3];
  void* dlam;
  void* du;
  int64_t B, C, H, W;
  uint32_t mask;
  int64_t G;
  gspn_dtype dtype;
  bool aligned_vec4;   // every pointer aligned to 4 elements
  bool aligned_pair;   // every pointer aligned to 2 elements
  int64_t Cl;          // logit channels (Cl divides C; Cl == C: unshared)
  // Cl < C: the kernels write each plane's logit gradients here in fp32
  // ([3][B*C*H*W]) and bwd_reduce_logits sums each group into dl[]
  float* dlw;
};

// Records caller-owned events around kernel launches (gspn_trace_events),
// and the kernel name and plane count of each launch.
constexpr int kTraceMax = 64;   // launches named per traced call
struct Tracer {
  hipEvent_t* events = nullptr;
  int pairs = 0;
  int count = 0;
  const char* names[kTraceMax] = {};
  int64_t planes[kTraceMax] = {};
  void before(hipStream_t s, const char* name, int64_t np) {
    if (count < kTraceMax) { names[count] = name; planes[count] = np; }
    if (events && count < pairs) (void)hipEventRecord(events[2 * count], s);
  }
  void after(hipStream_t s) {
    if (events && count < pairs) (void)hipEventRecord(events[2 * count + 1], s);
    ++count;
  }
};

// plane-resident path (gspn_plane.hip)
bool plane_fits(int64_t H, int64_t W);
int plane_seg(int64_t H, int64_t W);
size_t plane_lds_bytes(int64_t H, int64_t W);
hipError_t launch_plane(const Problem& pr, hipStream_t stream, Tracer* tr);

// band-resident path for small local groups (gspn_band.hip)
bool band_fits(int64_t H, int64_t W, int64_t G);
hipError_t launch_band(const Problem& pr, hipStream_t stream, Tracer* tr);

// large-plane transpose pipeline (gspn_tpipe.hip)
bool tpipe_fits(int64_t H, int64_t W);
// Plane groups of the large-plane pipelines: each group's chain of launches
// runs on its own stream (the caller's, then helper streams), so that one
// group's tail overlaps the next launch of another.
constexpr int kMaxGroups = 4;
int cu_count();                        // compute units of the current device
hipStream_t aux_stream(int i);         // helper stream i < kMaxGroups - 1 of the device
int tpipe_groups(int64_t planes);      // number of plane groups for a launch
// Calls fn(p0, np, s) for each of tpipe_groups(planes) contiguous plane
// groups [p0, p0 + np): group 0 on `stream`, group g > 0 on helper stream
// g - 1, forked from `stream` before and joined back into it after; the
// first error stops the calls (the forked streams are still joined).
hipError_t run_plane_groups(int64_t planes, hipStream_t stream,
                            const std::function<hipError_t(int64_t, int64_t, hipStream_t)>& fn);
size_t tpipe_workspace_bytes(int64_t planes, int64_t H, int64_t W, gspn_dtype dt);
hipError_t launch_tpipe(const Problem& pr, void* ws, hipStream_t stream, Tracer* tr);

// streaming per-direction path (gspn_stream.hip)
int64_t stream_max_orth();
hipError_t launch_stream(const Problem& pr, float* acc, hipStream_t stream, Tracer* tr);

// per-direction parameters with a per-channel merger (gspn_dirs.hip)
int64_t dirs_max_orth();
size_t dirs_workspace_bytes(int64_t planes, int64_t H, int64_t W, uint32_t mask, gspn_dtype dt);
hipError_t launch_dirs(const Problem& pr, void* ws, hipStream_t stream, Tracer* tr);
// dst[k] = src[k] transposed plane by plane ([planes][R][C] -> [planes][C][R]),
// k < n <= 11, one launch traced as `name` over planes * n units; bf16 with
// even sides and 4-byte aligned tensors moves element pairs
template <typename E>
hipError_t transpose_planes(const E* const* src, E* const* dst, int n, int64_t planes, int R, int C,
                            const char* name, hipStream_t stream, Tracer* tr);

// module prologue: the 1x1 convolutions producing x, the logits, lambda and u
// (gspn_prologue.hip); all tensors [B, *, H, W] of one dtype
struct PrologueProblem {
  const void* x_in;    // [B, Cin, H, W]
  const void* w_r;     // [C, Cin]
  const void* b_r;     // [C] or null
  const void* w_p;     // [5C, C]: l0, l1, l2, lambda, u blocks of C rows
  const void* b_p;     // [5C] or null
  void* x_out;         // [B, C, H, W]
  void* p_out[5];      // l0, l1, l2, lambda, u: [B, C, H, W] each
  int64_t B, Cin, C, H, W;
  gspn_dtype dtype;
};
hipError_t launch_prologue(const PrologueProblem& pr, hipStream_t stream, Tracer* tr);
// the first product alone (x = W_r X_in + b_r into pr.x_out)
hipError_t launch_prologue_reduce(const PrologueProblem& pr, hipStream_t stream, Tracer* tr);

// the parameter product fused with the propagation for small bf16 planes
// (gspn_fused.hip): reads x (as launch_prologue_reduce stored it), W_p and
// b_p of pr, writes out; the parameter tensors are never stored
bool fused_unit_fits(const PrologueProblem& pr);
hipError_t launch_fused_unit(const PrologueProblem& pr, const void* x, void* out, uint32_t mask,
                             int64_t G, hipStream_t stream, Tracer* tr);

// backward pass, plane-resident path for H, W <= 64 (gspn_bwd_plane.hip)
size_t bplane_lds_bytes(int64_t H, int64_t W);
hipError_t launch_bplane(const BwdProblem& pr, hipStream_t stream, Tracer* tr);

// backward pass, band path for local groups G <= 8 (gspn_bwd_band.hip)
bool bband_fits(int64_t H, int64_t W, int64_t G);
size_t bband_workspace_bytes(int64_t planes, int64_t H, int64_t W, uint32_t mask);
hipError_t launch_bband(const BwdProblem& pr, void* ws, hipStream_t stream, Tracer* tr);

// sum per-plane logit gradients over the channels sharing each logit plane
hipError_t launch_bwd_reduce_logits(const BwdProblem& pr, hipStream_t stream, Tracer* tr);

// backward pass, streaming path for any plane (gspn_bwd_stream.hip)
size_t bwd_stream_workspace_bytes(int64_t planes, int64_t H, int64_t W, uint32_t mask,
                                  gspn_dtype dt);
hipError_t launch_bwd_stream(const BwdProblem& pr, void* ws, hipStream_t stream, Tracer* tr);

// backward pass of the per-direction layer (gspn_bwd_stream.hip): pr's
// lambda, logits and u are direction 0's, direction d's sit at element
// offset d * dir_stride; the gradients dl / dlam / du are [4][B*C*H*W]
// (slice d = direction d), dx [B*C*H*W]; dmerge [4][C] fp32, or null
struct BwdDirsExtra {
  int64_t dir_stride;
  const float* merge;   // [4][C] device, or null (all ones)
  float* dmerge;
};
size_t bwd_dirs_workspace_bytes(int64_t planes, int64_t H, int64_t W, uint32_t mask,
                                gspn_dtype dt);
hipError_t launch_bwd_dirs(const BwdProblem& pr, const BwdDirsExtra& ex, void* ws,
                           hipStream_t stream, Tracer* tr);

// backward pass, large-plane pipeline (gspn_bwd_tpipe.hip): planes with both
// sides even, W <= 1024, H <= 2048, every pointer aligned to 2 elements
bool btpipe_fits(int64_t H, int64_t W);
size_t bwd_tpipe_workspace_bytes(int64_t planes, int64_t H, int64_t W, uint32_t mask,
                                 gspn_dtype dt);
hipError_t launch_bwd_tpipe(const BwdProblem& pr, void* ws, hipStream_t stream, Tracer* tr);

}  // namespace gspn
