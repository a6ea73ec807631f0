/*
 * gspn.h -- C ABI of the MI355X (gfx950) GSPN 2D line-scan propagation.
 *
 * The operation (CSDN page "GSPN——在convolution基础上并行序列建模", sections
 * 方法 and 如何设计一个高效的传播层; aitntnews page on GSPN, section
 * 传播层的关键实现):
 *
 *   for every plane (b, c) and every scan direction d selected in dir_mask,
 *     h_s = w_s h_{s-1} + lambda_s (.) x_s,   h before the first line = 0,
 *   where line s is a row (vertical scans) or a column (horizontal scans) and
 *   w_s is tridiagonal: pixel o of line s mixes pixels o-1, o, o+1 of line
 *   s-1 (up-left, up, up-right for the top->bottom scan) with weights
 *     w_k = sigmoid(l_k) / sum over in-range k' of sigmoid(l_k'),
 *   l_k being the logit stored at pixel (line s, o) for orthogonal offset
 *   k-1 in image coordinates. Every row of w_s sums to one (row-stochastic:
 *   section 稳定性-上下文条件, Theorem 1). Neighbours outside the image do not
 *   exist (edge pixels normalise over two, or one, neighbours).
 *
 *   out = sum over selected d of u (.) h_d       (output gate y = u (.) h,
 *                                                 four-direction merge as a sum)
 *
 *   Local variant (section GSPN模块的设计): with group_rows = G >= 1 the scan
 *   axis is cut into blocks of G consecutive positions [mG, (m+1)G) in image
 *   coordinates (the last block may be shorter) and the state restarts at 0
 *   whenever a scan enters a block, on both axes and in both scan orders.
 *
 * Layout: every tensor is a contiguous [B, C, H, W] array (W fastest) of one
 * element type (dtype); all pointers are device memory owned by the caller.
 * Arithmetic is fp32 for both storage types; bf16 outputs are rounded once
 * (round-to-nearest-even) from the fp32 sum.
 *
 * Errors: every argument is validated on the host before anything is
 * enqueued; on an error nothing is enqueued and out is untouched. Launch
 * failures are reported as GSPN_E_HIP with the HIP error text available from
 * gspn_last_error(). Work is asynchronous on `stream`; faults inside a kernel
 * surface at the caller's next synchronisation. No call keeps a pointer after
 * it returns. Calls are reentrant; gspn_last_error() is per thread.
 */
#ifndef GSPN_H
#define GSPN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GSPN_F32 = 0,
  GSPN_BF16 = 1,
  /* Not element types. They give gspn_dtype the range of a 32-bit int, so
   * that any value a caller passes is a valid value of the type and can be
   * checked (GSPN_E_DTYPE) without undefined behaviour in C++. */
  GSPN_DTYPE_RANGE_MIN_ = -2147483647 - 1,
  GSPN_DTYPE_RANGE_MAX_ = 2147483647
} gspn_dtype;

/* scan directions: top->bottom, bottom->top, left->right, right->left */
enum {
  GSPN_T2B = 1u,
  GSPN_B2T = 2u,
  GSPN_L2R = 4u,
  GSPN_R2L = 8u,
  GSPN_ALL = 15u
};

typedef enum {
  GSPN_OK = 0,
  GSPN_E_NULL = 1,      /* a required pointer is NULL                      */
  GSPN_E_SHAPE = 2,     /* B, C < 0, H, W < 1, or the size overflows       */
  GSPN_E_DIRMASK = 3,   /* dir_mask is 0 or has bits above GSPN_ALL        */
  GSPN_E_GROUP = 4,     /* group_rows < 0                                  */
  GSPN_E_DTYPE = 5,     /* dtype is not a gspn_dtype                       */
  GSPN_E_ALIGN = 6,     /* a pointer is not aligned to its element size    */
  GSPN_E_ALIAS = 7,     /* an output overlaps an input or another output   */
  GSPN_E_NOMEM = 8,     /* the stream-ordered workspace allocation failed  */
  GSPN_E_HIP = 9,       /* a HIP call or kernel launch failed              */
  GSPN_E_WORKSPACE = 10 /* workspace is NULL or smaller than required      */
} gspn_status;

/*
 * gspn_propagate -- out = sum_{d in dir_mask} u (.) h_d (see above).
 *   x, lambda, u        inputs [B, C, H, W]
 *   w_logits[0..2]      logits for orthogonal offsets -1, 0, +1
 *   dir_mask            OR of GSPN_T2B/B2T/L2R/R2L
 *   group_rows          0: global scan; G >= 1: local groups of G positions
 *                       (G >= max(H, W) is the same as global)
 *   dtype               element type of all seven tensors
 *   out                 [B, C, H, W], write-only, fully overwritten; must not
 *                       overlap any input
 *   stream              HIP stream the work is enqueued on (0 = default)
 * B*C == 0 is valid and enqueues nothing. When the chosen plan needs scratch
 * memory (gspn_workspace_bytes > 0) it is taken with hipMallocAsync and given
 * back with hipFreeAsync on `stream`.
 */
gspn_status gspn_propagate(const void* x, const void* const w_logits[3],
                           const void* lambda, const void* u, int64_t B,
                           int64_t C, int64_t H, int64_t W, uint32_t dir_mask,
                           int64_t group_rows, gspn_dtype dtype, void* out,
                           hipStream_t stream);

/*
 * gspn_propagate_noalloc -- gspn_propagate for callers that cannot allocate
 * device memory (code under HIP graph capture, serving loops, harnesses that
 * forbid hipMalloc). Same arguments, layout and result as gspn_propagate; it
 * calls no hipMalloc, hipFree or other allocating routine, creates no stream
 * or event, and enqueues every launch on `stream`.
 *
 * Scratch memory comes from one array of gspn_noalloc_scratch_bytes()
 * (64 MiB) per device, a static device variable of the library: each device
 * the library runs on holds it from the library's load until the process
 * ends. A problem whose gspn_workspace_bytes() exceeds that size returns
 * GSPN_E_WORKSPACE before anything is enqueued. Every call on one device uses
 * the same array and leaves its contents behind (nothing in it needs to start
 * at zero): calls whose work overlaps in time on one device, on different
 * streams or from different threads, race on it and give wrong results, so
 * the caller serialises them. The array's address is looked up once per
 * device (on that device's first call whose plan needs scratch).
 */
gspn_status gspn_propagate_noalloc(const void* x, const void* const w_logits[3],
                                   const void* lambda, const void* u, int64_t B,
                                   int64_t C, int64_t H, int64_t W, uint32_t dir_mask,
                                   int64_t group_rows, gspn_dtype dtype, void* out,
                                   hipStream_t stream);

/* gspn_noalloc_scratch_bytes -- size of gspn_propagate_noalloc's per-device
 * scratch array in bytes. */
size_t gspn_noalloc_scratch_bytes(void);

/*
 * gspn_workspace_bytes -- scratch bytes gspn_propagate_ws needs for this
 * problem (0 when the plan keeps everything on chip). Returns 0 for invalid
 * arguments as well; gspn_propagate_ws reports those.
 */
size_t gspn_workspace_bytes(int64_t B, int64_t C, int64_t H, int64_t W,
                            uint32_t dir_mask, int64_t group_rows,
                            gspn_dtype dtype);

/*
 * gspn_propagate_ws -- gspn_propagate with caller-owned scratch memory:
 * `workspace` is device memory of at least ws_bytes >= gspn_workspace_bytes()
 * bytes, 256-byte aligned, not overlapping any tensor, and not used by
 * anything else until the enqueued work has finished. It may be NULL when the
 * required size is 0.
 */
gspn_status gspn_propagate_ws(const void* x, const void* const w_logits[3],
                              const void* lambda, const void* u, int64_t B,
                              int64_t C, int64_t H, int64_t W,
                              uint32_t dir_mask, int64_t group_rows,
                              gspn_dtype dtype, void* out, void* workspace,
                              size_t ws_bytes, hipStream_t stream);

/*
 * gspn_plan_name -- name of the kernel plan gspn_propagate would use for this
 * problem ("plane16", "plane64", "stream", ...), or "invalid". Host-only.
 */
const char* gspn_plan_name(int64_t B, int64_t C, int64_t H, int64_t W,
                           uint32_t dir_mask, int64_t group_rows,
                           gspn_dtype dtype);

/*
 * gspn_trace_events -- optional launch tracing for benchmarks and profilers.
 * While `events` is non-NULL, every following gspn_propagate* call made by
 * the calling thread records events[2*i] right before and events[2*i + 1]
 * right after its i-th kernel launch (for i < n_pairs) on the call's stream.
 * The events are created and destroyed by the caller (hipEventCreate); the
 * library only records them. gspn_trace_count() returns how many launches the
 * last traced call made (which may exceed n_pairs). Pass NULL to stop.
 */
void gspn_trace_events(hipEvent_t* events, int n_pairs);
int gspn_trace_count(void);

/*
 * gspn_trace_kernel -- name of the kernel of launch i of the last traced call
 * (static string), storing the number of planes it processed in *planes;
 * NULL when i is out of range (the first 64 launches of a call are named).
 * Launches may run on a library-owned helper
 * stream that is forked from and joined back to the caller's stream; each
 * launch's events are recorded on the stream that launch runs on.
 */
const char* gspn_trace_kernel(int i, int64_t* planes);

/* gspn_status_str -- static text of a status code. */
const char* gspn_status_str(gspn_status status);

/* gspn_last_error -- detail of the calling thread's last failed call
 * (e.g. the HIP error string); "" if none. Valid until the next call. */
const char* gspn_last_error(void);

/* gspn_abi_version -- version of this ABI (bumped on incompatible change). */
int gspn_abi_version(void);

/*
 * gspn_propagate_backward -- gradients of every input of gspn_propagate
 * (CSDN page, section 反向传播: the gradient of a line's hidden state collects
 * what the later lines send back, the input gradient goes through the lambda
 * factor, and the gate gradients pair the error term with the previous hidden
 * state). For a scalar loss L and grad_out = dL/dout:
 *   e_{d,s} = u (.) grad_out + w_{d,s+1}^T e_{d,s+1}
 *       (reverse scan with the transposed tridiagonal; a line that restarts
 *        sends nothing back to the line before it)
 *   grad_x      = lambda (.) sum_d e_d
 *   grad_lambda = x (.) sum_d e_d
 *   grad_u      = grad_out (.) sum_d h_d
 *   grad_logits[k] at pixel (s, o) = sum_d e_{d,s}[o] w_k (1 - sigmoid(l_k))
 *       (h_{d,s-1}[o+k-1] - sum_j w_j h_{d,s-1}[o+j-1])
 *       -- the chain rule through the row normalisation and the sigmoid;
 *       0 on restart lines and for links that would leave the image.
 * Problem arguments (x, w_logits, lambda, u, B, C, H, W, dir_mask,
 * group_rows, dtype, stream) as for gspn_propagate. grad_out has the same
 * layout and dtype. grad_x, grad_logits[0..2], grad_lambda and grad_u are
 * [B, C, H, W] in dtype (bf16 rounded once from the fp32 result),
 * write-only, fully overwritten, and may not overlap an input or each other
 * (GSPN_E_ALIAS). Scratch memory (gspn_backward_workspace_bytes) is taken
 * with hipMallocAsync and given back with hipFreeAsync on `stream`.
 * Errors as for gspn_propagate.
 */
gspn_status gspn_propagate_backward(const void* x, const void* const w_logits[3],
                                    const void* lambda, const void* u,
                                    const void* grad_out, int64_t B, int64_t C,
                                    int64_t H, int64_t W, uint32_t dir_mask,
                                    int64_t group_rows, gspn_dtype dtype,
                                    void* grad_x, void* const grad_logits[3],
                                    void* grad_lambda, void* grad_u,
                                    hipStream_t stream);

/* gspn_backward_workspace_bytes -- scratch bytes gspn_propagate_backward_ws
 * needs (0 for invalid arguments, which the call itself reports). */
size_t gspn_backward_workspace_bytes(int64_t B, int64_t C, int64_t H, int64_t W,
                                     uint32_t dir_mask, int64_t group_rows,
                                     gspn_dtype dtype);

/* gspn_propagate_backward_ws -- gspn_propagate_backward with caller-owned
 * scratch memory, under the same rules as gspn_propagate_ws. */
gspn_status gspn_propagate_backward_ws(const void* x, const void* const w_logits[3],
                                       const void* lambda, const void* u,
                                       const void* grad_out, int64_t B, int64_t C,
                                       int64_t H, int64_t W, uint32_t dir_mask,
                                       int64_t group_rows, gspn_dtype dtype,
                                       void* grad_x, void* const grad_logits[3],
                                       void* grad_lambda, void* grad_u,
                                       void* workspace, size_t ws_bytes,
                                       hipStream_t stream);

/*
 * Channel-shared logits (CSDN page, section 局限性: the speed test sets the
 * weights' feature dimension to 1). The three logit tensors are
 * [B, logit_channels, H, W] with logit_channels dividing C; channel c uses
 * logit channel c / (C / logit_channels) of its batch entry.
 * logit_channels == C is the unshared layer. A logit_channels that is < 1 or
 * does not divide C gives GSPN_E_SHAPE.
 *
 * gspn_propagate_shared_ws -- gspn_propagate_ws with shared logits (same
 * workspace size: gspn_workspace_bytes).
 */
gspn_status gspn_propagate_shared_ws(const void* x, const void* const w_logits[3],
                                     int64_t logit_channels, const void* lambda,
                                     const void* u, int64_t B, int64_t C, int64_t H,
                                     int64_t W, uint32_t dir_mask, int64_t group_rows,
                                     gspn_dtype dtype, void* out, void* workspace,
                                     size_t ws_bytes, hipStream_t stream);

/*
 * gspn_propagate_backward_shared_ws -- gspn_propagate_backward_ws with
 * shared logits. grad_logits[0..2] are [B, logit_channels, H, W]: each is the
 * sum, in channel order, over the channels that read that logit. The
 * workspace (gspn_backward_workspace_bytes_shared) then also holds the fp32
 * per-channel logit gradients before that sum.
 */
gspn_status gspn_propagate_backward_shared_ws(const void* x, const void* const w_logits[3],
                                              int64_t logit_channels, const void* lambda,
                                              const void* u, const void* grad_out,
                                              int64_t B, int64_t C, int64_t H, int64_t W,
                                              uint32_t dir_mask, int64_t group_rows,
                                              gspn_dtype dtype, void* grad_x,
                                              void* const grad_logits[3],
                                              void* grad_lambda, void* grad_u,
                                              void* workspace, size_t ws_bytes,
                                              hipStream_t stream);
size_t gspn_backward_workspace_bytes_shared(int64_t B, int64_t C, int64_t H, int64_t W,
                                            int64_t logit_channels, uint32_t dir_mask,
                                            int64_t group_rows, gspn_dtype dtype);

/*
 * Per-direction parameters with a per-channel merger (aitntnews page, sections
 * 二维线性传播 and GSPN架构: every scan direction has its own normalised
 * weight matrices, and a learnable merger combines the directions; CSDN page,
 * section GSPN模块的设计: the merger is a linear layer over the directions).
 *
 *   out[b,c] = sum over d in dir_mask of merge[d * C + c] * u_d (.) h_d,
 *   h_d = direction d's line scan of x with lambda_d and logits l_{d,0..2}.
 *
 * Direction d (0 top->bottom, 1 bottom->top, 2 left->right, 3 right->left)
 * reads lambda, w_logits[0..2] and u at element offset d * dir_stride from the
 * given pointers, each a contiguous [B, C, H, W] tensor; x is shared by all
 * directions. dir_stride = 0 gives every direction the same parameters, and
 * with merge = NULL that is gspn_propagate_ws's result. A dir_stride between
 * 1 and B*C*H*W - 1 (overlapping directions) gives GSPN_E_SHAPE.
 *
 * merge: device memory, 4 * C fp32 values, direction-major, caller-owned, or
 * NULL for all ones; only the selected directions' rows are read.
 * H and W must be <= 8192 (GSPN_E_SHAPE). out may overlap no byte that the
 * call reads (GSPN_E_ALIAS). The sum over directions is taken in fp32 in the
 * fixed order left->right, right->left, top->bottom, bottom->top and rounded
 * once to the storage type.
 *
 * Workspace: gspn_workspace_bytes_dirs() bytes, 256-byte aligned, caller-owned:
 * fp32 partial sums, and with a horizontal direction selected, transposed
 * copies of x and of each selected horizontal direction's five tensors. It is
 * 0 for a single vertical direction and for planes up to 64 x 64 (one
 * wavefront per plane, the sum over the directions kept on chip); workspace
 * may then be NULL. Same status codes as gspn_propagate_ws.
 */
gspn_status gspn_propagate_dirs_ws(const void* x, const void* const w_logits[3],
                                   const void* lambda, const void* u, int64_t dir_stride,
                                   const float* merge, int64_t B, int64_t C, int64_t H,
                                   int64_t W, uint32_t dir_mask, int64_t group_rows,
                                   gspn_dtype dtype, void* out, void* workspace,
                                   size_t ws_bytes, hipStream_t stream);
size_t gspn_workspace_bytes_dirs(int64_t B, int64_t C, int64_t H, int64_t W,
                                 uint32_t dir_mask, int64_t group_rows, gspn_dtype dtype);

/*
 * Backward pass of the per-direction layer (CSDN page, section 反向传播; the
 * layer as gspn_propagate_dirs_ws). Direction d is one scan with its own
 * lambda, logits and u whose error term starts from merge[d * C + c] * u_d *
 * grad_out; the results are
 *   grad_x                 = sum over d of lambda_d (.) e_d   (e_d summed along its scan),
 *   grad_lambda slice d    = x (.) e_d,
 *   grad_logits[k] slice d = the logit gradients of direction d's scan,
 *   grad_u slice d         = merge[d * C + c] * grad_out (.) h_d,
 *   grad_merge[d * C + c]  = sum over the batch and the pixels of u_d grad_out h_d.
 * Inputs as gspn_propagate_dirs_ws (x, w_logits, lambda, u, dir_stride,
 * merge), plus grad_out [B, C, H, W] in the storage type. Outputs, device
 * memory in the storage type, caller-owned, fully overwritten: grad_x
 * [B, C, H, W]; grad_logits[0..2], grad_lambda, grad_u [4, B, C, H, W] (slice
 * d = direction d, dense, whatever dir_stride is; zero for directions outside
 * dir_mask); grad_merge: 4 * C fp32 values, or NULL to skip them. No output
 * may overlap an input or another output (GSPN_E_ALIAS); H and W <= 8192.
 * Every direction runs as its own scan pair; the horizontal ones on
 * transposed copies. Workspace: gspn_backward_workspace_bytes_dirs() bytes,
 * 256-byte aligned, caller-owned (the stored states, an fp32 sum for grad_x,
 * with a horizontal direction selected the transposed copies, and four fp64
 * merge-gradient partials per plane). Same status codes as
 * gspn_propagate_backward_ws.
 */
gspn_status gspn_propagate_backward_dirs_ws(
    const void* x, const void* const w_logits[3], const void* lambda, const void* u,
    int64_t dir_stride, const float* merge, const void* grad_out, int64_t B, int64_t C,
    int64_t H, int64_t W, uint32_t dir_mask, int64_t group_rows, gspn_dtype dtype, void* grad_x,
    void* const grad_logits[3], void* grad_lambda, void* grad_u, float* grad_merge,
    void* workspace, size_t ws_bytes, hipStream_t stream);
size_t gspn_backward_workspace_bytes_dirs(int64_t B, int64_t C, int64_t H, int64_t W,
                                          uint32_t dir_mask, int64_t group_rows,
                                          gspn_dtype dtype);

/*
 * The module prologue (aitntnews page, section GSPN架构: a shared 1x1
 * convolution reduces the channels, then three independent 1x1 convolutions
 * produce the input-dependent propagation parameters). Per pixel:
 *
 *   x      = w_reduce (C x Cin) x_in + b_reduce          -> x_out
 *   params = w_params (5C x C)  x    + b_params          -> params_out[0..4]
 *
 * where params rows t*C .. t*C+C-1 are l0, l1, l2, lambda, u for t = 0..4
 * (the logit convolution is rows 0 .. 3C-1). Every output is rounded once,
 * to nearest even, to the storage dtype, and the parameter convolutions read
 * x as stored. No activation is applied (the propagation takes logits).
 *
 * x_in [B, Cin, H, W]; w_reduce [C, Cin]; b_reduce [C] or NULL (zero);
 * w_params [5C, C]; b_params [5C] or NULL; x_out and params_out[0..4]
 * [B, C, H, W]. All device memory of one dtype, caller-owned. Outputs may
 * overlap neither an input nor each other (GSPN_E_ALIAS). B <= 65535 and
 * H * W < 2^31 (GSPN_E_SHAPE). Computed with MFMA in fp32 accumulation.
 * Enqueued on `stream`; no workspace.
 */
gspn_status gspn_prologue(const void* x_in, int64_t Cin, const void* w_reduce,
                          const void* b_reduce, const void* w_params, const void* b_params,
                          int64_t B, int64_t C, int64_t H, int64_t W, gspn_dtype dtype,
                          void* x_out, void* const params_out[5], hipStream_t stream);

/*
 * The whole GSPN unit: gspn_prologue into the workspace, then
 * gspn_propagate_ws on its outputs, out = sum_d u (.) h_d over dir_mask.
 * Workspace: gspn_module_workspace_bytes() bytes, 256-byte aligned,
 * caller-owned (the prologue's six tensors and the propagation's
 * workspace). out [B, C, H, W] may not overlap an input or the workspace.
 * Same status codes as gspn_prologue and gspn_propagate_ws.
 */
gspn_status gspn_module_ws(const void* x_in, int64_t Cin, const void* w_reduce,
                           const void* b_reduce, const void* w_params, const void* b_params,
                           int64_t B, int64_t C, int64_t H, int64_t W, uint32_t dir_mask,
                           int64_t group_rows, gspn_dtype dtype, void* out, void* workspace,
                           size_t ws_bytes, hipStream_t stream);
size_t gspn_module_workspace_bytes(int64_t B, int64_t C, int64_t H, int64_t W,
                                   uint32_t dir_mask, int64_t group_rows, gspn_dtype dtype);

/* gspn_backward_plan_name -- kernel plan gspn_propagate_backward would use,
 * or "invalid". Host-only. */
const char* gspn_backward_plan_name(int64_t B, int64_t C, int64_t H, int64_t W,
                                    uint32_t dir_mask, int64_t group_rows,
                                    gspn_dtype dtype);

#ifdef __cplusplus
}
#endif

#endif /* GSPN_H */
