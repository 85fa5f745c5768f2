/*
 * lapattn.h -- Nystrom-approximated, softmax-free kernel attention (forward)
 * for AMD Instinct MI355X (gfx950).  Plain C ABI: no C++ types, no exceptions,
 * no allocation inside the library's compute entry points.
 *
 * What one call computes, independently for every head (b, h):
 *
 *   L     = average pool of K over non-overlapping pool_h x pool_w windows of
 *           the grid_h x grid_w token grid, windows in raster order
 *           (SOFT review, "method": bottleneck tokens by average pooling;
 *           LaplacianFormer summaries, Nystrom paragraph: landmark keys by
 *           average pooling)                                         [m x d]
 *   K_QL  = k(Q, L),  K_LK = k(L, K)                   [N x m], [m x N]
 *           Laplacian k(x, y) = exp(-||x - y||_1 / lambda)
 *           (LaplacianFormer summaries, kernel definition in the method
 *           section);  Gaussian variant k(x, y) = exp(-||x - y||_2^2 / lambda)
 *           (SOFT review, "method": symmetric kernel S = exp(Q (-) K); the
 *           caller passes lambda = 2 sqrt(d) for SOFT's scale)
 *   A     = k(L, L) + eps I   (diagonal perturbation that makes the landmark
 *           matrix strictly positive definite; LaplacianFormer summaries,
 *           Newton-Schulz paragraph)                                 [m x m]
 *   X     = Newton-Schulz inverse of A: X_0 = alpha A,
 *           X_{t+1} = 2 X_t - X_t A X_t, exactly `iters` steps,
 *           alpha = 1 / (||A||_1 ||A||_inf)
 *           (SOFT review, "method": the A_0 / A_{k+1} recursion)     [m x m]
 *   O     = K_QL (X (K_LK V))   (SOFT review, "method": S_hat = P^T A^+ P,
 *           applied to V with no further normalisation)              [N x d]
 *
 * Data layout.  Q, K, V and O are device pointers to [B, H, N, d] C-contiguous
 * tensors, 16-byte aligned, N = grid_h * grid_w, token n = row * grid_w + col.  The element
 * type is fp32 (LAPATTN_F32) or bf16 (LAPATTN_BF16) for all four.  Accuracy
 * is that of fp32: kernel values in fp32; the Newton-Schulz products, X W
 * and K_QL Y as fp32 sums of fp16 two-part operands scaled by powers of two
 * (about 22 significant bits per operand); K_LK V in fp32.  bf16 outputs
 * are rounded to nearest even.
 *
 * Ownership.  The caller allocates and frees Q, K, V, O and the workspace.
 * Compute entry points never allocate or free memory and never synchronise
 * with the host: work is enqueued on `stream` (a hipStream_t passed as void*;
 * NULL is the default stream) and the call returns after the enqueue.  K may
 * be the same pointer as Q (the shared projection of the Gaussian variant);
 * O must not overlap Q, K, V or the workspace.
 *
 * Errors.  Every entry point returning int returns LAPATTN_OK (0) or one of
 * the negative codes below.  All argument checks run on the host before the
 * first launch, so on an argument error nothing is enqueued.  Inputs are not
 * scanned: NaN and Inf propagate to the output.
 */
#ifndef LAPATTN_H
#define LAPATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LAPATTN_VERSION 1
#define LAPATTN_MAX_LANDMARKS 64
#define LAPATTN_MAX_ITERS 64

typedef enum {
  LAPATTN_KERNEL_LAPLACIAN = 0,   /* exp(-||x - y||_1 / lambda)   */
  LAPATTN_KERNEL_GAUSSIAN = 1     /* exp(-||x - y||_2^2 / lambda) */
} lapattn_kernel_t;

typedef enum {
  LAPATTN_F32 = 0,
  LAPATTN_BF16 = 1
} lapattn_dtype_t;

/* Launch-plan flags (lapattn_desc_t.flags). */
#define LAPATTN_FLAG_SERIAL 1u  /* launch the Newton-Schulz solver and the
                                   kernel-map/W stage as two kernels, one after
                                   the other; by default one launch carries
                                   both as separate workgroup roles, so the
                                   solver overlaps the map stage.  Results are
                                   bitwise identical either way. */
#define LAPATTN_FLAG_TICKETS 2u /* hand the main launch's workgroup roles out
                                   by ticket, in the order workgroups start,
                                   instead of by workgroup index.  By default
                                   each XCD dispatching its workgroups in
                                   index order guarantees that producers run
                                   before their consumers wait; tickets drop
                                   that assumption, at the cost of a few us of
                                   contended counters per launch.  Results are
                                   bitwise identical either way. */

enum {
  LAPATTN_OK = 0,
  LAPATTN_ERR_NULL = -1,         /* a required pointer is NULL              */
  LAPATTN_ERR_SHAPE = -2,        /* non-positive size, grid not divisible by
                                    the pool, unsupported head dim d          */
  LAPATTN_ERR_M_TOO_LARGE = -3,  /* m = (grid_h/pool_h)*(grid_w/pool_w) > 64 */
  LAPATTN_ERR_PARAM = -4,        /* lambda <= 0 or not finite, eps < 0 or not
                                    finite, iters outside [0, 64], bad kernel
                                    or flags                                  */
  LAPATTN_ERR_DTYPE = -5,        /* unknown dtype                             */
  LAPATTN_ERR_ALIAS = -6,        /* O overlaps an input or the workspace      */
  LAPATTN_ERR_WORKSPACE = -7,    /* workspace smaller than required / unaligned*/
  LAPATTN_ERR_HIP = -8,          /* a HIP runtime call or launch failed       */
  LAPATTN_ERR_ALIGN = -9,        /* q, k, v or out not 16-byte aligned        */
  LAPATTN_ERR_SCRATCH = -10      /* lapattn_forward_noalloc: the call needs
                                    more workspace than the static scratch   */
};

/* Size of the static device scratch behind lapattn_forward_noalloc. */
#define LAPATTN_NOALLOC_SCRATCH_BYTES (128u << 20)

/* Launch slots of one forward or backward call, in launch order (for
 * lapattn_set_stage_events). */
#define LAPATTN_STAGE_POOL 0     /* landmark average pool                      */
#define LAPATTN_STAGE_MAIN 1     /* A = k(L,L) + eps I, alpha and Newton-Schulz;
                                    in the default plan also the K_QL / K_LK
                                    maps, W = K_LK V, Y = X W and (Q != K) the
                                    output rows                                */
#define LAPATTN_STAGE_MAPS 2     /* LAPATTN_FLAG_SERIAL only: the map roles as
                                    a launch of their own                      */
#define LAPATTN_STAGE_OUT 3      /* O = K_QL Y as its own launch: when K == Q,
                                    or when the main grid cannot be resident
                                    on the device at once (lapattn_launches
                                    reports which)                             */
/* lapattn_backward's launches (the pool of slot 0 comes first) */
#define LAPATTN_STAGE_BWD_PART 4 /* A, alpha and Newton-Schulz with every iterate
                                    stored, beside the W^T and dY^T partials  */
#define LAPATTN_STAGE_BWD_HEAD 5 /* per head: W, dY, Y, dX, dW             */
#define LAPATTN_STAGE_BWD_GRAD 6 /* the Newton-Schulz backward and dL from A,
                                    beside per token tile: dQ, direct dK, dV
                                    and the dL partials                       */
#define LAPATTN_STAGE_BWD_DK 7   /* dK += pool backward of dL                 */
#define LAPATTN_NUM_STAGES 8

typedef struct {
  int32_t B, H;            /* batch and heads; every (b, h) is independent   */
  int32_t grid_h, grid_w;  /* token grid; N = grid_h * grid_w                 */
  int32_t d;               /* head dimension: 16, 32 or 64                    */
  int32_t pool_h, pool_w;  /* average-pool window = stride; must divide grid  */
  int32_t kernel;          /* lapattn_kernel_t                                */
  int32_t dtype;           /* lapattn_dtype_t, for Q, K, V and O              */
  uint32_t flags;          /* LAPATTN_FLAG_*                                  */
} lapattn_desc_t;

/* Library version (LAPATTN_VERSION). */
int lapattn_version(void);

/* Static text for a status code; never NULL. */
const char* lapattn_strerror(int status);

/* Validates a descriptor and the scalar parameters without touching any
 * device.  Returns LAPATTN_OK or the error lapattn_forward would return for
 * the same arguments (pointer checks aside). */
int lapattn_check(const lapattn_desc_t* desc, float lambda, float eps, int32_t iters);

/* Bytes of device workspace lapattn_forward needs for `desc` (256-byte
 * aligned base required); 0 if the descriptor is invalid.  The size is linear
 * in B*H*N.
 * The launch plan (tiles per key workgroup, hence the workspace size, the
 * order in which W's partial sums are added and so the bitwise result) is
 * derived from the compute-unit count of the device that is current on the
 * calling thread (256 is assumed when no device can be queried).  Size the
 * workspace, and call lapattn_forward, with the same device current. */
size_t lapattn_workspace_bytes(const lapattn_desc_t* desc);

/* Byte offset, inside the workspace of a call with this descriptor, of the
 * call's status word (uint32, 4-byte aligned; (size_t)-1 if the descriptor is
 * invalid).  Every forward call sets it to 0 in its first launch; afterwards
 * it holds the number of in-launch waits of that call that ran out of time
 * (see lapattn_forward).  A nonzero value means the call's output is INVALID.
 * Read it (e.g. a 4-byte device-to-host copy ordered after the call on the
 * same stream) before the workspace is used by another call. */
size_t lapattn_status_offset(const lapattn_desc_t* desc);

/* Checks that a HIP device is current and caches its compute-unit count (the
 * only per-device state the library keeps: one int per device, written once,
 * read by the launch plan).  Optional; it exists so that callers can fail
 * early. */
int lapattn_init(void);

/* O = K_QL (X (K_LK V)) per head, as defined at the top of this file.
 *   q, k, v   device, [B, H, N, d], element type desc->dtype (k may equal q)
 *   lambda    kernel length scale (> 0)
 *   eps       diagonal perturbation of the landmark matrix (>= 0)
 *   iters     Newton-Schulz steps, exact (0 .. 64), no early exit
 *   out       device, [B, H, N, d], element type desc->dtype
 *   workspace device scratch of lapattn_workspace_bytes(desc) bytes, 256-byte
 *             aligned; its contents on entry are ignored
 *   stream    hipStream_t (as void*) the work is ordered on
 * Concurrent calls that share a workspace race.  Within a call, workgroups
 * of one launch hand per-head results to each other through the workspace
 * (device-scope stores, then a per-workgroup flag).  Every such wait is
 * bounded (20 ms of the device clock); a wait that runs out counts one in the
 * call's status word (lapattn_status_offset) and the call's output is then
 * invalid, although the call itself has returned LAPATTN_OK (the library
 * never synchronises, so it cannot report it as a return value). */
int lapattn_forward(const lapattn_desc_t* desc, const void* q, const void* k,
                    const void* v, float lambda, float eps, int32_t iters,
                    void* out, void* workspace, size_t workspace_bytes,
                    void* stream);

/* Backward pass: gradients of a scalar loss with respect to Q, K and V given
 * dO, its gradient with respect to O = lapattn_forward(Q, K, V).  The
 * LaplacianFormer summaries say the method's custom kernels serve the
 * backward pass as well as the forward pass (Dutch summary, "Methodologie"
 * item 3; Arabic summary, section 2(c) item 3) without giving formulas; this
 * is the exact reverse-mode derivative of the forward defined at the top of
 * this file, step by step (the Newton-Schulz steps, alpha's maxima and the
 * landmark pool included).  Where the forward is not differentiable the
 * subgradient is: d|t|/dt = sign(t) with sign(0) = 0; alpha's derivative
 * through the first column (= row, A being exactly symmetric) of largest
 * abs-sum.
 *   q, k, v, dout   device, [B, H, N, d], element type desc->dtype (k may
 *                   equal q: the shared projection's gradient is dq + dk)
 *   lambda, eps, iters  as for lapattn_forward
 *   dq, dk, dv      device, [B, H, N, d], element type desc->dtype; written
 *                   in full; they must not overlap each other, an input or
 *                   the workspace
 *   workspace       device scratch of lapattn_backward_workspace_bytes(desc,
 *                   iters) bytes, 256-byte aligned; contents on entry ignored
 * The forward quantities it needs (landmarks, kernel maps, every
 * Newton-Schulz iterate, W, Y) are recomputed, not taken from a forward call.
 * desc->flags is ignored.  Compute is fp32 (MFMA for the products, FP32 VALU
 * for the distance derivatives); bf16 outputs are rounded to nearest even.
 * Five launches on `stream`; no waits across workgroups, no allocation, no
 * synchronisation.  Returns LAPATTN_OK or the argument errors of
 * lapattn_forward. */
size_t lapattn_backward_workspace_bytes(const lapattn_desc_t* desc, int32_t iters);
int lapattn_backward(const lapattn_desc_t* desc, const void* q, const void* k,
                     const void* v, const void* dout, float lambda, float eps,
                     int32_t iters, void* dq, void* dk, void* dv,
                     void* workspace, size_t workspace_bytes, void* stream);

/* LaplacianFormer's normalised feature map in place of the raw query-side
 * kernel values (Arabic summary, section 2(b); Dutch summary, "Methodologie"
 * item 1: each query's similarity vector centred and whitened, with a
 * diagonal estimator that normalises every feature dimension on its own
 * across the batch instead of the covariance's inverse square root):
 *   Z = (K_QL - mu) / sqrt(var + delta), mu_j and var_j the mean and the
 *   population variance of column j (landmark j) of K_QL over the head's N
 *   queries;  O = Z (X (K_LK V)).
 * Readings (the pages print no formula): the similarity vector of query i is
 * row i of K_QL; the batch is the head's N queries; delta >= 0 is the
 * whitening's stabiliser.  Arguments and workspace as for lapattn_forward,
 * plus delta (LAPATTN_ERR_PARAM when negative or not finite).  Takes the
 * output-launch plan (K_QL stored), plus one statistics launch. */
int lapattn_forward_normalized(const lapattn_desc_t* desc, const void* q,
                               const void* k, const void* v, float lambda,
                               float eps, int32_t iters, float delta, void* out,
                               void* workspace, size_t workspace_bytes,
                               void* stream);

/* The landmark solve on its own: Y = A^{-1} W per head, A = k(L, L) + eps I
 * built as in lapattn_forward, by one of two solvers, for the comparison the
 * LaplacianFormer summaries draw between them (Arabic summary, section 4,
 * efficiency analysis: Newton-Schulz more stable and better converging than
 * conjugate-gradient solvers, above all on ill-conditioned matrices):
 *   LAPATTN_SOLVER_NEWTON_SCHULZ  Y = X_iters W, X_iters from the forward's
 *                                 solver (same arithmetic)
 *   LAPATTN_SOLVER_CG             `iters` steps of conjugate gradient
 *                                 (Hestenes-Stiefel) on A y = w for every
 *                                 column w of W, from y = 0, fp32
 *   landmarks  device, fp32 [B, H, m, d] (the pool of lapattn_forward_stages)
 *   w          device, fp32 [B, H, m, d]
 *   y          device, fp32 [B, H, m, d], written
 * One launch, one workgroup per head, no workspace; errors as for
 * lapattn_forward (LAPATTN_ERR_PARAM for an unknown solver). */
#define LAPATTN_SOLVER_NEWTON_SCHULZ 0
#define LAPATTN_SOLVER_CG 1
int lapattn_landmark_solve(const lapattn_desc_t* desc, const float* landmarks,
                           const float* w, float lambda, float eps, int32_t iters,
                           int32_t solver, float* y, void* stream);

/* One attention block around the Nystrom attention, on the tokens of one
 * stage of a pyramid backbone (the SOFT review instantiates SOFT as one
 * layer of such a backbone, "proposed method", last bullet; its symmetric
 * kernel S = exp(Q (-) K) shares the query and key projection):
 *   Q = X Wq, K = X Wk (wk == NULL: K = Q), V = X Wv, each split into the
 *   desc->H heads of desc->d columns (columns h d .. h d + d - 1 are head h),
 *   O_h = lapattn_forward(Q_h, K_h, V_h), Y = concat_h(O_h) Wo.
 *   x        device, [B, N, C] (N = grid_h grid_w, tokens in raster order)
 *   wq, wk, wv  device, [C, H d] row-major, no bias
 *   wo       device, [H d, C] row-major
 *   y        device, [B, N, C]
 * All in desc->dtype; Q, K, V and O are stored in that type in the
 * workspace (rounded to nearest even for bf16); every product accumulates in
 * fp32 (the projections on fp32 MFMA).  C and H d must be multiples of 32
 * (LAPATTN_ERR_SHAPE).  The workspace (lapattn_block_workspace_bytes,
 * 256-byte aligned) starts with the call's status word (uint32 at offset 0,
 * as lapattn_status_offset describes for lapattn_forward).  Three or four
 * launches on `stream`; errors as for lapattn_forward. */
size_t lapattn_block_workspace_bytes(const lapattn_desc_t* desc, int32_t C);
int lapattn_block_forward(const lapattn_desc_t* desc, int32_t C, const void* x,
                          const void* wq, const void* wk, const void* wv,
                          const void* wo, float lambda, float eps, int32_t iters,
                          void* y, void* workspace, size_t workspace_bytes,
                          void* stream);

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * forward as lapattn_forward (same arguments, plan, kernels and bitwise
 * result), with the workspace taken from a static device array of
 * LAPATTN_NOALLOC_SCRATCH_BYTES (128 MiB) that the library holds on each
 * device it runs on until the process ends.  The call allocates and frees
 * nothing; its first call on a device (or lapattn_init with that device
 * current) looks the array's device address up once.
 *   status  device pointer to a uint32 (4-byte aligned) that the call sets
 *           to its count of timed-out in-launch waits (nonzero: the output
 *           is invalid); NULL: not reported
 * Returns LAPATTN_ERR_SCRATCH when lapattn_workspace_bytes(desc) exceeds the
 * scratch (nothing is enqueued), else what lapattn_forward returns.  Every
 * call on a device shares that device's scratch, which keeps the last call's
 * contents: calls that overlap on one device (other streams, other host
 * threads) race and must be serialised by the caller. */
int lapattn_forward_noalloc(const lapattn_desc_t* desc, const void* q,
                            const void* k, const void* v, float lambda,
                            float eps, int32_t iters, void* out,
                            uint32_t* status, void* stream);

/* lapattn_forward plus device copies of every intermediate, for stage-wise
 * checking.  Each stage pointer may be NULL (not written).  All fp32:
 *   L   [B, H, m, d]   landmarks
 *   kql [B, H, N, m]   k(Q, L)
 *   klk [B, H, m, N]   k(L, K)
 *   a   [B, H, m, m]   k(L, L) + eps I
 *   x   [B, H, m, m]   Newton-Schulz result after `iters` steps
 *   w   [B, H, m, d]   K_LK V */
int lapattn_forward_stages(const lapattn_desc_t* desc, const void* q,
                           const void* k, const void* v, float lambda,
                           float eps, int32_t iters, void* out,
                           void* workspace, size_t workspace_bytes,
                           void* stream, float* L, float* kql, float* klk,
                           float* a, float* x, float* w);

/* Launch slots (bit s for LAPATTN_STAGE_s) that a forward call with this
 * descriptor enqueues; q_is_k says whether k will be the same pointer as q.
 * Host-only, no GPU work.  Returns a negative error code for a bad desc. */
int lapattn_launches(const lapattn_desc_t* desc, int q_is_k);

/* Profiling hook.  For the calling host thread, makes every later forward
 * call launch the kernel of slot s (LAPATTN_STAGE_*) through
 * hipExtLaunchKernel with events[2*s] and events[2*s+1] as its start and stop
 * events: hipEventElapsedTime(events[2*s], events[2*s+1]) is then that
 * kernel's own execution time.  Slots without a launch in the call are left
 * unrecorded: LAPATTN_STAGE_MAPS outside LAPATTN_FLAG_SERIAL, and
 * LAPATTN_STAGE_OUT unless K is the same pointer as Q or the main grid cannot
 * be resident at once (lapattn_launches tells which slots a call uses); a
 * backward call records slot 0 and the LAPATTN_STAGE_BWD_* slots.
 * `events` holds 2 * LAPATTN_NUM_STAGES hipEvent_t handles (as void*) created
 * by the caller with timing enabled, and must stay valid until the hook is
 * cleared with (NULL, 0).  n must be 0 or 2 * LAPATTN_NUM_STAGES. */
int lapattn_set_stage_events(void* const* events, int n);

#ifdef __cplusplus
}
#endif

#endif /* LAPATTN_H */
