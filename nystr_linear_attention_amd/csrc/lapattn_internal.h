// Internal launch plan shared by the C-ABI front end and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lapattn {

// Small per-head matrices (A, X, W^T, Y^T) are stored padded to MP columns;
// padding holds exact zeros.
constexpr int MP = 64;
// Hand-off words per head (and once more for the words of the whole call).
constexpr int kSyncHead = 256;
// 64-token tiles per query workgroup when it forms its output rows in the
// main launch (their K_QL rows stay in LDS).
constexpr int kQueryTiles = 2;
// Query tiles per workgroup when the grid cannot be resident at once (the
// output-launch plan stores K_QL, so a workgroup can take more tiles).
constexpr int kQueryTilesOut = 4;
// Tiles per key workgroup at most when the output-launch plan lengthens key
// workgroups so that they are all resident at once.
constexpr int kMaxKeyTilesOut = 4;
// least tiles per key workgroup when the whole grid is resident
constexpr int kMinKeyTiles = 3;
// W partials per head at most (key ready flags per head).
constexpr int kMaxPartials = 128;
// Main-kernel workgroups taken to be resident at once: two per CU (LDS and
// registers allow two) less a margin of 64; 448 on a 256-CU MI355X.  This
// only chooses the faster plan: no plan depends on the whole grid being
// resident for its hand-offs (see take_role in the kernels).
constexpr long kResidentPerCU = 2;
constexpr long kResidentMargin = 64;

struct Plan {
  int B, H, gh, gw, D, ph, pw;
  int kernel;   // 0 Laplacian, 1 Gaussian
  int bf16;     // 0 fp32 I/O, 1 bf16 I/O
  int N, m, BH;
  int mpad;     // 16 * ceil(m / 16): row length of the stored K_QL
  int ns_mb;    // 16x16 MFMA blocks per side in the solver interior
  int nT;       // 64-token tiles per head
  int S;        // tiles per key-side workgroup
  int qt;       // tiles per query workgroup when K_QL is stored (output-launch
                // plan); the main launch's output rows take kQueryTiles
  int nP;       // key-side workgroups (= W partials) per head
  long resident;  // main-kernel workgroups resident at once on the device
  // workspace byte offsets
  size_t off_L, off_kql, off_wpart, off_x, off_wt, off_yt, off_mu, off_sync;
  size_t total;
};

struct Buffers {
  float* L;      // [BH][m][D]     landmarks
  float* kql;    // [BH][N][mpad]  k(q_n, l_j), zero for j >= m
  float* wpart;  // [BH][nP][D][MP] partial W^T
  float* x;      // [BH][MP][MP]   Newton-Schulz result
  float* wt;     // [BH][D][MP]    W^T = (K_LK V)^T, zero for columns >= m
  float* yt;     // [BH][D][MP]    Y^T = (X W)^T
  float* mu;     // [BH][MP]       column means of K_QL (normalised map only)
  unsigned* sync;  // [kSyncHead (BH + 1)] hand-off words (see the main kernel)
  unsigned* timeouts;  // the call's count of timed-out waits (word 0 of sync,
                       // or a word the caller owns)
};

struct Args {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float lambda, eps;
  int iters;
  int shared_qk;
  int out_in_main;  // query workgroups form O inside the main launch
  unsigned* status;  // where the timeout count goes (null: word 0 of the
                     // workspace's hand-off words)
  int tickets;       // main-launch roles by ticket (LAPATTN_FLAG_TICKETS)
  int normalized;    // the normalised feature map in place of K_QL
  float delta;       // its whitening stabiliser
  // optional fp32 stage copies (may be null)
  float* st_L;
  float* st_kql;
  float* st_klk;
  float* st_a;
  float* st_x;
  float* st_w;
};

// Optional profiling events of one launch.  When set, the launch goes through
// hipExtLaunchKernel, which records the kernel's own start and end time into
// them (no extra packets on the stream).
struct Ev {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

// Stage launchers.  `with_solver` / `with_maps` select which workgroup roles
// the main launch carries: both (one fused launch), or one each in two
// launches.  launch_out forms O when the main launch does not (Q and K the
// same tensor, or a grid too large to be resident at once; see
// out_in_main_launch).
hipError_t launch_pool(const Plan& p, const Args& a, const Buffers& b, hipStream_t s, Ev ev);
hipError_t launch_main(const Plan& p, const Args& a, const Buffers& b, bool with_solver,
                       bool with_maps, hipStream_t s, Ev ev);
hipError_t launch_out(const Plan& p, const Args& a, const Buffers& b, hipStream_t s, Ev ev);
// Normalised feature map: per head, the column means mu and variances of the
// stored K_QL, and Y^T scaled in place by 1 / sqrt(var + delta) per column.
hipError_t launch_norm_stats(const Plan& p, const Args& a, const Buffers& b, hipStream_t s);

// Backward pass (lapattn_backward): launch plan and workspace layout.
struct BwdPlan {
  int B, H, gh, gw, D, ph, pw;
  int kernel, bf16;
  int N, m, BH;
  int ns_mb;  // 16x16 blocks per side of the padded Newton-Schulz matrix
  int nT;     // 64-token tiles per head
  int S;      // tiles per workgroup of the partial launch
  int nP;     // partials per head and side (= ceil(nT / S))
  int iters;
  size_t off_L, off_xiter, off_amat, off_hscal, off_wpart, off_dypart, off_ymat, off_dwmat,
      off_dxmat, off_dlpart, off_dkd, off_sync;
  size_t total;
};

struct BwdCall {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  void* workspace;
  float lambda, eps;
  int iters;
  Ev ev[5];  // profiling events of the pool, part, head, grad and dk launches
};

hipError_t launch_backward(const BwdPlan& p, const BwdCall& c, hipStream_t s);

// The landmark solve Y = A^{-1} W alone (lapattn_landmark_solve): Newton-
// Schulz (cg = 0) or conjugate gradient (cg = 1), one workgroup per head.
hipError_t launch_landmark_solve(const Plan& p, const float* L, const float* W, float lambda, float eps,
                                 int iters, int cg, float* Y, hipStream_t s);

// The block's projection GEMM: mode 0 = tokens [M][Kd] times nz weights
// [Kd][Nc] into the heads' [B][H][N][d] layouts; mode 1 = heads [B][H][N][d]
// gathered as rows of H d, times one weight [Kd][Nc] into [M][Nc].
hipError_t launch_block_proj(int mode, const void* a, const void* const* w, void* const* out, int nz, int M,
                             int Kd, int Nc, int N, int H, int d, int bf16, hipStream_t s);

// Whether query workgroups form O inside the main launch: only when there are
// query workgroups (Q != K) and every workgroup of the launch can be resident
// at once.  (Larger grids would be correct too, but query workgroups waiting
// for X would hold CUs that later heads' map workgroups could use; they
// store K_QL and an output launch forms O.)
bool out_in_main_launch(const Plan& p, int shared_qk);

}  // namespace lapattn
