// C-ABI front end: argument validation, workspace plan, launch sequence.
// The entry points are declared (with their contracts) in include/lapattn.h.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>

#include "lapattn.h"
#include "lapattn_internal.h"

namespace lapattn {
namespace {

constexpr size_t kAlign = 256;

// Workspace of lapattn_forward_noalloc: a static device array that each
// device the library runs on holds until the process ends.  In host code its
// name is a host-side stand-in, never a device address: kernels and copies
// get the per-device address that hipGetSymbolAddress returns (scratch_ptr).
static __device__ __align__(256) unsigned char scratch[LAPATTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];

// Device address of `scratch` on the current device, looked up once per
// device (lapattn_init, or the first no-alloc call on the device); null with
// *err set when no device is current or the lookup fails.
void* scratch_ptr(int* err) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    *err = LAPATTN_ERR_HIP;
    return nullptr;
  }
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
    (void)hipGetLastError();
    *err = LAPATTN_ERR_HIP;
    return nullptr;
  }
  g_scratch[dev].store(p, std::memory_order_release);
  return p;
}

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int check_desc(const lapattn_desc_t* d) {
  if (!d) return LAPATTN_ERR_NULL;
  if (d->B <= 0 || d->H <= 0 || d->grid_h <= 0 || d->grid_w <= 0 || d->d <= 0 ||
      d->pool_h <= 0 || d->pool_w <= 0)
    return LAPATTN_ERR_SHAPE;
  if (d->d != 16 && d->d != 32 && d->d != 64) return LAPATTN_ERR_SHAPE;
  if (d->grid_h % d->pool_h || d->grid_w % d->pool_w) return LAPATTN_ERR_SHAPE;
  const long long N = static_cast<long long>(d->grid_h) * d->grid_w;
  const long long BH = static_cast<long long>(d->B) * d->H;
  // Index arithmetic inside the kernels is 32-bit per head and per launch.
  if (N > (1LL << 24) || BH > (1LL << 20) || BH * ((N + 63) / 64) * 16 > (1LL << 31))
    return LAPATTN_ERR_SHAPE;
  const long long m = static_cast<long long>(d->grid_h / d->pool_h) * (d->grid_w / d->pool_w);
  if (m > LAPATTN_MAX_LANDMARKS) return LAPATTN_ERR_M_TOO_LARGE;
  if (d->kernel != LAPATTN_KERNEL_LAPLACIAN && d->kernel != LAPATTN_KERNEL_GAUSSIAN)
    return LAPATTN_ERR_PARAM;
  if (d->dtype != LAPATTN_F32 && d->dtype != LAPATTN_BF16) return LAPATTN_ERR_DTYPE;
  if (d->flags & ~(LAPATTN_FLAG_SERIAL | LAPATTN_FLAG_TICKETS)) return LAPATTN_ERR_PARAM;
  return LAPATTN_OK;
}

int check_params(float lambda, float eps, int32_t iters) {
  if (!std::isfinite(lambda) || !(lambda > 0.f)) return LAPATTN_ERR_PARAM;
  if (!std::isfinite(eps) || eps < 0.f) return LAPATTN_ERR_PARAM;
  if (iters < 0 || iters > LAPATTN_MAX_ITERS) return LAPATTN_ERR_PARAM;
  return LAPATTN_OK;
}

// Compute units of the current device, cached per device; 256 (MI355X) when
// no device can be queried (host-only use such as sizing the workspace).
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return 256;
  }
  int cus = cache[dev].load(std::memory_order_relaxed);
  if (cus > 0) return cus;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0) {
    (void)hipGetLastError();
    return 256;
  }
  cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

Plan make_plan(const lapattn_desc_t* d) {
  Plan p{};
  p.B = d->B;
  p.H = d->H;
  p.gh = d->grid_h;
  p.gw = d->grid_w;
  p.D = d->d;
  p.ph = d->pool_h;
  p.pw = d->pool_w;
  p.kernel = d->kernel;
  p.bf16 = d->dtype == LAPATTN_BF16;
  p.N = p.gh * p.gw;
  p.m = (p.gh / p.ph) * (p.gw / p.pw);
  p.BH = p.B * p.H;
  p.mpad = 16 * ((p.m + 15) / 16);
  // Solver: the matrix zero padded up to whole 16x16 blocks.
  p.ns_mb = (p.m + 15) / 16;
  p.nT = (p.N + 63) / 64;
  // Key-side workgroups cover S tiles each.  At most 32 W partials per head
  // when the last key workgroup reduces them alone (output-launch plan).
  // When the whole grid can be resident at once (the query workgroups then
  // reduce the partials in slices), the fewest tiles per key workgroup that
  // keep it resident, up to 128 partials per head; the plan assumes separate
  // Q and K (query workgroups present), which only sizes the workspace
  // larger when they are the same tensor.
  p.resident = kResidentPerCU * device_cus() - kResidentMargin;
  p.S = (p.nT + 31) / 32;
  {
    const long nQ = (p.nT + kQueryTiles - 1) / kQueryTiles;
    for (int S = 1; S < p.S; ++S) {
      const long nP = (p.nT + S - 1) / S;
      if (nP <= kMaxPartials && static_cast<long>(p.BH) * (1 + nP + nQ) <= p.resident) {
        p.S = S;
        break;
      }
    }
    // A resident grid takes at least kMinKeyTiles tiles per key workgroup:
    // fewer partials to write and read back, and fewer workgroups beside
    // the solvers (8 heads of 3136 tokens: 3 tiles instead of 2 cut the
    // launch's HBM traffic by 2.3 MB and its time by 0.15 us; 4 tiles were
    // 2 us slower).
    const long nPm = (p.nT + kMinKeyTiles - 1) / kMinKeyTiles;
    if (p.S < kMinKeyTiles && static_cast<long>(p.BH) * (1 + nPm + nQ) <= p.resident)
      p.S = kMinKeyTiles;
  }
  // A grid that cannot be resident at once runs in rounds of workgroups
  // (output-launch plan), each workgroup paying its fixed latency (set-up,
  // first loads) once.  When up to 4 tiles per key workgroup let the key
  // workgroups and the solvers all be resident at once (one round, as for
  // Q == K, which has no query workgroups), take the fewest such tiles;
  // otherwise the rounds are unavoidable and short workgroups balance best.
  {
    const long nQ = (p.nT + kQueryTiles - 1) / kQueryTiles;
    const long nP = (p.nT + p.S - 1) / p.S;
    p.qt = kQueryTiles;
    if (static_cast<long>(p.BH) * (1 + nP + nQ) > p.resident) {
      bool one_round = false;
      for (int S = p.S + 1; S <= kMaxKeyTilesOut; ++S) {
        const long nPS = (p.nT + S - 1) / S;
        if (static_cast<long>(p.BH) * (1 + nPS) <= p.resident) {
          p.S = S;
          one_round = true;
          break;
        }
      }
      // Rounds either way: 2 key tiles and 4 query tiles per workgroup
      // amortise each workgroup's fixed latency and still balance (160 heads
      // of 784 bf16 tokens: main launch 104 -> 91 us; 1 / 2, 3 / 2, 7 / 7
      // and 13 / 13 tiles were slower)
      if (!one_round) p.S = p.S > 2 ? p.S : 2;
      p.qt = kQueryTilesOut;
    }
  }
  p.nP = (p.nT + p.S - 1) / p.S;

  const size_t BH = static_cast<size_t>(p.BH);
  const size_t f = sizeof(float);
  size_t off = 0;
  p.off_L = off;
  off = align_up(off + BH * p.m * p.D * f);
  p.off_kql = off;
  off = align_up(off + BH * p.N * p.mpad * f);
  p.off_wpart = off;
  off = align_up(off + BH * p.nP * p.D * MP * f);
  p.off_x = off;
  off = align_up(off + BH * MP * MP * f);
  p.off_wt = off;
  off = align_up(off + BH * p.D * MP * f);
  p.off_yt = off;
  off = align_up(off + BH * p.D * MP * f);
  p.off_mu = off;
  off = align_up(off + BH * MP * f);
  p.off_sync = off;
  off = align_up(off + kSyncHead * (BH + 1) * sizeof(unsigned));
  p.total = off;
  return p;
}

// Backward pass: tiles per workgroup of the partial launch so that each head
// has at most 64 partials per side, and at least kMinKeyTiles (fewer
// partials for the head reduction: 8 heads of 3136 tokens, 17 instead of 49
// per side, head launch 10.5 -> 9.3 us); every buffer 256-byte aligned.
BwdPlan make_bwd_plan(const lapattn_desc_t* d, int32_t iters) {
  BwdPlan p{};
  p.B = d->B;
  p.H = d->H;
  p.gh = d->grid_h;
  p.gw = d->grid_w;
  p.D = d->d;
  p.ph = d->pool_h;
  p.pw = d->pool_w;
  p.kernel = d->kernel;
  p.bf16 = d->dtype == LAPATTN_BF16;
  p.N = p.gh * p.gw;
  p.m = (p.gh / p.ph) * (p.gw / p.pw);
  p.BH = p.B * p.H;
  p.ns_mb = (p.m + 15) / 16;
  p.nT = (p.N + 63) / 64;
  p.S = (p.nT + 63) / 64;
  if (p.S < kMinKeyTiles) p.S = kMinKeyTiles;
  p.nP = (p.nT + p.S - 1) / p.S;
  p.iters = iters < 0 ? 0 : iters;
  const size_t BH = static_cast<size_t>(p.BH), f = sizeof(float);
  size_t off = 0;
  p.off_L = off;
  off = align_up(off + BH * p.m * p.D * f);
  p.off_xiter = off;
  off = align_up(off + BH * (p.iters + 1) * MP * MP * f);
  p.off_amat = off;
  off = align_up(off + BH * MP * MP * f);
  p.off_hscal = off;
  off = align_up(off + BH * 4 * f);
  p.off_wpart = off;
  off = align_up(off + BH * p.nP * p.D * MP * f);
  p.off_dypart = off;
  off = align_up(off + BH * p.nP * p.D * MP * f);
  p.off_ymat = off;
  off = align_up(off + BH * MP * p.D * f);
  p.off_dwmat = off;
  off = align_up(off + BH * MP * p.D * f);
  p.off_dxmat = off;
  off = align_up(off + BH * MP * MP * f);
  p.off_dlpart = off;
  off = align_up(off + BH * 2 * p.nT * MP * p.D * f);
  p.off_dkd = off;
  off = align_up(off + BH * p.N * p.D * f);
  p.off_sync = off;
  off = align_up(off + kSyncHead * (BH + 1) * sizeof(unsigned));
  p.total = off;
  return p;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// Per-thread stage events (profiling hook).
thread_local void* const* t_events = nullptr;

// Events of one launch slot, or none when the hook is not set.
inline Ev slot(int st) {
  if (!t_events) return {};
  return {static_cast<hipEvent_t>(t_events[2 * st]), static_cast<hipEvent_t>(t_events[2 * st + 1])};
}

bool misaligned16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 != 0; }

int run(const lapattn_desc_t* desc, const Args& args, void* workspace, size_t ws_bytes,
        hipStream_t stream) {
  const Plan p = make_plan(desc);
  Args a = args;
  // the normalised map needs every query's K_QL before any output row: it
  // always takes the output-launch plan
  a.out_in_main = (!a.normalized && out_in_main_launch(p, a.shared_qk)) ? 1 : 0;
  if (misaligned16(a.q) || misaligned16(a.k) || misaligned16(a.v) || misaligned16(a.out))
    return LAPATTN_ERR_ALIGN;
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign) return LAPATTN_ERR_WORKSPACE;
  if (ws_bytes < p.total) return LAPATTN_ERR_WORKSPACE;
  const size_t esize = p.bf16 ? 2 : 4;
  const size_t io = static_cast<size_t>(p.BH) * p.N * p.D * esize;
  if (overlaps(a.out, io, a.q, io) || overlaps(a.out, io, a.k, io) ||
      overlaps(a.out, io, a.v, io) || overlaps(a.out, io, workspace, ws_bytes))
    return LAPATTN_ERR_ALIAS;
  if (a.status && (reinterpret_cast<uintptr_t>(a.status) % 4 ||
                   overlaps(a.status, 4, a.out, io) || overlaps(a.status, 4, a.q, io) ||
                   overlaps(a.status, 4, a.k, io) || overlaps(a.status, 4, a.v, io) ||
                   overlaps(a.status, 4, workspace, ws_bytes)))
    return LAPATTN_ERR_ALIAS;

  char* ws = static_cast<char*>(workspace);
  Buffers b;
  b.L = reinterpret_cast<float*>(ws + p.off_L);
  b.kql = reinterpret_cast<float*>(ws + p.off_kql);
  b.wpart = reinterpret_cast<float*>(ws + p.off_wpart);
  b.x = reinterpret_cast<float*>(ws + p.off_x);
  b.wt = reinterpret_cast<float*>(ws + p.off_wt);
  b.yt = reinterpret_cast<float*>(ws + p.off_yt);
  b.mu = reinterpret_cast<float*>(ws + p.off_mu);
  b.sync = reinterpret_cast<unsigned*>(ws + p.off_sync);
  b.timeouts = a.status ? a.status : b.sync;

  if (launch_pool(p, a, b, stream, slot(LAPATTN_STAGE_POOL)) != hipSuccess) return LAPATTN_ERR_HIP;
  if (desc->flags & LAPATTN_FLAG_SERIAL) {
    if (launch_main(p, a, b, true, false, stream, slot(LAPATTN_STAGE_MAIN)) != hipSuccess ||
        launch_main(p, a, b, false, true, stream, slot(LAPATTN_STAGE_MAPS)) != hipSuccess)
      return LAPATTN_ERR_HIP;
  } else {
    // one launch carries both roles; the MAPS slot is left untouched
    if (launch_main(p, a, b, true, true, stream, slot(LAPATTN_STAGE_MAIN)) != hipSuccess)
      return LAPATTN_ERR_HIP;
  }
  // W = K_LK V, Y = X W and (when Q != K) the output rows are formed inside the
  // main launch; with Q == K there are no query workgroups and the output
  // product runs as its own launch.
  if (a.normalized && launch_norm_stats(p, a, b, stream) != hipSuccess) return LAPATTN_ERR_HIP;
  if (!a.out_in_main && launch_out(p, a, b, stream, slot(LAPATTN_STAGE_OUT)) != hipSuccess)
    return LAPATTN_ERR_HIP;
  return LAPATTN_OK;
}

int forward_common(const lapattn_desc_t* desc, const void* q, const void* k, const void* v,
                   float lambda, float eps, int32_t iters, void* out, void* workspace,
                   size_t workspace_bytes, void* stream, float* L, float* kql, float* klk,
                   float* am, float* x, float* w, unsigned* status = nullptr) {
  int st = check_desc(desc);
  if (st != LAPATTN_OK) return st;
  st = check_params(lambda, eps, iters);
  if (st != LAPATTN_OK) return st;
  if (!q || !k || !v || !out || !workspace) return LAPATTN_ERR_NULL;
  Args a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.lambda = lambda;
  a.eps = eps;
  a.iters = iters;
  a.shared_qk = (q == k) ? 1 : 0;
  a.st_L = L;
  a.st_kql = kql;
  a.st_klk = klk;
  a.st_a = am;
  a.st_x = x;
  a.st_w = w;
  a.status = status;
  a.tickets = (desc->flags & LAPATTN_FLAG_TICKETS) ? 1 : 0;
  return run(desc, a, workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

}  // namespace
}  // namespace lapattn

extern "C" {

int lapattn_version(void) { return LAPATTN_VERSION; }

const char* lapattn_strerror(int status) {
  switch (status) {
    case LAPATTN_OK: return "ok";
    case LAPATTN_ERR_NULL: return "a required pointer is NULL";
    case LAPATTN_ERR_SHAPE:
      return "invalid shape: non-positive size, grid not divisible by pool, or head dim not in {16, 32, 64}";
    case LAPATTN_ERR_M_TOO_LARGE: return "more than 64 landmarks";
    case LAPATTN_ERR_PARAM: return "invalid parameter: lambda, eps, iters, kernel or flags";
    case LAPATTN_ERR_DTYPE: return "unknown dtype";
    case LAPATTN_ERR_ALIAS: return "output overlaps an input or the workspace";
    case LAPATTN_ERR_WORKSPACE: return "workspace too small or not 256-byte aligned";
    case LAPATTN_ERR_HIP: return "HIP runtime or kernel launch failure";
    case LAPATTN_ERR_ALIGN: return "q, k, v or out is not 16-byte aligned";
    case LAPATTN_ERR_SCRATCH:
      return "the call needs more workspace than the no-alloc entry point's static scratch holds";
  }
  return "unknown status";
}

int lapattn_check(const lapattn_desc_t* desc, float lambda, float eps, int32_t iters) {
  const int st = lapattn::check_desc(desc);
  if (st != LAPATTN_OK) return st;
  return lapattn::check_params(lambda, eps, iters);
}

size_t lapattn_workspace_bytes(const lapattn_desc_t* desc) {
  if (lapattn::check_desc(desc) != LAPATTN_OK) return 0;
  return lapattn::make_plan(desc).total;
}

size_t lapattn_backward_workspace_bytes(const lapattn_desc_t* desc, int32_t iters) {
  if (lapattn::check_desc(desc) != LAPATTN_OK) return 0;
  if (iters < 0 || iters > LAPATTN_MAX_ITERS) return 0;
  return lapattn::make_bwd_plan(desc, iters).total;
}

int lapattn_backward(const lapattn_desc_t* desc, const void* q, const void* k, const void* v,
                     const void* dout, float lambda, float eps, int32_t iters, void* dq, void* dk,
                     void* dv, void* workspace, size_t workspace_bytes, void* stream) {
  using namespace lapattn;
  int st = check_desc(desc);
  if (st != LAPATTN_OK) return st;
  st = check_params(lambda, eps, iters);
  if (st != LAPATTN_OK) return st;
  if (!q || !k || !v || !dout || !dq || !dk || !dv || !workspace) return LAPATTN_ERR_NULL;
  const BwdPlan p = make_bwd_plan(desc, iters);
  if (misaligned16(q) || misaligned16(k) || misaligned16(v) || misaligned16(dout) ||
      misaligned16(dq) || misaligned16(dk) || misaligned16(dv))
    return LAPATTN_ERR_ALIGN;
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign || workspace_bytes < p.total)
    return LAPATTN_ERR_WORKSPACE;
  const size_t io = static_cast<size_t>(p.BH) * p.N * p.D * (p.bf16 ? 2 : 4);
  const void* ins[4] = {q, k, v, dout};
  void* outs[3] = {dq, dk, dv};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 4; ++j)
      if (overlaps(outs[i], io, ins[j], io)) return LAPATTN_ERR_ALIAS;
    for (int j = i + 1; j < 3; ++j)
      if (overlaps(outs[i], io, outs[j], io)) return LAPATTN_ERR_ALIAS;
    if (overlaps(outs[i], io, workspace, workspace_bytes)) return LAPATTN_ERR_ALIAS;
  }
  BwdCall c{};
  c.q = q;
  c.k = k;
  c.v = v;
  c.dout = dout;
  c.dq = dq;
  c.dk = dk;
  c.dv = dv;
  c.workspace = workspace;
  c.lambda = lambda;
  c.eps = eps;
  c.iters = iters;
  c.ev[0] = slot(LAPATTN_STAGE_POOL);
  c.ev[1] = slot(LAPATTN_STAGE_BWD_PART);
  c.ev[2] = slot(LAPATTN_STAGE_BWD_HEAD);
  c.ev[3] = slot(LAPATTN_STAGE_BWD_GRAD);
  c.ev[4] = slot(LAPATTN_STAGE_BWD_DK);
  if (launch_backward(p, c, static_cast<hipStream_t>(stream)) != hipSuccess) return LAPATTN_ERR_HIP;
  return LAPATTN_OK;
}

int lapattn_landmark_solve(const lapattn_desc_t* desc, const float* landmarks, const float* w,
                           float lambda, float eps, int32_t iters, int32_t solver, float* y,
                           void* stream) {
  using namespace lapattn;
  int st = check_desc(desc);
  if (st != LAPATTN_OK) return st;
  st = check_params(lambda, eps, iters);
  if (st != LAPATTN_OK) return st;
  if (solver != LAPATTN_SOLVER_NEWTON_SCHULZ && solver != LAPATTN_SOLVER_CG) return LAPATTN_ERR_PARAM;
  if (!landmarks || !w || !y) return LAPATTN_ERR_NULL;
  if (misaligned16(landmarks) || misaligned16(w) || misaligned16(y)) return LAPATTN_ERR_ALIGN;
  const Plan p = make_plan(desc);
  const size_t n = static_cast<size_t>(p.BH) * p.m * p.D * sizeof(float);
  if (overlaps(y, n, landmarks, n) || overlaps(y, n, w, n)) return LAPATTN_ERR_ALIAS;
  if (launch_landmark_solve(p, landmarks, w, lambda, eps, iters, solver, y,
                            static_cast<hipStream_t>(stream)) != hipSuccess)
    return LAPATTN_ERR_HIP;
  return LAPATTN_OK;
}

// Block workspace: the status word (256 bytes), Q, K, V, O in the heads'
// layout and I/O type, then the attention's workspace.
namespace lapattn {
namespace {
int check_block(const lapattn_desc_t* desc, int32_t C) {
  const int st = check_desc(desc);
  if (st != LAPATTN_OK) return st;
  if (C <= 0 || C % 32 || (desc->H * desc->d) % 32) return LAPATTN_ERR_SHAPE;
  return LAPATTN_OK;
}
size_t block_io_bytes(const lapattn_desc_t* d) {
  return align_up(static_cast<size_t>(d->B) * d->H * d->grid_h * d->grid_w * d->d *
                  (d->dtype == LAPATTN_BF16 ? 2 : 4));
}
}  // namespace
}  // namespace lapattn

size_t lapattn_block_workspace_bytes(const lapattn_desc_t* desc, int32_t C) {
  if (lapattn::check_block(desc, C) != LAPATTN_OK) return 0;
  return lapattn::kAlign + 4 * lapattn::block_io_bytes(desc) + lapattn::make_plan(desc).total;
}

int lapattn_block_forward(const lapattn_desc_t* desc, int32_t C, const void* x, const void* wq,
                          const void* wk, const void* wv, const void* wo, float lambda, float eps,
                          int32_t iters, void* y, void* workspace, size_t workspace_bytes,
                          void* stream) {
  using namespace lapattn;
  int st = check_block(desc, C);
  if (st != LAPATTN_OK) return st;
  st = check_params(lambda, eps, iters);
  if (st != LAPATTN_OK) return st;
  if (!x || !wq || !wv || !wo || !y || !workspace) return LAPATTN_ERR_NULL;
  if (misaligned16(x) || misaligned16(wq) || (wk && misaligned16(wk)) || misaligned16(wv) ||
      misaligned16(wo) || misaligned16(y))
    return LAPATTN_ERR_ALIGN;
  const Plan p = make_plan(desc);
  const size_t io = block_io_bytes(desc);
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign ||
      workspace_bytes < kAlign + 4 * io + p.total)
    return LAPATTN_ERR_WORKSPACE;
  const size_t es = p.bf16 ? 2 : 4;
  const size_t xb = static_cast<size_t>(p.B) * p.N * C * es;
  const size_t wb = static_cast<size_t>(C) * p.H * p.D * es;
  if (overlaps(y, xb, x, xb) || overlaps(y, xb, wq, wb) || (wk && overlaps(y, xb, wk, wb)) ||
      overlaps(y, xb, wv, wb) || overlaps(y, xb, wo, wb) || overlaps(y, xb, workspace, workspace_bytes))
    return LAPATTN_ERR_ALIAS;
  char* ws = static_cast<char*>(workspace);
  unsigned* status = reinterpret_cast<unsigned*>(ws);
  void* Q = ws + kAlign;
  void* K = ws + kAlign + io;
  void* V = ws + kAlign + 2 * io;
  void* O = ws + kAlign + 3 * io;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int M = p.B * p.N, HD = p.H * p.D;
  // Q (and K unless shared) and V, one launch
  {
    const void* w3[3] = {wq, wk ? wk : wv, wv};
    void* o3[3] = {Q, wk ? K : V, V};
    if (launch_block_proj(0, x, w3, o3, wk ? 3 : 2, M, C, HD, p.N, p.H, p.D, p.bf16, s) != hipSuccess)
      return LAPATTN_ERR_HIP;
  }
  Args a{};
  a.q = Q;
  a.k = wk ? K : Q;
  a.v = V;
  a.out = O;
  a.lambda = lambda;
  a.eps = eps;
  a.iters = iters;
  a.shared_qk = wk ? 0 : 1;
  a.status = status;
  a.tickets = (desc->flags & LAPATTN_FLAG_TICKETS) ? 1 : 0;
  st = run(desc, a, ws + kAlign + 4 * io, p.total, s);
  if (st != LAPATTN_OK) return st;
  {
    const void* w1[1] = {wo};
    void* o1[1] = {y};
    if (launch_block_proj(1, O, w1, o1, 1, M, HD, C, p.N, p.H, p.D, p.bf16, s) != hipSuccess)
      return LAPATTN_ERR_HIP;
  }
  return LAPATTN_OK;
}

size_t lapattn_status_offset(const lapattn_desc_t* desc) {
  if (lapattn::check_desc(desc) != LAPATTN_OK) return static_cast<size_t>(-1);
  // word 0 of the hand-off words: timed-out waits of the call
  return lapattn::make_plan(desc).off_sync;
}

int lapattn_launches(const lapattn_desc_t* desc, int q_is_k) {
  const int st = lapattn::check_desc(desc);
  if (st != LAPATTN_OK) return st;
  const lapattn::Plan p = lapattn::make_plan(desc);
  int mask = (1 << LAPATTN_STAGE_POOL) | (1 << LAPATTN_STAGE_MAIN);
  if (desc->flags & LAPATTN_FLAG_SERIAL) mask |= 1 << LAPATTN_STAGE_MAPS;
  if (!lapattn::out_in_main_launch(p, q_is_k ? 1 : 0)) mask |= 1 << LAPATTN_STAGE_OUT;
  return mask;
}

int lapattn_set_stage_events(void* const* events, int n) {
  if (n != 0 && n != 2 * LAPATTN_NUM_STAGES) return LAPATTN_ERR_PARAM;
  if (n != 0 && !events) return LAPATTN_ERR_NULL;
  lapattn::t_events = n ? events : nullptr;
  return LAPATTN_OK;
}

int lapattn_init(void) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return LAPATTN_ERR_HIP;
  (void)lapattn::device_cus();
  int err = LAPATTN_OK;
  if (!lapattn::scratch_ptr(&err)) return err;
  return LAPATTN_OK;
}

int lapattn_forward(const lapattn_desc_t* desc, const void* q, const void* k, const void* v,
                    float lambda, float eps, int32_t iters, void* out, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return lapattn::forward_common(desc, q, k, v, lambda, eps, iters, out, workspace,
                                 workspace_bytes, stream, nullptr, nullptr, nullptr, nullptr,
                                 nullptr, nullptr);
}

int lapattn_forward_normalized(const lapattn_desc_t* desc, const void* q, const void* k,
                               const void* v, float lambda, float eps, int32_t iters, float delta,
                               void* out, void* workspace, size_t workspace_bytes, void* stream) {
  using namespace lapattn;
  int st = check_desc(desc);
  if (st != LAPATTN_OK) return st;
  st = check_params(lambda, eps, iters);
  if (st != LAPATTN_OK) return st;
  if (!std::isfinite(delta) || delta < 0.f) return LAPATTN_ERR_PARAM;
  if (!q || !k || !v || !out || !workspace) return LAPATTN_ERR_NULL;
  Args a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.lambda = lambda;
  a.eps = eps;
  a.iters = iters;
  a.shared_qk = (q == k) ? 1 : 0;
  a.tickets = (desc->flags & LAPATTN_FLAG_TICKETS) ? 1 : 0;
  a.normalized = 1;
  a.delta = delta;
  return run(desc, a, workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

int lapattn_forward_noalloc(const lapattn_desc_t* desc, const void* q, const void* k,
                            const void* v, float lambda, float eps, int32_t iters, void* out,
                            uint32_t* status, void* stream) {
  // every argument check first: nothing is looked up or enqueued on an error
  int st = lapattn::check_desc(desc);
  if (st != LAPATTN_OK) return st;
  st = lapattn::check_params(lambda, eps, iters);
  if (st != LAPATTN_OK) return st;
  if (!q || !k || !v || !out) return LAPATTN_ERR_NULL;
  if (lapattn::make_plan(desc).total > LAPATTN_NOALLOC_SCRATCH_BYTES) return LAPATTN_ERR_SCRATCH;
  int err = LAPATTN_OK;
  void* ws = lapattn::scratch_ptr(&err);
  if (!ws) return err;
  return lapattn::forward_common(desc, q, k, v, lambda, eps, iters, out, ws,
                                 LAPATTN_NOALLOC_SCRATCH_BYTES, stream, nullptr, nullptr,
                                 nullptr, nullptr, nullptr, nullptr, status);
}

int lapattn_forward_stages(const lapattn_desc_t* desc, const void* q, const void* k,
                           const void* v, float lambda, float eps, int32_t iters, void* out,
                           void* workspace, size_t workspace_bytes, void* stream, float* L,
                           float* kql, float* klk, float* a, float* x, float* w) {
  return lapattn::forward_common(desc, q, k, v, lambda, eps, iters, out, workspace,
                                 workspace_bytes, stream, L, kql, klk, a, x, w);
}

}  // extern "C"
