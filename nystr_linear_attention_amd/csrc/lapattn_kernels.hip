// HIP kernels for Nystrom kernel attention (forward) on gfx950.
//
// Two launches per forward call (three when Q and K are the same tensor, or
// when the main grid cannot be resident at once), back to back on the
// caller's stream:
//   pool : landmarks L = window means of K (one or four landmarks per
//          workgroup)                                             (HBM stream)
//   main : role-split workgroups
//          - solver WGs (one per head, first in the grid, raised wave
//            priority): A = k(L, L) + eps I, alpha, then the Newton-Schulz
//            steps held in LDS on fp16 MFMA with scaled two-part operands
//          - map WGs: kernel values of 64 tokens against every landmark on
//            FP32 VALU (landmark coordinates are wave-uniform scalar operands);
//            key tiles contract K_LK V on fp32 MFMA into per-workgroup
//            partials of W^T; query tiles keep their K_QL rows in LDS
//          - hand-offs: query WGs reduce the partials in fixed-order slices,
//            copy W^T, wait for X from the solver, form Y = X W in LDS and
//            write O = K_QL Y (fp16 MFMA, scaled two-part operands); on the
//            output-launch plan the last key WG reduces and the second of
//            (W^T, X) forms Y^T for the output launch
//   out  : O = K_QL Y from K_QL stored by the map WGs, on fp16 MFMA with
//          scaled two-part operands (4 tiles per workgroup).
// Outputs are fp32 or bf16 (RNE).
//
// Pages behind each step: average-pool landmarks (SOFT review, "method";
// LaplacianFormer summaries, Nystrom paragraph), Laplacian kernel
// exp(-||x-y||_1/lambda) (LaplacianFormer summaries, kernel definition),
// Gaussian exp(Q (-) K) (SOFT review, "method"), eps I perturbation and the
// Newton-Schulz recursion A_0 = alpha A, A_{k+1} = 2 A_k - A_k A A_k
// (LaplacianFormer summaries; SOFT review, "method"), S_hat = P^T A^+ P
// (SOFT review, "method").
//
// Device code shared with the backward pass (solver and map roles, helpers)
// is in lapattn_device.h.

#include <algorithm>

#include "lapattn_device.h"

namespace lapattn {
namespace {

// ---------------------------------------------------------------------------
// Roles of the main launch.  Every wait inside the launch is on a producer of
// the same head: query workgroups wait for the key workgroups' W^T partials,
// for the W^T slices of the head's first R <= 32 query workgroups and for the
// solver's X.  Solvers and key workgroups never wait.
//
// Default (static roles, by workgroup index): the solvers come first, then
// the map units.  When 8 divides BH, workgroup index x (mod 8) -- which the
// dispatcher places round-robin on the 8 XCDs -- works through heads
// x, x + 8, ... in order, each head's key units before its query units: a
// head's workgroups share one XCD's L2 and scalar caches (landmarks, X, W^T)
// and every producer has a lower index than its consumers on the same XCD.
// Otherwise all key units precede all query units.  Either way, with each
// XCD dispatching its workgroups in index order, a consumer is dispatched
// only after every producer it waits for on its XCD, or (heads spread over
// XCDs) after every producer-class workgroup of that XCD, and producers run
// to completion without waiting; so no residency beyond the slice exchange
// (at most 32 workgroups of one head at once) is needed, whatever else runs
// on the device.
//
// LAPATTN_FLAG_TICKETS drops the dispatch-order assumption: roles are handed
// out by ticket, in the order in which workgroups start running.  The heads
// are split into queues (queue x: heads x, x + nq, ...), each with its own
// counter, and a queue's tickets run through its solvers, then per head its
// key units, then its query units, so every producer a workgroup waits for
// has already started.  The counters cost time: 50 to 215 workgroups take
// their tickets from one word at the start of the launch, and those read-
// modify-writes serialise at memory.  With 8 queues, queue x takes the
// workgroups with index = x (mod 8) (the same XCD placement as above);
// otherwise the queues take consecutive ranges of workgroup indices.
// Both give bitwise identical results: the arithmetic of a unit does not
// depend on which workgroup runs it.
// ---------------------------------------------------------------------------
struct Role {
  int kind;  // 0 solver, 1 key unit, 2 query unit
  int bh;    // head
  int u;     // unit index within the head (key: partial index; query: tile pair)
};

__device__ __forceinline__ Role static_role(const MainArgs& a, int b) {
  if (b < a.ns_blocks) return Role{0, b, 0};
  b -= a.ns_blocks;
  const int nK = a.nP;
  if (a.BH % 8 == 0) {
    const int per_head = nK + a.nQ;
    const int x = b % 8, i = b / 8;
    const int hh = i / per_head, u = i % per_head;  // head slot within the XCD, unit
    const int head = 8 * hh + x;
    return u < nK ? Role{1, head, u} : Role{2, head, u - nK};
  }
  if (b < a.BH * nK) return Role{1, b / nK, b % nK};
  const int bq = b - a.BH * nK;
  return Role{2, bq / a.nQ, bq % a.nQ};
}

__device__ __forceinline__ Role take_role(const MainArgs& a, int b) {
  if (!a.tickets) return static_role(a, b);
  const int nq = a.nq;
  const int per = (a.ns_blocks ? 1 : 0) + a.nP + a.nQ;  // units per head
  int x;
  if (nq == 8 && a.BH % 8 == 0) {
    x = b & 7;
  } else {
    int start = 0;
    for (x = 0; x + 1 < nq; ++x) {
      const int size = ((a.BH - x + nq - 1) / nq) * per;
      if (b < start + size) break;
      start += size;
    }
  }
  __shared__ unsigned ticket_s;
  if (threadIdx.x == 0)
    ticket_s = __hip_atomic_fetch_add(a.sync + 32 * x + 1, 1u, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int t = static_cast<int>(ticket_s);
  const int nh = (a.BH - x + nq - 1) / nq;  // heads of queue x
  const int ns = a.ns_blocks ? nh : 0;
  if (t < ns) return Role{0, x + nq * t, 0};
  const int i = t - ns, np = a.nP + a.nQ;
  const int head = x + nq * (i / np), u = i % np;
  return u < a.nP ? Role{1, head, u} : Role{2, head, u - a.nP};
}

// Read-only inputs are separate __restrict__ parameters so that wave-uniform
// reads of them (the landmark coordinates) compile to scalar loads.  At least
// 4 waves per SIMD (at most 128 VGPRs): two workgroups per CU, which the
// in-launch hand-offs count on (every workgroup of the grid resident).  One
// kernel per kernel kind and I/O type, so that a launch carries the code of
// its own map role only (the code of all four exceeds the instruction cache).
template <int D, int MB, int KIND, bool BF16>
__global__ __launch_bounds__(WGM, 4) void main_kernel(MainArgs a, const void* __restrict__ q,
                                                    const void* __restrict__ k,
                                                    const void* __restrict__ v,
                                                    const float* __restrict__ L) {
  constexpr int MAP_SMEM = map_smem<D, KIND>();
  // solver: the Newton-Schulz arrays plus a W^T copy (landmarks while A is
  // built)
  constexpr int SOLVER_SMEM = NsGeom<MB, D>::SMEM;
  // two workgroups per CU (160 KB of LDS), which the in-launch hand-offs
  // count on
  static_assert(4 * (MAP_SMEM > SOLVER_SMEM ? MAP_SMEM : SOLVER_SMEM) <= 80 * 1024,
                "LDS of two workgroups per CU");
  __shared__ __attribute__((aligned(16)))
  float smem[MAP_SMEM > SOLVER_SMEM ? MAP_SMEM : SOLVER_SMEM];
  const Role r = take_role(a, blockIdx.x);
  if (r.kind == 0) {
    solver_role<D, MB, KIND>(a, r.bh, smem);
  } else {
    map_role<D, KIND, BF16>(a, q, k, v, L, r.bh, r.kind == 1, r.u, smem);
  }
}

// ---------------------------------------------------------------------------
// pool: one workgroup per (LPW consecutive landmarks, head).  Thread
// (g, c4) sums a float4 column chunk over every G-th token of each window,
// the loads of all LPW windows (U tokens each per pass) issued together; a
// fixed-order LDS reduction over g finishes each mean.  LPW > 1 when the
// grid of one landmark per workgroup would not be resident at once: fewer,
// longer workgroups with more loads in flight.
// ---------------------------------------------------------------------------
template <int D, bool BF16, int LPW, int U>
__global__ __launch_bounds__(WGS) void pool_kernel(const void* __restrict__ K,
                                                   float* __restrict__ L,
                                                   float* __restrict__ st_L,
                                                   unsigned* __restrict__ sync,
                                                   unsigned* __restrict__ timeouts, int gw,
                                                   int ph, int pw, int m, int N) {
  constexpr int C4 = D / 4;
  constexpr int G = WGS / C4;
  __shared__ f4 part[LPW][WGS];
  const int j0 = blockIdx.x * LPW, bh = blockIdx.y;
  const int tid = threadIdx.x, c4 = tid % C4, g = tid / C4;
  // hand-off words of the main launch start at zero every call
  if (blockIdx.x == 0) {
    for (int e = tid; e < kSyncHead; e += WGS) sync[kSyncHead * (bh + 1) + e] = 0u;
    if (bh == 0) {
      // the call's words: ticket counters of the main launch (word 32 x + 1
      // of queue x, one cache line each) and the timeout count
      for (int e = tid; e < kSyncHead; e += WGS) sync[e] = 0u;
      if (tid == 0) *timeouts = 0u;
    }
  }
  const int mw = gw / pw;
  const int cnt = ph * pw;
  const size_t base = static_cast<size_t>(bh) * N;
  f4 s[LPW];
#pragma unroll
  for (int l = 0; l < LPW; ++l) s[l] = f4{0.f, 0.f, 0.f, 0.f};
  for (int t0 = g; t0 < cnt; t0 += U * G) {
    f4 v[LPW][U];
#pragma unroll
    for (int l = 0; l < LPW; ++l) {
      // landmarks past m read window 0 and are dropped below
      const int j = j0 + l < m ? j0 + l : 0;
      const int R = j / mw, C = j % mw;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        // tokens past the window are clamped to its first token and dropped below
        const int t = t0 + u * G < cnt ? t0 + u * G : 0;
        const int n = (R * ph + t / pw) * gw + C * pw + t % pw;
        v[l][u] = load4_io(K, (base + n) * D + 4 * c4, BF16);
      }
    }
#pragma unroll
    for (int l = 0; l < LPW; ++l)
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (t0 + u * G < cnt) s[l] += v[l][u];
  }
#pragma unroll
  for (int l = 0; l < LPW; ++l) part[l][tid] = s[l];
  __syncthreads();
  if (tid < LPW * C4) {
    const int l = tid / C4, c = tid % C4, j = j0 + l;
    if (j < m) {
      f4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int i = 0; i < G; ++i) acc += part[l][i * C4 + c];
      const f4 mean = acc / static_cast<float>(cnt);
      st4(L + (static_cast<size_t>(bh) * m + j) * D + 4 * c, mean);
      if (st_L) st4(st_L + (static_cast<size_t>(bh) * m + j) * D + 4 * c, mean);
    }
  }
}

// ---------------------------------------------------------------------------
// out: O = K_QL Y for the output-launch plan.  Workgroup = (head, 4 tiles of
// 64 tokens) with 16 waves; Y^T (from compute_y, columns >= m zero) is scaled
// per row into fp16 range and split in LDS once per workgroup; wave w forms
// the output rows of token block w % 4 of tile w / 4 on fp16 MFMA with
// two-part operands, K_QL scaled by 2^14 and split in registers (the
// arithmetic of out_tile in the main launch).  One 16-token block per wave
// keeps each wave's load -> product -> store chain short and many waves in
// flight.  Contraction chunks of 32 landmarks past mpad read as zero.
// ---------------------------------------------------------------------------
constexpr int WGO = 1024;             // output workgroup: 16 waves
constexpr int OUT_TILES = WGO / 256;  // tiles per output workgroup (4 waves each)

template <int D>
__global__ __launch_bounds__(WGO) void out_kernel(const float* __restrict__ kql,
                                                  const float* __restrict__ yt,
                                                  void* __restrict__ O, int bf16, int N,
                                                  int mpad, int nWo,
                                                  const float* __restrict__ mu) {
  constexpr int CBN = D / 16;
  __shared__ __attribute__((aligned(16))) uint16_t YH[D * WLD];
  __shared__ __attribute__((aligned(16))) uint16_t YL[D * WLD];
  __shared__ int EW[D];
  const int bh = blockIdx.x / nWo, wo = blockIdx.x % nWo;
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
  const int lr = lane & 15, lg = lane >> 4;
  const int t = wo * OUT_TILES + (w >> 2), tb = w & 3;  // this wave's tile and block
  const int n0 = t * TILE + 16 * tb;
  const bool active = n0 < N;
  // K_QL operands of the block, loads issued before the Y^T split so that
  // the two memory latencies overlap
  const float* kb = kql + static_cast<size_t>(bh) * N * mpad;
  f4 av[2][2];
  {
    const int n = n0 + lr;
    const float* ar = kb + static_cast<size_t>(n < N ? n : N - 1) * mpad;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int k = 32 * p + 8 * lg;
      if (active && k < mpad) {
        av[p][0] = ld4(ar + k);
        av[p][1] = ld4(ar + k + 4);
      } else {
        av[p][0] = av[p][1] = f4{0.f, 0.f, 0.f, 0.f};
      }
    }
  }
  // row c of Y^T by 8 consecutive lanes (8 values each), scaled by 2^EW[c]
  // into fp16 range and split
  {
    const float* yg = yt + static_cast<size_t>(bh) * D * MP;
    for (int e = tid; e < D * (MP / 8); e += WGO) {
      const int row = e / (MP / 8), k8 = 8 * (e % (MP / 8));
      const f4 v0 = ld4(yg + row * MP + k8), v1 = ld4(yg + row * MP + k8 + 4);
      unsigned mx = 0u;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        mx = max(mx, max(__float_as_uint(v0[i]) & 0x7fffffffu, __float_as_uint(v1[i]) & 0x7fffffffu));
      const int ew = fp16_scale(__uint_as_float(max8_u(mx)));
      u32x4 hv, lv;
      split8h(v0, v1, ew, hv, lv);
      *reinterpret_cast<u32x4*>(YH + row * WLD + k8) = hv;
      *reinterpret_cast<u32x4*>(YL + row * WLD + k8) = lv;
      if (k8 == 0) EW[row] = ew;
    }
  }
  __syncthreads();
  if (!active) return;
  if (mu) {
    // normalised map: K_QL centred per column (the column scales are in Y)
    const float* mh = mu + static_cast<size_t>(bh) * MP;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int k = 32 * p + 8 * lg;
      if (active && k < mpad) {
        av[p][0] -= ld4(mh + k);
        av[p][1] -= ld4(mh + k + 4);
      }
    }
  }
  u32x4 kh[2], kl[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) split8h(av[p][0], av[p][1], 14, kh[p], kl[p]);
  f4 cs[CBN];
#pragma unroll
  for (int cb = 0; cb < CBN; ++cb) {
    f4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int o = (16 * cb + lr) * WLD + 32 * p + 8 * lg;
      const u32x4 yh = *reinterpret_cast<const u32x4*>(YH + o);
      const u32x4 yl = *reinterpret_cast<const u32x4*>(YL + o);
      c = mfma_h(yh, kh[p], c);
      c = mfma_h(yh, kl[p], c);
      c = mfma_h(yl, kh[p], c);
    }
    // a block of O^T: lane (g, lr) holds columns 16 cb + 4 g .. + 3 of token
    // n0 + lr
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = ldexpf(c[i], -14 - EW[16 * cb + 4 * lg + i]);
    cs[cb] = c;
    if (CBN % 2 == 0 && !bf16) continue;
    const int n = n0 + lr;
    if (n < N) store_o4(O, bf16, (static_cast<size_t>(bh) * N + n) * D + 16 * cb + 4 * lg, c);
  }
  // fp32 rows of whole 128-byte lines: a line per store instruction
  if (CBN % 2 == 0 && !bf16) {
#pragma unroll
    for (int cb = 0; cb < CBN; cb += 2)
      store_o_lines<D>(O, static_cast<size_t>(bh) * N, n0, N, 16 * cb, cs[cb], cs[cb + 1]);
  }
}

inline float exp2_scale(float lambda) {
  // exp(-d / lambda) = exp2(d * (-log2(e) / lambda))
  return static_cast<float>(-1.4426950408889634 / static_cast<double>(lambda));
}

template <int D, int LPW, int U>
hipError_t launch_pool_dl(const Plan& p, const Args& a, const Buffers& b, hipStream_t s, Ev ev) {
  const dim3 grid((p.m + LPW - 1) / LPW, p.BH);
  if (p.bf16)
    return launch(pool_kernel<D, true, LPW, U>, grid, dim3(WGS), s, ev, a.k, b.L, a.st_L, b.sync,
                  b.timeouts, p.gw, p.ph, p.pw, p.m, p.N);
  return launch(pool_kernel<D, false, LPW, U>, grid, dim3(WGS), s, ev, a.k, b.L, a.st_L, b.sync,
                b.timeouts, p.gw, p.ph, p.pw, p.m, p.N);
}

template <int D>
hipError_t launch_pool_d(const Plan& p, const Args& a, const Buffers& b, hipStream_t s, Ev ev) {
  // One landmark per workgroup while that grid is resident at once (8
  // workgroups of 256 threads per CU), else four, with all their loads in
  // flight together.  A thread takes up to 4 tokens of a window, or one when
  // the window has at most one token per thread group (160 heads of 4 x 4
  // windows: the three clamped loads that no token needed made the launch
  // 10.2 instead of 6.5 us).
  const bool one = p.ph * p.pw <= WGS / (D / 4);
  if (static_cast<long>(p.m) * p.BH <= 2048)
    return one ? launch_pool_dl<D, 1, 1>(p, a, b, s, ev) : launch_pool_dl<D, 1, 4>(p, a, b, s, ev);
  return one ? launch_pool_dl<D, 4, 1>(p, a, b, s, ev) : launch_pool_dl<D, 4, 4>(p, a, b, s, ev);
}

template <int D, int MB>
hipError_t launch_main_dm(const MainArgs& ma, unsigned grid, hipStream_t s, Ev ev) {
  if (ma.kind == 0) {
    if (ma.bf16)
      return launch(main_kernel<D, MB, 0, true>, dim3(grid), dim3(WGM), s, ev, ma, ma.q, ma.k, ma.v, ma.L);
    return launch(main_kernel<D, MB, 0, false>, dim3(grid), dim3(WGM), s, ev, ma, ma.q, ma.k, ma.v, ma.L);
  }
  if (ma.bf16)
    return launch(main_kernel<D, MB, 1, true>, dim3(grid), dim3(WGM), s, ev, ma, ma.q, ma.k, ma.v, ma.L);
  return launch(main_kernel<D, MB, 1, false>, dim3(grid), dim3(WGM), s, ev, ma, ma.q, ma.k, ma.v, ma.L);
}

template <int D>
hipError_t launch_main_d(const Plan& p, const MainArgs& ma, unsigned grid, hipStream_t s, Ev ev) {
  switch (p.ns_mb) {
    case 1: return launch_main_dm<D, 1>(ma, grid, s, ev);
    case 2: return launch_main_dm<D, 2>(ma, grid, s, ev);
    case 3: return launch_main_dm<D, 3>(ma, grid, s, ev);
    case 4: return launch_main_dm<D, 4>(ma, grid, s, ev);
  }
  return hipErrorInvalidValue;
}

template <int D>
hipError_t launch_out_d(const Plan& p, const Args& a, const Buffers& b, hipStream_t s, Ev ev) {
  const int nWo = (p.nT + OUT_TILES - 1) / OUT_TILES;
  const dim3 grid(p.BH * nWo);
  return launch(out_kernel<D>, grid, dim3(WGO), s, ev, b.kql, b.yt, a.out, p.bf16, p.N, p.mpad,
                nWo, a.normalized ? static_cast<const float*>(b.mu) : nullptr);
}

// ---------------------------------------------------------------------------
// Normalised feature map (LaplacianFormer summaries: Arabic summary, section
// 2(b); Dutch summary, "Methodologie" item 1): Z = (K_QL - mu) / sqrt(var +
// delta) per column, mu and var over the head's N queries.  Workgroup (head,
// chunk c) reads rows [c R, (c + 1) R) of the stored K_QL: thread (column j,
// row group g) sums k - s and (k - s)^2 over rows g, g + 8, ... of the chunk
// (8 loads in flight) with s = K_QL[0][j] (a shift that keeps the variance
// free of cancellation); the 8 groups are added in order and the chunk's
// sums published; the last chunk of the head to arrive adds the chunks' sums
// in a fixed order (8 contiguous runs of chunks, each in chunk order, then
// the runs in order; so the result does not depend on timing): mu = s + S1 / N,
// var = S2 / N - (S1 / N)^2.  mu goes to the workspace (the output launch
// centres K_QL with it) and Y^T's column j is scaled by 1 / sqrt(var +
// delta), so O = (K_QL - mu) (Y / sqrt(var + delta)) = Z Y.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(WGM) void norm_stats_kernel(const float* __restrict__ kql, float* yt,
                                                         float* mu, float* part, unsigned* sync,
                                                         int N, int m, int mpad, int R,
                                                         float delta) {
  constexpr int G = WGM / MP;  // row groups
  constexpr int U = 8;         // loads in flight per thread
  __shared__ float s1[WGM], s2[WGM];
  __shared__ float rs[MP];
  const int bh = blockIdx.x, c = blockIdx.y, nc = gridDim.y, tid = threadIdx.x;
  const int j = tid % MP, g = tid / MP;
  const float* kb = kql + static_cast<size_t>(bh) * N * mpad;
  const int r0 = c * R, r1 = min(N, r0 + R);
  float a1 = 0.f, a2 = 0.f;
  if (j < m) {
    const float sh = kb[j];
    for (int i0 = r0 + g; i0 < r1; i0 += U * G) {
      float v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = i0 + u * G;
        v[u] = i < r1 ? kb[static_cast<size_t>(i) * mpad + j] - sh : 0.f;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        a1 += v[u];
        a2 = fmaf(v[u], v[u], a2);
      }
    }
  }
  s1[tid] = a1;
  s2[tid] = a2;
  __syncthreads();
  // this chunk's sums, published for the head's last chunk
  float* pc = part + (static_cast<size_t>(bh) * nc + c) * 2 * MP;
  if (tid < MP) {
    float t1 = 0.f, t2 = 0.f;
    for (int u = 0; u < G; ++u) {
      t1 += s1[u * MP + tid];
      t2 += s2[u * MP + tid];
    }
    st_dev(pc + tid, t1);
    st_dev(pc + MP + tid, t2);
  }
  unsigned* cnt = sync + kSyncHead * (bh + 1) + kNormCount;
  if (publish_arrive(cnt) != static_cast<unsigned>(nc - 1)) return;
  {
    // the head's chunk sums in chunk order: thread (j, g) sums chunks
    // [g P, (g + 1) P) with up to 8 chunks' loads in flight, then the G
    // group sums are added in order of g (one load in flight per chunk made
    // this sum a chain of nc memory latencies)
    const float* ph = part + static_cast<size_t>(bh) * nc * 2 * MP;
    const int P = (nc + G - 1) / G;
    const int u1 = min(nc, (g + 1) * P);
    float t1 = 0.f, t2 = 0.f;
    for (int p0 = g * P; p0 < u1; p0 += 8) {
      float v1[8], v2[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const bool ok = p0 + q < u1;
        v1[q] = ok ? ph[(p0 + q) * 2 * MP + j] : 0.f;
        v2[q] = ok ? ph[(p0 + q) * 2 * MP + MP + j] : 0.f;
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if (p0 + q < u1) {
          t1 += v1[q];
          t2 += v2[q];
        }
      }
    }
    __syncthreads();  // s1 and s2 held this chunk's sums
    s1[tid] = t1;
    s2[tid] = t2;
    __syncthreads();
  }
  if (tid < MP) {
    float t1 = 0.f, t2 = 0.f;
    for (int u = 0; u < G; ++u) {
      t1 += s1[u * MP + tid];
      t2 += s2[u * MP + tid];
    }
    float mean = 0.f, r = 0.f;
    if (tid < m) {
      const float inv = 1.0f / static_cast<float>(N);
      const float d1 = t1 * inv;
      const float var = fmaxf(t2 * inv - d1 * d1, 0.f);
      mean = kb[tid] + d1;
      r = 1.0f / sqrtf(var + delta);
    }
    mu[static_cast<size_t>(bh) * MP + tid] = mean;
    rs[tid] = r;
  }
  __syncthreads();
  float* y = yt + static_cast<size_t>(bh) * D * MP;
  for (int e = tid; e < D * MP; e += WGM) y[e] *= rs[e % MP];
}

}  // namespace

bool out_in_main_launch(const Plan& p, int shared_qk) {
  if (shared_qk) return false;
  const long nQ = (p.nT + QT - 1) / QT;
  return static_cast<long>(p.BH) * (1 + p.nP + nQ) <= p.resident;
}

hipError_t launch_pool(const Plan& p, const Args& a, const Buffers& b, hipStream_t s, Ev ev) {
  switch (p.D) {
    case 16: return launch_pool_d<16>(p, a, b, s, ev);
    case 32: return launch_pool_d<32>(p, a, b, s, ev);
    case 64: return launch_pool_d<64>(p, a, b, s, ev);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_main(const Plan& p, const Args& a, const Buffers& b, bool with_solver,
                       bool with_maps, hipStream_t s, Ev ev) {
  MainArgs ma{};
  ma.q = a.q;
  ma.k = a.k;
  ma.v = a.v;
  ma.L = b.L;
  ma.kql = b.kql;
  ma.wpart = b.wpart;
  ma.xw = b.x;
  ma.wt = b.wt;
  ma.yt = b.yt;
  ma.out = a.out;
  ma.sync = b.sync;
  ma.timeouts = b.timeouts;
  ma.st_a = a.st_a;
  ma.st_x = a.st_x;
  ma.st_kql = a.st_kql;
  ma.st_klk = a.st_klk;
  ma.st_w = a.st_w;
  ma.N = p.N;
  ma.m = p.m;
  ma.BH = p.BH;
  ma.nT = p.nT;
  ma.S = p.S;
  ma.nP = p.nP;
  ma.mpad = p.mpad;
  ma.shared_qk = a.shared_qk;
  ma.out_in_main = a.out_in_main;
  ma.qt = a.out_in_main ? QT : p.qt;
  ma.nQ = a.shared_qk ? 0 : (p.nT + ma.qt - 1) / ma.qt;
  ma.kind = p.kernel;
  ma.bf16 = p.bf16;
  ma.iters = a.iters;
  ma.c_exp2 = exp2_scale(a.lambda);
  ma.eps = a.eps;
  ma.ns_blocks = with_solver ? p.BH : 0;
  // roles by ticket on request; a solver-only launch (serial plan) has no
  // waits and keeps workgroup b on head b
  ma.tickets = (with_maps && a.tickets) ? 1 : 0;
  ma.nq = p.BH % 8 == 0 ? 8 : (p.BH < 8 ? p.BH : 8);
  const long map_wgs = with_maps ? static_cast<long>(p.BH) * (p.nP + ma.nQ) : 0;
  const unsigned grid = static_cast<unsigned>(ma.ns_blocks + map_wgs);
  if (grid == 0) return hipSuccess;
  switch (p.D) {
    case 16: return launch_main_d<16>(p, ma, grid, s, ev);
    case 32: return launch_main_d<32>(p, ma, grid, s, ev);
    case 64: return launch_main_d<64>(p, ma, grid, s, ev);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_norm_stats(const Plan& p, const Args& a, const Buffers& b, hipStream_t s) {
  // chunks of rows per head: enough workgroups to spread over the device, at
  // least 64 rows each, and their sums (2 MP floats per chunk) within the W^T
  // partials buffer, which the output-launch plan has consumed by now
  const int want = std::max(1, std::min((p.N + 63) / 64, (512 + p.BH - 1) / p.BH));
  const int cap = std::max(1, p.nP * p.D / 2);
  const int nc0 = std::min(want, cap);
  const int R = (p.N + nc0 - 1) / nc0;
  const int nc = (p.N + R - 1) / R;
  const dim3 grid(p.BH, nc);
  switch (p.D) {
    case 16: return launch(norm_stats_kernel<16>, grid, dim3(WGM), s, Ev{}, b.kql, b.yt, b.mu, b.wpart, b.sync, p.N, p.m, p.mpad, R, a.delta);
    case 32: return launch(norm_stats_kernel<32>, grid, dim3(WGM), s, Ev{}, b.kql, b.yt, b.mu, b.wpart, b.sync, p.N, p.m, p.mpad, R, a.delta);
    case 64: return launch(norm_stats_kernel<64>, grid, dim3(WGM), s, Ev{}, b.kql, b.yt, b.mu, b.wpart, b.sync, p.N, p.m, p.mpad, R, a.delta);
  }
  return hipErrorInvalidValue;
}


hipError_t launch_out(const Plan& p, const Args& a, const Buffers& b, hipStream_t s, Ev ev) {
  switch (p.D) {
    case 16: return launch_out_d<16>(p, a, b, s, ev);
    case 32: return launch_out_d<32>(p, a, b, s, ev);
    case 64: return launch_out_d<64>(p, a, b, s, ev);
  }
  return hipErrorInvalidValue;
}

}  // namespace lapattn
