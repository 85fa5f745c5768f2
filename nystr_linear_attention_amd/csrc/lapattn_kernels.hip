// HIP kernels for Nystrom kernel attention (forward) on gfx950.
//
// Two launches per forward call (three when Q and K are the same tensor),
// back to back on the caller's stream:
//   pool : landmarks L = window means of K                         (HBM stream)
//   main : role-split workgroups
//          - solver WGs (one per head, first in the grid, raised wave
//            priority): A = k(L, L) + eps I, alpha, then the Newton-Schulz
//            steps held in LDS on fp32 MFMA
//          - map WGs: kernel values of 64 tokens against every landmark on
//            FP32 VALU (landmark coordinates are wave-uniform scalar operands);
//            key tiles contract K_LK V on fp32 MFMA into per-workgroup
//            partials of W^T; query tiles keep their K_QL rows in LDS
//          - hand-offs: the last key WG of a head reduces the partials (fixed
//            order, deterministic) into W^T; the second of (W^T, X) forms
//            Y^T = W^T X^T; query WGs wait for it and write O = K_QL Y
//   out  : (Q == K only) O = K_QL Y on fp32 MFMA from K_QL stored by the key
//          tiles.
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
// MFMA operand convention used throughout (v_mfma_f32_16x16x4f32): for an
// output block D[16][16] += sum_k A[i][k] B[k][j], lane l = 16*g + r supplies
// A[r][k] and B[k][r] at sub-step s with k = KS*g + s (KS sub-steps), so each
// lane reads KS *contiguous* k values of one row of A and one row of B^T.
// The accumulator holds D[4g + i][r], i = 0..3.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>
#include <utility>

#include "lapattn_internal.h"

namespace lapattn {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int LS = 68;        // LDS row stride (floats) of 64-wide tiles: 16-B rows
constexpr int WGM = 512;      // main kernel: 8 wave64
constexpr int WGS = 256;      // pool / out kernels: 4 wave64
constexpr int TILE = 64;      // tokens per map tile (one per lane)
constexpr int NGRP = 8;       // landmark groups per map tile (one per wave)
constexpr int QT = 2;         // 64-token tiles per query workgroup

__device__ __forceinline__ f4 mfma4(float a, float b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

__device__ __forceinline__ f4 ld4(const float* p) { return *reinterpret_cast<const f4*>(p); }
__device__ __forceinline__ void st4(float* p, f4 v) { *reinterpret_cast<f4*>(p) = v; }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Four consecutive elements (16-B aligned for fp32, 8-B for bf16) as fp32.
__device__ __forceinline__ f4 load4_io(const void* base, size_t idx, int bf16) {
  if (bf16) {
    const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + idx);
    return f4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
              __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u)};
  }
  return ld4(static_cast<const float*>(base) + idx);
}

__device__ __forceinline__ float load1_io(const void* base, size_t idx, int bf16) {
  if (bf16) return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(base)[idx]) << 16);
  return static_cast<const float*>(base)[idx];
}

// One token row of D elements into registers.
template <int D>
__device__ __forceinline__ void load_row(const void* base, size_t row, int bf16, float* x) {
  if (bf16) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + row * D);
#pragma unroll
    for (int i = 0; i < D / 8; ++i) {
      const uint4 u = p[i];
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        x[8 * i + 2 * h] = __uint_as_float(w[h] << 16);
        x[8 * i + 2 * h + 1] = __uint_as_float(w[h] & 0xffff0000u);
      }
    }
  } else {
    const f4* p = reinterpret_cast<const f4*>(static_cast<const float*>(base) + row * D);
#pragma unroll
    for (int i = 0; i < D / 4; ++i) {
      const f4 u = p[i];
      x[4 * i] = u[0];
      x[4 * i + 1] = u[1];
      x[4 * i + 2] = u[2];
      x[4 * i + 3] = u[3];
    }
  }
}

// Distances of a register-resident point to two wave-uniform points l0, l1
// (scalar loads issued together, so their latencies overlap).  Holding more
// landmark coordinates in flight than this spills scalar registers.
template <int D, int KIND>
__device__ __forceinline__ void dist_to2(const float* x, const float* __restrict__ l0,
                                         const float* __restrict__ l1, float& r0, float& r1) {
  float a0 = 0.f, a1 = 0.f, b0 = 0.f, b1 = 0.f;
#pragma unroll
  for (int k = 0; k < D; k += 2) {
    const float s0 = x[k] - l0[k], s1 = x[k + 1] - l0[k + 1];
    const float t0 = x[k] - l1[k], t1 = x[k + 1] - l1[k + 1];
    if constexpr (KIND == 0) {
      a0 += fabsf(s0);
      a1 += fabsf(s1);
      b0 += fabsf(t0);
      b1 += fabsf(t1);
    } else {
      a0 = fmaf(s0, s0, a0);
      a1 = fmaf(s1, s1, a1);
      b0 = fmaf(t0, t0, b0);
      b1 = fmaf(t1, t1, b1);
    }
  }
  r0 = a0 + a1;
  r1 = b0 + b1;
}

// Distance of a register-resident point to a wave-uniform point `l`
// (scalar loads): L1 for KIND 0, squared L2 for KIND 1.  Two partial sums.
template <int D, int KIND>
__device__ __forceinline__ float dist_to(const float* x, const float* __restrict__ l) {
  float d0 = 0.f, d1 = 0.f;
#pragma unroll
  for (int k = 0; k < D; k += 2) {
    const float t0 = x[k] - l[k];
    const float t1 = x[k + 1] - l[k + 1];
    if constexpr (KIND == 0) {
      d0 += fabsf(t0);
      d1 += fabsf(t1);
    } else {
      d0 = fmaf(t0, t0, d0);
      d1 = fmaf(t1, t1, d1);
    }
  }
  return d0 + d1;
}

struct MainArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* L;     // [BH][m][D]
  float* kql;         // [BH][N][mpad]
  float* wpart;       // [BH][nP][D][MP]
  float* xw;          // [BH][MP][MP]
  float* wt;          // [BH][D][MP]  W^T (reduced partials)
  float* yt;          // [BH][D][MP]  Y^T = (X W)^T
  void* out;          // [BH][N][D]   O (query workgroups write it)
  unsigned* sync;     // hand-off words, zeroed by the pool launch:
                      //   [0] count of bounded waits that timed out,
                      //   [4 + bh] key-workgroup arrivals, [4 + BH + bh]
                      //   arrivals of W and X, [4 + 2 BH + bh] Y-ready flag
  float* st_a;
  float* st_x;
  float* st_kql;
  float* st_klk;
  float* st_w;
  int N, m, BH, nT, S, nP, mpad;
  int ns_blocks;      // workgroups [0, ns_blocks) are solver workgroups
  int nQ;             // query workgroups per head, QT tiles each (0 when Q == K)
  int shared_qk;      // Q and K are the same tensor
  int out_in_main;    // query workgroups wait for Y and write O (else they
                      // store K_QL and the output launch forms O)
  int kind, bf16, iters;
  float c_exp2, eps;
};

// ---------------------------------------------------------------------------
// Hand-offs inside the main launch.  Per head: the key workgroups publish W^T
// partials and count their arrivals; the last one reduces them (fixed order,
// so the result does not depend on which one is last) and publishes W^T.  W^T
// and X (from the solver workgroup) each count one arrival; whichever is
// second forms Y^T = W^T X^T and raises the head's Y-ready flag, on which the
// query workgroups wait before forming their output rows.
//
// Coherence across XCDs without cache-wide fences: everything handed over
// inside the launch (partials, W^T, X, Y^T) is stored with device-scope
// relaxed atomic stores, which write through the per-XCD L2 to memory; a
// publisher drains its stores (vmcnt(0)) and meets its workgroup at a
// barrier before one thread counts the arrival or raises the flag (device-
// scope atomics).  Consumers read the handed-over data with plain loads
// after seeing the count or flag: no XCD touches those addresses earlier in
// the launch, and every launch starts with invalidated caches, so the loads
// miss to memory.  (A device-scope release / acquire fence would instead
// write back / invalidate the whole L2 of the XCD, which costs microseconds
// and evicts what the map workgroups stream; device-scope loads of the data
// itself are several times slower than plain misses.)
//
// Forward progress: solver workgroups come first in the grid and each head's
// key workgroups precede its query workgroups, so with in-order dispatch
// every producer has started before a consumer can wait on it.  The wait is
// bounded in time regardless (it then counts a timeout in sync[0] and goes
// on), so no wave can spin forever.
// ---------------------------------------------------------------------------
constexpr long long kWaitTicks = 2000000;  // 20 ms of the 100 MHz device clock

__device__ __forceinline__ unsigned* cnt_w(const MainArgs& a, int bh) { return a.sync + 4 + bh; }
__device__ __forceinline__ unsigned* cnt_y(const MainArgs& a, int bh) {
  return a.sync + 4 + a.BH + bh;
}
__device__ __forceinline__ unsigned* flag_y(const MainArgs& a, int bh) {
  return a.sync + 4 + 2 * a.BH + bh;
}

__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Waits until this thread's global stores have completed.
__device__ __forceinline__ void drain_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Completes this workgroup's device-scope stores, then counts one arrival at
// *ctr; returns the previous count in every thread.
__device__ __forceinline__ unsigned publish_arrive(unsigned* ctr) {
  __shared__ unsigned old_s;
  drain_stores();
  __syncthreads();
  if (threadIdx.x == 0) old_s = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  return old_s;
}

__device__ __forceinline__ void raise_flag(unsigned* flag) {
  drain_stores();
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_store(flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void wait_flag(unsigned* flag, unsigned* timeouts) {
  if (threadIdx.x == 0) {
    const long long t0 = wall_clock64();
    while (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u) {
      if (wall_clock64() - t0 > kWaitTicks) {
        __hip_atomic_fetch_add(timeouts, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  __syncthreads();
}

// Y^T = W^T X^T for one head on fp32 MFMA, D x 64 outputs (columns >= m are
// zero because X is zero padded).  W^T rows have stride wts; X has xrows
// rows of stride xs (columns >= xs and rows >= xrows read as zero), so the
// operands may come from global memory or from the solver's LDS: the same
// values in the same MFMA order give the same Y^T either way.
template <int D>
__device__ void compute_y(const float* wt, int wts, const float* x, int xs, int xrows,
                          float* yg) {
  constexpr int CBN = D / 16;
  constexpr int NBLK = 4 * CBN;  // 16x16 output blocks
  const int lane = threadIdx.x & 63, w = wave_id();
  const int lr = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int s = 0; s < (NBLK + 7) / 8; ++s) {
    const int blk = w + 8 * s;
    if (blk < NBLK) {
      const int cb = blk / 4, jb = blk % 4;
      // lane (g, r) supplies W^T[16 cb + r][16 g + u] and X[16 jb + r][16 g + u]
      const float* ar = wt + (16 * cb + lr) * wts + 16 * lg;
      const int xr = 16 * jb + lr;
      f4 av[4], bv[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        av[q] = ld4(ar + 4 * q);
        const int c0 = 16 * lg + 4 * q;
        bv[q] = (xr < xrows && c0 < xs) ? ld4(x + xr * xs + c0) : f4{0.f, 0.f, 0.f, 0.f};
      }
      f4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int h = 0; h < 4; ++h) c = mfma4(av[q][h], bv[q][h], c);
#pragma unroll
      for (int i = 0; i < 4; ++i) st_dev(yg + (16 * cb + 4 * lg + i) * MP + 16 * jb + lr, c[i]);
    }
  }
}

template <int D>
__device__ __forceinline__ void compute_y_global(const MainArgs& a, int bh) {
  compute_y<D>(a.wt + static_cast<size_t>(bh) * D * MP, MP,
               a.xw + static_cast<size_t>(bh) * MP * MP, MP, MP,
               a.yt + static_cast<size_t>(bh) * D * MP);
}

// Second arrival of (W^T, X) for head bh forms Y^T and raises the flag.
template <int D>
__device__ void arrive_y(const MainArgs& a, int bh) {
  if (publish_arrive(cnt_y(a, bh)) == 1u) {
    compute_y_global<D>(a, bh);
    raise_flag(flag_y(a, bh));
  }
}

// ---------------------------------------------------------------------------
// Solver role: X_0 = alpha A, X_{t+1} = 2 X_t - X_t (A X_t), exactly `iters`
// steps, one workgroup per head, everything in LDS and registers.
//
// m = 16 MB + r with r <= 1 border row/column (other sizes are zero padded to
// 16 MB and r = 0; the border code is written for any r <= 4).  Both products are full and unsymmetrised:
// forcing the iterates symmetric turns the quadratic error contraction of the
// Newton step into a linear map with gain up to (1 + cond(A)) / 2, which
// diverges near convergence for ill-conditioned A.
//
// Interior wave c < MB owns column block c (16 columns) of X_t, of
// T = A X_t and of X_{t+1}:
//   T[:, c]       = A X_t[:, c]              (needs only its own X columns)
//   X_{t+1}[:, c] = 2 X_t[:, c] - X_t T[:, c] (needs the rows of X_t)
// With the contraction index of MFMA sub-step s = 4 i + j taken as
// k = 16 i + 4 g + j for lane (g, lr), the accumulator layout of a 16 x 16
// block (lane (g, lr) holds rows 4 g + j of column lr) is exactly the B
// operand layout, so X_t[:, c] and T[:, c] never leave registers; the A
// operands (rows of A, rows of X_t) are 16-byte LDS reads.  Only the rows of
// X_t are exchanged, once per step: one barrier per step.
// The border: interior waves compute T and X_{t+1} on the border rows of
// their own columns (VALU dot products and a 4-lane reduction); border wave
// b < r computes border column 16 MB + b of T and X_{t+1} (one row per lane).
// Border terms of the interior blocks (k >= 16 MB) initialise the
// accumulators.  A is bitwise symmetric (|a - b| = |b - a| term by term), so
// its border columns are read as rows.
//
// LDS (floats, row stride SLS): A, X[2] (row-major, double buffered),
// XTB[2][4][64] (border columns of X_t, transposed), TX[4][64] (border columns
// of T, private to each border wave), scalars.
// ---------------------------------------------------------------------------
template <int MB>
struct NsGeom {
  static constexpr int N16 = 16 * MB;               // interior size
  // rows and row stride: the interior plus up to 4 border rows / columns.
  // Strides are 4 or 20 (mod 32) floats, so 16-byte reads of 8 consecutive
  // rows fall on distinct LDS banks.
  static constexpr int ROWS = MB == 4 ? 64 : N16 + 4;
  static constexpr int SLS = MB == 4 ? 68 : N16 + 4;
  static constexpr int MAT = ROWS * SLS;
  static constexpr int NQ = ROWS / 4;               // float4 per border dot
  static constexpr int OFF_XTB = 3 * MAT;
  static constexpr int OFF_TX = OFF_XTB + 2 * 4 * 64;
  static constexpr int OFF_RED = OFF_TX + 4 * 64;
  static constexpr int SMEM = OFF_RED + 4;
};

// Sum over the 4 lanes (g = 0..3) that share lr, on VALU: a lane-half swap
// with itself leaves v[l] + v[l ^ 32] as the sum of the two results (and
// likewise for 16-lane rows).
__device__ __forceinline__ float sum_over_g(float v) {
  const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(h[0]) + __uint_as_float(h[1]);
  const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

template <int MB, int R>
__device__ void ns_interior_wave(const MainArgs& a, float* smem, int c, int lane) {
  constexpr int r = R;  // border width
  using G = NsGeom<MB>;
  constexpr int S = G::SLS, N16 = G::N16;
  // Buffers are addressed by offsets from the shared base (never through a
  // table of pointers) so that every access stays an LDS instruction.
  const float* A = smem;
  const float* X0 = smem + G::MAT;
  const int lr = lane & 15, lg = lane >> 4;
  const int col = 16 * c + lr;

  // own columns of X_0 (accumulator layout) and of its border rows
  f4 xc[MB];
  float xbr[4];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) xc[i][j] = X0[(16 * i + 4 * lg + j) * S + col];
#pragma unroll
  for (int b = 0; b < 4; ++b) xbr[b] = b < r ? X0[(N16 + b) * S + col] : 0.f;
  // constant operands: the border rows of A at the own k (for T's border
  // rows), A's border corner
  f4 abr[4][MB];
  float acor[4][4];
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int i = 0; i < MB; ++i)
      abr[b][i] = b < r ? ld4(A + (N16 + b) * S + 16 * i + 4 * lg) : f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) acor[b][bb] = (b < r && bb < r) ? A[(N16 + b) * S + N16 + bb] : 0.f;

  // Output blocks are computed one after another (a single accumulation
  // chain runs at the full MFMA rate), so that each block's epilogue and the
  // next block's operand reads overlap the running MFMAs.  The A operand of
  // the first block of phase 1 is constant and is read before the barrier.
  f4 aop[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i) aop[i] = ld4(A + lr * S + 16 * i + 4 * lg);

  for (int t = 0; t < a.iters; ++t) {
    const int cb = t & 1;
    const float* cur = smem + G::MAT * (1 + cb);
    float* nxt = smem + G::MAT * (2 - cb);
    const float* xtb = smem + G::OFF_XTB + 256 * cb;

    // reads that only need X_t: the phase-2 operand of block 0, the border
    // columns of X_t at the own rows, the border rows of X_t at the own k
    f4 xop[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i) xop[i] = ld4(cur + lr * S + 16 * i + 4 * lg);
    f4 xbc[4][MB], xbrow[4][MB];
    float xcor[4][4];
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        xbc[b][i] = b < r ? ld4(xtb + 64 * b + 16 * i + 4 * lg) : f4{0.f, 0.f, 0.f, 0.f};
        xbrow[b][i] = b < r ? ld4(cur + (N16 + b) * S + 16 * i + 4 * lg) : f4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) xcor[b][bb] = (b < r && bb < r) ? cur[(N16 + b) * S + N16 + bb] : 0.f;

    // phase 1: T[:, c] = A X_t[:, c], block by block; the border terms
    // (k >= 16 MB) initialise each block: A[rows][N16+b] = A[N16+b][rows].
    // The scheduling fences keep every operand read ahead of the MFMAs of
    // the block before the one that needs it, and put VALU work between
    // MFMAs, so the matrix pipe never waits on LDS.
    f4 tc[MB];
    float tbr[4];
#pragma unroll
    for (int ip = 0; ip < MB; ++ip) {
      f4 anx[MB];
      if (ip + 1 < MB) {
#pragma unroll
        for (int i = 0; i < MB; ++i) anx[i] = ld4(A + (16 * (ip + 1) + lr) * S + 16 * i + 4 * lg);
      }
      f4 t4 = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int b = 0; b < 4; ++b)
        if (b < r) {
#pragma unroll
          for (int j = 0; j < 4; ++j) t4[j] = fmaf(abr[b][ip][j], xbr[b], t4[j]);
        }
      __builtin_amdgcn_sched_barrier(0);
      t4 = mfma4(aop[0][0], xc[0][0], t4);
      t4 = mfma4(aop[0][1], xc[0][1], t4);
      __builtin_amdgcn_sched_barrier(0);
      if (ip == 0) {
        // T on the border rows of the own columns:
        // T[N16+b][col] = sum_k A[N16+b][k] X_t[k][col]
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          tbr[b] = 0.f;
          if (b < r) {
            float p = 0.f;
#pragma unroll
            for (int i = 0; i < MB; ++i)
#pragma unroll
              for (int j = 0; j < 4; ++j) p = fmaf(abr[b][i][j], xc[i][j], p);
            p = sum_over_g(p);
#pragma unroll
            for (int bb = 0; bb < 4; ++bb)
              if (bb < r) p = fmaf(acor[b][bb], xbr[bb], p);
            tbr[b] = p;
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s4 = 2; s4 < 4 * MB; ++s4) t4 = mfma4(aop[s4 / 4][s4 % 4], xc[s4 / 4][s4 % 4], t4);
      __builtin_amdgcn_sched_barrier(0);
      tc[ip] = t4;
      if (ip + 1 < MB) {
#pragma unroll
        for (int i = 0; i < MB; ++i) aop[i] = anx[i];
      }
    }

    // phase 2: X_{t+1}[:, c] = 2 X_t[:, c] - X_t T[:, c], block by block;
    // border terms X_t[rows][N16+b] T[N16+b][col] initialise each block.
    // The epilogue of block ip - 1 (2 X - acc, row-major LDS store) runs
    // between the MFMAs of block ip.
    float xbn[4];
    f4 prev = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ip = 0; ip < MB; ++ip) {
      f4 xnx[MB];
      if (ip + 1 < MB) {
#pragma unroll
        for (int i = 0; i < MB; ++i) xnx[i] = ld4(cur + (16 * (ip + 1) + lr) * S + 16 * i + 4 * lg);
      } else {
        // the constant phase-1 operand of the next step (block 0)
#pragma unroll
        for (int i = 0; i < MB; ++i) xnx[i] = ld4(A + lr * S + 16 * i + 4 * lg);
      }
      f4 t4 = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int b = 0; b < 4; ++b)
        if (b < r) {
#pragma unroll
          for (int j = 0; j < 4; ++j) t4[j] = fmaf(xbc[b][ip][j], tbr[b], t4[j]);
        }
      __builtin_amdgcn_sched_barrier(0);
      t4 = mfma4(xop[0][0], tc[0][0], t4);
      t4 = mfma4(xop[0][1], tc[0][1], t4);
      __builtin_amdgcn_sched_barrier(0);
      if (ip > 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          xc[ip - 1][j] = 2.0f * xc[ip - 1][j] - prev[j];
          nxt[(16 * (ip - 1) + 4 * lg + j) * S + col] = xc[ip - 1][j];
        }
      } else {
        // X_{t+1} on the border rows of the own columns:
        // 2 X_t[N16+b][col] - sum_k X_t[N16+b][k] T[k][col]
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          xbn[b] = 0.f;
          if (b < r) {
            float p = 0.f;
#pragma unroll
            for (int i = 0; i < MB; ++i)
#pragma unroll
              for (int j = 0; j < 4; ++j) p = fmaf(xbrow[b][i][j], tc[i][j], p);
            p = sum_over_g(p);
#pragma unroll
            for (int bb = 0; bb < 4; ++bb)
              if (bb < r) p = fmaf(xcor[b][bb], tbr[bb], p);
            xbn[b] = 2.0f * xbr[b] - p;
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s4 = 2; s4 < 4 * MB; ++s4) t4 = mfma4(xop[s4 / 4][s4 % 4], tc[s4 / 4][s4 % 4], t4);
      __builtin_amdgcn_sched_barrier(0);
      prev = t4;
      if (ip + 1 < MB) {
#pragma unroll
        for (int i = 0; i < MB; ++i) xop[i] = xnx[i];
      } else {
#pragma unroll
        for (int i = 0; i < MB; ++i) aop[i] = xnx[i];
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      xc[MB - 1][j] = 2.0f * xc[MB - 1][j] - prev[j];
      nxt[(16 * (MB - 1) + 4 * lg + j) * S + col] = xc[MB - 1][j];
    }
#pragma unroll
    for (int b = 0; b < 4; ++b)
      if (b < r) {
        xbr[b] = xbn[b];
        if (lg == 0) nxt[(N16 + b) * S + col] = xbr[b];
      }
    __syncthreads();
  }
}

// Border wave b: column N16 + b of T and X_{t+1}, lane k = row k (k < m).
template <int MB>
__device__ void ns_border_wave(const MainArgs& a, float* smem, int b, int lane) {
  using G = NsGeom<MB>;
  constexpr int S = G::SLS, N16 = G::N16;
  const float* A = smem;
  float* TX = smem + G::OFF_TX + 64 * b;
  const int k = lane;
  const bool row = k < a.m;           // m <= ROWS
  float xk = row ? smem[G::MAT + k * S + N16 + b] : 0.f;

  for (int t = 0; t < a.iters; ++t) {
    const int cb = t & 1;
    const float* cur = smem + G::MAT * (1 + cb);
    float* nxt = smem + G::MAT * (2 - cb);
    const float* xtb = smem + G::OFF_XTB + 256 * cb + 64 * b;
    float* xtn = smem + G::OFF_XTB + 256 * (1 - cb) + 64 * b;
    // T[k][N16+b] = sum_k' A[k][k'] X_t[k'][N16+b]
    float tk = 0.f;
    if (row) {
      float d[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < G::NQ; ++q) {
        const f4 ar = ld4(A + k * S + 4 * q), xv = ld4(xtb + 4 * q);
        d[q & 3] = fmaf(ar[3], xv[3], fmaf(ar[2], xv[2], fmaf(ar[1], xv[1], fmaf(ar[0], xv[0], d[q & 3]))));
      }
      tk = (d[0] + d[1]) + (d[2] + d[3]);
    }
    TX[k] = tk;  // rows >= m are zero
    // make the whole column visible to every lane of this wave
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // X_{t+1}[k][N16+b] = 2 X_t[k][N16+b] - sum_k' X_t[k][k'] T[k'][N16+b]
    if (row) {
      float d[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < G::NQ; ++q) {
        const f4 xr = ld4(cur + k * S + 4 * q), tv = ld4(TX + 4 * q);
        d[q & 3] = fmaf(xr[3], tv[3], fmaf(xr[2], tv[2], fmaf(xr[1], tv[1], fmaf(xr[0], tv[0], d[q & 3]))));
      }
      xk = 2.0f * xk - ((d[0] + d[1]) + (d[2] + d[3]));
      nxt[k * S + N16 + b] = xk;
      xtn[k] = xk;
    }
    __syncthreads();
  }
}

// The 2 x 2 blocks of the upper triangle of A = k(L, L) + eps I (see
// solver_role): landmarks staged in Ls (rows of LDL floats), A in LDS with
// row stride S.
template <int D, int KIND>
__device__ void build_a(const MainArgs& a, int bh, const float* Ls, float* A, int S) {
  constexpr int LDL = D + 4;
  const int m = a.m, nb = (m + 1) / 2;
  float* sa = a.st_a ? a.st_a + static_cast<size_t>(bh) * m * m : nullptr;
  for (int blk = threadIdx.x; blk < nb * (nb + 1) / 2; blk += WGM) {
    // blk = bj (bj + 1) / 2 + bi with bi <= bj
    int bj = static_cast<int>((sqrtf(8.0f * blk + 1.0f) - 1.0f) * 0.5f);
    while (bj * (bj + 1) / 2 > blk) --bj;
    while ((bj + 1) * (bj + 2) / 2 <= blk) ++bj;
    const int bi = blk - bj * (bj + 1) / 2;
    const float* r0 = Ls + (2 * bi) * LDL;
    const float* r1 = r0 + LDL;
    const float* c0 = Ls + (2 * bj) * LDL;
    const float* c1 = c0 + LDL;
    // d[u][h]: pair u = (row, col) in {00, 01, 10, 11}, two partial sums
    float d[4][2] = {{0.f, 0.f}, {0.f, 0.f}, {0.f, 0.f}, {0.f, 0.f}};
    // partial unroll: full unrolling hoists every row read and spills
#pragma unroll 4
    for (int q = 0; q < D / 4; ++q) {
      const f4 x0 = ld4(r0 + 4 * q), x1 = ld4(r1 + 4 * q);
      const f4 y0 = ld4(c0 + 4 * q), y1 = ld4(c1 + 4 * q);
      const f4 t[4] = {x0 - y0, x0 - y1, x1 - y0, x1 - y1};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if constexpr (KIND == 0) {
          d[u][0] += fabsf(t[u][0]) + fabsf(t[u][2]);
          d[u][1] += fabsf(t[u][1]) + fabsf(t[u][3]);
        } else {
          d[u][0] = fmaf(t[u][0], t[u][0], fmaf(t[u][2], t[u][2], d[u][0]));
          d[u][1] = fmaf(t[u][1], t[u][1], fmaf(t[u][3], t[u][3], d[u][1]));
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = 2 * bi + (u >> 1), j = 2 * bj + (u & 1);
      // in the diagonal block, (2bi+1, 2bi) repeats (2bi, 2bi+1)
      if (i < m && j < m && i <= j) {
        float v = exp2f((d[u][0] + d[u][1]) * a.c_exp2);
        if (i == j) v += a.eps;
        A[i * S + j] = v;
        A[j * S + i] = v;
        if (sa) {
          sa[i * m + j] = v;
          sa[j * m + i] = v;
        }
      }
    }
  }
}

template <int D, int MB>
__device__ void solver_role(const MainArgs& a, int bh, float* smem) {
  using G = NsGeom<MB>;
  constexpr int S = G::SLS, N16 = G::N16;
  float* A = smem;
  float* X0 = smem + G::MAT;
  float* X1 = smem + 2 * G::MAT;
  float* XTB = smem + G::OFF_XTB;
  float* red = smem + G::OFF_RED;
  constexpr int WLS = MP + 4;              // row stride of the W^T copy
  float* WTL = smem + G::SMEM;             // [D][WLS] W^T copy (see below)
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
  const int m = a.m;
  const int r = m > N16 ? m - N16 : 0;  // border width (0 when padded)
  __builtin_amdgcn_s_setprio(3);

  // A = k(L, L) + eps I, built here in LDS.  The landmarks are staged in LDS
  // (over the iterate buffers, which are initialised afterwards; rows up to
  // an even count, padding zero).  Each thread computes a 2 x 2 block (rows 2 bi, 2 bi + 1; columns 2 bj, 2 bj + 1), bi <= bj, of
  // the upper triangle, streaming the four landmark rows; every unordered
  // pair is computed once and written to A[i][j] and A[j][i], so A is exactly
  // symmetric (the border code relies on it).
  constexpr int LDL = D + 4;
  float* Ls = smem + G::MAT;
  const int nb = (m + 1) / 2;
  {
    const float* Lg = a.L + static_cast<size_t>(bh) * m * D;
    for (int e = tid; e < 2 * nb * (D / 4); e += WGM) {
      const int row = e / (D / 4), c4 = e % (D / 4);
      st4(Ls + row * LDL + 4 * c4, row < m ? ld4(Lg + row * D + 4 * c4) : f4{0.f, 0.f, 0.f, 0.f});
    }
    for (int e = tid; e < G::ROWS * S; e += WGM) A[e] = 0.f;
  }
  __syncthreads();
  if (a.kind == 0) build_a<D, 0>(a, bh, Ls, A, S);
  else build_a<D, 1>(a, bh, Ls, A, S);
  __syncthreads();
  // alpha = 1 / (max column abs-sum * max row abs-sum); A is symmetric, so
  // its largest column sum equals its largest row sum.
  if (w == 0) {
    float sum = 0.f;
    if (lane < m) {
      for (int q = 0; q < (m + 3) / 4; ++q) {
        const f4 v = ld4(A + lane * S + 4 * q);  // zero beyond m
        sum += fabsf(v[0]) + fabsf(v[1]) + fabsf(v[2]) + fabsf(v[3]);
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) sum = fmaxf(sum, __shfl_xor(sum, o));
    if (lane == 0) {
      red[0] = sum;
      red[1] = 0.f;  // set once W^T is in LDS
    }
  }
  __syncthreads();
  const float alpha = 1.0f / (red[0] * red[0]);
  // X_0 = alpha A; the second buffer zero (its padding stays zero)
  for (int e = tid; e < G::MAT; e += WGM) {
    X0[e] = alpha * A[e];
    X1[e] = 0.f;
  }
  for (int e = tid; e < 2 * 4 * 64; e += WGM) {
    const int buf = e / 256, bb = (e / 64) % 4, kk = e % 64;
    XTB[e] = (buf == 0 && bb < r && kk < m) ? alpha * A[kk * S + N16 + bb] : 0.f;
  }
  __syncthreads();

  if (w < MB) {
    if constexpr (MB > 0) {
      // the border width is a template argument so that the border code is
      // straight-line
      if (MB < 4 && r == 1) ns_interior_wave<MB, (MB < 4 ? 1 : 0)>(a, smem, w, lane);
      else ns_interior_wave<MB, 0>(a, smem, w, lane);
    }
  } else if (w - MB < r) {
    ns_border_wave<MB>(a, smem, w - MB, lane);
  } else {
    // idle waves; the first one watches for the head's W^T (published by the
    // last key workgroup) during the second half of the steps and copies it
    // to LDS, so that Y can be formed right after the last step.  Each global
    // read is issued before a barrier and consumed after it (a barrier does
    // not wait for global loads), so the watcher never delays the steps.
    const bool watcher = w == MB + r;
    constexpr int NW = D * (MP / 4) / 64;  // float4 of W^T per lane
    const float* wg = a.wt + static_cast<size_t>(bh) * D * MP;
    int state = 0;  // 0 polling, 1 W^T reads in flight, 2 copied
    bool polled = false;
    unsigned cnt = 0u;
    f4 wv[NW];
    for (int t = 0; t < a.iters; ++t) {
      if (watcher) {
        if (state == 1) {
#pragma unroll
          for (int u = 0; u < NW; ++u) {
            const int e = lane + 64 * u, row = e / (MP / 4), c4 = e % (MP / 4);
            st4(WTL + row * WLS + 4 * c4, wv[u]);
          }
          if (lane == 0) red[1] = 1.0f;
          state = 2;
        }
        if (state == 0 && polled && __builtin_amdgcn_readfirstlane(cnt) >= 1u) {
#pragma unroll
          for (int u = 0; u < NW; ++u) {
            const int e = lane + 64 * u, row = e / (MP / 4), c4 = e % (MP / 4);
            wv[u] = ld4(wg + row * MP + 4 * c4);
          }
          state = 1;
        }
        if (state == 0 && 2 * t >= a.iters) {
          if (lane == 0) cnt = __hip_atomic_load(cnt_y(a, bh), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          polled = true;
        }
      }
      __syncthreads();
      asm volatile("" : "+v"(cnt));
    }
    if (watcher && state == 1) {
#pragma unroll
      for (int u = 0; u < NW; ++u) {
        const int e = lane + 64 * u, row = e / (MP / 4), c4 = e % (MP / 4);
        st4(WTL + row * WLS + 4 * c4, wv[u]);
      }
      if (lane == 0) red[1] = 1.0f;
    }
  }
  __syncthreads();  // the W^T copy and its flag are complete

  const float* Xf = (a.iters & 1) ? X1 : X0;
  if (a.st_x) {
    for (int e = tid; e < m * m; e += WGM)
      a.st_x[static_cast<size_t>(bh) * m * m + e] = Xf[(e / m) * S + (e % m)];
  }
  if (red[1] != 0.f) {
    // W^T is already published (its arrival counted) and copied to LDS: this
    // workgroup is the second of (W, X) and forms Y^T from LDS directly
    compute_y<D>(WTL, WLS, Xf, S, G::ROWS, a.yt + static_cast<size_t>(bh) * D * MP);
    raise_flag(flag_y(a, bh));
    return;
  }
  // otherwise publish X and count its arrival
  float* Xg = a.xw + static_cast<size_t>(bh) * MP * MP;
  for (int e = tid; e < MP * MP; e += WGM) {
    const int row = e / MP, col = e % MP;
    st_dev(Xg + e, (row < G::ROWS && col < S) ? Xf[row * S + col] : 0.f);
  }
  arrive_y<D>(a, bh);
}

// ---------------------------------------------------------------------------
// Map role.  Workgroup = one head and S consecutive 64-token tiles of either
// the keys (key role: W partial; also K_QL when Q == K) or the queries (query
// role: K_QL rows).  Wave g computes landmarks [g m / 8, (g+1) m / 8) for the
// 64 tokens of the tile (lane = token); the tile's kernel values meet in LDS.
// ---------------------------------------------------------------------------
// W^T[c][j] = sum of the nP partials in partial order, zero for j >= m; run
// by the last key workgroup of the head.  Thread: 8 elements (stride WGM),
// 8 partials of each in flight.
template <int D>
__device__ void reduce_w(const MainArgs& a, int bh) {
  constexpr int EPT = D * MP / WGM;  // elements per thread
  const int nP = a.nP, m = a.m;
  const size_t ps = static_cast<size_t>(D) * MP;
  const float* pb = a.wpart + static_cast<size_t>(bh) * nP * ps;
  float* wg = a.wt + static_cast<size_t>(bh) * ps;
  const int tid = threadIdx.x;
  float sum[EPT];
#pragma unroll
  for (int u = 0; u < EPT; ++u) sum[u] = 0.f;
  int p = 0;
  for (; p + 8 <= nP; p += 8) {
    float v[EPT][8];
#pragma unroll
    for (int u = 0; u < EPT; ++u)
#pragma unroll
      for (int q = 0; q < 8; ++q) v[u][q] = pb[(p + q) * ps + tid + u * WGM];
#pragma unroll
    for (int u = 0; u < EPT; ++u)
#pragma unroll
      for (int q = 0; q < 8; ++q) sum[u] += v[u][q];
  }
  for (; p < nP; ++p) {
#pragma unroll
    for (int u = 0; u < EPT; ++u) sum[u] += pb[p * ps + tid + u * WGM];
  }
#pragma unroll
  for (int u = 0; u < EPT; ++u) {
    const int e = tid + u * WGM, c = e / MP, j = e % MP;
    const float w = j < m ? sum[u] : 0.f;
    st_dev(wg + e, w);
    if (a.st_w && j < m) a.st_w[(static_cast<size_t>(bh) * m + j) * D + c] = w;
  }
}

// O rows of one 64-token tile: K_QL tile (PT, LDS, zero beyond m) times Y
// (rows of Y^T from global memory) on fp32 MFMA.  Wave w: tokens
// 16 (w % 4) .. +15, column blocks w / 4, w / 4 + 2, ...
template <int D>
__device__ void out_tile(const MainArgs& a, int bh, int t, const float* PT) {
  constexpr int CBN = D / 16;
  const int lane = threadIdx.x & 63, w = wave_id();
  const int lr = lane & 15, lg = lane >> 4;
  const int tb = w & 3, ch = w >> 2;
  const float* yg = a.yt + static_cast<size_t>(bh) * D * MP;
  f4 av[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) av[q] = ld4(PT + (16 * tb + lr) * LS + 16 * lg + 4 * q);
#pragma unroll
  for (int cb = ch; cb < CBN; cb += 2) {
    const float* br = yg + (16 * cb + lr) * MP + 16 * lg;
    f4 bv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) bv[q] = ld4(br + 4 * q);
    f4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int h = 0; h < 4; ++h) c = mfma4(av[q][h], bv[q][h], c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = t * TILE + 16 * tb + 4 * lg + i;
      if (n < a.N) {
        const size_t o = (static_cast<size_t>(bh) * a.N + n) * D + 16 * cb + lr;
        if (a.bf16) static_cast<uint16_t*>(a.out)[o] = f32_to_bf16_rne(c[i]);
        else static_cast<float*>(a.out)[o] = c[i];
      }
    }
  }
}

// Squared-L2 kernel values of one 64-token tile against every landmark, with
// the distance recast as |x|^2 + |l|^2 - 2 x.l and x.l on fp32 MFMA (clamped
// at zero: the expanded form can round slightly below it).  Wave w computes
// the 16x16 blocks (tokens 16 (w % 4) .., landmarks 16 jb ..) for
// jb = w / 4, w / 4 + 2; lane (g, r) supplies coordinates
// (D/4) g .. (D/4) g + D/4 - 1 of token / landmark r of its blocks, read
// straight from global memory.  Writes PTt[token][j] and, for key tiles,
// PJ[j][token]; landmarks j in [m, 16 ceil(m/16)) get exact zeros.
template <int D, bool BF16>
__device__ void gauss_tile(const MainArgs& a, const void* src, const float* Lh, int bh, int t,
                           float* PTt, float* PJ, float* xx, bool key_role) {
  constexpr int KS = D / 4;  // MFMA sub-steps; floats per lane per operand
  const int lane = threadIdx.x & 63, w = wave_id();
  const int lr = lane & 15, lg = lane >> 4;
  const int tb = w & 3;
  const int m = a.m, N = a.N;
  const int mby = (m + 15) >> 4;
  // token operand: KS coordinates of token 16 tb + lr
  const int n = t * TILE + 16 * tb + lr;
  const size_t row = static_cast<size_t>(bh) * N + (n < N ? n : N - 1);
  float av[KS];
#pragma unroll
  for (int q = 0; q < KS / 4; ++q) {
    const f4 u = load4_io(src, row * D + KS * lg + 4 * q, BF16);
    av[4 * q] = u[0];
    av[4 * q + 1] = u[1];
    av[4 * q + 2] = u[2];
    av[4 * q + 3] = u[3];
  }
  float px = 0.f;
#pragma unroll
  for (int s = 0; s < KS; ++s) px = fmaf(av[s], av[s], px);
  px = sum_over_g(px);
  if (w < 4 && lg == 0) xx[16 * tb + lr] = px;
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int jb = (w >> 2) + 2 * h;
    if (jb < mby) {
      const int j = 16 * jb + lr;
      float bv[KS];
#pragma unroll
      for (int q = 0; q < KS / 4; ++q) {
        const f4 u = j < m ? ld4(Lh + j * D + KS * lg + 4 * q) : f4{0.f, 0.f, 0.f, 0.f};
        bv[4 * q] = u[0];
        bv[4 * q + 1] = u[1];
        bv[4 * q + 2] = u[2];
        bv[4 * q + 3] = u[3];
      }
      float pl = 0.f;
#pragma unroll
      for (int s = 0; s < KS; ++s) pl = fmaf(bv[s], bv[s], pl);
      pl = sum_over_g(pl);
      f4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) c = mfma4(av[s], bv[s], c);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tt = 16 * tb + 4 * lg + i;
        const float d = fmaxf(fmaf(-2.0f, c[i], xx[tt] + pl), 0.0f);
        const float kv = (j < m && t * TILE + tt < N) ? exp2f(d * a.c_exp2) : 0.f;
        PTt[tt * LS + j] = kv;
        if (key_role) PJ[j * LS + tt] = kv;
      }
    }
  }
}

template <int D, int KIND, bool BF16>
__device__ void map_role(const MainArgs& a, const void* __restrict__ q, const void* __restrict__ k,
                         const void* __restrict__ v, const float* __restrict__ Lw, int b,
                         float* smem) {
  constexpr int CBN = D / 16;
  float* PJ = smem;                // [64 landmarks][LS]: P[j][token]
  float* PT = smem + MP * LS;      // [64 tokens][LS]:    P[j] of token at [token][j]
  float* VT = smem + 2 * MP * LS;  // [D][LS]:            V[token][c] at [c][token]
  float* xx = smem + 3 * MP * LS;  // [64]: squared norms of a tile's tokens (Gaussian)
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
  const int lr = lane & 15, lg = lane >> 4;
  const int m = a.m, N = a.N;
  const int nK = a.nP;
  // Workgroups are dispatched round-robin over the 8 XCDs.  When the heads
  // divide evenly, renumber so that XCD x (= b % 8) works through heads
  // x, x + 8, ... in order: each XCD's L2 and scalar caches then hold the
  // landmarks of only 1/8 of the heads.
  if (a.BH % 8 == 0) {
    const int per_head = nK + a.nQ;
    const int per_xcd = (a.BH / 8) * per_head;
    const int x = b % 8, i = b / 8;
    const int hh = i / per_head, u = i % per_head;  // head slot within the XCD, unit
    const int head = 8 * hh + x;
    b = u < nK ? head * nK + u : a.BH * nK + head * a.nQ + (u - nK);
    (void)per_xcd;
  }
  const bool key_role = b < a.BH * nK;
  int bh, t_beg, t_end;
  if (key_role) {
    bh = b / nK;
    const int kw = b % nK;
    t_beg = kw * a.S;
    t_end = min(t_beg + a.S, a.nT);
  } else {
    // QT tiles per query workgroup (their K_QL rows stay in LDS until Y is
    // ready, in PT and in the V^T area, which query tiles do not use)
    const int bq = b - a.BH * nK;
    bh = bq / a.nQ;
    t_beg = QT * (bq % a.nQ);
    t_end = min(t_beg + QT, a.nT);
  }
  // K_QL goes to global memory only when Q == K (the output launch reads
  // it); query tiles keep theirs in LDS and form their output rows here.
  const bool store_kql = key_role ? a.shared_qk != 0 : a.out_in_main == 0;
  const bool stage_kql = a.st_kql && (!key_role || a.shared_qk);
  const void* src = key_role ? k : q;
  const int mby = (m + 15) >> 4;
  const int nwb = CBN * mby;  // W output blocks

  // padding rows / columns j in [m, 64) stay zero for the whole workgroup
  for (int e = tid; e < MP * LS; e += WGM) {
    PJ[e] = 0.f;
    PT[e] = 0.f;
    if (!key_role) VT[e] = 0.f;
  }
  __syncthreads();

  const int jb = (w * m) / NGRP, je = ((w + 1) * m) / NGRP;
  const float* Lh = Lw + static_cast<size_t>(bh) * m * D;
  f4 wacc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};

  for (int t = t_beg; t < t_end; ++t) {
    float* PTt = (key_role || t == t_beg) ? PT : VT;  // this tile's K_QL rows
    const int n = t * TILE + lane;
    const bool valid = n < N;
    float x[KIND == 0 ? D : 1];
    if constexpr (KIND == 0) load_row<D>(src, static_cast<size_t>(bh) * N + (valid ? n : N - 1), BF16, x);
    if (key_role) {
      // V tile -> VT[c][token]; thread (c, group of TPT tokens); all loads
      // are issued before the LDS writes (rows past N are clamped, then zeroed)
      const int c = tid % D, tg = tid / D;
      constexpr int TPT = TILE * D / WGM;
      float vv[TPT];
#pragma unroll
      for (int u = 0; u < TPT; ++u) {
        const int nv = t * TILE + tg * TPT + u;
        vv[u] = load1_io(v, (static_cast<size_t>(bh) * N + (nv < N ? nv : N - 1)) * D + c, BF16);
      }
#pragma unroll
      for (int u = 0; u < TPT; ++u) {
        const int tok = tg * TPT + u;
        VT[c * LS + tok] = t * TILE + tok < N ? vv[u] : 0.f;
      }
    }
    if constexpr (KIND == 0) {
      // L1 distances on VALU: landmarks two at a time (their scalar loads
      // overlap); an odd last landmark is paired with itself and stored once
      for (int j = jb; j < je; j += 2) {
        const int j1 = j + 1 < je ? j + 1 : j;
        float d0, d1;
        dist_to2<D, KIND>(x, Lh + j * D, Lh + j1 * D, d0, d1);
        const float k0 = valid ? exp2f(d0 * a.c_exp2) : 0.f;
        const float k1 = valid ? exp2f(d1 * a.c_exp2) : 0.f;
        if (key_role) {
          PJ[j * LS + lane] = k0;
          PJ[j1 * LS + lane] = k1;
        }
        PTt[lane * LS + j] = k0;
        PTt[lane * LS + j1] = k1;
      }
    } else {
      gauss_tile<D, BF16>(a, src, Lh, bh, t, PTt, PJ, xx, key_role);
    }
    __syncthreads();
    if (store_kql) {
      // 64 rows of mpad floats, contiguous in global memory
      const int q4 = a.mpad / 4;
      float* dst = a.kql + (static_cast<size_t>(bh) * N + t * TILE) * a.mpad;
      for (int e = tid; e < TILE * q4; e += WGM) {
        const int tok = e / q4, c4 = e % q4;
        if (t * TILE + tok < N) st4(dst + tok * a.mpad + 4 * c4, ld4(PTt + tok * LS + 4 * c4));
      }
    }
    if (stage_kql) {
      for (int e = tid; e < TILE * m; e += WGM) {
        const int tok = e / m, j = e % m;
        if (t * TILE + tok < N)
          a.st_kql[(static_cast<size_t>(bh) * N + t * TILE + tok) * m + j] = PTt[tok * LS + j];
      }
    }
    if (key_role) {
      if (a.st_klk) {
        for (int e = tid; e < m * TILE; e += WGM) {
          const int j = e / TILE, tok = e % TILE;
          if (t * TILE + tok < N)
            a.st_klk[(static_cast<size_t>(bh) * m + j) * N + t * TILE + tok] = PJ[j * LS + tok];
        }
      }
      // W^T[c][j] += sum_token V^T[c][token] P[j][token]
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int blk = w + 8 * s;
        if (blk < nwb) {
          const int cb = blk % CBN, jbk = blk / CBN;
          const float* ar = VT + (16 * cb + lr) * LS + 16 * lg;
          const float* br = PJ + (16 * jbk + lr) * LS + 16 * lg;
          f4 c = wacc[s];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f4 a4 = ld4(ar + 4 * q), b4 = ld4(br + 4 * q);
            c = mfma4(a4[0], b4[0], c);
            c = mfma4(a4[1], b4[1], c);
            c = mfma4(a4[2], b4[2], c);
            c = mfma4(a4[3], b4[3], c);
          }
          wacc[s] = c;
        }
      }
    }
    __syncthreads();
  }
  if (!key_role) {
    if (!a.out_in_main) return;  // K_QL stored; the output launch forms O
    // the tiles' K_QL rows are still in LDS: wait for Y of the head
    wait_flag(flag_y(a, bh), a.sync);
    out_tile<D>(a, bh, t_beg, PT);
    if (t_beg + 1 < t_end) out_tile<D>(a, bh, t_beg + 1, VT);
    return;
  }

  const int kw = b % nK;
  float* part = a.wpart + (static_cast<size_t>(bh) * nK + kw) * D * MP;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int blk = w + 8 * s;
    if (blk < nwb) {
      const int cb = blk % CBN, jbk = blk / CBN;
#pragma unroll
      for (int i = 0; i < 4; ++i) st_dev(part + (16 * cb + 4 * lg + i) * MP + 16 * jbk + lr, wacc[s][i]);
    }
  }
  // the last key workgroup of the head reduces the partials
  if (publish_arrive(cnt_w(a, bh)) == static_cast<unsigned>(nK - 1)) {
    reduce_w<D>(a, bh);
    arrive_y<D>(a, bh);
  }
}

// Read-only inputs are separate __restrict__ parameters so that wave-uniform
// reads of them (the landmark coordinates) compile to scalar loads.
template <int D, int MB>
__global__ __launch_bounds__(WGM) void main_kernel(MainArgs a, const void* __restrict__ q,
                                                    const void* __restrict__ k,
                                                    const void* __restrict__ v,
                                                    const float* __restrict__ L) {
  constexpr int MAP_SMEM = 3 * MP * LS + TILE;
  // solver: the Newton-Schulz layout plus a W^T copy; landmark staging
  // while A is built
  constexpr int SOLVER_A = NsGeom<MB>::SMEM + D * (MP + 4);
  constexpr int SOLVER_B = NsGeom<MB>::MAT + MP * (D + 4);
  constexpr int SOLVER_SMEM = SOLVER_A > SOLVER_B ? SOLVER_A : SOLVER_B;
  __shared__ __attribute__((aligned(16)))
  float smem[MAP_SMEM > SOLVER_SMEM ? MAP_SMEM : SOLVER_SMEM];
  const int b = blockIdx.x;
  if (b < a.ns_blocks) {
    solver_role<D, MB>(a, b, smem);
  } else {
    const int mb = b - a.ns_blocks;
    if (a.kind == 0) {
      if (a.bf16) map_role<D, 0, true>(a, q, k, v, L, mb, smem);
      else map_role<D, 0, false>(a, q, k, v, L, mb, smem);
    } else {
      if (a.bf16) map_role<D, 1, true>(a, q, k, v, L, mb, smem);
      else map_role<D, 1, false>(a, q, k, v, L, mb, smem);
    }
  }
}

// ---------------------------------------------------------------------------
// pool: one workgroup per (landmark, head).  Thread (g, c4) sums a float4
// column chunk over every G-th token of the window (loads issued 4 at a
// time); a fixed-order LDS reduction over g finishes the mean.
// ---------------------------------------------------------------------------
template <int D, bool BF16>
__global__ __launch_bounds__(WGS) void pool_kernel(const void* __restrict__ K,
                                                   float* __restrict__ L,
                                                   float* __restrict__ st_L,
                                                   unsigned* __restrict__ sync, int gw, int ph,
                                                   int pw, int m, int N) {
  constexpr int C4 = D / 4;
  constexpr int G = WGS / C4;
  constexpr int U = 4;  // loads in flight per thread
  __shared__ f4 part[WGS];
  const int j = blockIdx.x, bh = blockIdx.y;
  const int tid = threadIdx.x, c4 = tid % C4, g = tid / C4;
  // hand-off words of the main launch start at zero every call
  if (j == 0 && tid == 0) {
    const int BH = gridDim.y;
    sync[4 + bh] = 0u;
    sync[4 + BH + bh] = 0u;
    sync[4 + 2 * BH + bh] = 0u;
    if (bh == 0) sync[0] = 0u;
  }
  const int mw = gw / pw;
  const int R = j / mw, C = j % mw;
  const int cnt = ph * pw;
  const size_t base = static_cast<size_t>(bh) * N;
  f4 s = {0.f, 0.f, 0.f, 0.f};
  for (int t0 = g; t0 < cnt; t0 += U * G) {
    f4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // tokens past the window are clamped to its first token and dropped below
      const int t = t0 + u * G < cnt ? t0 + u * G : 0;
      const int n = (R * ph + t / pw) * gw + C * pw + t % pw;
      v[u] = load4_io(K, (base + n) * D + 4 * c4, BF16);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (t0 + u * G < cnt) s += v[u];
  }
  part[tid] = s;
  __syncthreads();
  if (tid < C4) {
    f4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < G; ++i) acc += part[i * C4 + tid];
    const f4 mean = acc / static_cast<float>(cnt);
    float* dst = L + (static_cast<size_t>(bh) * m + j) * D + 4 * tid;
    st4(dst, mean);
    if (st_L) st4(st_L + (static_cast<size_t>(bh) * m + j) * D + 4 * tid, mean);
  }
}

// ---------------------------------------------------------------------------
// out: O = K_QL Y.  Workgroup = (head, 64 tokens); wave w computes tokens
// 16w..16w+15 of the tile against all D columns, contraction over KS*4 =
// 16 ceil(m/16) landmarks (zero padded).
// ---------------------------------------------------------------------------
template <int D, int KS>
__global__ __launch_bounds__(WGS) void out_kernel(const float* __restrict__ kql,
                                                  const float* __restrict__ yt,
                                                  void* __restrict__ O, int bf16, int N,
                                                  int mpad, int nT) {
  constexpr int CBN = D / 16;
  const int bh = blockIdx.x / nT, t = blockIdx.x % nT;
  const int lane = threadIdx.x & 63, w = wave_id();
  const int lr = lane & 15, lg = lane >> 4;
  const int tok = t * TILE + 16 * w + lr;
  const int tokc = tok < N ? tok : N - 1;
  const float* ar = kql + (static_cast<size_t>(bh) * N + tokc) * mpad + KS * lg;
  float av[KS];
#pragma unroll
  for (int q = 0; q < KS / 4; ++q) {
    const f4 u = ld4(ar + 4 * q);
    av[4 * q] = u[0];
    av[4 * q + 1] = u[1];
    av[4 * q + 2] = u[2];
    av[4 * q + 3] = u[3];
  }
  f4 acc[CBN];
#pragma unroll
  for (int cb = 0; cb < CBN; ++cb) {
    const float* br = yt + (static_cast<size_t>(bh) * D + 16 * cb + lr) * MP + KS * lg;
    f4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < KS / 4; ++q) {
      const f4 b4 = ld4(br + 4 * q);
      c = mfma4(av[4 * q], b4[0], c);
      c = mfma4(av[4 * q + 1], b4[1], c);
      c = mfma4(av[4 * q + 2], b4[2], c);
      c = mfma4(av[4 * q + 3], b4[3], c);
    }
    acc[cb] = c;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int n = t * TILE + 16 * w + 4 * lg + i;
    if (n < N) {
      const size_t o = (static_cast<size_t>(bh) * N + n) * D + lr;
#pragma unroll
      for (int cb = 0; cb < CBN; ++cb) {
        if (bf16) {
          static_cast<uint16_t*>(O)[o + 16 * cb] = f32_to_bf16_rne(acc[cb][i]);
        } else {
          static_cast<float*>(O)[o + 16 * cb] = acc[cb][i];
        }
      }
    }
  }
}

// Launches kernel `k` with arguments converted to its parameter types,
// through hipExtLaunchKernel so that optional events time the kernel itself;
// returns the launch status.
template <typename... P, typename... A, size_t... I>
hipError_t launch_impl(void (*k)(P...), dim3 grid, dim3 block, hipStream_t s, Ev ev,
                       std::index_sequence<I...>, A&&... a) {
  std::tuple<P...> t(std::forward<A>(a)...);
  void* ptrs[sizeof...(P) > 0 ? sizeof...(P) : 1] = {static_cast<void*>(&std::get<I>(t))...};
  return hipExtLaunchKernel(reinterpret_cast<const void*>(k), grid, block, ptrs, 0, s, ev.start,
                            ev.stop, 0);
}

template <typename... P, typename... A>
hipError_t launch(void (*k)(P...), dim3 grid, dim3 block, hipStream_t s, Ev ev, A&&... a) {
  static_assert(sizeof...(P) == sizeof...(A), "kernel argument count");
  return launch_impl(k, grid, block, s, ev, std::index_sequence_for<P...>{},
                     std::forward<A>(a)...);
}

inline float exp2_scale(float lambda) {
  // exp(-d / lambda) = exp2(d * (-log2(e) / lambda))
  return static_cast<float>(-1.4426950408889634 / static_cast<double>(lambda));
}

template <int D>
hipError_t launch_pool_d(const Plan& p, const Args& a, const Buffers& b, hipStream_t s, Ev ev) {
  const dim3 grid(p.m, p.BH);
  if (p.bf16)
    return launch(pool_kernel<D, true>, grid, dim3(WGS), s, ev, a.k, b.L, a.st_L, b.sync, p.gw,
                  p.ph, p.pw, p.m, p.N);
  return launch(pool_kernel<D, false>, grid, dim3(WGS), s, ev, a.k, b.L, a.st_L, b.sync, p.gw,
                p.ph, p.pw, p.m, p.N);
}

template <int D, int MB>
hipError_t launch_main_dm(const MainArgs& ma, unsigned grid, hipStream_t s, Ev ev) {
  return launch(main_kernel<D, MB>, dim3(grid), dim3(WGM), s, ev, ma, ma.q, ma.k, ma.v, ma.L);
}

template <int D>
hipError_t launch_main_d(const Plan& p, const MainArgs& ma, unsigned grid, hipStream_t s, Ev ev) {
  switch (p.ns_mb) {
    case 0: return launch_main_dm<D, 0>(ma, grid, s, ev);
    case 1: return launch_main_dm<D, 1>(ma, grid, s, ev);
    case 2: return launch_main_dm<D, 2>(ma, grid, s, ev);
    case 3: return launch_main_dm<D, 3>(ma, grid, s, ev);
    case 4: return launch_main_dm<D, 4>(ma, grid, s, ev);
  }
  return hipErrorInvalidValue;
}

template <int D>
hipError_t launch_out_d(const Plan& p, const Args& a, const Buffers& b, hipStream_t s, Ev ev) {
  const dim3 grid(p.BH * p.nT);
  switch (p.mpad / 16) {
    case 1:
      return launch(out_kernel<D, 4>, grid, dim3(WGS), s, ev, b.kql, b.yt, a.out, p.bf16, p.N,
                    p.mpad, p.nT);
    case 2:
      return launch(out_kernel<D, 8>, grid, dim3(WGS), s, ev, b.kql, b.yt, a.out, p.bf16, p.N,
                    p.mpad, p.nT);
    case 3:
      return launch(out_kernel<D, 12>, grid, dim3(WGS), s, ev, b.kql, b.yt, a.out, p.bf16, p.N,
                    p.mpad, p.nT);
    default:
      return launch(out_kernel<D, 16>, grid, dim3(WGS), s, ev, b.kql, b.yt, a.out, p.bf16, p.N,
                    p.mpad, p.nT);
  }
}

}  // namespace

bool out_in_main_launch(const Plan& p, int shared_qk) {
  // 256 CUs x 2 main-kernel workgroups (LDS and registers allow two), with
  // some margin
  constexpr long kResident = 448;
  if (shared_qk) return false;
  const long nQ = (p.nT + QT - 1) / QT;
  return static_cast<long>(p.BH) * (1 + p.nP + nQ) <= kResident;
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
  ma.nQ = a.shared_qk ? 0 : (p.nT + QT - 1) / QT;
  ma.kind = p.kernel;
  ma.bf16 = p.bf16;
  ma.iters = a.iters;
  ma.c_exp2 = exp2_scale(a.lambda);
  ma.eps = a.eps;
  ma.ns_blocks = with_solver ? p.BH : 0;
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

hipError_t launch_out(const Plan& p, const Args& a, const Buffers& b, hipStream_t s, Ev ev) {
  switch (p.D) {
    case 16: return launch_out_d<16>(p, a, b, s, ev);
    case 32: return launch_out_d<32>(p, a, b, s, ev);
    case 64: return launch_out_d<64>(p, a, b, s, ev);
  }
  return hipErrorInvalidValue;
}

}  // namespace lapattn
