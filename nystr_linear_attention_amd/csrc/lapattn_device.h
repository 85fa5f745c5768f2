// Device code shared by the forward and backward kernels: I/O helpers, the
// Newton-Schulz solver role, the kernel-map role, and the hand-off words of
// the role-split launches.  Included by one translation unit each; everything
// lives in an anonymous namespace.
//
// MFMA operand convention: for an output block D[16][16] += sum_k A[i][k]
// B[k][j], lane l = 16*g + r supplies A[r][k] and B[k][r] for the k values of
// lane group g (v_mfma_f32_16x16x4f32: k = KS*g + s at sub-step s, so each
// lane reads KS contiguous k values of one row of A and one row of B^T;
// 16x16x32 fp16: 8 k values per instruction, assigned per use below).  The
// accumulator holds D[4g + i][r], i = 0..3.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>
#include <type_traits>
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
constexpr int QT = kQueryTiles;  // 64-token tiles per query workgroup

__device__ __forceinline__ f4 mfma4(float a, float b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// 2^x on the hardware exponential.  Kernel values are exp2 of
// -dist / lambda * log2(e) <= 0; for arguments down to -126 this is exactly
// what exp2f returns (exp2f adds only a rescaling for results below the
// normal range, ~1e-38, where the map value is zero for any purpose here).
__device__ __forceinline__ float exp2_map(float x) { return __builtin_amdgcn_exp2f(x); }

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
  unsigned* sync;     // hand-off words, zeroed by the pool launch; head bh
                      // owns the kSyncHead words from kSyncHead (bh + 1)
                      // (see below)
  unsigned* timeouts; // counts bounded waits that timed out (zeroed by the
                      // pool launch)
  float* st_a;
  float* st_x;
  float* st_kql;
  float* st_klk;
  float* st_w;
  int N, m, BH, nT, S, nP, mpad;
  int ns_blocks;      // solver workgroups in the launch (0 or BH)
  int tickets;        // roles come from per-queue tickets (else workgroup b
                      // of a solver-only launch solves head b)
  int nq;             // ticket queues (8 when 8 divides BH, else min(BH, 8))
  int nQ;             // query workgroups per head, qt tiles each (0 when Q == K)
  int qt;             // tiles per query workgroup (QT when the output rows are
                      // formed here, which keeps the K_QL rows in LDS)
  int shared_qk;      // Q and K are the same tensor
  int out_in_main;    // query workgroups wait for Y and write O (else they
                      // store K_QL and the output launch forms O)
  int kind, bf16, iters;
  float c_exp2, eps;
  int partials_only;  // key units store their W^T partial and stop (the
                      // backward pass reduces the partials in a later launch)
};

// ---------------------------------------------------------------------------
// Hand-offs inside the main launch.  Per head, the key workgroups publish
// W^T partials and the solver workgroup publishes X.  Then either
//  - (query workgroups form the output rows here) each key workgroup raises
//    its own ready flag; query workgroup u < R reduces lines [u LPS, ..) of
//    W^T (fixed partial order, so the result does not depend on timing) and
//    raises its slice flag; every query workgroup waits for all slices and
//    X, forms Y^T = W^T X^T in its LDS and writes its output rows; or
//  - (the output launch forms O) the key workgroups count their arrivals;
//    the last one reduces the partials (same order) and publishes W^T.  W^T
//    and X each count one arrival; whichever is second forms Y^T for the
//    output launch.
// Words of head bh (kSyncHead from kSyncHead (bh + 1), each group on its own
// cache lines): [0, 128) key ready flags, [128, 160) W^T slice flags, [192]
// X ready (its value carries the scale exponent of the published X), [224]
// key arrivals, [225] arrivals of W and X, [226] Y ready, [227] chunks of
// the normalised map's statistics (a later launch).
// Flags are plain device-scope stores (no read-modify-write on a shared word,
// which serialises at memory when many workgroups arrive at once).
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
// Forward progress: see take_role (producers of a head are dispatched, or by
// ticket start, before its consumers).  Every wait is bounded in time
// regardless (it then counts a timeout in *timeouts and goes on), so no wave
// can spin forever.
// ---------------------------------------------------------------------------
constexpr long long kWaitTicks = 2000000;  // 20 ms of the 100 MHz device clock

__device__ __forceinline__ unsigned* head_sync(const MainArgs& a, int bh) {
  return a.sync + kSyncHead * (bh + 1);
}
__device__ __forceinline__ unsigned* key_flags(const MainArgs& a, int bh) { return head_sync(a, bh); }
__device__ __forceinline__ unsigned* slice_flags(const MainArgs& a, int bh) { return head_sync(a, bh) + 128; }
__device__ __forceinline__ unsigned* flag_x(const MainArgs& a, int bh) { return head_sync(a, bh) + 192; }
__device__ __forceinline__ unsigned* cnt_w(const MainArgs& a, int bh) { return head_sync(a, bh) + 224; }
__device__ __forceinline__ unsigned* cnt_y(const MainArgs& a, int bh) { return head_sync(a, bh) + 225; }
__device__ __forceinline__ unsigned* flag_y(const MainArgs& a, int bh) { return head_sync(a, bh) + 226; }
// word of head bh counting the chunks of the normalised map's statistics
constexpr int kNormCount = 227;
// word of head bh counting the slices of the backward's head reduction
constexpr int kBwdHeadCount = 228;

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

// Completes this workgroup's device-scope stores, then sets *flag to v.
__device__ __forceinline__ void raise_flag(unsigned* flag, unsigned v = 1u) {
  drain_stores();
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_store(flag, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Waits until *flag is nonzero (bounded in time: then counts a timeout and
// goes on); returns the value seen, in every thread.
__device__ __forceinline__ unsigned wait_flag(unsigned* flag, unsigned* timeouts) {
  __shared__ unsigned seen;
  if (threadIdx.x == 0) {
    const long long t0 = wall_clock64();
    unsigned v;
    while ((v = __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) == 0u) {
      if (wall_clock64() - t0 > kWaitTicks) {
        __hip_atomic_fetch_add(timeouts, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    seen = v;
  }
  __syncthreads();
  return seen;
}

// Waits until flags[0 .. n) (n <= 128) are all set: lane l of wave 0 polls
// words l and l + 64; bounded in time like wait_flag.
__device__ __forceinline__ void wait_flags(const unsigned* flags, int n, unsigned* timeouts) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    bool d0 = lane >= n, d1 = lane + 64 >= n;
    const long long t0 = wall_clock64();
    while (true) {
      if (!d0) d0 = __hip_atomic_load(flags + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u;
      if (!d1) d1 = __hip_atomic_load(flags + lane + 64, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u;
      if (__all(d0 && d1)) break;
      if (wall_clock64() - t0 > kWaitTicks) {
        if (lane == 0) __hip_atomic_fetch_add(timeouts, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  __syncthreads();
}

// Y^T = W^T X^T for one head on fp32 MFMA, D x 64 outputs (columns >= m are
// zero because X is zero padded).  W^T rows have stride wts; X has xrows
// rows of stride xs (columns >= xcols and rows >= xrows read as zero), so the
// operands may come from global memory or from the solver's LDS: the same
// values in the same MFMA order give the same Y^T either way.  The result
// goes to global memory (device-scope stores, row stride MP).
template <int D>
__device__ void compute_y(const float* wt, int wts, const float* x, int xs, int xrows, int xcols,
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
        bv[q] = (xr < xrows && c0 < xcols) ? ld4(x + xr * xs + c0) : f4{0.f, 0.f, 0.f, 0.f};
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
               a.xw + static_cast<size_t>(bh) * MP * MP, MP, MP, MP,
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
// Both products are full and unsymmetrised: forcing the iterates symmetric
// turns the quadratic error contraction of the Newton step into a linear map
// with gain up to (1 + cond(A)) / 2, which diverges near convergence for
// ill-conditioned A.
//
// The m x m problem is zero padded to n = 16 MB, MB = ceil(m / 16).  The
// padding rows and columns of A, and so of X_0 = alpha A and of every later
// iterate, are zero, and the leading m x m block evolves exactly as the
// unpadded iteration.
//
// Products run on fp16 MFMA (16x16x32, fp32 accumulation) with each operand
// split in two: x = hi + lo, hi = fp16(x), lo = fp16(x - hi), both rounded
// to nearest, after scaling by a power of two that keeps every entry inside
// fp16 range.  A product is formed as hi hi + lo hi + hi lo: about 22
// significant bits per operand (fp32 has 24) at a quarter of the matrix-core
// cycles of fp32 MFMA.  The scales are exact powers of two, removed from the
// fp32 accumulators:
//   A   : 2^eA with max|A| 2^eA < 2^14;
//   T   : 2^14.  T = A X_t is a polynomial in A with eigenvalues in (0, 1]
//         (mu -> 2 mu - mu^2 from mu = alpha lambda^2 <= 1), so |T_ij| <= 1;
//   X_t : 2^e_t, shared by the workgroup, with max|X_{t-2}| 2^e_t < 2^7 (the
//         column-block maxima are published in LDS).  X_t is positive
//         semi-definite with spectral norm at most twice that of X_{t-1}, and
//         max|X| >= ||X||_2 / n, so max|X_t| 2^e_t < 4 n 2^7 <= 2^15 for
//         n <= 64: no overflow.
//
// Wave c < MB owns column block c (16 columns) of X_t, of T = A X_t and of
// X_{t+1}:
//   T[:, c]       = A X_t[:, c]              (needs only its own X columns)
//   X_{t+1}[:, c] = 2 X_t[:, c] - X_t T[:, c] (needs the rows of X_t)
// Chunk p of the contraction covers 16-row blocks 2p and 2p + 1: slot s of
// lane (g, lr) takes k = 16 (2p + s / 4) + 4 g + s % 4.  The accumulators of
// blocks 2p and 2p + 1 (lane (g, lr) holds rows 4 g + j of column lr) are then
// exactly the B operand, so X_t[:, c] and T[:, c] stay in registers, in fp32
// and split.  The A operands (rows of A, rows of X_t) come from half-precision
// arrays in LDS whose columns are permuted (hpos) so that a lane's 8 values
// are one 16-byte read.  Only X_t is exchanged, once per step: one barrier
// per step.
// ---------------------------------------------------------------------------
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f4 mfma_h(u32x4 a, u32x4 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, a), __builtin_bit_cast(h8, b),
                                                 c, 0, 0, 0);
}

// Two values into packed fp16 high parts and packed fp16 remainders.
__device__ __forceinline__ void split2(float x0, float x1, unsigned& hi, unsigned& lo) {
  const h2 h = __builtin_convertvector(f2{x0, x1}, h2);
  const float r0 = x0 - static_cast<float>(h[0]);
  const float r1 = x1 - static_cast<float>(h[1]);
  hi = __builtin_bit_cast(unsigned, h);
  lo = __builtin_bit_cast(unsigned, __builtin_convertvector(f2{r0, r1}, h2));
}

// split2 with the remainders formed in fp32 by mixed-precision FMAs,
// r = fma(x, one, -hi) with hi in fp16 (exact, as x - hi is), then one
// packed conversion: the same bits as split2 in 4 instructions instead of
// 6.  `one` must be 1.0 in a register (a literal lets the compiler fold the
// FMA back into a conversion and a subtraction).
__device__ __forceinline__ void split2_mix(float x0, float x1, float one, unsigned& hi, unsigned& lo) {
  const h2 h = __builtin_convertvector(f2{x0, x1}, h2);
  const float r0 = __builtin_fmaf(x0, one, -static_cast<float>(h[0]));
  const float r1 = __builtin_fmaf(x1, one, -static_cast<float>(h[1]));
  hi = __builtin_bit_cast(unsigned, h);
  lo = __builtin_bit_cast(unsigned, __builtin_convertvector(f2{r0, r1}, h2));
}

// 1.0 in a register the compiler cannot see through (for split2_mix).
__device__ __forceinline__ float opaque_one() {
  float one = 1.0f;
  asm("" : "+v"(one));
  return one;
}

// Sum over the 4 lanes (g = 0..3) that share lr, on VALU: a lane-half swap
// with itself leaves v[l] + v[l ^ 32] as the sum of the two results (and
// likewise for 16-lane rows).
__device__ __forceinline__ float sum_over_g(float v) {
  const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(h[0]) + __uint_as_float(h[1]);
  const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// Eight consecutive values (two float4), scaled by 2^e, into one fp16
// operand pair (hi, lo).
__device__ __forceinline__ void split8h(f4 a, f4 b, int e, u32x4& hi, u32x4& lo) {
  unsigned h[4], l[4];
  split2(ldexpf(a[0], e), ldexpf(a[1], e), h[0], l[0]);
  split2(ldexpf(a[2], e), ldexpf(a[3], e), h[1], l[1]);
  split2(ldexpf(b[0], e), ldexpf(b[1], e), h[2], l[2]);
  split2(ldexpf(b[2], e), ldexpf(b[3], e), h[3], l[3]);
  hi = u32x4{h[0], h[1], h[2], h[3]};
  lo = u32x4{l[0], l[1], l[2], l[3]};
}

// Maximum of non-negative v over the 8 lanes of an aligned 8-lane group, in
// every lane of the group; magnitudes compare as unsigned bit patterns.
__device__ __forceinline__ unsigned max8_u(unsigned v) {
  v = max(v, static_cast<unsigned>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0xB1, 0xF, 0xF, false)));
  v = max(v, static_cast<unsigned>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x4E, 0xF, 0xF, false)));
  return max(v, static_cast<unsigned>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x141, 0xF, 0xF, false)));
}

// Exponent e with max 2^e < 2^15 (0 for max = 0).
__device__ __forceinline__ int fp16_scale(float mx) {
  return mx > 0.f ? 15 - __builtin_amdgcn_frexp_expf(mx) : 0;
}

// Maximum over the 64 lanes of a wave, in every lane.
__device__ __forceinline__ unsigned wave_max_u(unsigned v) {
  const auto h = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  v = max(h[0], h[1]);
  const auto q = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = max(q[0], q[1]);
  v = max(v, static_cast<unsigned>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0xB1, 0xF, 0xF, false)));
  v = max(v, static_cast<unsigned>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x4E, 0xF, 0xF, false)));
  v = max(v, static_cast<unsigned>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x141, 0xF, 0xF, false)));
  v = max(v, static_cast<unsigned>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x140, 0xF, 0xF, false)));
  return v;
}

template <int MB, int D>
struct NsGeom {
  static constexpr int N16 = 16 * MB;          // padded size
  static constexpr int NC = (MB + 1) / 2;      // 32-wide contraction chunks
  static constexpr bool ODD = (MB & 1) != 0;   // the last chunk holds one block
  // A in half precision, row major: N16 rows of RSW 32-bit words, columns
  // permuted (hpos).  RSW / 4 is odd, so the 16-byte reads of 16
  // consecutive rows fall on distinct bank groups.
  static constexpr int RSW = 8 * MB + 4;
  static constexpr int RSH = 2 * RSW;          // row stride in halves
  static constexpr int ARR = N16 * RSW;        // words per array
  // X_t in half precision, column major: line k holds X_t[0..N16)[k] in
  // 8-byte chunks of 4 rows, chunk c of line k stored at position
  // c ^ ((k >> 2) & 3) (xchunk); lines of XSW words (8 mod 32).  The reads of
  // 4 chunks of 4 lines per 16 lanes and the writes of one chunk of 16
  // consecutive lines per 16 lanes then both fall on distinct banks (without
  // the swizzle the writes were 4-way bank conflicts).
  static constexpr int XSW = 40;
  static constexpr int XSH = 2 * XSW;          // line stride in halves
  static constexpr int XARR = N16 * XSW;       // words per array
  static constexpr int SX = N16 + 4;           // fp32 row stride (A while set up, final X)
  static constexpr int OFF_AH = 0;             // A hi, A lo
  static constexpr int OFF_AL = ARR;
  static constexpr int OFF_X = 2 * ARR;        // [parity][hi, lo] X_t halves
  static constexpr int OFF_SLOT = 2 * ARR + 4 * XARR;  // [parity][4][64] column-block
                                               // maxima of X, one copy per lane
  static constexpr int OFF_RED = OFF_SLOT + 512; // row-sum maximum, W^T flag, max|A|,
                                                 // scale exponent of the final X
  static constexpr int OFF_WT = OFF_RED + 4;   // W^T copy; landmarks while A is built
  static constexpr int WLS = MP + 4;           // row stride of the W^T copy
  static constexpr int TAIL = D * WLS > MP * (D + 4) ? D * WLS : MP * (D + 4);
  static constexpr int SMEM = OFF_WT + TAIL;
  static_assert(N16 * SX <= 2 * XARR, "fp32 matrix fits one parity of the X halves");
  static_assert(N16 / 2 <= XSW, "X line fits");
};

// Position (in halves) of column k in a row of a half-precision array.  The
// 16-column blocks go in pairs (2p, 2p + 1); within pair p, lane group q's
// four columns of block 2p and four of block 2p + 1 are 8 consecutive
// halves.  An odd last block stands alone, 4 halves per lane group.
template <int MB>
__device__ __forceinline__ int hpos(int k) {
  const int c = k >> 4, q = (k >> 2) & 3, j = k & 3;
  if ((MB & 1) && c == MB - 1) return 16 * c + 4 * q + j;
  return 32 * (c >> 1) + 8 * q + 4 * (c & 1) + j;
}

// A operand of one 16-row block: row `row` of the arrays at word offsets
// offh (hi) and offl (lo), chunks 0..NC-1 (the lone block of an odd last
// chunk fills slots 0..3, slots 4..7 are zero).
template <int MB, int D>
__device__ __forceinline__ void load_op(const float* smem, int offh, int offl, int row, int lg,
                                        u32x4* h, u32x4* l) {
  using G = NsGeom<MB, D>;
  const int base = row * G::RSW;
#pragma unroll
  for (int p = 0; p < G::NC; ++p) {
    if (G::ODD && p == G::NC - 1) {
      const u32x2 vh = *reinterpret_cast<const u32x2*>(smem + offh + base + 16 * p + 2 * lg);
      const u32x2 vl = *reinterpret_cast<const u32x2*>(smem + offl + base + 16 * p + 2 * lg);
      h[p] = u32x4{vh[0], vh[1], 0u, 0u};
      l[p] = u32x4{vl[0], vl[1], 0u, 0u};
    } else {
      h[p] = *reinterpret_cast<const u32x4*>(smem + offh + base + 16 * p + 4 * lg);
      l[p] = *reinterpret_cast<const u32x4*>(smem + offl + base + 16 * p + 4 * lg);
    }
  }
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Position of 8-byte chunk c (rows 4c .. 4c + 3) within line k of the
// half-precision X_t arrays (see NsGeom).
__device__ __forceinline__ int xchunk(int k, int c) { return c ^ ((k >> 2) & 3); }

// A operand of one 16-row block of X_t (rows r0 .. r0 + 15) from the column-
// major arrays at word offsets offh / offl, with transposing LDS reads: in
// each 16-lane group, lane i receives half i % 4 of the 8 bytes read by lane
// 4 j + i / 4 as its element j.  So lane L = 4 j + q of group g reads rows
// r0 + 4q .. + 3 of line k = 16 (2p + h) + 4 g + j, and lane (g, lr) ends up
// with X_t[r0 + lr][k] for j = 0..3: slots 4 h .. 4 h + 3 of chunk p.
template <int MB, int D>
__device__ __forceinline__ void load_xop(float* smem, int offh, int offl, int r0, int lane,
                                         u32x4* h, u32x4* l) {
  using G = NsGeom<MB, D>;
  const int lg = lane >> 4, j = (lane >> 2) & 3, q = lane & 3;
  // halves offset of (line 4 g + j, rows r0 + 4 q ..): r0 is a multiple of
  // 16 and lines 16 (2p + h) + 4 g + j all have (k >> 2) & 3 = g
  const int base = (4 * lg + j) * G::XSH + 4 * xchunk(4 * lg + j, r0 / 4 + q);
  uint16_t* H = reinterpret_cast<uint16_t*>(smem + offh);
  uint16_t* L = reinterpret_cast<uint16_t*>(smem + offl);
#pragma unroll
  for (int p = 0; p < G::NC; ++p) {
    u32x2 v[2][2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      if (G::ODD && p == G::NC - 1 && hh == 1) {
        v[0][hh] = v[1][hh] = u32x2{0u, 0u};
      } else {
        const int o = base + 16 * (2 * p + hh) * G::XSH;
        v[0][hh] = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                 (lds_s16x4*)(H + o)));
        v[1][hh] = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                 (lds_s16x4*)(L + o)));
      }
    }
    h[p] = u32x4{v[0][0][0], v[0][0][1], v[0][1][0], v[0][1][1]};
    l[p] = u32x4{v[1][0][0], v[1][0][1], v[1][1][0], v[1][1][1]};
  }
}

// split_block with split2_mix.
__device__ __forceinline__ void split_block_mix(f4 x, int i, float one, u32x4* h, u32x4* l) {
  unsigned h0, l0, h1, l1;
  split2_mix(x[0], x[1], one, h0, l0);
  split2_mix(x[2], x[3], one, h1, l1);
  h[i >> 1][2 * (i & 1)] = h0;
  h[i >> 1][2 * (i & 1) + 1] = h1;
  l[i >> 1][2 * (i & 1)] = l0;
  l[i >> 1][2 * (i & 1) + 1] = l1;
}

// Splits accumulator block i into the B operand registers of its chunk.
__device__ __forceinline__ void split_block(f4 x, int i, u32x4* h, u32x4* l) {
  unsigned h0, l0, h1, l1;
  split2(x[0], x[1], h0, l0);
  split2(x[2], x[3], h1, l1);
  h[i >> 1][2 * (i & 1)] = h0;
  h[i >> 1][2 * (i & 1) + 1] = h1;
  l[i >> 1][2 * (i & 1)] = l0;
  l[i >> 1][2 * (i & 1) + 1] = l1;
}

// Interior wave c: the Newton-Schulz steps on column block c.
// With ITERS, every iterate X_1 .. X_T also goes to global memory, fp32,
// row-major with row stride MP: X_t at xiter + t MP MP (rows and columns
// below 16 MB; X_0 is stored by the set-up).
template <int MB, int D, bool ITERS = false>
__device__ __forceinline__ void ns_wave(const MainArgs& a, float* smem, int c, int lane, float alpha, int eA,
                        int e0, float* xiter = nullptr) {
  using G = NsGeom<MB, D>;
  constexpr int NC = G::NC, XSH = G::XSH, SX = G::SX, XARR = G::XARR;
  const int lr = lane & 15, lg = lane >> 4;
  const int col = 16 * c + lr;
  const int iters = a.iters;
  float* slot = smem + G::OFF_SLOT;
  // ITERS: X_1 .. X_T through a buffer resource over the head's iterates
  // ((iters + 1) MP MP floats from xiter); the lane's byte offset of row
  // 4 g, column col; the iterate and block rows go in the scalar offset
  const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
      xiter, static_cast<short>(0), ITERS ? (iters + 1) * MP * MP * 4 : 0, 0x00020000);
  const int xoff = (4 * lg * MP + col) * 4;

  // X-hat_0 = 2^e0 alpha A on the own columns, fp32 and split (the same
  // arithmetic as the shared copy, so the two agree bit for bit)
  f4 xs[MB];
  u32x4 xh[NC], xl[NC];
  {
    const float* Af = smem + G::OFF_X + 2 * G::XARR;
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) xs[i][j] = ldexpf(alpha * Af[(16 * i + 4 * lg + j) * SX + col], e0);
  }
#pragma unroll
  for (int p = 0; p < NC; ++p) xh[p] = xl[p] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < MB; ++i) split_block(xs[i], i, xh, xl);
  __syncthreads();  // the fp32 A (in the parity-1 X halves) is dead from here

  int ep = e0, ec = e0;  // scale exponents of X_{t-1} and X_t
  const float one = opaque_one();
  // A step is 2 MB blocks: q < MB is phase-1 block q (operand: rows 16 q ..
  // of A), q >= MB is phase-2 block q - MB (operand: rows of X_t).  Operands
  // go through a ring of 3 register slots, read 2 blocks ahead; the reads of
  // the first two blocks, rows of A, which never changes, are issued at the
  // end of the step before and stay in flight across its barrier.
  u32x4 bh[3][NC], bl[3][NC];
  auto load_block = [&](int q, int xoh, int xol, u32x4* h, u32x4* l) {
    if (q < MB) load_op<MB, D>(smem, G::OFF_AH, G::OFF_AL, 16 * q + lr, lg, h, l);
    else load_xop<MB, D>(smem, xoh, xol, 16 * (q - MB), lane, h, l);
  };
  constexpr int NPRE = MB >= 2 ? 2 : 1;  // leading blocks that are rows of A
#pragma unroll
  for (int q = 0; q < NPRE; ++q) load_block(q, 0, 0, bh[q], bl[q]);

  // One step; the last one writes X_{t+1} in fp32 instead of split.
  auto step = [&](int t, auto last_c) {
    constexpr bool LAST = decltype(last_c)::value;
    const int cb = t & 1;
    const int xoh = G::OFF_X + 2 * XARR * cb, xol = xoh + XARR;        // X_t
    const int noh = G::OFF_X + 2 * XARR * (1 - cb), nol = noh + XARR;  // X_{t+1}
    // column-block maxima of X-hat_{t-1} (units 2^ep): the scale of X_{t+1}
    float sv[MB];
    if (!LAST) {
#pragma unroll
      for (int i = 0; i < MB; ++i) sv[i] = slot[256 * (1 - cb) + 64 * i + lane];
    }
    // leading blocks that are rows of X_t (only when MB == 1)
#pragma unroll
    for (int q = NPRE; q < 2; ++q) load_block(q, xoh, xol, bh[q], bl[q]);

    const int sT = 14 - eA - ec;  // T-hat = 2^sT (A-hat X-hat_t)

    u32x4 th[NC], tl[NC];
#pragma unroll
    for (int p = 0; p < NC; ++p) th[p] = tl[p] = u32x4{0u, 0u, 0u, 0u};
    int eN = ec;
    float c1 = 0.f, c2 = 0.f;
    uint16_t* H = reinterpret_cast<uint16_t*>(smem + noh);
    uint16_t* L = reinterpret_cast<uint16_t*>(smem + nol);
    float* XF = smem + noh;

    // MFMAs of chunks [p0, p1) of block q into acc.
    auto mfmas = [&](int q, int p0, int p1, f4 acc) -> f4 {
      const u32x4* oh = bh[q % 3];
      const u32x4* ol = bl[q % 3];
#pragma unroll
      for (int p = 0; p < NC; ++p) {
        if (p < p0 || p >= p1) continue;
        if (q < MB) {
          // phase 1: T-hat[:, c] = 2^(14 - eA - ec) A-hat X-hat_t[:, c]
          acc = mfma_h(oh[p], xh[p], acc);
          acc = mfma_h(ol[p], xh[p], acc);
          acc = mfma_h(oh[p], xl[p], acc);
        } else {
          // phase 2: X_{t+1}[:, c] = 2 X_t[:, c] - X_t T[:, c]
          acc = mfma_h(oh[p], th[p], acc);
          acc = mfma_h(ol[p], th[p], acc);
          acc = mfma_h(oh[p], tl[p], acc);
        }
      }
      return acc;
    };
    // What block q's result feeds: T-hat parts (phase 1) or X_{t+1} (phase 2).
    auto epilogue = [&](int q, f4 acc) {
      if (q < MB) {
        const int ip = q;
        if (!LAST && ip == 0) {
          // publish max|X-hat_t| of the own columns (units 2^ec), one copy per
          // lane (across lanes, the non-negative maxima compare as unsigned
          // bit patterns)
          float mx = 0.f;
#pragma unroll
          for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) mx = fmaxf(mx, fabsf(xs[i][j]));
          slot[256 * cb + 64 * c + lane] = __uint_as_float(wave_max_u(__float_as_uint(mx)));
        }
        f4 tv;
#pragma unroll
        for (int j = 0; j < 4; ++j) tv[j] = ldexpf(acc[j], sT);
        split_block_mix(tv, ip, one, th, tl);
        if (ip == MB - 1) {
          // scale of X_{t+1}: max|X_{t-1}| 2^eN < 2^7 (the last X stays at
          // 2^ec); X-hat_{t+1} = 2^(eN - ec + 1) X-hat_t
          //                      - 2^(eN - ec - 14) (X-hat_t T-hat)
          if (!LAST) {
            float mp = sv[0];
#pragma unroll
            for (int i = 1; i < MB; ++i) mp = fmaxf(mp, sv[i]);
            if (mp > 0.f) eN = ep + 7 - __builtin_amdgcn_frexp_expf(mp);
          }
          c1 = ldexpf(1.0f, eN - ec + 1);
          c2 = -ldexpf(1.0f, eN - ec - 14);
        }
      } else {
        const int ip = q - MB;
#pragma unroll
        for (int j = 0; j < 4; ++j) xs[ip][j] = fmaf(acc[j], c2, c1 * xs[ip][j]);
        if constexpr (ITERS) {
          // buffer stores: the iterate's offset in a scalar register, one
          // 32-bit lane offset (64-bit lane addresses pushed the step loop
          // into register spills)
          const int so = ((t + 1) * MP * MP + 16 * ip * MP) * 4;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(ldexpf(xs[ip][j], -eN)), xrs,
                                                  xoff, so + j * MP * 4, 0);
        }
        if (!LAST) {
          split_block_mix(xs[ip], ip, one, xh, xl);
          // rows 16 ip + 4 g .. + 3 of line col: one 8-byte store per part
          const int o = col * XSH + 4 * xchunk(col, 4 * ip + lg);
          *reinterpret_cast<u32x2*>(H + o) =
              u32x2{xh[ip >> 1][2 * (ip & 1)], xh[ip >> 1][2 * (ip & 1) + 1]};
          *reinterpret_cast<u32x2*>(L + o) =
              u32x2{xl[ip >> 1][2 * (ip & 1)], xl[ip >> 1][2 * (ip & 1) + 1]};
        } else {
          // the final iterate in fp32, over the X_{t+1} halves
#pragma unroll
          for (int j = 0; j < 4; ++j) XF[(16 * ip + 4 * lg + j) * SX + col] = ldexpf(xs[ip][j], -eN);
        }
      }
    };

    // Software pipeline: block q's operand reads go out 2 blocks ahead, and
    // block q - 1's epilogue, which needs only block q - 1's results, is
    // interleaved with block q's MFMAs so that it runs in their shadows.  The
    // last phase-1 block feeds the phase-2 operand's chunk (MB - 1) / 2:
    // deferring its epilogue into the first phase-2 block works only when
    // that is not chunk 0.
    constexpr bool DEFER_LAST_T = (MB - 1) / 2 > 0;
    f4 prev = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < 2 * MB; ++q) {
      if (q + 2 < 2 * MB) load_block(q + 2, xoh, xol, bh[(q + 2) % 3], bl[(q + 2) % 3]);
      __builtin_amdgcn_sched_barrier(0);
      f4 acc = mfmas(q, 0, 1, f4{0.f, 0.f, 0.f, 0.f});
      if (q > 0 && !(q == MB && !DEFER_LAST_T)) epilogue(q - 1, prev);
      acc = mfmas(q, 1, NC, acc);
      // the compiler interleaves the epilogue's vector instructions with
      // this block's MFMAs (a fixed pattern of one MFMA, then 3, 6 or 10 VALU,
      // was 0.8 - 1.4 us per solve slower)
      __builtin_amdgcn_sched_barrier(0);
      prev = acc;
      if (q == MB - 1 && !DEFER_LAST_T) epilogue(q, prev);
    }
    epilogue(2 * MB - 1, prev);
    ep = ec;
    ec = eN;
    if (!LAST) {
      // The next step's leading operands (rows of A, which never changes)
      // are read after this step's stores and may still be in flight at the
      // barrier: wait only until the stores (issued before those 2 NC NPRE
      // reads) have completed.  LDS operations of a wave complete in order.
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < NPRE; ++q) load_block(q, 0, 0, bh[q], bl[q]);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (2 * NC * NPRE == 8) asm volatile("s_waitcnt lgkmcnt(8)" ::: "memory");
      else if constexpr (2 * NC * NPRE == 4) asm volatile("s_waitcnt lgkmcnt(4)" ::: "memory");
      else asm volatile("s_waitcnt lgkmcnt(2)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("" ::: "memory");
    } else {
      __syncthreads();
    }
  };

  // two steps per loop iteration: the registers carried from step to step
  // then need no copies at the back edge (about 20 moves per step otherwise)
  int t = 0;
  for (; t + 2 < iters; t += 2) {
    step(t, std::false_type{});
    step(t + 1, std::false_type{});
  }
  if (t + 1 < iters) step(t, std::false_type{});
  if (iters > 0) step(iters - 1, std::true_type{});
  // the final iterate's scale: max|X| 2^ec < 2^15
  if (c == 0 && lane == 0) smem[G::OFF_RED + 3] = __int_as_float(ec);
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

// Abs-sum of row `row` of the fp32 A in LDS (row stride SX, zero beyond m),
// over all N16 columns (the zeros add nothing): all loads issued at once.
template <int N16, int SX>
__device__ __forceinline__ float a_row_abs_sum(const float* Af, int row) {
  f4 v[N16 / 4];
#pragma unroll
  for (int q = 0; q < N16 / 4; ++q) v[q] = ld4(Af + row * SX + 4 * q);
  float sum = 0.f;
#pragma unroll
  for (int q = 0; q < N16 / 4; ++q) sum += fabsf(v[q][0]) + fabsf(v[q][1]) + fabsf(v[q][2]) + fabsf(v[q][3]);
  return sum;
}

// Set-up of a solver workgroup: A = k(L, L) + eps I in LDS (fp32, row stride
// SX, at the parity-1 X halves, where it stays until the first step's
// barrier), alpha, and the scaled split arrays of A and X_0 = alpha A.
// Returns alpha and the scale exponents of A and X_0.  With xiter, X_0 also
// goes to global memory (fp32, row stride MP).
template <int D, int MB, int KIND>
__device__ __forceinline__ void solver_setup(const MainArgs& a, int bh, float* smem, float& alpha_out,
                                             int& eA_out, int& e0_out, float* xiter = nullptr) {
  using G = NsGeom<MB, D>;
  constexpr int SX = G::SX, N16 = G::N16, RSH = G::RSH;
  float* Af = smem + G::OFF_X + 2 * G::XARR;  // A in fp32 while set up
  float* red = smem + G::OFF_RED;
  float* slot = smem + G::OFF_SLOT;
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
  const int m = a.m;

  // A = k(L, L) + eps I, built here in LDS.  The landmarks are staged in LDS
  // (rows up to an even count, padding zero).  Each thread computes a 2 x 2
  // block (rows 2 bi, 2 bi + 1; columns 2 bj, 2 bj + 1), bi <= bj, of the
  // upper triangle, streaming the four landmark rows; every unordered pair is
  // computed once and written to A[i][j] and A[j][i], so A is exactly
  // symmetric.
  constexpr int LDL = D + 4;
  float* Ls = smem + G::OFF_WT;
  const int nb = (m + 1) / 2;
  {
    const float* Lg = a.L + static_cast<size_t>(bh) * m * D;
    for (int e = tid; e < 2 * nb * (D / 4); e += WGM) {
      const int row = e / (D / 4), c4 = e % (D / 4);
      st4(Ls + row * LDL + 4 * c4, row < m ? ld4(Lg + row * D + 4 * c4) : f4{0.f, 0.f, 0.f, 0.f});
    }
    for (int e = tid; e < N16 * SX; e += WGM) Af[e] = 0.f;
  }
  __syncthreads();
  build_a<D, KIND>(a, bh, Ls, Af, SX);
  __syncthreads();
  // alpha = 1 / (max column abs-sum * max row abs-sum); A is symmetric, so
  // its largest column sum equals its largest row sum.  Also max|A|.
  if (w == 0) {
    const float sum = lane < N16 ? a_row_abs_sum<N16, SX>(Af, lane) : 0.f;
    // non-negative, so it compares as an unsigned bit pattern
    const float mx = __uint_as_float(wave_max_u(__float_as_uint(sum)));
    if (lane == 0) {
      red[0] = mx;
      red[1] = 0.f;  // set once W^T is in LDS
    }
  }
  __syncthreads();
  const float alpha = 1.0f / (red[0] * red[0]);
  // max|A| is the diagonal's 1 + eps: every other entry is exp2 of a
  // non-positive argument (eps >= 0 is checked at the boundary)
  const float amax = 1.0f + a.eps;
  const int eA = 14 - __builtin_amdgcn_frexp_expf(amax);
  const float m0 = alpha * amax;  // max|X_0|
  const int e0 = 7 - __builtin_amdgcn_frexp_expf(m0);
  // A and X_0 = alpha A, scaled and split, into the half-precision arrays
  // (four consecutive columns per thread: 8-byte stores); with no steps to
  // run, X_0 in fp32 instead
  {
    constexpr int Q4 = N16 / 4;
    uint16_t* AH = reinterpret_cast<uint16_t*>(smem + G::OFF_AH);
    uint16_t* AL = reinterpret_cast<uint16_t*>(smem + G::OFF_AL);
    uint16_t* XH = reinterpret_cast<uint16_t*>(smem + G::OFF_X);
    uint16_t* XL = reinterpret_cast<uint16_t*>(smem + G::OFF_X + G::XARR);
    // every row read issued before the first store
    constexpr int NR = (N16 * Q4 + WGM - 1) / WGM;
    f4 avs[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int e = tid + r * WGM;
      if (e < N16 * Q4) avs[r] = ld4(Af + (e / Q4) * SX + 4 * (e % Q4));
    }
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int e = tid + r * WGM;
      if (e >= N16 * Q4) break;
      const int i = e / Q4, q = e % Q4;
      const f4 av = avs[r];
      const int h0 = i * RSH + hpos<MB>(4 * q);  // a multiple of 4
      unsigned h0w, l0w, h1w, l1w;
      split2(ldexpf(av[0], eA), ldexpf(av[1], eA), h0w, l0w);
      split2(ldexpf(av[2], eA), ldexpf(av[3], eA), h1w, l1w);
      *reinterpret_cast<u32x2*>(AH + h0) = u32x2{h0w, h1w};
      *reinterpret_cast<u32x2*>(AL + h0) = u32x2{l0w, l1w};
      const f4 xv = {alpha * av[0], alpha * av[1], alpha * av[2], alpha * av[3]};
      if (a.iters > 0) {
        // X_0 is exactly symmetric: its line i (column i) is its row i
        split2(ldexpf(xv[0], e0), ldexpf(xv[1], e0), h0w, l0w);
        split2(ldexpf(xv[2], e0), ldexpf(xv[3], e0), h1w, l1w);
        *reinterpret_cast<u32x2*>(XH + i * G::XSH + 4 * xchunk(i, q)) = u32x2{h0w, h1w};
        *reinterpret_cast<u32x2*>(XL + i * G::XSH + 4 * xchunk(i, q)) = u32x2{l0w, l1w};
      } else {
        st4(smem + G::OFF_X + i * SX + 4 * q, xv);
      }
      if (xiter) st4(xiter + i * MP + 4 * q, xv);
    }
    // the first step reads these as the maxima of the step before
    slot[tid] = ldexpf(m0, e0);
  }
  __syncthreads();
  alpha_out = alpha;
  eA_out = eA;
  e0_out = e0;
}

template <int D, int MB, int KIND>
__device__ __forceinline__ void solver_role(const MainArgs& a, int bh, float* smem) {
  using G = NsGeom<MB, D>;
  constexpr int SX = G::SX, N16 = G::N16, WLS = G::WLS;
  float* red = smem + G::OFF_RED;
  float* WTL = smem + G::OFF_WT;             // [D][WLS] W^T copy (see below)
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
  const int m = a.m;
  __builtin_amdgcn_s_setprio(3);
  float alpha;
  int eA, e0;
  solver_setup<D, MB, KIND>(a, bh, smem, alpha, eA, e0);

  if (w < MB) {
    ns_wave<MB, D>(a, smem, w, lane, alpha, eA, e0);
  } else {
    // idle waves; the first one watches for the head's W^T (published by the
    // last key workgroup) during the second half of the steps and copies it
    // to LDS, so that Y can be formed right after the last step.  Each global
    // read is issued before a barrier and consumed after it (a barrier does
    // not wait for global loads), so the watcher never delays the steps.
    __syncthreads();  // matches the set-up barrier of the solving waves
    const bool watcher = w == MB && !a.out_in_main;
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
        if (state == 0 && polled && static_cast<unsigned>(__builtin_amdgcn_readfirstlane(cnt)) >= 1u) {
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

  // the final iterate, fp32, row stride SX (zero in the padding)
  const float* Xf = smem + G::OFF_X + 2 * G::XARR * (a.iters & 1);
  if (a.st_x) {
    for (int e = tid; e < m * m; e += WGM)
      a.st_x[static_cast<size_t>(bh) * m * m + e] = Xf[(e / m) * SX + (e % m)];
  }
  if (a.out_in_main) {
    // the query workgroups form Y themselves: publish 2^ex X (max < 2^15,
    // ex from the Newton-Schulz scales) split into fp16 parts (hi [MP][MP],
    // then lo [MP][MP], two per 32-bit word) and ex, then raise the flag
    const int ex = __float_as_int(red[3]);
    unsigned* Xh = reinterpret_cast<unsigned*>(a.xw + static_cast<size_t>(bh) * MP * MP);
    unsigned* Xl = Xh + MP * MP / 2;
    for (int e = tid; e < MP * MP / 2; e += WGM) {
      const int row = e / (MP / 2), col = 2 * (e % (MP / 2));
      const bool in = row < N16 && col < N16;  // N16 is even
      unsigned hw, lw;
      split2(in ? ldexpf(Xf[row * SX + col], ex) : 0.f, in ? ldexpf(Xf[row * SX + col + 1], ex) : 0.f,
             hw, lw);
      __hip_atomic_store(Xh + e, hw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(Xl + e, lw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // the flag's value carries ex (nonzero for any ex)
    raise_flag(flag_x(a, bh), 0x10000u | (static_cast<unsigned>(ex) & 0xffffu));
    return;
  }
  if (red[1] != 0.f) {
    // W^T is already published (its arrival counted) and copied to LDS: this
    // workgroup is the second of (W, X) and forms Y^T from LDS directly
    compute_y<D>(WTL, WLS, Xf, SX, N16, N16, a.yt + static_cast<size_t>(bh) * D * MP);
    raise_flag(flag_y(a, bh));
    return;
  }
  // otherwise publish X and count its arrival
  float* Xg = a.xw + static_cast<size_t>(bh) * MP * MP;
  for (int e = tid; e < MP * MP; e += WGM) {
    const int row = e / MP, col = e % MP;
    st_dev(Xg + e, (row < N16 && col < N16) ? Xf[row * SX + col] : 0.f);
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

// Single (not iterated) products also run on fp16 MFMA with two-part
// operands (hi hi + lo hi + hi lo), each operand scaled by a power of two
// into fp16 range first: per row for W^T and Y^T, one exponent for X (from
// the Newton-Schulz scales), 2^14 for K_QL (values in (0, 1]).  Sums with
// cancellation (Y and O mix signs) keep about 22 significant bits of each
// term.
constexpr int WLD = MP + 8;  // row stride (halves) of the split W^T / Y^T copies

// Layout of the query workgroups' first LDS area: the split W^T / Y^T copies
// (hi, lo: D rows of WLD halves each) and the per-row exponents EW.
template <int D>
struct QGeom {
  static constexpr int OFF_WL = D * WLD / 2;   // floats
  static constexpr int OFF_EW = D * WLD;
  static constexpr int SIZE = OFF_EW + D;
};

// Floats of the map role's first LDS area: P[j][token], or the query
// workgroups' split copies of W^T / Y^T.
template <int D>
constexpr int map_pj_size() {
  return MP * LS > QGeom<D>::SIZE ? MP * LS : QGeom<D>::SIZE;
}

// Row stride (floats) of the Laplacian tiles' staged token rows: 16-byte
// reads of one row per lane fall on distinct banks for D = 16, 32, 64.
template <int D>
constexpr int row_stride() { return D + 4; }

// Floats of LDS the map role uses: P, the token-major K_QL rows, V^T (or the
// query workgroups' second K_QL tile), the Gaussian tiles' squared norms and
// the Laplacian tiles' staged token rows.
template <int D, int KIND>
constexpr int map_smem() {
  return map_pj_size<D>() + 2 * MP * LS + TILE + (KIND == 0 ? TILE * row_stride<D>() : 0) + 8;
}

// Key tiles' operands of the W^T product as scaled fp16 parts (hi, lo):
// rows of 64 halves (one per token), the 16-byte chunks of row r permuted
// (chunk c at position c ^ (r & 7)) so that the operand reads of 16
// consecutive rows spread over the banks.  Position (in halves) of token k
// of row r:
__device__ __forceinline__ int hsw(int r, int k) { return r * 64 + ((((k >> 3) ^ r) & 7) << 3) + (k & 7); }

// Y^T = W^T X^T in place: the split, row-scaled W^T in LDS (row c scaled by
// 2^EW[c]) is replaced by the split Y^T with the same row scales times
// 2^(ex - 22); X comes split from global memory (hi then lo, rows of MP
// halves, scaled by 2^ex), every operand load issued before the first MFMA.
// Lane (g, r), slot s of chunk p: contraction index 32 p + 8 g + s.
// Each term of a row's sums is below 2^15 2^15 and n <= 64 terms, so the
// accumulator is below 2^36 and 2^-22 of it is in fp16 range; values that
// fall below fp16's normal range carry less than the fp32 accumulation's own
// error.
template <int D>
__device__ void y_in_lds(float* Q, const uint16_t* xh, const uint16_t* xl) {
  using QG = QGeom<D>;
  constexpr int CBN = D / 16;
  constexpr int NBLK = 4 * CBN;          // 16x16 output blocks
  constexpr int NSB = (NBLK + 7) / 8;    // blocks per wave
  uint16_t* WH = reinterpret_cast<uint16_t*>(Q);
  uint16_t* WL = reinterpret_cast<uint16_t*>(Q + QG::OFF_WL);
  const int lane = threadIdx.x & 63, w = wave_id();
  const int lr = lane & 15, lg = lane >> 4;
  // a wave's blocks w, w + 8 share column block jb = w % 4, so X rows
  // 16 jb .. + 15 are read once per wave
  const int jb = w % 4;
  u32x4 bh[2], bl[2];
  if (w < NBLK) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int o = (16 * jb + lr) * MP + 32 * p + 8 * lg;
      bh[p] = *reinterpret_cast<const u32x4*>(xh + o);
      bl[p] = *reinterpret_cast<const u32x4*>(xl + o);
    }
  }
  f4 acc[NSB];
#pragma unroll
  for (int s = 0; s < NSB; ++s) {
    const int blk = w + 8 * s;
    acc[s] = f4{0.f, 0.f, 0.f, 0.f};
    if (blk < NBLK) {
      const int cb = blk / 4;
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int o = (16 * cb + lr) * WLD + 32 * p + 8 * lg;
        const u32x4 ah = *reinterpret_cast<const u32x4*>(WH + o);
        const u32x4 al = *reinterpret_cast<const u32x4*>(WL + o);
        acc[s] = mfma_h(ah, bh[p], acc[s]);
        acc[s] = mfma_h(al, bh[p], acc[s]);
        acc[s] = mfma_h(ah, bl[p], acc[s]);
      }
    }
  }
  __syncthreads();  // every wave has read its W^T rows
#pragma unroll
  for (int s = 0; s < NSB; ++s) {
    const int blk = w + 8 * s;
    if (blk < NBLK) {
      const int cb = blk / 4;
      unsigned h[2], l[2];
      split2(ldexpf(acc[s][0], -22), ldexpf(acc[s][1], -22), h[0], l[0]);
      split2(ldexpf(acc[s][2], -22), ldexpf(acc[s][3], -22), h[1], l[1]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int o = (16 * cb + 4 * lg + i) * WLD + 16 * jb + lr;
        WH[o] = static_cast<uint16_t>(h[i >> 1] >> (16 * (i & 1)));
        WL[o] = static_cast<uint16_t>(l[i >> 1] >> (16 * (i & 1)));
      }
    }
  }
  __syncthreads();
}

// Lines [l0, l1) (32 floats each) of W^T, nP <= 128 partials, in chunks of
// at most 512 elements: G threads per element (G = 512 / elements, at most
// 8, a power of two), thread g sums partials [g P, (g + 1) P) in order with
// the loads of up to 16 in flight, and the G sums are added in order of g
// through LDS (red, up to 512 floats).  Slices are whole cache lines, so no
// line of W^T is written by two workgroups.
template <int D>
__device__ void reduce_w_lines(const MainArgs& a, int bh, int l0, int l1, float* red) {
  const int nP = a.nP, m = a.m;
  const size_t ps = static_cast<size_t>(D) * MP;
  const float* pb = a.wpart + static_cast<size_t>(bh) * nP * ps;
  float* wg = a.wt + static_cast<size_t>(bh) * ps;
  const int tid = threadIdx.x;
  for (int e0 = 32 * l0; e0 < 32 * l1; e0 += WGM) {
    const int E = min(WGM, 32 * l1 - e0);
    int G = 1;
    while (G < 8 && 2 * G * E <= WGM) G *= 2;
    const int P = (nP + G - 1) / G;
    const int el = tid % E, g = tid / E;
    if (g < G) {
      const int pe = min(nP, (g + 1) * P);
      float sum = 0.f;
      for (int p0 = g * P; p0 < pe; p0 += 16) {
        const int np = min(pe - p0, 16);
        float v[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) v[q] = q < np ? pb[(p0 + q) * ps + e0 + el] : 0.f;
#pragma unroll
        for (int q = 0; q < 16; ++q)
          if (q < np) sum += v[q];
      }
      red[g * E + el] = sum;
    }
    __syncthreads();
    if (tid < E) {
      float sum = red[tid];
      for (int h = 1; h < G; ++h) sum += red[h * E + tid];
      const int e = e0 + tid;
      const int c = e / MP, j = e % MP;
      const float w = j < m ? sum : 0.f;
      st_dev(wg + e, w);
      if (a.st_w && j < m) a.st_w[(static_cast<size_t>(bh) * m + j) * D + c] = w;
    }
    __syncthreads();  // red is reused by the next chunk
  }
}

// Offset of K_QL[token][j] in a tile's token-major rows (row stride LS).  The
// row of token t starts (t >> 3) & 3 floats in, so that the map waves' stores
// of one landmark column for 64 tokens (lane = token) fall on distinct banks
// (with no offset, 32 lanes at stride LS = 68 share 8 banks); readers use
// scalar loads, since the rows are no longer 16-byte aligned.
__device__ __forceinline__ int ptj(int tok, int j) { return tok * LS + j + ((tok >> 3) & 3); }

// Four consecutive output columns of one token at element offset o: one
// 16-byte streaming store (fp32) or one 8-byte store (bf16, round to nearest
// even).  fp32 O rows are written with streaming (non-temporal) stores:
// nothing in the launch reads them again, and the end-of-kernel write-back of
// O is shorter.
__device__ __forceinline__ void store_o4(void* out, int bf16, size_t o, f4 v) {
  if (bf16) {
    const uint2 u = {static_cast<uint32_t>(f32_to_bf16_rne(v[0])) |
                         (static_cast<uint32_t>(f32_to_bf16_rne(v[1])) << 16),
                     static_cast<uint32_t>(f32_to_bf16_rne(v[2])) |
                         (static_cast<uint32_t>(f32_to_bf16_rne(v[3])) << 16)};
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + o) = u;
  } else {
    __builtin_nontemporal_store(v, reinterpret_cast<f4*>(static_cast<float*>(out) + o));
  }
}

// fp32 O columns col .. col + 31 (one 128-byte line per row) of tokens n0 ..
// n0 + 15, held as two 16x16 blocks of O^T: lane (g, r) has columns
// col + 4 g .. + 3 (c0) and col + 16 + 4 g .. + 3 (c1) of token n0 + r.
// Lanes r and r ^ 8 trade one block (DPP row rotation by 8) so that each of
// the two stores writes whole lines (a streaming store of part of a line
// can leave L2 as a partial line): first tokens n0 .. n0 + 7 (lanes r < 8
// their c0, lanes r >= 8 the c1 of token r - 8), then n0 + 8 .. n0 + 15.
// Rows from N on are not written; row n of the head is at rows + n.
template <int D>
__device__ __forceinline__ void store_o_lines(void* out, size_t rows, int n0, int N, int col, f4 c0, f4 c1) {
  const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const bool lo = lr < 8;
  const f4 x = lo ? c1 : c0;
  f4 y;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    y[i] = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x[i]), 0x128, 0xF, 0xF, false));
  const int c = col + (lo ? 0 : 16) + 4 * lg;
  const int n1 = n0 + (lo ? lr : lr - 8), n2 = n1 + 8;
  if (n1 < N) store_o4(out, 0, (rows + n1) * D + c, lo ? c0 : y);
  if (n2 < N) store_o4(out, 0, (rows + n2) * D + c, lo ? y : c1);
}

// O rows of one 64-token tile: K_QL tile (PT, LDS, zero beyond m) times Y on
// fp16 MFMA, with Y^T split in LDS (row c scaled by 2^(EW[c] + ex - 22),
// y_in_lds) and the tile's K_QL rows scaled by 2^14 and split here, once per
// tile.  Each product forms a block of O^T (Y^T rows as the first operand),
// so that lane (g, r) holds four consecutive columns 16 cb + 4 g .. + 3 of
// token 16 tb + r: one 16-byte store.  Wave w: tokens 16 (w % 4) .. +15;
// waves 0-3 take the first half of the column blocks, waves 4-7 the second,
// so that each 128-byte line of an O row is written by one wave.  (Trading
// blocks between lanes so that one store writes whole lines, as the output
// launch does, cut the written bytes by 1.3 MB on 8 heads of 3136 tokens but
// put 0.5 us on the end of the launch, which this tail sets.)
template <int D>
__device__ void out_tile(const MainArgs& a, int bh, int t, const float* PT, const float* Q, int ex) {
  using QG = QGeom<D>;
  constexpr int CBN = D / 16;
  const uint16_t* YH = reinterpret_cast<const uint16_t*>(Q);
  const uint16_t* YL = reinterpret_cast<const uint16_t*>(Q + QG::OFF_WL);
  const int* EW = reinterpret_cast<const int*>(Q + QG::OFF_EW);
  const int lane = threadIdx.x & 63, w = wave_id();
  const int lr = lane & 15, lg = lane >> 4;
  const int tb = w & 3, ch = w >> 2;
  u32x4 kh[2], kl[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const float* ar = PT + ptj(16 * tb + lr, 32 * p + 8 * lg);
    split8h(f4{ar[0], ar[1], ar[2], ar[3]}, f4{ar[4], ar[5], ar[6], ar[7]}, 14, kh[p], kl[p]);
  }
  constexpr int CBW = (CBN + 1) / 2;  // column blocks per wave
#pragma unroll
  for (int k = 0; k < CBW; ++k) {
    const int cb = CBW * ch + k;
    if (cb >= CBN) break;
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
    // lane (g, lr): O[token 16 tb + lr][16 cb + 4 g + i]; scale
    // 2^(22 - 14 - (EW + ex)) per column
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = ldexpf(c[i], 8 - ex - EW[16 * cb + 4 * lg + i]);
    const int n = t * TILE + 16 * tb + lr;
    if (n < a.N) store_o4(a.out, a.bf16, (static_cast<size_t>(bh) * a.N + n) * D + 16 * cb + 4 * lg, c);
  }
}

// Squared-L2 kernel values of one 64-token tile against every landmark, with
// the distance recast as |x|^2 + |l|^2 - 2 x.l and x.l on fp32 MFMA (clamped
// at zero: the expanded form can round slightly below it).  Wave w computes
// the 16x16 blocks (tokens 16 (w % 4) .., landmarks 16 jb ..) for
// jb = w / 4, w / 4 + 2; lane (g, r) supplies coordinates
// (D/4) g .. (D/4) g + D/4 - 1 of token / landmark r of its blocks: the
// token's come in av (gauss_rows), the landmark's are read from global
// memory.  Writes PTt[token][j] and, for key tiles, PJ[j][token]; landmarks
// j in [m, 16 ceil(m/16)) get exact zeros.
template <int D, bool BF16>
__device__ __forceinline__ void gauss_rows(const MainArgs& a, const void* src, int bh, int t,
                                           float (&av)[D / 4]) {
  constexpr int KS = D / 4;
  const int lane = threadIdx.x & 63, w = wave_id();
  const int lr = lane & 15, lg = lane >> 4;
  // token operand: KS coordinates of token 16 (w % 4) + lr (clamped past N)
  const int n = t * TILE + 16 * (w & 3) + lr;
  const size_t row = static_cast<size_t>(bh) * a.N + (n < a.N ? n : a.N - 1);
#pragma unroll
  for (int q = 0; q < KS / 4; ++q) {
    const f4 u = load4_io(src, row * D + KS * lg + 4 * q, BF16);
    av[4 * q] = u[0];
    av[4 * q + 1] = u[1];
    av[4 * q + 2] = u[2];
    av[4 * q + 3] = u[3];
  }
}

// Scale exponent s of a vector with squared norm p: every coordinate times
// 2^s is below 2^14 (|x_k| <= sqrt(p) < 2^ceil(e / 2) for p < 2^e).
__device__ __forceinline__ int norm_scale(float p) {
  const int e = p > 0.f ? __builtin_amdgcn_frexp_expf(p) : 0;
  return 14 - ((e + 1) >> 1);
}

template <int D, bool BF16>
__device__ __forceinline__ void gauss_tile(const MainArgs& a, const float (&av)[D / 4], const float* Lh,
                                           int t, float* PTt, uint16_t* PJH, uint16_t* PJL, float* xx,
                                           bool key_role, bool write_pt, float* kdst) {
  constexpr int KS = D / 4;  // MFMA sub-steps; floats per lane per operand
  const int lane = threadIdx.x & 63, w = wave_id();
  const int lr = lane & 15, lg = lane >> 4;
  const int tb = w & 3;
  const int m = a.m, N = a.N;
  const int mby = (m + 15) >> 4;
  float px = 0.f;
#pragma unroll
  for (int s = 0; s < KS; ++s) px = fmaf(av[s], av[s], px);
  px = sum_over_g(px);
  if (w < 4 && lg == 0) xx[16 * tb + lr] = px;
  // x.l on fp16 MFMA with scaled two-part operands (hi hi + lo hi + hi lo):
  // lane (g, r) supplies its KS coordinates in chunks of 8 (any order of the
  // k terms gives the same dot product, as long as both operands use it);
  // the token's scale comes from its squared norm, so the epilogue can
  // recompute it from xx
  constexpr int NCH = (KS + 7) / 8;
  u32x4 xh[NCH], xl[NCH];
  {
    const int sx = norm_scale(px);
#pragma unroll
    for (int p = 0; p < NCH; ++p) {
      const f4 v0 = {av[8 * p], av[8 * p + 1], av[8 * p + 2], av[8 * p + 3]};
      const f4 v1 = KS >= 8 ? f4{av[(8 * p + 4) % KS], av[(8 * p + 5) % KS], av[(8 * p + 6) % KS],
                                 av[(8 * p + 7) % KS]}
                            : f4{0.f, 0.f, 0.f, 0.f};
      split8h(v0, v1, sx, xh[p], xl[p]);
    }
  }
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
      const int sl = norm_scale(pl);
      f4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int p = 0; p < NCH; ++p) {
        const f4 v0 = {bv[8 * p], bv[8 * p + 1], bv[8 * p + 2], bv[8 * p + 3]};
        const f4 v1 = KS >= 8 ? f4{bv[(8 * p + 4) % KS], bv[(8 * p + 5) % KS], bv[(8 * p + 6) % KS],
                                   bv[(8 * p + 7) % KS]}
                              : f4{0.f, 0.f, 0.f, 0.f};
        u32x4 lh, ll;
        split8h(v0, v1, sl, lh, ll);
        c = mfma_h(xh[p], lh, c);
        c = mfma_h(xl[p], lh, c);
        c = mfma_h(xh[p], ll, c);
      }
      f4 kq;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tt = 16 * tb + 4 * lg + i;
        const float xt = xx[tt];
        const float dot = ldexpf(c[i], -(norm_scale(xt) + sl));
        const float d = fmaxf(fmaf(-2.0f, dot, xt + pl), 0.0f);
        const float kv = (j < m && t * TILE + tt < N) ? exp2_map(d * a.c_exp2) : 0.f;
        if (write_pt) PTt[ptj(tt, j)] = kv;
        // K_QL row tt of the tile straight to global memory (zero columns
        // j >= m included): no pass through LDS after the tile's barrier
        if (kdst && t * TILE + tt < N) kdst[tt * a.mpad + j] = kv;
        kq[i] = kv;
      }
      if (key_role) {
        // 4 consecutive tokens of row j: half a chunk per part, 2^14 k
        unsigned h0, l0, h1, l1;
        split2(kq[0] * 16384.f, kq[1] * 16384.f, h0, l0);
        split2(kq[2] * 16384.f, kq[3] * 16384.f, h1, l1);
        const int o = hsw(j, 16 * tb + 4 * lg);
        *reinterpret_cast<u32x2*>(PJH + o) = u32x2{h0, h1};
        *reinterpret_cast<u32x2*>(PJL + o) = u32x2{l0, l1};
      }
    }
  }
}

template <int D, int KIND, bool BF16>
__device__ __forceinline__ void map_role(const MainArgs& a, const void* __restrict__ q, const void* __restrict__ k,
                         const void* __restrict__ v, const float* __restrict__ Lw, int bh,
                         bool key_role, int unit, float* smem) {
  constexpr int CBN = D / 16;
  // PJ also holds the split W^T / Y^T copies of query workgroups
  constexpr int PJS = map_pj_size<D>();
  float* PJ = smem;                      // [64 landmarks][LS]: P[j][token]
  float* PT = smem + PJS;                // [64 tokens][LS]:    P[j] of token at [token][j]
  float* VT = smem + PJS + MP * LS;      // [D][LS]:            V[token][c] at [c][token]
  float* xx = smem + PJS + 2 * MP * LS;  // [64]: squared norms of a tile's tokens (Gaussian)
  float* XR = xx + TILE;                 // [64 tokens][XS]: token rows (Laplacian)
  // Gaussian key tiles: K_LK [landmark][token] and V^T [c][token] as fp16
  // parts of 2^14 K_LK and 2^sv V (hsw layout) in the PJ and VT areas, and
  // the per-wave maxima of |V| of the next tile (sv); their W^T product runs
  // on fp16 MFMA.  Laplacian key tiles keep both in fp32 (fp32 MFMA): their
  // maps write K_LK one token per lane, and splitting it there cost more
  // VALU time than the product saved (160-head bf16: +1.7 us per forward;
  // Gaussian Q = K: -3.6 us).
  constexpr bool SPLIT_W = KIND == 1;
  uint16_t* const PJH = reinterpret_cast<uint16_t*>(PJ);
  uint16_t* const PJL = PJH + MP * 64;
  uint16_t* const VTH = reinterpret_cast<uint16_t*>(VT);
  uint16_t* const VTL = VTH + MP * 64;
  float* const vmax = XR + (KIND == 0 ? TILE * row_stride<D>() : 0);
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
  const int lr = lane & 15, lg = lane >> 4;
  const int m = a.m, N = a.N;
  const int nK = a.nP;
  int t_beg, t_end;
  if (key_role) {
    t_beg = unit * a.S;
    t_end = min(t_beg + a.S, a.nT);
  } else {
    // qt tiles per query workgroup.  When they form their output rows here
    // (qt = QT), the K_QL rows stay in LDS until Y is ready, in PT and in the
    // V^T area, which query tiles do not use; otherwise every tile's rows are
    // stored before the next tile reuses the V^T area.
    t_beg = a.qt * unit;
    t_end = min(t_beg + a.qt, a.nT);
  }
  // K_QL goes to global memory only when Q == K (the output launch reads
  // it); query tiles keep theirs in LDS and form their output rows here.
  const bool store_kql = key_role ? a.shared_qk != 0 : a.out_in_main == 0;
  const bool stage_kql = a.st_kql && (!key_role || a.shared_qk);
  // token-major K_QL rows: query tiles (their output rows) and key tiles
  // whose K_QL is stored or staged (Q == K); other key tiles need only the
  // landmark-major rows of the W^T product
  // Gaussian tiles write their stored K_QL rows from registers
  const bool kql_direct = KIND == 1 && store_kql;
  const bool write_pt = (!key_role && a.out_in_main) || (store_kql && !kql_direct) || stage_kql;
  const void* src = key_role ? k : q;
  const int mby = (m + 15) >> 4;
  const int nwb = CBN * mby;  // W output blocks

  const int jb = (w * m) / NGRP, je = ((w + 1) * m) / NGRP;
  const float* Lh = Lw + static_cast<size_t>(bh) * m * D;
  f4 wacc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};

  // V rows of the next key tile are loaded right after this tile's kernel
  // values, before its stores and products: global loads and stores share
  // one in-order counter, so loads issued after a tile's stores would wait
  // for them too, and the load latency now overlaps the rest of the tile.
  // Gaussian tiles load the next tile's token operand (D/4 floats per lane)
  // at the same point, and Laplacian tiles the runs of their token rows.
  const int vc = tid % D, vtg = tid / D;
  constexpr int TPT = TILE * D / WGM;
  float vv[TPT];
  auto load_v = [&](int t) {
    if (key_role) {
      // V rows: thread (c, group of TPT tokens); rows past N are clamped
      // here and zeroed when staged
#pragma unroll
      for (int u = 0; u < TPT; ++u) {
        const int nv = t * TILE + vtg * TPT + u;
        vv[u] = load1_io(v, (static_cast<size_t>(bh) * N + (nv < N ? nv : N - 1)) * D + vc, BF16);
      }
    }
  };
  // max|V| of the loaded tile over this wave's threads into vmax[w] (the
  // clamped rows past N only make the scale conservative); read by every
  // wave after the next barrier, when the tile is staged
  auto publish_vmax = [&]() {
    if (SPLIT_W && key_role) {
      float mx = 0.f;
#pragma unroll
      for (int u = 0; u < TPT; ++u) mx = fmaxf(mx, fabsf(vv[u]));
      // non-negative: compares as an unsigned bit pattern
      mx = __uint_as_float(wave_max_u(__float_as_uint(mx)));
      if (lane == 0) vmax[w] = mx;
    }
  };
  float ga[KIND == 1 ? D / 4 : 1];

  // Laplacian token rows pass through LDS: thread i < 8 D loads the i-th run
  // of 8 elements of the tile (16-byte loads, consecutive threads on
  // consecutive addresses), and every wave then reads one row per lane from
  // LDS.  Read straight from global memory, each of the 8 waves fetched all
  // 64 rows with one cache line per lane and load.  The next tile's runs are
  // loaded after this tile's distances and stored after its products.
  constexpr int XS = row_stride<D>();
  const bool row_thread = KIND == 0 && tid < TILE * D / 8;
  const int rtok = tid / (D / 8), rcol = 8 * (tid % (D / 8));
  f4 rf0, rf1;  // fp32 rows: the run
  u32x4 rbv;    // bf16 rows: the run, widened when stored
  auto fetch_rows = [&](int t) {
    if (row_thread) {
      const int nt = t * TILE + rtok;
      const size_t e = (static_cast<size_t>(bh) * N + (nt < N ? nt : N - 1)) * D + rcol;
      if constexpr (BF16) {
        rbv = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(src) + e);
      } else {
        const f4* p = reinterpret_cast<const f4*>(static_cast<const float*>(src) + e);
        rf0 = p[0];
        rf1 = p[1];
      }
    }
  };
  auto stage_rows = [&]() {
    if (row_thread) {
      float* dst = XR + rtok * XS + rcol;
      if constexpr (BF16) {
        st4(dst, f4{__uint_as_float(rbv[0] << 16), __uint_as_float(rbv[0] & 0xffff0000u),
                    __uint_as_float(rbv[1] << 16), __uint_as_float(rbv[1] & 0xffff0000u)});
        st4(dst + 4, f4{__uint_as_float(rbv[2] << 16), __uint_as_float(rbv[2] & 0xffff0000u),
                        __uint_as_float(rbv[3] << 16), __uint_as_float(rbv[3] & 0xffff0000u)});
      } else {
        st4(dst, rf0);
        st4(dst + 4, rf1);
      }
    }
  };
  if (t_beg < t_end) {
    load_v(t_beg);
    if constexpr (KIND == 1) gauss_rows<D, BF16>(a, src, bh, t_beg, ga);
    if constexpr (KIND == 0) fetch_rows(t_beg);
  }
  // padding rows / columns j in [m, 64) stay zero for the whole workgroup
  for (int e = tid; e < MP * LS; e += WGM) {
    PJ[e] = 0.f;
    PT[e] = 0.f;
    if (!key_role) VT[e] = 0.f;
  }
  if (KIND == 0 && t_beg < t_end) stage_rows();
  if (t_beg < t_end) publish_vmax();
  __syncthreads();

  for (int t = t_beg; t < t_end; ++t) {
    float* PTt = (key_role || t == t_beg) ? PT : VT;  // this tile's K_QL rows
    const int n = t * TILE + lane;
    const bool valid = n < N;
    float x[KIND == 0 ? D : 1];
    if constexpr (KIND == 0) {
#pragma unroll
      for (int i = 0; i < D / 4; ++i) {
        const f4 u = ld4(XR + lane * XS + 4 * i);
        x[4 * i] = u[0];
        x[4 * i + 1] = u[1];
        x[4 * i + 2] = u[2];
        x[4 * i + 3] = u[3];
      }
    }
    int sv = 0;  // V^T scale of this tile: max|V| 2^sv < 2^15
    if (key_role && !SPLIT_W) {
      // V tile -> VT[c][token] (VT is free: the previous tile's products
      // finished before the barrier that ended its iteration).  A thread's
      // TPT consecutive tokens of column c go out as 16-byte stores: lanes
      // c = 0..15 of a store then cover all banks (single stores put lanes
      // c and c + 16 on one bank).
      float vz[TPT];
#pragma unroll
      for (int u = 0; u < TPT; ++u) vz[u] = t * TILE + vtg * TPT + u < N ? vv[u] : 0.f;
      float* vdst = VT + vc * LS + vtg * TPT;
      if constexpr (TPT % 4 == 0) {
#pragma unroll
        for (int u = 0; u < TPT; u += 4) st4(vdst + u, f4{vz[u], vz[u + 1], vz[u + 2], vz[u + 3]});
      } else {
#pragma unroll
        for (int u = 0; u < TPT; ++u) vdst[u] = vz[u];
      }
    }
    if (key_role && SPLIT_W) {
      // V tile -> V^T as fp16 parts of 2^sv V (the VT area is free: the
      // previous tile's products finished before the barrier that ended its
      // iteration).  A thread's TPT consecutive tokens of column c are one
      // run of a row: one store per part.
      float mxv = vmax[0];
#pragma unroll
      for (int i = 1; i < WGM / 64; ++i) mxv = fmaxf(mxv, vmax[i]);
      // (capped so that 2^-(sv + 14) stays a normal fp32 number)
      sv = min(fp16_scale(mxv), 100);
      float vz[TPT];
#pragma unroll
      for (int u = 0; u < TPT; ++u) vz[u] = t * TILE + vtg * TPT + u < N ? ldexpf(vv[u], sv) : 0.f;
      unsigned hv[TPT / 2], lv[TPT / 2];
#pragma unroll
      for (int u = 0; u < TPT; u += 2) split2(vz[u], vz[u + 1], hv[u / 2], lv[u / 2]);
      const int o = hsw(vc, vtg * TPT);
      if constexpr (TPT == 8) {
        *reinterpret_cast<u32x4*>(VTH + o) = u32x4{hv[0], hv[1], hv[2], hv[3]};
        *reinterpret_cast<u32x4*>(VTL + o) = u32x4{lv[0], lv[1], lv[2], lv[3]};
      } else if constexpr (TPT == 4) {
        *reinterpret_cast<u32x2*>(VTH + o) = u32x2{hv[0], hv[1]};
        *reinterpret_cast<u32x2*>(VTL + o) = u32x2{lv[0], lv[1]};
      } else {
        static_assert(TPT == 2, "runs of 2, 4 or 8 tokens");
        *reinterpret_cast<unsigned*>(VTH + o) = hv[0];
        *reinterpret_cast<unsigned*>(VTL + o) = lv[0];
      }
    }
    if constexpr (KIND == 0) {
      // L1 distances on VALU: landmarks two at a time (their scalar loads
      // overlap); an odd last landmark on its own
      int j = jb;
      for (; j + 1 < je; j += 2) {
        float d0, d1;
        dist_to2<D, KIND>(x, Lh + j * D, Lh + (j + 1) * D, d0, d1);
        const float k0 = valid ? exp2_map(d0 * a.c_exp2) : 0.f;
        const float k1 = valid ? exp2_map(d1 * a.c_exp2) : 0.f;
        if (key_role) {
          PJ[j * LS + lane] = k0;
          PJ[(j + 1) * LS + lane] = k1;
        }
        if (write_pt) {
          PTt[ptj(lane, j)] = k0;
          PTt[ptj(lane, j + 1)] = k1;
        }
      }
      if (j < je) {
        const float k0 = valid ? exp2_map(dist_to<D, KIND>(x, Lh + j * D) * a.c_exp2) : 0.f;
        if (key_role) PJ[j * LS + lane] = k0;
        if (write_pt) PTt[ptj(lane, j)] = k0;
      }
    } else {
      gauss_tile<D, BF16>(a, ga, Lh, t, PTt, PJH, PJL, xx, key_role, write_pt,
                          kql_direct ? a.kql + (static_cast<size_t>(bh) * N + t * TILE) * a.mpad : nullptr);
    }
    if (t + 1 < t_end) {
      load_v(t + 1);
      if constexpr (KIND == 1) gauss_rows<D, BF16>(a, src, bh, t + 1, ga);
      if constexpr (KIND == 0) fetch_rows(t + 1);
    }
    __syncthreads();
    if (store_kql && !kql_direct) {
      // 64 rows of mpad floats, contiguous in global memory
      const int q4 = a.mpad / 4;
      float* dst = a.kql + (static_cast<size_t>(bh) * N + t * TILE) * a.mpad;
      for (int e = tid; e < TILE * q4; e += WGM) {
        const int tok = e / q4, c4 = e % q4;
        const float* src4 = PTt + ptj(tok, 4 * c4);
        if (t * TILE + tok < N) st4(dst + tok * a.mpad + 4 * c4, f4{src4[0], src4[1], src4[2], src4[3]});
      }
    }
    if (stage_kql) {
      for (int e = tid; e < TILE * m; e += WGM) {
        const int tok = e / m, j = e % m;
        if (t * TILE + tok < N)
          a.st_kql[(static_cast<size_t>(bh) * N + t * TILE + tok) * m + j] = PTt[ptj(tok, j)];
      }
    }
    if (key_role) {
      if (a.st_klk) {
        for (int e = tid; e < m * TILE; e += WGM) {
          const int j = e / TILE, tok = e % TILE;
          float kv = PJ[j * LS + tok];
          if constexpr (SPLIT_W) {
            const int o = hsw(j, tok);
            kv = (static_cast<float>(__builtin_bit_cast(_Float16, PJH[o])) +
                  static_cast<float>(__builtin_bit_cast(_Float16, PJL[o]))) * 0x1p-14f;
          }
          if (t * TILE + tok < N) a.st_klk[(static_cast<size_t>(bh) * m + j) * N + t * TILE + tok] = kv;
        }
      }
      // W^T[c][j] += sum_token V^T[c][token] P[j][token]: on fp32 MFMA, or
      // (Gaussian) on fp16 MFMA with the scaled two-part operands (hi hi +
      // lo hi + hi lo), the tile's scale 2^(sv + 14) taken out as it is added
      const float unscale = ldexpf(1.0f, -(sv + 14));
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int blk = w + 8 * s;
        if (!SPLIT_W && blk < nwb) {
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
        if (SPLIT_W && blk < nwb) {
          const int cb = blk % CBN, jbk = blk / CBN;
          const int ra = 16 * cb + lr, rb = 16 * jbk + lr;
          f4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            const int k0 = 32 * p + 8 * lg;
            const u32x4 ah = *reinterpret_cast<const u32x4*>(VTH + hsw(ra, k0));
            const u32x4 al = *reinterpret_cast<const u32x4*>(VTL + hsw(ra, k0));
            const u32x4 bh2 = *reinterpret_cast<const u32x4*>(PJH + hsw(rb, k0));
            const u32x4 bl2 = *reinterpret_cast<const u32x4*>(PJL + hsw(rb, k0));
            c = mfma_h(ah, bh2, c);
            c = mfma_h(al, bh2, c);
            c = mfma_h(ah, bl2, c);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) wacc[s][i] = fmaf(c[i], unscale, wacc[s][i]);
        }
      }
    }
    // every wave read this tile's rows before the barrier above
    if (KIND == 0 && t + 1 < t_end) stage_rows();
    if (t + 1 < t_end) publish_vmax();
    __syncthreads();
  }
  if (!key_role) {
    if (!a.out_in_main) return;  // K_QL stored; the output launch forms O
    // Query workgroup u < R reduces its slice of W^T once every key
    // workgroup of the head has published its partial.
    const int u = unit;
    constexpr int LINES = D * MP / 32;  // cache lines of W^T
    const int R = a.nQ < 32 ? a.nQ : 32;
    const int lps = (LINES + R - 1) / R;
    const int nslice = (LINES + lps - 1) / lps;
    if (u < nslice) {
      wait_flags(key_flags(a, bh), nK, a.timeouts);
      reduce_w_lines<D>(a, bh, u * lps, min((u + 1) * lps, LINES), PJ);
      raise_flag(slice_flags(a, bh) + u);
    }
    // W^T complete: copy it to LDS (PJ is unused by query tiles) while the
    // solver may still be running; then Y^T = W^T X^T in place, then the
    // output rows of the tiles (K_QL rows in LDS)
    wait_flags(slice_flags(a, bh), nslice, a.timeouts);
    {
      // row c of W^T (8 threads, consecutive lanes) scaled by 2^EW[c] into
      // fp16 range, split
      using QG = QGeom<D>;
      static_assert(D * (MP / 8) <= WGM, "one W^T chunk per thread");
      uint16_t* WH = reinterpret_cast<uint16_t*>(PJ);
      uint16_t* WL = reinterpret_cast<uint16_t*>(PJ + QG::OFF_WL);
      int* EW = reinterpret_cast<int*>(PJ + QG::OFF_EW);
      const float* wg = a.wt + static_cast<size_t>(bh) * D * MP;
      if (tid < D * (MP / 8)) {
        const int row = tid / (MP / 8), k8 = 8 * (tid % (MP / 8));
        const f4 v0 = ld4(wg + row * MP + k8), v1 = ld4(wg + row * MP + k8 + 4);
        unsigned m = 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          m = max(m, max(__float_as_uint(v0[i]) & 0x7fffffffu, __float_as_uint(v1[i]) & 0x7fffffffu));
        const int ew = fp16_scale(__uint_as_float(max8_u(m)));
        u32x4 hv, lv;
        split8h(v0, v1, ew, hv, lv);
        *reinterpret_cast<u32x4*>(WH + row * WLD + k8) = hv;
        *reinterpret_cast<u32x4*>(WL + row * WLD + k8) = lv;
        if (k8 == 0) EW[row] = ew;
      }
    }
    const int ex = static_cast<int16_t>(wait_flag(flag_x(a, bh), a.timeouts) & 0xffffu);
    {
      const uint16_t* xh = reinterpret_cast<const uint16_t*>(a.xw + static_cast<size_t>(bh) * MP * MP);
      y_in_lds<D>(PJ, xh, xh + MP * MP);
    }
    out_tile<D>(a, bh, t_beg, PT, PJ, ex);
    if (t_beg + 1 < t_end) out_tile<D>(a, bh, t_beg + 1, VT, PJ, ex);
    return;
  }

  const int kw = unit;
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
  if (a.partials_only) return;
  if (a.out_in_main) {
    // the query workgroups reduce the partials
    raise_flag(key_flags(a, bh) + kw);
    return;
  }
  // the last key workgroup of the head reduces the partials
  if (publish_arrive(cnt_w(a, bh)) == static_cast<unsigned>(nK - 1)) {
    reduce_w<D>(a, bh);
    arrive_y<D>(a, bh);
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

}  // namespace
}  // namespace lapattn
