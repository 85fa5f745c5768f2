// HIP kernels for Nystrom kernel attention (forward) on gfx950.
//
// Stages (one head = one (b, h) pair, all heads batched in every launch):
//   pool  : landmarks L = window means of K                   (HBM stream)
//   ns    : A = k(L, L) + eps I, alpha, Newton-Schulz in LDS   (one CU per head,
//           fp32 MFMA 16x16x4)
//   maps  : K_QL^T, K_LK^T = exp(-dist(token, landmark)/lambda) (FP32 VALU; the
//           landmark coordinates are wave-uniform scalar operands)
//   w     : W = K_LK V as per-chunk partials on fp32 MFMA, deterministic
//           last-block reduction, then the join that forms Y = X W
//   out   : O = K_QL Y on fp32 MFMA, fp32 or bf16 (RNE) store
//
// Pages behind each step: average-pool landmarks (SOFT review, "method";
// LaplacianFormer summaries, Nystrom paragraph), Laplacian kernel
// exp(-||x-y||_1/lambda) (LaplacianFormer summaries, kernel definition),
// Gaussian exp(Q (-) K) (SOFT review, "method"), eps I perturbation and the
// Newton-Schulz recursion A_0 = alpha A, A_{k+1} = 2 A_k - A_k A A_k
// (LaplacianFormer summaries; SOFT review, "method"), S_hat = P^T A^+ P
// (SOFT review, "method").

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lapattn_internal.h"

namespace lapattn {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int LDA = MP + 1;   // LDS row stride of the 64x64 solver matrices
constexpr int WG = 256;       // 4 wave64 per workgroup everywhere

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

template <bool BF16>
__device__ __forceinline__ float load_elem(const void* p, size_t i) {
  if constexpr (BF16) {
    return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
  } else {
    return static_cast<const float*>(p)[i];
  }
}

// Loads D consecutive elements (one token row) into registers as fp32.
template <int D, bool BF16>
__device__ __forceinline__ void load_row(const void* base, size_t row, float* x) {
  if constexpr (BF16) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + row * D);
#pragma unroll
    for (int i = 0; i < D / 8; ++i) {
      uint4 u = p[i];
      uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        x[8 * i + 2 * h] = __uint_as_float(w[h] << 16);
        x[8 * i + 2 * h + 1] = __uint_as_float(w[h] & 0xffff0000u);
      }
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + row * D);
#pragma unroll
    for (int i = 0; i < D / 4; ++i) {
      float4 u = p[i];
      x[4 * i] = u.x;
      x[4 * i + 1] = u.y;
      x[4 * i + 2] = u.z;
      x[4 * i + 3] = u.w;
    }
  }
}

__device__ __forceinline__ f4 mfma4(float a, float b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

// ---------------------------------------------------------------------------
// pool: one workgroup per (landmark, head).  Thread (g, c) sums coordinate c
// over every (WG/D)-th token of the window; a fixed-order LDS reduction
// finishes the mean.  Workgroup (0, bh) also clears the head's counters.
// ---------------------------------------------------------------------------
template <int D, bool BF16>
__global__ __launch_bounds__(WG) void pool_kernel(const void* __restrict__ K,
                                                  float* __restrict__ L,
                                                  unsigned* __restrict__ ctr,
                                                  float* __restrict__ st_L, int gw,
                                                  int ph, int pw, int m, int N) {
  constexpr int G = WG / D;
  __shared__ float part[WG];
  const int j = blockIdx.x, bh = blockIdx.y;
  const int tid = threadIdx.x, c = tid % D, g = tid / D;
  const int mw = gw / pw;
  const int R = j / mw, C = j % mw;
  const int cnt = ph * pw;
  float s = 0.f;
  for (int t = g; t < cnt; t += G) {
    const int n = (R * ph + t / pw) * gw + C * pw + t % pw;
    s += load_elem<BF16>(K, (static_cast<size_t>(bh) * N + n) * D + c);
  }
  part[tid] = s;
  __syncthreads();
  if (g == 0) {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < G; ++i) acc += part[i * D + c];
    const float mean = acc / static_cast<float>(cnt);
    L[(static_cast<size_t>(bh) * m + j) * D + c] = mean;
    if (st_L) st_L[(static_cast<size_t>(bh) * m + j) * D + c] = mean;
  }
  if (j == 0 && tid < CTR_PER_HEAD) ctr[bh * CTR_PER_HEAD + tid] = 0u;
}

// ---------------------------------------------------------------------------
// Y = X W for one head, all 256 threads: wave w computes rows 16w..16w+15.
// X [MP][MP] and W [MP][D] are read from global memory (after an acquire).
// ---------------------------------------------------------------------------
template <int D>
__device__ void compute_y(const float* __restrict__ X, const float* __restrict__ W,
                          float* __restrict__ Y, int m) {
  constexpr int CB = D / 16;
  const int lane = threadIdx.x & 63, w = wave_id();
  const int ksteps = (m + 3) >> 2;
  f4 acc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) acc[cb] = f4{0.f, 0.f, 0.f, 0.f};
  for (int kk = 0; kk < ksteps; ++kk) {
    const int kr = 4 * kk + (lane >> 4);
    const float a = X[(16 * w + (lane & 15)) * MP + kr];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const float b = W[kr * D + 16 * cb + (lane & 15)];
      acc[cb] = mfma4(a, b, acc[cb]);
    }
  }
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      Y[(16 * w + 4 * (lane >> 4) + i) * D + 16 * cb + (lane & 15)] = acc[cb][i];
}

// Last-arrival join: returns true in every thread of the workgroup that
// completes the count.  All prior global stores of the workgroup are released
// before the increment and the winner acquires before returning.
__device__ __forceinline__ bool arrive(unsigned* counter, unsigned target, int* flag_lds) {
  __syncthreads();
  if (threadIdx.x == 0) {
    __threadfence();
    const unsigned old = atomicAdd(counter, 1u);
    *flag_lds = (old + 1u == target) ? 1 : 0;
  }
  __syncthreads();
  const bool last = *flag_lds != 0;
  if (last) __threadfence();
  return last;
}

// ---------------------------------------------------------------------------
// ns: one workgroup per head.  A = k(L, L) + eps I is built in LDS, then
// `iters` Newton-Schulz steps run on fp32 MFMA with every matrix held in LDS:
//   T = A X_t        (A operand held in registers for the whole solve)
//   X_{t+1} = 2 X_t - X_t T
// Wave w owns block-row w (rows 16w..16w+15) of every product.
// ---------------------------------------------------------------------------
template <int D, int KIND>
__global__ __launch_bounds__(WG) void ns_kernel(const float* __restrict__ Lw,
                                                float* __restrict__ Xw,
                                                const float* __restrict__ Ww,
                                                float* __restrict__ Yw,
                                                unsigned* __restrict__ ctr,
                                                float* __restrict__ st_a,
                                                float* __restrict__ st_x, int m,
                                                float c_exp2, float eps, int iters,
                                                int join_target) {
  __shared__ float S0[MP * LDA];  // L, then T
  __shared__ float S1[MP * LDA];  // A, then X buffer 1
  __shared__ float S2[MP * LDA];  // X buffer 0
  __shared__ float red[2 * WG];
  __shared__ int flag;
  const int bh = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
  const int lr = lane & 15, lg = lane >> 4;
  const int ksteps = (m + 3) >> 2;

  // Landmarks -> LDS (row stride D+1), zero the A buffer.
  const float* L = Lw + static_cast<size_t>(bh) * m * D;
  for (int e = tid; e < m * D; e += WG) S0[(e / D) * (D + 1) + (e % D)] = L[e];
  for (int e = tid; e < MP * LDA; e += WG) S1[e] = 0.f;
  __syncthreads();

  // A[i][j] for i <= j, mirrored: the distance is symmetric term by term.
  for (int e = tid; e < m * m; e += WG) {
    const int i = e / m, j = e - i * m;
    if (i > j) continue;
    const float* li = S0 + i * (D + 1);
    const float* lj = S0 + j * (D + 1);
    float d0 = 0.f, d1 = 0.f;
#pragma unroll
    for (int k = 0; k < D; k += 2) {
      const float t0 = li[k] - lj[k];
      const float t1 = li[k + 1] - lj[k + 1];
      if constexpr (KIND == 0) {
        d0 += fabsf(t0);
        d1 += fabsf(t1);
      } else {
        d0 = fmaf(t0, t0, d0);
        d1 = fmaf(t1, t1, d1);
      }
    }
    float a = exp2f((d0 + d1) * c_exp2);
    if (i == j) a += eps;
    S1[i * LDA + j] = a;
    S1[j * LDA + i] = a;
  }
  __syncthreads();

  if (st_a) {
    for (int e = tid; e < m * m; e += WG)
      st_a[static_cast<size_t>(bh) * m * m + e] = S1[(e / m) * LDA + (e % m)];
  }

  // alpha = 1 / (max column abs-sum * max row abs-sum).
  {
    float cs = 0.f, rs = 0.f;
    if (tid < m) {
      for (int i = 0; i < m; ++i) {
        cs += fabsf(S1[i * LDA + tid]);
        rs += fabsf(S1[tid * LDA + i]);
      }
    }
    red[tid] = cs;
    red[WG + tid] = rs;
  }
  __syncthreads();
  for (int s = WG / 2; s > 0; s >>= 1) {
    if (tid < s) {
      red[tid] = fmaxf(red[tid], red[tid + s]);
      red[WG + tid] = fmaxf(red[WG + tid], red[WG + tid + s]);
    }
    __syncthreads();
  }
  const float alpha = 1.0f / (red[0] * red[WG]);

  // A operand of T = A X (block-row w) stays in registers.
  float a_reg[16];
#pragma unroll
  for (int kk = 0; kk < 16; ++kk) a_reg[kk] = S1[(16 * w + lr) * LDA + 4 * kk + lg];
  // X_0 = alpha A, block-row w in accumulator layout.
  f4 xr[4];
#pragma unroll
  for (int bj = 0; bj < 4; ++bj)
#pragma unroll
    for (int i = 0; i < 4; ++i) xr[bj][i] = alpha * S1[(16 * w + 4 * lg + i) * LDA + 16 * bj + lr];
#pragma unroll
  for (int bj = 0; bj < 4; ++bj)
#pragma unroll
    for (int i = 0; i < 4; ++i) S2[(16 * w + 4 * lg + i) * LDA + 16 * bj + lr] = xr[bj][i];
  __syncthreads();

  for (int t = 0; t < iters; ++t) {
    float* Xc = (t & 1) ? S1 : S2;
    float* Xn = (t & 1) ? S2 : S1;
    // T = A X_t
    f4 acc[4];
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) acc[bj] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      if (kk < ksteps) {
#pragma unroll
        for (int bj = 0; bj < 4; ++bj) {
          const float b = Xc[(4 * kk + lg) * LDA + 16 * bj + lr];
          acc[bj] = mfma4(a_reg[kk], b, acc[bj]);
        }
      }
    }
#pragma unroll
    for (int bj = 0; bj < 4; ++bj)
#pragma unroll
      for (int i = 0; i < 4; ++i) S0[(16 * w + 4 * lg + i) * LDA + 16 * bj + lr] = acc[bj][i];
    __syncthreads();
    // X_{t+1} = 2 X_t - X_t T
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) acc[bj] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      if (kk < ksteps) {
        const float a = Xc[(16 * w + lr) * LDA + 4 * kk + lg];
#pragma unroll
        for (int bj = 0; bj < 4; ++bj) {
          const float b = S0[(4 * kk + lg) * LDA + 16 * bj + lr];
          acc[bj] = mfma4(a, b, acc[bj]);
        }
      }
    }
#pragma unroll
    for (int bj = 0; bj < 4; ++bj)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xr[bj][i] = 2.0f * xr[bj][i] - acc[bj][i];
        Xn[(16 * w + 4 * lg + i) * LDA + 16 * bj + lr] = xr[bj][i];
      }
    __syncthreads();
  }

  float* X = Xw + static_cast<size_t>(bh) * MP * MP;
#pragma unroll
  for (int bj = 0; bj < 4; ++bj)
#pragma unroll
    for (int i = 0; i < 4; ++i) X[(16 * w + 4 * lg + i) * MP + 16 * bj + lr] = xr[bj][i];
  if (st_x) {
#pragma unroll
    for (int bj = 0; bj < 4; ++bj)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + 4 * lg + i, c = 16 * bj + lr;
        if (r < m && c < m) st_x[static_cast<size_t>(bh) * m * m + r * m + c] = xr[bj][i];
      }
  }

  if (arrive(&ctr[bh * CTR_PER_HEAD + 1], static_cast<unsigned>(join_target), &flag)) {
    compute_y<D>(X, Ww + static_cast<size_t>(bh) * MP * D, Yw + static_cast<size_t>(bh) * MP * D, m);
  }
}

// ---------------------------------------------------------------------------
// maps: each wave computes the kernel values of 64 tokens (one per lane, the
// token's D coordinates in registers) against a group of landmarks.  The
// landmark coordinates are wave-uniform and are read with scalar loads, so the
// inner loop is two VALU operations per coordinate pair (sub, add with |.|
// modifier; sub, fma for the Gaussian).  Results go to [m][N] rows so every
// store is one coalesced 256-byte line per landmark.
// Work unit u = (role, head, tile, group), group fastest.
// ---------------------------------------------------------------------------
template <int D, int KIND, bool BF16>
__global__ __launch_bounds__(WG) void maps_kernel(const void* __restrict__ Q,
                                                  const void* __restrict__ K,
                                                  const float* __restrict__ Lw,
                                                  float* __restrict__ kqlt,
                                                  float* __restrict__ klkt, int N, int m,
                                                  int nT, int ng, int nroles, int BH,
                                                  float c_exp2) {
  const int lane = threadIdx.x & 63;
  const int u = blockIdx.x * (WG / 64) + wave_id();
  const int total = nroles * BH * nT * ng;
  if (u >= total) return;
  const int g = u % ng;
  const int r1 = u / ng;
  const int t = r1 % nT;
  const int r2 = r1 / nT;
  const int bh = r2 % BH;
  const int role = r2 / BH;  // 0: keys -> K_LK^T, 1: queries -> K_QL^T
  const void* src = role == 0 ? K : Q;
  float* dst = role == 0 ? klkt : kqlt;

  const int n = t * 64 + lane;
  const int nc = n < N ? n : N - 1;
  float x[D];
  load_row<D, BF16>(src, static_cast<size_t>(bh) * N + nc, x);

  const int jb = (g * m) / ng, je = ((g + 1) * m) / ng;
  const float* Lh = Lw + static_cast<size_t>(bh) * m * D;
  float* out = dst + static_cast<size_t>(bh) * m * N + n;
  for (int j = jb; j < je; ++j) {
    const float* lj = Lh + j * D;
    float d0 = 0.f, d1 = 0.f;
#pragma unroll
    for (int k = 0; k < D; k += 2) {
      const float t0 = x[k] - lj[k];
      const float t1 = x[k + 1] - lj[k + 1];
      if constexpr (KIND == 0) {
        d0 += fabsf(t0);
        d1 += fabsf(t1);
      } else {
        d0 = fmaf(t0, t0, d0);
        d1 = fmaf(t1, t1, d1);
      }
    }
    const float kv = exp2f((d0 + d1) * c_exp2);
    if (n < N) out[static_cast<size_t>(j) * N] = kv;
  }
}

// ---------------------------------------------------------------------------
// w: W = K_LK V.  Workgroup (head, chunk) reduces CH tokens on fp32 MFMA
// (wave w: landmark rows 16w..16w+15, all D columns) into a partial; the last
// chunk of a head sums the partials in fixed order (deterministic), then
// joins with the solver: whichever finishes second forms Y = X W.
// Within a 16-token step, lane group g = lane/16 owns tokens 4g..4g+3 and MFMA
// sub-step s consumes token 4g+s from both operands.
// ---------------------------------------------------------------------------
template <int D, bool BF16>
__global__ __launch_bounds__(WG) void w_kernel(const float* __restrict__ klkt,
                                               const void* __restrict__ V,
                                               float* __restrict__ wpart,
                                               float* __restrict__ Ww,
                                               const float* __restrict__ Xw,
                                               float* __restrict__ Yw,
                                               unsigned* __restrict__ ctr,
                                               float* __restrict__ st_w, int N, int m,
                                               int CH, int nC, int join_target) {
  constexpr int CB = D / 16;
  __shared__ int flag;
  const int bh = blockIdx.x / nC, ch = blockIdx.x % nC;
  const int lane = threadIdx.x & 63, w = wave_id();
  const int lr = lane & 15, lg = lane >> 4;
  const int row = 16 * w + lr;
  const bool row_ok = row < m;
  const float* P = klkt + (static_cast<size_t>(bh) * m + (row_ok ? row : 0)) * N;
  const size_t vbase = static_cast<size_t>(bh) * N;

  f4 acc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) acc[cb] = f4{0.f, 0.f, 0.f, 0.f};
  const int n_beg = ch * CH;
  const int n_end = min(n_beg + CH, N);
  for (int n0 = n_beg; n0 < n_end; n0 += 16) {
    const int nt = n0 + 4 * lg;
    float pa[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) pa[s] = (row_ok && nt + s < n_end) ? P[nt + s] : 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int nv = nt + s;
      const bool ok = nv < n_end;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const float b = ok ? load_elem<BF16>(V, (vbase + nv) * D + 16 * cb + lr) : 0.f;
        acc[cb] = mfma4(pa[s], b, acc[cb]);
      }
    }
  }
  float* part = wpart + (static_cast<size_t>(bh) * nC + ch) * MP * D;
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int i = 0; i < 4; ++i) part[(16 * w + 4 * lg + i) * D + 16 * cb + lr] = acc[cb][i];

  if (!arrive(&ctr[bh * CTR_PER_HEAD + 0], static_cast<unsigned>(nC), &flag)) return;

  // Last chunk of this head: W = sum of partials, chunk order 0..nC-1.
  const float* pbase = wpart + static_cast<size_t>(bh) * nC * MP * D;
  float* W = Ww + static_cast<size_t>(bh) * MP * D;
  for (int e = threadIdx.x; e < MP * D; e += WG) {
    const int r = e / D;
    float s = 0.f;
    if (r < m) {
      for (int c = 0; c < nC; ++c) s += pbase[static_cast<size_t>(c) * MP * D + e];
      if (st_w) st_w[(static_cast<size_t>(bh) * m + r) * D + (e % D)] = s;
    }
    W[e] = s;
  }
  if (arrive(&ctr[bh * CTR_PER_HEAD + 1], static_cast<unsigned>(join_target), &flag)) {
    compute_y<D>(Xw + static_cast<size_t>(bh) * MP * MP, W, Yw + static_cast<size_t>(bh) * MP * D, m);
  }
}

// ---------------------------------------------------------------------------
// out: O = K_QL Y.  Workgroup = (head, 64 tokens); wave w computes tokens
// 16w..16w+15 of the tile against all D columns, contraction over landmarks.
// ---------------------------------------------------------------------------
template <int D, bool BF16>
__global__ __launch_bounds__(WG) void out_kernel(const float* __restrict__ kqlt,
                                                 const float* __restrict__ Yw,
                                                 void* __restrict__ O, int N, int m,
                                                 int nT) {
  constexpr int CB = D / 16;
  const int bh = blockIdx.x / nT, t = blockIdx.x % nT;
  const int lane = threadIdx.x & 63, w = wave_id();
  const int lr = lane & 15, lg = lane >> 4;
  const int nb = t * 64 + 16 * w;
  const int na = nb + lr;
  const bool na_ok = na < N;
  const float* P = kqlt + static_cast<size_t>(bh) * m * N + (na_ok ? na : 0);
  const float* Y = Yw + static_cast<size_t>(bh) * MP * D;
  const int ksteps = (m + 3) >> 2;
  f4 acc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) acc[cb] = f4{0.f, 0.f, 0.f, 0.f};
  for (int kk = 0; kk < ksteps; ++kk) {
    const int j = 4 * kk + lg;
    const float a = (na_ok && j < m) ? P[static_cast<size_t>(j) * N] : 0.f;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[cb] = mfma4(a, Y[j * D + 16 * cb + lr], acc[cb]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int n = nb + 4 * lg + i;
    if (n < N) {
      const size_t o = (static_cast<size_t>(bh) * N + n) * D + lr;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        if constexpr (BF16) {
          static_cast<uint16_t*>(O)[o + 16 * cb] = f32_to_bf16_rne(acc[cb][i]);
        } else {
          static_cast<float*>(O)[o + 16 * cb] = acc[cb][i];
        }
      }
    }
  }
}

// Stage export: K_QL in [N][m] layout and K_LK in [m][N] layout.
__global__ __launch_bounds__(WG) void export_kernel(const float* __restrict__ kqlt,
                                                    const float* __restrict__ klkt,
                                                    float* __restrict__ st_kql,
                                                    float* __restrict__ st_klk, int N,
                                                    int m, size_t total) {
  for (size_t e = blockIdx.x * static_cast<size_t>(WG) + threadIdx.x; e < total;
       e += static_cast<size_t>(gridDim.x) * WG) {
    const size_t bh = e / (static_cast<size_t>(m) * N);
    const size_t r = e % (static_cast<size_t>(m) * N);
    const size_t j = r / N, n = r % N;
    if (st_klk) st_klk[e] = klkt[e];
    if (st_kql) st_kql[(bh * N + n) * m + j] = kqlt[e];
  }
}

inline float exp2_scale(float lambda) {
  // exp(-d / lambda) = exp2(d * (-log2(e) / lambda))
  return static_cast<float>(-1.4426950408889634 / static_cast<double>(lambda));
}

template <int D>
hipError_t launch_pool_d(const Plan& p, const Args& a, const Buffers& b, hipStream_t s) {
  dim3 grid(p.m, p.BH);
  if (p.bf16)
    hipLaunchKernelGGL((pool_kernel<D, true>), grid, dim3(WG), 0, s, a.k, b.L, b.ctr, a.st_L,
                       p.gw, p.ph, p.pw, p.m, p.N);
  else
    hipLaunchKernelGGL((pool_kernel<D, false>), grid, dim3(WG), 0, s, a.k, b.L, b.ctr, a.st_L,
                       p.gw, p.ph, p.pw, p.m, p.N);
  return hipGetLastError();
}

template <int D>
hipError_t launch_ns_d(const Plan& p, const Args& a, const Buffers& b, int jt, hipStream_t s) {
  const float c = exp2_scale(a.lambda);
  if (p.kernel == 0)
    hipLaunchKernelGGL((ns_kernel<D, 0>), dim3(p.BH), dim3(WG), 0, s, b.L, b.x, b.w, b.y, b.ctr,
                       a.st_a, a.st_x, p.m, c, a.eps, a.iters, jt);
  else
    hipLaunchKernelGGL((ns_kernel<D, 1>), dim3(p.BH), dim3(WG), 0, s, b.L, b.x, b.w, b.y, b.ctr,
                       a.st_a, a.st_x, p.m, c, a.eps, a.iters, jt);
  return hipGetLastError();
}

template <int D, int KIND>
hipError_t launch_maps_dk(const Plan& p, const Args& a, const Buffers& b, hipStream_t s) {
  const int nroles = a.shared_qk ? 1 : 2;
  const long units = static_cast<long>(nroles) * p.BH * p.nT * p.ng;
  const unsigned blocks = static_cast<unsigned>((units + 3) / 4);
  const float c = exp2_scale(a.lambda);
  if (p.bf16)
    hipLaunchKernelGGL((maps_kernel<D, KIND, true>), dim3(blocks), dim3(WG), 0, s, a.q, a.k, b.L,
                       b.kqlt, b.klkt, p.N, p.m, p.nT, p.ng, nroles, p.BH, c);
  else
    hipLaunchKernelGGL((maps_kernel<D, KIND, false>), dim3(blocks), dim3(WG), 0, s, a.q, a.k, b.L,
                       b.kqlt, b.klkt, p.N, p.m, p.nT, p.ng, nroles, p.BH, c);
  return hipGetLastError();
}

template <int D>
hipError_t launch_w_d(const Plan& p, const Args& a, const Buffers& b, int jt, hipStream_t s) {
  dim3 grid(p.BH * p.nC);
  if (p.bf16)
    hipLaunchKernelGGL((w_kernel<D, true>), grid, dim3(WG), 0, s, b.klkt, a.v, b.wpart, b.w, b.x,
                       b.y, b.ctr, a.st_w, p.N, p.m, p.CH, p.nC, jt);
  else
    hipLaunchKernelGGL((w_kernel<D, false>), grid, dim3(WG), 0, s, b.klkt, a.v, b.wpart, b.w, b.x,
                       b.y, b.ctr, a.st_w, p.N, p.m, p.CH, p.nC, jt);
  return hipGetLastError();
}

template <int D>
hipError_t launch_out_d(const Plan& p, const Args& a, const Buffers& b, hipStream_t s) {
  const float* kql = a.shared_qk ? b.klkt : b.kqlt;
  dim3 grid(p.BH * p.nT);
  if (p.bf16)
    hipLaunchKernelGGL((out_kernel<D, true>), grid, dim3(WG), 0, s, kql, b.y, a.out, p.N, p.m,
                       p.nT);
  else
    hipLaunchKernelGGL((out_kernel<D, false>), grid, dim3(WG), 0, s, kql, b.y, a.out, p.N, p.m,
                       p.nT);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pool(const Plan& p, const Args& a, const Buffers& b, hipStream_t s) {
  switch (p.D) {
    case 16: return launch_pool_d<16>(p, a, b, s);
    case 32: return launch_pool_d<32>(p, a, b, s);
    case 64: return launch_pool_d<64>(p, a, b, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_ns(const Plan& p, const Args& a, const Buffers& b, int jt, hipStream_t s) {
  switch (p.D) {
    case 16: return launch_ns_d<16>(p, a, b, jt, s);
    case 32: return launch_ns_d<32>(p, a, b, jt, s);
    case 64: return launch_ns_d<64>(p, a, b, jt, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_maps(const Plan& p, const Args& a, const Buffers& b, hipStream_t s) {
  const bool gauss = p.kernel != 0;
  switch (p.D) {
    case 16: return gauss ? launch_maps_dk<16, 1>(p, a, b, s) : launch_maps_dk<16, 0>(p, a, b, s);
    case 32: return gauss ? launch_maps_dk<32, 1>(p, a, b, s) : launch_maps_dk<32, 0>(p, a, b, s);
    case 64: return gauss ? launch_maps_dk<64, 1>(p, a, b, s) : launch_maps_dk<64, 0>(p, a, b, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_w(const Plan& p, const Args& a, const Buffers& b, int jt, hipStream_t s) {
  switch (p.D) {
    case 16: return launch_w_d<16>(p, a, b, jt, s);
    case 32: return launch_w_d<32>(p, a, b, jt, s);
    case 64: return launch_w_d<64>(p, a, b, jt, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_out(const Plan& p, const Args& a, const Buffers& b, hipStream_t s) {
  switch (p.D) {
    case 16: return launch_out_d<16>(p, a, b, s);
    case 32: return launch_out_d<32>(p, a, b, s);
    case 64: return launch_out_d<64>(p, a, b, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_export(const Plan& p, const Args& a, const Buffers& b, hipStream_t s) {
  if (!a.st_kql && !a.st_klk) return hipSuccess;
  const float* kql = a.shared_qk ? b.klkt : b.kqlt;
  const size_t total = static_cast<size_t>(p.BH) * p.m * p.N;
  const unsigned blocks = static_cast<unsigned>((total + WG - 1) / WG < 4096 ? (total + WG - 1) / WG : 4096);
  hipLaunchKernelGGL(export_kernel, dim3(blocks), dim3(WG), 0, s, kql, b.klkt, a.st_kql, a.st_klk,
                     p.N, p.m, total);
  return hipGetLastError();
}

}  // namespace lapattn
