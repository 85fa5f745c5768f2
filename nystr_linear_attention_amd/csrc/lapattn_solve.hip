// The landmark solve Y = A^{-1} W on its own (one workgroup per head), by the
// Newton-Schulz iteration of the forward pass or by conjugate gradient, for
// the comparison the LaplacianFormer summaries draw between the two
// (Arabic summary, section 4, efficiency analysis: Newton-Schulz more stable
// and better converging than conjugate-gradient solvers, above all on
// ill-conditioned matrices).
//
//   A = k(L, L) + eps I (the forward's A, built the same way)
//   Newton-Schulz: X_T by the forward's solver (fp16 MFMA on scaled two-part
//                  operands), then Y = X_T W in fp32
//   CG:            every column of W its own system A y = w, from y = 0,
//                  exactly T steps of Hestenes-Stiefel conjugate gradient:
//                  q = A p; a = r.r / p.q; y += a p; r -= a q;
//                  b = r'.r' / r.r; p = r + b p  (a column with r = 0 stops)
//                  A p on fp32 MFMA, the rest on FP32 VALU, all in LDS.

#include "lapattn_device.h"

namespace lapattn {
namespace {

constexpr int SS = 68;  // LDS row stride (floats) of 64-wide matrices

// Rows of A (64 x 64, stride SS) against rows of P^T (D x 64): the 16 x 16
// block (bi, bj) of A P; lane (g, r) reads k = 16 g .. 16 g + 15.
__device__ __forceinline__ f4 solve_rows_mm(const float* A, const float* BT, int bi, int bj) {
  const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const float* ap = A + (16 * bi + lr) * SS + 16 * lg;
  const float* bp = BT + (16 * bj + lr) * SS + 16 * lg;
  f4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const f4 av = ld4(ap + 4 * q), bv = ld4(bp + 4 * q);
#pragma unroll
    for (int h = 0; h < 4; ++h) c = mfma4(av[h], bv[h], c);
  }
  return c;
}

template <int D, int KIND>
__device__ void cg_role(const MainArgs& a, int bh, const float* W, float* Y, float* sm) {
  // LDS: A [64][SS], P^T [D][SS] (columns of P as rows), R^T, Y^T, Q^T, the
  // landmarks while A is built, and per-column scalars
  float* A = sm;
  float* PT = A + MP * SS;
  float* RT = PT + D * SS;
  float* YT = RT + D * SS;
  float* QT = YT + D * SS;
  float* Ls = QT + D * SS;            // landmarks (rows of D + 4), 64 rows
  float* rr = Ls + MP * (D + 4);      // [D] r.r
  float* pq = rr + D;                 // [D] p.q
  const int tid = threadIdx.x, w = wave_id(), lane = tid & 63;
  const int m = a.m;
  constexpr int LDL = D + 4;
  const int nb = (m + 1) / 2;
  {
    const float* Lg = a.L + static_cast<size_t>(bh) * m * D;
    for (int e = tid; e < 2 * nb * (D / 4); e += WGM) {
      const int row = e / (D / 4), c4 = e % (D / 4);
      st4(Ls + row * LDL + 4 * c4, row < m ? ld4(Lg + row * D + 4 * c4) : f4{0.f, 0.f, 0.f, 0.f});
    }
    for (int e = tid; e < MP * SS; e += WGM) A[e] = 0.f;
    // R = W (columns of W as rows of R^T), P = R, Y = 0; zero beyond m
    const float* wg = W + static_cast<size_t>(bh) * m * D;
    for (int e = tid; e < D * MP; e += WGM) {
      const int c = e / MP, i = e % MP;
      const float v = i < m ? wg[i * D + c] : 0.f;
      RT[c * SS + i] = v;
      PT[c * SS + i] = v;
      YT[c * SS + i] = 0.f;
    }
  }
  __syncthreads();
  build_a<D, KIND>(a, bh, Ls, A, SS);
  __syncthreads();
  // r.r per column: 8 threads per column, fixed order
  auto col_dot = [&](const float* X1, const float* X2, float* out) {
    if (tid < 8 * D) {
      const int c = tid >> 3, part = tid & 7;
      float s = 0.f;
      for (int i = part; i < MP; i += 8) s = fmaf(X1[c * SS + i], X2[c * SS + i], s);
      s += __shfl_xor(s, 1);
      s += __shfl_xor(s, 2);
      s += __shfl_xor(s, 4);
      if (part == 0) out[c] = s;
    }
  };
  col_dot(RT, RT, rr);
  __syncthreads();
  constexpr int NBLK = 4 * (D / 16);  // 16 x 16 blocks of Q = A P (64 x D)
  for (int t = 0; t < a.iters; ++t) {
    // Q = A P (rows >= m zero because A's are)
    for (int blk = w; blk < NBLK; blk += WGM / 64) {
      const int bi = blk / (D / 16), bj = blk % (D / 16);
      const f4 c = solve_rows_mm(A, PT, bi, bj);
      const int lr = lane & 15, lg = lane >> 4;
#pragma unroll
      for (int i = 0; i < 4; ++i) QT[(16 * bj + lr) * SS + 16 * bi + 4 * lg + i] = c[i];
    }
    __syncthreads();
    col_dot(PT, QT, pq);
    __syncthreads();
    // y += a p; r -= a q
    for (int e = tid; e < D * MP; e += WGM) {
      const int c = e / MP, i = e % MP;
      const float al = pq[c] != 0.f ? rr[c] / pq[c] : 0.f;
      YT[c * SS + i] = fmaf(al, PT[c * SS + i], YT[c * SS + i]);
      RT[c * SS + i] = fmaf(-al, QT[c * SS + i], RT[c * SS + i]);
    }
    __syncthreads();
    // b = r'.r' / r.r (into pq); p = r + b p; then r.r = r'.r'
    col_dot(RT, RT, pq);
    __syncthreads();
    for (int e = tid; e < D * MP; e += WGM) {
      const int c = e / MP, i = e % MP;
      const float be = rr[c] != 0.f ? pq[c] / rr[c] : 0.f;
      PT[c * SS + i] = fmaf(be, PT[c * SS + i], RT[c * SS + i]);
    }
    __syncthreads();
    if (tid < D) rr[tid] = pq[tid];
    __syncthreads();
  }
  float* yg = Y + static_cast<size_t>(bh) * m * D;
  for (int e = tid; e < m * D; e += WGM) {
    const int i = e / D, c = e % D;
    yg[e] = YT[c * SS + i];
  }
}

template <int D, int MB, int KIND>
__device__ void ns_solve_role(const MainArgs& a, int bh, const float* W, float* Y, float* smem) {
  using G = NsGeom<MB, D>;
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
  float alpha;
  int eA, e0;
  solver_setup<D, MB, KIND>(a, bh, smem, alpha, eA, e0);
  if (w < MB) {
    ns_wave<MB, D>(a, smem, w, lane, alpha, eA, e0);
  } else {
    __syncthreads();  // the steps' barriers: one after the set-up, one per step
    for (int t = 0; t < a.iters; ++t) __syncthreads();
  }
  __syncthreads();
  // the final iterate, fp32, row stride SX (zero in the padding); Y = X W
  const float* Xf = smem + G::OFF_X + 2 * G::XARR * (a.iters & 1);
  const int m = a.m;
  const float* wg = W + static_cast<size_t>(bh) * m * D;
  float* yg = Y + static_cast<size_t>(bh) * m * D;
  for (int e = tid; e < m * D; e += WGM) {
    const int i = e / D, c = e % D;
    float s = 0.f;
    for (int j = 0; j < m; ++j) s = fmaf(Xf[i * G::SX + j], wg[j * D + c], s);
    yg[e] = s;
  }
}

template <int D>
constexpr int cg_smem() {
  return MP * SS + 4 * D * SS + MP * (D + 4) + 2 * D;
}

template <int D, int MB, int KIND>
__global__ __launch_bounds__(WGM) void solve_kernel(MainArgs a, const float* __restrict__ W, float* Y,
                                                    int cg) {
  constexpr int NS = NsGeom<MB, D>::SMEM;
  constexpr int CG = cg_smem<D>();
  __shared__ __attribute__((aligned(16))) float smem[NS > CG ? NS : CG];
  if (cg) cg_role<D, KIND>(a, blockIdx.x, W, Y, smem);
  else ns_solve_role<D, MB, KIND>(a, blockIdx.x, W, Y, smem);
}

template <int D, int MB>
hipError_t launch_solve_dm(const MainArgs& ma, const float* W, float* Y, int cg, hipStream_t s) {
  if (ma.kind == 0)
    return launch(solve_kernel<D, MB, 0>, dim3(ma.BH), dim3(WGM), s, Ev{}, ma, W, Y, cg);
  return launch(solve_kernel<D, MB, 1>, dim3(ma.BH), dim3(WGM), s, Ev{}, ma, W, Y, cg);
}

template <int D>
hipError_t launch_solve_d(const MainArgs& ma, int mb, const float* W, float* Y, int cg, hipStream_t s) {
  switch (mb) {
    case 1: return launch_solve_dm<D, 1>(ma, W, Y, cg, s);
    case 2: return launch_solve_dm<D, 2>(ma, W, Y, cg, s);
    case 3: return launch_solve_dm<D, 3>(ma, W, Y, cg, s);
    case 4: return launch_solve_dm<D, 4>(ma, W, Y, cg, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_landmark_solve(const Plan& p, const float* L, const float* W, float lambda, float eps,
                                 int iters, int cg, float* Y, hipStream_t s) {
  MainArgs ma{};
  ma.L = L;
  ma.m = p.m;
  ma.BH = p.BH;
  ma.kind = p.kernel;
  ma.iters = iters;
  ma.c_exp2 = static_cast<float>(-1.4426950408889634 / static_cast<double>(lambda));
  ma.eps = eps;
  switch (p.D) {
    case 16: return launch_solve_d<16>(ma, p.ns_mb, W, Y, cg, s);
    case 32: return launch_solve_d<32>(ma, p.ns_mb, W, Y, cg, s);
    case 64: return launch_solve_d<64>(ma, p.ns_mb, W, Y, cg, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace lapattn
