// HIP kernels for the backward pass of Nystrom kernel attention on gfx950.
//
// The LaplacianFormer summaries say the method's custom kernels serve the
// backward pass as well as the forward pass (Dutch summary, "Methodologie"
// item 3; Arabic summary, section 2(c) item 3) but print no formulas for it,
// so the backward pass here is the exact reverse-mode derivative of the
// forward (see lapattn_kernels.hip), per head:
//
//   forward      L = pool(K); K_QL = k(Q, L); K_LK = k(L, K); A = k(L, L) + eps I
//                X_0 = alpha A, X_{t+1} = 2 X_t - X_t A X_t (T steps), X = X_T
//                W = K_LK V; Y = X W; O = K_QL Y
//   given dO     dK_QL = dO Y^T          dY = K_QL^T dO
//                dX = dY W^T             dW = X^T dY
//                dK_LK = dW V^T          dV = K_LK^T dW
//                Newton-Schulz, from G = dX, t = T-1 .. 0:
//                  dA -= X_t^T G X_t^T;  G <- 2 G - G (A X_t)^T - (X_t A)^T G
//                then dA += alpha G and alpha's own derivative through the
//                first column of largest abs-sum (A is exactly symmetric, so
//                it is also the first row of largest abs-sum)
//                k(x, y) = exp(-D(x, y) / lambda):
//                  dD = -dk k / lambda; D = ||x - y||_1: dx = dD sign(x - y),
//                  dy = -dx (sign(0) = 0); D = ||x - y||^2: dx = 2 dD (x - y)
//                dL from A (both arguments), K_QL and K_LK; dQ from K_QL;
//                dK = (direct part from K_LK) + dL of its window / (ph pw)
//
// Launches, back to back on the caller's stream:
//   pool  (shared with the forward)        K -> L
//   part  solver WGs: A, alpha, Newton-Schulz (the forward's solver, every
//         iterate X_0 .. X_T stored in fp32);  key tiles: W^T partials
//         (K_LK V, the forward's key path);  query tiles: dY^T partials
//         (K_QL dO, the same path with Q for K and dO for V)
//   head  one workgroup per head: W, dY; Y = X W; dX, dW; the Newton-Schulz
//         backward on fp32 MFMA in LDS; dA; dL from A
//   grad  one workgroup per 64-token tile of Q or K: the kernel map again,
//         dK_QL = dO Y^T (or dK_LK^T = V dW^T) on fp32 MFMA, the gradient
//         map on FP32 VALU (dQ or the direct dK rows, and the tile's dL
//         partial), and for key tiles dV = K_LK^T dW
//   dk    one workgroup per landmark window: dL = its partials in fixed order,
//         dK rows of the window = direct part + dL / (ph pw)
// Every reduction runs in a fixed order, so results do not depend on timing.

#include "lapattn_device.h"

namespace lapattn {
namespace {

constexpr int BS = 68;  // LDS row stride (floats) of 64-wide matrices

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  const float* L;      // [BH][m][D]
  const float* xiter;  // [BH][T + 1][MP][MP]  X_0 .. X_T (rows, columns < 16 ceil(m/16))
  const float* amat;   // [BH][MP][MP]         A, zero beyond m
  const float* hscal;  // [BH][4]              alpha, first column of largest abs-sum, that sum
  const float* wpart;  // [BH][nP][D][MP]      W^T partials (columns < 16 ceil(m/16))
  const float* dypart; // [BH][nP][D][MP]      dY^T partials
  float* ymat;         // [BH][MP][D]          Y = X W (rows >= m zero)
  float* dwmat;        // [BH][MP][D]          dW = X^T dY (rows >= m zero)
  float* dla;          // [BH][MP][D]          dL from A (rows >= m zero)
  float* dlpart;       // [BH][2 nT][MP][D]    dL partials of the gradient tiles
  float* dkd;          // [BH][N][D]           direct part of dK
  int N, m, BH, nT, nP, gw, ph, pw, iters, kind, bf16;
  float lambda, eps, c_exp2;
};

// ---------------------------------------------------------------------------
// part: solver workgroups (one per head) and map tiles.
// ---------------------------------------------------------------------------
template <int D, int MB, int KIND>
__device__ __forceinline__ void bwd_solver(const MainArgs& a, int bh, float* smem, float* xiter_all,
                                           float* amat, float* hscal) {
  using G = NsGeom<MB, D>;
  constexpr int SX = G::SX;
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
  const int m = a.m;
  float* xi = xiter_all + static_cast<size_t>(bh) * (a.iters + 1) * MP * MP;
  float alpha;
  int eA, e0;
  solver_setup<D, MB, KIND>(a, bh, smem, alpha, eA, e0, xi);
  // A in fp32 is still in LDS until the first step's barrier: store it, and
  // alpha with the first column of largest abs-sum (A is exactly symmetric:
  // row sums are the column sums, summed in the order the set-up uses)
  const float* Af = smem + G::OFF_X + 2 * G::XARR;
  float* ag = amat + static_cast<size_t>(bh) * MP * MP;
  for (int e = tid; e < MP * MP; e += WGM) {
    const int r = e / MP, c = e % MP;
    ag[e] = (r < m && c < m) ? Af[r * SX + c] : 0.f;
  }
  if (w == 0) {
    float sum = 0.f;
    if (lane < m) {
      for (int q = 0; q < (m + 3) / 4; ++q) {
        const f4 v = ld4(Af + lane * SX + 4 * q);  // zero beyond m
        sum += fabsf(v[0]) + fabsf(v[1]) + fabsf(v[2]) + fabsf(v[3]);
      }
    }
    const float mx = __uint_as_float(wave_max_u(__float_as_uint(sum)));
    const unsigned long long hit = __ballot(lane < m && sum == mx);
    const int jc = static_cast<int>(__builtin_ctzll(hit));
    if (lane == 0) {
      float* hs = hscal + 4 * static_cast<size_t>(bh);
      hs[0] = alpha;
      hs[1] = __int_as_float(jc);
      hs[2] = mx;
      hs[3] = 0.f;
    }
  }
  if (w < MB) {
    ns_wave<MB, D, true>(a, smem, w, lane, alpha, eA, e0, xi);
  } else {
    __syncthreads();  // the steps' barriers: one after the set-up, one per step
    for (int t = 0; t < a.iters; ++t) __syncthreads();
  }
}

template <int D, int MB, int KIND, bool BF16>
__global__ __launch_bounds__(WGM, 4) void bwd_part_kernel(MainArgs a, const void* __restrict__ q,
                                                        const void* __restrict__ k,
                                                        const void* __restrict__ v,
                                                        const void* __restrict__ dout,
                                                        const float* __restrict__ L, float* dypart,
                                                        float* xiter, float* amat, float* hscal) {
  constexpr int MAP_SMEM = map_pj_size<D>() + 2 * MP * LS + TILE;
  constexpr int SOLVER_SMEM = NsGeom<MB, D>::SMEM;
  __shared__ __attribute__((aligned(16)))
  float smem[MAP_SMEM > SOLVER_SMEM ? MAP_SMEM : SOLVER_SMEM];
  int b = blockIdx.x;
  if (b < a.BH) {
    bwd_solver<D, MB, KIND>(a, b, smem, xiter, amat, hscal);
    return;
  }
  b -= a.BH;
  if (b < a.BH * a.nP) {
    // K_LK V: the forward's key path
    map_role<D, KIND, BF16>(a, q, k, v, L, b / a.nP, true, b % a.nP, smem);
  } else {
    // K_QL^T dO: the same path with the queries for the keys and dO for V
    b -= a.BH * a.nP;
    MainArgs a2 = a;
    a2.wpart = dypart;
    map_role<D, KIND, BF16>(a2, q, q, dout, L, b / a.nP, true, b % a.nP, smem);
  }
}

// ---------------------------------------------------------------------------
// head: one workgroup (8 waves) per head, small matrices in LDS on fp32 MFMA.
// ---------------------------------------------------------------------------
// C[16 bi + .., 16 bj + ..] (this wave's blocks blk = w, w + 8, ..., nblk
// blocks of 16 x 16, 4 column blocks per block row) = sum over k < 64 of
// A(i, k) B(k, j) with A(i, k) = pa[i ar + k ac] and B(k, j) = pb[k br + j bc]
// in LDS.  16 MFMAs per block (lane group g takes k = 16 g + s at sub-step s).
// The accumulator of block s holds C[16 bi + 4 g + i][16 bj + r].
template <int NBLK>
__device__ __forceinline__ void lds_mm(const float* pa, int ar, int ac, const float* pb, int br, int bc,
                                       int ncb, f4 (&acc)[(NBLK + 7) / 8]) {
  const int lane = threadIdx.x & 63, w = wave_id();
  const int lr = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int s = 0; s < (NBLK + 7) / 8; ++s) {
    acc[s] = f4{0.f, 0.f, 0.f, 0.f};
    const int blk = w + 8 * s;
    if (blk < NBLK) {
      const int bi = blk / ncb, bj = blk % ncb;
      const float* ap = pa + (16 * bi + lr) * ar + 16 * lg * ac;
      const float* bp = pb + 16 * lg * br + (16 * bj + lr) * bc;
      f4 c = acc[s];
#pragma unroll
      for (int kk = 0; kk < 16; ++kk) c = mfma4(ap[kk * ac], bp[kk * br], c);
      acc[s] = c;
    }
  }
}

// Block accumulators to LDS (row stride BS): dst[i][j] = scale * acc (+ beta * dst).
template <int NBLK>
__device__ __forceinline__ void lds_store(float* dst, int ncb, const f4 (&acc)[(NBLK + 7) / 8],
                                          float scale, float beta) {
  const int lane = threadIdx.x & 63, w = wave_id();
  const int lr = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int s = 0; s < (NBLK + 7) / 8; ++s) {
    const int blk = w + 8 * s;
    if (blk < NBLK) {
      const int bi = blk / ncb, bj = blk % ncb;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float* p = dst + (16 * bi + 4 * lg + i) * BS + 16 * bj + lr;
        *p = beta == 0.f ? scale * acc[s][i] : fmaf(beta, *p, scale * acc[s][i]);
      }
    }
  }
}

// Loads an MP x MP fp32 matrix from global memory into LDS (row stride BS),
// zero outside rows, columns < m.
__device__ __forceinline__ void load_mm(float* dst, const float* src, int m) {
  for (int e = threadIdx.x; e < MP * MP; e += WGM) {
    const int r = e / MP, c = e % MP;
    dst[r * BS + c] = (r < m && c < m) ? src[e] : 0.f;
  }
}

template <int D, int KIND>
__global__ __launch_bounds__(WGM) void bwd_head_kernel(BwdArgs a) {
  constexpr int NB64 = 16;           // 16 x 16 blocks of a 64 x 64 product
  constexpr int NBD = 4 * (D / 16);  // blocks of a 64 x D product
  __shared__ __attribute__((aligned(16))) float sm[6 * MP * BS + 8];
  float* M0 = sm;
  float* M1 = sm + MP * BS;
  float* M2 = sm + 2 * MP * BS;
  float* M3 = sm + 3 * MP * BS;
  float* M4 = sm + 4 * MP * BS;
  float* M5 = sm + 5 * MP * BS;
  float* red = sm + 6 * MP * BS;
  const int bh = blockIdx.x, tid = threadIdx.x;
  const int m = a.m, nP = a.nP, T = a.iters;
  const size_t ps = static_cast<size_t>(D) * MP;

  // W[j][c] and dY[j][c] (row stride BS), the partials summed in order
  {
    const float* wp = a.wpart + static_cast<size_t>(bh) * nP * ps;
    const float* dp = a.dypart + static_cast<size_t>(bh) * nP * ps;
    for (int e = tid; e < MP * MP; e += WGM) {
      const int j = e / MP, c = e % MP;
      float sw = 0.f, sd = 0.f;
      if (j < m && c < D) {
        for (int p = 0; p < nP; ++p) {
          sw += wp[p * ps + c * MP + j];
          sd += dp[p * ps + c * MP + j];
        }
      }
      M0[j * BS + c] = sw;
      M1[j * BS + c] = sd;
    }
  }
  load_mm(M2, a.xiter + (static_cast<size_t>(bh) * (T + 1) + T) * MP * MP, m);  // X = X_T
  __syncthreads();
  {
    // Y = X W; dW = X^T dY  (m x D) to global memory
    f4 acc[(NBD + 7) / 8];
    lds_mm<NBD>(M2, BS, 1, M0, BS, 1, D / 16, acc);
    const int lane = tid & 63, w = wave_id(), lr = lane & 15, lg = lane >> 4;
#pragma unroll
    for (int s = 0; s < (NBD + 7) / 8; ++s) {
      const int blk = w + 8 * s;
      if (blk < NBD) {
        const int bi = blk / (D / 16), bj = blk % (D / 16);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          a.ymat[(static_cast<size_t>(bh) * MP + 16 * bi + 4 * lg + i) * D + 16 * bj + lr] = acc[s][i];
      }
    }
    lds_mm<NBD>(M2, 1, BS, M1, BS, 1, D / 16, acc);
#pragma unroll
    for (int s = 0; s < (NBD + 7) / 8; ++s) {
      const int blk = w + 8 * s;
      if (blk < NBD) {
        const int bi = blk / (D / 16), bj = blk % (D / 16);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          a.dwmat[(static_cast<size_t>(bh) * MP + 16 * bi + 4 * lg + i) * D + 16 * bj + lr] = acc[s][i];
      }
    }
    // G = dX = dY W^T  (m x m): rows of dY against rows of W
    f4 g[2];
    lds_mm<NB64>(M1, BS, 1, M0, 1, BS, 4, g);
    lds_store<NB64>(M3, 4, g, 1.f, 0.f);
  }
  load_mm(M4, a.amat + static_cast<size_t>(bh) * MP * MP, m);  // A
  for (int e = tid; e < MP * BS; e += WGM) M5[e] = 0.f;       // dA
  __syncthreads();

  // Newton-Schulz backward, t = T-1 .. 0.  X_t commutes with A and is
  // symmetric in exact arithmetic, so (X_t A)^T is taken as A X_t (the
  // difference is rounding of X_t, and the recursion is linear in G).
  for (int t = T - 1; t >= 0; --t) {
    load_mm(M2, a.xiter + (static_cast<size_t>(bh) * (T + 1) + t) * MP * MP, m);  // X_t
    __syncthreads();
    f4 acc[2];
    lds_mm<NB64>(M4, BS, 1, M2, BS, 1, 4, acc);  // Q1 = A X_t
    lds_store<NB64>(M0, 4, acc, 1.f, 0.f);
    lds_mm<NB64>(M2, 1, BS, M3, BS, 1, 4, acc);  // P1 = X_t^T G
    lds_store<NB64>(M1, 4, acc, 1.f, 0.f);
    __syncthreads();
    lds_mm<NB64>(M1, BS, 1, M2, 1, BS, 4, acc);  // P1 X_t^T
    lds_store<NB64>(M5, 4, acc, -1.f, 1.f);      // dA -= P1 X_t^T
    f4 gq[2], qg[2];
    lds_mm<NB64>(M3, BS, 1, M0, 1, BS, 4, gq);   // G Q1^T
    lds_mm<NB64>(M0, BS, 1, M3, BS, 1, 4, qg);   // Q1 G
    __syncthreads();                             // every read of G is done
    {
      const int lane = tid & 63, w = wave_id(), lr = lane & 15, lg = lane >> 4;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int blk = w + 8 * s, bi = blk / 4, bj = blk % 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float* p = M3 + (16 * bi + 4 * lg + i) * BS + 16 * bj + lr;
          *p = 2.f * *p - gq[s][i] - qg[s][i];
        }
      }
    }
    __syncthreads();
  }
  // dA += alpha G; d alpha = <G, A> flows through alpha = 1 / (c r), c = r =
  // the largest column (row) abs-sum: dA[:, jc] and dA[jc, :] each gain
  // -d alpha alpha / c sign(A)
  const float* hs = a.hscal + 4 * static_cast<size_t>(bh);
  const float alpha = hs[0], csum = hs[2];
  const int jc = __float_as_int(hs[1]);
  {
    float part = 0.f;
    for (int e = tid; e < MP * MP; e += WGM) {
      const int r = e / MP, c = e % MP;
      part = fmaf(M3[r * BS + c], M4[r * BS + c], part);
    }
    // fixed-order sum: per wave, then over waves
    for (int o = 32; o > 0; o >>= 1) part += __shfl_xor(part, o);
    if ((tid & 63) == 0) red[wave_id()] = part;
    __syncthreads();
    float dalpha = 0.f;
    for (int i = 0; i < WGM / 64; ++i) dalpha += red[i];
    const float dc = -dalpha * alpha / csum;
    for (int e = tid; e < MP * MP; e += WGM) {
      const int r = e / MP, c = e % MP;
      float v = fmaf(alpha, M3[r * BS + c], M5[r * BS + c]);
      if (r < m && c < m) {
        const float av = M4[r * BS + c];
        const float sg = av > 0.f ? 1.f : (av < 0.f ? -1.f : 0.f);
        if (c == jc) v = fmaf(dc, sg, v);
        if (r == jc) v = fmaf(dc, sg, v);
      }
      M5[r * BS + c] = v;
    }
  }
  __syncthreads();
  // dL from A = k(L, L) + eps I: dd = -dA k(L, L) / lambda, and for landmark
  // p: sum_j (dd[p][j] + dd[j][p]) s(l_p - l_j), s = sign (Laplacian) or 2 x
  // (Gaussian).  Landmarks in M0 (rows of D floats, stride BS).
  {
    const float* Lg = a.L + static_cast<size_t>(bh) * m * D;
    for (int e = tid; e < MP * D; e += WGM) {
      const int r = e / D, c = e % D;
      M0[r * BS + c] = r < m ? Lg[r * D + c] : 0.f;
    }
    const float il = 1.0f / a.lambda;
    for (int e = tid; e < MP * MP; e += WGM) {
      const int r = e / MP, c = e % MP;
      const float kv = (r < m && c < m) ? M4[r * BS + c] - (r == c ? a.eps : 0.f) : 0.f;
      M1[r * BS + c] = -M5[r * BS + c] * kv * il;
    }
    __syncthreads();
    for (int e = tid; e < MP * D; e += WGM) {
      const int p = e / D, c = e % D;
      float acc = 0.f;
      if (p < m) {
        const float lp = M0[p * BS + c];
        for (int j = 0; j < m; ++j) {
          const float x = lp - M0[j * BS + c];
          float s;
          if constexpr (KIND == 0) s = x > 0.f ? 1.f : (x < 0.f ? -1.f : 0.f);
          else s = 2.f * x;
          acc = fmaf(M1[p * BS + j] + M1[j * BS + p], s, acc);
        }
      }
      a.dla[(static_cast<size_t>(bh) * MP + p) * D + c] = acc;
    }
  }
}

// ---------------------------------------------------------------------------
// grad: one workgroup (4 waves) per 64-token tile of Q (side 0) or K (side 1).
// ---------------------------------------------------------------------------
constexpr int WGG = 256;

// sign(x) with sign(0) = 0 (Laplacian) or 2 x (Gaussian): the derivative of
// the coordinate's distance term.  For the sign, x is scaled by 2^252 in two
// exact steps (every nonzero fp32 difference then has magnitude >= 1, and
// large ones become infinite) and clamped to [-1, 1].
template <int KIND>
__device__ __forceinline__ float dterm(float x) {
  if constexpr (KIND == 0)
    return __builtin_amdgcn_fmed3f((x * 0x1p126f) * 0x1p126f, -1.0f, 1.0f);
  else
    return x + x;
}

template <int D, int KIND, bool BF16>
__global__ __launch_bounds__(WGG) void bwd_grad_kernel(BwdArgs a) {
  constexpr int XS = D + 4;     // row stride of token / landmark rows
  constexpr int R = 64 / D;     // tokens per wave row (lane = r D + k)
  constexpr int TPW = TILE / 4; // tokens per wave
  constexpr int NBLK = 16;      // 64 x 64 product blocks
  // LDS: token rows XT, landmarks LM, w transposed WT[j][token]; the kernel
  // values P, the second operand VO and the small matrix YB share the area of
  // the wave partials of dL, PL (used after them)
  constexpr int OFF_XT = 0;
  constexpr int OFF_LM = OFF_XT + TILE * XS;
  constexpr int OFF_WT = OFF_LM + MP * XS;
  constexpr int OFF_U = OFF_WT + MP * BS;
  constexpr int OFF_P = OFF_U;
  constexpr int OFF_VO = OFF_P + TILE * BS;
  constexpr int OFF_YB = OFF_VO + TILE * XS;
  constexpr int U1 = TILE * BS + TILE * XS + MP * XS;
  constexpr int U2 = 4 * R * MP * D;
  constexpr int SMEM = OFF_U + (U1 > U2 ? U1 : U2);
  __shared__ __attribute__((aligned(16))) float sm[SMEM];
  float* XT = sm + OFF_XT;
  float* LM = sm + OFF_LM;
  float* WT = sm + OFF_WT;
  float* P = sm + OFF_P;
  float* VO = sm + OFF_VO;
  float* YB = sm + OFF_YB;
  float* PL = sm + OFF_U;

  const int nT = a.nT, N = a.N, m = a.m;
  const int bh = blockIdx.x / (2 * nT);
  const int side = (blockIdx.x / nT) & 1;  // 0: query tile, 1: key tile
  const int t = blockIdx.x % nT;
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
  const void* xsrc = side ? a.k : a.q;
  const void* osrc = side ? a.v : a.dout;
  const float* ysrc = (side ? a.dwmat : a.ymat) + static_cast<size_t>(bh) * MP * D;
  const float* Lg = a.L + static_cast<size_t>(bh) * m * D;

  // token rows of x and of dO (query tile) or V (key tile); landmarks; Y
  // (query tile) or dW (key tile); rows past N or m are zero
  for (int e = tid; e < TILE * (D / 4); e += WGG) {
    const int r = e / (D / 4), c4 = e % (D / 4);
    const int n = t * TILE + r;
    const size_t gi = (static_cast<size_t>(bh) * N + n) * D + 4 * c4;
    const f4 z = {0.f, 0.f, 0.f, 0.f};
    st4(XT + r * XS + 4 * c4, n < N ? load4_io(xsrc, gi, BF16) : z);
    st4(VO + r * XS + 4 * c4, n < N ? load4_io(osrc, gi, BF16) : z);
  }
  for (int e = tid; e < MP * (D / 4); e += WGG) {
    const int r = e / (D / 4), c4 = e % (D / 4);
    const f4 z = {0.f, 0.f, 0.f, 0.f};
    st4(LM + r * XS + 4 * c4, r < m ? ld4(Lg + r * D + 4 * c4) : z);
    st4(YB + r * XS + 4 * c4, ld4(ysrc + r * D + 4 * c4));  // zero rows beyond m
  }
  __syncthreads();
  // kernel values P[token][j] = k(x_token, l_j) (zero for j >= m or token
  // past N): thread (token, landmark group), the token row in registers
  {
    const int tok = tid & 63, jg = tid >> 6;
    float xr[D];
#pragma unroll
    for (int c = 0; c < D; ++c) xr[c] = XT[tok * XS + c];
    const bool valid = t * TILE + tok < N;
    for (int j = jg; j < MP; j += 4) {
      float kv = 0.f;
      if (j < m && valid) {
        float d0 = 0.f, d1 = 0.f;
#pragma unroll
        for (int c = 0; c < D; c += 4) {
          const f4 l = ld4(LM + j * XS + c);
#pragma unroll
          for (int u = 0; u < 4; u += 2) {
            const float s0 = xr[c + u] - l[u], s1 = xr[c + u + 1] - l[u + 1];
            if constexpr (KIND == 0) {
              d0 += fabsf(s0);
              d1 += fabsf(s1);
            } else {
              d0 = fmaf(s0, s0, d0);
              d1 = fmaf(s1, s1, d1);
            }
          }
        }
        kv = exp2_map((d0 + d1) * a.c_exp2);
      }
      P[tok * BS + j] = kv;
    }
  }
  __syncthreads();
  // dK_map[token][j] = sum_c VO[token][c] YB[j][c]  (query tile: dK_QL = dO Y^T;
  // key tile: dK_LK^T = V dW^T); w = -dK_map P / lambda, stored transposed
  {
    const int lr = lane & 15, lg = lane >> 4;
    constexpr int KS = D / 4;
    const float il = -1.0f / a.lambda;
#pragma unroll
    for (int s = 0; s < NBLK / 4; ++s) {
      const int blk = w + 4 * s, bi = blk / 4, bj = blk % 4;
      const float* ap = VO + (16 * bi + lr) * XS + KS * lg;
      const float* bp = YB + (16 * bj + lr) * XS + KS * lg;
      f4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) c = mfma4(ap[kk], bp[kk], c);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = 16 * bi + 4 * lg + i, j = 16 * bj + lr;
        WT[j * BS + tok] = c[i] * P[tok * BS + j] * il;
      }
    }
  }
  if (side) {
    // dV[token][c] = sum_j P[token][j] dW[j][c]  (dW rows beyond m are zero)
    const int lr = lane & 15, lg = lane >> 4;
    constexpr int NBV = 4 * (D / 16);
    for (int blk = w; blk < NBV; blk += 4) {
      const int bi = blk / (D / 16), bj = blk % (D / 16);
      const float* ap = P + (16 * bi + lr) * BS + 16 * lg;
      const float* bp = YB + (16 * lg) * XS + 16 * bj + lr;
      f4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 16; ++kk) c = mfma4(ap[kk], bp[kk * XS], c);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = t * TILE + 16 * bi + 4 * lg + i;
        if (n < N) {
          const size_t o = (static_cast<size_t>(bh) * N + n) * D + 16 * bj + lr;
          if (BF16) static_cast<uint16_t*>(a.dv)[o] = f32_to_bf16_rne(c[i]);
          else static_cast<float*>(a.dv)[o] = c[i];
        }
      }
    }
  }
  __syncthreads();  // WT complete; P, VO and YB are dead (PL reuses them)
  // Gradient map: lane (r, k) of wave w takes coordinate k of tokens
  // 16 w + R it + r.  dx[token][k] = sum_j w[token][j] s(x - l_j)[k];
  // dL partial[j][k] = -sum_token w[token][j] s(x - l_j)[k].
  {
    const int r = lane / D, k = lane % D;
    float xr[TPW / R], dx[TPW / R];
#pragma unroll
    for (int it = 0; it < TPW / R; ++it) {
      xr[it] = XT[(TPW * w + R * it + r) * XS + k];
      dx[it] = 0.f;
    }
    float* pl = PL + (w * R + r) * MP * D;
    for (int j = 0; j < m; ++j) {
      const float l = LM[j * XS + k];
      const float* wr = WT + j * BS + TPW * w + r;
      float al = 0.f;
#pragma unroll
      for (int it = 0; it < TPW / R; ++it) {
        const float wv = wr[R * it];
        const float sv = dterm<KIND>(xr[it] - l);
        dx[it] = fmaf(wv, sv, dx[it]);
        al = fmaf(wv, sv, al);
      }
      pl[j * D + k] = -al;
    }
    // rows of dx: dQ (query tile, output type) or the direct part of dK
#pragma unroll
    for (int it = 0; it < TPW / R; ++it) {
      const int n = t * TILE + TPW * w + R * it + r;
      if (n < N) {
        const size_t o = (static_cast<size_t>(bh) * N + n) * D + k;
        if (side) a.dkd[o] = dx[it];
        else if (BF16) static_cast<uint16_t*>(a.dq)[o] = f32_to_bf16_rne(dx[it]);
        else static_cast<float*>(a.dq)[o] = dx[it];
      }
    }
  }
  __syncthreads();
  // the tile's dL partial: the 4 R wave rows summed in order
  {
    float* dst = a.dlpart + ((static_cast<size_t>(bh) * 2 + side) * nT + t) * MP * D;
    for (int e = tid; e < MP * D; e += WGG) {
      float s = 0.f;
      if (e < m * D) {
#pragma unroll
        for (int u = 0; u < 4 * R; ++u) s += PL[u * MP * D + e];
      }
      dst[e] = s;
    }
  }
}

// ---------------------------------------------------------------------------
// dk: one workgroup per (landmark window j, head): dL[j] = dL_A[j] + its
// 2 nT tile partials (query tiles, then key tiles, in order); the window's
// dK rows = direct part + dL[j] / (ph pw).
// ---------------------------------------------------------------------------
template <int D, bool BF16>
__global__ __launch_bounds__(WGG) void bwd_dk_kernel(BwdArgs a) {
  constexpr int G = WGG / D;
  __shared__ float part[WGG];
  __shared__ float dl[D];
  const int j = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int c = tid % D, g = tid / D;
  const int np = 2 * a.nT;
  const float* pb = a.dlpart + static_cast<size_t>(bh) * np * MP * D + j * D + c;
  float s = 0.f;
  for (int p = g; p < np; p += G) s += pb[static_cast<size_t>(p) * MP * D];
  part[tid] = s;
  __syncthreads();
  if (tid < D) {
    float acc = a.dla[(static_cast<size_t>(bh) * MP + j) * D + tid];
    for (int u = 0; u < G; ++u) acc += part[u * D + tid];
    dl[tid] = acc / static_cast<float>(a.ph * a.pw);
  }
  __syncthreads();
  const int mw = a.gw / a.pw, R0 = j / mw, C0 = j % mw;
  const int cnt = a.ph * a.pw;
  for (int e = tid; e < cnt * D; e += WGG) {
    const int tk = e / D, cc = e % D;
    const int n = (R0 * a.ph + tk / a.pw) * a.gw + C0 * a.pw + tk % a.pw;
    const size_t o = (static_cast<size_t>(bh) * a.N + n) * D + cc;
    const float v = a.dkd[o] + dl[cc];
    if (BF16) static_cast<uint16_t*>(a.dk)[o] = f32_to_bf16_rne(v);
    else static_cast<float*>(a.dk)[o] = v;
  }
}

template <int D, int MB>
hipError_t launch_part_dm(const MainArgs& ma, const void* dout, float* dypart, float* xiter, float* amat,
                          float* hscal, unsigned grid, hipStream_t s) {
  const Ev ev{};
  if (ma.kind == 0) {
    if (ma.bf16)
      return launch(bwd_part_kernel<D, MB, 0, true>, dim3(grid), dim3(WGM), s, ev, ma, ma.q, ma.k, ma.v,
                    dout, ma.L, dypart, xiter, amat, hscal);
    return launch(bwd_part_kernel<D, MB, 0, false>, dim3(grid), dim3(WGM), s, ev, ma, ma.q, ma.k, ma.v,
                  dout, ma.L, dypart, xiter, amat, hscal);
  }
  if (ma.bf16)
    return launch(bwd_part_kernel<D, MB, 1, true>, dim3(grid), dim3(WGM), s, ev, ma, ma.q, ma.k, ma.v,
                  dout, ma.L, dypart, xiter, amat, hscal);
  return launch(bwd_part_kernel<D, MB, 1, false>, dim3(grid), dim3(WGM), s, ev, ma, ma.q, ma.k, ma.v,
                dout, ma.L, dypart, xiter, amat, hscal);
}

template <int D>
hipError_t launch_bwd_d(const BwdPlan& p, const BwdArgs& ba, const MainArgs& ma, float* dypart,
                        float* xiter, float* amat, float* hscal, hipStream_t s) {
  const unsigned gpart = static_cast<unsigned>(p.BH + 2 * p.BH * p.nP);
  hipError_t e = hipErrorInvalidValue;
  switch (p.ns_mb) {
    case 1: e = launch_part_dm<D, 1>(ma, ba.dout, dypart, xiter, amat, hscal, gpart, s); break;
    case 2: e = launch_part_dm<D, 2>(ma, ba.dout, dypart, xiter, amat, hscal, gpart, s); break;
    case 3: e = launch_part_dm<D, 3>(ma, ba.dout, dypart, xiter, amat, hscal, gpart, s); break;
    case 4: e = launch_part_dm<D, 4>(ma, ba.dout, dypart, xiter, amat, hscal, gpart, s); break;
  }
  if (e != hipSuccess) return e;
  const Ev ev{};
  e = p.kernel == 0 ? launch(bwd_head_kernel<D, 0>, dim3(p.BH), dim3(WGM), s, ev, ba)
                    : launch(bwd_head_kernel<D, 1>, dim3(p.BH), dim3(WGM), s, ev, ba);
  if (e != hipSuccess) return e;
  const dim3 gg(static_cast<unsigned>(p.BH * 2 * p.nT));
  if (p.kernel == 0)
    e = p.bf16 ? launch(bwd_grad_kernel<D, 0, true>, gg, dim3(WGG), s, ev, ba)
               : launch(bwd_grad_kernel<D, 0, false>, gg, dim3(WGG), s, ev, ba);
  else
    e = p.bf16 ? launch(bwd_grad_kernel<D, 1, true>, gg, dim3(WGG), s, ev, ba)
               : launch(bwd_grad_kernel<D, 1, false>, gg, dim3(WGG), s, ev, ba);
  if (e != hipSuccess) return e;
  const dim3 gk(static_cast<unsigned>(p.m), static_cast<unsigned>(p.BH));
  return p.bf16 ? launch(bwd_dk_kernel<D, true>, gk, dim3(WGG), s, ev, ba)
                : launch(bwd_dk_kernel<D, false>, gk, dim3(WGG), s, ev, ba);
}

}  // namespace

hipError_t launch_backward(const BwdPlan& p, const BwdCall& c, hipStream_t s) {
  // Buffers of the workspace
  char* ws = static_cast<char*>(c.workspace);
  float* L = reinterpret_cast<float*>(ws + p.off_L);
  float* xiter = reinterpret_cast<float*>(ws + p.off_xiter);
  float* amat = reinterpret_cast<float*>(ws + p.off_amat);
  float* hscal = reinterpret_cast<float*>(ws + p.off_hscal);
  float* wpart = reinterpret_cast<float*>(ws + p.off_wpart);
  float* dypart = reinterpret_cast<float*>(ws + p.off_dypart);
  unsigned* sync = reinterpret_cast<unsigned*>(ws + p.off_sync);

  // pool: the forward's landmark launch
  {
    Plan fp{};
    fp.B = p.B;
    fp.H = p.H;
    fp.gh = p.gh;
    fp.gw = p.gw;
    fp.D = p.D;
    fp.ph = p.ph;
    fp.pw = p.pw;
    fp.kernel = p.kernel;
    fp.bf16 = p.bf16;
    fp.N = p.N;
    fp.m = p.m;
    fp.BH = p.BH;
    Args fa{};
    fa.k = c.k;
    Buffers fb{};
    fb.L = L;
    fb.sync = sync;
    fb.timeouts = sync;
    const hipError_t e = launch_pool(fp, fa, fb, s, Ev{});
    if (e != hipSuccess) return e;
  }
  MainArgs ma{};
  ma.q = c.q;
  ma.k = c.k;
  ma.v = c.v;
  ma.L = L;
  ma.wpart = wpart;
  ma.sync = sync;
  ma.timeouts = sync;
  ma.N = p.N;
  ma.m = p.m;
  ma.BH = p.BH;
  ma.nT = p.nT;
  ma.S = p.S;
  ma.nP = p.nP;
  ma.mpad = 16 * ((p.m + 15) / 16);
  ma.ns_blocks = p.BH;
  ma.kind = p.kernel;
  ma.bf16 = p.bf16;
  ma.iters = c.iters;
  ma.c_exp2 = static_cast<float>(-1.4426950408889634 / static_cast<double>(c.lambda));
  ma.eps = c.eps;
  ma.partials_only = 1;

  BwdArgs ba{};
  ba.q = c.q;
  ba.k = c.k;
  ba.v = c.v;
  ba.dout = c.dout;
  ba.dq = c.dq;
  ba.dk = c.dk;
  ba.dv = c.dv;
  ba.L = L;
  ba.xiter = xiter;
  ba.amat = amat;
  ba.hscal = hscal;
  ba.wpart = wpart;
  ba.dypart = dypart;
  ba.ymat = reinterpret_cast<float*>(ws + p.off_ymat);
  ba.dwmat = reinterpret_cast<float*>(ws + p.off_dwmat);
  ba.dla = reinterpret_cast<float*>(ws + p.off_dla);
  ba.dlpart = reinterpret_cast<float*>(ws + p.off_dlpart);
  ba.dkd = reinterpret_cast<float*>(ws + p.off_dkd);
  ba.N = p.N;
  ba.m = p.m;
  ba.BH = p.BH;
  ba.nT = p.nT;
  ba.nP = p.nP;
  ba.gw = p.gw;
  ba.ph = p.ph;
  ba.pw = p.pw;
  ba.iters = c.iters;
  ba.kind = p.kernel;
  ba.bf16 = p.bf16;
  ba.lambda = c.lambda;
  ba.eps = c.eps;
  ba.c_exp2 = ma.c_exp2;
  switch (p.D) {
    case 16: return launch_bwd_d<16>(p, ba, ma, dypart, xiter, amat, hscal, s);
    case 32: return launch_bwd_d<32>(p, ba, ma, dypart, xiter, amat, hscal, s);
    case 64: return launch_bwd_d<64>(p, ba, ma, dypart, xiter, amat, hscal, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace lapattn
