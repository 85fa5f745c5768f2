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
//   head  one workgroup per head: W, dY (partials summed in order); Y = X W,
//         dW = X^T dY, dX = dY W^T
//   grad  Newton-Schulz backward workgroups (one per head, split fp16
//         operands on fp16 MFMA in LDS, then dA and dd = -dA k(L, L) /
//         lambda) beside one workgroup per 64-token tile of Q
//         or K: the kernel map again, dK_QL = dO Y^T (or dK_LK^T = V dW^T)
//         on fp32 MFMA, the gradient map on FP32 VALU (dQ or the direct dK
//         rows, and the tile's dL partial), and for key tiles dV = K_LK^T dW;
//         the two roles do not wait for each other
//   dk    one workgroup per landmark window: dL = its part from A (from dd)
//         and its tile partials in fixed order, dK rows of the window =
//         direct part + dL / (ph pw)
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
  float* dxmat;        // [BH][MP][MP]         dX = dY W^T (rows, columns >= m zero);
                       //                      then dd = -dA k(L, L) / lambda (from the
                       //                      Newton-Schulz backward, for dk)
  float* dlpart;       // [BH][2 nT][MP][D]    dL partials of the gradient tiles
  float* dkd;          // [BH][N][D]           direct part of dK
  unsigned* sync;      // hand-off words (zeroed by the pool launch)
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
    const float sum = lane < m ? a_row_abs_sum<G::N16, SX>(Af, lane) : 0.f;
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
  constexpr int MAP_SMEM = map_smem<D, KIND>();
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

// Head reduction, in kBwdHeadSlices workgroups per head: workgroup r sums
// elements [r E, (r + 1) E) of the W^T and the dY^T partials (one thread per
// element, partials in order, 32 loads in flight), stores the sums with
// device-scope stores into Y's and dW's buffers (free until the products
// below) and counts its arrival; the head's last workgroup to arrive reads
// W and dY back and forms the products.  With one workgroup per head the
// reduction ran at one CU's load latency (31 us for 8 heads of 25 partials).
constexpr int kBwdHeadSlices = 16;

template <int D>
__global__ __launch_bounds__(WGM) void bwd_heada_kernel(BwdArgs a) {
  constexpr int NB64 = 16;           // 16 x 16 blocks of a 64 x 64 product
  constexpr int NBD = 4 * (D / 16);  // blocks of a 64 x D product
  constexpr int E = D * MP / kBwdHeadSlices;
  static_assert(2 * E <= WGM, "one thread per element of the slice");
  __shared__ __attribute__((aligned(16))) float sm[3 * MP * BS];
  float* M0 = sm;
  float* M1 = sm + MP * BS;
  float* M2 = sm + 2 * MP * BS;
  const int bh = blockIdx.y, tid = threadIdx.x;
  const int m = a.m, nP = a.nP, T = a.iters;
  const size_t ps = static_cast<size_t>(D) * MP;
  const int lane = tid & 63, w = wave_id(), lr = lane & 15, lg = lane >> 4;
  float* wred = a.ymat + static_cast<size_t>(bh) * MP * D;    // W^T [D][MP] until the products
  float* dyred = a.dwmat + static_cast<size_t>(bh) * MP * D;  // dY^T [D][MP] likewise

  if (tid < 2 * E) {
    const bool isw = tid < E;
    const int o = static_cast<int>(blockIdx.x) * E + (isw ? tid : tid - E);  // c MP + j
    const float* src = (isw ? a.wpart : a.dypart) + static_cast<size_t>(bh) * nP * ps + o;
    float sum = 0.f;
    if (o % MP < m) {
      for (int p0 = 0; p0 < nP; p0 += 32) {
        float v[32];
#pragma unroll
        for (int u = 0; u < 32; ++u) v[u] = p0 + u < nP ? src[(p0 + u) * ps] : 0.f;
#pragma unroll
        for (int u = 0; u < 32; ++u)
          if (p0 + u < nP) sum += v[u];
      }
    }
    st_dev((isw ? wred : dyred) + o, sum);
  }
  unsigned* cnt = a.sync + kSyncHead * (bh + 1) + kBwdHeadCount;
  if (publish_arrive(cnt) != static_cast<unsigned>(kBwdHeadSlices - 1)) return;

  // the last workgroup: W[j][c] and dY[j][c] (row stride BS), zero beyond m
  // and D
  for (int e = tid; e < MP * MP; e += WGM) {
    const int c = e / MP, j = e % MP;
    float vw = 0.f, vd = 0.f;
    if (c < D) {
      vw = wred[e];
      vd = dyred[e];
    }
    M0[j * BS + c] = vw;
    M1[j * BS + c] = vd;
  }
  load_mm(M2, a.xiter + (static_cast<size_t>(bh) * (T + 1) + T) * MP * MP, m);  // X = X_T
  __syncthreads();
  // Y = X W and dW = X^T dY (64 x D, rows >= m zero) to global memory
  f4 acc[(NBD + 7) / 8];
  for (int pass = 0; pass < 2; ++pass) {
    if (pass == 0) lds_mm<NBD>(M2, BS, 1, M0, BS, 1, D / 16, acc);
    else lds_mm<NBD>(M2, 1, BS, M1, BS, 1, D / 16, acc);
    float* dst = (pass == 0 ? a.ymat : a.dwmat) + static_cast<size_t>(bh) * MP * D;
#pragma unroll
    for (int s = 0; s < (NBD + 7) / 8; ++s) {
      const int blk = w + 8 * s;
      if (blk < NBD) {
        const int bi = blk / (D / 16), bj = blk % (D / 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[(16 * bi + 4 * lg + i) * D + 16 * bj + lr] = acc[s][i];
      }
    }
  }
  // dX = dY W^T (64 x 64): rows of dY against rows of W
  f4 g[2];
  lds_mm<NB64>(M1, BS, 1, M0, 1, BS, 4, g);
  float* dx = a.dxmat + static_cast<size_t>(bh) * MP * MP;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int blk = w + 8 * s, bi = blk / 4, bj = blk % 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) dx[(16 * bi + 4 * lg + i) * MP + 16 * bj + lr] = g[s][i];
  }
}

// ---------------------------------------------------------------------------
// The fused launch: Newton-Schulz backward workgroups (one per head, first in
// the grid) beside the gradient tiles; neither waits for the other.
// ---------------------------------------------------------------------------
constexpr int WGG = 256;

// Operands of the Newton-Schulz backward products: a 64 x 64 matrix M as
// fp16 hi and lo parts of 2^s M (s keeps the magnitudes below 2^15), rows of
// HSH halves; the 16-byte reads of 16 consecutive rows fall on distinct
// banks.
constexpr int HSH = 72;
constexpr int HMAT = MP * HSH / 2;  // floats per part
constexpr int NSB_HALVES = 14;      // A, X, X^T, G, G^T, Q1, P1: hi and lo
constexpr int NSB_SLOTS = NSB_HALVES * HMAT;
constexpr int NSB_SMEM = NSB_SLOTS + 16;
static_assert(NSB_SLOTS >= 7 * MP * BS + 8, "the fp32 matrices of the last part fit");

// Split operand rows 16 b + r (lane (g, r)), halves 32 p + 8 g .. + 7 of
// both chunks, and the 6 MFMAs of one block of sum over k < 64 of
// A[i][k] B^T[j][k] from the rows of A and of B^T (hi hi + lo hi + hi lo on
// fp16 MFMA).
struct HOp {
  u32x4 h[2], l[2];
};
__device__ __forceinline__ HOp load_hop(const uint16_t* H, const uint16_t* L, int b) {
  const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int o = (16 * b + lr) * HSH + 8 * lg;
  HOp r;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    r.h[p] = *reinterpret_cast<const u32x4*>(H + o + 32 * p);
    r.l[p] = *reinterpret_cast<const u32x4*>(L + o + 32 * p);
  }
  return r;
}
__device__ __forceinline__ f4 mm_hop(const HOp& a, const HOp& b, f4 c) {
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    c = mfma_h(a.h[p], b.h[p], c);
    c = mfma_h(a.l[p], b.h[p], c);
    c = mfma_h(a.h[p], b.l[p], c);
  }
  return c;
}

// Block (bi, bj) of accumulator c, times the power of two sc, split into
// the half matrices (H, L) and, with HT, into the transposed ones too.
__device__ __forceinline__ void put_block_h(uint16_t* H, uint16_t* L, uint16_t* HT, uint16_t* LT, int bi, int bj,
                                            f4 c, float sc, float one) {
  const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  unsigned h01, l01, h23, l23;
  split2_mix(c[0] * sc, c[1] * sc, one, h01, l01);
  split2_mix(c[2] * sc, c[3] * sc, one, h23, l23);
  const unsigned hv[4] = {h01 & 0xffffu, h01 >> 16, h23 & 0xffffu, h23 >> 16};
  const unsigned lv[4] = {l01 & 0xffffu, l01 >> 16, l23 & 0xffffu, l23 >> 16};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int o = (16 * bi + 4 * lg + i) * HSH + 16 * bj + lr;
    H[o] = static_cast<uint16_t>(hv[i]);
    L[o] = static_cast<uint16_t>(lv[i]);
  }
  if (HT) {
    // row 16 bj + r, columns 16 bi + 4 g .. + 3: one 8-byte store per part
    const int o = (16 * bj + lr) * HSH + 16 * bi + 4 * lg;
    *reinterpret_cast<u32x2*>(HT + o) = u32x2{h01, h23};
    *reinterpret_cast<u32x2*>(LT + o) = u32x2{l01, l23};
  }
}

// Four consecutive elements (row r, columns 4 c4 ..) of a matrix, times sc,
// split into the half matrices (H, L) and the transposed ones (HT, LT).
__device__ __forceinline__ void put_row4_h(uint16_t* H, uint16_t* L, uint16_t* HT, uint16_t* LT, int r, int c4,
                                           f4 v, float sc, float one) {
  unsigned h01, l01, h23, l23;
  split2_mix(v[0] * sc, v[1] * sc, one, h01, l01);
  split2_mix(v[2] * sc, v[3] * sc, one, h23, l23);
  const int o = r * HSH + 4 * c4;
  *reinterpret_cast<u32x2*>(H + o) = u32x2{h01, h23};
  *reinterpret_cast<u32x2*>(L + o) = u32x2{l01, l23};
  if (HT) {
    const unsigned hv[4] = {h01 & 0xffffu, h01 >> 16, h23 & 0xffffu, h23 >> 16};
    const unsigned lv[4] = {l01 & 0xffffu, l01 >> 16, l23 & 0xffffu, l23 >> 16};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ot = (4 * c4 + i) * HSH + r;
      HT[ot] = static_cast<uint16_t>(hv[i]);
      LT[ot] = static_cast<uint16_t>(lv[i]);
    }
  }
}

// Scale exponent of a matrix with maximum mx for nsb_role: fp16_scale, at
// most 40.  G shrinks by orders of magnitude per step once the forward has
// converged (its step map is flat at the fixed point); the cap keeps every
// scale and its inverse finite, and a G that small adds nothing measurable.
__device__ __forceinline__ int nsb_scale(float mx) {
  const int s = fp16_scale(mx);
  return s < 40 ? s : 40;
}

// Maximum of non-negative v over the 4 waves of the workgroup: each wave's
// maximum goes to slot[w]; every thread reads the four after the next
// barrier (max4_slots).
__device__ __forceinline__ void wave_max_to_slot(float* slot, float v) {
  v = __uint_as_float(wave_max_u(__float_as_uint(v)));
  if ((threadIdx.x & 63) == 0) slot[wave_id()] = v;
}
__device__ __forceinline__ float max4_slots(const float* slot) {
  const f4 v = ld4(slot);
  return fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
}

// Newton-Schulz backward of one head (4 waves).  LDS holds A, X_t and X_t^T,
// G and G^T, Q1 = A X_t and P1 = X_t^T G as split fp16 operands, so that
// every product reads rows of both operands on fp16 MFMA (three products
// per contraction chunk, about 22 significant bits, as in the forward).
// Scales: A, X_t and G by their maxima (nsb_scale), Q1 and P1 by 2^-22 of
// their products' scales (every term of a product is below 2^30 and there
// are 64, so the accumulator is below 2^36).  Wave w owns the blocks w,
// w + 4, w + 8, w + 12 of dA and of G (fp32, in registers across the
// steps).  X_{t-1} is read from global memory during step t.
template <int D, int KIND>
__device__ void nsb_role(const BwdArgs& a, int bh, float* sm) {
  float* MA = sm;
  float* MG = sm + 3 * MP * BS;
  float* red = sm + 7 * MP * BS;
  const int tid = threadIdx.x, w = wave_id();
  const int m = a.m, T = a.iters;
  const float* xi = a.xiter + static_cast<size_t>(bh) * (T + 1) * MP * MP;
  // A, G = dX and X_{T-1} (or nothing to do when T == 0): their maxima,
  // then their split parts into LDS; G of the own blocks into registers
  uint16_t* hbase = reinterpret_cast<uint16_t*>(sm);
  auto half = [&](int k) { return hbase + static_cast<size_t>(k) * HMAT * 2; };
  uint16_t *AH = half(0), *AL = half(1), *XH = half(2), *XL = half(3), *XTH = half(4), *XTL = half(5);
  uint16_t *GH = half(6), *GL = half(7), *GTH = half(8), *GTL = half(9), *QH = half(10), *QL = half(11);
  uint16_t *PH = half(12), *PL = half(13);
  float* slot = sm + NSB_SLOTS;  // [3][4]: maxima of A (or G'), X, G
  const int lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const float one = opaque_one();
  constexpr int R4 = MP * MP / 4 / WGG;  // rows-of-4 per thread of a 64 x 64 matrix
  f4 av[R4], gv4[R4], xv[R4];
  {
    const float* ag = a.amat + static_cast<size_t>(bh) * MP * MP;
    const float* dg = a.dxmat + static_cast<size_t>(bh) * MP * MP;
    const float* xg = xi + static_cast<size_t>(T > 0 ? T - 1 : 0) * MP * MP;
    float ma = 0.f, mg = 0.f, mx = 0.f;
#pragma unroll
    for (int u = 0; u < R4; ++u) {
      const int e4 = tid + WGG * u, r = e4 / 16, c4 = e4 % 16;
      av[u] = ld4(ag + r * MP + 4 * c4);
      gv4[u] = ld4(dg + r * MP + 4 * c4);
      const f4 x = ld4(xg + r * MP + 4 * c4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xv[u][i] = (r < m && 4 * c4 + i < m) ? x[i] : 0.f;
        ma = fmaxf(ma, fabsf(av[u][i]));
        mg = fmaxf(mg, fabsf(gv4[u][i]));
        mx = fmaxf(mx, fabsf(xv[u][i]));
      }
    }
    wave_max_to_slot(slot, ma);
    wave_max_to_slot(slot + 4, mx);
    wave_max_to_slot(slot + 8, mg);
  }
  f4 g[4];
  {
    const float* dg = a.dxmat + static_cast<size_t>(bh) * MP * MP;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int blk = w + 4 * s, bi = blk >> 2, bj = blk & 3;
#pragma unroll
      for (int i = 0; i < 4; ++i) g[s][i] = dg[(16 * bi + 4 * lg + i) * MP + 16 * bj + lr];
    }
  }
  __syncthreads();
  const int sA = nsb_scale(max4_slots(slot));
  int sX = nsb_scale(max4_slots(slot + 4));
  int sG = nsb_scale(max4_slots(slot + 8));
#pragma unroll
  for (int u = 0; u < R4; ++u) {
    const int e4 = tid + WGG * u, r = e4 / 16, c4 = e4 % 16;
    put_row4_h(AH, AL, nullptr, nullptr, r, c4, av[u], ldexpf(1.0f, sA), one);
    put_row4_h(GH, GL, GTH, GTL, r, c4, gv4[u], ldexpf(1.0f, sG), one);
    put_row4_h(XH, XL, XTH, XTL, r, c4, xv[u], ldexpf(1.0f, sX), one);
  }
  __syncthreads();
  f4 da[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) da[s] = f4{0.f, 0.f, 0.f, 0.f};
  // X_{t-1} is consumed in step t (after its second barrier) and read two
  // steps ahead: nx holds X_{t-1}, nn receives X_{t-2}
  auto read_x = [&](int i, f4 (&dst)[R4]) {
    const float* xg = xi + static_cast<size_t>(i) * MP * MP;
#pragma unroll
    for (int u = 0; u < R4; ++u) {
      const int e4 = tid + WGG * u, r = e4 / 16, c4 = e4 % 16;
      dst[u] = ld4(xg + r * MP + 4 * c4);
    }
  };
  f4 nx[R4], nn[R4];
  if (T >= 2) read_x(T - 2, nx);
  for (int t = T - 1; t >= 0; --t) {
    if (t >= 2) read_x(t - 2, nn);
    // Q1 = A X_t (rows of A, rows of X_t^T); P1 = X_t^T G (rows of X_t^T,
    // rows of G^T), each stored at 2^-22 of its accumulator's scale
    // (wave w owns column block w, row blocks 0..3: the second operand of
    // every product is read once per phase; all products of a phase come
    // before its stores, so that no operand read waits behind a store)
    const int sQ = sA + sX - 22, sP = sX + sG - 22;
    const HOp bxt = load_hop(XTH, XTL, w), bgt = load_hop(GTH, GTL, w);
    {
      f4 aq[4], ap[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        aq[s] = mm_hop(load_hop(AH, AL, s), bxt, f4{0.f, 0.f, 0.f, 0.f});
        ap[s] = mm_hop(load_hop(XTH, XTL, s), bgt, f4{0.f, 0.f, 0.f, 0.f});
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        put_block_h(QH, QL, nullptr, nullptr, s, w, aq[s], 0x1p-22f, one);
        put_block_h(PH, PL, nullptr, nullptr, s, w, ap[s], 0x1p-22f, one);
      }
    }
    __syncthreads();
    // dA -= P1 X_t^T (rows of P1, rows of X_t); G' = 2 G - G Q1^T - Q1 G,
    // with (X_t A)^T taken as A X_t: X_t commutes with A and is symmetric in
    // exact arithmetic, and the recursion is linear in G, so the rounding
    // difference of the two stays at rounding level
    const float upd = ldexpf(1.0f, -(sP + sX)), ugq = ldexpf(1.0f, -(sG + sQ));
    float mg = 0.f;
    const HOp bx = load_hop(XH, XL, w), bq = load_hop(QH, QL, w);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const f4 pd = mm_hop(load_hop(PH, PL, s), bx, f4{0.f, 0.f, 0.f, 0.f});
      f4 gq = mm_hop(load_hop(GH, GL, s), bq, f4{0.f, 0.f, 0.f, 0.f});
      gq = mm_hop(load_hop(QH, QL, s), bgt, gq);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        da[s][i] = fmaf(-pd[i], upd, da[s][i]);
        g[s][i] = fmaf(-gq[i], ugq, 2.f * g[s][i]);
        mg = fmaxf(mg, fabsf(g[s][i]));
      }
    }
    wave_max_to_slot(slot + 8, mg);
    if (t > 0) {
      float mx = 0.f;
#pragma unroll
      for (int u = 0; u < R4; ++u) {
        const int e4 = tid + WGG * u, r = e4 / 16, c4 = e4 % 16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          nx[u][i] = (r < m && 4 * c4 + i < m) ? nx[u][i] : 0.f;
          mx = fmaxf(mx, fabsf(nx[u][i]));
        }
      }
      wave_max_to_slot(slot + 4, mx);
    }
    __syncthreads();  // every read of G, X_t, Q1, P1 is done; the maxima are in
    sG = nsb_scale(max4_slots(slot + 8));
    const float scg = ldexpf(1.0f, sG);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int blk = w + 4 * s;
      put_block_h(GH, GL, GTH, GTL, blk >> 2, blk & 3, g[s], scg, one);
    }
    if (t > 0) {
      sX = nsb_scale(max4_slots(slot + 4));
      const float scx = ldexpf(1.0f, sX);
#pragma unroll
      for (int u = 0; u < R4; ++u) {
        const int e4 = tid + WGG * u, r = e4 / 16, c4 = e4 % 16;
        put_row4_h(XH, XL, XTH, XTL, r, c4, nx[u], scx, one);
      }
    }
#pragma unroll
    for (int u = 0; u < R4; ++u) nx[u] = nn[u];
    __syncthreads();
  }
  // the last part in fp32: A from global memory, G from the registers
  {
    const float* ag = a.amat + static_cast<size_t>(bh) * MP * MP;
    for (int e = tid; e < MP * MP; e += WGG) MA[(e / MP) * BS + e % MP] = ag[e];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int blk = w + 4 * s, bi = blk >> 2, bj = blk & 3;
#pragma unroll
      for (int i = 0; i < 4; ++i) MG[(16 * bi + 4 * lg + i) * BS + 16 * bj + lr] = g[s][i];
    }
  }
  __syncthreads();
  // dA += alpha G; d alpha = <G, A> flows through alpha = 1 / (c r), c = r =
  // the largest column (row) abs-sum: dA[:, jc] and dA[jc, :] each gain
  // -d alpha alpha / c sign(A)
  const float* hs = a.hscal + 4 * static_cast<size_t>(bh);
  const float alpha = hs[0], csum = hs[2];
  const int jc = __float_as_int(hs[1]);
  {
    float part = 0.f;
    for (int e = tid; e < MP * MP; e += WGG) {
      const int r = e / MP, c = e % MP;
      part = fmaf(MG[r * BS + c], MA[r * BS + c], part);
    }
    // fixed-order sum: per wave, then over waves
    for (int o = 32; o > 0; o >>= 1) part += __shfl_xor(part, o);
    if ((tid & 63) == 0) red[w] = part;
    __syncthreads();
    float dalpha = 0.f;
    for (int i = 0; i < WGG / 64; ++i) dalpha += red[i];
    const float dc = -dalpha * alpha / csum;
    const int lane = tid & 63, lr = lane & 15, lg = lane >> 4;
    const float il = 1.0f / a.lambda;
    // dd = -dA k(L, L) / lambda (k(L, L) = A - eps I inside m x m)
    float* ddg = a.dxmat + static_cast<size_t>(bh) * MP * MP;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int blk = w + 4 * s, bi = blk >> 2, bj = blk & 3;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * bi + 4 * lg + i, c = 16 * bj + lr;
        float v = fmaf(alpha, MG[r * BS + c], da[s][i]);
        float dd = 0.f;
        if (r < m && c < m) {
          const float av = MA[r * BS + c];
          const float sg = av > 0.f ? 1.f : (av < 0.f ? -1.f : 0.f);
          if (c == jc) v = fmaf(dc, sg, v);
          if (r == jc) v = fmaf(dc, sg, v);
          dd = -v * (av - (r == c ? a.eps : 0.f)) * il;
        }
        // dX (read at the start) is dead: dd takes its place, and the dk
        // launch forms dL from it, one landmark per workgroup
        ddg[r * MP + c] = dd;
      }
    }
  }
}

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

// LDS floats of one gradient tile (see grad_tile).
template <int D>
constexpr int grad_smem() {
  constexpr int XS = D + 4, R = 64 / D;
  constexpr int U1 = TILE * BS + TILE * XS + MP * XS;
  constexpr int U2 = 4 * R * MP * D;
  return TILE * XS + MP * XS + MP * BS + (U1 > U2 ? U1 : U2);
}

// One workgroup (4 waves) per 64-token tile of Q (side 0) or K (side 1).
template <int D, int KIND, bool BF16>
__device__ void grad_tile(const BwdArgs& a, int tile, float* sm) {
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
  float* XT = sm + OFF_XT;
  float* LM = sm + OFF_LM;
  float* WT = sm + OFF_WT;
  float* P = sm + OFF_P;
  float* VO = sm + OFF_VO;
  float* YB = sm + OFF_YB;
  float* PL = sm + OFF_U;

  const int nT = a.nT, N = a.N, m = a.m;
  const int bh = tile / (2 * nT);
  const int side = (tile / nT) & 1;  // 0: query tile, 1: key tile
  const int t = tile % nT;
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

template <int D, int KIND, bool BF16>
__global__ __launch_bounds__(WGG) void bwd_fused_kernel(BwdArgs a) {
  constexpr int G = grad_smem<D>();
  __shared__ __attribute__((aligned(16))) float sm[G > NSB_SMEM ? G : NSB_SMEM];
  if (static_cast<int>(blockIdx.x) < a.BH) nsb_role<D, KIND>(a, blockIdx.x, sm);
  else grad_tile<D, KIND, BF16>(a, blockIdx.x - a.BH, sm);
}

// ---------------------------------------------------------------------------
// dk: one workgroup per (landmark window j, head): dL[j] = its part from A
// plus its 2 nT tile partials (thread (g, c) takes partials and landmarks
// g, g + G, ..., then the G sums are added in order); the window's dK rows =
// direct part + dL[j] / (ph pw).
// ---------------------------------------------------------------------------
template <int D, bool BF16>
__global__ __launch_bounds__(WGG) void bwd_dk_kernel(BwdArgs a) {
  constexpr int G = WGG / D;
  __shared__ float part[WGG];
  __shared__ float dl[D];
  __shared__ float dds[MP];
  const int j = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int c = tid % D, g = tid / D;
  const int np = 2 * a.nT, m = a.m;
  // dd[j][p] + dd[p][j] for the part of dL from A (dd from the Newton-Schulz
  // backward)
  if (tid < MP) {
    const float* dd = a.dxmat + static_cast<size_t>(bh) * MP * MP;
    dds[tid] = tid < m ? dd[j * MP + tid] + dd[tid * MP + j] : 0.f;
  }
  const float* pb = a.dlpart + static_cast<size_t>(bh) * np * MP * D + j * D + c;
  float s = 0.f;
  // partials g, g + G, ... in order, 16 loads in flight
  for (int p0 = g; p0 < np; p0 += 16 * G) {
    float v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int p = p0 + G * u;
      v[u] = p < np ? pb[static_cast<size_t>(p) * MP * D] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (p0 + G * u < np) s += v[u];
  }
  // landmark coordinates l_p[c] of this thread's landmarks p = g, g + G, ...
  const float* Lh = a.L + static_cast<size_t>(bh) * m * D;
  const float lj = Lh[j * D + c];
  float lp[MP / G];
#pragma unroll
  for (int k = 0; k < MP / G; ++k) {
    const int p = g + G * k;
    lp[k] = p < m ? Lh[p * D + c] : lj;
  }
  __syncthreads();
  // dL from A: sum over landmarks p of (dd[j][p] + dd[p][j]) s(l_j - l_p),
  // s = sign (Laplacian) or 2 x (Gaussian)
#pragma unroll
  for (int k = 0; k < MP / G; ++k) {
    const int p = g + G * k;
    const float x = lj - lp[k];
    const float sv = a.kind == 0 ? (x > 0.f ? 1.f : (x < 0.f ? -1.f : 0.f)) : 2.f * x;
    if (p < m) s = fmaf(dds[p], sv, s);
  }
  part[tid] = s;
  __syncthreads();
  if (tid < D) {
    float acc = 0.f;
    for (int u = 0; u < G; ++u) acc += part[u * D + tid];
    dl[tid] = acc / static_cast<float>(a.ph * a.pw);
  }
  __syncthreads();
  const int mw = a.gw / a.pw, R0 = j / mw, C0 = j % mw;
  const int cnt = a.ph * a.pw;
  // 16 rows' loads in flight before their stores
  for (int e0 = tid; e0 < cnt * D; e0 += 16 * WGG) {
    float v[16];
    size_t o[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int e = e0 + u * WGG;
      const int ec = e < cnt * D ? e : cnt * D - 1;  // in bounds either way
      const int tk = ec / D, cc = ec % D;
      const int n = (R0 * a.ph + tk / a.pw) * a.gw + C0 * a.pw + tk % a.pw;
      o[u] = (static_cast<size_t>(bh) * a.N + n) * D + cc;
      v[u] = e < cnt * D ? a.dkd[o[u]] + dl[cc] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      if (e0 + u * WGG >= cnt * D) break;
      if (BF16) static_cast<uint16_t*>(a.dk)[o[u]] = f32_to_bf16_rne(v[u]);
      else static_cast<float*>(a.dk)[o[u]] = v[u];
    }
  }
}

template <int D, int MB>
hipError_t launch_part_dm(const MainArgs& ma, const void* dout, float* dypart, float* xiter, float* amat,
                          float* hscal, unsigned grid, hipStream_t s, Ev ev) {
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
                        float* xiter, float* amat, float* hscal, hipStream_t s, const Ev* ev) {
  const unsigned gpart = static_cast<unsigned>(p.BH + 2 * p.BH * p.nP);
  hipError_t e = hipErrorInvalidValue;
  switch (p.ns_mb) {
    case 1: e = launch_part_dm<D, 1>(ma, ba.dout, dypart, xiter, amat, hscal, gpart, s, ev[1]); break;
    case 2: e = launch_part_dm<D, 2>(ma, ba.dout, dypart, xiter, amat, hscal, gpart, s, ev[1]); break;
    case 3: e = launch_part_dm<D, 3>(ma, ba.dout, dypart, xiter, amat, hscal, gpart, s, ev[1]); break;
    case 4: e = launch_part_dm<D, 4>(ma, ba.dout, dypart, xiter, amat, hscal, gpart, s, ev[1]); break;
  }
  if (e != hipSuccess) return e;
  e = launch(bwd_heada_kernel<D>, dim3(kBwdHeadSlices, p.BH), dim3(WGM), s, ev[2], ba);
  if (e != hipSuccess) return e;
  // Newton-Schulz backward workgroups first, then the gradient tiles
  const dim3 gg(static_cast<unsigned>(p.BH + p.BH * 2 * p.nT));
  if (p.kernel == 0)
    e = p.bf16 ? launch(bwd_fused_kernel<D, 0, true>, gg, dim3(WGG), s, ev[3], ba)
               : launch(bwd_fused_kernel<D, 0, false>, gg, dim3(WGG), s, ev[3], ba);
  else
    e = p.bf16 ? launch(bwd_fused_kernel<D, 1, true>, gg, dim3(WGG), s, ev[3], ba)
               : launch(bwd_fused_kernel<D, 1, false>, gg, dim3(WGG), s, ev[3], ba);
  if (e != hipSuccess) return e;
  const dim3 gk(static_cast<unsigned>(p.m), static_cast<unsigned>(p.BH));
  return p.bf16 ? launch(bwd_dk_kernel<D, true>, gk, dim3(WGG), s, ev[4], ba)
                : launch(bwd_dk_kernel<D, false>, gk, dim3(WGG), s, ev[4], ba);
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
    const hipError_t e = launch_pool(fp, fa, fb, s, c.ev[0]);
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
  ba.dxmat = reinterpret_cast<float*>(ws + p.off_dxmat);
  ba.sync = sync;
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
    case 16: return launch_bwd_d<16>(p, ba, ma, dypart, xiter, amat, hscal, s, c.ev);
    case 32: return launch_bwd_d<32>(p, ba, ma, dypart, xiter, amat, hscal, s, c.ev);
    case 64: return launch_bwd_d<64>(p, ba, ma, dypart, xiter, amat, hscal, s, c.ev);
  }
  return hipErrorInvalidValue;
}

}  // namespace lapattn
