// The attention block around the Nystrom attention: the projections of
// tokens X [B, N, C] into the heads' Q, K, V and of the heads' outputs back,
// as one SOFT layer of a pyramid backbone (SOFT review, "proposed method",
// last bullet; the symmetric kernel S = exp(Q (-) K) shares the query and key
// projection).
//
//   in  : Q = X Wq, K = X Wk (or Q), V = X Wv, weights [C, H d], written
//         straight into the heads' [B, H, N, d] layout (head h = columns
//         h d .. h d + d - 1) in the I/O type
//   attn: lapattn_forward on (Q, K, V)
//   out : Y = concat_h(O_h) Wo, Wo [H d, C], the heads gathered from
//         [B, H, N, d] while the tiles load
//
// One GEMM kernel for both: 64 x 64 output tiles, 4 waves of 32 x 32, the
// contraction in chunks of 32 staged in LDS as fp32 rows of both operands
// (the next chunk's loads in flight during the current chunk's products),
// fp32 MFMA (16x16x4, k = 8 g + s for lane group g at sub-step s), fp32
// accumulation; bf16 operands are widened exactly, bf16 outputs rounded to
// nearest even.

#include "lapattn_device.h"

namespace lapattn {
namespace {

constexpr int GT = 64;      // output tile side
constexpr int GK = 32;      // contraction chunk
constexpr int GS = GK + 4;  // LDS row stride of the staged chunks
constexpr int WGP = 256;    // 4 waves

struct ProjArgs {
  const void* a;      // MODE 0: X [M][Kd]; MODE 1: O [B][H][N][d]
  const void* w[3];   // weights [Kd][Nc], row-major
  void* out[3];       // MODE 0: [B][H][N][d]; MODE 1: Y [M][Nc]
  int M, Kd, Nc;      // rows (B N), contraction, columns
  int N, H, d;
  int bf16;
};

// Eight consecutive elements (fp32 or bf16, 16-byte aligned) as fp32.
__device__ __forceinline__ void load8(const void* base, size_t idx, int bf16, float* v) {
  if (bf16) {
    const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + idx);
    const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      v[2 * h] = __uint_as_float(w4[h] << 16);
      v[2 * h + 1] = __uint_as_float(w4[h] & 0xffff0000u);
    }
  } else {
    const f4 x0 = ld4(static_cast<const float*>(base) + idx), x1 = ld4(static_cast<const float*>(base) + idx + 4);
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      v[h] = x0[h];
      v[4 + h] = x1[h];
    }
  }
}

template <int MODE>
__global__ __launch_bounds__(WGP) void proj_kernel(ProjArgs p) {
  constexpr int OS = GT + 4;  // row stride of the staged output tile
  static_assert(GT * OS <= 2 * GT * GS, "output tile fits the operand arrays");
  __shared__ __attribute__((aligned(16))) float smem[2 * GT * GS];
  float* As = smem;            // [row][k]
  float* Bs = smem + GT * GS;  // [col][k]
  const int z = blockIdx.z;
  const void* w = p.w[z];
  void* out = p.out[z];
  const int r0 = blockIdx.x * GT, c0 = blockIdx.y * GT;
  const int tid = threadIdx.x, lane = tid & 63, wv = wave_id();
  const int lr = lane & 15, lg = lane >> 4;
  const int wr = 32 * (wv >> 1), wc = 32 * (wv & 1);  // this wave's 32 x 32 quadrant
  f4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

  // thread's slots of a chunk: A row ar (8 consecutive k at ak); B row bk of
  // the chunk (8 consecutive columns at bc; consecutive lanes take
  // consecutive k, so the transposed LDS stores fall on distinct banks)
  const int ar = tid >> 2, ak = 8 * (tid & 3);
  const int bk = tid & 31, bc = 8 * (tid >> 5);
  const int arow = r0 + ar, bcol = c0 + bc;
  // MODE 1: the A row is token (b, n) of the heads' layout
  size_t abase = 0;
  if constexpr (MODE == 1) {
    const int b = arow / p.N, n = arow % p.N;
    abase = (static_cast<size_t>(b) * p.H * p.N + n) * p.d;
  }
  float va[8], vb[8];
  auto fetch = [&](int k0) {
    if (arow < p.M) {
      size_t idx;
      if constexpr (MODE == 0) {
        idx = static_cast<size_t>(arow) * p.Kd + k0 + ak;
      } else {
        // k = h d + c  ->  O[b][h][n][c]
        const int k = k0 + ak, h = k / p.d, c = k - h * p.d;
        idx = abase + static_cast<size_t>(h) * p.N * p.d + c;
      }
      load8(p.a, idx, p.bf16, va);
    } else {
#pragma unroll
      for (int u = 0; u < 8; ++u) va[u] = 0.f;
    }
    if (bcol < p.Nc) {
      load8(w, static_cast<size_t>(k0 + bk) * p.Nc + bcol, p.bf16, vb);
    } else {
#pragma unroll
      for (int u = 0; u < 8; ++u) vb[u] = 0.f;
    }
  };
  // software pipeline: the next chunk's loads are in flight during this
  // chunk's products
  fetch(0);
  for (int k0 = 0; k0 < p.Kd; k0 += GK) {
    __syncthreads();  // the previous chunk's products are done with As, Bs
    st4(As + ar * GS + ak, f4{va[0], va[1], va[2], va[3]});
    st4(As + ar * GS + ak + 4, f4{va[4], va[5], va[6], va[7]});
#pragma unroll
    for (int u = 0; u < 8; ++u) Bs[(bc + u) * GS + bk] = vb[u];
    __syncthreads();
    if (k0 + GK < p.Kd) fetch(k0 + GK);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const float* ap = As + (wr + 16 * i + lr) * GS + 8 * lg;
      const f4 a0 = ld4(ap), a1 = ld4(ap + 4);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float* bp = Bs + (wc + 16 * j + lr) * GS + 8 * lg;
        const f4 b0 = ld4(bp), b1 = ld4(bp + 4);
        f4 c = acc[i][j];
#pragma unroll
        for (int s = 0; s < 4; ++s) c = mfma4(a0[s], b0[s], c);
#pragma unroll
        for (int s = 0; s < 4; ++s) c = mfma4(a1[s], b1[s], c);
        acc[i][j] = c;
      }
    }
  }
  // The tile goes through LDS so that every row leaves as whole 16-byte
  // chunks (4 consecutive columns, in one head for MODE 0 since 4 divides d).
  // accumulator of block (i, j): element (wr + 16 i + 4 lg + e, wc + 16 j + lr)
  __syncthreads();  // every wave is done with As, Bs
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) smem[(wr + 16 * i + 4 * lg + e) * OS + wc + 16 * j + lr] = acc[i][j][e];
  __syncthreads();
  // thread: chunk c4 = tid % 16 of rows tid / 16 + 16 q.  Output offsets
  // separate into a row part and a column part: MODE 0,
  // ((b H + h) N + n) d + c = (b H N + n) d + h N d + c; MODE 1, row Nc + col.
  const int c4 = tid & 15;
  const int col = c0 + 4 * c4;
  size_t coff;
  if constexpr (MODE == 0) {
    const int h = col / p.d, c = col - h * p.d;
    coff = static_cast<size_t>(h) * p.N * p.d + c;
  } else {
    coff = col;
  }
#pragma unroll
  for (int q = 0; q < GT / 16; ++q) {
    const int rl = (tid >> 4) + 16 * q, row = r0 + rl;
    if (row >= p.M || col >= p.Nc) continue;
    size_t roff;
    if constexpr (MODE == 0) {
      const int b = row / p.N, n = row - b * p.N;
      roff = (static_cast<size_t>(b) * p.H * p.N + n) * p.d;
    } else {
      roff = static_cast<size_t>(row) * p.Nc;
    }
    // Nc is a multiple of 32 (checked at the entry point): whole chunks
    const f4 v = ld4(smem + rl * OS + 4 * c4);
    const size_t o = roff + coff;
    if (p.bf16) {
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + o) =
          uint2{static_cast<unsigned>(f32_to_bf16_rne(v[0])) | (static_cast<unsigned>(f32_to_bf16_rne(v[1])) << 16),
                static_cast<unsigned>(f32_to_bf16_rne(v[2])) | (static_cast<unsigned>(f32_to_bf16_rne(v[3])) << 16)};
    } else {
      st4(static_cast<float*>(out) + o, v);
    }
  }
}

}  // namespace

hipError_t launch_block_proj(int mode, const void* a, const void* const* w, void* const* out, int nz, int M,
                             int Kd, int Nc, int N, int H, int d, int bf16, hipStream_t s) {
  ProjArgs p{};
  p.a = a;
  for (int z = 0; z < nz; ++z) {
    p.w[z] = w[z];
    p.out[z] = out[z];
  }
  p.M = M;
  p.Kd = Kd;
  p.Nc = Nc;
  p.N = N;
  p.H = H;
  p.d = d;
  p.bf16 = bf16;
  const dim3 grid((M + GT - 1) / GT, (Nc + GT - 1) / GT, nz);
  if (mode == 0) return launch(proj_kernel<0>, grid, dim3(WGP), s, Ev{}, p);
  return launch(proj_kernel<1>, grid, dim3(WGP), s, Ev{}, p);
}

}  // namespace lapattn
