// Internal launch plan shared by the C-ABI front end and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lapattn {

// Landmarks are padded to MP rows/columns inside the solver and the small
// contractions; padding rows and columns hold exact zeros.
constexpr int MP = 64;
// Counters per head in the workspace: [0] W partials done, [1] join of the
// solver and the W reduction.
constexpr int CTR_PER_HEAD = 4;

struct Plan {
  int B, H, gh, gw, D, ph, pw;
  int kernel;   // 0 Laplacian, 1 Gaussian
  int bf16;     // 0 fp32 I/O, 1 bf16 I/O
  int N, m, BH;
  int nT;       // 64-token tiles per head
  int ng;       // landmark groups per tile in the map stage
  int CH;       // tokens per W-partial chunk (multiple of 16)
  int nC;       // W-partial chunks per head
  // workspace byte offsets
  size_t off_ctr, off_L, off_kqlt, off_klkt, off_wpart, off_w, off_x, off_y;
  size_t total;
};

struct Buffers {
  unsigned* ctr;
  float* L;      // [BH][m][D]
  float* kqlt;   // [BH][m][N]  k(q_n, l_j) at [j][n]
  float* klkt;   // [BH][m][N]  k(l_j, k_n) at [j][n]
  float* wpart;  // [BH][nC][MP][D]
  float* w;      // [BH][MP][D]
  float* x;      // [BH][MP][MP]
  float* y;      // [BH][MP][D]
};

struct Args {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float lambda, eps;
  int iters;
  int shared_qk;
  // optional fp32 stage copies (may be null)
  float* st_L;
  float* st_kql;
  float* st_klk;
  float* st_a;
  float* st_x;
  float* st_w;
};

hipError_t launch_pool(const Plan& p, const Args& a, const Buffers& b, hipStream_t s);
hipError_t launch_ns(const Plan& p, const Args& a, const Buffers& b, int join_target, hipStream_t s);
hipError_t launch_maps(const Plan& p, const Args& a, const Buffers& b, hipStream_t s);
hipError_t launch_w(const Plan& p, const Args& a, const Buffers& b, int join_target, hipStream_t s);
hipError_t launch_out(const Plan& p, const Args& a, const Buffers& b, hipStream_t s);
hipError_t launch_export(const Plan& p, const Args& a, const Buffers& b, hipStream_t s);

}  // namespace lapattn
