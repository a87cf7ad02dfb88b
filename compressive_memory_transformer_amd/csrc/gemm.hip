// The projections on either side of the segment forward (close-reading page
// "精读笔记：Infini-attention": section 3.1, Q = X W_Q, K = X W_K, V = X W_V per
// head; section 3.6, O = [A^1; ...; A^H] W_O), as one bf16 MFMA GEMM
// C = A B (fp32 accumulation, bf16 result) with the head layout folded into
// its loads and stores, so no transpose pass touches HBM:
//   the QKV projection reads X [B L, d_model] by rows and stores each output
//   column straight into q, k or v [B, H, L, d] (columns: the H query heads, then
//   the H key heads, then the H value heads);
//   the output projection reads its A operand from the heads' outputs
//   A [B, H, L, d_value] as the rows of [B L, H d_value] (row (b, t), columns of
//   head h at h d_value) and stores Y [B L, d_model] by rows.
//
// Tiling: one workgroup (4 waves) per 128 x 128 output tile, K in steps of 64
// staged through two LDS buffers (the next step's global loads issued before the
// current step's products); each wave owns 64 x 64 (2 x 2 tiles of
// v_mfma_f32_32x32x16_bf16).  A is read by rows from LDS; B (row-major [K][N])
// through the transposing LDS read.
#include "common.h"
#include "kernels.h"

namespace infini {

namespace {

constexpr int kGT = 128;          // output tile edge
constexpr int kGK = 64;           // K step
constexpr int kGThreads = 256;
constexpr int kPA = kGK + 8;      // LDS pitch of the A tile (elements)
constexpr int kPB = kGT + 8;      // LDS pitch of the B tile

// Row operand from a row-major LDS tile: lane l gets X[r0 + l % 32][k0 + 8 (l / 32) + 0..7].
__device__ __forceinline__ bf16x8 g_row_op(const bf16* X, int pitch, int r0, int k0, int lane) {
  return lds_read8(X + (r0 + (lane & 31)) * pitch + k0 + 8 * (lane >> 5));
}
// B operand from a row-major [K][N] LDS tile: lane l gets X[k0 + 8 (l / 32) + e][n0 + l % 32].
__device__ __forceinline__ bf16x8 g_col_op(const bf16* X, int pitch, int k0, int n0, int lane) {
  const int h = lane >> 5, g = (lane >> 4) & 3, s = lane & 15;
  return lds_operand_tr(X, pitch, k0 + 8 * h, k0 + 8 * h + 4, n0 + 16 * (g & 1), s);
}

__device__ __forceinline__ int g_acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// Global address of A[m][k .. k + 7] (k a multiple of 8).
__device__ __forceinline__ const bf16* a_ptr(const GemmArgs& g, int m, int k) {
  if (g.a_heads) {
    const int b = m / g.L, t = m % g.L, h = k / g.dv, c = k % g.dv;
    return g.a + (((int64_t)b * g.H + h) * g.L + t) * g.dv + c;
  }
  return g.a + (int64_t)m * g.K + k;
}

}  // namespace

__global__ __launch_bounds__(kGThreads) void gemm_bf16_kernel(GemmArgs g) {
  const int nt = blockIdx.x, mt = blockIdx.y;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, l32 = lane & 31, hh = lane >> 5;
  const int wm = (w >> 1) * 64, wn = (w & 1) * 64;   // the wave's 64 x 64 corner of the tile
  __shared__ __attribute__((aligned(16))) bf16 as[2][kGT * kPA];
  __shared__ __attribute__((aligned(16))) bf16 bs[2][kGK * kPB];
  const int m0 = mt * kGT, n0 = nt * kGT;
  // staging: A tile 128 x 64 and B tile 64 x 128, 1024 pieces of 16 bytes each
  bf16x8 pa[4], pb[4];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = t + kGThreads * i;
      const int ar = p >> 3, ac = (p & 7) * 8;                       // A: row ar, columns ac .. ac + 7
      pa[i] = *reinterpret_cast<const bf16x8*>(a_ptr(g, min(m0 + ar, g.M - 1), k0 + ac));
      const int br = p >> 4, bc = (p & 15) * 8;                      // B: row br, columns bc .. bc + 7
      pb[i] = *reinterpret_cast<const bf16x8*>(g.b + (int64_t)(k0 + br) * g.N + min(n0 + bc, g.N - 8));
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = t + kGThreads * i;
      *reinterpret_cast<bf16x8*>(as[buf] + (p >> 3) * kPA + (p & 7) * 8) = pa[i];
      *reinterpret_cast<bf16x8*>(bs[buf] + (p >> 4) * kPB + (p & 15) * 8) = pb[i];
    }
  };
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  load(0);
  store(0);
  __syncthreads();
  for (int k0 = 0, buf = 0; k0 < g.K; k0 += kGK, buf ^= 1) {
    const bool next = k0 + kGK < g.K;
    if (next) load(k0 + kGK);
#pragma unroll
    for (int ks = 0; ks < kGK / 16; ++ks) {
      bf16x8 ao[2], bo[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) ao[i] = g_row_op(as[buf], kPA, wm + 32 * i, 16 * ks, lane);
#pragma unroll
      for (int j = 0; j < 2; ++j) bo[j] = g_col_op(bs[buf], kPB, 16 * ks, wn + 32 * j, lane);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(ao[i], bo[j], acc[i][j]);
    }
    if (next) store(buf ^ 1);
    __syncthreads();
  }
  // epilogue: lane holds rows m0 + wm + 32 i + acc_row, column n0 + wn + 32 j + l32
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + wn + 32 * j + l32;
    if (n >= g.N) continue;
    bf16* dst;
    int64_t stride_m, col;
    // destination of column n: a row-major C, or one head of q, k or v
    int d = 0, hq = 0;
    if (g.c_heads) {
      const int nq = g.H * g.dk;
      if (n < nq) {
        dst = g.q; d = g.dk; hq = n / g.dk; col = n % g.dk;
      } else if (n < 2 * nq) {
        dst = g.k; d = g.dk; hq = (n - nq) / g.dk; col = (n - nq) % g.dk;
      } else {
        dst = g.v; d = g.dv; hq = (n - 2 * nq) / g.dv; col = (n - 2 * nq) % g.dv;
      }
      stride_m = d;
    } else {
      dst = g.c;
      stride_m = g.N;
      col = n;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm + 32 * i + g_acc_row(r, hh);
        if (m >= g.M) continue;
        int64_t off;
        if (g.c_heads) {
          const int b = m / g.L, tt = m % g.L;
          off = (((int64_t)b * g.H + hq) * g.L + tt) * stride_m + col;
        } else {
          off = (int64_t)m * stride_m + col;
        }
        dst[off] = f2bf(acc[i][j][r]);
      }
  }
}

hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t stream) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  if (g.K % kGK != 0 || g.N % 8 != 0) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((g.N + kGT - 1) / kGT), (unsigned)((g.M + kGT - 1) / kGT));
  hipLaunchKernelGGL(gemm_bf16_kernel, grid, dim3(kGThreads), 0, stream, g);
  return hipGetLastError();
}

}  // namespace infini
