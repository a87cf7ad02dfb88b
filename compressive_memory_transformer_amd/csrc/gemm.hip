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
// Tiling: one workgroup per 256 x 256 output tile (8 waves of 64 x 128) for large
// products, 128 x 128 (4 waves of 64 x 64) for small ones; K in steps of 64 staged
// through two LDS buffers (the next step's global loads issued before the current
// step's products), v_mfma_f32_32x32x16_bf16 tiles.  A is read by rows from LDS; B
// (row-major [K][N]) through the transposing LDS read.
#include "common.h"
#include "kernels.h"

namespace infini {

namespace {

constexpr int kGK = 64;           // K step

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

// TM x TN output tile per workgroup; waves of WM x WN (WM / 32 x WN / 32 MFMA tiles).
template <int TM, int TN, int WM, int WN>
__global__ __launch_bounds__(64 * (TM / WM) * (TN / WN)) void gemm_bf16_kernel(GemmArgs g) {
  constexpr int NW = (TM / WM) * (TN / WN), NT = 64 * NW;
  constexpr int PA = kGK + 8, PB = TN + 8;            // LDS pitches (elements)
  constexpr int IA = TM * kGK / 8 / NT, IB = kGK * TN / 8 / NT;   // 16-byte pieces per thread
  constexpr int FM = WM / 32, FN = WN / 32;
  const int nt = blockIdx.x, mt = blockIdx.y;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, hh = lane >> 5, l32 = lane & 31;
  const int wm = (w / (TN / WN)) * WM, wn = (w % (TN / WN)) * WN;   // the wave's corner of the tile
  __shared__ __attribute__((aligned(16))) bf16 as[2][TM * PA];
  __shared__ __attribute__((aligned(16))) bf16 bs[2][kGK * PB];
  const int m0 = mt * TM, n0 = nt * TN;
  bf16x8 pa[IA], pb[IB];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < IA; ++i) {
      const int p = t + NT * i, ar = p / (kGK / 8), ac = (p % (kGK / 8)) * 8;
      pa[i] = *reinterpret_cast<const bf16x8*>(a_ptr(g, min(m0 + ar, g.M - 1), k0 + ac));
    }
#pragma unroll
    for (int i = 0; i < IB; ++i) {
      const int p = t + NT * i, br = p / (TN / 8), bc = (p % (TN / 8)) * 8;
      pb[i] = *reinterpret_cast<const bf16x8*>(g.b + (int64_t)(k0 + br) * g.N + min(n0 + bc, g.N - 8));
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < IA; ++i) {
      const int p = t + NT * i;
      *reinterpret_cast<bf16x8*>(as[buf] + (p / (kGK / 8)) * PA + (p % (kGK / 8)) * 8) = pa[i];
    }
#pragma unroll
    for (int i = 0; i < IB; ++i) {
      const int p = t + NT * i;
      *reinterpret_cast<bf16x8*>(bs[buf] + (p / (TN / 8)) * PB + (p % (TN / 8)) * 8) = pb[i];
    }
  };
  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
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
      bf16x8 ao[FM], bo[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) ao[i] = g_row_op(as[buf], PA, wm + 32 * i, 16 * ks, lane);
#pragma unroll
      for (int j = 0; j < FN; ++j) bo[j] = g_col_op(bs[buf], PB, 16 * ks, wn + 32 * j, lane);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma32(ao[i], bo[j], acc[i][j]);
    }
    if (next) store(buf ^ 1);
    __syncthreads();
  }
  // epilogue: lane holds rows m0 + wm + 32 i + acc_row, column n0 + wn + 32 j + l32
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int n = n0 + wn + 32 * j + l32;
    if (n >= g.N) continue;
    bf16* dst;
    int64_t stride_m, col;
    int hq = 0;
    // destination of column n: a row-major C, or one head of q, k or v
    if (g.c_heads) {
      const int nq = g.H * g.dk;
      if (n < nq) {
        dst = g.q; stride_m = g.dk; hq = n / g.dk; col = n % g.dk;
      } else if (n < 2 * nq) {
        dst = g.k; stride_m = g.dk; hq = (n - nq) / g.dk; col = (n - nq) % g.dk;
      } else {
        dst = g.v; stride_m = g.dv; hq = (n - 2 * nq) / g.dv; col = (n - 2 * nq) % g.dv;
      }
    } else {
      dst = g.c;
      stride_m = g.N;
      col = n;
    }
#pragma unroll
    for (int i = 0; i < FM; ++i)
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
  // 256 x 256 tiles (8 waves of 64 x 128, twice the products per staged byte of
  // 128 x 128) once there are enough of them to fill the chip
  const int64_t big = ((int64_t)(g.M + 255) / 256) * ((g.N + 255) / 256);
  if (big >= 256) {
    const dim3 grid((unsigned)((g.N + 255) / 256), (unsigned)((g.M + 255) / 256));
    hipLaunchKernelGGL((gemm_bf16_kernel<256, 256, 64, 128>), grid, dim3(512), 0, stream, g);
  } else {
    const dim3 grid((unsigned)((g.N + 127) / 128), (unsigned)((g.M + 127) / 128));
    hipLaunchKernelGGL((gemm_bf16_kernel<128, 128, 64, 64>), grid, dim3(256), 0, stream, g);
  }
  return hipGetLastError();
}

}  // namespace infini
