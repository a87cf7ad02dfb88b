// MFMA operand helpers for v_mfma_f32_32x32x16_bf16 over row-major bf16 LDS
// tiles (operand and accumulator layouts in common.h).
#pragma once

#include "common.h"

namespace infini {

// Row operand: lane l gets X[r0 + l % 32][k0 + 8 (l / 32) + 0..7] (an A operand, or
// the B operand of a product with X^T).
__device__ __forceinline__ bf16x8 mo_row(const bf16* X, int pitch, int r0, int k0, int lane) {
  return lds_read8(X + (r0 + (lane & 31)) * pitch + k0 + 8 * (lane >> 5));
}

// Transposed operand in natural contraction order: lane l gets
// X[r0 + 8 (l / 32) + e][c0 + l % 32], e = 0..7.
__device__ __forceinline__ bf16x8 mo_col(const bf16* X, int pitch, int r0, int c0, int lane) {
  const int h = lane >> 5, g = (lane >> 4) & 3, s = lane & 15;
  return lds_operand_tr(X, pitch, r0 + 8 * h, r0 + 8 * h + 4, c0 + 16 * (g & 1), s);
}

// Transposed operand in the row order of a 32 x 32 accumulator used as the other
// operand: lane l gets X[r0 + 4 h + e][c0 + l % 32] and X[r0 + 8 + 4 h + e][...].
__device__ __forceinline__ bf16x8 mo_col_acc(const bf16* X, int pitch, int r0, int c0, int lane) {
  const int h = lane >> 5, g = (lane >> 4) & 3, s = lane & 15;
  return lds_operand_tr(X, pitch, r0 + 4 * h, r0 + 8 + 4 * h, c0 + 16 * (g & 1), s);
}

// Row-major [rows x P] bf16 tiles (P = 128 or 64 elements) in LDS whose rows are
// the contraction index, read as v_mfma_f32_32x32x16_bf16 operands by
// ds_read_b64_tr_b16.  A 32-lane half of a read covers 4 consecutive rows x 4
// 16-byte chunks; the chunk swizzle moves rows r % 4 (P = 128) or (r / 2) % 2
// (P = 64) to disjoint groups of 4 chunks, so each half touches 16 distinct bank
// groups.  Physical chunk of logical chunk c in row r (an XOR: also the inverse):
template <int P>
__device__ __forceinline__ int trt_chunk(int r, int c) { return c ^ (P == 128 ? (r & 3) << 2 : ((r >> 1) & 1) << 2); }

// Element offset (relative to a 16-row step) of this lane's first transposing
// read for 32-column block cb; the second read is 8 rows further.  Lane l gets
// column 32 cb + l % 32 of rows {4 hi + e, 8 + 4 hi + e}, e = 0..3 (a fixed
// permutation of the 16 rows, the same for every operand read this way).
template <int P>
__device__ __forceinline__ int trt_offset(int lane, int cb) {
  const int hi = lane >> 5, grp = lane >> 4, sidx = lane & 15;
  const int row = 4 * hi + (sidx >> 2);
  const int col = 32 * cb + 16 * (grp & 1) + 4 * (sidx & 3);
  return row * P + 8 * trt_chunk<P>(row, col >> 3) + (col & 7);
}

template <int P>
__device__ __forceinline__ bf16x8 trt_read(const bf16* tile, int ofs) {
  const s16x4 x = lds_read_tr16(tile + ofs);
  const s16x4 y = lds_read_tr16(tile + ofs + 8 * P);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Rows 8 ks .. 8 ks + 7 of an accumulator as a bf16 B operand.
__device__ __forceinline__ bf16x8 mo_acc(const f32x16& c, int ks) {
  bf16x8 b;
#pragma unroll
  for (int j = 0; j < 8; ++j) b[j] = f2bf(c[8 * ks + j]);
  return b;
}

__device__ __forceinline__ f32x16 mo_zero() {
  f32x16 z;
#pragma unroll
  for (int r = 0; r < 16; ++r) z[r] = 0.f;
  return z;
}

// Row of accumulator element r for lane half h.
__device__ __forceinline__ int mo_acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// Column sums of a row-major fp32 [R][C] matrix in global memory (C <= 128) by a
// workgroup of 256 threads: threads t and t + 128 take alternate rows of column
// t % 128 with four loads in flight each, and meet in `tmp` (128 floats of LDS).
// Call from every thread; out[c] (c < C) is written by threads c < C after the
// internal barrier (readers need a barrier of their own).
__device__ __forceinline__ void block_colsum256(const float* X, int R, int C, float* out, float* tmp) {
  const int t = threadIdx.x, c = t & 127, half = t >> 7;
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  if (c < C) {
    int r = half;
    for (; r + 6 < R; r += 8) {
      a0 += X[(int64_t)r * C + c];
      a1 += X[(int64_t)(r + 2) * C + c];
      a2 += X[(int64_t)(r + 4) * C + c];
      a3 += X[(int64_t)(r + 6) * C + c];
    }
    for (; r < R; r += 2) a0 += X[(int64_t)r * C + c];
  }
  const float sum = (a0 + a1) + (a2 + a3);
  if (half == 1) tmp[c] = sum;
  __syncthreads();
  if (half == 0 && c < C) out[c] = sum + tmp[c];
}

}  // namespace infini
