// Causal kernel linear attention (page "第24章 Sparse与Infinite Attention",
// section 24.4): O_i = phi(q_i)^T S_i / (phi(q_i)^T Z_i) with the prefix states
// S_i = sum_{j <= i} phi(k_j) v_j^T, Z_i = sum_{j <= i} phi(k_j) over the stream,
// phi = ELU + 1.
//
// The stream is cut into chunks (the state's segment length).  The linear-rule
// state kernels give every chunk's starting state (bf16 M^T, fp32 z); this kernel
// adds the chunk's own keys up to each query:
//   num_i = phi(q_i) M + sum_{j <= i} w_ij v_j,
//   den_i = phi(q_i) . z + sum_{j <= i} w_ij,      w_ij = phi(q_i) . phi(k_j),
// with phi(q) and phi(k) rounded to bf16 as MFMA operands.  Every term of w_ij and
// of phi(q) M is then a product of positive (or, for M, bounded) factors each
// carrying bf16's relative precision whatever the magnitude of phi: a 128-term
// weight is good to about 2e-4 relative both for inputs near 0 (phi ~ 1) and for
// strongly negative inputs (phi ~ e^x << 1), where forming w as
// d + sum (phi(k) - 1) + sum (phi(q) - 1) + (phi(q) - 1).(phi(k) - 1) cancels
// almost completely.  The denominator's memory part phi(q) . z is an fp32 dot
// product.  One workgroup (4 waves) per 128 queries of a chunk, one wave per 32;
// weights transposed (keys x queries) so the accumulator feeds the product with
// V^T directly.
#include "common.h"
#include "kernels.h"
#include "mfma_ops.h"

namespace infini {

namespace {
constexpr int kKlWaves = 4;
constexpr int kKlBlock = 32 * kKlWaves;   // queries per workgroup
constexpr int kKlChunk = 64;              // keys per staged step
}  // namespace

template <int D>
__global__ __launch_bounds__(64 * kKlWaves) void kla_kernel(FaArgs a) {
  constexpr int P = D + 8, KS = D / 16, DB = D / 32;
  constexpr int PIECES = kKlChunk * D / 8 / (64 * kKlWaves);
  const int qb = blockIdx.x, s = blockIdx.y, bh = blockIdx.z;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, l32 = lane & 31, hh = lane >> 5;
  __shared__ __attribute__((aligned(16))) bf16 kc[2][kKlChunk * P];
  __shared__ __attribute__((aligned(16))) bf16 vc[2][kKlChunk * P];
  __shared__ float zsh[D];
  const int64_t seg = (int64_t)bh * a.S + s;
  const int64_t seg0 = (int64_t)bh * a.L + (int64_t)s * a.N;
  const int q0 = qb * kKlBlock, qw0 = q0 + 32 * w;
  const bool qvalid = qw0 < a.N;
  const int qcol = qw0 + l32;
  const int64_t qrow = seg0 + min(qcol, a.N - 1);
  const int kend = min(a.N, q0 + kKlBlock);

  // the chunk's starting z (M^T itself is read as an operand straight from
  // memory at the end)
  if (t < D) zsh[t] = a.snapz[seg * D + t];
  // the lane's query: phi(q) as the B operand (natural order) and in fp32
  bf16x8 qm[KS];
  float qf[KS][8];
#pragma unroll
  for (int c = 0; c < KS; ++c) {
    const bf16x8 x = *reinterpret_cast<const bf16x8*>(a.q + qrow * D + 16 * c + 8 * hh);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float v = bf2f(x[j]);
      const float f = v > 0.f ? v + 1.f : exp_e(v);
      qf[c][j] = f;
      qm[c][j] = f2bf(f);
    }
  }

  // staging of one key chunk: phi(k) into kc, v into vc
  bf16x8 pk[PIECES], pv[PIECES];
  auto load = [&](int kc0) {
#pragma unroll
    for (int i = 0; i < PIECES; ++i) {
      const int p = t + 64 * kKlWaves * i, r = p / (D / 8), c8 = p % (D / 8);
      pk[i] = *reinterpret_cast<const bf16x8*>(a.k + (seg0 + kc0 + r) * D + 8 * c8);
      pv[i] = *reinterpret_cast<const bf16x8*>(a.v + (seg0 + kc0 + r) * D + 8 * c8);
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PIECES; ++i) {
      const int p = t + 64 * kKlWaves * i, r = p / (D / 8), c8 = p % (D / 8);
      bf16x8 kp;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float v = bf2f(pk[i][j]);
        kp[j] = f2bf(v > 0.f ? v + 1.f : exp_e(v));
      }
      *reinterpret_cast<bf16x8*>(kc[buf] + r * P + 8 * c8) = kp;
      *reinterpret_cast<bf16x8*>(vc[buf] + r * P + 8 * c8) = pv[i];
    }
  };

  f32x16 o[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d) o[d] = mo_zero();
  float den = 0.f;
  load(0);
  store(0);
  __syncthreads();
  for (int kc0 = 0, buf = 0; kc0 < kend; kc0 += kKlChunk, buf ^= 1) {
    const bool next = kc0 + kKlChunk < kend;
    if (next) load(kc0 + kKlChunk);
    if (qvalid && kc0 <= qw0 + 31) {   // a chunk wholly after the wave's queries is skipped
      const bool below = kc0 + kKlChunk - 1 <= qw0;
      f32x16 sa[2] = {mo_zero(), mo_zero()};
#pragma unroll
      for (int c = 0; c < KS; ++c)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) sa[kt] = mfma32(mo_row(kc[buf], P, 32 * kt, 16 * c, lane), qm[c], sa[kt]);
      bf16x8 pb[2][2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        if (below) {   // every key of the chunk precedes every query of the wave
#pragma unroll
          for (int r = 0; r < 16; ++r) den += sa[kt][r];
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kl = 32 * kt + mo_acc_row(r, hh);
            const float wv = kc0 + kl <= qcol ? sa[kt][r] : 0.f;
            sa[kt][r] = wv;
            den += wv;
          }
        }
        pb[kt][0] = mo_acc(sa[kt], 0);
        pb[kt][1] = mo_acc(sa[kt], 1);
      }
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          o[d] = mfma32(mo_col_acc(vc[buf], P, 32 * kt, 32 * d, lane), pb[kt][0], o[d]);
          o[d] = mfma32(mo_col_acc(vc[buf], P, 32 * kt + 16, 32 * d, lane), pb[kt][1], o[d]);
        }
    }
    if (next) store(buf ^ 1);
    __syncthreads();
  }
  // phi(q) . z of the starting state
  float dz = 0.f;
#pragma unroll
  for (int c = 0; c < KS; ++c)
#pragma unroll
    for (int j = 0; j < 8; ++j) dz = __builtin_fmaf(qf[c][j], zsh[16 * c + 8 * hh + j], dz);
  den += __shfl_xor(den, 32);
  dz += __shfl_xor(dz, 32);
  // The exact denominator is > 0 (the query's own key is in the sum); a
  // non-positive one (only from underflow of every phi) gives a zero row, the
  // rule of the forward retrieval.
  const float tot = den + dz;
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  if (!qvalid) return;
#pragma unroll
  for (int d = 0; d < DB; ++d) {
    f32x16 rt = mo_zero();
#pragma unroll
    for (int c = 0; c < KS; ++c) {
      // A operand: row 32 d + l % 32 of M^T (d_value), columns 16 c + 8 (l / 32) ..
      const bf16x8 ma = *reinterpret_cast<const bf16x8*>(a.snapM + seg * D * D + (32 * d + l32) * D + 16 * c + 8 * hh);
      rt = mfma32(ma, qm[c], rt);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int col = 32 * d + mo_acc_row(r, hh);
      a.out[qrow * D + col] = f2bf((rt[r] + o[d][r]) * inv);
    }
  }
}

template <int D>
hipError_t launch_kla(const FaArgs& a, hipStream_t stream) {
  if (a.N % kKlChunk != 0) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((a.N + kKlBlock - 1) / kKlBlock), (unsigned)a.S, (unsigned)(a.B * a.H));
  hipLaunchKernelGGL(kla_kernel<D>, grid, dim3(64 * kKlWaves), 0, stream, a);
  return hipGetLastError();
}
template hipError_t launch_kla<64>(const FaArgs&, hipStream_t);
template hipError_t launch_kla<128>(const FaArgs&, hipStream_t);

}  // namespace infini
