// Local attention part of the gradients on the bf16 MFMA units (the chain rule
// through A_dot = softmax(scale Q K^T, causal) V of the close-reading page
// "精读笔记：Infini-attention", section 3.1 with the mask of section 3.8 step 2).
//
//   bwd_q_mfma_kernel<D>: one workgroup (4 waves) per 128 query rows of a
//     segment, one wave per 32 rows.  First sweep over the keys: the row's
//     softmax maximum and sum, A_dot, then E = <dA, A_dot> and D = (1 - g) E.
//     The retrieval (section 3.3) from M_{s-1} staged in LDS as bf16:
//     A_mem = (colsum(M) + (sigma(q) - 1) M) / (sigma(q) z) (the column sums in
//     fp32 keep sigma(q) ~ 1 from costing bf16 precision), the gate's share of
//     dbeta, rs = g / den and dden.  Second sweep: dS = P ((1 - g) dP - D) and
//     dq += scale dS K; then the retrieval's dq = (M (rs dA) + dden z) sigma'(q).  Scores are
//     computed transposed (keys x queries), so every register operand is already
//     in the accumulator layout of the product that consumes it.
//   bwd_kv_mfma_kernel<D>: one workgroup per 128 keys, one wave per 32 keys,
//     the wave's keys and values held as operands in registers; for every chunk
//     of 64 later queries: S, dP, P, dS, then dv += (1 - g) P^T dA and
//     dk += scale dS^T Q.
//
// Operands (v_mfma_f32_32x32x16_bf16): a row-major LDS tile X is read either by
// rows (row_op: lane l gets X[r0 + l % 32][k0 + 8 (l / 32) + 0..7]) or, for a
// contraction over its rows, with the transposing LDS read (tr_op: lane l gets
// X[r0 + 4 h + e][c0 + l % 32] and X[r0 + 8 + 4 h + e][...], h = l / 32), whose
// row order matches a 32 x 32 accumulator used as the other operand (lane l
// holds rows 8 (r / 4) + 4 h + r % 4 of column l % 32).  Chunks of K, V (or Q,
// dA) are staged through two LDS buffers, the next chunk's global loads issued
// before the current chunk's products.
#include "common.h"
#include "kernels.h"
#include "mfma_ops.h"

namespace infini {

namespace {

constexpr int kBwdWaves = 4;
constexpr int kBwdBlock = 32 * kBwdWaves;   // rows (queries or keys) per workgroup
constexpr int kChunk = 64;                  // rows of the streamed operand per step

__device__ __forceinline__ bf16x8 row_op(const bf16* X, int pitch, int r0, int k0, int lane) {
  return lds_read8(X + (r0 + (lane & 31)) * pitch + k0 + 8 * (lane >> 5));
}

__device__ __forceinline__ bf16x8 tr_op(const bf16* X, int pitch, int r0, int c0, int lane) {
  const int h = lane >> 5, g = (lane >> 4) & 3, s = lane & 15;
  return lds_operand_tr(X, pitch, r0 + 4 * h, r0 + 8 + 4 * h, c0 + 16 * (g & 1), s);
}

// Transposed operand in natural contraction order (for a B operand loaded by
// rows): lane l gets X[r0 + 8 h + e][c0 + l % 32], e = 0..7.
__device__ __forceinline__ bf16x8 tr_nat(const bf16* X, int pitch, int r0, int c0, int lane) {
  const int h = lane >> 5, g = (lane >> 4) & 3, s = lane & 15;
  return lds_operand_tr(X, pitch, r0 + 8 * h, r0 + 8 * h + 4, c0 + 16 * (g & 1), s);
}

// Accumulator rows 8 ks .. 8 ks + 7 of `c` as a bf16 B operand.
__device__ __forceinline__ bf16x8 acc_op(const f32x16& c, int ks) {
  bf16x8 b;
#pragma unroll
  for (int j = 0; j < 8; ++j) b[j] = f2bf(c[8 * ks + j]);
  return b;
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int r = 0; r < 16; ++r) z[r] = 0.f;
  return z;
}

// Row of accumulator element r for lane half h.
__device__ __forceinline__ int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// Loads a 64-row chunk of two row-major [rows][D] bf16 tensors into registers
// (16 bytes per piece) and stores it into LDS tiles of pitch D + 8.
template <int D>
struct ChunkPair {
  static constexpr int P = D + 8;
  static constexpr int PIECES = kChunk * D / 8 / (64 * kBwdWaves);
  bf16x8 x[PIECES], y[PIECES];
  __device__ __forceinline__ void load(const bf16* X, const bf16* Y, int64_t row0) {
#pragma unroll
    for (int i = 0; i < PIECES; ++i) {
      const int p = threadIdx.x + 64 * kBwdWaves * i, r = p / (D / 8), c8 = p % (D / 8);
      x[i] = *reinterpret_cast<const bf16x8*>(X + (row0 + r) * D + 8 * c8);
      y[i] = *reinterpret_cast<const bf16x8*>(Y + (row0 + r) * D + 8 * c8);
    }
  }
  __device__ __forceinline__ void store(bf16* xs, bf16* ys) const {
#pragma unroll
    for (int i = 0; i < PIECES; ++i) {
      const int p = threadIdx.x + 64 * kBwdWaves * i, r = p / (D / 8), c8 = p % (D / 8);
      *reinterpret_cast<bf16x8*>(xs + r * P + 8 * c8) = x[i];
      *reinterpret_cast<bf16x8*>(ys + r * P + 8 * c8) = y[i];
    }
  }
};

}  // namespace

template <int D>
__global__ __launch_bounds__(64 * kBwdWaves) void bwd_q_mfma_kernel(BwdArgs a) {
  constexpr int P = D + 8, KS = D / 16, DB = D / 32;
  const int qb = blockIdx.x, s = blockIdx.y, bh = blockIdx.z, h = bh % a.H;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, l32 = lane & 31, hh = lane >> 5;
  const bf16* Q = static_cast<const bf16*>(a.q);
  const bf16* K = static_cast<const bf16*>(a.k);
  const bf16* V = static_cast<const bf16*>(a.v);
  const bf16* DO = static_cast<const bf16*>(a.dout);
  __shared__ __attribute__((aligned(16))) bf16 kc[2][kChunk * P];
  __shared__ __attribute__((aligned(16))) bf16 vc[2][kChunk * P];
  __shared__ __attribute__((aligned(16))) bf16 ms[D * P];   // M_{s-1} [d_key][d_value] in bf16
  __shared__ float msum[D], zsh[D], ctmp[128];
  const int64_t seg0 = (int64_t)bh * a.L + (int64_t)s * a.N;
  const int q0 = qb * kBwdBlock, qw0 = q0 + 32 * w;
  const bool has_mem = a.seg_base + s > 0;
  const bool qvalid = qw0 < a.N;
  const int qcol = qw0 + l32;                      // this lane's query (column of S^T)
  const int64_t qrow = seg0 + min(qcol, a.N - 1);
  const float g = sigmoid_gate(a.beta[h]);
  const float sl2 = a.scale * kLog2e;
  bf16x8 qr[KS], dr[KS];
#pragma unroll
  for (int c = 0; c < KS; ++c) {
    qr[c] = *reinterpret_cast<const bf16x8*>(Q + qrow * D + 16 * c + 8 * hh);
    dr[c] = *reinterpret_cast<const bf16x8*>(DO + qrow * D + 16 * c + 8 * hh);
  }
  const int kend = min(a.N, q0 + kBwdBlock);
  {
    const float* Mg = a.snapM + ((int64_t)bh * a.S + s) * D * D;
    for (int x = threadIdx.x; x < D * D; x += 64 * kBwdWaves) ms[(x / D) * P + x % D] = f2bf(Mg[x]);
    if (threadIdx.x < D) zsh[threadIdx.x] = a.snapz[((int64_t)bh * a.S + s) * D + threadIdx.x];
    block_colsum256(Mg, D, D, msum, ctmp);
  }

  // ---- first sweep: maximum, sum and A_dot^T of the wave's 32 query columns
  f32x16 o[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d) o[d] = zero16();
  float m2 = -__builtin_inff(), l = 0.f;
  ChunkPair<D> cp;
  cp.load(K, V, seg0);
  cp.store(kc[0], vc[0]);
  __syncthreads();
  for (int kc0 = 0, buf = 0; kc0 < kend; kc0 += kChunk, buf ^= 1) {
    const bool next = kc0 + kChunk < kend;
    if (next) cp.load(K, V, seg0 + kc0 + kChunk);
    // both 32-key halves of the chunk at once: four independent product chains,
    // one rescale per 64 keys (a chunk wholly after the wave's queries is skipped)
    if (qvalid && kc0 <= qw0 + 31) {
      f32x16 sa[2] = {zero16(), zero16()};
#pragma unroll
      for (int c = 0; c < KS; ++c)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) sa[kt] = mfma32(row_op(kc[buf], P, 32 * kt, 16 * c, lane), qr[c], sa[kt]);
      float mx = -__builtin_inff();
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float v = kc0 + 32 * kt + acc_row(r, hh) <= qcol ? sa[kt][r] * sl2 : -__builtin_inff();
          sa[kt][r] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mn = fmaxf(m2, mx);               // finite: key 0 is in the first chunk
      const float alpha = exp2_fast(m2 - mn);
      l *= alpha;
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[d][r] *= alpha;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = exp2_fast(sa[kt][r] - mn);
          sa[kt][r] = p;
          l += p;
        }
      m2 = mn;
      bf16x8 pb[2][2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        pb[kt][0] = acc_op(sa[kt], 0);
        pb[kt][1] = acc_op(sa[kt], 1);
      }
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          o[d] = mfma32(tr_op(vc[buf], P, 32 * kt, 32 * d, lane), pb[kt][0], o[d]);
          o[d] = mfma32(tr_op(vc[buf], P, 32 * kt + 16, 32 * d, lane), pb[kt][1], o[d]);
        }
    }
    if (next) cp.store(kc[buf ^ 1], vc[buf ^ 1]);
    __syncthreads();
  }
  const float lt = l + __shfl_xor(l, 32);
  const float lse2 = m2 + log2f(lt);
  const float inv_l = 1.f / lt;
  // A_mem^T = (colsum(M) + M^T (sigma(q) - 1)^T) / den for the lane's query
  bf16x8 qm[KS];
  float den = 0.f;
#pragma unroll
  for (int c = 0; c < KS; ++c)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float x = bf2f(qr[c][j]);
      const float f = x > 0.f ? x : exp_e(x) - 1.f;
      qm[c][j] = f2bf(f);
      den = __builtin_fmaf(f + 1.f, zsh[16 * c + 8 * hh + j], den);
    }
  den += __shfl_xor(den, 32);
  const bool has = has_mem && den > 0.f;
  const float inv_den = has ? 1.f / den : 0.f;
  // E = <dA, A_dot> and <dA, A_mem> of the lane's query: the lane holds 16 DB
  // values of each transposed row
  float e = 0.f, em = 0.f;
#pragma unroll
  for (int d = 0; d < DB; ++d) {
    f32x16 am = zero16();
    if (has_mem) {
#pragma unroll
      for (int c = 0; c < KS; ++c) am = mfma32(tr_nat(ms, P, 16 * c, 32 * d, lane), qm[c], am);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int col = 32 * d + acc_row(r, hh);
      const float da = bf2f(DO[qrow * D + col]);
      e = __builtin_fmaf(da, o[d][r], e);
      em = __builtin_fmaf(da, (msum[col] + am[r]) * inv_den, em);
    }
  }
  e = (e + __shfl_xor(e, 32)) * inv_l;
  em += __shfl_xor(em, 32);
  const float Dv = (1.f - g) * e;
  const float rs = g * inv_den;
  const float dden = -g * em * inv_den;
  if (qvalid && hh == 0) {
    a.lse[qrow] = lse2 * (1.f / kLog2e);
    a.drow[qrow] = Dv;
    a.rs[qrow] = rs;
    a.dden[qrow] = dden;
  }
  // the gate's share of dbeta for the wave's 32 queries: g (1 - g) sum (<dA, A_mem> - E)
  {
    const float bt = wave_sum(qvalid && hh == 0 ? em - e : 0.f);
    if (qvalid && lane == 0) a.dbeta_part[((int64_t)bh * a.S + s) * a.nqb + qw0 / 32] = bt * g * (1.f - g);
  }

  // ---- second sweep: dq^T += K^T dS^T
  f32x16 dq[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d) dq[d] = zero16();
  cp.load(K, V, seg0);
  cp.store(kc[0], vc[0]);
  __syncthreads();
  for (int kc0 = 0, buf = 0; kc0 < kend; kc0 += kChunk, buf ^= 1) {
    const bool next = kc0 + kChunk < kend;
    if (next) cp.load(K, V, seg0 + kc0 + kChunk);
    if (qvalid && kc0 <= qw0 + 31) {
      f32x16 sa[2] = {zero16(), zero16()}, pa[2] = {zero16(), zero16()};
#pragma unroll
      for (int c = 0; c < KS; ++c)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          sa[kt] = mfma32(row_op(kc[buf], P, 32 * kt, 16 * c, lane), qr[c], sa[kt]);
          pa[kt] = mfma32(row_op(vc[buf], P, 32 * kt, 16 * c, lane), dr[c], pa[kt]);
        }
      bf16x8 db[2][2];
      const bool below = kc0 + kChunk - 1 <= qw0;   // every key of the chunk precedes every query
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        if (below) {
#pragma unroll
          for (int r = 0; r < 16; ++r) sa[kt][r] = exp2_fast(sa[kt][r] * sl2 - lse2) * ((1.f - g) * pa[kt][r] - Dv);
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const bool vis = kc0 + 32 * kt + acc_row(r, hh) <= qcol;
            const float p = vis ? exp2_fast(sa[kt][r] * sl2 - lse2) : 0.f;
            sa[kt][r] = p * ((1.f - g) * pa[kt][r] - Dv);
          }
        }
        db[kt][0] = acc_op(sa[kt], 0);
        db[kt][1] = acc_op(sa[kt], 1);
      }
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          dq[d] = mfma32(tr_op(kc[buf], P, 32 * kt, 32 * d, lane), db[kt][0], dq[d]);
          dq[d] = mfma32(tr_op(kc[buf], P, 32 * kt + 16, 32 * d, lane), db[kt][1], dq[d]);
        }
    }
    if (next) cp.store(kc[buf ^ 1], vc[buf ^ 1]);
    __syncthreads();
  }
  // the retrieval's dq^T = (M (rs dA)^T + dden z) sigma'(q): M rows from LDS,
  // rs dA as the B operand from the dA rows already in registers
  bf16x8 dn[KS];
#pragma unroll
  for (int c = 0; c < KS; ++c)
#pragma unroll
    for (int j = 0; j < 8; ++j) dn[c][j] = f2bf(rs * bf2f(dr[c][j]));
  if (qvalid) {
#pragma unroll
    for (int d = 0; d < DB; ++d) {
      f32x16 dm = zero16();
      if (has_mem) {   // wave-uniform; rows without memory have rs = dden = 0
#pragma unroll
        for (int c = 0; c < KS; ++c) dm = mfma32(row_op(ms, P, 32 * d, 16 * c, lane), dn[c], dm);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int col = 32 * d + acc_row(r, hh);
        const float x = bf2f(Q[qrow * D + col]);
        const float sp = x > 0.f ? 1.f : exp_e(x);
        a.dq_acc[qrow * D + col] = __builtin_fmaf(a.scale, dq[d][r], (dm[r] + dden * zsh[col]) * sp);
      }
    }
  }
}

template <int D>
__global__ __launch_bounds__(64 * kBwdWaves) void bwd_kv_mfma_kernel(BwdArgs a) {
  constexpr int P = D + 8, KS = D / 16, DB = D / 32;
  const int kb = blockIdx.x, s = blockIdx.y, bh = blockIdx.z, h = bh % a.H;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, l32 = lane & 31, hh = lane >> 5;
  const bf16* Q = static_cast<const bf16*>(a.q);
  const bf16* K = static_cast<const bf16*>(a.k);
  const bf16* V = static_cast<const bf16*>(a.v);
  const bf16* DO = static_cast<const bf16*>(a.dout);
  __shared__ __attribute__((aligned(16))) bf16 qc[2][kChunk * P];
  __shared__ __attribute__((aligned(16))) bf16 dc[2][kChunk * P];
  __shared__ __attribute__((aligned(16))) float lc[2][kChunk];
  __shared__ __attribute__((aligned(16))) float dcr[2][kChunk];
  const int64_t seg0 = (int64_t)bh * a.L + (int64_t)s * a.N;
  const int j0 = kb * kBwdBlock, kw0 = j0 + 32 * w;
  const bool kvalid = kw0 < a.N;
  const int kcol = kw0 + l32;                      // this lane's key (column of S)
  const int64_t krow = seg0 + min(kcol, a.N - 1);
  const float g = sigmoid_gate(a.beta[h]);
  const float sl2 = a.scale * kLog2e;
  bf16x8 kr[KS], vr[KS];
#pragma unroll
  for (int c = 0; c < KS; ++c) {
    kr[c] = *reinterpret_cast<const bf16x8*>(K + krow * D + 16 * c + 8 * hh);
    vr[c] = *reinterpret_cast<const bf16x8*>(V + krow * D + 16 * c + 8 * hh);
  }
  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d) dk[d] = dv[d] = zero16();
  ChunkPair<D> cp;
  const int qbeg = min(j0, a.N - kChunk);          // queries before j0 see none of these keys
  cp.load(Q, DO, seg0 + qbeg);
  cp.store(qc[0], dc[0]);
  if (threadIdx.x < kChunk) {
    lc[0][threadIdx.x] = a.lse[seg0 + qbeg + threadIdx.x] * kLog2e;
    dcr[0][threadIdx.x] = a.drow[seg0 + qbeg + threadIdx.x];
  }
  __syncthreads();
  for (int qc0 = qbeg, buf = 0; qc0 < a.N; qc0 += kChunk, buf ^= 1) {
    const bool next = qc0 + kChunk < a.N;
    float nl = 0.f, nd = 0.f;
    if (next) {
      cp.load(Q, DO, seg0 + qc0 + kChunk);
      if (threadIdx.x < kChunk) {
        nl = a.lse[seg0 + qc0 + kChunk + threadIdx.x];
        nd = a.drow[seg0 + qc0 + kChunk + threadIdx.x];
      }
    }
    // both 32-query halves of the chunk at once (a chunk wholly before the wave's
    // keys is skipped)
    if (kvalid && qc0 + kChunk - 1 >= kw0) {
      const bool below = qc0 >= kw0 + 31;   // wave-uniform
      f32x16 sa[2] = {zero16(), zero16()}, pa[2] = {zero16(), zero16()};
#pragma unroll
      for (int c = 0; c < KS; ++c)
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          sa[qt] = mfma32(row_op(qc[buf], P, 32 * qt, 16 * c, lane), kr[c], sa[qt]);
          pa[qt] = mfma32(row_op(dc[buf], P, 32 * qt, 16 * c, lane), vr[c], pa[qt]);
        }
      // S: rows are queries qc0 + 32 qt + acc_row, the lane's column the key kcol
      bf16x8 pb[2][2], db[2][2];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        // the rows' log-normalisers and D: accumulator rows come in runs of four
        f32x4 lq[4], dq4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          lq[j] = *reinterpret_cast<const f32x4*>(&lc[buf][32 * qt + 8 * j + 4 * hh]);
          dq4[j] = *reinterpret_cast<const f32x4*>(&dcr[buf][32 * qt + 8 * j + 4 * hh]);
        }
        f32x16 ds;
        if (below) {   // every query of the chunk follows every key of the wave
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = exp2_fast(sa[qt][r] * sl2 - lq[r >> 2][r & 3]);
            sa[qt][r] = p;
            ds[r] = p * ((1.f - g) * pa[qt][r] - dq4[r >> 2][r & 3]);
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int il = 32 * qt + acc_row(r, hh);
            const bool vis = kcol <= qc0 + il;
            const float p = vis ? exp2_fast(sa[qt][r] * sl2 - lq[r >> 2][r & 3]) : 0.f;
            sa[qt][r] = p;
            ds[r] = p * ((1.f - g) * pa[qt][r] - dq4[r >> 2][r & 3]);
          }
        }
        pb[qt][0] = acc_op(sa[qt], 0);
        pb[qt][1] = acc_op(sa[qt], 1);
        db[qt][0] = acc_op(ds, 0);
        db[qt][1] = acc_op(ds, 1);
      }
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          dv[d] = mfma32(tr_op(dc[buf], P, 32 * qt, 32 * d, lane), pb[qt][0], dv[d]);
          dv[d] = mfma32(tr_op(dc[buf], P, 32 * qt + 16, 32 * d, lane), pb[qt][1], dv[d]);
          dk[d] = mfma32(tr_op(qc[buf], P, 32 * qt, 32 * d, lane), db[qt][0], dk[d]);
          dk[d] = mfma32(tr_op(qc[buf], P, 32 * qt + 16, 32 * d, lane), db[qt][1], dk[d]);
        }
    }
    if (next) {
      cp.store(qc[buf ^ 1], dc[buf ^ 1]);
      if (threadIdx.x < kChunk) {
        lc[buf ^ 1][threadIdx.x] = nl * kLog2e;
        dcr[buf ^ 1][threadIdx.x] = nd;
      }
    }
    __syncthreads();
  }
  if (kvalid) {
#pragma unroll
    for (int d = 0; d < DB; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t i = krow * D + 32 * d + acc_row(r, hh);
        a.dv_acc[i] = (1.f - g) * dv[d][r];
        a.dk_acc[i] = a.scale * dk[d][r];
      }
  }
}

// Linear rule, per 128 tokens of a segment (one wave per 32), given G = dL/dM_s
// (fp32 [d_key][d_value], staged in LDS as bf16 with fp32 column sums):
//   dv += sigma(K) G = colsum(G) + (sigma(K) - 1) G;   d sigma(K) = V G^T.
template <int D>
__global__ __launch_bounds__(64 * kBwdWaves) void bwd_lin_update_mfma_kernel(BwdArgs a) {
  constexpr int P = D + 8, KS = D / 16, DB = D / 32;
  const int rb = blockIdx.x, s = blockIdx.y, bh = blockIdx.z;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, l32 = lane & 31, hh = lane >> 5;
  const bf16* K = static_cast<const bf16*>(a.k);
  const bf16* V = static_cast<const bf16*>(a.v);
  __shared__ __attribute__((aligned(16))) bf16 gs[D * P];
  __shared__ float gsum[D], ctmp[128];
  const float* Gg = a.dMr + ((int64_t)bh * a.S + s) * D * D;
  for (int x = threadIdx.x; x < D * D; x += 64 * kBwdWaves) gs[(x / D) * P + x % D] = f2bf(Gg[x]);
  block_colsum256(Gg, D, D, gsum, ctmp);
  const int t0 = rb * kBwdBlock + 32 * w;           // the wave's first token in the segment
  const bool valid = t0 < a.N;
  const int64_t row = (int64_t)bh * a.L + (int64_t)s * a.N + min(t0 + l32, a.N - 1);
  bf16x8 kp[KS], vr[KS];
#pragma unroll
  for (int c = 0; c < KS; ++c) {
    const bf16x8 kx = *reinterpret_cast<const bf16x8*>(K + row * D + 16 * c + 8 * hh);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float x = bf2f(kx[j]);
      kp[c][j] = f2bf(x > 0.f ? x : exp_e(x) - 1.f);
    }
    vr[c] = *reinterpret_cast<const bf16x8*>(V + row * D + 16 * c + 8 * hh);
  }
  __syncthreads();
  if (!valid) return;
  const int64_t out0 = (int64_t)bh * a.L + (int64_t)s * a.N + t0;
#pragma unroll
  for (int d = 0; d < DB; ++d) {
    f32x16 dv = zero16(), df = zero16();
#pragma unroll
    for (int c = 0; c < KS; ++c) {
      dv = mfma32(kp[c], tr_nat(gs, P, 16 * c, 32 * d, lane), dv);
      df = mfma32(vr[c], row_op(gs, P, 32 * d, 16 * c, lane), df);
    }
    const int col = 32 * d + l32;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t i = (out0 + acc_row(r, hh)) * D + col;
      a.dv_acc[i] += gsum[col] + dv[r];
      a.dfk_acc[i] = df[r];
    }
  }
}

// A per-segment Gram product on MFMA, one workgroup per segment, 64 tokens per
// step, both operands read transposed from LDS:
//   GRAM = false (delta rule): A_s = sigma(K)^T diag(w) sigma(K), w_t = 1 / (sigma(K_t) .
//     z_{s-1}) (0 in a stream's first segment).  With sigma(K) = 1 + K' (K' rounded
//     to bf16 for the product) A_s = (sum w) 1 1^T + 1 u^T + u 1^T + K'^T diag(w) K',
//     u = K'^T w, the rank-one terms in fp32;
//   GRAM = true (retrieval gradients, both rules): dMr_s = sigma(Q)^T diag(rs) dA =
//     1 (dA^T rs)^T + Q'^T diag(rs) dA and dzr_s = sigma(Q)^T dden, the column sums
//     in fp32 from the inputs.
template <int D, bool RETR>
__global__ __launch_bounds__(64 * kBwdWaves) void bwd_gram_kernel(BwdArgs a) {
  constexpr int P = D + 8, NT = D / 32;
  constexpr int TPW = NT * NT / kBwdWaves > 0 ? NT * NT / kBwdWaves : 1;   // output tiles per wave
  const int s = blockIdx.x, bh = blockIdx.y;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const bf16* X = static_cast<const bf16*>(RETR ? a.q : a.k);
  const bf16* Y = static_cast<const bf16*>(a.dout);
  __shared__ __attribute__((aligned(16))) bf16 xs[kChunk * P];
  __shared__ __attribute__((aligned(16))) bf16 ys[kChunk * P];
  __shared__ float zsh[D], ush[D], wsh[kChunk], dsh[kChunk];
  const int64_t seg = (int64_t)bh * a.S + s;
  float* out = (RETR ? a.dMr : a.Amat) + seg * D * D;
  if (!RETR && a.seg_base + s == 0) {
    for (int i = t; i < D * D; i += 64 * kBwdWaves) out[i] = 0.f;
    return;
  }
  if (t < D) {
    zsh[t] = RETR ? 0.f : a.snapz[seg * D + t];
    ush[t] = 0.f;
  }
  f32x16 acc[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) acc[i] = zero16();
  float wsum = 0.f, upart = 0.f, zpart = 0.f;
  const int64_t seg0 = (int64_t)bh * a.L + (int64_t)s * a.N;
  const int tt = t >> 2, qq = t & 3;   // staging: token tt, quarter qq of its row
  constexpr int QW = D / 4;
  __syncthreads();
  for (int t0 = 0; t0 < a.N; t0 += kChunk) {
    const int64_t row = seg0 + t0 + tt;
    float xv[QW];
    float e = 0.f;
#pragma unroll
    for (int i = 0; i < QW / 8; ++i) {
      const bf16x8 x = *reinterpret_cast<const bf16x8*>(X + row * D + qq * QW + 8 * i);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float v = bf2f(x[j]);
        const float f = v > 0.f ? v : exp_e(v) - 1.f;
        xv[8 * i + j] = f;
        if (!RETR) e = __builtin_fmaf(f + 1.f, zsh[qq * QW + 8 * i + j], e);
      }
    }
    float wt;
    if (RETR) {
      wt = a.rs[row];
    } else {
      e += __shfl_xor(e, 1);
      e += __shfl_xor(e, 2);
      wt = e > 0.f ? 1.f / e : 0.f;
    }
#pragma unroll
    for (int i = 0; i < QW / 8; ++i) {
      bf16x8 xb, yb;
      if (RETR) {
        const bf16x8 y = *reinterpret_cast<const bf16x8*>(Y + row * D + qq * QW + 8 * i);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          xb[j] = f2bf(xv[8 * i + j]);
          yb[j] = f2bf(wt * bf2f(y[j]));
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          xb[j] = f2bf(xv[8 * i + j]);
          yb[j] = f2bf(wt * xv[8 * i + j]);
        }
      }
      *reinterpret_cast<bf16x8*>(xs + tt * P + qq * QW + 8 * i) = xb;
      *reinterpret_cast<bf16x8*>(ys + tt * P + qq * QW + 8 * i) = yb;
    }
    if (qq == 0) {
      wsh[tt] = wt;
      if (RETR) dsh[tt] = a.dden[row];
    }
    __syncthreads();
    if (t < D) {
      if (RETR) {
        // fp32 column sums from the inputs: sum_t rs_t dA_t and sum_t dden_t sigma(q_t)
        for (int r = 0; r < kChunk; ++r) {
          const int64_t rr = seg0 + t0 + r;
          upart = __builtin_fmaf(wsh[r], bf2f(Y[rr * D + t]), upart);
          const float q = bf2f(X[rr * D + t]);
          zpart = __builtin_fmaf(dsh[r], q > 0.f ? q + 1.f : exp_e(q), zpart);
        }
      } else {
        for (int r = 0; r < kChunk; ++r) upart = __builtin_fmaf(wsh[r], bf2f(xs[r * P + t]), upart);
      }
    }
    if (!RETR && t == 0)
      for (int r = 0; r < kChunk; ++r) wsum += wsh[r];
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int tile = w * TPW + i, bi = tile / NT, bj = tile % NT;
#pragma unroll
      for (int ks = 0; ks < kChunk / 16; ++ks)
        acc[i] = mfma32(tr_nat(xs, P, 16 * ks, 32 * bi, lane), tr_nat(ys, P, 16 * ks, 32 * bj, lane), acc[i]);
    }
    __syncthreads();
  }
  if (t < D) ush[t] = upart;
  if (t == 0) wsh[0] = wsum;
  if (RETR && t < D) a.dzr[seg * D + t] = zpart;
  __syncthreads();
  const float ws = wsh[0];
  const int l32 = lane & 31, hh = lane >> 5;
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int tile = w * TPW + i, bi = tile / NT, bj = tile % NT;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int x = 32 * bi + acc_row(r, hh), y = 32 * bj + l32;
      out[x * D + y] = RETR ? acc[i][r] + ush[y] : acc[i][r] + ws + ush[x] + ush[y];
    }
  }
}

// Delta rule, per 128 tokens of a segment (one wave per 32, lanes = tokens),
// given G = dL/dM_s (in dMr after the backward chain), M_{s-1}, z_{s-1}:
//   dU = sigma(K) G,  R = sigma(K) M_{s-1} / e (0 in the first segment),
//   U = V - R;  dv += dU;  d sigma(K) = U G^T - M_{s-1} (dU / e)^T;
//   de_t = <dU_t, R_t> / e_t  (the gradient of the token's denominator).
// Transposed products (d_value x tokens) keep every register operand in the
// accumulator layout of the product that consumes it.
template <int D>
__global__ __launch_bounds__(64 * kBwdWaves) void bwd_delta_update_mfma_kernel(BwdArgs a) {
  constexpr int P = D + 8, KS = D / 16, DB = D / 32;
  const int rb = blockIdx.x, s = blockIdx.y, bh = blockIdx.z;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, l32 = lane & 31, hh = lane >> 5;
  const bf16* K = static_cast<const bf16*>(a.k);
  const bf16* V = static_cast<const bf16*>(a.v);
  __shared__ __attribute__((aligned(16))) bf16 gs[D * P];
  __shared__ __attribute__((aligned(16))) bf16 msb[D * P];
  __shared__ float gsum[D], msum[D], zsh[D], ctmp[128], ctmp2[128];
  const int64_t seg = (int64_t)bh * a.S + s;
  const float* Gg = a.dMr + seg * D * D;
  const float* Mg = a.snapM + seg * D * D;
  for (int x = threadIdx.x; x < D * D; x += 64 * kBwdWaves) {
    gs[(x / D) * P + x % D] = f2bf(Gg[x]);
    msb[(x / D) * P + x % D] = f2bf(Mg[x]);
  }
  if (threadIdx.x < D) zsh[threadIdx.x] = a.snapz[seg * D + threadIdx.x];
  block_colsum256(Gg, D, D, gsum, ctmp);
  block_colsum256(Mg, D, D, msum, ctmp2);
  const bool first = a.seg_base + s == 0;
  const int t0 = rb * kBwdBlock + 32 * w;
  const bool valid = t0 < a.N;
  const int64_t row = (int64_t)bh * a.L + (int64_t)s * a.N + min(t0 + l32, a.N - 1);
  __syncthreads();
  bf16x8 kp[KS];
  float e = 0.f;
#pragma unroll
  for (int c = 0; c < KS; ++c) {
    const bf16x8 kx = *reinterpret_cast<const bf16x8*>(K + row * D + 16 * c + 8 * hh);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float x = bf2f(kx[j]);
      const float f = x > 0.f ? x : exp_e(x) - 1.f;
      kp[c][j] = f2bf(f);
      e = __builtin_fmaf(f + 1.f, zsh[16 * c + 8 * hh + j], e);
    }
  }
  e += __shfl_xor(e, 32);
  const float wt = (!first && e > 0.f) ? 1.f / e : 0.f;
  if (!valid) return;
  // dU^T, R^T, U^T per 32-row tile of d_value; B operands for d sigma(K)^T
  bf16x8 ub[DB][2], db[DB][2];
  float de = 0.f;
#pragma unroll
  for (int d = 0; d < DB; ++d) {
    f32x16 du = zero16(), re = zero16();
#pragma unroll
    for (int c = 0; c < KS; ++c) {
      du = mfma32(tr_nat(gs, P, 16 * c, 32 * d, lane), kp[c], du);
      if (!first) re = mfma32(tr_nat(msb, P, 16 * c, 32 * d, lane), kp[c], re);
    }
    f32x16 u, dw;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int col = 32 * d + acc_row(r, hh);
      const float dut = du[r] + gsum[col];
      const float R = first ? 0.f : (re[r] + msum[col]) * wt;
      a.dv_acc[row * D + col] += dut;
      u[r] = bf2f(V[row * D + col]) - R;
      dw[r] = -dut * wt;
      de = __builtin_fmaf(dut, R, de);
    }
    ub[d][0] = acc_op(u, 0);
    ub[d][1] = acc_op(u, 1);
    db[d][0] = acc_op(dw, 0);
    db[d][1] = acc_op(dw, 1);
  }
  de = (de + __shfl_xor(de, 32)) * wt;
  if (hh == 0) a.de[row] = de;
  // d sigma(K)^T = G U^T - M (dU w)^T: A operands are rows of G and M read at the
  // accumulator's row order (two 4-element pieces per lane)
#pragma unroll
  for (int d2 = 0; d2 < DB; ++d2) {
    f32x16 df = zero16();
    const int xr = 32 * d2 + l32;
#pragma unroll
    for (int d = 0; d < DB; ++d)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int c0 = 32 * d + 16 * ks + 4 * hh;
        bf16x8 ga, ma;
        const bf16x4 g0 = *reinterpret_cast<const bf16x4*>(gs + xr * P + c0);
        const bf16x4 g1 = *reinterpret_cast<const bf16x4*>(gs + xr * P + c0 + 8);
        const bf16x4 m0 = *reinterpret_cast<const bf16x4*>(msb + xr * P + c0);
        const bf16x4 m1 = *reinterpret_cast<const bf16x4*>(msb + xr * P + c0 + 8);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          ga[j] = g0[j];
          ga[4 + j] = g1[j];
          ma[j] = m0[j];
          ma[4 + j] = m1[j];
        }
        df = mfma32(ga, ub[d][ks], df);
        if (!first) df = mfma32(ma, db[d][ks], df);
      }
#pragma unroll
    for (int r = 0; r < 16; ++r) a.dfk_acc[row * D + 32 * d2 + acc_row(r, hh)] = df[r];
  }
}

int bwd_mfma_blocks(int N) { return (N + kBwdBlock - 1) / kBwdBlock; }

template <int D>
hipError_t launch_backward_attention_mfma(const BwdArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)bwd_mfma_blocks(a.N), (unsigned)a.S, (unsigned)a.BH);
  hipLaunchKernelGGL(bwd_q_mfma_kernel<D>, grid, dim3(64 * kBwdWaves), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_kv_mfma_kernel<D>, grid, dim3(64 * kBwdWaves), 0, stream, a);
  return hipGetLastError();
}
template hipError_t launch_backward_attention_mfma<64>(const BwdArgs&, hipStream_t);
template hipError_t launch_backward_attention_mfma<128>(const BwdArgs&, hipStream_t);

template <int D>
hipError_t launch_backward_lin_update_mfma(const BwdArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)bwd_mfma_blocks(a.N), (unsigned)a.S, (unsigned)a.BH);
  hipLaunchKernelGGL(bwd_lin_update_mfma_kernel<D>, grid, dim3(64 * kBwdWaves), 0, stream, a);
  return hipGetLastError();
}
template hipError_t launch_backward_lin_update_mfma<64>(const BwdArgs&, hipStream_t);
template hipError_t launch_backward_lin_update_mfma<128>(const BwdArgs&, hipStream_t);

template <int D>
hipError_t launch_backward_delta_amat_mfma(const BwdArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((bwd_gram_kernel<D, false>), dim3((unsigned)a.S, (unsigned)a.BH), dim3(64 * kBwdWaves), 0, stream,
                     a);
  return hipGetLastError();
}
template <int D>
hipError_t launch_backward_delta_update_mfma(const BwdArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)bwd_mfma_blocks(a.N), (unsigned)a.S, (unsigned)a.BH);
  hipLaunchKernelGGL(bwd_delta_update_mfma_kernel<D>, grid, dim3(64 * kBwdWaves), 0, stream, a);
  return hipGetLastError();
}
template <int D>
hipError_t launch_backward_retrieval_grad_mfma(const BwdArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((bwd_gram_kernel<D, true>), dim3((unsigned)a.S, (unsigned)a.BH), dim3(64 * kBwdWaves), 0,
                     stream, a);
  return hipGetLastError();
}
template hipError_t launch_backward_retrieval_grad_mfma<64>(const BwdArgs&, hipStream_t);
template hipError_t launch_backward_retrieval_grad_mfma<128>(const BwdArgs&, hipStream_t);
template hipError_t launch_backward_delta_amat_mfma<64>(const BwdArgs&, hipStream_t);
template hipError_t launch_backward_delta_amat_mfma<128>(const BwdArgs&, hipStream_t);
template hipError_t launch_backward_delta_update_mfma<64>(const BwdArgs&, hipStream_t);
template hipError_t launch_backward_delta_update_mfma<128>(const BwdArgs&, hipStream_t);

}  // namespace infini
