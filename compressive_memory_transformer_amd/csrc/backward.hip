// Gradients of the segment stream (training through the layer: close-reading
// page "精读笔记：Infini-attention", section 4).  The pages print no backward
// formulas; every kernel below applies the chain rule to the forward equations
// (section 3.1 with the causal mask of section 3.8 step 2 for A_dot, 3.3 for
// A_mem, 3.5 for the gate, 3.4 and the CSDN page's section 2.1 for the linear and
// delta updates).  For the loss <dA, A> + <dM, M_S> + <dz, z_S>:
//
//   snap        delta rule, fp32 path: replays the memory updates and keeps every
//               M_{s-1}, z_{s-1} (fp32);
//   query       (fp32 path) per 32 query rows of a segment: the row's softmax statistics and
//               A_dot (first sweep over the keys), A_mem, the gate's share of
//               dbeta, D = <(1 - g) dA, A_dot>, the retrieval's share of dq, then
//               the local attention's share of dq (second sweep);
//   key         (fp32 path) per 32 keys of a segment: the local attention's dk and dv;
//               the bf16 path runs both on the MFMA units (backward_mfma.hip);
//   tall        per segment and 32 columns: the retrieval's gradient of M_{s-1}
//               and z_{s-1}; for the linear rule also the replay's contributions;
//   scan        linear rule: prefix sums of the contributions (the replay) and
//               suffix sums of the retrieval gradients (dL/dM_s);
//   lin_update  linear rule, per 64 tokens: the update's dv and d sigma(K);
//   delta_chain delta rule, bf16 path: the replay and the backward carry of dL/dM_s
//               as d x d x 16 products with A_s (the per-token work on MFMA);
//   chain       delta rule, fp32 path, per 16 columns of M, segments in reverse: dL/dM_s carried back,
//               the update's dv, its d sigma(K) (atomically summed over the column
//               blocks) and, for the delta rule, the gradient of each token's
//               denominator;
//   ez, zchain  dL/dz_s carried back;  finish  the outputs in the input dtype;
//   dbeta       the per-block shares of dbeta summed in a fixed order.
//
// All arithmetic is fp32 on the VALU, tiles staged in LDS.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace infini {

namespace {

constexpr int kThreads = 256;
constexpr int kTok = 64;      // token chunk of the state kernels
constexpr int kColB = 16;     // columns of M per chain / snapshot workgroup
constexpr int kChainCB = 4;   // columns of M per workgroup of the bf16 path's delta chains
constexpr int kQB = 32;       // query rows per query-block workgroup
constexpr int kKC = 64;       // key chunk
constexpr int kKB = 32;       // keys per key-block workgroup
constexpr int kQC = 64;       // query chunk of the key-block kernel
constexpr int kP = 129;       // LDS pitch of 128-wide fp32 rows

__device__ __forceinline__ float ld(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ld(const bf16* p, int64_t i) { return bf2f(p[i]); }
__device__ __forceinline__ void st(float* p, int64_t i, float x) { p[i] = x; }
__device__ __forceinline__ void st(bf16* p, int64_t i, float x) { p[i] = f2bf(x); }

__device__ __forceinline__ float sig(float x) { return x > 0.f ? x + 1.f : exp_e(x); }
__device__ __forceinline__ float sig_prime(float x) { return x > 0.f ? 1.f : exp_e(x); }

// Sum over the 8 consecutive lanes that share a row.
__device__ __forceinline__ float row8_sum(float x) {
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  x += __shfl_xor(x, 4);
  return x;
}
__device__ __forceinline__ float row8_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 1));
  x = fmaxf(x, __shfl_xor(x, 2));
  x = fmaxf(x, __shfl_xor(x, 4));
  return x;
}

__device__ __forceinline__ bool is_first(const BwdArgs& a, int s) { return a.seg_base + s == 0; }

}  // namespace

// ------------------------------------------------------------------ snap
// grid (column blocks, BH).  Replays the updates of the stream for 16 columns
// of M and writes M_{s-1}[:, cols] (and, from column block 0, z_{s-1}) for
// every segment s.
template <typename T>
__global__ __launch_bounds__(kThreads) void bwd_snap_kernel(BwdArgs a) {
  const int cb = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
  const T* K = static_cast<const T*>(a.k);
  const T* V = static_cast<const T*>(a.v);
  __shared__ float Ms[128][kColB + 1];
  __shared__ float zs[128];
  __shared__ float fk[kTok][kP];
  __shared__ float uu[kTok][kColB + 1];
  __shared__ float ee[kTok];
  for (int i = t; i < 128 * kColB; i += kThreads) {
    const int r = i / kColB, c = i % kColB, col = cb * kColB + c;
    Ms[r][c] = (r < a.dk && col < a.dv) ? a.M0[((int64_t)bh * a.dk + r) * a.dv + col] : 0.f;
  }
  if (t < 128) zs[t] = t < a.dk ? a.z0[(int64_t)bh * a.dk + t] : 0.f;
  __syncthreads();
  for (int s = 0; s < a.S; ++s) {
    const bool hasd = a.delta && !is_first(a, s);
    float* snap = a.snapM + ((int64_t)bh * a.S + s) * a.dk * a.dv;
    for (int i = t; i < a.dk * kColB; i += kThreads) {
      const int r = i / kColB, c = i % kColB, col = cb * kColB + c;
      if (col < a.dv) snap[(int64_t)r * a.dv + col] = Ms[r][c];
    }
    if (cb == 0 && t < a.dk) a.snapz[((int64_t)bh * a.S + s) * a.dk + t] = zs[t];
    float dM[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float zacc = 0.f;
    for (int t0 = 0; t0 < a.N; t0 += kTok) {
      const int64_t row0 = (int64_t)bh * a.L + (int64_t)s * a.N + t0;
      for (int i = t; i < kTok * 128; i += kThreads) {
        const int r = i >> 7, c = i & 127;
        fk[r][c] = (t0 + r < a.N && c < a.dk) ? sig(ld(K, (row0 + r) * a.dk + c)) : 0.f;
      }
      for (int i = t; i < kTok * kColB; i += kThreads) {
        const int r = i / kColB, c = i % kColB, col = cb * kColB + c;
        uu[r][c] = (t0 + r < a.N && col < a.dv) ? ld(V, (row0 + r) * a.dv + col) : 0.f;
      }
      __syncthreads();
      if (hasd) {
        if (t < kTok) {
          float e = 0.f;
          for (int c = 0; c < a.dk; ++c) e = __builtin_fmaf(fk[t][c], zs[c], e);
          ee[t] = e;
        }
        __syncthreads();
        float u[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = t + kThreads * r, tt = i / kColB, c = i % kColB;
          float num = 0.f;
          for (int x = 0; x < a.dk; ++x) num = __builtin_fmaf(fk[tt][x], Ms[x][c], num);
          u[r] = uu[tt][c] - (ee[tt] > 0.f ? num / ee[tt] : 0.f);
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = t + kThreads * r;
          uu[i / kColB][i % kColB] = u[r];
        }
        __syncthreads();
      }
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int i = t + kThreads * r, x = i / kColB, c = i % kColB;
        float acc = dM[r];
        for (int tt = 0; tt < kTok; ++tt) acc = __builtin_fmaf(fk[tt][x], uu[tt][c], acc);
        dM[r] = acc;
      }
      if (t < 128)
        for (int tt = 0; tt < kTok; ++tt) zacc += fk[tt][t];
      __syncthreads();
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int i = t + kThreads * r;
      Ms[i / kColB][i % kColB] += dM[r];
    }
    if (t < 128) zs[t] += zacc;
    __syncthreads();
  }
}

// ----------------------------------------------------------------- query
// grid (query blocks of 32, S, BH).  Thread = (row i = t / 8, part p = t % 8).
template <typename T>
__global__ __launch_bounds__(kThreads) void bwd_query_kernel(BwdArgs a) {
  const int qb = blockIdx.x, s = blockIdx.y, bh = blockIdx.z, h = bh % a.H, t = threadIdx.x;
  const int i = t >> 3, p = t & 7;
  const T* Q = static_cast<const T*>(a.q);
  const T* K = static_cast<const T*>(a.k);
  const T* V = static_cast<const T*>(a.v);
  const T* DO = static_cast<const T*>(a.dout);
  __shared__ float qs[kQB][kP];
  __shared__ float das[kQB][kP];
  __shared__ float kv[2 * kKC * kP];   // key / value chunk; later M_{s-1}
  __shared__ float ps[kQB][kKC + 1];
  __shared__ float dn[kQB][kP];
  __shared__ float zsh[128];
  __shared__ float red[kThreads / 64];
  float (*ks)[kP] = reinterpret_cast<float (*)[kP]>(kv);
  float (*vs)[kP] = reinterpret_cast<float (*)[kP]>(kv + kKC * kP);

  const int i0 = qb * kQB;
  const int qi = i0 + i;                          // row in the segment
  const bool valid = qi < a.N;
  const int64_t seg0 = (int64_t)bh * a.L + (int64_t)s * a.N;
  const float g = sigmoid_gate(a.beta[h]);
  const bool first = is_first(a, s);
  for (int x = t; x < kQB * 128; x += kThreads) {
    const int r = x >> 7, c = x & 127;
    const bool ok = i0 + r < a.N;
    qs[r][c] = (ok && c < a.dk) ? ld(Q, (seg0 + i0 + r) * a.dk + c) : 0.f;
    das[r][c] = (ok && c < a.dv) ? ld(DO, (seg0 + i0 + r) * a.dv + c) : 0.f;
  }
  const int kend = min(a.N, i0 + kQB);            // keys any row of the block sees

  // first sweep: softmax statistics and A_dot (columns c = 16 p + e)
  float m = -__builtin_inff(), l = 0.f, o[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) o[e] = 0.f;
  for (int kc = 0; kc < kend; kc += kKC) {
    __syncthreads();
    for (int x = t; x < kKC * 128; x += kThreads) {
      const int r = x >> 7, c = x & 127;
      const bool ok = kc + r < kend;
      ks[r][c] = (ok && c < a.dk) ? ld(K, (seg0 + kc + r) * a.dk + c) : 0.f;
      vs[r][c] = (ok && c < a.dv) ? ld(V, (seg0 + kc + r) * a.dv + c) : 0.f;
    }
    __syncthreads();
    float sc[8], cmax = -__builtin_inff();
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = p + 8 * u;
      float d = 0.f;
      for (int c = 0; c < a.dk; ++c) d = __builtin_fmaf(qs[i][c], ks[j][c], d);
      sc[u] = (valid && kc + j <= qi) ? d * a.scale : -__builtin_inff();
      cmax = fmaxf(cmax, sc[u]);
    }
    cmax = row8_max(cmax);
    const float mn = fmaxf(m, cmax);
    const float alpha = mn == -__builtin_inff() ? 1.f : exp_e(m - mn);
    float lsum = 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float pe = sc[u] == -__builtin_inff() ? 0.f : exp_e(sc[u] - mn);
      ps[i][p + 8 * u] = pe;
      lsum += pe;
    }
    l = l * alpha + row8_sum(lsum);
    m = mn;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int c = 16 * p + e;
      float acc = o[e] * alpha;
      if (c < a.dv)
        for (int j = 0; j < kKC; ++j) acc = __builtin_fmaf(ps[i][j], vs[j][c], acc);
      o[e] = acc;
    }
  }
  const float lse = valid ? m + __logf(l) : 0.f;
  const float inv_l = valid ? 1.f / l : 0.f;

  // retrieval from M_{s-1}, z_{s-1}; the gate; D; the retrieval's dq
  __syncthreads();
  const float* Mg = a.snapM + ((int64_t)bh * a.S + s) * a.dk * a.dv;
  for (int x = t; x < a.dk * a.dv; x += kThreads) kv[x] = Mg[x];
  if (t < 128) zsh[t] = t < a.dk ? a.snapz[((int64_t)bh * a.S + s) * a.dk + t] : 0.f;
  __syncthreads();
  float num[16], dpart = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) num[e] = 0.f;
  for (int x = 0; x < a.dk; ++x) {
    const float f = sig(qs[i][x]);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int c = 16 * p + e;
      if (c < a.dv) num[e] = __builtin_fmaf(f, kv[x * a.dv + c], num[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int x = 16 * p + e;
    if (x < a.dk) dpart = __builtin_fmaf(sig(qs[i][x]), zsh[x], dpart);
  }
  const float den = row8_sum(dpart);
  const bool has = valid && !first && den > 0.f;
  float dsum = 0.f, bsum = 0.f, msum = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int c = 16 * p + e;
    if (c < a.dv) {
      const float adot = o[e] * inv_l;
      const float amem = has ? num[e] / den : 0.f;
      const float d = das[i][c];
      dsum = __builtin_fmaf(d, adot, dsum);
      bsum = __builtin_fmaf(d, amem - adot, bsum);
      msum = __builtin_fmaf(d, amem, msum);
    }
  }
  const float D = (1.f - g) * row8_sum(dsum);
  const float rs = has ? g / den : 0.f;
  const float msum_row = row8_sum(msum);
  const float dden = has ? -g * msum_row / den : 0.f;
  bsum = valid ? bsum : 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int c = 16 * p + e;
    if (c < 128) dn[i][c] = rs * das[i][c];
  }
  if (valid && p == 0) {
    const int64_t row = seg0 + qi;
    a.lse[row] = lse;
    a.drow[row] = D;
    a.rs[row] = rs;
    a.dden[row] = dden;
  }
  // dbeta share of the block: g (1 - g) sum dA (A_mem - A_dot)
  float bt = wave_sum(bsum);
  if ((t & 63) == 0) red[t >> 6] = bt;
  __syncthreads();
  if (t == 0) {
    float b = 0.f;
    for (int w = 0; w < kThreads / 64; ++w) b += red[w];
    a.dbeta_part[((int64_t)bh * a.S + s) * a.nqb + qb] = b * g * (1.f - g);
  }
  float dq[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int x = 16 * p + e;
    float acc = 0.f;
    if (x < a.dk) {
      for (int c = 0; c < a.dv; ++c) acc = __builtin_fmaf(kv[x * a.dv + c], dn[i][c], acc);
      acc = (acc + dden * zsh[x]) * sig_prime(qs[i][x]);
    }
    dq[e] = acc;
  }

  // second sweep: the local attention's dq = scale sum_j dS_ij k_j
  for (int kc = 0; kc < kend; kc += kKC) {
    __syncthreads();
    for (int x = t; x < kKC * 128; x += kThreads) {
      const int r = x >> 7, c = x & 127;
      const bool ok = kc + r < kend;
      ks[r][c] = (ok && c < a.dk) ? ld(K, (seg0 + kc + r) * a.dk + c) : 0.f;
      vs[r][c] = (ok && c < a.dv) ? ld(V, (seg0 + kc + r) * a.dv + c) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = p + 8 * u;
      float ds = 0.f;
      if (valid && kc + j <= qi) {
        float d = 0.f, dp = 0.f;
        for (int c = 0; c < a.dk; ++c) d = __builtin_fmaf(qs[i][c], ks[j][c], d);
        for (int c = 0; c < a.dv; ++c) dp = __builtin_fmaf(das[i][c], vs[j][c], dp);
        const float pe = exp_e(d * a.scale - lse);
        ds = pe * ((1.f - g) * dp - D);
      }
      ps[i][j] = ds;
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int x = 16 * p + e;
      if (x < a.dk) {
        float acc = 0.f;
        for (int j = 0; j < kKC; ++j) acc = __builtin_fmaf(ps[i][j], ks[j][x], acc);
        dq[e] = __builtin_fmaf(a.scale, acc, dq[e]);
      }
    }
  }
  if (valid) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int x = 16 * p + e;
      if (x < a.dk) a.dq_acc[(seg0 + qi) * a.dk + x] = dq[e];
    }
  }
}

// ------------------------------------------------------------------- key
// grid (key blocks of 32, S, BH).  Thread = (key j = t / 8, part p = t % 8).
template <typename T>
__global__ __launch_bounds__(kThreads) void bwd_key_kernel(BwdArgs a) {
  const int kb = blockIdx.x, s = blockIdx.y, bh = blockIdx.z, h = bh % a.H, t = threadIdx.x;
  const int j = t >> 3, p = t & 7;
  const T* Q = static_cast<const T*>(a.q);
  const T* K = static_cast<const T*>(a.k);
  const T* V = static_cast<const T*>(a.v);
  const T* DO = static_cast<const T*>(a.dout);
  __shared__ float kbs[kKB][kP];
  __shared__ float vbs[kKB][kP];
  __shared__ float qc[kQC][kP];
  __shared__ float dac[kQC][kP];
  __shared__ float lc[kQC], dc[kQC];
  __shared__ float pss[kKB][kQC + 1];
  __shared__ float dss[kKB][kQC + 1];
  const int j0 = kb * kKB, kj = j0 + j;
  const bool valid = kj < a.N;
  const int64_t seg0 = (int64_t)bh * a.L + (int64_t)s * a.N;
  const float g = sigmoid_gate(a.beta[h]);
  for (int x = t; x < kKB * 128; x += kThreads) {
    const int r = x >> 7, c = x & 127;
    const bool ok = j0 + r < a.N;
    kbs[r][c] = (ok && c < a.dk) ? ld(K, (seg0 + j0 + r) * a.dk + c) : 0.f;
    vbs[r][c] = (ok && c < a.dv) ? ld(V, (seg0 + j0 + r) * a.dv + c) : 0.f;
  }
  float dkv[16], dvv[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) dkv[e] = dvv[e] = 0.f;
  for (int qc0 = j0; qc0 < a.N; qc0 += kQC) {
    __syncthreads();
    for (int x = t; x < kQC * 128; x += kThreads) {
      const int r = x >> 7, c = x & 127;
      const bool ok = qc0 + r < a.N;
      qc[r][c] = (ok && c < a.dk) ? ld(Q, (seg0 + qc0 + r) * a.dk + c) : 0.f;
      dac[r][c] = (ok && c < a.dv) ? ld(DO, (seg0 + qc0 + r) * a.dv + c) : 0.f;
    }
    if (t < kQC) {
      const bool ok = qc0 + t < a.N;
      lc[t] = ok ? a.lse[seg0 + qc0 + t] : 0.f;
      dc[t] = ok ? a.drow[seg0 + qc0 + t] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int ii = p + 8 * u, qi = qc0 + ii;
      float pe = 0.f, ds = 0.f;
      if (valid && qi < a.N && kj <= qi) {
        float d = 0.f, dp = 0.f;
        for (int c = 0; c < a.dk; ++c) d = __builtin_fmaf(qc[ii][c], kbs[j][c], d);
        for (int c = 0; c < a.dv; ++c) dp = __builtin_fmaf(dac[ii][c], vbs[j][c], dp);
        pe = exp_e(d * a.scale - lc[ii]);
        ds = pe * ((1.f - g) * dp - dc[ii]);
      }
      pss[j][ii] = pe;
      dss[j][ii] = ds;
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int c = 16 * p + e;
      float av = dvv[e], ak = dkv[e];
      for (int ii = 0; ii < kQC; ++ii) {
        av = __builtin_fmaf(pss[j][ii], dac[ii][c], av);
        ak = __builtin_fmaf(dss[j][ii], qc[ii][c], ak);
      }
      dvv[e] = av;
      dkv[e] = ak;
    }
  }
  if (valid) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int c = 16 * p + e;
      if (c < a.dv) a.dv_acc[(seg0 + kj) * a.dv + c] = (1.f - g) * dvv[e];
      if (c < a.dk) a.dk_acc[(seg0 + kj) * a.dk + c] = a.scale * dkv[e];
    }
  }
}

// ----------------------------------------------------------------- chain
// grid (column blocks, BH).  dL/dM_s for 16 columns carried from the last
// segment to the first.
template <typename T>
__global__ __launch_bounds__(kThreads) void bwd_chain_kernel(BwdArgs a) {
  const int cb = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
  const T* K = static_cast<const T*>(a.k);
  const T* V = static_cast<const T*>(a.v);
  __shared__ float GMs[128][kColB + 1];
  __shared__ float Ms[128][kColB + 1];
  __shared__ float zs[128];
  __shared__ float fk[kTok][kP];
  __shared__ float du[kTok][kColB + 1];
  __shared__ float rr[kTok][kColB + 1];
  __shared__ float uu[kTok][kColB + 1];
  __shared__ float ee[kTok];
  for (int i = t; i < 128 * kColB; i += kThreads) {
    const int r = i / kColB, c = i % kColB, col = cb * kColB + c;
    GMs[r][c] = (a.dM && r < a.dk && col < a.dv) ? a.dM[((int64_t)bh * a.dk + r) * a.dv + col] : 0.f;
  }
  for (int s = a.S - 1; s >= 0; --s) {
    const bool hasd = a.delta && !is_first(a, s);
    const float* snap = a.snapM + ((int64_t)bh * a.S + s) * a.dk * a.dv;
    __syncthreads();
    for (int i = t; i < 128 * kColB; i += kThreads) {
      const int r = i / kColB, c = i % kColB, col = cb * kColB + c;
      Ms[r][c] = (r < a.dk && col < a.dv) ? snap[(int64_t)r * a.dv + col] : 0.f;
    }
    if (t < 128) zs[t] = t < a.dk ? a.snapz[((int64_t)bh * a.S + s) * a.dk + t] : 0.f;
    float gacc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int t0 = 0; t0 < a.N; t0 += kTok) {
      const int64_t row0 = (int64_t)bh * a.L + (int64_t)s * a.N + t0;
      __syncthreads();
      for (int i = t; i < kTok * 128; i += kThreads) {
        const int r = i >> 7, c = i & 127;
        fk[r][c] = (t0 + r < a.N && c < a.dk) ? sig(ld(K, (row0 + r) * a.dk + c)) : 0.f;
      }
      __syncthreads();
      if (t < kTok) {
        float e = 0.f;
        if (hasd)
          for (int c = 0; c < a.dk; ++c) e = __builtin_fmaf(fk[t][c], zs[c], e);
        ee[t] = e;
      }
      __syncthreads();
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = t + kThreads * r, tt = i / kColB, c = i % kColB, col = cb * kColB + c;
        const bool ok = t0 + tt < a.N && col < a.dv;
        float d = 0.f, R = 0.f;
        for (int x = 0; x < a.dk; ++x) d = __builtin_fmaf(fk[tt][x], GMs[x][c], d);
        if (hasd && ee[tt] > 0.f) {
          float n = 0.f;
          for (int x = 0; x < a.dk; ++x) n = __builtin_fmaf(fk[tt][x], Ms[x][c], n);
          R = n / ee[tt];
        }
        const float vv = ok ? ld(V, (row0 + tt) * a.dv + col) : 0.f;
        du[tt][c] = ok ? d : 0.f;
        rr[tt][c] = ok ? R : 0.f;
        uu[tt][c] = ok ? vv - R : 0.f;
        if (ok) a.dv_acc[(row0 + tt) * a.dv + col] += d;
      }
      __syncthreads();
      // d sigma(K) share of these columns: U GM^T (+ M dr for the delta rule)
      for (int r = 0; r < kTok * 128 / kThreads; ++r) {
        const int i = t + kThreads * r, tt = i >> 7, x = i & 127;
        if (t0 + tt >= a.N || x >= a.dk) continue;
        float val = 0.f;
#pragma unroll
        for (int c = 0; c < kColB; ++c) val = __builtin_fmaf(uu[tt][c], GMs[x][c], val);
        if (hasd && ee[tt] > 0.f) {
          const float ie = 1.f / ee[tt];
          float mdr = 0.f;
#pragma unroll
          for (int c = 0; c < kColB; ++c) mdr = __builtin_fmaf(Ms[x][c], du[tt][c], mdr);
          val -= mdr * ie;
        }
        atomicAdd(&a.dfk_acc[(row0 + tt) * a.dk + x], val);
      }
      if (hasd && t < kTok && t0 + t < a.N && ee[t] > 0.f) {
        float sde = 0.f;
#pragma unroll
        for (int c = 0; c < kColB; ++c) sde = __builtin_fmaf(du[t][c], rr[t][c], sde);
        atomicAdd(&a.de[row0 + t], sde / ee[t]);
      }
      if (hasd) {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int i = t + kThreads * r, x = i / kColB, c = i % kColB;
          float acc = gacc[r];
          for (int tt = 0; tt < kTok; ++tt)
            if (ee[tt] > 0.f) acc -= fk[tt][x] * du[tt][c] / ee[tt];
          gacc[r] = acc;
        }
      }
    }
    __syncthreads();
    const float* dmr = a.dMr + ((int64_t)bh * a.S + s) * a.dk * a.dv;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int i = t + kThreads * r, x = i / kColB, c = i % kColB, col = cb * kColB + c;
      if (x < a.dk && col < a.dv) GMs[x][c] += gacc[r] + dmr[(int64_t)x * a.dv + col];
    }
  }
  __syncthreads();
  if (a.dM0)
    for (int i = t; i < a.dk * kColB; i += kThreads) {
      const int r = i / kColB, c = i % kColB, col = cb * kColB + c;
      if (col < a.dv) a.dM0[((int64_t)bh * a.dk + r) * a.dv + col] = GMs[r][c];
    }
}

// -------------------------------------------------------- ez and zchain
// grid (S, BH), 128 threads: ez_s = sum_t de_t sigma(K_t) (delta rule, not the
// stream's first segment).
template <typename T>
__global__ __launch_bounds__(kThreads) void bwd_ez_kernel(BwdArgs a) {
  const int s = blockIdx.x, bh = blockIdx.y, t = threadIdx.x, x = t & 127, half = t >> 7;
  const T* K = static_cast<const T*>(a.k);
  __shared__ float part[128];
  const int64_t seg0 = (int64_t)bh * a.L + (int64_t)s * a.N;
  float acc = 0.f;
  if (a.delta && !is_first(a, s) && x < a.dk) {
    // rows half, half + 2, ...: eight independent partial sums keep the loads in flight
    float p[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int r = half;
    for (; r + 14 < a.N; r += 16)
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t row = seg0 + r + 2 * u;
        p[u] = __builtin_fmaf(a.de[row], sig(ld(K, row * a.dk + x)), p[u]);
      }
    for (; r < a.N; r += 2) p[0] = __builtin_fmaf(a.de[seg0 + r], sig(ld(K, (seg0 + r) * a.dk + x)), p[0]);
    acc = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
  }
  if (half == 1) part[x] = acc;
  __syncthreads();
  if (half == 0 && x < a.dk) a.ez[((int64_t)bh * a.S + s) * a.dk + x] = acc + part[x];
}

// bf16 keys, d_key = D in {64, 128}: the same sums with 16-byte key loads; thread
// t takes columns 8 (t % (D / 8)) .. + 7 of rows t / (D / 8) + G i (G row groups,
// four rows in flight), and the groups meet in LDS.
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_ez_vec_kernel(BwdArgs a) {
  constexpr int C8 = D / 8, G = kThreads / C8;
  const int s = blockIdx.x, bh = blockIdx.y, t = threadIdx.x, c8 = t % C8, g = t / C8;
  const bf16* K = static_cast<const bf16*>(a.k);
  __shared__ float red[G * D];
  const int64_t seg0 = (int64_t)bh * a.L + (int64_t)s * a.N;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (!is_first(a, s)) {
    int r = g;
    for (; r + 3 * G < a.N; r += 4 * G) {
      bf16x8 kx[4];
      float dw[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t row = seg0 + r + G * u;
        kx[u] = *reinterpret_cast<const bf16x8*>(K + row * D + 8 * c8);
        dw[u] = a.de[row];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = __builtin_fmaf(dw[u], sig(bf2f(kx[u][j])), acc[j]);
    }
    for (; r < a.N; r += G) {
      const int64_t row = seg0 + r;
      const bf16x8 kx = *reinterpret_cast<const bf16x8*>(K + row * D + 8 * c8);
      const float dw = a.de[row];
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = __builtin_fmaf(dw, sig(bf2f(kx[j])), acc[j]);
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) red[g * D + 8 * c8 + j] = acc[j];
  __syncthreads();
  if (t < D) {
    float sum = 0.f;
    for (int q = 0; q < G; ++q) sum += red[q * D + t];
    a.ez[((int64_t)bh * a.S + s) * D + t] = sum;
  }
}

// grid (BH), 128 threads: gzs_s = dL/dz_s; dz0 = dL/dz_0.
__global__ __launch_bounds__(128) void bwd_zchain_kernel(BwdArgs a) {
  const int bh = blockIdx.x, x = threadIdx.x;
  if (x >= a.dk) return;
  float gz = a.dz ? a.dz[(int64_t)bh * a.dk + x] : 0.f;
  for (int s = a.S - 1; s >= 0; --s) {
    const int64_t i = ((int64_t)bh * a.S + s) * a.dk + x;
    a.gzs[i] = gz;
    gz += a.dzr[i] + (a.delta ? a.ez[i] : 0.f);
  }
  if (a.dz0) a.dz0[(int64_t)bh * a.dk + x] = gz;
}

// ------------------------------------------------------------------ tall
// grid (column blocks of 32, S, BH).  A per-segment product over the segment's
// rows, out_s = X^T Y (d_key x d_value, this block's 32 columns) and, from column
// block 0, the weighted column sums colsum_s = X^T w:
//   MODE 0 (linear rule, replay): X = sigma(K), Y = V, w = 1; written into the
//     snapshot buffers as C_s and c_s, then turned into M_{s-1}, z_{s-1} by the
//     prefix kernel;
//   MODE 1 (both rules): X = sigma(Q), Y = rs dA, w = dden: the retrieval's
//     gradient of M_{s-1} and z_{s-1}.
template <typename T, int MODE>
__global__ __launch_bounds__(kThreads) void bwd_tall_kernel(BwdArgs a) {
  const int cb = blockIdx.x, s = blockIdx.y, bh = blockIdx.z, t = threadIdx.x;
  const T* X = static_cast<const T*>(MODE == 0 ? a.k : a.q);
  const T* Y = static_cast<const T*>(MODE == 0 ? a.v : a.dout);
  __shared__ float xs[32][kP];
  __shared__ float ys[32][33];
  __shared__ float ws[32];
  const int c = t & 31, ah = t >> 5, col = cb * 32 + c;
  const int64_t seg0 = (int64_t)bh * a.L + (int64_t)s * a.N;
  float acc[16];
#pragma unroll
  for (int m = 0; m < 16; ++m) acc[m] = 0.f;
  float zacc = 0.f;
  for (int r0 = 0; r0 < a.N; r0 += 32) {
    __syncthreads();
    for (int x = t; x < 32 * 128; x += kThreads) {
      const int r = x >> 7, cc = x & 127;
      xs[r][cc] = (r0 + r < a.N && cc < a.dk) ? sig(ld(X, (seg0 + r0 + r) * a.dk + cc)) : 0.f;
    }
    for (int x = t; x < 32 * 32; x += kThreads) {
      const int r = x >> 5, cc = x & 31, cl = cb * 32 + cc;
      const int64_t row = seg0 + r0 + r;
      float y = 0.f;
      if (r0 + r < a.N && cl < a.dv) y = MODE == 0 ? ld(Y, row * a.dv + cl) : a.rs[row] * ld(Y, row * a.dv + cl);
      ys[r][cc] = y;
    }
    if (t < 32) ws[t] = r0 + t < a.N ? (MODE == 0 ? 1.f : a.dden[seg0 + r0 + t]) : 0.f;
    __syncthreads();
#pragma unroll 2
    for (int r = 0; r < 32; ++r) {
      const float yv = ys[r][c];
#pragma unroll
      for (int m = 0; m < 16; ++m) acc[m] = __builtin_fmaf(xs[r][ah + 8 * m], yv, acc[m]);
    }
    if (cb == 0 && t < 128)
      for (int r = 0; r < 32; ++r) zacc = __builtin_fmaf(ws[r], xs[r][t], zacc);
  }
  float* out = (MODE == 0 ? a.snapM : a.dMr) + ((int64_t)bh * a.S + s) * a.dk * a.dv;
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    const int x = ah + 8 * m;
    if (x < a.dk && col < a.dv) out[(int64_t)x * a.dv + col] = acc[m];
  }
  if (cb == 0 && t < a.dk) (MODE == 0 ? a.snapz : a.dzr)[((int64_t)bh * a.S + s) * a.dk + t] = zacc;
}

// ----------------------------------------------------------------- scans
// One thread per element of M (and of z): REVERSE = false turns the
// contributions C_s, c_s in snapM / snapz into M_{s-1} = M_0 + sum_{s' < s} C_s'
// (z likewise; with FROM_T the contributions C_s^T come from dMr, the layout
// of the MFMA contribution kernel); REVERSE = true turns the retrieval
// gradients dMr_s into dL/dM_s = dM + sum_{s' > s} dMr_s' and writes dL/dM_0.
template <bool REVERSE, bool FROM_T>
__global__ __launch_bounds__(kThreads) void bwd_scan_kernel(BwdArgs a) {
  const int64_t per = (int64_t)a.dk * a.dv + (REVERSE ? 0 : a.dk);
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= (int64_t)a.BH * per) return;
  const int bh = (int)(i / per);
  const int64_t e = i % per;
  const bool isz = e >= (int64_t)a.dk * a.dv;
  const int64_t ez = e - (int64_t)a.dk * a.dv;
  float* base = REVERSE ? a.dMr : (isz ? a.snapz : a.snapM);
  const int64_t stride = isz ? a.dk : (int64_t)a.dk * a.dv;
  const int64_t off = (int64_t)bh * a.S * stride + (isz ? ez : e);
  float run;
  if (REVERSE) run = a.dM ? a.dM[(int64_t)bh * a.dk * a.dv + e] : 0.f;
  else run = isz ? a.z0[(int64_t)bh * a.dk + ez] : a.M0[(int64_t)bh * a.dk * a.dv + e];
  if (REVERSE) {
    for (int s = a.S - 1; s >= 0; --s) {
      float* p = base + off + (int64_t)s * stride;
      const float c = *p;
      *p = run;
      run += c;
    }
    if (a.dM0) a.dM0[(int64_t)bh * a.dk * a.dv + e] = run;
  } else {
    // element (x, y) of M reads C_s^T[y][x] when the contributions are transposed
    const int64_t et = isz ? 0 : (e % a.dv) * a.dk + e / a.dv;
    for (int s = 0; s < a.S; ++s) {
      float* p = base + off + (int64_t)s * stride;
      const float c = (FROM_T && !isz) ? a.dMr[((int64_t)bh * a.S + s) * stride + et] : *p;
      *p = run;
      run += c;
    }
  }
}

// ------------------------------------------------------------ lin_update
// grid (blocks of 64 tokens, S, BH).  Linear rule, given G = dL/dM_s (in dMr
// after the reverse scan): dv += sigma(K) G and d sigma(K) = V G^T (the z share
// is added by the finish kernel).
template <typename T>
__global__ __launch_bounds__(kThreads) void bwd_lin_update_kernel(BwdArgs a) {
  const int rb = blockIdx.x, s = blockIdx.y, bh = blockIdx.z, t = threadIdx.x;
  const T* K = static_cast<const T*>(a.k);
  const T* V = static_cast<const T*>(a.v);
  __shared__ float G[128 * kP];
  __shared__ float fk[kTok][kP];
  __shared__ float vs[kTok][kP];
  const int64_t row0 = (int64_t)bh * a.L + (int64_t)s * a.N + (int64_t)rb * kTok;
  const int nrow = min(kTok, a.N - rb * kTok);
  const float* Gg = a.dMr + ((int64_t)bh * a.S + s) * a.dk * a.dv;
  for (int x = t; x < a.dk * a.dv; x += kThreads) G[(x / a.dv) * kP + x % a.dv] = Gg[x];
  for (int x = t; x < kTok * 128; x += kThreads) {
    const int r = x >> 7, c = x & 127;
    fk[r][c] = (r < nrow && c < a.dk) ? sig(ld(K, (row0 + r) * a.dk + c)) : 0.f;
    vs[r][c] = (r < nrow && c < a.dv) ? ld(V, (row0 + r) * a.dv + c) : 0.f;
  }
  __syncthreads();
  const int c = t & 127, rh = t >> 7;
  if (c < a.dv) {
    for (int m = 0; m < kTok / 2; ++m) {
      const int r = rh + 2 * m;
      if (r >= nrow) break;
      float acc = 0.f;
      for (int x = 0; x < a.dk; ++x) acc = __builtin_fmaf(fk[r][x], G[x * kP + c], acc);
      a.dv_acc[(row0 + r) * a.dv + c] += acc;
    }
  }
  if (c < a.dk) {
    for (int m = 0; m < kTok / 2; ++m) {
      const int r = rh + 2 * m;
      if (r >= nrow) break;
      float acc = 0.f;
      for (int y = 0; y < a.dv; ++y) acc = __builtin_fmaf(vs[r][y], G[c * kP + y], acc);
      a.dfk_acc[(row0 + r) * a.dk + c] = acc;
    }
  }
}

// ------------------------------------------------------- delta, bf16 path
// With A_s = sigma(K)^T diag(1 / e) sigma(K) (e_t = sigma(K_t) . z_{s-1}; A_s = 0
// in a stream's first segment), the delta update is M_s = (I - A_s) M_{s-1} + C_s
// (C_s = sigma(K)^T V) and its gradient dL/dM_{s-1} = (I - A_s) dL/dM_s + dMr_s
// (A_s is symmetric).  A_s and C_s come from parallel kernels; the two chains
// below carry only a d_key x d_key x 16 product per segment.
// grid (column blocks of CB, BH).  FWD: M_{s-1} snapshots from C_s^T (in dMr).
// !FWD: dMr_s replaced by dL/dM_s, dL/dM_0 to dM0.
template <bool FWD, int CB>
__global__ __launch_bounds__(kThreads) void bwd_delta_chain_kernel(BwdArgs a) {
  constexpr int RPT = 128 * CB / kThreads, RS = kThreads / CB;   // rows per thread, row stride
  constexpr int kAP = 132;   // LDS pitch of A_s rows (16-byte aligned rows, 4 banks apart)
  const int cb = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
  __shared__ __attribute__((aligned(16))) float As[128 * kAP];
  __shared__ float Xs[128][CB + 1];
  const int D = a.dk, na = D * D / (4 * kThreads);   // float4 pieces of A_s per thread (<= 16)
  const int c = t % CB, col = cb * CB + c, x0 = t / CB;   // the thread's rows: x0 + RS r
  const bool cok = col < a.dv;
  for (int i = t; i < 128 * CB; i += kThreads) {
    const int r = i / CB, cc = i % CB, cl = cb * CB + cc;
    float x = 0.f;
    if (r < D && cl < a.dv) {
      const int64_t m = ((int64_t)bh * D + r) * a.dv + cl;
      x = FWD ? a.M0[m] : (a.dM ? a.dM[m] : 0.f);
    }
    Xs[r][cc] = x;
  }
  // The next segment's A_s and additive term are fetched into registers while
  // the current product runs.
  f32x4 an[16];
  float ad[RPT];
  auto seg_of = [&](int k) __attribute__((always_inline)) { return FWD ? k : a.S - 1 - k; };
  auto fetch = [&](int k) __attribute__((always_inline)) {
    const int s = seg_of(k);
    const int64_t seg = (int64_t)bh * a.S + s;
    if (!is_first(a, s)) {
      const f32x4* src = reinterpret_cast<const f32x4*>(a.Amat + seg * D * D);
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (j < na) an[j] = src[t + kThreads * j];
    }
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      const int x = x0 + RS * r;
      ad[r] = 0.f;
      if (x < D && cok)   // FWD: C_s^T[col][x]; else dMr_s[x][col]
        ad[r] = FWD ? a.dMr[seg * D * a.dv + (int64_t)col * D + x] : a.dMr[seg * D * a.dv + (int64_t)x * a.dv + col];
    }
  };
  auto put_a = [&](int k) __attribute__((always_inline)) {
    if (is_first(a, seg_of(k))) return;
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (j < na) {
        const int i = t + kThreads * j, r = i / (D / 4), q = i % (D / 4);
        *reinterpret_cast<f32x4*>(&As[r * kAP + 4 * q]) = an[j];
      }
  };
  fetch(0);
  put_a(0);
  __syncthreads();
  for (int k = 0; k < a.S; ++k) {
    const int s = seg_of(k);
    const bool first = is_first(a, s);
    const int64_t seg = (int64_t)bh * a.S + s;
    float add[RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r) add[r] = ad[r];
    // the carried matrix at this segment: FWD the snapshot M_{s-1}, else dL/dM_s
    // (in place of dMr_s, already read)
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      const int x = x0 + RS * r;
      if (x < D && cok) {
        float* dst = (FWD ? a.snapM : a.dMr) + seg * D * a.dv + (int64_t)x * a.dv + col;
        *dst = Xs[x][c];
      }
    }
    if (k + 1 < a.S) fetch(k + 1);
    float acc[RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r) acc[r] = 0.f;
    if (!first) {
      for (int y = 0; y < D; y += 4) {
        const float x0v = Xs[y][c], x1v = Xs[y + 1][c], x2v = Xs[y + 2][c], x3v = Xs[y + 3][c];
#pragma unroll
        for (int r = 0; r < RPT; ++r)
          if (x0 + RS * r < D) {
            const f32x4 av = *reinterpret_cast<const f32x4*>(&As[(x0 + RS * r) * kAP + y]);
            acc[r] = __builtin_fmaf(av[0], x0v, acc[r]);
            acc[r] = __builtin_fmaf(av[1], x1v, acc[r]);
            acc[r] = __builtin_fmaf(av[2], x2v, acc[r]);
            acc[r] = __builtin_fmaf(av[3], x3v, acc[r]);
          }
      }
    }
    float nx[RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      const int x = x0 + RS * r;
      nx[r] = x < D ? Xs[x][c] - acc[r] + add[r] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < RPT; ++r) Xs[x0 + RS * r][c] = nx[r];
    if (k + 1 < a.S) put_a(k + 1);
    __syncthreads();
  }
  if (!FWD && a.dM0)
    for (int i = t; i < D * CB; i += kThreads) {
      const int r = i / CB, cc = i % CB, cl = cb * CB + cc;
      if (cl < a.dv) a.dM0[((int64_t)bh * D + r) * a.dv + cl] = Xs[r][cc];
    }
}

// z_{s-1} = z_0 + sum_{s' < s} c_s' in place in snapz (c_s from the contribution
// kernel), one thread per (head, d_key).
__global__ __launch_bounds__(kThreads) void bwd_zscan_kernel(BwdArgs a) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= (int64_t)a.BH * a.dk) return;
  const int bh = (int)(i / a.dk), x = (int)(i % a.dk);
  float run = a.z0[i];
  for (int s = 0; s < a.S; ++s) {
    float* p = a.snapz + ((int64_t)bh * a.S + s) * a.dk + x;
    const float c = *p;
    *p = run;
    run += c;
  }
}

// ---------------------------------------------------------------- finish
// dq, dk, dv in the I/O dtype: dk = dk_att + (d sigma(K) + dL/dz_s [+ de z_{s-1}]) sigma'(k).
// Four consecutive elements per thread when d_key and d_value are multiples of 4,
// else one; grid-stride over (rows x groups of d_key) then (rows x groups of d_value).
__device__ __forceinline__ void st4(bf16* p, const float (&x)[4]) {
  bf16x4 v;
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = f2bf(x[j]);
  *reinterpret_cast<bf16x4*>(p) = v;
}
__device__ __forceinline__ void st4(float* p, const float (&x)[4]) {
  *reinterpret_cast<f32x4*>(p) = f32x4{x[0], x[1], x[2], x[3]};
}
// DIRECT (the bf16 MFMA path): dq and dv were written in their final form by the
// query kernel and the update kernels; only dk is left.
template <typename T, int W, bool DIRECT>
__global__ __launch_bounds__(kThreads) void bwd_finish_kernel(BwdArgs a) {
  const int gk = a.dk / W, gv = a.dv / W;
  const int64_t rows = (int64_t)a.BH * a.L, nk = rows * gk, nv = DIRECT ? 0 : rows * gv;
  const T* K = static_cast<const T*>(a.k);
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nk + nv; i += (int64_t)gridDim.x * kThreads) {
    if (i < nk) {
      const int64_t row = i / gk;
      const int x0 = W * (int)(i % gk);
      const int bh = (int)(row / a.L), s = (int)((row % a.L) / a.N);
      const bool hasd = a.delta && !is_first(a, s);
      const int64_t zi = ((int64_t)bh * a.S + s) * a.dk + x0, ri = row * a.dk + x0;
      const float de = hasd ? a.de[row] : 0.f;
      float dk[W], dq[W];
#pragma unroll
      for (int j = 0; j < W; ++j) {
        const float dfk = __builtin_fmaf(de, a.snapz[zi + j], a.dfk_acc[ri + j] + a.gzs[zi + j]);
        dk[j] = a.dk_acc[ri + j] + dfk * sig_prime(ld(K, ri + j));
        dq[j] = DIRECT ? 0.f : a.dq_acc[ri + j];
      }
      if constexpr (W == 4) {
        st4(static_cast<T*>(a.dk_out) + ri, dk);
        if (!DIRECT) st4(static_cast<T*>(a.dq_out) + ri, dq);
      } else {
#pragma unroll
        for (int j = 0; j < W; ++j) {
          st(static_cast<T*>(a.dk_out), ri + j, dk[j]);
          if (!DIRECT) st(static_cast<T*>(a.dq_out), ri + j, dq[j]);
        }
      }
    } else {
      const int64_t j0 = i - nk, row = j0 / gv;
      const int64_t ri = row * a.dv + W * (j0 % gv);
      float dv[W];
#pragma unroll
      for (int j = 0; j < W; ++j) dv[j] = a.dv_acc[ri + j];
      if constexpr (W == 4) {
        st4(static_cast<T*>(a.dv_out) + ri, dv);
      } else {
#pragma unroll
        for (int j = 0; j < W; ++j) st(static_cast<T*>(a.dv_out), ri + j, dv[j]);
      }
    }
  }
}

// grid (H), 256 threads: dbeta_h = sum over batch, segments and query blocks.
__global__ __launch_bounds__(kThreads) void bwd_dbeta_kernel(BwdArgs a) {
  const int h = blockIdx.x, t = threadIdx.x;
  __shared__ float red[kThreads];
  const int64_t per = (int64_t)a.S * a.nqb;
  float acc = 0.f;
  for (int b = 0; b < a.B; ++b) {
    const float* src = a.dbeta_part + (int64_t)(b * a.H + h) * per;
    for (int64_t i = t; i < per; i += kThreads) acc += src[i];
  }
  red[t] = acc;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if (t < w) red[t] += red[t + w];
    __syncthreads();
  }
  if (t == 0) a.dbeta[h] = red[0];
}

__global__ void bwd_zero_kernel(float* p, int64_t n, float* p2, int64_t n2) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n + n2; i += (int64_t)gridDim.x * blockDim.x) {
    if (i < n) p[i] = 0.f;
    else p2[i - n] = 0.f;
  }
}

int bwd_query_blocks(int N) { return (N + kQB - 1) / kQB; }

template <typename T>
static hipError_t launch_all(const BwdArgs& a, bool mfma, hipStream_t stream) {
  const unsigned BH = (unsigned)a.BH, S = (unsigned)a.S;
  const unsigned ncb = (unsigned)((a.dv + kColB - 1) / kColB);
  hipError_t e;
#define INFINI_BWD_LAUNCH(...)                    \
  do {                                            \
    hipLaunchKernelGGL(__VA_ARGS__);              \
    if ((e = hipGetLastError()) != hipSuccess) return e; \
  } while (0)
  const unsigned ncb32 = (unsigned)((a.dv + 31) / 32);
  const unsigned ncb_chain = (unsigned)((a.dv + kChainCB - 1) / kChainCB);
  const bool delta_mfma = mfma && a.delta;
  if (a.delta && !mfma) {
    INFINI_BWD_LAUNCH(bwd_snap_kernel<T>, dim3(ncb, BH), dim3(kThreads), 0, stream, a);
  } else {
    const int64_t n = (int64_t)a.BH * ((int64_t)a.dk * a.dv + a.dk);
    const dim3 sg((unsigned)((n + kThreads - 1) / kThreads));
    if (mfma) {
      // the forward's MFMA contribution kernel: C_s^T into dMr (free until the
      // retrieval gradients), c_s into snapz
      const LinContribArgs lc{static_cast<const bf16*>(a.k), static_cast<const bf16*>(a.v), a.dMr, a.snapz,
                              a.B, a.H, a.S, a.N, a.L};
      e = a.dk == 128 ? launch_lin_contrib<128>(lc, stream) : launch_lin_contrib<64>(lc, stream);
      if (e != hipSuccess) return e;
      if (delta_mfma) {
        const int64_t nz = (int64_t)a.BH * a.dk;
        INFINI_BWD_LAUNCH(bwd_zscan_kernel, dim3((unsigned)((nz + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                          stream, a);
        e = a.dk == 128 ? launch_backward_delta_amat_mfma<128>(a, stream)
                        : launch_backward_delta_amat_mfma<64>(a, stream);
        if (e != hipSuccess) return e;
        INFINI_BWD_LAUNCH((bwd_delta_chain_kernel<true, kChainCB>), dim3(ncb_chain, BH), dim3(kThreads), 0, stream, a);
      } else {
        INFINI_BWD_LAUNCH((bwd_scan_kernel<false, true>), sg, dim3(kThreads), 0, stream, a);
      }
    } else {
      INFINI_BWD_LAUNCH((bwd_tall_kernel<T, 0>), dim3(ncb32, S, BH), dim3(kThreads), 0, stream, a);
      INFINI_BWD_LAUNCH((bwd_scan_kernel<false, false>), sg, dim3(kThreads), 0, stream, a);
    }
  }
  if (mfma) {
    e = a.dk == 128 ? launch_backward_attention_mfma<128>(a, stream) : launch_backward_attention_mfma<64>(a, stream);
    if (e != hipSuccess) return e;
  } else {
    INFINI_BWD_LAUNCH(bwd_query_kernel<T>, dim3((unsigned)a.nqb, S, BH), dim3(kThreads), 0, stream, a);
    INFINI_BWD_LAUNCH(bwd_key_kernel<T>, dim3((unsigned)((a.N + kKB - 1) / kKB), S, BH), dim3(kThreads), 0, stream,
                      a);
  }
  if (mfma) {
    e = a.dk == 128 ? launch_backward_retrieval_grad_mfma<128>(a, stream)
                    : launch_backward_retrieval_grad_mfma<64>(a, stream);
    if (e != hipSuccess) return e;
  } else {
    INFINI_BWD_LAUNCH((bwd_tall_kernel<T, 1>), dim3(ncb32, S, BH), dim3(kThreads), 0, stream, a);
  }
  if (delta_mfma) {
    INFINI_BWD_LAUNCH((bwd_delta_chain_kernel<false, kChainCB>), dim3(ncb_chain, BH), dim3(kThreads), 0, stream, a);
    e = a.dk == 128 ? launch_backward_delta_update_mfma<128>(a, stream)
                    : launch_backward_delta_update_mfma<64>(a, stream);
    if (e != hipSuccess) return e;
  } else if (a.delta) {
    const int64_t n1 = (int64_t)a.BH * a.L * a.dk, n2 = (int64_t)a.BH * a.L;
    const int64_t blocks = std::min<int64_t>((n1 + n2 + kThreads - 1) / kThreads, 65536);
    INFINI_BWD_LAUNCH(bwd_zero_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a.dfk_acc, n1, a.de, n2);
    INFINI_BWD_LAUNCH(bwd_chain_kernel<T>, dim3(ncb, BH), dim3(kThreads), 0, stream, a);
  } else {
    const int64_t n = (int64_t)a.BH * a.dk * a.dv;
    INFINI_BWD_LAUNCH((bwd_scan_kernel<true, false>), dim3((unsigned)((n + kThreads - 1) / kThreads)),
                      dim3(kThreads), 0, stream, a);
    if (mfma) {
      // the z chain needs only the retrieval's gradient of z here, and the update
      // kernel finishes dk and dv with it
      INFINI_BWD_LAUNCH(bwd_zchain_kernel, dim3(BH), dim3(128), 0, stream, a);
      e = a.dk == 128 ? launch_backward_lin_update_mfma<128>(a, stream) : launch_backward_lin_update_mfma<64>(a, stream);
      if (e != hipSuccess) return e;
    } else {
      INFINI_BWD_LAUNCH(bwd_lin_update_kernel<T>, dim3((unsigned)((a.N + kTok - 1) / kTok), S, BH), dim3(kThreads),
                        0, stream, a);
    }
  }
  if (!(mfma && !a.delta)) {   // (the linear rule's MFMA update kernel finished dk and dv)
    if (delta_mfma) {
      if (a.dk == 128) INFINI_BWD_LAUNCH(bwd_ez_vec_kernel<128>, dim3(S, BH), dim3(kThreads), 0, stream, a);
      else INFINI_BWD_LAUNCH(bwd_ez_vec_kernel<64>, dim3(S, BH), dim3(kThreads), 0, stream, a);
    } else {
      INFINI_BWD_LAUNCH(bwd_ez_kernel<T>, dim3(S, BH), dim3(kThreads), 0, stream, a);
    }
    INFINI_BWD_LAUNCH(bwd_zchain_kernel, dim3(BH), dim3(128), 0, stream, a);
    {
      const uintptr_t al = 4 * sizeof(T) - 1;
      const bool vec = a.dk % 4 == 0 && a.dv % 4 == 0 &&
                       ((reinterpret_cast<uintptr_t>(a.dq_out) | reinterpret_cast<uintptr_t>(a.dk_out) |
                         reinterpret_cast<uintptr_t>(a.dv_out)) & al) == 0;
      // the MFMA path wrote dq and dv already (its outputs are 16-byte aligned)
      const int64_t n = (int64_t)a.BH * a.L * (a.dk + (mfma ? 0 : a.dv)) / (vec ? 4 : 1);
      const dim3 grid((unsigned)std::min<int64_t>((n + kThreads - 1) / kThreads, 1 << 20));
      if (mfma) INFINI_BWD_LAUNCH((bwd_finish_kernel<T, 4, true>), grid, dim3(kThreads), 0, stream, a);
      else if (vec) INFINI_BWD_LAUNCH((bwd_finish_kernel<T, 4, false>), grid, dim3(kThreads), 0, stream, a);
      else INFINI_BWD_LAUNCH((bwd_finish_kernel<T, 1, false>), grid, dim3(kThreads), 0, stream, a);
    }
  }
  INFINI_BWD_LAUNCH(bwd_dbeta_kernel, dim3((unsigned)a.H), dim3(kThreads), 0, stream, a);
#undef INFINI_BWD_LAUNCH
  return hipSuccess;
}

hipError_t launch_backward(const BwdArgs& a, bool bf16_io, hipStream_t stream) {
  if (a.dk > 128 || a.dv > 128 || a.N < 1 || a.S < 1) return hipErrorInvalidValue;
  // the bf16 path (d_key = d_value in {64, 128}, N a multiple of 64) takes the
  // MFMA kernels for the local attention
  const bool mfma = bf16_io && a.dk == a.dv && (a.dk == 64 || a.dk == 128) && a.N % 64 == 0;
  return bf16_io ? launch_all<bf16>(a, mfma, stream) : launch_all<float>(a, false, stream);
}

}  // namespace infini
