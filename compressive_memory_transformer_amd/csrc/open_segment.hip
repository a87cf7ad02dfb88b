// Tokens of an open segment (streaming inference, ragged tails): queries that
// arrive before their segment is complete (page "精读笔记：Infini-attention",
// abstract: streaming inference; section 3.1 with the causal mask of section 3.8
// step 2 for A_dot, section 3.3 for A_mem, section 3.5 for the gate).
//
// A query at position p of the open segment attends to the segment's keys
// 0..p (those before pos0 from the open-segment buffers, the new ones straight
// from the input) and reads the memory (M, z) as it stands, i.e. as of the
// segment's start.  Both dtypes run in fp32 arithmetic.
//
// Appends of 64 or more tokens (bf16) take open_attn_mfma_kernel (below); the
// rest split over keys and memory rows (the decode case has one query per head,
// up to N keys and a 64 KiB memory per head at d = 128):
//   open_attn_partial: one workgroup per (slot, group of 8 queries, head).  Slots
//     below P are 128-key partitions: scores, the partition's maximum and sum,
//     and its share of P V.  The R slots after them each take 16 rows of M and z:
//     their share of sigma(q) M and of sigma(q) z;
//   open_attn_combine: one workgroup per (query, head); the key partitions merged
//     in a fixed order, the memory shares summed in a fixed order, the retrieval
//     sigma(q) M / (sigma(q) z), the gate, the output, and the query's key and
//     value rows copied into the open-segment buffers (after the partial kernel
//     has read them, in stream order).
#include "common.h"
#include "kernels.h"
#include "mfma_ops.h"

namespace infini {

namespace {

constexpr int kOpenThreads = 128;   // threads per workgroup = keys per partition
constexpr int kOpenQ = 8;           // queries per partial workgroup
constexpr int kMemRows = 16;        // rows of M per memory slot

__device__ __forceinline__ float load_elem(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float load_elem(const bf16* p, int64_t i) { return bf2f(p[i]); }
__device__ __forceinline__ void store_elem(float* p, int64_t i, float x) { p[i] = x; }
__device__ __forceinline__ void store_elem(bf16* p, int64_t i, float x) { p[i] = f2bf(x); }

// Eight consecutive elements starting at p (16-byte aligned for bf16, 32 for fp32).
__device__ __forceinline__ void load8(const bf16* p, float (&x)[8]) {
  const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = bf2f(v[e]);
}
__device__ __forceinline__ void load8(const float* p, float (&x)[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[e] = a[e];
    x[4 + e] = b[e];
  }
}

// Maximum / sum over the workgroup (two waves) in a fixed order.
__device__ __forceinline__ float wg_max(float x, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  return fmaxf(red[0], red[1]);
}
__device__ __forceinline__ float wg_sum(float x, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  return red[0] + red[1];
}

}  // namespace

// Q queries per workgroup: 1 for a decode step, kOpenQ otherwise.  With one
// query, each thread issues all of its K row loads (and later its 16 V row
// loads) at once: a decode step is a few dependent memory round trips.  With
// eight, the accumulators take the registers and the loads go one at a time.
template <typename T, int Q>
__global__ __launch_bounds__(kOpenThreads)
void open_attn_partial_kernel(OpenAttnArgs a) {
  constexpr int kOpenQ = Q;
  constexpr int LB = Q == 1 ? 16 : 1;
  const int part = blockIdx.x, j0 = blockIdx.y * kOpenQ, bh = blockIdx.z;
  const int t = threadIdx.x;
  const int nq = min(kOpenQ, a.m - j0);
  const int nkeys = a.pos0 + a.m;               // keys of the open segment after the append
  const int slot_stride = a.P + a.R;
  const T* q = static_cast<const T*>(a.q);
  const T* kseg = static_cast<const T*>(a.kseg);
  const T* vseg = static_cast<const T*>(a.vseg);
  const T* knew = static_cast<const T*>(a.knew);
  const T* vnew = static_cast<const T*>(a.vnew);
  __shared__ float qs[kOpenQ][128];
  __shared__ float ps[kOpenQ][kOpenThreads];
  __shared__ float pv[kOpenThreads / 16][kOpenQ][128];   // P V shares of the 8 key groups
  __shared__ float red[2];
  for (int i = t; i < kOpenQ * a.dk; i += kOpenThreads) {
    const int jj = i / a.dk, c = i % a.dk;
    qs[jj][c] = jj < nq ? load_elem(q, ((int64_t)bh * a.q_stride + j0 + jj) * a.dk + c) : 0.f;
  }
  __syncthreads();

  if (part >= a.P) {
    // memory slot: rows r0 .. r0 + 15 of M and z.  The loads are issued
    // together (rows past d_key clamped to the last one and then ignored).
    const int r0 = (part - a.P) * kMemRows;
    if (t < a.dv) {
      const float* Mh = a.M + (int64_t)bh * a.dk * a.dv + t;
      float mv[kMemRows];
#pragma unroll
      for (int i = 0; i < kMemRows; ++i) mv[i] = Mh[(int64_t)min(r0 + i, a.dk - 1) * a.dv];
      float num[kOpenQ];
#pragma unroll
      for (int jj = 0; jj < kOpenQ; ++jj) num[jj] = 0.f;
#pragma unroll
      for (int i = 0; i < kMemRows; ++i) {
        if (r0 + i >= a.dk) break;
#pragma unroll
        for (int jj = 0; jj < kOpenQ; ++jj) {
          const float x = qs[jj][r0 + i];
          num[jj] = __builtin_fmaf(x > 0.f ? x + 1.f : exp_e(x), mv[i], num[jj]);
        }
      }
#pragma unroll
      for (int jj = 0; jj < kOpenQ; ++jj)
        if (jj < nq) a.part[(((int64_t)bh * a.m + j0 + jj) * slot_stride + part) * (a.dv + 2) + t] = num[jj];
    }
    if (t < nq) {
      float zv[kMemRows];
#pragma unroll
      for (int i = 0; i < kMemRows; ++i) zv[i] = a.z[(int64_t)bh * a.dk + min(r0 + i, a.dk - 1)];
      float den = 0.f;
#pragma unroll
      for (int i = 0; i < kMemRows; ++i) {
        if (r0 + i >= a.dk) break;
        const float x = qs[t][r0 + i];
        den = __builtin_fmaf(x > 0.f ? x + 1.f : exp_e(x), zv[i], den);
      }
      a.part[(((int64_t)bh * a.m + j0 + t) * slot_stride + part) * (a.dv + 2) + a.dv] = den;
    }
    return;
  }

  // score of this thread's key for every query of the group (-inf where the
  // query may not see the key)
  const int kk = part * kOpenThreads + t;
  const int kr = min(kk, nkeys - 1);            // rows past the last key: clamped, masked below
  float s[kOpenQ];
#pragma unroll
  for (int jj = 0; jj < kOpenQ; ++jj) s[jj] = 0.f;
  {
    const T* krow = kr < a.pos0 ? kseg + ((int64_t)bh * a.N + kr) * a.dk
                                : knew + ((int64_t)bh * a.q_stride + kr - a.pos0) * a.dk;
    if (a.dk % 8 == 0) {
      // the row's loads LB at a time (columns past d_key clamped, then skipped)
      for (int cb = 0; cb < 16; cb += LB) {
        if (8 * cb >= a.dk) break;
        float x[LB][8];
#pragma unroll
        for (int i = 0; i < LB; ++i) load8(krow + min(8 * (cb + i), a.dk - 8), x[i]);
#pragma unroll
        for (int i = 0; i < LB; ++i) {
          if (8 * (cb + i) >= a.dk) break;
#pragma unroll
          for (int e = 0; e < 8; ++e)
#pragma unroll
            for (int jj = 0; jj < kOpenQ; ++jj) s[jj] = __builtin_fmaf(qs[jj][8 * (cb + i) + e], x[i][e], s[jj]);
        }
      }
    } else {
      for (int c = 0; c < a.dk; ++c) {
        const float x = load_elem(krow, c);
#pragma unroll
        for (int jj = 0; jj < kOpenQ; ++jj) s[jj] = __builtin_fmaf(qs[jj][c], x, s[jj]);
      }
    }
  }
  float mx[kOpenQ], l[kOpenQ];
#pragma unroll
  for (int jj = 0; jj < kOpenQ; ++jj) {
    ps[jj][t] = 0.f;
    mx[jj] = -__builtin_inff();
    l[jj] = 0.f;
    if (jj >= nq) continue;   // uniform over the workgroup
    const bool vis = kk < nkeys && kk <= a.pos0 + j0 + jj;
    const float sc = vis ? s[jj] * a.scale : -__builtin_inff();
    mx[jj] = wg_max(sc, red);
    const float p = (mx[jj] == -__builtin_inff() || !vis) ? 0.f : exp_e(sc - mx[jj]);
    l[jj] = wg_sum(p, red);
    ps[jj][t] = p;
  }
  __syncthreads();

  // this partition's share of P V
  const int k0 = part * kOpenThreads;
  const int kend = min(kOpenThreads, nkeys - k0);
  if (Q == 1 && a.dv % 8 == 0) {
    // thread = (key group kg of 16 keys, 8 columns cg); its row loads are
    // issued LB at a time (keys past the last clamped, weighted 0), then the 8
    // key groups are summed through LDS
    const int cg = t & 15, kg = t >> 4;
    if (8 * cg < a.dv) {
      float o[kOpenQ][8];
#pragma unroll
      for (int jj = 0; jj < kOpenQ; ++jj)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[jj][e] = 0.f;
      for (int ib = 0; ib < 16; ib += LB) {
        if (kg + 8 * ib >= kend) break;
        float x[LB][8];
#pragma unroll
        for (int i = 0; i < LB; ++i) {
          const int key = k0 + min(kg + 8 * (ib + i), kend - 1);
          const T* vrow = key < a.pos0 ? vseg + ((int64_t)bh * a.N + key) * a.dv
                                       : vnew + ((int64_t)bh * a.q_stride + key - a.pos0) * a.dv;
          load8(vrow + 8 * cg, x[i]);
        }
#pragma unroll
        for (int i = 0; i < LB; ++i) {
          const int kl = kg + 8 * (ib + i);
          const bool in = kl < kend;
#pragma unroll
          for (int jj = 0; jj < kOpenQ; ++jj) {
            const float p = in ? ps[jj][kl] : 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) o[jj][e] = __builtin_fmaf(p, in ? x[i][e] : 0.f, o[jj][e]);
          }
        }
      }
#pragma unroll
      for (int jj = 0; jj < kOpenQ; ++jj)
        if (jj < nq)
#pragma unroll
          for (int e = 0; e < 8; ++e) pv[kg][jj][8 * cg + e] = o[jj][e];
    }
    __syncthreads();
    if (t < a.dv) {
#pragma unroll
      for (int jj = 0; jj < kOpenQ; ++jj) {
        if (jj >= nq) break;
        float o = 0.f;
#pragma unroll
        for (int g = 0; g < kOpenThreads / 16; ++g) o += pv[g][jj][t];
        float* dst = a.part + (((int64_t)bh * a.m + j0 + jj) * slot_stride + part) * (a.dv + 2);
        dst[t] = o;
        if (t == 0) {
          dst[a.dv] = mx[jj];
          dst[a.dv + 1] = l[jj];
        }
      }
    }
  } else if (t < a.dv) {
    // thread t holds column t of d_value
    float o[kOpenQ];
#pragma unroll
    for (int jj = 0; jj < kOpenQ; ++jj) o[jj] = 0.f;
    for (int i = 0; i < kend; ++i) {
      const int key = k0 + i;
      const float x = key < a.pos0 ? load_elem(vseg, ((int64_t)bh * a.N + key) * a.dv + t)
                                   : load_elem(vnew, ((int64_t)bh * a.q_stride + key - a.pos0) * a.dv + t);
#pragma unroll
      for (int jj = 0; jj < kOpenQ; ++jj) o[jj] = __builtin_fmaf(ps[jj][i], x, o[jj]);
    }
#pragma unroll
    for (int jj = 0; jj < kOpenQ; ++jj) {
      if (jj >= nq) break;
      float* dst = a.part + (((int64_t)bh * a.m + j0 + jj) * slot_stride + part) * (a.dv + 2);
      dst[t] = o[jj];
      if (t == 0) {
        dst[a.dv] = mx[jj];
        dst[a.dv + 1] = l[jj];
      }
    }
  }
}

template <typename T>
__global__ __launch_bounds__(kOpenThreads)
void open_attn_combine_kernel(OpenAttnArgs a) {
  const int j = blockIdx.x, bh = blockIdx.y, h = bh % a.H;
  const int t = threadIdx.x;
  const int nslots = a.P + a.R;
  const float g = sigmoid_gate(a.beta[h]);
  const float* parts = a.part + ((int64_t)bh * a.m + j) * nslots * (a.dv + 2);

  // One pass over the slots, 16 at a time with their loads issued together
  // (slots past the last clamped, then skipped).  Key partitions are merged
  // online against the running maximum, in partition order; the memory slots'
  // shares of sigma(q) M and sigma(q) z are summed in slot order.
  float mx = -__builtin_inff(), l = 0.f, o = 0.f, num = 0.f, den = 0.f;
  for (int s0 = 0; s0 < nslots; s0 += 16) {
    float vo[16], vm[16], vl[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float* src = parts + (int64_t)min(s0 + i, nslots - 1) * (a.dv + 2);
      vo[i] = src[min(t, a.dv - 1)];
      vm[i] = src[a.dv];
      vl[i] = src[a.dv + 1];
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int sl = s0 + i;
      if (sl >= nslots) break;
      if (sl < a.P) {
        if (vm[i] == -__builtin_inff()) continue;   // no visible key in this partition
        const float nm = fmaxf(mx, vm[i]);
        const float ca = exp_e(mx - nm), cb = exp_e(vm[i] - nm);   // exp(-inf) = 0 on the first
        l = l * ca + vl[i] * cb;
        o = o * ca + vo[i] * cb;
        mx = nm;
      } else {
        num += vo[i];
        den += vm[i];
      }
    }
  }
  const float a_dot = o / l;   // l > 0: every query sees at least its own key
  // A_mem = sigma(q) M / (sigma(q) z), 0 for a stream's first segment
  const float a_mem = a.has_memory && den > 0.f ? num / den : 0.f;
  const int64_t qrow = ((int64_t)bh * a.q_stride + j);
  if (t < a.dv) store_elem(static_cast<T*>(a.out), qrow * a.dv + t, g * a_mem + (1.f - g) * a_dot);
  // the new token's key and value join the open segment
  const int64_t orow = (int64_t)bh * a.N + a.pos0 + j;
  if (t < a.dk) static_cast<T*>(a.kseg_out)[orow * a.dk + t] = static_cast<const T*>(a.knew)[qrow * a.dk + t];
  if (t < a.dv) static_cast<T*>(a.vseg_out)[orow * a.dv + t] = static_cast<const T*>(a.vnew)[qrow * a.dv + t];
}

// Many queries at once (bf16, d_key = d_value = D): one workgroup (4 waves) per 128
// of the m new queries, one wave per 32, the segment's keys up to the block's last
// query in chunks of 64 (those before pos0 from the open-segment buffers, the new
// ones from the input) staged through two LDS buffers.  Scores transposed (keys x
// queries) with an online softmax per query column, then the retrieval from
// (M, z) (M staged as bf16 with fp32 column sums, (sigma(q) - 1) as the operand),
// the gate, and the new rows copied into the open segment.
template <int D>
__global__ __launch_bounds__(256) void open_attn_mfma_kernel(OpenAttnArgs a) {
  constexpr int P = D + 8, KS = D / 16, DB = D / 32, CH = 64;
  constexpr int PIECES = CH * D / 8 / 256;
  const int qb = blockIdx.x, bh = blockIdx.y, h = bh % a.H;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, l32 = lane & 31, hh = lane >> 5;
  const bf16* Q = static_cast<const bf16*>(a.q);
  const bf16* kseg = static_cast<const bf16*>(a.kseg);
  const bf16* vseg = static_cast<const bf16*>(a.vseg);
  const bf16* knew = static_cast<const bf16*>(a.knew);
  const bf16* vnew = static_cast<const bf16*>(a.vnew);
  __shared__ __attribute__((aligned(16))) bf16 kc[2][CH * P];
  __shared__ __attribute__((aligned(16))) bf16 vc[2][CH * P];
  __shared__ __attribute__((aligned(16))) bf16 ms[D * P];
  __shared__ float msum[D], zsh[D], ctmp[128];
  const int j0 = qb * 128 + 32 * w;                  // the wave's first new query
  const bool qvalid = j0 < a.m;
  const int jq = min(j0 + l32, a.m - 1);             // the lane's query (column of S^T)
  const int qpos = a.pos0 + j0 + l32;                // its position in the segment
  const int64_t qrow = (int64_t)bh * a.q_stride + jq;
  const int kend = min(a.pos0 + a.m, a.pos0 + qb * 128 + 128);   // keys the block's queries see
  const float sl2 = a.scale * kLog2e;
  if (a.has_memory) {   // uniform over the workgroup
    const float* Mg = a.M + (int64_t)bh * D * D;
    for (int x = t; x < D * D; x += 256) ms[(x / D) * P + x % D] = f2bf(Mg[x]);
    if (t < D) zsh[t] = a.z[(int64_t)bh * D + t];
    block_colsum256(Mg, D, D, msum, ctmp);
  }
  bf16x8 qr[KS];
#pragma unroll
  for (int c = 0; c < KS; ++c) qr[c] = *reinterpret_cast<const bf16x8*>(Q + qrow * D + 16 * c + 8 * hh);
  // key row r of the segment (clamped to the last key; later ones are masked)
  auto krow = [&](const bf16* seg, const bf16* nw, int r) -> const bf16* {
    r = min(r, kend - 1);
    return r < a.pos0 ? seg + ((int64_t)bh * a.N + r) * D : nw + ((int64_t)bh * a.q_stride + r - a.pos0) * D;
  };
  bf16x8 pk[PIECES], pv[PIECES];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < PIECES; ++i) {
      const int p = t + 256 * i, r = p / (D / 8), c8 = p % (D / 8);
      pk[i] = *reinterpret_cast<const bf16x8*>(krow(kseg, knew, k0 + r) + 8 * c8);
      pv[i] = *reinterpret_cast<const bf16x8*>(krow(vseg, vnew, k0 + r) + 8 * c8);
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PIECES; ++i) {
      const int p = t + 256 * i, r = p / (D / 8), c8 = p % (D / 8);
      *reinterpret_cast<bf16x8*>(kc[buf] + r * P + 8 * c8) = pk[i];
      *reinterpret_cast<bf16x8*>(vc[buf] + r * P + 8 * c8) = pv[i];
    }
  };
  f32x16 o[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d) o[d] = mo_zero();
  float m2 = -__builtin_inff(), l = 0.f;
  load(0);
  store(0);
  __syncthreads();
  for (int k0 = 0, buf = 0; k0 < kend; k0 += CH, buf ^= 1) {
    const bool next = k0 + CH < kend;
    if (next) load(k0 + CH);
    if (qvalid && k0 <= a.pos0 + j0 + 31) {
      f32x16 sa[2] = {mo_zero(), mo_zero()};
#pragma unroll
      for (int c = 0; c < KS; ++c)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) sa[kt] = mfma32(mo_row(kc[buf], P, 32 * kt, 16 * c, lane), qr[c], sa[kt]);
      float mx = -__builtin_inff();
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float v = k0 + 32 * kt + mo_acc_row(r, hh) <= qpos ? sa[kt][r] * sl2 : -__builtin_inff();
          sa[kt][r] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mn = fmaxf(m2, mx);                // finite: key 0 is in the first chunk
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
          const float pe = exp2_fast(sa[kt][r] - mn);
          sa[kt][r] = pe;
          l += pe;
        }
      m2 = mn;
      bf16x8 pb[2][2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
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
  const float inv_l = 1.f / (l + __shfl_xor(l, 32));
  // retrieval: (colsum(M) + M^T (sigma(q) - 1)) / (sigma(q) . z); 0 in a stream's first segment
  bf16x8 qm[KS];
  float den = 0.f;
#pragma unroll
  for (int c = 0; c < KS; ++c)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float x = bf2f(qr[c][j]);
      const float f = x > 0.f ? x : exp_e(x) - 1.f;
      qm[c][j] = f2bf(f);
      if (a.has_memory) den = __builtin_fmaf(f + 1.f, zsh[16 * c + 8 * hh + j], den);
    }
  den += __shfl_xor(den, 32);
  const float g = sigmoid_gate(a.beta[h]);
  const float wm = a.has_memory && den > 0.f ? g / den : 0.f;
  const float wd = (1.f - g) * inv_l;
  if (!qvalid) return;
  bf16* out = static_cast<bf16*>(a.out);
  const bool mine = j0 + l32 < a.m;
#pragma unroll
  for (int d = 0; d < DB; ++d) {
    f32x16 am = mo_zero();
    if (a.has_memory) {
#pragma unroll
      for (int c = 0; c < KS; ++c) am = mfma32(mo_col(ms, P, 16 * c, 32 * d, lane), qm[c], am);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int col = 32 * d + mo_acc_row(r, hh);
      const float mem = a.has_memory ? msum[col] + am[r] : 0.f;
      if (mine) out[qrow * D + col] = f2bf(__builtin_fmaf(o[d][r], wd, mem * wm));
    }
  }
  // the new key and value rows join the open segment (rows pos0 + j; the reads of
  // this launch take new keys from the input, so these writes race with none)
  if (mine) {
    const int64_t orow = (int64_t)bh * a.N + a.pos0 + jq;
#pragma unroll
    for (int c = 0; c < KS; ++c) {
      *reinterpret_cast<bf16x8*>(static_cast<bf16*>(a.kseg_out) + orow * D + 16 * c + 8 * hh) =
          *reinterpret_cast<const bf16x8*>(knew + qrow * D + 16 * c + 8 * hh);
      *reinterpret_cast<bf16x8*>(static_cast<bf16*>(a.vseg_out) + orow * D + 16 * c + 8 * hh) =
          *reinterpret_cast<const bf16x8*>(vnew + qrow * D + 16 * c + 8 * hh);
    }
  }
}

int open_attn_slots(int keys, int dk) {
  return (keys + kOpenThreads - 1) / kOpenThreads + (dk + kMemRows - 1) / kMemRows;
}

hipError_t launch_open_attn(const OpenAttnArgs& args, hipStream_t stream) {
  OpenAttnArgs a = args;
  if (a.m <= 0) return hipSuccess;
  if (a.dk > 128 || a.dv > 128 || a.pos0 + a.m > a.N) return hipErrorInvalidValue;
  a.P = (a.pos0 + a.m + kOpenThreads - 1) / kOpenThreads;
  a.R = a.has_memory ? (a.dk + kMemRows - 1) / kMemRows : 0;
  if (a.bf16 && a.dk == a.dv && (a.dk == 64 || a.dk == 128) && a.m >= 64) {
    // many queries: the MFMA kernel (no partial results, one launch)
    const dim3 grid((unsigned)((a.m + 127) / 128), (unsigned)a.BH);
    if (a.dk == 128) hipLaunchKernelGGL(open_attn_mfma_kernel<128>, grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL(open_attn_mfma_kernel<64>, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  const bool one = a.m == 1;
  const dim3 gp((unsigned)(a.P + a.R), (unsigned)(one ? 1 : (a.m + kOpenQ - 1) / kOpenQ), (unsigned)a.BH);
  const dim3 gc((unsigned)a.m, (unsigned)a.BH);
  if (a.bf16) {
    if (one)
      hipLaunchKernelGGL((open_attn_partial_kernel<bf16, 1>), gp, dim3(kOpenThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((open_attn_partial_kernel<bf16, kOpenQ>), gp, dim3(kOpenThreads), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(open_attn_combine_kernel<bf16>, gc, dim3(kOpenThreads), 0, stream, a);
  } else {
    if (one)
      hipLaunchKernelGGL((open_attn_partial_kernel<float, 1>), gp, dim3(kOpenThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((open_attn_partial_kernel<float, kOpenQ>), gp, dim3(kOpenThreads), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(open_attn_combine_kernel<float>, gc, dim3(kOpenThreads), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace infini
