// Local attention part of the gradients on the bf16 MFMA units (the chain rule
// through A_dot = softmax(scale Q K^T, causal) V of the close-reading page
// "精读笔记：Infini-attention", section 3.1 with the mask of section 3.8 step 2),
// and the retrieval's share of the query gradient (section 3.3).
//
//   bwd_q2_kernel<D>: query-stationary.  One workgroup (8 waves, two per SIMD)
//     per pair of 256-query tiles of one segment (tile t and NT-1-t, so that the
//     causal work is equal), one wave per 32 queries.  First sweep over the
//     keys: softmax statistics (log2 normaliser) and A_dot, then E = <dA, A_dot>
//     and D = (1 - g) E.  Second sweep: dS = P ((1 - g) dP - D) and
//     dq = scale dS K.  Then the retrieval, with M_{s-1} staged once per
//     workgroup in LDS as bf16: A_mem = (colsum(M) + (sigma(q) - 1) M) /
//     (sigma(q) z) (the column sums in fp32 keep sigma(q) ~ 1 from costing bf16
//     precision), <dA, A_mem>, rs = g / den, dden, the gate's share of dbeta,
//     and dq += (M (rs dA) + dden z) sigma'(q), written once in bf16.
//   bwd_kv2_kernel<D>: key-stationary.  One workgroup (8 waves) per pair of
//     256-key tiles, one wave per 32 keys; the tile's keys sit in LDS, the
//     wave's values in registers.  For every 32 later queries: S, dP, P, dS,
//     then dv += (1 - g) P^T dA and dk += scale dS^T Q.
//
// Scores are computed with the stationary rows as accumulator columns (keys x
// queries in the query kernel, queries x keys in the key kernel), so the
// probabilities and dS feed the next product straight from the accumulators:
// a row-major LDS tile X is read either by rows (lane l gets
// X[r0 + l % 32][k0 + 8 (l / 32) + 0..7]) or, for a contraction over its rows,
// with the transposing LDS read (lane l gets X[r0 + 4 h + e][c0 + l % 32] and
// X[r0 + 8 + 4 h + e][...], h = l / 32), whose row order matches a 32 x 32
// accumulator used as the other operand (lane l holds rows 8 (r / 4) + 4 h +
// r % 4 of column l % 32).
//
// The streamed operand (K and V, or Q, dA and the rows' statistics) moves
// HBM -> LDS in 64-row steps with buffer_load ... lds (no staging registers)
// through a ring of LDS slots, each slot an array of its own so that the
// compiler never waits on loads into another slot.  Both read patterns hit
// every tile, so one XOR swizzle of the 16-byte chunks serves both: rows
// r % 4 and (r / 4) % 4 (D = 128) or (r / 2) % 2 and (r / 4) % 4 (D = 64) pick
// the chunk permutation, which makes 16 consecutive rows of one logical chunk
// and 4 consecutive rows x 4 consecutive chunks each hit 16 distinct bank
// groups.
#include <algorithm>

#include "common.h"
#include "kernels.h"
#include "mfma_ops.h"

namespace infini {

namespace {

constexpr int kBwdWaves = 4;                // waves of the Gram kernel's workgroup
constexpr int kUpdWaves = 8;                // waves of the linear-update kernel
constexpr int kUpdBlock = 32 * kUpdWaves;   // tokens per workgroup of that kernel
constexpr int kXtP = 36;                    // row pitch (floats) of its transposing tiles
constexpr int kDuWaves = 8;                 // waves of the delta-update kernel (two staged
constexpr int kDuBlock = 32 * kDuWaves;     // matrices shared by 256 tokens)
constexpr int kChunk = 64;                  // tokens per step of the Gram kernel

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

// Stages a row-major fp32 [D][D] matrix into LDS as bf16 (pitch D + 8) and its
// column sums in fp32, by a workgroup of NT threads: thread t loads the 16-byte
// pieces t + NT j (always the same four columns), keeps their partial column
// sums, and the NT / (D / 4) row groups meet in `red` (4 NT floats).  Ends with a
// barrier.
template <int D, int NT>
__device__ __forceinline__ void stage_mat(const float* X, bf16* xs, float* colsum, float* red) {
  constexpr int P = D + 8, Q4 = D / 4, NJ = D * D / 4 / NT, G = NT / Q4;
  static_assert(G * D == 4 * NT && NJ * NT * 4 == D * D, "row groups x columns fill the reduction array");
  const int t = threadIdx.x, c4 = t % Q4, r0 = t / Q4;
  f32x4 v[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) v[j] = reinterpret_cast<const f32x4*>(X)[t + NT * j];
  f32x4 cs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    bf16x4 b;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      cs[e] += v[j][e];
      b[e] = f2bf(v[j][e]);
    }
    *reinterpret_cast<bf16x4*>(xs + (r0 + G * j) * P + 4 * c4) = b;
  }
  *reinterpret_cast<f32x4*>(red + r0 * D + 4 * c4) = cs;
  __syncthreads();
  if (t < D) {
    float sum = 0.f;
#pragma unroll
    for (int g = 0; g < G; ++g) sum += red[g * D + t];
    colsum[t] = sum;
  }
  __syncthreads();
}

// ------------------------------------------- streamed tiles of the attention kernels
constexpr int kBw = 8;                  // waves per workgroup
constexpr int kBwRows = 32 * kBw;       // stationary rows per tile
constexpr int kBwStep = 64;             // streamed rows per step

template <int D>
struct BwL {
  static constexpr int KS = D / 16;                  // 16-column steps of a row
  static constexpr int DB = D / 32;                  // 32-column blocks of a row
  static constexpr int CH = D / 8;                   // 16-byte chunks per row
  static constexpr int RPI = 64 / CH;                // rows per 1 KB wave-wide load
  static constexpr int NIN = kBwStep / RPI / kBw;    // loads per wave per streamed tile
  static constexpr int TILE = kBwStep * D;           // elements per streamed tile
  static_assert(NIN >= 1 && NIN * RPI * kBw == kBwStep, "a step's rows split evenly over the waves");
};

// Physical-chunk XOR of row r (the same map takes logical to physical and back).
template <int D>
__device__ __forceinline__ int bw_swz(int r) {
  return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

#if defined(__HIP_DEVICE_COMPILE__)
// Buffer resource over `bytes` bytes at `base`; wave-uniform (scalar registers).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t bw_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  void* ub = (void*)(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}
#endif

// Per-lane offsets into swizzled [rows x D] tiles.
template <int D>
struct BwOfs {
  using L = BwL<D>;
  int dma[L::NIN];   // bytes: this lane's 16-byte piece of the wave's loads of a 64-row tile
  int row[4];        // elements: row reads at r0 = 0, 16-column steps 0..3
  int rowd;          // D = 128: steps 4..7 sit at row[i] + rowd
  int tr[L::DB];     // elements: transposing reads at r0 = 0, first 4-row group, per 32-column block
  int trd;           // the second 4-row group (8 rows further)
  __device__ __forceinline__ void init(int lane, int wave) {
#pragma unroll
    for (int j = 0; j < L::NIN; ++j) {
      const int ins = wave * L::NIN + j;
      const int r = ins * L::RPI + lane / L::CH;
      dma[j] = 2 * (r * D + 8 * ((lane % L::CH) ^ bw_swz<D>(r)));
    }
    const int l32 = lane & 31, hh = lane >> 5, sw = bw_swz<D>(l32);
#pragma unroll
    for (int i = 0; i < 4; ++i) row[i] = l32 * D + 8 * ((2 * i + hh) ^ sw);
    rowd = (sw & 8) ? -64 : 64;   // logical chunk + 8 flips bit 3 of the physical one
    const int s = lane & 15, g1 = (lane >> 4) & 1, ra = 4 * hh + (s >> 2);
#pragma unroll
    for (int db = 0; db < L::DB; ++db) {
      const int cc = 4 * db + 2 * g1 + ((s & 3) >> 1);
      tr[db] = ra * D + 8 * (cc ^ bw_swz<D>(ra)) + 4 * (s & 1);
    }
    // 8 rows further the XOR flips bit 1 of the physical chunk, which is g1 here
    trd = 8 * D + (g1 ? -16 : 16);
  }
  // Called once per step: the sums of an LDS array's address and these offsets
  // are then formed in the step (a few adds) instead of being hoisted out of the
  // loop as one live register per array and offset (the compiler does not fold
  // the arrays' addresses into the instructions' immediate offsets).
  __device__ __forceinline__ void opaque() {
#pragma unroll
    for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(row[i]));
    asm volatile("" : "+v"(rowd));
#pragma unroll
    for (int db = 0; db < L::DB; ++db) asm volatile("" : "+v"(tr[db]));
    asm volatile("" : "+v"(trd));
  }
  // Row operand, 16-column step c, rows r0 + [0, 32) (r0 a multiple of 32).
  __device__ __forceinline__ int rd(int c, int r0) const {
    return row[c & 3] + (c >= 4 ? rowd : 0) + r0 * D;
  }
};

template <int D>
__device__ __forceinline__ bf16x8 bw_row(const bf16* X, const BwOfs<D>& of, int c, int r0) {
  return lds_read8(X + of.rd(c, r0));
}
// Transposed operand of 32-column block db over rows r0 + [0, 16) (r0 a multiple of 16).
template <int D>
__device__ __forceinline__ bf16x8 bw_tr(const bf16* X, const BwOfs<D>& of, int db, int r0) {
  const bf16* p = X + of.tr[db] + r0 * D;
  const s16x4 x = lds_read_tr16(p);
  const s16x4 y = lds_read_tr16(p + of.trd);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7));
}

// This wave's share of the loads of the 64 rows at `src` (row-major, D columns)
// into a swizzled LDS tile.
template <int D>
__device__ __forceinline__ void bw_dma(const bf16* src, bf16* dst, int wave, const BwOfs<D>& of) {
#if defined(__HIP_DEVICE_COMPILE__)
  const __amdgpu_buffer_rsrc_t rsrc = bw_rsrc(src, kBwStep * D * 2);
  const int wv = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
  for (int j = 0; j < BwL<D>::NIN; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (INFINI_LDS void*)(dst + (wv * BwL<D>::NIN + j) * 512), 16,
                                             of.dma[j], 0, 0, 0);
#endif
}

// Waits until at most VM of this wave's vector memory operations are in flight
// and its LDS operations are done, then synchronises the workgroup.
template <int VM>
__device__ __forceinline__ void bw_wait_sync() {
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | 0x0070);
  __builtin_amdgcn_s_barrier();
}

__device__ __forceinline__ float bw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Four-element accesses within a wave's 32 rows of D elements at the
// wave-uniform `base`: the lane's byte offset `vb` in a vector register, a
// compile-time constant one `sb` in a scalar register, so that the accesses of
// a 32 x 32 block need no 64-bit address each.
template <int D>
__device__ __forceinline__ f32x4 wv_ld4(const float* base, int vb, int sb) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(bw_rsrc(base, 32 * D * 4), vb, sb, 0));
#else
  return f32x4{};
#endif
}
template <int D>
__device__ __forceinline__ bf16x4 wv_ld4(const bf16* base, int vb, int sb) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_raw_buffer_load_b64(bw_rsrc(base, 32 * D * 2), vb, sb, 0));
#else
  return bf16x4{};
#endif
}
template <int D>
__device__ __forceinline__ void wv_st4(float* base, int vb, int sb, f32x4 x) {
#if defined(__HIP_DEVICE_COMPILE__)
  using u4 = __attribute__((ext_vector_type(4))) unsigned int;
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, x), bw_rsrc(base, 32 * D * 4), vb, sb, 0);
#endif
}
template <int D>
__device__ __forceinline__ void wv_st4(bf16* base, int vb, int sb, bf16x4 x) {
#if defined(__HIP_DEVICE_COMPILE__)
  using u2 = __attribute__((ext_vector_type(2))) unsigned int;
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u2, x), bw_rsrc(base, 32 * D * 2), vb, sb, 0);
#endif
}

// Turns f times a 32 x 32 accumulator block (lane ln holds column ln % 32, rows
// 8 j4 + 4 (ln / 32) + 0..3 at elements 4 j4 ..) into row pieces: piece[it] =
// row ln / 8 + 8 it, columns 4 (ln % 8) .. + 3 of the block's transpose, i.e.
// the lane's column-major element runs become eight-lanes-per-row pieces.  `xw`
// is the wave's own 4 KB LDS tile; its 16-byte chunk c of row r sits at
// c ^ (r % 8).
__device__ __forceinline__ void turn32(float* xw, const f32x16& acc, float f, int ln, f32x4* piece) {
  const int r32 = ln & 31, h2 = ln >> 5, tr = (ln >> 3) & 7, c8 = ln & 7;
#pragma unroll
  for (int j4 = 0; j4 < 4; ++j4) {
    f32x4 x;
#pragma unroll
    for (int j = 0; j < 4; ++j) x[j] = f * acc[4 * j4 + j];
    *reinterpret_cast<f32x4*>(xw + 32 * r32 + 4 * ((2 * j4 + h2) ^ (r32 & 7))) = x;
  }
  __builtin_amdgcn_wave_barrier();   // (a wave's LDS operations complete in order)
#pragma unroll
  for (int it = 0; it < 4; ++it) piece[it] = *reinterpret_cast<const f32x4*>(xw + 32 * (tr + 8 * it) + 4 * (c8 ^ tr));
  __builtin_amdgcn_wave_barrier();
}

}  // namespace

template <int D, bool SAVED>
__global__ __launch_bounds__(64 * kBw) void bwd_q2_kernel(BwdArgs a) {
  using L = BwL<D>;
  constexpr int KS = L::KS, DB = L::DB;
  constexpr int P = D + 8;
  __shared__ __attribute__((aligned(1024))) bf16 ks0[L::TILE], ks1[L::TILE];
  __shared__ __attribute__((aligned(1024))) bf16 vs0[L::TILE], vs1[L::TILE];
  __shared__ __attribute__((aligned(16))) bf16 ms[D * P];   // M_{s-1} [d_key][d_value] in bf16
  __shared__ float msum[D], zsh[D];                         // its column sums, z_{s-1}
  static_assert(4 * 64 * kBw * sizeof(float) <= sizeof(ks0), "the staging reduction fits a streamed tile");
  const int lane = threadIdx.x & 63, l32 = lane & 31, hh = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int NT = (a.N + kBwRows - 1) / kBwRows, npair = (NT + 1) / 2;
  const int id = xcd_logical_block(blockIdx.x, gridDim.x);
  const int pr = id % npair, sh = id / npair;    // sh = bh * S + s
  const int s = sh % a.S, bh = sh / a.S, h = bh % a.H;
  const int64_t seg0 = (int64_t)bh * a.L + (int64_t)s * a.N;
  const bool has_mem = a.seg_base + s > 0;
  const bf16* Q = static_cast<const bf16*>(a.q);
  const bf16* K = static_cast<const bf16*>(a.k) + seg0 * D;
  const bf16* V = static_cast<const bf16*>(a.v) + seg0 * D;
  const bf16* DO = static_cast<const bf16*>(a.dout);
  const float g = sigmoid_gate(a.beta[h]);
  const float omg = 1.f - g, sl2 = a.scale * kLog2e;
  // the memory the segment's queries read, staged once for both tiles (the first
  // streamed slot holds the reduction of its column sums; the staging ends with
  // a barrier before any load into that slot)
  if (threadIdx.x < D) zsh[threadIdx.x] = a.snapz[(int64_t)sh * D + threadIdx.x];
  stage_mat<D, 64 * kBw>(a.snapM + (int64_t)sh * D * D, ms, msum, reinterpret_cast<float*>(ks0));
  BwOfs<D> of;
  of.init(lane, w);
  auto issue = [&](int st, bf16* kd, bf16* vd) {
    bw_dma<D>(K + (int64_t)st * kBwStep * D, kd, w, of);
    bw_dma<D>(V + (int64_t)st * kBwStep * D, vd, w, of);
  };
  // Steps 0 .. ns-1 over the segment's first ns * 64 keys: step st sits in slot
  // st % 2; the loads of step st + 1 go out once every wave is done with step
  // st - 1, and are the only ones in flight when step st + 1 begins.
  auto ring = [&](int ns, auto&& compute) {
    issue(0, ks0, vs0);
    for (int st = 0; st < ns; st += 2) {
      bw_wait_sync<0>();
      if (st + 1 < ns) issue(st + 1, ks1, vs1);
      compute(ks0, vs0, st);
      if (st + 1 >= ns) break;
      bw_wait_sync<0>();
      if (st + 2 < ns) issue(st + 2, ks0, vs0);
      compute(ks1, vs1, st + 1);
    }
    bw_wait_sync<0>();   // every wave is done with the slots before they are refilled
  };
  for (int pass = 0; pass < 2; ++pass) {
    const int t = pass == 0 ? NT - 1 - pr : pr;   // the longer tile first
    if (pass == 1 && t == NT - 1 - pr) break;
    const int q0 = kBwRows * t, ns = min(a.N, q0 + kBwRows) / kBwStep;
    const int qw0 = q0 + 32 * w;
    const bool qvalid = qw0 < a.N;
    const int qcol = qw0 + l32;
    const int64_t qrow = seg0 + min(qcol, a.N - 1);
    bf16x8 qr[KS];
#pragma unroll
    for (int c = 0; c < KS; ++c) qr[c] = *reinterpret_cast<const bf16x8*>(Q + qrow * D + 16 * c + 8 * hh);

    // With the forward's output and log-normalisers (SAVED) the first sweep is
    // not needed: D = (1 - g) <dA, A_dot> = <dA, A> - g <dA, A_mem>, and <dA, A_mem>
    // comes with the retrieval below.
    float lse2 = 0.f, Dv = 0.f;
    if constexpr (!SAVED) {
      // ---- first sweep: statistics and A_dot^T of the wave's 32 query columns.
      // m is a reference maximum (log2 units) raised only when a block's maximum
      // exceeds it by more than 8, so probabilities stay below 2^8 and the rescale
      // of O and l is rare; the result is exact for any m.
      f32x16 o[DB];
#pragma unroll
      for (int d = 0; d < DB; ++d) o[d] = zero16();
      float m = -__builtin_inff(), l = 0.f;
      ring(ns, [&](const bf16* kt, const bf16* vt, int st) {
        if (!qvalid) return;
        of.opaque();
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const int kb = kBwStep * st + 32 * b;
          if (kb > qw0) break;   // the wave's queries see no key of this block (nor the next)
          f32x16 sc = zero16();
#pragma unroll
          for (int c = 0; c < KS; ++c) sc = mfma32(bw_row<D>(kt, of, c, 32 * b), qr[c], sc);
          const bool diag = kb + 31 > qw0;
          float mx = -__builtin_inff();
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float v = sc[r] * sl2;
            if (diag && kb + acc_row(r, hh) > qcol) v = -__builtin_inff();
            sc[r] = v;
            mx = fmaxf(mx, v);
          }
          mx = fmaxf(mx, __shfl_xor(mx, 32));   // finite: key kb precedes every query of the wave
          if (__ballot(mx > m + 8.f)) {
            const float mn = fmaxf(m, mx);
            const float al = bw_exp2(m - mn);
            l *= al;
#pragma unroll
            for (int d = 0; d < DB; ++d)
#pragma unroll
              for (int r = 0; r < 16; ++r) o[d][r] *= al;
            m = mn;
          }
          float ps = 0.f;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = bw_exp2(sc[r] - m);
            sc[r] = p;
            ps += p;
          }
          l += ps;
          const bf16x8 p0 = acc_op(sc, 0), p1 = acc_op(sc, 1);
#pragma unroll
          for (int d = 0; d < DB; ++d) {
            o[d] = mfma32(bw_tr<D>(vt, of, d, 32 * b), p0, o[d]);
            o[d] = mfma32(bw_tr<D>(vt, of, d, 32 * b + 16), p1, o[d]);
          }
        }
      });
      const float lt = l + __shfl_xor(l, 32);
      const float lse2s = m + __log2f(lt);
      // E = <dA, A_dot>: the lane holds 16 DB values of its query's row of O^T, in
      // runs of four
      float e = 0.f;
      if (qvalid) {
#pragma unroll
        for (int d = 0; d < DB; ++d)
#pragma unroll
          for (int j4 = 0; j4 < 4; ++j4) {
            const bf16x4 da = *reinterpret_cast<const bf16x4*>(DO + qrow * D + 32 * d + 8 * j4 + 4 * hh);
#pragma unroll
            for (int j = 0; j < 4; ++j) e = __builtin_fmaf(bf2f(da[j]), o[d][4 * j4 + j], e);
          }
      }
      e = (e + __shfl_xor(e, 32)) / lt;
      Dv = omg * e;
      lse2 = lse2s;
      if (qvalid && hh == 0) a.lse[qrow] = lse2;
    } else {
      lse2 = a.lse[qrow];
    }

    // ---- the retrieval's statistics of the wave's queries.  The lane's LDS
    // addresses are formed here, not hoisted to the kernel's entry where they
    // would stay live through the sweeps.
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int lh = ln >> 5;
    // q' = sigma(q) - 1 and the denominator sigma(q) z of the lane's query
    float den = 0.f;
    bf16x8 qm[KS];
#pragma unroll
    for (int c = 0; c < KS; ++c)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float x = bf2f(qr[c][j]);
        const float f = x > 0.f ? x : exp_e(x) - 1.f;
        qm[c][j] = f2bf(f);
        den = __builtin_fmaf(f + 1.f, zsh[16 * c + 8 * lh + j], den);
      }
    den += __shfl_xor(den, 32);
    const float inv_den = has_mem && den > 0.f ? 1.f / den : 0.f;
    // <dA, A_mem> with A_mem^T = (colsum(M) + M^T q'^T) / den; the lane holds 16 DB
    // values of its query's transposed row, in runs of four
    float em = 0.f, ea = 0.f;   // <dA, A_mem>, and (SAVED) <dA, A>
#pragma unroll
    for (int d = 0; d < DB; ++d) {
      f32x16 am = zero16();
      if (has_mem) {
#pragma unroll
        for (int c = 0; c < KS; ++c) am = mfma32(tr_nat(ms, P, 16 * c, 32 * d, ln), qm[c], am);
      }
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        const int col = 32 * d + 8 * j4 + 4 * lh;
        const bf16x4 da = *reinterpret_cast<const bf16x4*>(DO + qrow * D + col);
#pragma unroll
        for (int j = 0; j < 4; ++j) em = __builtin_fmaf(bf2f(da[j]), (msum[col + j] + am[4 * j4 + j]) * inv_den, em);
        if constexpr (SAVED) {
          const bf16x4 ao = *reinterpret_cast<const bf16x4*>(static_cast<const bf16*>(a.out_fw) + qrow * D + col);
#pragma unroll
          for (int j = 0; j < 4; ++j) ea = __builtin_fmaf(bf2f(da[j]), bf2f(ao[j]), ea);
        }
      }
    }
    em += __shfl_xor(em, 32);
    if constexpr (SAVED) Dv = (ea + __shfl_xor(ea, 32)) - g * em;
    const float rs = g * inv_den;
    const float dden = -g * em * inv_den;
    if (qvalid && hh == 0) {
      a.rs[qrow] = rs;
      a.dden[qrow] = dden;
      a.drow[qrow] = Dv;
    }
    {   // the gate's share of dbeta for the wave's 32 queries:
        // g (1 - g) sum (<dA, A_mem> - <dA, A_dot>) = g sum ((1 - g) <dA, A_mem> - D)
      const float bt = wave_sum(qvalid && hh == 0 ? omg * em - Dv : 0.f);
      if (qvalid && lane == 0) a.dbeta_part[((int64_t)bh * a.S + s) * a.nqb + qw0 / 32] = bt * g;
    }

    // ---- second sweep: dq^T += K^T dS^T
    bf16x8 dr[KS];
#pragma unroll
    for (int c = 0; c < KS; ++c) dr[c] = *reinterpret_cast<const bf16x8*>(DO + qrow * D + 16 * c + 8 * hh);
    f32x16 dq[DB];
#pragma unroll
    for (int d = 0; d < DB; ++d) dq[d] = zero16();
    ring(ns, [&](const bf16* kt, const bf16* vt, int st) {
      if (!qvalid) return;
      of.opaque();
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int kb = kBwStep * st + 32 * b;
        if (kb > qw0) break;
        f32x16 sc = zero16(), dp = zero16();
#pragma unroll
        for (int c = 0; c < KS; ++c) {
          sc = mfma32(bw_row<D>(kt, of, c, 32 * b), qr[c], sc);
          dp = mfma32(bw_row<D>(vt, of, c, 32 * b), dr[c], dp);
        }
        const bool diag = kb + 31 > qw0;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = bw_exp2(__builtin_fmaf(sc[r], sl2, -lse2));
          if (diag && kb + acc_row(r, hh) > qcol) p = 0.f;
          sc[r] = p * __builtin_fmaf(omg, dp[r], -Dv);
        }
        const bf16x8 d0 = acc_op(sc, 0), d1 = acc_op(sc, 1);
#pragma unroll
        for (int d = 0; d < DB; ++d) {
          dq[d] = mfma32(bw_tr<D>(kt, of, d, 32 * b), d0, dq[d]);
          dq[d] = mfma32(bw_tr<D>(kt, of, d, 32 * b + 16), d1, dq[d]);
        }
      }
    });
    // ---- the final dq = (M (rs dA)^T + dden z) sigma'(q) + scale dS K, in bf16:
    // M rows from LDS, rs dA (in place of dA) as the B operand
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int c = 0; c < KS; ++c)
#pragma unroll
      for (int j = 0; j < 8; ++j) dr[c][j] = f2bf(rs * bf2f(dr[c][j]));
    if (qvalid && D == 128) {
      // through a 4 KB tile per wave in the second ring slots (no load goes
      // there before the next sweep's first barrier): (M (rs dA)^T + dden z) and
      // scale dS K turned into row pieces (query tr + 8 it, columns 4 c8 ..
      // 4 c8 + 3), then sigma'(q) from the matching piece of Q
      float* xw = reinterpret_cast<float*>(w < 4 ? ks1 : vs1) + 1024 * (w & 3);
      const int vb = 2 * ((ln >> 3) * D + 4 * (ln & 7));
      const bf16* qw = Q + (seg0 + qw0) * D;
      bf16* dqw = static_cast<bf16*>(a.dq_out) + (seg0 + qw0) * D;
#pragma unroll
      for (int d = 0; d < DB; ++d) {
        bf16x4 xq[4];
#pragma unroll
        for (int it = 0; it < 4; ++it) xq[it] = wv_ld4<D>(qw, vb, 2 * (8 * it * D + 32 * d));
        f32x16 dm = zero16();
        if (has_mem) {   // wave-uniform; rows without memory have rs = dden = 0
#pragma unroll
          for (int c = 0; c < KS; ++c) dm = mfma32(row_op(ms, P, 32 * d, 16 * c, ln), dr[c], dm);
        }
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4)
#pragma unroll
          for (int j = 0; j < 4; ++j) dm[4 * j4 + j] += dden * zsh[32 * d + 8 * j4 + 4 * lh + j];
        f32x4 tm[4], ta[4];
        turn32(xw, dm, 1.f, ln, tm);
        turn32(xw, dq[d], a.scale, ln, ta);
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          bf16x4 o;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float x = bf2f(xq[it][j]);
            const float sp = x > 0.f ? 1.f : exp_e(x);
            o[j] = f2bf(__builtin_fmaf(tm[it][j], sp, ta[it][j]));
          }
          wv_st4<D>(dqw, vb, 2 * (8 * it * D + 32 * d), o);
        }
      }
    } else if (qvalid) {
#pragma unroll
      for (int d = 0; d < DB; ++d) {
        f32x16 dm = zero16();
        if (has_mem) {   // wave-uniform; rows without memory have rs = dden = 0
#pragma unroll
          for (int c = 0; c < KS; ++c) dm = mfma32(row_op(ms, P, 32 * d, 16 * c, ln), dr[c], dm);
        }
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4) {
          const int col = 32 * d + 8 * j4 + 4 * lh;
          const bf16x4 xq = *reinterpret_cast<const bf16x4*>(Q + qrow * D + col);
          bf16x4 o;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float x = bf2f(xq[j]);
            const float sp = x > 0.f ? 1.f : exp_e(x);
            o[j] = f2bf(__builtin_fmaf(a.scale, dq[d][4 * j4 + j], (dm[4 * j4 + j] + dden * zsh[col + j]) * sp));
          }
          *reinterpret_cast<bf16x4*>(static_cast<bf16*>(a.dq_out) + qrow * D + col) = o;
        }
      }
    }
  }
}

template <int D>
__global__ __launch_bounds__(64 * kBw) void bwd_kv2_kernel(BwdArgs a) {
  using L = BwL<D>;
  constexpr int KS = L::KS, DB = L::DB;
  __shared__ __attribute__((aligned(1024))) bf16 qs0[L::TILE], qs1[L::TILE];
  __shared__ __attribute__((aligned(1024))) bf16 es0[L::TILE], es1[L::TILE];   // dA rows
  __shared__ __attribute__((aligned(1024))) bf16 kst[kBwRows * D];              // the tile's keys
  __shared__ __attribute__((aligned(16))) float ld0[2 * kBwStep], ld1[2 * kBwStep];   // log2 normaliser, D
  const int lane = threadIdx.x & 63, l32 = lane & 31, hh = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int NT = (a.N + kBwRows - 1) / kBwRows, npair = (NT + 1) / 2;
  const int id = xcd_logical_block(blockIdx.x, gridDim.x);
  const int pr = id % npair, sh = id / npair;
  const int s = sh % a.S, bh = sh / a.S, h = bh % a.H;
  const int64_t seg0 = (int64_t)bh * a.L + (int64_t)s * a.N;
  const bf16* Q = static_cast<const bf16*>(a.q) + seg0 * D;
  const bf16* K = static_cast<const bf16*>(a.k) + seg0 * D;
  const bf16* V = static_cast<const bf16*>(a.v);
  const bf16* DO = static_cast<const bf16*>(a.dout) + seg0 * D;
  const float g = sigmoid_gate(a.beta[h]);
  const float omg = 1.f - g, sl2 = a.scale * kLog2e;
  BwOfs<D> of;
  of.init(lane, w);
  // queries q0 + 64 st .. of step st; each wave also brings 16 of the 64 log2
  // normalisers (waves 0-3) or D values (waves 4-7) with four lanes
  auto issue = [&](int q0, bf16* qd, bf16* ed, float* ldd) {
    bw_dma<D>(Q + (int64_t)q0 * D, qd, w, of);
    bw_dma<D>(DO + (int64_t)q0 * D, ed, w, of);
#if defined(__HIP_DEVICE_COMPILE__)
    if (lane < 4) {
      const float* src = (w < 4 ? a.lse : a.drow) + seg0 + q0 + 16 * (w & 3);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(bw_rsrc(src, 64), (INFINI_LDS void*)(ldd + 16 * w), 16, 16 * lane, 0,
                                               0, 0);
    }
#endif
  };
  for (int pass = 0; pass < 2; ++pass) {
    const int t = pass == 0 ? pr : NT - 1 - pr;   // the longer tile (more later queries) first
    if (pass == 1 && t == pr) break;
    const int k0 = kBwRows * t, nkeys = min(a.N - k0, kBwRows);
    const int kw0 = k0 + 32 * w;
    const bool kvalid = kw0 < a.N;
    const int kcol = kw0 + l32;
    const int64_t krow = seg0 + min(kcol, a.N - 1);
    const int ns = (a.N - k0) / kBwStep;
    // the tile's keys (64-row pieces) and the first step
    for (int p = 0; p < nkeys / kBwStep; ++p) bw_dma<D>(K + (int64_t)(k0 + kBwStep * p) * D, kst + p * L::TILE, w, of);
    issue(k0, qs0, es0, ld0);
    bf16x8 vr[KS];
#pragma unroll
    for (int c = 0; c < KS; ++c) vr[c] = *reinterpret_cast<const bf16x8*>(V + krow * D + 16 * c + 8 * hh);
    f32x16 dk[DB], dv[DB];
#pragma unroll
    for (int d = 0; d < DB; ++d) dk[d] = dv[d] = zero16();
    auto compute = [&](const bf16* qt, const bf16* et, const float* ldt, int st) {
      if (!kvalid) return;
      of.opaque();
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int qb = k0 + kBwStep * st + 32 * b;
        if (qb + 31 < kw0) continue;   // every query of the block precedes the wave's keys
        f32x16 sc = zero16(), dp = zero16();
#pragma unroll
        for (int c = 0; c < KS; ++c) {
          sc = mfma32(bw_row<D>(qt, of, c, 32 * b), bw_row<D>(kst, of, c, 32 * w), sc);
          dp = mfma32(bw_row<D>(et, of, c, 32 * b), vr[c], dp);
        }
        const bool diag = qb < kw0 + 31;
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4) {
          const f32x4 lq = *reinterpret_cast<const f32x4*>(ldt + 32 * b + 8 * j4 + 4 * hh);
          const f32x4 dq = *reinterpret_cast<const f32x4*>(ldt + kBwStep + 32 * b + 8 * j4 + 4 * hh);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int r = 4 * j4 + j;
            float p = bw_exp2(__builtin_fmaf(sc[r], sl2, -lq[j]));
            if (diag && kcol > qb + 8 * j4 + 4 * hh + j) p = 0.f;
            sc[r] = p;
            dp[r] = p * __builtin_fmaf(omg, dp[r], -dq[j]);
          }
        }
        const bf16x8 p0 = acc_op(sc, 0), p1 = acc_op(sc, 1), d0 = acc_op(dp, 0), d1 = acc_op(dp, 1);
#pragma unroll
        for (int d = 0; d < DB; ++d) {
          dv[d] = mfma32(bw_tr<D>(et, of, d, 32 * b), p0, dv[d]);
          dv[d] = mfma32(bw_tr<D>(et, of, d, 32 * b + 16), p1, dv[d]);
          dk[d] = mfma32(bw_tr<D>(qt, of, d, 32 * b), d0, dk[d]);
          dk[d] = mfma32(bw_tr<D>(qt, of, d, 32 * b + 16), d1, dk[d]);
        }
      }
    };
    // two slots: the loads of step st + 1 go out once every wave is done with
    // step st - 1, and are the only ones in flight when step st + 1 begins
    for (int st = 0; st < ns; st += 2) {
      bw_wait_sync<0>();
      if (st + 1 < ns) issue(k0 + kBwStep * (st + 1), qs1, es1, ld1);
      compute(qs0, es0, ld0, st);
      if (st + 1 >= ns) break;
      bw_wait_sync<0>();
      if (st + 2 < ns) issue(k0 + kBwStep * (st + 2), qs0, es0, ld0);
      compute(qs1, es1, ld1, st + 1);
    }
    bw_wait_sync<0>();
    if (!kvalid) continue;
    if constexpr (D == 128) {
      // The accumulators hold key l32 and columns 8 j4 + 4 hh + 0..3 of each
      // 32-column block; a 4 KB tile per wave in the second ring slots (no load
      // goes there before the next pass's first barrier) turns each block into
      // row pieces (key tr + 8 it, columns 4 c8 .. 4 c8 + 3: eight lanes per
      // 128-byte row piece).  The lane's offsets are formed here, not hoisted
      // into the sweep.
      int ln = lane;
      asm volatile("" : "+v"(ln));
      float* xw = reinterpret_cast<float*>(w < 4 ? qs1 : es1) + 1024 * (w & 3);
      const int vb = 4 * ((ln >> 3) * D + 4 * (ln & 7));
      float* dvw = a.dv_acc + (seg0 + kw0) * D;
      float* dkw = a.dk_acc + (seg0 + kw0) * D;
#pragma unroll
      for (int d = 0; d < DB; ++d) {
        f32x4 x[4];
        turn32(xw, dv[d], omg, ln, x);
#pragma unroll
        for (int it = 0; it < 4; ++it) wv_st4<D>(dvw, vb, 4 * (8 * it * D + 32 * d), x[it]);
        turn32(xw, dk[d], a.scale, ln, x);
#pragma unroll
        for (int it = 0; it < 4; ++it) wv_st4<D>(dkw, vb, 4 * (8 * it * D + 32 * d), x[it]);
      }
    } else {
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4) {
          const int64_t i = krow * D + 32 * d + 8 * j4 + 4 * hh;
          f32x4 xv, xk;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            xv[j] = omg * dv[d][4 * j4 + j];
            xk[j] = a.scale * dk[d][4 * j4 + j];
          }
          *reinterpret_cast<f32x4*>(a.dv_acc + i) = xv;
          *reinterpret_cast<f32x4*>(a.dk_acc + i) = xk;
        }
    }
  }
}

// Linear rule, per 256 tokens of a segment (one wave per 32), given G = dL/dM_s
// (fp32 [d_key][d_value], staged in LDS as bf16 with fp32 column sums) and
// dL/dz_s: the final dv and dk in bf16,
//   dv = dv_acc + sigma(K) G = dv_acc + colsum(G) + (sigma(K) - 1) G,
//   dk = dk_acc + (V G^T + dL/dz_s) sigma'(K).
template <int D>
__global__ __launch_bounds__(64 * kUpdWaves) void bwd_lin_update_mfma_kernel(BwdArgs a) {
  constexpr int P = D + 8, KS = D / 16, DB = D / 32;
  const int rb = blockIdx.x, s = blockIdx.y, bh = blockIdx.z;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, l32 = lane & 31, hh = lane >> 5;
  const bf16* K = static_cast<const bf16*>(a.k);
  const bf16* V = static_cast<const bf16*>(a.v);
  __shared__ __attribute__((aligned(16))) bf16 gs[D * P];
  __shared__ __attribute__((aligned(16))) float red[4 * 64 * kUpdWaves];
  __shared__ float gsum[D];
  __shared__ __attribute__((aligned(16))) float xt[kUpdWaves][32 * kXtP];   // each wave's transposing tile
  stage_mat<D, 64 * kUpdWaves>(a.dMr + ((int64_t)bh * a.S + s) * D * D, gs, gsum, red);
  const int t0 = rb * kUpdBlock + 32 * w;           // the wave's first token in the segment
  if (t0 >= a.N) return;                            // (after the staging's barriers)
  // a valid wave's 32 tokens all lie in the segment
  const int64_t out0 = (int64_t)bh * a.L + (int64_t)s * a.N + t0;
  const int64_t row = out0 + l32;
  const float* gz = a.gzs + ((int64_t)bh * a.S + s) * D;   // dL/dz_s, which every sigma(k) of the segment adds to
  // The products leave token (acc_row(r, hh)) x column (l32) in the accumulators;
  // the wave's own LDS tile turns a 32 x 32 block around so that the lane takes
  // rows tr + 8 it, columns tc .. tc + 3 (eight lanes per 128-byte row piece).
  // The epilogue's loads of block d + 1 go out before the stores of block d.
  float* xw = xt[w];
  const int tr = lane >> 3, tc = 4 * (lane & 7);
  auto turn = [&](const f32x16& acc, f32x4* out) {
#pragma unroll
    for (int r = 0; r < 16; ++r) xw[acc_row(r, hh) * kXtP + l32] = acc[r];
    __builtin_amdgcn_wave_barrier();   // (a wave's LDS operations complete in order)
#pragma unroll
    for (int it = 0; it < 4; ++it) out[it] = *reinterpret_cast<const f32x4*>(xw + (tr + 8 * it) * kXtP + tc);
    __builtin_amdgcn_wave_barrier();
  };
  // dk = dk_acc + (V G^T + dL/dz_s) sigma'(K)
  {
    bf16x8 vr[KS];
#pragma unroll
    for (int c = 0; c < KS; ++c) vr[c] = *reinterpret_cast<const bf16x8*>(V + row * D + 16 * c + 8 * hh);
    f32x4 xa[2][4];
    bf16x4 xk[2][4];
    auto load = [&](int d, f32x4* pa, bf16x4* pk) {
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int64_t i = (out0 + tr + 8 * it) * D + 32 * d + tc;
        pa[it] = *reinterpret_cast<const f32x4*>(a.dk_acc + i);
        pk[it] = *reinterpret_cast<const bf16x4*>(K + i);
      }
    };
    load(0, xa[0], xk[0]);
#pragma unroll
    for (int d = 0; d < DB; ++d) {
      f32x16 df = zero16();
#pragma unroll
      for (int c = 0; c < KS; ++c) df = mfma32(vr[c], row_op(gs, P, 32 * d, 16 * c, lane), df);
      f32x4 dt[4];
      turn(df, dt);
      if (d + 1 < DB) load(d + 1, xa[(d + 1) & 1], xk[(d + 1) & 1]);
      const f32x4 gzc = *reinterpret_cast<const f32x4*>(gz + 32 * d + tc);
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        bf16x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float x = bf2f(xk[d & 1][it][j]);
          const float sp = x > 0.f ? 1.f : exp_e(x);
          o[j] = f2bf(__builtin_fmaf(dt[it][j] + gzc[j], sp, xa[d & 1][it][j]));
        }
        *reinterpret_cast<bf16x4*>(static_cast<bf16*>(a.dk_out) + (out0 + tr + 8 * it) * D + 32 * d + tc) = o;
      }
    }
  }
  // dv = dv_acc + sigma(K) G = dv_acc + colsum(G) + (sigma(K) - 1) G
  bf16x8 kp[KS];
#pragma unroll
  for (int c = 0; c < KS; ++c) {
    const bf16x8 kx = *reinterpret_cast<const bf16x8*>(K + row * D + 16 * c + 8 * hh);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float x = bf2f(kx[j]);
      kp[c][j] = f2bf(x > 0.f ? x : exp_e(x) - 1.f);
    }
  }
  f32x4 xa[2][4];
  auto load = [&](int d, f32x4* pa) {
#pragma unroll
    for (int it = 0; it < 4; ++it) pa[it] = *reinterpret_cast<const f32x4*>(a.dv_acc + (out0 + tr + 8 * it) * D + 32 * d + tc);
  };
  load(0, xa[0]);
#pragma unroll
  for (int d = 0; d < DB; ++d) {
    f32x16 dv = zero16();
#pragma unroll
    for (int c = 0; c < KS; ++c) dv = mfma32(kp[c], tr_nat(gs, P, 16 * c, 32 * d, lane), dv);
    f32x4 dt[4];
    turn(dv, dt);
    if (d + 1 < DB) load(d + 1, xa[(d + 1) & 1]);
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      bf16x4 o;
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = f2bf(xa[d & 1][it][j] + (gsum[32 * d + tc + j] + dt[it][j]));
      *reinterpret_cast<bf16x4*>(static_cast<bf16*>(a.dv_out) + (out0 + tr + 8 * it) * D + 32 * d + tc) = o;
    }
  }
}

// A per-segment Gram product on MFMA, two workgroups per segment (each half of
// the 64-token chunks; the second writes its partial into gpart and a combining
// pass adds it, so the sums keep a fixed order), both operands read transposed
// from LDS:
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
  const int s = blockIdx.x, bh = blockIdx.y, part = blockIdx.z;   // part: which half of the token chunks
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const bf16* X = static_cast<const bf16*>(RETR ? a.q : a.k);
  const bf16* Y = static_cast<const bf16*>(a.dout);
  __shared__ __attribute__((aligned(16))) bf16 xs[kChunk * P];
  __shared__ __attribute__((aligned(16))) bf16 ys[kChunk * P];
  __shared__ float zsh[D], ush[D], wred[kChunk];
  __shared__ float red[kChunk * D];   // the column sums' partials, one row per token thread
  const int64_t seg = (int64_t)bh * a.S + s;
  const int64_t nseg = (int64_t)a.BH * a.S;
  // the first half writes the result in place, the second its partial into gpart
  float* out = (part ? a.gpart : (RETR ? a.dMr : a.Amat)) + seg * D * D;
  float* zout = part ? a.gpart + nseg * D * D : a.dzr;
  if (!RETR && a.seg_base + s == 0) {
    for (int i = t; i < D * D; i += 64 * kBwdWaves) out[i] = 0.f;
    return;
  }
  if (t < D) zsh[t] = RETR ? 0.f : a.snapz[seg * D + t];
  f32x16 acc[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) acc[i] = zero16();
  const int64_t seg0 = (int64_t)bh * a.L + (int64_t)s * a.N;
  const int tt = t >> 2, qq = t & 3;   // staging: token tt, quarter qq of its row
  constexpr int QW = D / 4;
  // column sums, accumulated by each staging thread over its tokens (from the
  // fp32 inputs for the retrieval: sum_t rs_t dA_t and sum_t dden_t sigma(q_t);
  // from the bf16 K' of the product for A_s) and met across the threads at the end
  float up[QW], zp[QW], wsum = 0.f;
#pragma unroll
  for (int j = 0; j < QW; ++j) up[j] = zp[j] = 0.f;
  __syncthreads();
  const int nch = a.N / kChunk, chalf = (nch + 1) / 2;
  const int c0 = part ? chalf : 0, c1 = part ? nch : chalf;
  for (int t0 = c0 * kChunk; t0 < c1 * kChunk; t0 += kChunk) {
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
    float wt, dd = 0.f;
    if (RETR) {
      wt = a.rs[row];
      dd = a.dden[row];
    } else {
      e += __shfl_xor(e, 1);
      e += __shfl_xor(e, 2);
      wt = e > 0.f ? 1.f / e : 0.f;
    }
    wsum += wt;
#pragma unroll
    for (int i = 0; i < QW / 8; ++i) {
      bf16x8 xb, yb;
      if (RETR) {
        const bf16x8 y = *reinterpret_cast<const bf16x8*>(Y + row * D + qq * QW + 8 * i);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float yv = bf2f(y[j]);
          xb[j] = f2bf(xv[8 * i + j]);
          yb[j] = f2bf(wt * yv);
          up[8 * i + j] = __builtin_fmaf(wt, yv, up[8 * i + j]);
          zp[8 * i + j] = __builtin_fmaf(dd, xv[8 * i + j] + 1.f, zp[8 * i + j]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          xb[j] = f2bf(xv[8 * i + j]);
          yb[j] = f2bf(wt * xv[8 * i + j]);
          up[8 * i + j] = __builtin_fmaf(wt, bf2f(xb[j]), up[8 * i + j]);
        }
      }
      *reinterpret_cast<bf16x8*>(xs + tt * P + qq * QW + 8 * i) = xb;
      *reinterpret_cast<bf16x8*>(ys + tt * P + qq * QW + 8 * i) = yb;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int tile = w * TPW + i, bi = tile / NT, bj = tile % NT;
#pragma unroll
      for (int ks = 0; ks < kChunk / 16; ++ks)
        acc[i] = mfma32(tr_nat(xs, P, 16 * ks, 32 * bi, lane), tr_nat(ys, P, 16 * ks, 32 * bj, lane), acc[i]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int j = 0; j < QW; ++j) red[tt * D + qq * QW + j] = up[j];
  if (qq == 0) wred[tt] = wsum;
  __syncthreads();
  float colsum = 0.f, wtot = 0.f;
  if (t < D)
    for (int r = 0; r < kChunk; ++r) colsum += red[r * D + t];
  for (int r = 0; r < kChunk; ++r) wtot += wred[r];
  if (RETR) {
    __syncthreads();
#pragma unroll
    for (int j = 0; j < QW; ++j) red[tt * D + qq * QW + j] = zp[j];
    __syncthreads();
    if (t < D) {
      float z = 0.f;
      for (int r = 0; r < kChunk; ++r) z += red[r * D + t];
      zout[seg * D + t] = z;
    }
  }
  if (t < D) ush[t] = colsum;
  __syncthreads();
  const float ws = wtot;
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

// Delta rule, per 256 tokens of a segment (one wave per 32, lanes = tokens),
// given G = dL/dM_s (in dMr after the backward chain), M_{s-1}, z_{s-1}:
//   dU = sigma(K) G,  R = sigma(K) M_{s-1} / e (0 in the first segment),
//   U = V - R;  dv += dU;  d sigma(K) = U G^T - M_{s-1} (dU / e)^T;
//   de_t = <dU_t, R_t> / e_t  (the gradient of the token's denominator).
// Transposed products (d_value x tokens) keep every register operand in the
// accumulator layout of the product that consumes it.
template <int D>
__global__ __launch_bounds__(64 * kDuWaves) void bwd_delta_update_mfma_kernel(BwdArgs a) {
  constexpr int P = D + 8, KS = D / 16, DB = D / 32;
  const int rb = blockIdx.x, s = blockIdx.y, bh = blockIdx.z;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, l32 = lane & 31, hh = lane >> 5;
  const bf16* K = static_cast<const bf16*>(a.k);
  const bf16* V = static_cast<const bf16*>(a.v);
  __shared__ __attribute__((aligned(16))) bf16 gs[D * P];
  __shared__ __attribute__((aligned(16))) bf16 msb[D * P];
  __shared__ __attribute__((aligned(16))) float red[4 * 64 * kDuWaves];
  __shared__ float gsum[D], msum[D], zsh[D];
  __shared__ __attribute__((aligned(16))) float xt[kDuWaves][32 * kXtP];   // each wave's transposing tile
  const int64_t seg = (int64_t)bh * a.S + s;
  if (threadIdx.x < D) zsh[threadIdx.x] = a.snapz[seg * D + threadIdx.x];
  stage_mat<D, 64 * kDuWaves>(a.dMr + seg * D * D, gs, gsum, red);
  stage_mat<D, 64 * kDuWaves>(a.snapM + seg * D * D, msb, msum, red);
  const bool first = a.seg_base + s == 0;
  const int t0 = rb * kDuBlock + 32 * w;
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
  // A valid wave's 32 tokens all lie in the segment.  The products hold token
  // l32 and columns 8 j4 + 4 hh + 0..3 of a 32-column block per lane; global
  // memory is read and written in row pieces (token tr + 8 it, columns tc ..
  // tc + 3: eight lanes per 128-byte row piece), turned around in the wave's own
  // LDS tile.  The loads of block d + 1 go out before the stores of block d.
  const int64_t out0 = row - l32;
  const int tr = lane >> 3, tc = 4 * (lane & 7);
  float* xw = xt[w];
  auto to_acc = [&](const f32x4* piece, f32x4* run) {
#pragma unroll
    for (int it = 0; it < 4; ++it) *reinterpret_cast<f32x4*>(xw + (tr + 8 * it) * kXtP + tc) = piece[it];
    __builtin_amdgcn_wave_barrier();   // (a wave's LDS operations complete in order)
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) run[j4] = *reinterpret_cast<const f32x4*>(xw + l32 * kXtP + 8 * j4 + 4 * hh);
    __builtin_amdgcn_wave_barrier();
  };
  auto to_rows = [&](const f32x4* run, f32x4* piece) {
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) *reinterpret_cast<f32x4*>(xw + l32 * kXtP + 8 * j4 + 4 * hh) = run[j4];
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int it = 0; it < 4; ++it) piece[it] = *reinterpret_cast<const f32x4*>(xw + (tr + 8 * it) * kXtP + tc);
    __builtin_amdgcn_wave_barrier();
  };
  f32x4 pa[4];   // local attention's dv
  bf16x4 pv[4];  // V
  // element (tr + 8 it, 32 d + tc) of the wave's rows: lane part ve, constant part
  const int ve = tr * D + tc;
  const float* dva = a.dv_acc + out0 * D;
  const bf16* vw = V + out0 * D;
  bf16* dvo = static_cast<bf16*>(a.dv_out) + out0 * D;
  float* dfo = a.dfk_acc + out0 * D;
  auto load = [&](int d, f32x4* a4, bf16x4* v4) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int se = 8 * it * D + 32 * d;
      a4[it] = wv_ld4<D>(dva, 4 * ve, 4 * se);
      v4[it] = wv_ld4<D>(vw, 2 * ve, 2 * se);
    }
  };
  load(0, pa, pv);
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
    f32x4 dvl[4], vvf[4], tmp[4];
    to_acc(pa, dvl);
#pragma unroll
    for (int it = 0; it < 4; ++it)
#pragma unroll
      for (int j = 0; j < 4; ++j) tmp[it][j] = bf2f(pv[it][j]);
    to_acc(tmp, vvf);
    if (d + 1 < DB) load(d + 1, pa, pv);
    f32x16 u, dw;
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {   // accumulator rows come in runs of four columns
      const int col = 32 * d + 8 * j4 + 4 * hh;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 4 * j4 + j;
        const float dut = du[r] + gsum[col + j];
        const float R = first ? 0.f : (re[r] + msum[col + j]) * wt;
        tmp[j4][j] = dvl[j4][j] + dut;
        u[r] = vvf[j4][j] - R;
        dw[r] = -dut * wt;
        de = __builtin_fmaf(dut, R, de);
      }
    }
    ub[d][0] = acc_op(u, 0);
    ub[d][1] = acc_op(u, 1);
    db[d][0] = acc_op(dw, 0);
    db[d][1] = acc_op(dw, 1);
    to_rows(tmp, dvl);
#pragma unroll
    for (int it = 0; it < 4; ++it) {   // the final dv
      bf16x4 o;
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = f2bf(dvl[it][j]);
      wv_st4<D>(dvo, 2 * ve, 2 * (8 * it * D + 32 * d), o);
    }
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
    f32x4 run[4], piece[4];
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4)
#pragma unroll
      for (int j = 0; j < 4; ++j) run[j4][j] = df[4 * j4 + j];
    to_rows(run, piece);
#pragma unroll
    for (int it = 0; it < 4; ++it) wv_st4<D>(dfo, 4 * ve, 4 * (8 * it * D + 32 * d2), piece[it]);
  }
}

int bwd_mfma_blocks(int N) { return (N + kUpdBlock - 1) / kUpdBlock; }

template <int D>
hipError_t launch_backward_attention_mfma(const BwdArgs& a, hipStream_t stream) {
  // the query kernel writes dq, rs, dden, dbeta's shares and the softmax
  // statistics the key kernel reads
  hipError_t e;
  const int64_t npair = ((a.N + kBwRows - 1) / kBwRows + 1) / 2;
  const int64_t nblk = npair * a.S * a.BH;
  if (nblk > 0x7fffffff) return hipErrorInvalidValue;
  if (a.out_fw) hipLaunchKernelGGL((bwd_q2_kernel<D, true>), dim3((unsigned)nblk), dim3(64 * kBw), 0, stream, a);
  else hipLaunchKernelGGL((bwd_q2_kernel<D, false>), dim3((unsigned)nblk), dim3(64 * kBw), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_kv2_kernel<D>, dim3((unsigned)nblk), dim3(64 * kBw), 0, stream, a);
  return hipGetLastError();
}
template hipError_t launch_backward_attention_mfma<64>(const BwdArgs&, hipStream_t);
template hipError_t launch_backward_attention_mfma<128>(const BwdArgs&, hipStream_t);

template <int D>
hipError_t launch_backward_lin_update_mfma(const BwdArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)bwd_mfma_blocks(a.N), (unsigned)a.S, (unsigned)a.BH);
  hipLaunchKernelGGL(bwd_lin_update_mfma_kernel<D>, grid, dim3(64 * kUpdWaves), 0, stream, a);
  return hipGetLastError();
}
template hipError_t launch_backward_lin_update_mfma<64>(const BwdArgs&, hipStream_t);
template hipError_t launch_backward_lin_update_mfma<128>(const BwdArgs&, hipStream_t);

// Adds the second halves' partials of the Gram kernel: out += part (n floats),
// and for the retrieval zout += zpart (nz floats), four at a time.
__global__ __launch_bounds__(256) void bwd_gram_combine_kernel(float* out, const float* part, int64_t n4,
                                                               float* zout, const float* zpart, int64_t nz4) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4 + nz4; i += (int64_t)gridDim.x * 256) {
    f32x4* o = reinterpret_cast<f32x4*>(i < n4 ? out : zout) + (i < n4 ? i : i - n4);
    const f32x4 p = reinterpret_cast<const f32x4*>(i < n4 ? part : zpart)[i < n4 ? i : i - n4];
    f32x4 x = *o;
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] += p[e];
    *o = x;
  }
}

template <int D, bool RETR>
static hipError_t launch_gram(const BwdArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((bwd_gram_kernel<D, RETR>), dim3((unsigned)a.S, (unsigned)a.BH, 2u), dim3(64 * kBwdWaves), 0,
                     stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t nseg = (int64_t)a.BH * a.S, n4 = nseg * D * D / 4, nz4 = RETR ? nseg * D / 4 : 0;
  const int64_t blocks = std::min<int64_t>((n4 + nz4 + 255) / 256, 1 << 16);
  hipLaunchKernelGGL(bwd_gram_combine_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     RETR ? a.dMr : a.Amat, a.gpart, n4, a.dzr, a.gpart + nseg * D * D, nz4);
  return hipGetLastError();
}

template <int D>
hipError_t launch_backward_delta_amat_mfma(const BwdArgs& a, hipStream_t stream) {
  return launch_gram<D, false>(a, stream);
}
template <int D>
hipError_t launch_backward_delta_update_mfma(const BwdArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)((a.N + kDuBlock - 1) / kDuBlock), (unsigned)a.S, (unsigned)a.BH);
  hipLaunchKernelGGL(bwd_delta_update_mfma_kernel<D>, grid, dim3(64 * kDuWaves), 0, stream, a);
  return hipGetLastError();
}
template <int D>
hipError_t launch_backward_retrieval_grad_mfma(const BwdArgs& a, hipStream_t stream) {
  return launch_gram<D, true>(a, stream);
}
template hipError_t launch_backward_retrieval_grad_mfma<64>(const BwdArgs&, hipStream_t);
template hipError_t launch_backward_retrieval_grad_mfma<128>(const BwdArgs&, hipStream_t);
template hipError_t launch_backward_delta_amat_mfma<64>(const BwdArgs&, hipStream_t);
template hipError_t launch_backward_delta_amat_mfma<128>(const BwdArgs&, hipStream_t);
template hipError_t launch_backward_delta_update_mfma<64>(const BwdArgs&, hipStream_t);
template hipError_t launch_backward_delta_update_mfma<128>(const BwdArgs&, hipStream_t);

}  // namespace infini
