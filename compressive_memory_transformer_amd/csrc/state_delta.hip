// Delta-rule memory state for the bf16 path (page "精读笔记：Infini-attention",
// section 3.4, delta rule; page "忘记遗忘：解锁无限上下文的 Infini-attention",
// section 2.1, for the unambiguous fraction; z as in section 3.3):
//   U_s = V_s - sigma(K_s) M_{s-1} / (sigma(K_s) z_{s-1})       (0 / 0 read as 0)
//   M_s = M_{s-1} + sigma(K_s)^T U_s,   z_s = z_{s-1} + sum_t sigma(K_s[t])
// with sigma(x) = ELU(x) + 1.  With w_t = 1 / (sigma(K_t) . z_{s-1}) (0 in a
// stream's first segment and for a zero denominator) this is the matrix
// recurrence
//   M_s = M_{s-1} + C_s - A_s M_{s-1},   C_s = sigma(K_s)^T V_s,
//   A_s = sigma(K_s)^T diag(w) sigma(K_s)   (d_key x d_key, symmetric),
// whose only sequential part is one d x d product per segment.  Everything else
// runs in parallel over all segments first:
//   lin_contrib (the linear rule's kernel): C_s and c_s = sum_t sigma(K_t);
//   delta_zscan: z_{s-1} of every segment (a prefix over the c_s), the final z;
//   delta_amat:  A_s = X^T X with X = sqrt(w) sigma(K) rounded to bf16, fp32
//                sums on MFMA, stored as an exact pair of bf16 parts hi + lo;
// then delta_chain, per (b, h) and 16 columns of M, walks the S segments:
//   P_s = P_{s-1} + C_s^T - P_{s-1} A_s     (P = M^T restricted to 16 rows)
// with the product on MFMA from hi/lo parts of both factors
// (P_hi A_hi + P_lo A_hi + P_hi A_lo, about 16 bits each), and emits the
// snapshot of every M_{s-1} for the fused attention kernel.
//
// Precision (float simulation of this arithmetic against float64, 48-256
// segments of the workloads' inputs and of keys around -3): final M within
// 2-3e-5 relative; bf16 factors without the lo parts in the chain give 1e-4.
// The hi/lo split keeps its precision for sigma near 1 (keys near 0) and for
// sigma << 1 (strongly negative keys) alike.
#include "common.h"
#include "kernels.h"
#include "mfma_ops.h"

namespace infini {

// z_{s-1} of every segment (snapshots) and the final z: a prefix over the
// segments of one head, one thread per d_key entry, in a fixed order.  The
// per-segment sums are loaded 32 at a time (independent loads at clamped
// indices), so they overlap instead of forming one dependent chain.
template <int D>
__global__ __launch_bounds__(D)
void delta_zscan_kernel(DeltaArgs a) {
  constexpr int kBatch = 32;
  const int bh = blockIdx.x, dk = threadIdx.x;
  const float* cz = a.cz + (int64_t)bh * a.S * D + dk;
  float* sz = a.snapz + (int64_t)bh * a.S * D + dk;
  float z = a.z[(int64_t)bh * D + dk];
  for (int s0 = 0; s0 < a.S; s0 += kBatch) {
    float c[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) c[i] = cz[(int64_t)min(s0 + i, a.S - 1) * D];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      if (s0 + i < a.S) {
        sz[(int64_t)(s0 + i) * D] = z;
        z += c[i];
      }
    }
  }
  a.z[(int64_t)bh * D + dk] = z;
}

// ------------------------------------------------------------------ A_s
namespace {
constexpr int kAmThreads = 256;   // 4 waves
constexpr int kAmT = 64;          // tokens per stage

template <int D>
struct AmCfg {
  static constexpr int TPT = kAmThreads / kAmT;   // threads per token
  static constexpr int EPT = D / TPT;             // elements of a token per thread
  static constexpr int CPT = EPT / 8;             // 16-byte chunks per thread
  static constexpr int NB = D / 32;               // 32-wide blocks of d_key
  static constexpr int TW = NB * NB / 4;          // 32 x 32 output tiles per wave
  static_assert(TW >= 1 && CPT >= 1, "shape");
};
}  // namespace

// A_s = X^T X, X = bf16(sqrt(w_t) sigma(K_t)) for the tokens t of one (b, h,
// segment); one workgroup (4 waves) per segment.  64-token stages of K are loaded
// into registers one stage ahead; per stage each group of four threads forms one
// token's sigma, its denominator sigma . z_{s-1} (a four-lane reduction) and its
// row of X, written to LDS in the layout of the transposing operand reads; the
// products run on v_mfma_f32_32x32x16_bf16 (tile (m, n) of A: the 32-column blocks
// m and n of X as the two operands).  Stored as bf16 hi [D][D] then lo [D][D].
template <int D>
__global__ __launch_bounds__(kAmThreads, 2)
void delta_amat_kernel(DeltaArgs a) {
  using C = AmCfg<D>;
  __shared__ __attribute__((aligned(16))) bf16 xs0[kAmT * D];
  __shared__ __attribute__((aligned(16))) bf16 xs1[kAmT * D];
  __shared__ float zs[D];
  const int sh = blockIdx.x;
  const int bh = sh / a.S, s = sh % a.S;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  bf16* __restrict__ ahi = a.amat + (int64_t)sh * 2 * D * D;
  bf16* __restrict__ alo = ahi + D * D;
  if (a.seg_base + s == 0) {   // a stream's first segment reads an empty memory: A = 0
    bf16x8 zero;
#pragma unroll
    for (int j = 0; j < 8; ++j) zero[j] = f2bf(0.f);
    for (int i = t; i < 2 * D * D / 8; i += kAmThreads) *reinterpret_cast<bf16x8*>(ahi + 8 * i) = zero;
    return;
  }
  if (t < D) zs[t] = a.snapz[(int64_t)sh * D + t];
  __syncthreads();
  const int tok = t / C::TPT, part = t % C::TPT;
  // Thread (tok, part) holds the logical 16-byte chunks TPT c + part, c < CPT, of
  // its token: the TPT threads of a token read one contiguous piece per load, and
  // the 16 lanes of an LDS write (four tokens x four parts) land on 16 distinct
  // bank groups under the XOR swizzle of the X layout.
  float zr[C::EPT];
#pragma unroll
  for (int c = 0; c < C::CPT; ++c)
#pragma unroll
    for (int j = 0; j < 8; ++j) zr[8 * c + j] = zs[8 * (C::TPT * c + part) + j];
  const bf16* kseg = a.k + ((int64_t)bh * a.L + (int64_t)s * a.N) * D;
  const int nst = a.N / kAmT;

  // this wave's tiles (m, n) = (i / NB, i % NB), i = wave * TW + j
  int offA[C::TW], offB[C::TW];
#pragma unroll
  for (int j = 0; j < C::TW; ++j) {
    const int i = wave * C::TW + j;
    offA[j] = trt_offset<D>(lane, i / C::NB);
    offB[j] = trt_offset<D>(lane, i % C::NB);
  }
  f32x16 acc[C::TW];
#pragma unroll
  for (int j = 0; j < C::TW; ++j) acc[j] = mo_zero();

  bf16x8 raw[C::CPT];
  auto load = [&](int q) {   // stage q's K chunks of this thread (clamped: a load past the end is unused)
    const int qq = q < nst ? q : nst - 1;
    const bf16* p = kseg + ((int64_t)qq * kAmT + tok) * D + 8 * part;
#pragma unroll
    for (int c = 0; c < C::CPT; ++c) raw[c] = *reinterpret_cast<const bf16x8*>(p + 8 * C::TPT * c);
  };
  auto convert = [&](bf16* X) {   // row tok of X from the raw K chunks
    float f[C::EPT];
    float den = 0.f;
#pragma unroll
    for (int c = 0; c < C::CPT; ++c)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float x = bf2f(raw[c][j]);
        const float sg = x > 0.f ? x + 1.f : exp_e(x);
        f[8 * c + j] = sg;
        den = __builtin_fmaf(sg, zr[8 * c + j], den);
      }
    den += __shfl_xor(den, 1);
    den += __shfl_xor(den, 2);
    const float sw = den > 0.f ? rsqrtf(den) : 0.f;
#pragma unroll
    for (int c = 0; c < C::CPT; ++c) {
      bf16x8 o;
#pragma unroll
      for (int j = 0; j < 8; ++j) o[j] = f2bf(sw * f[8 * c + j]);
      const int phys = trt_chunk<D>(tok, C::TPT * c + part);
      *(INFINI_LDS bf16x8*)(X + tok * D + 8 * phys) = o;
    }
  };
  // Stage q: row tok of X into its buffer, the next stage's loads, then the
  // products.  A buffer is rewritten two stages after it was read, and every wave
  // has passed the barrier of the stage in between.
#define INFINI_AM_STAGE(Q, X)                                                     \
  if ((Q) < nst) {                                                                \
    convert(X);                                                                   \
    load((Q) + 1);                                                                \
    lds_sync();                                                                   \
    _Pragma("unroll")                                                             \
    for (int st = 0; st < kAmT / 16; ++st) {                                      \
      const bf16* base = X + 16 * st * D;                                         \
      _Pragma("unroll")                                                           \
      for (int j = 0; j < C::TW; ++j)                                             \
        acc[j] = mfma32(trt_read<D>(base, offA[j]), trt_read<D>(base, offB[j]), acc[j]); \
    }                                                                             \
  }
  load(0);
  for (int q = 0; q < nst; q += 2) {
    INFINI_AM_STAGE(q, xs0)
    INFINI_AM_STAGE(q + 1, xs1)
  }
#undef INFINI_AM_STAGE
  const int hi = lane >> 5, l32 = lane & 31;
#pragma unroll
  for (int j = 0; j < C::TW; ++j) {
    const int i = wave * C::TW + j, m = i / C::NB, n = i % C::NB;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 32 * m + mo_acc_row(r, hi), col = 32 * n + l32;
      const bf16 h = f2bf(acc[j][r]);
      ahi[row * D + col] = h;
      alo[row * D + col] = f2bf(acc[j][r] - bf2f(h));
    }
  }
}

// ------------------------------------------------------------------- chain
namespace {
template <int D>
struct ChainCfg {
  static constexpr int NW = D / 16;     // waves: one 16-column tile of P A each
  static constexpr int NT = 64 * NW;    // threads
  static constexpr int KS = D / 32;     // 32-deep steps of the product
  static constexpr int LDP = D + 4;     // row pitch of the fp32 stage of P (floats)
  static constexpr int LDB = D + 8;     // row pitch of the bf16 planes of P (elements)
  static constexpr int TPR = NT / 16;   // threads per row of P in the snapshot pass
  static constexpr int EPR = D / TPR;   // elements per thread in the snapshot pass
  static_assert(EPR == 4, "the snapshot pass moves four elements per thread");
};

// v moved across the lanes of each row of 16 by the DPP control CTRL.
template <int CTRL>
__device__ __forceinline__ float dpp_row(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
// Sum over each row of 16 lanes by DPP lane moves (quad sums, then the half rows
// and the rows by mirrors); every lane of the row gets the sum.
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_row<0xB1>(x);    // quad_perm [1, 0, 3, 2]
  x += dpp_row<0x4E>(x);    // quad_perm [2, 3, 0, 1]
  x += dpp_row<0x141>(x);   // row_half_mirror
  x += dpp_row<0x140>(x);   // row_mirror
  return x;
}

// Operands of one segment's step for one lane: row col of A_s (bf16 hi and lo,
// k = 32 ks + 8 (l / 16) ..) and C_s^T at rows 4 (l / 16) + r, column col.
template <int D>
struct ChainOps {
  bf16x8 h[D / 32];
  bf16x8 l[D / 32];
  float c[4];
};
}  // namespace

// The chain over the segments of one head for 16 columns of M (rows of P = M^T;
// the columns of M are independent: column j of A_s M needs only column j of M).
// One workgroup of D / 16 waves per (b, h, column block); wave w computes the
// 16 x 16 tile (rows of the block) x (d_key columns 16 w ..) of P A on
// v_mfma_f32_16x16x32_bf16.  Each step:
//   each wave writes its tile of P (fp32, accumulator layout in registers) into
//   LDS as bf16 hi and lo planes, and its partial row sums (a 16-lane DPP sum);
//   snapshot of M_{s-1}: its 16 rows of M^T in bf16 with their bf16 remainders
//   straight from the planes, and their sums (column sums of M over d_key, the
//   waves' partials added), for the fused kernel;
//   A operand P_hi, P_lo from the planes; B operands A_hi, A_lo straight from
//   memory (A_s is symmetric, so row n of A_s is column n);
//   P += C_s^T - (P_hi A_hi + P_lo A_hi + P_hi A_lo).
// The operands of the next two segments are loaded into registers ahead of
// their step (a ring unrolled over its slots); the planes are double-buffered,
// so one LDS-only barrier per step suffices.
template <int D>
__global__ __launch_bounds__(64 * (D / 16), 1)
void delta_chain_kernel(DeltaArgs a) {
  using C = ChainCfg<D>;
  constexpr int KS = C::KS;
  constexpr int kRing = 2;
  __shared__ __attribute__((aligned(16))) float pl0[16 * C::LDP];   // P at the start and the end
  __shared__ __attribute__((aligned(16))) bf16 ph0[16 * C::LDB], ph1[16 * C::LDB];     // P_hi per step parity
  __shared__ __attribute__((aligned(16))) bf16 plo0[16 * C::LDB], plo1[16 * C::LDB];   // P_lo
  __shared__ float rsum0[C::NW * 16], rsum1[C::NW * 16];   // per-wave partial row sums
  constexpr int ncb = D / 16;
  const int blk = xcd_logical_block(blockIdx.x, gridDim.x);
  const int bh = blk / ncb, cb = blk % ncb;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int col = 16 * wave + l16;   // d_key column of this lane's outputs
  float* __restrict__ Mg = a.M + (int64_t)bh * D * D;

  // P[row][k] = M[k][16 cb + row] from the state
  for (int i = t; i < 16 * D; i += C::NT) {
    const int k = i / 16, row = i % 16;
    pl0[row * C::LDP + k] = Mg[(int64_t)k * D + 16 * cb + row];
  }
  __syncthreads();
  float p[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) p[r] = pl0[(4 * g + r) * C::LDP + col];
  __syncthreads();

  // segments s0 .. s0 + S - 1 of the head (a range of the stream, or all of it)
  const int s0 = a.s0, S = a.sn > 0 ? a.sn : a.S;
  const bf16* Abase = a.amat + ((int64_t)bh * a.S + s0) * 2 * D * D + (int64_t)col * D + 8 * g;
  const float* Cbase = a.cM + ((int64_t)bh * a.S + s0) * D * D + (int64_t)(16 * cb + 4 * g) * D + col;
  auto fetch = [&](ChainOps<D>& o, int s) {   // clamped: a load past the last segment is unused
    const int ss = s < S ? s : S - 1;
    const bf16* A0 = Abase + (int64_t)ss * 2 * D * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      o.h[ks] = *reinterpret_cast<const bf16x8*>(A0 + 32 * ks);
      o.l[ks] = *reinterpret_cast<const bf16x8*>(A0 + D * D + 32 * ks);
    }
    const float* C0 = Cbase + (int64_t)ss * D * D;
#pragma unroll
    for (int r = 0; r < 4; ++r) o.c[r] = C0[r * D];
  };
  // snapshot pass: row t / TPR, elements 4 (t % TPR) ..
  const int srow = t / C::TPR, sk = (t % C::TPR) * C::EPR;
  auto step = [&](const ChainOps<D>& o, int s) {
    // P_{s-1} as bf16 hi and lo planes (each wave converts its own tile) and the
    // wave's partial row sums (over its 16 d_key columns, exact in fp32)
    bf16* ph_s = (s & 1) ? ph1 : ph0;
    bf16* pl_s = (s & 1) ? plo1 : plo0;
    float* rs_s = (s & 1) ? rsum1 : rsum0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bf16 hb = f2bf(p[r]);
      ph_s[(4 * g + r) * C::LDB + col] = hb;
      pl_s[(4 * g + r) * C::LDB + col] = f2bf(p[r] - bf2f(hb));
      const float rr = row16_sum(p[r]);
      if (l16 == 0) rs_s[wave * 16 + 4 * g + r] = rr;
    }
    lds_sync();
    const int64_t shg = (int64_t)bh * a.S + s0 + s;
    {   // snapshot of M_{s-1}: 16 rows of M^T in bf16 hi and lo, and their sums
      const bf16x4 hv = *(const INFINI_LDS bf16x4*)(ph_s + srow * C::LDB + sk);
      const bf16x4 lv = *(const INFINI_LDS bf16x4*)(pl_s + srow * C::LDB + sk);
      *reinterpret_cast<bf16x4*>(a.snapM + (shg * D + 16 * cb + srow) * D + sk) = hv;
      *reinterpret_cast<bf16x4*>(a.snapMlo + (shg * D + 16 * cb + srow) * D + sk) = lv;
      if (t < 16) {
        float rs = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < C::NW; ++w2) rs += rs_s[w2 * 16 + t];
        a.snapc[shg * D + 16 * cb + t] = rs;
      }
    }
    bf16x8 ph[KS], plo[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      ph[ks] = *(const INFINI_LDS bf16x8*)(ph_s + l16 * C::LDB + 32 * ks + 8 * g);
      plo[ks] = *(const INFINI_LDS bf16x8*)(pl_s + l16 * C::LDB + 32 * ks + 8 * g);
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      acc = mfma16(ph[ks], o.h[ks], acc);
      acc = mfma16(plo[ks], o.h[ks], acc);
      acc = mfma16(ph[ks], o.l[ks], acc);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] += o.c[r] - acc[r];
  };

  ChainOps<D> o0, o1;
  fetch(o0, 0);
  fetch(o1, 1);
  int s = 0;
  // every iteration issues the same loads (no branch around them), so the
  // compiler's waits stay exact
  for (; s + kRing <= S; s += kRing) {
    step(o0, s);
    fetch(o0, s + kRing);
    step(o1, s + 1);
    fetch(o1, s + 1 + kRing);
  }
  if (s < S) step(o0, s);

  // M_S = P^T back into the state
  lds_sync();
#pragma unroll
  for (int r = 0; r < 4; ++r) pl0[(4 * g + r) * C::LDP + col] = p[r];
  __syncthreads();
  for (int i = t; i < 16 * D; i += C::NT) {
    const int k = i / 16, row = i % 16;
    Mg[(int64_t)k * D + 16 * cb + row] = pl0[row * C::LDP + k];
  }
}

// ------------------------------------------------------------------ launchers
template <int D>
hipError_t launch_delta_prep(const DeltaArgs& a, hipStream_t stream) {
  const int64_t seg_heads = (int64_t)a.BH * a.S;
  if (seg_heads <= 0) return hipSuccess;
  if (seg_heads > 0x7fffffff || a.N % kAmT != 0) return hipErrorInvalidValue;
  // C_s and c_s: the linear rule's contribution kernel (it takes B * H heads)
  LinContribArgs c{a.k, a.v, a.cM, a.cz, 1, a.BH, a.S, a.N, a.L};
  hipError_t e = launch_lin_contrib<D>(c, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(delta_zscan_kernel<D>, dim3((unsigned)a.BH), dim3(D), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(delta_amat_kernel<D>, dim3((unsigned)seg_heads), dim3(kAmThreads), 0, stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_delta_chain(const DeltaArgs& a, hipStream_t stream) {
  const int sn = a.sn > 0 ? a.sn : a.S;
  if ((int64_t)a.BH * a.S <= 0 || sn <= 0) return hipSuccess;
  if (a.s0 < 0 || a.s0 + sn > a.S) return hipErrorInvalidValue;
  hipLaunchKernelGGL(delta_chain_kernel<D>, dim3((unsigned)(a.BH * (D / 16))), dim3(64 * (D / 16)), 0, stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_delta_state(const DeltaArgs& a, hipStream_t stream) {
  hipError_t e = launch_delta_prep<D>(a, stream);
  if (e != hipSuccess) return e;
  DeltaArgs all = a;
  all.s0 = 0;
  all.sn = a.S;
  return launch_delta_chain<D>(all, stream);
}

template hipError_t launch_delta_state<64>(const DeltaArgs&, hipStream_t);
template hipError_t launch_delta_state<128>(const DeltaArgs&, hipStream_t);
template hipError_t launch_delta_prep<64>(const DeltaArgs&, hipStream_t);
template hipError_t launch_delta_prep<128>(const DeltaArgs&, hipStream_t);
template hipError_t launch_delta_chain<64>(const DeltaArgs&, hipStream_t);
template hipError_t launch_delta_chain<128>(const DeltaArgs&, hipStream_t);

}  // namespace infini
