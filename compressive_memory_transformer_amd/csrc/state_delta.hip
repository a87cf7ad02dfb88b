// Delta-rule memory state for the bf16 path (page "精读笔记：Infini-attention",
// section 3.4, delta rule; z as in section 3.3):
//   U_s  = V_s - sigma(K_s) M_{s-1} / (sigma(K_s) z_{s-1})   (0 / 0 read as 0)
//   M_s  = M_{s-1} + sigma(K_s)^T U_s,    z_s = z_{s-1} + sum_t sigma(K_s[t])
// with sigma(x) = ELU(x) + 1.
//
// Everything that depends on K alone runs in parallel before the chain:
//   delta_ksig: k' = sigma(K) - 1 as bf16 (full relative precision of the
//               deviation from 1) and the column sums of sigma(K) per segment;
//   delta_zscan: z_{s-1} for every segment (the snapshots) and the final z;
//   delta_den:  1 / (sigma(K_s[t]) z_{s-1}) per token, in fp32 from K.
// The chain then needs per segment only k', V and 1/den, and splits
//   sigma(K) M = colsum(M) + k' M          (read-back, one bf16 MFMA product)
//   sigma(K)^T U = 1 colsum_t(U) + k'^T U  (update; U split into bf16 hi + lo,
//                                          two MFMA products)
// where colsum(M) (over d_key) and colsum_t(U) (over tokens) are fp32.
#include "common.h"
#include "kernels.h"

namespace infini {

namespace {

constexpr int kThreads = 256;
constexpr int kCB = 16;          // columns of M (d_value) per chain workgroup
constexpr int kChainWaves = 4;   // chain workgroup: one wave per SIMD
constexpr int kChainSlots = 4;   // LDS chunk slots: three chunks in flight while one is used
constexpr int kChunk = 32 * kChainWaves;   // tokens per LDS chunk: one 32-token block per wave
constexpr int kInvSlot = 256;    // floats per 1/den slot: one wave-wide 16-byte load writes 1 KB
constexpr int kPart = 256;       // tokens per workgroup of the 1/den kernel

// ------------------------------------------------------------------ pre-pass
// Lanes per token and tokens per pass of a 256-thread block when each lane
// handles 8 consecutive d_key entries of a token.
template <int D>
struct TokLanes {
  static constexpr int LPT = D / 8;
  static constexpr int TPI = kThreads / LPT;
};

}  // namespace

// k' = sigma(K) - 1 (bf16) and the column sums of sigma(K) over a segment.  One
// workgroup per (b, h, segment); the sums are reduced in a fixed order.
template <int D>
__global__ __launch_bounds__(kThreads)
void delta_ksig_kernel(DeltaArgs a) {
  using T = TokLanes<D>;
  __shared__ float red[T::TPI][D];
  const int sh = blockIdx.x;
  const int bh = sh / a.S, s = sh % a.S;
  const int t = threadIdx.x, sub = t / T::LPT, d0 = (t % T::LPT) * 8;
  const int64_t tok0 = (int64_t)bh * a.L + (int64_t)s * a.N;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll 4
  for (int i = sub; i < a.N; i += T::TPI) {
    const bf16x8 kx = *reinterpret_cast<const bf16x8*>(a.k + (tok0 + i) * D + d0);
    bf16x8 kp;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = bf2f(kx[e]);
      const float f = x > 0.f ? x : exp_e(x) - 1.f;
      acc[e] += f + 1.f;
      kp[e] = f2bf(f);
    }
    *reinterpret_cast<bf16x8*>(a.kp + (tok0 + i) * D + d0) = kp;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[sub][d0 + e] = acc[e];
  __syncthreads();
  if (t < D) {
    float c = 0.f;
    for (int r = 0; r < T::TPI; ++r) c += red[r][t];
    a.czp[(int64_t)sh * D + t] = c;
  }
}

// z_{s-1} of every segment (snapshots) and the final z: a prefix over the
// segments of one head, one thread per d_key entry, in a fixed order.  The
// per-segment sums are loaded 32 at a time (independent loads at clamped
// indices), so they overlap instead of forming one dependent chain.
template <int D>
__global__ __launch_bounds__(D)
void delta_zscan_kernel(DeltaArgs a) {
  constexpr int kBatch = 32;
  const int bh = blockIdx.x, dk = threadIdx.x;
  const float* cz = a.czp + (int64_t)bh * a.S * D + dk;
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

// 1 / (sigma(K_s[t]) z_{s-1}) per token (0 for the first segment of the stream
// or a zero denominator).  One workgroup per (b, h, segment, part).
template <int D>
__global__ __launch_bounds__(kThreads)
void delta_den_kernel(DeltaArgs a) {
  using T = TokLanes<D>;
  __shared__ float zs[D];
  const int sh = blockIdx.x / a.nparts, part = blockIdx.x % a.nparts;
  const int bh = sh / a.S, s = sh % a.S;
  const int t = threadIdx.x, sub = t / T::LPT, d0 = (t % T::LPT) * 8;
  const bool has_memory = (a.seg_base + s) > 0;
  if (t < D) zs[t] = a.snapz[(int64_t)sh * D + t];
  __syncthreads();
  const int64_t tok0 = (int64_t)bh * a.L + (int64_t)s * a.N + (int64_t)part * kPart;
  const int ntok = min(kPart, a.N - part * kPart);
  // every lane of a token group runs the same trip count (the reduction below
  // exchanges within the group)
#pragma unroll 4
  for (int i = sub; i < ntok; i += T::TPI) {
    const bf16x8 kx = *reinterpret_cast<const bf16x8*>(a.k + (tok0 + i) * D + d0);
    float part_den = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = bf2f(kx[e]);
      part_den = __builtin_fmaf(x > 0.f ? x + 1.f : exp_e(x), zs[d0 + e], part_den);
    }
#pragma unroll
    for (int o = 1; o < T::LPT; o <<= 1) part_den += __shfl_xor(part_den, o);
    if (t % T::LPT == 0) a.inv_den[tok0 + i] = (has_memory && part_den > 0.f) ? 1.f / part_den : 0.f;
  }
}

// ------------------------------------------------------------------- chain
namespace {

// Physical 16-byte chunk of logical chunk c in row r of a k' chunk in LDS.  The
// tile is read two ways: 16 bytes per lane by 16 consecutive rows (read-back
// operand) and by ds_read_b64_tr_b16 over 8 rows x 2 chunks per half-wave
// (update operand).  The map below gives 16 distinct bank groups for the first
// and 32 distinct 8-byte banks for the second.
template <int D>
__device__ __forceinline__ int kp_swz(int r) {
  return D == 128 ? (((r & 7) << 1) | ((r >> 3) & 1)) : ((((r >> 1) & 3) << 1) | ((r >> 3) & 1));
}

template <int D>
struct ChainLayout {
  static constexpr int CHUNKS = D / 8;
  static constexpr int KP_ELEMS = kChunk * D;
  static constexpr int RPI = 64 * 8 / D;                      // k' rows per wave-wide 16-byte load
  static constexpr int NIK = kChunk / RPI / kChainWaves;                // k' loads per wave and chunk
  static constexpr int NIV = kChunk * kCB * 2 / 1024 / kChainWaves;     // V loads per wave and chunk
  static_assert(NIK >= 1 && NIV >= 1, "chunk too small");
  static_assert(kChainWaves * D * kCB * 4 <= KP_ELEMS * 2, "update reduction must fit a k' chunk");
  static_assert(kInvSlot * 4 == 1024 && kChunk <= kInvSlot, "1/den slot holds one 64-lane load");
  static_assert(NIK * kChainWaves * 1024 == KP_ELEMS * 2 && NIV * kChainWaves * 1024 == kChunk * kCB * 2,
                "loads fill the slots exactly");
};

#if defined(__HIP_DEVICE_COMPILE__)
// Wave-uniform descriptor (see fa_fwd.hip): readfirstlane keeps it in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t chain_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  void* ub = (void*)(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}
#endif

// Per-workgroup context of the chain.
template <int D>
struct ChainCtx {
  const bf16* kp;      // k' of this head, [L][D]
  const bf16* v;       // V of this head, [L][D], shifted to column block cb
  const float* inv;    // 1/den of this head, [L]
  int N, cps, wave, lane;
};

// Direct-to-LDS loads of chunk q of the head's stream (segment q / cps, chunk
// q % cps; zeros past the segment or past the last segment, so that every
// chunk issues the same number of loads): k' rows with the swizzle, 16 V
// columns per token, 1/den (wave 0).
template <int D>
__device__ __forceinline__ void chain_issue(const ChainCtx<D>& cx, int q, int S, bf16* kpl, bf16* vl, float* il) {
#if defined(__HIP_DEVICE_COMPILE__)
  using CL = ChainLayout<D>;
  const int s = q / cx.cps, c = q % cx.cps;
  const int first = c * kChunk;                                   // first token of the chunk in the segment
  const int64_t tok = s < S ? (int64_t)s * cx.N + first : 0;      // within the head
  const uint32_t left = (s < S && first < cx.N) ? (uint32_t)(cx.N - first) : 0u;
  const int wv = __builtin_amdgcn_readfirstlane(cx.wave);
  {
    const __amdgpu_buffer_rsrc_t r = chain_rsrc(cx.kp + tok * D, left * D * 2);
#pragma unroll
    for (int j = 0; j < CL::NIK; ++j) {
      const int ins = wv * CL::NIK + j;
      const int row = ins * CL::RPI + cx.lane / CL::CHUNKS;
      const int phys = cx.lane % CL::CHUNKS;
      const int off = 2 * (row * D + 8 * (phys ^ kp_swz<D>(row)));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (INFINI_LDS void*)(kpl + ins * 512), 16, off, 0, 0, 0);
    }
  }
  {
    // token row pitch D in HBM; the descriptor spans whole rows, the last one to
    // this block's 16 columns
    const uint32_t bytes = left ? (left - 1) * D * 2 + kCB * 2 : 0u;
    const __amdgpu_buffer_rsrc_t r = chain_rsrc(cx.v + tok * D, bytes);
#pragma unroll
    for (int j = 0; j < CL::NIV; ++j) {
      const int ins = wv * CL::NIV + j;
      const int token = ins * 32 + cx.lane / 2;
      const int off = token * D * 2 + 16 * (cx.lane & 1);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (INFINI_LDS void*)(vl + ins * 512), 16, off, 0, 0, 0);
    }
  }
  if (wv == 0) {
    const __amdgpu_buffer_rsrc_t r = chain_rsrc(cx.inv + tok, left * 4);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (INFINI_LDS void*)il, 16, 16 * cx.lane, 0, 0, 0);
  }
#endif
}

// Waits until at most the loads of the two most recently issued chunks are in
// flight (vmcnt over this wave's loads per chunk: the k' and V shares, plus 1/den
// on wave 0) and this wave's LDS accesses are done.
// Workgroup barrier for LDS traffic only.  (__syncthreads() also orders global
// memory, which makes it wait for every load into LDS still in flight.)
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
}

template <int D>
__device__ __forceinline__ void chain_wait_older(int wave) {
  using CL = ChainLayout<D>;
  constexpr int L = CL::NIK + CL::NIV;
  constexpr int W0 = 2 * (L + 1), WN = 2 * L;
  static_assert(W0 < 64, "vmcnt range");
  if (__builtin_amdgcn_readfirstlane(wave) == 0) __builtin_amdgcn_s_waitcnt((W0 & 15) | ((W0 >> 4) << 14) | 0x0070);
  else __builtin_amdgcn_s_waitcnt((WN & 15) | ((WN >> 4) << 14) | 0x0070);
}

// Per-wave state of one segment: the B operand of the read-back (bf16 M, d_key
// rows 32c + 8g + j of column l % 16), colsum(M) of the lane's column, the
// update accumulators (dk rows 16 dkb + 4g + r, column l % 16) and the lane's
// share of colsum_t(U).
template <int D>
struct ChainSeg {
  bf16x8 mop[D / 32];
  float cs;
  f32x4 dm[D / 16];
  float ucol;
};

// One 32-token block (rows 32 b .. 32 b + 31 of the chunk in LDS).
template <int D>
__device__ __forceinline__ void chain_block(ChainSeg<D>& sg, const bf16* __restrict__ kpl,
                                            const bf16* __restrict__ vl, const float* __restrict__ il, int b) {
  const int lane = threadIdx.x & 63, col = lane & 15, g = lane >> 4;
  // read-back R' = k' M for the block's two 16-token halves: lane holds tokens
  // 16 h2 + 4 g + r, column col
  f32x4 u[2];
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    const int row = 32 * b + 16 * h2 + col;                 // token of the A operand rows (l % 16)
    const bf16* base = kpl + row * D;
    f32x4 r4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
      const bf16x8 ka = lds_read8(base + 8 * ((4 * c + g) ^ kp_swz<D>(col)));
      r4 = mfma16(ka, sg.mop[c], r4);
    }
    // V[token 16 h2 + 4 g + e][col] by a transposing read of the [token][16] tile
    const int vr = 32 * b + 16 * h2 + 4 * g + ((lane & 15) >> 2);
    const s16x4 vv = lds_read_tr16(vl + vr * kCB + 4 * (lane & 3));
    const f32x4 iv = *(const INFINI_LDS f32x4*)(il + 32 * b + 16 * h2 + 4 * g);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float x = bf16_bits_to_f32(vv[r]);
      u[h2][r] = __builtin_fmaf(-(sg.cs + r4[r]), iv[r], x);
      sg.ucol += u[h2][r];
    }
  }
  // B operands of the update: U = hi + lo (bf16 each), rows in the key order
  // tau(g, j) = 16 (j / 4) + 4 g + j % 4
  bf16x8 ub, ul;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    ub[r] = f2bf(u[0][r]);
    ub[4 + r] = f2bf(u[1][r]);
    ul[r] = f2bf(u[0][r] - bf2f(ub[r]));
    ul[4 + r] = f2bf(u[1][r] - bf2f(ub[4 + r]));
  }
  // update dM[dk][col] += sum_t k'[t][dk] U[t][col]; A operand k'^T by
  // transposing reads: rows 32 b + 4 g + a (+ 16), columns 16 dkb + 4 (l % 4)
  const int a4 = (lane & 15) >> 2, bb = lane & 3;
  const int rw = 4 * g + a4;                                  // row within 16 (the swizzle key)
  const int sw = kp_swz<D>(rw);
  const bf16* r0 = kpl + (32 * b + rw) * D + 4 * (bb & 1);
#pragma unroll
  for (int dkb = 0; dkb < D / 16; ++dkb) {
    const int ch = (2 * dkb + (bb >> 1)) ^ sw;
    const s16x4 x = lds_read_tr16(r0 + 8 * ch);
    const s16x4 y = lds_read_tr16(r0 + 16 * D + 8 * ch);
    const bf16x8 kt = __builtin_bit_cast(bf16x8, __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7));
    sg.dm[dkb] = mfma16(kt, ub, sg.dm[dkb]);
    sg.dm[dkb] = mfma16(kt, ul, sg.dm[dkb]);
  }
}

}  // namespace

// The chain over the segments of one head for 16 columns of M (columns of M are
// independent under the delta rule: column j of the read-back needs only
// column j of M).  One workgroup of 4 waves per (b, h, column block), one
// workgroup per CU; k', V and 1/den stream through four LDS chunk slots
// (direct-to-LDS loads, three chunks in flight while one is used: the chain is
// bound by the bytes in flight per CU, not by its arithmetic).  Each wave takes
// one 32-token block of a 128-token chunk and accumulates its own share of the
// update; the shares and colsum_t(U) are reduced in a fixed order at the end of
// each segment (deterministic).
template <int D>
__global__ __launch_bounds__(64 * kChainWaves, 1)
void delta_chain_kernel(DeltaArgs a) {
  using CL = ChainLayout<D>;
  constexpr int NT = 64 * kChainWaves;   // threads
  constexpr int NCB = D / kCB;
  constexpr int RG = NT / kCB;           // row groups of M (thread: column t % 16, rows RPT (t / 16) ..)
  constexpr int RPT = D / RG;
  // four slots, each a distinct object so that reads of one slot never wait on
  // loads into another
  static_assert(kChainSlots == 4, "the chunk loop is unrolled over the four slots");
  __shared__ __attribute__((aligned(1024))) bf16 kp0[CL::KP_ELEMS], kp1[CL::KP_ELEMS], kp2[CL::KP_ELEMS],
      kp3[CL::KP_ELEMS];
  __shared__ __attribute__((aligned(1024))) bf16 vc0[kChunk * kCB], vc1[kChunk * kCB], vc2[kChunk * kCB],
      vc3[kChunk * kCB];
  __shared__ __attribute__((aligned(16))) float iv0[kInvSlot], iv1[kInvSlot], iv2[kInvSlot], iv3[kInvSlot];
  __shared__ __attribute__((aligned(16))) bf16 mts[kCB * D];   // M^T rows (bf16) of this block
  __shared__ float csred[RG][kCB];
  __shared__ float ucs[kChainWaves][kCB];

  const int blk = xcd_logical_block(blockIdx.x, gridDim.x);
  const int bh = blk / NCB, cb = blk % NCB;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int mcol = t % kCB, mrow0 = RPT * (t / kCB);

  ChainCtx<D> cx;
  cx.kp = a.kp + (int64_t)bh * a.L * D;
  cx.v = a.v + (int64_t)bh * a.L * D + cb * kCB;
  cx.inv = a.inv_den + (int64_t)bh * a.L;
  cx.N = a.N;
  cx.cps = ((a.N + kChunk - 1) / kChunk + 3) & ~3;   // chunks per segment, padded to a multiple of 4
  cx.wave = wave;
  cx.lane = lane;

  float m[RPT];
  float* __restrict__ Mg = a.M + (int64_t)bh * D * D;
#pragma unroll
  for (int i = 0; i < RPT; ++i) m[i] = Mg[(int64_t)(mrow0 + i) * D + cb * kCB + mcol];

  chain_issue<D>(cx, 0, a.S, kp0, vc0, iv0);
  chain_issue<D>(cx, 1, a.S, kp1, vc1, iv1);
  chain_issue<D>(cx, 2, a.S, kp2, vc2, iv2);
  chain_wait_older<D>(wave);
  lds_barrier();

  for (int s = 0; s < a.S; ++s) {
    const int64_t sh = (int64_t)bh * a.S + s;
    // ---- publish M_{s-1}: bf16 M^T rows, colsum(M), snapshots
    {
      float part = 0.f;
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        mts[mcol * D + mrow0 + i] = f2bf(m[i]);
        part += m[i];
      }
      csred[t / kCB][mcol] = part;     // t / kCB < RG
    }
    lds_barrier();
    ChainSeg<D> sg;
    {
      const int col = lane & 15, g = lane >> 4;
      float c = 0.f;
#pragma unroll
      for (int r = 0; r < RG; ++r) c += csred[r][col];
      sg.cs = c;
#pragma unroll
      for (int k = 0; k < D / 32; ++k) sg.mop[k] = lds_read8(mts + col * D + 32 * k + 8 * g);
      if (t < kCB) a.snapc[sh * D + cb * kCB + t] = c;
      // snapshot rows: column cb*16 + j of M is row cb*16 + j of M^T
      for (int i = t; i < kCB * D / 8; i += NT) {
        const int j = i / (D / 8), c8 = (i % (D / 8)) * 8;
        *reinterpret_cast<bf16x8*>(a.snapM + sh * D * D + (int64_t)(cb * kCB + j) * D + c8) =
            lds_read8(mts + j * D + c8);
      }
    }
#pragma unroll
    for (int k = 0; k < D / 16; ++k) sg.dm[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    sg.ucol = 0.f;

    // ---- chunks: step c uses slot c % 4 and loads chunk c + 3 of the stream
    // (past the segment's end: the next segment's first chunks) into the slot of
    // chunk c - 1, which every wave has finished with at the last barrier.
    const int q0 = s * cx.cps;
#define INFINI_CHAIN_STEP(C, KC, VC, IC, KN, VN, IN)                                       \
    {                                                                                      \
      const int c_ = (C);                                                                  \
      chain_issue<D>(cx, q0 + c_ + 3, a.S, KN, VN, IN);                                    \
      chain_block<D>(sg, KC, VC, IC, wave);                                                \
      chain_wait_older<D>(wave);                                                           \
      lds_barrier();                                                                     \
    }
    for (int c = 0; c < cx.cps; c += 4) {
      INFINI_CHAIN_STEP(c, kp0, vc0, iv0, kp3, vc3, iv3)
      INFINI_CHAIN_STEP(c + 1, kp1, vc1, iv1, kp0, vc0, iv0)
      INFINI_CHAIN_STEP(c + 2, kp2, vc2, iv2, kp1, vc1, iv1)
      INFINI_CHAIN_STEP(c + 3, kp3, vc3, iv3, kp2, vc2, iv2)
    }
#undef INFINI_CHAIN_STEP

    // ---- M_s = M_{s-1} + 1 colsum_t(U) + sum over waves of k'^T U (slot 3 is free:
    // the last chunk of the segment used it, the next three are in slots 0-2)
    {
      const int col = lane & 15, g = lane >> 4;
      float uc = sg.ucol;
      uc += __shfl_xor(uc, 16);
      uc += __shfl_xor(uc, 32);
      if (g == 0) ucs[wave][col] = uc;
      float* red = reinterpret_cast<float*>(kp3);          // [waves][D][16]
#pragma unroll
      for (int k = 0; k < D / 16; ++k)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[(wave * D + 16 * k + 4 * g + r) * kCB + col] = sg.dm[k][r];
    }
    lds_barrier();
    {
      const float* red = reinterpret_cast<const float*>(kp3);
      float ucsum = 0.f;
#pragma unroll
      for (int w = 0; w < kChainWaves; ++w) ucsum += ucs[w][mcol];
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const int dk = mrow0 + i;
        float d = 0.f;
#pragma unroll
        for (int w = 0; w < kChainWaves; ++w) d += red[(w * D + dk) * kCB + mcol];
        m[i] += ucsum + d;
      }
    }
    lds_barrier();   // slot 3, ucs and csred are reused by the next segment
  }

#pragma unroll
  for (int i = 0; i < RPT; ++i) Mg[(int64_t)(mrow0 + i) * D + cb * kCB + mcol] = m[i];
}

// ------------------------------------------------------------------ launchers
int delta_parts(int N) { return (N + kPart - 1) / kPart; }   // blocks of the 1/den kernel per segment

template <int D>
hipError_t launch_delta_state(const DeltaArgs& args, hipStream_t stream) {
  DeltaArgs a = args;
  a.nparts = delta_parts(a.N);
  const int64_t seg_heads = (int64_t)a.BH * a.S;
  if (seg_heads <= 0) return hipSuccess;
  const int64_t pblocks = seg_heads * a.nparts;
  if (pblocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(delta_ksig_kernel<D>, dim3((unsigned)seg_heads), dim3(kThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(delta_zscan_kernel<D>, dim3((unsigned)a.BH), dim3(D), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(delta_den_kernel<D>, dim3((unsigned)pblocks), dim3(kThreads), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(delta_chain_kernel<D>, dim3((unsigned)(a.BH * (D / kCB))), dim3(64 * kChainWaves), 0, stream, a);
  return hipGetLastError();
}

template hipError_t launch_delta_state<64>(const DeltaArgs&, hipStream_t);
template hipError_t launch_delta_state<128>(const DeltaArgs&, hipStream_t);

}  // namespace infini
