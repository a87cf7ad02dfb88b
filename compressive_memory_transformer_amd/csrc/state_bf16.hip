// Linear-rule memory state of the bf16 path (page "精读笔记：Infini-attention",
// section 3.4, linear rule; z as in section 3.3):
//
//   M_s = M_{s-1} + sigma(K)^T V,   z_s = z_{s-1} + sum_t sigma(K_t)
//
// It leaves a snapshot of (M_{s-1}^T as bf16 plus its bf16 remainder, z_{s-1}
// and colsum(M_{s-1}) in fp32) per segment for the fused attention kernel and the
// final (M_S, z_S) in the fp32 state.  The delta rule lives in state_delta.hip.
//
// Precision.  sigma(K) is split exactly into two bf16 parts, sigma = hi + lo with
// hi = bf16(sigma) and lo = bf16(sigma - hi), and the contribution GEMM runs as two
// bf16 products into one fp32 accumulator (V is exact in bf16):
//   sigma(K)^T V = hi^T V + lo^T V,
// which keeps about 16 bits of sigma whatever its size: for keys near 0
// (sigma ~ 1 + k, where bf16(sigma) alone would keep only a few bits of k) and for
// strongly negative keys (sigma ~ e^k << 1, where writing sigma as
// 1 + (sigma - 1) would cancel).
#include <atomic>

#include "common.h"
#include "kernels.h"

namespace infini {

namespace {
constexpr int kThreads = 256;
}  // namespace

// =================================================================== linear
// One workgroup (8 waves) per (b, h, s) and 64-column block of d_key; the two
// blocks of a segment (d = 128) run on the same XCD and share its V through L2.
// 64-token stages of K (this block's columns) and V stream into a 4-slot LDS
// ring with buffer_load ... lds (three stages in flight).  Per stage each thread
// turns 8 elements of K into sigma(K) = hi + lo (bf16 each), written to two LDS
// buffers in the layout of the transposing operand reads; then C^T[d_value][d_key]
// += V^T hi + V^T lo on v_mfma_f32_32x32x16_bf16 (both products into one fp32
// accumulator), one 32 x 32 output tile per wave (d = 128; at d = 64 two waves
// share a tile, taking alternate 16-token steps).  c = sum_t sigma(K_t) is
// reduced over the workgroup at the end in a fixed order.
namespace {
constexpr int kLcWaves = 8;
constexpr int kLcThreads = 64 * kLcWaves;
constexpr int kLcKb = 64;        // d_key columns per workgroup
constexpr int kLcTt = 64;        // tokens per stage
constexpr int kLcStages = 4;     // ring slots

// Physical 16-byte chunk of logical chunk c in row r of a [tokens x P] tile read
// by ds_read_b64_tr_b16 (P = 128 or 64 elements): a 32-lane half of a read covers
// 4 consecutive rows x 4 chunks, and rows r % 4 (P = 128) or (r / 2) % 2 (P = 64)
// move them to disjoint groups of 4 chunks.
template <int P>
__device__ __forceinline__ int lc_chunk(int r, int c) { return c ^ (P == 128 ? (r & 3) << 2 : ((r >> 1) & 1) << 2); }

// Element offset (relative to a 16-token step) of this lane's first transposing
// read for 32-column block cb of a [tokens x P] tile; the second read is 8 rows
// further.  Lane l gets column 32 cb + l % 32 of tokens {4 hi + e, 8 + 4 hi + e}.
template <int P>
__device__ __forceinline__ int lc_tr_offset(int lane, int cb) {
  const int hi = lane >> 5, grp = lane >> 4, sidx = lane & 15;
  const int row = 4 * hi + (sidx >> 2);
  const int col = 32 * cb + 16 * (grp & 1) + 4 * (sidx & 3);
  return row * P + 8 * lc_chunk<P>(row, col >> 3) + (col & 7);
}

template <int P>
__device__ __forceinline__ bf16x8 lc_read_tr(const bf16* tile, int ofs) {
  const s16x4 x = lds_read_tr16(tile + ofs);
  const s16x4 y = lds_read_tr16(tile + ofs + 8 * P);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7));
}

#if defined(__HIP_DEVICE_COMPILE__)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t lc_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  void* ub = (void*)(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}
#endif

// Direct-to-LDS loads of stage q (tokens [64 q, 64 q + 64) of the segment; zeros
// past its end): this wave's share of the K block (one 1 KB load: 8 rows x 128 B,
// row-major) and of V (1 KB loads of 1024 / (2 D) rows each, swizzled).
template <int D>
__device__ __forceinline__ void lc_issue(const bf16* kseg, const bf16* vseg, int N, int q, int dkb, bf16* ks,
                                         bf16* vs, int wave, int lane) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int VI = kLcTt * D * 2 / 1024 / kLcWaves;   // V loads per wave and stage
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int t0 = q * kLcTt;
  const uint32_t rows = t0 < N ? (uint32_t)(N - t0) : 0u;
  {
    const __amdgpu_buffer_rsrc_t r = lc_rsrc(kseg + (int64_t)(t0 < N ? t0 : 0) * D, rows * D * 2);
    const int row = 8 * wv + lane / 8;
    const int off = 2 * (row * D + dkb * kLcKb + 8 * (lane % 8));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (INFINI_LDS void*)(ks + wv * 512), 16, off, 0, 0, 0);
  }
  {
    constexpr int RPI = 512 / D;   // rows per 1 KB load
    const __amdgpu_buffer_rsrc_t r = lc_rsrc(vseg + (int64_t)(t0 < N ? t0 : 0) * D, rows * D * 2);
#pragma unroll
    for (int j = 0; j < VI; ++j) {
      const int ins = VI * wv + j;
      const int row = RPI * ins + lane / (D / 8);
      const int phys = lane % (D / 8);
      const int off = 2 * (row * D + 8 * lc_chunk<D>(row, phys));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (INFINI_LDS void*)(vs + ins * 512), 16, off, 0, 0, 0);
    }
  }
#endif
}
}  // namespace

template <int D>
__global__ __launch_bounds__(kLcThreads, 1)
void lin_contrib_kernel(LinContribArgs a) {
  constexpr int NKB = D / kLcKb;                 // d_key blocks per segment
  constexpr int KT = kLcTt * kLcKb;              // elements of a K stage
  constexpr int VT = kLcTt * D;                  // elements of a V stage
  constexpr int NDV = D / 32;                    // 32-row blocks of d_value
  constexpr int TILES = NDV * (kLcKb / 32);      // output tiles per workgroup
  constexpr int SHARE = kLcWaves / TILES;        // waves per tile (token steps interleaved)
  constexpr int NST = kLcTt / 16 / SHARE;        // 16-token steps per wave and stage
  constexpr int EPS = 8 / NST;                   // sigma(K) elements per step
  constexpr int IPW = 1 + kLcTt * D * 2 / 1024 / kLcWaves;   // loads per wave and stage
  static_assert(TILES * SHARE == kLcWaves && (SHARE == 1 || SHARE == 2), "tiles per wave");
  static_assert(KT / kLcThreads == 8, "one 16-byte chunk of K per thread and stage");
  static_assert(kLcStages == 4, "the stage loop is unrolled over the four slots");
  // Each slot and buffer is an array of its own, and the loop is unrolled over
  // the slots: the compiler then sees that the LDS reads of one slot never
  // alias the direct-to-LDS loads into another and does not wait for them.
  __shared__ __attribute__((aligned(1024))) bf16 ks0[KT], ks1[KT], ks2[KT], ks3[KT];
  __shared__ __attribute__((aligned(1024))) bf16 vs0[VT], vs1[VT], vs2[VT], vs3[VT];
  __shared__ __attribute__((aligned(1024))) bf16 kh0[KT], kh1[KT];   // hi parts of sigma(K)
  __shared__ __attribute__((aligned(1024))) bf16 kl0[KT], kl1[KT];   // lo parts
  __shared__ float lc_red[kLcTt * (kLcKb + 1)];   // end-of-kernel reductions
  static_assert(SHARE == 1 || TILES * 1024 <= kLcTt * (kLcKb + 1), "partials fit the reduction area");

  const int blk = xcd_logical_block(blockIdx.x, gridDim.x);
  const int sh = blk / NKB, dkb = blk % NKB;
  const int bh = sh / a.S, s = sh % a.S;
  const int64_t tok0 = (int64_t)bh * a.L + (int64_t)s * a.N;
  const bf16* kseg = a.k + tok0 * D;
  const bf16* vseg = a.v + tok0 * D;

  const int th = threadIdx.x, lane = th & 63, wave = th >> 6;
  const int tile = wave % TILES, part = wave / TILES;
  const int dvb = tile % NDV, dkq = tile / NDV;
  const int vofs = lc_tr_offset<D>(lane, dvb);
  const int kofs = lc_tr_offset<kLcKb>(lane, dkq);
  // sigma(K) pass: row th / 8 of the stage, logical chunk th % 8
  const int srow = th >> 3, sch = th & 7;
  const int ssrc = srow * kLcKb + 8 * sch;
  const int sdst = srow * kLcKb + 8 * lc_chunk<kLcKb>(srow, sch);

  const int nst = a.N / kLcTt;
  lc_issue<D>(kseg, vseg, a.N, 0, dkb, ks0, vs0, wave, lane);
  lc_issue<D>(kseg, vseg, a.N, 1, dkb, ks1, vs1, wave, lane);
  lc_issue<D>(kseg, vseg, a.N, 2, dkb, ks2, vs2, wave, lane);

  float zp[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) zp[i] = 0.f;
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;

  // sigma(K) = hi + lo of elements [i0, i0 + n) of this thread's chunk (bf16
  // each) and its column sums (fp32)
  auto sigma_part = [&](const bf16x8& kx, bf16x8& h8, bf16x8& l8, int i0, int n) {
#pragma unroll
    for (int i = i0; i < i0 + n; ++i) {
      const float x = bf2f(kx[i]);
      const float f = x > 0.f ? x + 1.f : exp_e(x);
      zp[i] += f;
      h8[i] = f2bf(f);
      l8[i] = f2bf(f - bf2f(h8[i]));
    }
  };

  // prologue: stage 0 landed, its sigma(K) parts in buffer 0
  {
    constexpr int VM = 2 * IPW;
    __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | 0x0F70);
    __builtin_amdgcn_s_barrier();
    const bf16x8 kx = *(const INFINI_LDS bf16x8*)(ks0 + ssrc);
    bf16x8 h8, l8;
    sigma_part(kx, h8, l8, 0, 8);
    *(INFINI_LDS bf16x8*)(kh0 + sdst) = h8;
    *(INFINI_LDS bf16x8*)(kl0 + sdst) = l8;
  }
  // Iteration q: the products of stage q (MFMA, slot q % 4, buffer q % 2)
  // interleaved with k' of stage q+1 (VALU, into the other buffer); the loads
  // of stage q+3 go into the slot of stage q-1, which every wave has finished
  // reading at the barrier.
#define INFINI_LC_ITER(Q, VC, KN, KHC, KHN, KLC, KLN, KLD, VLD)                                   \
  {                                                                                             \
    const int q_ = (Q);                                                                         \
    /* stage q+1 has landed once at most stage q+2's loads are in flight */                      \
    __builtin_amdgcn_s_waitcnt((IPW & 15) | ((IPW >> 4) << 14) | 0x0070);  /* and lgkmcnt(0) */ \
    __builtin_amdgcn_s_barrier();                                                               \
    lc_issue<D>(kseg, vseg, a.N, q_ + 3, dkb, KLD, VLD, wave, lane);                            \
    if (q_ < nst) {                                                                             \
      const bool more_ = q_ + 1 < nst;                                                          \
      /* all operand reads of the stage first: one LDS latency per stage */                     \
      const bf16x8 kx_ = *(const INFINI_LDS bf16x8*)(KN + ssrc);                                \
      bf16x8 va_[NST], vk_[NST], vl_[NST];                                                      \
      _Pragma("unroll")                                                                         \
      for (int j = 0; j < NST; ++j) {                                                           \
        const int st = part + SHARE * j;                                                        \
        va_[j] = lc_read_tr<D>(VC, 16 * st * D + vofs);                                         \
        vk_[j] = lc_read_tr<kLcKb>(KHC, 16 * st * kLcKb + kofs);                                \
        vl_[j] = lc_read_tr<kLcKb>(KLC, 16 * st * kLcKb + kofs);                                \
      }                                                                                         \
      bf16x8 h8_, l8_;                                                                          \
      _Pragma("unroll")                                                                         \
      for (int j = 0; j < NST; ++j) {                                                           \
        acc = mfma32(va_[j], vk_[j], acc);                                                      \
        acc = mfma32(va_[j], vl_[j], acc);                                                      \
        if (more_) sigma_part(kx_, h8_, l8_, EPS * j, EPS);                                     \
      }                                                                                         \
      if (more_) {                                                                              \
        *(INFINI_LDS bf16x8*)(KHN + sdst) = h8_;                                                \
        *(INFINI_LDS bf16x8*)(KLN + sdst) = l8_;                                                \
      }                                                                                         \
    }                                                                                           \
  }
  // Iterations past the last stage (when the stage count is not a multiple of
  // four) only wait, synchronise and issue empty loads: every load is issued
  // unconditionally, so the compiler tracks exactly which slots have loads in
  // flight and adds no waits of its own.
  for (int q = 0; q < nst; q += 4) {
    INFINI_LC_ITER(q, vs0, ks1, kh0, kh1, kl0, kl1, ks3, vs3)
    INFINI_LC_ITER(q + 1, vs1, ks2, kh1, kh0, kl1, kl0, ks0, vs0)
    INFINI_LC_ITER(q + 2, vs2, ks3, kh0, kh1, kl0, kl1, ks1, vs1)
    INFINI_LC_ITER(q + 3, vs3, ks0, kh1, kh0, kl1, kl0, ks2, vs2)
  }
#undef INFINI_LC_ITER
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // token-interleaved partials of one tile are summed in wave order (d = 64)
  float* red = lc_red;
  if (SHARE > 1) {
    if (part > 0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) red[tile * 1024 + r * 64 + lane] = acc[r];
    }
    __syncthreads();
    if (part == 0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] += red[tile * 1024 + r * 64 + lane];
    }
    __syncthreads();
  }
  float* __restrict__ cm = a.cM + (int64_t)sh * D * D;
  if (part == 0) {
    const int hi = lane >> 5, l32 = lane & 31;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int dv = 32 * dvb + 8 * (r >> 2) + 4 * hi + (r & 3);
      cm[dv * D + dkb * kLcKb + 32 * dkq + l32] = acc[r];
    }
  }
  // c: column sums of sigma(K) over the 64 row positions, in row order
  float* zred = red;   // [64 rows][kLcKb + 1]
#pragma unroll
  for (int i = 0; i < 8; ++i) zred[srow * (kLcKb + 1) + 8 * sch + i] = zp[i];
  __syncthreads();
  if (th < kLcKb) {
    float sum = 0.f;
    for (int r = 0; r < kLcTt; ++r) sum += zred[r * (kLcKb + 1) + th];
    a.cz[(int64_t)sh * D + dkb * kLcKb + th] = sum;
  }
}

// d = 128: one work item per (b, h, s), the whole segment, so that V is read
// from memory once (the two 64-column halves of d_key in separate workgroups
// share it only while they run side by side).  Persistent: one workgroup
// (8 waves) per compute unit walks the items lw, lw + G, ... (lw its
// XCD-grouped logical index); their 32-token stages of K and V (8 KB each) form
// one stream through an 8-slot LDS ring, filled by buffer_load ... lds seven
// stages ahead, across item boundaries.  Both tensors arrive in the layout of
// the transposing operand reads (chunks swizzled as lc_chunk<128>).  Per stage
// each thread turns one 16-byte chunk of K into sigma(K) = hi + lo: hi in place
// in the K slot, lo into one of two LDS buffers; each wave owns two 32 x 32
// tiles of C^T (one 32-row block of d_value, two 32-column blocks of d_key) and
// adds V^T hi + V^T lo to both (v_mfma_f32_32x32x16_bf16, one fp32 accumulator
// each).  At the end of an item its tiles go out and c = sum_t sigma(K_t) is
// reduced over the workgroup in a fixed order.
namespace {
constexpr int kSgWaves = 8;
constexpr int kSgThreads = 64 * kSgWaves;
constexpr int kSgTt = 32;        // tokens per stage
constexpr int kSgSlots = 8;      // ring slots (seven stages in flight)
constexpr int kSgIpw = 2;        // loads per wave and stage (one 1 KB piece of K, one of V)

struct SgPos {
  int64_t tok0;
  int sh, q, k;
  bool valid;
};

__device__ __forceinline__ void sg_item(const LinContribArgs& a, int lw, int G, int items, SgPos& p) {
  const int item = lw + p.k * G;
  p.valid = item < items;
  p.sh = p.valid ? item : lw;
  const int bh = p.sh / a.S, s = p.sh - bh * a.S;
  p.tok0 = (int64_t)bh * a.L + (int64_t)s * a.N;
}

__device__ __forceinline__ void sg_advance(const LinContribArgs& a, int lw, int G, int items, int nst, SgPos& p) {
  if (++p.q == nst) {
    p.q = 0;
    ++p.k;
    sg_item(a, lw, G, items, p);
  }
}

// This wave's loads of one stage: rows 4 w .. 4 w + 3 of the stage's K and V
// (1 KB each, 16 bytes per lane, chunks swizzled); zeros past the segment end or
// the last item.
__device__ __forceinline__ void sg_issue(const LinContribArgs& a, const SgPos& p, bf16* ks, bf16* vs, int wave,
                                         int lane) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int D = 128;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int t0 = p.q * kSgTt;
  const uint32_t rows = p.valid && t0 < a.N ? (uint32_t)(a.N - t0) : 0u;
  const int64_t e0 = (p.tok0 + t0) * D;
  const int row = 4 * wv + lane / 16;
  const int off = 2 * (row * D + 8 * lc_chunk<D>(row, lane % 16));
  const __amdgpu_buffer_rsrc_t rk = lc_rsrc(a.k + e0, rows * D * 2);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (INFINI_LDS void*)(ks + wv * 512), 16, off, 0, 0, 0);
  const __amdgpu_buffer_rsrc_t rv = lc_rsrc(a.v + e0, rows * D * 2);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (INFINI_LDS void*)(vs + wv * 512), 16, off, 0, 0, 0);
#endif
}
}  // namespace

__global__ __launch_bounds__(kSgThreads, 1)
void lin_contrib_seg_kernel(LinContribArgs a) {
  constexpr int D = 128;
  constexpr int ST = kSgTt * D;                  // elements of a K or V stage
  static_assert(ST / kSgThreads == 8, "one 16-byte chunk of K per thread and stage");
  static_assert(kSgSlots == 8, "the stage loop is unrolled over the eight slots");
  // Each slot and buffer is an array of its own, and the loop is unrolled over
  // them: the compiler then sees that the LDS accesses of one slot never alias
  // the direct-to-LDS loads into another and does not wait for them.
  __shared__ __attribute__((aligned(1024))) bf16 ks0[ST], ks1[ST], ks2[ST], ks3[ST], ks4[ST], ks5[ST], ks6[ST],
      ks7[ST];
  __shared__ __attribute__((aligned(1024))) bf16 vs0[ST], vs1[ST], vs2[ST], vs3[ST], vs4[ST], vs5[ST], vs6[ST],
      vs7[ST];
  __shared__ __attribute__((aligned(1024))) bf16 kl0[ST], kl1[ST];   // lo parts of sigma(K)
  __shared__ float zred[kSgWaves * D];                             // per-wave column sums of sigma(K)

  const int nst = a.N / kSgTt;
  const int items = a.B * a.H * a.S;             // below 2^31 (checked by the host)
  const int G = (int)gridDim.x;
  const int lw = xcd_logical_block(blockIdx.x, G);
  if (lw >= items) return;
  const int total = ((items - lw + G - 1) / G) * nst;   // stream positions of this workgroup

  const int th = threadIdx.x, lane = th & 63, wave = th >> 6;
  // wave: C^T tiles (d_value block dv0, d_key block dkb) and (dv0 + 1, dkb), so a
  // 16-token step reads two V operands and one hi / lo pair of sigma(K) operands
  // (a tile pair along d_key would read one V operand and two pairs)
  const int dv0 = 2 * (wave & 1), dkb = wave >> 1;
  const int vofs0 = lc_tr_offset<D>(lane, dv0);
  const int vofs1 = lc_tr_offset<D>(lane, dv0 + 1);
  const int kofs = lc_tr_offset<D>(lane, dkb);
  // sigma(K) pass: row th / 16 of the stage, logical chunk th % 16, at its
  // physical position (the loads placed it there)
  const int srow = th >> 4, sch = th & 15;
  const int sdst = srow * D + 8 * lc_chunk<D>(srow, sch);

  // cur: the position being multiplied; ld: the next position to load
  SgPos cur;
  cur.q = 0;
  cur.k = 0;
  sg_item(a, lw, G, items, cur);
  SgPos ld = cur;
#define INFINI_SG_PRE(KS, VS)                 \
  sg_issue(a, ld, KS, VS, wave, lane);        \
  sg_advance(a, lw, G, items, nst, ld);
  INFINI_SG_PRE(ks0, vs0)
  INFINI_SG_PRE(ks1, vs1)
  INFINI_SG_PRE(ks2, vs2)
  INFINI_SG_PRE(ks3, vs3)
  INFINI_SG_PRE(ks4, vs4)
  INFINI_SG_PRE(ks5, vs5)
  INFINI_SG_PRE(ks6, vs6)
#undef INFINI_SG_PRE

  float zp[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) zp[i] = 0.f;
  f32x16 acc0, acc1;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc0[r] = acc1[r] = 0.f;

  // sigma(K) = hi + lo of elements [i0, i0 + n) of this thread's chunk (bf16
  // each) and its column sums (fp32)
  auto sigma_part = [&](const bf16x8& kx, bf16x8& h8, bf16x8& l8, int i0, int n) {
#pragma unroll
    for (int i = i0; i < i0 + n; ++i) {
      const float x = bf2f(kx[i]);
      const float f = x > 0.f ? x + 1.f : exp_e(x);
      zp[i] += f;
      h8[i] = f2bf(f);
      l8[i] = f2bf(f - bf2f(h8[i]));
    }
  };

  // End of an item: its two C^T tiles per wave and c, the column sums of
  // sigma(K) (over the 4 row positions of a wave by lane exchanges, then over
  // the waves in order).
  auto finish_item = [&](const SgPos& p, const float (&zf)[8]) {
    // lane-derived indices recomputed here behind an opaque value, so that the
    // store addresses are not hoisted out of the stage loop and kept live
    unsigned base = 0;
    asm volatile("" : "+v"(base));
    const int ln = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, base));
    float z[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float x = zf[i];
      x += __shfl_xor(x, 16);
      x += __shfl_xor(x, 32);
      z[i] = x;
    }
    if (ln < 16) {
#pragma unroll
      for (int i = 0; i < 8; ++i) zred[wave * D + 8 * ln + i] = z[i];
    }
    float* __restrict__ cm = a.cM + (int64_t)p.sh * D * D;
    const int hi = ln >> 5, l32 = ln & 31;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int dv = 32 * dv0 + 8 * (r >> 2) + 4 * hi + (r & 3);
      cm[dv * D + 32 * dkb + l32] = acc0[r];
      cm[(dv + 32) * D + 32 * dkb + l32] = acc1[r];
    }
    // barrier after this wave's LDS writes only: an LDS fence would also wait for
    // the ring's direct-to-LDS loads in flight
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    const int t = ln + 64 * wave;
    if (t < D) {
      float sum = 0.f;
#pragma unroll
      for (int w = 0; w < kSgWaves; ++w) sum += zred[w * D + t];
      a.cz[(int64_t)p.sh * D + t] = sum;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) acc0[r] = acc1[r] = 0.f;
    // zred is read above before the next item's writes (a barrier per stage
    // separates them)
  };

  // prologue: position 0 landed, its sigma(K) parts in place
  {
    constexpr int VM = 6 * kSgIpw;
    __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | 0x0F70);
    __builtin_amdgcn_s_barrier();
    const bf16x8 kx = *(const INFINI_LDS bf16x8*)(ks0 + sdst);
    bf16x8 h8, l8;
    sigma_part(kx, h8, l8, 0, 8);
    *(INFINI_LDS bf16x8*)(ks0 + sdst) = h8;
    *(INFINI_LDS bf16x8*)(kl0 + sdst) = l8;
  }
  // Iteration g: the products of position g (MFMA, slot g % 8, lo buffer g % 2)
  // interleaved with sigma(K) of position g+1 (VALU, in place in its slot, lo
  // into the other buffer); the loads of position g+7 (cursor ld) go into the
  // slot of position g-1, which every wave has finished reading at the barrier.
#define INFINI_SG_ITER(GI, KC, VC, KN, KLC, KLN, KLD, VLD)                                         \
  {                                                                                             \
    const int g_ = (GI);                                                                        \
    /* position g+1 has landed once at most positions g+2 .. g+6 are in flight */              \
    __builtin_amdgcn_s_waitcnt(((5 * kSgIpw) & 15) | (((5 * kSgIpw) >> 4) << 14) | 0x0070);     \
    __builtin_amdgcn_s_barrier();                                                               \
    sg_issue(a, ld, KLD, VLD, wave, lane);                                                      \
    sg_advance(a, lw, G, items, nst, ld);                                                       \
    if (g_ < total) {                                                                           \
      const bool more_ = g_ + 1 < total;                                                        \
      const bool last_ = cur.q + 1 == nst;   /* position g ends its item */                     \
      float zf_[8];                                                                             \
      if (last_) {                                                                              \
        _Pragma("unroll")                                                                       \
        for (int i = 0; i < 8; ++i) { zf_[i] = zp[i]; zp[i] = 0.f; }                            \
      }                                                                                         \
      /* all operand reads of the stage first: one LDS latency per stage */                     \
      const bf16x8 kx_ = *(const INFINI_LDS bf16x8*)(KN + sdst);                                \
      bf16x8 v0_[2], v1_[2], kh_[2], kl_[2];                                                    \
      _Pragma("unroll")                                                                         \
      for (int st = 0; st < 2; ++st) {                                                          \
        v0_[st] = lc_read_tr<D>(VC, 16 * st * D + vofs0);                                       \
        v1_[st] = lc_read_tr<D>(VC, 16 * st * D + vofs1);                                       \
        kh_[st] = lc_read_tr<D>(KC, 16 * st * D + kofs);                                        \
        kl_[st] = lc_read_tr<D>(KLC, 16 * st * D + kofs);                                       \
      }                                                                                         \
      bf16x8 h8_, l8_;                                                                          \
      _Pragma("unroll")                                                                         \
      for (int st = 0; st < 2; ++st) {                                                          \
        acc0 = mfma32(v0_[st], kh_[st], acc0);                                                  \
        acc0 = mfma32(v0_[st], kl_[st], acc0);                                                  \
        acc1 = mfma32(v1_[st], kh_[st], acc1);                                                  \
        acc1 = mfma32(v1_[st], kl_[st], acc1);                                                  \
        if (more_) sigma_part(kx_, h8_, l8_, 4 * st, 4);                                        \
      }                                                                                         \
      if (more_) {                                                                              \
        *(INFINI_LDS bf16x8*)(KN + sdst) = h8_;                                                 \
        *(INFINI_LDS bf16x8*)(KLN + sdst) = l8_;                                                \
      }                                                                                         \
      if (last_) finish_item(cur, zf_);                                                         \
      sg_advance(a, lw, G, items, nst, cur);                                                    \
    }                                                                                           \
  }
  // Iterations past the last position (when the position count is not a
  // multiple of eight) only wait, synchronise and issue empty loads: every load
  // is issued unconditionally, so the compiler tracks exactly which slots have
  // loads in flight and adds no waits of its own.
#pragma unroll 1
  for (int g = 0; g < total; g += 8) {
    INFINI_SG_ITER(g, ks0, vs0, ks1, kl0, kl1, ks7, vs7)
    INFINI_SG_ITER(g + 1, ks1, vs1, ks2, kl1, kl0, ks0, vs0)
    INFINI_SG_ITER(g + 2, ks2, vs2, ks3, kl0, kl1, ks1, vs1)
    INFINI_SG_ITER(g + 3, ks3, vs3, ks4, kl1, kl0, ks2, vs2)
    INFINI_SG_ITER(g + 4, ks4, vs4, ks5, kl0, kl1, ks3, vs3)
    INFINI_SG_ITER(g + 5, ks5, vs5, ks6, kl1, kl0, ks4, vs4)
    INFINI_SG_ITER(g + 6, ks6, vs6, ks7, kl0, kl1, ks5, vs5)
    INFINI_SG_ITER(g + 7, ks7, vs7, ks0, kl1, kl0, ks6, vs6)
  }
#undef INFINI_SG_ITER
  __builtin_amdgcn_s_waitcnt(0);
}

// v moved across lanes by the DPP control CTRL; lanes outside ROW_MASK (rows of 16
// lanes) get old.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_move(float old, float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old), __builtin_bit_cast(int, v),
                                                               CTRL, ROW_MASK, 0xf, false));
}

// Sum over each group of TPR (32 or 64) consecutive lanes in a fixed order, on
// DPP lane moves (no LDS): quad sums, then half rows and rows of 16 lanes by
// mirrors, then rows combined by broadcasts.  The group's last lane holds the sum.
template <int TPR>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp_move<0xB1, 0xf>(0.f, x);    // quad_perm [1, 0, 3, 2]
  x += dpp_move<0x4E, 0xf>(0.f, x);    // quad_perm [2, 3, 0, 1]
  x += dpp_move<0x141, 0xf>(0.f, x);   // row_half_mirror
  x += dpp_move<0x140, 0xf>(0.f, x);   // row_mirror
  x += dpp_move<0x142, 0xa>(0.f, x);   // row_bcast:15 into rows 1 and 3
  if (TPR == 64) x += dpp_move<0x143, 0xc>(0.f, x);   // row_bcast:31 into rows 2 and 3
  return x;
}

// Exclusive prefix over segments.  Each thread carries two adjacent elements of
// one row of M^T (a row of d_key elements is one wave at d = 128, half a wave at
// d = 64), so the snapshot's column sum of M (row sum of M^T) is a reduction over
// the lanes of a wave with no LDS or barrier; the last workgroup of each head
// carries z.  The
// contributions of the next kPf segments are loaded while the current kPf are
// folded in, so the chain over segments runs at arithmetic speed instead of one
// memory latency per segment.
constexpr int kPf = 16;

template <int D>
__global__ __launch_bounds__(kThreads)
void lin_scan_kernel(LinScanArgs a) {
  constexpr int MB = D * D / (2 * kThreads);   // workgroups holding M^T per head
  constexpr int TPR = D / 2;                   // threads per row of M^T
  static_assert(D * D % (2 * kThreads) == 0 && (TPR == 64 || TPR == 32), "shape");
  const int bh = blockIdx.x / (MB + 1);
  const int sub = blockIdx.x % (MB + 1);
  const int64_t base = (int64_t)bh * a.S;
  if (sub == MB) {
    const int dk = threadIdx.x;
    if (dk >= D) return;
    float run = a.z[(int64_t)bh * D + dk];
    float cur[kPf], nxt[kPf];
#pragma unroll
    for (int i = 0; i < kPf; ++i) cur[i] = i < a.S ? a.cz[(base + i) * D + dk] : 0.f;
    for (int s0 = 0; s0 < a.S; s0 += kPf) {
#pragma unroll
      for (int i = 0; i < kPf; ++i) nxt[i] = s0 + kPf + i < a.S ? a.cz[(base + s0 + kPf + i) * D + dk] : 0.f;
#pragma unroll
      for (int i = 0; i < kPf; ++i) {
        if (s0 + i < a.S) {
          a.snapz[(base + s0 + i) * D + dk] = run;
          run += cur[i];
        }
      }
#pragma unroll
      for (int i = 0; i < kPf; ++i) cur[i] = nxt[i];
    }
    a.z[(int64_t)bh * D + dk] = run;
    return;
  }
  const int e = 2 * (sub * kThreads + threadIdx.x);   // elements e, e + 1 of M^T
  const int dv = e / D, dk = e % D;
  const float* __restrict__ cm = a.cM + base * D * D + e;
  const float* __restrict__ m0 = a.M + (int64_t)bh * D * D;
  float r0 = m0[dk * D + dv], r1 = m0[(dk + 1) * D + dv];
  float2 cur[kPf], nxt[kPf];
#pragma unroll
  for (int i = 0; i < kPf; ++i)
    cur[i] = i < a.S ? *reinterpret_cast<const float2*>(cm + (int64_t)i * D * D) : make_float2(0.f, 0.f);
  for (int s0 = 0; s0 < a.S; s0 += kPf) {
#pragma unroll
    for (int i = 0; i < kPf; ++i)
      nxt[i] = s0 + kPf + i < a.S ? *reinterpret_cast<const float2*>(cm + (int64_t)(s0 + kPf + i) * D * D)
                                  : make_float2(0.f, 0.f);
#pragma unroll
    for (int i = 0; i < kPf; ++i) {
      if (s0 + i < a.S) {
        const int64_t sh = base + s0 + i;
        bf16x2 pk, pl;
        pk[0] = f2bf(r0);
        pk[1] = f2bf(r1);
        pl[0] = f2bf(r0 - bf2f(pk[0]));
        pl[1] = f2bf(r1 - bf2f(pk[1]));
        *reinterpret_cast<bf16x2*>(a.snapM + sh * D * D + e) = pk;
        *reinterpret_cast<bf16x2*>(a.snapMlo + sh * D * D + e) = pl;
        const float c = group_sum<TPR>(r0 + r1);
        if (threadIdx.x % TPR == TPR - 1) a.snapc[sh * D + dv] = c;
        r0 += cur[i].x;
        r1 += cur[i].y;
      }
    }
#pragma unroll
    for (int i = 0; i < kPf; ++i) cur[i] = nxt[i];
  }
  float* __restrict__ mout = a.M + (int64_t)bh * D * D;
  mout[dk * D + dv] = r0;
  mout[(dk + 1) * D + dv] = r1;
}

// ------------------------------------------------------------------ launchers
int device_compute_units() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <int D>
hipError_t launch_lin_contrib(const LinContribArgs& a, hipStream_t stream) {
  if (a.N % kLcTt != 0) return hipErrorInvalidValue;
  // whole segments per workgroup once there are at least as many segments as
  // compute units; below that, half segments (twice the workgroups) fill the
  // chip better
  if (D == 128 && (int64_t)a.B * a.H * a.S >= device_compute_units()) {
    const int64_t items = (int64_t)a.B * a.H * a.S;
    // one persistent workgroup per compute unit (the LDS use allows one)
    const int64_t cus = device_compute_units();
    const int64_t blocks = items < cus ? items : cus;
    const int64_t positions = (items + blocks - 1) / blocks * (a.N / kSgTt);
    if (items > 0x7fffffff || positions + kSgSlots > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(lin_contrib_seg_kernel, dim3((unsigned)blocks), dim3(kSgThreads), 0, stream, a);
    return hipGetLastError();
  }
  const int64_t blocks = (int64_t)a.B * a.H * a.S * (D / kLcKb);
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(lin_contrib_kernel<D>, dim3((unsigned)blocks), dim3(kLcThreads), 0, stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_lin_scan(const LinScanArgs& a, hipStream_t stream) {
  const int64_t blocks = (int64_t)a.BH * (D * D / (2 * kThreads) + 1);
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(lin_scan_kernel<D>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template hipError_t launch_lin_contrib<64>(const LinContribArgs&, hipStream_t);
template hipError_t launch_lin_contrib<128>(const LinContribArgs&, hipStream_t);
template hipError_t launch_lin_scan<64>(const LinScanArgs&, hipStream_t);
template hipError_t launch_lin_scan<128>(const LinScanArgs&, hipStream_t);

}  // namespace infini
