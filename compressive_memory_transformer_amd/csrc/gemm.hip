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
// Tiling: large products run the 256 x 256 kernel below (direct-to-LDS loads
// through a 4-slot ring); small ones one workgroup per 128 x 128 output tile
// (4 waves of 64 x 64), K in steps of 64 staged through two LDS buffers (the
// next step's global loads issued before the current step's products).  Both on
// v_mfma_f32_32x32x16_bf16 tiles, A read by rows from LDS and B (row-major
// [K][N]) through the transposing LDS read.
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

// Large products: 256 x 256 output tiles, 8 waves of 128 (rows of C) x 64
// (columns), K in stages of 32 through a 4-slot LDS ring filled by
// buffer_load ... lds three stages ahead (no staging registers, one barrier per
// stage).  The tile order is XCD-grouped: the N tiles of one row block of A run
// on one XCD and share its L2.  Each wave computes C^T blocks (MFMA A operand =
// W^T from the [K][N] tile by transposing reads, B operand = A^T from the
// row-major A tile by plain 16-byte reads), so that a lane holds 4 consecutive
// columns of a row of C; the result leaves through LDS as whole 128-byte row
// segments.
// Slot layouts (16-byte chunks swizzled by an XOR, so that the operand reads
// are free of bank conflicts): A tile [256 rows][32 k] (64 bytes a row), chunk c
// of row r at c ^ ((r / 4) % 4); W tile [32 k][256 columns] (512 bytes a row),
// chunk c of row r at c ^ 4 (r % 4).
namespace {
constexpr int kG2M = 256, kG2N = 256, kG2K = 32;
constexpr int kG2Waves = 8, kG2Threads = 64 * kG2Waves;
constexpr int kG2Slots = 4;        // ring slots (three stages in flight; the stage loop is unrolled over them)
constexpr int kG2Ipw = 4;        // loads per wave and stage: two 1 KB pieces of A, two of W

__device__ __forceinline__ int g2_a_chunk(int r, int c) { return c ^ ((r >> 2) & 3); }
__device__ __forceinline__ int g2_w_chunk(int r, int c) { return c ^ ((r & 3) << 2); }

#if defined(__HIP_DEVICE_COMPILE__)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t g2_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  void* ub = (void*)(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}
#endif

// Per-lane pieces of one stage's loads: a_off[j] (element offset of this lane's
// 16 bytes of A for piece j, relative to the A base, k0 = 0; rows past M are
// clamped to row M - 1) and w_off[j] (relative to the W tile's first element).
// With the head layout of A a row's 32-column stage lies inside one head
// (d_value a multiple of 32), so its 16-byte pieces stay contiguous.
struct G2Lane {
  int64_t a_row[2];     // element offset of this lane's A row (k = 0)
  int a_col[2];         // this lane's column within a stage (8 * logical chunk)
  int w_off[2];
};
}  // namespace

__global__ __launch_bounds__(kG2Threads, 1)
void gemm_bf16_big_kernel(GemmArgs g) {
  constexpr int AT = kG2M * kG2K, WT = kG2K * kG2N;     // elements of an A / W stage
  static_assert(kG2Slots == 4, "the stage loop is unrolled over the four slots");
  __shared__ __attribute__((aligned(1024))) bf16 as0[AT], as1[AT], as2[AT], as3[AT];
  __shared__ __attribute__((aligned(1024))) bf16 ws0[WT], ws1[WT], ws2[WT], ws3[WT];

  const int ntn = (g.N + kG2N - 1) / kG2N, ntm = (g.M + kG2M - 1) / kG2M;
  const int blk = xcd_logical_block(blockIdx.x, gridDim.x);
  if (blk >= ntn * ntm) return;
  const int mt = blk / ntn, nt = blk % ntn;
  const int m0 = mt * kG2M, n0 = nt * kG2N;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int hi = lane >> 5, l32 = lane & 31;
  const int wm = 128 * (wave >> 2), wn = 64 * (wave & 3);   // the wave's corner of the tile
  const int nst = g.K / kG2K;

  // load pieces: A piece j of this wave covers rows 16 (2 w + j) + lane / 4;
  // W piece j covers rows 2 (2 w + j) + lane / 32
  G2Lane L;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int ins = 2 * wv + j;
    const int ar = 16 * ins + lane / 4, ac = 8 * g2_a_chunk(ar, lane % 4);
    const int m = min(m0 + ar, g.M - 1);
    if (g.a_heads) {
      const int b = m / g.L, t = m % g.L;
      L.a_row[j] = ((int64_t)b * g.H * g.L + t) * g.dv;   // head 0; + h L dv per head
    } else {
      L.a_row[j] = (int64_t)m * g.K;
    }
    L.a_col[j] = ac;
    const int wr = 2 * ins + lane / 32;
    L.w_off[j] = wr * g.N + 8 * g2_w_chunk(wr, lane % 32);
  }
#if defined(__HIP_DEVICE_COMPILE__)
  const __amdgpu_buffer_rsrc_t ra = g2_rsrc(g.a, (uint32_t)g.M * g.K * 2);   // rows are clamped below M
  const uint32_t wbytes = (uint32_t)g.K * g.N * 2;
#endif
  auto issue = [&](int s, bf16* as, bf16* ws) {
#if defined(__HIP_DEVICE_COMPILE__)
    const bool in = s < nst;
    const int k0 = in ? s * kG2K : 0;
    // A: this stage's head (head layout) or columns k0 .. k0 + 31
    int64_t acol;
    if (g.a_heads) {
      const int h = k0 / g.dv, c = k0 % g.dv;
      acol = (int64_t)h * g.L * g.dv + c;
    } else {
      acol = k0;
    }
    const __amdgpu_buffer_rsrc_t rw = g2_rsrc(g.b + (int64_t)k0 * g.N + n0, in ? wbytes - (uint32_t)(k0 * g.N + n0) * 2 : 0u);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int ins = 2 * wv + j;
      const int64_t ae = L.a_row[j] + acol + L.a_col[j];
      // per-lane byte offset from the tensor base; a piece past the last stage
      // re-reads stage 0 (its slot is never multiplied)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (INFINI_LDS void*)(as + ins * 512), 16, (int)(ae * 2), 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (INFINI_LDS void*)(ws + ins * 512), 16, L.w_off[j] * 2, 0, 0, 0);
    }
#endif
  };

  // operand read offsets (elements, relative to a slot)
  // B operand (A^T, 32 rows of the wave's m block mb): row wm + 32 mb + l32, k chunk 2 ks + hi
  int aoff[4][2];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int r = wm + 32 * mb + l32;
      aoff[mb][ks] = r * kG2K + 8 * g2_a_chunk(r, 2 * ks + hi);
    }
  // A operand (W^T, 32 columns of the wave's n block nb) by two transposing reads:
  // rows 16 ks + 8 hi + sidx / 4 (+ 4), columns wn + 32 nb + 16 (grp % 2) + 4 (sidx % 4)
  int woff[2][2];
  {
    const int grp = lane >> 4, sidx = lane & 15;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int r = 16 * ks + 8 * hi + (sidx >> 2);
        const int col = wn + 32 * nb + 16 * (grp & 1) + 4 * (sidx & 3);
        woff[nb][ks] = r * kG2N + 8 * g2_w_chunk(r, col >> 3) + (col & 7);
      }
  }

  f32x16 acc[2][4];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[nb][mb][r] = 0.f;

  issue(0, as0, ws0);
  issue(1, as1, ws1);
  issue(2, as2, ws2);

  // Stage s: products from slot s % 4; the loads of stage s + 3 go into the slot
  // of stage s - 1, which every wave has finished reading at the barrier.
#define INFINI_G2_STAGE(S, AC, WC, AL, WL)                                                       \
  {                                                                                             \
    const int s_ = (S);                                                                         \
    /* stage s has landed once at most stages s+1, s+2 are in flight */                         \
    __builtin_amdgcn_s_waitcnt(((2 * kG2Ipw) & 15) | (((2 * kG2Ipw) >> 4) << 14) | 0x0070);     \
    __builtin_amdgcn_s_barrier();                                                               \
    issue(s_ + 3, AL, WL);                                                                      \
    if (s_ < nst) {                                                                             \
      _Pragma("unroll")                                                                         \
      for (int ks = 0; ks < 2; ++ks) {                                                          \
        bf16x8 bo[4], ao[2];                                                                    \
        _Pragma("unroll")                                                                       \
        for (int mb = 0; mb < 4; ++mb) bo[mb] = lds_read8(AC + aoff[mb][ks]);                   \
        _Pragma("unroll")                                                                       \
        for (int nb = 0; nb < 2; ++nb) {                                                        \
          const s16x4 x = lds_read_tr16(WC + woff[nb][ks]);                                     \
          const s16x4 y = lds_read_tr16(WC + woff[nb][ks] + 4 * kG2N);                          \
          ao[nb] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7)); \
        }                                                                                       \
        _Pragma("unroll")                                                                       \
        for (int nb = 0; nb < 2; ++nb)                                                          \
          _Pragma("unroll")                                                                     \
          for (int mb = 0; mb < 4; ++mb) acc[nb][mb] = mfma32(ao[nb], bo[mb], acc[nb][mb]);      \
      }                                                                                         \
    }                                                                                           \
  }
#pragma unroll 1
  for (int s = 0; s < nst; s += 4) {
    INFINI_G2_STAGE(s, as0, ws0, as3, ws3)
    INFINI_G2_STAGE(s + 1, as1, ws1, as0, ws0)
    INFINI_G2_STAGE(s + 2, as2, ws2, as1, ws1)
    INFINI_G2_STAGE(s + 3, as3, ws3, as2, ws2)
  }
#undef INFINI_G2_STAGE
  __builtin_amdgcn_s_waitcnt(0);

  // Epilogue through LDS: acc[nb][mb] element r of lane l is C[m][n] with
  // m = wm + 32 mb + l32, n = wn + 32 nb + 8 (r / 4) + 4 hi + r % 4 (relative to
  // the tile).  Each wave writes its 128 x 64 block as bf16 into one 16 KB ring
  // array (row-major, 16-byte chunk c of row m at c ^ (m % 8)), then reads it
  // back 8 rows at a time so that every global store covers a whole 128-byte
  // row segment.
  __builtin_amdgcn_s_waitcnt(0);   // the ring's loads (past the last stage too) have landed
  __builtin_amdgcn_s_barrier();    // and every wave has finished reading it
  bf16* const st = wave == 0 ? as0 : wave == 1 ? as1 : wave == 2 ? as2 : wave == 3 ? as3
                 : wave == 4 ? ws0 : wave == 5 ? ws1 : wave == 6 ? ws2 : ws3;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const int m = 32 * mb + l32;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = f2bf(acc[nb][mb][4 * j + e]);
        const int pc = (4 * nb + j) ^ (m & 7);
        *(INFINI_LDS bf16x4*)(st + m * 64 + 8 * pc + 4 * hi) = v4;
      }
  }
  // the block is private to the wave and LDS runs a wave's accesses in order
  // this lane's 16-byte column chunk c (fixed: the rows it reads all have the
  // same row % 8) and its destination; rows advance by 8 per read
  const int pc = lane & 7, r0 = lane >> 3;
  const int c = pc ^ (r0 & 7);
  const int n = n0 + wn + 8 * c;
  bf16* cbase;
  int64_t cpart;
  int cd;
  if (g.c_heads) {
    // a query, key or value head (d_key and d_value multiples of 8, so the 8
    // columns stay in one head)
    const int nq = g.H * g.dk;
    int hq, cc;
    if (n < nq) { cbase = g.q; hq = n / g.dk; cc = n % g.dk; cd = g.dk; }
    else if (n < 2 * nq) { cbase = g.k; hq = (n - nq) / g.dk; cc = (n - nq) % g.dk; cd = g.dk; }
    else { cbase = g.v; hq = (n - 2 * nq) / g.dv; cc = (n - 2 * nq) % g.dv; cd = g.dv; }
    cpart = (int64_t)hq * g.L * cd + cc;
  } else {
    cbase = g.c;
    cpart = n;
    cd = g.N;
  }
  int m = m0 + wm + r0;
  int b = m / g.L, t = m % g.L;   // head layout: row (b, t)
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const bf16x8 x = *(const INFINI_LDS bf16x8*)(st + (8 * i + r0) * 64 + 8 * pc);
    if (m < g.M && n < g.N) {
      const int64_t rp = g.c_heads ? (int64_t)b * g.H * g.L + t : (int64_t)m;
      *reinterpret_cast<bf16x8*>(cbase + rp * cd + cpart) = x;
    }
    m += 8;
    t += 8;
    while (t >= g.L) { t -= g.L; ++b; }
  }
}

hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t stream) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  if (g.K % kGK != 0 || g.N % 8 != 0) return hipErrorInvalidValue;
  // 256 x 256 tiles once there are enough of them to fill the chip (and the
  // operands' byte offsets fit the 32-bit buffer offsets)
  const int64_t big = ((int64_t)(g.M + 255) / 256) * ((g.N + 255) / 256);
  if (big >= 256 && (int64_t)g.M * g.K * 2 < 0x7fffffff && (int64_t)g.K * g.N * 2 < 0x7fffffff) {
    hipLaunchKernelGGL(gemm_bf16_big_kernel, dim3((unsigned)big), dim3(kG2Threads), 0, stream, g);
  } else {
    const dim3 grid((unsigned)((g.N + 127) / 128), (unsigned)((g.M + 127) / 128));
    hipLaunchKernelGGL((gemm_bf16_kernel<128, 128, 64, 64>), grid, dim3(256), 0, stream, g);
  }
  return hipGetLastError();
}

}  // namespace infini
