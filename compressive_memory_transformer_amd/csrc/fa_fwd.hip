// Fused segment kernel for the bf16 path: local causal attention (flash style,
// online softmax in fp32), retrieval from the compressive memory snapshot,
// sigmoid gate, bf16 output.
//
// Equations (page "精读笔记：Infini-attention"): A_dot of section 3.1 with the
// causal mask of section 3.8 step 2, restricted to the current segment; A_mem of
// section 3.3; the gate of section 3.5.  The N x N score matrix never leaves
// registers (chapter-24 page, section 24.1.2).
//
// Work decomposition.  One workgroup = 4 waves = one pair of 128-row query tiles
// of one (b, h, segment): tile w and tile NQ-1-w, so every workgroup does the
// same amount of causal work.  Wave v owns 32 query rows.  Per 64-key tile:
//   S^T (64 keys x 32 queries) = K Q^T on v_mfma_f32_32x32x16_bf16, so that each
//   lane holds one query column and the softmax row statistics are per lane (one
//   cross-lane exchange with lane l^32 for the other half of the keys);
//   O^T (D x 32) += V^T P^T, with V^T read from the row-major V tile in LDS by
//   ds_read_b64_tr_b16 and P^T taken straight from the S^T accumulators (the key
//   order inside each 16-key step is permuted identically on both operands).
// Epilogue: A_mem^T = M^T sigma(Q)^T on MFMA from the bf16 snapshot of M_{s-1}^T,
// denominator sigma(Q) z_{s-1} in fp32, gate, round to bf16, store.
#include "common.h"
#include "kernels.h"

namespace infini {

namespace {

constexpr int kBM = 128;   // query rows per tile (4 waves x 32)
constexpr int kBN = 64;    // keys per LDS tile
constexpr int kThreads = 256;

template <int D>
struct FaLayout {
  static constexpr int KP = D + 8;    // K row pitch: conflict-free ds_read_b128 on 8-lane phases
  static constexpr int VP = D + 16;   // V row pitch: 4 rows x 32 B of a tr16 group hit distinct banks
  static constexpr int K_ELEMS = kBN * KP;
  static constexpr int V_ELEMS = kBN * VP;
  static constexpr int TOTAL = 2 * K_ELEMS + 2 * V_ELEMS;  // double-buffered K and V
  // The epilogue reuses both K buffers for the D x D snapshot of M^T (pitch KP).
  static_assert(D * KP <= 2 * K_ELEMS, "snapshot does not fit the K buffers");
  static constexpr int PASSES = (kBN * D / 8) / kThreads;  // 16-byte chunks per thread per tile
  static constexpr int TPR = D / 8;                         // threads per row
  static constexpr int RPP = kThreads / TPR;                // rows per pass
};

template <int D>
__device__ __forceinline__ void load_tile_regs(const bf16* __restrict__ src, int row0, u32x4 (&regs)[FaLayout<D>::PASSES]) {
  using L = FaLayout<D>;
  const int t = threadIdx.x;
  const int col = (t % L::TPR) * 8;
#pragma unroll
  for (int p = 0; p < L::PASSES; ++p) {
    const int row = row0 + t / L::TPR + p * L::RPP;
    regs[p] = *reinterpret_cast<const u32x4*>(src + (int64_t)row * D + col);
  }
}

template <int D, int PITCH>
__device__ __forceinline__ void store_tile_lds(bf16* dst, const u32x4 (&regs)[FaLayout<D>::PASSES]) {
  using L = FaLayout<D>;
  const int t = threadIdx.x;
  const int col = (t % L::TPR) * 8;
#pragma unroll
  for (int p = 0; p < L::PASSES; ++p) {
    const int row = t / L::TPR + p * L::RPP;
    *(INFINI_LDS u32x4*)(dst + row * PITCH + col) = regs[p];
  }
}

}  // namespace

template <int D>
__global__ __launch_bounds__(kThreads, 2)
void fa_fwd_kernel(FaArgs a) {
  using L = FaLayout<D>;
  __shared__ __attribute__((aligned(16))) bf16 smem[L::TOTAL];
  __shared__ float zsh[D];

  const int npair = (a.nq + 1) / 2;
  const int blk = xcd_logical_block(blockIdx.x, gridDim.x);
  const int sh = blk / npair;            // (b*H + h) * S + s
  const int pair = blk % npair;
  const int bh = sh / a.S;
  const int s = sh % a.S;
  const int h = bh % a.H;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int grp = lane >> 4;
  const int sidx = lane & 15;

  const int64_t tok0 = (int64_t)bh * a.L + (int64_t)s * a.N;
  const bf16* __restrict__ qb = a.q + tok0 * D;
  const bf16* __restrict__ kb = a.k + tok0 * D;
  const bf16* __restrict__ vb = a.v + tok0 * D;
  bf16* __restrict__ ob = a.out + tok0 * D;

  const bool has_memory = (a.seg_base + s) > 0;
  const float g = sigmoid_gate(a.beta[h]);
  const float sc = a.sc_log2;
  const int nk = a.N / kBN;


  for (int pass = 0; pass < 2; ++pass) {
    const int qt = pass == 0 ? pair : a.nq - 1 - pair;
    if (pass == 1 && qt == pair) break;
    const int q0 = qt * kBM;
    const int r0 = q0 + 32 * wave;            // first query row of this wave
    const bool active = r0 < a.N;
    const int my_row = r0 + l32;               // query of this lane

    // Q^T as the B operand: lane holds Q[my_row][16c + 8hi .. +7].
    bf16x8 qreg[D / 16];
    if (active) {
#pragma unroll
      for (int c = 0; c < D / 16; ++c)
        qreg[c] = *reinterpret_cast<const bf16x8*>(qb + (int64_t)my_row * D + 16 * c + 8 * hi);
    }

    f32x16 o[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
    float m_run = -__builtin_inff();
    float l_run = 0.f;

    const int last = min(nk - 1, (q0 + kBM - 1) / kBN);
    u32x4 pk[L::PASSES], pv[L::PASSES];
    load_tile_regs<D>(kb, 0, pk);
    load_tile_regs<D>(vb, 0, pv);
    store_tile_lds<D, L::KP>(smem, pk);
    store_tile_lds<D, L::VP>(smem + 2 * L::K_ELEMS, pv);
    __syncthreads();

    for (int kt = 0; kt <= last; ++kt) {
      const int cur = kt & 1;
      if (kt < last) {
        load_tile_regs<D>(kb, (kt + 1) * kBN, pk);
        load_tile_regs<D>(vb, (kt + 1) * kBN, pv);
      }
      const int k0 = kt * kBN;
      if (active && k0 <= r0 + 31) {
        const bf16* kt_lds = smem + cur * L::K_ELEMS;
        const bf16* vt_lds = smem + 2 * L::K_ELEMS + cur * L::V_ELEMS;
        // ---- S^T = K Q^T for two 32-key blocks
        f32x16 sacc[2];
#pragma unroll
        for (int b2 = 0; b2 < 2; ++b2) {
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[b2][r] = 0.f;
#pragma unroll
          for (int c = 0; c < D / 16; ++c) {
            bf16x8 ka = lds_read8(kt_lds + (32 * b2 + l32) * L::KP + 16 * c + 8 * hi);
            sacc[b2] = mfma32(ka, qreg[c], sacc[b2]);
          }
        }
        // ---- causal mask (only tiles that reach past the wave's first row)
        if (k0 + kBN - 1 > r0) {
#pragma unroll
          for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = k0 + 32 * b2 + 8 * (r >> 2) + 4 * hi + (r & 3);
              if (key > my_row) sacc[b2][r] = -__builtin_inff();
            }
        }
        // ---- online softmax (log2 domain)
        float mx = -__builtin_inff();
#pragma unroll
        for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[b2][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx * sc);
        const float alpha = exp2_fast(m_run - m_new);
        m_run = m_new;
        float psum = 0.f;
        bf16x8 pb[2][2];
#pragma unroll
        for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
          for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const float p = exp2_fast(__builtin_fmaf(sacc[b2][8 * hf + i], sc, -m_new));
              psum += p;
              pb[b2][hf][i] = f2bf(p);
            }
        l_run = l_run * alpha + psum;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
        // ---- O^T += V^T P^T
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
              const int base = 32 * b2 + 16 * hf + 4 * hi;
              bf16x8 va = lds_operand_tr(vt_lds, L::VP, base, base + 8, 32 * db + 16 * (grp & 1), sidx);
              o[db] = mfma32(va, pb[b2][hf], o[db]);
            }
      }
      if (kt < last) {
        store_tile_lds<D, L::KP>(smem + (cur ^ 1) * L::K_ELEMS, pk);
        store_tile_lds<D, L::VP>(smem + 2 * L::K_ELEMS + (cur ^ 1) * L::V_ELEMS, pv);
      }
      __syncthreads();
    }

    // ---- normalise the local attention
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv_l = 1.f / l_tot;

    // ---- retrieval epilogue: stage the M^T snapshot (bf16, D x D) and z in LDS
    f32x16 am[D / 32];
    float den = 0.f;
    if (has_memory) {
      const bf16* mt = a.snapM + (int64_t)sh * D * D;
      const float* zs = a.snapz + (int64_t)sh * D;
      bf16* mt_lds = smem;
      for (int i = threadIdx.x; i < D * D / 8; i += kThreads) {
        const int row = i / (D / 8), col = (i % (D / 8)) * 8;
        *(INFINI_LDS u32x4*)(mt_lds + row * L::KP + col) = *reinterpret_cast<const u32x4*>(mt + row * D + col);
      }
      for (int i = threadIdx.x; i < D; i += kThreads) zsh[i] = zs[i];
      __syncthreads();
      if (active) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) am[db][r] = 0.f;
#pragma unroll
        for (int c = 0; c < D / 16; ++c) {
          bf16x8 sq;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float f = elu1(bf2f(qreg[c][i]));
            den = __builtin_fmaf(f, zsh[16 * c + 8 * hi + i], den);
            sq[i] = f2bf(f);
          }
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            bf16x8 ma = lds_read8(mt_lds + (32 * db + l32) * L::KP + 16 * c + 8 * hi);
            am[db] = mfma32(ma, sq, am[db]);
          }
        }
        den += __shfl_xor(den, 32);
      }
      __syncthreads();  // LDS is reused by the next tile pair
    }

    // ---- gate and store: lane holds query my_row, values d = 32db + 8j + 4hi + 0..3
    if (active) {
      const float inv_den = (has_memory && den > 0.f) ? 1.f / den : 0.f;
      const float wg_mem = g * inv_den;
      const float wg_dot = (1.f - g) * inv_l;
      bf16* orow = ob + (int64_t)my_row * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          bf16x4 outv;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float mem = has_memory ? am[db][4 * j + e] * wg_mem : 0.f;
            outv[e] = f2bf(__builtin_fmaf(o[db][4 * j + e], wg_dot, mem));
          }
          *reinterpret_cast<bf16x4*>(orow + 32 * db + 8 * j + 4 * hi) = outv;
        }
    }
  }
}

template <int D>
hipError_t launch_fa_fwd(const FaArgs& a, hipStream_t stream) {
  const int npair = (a.nq + 1) / 2;
  const int64_t blocks = (int64_t)a.B * a.H * a.S * npair;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(fa_fwd_kernel<D>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template hipError_t launch_fa_fwd<64>(const FaArgs&, hipStream_t);
template hipError_t launch_fa_fwd<128>(const FaArgs&, hipStream_t);

}  // namespace infini
