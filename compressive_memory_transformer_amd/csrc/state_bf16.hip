// Linear-rule memory state of the bf16 path (page "精读笔记：Infini-attention",
// section 3.4, linear rule; z as in section 3.3):
//
//   M_s = M_{s-1} + sigma(K)^T V,   z_s = z_{s-1} + sum_t sigma(K_t)
//
// It leaves a snapshot of (M_{s-1}^T in bf16, z_{s-1} and colsum(M_{s-1}) in
// fp32) per segment for the fused attention kernel and the final (M_S, z_S) in
// the fp32 state.  The delta rule lives in state_delta.hip.
//
// Precision.  sigma(K) = 1 + k for the small keys of these workloads, so rounding
// sigma(K) to bf16 keeps only a few bits of k.  The contribution GEMM therefore
// splits sigma(K) into bf16 hi + lo parts (x = hi + lo to about 16 bits) and sums
// the hi*V and lo*V products in fp32 (V is exact in bf16).
#include "common.h"
#include "kernels.h"

namespace infini {

namespace {
constexpr int kThreads = 256;

// x = hi + lo with hi = bf16(x), lo = bf16(x - hi).
__device__ __forceinline__ bf16 lo_part(float x, bf16 hi) { return f2bf(x - bf2f(hi)); }
}  // namespace

// =================================================================== linear
// One workgroup per (b, h, s, 32-column block of d_key).  sigma(K) of the block
// is computed once per element (split into bf16 hi + lo) and staged in LDS with
// V (row-major); the contraction over tokens reads both operands transposed with
// ds_read_b64_tr_b16.  Output C^T[d_value][d_key block] on
// v_mfma_f32_32x32x16_bf16, plus c[d_key block] = sum_t sigma(K_t).  The next
// 64-token tile is prefetched into registers while the current one is used.
template <int D>
__global__ __launch_bounds__(kThreads, 2)
void lin_contrib_kernel(LinContribArgs a) {
  constexpr int KB = 32;               // d_key columns per workgroup
  constexpr int NKB = D / KB;
  constexpr int KP = KB + 16;          // sigma(K) tile pitch: 4 rows x 32 B of a tr16 group on distinct banks
  constexpr int VP = D + 16;           // V tile pitch
  constexpr int VCH = D / 8;           // 16-byte chunks per V row
  constexpr int VPT = 64 * VCH / kThreads;
  constexpr int NDVB = D / 32;         // 32-row blocks of d_value = output blocks
  constexpr int WPB = 4 / NDVB;        // waves sharing one output block (token-interleaved)
  __shared__ __attribute__((aligned(16))) bf16 khi[64 * KP];
  __shared__ __attribute__((aligned(16))) bf16 klo[64 * KP];
  __shared__ __attribute__((aligned(16))) bf16 vt[64 * VP];
  __shared__ float zred[64][KB + 1];

  const int blk = xcd_logical_block(blockIdx.x, gridDim.x);
  const int sh = blk / NKB, dkb = blk % NKB;
  const int bh = sh / a.S, s = sh % a.S;
  const int64_t tok0 = (int64_t)bh * a.L + (int64_t)s * a.N;
  const bf16* __restrict__ kb = a.k + tok0 * D + dkb * KB;
  const bf16* __restrict__ vb = a.v + tok0 * D;

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int hi = lane >> 5, grp = lane >> 4, sidx = lane & 15, l32 = lane & 31;
  const int krow = t >> 2, kch = t & 3;            // this thread's 16-byte chunk of the K block
  const int dvb = wave % NDVB, part = wave / NDVB;

  bf16x8 kx = *reinterpret_cast<const bf16x8*>(kb + (int64_t)krow * D + kch * 8);
  u32x4 vx[VPT];
#pragma unroll
  for (int p = 0; p < VPT; ++p) {
    const int c = t + kThreads * p;
    vx[p] = *reinterpret_cast<const u32x4*>(vb + (int64_t)(c / VCH) * D + (c % VCH) * 8);
  }
  float zp[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) zp[i] = 0.f;
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;

  for (int t0 = 0; t0 < a.N; t0 += 64) {
    bf16x8 h8, l8;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float f = elu1(bf2f(kx[i]));
      zp[i] += f;
      h8[i] = f2bf(f);
      l8[i] = lo_part(f, h8[i]);
    }
    *(INFINI_LDS bf16x8*)(khi + krow * KP + kch * 8) = h8;
    *(INFINI_LDS bf16x8*)(klo + krow * KP + kch * 8) = l8;
#pragma unroll
    for (int p = 0; p < VPT; ++p) {
      const int c = t + kThreads * p;
      *(INFINI_LDS u32x4*)(vt + (c / VCH) * VP + (c % VCH) * 8) = vx[p];
    }
    if (t0 + 64 < a.N) {
      kx = *reinterpret_cast<const bf16x8*>(kb + (int64_t)(t0 + 64 + krow) * D + kch * 8);
#pragma unroll
      for (int p = 0; p < VPT; ++p) {
        const int c = t + kThreads * p;
        vx[p] = *reinterpret_cast<const u32x4*>(vb + (int64_t)(t0 + 64 + c / VCH) * D + (c % VCH) * 8);
      }
    }
    __syncthreads();
#pragma unroll
    for (int ks = part; ks < 4; ks += WPB) {
      const int ra = 16 * ks + 8 * hi;
      const bf16x8 va = lds_operand_tr(vt, VP, ra, ra + 4, 32 * dvb + 16 * (grp & 1), sidx);
      const bf16x8 bh8 = lds_operand_tr(khi, KP, ra, ra + 4, 16 * (grp & 1), sidx);
      const bf16x8 bl8 = lds_operand_tr(klo, KP, ra, ra + 4, 16 * (grp & 1), sidx);
      acc = mfma32(va, bh8, acc);
      acc = mfma32(va, bl8, acc);
    }
    __syncthreads();
  }

  // token-interleaved partials of one block are summed in wave order (D = 64)
  float* red = reinterpret_cast<float*>(vt);
  if (WPB > 1) {
    if (part > 0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) red[((part - 1) * NDVB + dvb) * 1024 + r * 64 + lane] = acc[r];
    }
    __syncthreads();
    if (part == 0) {
#pragma unroll
      for (int w = 1; w < WPB; ++w)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] += red[((w - 1) * NDVB + dvb) * 1024 + r * 64 + lane];
    }
  }
  float* __restrict__ cm = a.cM + (int64_t)sh * D * D;
  if (part == 0) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int dv = 32 * dvb + 8 * (r >> 2) + 4 * hi + (r & 3);
      cm[dv * D + dkb * KB + l32] = acc[r];
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) zred[krow][kch * 8 + i] = zp[i];
  __syncthreads();
  if (t < KB) {
    float sum = 0.f;
    for (int r = 0; r < 64; ++r) sum += zred[r][t];
    a.cz[(int64_t)sh * D + dkb * KB + t] = sum;
  }
}

// Exclusive prefix over segments.  One thread per element of M^T; the last
// workgroup of each head carries z.  The contributions of the next kPf segments
// are loaded while the current kPf are folded in, so the chain over segments
// runs at arithmetic speed instead of one memory latency per segment.  Each
// snapshot also gets the fp32 column sums of M over d_key (row sums of M^T),
// reduced in a fixed order (wave sums, then the waves of a row in order).
constexpr int kPf = 16;

template <int D>
__global__ __launch_bounds__(kThreads)
void lin_scan_kernel(LinScanArgs a) {
  constexpr int MB = D * D / kThreads;     // workgroups holding M^T per head
  constexpr int WPR = D / 64;              // waves per row of M^T
  static_assert(D * D % kThreads == 0 && D % 64 == 0, "shape");
  __shared__ float red[kPf][kThreads / 64];
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
  const int e = sub * kThreads + threadIdx.x;
  const int dv = e / D, dk = e % D;
  const int wave = threadIdx.x >> 6;
  const float* __restrict__ cm = a.cM + base * D * D + e;
  float run = a.M[(int64_t)bh * D * D + dk * D + dv];
  float cur[kPf], nxt[kPf];
#pragma unroll
  for (int i = 0; i < kPf; ++i) cur[i] = i < a.S ? cm[(int64_t)i * D * D] : 0.f;
  for (int s0 = 0; s0 < a.S; s0 += kPf) {
#pragma unroll
    for (int i = 0; i < kPf; ++i)
      nxt[i] = s0 + kPf + i < a.S ? cm[(int64_t)(s0 + kPf + i) * D * D] : 0.f;
#pragma unroll
    for (int i = 0; i < kPf; ++i) {
      if (s0 + i < a.S) {
        a.snapM[(base + s0 + i) * D * D + e] = f2bf(run);
        const float part = wave_sum(run);
        if ((threadIdx.x & 63) == 0) red[i][wave] = part;
        run += cur[i];
      }
    }
    __syncthreads();
    if (threadIdx.x % D == 0) {
      for (int i = 0; i < kPf && s0 + i < a.S; ++i) {
        float c = 0.f;
#pragma unroll
        for (int w = 0; w < WPR; ++w) c += red[i][wave + w];
        a.snapc[(base + s0 + i) * D + dv] = c;
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kPf; ++i) cur[i] = nxt[i];
  }
  a.M[(int64_t)bh * D * D + dk * D + dv] = run;
}

// ------------------------------------------------------------------ launchers
template <int D>
hipError_t launch_lin_contrib(const LinContribArgs& a, hipStream_t stream) {
  const int64_t blocks = (int64_t)a.B * a.H * a.S * (D / 32);
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(lin_contrib_kernel<D>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_lin_scan(const LinScanArgs& a, hipStream_t stream) {
  const int64_t blocks = (int64_t)a.BH * (D * D / kThreads + 1);
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(lin_scan_kernel<D>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template hipError_t launch_lin_contrib<64>(const LinContribArgs&, hipStream_t);
template hipError_t launch_lin_contrib<128>(const LinContribArgs&, hipStream_t);
template hipError_t launch_lin_scan<64>(const LinScanArgs&, hipStream_t);
template hipError_t launch_lin_scan<128>(const LinScanArgs&, hipStream_t);

}  // namespace infini
