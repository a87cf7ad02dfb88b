// Compressive-memory state kernels of the bf16 path (page "精读笔记：Infini-attention",
// section 3.4; delta fraction as written in section 2.1 of the CSDN page).
//
//   linear: M_s = M_{s-1} + sigma(K)^T V, z_s = z_{s-1} + sum_t sigma(K_t)
//   delta : M_s = M_{s-1} + sigma(K)^T (V - sigma(K) M_{s-1} / (sigma(K) z_{s-1}))
//
// Both leave a snapshot of (M_{s-1}^T in bf16, z_{s-1} in fp32) per segment for
// the fused attention kernel and the final (M_S, z_S) in the fp32 state.
//
// Precision.  sigma(K) = 1 + k for the small keys of these workloads, so rounding
// sigma(K) to bf16 keeps only a few bits of k.  Every GEMM whose result is
// accumulated into M therefore splits its fp32 operands into bf16 hi + lo parts
// (x = hi + lo to about 16 bits) and sums the hi*hi, hi*lo and lo*hi products in
// fp32: sigma(K) in the linear contributions (V is exact in bf16), sigma(K) and
// the residual U = V - R in the delta update.  The delta read-back R and the
// retrieval use single bf16 operands, whose error does not accumulate.
#include "common.h"
#include "kernels.h"

namespace infini {

namespace {
constexpr int kThreads = 256;

__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

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
// workgroup of each head carries z.  Each snapshot also gets the fp32 column sums
// of M over d_key (row sums of M^T), reduced in a fixed order.
template <int D>
__global__ __launch_bounds__(kThreads)
void lin_scan_kernel(LinScanArgs a) {
  constexpr int MB = D * D / kThreads;     // workgroups holding M^T per head
  constexpr int WPR = D / 64;              // waves per row of M^T
  static_assert(D * D % kThreads == 0 && D % 64 == 0, "shape");
  __shared__ float red[2][kThreads / 64];
  const int bh = blockIdx.x / (MB + 1);
  const int sub = blockIdx.x % (MB + 1);
  const int64_t base = (int64_t)bh * a.S;
  if (sub == MB) {
    const int dk = threadIdx.x;
    if (dk >= D) return;
    float run = a.z[(int64_t)bh * D + dk];
    for (int s = 0; s < a.S; ++s) {
      a.snapz[(base + s) * D + dk] = run;
      run += a.cz[(base + s) * D + dk];
    }
    a.z[(int64_t)bh * D + dk] = run;
    return;
  }
  const int e = sub * kThreads + threadIdx.x;
  const int dv = e / D, dk = e % D;
  const int wave = threadIdx.x >> 6;
  float run = a.M[(int64_t)bh * D * D + dk * D + dv];
  for (int s = 0; s < a.S; ++s) {
    const int64_t sh = base + s;
    a.snapM[sh * D * D + e] = f2bf(run);
    const float part = wave_sum(run);
    if ((threadIdx.x & 63) == 0) red[s & 1][wave] = part;
    __syncthreads();
    if (threadIdx.x % D == 0) {
      float c = 0.f;
#pragma unroll
      for (int w = 0; w < WPR; ++w) c += red[s & 1][wave + w];
      a.snapc[sh * D + dv] = c;
    }
    run += a.cM[sh * D * D + e];
  }
  a.M[(int64_t)bh * D * D + dk * D + dv] = run;
}

// ==================================================================== delta
// One workgroup per (b, h, 16-column block of M); the chain over segments runs
// inside the kernel with the fp32 block of M^T and z resident in LDS.  The
// columns of M are independent under the delta rule (column j of the read-back
// needs only column j of M; z is shared and depends on K alone), so the blocks
// of a head never communicate.  Each of the 4 waves takes every 4th 32-token
// sub-tile of the segment; the per-wave partial updates are summed in a fixed
// order at the end of the segment (deterministic).
template <int D>
__global__ __launch_bounds__(kThreads)
void delta_chain_kernel(DeltaArgs a) {
  constexpr int CB = 16;              // columns per workgroup
  constexpr int NCB = D / CB;
  constexpr int P = D + 16;           // staging pitch (elements)
  constexpr int STAGE = 32 * P;       // one 32-token sigma(K) tile
  __shared__ float mt[CB][D];         // M^T block (row = column of M), fp32
  __shared__ float zs[D];
  __shared__ float zred[4][D];
  __shared__ float csum[CB];          // column sums of the M block over d_key (fp32)
  __shared__ __attribute__((aligned(16))) bf16 stage[4][2][STAGE];  // per wave: hi, lo

  const int blk = xcd_logical_block(blockIdx.x, gridDim.x);
  const int bh = blk / NCB, cb = blk % NCB;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int grp = lane >> 4, sidx = lane & 15;

  float* __restrict__ Mg = a.M + (int64_t)bh * D * D;
  float* __restrict__ zg = a.z + (int64_t)bh * D;
  for (int i = t; i < CB * D; i += kThreads) {
    const int j = i / D, dk = i % D;
    mt[j][dk] = Mg[dk * D + cb * CB + j];
  }
  for (int i = t; i < D; i += kThreads) zs[i] = zg[i];
  __syncthreads();

  bf16* khs = stage[wave][0];
  bf16* kls = stage[wave][1];
  float* red = reinterpret_cast<float*>(&stage[0][0][0]);  // [4][CB][D] after the token loop
  static_assert(4 * CB * D * sizeof(float) <= sizeof(stage), "reduction buffer too small");

  for (int s = 0; s < a.S; ++s) {
    const int64_t sh = (int64_t)bh * a.S + s;
    const bool has_memory = (a.seg_base + s) > 0;
    // ---- snapshot of M_{s-1}^T (this block's rows) and z_{s-1}
    for (int i = t; i < CB * D / 8; i += kThreads) {
      const int j = i / (D / 8), c8 = (i % (D / 8)) * 8;
      bf16x8 w8;
#pragma unroll
      for (int e = 0; e < 8; ++e) w8[e] = f2bf(mt[j][c8 + e]);
      *reinterpret_cast<bf16x8*>(a.snapM + sh * D * D + (int64_t)(cb * CB + j) * D + c8) = w8;
    }
    if (cb == 0)
      for (int i = t; i < D; i += kThreads) a.snapz[sh * D + i] = zs[i];
    {
      // column sums: 16 threads per column, fixed-order reduction
      const int j = t >> 4, q16 = t & 15;
      float part = 0.f;
      for (int i = q16; i < D; i += 16) part += mt[j][i];
      part += __shfl_xor(part, 1);
      part += __shfl_xor(part, 2);
      part += __shfl_xor(part, 4);
      part += __shfl_xor(part, 8);
      if (q16 == 0) {
        csum[j] = part;
        a.snapc[sh * D + cb * CB + j] = part;
      }
    }
    __syncthreads();

    // ---- B operand of the read-back: M[dk][col] = mt[col][dk], bf16
    bf16x8 mop[D / 32];
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
#pragma unroll
      for (int i = 0; i < 8; ++i) mop[c][i] = f2bf(mt[sidx][32 * c + 8 * grp + i]);

    f32x4 acc[D / 16];
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[nb][r] = 0.f;
    float zacc[D / 32][8];
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
#pragma unroll
      for (int i = 0; i < 8; ++i) zacc[c][i] = 0.f;

    const int64_t tok0 = (int64_t)bh * a.L + (int64_t)s * a.N;
    const bf16* __restrict__ kb = a.k + tok0 * D;
    const bf16* __restrict__ vb = a.v + tok0 * D + cb * CB;

    for (int st = wave; st < a.N / 32; st += 4) {
      bf16 uh[2][4], ul[2][4];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int trow = 32 * st + 16 * h2 + sidx;  // token whose key this lane loads
        float den = 0.f;
        bf16x8 kop[D / 32];
#pragma unroll
        for (int c = 0; c < D / 32; ++c) {
          const bf16x8 kx = *reinterpret_cast<const bf16x8*>(kb + (int64_t)trow * D + 32 * c + 8 * grp);
          bf16x8 h8, l8;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float x = bf2f(kx[i]);
            const float kp = x > 0.f ? x : exp_e(x) - 1.f;   // k' = sigma(k) - 1
            const float f = kp + 1.f;
            zacc[c][i] += f;
            den = __builtin_fmaf(f, zs[32 * c + 8 * grp + i], den);
            h8[i] = f2bf(f);
            l8[i] = lo_part(f, h8[i]);
            kop[c][i] = f2bf(kp);
          }
          *(INFINI_LDS bf16x8*)(khs + (16 * h2 + sidx) * P + 32 * c + 8 * grp) = h8;
          *(INFINI_LDS bf16x8*)(kls + (16 * h2 + sidx) * P + 32 * c + 8 * grp) = l8;
        }
        den += __shfl_xor(den, 16);
        den += __shfl_xor(den, 32);
        // R = sigma(K) M_{s-1} = colsum(M) + K' M: lane holds (K' M)[token 4*grp + r][col sidx]
        f32x4 r4 = {0.f, 0.f, 0.f, 0.f};
        if (has_memory) {
#pragma unroll
          for (int c = 0; c < D / 32; ++c) r4 = mfma16(kop[c], mop[c], r4);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int tl = 4 * grp + r;                     // token within the 16-row half
          const float den_t = __shfl(den, tl);
          const float vv = bf2f(vb[(int64_t)(32 * st + 16 * h2 + tl) * D + sidx]);
          const float u = (has_memory && den_t > 0.f) ? vv - (csum[sidx] + r4[r]) / den_t : vv;
          uh[h2][r] = f2bf(u);
          ul[h2][r] = lo_part(u, uh[h2][r]);
        }
      }
      wave_lds_fence();
      // ---- M^T[col][dk] += U^T sigma(K) over the 32 tokens (hi*hi + lo*hi + hi*lo)
      bf16x8 ua, ub;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        ua[r] = uh[0][r];
        ua[4 + r] = uh[1][r];
        ub[r] = ul[0][r];
        ub[4 + r] = ul[1][r];
      }
#pragma unroll
      for (int nb = 0; nb < D / 16; ++nb) {
        const bf16x8 kh = lds_operand_tr(khs, P, 4 * grp, 16 + 4 * grp, 16 * nb, sidx);
        const bf16x8 kl = lds_operand_tr(kls, P, 4 * grp, 16 + 4 * grp, 16 * nb, sidx);
        acc[nb] = mfma16(ua, kh, acc[nb]);
        acc[nb] = mfma16(ub, kh, acc[nb]);
        acc[nb] = mfma16(ua, kl, acc[nb]);
      }
      wave_lds_fence();
    }
    // ---- z partial of this wave: reduce over the 16 lanes of each group
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float x = zacc[c][i];
        x += __shfl_xor(x, 1);
        x += __shfl_xor(x, 2);
        x += __shfl_xor(x, 4);
        x += __shfl_xor(x, 8);
        zacc[c][i] = x;
      }
    __syncthreads();  // every wave is done with its staging tiles
    if (sidx == 0) {
#pragma unroll
      for (int c = 0; c < D / 32; ++c)
#pragma unroll
        for (int i = 0; i < 8; ++i) zred[wave][32 * c + 8 * grp + i] = zacc[c][i];
    }
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[(wave * CB + 4 * grp + r) * D + 16 * nb + sidx] = acc[nb][r];
    __syncthreads();
    for (int i = t; i < CB * D; i += kThreads) {
      const int j = i / D, dk = i % D;
      mt[j][dk] += ((red[(0 * CB + j) * D + dk] + red[(1 * CB + j) * D + dk]) +
                    red[(2 * CB + j) * D + dk]) + red[(3 * CB + j) * D + dk];
    }
    for (int i = t; i < D; i += kThreads) zs[i] += ((zred[0][i] + zred[1][i]) + zred[2][i]) + zred[3][i];
    __syncthreads();
  }

  for (int i = t; i < CB * D; i += kThreads) {
    const int j = i / D, dk = i % D;
    Mg[dk * D + cb * CB + j] = mt[j][dk];
  }
  if (cb == 0)
    for (int i = t; i < D; i += kThreads) zg[i] = zs[i];
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

template <int D>
hipError_t launch_delta_chain(const DeltaArgs& a, hipStream_t stream) {
  const int64_t blocks = (int64_t)a.BH * (D / 16);
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(delta_chain_kernel<D>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template hipError_t launch_lin_contrib<64>(const LinContribArgs&, hipStream_t);
template hipError_t launch_lin_contrib<128>(const LinContribArgs&, hipStream_t);
template hipError_t launch_lin_scan<64>(const LinScanArgs&, hipStream_t);
template hipError_t launch_lin_scan<128>(const LinScanArgs&, hipStream_t);
template hipError_t launch_delta_chain<64>(const DeltaArgs&, hipStream_t);
template hipError_t launch_delta_chain<128>(const DeltaArgs&, hipStream_t);

}  // namespace infini
