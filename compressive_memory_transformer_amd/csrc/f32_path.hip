// The VALU path: plain kernels, one segment per launch, for any widths d_key,
// d_value up to 128 and any segment length up to 4096.  It serves every fp32
// state, and bf16 states whose shapes the MFMA kernels do not take (d_key !=
// d_value, widths other than 64 and 128, segment lengths that are not a
// multiple of 64).  Same equations as the MFMA path (page "精读笔记：
// Infini-attention", sections 3.1, 3.3, 3.4, 3.5); q, k, v and the output in the
// state's dtype (T = float or bf16), all arithmetic in fp32.
#include "common.h"
#include "kernels.h"

namespace infini {

namespace {
constexpr int kThreads = 256;
constexpr int kRows = 4;          // query rows per workgroup
constexpr int kMaxN = 4096;       // scores of kRows rows kept in LDS
constexpr int kMaxD = 128;
__device__ __forceinline__ float ld(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ld(const bf16* p, int64_t i) { return bf2f(p[i]); }
__device__ __forceinline__ void st(float* p, int64_t i, float x) { p[i] = x; }
__device__ __forceinline__ void st(bf16* p, int64_t i, float x) { p[i] = f2bf(x); }
}  // namespace

// One workgroup per (head, block of kRows query rows).  Scores for the block are
// materialised in LDS (masked softmax over keys j <= i of this segment), then
// A_dot, A_mem and the gate are formed with one thread per output element.
template <typename T>
__global__ __launch_bounds__(kThreads)
void f32_attn_kernel(F32AttnArgs a) {
  __shared__ float sc[kRows][kMaxN];
  __shared__ float qs[kRows][kMaxD];
  __shared__ float rowstat[kRows][2];
  const int nrb = (a.N + kRows - 1) / kRows;
  const int bh = blockIdx.x / nrb;
  const int r0 = (blockIdx.x % nrb) * kRows;
  const int h = bh % a.H;
  const int t = threadIdx.x;
  const int64_t row0 = (int64_t)bh * a.L + a.seg_off;
  const T* __restrict__ q = static_cast<const T*>(a.q) + row0 * a.dk;
  const T* __restrict__ k = static_cast<const T*>(a.k) + row0 * a.dk;
  const T* __restrict__ v = static_cast<const T*>(a.v) + row0 * a.dv;
  T* __restrict__ o = static_cast<T*>(a.out) + row0 * a.dv;
  const int nr = min(kRows, a.N - r0);

  for (int i = t; i < kRows * a.dk; i += kThreads) {
    const int r = i / a.dk, c = i % a.dk;
    qs[r][c] = r < nr ? ld(q, (int64_t)(r0 + r) * a.dk + c) : 0.f;
  }
  __syncthreads();
  const int nkeys = r0 + nr;  // keys 0 .. r0+nr-1 may be needed
  for (int i = t; i < nr * nkeys; i += kThreads) {
    const int r = i / nkeys, j = i % nkeys;
    float s = -__builtin_inff();
    if (j <= r0 + r) {
      float d = 0.f;
      for (int c = 0; c < a.dk; ++c) d = __builtin_fmaf(qs[r][c], ld(k, (int64_t)j * a.dk + c), d);
      s = d * a.scale;
    }
    sc[r][j] = s;
  }
  __syncthreads();
  const int wave = t >> 6, lane = t & 63;
  if (wave < nr) {
    float mx = -__builtin_inff();
    for (int j = lane; j < nkeys; j += 64) mx = fmaxf(mx, sc[wave][j]);
    mx = wave_max(mx);
    float sum = 0.f;
    for (int j = lane; j < nkeys; j += 64) {
      const float p = expf(sc[wave][j] - mx);
      sc[wave][j] = p;
      sum += p;
    }
    sum = wave_sum(sum);
    if (lane == 0) rowstat[wave][0] = sum;
    if (a.has_memory) {
      // denominator sigma(q) . z_{s-1}
      float den = 0.f;
      for (int c = lane; c < a.dk; c += 64) {
        const float x = qs[wave][c];
        den += (x > 0.f ? x + 1.f : expf(x)) * a.z[(int64_t)bh * a.dk + c];
      }
      den = wave_sum(den);
      if (lane == 0) rowstat[wave][1] = den;
    }
  }
  __syncthreads();
  const float beta = a.beta[h];
  const float g = 1.f / (1.f + expf(-beta));
  const float* __restrict__ M = a.M + (int64_t)bh * a.dk * a.dv;
  for (int i = t; i < nr * a.dv; i += kThreads) {
    const int r = i / a.dv, c = i % a.dv;
    float acc = 0.f;
    for (int j = 0; j <= r0 + r; ++j) acc = __builtin_fmaf(sc[r][j], ld(v, (int64_t)j * a.dv + c), acc);
    const float a_dot = acc / rowstat[r][0];
    float a_mem = 0.f;
    if (a.has_memory) {
      float num = 0.f;
      for (int kk = 0; kk < a.dk; ++kk) {
        const float x = qs[r][kk];
        num = __builtin_fmaf(x > 0.f ? x + 1.f : expf(x), M[(int64_t)kk * a.dv + c], num);
      }
      const float den = rowstat[r][1];
      a_mem = den > 0.f ? num / den : 0.f;
    }
    st(o, (int64_t)(r0 + r) * a.dv + c, g * a_mem + (1.f - g) * a_dot);
  }
}

// Delta rule, step 1: U = V - sigma(K) M_{s-1} / (sigma(K) z_{s-1}), one thread per
// (token, column); the denominator is recomputed per thread (small widths only).
template <typename T>
__global__ __launch_bounds__(kThreads)
void f32_residual_kernel(F32UpdateArgs a) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t per_head = (int64_t)a.N * a.dv;
  if (i >= (int64_t)a.BH * per_head) return;
  const int bh = (int)(i / per_head);
  const int tt = (int)((i % per_head) / a.dv), c = (int)(i % a.dv);
  const int64_t row = (int64_t)bh * a.L + a.seg_off + tt;
  const T* __restrict__ kr = static_cast<const T*>(a.k) + row * a.dk;
  const float vv = ld(static_cast<const T*>(a.v), row * a.dv + c);
  float u = vv;
  if (a.has_memory) {
    const float* __restrict__ M = a.M + (int64_t)bh * a.dk * a.dv;
    const float* __restrict__ z = a.z + (int64_t)bh * a.dk;
    float num = 0.f, den = 0.f;
    for (int kk = 0; kk < a.dk; ++kk) {
      const float x = ld(kr, kk);
      const float f = x > 0.f ? x + 1.f : expf(x);
      num = __builtin_fmaf(f, M[(int64_t)kk * a.dv + c], num);
      den = __builtin_fmaf(f, z[kk], den);
    }
    if (den > 0.f) u = vv - num / den;
  }
  a.U[(int64_t)bh * per_head + (int64_t)tt * a.dv + c] = u;
}

// Step 2 (both rules): M[i][c] += sum_t sigma(K[t][i]) W[t][c] with W = V (linear)
// or U (delta); one thread per element of M.
template <typename T>
__global__ __launch_bounds__(kThreads)
void f32_bind_kernel(F32UpdateArgs a) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t per_head = (int64_t)a.dk * a.dv;
  if (i >= (int64_t)a.BH * per_head) return;
  const int bh = (int)(i / per_head);
  const int r = (int)((i % per_head) / a.dv), c = (int)(i % a.dv);
  const int64_t row0 = (int64_t)bh * a.L + a.seg_off;
  float acc = 0.f;
  for (int tt = 0; tt < a.N; ++tt) {
    const float x = ld(static_cast<const T*>(a.k), (row0 + tt) * a.dk + r);
    const float f = x > 0.f ? x + 1.f : expf(x);
    const float w = a.delta ? a.U[(int64_t)bh * a.N * a.dv + (int64_t)tt * a.dv + c]
                            : ld(static_cast<const T*>(a.v), (row0 + tt) * a.dv + c);
    acc = __builtin_fmaf(f, w, acc);
  }
  a.M[(int64_t)bh * per_head + (int64_t)r * a.dv + c] += acc;
}

// Step 3: z[i] += sum_t sigma(K[t][i]); after step 2 so that the delta read-back
// above used z_{s-1}.
template <typename T>
__global__ __launch_bounds__(kThreads)
void f32_znorm_kernel(F32UpdateArgs a) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= (int64_t)a.BH * a.dk) return;
  const int bh = (int)(i / a.dk), r = (int)(i % a.dk);
  const int64_t row0 = (int64_t)bh * a.L + a.seg_off;
  float acc = 0.f;
  for (int tt = 0; tt < a.N; ++tt) {
    const float x = ld(static_cast<const T*>(a.k), (row0 + tt) * a.dk + r);
    acc += x > 0.f ? x + 1.f : expf(x);
  }
  a.z[i] += acc;
}

// Zeroes p[0, n) and p2[0, n2) (two ranges in one launch).
__global__ void fill_zero_kernel(float* p, int64_t n, float* p2, int64_t n2) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n + n2; i += (int64_t)gridDim.x * blockDim.x) {
    if (i < n) p[i] = 0.f;
    else p2[i - n] = 0.f;
  }
}

hipError_t launch_f32_attn(const F32AttnArgs& a, hipStream_t stream) {
  if (a.N > kMaxN || a.dk > kMaxD || a.dv > kMaxD) return hipErrorInvalidValue;
  const int64_t blocks = (int64_t)a.BH * ((a.N + kRows - 1) / kRows);
  if (blocks <= 0) return hipSuccess;
  if (a.bf16) hipLaunchKernelGGL(f32_attn_kernel<bf16>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
  else hipLaunchKernelGGL(f32_attn_kernel<float>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <typename T>
static hipError_t f32_update(const F32UpdateArgs& a, hipStream_t stream) {
  auto grid = [](int64_t n) { return dim3((unsigned)((n + kThreads - 1) / kThreads)); };
  if (a.delta) {
    const int64_t n = (int64_t)a.BH * a.N * a.dv;
    hipLaunchKernelGGL(f32_residual_kernel<T>, grid(n), dim3(kThreads), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(f32_bind_kernel<T>, grid((int64_t)a.BH * a.dk * a.dv), dim3(kThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(f32_znorm_kernel<T>, grid((int64_t)a.BH * a.dk), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_f32_update(const F32UpdateArgs& a, hipStream_t stream) {
  return a.bf16 ? f32_update<bf16>(a, stream) : f32_update<float>(a, stream);
}

hipError_t launch_fill_zero(float* p, int64_t n, float* p2, int64_t n2, hipStream_t stream) {
  if (n < 0 || n2 < 0) return hipErrorInvalidValue;
  if (n + n2 == 0) return hipSuccess;
  const int64_t want = (n + n2 + kThreads - 1) / kThreads;
  const unsigned blocks = (unsigned)(want < 4096 ? want : 4096);
  hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks), dim3(kThreads), 0, stream, p, n, p2, n2);
  return hipGetLastError();
}

}  // namespace infini
