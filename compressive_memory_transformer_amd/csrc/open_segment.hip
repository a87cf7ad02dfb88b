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
// Split over keys (the decode case has one query per head and up to N keys):
//   open_attn_partial: one workgroup per (128-key partition, group of 8 queries,
//     head); scores, the partition's maximum and sum, and its share of P V;
//   open_attn_combine: one workgroup per (query, head); the partitions merged in
//     a fixed order, the retrieval sigma(q) M / (sigma(q) z), the gate, the output,
//     and the query's key and value rows copied into the open-segment buffers
//     (after the partial kernel has read them, in stream order).
#include "common.h"
#include "kernels.h"

namespace infini {

namespace {

constexpr int kOpenThreads = 128;   // threads per workgroup = keys per partition
constexpr int kOpenQ = 8;           // queries per partial workgroup

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

template <typename T>
__global__ __launch_bounds__(kOpenThreads)
void open_attn_partial_kernel(OpenAttnArgs a) {
  const int part = blockIdx.x, j0 = blockIdx.y * kOpenQ, bh = blockIdx.z;
  const int t = threadIdx.x;
  const int nq = min(kOpenQ, a.m - j0);
  const int nkeys = a.pos0 + a.m;               // keys of the open segment after the append
  const T* q = static_cast<const T*>(a.q);
  const T* kseg = static_cast<const T*>(a.kseg);
  const T* vseg = static_cast<const T*>(a.vseg);
  const T* knew = static_cast<const T*>(a.knew);
  const T* vnew = static_cast<const T*>(a.vnew);
  __shared__ float qs[kOpenQ][128];
  __shared__ float ps[kOpenQ][kOpenThreads];
  __shared__ float red[2];
  for (int i = t; i < kOpenQ * a.dk; i += kOpenThreads) {
    const int jj = i / a.dk, c = i % a.dk;
    qs[jj][c] = jj < nq ? load_elem(q, ((int64_t)bh * a.q_stride + j0 + jj) * a.dk + c) : 0.f;
  }
  __syncthreads();

  // score of this thread's key for every query of the group (-inf where the
  // query may not see the key)
  const int kk = part * kOpenThreads + t;
  float s[kOpenQ];
#pragma unroll
  for (int jj = 0; jj < kOpenQ; ++jj) s[jj] = 0.f;
  if (kk < nkeys) {
    const T* krow = kk < a.pos0 ? kseg + ((int64_t)bh * a.N + kk) * a.dk
                                : knew + ((int64_t)bh * a.q_stride + kk - a.pos0) * a.dk;
    if (a.dk % 8 == 0) {
      for (int c = 0; c < a.dk; c += 8) {
        float x[8];
        load8(krow + c, x);
#pragma unroll
        for (int e = 0; e < 8; ++e)
#pragma unroll
          for (int jj = 0; jj < kOpenQ; ++jj) s[jj] = __builtin_fmaf(qs[jj][c + e], x[e], s[jj]);
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
    const bool vis = jj < nq && kk < nkeys && kk <= a.pos0 + j0 + jj;
    const float sc = vis ? s[jj] * a.scale : -__builtin_inff();
    mx[jj] = wg_max(sc, red);
    const float p = (mx[jj] == -__builtin_inff() || !vis) ? 0.f : exp_e(sc - mx[jj]);
    l[jj] = wg_sum(p, red);
    ps[jj][t] = p;
  }
  __syncthreads();

  // this partition's share of P V: thread t holds column t of d_value
  if (t < a.dv) {
    float o[kOpenQ];
#pragma unroll
    for (int jj = 0; jj < kOpenQ; ++jj) o[jj] = 0.f;
    const int k0 = part * kOpenThreads;
    const int kend = min(kOpenThreads, nkeys - k0);
    for (int i = 0; i < kend; ++i) {
      const int key = k0 + i;
      const float x = key < a.pos0 ? load_elem(vseg, ((int64_t)bh * a.N + key) * a.dv + t)
                                   : load_elem(vnew, ((int64_t)bh * a.q_stride + key - a.pos0) * a.dv + t);
#pragma unroll
      for (int jj = 0; jj < kOpenQ; ++jj) o[jj] = __builtin_fmaf(ps[jj][i], x, o[jj]);
    }
#pragma unroll
    for (int jj = 0; jj < kOpenQ; ++jj) {
      if (jj < nq) {
        float* dst = a.part + (((int64_t)bh * a.m + j0 + jj) * a.P + part) * (a.dv + 2);
        dst[t] = o[jj];
        if (t == 0) {
          dst[a.dv] = mx[jj];
          dst[a.dv + 1] = l[jj];
        }
      }
    }
  }
}

template <typename T>
__global__ __launch_bounds__(kOpenThreads)
void open_attn_combine_kernel(OpenAttnArgs a) {
  const int j = blockIdx.x, bh = blockIdx.y, h = bh % a.H;
  const int t = threadIdx.x;
  const T* q = static_cast<const T*>(a.q);
  __shared__ float sq[128];
  __shared__ float red[2];
  const float* parts = a.part + ((int64_t)bh * a.m + j) * a.P * (a.dv + 2);

  // A_dot: the partitions merged against the overall maximum, in partition order
  float mx = -__builtin_inff();
  for (int p = 0; p < a.P; ++p) mx = fmaxf(mx, parts[(int64_t)p * (a.dv + 2) + a.dv]);
  float l = 0.f, o = 0.f;
  for (int p = 0; p < a.P; ++p) {
    const float* src = parts + (int64_t)p * (a.dv + 2);
    const float mp = src[a.dv];
    if (mp == -__builtin_inff()) continue;
    const float w = exp_e(mp - mx);
    l = __builtin_fmaf(w, src[a.dv + 1], l);
    if (t < a.dv) o = __builtin_fmaf(w, src[t], o);
  }
  const float a_dot = o / l;   // l > 0: every query sees at least its own key

  // A_mem = sigma(q) M / (sigma(q) z), 0 for a stream's first segment
  const int64_t qrow = ((int64_t)bh * a.q_stride + j);
  if (t < a.dk) {
    const float x = load_elem(q, qrow * a.dk + t);
    sq[t] = x > 0.f ? x + 1.f : exp_e(x);
  }
  __syncthreads();
  const float den = wg_sum(t < a.dk ? sq[t] * a.z[(int64_t)bh * a.dk + t] : 0.f, red);
  float a_mem = 0.f;
  if (a.has_memory && den > 0.f && t < a.dv) {
    const float* Mh = a.M + (int64_t)bh * a.dk * a.dv + t;
    float num = 0.f;
    for (int c = 0; c < a.dk; ++c) num = __builtin_fmaf(sq[c], Mh[(int64_t)c * a.dv], num);
    a_mem = num / den;
  }
  if (t < a.dv) {
    const float g = sigmoid_gate(a.beta[h]);
    store_elem(static_cast<T*>(a.out), qrow * a.dv + t, g * a_mem + (1.f - g) * a_dot);
  }
  // the new token's key and value join the open segment
  const int64_t orow = (int64_t)bh * a.N + a.pos0 + j;
  if (t < a.dk) static_cast<T*>(a.kseg_out)[orow * a.dk + t] = static_cast<const T*>(a.knew)[qrow * a.dk + t];
  if (t < a.dv) static_cast<T*>(a.vseg_out)[orow * a.dv + t] = static_cast<const T*>(a.vnew)[qrow * a.dv + t];
}

int open_attn_parts(int keys) { return (keys + kOpenThreads - 1) / kOpenThreads; }

hipError_t launch_open_attn(const OpenAttnArgs& args, hipStream_t stream) {
  OpenAttnArgs a = args;
  if (a.m <= 0) return hipSuccess;
  if (a.dk > 128 || a.dv > 128 || a.pos0 + a.m > a.N) return hipErrorInvalidValue;
  a.P = open_attn_parts(a.pos0 + a.m);
  const dim3 gp((unsigned)a.P, (unsigned)((a.m + kOpenQ - 1) / kOpenQ), (unsigned)a.BH);
  const dim3 gc((unsigned)a.m, (unsigned)a.BH);
  if (a.bf16) {
    hipLaunchKernelGGL(open_attn_partial_kernel<bf16>, gp, dim3(kOpenThreads), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(open_attn_combine_kernel<bf16>, gc, dim3(kOpenThreads), 0, stream, a);
  } else {
    hipLaunchKernelGGL(open_attn_partial_kernel<float>, gp, dim3(kOpenThreads), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(open_attn_combine_kernel<float>, gc, dim3(kOpenThreads), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace infini
