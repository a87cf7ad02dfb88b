// Device-side helpers shared by the gfx950 kernels of the Infini-attention library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace infini {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

#define INFINI_LDS __attribute__((address_space(3)))

// ---------------------------------------------------------------- MFMA
// v_mfma_f32_32x32x16_bf16.  Operand layouts (checked on gfx950 hardware):
//   A (32 x 16): lane l holds A[l % 32][8 * (l / 32) + j], j = 0..7
//   B (16 x 32): lane l holds B[8 * (l / 32) + j][l % 32]
//   C (32 x 32): lane l holds C[8 * (r / 4) + 4 * (l / 32) + r % 4][l % 32], r = 0..15
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// v_mfma_f32_16x16x32_bf16:
//   A (16 x 32): lane l holds A[l % 16][8 * (l / 16) + j]
//   B (32 x 16): lane l holds B[8 * (l / 16) + j][l % 16]
//   C (16 x 16): lane l holds C[4 * (l / 16) + r][l % 16], r = 0..3
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------- LDS transpose read
// ds_read_b64_tr_b16 (gfx950): within each group of 16 lanes, output lane i,
// element e receives element (i % 4) of the 8-byte row read by lane 4 * e + i / 4
// of the same group.  If lane 4a + b of a group reads X[row0 + a][col0 + 4b ..],
// lane i receives X[row0 + e][col0 + i] for e = 0..3: four consecutive rows of one
// column, i.e. a row-major tile read as its transpose.
__device__ __forceinline__ s16x4 lds_read_tr16(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((INFINI_LDS s16x4*)(p));
}

// An 8-element MFMA operand for a contraction over the ROWS of a row-major
// bf16 tile X (pitch in elements) held in LDS.  Lane l (group g = (l % 64) / 16,
// s = l % 16) receives X[rowA + e][col0 + i] in elements e = 0..3 and
// X[rowB + e][col0 + i] in elements 4..7, where i = s and col0 already includes
// 16 * (g & 1).  rowA/rowB are the first rows of the two 4-row groups this lane's
// group reads.
__device__ __forceinline__ bf16x8 lds_operand_tr(const bf16* tile, int pitch, int rowA, int rowB,
                                                 int col0, int s) {
  const int r = s >> 2, c = (s & 3) * 4;
  s16x4 x = lds_read_tr16(tile + (rowA + r) * pitch + col0 + c);
  s16x4 y = lds_read_tr16(tile + (rowB + r) * pitch + col0 + c);
  s16x8 xy = __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, xy);
}

__device__ __forceinline__ bf16x8 lds_read8(const bf16* p) {
  return *(const INFINI_LDS bf16x8*)(p);
}

// -------------------------------------------------------------- elementwise
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// e^x as 2^(x log2 e) on the hardware exp2 unit.
__device__ __forceinline__ float exp_e(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

__device__ __forceinline__ float bf2f(bf16 x) { return (float)x; }
// A bf16 held as the raw 16 bits of a short (e.g. an element of a transposing
// LDS read) widened to fp32 by placing the bits in the upper half.  (A
// __builtin_bit_cast of a vector element to __bf16 has compiled to the wrong
// element here.)
__device__ __forceinline__ float bf16_bits_to_f32(short b) {
  return __builtin_bit_cast(float, (unsigned)(unsigned short)b << 16);
}
__device__ __forceinline__ bf16 f2bf(float x) { return (bf16)x; }  // round to nearest even

// sigmoid(beta) with exact limits: beta = +inf -> 1, beta = -inf -> 0.
__device__ __forceinline__ float sigmoid_gate(float beta) { return 1.f / (1.f + exp_e(-beta)); }

// ------------------------------------------------------------ block mapping
// Consecutive workgroup ids are dealt round-robin to the 8 XCDs of the chip.
// This maps the hardware id to a logical id so that each XCD receives one
// contiguous range of logical ids (which share data through that XCD's L2).
__device__ __forceinline__ int xcd_logical_block(int hw, int nblocks) {
  constexpr int kXcd = 8;
  if (nblocks % kXcd != 0) return hw;
  return (hw % kXcd) * (nblocks / kXcd) + hw / kXcd;
}

// Workgroup barrier that orders LDS accesses only: the fences are restricted to
// the LDS address space, so the barrier waits for this wave's LDS operations
// (lgkmcnt) but not for its global loads in flight (register prefetches).
__device__ __forceinline__ void lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

}  // namespace infini
