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
// K and V tiles stream from HBM straight into LDS (global_load_lds, 16 bytes per
// lane, double-buffered, no staging registers) in an XOR-swizzled layout whose
// reads are free of bank conflicts.  The softmax keeps a reference maximum per
// query and rescales the accumulator only when a new score exceeds it by more
// than 2^8 (exact: the final division uses the same reference maximum).
//
// Epilogue: with sigma(q) = 1 + q', q' = sigma(q) - 1,
//   sigma(q) M = colsum(M) + q' M   and   sigma(q) z = sum(z) + q' z,
// where colsum(M) (sum over d_key) comes in fp32 with the snapshot and q' M runs
// on MFMA from the bf16 snapshot of M_{s-1}^T.  q' keeps the full relative
// precision of bf16, unlike sigma(q) ~ 1 + q itself.  Gate, round to bf16, store.
#include "common.h"
#include "kernels.h"

namespace infini {

namespace {

constexpr int kBM = 128;   // query rows per tile (4 waves x 32)
constexpr int kBN = 64;    // keys per LDS tile
constexpr int kThreads = 256;
constexpr float kRescaleSlack = 8.f;  // log2 units

template <int D>
struct FaLayout {
  static constexpr int CHUNKS = D / 8;                 // 16-byte chunks per row
  static constexpr int TILE_ELEMS = kBN * D;           // one K or V tile, unpadded
  static constexpr int ROWS_PER_INSTR = 64 * 8 / D;    // rows one wave-wide 16-byte load covers
  static constexpr int INSTR_PER_WAVE = kBN / ROWS_PER_INSTR / 4;   // per 64-row tile
  static_assert(D <= 2 * kBN, "the snapshot of M^T must fit the two K buffers");
};

// Physical 16-byte chunk of logical chunk c in row r.  K rows are read 16 bytes
// at a time by 8 consecutive rows per LDS phase: XOR with r % 8.  V rows are
// read by ds_read_b64_tr_b16 as 32-byte pieces of 4 consecutive rows: XOR with an
// even offset keeps each piece contiguous and spreads the 4 rows over the banks.
template <int D>
__device__ __forceinline__ int k_chunk(int r, int c) { return c ^ (r & 7); }
template <int D>
__device__ __forceinline__ int v_chunk(int r, int c) { return c ^ ((r & (FaLayout<D>::CHUNKS / 2 - 1)) << 1); }

// Issue this wave's share of the direct-to-LDS loads of a row-major [rows x D]
// tile: wave-wide instruction `ins` fills bytes [1024 ins, 1024 ins + 1024) of the
// LDS tile, lane l landing at 16 l (row ROWS_PER_INSTR * ins + l / CHUNKS).  The
// global address is a uniform base plus a 32-bit per-lane element offset.
template <int D, bool IS_V>
__device__ __forceinline__ int tile_lane_offset(int ins, int lane) {
  using L = FaLayout<D>;
  const int row = ins * L::ROWS_PER_INSTR + lane / L::CHUNKS;
  const int phys = lane % L::CHUNKS;
  const int logical = IS_V ? v_chunk<D>(row, phys) : k_chunk<D>(row, phys);
  return row * D + logical * 8;
}

// Buffer resource over `bytes` bytes at `base` (raw buffer, no stride); reads past
// the end return zeros instead of faulting.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Per-lane byte offsets of this wave's NI load instructions for one tile.
template <int D, bool IS_V, int NI>
__device__ __forceinline__ void tile_offsets(int (&off)[NI], int wave, int lane) {
#pragma unroll
  for (int j = 0; j < NI; ++j) off[j] = 2 * tile_lane_offset<D, IS_V>(wave * NI + j, lane);
}

// buffer_load_dwordx4 ... lds: uniform descriptor + 32-bit per-lane offset; the
// tile's position in the buffer goes into the scalar offset.
template <int NI>
__device__ __forceinline__ void issue_tile(const bf16* base, uint32_t bytes, const int* off, int soff_bytes,
                                           bf16* lds_tile, int wave) {
  const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(base, bytes);
#pragma unroll
  for (int j = 0; j < NI; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (INFINI_LDS void*)(lds_tile + (wave * NI + j) * 512), 16,
                                             off[j], soff_bytes, 0, 0);
}

__device__ __forceinline__ void wait_loads_and_sync() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's LDS-bound loads have landed
  __syncthreads();
}

}  // namespace

// Per-wave running state of one 32-row query block.
template <int D>
struct RowState {
  bf16x8 qreg[D / 16];   // Q^T as the B operand: lane holds Q[row][16c + 8hi .. +7]
  f32x16 o[D / 32];      // O^T accumulator: lane holds O[row][32db + 8(r/4) + 4hi + r%4]
  float m_run;           // reference maximum of the row (log2 domain)
  float l_run;           // this lane's share of the softmax denominator
};

// One 64-key tile: optionally start the DMA of the next tile into the other pair
// of buffers, then S^T, mask, softmax and O^T update for the keys of this tile
// that the wave's rows can see.  The current and next buffers are distinct
// objects, so the compiler never waits on the DMA before reading this tile.
template <int D>
__device__ __forceinline__ void attend_tile(RowState<D>& st, const bf16* __restrict__ kt_lds,
                                            const bf16* __restrict__ vt_lds, bf16* __restrict__ k_next,
                                            bf16* __restrict__ v_next, bool prefetch,
                                            const bf16* kseg, const bf16* vseg, uint32_t seg_bytes,
                                            const int (&koff)[FaLayout<D>::INSTR_PER_WAVE],
                                            const int (&voff)[FaLayout<D>::INSTR_PER_WAVE], int next_soff,
                                            int k0, int r0, int my_row, bool active, float sc) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, hi = lane >> 5, grp = lane >> 4, sidx = lane & 15;
  if (prefetch) {
    issue_tile<FaLayout<D>::INSTR_PER_WAVE>(kseg, seg_bytes, koff, next_soff, k_next, wave);
    issue_tile<FaLayout<D>::INSTR_PER_WAVE>(vseg, seg_bytes, voff, next_soff, v_next, wave);
  }
  if (!active || k0 > r0 + 31) return;
#pragma unroll
  for (int b2 = 0; b2 < 2; ++b2) {
    const int kb0 = k0 + 32 * b2;          // first key of this 32-key block
    if (kb0 > r0 + 31) break;              // block entirely above the diagonal
    // ---- S^T = K Q^T for 32 keys
    f32x16 sacc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
    const int row = 32 * b2 + l32;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      const bf16x8 ka = lds_read8(kt_lds + row * D + 8 * k_chunk<D>(row, 2 * c + hi));
      sacc = mfma32(ka, st.qreg[c], sacc);
    }
    // ---- causal mask (only blocks that reach past the wave's first row)
    if (kb0 + 31 > r0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kb0 + 8 * (r >> 2) + 4 * hi + (r & 3);
        if (key > my_row) sacc[r] = -__builtin_inff();
      }
    }
    // ---- online softmax (log2 domain) with lazy rescaling
    float mx = sacc[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sacc[r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mxs = mx * sc;
    const bool grow = mxs > st.m_run + kRescaleSlack;
    if (__any(grow)) {
      const float alpha = grow ? exp2_fast(st.m_run - mxs) : 1.f;
      st.m_run = grow ? mxs : st.m_run;
      st.l_run *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) st.o[db][r] *= alpha;
    }
    bf16x8 pb[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float p = exp2_fast(__builtin_fmaf(sacc[8 * hf + i], sc, -st.m_run));
        st.l_run += p;
        pb[hf][i] = f2bf(p);
      }
    // ---- O^T += V^T P^T
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int rowA = 32 * b2 + 16 * hf + 4 * hi + (sidx >> 2);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int col = 32 * db + 16 * (grp & 1) + 4 * (sidx & 3);
        const int cw = col & 7;                // element offset inside the 16-byte chunk
        const s16x4 x = lds_read_tr16(vt_lds + rowA * D + 8 * v_chunk<D>(rowA, col >> 3) + cw);
        const s16x4 y = lds_read_tr16(vt_lds + (rowA + 8) * D + 8 * v_chunk<D>(rowA + 8, col >> 3) + cw);
        const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7));
        st.o[db] = mfma32(va, pb[hf], st.o[db]);
      }
    }
  }
}

template <int D>
__global__ __launch_bounds__(kThreads, 2)
void fa_fwd_kernel(FaArgs a) {
  using L = FaLayout<D>;
  __shared__ __attribute__((aligned(1024))) bf16 kt0[L::TILE_ELEMS];
  __shared__ __attribute__((aligned(1024))) bf16 kt1[L::TILE_ELEMS];
  __shared__ __attribute__((aligned(1024))) bf16 vt0[L::TILE_ELEMS];
  __shared__ __attribute__((aligned(1024))) bf16 vt1[L::TILE_ELEMS];
  __shared__ float zsh[D];
  __shared__ __attribute__((aligned(16))) float csh[D];

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

  const int64_t tok0 = (int64_t)bh * a.L + (int64_t)s * a.N;
  const bf16* __restrict__ qb = a.q + tok0 * D;
  bf16* __restrict__ ob = a.out + tok0 * D;

  const bool has_memory = (a.seg_base + s) > 0;
  const float g = sigmoid_gate(a.beta[h]);
  const float sc = a.sc_log2;
  const int nk = a.N / kBN;

  const uint32_t seg_bytes = (uint32_t)a.N * D * 2;
  const bf16* kseg = a.k + tok0 * D;
  const bf16* vseg = a.v + tok0 * D;
  int koff[L::INSTR_PER_WAVE], voff[L::INSTR_PER_WAVE];
  tile_offsets<D, false>(koff, wave, lane);
  tile_offsets<D, true>(voff, wave, lane);
  constexpr int kTileBytes = kBN * D * 2;

  for (int pass = 0; pass < 2; ++pass) {
    const int qt = pass == 0 ? pair : a.nq - 1 - pair;
    if (pass == 1 && qt == pair) break;
    const int q0 = qt * kBM;
    const int r0 = q0 + 32 * wave;            // first query row of this wave
    const bool active = r0 < a.N;
    const int my_row = r0 + l32;               // query of this lane
    const int last = min(nk - 1, (q0 + kBM - 1) / kBN);

    issue_tile<L::INSTR_PER_WAVE>(kseg, seg_bytes, koff, 0, kt0, wave);
    issue_tile<L::INSTR_PER_WAVE>(vseg, seg_bytes, voff, 0, vt0, wave);

    RowState<D> st;
    if (active) {
#pragma unroll
      for (int c = 0; c < D / 16; ++c)
        st.qreg[c] = *reinterpret_cast<const bf16x8*>(qb + (int64_t)my_row * D + 16 * c + 8 * hi);
    }
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.o[db][r] = 0.f;
    st.m_run = -__builtin_inff();
    st.l_run = 0.f;

    wait_loads_and_sync();
    for (int kt = 0; kt <= last; kt += 2) {
      attend_tile<D>(st, kt0, vt0, kt1, vt1, kt < last, kseg, vseg, seg_bytes, koff, voff, (kt + 1) * kTileBytes,
                     kt * kBN, r0, my_row, active, sc);
      wait_loads_and_sync();
      if (kt + 1 <= last) {
        attend_tile<D>(st, kt1, vt1, kt0, vt0, kt + 1 < last, kseg, vseg, seg_bytes, koff, voff, (kt + 2) * kTileBytes,
                       (kt + 1) * kBN, r0, my_row, active, sc);
        wait_loads_and_sync();
      }
    }

    const float l_tot = st.l_run + __shfl_xor(st.l_run, 32);
    const float inv_l = 1.f / l_tot;

    // ---- retrieval epilogue: rows [0, 64) of the M^T snapshot go to kt0, the
    // rest to kt1 (same layout and swizzle as a K tile)
    f32x16 am[D / 32];
    float den = 0.f;
    if (has_memory) {
      {
        const bf16* snap = a.snapM + (int64_t)sh * D * D;
        issue_tile<L::INSTR_PER_WAVE>(snap, kBN * D * 2, koff, 0, kt0, wave);
        if (D > kBN) issue_tile<L::INSTR_PER_WAVE>(snap + kBN * D, (D - kBN) * D * 2, koff, 0, kt1, wave);
      }
      for (int i = threadIdx.x; i < D; i += kThreads) {
        zsh[i] = a.snapz[(int64_t)sh * D + i];
        csh[i] = a.snapc[(int64_t)sh * D + i];
      }
      wait_loads_and_sync();
      if (active) {
        // accumulator starts at colsum(M)[d_value of each element]
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const f32x4 c4 = *(const INFINI_LDS f32x4*)(csh + 32 * db + 8 * j + 4 * hi);
#pragma unroll
            for (int e = 0; e < 4; ++e) am[db][4 * j + e] = c4[e];
          }
        float zpart = 0.f;
#pragma unroll
        for (int c = 0; c < D / 16; ++c) {
          bf16x8 qp;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float x = bf2f(st.qreg[c][i]);
            const float f = x > 0.f ? x : exp_e(x) - 1.f;   // q' = sigma(q) - 1
            const float zz = zsh[16 * c + 8 * hi + i];
            den = __builtin_fmaf(f, zz, den);
            zpart += zz;
            qp[i] = f2bf(f);
          }
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            const int row = 32 * db + l32;
            const bf16* mt = row < kBN ? kt0 : kt1;
            const int rr = row & (kBN - 1);
            const bf16x8 ma = lds_read8(mt + rr * D + 8 * k_chunk<D>(rr, 2 * c + hi));
            am[db] = mfma32(ma, qp, am[db]);
          }
        }
        den += zpart;                      // sum(z) over this lane's half of d_key
        den += __shfl_xor(den, 32);
      }
    } else {
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) am[db][r] = 0.f;
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
          for (int e = 0; e < 4; ++e)
            outv[e] = f2bf(__builtin_fmaf(st.o[db][4 * j + e], wg_dot, am[db][4 * j + e] * wg_mem));
          *reinterpret_cast<bf16x4*>(orow + 32 * db + 8 * j + 4 * hi) = outv;
        }
    }
    if (has_memory) __syncthreads();  // LDS (snapshot, z, colsum) is reused by the next tile pair
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
