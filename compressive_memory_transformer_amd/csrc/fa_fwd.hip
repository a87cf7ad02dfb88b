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
// same amount of causal work.  Each wave owns 32 query rows.  Per 64-key tile:
//   S^T (64 keys x 32 queries) = K Q^T on v_mfma_f32_32x32x16_bf16, so that each
//   lane holds one query column and the softmax row statistics are per lane (one
//   cross-lane exchange with lane l^32 for the other half of the keys);
//   O^T (D x 32) += V^T P^T, with V^T read from the row-major V tile in LDS by
//   ds_read_b64_tr_b16 and P^T taken straight from the S^T accumulators (the key
//   order inside each 16-key step is permuted identically on both operands).
// K and V tiles stream from HBM straight into LDS (buffer_load ... lds, 16 bytes
// per lane, no staging registers) through two distinct LDS tiles (ping-pong):
// the load of tile t+1 is in flight while tile t is used.  The tiles use an
// XOR-swizzled layout whose operand reads are free of bank conflicts.  The
// softmax keeps a reference maximum per
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

constexpr int kWaves = 4;
constexpr int kBM = 32 * kWaves;   // query rows per tile
constexpr int kBN = 64;            // keys per LDS tile
constexpr int kThreads = 64 * kWaves;
constexpr int kStages = 2;         // LDS ring depth (the tile in use + the one in flight)
constexpr float kRescaleSlack = 8.f;  // log2 units

template <int D>
struct FaLayout {
  static constexpr int CHUNKS = D / 8;                 // 16-byte chunks per row
  static constexpr int TILE_ELEMS = kBN * D;           // one K or V tile, unpadded
  static constexpr int ROWS_PER_INSTR = 64 * 8 / D;    // rows one wave-wide 16-byte load covers
  static constexpr int INSTR_PER_WAVE = kBN / ROWS_PER_INSTR / kWaves;  // per 64-row tile and tensor
  static_assert(INSTR_PER_WAVE >= 1, "tile too small for the wave count");
  static_assert(D <= 2 * kBN, "the snapshot of M^T must fit the two K buffers");
};

// Physical 16-byte chunk of logical chunk c in row r (an XOR, so the same map
// takes physical to logical).  An LDS read of 16 bytes per lane is served 16
// lanes at a time and a 32-row transposing read 32 lanes at a time; each group
// must touch 16 distinct 16-byte bank groups of the 256-byte bank line.
//   K: lanes 0-15 of an operand read read the same logical chunk of 16
//   consecutive rows: XOR with r % 16 (D = 128, one row per bank line) or with
//   (r / 2) % 8 (D = 64, two rows per bank line).
//   V: a 32-lane half of a transposing read covers 4 consecutive rows x 4
//   logical chunks: rows r % 4 (D = 128) or (r / 2) % 2 (D = 64) move to
//   disjoint groups of 4 chunks.
template <int D>
__device__ __forceinline__ int k_swz(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int D>
__device__ __forceinline__ int k_chunk(int r, int c) { return c ^ k_swz<D>(r); }
template <int D>
__device__ __forceinline__ int v_chunk(int r, int c) { return c ^ (D == 128 ? (r & 3) << 2 : ((r >> 1) & 1) << 2); }

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

// buffer_load_dwordx4 ... lds: uniform descriptor + 32-bit per-lane offset; the
// tile's position in the buffer goes into the scalar offset.  The per-lane
// offsets are recomputed at each issue (a few integer ops) rather than kept in
// registers across the tile loop: the lane id passes through an empty asm so the
// arithmetic is not hoisted.
template <int D, bool IS_V, int NI>
__device__ __forceinline__ void issue_tile(const bf16* base, uint32_t bytes, int soff_bytes, bf16* lds_tile,
                                           int wave) {
  const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(base, bytes);
  // the LDS destination (M0) is wave-uniform: derive it in scalar registers
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  int lane = threadIdx.x & 63;
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" : "+v"(lane));  // device pass only: "v" is a gfx register class
#endif
#pragma unroll
  for (int j = 0; j < NI; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (INFINI_LDS void*)(lds_tile + (wv * NI + j) * 512), 16,
                                             2 * tile_lane_offset<D, IS_V>(wv * NI + j, lane), soff_bytes, 0, 0);
}

__device__ __forceinline__ void wait_loads_and_sync() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's LDS-bound loads have landed
  __syncthreads();
}

}  // namespace

// Per-lane LDS element offsets, relative to a tile's base, of the MFMA operand
// reads of attend_tile; they do not depend on the tile or stage, so the tile
// loop needs only these registers plus immediate offsets.
//   K: logical chunk 2c + hi of row 32 b2 + l32, c = 4m + j, sits at physical
//   chunk (2c + hi) ^ w, w = k_swz(l32) (row steps of 32 keep w): element offset
//   k[j] + m * kd + 32 b2 D, where k[j] covers m = 0 and kd = +-64 flips bit 3
//   of the chunk for m = 1 (D = 128 only).
//   V^T (tr16 reads): rows 32 b2 + 16 hf + 4 hi + sidx / 4 (+ 8), column 32 db + ...,
//   element offset v[db] + (32 b2 + 16 hf) D (+ 8 D); those row steps keep the
//   swizzle unchanged.
template <int D>
struct LdsAddr {
  int k[4];
  int kd;
  int v[D / 32];
  __device__ __forceinline__ void init(int lane) {
    const int l32 = lane & 31, hi = lane >> 5, grp = lane >> 4, sidx = lane & 15;
    const int w = k_swz<D>(l32);
#pragma unroll
    for (int j = 0; j < 4; ++j) k[j] = l32 * D + 8 * ((2 * j + hi) ^ w);
    kd = (w & 8) ? -64 : 64;
    const int rowA = 4 * hi + (sidx >> 2);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int col = 32 * db + 16 * (grp & 1) + 4 * (sidx & 3);
      v[db] = rowA * D + 8 * v_chunk<D>(rowA, col >> 3) + (col & 7);
    }
  }
  // K operand offset of 16-column step c (0 <= c < D / 16) of row l32
  __device__ __forceinline__ int kofs(int c) const { return c < 4 ? k[c] : k[c - 4] + kd; }
};

// Per-wave running state of one 32-row query block.
template <int D>
struct RowState {
  bf16x8 qreg[D / 16];   // Q^T as the B operand: lane holds Q[row][16c + 8hi .. +7]
  f32x16 o[D / 32];      // O^T accumulator: lane holds O[row][32db + 8(r/4) + 4hi + r%4]
  float m_run;           // reference maximum of the row (log2 domain)
  float l_run;           // this lane's share of the softmax denominator
};

// S^T for 32 keys (block b2 of the tile): K operands read four at a time.
template <int D>
__device__ __forceinline__ void s_block(f32x16& acc, const bf16* __restrict__ kt_lds, int b2, const LdsAddr<D>& ad,
                                        const bf16x8 (&qreg)[D / 16]) {
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
  for (int m = 0; m < D / 64; ++m) {
    bf16x8 ka[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) ka[j] = lds_read8(kt_lds + 32 * b2 * D + ad.kofs(4 * m + j));
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = mfma32(ka[j], qreg[4 * m + j], acc);
  }
}

// O^T += V^T P^T for 32 keys (block b2 of the tile).
template <int D>
__device__ __forceinline__ void pv_block(RowState<D>& st, const bf16* __restrict__ vt_lds, int b2,
                                         const LdsAddr<D>& ad, const bf16x8 (&pb)[2]) {
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    bf16x8 va[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const bf16* p = vt_lds + (32 * b2 + 16 * hf) * D + ad.v[db];
      const s16x4 x = lds_read_tr16(p);
      const s16x4 y = lds_read_tr16(p + 8 * D);
      va[db] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7));
    }
#pragma unroll
    for (int db = 0; db < D / 32; ++db) st.o[db] = mfma32(va[db], pb[hf], st.o[db]);
  }
}

// Softmax of one 32-key block, first part (no branches, no state change): the
// probabilities against the current reference maximum of the row.  Returns
// whether one of them exceeds 2^8, i.e. a score grew past the reference by more
// than the slack (then the caller rescales).  The row maximum itself is only
// needed in that rare case.
__device__ __forceinline__ bool softmax_exp(const f32x16& s, float m_run, float sc, f32x16& p) {
#pragma unroll
  for (int r = 0; r < 16; ++r) p[r] = exp2_fast(__builtin_fmaf(s[r], sc, -m_run));
  float pm = p[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) pm = fmaxf(pm, p[r]);
  return pm > 256.f;  // exp2(kRescaleSlack)
}

// Causal mask of a block whose first key is kb0: keys after the lane's query get -inf.
__device__ __forceinline__ void mask_block(f32x16& sacc, int kb0, int my_row) {
  int lane = threadIdx.x & 63;
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" : "+v"(lane));  // recomputed here, not kept live across the tile loop
#endif
  const int hi = lane >> 5;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int key = kb0 + 8 * (r >> 2) + 4 * hi + (r & 3);
    if (key > my_row) sacc[r] = -__builtin_inff();
  }
}

// Second part: if some row's maximum grew past the slack (rare after the first
// block of a row), move that row's reference to its new maximum (the two lanes
// holding a row take the same decision), rescale the accumulator and recompute
// the probabilities; then add them to the denominator and pack them to bf16.
template <int D>
__device__ __forceinline__ void softmax_finish(RowState<D>& st, const f32x16& s, f32x16& p, float sc, bool big,
                                               bf16x8 (&pb)[2]) {
  if (__any(big)) {
    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mxs = mx * sc;
    const bool grow = mxs > st.m_run + kRescaleSlack;
    const float alpha = grow ? exp2_fast(st.m_run - mxs) : 1.f;
    st.m_run = grow ? mxs : st.m_run;
    st.l_run *= alpha;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.o[db][r] *= alpha;
#pragma unroll
    for (int r = 0; r < 16; ++r) p[r] = exp2_fast(__builtin_fmaf(s[r], sc, -st.m_run));
  }
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      st.l_run += p[8 * hf + i];
      pb[hf][i] = f2bf(p[8 * hf + i]);
    }
}

// One 64-key tile: S^T, mask, softmax and O^T update for the keys of this tile
// that the wave's rows can see.  (The DMA of the next tile into the other pair
// of buffers is issued just before; the buffers are distinct objects, so the
// compiler never waits on that DMA before reading this tile.)  A tile wholly
// below the wave's diagonal runs software-pipelined: the S^T MFMAs of the
// second 32-key block are issued next to the softmax VALU work of the first,
// and the PV MFMAs of the first next to the softmax of the second.
template <int D>
__device__ __forceinline__ void attend_tile(RowState<D>& st, const bf16* __restrict__ kt_lds,
                                            const bf16* __restrict__ vt_lds, const LdsAddr<D>& ad, int k0,
                                            int r0, int my_row, bool active, float sc) {
  const int lane = threadIdx.x & 63;
  const int hi = lane >> 5;
  if (!active || k0 > r0 + 31) return;
  if (k0 + kBN - 1 <= r0) {
    // full tile: no mask, pipelined
    f32x16 s0, s1, p;
    bf16x8 pb0[2], pb1[2];
    s_block<D>(s0, kt_lds, 0, ad, st.qreg);
    s_block<D>(s1, kt_lds, 1, ad, st.qreg);
    const bool g0 = softmax_exp(s0, st.m_run, sc, p);
    softmax_finish<D>(st, s0, p, sc, g0, pb0);
    pv_block<D>(st, vt_lds, 0, ad, pb0);
    const bool g1 = softmax_exp(s1, st.m_run, sc, p);
    softmax_finish<D>(st, s1, p, sc, g1, pb1);
    pv_block<D>(st, vt_lds, 1, ad, pb1);
    return;
  }
  // tile on the diagonal: per 32-key block, masked
#pragma unroll
  for (int b2 = 0; b2 < 2; ++b2) {
    const int kb0 = k0 + 32 * b2;          // first key of this 32-key block
    if (kb0 > r0 + 31) break;              // block entirely above the diagonal
    f32x16 sacc;
    s_block<D>(sacc, kt_lds, b2, ad, st.qreg);
    const bool masked = kb0 + 31 > r0;
    if (masked) mask_block(sacc, kb0, my_row);
    f32x16 p;
    bf16x8 pb[2];
    const bool g = softmax_exp(sacc, st.m_run, sc, p);
    softmax_finish<D>(st, sacc, p, sc, g, pb);
    pv_block<D>(st, vt_lds, b2, ad, pb);
  }
}

// Waits until this wave's loads of the tile needed next have landed (the loads
// of `later` younger tiles may stay in flight), then synchronises the workgroup.
template <int NI>
__device__ __forceinline__ void stage_barrier(int later) {
  // s_waitcnt vmcnt(n) lgkmcnt(0); n = 2 * NI * later (K and V instructions per tile)
  if (later >= 2)
    __builtin_amdgcn_s_waitcnt((4 * NI) | 0x0070);
  else if (later == 1)
    __builtin_amdgcn_s_waitcnt((2 * NI) | 0x0070);
  else
    __builtin_amdgcn_s_waitcnt(0x0070);
  __builtin_amdgcn_s_barrier();
}

template <int D>
__global__ __launch_bounds__(kThreads, 2)
void fa_fwd_kernel(FaArgs a) {
  using L = FaLayout<D>;
  constexpr int NI = L::INSTR_PER_WAVE;
  __shared__ __attribute__((aligned(1024))) bf16 ks0[L::TILE_ELEMS];
  __shared__ __attribute__((aligned(1024))) bf16 ks1[L::TILE_ELEMS];
  __shared__ __attribute__((aligned(1024))) bf16 vs0[L::TILE_ELEMS];
  __shared__ __attribute__((aligned(1024))) bf16 vs1[L::TILE_ELEMS];
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
  const int rowblk = wave;

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
  constexpr int kTileBytes = kBN * D * 2;
  LdsAddr<D> ad;
  ad.init(lane);

  for (int pass = 0; pass < 2; ++pass) {
    const int qt = pass == 0 ? pair : a.nq - 1 - pair;
    if (pass == 1 && qt == pair) break;
    const int q0 = qt * kBM;
    const int r0 = q0 + 32 * rowblk;          // first query row of this wave
    const bool active = r0 < a.N;
    const int my_row = r0 + l32;               // query of this lane
    const int last = min(nk - 1, (q0 + kBM - 1) / kBN);

    // Q^T as the B operand (issued first: the oldest loads of this pass)
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

    // prologue: tile 0 into stage 0; wait for it (and Q)
    issue_tile<D, false, NI>(kseg, seg_bytes, 0, ks0, wave);
    issue_tile<D, true, NI>(vseg, seg_bytes, 0, vs0, wave);
    stage_barrier<NI>(0);

    // One step: prefetch tile t+1 into the other stage, use tile t, wait for t+1.
#define INFINI_FA_STEP(T, KC, VC, KN, VN)                                                              \
    {                                                                                                  \
      const int t_ = (T);                                                                              \
      if (t_ + 1 <= last) {                                                                            \
        issue_tile<D, false, NI>(kseg, seg_bytes, (t_ + 1) * kTileBytes, KN, wave);                     \
        issue_tile<D, true, NI>(vseg, seg_bytes, (t_ + 1) * kTileBytes, VN, wave);                      \
      }                                                                                                \
      attend_tile<D>(st, KC, VC, ad, t_ * kBN, r0, my_row, active, sc);                               \
      stage_barrier<NI>(0);                                                                            \
    }
    for (int kt = 0; kt <= last; kt += kStages) {
      INFINI_FA_STEP(kt, ks0, vs0, ks1, vs1)
      if (kt + 1 > last) break;
      INFINI_FA_STEP(kt + 1, ks1, vs1, ks0, vs0)
    }
#undef INFINI_FA_STEP

    const float l_tot = st.l_run + __shfl_xor(st.l_run, 32);
    const float inv_l = 1.f / l_tot;

    // ---- retrieval epilogue: rows [0, 64) of the M^T snapshot go to ks0, the
    // rest to ks1 (same layout and swizzle as a K tile)
    f32x16 am[D / 32];
    float den = 0.f;
    if (has_memory) {
      {
        const bf16* snap = a.snapM + (int64_t)sh * D * D;
        issue_tile<D, false, NI>(snap, kBN * D * 2, 0, ks0, wave);
        if (D > kBN) issue_tile<D, false, NI>(snap + kBN * D, (D - kBN) * D * 2, 0, ks1, wave);
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
            // row 32 db + l32 of M^T: rows [0, 64) in ks0, [64, 128) in ks1
            const bf16* mt = (db < 2 ? ks0 : ks1) + 32 * (db & 1) * D;
            const bf16x8 ma = lds_read8(mt + ad.kofs(c));
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
    __syncthreads();  // every stage (snapshot, z, colsum) is reused by the next tile pair
  }
}

int64_t fa_fwd_blocks(int64_t seg_heads, int N) {
  const int nq = (N + kBM - 1) / kBM;
  return seg_heads * ((nq + 1) / 2);
}

template <int D>
hipError_t launch_fa_fwd(const FaArgs& args, hipStream_t stream) {
  FaArgs a = args;
  a.nq = (a.N + kBM - 1) / kBM;
  const int64_t blocks = fa_fwd_blocks((int64_t)a.B * a.H * a.S, a.N);
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(fa_fwd_kernel<D>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template hipError_t launch_fa_fwd<64>(const FaArgs&, hipStream_t);
template hipError_t launch_fa_fwd<128>(const FaArgs&, hipStream_t);

}  // namespace infini
