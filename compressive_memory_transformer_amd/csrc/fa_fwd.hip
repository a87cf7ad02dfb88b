// Fused segment kernel for the bf16 path: local causal attention (flash style,
// online softmax in fp32), retrieval from the compressive memory snapshot,
// sigmoid gate, bf16 output.
//
// Equations (page "精读笔记：Infini-attention"): A_dot of section 3.1 with the
// causal mask of section 3.8 step 2, restricted to the current segment; A_mem of
// section 3.3; the gate of section 3.5.  The N x N score matrix never leaves
// registers (chapter-24 page, section 24.1.2).
//
// Work decomposition.  An item is a pair of 256-row query tiles of one (b, h,
// segment): tile w and tile NQ-1-w, so that every item holds the same causal
// work.  One workgroup (8 waves, two per SIMD) per CU walks the items of its
// XCD in turn (a persistent grid; a launch over a range of segments runs one
// workgroup per item instead), each pass overlapping the next one's first
// loads whether or not it belongs to the same item.  Wave w owns
// the 32-row query block 32 w + [0, 32) of a tile.  The two waves of a SIMD
// interleave in hardware: while one runs its softmax (VALU) or waits for LDS,
// the other keeps the matrix pipe busy.  Per 32-key block of a 128-key tile:
//   S^T (32 keys x 32 queries) = K Q^T on v_mfma_f32_32x32x16_bf16: each lane
//   holds one query column, so the softmax statistics are per lane (one
//   exchange with lane l^32 holds the rest of a row);
//   O^T (D x 32) += V^T P^T, with V^T read from the row-major V tile by
//   ds_read_b64_tr_b16 and P^T taken straight from the S^T accumulators (the key
//   order inside each 16-key step is permuted identically on both operands).
// Within a wave, the S^T products of block j+1 are issued next to the softmax
// of block j.
//
// Data movement.  K and V tiles stream from HBM into LDS with buffer_load ... lds
// (16 bytes per lane, no staging registers) through two LDS slots; tile t of a
// pass sits in slot t % 2 and the load of item t+1 is in flight while tile t is
// used.  Every pass covers an even number of key tiles, so the last one uses
// slot 1 and brings the memory snapshot (M^T, z, colsum(M)) into slot 0 along
// with the V part of the next pass's tile 0; the slot of every load is known at
// compile time (the step loop is unrolled by two), so the compiler never waits
// on a load into the other slot.  The slot layouts are XOR-swizzled so that the
// operand reads are free of bank conflicts.
//
// Softmax.  Each query keeps a reference maximum m, set before the tile loop to
// the exact maximum of its first 32-key block (which always holds an unmasked
// key); probabilities are exp2(s * scale * log2 e - m) and are never rescaled.
// The result is exact for any m; m only has to keep the sums finite.  A block
// whose probabilities sum past 2^64 (or to inf or NaN) raises a flag, and a
// flagged query block is recomputed after the loop by a slow two-sweep path
// (exact row maximum first) that reads K and V straight from memory.
//
// Epilogue: with sigma(q) = 1 + q', q' = sigma(q) - 1,
//   sigma(q) M = colsum(M) + q' M   and   sigma(q) z = sum(z) + q' z,
// where colsum(M) (sum over d_key) comes in fp32 with the snapshot and q' M runs
// on MFMA from the bf16 snapshot of M_{s-1}^T.  q' keeps the full relative
// precision of bf16, unlike sigma(q) ~ 1 + q itself.  Gate, round to bf16, store
// through a small LDS stage per wave as whole 64-byte row segments.
//
// Q rows reach LDS like K and V: a pass's 256 rows load into slot 1 (free while
// the epilogue of the previous pass runs, or with tile 0 for the first pass), so
// their memory latency hides behind other work; each wave reads its 32 rows
// from there before the first key tile.
#include "common.h"
#include "kernels.h"

namespace infini {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;   // query rows per tile: one 32-row block per wave
constexpr int kBN = 128;           // keys per LDS tile
constexpr int kKB = kBN / 32;      // 32-key blocks per tile
constexpr int kDmaBlocks = 2;      // blocks of a tile that issue the next load item
constexpr float kSumLimit = 18446744073709551616.f;  // 2^64
// A query block with a component of magnitude above this takes the precise
// retrieval (exact q re-read, q' and M each as bf16 hi + lo).  Below it the
// query-dependent part q' M is a small share of the retrieval and one bf16 part
// of each is exact enough.
constexpr float kPreciseQ = 0.5f;

template <int D>
struct FaLayout {
  static constexpr int CHUNKS = D / 8;                 // 16-byte chunks per row
  static constexpr int TILE_ELEMS = kBN * D;           // one K or V tile, unpadded
  static constexpr int ROWS_PER_INSTR = 64 * 8 / D;    // rows one wave-wide 16-byte load covers
  static constexpr int NI = kBN / ROWS_PER_INSTR / kWaves;  // loads per wave, tensor and tile
  static constexpr int KPER = 16 / ROWS_PER_INSTR;     // instructions per period of the K swizzle
  static_assert(NI >= 1 && (2 * NI) % kDmaBlocks == 0, "tile loads must split evenly over the blocks");
  static_assert(NI % KPER == 0, "each wave's first load starts a K swizzle period");
  static_assert(D <= kBN, "the snapshot of M^T must fit a K slot");
  static_assert(D <= 256, "z and colsum must fit their LDS array");
  static_assert(kBM == 2 * kBN, "the Q rows of a query tile fill the two parts of a slot");
};

// Output stage: 32 rows x 32 columns (bf16) per wave.
constexpr int kStageElems = 32 * 32;

// Physical 16-byte chunk of logical chunk c in row r (an XOR, so the same map
// takes physical to logical).  An LDS read of 16 bytes per lane is served 16
// lanes at a time and a transposing read 32 lanes at a time; each group must
// touch 16 distinct 16-byte bank groups of the 256-byte bank line.
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

// Issue this wave's share of the direct-to-LDS loads of a row-major [kBN x D]
// tile: wave-wide instruction `ins` fills bytes [1024 ins, 1024 ins + 1024) of the
// LDS tile, lane l landing at 16 l (row ROWS_PER_INSTR * ins + l / CHUNKS).
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
#if defined(__HIP_DEVICE_COMPILE__)
// The arguments are wave-uniform; readfirstlane states it, so the descriptor
// lives in scalar registers (a descriptor in vector registers makes the
// compiler wrap each load in a per-lane loop).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  void* ub = (void*)(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}
#endif

// Per-lane byte offsets of the direct-to-LDS loads.  Wave-wide instruction ins
// of a [kBN x D] tile fills bytes [1024 ins, 1024 ins + 1024) of the LDS tile;
// the K swizzle repeats every KPER instructions and the V swizzle does not
// depend on the instruction, so lane l's global offset is k[ins % KPER] + 1024
// (ins - ins % KPER) for K and v + 1024 ins for V (same row pitch in HBM and LDS).
template <int D>
struct DmaOfs {
  int k[FaLayout<D>::KPER];
  int v;
  __device__ __forceinline__ void init(int lane) {
#pragma unroll
    for (int i = 0; i < FaLayout<D>::KPER; ++i) k[i] = 2 * tile_lane_offset<D, false>(i, lane);
    v = 2 * tile_lane_offset<D, true>(0, lane);
  }
};

// buffer_load_dwordx4 ... lds: uniform descriptor (base = the tile's first
// element, num_records = bytes left in the tensor range) + 32-bit per-lane
// offset, which is what the bounds check compares; instructions [j0, j0 + CNT)
// of this wave's NI.  A range of 0 bytes issues loads that
// write zeros (used to keep the number of loads per step uniform).
template <int D, bool IS_V, int CNT>
__device__ __forceinline__ void issue_part(int j0, const bf16* base, uint32_t bytes, bf16* lds_tile, int wave,
                                           const DmaOfs<D>& dof) {
#if defined(__HIP_DEVICE_COMPILE__)  // the buffer builtins exist in the device pass only
  constexpr int NI = FaLayout<D>::NI;
  constexpr int KPER = FaLayout<D>::KPER;
  const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(base, bytes);
  // the LDS destination (M0) and the instruction's share of the offset are
  // wave-uniform: derive them in scalar registers
  const int wv = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
  for (int jj = 0; jj < CNT; ++jj) {
    const int j = j0 + jj;
    const int ins = wv * NI + j;   // ins % KPER == j % KPER (NI is a multiple of KPER)
    const int voff = IS_V ? dof.v + 1024 * ins : dof.k[j % KPER] + 1024 * (ins - j % KPER);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (INFINI_LDS void*)(lds_tile + ins * 512), 16, voff, 0, 0, 0);
  }
#endif
}
template <int D, bool IS_V>
__device__ __forceinline__ void issue_tile(const bf16* base, uint32_t bytes, bf16* lds_tile, int wave,
                                           const DmaOfs<D>& dof) {
  issue_part<D, IS_V, FaLayout<D>::NI>(0, base, bytes, lds_tile, wave, dof);
}

// One wave-wide 16-byte-per-lane load of `bytes` (<= 1024) contiguous bytes into LDS.
__device__ __forceinline__ void issue_row(const void* base, uint32_t bytes, void* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(base, bytes);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (INFINI_LDS void*)lds, 16, 16 * (int)(threadIdx.x & 63), 0, 0, 0);
#endif
}

// Waits until this wave's outstanding loads (LDS-bound and register-bound) have
// landed, then synchronises the workgroup.
__device__ __forceinline__ void wait_loads_and_sync() {
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
}

// Waits for this wave's LDS accesses only (stores and loads to memory may stay in
// flight), then synchronises the workgroup.
__device__ __forceinline__ void wait_lds_and_sync() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
}

}  // namespace

// Per-lane LDS element offsets, relative to a tile's base, of the MFMA operand
// reads; they do not depend on the tile or slot, so the tile loop needs only
// these registers plus immediate offsets.
//   K: logical chunk 2c + hi of row 32 j + l32, c = 4m + i, sits at physical
//   chunk (2c + hi) ^ w, w = k_swz(l32) (row steps of 32 keep w): element offset
//   k[i] + m * kd + 32 j D, where k[i] covers m = 0 and kd = +-64 flips bit 3
//   of the chunk for m = 1 (D = 128 only).
//   V^T (tr16 reads): rows 32 j + 16 hf + 4 hi + sidx / 4 (+ 8), column 32 db + ...,
//   element offset v[db] + (32 j + 16 hf) D (+ 8 D); those row steps keep the
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
    for (int i = 0; i < 4; ++i) k[i] = l32 * D + 8 * ((2 * i + hi) ^ w);
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

// Running state of one 32-row query block of a wave.
template <int D>
struct QBlock {
  bf16x8 q[D / 16];    // Q^T * scale * log2 e as the B operand: lane holds Q[row][16c + 8hi .. +7]
  f32x16 o[D / 32];    // O^T accumulator: lane holds O[row][32db + 8(r/4) + 4hi + r%4]
  f32x16 mneg;         // -m in every element: the initial accumulator of S^T
  float m;             // reference maximum of the row (log2 domain)
  float l;             // this lane's share of the softmax denominator
  bool bad;            // some block summed past the limit: recompute the block
  bool big;            // some query component of the block exceeds kPreciseQ (wave-uniform)
};

// The load item a step brings into the other slot: a K part and a V part, NI
// wave-wide instructions each; empty ranges load zeros.
template <int D>
struct Prefetch {
  const bf16* kb;
  const bf16* vb;
  uint32_t kbytes, vbytes;
  bf16* kn;
  bf16* vn;
  int wave;
  const DmaOfs<D>* dof;
  template <int CNT>
  __device__ __forceinline__ void issue(int j0) const {
    issue_part<D, false, CNT>(j0, kb, kbytes, kn, wave, *dof);
    issue_part<D, true, CNT>(j0, vb, vbytes, vn, wave, *dof);
  }
};

// S^T of key block j of the tile for one query block (K operands from LDS),
// from a zero accumulator.
template <int D>
__device__ __forceinline__ f32x16 s_block(const bf16* __restrict__ kt, int j, const LdsAddr<D>& ad,
                                          const bf16x8 (&q)[D / 16]) {
  f32x16 s;
#pragma unroll
  for (int r = 0; r < 16; ++r) s[r] = 0.f;
  bf16x8 ka[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) ka[c] = lds_read8(kt + 32 * j * D + ad.kofs(c));
  __builtin_amdgcn_sched_barrier(0);   // every read in flight before the first product
#pragma unroll
  for (int c = 0; c < D / 16; ++c) s = mfma32(ka[c], q[c], s);
  return s;
}

// Causal mask of a block whose first key is kb0: keys after the lane's query get -inf.
__device__ __forceinline__ void mask_block(f32x16& sacc, int kb0, int my_row) {
  const int hi = (threadIdx.x >> 5) & 1;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int key = kb0 + 8 * (r >> 2) + 4 * hi + (r & 3);
    if (key > my_row) sacc[r] = -__builtin_inff();
  }
}

// Row maximum of a 32 x 32 score block (log2 domain: Q carries the scale); the
// two lanes holding a row exchange their halves.
__device__ __forceinline__ float block_row_max(const f32x16& s) {
  float mx = s[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
  return fmaxf(mx, __shfl_xor(mx, 32));
}

// s - m for a block computed from a zero accumulator.
__device__ __forceinline__ void sub_m(f32x16& s, float m) {
#pragma unroll
  for (int r = 0; r < 16; ++r) s[r] -= m;
}

template <int D>
__device__ __forceinline__ void set_m(QBlock<D>& X, float m) {
  X.m = m;
#pragma unroll
  for (int r = 0; r < 16; ++r) X.mneg[r] = -m;
}


// Causal mask of a 32 x 32 score block by lane masks: element r of lane l holds
// key 8 (r / 4) + 4 (l / 32) + r % 4 of the block for query l % 32, so the lanes
// that mask element r on the diagonal block form a fixed 64-bit set.
__host__ __device__ constexpr uint64_t diag_lane_mask(int r) {
  return ((1ull << (8 * (r / 4) + r % 4)) - 1) | (((1ull << (8 * (r / 4) + r % 4 + 4)) - 1) << 32);
}

// Scores of key block kb for the query block starting at row r0 (both multiples
// of 32, wave-uniform): unchanged left of the diagonal, causally masked on it,
// all -inf right of it (one v_cndmask per element, lane set in scalar registers).
__device__ __forceinline__ void mask_scores(f32x16& s, int kb, int r0) {
#if defined(__HIP_DEVICE_COMPILE__)
  const int d = __builtin_amdgcn_readfirstlane(kb - r0);
  const float ninf = -__builtin_inff();
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const uint64_t m = d < 0 ? 0ull : (d == 0 ? diag_lane_mask(r) : ~0ull);
    float out;
    asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(out) : "v"(s[r]), "v"(ninf), "s"(m));
    s[r] = out;
  }
#endif
}

// Compiler fence: nothing is moved across it, so the slots of the tile pipeline
// keep the order in which they are written.
#define INFINI_FENCE() __builtin_amdgcn_sched_barrier(0)

// A 128-key tile through the software pipeline over its four 32-key blocks j.
// A wave issues in order, so its own MFMA and VALU work only overlap when they
// alternate in its instruction stream (the other wave of the SIMD fills what is
// left).  Each block is written as two phases of slots, one MFMA per slot
// followed by that slot's share of the other work:
//   phase 1: S^T(j+1) MFMAs | probabilities of block j (exp2, sums, bf16
//            packing, a few elements per slot) and the V^T operand reads of
//            block j
//   phase 2: O^T += V^T P^T MFMAs of block j | K operand reads of block j+2 and
//            the block's share of the next load item
// MASK: the tile holds the diagonal of the query block starting at row r0
// (blocks right of it are fully masked).
template <int D, bool MASK>
__device__ __forceinline__ void tile_pipe(QBlock<D>& X, const bf16* __restrict__ kt, const bf16* __restrict__ vt,
                                          const LdsAddr<D>& ad, const Prefetch<D>& pf, int k0, int r0) {
  constexpr int NI = FaLayout<D>::NI;          // prefetch instructions per tensor
  constexpr int DPB = 2 * NI / kDmaBlocks;     // prefetch instructions per block (K and V)
  constexpr int KS = D / 16;                   // 16-deep steps of an S^T chain = phase-1 slots
  constexpr int NV = D / 32;                   // O^T accumulators
  constexpr int N2 = 2 * NV;                   // phase-2 slots (O^T MFMAs)
  constexpr int E = 16 / KS;                   // softmax elements per phase-1 slot
  constexpr int DPS = (DPB + N2 - 1) / N2;     // prefetch instructions per phase-2 slot
  static_assert(2 * NV <= KS && KS <= N2, "slot shares");
  bf16x8 ko[KS];
  bf16x8 vo[2][NV];
  f32x16 s;   // S^T - m of the current block
  // all of block 0's K operand reads in flight before its first product (every
  // wave enters here from the same barrier, so a read-wait-product sequence
  // would leave the matrix pipe idle for one LDS round trip per product)
#pragma unroll
  for (int c = 0; c < KS; ++c) ko[c] = lds_read8(kt + ad.kofs(c));
  INFINI_FENCE();
  s = mfma32(ko[0], X.q[0], X.mneg);
#pragma unroll
  for (int c = 1; c < KS; ++c) s = mfma32(ko[c], X.q[c], s);
#pragma unroll
  for (int c = 0; c < KS; ++c) ko[c] = lds_read8(kt + 32 * D + ad.kofs(c));
  INFINI_FENCE();
  // On a diagonal tile the blocks right of the wave's diagonal block jd hold
  // masked keys only: the loop leaves after jd, and the skipped blocks' share of
  // the next load item is issued after it.
  const int jd = MASK ? __builtin_amdgcn_readfirstlane((r0 - k0) >> 5) : kKB - 1;
#pragma unroll
  for (int j = 0; j < kKB; ++j) {
    if (MASK && j > jd) break;
    const bool more = j + 1 < kKB;   // (on a diagonal tile, computed also for the block after jd)
    if (MASK) mask_scores(s, k0 + 32 * j, r0);
    f32x16 ns;
    bf16x8 p[2];
    float t = 0.f;
    INFINI_FENCE();
    // Phase 1 runs at raised issue priority: of the two waves of a SIMD, the one
    // in its softmax phase issues first, so the pair tends to alternate (one
    // wave's exponentials next to the other's P V products) instead of running
    // the same phase side by side.
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = 0; i < KS; ++i) {
      if (more) ns = mfma32(ko[i], X.q[i], i == 0 ? X.mneg : ns);
      if (i < 2 * NV) {
        const int hf = i / NV, db = i % NV;
        const bf16* pv = vt + (32 * j + 16 * hf) * D + ad.v[db];
        const s16x4 x = lds_read_tr16(pv);
        const s16x4 y = lds_read_tr16(pv + 8 * D);
        vo[hf][db] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
      for (int u = 0; u < E; ++u) {
        const int r = E * i + u;
        const float e = exp2_fast(s[r]);
        t += e;
        p[r / 8][r % 8] = f2bf(e);
      }
      INFINI_FENCE();
    }
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int i = 0; i < N2; ++i) {
      const int hf = i / NV, db = i % NV;
      X.o[db] = mfma32(vo[hf][db], p[hf], X.o[db]);
      if (j + 2 < kKB && i < KS) ko[i] = lds_read8(kt + 32 * (j + 2) * D + ad.kofs(i));
      if (j < kDmaBlocks) {
#pragma unroll
        for (int w = 0; w < DPS; ++w) {
          const int u = DPB * j + DPS * i + w;   // instruction u of this wave's K then V loads
          if (DPS * i + w < DPB && u < NI) issue_part<D, false, 1>(u, pf.kb, pf.kbytes, pf.kn, pf.wave, *pf.dof);
          else if (DPS * i + w < DPB) issue_part<D, true, 1>(u - NI, pf.vb, pf.vbytes, pf.vn, pf.wave, *pf.dof);
        }
      }
      if (i == 0) {
        X.bad |= !(t <= kSumLimit);
        X.l += t;
      }
      INFINI_FENCE();
    }
    if (more) s = ns;
  }
  // the skipped blocks' shares of the next load item
  if (MASK) {
#pragma unroll
    for (int j = 1; j < kDmaBlocks; ++j)
      if (j > jd) {
#pragma unroll
        for (int w = 0; w < DPB; ++w) {
          const int u = DPB * j + w;   // instruction u of this wave's K then V loads
          if (u < NI) issue_part<D, false, 1>(u, pf.kb, pf.kbytes, pf.kn, pf.wave, *pf.dof);
          else issue_part<D, true, 1>(u - NI, pf.vb, pf.vbytes, pf.vn, pf.wave, *pf.dof);
        }
      }
  }
}

// Reference maximum before the tile loop: the exact row maximum of key block 0,
// the first block every query sees (tile 0 is in LDS).
template <int D>
__device__ __forceinline__ void init_m(QBlock<D>& X, const bf16* __restrict__ kt, const LdsAddr<D>& ad, int r0) {
  f32x16 s = s_block<D>(kt, 0, ad, X.q);
  if (r0 == 0) mask_block(s, 0, threadIdx.x & 31);
  set_m(X, block_row_max(s));
}

// Slow, exact recompute of one query block whose sums left the safe range: two
// sweeps over its keys (row maxima, then probabilities against them, all <= 1),
// with K and V operands loaded straight from memory (no LDS, no barriers).
template <int D>
__device__ void recompute_block(QBlock<D>& X, int r0, const bf16* __restrict__ kseg,
                                const bf16* __restrict__ vseg) {
  const int lane = threadIdx.x & 63, l32 = lane & 31, hi = lane >> 5;
  auto scores = [&](int kb) {
    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      const bf16x8 ka = *reinterpret_cast<const bf16x8*>(kseg + (int64_t)(kb + l32) * D + 16 * c + 8 * hi);
      s = mfma32(ka, X.q[c], s);
    }
    if (kb == r0) mask_block(s, kb, r0 + l32);
    return s;
  };
  float m = -__builtin_inff();
#pragma unroll 1
  for (int kb = 0; kb <= r0; kb += 32) m = fmaxf(m, block_row_max(scores(kb)));
  set_m(X, m);
  X.l = 0.f;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) X.o[db][r] = 0.f;
#pragma unroll 1
  for (int kb = 0; kb <= r0; kb += 32) {
    const f32x16 s = scores(kb);
    bf16x8 p[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float e = exp2_fast(s[r] - m);
      X.l += e;
      p[r >> 3][r & 7] = f2bf(e);
    }
    // V^T operand: key order of the P^T rows (see pv_pair), column d_value 32 db + l32
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        bf16x8 va;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int key = kb + 16 * hf + (j < 4 ? 4 * hi + j : 8 + 4 * hi + (j - 4));
          va[j] = vseg[(int64_t)key * D + 32 * db + l32];
        }
        X.o[db] = mfma32(va, p[hf], X.o[db]);
      }
  }
  X.bad = false;
}

// Retrieval, gate and store of one query block.  mt: M^T snapshot (K-slot
// layout), zs / cs: z and colsum(M) in LDS, ob: the block's first output row,
// stages: 2 KB of LDS per wave for the output.  First q' and the denominator
// for all of d_key; then, one 32-column group of d_value at a time, the
// retrieval accumulator (colsum + M^T q'), the gate and the output, so that only
// one group's accumulator is live.
// Precise path (a block with a large query component, X.big): q is read again
// from memory (qg: the block's first query row) instead of being recovered from
// the scaled bf16 operand, q' = sigma(q) - 1 is split into bf16 hi + lo, and the
// product takes the snapshot's bf16 remainder (mlo: this segment's M^T
// remainder, row-major) as well: colsum + M_hi q'_hi + M_hi q'_lo + M_lo q'_hi.
template <int D>
__device__ __forceinline__ void finish_block(const QBlock<D>& X, const bf16* __restrict__ mt,
                                             const float* __restrict__ zs, const float* __restrict__ cs,
                                             const LdsAddr<D>& ad, bool has_memory, float beta, float inv_sc,
                                             bf16* __restrict__ ob, bf16* __restrict__ stages, int wave,
                                             const bf16* __restrict__ qg, const bf16* __restrict__ mlo,
                                             float* __restrict__ lrow) {
  // The lane index is computed here (from the exec mask, with an opaque base) so
  // that it and the per-lane addresses below are not hoisted to the kernel start
  // and kept live (spilled) across the tile loop: the reload of a spill here
  // would wait for the next pass's Q loads in flight.
  unsigned base = 0;
  asm volatile("" : "+v"(base));
  const int lane = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, base));
  asm volatile("" : "+v"(wave));
  bf16* const stage = stages + kStageElems * wave;
  // Likewise the gate is computed here from beta (a scalar register): a vector
  // copy kept from the kernel start is spilled, and its reload here would wait
  // for the next pass's Q loads in flight.
  beta = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, beta)));
  asm volatile("" : "+s"(beta));
  const float g = sigmoid_gate(beta);
  const int l32 = lane & 31, hi = lane >> 5;
  const float l_tot = X.l + __shfl_xor(X.l, 32);
  const float inv_l = 1.f / l_tot;
  if (lrow && hi == 0) lrow[l32] = X.m + __log2f(l_tot);   // the row's log-normaliser, when kept
  bf16x8 qp[D / 16];                   // q' = sigma(q) - 1 (bf16), the B operand of M^T q'
  bf16x8 ql[D / 16];                   // precise path: q' - qp (bf16)
  const bool precise = X.big;
  float den = 0.f;
  if (has_memory && precise) {
    float zpart = 0.f;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      const f32x4 z0 = *(const INFINI_LDS f32x4*)(zs + 16 * c + 8 * hi);
      const f32x4 z1 = *(const INFINI_LDS f32x4*)(zs + 16 * c + 8 * hi + 4);
      const bf16x8 qx = *reinterpret_cast<const bf16x8*>(qg + (int64_t)l32 * D + 16 * c + 8 * hi);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float x = bf2f(qx[i]);
        const float f = x > 0.f ? x : exp_e(x) - 1.f;
        const float zz = i < 4 ? z0[i] : z1[i - 4];
        den = __builtin_fmaf(f, zz, den);
        zpart += zz;
        qp[c][i] = f2bf(f);
        ql[c][i] = f2bf(f - bf2f(qp[c][i]));
      }
    }
    den += zpart;
    den += __shfl_xor(den, 32);
  } else if (has_memory) {
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      const f32x4 z0 = *(const INFINI_LDS f32x4*)(zs + 16 * c + 8 * hi);
      const f32x4 z1 = *(const INFINI_LDS f32x4*)(zs + 16 * c + 8 * hi + 4);
      // unpacked from the packed operand registers (opaque, so the compiler does
      // not keep separate unpacked copies of Q alive through the tile loop)
      u32x4 qw = __builtin_bit_cast(u32x4, X.q[c]);
      asm volatile("" : "+v"(qw));
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const unsigned wq = qw[i / 2];
        const float qs = __builtin_bit_cast(float, (i & 1) ? (wq & 0xffff0000u) : (wq << 16));
        const float x = qs * inv_sc;                    // q (the registers hold q * scale * log2 e)
        const float f = x > 0.f ? x : exp_e(x) - 1.f;   // q' = sigma(q) - 1
        const float zz = i < 4 ? z0[i] : z1[i - 4];
        den = __builtin_fmaf(f, zz, den);
        qp[c][i] = f2bf(f);
      }
    }
    den += __shfl_xor(den, 32);
    // sigma(q) . z = sum(z) + q' . z; sum(z) by a reduction over the wave
    float zsum = *(const INFINI_LDS float*)(zs + lane);
    if (D > 64) zsum += *(const INFINI_LDS float*)(zs + lane + 64);
    den += wave_sum(zsum);
  }
  // lane holds row l32 of the block, values d = 32db + 8j + 4hi + 0..3
  const float inv_den = (has_memory && den > 0.f) ? 1.f / den : 0.f;
  const float wg_mem = g * inv_den;
  const float wg_dot = (1.f - g) * inv_l;
  // The rows go out through LDS, 32 columns at a time: each lane writes its
  // 8-byte pieces of row l32 into a [32 x 32] stage (16-byte chunk k of row r at
  // chunk k ^ ((r / 4) % 4): the reads below are free of bank conflicts, the
  // writes conflict two ways), then reads back 16 bytes of row 16 i + lane / 4 so
  // that every global store writes whole 64-byte row segments.  The stage is
  // private to the wave, and LDS executes a wave's accesses in order, so no
  // barrier is needed.
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    f32x16 am;
    if (has_memory) {
      // accumulator starts at colsum(M)[d_value of each element]
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 c4 = *(const INFINI_LDS f32x4*)(cs + 32 * db + 8 * j + 4 * hi);
#pragma unroll
        for (int e = 0; e < 4; ++e) am[4 * j + e] = c4[e];
      }
      bf16x8 ma[D / 16];
#pragma unroll
      for (int c = 0; c < D / 16; ++c) ma[c] = lds_read8(mt + 32 * db * D + ad.kofs(c));
#pragma unroll
      for (int c = 0; c < D / 16; ++c) am = mfma32(ma[c], qp[c], am);
      if (precise) {
#pragma unroll
        for (int c = 0; c < D / 16; ++c) am = mfma32(ma[c], ql[c], am);
#pragma unroll
        for (int c = 0; c < D / 16; ++c) {
          const bf16x8 ml = *reinterpret_cast<const bf16x8*>(mlo + (int64_t)(32 * db + l32) * D + 16 * c + 8 * hi);
          am = mfma32(ml, qp[c], am);
        }
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) am[r] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x4 outv;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        outv[e] = f2bf(__builtin_fmaf(X.o[db][4 * j + e], wg_dot, am[4 * j + e] * wg_mem));
      const int chunk = j ^ ((l32 >> 2) & 3);
      *(INFINI_LDS bf16x4*)(stage + l32 * 32 + 8 * chunk + 4 * hi) = outv;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = 16 * i + (lane >> 2), c = lane & 3;
      const bf16x8 x = *(const INFINI_LDS bf16x8*)(stage + r * 32 + 8 * (c ^ ((r >> 2) & 3)));
      *reinterpret_cast<bf16x8*>(ob + (int64_t)r * D + 32 * db + 8 * c) = x;
    }
  }
}

// Per-workgroup context shared by both passes.
template <int D>
struct FaCtx {
  const bf16* qb;          // Q rows of this (b, h, segment)
  bf16* ob;
  const bf16* kseg;
  const bf16* vseg;
  const bf16* snapM;       // M^T snapshot of this (b, h, segment)
  const bf16* snapMlo;     // its bf16 remainder
  const float* snapz;
  const float* snapc;
  float* lb;               // the segment's log-normalisers, or null
  uint32_t seg_bytes;
  int N, nk, wave;
  bool has_memory;
  float beta, sc;
};

// Direct-to-LDS loads of the Q rows of query tile qt into slot 1: rows 0-127 of
// the tile into its K part, rows 128-255 into its V part, both in the K layout,
// so that a wave reads its 32 rows as it reads a 32-key block of K.  Rows past
// the segment end load zeros (their results are never used).
template <int D>
__device__ __forceinline__ void issue_q(const bf16* qb, int N, int wave, int qt, bf16* k1s, bf16* v1s,
                                        const DmaOfs<D>& dof) {
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int r = qt * kBM + half * kBN;
    const bool in = r < N;
    issue_tile<D, false>(qb + (in ? (int64_t)r * D : 0), in ? (uint32_t)(N - r) * D * 2 : 0u,
                         half ? v1s : k1s, wave, dof);
  }
}

// The pass after the current one: its query tile (qt < 0: none) and the Q rows
// and V tensor of its (b, h, segment), which may be another item's.
struct NextPass {
  const bf16* qb;
  const bf16* vseg;
  int qt;
};

// The load item after step t of a pass with nsteps steps: tile t+1 (zeros past
// the segment), or after the last step the snapshot of M^T (K part) together
// with the V part of the next pass's tile 0 (zeros when there is none).
template <int D>
__device__ __forceinline__ Prefetch<D> next_item(const FaCtx<D>& cx, int t, int nsteps, const NextPass& np,
                                                bf16* kn, bf16* vn, const DmaOfs<D>& dof) {
  Prefetch<D> pf;
  pf.kn = kn;
  pf.vn = vn;
  pf.wave = cx.wave;
  pf.dof = &dof;
  if (t + 1 < nsteps) {
    const uint32_t off = (uint32_t)(t + 1) * kBN * D * 2;   // byte offset of tile t+1
    const uint32_t left = off < cx.seg_bytes ? cx.seg_bytes - off : 0u;
    pf.kb = cx.kseg + (off < cx.seg_bytes ? off / 2 : 0u);
    pf.vb = cx.vseg + (off < cx.seg_bytes ? off / 2 : 0u);
    pf.kbytes = pf.vbytes = left;
  } else {
    pf.kb = cx.snapM;
    pf.kbytes = cx.has_memory ? (uint32_t)(D * D * 2) : 0u;
    pf.vb = np.qt >= 0 ? np.vseg : cx.vseg;
    pf.vbytes = np.qt >= 0 ? cx.seg_bytes : 0u;
  }
  return pf;
}

// One query tile (pass) of the workgroup.  Tile t of the pass sits in slot t % 2
// (k0s/v0s, k1s/v1s); every pass has an even number of steps, so the last one
// uses slot 1 and brings the snapshot of M^T into k0s (with z and colsum into
// zc) and, with a next pass (np.qt >= 0, of this or another (b, h, segment)),
// the V part of its tile 0 into v0s; the Q rows of that pass go into slot 1
// during the epilogue.  On entry tile 0 is in slot 0 and the pass's Q rows in
// slot 1 (waited for and synchronised).
template <int D>
__device__ __forceinline__ void run_pass(const FaCtx<D>& cx, int qt, const NextPass& np, bf16* k0s, bf16* v0s,
                                         bf16* k1s, bf16* v1s, float* zc, bf16* stg, const LdsAddr<D>& ad,
                                         const DmaOfs<D>& dof) {
  const bool next = np.qt >= 0;
  const int q0 = qt * kBM;
  const int r0 = q0 + 32 * cx.wave;          // first row of this wave's query block
  const bool act = r0 < cx.N;
  const int last = min(cx.nk - 1, (q0 + kBM - 1) / kBN);
  const int nsteps = (last + 2) & ~1;        // even: pads with a tile beyond the segment

  QBlock<D> X;
  // Q^T * scale * log2 e (rounded to bf16): the scores come out in the log2 domain
  {
    const bf16* qs = (cx.wave < 4 ? k1s : v1s) + 32 * (cx.wave & 3) * D;
    bf16x8 qr[D / 16];
#pragma unroll
    for (int c = 0; c < D / 16; ++c) qr[c] = lds_read8(qs + ad.kofs(c));
    bool big = false;
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float x = bf2f(qr[c][i]);
        X.q[c][i] = f2bf(x * cx.sc);
        big |= fabsf(x) > kPreciseQ;
      }
    X.big = __any(big) != 0;
  }
  // every wave has its Q rows before step 0 loads tile 1 into slot 1
  wait_lds_and_sync();
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) X.o[db][r] = 0.f;
  set_m(X, 0.f);
  X.l = 0.f;
  X.bad = false;
  if (act) init_m<D>(X, k0s, ad, r0);

  // Step t uses slot t % 2 and loads item t+1 into the other slot.
#define INFINI_FA_STEP(T, KC, VC, KN, VN)                                                        \
  {                                                                                              \
    const int t_ = (T);                                                                          \
    const Prefetch<D> pf_ = next_item<D>(cx, t_, nsteps, np, KN, VN, dof);                     \
    if (t_ + 1 == nsteps && cx.has_memory && cx.wave == 0) {                                     \
      issue_row(cx.snapz, D * 4, zc);                                                            \
      issue_row(cx.snapc, D * 4, zc + 256);                                                      \
    }                                                                                            \
    const int k0_ = t_ * kBN;                                                                    \
    if (act && k0_ + kBN <= r0)                                                                  \
      tile_pipe<D, false>(X, KC, VC, ad, pf_, k0_, r0);                                          \
    else if (act && k0_ <= r0 && r0 < k0_ + kBN)                                                 \
      tile_pipe<D, true>(X, KC, VC, ad, pf_, k0_, r0);                                           \
    else                                                                                         \
      pf_.template issue<FaLayout<D>::NI>(0);                                                    \
    wait_loads_and_sync();                                                                       \
  }
  for (int t = 0; t < nsteps; t += 2) {
    INFINI_FA_STEP(t, k0s, v0s, k1s, v1s)
    INFINI_FA_STEP(t + 1, k1s, v1s, k0s, v0s)
  }
#undef INFINI_FA_STEP

  // slot 1 is free after the last step: the next pass's Q rows load during the
  // epilogue
  if (next) issue_q<D>(np.qb, cx.N, cx.wave, np.qt, k1s, v1s, dof);
  if (act && __any(X.bad)) recompute_block<D>(X, r0, cx.kseg, cx.vseg);

  if (act) finish_block<D>(X, k0s, zc, zc + 256, ad, cx.has_memory, cx.beta, 1.f / cx.sc, cx.ob + (int64_t)r0 * D,
                           stg, cx.wave, cx.qb + (int64_t)r0 * D, cx.snapMlo, cx.lb ? cx.lb + r0 : nullptr);
  // the snapshot in k0s is no longer read (the output stores stay in flight)
  if (next) wait_lds_and_sync();
}

// First token (in units of rows of q, k, v, out) of the (b, h, segment) of item it.
__device__ __forceinline__ int64_t item_tok0(const FaArgs& a, int it, int npair, int sn) {
  const int shl = it / npair;
  const int bh = shl / sn;
  const int s = a.s0 + shl % sn;
  return (int64_t)bh * a.L + (int64_t)s * a.N;
}

// Context of the (b, h, segment) of item it.
template <int D>
__device__ __forceinline__ FaCtx<D> item_ctx(const FaArgs& a, int it, int npair, int sn, int wave) {
  const int shl = it / npair;
  const int bh = shl / sn;
  const int s = a.s0 + shl % sn;
  const int sh = bh * a.S + s;           // (b*H + h) * S + s
  const int h = bh % a.H;
  const int64_t tok0 = (int64_t)bh * a.L + (int64_t)s * a.N;
  FaCtx<D> cx;
  cx.qb = a.q + tok0 * D;
  cx.ob = a.out + tok0 * D;
  cx.kseg = a.k + tok0 * D;
  cx.vseg = a.v + tok0 * D;
  cx.snapM = a.snapM + (int64_t)sh * D * D;
  cx.snapMlo = a.snapMlo + (int64_t)sh * D * D;
  cx.snapz = a.snapz + (int64_t)sh * D;
  cx.snapc = a.snapc + (int64_t)sh * D;
  cx.lb = a.lse ? a.lse + tok0 : nullptr;
  cx.seg_bytes = (uint32_t)a.N * D * 2;
  cx.N = a.N;
  cx.nk = (a.N + kBN - 1) / kBN;
  cx.wave = wave;
  cx.has_memory = (a.seg_base + s) > 0;
  cx.beta = a.beta[h];
  cx.sc = a.sc_log2;
  return cx;
}

template <int D>
__global__ __launch_bounds__(kThreads, 1)
void fa_fwd_kernel(FaArgs a) {
  using L = FaLayout<D>;
  __shared__ __attribute__((aligned(1024))) bf16 k0s[L::TILE_ELEMS];
  __shared__ __attribute__((aligned(1024))) bf16 v0s[L::TILE_ELEMS];
  __shared__ __attribute__((aligned(1024))) bf16 k1s[L::TILE_ELEMS];
  __shared__ __attribute__((aligned(1024))) bf16 v1s[L::TILE_ELEMS];
  __shared__ __attribute__((aligned(1024))) float zc[512];   // z at [0, D), colsum(M) at [256, 256 + D)
  __shared__ __attribute__((aligned(1024))) bf16 stg[kWaves * kStageElems];   // output stages

  // Items: (b, h, segment) tile x pair of query tiles, the pair fastest.  With G
  // workgroups (G a multiple of the 8 XCDs), XCD x (hardware id % 8) owns the
  // items [x n / 8, (x + 1) n / 8) and its G / 8 workgroups take them in turn, so
  // the workgroups of one XCD work on consecutive items (the pairs of a segment
  // together, sharing its K/V tiles in that XCD's L2).  With G = n each workgroup
  // does one item; with G = the number of compute units the kernel is persistent
  // and the next item's Q rows and tile 0 load during the current epilogue.
  const int npair = (a.nq + 1) / 2;
  const int sn = a.sn > 0 ? a.sn : a.S;  // the launch covers segments s0 .. s0 + sn - 1 of every head
  const int nitems = a.B * a.H * sn * npair;
  const int G = gridDim.x, g = blockIdx.x;
  int it, it_end, it_step;
  if (G % 8 == 0) {
    const int x = g % 8;
    it = (int)((int64_t)x * nitems / 8) + g / 8;
    it_end = (int)((int64_t)(x + 1) * nitems / 8);
    it_step = G / 8;
  } else {
    it = g;
    it_end = nitems;
    it_step = G;
  }
  if (it >= it_end) return;   // uniform over the workgroup, before any barrier

  const int wave = threadIdx.x >> 6;
  FaCtx<D> cx = item_ctx<D>(a, it, npair, sn, wave);
  LdsAddr<D> ad;
  ad.init(threadIdx.x & 63);
  DmaOfs<D> dof;
  dof.init(threadIdx.x & 63);

  // the longer query tile first: the workgroups of one (b, h, segment) then
  // stream the same K/V tiles at about the same time (L2 reuse)
  int pair = it % npair;
  issue_tile<D, false>(cx.kseg, cx.seg_bytes, k0s, wave, dof);
  issue_tile<D, true>(cx.vseg, cx.seg_bytes, v0s, wave, dof);
  issue_q<D>(cx.qb, cx.N, wave, a.nq - 1 - pair, k1s, v1s, dof);
  wait_loads_and_sync();
  // One copy of the pass code serves every pass (the loop is not unrolled).
  // Between passes, the K part of the next pass's tile 0 goes into k0s (free
  // once the snapshot has been used); its V part is already in v0s and its Q
  // rows in slot 1.
  bool second = false;
#pragma unroll 1
  for (;;) {
    const int qt = second ? pair : a.nq - 1 - pair;
    const bool same_item = !second && pair != a.nq - 1 - pair;   // the pair's second tile follows
    NextPass np;
    if (same_item) {
      np.qb = cx.qb;
      np.vseg = cx.vseg;
      np.qt = pair;
    } else if (it + it_step < it_end) {
      const int64_t t0 = item_tok0(a, it + it_step, npair, sn);
      np.qb = a.q + t0 * D;
      np.vseg = a.v + t0 * D;
      np.qt = a.nq - 1 - (it + it_step) % npair;
    } else {
      np.qb = cx.qb;
      np.vseg = cx.vseg;
      np.qt = -1;
    }
    run_pass<D>(cx, qt, np, k0s, v0s, k1s, v1s, zc, stg, ad, dof);
    if (np.qt < 0) break;
    if (same_item) {
      second = true;
    } else {
      it += it_step;
      pair = it % npair;
      second = false;
      cx = item_ctx<D>(a, it, npair, sn, wave);
    }
    issue_tile<D, false>(cx.kseg, cx.seg_bytes, k0s, wave, dof);
    wait_loads_and_sync();
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
  const int sn = a.sn > 0 ? a.sn : a.S;
  if (a.s0 < 0 || a.s0 + sn > a.S) return hipErrorInvalidValue;
  const int64_t blocks = fa_fwd_blocks((int64_t)a.B * a.H * sn, a.N);
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  // A launch over whole streams runs persistent, one workgroup per compute unit
  // (the kernel's LDS admits one per CU).  A launch over a range of segments
  // runs one workgroup per item: it shares the device with the delta chain,
  // which holds some CUs, and a persistent grid would leave the share of the
  // workgroups waiting for those CUs to the end.
  int64_t grid = blocks;
  if (args.sn <= 0) {
    const int cus = device_compute_units();
    const int64_t slots = cus >= 8 ? cus / 8 * 8 : cus;
    if (slots > 0 && grid > slots) grid = slots;
  }
  hipLaunchKernelGGL(fa_fwd_kernel<D>, dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template hipError_t launch_fa_fwd<64>(const FaArgs&, hipStream_t);
template hipError_t launch_fa_fwd<128>(const FaArgs&, hipStream_t);

}  // namespace infini
