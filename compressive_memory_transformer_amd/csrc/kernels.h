// Internal launcher interface between the C ABI host code and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace infini {

typedef __bf16 bf16;

// ------------------------------------------------------------------ bf16 path
// Tensors cover S segments of N tokens for each of B*H heads; token t of head
// bh lives at row bh * L + t, L = S * N.
struct FaArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const float* beta;     // [H]
  const bf16* snapM;     // [B*H*S][D][D] bf16 snapshot of M_{s-1}^T (row = d_value)
  const bf16* snapMlo;   // [B*H*S][D][D] bf16 remainder: M^T = snapM + snapMlo to ~16 bits
  const float* snapz;    // [B*H*S][D]    fp32 snapshot of z_{s-1}
  const float* snapc;    // [B*H*S][D]    fp32 column sums of M_{s-1} over d_key
  bf16* out;
  int B, H, S, N;
  int64_t L;
  int nq;                // query tiles per segment (set by the launcher)
  int64_t seg_base;      // segments folded into the state before this call
  float sc_log2;         // softmax scale * log2(e)
  float* lse;            // [B*H*L] or null: log2 of each query row's local softmax denominator
                         // over the base-2 scores sc_log2 q.k (reference maximum included)
  int s0, sn;            // segments s0 .. s0 + sn - 1 of every head (sn = 0: all S)
};
template <int D> hipError_t launch_fa_fwd(const FaArgs& a, hipStream_t stream);
// Workgroups of one fused-kernel launch over seg_heads (b, h, segment) tiles.
int64_t fa_fwd_blocks(int64_t seg_heads, int N);

// Linear rule, phase 1: per-segment contributions C_s^T = V^T sigma(K) (fp32, row =
// d_value) and c_s = sum_t sigma(K_t).
struct LinContribArgs {
  const bf16* k;
  const bf16* v;
  float* cM;             // [B*H*S][D][D]
  float* cz;             // [B*H*S][D]
  int B, H, S, N;
  int64_t L;
};
template <int D> hipError_t launch_lin_contrib(const LinContribArgs& a, hipStream_t stream);

// Linear rule, phase 2: exclusive prefix over segments.  Writes the snapshots
// read by the fused kernel and leaves M_S, z_S in the state.
struct LinScanArgs {
  const float* cM;
  const float* cz;
  float* M;              // state [B*H][D][D] (row = d_key), read then overwritten
  float* z;              // state [B*H][D]
  bf16* snapM;           // [B*H*S][D][D] (row = d_value)
  bf16* snapMlo;         // [B*H*S][D][D] remainder M^T - snapM in bf16
  float* snapz;          // [B*H*S][D]
  float* snapc;          // [B*H*S][D] column sums of M over d_key
  int BH, S;
};
template <int D> hipError_t launch_lin_scan(const LinScanArgs& a, hipStream_t stream);

// Delta rule as the matrix recurrence M_s = M_{s-1} + C_s - A_s M_{s-1} with
// C_s = sigma(K)^T V and A_s = sigma(K)^T diag(w) sigma(K), w_t = 1 / (sigma(K_t) .
// z_{s-1}) (0 in a stream's first segment): C_s, c_s (the linear rule's
// contribution kernel), the z snapshots (a prefix scan) and A_s (MFMA) for all
// segments in parallel, then the chain over the S segments of each head, one
// workgroup per 16 columns of M.  Emits the snapshots and updates the state.
struct DeltaArgs {
  const bf16* k;
  const bf16* v;
  float* M;              // state [B*H][D][D] (row = d_key)
  float* z;              // state [B*H][D]
  bf16* snapM;           // [B*H*S][D][D] (row = d_value)
  bf16* snapMlo;         // [B*H*S][D][D] remainder M^T - snapM in bf16
  float* snapz;          // [B*H*S][D]
  float* snapc;          // [B*H*S][D]
  float* cM;             // workspace [B*H*S][D][D]: C_s^T (row = d_value)
  float* cz;             // workspace [B*H*S][D]: c_s
  bf16* amat;            // workspace [B*H*S][2][D][D]: A_s as bf16 hi, then lo
  int BH, S, N;
  int64_t L;
  int64_t seg_base;
  int s0, sn;            // the chain's segments s0 .. s0 + sn - 1 (sn = 0: all S), from M, z
};
// The whole state stage: launch_delta_prep, then the chain over every segment.
template <int D> hipError_t launch_delta_state(const DeltaArgs& a, hipStream_t stream);
// Its parallel part: C_s, c_s, the z prefix (snapshots of z) and A_s of every segment.
template <int D> hipError_t launch_delta_prep(const DeltaArgs& a, hipStream_t stream);
// Its sequential part over a.s0 .. a.s0 + a.sn - 1 (after launch_delta_prep): from
// the state M (M_{s0-1}), the snapshots of M_{s-1} for those segments; the state
// ends as M_{s0+sn-1}.  Consecutive ranges on one stream chain exactly.
template <int D> hipError_t launch_delta_chain(const DeltaArgs& a, hipStream_t stream);

// ------------------------------------------------------------------ VALU path
// fp32 states and the bf16 shapes without MFMA kernels.  One segment per launch;
// M and z are read as M_{s-1}, z_{s-1}.  q, k, v, out in the state's dtype (bf16
// when the flag is set, else fp32).
struct F32AttnArgs {
  const void* q;         // rows of this segment: q + (bh * L + seg_off) * dk
  const void* k;
  const void* v;
  const float* beta;
  const float* M;        // [BH][dk][dv]
  const float* z;        // [BH][dk]
  void* out;
  int H, BH, N, dk, dv;
  int64_t L, seg_off;
  int has_memory;
  float scale;
  int bf16;
};
hipError_t launch_f32_attn(const F32AttnArgs& a, hipStream_t stream);

struct F32UpdateArgs {
  const void* k;
  const void* v;
  float* M;
  float* z;
  float* U;              // workspace [BH][N][dv] (delta rule)
  int BH, N, dk, dv;
  int64_t L, seg_off;
  int delta, has_memory;
  int bf16;
};
hipError_t launch_f32_update(const F32UpdateArgs& a, hipStream_t stream);

// ------------------------------------------------------------ open segment
// Queries j < m that arrive at positions pos0 + j of an open segment whose
// earlier keys and values (rows bh * N + t, t < pos0) are in kseg / vseg; the new
// ones are knew / vnew, row bh * q_stride + j like the queries and outputs, and
// are copied into the open segment (kseg_out / vseg_out, the same buffers) by the
// second kernel.  The memory (M, z) is read as it stands.  part: workspace
// [BH][m][P + R][dv + 2] (P key partitions and R memory slots, set by the
// launcher).
struct OpenAttnArgs {
  const void* q;
  const void* knew;
  const void* vnew;
  const void* kseg;
  const void* vseg;
  void* kseg_out;
  void* vseg_out;
  const float* beta;
  const float* M;
  const float* z;
  void* out;
  float* part;
  int BH, H, N, dk, dv, m, pos0, P, R;
  int64_t q_stride;
  int has_memory, bf16;
  float scale;
};
hipError_t launch_open_attn(const OpenAttnArgs& a, hipStream_t stream);
// Workspace slots (key partitions plus memory slots) per query of the
// open-segment attention for `keys` keys and d_key = dk.
int open_attn_slots(int keys, int dk);

// ------------------------------------------------------------------ backward
// Gradients of forward_sequence for the loss <dA, A> + <dM, M_S> + <dz, z_S>.
// q, k, v, dout, dq, dk, dv in the I/O dtype; everything else fp32.  Workspace
// arrays (row = bh * L + t, segment index = bh * S + s):
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  const float* beta;     // [H]
  const float* M0;       // [BH][dk][dv] state before the stream
  const float* z0;       // [BH][dk]
  const float* dM;       // [BH][dk][dv] gradient of M_S, or null (zero)
  const float* dz;       // [BH][dk] or null
  void* dq_out;
  void* dk_out;
  void* dv_out;
  float* dbeta;          // [H]
  float* dM0;            // [BH][dk][dv] or null
  float* dz0;            // [BH][dk] or null
  float* snapM;          // [BH*S][dk][dv] M_{s-1}
  float* snapz;          // [BH*S][dk]
  float* dMr;            // [BH*S][dk][dv] retrieval's gradient of M_{s-1}
  float* dzr;            // [BH*S][dk]
  float* ez;             // [BH*S][dk]
  float* gzs;            // [BH*S][dk] dL/dz_s
  float* lse;            // [BH*L] softmax log-normaliser of each row (natural log on the VALU
                         // path, base 2 on the MFMA path; the forward's, read only, when out_fw is set)
  float* drow;           // [BH*L] <(1 - g) dA, A_dot>
  float* rs;             // [BH*L] g / den (0 without memory)
  float* dden;           // [BH*L]
  float* de;             // [BH*L] delta rule: gradient of sigma(K_t) . z_{s-1}
  float* dq_acc;         // [BH*L][dk] (null on the MFMA path: its query kernel writes dq_out whole)
  float* dk_acc;         // [BH*L][dk] local attention's dk
  float* dv_acc;         // [BH*L][dv] (MFMA path: local attention's; the update kernels write dv_out)
  float* dfk_acc;        // [BH*L][dk] update's d sigma(K) (unused by the linear rule's MFMA path)
  float* dbeta_part;     // [BH*S][nqb]
  float* Amat;           // delta rule, bf16 path: [BH*S][dk][dk] sigma(K)^T diag(1/e) sigma(K)
  float* gpart;          // bf16 MFMA path: [BH*S][dk][dv] + [BH*S][dk], the Gram kernels' second halves
  const void* out_fw;    // bf16 MFMA path, or null: the forward's output A [BH*L][dv], with its
                         // log-normalisers in lse (the softmax statistics are then not recomputed)
  int B, H, BH, N, S, dk, dv, nqb;
  int64_t L, seg_base;
  int delta;
  float scale;
};
hipError_t launch_backward(const BwdArgs& a, bool bf16_io, hipStream_t stream);
// Query blocks per segment of the backward (the dbeta_part width).
int bwd_query_blocks(int N);
// bf16 path: the local attention's and the retrieval's dq (with the softmax
// statistics, D, rs, dden of every row and the dbeta shares) and the local
// attention's dk, dv on the MFMA units; N a multiple of 64.
template <int D> hipError_t launch_backward_attention_mfma(const BwdArgs& a, hipStream_t stream);
// bf16 path, linear rule: the update's dv and d sigma(K) on the MFMA units.
template <int D> hipError_t launch_backward_lin_update_mfma(const BwdArgs& a, hipStream_t stream);
// bf16 path, delta rule: A_s per segment, and (after the chains) the update's dv,
// d sigma(K) and the denominators' gradients de on the MFMA units.
template <int D> hipError_t launch_backward_delta_amat_mfma(const BwdArgs& a, hipStream_t stream);
// bf16 path: the retrieval's gradients dMr, dzr of every segment on the MFMA units.
template <int D> hipError_t launch_backward_retrieval_grad_mfma(const BwdArgs& a, hipStream_t stream);
template <int D> hipError_t launch_backward_delta_update_mfma(const BwdArgs& a, hipStream_t stream);

// ----------------------------------------------------- kernel linear attention
// Causal kernel linear attention over chunks of N tokens, given every chunk's
// starting state in snapM / snapz / snapc (the linear-rule state kernels' output);
// beta, nq, seg_base and sc_log2 of FaArgs are not used.  N a multiple of 64.
template <int D> hipError_t launch_kla(const FaArgs& a, hipStream_t stream);

// ---------------------------------------------------------------- projections
// C = A B in bf16 with fp32 accumulation; B row-major [K][N].  a_heads: A is the
// heads' outputs [B, H, L, dv] read as [B L, H dv] (K = H dv); else row-major
// [M][K].  c_heads: column n of C goes to q (n < H dk), k (n < 2 H dk) or v,
// each [B, H, L, d]; else C is row-major [M][N].  K a multiple of 64, N of 8.
struct GemmArgs {
  const bf16* a;
  const bf16* b;
  bf16* c;
  bf16* q;
  bf16* k;
  bf16* v;
  int M, N, K;
  int a_heads, c_heads;
  int L, H, dk, dv;
};
hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t stream);

// Compute units of the current device (looked up once per device).
int device_compute_units();

// Zero n floats at p and n2 floats at p2 (one launch).
hipError_t launch_fill_zero(float* p, int64_t n, float* p2, int64_t n2, hipStream_t stream);

}  // namespace infini
