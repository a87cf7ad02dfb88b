// C ABI of the Infini-attention segment forward (declared in include/infini_attn.h).
//
// Host side only: argument validation (always before the first HIP call),
// workspace carving, and the launch sequence on the caller's stream.
//
//   bf16, linear: lin_contrib (all segments in parallel) -> lin_scan (snapshots
//                 M_{s-1}, z_{s-1} and the final state) -> fused attention kernel
//   bf16, delta : delta_chain (persistent, sequential over segments, snapshots and
//                 the final state) -> fused attention kernel
//   fp32        : per segment, attention (reads M_{s-1}, z_{s-1}) then update
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <utility>

#include "../../include/infini_attn.h"
#include "kernels.h"

namespace {

thread_local std::string g_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_error = buf;
  return code;
}

int ok() {
  g_error.clear();
  return INFINI_OK;
}

constexpr int64_t kMaxElems = (int64_t)1 << 60;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > kMaxElems / a) return false;
  *out = a * b;
  return true;
}

// Shapes the MFMA kernels take (bf16 only); every other supported shape runs the
// VALU path.
bool mfma_shape(int32_t dk, int32_t dv, int32_t N) { return dk == dv && (dk == 64 || dk == 128) && N % 64 == 0; }

bool mfma_path(const infini_attn_state* st) {
  return st->dtype == INFINI_BF16 && mfma_shape(st->d_key, st->d_value, st->segment_len);
}

// Validates a configuration; returns INFINI_OK or an error code with the message set.
int check_config(int32_t B, int32_t H, int32_t dk, int32_t dv, int32_t N, int32_t dtype, int32_t rule,
                 float scale) {
  if (B <= 0 || H <= 0 || dk <= 0 || dv <= 0 || N <= 0)
    return fail(INFINI_EINVAL, "batch, heads, d_key, d_value and segment_len must be positive "
                               "(got %d, %d, %d, %d, %d)", B, H, dk, dv, N);
  if (dtype != INFINI_F32 && dtype != INFINI_BF16) return fail(INFINI_EINVAL, "unknown dtype %d", dtype);
  if (rule != INFINI_RULE_LINEAR && rule != INFINI_RULE_DELTA) return fail(INFINI_EINVAL, "unknown rule %d", rule);
  if (std::isinf(scale)) return fail(INFINI_EINVAL, "scale must be finite");
  int64_t t;
  if (!mul_ok((int64_t)B * H, (int64_t)dk * dv, &t)) return fail(INFINI_EINVAL, "state too large");
  if (dtype == INFINI_BF16 && mfma_shape(dk, dv, N)) return INFINI_OK;
  // the VALU path (fp32, and bf16 shapes the MFMA kernels do not take)
  if (dk > 128 || dv > 128)
    return fail(INFINI_EUNSUPPORTED, "d_key and d_value must be <= 128 (got %d, %d)", dk, dv);
  if (N > 4096)
    return fail(INFINI_EUNSUPPORTED, "segment_len must be <= 4096 (got %d) unless the state is bf16 with "
                                     "d_key == d_value in {64, 128} and segment_len a multiple of 64", N);
  return INFINI_OK;
}

int check_state(const infini_attn_state* st) {
  if (!st) return fail(INFINI_EINVAL, "state pointer is NULL");
  int rc = check_config(st->batch, st->heads, st->d_key, st->d_value, st->segment_len, st->dtype, st->rule,
                        st->scale);
  if (rc != INFINI_OK) return rc;
  if (!(st->scale > 0.f)) return fail(INFINI_EINVAL, "state scale must be positive (state not initialised?)");
  if (!st->M || !st->z) return fail(INFINI_EINVAL, "state M or z is NULL");
  if (st->segments_done < 0) return fail(INFINI_EINVAL, "negative segments_done");
  return INFINI_OK;
}

struct WsLayout {
  size_t snapM = 0, snapMlo = 0, snapz = 0, snapc = 0, cM = 0, cz = 0, amat = 0, U = 0, total = 0;
};

// Workspace regions for S segments whose tokens sit at a row stride of L per
// (b, h) (L = S * N for a whole stream), each 256-byte aligned.  Returns false on
// overflow.
bool workspace_layout(const infini_attn_state* st, int64_t S, int64_t L, WsLayout* w) {
  const int64_t BH = (int64_t)st->batch * st->heads;
  int64_t seg_heads, n;
  if (!mul_ok(BH, S, &seg_heads)) return false;
  size_t off = 0;
  if (mfma_path(st)) {
    const int64_t D = st->d_key;
    if (!mul_ok(seg_heads, D * D, &n)) return false;
    w->snapM = off; off = align_up(off + (size_t)n * 2);
    w->snapMlo = off; off = align_up(off + (size_t)n * 2);
    w->snapz = off; off = align_up(off + (size_t)(seg_heads * D) * 4);
    w->snapc = off; off = align_up(off + (size_t)(seg_heads * D) * 4);
    // both rules: the per-segment contributions C_s^T and c_s
    w->cM = off; off = align_up(off + (size_t)n * 4);
    w->cz = off; off = align_up(off + (size_t)(seg_heads * D) * 4);
    // delta rule: A_s per segment as two bf16 parts
    if (st->rule == INFINI_RULE_DELTA) { w->amat = off; off = align_up(off + (size_t)n * 4); }
    (void)L;
  } else if (st->rule == INFINI_RULE_DELTA) {
    if (!mul_ok(BH, (int64_t)st->segment_len * st->d_value, &n)) return false;
    w->U = off; off = align_up(off + (size_t)n * 4);
  }
  w->total = off < kAlign ? kAlign : off;
  return true;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const char* x = static_cast<const char*>(a);
  const char* y = static_cast<const char*>(b);
  return x < y + nb && y < x + na;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(INFINI_EHIP, "%s: %s", what, hipGetErrorString(e));
}

int record(void* const* events, int i, hipStream_t stream) {
  if (!events) return INFINI_OK;
  hipError_t e = hipEventRecord(static_cast<hipEvent_t>(events[i]), stream);
  return e == hipSuccess ? INFINI_OK : hip_fail(e, "hipEventRecord");
}

// ------------------------------------------------------------------ delta pipeline
// The delta rule's chain is sequential over the segments and keeps few CUs busy.
// On the pipelined path it runs on a side stream in kPipeChunks ranges of
// segments, and the fused attention of each range follows on the caller's stream
// once that range is chained, beside the chain of the later ranges.  One side
// stream (default priority) and kPipeChunks + 1 events per device, created on
// first use and kept until the process ends; a call's records and waits are
// enqueued under g_pipe_mu so that calls from several host threads do not
// interleave them (a wait binds to the event's latest record when it is enqueued).
constexpr int kPipeChunks = 8;
constexpr int kPipeDevices = 64;
struct Pipe {
  hipStream_t side = nullptr;
  hipEvent_t ev[kPipeChunks + 1] = {};
  bool ready = false;
  int cus = 0;   // compute units of the device
};
std::mutex g_pipe_mu;
Pipe g_pipe[kPipeDevices];

// The current device's entry (g_pipe_mu held), with its compute-unit count.
int pipe_device(Pipe** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kPipeDevices) return fail(INFINI_EUNSUPPORTED, "device index %d out of range", dev);
  Pipe& p = g_pipe[dev];
  if (p.cus <= 0 && (e = hipDeviceGetAttribute(&p.cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) {
    p.cus = 0;
    return hip_fail(e, "hipDeviceGetAttribute");
  }
  *out = &p;
  return INFINI_OK;
}

// Number of ranges for the pipelined delta path, or 0 when it does not pay: the
// chain's workgroups must leave at least half of the compute units to the fused
// kernel (they hold whole CUs), and each range's fused launch must still fill
// the device twice over.
int pipe_ranges(const Pipe& p, int64_t chain_wgs, int64_t fa_wgs_total, int S) {
  if (p.cus <= 0 || 2 * chain_wgs > p.cus) return 0;
  const int64_t by_fill = fa_wgs_total / (2 * (int64_t)p.cus);
  const int nc = (int)std::min<int64_t>(std::min<int64_t>(kPipeChunks, S), by_fill);
  return nc >= 2 ? nc : 0;
}

// Creates the device's side stream and events on first use (g_pipe_mu held).
int pipe_ready(Pipe& p) {
  hipError_t e;
  if (!p.ready) {
    if (!p.side && (e = hipStreamCreateWithFlags(&p.side, hipStreamNonBlocking)) != hipSuccess) {
      p.side = nullptr;
      return hip_fail(e, "hipStreamCreateWithFlags");
    }
    for (hipEvent_t& ev : p.ev)
      if (!ev && (e = hipEventCreateWithFlags(&ev, hipEventDisableTiming)) != hipSuccess) {
        ev = nullptr;
        return hip_fail(e, "hipEventCreateWithFlags");
      }
    p.ready = true;
  }
  return INFINI_OK;
}

template <int D>
int run_bf16(infini_attn_state* st, const void* q, const void* k, const void* v, int64_t L, int S,
             const float* beta, void* out, char* ws, const WsLayout& w, hipStream_t stream,
             void* const* events, float* lse = nullptr, bool pipeline = false) {
  int rc;
  if ((rc = record(events, 0, stream)) != INFINI_OK) return rc;
  using infini::bf16;
  const int B = st->batch, H = st->heads, N = st->segment_len;
  bf16* snapM = reinterpret_cast<bf16*>(ws + w.snapM);
  bf16* snapMlo = reinterpret_cast<bf16*>(ws + w.snapMlo);
  float* snapz = reinterpret_cast<float*>(ws + w.snapz);
  float* snapc = reinterpret_cast<float*>(ws + w.snapc);
  hipError_t e;
  if (st->rule == INFINI_RULE_LINEAR) {
    infini::LinContribArgs c{static_cast<const bf16*>(k), static_cast<const bf16*>(v),
                             reinterpret_cast<float*>(ws + w.cM), reinterpret_cast<float*>(ws + w.cz),
                             B, H, S, N, L};
    if ((e = infini::launch_lin_contrib<D>(c, stream)) != hipSuccess) return hip_fail(e, "lin_contrib launch");
    infini::LinScanArgs sarg{c.cM, c.cz, st->M, st->z, snapM, snapMlo, snapz, snapc, B * H, S};
    if ((e = infini::launch_lin_scan<D>(sarg, stream)) != hipSuccess) return hip_fail(e, "lin_scan launch");
  } else {
    infini::DeltaArgs d{static_cast<const bf16*>(k), static_cast<const bf16*>(v), st->M, st->z, snapM, snapMlo,
                        snapz, snapc, reinterpret_cast<float*>(ws + w.cM), reinterpret_cast<float*>(ws + w.cz),
                        reinterpret_cast<bf16*>(ws + w.amat), B * H, S, N, L, st->segments_done};
    // the pipelined path where it pays (the lock is held while its launches are enqueued)
    std::unique_lock<std::mutex> lock(g_pipe_mu, std::defer_lock);
    Pipe* pp = nullptr;
    int nc = 0;
    if (pipeline && !events && S >= 2) {
      lock.lock();
      if ((rc = pipe_device(&pp)) != INFINI_OK) return rc;
      nc = pipe_ranges(*pp, (int64_t)B * H * (D / 16), infini::fa_fwd_blocks((int64_t)B * H * S, N), S);
      if (nc == 0) lock.unlock();
    }
    if (nc > 0) {
      infini::FaArgs f{static_cast<const bf16*>(q), static_cast<const bf16*>(k), static_cast<const bf16*>(v), beta,
                       snapM, snapMlo, snapz, snapc, static_cast<bf16*>(out), B, H, S, N, L, 0,
                       st->segments_done, (float)((double)st->scale * 1.4426950408889634), lse};
      if ((rc = pipe_ready(*pp)) != INFINI_OK) return rc;
      if ((e = infini::launch_delta_prep<D>(d, stream)) != hipSuccess) return hip_fail(e, "delta state launch");
      if ((e = hipEventRecord(pp->ev[0], stream)) != hipSuccess) return hip_fail(e, "hipEventRecord");
      if ((e = hipStreamWaitEvent(pp->side, pp->ev[0], 0)) != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
      const int per = (S + nc - 1) / nc;
      for (int c = 0; c < nc && c * per < S; ++c) {
        d.s0 = c * per;
        d.sn = std::min(per, S - d.s0);
        if ((e = infini::launch_delta_chain<D>(d, pp->side)) != hipSuccess) return hip_fail(e, "delta chain launch");
        if ((e = hipEventRecord(pp->ev[1 + c], pp->side)) != hipSuccess) return hip_fail(e, "hipEventRecord");
      }
      for (int c = 0; c < nc && c * per < S; ++c) {
        if ((e = hipStreamWaitEvent(stream, pp->ev[1 + c], 0)) != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
        f.s0 = c * per;
        f.sn = std::min(per, S - f.s0);
        if ((e = infini::launch_fa_fwd<D>(f, stream)) != hipSuccess) return hip_fail(e, "fa_fwd launch");
      }
      return INFINI_OK;
    }
    if ((e = infini::launch_delta_state<D>(d, stream)) != hipSuccess) return hip_fail(e, "delta state launch");
  }
  if ((rc = record(events, 1, stream)) != INFINI_OK) return rc;
  infini::FaArgs f{static_cast<const bf16*>(q), static_cast<const bf16*>(k), static_cast<const bf16*>(v), beta,
                   snapM, snapMlo, snapz, snapc, static_cast<bf16*>(out), B, H, S, N, L, 0,
                   st->segments_done, (float)((double)st->scale * 1.4426950408889634), lse};
  if ((e = infini::launch_fa_fwd<D>(f, stream)) != hipSuccess) return hip_fail(e, "fa_fwd launch");
  return record(events, 2, stream);
}

int run_f32(infini_attn_state* st, const void* q, const void* k, const void* v, int64_t L, int S,
            const float* beta, void* out, char* ws, const WsLayout& w, hipStream_t stream,
            void* const* events) {
  const int BH = st->batch * st->heads, N = st->segment_len;
  int rc;
  if ((rc = record(events, 0, stream)) != INFINI_OK) return rc;
  for (int s = 0; s < S; ++s) {
    const int64_t off = (int64_t)s * N;
    const int has_memory = (st->segments_done + s) > 0;
    infini::F32AttnArgs a{q, k, v, beta, st->M, st->z, out, st->heads, BH, N, st->d_key, st->d_value,
                          L, off, has_memory, st->scale, st->dtype == INFINI_BF16};
    hipError_t e = infini::launch_f32_attn(a, stream);
    if (e != hipSuccess) return hip_fail(e, "f32 attention launch");
    infini::F32UpdateArgs u{k, v, st->M, st->z, reinterpret_cast<float*>(ws + w.U), BH, N, st->d_key,
                            st->d_value, L, off, st->rule == INFINI_RULE_DELTA, has_memory,
                            st->dtype == INFINI_BF16};
    e = infini::launch_f32_update(u, stream);
    if (e != hipSuccess) return hip_fail(e, "f32 update launch");
  }
  if ((rc = record(events, 1, stream)) != INFINI_OK) return rc;
  return record(events, 2, stream);
}

// ------------------------------------------------------------------ open segment
// Workspace of infini_attn_append for n tokens: the largest of the three stages
// it runs one after another on the stream (whole segments straight from the
// input at a row stride of n, the commit of a completed open segment, and the
// open-segment attention's key partitions).
bool append_layout(const infini_attn_state* st, int64_t n, WsLayout* whole, WsLayout* one, size_t* part_off,
                   size_t* total) {
  const int64_t N = st->segment_len, BH = (int64_t)st->batch * st->heads;
  const int64_t S = n / N;
  if (S > 0 && !workspace_layout(st, S, n, whole)) return false;
  if (!workspace_layout(st, 1, N, one)) return false;
  const int64_t mq = n < N - 1 ? n : N - 1;   // queries of one open-segment piece
  int64_t parts;
  if (!mul_ok(BH * mq, (int64_t)infini::open_attn_slots((int)N, st->d_key) * (st->d_value + 2), &parts)) return false;
  *part_off = 0;
  size_t t = one->total;
  if (S > 0 && whole->total > t) t = whole->total;
  if (align_up((size_t)parts * 4) > t) t = align_up((size_t)parts * 4);
  *total = t;
  return true;
}

// Folds the completed open segment (N tokens per (b, h) in k_open, v_open) into
// (M, z) with the state's rule.
int commit_open(infini_attn_state* st, const infini_attn_open_segment* os, char* ws, const WsLayout& w,
                hipStream_t stream) {
  const int B = st->batch, H = st->heads, N = st->segment_len;
  hipError_t e;
  if (mfma_path(st)) {
    using infini::bf16;
    bf16* snapM = reinterpret_cast<bf16*>(ws + w.snapM);
    bf16* snapMlo = reinterpret_cast<bf16*>(ws + w.snapMlo);
    float* snapz = reinterpret_cast<float*>(ws + w.snapz);
    float* snapc = reinterpret_cast<float*>(ws + w.snapc);
    const bf16* k = static_cast<const bf16*>(os->k_open);
    const bf16* v = static_cast<const bf16*>(os->v_open);
    if (st->rule == INFINI_RULE_LINEAR) {
      infini::LinContribArgs c{k, v, reinterpret_cast<float*>(ws + w.cM), reinterpret_cast<float*>(ws + w.cz),
                               B, H, 1, N, N};
      infini::LinScanArgs sarg{c.cM, c.cz, st->M, st->z, snapM, snapMlo, snapz, snapc, B * H, 1};
      e = st->d_key == 128 ? infini::launch_lin_contrib<128>(c, stream) : infini::launch_lin_contrib<64>(c, stream);
      if (e != hipSuccess) return hip_fail(e, "lin_contrib launch");
      e = st->d_key == 128 ? infini::launch_lin_scan<128>(sarg, stream) : infini::launch_lin_scan<64>(sarg, stream);
      if (e != hipSuccess) return hip_fail(e, "lin_scan launch");
    } else {
      infini::DeltaArgs d{k, v, st->M, st->z, snapM, snapMlo, snapz, snapc, reinterpret_cast<float*>(ws + w.cM),
                          reinterpret_cast<float*>(ws + w.cz), reinterpret_cast<bf16*>(ws + w.amat), B * H, 1, N,
                          (int64_t)N, st->segments_done};
      e = st->d_key == 128 ? infini::launch_delta_state<128>(d, stream) : infini::launch_delta_state<64>(d, stream);
      if (e != hipSuccess) return hip_fail(e, "delta state launch");
    }
  } else {
    infini::F32UpdateArgs u{os->k_open, os->v_open, st->M, st->z, reinterpret_cast<float*>(ws + w.U), B * H, N,
                            st->d_key, st->d_value, (int64_t)N, 0, st->rule == INFINI_RULE_DELTA,
                            st->segments_done > 0, st->dtype == INFINI_BF16};
    if ((e = infini::launch_f32_update(u, stream)) != hipSuccess) return hip_fail(e, "f32 update launch");
  }
  return INFINI_OK;
}

int zero_state(infini_attn_state* st, float* M, float* z, hipStream_t stream) {
  const int64_t BH = (int64_t)st->batch * st->heads;
  const hipError_t e = infini::launch_fill_zero(M, BH * st->d_key * st->d_value, z, BH * st->d_key, stream);
  if (e != hipSuccess) return hip_fail(e, "fill launch");
  return INFINI_OK;
}

struct BwdLayout {
  size_t snapM, snapz, dMr, dzr, ez, gzs, lse, drow, rs, dden, de, dq, dk, dv, dfk, dbp, amat, gpart, total;
};

bool backward_layout(const infini_attn_state* st, int64_t seq_len, BwdLayout* w) {
  const int64_t BH = (int64_t)st->batch * st->heads, S = seq_len / st->segment_len;
  const int64_t dk = st->d_key, dv = st->d_value;
  int64_t segs, rows, mm, rk, rv, nb;
  if (!mul_ok(BH, S, &segs) || !mul_ok(BH, seq_len, &rows) || !mul_ok(segs, dk * dv, &mm) ||
      !mul_ok(rows, dk, &rk) || !mul_ok(rows, dv, &rv) || !mul_ok(segs, infini::bwd_query_blocks(st->segment_len), &nb))
    return false;
  size_t off = 0;
  auto take = [&](size_t* field, int64_t floats) { *field = off; off = align_up(off + (size_t)floats * 4); };
  take(&w->snapM, mm);
  take(&w->snapz, segs * dk);
  take(&w->dMr, mm);
  take(&w->dzr, segs * dk);
  take(&w->ez, segs * dk);
  take(&w->gzs, segs * dk);
  take(&w->lse, rows);
  take(&w->drow, rows);
  take(&w->rs, rows);
  take(&w->dden, rows);
  take(&w->de, rows);
  // bf16 MFMA path: the query kernel writes dq in one piece (no fp32 accumulator)
  const bool mfma = st->dtype == INFINI_BF16 && mfma_shape(st->d_key, st->d_value, st->segment_len);
  take(&w->dq, mfma ? 0 : rk);
  take(&w->dk, rk);
  take(&w->dv, rv);
  take(&w->dfk, rk);
  take(&w->dbp, nb);
  // delta rule on the bf16 path: sigma(K)^T diag(1/e) sigma(K) per segment
  const bool amat = st->rule == INFINI_RULE_DELTA && st->dtype == INFINI_BF16;
  take(&w->amat, amat ? segs * dk * dk : 0);
  // bf16 MFMA path: the second halves of the per-segment Gram products
  take(&w->gpart, mfma ? mm + segs * dk : 0);
  w->total = off;
  return true;
}

}  // namespace

// ------------------------------------------------------------------ allocation-free forward
// The workspace of infini_attn_forward_sequence_noalloc: a file-scope device
// array that every GPU the library runs on holds until the process ends.  In host
// code `scratch` names a host-side stand-in, not the device memory: host code
// only ever uses the device address that hipGetSymbolAddress returns for the
// current device (kept per device below).
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch array, looked up once per device with
// that device current.
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(INFINI_EUNSUPPORTED, "device index %d above %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(INFINI_EHIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return INFINI_OK;
}
}  // namespace

extern "C" {

int infini_attn_abi_version(void) { return 1; }

size_t infini_attn_noalloc_scratch_bytes(void) { return kScratchBytes; }

const char* infini_attn_last_error(void) { return g_error.c_str(); }

int infini_attn_init_state(infini_attn_state* st, int32_t batch, int32_t heads, int32_t d_key, int32_t d_value,
                           int32_t segment_len, int32_t dtype, int32_t rule, float scale, float* M, float* z,
                           void* stream) {
  if (!st) return fail(INFINI_EINVAL, "state pointer is NULL");
  int rc = check_config(batch, heads, d_key, d_value, segment_len, dtype, rule, scale);
  if (rc != INFINI_OK) return rc;
  if (!M || !z) return fail(INFINI_EINVAL, "M and z must be device pointers (got NULL)");
  if ((reinterpret_cast<uintptr_t>(M) | reinterpret_cast<uintptr_t>(z)) % 4 != 0)
    return fail(INFINI_EINVAL, "M and z must be 4-byte aligned");
  infini_attn_state next;
  next.batch = batch;
  next.heads = heads;
  next.d_key = d_key;
  next.d_value = d_value;
  next.segment_len = segment_len;
  next.dtype = dtype;
  next.rule = rule;
  next.scale = scale > 0.f ? scale : (float)(1.0 / std::sqrt((double)d_key));
  next.M = M;
  next.z = z;
  next.segments_done = 0;
  const int64_t nM = (int64_t)batch * heads * d_key * d_value, nz = (int64_t)batch * heads * d_key;
  if (overlaps(M, (size_t)nM * 4, z, (size_t)nz * 4)) return fail(INFINI_EINVAL, "M and z overlap");
  rc = zero_state(&next, M, z, static_cast<hipStream_t>(stream));
  if (rc != INFINI_OK) return rc;
  *st = next;
  return ok();
}

size_t infini_attn_workspace_bytes(const infini_attn_state* st, int64_t seq_len) {
  if (check_state(st) != INFINI_OK) return 0;
  if (seq_len <= 0 || seq_len % st->segment_len != 0) return 0;
  WsLayout w;
  if (!workspace_layout(st, seq_len / st->segment_len, seq_len, &w)) return 0;
  return w.total;
}

static int forward_impl(infini_attn_state* st, const void* q, const void* k, const void* v, int64_t seq_len,
                        const float* beta, void* out, void* workspace, size_t workspace_bytes, void* stream,
                        void* const* events, float* lse = nullptr, bool pipeline = true) {
  int rc = check_state(st);
  if (rc != INFINI_OK) return rc;
  if (!q || !k || !v || !beta || !out) return fail(INFINI_EINVAL, "q, k, v, beta and out must be non-NULL");
  if (seq_len <= 0 || seq_len % st->segment_len != 0)
    return fail(INFINI_EINVAL, "seq_len (%lld) must be a positive multiple of segment_len (%d)",
                (long long)seq_len, st->segment_len);
  const int64_t S64 = seq_len / st->segment_len;
  if (S64 > 0x7fffffff) return fail(INFINI_EINVAL, "too many segments");
  const int S = (int)S64;
  const int64_t BH = (int64_t)st->batch * st->heads;
  int64_t rows, nqk, nvo;
  if (!mul_ok(BH, seq_len, &rows) || !mul_ok(rows, st->d_key, &nqk) || !mul_ok(rows, st->d_value, &nvo))
    return fail(INFINI_EINVAL, "tensor sizes overflow");
  const size_t esz = st->dtype == INFINI_BF16 ? 2 : 4;
  const uintptr_t align = st->dtype == INFINI_BF16 ? 16 : 4;
  for (const void* p : {q, k, v, static_cast<const void*>(out)})
    if (reinterpret_cast<uintptr_t>(p) % align != 0)
      return fail(INFINI_EINVAL, "q, k, v and out must be %d-byte aligned", (int)align);
  if (reinterpret_cast<uintptr_t>(beta) % 4 != 0) return fail(INFINI_EINVAL, "beta must be 4-byte aligned");
  const size_t out_bytes = (size_t)nvo * esz;
  if (overlaps(out, out_bytes, q, (size_t)nqk * esz) || overlaps(out, out_bytes, k, (size_t)nqk * esz) ||
      overlaps(out, out_bytes, v, (size_t)nvo * esz))
    return fail(INFINI_EINVAL, "out must not alias q, k or v");
  const size_t m_bytes = (size_t)BH * st->d_key * st->d_value * 4, z_bytes = (size_t)BH * st->d_key * 4;
  if (overlaps(out, out_bytes, st->M, m_bytes) || overlaps(out, out_bytes, st->z, z_bytes))
    return fail(INFINI_EINVAL, "out must not alias the state");
  WsLayout w;
  if (!workspace_layout(st, S, seq_len, &w)) return fail(INFINI_EINVAL, "workspace size overflows");
  if (!workspace || workspace_bytes < w.total)
    return fail(INFINI_EWORKSPACE, "workspace of %zu bytes required, %zu given%s", w.total, workspace_bytes,
                workspace ? "" : " (NULL)");
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0)
    return fail(INFINI_EWORKSPACE, "workspace must be 256-byte aligned");
  if (overlaps(workspace, w.total, out, out_bytes) || overlaps(workspace, w.total, st->M, m_bytes) ||
      overlaps(workspace, w.total, st->z, z_bytes))
    return fail(INFINI_EWORKSPACE, "workspace must not alias out or the state");
  if (lse) {
    if (!mfma_path(st))
      return fail(INFINI_EUNSUPPORTED, "the log-normalisers are kept on the bf16 MFMA path only "
                  "(d_key = d_value in {64, 128}, segment_len a multiple of 64)");
    if (reinterpret_cast<uintptr_t>(lse) % 4 != 0) return fail(INFINI_EINVAL, "lse must be 4-byte aligned");
    const size_t lb = (size_t)rows * 4;
    if (overlaps(lse, lb, out, out_bytes) || overlaps(lse, lb, q, (size_t)nqk * esz) ||
        overlaps(lse, lb, k, (size_t)nqk * esz) || overlaps(lse, lb, v, (size_t)nvo * esz) ||
        overlaps(lse, lb, st->M, m_bytes) || overlaps(lse, lb, st->z, z_bytes) ||
        overlaps(lse, lb, workspace, w.total) || overlaps(lse, lb, beta, (size_t)st->heads * 4))
      return fail(INFINI_EINVAL, "lse must not alias out, the inputs, the state or the workspace");
  }
  if (mfma_path(st)) {
    const int64_t fa_blocks = infini::fa_fwd_blocks(BH * S64, st->segment_len);
    if (fa_blocks > 0x7fffffff) return fail(INFINI_EUNSUPPORTED, "launch grid too large; split the call");
  }

  hipStream_t strm = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  if (mfma_path(st)) {
    rc = st->d_key == 128 ? run_bf16<128>(st, q, k, v, seq_len, S, beta, out, ws, w, strm, events, lse, pipeline)
                          : run_bf16<64>(st, q, k, v, seq_len, S, beta, out, ws, w, strm, events, lse, pipeline);
  } else {
    rc = run_f32(st, q, k, v, seq_len, S, beta, out, ws, w, strm, events);
  }
  if (rc != INFINI_OK) return rc;
  st->segments_done += S;
  return ok();
}

int infini_attn_forward_sequence(infini_attn_state* st, const void* q, const void* k, const void* v,
                                 int64_t seq_len, const float* beta, void* out, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  return forward_impl(st, q, k, v, seq_len, beta, out, workspace, workspace_bytes, stream, nullptr);
}

int infini_attn_forward_sequence_train(infini_attn_state* st, const void* q, const void* k, const void* v,
                                       int64_t seq_len, const float* beta, void* out, float* lse, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  if (!lse) return fail(INFINI_EINVAL, "lse must be non-NULL");
  return forward_impl(st, q, k, v, seq_len, beta, out, workspace, workspace_bytes, stream, nullptr, lse);
}

int infini_attn_forward_sequence_noalloc(infini_attn_state* st, const void* q, const void* k, const void* v,
                                         int64_t seq_len, const float* beta, void* out, void* stream) {
  int rc = check_state(st);
  if (rc != INFINI_OK) return rc;
  if (seq_len <= 0 || seq_len % st->segment_len != 0)
    return fail(INFINI_EINVAL, "seq_len (%lld) must be a positive multiple of segment_len (%d)",
                (long long)seq_len, st->segment_len);
  WsLayout w;
  if (!workspace_layout(st, seq_len / st->segment_len, seq_len, &w)) return fail(INFINI_EINVAL, "workspace size overflows");
  if (w.total > kScratchBytes)
    return fail(INFINI_EWORKSPACE, "this call needs %zu bytes of scratch; the allocation-free entry point has %zu "
                "(split the stream into shorter calls, or use infini_attn_forward_sequence with a workspace)",
                w.total, kScratchBytes);
  void* ws = nullptr;
  if ((rc = scratch_address(&ws)) != INFINI_OK) return rc;
  // (not pipelined: the side stream and its events are resources created on first use)
  return forward_impl(st, q, k, v, seq_len, beta, out, ws, kScratchBytes, stream, nullptr, nullptr, false);
}

int infini_attn_forward_sequence_profiled(infini_attn_state* st, const void* q, const void* k, const void* v,
                                          int64_t seq_len, const float* beta, void* out, void* workspace,
                                          size_t workspace_bytes, void* stream, void* const* events,
                                          int32_t n_events) {
  if (!events || n_events != 3 || !events[0] || !events[1] || !events[2])
    return fail(INFINI_EINVAL, "profiled forward needs exactly 3 non-NULL events");
  return forward_impl(st, q, k, v, seq_len, beta, out, workspace, workspace_bytes, stream, events);
}

size_t infini_attn_backward_workspace_bytes(const infini_attn_state* st, int64_t seq_len) {
  if (check_state(st) != INFINI_OK) return 0;
  if (seq_len <= 0 || seq_len % st->segment_len != 0) return 0;
  BwdLayout w;
  if (!backward_layout(st, seq_len, &w)) return 0;
  return w.total;
}

static int backward_impl(const infini_attn_state* st, const void* q, const void* k, const void* v,
                         int64_t seq_len, const float* beta, const void* out_fw, const float* lse_fw,
                         const void* dout, const float* dM, const float* dz, void* dq, void* dk, void* dv,
                         float* dbeta, float* dM0, float* dz0, void* workspace, size_t workspace_bytes,
                         void* stream) {
  int rc = check_state(st);
  if (rc != INFINI_OK) return rc;
  const bool saved = out_fw != nullptr;
  if (saved && !mfma_path(st))
    return fail(INFINI_EUNSUPPORTED, "the saved-statistics backward runs on the bf16 MFMA path only "
                "(d_key = d_value in {64, 128}, segment_len a multiple of 64)");
  if (!q || !k || !v || !beta || !dout || !dq || !dk || !dv || !dbeta)
    return fail(INFINI_EINVAL, "q, k, v, beta, dout, dq, dk, dv and dbeta must be non-NULL");
  if (seq_len <= 0 || seq_len % st->segment_len != 0)
    return fail(INFINI_EINVAL, "seq_len (%lld) must be a positive multiple of segment_len (%d)",
                (long long)seq_len, st->segment_len);
  const int64_t S64 = seq_len / st->segment_len;
  if (S64 > 65535) return fail(INFINI_EUNSUPPORTED, "more than 65535 segments in one backward call");
  const int64_t BH = (int64_t)st->batch * st->heads;
  if (BH > 65535) return fail(INFINI_EUNSUPPORTED, "batch * heads above 65535 for the backward kernels");
  int64_t rows, nqk, nvo;
  if (!mul_ok(BH, seq_len, &rows) || !mul_ok(rows, st->d_key, &nqk) || !mul_ok(rows, st->d_value, &nvo))
    return fail(INFINI_EINVAL, "tensor sizes overflow");
  if ((rows + 1) / 2 > 0x7fffffff) return fail(INFINI_EUNSUPPORTED, "launch grid too large; split the call");
  const size_t esz = st->dtype == INFINI_BF16 ? 2 : 4;
  // bf16: the MFMA kernels read and write whole 16-byte row pieces; fp32: the
  // final stores take 16-byte vectors only where the outputs allow it
  const uintptr_t align = st->dtype == INFINI_BF16 ? 16 : 4;
  for (const void* p : {q, k, v, dout, static_cast<const void*>(dq), static_cast<const void*>(dk),
                        static_cast<const void*>(dv)})
    if (reinterpret_cast<uintptr_t>(p) % align != 0)
      return fail(INFINI_EINVAL, "q, k, v, dout, dq, dk and dv must be %d-byte aligned", (int)align);
  for (const void* p : {static_cast<const void*>(beta), static_cast<const void*>(dM), static_cast<const void*>(dz),
                        static_cast<const void*>(dbeta), static_cast<const void*>(dM0), static_cast<const void*>(dz0),
                        static_cast<const void*>(lse_fw)})
    if (reinterpret_cast<uintptr_t>(p) % 4 != 0) return fail(INFINI_EINVAL, "fp32 arguments must be 4-byte aligned");
  if (saved && reinterpret_cast<uintptr_t>(out_fw) % align != 0)
    return fail(INFINI_EINVAL, "out must be %d-byte aligned", (int)align);
  const size_t qkb = (size_t)nqk * esz, vb = (size_t)nvo * esz;
  const size_t mb = (size_t)BH * st->d_key * st->d_value * 4, zb = (size_t)BH * st->d_key * 4;
  BwdLayout w;
  if (!backward_layout(st, seq_len, &w)) return fail(INFINI_EINVAL, "workspace size overflows");
  if (!workspace || workspace_bytes < w.total)
    return fail(INFINI_EWORKSPACE, "workspace of %zu bytes required, %zu given%s", w.total, workspace_bytes,
                workspace ? "" : " (NULL)");
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0)
    return fail(INFINI_EWORKSPACE, "workspace must be 256-byte aligned");
  struct Buf { const void* p; size_t n; };
  const Buf outs[] = {{dq, qkb}, {dk, qkb}, {dv, vb}, {dbeta, (size_t)st->heads * 4}, {dM0, dM0 ? mb : 0},
                      {dz0, dz0 ? zb : 0}, {workspace, w.total}};
  const Buf ins[] = {{q, qkb}, {k, qkb}, {v, vb}, {dout, vb}, {beta, (size_t)st->heads * 4}, {dM, dM ? mb : 0},
                     {dz, dz ? zb : 0}, {st->M, mb}, {st->z, zb}, {out_fw, saved ? vb : 0},
                     {lse_fw, saved ? (size_t)rows * 4 : 0}};
  for (size_t i = 0; i < sizeof(outs) / sizeof(outs[0]); ++i) {
    if (!outs[i].n) continue;
    for (size_t j = i + 1; j < sizeof(outs) / sizeof(outs[0]); ++j)
      if (outs[j].n && overlaps(outs[i].p, outs[i].n, outs[j].p, outs[j].n))
        return fail(INFINI_EINVAL, "the outputs and the workspace must not overlap each other");
    for (const Buf& b : ins)
      if (b.n && overlaps(outs[i].p, outs[i].n, b.p, b.n))
        return fail(INFINI_EINVAL, "the outputs and the workspace must not alias the inputs or the state");
  }

  char* ws = static_cast<char*>(workspace);
  auto f = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
  infini::BwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.dout = dout; a.beta = beta; a.M0 = st->M; a.z0 = st->z; a.dM = dM; a.dz = dz;
  a.dq_out = dq; a.dk_out = dk; a.dv_out = dv; a.dbeta = dbeta; a.dM0 = dM0; a.dz0 = dz0;
  a.snapM = f(w.snapM); a.snapz = f(w.snapz); a.dMr = f(w.dMr); a.dzr = f(w.dzr); a.ez = f(w.ez); a.gzs = f(w.gzs);
  a.lse = saved ? const_cast<float*>(lse_fw) : f(w.lse); a.drow = f(w.drow); a.out_fw = out_fw; a.rs = f(w.rs); a.dden = f(w.dden); a.de = f(w.de);
  a.dq_acc = mfma_path(st) ? nullptr : f(w.dq); a.dk_acc = f(w.dk); a.dv_acc = f(w.dv); a.dfk_acc = f(w.dfk); a.dbeta_part = f(w.dbp);
  a.Amat = f(w.amat);
  a.gpart = f(w.gpart);
  a.B = st->batch; a.H = st->heads; a.BH = (int)BH; a.N = st->segment_len; a.S = (int)S64;
  a.dk = st->d_key; a.dv = st->d_value; a.nqb = infini::bwd_query_blocks(st->segment_len);
  a.L = seq_len; a.seg_base = st->segments_done; a.delta = st->rule == INFINI_RULE_DELTA; a.scale = st->scale;
  const hipError_t e = infini::launch_backward(a, st->dtype == INFINI_BF16, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "backward launch");
  return ok();
}

int infini_attn_backward_sequence(const infini_attn_state* st, const void* q, const void* k, const void* v,
                                  int64_t seq_len, const float* beta, const void* dout, const float* dM,
                                  const float* dz, void* dq, void* dk, void* dv, float* dbeta, float* dM0,
                                  float* dz0, void* workspace, size_t workspace_bytes, void* stream) {
  return backward_impl(st, q, k, v, seq_len, beta, nullptr, nullptr, dout, dM, dz, dq, dk, dv, dbeta, dM0, dz0,
                       workspace, workspace_bytes, stream);
}

int infini_attn_backward_sequence_saved(const infini_attn_state* st, const void* q, const void* k, const void* v,
                                        int64_t seq_len, const float* beta, const void* out, const float* lse,
                                        const void* dout, const float* dM, const float* dz, void* dq, void* dk,
                                        void* dv, float* dbeta, float* dM0, float* dz0, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  if (!out || !lse) return fail(INFINI_EINVAL, "out and lse must be non-NULL");
  return backward_impl(st, q, k, v, seq_len, beta, out, lse, dout, dM, dz, dq, dk, dv, dbeta, dM0, dz0, workspace,
                       workspace_bytes, stream);
}

// ------------------------------------------------------------------ layer
namespace {
// Workspace of the layer: q, k, v and the heads' outputs (bf16 [B, H, L, d]), then
// the forward's own workspace.
bool layer_layout(const infini_attn_state* st, int64_t seq_len, size_t* qo, size_t* ko, size_t* vo, size_t* ao,
                  size_t* fo, WsLayout* fw, size_t* total) {
  const int64_t BH = (int64_t)st->batch * st->heads;
  int64_t rows, nq, nv;
  if (!mul_ok(BH, seq_len, &rows) || !mul_ok(rows, st->d_key, &nq) || !mul_ok(rows, st->d_value, &nv)) return false;
  if (!workspace_layout(st, seq_len / st->segment_len, seq_len, fw)) return false;
  size_t off = 0;
  *qo = off; off = align_up(off + (size_t)nq * 2);
  *ko = off; off = align_up(off + (size_t)nq * 2);
  *vo = off; off = align_up(off + (size_t)nv * 2);
  *ao = off; off = align_up(off + (size_t)nv * 2);
  *fo = off; off = align_up(off + fw->total);
  *total = off;
  return true;
}
}  // namespace

size_t infini_attn_layer_workspace_bytes(const infini_attn_state* st, int32_t d_model, int64_t seq_len) {
  if (check_state(st) != INFINI_OK || !mfma_path(st) || d_model <= 0 || d_model % 64 != 0) return 0;
  if (seq_len <= 0 || seq_len % st->segment_len != 0) return 0;
  size_t qo, ko, vo, ao, fo, total;
  WsLayout fw;
  if (!layer_layout(st, seq_len, &qo, &ko, &vo, &ao, &fo, &fw, &total)) return 0;
  return total;
}

int infini_attn_layer_forward(infini_attn_state* st, const void* x, int32_t d_model, const void* w_qkv,
                              const void* w_o, int64_t seq_len, const float* beta, void* y, void* workspace,
                              size_t workspace_bytes, void* stream) {
  int rc = check_state(st);
  if (rc != INFINI_OK) return rc;
  if (!mfma_path(st))
    return fail(INFINI_EUNSUPPORTED, "the layer entry point runs the MFMA path only (bf16, d_key == d_value in "
                                     "{64, 128}, segment_len a multiple of 64)");
  if (!x || !w_qkv || !w_o || !beta || !y) return fail(INFINI_EINVAL, "x, w_qkv, w_o, beta and y must be non-NULL");
  if (d_model <= 0 || d_model % 64 != 0)
    return fail(INFINI_EUNSUPPORTED, "d_model must be a positive multiple of 64 (got %d)", d_model);
  if (seq_len <= 0 || seq_len % st->segment_len != 0)
    return fail(INFINI_EINVAL, "seq_len (%lld) must be a positive multiple of segment_len (%d)",
                (long long)seq_len, st->segment_len);
  const int64_t S64 = seq_len / st->segment_len;
  if (S64 > 0x7fffffff) return fail(INFINI_EINVAL, "too many segments");
  const int64_t BH = (int64_t)st->batch * st->heads;
  const int64_t M = (int64_t)st->batch * seq_len;
  const int64_t nqkv = (int64_t)st->heads * (2 * st->d_key + st->d_value);
  if (M > 0x7fffffff - 256 || (M + 127) / 128 > 65535)
    return fail(INFINI_EUNSUPPORTED, "batch * seq_len too large for one layer call; split the call");
  for (const void* p : {x, w_qkv, w_o, static_cast<const void*>(y)})
    if (reinterpret_cast<uintptr_t>(p) % 16 != 0) return fail(INFINI_EINVAL, "x, w_qkv, w_o and y must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(beta) % 4 != 0) return fail(INFINI_EINVAL, "beta must be 4-byte aligned");
  size_t qo, ko, vo, ao, fo, total;
  WsLayout fw;
  if (!layer_layout(st, seq_len, &qo, &ko, &vo, &ao, &fo, &fw, &total))
    return fail(INFINI_EINVAL, "workspace size overflows");
  if (!workspace || workspace_bytes < total)
    return fail(INFINI_EWORKSPACE, "workspace of %zu bytes required, %zu given%s", total, workspace_bytes,
                workspace ? "" : " (NULL)");
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0)
    return fail(INFINI_EWORKSPACE, "workspace must be 256-byte aligned");
  const size_t xb = (size_t)M * d_model * 2, wqb = (size_t)d_model * nqkv * 2;
  const size_t wob = (size_t)st->heads * st->d_value * d_model * 2;
  const size_t mb = (size_t)BH * st->d_key * st->d_value * 4, zb = (size_t)BH * st->d_key * 4;
  for (const auto& in : {std::make_pair(x, xb), std::make_pair(w_qkv, wqb), std::make_pair(w_o, wob),
                         std::make_pair(static_cast<const void*>(st->M), mb),
                         std::make_pair(static_cast<const void*>(st->z), zb)}) {
    if (overlaps(y, xb, in.first, in.second)) return fail(INFINI_EINVAL, "y must not alias the inputs or the state");
    if (overlaps(workspace, total, in.first, in.second))
      return fail(INFINI_EWORKSPACE, "workspace must not alias the inputs or the state");
  }
  if (overlaps(workspace, total, y, xb)) return fail(INFINI_EWORKSPACE, "workspace must not alias y");
  const int64_t fa_blocks = infini::fa_fwd_blocks(BH * S64, st->segment_len);
  if (fa_blocks > 0x7fffffff) return fail(INFINI_EUNSUPPORTED, "launch grid too large; split the call");

  hipStream_t strm = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  typedef infini::bf16 bf;
  bf* q = reinterpret_cast<bf*>(ws + qo);
  bf* k = reinterpret_cast<bf*>(ws + ko);
  bf* v = reinterpret_cast<bf*>(ws + vo);
  bf* a = reinterpret_cast<bf*>(ws + ao);
  infini::GemmArgs g1{static_cast<const bf*>(x), static_cast<const bf*>(w_qkv), nullptr, q, k, v,
                      (int)M, (int)nqkv, d_model, 0, 1, (int)seq_len, st->heads, st->d_key, st->d_value};
  hipError_t e = infini::launch_gemm_bf16(g1, strm);
  if (e != hipSuccess) return hip_fail(e, "QKV projection launch");
  infini_attn_state s = *st;
  rc = s.d_key == 128 ? run_bf16<128>(&s, q, k, v, seq_len, (int)S64, beta, a, ws + fo, fw, strm, nullptr, nullptr, true)
                      : run_bf16<64>(&s, q, k, v, seq_len, (int)S64, beta, a, ws + fo, fw, strm, nullptr, nullptr, true);
  if (rc != INFINI_OK) return rc;
  infini::GemmArgs g2{a, static_cast<const bf*>(w_o), static_cast<bf*>(y), nullptr, nullptr, nullptr,
                      (int)M, d_model, st->heads * st->d_value, 1, 0, (int)seq_len, st->heads, st->d_key,
                      st->d_value};
  e = infini::launch_gemm_bf16(g2, strm);
  if (e != hipSuccess) return hip_fail(e, "output projection launch");
  st->segments_done += S64;
  return ok();
}

int infini_attn_kernel_linear_attention(infini_attn_state* st, const void* q, const void* k, const void* v,
                                        int64_t seq_len, void* out, void* workspace, size_t workspace_bytes,
                                        void* stream) {
  int rc = check_state(st);
  if (rc != INFINI_OK) return rc;
  if (!mfma_path(st))
    return fail(INFINI_EUNSUPPORTED, "kernel linear attention runs on the MFMA path only (bf16, d_key == d_value "
                                     "in {64, 128}, segment_len a multiple of 64)");
  if (st->rule != INFINI_RULE_LINEAR)
    return fail(INFINI_EINVAL, "kernel linear attention needs a state with the linear update rule");
  if (!q || !k || !v || !out) return fail(INFINI_EINVAL, "q, k, v and out must be non-NULL");
  if (seq_len <= 0 || seq_len % st->segment_len != 0)
    return fail(INFINI_EINVAL, "seq_len (%lld) must be a positive multiple of segment_len (%d)",
                (long long)seq_len, st->segment_len);
  const int64_t S64 = seq_len / st->segment_len;
  const int64_t BH = (int64_t)st->batch * st->heads;
  if (S64 > 65535 || BH > 65535) return fail(INFINI_EUNSUPPORTED, "launch grid too large; split the call");
  int64_t rows, nqk;
  if (!mul_ok(BH, seq_len, &rows) || !mul_ok(rows, st->d_key, &nqk))
    return fail(INFINI_EINVAL, "tensor sizes overflow");
  for (const void* p : {q, k, v, static_cast<const void*>(out)})
    if (reinterpret_cast<uintptr_t>(p) % 16 != 0) return fail(INFINI_EINVAL, "q, k, v and out must be 16-byte aligned");
  const size_t tb = (size_t)nqk * 2;
  const size_t mb = (size_t)BH * st->d_key * st->d_value * 4, zb = (size_t)BH * st->d_key * 4;
  if (overlaps(out, tb, q, tb) || overlaps(out, tb, k, tb) || overlaps(out, tb, v, tb) ||
      overlaps(out, tb, st->M, mb) || overlaps(out, tb, st->z, zb))
    return fail(INFINI_EINVAL, "out must not alias q, k, v or the state");
  WsLayout w;
  if (!workspace_layout(st, S64, seq_len, &w)) return fail(INFINI_EINVAL, "workspace size overflows");
  if (!workspace || workspace_bytes < w.total)
    return fail(INFINI_EWORKSPACE, "workspace of %zu bytes required, %zu given%s", w.total, workspace_bytes,
                workspace ? "" : " (NULL)");
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0)
    return fail(INFINI_EWORKSPACE, "workspace must be 256-byte aligned");
  if (overlaps(workspace, w.total, out, tb) || overlaps(workspace, w.total, st->M, mb) ||
      overlaps(workspace, w.total, st->z, zb))
    return fail(INFINI_EWORKSPACE, "workspace must not alias out or the state");

  using infini::bf16;
  hipStream_t strm = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const int B = st->batch, H = st->heads, N = st->segment_len, S = (int)S64, D = st->d_key;
  bf16* snapM = reinterpret_cast<bf16*>(ws + w.snapM);
  bf16* snapMlo = reinterpret_cast<bf16*>(ws + w.snapMlo);
  float* snapz = reinterpret_cast<float*>(ws + w.snapz);
  float* snapc = reinterpret_cast<float*>(ws + w.snapc);
  infini::LinContribArgs c{static_cast<const bf16*>(k), static_cast<const bf16*>(v),
                           reinterpret_cast<float*>(ws + w.cM), reinterpret_cast<float*>(ws + w.cz), B, H, S, N,
                           seq_len};
  hipError_t e = D == 128 ? infini::launch_lin_contrib<128>(c, strm) : infini::launch_lin_contrib<64>(c, strm);
  if (e != hipSuccess) return hip_fail(e, "lin_contrib launch");
  infini::LinScanArgs sarg{c.cM, c.cz, st->M, st->z, snapM, snapMlo, snapz, snapc, B * H, S};
  e = D == 128 ? infini::launch_lin_scan<128>(sarg, strm) : infini::launch_lin_scan<64>(sarg, strm);
  if (e != hipSuccess) return hip_fail(e, "lin_scan launch");
  infini::FaArgs f{static_cast<const bf16*>(q), static_cast<const bf16*>(k), static_cast<const bf16*>(v), nullptr,
                   snapM, snapMlo, snapz, snapc, static_cast<bf16*>(out), B, H, S, N, seq_len, 0, st->segments_done,
                   0.f};
  e = D == 128 ? infini::launch_kla<128>(f, strm) : infini::launch_kla<64>(f, strm);
  if (e != hipSuccess) return hip_fail(e, "kernel linear attention launch");
  st->segments_done += S64;
  return ok();
}

int infini_attn_forward_segment(infini_attn_state* st, const void* q, const void* k, const void* v,
                                const float* beta, void* out, void* workspace, size_t workspace_bytes,
                                void* stream) {
  if (!st) return fail(INFINI_EINVAL, "state pointer is NULL");
  return infini_attn_forward_sequence(st, q, k, v, st->segment_len, beta, out, workspace, workspace_bytes, stream);
}

int infini_attn_open_segment_init(const infini_attn_state* st, infini_attn_open_segment* os, void* k_open,
                                  void* v_open) {
  int rc = check_state(st);
  if (rc != INFINI_OK) return rc;
  if (!os) return fail(INFINI_EINVAL, "open-segment pointer is NULL");
  if (!k_open || !v_open) return fail(INFINI_EINVAL, "open-segment buffers must be device pointers (got NULL)");
  const uintptr_t align = st->dtype == INFINI_BF16 ? 16 : 4;
  if ((reinterpret_cast<uintptr_t>(k_open) | reinterpret_cast<uintptr_t>(v_open)) % align != 0)
    return fail(INFINI_EINVAL, "open-segment buffers must be %d-byte aligned", (int)align);
  const int64_t BH = (int64_t)st->batch * st->heads;
  const size_t esz = st->dtype == INFINI_BF16 ? 2 : 4;
  const size_t kb = (size_t)BH * st->segment_len * st->d_key * esz, vb = (size_t)BH * st->segment_len * st->d_value * esz;
  const size_t mb = (size_t)BH * st->d_key * st->d_value * 4, zb = (size_t)BH * st->d_key * 4;
  if (overlaps(k_open, kb, v_open, vb) || overlaps(k_open, kb, st->M, mb) || overlaps(k_open, kb, st->z, zb) ||
      overlaps(v_open, vb, st->M, mb) || overlaps(v_open, vb, st->z, zb))
    return fail(INFINI_EINVAL, "open-segment buffers must not overlap each other or the state");
  os->k_open = k_open;
  os->v_open = v_open;
  os->filled = 0;
  return ok();
}

size_t infini_attn_append_workspace_bytes(const infini_attn_state* st, int64_t n_tokens) {
  if (check_state(st) != INFINI_OK || n_tokens < 1) return 0;
  WsLayout whole, one;
  size_t part_off, total;
  if (!append_layout(st, n_tokens, &whole, &one, &part_off, &total)) return 0;
  return total;
}

int infini_attn_append(infini_attn_state* st, infini_attn_open_segment* os, const void* q, const void* k,
                       const void* v, int64_t n_tokens, const float* beta, void* out, void* workspace,
                       size_t workspace_bytes, void* stream) {
  int rc = check_state(st);
  if (rc != INFINI_OK) return rc;
  if (!os) return fail(INFINI_EINVAL, "open-segment pointer is NULL");
  const int N = st->segment_len;
  if (!os->k_open || !os->v_open || os->filled < 0 || os->filled >= N)
    return fail(INFINI_EINVAL, "open segment not initialised (buffers NULL or filled %d outside [0, %d))",
                os->filled, N);
  if (!q || !k || !v || !beta || !out) return fail(INFINI_EINVAL, "q, k, v, beta and out must be non-NULL");
  if (n_tokens < 1) return fail(INFINI_EINVAL, "n_tokens must be positive (got %lld)", (long long)n_tokens);
  const int64_t BH = (int64_t)st->batch * st->heads;
  int64_t rows, nqk, nvo;
  if (!mul_ok(BH, n_tokens, &rows) || !mul_ok(rows, st->d_key, &nqk) || !mul_ok(rows, st->d_value, &nvo))
    return fail(INFINI_EINVAL, "tensor sizes overflow");
  if (n_tokens / N > 0x7fffffff) return fail(INFINI_EINVAL, "too many segments");
  const size_t esz = st->dtype == INFINI_BF16 ? 2 : 4;
  const uintptr_t align = st->dtype == INFINI_BF16 ? 16 : 4;
  for (const void* p : {q, k, v, static_cast<const void*>(out), static_cast<const void*>(os->k_open),
                        static_cast<const void*>(os->v_open)})
    if (reinterpret_cast<uintptr_t>(p) % align != 0)
      return fail(INFINI_EINVAL, "q, k, v, out and the open-segment buffers must be %d-byte aligned", (int)align);
  if (reinterpret_cast<uintptr_t>(beta) % 4 != 0) return fail(INFINI_EINVAL, "beta must be 4-byte aligned");
  const size_t out_bytes = (size_t)nvo * esz;
  const size_t kob = (size_t)BH * N * st->d_key * esz, vob = (size_t)BH * N * st->d_value * esz;
  const size_t m_bytes = (size_t)BH * st->d_key * st->d_value * 4, z_bytes = (size_t)BH * st->d_key * 4;
  if (overlaps(out, out_bytes, q, (size_t)nqk * esz) || overlaps(out, out_bytes, k, (size_t)nqk * esz) ||
      overlaps(out, out_bytes, v, (size_t)nvo * esz) || overlaps(out, out_bytes, st->M, m_bytes) ||
      overlaps(out, out_bytes, st->z, z_bytes) || overlaps(out, out_bytes, os->k_open, kob) ||
      overlaps(out, out_bytes, os->v_open, vob))
    return fail(INFINI_EINVAL, "out must not alias q, k, v, the state or the open-segment buffers");
  WsLayout whole, one;
  size_t part_off, total;
  if (!append_layout(st, n_tokens, &whole, &one, &part_off, &total))
    return fail(INFINI_EINVAL, "workspace size overflows");
  if (!workspace || workspace_bytes < total)
    return fail(INFINI_EWORKSPACE, "workspace of %zu bytes required, %zu given%s", total, workspace_bytes,
                workspace ? "" : " (NULL)");
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0)
    return fail(INFINI_EWORKSPACE, "workspace must be 256-byte aligned");
  if (overlaps(workspace, total, out, out_bytes) || overlaps(workspace, total, st->M, m_bytes) ||
      overlaps(workspace, total, st->z, z_bytes) || overlaps(workspace, total, os->k_open, kob) ||
      overlaps(workspace, total, os->v_open, vob))
    return fail(INFINI_EWORKSPACE, "workspace must not alias out, the state or the open-segment buffers");
  if (mfma_path(st) && n_tokens >= N) {
    const int64_t fa_blocks = infini::fa_fwd_blocks(BH * (n_tokens / N), N);
    if (fa_blocks > 0x7fffffff) return fail(INFINI_EUNSUPPORTED, "launch grid too large; split the call");
  }
  if (BH > 65535) return fail(INFINI_EUNSUPPORTED, "batch * heads above 65535 for the open-segment kernels");

  hipStream_t strm = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const char* qb = static_cast<const char*>(q);
  const char* kb = static_cast<const char*>(k);
  const char* vb = static_cast<const char*>(v);
  char* ob = static_cast<char*>(out);
  const size_t qrow = (size_t)st->d_key * esz, vrow = (size_t)st->d_value * esz;
  infini_attn_state s = *st;
  infini_attn_open_segment o = *os;
  int64_t t = 0;
  while (t < n_tokens) {
    if (o.filled > 0 || n_tokens - t < N) {
      // into the open segment: answer the queries (the kernels also copy the new
      // keys and values into the open-segment buffers)
      const int m = (int)std::min<int64_t>(N - o.filled, n_tokens - t);
      infini::OpenAttnArgs a{qb + (size_t)t * qrow, kb + (size_t)t * qrow, vb + (size_t)t * vrow, o.k_open,
                             o.v_open, o.k_open, o.v_open, beta, s.M, s.z, ob + (size_t)t * vrow,
                             reinterpret_cast<float*>(ws + part_off), (int)BH, s.heads, N, s.d_key, s.d_value, m,
                             o.filled, 0, 0, n_tokens, s.segments_done > 0, s.dtype == INFINI_BF16, s.scale};
      const hipError_t e = infini::launch_open_attn(a, strm);
      if (e != hipSuccess) return hip_fail(e, "open-segment attention launch");
      o.filled += m;
      t += m;
      if (o.filled == N) {
        if ((rc = commit_open(&s, &o, ws, one, strm)) != INFINI_OK) return rc;
        s.segments_done += 1;
        o.filled = 0;
      }
    } else {
      // whole segments straight from the input (row stride n_tokens per (b, h))
      const int S = (int)((n_tokens - t) / N);
      if (mfma_path(&s)) {
        rc = s.d_key == 128
                 ? run_bf16<128>(&s, qb + t * qrow, kb + t * qrow, vb + t * vrow, n_tokens, S, beta,
                                 ob + t * vrow, ws, whole, strm, nullptr)
                 : run_bf16<64>(&s, qb + t * qrow, kb + t * qrow, vb + t * vrow, n_tokens, S, beta,
                                ob + t * vrow, ws, whole, strm, nullptr);
      } else {
        rc = run_f32(&s, qb + t * qrow, kb + t * qrow, vb + t * vrow, n_tokens, S, beta, ob + t * vrow, ws, whole,
                     strm, nullptr);
      }
      if (rc != INFINI_OK) return rc;
      s.segments_done += S;
      t += (int64_t)S * N;
    }
  }
  *st = s;
  *os = o;
  return ok();
}

int infini_attn_reset(infini_attn_state* st, void* stream) {
  int rc = check_state(st);
  if (rc != INFINI_OK) return rc;
  rc = zero_state(st, st->M, st->z, static_cast<hipStream_t>(stream));
  if (rc != INFINI_OK) return rc;
  st->segments_done = 0;
  return ok();
}

}  // extern "C"
