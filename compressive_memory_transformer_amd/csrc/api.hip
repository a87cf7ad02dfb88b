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
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

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
  if (dtype == INFINI_BF16) {
    if (dk != dv || (dk != 64 && dk != 128))
      return fail(INFINI_EUNSUPPORTED, "bf16 path needs d_key == d_value in {64, 128} (got %d, %d)", dk, dv);
    if (N % 64 != 0) return fail(INFINI_EUNSUPPORTED, "bf16 path needs segment_len %% 64 == 0 (got %d)", N);
  } else {
    if (dk > 128 || dv > 128)
      return fail(INFINI_EUNSUPPORTED, "fp32 path supports d_key, d_value <= 128 (got %d, %d)", dk, dv);
    if (N > 4096) return fail(INFINI_EUNSUPPORTED, "fp32 path supports segment_len <= 4096 (got %d)", N);
  }
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
  size_t snapM = 0, snapz = 0, snapc = 0, cM = 0, cz = 0, kp = 0, czp = 0, inv = 0, U = 0, total = 0;
};

// Workspace regions, each 256-byte aligned.  Returns false on overflow.
bool workspace_layout(const infini_attn_state* st, int64_t S, WsLayout* w) {
  const int64_t BH = (int64_t)st->batch * st->heads;
  int64_t seg_heads, n;
  if (!mul_ok(BH, S, &seg_heads)) return false;
  size_t off = 0;
  if (st->dtype == INFINI_BF16) {
    const int64_t D = st->d_key;
    if (!mul_ok(seg_heads, D * D, &n)) return false;
    w->snapM = off; off = align_up(off + (size_t)n * 2);
    w->snapz = off; off = align_up(off + (size_t)(seg_heads * D) * 4);
    w->snapc = off; off = align_up(off + (size_t)(seg_heads * D) * 4);
    if (st->rule == INFINI_RULE_LINEAR) {
      w->cM = off; off = align_up(off + (size_t)n * 4);
      w->cz = off; off = align_up(off + (size_t)(seg_heads * D) * 4);
    } else {
      int64_t tokens, parts;
      if (!mul_ok(BH, S * (int64_t)st->segment_len, &tokens)) return false;
      if (!mul_ok(seg_heads, D, &parts)) return false;
      w->kp = off; off = align_up(off + (size_t)tokens * D * 2);
      w->czp = off; off = align_up(off + (size_t)parts * 4);
      w->inv = off; off = align_up(off + (size_t)tokens * 4);
    }
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

template <int D>
int run_bf16(infini_attn_state* st, const void* q, const void* k, const void* v, int64_t L, int S,
             const float* beta, void* out, char* ws, const WsLayout& w, hipStream_t stream,
             void* const* events) {
  int rc;
  if ((rc = record(events, 0, stream)) != INFINI_OK) return rc;
  using infini::bf16;
  const int B = st->batch, H = st->heads, N = st->segment_len;
  bf16* snapM = reinterpret_cast<bf16*>(ws + w.snapM);
  float* snapz = reinterpret_cast<float*>(ws + w.snapz);
  float* snapc = reinterpret_cast<float*>(ws + w.snapc);
  hipError_t e;
  if (st->rule == INFINI_RULE_LINEAR) {
    infini::LinContribArgs c{static_cast<const bf16*>(k), static_cast<const bf16*>(v),
                             reinterpret_cast<float*>(ws + w.cM), reinterpret_cast<float*>(ws + w.cz),
                             B, H, S, N, L};
    if ((e = infini::launch_lin_contrib<D>(c, stream)) != hipSuccess) return hip_fail(e, "lin_contrib launch");
    infini::LinScanArgs sarg{c.cM, c.cz, st->M, st->z, snapM, snapz, snapc, B * H, S};
    if ((e = infini::launch_lin_scan<D>(sarg, stream)) != hipSuccess) return hip_fail(e, "lin_scan launch");
  } else {
    infini::DeltaArgs d{static_cast<const bf16*>(k), static_cast<const bf16*>(v), st->M, st->z, snapM, snapz,
                        snapc, reinterpret_cast<bf16*>(ws + w.kp), reinterpret_cast<float*>(ws + w.czp),
                        reinterpret_cast<float*>(ws + w.inv), B * H, S, N, L, st->segments_done, 0};
    if ((e = infini::launch_delta_state<D>(d, stream)) != hipSuccess) return hip_fail(e, "delta state launch");
  }
  if ((rc = record(events, 1, stream)) != INFINI_OK) return rc;
  infini::FaArgs f{static_cast<const bf16*>(q), static_cast<const bf16*>(k), static_cast<const bf16*>(v), beta,
                   snapM, snapz, snapc, static_cast<bf16*>(out), B, H, S, N, L, 0,
                   st->segments_done, (float)((double)st->scale * 1.4426950408889634)};
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
    infini::F32AttnArgs a{static_cast<const float*>(q), static_cast<const float*>(k), static_cast<const float*>(v),
                          beta, st->M, st->z, static_cast<float*>(out), st->heads, BH, N, st->d_key, st->d_value,
                          L, off, has_memory, st->scale};
    hipError_t e = infini::launch_f32_attn(a, stream);
    if (e != hipSuccess) return hip_fail(e, "f32 attention launch");
    infini::F32UpdateArgs u{static_cast<const float*>(k), static_cast<const float*>(v), st->M, st->z,
                            reinterpret_cast<float*>(ws + w.U), BH, N, st->d_key, st->d_value, L, off,
                            st->rule == INFINI_RULE_DELTA, has_memory};
    e = infini::launch_f32_update(u, stream);
    if (e != hipSuccess) return hip_fail(e, "f32 update launch");
  }
  if ((rc = record(events, 1, stream)) != INFINI_OK) return rc;
  return record(events, 2, stream);
}

int zero_state(infini_attn_state* st, float* M, float* z, hipStream_t stream) {
  const int64_t BH = (int64_t)st->batch * st->heads;
  const hipError_t e = infini::launch_fill_zero(M, BH * st->d_key * st->d_value, z, BH * st->d_key, stream);
  if (e != hipSuccess) return hip_fail(e, "fill launch");
  return INFINI_OK;
}

}  // namespace

extern "C" {

int infini_attn_abi_version(void) { return 1; }

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
  if (!workspace_layout(st, seq_len / st->segment_len, &w)) return 0;
  return w.total;
}

static int forward_impl(infini_attn_state* st, const void* q, const void* k, const void* v, int64_t seq_len,
                        const float* beta, void* out, void* workspace, size_t workspace_bytes, void* stream,
                        void* const* events) {
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
  if (!workspace_layout(st, S, &w)) return fail(INFINI_EINVAL, "workspace size overflows");
  if (!workspace || workspace_bytes < w.total)
    return fail(INFINI_EWORKSPACE, "workspace of %zu bytes required, %zu given%s", w.total, workspace_bytes,
                workspace ? "" : " (NULL)");
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0)
    return fail(INFINI_EWORKSPACE, "workspace must be 256-byte aligned");
  if (overlaps(workspace, w.total, out, out_bytes) || overlaps(workspace, w.total, st->M, m_bytes) ||
      overlaps(workspace, w.total, st->z, z_bytes))
    return fail(INFINI_EWORKSPACE, "workspace must not alias out or the state");
  if (st->dtype == INFINI_BF16) {
    const int64_t fa_blocks = infini::fa_fwd_blocks(BH * S64, st->segment_len);
    if (fa_blocks > 0x7fffffff) return fail(INFINI_EUNSUPPORTED, "launch grid too large; split the call");
  }

  hipStream_t strm = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  if (st->dtype == INFINI_BF16) {
    rc = st->d_key == 128 ? run_bf16<128>(st, q, k, v, seq_len, S, beta, out, ws, w, strm, events)
                          : run_bf16<64>(st, q, k, v, seq_len, S, beta, out, ws, w, strm, events);
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

int infini_attn_forward_sequence_profiled(infini_attn_state* st, const void* q, const void* k, const void* v,
                                          int64_t seq_len, const float* beta, void* out, void* workspace,
                                          size_t workspace_bytes, void* stream, void* const* events,
                                          int32_t n_events) {
  if (!events || n_events != 3 || !events[0] || !events[1] || !events[2])
    return fail(INFINI_EINVAL, "profiled forward needs exactly 3 non-NULL events");
  return forward_impl(st, q, k, v, seq_len, beta, out, workspace, workspace_bytes, stream, events);
}

int infini_attn_forward_segment(infini_attn_state* st, const void* q, const void* k, const void* v,
                                const float* beta, void* out, void* workspace, size_t workspace_bytes,
                                void* stream) {
  if (!st) return fail(INFINI_EINVAL, "state pointer is NULL");
  return infini_attn_forward_sequence(st, q, k, v, st->segment_len, beta, out, workspace, workspace_bytes, stream);
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
