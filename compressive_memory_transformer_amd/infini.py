"""ctypes binding of libinfini_attn.so (C ABI in include/infini_attn.h).

Argument marshalling only: every step of the segment forward runs in the HIP
kernels of the library.  The functions below carry the C names without the
``infini_attn_`` prefix and take device pointers as Python ints (or torch
tensors, whose ``data_ptr()`` is used).  ``InfiniAttention`` wraps one state
together with torch-allocated M, z and workspace buffers.

The library is loaded from this package directory; there is no fallback: if it
has not been built, loading raises ``LibraryNotBuilt``.
"""

from __future__ import annotations

import ctypes
import os
import re

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
# INFINI_ATTN_LIB selects another build of the same library (the host-sanitized
# copy of the CPU checks); by default the in-tree build next to this file.
LIB_PATH = os.environ.get("INFINI_ATTN_LIB") or os.path.join(PKG_DIR, "libinfini_attn.so")
HEADER = os.path.join(os.path.dirname(PKG_DIR), "include", "infini_attn.h")

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP = 0, -1, -2, -3, -4
RULE_LINEAR, RULE_DELTA = 0, 1
F32, BF16 = 0, 1
RULES = {"linear": RULE_LINEAR, "delta": RULE_DELTA}
DTYPES = {"f32": F32, "bf16": BF16}


class LibraryNotBuilt(RuntimeError):
    pass


class InfiniError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"infini_attn error {code}: {message}")
        self.code = code
        self.message = message


class State(ctypes.Structure):
    """Mirror of infini_attn_state."""
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("heads", ctypes.c_int32),
        ("d_key", ctypes.c_int32),
        ("d_value", ctypes.c_int32),
        ("segment_len", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("rule", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("M", ctypes.c_void_p),
        ("z", ctypes.c_void_p),
        ("segments_done", ctypes.c_int64),
    ]


_lib = None


class OpenSegment(ctypes.Structure):
    """Mirror of infini_attn_open_segment."""
    _fields_ = [
        ("k_open", ctypes.c_void_p),
        ("v_open", ctypes.c_void_p),
        ("filled", ctypes.c_int32),
    ]


def load_library(path: str | None = None) -> ctypes.CDLL:
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    try:
        # torch ships its own libamdhip64; loading it first makes the library bind to
        # that same HIP runtime (matched by soname) instead of a second copy.
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(p):
        raise LibraryNotBuilt(f"{p} not found: build it with `python -m compressive_memory_transformer_amd.build`")
    lib = ctypes.CDLL(p)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    sp = ctypes.POINTER(State)
    lib.infini_attn_init_state.argtypes = [sp, i32, i32, i32, i32, i32, i32, i32, f32, vp, vp, vp]
    lib.infini_attn_init_state.restype = ctypes.c_int
    lib.infini_attn_workspace_bytes.argtypes = [sp, i64]
    lib.infini_attn_workspace_bytes.restype = sz
    lib.infini_attn_forward_sequence.argtypes = [sp, vp, vp, vp, i64, vp, vp, vp, sz, vp]
    lib.infini_attn_forward_sequence.restype = ctypes.c_int
    lib.infini_attn_forward_sequence_noalloc.argtypes = [sp, vp, vp, vp, i64, vp, vp, vp]
    lib.infini_attn_forward_sequence_noalloc.restype = ctypes.c_int
    lib.infini_attn_noalloc_scratch_bytes.argtypes = []
    lib.infini_attn_noalloc_scratch_bytes.restype = sz
    lib.infini_attn_forward_sequence_profiled.argtypes = [sp, vp, vp, vp, i64, vp, vp, vp, sz, vp,
                                                          ctypes.POINTER(vp), i32]
    lib.infini_attn_forward_sequence_profiled.restype = ctypes.c_int
    lib.infini_attn_forward_segment.argtypes = [sp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.infini_attn_forward_segment.restype = ctypes.c_int
    op = ctypes.POINTER(OpenSegment)
    lib.infini_attn_open_segment_init.argtypes = [sp, op, vp, vp]
    lib.infini_attn_open_segment_init.restype = ctypes.c_int
    lib.infini_attn_append_workspace_bytes.argtypes = [sp, i64]
    lib.infini_attn_append_workspace_bytes.restype = sz
    lib.infini_attn_append.argtypes = [sp, op, vp, vp, vp, i64, vp, vp, vp, sz, vp]
    lib.infini_attn_append.restype = ctypes.c_int
    lib.infini_attn_backward_workspace_bytes.argtypes = [sp, i64]
    lib.infini_attn_backward_workspace_bytes.restype = sz
    lib.infini_attn_backward_sequence.argtypes = [sp, vp, vp, vp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                                  vp, sz, vp]
    lib.infini_attn_backward_sequence.restype = ctypes.c_int
    lib.infini_attn_forward_sequence_train.argtypes = [sp, vp, vp, vp, i64, vp, vp, vp, vp, sz, vp]
    lib.infini_attn_forward_sequence_train.restype = ctypes.c_int
    lib.infini_attn_backward_sequence_saved.argtypes = [sp, vp, vp, vp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                                        vp, vp, vp, vp, sz, vp]
    lib.infini_attn_backward_sequence_saved.restype = ctypes.c_int
    lib.infini_attn_layer_workspace_bytes.argtypes = [sp, i32, i64]
    lib.infini_attn_layer_workspace_bytes.restype = sz
    lib.infini_attn_layer_forward.argtypes = [sp, vp, i32, vp, vp, i64, vp, vp, vp, sz, vp]
    lib.infini_attn_layer_forward.restype = ctypes.c_int
    lib.infini_attn_kernel_linear_attention.argtypes = [sp, vp, vp, vp, i64, vp, vp, sz, vp]
    lib.infini_attn_kernel_linear_attention.restype = ctypes.c_int
    lib.infini_attn_reset.argtypes = [sp, vp]
    lib.infini_attn_reset.restype = ctypes.c_int
    lib.infini_attn_last_error.argtypes = []
    lib.infini_attn_last_error.restype = ctypes.c_char_p
    lib.infini_attn_abi_version.argtypes = []
    lib.infini_attn_abi_version.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def header_functions(header: str = HEADER) -> list[str]:
    """Names of the functions declared in the C header."""
    text = open(header).read()
    return sorted(set(re.findall(r"\b(infini_attn_[a-z_]+)\s*\(", text)))


def _ptr(x) -> int | None:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _check(rc: int) -> int:
    if rc != OK:
        raise InfiniError(rc, last_error())
    return rc


def last_error() -> str:
    return load_library().infini_attn_last_error().decode()


def abi_version() -> int:
    return load_library().infini_attn_abi_version()


def init_state(st: State, batch, heads, d_key, d_value, segment_len, dtype, rule, scale, M, z, stream=None,
               check=True) -> int:
    rc = load_library().infini_attn_init_state(ctypes.byref(st), batch, heads, d_key, d_value, segment_len, dtype,
                                               rule, scale, _ptr(M), _ptr(z), stream)
    return _check(rc) if check else rc


def workspace_bytes(st: State, seq_len: int) -> int:
    return load_library().infini_attn_workspace_bytes(ctypes.byref(st), seq_len)


def forward_sequence(st: State, q, k, v, seq_len, beta, out, workspace, ws_bytes, stream=None, check=True) -> int:
    rc = load_library().infini_attn_forward_sequence(ctypes.byref(st), _ptr(q), _ptr(k), _ptr(v), seq_len,
                                                     _ptr(beta), _ptr(out), _ptr(workspace), ws_bytes, stream)
    return _check(rc) if check else rc


def forward_sequence_noalloc(st: State, q, k, v, seq_len, beta, out, stream=None, check=True) -> int:
    """forward_sequence on the library's own device scratch array (no workspace)."""
    rc = load_library().infini_attn_forward_sequence_noalloc(ctypes.byref(st), _ptr(q), _ptr(k), _ptr(v), seq_len,
                                                             _ptr(beta), _ptr(out), stream)
    return _check(rc) if check else rc


def noalloc_scratch_bytes() -> int:
    return load_library().infini_attn_noalloc_scratch_bytes()


def forward_sequence_profiled(st: State, q, k, v, seq_len, beta, out, workspace, ws_bytes, stream, events,
                              check=True) -> int:
    """forward_sequence recording the HIP events ``events`` (3 raw hipEvent_t handles)
    before the state stage, between the stages and after the attention stage."""
    arr = (ctypes.c_void_p * len(events))(*events)
    rc = load_library().infini_attn_forward_sequence_profiled(
        ctypes.byref(st), _ptr(q), _ptr(k), _ptr(v), seq_len, _ptr(beta), _ptr(out), _ptr(workspace), ws_bytes,
        stream, arr, len(events))
    return _check(rc) if check else rc


def forward_segment(st: State, q, k, v, beta, out, workspace, ws_bytes, stream=None, check=True) -> int:
    rc = load_library().infini_attn_forward_segment(ctypes.byref(st), _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                                                    _ptr(out), _ptr(workspace), ws_bytes, stream)
    return _check(rc) if check else rc


def open_segment_init(st: State, os_: OpenSegment, k_open, v_open, check=True) -> int:
    rc = load_library().infini_attn_open_segment_init(ctypes.byref(st), ctypes.byref(os_), _ptr(k_open),
                                                      _ptr(v_open))
    return _check(rc) if check else rc


def append_workspace_bytes(st: State, n_tokens: int) -> int:
    return load_library().infini_attn_append_workspace_bytes(ctypes.byref(st), n_tokens)


def append(st: State, os_: OpenSegment, q, k, v, n_tokens, beta, out, workspace, ws_bytes, stream=None,
           check=True) -> int:
    rc = load_library().infini_attn_append(ctypes.byref(st), ctypes.byref(os_), _ptr(q), _ptr(k), _ptr(v),
                                           n_tokens, _ptr(beta), _ptr(out), _ptr(workspace), ws_bytes, stream)
    return _check(rc) if check else rc


def backward_workspace_bytes(st: State, seq_len: int) -> int:
    return load_library().infini_attn_backward_workspace_bytes(ctypes.byref(st), seq_len)


def backward_sequence(st: State, q, k, v, seq_len, beta, dout, dM, dz, dq, dk, dv, dbeta, dM0, dz0, workspace,
                      ws_bytes, stream=None, check=True) -> int:
    rc = load_library().infini_attn_backward_sequence(
        ctypes.byref(st), _ptr(q), _ptr(k), _ptr(v), seq_len, _ptr(beta), _ptr(dout), _ptr(dM), _ptr(dz),
        _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dbeta), _ptr(dM0), _ptr(dz0), _ptr(workspace), ws_bytes, stream)
    return _check(rc) if check else rc


def forward_sequence_train(st: State, q, k, v, seq_len, beta, out, lse, workspace, ws_bytes, stream=None,
                           check=True) -> int:
    """forward_sequence that also writes each query row's base-2 softmax
    log-normaliser into lse (fp32 [B, H, seq_len]) for backward_sequence_saved."""
    rc = load_library().infini_attn_forward_sequence_train(ctypes.byref(st), _ptr(q), _ptr(k), _ptr(v), seq_len,
                                                           _ptr(beta), _ptr(out), _ptr(lse), _ptr(workspace),
                                                           ws_bytes, stream)
    return _check(rc) if check else rc


def backward_sequence_saved(st: State, q, k, v, seq_len, beta, out, lse, dout, dM, dz, dq, dk, dv, dbeta, dM0,
                            dz0, workspace, ws_bytes, stream=None, check=True) -> int:
    """backward_sequence given the output and lse of a forward_sequence_train call."""
    rc = load_library().infini_attn_backward_sequence_saved(
        ctypes.byref(st), _ptr(q), _ptr(k), _ptr(v), seq_len, _ptr(beta), _ptr(out), _ptr(lse), _ptr(dout),
        _ptr(dM), _ptr(dz), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dbeta), _ptr(dM0), _ptr(dz0), _ptr(workspace),
        ws_bytes, stream)
    return _check(rc) if check else rc


def layer_workspace_bytes(st: State, d_model: int, seq_len: int) -> int:
    return load_library().infini_attn_layer_workspace_bytes(ctypes.byref(st), d_model, seq_len)


def layer_forward(st: State, x, d_model, w_qkv, w_o, seq_len, beta, y, workspace, ws_bytes, stream=None,
                  check=True) -> int:
    rc = load_library().infini_attn_layer_forward(ctypes.byref(st), _ptr(x), d_model, _ptr(w_qkv), _ptr(w_o),
                                                  seq_len, _ptr(beta), _ptr(y), _ptr(workspace), ws_bytes, stream)
    return _check(rc) if check else rc


def kernel_linear_attention(st: State, q, k, v, seq_len, out, workspace, ws_bytes, stream=None, check=True) -> int:
    rc = load_library().infini_attn_kernel_linear_attention(ctypes.byref(st), _ptr(q), _ptr(k), _ptr(v), seq_len,
                                                            _ptr(out), _ptr(workspace), ws_bytes, stream)
    return _check(rc) if check else rc


def reset(st: State, stream=None, check=True) -> int:
    rc = load_library().infini_attn_reset(ctypes.byref(st), stream)
    return _check(rc) if check else rc


def _stream_handle(torch, stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


class InfiniAttention:
    """One Infini-attention state on a GPU with torch-owned buffers.

    Inputs are device tensors [B, H, L, d] of the state's dtype (torch.bfloat16
    or torch.float32); beta is a device fp32 tensor [H]."""

    def __init__(self, batch, heads, d_key, d_value, segment_len, dtype="bf16", rule="linear", scale=0.0,
                 device="cuda", stream=None):
        import torch

        self.torch = torch
        self.device = torch.device(device)
        self.dtype_code = DTYPES[dtype] if isinstance(dtype, str) else int(dtype)
        self.rule_code = RULES[rule] if isinstance(rule, str) else int(rule)
        self.M = torch.empty((batch, heads, d_key, d_value), dtype=torch.float32, device=self.device)
        self.z = torch.empty((batch, heads, d_key), dtype=torch.float32, device=self.device)
        self.state = State()
        self._ws = None
        self._ws_bytes = 0
        init_state(self.state, batch, heads, d_key, d_value, segment_len, self.dtype_code, self.rule_code,
                   float(scale), self.M, self.z, _stream_handle(torch, stream))

    @property
    def torch_dtype(self):
        return self.torch.bfloat16 if self.dtype_code == BF16 else self.torch.float32

    @property
    def segments_done(self) -> int:
        return int(self.state.segments_done)

    def workspace(self, seq_len: int):
        need = workspace_bytes(self.state, seq_len)
        if need == 0:
            raise InfiniError(EINVAL, f"no workspace size for seq_len={seq_len}")
        if self._ws_bytes < need:
            raw = self.torch.empty(need + 256, dtype=self.torch.uint8, device=self.device)
            off = (-raw.data_ptr()) % 256
            self._ws_raw, self._ws, self._ws_bytes = raw, raw[off:off + need], need
        return self._ws, self._ws_bytes

    def forward_sequence(self, q, k, v, beta, out=None, stream=None):
        seq_len = q.shape[2]
        if out is None:
            out = self.torch.empty((*q.shape[:3], v.shape[3]), dtype=q.dtype, device=q.device)
        ws, nbytes = self.workspace(seq_len)
        forward_sequence(self.state, q, k, v, seq_len, beta, out, ws, nbytes, _stream_handle(self.torch, stream))
        return out

    def forward_sequence_train(self, q, k, v, beta, out=None, lse=None, stream=None):
        """forward_sequence that also returns each query row's base-2 softmax
        log-normaliser (fp32 [B, H, L]) for backward_sequence(..., saved=(out, lse))."""
        seq_len = q.shape[2]
        if out is None:
            out = self.torch.empty((*q.shape[:3], v.shape[3]), dtype=q.dtype, device=q.device)
        if lse is None:
            lse = self.torch.empty(q.shape[:3], dtype=self.torch.float32, device=q.device)
        ws, nbytes = self.workspace(seq_len)
        forward_sequence_train(self.state, q, k, v, seq_len, beta, out, lse, ws, nbytes,
                               _stream_handle(self.torch, stream))
        return out, lse

    def forward_segment(self, q, k, v, beta, out=None, stream=None):
        if out is None:
            out = self.torch.empty((*q.shape[:3], v.shape[3]), dtype=q.dtype, device=q.device)
        ws, nbytes = self.workspace(self.state.segment_len)
        forward_segment(self.state, q, k, v, beta, out, ws, nbytes, _stream_handle(self.torch, stream))
        return out

    def reset(self, stream=None):
        reset(self.state, _stream_handle(self.torch, stream))
        if getattr(self, "open", None) is not None:
            open_segment_init(self.state, self.open, self.k_open, self.v_open)

    def open_stream(self):
        """Allocates the open-segment buffers ([B, H, N, d]) and empties the open
        segment; append() then takes tokens in any number per call."""
        B, H, N = self.state.batch, self.state.heads, self.state.segment_len
        dt = self.torch_dtype
        self.k_open = self.torch.empty((B, H, N, self.state.d_key), dtype=dt, device=self.device)
        self.v_open = self.torch.empty((B, H, N, self.state.d_value), dtype=dt, device=self.device)
        self.open = OpenSegment()
        open_segment_init(self.state, self.open, self.k_open, self.v_open)

    @property
    def filled(self) -> int:
        return int(self.open.filled)

    def append_workspace(self, n_tokens: int):
        need = append_workspace_bytes(self.state, n_tokens)
        if need == 0:
            raise InfiniError(EINVAL, f"no workspace size for n_tokens={n_tokens}")
        if self._ws_bytes < need:
            raw = self.torch.empty(need + 256, dtype=self.torch.uint8, device=self.device)
            off = (-raw.data_ptr()) % 256
            self._ws_raw, self._ws, self._ws_bytes = raw, raw[off:off + need], need
        return self._ws, self._ws_bytes

    def append(self, q, k, v, beta, out=None, stream=None):
        """Appends q.shape[2] tokens per (b, h) (see open_stream)."""
        n = q.shape[2]
        if out is None:
            out = self.torch.empty((*q.shape[:3], v.shape[3]), dtype=q.dtype, device=q.device)
        ws, nbytes = self.append_workspace(n)
        append(self.state, self.open, q, k, v, n, beta, out, ws, nbytes, _stream_handle(self.torch, stream))
        return out

    def kernel_linear_attention(self, q, k, v, out=None, stream=None):
        """Causal kernel linear attention over q.shape[2] tokens (linear-rule state;
        its segment length is the chunk)."""
        seq_len = q.shape[2]
        if out is None:
            out = self.torch.empty((*q.shape[:3], v.shape[3]), dtype=q.dtype, device=q.device)
        ws, nbytes = self.workspace(seq_len)
        kernel_linear_attention(self.state, q, k, v, seq_len, out, ws, nbytes, _stream_handle(self.torch, stream))
        return out

    def layer_forward(self, x, w_qkv, w_o, beta, y=None, stream=None):
        """y = concat_h(A_h) w_o with q, k, v = x w_qkv split into heads (x: [B, L,
        d_model] bf16; w_qkv: [d_model, H (2 d_key + d_value)]; w_o: [H d_value,
        d_model])."""
        torch = self.torch
        d_model, seq_len = x.shape[2], x.shape[1]
        if y is None:
            y = torch.empty_like(x)
        need = layer_workspace_bytes(self.state, d_model, seq_len)
        if need == 0:
            raise InfiniError(EINVAL, f"no layer workspace size for d_model={d_model}, seq_len={seq_len}")
        if self._ws_bytes < need:
            raw = torch.empty(need + 256, dtype=torch.uint8, device=self.device)
            off = (-raw.data_ptr()) % 256
            self._ws_raw, self._ws, self._ws_bytes = raw, raw[off:off + need], need
        layer_forward(self.state, x, d_model, w_qkv, w_o, seq_len, beta, y, self._ws, self._ws_bytes,
                      _stream_handle(torch, stream))
        return y

    def backward_sequence(self, q, k, v, beta, dout, M0, z0, segments_done, dM=None, dz=None, stream=None,
                          saved=None):
        """Gradients of a forward_sequence call over q, k, v, beta that started
        from the state (M0, z0, segments_done), for the output gradient dout and
        the final-state gradients dM, dz (None for zero).  With saved = (out, lse)
        from forward_sequence_train over the same call, the softmax statistics are
        not recomputed.  Returns a dict with dq, dk, dv (input dtype), dbeta [H],
        dM0 and dz0 (fp32)."""
        torch = self.torch
        st = State.from_buffer_copy(self.state)
        st.M, st.z, st.segments_done = _ptr(M0), _ptr(z0), int(segments_done)
        seq_len = q.shape[2]
        need = backward_workspace_bytes(st, seq_len)
        if need == 0:
            raise InfiniError(EINVAL, f"no backward workspace size for seq_len={seq_len}")
        raw = torch.empty(need + 256, dtype=torch.uint8, device=self.device)
        off = (-raw.data_ptr()) % 256
        ws = raw[off:off + need]
        out = {"dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v),
               "dbeta": torch.empty(self.state.heads, dtype=torch.float32, device=self.device),
               "dM0": torch.empty_like(M0), "dz0": torch.empty_like(z0)}
        if saved is None:
            backward_sequence(st, q, k, v, seq_len, beta, dout, dM, dz, out["dq"], out["dk"], out["dv"],
                              out["dbeta"], out["dM0"], out["dz0"], ws, need, _stream_handle(torch, stream))
        else:
            backward_sequence_saved(st, q, k, v, seq_len, beta, saved[0], saved[1], dout, dM, dz, out["dq"],
                                    out["dk"], out["dv"], out["dbeta"], out["dM0"], out["dz0"], ws, need,
                                    _stream_handle(torch, stream))
        out["_workspace"] = raw   # kept alive until the caller synchronises
        return out
