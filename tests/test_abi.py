"""The C ABI on the CPU: the library loads, exports every declared function, and
rejects invalid arguments before any HIP call (no GPU is needed for these)."""

import ctypes
import subprocess

import pytest

from compressive_memory_transformer_amd import infini as ia

pytestmark = pytest.mark.skipif(not __import__("os").path.exists(ia.LIB_PATH),
                                reason="library not built")

FAKE = 1 << 40  # never dereferenced: every call below fails validation first


def _state(**over):
    st = ia.State()
    vals = dict(batch=1, heads=2, d_key=128, d_value=128, segment_len=2048, dtype=ia.BF16,
                rule=ia.RULE_LINEAR, scale=0.08838834764831845, M=FAKE, z=FAKE * 2, segments_done=0)
    vals.update(over)
    for k, v in vals.items():
        setattr(st, k, v)
    return st


def _snapshot(st):
    return tuple(getattr(st, f) for f, _ in ia.State._fields_)


def test_exports_every_declared_function():
    lib = ia.load_library()
    names = ia.header_functions()
    assert len(names) == 20
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", ia.LIB_PATH], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(names) <= exported
    assert ia.abi_version() == 1


def test_struct_layout_matches_header():
    assert ctypes.sizeof(ia.State) == 56
    assert ia.State.M.offset == 32 and ia.State.segments_done.offset == 48
    assert ctypes.sizeof(ia.OpenSegment) == 24 and ia.OpenSegment.filled.offset == 16


@pytest.mark.parametrize("args,code", [
    ((0, 2, 128, 128, 2048, ia.BF16, ia.RULE_LINEAR), ia.EINVAL),
    ((1, 0, 128, 128, 2048, ia.BF16, ia.RULE_LINEAR), ia.EINVAL),
    ((1, 2, 128, 128, 0, ia.BF16, ia.RULE_LINEAR), ia.EINVAL),
    ((1, 2, 128, 128, 2048, 7, ia.RULE_LINEAR), ia.EINVAL),
    ((1, 2, 128, 128, 2048, ia.BF16, 9), ia.EINVAL),
    ((1, 2, 256, 256, 2048, ia.BF16, ia.RULE_DELTA), ia.EUNSUPPORTED),
    ((1, 2, 96, 96, 8192, ia.BF16, ia.RULE_DELTA), ia.EUNSUPPORTED),
    ((1, 2, 128, 64, 8192, ia.BF16, ia.RULE_LINEAR), ia.EUNSUPPORTED),
    ((1, 2, 256, 32, 64, ia.F32, ia.RULE_LINEAR), ia.EUNSUPPORTED),
    ((1, 2, 32, 32, 8192, ia.F32, ia.RULE_LINEAR), ia.EUNSUPPORTED),
])
def test_init_state_rejects_bad_config(args, code):
    st = ia.State()
    before = _snapshot(st)
    rc = ia.init_state(st, *args, 0.0, FAKE, FAKE * 2, None, check=False)
    assert rc == code
    assert ia.last_error()
    assert _snapshot(st) == before


def test_init_state_rejects_null_and_inf():
    st = ia.State()
    assert ia.init_state(st, 1, 2, 32, 32, 64, ia.F32, 0, 0.0, None, FAKE, None, check=False) == ia.EINVAL
    assert ia.init_state(st, 1, 2, 32, 32, 64, ia.F32, 0, float("inf"), FAKE, FAKE * 2, None,
                         check=False) == ia.EINVAL
    assert ia.load_library().infini_attn_init_state(None, 1, 2, 32, 32, 64, 0, 0, 0.0, FAKE, FAKE, None) == ia.EINVAL


def test_workspace_bytes():
    st = _state(rule=ia.RULE_LINEAR)
    S, D, BH = 16, 128, 2
    # snapshots (bf16 M^T and its bf16 remainder, z, column sums), contributions C_s^T and c_s
    want = 2 * BH * S * D * D * 2 + 2 * BH * S * D * 4 + BH * S * D * D * 4 + BH * S * D * 4
    assert ia.workspace_bytes(st, S * 2048) == want
    st = _state(rule=ia.RULE_DELTA)
    L = S * 2048
    # snapshots, the contributions C_s^T and c_s, then A_s per segment as two bf16 parts
    want = 2 * BH * S * D * D * 2 + 2 * BH * S * D * 4 + BH * S * D * D * 4 + BH * S * D * 4 + BH * S * D * D * 4
    assert ia.workspace_bytes(st, L) == want
    assert ia.workspace_bytes(st, 2047) == 0
    assert ia.workspace_bytes(st, 0) == 0
    assert ia.workspace_bytes(_state(batch=0), 2048) == 0
    f32 = _state(dtype=ia.F32, d_key=32, d_value=16, segment_len=64, rule=ia.RULE_DELTA)
    assert ia.workspace_bytes(f32, 256) == 2 * 64 * 16 * 4
    assert ia.workspace_bytes(_state(dtype=ia.F32, d_key=32, d_value=32, segment_len=64), 256) == 256


@pytest.mark.parametrize("case", ["null_q", "null_beta", "ragged", "zero_len", "small_ws", "null_ws",
                                  "misaligned", "alias_out", "alias_state", "bad_state", "uninit"])
def test_forward_rejects_bad_arguments(case):
    st = _state()
    L = 2 * 2048
    need = ia.workspace_bytes(st, L)
    q, k, v, beta = FAKE * 4, FAKE * 5, FAKE * 6, FAKE * 7
    out, ws, nbytes = FAKE * 8, FAKE * 9, need
    expect = ia.EINVAL
    if case == "null_q":
        q = None
    elif case == "null_beta":
        beta = None
    elif case == "ragged":
        L = 2048 + 64
    elif case == "zero_len":
        L = 0
    elif case == "small_ws":
        nbytes, expect = need - 1, ia.EWORKSPACE
    elif case == "null_ws":
        ws, expect = None, ia.EWORKSPACE
    elif case == "misaligned":
        q = FAKE * 4 + 2
    elif case == "alias_out":
        out = k + 1024
    elif case == "alias_state":
        out = st.M - 64
    elif case == "bad_state":
        st.d_key = 200
        expect = ia.EUNSUPPORTED
    elif case == "uninit":
        st = ia.State()
    before = _snapshot(st)
    rc = ia.forward_sequence(st, q, k, v, L, beta, out, ws, nbytes, None, check=False)
    assert rc == expect, ia.last_error()
    assert ia.last_error()
    assert _snapshot(st) == before


def test_profiled_needs_three_events():
    st = _state()
    L = 2048
    need = ia.workspace_bytes(st, L)
    args = (st, FAKE * 4, FAKE * 5, FAKE * 6, L, FAKE * 7, FAKE * 8, FAKE * 9, need, None)
    assert ia.forward_sequence_profiled(*args, [FAKE, FAKE], check=False) == ia.EINVAL
    assert ia.forward_sequence_profiled(*args, [FAKE, None, FAKE], check=False) == ia.EINVAL


def test_segment_and_reset_validate():
    st = _state()
    before = _snapshot(st)
    assert ia.forward_segment(st, None, FAKE, FAKE, FAKE, FAKE, FAKE, 1, None, check=False) == ia.EINVAL
    assert ia.reset(ia.State(), None, check=False) == ia.EINVAL
    assert ia.load_library().infini_attn_reset(None, None) == ia.EINVAL
    assert _snapshot(st) == before


def _open(st, filled=0):
    os_ = ia.OpenSegment()
    assert ia.open_segment_init(st, os_, FAKE * 10, FAKE * 12, check=False) == ia.OK
    os_.filled = filled
    return os_


def test_open_segment_init_validates():
    st = _state()
    os_ = ia.OpenSegment()
    assert ia.open_segment_init(st, os_, None, FAKE, check=False) == ia.EINVAL
    assert ia.open_segment_init(st, os_, FAKE * 10 + 2, FAKE * 12, check=False) == ia.EINVAL
    assert ia.open_segment_init(st, os_, FAKE * 10, FAKE * 10 + 4096, check=False) == ia.EINVAL  # overlap
    assert ia.open_segment_init(ia.State(), os_, FAKE * 10, FAKE * 12, check=False) == ia.EINVAL
    assert ia.load_library().infini_attn_open_segment_init(ctypes.byref(st), None, FAKE, FAKE * 2) == ia.EINVAL
    os_.filled = 7
    assert ia.open_segment_init(st, os_, FAKE * 10, FAKE * 12) == ia.OK
    assert os_.filled == 0 and os_.k_open == FAKE * 10 and os_.v_open == FAKE * 12


def test_append_workspace_bytes():
    st = _state()                       # bf16, linear, N = 2048, BH = 2, d = 128
    one = ia.workspace_bytes(st, 2048)  # the commit of one segment
    parts = 2 * 1 * 16 * 130 * 4        # one query: 16 key partitions of d_value + 2 floats
    assert ia.append_workspace_bytes(st, 1) == max(one, -(-parts // 256) * 256)
    assert ia.append_workspace_bytes(st, 3 * 2048 + 5) >= ia.workspace_bytes(st, 3 * 2048)
    assert ia.append_workspace_bytes(st, 0) == 0
    assert ia.append_workspace_bytes(ia.State(), 1) == 0


@pytest.mark.parametrize("case", ["null_q", "null_os", "zero_len", "filled_range", "unbound", "small_ws",
                                  "misaligned", "alias_open", "alias_state"])
def test_append_rejects_bad_arguments(case):
    st = _state()
    os_ = _open(st, filled=5)
    n = 3
    need = ia.append_workspace_bytes(st, n)
    q, k, v, beta = FAKE * 4, FAKE * 5, FAKE * 6, FAKE * 7
    out, ws, nbytes = FAKE * 8, FAKE * 9, need
    expect = ia.EINVAL
    if case == "null_q":
        q = None
    elif case == "null_os":
        os_ = None
    elif case == "zero_len":
        n = 0
    elif case == "filled_range":
        os_.filled = 2048
    elif case == "unbound":
        os_ = ia.OpenSegment()
    elif case == "small_ws":
        nbytes, expect = need - 1, ia.EWORKSPACE
    elif case == "misaligned":
        v = FAKE * 6 + 8
    elif case == "alias_open":
        out = FAKE * 12 + 512
    elif case == "alias_state":
        out = st.z
    before = _snapshot(st)
    fill_before = None if os_ is None else os_.filled
    lib = ia.load_library()
    rc = lib.infini_attn_append(ctypes.byref(st), None if os_ is None else ctypes.byref(os_), q, k, v, n, beta, out,
                                ws, nbytes, None)
    assert rc == expect, ia.last_error()
    assert ia.last_error()
    assert _snapshot(st) == before
    if os_ is not None:
        assert os_.filled == fill_before


def test_backward_workspace_bytes():
    st = _state(rule=ia.RULE_DELTA)
    S, D, BH, N = 4, 128, 2, 2048
    L = S * N
    mm, seg, rows = BH * S * D * D, BH * S * D, BH * L
    # snapshots, retrieval gradients of M and (delta, bf16) A_s; four per-segment d_key vectors, five per-row
    # scalars, three per-row accumulators (the bf16 MFMA path writes dq without one), the dbeta shares (64
    # query blocks per segment), and on that path the Gram kernels' second-half partials (one d_key x d_value
    # matrix and one d_key vector per segment)
    want = 4 * (3 * mm + 4 * seg + 5 * rows + 3 * rows * D + BH * S * 64 + mm + seg)
    assert ia.backward_workspace_bytes(st, L) == want
    assert ia.backward_workspace_bytes(st, L + 1) == 0
    assert ia.backward_workspace_bytes(_state(batch=0), L) == 0


@pytest.mark.parametrize("case", ["null_dout", "null_dq", "ragged", "small_ws", "alias_out_in", "alias_outs",
                                  "alias_ws_state", "misaligned_beta", "misaligned_q", "misaligned_dv",
                                  "bad_state"])
def test_backward_rejects_bad_arguments(case):
    st = _state()
    L = 2 * 2048
    need = ia.backward_workspace_bytes(st, L)
    q, k, v, beta, dout = FAKE * 4, FAKE * 5, FAKE * 6, FAKE * 7, FAKE * 8
    dq, dk, dv, dbeta, dM0, dz0 = FAKE * 9, FAKE * 10, FAKE * 11, FAKE * 12, FAKE * 13, FAKE * 14
    dM, dz, ws, nbytes = None, None, FAKE * 15, need
    expect = ia.EINVAL
    if case == "null_dout":
        dout = None
    elif case == "null_dq":
        dq = None
    elif case == "ragged":
        L = 2048 + 64
    elif case == "small_ws":
        nbytes, expect = need - 1, ia.EWORKSPACE
    elif case == "alias_out_in":
        dk = k + 64
    elif case == "alias_outs":
        dv = dq + 64
    elif case == "alias_ws_state":
        ws = st.M - 256 * 4
    elif case == "misaligned_beta":
        beta = FAKE * 7 + 2
    elif case == "misaligned_q":
        q = FAKE * 4 + 8      # 8-byte aligned: the bf16 kernels read 16-byte row pieces
    elif case == "misaligned_dv":
        dv = FAKE * 11 + 2
    elif case == "bad_state":
        st.d_key = 200
        expect = ia.EUNSUPPORTED
    before = _snapshot(st)
    rc = ia.backward_sequence(st, q, k, v, L, beta, dout, dM, dz, dq, dk, dv, dbeta, dM0, dz0, ws, nbytes, None,
                              check=False)
    assert rc == expect, (case, ia.last_error())
    assert ia.last_error()
    assert _snapshot(st) == before


@pytest.mark.parametrize("case", ["null_lse", "f32", "misaligned_lse", "alias_lse_out", "alias_lse_ws",
                                  "small_ws"])
def test_forward_train_rejects_bad_arguments(case):
    st = _state()
    L = 2 * 2048
    need = ia.workspace_bytes(st, L)
    q, k, v, beta, out, lse, ws, nbytes = FAKE * 4, FAKE * 5, FAKE * 6, FAKE * 7, FAKE * 8, FAKE * 9, FAKE * 10, need
    expect = ia.EINVAL
    if case == "null_lse":
        lse = None
    elif case == "f32":
        st = _state(dtype=ia.F32, d_key=32, d_value=32, segment_len=64)
        L, nbytes, expect = 128, ia.workspace_bytes(st, 128), ia.EUNSUPPORTED
    elif case == "misaligned_lse":
        lse = FAKE * 9 + 2
    elif case == "alias_lse_out":
        lse = out + 1024
    elif case == "alias_lse_ws":
        lse = ws + 4096
    elif case == "small_ws":
        nbytes, expect = need - 1, ia.EWORKSPACE
    before = _snapshot(st)
    rc = ia.forward_sequence_train(st, q, k, v, L, beta, out, lse, ws, nbytes, None, check=False)
    assert rc == expect, (case, ia.last_error())
    assert ia.last_error()
    assert _snapshot(st) == before


@pytest.mark.parametrize("case", ["null_out", "null_lse", "f32", "misaligned_out", "misaligned_lse",
                                  "alias_dq_out", "alias_ws_lse", "small_ws"])
def test_backward_saved_rejects_bad_arguments(case):
    st = _state()
    L = 2 * 2048
    need = ia.backward_workspace_bytes(st, L)
    q, k, v, beta, dout = FAKE * 4, FAKE * 5, FAKE * 6, FAKE * 7, FAKE * 8
    dq, dk, dv, dbeta, dM0, dz0 = FAKE * 9, FAKE * 10, FAKE * 11, FAKE * 12, FAKE * 13, FAKE * 14
    out, lse = FAKE * 16, FAKE * 17
    dM, dz, ws, nbytes = None, None, FAKE * 15, need
    expect = ia.EINVAL
    if case == "null_out":
        out = None
    elif case == "null_lse":
        lse = None
    elif case == "f32":
        st = _state(dtype=ia.F32, d_key=32, d_value=32, segment_len=64)
        L, nbytes, expect = 128, ia.backward_workspace_bytes(st, 128), ia.EUNSUPPORTED
    elif case == "misaligned_out":
        out = FAKE * 16 + 8
    elif case == "misaligned_lse":
        lse = FAKE * 17 + 2
    elif case == "alias_dq_out":
        dq = out + 64
    elif case == "alias_ws_lse":
        lse = ws + 4096
    elif case == "small_ws":
        nbytes, expect = need - 1, ia.EWORKSPACE
    before = _snapshot(st)
    rc = ia.backward_sequence_saved(st, q, k, v, L, beta, out, lse, dout, dM, dz, dq, dk, dv, dbeta, dM0, dz0, ws,
                                    nbytes, None, check=False)
    assert rc == expect, (case, ia.last_error())
    assert ia.last_error()
    assert _snapshot(st) == before


def test_layer_workspace_bytes():
    st = _state()
    L, BH, D = 2 * 2048, 2, 128
    fwd = ia.workspace_bytes(st, L)
    assert ia.layer_workspace_bytes(st, 1024, L) == 4 * BH * L * D * 2 + fwd
    assert ia.layer_workspace_bytes(st, 1000, L) == 0
    assert ia.layer_workspace_bytes(_state(dtype=ia.F32, d_key=32, d_value=32, segment_len=64), 64, 128) == 0


@pytest.mark.parametrize("case", ["null_x", "bad_dmodel", "f32", "ragged", "misaligned", "small_ws", "alias_y",
                                  "alias_ws"])
def test_layer_rejects_bad_arguments(case):
    st = _state()
    L, dm = 2 * 2048, 1024
    need = ia.layer_workspace_bytes(st, dm, L)
    x, wq, wo, beta, y, ws, nbytes = FAKE * 4, FAKE * 5, FAKE * 6, FAKE * 7, FAKE * 8, FAKE * 9, need
    expect = ia.EINVAL
    if case == "null_x":
        x = None
    elif case == "bad_dmodel":
        dm, expect = 1000, ia.EUNSUPPORTED
    elif case == "f32":
        st = _state(dtype=ia.F32, d_key=32, d_value=32, segment_len=64)
        expect = ia.EUNSUPPORTED
    elif case == "ragged":
        L = 2048 + 64
    elif case == "misaligned":
        wq = FAKE * 5 + 8
    elif case == "small_ws":
        nbytes, expect = need - 1, ia.EWORKSPACE
    elif case == "alias_y":
        y = x + 4096
    elif case == "alias_ws":
        ws, expect = x + 256 * 16, ia.EWORKSPACE
    before = _snapshot(st)
    rc = ia.layer_forward(st, x, dm, wq, wo, L, beta, y, ws, nbytes, None, check=False)
    assert rc == expect, (case, ia.last_error())
    assert ia.last_error()
    assert _snapshot(st) == before


@pytest.mark.parametrize("case", ["null_q", "f32", "delta", "ragged", "misaligned", "small_ws", "alias_out"])
def test_kernel_linear_attention_rejects_bad_arguments(case):
    st = _state()
    L = 2 * 2048
    need = ia.workspace_bytes(st, L)
    q, k, v, out, ws, nbytes = FAKE * 4, FAKE * 5, FAKE * 6, FAKE * 7, FAKE * 8, need
    expect = ia.EINVAL
    if case == "null_q":
        q = None
    elif case == "f32":
        st = _state(dtype=ia.F32, d_key=32, d_value=32, segment_len=64)
        expect = ia.EUNSUPPORTED
    elif case == "delta":
        st = _state(rule=ia.RULE_DELTA)
    elif case == "ragged":
        L = 2048 + 64
    elif case == "misaligned":
        k = FAKE * 5 + 2
    elif case == "small_ws":
        nbytes, expect = need - 1, ia.EWORKSPACE
    elif case == "alias_out":
        out = v + 512
    before = _snapshot(st)
    rc = ia.kernel_linear_attention(st, q, k, v, L, out, ws, nbytes, None, check=False)
    assert rc == expect, (case, ia.last_error())
    assert _snapshot(st) == before


def test_noalloc_rejects_oversized_and_bad_calls():
    """The allocation-free forward checks the call's workspace against its fixed
    scratch array (64 MiB) before any HIP call."""
    assert ia.noalloc_scratch_bytes() == 64 << 20
    st = _state(heads=32)                       # 32 heads x 256 segments of 2048: far above 64 MiB
    before = _snapshot(st)
    rc = ia.forward_sequence_noalloc(st, FAKE * 4, FAKE * 5, FAKE * 6, 256 * 2048, FAKE * 7, FAKE * 8, None,
                                     check=False)
    assert rc == ia.EWORKSPACE and "scratch" in ia.last_error()
    assert _snapshot(st) == before
    rc = ia.forward_sequence_noalloc(st, FAKE * 4, FAKE * 5, FAKE * 6, 2047, FAKE * 7, FAKE * 8, None, check=False)
    assert rc == ia.EINVAL
    rc = ia.forward_sequence_noalloc(_state(d_key=200), FAKE * 4, FAKE * 5, FAKE * 6, 2048, FAKE * 7, FAKE * 8, None,
                                     check=False)
    assert rc == ia.EUNSUPPORTED
