"""The C-ABI library without a GPU: it loads, exports every symbol include/mtpv.h
declares, sizes workspaces, and its host-side validation returns each error code.
No compute call is made here."""
import ctypes
import os
import re

import pytest

import mtp_draft_verification_amd as mv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mtpv.h")

# synthetic, well-aligned fake device addresses: validation never dereferences them
A = 0x10000
WS = 0x200000


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"MTPV_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_symbol():
    L = mv.lib()
    names = declared_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(mv.EXPORTED)
    assert L.mtpv_version() >= 100


def test_status_strings():
    for code in mv.STATUS:
        s = mv.status_string(code)
        assert isinstance(s, str) and s
    assert mv.status_string(12345) == "unknown status"


def ws_bytes(mode=0, B=2, k=3, H=256, V=1000, dtype=0):
    return mv.workspace_bytes(B, k, H, V, dtype, mode)


def test_workspace_sizes():
    g = ws_bytes(0)
    s = ws_bytes(1)
    d = ws_bytes(2)
    assert g > 0 and s > g and d > 0
    # sample mode holds the fp32 logit spill for all target and drafter rows
    assert s >= (2 * 4 + 2 * 3) * 1000 * 4
    assert ws_bytes(0, V=0) == 0 and ws_bytes(0, H=12) == 0 and ws_bytes(5) == 0
    assert ws_bytes(2, k=0) == 0
    # full-size shapes fit comfortably in one GPU's HBM
    assert mv.workspace_bytes(256, 3, 7168, 129280, 0, 1) < 2 << 30


def check(**kw):
    args = dict(mode=0, B=2, k=3, H=256, V=1000, dtype=0, temperature=1.0, target_hidden=A, draft_hidden=A,
                W=A, drafts=A, accepted_len=A, out_tokens=A, workspace=WS, ws_bytes=None)
    args.update(kw)
    if args["ws_bytes"] is None:
        args["ws_bytes"] = max(1, ws_bytes(max(0, min(2, args["mode"])), max(1, args["B"]), max(0, args["k"]),
                                           args["H"] if args["H"] % 8 == 0 and args["H"] >= 8 else 256,
                                           max(1, args["V"]), 0))
    return mv.check_args(args["mode"], args["B"], args["k"], args["H"], args["V"], args["dtype"],
                         args["temperature"], args["target_hidden"], args["draft_hidden"], args["W"],
                         args["drafts"], args["accepted_len"], args["out_tokens"], args["workspace"],
                         args["ws_bytes"])


def test_valid_arguments_pass():
    assert check() == 0
    assert check(mode=1, temperature=0.7) == 0
    assert check(mode=2, target_hidden=None, accepted_len=None, out_tokens=None) == 0
    assert check(k=0, drafts=None) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), -1), (dict(k=-1), -1), (dict(k=65), -1), (dict(V=0), -1), (dict(H=0), -1),
    (dict(mode=7), -1), (dict(mode=1, temperature=0.0), -1), (dict(mode=1, temperature=float("nan")), -1),
    (dict(mode=1, temperature=-1.0), -1), (dict(mode=2, k=0), -1),
    (dict(H=260), -2), (dict(W=A + 8), -2), (dict(target_hidden=A + 4), -2), (dict(drafts=A + 2), -2),
    (dict(workspace=None), -3), (dict(workspace=WS + 64), -3), (dict(ws_bytes=16), -3),
    (dict(dtype=2), -4), (dict(dtype=-1), -4),
    (dict(W=None), -7), (dict(target_hidden=None), -7), (dict(drafts=None), -7),
    (dict(accepted_len=None), -7), (dict(out_tokens=None), -7),
    (dict(mode=1, draft_hidden=None), -7), (dict(mode=2, draft_hidden=None), -7),
])
def test_each_error_code(kw, code):
    assert check(**kw) == code


def test_greedy_ignores_temperature():
    assert check(temperature=0.0) == 0


def test_calls_reject_bad_arguments_before_touching_the_device():
    """The compute entry points validate on the host first: with invalid sizes they
    return the error without enqueueing anything (so this runs without a GPU)."""
    L = mv.lib()
    st = L.spec_verify_greedy(ctypes.c_void_p(A), ctypes.c_void_p(A), ctypes.c_void_p(A), 0, 3, 256, 1000, 0,
                              ctypes.c_void_p(A), ctypes.c_void_p(A), ctypes.c_void_p(WS), 1 << 20, None, None)
    assert st == -1
    st = L.spec_verify_sample(ctypes.c_void_p(A), ctypes.c_void_p(A), ctypes.c_void_p(A), ctypes.c_void_p(A), 2,
                              3, 256, 1000, 0, -1.0, 0, 0, ctypes.c_void_p(A), ctypes.c_void_p(A),
                              ctypes.c_void_p(WS), 1 << 30, None, None)
    assert st == -1
    st = L.spec_draft_sample(ctypes.c_void_p(A), ctypes.c_void_p(A), 2, 3, -1, 256, 1000, 0, 1.0, 0, 0,
                             ctypes.c_void_p(A), ctypes.c_void_p(WS), 1 << 30, None, None)
    assert st == -1
    assert L.mtpv_copy_bytes(ctypes.c_void_p(A), ctypes.c_void_p(A + 4), 16, None) == -2


def test_rate_probes_validate_on_the_host():
    """The achievable-rate probes reject NULL (MTPV_ENULL = -7), misaligned (-2) and
    out-of-range (-1) arguments without launching; a zero-byte read launches nothing."""
    L = mv.lib()
    vp = ctypes.c_void_p
    flops = ctypes.c_int64(-1)
    assert L.mtpv_read_bytes(None, 16, vp(A), None) == -7
    assert L.mtpv_read_bytes(vp(A), 16, None, None) == -7
    assert L.mtpv_read_bytes(vp(A + 4), 16, vp(A), None) == -2
    assert L.mtpv_read_bytes(vp(A), 24, vp(A), None) == -2
    assert L.mtpv_read_bytes(vp(A), 16, vp(A + 2), None) == -2
    assert L.mtpv_read_bytes(vp(A), 0, vp(A), None) == 0
    assert L.mtpv_mfma_rate(16, None, ctypes.byref(flops), None) == -7
    assert L.mtpv_mfma_rate(16, vp(A), None, None) == -7
    assert L.mtpv_mfma_rate(16, vp(A + 1), ctypes.byref(flops), None) == -2
    assert L.mtpv_mfma_rate(0, vp(A), ctypes.byref(flops), None) == -1
    assert L.mtpv_mfma_rate((1 << 24) + 1, vp(A), ctypes.byref(flops), None) == -1
    assert flops.value == -1


def test_ragged_and_dual_calls_validate_on_the_host():
    """The per-request-length and dual entry points return the host-side errors (bad
    sizes, NULL or misaligned draft_len / greedy outputs, small workspace) without
    enqueueing anything."""
    L = mv.lib()
    vp = ctypes.c_void_p
    ws_small = 1024
    # invalid B
    assert L.spec_verify_greedy_ragged(vp(A), vp(A), vp(A), vp(A), 0, 3, 256, 1000, 0, vp(A), vp(A), vp(WS),
                                       1 << 30, None, None) == -1
    # misaligned draft_len
    assert L.spec_verify_greedy_ragged(vp(A), vp(A), vp(A), vp(A + 2), 2, 3, 256, 1000, 0, vp(A), vp(A), vp(WS),
                                       1 << 30, None, None) == -2
    # workspace too small
    assert L.spec_verify_greedy_ragged(vp(A), vp(A), vp(A), None, 2, 3, 256, 1000, 0, vp(A), vp(A), vp(WS),
                                       ws_small, None, None) == -3
    # non-positive temperature
    assert L.spec_verify_sample_ragged(vp(A), vp(A), vp(A), vp(A), vp(A), 2, 3, 256, 1000, 0, 0.0, 0, 0, vp(A),
                                       vp(A), vp(WS), 1 << 30, None, None) == -1
    assert L.spec_verify_sample_ragged(vp(A), vp(A), vp(A), vp(A), vp(A + 1), 2, 3, 256, 1000, 0, 1.0, 0, 0,
                                       vp(A), vp(A), vp(WS), 1 << 30, None, None) == -2
    # dual: missing greedy outputs, misaligned greedy output, missing drafter rows
    assert L.spec_verify_dual(vp(A), vp(A), vp(A), vp(A), None, 2, 3, 256, 1000, 0, 1.0, 0, 0, None, vp(A),
                              vp(A), vp(A), vp(WS), 1 << 30, None, None) == -7
    assert L.spec_verify_dual(vp(A), vp(A), vp(A), vp(A), None, 2, 3, 256, 1000, 0, 1.0, 0, 0, vp(A + 2), vp(A),
                              vp(A), vp(A), vp(WS), 1 << 30, None, None) == -2
    assert L.spec_verify_dual(vp(A), None, vp(A), vp(A), None, 2, 3, 256, 1000, 0, 1.0, 0, 0, vp(A), vp(A),
                              vp(A), vp(A), vp(WS), 1 << 30, None, None) == -7
    assert L.spec_verify_dual(vp(A), vp(A), vp(A), vp(A), None, 2, 3, 256, 1000, 0, 1.0, 0, 0, vp(A), vp(A),
                              vp(A), vp(A), vp(WS), ws_small, None, None) == -3


def test_fuse_call_validates_on_the_host():
    """mtp_input_fuse: workspace sizing and every host-side error, without a GPU."""
    L = mv.lib()
    vp = ctypes.c_void_p
    assert L.mtpv_fuse_workspace_bytes(4, 5120) > 4 * 2 * 5120 * 2
    assert L.mtpv_fuse_workspace_bytes(0, 5120) == 0
    assert L.mtpv_fuse_workspace_bytes(4, 4) == 0
    ok = dict(tokens=vp(A), embed=vp(A), hidden=vp(A), ne=vp(A), nh=vp(A), W=vp(A), B=4, H=256, V=1000, eps=1e-6,
              out=vp(A), ws=vp(WS), wsb=1 << 30)

    def call(**kw):
        a = dict(ok, **kw)
        return L.mtp_input_fuse(a["tokens"], a["embed"], a["hidden"], a["ne"], a["nh"], a["W"], a["B"], a["H"],
                                a["V"], a["eps"], a["out"], a["ws"], a["wsb"], None)
    assert call(B=0) == -1
    assert call(V=0) == -1
    assert call(eps=-1.0) == -1
    assert call(eps=float("nan")) == -1
    assert call(H=260) == -2
    assert call(embed=None) == -7
    assert call(W=None) == -7
    assert call(out=vp(A + 4)) == -2
    assert call(tokens=vp(A + 2)) == -2
    assert call(hidden=vp(A + 8)) == -2
    assert call(wsb=1024) == -3
    assert call(ws=vp(WS + 16)) == -3


def test_loss_call_validates_on_the_host():
    """mtp_draft_loss_topk: workspace sizing and every host-side error, without a GPU."""
    L = mv.lib()
    vp = ctypes.c_void_p
    assert L.mtpv_loss_workspace_bytes(8, 256) >= 8 * 8 + 8 * 256 * (8 + 4)
    assert L.mtpv_loss_workspace_bytes(8, 0) == 0
    assert L.mtpv_loss_workspace_bytes(8, mv.LOSS_MAX_TOPK + 1) == 0
    assert L.mtpv_loss_workspace_bytes(-1, 4) == 0
    ok = dict(t=vp(A), s=vp(A), N=8, V=1000, k=256, scale=1.0, loss=vp(A), idx=None, grad=None, ws=vp(WS),
              wsb=1 << 30)

    def call(**kw):
        a = dict(ok, **kw)
        return L.mtp_draft_loss_topk(a["t"], a["s"], a["N"], a["V"], a["k"], a["scale"], a["loss"], a["idx"],
                                     a["grad"], a["ws"], a["wsb"], None)
    assert call(N=-1) == -1
    assert call(V=0) == -1
    assert call(k=0) == -1
    assert call(k=1001) == -1                       # topk > V
    assert call(k=mv.LOSS_MAX_TOPK + 1, V=4096) == -1
    assert call(scale=float("inf")) == -1
    assert call(N=0, t=None, s=None, loss=None) == 0   # nothing to do
    assert call(t=None) == -7
    assert call(loss=None) == -7
    assert call(s=vp(A + 2)) == -2
    assert call(grad=vp(A + 1)) == -2
    assert call(idx=vp(A + 2)) == -2
    assert call(wsb=64) == -3
    assert call(ws=vp(WS + 16)) == -3
    assert call(ws=None) == -3


def test_timing_hooks_on_the_host():
    """mtpv_timing_enable takes the interval of timed calls (0 = off, n >= 1 = one
    call in n) and rejects a negative one; reading with nothing timed touches no GPU."""
    L = mv.lib()
    assert L.mtpv_timing_enable(-1) == -1
    assert L.mtpv_timing_enable(4) == 0
    ms = ctypes.c_double(-1.0)
    n = ctypes.c_int64(-1)
    assert L.mtpv_timing_read(ctypes.byref(ms), ctypes.byref(n), 1) == 0
    assert ms.value == 0.0 and n.value == 0
    assert L.mtpv_timing_read(None, ctypes.byref(n), 0) == -7
    assert L.mtpv_timing_enable(0) == 0
    mv.timing_enable(True, every=16)
    assert mv.timing_read() == (0.0, 0)
    mv.timing_enable(False)


def test_status_values_match_the_header():
    """The status codes of the boundary, as the header declares them: the six codes
    of the verify calls keep fixed values, ENULL comes after them."""
    text = open(HEADER).read()
    decl = dict((n, int(v)) for n, v in re.findall(r"(MTPV_E?\w+)\s*=\s*(-?\d+)\s*[,}/]", text))
    want = {"MTPV_OK": 0, "MTPV_EINVAL": -1, "MTPV_EALIGN": -2, "MTPV_EWORKSPACE": -3, "MTPV_EDTYPE": -4,
            "MTPV_ELAUNCH": -5, "MTPV_EDEVICE": -6, "MTPV_ENULL": -7, "MTPV_ESCRATCH": -8}
    for name, value in want.items():
        assert decl.get(name) == value, (name, decl.get(name))
        assert mv.STATUS[value] == name
    assert mv.lib().mtpv_get_device_error(None, None, None) == -7


def test_workspace_bytes_argument_order():
    """mtpv_workspace_bytes(B, k, H, V, dtype, mode): the sample-mode workspace holds the
    fp32 spill of B(k+1) + Bk rows; greedy holds none."""
    L = mv.lib()
    B, k, H, V = 3, 2, 64, 4000
    s = L.mtpv_workspace_bytes(B, k, H, V, 0, 1)
    g = L.mtpv_workspace_bytes(B, k, H, V, 0, 0)
    assert s - g >= (B * (k + 1) + B * k) * V * 4
    assert L.mtpv_workspace_bytes(B, k, H, V, 0, 3) == 0   # no such mode
    assert L.mtpv_workspace_bytes(B, k, H, V, 2, 0) == 0   # no such dtype


def test_noalloc_entry_point_rejects_before_touching_the_gpu():
    """spec_verify_greedy_noalloc: argument errors and shapes beyond its scratch array
    come back from the host check (nothing enqueued, no GPU needed)."""
    L = mv.lib()
    vp = ctypes.c_void_p
    m = re.search(r"#define MTPV_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == mv.NOALLOC_SCRATCH_BYTES

    def call(B=2, k=3, H=256, V=1000, dtype=0, hidden=A, W=A, drafts=A, alen=A, out=A, err=None):
        return L.spec_verify_greedy_noalloc(vp(hidden), vp(W), vp(drafts), B, k, H, V, dtype, vp(alen), vp(out),
                                            vp(err), None)

    # 1024 requests x 4 rows of the 151936-token head: ~40 MB of partials > 16 MB
    assert mv.workspace_bytes(1024, 3, 5120, 151936, 0, 0) > mv.NOALLOC_SCRATCH_BYTES
    assert call(B=1024, k=3, H=5120, V=151936) == -8
    assert mv.status_string(-8) != "unknown status"
    assert call(W=None) == -7
    assert call(hidden=None) == -7
    assert call(H=12) == -2
    assert call(hidden=A + 2) == -2
    assert call(err=A + 2) == -2
    assert call(B=0) == -1
    assert call(dtype=7) == -4
