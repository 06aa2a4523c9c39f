"""MI355X (gfx950) vocab-side draft-and-verify step of MTP speculative decoding.

A thin ctypes binding over libmtpv.so, whose C ABI is declared in include/mtpv.h.
Every step of the verify path runs in the library's HIP kernels; this module only
marshals torch tensors (device memory) and the current HIP stream into the C calls.
There is no fallback: if the library is missing, every call raises.

Calls (names as in the C ABI):
  spec_verify_greedy(hidden[B,k+1,H], W[V,H], drafts[B,k], accepted_len[B], out_tokens[B,k+1], workspace)
  spec_verify_sample(target_hidden, draft_hidden[B,k,H], W, drafts, temperature, seed, offset,
                     accepted_len, out_tokens, workspace)
  spec_draft_sample(draft_hidden[B,kd,H], W, temperature, seed, offset, depth0, draft_tokens[B,kd], workspace)
  spec_verify_greedy_noalloc(hidden, W, drafts, accepted_len, out_tokens, device_error)  no workspace
  spec_verify_greedy_ragged / spec_verify_sample_ragged(..., draft_len[B], ...)  per-request draft counts
  spec_verify_dual(target_hidden, draft_hidden, W, drafts, draft_len, temperature, seed, offset,
                   accepted_len_greedy, out_tokens_greedy, accepted_len_sample, out_tokens_sample, workspace)
  mtp_input_fuse(tokens[B], embed[V,H], hidden[B,H], norm_emb[H], norm_hidden[H], W_fc[H,2H], eps, out[B,H],
                 workspace)
  mtp_draft_loss_topk(teacher[N,V], student[N,V], topk, loss[N], workspace, grad_scale, topk_index[N,topk],
                      grad[N,V])   top-k soft cross-entropy draft loss (fp32 logits)
"""
import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
# MTPV_LIBRARY: another build of the library (measurements of variants); default in-tree
LIB_PATH = os.environ.get("MTPV_LIBRARY") or os.path.join(PKG_DIR, "libmtpv.so")

MODE_GREEDY, MODE_SAMPLE, MODE_DRAFT = 0, 1, 2
DTYPE_BF16, DTYPE_F32 = 0, 1
DEVERR_DRAFT_RANGE = 1
DEVERR_DRAFT_LEN = 2
DEVERR_TOKEN_RANGE = 4
LOSS_MAX_TOPK = 512

STATUS = {0: "MTPV_OK", -1: "MTPV_EINVAL", -2: "MTPV_EALIGN", -3: "MTPV_EWORKSPACE", -4: "MTPV_EDTYPE",
          -5: "MTPV_ELAUNCH", -6: "MTPV_EDEVICE", -7: "MTPV_ENULL", -8: "MTPV_ESCRATCH"}
NOALLOC_SCRATCH_BYTES = 16 << 20


class MtpvError(RuntimeError):
    """A C-ABI call returned a negative status."""

    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({status_string(status)})")


class Debug(ctypes.Structure):
    """Mirror of struct mtpv_debug (optional parity-test exports)."""
    _fields_ = [("logits", ctypes.c_void_p), ("probs", ctypes.c_void_p), ("argmax", ctypes.c_void_p),
                ("row_stats", ctypes.c_void_p), ("pd_qd", ctypes.c_void_p)]


_lib = None
_vp, _i, _sz, _d, _u64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_double, ctypes.c_uint64

_SIGNATURES = {
    "mtpv_version": (_i, []),
    "mtpv_status_string": (ctypes.c_char_p, [_i]),
    "mtpv_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "mtpv_check_args": (_i, [_i, _i, _i, _i, _i, _i, _d, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz]),
    "spec_verify_greedy": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, _vp, _sz, _vp, _vp]),
    "spec_verify_sample": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _d, _u64, _u64, _vp, _vp, _vp, _sz,
                                _vp, _vp]),
    "spec_draft_sample": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _i, _d, _u64, _u64, _vp, _vp, _sz, _vp, _vp]),
    "spec_verify_greedy_noalloc": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp]),
    "spec_verify_greedy_ragged": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, _vp, _sz, _vp, _vp]),
    "spec_verify_sample_ragged": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _d, _u64, _u64, _vp, _vp,
                                       _vp, _sz, _vp, _vp]),
    "spec_verify_dual": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _d, _u64, _u64, _vp, _vp, _vp, _vp,
                              _vp, _sz, _vp, _vp]),
    "mtpv_fuse_workspace_bytes": (_sz, [_i, _i]),
    "mtp_input_fuse": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _d, _vp, _vp, _sz, _vp]),
    "mtpv_loss_workspace_bytes": (_sz, [_i, _i]),
    "mtp_draft_loss_topk": (_i, [_vp, _vp, _i, _i, _i, ctypes.c_float, _vp, _vp, _vp, _vp, _sz, _vp]),
    "mtpv_get_device_error": (_i, [_vp, ctypes.POINTER(ctypes.c_int32), _vp]),
    "mtpv_timing_enable": (_i, [_i]),
    "mtpv_timing_read": (_i, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64), _i]),
    "mtpv_copy_bytes": (_i, [_vp, _vp, _sz, _vp]),
    "mtpv_read_bytes": (_i, [_vp, _sz, _vp, _vp]),
    "mtpv_mfma_rate": (_i, [_i, _vp, ctypes.POINTER(ctypes.c_int64), _vp]),
}

EXPORTED = tuple(_SIGNATURES)


def lib():
    """The loaded libmtpv.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m mtp_draft_verification_amd.build`"
                               " (there is no non-HIP fallback)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def status_string(status):
    return lib().mtpv_status_string(int(status)).decode()


def _check(status, what):
    if status != 0:
        raise MtpvError(status, what)


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float32:
        return DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _contig(name, t):
    if t is not None and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def workspace_bytes(B, k, H, V, dtype, mode):
    """Workspace size in bytes (0 for an invalid shape). dtype: DTYPE_BF16 / DTYPE_F32; mode: MODE_*."""
    return int(lib().mtpv_workspace_bytes(B, k, H, V, dtype, mode))


def alloc_workspace(mode, B, k, H, V, dtype, device):
    """Allocate a workspace tensor for a call shape (done once, outside the hot loop)."""
    import torch
    n = workspace_bytes(B, k, H, V, dtype, mode)
    if n == 0:
        _check(-1, "workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device=device)


def check_args(mode, B, k, H, V, dtype, temperature, target_hidden, draft_hidden, W, drafts, accepted_len,
               out_tokens, workspace, ws_bytes):
    """Host-only argument check; pointer arguments are raw integers (or None). Returns the status."""
    v = lambda x: None if x is None else ctypes.c_void_p(int(x))
    return int(lib().mtpv_check_args(mode, B, k, H, V, dtype, float(temperature), v(target_hidden),
                                     v(draft_hidden), v(W), v(drafts), v(accepted_len), v(out_tokens),
                                     v(workspace), int(ws_bytes)))


def make_debug(logits=None, probs=None, argmax=None, row_stats=None, pd_qd=None):
    return Debug(*(None if t is None else t.data_ptr() for t in (logits, probs, argmax, row_stats, pd_qd)))


def _dbg(debug):
    return None if debug is None else ctypes.byref(debug)


def spec_verify_greedy(hidden, W, drafts, accepted_len, out_tokens, workspace, debug=None, stream=None):
    """Greedy verify: hidden [B,k+1,H], W [V,H] (bf16 or fp32), drafts [B,k] int32 -> fills
    accepted_len [B] and out_tokens [B,k+1] (int32)."""
    B, k1, H = hidden.shape
    V = W.shape[0]
    for n, t in (("hidden", hidden), ("W", W), ("drafts", drafts), ("workspace", workspace)):
        _contig(n, t)
    st = lib().spec_verify_greedy(_ptr(hidden), _ptr(W), _ptr(drafts), B, k1 - 1, H, V, _dtype_code(W),
                                  _ptr(accepted_len), _ptr(out_tokens), _ptr(workspace), workspace.numel(),
                                  _dbg(debug), _stream(stream))
    _check(st, "spec_verify_greedy")


def spec_verify_sample(target_hidden, draft_hidden, W, drafts, temperature, seed, offset, accepted_len,
                       out_tokens, workspace, debug=None, stream=None):
    """Stochastic verify: target_hidden [B,k+1,H], draft_hidden [B,k,H], W [V,H], drafts [B,k]."""
    B, k1, H = target_hidden.shape
    V = W.shape[0]
    for n, t in (("target_hidden", target_hidden), ("draft_hidden", draft_hidden), ("W", W),
                 ("drafts", drafts), ("workspace", workspace)):
        _contig(n, t)
    st = lib().spec_verify_sample(_ptr(target_hidden), _ptr(draft_hidden), _ptr(W), _ptr(drafts), B, k1 - 1, H,
                                  V, _dtype_code(W), float(temperature), int(seed) & (2**64 - 1),
                                  int(offset) & (2**64 - 1), _ptr(accepted_len), _ptr(out_tokens),
                                  _ptr(workspace), workspace.numel(), _dbg(debug), _stream(stream))
    _check(st, "spec_verify_sample")


def spec_verify_greedy_noalloc(hidden, W, drafts, accepted_len, out_tokens, device_error=None, stream=None):
    """spec_verify_greedy without a workspace (the library's per-GPU scratch array; for
    callers that cannot allocate). device_error: optional int32 device tensor [1]."""
    B, k1, H = hidden.shape
    V = W.shape[0]
    for n, t in (("hidden", hidden), ("W", W), ("drafts", drafts)):
        _contig(n, t)
    st = lib().spec_verify_greedy_noalloc(_ptr(hidden), _ptr(W), _ptr(drafts), B, k1 - 1, H, V, _dtype_code(W),
                                          _ptr(accepted_len), _ptr(out_tokens), _ptr(device_error),
                                          _stream(stream))
    _check(st, "spec_verify_greedy_noalloc")


def spec_verify_greedy_ragged(hidden, W, drafts, draft_len, accepted_len, out_tokens, workspace, debug=None,
                              stream=None):
    """Greedy verify with draft_len [B] int32 (k_b <= k drafts per request; None = all k)."""
    B, k1, H = hidden.shape
    V = W.shape[0]
    for n, t in (("hidden", hidden), ("W", W), ("drafts", drafts), ("draft_len", draft_len),
                 ("workspace", workspace)):
        _contig(n, t)
    st = lib().spec_verify_greedy_ragged(_ptr(hidden), _ptr(W), _ptr(drafts), _ptr(draft_len), B, k1 - 1, H, V,
                                         _dtype_code(W), _ptr(accepted_len), _ptr(out_tokens), _ptr(workspace),
                                         workspace.numel(), _dbg(debug), _stream(stream))
    _check(st, "spec_verify_greedy_ragged")


def spec_verify_sample_ragged(target_hidden, draft_hidden, W, drafts, draft_len, temperature, seed, offset,
                              accepted_len, out_tokens, workspace, debug=None, stream=None):
    """Stochastic verify with draft_len [B] int32 (k_b <= k drafts per request; None = all k)."""
    B, k1, H = target_hidden.shape
    V = W.shape[0]
    for n, t in (("target_hidden", target_hidden), ("draft_hidden", draft_hidden), ("W", W),
                 ("drafts", drafts), ("draft_len", draft_len), ("workspace", workspace)):
        _contig(n, t)
    st = lib().spec_verify_sample_ragged(_ptr(target_hidden), _ptr(draft_hidden), _ptr(W), _ptr(drafts),
                                         _ptr(draft_len), B, k1 - 1, H, V, _dtype_code(W), float(temperature),
                                         int(seed) & (2**64 - 1), int(offset) & (2**64 - 1), _ptr(accepted_len),
                                         _ptr(out_tokens), _ptr(workspace), workspace.numel(), _dbg(debug),
                                         _stream(stream))
    _check(st, "spec_verify_sample_ragged")


def spec_verify_dual(target_hidden, draft_hidden, W, drafts, draft_len, temperature, seed, offset,
                     accepted_len_greedy, out_tokens_greedy, accepted_len_sample, out_tokens_sample, workspace,
                     debug=None, stream=None):
    """Greedy and stochastic outcomes of the same drafts from one pass over W (sample-mode workspace)."""
    B, k1, H = target_hidden.shape
    V = W.shape[0]
    for n, t in (("target_hidden", target_hidden), ("draft_hidden", draft_hidden), ("W", W),
                 ("drafts", drafts), ("draft_len", draft_len), ("workspace", workspace)):
        _contig(n, t)
    st = lib().spec_verify_dual(_ptr(target_hidden), _ptr(draft_hidden), _ptr(W), _ptr(drafts), _ptr(draft_len),
                                B, k1 - 1, H, V, _dtype_code(W), float(temperature), int(seed) & (2**64 - 1),
                                int(offset) & (2**64 - 1), _ptr(accepted_len_greedy), _ptr(out_tokens_greedy),
                                _ptr(accepted_len_sample), _ptr(out_tokens_sample), _ptr(workspace),
                                workspace.numel(), _dbg(debug), _stream(stream))
    _check(st, "spec_verify_dual")


def alloc_fuse_workspace(B, H, device):
    import torch
    n = lib().mtpv_fuse_workspace_bytes(B, H)
    if n == 0:
        raise MtpvError(-1, "mtpv_fuse_workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device=device)


def mtp_input_fuse(tokens, embed, hidden, norm_emb, norm_hidden, W_fc, eps, out, workspace, stream=None):
    """MTP input fusion: tokens [B] int32, embed [V,H], hidden [B,H], norms [H], W_fc [H,2H] (bf16)
    -> out [B,H] fp32 = [rms(embed[tok]) | rms(hidden)] @ W_fc^T."""
    B, H = hidden.shape
    V = embed.shape[0]
    for n, t in (("tokens", tokens), ("embed", embed), ("hidden", hidden), ("norm_emb", norm_emb),
                 ("norm_hidden", norm_hidden), ("W_fc", W_fc), ("out", out), ("workspace", workspace)):
        _contig(n, t)
    st = lib().mtp_input_fuse(_ptr(tokens), _ptr(embed), _ptr(hidden), _ptr(norm_emb), _ptr(norm_hidden), _ptr(W_fc),
                              B, H, V, float(eps), _ptr(out), _ptr(workspace), workspace.numel(), _stream(stream))
    _check(st, "mtp_input_fuse")


def alloc_loss_workspace(N, topk, device):
    import torch
    n = lib().mtpv_loss_workspace_bytes(N, topk)
    if n == 0:
        raise MtpvError(-1, "mtpv_loss_workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device=device)


def mtp_draft_loss_topk(teacher, student, topk, loss, workspace, grad_scale=1.0, topk_index=None, grad=None,
                        stream=None):
    """Top-k soft cross-entropy draft loss: teacher, student [N,V] fp32 -> loss [N] fp32; optionally the
    kept teacher ids topk_index [N,topk] int32 (best first) and grad [N,V] fp32 = d(grad_scale*loss)/d student."""
    N, V = teacher.shape
    for n, t in (("teacher", teacher), ("student", student), ("loss", loss), ("workspace", workspace),
                 ("topk_index", topk_index), ("grad", grad)):
        if t is not None:
            _contig(n, t)
    if tuple(student.shape) != (N, V):
        raise ValueError("student must have the teacher's shape")
    st = lib().mtp_draft_loss_topk(_ptr(teacher), _ptr(student), N, V, int(topk), float(grad_scale), _ptr(loss),
                                   _ptr(topk_index), _ptr(grad), _ptr(workspace), workspace.numel(),
                                   _stream(stream))
    _check(st, "mtp_draft_loss_topk")


def spec_draft_sample(draft_hidden, W, temperature, seed, offset, depth0, draft_tokens, workspace, debug=None,
                      stream=None):
    """Drafter draws: draft_hidden [B,kd,H] -> draft_tokens [B,kd] (int32)."""
    B, kd, H = draft_hidden.shape
    V = W.shape[0]
    for n, t in (("draft_hidden", draft_hidden), ("W", W), ("workspace", workspace)):
        _contig(n, t)
    st = lib().spec_draft_sample(_ptr(draft_hidden), _ptr(W), B, kd, int(depth0), H, V, _dtype_code(W),
                                 float(temperature), int(seed) & (2**64 - 1), int(offset) & (2**64 - 1),
                                 _ptr(draft_tokens), _ptr(workspace), workspace.numel(), _dbg(debug),
                                 _stream(stream))
    _check(st, "spec_draft_sample")


def get_device_error(workspace, stream=None):
    """Waits for the stream and returns the last call's device error word."""
    err = ctypes.c_int32(0)
    _check(lib().mtpv_get_device_error(_ptr(workspace), ctypes.byref(err), _stream(stream)),
           "mtpv_get_device_error")
    return int(err.value)


def timing_enable(on=True, every=1):
    """Time one call in `every` (events around its dominant kernel) while `on`."""
    _check(lib().mtpv_timing_enable(int(every) if on else 0), "mtpv_timing_enable")


def timing_read(reset=True):
    """(total ms of the timed LM-head launches, number of launches)."""
    ms = ctypes.c_double(0.0)
    n = ctypes.c_int64(0)
    _check(lib().mtpv_timing_read(ctypes.byref(ms), ctypes.byref(n), 1 if reset else 0), "mtpv_timing_read")
    return float(ms.value), int(n.value)


def copy_bytes(dst, src, nbytes, stream=None):
    _check(lib().mtpv_copy_bytes(_ptr(dst), _ptr(src), int(nbytes), _stream(stream)), "mtpv_copy_bytes")


def read_bytes(src, nbytes, sink, stream=None):
    """Achievable-rate probe: one non-temporal read sweep of nbytes at src (a device
    tensor); sink: a device tensor of at least 4 bytes (never written)."""
    _check(lib().mtpv_read_bytes(_ptr(src), int(nbytes), _ptr(sink), _stream(stream)), "mtpv_read_bytes")


def mfma_rate(iters, sink, stream=None):
    """Achievable-rate probe: back-to-back bf16 MFMAs on every SIMD; returns the flops
    of the launch. sink: a device tensor of at least 4 bytes (never written)."""
    flops = ctypes.c_int64(0)
    _check(lib().mtpv_mfma_rate(int(iters), _ptr(sink), ctypes.byref(flops), _stream(stream)), "mtpv_mfma_rate")
    return int(flops.value)
