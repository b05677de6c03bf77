"""ctypes binding of libzmttt.so (the C ABI declared in include/zm_ttt.h).

Argument marshalling only: every step of the TTT layer runs in the HIP
library.  torch is used for device memory and for the current HIP stream.
If the library is missing, every call raises ZmError; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libzmttt.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, -1, -2, -3, -4
BF16, F32 = 0, 1
RENORM_NONE, RENORM_ROW = 0, 1
APPLY_THEN_UPDATE, UPDATE_THEN_APPLY = 0, 1
STREAM_EMIT_BF16, STREAM_REUSE_BF16 = 0x100, 0x200
SCRATCH_BYTES = 64 << 20  # ZM_TTT_SCRATCH_BYTES
STEP_GRADIENT, STEP_NEWTON_SCHULZ = 0, 1

EXPORTED = (
    "zm_ttt_workspace_size", "zm_ttt_update", "zm_ttt_update_loss", "zm_ttt_apply",
    "zm_ttt_update_apply", "zm_ttt_update_apply_scratch",
    "zm_ttt_stream_step", "zm_ttt_chunked", "zm_ttt_layer_workspace_size", "zm_ttt_layer",
    "zm_status_string", "zm_ttt_last_error", "zm_ttt_version", "zm_ttt_set_profile_events",
)


class ZmError(RuntimeError):
    def __init__(self, msg, status=None):
        super().__init__(msg)
        self.status = status


class Desc(ctypes.Structure):
    _fields_ = [
        ("heads", ctypes.c_int32),
        ("d_head", ctypes.c_int32),
        ("d_hidden", ctypes.c_int32),
        ("io_dtype", ctypes.c_int32),
        ("renorm", ctypes.c_int32),
        ("step_rule", ctypes.c_int32),
        ("ld_tok", ctypes.c_int64),
    ]


class LayerWeights(ctypes.Structure):
    _fields_ = [
        ("w_in", ctypes.c_void_p),
        ("w_gate", ctypes.c_void_p),
        ("gamma", ctypes.c_void_p),
        ("d_in", ctypes.c_int32),
        ("eta_scale", ctypes.c_float),
        ("rms_eps", ctypes.c_float),
        ("reserved", ctypes.c_int32),
    ]


_lib = None
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_DESC = ctypes.POINTER(Desc)


def load_library(path: str | None = None):
    """Load (once) and return the ctypes handle of libzmttt.so."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ZmError(f"HIP library not found at {p}; build it with "
                      "`python -m reconstruction_lact_chunk_amd.build_lib`")
    lib = ctypes.CDLL(p)
    lib.zm_ttt_workspace_size.argtypes = [_DESC, _I64, _I64, ctypes.POINTER(_SZ)]
    lib.zm_ttt_update.argtypes = [_DESC, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]
    lib.zm_ttt_update_loss.argtypes = [_DESC, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                       _SZ, _P]
    lib.zm_ttt_apply.argtypes = [_DESC, _I64, _P, _P, _P, _P, _P, _P, _SZ, _P]
    lib.zm_ttt_update_apply.argtypes = [_DESC, _I64, _P, _P, _P, _I64, _P, _P, _P, _P, _P, _P, _P,
                                        _P, _P, _SZ, _P]
    lib.zm_ttt_update_apply_scratch.argtypes = [_DESC, _I64, _P, _P, _P, _I64, _P, _P, _P, _P, _P,
                                                _P, _P, _P, _P]
    lib.zm_ttt_stream_step.argtypes = [_DESC, ctypes.c_int, _I64, _P, _P, _P, _P, _P, _P, _P, _P,
                                       _P, _SZ, _P]
    lib.zm_ttt_chunked.argtypes = [_DESC, ctypes.c_int, _I64, _P, _P, ctypes.c_int, _P, _P, _P,
                                   _P, _P, _P, _P, _P, _P, _SZ, _P]
    _LW = ctypes.POINTER(LayerWeights)
    lib.zm_ttt_layer_workspace_size.argtypes = [_DESC, _LW, _I64, ctypes.POINTER(_SZ)]
    lib.zm_ttt_layer.argtypes = [_DESC, _LW, _I64, _P, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _SZ,
                                 _P]
    lib.zm_status_string.argtypes = [ctypes.c_int]
    lib.zm_status_string.restype = ctypes.c_char_p
    lib.zm_ttt_last_error.argtypes = []
    lib.zm_ttt_last_error.restype = ctypes.c_char_p
    lib.zm_ttt_version.argtypes = []
    lib.zm_ttt_set_profile_events.argtypes = [ctypes.POINTER(_P), ctypes.c_int]
    for name in ("zm_ttt_workspace_size", "zm_ttt_update", "zm_ttt_update_loss", "zm_ttt_apply",
                 "zm_ttt_update_apply", "zm_ttt_update_apply_scratch",
                 "zm_ttt_stream_step", "zm_ttt_chunked", "zm_ttt_layer_workspace_size",
                 "zm_ttt_layer", "zm_ttt_version", "zm_ttt_set_profile_events"):
        getattr(lib, name).restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().zm_status_string(int(status)).decode()


def version() -> int:
    return int(load_library().zm_ttt_version())


def last_error() -> str:
    return load_library().zm_ttt_last_error().decode()


def _check(status: int, what: str):
    if status != OK:
        detail = f"; {last_error()}" if status == ERR_HIP else ""
        raise ZmError(f"{what}: {status_string(status)} ({status}){detail}", status)


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------
_IO = {torch.bfloat16: BF16, torch.float32: F32}


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check_weights(w1, w2, w3, device=True):
    for w in (w1, w2, w3):
        if w.dtype != torch.float32 or not w.is_contiguous() or w.dim() != 3:
            raise ZmError("weights must be contiguous fp32 [heads, h, d] / [heads, d, h]")
    heads, h, d = w1.shape
    if w3.shape != w1.shape or tuple(w2.shape) != (heads, d, h):
        raise ZmError("weight shapes disagree: W1, W3 [H, h, d]; W2 [H, d, h]")
    if device:
        _on_gpu(w1, w2, w3, what="weights")
    return heads, d, h


def _on_gpu(*tensors, what="tensors"):
    """Device check, made after the shape checks so that a shape error is
    reported as such whatever the tensors' device."""
    for t in tensors:
        if t is not None and not t.is_cuda:
            raise ZmError(f"{what} must be on the GPU")


def _token_ld(x, heads, d, io, rows=None, name="token tensor"):
    """Checks one token tensor whatever its length (dtype, [n, H, d] shape,
    inner strides, row count when `rows` is given, device) and returns its token
    stride, or None when it has at most one row (no stride to agree on)."""
    if x is None:
        return None
    if x.dtype not in _IO or _IO[x.dtype] != io:
        raise ZmError(f"{name}: token tensors must all share the io dtype (bf16 or fp32)")
    if x.dim() != 3 or x.shape[1] != heads or x.shape[2] != d:
        raise ZmError(f"{name}: shape {tuple(x.shape)} != [n, {heads}, {d}]")
    if rows is not None and x.shape[0] != rows:
        raise ZmError(f"{name}: {x.shape[0]} rows, the call needs {rows}")
    if x.shape[0] > 0 and (x.stride(2) != 1 or x.stride(1) != d):
        raise ZmError(f"{name}: token tensors need unit stride on d and d on heads")
    return x.stride(0) if x.shape[0] > 1 else None


def make_desc(w1, w2, w3, io_dtype: int, renorm: bool, *tokens, step_rule: int = STEP_GRADIENT,
              rows=None, check_device=True) -> Desc:
    """Descriptor of a call on the weights w1..w3 and the token tensors
    `tokens`; every token tensor is checked, and `rows` (one entry per token
    tensor, None to skip) gives the row count each must have.  With
    check_device=False the caller checks the devices itself, last."""
    heads, d, h = _check_weights(w1, w2, w3, device=False)
    rows = rows if rows is not None else [None] * len(tokens)
    lds = set()
    for i, (x, r) in enumerate(zip(tokens, rows)):
        ld = _token_ld(x, heads, d, io_dtype, r, f"token tensor {i}")
        if ld is not None:
            lds.add(ld)
    if len(lds) > 1:
        raise ZmError("all token tensors of one call must share the token stride")
    if check_device:
        _on_gpu(w1, w2, w3, what="weights")
        _on_gpu(*tokens, what="token tensors")
    ld = lds.pop() if lds else heads * d
    return Desc(heads, d, h, io_dtype, RENORM_ROW if renorm else RENORM_NONE, int(step_rule), ld)


def _check_out_weights(outs, w1, w2, w3):
    """Output weights: fp32, contiguous and of the input weights' shapes (their
    device is checked with the call's other tensors)."""
    if len(outs) != 3:
        raise ZmError("need three output weight tensors (W1, W2, W3)")
    for o, w, nm in zip(outs, (w1, w2, w3), ("W1", "W2", "W3")):
        if tuple(o.shape) != tuple(w.shape):
            raise ZmError(f"output {nm} has shape {tuple(o.shape)}, the weights {tuple(w.shape)}")
    _check_weights(*outs, device=False)


def _io_of(*tokens) -> int:
    for x in tokens:
        if x is not None:
            if x.dtype not in _IO:
                raise ZmError(f"unsupported token dtype {x.dtype}")
            return _IO[x.dtype]
    raise ZmError("no token tensor given")


def _eta(eta, n, heads):
    if eta.dtype != torch.float32 or not eta.is_contiguous() or tuple(eta.shape) != (n, heads):
        raise ZmError(f"eta must be contiguous fp32 [{n}, {heads}]")


def _like_tokens(x):
    """An output with the same token stride as x (the ABI has one token stride)."""
    n, heads, d = x.shape
    if n <= 1 or x.stride(0) == heads * d:
        return torch.empty((n, heads, d), dtype=x.dtype, device=x.device)
    buf = torch.empty(n * x.stride(0), dtype=x.dtype, device=x.device)
    return buf.as_strided((n, heads, d), (x.stride(0), d, 1))


def workspace_size(desc: Desc, n_kv: int, n_q: int) -> int:
    out = ctypes.c_size_t(0)
    _check(load_library().zm_ttt_workspace_size(ctypes.byref(desc), int(n_kv), int(n_q),
                                                 ctypes.byref(out)), "zm_ttt_workspace_size")
    return int(out.value)


def _workspace(desc, n_kv, n_q, device, workspace):
    need = workspace_size(desc, n_kv, n_q)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    elif workspace.numel() * workspace.element_size() < need:
        raise ZmError(f"workspace of {workspace.numel()} bytes < {need} needed", ERR_WORKSPACE)
    return workspace, need


def _ws_bytes(ws):
    return ctypes.c_size_t(ws.numel() * ws.element_size())


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------
def update(k, v, eta, w1, w2, w3, renorm=False, out=None, workspace=None,
           step_rule=STEP_GRADIENT):
    """W_hat = step(W; k, v, eta) (+ row renorm).  Returns (W1_hat, W2_hat, W3_hat);
    pass out=(w1, w2, w3) to update in place."""
    io = _io_of(k, v)
    n = k.shape[0]
    desc = make_desc(w1, w2, w3, io, renorm, k, v, step_rule=step_rule, rows=[n, n],
                     check_device=False)
    _eta(eta, n, desc.heads)
    outs = out if out is not None else tuple(torch.empty_like(w) for w in (w1, w2, w3))
    _check_out_weights(outs, w1, w2, w3)
    _on_gpu(k, v, eta, w1, w2, w3, *outs)
    ws, _ = _workspace(desc, n, 0, w1.device, workspace)
    st = load_library().zm_ttt_update(ctypes.byref(desc), n, _ptr(k), _ptr(v), _ptr(eta),
                                      _ptr(w1), _ptr(w2), _ptr(w3), *map(_ptr, outs), _ptr(ws),
                                      _ws_bytes(ws), _stream(w1.device))
    _check(st, "zm_ttt_update")
    return outs


def update_loss(k, v, eta, w1, w2, w3, renorm=False, out=None, loss=None, workspace=None,
                step_rule=STEP_GRADIENT):
    """The update of `update` and its virtual loss at the incoming W:
    loss[h] = -sum_i eta_i f_W(k_i) . v_i per head (fp32, [H]), read from the
    update's registers.  Returns ((W1_hat, W2_hat, W3_hat), loss).  bf16
    narrow heads only."""
    io = _io_of(k, v)
    n = k.shape[0]
    desc = make_desc(w1, w2, w3, io, renorm, k, v, step_rule=step_rule, rows=[n, n],
                     check_device=False)
    _eta(eta, n, desc.heads)
    outs = out if out is not None else tuple(torch.empty_like(w) for w in (w1, w2, w3))
    _check_out_weights(outs, w1, w2, w3)
    if loss is None:
        loss = torch.empty(desc.heads, dtype=torch.float32, device=w1.device)
    if loss.dtype != torch.float32 or loss.numel() != desc.heads or not loss.is_contiguous():
        raise ZmError(f"loss must be a contiguous fp32 tensor of {desc.heads} elements")
    _on_gpu(k, v, eta, w1, w2, w3, *outs, loss)
    ws, _ = _workspace(desc, n, 0, w1.device, workspace)
    st = load_library().zm_ttt_update_loss(ctypes.byref(desc), n, _ptr(k), _ptr(v), _ptr(eta),
                                           _ptr(w1), _ptr(w2), _ptr(w3), *map(_ptr, outs),
                                           _ptr(loss), _ptr(ws), _ws_bytes(ws), _stream(w1.device))
    _check(st, "zm_ttt_update_loss")
    return outs, loss


def apply(q, w1, w2, w3, out=None, workspace=None):
    """o = f_W(q) per head; q [n, H, d] -> o [n, H, d] (same dtype)."""
    io = _io_of(q)
    o = out if out is not None else _like_tokens(q)
    n = q.shape[0]
    desc = make_desc(w1, w2, w3, io, False, q, o, rows=[n, n])  # checks every device
    ws, _ = _workspace(desc, 0, n, w1.device, workspace)
    st = load_library().zm_ttt_apply(ctypes.byref(desc), n, _ptr(q), _ptr(w1), _ptr(w2),
                                     _ptr(w3), _ptr(o), _ptr(ws), _ws_bytes(ws),
                                     _stream(w1.device))
    _check(st, "zm_ttt_apply")
    return o


def update_apply(k, v, eta, q, w1, w2, w3, renorm=False, w_out=None, out=None, workspace=None,
                 step_rule=STEP_GRADIENT):
    """Bidirectional chunk: update on (k, v, eta), then o = f_{W_hat}(q).
    Returns ((W1_hat, W2_hat, W3_hat), o)."""
    io = _io_of(k, v, q)
    o = out if out is not None else _like_tokens(q)
    n_kv, n_q = k.shape[0], q.shape[0]
    desc = make_desc(w1, w2, w3, io, renorm, k, v, q, o, step_rule=step_rule,
                     rows=[n_kv, n_kv, n_q, n_q], check_device=False)
    _eta(eta, n_kv, desc.heads)
    outs = w_out if w_out is not None else tuple(torch.empty_like(w) for w in (w1, w2, w3))
    _check_out_weights(outs, w1, w2, w3)
    _on_gpu(k, v, eta, q, o, w1, w2, w3, *outs)
    ws, _ = _workspace(desc, n_kv, n_q, w1.device, workspace)
    st = load_library().zm_ttt_update_apply(
        ctypes.byref(desc), n_kv, _ptr(k), _ptr(v), _ptr(eta), n_q, _ptr(q), _ptr(w1), _ptr(w2),
        _ptr(w3), *map(_ptr, outs), _ptr(o), _ptr(ws), _ws_bytes(ws), _stream(w1.device))
    _check(st, "zm_ttt_update_apply")
    return outs, o


def update_apply_scratch(k, v, eta, q, w1, w2, w3, renorm=False, w_out=None, out=None,
                         step_rule=STEP_GRADIENT):
    """update_apply run in the library's own device scratch instead of a
    workspace (zm_ttt_update_apply_scratch: for callers that cannot allocate;
    narrow heads, at most SCRATCH_BYTES of workspace need).  The outputs are
    allocated here unless w_out / out are given; pass them to allocate nothing."""
    io = _io_of(k, v, q)
    o = out if out is not None else _like_tokens(q)
    n_kv, n_q = k.shape[0], q.shape[0]
    desc = make_desc(w1, w2, w3, io, renorm, k, v, q, o, step_rule=step_rule,
                     rows=[n_kv, n_kv, n_q, n_q], check_device=False)
    _eta(eta, n_kv, desc.heads)
    outs = w_out if w_out is not None else tuple(torch.empty_like(w) for w in (w1, w2, w3))
    _check_out_weights(outs, w1, w2, w3)
    _on_gpu(k, v, eta, q, o, w1, w2, w3, *outs)
    st = load_library().zm_ttt_update_apply_scratch(
        ctypes.byref(desc), n_kv, _ptr(k), _ptr(v), _ptr(eta), n_q, _ptr(q), _ptr(w1), _ptr(w2),
        _ptr(w3), *map(_ptr, outs), _ptr(o), _stream(w1.device))
    _check(st, "zm_ttt_update_apply_scratch")
    return outs, o


def stream_step(q, k, v, eta, w1, w2, w3, renorm=False, order=APPLY_THEN_UPDATE, out=None,
                workspace=None, step_rule=STEP_GRADIENT, emit_bf16=False, reuse_bf16=False):
    """One frame of the streaming recursion; w1, w2, w3 are updated in place.
    Returns o (read with W(t-1) for APPLY_THEN_UPDATE, W(t) otherwise).
    emit_bf16 / reuse_bf16: the STREAM_EMIT_BF16 / STREAM_REUSE_BF16 flags
    (keep W's bf16 operand copies in `workspace` from one frame to the next;
    reuse needs the same workspace as the previous emitting call)."""
    if reuse_bf16 and workspace is None:
        raise ZmError("reuse_bf16 needs the workspace of the previous call")
    io = _io_of(q, k, v)
    o = out if out is not None else _like_tokens(q)
    n = q.shape[0]
    desc = make_desc(w1, w2, w3, io, renorm, q, k, v, o, step_rule=step_rule, rows=[n] * 4,
                     check_device=False)
    _eta(eta, n, desc.heads)
    _on_gpu(q, k, v, o, eta, w1, w2, w3)
    ws, _ = _workspace(desc, n, n, w1.device, workspace)
    flags = (STREAM_EMIT_BF16 if emit_bf16 else 0) | (STREAM_REUSE_BF16 if reuse_bf16 else 0)
    st = load_library().zm_ttt_stream_step(ctypes.byref(desc), int(order) | flags, n, _ptr(q),
                                           _ptr(k),
                                           _ptr(v), _ptr(eta), _ptr(w1), _ptr(w2), _ptr(w3),
                                           _ptr(o), _ptr(ws), _ws_bytes(ws), _stream(w1.device))
    _check(st, "zm_ttt_stream_step")
    return o


def chunked(q, k, v, eta, offsets, w1, w2, w3, renorm=False, order=UPDATE_THEN_APPLY,
            update_mask=None, inner_steps=1, out=None, workspace=None, step_rule=STEP_GRADIENT):
    """A sequence cut into chunks [offsets[c], offsets[c+1]) read and written
    chunk after chunk; w1, w2, w3 are updated in place.  update_mask: a
    sequence of n_chunks booleans (False: read only).  Returns o."""
    io = _io_of(q, k, v)
    o = out if out is not None else _like_tokens(q)
    offs = [int(x) for x in offsets]
    n_chunks = len(offs) - 1
    if n_chunks < 0:
        raise ZmError("offsets needs at least one entry")
    n = offs[-1]
    desc = make_desc(w1, w2, w3, io, renorm, q, k, v, o, step_rule=step_rule, rows=[n] * 4,
                     check_device=False)
    _eta(eta, n, desc.heads)
    _on_gpu(q, k, v, o, eta, w1, w2, w3)
    longest = max([b - a for a, b in zip(offs, offs[1:])] + [0])
    ws, _ = _workspace(desc, longest, longest, w1.device, workspace)
    off_arr = (ctypes.c_int64 * len(offs))(*offs)
    mask_arr = None
    if update_mask is not None:
        if len(update_mask) != n_chunks:
            raise ZmError("update_mask needs one entry per chunk")
        mask_arr = (ctypes.c_uint8 * max(n_chunks, 1))(*[1 if m else 0 for m in update_mask])
    st = load_library().zm_ttt_chunked(
        ctypes.byref(desc), int(order), n_chunks, off_arr, mask_arr, int(inner_steps), _ptr(q),
        _ptr(k), _ptr(v), _ptr(eta), _ptr(w1), _ptr(w2), _ptr(w3), _ptr(o), _ptr(ws),
        _ws_bytes(ws), _stream(w1.device))
    _check(st, "zm_ttt_chunked")
    return o


def make_layer_weights(w_in, w_gate, gamma, eta_scale=0.01, rms_eps=1e-6) -> LayerWeights:
    for t, nm in ((w_in, "w_in"), (w_gate, "w_gate")):
        if t.dtype != torch.bfloat16 or not t.is_contiguous() or t.dim() != 2 or not t.is_cuda:
            raise ZmError(f"{nm} must be a contiguous 2-D bf16 GPU tensor")
    if gamma.dtype != torch.float32 or not gamma.is_contiguous() or not gamma.is_cuda:
        raise ZmError("gamma must be a contiguous fp32 GPU tensor")
    return LayerWeights(w_in.data_ptr(), w_gate.data_ptr(), gamma.data_ptr(), w_in.shape[1],
                        float(eta_scale), float(rms_eps), 0)


def layer_workspace_size(desc: Desc, lw: LayerWeights, n: int) -> int:
    out = ctypes.c_size_t(0)
    _check(load_library().zm_ttt_layer_workspace_size(ctypes.byref(desc), ctypes.byref(lw), int(n),
                                                       ctypes.byref(out)),
           "zm_ttt_layer_workspace_size")
    return int(out.value)


def layer(x, w_in, w_gate, gamma, w1, w2, w3, eta_scale=0.01, rms_eps=1e-6, renorm=False,
          step_rule=STEP_GRADIENT, w_out=None, out=None, workspace=None):
    """The whole layer on one chunk: projections of x [n, d_in] (bf16) to q, k,
    v and the rate, update, apply, output gate.  Returns ((W1_hat, W2_hat,
    W3_hat), o [n, H d] bf16)."""
    heads, d, h = _check_weights(w1, w2, w3, device=False)
    if x.dtype != torch.bfloat16 or x.dim() != 2 or (x.shape[0] > 0 and x.stride(1) != 1):
        raise ZmError("x must be a 2-D bf16 tensor with unit column stride")
    n = x.shape[0]
    if tuple(w_in.shape) != (3 * heads * d + heads, x.shape[1]):
        raise ZmError(f"w_in must be [{3 * heads * d + heads}, {x.shape[1]}]")
    if tuple(w_gate.shape) != (heads * d, heads * d) or tuple(gamma.shape) != (heads * d,):
        raise ZmError("w_gate must be [H d, H d] and gamma [H d]")
    o = out if out is not None else torch.empty((n, heads * d), dtype=torch.bfloat16,
                                                device=x.device)
    if o.dtype != torch.bfloat16 or o.dim() != 2 or tuple(o.shape) != (n, heads * d):
        raise ZmError(f"out must be bf16 [{n}, {heads * d}], got {o.dtype} {tuple(o.shape)}")
    if n > 0 and o.stride(1) != 1:
        raise ZmError("out needs unit column stride")
    outs = w_out if w_out is not None else tuple(torch.empty_like(w) for w in (w1, w2, w3))
    _check_out_weights(outs, w1, w2, w3)
    _on_gpu(x, w1, w2, w3, w_in, w_gate, gamma, o, *outs, what="the layer's tensors")
    desc = Desc(heads, d, h, BF16, RENORM_ROW if renorm else RENORM_NONE, int(step_rule),
                o.stride(0) if n > 1 else heads * d)
    lw = make_layer_weights(w_in, w_gate, gamma, eta_scale, rms_eps)
    need = layer_workspace_size(desc, lw, n)
    ws = workspace if workspace is not None else torch.empty(max(need, 256), dtype=torch.uint8,
                                                             device=x.device)
    st = load_library().zm_ttt_layer(
        ctypes.byref(desc), ctypes.byref(lw), n, _ptr(x), x.stride(0) if n > 1 else x.shape[1],
        _ptr(w1), _ptr(w2), _ptr(w3), *map(_ptr, outs), _ptr(o), _ptr(ws), _ws_bytes(ws),
        _stream(x.device))
    _check(st, "zm_ttt_layer")
    return outs, o


def set_profile_events(events):
    """events: 8, 10 or 14 torch.cuda.Event (or None entries) recorded around
    the kernel stages (cast, update partials, reduce, apply, Newton-Schulz,
    projections, output gate); None switches off."""
    lib = load_library()
    if events is None:
        _check(lib.zm_ttt_set_profile_events(None, 0), "zm_ttt_set_profile_events")
        return
    if len(events) not in (8, 10, 14):
        raise ZmError("need 8, 10 or 14 event slots")
    arr = (ctypes.c_void_p * len(events))()
    for i, e in enumerate(events):
        arr[i] = None if e is None else ctypes.c_void_p(int(e.cuda_event))
    _check(lib.zm_ttt_set_profile_events(arr, len(events)), "zm_ttt_set_profile_events")
