"""MI355X (gfx950) verify-and-supervise pass for diffusion-drafter speculative decoding.

A thin ctypes binding over the C ABI in ``include/adaflash.h`` (built into
``libadaflash.so`` next to this file).  The binding only marshals arguments:
torch tensors provide device memory and the current HIP stream; every step of
the computation runs in the library's kernels.  There is no CPU fallback: if
the library is missing or the tensors are not on the GPU, calls raise.

Entry points (same names as the C ABI):
  adaflash_verify(...)            speculative verification, optional fused supervision
  adaflash_opd_loss_fwd_bwd(...)  supervision only
  adaflash_verify_packed(...), adaflash_opd_loss_fwd_bwd_packed(...)
                                  the same on logits packed request after request
  adaflash_workspace_bytes(B, k, V)
Convenience wrappers allocating the outputs: ``verify`` and ``opd_loss_fwd_bwd``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# ADAFLASH_LIB may name another build of the same library (for example an
# instrumented one); by default the in-tree build next to this file is used.
LIB_PATH = os.environ.get("ADAFLASH_LIB") or os.path.join(_PKG, "libadaflash.so")

ADAFLASH_F32 = 0
ADAFLASH_BF16 = 1
FLAG_BAD_VERIFY_LEN = 1
FLAG_BAD_TOKEN = 2
FLAG_NONFINITE = 4
FLAG_SYNC_TIMEOUT = 8

_lib = None


class AdaflashError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"adaflash error {code}: {msg}")
        self.code = code


def load_library() -> ctypes.CDLL:
    """Loads libadaflash.so (after torch, so both share one HIP runtime)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                              "(the GPU path has no fallback)")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        lib.adaflash_version.restype = i32
        lib.adaflash_version.argtypes = []
        lib.adaflash_last_error.restype = ctypes.c_char_p
        lib.adaflash_last_error.argtypes = []
        lib.adaflash_workspace_bytes.restype = sz
        lib.adaflash_workspace_bytes.argtypes = [i32, i32, i32]
        lib.adaflash_verify.restype = i32
        lib.adaflash_verify.argtypes = [i32, vp, vp, vp, vp, vp, i32, i32, i32, f32, vp, vp, vp,
                                        f32, f32, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.adaflash_verify_noalloc.restype = i32
        lib.adaflash_verify_noalloc.argtypes = [i32, vp, vp, vp, vp, vp, i32, i32, i32, f32, vp, vp, vp,
                                                f32, f32, vp, vp, vp, vp, vp, vp]
        lib.adaflash_opd_loss_fwd_bwd.restype = i32
        lib.adaflash_opd_loss_fwd_bwd.argtypes = [i32, vp, vp, vp, i32, i32, i32, f32, f32, vp, vp,
                                                  vp, vp, vp, vp, sz, vp]
        lib.adaflash_timing_enable.restype = i32
        lib.adaflash_timing_enable.argtypes = [i32]
        lib.adaflash_timing_read.restype = i32
        lib.adaflash_timing_read.argtypes = [ctypes.POINTER(ctypes.c_float), i32]
        lib.adaflash_timing_every.restype = i32
        lib.adaflash_timing_every.argtypes = [i32]
        lib.adaflash_verify_packed.restype = i32
        lib.adaflash_verify_packed.argtypes = lib.adaflash_verify.argtypes
        lib.adaflash_opd_loss_fwd_bwd_packed.restype = i32
        lib.adaflash_opd_loss_fwd_bwd_packed.argtypes = lib.adaflash_opd_loss_fwd_bwd.argtypes
        lib.adaflash_loss_variant_fwd_bwd.restype = i32
        lib.adaflash_loss_variant_fwd_bwd.argtypes = [i32, vp, vp, vp, i32, i32, i32, i32, f32, f32, vp, vp, vp,
                                                      vp, vp, sz, vp]
        i64p = ctypes.POINTER(ctypes.c_int64)
        lib.adaflash_admission_create.restype = vp
        lib.adaflash_admission_create.argtypes = [ctypes.c_double, ctypes.c_double, ctypes.c_int64]
        lib.adaflash_admission_destroy.restype = None
        lib.adaflash_admission_destroy.argtypes = [vp]
        lib.adaflash_admission_enqueue.restype = i32
        lib.adaflash_admission_enqueue.argtypes = [vp, i64p, i32]
        lib.adaflash_admission_propose.restype = i32
        lib.adaflash_admission_propose.argtypes = [vp, i64p, i32]
        lib.adaflash_admission_commit.restype = i32
        lib.adaflash_admission_commit.argtypes = [vp, ctypes.POINTER(ctypes.c_int32), i32, i64p]
        lib.adaflash_admission_finish.restype = i32
        lib.adaflash_admission_finish.argtypes = [vp, i64p, i32]
        lib.adaflash_admission_estimate.restype = ctypes.c_double
        lib.adaflash_admission_estimate.argtypes = [vp]
        lib.adaflash_admission_pending.restype = i32
        lib.adaflash_admission_pending.argtypes = [vp]
        lib.adaflash_length_head_workspace_bytes.restype = sz
        lib.adaflash_length_head_workspace_bytes.argtypes = [i32, i32, i32, i32]
        lib.adaflash_length_head_forward.restype = i32
        lib.adaflash_length_head_forward.argtypes = [vp, vp, vp, vp, f32, i32, i32, i32, i32, f32, vp, vp,
                                                     vp, sz, vp]
        lib.adaflash_length_head_backward.restype = i32
        lib.adaflash_length_head_backward.argtypes = [vp, vp, vp, vp, f32, i32, i32, i32, i32, vp, vp, vp,
                                                      vp, vp, vp, vp, vp, sz, vp]
        lib.adaflash_length_head_forward_cached.restype = i32
        lib.adaflash_length_head_forward_cached.argtypes = (lib.adaflash_length_head_forward.argtypes[:12] + [vp]
                                                            + lib.adaflash_length_head_forward.argtypes[12:])
        lib.adaflash_length_head_backward_cached.restype = i32
        lib.adaflash_length_head_backward_cached.argtypes = (lib.adaflash_length_head_backward.argtypes[:16] + [vp]
                                                             + lib.adaflash_length_head_backward.argtypes[16:])
        _lib = lib
    return _lib


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("adaflash works on GPU tensors only")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return ADAFLASH_BF16
    if t.dtype == torch.float32:
        return ADAFLASH_F32
    raise TypeError("logits must be bfloat16 or float32")


def _arg(t: Optional[torch.Tensor], name: str, dtype, shape=None, min_rows=None, row_len=None,
         optional: bool = False) -> None:
    """Host-side check of one tensor argument before its pointer reaches the
    library (the C ABI sees raw pointers and cannot check sizes itself):
    dtype, exact shape, or at least ``min_rows`` leading rows of ``row_len``
    entries each."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    dts = dtype if isinstance(dtype, tuple) else (dtype,)
    if t.dtype not in dts:
        raise TypeError(f"{name} must be {' or '.join(str(d) for d in dts)}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if min_rows is not None:
        if row_len is None:
            if t.dim() != 1 or t.shape[0] < min_rows:
                raise ValueError(f"{name} must be 1-D with at least {min_rows} entries, got {tuple(t.shape)}")
        elif t.dim() != 2 or t.shape[0] < min_rows or t.shape[1] != row_len:
            raise ValueError(f"{name} must be [>= {min_rows}, {row_len}], got {tuple(t.shape)}")


def _logits(t: torch.Tensor, name: str, ndim: int) -> None:
    if t is None:
        raise ValueError(f"{name} is required")
    _dtype_code(t)
    if t.dim() != ndim:
        raise ValueError(f"{name} must be {ndim}-D, got {tuple(t.shape)}")


def _check_outputs(B: int, k: int, V: int, ldtype, n_rows: int, accept_len=None, out_tokens=None, margins=None,
                   row_offsets=None, loss_ce=None, loss_rkl=None, grad=None, status=None, ws=None,
                   verify: bool = True) -> None:
    if verify:
        _arg(accept_len, "accept_len", torch.int32, (B,))
        _arg(out_tokens, "out_tokens", torch.int32, (B, k + 1))
        _arg(margins, "margins", torch.float32, (B, k + 1), optional=True)
    _arg(row_offsets, "row_offsets", torch.int32, (B + 1,))
    _arg(loss_ce, "loss_ce", torch.float32, min_rows=n_rows, optional=True)
    _arg(loss_rkl, "loss_rkl", torch.float32, min_rows=n_rows, optional=True)
    _arg(grad, "grad_draft", ldtype, min_rows=n_rows, row_len=V, optional=True)
    if status is not None:
        _arg(status, "status", torch.int32, min_rows=1)
    if ws is not None and ws.dtype != torch.uint8:
        raise TypeError("the workspace must be a uint8 tensor (its size is counted in bytes)")


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _check(rc: int):
    if rc != 0:
        raise AdaflashError(rc, load_library().adaflash_last_error().decode())


class PreparedCall:
    """One entry-point call, checked and marshalled once, for repetition:
    run() repeats the C call with the same tensors, sizes and stream (the
    tensors must keep their storage, shapes and dtypes meanwhile; the object
    holds references to them).  Returned by the direct bindings when called
    with prepare=True."""

    def __init__(self, fn, args, keep):
        self._fn = fn
        self._args = tuple(t(a) for t, a in zip(fn.argtypes, args))
        self._keep = keep

    def run(self) -> None:
        rc = self._fn(*self._args)
        if rc != 0:
            _check(rc)


def _invoke(fn, args, keep, prepare: bool):
    if prepare:
        return PreparedCall(fn, args, keep)
    _check(fn(*args))


def adaflash_timing_enable(max_records: int) -> None:
    """Direct binding of adaflash_timing_enable (benchmark hook)."""
    _check(load_library().adaflash_timing_enable(int(max_records)))


def adaflash_timing_every(n: int) -> None:
    """Direct binding of adaflash_timing_every (events on every n-th call)."""
    _check(load_library().adaflash_timing_every(int(n)))


def adaflash_timing_read(cap: int) -> list:
    """Direct binding of adaflash_timing_read: the recorded dominant-kernel
    durations in milliseconds."""
    buf = (ctypes.c_float * max(int(cap), 1))()
    n = load_library().adaflash_timing_read(buf, int(cap))
    if n < 0:
        _check(n)
    return [float(buf[i]) for i in range(n)]


def adaflash_workspace_bytes(B: int, k: int, V: int) -> int:
    return int(load_library().adaflash_workspace_bytes(B, k, V))


def workspace(B: int, k: int, V: int, device="cuda") -> torch.Tensor:
    n = adaflash_workspace_bytes(B, k, V)
    if n == 0:
        raise ValueError("invalid sizes")
    return torch.empty(n, dtype=torch.uint8, device=device)


def adaflash_verify(target, draft, tokens, verify_len, uniforms, T, accept_len, out_tokens, margins,
                    clip_c, lam, row_offsets, loss_ce, loss_rkl, grad_draft, status, ws,
                    stream=None, prepare: bool = False):
    """Direct binding of adaflash_verify (see include/adaflash.h)."""
    _logits(target, "target", 3)
    B, k1, V = target.shape
    k = k1 - 1
    opd = loss_ce is not None or loss_rkl is not None or grad_draft is not None
    _arg(draft, "draft", target.dtype, (B, k, V), optional=(T == 0 and not opd))
    _arg(tokens, "tokens", torch.int32, (B, k))
    _arg(verify_len, "verify_len", torch.int32, (B,))
    _arg(uniforms, "uniforms", torch.float32, (B, k + 1), optional=(T == 0))
    _check_outputs(B, k, V, target.dtype, B * k, accept_len, out_tokens, margins, row_offsets, loss_ce, loss_rkl,
                   grad_draft, status, ws)
    args = (
        _dtype_code(target), _ptr(target), _ptr(draft), _ptr(tokens), _ptr(verify_len), _ptr(uniforms),
        B, k1 - 1, V, float(T), _ptr(accept_len), _ptr(out_tokens), _ptr(margins), float(clip_c),
        float(lam), _ptr(row_offsets), _ptr(loss_ce), _ptr(loss_rkl), _ptr(grad_draft), _ptr(status),
        _ptr(ws), ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream))
    keep = (accept_len, draft, grad_draft, loss_ce, loss_rkl, margins, out_tokens, row_offsets, status, target,
            tokens, uniforms, verify_len, ws)
    return _invoke(load_library().adaflash_verify, args, keep, prepare)


NOALLOC_WORKSPACE_BYTES = 16 << 20  # ADAFLASH_NOALLOC_WORKSPACE_BYTES


def adaflash_verify_noalloc(target, draft, tokens, verify_len, uniforms, T, accept_len, out_tokens, margins,
                            clip_c, lam, row_offsets, loss_ce, loss_rkl, grad_draft, status, stream=None,
                            prepare: bool = False):
    """Direct binding of adaflash_verify_noalloc: adaflash_verify without a
    workspace argument (the library's own device array is used; calls that
    overlap on one GPU race)."""
    _logits(target, "target", 3)
    B, k1, V = target.shape
    k = k1 - 1
    opd = loss_ce is not None or loss_rkl is not None or grad_draft is not None
    _arg(draft, "draft", target.dtype, (B, k, V), optional=(T == 0 and not opd))
    _arg(tokens, "tokens", torch.int32, (B, k))
    _arg(verify_len, "verify_len", torch.int32, (B,))
    _arg(uniforms, "uniforms", torch.float32, (B, k + 1), optional=(T == 0))
    _check_outputs(B, k, V, target.dtype, B * k, accept_len, out_tokens, margins, row_offsets, loss_ce, loss_rkl,
                   grad_draft, status)
    args = (
        _dtype_code(target), _ptr(target), _ptr(draft), _ptr(tokens), _ptr(verify_len), _ptr(uniforms),
        B, k, V, float(T), _ptr(accept_len), _ptr(out_tokens), _ptr(margins), float(clip_c),
        float(lam), _ptr(row_offsets), _ptr(loss_ce), _ptr(loss_rkl), _ptr(grad_draft), _ptr(status),
        _stream(stream))
    keep = (accept_len, draft, grad_draft, loss_ce, loss_rkl, margins, out_tokens, row_offsets, status, target,
            tokens, uniforms, verify_len)
    return _invoke(load_library().adaflash_verify_noalloc, args, keep, prepare)


def adaflash_opd_loss_fwd_bwd(target, draft, verify_len, clip_c, lam, row_offsets, loss_ce,
                              loss_rkl, grad_draft, status, ws, stream=None, prepare: bool = False):
    """Direct binding of adaflash_opd_loss_fwd_bwd (see include/adaflash.h)."""
    _logits(target, "target", 3)
    B, k1, V = target.shape
    _arg(draft, "draft", target.dtype, (B, k1 - 1, V))
    _arg(verify_len, "verify_len", torch.int32, (B,), optional=True)
    _check_outputs(B, k1 - 1, V, target.dtype, B * (k1 - 1), row_offsets=row_offsets, loss_ce=loss_ce,
                   loss_rkl=loss_rkl, grad=grad_draft, status=status, ws=ws, verify=False)
    args = (
        _dtype_code(target), _ptr(target), _ptr(draft), _ptr(verify_len), B, k1 - 1, V, float(clip_c),
        float(lam), _ptr(row_offsets), _ptr(loss_ce), _ptr(loss_rkl), _ptr(grad_draft), _ptr(status),
        _ptr(ws), ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream))
    keep = (draft, grad_draft, loss_ce, loss_rkl, row_offsets, status, target, verify_len, ws)
    return _invoke(load_library().adaflash_opd_loss_fwd_bwd, args, keep, prepare)


def adaflash_verify_packed(target, draft, tokens, verify_len, uniforms, T, accept_len, out_tokens, margins,
                           clip_c, lam, row_offsets, loss_ce, loss_rkl, grad_draft, status, ws,
                           stream=None, prepare: bool = False):
    """Direct binding of adaflash_verify_packed: target [sum(L_b+1), V], draft
    [sum L_b, V]; B and k come from tokens [B, k].  The row counts must match
    the device-side verify lengths (sum(L_b + 1) and sum L_b rows): the library
    locates rows through them."""
    _logits(target, "target", 2)
    _arg(tokens, "tokens", torch.int32)
    if tokens.dim() != 2:
        raise ValueError(f"tokens must be [B, k], got {tuple(tokens.shape)}")
    B, k = tokens.shape
    V = target.shape[-1]
    opd = loss_ce is not None or loss_rkl is not None or grad_draft is not None
    _arg(draft, "draft", target.dtype, optional=(T == 0 and not opd))
    n_rows = target.shape[0] - B
    if draft is not None:
        if draft.dim() != 2 or draft.shape[1] != V or draft.shape[0] + B != target.shape[0]:
            raise ValueError(f"packed draft must be [sum L_b, V] with sum L_b = target rows - B, got "
                             f"{tuple(draft.shape)} for target {tuple(target.shape)} and B = {B}")
        n_rows = draft.shape[0]
    if target.shape[0] < 2 * B or target.shape[0] > B * (k + 1):
        raise ValueError(f"packed target must hold between 2 B and B (k + 1) rows, got {target.shape[0]}")
    _arg(verify_len, "verify_len", torch.int32, (B,))
    _arg(uniforms, "uniforms", torch.float32, (B, k + 1), optional=(T == 0))
    _check_outputs(B, k, V, target.dtype, n_rows, accept_len, out_tokens, margins, row_offsets, loss_ce, loss_rkl,
                   grad_draft, status, ws)
    args = (
        _dtype_code(target), _ptr(target), _ptr(draft), _ptr(tokens), _ptr(verify_len), _ptr(uniforms),
        B, k, V, float(T), _ptr(accept_len), _ptr(out_tokens), _ptr(margins), float(clip_c),
        float(lam), _ptr(row_offsets), _ptr(loss_ce), _ptr(loss_rkl), _ptr(grad_draft), _ptr(status),
        _ptr(ws), ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream))
    keep = (accept_len, draft, grad_draft, loss_ce, loss_rkl, margins, out_tokens, row_offsets, status, target,
            tokens, uniforms, verify_len, ws)
    return _invoke(load_library().adaflash_verify_packed, args, keep, prepare)


def adaflash_opd_loss_fwd_bwd_packed(target, draft, verify_len, k, clip_c, lam, row_offsets, loss_ce,
                                     loss_rkl, grad_draft, status, ws, stream=None, prepare: bool = False):
    """Direct binding of adaflash_opd_loss_fwd_bwd_packed: target
    [sum(L_b+1), V], draft [sum L_b, V]; B from verify_len [B]."""
    _logits(target, "target", 2)
    _arg(verify_len, "verify_len", torch.int32)
    if verify_len.dim() != 1:
        raise ValueError(f"verify_len must be [B], got {tuple(verify_len.shape)}")
    B = verify_len.shape[0]
    V = target.shape[-1]
    _logits(draft, "draft", 2)
    _arg(draft, "draft", target.dtype)
    if draft.shape[1] != V or draft.shape[0] + B != target.shape[0] or draft.shape[0] > B * int(k):
        raise ValueError(f"packed draft must be [sum L_b, V] with sum L_b = target rows - B <= B k, got "
                         f"{tuple(draft.shape)} for target {tuple(target.shape)}, B = {B}, k = {k}")
    _check_outputs(B, int(k), V, target.dtype, draft.shape[0], row_offsets=row_offsets, loss_ce=loss_ce,
                   loss_rkl=loss_rkl, grad=grad_draft, status=status, ws=ws, verify=False)
    args = (
        _dtype_code(target), _ptr(target), _ptr(draft), _ptr(verify_len), B, int(k), V, float(clip_c),
        float(lam), _ptr(row_offsets), _ptr(loss_ce), _ptr(loss_rkl), _ptr(grad_draft), _ptr(status),
        _ptr(ws), ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream))
    keep = (draft, grad_draft, loss_ce, loss_rkl, row_offsets, status, target, verify_len, ws)
    return _invoke(load_library().adaflash_opd_loss_fwd_bwd_packed, args, keep, prepare)


def verify(target: torch.Tensor, draft: Optional[torch.Tensor], tokens: torch.Tensor,
           verify_len: torch.Tensor, uniforms: Optional[torch.Tensor], T: float,
           opd: bool = False, clip_c: float = 10.0, lam: float = 1.0, margins: bool = True,
           ws: Optional[torch.Tensor] = None, stream=None) -> dict:
    """Allocates the outputs and calls adaflash_verify.  The supervision
    outputs (loss_ce, loss_rkl, grad [B*k, V] of which N rows are written)
    are produced only when ``opd`` is true."""
    B, k1, V = target.shape
    k = k1 - 1
    dev = target.device
    out = {
        "accept_len": torch.empty(B, dtype=torch.int32, device=dev),
        "out_tokens": torch.empty(B, k1, dtype=torch.int32, device=dev),
        "margins": torch.empty(B, k1, dtype=torch.float32, device=dev) if margins else None,
        "row_offsets": torch.empty(B + 1, dtype=torch.int32, device=dev),
        "status": torch.empty(1, dtype=torch.int32, device=dev),
        "loss_ce": None, "loss_rkl": None, "grad": None,
    }
    if opd:
        out["loss_ce"] = torch.empty(B * k, dtype=torch.float32, device=dev)
        out["loss_rkl"] = torch.empty(B * k, dtype=torch.float32, device=dev)
        out["grad"] = torch.empty(B * k, V, dtype=target.dtype, device=dev)
    if ws is None:
        ws = workspace(B, k, V, dev)
    adaflash_verify(target, draft, tokens, verify_len, uniforms, T, out["accept_len"],
                    out["out_tokens"], out["margins"], clip_c, lam, out["row_offsets"], out["loss_ce"],
                    out["loss_rkl"], out["grad"], out["status"], ws, stream)
    return out


def opd_loss_fwd_bwd(target: torch.Tensor, draft: torch.Tensor, verify_len: Optional[torch.Tensor],
                     clip_c: float = 10.0, lam: float = 1.0, with_grad: bool = True,
                     ws: Optional[torch.Tensor] = None, stream=None) -> dict:
    """Allocates the outputs and calls adaflash_opd_loss_fwd_bwd."""
    B, k1, V = target.shape
    k = k1 - 1
    dev = target.device
    out = {
        "row_offsets": torch.empty(B + 1, dtype=torch.int32, device=dev),
        "status": torch.empty(1, dtype=torch.int32, device=dev),
        "loss_ce": torch.empty(B * k, dtype=torch.float32, device=dev),
        "loss_rkl": torch.empty(B * k, dtype=torch.float32, device=dev),
        "grad": torch.empty(B * k, V, dtype=target.dtype, device=dev) if with_grad else None,
    }
    if ws is None:
        ws = workspace(B, k, V, dev)
    adaflash_opd_loss_fwd_bwd(target, draft, verify_len, clip_c, lam, out["row_offsets"],
                              out["loss_ce"], out["loss_rkl"], out["grad"], out["status"], ws, stream)
    return out


def verify_packed(target: torch.Tensor, draft: Optional[torch.Tensor], tokens: torch.Tensor,
                  verify_len: torch.Tensor, uniforms: Optional[torch.Tensor], T: float,
                  opd: bool = False, clip_c: float = 10.0, lam: float = 1.0, margins: bool = True,
                  ws: Optional[torch.Tensor] = None, stream=None) -> dict:
    """As ``verify`` on packed logits (target [sum(L_b+1), V], draft
    [sum L_b, V]); the gradient has one row per draft row."""
    B, k = tokens.shape
    V = target.shape[-1]
    dev = target.device
    out = {
        "accept_len": torch.empty(B, dtype=torch.int32, device=dev),
        "out_tokens": torch.empty(B, k + 1, dtype=torch.int32, device=dev),
        "margins": torch.empty(B, k + 1, dtype=torch.float32, device=dev) if margins else None,
        "row_offsets": torch.empty(B + 1, dtype=torch.int32, device=dev),
        "status": torch.empty(1, dtype=torch.int32, device=dev),
        "loss_ce": None, "loss_rkl": None, "grad": None,
    }
    if opd:
        n = draft.shape[0]
        out["loss_ce"] = torch.empty(max(n, 1), dtype=torch.float32, device=dev)
        out["loss_rkl"] = torch.empty(max(n, 1), dtype=torch.float32, device=dev)
        out["grad"] = torch.empty(max(n, 1), V, dtype=target.dtype, device=dev)
    if ws is None:
        ws = workspace(B, k, V, dev)
    adaflash_verify_packed(target, draft, tokens, verify_len, uniforms, T, out["accept_len"],
                           out["out_tokens"], out["margins"], clip_c, lam, out["row_offsets"], out["loss_ce"],
                           out["loss_rkl"], out["grad"], out["status"], ws, stream)
    return out


def opd_loss_fwd_bwd_packed(target: torch.Tensor, draft: torch.Tensor, verify_len: torch.Tensor, k: int,
                            clip_c: float = 10.0, lam: float = 1.0, with_grad: bool = True,
                            ws: Optional[torch.Tensor] = None, stream=None) -> dict:
    """As ``opd_loss_fwd_bwd`` on packed logits."""
    B = verify_len.shape[0]
    V = target.shape[-1]
    dev = target.device
    n = max(draft.shape[0], 1)
    out = {
        "row_offsets": torch.empty(B + 1, dtype=torch.int32, device=dev),
        "status": torch.empty(1, dtype=torch.int32, device=dev),
        "loss_ce": torch.empty(n, dtype=torch.float32, device=dev),
        "loss_rkl": torch.empty(n, dtype=torch.float32, device=dev),
        "grad": torch.empty(n, V, dtype=target.dtype, device=dev) if with_grad else None,
    }
    if ws is None:
        ws = workspace(B, k, V, dev)
    adaflash_opd_loss_fwd_bwd_packed(target, draft, verify_len, k, clip_c, lam, out["row_offsets"],
                                     out["loss_ce"], out["loss_rkl"], out["grad"], out["status"], ws, stream)
    return out


# ----------------------------------------------------------- loss variants

LOSS_VARIANTS = {"rkl": 1, "rkl_clip": 2, "mixture": 3, "fkl": 4, "wce": 5}


def adaflash_loss_variant_fwd_bwd(target, draft, verify_len, variant, p1, p2, row_offsets, loss, grad_draft, status,
                                  ws, stream=None, prepare: bool = False):
    """Direct binding of adaflash_loss_variant_fwd_bwd (see include/adaflash.h)."""
    _logits(target, "target", 3)
    B, k1, V = target.shape
    _arg(draft, "draft", target.dtype, (B, k1 - 1, V))
    _arg(verify_len, "verify_len", torch.int32, (B,), optional=True)
    _check_outputs(B, k1 - 1, V, target.dtype, B * (k1 - 1), row_offsets=row_offsets, loss_ce=loss, grad=grad_draft,
                   status=status, ws=ws, verify=False)
    code = LOSS_VARIANTS[variant] if isinstance(variant, str) else int(variant)
    args = (
        _dtype_code(target), _ptr(target), _ptr(draft), _ptr(verify_len), B, k1 - 1, V, code, float(p1),
        float(p2), _ptr(row_offsets), _ptr(loss), _ptr(grad_draft), _ptr(status), _ptr(ws),
        ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream))
    keep = (draft, grad_draft, loss, row_offsets, status, target, verify_len, ws)
    return _invoke(load_library().adaflash_loss_variant_fwd_bwd, args, keep, prepare)


def loss_variant_fwd_bwd(target: torch.Tensor, draft: torch.Tensor, verify_len: Optional[torch.Tensor], variant,
                         p1: float = 0.0, p2: float = 0.0, with_grad: bool = True, ws: Optional[torch.Tensor] = None,
                         stream=None) -> dict:
    """Allocates the outputs and calls adaflash_loss_variant_fwd_bwd."""
    B, k1, V = target.shape
    k = k1 - 1
    dev = target.device
    out = {
        "row_offsets": torch.empty(B + 1, dtype=torch.int32, device=dev),
        "status": torch.empty(1, dtype=torch.int32, device=dev),
        "loss": torch.empty(B * k, dtype=torch.float32, device=dev),
        "grad": torch.empty(B * k, V, dtype=target.dtype, device=dev) if with_grad else None,
    }
    if ws is None:
        ws = workspace(B, k, V, dev)
    adaflash_loss_variant_fwd_bwd(target, draft, verify_len, variant, p1, p2, out["row_offsets"], out["loss"],
                                  out["grad"], out["status"], ws, stream)
    return out


# ------------------------------------------------------------- length head


def adaflash_length_head_workspace_bytes(B: int, k: int, H: int, Hp: int) -> int:
    return int(load_library().adaflash_length_head_workspace_bytes(B, k, H, Hp))


def length_head_workspace(B: int, k: int, H: int, Hp: int, device="cuda") -> torch.Tensor:
    n = adaflash_length_head_workspace_bytes(B, k, H, Hp)
    if n == 0:
        raise ValueError("invalid sizes")
    return torch.empty(n, dtype=torch.uint8, device=device)


def _lh_inputs(hidden, W1, b1, w2):
    _arg(hidden, "hidden", torch.bfloat16)
    if hidden.dim() != 3:
        raise ValueError(f"hidden must be [B, k, H], got {tuple(hidden.shape)}")
    B, k, H = hidden.shape
    _arg(W1, "W1", torch.bfloat16)
    if W1.dim() != 2 or W1.shape[1] != H:
        raise ValueError(f"W1 must be [H', {H}], got {tuple(W1.shape)}")
    Hp = W1.shape[0]
    _arg(b1, "b1", torch.float32, (Hp,))
    _arg(w2, "w2", torch.float32, (Hp,))
    return B, k, H, Hp


def _lh_workspace(ws):
    if ws is not None and ws.dtype != torch.uint8:
        raise TypeError("the workspace must be a uint8 tensor (its size is counted in bytes)")
    return ws.numel() * ws.element_size() if ws is not None else 0


def adaflash_length_head_forward(hidden, W1, b1, w2, b2, gamma, a_hat, k_hat, ws, stream=None,
                                 z1_cache=None, prepare: bool = False):
    """Direct binding of adaflash_length_head_forward, or of
    adaflash_length_head_forward_cached when z1_cache ([B k, H'] fp32) is given."""
    B, k, H, Hp = _lh_inputs(hidden, W1, b1, w2)
    _arg(a_hat, "a_hat", torch.float32, (B,), optional=True)
    _arg(k_hat, "k_hat", torch.int32, (B,), optional=True)
    _arg(z1_cache, "z1_cache", torch.float32, (B * k, Hp), optional=True)
    lib = load_library()
    head = (_ptr(hidden), _ptr(W1), _ptr(b1), _ptr(w2), float(b2), B, k, H, Hp, float(gamma), _ptr(a_hat),
            _ptr(k_hat))
    tail = (_ptr(ws), _lh_workspace(ws), _stream(stream))
    keep = (hidden, W1, b1, w2, a_hat, k_hat, z1_cache, ws)
    if z1_cache is None:
        return _invoke(lib.adaflash_length_head_forward, head + tail, keep, prepare)
    return _invoke(lib.adaflash_length_head_forward_cached, head + (_ptr(z1_cache),) + tail, keep, prepare)


def adaflash_length_head_backward(hidden, W1, b1, w2, b2, accept_len, verify_len, loss, dW1, db1, dw2, db2, ws,
                                  stream=None, z1_cache=None, prepare: bool = False):
    """Direct binding of adaflash_length_head_backward, or of
    adaflash_length_head_backward_cached when z1_cache (the forward's) is given."""
    B, k, H, Hp = _lh_inputs(hidden, W1, b1, w2)
    _arg(accept_len, "accept_len", torch.int32, (B,))
    _arg(verify_len, "verify_len", torch.int32, (B,))
    _arg(loss, "loss", torch.float32, (B,), optional=True)
    _arg(dW1, "dW1", torch.float32, (Hp, H), optional=True)
    _arg(db1, "db1", torch.float32, (Hp,), optional=True)
    _arg(dw2, "dw2", torch.float32, (Hp,), optional=True)
    _arg(db2, "db2", torch.float32, min_rows=1, optional=True)
    _arg(z1_cache, "z1_cache", torch.float32, (B * k, Hp), optional=True)
    lib = load_library()
    head = (_ptr(hidden), _ptr(W1), _ptr(b1), _ptr(w2), float(b2), B, k, H, Hp, _ptr(accept_len), _ptr(verify_len),
            _ptr(loss), _ptr(dW1), _ptr(db1), _ptr(dw2), _ptr(db2))
    tail = (_ptr(ws), _lh_workspace(ws), _stream(stream))
    keep = (hidden, W1, b1, w2, accept_len, verify_len, loss, dW1, db1, dw2, db2, z1_cache, ws)
    if z1_cache is None:
        return _invoke(lib.adaflash_length_head_backward, head + tail, keep, prepare)
    return _invoke(lib.adaflash_length_head_backward_cached, head + (_ptr(z1_cache),) + tail, keep, prepare)


def length_head_forward(hidden: torch.Tensor, W1: torch.Tensor, b1: torch.Tensor, w2: torch.Tensor, b2: float,
                        gamma: float = 1.0, ws: Optional[torch.Tensor] = None, stream=None,
                        keep_projection: bool = False) -> dict:
    """Allocates the outputs and calls adaflash_length_head_forward; with
    keep_projection, out["z1"] holds the projection for the backward."""
    B, k, H = hidden.shape
    dev = hidden.device
    out = {"a_hat": torch.empty(B, dtype=torch.float32, device=dev),
           "k_hat": torch.empty(B, dtype=torch.int32, device=dev)}
    if keep_projection:
        out["z1"] = torch.empty(B * k, W1.shape[0], dtype=torch.float32, device=dev)
    if ws is None:
        ws = length_head_workspace(B, k, H, W1.shape[0], dev)
    adaflash_length_head_forward(hidden, W1, b1, w2, b2, gamma, out["a_hat"], out["k_hat"], ws, stream,
                                 z1_cache=out.get("z1"))
    return out


def length_head_backward(hidden: torch.Tensor, W1: torch.Tensor, b1: torch.Tensor, w2: torch.Tensor, b2: float,
                         accept_len: torch.Tensor, verify_len: torch.Tensor, ws: Optional[torch.Tensor] = None,
                         stream=None, z1: Optional[torch.Tensor] = None) -> dict:
    """Allocates the outputs and calls adaflash_length_head_backward (with z1,
    the forward's kept projection, instead of recomputing it)."""
    B, k, H = hidden.shape
    Hp = W1.shape[0]
    dev = hidden.device
    out = {"loss": torch.empty(B, dtype=torch.float32, device=dev),
           "dW1": torch.empty(Hp, H, dtype=torch.float32, device=dev),
           "db1": torch.empty(Hp, dtype=torch.float32, device=dev),
           "dw2": torch.empty(Hp, dtype=torch.float32, device=dev),
           "db2": torch.empty(1, dtype=torch.float32, device=dev)}
    if ws is None:
        ws = length_head_workspace(B, k, H, Hp, dev)
    adaflash_length_head_backward(hidden, W1, b1, w2, b2, accept_len, verify_len, out["loss"], out["dW1"],
                                  out["db1"], out["dw2"], out["db2"], ws, stream, z1_cache=z1)
    return out


# -------------------------------------------------------- admission control


class Admission:
    """Host-side admission controller (binding of adaflash_admission_*)."""

    def __init__(self, beta: float, n_hat0: float, budget_tokens: int):
        import numpy as np
        self._np = np
        self._lib = load_library()
        self._h = self._lib.adaflash_admission_create(float(beta), float(n_hat0), int(budget_tokens))
        if not self._h:
            raise ValueError("need 0 < beta <= 1, n_hat0 >= 0, budget_tokens >= 1")
        self._buf = np.empty(1024, dtype=np.int64)

    def __del__(self):
        if getattr(self, "_h", None):
            self._lib.adaflash_admission_destroy(self._h)
            self._h = None

    def _i64(self, a):
        a = self._np.ascontiguousarray(a, dtype=self._np.int64)
        return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))

    def enqueue(self, ids):
        a, p = self._i64(ids)
        _check(self._lib.adaflash_admission_enqueue(self._h, p, len(a)))

    def propose(self):
        while True:
            n = self._lib.adaflash_admission_propose(self._h, self._buf.ctypes.data_as(
                ctypes.POINTER(ctypes.c_int64)), len(self._buf))
            if n >= 0:
                return self._buf[:n].tolist()
            self._buf = self._np.empty(2 * len(self._buf), dtype=self._np.int64)

    def commit(self, k_hat):
        k = self._np.ascontiguousarray(k_hat, dtype=self._np.int32)
        out = self._np.empty(max(1, len(k)), dtype=self._np.int64)
        m = self._lib.adaflash_admission_commit(self._h, k.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), len(k),
                                                out.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)))
        if m < 0:
            _check(m)
        return out[:m].tolist()

    def finish(self, done_ids):
        a, p = self._i64(done_ids)
        _check(self._lib.adaflash_admission_finish(self._h, p, len(a)))

    @property
    def n_hat(self) -> float:
        return float(self._lib.adaflash_admission_estimate(self._h))

    @property
    def pending(self) -> int:
        return int(self._lib.adaflash_admission_pending(self._h))
