"""CPU oracle -- TEST INFRASTRUCTURE ONLY.

ctypes wrapper over ``oracle.cpp`` (built into ``liboracle.so``): a plain
double-precision reference for the verify-and-supervise pass.  Only the tests,
the package smoke check and the benchmark's CPU-baseline leg may import this
module.  It shares no code with the GPU library and never imports it.

The functions follow, in order, the AdaFlash review's speculative-sampling
steps and Algorithms 1-2 and the DFlash reading notes' section 5 (eqs. 6-8);
see ``oracle.cpp`` for the passage each step follows and the readings taken
where the pages leave a step open.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")

NEG_RESAMPLE_TARGET = 1
NEG_ARGMAX = 2


def build(verbose: bool = False) -> str:
    """Compile oracle.cpp into liboracle.so (host code, no fast-math, no FMA contraction)."""
    import subprocess
    src = os.path.join(_HERE, "oracle.cpp")
    tmp = LIB_PATH + ".tmp"
    cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
           "-fno-fast-math", "-o", tmp, src]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, f64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        lib.oracle_verify.restype = i32
        lib.oracle_verify.argtypes = [i32, vp, vp, vp, vp, vp, i32, i32, i32, f64, vp, vp, vp, vp,
                                      vp, i32, i32]
        lib.oracle_opd.restype = i64
        lib.oracle_opd.argtypes = [i32, vp, vp, vp, i32, i32, i32, f64, f64, vp, i64, vp, vp, vp, i32]
        _lib = lib
    return _lib


def _threads(n: Optional[int]) -> int:
    return n if n else max(1, min(16, os.cpu_count() or 1))


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return 1
    if a.dtype == np.float32:
        return 0
    raise TypeError("logits must be float32 or uint16 (bf16 bits)")


def _ptr(a):
    return None if a is None else a.ctypes.data


def verify(target: np.ndarray, draft: Optional[np.ndarray], tokens: np.ndarray,
           verify_len: Optional[np.ndarray], uniforms: np.ndarray, T: float, flags: int = 0,
           nthreads: Optional[int] = None) -> dict:
    """Speculative verification of a batch in double precision.

    Returns accept_len [B], out_tokens [B, k+1], margins [B, k+1],
    sample_info [B, 4] = (total mass, threshold, running sum before the token,
    running sum after it) and accept_pq [B, k, 2] = (p(x_i), u_i q(x_i)) of
    every accept test (NaN where no test is defined)."""
    B, k1, V = target.shape
    k = k1 - 1
    target = np.ascontiguousarray(target)
    draft = None if draft is None else np.ascontiguousarray(draft)
    if T > 0 and draft is None:
        raise ValueError("sampled verification needs draft logits")
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    vl = None if verify_len is None else np.ascontiguousarray(verify_len, dtype=np.int32)
    uni = np.ascontiguousarray(uniforms, dtype=np.float32)
    acc = np.empty((B,), dtype=np.int32)
    out = np.empty((B, k + 1), dtype=np.int32)
    mg = np.empty((B, k + 1), dtype=np.float64)
    si = np.empty((B, 4), dtype=np.float64)
    pq = np.empty((B, k, 2), dtype=np.float64)
    rc = _load().oracle_verify(_dtype_code(target), _ptr(target), _ptr(draft), _ptr(tokens), _ptr(vl),
                               _ptr(uni), B, k, V, float(T), _ptr(acc), _ptr(out), _ptr(mg), _ptr(si),
                               _ptr(pq), int(flags), _threads(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_verify rejected its arguments ({rc})")
    return {"accept_len": acc, "out_tokens": out, "margins": mg, "sample_info": si, "accept_pq": pq}


def opd(target: np.ndarray, draft: np.ndarray, verify_len: Optional[np.ndarray], clip_c: float,
        lam: float, rows: Optional[np.ndarray] = None, with_grad: bool = True,
        nthreads: Optional[int] = None) -> dict:
    """Per-row hard-label CE, entry-wise clipped reverse KL and d(CE + lam*R)/dz_q.

    ``rows`` selects packed rows (default: all).  Returns loss_ce, loss_rkl,
    grad (float64, or None) and N, the number of packed rows."""
    B, k1, V = target.shape
    k = k1 - 1
    if draft.shape != (B, k, V):
        raise ValueError("draft must be [B, k, V]")
    target = np.ascontiguousarray(target)
    draft = np.ascontiguousarray(draft)
    vl = None if verify_len is None else np.ascontiguousarray(verify_len, dtype=np.int32)
    if rows is None:
        Lc = np.full((B,), k) if vl is None else np.clip(vl, 1, k)
        n_eval = int(Lc.sum())
        rws = None
    else:
        rws = np.ascontiguousarray(rows, dtype=np.int64)
        n_eval = int(rws.shape[0])
    ce = np.empty((n_eval,), dtype=np.float64)
    rk = np.empty((n_eval,), dtype=np.float64)
    g = np.empty((n_eval, V), dtype=np.float64) if with_grad else None
    N = _load().oracle_opd(_dtype_code(target), _ptr(target), _ptr(draft), _ptr(vl), B, k, V,
                           float(clip_c), float(lam), _ptr(rws), n_eval, _ptr(ce), _ptr(rk), _ptr(g),
                           _threads(nthreads))
    if N < 0:
        raise ValueError(f"oracle_opd rejected its arguments ({N})")
    return {"loss_ce": ce, "loss_rkl": rk, "grad": g, "N": int(N)}
