"""Seeded synthetic inputs for the verify-and-supervise pass.

Holds the named workload presets and a ctypes wrapper over ``gen.cpp`` (built
into ``libworkloads.so``).  Nothing here computes any part of the verifier or
the supervision loss; it only synthesises the arrays both the CPU oracle and
the GPU library read.

Workloads (vocabulary V = 151936, the Qwen3 vocabulary; k = 16 draft tokens as
in the AdaFlash review's notation table and hyper-parameters; concurrency
levels 1/32/128 as in its main-results table):

1. ``tiny``: B=4, 15 drafts + 1 bonus row, V=64, fp32.  z_p ~ N(0, 1.5^2),
   z_q = 0.8 z_p + 0.6 N(0,1), T=1, verify_len = 15.
2. ``single``: B=1, k=16, bf16.  z_p[v] = 2 N(0,1) - 1.1 ln(v+1) (Zipf(1.1)
   log-prior), z_q = 0.7 z_p + N(0,1), verify_len = 16; T=0 and T=1.
3. ``c32``: B=32, k=16, bf16, verify_len ~ U{1..16}, per-request noise
   sigma_b ~ U{0.3, 1.0, 2.0}, z_q = 0.7 z_p + sigma_b N(0,1), T=1.
4. ``c128``: as ``c32`` with B=128, plus the fused supervision (c=10, lambda=1).
5. ``replay``: 512 blocks x 16 positions, the ``single`` generator (sigma=1),
   supervision only (c=10, lambda=1).

``two_level`` builds the constructed case with sum_v min(p, q) = a per position
(q uniform; p = q(1+d) on the lower half of ids and q(1-d) on the upper half,
d = 2(1-a)).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libworkloads.so")
V_QWEN3 = 151936
SEED_BASE = 0xADAF1A50

WL_GAUSS, WL_ZIPF, WL_TWO_LEVEL = 0, 1, 2


class _Spec(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("k", ctypes.c_int32), ("V", ctypes.c_int32),
        ("bf16", ctypes.c_int32), ("model", ctypes.c_int32), ("ragged", ctypes.c_int32),
        ("sigma_choice", ctypes.c_int32), ("nthreads", ctypes.c_int32),
        ("seed", ctypes.c_uint64), ("round", ctypes.c_uint32), ("logits_round", ctypes.c_uint32),
        ("T", ctypes.c_double), ("p_scale", ctypes.c_double), ("q_coef", ctypes.c_double),
        ("zipf_s", ctypes.c_double), ("two_level_d", ctypes.c_double),
        ("sigmas", ctypes.c_double * 3),
    ]


def build(verbose: bool = False) -> str:
    """Compile gen.cpp into libworkloads.so (host code only)."""
    import subprocess
    src = os.path.join(_HERE, "gen.cpp")
    tmp = LIB_PATH + ".tmp"
    cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
           "-o", tmp, src]
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
        lib.wl_generate.restype = ctypes.c_int
        lib.wl_generate.argtypes = [ctypes.POINTER(_Spec)] + [ctypes.c_void_p] * 6
        lib.wl_philox4x32_10.restype = None
        lib.wl_philox4x32_10.argtypes = [ctypes.c_void_p] * 3
        _lib = lib
    return _lib


def philox4x32_10(ctr, key) -> np.ndarray:
    """One raw Philox4x32-10 block (for known-answer tests)."""
    c = np.ascontiguousarray(np.asarray(ctr, dtype=np.uint32))
    kk = np.ascontiguousarray(np.asarray(key, dtype=np.uint32))
    out = np.zeros(4, dtype=np.uint32)
    _load().wl_philox4x32_10(c.ctypes.data, kk.ctypes.data, out.ctypes.data)
    return out


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    k: int
    V: int
    bf16: bool
    model: int
    T: float
    ragged: bool = False
    sigma_choice: bool = False
    p_scale: float = 1.0
    q_coef: float = 0.7
    zipf_s: float = 0.0
    two_level_d: float = 0.0
    sigmas: tuple = (1.0, 1.0, 1.0)
    seed: int = SEED_BASE
    rounds: int = 1
    opd: bool = False
    clip_c: float = 10.0
    lam: float = 1.0
    verify: bool = True


WORKLOADS = {
    1: Workload("tiny", B=4, k=15, V=64, bf16=False, model=WL_GAUSS, T=1.0, p_scale=1.5,
                q_coef=0.8, sigmas=(0.6, 0.6, 0.6), seed=SEED_BASE + 1, rounds=20000),
    2: Workload("single", B=1, k=16, V=V_QWEN3, bf16=True, model=WL_ZIPF, T=1.0, p_scale=2.0,
                q_coef=0.7, zipf_s=1.1, sigmas=(1.0, 1.0, 1.0), seed=SEED_BASE + 2, rounds=1000),
    3: Workload("c32", B=32, k=16, V=V_QWEN3, bf16=True, model=WL_ZIPF, T=1.0, p_scale=2.0,
                q_coef=0.7, zipf_s=1.1, ragged=True, sigma_choice=True, sigmas=(0.3, 1.0, 2.0),
                seed=SEED_BASE + 3, rounds=200),
    4: Workload("c128", B=128, k=16, V=V_QWEN3, bf16=True, model=WL_ZIPF, T=1.0, p_scale=2.0,
                q_coef=0.7, zipf_s=1.1, ragged=True, sigma_choice=True, sigmas=(0.3, 1.0, 2.0),
                seed=SEED_BASE + 4, rounds=50, opd=True, clip_c=10.0, lam=1.0),
    5: Workload("replay", B=512, k=16, V=V_QWEN3, bf16=True, model=WL_ZIPF, T=1.0, p_scale=2.0,
                q_coef=0.7, zipf_s=1.1, sigmas=(1.0, 1.0, 1.0), seed=SEED_BASE + 5, rounds=1,
                opd=True, clip_c=10.0, lam=1.0, verify=False),
}


def two_level(a: float, B: int = 4, k: int = 15, V: int = 64, seed: int = SEED_BASE + 11) -> Workload:
    """Constructed case: q uniform, sum_v min(p, q) = a at every position."""
    return Workload(f"two_level_{a}", B=B, k=k, V=V, bf16=False, model=WL_TWO_LEVEL, T=1.0,
                    two_level_d=2.0 * (1.0 - a), seed=seed)


@dataclass
class Batch:
    wl: Workload
    round: int
    target: np.ndarray      # [B, k+1, V] float32, or uint16 holding bf16 bits
    draft: Optional[np.ndarray]  # [B, k, V]
    tokens: Optional[np.ndarray]  # int32 [B, k]
    verify_len: np.ndarray  # int32 [B]
    uniforms: np.ndarray    # float32 [B, k+1]
    sigma: np.ndarray       # float32 [B]

    @property
    def n_rows(self) -> int:
        return int(self.verify_len.sum())


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def generate(wl: Workload, round: int = 0, logits_round: Optional[int] = None, T: Optional[float] = None,
             with_draft: bool = True, with_tokens: bool = True, nthreads: Optional[int] = None,
             out: Optional[Batch] = None) -> Batch:
    """Synthesise one batch.  ``logits_round`` lets the logits stay fixed while tokens and
    uniforms vary with ``round``; ``T`` overrides the drafter temperature."""
    lib = _load()
    B, k, V = wl.B, wl.k, wl.V
    Tv = wl.T if T is None else T
    sp = _Spec()
    sp.B, sp.k, sp.V = B, k, V
    sp.bf16 = 1 if wl.bf16 else 0
    sp.model = wl.model
    sp.ragged = 1 if wl.ragged else 0
    sp.sigma_choice = 1 if wl.sigma_choice else 0
    sp.nthreads = nthreads or default_threads()
    sp.seed = wl.seed
    sp.round = round
    sp.logits_round = round if logits_round is None else logits_round
    sp.T = Tv
    sp.p_scale, sp.q_coef, sp.zipf_s, sp.two_level_d = wl.p_scale, wl.q_coef, wl.zipf_s, wl.two_level_d
    for i in range(3):
        sp.sigmas[i] = wl.sigmas[i]
    dt = np.uint16 if wl.bf16 else np.float32
    if out is not None:
        target, draft = out.target, out.draft
    else:
        target = np.empty((B, k + 1, V), dtype=dt)
        draft = np.empty((B, k, V), dtype=dt) if with_draft else None
    tokens = np.empty((B, k), dtype=np.int32) if (with_tokens and draft is not None) else None
    vl = np.empty((B,), dtype=np.int32)
    uni = np.empty((B, k + 1), dtype=np.float32)
    sig = np.empty((B,), dtype=np.float32)

    def p(a):
        return None if a is None else a.ctypes.data

    rc = lib.wl_generate(ctypes.byref(sp), p(target), p(draft), p(tokens), p(vl), p(uni), p(sig))
    if rc != 0:
        raise ValueError(f"wl_generate failed ({rc})")
    return Batch(wl=wl, round=round, target=target, draft=draft, tokens=tokens, verify_len=vl,
                 uniforms=uni, sigma=sig)


def bf16_bits_to_f32(a: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) to float32, exactly."""
    return (a.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 to bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


# ------------------------------------------------------------- length head

@dataclass
class LengthHeadBatch:
    hidden: np.ndarray      # [B, k, H] bf16 bits
    W1: np.ndarray          # [Hp, H] bf16 bits
    b1: np.ndarray          # [Hp] float32
    w2: np.ndarray          # [Hp] float32
    b2: float
    accept_len: np.ndarray  # [B] int32, A_b in [0, L_b]
    verify_len: np.ndarray  # [B] int32, L_b in [1, k]


def length_head_inputs(B: int, k: int = 16, H: int = 4096, Hp: int = 256, seed: int = SEED_BASE + 21
                       ) -> LengthHeadBatch:
    """Synthetic hidden states and head weights for the adaptive length head:
    h ~ N(0, 1) and W1 ~ N(0, 1/H) (so the projection is about N(0, 1)), both
    rounded to bf16; b1 ~ N(0, 0.1^2), w2 ~ N(0, 4/Hp), b2 = 0.3; verify
    lengths U{1..k} and accept lengths U{0..L} (numpy's seeded generator)."""
    rng = np.random.default_rng(seed)
    hidden = f32_to_bf16_bits(rng.standard_normal((B, k, H), dtype=np.float32))
    W1 = f32_to_bf16_bits((rng.standard_normal((Hp, H)) / np.sqrt(H)).astype(np.float32))
    b1 = (0.1 * rng.standard_normal(Hp)).astype(np.float32)
    w2 = (2.0 / np.sqrt(Hp) * rng.standard_normal(Hp)).astype(np.float32)
    vl = rng.integers(1, k + 1, size=B).astype(np.int32)
    al = np.array([rng.integers(0, L + 1) for L in vl], dtype=np.int32)
    return LengthHeadBatch(hidden=hidden, W1=W1, b1=b1, w2=w2, b2=0.3, accept_len=al, verify_len=vl)
