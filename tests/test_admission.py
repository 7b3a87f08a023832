"""Admission controller: pins of the Python oracle (oracle/admission.py)
against the EMA's closed form and the scheduler's invariants, and the native
controller (adaflash_admission_* through the C ABI, host only) against the
oracle on seeded simulated traffic, round by round."""
import math

import numpy as np
import pytest

from oracle.admission import Admission as Ref


def test_ema_closed_form_for_a_constant_batch():
    # The budget (N tokens, k_hat = 1) holds every round to exactly N requests
    # while N_hat >= N proposes at least N: N_hat_t = N + (N_hat_0 - N)(1 - beta)^t.
    beta, n0, N = 0.25, 10.0, 6
    a = Ref(beta, n0, budget=N)
    a.enqueue(range(1000))
    for t in range(1, 30):
        b = a.propose()
        assert len(b) >= N
        assert len(a.commit([1] * len(b))) == N
        assert abs(a.n_hat - (N + (n0 - N) * (1 - beta) ** t)) < 1e-12


def test_beta_one_tracks_the_last_batch():
    a = Ref(1.0, 3.0, budget=20)
    a.enqueue(range(50))
    b = a.propose()
    assert len(b) == 3
    out = a.commit([8, 8, 8])          # 24 > 20: the last request goes back
    assert out == b[:2] and a.n_hat == 2.0 and list(a.pending)[:1] == [b[2]]


def test_budget_fifo_and_liveness():
    rng = np.random.default_rng(0)
    a = Ref(0.3, 4.0, budget=48)
    a.enqueue(range(200))
    remaining = {r: int(rng.integers(1, 6)) for r in range(200)}
    admitted_order = []
    done = set()
    for _ in range(2000):
        if len(done) == 200:
            break
        b = a.propose()
        for r in b:
            if r not in admitted_order:
                admitted_order.append(r)
        k = rng.integers(1, 17, size=len(b))
        out = a.commit(k)
        assert sum(k[:len(out)]) <= 48 or len(out) == 1     # the budget holds
        assert out == b[:len(out)]                           # overflow leaves from the end
        fin = [r for r in out if remaining[r] == 1]
        for r in out:
            remaining[r] -= 1
        done.update(fin)
        a.finish(fin)
    assert len(done) == 200                                  # every request is served
    assert admitted_order == sorted(admitted_order)          # first admitted in arrival order


def test_invalid_arguments():
    with pytest.raises(ValueError):
        Ref(0.0, 1.0, 10)
    with pytest.raises(ValueError):
        Ref(0.5, 1.0, 0)
    a = Ref(0.5, 2.0, 10)
    a.enqueue([1, 2, 3])
    a.propose()
    with pytest.raises(ValueError):
        a.commit([1])


@pytest.mark.parametrize("seed,beta,budget", [(1, 0.2, 64), (2, 0.5, 40), (3, 0.9, 200), (4, 1.0, 16)])
def test_native_matches_oracle(seed, beta, budget):
    import diffusion_drafter_verification_amd as ada
    rng = np.random.default_rng(seed)
    ref, nat = Ref(beta, 4.0, budget), ada.Admission(beta, 4.0, budget)
    remaining = {}
    next_id = 0
    for rnd in range(400):
        arrivals = int(rng.poisson(2.0))
        ids = list(range(next_id, next_id + arrivals))
        next_id += arrivals
        for r in ids:
            remaining[r] = int(rng.integers(1, 8))
        ref.enqueue(ids)
        nat.enqueue(ids)
        b1, b2 = ref.propose(), nat.propose()
        assert b1 == b2, rnd
        k = rng.integers(1, 17, size=len(b1))
        o1, o2 = ref.commit(k), nat.commit(k)
        assert o1 == o2 and ref.n_hat == nat.n_hat and len(ref.pending) == nat.pending, rnd
        fin = [r for r in o1 if remaining[r] == 1]
        for r in o1:
            remaining[r] -= 1
        ref.finish(fin)
        nat.finish(fin)


def test_native_rejects_bad_calls():
    import ctypes
    import diffusion_drafter_verification_amd as ada
    lib = ada.load_library()
    assert not lib.adaflash_admission_create(0.0, 1.0, 10)
    assert not lib.adaflash_admission_create(0.5, float("nan"), 10)
    assert not lib.adaflash_admission_create(0.5, 1.0, 0)
    nat = ada.Admission(0.5, 3.0, 100)
    nat.enqueue([7, 8, 9, 10])
    buf = (ctypes.c_int64 * 2)()
    assert lib.adaflash_admission_propose(nat._h, buf, 2) < 0      # capacity too small: nothing changes
    assert nat.propose() == [7, 8, 9]
    k = (ctypes.c_int32 * 2)(1, 1)
    out = (ctypes.c_int64 * 4)()
    assert lib.adaflash_admission_commit(nat._h, k, 2, out) < 0    # count differs from the proposal
    assert nat.commit([1, 1, 1]) == [7, 8, 9]
    assert math.isnan(lib.adaflash_admission_estimate(None))
