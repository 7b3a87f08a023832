"""Admission-controller oracle -- TEST INFRASTRUCTURE ONLY.

A plain Python model of the verification-batch scheduler step.  Only the
tests and the benchmark's CPU-baseline leg may import it; it shares nothing
with the native library and never imports it.

Source: "AdaFlash：基于在策略蒸馏扩散草稿器的自适应投机解码" (review, ZH), section
2.3: the verify batch packs the real verify tokens of each request (total
length sum_i k_hat_i instead of bs x k); the scheduler smooths the number of
requests a round actually advanced, N_hat <- (1 - beta) N_hat + beta N, to
decide how many to admit next; requests that still overflow the budget go
back to the pending queue.  The AdaFlash review (EN), "Adaptive request
scheduling for variable verification lengths", states the same.

Readings where the pages leave a step open (each is listed in the design doc):
  * A round's admission target is max(1, floor(N_hat + 0.5)): running
    requests stay; pending requests are admitted in arrival order until the
    batch holds that many.
  * The budget caps the packed verify tokens, sum of k_hat over the batch.
    While it is exceeded (and more than one request is in the batch), the
    most recently placed request leaves the batch and returns to the FRONT of
    the pending queue (so returned requests keep their order and go first).
  * N is the size of the batch that is verified (after the overflow step).
"""
from __future__ import annotations

import math
from collections import deque


class Admission:
    def __init__(self, beta: float, n_hat0: float, budget: int):
        if not (0.0 < beta <= 1.0) or budget < 1 or not (n_hat0 >= 0.0):
            raise ValueError("need 0 < beta <= 1, budget >= 1, n_hat0 >= 0")
        self.beta = float(beta)
        self.n_hat = float(n_hat0)
        self.budget = int(budget)
        self.pending = deque()
        self.active = []

    def enqueue(self, ids):
        self.pending.extend(int(x) for x in ids)

    def target(self) -> int:
        return max(1, int(math.floor(self.n_hat + 0.5)))

    def propose(self):
        """The candidate batch: the running requests, then pending ones in
        arrival order up to the admission target."""
        t = self.target()
        while len(self.active) < t and self.pending:
            self.active.append(self.pending.popleft())
        return list(self.active)

    def commit(self, k_hat):
        """Applies the budget to the proposed batch (k_hat aligned with it),
        updates the estimate, and returns the batch to verify."""
        batch = list(self.active)
        ks = [int(x) for x in k_hat]
        if len(ks) != len(batch):
            raise ValueError("k_hat must match the proposed batch")
        total = sum(ks)
        back = []
        while total > self.budget and len(batch) > 1:
            back.append(batch.pop())
            total -= ks.pop()
        for rid in back:              # last removed first: the original order is restored
            self.pending.appendleft(rid)
        self.active = batch
        n = len(batch)
        self.n_hat = (1.0 - self.beta) * self.n_hat + self.beta * n
        return list(batch)

    def finish(self, done_ids):
        done = set(int(x) for x in done_ids)
        self.active = [r for r in self.active if r not in done]
