"""CPU / GPU share policy of the sequence-dimension split (oracle; test infrastructure only).

[InplaceKVCache] "Physically Partitioned KVCache Format for CPU-GPU Load Balancing in MoE
Inference":
  §5.1  r is the CPU's share of a sequence of already-placed length L; the CPU takes the
        oldest r L tokens, the GPU the rest.
  §5.2  Eq. 1, the two engines' per-step latencies; the end-to-end step is their maximum plus
        an r-independent merge.
  §5.3  Eq. 2, their balance clamped to [0, 1]; its limit p = B / (A + B); the cumulative
        share R(L) = p + (R(L0) - p) L0 / L reached by giving new tokens the marginal share p;
        A re-estimated from a sliding average of the measured CPU latency per step; the
        parameters calibrated offline by scanning data volumes.

Readings (the pages leave these open):
  * Batches leaving the staging window go to one side whole.  A batch goes to the CPU iff
    that leaves the cumulative CPU token count nearer the target r(L') L' for the new placed
    length L' (ties stay on the GPU).  With constant A, B, C this hands the CPU a fraction p of
    the batches, which is the pages' marginal-share rule, and keeps R(L') within D / (2 L') of
    r(L').
  * The prefill's CPU share is r(L0) L0 rounded to the nearest whole block (half away from
    zero), at most the whole blocks of L0.
  * A = (sum of window latencies - k C_CPU) / (sum of window CPU tokens) over the k = window
    most recent samples, refreshed once per routed batch once the window is full; before that
    (or if the estimate is not positive) the calibrated A stays.
  * Offline calibration is an ordinary least-squares line, latency against token count.

Plain float64 arithmetic, steps in the order the definitions give them; the routing choice
between two integer token counts is then made exactly.
"""

from fractions import Fraction

import numpy as np


def step_latencies(r, L, A, B, C_cpu, C_gpu):
    """Eq. 1: (T_CPU(r), T_GPU(r)) for CPU share r of L placed tokens."""
    return r * A * L + C_cpu, (1.0 - r) * B * L + C_gpu


def optimum(A, B, C_cpu, C_gpu, L):
    """Eq. 2: r(L) = min(1, max(0, B / (A + B) + Delta / ((A + B) L))), Delta = C_GPU - C_CPU."""
    delta = C_gpu - C_cpu
    unclamped = B / (A + B) + delta / ((A + B) * L)
    return min(1.0, max(0.0, unclamped))


def converged(A, B):
    """p = B / (A + B), the limit of r(L) for long sequences."""
    return B / (A + B)


def cumulative_share(R0, L0, L, p):
    """R(L) = p + (R(L0) - p) L0 / L."""
    return p + (R0 - p) * L0 / L


def fit_line(tokens, seconds):
    """Least-squares (slope, intercept) of seconds ~ slope * tokens + intercept."""
    x = np.asarray(tokens, np.float64)
    y = np.asarray(seconds, np.float64)
    design = np.stack([x, np.ones_like(x)], axis=1)
    (slope, intercept), *_ = np.linalg.lstsq(design, y, rcond=None)
    return float(slope), float(intercept)


def _round_half_away(x):
    whole = int(x)
    return whole + (1 if x - whole >= 0.5 else 0)


class Controller:
    """Admission share, A tracking and routing of evicted batches for one sequence."""

    def __init__(self, A, B, C_cpu, C_gpu, window):
        self.A, self.B, self.C_cpu, self.C_gpu = float(A), float(B), float(C_cpu), float(C_gpu)
        self.window = int(window)
        self.samples = []          # (latency, cpu tokens), oldest first
        self.L = 0                 # placed tokens
        self.c = 0                 # CPU tokens
        self.cpu_batches = 0
        self.batches = 0
        self.decisions = []
        self.admitted = False

    def admit(self, L0, block_tokens):
        self.admitted = True
        c = 0
        if L0 > 0:
            r = optimum(self.A, self.B, self.C_cpu, self.C_gpu, float(L0))
            blocks = _round_half_away(r * float(L0) / float(block_tokens))
            c = min(blocks, L0 // block_tokens) * block_tokens
        self.L, self.c = L0, c
        return c

    def observe(self, latency, cpu_tokens):
        self.samples.append((float(latency), float(cpu_tokens)))
        if len(self.samples) > self.window:
            self.samples.pop(0)

    def _refresh_cost(self):
        if len(self.samples) < self.window:
            return
        total_t = 0.0
        total_n = 0.0
        for t, n in self.samples:
            total_t += t
            total_n += n
        if total_n > 0:
            a = (total_t - self.window * self.C_cpu) / total_n
            if a > 0 and np.isfinite(a):
                self.A = a

    def route(self, D):
        self._refresh_cost()
        L_new = self.L + D
        target = optimum(self.A, self.B, self.C_cpu, self.C_gpu, float(L_new)) * float(L_new)
        # nearer the target, decided exactly (rationals) for the computed float64 target
        t = Fraction(target)
        to_cpu = abs(Fraction(self.c + D) - t) < abs(Fraction(self.c) - t)
        if to_cpu:
            self.c += D
            self.cpu_batches += 1
        self.batches += 1
        self.L = L_new
        self.decisions.append(to_cpu)
        return to_cpu
