"""Seeded synthetic inputs for the FP8-activation x block-scaled FP4 expert GEMM.

This module holds no step of the method: it draws random activations, random weight nibbles and
random scale codes, and builds routing tables.  Scale codes are drawn from stated byte ranges; what
those bytes decode to is checked by the oracle's tests, never computed here.  Both the HIP path (via
the tests and the benchmark) and the CPU oracle consume exactly these arrays.

Workloads (sizes from the pages' expert shapes; distributions stated per function):
  config0  single NVFP4 expert, g=4, k=512, n=256
  config1  single MXFP4 expert, g in {1,2,4,8}, k=7168, n=2048 (decode-shaped)
  config2  single NVFP4 down-projection expert, g=16, k=2048, n=7168, 1% outliers x40
  config3  grouped NVFP4 decode step: 512 tokens, 256 experts, top-8, k=7168, n=2048
  config4  grouped prefill: 8192 tokens, 256 experts (255 NVFP4 + 1 MXFP4), Zipf(1.1) top-8,
           k=7168, n=4096, Student-t(3) activations
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

NVFP4 = 0
MXFP4 = 1
GROUP_SIZE = {NVFP4: 16, MXFP4: 32}

SEED_BASE = 20261202

# E4M3 scale bytes drawn for NVFP4 weights: every positive code from 0x20 to 0x48 inclusive
# (41 codes; the oracle tests check they are exactly the E4M3 values in [2^-3, 2^2]).
NVFP4_SCALE_CODE_RANGE = (0x20, 0x48)
# E8M0 biased exponents drawn for MXFP4 weights.
MXFP4_SCALE_CODE_RANGE = (117, 124)
# Per-expert NVFP4 scale2 choices for the grouped workloads: the powers of two 2^-8 .. 2^-5.
GROUPED_SCALE2_CHOICES = (2.0 ** -8, 2.0 ** -7, 2.0 ** -6, 2.0 ** -5)

# Exact-by-construction inputs.  E4M3 bytes of the integers 0..16 (the oracle tests check that each
# decodes to its integer), used with both signs; weight scale bytes for NVFP4 (E4M3 1, 2, 4) and
# MXFP4 (E8M0 0.5, 1, 2).  With activation scale 1 and scale2 1 every product is a multiple of 1/4
# and every partial sum of k <= 7168 terms stays below 2^22, so any f32 summation order is exact.
EXACT_INT_E4M3_CODES = (0x00, 0x38, 0x40, 0x44, 0x48, 0x4A, 0x4C, 0x4E, 0x50, 0x51, 0x52, 0x53,
                        0x54, 0x55, 0x56, 0x57, 0x58)
EXACT_NVFP4_SCALE_CODES = (0x38, 0x40, 0x48)
EXACT_MXFP4_SCALE_CODES = (126, 127, 128)


def rng_for(config: int, variant: int = 0) -> np.random.Generator:
    return np.random.default_rng([SEED_BASE, config, variant])


def random_nibbles(rng, n: int, k: int) -> np.ndarray:
    """Uniform 4-bit codes packed two per byte, [n, k/2] (uniform bytes are exactly that)."""
    return np.frombuffer(rng.bytes(n * (k // 2)), dtype=np.uint8).reshape(n, k // 2).copy()


def random_scale_codes(rng, kind: int, n: int, k: int) -> np.ndarray:
    lo, hi = NVFP4_SCALE_CODE_RANGE if kind == NVFP4 else MXFP4_SCALE_CODE_RANGE
    return rng.integers(lo, hi + 1, size=(n, k // GROUP_SIZE[kind]), dtype=np.uint8)


@dataclass
class Expert:
    kind: int
    w: np.ndarray        # u8 [n, k/2], even k in the low nibble
    s: np.ndarray        # u8 [n, k/gs]
    scale2: float        # NVFP4 per-tensor f32 scale (ignored for MXFP4)


@dataclass
class SingleWorkload:
    name: str
    x: np.ndarray        # f32 [g, k]
    expert: Expert

    @property
    def g(self): return self.x.shape[0]

    @property
    def k(self): return self.x.shape[1]

    @property
    def n(self): return self.expert.w.shape[0]


@dataclass
class GroupedWorkload:
    name: str
    x: np.ndarray              # f32 [T, k] token activations
    row_ids: np.ndarray        # int32 [R]: token of each packed row
    offsets: np.ndarray        # int32 [E+1]: expert e owns packed rows offsets[e]..offsets[e+1]-1
    kinds: np.ndarray          # int32 [E]
    scale2: np.ndarray         # f32 [E]
    w_bank: np.ndarray         # u8, all experts' nibble planes back to back
    s_bank: np.ndarray         # u8, all experts' scale planes back to back
    w_off: np.ndarray          # int64 [E] byte offset of expert e's nibble plane in w_bank
    s_off: np.ndarray          # int64 [E] byte offset of expert e's scale plane in s_bank
    n: int
    k: int
    extra: dict = field(default_factory=dict)
    logits: np.ndarray | None = None   # f32 [T, E] router logits the tables were built from

    @property
    def E(self): return len(self.kinds)

    @property
    def R(self): return int(self.offsets[-1])

    def w_of(self, e: int) -> np.ndarray:
        o = int(self.w_off[e])
        return self.w_bank[o:o + self.n * self.k // 2].reshape(self.n, self.k // 2)

    def s_of(self, e: int) -> np.ndarray:
        gs = GROUP_SIZE[int(self.kinds[e])]
        o = int(self.s_off[e])
        return self.s_bank[o:o + self.n * self.k // gs].reshape(self.n, self.k // gs)

    def weight_stream_bytes(self) -> int:
        """Nibble + scale-plane + scale2 bytes of every expert that owns at least one row."""
        total = 0
        for e in range(self.E):
            if self.offsets[e + 1] > self.offsets[e]:
                total += self.n * self.k // 2 + self.n * self.k // GROUP_SIZE[int(self.kinds[e])]
                total += 4 if int(self.kinds[e]) == NVFP4 else 0
        return total


# --------------------------------------------------------------------------- single experts
def config0() -> SingleWorkload:
    rng = rng_for(0)
    x = rng.standard_normal((4, 512), dtype=np.float32)
    ex = Expert(NVFP4, random_nibbles(rng, 256, 512), random_scale_codes(rng, NVFP4, 256, 512),
                2.0 ** -6)
    return SingleWorkload("config0: single NVFP4 expert g=4 k=512 n=256", x, ex)


def config1(g: int) -> SingleWorkload:
    rng = rng_for(1, g)
    x = rng.standard_normal((g, 7168), dtype=np.float32)
    ex = Expert(MXFP4, random_nibbles(rng, 2048, 7168), random_scale_codes(rng, MXFP4, 2048, 7168),
                0.0)
    return SingleWorkload(f"config1: single MXFP4 expert g={g} k=7168 n=2048", x, ex)


def config2() -> SingleWorkload:
    rng = rng_for(2)
    g, k, n = 16, 2048, 7168
    x = (0.5 * rng.standard_normal((g, k), dtype=np.float32)).astype(np.float32)
    n_out = int(round(0.01 * g * k))
    idx = rng.choice(g * k, size=n_out, replace=False)
    x.reshape(-1)[idx] *= np.float32(40.0)
    ex = Expert(NVFP4, random_nibbles(rng, n, k), random_scale_codes(rng, NVFP4, n, k), 2.0 ** -7)
    return SingleWorkload("config2: single NVFP4 down-proj expert g=16 k=2048 n=7168 (1% x40)",
                          x, ex)


def single_random(seed: int, g: int, n: int, k: int, kind: int, scale2: float = 2.0 ** -6,
                  x_scale: float = 1.0) -> SingleWorkload:
    """A small random expert of any shape (parity cases: ragged n, odd g, several tiles)."""
    rng = np.random.default_rng([SEED_BASE, 100, seed])
    x = (x_scale * rng.standard_normal((g, k), dtype=np.float32)).astype(np.float32)
    ex = Expert(kind, random_nibbles(rng, n, k), random_scale_codes(rng, kind, n, k),
                scale2 if kind == NVFP4 else 0.0)
    return SingleWorkload(f"random seed={seed} g={g} n={n} k={k} kind={kind}", x, ex)


def exact_arm(seed: int, g: int, n: int, k: int, kind: int):
    """Quantized GEMM inputs given directly as codes: (a_codes, a_scales=1, Expert(scale2=1))."""
    rng = np.random.default_rng([SEED_BASE, 200, seed])
    mags = np.array(EXACT_INT_E4M3_CODES, dtype=np.uint8)
    a = mags[rng.integers(0, len(mags), size=(g, k))]
    a |= (rng.integers(0, 2, size=(g, k), dtype=np.uint8) << 7)
    a_scales = np.ones((g, k // 128), dtype=np.float32)
    codes = EXACT_NVFP4_SCALE_CODES if kind == NVFP4 else EXACT_MXFP4_SCALE_CODES
    s = np.array(codes, dtype=np.uint8)[rng.integers(0, 3, size=(n, k // GROUP_SIZE[kind]))]
    ex = Expert(kind, random_nibbles(rng, n, k), s, 1.0 if kind == NVFP4 else 0.0)
    return a.astype(np.uint8), a_scales, ex


# --------------------------------------------------------------------------- routing
def route_topk(logits: np.ndarray, top: int):
    """Top-`top` experts per token by logit, ties to the lower expert id; rows packed per expert in
    ascending token order.  Returns (row_ids int32 [T*top], offsets int32 [E+1])."""
    T, E = logits.shape
    order = np.argsort(-logits, axis=1, kind="stable")[:, :top]       # [T, top]
    tok = np.repeat(np.arange(T, dtype=np.int64), top)
    exp = order.reshape(-1)
    perm = np.lexsort((tok, exp))                                      # by expert, then token
    row_ids = tok[perm].astype(np.int32)
    counts = np.bincount(exp, minlength=E)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    return row_ids, offsets


def _bank(rng, kinds, n, k):
    E = len(kinds)
    w_off = np.arange(E, dtype=np.int64) * (n * k // 2)
    w_bank = np.frombuffer(rng.bytes(E * n * k // 2), dtype=np.uint8).copy()
    s_sizes = np.array([n * k // GROUP_SIZE[int(kd)] for kd in kinds], dtype=np.int64)
    s_off = np.zeros(E, dtype=np.int64)
    s_off[1:] = np.cumsum(s_sizes)[:-1]
    s_bank = np.empty(int(s_sizes.sum()), dtype=np.uint8)
    for kd in (NVFP4, MXFP4):
        sel = [e for e in range(E) if int(kinds[e]) == kd]
        if not sel:
            continue
        lo, hi = NVFP4_SCALE_CODE_RANGE if kd == NVFP4 else MXFP4_SCALE_CODE_RANGE
        draws = rng.integers(lo, hi + 1, size=len(sel) * (n * k // GROUP_SIZE[kd]), dtype=np.uint8)
        per = n * k // GROUP_SIZE[kd]
        for i, e in enumerate(sel):
            s_bank[s_off[e]:s_off[e] + per] = draws[i * per:(i + 1) * per]
    return w_bank, s_bank, w_off, s_off


def grouped_random(seed: int, T: int, E: int, top: int, n: int, k: int, kinds=None,
                   empty_experts=(), zipf: float | None = None, x_dist: str = "normal"):
    """A grouped workload of any size (parity cases).  `empty_experts` get no rows."""
    rng = np.random.default_rng([SEED_BASE, 300, seed])
    kinds = np.zeros(E, dtype=np.int32) if kinds is None else np.asarray(kinds, dtype=np.int32)
    x = (rng.standard_t(3, size=(T, k)) if x_dist == "t3" else rng.standard_normal((T, k))).astype(np.float32)
    if zipf is not None:
        ranks = rng.permutation(E) + 1
        logits = -zipf * np.log(ranks)[None, :] + rng.gumbel(size=(T, E))
    else:
        logits = rng.standard_normal((T, E))
    logits = logits.astype(np.float32)
    for e in empty_experts:
        logits[:, e] = -np.inf
    row_ids, offsets = route_topk(logits, top)
    scale2 = np.array(GROUPED_SCALE2_CHOICES, dtype=np.float32)[rng.integers(0, 4, size=E)]
    scale2[kinds == MXFP4] = 0.0
    w_bank, s_bank, w_off, s_off = _bank(rng, kinds, n, k)
    return GroupedWorkload(f"grouped seed={seed} T={T} E={E} top={top} n={n} k={k}", x, row_ids,
                           offsets, kinds, scale2, w_bank, s_bank, w_off, s_off, n, k, logits=logits)


def _config3_tokens():
    rng = rng_for(3)
    T, E, k = 512, 256, 7168
    x = rng.standard_normal((T, k), dtype=np.float32)
    logits = rng.standard_normal((T, E), dtype=np.float32)
    return rng, x, logits


def config3_logits() -> np.ndarray:
    """The decode workload's router logits alone (f32 [512, 256]), without its weight bank."""
    return _config3_tokens()[2]


def config3() -> GroupedWorkload:
    T, E, top, n, k = 512, 256, 8, 2048, 7168
    rng, x, logits = _config3_tokens()
    row_ids, offsets = route_topk(logits, top)
    kinds = np.zeros(E, dtype=np.int32)
    scale2 = np.array(GROUPED_SCALE2_CHOICES, dtype=np.float32)[rng.integers(0, 4, size=E)]
    w_bank, s_bank, w_off, s_off = _bank(rng, kinds, n, k)
    return GroupedWorkload("config3: grouped NVFP4 decode, 512 tokens, E=256, top-8, k=7168, n=2048",
                           x, row_ids, offsets, kinds, scale2, w_bank, s_bank, w_off, s_off, n, k,
                           logits=logits)


def _config4_tokens():
    rng = rng_for(4)
    T, E, k = 8192, 256, 7168
    x = rng.standard_t(3, size=(T, k)).astype(np.float32)
    ranks = rng.permutation(E) + 1
    logits = (-1.1 * np.log(ranks)[None, :] + rng.gumbel(size=(T, E))).astype(np.float32)
    return rng, x, logits


def config4_logits() -> np.ndarray:
    """The prefill workload's Zipf(1.1) router logits alone (f32 [8192, 256]), without its bank."""
    return _config4_tokens()[2]


def config4() -> GroupedWorkload:
    T, E, top, n, k = 8192, 256, 8, 4096, 7168
    rng, x, logits = _config4_tokens()
    row_ids, offsets = route_topk(logits, top)
    kinds = np.zeros(E, dtype=np.int32)
    kinds[E - 1] = MXFP4
    scale2 = np.array(GROUPED_SCALE2_CHOICES, dtype=np.float32)[rng.integers(0, 4, size=E)]
    scale2[E - 1] = 0.0
    w_bank, s_bank, w_off, s_off = _bank(rng, kinds, n, k)
    return GroupedWorkload("config4: grouped prefill, 8192 tokens, E=256 (255 NVFP4 + 1 MXFP4), "
                           "Zipf(1.1) top-8, k=7168, n=4096, Student-t(3)",
                           x, row_ids, offsets, kinds, scale2, w_bank, s_bank, w_off, s_off, n, k,
                           logits=logits)


@dataclass
class ExpertChainWorkload:
    """One MoE expert layer: token activations x [T, hidden], top-k routing packed per expert, a
    per-packed-row routing weight, the fused gate/up projection bank (n = 2*inter, k = hidden: gate
    rows first, then up rows) and the down projection bank (n = hidden, k = inter)."""
    name: str
    x: np.ndarray
    row_ids: np.ndarray
    offsets: np.ndarray
    route_w: np.ndarray            # f32 [R]
    kinds: np.ndarray
    limit: float
    up: GroupedWorkload            # gate/up projection (shares x, row_ids, offsets)
    down: GroupedWorkload          # down projection (its x is unused: it consumes the activation)
    logits: np.ndarray | None = None   # f32 [T, E] router logits the tables were built from

    @property
    def R(self): return int(self.offsets[-1])

    @property
    def hidden(self): return self.x.shape[1]

    @property
    def inter(self): return self.up.n // 2


def expert_chain(seed: int, T: int, E: int, top: int, hidden: int, inter: int, kinds=None,
                 x_scale: float = 1.0, limit: float = 7.0, zipf: float | None = None) -> ExpertChainWorkload:
    """Seeded inputs for the gate/up -> activation -> down chain (parity cases).  Routing weights are
    uniform draws in [0.05, 1]; x_scale multiplies the N(0,1) activations (x50 drives both clamps of
    the activation, as in the pages' saturation cell)."""
    rng = np.random.default_rng([SEED_BASE, 400, seed])
    kinds = np.zeros(E, dtype=np.int32) if kinds is None else np.asarray(kinds, dtype=np.int32)
    x = (rng.standard_normal((T, hidden)) * x_scale).astype(np.float32)
    if zipf is not None:
        ranks = rng.permutation(E) + 1
        logits = -zipf * np.log(ranks)[None, :] + rng.gumbel(size=(T, E))
    else:
        logits = rng.standard_normal((T, E))
    logits = logits.astype(np.float32)
    row_ids, offsets = route_topk(logits, top)
    route_w = rng.uniform(0.05, 1.0, size=int(offsets[-1])).astype(np.float32)
    banks = []
    for n, k in ((2 * inter, hidden), (hidden, inter)):
        scale2 = np.array(GROUPED_SCALE2_CHOICES, dtype=np.float32)[rng.integers(0, 4, size=E)]
        scale2[kinds == MXFP4] = 0.0
        w_bank, s_bank, w_off, s_off = _bank(rng, kinds, n, k)
        banks.append(GroupedWorkload(f"chain seed={seed} n={n} k={k}", x if k == hidden else
                                     np.zeros((0, k), np.float32), row_ids, offsets, kinds, scale2,
                                     w_bank, s_bank, w_off, s_off, n, k))
    return ExpertChainWorkload(f"expert chain seed={seed} T={T} E={E} top={top} hidden={hidden} "
                               f"inter={inter} x_scale={x_scale}", x, row_ids, offsets, route_w, kinds,
                               float(limit), banks[0], banks[1], logits)


def config4_chain() -> ExpertChainWorkload:
    """The grouped prefill layer as a whole expert chain: config4's tokens, router logits, routing and
    fused gate/up bank (n = 4096 = 2 x 2048, k = 7168), plus a down projection bank (n = 7168,
    k = 2048) in the same formats (255 NVFP4 + 1 MXFP4), limit 7.  route_w (uniform in [0.05, 1]) is
    a stand-in per-row weight; a run that routes on the device takes the softmax weights instead."""
    up = config4()
    rng = rng_for(4, 1)
    inter = up.n // 2
    scale2 = np.array(GROUPED_SCALE2_CHOICES, dtype=np.float32)[rng.integers(0, 4, size=up.E)]
    scale2[up.kinds == MXFP4] = 0.0
    w_bank, s_bank, w_off, s_off = _bank(rng, up.kinds, up.k, inter)
    down = GroupedWorkload("config4 down projection", np.zeros((0, inter), np.float32), up.row_ids,
                           up.offsets, up.kinds, scale2, w_bank, s_bank, w_off, s_off, up.k, inter)
    route_w = rng.uniform(0.05, 1.0, size=up.R).astype(np.float32)
    return ExpertChainWorkload("config4 expert layer: gate/up (n=4096, k=7168) -> swiglu limit 7 -> "
                               "down (n=7168, k=2048); 8192 tokens, E=256, Zipf(1.1) top-8",
                               up.x, up.row_ids, up.offsets, route_w, up.kinds, 7.0, up, down, up.logits)


# --------------------------------------------------------------------------- W4A4 arms
W4A4_HOT_CHANNELS = 8


def w4a4_case(seed: int, T: int, n: int, k: int, arm: str = "uniform"):
    """Activations and an NVFP4 expert for the W4A4 arms: x = 0.1 U[0, 1) per element ("uniform");
    token j additionally scaled by 10^((j mod 7) - 3) ("dyn"); and on top of that 8 fixed channels
    (977 c + 13) mod k amplified x300 ("res").  Returns (x f32 [T, k], Expert)."""
    rng = np.random.default_rng([SEED_BASE, 500, seed])
    x = rng.random((T, k)) * 0.1
    if arm in ("dyn", "res"):
        x *= 10.0 ** ((np.arange(T) % 7) - 3)[:, None]
    if arm == "res":
        hot = [(c * 977 + 13) % k for c in range(W4A4_HOT_CHANNELS)]
        x[:, hot] *= 300.0
    ex = Expert(NVFP4, random_nibbles(rng, n, k), random_scale_codes(rng, NVFP4, n, k),
                float(GROUPED_SCALE2_CHOICES[1]))
    return x.astype(np.float32), ex


def w4a4_hot_channels(k: int) -> list:
    return [(c * 977 + 13) % k for c in range(W4A4_HOT_CHANNELS)]
