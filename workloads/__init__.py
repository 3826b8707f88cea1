"""Seeded synthetic inputs for the NAtS-L hybrid layer, shared by the tests, the
benchmark and the oracle checks.  This module holds none of the layer's
arithmetic: it draws random tensors, rounds them to bf16 where the workload is
bf16, and plants route patterns by shifting whole chunks of x along one fixed
direction of the score weights (it never pools, scores or routes anything).

The five workloads (sizes from the layer's benchmark description):
  tiny    fp32  B=1  H=1  L=256   D=64  d=64    natural routes, every |margin| > 1e-3
  prefill bf16  B=4  H=16 L=4096  D=128 d=2048  natural routes, ~50% softmax, random order
  long    bf16  B=1  H=16 L=32768 D=128 d=2048  25% softmax: 3 bursts (96 chunks) + 32 singles
  degen   bf16  B=2  H=16 L=8192  D=128 d=2048  route forced all-softmax / all-linear
  decode  bf16  B=64 H=16 D=128 d=2048          one new token against a compacted cache
                                               (~25% of a 32768-token context kept)

Distributions: x, q, v ~ N(0,1); k ~ N(0,1) then L2-normalised per token;
beta = sigmoid(N(0,1)); alpha ~ U(0.90, 0.999); W_score ~ N(0, 0.02^2);
W_mix ~ N(0, 0.1^2) (the second argument of N(.,.) read as a standard
deviation); b_score = 0; RMSNorm gains = 1.  alpha, beta and all weights stay
fp32 in every workload; bf16 workloads round x, q, k, v (k after
normalisation) to bf16 with round-to-nearest-even.
"""
from __future__ import annotations

import os
from dataclasses import dataclass, field

import numpy as np

CHUNK = 64


@dataclass(frozen=True)
class Workload:
    name: str
    io: str            # "f32" or "bf16"
    B: int
    H: int
    L: int             # prefill length (decode: context length the cache summarises)
    D: int
    d: int
    routing: str       # "natural", "planted", "forced", "decode"
    seed: int
    extra: dict = field(default_factory=dict)

    @property
    def nc(self):
        return self.L // CHUNK


# Seeds for natural routing were found by tests/golden/find_seeds.py (which
# calls only the oracle) and are re-checked by tests/test_workloads.py.
WORKLOADS = {
    "tiny": Workload("tiny", "f32", 1, 1, 256, 64, 64, "natural", seed=0),
    "prefill": Workload("prefill", "bf16", 4, 16, 4096, 128, 2048, "natural", seed=1),
    "long": Workload("long", "bf16", 1, 16, 32768, 128, 2048, "planted", seed=2,
                     extra=dict(n_sm=128, n_burst=3, burst_total=96, min_burst=16)),
    "degen": Workload("degen", "bf16", 2, 16, 8192, 128, 2048, "forced", seed=3),
    "decode": Workload("decode", "bf16", 64, 16, 32768, 128, 2048, "decode", seed=4,
                       extra=dict(nsel_lo=120, nsel_hi=136)),
}
ORDER = ["tiny", "prefill", "long", "degen", "decode"]


def round_bf16(a):
    """Round float32 values to the nearest bf16 (ties to even); returns
    float32 arrays holding exactly representable bf16 values."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    r = ((u + bias) & np.uint32(0xFFFF0000)).astype(np.uint32)
    return r.view(np.float32)


def bf16_bits(a):
    """bf16 bit patterns (uint16) of float32 values already rounded to bf16."""
    return (np.ascontiguousarray(a, dtype=np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bits_to_f32(u):
    """float32 values of bf16 bit patterns."""
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _streams(seed, n=12):
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(n)]


def _unit_rows(a):
    return a / np.linalg.norm(a, axis=-1, keepdims=True)


def _io(a, io):
    a = np.asarray(a, dtype=np.float32)
    return round_bf16(a) if io == "bf16" else a


def score_weights(wl: Workload, seed=None):
    """W_score [d, 2] and W_mix [D, 2] (fp32)."""
    rs = _streams(wl.seed if seed is None else seed)
    w_score = rs[0].normal(0.0, 0.02, size=(wl.d, 2)).astype(np.float32)
    w_mix = rs[1].normal(0.0, 0.1, size=(wl.D, 2)).astype(np.float32)
    return w_score, w_mix


def layer_input(wl: Workload, seed=None, L=None):
    """x [B, L, d] before any planting (fp32, not yet rounded)."""
    rs = _streams(wl.seed if seed is None else seed)
    L = wl.L if L is None else L
    return rs[2].standard_normal(size=(wl.B, L, wl.d), dtype=np.float32)


def plan_bursts(nc, n_sm, n_burst, burst_total, min_burst, rng):
    """Route plan with n_burst runs of softmax chunks (lengths summing to
    burst_total, each >= min_burst, at random non-overlapping positions with
    at least one linear chunk between runs) plus n_sm - burst_total isolated
    softmax chunks, none adjacent to a run or to each other."""
    free = burst_total - n_burst * min_burst
    lens = min_burst + rng.multinomial(free, [1.0 / n_burst] * n_burst)
    plan = np.ones(nc, dtype=np.int32)  # 1 = linear
    blocked = np.zeros(nc, dtype=bool)
    for ln in lens:
        for _ in range(10000):
            s = int(rng.integers(1, nc - ln - 1))
            if not blocked[s - 1:s + ln + 1].any():
                plan[s:s + ln] = 0
                blocked[s - 1:s + ln + 1] = True
                break
        else:
            raise RuntimeError("could not place burst")
    n_single = n_sm - burst_total
    placed = 0
    for _ in range(100000):
        if placed == n_single:
            break
        s = int(rng.integers(0, nc))
        lo, hi = max(0, s - 1), min(nc, s + 2)
        if not blocked[lo:hi].any():
            plan[s] = 0
            blocked[lo:hi] = True
            placed += 1
    if placed != n_single:
        raise RuntimeError("could not place singles")
    return plan


def plant(x, w_score, plan, shift=1.0):
    """Shift every token of chunk c by +-shift * u, u = dw / |dw|^2 with
    dw = W_score[:,0] - W_score[:,1]: this moves the chunk's softmax-minus-
    linear score difference by +-shift (plus for planned softmax chunks).
    With shift = 1 the natural spread of that difference (std ~0.16 for
    d = 2048) cannot flip the planned sign."""
    dw = (w_score[:, 0].astype(np.float64) - w_score[:, 1].astype(np.float64))
    u = (dw / (dw @ dw)).astype(np.float32)
    sign = np.where(np.asarray(plan) == 0, 1.0, -1.0).astype(np.float32)  # [Nc]
    B, L, d = x.shape
    xs = x.reshape(B, -1, CHUNK, d)
    xs += (shift * sign)[None, :, None, None] * u[None, None, None, :]
    return xs.reshape(B, L, d)


def make_prefill(wl: Workload, seed=None, L=None, B=None, H=None, alpha_range=(0.90, 0.999),
                 q_scale=1.0, routing=None, sm_frac=0.5):
    """All prefill inputs of a workload as numpy arrays (float32 holding the
    exact values the GPU receives).  L, B, H may shrink the workload for
    quick cases; alpha_range and q_scale give the slow-decay and sharp-
    attention variants.  routing overrides the workload's own: "natural"
    (no planting), "planted" (bursts + singles), "iid" (every chunk planted
    softmax with probability sm_frac, independently)."""
    seed = wl.seed if seed is None else seed
    rs = _streams(seed)
    B = wl.B if B is None else B
    H = wl.H if H is None else H
    L = wl.L if L is None else L
    D, d = wl.D, wl.d
    w_score, w_mix = score_weights(wl, seed)
    x = rs[2].standard_normal(size=(B, L, d), dtype=np.float32)
    plan = None
    routing = wl.routing if routing is None else routing
    if routing == "iid":
        plan = np.where(rs[3].random(L // CHUNK) < sm_frac, 0, 1).astype(np.int32)
        x = plant(x, w_score, plan)
    elif routing == "forced":
        pass  # routes come from forced_routes() through route_override; x stays unplanted
    elif routing == "planted":
        e = wl.extra
        nc = L // CHUNK
        scale = nc / wl.nc
        plan = plan_bursts(nc, int(e["n_sm"] * scale), e["n_burst"], int(e["burst_total"] * scale),
                           max(1, int(e["min_burst"] * scale)), rs[3])
        x = plant(np.ascontiguousarray(x), w_score, plan)
    elif routing != "natural":
        raise ValueError(f"unknown routing {routing!r}")
    q = q_scale * rs[4].standard_normal(size=(B, H, L, D), dtype=np.float32)
    k = _unit_rows(rs[5].standard_normal(size=(B, H, L, D), dtype=np.float32))
    v = rs[6].standard_normal(size=(B, H, L, D), dtype=np.float32)
    beta = (1.0 / (1.0 + np.exp(-rs[7].standard_normal(size=(B, H, L))))).astype(np.float32)
    alpha = rs[8].uniform(alpha_range[0], alpha_range[1], size=(B, H, L)).astype(np.float32)
    io = wl.io
    return dict(x=_io(x, io), q=_io(q, io), k=_io(k, io), v=_io(v, io), alpha=alpha, beta=beta,
                w_score=w_score, w_mix=w_mix, b_score=np.zeros(2, np.float32),
                g_sm=np.ones(D, np.float32), g_lin=np.ones(D, np.float32), plan=plan, io=io)


# Native Hybrid Attention inputs (slots + sliding window): the long prefill's
# shape with 64 slots and a 2048-token window
NHA = dict(B=1, H=16, L=32768, D=128, slots=64, window=2048, seed=6)


def make_nha(B, H, L, D, slots, io="bf16", seed=6, q_scale=1.0, gate_mean=2.0):
    """q, v ~ N(0, 1), k ~ N(0, 1) L2-normalised per token (q scaled by
    q_scale for sharp attention), slot gates sigmoid(N(gate_mean, 1)) per
    token and slot (mean ~0.85: slots forget over a few tokens to a few tens
    of tokens); bf16 io rounds q, k, v.  Returns numpy float32 arrays."""
    rs = _streams(seed)
    q = q_scale * rs[4].standard_normal(size=(B, H, L, D), dtype=np.float32)
    k = _unit_rows(rs[5].standard_normal(size=(B, H, L, D), dtype=np.float32))
    v = rs[6].standard_normal(size=(B, H, L, D), dtype=np.float32)
    gate = (1.0 / (1.0 + np.exp(-(gate_mean + rs[7].standard_normal(size=(B, H, L, slots)))))).astype(np.float32)
    return dict(q=_io(q, io), k=_io(k, io), v=_io(v, io), gate=gate, io=io)


def forced_routes(B, nc, kind, G=1):
    """route [B, G, Nc] int32 for forced runs: 'sm' (all softmax) or 'lin'."""
    return np.full((B, G, nc), 0 if kind == "sm" else 1, dtype=np.int32)


def make_decode(wl: Workload, seed=None, B=None, H=None, cap=None, n_open=0):
    """Decode workload: a compacted cache per sequence plus one new token.

    n_sel[b] ~ U{lo..hi} softmax chunks are kept (64 * n_sel rows of unit-norm
    K and N(0,1) V per head); rows of an open chunk (n_open tokens) follow
    them.  S_carry (and S_work) ~ N(0, 1/Dk) fp32; x_sum = sum of n_open
    N(0,1) rows (0 when n_open = 0).  New x, q, k, v, alpha, beta use the
    prefill distributions.  The cache rows k, v are returned as bf16 bit
    patterns (uint16); bits_to_f32 gives their values."""
    seed = wl.seed if seed is None else seed
    rs = _streams(seed)
    B = wl.B if B is None else B
    H = wl.H if H is None else H
    D, d = wl.D, wl.d
    e = wl.extra
    n_sel = rs[3].integers(e["nsel_lo"], e["nsel_hi"] + 1, size=B)
    n_committed = (CHUNK * n_sel).astype(np.int32)
    if cap is None:
        cap = CHUNK * int(e["nsel_hi"]) + CHUNK
    kc = np.zeros((B, H, cap, D), np.uint16)  # bf16 bit patterns
    vc = np.zeros((B, H, cap, D), np.uint16)
    seq_seeds = np.random.SeedSequence([seed, 4]).spawn(B)  # one stream per sequence

    def fill(b):
        r = np.random.Generator(np.random.PCG64(seq_seeds[b]))
        n = int(n_committed[b]) + n_open
        kc[b, :, :n] = bf16_bits(round_bf16(_unit_rows(r.standard_normal(size=(H, n, D), dtype=np.float32))))
        vc[b, :, :n] = bf16_bits(round_bf16(r.standard_normal(size=(H, n, D), dtype=np.float32)))

    import concurrent.futures as cf
    with cf.ThreadPoolExecutor(min(16, os.cpu_count() or 4)) as ex:
        list(ex.map(fill, range(B)))
    S_carry = (rs[6].standard_normal(size=(B, H, D, D), dtype=np.float32) / np.sqrt(D)).astype(np.float32)
    S_work = (rs[7].standard_normal(size=(B, H, D, D), dtype=np.float32) / np.sqrt(D)).astype(np.float32)
    x_sum = np.zeros((B, 1, d), np.float32)
    if n_open:
        x_sum[:, 0] = rs[8].standard_normal(size=(B, n_open, d), dtype=np.float32).sum(axis=1)
    w_score, w_mix = score_weights(wl, seed)
    x = round_bf16(rs[9].standard_normal(size=(B, d), dtype=np.float32))
    q = round_bf16(rs[10].standard_normal(size=(B, H, D), dtype=np.float32))
    r2 = rs[11]
    k = round_bf16(_unit_rows(r2.standard_normal(size=(B, H, D), dtype=np.float32)))
    v = round_bf16(r2.standard_normal(size=(B, H, D), dtype=np.float32))
    beta = (1.0 / (1.0 + np.exp(-r2.standard_normal(size=(B, H))))).astype(np.float32)
    alpha = r2.uniform(0.90, 0.999, size=(B, H)).astype(np.float32)
    cache = dict(k=kc, v=vc, n_committed=n_committed.reshape(B, 1),
                 n_open=np.full((B, 1), n_open, np.int32), S_carry=S_carry, S_work=S_work,
                 x_sum=x_sum, err=0)
    return cache, dict(x=x, q=q, k=k, v=v, alpha=alpha, beta=beta, w_score=w_score, w_mix=w_mix,
                       b_score=np.zeros(2, np.float32), g_sm=np.ones(D, np.float32),
                       g_lin=np.ones(D, np.float32), io="bf16")
