"""GPU parity of Native Hybrid Attention (one softmax over gated key-value
slots plus a sliding window) against the oracle's per-token definition,
through the C ABI.  Bars: fp32 max abs <= 1e-4 on the output; bf16 max abs
<= 3e-2 on the RMS-normalised output."""
import sys

import numpy as np
import pytest
import torch

import linear_attention_natsl_amd as N
import oracle as O
import workloads as W
from tests.gpu_util import TOL_BF16, TOL_F32, dev, host, maxerr, rmsn, rows_of_blocks

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run(inp, B, H, L, D, window):
    io = inp["io"]
    dm = N.dims(B, H, L, D, 64, N.BF16 if io == "bf16" else N.F32)
    out = N.nha_attention(dm, dev(inp["q"], io), dev(inp["k"], io), dev(inp["v"], io), dev(inp["gate"]), window)
    torch.cuda.synchronize()
    return host(out)


@pytest.mark.parametrize("io,D,m,L,window,q_scale", [
    ("f32", 64, 16, 320, 128, 1.0),
    ("f32", 64, 64, 448, 0, 1.0),      # window 0: the slots alone
    ("f32", 128, 32, 256, 64, 1.0),
    ("bf16", 128, 64, 640, 256, 1.0),
    ("bf16", 128, 64, 576, 576, 1.0),  # window covers the sequence: causal attention
    ("bf16", 128, 16, 704, 64, 4.0),   # sharp attention: a misplaced key or slot shows
    ("bf16", 128, 32, 512, 192, 2.0),  # 32 slots at bf16 D = 128, a three-chunk window
    ("bf16", 64, 32, 384, 128, 1.0),
    ("bf16", 128, 64, 448, 0, 1.0),
    ("f32", 128, 64, 320, 128, 1.0),   # the largest LDS footprint of the slot and chunk kernels
])
def test_nha_matches_oracle(io, D, m, L, window, q_scale):
    B, H = 2, 2
    say(f"[nha] io={io} D={D} m={m} L={L} window={window} q x{q_scale}")
    inp = W.make_nha(B, H, L, D, m, io=io, seed=L + m, q_scale=q_scale)
    out = run(inp, B, H, L, D, window)
    ref = O.nha_attention(inp["q"], inp["k"], inp["v"], inp["gate"], window)
    if io == "f32":
        e = maxerr(out, ref)
        say(f"  out err {e:.3e}")
        assert e <= TOL_F32
    else:
        e = maxerr(rmsn(out), rmsn(ref))
        say(f"  rms-normalised out err {e:.3e} (raw {maxerr(out, ref):.3e})")
        assert e <= TOL_BF16


def test_nha_gates_exactly_zero_and_one():
    """Gates of exactly 0 (overwrite) and 1 (keep, write nothing) mixed per
    slot and token: the running products stay exact."""
    B, H, L, D, m = 1, 2, 320, 64, 16
    inp = W.make_nha(B, H, L, D, m, io="f32", seed=5)
    r = np.random.default_rng(5).random(inp["gate"].shape)
    inp["gate"] = np.where(r < 0.2, 0.0, np.where(r > 0.8, 1.0, inp["gate"])).astype(np.float32)
    say("[nha] gates 0 / 1")
    out = run(inp, B, H, L, D, 128)
    ref = O.nha_attention(inp["q"], inp["k"], inp["v"], inp["gate"], 128)
    e = maxerr(out, ref)
    say(f"  out err {e:.3e}")
    assert e <= TOL_F32


def test_nha_full_size_sampled():
    """The NHA workload at its full size (B=1 H=16 L=32768 D=128, 64 slots,
    2048-token window, bf16) on sampled heads and query blocks (the oracle's
    slots still take every token)."""
    c = W.NHA
    inp = W.make_nha(c["B"], c["H"], c["L"], c["D"], c["slots"], io="bf16", seed=c["seed"])
    say(f"[nha] full size L={c['L']} window={c['window']}")
    out = run(inp, c["B"], c["H"], c["L"], c["D"], c["window"])
    blocks = [0, 1, 31, 32, 33, 200, 511]
    rows = rows_of_blocks(blocks)
    worst = 0.0
    for h in (0, 11):
        sl = lambda a: a[:, h:h + 1]
        ref = O.nha_attention(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["gate"]), c["window"],
                              query_blocks=blocks)
        e = maxerr(rmsn(out[0, h][rows]), rmsn(ref[0, 0][rows]))
        say(f"  h={h} rms-normalised out err {e:.3e}")
        worst = max(worst, e)
    assert worst <= TOL_BF16
