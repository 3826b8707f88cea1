"""GPU parity of the router's gradient (straight-through reading of
"Technische Samenvatting: Neural Attention Search Linear (NAtS-L)",
Kernmechanismen 5): the gate derivatives of both branches and
natsl_route_backward, through the C ABI, against the oracle.  Each value is
compared relative to the largest magnitude of its kind."""
import sys

import numpy as np
import pytest
import torch

import linear_attention_natsl_amd as N
import oracle as O
import workloads as W
from tests.gpu_util import dev, host, maxerr

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def case(io, B, H, L, D, seed, alpha=(0.9, 0.999), q_scale=1.0):
    base = W.WORKLOADS["tiny"] if io == "f32" else W.WORKLOADS["prefill"]
    wl = W.Workload("case", io, B, H, L, D, 64 if io == "f32" else base.d, "iid", seed)
    return wl, W.make_prefill(wl, alpha_range=alpha, q_scale=q_scale, routing="iid", sm_frac=0.5)


def rel(got, ref):
    return maxerr(got, ref) / max(1e-30, float(np.abs(ref).max()))


@pytest.mark.parametrize("io,D,L,per_head,q_scale", [("f32", 64, 320, False, 1.0), ("bf16", 128, 640, False, 2.0),
                                                     ("bf16", 128, 576, True, 1.0)])
def test_softmax_gate_gradient(io, D, L, per_head, q_scale):
    """Every chunk's softmax-gate derivative (selected or not) against the
    oracle; dq, dk, dv are bit-identical with and without the gate output."""
    B, H = 2, 2
    G = H if per_head else 1
    nc = L // 64
    wl, inp = case(io, B, H, L, D, seed=91, q_scale=q_scale)
    r = (np.random.default_rng(91).random((B, G, nc)) < 0.5).astype(np.int32)
    r[:, :, 0] = 0
    sel, nsb = O.compact(r)
    dm = N.dims(B, H, L, D, wl.d, N.BF16 if io == "bf16" else N.F32, groups=G)
    say(f"[softmax gate] io={io} D={D} L={L} G={G}")
    tq, tk, tv = dev(inp["q"], io), dev(inp["k"], io), dev(inp["v"], io)
    io_t = torch.bfloat16 if io == "bf16" else torch.float32
    o, lse = N.softmax_masked(dm, tq, tk, tv, dev(sel), dev(nsb), o_dtype=io_t, want_lse=True)
    d_o = np.random.default_rng(92).standard_normal(inp["q"].shape).astype(np.float32)
    if io == "bf16":
        d_o = torch.from_numpy(d_o).to(torch.bfloat16).float().numpy()
    td_o = dev(d_o, io)
    dq, dk, dv, dg = N.softmax_masked_backward(dm, tq, tk, tv, dev(sel), dev(nsb), o, lse, td_o, want_gate=True)
    dq0, dk0, dv0 = N.softmax_masked_backward(dm, tq, tk, tv, dev(sel), dev(nsb), o, lse, td_o)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq0) and torch.equal(dk, dk0) and torch.equal(dv, dv0)
    *_, ref = O.softmax_branch_backward(inp["q"], inp["k"], inp["v"], r, d_o, with_gate=True)
    e = rel(host(dg), ref)
    say(f"  dgate rel err {e:.3e} (max |ref| {np.abs(ref).max():.3e})")
    assert e <= (1e-4 if io == "f32" else 3e-2)
    assert np.all(host(dg)[:, :, -1] == 0.0)


@pytest.mark.parametrize("io,D,L,per_head", [("f32", 64, 256, False), ("bf16", 128, 384, True)])
def test_gdn_gate_gradient(io, D, L, per_head):
    """Every chunk's linear-gate derivative against the oracle (fp32 within
    1e-4 of the largest magnitude, bf16 within 2e-2: bf16 matrix operands);
    the other gradients are bit-identical with and without it."""
    B, H = 2, 2
    G = H if per_head else 1
    wl, inp = case(io, B, H, L, D, seed=93, alpha=(0.995, 1.0))
    rng = np.random.default_rng(93)
    r = (rng.random((B, G, L // 64)) < 0.5).astype(np.int32)
    S0 = (rng.standard_normal((B, H, D, D)) / np.sqrt(D)).astype(np.float32)
    d_o = rng.standard_normal((B, H, L, D)).astype(np.float32)
    dS = rng.standard_normal((B, H, D, D)).astype(np.float32)
    dm = N.dims(B, H, L, D, wl.d, N.BF16 if io == "bf16" else N.F32, groups=G)
    say(f"[gdn gate] io={io} D={D} L={L} G={G}")
    args = (dm, dev(inp["q"], io), dev(inp["k"], io), dev(inp["v"], io), dev(inp["alpha"]), dev(inp["beta"]), dev(r),
            dev(d_o))
    got = N.gdn_backward(*args, S_init=dev(S0), dS_final=dev(dS), want_gate=True)
    got0 = N.gdn_backward(*args, S_init=dev(S0), dS_final=dev(dS))
    torch.cuda.synchronize()
    for a, b in zip(got[:6], got0):
        assert torch.equal(a, b)
    *_, ref = O.gdn_branch_backward(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], r, d_o, S_init=S0,
                                    dS_final=dS, with_gate=True)
    e = rel(host(got[6]), ref)
    say(f"  dgate rel err {e:.3e} (max |ref| {np.abs(ref).max():.3e})")
    assert e <= (1e-4 if io == "f32" else 2e-2)


@pytest.mark.parametrize("io,d,G,H,L", [("f32", 64, 1, 2, 320), ("bf16", 2048, 1, 4, 512), ("f32", 256, 4, 4, 256)])
def test_route_backward(io, d, G, H, L):
    """The straight-through step and the score layer's gradient (dW, db, dx)
    from given gate derivatives, against the oracle; the GPU takes the scores
    of its own router (fp32) where the oracle recomputes them in fp64."""
    B = 2
    rng = np.random.default_rng(95)
    x = rng.standard_normal((B, L, d)).astype(np.float32)
    if io == "bf16":
        x = W.round_bf16(x)
    w = rng.normal(0, 0.3, (d, 2 * G)).astype(np.float32)
    bias = rng.normal(0, 0.1, 2 * G).astype(np.float32)
    nc = L // 64
    dgs = rng.standard_normal((B, H, nc)).astype(np.float32)
    dgl = rng.standard_normal((B, H, nc)).astype(np.float32)
    dm = N.dims(B, H, L, 64, d, N.BF16 if io == "bf16" else N.F32, groups=G)
    say(f"[route backward] io={io} d={d} G={G}")
    tx = dev(x, io)
    _, _, _, scores = N.route(dm, tx, dev(w), dev(bias))
    dx, dW, db = N.route_backward(dm, tx, dev(w), scores, dev(dgs), dev(dgl))
    torch.cuda.synchronize()
    rdx, rdW, rdb, _ = O.route_backward(x, w, dgs, dgl, b_score=bias, groups=G)
    for name, g, rf in (("dx", dx, rdx), ("dW", dW, rdW), ("db", db, rdb)):
        e = rel(host(g), rf)
        say(f"  {name} rel err {e:.3e}")
        assert e <= 1e-4, name
