"""GPU parity: the HIP library, called through its C ABI, against the fp64
oracle on the same seeded inputs.

Bars: routes bit-exact; fp32 workloads max abs <= 1e-4 on out and on each
RMS-normalised branch; bf16 workloads max abs <= 3e-2 on RMS-normalised
outputs (out, n_sm, n_lin).  Full-size workloads are compared on sampled
heads / query blocks that the oracle computes one by one.
"""
import sys

import numpy as np
import pytest
import torch

import linear_attention_natsl_amd as N
import oracle as O
import workloads as W
from tests.gpu_util import (TOL_BF16, TOL_F32, dev, dev_bits, host, maxerr, oracle_head, prefill_tensors,
                            rmsn, rows_of_blocks)

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def io_code(inp):
    return N.BF16 if inp["io"] == "bf16" else N.F32


def run_forward(inp, wl_d, B, H, L, D, route_override=None, branch=None, groups=1, S_init=None):
    t = prefill_tensors(inp)
    dm = N.dims(B, H, L, D, wl_d, io_code(inp), groups=groups)
    ro = None if route_override is None else dev(np.ascontiguousarray(route_override, dtype=np.int32))
    Si = None if S_init is None else dev(S_init.astype(np.float32))
    f = N.Forward(dm, branch_dtype=branch, debug=True, want_state=True)
    f(t["x"] if route_override is None else None, t["q"], t["k"], t["v"], t["alpha"], t["beta"],
      t["w_score"] if route_override is None else None, t["w_mix"], b_score=t["b_score"] if route_override is None else None,
      g_sm=t["g_sm"], g_lin=t["g_lin"], route_override=ro, S_init=Si)
    torch.cuda.synchronize()
    return f


# ------------------------------------------------------------------ router ----
@pytest.mark.parametrize("name", ["tiny", "prefill", "long"])
def test_route_full_size_bitexact(name):
    wl = W.WORKLOADS[name]
    inp = W.make_prefill(wl)
    say(f"[route] {name} B={wl.B} L={wl.L} d={wl.d}")
    r_ref, margin = O.route(inp["x"], inp["w_score"], inp["b_score"])
    sel_ref, nsb_ref = O.compact(r_ref)
    dm = N.dims(wl.B, wl.H, wl.L, wl.D, wl.d, io_code(inp))
    r, sel, nsb, sc = N.route(dm, dev(inp["x"], inp["io"]), dev(inp["w_score"]), dev(inp["b_score"]))
    torch.cuda.synchronize()
    assert np.array_equal(r.cpu().numpy(), r_ref)
    assert np.array_equal(sel.cpu().numpy(), sel_ref)
    assert np.array_equal(nsb.cpu().numpy(), nsb_ref)
    s_ref = O.route_scores(inp["x"], inp["w_score"], inp["b_score"])
    assert maxerr(host(sc), s_ref) < 1e-5


def test_route_tie_and_forced():
    """Equal score columns tie exactly on the GPU too (same fp32 sums) and go
    to softmax; a forced route is copied and compacted."""
    wl = W.WORKLOADS["tiny"]
    inp = W.make_prefill(wl)
    w = np.repeat(inp["w_score"][:, :1], 2, axis=1).copy()
    dm = N.dims(1, 1, 256, 64, 64, N.F32)
    r, _, nsb, _ = N.route(dm, dev(inp["x"]), dev(w))
    assert (r.cpu().numpy() == 0).all() and nsb.cpu().numpy()[0, 0, -1] == 4
    forced = np.array([[[1, 0, 1, 0]]], np.int32)
    r2, sel2, nsb2, _ = N.route(dm, None, None, route_in=dev(forced))
    assert np.array_equal(r2.cpu().numpy(), forced)
    assert sel2.cpu().numpy()[0, 0].tolist() == [1, 3, -1, -1]
    assert nsb2.cpu().numpy()[0, 0].tolist() == [0, 0, 1, 1, 2]


def test_route_groups_per_head():
    """route_groups = H: every head has its own score columns."""
    r0 = np.random.default_rng(7)
    B, H, L, d = 2, 4, 512, 64
    x = r0.standard_normal((B, L, d)).astype(np.float32)
    w = r0.normal(0, 0.3, (d, 2 * H)).astype(np.float32)
    r_ref, m = O.route(x, w, groups=H)
    assert np.abs(m).min() > 1e-4
    dm = N.dims(B, H, L, 64, d, N.F32, groups=H)
    r, sel, nsb, _ = N.route(dm, dev(x), dev(w))
    assert np.array_equal(r.cpu().numpy(), r_ref)
    assert np.array_equal(nsb.cpu().numpy(), O.compact(r_ref)[1])


# ---------------------------------------------------------------- branches ----
def small_case(io="f32", B=1, H=2, L=640, D=64, seed=11, alpha=(0.9, 0.999), q_scale=1.0, sm_frac=0.5):
    base = W.WORKLOADS["tiny"] if io == "f32" else W.WORKLOADS["prefill"]
    wl = W.Workload("case", io, B, H, L, D, 64 if io == "f32" else base.d, "iid", seed)
    return wl, W.make_prefill(wl, alpha_range=alpha, q_scale=q_scale, routing="iid", sm_frac=sm_frac)


@pytest.mark.parametrize("io,D,L,q_scale", [("f32", 64, 256, 1.0), ("f32", 64, 576, 8.0), ("f32", 128, 320, 1.0),
                                            ("bf16", 128, 640, 1.0), ("bf16", 128, 576, 8.0), ("bf16", 64, 448, 1.0)])
def test_softmax_masked_parity(io, D, L, q_scale):
    """Odd chunk counts exercise the single-chunk last block; q x 8 gives
    sharp attention where one wrongly masked key shows."""
    wl, inp = small_case(io, B=2, H=2, L=L, D=D, q_scale=q_scale)
    say(f"[softmax] io={io} D={D} L={L} qs={q_scale}")
    r = np.broadcast_to(inp["plan"], (2, 1, L // 64)).copy()
    sel, nsb = O.compact(r)
    dm = N.dims(2, 2, L, D, wl.d, io_code(inp))
    o, lse = N.softmax_masked(dm, dev(inp["q"], io), dev(inp["k"], io), dev(inp["v"], io), dev(sel), dev(nsb),
                              want_lse=True)
    torch.cuda.synchronize()
    ref, lse_ref = O.softmax_branch(inp["q"], inp["k"], inp["v"], r, with_lse=True)
    tol = TOL_F32 if io == "f32" else TOL_BF16
    e = maxerr(rmsn(host(o)), rmsn(ref))
    say(f"  n_sm err {e:.3e}  raw {maxerr(host(o), ref):.3e}  lse {maxerr(host(lse), lse_ref):.3e}")
    assert e <= tol
    assert maxerr(host(lse), lse_ref) <= (1e-4 if io == "f32" else 2e-2)


@pytest.mark.parametrize("io,D,L,alpha", [("f32", 64, 256, (0.9, 0.999)), ("f32", 64, 640, (0.995, 1.0)),
                                          ("f32", 128, 320, (0.9, 0.999)), ("bf16", 128, 640, (0.9, 0.999)),
                                          ("bf16", 128, 640, (0.995, 1.0)), ("bf16", 64, 448, (0.9, 0.999))])
def test_gdn_chunk_parity(io, D, L, alpha):
    """alpha ~ U(0.995, 1) keeps old state alive so a rollback bug several
    chunks back still shows; a nonzero initial state checks S_init."""
    wl, inp = small_case(io, B=2, H=2, L=L, D=D, alpha=alpha, seed=12)
    say(f"[gdn] io={io} D={D} L={L} alpha={alpha}")
    r = np.broadcast_to(inp["plan"], (2, 1, L // 64)).copy()
    S0 = (np.random.default_rng(3).standard_normal((2, 2, D, D)) / np.sqrt(D)).astype(np.float32)
    dm = N.dims(2, 2, L, D, wl.d, io_code(inp))
    o, Sf = N.gdn_chunk(dm, dev(inp["q"], io), dev(inp["k"], io), dev(inp["v"], io), dev(inp["alpha"]),
                        dev(inp["beta"]), dev(r), S_init=dev(S0))
    torch.cuda.synchronize()
    ref, Sref = O.gdn_branch(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], r, S_init=S0)
    tol = TOL_F32 if io == "f32" else TOL_BF16
    e = maxerr(rmsn(host(o)), rmsn(ref))
    es = maxerr(host(Sf), Sref) / max(1.0, np.abs(Sref).max())
    say(f"  n_lin err {e:.3e} raw {maxerr(host(o), ref):.3e}  S_final rel {es:.3e}")
    assert e <= tol
    assert es <= (1e-4 if io == "f32" else 3e-2)


@pytest.mark.parametrize("per_head", [False, True])
def test_gdn_chunk_many_heads(per_head):
    """B * H = 128 heads: the bf16 D = 128 scan then runs one workgroup of
    eight waves per head (its U~ through one LDS buffer) instead of two of
    four.  Five chunks (an odd count), slow decay and an initial state; with
    per-head routes every head commits a different chunk set."""
    B, H, L, D = 8, 16, 320, 128
    wl, inp = small_case("bf16", B=B, H=H, L=L, D=D, alpha=(0.995, 1.0), seed=14)
    nc = L // 64
    rng = np.random.default_rng(5)
    if per_head:
        r = (rng.random((B, H, nc)) < 0.5).astype(np.int32)
    else:
        r = np.broadcast_to(inp["plan"], (B, 1, nc)).copy()
    G = H if per_head else 1
    say(f"[gdn many heads] B={B} H={H} L={L} per_head={per_head}")
    S0 = (rng.standard_normal((B, H, D, D)) / np.sqrt(D)).astype(np.float32)
    dm = N.dims(B, H, L, D, wl.d, io_code(inp), groups=G)
    o, Sf = N.gdn_chunk(dm, dev(inp["q"], "bf16"), dev(inp["k"], "bf16"), dev(inp["v"], "bf16"), dev(inp["alpha"]),
                        dev(inp["beta"]), dev(r), S_init=dev(S0))
    torch.cuda.synchronize()
    ref, Sref = O.gdn_branch(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], r, S_init=S0)
    e = maxerr(rmsn(host(o)), rmsn(ref))
    es = maxerr(host(Sf), Sref) / max(1.0, np.abs(Sref).max())
    say(f"  n_lin err {e:.3e}  S_final rel {es:.3e}")
    assert e <= TOL_BF16
    assert es <= 3e-2


@pytest.mark.parametrize("io,branch,D", [("f32", "f32", 64), ("bf16", "bf16", 128), ("bf16", "f32", 128),
                                         ("f32", "bf16", 128)])
def test_merge_parity(io, branch, D):
    rng = np.random.default_rng(5)
    B, H, L = 2, 3, 128
    q = rng.standard_normal((B, H, L, D)).astype(np.float32)
    a = (rng.standard_normal((B, H, L, D)) * 3).astype(np.float32)
    b = (rng.standard_normal((B, H, L, D)) * 0.1).astype(np.float32)
    if io == "bf16":
        q = W.round_bf16(q)
    if branch == "bf16":
        a, b = W.round_bf16(a), W.round_bf16(b)
    w_mix = rng.normal(0, 0.3, (H, D, 2)).astype(np.float32)
    gs = rng.uniform(0.5, 1.5, D).astype(np.float32)
    gl = rng.uniform(0.5, 1.5, D).astype(np.float32)
    dm = N.dims(B, H, L, D, 64, N.BF16 if io == "bf16" else N.F32)
    say(f"[merge] io={io} branch={branch} D={D}")
    out = N.merge(dm, dev(q, io), dev(a, branch), dev(b, branch), dev(w_mix), w_mix_head_stride=2 * D,
                  g_sm=dev(gs), g_lin=dev(gl))
    torch.cuda.synchronize()
    ref, _, _, _ = O.merge(q, a, b, w_mix, gs, gl)
    e = maxerr(host(out), ref)
    say(f"  out err {e:.3e}")
    assert e <= (TOL_F32 if io == "f32" else 2e-2)


# ----------------------------------------------------------------- forward ----
def test_forward_tiny_fp32():
    wl = W.WORKLOADS["tiny"]
    inp = W.make_prefill(wl)
    say("[forward] tiny fp32")
    f = run_forward(inp, wl.d, wl.B, wl.H, wl.L, wl.D)
    ref = O.forward(inp["x"], inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["w_score"],
                    inp["w_mix"], b_score=inp["b_score"], g_sm=inp["g_sm"], g_lin=inp["g_lin"])
    assert np.array_equal(f.route.cpu().numpy(), ref["route"])
    eo = maxerr(host(f.out), ref["out"])
    es = maxerr(rmsn(host(f.o_sm)), ref["n_sm"])
    el = maxerr(rmsn(host(f.o_gdn)), ref["n_lin"])
    say(f"  out {eo:.3e} n_sm {es:.3e} n_lin {el:.3e}")
    assert max(eo, es, el) <= TOL_F32


@pytest.mark.parametrize("kind", ["sm", "lin"])
def test_forward_forced_routes_small(kind):
    """All-softmax must be full causal attention; all-linear pure Gated
    DeltaNet (both pinned in the oracle tests)."""
    wl, inp = small_case("bf16", B=2, H=2, L=512, D=128, seed=21)
    r = W.forced_routes(2, 8, kind)
    say(f"[forward] forced {kind}")
    f = run_forward(inp, wl.d, 2, 2, 512, 128, route_override=r)
    ref = O.forward(None, inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], None, inp["w_mix"],
                    route_override=r, g_sm=inp["g_sm"], g_lin=inp["g_lin"])
    eo = maxerr(host(f.out), ref["out"])
    es = maxerr(rmsn(host(f.o_sm)), ref["n_sm"])
    el = maxerr(rmsn(host(f.o_gdn)), ref["n_lin"])
    say(f"  out {eo:.3e} n_sm {es:.3e} n_lin {el:.3e}")
    assert max(eo, es, el) <= TOL_BF16


def test_forward_edge_shapes():
    """L = 64 (one chunk), an odd chunk count, B = 0 (no-op), and G = H."""
    for (B, H, L, G) in [(1, 1, 64, 1), (3, 2, 192, 1), (2, 4, 320, 4)]:
        wl, inp = small_case("f32", B=B, H=H, L=L, D=64, seed=31 + L)
        say(f"[forward] edge B={B} H={H} L={L} G={G}")
        if G == 1:
            r = np.broadcast_to(inp["plan"], (B, 1, L // 64)).copy()
        else:
            r = (np.random.default_rng(L).random((B, G, L // 64)) < 0.5).astype(np.int32)
        f = run_forward(inp, wl.d, B, H, L, 64, route_override=r, groups=G)
        ref = O.forward(None, inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], None, inp["w_mix"],
                        route_override=r, groups=G)
        e = maxerr(host(f.out), ref["out"])
        say(f"  out err {e:.3e}")
        assert e <= TOL_F32
    dm = N.dims(0, 2, 128, 64, 64, N.F32)
    z = torch.empty(0, 2, 128, 64, device="cuda")
    out = N.softmax_masked(dm, z, z, z, torch.empty(0, 1, 2, dtype=torch.int32, device="cuda"),
                           torch.empty(0, 1, 3, dtype=torch.int32, device="cuda"))[0]
    assert out.numel() == 0


def test_forward_deterministic():
    wl, inp = small_case("bf16", B=1, H=4, L=1024, D=128, seed=41)
    r = np.broadcast_to(inp["plan"], (1, 1, 16)).copy()
    say("[forward] determinism")
    f1 = run_forward(inp, wl.d, 1, 4, 1024, 128, route_override=r)
    o1 = f1.out.clone()
    f2 = run_forward(inp, wl.d, 1, 4, 1024, 128, route_override=r)
    assert torch.equal(o1, f2.out)


# --------------------------------------------------------- full-size sampled ----
def full_forward_check(name, heads, query_blocks=None, route_kind=None, branch=None):
    wl = W.WORKLOADS[name]
    inp = W.make_prefill(wl)
    r_ref = W.forced_routes(wl.B, wl.nc, route_kind) if route_kind else O.route(inp["x"], inp["w_score"],
                                                                                 inp["b_score"])[0]
    say(f"[forward] full {name} {route_kind or ''} branch={branch} B={wl.B} H={wl.H} L={wl.L}")
    f = run_forward(inp, wl.d, wl.B, wl.H, wl.L, wl.D, route_override=r_ref if route_kind else None, branch=branch)
    if not route_kind:
        assert np.array_equal(f.route.cpu().numpy(), r_ref)
    worst = 0.0
    for (b, h) in heads:
        ref = oracle_head(inp, b, h, r_ref[b], query_blocks=query_blocks)
        rows = slice(None) if query_blocks is None else rows_of_blocks(query_blocks)
        out = host(f.out[b, h])
        eo = maxerr(out[rows], ref["out"][rows])
        es = maxerr(rmsn(host(f.o_sm[b, h]))[rows], ref["n_sm"][rows])
        el = maxerr(rmsn(host(f.o_gdn[b, h])), ref["n_lin"])
        say(f"  (b={b},h={h}) out {eo:.3e} n_sm {es:.3e} n_lin {el:.3e}")
        worst = max(worst, eo, es, el)
    assert worst <= TOL_BF16


def test_forward_per_head_mix_bf16():
    """bf16 D = 128 forward with per-head W_mix and branch gains.  This form
    takes the merge's mixing scores from the softmax branch (computed from the
    q fragments it holds) instead of re-reading q: checked against the oracle
    and against the public merge of the same branch outputs, which computes
    them from q."""
    B, H, L, D = 2, 4, 576, 128
    wl, inp = small_case("bf16", B=B, H=H, L=L, D=D, seed=77)
    say("[forward] bf16 D=128, per-head W_mix and gains")
    rng = np.random.default_rng(77)
    wmix = rng.normal(0, 0.3, (H, D, 2)).astype(np.float32)
    # gains <= 1, so the RMS-normalised outputs' tolerance bounds out as well
    g_sm = rng.uniform(0.5, 1.0, D).astype(np.float32)
    g_lin = rng.uniform(0.5, 1.0, D).astype(np.float32)
    t = prefill_tensors(inp)
    dm = N.dims(B, H, L, D, wl.d, N.BF16)
    f = N.Forward(dm, debug=True)
    f(t["x"], t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["w_score"], dev(wmix), b_score=t["b_score"],
      g_sm=dev(g_sm), g_lin=dev(g_lin), w_mix_head_stride=2 * D)
    m = N.merge(dm, t["q"], f.o_sm, f.o_gdn, dev(wmix), w_mix_head_stride=2 * D, g_sm=dev(g_sm), g_lin=dev(g_lin))
    torch.cuda.synchronize()
    ref = O.forward(inp["x"], inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["w_score"], wmix,
                    inp["b_score"], g_sm, g_lin)
    assert np.array_equal(f.route.cpu().numpy(), ref["route"])
    e = maxerr(host(f.out), ref["out"])
    e2 = maxerr(host(f.out), host(m))
    say(f"  out err vs oracle {e:.3e}, vs merge from q {e2:.3e}")
    assert e <= TOL_BF16
    # the same bf16 branch outputs mixed two ways: at most a few bf16 roundings apart
    assert e2 <= 1e-2


def per_group_scores(w1, G):
    """W_score [d, 2G] whose odd groups score with the shared columns swapped:
    on x planted for w1 (|margin| ~ 1) the odd groups take the opposite route
    of the even ones, so routes differ between heads and stay far from ties."""
    return np.ascontiguousarray(np.concatenate([w1 if g % 2 == 0 else w1[:, ::-1] for g in range(G)], axis=1))


@pytest.mark.parametrize("L,alpha,q_scale,routing", [(640, (0.9, 0.999), 1.0, "router"),
                                                      (2112, (0.995, 1.0), 1.0, "forced"),
                                                      (576, (0.9, 0.999), 8.0, "forced")])
def test_forward_groups_per_head_bf16_d128(L, alpha, q_scale, routing):
    """route_groups = H on the bf16 D = 128 path (k_softmax_v2 with one tile
    list per head, the head-form scan with per-head routes), element by
    element against the oracle's G = H forward: routes bit-exact, out, n_sm
    and n_lin within the bf16 tolerance.  "router": the GPU router scores
    every head with its own columns and a per-group bias; "forced": random
    per-head routes.  alpha ~ U(0.995, 1) keeps a wrong rollback visible many
    chunks later; q x 8 makes one wrongly masked key visible."""
    B, H, D = 2, 4, 128
    G = H
    wl, inp = small_case("bf16", B=B, H=H, L=L, D=D, seed=79, alpha=alpha, q_scale=q_scale, sm_frac=0.5)
    nc = L // 64
    say(f"[forward] bf16 D=128 G=H L={L} alpha={alpha} q x{q_scale} {routing}")
    rng = np.random.default_rng(L)
    wmix = rng.normal(0, 0.3, (H, D, 2)).astype(np.float32)
    t = prefill_tensors(inp)
    dm = N.dims(B, H, L, D, wl.d, N.BF16, groups=G)
    f = N.Forward(dm, debug=True, want_state=True)
    if routing == "router":
        wG = per_group_scores(inp["w_score"], G)
        bG = np.tile(np.array([0.05, -0.05], np.float32), G)
        f(t["x"], t["q"], t["k"], t["v"], t["alpha"], t["beta"], dev(wG), dev(wmix), b_score=dev(bG),
          g_sm=t["g_sm"], g_lin=t["g_lin"], w_mix_head_stride=2 * D)
        torch.cuda.synchronize()
        ref = O.forward(inp["x"], inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], wG, wmix, b_score=bG,
                        g_sm=inp["g_sm"], g_lin=inp["g_lin"], groups=G)
        assert np.abs(ref["margin"]).min() > 1e-3
        assert (ref["route"][:, 0] != ref["route"][:, 1]).all()
    else:
        r = (rng.random((B, G, nc)) < 0.5).astype(np.int32)
        r[:, :, 0] = 0
        f(None, t["q"], t["k"], t["v"], t["alpha"], t["beta"], None, dev(wmix), g_sm=t["g_sm"], g_lin=t["g_lin"],
          route_override=dev(r), w_mix_head_stride=2 * D)
        torch.cuda.synchronize()
        ref = O.forward(None, inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], None, wmix,
                        route_override=r, g_sm=inp["g_sm"], g_lin=inp["g_lin"], groups=G)
    assert np.array_equal(f.route.cpu().numpy(), ref["route"])
    eo = maxerr(host(f.out), ref["out"])
    es = maxerr(rmsn(host(f.o_sm)), ref["n_sm"])
    el = maxerr(rmsn(host(f.o_gdn)), ref["n_lin"])
    eS = maxerr(host(f.S_final), ref["S_final"]) / max(1.0, np.abs(ref["S_final"]).max())
    say(f"  out {eo:.3e} n_sm {es:.3e} n_lin {el:.3e} S_final rel {eS:.3e}")
    assert max(eo, es, el) <= TOL_BF16
    assert eS <= TOL_BF16


@pytest.mark.parametrize("branch", [None, torch.float32])
def test_forward_prefill_full_sampled(branch):
    full_forward_check("prefill", heads=[(0, 0), (1, 7), (3, 15)], branch=branch)


def test_forward_long_full_sampled():
    blocks = [0, 1, 100, 255, 256, 300, 400, 477, 510, 511]
    full_forward_check("long", heads=[(0, 5)], query_blocks=blocks)


@pytest.mark.parametrize("kind", ["sm", "lin"])
def test_forward_degen_full_sampled(kind):
    blocks = [0, 1, 63, 64, 127] if kind == "sm" else None
    full_forward_check("degen", heads=[(0, 0), (1, 9)], query_blocks=blocks, route_kind=kind)


# ------------------------------------------------------------------ decode ----
def load_state(cache, B, H, D, d, io, groups=1):
    st = N.DecodeState(B, H, D, d, cache["k"].shape[2], groups=groups,
                       io=torch.bfloat16 if io == "bf16" else torch.float32)
    if cache["k"].dtype == np.uint16:
        st.k.copy_(dev_bits(cache["k"]))
        st.v.copy_(dev_bits(cache["v"]))
    else:
        st.k.copy_(dev(cache["k"].astype(np.float32), io))
        st.v.copy_(dev(cache["v"].astype(np.float32), io))
    st.n_committed.copy_(dev(np.asarray(cache["n_committed"], np.int32).reshape(B, groups)))
    st.n_open.copy_(dev(np.asarray(cache["n_open"], np.int32).reshape(B, -1)[:, 0].copy()))
    st.S_carry.copy_(dev(cache["S_carry"].astype(np.float32)))
    st.S_work.copy_(dev(cache["S_work"].astype(np.float32)))
    xs = np.asarray(cache["x_sum"], np.float32).reshape(B, -1, d)[:, 0]
    st.x_sum.copy_(dev(np.ascontiguousarray(xs)))
    return st


@pytest.mark.parametrize("io,D", [("f32", 64), ("bf16", 128)])
def test_decode_steps_match_oracle(io, D):
    """Prefix of 100 tokens, then 150 decode steps one at a time, crossing
    chunk completions of both routes; every step's output and the final
    counters and states against the oracle's decode."""
    B, H, L = 2, 2, 256
    wl, inp = small_case(io, B=B, H=H, L=L, D=D, seed=51, sm_frac=0.5)
    d = wl.d
    n0 = 100
    say(f"[decode] steps io={io} D={D}")
    cache = O.build_cache(inp["x"][:, :n0], inp["k"][:, :, :n0], inp["v"][:, :, :n0], inp["alpha"][:, :, :n0],
                          inp["beta"][:, :, :n0], inp["w_score"], cap=L + 64)
    st = load_state(cache, B, H, D, d, io)
    dm = N.dims(B, H, L, D, d, N.BF16 if io == "bf16" else N.F32)
    dec = N.Decode(dm, st, debug=True)
    t = prefill_tensors(inp)
    tol = TOL_F32 if io == "f32" else TOL_BF16
    worst = 0.0
    seen = set()
    for tok in range(n0, L):
        args = [t["x"][:, tok].contiguous(), t["q"][:, :, tok].contiguous(), t["k"][:, :, tok].contiguous(),
                t["v"][:, :, tok].contiguous(), t["alpha"][:, :, tok].contiguous(),
                t["beta"][:, :, tok].contiguous(), t["w_score"], t["w_mix"]]
        dec(*args)
        out_ref, br, cache = O.decode_step(cache, inp["x"][:, tok], inp["q"][:, :, tok], inp["k"][:, :, tok],
                                           inp["v"][:, :, tok], inp["alpha"][:, :, tok], inp["beta"][:, :, tok],
                                           inp["w_score"], inp["w_mix"])
        torch.cuda.synchronize()
        routes = dec.route.cpu().numpy()
        assert np.array_equal(routes, br["routes"]), f"tok {tok}"
        seen.update(int(x) for x in routes.ravel() if x >= 0)
        e = max(maxerr(host(dec.out), out_ref), maxerr(rmsn(host(dec.o_sm)), br["n_sm"]),
                maxerr(rmsn(host(dec.o_gdn)), br["n_lin"]))
        worst = max(worst, e)
        assert e <= tol, f"tok {tok}: err {e}"
    say(f"  worst err {worst:.3e}, routes seen {seen}")
    assert seen == {0, 1}
    assert np.array_equal(st.n_committed.cpu().numpy(), cache["n_committed"].astype(np.int32))
    assert np.array_equal(st.n_open.cpu().numpy(), cache["n_open"][:, 0].astype(np.int32))
    assert maxerr(host(st.S_carry), cache["S_carry"]) <= (1e-4 if io == "f32" else 1e-2)
    assert int(st.err.item()) == 0


@pytest.mark.parametrize("io,D,L,q_scale,per_head,H", [("f32", 64, 256, 1.0, False, 2), ("f32", 128, 320, 1.0, False, 2),
                                                        ("bf16", 128, 640, 1.0, False, 2),
                                                        ("bf16", 128, 576, 8.0, False, 2),
                                                        ("bf16", 64, 448, 1.0, True, 2),
                                                        ("bf16", 128, 448, 2.0, True, 4)])
def test_softmax_backward_parity(io, D, L, q_scale, per_head, H):
    """Gradient of the softmax branch against the oracle's derivative, from
    the GPU forward's o and lse; the error is taken relative to each
    gradient's largest magnitude (bf16: P and dS are rounded to bf16 for the
    matrix cores, and o is the bf16 forward output).  B * H = 8 takes the
    kernels' XCD-aware block order; 7 chunks leave a ragged last block of 4."""
    B = 2
    wl, inp = small_case(io, B=B, H=H, L=L, D=D, q_scale=q_scale, seed=81)
    G = H if per_head else 1
    nc = L // 64
    if per_head:
        r = (np.random.default_rng(81).random((B, G, nc)) < 0.5).astype(np.int32)
    else:
        r = np.broadcast_to(inp["plan"], (B, 1, nc)).copy()
    sel, nsb = O.compact(r)
    dm = N.dims(B, H, L, D, wl.d, io_code(inp), groups=G)
    say(f"[softmax backward] io={io} D={D} L={L} qs={q_scale} G={G}")
    tq, tk, tv = dev(inp["q"], io), dev(inp["k"], io), dev(inp["v"], io)
    io_t = torch.bfloat16 if io == "bf16" else torch.float32
    o, lse = N.softmax_masked(dm, tq, tk, tv, dev(sel), dev(nsb), o_dtype=io_t, want_lse=True)
    d_o = np.random.default_rng(82).standard_normal(inp["q"].shape).astype(np.float32)
    if io == "bf16":
        d_o = torch.from_numpy(d_o).to(torch.bfloat16).float().numpy()
    dq, dk, dv = N.softmax_masked_backward(dm, tq, tk, tv, dev(sel), dev(nsb), o, lse, dev(d_o, io))
    torch.cuda.synchronize()
    ref = O.softmax_branch_backward(inp["q"], inp["k"], inp["v"], r, d_o)
    tol = 1e-4 if io == "f32" else 3e-2
    for name, got, rf in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        e = maxerr(host(got), rf) / max(1e-30, float(np.abs(rf).max()))
        say(f"  {name} rel err {e:.3e}")
        assert e <= tol, (name, e)


@pytest.mark.parametrize("io,D,L,per_head,alpha", [("f32", 64, 256, False, (0.9, 0.999)),
                                                   ("f32", 128, 320, False, (0.995, 1.0)),
                                                   ("bf16", 128, 384, True, (0.9, 0.999)),
                                                   ("bf16", 64, 448, False, (0.995, 1.0)),
                                                   ("bf16", 128, 8192, False, (0.995, 1.0)),
                                                   ("bf16", 128, 64, False, (0.9, 0.999)),
                                                   ("f32", 64, 128, True, (0.9, 0.999))])
def test_gdn_backward_parity(io, D, L, per_head, alpha):
    """Gradient of the Gated DeltaNet branch through the rollback (q, k, v,
    alpha, beta and the initial state, with upstream gradients on the outputs
    and on the final carried state) against the oracle's exact derivative.
    Mixed routes, so both the commit and the restore paths carry gradient;
    alpha ~ U(0.995, 1) keeps gradients flowing many chunks back.  fp32:
    each gradient within 1e-4 of its largest magnitude; bf16: within 2e-2
    (the chunk form's matrix products take bf16 operands with fp32
    accumulation, as the forward's do: about ten bf16 roundings of the
    largest term)."""
    B, H = 2, 2
    G = H if per_head else 1
    wl, inp = small_case(io, B=B, H=H, L=L, D=D, alpha=alpha, seed=81)
    say(f"[gdn backward] io={io} D={D} L={L} G={G} alpha={alpha}")
    rng = np.random.default_rng(82)
    if per_head:
        r = (rng.random((B, G, L // 64)) < 0.5).astype(np.int32)
    else:
        r = np.broadcast_to(inp["plan"], (B, 1, L // 64)).copy().astype(np.int32)
    S0 = (rng.standard_normal((B, H, D, D)) / np.sqrt(D)).astype(np.float32)
    d_o = rng.standard_normal((B, H, L, D)).astype(np.float32)
    dS = rng.standard_normal((B, H, D, D)).astype(np.float32)
    dm = N.dims(B, H, L, D, wl.d, io_code(inp), groups=G)
    got = N.gdn_backward(dm, dev(inp["q"], io), dev(inp["k"], io), dev(inp["v"], io), dev(inp["alpha"]),
                         dev(inp["beta"]), dev(r), dev(d_o), S_init=dev(S0), dS_final=dev(dS))
    torch.cuda.synchronize()
    ref = O.gdn_branch_backward(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], r, d_o, S_init=S0,
                                dS_final=dS)
    tol = 1e-4 if io == "f32" else 2e-2
    errs = {}
    for name, g, rf in zip(("dq", "dk", "dv", "dalpha", "dbeta", "dS_init"), got, ref):
        errs[name] = maxerr(host(g), rf) / max(1.0, np.abs(rf).max())
        say(f"  {name}: rel err {errs[name]:.2e} (max |ref| {np.abs(rf).max():.2e})")
    assert all(e <= tol for e in errs.values()), errs


@pytest.mark.parametrize("io,D,per_head", [("bf16", 128, False), ("bf16", 128, True), ("f32", 64, False),
                                            ("f32", 128, True), ("bf16", 64, False)])
def test_gdn_backward_overlap_matches_sequential(io, D, per_head):
    """With the overlapping workspace natsl_gdn_backward runs the state scan
    and the reverse scan at the same time on two streams; every output (and
    the gate derivative) is bit-identical to the sequential schedule's, and the
    sequential call after it (its region shared again) is unaffected."""
    B, H, L = 2, 4, 1280
    G = H if per_head else 1
    wl, inp = small_case(io, B=B, H=H, L=L, D=D, alpha=(0.995, 1.0), seed=85)
    say(f"[gdn backward overlap] io={io} D={D} G={G}")
    rng = np.random.default_rng(86)
    r = (rng.random((B, G, L // 64)) < 0.5).astype(np.int32)
    S0 = (rng.standard_normal((B, H, D, D)) / np.sqrt(D)).astype(np.float32)
    d_o = rng.standard_normal((B, H, L, D)).astype(np.float32)
    dS = rng.standard_normal((B, H, D, D)).astype(np.float32)
    dm = N.dims(B, H, L, D, wl.d, io_code(inp), groups=G)
    args = (dm, dev(inp["q"], io), dev(inp["k"], io), dev(inp["v"], io), dev(inp["alpha"]), dev(inp["beta"]), dev(r),
            dev(d_o))
    kw = dict(S_init=dev(S0), dS_final=dev(dS), want_gate=True)
    seq = N.gdn_backward(*args, **kw)
    ovl = N.gdn_backward(*args, overlap=True, **kw)
    seq2 = N.gdn_backward(*args, **kw)
    torch.cuda.synchronize()
    for name, a, b, c in zip(("dq", "dk", "dv", "dalpha", "dbeta", "dS_init", "dgate"), seq, ovl, seq2):
        assert torch.equal(a, b), name
        assert torch.equal(a, c), name


@pytest.mark.parametrize("io,branch,D,per_head,gains,shape", [("f32", "f32", 64, False, False, (2, 3, 128)),
                                                              ("bf16", "bf16", 128, True, True, (2, 3, 128)),
                                                              ("bf16", "f32", 128, False, True, (2, 3, 128)),
                                                              ("bf16", "bf16", 128, False, True, (1, 2, 70016)),
                                                              ("bf16", "bf16", 128, True, False, (1, 2, 70016))])
def test_merge_backward_parity(io, branch, D, per_head, gains, shape):
    """Gradient of the merge (both branch outputs, q through the mixing
    weights, W_mix shared or per head, the gains) against the oracle's exact
    derivative; each within 1e-4 of its largest magnitude (the kernel works in
    fp32 on the same inputs; W_mix and gain gradients are sums over every
    token, added in a fixed order).  The 70016-token cases give the reduce of
    the blocks' partials long, uneven ranges (8752 blocks over 64 ranges shared,
    4376 per head), so that both its 16-load rounds and its tail run."""
    B, H, L = shape
    say(f"[merge backward] io={io} branch={branch} D={D} per_head={per_head} gains={gains}")
    rng = np.random.default_rng(95)
    io_t = torch.bfloat16 if io == "bf16" else torch.float32
    br_t = torch.bfloat16 if branch == "bf16" else torch.float32
    mk = lambda scale, dt: torch.from_numpy((scale * rng.standard_normal((B, H, L, D))).astype(np.float32)).cuda().to(dt)
    q, a, b = mk(1.0, io_t), mk(2.0, br_t), mk(0.5, br_t)
    wm = rng.normal(0, 0.3, (H, D, 2) if per_head else (D, 2)).astype(np.float32)
    gs = rng.uniform(0.5, 1.5, D).astype(np.float32) if gains else None
    gl = rng.uniform(0.5, 1.5, D).astype(np.float32) if gains else None
    d_out = rng.standard_normal((B, H, L, D)).astype(np.float32)
    dm = N.dims(B, H, L, D, 64, N.BF16 if io == "bf16" else N.F32)
    got = N.merge_backward(dm, q, a, b, dev(wm), dev(d_out), w_mix_head_stride=2 * D if per_head else 0,
                           g_sm=None if gs is None else dev(gs), g_lin=None if gl is None else dev(gl))
    torch.cuda.synchronize()
    h64 = lambda x: x.float().cpu().numpy().astype(np.float64)
    ref = O.merge_backward(h64(q), h64(a), h64(b), wm, d_out, gs, gl)
    for name, g, rf in zip(("d_o_sm", "d_o_gdn", "dq", "dw_mix", "dg_sm", "dg_lin"), got, ref):
        e = maxerr(h64(g), rf) / max(1.0, np.abs(rf).max())
        say(f"  {name}: rel err {e:.2e}")
        assert e <= 1e-4, name


@pytest.mark.parametrize("io,D", [("f32", 64), ("bf16", 128)])
def test_layer_gradient_chain(io, D):
    """The layer's gradient for fixed routes on the GPU: the forward's branch
    outputs (natsl_softmax_masked with lse, natsl_gdn_chunk), then
    natsl_merge_backward, natsl_softmax_masked_backward (upstream gradient in
    the io dtype, as that entry takes it) and natsl_gdn_backward, the three
    shares of dq summed.  Against the oracle's chain (pinned on the CPU by
    central differences of the whole layer).  fp32: within 1e-4 of each
    gradient's largest magnitude; bf16: 1e-2 (the softmax branch's upstream
    gradient is rounded to bf16)."""
    B, H, L = 2, 2, 320
    wl, inp = small_case(io, B=B, H=H, L=L, D=D, seed=99)
    say(f"[layer gradient] io={io} D={D}")
    rng = np.random.default_rng(98)
    r = np.broadcast_to(inp["plan"], (B, 1, L // 64)).copy().astype(np.int32)
    gs = rng.uniform(0.5, 1.5, D).astype(np.float32)
    gl = rng.uniform(0.5, 1.5, D).astype(np.float32)
    d_out = rng.standard_normal((B, H, L, D)).astype(np.float32)
    io_t = torch.bfloat16 if io == "bf16" else torch.float32
    dm = N.dims(B, H, L, D, wl.d, io_code(inp))
    tq, tk, tv = dev(inp["q"], io), dev(inp["k"], io), dev(inp["v"], io)
    ta, tb, tr = dev(inp["alpha"]), dev(inp["beta"]), dev(r)
    _, sel, nsb, _ = N.route(dm, None, None, route_in=tr)
    o_sm, lse = N.softmax_masked(dm, tq, tk, tv, sel, nsb, o_dtype=io_t, want_lse=True)
    o_gdn, _ = N.gdn_chunk(dm, tq, tk, tv, ta, tb, tr, o_dtype=io_t)
    d_sm, d_gdn, dq_mix, dwm, dgs, dgl = N.merge_backward(dm, tq, o_sm, o_gdn, dev(inp["w_mix"]), dev(d_out),
                                                          g_sm=dev(gs), g_lin=dev(gl))
    dq1, dk1, dv1 = N.softmax_masked_backward(dm, tq, tk, tv, sel, nsb, o_sm, lse, d_sm.to(io_t))
    dq2, dk2, dv2, da, db, _ = N.gdn_backward(dm, tq, tk, tv, ta, tb, tr, d_gdn)
    got = {"dq": dq_mix + dq1 + dq2, "dk": dk1 + dk2, "dv": dv1 + dv2, "dalpha": da, "dbeta": db,
           "dw_mix": dwm, "dg_sm": dgs, "dg_lin": dgl}
    torch.cuda.synchronize()
    fwd = O.forward(inp["x"], inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], None, inp["w_mix"],
                    g_sm=gs, g_lin=gl, route_override=r)
    e_sm, e_gdn, eq_mix, ewm, egs, egl = O.merge_backward(inp["q"], fwd["o_sm"], fwd["o_gdn"], inp["w_mix"], d_out,
                                                          gs, gl)
    eq1, ek1, ev1 = O.softmax_branch_backward(inp["q"], inp["k"], inp["v"], r, e_sm)
    eq2, ek2, ev2, ea, eb, _ = O.gdn_branch_backward(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], r, e_gdn)
    ref = {"dq": eq_mix + eq1 + eq2, "dk": ek1 + ek2, "dv": ev1 + ev2, "dalpha": ea, "dbeta": eb, "dw_mix": ewm,
           "dg_sm": egs, "dg_lin": egl}
    tol = 1e-4 if io == "f32" else 1e-2
    for name in ref:
        e = maxerr(host(got[name]), ref[name]) / max(1.0, np.abs(ref[name]).max())
        say(f"  {name}: rel err {e:.2e}")
        assert e <= tol, name


@pytest.mark.parametrize("io,D", [("f32", 64), ("bf16", 128)])
def test_decode_handoff_then_decode(io, D):
    """natsl_forward over a 192-token prefix, natsl_decode_handoff of its
    route, K/V and final state, then 64 decode steps (one chunk completion):
    the handed-off cache equals the oracle's cache for the prefix (rows and
    counters bit-exact, S_carry = the forward's S_final), and every decoded
    output matches the oracle's decode from that cache."""
    B, H, L, n0 = 2, 2, 256, 192
    wl, inp = small_case(io, B=B, H=H, L=L, D=D, seed=61, sm_frac=0.5)
    d = wl.d
    say(f"[handoff] io={io} D={D}")
    pre = {k: (val[:, :n0] if k == "x" else val[:, :, :n0]) if k in ("x", "q", "k", "v", "alpha", "beta") else val
           for k, val in inp.items()}
    f = run_forward(pre, d, B, H, n0, D)
    cap = L + 64
    st = N.DecodeState(B, H, D, d, cap, io=torch.bfloat16 if io == "bf16" else torch.float32)
    st.n_committed.fill_(5)
    st.n_open.fill_(7)
    st.err.fill_(3)
    st.x_sum.fill_(1.0)
    st.S_work.fill_(2.0)
    dm_pre = N.dims(B, H, n0, D, d, io_code(inp))
    tp = prefill_tensors(pre)
    N.decode_handoff(dm_pre, f.route, tp["k"], tp["v"], f.S_final, st)
    torch.cuda.synchronize()
    ref = O.build_cache(pre["x"], pre["k"], pre["v"], pre["alpha"], pre["beta"], pre["w_score"], pre["b_score"],
                        cap=cap)
    nco = ref["n_committed"].astype(np.int32)
    assert np.array_equal(st.n_committed.cpu().numpy(), nco)
    assert np.array_equal(st.n_open.cpu().numpy(), np.zeros(B, np.int32))
    assert int(st.err.item()) == 0
    assert not st.x_sum.any() and not st.S_work.any()
    assert torch.equal(st.S_carry, f.S_final)
    kc, vc = host(st.k), host(st.v)
    for b in range(B):
        n = int(nco[b, 0])
        assert 0 < n < n0
        assert np.array_equal(kc[b, :, :n], ref["k"][b, :, :n]) and np.array_equal(vc[b, :, :n], ref["v"][b, :, :n])
    e_state = maxerr(host(st.S_carry), ref["S_carry"])
    say(f"  S_carry err {e_state:.3e}")
    assert e_state <= (1e-4 if io == "f32" else 1e-2)
    # continue with decode steps from the handed-off cache
    dm = N.dims(B, H, L, D, d, io_code(inp))
    dec = N.Decode(dm, st, debug=True)
    t = prefill_tensors(inp)
    tol = TOL_F32 if io == "f32" else TOL_BF16
    cache = ref
    worst = 0.0
    for tok in range(n0, L):
        dec(t["x"][:, tok].contiguous(), t["q"][:, :, tok].contiguous(), t["k"][:, :, tok].contiguous(),
            t["v"][:, :, tok].contiguous(), t["alpha"][:, :, tok].contiguous(), t["beta"][:, :, tok].contiguous(),
            t["w_score"], t["w_mix"], b_score=t["b_score"], g_sm=t["g_sm"], g_lin=t["g_lin"])
        out_ref, br, cache = O.decode_step(cache, inp["x"][:, tok], inp["q"][:, :, tok], inp["k"][:, :, tok],
                                           inp["v"][:, :, tok], inp["alpha"][:, :, tok], inp["beta"][:, :, tok],
                                           inp["w_score"], inp["w_mix"], inp["b_score"], inp["g_sm"], inp["g_lin"])
        torch.cuda.synchronize()
        assert np.array_equal(dec.route.cpu().numpy(), br["routes"]), f"tok {tok}"
        e = maxerr(host(dec.out), out_ref)
        worst = max(worst, e)
        assert e <= tol, f"tok {tok}: err {e}"
    say(f"  decode worst err {worst:.3e}")
    assert np.array_equal(st.n_committed.cpu().numpy(), cache["n_committed"].astype(np.int32))
    assert int(st.err.item()) == 0


def test_decode_handoff_groups_and_capacity():
    """route_groups = H with forced per-head routes: each head's cache holds
    its own softmax chunks and S_carry follows its own linear chunks; with a
    capacity below the retained rows the flag is raised, the rows that fit
    are written and the counters still count every row."""
    B, H, L, D = 2, 4, 512, 128
    G = H
    wl, inp = small_case("bf16", B=B, H=H, L=L, D=D, seed=67, sm_frac=0.5)
    rng = np.random.default_rng(67)
    r = (rng.random((B, G, L // 64)) < 0.5).astype(np.int32)  # 1 = linear
    r[:, :, 0] = 0
    say("[handoff] groups = H, capacity")
    f = run_forward(inp, wl.d, B, H, L, D, route_override=r, groups=G)
    assert np.array_equal(f.route.cpu().numpy(), r)
    ref = O.forward(None, inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], None, inp["w_mix"],
                    route_override=r, g_sm=inp["g_sm"], g_lin=inp["g_lin"], groups=G)
    eo = maxerr(host(f.out), ref["out"])
    say(f"  forward out err vs oracle {eo:.3e}")
    assert eo <= TOL_BF16
    dm = N.dims(B, H, L, D, wl.d, N.BF16, groups=G)
    t = prefill_tensors(inp)
    nsm = (r == 0).sum(axis=2) * 64
    _, S_ref = O.gdn_branch(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], r)
    for cap in (L, int(nsm.max()) - 32):
        st = N.DecodeState(B, H, D, wl.d, cap, groups=G, io=torch.bfloat16)
        N.decode_handoff(dm, f.route, t["k"], t["v"], f.S_final, st)
        torch.cuda.synchronize()
        assert np.array_equal(st.n_committed.cpu().numpy(), nsm.astype(np.int32))
        assert int(st.err.item()) == (1 if cap < nsm.max() else 0)
        kc = host(st.k)
        for b in range(B):
            for h in range(H):
                rows = np.concatenate([inp["k"][b, h, c * 64:(c + 1) * 64] for c in range(L // 64) if r[b, h, c] == 0])
                n = min(len(rows), cap)
                assert np.array_equal(kc[b, h, :n], rows[:n]), (cap, b, h)
        assert torch.equal(st.S_carry, f.S_final)
    e = maxerr(host(f.S_final), S_ref)
    say(f"  S_final err {e:.3e}")
    assert e <= 1e-2


@pytest.mark.parametrize("io,D", [("f32", 64), ("bf16", 128)])
def test_decode_groups_per_head_mix(io, D):
    """Per-head routing in decode (route_groups = H), a score bias, per-head
    W_mix and branch gains.  Odd groups score with the two columns swapped,
    so their routes are the opposite of the even groups' at the same planted
    margin (|margin| ~ 1, the +-0.1 bias cannot flip it).  150 steps from a
    100-token prefix against the oracle's decode (fp32 D = 64 and the bf16
    D = 128 cache of the decode workload)."""
    B, H, L = 2, 4, 256
    G = H
    wl, inp = small_case(io, B=B, H=H, L=L, D=D, seed=71, sm_frac=0.5)
    d = wl.d
    wG = per_group_scores(inp["w_score"], G)
    bG = np.tile(np.array([0.1, -0.1], np.float32), G)
    wmix = np.random.default_rng(71).normal(0, 0.3, (H, D, 2)).astype(np.float32)
    n0 = 100
    say(f"[decode] groups = H, per-head W_mix, score bias, io={io} D={D}")
    cache = O.build_cache(inp["x"][:, :n0], inp["k"][:, :, :n0], inp["v"][:, :, :n0], inp["alpha"][:, :, :n0],
                          inp["beta"][:, :, :n0], wG, bG, cap=L + 64, groups=G)
    st = load_state(cache, B, H, D, d, io, groups=G)
    dm = N.dims(B, H, L, D, d, io_code(inp), groups=G)
    dec = N.Decode(dm, st, debug=True)
    t = prefill_tensors(inp)
    twG, tbG, twmix = dev(wG), dev(bG), dev(wmix)
    worst = 0.0
    seen = set()
    for tok in range(n0, L):
        dec(t["x"][:, tok].contiguous(), t["q"][:, :, tok].contiguous(), t["k"][:, :, tok].contiguous(),
            t["v"][:, :, tok].contiguous(), t["alpha"][:, :, tok].contiguous(), t["beta"][:, :, tok].contiguous(),
            twG, twmix, b_score=tbG, g_sm=t["g_sm"], g_lin=t["g_lin"], w_mix_head_stride=2 * D)
        out_ref, br, cache = O.decode_step(cache, inp["x"][:, tok], inp["q"][:, :, tok], inp["k"][:, :, tok],
                                           inp["v"][:, :, tok], inp["alpha"][:, :, tok], inp["beta"][:, :, tok],
                                           wG, wmix, bG, inp["g_sm"], inp["g_lin"])
        torch.cuda.synchronize()
        routes = dec.route.cpu().numpy()
        assert np.array_equal(routes, br["routes"]), f"tok {tok}"
        if (routes >= 0).any():
            assert np.array_equal(routes[:, 0::2], 1 - routes[:, 1::2]), "odd groups route opposite"
        seen.update(int(x) for x in routes.ravel() if x >= 0)
        e = max(maxerr(host(dec.out), out_ref), maxerr(rmsn(host(dec.o_sm)), br["n_sm"]),
                maxerr(rmsn(host(dec.o_gdn)), br["n_lin"]))
        worst = max(worst, e)
        assert e <= (TOL_F32 if io == "f32" else TOL_BF16), f"tok {tok}: err {e}"
    say(f"  worst err {worst:.3e}, routes seen {seen}")
    assert seen == {0, 1}
    assert np.array_equal(st.n_committed.cpu().numpy(), cache["n_committed"].astype(np.int32))
    assert maxerr(host(st.S_carry), cache["S_carry"]) <= (1e-4 if io == "f32" else 1e-3)
    # the cached rows of every head are its own softmax chunks' rows, bit for bit
    nco = st.n_committed.cpu().numpy()
    kc = host(st.k)
    for b in range(B):
        for h in range(H):
            n = int(nco[b, h])
            assert np.array_equal(kc[b, h, :n], cache["k"][b, h, :n]), (b, h)


def test_chunked_prefill_long_tile_list():
    """bf16 D = 128 prefill segment over a decode cache of 4096 chunks of
    capacity: the segment's key-tile list (the cache's chunks + its own) no
    longer fits the fast softmax kernel's 4096-entry LDS list, so the launch
    takes the generic kernel, which reads the chunk list from global memory.
    Outputs match the oracle and the one-shot prefill to the bf16 tolerance,
    routes and final state match the one-shot prefill bit for bit."""
    B, H, L, L1, D = 1, 2, 576, 320, 128
    cap = 4096 * 64
    wl, inp = small_case("bf16", B=B, H=H, L=L, D=D, seed=79, sm_frac=0.5)
    d = wl.d
    say(f"[chunked prefill, long tile list] cap={cap}")
    seg = lambda a, lo, hi: {k: ((val[:, lo:hi] if k == "x" else val[:, :, lo:hi])
                                 if k in ("x", "q", "k", "v", "alpha", "beta") else val) for k, val in a.items()}
    s1, s2 = seg(inp, 0, L1), seg(inp, L1, L)
    full = run_forward(inp, d, B, H, L, D)
    f1 = run_forward(s1, d, B, H, L1, D)
    st = N.DecodeState(B, H, D, d, cap, io=torch.bfloat16)
    t1 = prefill_tensors(s1)
    N.decode_handoff(N.dims(B, H, L1, D, d, io_code(inp)), f1.route, t1["k"], t1["v"], f1.S_final, st)
    dm2 = N.dims(B, H, L - L1, D, d, io_code(inp))
    f2 = N.Forward(dm2, debug=True, want_state=True)
    t2 = prefill_tensors(s2)
    f2(t2["x"], t2["q"], t2["k"], t2["v"], t2["alpha"], t2["beta"], t2["w_score"], t2["w_mix"],
       b_score=t2["b_score"], g_sm=t2["g_sm"], g_lin=t2["g_lin"], prefix=st)
    torch.cuda.synchronize()
    assert int(st.err.item()) == 0
    assert torch.equal(f2.route, full.route[:, :, L1 // 64:])
    assert torch.equal(f2.S_final, full.S_final)
    ref = O.forward(inp["x"], inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["w_score"],
                    inp["w_mix"], inp["b_score"], inp["g_sm"], inp["g_lin"])
    e = maxerr(host(f2.out), ref["out"][:, :, L1:])
    e_full = maxerr(host(f2.out), host(full.out)[:, :, L1:])
    say(f"  segment out err vs oracle {e:.3e}, vs one-shot {e_full:.3e}")
    assert e <= TOL_BF16 and e_full <= TOL_BF16


@pytest.mark.parametrize("io,D,per_head", [("f32", 64, False), ("bf16", 128, False), ("bf16", 128, True)])
def test_chunked_prefill_equals_one_shot(io, D, per_head):
    """Chunked prefill: forward over the first 320 tokens, handoff, forward
    over the remaining 256 tokens on top of that cache (prefix), handoff with
    append.  The queries see the same keys in the same chunk order and the
    state is carried exactly, so the second segment's outputs, routes and
    final state, and the final cache, are bit-identical to one prefill over
    all 576 tokens and its handoff (and the outputs match the oracle)."""
    B, H, L, L1 = 2, 4, 576, 320
    G = H if per_head else 1
    wl, inp = small_case(io, B=B, H=H, L=L, D=D, seed=73, sm_frac=0.5)
    d = wl.d
    say(f"[chunked prefill] io={io} D={D} G={G}")
    r = None
    if per_head:
        rng = np.random.default_rng(73)
        r = (rng.random((B, G, L // 64)) < 0.5).astype(np.int32)
    seg = lambda a, lo, hi: {k: ((val[:, lo:hi] if k == "x" else val[:, :, lo:hi])
                                 if k in ("x", "q", "k", "v", "alpha", "beta") else val) for k, val in a.items()}
    s1, s2 = seg(inp, 0, L1), seg(inp, L1, L)
    cap = L + 64
    io_t = torch.bfloat16 if io == "bf16" else torch.float32
    full = run_forward(inp, d, B, H, L, D, route_override=r, groups=G)
    st_full = N.DecodeState(B, H, D, d, cap, groups=G, io=io_t)
    t_full = prefill_tensors(inp)
    N.decode_handoff(N.dims(B, H, L, D, d, io_code(inp), groups=G), full.route, t_full["k"], t_full["v"],
                     full.S_final, st_full)
    f1 = run_forward(s1, d, B, H, L1, D, route_override=None if r is None else r[:, :, :L1 // 64], groups=G)
    st = N.DecodeState(B, H, D, d, cap, groups=G, io=io_t)
    t1 = prefill_tensors(s1)
    N.decode_handoff(N.dims(B, H, L1, D, d, io_code(inp), groups=G), f1.route, t1["k"], t1["v"], f1.S_final, st)
    dm2 = N.dims(B, H, L - L1, D, d, io_code(inp), groups=G)
    f2 = N.Forward(dm2, debug=True, want_state=True)
    t2 = prefill_tensors(s2)
    ro2 = None if r is None else dev(np.ascontiguousarray(r[:, :, L1 // 64:]))
    f2(t2["x"] if r is None else None, t2["q"], t2["k"], t2["v"], t2["alpha"], t2["beta"],
       t2["w_score"] if r is None else None, t2["w_mix"], b_score=t2["b_score"] if r is None else None,
       g_sm=t2["g_sm"], g_lin=t2["g_lin"], route_override=ro2, prefix=st)
    N.decode_handoff(dm2, f2.route, t2["k"], t2["v"], f2.S_final, st, append=True)
    torch.cuda.synchronize()
    assert torch.equal(f2.route, full.route[:, :, L1 // 64:])
    assert torch.equal(f2.out, full.out[:, :, L1:]), "segment outputs differ from the one-shot prefill"
    assert torch.equal(f2.S_final, full.S_final)
    assert torch.equal(st.n_committed, st_full.n_committed)
    assert int(st.err.item()) == 0 and int(st_full.err.item()) == 0
    assert not st.n_open.any() and torch.equal(st.S_carry, st_full.S_carry)
    nco = st.n_committed.cpu().numpy()
    for b in range(B):
        for h in range(H):
            n = int(nco[b, h if G > 1 else 0])
            assert torch.equal(st.k[b, h, :n], st_full.k[b, h, :n]) and torch.equal(st.v[b, h, :n], st_full.v[b, h, :n])
    if per_head:
        ref = O.forward(None, inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], None, inp["w_mix"],
                        route_override=r, g_sm=inp["g_sm"], g_lin=inp["g_lin"], groups=G)
    else:
        ref = O.forward(inp["x"], inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["w_score"],
                        inp["w_mix"], inp["b_score"], inp["g_sm"], inp["g_lin"])
    e = maxerr(host(f2.out), ref["out"][:, :, L1:])
    e1 = maxerr(host(f1.out), ref["out"][:, :, :L1])
    say(f"  segment out err vs oracle {e:.3e}, first segment {e1:.3e}")
    assert max(e, e1) <= (TOL_F32 if io == "f32" else TOL_BF16)


def test_decode_full_sampled():
    """The decode workload at full size (B=64, ~8192 cached rows per head),
    one step; sampled sequences against the oracle."""
    wl = W.WORKLOADS["decode"]
    cache, new = W.make_decode(wl)
    B, H, D, d = wl.B, wl.H, wl.D, wl.d
    say(f"[decode] full B={B} cap={cache['k'].shape[2]}")
    st = load_state(cache, B, H, D, d, "bf16")
    dm = N.dims(B, H, 1, D, d, N.BF16)
    dec = N.Decode(dm, st, debug=True)
    args = [dev(new["x"], "bf16"), dev(new["q"], "bf16"), dev(new["k"], "bf16"), dev(new["v"], "bf16"),
            dev(new["alpha"]), dev(new["beta"]), dev(new["w_score"]), dev(new["w_mix"])]
    dec(*args)
    torch.cuda.synchronize()
    for b in (0, 17, 63):
        sub = dict(k=W.bits_to_f32(cache["k"][b:b + 1]), v=W.bits_to_f32(cache["v"][b:b + 1]),
                   n_committed=cache["n_committed"][b:b + 1], n_open=cache["n_open"][b:b + 1],
                   S_carry=cache["S_carry"][b:b + 1], S_work=cache["S_work"][b:b + 1],
                   x_sum=cache["x_sum"][b:b + 1], err=0)
        out_ref, br, _ = O.decode_step(sub, new["x"][b:b + 1], new["q"][b:b + 1], new["k"][b:b + 1],
                                       new["v"][b:b + 1], new["alpha"][b:b + 1], new["beta"][b:b + 1],
                                       new["w_score"], new["w_mix"])
        e = max(maxerr(host(dec.out[b:b + 1]), out_ref), maxerr(rmsn(host(dec.o_sm[b:b + 1])), br["n_sm"]),
                maxerr(rmsn(host(dec.o_gdn[b:b + 1])), br["n_lin"]))
        say(f"  b={b} err {e:.3e}")
        assert e <= TOL_BF16
    n = int(cache["n_committed"][0, 0])
    assert torch.equal(st.k[0, :, n], args[2][0])
    assert (st.n_open.cpu().numpy() == 1).all()


def test_decode_capacity_flag():
    """A full cache sets err_flag and writes nothing past its end."""
    B, H, D, d, cap = 1, 2, 64, 64, 128
    st = N.DecodeState(B, H, D, d, cap, io=torch.float32)
    st.n_committed.fill_(128)
    dm = N.dims(B, H, 1, D, d, N.F32)
    dec = N.Decode(dm, st)
    rng = np.random.default_rng(0)
    mk = lambda *s: dev(rng.standard_normal(s).astype(np.float32))
    dec(mk(B, d), mk(B, H, D), mk(B, H, D), mk(B, H, D), dev(np.full((B, H), 0.9, np.float32)),
        dev(np.full((B, H), 0.5, np.float32)), mk(d, 2), mk(D, 2))
    torch.cuda.synchronize()
    assert int(st.err.item()) == 1
    assert torch.isfinite(dec.out).all()
