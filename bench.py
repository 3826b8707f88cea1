"""Benchmark of the NAtS-L hybrid layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long] [--no-cpu] [--no-decode]

A step is one full prefill forward of the layer (router + compaction, Gated
DeltaNet branch, softmax branch, merge) over the "long" workload
(B=1, H=16, L=32768, D=128, d_model=2048, bf16, 25% softmax chunks in 3
bursts + 32 singles).  Inputs are resident in HBM before timing starts; W
untimed warm-up steps, then K timed steps between device synchronisations.

The decode step (B=64, H=16, ~8192 cached rows per head) is measured in the
same run and reported under "decode".

roofline: the dominant kernel of each phase, timed live with HIP events that
the library records around its own launches (on the stream each kernel runs
on) during the timed region:
  prefill  softmax_masked, MFMA-bound: algorithmic FLOPs 4*D*(visible pairs)
           of the realised routes / average launch time, against 2.5 PFLOP/s
           dense bf16;
  decode   decode_attn, HBM-bound: the cached K/V bytes it must read / average
           launch time, against 8 TB/s.
cpu_baseline: the fp64 oracle on a bounded sample (one head: router on all
chunks, Gated DeltaNet on all tokens, softmax on every 2nd query block), the
per-head time scaled to all heads.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_FP32_VALU_TFLOPS = 157.3  # MI355X fp32 vector


def sm_pairs(route_bgc, H, chunk=64):
    """Visible (query, key) pairs of the softmax branch for realised routes:
    every query sees the earlier softmax chunks in full and its own chunk
    causally."""
    r = np.asarray(route_bgc)
    B, G, nc = r.shape
    total = 0
    for b in range(B):
        for g in range(G):
            is_sm = (r[b, g] == 0).astype(np.int64)
            nsb = np.concatenate([[0], np.cumsum(is_sm)[:-1]])
            per_head = int((chunk * chunk * nsb).sum()) + nc * chunk * (chunk + 1) // 2
            total += per_head * (H // G)
    return total


def gdn_flops(B, H, nc, n_lin, D, chunk=64):
    """Chunkwise Gated DeltaNet work: per chunk-head 10 C^2 D + 4 C D^2, plus
    2 C D^2 for every committed (linear) chunk (the C^3 solve is excluded)."""
    return B * H * (nc * (10 * chunk * chunk * D + 4 * chunk * D * D)) + H * n_lin * 2 * chunk * D * D


def source_hash(*names):
    """Hash of the kernel sources and of the compiler flags they are built with."""
    from linear_attention_natsl_amd import build as B
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "linear_attention_natsl_amd", "csrc", n), "rb") as f:
            h.update(f.read())
        h.update(" ".join(B.FLAGS[:-1] + B.FILE_FLAGS.get(n, [])).encode())
    return h.hexdigest()[:16]


def counters_traffic(kernel, workload, src_hash, launches_bytes_hint=None):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when it is missing or the kernel source changed since."""
    p = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_counters.txt")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        c = json.load(f)
    if c.get("source_hash") != src_hash:
        return None
    return c.get("hbm_bytes_per_launch")


SETTLE_S = 0.3


def settle(fn, seconds=SETTLE_S):
    """Runs fn untimed for `seconds`: the GPU's clocks take tens of milliseconds
    of sustained load to leave their idle state (the first forward steps of a
    cold GPU run up to 30% slower), and the timed steps should see the steady
    state a serving or training loop sees."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(5):
            fn()
        torch.cuda.synchronize()


def kernel_table(N, fn, names, reps):
    """Average duration of every kernel of a step, from `reps` untimed steps
    with each kernel bracketed by events (the timed steps bracket only the
    roofline kernel, so that the events do not lengthen the step)."""
    import torch
    N.profile_select(None)
    N.profile_reset()
    for _ in range(reps):
        fn()
    torch.cuda.synchronize()
    out = {}
    for name in names:
        n, ms = N.profile_read(name)
        out[name] = dict(launches=n, avg_us=round(1000.0 * ms / max(n, 1), 2))
    return out


def time_softmax_alone(N, dm, route, t, io_t, reps):
    """Average duration of the softmax branch's launch on the forward's
    compaction of `route`, with nothing else on the GPU: events around `reps`
    back-to-back launches after a settle."""
    import torch
    _, sel, nsb, _ = N.route(dm, None, None, route_in=route)
    call = lambda: N.softmax_masked(dm, t["q"], t["k"], t["v"], sel, nsb, o_dtype=io_t)
    settle(call)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        call()
    e1.record()
    torch.cuda.synchronize()
    return 1000.0 * e0.elapsed_time(e1) / reps


def time_route_alone(N, dm, t, wl, reps=50):
    """The router + compaction on the prefill's x with the GPU to itself: one
    pass over x (B L d_model values) per launch, set against the HBM peak."""
    import torch
    call = lambda: N.route(dm, t["x"], t["w_score"], t["b_score"])
    settle(call, 0.1)
    N.profile_enable(True)
    N.profile_select(None)
    N.profile_reset()
    for _ in range(reps):
        call()
    torch.cuda.synchronize()
    n, ms = N.profile_read("route")
    nc, mc = N.profile_read("compact")
    N.profile_enable(False)
    us = 1000.0 * ms / max(n, 1)
    nbytes = wl.B * wl.L * wl.d * t["x"].element_size()
    gbs = nbytes / (us * 1e-6) / 1e9
    return dict(avg_us=round(us, 2), compact_avg_us=round(1000.0 * mc / max(nc, 1), 2), bytes=nbytes,
                gbs=round(gbs, 1), frac_hbm=round(gbs / PEAK_HBM_GBS, 4))


def time_handoff(N, dm, route, t, wl, reps=20):
    """The prefill -> decode handoff of this prefill (its routes, K and V) into
    a decode cache sized for its softmax rows: bytes moved = the softmax
    chunks' K/V rows read and written + S_final read + S_carry, S_work
    written; timed with events around the whole call."""
    import torch
    dev = t["k"].device
    nsm = int((route == 0).sum(dim=2).max().item()) * 64
    cap = nsm + 64
    st = N.DecodeState(wl.B, wl.H, wl.D, wl.d, cap, groups=dm.route_groups, io=t["k"].dtype, device=dev)
    S_final = torch.zeros(wl.B, wl.H, wl.D, wl.D, dtype=torch.float32, device=dev)
    for _ in range(3):
        N.decode_handoff(dm, route, t["k"], t["v"], S_final, st)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        N.decode_handoff(dm, route, t["k"], t["v"], S_final, st)
    e1.record()
    torch.cuda.synchronize()
    us = 1000.0 * e0.elapsed_time(e1) / reps
    rows = int((route == 0).sum().item()) * 64 * (wl.H // dm.route_groups)
    nbytes = 2 * 2 * rows * wl.D * t["k"].element_size() + 3 * wl.B * wl.H * wl.D * wl.D * 4
    return dict(workload=f"handoff of the {wl.name} prefill: {rows} softmax rows of K and V, cache capacity {cap}",
                us=round(us, 2), bytes=nbytes, gbs=round(nbytes / (us * 1e-6) / 1e9, 1),
                frac_hbm=round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4))


def time_softmax_backward(N, dm, t, wl, pairs, reps=3):
    """Gradient of the softmax branch on this workload (dq, dk, dv from the
    forward's o and lse and a random upstream gradient), timed with events;
    algorithmic work 10 D FLOP per visible pair (recomputed scores, dP, dQ,
    dK, dV; the kernels recompute scores and dP twice, 14 D)."""
    import torch
    _, sel, nsb, _ = N.route(dm, t["x"], t["w_score"], t["b_score"])
    o, lse = N.softmax_masked(dm, t["q"], t["k"], t["v"], sel, nsb, o_dtype=t["q"].dtype, want_lse=True)
    d_o = torch.randn_like(t["q"])
    for _ in range(2):
        N.softmax_masked_backward(dm, t["q"], t["k"], t["v"], sel, nsb, o, lse, d_o)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        N.softmax_masked_backward(dm, t["q"], t["k"], t["v"], sel, nsb, o, lse, d_o)
    e1.record()
    torch.cuda.synchronize()
    us = 1000.0 * e0.elapsed_time(e1) / reps
    flops = 10 * wl.D * pairs
    tf = flops / (us * 1e-6) / 1e12
    return dict(workload=f"gradient of the softmax branch on the {wl.name} prefill", us=round(us, 1),
                flops=flops, tflops=round(tf, 1), frac_mfma=round(tf / PEAK_BF16_TFLOPS, 4))


def time_route_gradient(N, dm, t, wl, reps=3):
    """The router's gradient on this workload (straight-through reading): the
    softmax branch's gradient with and without its gate derivatives (with
    them every linear-routed key chunk also visits all later query chunks:
    full causal attention work for the scores and dP), the Gated DeltaNet
    gradient's gate partials, and natsl_route_backward (one pass over x plus
    the score layer), each timed with events."""
    import torch
    r, sel, nsb, scores = N.route(dm, t["x"], t["w_score"], t["b_score"])
    o, lse = N.softmax_masked(dm, t["q"], t["k"], t["v"], sel, nsb, o_dtype=t["q"].dtype, want_lse=True)
    d_o = torch.randn_like(t["q"])
    dg = torch.randn(wl.B, wl.H, wl.nc, dtype=torch.float32, device=t["q"].device)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return round(1000.0 * e0.elapsed_time(e1) / reps, 1)
    sm = timed(lambda: N.softmax_masked_backward(dm, t["q"], t["k"], t["v"], sel, nsb, o, lse, d_o))
    sm_g = timed(lambda: N.softmax_masked_backward(dm, t["q"], t["k"], t["v"], sel, nsb, o, lse, d_o, want_gate=True))
    rb = timed(lambda: N.route_backward(dm, t["x"], t["w_score"], scores, dg, dg))
    pairs_all = wl.B * wl.H * (wl.nc * (wl.nc - 1) // 2) * 64 * 64
    return dict(workload=f"router gradient on the {wl.name} prefill (straight-through)",
                softmax_backward_us=sm, softmax_backward_with_gate_us=sm_g, route_backward_us=rb,
                gate_pairs=pairs_all,
                note="the softmax gate needs p~ and dP for every (later query, key) pair: 4 D FLOPs per pair on the "
                     "matrix cores for the pairs the forward skipped")


def time_gdn_backward(N, dm, t, wl, route, reps=3):
    """Gradient of the Gated DeltaNet branch on this workload (a random fp32
    upstream gradient on o_gdn), timed with events.  Chunk form on the matrix
    cores; its matrix products per chunk-head (C = 64 tokens) are 36 C^2 D +
    16 C D^2 + 4 C^3 FLOP: the forward prep (K K^T, Q K^T, U~, W), the state
    scan (W S, K~^T U), the backward prep (K K^T, Q K^T, W), the reverse scan
    (K Gc, P^T dO, Q^T dO, W^T dU) and the chunk gradients (A, P, dP, dO S0^T,
    U Gc^T, TdU S0^T, T^T dU, A U, dT, T^T dT T^T, E K, E^T K, F K, F^T Q).
    Two of its five launches are sequential over the 512 chunks, so it is
    latency-bound, not set against a roofline.  Timed in both workspace
    layouts: the default (one region shared by the two sweeps, run one after
    the other) and the overlapping one (the sweeps at the same time on two
    streams)."""
    import torch
    d_o = torch.randn(t["q"].shape, dtype=torch.float32, device=t["q"].device)

    def timed(overlap):
        N.gdn_backward(dm, t["q"], t["k"], t["v"], t["alpha"], t["beta"], route, d_o, overlap=overlap)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            N.gdn_backward(dm, t["q"], t["k"], t["v"], t["alpha"], t["beta"], route, d_o, overlap=overlap)
        e1.record()
        torch.cuda.synchronize()
        return 1000.0 * e0.elapsed_time(e1) / reps

    us, us_ov = timed(False), timed(True)
    C, D = 64, wl.D
    flops = (36 * C * C * D + 16 * C * D * D + 4 * C ** 3) * wl.B * wl.H * (wl.L // C)
    tf = flops / (us * 1e-6) / 1e12
    ws = N.workspace_size(N.ENTRY_GDN_BACKWARD, dm)
    ws_ov = N.workspace_size(N.ENTRY_GDN_BACKWARD_OVERLAP, dm)
    return dict(workload=f"gradient of the Gated DeltaNet branch on the {wl.name} prefill (chunk form)",
                us=round(us, 1), flops=flops, tflops=round(tf, 1), frac_bf16_mfma=round(tf / PEAK_BF16_TFLOPS, 4),
                workspace_bytes=int(ws), note="latency-bound: two sequential sweeps over the chunks",
                overlap=dict(us=round(us_ov, 1), workspace_bytes=int(ws_ov),
                             note="the same gradient with the larger workspace layout: the state scan and the "
                                  "reverse scan at the same time on two streams (bit-identical results)"))


def time_merge_backward(N, dm, t, wl, reps=5):
    """Gradient of the merge on this workload (random bf16 branch outputs, a
    random fp32 upstream gradient), timed with events; HBM-bound: it reads q,
    both branch outputs and d_out and writes three fp32 gradients."""
    import torch
    shp = t["q"].shape
    o_sm = torch.randn(shp, dtype=torch.bfloat16, device=t["q"].device)
    o_gdn = torch.randn_like(o_sm)
    d_out = torch.randn(shp, dtype=torch.float32, device=t["q"].device)
    call = lambda: N.merge_backward(dm, t["q"], o_sm, o_gdn, t["w_mix"], d_out)
    call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        call()
    e1.record()
    torch.cuda.synchronize()
    us = 1000.0 * e0.elapsed_time(e1) / reps
    n = int(np.prod(shp))
    nbytes = n * (2 + 2 + 2 + 4) + 3 * n * 4
    return dict(workload=f"gradient of the merge on the {wl.name} prefill", us=round(us, 1), bytes=nbytes,
                gbs=round(nbytes / (us * 1e-6) / 1e9, 1), frac_hbm=round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4))


class Flusher:
    """Writes a 512 MiB scratch buffer: evicts the L2 of every XCD and the
    256 MB MALL, so that a step timed after it reads its inputs from HBM."""

    def __init__(self, device, mib=512):
        import torch
        self.buf = torch.empty(mib * 2 ** 20 // 4, dtype=torch.float32, device=device)

    def __call__(self):
        self.buf.fill_(1.0)


def evented_steps(call, n, flush=None, setup=None):
    """n steps, each bracketed by its own pair of HIP events on the current
    stream (the forward joins its helper stream back into it), with `setup`
    (state restore) and `flush` run between steps, outside the events.
    Returns mean, median and minimum per-step milliseconds."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in evs:
        if setup:
            setup()
        if flush:
            flush()
        a.record()
        call()
        b.record()
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in evs])
    return dict(n=n, flushed_between_steps=flush is not None, mean_ms=round(float(ms.mean()), 4),
                median_ms=round(float(np.median(ms)), 4), min_ms=round(float(ms.min()), 4))


def prefill_inputs(N, W, name, dev):
    import torch
    wl = W.WORKLOADS[name]
    inp = W.make_prefill(wl)
    io_t = torch.bfloat16 if inp["io"] == "bf16" else torch.float32
    t = {k: torch.from_numpy(np.ascontiguousarray(inp[k])).to(dev).to(io_t) for k in ("x", "q", "k", "v")}
    for k in ("alpha", "beta", "w_score", "w_mix", "b_score", "g_sm", "g_lin"):
        t[k] = torch.from_numpy(np.ascontiguousarray(inp[k])).to(dev)
    dm = N.dims(wl.B, wl.H, wl.L, wl.D, wl.d, N.BF16 if inp["io"] == "bf16" else N.F32)
    return wl, inp, t, dm, io_t


def run_prefill_case(args, N, W, wl, inp, t, dm, route_kind=None, steps=None, warmup=None, flusher=None):
    """Times one prefill workload: `steps` back-to-back forward steps between
    device synchronisations (the whole-job clock), the softmax kernel's
    average launch from HIP events the library records around it during
    those steps, then per-step events with L2 + MALL flushed between steps
    (median / min), and a per-kernel table from extra untimed steps.
    route_kind "sm" / "lin" forces every chunk to softmax / linear through
    route_override (the router is skipped, as the workload prescribes)."""
    import torch
    steps = args.steps if steps is None else steps
    warmup = args.warmup if warmup is None else warmup
    fwd = N.Forward(dm, device=t["q"].device)
    ro = None
    if route_kind:
        ro = torch.from_numpy(W.forced_routes(wl.B, wl.nc, route_kind)).to(t["q"].device)
        call = lambda: fwd(None, t["q"], t["k"], t["v"], t["alpha"], t["beta"], None, t["w_mix"],
                           g_sm=t["g_sm"], g_lin=t["g_lin"], route_override=ro)
    else:
        call = lambda: fwd(t["x"], t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["w_score"], t["w_mix"],
                           b_score=t["b_score"], g_sm=t["g_sm"], g_lin=t["g_lin"])
    settle(call)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    # timed steps: only the roofline kernel is bracketed by events
    N.profile_enable(True)
    N.profile_select("softmax_masked")
    N.profile_reset()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    n, ms = N.profile_read("softmax_masked")
    sm_avg_us = 1000.0 * ms / max(n, 1)
    N.profile_enable(False)
    per_step = evented_steps(call, max(10, steps), flush=flusher)
    warm_steps = evented_steps(call, max(10, steps))
    N.profile_enable(True)
    kernels = kernel_table(N, call, ("route", "compact", "gdn_prep", "gdn_scan", "softmax_masked", "merge"),
                           max(5, steps // 5))
    N.profile_enable(False)
    route = fwd.route.cpu().numpy()
    pairs = sm_pairs(route, wl.H)
    f_sm = 4 * wl.D * pairs
    n_lin = int((route == 1).sum())
    f_gdn = gdn_flops(wl.B, wl.H, wl.nc, n_lin, wl.D)
    step_s = dt / steps
    return dict(fwd=fwd, call=call, route=route, dt=dt, step_s=step_s, sm_avg_us=sm_avg_us, f_sm=f_sm, f_gdn=f_gdn,
                pairs=pairs, kernels=kernels, per_step=per_step, warm_steps=warm_steps)


def layer_bytes(wl, io_bytes, with_x):
    """Algorithmic HBM bytes of one forward: x (router) + q, k, v + alpha,
    beta + out, weights negligible."""
    n = wl.B * wl.H * wl.L
    return (wl.B * wl.L * wl.d * io_bytes if with_x else 0) + 4 * n * wl.D * io_bytes + 2 * n * 4


def time_prefill(args, N, W):
    """The headline prefill (the long workload) with its extras."""
    import torch
    dev = torch.device("cuda:0")
    wl, inp, t, dm, io_t = prefill_inputs(N, W, args.workload, dev)
    flusher = Flusher(dev)
    r = run_prefill_case(args, N, W, wl, inp, t, dm, flusher=flusher)
    fwd = r["fwd"]
    sm_alone_us = None if args.no_alone else time_softmax_alone(N, dm, fwd.route, t, io_t, max(10, args.steps // 2))
    route_alone = None if args.no_alone else time_route_alone(N, dm, t, wl)
    extras = {}
    if not args.no_extras:
        extras = dict(handoff=time_handoff(N, dm, fwd.route, t, wl),
                      softmax_backward=time_softmax_backward(N, dm, t, wl, r["pairs"]),
                      gdn_backward=time_gdn_backward(N, dm, t, wl, fwd.route),
                      merge_backward=time_merge_backward(N, dm, t, wl),
                      route_gradient=time_route_gradient(N, dm, t, wl))
    route = r["route"]

    f_sm, f_gdn, step_s = r["f_sm"], r["f_gdn"], r["step_s"]
    sm_us = round(r["sm_avg_us"], 2)
    achieved = f_sm / (sm_us * 1e-6) / 1e12
    traffic = counters_traffic("softmax_masked", args.workload, source_hash("softmax_masked.hip", "common.hpp"))
    res = dict(
        metric="hybrid-layer prefill tokens/sec + % bf16 MFMA peak; decode-step % HBM peak",
        value=round(wl.B * wl.L / step_s, 1), unit="tokens/s", n_gpus=1, steps=args.steps, warmup=args.warmup,
        ms_per_step=round(1000.0 * step_s, 4), higher_is_better=True, scaling="weak", vs_baseline=None,
        dtype="bf16" if inp["io"] == "bf16" else "f32", data="synthetic",
        config=dict(workload=f"{args.workload} prefill: B={wl.B} H={wl.H} L={wl.L} D={wl.D} d_model={wl.d}, "
                    f"chunk 64, {inp['io']} io and branch outputs / fp32 accumulate",
                    B=wl.B, H=wl.H, L=wl.L, D=wl.D, d_model=wl.d, seed=wl.seed,
                    softmax_chunk_fraction=round(float((route == 0).mean()), 4),
                    route_check="bit-exact against the oracle router at this size in "
                                "tests/test_gpu_parity.py::test_route_full_size_bitexact",
                    parallelism="single GPU"),
        roofline=dict(bound="mfma", kernel="softmax_masked", achieved=round(achieved, 1), peak=PEAK_BF16_TFLOPS,
                      unit="TFLOP/s", frac=round(achieved / PEAK_BF16_TFLOPS, 4), traffic=traffic,
                      flops_per_launch=f_sm, avg_launch_us=sm_us,
                      alone=None if sm_alone_us is None else dict(
                          avg_launch_us=round(sm_alone_us, 2), achieved=round(f_sm / (sm_alone_us * 1e-6) / 1e12, 1),
                          frac=round(f_sm / (sm_alone_us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4),
                          note="the same launch with the GPU to itself (in the forward it shares the GPU with the "
                               "Gated DeltaNet prep and scan)")),
        layer=dict(flops_softmax=f_sm, flops_gdn=f_gdn,
                   layer_tflops=round((f_sm + f_gdn) / step_s / 1e12, 1),
                   layer_frac_of_mfma_peak=round((f_sm + f_gdn) / step_s / 1e12 / PEAK_BF16_TFLOPS, 4),
                   step_stats=dict(flushed=r["per_step"], back_to_back=r["warm_steps"]),
                   kernels=r["kernels"], route_alone=route_alone),
        critical_path=dict(
            gdn_prep_plus_scan_us=round(r["kernels"]["gdn_prep"]["avg_us"] + r["kernels"]["gdn_scan"]["avg_us"], 1),
            softmax_us=sm_us, step_us=round(1e6 * step_s, 1),
            note=f"the branches run on two streams and the merge follows both: the step is bounded by the longer of "
                 f"the Gated DeltaNet chain (the prep, then {wl.nc} dependent scan steps per (b, h)) and the softmax "
                 f"launch, each measured while sharing the GPU with the other"),
        **extras,
    )
    return res, inp, route


def time_prefill_config(args, N, W, name, route_kind=None):
    """A prefill workload other than the headline one, as a sub-record:
    tokens/s and its own roofline.  Mixed and all-softmax routes: the softmax
    kernel against the bf16 MFMA peak, plus the layer's (F_sm + F_gdn) / t.
    All-linear routes: the layer is HBM- and scan-bound (the scan takes Nc
    dependent chunk steps), so the Gated DeltaNet chain (prep + scan, one
    stream) is set against the HBM peak with the branch's algorithmic bytes
    (q, k, v, alpha, beta in, its output out), and the per-chunk-step
    latency of the scan is reported."""
    import torch
    dev = torch.device("cuda:0")
    wl, inp, t, dm, io_t = prefill_inputs(N, W, name, dev)
    steps = max(10, args.steps)
    r = run_prefill_case(args, N, W, wl, inp, t, dm, route_kind=route_kind, steps=steps, flusher=Flusher(dev))
    step_s = r["step_s"]
    io_b = 2 if inp["io"] == "bf16" else 4
    k = r["kernels"]
    out = dict(
        workload=f"{name} prefill: B={wl.B} H={wl.H} L={wl.L} D={wl.D} d_model={wl.d}, "
                 + (f"routes forced all-{'softmax' if route_kind == 'sm' else 'linear'}" if route_kind
                    else f"natural routes, seed {wl.seed}"),
        value=round(wl.B * wl.L / step_s, 1), unit="tokens/s", steps=steps, ms_per_step=round(1000 * step_s, 4),
        softmax_chunk_fraction=round(float((r["route"] == 0).mean()), 4),
        layer=dict(flops_softmax=r["f_sm"], flops_gdn=r["f_gdn"],
                   layer_frac_of_mfma_peak=round((r["f_sm"] + r["f_gdn"]) / step_s / 1e12 / PEAK_BF16_TFLOPS, 4),
                   hbm_bytes=layer_bytes(wl, io_b, route_kind is None),
                   layer_frac_of_hbm_peak=round(layer_bytes(wl, io_b, route_kind is None) / step_s / 1e9 / PEAK_HBM_GBS, 4),
                   step_stats=dict(flushed=r["per_step"], back_to_back=r["warm_steps"]), kernels=k))
    if route_kind == "lin":
        n = wl.B * wl.H * wl.L
        branch_bytes = 4 * n * wl.D * io_b + 2 * n * 4
        chain_us = k["gdn_prep"]["avg_us"] + k["gdn_scan"]["avg_us"]
        gbs = branch_bytes / (chain_us * 1e-6) / 1e9
        out["roofline"] = dict(bound="hbm", kernel="gdn_prep+gdn_scan", achieved=round(gbs, 1), peak=PEAK_HBM_GBS,
                               unit="GB/s", frac=round(gbs / PEAK_HBM_GBS, 4),
                               traffic=counters_traffic("gdn_chain", "degen_lin", source_hash("gdn.hip", "common.hpp")),
                               bytes_per_launch=branch_bytes, avg_launch_us=round(chain_us, 2),
                               scan_us_per_chunk_step=round(k["gdn_scan"]["avg_us"] / wl.nc, 3),
                               note=f"the scan is {wl.nc} dependent chunk steps per (b, h)")
    else:
        sm_us = round(r["sm_avg_us"], 2)
        ach = r["f_sm"] / (sm_us * 1e-6) / 1e12
        wl_key = name if route_kind is None else f"{name}_{route_kind}"
        out["roofline"] = dict(bound="mfma", kernel="softmax_masked", achieved=round(ach, 1), peak=PEAK_BF16_TFLOPS,
                               unit="TFLOP/s", frac=round(ach / PEAK_BF16_TFLOPS, 4),
                               traffic=counters_traffic("softmax_masked", wl_key,
                                                        source_hash("softmax_masked.hip", "common.hpp")),
                               flops_per_launch=r["f_sm"], avg_launch_us=sm_us)
        chain_us = k["gdn_prep"]["avg_us"] + k["gdn_scan"]["avg_us"]
        out["critical_path"] = dict(
            gdn_prep_plus_scan_us=round(chain_us, 1), softmax_us=sm_us, step_us=round(1e6 * step_s, 1),
            note=f"the branches run on two streams and the merge follows both: the step is bounded by the longer of "
                 f"the Gated DeltaNet chain (the prep, then {wl.nc} dependent scan steps per (b, h)) and the softmax "
                 f"launch, each measured while sharing the GPU with the other")
    return out, inp, r["route"]


def time_nha(args, N, W, reps=10):
    """Native Hybrid Attention on its workload (the long prefill's shape, 64
    slots, a 2048-token window, bf16): the whole call timed with events, the
    four kernels from the library's events.  Algorithmic work: 4 D FLOPs per
    (query, window key) pair and per (query, slot) pair (scores and read-out,
    as for softmax attention), plus 4 D FLOPs per (token, slot) for the slot
    update (K~ and V~, two multiply-adds each)."""
    import torch
    c = W.NHA
    B, H, L, D, m, w = c["B"], c["H"], c["L"], c["D"], c["slots"], c["window"]
    inp = W.make_nha(B, H, L, D, m, io="bf16", seed=c["seed"])
    dev = torch.device("cuda:0")
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(torch.bfloat16)
    q, k, v = bf(inp["q"]), bf(inp["k"]), bf(inp["v"])
    gate = torch.from_numpy(inp["gate"]).to(dev)
    del inp
    dm = N.dims(B, H, L, D, 64, N.BF16)
    ws = N.workspace(N.nha_workspace_size(dm, m, w), dev)
    call = lambda: N.nha_attention(dm, q, k, v, gate, w, ws=ws)
    settle(call)
    stats = evented_steps(call, reps, flush=Flusher(dev))
    warm = evented_steps(call, reps)
    N.profile_enable(True)
    kernels = kernel_table(N, call, ("nha_window", "nha_chunk", "nha_scan", "nha_slots"), 5)
    N.profile_enable(False)
    pairs_win = B * H * sum(min(t + 1, w) for t in range(L))
    f_win = 4 * D * pairs_win
    nct = L - w if L > w else 0  # queries whose slots are in use
    f_slots = 4 * D * m * B * H * nct          # scores and read-out over the slots
    f_update = 4 * D * m * B * H * L           # slot updates
    med = warm["median_ms"]
    work = {"nha_window": ("mfma", f_win, PEAK_BF16_TFLOPS, "TFLOP/s"),
            "nha_slots": ("alu", f_slots + f_update, PEAK_FP32_VALU_TFLOPS, "TFLOP/s"),
            "nha_chunk": ("alu", 4 * D * m * B * H * L, PEAK_FP32_VALU_TFLOPS, "TFLOP/s"),
            "nha_scan": ("hbm", 2 * 2 * B * H * max(L // 64 - w // 64, 0) * m * D * 4, PEAK_HBM_GBS, "GB/s")}
    dom = max(work, key=lambda n: kernels[n]["avg_us"])
    bound, amount, peak, unit = work[dom]
    us = kernels[dom]["avg_us"]
    ach = amount / (us * 1e-6) / (1e12 if unit == "TFLOP/s" else 1e9)
    rl = dict(bound=bound, kernel=dom, achieved=round(ach, 1), peak=peak, unit=unit, frac=round(ach / peak, 4),
              traffic=None, avg_launch_us=us)
    rl["flops_per_launch" if unit == "TFLOP/s" else "bytes_per_launch"] = amount
    if dom == "nha_window":
        rl["note"] = ("the window's softmax runs on the library's helper stream beside nha_chunk and nha_scan, so "
                      "its launch shares the GPU with them for part of its duration")
    return dict(workload=f"Native Hybrid Attention: B={B} H={H} L={L} D={D}, {m} slots, window {w} tokens, bf16",
                value=round(B * L / (med * 1e-3), 1), unit="tokens/s", ms_per_call_median=med,
                step_stats=dict(flushed=stats, back_to_back=warm),
                flops=dict(window=f_win, slots=f_slots, slot_updates=f_update),
                layer_frac_of_mfma_peak=round((f_win + f_slots + f_update) / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                roofline=rl, kernels=kernels)


def decode_state(N, W, dev, n_open=0):
    """The decode workload's cache on the device (n_open = 0 as generated:
    position 32768 starts a chunk); inputs of the new token."""
    import torch
    wl = W.WORKLOADS["decode"]
    cache, new = W.make_decode(wl)
    B, H, D, d = wl.B, wl.H, wl.D, wl.d
    cap = cache["k"].shape[2]
    st = N.DecodeState(B, H, D, d, cap, io=torch.bfloat16, device=dev)
    bits = lambda u: torch.from_numpy(np.ascontiguousarray(u).view(np.int16)).to(dev).view(torch.bfloat16)
    st.k.copy_(bits(cache["k"]))
    st.v.copy_(bits(cache["v"]))
    st.n_committed.copy_(torch.from_numpy(cache["n_committed"].astype(np.int32)).to(dev))
    st.n_open.copy_(torch.from_numpy(cache["n_open"][:, 0].astype(np.int32)).to(dev))
    st.S_carry.copy_(torch.from_numpy(cache["S_carry"]).to(dev))
    st.S_work.copy_(torch.from_numpy(cache["S_work"]).to(dev))
    del cache
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(torch.bfloat16)
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    a = [bf(new["x"]), bf(new["q"]), bf(new["k"]), bf(new["v"]), f32(new["alpha"]), f32(new["beta"]),
         f32(new["w_score"]), f32(new["w_mix"])]
    return wl, st, a


def decode_step_bytes(wl, rows_mean, completing_lin=0):
    """Algorithmic bytes of one decode step: the cached K/V rows read, the new
    K/V row written, the state read (S_carry or S_work) and S_work written,
    q/k/v/out of the new token, x and the fp32 x_sum read and written (and, for
    a chunk that commits its state, S_carry written)."""
    B, H, D, d = wl.B, wl.H, wl.D, wl.d
    kv = B * H * rows_mean * 2 * D * 2
    return kv, kv + B * H * (2 * D * 2 + 2 * D * D * 4 + 4 * D * 2) + B * d * (2 + 8) + completing_lin * D * D * 4


def time_decode(args, N, W, wl_state=None):
    """The decode workload: steps back to back from n_open = 0 (a decode of
    `decode_steps` tokens; none completes a chunk), the decode_attn kernel's
    average launch from the library's HIP events."""
    import torch
    dev = torch.device("cuda:0")
    wl, st, a = wl_state if wl_state else decode_state(N, W, dev)
    B, H, D, d = wl.B, wl.H, wl.D, wl.d
    dm = N.dims(B, H, 1, D, d, N.BF16)
    dec = N.Decode(dm, st, device=dev)
    rows0 = (st.n_committed[:, 0] + st.n_open).cpu().numpy().astype(np.int64)
    steps, warm = args.decode_steps, 3
    # settle the clocks with bursts of steps, each followed by a restore of the
    # counters and states (the cache rows the burst appended are rewritten by
    # the timed steps), so the cache never grows past its capacity
    saved = [x.clone() for x in (st.n_committed, st.n_open, st.S_carry, st.S_work, st.x_sum, st.err)]

    def restore():
        for x, y in zip((st.n_committed, st.n_open, st.S_carry, st.S_work, st.x_sum, st.err), saved):
            x.copy_(y)

    def burst():
        for _ in range(32):
            dec(*a)
        restore()
    settle(burst)
    for _ in range(warm):
        dec(*a)
    torch.cuda.synchronize()
    rows_start = (st.n_committed[:, 0] + st.n_open).cpu().numpy().astype(np.int64)
    N.profile_enable(True)
    N.profile_select("decode_attn")
    N.profile_reset()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        dec(*a)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    n, ms = N.profile_read("decode_attn")
    attn_us = round(1000.0 * ms / max(n, 1), 2)
    assert int(st.err.item()) == 0
    kernels = kernel_table(N, lambda: dec(*a), ("decode_route", "decode_gdn", "decode_attn", "decode_combine",
                                                "decode_commit"), 10)
    N.profile_enable(False)
    assert int(st.err.item()) == 0
    restore()
    # rows read per step: step i reads rows_start + i cached rows per (b, h)
    mean_rows = float((rows_start[:, None] + np.arange(steps)[None, :]).mean())
    kv_bytes, step_bytes = decode_step_bytes(wl, mean_rows)
    achieved = kv_bytes / (attn_us * 1e-6) / 1e9
    traffic = counters_traffic("decode_attn", "decode", source_hash("decode.hip", "common.hpp"))
    # per-step events, the state restored and the caches flushed between steps
    flushed = evented_steps(lambda: dec(*a), 30, flush=Flusher(dev), setup=restore)
    restore()
    torch.cuda.synchronize()
    return dict(
        workload=f"decode: B={B} H={H} D={D} d_model={d}, ~{rows0.mean():.0f} cached rows per head, bf16 cache",
        value=round(B / (dt / steps), 1), unit="tokens/s", steps=steps, warmup=warm,
        ms_per_step=round(1000.0 * dt / steps, 4),
        step_bytes=int(step_bytes), step_hbm_frac=round(step_bytes / (dt / steps) / 1e9 / PEAK_HBM_GBS, 4),
        step_stats=dict(flushed_n_open_0=flushed),
        roofline=dict(bound="hbm", kernel="decode_attn", achieved=round(achieved, 1), peak=PEAK_HBM_GBS,
                      unit="GB/s", frac=round(achieved / PEAK_HBM_GBS, 4), traffic=traffic,
                      bytes_per_launch=int(kv_bytes), avg_launch_us=attn_us),
        kernels=kernels), (wl, st, a)


def time_decode_open(args, N, W, wl_state, n_open):
    """One decode step of a sequence whose open chunk already holds n_open
    tokens (n_open = 63: the step completes the chunk, routes it from x_sum
    and commits it), timed step by step with per-step events; the counters,
    states and x_sum are restored and the caches flushed between steps, so
    every timed step is the same step."""
    import torch
    wl, st, a = wl_state
    B, H, D, d = wl.B, wl.H, wl.D, wl.d
    dev = st.k.device
    dm = N.dims(B, H, 1, D, d, N.BF16)
    dec = N.Decode(dm, st, device=dev)
    saved = [x.clone() for x in (st.n_committed, st.n_open, st.S_carry, st.S_work, st.x_sum, st.err)]
    # the open chunk: rows n_committed .. n_committed + n_open - 1 (inside the
    # capacity: cap = 64 * max n_sel + 64), S_work as the pseudo-updated state,
    # x_sum of n_open N(0, 1) rows so the completing chunk routes either way
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    st.n_open.fill_(n_open)
    st.x_sum.copy_(torch.randn(st.x_sum.shape, generator=g, device=dev) * float(np.sqrt(n_open)))
    opened = [x.clone() for x in (st.n_committed, st.n_open, st.S_carry, st.S_work, st.x_sum, st.err)]

    def restore(src=opened):
        for x, y in zip((st.n_committed, st.n_open, st.S_carry, st.S_work, st.x_sum, st.err), src):
            x.copy_(y)
    dec(*a)
    torch.cuda.synchronize()
    routes = dec.route.cpu().numpy()
    restore()
    settle(lambda: (restore(), dec(*a)))
    stats = evented_steps(lambda: dec(*a), 30, flush=Flusher(dev), setup=restore)
    warm = evented_steps(lambda: dec(*a), 30, setup=restore)
    N.profile_enable(True)
    kernels = kernel_table(N, lambda: (restore(), dec(*a)), ("decode_route", "decode_gdn", "decode_attn",
                                                            "decode_combine", "decode_commit"), 10)
    N.profile_enable(False)
    assert int(st.err.item()) == 0
    restore(saved)
    torch.cuda.synchronize()
    nco = saved[0][:, 0].cpu().numpy().astype(np.int64)
    mean_rows = float((nco + n_open).mean())
    n_lin = int((routes == 1).sum()) * H if n_open == 63 else 0
    kv_bytes, step_bytes = decode_step_bytes(wl, mean_rows, completing_lin=n_lin)
    attn_us = kernels["decode_attn"]["avg_us"]
    ach = kv_bytes / (attn_us * 1e-6) / 1e9
    med = stats["median_ms"]
    res = dict(workload=f"decode step with {n_open} tokens already in the open chunk"
                        + (" (completes it: route, commit)" if n_open == 63 else ""),
               value=round(B / (med * 1e-3), 1), unit="tokens/s", ms_per_step_median_flushed=med,
               step_stats=dict(flushed=stats, warm=warm), step_bytes=int(step_bytes),
               step_hbm_frac=round(step_bytes / (med * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
               roofline=dict(bound="hbm", kernel="decode_attn", achieved=round(ach, 1), peak=PEAK_HBM_GBS,
                             unit="GB/s", frac=round(ach / PEAK_HBM_GBS, 4), traffic=None,
                             bytes_per_launch=int(kv_bytes), avg_launch_us=attn_us),
               kernels=kernels)
    if n_open == 63:
        res["completed_routes"] = dict(softmax=int((routes == 0).sum()), linear=int((routes == 1).sum()))
    return res


def cpu_cores():
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))
    except Exception:
        return len(os.sched_getaffinity(0))


def cpu_baseline(W, O, inp, route, workload):
    """The oracle as it stands, on head 0 of the prefill workload: router on
    all chunks, Gated DeltaNet over every token, softmax on every 2nd 64-row
    query block (about 10-15 s of CPU work); scaled to the whole job."""
    wl = W.WORKLOADS[workload]
    sl = lambda a: a[:, :1]
    t0 = time.perf_counter()
    r, _ = O.route(inp["x"], inp["w_score"], inp["b_score"])
    t_route = time.perf_counter() - t0
    t0 = time.perf_counter()
    o_gdn, _ = O.gdn_branch(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["alpha"]), sl(inp["beta"]), r)
    t_gdn = time.perf_counter() - t0
    blocks = list(range(0, wl.nc, 2))
    t0 = time.perf_counter()
    o_sm = O.softmax_branch(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), r, query_blocks=blocks)
    t_sm = time.perf_counter() - t0
    t0 = time.perf_counter()
    O.merge(sl(inp["q"]), o_sm, o_gdn, inp["w_mix"])
    t_merge = time.perf_counter() - t0
    per_head = t_gdn + t_sm * (wl.nc / len(blocks)) + t_merge
    total = t_route + wl.H * per_head
    return dict(value=round(wl.B * wl.L / total, 2), unit="tokens/s", cores=cpu_cores(), kind="oracle",
                sample=f"{workload}: head 0 of {wl.H}; router on all {wl.nc} chunks ({t_route:.2f}s), Gated DeltaNet "
                       f"on all {wl.L} tokens ({t_gdn:.2f}s), softmax on {len(blocks)} of {wl.nc} query blocks "
                       f"({t_sm:.2f}s), merge ({t_merge:.2f}s); per-head time scaled by {wl.nc // len(blocks)} for "
                       f"the softmax and by {wl.H} heads",
                seconds_measured=round(t_route + t_gdn + t_sm + t_merge, 2))


def cpu_baseline_prefill(W, O, inp, name, route_kind=None, block_stride=1):
    """Oracle time of one prefill workload on a bounded sample: the router on
    every chunk (skipped for forced routes), sequence 0 / head 0 with the
    Gated DeltaNet branch over every token and the softmax branch on every
    block_stride-th query block, scaled to all blocks and all (b, h)."""
    wl = W.WORKLOADS[name]
    sl = lambda a: a[:1, :1]
    t0 = time.perf_counter()
    if route_kind:
        r = W.forced_routes(wl.B, wl.nc, route_kind)
    else:
        r, _ = O.route(inp["x"], inp["w_score"], inp["b_score"])
    t_route = time.perf_counter() - t0 if not route_kind else 0.0
    t0 = time.perf_counter()
    o_gdn, _ = O.gdn_branch(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["alpha"]), sl(inp["beta"]), r[:1])
    t_gdn = time.perf_counter() - t0
    blocks = list(range(0, wl.nc, block_stride))
    t0 = time.perf_counter()
    o_sm = O.softmax_branch(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), r[:1], query_blocks=blocks)
    t_sm = time.perf_counter() - t0
    t0 = time.perf_counter()
    O.merge(sl(inp["q"]), o_sm, o_gdn, inp["w_mix"])
    t_merge = time.perf_counter() - t0
    per_head = t_gdn + t_sm * (wl.nc / len(blocks)) + t_merge
    total = t_route + wl.B * wl.H * per_head
    what = f"routes forced all-{'softmax' if route_kind == 'sm' else 'linear'}" if route_kind else \
        f"router on all {wl.B * wl.nc} chunks ({t_route:.2f}s)"
    return dict(value=round(wl.B * wl.L / total, 2), unit="tokens/s", cores=cpu_cores(), kind="oracle",
                sample=f"{name}: {what}; (b=0, h=0) of {wl.B * wl.H}: Gated DeltaNet on all {wl.L} tokens "
                       f"({t_gdn:.2f}s), softmax on {len(blocks)} of {wl.nc} query blocks ({t_sm:.2f}s), merge "
                       f"({t_merge:.2f}s); scaled to all blocks and all {wl.B * wl.H} (b, h)",
                seconds_measured=round(t_route + t_gdn + t_sm + t_merge, 2))


def cpu_baseline_tiny(W, O):
    wl = W.WORKLOADS["tiny"]
    inp = W.make_prefill(wl)
    t0 = time.perf_counter()
    O.forward(inp["x"], inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["w_score"], inp["w_mix"],
              b_score=inp["b_score"])
    dt = time.perf_counter() - t0
    return dict(value=round(wl.B * wl.L / dt, 2), unit="tokens/s", cores=cpu_cores(), kind="oracle",
                sample=f"tiny: the whole forward ({dt:.3f}s)", seconds_measured=round(dt, 3))


def cpu_baseline_decode(W, O, nseq=2):
    """Oracle decode step on the first nseq sequences of the decode workload
    (all heads, ~8192 cached rows each), scaled to B sequences."""
    wl = W.WORKLOADS["decode"]
    cache, new = W.make_decode(wl, B=nseq)
    sub = dict(k=W.bits_to_f32(cache["k"]), v=W.bits_to_f32(cache["v"]), n_committed=cache["n_committed"],
               n_open=cache["n_open"], S_carry=cache["S_carry"], S_work=cache["S_work"], x_sum=cache["x_sum"], err=0)
    t0 = time.perf_counter()
    O.decode_step(sub, new["x"], new["q"], new["k"], new["v"], new["alpha"], new["beta"], new["w_score"],
                  new["w_mix"])
    dt = time.perf_counter() - t0
    per_seq = dt / nseq
    return dict(value=round(1.0 / per_seq, 2), unit="tokens/s", cores=cpu_cores(), kind="oracle",
                sample=f"decode: one step of {nseq} of {wl.B} sequences, all {wl.H} heads ({dt:.2f}s); a step of "
                       f"all {wl.B} sequences would take {per_seq * wl.B:.2f}s",
                seconds_measured=round(dt, 2))


def achievable_peaks():
    """What this GPU reaches on plain library work, as context for the
    datasheet peaks the roofline uses: a large bf16 GEMM (torch / hipBLASLt,
    both operands contiguous) and a 1 GiB device-to-device copy.  Untimed
    by the step clock; run after the timed regions."""
    import torch
    n = 8192
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    c = torch.empty(n, n, device="cuda", dtype=torch.bfloat16)
    settle(lambda: torch.mm(a, b, out=c), 0.2)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        torch.mm(a, b, out=c)
    e1.record()
    torch.cuda.synchronize()
    gemm_tf = 10 * 2 * n ** 3 / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del a, b, c
    x = torch.empty(2 ** 28, device="cuda", dtype=torch.float32)  # 1 GiB
    y = torch.empty_like(x)
    x.fill_(1.0)
    settle(lambda: y.copy_(x), 0.1)
    e0.record()
    for _ in range(10):
        y.copy_(x)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 10 * 2 * x.numel() * 4 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del x, y
    return dict(gemm_bf16_8192_tflops=round(gemm_tf, 1), gemm_frac_of_peak=round(gemm_tf / PEAK_BF16_TFLOPS, 4),
                copy_1GiB_gbs=round(copy_gbs, 1), copy_frac_of_peak=round(copy_gbs / PEAK_HBM_GBS, 4))


PROFILE_BASE = "python3 bench.py --steps 10 --warmup 2 --no-cpu --no-calib --no-alone --decode-steps 20 --profile-copy"
PROFILE_PARTS = {  # part -> bench.py command profiled (one rocprofv3 run per pass)
    "headline": PROFILE_BASE + " --only headline --no-extras",
    "gradients": PROFILE_BASE + " --only headline --no-decode",
    "prefill": PROFILE_BASE + " --only prefill",
    "degen_sm": PROFILE_BASE + " --only degen_sm",
    "degen_lin": PROFILE_BASE + " --only degen_lin",
    "nha": PROFILE_BASE + " --only nha",
}
PROFILE_PASSES = {  # pass -> rocprofv3 options
    "trace": "--kernel-trace --stats",
    "fetch": "--pmc FETCH_SIZE",
    "write": "--pmc WRITE_SIZE",
    "mfma": "--pmc MfmaUtil MfmaFlopsBF16 SQ_BUSY_CU_CYCLES GRBM_GUI_ACTIVE",
}
KERNEL_NAMES = [  # substring of the kernel symbol -> short name
    ("k_softmax_v2", "softmax_masked"), ("k_route_bwd_x", "route_bwd_x"), ("k_route_bwd_w_final", "route_bwd_w_final"),
    ("k_route_bwd_w", "route_bwd_w"), ("k_route", "route"), ("k_compact", "compact"), ("k_gdn_prep", "gdn_prep"),
    ("k_gdn_scan_headIDF16bLi4ELi2ELb1", "gdn_state_scan"), ("k_gdn_scan_head<__bf16, 4, 2, true>", "gdn_state_scan"),
    ("k_gdn_scan", "gdn_scan"), ("k_gdn_bwd_prep", "gdn_bwd_prep"), ("k_gdn_bwd_scan", "gdn_bwd_scan"),
    ("k_gdn_bwd_chunk", "gdn_bwd_chunk"), ("k_mergeI", "merge"), ("k_decode_route", "decode_route"),
    ("k_decode_gdn", "decode_gdn"), ("k_decode_attn", "decode_attn"), ("k_decode_combine", "decode_combine"),
    ("k_decode_commit", "decode_commit"), ("k_handoff_state", "handoff_state"), ("k_handoff_kv", "handoff_kv"),
    ("k_sm_bwd_delta", "sm_bwd_delta"), ("k_sm_bwd_dq", "sm_bwd_dq"), ("k_sm_bwd_dkdv", "sm_bwd_dkdv"),
    ("k_merge_bwd_reduce", "merge_bwd_reduce"), ("k_merge_bwd_final", "merge_bwd_final"), ("k_merge_bwdI", "merge_bwd"),
    ("k_softmax_masked", "nha_window"), ("k_nha_chunk", "nha_chunk"), ("k_nha_scan", "nha_scan"),
    ("k_nha_slots", "nha_slots"),
    ("AUnaryFunctor<float, float", "calib_mul_256MiB"), ("Cijk_", "calib_gemm_bf16_4096"),
]
MFMA_KERNELS = ("softmax_masked", "gdn_prep", "gdn_scan", "sm_bwd_dq", "sm_bwd_dkdv", "gdn_bwd_prep", "gdn_bwd_scan",
                "gdn_bwd_chunk", "gdn_state_scan", "calib_gemm_bf16_4096")


def profile_commands(part):
    return "\n".join(f"    rocprofv3 {o} --output-format csv -d <dir>/{part}/{p} -o b -- {PROFILE_PARTS[part]}"
                     for p, o in PROFILE_PASSES.items())


def summarize_profiles(d):
    """Writes the profiles/ summaries from the rocprofv3 runs under directory d:
    for every part of PROFILE_PARTS that is present, <part>/trace
    (--kernel-trace --stats; the run's stdout and stderr in <part>/trace.log),
    <part>/fetch, <part>/write and <part>/mfma (one --pmc pass each).  Counters
    are per dispatch.  FETCH_SIZE / WRITE_SIZE (KiB) are scaled by what they
    read for the 256 MiB read + 256 MiB write calibration kernel of
    --profile-copy; the MFMA counters are checked against the calibration GEMM
    (2 * 4096^3 FLOPs) of the same run."""
    import csv
    import glob

    def short(name):
        for sub, n in KERNEL_NAMES:
            if sub in name:
                return n
        return None

    def find(sub, fname):
        hits = glob.glob(os.path.join(d, sub, "**", fname), recursive=True)
        return hits[0] if hits else None

    out = os.path.join(ROOT, "profiles")
    calib = 256 * 2 ** 20
    for part in PROFILE_PARTS:
        tr = find(os.path.join(part, "trace"), "*kernel_stats.csv")
        if tr is None:
            continue
        stats = {}
        for r in csv.DictReader(open(tr)):
            n = short(r["Name"])
            if n:
                stats[n] = dict(calls=int(r["Calls"]), avg_us=float(r["AverageNs"]) / 1e3,
                                min_us=float(r["MinNs"]) / 1e3, max_us=float(r["MaxNs"]) / 1e3, symbol=r["Name"])
        ctr = {}
        for key in ("fetch", "write", "mfma"):
            f = find(os.path.join(part, key), "*counter_collection.csv")
            vals = {}
            if f:
                for r in csv.DictReader(open(f)):
                    n = short(r["Kernel_Name"])
                    if n:
                        vals.setdefault((n, r["Counter_Name"]), []).append(float(r["Counter_Value"]))
            ctr[key] = {k: sum(v) / len(v) for k, v in vals.items()}
        fscale = calib / (1024.0 * ctr["fetch"][("calib_mul_256MiB", "FETCH_SIZE")])
        wscale = calib / (1024.0 * ctr["write"][("calib_mul_256MiB", "WRITE_SIZE")])
        rd = lambda n: ctr["fetch"].get((n, "FETCH_SIZE"), 0.0) * 1024.0 * fscale
        wr = lambda n: ctr["write"].get((n, "WRITE_SIZE"), 0.0) * 1024.0 * wscale
        mf = lambda n, c: ctr["mfma"].get((n, c))
        bench_line = None
        for line in open(os.path.join(d, part, "trace.log")):
            if line.startswith('{"metric"'):
                bench_line = json.loads(line)
        if bench_line is None:
            raise SystemExit(f"no bench line in {part}/trace.log")
        cmds = profile_commands(part)
        scaling = (f"Counter scaling: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled by what they read for a "
                   f"plain elementwise kernel that reads 256 MiB and writes 256 MiB (torch.mul over 64 Mi fp32, run by "
                   f"`--profile-copy` in the same process): FETCH_SIZE x {fscale:.3f}, WRITE_SIZE x {wscale:.3f}. "
                   f"MfmaUtil is rocprofv3's derived metric (MFMA busy cycles summed over the SIMDs / (GPU active "
                   f"cycles x SIMDs)); MfmaFlopsBF16 = 512 x SQ_INSTS_VALU_MFMA_MOPS_BF16, the bf16 FLOPs the matrix "
                   f"cores executed.")
        g = ("calib_gemm_bf16_4096", "MfmaFlopsBF16")
        gemm_check = ""
        if g in ctr["mfma"]:
            gemm_check = (f" The calibration GEMM (torch.mm, 4096^3 bf16, 1.374e+11 FLOPs) reads "
                          f"MfmaFlopsBF16 = {ctr['mfma'][g]:.3e}.")
        # every kernel of the run
        lines = [f"# All kernels of the `{part}` profile run", "",
                 "Commands (from the repository root on one MI355X; rocprofv3 writes CSV; the runs are separate):", "",
                 cmds, ""]
        if "ms_per_step" in bench_line:
            lines.append(f"bench.py reported {bench_line['ms_per_step']} ms per forward step ({bench_line['value']:.0f} "
                         f"tokens/s)" + (f" and {bench_line['decode']['ms_per_step']} ms per decode step"
                                          if "decode" in bench_line else "") + " in the traced run.")
        for k, v in bench_line.get("configs", {}).items():
            ms = v.get("ms_per_step", v.get("ms_per_call_median"))
            lines.append(f"bench.py reported for `{k}`: {ms} ms per step ({v.get('value'):.0f} "
                         f"tokens/s) in the traced run.")
        lines += ["bench.py first runs each step untimed for 0.3 s (clock settle), so the dispatch counts include "
                  "those steps.", "",
                  "| kernel | calls | avg us | min us | max us | HBM read MB/launch | HBM write MB/launch | MfmaUtil % "
                  "| executed bf16 MFMA TFLOP/s |",
                  "|---|---|---|---|---|---|---|---|---|"]
        for n in dict.fromkeys(n for _, n in KERNEL_NAMES):
            if n in stats:
                st = stats[n]
                mu, fl = mf(n, "MfmaUtil"), mf(n, "MfmaFlopsBF16")
                mu_s = "" if mu is None else f"{mu:.1f}"
                fl_s = "" if fl is None else f"{fl / (st['avg_us'] * 1e-6) / 1e12:.1f}"
                lines.append(f"| {n} | {st['calls']} | {st['avg_us']:.1f} | {st['min_us']:.1f} | {st['max_us']:.1f} | "
                             f"{rd(n) / 1e6:.1f} | {wr(n) / 1e6:.1f} | {mu_s} | {fl_s} |")
        lines += ["", scaling + gemm_check,
                  "The forward's kernels overlap (the Gated DeltaNet prep and scan run on a helper stream beside "
                  "routing and softmax_masked), so their durations do not add up to the step time; MfmaUtil of a "
                  "kernel is taken over the GPU's active cycles while it runs, which includes the other stream's work."]
        with open(os.path.join(out, f"kernels_{part}.md"), "w") as f:
            f.write("\n".join(lines) + "\n")
        # roofline kernels with their counter files
        targets = []
        if part == "headline":
            targets = [("softmax_masked", "long", ("softmax_masked.hip", "common.hpp"),
                        "softmax_masked on the long prefill (B=1 H=16 L=32768 D=128, bf16, 25% softmax chunks)",
                        bench_line["roofline"]),
                       ("decode_attn", "decode", ("decode.hip", "common.hpp"),
                        "decode_attn on the decode step (B=64 H=16 D=128, about 8192 cached rows per head, bf16)",
                        bench_line["decode"]["roofline"])]
        elif part in ("prefill", "degen_sm"):
            wl = "prefill" if part == "prefill" else "degen_sm"
            targets = [("softmax_masked", wl, ("softmax_masked.hip", "common.hpp"),
                        f"softmax_masked on the {bench_line['configs'][part]['workload']}",
                        bench_line["configs"][part]["roofline"])]
        if part == "degen_lin":
            # the all-linear run's roofline is the Gated DeltaNet chain (prep + scan)
            h = source_hash("gdn.hip", "common.hpp")
            rf = bench_line["configs"]["degen_lin"]["roofline"]
            rb, wb = rd("gdn_prep") + rd("gdn_scan"), wr("gdn_prep") + wr("gdn_scan")
            chain_us = stats["gdn_prep"]["avg_us"] + stats["gdn_scan"]["avg_us"]
            c = dict(kernel="gdn_chain", workload="degen_lin", source_hash=h, hbm_bytes_per_launch=int(rb + wb),
                     hbm_read_bytes=int(rb), hbm_write_bytes=int(wb), fetch_scale=fscale, write_scale=wscale,
                     command=PROFILE_PARTS[part])
            with open(os.path.join(out, "gdn_chain_degen_lin_counters.txt"), "w") as f:
                json.dump(c, f, indent=1)
            ach = rf["bytes_per_launch"] / (chain_us * 1e-6) / 1e9
            lines = [f"# Gated DeltaNet chain (prep + scan) on the {bench_line['configs'][part]['workload']}", "",
                     "Commands:", "", cmds, "",
                     f"Kernels `{stats['gdn_prep']['symbol']}` and `{stats['gdn_scan']['symbol']}`, source hash {h}.",
                     "", "| figure | value |", "|---|---|",
                     f"| average duration, prep + scan (rocprofv3 kernel trace) | {stats['gdn_prep']['avg_us']:.1f} + "
                     f"{stats['gdn_scan']['avg_us']:.1f} = {chain_us:.1f} us |",
                     f"| average duration, prep + scan (bench.py HIP events, same run) | {rf['avg_launch_us']:.1f} us |",
                     f"| algorithmic bytes per launch (q, k, v, alpha, beta in; o_gdn out) | "
                     f"{rf['bytes_per_launch'] / 1e6:.1f} MB |",
                     f"| achieved (trace average) | {ach:.0f} GB/s = {100 * ach / rf['peak']:.1f}% of "
                     f"{rf['peak']:.0f} GB/s |",
                     f"| HBM read per launch, prep + scan (FETCH_SIZE scaled) | {rb / 1e6:.1f} MB |",
                     f"| HBM write per launch, prep + scan (WRITE_SIZE scaled) | {wb / 1e6:.1f} MB |",
                     f"| scan time per dependent chunk step | {stats['gdn_scan']['avg_us'] / 128:.2f} us |",
                     f"| MfmaUtil prep / scan | {mf('gdn_prep', 'MfmaUtil') or 0:.1f}% / "
                     f"{mf('gdn_scan', 'MfmaUtil') or 0:.1f}% |", "", scaling + gemm_check]
            with open(os.path.join(out, "gdn_chain_degen_lin.md"), "w") as f:
                f.write("\n".join(lines) + "\n")
        for n, wl, srcs, title, rf in targets:
            h = source_hash(*srcs)
            st = stats[n]
            c = dict(kernel=n, workload=wl, source_hash=h, hbm_bytes_per_launch=int(rd(n) + wr(n)),
                     hbm_read_bytes=int(rd(n)), hbm_write_bytes=int(wr(n)), fetch_scale=fscale, write_scale=wscale,
                     mfma_util_pct=mf(n, "MfmaUtil"), mfma_flops_bf16_per_launch=mf(n, "MfmaFlopsBF16"),
                     command=PROFILE_PARTS[part])
            with open(os.path.join(out, f"{n}_{wl}_counters.txt"), "w") as f:
                json.dump(c, f, indent=1)
            if rf["unit"] == "TFLOP/s":
                work = f"| algorithmic FLOPs per launch | {rf['flops_per_launch']:.3e} |"
                ach = rf["flops_per_launch"] / (st["avg_us"] * 1e-6) / 1e12
                achieved = (f"| achieved (trace average) | {ach:.1f} TFLOP/s = {100 * ach / rf['peak']:.1f}% of "
                            f"{rf['peak']:.0f} TFLOP/s |")
            else:
                work = f"| algorithmic bytes per launch | {rf['bytes_per_launch'] / 1e6:.1f} MB |"
                ach = rf["bytes_per_launch"] / (st["avg_us"] * 1e-6) / 1e9
                achieved = (f"| achieved (trace average) | {ach:.0f} GB/s = {100 * ach / rf['peak']:.1f}% of "
                            f"{rf['peak']:.0f} GB/s |")
            mu, fl = mf(n, "MfmaUtil"), mf(n, "MfmaFlopsBF16")
            lines = [f"# {title}", "", "Commands:", "", cmds, "",
                     f"Kernel `{st['symbol']}`, source hash {h}.", "",
                     "| figure | value |", "|---|---|",
                     f"| dispatches | {st['calls']} |",
                     f"| average duration (rocprofv3 kernel trace) | {st['avg_us']:.1f} us |",
                     f"| average duration (bench.py HIP events over its timed steps, same run) | "
                     f"{rf['avg_launch_us']:.1f} us |",
                     work, achieved,
                     f"| HBM read per launch (FETCH_SIZE scaled) | {rd(n) / 1e6:.1f} MB |",
                     f"| HBM write per launch (WRITE_SIZE scaled) | {wr(n) / 1e6:.1f} MB |"]
            if mu is not None:
                lines += [f"| MfmaUtil (rocprofv3 derived, during the launch) | {mu:.1f}% |",
                          f"| bf16 MFMA FLOPs executed per launch (MfmaFlopsBF16) | {fl:.3e} "
                          f"({fl / (st['avg_us'] * 1e-6) / 1e12:.1f} TFLOP/s at the trace average) |"]
            lines += ["", scaling + gemm_check]
            if n == "softmax_masked":
                lines.append("In the forward pass this kernel shares the GPU with the Gated DeltaNet chunk prep and "
                             "scan (second stream).")
            with open(os.path.join(out, f"{n}_{wl}.md"), "w") as f:
                f.write("\n".join(lines) + "\n")
    print("wrote", out)


CONFIG_NAMES = ("prefill", "degen_sm", "degen_lin", "decode_open32", "decode_open63", "nha")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="long", choices=["long", "prefill"])
    ap.add_argument("--decode-steps", type=int, default=50)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads (B=4 L=4096 prefill, the forced all-softmax / all-linear pair, "
                         "decode steps with 32 and 63 open tokens)")
    ap.add_argument("--no-extras", action="store_true", help="skip the handoff and gradient timings")
    ap.add_argument("--only", choices=("headline",) + CONFIG_NAMES, default=None,
                    help="profiling: run only this part (headline = the long prefill and the decode step)")
    ap.add_argument("--no-calib", action="store_true", help="skip the achievable-peak GEMM and copy")
    ap.add_argument("--no-alone", action="store_true",
                    help="skip timing the softmax branch alone (profiled runs: its launches would mix with the "
                         "forward's in the kernel trace)")
    ap.add_argument("--profile-copy", action="store_true",
                    help="first run a plain 256 MiB read + 256 MiB write elementwise kernel three times, "
                         "the known-size reference for scaling FETCH_SIZE / WRITE_SIZE counters, and a bf16 "
                         "GEMM of known FLOPs, the reference for the MFMA counters")
    ap.add_argument("--summarize-profiles", metavar="DIR", default=None,
                    help="CPU only: write the profiles/ summaries from the rocprofv3 runs of PROFILE_CMDS under DIR")
    args = ap.parse_args()
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles)
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not supported "
              "(shard over (batch, head) with one process per GPU; see the design notes)", file=sys.stderr)
        sys.exit(2)
    import torch
    import linear_attention_natsl_amd as N
    import workloads as W
    import oracle as O
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    N.lib()
    if args.profile_copy:
        a = torch.ones(64 * 2 ** 20, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            torch.mul(a, 2.0, out=b)
        ga = torch.randn(4096, 4096, dtype=torch.bfloat16, device="cuda")
        gb = torch.randn(4096, 4096, dtype=torch.bfloat16, device="cuda")
        for _ in range(3):
            torch.mm(ga, gb)
        torch.cuda.synchronize()
        del a, b, ga, gb
    only = args.only
    res = None
    if only in (None, "headline"):
        res, inp, route = time_prefill(args, N, W)
        print(f"prefill: {res['ms_per_step']} ms/step, {res['value']:.0f} tok/s, softmax "
              f"{res['roofline']['frac']*100:.1f}% of MFMA peak, layer {res['layer']['layer_frac_of_mfma_peak']*100:.1f}%",
              file=sys.stderr, flush=True)
    else:
        res = dict(metric="hybrid-layer prefill tokens/sec + % bf16 MFMA peak; decode-step % HBM peak",
                   profiled_part=only)
    dstate = None
    if not args.no_decode and only in (None, "headline", "decode_open32", "decode_open63"):
        if only in (None, "headline"):
            res["decode"], dstate = time_decode(args, N, W)
            print(f"decode: {res['decode']['ms_per_step']} ms/step, attn {res['decode']['roofline']['frac']*100:.1f}% "
                  f"of HBM peak", file=sys.stderr, flush=True)
        else:
            import torch as _t
            dstate = decode_state(N, W, _t.device("cuda:0"))
    configs = {}
    if not args.no_configs:
        for name, fn in (("prefill", lambda: time_prefill_config(args, N, W, "prefill")),
                         ("degen_sm", lambda: time_prefill_config(args, N, W, "degen", "sm")),
                         ("degen_lin", lambda: time_prefill_config(args, N, W, "degen", "lin"))):
            if only in (None, name):
                configs[name] = fn()
                print(f"{name}: {configs[name][0]['ms_per_step']} ms/step, roofline "
                      f"{configs[name][0]['roofline']['frac']*100:.1f}%", file=sys.stderr, flush=True)
        if dstate is not None:
            for n_open in (32, 63):
                name = f"decode_open{n_open}"
                if only in (None, name):
                    configs[name] = (time_decode_open(args, N, W, dstate, n_open), None, None)
                    print(f"{name}: {configs[name][0]['ms_per_step_median_flushed']} ms/step (median, flushed)",
                          file=sys.stderr, flush=True)
        if only in (None, "nha"):
            configs["nha"] = (time_nha(args, N, W), None, None)
            print(f"nha: {configs['nha'][0]['ms_per_call_median']} ms/call, dominant {configs['nha'][0]['roofline']['kernel']} "
                  f"{configs['nha'][0]['roofline']['frac']*100:.1f}%", file=sys.stderr, flush=True)
    del dstate
    if configs:
        res["configs"] = {k: v[0] for k, v in configs.items()}
    if not args.no_calib and only is None:
        res["achievable"] = achievable_peaks()
    if not args.no_cpu and only is None:
        res["cpu_baseline"] = cpu_baseline(W, O, inp, route, args.workload)
        per = dict(tiny=cpu_baseline_tiny(W, O))
        if "prefill" in configs:
            per["prefill"] = cpu_baseline_prefill(W, O, configs["prefill"][1], "prefill", block_stride=2)
        if "degen_sm" in configs:
            per["degen_sm"] = cpu_baseline_prefill(W, O, configs["degen_sm"][1], "degen", "sm", block_stride=8)
        if "degen_lin" in configs:
            per["degen_lin"] = cpu_baseline_prefill(W, O, configs["degen_lin"][1], "degen", "lin", block_stride=8)
        if not args.no_decode:
            per["decode"] = cpu_baseline_decode(W, O)
        res["cpu_baseline_per_config"] = per
    print(json.dumps(res))


if __name__ == "__main__":
    main()
