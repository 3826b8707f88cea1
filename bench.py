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


def time_gdn_backward(N, dm, t, wl, route, reps=2):
    """Gradient of the Gated DeltaNet branch on this workload (a random fp32
    upstream gradient on o_gdn), timed with events.  Plain fp32 VALU work, so
    it is set against the fp32 vector peak; algorithmic work 16 D^2 FLOP per
    token for the reverse step (outer product, two column and two row
    contractions, the decay gradient, the erase of G), not counting the two
    forward recomputations the per-token form also runs."""
    import torch
    d_o = torch.randn(t["q"].shape, dtype=torch.float32, device=t["q"].device)
    N.gdn_backward(dm, t["q"], t["k"], t["v"], t["alpha"], t["beta"], route, d_o)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        N.gdn_backward(dm, t["q"], t["k"], t["v"], t["alpha"], t["beta"], route, d_o)
    e1.record()
    torch.cuda.synchronize()
    us = 1000.0 * e0.elapsed_time(e1) / reps
    flops = 16 * wl.D * wl.D * wl.B * wl.H * wl.L
    tf = flops / (us * 1e-6) / 1e12
    return dict(workload=f"gradient of the Gated DeltaNet branch on the {wl.name} prefill (per-token form)",
                us=round(us, 1), flops=flops, tflops=round(tf, 2), bound="alu",
                frac_fp32_valu=round(tf / PEAK_FP32_VALU_TFLOPS, 4))


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


def time_prefill(args, N, W, O):
    import torch
    wl = W.WORKLOADS[args.workload]
    inp = W.make_prefill(wl)
    dev = torch.device("cuda:0")
    io_t = torch.bfloat16 if inp["io"] == "bf16" else torch.float32
    t = {k: torch.from_numpy(np.ascontiguousarray(inp[k])).to(dev).to(io_t) for k in ("x", "q", "k", "v")}
    for k in ("alpha", "beta", "w_score", "w_mix", "b_score", "g_sm", "g_lin"):
        t[k] = torch.from_numpy(np.ascontiguousarray(inp[k])).to(dev)
    dm = N.dims(wl.B, wl.H, wl.L, wl.D, wl.d, N.BF16 if inp["io"] == "bf16" else N.F32)
    fwd = N.Forward(dm, device=dev)
    call = lambda: fwd(t["x"], t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["w_score"], t["w_mix"],
                       b_score=t["b_score"], g_sm=t["g_sm"], g_lin=t["g_lin"])
    settle(call)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    # timed steps: only the roofline kernel is bracketed by events
    N.profile_enable(True)
    N.profile_select("softmax_masked")
    N.profile_reset()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        call()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    n, ms = N.profile_read("softmax_masked")
    sm_avg_us = 1000.0 * ms / max(n, 1)
    kernels = kernel_table(N, call, ("route", "compact", "gdn_prep", "gdn_scan", "softmax_masked", "merge"),
                           max(5, args.steps // 5))
    N.profile_enable(False)
    sm_alone_us = None if args.no_alone else time_softmax_alone(N, dm, fwd.route, t, io_t, max(10, args.steps // 2))
    handoff = time_handoff(N, dm, fwd.route, t, wl)
    backward = time_softmax_backward(N, dm, t, wl, sm_pairs(fwd.route.cpu().numpy(), wl.H))
    gdn_backward = time_gdn_backward(N, dm, t, wl, fwd.route)
    merge_backward = time_merge_backward(N, dm, t, wl)
    route = fwd.route.cpu().numpy()
    ref_route = O.route(inp["x"], inp["w_score"], inp["b_score"])[0] if args.check_route else None
    pairs = sm_pairs(route, wl.H)
    f_sm = 4 * wl.D * pairs
    n_lin = int((route == 1).sum())
    f_gdn = gdn_flops(wl.B, wl.H, wl.nc, n_lin, wl.D)
    ms_step = 1000.0 * dt / args.steps
    tok_s = wl.B * wl.L / (dt / args.steps)
    sm_us = round(sm_avg_us, 2)
    achieved = f_sm / (sm_us * 1e-6) / 1e12
    traffic = counters_traffic("softmax_masked", args.workload, source_hash("softmax_masked.hip", "common.hpp"))
    res = dict(
        metric="hybrid-layer prefill tokens/sec + % bf16 MFMA peak; decode-step % HBM peak",
        value=round(tok_s, 1), unit="tokens/s", n_gpus=1, steps=args.steps, warmup=args.warmup,
        ms_per_step=round(ms_step, 4), higher_is_better=True, scaling="weak", vs_baseline=None,
        dtype="bf16" if inp["io"] == "bf16" else "f32", data="synthetic",
        config=dict(workload=f"{args.workload} prefill: B={wl.B} H={wl.H} L={wl.L} D={wl.D} d_model={wl.d}, "
                    f"chunk 64, {inp['io']} io and branch outputs / fp32 accumulate",
                    B=wl.B, H=wl.H, L=wl.L, D=wl.D, d_model=wl.d, seed=wl.seed,
                    softmax_chunk_fraction=round(float((route == 0).mean()), 4),
                    route_matches_oracle=None if ref_route is None else bool(np.array_equal(route, ref_route)),
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
                   layer_tflops=round((f_sm + f_gdn) / (dt / args.steps) / 1e12, 1),
                   layer_frac_of_mfma_peak=round((f_sm + f_gdn) / (dt / args.steps) / 1e12 / PEAK_BF16_TFLOPS, 4),
                   kernels=kernels),
        handoff=handoff,
        softmax_backward=backward,
        gdn_backward=gdn_backward,
        merge_backward=merge_backward,
    )
    return res, inp, route


def time_decode(args, N, W):
    import torch
    wl = W.WORKLOADS["decode"]
    cache, new = W.make_decode(wl)
    dev = torch.device("cuda:0")
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
    dm = N.dims(B, H, 1, D, d, N.BF16)
    dec = N.Decode(dm, st, device=dev)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(torch.bfloat16)
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    a = [bf(new["x"]), bf(new["q"]), bf(new["k"]), bf(new["v"]), f32(new["alpha"]), f32(new["beta"]),
         f32(new["w_score"]), f32(new["w_mix"])]
    rows0 = (st.n_committed[:, 0] + st.n_open).cpu().numpy().astype(np.int64)
    steps, warm = args.decode_steps, 3
    # settle the clocks with bursts of steps, each followed by a restore of the
    # counters and states (the cache rows the burst appended are rewritten by
    # the timed steps), so the cache never grows past its capacity
    saved = [x.clone() for x in (st.n_committed, st.n_open, st.S_carry, st.S_work, st.x_sum, st.err)]

    def burst():
        for _ in range(32):
            dec(*a)
        for x, y in zip((st.n_committed, st.n_open, st.S_carry, st.S_work, st.x_sum, st.err), saved):
            x.copy_(y)
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
    # per-kernel table from an untimed burst, restored afterwards as above
    kernels = kernel_table(N, lambda: dec(*a), ("decode_route", "decode_gdn", "decode_attn", "decode_combine",
                                                "decode_commit"), 10)
    N.profile_enable(False)
    assert int(st.err.item()) == 0
    for x, y in zip((st.n_committed, st.n_open, st.S_carry, st.S_work, st.x_sum, st.err), saved):
        x.copy_(y)
    # rows read per step: step i reads rows_start + i cached rows per (b, h)
    mean_rows = float((rows_start[:, None] + np.arange(steps)[None, :]).mean())
    kv_bytes = B * H * mean_rows * 2 * D * 2
    step_bytes = kv_bytes + B * H * (2 * D * 2 + 2 * D * D * 4 + 4 * D * 2) + B * d * (2 + 8)
    achieved = kv_bytes / (attn_us * 1e-6) / 1e9
    traffic = counters_traffic("decode_attn", "decode", source_hash("decode.hip", "common.hpp"))
    return dict(
        workload=f"decode: B={B} H={H} D={D} d_model={d}, ~{rows0.mean():.0f} cached rows per head, bf16 cache",
        value=round(B / (dt / steps), 1), unit="tokens/s", steps=steps, warmup=warm,
        ms_per_step=round(1000.0 * dt / steps, 4),
        step_bytes=int(step_bytes), step_hbm_frac=round(step_bytes / (dt / steps) / 1e9 / PEAK_HBM_GBS, 4),
        roofline=dict(bound="hbm", kernel="decode_attn", achieved=round(achieved, 1), peak=PEAK_HBM_GBS,
                      unit="GB/s", frac=round(achieved / PEAK_HBM_GBS, 4), traffic=traffic,
                      bytes_per_launch=int(kv_bytes), avg_launch_us=attn_us),
        kernels=kernels)


def cpu_baseline(W, O, inp, route, workload):
    """The oracle as it stands, on head 0 of the prefill workload: router on
    all chunks, Gated DeltaNet over every token, softmax on every 2nd 64-row
    query block (about 10-15 s of CPU work); scaled to the whole job."""
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
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
    return dict(value=round(wl.B * wl.L / total, 2), unit="tokens/s", cores=int(cores), kind="oracle",
                sample=f"{workload}: head 0 of {wl.H}; router on all {wl.nc} chunks ({t_route:.2f}s), Gated DeltaNet "
                       f"on all {wl.L} tokens ({t_gdn:.2f}s), softmax on {len(blocks)} of {wl.nc} query blocks "
                       f"({t_sm:.2f}s), merge ({t_merge:.2f}s); per-head time scaled by {wl.nc // len(blocks)} for "
                       f"the softmax and by {wl.H} heads",
                seconds_measured=round(t_route + t_gdn + t_sm + t_merge, 2))


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


PROFILE_CMD = "python3 bench.py --steps 10 --warmup 2 --no-cpu --no-calib --no-alone --decode-steps 20 --profile-copy"
KERNEL_NAMES = [  # substring of the kernel symbol -> short name
    ("k_softmax_v2", "softmax_masked"), ("k_route", "route"), ("k_compact", "compact"), ("k_gdn_prep", "gdn_prep"),
    ("k_gdn_scan", "gdn_scan"), ("k_mergeI", "merge"), ("k_decode_route", "decode_route"),
    ("k_decode_gdn", "decode_gdn"), ("k_decode_attn", "decode_attn"), ("k_decode_combine", "decode_combine"),
    ("k_decode_commit", "decode_commit"), ("k_handoff_state", "handoff_state"), ("k_handoff_kv", "handoff_kv"),
    ("k_sm_bwd_delta", "sm_bwd_delta"), ("k_sm_bwd_dq", "sm_bwd_dq"), ("k_sm_bwd_dkdv", "sm_bwd_dkdv"),
    ("k_gdn_bwd_ckpt", "gdn_bwd_ckpt"), ("k_gdn_bwdI", "gdn_bwd"), ("k_gdn_bwd_reduce", "gdn_bwd_reduce"),
    ("k_merge_bwd_reduce", "merge_bwd_reduce"), ("k_merge_bwd_final", "merge_bwd_final"), ("k_merge_bwdI", "merge_bwd"),
    ("AUnaryFunctor<float, float", "calib_mul_256MiB"),
]


def summarize_profiles(d):
    """Writes the profiles/ summaries from the rocprofv3 runs of PROFILE_CMD
    under directory d: prof_trace/ (--kernel-trace --stats, whose stdout went
    to prof_trace.log), prof_fetch/ (--pmc FETCH_SIZE), prof_write/ (--pmc
    WRITE_SIZE).  Counters are KiB per dispatch, scaled by what they read for
    the 256 MiB read + 256 MiB write calibration kernel of --profile-copy."""
    import csv
    import glob

    def short(name):
        for sub, n in KERNEL_NAMES:
            if sub in name:
                return n
        return None

    def find(sub, fname):
        hits = glob.glob(os.path.join(d, sub, "**", fname), recursive=True)
        if not hits:
            raise SystemExit(f"no {fname} under {os.path.join(d, sub)}")
        return hits[0]

    stats = {}
    for r in csv.DictReader(open(find("prof_trace", "*kernel_stats.csv"))):
        n = short(r["Name"])
        if n:
            stats[n] = dict(calls=int(r["Calls"]), avg_us=float(r["AverageNs"]) / 1e3, min_us=float(r["MinNs"]) / 1e3,
                            max_us=float(r["MaxNs"]) / 1e3, symbol=r["Name"])
    ctr = {}
    for key, sub in (("fetch", "prof_fetch"), ("write", "prof_write")):
        vals = {}
        for r in csv.DictReader(open(find(sub, "*counter_collection.csv"))):
            n = short(r["Kernel_Name"])
            if n:
                vals.setdefault(n, []).append(float(r["Counter_Value"]) * 1024.0)
        ctr[key] = {n: sum(v) / len(v) for n, v in vals.items()}
    calib = 256 * 2 ** 20
    fscale = calib / ctr["fetch"]["calib_mul_256MiB"]
    wscale = calib / ctr["write"]["calib_mul_256MiB"]
    bench_line = None
    for line in open(os.path.join(d, "prof_trace.log")):
        if line.startswith('{"metric"'):
            bench_line = json.loads(line)
    if bench_line is None:
        raise SystemExit("no bench line in prof_trace.log")
    cmds = "\n".join(f"    rocprofv3 {a} --output-format csv -d <dir>/{b} -o b -- {PROFILE_CMD}" for a, b in
                     (("--kernel-trace --stats", "prof_trace"), ("--pmc FETCH_SIZE", "prof_fetch"),
                      ("--pmc WRITE_SIZE", "prof_write")))
    scaling = (f"Counter scaling: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled by what they read for a plain "
               f"elementwise kernel that reads 256 MiB and writes 256 MiB (torch.mul over 64 Mi fp32, run by "
               f"`--profile-copy` in the same process): FETCH_SIZE x {fscale:.3f}, WRITE_SIZE x {wscale:.3f}.")
    rd = lambda n: ctr["fetch"].get(n, 0.0) * fscale
    wr = lambda n: ctr["write"].get(n, 0.0) * wscale
    out = os.path.join(ROOT, "profiles")
    # all kernels
    lines = ["# All kernels of one bench run (long prefill forward + decode step + handoff + both branch gradients)", "",
             "Commands (from the repository root on one MI355X; rocprofv3 writes CSV; the three runs are separate):", "",
             cmds, "",
             f"bench.py reported {bench_line['ms_per_step']} ms per forward step ({bench_line['value']:.0f} tokens/s) "
             f"and {bench_line['decode']['ms_per_step']} ms per decode step in the traced run. bench.py first runs each "
             f"step untimed for 0.3 s (clock settle), so the dispatch counts include those steps.", "",
             "| kernel | calls | avg us | min us | max us | HBM read MB/launch | HBM write MB/launch |",
             "|---|---|---|---|---|---|---|"]
    for _, n in KERNEL_NAMES:
        if n in stats:
            st = stats[n]
            lines.append(f"| {n} | {st['calls']} | {st['avg_us']:.1f} | {st['min_us']:.1f} | {st['max_us']:.1f} | "
                         f"{rd(n) / 1e6:.1f} | {wr(n) / 1e6:.1f} |")
    lines += ["", scaling,
              "The forward's kernels overlap (the Gated DeltaNet prep and scan run on a helper stream beside routing and "
              "softmax_masked), so their durations do not add up to the step time."]
    with open(os.path.join(out, "kernels_long_and_decode.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    # roofline kernels
    for n, wl, srcs, title, bench_part in (
            ("softmax_masked", "long", ("softmax_masked.hip", "common.hpp"),
             "softmax_masked on the long prefill (B=1 H=16 L=32768 D=128, bf16, 25% softmax chunks)", bench_line),
            ("decode_attn", "decode", ("decode.hip", "common.hpp"),
             "decode_attn on the decode step (B=64 H=16 D=128, about 8192 cached rows per head, bf16)",
             bench_line["decode"])):
        h = source_hash(*srcs)
        rf = bench_part["roofline"]
        st = stats[n]
        c = dict(kernel=n, workload=wl, source_hash=h, hbm_bytes_per_launch=int(rd(n) + wr(n)),
                 hbm_read_bytes=int(rd(n)), hbm_write_bytes=int(wr(n)), fetch_scale=fscale, write_scale=wscale,
                 command=PROFILE_CMD)
        with open(os.path.join(out, f"{n}_{wl}_counters.txt"), "w") as f:
            json.dump(c, f, indent=1)
        if rf["unit"] == "TFLOP/s":
            work = f"| algorithmic FLOPs per launch | {rf['flops_per_launch']:.3e} |"
            ach = rf["flops_per_launch"] / (st["avg_us"] * 1e-6) / 1e12
            achieved = f"| achieved (trace average) | {ach:.1f} TFLOP/s = {100 * ach / rf['peak']:.1f}% of {rf['peak']:.0f} TFLOP/s |"
        else:
            work = f"| algorithmic bytes per launch | {rf['bytes_per_launch'] / 1e6:.1f} MB |"
            ach = rf["bytes_per_launch"] / (st["avg_us"] * 1e-6) / 1e9
            achieved = f"| achieved (trace average) | {ach:.0f} GB/s = {100 * ach / rf['peak']:.1f}% of {rf['peak']:.0f} GB/s |"
        lines = [f"# {title}", "", "Commands:", "", cmds, "",
                 f"Kernel `{st['symbol']}`, source hash {h}.", "",
                 "| figure | value |", "|---|---|",
                 f"| dispatches | {st['calls']} |",
                 f"| average duration (rocprofv3 kernel trace) | {st['avg_us']:.1f} us |",
                 f"| average duration (bench.py HIP events over its timed steps, same run) | {rf['avg_launch_us']:.1f} us |",
                 work, achieved,
                 f"| HBM read per launch (FETCH_SIZE scaled) | {rd(n) / 1e6:.1f} MB |",
                 f"| HBM write per launch (WRITE_SIZE scaled) | {wr(n) / 1e6:.1f} MB |", "", scaling]
        if n == "softmax_masked":
            lines.append("In the forward pass this kernel shares the GPU with the Gated DeltaNet chunk prep and scan "
                         "(second stream).")
        with open(os.path.join(out, f"{n}_{wl}.md"), "w") as f:
            f.write("\n".join(lines) + "\n")
    print("wrote", out)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="long", choices=["long", "prefill", "degen"])
    ap.add_argument("--decode-steps", type=int, default=50)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-calib", action="store_true", help="skip the achievable-peak GEMM and copy")
    ap.add_argument("--no-alone", action="store_true",
                    help="skip timing the softmax branch alone (profiled runs: its launches would mix with the "
                         "forward's in the kernel trace)")
    ap.add_argument("--check-route", action="store_true")
    ap.add_argument("--profile-copy", action="store_true",
                    help="first run a plain 256 MiB read + 256 MiB write elementwise kernel three times, "
                         "the known-size reference for scaling FETCH_SIZE / WRITE_SIZE counters")
    ap.add_argument("--summarize-profiles", metavar="DIR", default=None,
                    help="CPU only: write the profiles/ summaries from the rocprofv3 runs of PROFILE_CMD under DIR")
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
        torch.cuda.synchronize()
        del a, b
    res, inp, route = time_prefill(args, N, W, O)
    print(f"prefill: {res['ms_per_step']} ms/step, {res['value']:.0f} tok/s, softmax "
          f"{res['roofline']['frac']*100:.1f}% of MFMA peak", file=sys.stderr, flush=True)
    if not args.no_decode:
        res["decode"] = time_decode(args, N, W)
        print(f"decode: {res['decode']['ms_per_step']} ms/step, attn {res['decode']['roofline']['frac']*100:.1f}% "
              f"of HBM peak", file=sys.stderr, flush=True)
    if not args.no_calib:
        res["achievable"] = achievable_peaks()
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(W, O, inp, route, args.workload)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
