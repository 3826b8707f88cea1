"""GPU checks of the C ABI's boundary behaviour: concurrent callers, the
longest supported prefill, and the kernel that serves softmax tile lists
longer than the fast kernel's LDS list.  Every call goes through the C ABI;
results are compared with serial runs or with the fp64 oracle."""
import sys
import threading

import numpy as np
import pytest
import torch

import linear_attention_natsl_amd as N
import oracle as O
import workloads as W
from tests.gpu_util import TOL_BF16, dev, host, maxerr, oracle_head, prefill_tensors, rmsn, rows_of_blocks

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def case(B, H, L, D, d, seed, routing="iid", extra=None, sm_frac=0.5):
    wl = W.Workload("case", "bf16", B, H, L, D, d, routing, seed, extra or {})
    return wl, W.make_prefill(wl, routing=routing, sm_frac=sm_frac)


def test_concurrent_forwards_two_threads_two_streams():
    """Two host threads call natsl_forward at the same time, each on its own
    stream with its own inputs and workspace, 12 times each; every result is
    bit-identical to the same call run alone.  Each call takes its own helper
    stream and events, so neither can wait on the other's records."""
    B, H, L, D, d = 1, 4, 2048, 128, 256
    runs = []
    for seed in (81, 82):
        wl, inp = case(B, H, L, D, d, seed)
        t = prefill_tensors(inp)
        dm = N.dims(B, H, L, D, d, N.BF16)
        f = N.Forward(dm, want_state=True)
        runs.append((t, f))
    say("[boundary] concurrent forwards: serial references")
    refs = []
    for t, f in runs:
        f(t["x"], t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["w_score"], t["w_mix"], b_score=t["b_score"])
        torch.cuda.synchronize()
        refs.append((f.out.clone(), f.route.clone(), f.S_final.clone()))
        f.out.zero_()
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    errors = []
    barrier = threading.Barrier(2)

    def worker(i):
        try:
            t, f = runs[i]
            s = streams[i]
            barrier.wait()
            with torch.cuda.stream(s):
                for it in range(12):
                    f(t["x"], t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["w_score"], t["w_mix"],
                      b_score=t["b_score"])
                    if it % 4 == 3:
                        s.synchronize()
                        o, r, S = refs[i]
                        if not (torch.equal(f.out, o) and torch.equal(f.route, r) and torch.equal(f.S_final, S)):
                            errors.append(f"thread {i} iteration {it}: differs from the serial run")
        except Exception as e:  # pragma: no cover - reported below
            errors.append(f"thread {i}: {e!r}")

    say("[boundary] concurrent forwards: two threads")
    th = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for x in th:
        x.start()
    for x in th:
        x.join(timeout=120)
    assert not any(x.is_alive() for x in th), "a worker thread did not finish"
    torch.cuda.synchronize()
    assert not errors, errors


def test_concurrent_nha_two_threads_two_streams():
    """Two host threads call natsl_nha_attention at the same time, each on its
    own stream with its own inputs and workspace, 8 times each; every output is
    bit-identical to the same call run alone.  Each call forks its window's
    softmax onto a helper stream that it takes from the per-device pool for
    the call, so neither call can wait on the other's events."""
    B, H, L, D, m, win = 1, 4, 4096, 128, 16, 1024
    runs = []
    for seed in (83, 84):
        inp = W.make_nha(B, H, L, D, m, io="bf16", seed=seed)
        bf = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda().to(torch.bfloat16)
        q, k, v = bf(inp["q"]), bf(inp["k"]), bf(inp["v"])
        gate = torch.from_numpy(np.ascontiguousarray(inp["gate"])).cuda()
        dm = N.dims(B, H, L, D, 64, N.BF16)
        ws = N.workspace(N.nha_workspace_size(dm, m, win), q.device)
        runs.append((dm, q, k, v, gate, ws))
    say("[boundary] concurrent NHA calls: serial references")
    refs = []
    for dm, q, k, v, gate, ws in runs:
        refs.append(N.nha_attention(dm, q, k, v, gate, win, ws=ws).clone())
        torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    errors = []
    barrier = threading.Barrier(2)

    def worker(i):
        try:
            dm, q, k, v, gate, ws = runs[i]
            s = streams[i]
            barrier.wait()
            with torch.cuda.stream(s):
                for it in range(8):
                    o = N.nha_attention(dm, q, k, v, gate, win, ws=ws, stream=s)
                    if it % 4 == 3:
                        s.synchronize()
                        if not torch.equal(o, refs[i]):
                            errors.append(f"thread {i} iteration {it}: differs from the serial run")
        except Exception as e:  # pragma: no cover - reported below
            errors.append(f"thread {i}: {e!r}")

    say("[boundary] concurrent NHA calls: two threads")
    th = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for x in th:
        x.start()
    for x in th:
        x.join(timeout=120)
    assert not any(x.is_alive() for x in th), "a worker thread did not finish"
    torch.cuda.synchronize()
    assert not errors, errors


def test_forward_128k_tokens_sampled():
    """A 131072-token bf16 D = 128 prefill (2048 chunks: a softmax tile list
    of up to 2048 entries, 2048 route bytes in the scan's LDS), 25% softmax
    chunks in bursts and singles, against the oracle: every head's n_lin, and
    out / n_sm on sampled query blocks, within the bf16 tolerance."""
    L = 131072
    wl, inp = case(1, 2, L, 128, 256, 5, routing="planted",
                   extra=dict(n_sm=512, n_burst=3, burst_total=384, min_burst=64))
    say(f"[boundary] forward L={L}")
    r_ref = O.route(inp["x"], inp["w_score"], inp["b_score"])[0]
    assert abs((r_ref == 0).mean() - 0.25) < 1e-9
    t = prefill_tensors(inp)
    dm = N.dims(1, 2, L, 128, 256, N.BF16)
    f = N.Forward(dm, debug=True, want_state=True)
    f(t["x"], t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["w_score"], t["w_mix"], b_score=t["b_score"])
    torch.cuda.synchronize()
    assert np.array_equal(f.route.cpu().numpy(), r_ref)
    blocks = [0, 1, 700, 1500, 2046, 2047]
    rows = rows_of_blocks(blocks)
    worst = 0.0
    for h in range(2):
        ref = oracle_head(inp, 0, h, r_ref[0], query_blocks=blocks)
        eo = maxerr(host(f.out[0, h])[rows], ref["out"][rows])
        es = maxerr(rmsn(host(f.o_sm[0, h]))[rows], ref["n_sm"][rows])
        el = maxerr(rmsn(host(f.o_gdn[0, h])), ref["n_lin"])
        eS = maxerr(host(f.S_final[0, h]), ref["S_final"]) / max(1.0, np.abs(ref["S_final"]).max())
        say(f"  h={h} out {eo:.3e} n_sm {es:.3e} n_lin {el:.3e} S_final rel {eS:.3e}")
        worst = max(worst, eo, es, el, eS)
    assert worst <= TOL_BF16


def test_softmax_long_tile_list_kernel_bf16_d128():
    """A prefill segment on top of a decode cache whose capacity holds more
    than 4096 chunks: the fast kernel's LDS tile list cannot take it, so the
    kernel that reads the chunk list from global memory serves bf16 D = 128.
    The segment's outputs match the oracle's one-shot prefill over prefix and
    segment (forced routes, sharp q so a wrongly masked key shows)."""
    B, H, D, d = 1, 2, 128, 256
    L0, L1 = 256, 640
    L = L0 + L1
    wl = W.Workload("case", "bf16", B, H, L, D, d, "iid", 91)
    inp = W.make_prefill(wl, routing="iid", q_scale=4.0)
    rng = np.random.default_rng(91)
    r = (rng.random((B, 1, L // 64)) < 0.5).astype(np.int32)
    r[:, :, 0] = 0
    seg = lambda lo, hi: {k: ((val[:, lo:hi] if k == "x" else val[:, :, lo:hi])
                              if k in ("x", "q", "k", "v", "alpha", "beta") else val) for k, val in inp.items()}
    s0, s1 = seg(0, L0), seg(L0, L)
    cap = 4100 * 64  # 262400 rows: more chunks than the fast kernel's 4096-entry list
    say(f"[boundary] long tile list: cache capacity {cap} rows")
    st = N.DecodeState(B, H, D, d, cap, io=torch.bfloat16)
    t0 = prefill_tensors(s0)
    dm0 = N.dims(B, H, L0, D, d, N.BF16)
    f0 = N.Forward(dm0, want_state=True)
    f0(None, t0["q"], t0["k"], t0["v"], t0["alpha"], t0["beta"], None, t0["w_mix"],
       route_override=dev(np.ascontiguousarray(r[:, :, :L0 // 64])))
    N.decode_handoff(dm0, f0.route, t0["k"], t0["v"], f0.S_final, st)
    t1 = prefill_tensors(s1)
    dm1 = N.dims(B, H, L1, D, d, N.BF16)
    f1 = N.Forward(dm1, debug=True)
    f1(None, t1["q"], t1["k"], t1["v"], t1["alpha"], t1["beta"], None, t1["w_mix"],
       route_override=dev(np.ascontiguousarray(r[:, :, L0 // 64:])), prefix=st)
    torch.cuda.synchronize()
    ref = O.forward(None, inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], None, inp["w_mix"],
                    route_override=r)
    eo = maxerr(host(f1.out), ref["out"][:, :, L0:])
    es = maxerr(rmsn(host(f1.o_sm)), ref["n_sm"][:, :, L0:])
    el = maxerr(rmsn(host(f1.o_gdn)), ref["n_lin"][:, :, L0:])
    say(f"  out {eo:.3e} n_sm {es:.3e} n_lin {el:.3e}")
    assert max(eo, es, el) <= TOL_BF16


def test_sync_check_mode_forward_and_decode(capfd):
    """Synchronous-check debug mode: with level 1 the forward and a decode
    step wait for their stream and succeed with results bit-identical to
    level 0; level 2 also names each entry point on stderr before its wait."""
    B, H, L, D, d = 1, 4, 1024, 128, 256
    wl, inp = case(B, H, L, D, d, 83)
    t = prefill_tensors(inp)
    dm = N.dims(B, H, L, D, d, N.BF16)
    f = N.Forward(dm, want_state=True)
    args = (t["x"], t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["w_score"], t["w_mix"])
    try:
        say("[boundary] sync check: level 0 reference")
        N.set_sync_check(0)
        f(*args, b_score=t["b_score"])
        torch.cuda.synchronize()
        ref = (f.out.clone(), f.route.clone(), f.S_final.clone())
        for lv in (1, 2):
            say(f"[boundary] sync check: level {lv}")
            f.out.zero_()
            N.set_sync_check(lv)
            f(*args, b_score=t["b_score"])
            # no synchronize here: level >= 1 has already waited for the stream
            assert torch.equal(f.out, ref[0]) and torch.equal(f.route, ref[1]) and torch.equal(f.S_final, ref[2])
        err = capfd.readouterr().err
        assert "natsl sync check: natsl_forward" in err
        st = N.DecodeState(B, H, D, d, cap=256)
        dd = N.dims(B, H, 256, D, d, N.BF16)
        step = N.Decode(dd, st)
        g = torch.Generator().manual_seed(5)
        mk = lambda *s: torch.randn(*s, generator=g).to("cuda")
        x, q, k, v = (mk(B, d).bfloat16(), mk(B, H, D).bfloat16(), mk(B, H, D).bfloat16(), mk(B, H, D).bfloat16())
        alpha = torch.full((B, H), 0.95, device="cuda")
        beta = torch.full((B, H), 0.5, device="cuda")
        step(x, q, k, v, alpha, beta, t["w_score"], t["w_mix"])
        assert "natsl sync check: natsl_decode_step" in capfd.readouterr().err
        assert torch.isfinite(step.out.float()).all()
    finally:
        N.set_sync_check(0)
