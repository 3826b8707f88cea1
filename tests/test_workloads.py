"""The seeded workloads have the structure their descriptions promise,
checked through the oracle's router (never through the HIP path)."""
import numpy as np
import pytest

import oracle as O
import workloads as W


@pytest.mark.parametrize("name", ["tiny", "prefill"])
def test_natural_seed_conditions(name):
    """Every chunk margin exceeds 1e-3, both routes occur, and the prefill
    workload routes 45-55% of chunks to softmax in no fixed order."""
    wl = W.WORKLOADS[name]
    inp = W.make_prefill(wl)
    r, m = O.route(inp["x"], inp["w_score"], inp["b_score"])
    assert np.abs(m).min() > 1e-3
    f = (r == O.SM).mean()
    assert 0 < f < 1
    if name == "prefill":
        assert 0.45 <= f <= 0.55


def test_long_planted_bursts():
    """25% softmax: 3 bursts totalling 96 chunks plus 32 isolated singles;
    the oracle's router reproduces the plan with margins far from zero."""
    wl = W.WORKLOADS["long"]
    inp = W.make_prefill(wl)
    plan = inp["plan"]
    r, m = O.route(inp["x"], inp["w_score"], inp["b_score"])
    np.testing.assert_array_equal(r[0, 0], plan)
    assert np.abs(m).min() > 0.1
    assert (plan == 0).sum() == 128
    runs, cur = [], 0
    for p in plan:
        if p == 0:
            cur += 1
        elif cur:
            runs.append(cur)
            cur = 0
    if cur:
        runs.append(cur)
    big = [x for x in runs if x > 1]
    assert len(big) == 3 and sum(big) == 96 and min(big) >= 16
    assert runs.count(1) == 32
    # x keeps its N(0,1) character after planting and bf16 rounding
    assert abs(inp["x"].std() - 1) < 0.01


def test_iid_planting_small():
    wl = W.WORKLOADS["prefill"]
    inp = W.make_prefill(wl, L=1024, B=2, H=2, routing="iid")
    r, m = O.route(inp["x"], inp["w_score"], inp["b_score"])
    np.testing.assert_array_equal(r[:, 0], np.broadcast_to(inp["plan"], r[:, 0].shape))
    assert np.abs(m).min() > 0.1


def test_bf16_rounding_is_rne():
    a = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5e-3], np.float32)
    r = W.round_bf16(a)
    assert r[0] == 1.0
    assert r[1] == 1.0                      # tie -> even (mantissa 0)
    assert r[2] == 1.0 + 4 * 2 ** -8        # tie -> even (rounds up)
    assert r[3] == 1.0
    assert (r.view(np.uint32) & 0xFFFF).max() == 0


def test_prefill_distributions():
    inp = W.make_prefill(W.WORKLOADS["tiny"])
    n = np.linalg.norm(inp["k"], axis=-1)
    np.testing.assert_allclose(n, 1.0, atol=1e-6)
    assert (inp["alpha"] >= 0.9).all() and (inp["alpha"] < 0.999).all()
    assert (inp["beta"] > 0).all() and (inp["beta"] < 1).all()
    assert inp["x"].dtype == np.float32


def test_decode_workload_small():
    cache, new = W.make_decode(W.WORKLOADS["decode"], B=4, H=2)
    assert cache["k"].shape[2] == 64 * 136 + 64
    nc = cache["n_committed"][:, 0]
    assert ((nc % 64) == 0).all() and (nc >= 64 * 120).all() and (nc <= 64 * 136).all()
    for b in range(4):
        n = int(nc[b])
        kk = W.bits_to_f32(cache["k"][b, :, :n])
        np.testing.assert_allclose(np.linalg.norm(kk, axis=-1), 1.0, atol=1e-2)
        assert (cache["k"][b, :, n:] == 0).all()
