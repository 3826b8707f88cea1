"""Pins for the oracle's per-head routing paths (route_groups G = H) and its
per-head mixing weights.

The pages leave the routing granularity open ("Technische Samenvatting:
Neural Attention Search Linear (NAtS-L)", Kernmechanismen 1: every chunk is
mapped to a set of scores, one per operation type).  The G = 1 paths are
pinned against library routines and closed forms in test_oracle_pins.py; the
G = H paths are pinned here to those G = 1 paths, two ways:
  * G = H with the same route for every head is bit-identical to G = 1
    (catches a G = H path that computes something other than the shared one);
  * every head of a G = H run equals a G = 1 run on that head's slice alone,
    with that head's own route, score columns and bias (catches a wrong head
    -> group mapping, a route or score column taken from another head, and
    heads leaking into each other).
"""
import numpy as np

import oracle as O

RNG = np.random.default_rng(4321)


def inputs(B=2, H=3, L=320, D=6, d=12, seed=0, alpha=(0.95, 1.0)):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, H, L, D)) * 2.0
    k = r.standard_normal((B, H, L, D))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((B, H, L, D))
    a = r.uniform(*alpha, size=(B, H, L))
    b = 1 / (1 + np.exp(-r.standard_normal((B, H, L))))
    x = r.standard_normal((B, L, d))
    return x, q, k, v, a, b


def per_head_routes(B, H, nc, seed=1):
    """Random routes in which every (sequence, group) sees both kinds and, for
    more than one group, the groups differ."""
    r = np.random.default_rng(seed)
    for _ in range(1000):
        rt = (r.random((B, H, nc)) < 0.5).astype(np.int32)
        if all(0 < rt[bb, h].sum() < nc for bb in range(B) for h in range(H)) and \
                (H == 1 or not all(np.array_equal(rt[:, 0], rt[:, h]) for h in range(H))):
            return rt
    raise RuntimeError("no route pattern found")


def sl(a, h):
    return a[:, h:h + 1]


# ---------------------------------------------------------------- branches ----
def test_softmax_groups_equal_routes_match_shared():
    x, q, k, v, a, b = inputs()
    B, H, L = q.shape[:3]
    r1 = per_head_routes(B, 1, L // 64)
    rH = np.repeat(r1, H, axis=1)
    o1, l1 = O.softmax_branch(q, k, v, r1, with_lse=True)
    oH, lH = O.softmax_branch(q, k, v, rH, with_lse=True)
    np.testing.assert_array_equal(o1, oH)
    np.testing.assert_array_equal(l1, lH)


def test_softmax_groups_head_by_head():
    x, q, k, v, a, b = inputs()
    B, H, L = q.shape[:3]
    rH = per_head_routes(B, H, L // 64)
    oH, lH = O.softmax_branch(q, k, v, rH, with_lse=True)
    for h in range(H):
        oh, lh = O.softmax_branch(sl(q, h), sl(k, h), sl(v, h), rH[:, h:h + 1], with_lse=True)
        np.testing.assert_array_equal(oH[:, h:h + 1], oh, err_msg=f"head {h}")
        np.testing.assert_array_equal(lH[:, h:h + 1], lh)
    # the brute-force twin reads the group mapping on its own; same values
    np.testing.assert_allclose(O.softmax_branch_bruteforce(q, k, v, rH), oH, atol=1e-12)


def test_gdn_groups_equal_routes_match_shared():
    x, q, k, v, a, b = inputs()
    B, H, L = q.shape[:3]
    S0 = RNG.standard_normal((B, H, q.shape[3], v.shape[3]))
    r1 = per_head_routes(B, 1, L // 64, seed=2)
    rH = np.repeat(r1, H, axis=1)
    o1, s1 = O.gdn_branch(q, k, v, a, b, r1, S_init=S0)
    oH, sH = O.gdn_branch(q, k, v, a, b, rH, S_init=S0)
    np.testing.assert_array_equal(o1, oH)
    np.testing.assert_array_equal(s1, sH)


def test_gdn_groups_head_by_head():
    """alpha ~ U(0.95, 1) keeps old state visible, so a carried state taken
    from another head's route shows in the outputs."""
    x, q, k, v, a, b = inputs()
    B, H, L = q.shape[:3]
    S0 = RNG.standard_normal((B, H, q.shape[3], v.shape[3]))
    rH = per_head_routes(B, H, L // 64, seed=3)
    oH, sH = O.gdn_branch(q, k, v, a, b, rH, S_init=S0)
    for h in range(H):
        oh, s_h = O.gdn_branch(sl(q, h), sl(k, h), sl(v, h), sl(a, h), sl(b, h), rH[:, h:h + 1],
                               S_init=S0[:, h:h + 1])
        np.testing.assert_array_equal(oH[:, h:h + 1], oh, err_msg=f"head {h}")
        np.testing.assert_array_equal(sH[:, h:h + 1], s_h)
    np.testing.assert_allclose(O.gdn_branch_bruteforce(q, k, v, a, b, rH, S_init=S0), oH, atol=1e-12)


def test_gdn_backward_groups_head_by_head():
    x, q, k, v, a, b = inputs(L=192, D=4)
    B, H, L = q.shape[:3]
    rH = per_head_routes(B, H, L // 64, seed=4)
    d_o = RNG.standard_normal(v.shape)
    dS = RNG.standard_normal((B, H, 4, 4))
    gH = O.gdn_branch_backward(q, k, v, a, b, rH, d_o, dS_final=dS)
    for h in range(H):
        gh = O.gdn_branch_backward(sl(q, h), sl(k, h), sl(v, h), sl(a, h), sl(b, h), rH[:, h:h + 1],
                                   sl(d_o, h), dS_final=sl(dS, h))
        for full, one in zip(gH, gh):
            np.testing.assert_array_equal(full[:, h:h + 1], one)


def test_softmax_backward_groups_head_by_head():
    x, q, k, v, a, b = inputs(L=192, D=4)
    B, H, L = q.shape[:3]
    rH = per_head_routes(B, H, L // 64, seed=5)
    d_o = RNG.standard_normal(v.shape)
    gH = O.softmax_branch_backward(q, k, v, rH, d_o)
    for h in range(H):
        gh = O.softmax_branch_backward(sl(q, h), sl(k, h), sl(v, h), rH[:, h:h + 1], sl(d_o, h))
        for full, one in zip(gH, gh):
            np.testing.assert_array_equal(full[:, h:h + 1], one)


# ------------------------------------------------------------------- merge ----
def test_merge_per_head_weights_head_by_head():
    """W_mix [H, Dk, 2]: head h mixes with its own matrix, exactly as a shared
    W_mix equal to that matrix mixes head h."""
    B, H, L, D = 2, 3, 5, 6
    q = RNG.standard_normal((B, H, L, D))
    o_sm = RNG.standard_normal((B, H, L, D)) * 3
    o_gdn = RNG.standard_normal((B, H, L, D)) * 0.2
    wm = RNG.normal(0, 0.5, (H, D, 2))
    gs, gl = RNG.uniform(0.5, 1.5, D), RNG.uniform(0.5, 1.5, D)
    out, n_sm, n_lin, w = O.merge(q, o_sm, o_gdn, wm, gs, gl)
    # the per-head scores are an einsum, the shared ones a matmul: the two sum
    # in different orders, so they agree to rounding, not bit for bit
    for h in range(H):
        o1, _, _, w1 = O.merge(sl(q, h), sl(o_sm, h), sl(o_gdn, h), wm[h], gs, gl)
        np.testing.assert_allclose(out[:, h:h + 1], o1, rtol=0, atol=1e-14)
        np.testing.assert_allclose(w[:, h:h + 1], w1, rtol=0, atol=1e-15)
    # and all heads sharing one matrix equals the shared form
    out_s = O.merge(q, o_sm, o_gdn, np.repeat(wm[:1], H, axis=0), gs, gl)[0]
    np.testing.assert_allclose(out_s, O.merge(q, o_sm, o_gdn, wm[0], gs, gl)[0], rtol=0, atol=1e-14)
    # a head's weights depend on its own matrix: giving head 0 head 1's matrix changes them
    assert not np.allclose(w[:, 0], O.mix_weights(sl(q, 0), wm[1])[:, 0])


# ------------------------------------------------------------------ router ----
def test_router_groups_head_by_head_and_shared():
    """Group g scores with columns (2g, 2g+1) and bias (2g, 2g+1); the same
    columns in every group reproduce the shared router."""
    B, L, d, G = 2, 320, 12, 3
    x = RNG.standard_normal((B, L, d))
    w = RNG.normal(0, 0.5, (d, 2 * G))
    bias = RNG.normal(0, 0.1, 2 * G)
    rG, mG = O.route(x, w, bias, groups=G)
    for g in range(G):
        r1, m1 = O.route(x, w[:, 2 * g:2 * g + 2], bias[2 * g:2 * g + 2])
        np.testing.assert_array_equal(rG[:, g:g + 1], r1)
        np.testing.assert_array_equal(mG[:, g:g + 1], m1)
    rS, _ = O.route(x, np.tile(w[:, :2], (1, G)), np.tile(bias[:2], G), groups=G)
    np.testing.assert_array_equal(rS, np.repeat(O.route(x, w[:, :2], bias[:2])[0], G, axis=1))


# ------------------------------------------------------------------ decode ----
def _decode_case(seed=6):
    B, H, L, D, d = 2, 3, 256, 5, 12
    x, q, k, v, a, b = inputs(B=B, H=H, L=L, D=D, d=d, seed=seed)
    # per-group score columns chosen so the groups route differently
    w = RNG.normal(0, 0.6, (d, 2 * H))
    bias = RNG.normal(0, 0.05, 2 * H)
    wm = RNG.normal(0, 0.3, (H, D, 2))
    return B, H, L, D, d, x, q, k, v, a, b, w, bias, wm


def test_build_cache_groups_head_by_head():
    B, H, L, D, d, x, q, k, v, a, b, w, bias, wm = _decode_case()
    n0 = 160  # two complete chunks and an open half chunk
    cG = O.build_cache(x[:, :n0], k[:, :, :n0], v[:, :, :n0], a[:, :, :n0], b[:, :, :n0], w, bias, cap=L,
                       groups=H)
    for h in range(H):
        c1 = O.build_cache(x[:, :n0], sl(k, h)[:, :, :n0], sl(v, h)[:, :, :n0], sl(a, h)[:, :, :n0],
                           sl(b, h)[:, :, :n0], w[:, 2 * h:2 * h + 2], bias[2 * h:2 * h + 2], cap=L)
        for key in ("k", "v", "S_carry", "S_work"):
            np.testing.assert_array_equal(cG[key][:, h:h + 1], c1[key], err_msg=f"{key} head {h}")
        for key in ("n_committed", "n_open", "x_sum"):
            np.testing.assert_array_equal(cG[key][:, h:h + 1], c1[key], err_msg=f"{key} head {h}")


def test_decode_groups_head_by_head():
    """150 decode steps from a 100-token prefix with G = H (own score columns,
    bias and W_mix per head) equal, head by head, the G = 1 decode of that
    head alone; the heads' routes differ somewhere, so a route taken from the
    wrong group changes the cache."""
    B, H, L, D, d, x, q, k, v, a, b, w, bias, wm = _decode_case()
    n0 = 100
    cG = O.build_cache(x[:, :n0], k[:, :, :n0], v[:, :, :n0], a[:, :, :n0], b[:, :, :n0], w, bias, cap=L,
                       groups=H)
    c1 = [O.build_cache(x[:, :n0], sl(k, h)[:, :, :n0], sl(v, h)[:, :, :n0], sl(a, h)[:, :, :n0],
                        sl(b, h)[:, :, :n0], w[:, 2 * h:2 * h + 2], bias[2 * h:2 * h + 2], cap=L) for h in range(H)]
    routes_seen = []
    for t in range(n0, L):
        outG, brG, cG = O.decode_step(cG, x[:, t], q[:, :, t], k[:, :, t], v[:, :, t], a[:, :, t], b[:, :, t],
                                      w, wm, bias)
        for h in range(H):
            out1, br1, c1[h] = O.decode_step(c1[h], x[:, t], sl(q, h)[:, :, t], sl(k, h)[:, :, t],
                                             sl(v, h)[:, :, t], sl(a, h)[:, :, t], sl(b, h)[:, :, t],
                                             w[:, 2 * h:2 * h + 2], wm[h], bias[2 * h:2 * h + 2])
            # the mixing scores sum in a different order for per-head W_mix (see the merge pin)
            np.testing.assert_allclose(outG[:, h:h + 1], out1, rtol=0, atol=1e-13, err_msg=f"t={t} head {h}")
            np.testing.assert_array_equal(brG["o_sm"][:, h:h + 1], br1["o_sm"])
            np.testing.assert_array_equal(brG["o_gdn"][:, h:h + 1], br1["o_gdn"])
            np.testing.assert_array_equal(brG["routes"][:, h:h + 1], br1["routes"])
        if (brG["routes"] >= 0).any():
            routes_seen.append(brG["routes"].copy())
    for h in range(H):
        for key in ("k", "v", "S_carry", "S_work", "n_committed", "n_open", "x_sum"):
            np.testing.assert_array_equal(cG[key][:, h:h + 1], c1[h][key], err_msg=f"{key} head {h}")
    rs = np.stack(routes_seen)  # [events, B, H]
    assert any(not np.array_equal(rs[..., 0], rs[..., h]) for h in range(1, H)), "groups never routed differently"
    assert set(np.unique(rs)) == {O.SM, O.LIN}


def test_decode_groups_equal_routes_match_shared():
    """G = H whose groups all use the same score columns is the shared (G = 1)
    decode, bit for bit."""
    B, H, L, D, d, x, q, k, v, a, b, w, bias, wm = _decode_case(seed=8)
    w1, b1 = w[:, :2], bias[:2]
    wG, bG = np.tile(w1, (1, H)), np.tile(b1, H)
    n0 = 100
    c1 = O.build_cache(x[:, :n0], k[:, :, :n0], v[:, :, :n0], a[:, :, :n0], b[:, :, :n0], w1, b1, cap=L)
    cG = O.build_cache(x[:, :n0], k[:, :, :n0], v[:, :, :n0], a[:, :, :n0], b[:, :, :n0], wG, bG, cap=L, groups=H)
    for t in range(n0, L):
        o1, br1, c1 = O.decode_step(c1, x[:, t], q[:, :, t], k[:, :, t], v[:, :, t], a[:, :, t], b[:, :, t],
                                    w1, wm[0], b1)
        oG, brG, cG = O.decode_step(cG, x[:, t], q[:, :, t], k[:, :, t], v[:, :, t], a[:, :, t], b[:, :, t],
                                    wG, wm[0], bG)
        np.testing.assert_array_equal(o1, oG)
        np.testing.assert_array_equal(np.repeat(br1["routes"], H, axis=1), brG["routes"])
    np.testing.assert_array_equal(c1["S_carry"], cG["S_carry"])
    np.testing.assert_array_equal(np.repeat(c1["n_committed"], H, axis=1), cG["n_committed"])
