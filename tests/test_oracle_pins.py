"""Pins for the fp64 oracle, against facts the pages and mathematics fix
rather than against the oracle itself.

Each test names the mistake it is there to catch.  Page references:
  [NL] "Technische Samenvatting: Neural Attention Search Linear (NAtS-L)",
       Kernmechanismen 1-4;  [DE] the German explainer, "Die Chunking-Strategie".
"""
import numpy as np
import pytest
import torch

import oracle as O
from tests.chunkwise_model import gdn_chunkwise, gdn_chunkwise_backward

RNG = np.random.default_rng(1234)


def rand_inputs(B=1, H=2, L=256, D=8, d=16, seed=0, alpha=(0.9, 0.999), chunk=64):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, H, L, D))
    k = r.standard_normal((B, H, L, D))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((B, H, L, D))
    a = r.uniform(*alpha, size=(B, H, L))
    b = 1 / (1 + np.exp(-r.standard_normal((B, H, L))))
    x = r.standard_normal((B, L, d))
    return x, q, k, v, a, b


def sdpa(q, k, v, causal=True):
    """torch's CPU scaled_dot_product_attention in fp64 (library routine)."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    return torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=causal).numpy()


# ---------------------------------------------------------------- router ----
def test_router_tie_goes_to_softmax():
    """Equal score columns give an exact tie on every chunk; the first-maximum
    rule assigns softmax.  Catches a swapped comparison (> instead of >=)."""
    x = RNG.standard_normal((2, 256, 16))
    w = np.repeat(RNG.standard_normal((16, 1)), 2, axis=1)
    r, m = O.route(x, w)
    assert np.all(m == 0.0) and np.all(r == O.SM)


def test_router_mean_pool_constant_chunks():
    """A chunk whose 64 tokens all equal z pools to z, so its scores are
    z . W + b exactly.  Catches sum-instead-of-mean, a wrong chunk size
    ([DE] Chunking-Strategie: 64) and a missing bias."""
    d = 8
    z = RNG.standard_normal((3, d))
    x = np.repeat(z, 64, axis=0)[None]  # [1, 192, d]
    w = RNG.standard_normal((d, 2))
    b = np.array([0.25, -0.5])
    s = O.route_scores(x, w, b)
    np.testing.assert_allclose(s[0, 0], z @ w + b, rtol=0, atol=1e-14)


def test_router_linear_shift_moves_margin_exactly():
    """Adding c * u (u = dw/|dw|^2, dw = W[:,0]-W[:,1]) to every token of a
    chunk moves its margin by exactly c (linearity of mean-pool + linear
    layer).  Catches a transposed W, wrong column order (margin moves by -c)
    and per-token instead of per-chunk scoring."""
    x = RNG.standard_normal((1, 256, 32))
    w = RNG.normal(0, 0.02, (32, 2))
    dw = w[:, 0] - w[:, 1]
    u = dw / (dw @ dw)
    c = np.array([0.7, -1.3, 0.0, 2.0])
    x2 = x + np.repeat(c, 64)[None, :, None] * u[None, None, :]
    _, m1 = O.route(x, w)
    _, m2 = O.route(x2, w)
    np.testing.assert_allclose(m2 - m1, c[None, None, :], atol=1e-12)


def test_router_groups_use_their_columns():
    """With groups=2 the second group's scores come from columns 2 and 3."""
    x = RNG.standard_normal((1, 128, 8))
    w = RNG.standard_normal((8, 4))
    s = O.route_scores(x, w, groups=2)
    s0 = O.route_scores(x, w[:, :2])
    s1 = O.route_scores(x, w[:, 2:])
    np.testing.assert_array_equal(s[:, 0], s0[:, 0])
    np.testing.assert_array_equal(s[:, 1], s1[:, 0])


def test_compaction():
    r = np.array([[[1, 0, 0, 1, 0]]], dtype=np.int32)
    sel, nsb = O.compact(r)
    assert sel[0, 0].tolist() == [1, 2, 4, -1, -1]
    assert nsb[0, 0].tolist() == [0, 0, 1, 2, 2, 3]


# --------------------------------------------------------------- softmax ----
def test_softmax_all_sm_is_full_causal_attention():
    """All chunks routed to softmax keeps every KV: the branch is ordinary
    causal attention ([NL] Kernmechanismen 3).  Pinned to torch's SDPA."""
    _, q, k, v, _, _ = rand_inputs(B=2, H=2, L=256, D=16)
    r = np.zeros((2, 1, 4), np.int32)
    o = O.softmax_branch(q, k, v, r)
    np.testing.assert_allclose(o, sdpa(q, k, v), atol=1e-12, rtol=0)


def test_softmax_all_lin_is_blockdiagonal_attention():
    """All chunks routed linear: each chunk only sees its own causal prefix,
    i.e. causal attention run separately inside every 64-token chunk."""
    _, q, k, v, _, _ = rand_inputs(B=1, H=2, L=256, D=16)
    r = np.ones((1, 1, 4), np.int32)
    o = O.softmax_branch(q, k, v, r)
    ref = np.concatenate([sdpa(q[:, :, s:s + 64], k[:, :, s:s + 64], v[:, :, s:s + 64])
                          for s in range(0, 256, 64)], axis=2)
    np.testing.assert_allclose(o, ref, atol=1e-12, rtol=0)


def test_softmax_matches_bruteforce_mixed_routes():
    """Explicit per-query key lists with a softmax over exactly those keys.
    Small chunk (8) so several chunks of each route fit a tiny input.
    Catches masking the wrong chunks or dropping the own-chunk prefix."""
    _, q, k, v, _, _ = rand_inputs(B=1, H=2, L=48, D=5)
    r = np.array([[[1, 0, 1, 1, 0, 1]]], np.int32)
    o = O.softmax_branch(q, k, v, r, chunk=8)
    ob = O.softmax_branch_bruteforce(q, k, v, r, chunk=8)
    np.testing.assert_allclose(o, ob, atol=1e-13, rtol=0)


def test_softmax_lse_all_sm():
    from scipy.special import logsumexp
    _, q, k, v, _, _ = rand_inputs(B=1, H=1, L=128, D=8)
    r = np.zeros((1, 1, 2), np.int32)
    _, lse = O.softmax_branch(q, k, v, r, with_lse=True)
    z = (q[0, 0] @ k[0, 0].T) / np.sqrt(8)
    z = np.where(np.tril(np.ones((128, 128), bool)), z, -np.inf)
    np.testing.assert_allclose(lse[0, 0], logsumexp(z, axis=1), atol=1e-12)


def test_single_chunk_is_route_independent():
    """L = 64: one chunk only ever sees itself, whatever its route."""
    x, q, k, v, a, b = rand_inputs(B=1, H=1, L=64, D=8)
    for name, fn in (("sm", lambda r: O.softmax_branch(q, k, v, r)),
                     ("gdn", lambda r: O.gdn_branch(q, k, v, a, b, r)[0])):
        o0 = fn(np.zeros((1, 1, 1), np.int32))
        o1 = fn(np.ones((1, 1, 1), np.int32))
        np.testing.assert_array_equal(o0, o1, err_msg=name)


# ------------------------------------------------------------------- GDN ----
def pure_gdn(q, k, v, a, b):
    """Gated delta rule with no routing at all, written in torch fp64 as
    S_t = S_{t-1} diag... in the (Dv x Dk) value-major convention of the
    published Gated DeltaNet: M_t = a_t M_{t-1} (I - b_t k k^T) + b_t v k^T,
    o_t = M_t q_t.  Independent of the oracle's key-major code."""
    q, k, v, a, b = (torch.from_numpy(np.ascontiguousarray(t)) for t in (q, k, v, a, b))
    B, H, L, D = q.shape
    M = torch.zeros(B, H, v.shape[-1], D, dtype=torch.float64)
    eye = torch.eye(D, dtype=torch.float64)
    out = torch.zeros(B, H, L, v.shape[-1], dtype=torch.float64)
    for t in range(L):
        kt = k[:, :, t]
        proj = eye - b[:, :, t, None, None] * kt[..., :, None] * kt[..., None, :]
        M = a[:, :, t, None, None] * (M @ proj) + b[:, :, t, None, None] * v[:, :, t, :, None] * kt[..., None, :]
        out[:, :, t] = (M @ q[:, :, t, :, None])[..., 0]
    return out.numpy(), M.transpose(-1, -2).numpy()


def test_gdn_all_lin_is_pure_gated_deltanet():
    """No chunk rolled back: the branch is the plain gated delta rule."""
    x, q, k, v, a, b = rand_inputs(B=2, H=2, L=192, D=6)
    r = np.ones((2, 1, 3), np.int32)
    o, S = O.gdn_branch(q, k, v, a, b, r)
    ref, Sref = pure_gdn(q, k, v, a, b)
    np.testing.assert_allclose(o, ref, atol=1e-12, rtol=0)
    np.testing.assert_allclose(S, Sref, atol=1e-12, rtol=0)


def test_gdn_all_sm_restarts_every_chunk():
    """Every chunk rolled back: each chunk runs the gated delta rule from the
    initial state (zero here), and the carried state never changes."""
    x, q, k, v, a, b = rand_inputs(B=1, H=2, L=192, D=6)
    r = np.zeros((1, 1, 3), np.int32)
    o, S = O.gdn_branch(q, k, v, a, b, r)
    for s in range(0, 192, 64):
        ref, _ = pure_gdn(q[:, :, s:s + 64], k[:, :, s:s + 64], v[:, :, s:s + 64],
                          a[:, :, s:s + 64], b[:, :, s:s + 64])
        np.testing.assert_allclose(o[:, :, s:s + 64], ref, atol=1e-12, rtol=0)
    assert np.all(S == 0)


def test_gdn_bruteforce_bitexact():
    """Rollback == rerunning from scratch over only the surviving tokens.
    Same operations in the same order, so equality is bit-exact.  Small
    chunk (8) and a nonzero initial state."""
    x, q, k, v, a, b = rand_inputs(B=1, H=2, L=32, D=5, alpha=(0.5, 1.0))
    S0 = RNG.standard_normal((1, 2, 5, 5))
    r = np.array([[[1, 0, 1, 0]]], np.int32)
    o, _ = O.gdn_branch(q, k, v, a, b, r, S_init=S0, chunk=8)
    ob = O.gdn_branch_bruteforce(q, k, v, a, b, r, S_init=S0, chunk=8)
    np.testing.assert_array_equal(o, ob)


def test_gdn_beta_zero_only_decays():
    """beta = 0 writes and erases nothing: S_t = (prod alpha) S_init, and with
    all chunks linear the final state is the full product times S_init."""
    x, q, k, v, a, _ = rand_inputs(B=1, H=1, L=128, D=4)
    b = np.zeros_like(a)
    S0 = RNG.standard_normal((1, 1, 4, 4))
    o, S = O.gdn_branch(q, k, v, a, b, np.ones((1, 1, 2), np.int32), S_init=S0)
    np.testing.assert_allclose(S, np.prod(a) * S0, rtol=1e-12)
    pa = np.cumprod(a[0, 0])
    np.testing.assert_allclose(o[0, 0], pa[:, None] * (q[0, 0] @ S0[0, 0]), rtol=1e-12, atol=1e-14)


def test_gdn_orthonormal_keys_closed_form_with_rollback():
    """beta = 1 and orthonormal keys (Dk >= L) make the erase term vanish, so
    S_t = alpha_t S_{t-1} + k_t v_t^T: o_t = sum over surviving tokens i <= t
    of (prod of alpha_j over surviving j in (i, t]) (q_t . k_i) v_i, where the
    surviving tokens are those of earlier linear chunks plus t's own chunk
    prefix.  Catches a dropped decay, decays not rolled back with the state
    ([NL] Kernmechanismen 3: reset to the chunk start), and rollback to zero
    instead of to the chunk start."""
    L, C = 32, 8
    Dk = 32
    Q = np.linalg.qr(RNG.standard_normal((Dk, Dk)))[0]
    k = Q[:L][None, None]  # orthonormal rows
    q = RNG.standard_normal((1, 1, L, Dk))
    v = RNG.standard_normal((1, 1, L, 3))
    a = RNG.uniform(0.5, 1.0, (1, 1, L))
    b = np.ones((1, 1, L))
    r = np.array([[[1, 0, 0, 1]]], np.int32)
    o, _ = O.gdn_branch(q, k, v, a, b, r, chunk=C)
    for t in range(L):
        ct = t // C
        surv = [i for i in range(t + 1) if i // C == ct or r[0, 0, i // C] == 1]
        ref = np.zeros(3)
        for i in surv:
            decay = np.prod([a[0, 0, j] for j in surv if i < j <= t])
            ref += decay * (q[0, 0, t] @ k[0, 0, i]) * v[0, 0, i]
        np.testing.assert_allclose(o[0, 0, t], ref, atol=1e-12)


def test_gdn_repeated_key_is_exponential_average():
    """One key repeated, alpha = 1: k^T S follows r_t = (1 - beta_t) r_{t-1}
    + beta_t v_t (the delta rule overwrites what k retrieves); reading out
    with q = k returns r_t.  Catches beta applied to the decay or a missing
    erase term."""
    L, D = 64, 6
    kk = RNG.standard_normal(D)
    kk /= np.linalg.norm(kk)
    k = np.tile(kk, (1, 1, L, 1))
    q = k.copy()
    v = RNG.standard_normal((1, 1, L, 2))
    a = np.ones((1, 1, L))
    b = RNG.uniform(0.1, 0.9, (1, 1, L))
    o, _ = O.gdn_branch(q, k, v, a, b, np.ones((1, 1, 1), np.int32))
    rr = np.zeros(2)
    for t in range(L):
        rr = (1 - b[0, 0, t]) * rr + b[0, 0, t] * v[0, 0, t]
        np.testing.assert_allclose(o[0, 0, t], rr, atol=1e-12)


def test_chunkwise_algebra_matches_oracle():
    """The UT/WY chunkwise form the kernels use reproduces the per-token
    oracle (mixed routes, nonzero initial state, D = 16, chunk 64)."""
    x, q, k, v, a, b = rand_inputs(B=1, H=2, L=320, D=16, alpha=(0.8, 1.0))
    S0 = RNG.standard_normal((1, 2, 16, 16)) * 0.1
    r = np.array([[[1, 0, 1, 1, 0]]], np.int32)
    o, S = O.gdn_branch(q, k, v, a, b, r, S_init=S0)
    oc, Sc = gdn_chunkwise(q, k, v, a, b, r, S_init=S0)
    np.testing.assert_allclose(oc, o, atol=1e-11)
    np.testing.assert_allclose(Sc, S, atol=1e-11)


def test_chunkwise_gradient_algebra_matches_oracle():
    """The chunkwise gradient the kernels use (the chunk form's derivative,
    chunk by chunk in reverse: a backward state scan over chunks, then every
    chunk's token gradients from its start state and the carried gradient)
    reproduces the oracle's per-token reverse sweep, gate derivatives
    included (mixed routes, nonzero initial state and final-state gradient)."""
    r = np.random.default_rng(41)
    B, H, L, D = 1, 2, 320, 8
    q = r.standard_normal((B, H, L, D))
    k = r.standard_normal((B, H, L, D))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((B, H, L, D))
    a = r.uniform(0.8, 1.0, (B, H, L))
    b = 1 / (1 + np.exp(-r.standard_normal((B, H, L))))
    route = np.array([[[1, 0, 1, 1, 0]]], np.int32)
    d_o = r.standard_normal((B, H, L, D))
    S0 = r.standard_normal((B, H, D, D)) * 0.3
    dSf = r.standard_normal((B, H, D, D))
    ref = O.gdn_branch_backward(q, k, v, a, b, route, d_o, S_init=S0, dS_final=dSf, with_gate=True)
    got = gdn_chunkwise_backward(q, k, v, a, b, route, d_o, S_init=S0, dS_final=dSf)
    for name, x, y in zip(("dq", "dk", "dv", "dalpha", "dbeta", "dS_init", "dgate"), got, ref):
        np.testing.assert_allclose(x, y, atol=1e-11 * max(1.0, np.abs(y).max()), err_msg=name)


# ----------------------------------------------------------------- merge ----
def test_merge_hand_example():
    """D = 2 worked by hand: o_sm = (3, 4) has RMS sqrt(12.5), o_gdn = (1, -1)
    has RMS 1; W_mix = 0 gives weights (1/2, 1/2); gains (2, 1) and (1, 1)."""
    q = np.array([[[[0.3, -0.7]]]])
    o_sm = np.array([[[[3.0, 4.0]]]])
    o_gdn = np.array([[[[1.0, -1.0]]]])
    out, n_sm, n_lin, w = O.merge(q, o_sm, o_gdn, np.zeros((2, 2)), g_sm=np.array([2.0, 1.0]), eps=0.0)
    r = np.sqrt(12.5)
    np.testing.assert_allclose(n_sm[0, 0, 0], [6 / r, 4 / r], atol=1e-15)
    np.testing.assert_allclose(n_lin[0, 0, 0], [1.0, -1.0], atol=1e-15)
    np.testing.assert_allclose(w[0, 0, 0], [0.5, 0.5], atol=1e-15)
    np.testing.assert_allclose(out[0, 0, 0], [0.5 * (6 / r + 1), 0.5 * (4 / r - 1)], atol=1e-15)


def test_merge_weights_follow_q():
    """q . W_mix = (z0, z1): weights are the logistic of z0 - z1, column 0
    weighting the softmax branch.  Catches swapped mixing columns."""
    q = np.array([[[[1.0, 0.0]]]])
    w_mix = np.array([[2.0, 0.0], [0.0, 0.0]])
    o_sm = np.array([[[[1.0, 1.0]]]])
    o_gdn = np.array([[[[-1.0, -1.0]]]])
    out, _, _, w = O.merge(q, o_sm, o_gdn, w_mix, eps=0.0)
    s = 1 / (1 + np.exp(-2.0))
    np.testing.assert_allclose(w[0, 0, 0], [s, 1 - s], atol=1e-15)
    np.testing.assert_allclose(out[0, 0, 0], [2 * s - 1] * 2, atol=1e-15)


def test_merge_rms_is_one():
    o = RNG.standard_normal((1, 2, 5, 16)) * 7
    n = O.rmsnorm(o, eps=0.0)
    np.testing.assert_allclose(np.sqrt((n ** 2).mean(-1)), 1.0, atol=1e-14)


def test_rmsnorm_eps_inside_sqrt():
    """eps is added to the mean square before the square root: a vector of
    entries 1e-3 with eps = 1e-6 normalises to 1e-3 / sqrt(2e-6) = 1/sqrt(2)
    per entry.  Catches eps added after the square root."""
    o = np.full((1, 1, 1, 4), 1e-3)
    n = O.rmsnorm(o, eps=1e-6)
    np.testing.assert_allclose(n, 1 / np.sqrt(2.0), rtol=1e-12)


# ------------------------------------------------------------ end to end ----
def layer(x, q, k, v, a, b, w_score, w_mix, **kw):
    return O.forward(x, q, k, v, a, b, w_score, w_mix, **kw)


def test_last_chunk_route_does_not_matter():
    """A chunk's own outputs never depend on its own route (its outputs see
    its own tokens through both branches either way), so flipping the last
    chunk's route leaves every output bit-identical."""
    x, q, k, v, a, b = rand_inputs(B=1, H=2, L=256, D=8, d=16)
    w_mix = RNG.normal(0, 0.1, (8, 2))
    r = np.array([[[0, 1, 0, 1]]], np.int32)
    r2 = r.copy()
    r2[..., -1] = 0
    o1 = layer(x, q, k, v, a, b, None, w_mix, route_override=r)["out"]
    o2 = layer(x, q, k, v, a, b, None, w_mix, route_override=r2)["out"]
    np.testing.assert_array_equal(o1, o2)


def test_causality():
    """Perturbing every token after position t (inputs and router input)
    leaves all outputs up to t bit-identical."""
    x, q, k, v, a, b = rand_inputs(B=1, H=2, L=256, D=8, d=16)
    w_score = RNG.normal(0, 0.5, (16, 2))
    w_mix = RNG.normal(0, 0.1, (8, 2))
    t = 150
    outs = []
    for pert in (0.0, 1.0):
        xs = [arr.copy() for arr in (x, q, k, v, a, b)]
        xs[0][:, t + 1:] += pert
        for arr in xs[1:4]:
            arr[:, :, t + 1:] += pert
        xs[4][:, :, t + 1:] *= 0.5 if pert else 1.0
        outs.append(layer(*xs, w_score, w_mix)["out"])
    np.testing.assert_array_equal(outs[0][:, :, :t + 1], outs[1][:, :, :t + 1])


def test_decode_equals_prefill():
    """Prefill a 96-token prefix, decode 160 more tokens one at a time
    (crossing chunk completions of both routes): every decoded output equals
    the prefill output of the full 256-token sequence at that position."""
    B, H, L, D, d = 2, 2, 256, 8, 16
    x, q, k, v, a, b = rand_inputs(B=B, H=H, L=L, D=D, d=d, seed=5)
    w_score = RNG.normal(0, 0.5, (d, 2))
    w_mix = RNG.normal(0, 0.1, (D, 2))
    full = layer(x, q, k, v, a, b, w_score, w_mix)
    assert 0 < (full["route"] == O.SM).mean() < 1
    n0 = 96
    cache = O.build_cache(x[:, :n0], k[:, :, :n0], v[:, :, :n0], a[:, :, :n0], b[:, :, :n0],
                          w_score, cap=L)
    seen_routes = set()
    for t in range(n0, L):
        out, br, cache = O.decode_step(cache, x[:, t], q[:, :, t], k[:, :, t], v[:, :, t],
                                       a[:, :, t], b[:, :, t], w_score, w_mix)
        np.testing.assert_allclose(out, full["out"][:, :, t], atol=1e-12, err_msg=f"t={t}")
        np.testing.assert_allclose(br["o_gdn"], full["o_gdn"][:, :, t], atol=1e-12)
        seen_routes.update(int(r) for r in br["routes"].ravel() if r >= 0)
    assert seen_routes == {O.SM, O.LIN}
    # the cache after the last token equals a cache built from the whole sequence
    ref = O.build_cache(x, k, v, a, b, w_score, cap=L)
    np.testing.assert_array_equal(cache["n_committed"], ref["n_committed"])
    np.testing.assert_allclose(cache["S_carry"], ref["S_carry"], atol=1e-12)


def test_decode_capacity_flag():
    """A full cache sets the error flag instead of writing past its end."""
    B, H, D, d = 1, 1, 4, 8
    cache = O.empty_cache(B, H, D, d, cap=2)
    cache["n_committed"][:] = 2
    args = [RNG.standard_normal(s) for s in ((B, d), (B, H, D), (B, H, D), (B, H, D))]
    _, _, c2 = O.decode_step(cache, *args, np.full((B, H), 0.9), np.full((B, H), 0.5),
                             RNG.standard_normal((d, 2)), np.zeros((D, 2)))
    assert c2["err"] == 1


# ------------------------------------------------- softmax branch gradient ----
def _sm_loss(q, k, v, r, d_o):
    return float(np.sum(d_o * O.softmax_branch(q, k, v, r)))


def test_softmax_backward_finite_differences():
    """Central differences of <d_o, softmax_branch(q, k, v)> on a 3-chunk case
    whose middle chunk is linear (the last chunk's queries skip it): catches a
    dropped delta term, a transposed product, or a gradient leaking into
    masked keys."""
    _, q, k, v, _, _ = rand_inputs(B=1, H=2, L=192, D=4, seed=21)
    r = np.array([[[O.SM, O.LIN, O.SM]]])
    d_o = np.random.default_rng(22).standard_normal(v.shape)
    dq, dk, dv = O.softmax_branch_backward(q, k, v, r, d_o)
    rng = np.random.default_rng(23)
    eps = 1e-6
    for name, arr, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(12):
            idx = tuple(rng.integers(0, s) for s in arr.shape)
            args = {"q": q, "k": k, "v": v}
            plus, minus = {n: a.copy() for n, a in args.items()}, {n: a.copy() for n, a in args.items()}
            plus[name][idx] += eps
            minus[name][idx] -= eps
            fd = (_sm_loss(plus["q"], plus["k"], plus["v"], r, d_o) -
                  _sm_loss(minus["q"], minus["k"], minus["v"], r, d_o)) / (2 * eps)
            assert abs(fd - grad[idx]) <= 1e-7 * max(1.0, abs(fd)), (name, idx, fd, grad[idx])
    # the keys of the linear chunk get a gradient only from their own chunk's
    # queries: zeroing the later queries' upstream gradient leaves it unchanged
    d_o2 = d_o.copy()
    d_o2[:, :, 128:] = 0.0
    _, dk2, dv2 = O.softmax_branch_backward(q, k, v, r, d_o2)
    np.testing.assert_allclose(dk2[:, :, 64:128], dk[:, :, 64:128], atol=1e-14)
    np.testing.assert_allclose(dv2[:, :, 64:128], dv[:, :, 64:128], atol=1e-14)


def _sdpa_grads(q, k, v, d_o):
    """dq, dk, dv of torch's fp64 causal scaled_dot_product_attention
    (library routine and autograd)."""
    t = [torch.from_numpy(np.ascontiguousarray(a)).requires_grad_(True) for a in (q, k, v)]
    out = torch.nn.functional.scaled_dot_product_attention(*t, is_causal=True)
    return [g.numpy() for g in torch.autograd.grad(out, t, torch.from_numpy(d_o))]


def test_softmax_backward_all_softmax_is_causal_attention():
    """Every chunk softmax-routed: the branch is plain causal attention, so its
    gradient is torch's autograd of causal attention.  Catches a wrong scale
    placement or a causal-mask off-by-one in the gradient."""
    _, q, k, v, _, _ = rand_inputs(B=2, H=2, L=192, D=8, seed=31)
    d_o = np.random.default_rng(32).standard_normal(v.shape)
    r = np.zeros((2, 1, 3), np.int32)
    got = O.softmax_branch_backward(q, k, v, r, d_o)
    for g, ref in zip(got, _sdpa_grads(q, k, v, d_o)):
        np.testing.assert_allclose(g, ref, atol=1e-10)


def test_softmax_backward_all_linear_is_per_chunk_attention():
    """Every chunk linear-routed: each chunk attends causally to itself only,
    so the gradient is chunk-by-chunk causal attention's.  Catches gradient
    flowing across chunk boundaries."""
    _, q, k, v, _, _ = rand_inputs(B=1, H=2, L=192, D=8, seed=41)
    d_o = np.random.default_rng(42).standard_normal(v.shape)
    r = np.ones((1, 1, 3), np.int32)
    got = O.softmax_branch_backward(q, k, v, r, d_o)
    for c in range(3):
        sl = slice(64 * c, 64 * (c + 1))
        ref = _sdpa_grads(q[:, :, sl], k[:, :, sl], v[:, :, sl], d_o[:, :, sl])
        for g, rf in zip(got, ref):
            np.testing.assert_allclose(g[:, :, sl], rf, atol=1e-10)


# ------------------------------------------------- Gated DeltaNet gradient ----
def _gdn_inputs(B=1, H=2, L=12, Dk=3, Dv=2, seed=51):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, L, Dk))
    k = rng.standard_normal((B, H, L, Dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, H, L, Dv))
    a = rng.uniform(0.8, 0.99, (B, H, L))
    b = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, H, L))))
    S0 = rng.standard_normal((B, H, Dk, Dv))
    return q, k, v, a, b, S0


def _gdn_loss(args, r, d_o, dS, chunk):
    o, Sf = O.gdn_branch(args["q"], args["k"], args["v"], args["a"], args["b"], r, S_init=args["S0"], chunk=chunk)
    return float(np.sum(o * d_o) + np.sum(Sf * dS))


def test_gdn_backward_finite_differences():
    """Every gradient of the Gated DeltaNet branch (q, k, v, alpha, beta and
    the initial state, with an upstream gradient on the outputs and on the
    final carried state) against central differences of gdn_branch itself.
    Three chunks of 4 tokens routed linear, softmax, linear, so both the
    commit and the rollback paths carry gradient.  Catches a wrong sign or
    term anywhere in the reverse step and a wrong rollback rule."""
    q, k, v, a, b, S0 = _gdn_inputs()
    chunk = 4
    r = np.array([[[O.LIN, O.SM, O.LIN]]])
    rng = np.random.default_rng(52)
    d_o = rng.standard_normal(v.shape)
    dS = rng.standard_normal(S0.shape)
    got = O.gdn_branch_backward(q, k, v, a, b, r, d_o, S_init=S0, dS_final=dS, chunk=chunk)
    args = {"q": q, "k": k, "v": v, "a": a, "b": b, "S0": S0}
    eps = 1e-6
    for name, grad in zip(("q", "k", "v", "a", "b", "S0"), got):
        arr = args[name]
        for _ in range(10):
            idx = tuple(int(rng.integers(0, s)) for s in arr.shape)
            plus = {n: x.copy() for n, x in args.items()}
            minus = {n: x.copy() for n, x in args.items()}
            plus[name][idx] += eps
            minus[name][idx] -= eps
            fd = (_gdn_loss(plus, r, d_o, dS, chunk) - _gdn_loss(minus, r, d_o, dS, chunk)) / (2 * eps)
            assert abs(fd - grad[idx]) <= 1e-7 * max(1.0, abs(fd)), (name, idx, fd, grad[idx])


def _gdn_torch_grads(q, k, v, a, b, r, d_o, S0, chunk):
    """Gradients by torch autograd (fp64) of the rollback recurrence written
    value-major here: state M [Dv, Dk] = S^T, M <- a (M - b (M k) k^T) + b v k^T,
    o = M q; a chunk routed to softmax restores its chunk-start M."""
    T = lambda x: torch.from_numpy(np.ascontiguousarray(x)).requires_grad_(True)
    tq, tk, tv, ta, tb, tS = map(T, (q, k, v, a, b, S0))
    B, H, L, _ = q.shape
    outs = []
    for bb in range(B):
        for h in range(H):
            M = tS[bb, h].T
            ob = []
            for c0 in range(0, L, chunk):
                M0 = M
                for t in range(c0, c0 + chunk):
                    kt = tk[bb, h, t]
                    M = ta[bb, h, t] * (M - tb[bb, h, t] * torch.outer(M @ kt, kt)) + tb[bb, h, t] * torch.outer(tv[bb, h, t], kt)
                    ob.append(M @ tq[bb, h, t])
                if int(r[bb, 0, c0 // chunk]) != O.LIN:
                    M = M0
            outs.append(torch.stack(ob))
    o = torch.stack(outs).reshape(B, H, L, -1)
    return [g.numpy() for g in torch.autograd.grad(o, (tq, tk, tv, ta, tb, tS), torch.from_numpy(d_o))]


def test_gdn_backward_matches_autograd():
    """The same gradients by torch autograd of an independently written
    (value-major) rollback recurrence, on a larger case with every route
    pattern: linear/softmax runs and both single chunks."""
    q, k, v, a, b, S0 = _gdn_inputs(B=2, H=2, L=48, Dk=5, Dv=4, seed=61)
    chunk = 8
    r = np.array([[[O.LIN, O.LIN, O.SM, O.LIN, O.SM, O.SM]], [[O.SM, O.LIN, O.SM, O.SM, O.LIN, O.LIN]]])
    d_o = np.random.default_rng(62).standard_normal(v.shape)
    got = O.gdn_branch_backward(q, k, v, a, b, r, d_o, S_init=S0, chunk=chunk)
    ref = _gdn_torch_grads(q, k, v, a, b, r, d_o, S0, chunk)
    for name, g, rf in zip(("q", "k", "v", "alpha", "beta", "S_init"), got, ref):
        np.testing.assert_allclose(g, rf, atol=1e-10, err_msg=name)


# --------------------------------------------------------- merge gradient ----
def test_merge_backward_matches_autograd_and_fd():
    """The merge's gradient (both branch outputs, q through the mixing weights,
    W_mix shared and per head, and both gains) against torch autograd of the
    merge written out in torch, and a few entries against central differences
    of merge itself.  Catches a dropped RMS-norm term, a wrong softmax-of-two
    derivative or swapped mixing columns."""
    rng = np.random.default_rng(91)
    B, H, L, D = 2, 3, 5, 6
    q, a, b, d_out = (rng.standard_normal((B, H, L, D)) for _ in range(4))
    gs, gl = rng.uniform(0.5, 1.5, D), rng.uniform(0.5, 1.5, D)
    for wm in (rng.standard_normal((D, 2)), rng.standard_normal((H, D, 2))):
        got = O.merge_backward(q, a, b, wm, d_out, gs, gl)
        T = lambda x: torch.from_numpy(np.ascontiguousarray(x)).requires_grad_(True)
        tq, ta, tb, tw, tgs, tgl = map(T, (q, a, b, wm, gs, gl))
        eps = 1e-6
        ns = ta / torch.sqrt((ta * ta).mean(-1, keepdim=True) + eps) * tgs
        nl = tb / torch.sqrt((tb * tb).mean(-1, keepdim=True) + eps) * tgl
        z = tq @ tw if wm.ndim == 2 else torch.einsum("bhtk,hkj->bhtj", tq, tw)
        w = torch.softmax(z, dim=-1)
        out = w[..., 0:1] * ns + w[..., 1:2] * nl
        ref = torch.autograd.grad(out, (ta, tb, tq, tw, tgs, tgl), torch.from_numpy(d_out))
        for name, g, r in zip(("d_o_sm", "d_o_gdn", "dq", "dw_mix", "dg_sm", "dg_lin"), got, ref):
            np.testing.assert_allclose(g, r.numpy(), atol=1e-12, err_msg=name)
        loss = lambda q_, a_, b_: float(np.sum(O.merge(q_, a_, b_, wm, gs, gl)[0] * d_out))
        h = 1e-6
        for arr_i, grad in ((0, got[2]), (1, got[0]), (2, got[1])):
            for _ in range(4):
                idx = tuple(int(rng.integers(0, s)) for s in q.shape)
                args_p = [q.copy(), a.copy(), b.copy()]
                args_m = [q.copy(), a.copy(), b.copy()]
                args_p[arr_i][idx] += h
                args_m[arr_i][idx] -= h
                fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
                assert abs(fd - grad[idx]) <= 1e-7 * max(1.0, abs(fd))


def test_layer_gradient_chain_matches_finite_differences():
    """The layer's gradient for fixed routes is the merge's gradient followed
    by both branches' (q collects three shares: the mixing weights', the
    softmax branch's and the Gated DeltaNet branch's).  That chain of oracle
    gradients against central differences of the whole oracle forward (all
    inputs but the routes; softmax / linear / softmax chunks of 4 tokens)."""
    rng = np.random.default_rng(97)
    B, H, L, D, chunk = 1, 2, 12, 4, 4
    q, k, v = (rng.standard_normal((B, H, L, D)) for _ in range(3))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    a = rng.uniform(0.8, 0.99, (B, H, L))
    b = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, H, L))))
    wm = rng.normal(0, 0.5, (D, 2))
    gs, gl = rng.uniform(0.5, 1.5, D), rng.uniform(0.5, 1.5, D)
    r = np.array([[[O.SM, O.LIN, O.SM]]])
    d_out = rng.standard_normal((B, H, L, D))
    x = np.zeros((B, L, 3))
    fwd = O.forward(x, q, k, v, a, b, None, wm, g_sm=gs, g_lin=gl, route_override=r, chunk=chunk)
    d_sm, d_gdn, dq_mix, dwm, dgs, dgl = O.merge_backward(q, fwd["o_sm"], fwd["o_gdn"], wm, d_out, gs, gl)
    dq1, dk1, dv1 = O.softmax_branch_backward(q, k, v, r, d_sm, chunk=chunk)
    dq2, dk2, dv2, da, db, _ = O.gdn_branch_backward(q, k, v, a, b, r, d_gdn, chunk=chunk)
    grads = {"q": dq_mix + dq1 + dq2, "k": dk1 + dk2, "v": dv1 + dv2, "a": da, "b": db, "wm": dwm,
             "gs": dgs, "gl": dgl}
    args = {"q": q, "k": k, "v": v, "a": a, "b": b, "wm": wm, "gs": gs, "gl": gl}

    def loss(p):
        o = O.forward(x, p["q"], p["k"], p["v"], p["a"], p["b"], None, p["wm"], g_sm=p["gs"], g_lin=p["gl"],
                      route_override=r, chunk=chunk)["out"]
        return float(np.sum(o * d_out))

    h = 1e-6
    for name, g in grads.items():
        for _ in range(6):
            idx = tuple(int(rng.integers(0, s)) for s in args[name].shape)
            pp = {n: x_.copy() for n, x_ in args.items()}
            pm = {n: x_.copy() for n, x_ in args.items()}
            pp[name][idx] += h
            pm[name][idx] -= h
            fd = (loss(pp) - loss(pm)) / (2 * h)
            assert abs(fd - g[idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, g[idx])
