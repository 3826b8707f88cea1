"""Pins for the oracle's Native Hybrid Attention function (one softmax over
compressed slots plus a sliding window; "Native Hybrid Attention for
Efficient Sequence Modeling", section 2 Methodologie, "Unificatie van
Intra-layer Hybridisatie").  Each test names the mistake it catches."""
import numpy as np
import torch

import oracle as O

RNG = np.random.default_rng(777)


def inputs(B=1, H=2, L=40, D=6, m=3, seed=0, gate=(0.3, 0.95)):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, H, L, D)) * 1.5
    k = r.standard_normal((B, H, L, D))
    v = r.standard_normal((B, H, L, D))
    a = r.uniform(*gate, size=(B, H, L, m))
    return q, k, v, a


def sdpa_causal(q, k, v):
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x))
    return torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=True).numpy()


def test_window_covering_the_sequence_is_causal_attention():
    """w >= L: no token ever leaves the window, the slots never join, and the
    result is causal softmax attention (torch SDPA in fp64).  Catches slots
    that join before anything has entered them."""
    q, k, v, a = inputs(L=48)
    for w in (48, 100):
        np.testing.assert_allclose(O.nha_attention(q, k, v, a, w), sdpa_causal(q, k, v), atol=1e-12)


def test_window_zero_one_slot_is_gated_linear_rnn():
    """w = 0 with one slot: the softmax over a single key is 1, so o_t is the
    slot value itself, a gated exponential moving average of v whose closed
    form is o_t = sum_{s <= t} (prod_{s < r <= t} a_r) (1 - a_s) v_s, built
    here from cumulative log-gates as one L x L matrix.  Catches a swapped
    forget / write orientation, an off-by-one in when a token enters, and
    w = 0 not including the query's own token."""
    q, k, v, a = inputs(L=32, m=1)
    o = O.nha_attention(q, k, v, a, 0)
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            lg = np.cumsum(np.log(a[b, h, :, 0]))
            t_idx, s_idx = np.meshgrid(np.arange(32), np.arange(32), indexing="ij")
            A = np.where(s_idx <= t_idx, np.exp(lg[t_idx] - lg[s_idx]) * (1 - a[b, h, s_idx, 0]), 0.0)
            np.testing.assert_allclose(o[b, h], A @ v[b, h], atol=1e-12)


def test_gates_one_keep_slots_at_zero_but_in_the_softmax():
    """a = 1 never writes (1 - a = 0) and never forgets, so the m slots stay
    zero: once a token has left the window they add m keys of score 0 and
    value 0, i.e. o_t = sum_win e^z v / (sum_win e^z + m e^0) for t >= w, and
    plain causal attention before.  Catches slots left out of the softmax
    and a wrong start of the slots' participation."""
    q, k, v, _ = inputs(L=30, m=4)
    a = np.ones(q.shape[:3] + (4,))
    w = 7
    o = O.nha_attention(q, k, v, a, w)
    sc = 1 / np.sqrt(q.shape[3])
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            for t in range(30):
                lo = max(0, t - w + 1)
                z = sc * k[b, h, lo:t + 1] @ q[b, h, t]
                e = np.exp(z)
                den = e.sum() + (4.0 if t >= w else 0.0)
                np.testing.assert_allclose(o[b, h, t], (e @ v[b, h, lo:t + 1]) / den, atol=1e-12)


def test_gates_zero_overwrite_every_slot_with_the_leaving_token():
    """a = 0 forgets everything and writes the whole token: every slot holds
    the token that left the window last (t - w), so that token appears m + 0
    times in the key set (m slot copies; it is no longer in the window).
    Catches a gate applied to the wrong term and a slot written with the
    wrong token."""
    q, k, v, _ = inputs(L=26, m=3)
    a = np.zeros(q.shape[:3] + (3,))
    w = 5
    o = O.nha_attention(q, k, v, a, w)
    sc = 1 / np.sqrt(q.shape[3])
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            for t in range(26):
                lo = max(0, t - w + 1)
                idx = list(range(lo, t + 1))
                mult = [1.0] * len(idx)
                if t - w >= 0:
                    idx.insert(0, t - w)
                    mult.insert(0, 3.0)
                z = sc * k[b, h, idx] @ q[b, h, t]
                e = np.exp(z) * np.array(mult)
                np.testing.assert_allclose(o[b, h, t], (e @ v[b, h, idx]) / e.sum(), atol=1e-12)


def test_matches_bruteforce_closed_form_slots():
    """The recurrence equals slots rebuilt from scratch per query as
    closed-form weighted sums (several windows, including 0 and 1).  Catches
    recurrence mistakes the special cases above do not exercise (several
    slots with their own gates, partial windows)."""
    q, k, v, a = inputs(L=33, m=3, seed=4)
    for w in (0, 1, 5, 16, 32):
        np.testing.assert_allclose(O.nha_attention(q, k, v, a, w), O.nha_attention_bruteforce(q, k, v, a, w),
                                   atol=1e-12, err_msg=f"w={w}")


def test_causality():
    """Perturbing tokens after t leaves outputs up to t bit-identical."""
    q, k, v, a = inputs(L=30, m=2, seed=5)
    t = 17
    o1 = O.nha_attention(q, k, v, a, 6)
    q2, k2, v2, a2 = (x.copy() for x in (q, k, v, a))
    for x in (q2, k2, v2):
        x[:, :, t + 1:] += 1.0
    a2[:, :, t + 1:] *= 0.5
    o2 = O.nha_attention(q2, k2, v2, a2, 6)
    np.testing.assert_array_equal(o1[:, :, :t + 1], o2[:, :, :t + 1])
