"""Pins for the router's gradient under the straight-through reading of
"Technische Samenvatting: Neural Attention Search Linear (NAtS-L)",
Kernmechanismen 5 (selection learned end to end; gradients for the attention
score layer).

The oracle's gate gradients (softmax_branch_backward / gdn_branch_backward
with_gate) are checked against torch autograd of an independently written
relaxed layer: chunk c's route as two continuous gates h_c, the softmax branch
weighting chunk c's keys by h_c[softmax] for later queries, the Gated DeltaNet
branch committing S_start + h_c[linear] (S_end - S_start).  At the one-hot h
of the routes that model equals the routed oracle (checked first), so its
gradient there is the derivative the straight-through estimator needs.  The
oracle's route_backward (softmax Jacobian, score layer, mean-pool) is checked
against torch autograd of that chain."""
import numpy as np
import pytest
import torch

import oracle as O

CH = 8  # small chunks keep the torch model quick; the oracle takes any chunk size


def inputs(B=2, H=2, L=48, D=4, seed=0):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, H, L, D)) * 1.5
    k = r.standard_normal((B, H, L, D))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((B, H, L, D))
    a = r.uniform(0.8, 1.0, (B, H, L))
    b = 1 / (1 + np.exp(-r.standard_normal((B, H, L))))
    return q, k, v, a, b


def relaxed_layer(q, k, v, a, b, hs, hl, groups):
    """Torch, fp64: the layer with gates.  hs, hl [B, G, Nc] tensors."""
    B, H, L, D = q.shape
    nc = L // CH
    scale = 1.0 / np.sqrt(D)
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x))
    q, k, v, a, b = map(t, (q, k, v, a, b))
    cs = torch.arange(L) // CH
    causal = torch.arange(L)[None, :] <= torch.arange(L)[:, None]
    same = cs[None, :] == cs[:, None]
    o_sm = torch.zeros(B, H, L, D, dtype=torch.float64)
    o_gdn = torch.zeros(B, H, L, D, dtype=torch.float64)
    S_fin = torch.zeros(B, H, D, D, dtype=torch.float64)
    for bb in range(B):
        for hh in range(H):
            g = hh // (H // groups)
            wk = torch.where(same, torch.ones(L, L, dtype=torch.float64), hs[bb, g][cs][None, :].expand(L, L))
            wk = torch.where(causal, wk, torch.zeros_like(wk))
            z = scale * q[bb, hh] @ k[bb, hh].T
            e = wk * torch.exp(z - z.max(dim=-1, keepdim=True).values.detach())
            o_sm[bb, hh] = (e @ v[bb, hh]) / e.sum(dim=-1, keepdim=True)
            carry = torch.zeros(D, D, dtype=torch.float64)
            for c in range(nc):
                S = carry
                for tt in range(c * CH, (c + 1) * CH):
                    kt, vt = k[bb, hh, tt], v[bb, hh, tt]
                    S = a[bb, hh, tt] * (S - b[bb, hh, tt] * torch.outer(kt, kt @ S)) + b[bb, hh, tt] * torch.outer(kt, vt)
                    o_gdn[bb, hh, tt] = S.T @ q[bb, hh, tt]
                carry = carry + hl[bb, g, c] * (S - carry)
            S_fin[bb, hh] = carry
    return o_sm, o_gdn, S_fin


@pytest.mark.parametrize("groups", [1, 2])
def test_gate_gradients_match_autograd_of_the_relaxed_layer(groups):
    B, H, L, D = 2, 2, 48, 4
    q, k, v, a, b = inputs(B, H, L, D)
    nc = L // CH
    r = np.random.default_rng(3)
    route = (r.random((B, groups, nc)) < 0.5).astype(np.int32)
    route[:, :, 0] = 0
    route[:, :, 1] = 1
    hs = torch.tensor((route == O.SM).astype(np.float64), requires_grad=True)
    hl = torch.tensor((route == O.LIN).astype(np.float64), requires_grad=True)
    o_sm, o_gdn, S_fin = relaxed_layer(q, k, v, a, b, hs, hl, groups)
    # the relaxed model is the routed layer at the one-hot gates
    ref_sm = O.softmax_branch(q, k, v, route, chunk=CH)
    ref_gdn, ref_S = O.gdn_branch(q, k, v, a, b, route, chunk=CH)
    np.testing.assert_allclose(o_sm.detach().numpy(), ref_sm, atol=1e-12)
    np.testing.assert_allclose(o_gdn.detach().numpy(), ref_gdn, atol=1e-12)
    np.testing.assert_allclose(S_fin.detach().numpy(), ref_S, atol=1e-12)
    A = r.standard_normal(o_sm.shape)
    Bm = r.standard_normal(o_gdn.shape)
    Cm = r.standard_normal(S_fin.shape)
    loss = (o_sm * torch.from_numpy(A)).sum() + (o_gdn * torch.from_numpy(Bm)).sum() + \
        (S_fin * torch.from_numpy(Cm)).sum()
    loss.backward()
    *_, dg_sm = O.softmax_branch_backward(q, k, v, route, A, chunk=CH, with_gate=True)
    *_, dg_lin = O.gdn_branch_backward(q, k, v, a, b, route, Bm, dS_final=Cm, chunk=CH, with_gate=True)
    # per-head gate gradients summed over each route group
    sum_g = lambda x: x.reshape(B, groups, H // groups, nc).sum(axis=2)
    np.testing.assert_allclose(sum_g(dg_sm), hs.grad.numpy(), atol=1e-10)
    np.testing.assert_allclose(sum_g(dg_lin), hl.grad.numpy(), atol=1e-10)
    # the softmax gate of the last chunk has no later queries; its linear gate
    # moves only the final state
    assert np.all(dg_sm[:, :, -1] == 0.0)


def test_gate_gradient_is_not_trivially_zero_for_unselected_chunks():
    """An unselected (linear-routed) chunk still has a softmax-gate gradient
    (what including its keys would change) and a softmax-routed chunk a
    linear-gate gradient: the estimator can move the routes both ways."""
    B, H, L, D = 1, 1, 48, 4
    q, k, v, a, b = inputs(B, H, L, D, seed=9)
    route = np.array([[[0, 1, 0, 1, 1, 0]]], np.int32)
    d_o = np.random.default_rng(1).standard_normal((B, H, L, D))
    *_, dg_sm = O.softmax_branch_backward(q, k, v, route, d_o, chunk=CH, with_gate=True)
    *_, dg_lin = O.gdn_branch_backward(q, k, v, a, b, route, d_o, chunk=CH, with_gate=True)
    assert np.all(np.abs(dg_sm[0, 0, [1, 3, 4]]) > 1e-6)
    assert np.all(np.abs(dg_lin[0, 0, [0, 2]]) > 1e-6)


@pytest.mark.parametrize("groups", [1, 3])
def test_route_backward_matches_autograd(groups):
    """Straight-through step: ds = J_softmax(s)^T dh, then the score layer and
    the mean-pool, against torch autograd of
    sum(softmax(mean_pool(x) W + b) * dh)."""
    B, L, d, H = 2, 40, 5, 3
    r = np.random.default_rng(11)
    x = r.standard_normal((B, L, d))
    w = r.standard_normal((d, 2 * groups))
    bias = r.standard_normal(2 * groups)
    nc = L // CH
    dgs = r.standard_normal((B, H, nc))
    dgl = r.standard_normal((B, H, nc))
    dx, dW, db, ds = O.route_backward(x, w, dgs, dgl, b_score=bias, chunk=CH, groups=groups)
    xt = torch.tensor(x, requires_grad=True)
    wt = torch.tensor(w, requires_grad=True)
    bt = torch.tensor(bias, requires_grad=True)
    pooled = xt.reshape(B, nc, CH, d).mean(dim=2)
    s = (pooled @ wt + bt).reshape(B, nc, groups, 2)
    pi = torch.softmax(s, dim=-1)
    dh = np.zeros((B, nc, groups, 2))
    for h in range(H):
        g = h // (H // groups)
        dh[:, :, g, 0] += dgs[:, h]
        dh[:, :, g, 1] += dgl[:, h]
    (pi * torch.from_numpy(dh)).sum().backward()
    np.testing.assert_allclose(dx, xt.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dW, wt.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(db, bt.grad.numpy(), atol=1e-12)
    # a score pair's gradient is antisymmetric (softmax over two logits)
    np.testing.assert_allclose(ds[..., 0], -ds[..., 1], atol=1e-14)
