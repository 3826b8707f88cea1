"""fp64 CPU oracle for the NAtS-L hybrid attention layer (forward, decode step,
and the gradients of the softmax and Gated DeltaNet branches and of the merge).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this module:
only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg use it.
It shares no code with the HIP library and imports nothing from it.

Pages cited (all from gist.science):
  [NL]  "Technische Samenvatting: Neural Attention Search Linear (NAtS-L)"
        (Dutch summary of arXiv 2602.03681)
  [DE]  "Neural Attention Search Linear: Towards Adaptive Token-Level Hybrid
        Attention Models" (German explainer of the same paper; its
        "Technisches Resümee" repeats [NL])
  [SA]  "Technische Samenvatting: Een Systematische Analyse van Hybride
        Lineaire Aandacht" (Dutch summary of arXiv 2507.06457)

What the layer computes (plain definitions, no chunkwise algebra):
  * route:   the sequence is cut into chunks of C = 64 tokens ([DE] "Die
             Chunking-Strategie"); each chunk is mean-pooled and passed through
             a linear layer that yields one score per operation type; the
             highest score picks the operation ([NL] Kernmechanismen 1).
  * softmax: plain causal softmax attention whose key set is the tokens of
             earlier softmax-routed chunks plus the causal prefix of the
             query's own chunk ([NL] Kernmechanismen 3: both correlations are
             computed inside every chunk; only the selected operation's KV is
             kept).
  * GDN:     the gated delta rule run token by token; at the end of every
             chunk the state is kept if the chunk was routed to the linear
             operation and restored to its chunk-start value otherwise
             ([NL] Kernmechanismen 3, "pseudo-update" then reset/rollback).
             Gated DeltaNet itself is only named on the pages; the recurrence
             used is the published gated delta rule, gating plus a delta rule
             that erases stale content ([SA] Methodologie, generation 3, and
             Belangrijkste Resultaten 3, "Gecontroleerd Vergeten").
  * merge:   each branch output is RMS-normalised and the two are summed with
             weights produced from Q ([NL] Kernmechanismen 4).

Readings where the pages are silent (each is also listed in the design doc):
  route column 0 = softmax, column 1 = linear; an exact tie goes to softmax;
  the router pools the layer input x; the decay alpha and write strength beta
  are per (b, h, t) scalars; S is key-major [Dk, Dv]; o_t = S_t^T q_t with no
  extra scale; the softmax scale defaults to 1/sqrt(Dk); RMSNorm has eps
  inside the square root and no mean subtraction; mixing weights are
  softmax(q_t . W_mix) with column 0 weighting the softmax branch.

Every function works in float64 on whatever values it is handed; callers pass
the exact (already bf16-rounded where applicable) values the GPU receives.
"""
from __future__ import annotations

import numpy as np

SM = 0   # route id of the softmax operation
LIN = 1  # route id of the Gated DeltaNet operation
CHUNK = 64  # [DE] "Die Chunking-Strategie": a stack of 64 notes is one chunk


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def group_of_head(h: int, H: int, G: int) -> int:
    """Route group used by head h.  G = 1 shares one route per chunk across
    all heads; G = H routes every head on its own."""
    return h // (H // G)


# ---------------------------------------------------------------------------
# Router  ([NL] Kernmechanismen 1; [DE] Chunking-Strategie / Verkehrspolizist)
# ---------------------------------------------------------------------------
def route_scores(x, w_score, b_score=None, chunk=CHUNK, groups=1):
    """Attention Score Layer: mean-pool every chunk of x, apply a linear layer.

    x        [B, L, d]      layer input (only complete chunks are scored)
    w_score  [d, 2*groups]  columns (2g, 2g+1) = (softmax, linear) of group g
    b_score  [2*groups] or None
    returns  scores [B, groups, Nc, 2]
    """
    x = _f64(x)
    w = _f64(w_score)
    B, L, d = x.shape
    nc = L // chunk
    pooled = x[:, : nc * chunk].reshape(B, nc, chunk, d).mean(axis=2)  # [B,Nc,d]
    s = pooled @ w  # [B, Nc, 2G]
    if b_score is not None:
        s = s + _f64(b_score)
    return s.reshape(B, nc, groups, 2).transpose(0, 2, 1, 3).copy()


def route_from_scores(scores):
    """The operation with the highest score wins; an exact tie goes to the
    softmax operation (column 0), the first-maximum rule of argmax."""
    return np.where(scores[..., SM] >= scores[..., LIN], SM, LIN).astype(np.int32)


def route(x, w_score, b_score=None, chunk=CHUNK, groups=1):
    """Returns (route [B,G,Nc] int32, margin [B,G,Nc] = s_softmax - s_linear)."""
    s = route_scores(x, w_score, b_score, chunk, groups)
    return route_from_scores(s), s[..., SM] - s[..., LIN]


def compact(route_bgc):
    """Index list of softmax-routed chunks, the prefill form of the softmax
    branch's retained KV ([NL] Kernmechanismen 3: only the selected
    operation's KV values are kept).

    returns sel_idx [B,G,Nc] (ascending SM chunk ids, padded with -1) and
            nsel_before [B,G,Nc+1] (number of SM chunks before chunk c)."""
    r = np.asarray(route_bgc)
    B, G, nc = r.shape
    sel = np.full((B, G, nc), -1, dtype=np.int32)
    nsb = np.zeros((B, G, nc + 1), dtype=np.int32)
    for b in range(B):
        for g in range(G):
            ids = [c for c in range(nc) if r[b, g, c] == SM]
            sel[b, g, : len(ids)] = ids
            cnt = 0
            for c in range(nc):
                nsb[b, g, c] = cnt
                cnt += int(r[b, g, c] == SM)
            nsb[b, g, nc] = cnt
    return sel, nsb


# ---------------------------------------------------------------------------
# Softmax branch  ([NL] Kernmechanismen 3)
# ---------------------------------------------------------------------------
def key_mask(route_c, L, chunk=CHUNK):
    """Boolean [L, L] mask M[t, s]: key s is visible to query t iff s <= t and
    (s is in t's own chunk, or s's chunk was routed to softmax).  route_c has
    one entry per chunk (a trailing partial chunk needs none: its own route
    never affects its outputs)."""
    t = np.arange(L)[:, None]
    s = np.arange(L)[None, :]
    cs, ct = s // chunk, t // chunk
    rc = np.asarray(route_c)
    rs = np.where(cs < len(rc), rc[np.minimum(cs, len(rc) - 1)], LIN)
    return (s <= t) & ((cs == ct) | (rs == SM))


def block_mask(route_c, t0, t1, chunk=CHUNK):
    """Rows t0..t1-1 of key_mask, restricted to keys 0..t1-1."""
    t = np.arange(t0, t1)[:, None]
    s = np.arange(t1)[None, :]
    cs, ct = s // chunk, t // chunk
    rc = np.asarray(route_c)
    rs = np.where(cs < len(rc), rc[np.minimum(cs, len(rc) - 1)], LIN)
    return (s <= t) & ((cs == ct) | (rs == SM))


def softmax_branch(q, k, v, route_bgc, scale=None, chunk=CHUNK, with_lse=False, query_blocks=None):
    """Naive masked two-pass softmax attention, one 64-row query block at a
    time (rows are independent, so blocking changes nothing).

    q, k [B,H,L,Dk]; v [B,H,L,Dv]; route_bgc [B,G,Nc] -> o_sm [B,H,L,Dv]
    (and the natural-log logsumexp [B,H,L] of the scaled scores if asked).
    query_blocks, if given, lists the 64-row query blocks to compute; the
    other rows are left at zero (used to sample very long sequences)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, L, Dk = q.shape
    G = route_bgc.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(Dk)
    o = np.zeros(v.shape[:3] + (v.shape[3],))
    lse = np.zeros((B, H, L))
    for b in range(B):
        for g in range(G):
            heads = [h for h in range(H) if group_of_head(h, H, G) == g]
            blocks = range(0, L, chunk) if query_blocks is None else [c * chunk for c in query_blocks]
            for t0 in blocks:
                t1 = min(L, t0 + chunk)
                m = block_mask(route_bgc[b, g], t0, t1, chunk)  # keys past t1 are never visible
                z = scale * np.einsum("hqd,hkd->hqk", q[b, heads, t0:t1], k[b, heads, :t1])
                z = np.where(m[None], z, -np.inf)
                zmax = z.max(axis=-1, keepdims=True)
                p = np.exp(z - zmax)
                den = p.sum(axis=-1, keepdims=True)
                o[b, heads, t0:t1] = np.einsum("hqk,hkd->hqd", p, v[b, heads, :t1]) / den
                lse[b, heads, t0:t1] = (zmax + np.log(den))[..., 0]
    return (o, lse) if with_lse else o


def softmax_branch_bruteforce(q, k, v, route_bgc, scale=None, chunk=CHUNK):
    """Brute-force twin: for every query, list its visible keys explicitly and
    take a softmax over that list.  Tiny inputs only."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, L, Dk = q.shape
    G = route_bgc.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(Dk)
    o = np.zeros(v.shape)
    for b in range(B):
        for h in range(H):
            r = route_bgc[b, group_of_head(h, H, G)]
            for t in range(L):
                keys = [s for s in range(t + 1)
                        if s // chunk == t // chunk or r[s // chunk] == SM]
                z = np.array([scale * float(q[b, h, t] @ k[b, h, s]) for s in keys])
                p = np.exp(z - z.max())
                p /= p.sum()
                o[b, h, t] = sum(pi * v[b, h, s] for pi, s in zip(p, keys))
    return o


def softmax_branch_backward(q, k, v, route_bgc, d_o, scale=None, chunk=CHUNK, with_gate=False):
    """Gradient of the softmax branch (softmax_branch above) for an upstream
    gradient d_o [B,H,L,Dv]: returns dq, dk, dv.  The pages define only the
    forward; this is its exact derivative, taken one 64-row query block at a
    time with the block's visible keys (block_mask):
        p  = softmax over the visible keys of scale * q k^T
        o  = p v
        dp = d_o v^T,  delta = rowsum(d_o * o),  ds = p * (dp - delta)
        dq = scale * ds k,   dk += scale * ds^T q,   dv += p^T d_o
    (masked keys have p = 0 and receive nothing).

    with_gate: also returns dgate [B,H,Nc], the derivative with respect to
    each chunk's softmax gate h_c (see route_backward): the layer with chunk
    c's keys weighted by h_c for the queries of later chunks, at h_c = 0 or 1;
    with p~ = exp(scale q.k - lse) over ALL keys of chunk c (visible or not),
        dgate[c] = sum_{t in later chunks} sum_{s in c} p~_ts (d_o_t . v_s - delta_t)."""
    q, k, v, d_o = _f64(q), _f64(k), _f64(v), _f64(d_o)
    B, H, L, Dk = q.shape
    G = route_bgc.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(Dk)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    nc = L // chunk
    dgate = np.zeros((B, H, nc))
    for b in range(B):
        for g in range(G):
            heads = [h for h in range(H) if group_of_head(h, H, G) == g]
            for t0 in range(0, L, chunk):
                t1 = min(L, t0 + chunk)
                m = block_mask(route_bgc[b, g], t0, t1, chunk)
                z = scale * np.einsum("hqd,hkd->hqk", q[b, heads, t0:t1], k[b, heads, :t1])
                z = np.where(m[None], z, -np.inf)
                p = np.exp(z - z.max(axis=-1, keepdims=True))
                p /= p.sum(axis=-1, keepdims=True)
                o = np.einsum("hqk,hkd->hqd", p, v[b, heads, :t1])
                g_o = d_o[b, heads, t0:t1]
                dp = np.einsum("hqd,hkd->hqk", g_o, v[b, heads, :t1])
                delta = np.sum(g_o * o, axis=-1, keepdims=True)
                ds = p * (dp - delta)
                dq[b, heads, t0:t1] = scale * np.einsum("hqk,hkd->hqd", ds, k[b, heads, :t1])
                dk[b, heads, :t1] += scale * np.einsum("hqk,hqd->hkd", ds, q[b, heads, t0:t1])
                dv[b, heads, :t1] += np.einsum("hqk,hqd->hkd", p, g_o)
                if with_gate and t0 >= chunk:
                    # every key of the chunks before this block, visible or not
                    zall = scale * np.einsum("hqd,hkd->hqk", q[b, heads, t0:t1], k[b, heads, :t0])
                    lse = (zmax_all := z.max(axis=-1, keepdims=True)) + np.log(
                        np.exp(z - zmax_all).sum(axis=-1, keepdims=True))
                    pt = np.exp(zall - lse)
                    dpa = np.einsum("hqd,hkd->hqk", g_o, v[b, heads, :t0])
                    contrib = (pt * (dpa - delta)).sum(axis=1)  # [heads, t0]
                    dgate[b, heads, :t0 // chunk] += contrib.reshape(len(heads), t0 // chunk, chunk).sum(axis=2)
    return (dq, dk, dv, dgate) if with_gate else (dq, dk, dv)


# ---------------------------------------------------------------------------
# Gated DeltaNet branch  ([NL] Kernmechanismen 3; [SA] generation 3)
# ---------------------------------------------------------------------------
def gdn_token_update(S, k_t, v_t, a_t, b_t):
    """One gated delta-rule step on key-major states S [..., Dk, Dv]:
        S <- a_t * (S - b_t * k_t (k_t^T S)) + b_t * k_t v_t^T
    (decay the state, erase what key k_t currently retrieves, write v_t)."""
    kS = np.einsum("...k,...kv->...v", k_t, S)
    a = np.asarray(a_t)[..., None, None]
    b = np.asarray(b_t)[..., None, None]
    return a * (S - b * k_t[..., :, None] * kS[..., None, :]) + b * k_t[..., :, None] * v_t[..., None, :]


def gdn_readout(S, q_t):
    """o_t = S_t^T q_t."""
    return np.einsum("...kv,...k->...v", S, q_t)


def gdn_branch(q, k, v, alpha, beta, route_bgc, S_init=None, chunk=CHUNK):
    """Per-token gated delta rule with per-chunk rollback.

    For every chunk the state starts from the carried state, is pseudo-updated
    token by token (every token reads out after its own update), and at the
    chunk's end is kept only if the chunk was routed to the linear operation.

    q, k [B,H,L,Dk]; v [B,H,L,Dv]; alpha, beta [B,H,L]; route [B,G,Nc]
    returns o_gdn [B,H,L,Dv], S_final [B,H,Dk,Dv] (the carried state)."""
    q, k, v, alpha, beta = map(_f64, (q, k, v, alpha, beta))
    B, H, L, Dk = q.shape
    Dv = v.shape[3]
    G = route_bgc.shape[1]
    carry = np.zeros((B, H, Dk, Dv)) if S_init is None else _f64(S_init).copy()
    gidx = np.array([group_of_head(h, H, G) for h in range(H)])
    o = np.zeros((B, H, L, Dv))
    for c0 in range(0, L, chunk):
        c = c0 // chunk
        S = carry.copy()
        for t in range(c0, min(L, c0 + chunk)):
            S = gdn_token_update(S, k[:, :, t], v[:, :, t], alpha[:, :, t], beta[:, :, t])
            o[:, :, t] = gdn_readout(S, q[:, :, t])
        if c0 + chunk <= L:  # only a complete chunk has a route and can commit
            keep = route_bgc[:, gidx, c] == LIN  # [B, H]
            carry = np.where(keep[:, :, None, None], S, carry)
    return o, carry


def gdn_branch_bruteforce(q, k, v, alpha, beta, route_bgc, S_init=None, chunk=CHUNK):
    """Brute-force twin of gdn_branch: for every token t, rerun the recurrence
    from S_init over exactly the tokens whose writes survive (all tokens of
    linear-routed chunks before t's chunk, in order) followed by t's own chunk
    up to t.  Tiny inputs only."""
    q, k, v, alpha, beta = map(_f64, (q, k, v, alpha, beta))
    B, H, L, Dk = q.shape
    Dv = v.shape[3]
    G = route_bgc.shape[1]
    o = np.zeros((B, H, L, Dv))
    for b in range(B):
        for h in range(H):
            r = route_bgc[b, group_of_head(h, H, G)]
            S0 = np.zeros((Dk, Dv)) if S_init is None else _f64(S_init)[b, h]
            for t in range(L):
                ct = t // chunk
                toks = [s for s in range(ct * chunk) if r[s // chunk] == LIN]
                toks += list(range(ct * chunk, t + 1))
                S = S0.copy()
                for s in toks:
                    S = gdn_token_update(S, k[b, h, s], v[b, h, s], alpha[b, h, s], beta[b, h, s])
                o[b, h, t] = gdn_readout(S, q[b, h, t])
    return o


def gdn_branch_backward(q, k, v, alpha, beta, route_bgc, d_o, S_init=None, dS_final=None, chunk=CHUNK,
                        with_gate=False):
    """Gradient of gdn_branch for an upstream gradient d_o [B,H,L,Dv] of its
    outputs (and dS_final [B,H,Dk,Dv] of its final carried state, if any):
    returns dq, dk, dv, dalpha, dbeta, dS_init.  The pages define only the
    forward; this is its exact derivative, taken token by token in reverse.

    With G = d loss / d S_t (key-major) and S = S_{t-1}, a = S^T k_t:
        G     += q_t d_o_t^T             (o_t = S_t^T q_t)
        dq_t   = S_t d_o_t
        w      = G^T k_t
        dv_t   = beta_t w
        dbeta  = w . (v_t - alpha_t a)
        dalpha = sum(G * (S - beta_t k_t a^T))
        dk_t   = beta_t G v_t - alpha_t beta_t (G a + S w)
        G      <- alpha_t (G - beta_t k_t w^T)   (the gradient of S_{t-1})
    Rollback: a chunk that keeps its end state (linear route) passes the
    carried state's gradient into its last token; one that restores its
    chunk-start state passes it straight to the chunk start, and its tokens
    see only their own outputs' gradients (G starts at zero).

    with_gate: also returns dgate [B,H,Nc], the derivative with respect to
    each chunk's linear gate h_c (see route_backward): the carried state after
    chunk c written as S_start + h_c (S_end - S_start), at h_c = 0 or 1, so
        dgate[c] = <d loss / d carried state after c, S_end - S_start>."""
    q, k, v, alpha, beta, d_o = map(_f64, (q, k, v, alpha, beta, d_o))
    B, H, L, Dk = q.shape
    Dv = v.shape[3]
    G_ = route_bgc.shape[1]
    gidx = np.array([group_of_head(h, H, G_) for h in range(H)])
    # chunk-start carried states of the forward
    carry = np.zeros((B, H, Dk, Dv)) if S_init is None else _f64(S_init).copy()
    starts = []
    for c0 in range(0, L, chunk):
        starts.append(carry.copy())
        S = carry.copy()
        for t in range(c0, min(L, c0 + chunk)):
            S = gdn_token_update(S, k[:, :, t], v[:, :, t], alpha[:, :, t], beta[:, :, t])
        if c0 + chunk <= L:
            keep = route_bgc[:, gidx, c0 // chunk] == LIN
            carry = np.where(keep[:, :, None, None], S, carry)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    dalpha, dbeta = np.zeros_like(alpha), np.zeros_like(beta)
    Gc = np.zeros((B, H, Dk, Dv)) if dS_final is None else _f64(dS_final).copy()  # d loss / d carried state
    dgate = np.zeros((B, H, L // chunk))
    for c0 in reversed(range(0, L, chunk)):
        c1 = min(L, c0 + chunk)
        keep = (route_bgc[:, gidx, c0 // chunk] == LIN) if c0 + chunk <= L else np.zeros((B, H), bool)
        kp = keep[:, :, None, None]
        # states before each token of the chunk
        prev = [starts[c0 // chunk]]
        for t in range(c0, c1 - 1):
            prev.append(gdn_token_update(prev[-1], k[:, :, t], v[:, :, t], alpha[:, :, t], beta[:, :, t]))
        if with_gate and c1 - c0 == chunk:
            S_end = gdn_token_update(prev[-1], k[:, :, c1 - 1], v[:, :, c1 - 1], alpha[:, :, c1 - 1],
                                     beta[:, :, c1 - 1])
            dgate[:, :, c0 // chunk] = np.sum(Gc * (S_end - prev[0]), axis=(-2, -1))
        G = np.where(kp, Gc, 0.0)
        for t in reversed(range(c0, c1)):
            S = prev[t - c0]
            kt, vt, qt, gt = k[:, :, t], v[:, :, t], q[:, :, t], d_o[:, :, t]
            at, bt = alpha[:, :, t][..., None], beta[:, :, t][..., None]
            St = gdn_token_update(S, kt, vt, alpha[:, :, t], beta[:, :, t])
            G = G + qt[..., :, None] * gt[..., None, :]
            dq[:, :, t] = np.einsum("...kv,...v->...k", St, gt)
            a = np.einsum("...kv,...k->...v", S, kt)
            w = np.einsum("...kv,...k->...v", G, kt)
            dv[:, :, t] = bt * w
            dbeta[:, :, t] = np.sum(w * (vt - at * a), axis=-1)
            dalpha[:, :, t] = np.sum(G * (S - bt[..., None] * kt[..., :, None] * a[..., None, :]), axis=(-2, -1))
            dk[:, :, t] = (bt * np.einsum("...kv,...v->...k", G, vt)
                           - at * bt * (np.einsum("...kv,...v->...k", G, a) + np.einsum("...kv,...v->...k", S, w)))
            G = at[..., None] * (G - bt[..., None] * kt[..., :, None] * w[..., None, :])
        Gc = G + np.where(kp, 0.0, Gc)
    out = (dq, dk, dv, dalpha, dbeta, Gc)
    return out + (dgate,) if with_gate else out


def route_backward(x, w_score, dgate_sm, dgate_lin, b_score=None, chunk=CHUNK, groups=1):
    """Gradient of the router under the straight-through reading of
    [NL] Kernmechanismen 5 (the operation selection is learned end to end,
    with gradients computed for the attention score layer; the pages do not
    say how the argmax is differentiated).

    The route of chunk c enters the layer as a one-hot gate h_c =
    onehot(argmax s_c): the softmax branch weights chunk c's keys by
    h_c[softmax] for the queries of later chunks, the Gated DeltaNet branch
    commits chunk c's end state with weight h_c[linear]; at h in {0, 1} that
    is exactly the routed forward.  Straight-through: the backward takes
    d h_c / d s_c to be the Jacobian of softmax(s_c).  Then with
    dh = (dgate_sm, dgate_lin) summed over the heads of each route group and
    pi = softmax(s_c):
        ds_c = pi * (dh - pi . dh)
        dW_score[:, 2g + o] = sum_{b, c} mean_c(x) ds[b, g, c, o],  db = sum ds,
        dx_t = W_score ds_{c(t)} / chunk
    x [B,L,d]; dgate_* [B,H,Nc] (per head); returns dx, dW_score, db, ds."""
    x = _f64(x)
    w = _f64(w_score)
    B, L, d = x.shape
    nc = L // chunk
    G = groups
    H = np.asarray(dgate_sm).shape[1]
    s = route_scores(x, w, b_score, chunk, G)  # [B, G, Nc, 2]
    z = s - s.max(axis=-1, keepdims=True)
    pi = np.exp(z) / np.exp(z).sum(axis=-1, keepdims=True)
    dh = np.zeros((B, G, nc, 2))
    for h in range(H):
        g = group_of_head(h, H, G)
        dh[:, g, :, SM] += _f64(dgate_sm)[:, h]
        dh[:, g, :, LIN] += _f64(dgate_lin)[:, h]
    ds = pi * (dh - (pi * dh).sum(axis=-1, keepdims=True))
    pooled = x[:, : nc * chunk].reshape(B, nc, chunk, d).mean(axis=2)  # [B, Nc, d]
    ds_flat = ds.transpose(0, 2, 1, 3).reshape(B, nc, 2 * G)           # columns (2g, 2g+1)
    dW = np.einsum("bcd,bco->do", pooled, ds_flat)
    db = ds_flat.sum(axis=(0, 1))
    dx = np.zeros_like(x)
    dx[:, : nc * chunk] = np.repeat(np.einsum("do,bco->bcd", w, ds_flat) / chunk, chunk, axis=1)
    return dx, dW, db, ds


# ---------------------------------------------------------------------------
# Output merging  ([NL] Kernmechanismen 4)
# ---------------------------------------------------------------------------
def rmsnorm(o, gain=None, eps=1e-6):
    o = _f64(o)
    n = o / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    return n if gain is None else n * _f64(gain)


def mix_weights(q, w_mix):
    """softmax over the two logits q_t . W_mix[:, 0] (softmax) and
    q_t . W_mix[:, 1] (linear).  w_mix is [Dk, 2] shared by all heads or
    [H, Dk, 2] per head."""
    q = _f64(q)
    w = _f64(w_mix)
    if w.ndim == 2:
        z = q @ w
    else:
        z = np.einsum("bhtk,hkj->bhtj", q, w)
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def merge(q, o_sm, o_gdn, w_mix, g_sm=None, g_lin=None, eps=1e-6):
    """returns out, n_sm, n_lin, weights [.., 2]"""
    n_sm = rmsnorm(o_sm, g_sm, eps)
    n_lin = rmsnorm(o_gdn, g_lin, eps)
    w = mix_weights(q, w_mix)
    out = w[..., 0:1] * n_sm + w[..., 1:2] * n_lin
    return out, n_sm, n_lin, w


def merge_backward(q, o_sm, o_gdn, w_mix, d_out, g_sm=None, g_lin=None, eps=1e-6):
    """Gradient of merge for an upstream gradient d_out [B,H,L,Dv]: returns
    d_o_sm, d_o_gdn, dq (the mixing weights' share of q's gradient), dw_mix
    (the shape of w_mix), dg_sm, dg_lin ([Dv]; ones when the gain is None).
    The pages define only the forward; this is its exact derivative:
        dn_x = w_x d_out,  dw_x = d_out . n_x
        dz_0 = w_0 w_1 (dw_0 - dw_1) = -dz_1          (softmax of two logits)
        dq = dz_0 (W_mix[:, 0] - W_mix[:, 1]),  dW_mix[:, c] += q dz_c
        with r_x = (mean(o_x^2) + eps)^(-1/2) and u = dn_x * g_x:
        d o_x = r_x u - (r_x^3 / Dv) o_x (u . o_x),   dg_x += dn_x * o_x r_x"""
    q, o_sm, o_gdn, d_out = map(_f64, (q, o_sm, o_gdn, d_out))
    Dv = o_sm.shape[-1]
    gs = np.ones(Dv) if g_sm is None else _f64(g_sm)
    gl = np.ones(Dv) if g_lin is None else _f64(g_lin)
    w = mix_weights(q, w_mix)
    wm = _f64(w_mix)
    outs = []
    for o, g, wx in ((o_sm, gs, w[..., 0:1]), (o_gdn, gl, w[..., 1:2])):
        r = 1.0 / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
        dn = wx * d_out
        u = dn * g
        do = r * u - (r ** 3 / Dv) * o * np.sum(u * o, axis=-1, keepdims=True)
        dg = np.sum(dn * o * r, axis=(0, 1, 2))
        dw = np.sum(d_out * (o * r * g), axis=-1)
        outs.append((do, dg, dw))
    (d_sm, dg_sm, dw0), (d_gdn, dg_lin, dw1) = outs
    dz0 = w[..., 0] * w[..., 1] * (dw0 - dw1)
    dz = np.stack([dz0, -dz0], axis=-1)
    if wm.ndim == 2:
        dq = np.einsum("bhtj,kj->bhtk", dz, wm)
        dwm = np.einsum("bhtk,bhtj->kj", q, dz)
    else:
        dq = np.einsum("bhtj,hkj->bhtk", dz, wm)
        dwm = np.einsum("bhtk,bhtj->hkj", q, dz)
    return d_sm, d_gdn, dq, dwm, dg_sm, dg_lin


# ---------------------------------------------------------------------------
# Whole layer forward
# ---------------------------------------------------------------------------
def forward(x, q, k, v, alpha, beta, w_score, w_mix, b_score=None, g_sm=None, g_lin=None,
            route_override=None, S_init=None, scale=None, eps=1e-6, groups=1, chunk=CHUNK):
    """Router -> softmax branch, GDN branch -> merge.  Returns a dict with
    route, margin, o_sm, o_gdn, S_final, n_sm, n_lin, out."""
    if route_override is None:
        r, margin = route(x, w_score, b_score, chunk, groups)
    else:
        r, margin = np.asarray(route_override, dtype=np.int32), None
    o_sm = softmax_branch(q, k, v, r, scale, chunk)
    o_gdn, S_final = gdn_branch(q, k, v, alpha, beta, r, S_init, chunk)
    out, n_sm, n_lin, w = merge(q, o_sm, o_gdn, w_mix, g_sm, g_lin, eps)
    return dict(route=r, margin=margin, o_sm=o_sm, o_gdn=o_gdn, S_final=S_final,
                n_sm=n_sm, n_lin=n_lin, weights=w, out=out)


# ---------------------------------------------------------------------------
# Decode  (the two hidden states of [NL] Kernmechanismen 3, kept online)
# ---------------------------------------------------------------------------
def empty_cache(B, H, D, d_model, cap, groups=1):
    return dict(k=np.zeros((B, H, cap, D)), v=np.zeros((B, H, cap, D)),
                n_committed=np.zeros((B, groups), np.int64), n_open=np.zeros((B, groups), np.int64),
                S_carry=np.zeros((B, H, D, D)), S_work=np.zeros((B, H, D, D)),
                x_sum=np.zeros((B, groups, d_model)), err=0)


def build_cache(x, k, v, alpha, beta, w_score, b_score=None, cap=None, groups=1, S_init=None,
                chunk=CHUNK):
    """Decode cache after a prefix of n = x.shape[1] tokens (any n):
       softmax-routed complete chunks keep their KV (compacted, in order),
       the open (incomplete) chunk's tokens sit after them, S_carry is the
       state after the committed linear chunks, S_work the open chunk's
       pseudo-updated state, x_sum the open chunk's sum of x."""
    x, k, v, alpha, beta = map(_f64, (x, k, v, alpha, beta))
    B, n, d = x.shape
    H, D = k.shape[1], k.shape[3]
    G = groups
    nc_full = n // chunk
    r, _ = route(x[:, : nc_full * chunk], w_score, b_score, chunk, G) if nc_full else (
        np.zeros((B, G, 0), np.int32), None)
    if cap is None:
        cap = n + chunk
    cache = empty_cache(B, H, D, d, cap, G)
    if S_init is not None:
        cache["S_carry"][:] = _f64(S_init)
    for b in range(B):
        for g in range(G):
            heads = [h for h in range(H) if group_of_head(h, H, G) == g]
            pos = 0
            for c in range(nc_full):
                if r[b, g, c] == SM:
                    sl = slice(c * chunk, (c + 1) * chunk)
                    cache["k"][b, heads, pos:pos + chunk] = k[b, heads, sl]
                    cache["v"][b, heads, pos:pos + chunk] = v[b, heads, sl]
                    pos += chunk
            n_open = n - nc_full * chunk
            cache["k"][b, heads, pos:pos + n_open] = k[b, heads, nc_full * chunk:]
            cache["v"][b, heads, pos:pos + n_open] = v[b, heads, nc_full * chunk:]
            cache["n_committed"][b, g] = pos
            cache["n_open"][b, g] = n_open
            cache["x_sum"][b, g] = x[b, nc_full * chunk:].sum(axis=0)
    # states: rerun the per-token rule with rollback over the prefix
    carry = np.zeros((B, H, D, D)) if S_init is None else _f64(S_init).copy()
    gidx = np.array([group_of_head(h, H, G) for h in range(H)])
    for c in range(nc_full):
        S = carry.copy()
        for t in range(c * chunk, (c + 1) * chunk):
            S = gdn_token_update(S, k[:, :, t], v[:, :, t], alpha[:, :, t], beta[:, :, t])
        keep = r[:, gidx, c] == LIN
        carry = np.where(keep[:, :, None, None], S, carry)
    S = carry.copy()
    for t in range(nc_full * chunk, n):
        S = gdn_token_update(S, k[:, :, t], v[:, :, t], alpha[:, :, t], beta[:, :, t])
    cache["S_carry"] = carry
    cache["S_work"] = S if n > nc_full * chunk else np.zeros_like(S)
    return cache


def decode_step(cache, x, q, k, v, alpha, beta, w_score, w_mix, b_score=None, g_sm=None, g_lin=None,
                scale=None, eps=1e-6, chunk=CHUNK):
    """One new token per sequence against the decode cache.

    x [B,d]; q, k, v [B,H,D]; alpha, beta [B,H].  Returns (out [B,H,D],
    dict of branch values, new cache).  The new token joins the open chunk:
    it attends to the committed softmax chunks, the open chunk's earlier
    tokens and itself; the GDN state is pseudo-updated from S_carry (first
    token of a chunk) or S_work.  When the chunk completes it is routed; a
    softmax route commits its KV, a linear route commits its state."""
    x, q, k, v, alpha, beta = map(_f64, (x, q, k, v, alpha, beta))
    c = {key: (val.copy() if isinstance(val, np.ndarray) else val) for key, val in cache.items()}
    B, H, D = q.shape
    G = c["n_open"].shape[1]
    cap = c["k"].shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    o_sm = np.zeros((B, H, D))
    o_gdn = np.zeros((B, H, D))
    for b in range(B):
        for h in range(H):
            g = group_of_head(h, H, G)
            nco, nop = int(c["n_committed"][b, g]), int(c["n_open"][b, g])
            S_src = c["S_carry"][b, h] if nop == 0 else c["S_work"][b, h]
            S_new = gdn_token_update(S_src, k[b, h], v[b, h], alpha[b, h], beta[b, h])
            c["S_work"][b, h] = S_new
            o_gdn[b, h] = gdn_readout(S_new, q[b, h])
            n = nco + nop
            keys = np.concatenate([c["k"][b, h, :n], k[b, h][None]], axis=0)
            vals = np.concatenate([c["v"][b, h, :n], v[b, h][None]], axis=0)
            z = scale * (keys @ q[b, h])
            p = np.exp(z - z.max())
            o_sm[b, h] = (p @ vals) / p.sum()
            if n < cap:
                c["k"][b, h, n] = k[b, h]
                c["v"][b, h, n] = v[b, h]
            else:
                c["err"] = 1
    out, n_sm, n_lin, w = merge(q[:, :, None], o_sm[:, :, None], o_gdn[:, :, None], w_mix,
                                g_sm, g_lin, eps)
    routes = np.full((B, G), -1, np.int32)
    for b in range(B):
        for g in range(G):
            c["x_sum"][b, g] += x[b]
            c["n_open"][b, g] += 1
            if c["n_open"][b, g] == chunk:
                s = (c["x_sum"][b, g] / chunk) @ _f64(w_score)[:, 2 * g:2 * g + 2]
                if b_score is not None:
                    s = s + _f64(b_score)[2 * g:2 * g + 2]
                rt = SM if s[0] >= s[1] else LIN
                routes[b, g] = rt
                heads = [h for h in range(H) if group_of_head(h, H, G) == g]
                if rt == SM:
                    c["n_committed"][b, g] += chunk
                else:
                    c["S_carry"][b, heads] = c["S_work"][b, heads]
                c["n_open"][b, g] = 0
                c["x_sum"][b, g] = 0.0
    return out[:, :, 0], dict(o_sm=o_sm, o_gdn=o_gdn, n_sm=n_sm[:, :, 0], n_lin=n_lin[:, :, 0],
                              weights=w[:, :, 0], routes=routes), c


# ---------------------------------------------------------------------------
# Native Hybrid Attention: one softmax over compressed slots + a sliding
# window ("Native Hybrid Attention for Efficient Sequence Modeling", section 2
# Methodologie, "Unificatie van Intra-layer Hybridisatie")
# ---------------------------------------------------------------------------
def nha_attention(q, k, v, slot_gate, window, scale=None, query_blocks=None, chunk=CHUNK):
    """Plain per-token definition.

    The page describes it this way: long-term information is compressed into
    a fixed number of key-value slots by a linear RNN update (after Gated Slot
    Attention); the slots are joined with the short-term tokens of a sliding
    window into ONE key-value set, and one softmax attention runs over that
    set.  A window of 0 leaves a pure linear RNN, a window of the whole
    sequence a full Transformer.

    Readings (the page gives no equations):
      * window w (tokens): query t sees the keys of tokens t-w+1 .. t itself;
      * token s enters the slots when it leaves the window, i.e. before query
        s + w is answered (w = 0: every token enters before its own query);
      * slot update, per slot i with the gate a_s[i] in (0, 1) of the
        entering token (the Gated Slot Attention form: forget, then write the
        complement):  K~[i] <- a_s[i] K~[i] + (1 - a_s[i]) k_s, the same for V~;
        slots start at zero;
      * the slots join the key set only once a token has entered them, so
        w >= L is exactly causal softmax attention.
    q, k, v [B,H,L,D]; slot_gate [B,H,L,m]; returns o [B,H,L,D].
    query_blocks, if given, lists the 64-row query blocks whose outputs are
    computed (the slots still take every token); other rows stay zero."""
    q, k, v, a = map(_f64, (q, k, v, slot_gate))
    B, H, L, D = q.shape
    m = a.shape[3]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    o = np.zeros_like(v)
    wanted = None if query_blocks is None else set(query_blocks)
    for b in range(B):
        for h in range(H):
            Ks = np.zeros((m, D))
            Vs = np.zeros((m, D))
            entered = 0
            for t in range(L):
                s = t - window  # the token that leaves the window before query t
                if s >= 0:
                    g = a[b, h, s][:, None]
                    Ks = g * Ks + (1.0 - g) * k[b, h, s][None, :]
                    Vs = g * Vs + (1.0 - g) * v[b, h, s][None, :]
                    entered += 1
                if wanted is not None and t // chunk not in wanted:
                    continue
                lo = max(0, t - window + 1)
                keys = [k[b, h, lo:t + 1]]
                vals = [v[b, h, lo:t + 1]]
                if entered:
                    keys.insert(0, Ks)
                    vals.insert(0, Vs)
                kk = np.concatenate(keys, axis=0)
                vv = np.concatenate(vals, axis=0)
                if kk.shape[0] == 0:
                    continue
                z = scale * (kk @ q[b, h, t])
                p = np.exp(z - z.max())
                o[b, h, t] = (p @ vv) / p.sum()
    return o


def nha_attention_bruteforce(q, k, v, slot_gate, window, scale=None):
    """Brute-force twin: every query builds its slots from scratch as the
    closed-form sum over the tokens that have entered them,
        K~_t[i] = sum_{s <= t-w} (prod_{s < r <= t-w} a_r[i]) (1 - a_s[i]) k_s,
    then takes one softmax over [slots; window keys].  Tiny inputs only."""
    q, k, v, a = map(_f64, (q, k, v, slot_gate))
    B, H, L, D = q.shape
    m = a.shape[3]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    o = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            for t in range(L):
                last = t - window
                keys, vals = [], []
                if last >= 0:
                    Ks = np.zeros((m, D))
                    Vs = np.zeros((m, D))
                    for s in range(last + 1):
                        wgt = (1.0 - a[b, h, s]) * np.prod(a[b, h, s + 1:last + 1], axis=0)
                        Ks += wgt[:, None] * k[b, h, s][None, :]
                        Vs += wgt[:, None] * v[b, h, s][None, :]
                    keys += list(Ks)
                    vals += list(Vs)
                for s in range(max(0, t - window + 1), t + 1):
                    keys.append(k[b, h, s])
                    vals.append(v[b, h, s])
                if not keys:
                    continue
                z = np.array([scale * float(q[b, h, t] @ kk) for kk in keys])
                p = np.exp(z - z.max())
                p /= p.sum()
                o[b, h, t] = sum(pi * vv for pi, vv in zip(p, vals))
    return o
