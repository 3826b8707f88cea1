"""Helpers shared by the GPU parity tests (test code only)."""
import numpy as np
import torch

import oracle as O
import workloads as W

TOL_F32 = 1e-4   # fp32 workloads: max abs on out and on each RMS-normalised branch
TOL_BF16 = 3e-2  # bf16 workloads: max abs on RMS-normalised outputs


def dev(a, io=None):
    """numpy -> cuda tensor; io="bf16" converts float32 values (already
    bf16-representable) to torch.bfloat16 exactly."""
    t = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    if io == "bf16" and t.dtype == torch.float32:
        t = t.to(torch.bfloat16)
    return t


def dev_bits(u):
    """bf16 bit patterns (uint16 numpy) -> cuda bfloat16 tensor."""
    return torch.from_numpy(np.ascontiguousarray(u).view(np.int16)).cuda().view(torch.bfloat16)


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def rmsn(o, eps=1e-6):
    o = np.asarray(o, np.float64)
    return o / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)


def maxerr(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64)))) if np.size(a) else 0.0


def prefill_tensors(inp):
    io = inp["io"]
    t = {k: dev(inp[k], io) for k in ("x", "q", "k", "v")}
    for k in ("alpha", "beta", "w_score", "w_mix", "b_score", "g_sm", "g_lin"):
        t[k] = dev(inp[k])
    return t


def oracle_head(inp, b, h, route_b, query_blocks=None, S_init=None):
    """Oracle branches and merge for one (b, h) of a prefill input.
    route_b is that sequence's route [G=1, Nc]."""
    sl = lambda a: a[b:b + 1, h:h + 1]
    r = np.asarray(route_b)[None]
    o_sm = O.softmax_branch(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), r, query_blocks=query_blocks)
    o_gdn, S = O.gdn_branch(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["alpha"]), sl(inp["beta"]), r,
                            S_init=None if S_init is None else S_init[b:b + 1, h:h + 1])
    out, n_sm, n_lin, _ = O.merge(sl(inp["q"]), o_sm, o_gdn, inp["w_mix"], inp["g_sm"], inp["g_lin"])
    return dict(out=out[0, 0], n_sm=n_sm[0, 0], n_lin=n_lin[0, 0], o_sm=o_sm[0, 0], o_gdn=o_gdn[0, 0],
                S_final=S[0, 0])


def rows_of_blocks(blocks, chunk=64):
    return np.concatenate([np.arange(c * chunk, (c + 1) * chunk) for c in blocks])
