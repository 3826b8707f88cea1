"""natsl_decode_step_noalloc (no workspace: the library's per-device scratch
array) against natsl_decode_step (caller's workspace), through the C ABI.

Two calls in a row, the second with a smaller input (fewer sequences and
heads, a smaller cache, so a different scratch layout over the same array):
each is compared with the workspace entry point run on an identical copy of
the cache, for a plain step and a chunk-completing step.  Both paths run the
same kernels on the same inputs, so outputs, routes and the whole cache must
be bit-identical (stricter than the bf16 / fp32 parity tolerances)."""
import sys

import numpy as np
import pytest
import torch

import linear_attention_natsl_amd as N

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def make_state(B, H, D, d, cap, io, n_committed, n_open, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    st = N.DecodeState(B, H, D, d, cap, io=io)
    st.k.copy_(torch.randn(st.k.shape, generator=g, device="cuda").to(io))
    st.v.copy_(torch.randn(st.v.shape, generator=g, device="cuda").to(io))
    st.n_committed.fill_(n_committed)
    st.n_open.fill_(n_open)
    st.S_carry.copy_(torch.randn(st.S_carry.shape, generator=g, device="cuda") / D ** 0.5)
    st.S_work.copy_(torch.randn(st.S_work.shape, generator=g, device="cuda") / D ** 0.5)
    st.x_sum.copy_(torch.randn(st.x_sum.shape, generator=g, device="cuda") * max(n_open, 1) ** 0.5)
    return st


def clone_state(st, B, H, D, d, io):
    c = N.DecodeState(B, H, D, d, st.cap, io=io)
    for name in ("k", "v", "n_committed", "n_open", "S_carry", "S_work", "x_sum", "err"):
        getattr(c, name).copy_(getattr(st, name))
    return c


def step_inputs(B, H, D, d, io, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    r = lambda *s: torch.randn(*s, generator=g, device="cuda")
    k = r(B, H, D)
    k = k / k.norm(dim=-1, keepdim=True)
    return [r(B, d).to(io), r(B, H, D).to(io), k.to(io), r(B, H, D).to(io),
            0.9 + 0.099 * torch.rand(B, H, generator=g, device="cuda"),
            torch.sigmoid(r(B, H)), r(d, 2) * 0.05, r(D, 2) * 0.1]


@pytest.mark.parametrize("io,D", [(torch.bfloat16, 128), (torch.float32, 64)])
def test_noalloc_decode_matches_workspace_entry(io, D):
    d = 256
    code = N.BF16 if io == torch.bfloat16 else N.F32
    # (B, H, cap, n_committed, n_open): large first, then smaller; n_open = 63
    # completes the chunk (route from x_sum, commit), 5 does not
    cases = [(32, 16, 4160, 4032, 63), (32, 16, 4160, 2048, 5), (4, 4, 1088, 960, 63), (3, 2, 576, 320, 5)]
    for i, (B, H, cap, nco, nop) in enumerate(cases):
        say(f"[noalloc] io={io} D={D} call {i}: B={B} H={H} cap={cap} n_committed={nco} n_open={nop}")
        need = N.workspace_size(N.ENTRY_DECODE_STEP, N.dims(B, H, cap, D, d, code))
        assert need <= N.DECODE_NOALLOC_SCRATCH_BYTES
        dm = N.dims(B, H, 1, D, d, code)
        st_ws = make_state(B, H, D, d, cap, io, nco, nop, seed=100 + i)
        st_na = clone_state(st_ws, B, H, D, d, io)
        args = step_inputs(B, H, D, d, io, seed=200 + i)
        dec_ws = N.Decode(dm, st_ws, debug=True)
        dec_na = N.Decode(dm, st_na, debug=True, noalloc=True)
        for _ in range(2):  # two steps each: the second reads what the first left in the cache
            dec_ws(*args)
            dec_na(*args)
        torch.cuda.synchronize()
        assert torch.equal(dec_ws.out, dec_na.out), "out differs"
        assert torch.equal(dec_ws.route, dec_na.route)
        assert torch.equal(dec_ws.o_sm, dec_na.o_sm) and torch.equal(dec_ws.o_gdn, dec_na.o_gdn)
        for name in ("k", "v", "n_committed", "n_open", "S_carry", "S_work", "x_sum", "err"):
            assert torch.equal(getattr(st_ws, name), getattr(st_na, name)), name
        assert torch.isfinite(dec_na.out.float()).all()
        # n_open = 63: the first step completed the chunk (63 -> 0), the second opened the next (-> 1)
        assert (st_na.n_open == (1 if nop == 63 else nop + 2)).all()
        say(f"  identical (routes {dec_na.route.flatten()[:4].tolist()} ...)")


def test_noalloc_rejects_oversized_dims():
    """Dims needing more scratch than the array holds fail with
    NATSL_ERR_WORKSPACE before anything is enqueued (the cache is untouched)."""
    B, H, D, d, cap = 64, 16, 128, 256, 40000
    need = N.workspace_size(N.ENTRY_DECODE_STEP, N.dims(B, H, cap, D, d, N.BF16))
    assert need > N.DECODE_NOALLOC_SCRATCH_BYTES
    st = N.DecodeState(B, H, D, d, cap, io=torch.bfloat16)
    dec = N.Decode(N.dims(B, H, 1, D, d, N.BF16), st, noalloc=True)
    args = step_inputs(B, H, D, d, torch.bfloat16, seed=5)
    with pytest.raises(N.NatslError) as e:
        dec(*args)
    assert e.value.status == 3
    torch.cuda.synchronize()
    assert int(st.n_open.sum().item()) == 0 and int(st.err.item()) == 0
