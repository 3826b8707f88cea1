"""Non-finite inputs on the GPU path, through the C ABI.  A NaN planted in
one element of one key or value row, or an infinity in a value row (head 1,
token t0 of chunk 9), must stay where the layer's data flow takes it:
  - the other heads and every token of head 1 before chunk 9 are
    bit-identical to the run without it (causality; heads are independent);
  - token t0's output row and every row after chunk 9 hold a non-finite value
    (the chunk is kept by one branch or the other, so everything after it
    depends on the row);
  - the final Gated DeltaNet state takes the row only when the chunk is
    routed to the linear branch: a softmax-routed chunk's state update is
    rolled back entirely (Kernmechanismen 3 of the NAtS-L summary), so the
    state is then bit-identical to the clean run.
Rows of chunk 9 before t0 are not checked: the blocked products multiply a
masked (zero) weight by the planted value, as any blocked attention does.  An
infinite key is not planted: a score of minus infinity gives its key weight
zero, so later rows may rightly stay finite."""
import sys

import numpy as np
import pytest
import torch

import linear_attention_natsl_amd as N
import workloads as W
from tests.gpu_util import prefill_tensors

pytestmark = pytest.mark.gpu

CH = 9          # chunk holding the planted value
T0 = 64 * CH + 10
HEAD = 1


@pytest.mark.parametrize("io,D", [("bf16", 128), ("f32", 64)])
@pytest.mark.parametrize("field,bad", [("v", float("nan")), ("v", float("inf")), ("k", float("nan"))])
@pytest.mark.parametrize("chunk_route", [N.ROUTE_SOFTMAX, N.ROUTE_LINEAR])
def test_nonfinite_row_is_confined(io, D, field, bad, chunk_route):
    B, H, L, d = 1, 4, 1024, 256
    print(f"[nonfinite] io={io} D={D} field={field} bad={bad} route={chunk_route}", flush=True)
    sys.stdout.flush()
    wl = W.Workload("nonfinite", io, B, H, L, D, d, "forced", 91, {})
    inp = W.make_prefill(wl)
    t = prefill_tensors(inp)
    nc = L // 64
    route = torch.tensor([[[c % 2 for c in range(nc)]]], dtype=torch.int32)
    route[0, 0, CH] = chunk_route
    route = route.cuda()
    dm = N.dims(B, H, L, D, d, N.BF16 if io == "bf16" else N.F32)
    f = N.Forward(dm, want_state=True)

    def run(v, k):
        f(t["x"], t["q"], k, v, t["alpha"], t["beta"], t["w_score"], t["w_mix"], b_score=t["b_score"],
          route_override=route)
        torch.cuda.synchronize()
        return f.out.clone(), f.S_final.clone()

    out0, S0 = run(t["v"], t["k"])
    assert torch.isfinite(out0).all() and torch.isfinite(S0).all()
    bad_t = t[field].clone()
    bad_t[0, HEAD, T0, 5] = bad
    out1, S1 = run(bad_t if field == "v" else t["v"], bad_t if field == "k" else t["k"])
    others = [h for h in range(H) if h != HEAD]
    assert torch.equal(out1[:, others], out0[:, others])
    assert torch.equal(S1[:, others], S0[:, others])
    assert torch.equal(out1[0, HEAD, :64 * CH], out0[0, HEAD, :64 * CH])
    assert not torch.isfinite(out1[0, HEAD, T0]).all()
    later = out1[0, HEAD, 64 * (CH + 1):]
    rows_bad = (~torch.isfinite(later)).any(dim=-1)
    assert rows_bad.all(), f"{int((~rows_bad).sum())} later rows are all finite"
    if chunk_route == N.ROUTE_LINEAR:
        assert not torch.isfinite(S1[0, HEAD]).all()
    else:
        assert torch.equal(S1[0, HEAD], S0[0, HEAD])
