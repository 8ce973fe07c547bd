"""The entry point that allocates nothing (moba_forward_noalloc) against
moba_forward_ex, through the C ABI: the same output, selection and
log-sum-exp bits on two calls in a row, the second on a smaller problem
(the scratch array keeps the first call's contents)."""

import pytest
import torch

import moba_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _pair(moba, w):
    q, k, v = moba_inputs.make_inputs(w, device=DEV)
    S = 1 if q.dim() == 3 else q.shape[0]
    Lq, H = q.shape[-3], q.shape[-2]
    ref, rsel, rlse = moba.moba_forward_ex(q, k, v, w.block_size, w.topk, return_selection=True,
                                           return_lse=True)
    out = torch.empty_like(q)
    sel = torch.full((S, H, Lq, w.topk), -7, dtype=torch.int32, device=DEV)
    lse = torch.full((S, H, Lq), 7.0, dtype=torch.float32, device=DEV)
    got = moba.moba_forward_noalloc(q, k, v, w.block_size, w.topk, out=out, sel_out=sel,
                                    lse_out=lse)
    torch.cuda.synchronize()
    bits = torch.int16 if q.dtype == torch.bfloat16 else torch.int32
    assert got is out
    assert torch.equal(out.view(bits), ref.view(bits)), w.name
    assert torch.equal(sel.view(rsel.shape), rsel), w.name
    assert torch.equal(lse.view(rlse.shape), rlse), w.name
    print(f"  {w.name}: bitwise equal to moba_forward_ex", flush=True)


def test_noalloc_equals_forward_ex_on_two_calls():
    moba = pytest.importorskip("block_sparse_attention_gate_amd")
    # 32K tokens, one head (the own block on the caller's stream, no internal
    # stream), then a smaller GQA problem with a ragged length
    _pair(moba, moba_inputs.WORKLOADS["micro_32k"])
    _pair(moba, moba_inputs.custom("noalloc_small", "bf16", 2, 3000, None, 4, 2, 128, 256, 4, 71))
