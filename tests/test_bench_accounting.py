"""The benchmark's work accounting (CPU only): the closed-form effective FLOPs
of bench.prefill_flops against the key sets the oracle actually selects, and
the routed-entry counts of the measured shapes."""

import numpy as np
import pytest

import bench
import moba_inputs
from oracle import moba_oracle as O


@pytest.mark.parametrize("L,Lq,B,topk,H,D", [(200, 200, 16, 3, 2, 8), (333, 333, 32, 5, 1, 4),
                                             (300, 77, 64, 2, 4, 8), (129, 129, 64, 12, 2, 4)])
def test_prefill_flops_equals_the_selected_key_count(L, Lq, B, topk, H, D):
    """4 D FLOPs per (query, key) pair over the keys each query attends
    (selected past blocks whole, its own block up to itself), counted from
    the oracle's selection on random inputs; full attention counts keys
    0..i.  Chunked queries (q_len < kv_len) and a partial last block
    included."""
    w = moba_inputs.custom("acct", "f32", 1, Lq, L, H, 1, D, B, topk, 3)
    rng = np.random.default_rng(L + Lq)
    q = rng.standard_normal((Lq, H, D))
    k = rng.standard_normal((L, 1, D))
    pos = (L - Lq) + np.arange(Lq)
    sel, _ = O.select_all(q, O.block_mean(k, B), B, topk, positions=pos)
    routed = own = full = 0
    for h in range(H):
        for r, i in enumerate(pos):
            b = i // B
            past = [j for j in sel[h, r] if 0 <= j < b]
            routed += B * len(past)
            own += i - b * B + 1
            full += i + 1
    f = 4 * D
    eff, froute, fown, ffull = bench.prefill_flops(w)
    assert (froute, fown, ffull) == (f * routed, f * own, f * full)
    assert eff == f * (routed + own)


@pytest.mark.parametrize("name,entries", [("micro_32k", 59_392),
                                          ("llama8b_128k", 37_486_592),
                                          ("prefill_1m", 360_448_000)])
def test_routed_entries_of_the_measured_shapes(name, entries):
    """Routed (query-head, past block) pairs E = H B sum_b min(k-1, b): 59,392
    at 32K (block 2048, top-k 3, one head), 37,486,592 at 128K and
    360,448,000 at 1M (32 heads, block 4096, top-k 12)."""
    w = moba_inputs.WORKLOADS[name]
    _, routed, _, _ = bench.prefill_flops(w)
    assert routed == 4 * w.head_dim * w.block_size * entries
