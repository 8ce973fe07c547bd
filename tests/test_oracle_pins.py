"""Pins of the CPU oracle to things other than itself (CPU only).

Each test names the passage or the mathematical fact it checks.  Together they
are meant to fail on any plausible slip in the oracle: a wrong softmax scale
or causal diagonal (SDPA pins, P5), a wrong tie-break (P2, P7, P8), a wrong
own-block count (P2, P6, golden example), a transposed gate (P6, P10), a
wrong GQA head map (GQA pin), a wrong pooling axis (block-mean pins) or a
wrong query alignment (decode pin).
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import moba_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _case(seed, L, H=1, Hkv=1, D=8, B=4, offset=0.5):
    rng = np.random.default_rng(seed)
    nb = -(-L // B)
    off = rng.standard_normal((nb, Hkv, D)) * offset
    q = rng.standard_normal((L, H, D))
    k = rng.standard_normal((L, Hkv, D)) + off[np.arange(L) // B]
    v = rng.standard_normal((L, Hkv, D))
    return q, k, v


def _sdpa(q, k, v, mask=None, causal=False):
    """torch CPU float64 scaled_dot_product_attention, KV heads repeated."""
    H, Hkv = q.shape[1], k.shape[1]
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(H // Hkv, 0)[None]
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(H // Hkv, 0)[None]
    m = None if mask is None else torch.from_numpy(mask)[None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m,
                                                         is_causal=causal)
    return o[0].permute(1, 0, 2).numpy()


# ---------------------------------------------------------------- golden ---
def test_golden_hand_worked_example():
    """Hand-derived closed forms for a 6-token case (tests/golden/)."""
    g = json.load(open(os.path.join(GOLDEN, "hand_worked_6tok.json")))
    L = g["seq_len"]
    q = np.array(g["q"], float).reshape(L, 1, 1)
    k = np.array(g["k"], float).reshape(L, 1, 1)
    v = np.array(g["v"], float).reshape(L, 1, 1)
    out, sel, gap = O.moba_reference(q, k, v, g["block_size"], g["topk"])
    env = {"e": math.e, "exp": math.exp}
    want = np.array([eval(x, {}, env) for x in g["out_closed_form"]])
    np.testing.assert_allclose(out[:, 0, 0], want, rtol=0, atol=1e-14)
    assert sel[0].tolist() == g["sel"]
    assert [float(x) for x in g["gap"]] == gap[0].tolist()


def test_golden_hand_worked_head_dim_4():
    """Hand-derived selections, gate gaps and outputs at head_dim 4
    (tests/golden/): integer block means and queries, so the gaps are exact
    integers of the UNSCALED gate (reading R1), while the attention logits
    carry the 1/sqrt(4) scale (R7).  A gate scaled by 1/sqrt(D), a gap taken
    at the wrong rank or a tie broken towards the higher index each change a
    value here."""
    g = json.load(open(os.path.join(GOLDEN, "hand_worked_8tok_d4.json")))
    L, D, B = g["seq_len"], g["head_dim"], g["block_size"]
    q = np.array(g["q"], float).reshape(L, 1, D)
    k = np.array(g["k"], float).reshape(L, 1, D)
    v = np.array(g["v"], float).reshape(L, 1, D)
    kb = O.block_mean(k, B)
    np.testing.assert_array_equal(kb[0], np.array(g["kbar"], float))
    np.testing.assert_array_equal(O.gate_scores(q[6, 0], kb[0], 3), [1.0, 4.0, -1.0])
    np.testing.assert_array_equal(O.gate_scores(q[7, 0], kb[0], 3), [0.0, 0.0, 1.0])
    assert O.select_blocks(O.gate_scores(q[7, 0], kb[0], 3), 3, 3) == ((0, 2, 3), 0.0)
    assert O.select_blocks(O.gate_scores(q[6, 0], kb[0], 3), 3, 2) == ((1, 3), 3.0)
    env = {"e": math.e, "exp": math.exp}
    for topk_s, case in g["cases"].items():
        topk = int(topk_s)
        out, sel, gap = O.moba_reference(q, k, v, B, topk)
        assert sel[0].tolist() == case["sel"], topk
        assert gap[0].tolist() == [float(x) for x in case["gap"]], topk
        sel2, gap2 = O.select_all(q, kb, B, topk)
        assert sel2[0].tolist() == case["sel"] and gap2[0].tolist() == gap[0].tolist()
        if "out0_closed_form" in case:
            want = np.array([eval(x, {}, env) for x in case["out0_closed_form"]])
            np.testing.assert_allclose(out[:, 0, 0], want, rtol=0, atol=1e-14)
            np.testing.assert_allclose(out[:, 0, 1], 1.0, rtol=0, atol=1e-14)
            np.testing.assert_array_equal(out[:, 0, 2:], 0.0)


def test_gap_is_the_boundary_difference_of_the_raw_scores_at_d128():
    """At head_dim 128 the gate gap equals the (k-1)-th minus the k-th largest
    past score of kbar @ q (no 1/sqrt(D) factor), taken from a full sort of
    the raw dot products of every query."""
    rng = np.random.default_rng(77)
    L, B, D, topk = 512, 32, 128, 4
    q = rng.standard_normal((L, 2, D))
    kb = rng.standard_normal((1, L // B, D)) * 0.5
    sel, gap = O.select_all(q, kb, B, topk)
    checked = 0
    for h in range(2):
        for i in range(L):
            b = i // B
            s = np.sort(np.array([np.dot(kb[0, j], q[i, h]) for j in range(b)]))[::-1]
            if b > topk - 1:
                assert gap[h, i] == pytest.approx(s[topk - 2] - s[topk - 1], abs=1e-12)
                checked += 1
            else:
                assert gap[h, i] == math.inf
    assert checked > 0


# ------------------------------------------------------------- pooling -----
def test_block_mean_ramp_and_partial_block():
    """Mean of a ramp K[t] = t is the block midpoint; a partial last block is
    averaged over the keys it holds (reading R11)."""
    B, L = 8, 29
    k = np.broadcast_to(np.arange(L, dtype=float)[:, None, None], (L, 2, 3)).copy()
    k[:, 1] *= -2.0
    kb = O.block_mean(k, B)
    assert kb.shape == (2, 4, 3)
    for j in range(4):
        lo, hi = j * B, min(L, (j + 1) * B)
        mid = (lo + hi - 1) / 2.0
        np.testing.assert_allclose(kb[0, j], mid, atol=1e-13)
        np.testing.assert_allclose(kb[1, j], -2 * mid, atol=1e-13)


def test_block_mean_block_size_one_is_identity():
    q, k, v = _case(3, 17, Hkv=2, D=5, B=1)
    np.testing.assert_array_equal(O.block_mean(k, 1), k.transpose(1, 0, 2))


# ------------------------------------------------------- P1 invariants -----
@pytest.mark.parametrize("seed,L,B,topk", [(0, 64, 8, 3), (1, 100, 16, 5), (2, 33, 4, 1),
                                           (3, 48, 8, 20), (4, 128, 32, 2)])
def test_p1_selection_invariants(seed, L, B, topk):
    """Own block present, it is the largest index, nothing from the future,
    size min(k, b+1), ascending and unique, -1 padding last (causality design
    of the AiBoss page; readings R2, R3)."""
    q, k, v = _case(seed, L, H=2, Hkv=1, D=6, B=B)
    sel, gap = O.select_all(q, O.block_mean(k, B), B, topk)
    for h in range(2):
        for i in range(L):
            b = i // B
            row = sel[h, i].tolist()
            valid = [x for x in row if x >= 0]
            assert row == valid + [-1] * (topk - len(valid))
            assert b in valid and max(valid) == b
            assert len(valid) == min(topk, b + 1)
            assert valid == sorted(set(valid))


# ------------------------------------------------------ P2 brute force -----
@pytest.mark.parametrize("B", [1, 2, 4, 8])
def test_p2_brute_force_selection(B):
    """Exhaustive subset enumeration on tiny inputs, with integer-valued data
    so that exact ties are common (reading R4: lowest index wins)."""
    rng = np.random.default_rng(10 + B)
    L, D = {1: 14, 2: 28, 4: 48, 8: 64}[B], 3
    q = rng.integers(-1, 2, size=(L, 1, D)).astype(float)
    k = rng.integers(-2, 3, size=(L, 1, D)).astype(float)
    kb = O.block_mean(k, B)
    nb = kb.shape[1]
    for topk in range(1, min(nb, 6) + 2):
        sel, _ = O.select_all(q, kb, B, topk)
        for i in range(L):
            b = i // B
            s = O.gate_scores(q[i, 0], kb[0], b)
            want = O.brute_force_select(s, b, topk)
            assert tuple(sel[0, i].tolist()) == want, (topk, i)
            assert O.select_blocks(s, b, topk)[0] == want


# ---------------------------------------------- P3 sparse -> full switch ----
@pytest.mark.parametrize("H,Hkv", [(1, 1), (4, 2), (4, 1)])
def test_p3_topk_all_equals_full_causal_attention(H, Hkv):
    """topk >= number of blocks is full causal attention (seamless full/sparse
    switching: MoBA card 'How It Works', AiBoss '主な機能'); checked against
    torch's float64 SDPA with is_causal (its default scale is 1/sqrt(D))."""
    L, B, D = 40, 8, 16
    q, k, v = _case(21, L, H, Hkv, D, B)
    nb = L // B
    for topk in (nb, nb + 3):
        out, sel, _ = O.moba_reference(q, k, v, B, topk)
        np.testing.assert_allclose(out, _sdpa(q, k, v, causal=True), atol=1e-12, rtol=0)
    np.testing.assert_allclose(O.full_reference(q, k, v), _sdpa(q, k, v, causal=True),
                               atol=1e-12, rtol=0)


# ------------------------------------------------ P4 mask form vs gather ----
@pytest.mark.parametrize("seed,L,B,topk,H,Hkv", [(31, 64, 8, 3, 1, 1), (32, 72, 8, 4, 4, 2),
                                                 (33, 50, 16, 2, 2, 2)])
def test_p4_gather_equals_mask_form_equals_sdpa(seed, L, B, topk, H, Hkv):
    """The naive mask version and the gathered version compute the same thing
    (Dev Tutorial step 1; MoBA card 'Limitations & Caveats'), and both equal
    torch SDPA with the boolean mask built from the selection."""
    q, k, v = _case(seed, L, H, Hkv, 16, B)
    out, sel, _ = O.moba_reference(q, k, v, B, topk)
    naive = O.naive_mask_reference(q, k, v, B, topk)
    np.testing.assert_allclose(out, naive, atol=1e-12, rtol=0)
    t = np.arange(L)
    mask = np.zeros((H, L, L), dtype=bool)
    for h in range(H):
        for i in range(L):
            chosen = [j for j in sel[h, i] if j >= 0]
            mask[h, i] = np.isin(t // B, chosen) & (t <= i)
    np.testing.assert_allclose(out, _sdpa(q, k, v, mask=mask), atol=1e-12, rtol=0)


# ------------------------------------------- property tests (hypothesis) ---
try:
    from hypothesis import given, settings, strategies as st
except ImportError:  # pragma: no cover - hypothesis is part of the test image
    given = None

if given is not None:
    _shapes = st.tuples(
        st.integers(0, 2**31 - 1),                       # seed
        st.integers(1, 256),                             # L
        st.sampled_from([1, 2, 4, 8, 16, 32, 64]),       # B
        st.sampled_from([(1, 1), (2, 1), (4, 2)]),       # (H, Hkv)
        st.integers(1, 8),                               # head dim
    )

    @settings(max_examples=60, deadline=None)
    @given(_shapes, st.data())
    def test_property_selection_invariants_and_forms(shape, data):
        """Random small shapes (L <= 256, B in 1..64, topk 1..nb+1, GQA):
        the selection keeps its invariants (own block present and largest,
        nothing from the future, min(k, b+1) blocks, ascending, -1 padding;
        readings R2, R3), and the gathered form equals the mask form (Dev
        Tutorial step 1; MoBA card 'Limitations & Caveats') and torch's
        float64 SDPA with the boolean mask built from the selection."""
        seed, L, B, (H, Hkv), D = shape
        nb = -(-L // B)
        topk = data.draw(st.integers(1, nb + 1), label="topk")
        q, k, v = _case(seed, L, H, Hkv, D, B)
        out, sel, _ = O.moba_reference(q, k, v, B, topk)
        t = np.arange(L)
        mask = np.zeros((H, L, L), dtype=bool)
        for h in range(H):
            for i in range(L):
                b = i // B
                row = sel[h, i].tolist()
                valid = [x for x in row if x >= 0]
                assert row == valid + [-1] * (topk - len(valid))
                assert b in valid and max(valid) == b
                assert len(valid) == min(topk, b + 1)
                assert valid == sorted(set(valid))
                mask[h, i] = np.isin(t // B, valid) & (t <= i)
        np.testing.assert_allclose(out, O.naive_mask_reference(q, k, v, B, topk),
                                   atol=1e-12, rtol=0)
        np.testing.assert_allclose(out, _sdpa(q, k, v, mask=mask), atol=1e-12, rtol=0)


# -------------------------------------------------- P5 local attention -----
def test_p5_topk_one_is_block_diagonal_causal():
    """k = 1 keeps only the own block with its causal mask: block-diagonal
    causal attention; a query at a block start sees only itself."""
    L, B = 48, 8
    q, k, v = _case(41, L, 2, 1, 8, B)
    out, sel, _ = O.moba_reference(q, k, v, B, 1)
    t = np.arange(L)
    mask = (t[None, :] <= t[:, None]) & (t[None, :] // B == t[:, None] // B)
    mask = np.broadcast_to(mask, (2, L, L)).copy()
    np.testing.assert_allclose(out, _sdpa(q, k, v, mask=mask), atol=1e-12, rtol=0)
    for i in range(0, L, B):
        np.testing.assert_allclose(out[i, :, :], np.repeat(v[i, 0][None], 2, 0), atol=1e-14)
    out3, _, _ = O.moba_reference(q, k, v, B, 3)
    np.testing.assert_allclose(out3[0], np.repeat(v[0, 0][None], 2, 0), atol=1e-14)


# --------------------------------------------- P6 token-level top-k --------
def test_p6_block_size_one_is_token_topk():
    """B = 1 makes every key its own block: Sel = {i} plus the k-1 earlier
    tokens with the largest q.k_t (ties to the lower index)."""
    L, topk = 30, 4
    q, k, v = _case(51, L, 1, 1, 5, 1)
    sel, _ = O.select_all(q, O.block_mean(k, 1), 1, topk)
    for i in range(L):
        s = k[:i, 0] @ q[i, 0]
        order = np.lexsort((np.arange(i), -s))[: topk - 1]
        want = sorted(order.tolist() + [i])
        want += [-1] * (topk - len(want))
        assert sel[0, i].tolist() == want


# --------------------------------------------- P7 zero query closed form ---
def test_p7_zero_query_closed_form():
    """q = 0 makes every gate score 0: the lowest-index past blocks win, and
    every attended key gets the same weight, so out is the plain mean of V
    over the attended keys."""
    L, B, topk = 64, 8, 3
    q, k, v = _case(61, L, 1, 1, 8, B)
    q[:] = 0.0
    out, sel, _ = O.moba_reference(q, k, v, B, topk)
    for i in range(L):
        b = i // B
        past = list(range(min(topk - 1, b)))
        assert [x for x in sel[0, i] if x >= 0] == past + [b]
        keys = [t for j in past for t in range(j * B, (j + 1) * B)] + list(range(b * B, i + 1))
        np.testing.assert_allclose(out[i, 0], v[keys, 0].mean(axis=0), atol=1e-13)


# ---------------------------------------------- P8 duplicate-block tie -----
def test_p8_duplicate_block_exact_tie_goes_to_lower_index():
    L, B, D = 64, 8, 8
    rng = np.random.default_rng(71)
    q = rng.standard_normal((L, 1, D))
    k = rng.standard_normal((L, 1, D)) * 0.1
    u = q[-1, 0] / np.linalg.norm(q[-1, 0])
    k[2 * B:3 * B, 0] = u * 5.0 + k[2 * B:3 * B, 0] * 0.01
    k[5 * B:6 * B] = k[2 * B:3 * B]                       # block 5 == block 2
    sel, gap = O.select_all(q, O.block_mean(k, B), B, 2)
    assert sel[0, L - 1].tolist() == [2, 7]
    assert gap[0, L - 1] == 0.0


# ------------------------------------------------- P9 softmax weights -----
def test_p9_one_hot_values_expose_the_weights():
    """With V[t] = e_t the output row is the attention weight vector: it sums
    to one, is zero off the key set, and equals exp-normalised logits."""
    L, B, topk = 24, 4, 3
    q, k, _ = _case(81, L, 1, 1, 6, B)
    v = np.eye(L)[:, None, :]
    out, sel, _ = O.moba_reference(q, k, v, B, topk)
    for i in range(L):
        keys = O.key_set(sel[0, i], i, B, L)
        w = out[i, 0]
        np.testing.assert_allclose(w.sum(), 1.0, atol=1e-14)
        off = np.setdiff1d(np.arange(L), keys)
        assert np.all(w[off] == 0.0)
        z = k[keys, 0] @ q[i, 0] / math.sqrt(6)
        ref = torch.softmax(torch.from_numpy(z), 0).numpy()
        np.testing.assert_allclose(w[keys], ref, atol=1e-14)
    vc = np.ones((L, 1, 5)) * np.array([1.5, -2.0, 0.0, 3.25, 7.0])
    outc, _, _ = O.moba_reference(q, k, vc, B, topk)
    np.testing.assert_allclose(outc[:, 0], np.broadcast_to(vc[0, 0], (L, 5)), atol=1e-13)


# ---------------------------------------- P10 scaling / head permutation ---
def test_p10_power_of_two_query_scaling_and_head_permutation():
    L, B, topk = 64, 8, 4
    q, k, v = _case(91, L, 4, 2, 8, B)
    kb = O.block_mean(k, B)
    sel, _ = O.select_all(q, kb, B, topk)
    for m in (-3, 5):
        sel2, _ = O.select_all(q * 2.0 ** m, kb, B, topk)
        np.testing.assert_array_equal(sel, sel2)
    out, _, _ = O.moba_reference(q, k, v, B, topk)
    perm = [1, 0, 3, 2]                                   # swap heads inside each group
    outp, selp, _ = O.moba_reference(q[:, perm], k, v, B, topk)
    np.testing.assert_allclose(outp, out[:, perm], atol=1e-14)
    np.testing.assert_array_equal(selp, sel[perm])


def test_gqa_head_map_uses_h_div_group():
    """Query head h reads KV head h // (H/Hkv) (reading R8): changing KV head 1
    leaves heads 0 and 1 untouched and changes heads 2 and 3."""
    L, B, topk = 48, 8, 3
    q, k, v = _case(101, L, 4, 2, 8, B)
    out, _, _ = O.moba_reference(q, k, v, B, topk)
    k2, v2 = k.copy(), v.copy()
    k2[:, 1] += 1.0
    v2[:, 1] *= -1.0
    out2, _, _ = O.moba_reference(q, k2, v2, B, topk)
    np.testing.assert_array_equal(out2[:, :2], out[:, :2])
    assert np.abs(out2[:, 2:] - out[:, 2:]).max() > 1e-3


# ------------------------------------------------ decode alignment pin -----
def test_decode_rows_equal_prefill_tail():
    """Queries given on their own against the full cache (q_len < kv_len) sit
    at the end of the cache (reading R10) and reproduce the prefill's last
    rows, selection included."""
    L, B, topk, lq = 64, 8, 3, 5
    q, k, v = _case(111, L, 4, 2, 8, B)
    out, sel, gap = O.moba_reference(q, k, v, B, topk)
    outd, seld, gapd = O.moba_reference(q[-lq:], k, v, B, topk)
    np.testing.assert_allclose(outd, out[-lq:], atol=1e-14)
    np.testing.assert_array_equal(seld, sel[:, -lq:])
    outb, selb, _ = O.moba_decode_reference(np.stack([q[-lq:], q[-lq:] * 0.5]),
                                            np.stack([k, k]), np.stack([v, v]), B, topk)
    np.testing.assert_allclose(outb[0], out[-lq:], atol=1e-14)


# --------------------------------------------------------- routing view ----
def test_routing_table_partitions_every_routed_pair():
    """Every (query, selected past block) pair lands exactly once in the bucket
    of (sequence, KV head, block), in ascending slot order; recounted by a
    direct loop."""
    L, B, topk, H, Hkv = 40, 8, 3, 4, 2
    q, k, v = _case(121, L, H, Hkv, 8, B)
    sel, _ = O.select_all(q, O.block_mean(k, B), B, topk)
    sel2 = np.stack([sel, sel[::-1]])                       # batch of 2
    nb = L // B
    counts, offsets, entries = O.routing_table(sel2, Hkv, nb, B, 0)
    buckets = {}
    kp = topk - 1
    for s in range(2):
        for h in range(H):
            for r in range(L):
                for slot in range(min(kp, r // B)):
                    j = int(sel2[s, h, r, slot])
                    assert 0 <= j < r // B
                    key = (s * Hkv + h // (H // Hkv)) * nb + j
                    buckets.setdefault(key, []).append(((s * H + h) * L + r) * kp + slot)
    for key in range(2 * Hkv * nb):
        got = entries[offsets[key]:offsets[key + 1]].tolist()
        assert got == buckets.get(key, []), key
        assert counts[key] == len(got)
    assert offsets[-1] == entries.size == sum(len(x) for x in buckets.values())


def test_select_all_explicit_positions_match_offsets():
    """Sampled rows given with explicit positions select exactly what the
    same rows select in the full query array."""
    L, B, topk = 96, 8, 4
    q, k, v = _case(131, L, 2, 1, 8, B)
    kb = O.block_mean(k, B)
    sel, gap = O.select_all(q, kb, B, topk)
    rows = np.array([0, 7, 8, 50, 95])
    sel2, gap2 = O.select_all(q[rows], kb, B, topk, positions=rows)
    np.testing.assert_array_equal(sel2, sel[:, rows])
    np.testing.assert_array_equal(gap2, gap[:, rows])


# ------------------------------------------------- backward (R15) pins -----
def _selection_mask(sel, L, Lq, B, q_off):
    """Boolean [H, Lq, L] mask of the keys each query attends (selected
    blocks, causal inside)."""
    H = sel.shape[0]
    t = np.arange(L)
    mask = np.zeros((H, Lq, L), dtype=bool)
    for h in range(H):
        for r in range(Lq):
            chosen = [j for j in sel[h, r] if j >= 0]
            mask[h, r] = np.isin(t // B, chosen) & (t <= q_off + r)
    return mask


def _autograd(q, k, v, dout, mask=None, causal=False):
    """torch float64 autograd of SDPA; KV heads repeated (their gradients
    summed back by autograd)."""
    H, Hkv = q.shape[1], k.shape[1]
    qt, kt, vt = (torch.from_numpy(x.copy()).requires_grad_() for x in (q, k, v))
    rep = lambda t: t.permute(1, 0, 2).repeat_interleave(H // Hkv, 0)[None]
    m = None if mask is None else torch.from_numpy(mask)[None]
    o = torch.nn.functional.scaled_dot_product_attention(
        qt.permute(1, 0, 2)[None], rep(kt), rep(vt), attn_mask=m, is_causal=causal)
    (o[0].permute(1, 0, 2) * torch.from_numpy(dout)).sum().backward()
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


@pytest.mark.parametrize("seed,L,Lq,B,topk,H,Hkv", [(61, 72, 72, 8, 4, 4, 2),
                                                    (62, 50, 50, 16, 2, 2, 2),
                                                    (63, 90, 37, 8, 3, 2, 1)])
def test_backward_equals_autograd_of_the_mask_form(seed, L, Lq, B, topk, H, Hkv):
    """R15: with the selection fixed, the oracle's hand-written gradients equal
    torch autograd through SDPA with the selection's boolean mask (ragged last
    block, GQA 2:1, and queries at the end of a longer cache)."""
    q, k, v = _case(seed, L, H, Hkv, 16, B)
    q = q[L - Lq:]
    dout = np.random.default_rng(seed + 100).standard_normal(q.shape)
    kbar = O.block_mean(k, B)
    sel, _ = O.select_all(q, kbar, B, topk, q_offset=L - Lq)
    dq, dk, dv = O.moba_backward_reference(q, k, v, dout, B, sel)
    aq, ak, av = _autograd(q, k, v, dout, mask=_selection_mask(sel, L, Lq, B, L - Lq))
    np.testing.assert_allclose(dq, aq, atol=1e-11, rtol=0)
    np.testing.assert_allclose(dk, ak, atol=1e-11, rtol=0)
    np.testing.assert_allclose(dv, av, atol=1e-11, rtol=0)


def test_backward_topk_all_equals_causal_sdpa_gradients():
    """topk >= nb: the gradients of full causal attention (SDPA is_causal)."""
    L, B, D = 40, 8, 16
    q, k, v = _case(64, L, 4, 1, D, B)
    dout = np.random.default_rng(7).standard_normal(q.shape)
    sel, _ = O.select_all(q, O.block_mean(k, B), B, 6)
    got = O.moba_backward_reference(q, k, v, dout, B, sel)
    want = _autograd(q, k, v, dout, causal=True)
    for g_, w_ in zip(got, want):
        np.testing.assert_allclose(g_, w_, atol=1e-11, rtol=0)


def test_backward_central_differences():
    """The definition of the derivative: central differences of
    sum(out * dout) (selection held fixed) on sampled coordinates of q, k, v."""
    L, B, topk, D = 24, 4, 3, 6
    q, k, v = _case(65, L, 2, 1, D, B)
    dout = np.random.default_rng(8).standard_normal(q.shape)
    sel, _ = O.select_all(q, O.block_mean(k, B), B, topk)
    grads = O.moba_backward_reference(q, k, v, dout, B, sel)

    def loss(q_, k_, v_):
        out, _, _ = O.moba_reference(q_, k_, v_, B, topk, sel=sel)
        return float((out * dout).sum())

    rng = np.random.default_rng(9)
    eps = 1e-6
    for which, g_ in enumerate(grads):
        base = (q, k, v)[which]
        for _ in range(8):
            idx = tuple(int(rng.integers(0, n)) for n in base.shape)
            args_p = [x.copy() for x in (q, k, v)]
            args_m = [x.copy() for x in (q, k, v)]
            args_p[which][idx] += eps
            args_m[which][idx] -= eps
            fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert abs(fd - g_[idx]) <= 1e-7 + 1e-6 * abs(fd), (which, idx, fd, g_[idx])


def test_backward_closed_form_sums():
    """Softmax gradients sum to zero over each query's keys, so the dK of a
    KV head sums to zero over all keys; the probabilities sum to one, so its
    dV sums to the group's dO summed over queries (chunked queries, GQA)."""
    L, Lq, B, topk, H, Hkv, D = 80, 30, 8, 3, 4, 2, 8
    q, k, v = _case(66, L, H, Hkv, D, B)
    q = q[L - Lq:]
    dout = np.random.default_rng(10).standard_normal(q.shape)
    sel, _ = O.select_all(q, O.block_mean(k, B), B, topk, q_offset=L - Lq)
    dq, dk, dv = O.moba_backward_reference(q, k, v, dout, B, sel)
    G = H // Hkv
    for g in range(Hkv):
        np.testing.assert_allclose(dk[:, g].sum(axis=0), 0.0, atol=1e-12)
        want = dout[:, g * G:(g + 1) * G].sum(axis=(0, 1))
        np.testing.assert_allclose(dv[:, g].sum(axis=0), want, atol=1e-12)


def test_lse_equals_logsumexp_of_the_masked_logits():
    """The kept log-sum-exp is torch.logsumexp of the scaled logits over each
    query's key set (masked logits at -inf)."""
    L, B, topk, H, Hkv, D = 60, 8, 3, 2, 1, 16
    q, k, v = _case(67, L, H, Hkv, D, B)
    sel, _ = O.select_all(q, O.block_mean(k, B), B, topk)
    lse = O.moba_lse_reference(q, k, B, sel)
    mask = _selection_mask(sel, L, L, B, 0)
    for h in range(H):
        z = torch.from_numpy(q[:, h] @ k[:, h // (H // Hkv)].T / math.sqrt(D))
        z = z.masked_fill(~torch.from_numpy(mask[h]), -math.inf)
        np.testing.assert_allclose(lse[h], torch.logsumexp(z, dim=1).numpy(), atol=1e-12)


def test_backward_with_a_given_output_differs_by_the_closed_form():
    """Reading dO.o from a given output o' = o + delta changes only the
    softmax term: ds_t changes by -p_t (dO.delta), so dq changes by
    -c (dO.delta) sum_t p_t k_t, dk_t by -c (dO.delta) p_t q, and dv not at
    all (closed form of the change, per query)."""
    L, B, topk, H, Hkv, D = 48, 8, 3, 2, 1, 8
    q, k, v = _case(68, L, H, Hkv, D, B)
    rng = np.random.default_rng(11)
    dout = rng.standard_normal(q.shape)
    sel, _ = O.select_all(q, O.block_mean(k, B), B, topk)
    out, _, _ = O.moba_reference(q, k, v, B, topk, sel=sel)
    delta = rng.standard_normal(out.shape) * 1e-2
    base = O.moba_backward_reference(q, k, v, dout, B, sel)
    same = O.moba_backward_reference(q, k, v, dout, B, sel, out=out)
    for a_, b_ in zip(base, same):
        np.testing.assert_allclose(a_, b_, atol=1e-12, rtol=0)
    dq2, dk2, dv2 = O.moba_backward_reference(q, k, v, dout, B, sel, out=out + delta)
    c = 1.0 / math.sqrt(D)
    want_dq = base[0].copy()
    want_dk = base[1].copy()
    for h in range(H):
        for i in range(L):
            keys = O.key_set(sel[h, i], i, B, L)
            z = k[keys, 0] @ q[i, h] * c
            p = np.exp(z - z.max())
            p /= p.sum()
            e = dout[i, h] @ delta[i, h]
            want_dq[i, h] -= c * e * (p @ k[keys, 0])
            want_dk[keys, 0] -= c * e * np.outer(p, q[i, h])
    np.testing.assert_allclose(dq2, want_dq, atol=1e-12, rtol=0)
    np.testing.assert_allclose(dk2, want_dk, atol=1e-12, rtol=0)
    np.testing.assert_allclose(dv2, base[2], atol=0, rtol=0)


def test_backward_restricted_to_rows_adds_up():
    """``pairs`` restricts the backward to some query rows: those rows' dq
    equal the full computation's, and dk, dv of two disjoint row sets add up
    to the full ones (each query contributes independently)."""
    L, B, topk, H, Hkv, D = 40, 8, 3, 2, 1, 8
    q, k, v = _case(69, L, H, Hkv, D, B)
    dout = np.random.default_rng(12).standard_normal(q.shape)
    sel, _ = O.select_all(q, O.block_mean(k, B), B, topk)
    full = O.moba_backward_reference(q, k, v, dout, B, sel)
    every = [(h, r) for h in range(H) for r in range(L)]
    a = O.moba_backward_reference(q, k, v, dout, B, sel, pairs=every[::2])
    b = O.moba_backward_reference(q, k, v, dout, B, sel, pairs=every[1::2])
    for h, r in every[::2]:
        np.testing.assert_array_equal(a[0][r, h], full[0][r, h])
    np.testing.assert_allclose(a[1] + b[1], full[1], atol=1e-12, rtol=0)
    np.testing.assert_allclose(a[2] + b[2], full[2], atol=1e-12, rtol=0)
