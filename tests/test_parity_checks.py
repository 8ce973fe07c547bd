"""The comparison helpers of the GPU tests reject what they must (CPU only).

The selection rule (MoBA project card, "How It Works": the gate keeps the best
blocks of every query token; reading R5: inside the 1e-3 tie window several
sets are correct) is checked here on hand-made scores, so that a helper that
accepts a wrong set cannot hide a wrong GPU selection.
"""

import numpy as np
import pytest

import parity


def _one_query(scores_past, topk):
    """kbar [1, nb, 1] holding the past scores and the own block, q = 1 at the
    first position of the own block (the block after the past ones)."""
    own = len(scores_past)
    kbar = np.array(list(scores_past) + [0.0], float).reshape(1, own + 1, 1)
    q = np.ones((1, 1, 1))
    B = 4
    return q, np.array([own * B]), kbar, B, own


def test_tie_window_rejects_a_set_that_drops_the_best_block():
    """Scores [10, 5, 4.9995, 1], top-k 3: the boundary gap 5e-4 is inside the
    window, so {0, 2} and {0, 1} are both correct, but {1, 2} drops block 0,
    which beats both kept blocks by ~5."""
    q, pos, kbar, B, own = _one_query([10.0, 5.0, 4.9995, 1.0], 3)
    ok = np.array([[[0, 1, own]]])
    ties, gap = parity.check_selection(q, pos, kbar, ok, B, 3)
    assert ties == 1 and gap[0, 0] == pytest.approx(5e-4)
    parity.check_selection(q, pos, kbar, np.array([[[0, 2, own]]]), B, 3)
    with pytest.raises(AssertionError):
        parity.check_selection(q, pos, kbar, np.array([[[1, 2, own]]]), B, 3)


def test_outside_the_window_the_set_must_equal_the_oracle():
    q, pos, kbar, B, own = _one_query([10.0, 5.0, 4.0, 1.0], 3)
    parity.check_selection(q, pos, kbar, np.array([[[0, 1, own]]]), B, 3)
    with pytest.raises(AssertionError):
        parity.check_selection(q, pos, kbar, np.array([[[0, 2, own]]]), B, 3)


@pytest.mark.parametrize("bad", [[0, 1, -1], [0, -1, 4], [0, 4, 1], [0, 0, 4],
                                 [0, 1, 5], [1, 0, 4]])
def test_tie_window_rejects_malformed_sets(bad):
    """Missing own block, short set, unsorted, repeated, a future block."""
    q, pos, kbar, B, own = _one_query([10.0, 5.0, 4.9995, 1.0], 3)
    assert own == 4
    with pytest.raises(AssertionError):
        parity.check_selection(q, pos, kbar, np.array([[bad]]), B, 3)


def test_tie_window_set_check_directly():
    s = np.array([10.0, 5.0, 4.9995, 1.0])
    parity.check_tie_window_set(s, [0, 2, 4], 4, 3)
    parity.check_tie_window_set(s, [0, 1, 4], 4, 3)
    with pytest.raises(AssertionError):
        parity.check_tie_window_set(s, [1, 2, 4], 4, 3)
    with pytest.raises(AssertionError):
        parity.check_tie_window_set(s, [0, 3, 4], 4, 3)


def _rows_case(seed, L=1024, B=64, D=16, topk=4):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((L, 1, D))
    kbar = rng.standard_normal((1, L // B, D)) * 0.5
    sel, gap = parity.O.select_all(q, kbar, B, topk)
    return q[:, 0], kbar[0], sel[0].copy(), gap[0], B, topk


def test_all_rows_check_accepts_the_oracle_selection():
    q, kbar, sel, gap, B, topk = _rows_case(1)
    ties, n = parity.check_selection_all_rows(q, kbar, sel, B, topk)
    assert n == q.shape[0] and ties == int((gap < parity.TIE).sum())


def test_all_rows_check_with_a_query_offset():
    q, kbar, sel, gap, B, topk = _rows_case(2)
    off = 300
    parity.check_selection_all_rows(q[off:], kbar, sel[off:], B, topk, q_offset=off)


@pytest.mark.parametrize("plant", ["swap_block", "drop_own", "unsorted", "future"])
def test_all_rows_check_rejects_a_planted_wrong_row(plant):
    q, kbar, sel, gap, B, topk = _rows_case(3)
    r = 1000                      # block 15: 3 of 15 past blocks kept
    assert gap[r] >= parity.TIE
    row = sel[r].copy()
    if plant == "swap_block":     # replace a kept past block by a dropped one
        dropped = [j for j in range(15) if j not in row]
        row[0] = dropped[0]
        row[:3] = np.sort(row[:3])
    elif plant == "drop_own":
        row[3] = -1
    elif plant == "unsorted":
        row[[0, 1]] = row[[1, 0]]
    else:
        row[2] = 15 + 1
    sel[r] = row
    with pytest.raises(AssertionError):
        parity.check_selection_all_rows(q, kbar, sel, B, topk)


def test_float32_every_row_reference_matches_the_oracle():
    """The float32 reference that checks every output row of the 128K and 1M
    GPU runs (tests/all_rows.py) against the oracle's forward on a small GQA
    case with a ragged last block; a selection with one past block swapped
    must move that row, so the reference attends the set it is given."""
    import torch
    from oracle import moba_oracle as O
    from tests.all_rows import reference_all_rows
    rng = np.random.default_rng(7)
    L, H, Hkv, D, B, topk = 300, 4, 2, 64, 64, 3
    q = rng.standard_normal((L, H, D))
    k = rng.standard_normal((L, Hkv, D))
    v = rng.standard_normal((L, Hkv, D))
    out, sel, _ = O.moba_reference(q, k, v, B, topk)
    t = lambda x: torch.tensor(x, dtype=torch.float32)
    ref = reference_all_rows(t(q), t(k), t(v), torch.tensor(sel, dtype=torch.int32), B)
    got = ref.permute(1, 0, 2).double().numpy()
    assert np.abs(got - out).max() < 1e-5
    # row 290 of head 1 (own block 4) keeps two of the past blocks 0..3;
    # give it the one it dropped instead of its first
    row = sel[1, 290].copy()
    dropped = [j for j in range(4) if j not in row][0]
    bad = sel.copy()
    bad[1, 290, 0] = dropped
    bad[1, 290] = np.sort(bad[1, 290])
    ref2 = reference_all_rows(t(q), t(k), t(v), torch.tensor(bad, dtype=torch.int32), B)
    assert np.abs(ref2[1, 290].double().numpy() - out[290, 1]).max() > 1e-3
    assert torch.equal(ref2[0], ref[0])


def test_float32_every_element_backward_reference_matches_the_oracle():
    """The float32 gradient reference of the 128K GPU backward run
    (tests/all_rows.py) against the oracle's backward on the same selection
    and forward output (GQA, ragged last block): dq, dk and dv within 1e-4 of
    the largest gradient."""
    import torch
    from oracle import moba_oracle as O
    from tests.all_rows import reference_backward_all
    rng = np.random.default_rng(11)
    L, H, Hkv, D, B, topk = 300, 4, 2, 64, 64, 3
    q = rng.standard_normal((L, H, D))
    k = rng.standard_normal((L, Hkv, D))
    v = rng.standard_normal((L, Hkv, D))
    dout = rng.standard_normal((L, H, D))
    out, sel, _ = O.moba_reference(q, k, v, B, topk)
    out = out + 1e-3 * rng.standard_normal(out.shape)  # a stored output, rounded
    ref = O.moba_backward_reference(q, k, v, dout, B, sel, out=out)
    t = lambda x: torch.tensor(x, dtype=torch.float32)
    got = reference_backward_all(t(q), t(k), t(v), t(out), t(dout),
                                 torch.tensor(sel, dtype=torch.int32), B)
    for g_, r_ in zip(got, ref):
        assert np.abs(g_.double().numpy() - r_).max() <= 1e-4 * np.abs(r_).max()
