"""Plain float64 CPU oracle for the MoBA (Mixture of Block Attention) forward.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` and by nothing else.  It shares no
code with the HIP library.  It is deliberately slow and written so that each
step can be checked against the pages by eye.

Sources (cited by page title and section):

* [MoBA card] "MoBA" project card (sourcepulse), sections "How It Works" and
  "Highlighted Details": the context is divided into blocks; a parameter-less
  top-k gate picks, for each query token, the most relevant KV blocks; the
  two knobs are "MoBA Block" (block size) and "MoBA Topk".
* [Dev Tutorial] "Dev Tutorial: Implementing Sparse Attention (MoBA) and
  Scalable Search Agents", Step-by-Step Guide step 1: divide the context into
  blocks, gate per query token, then mask; a naive (mask) version exists for
  analysing masks next to the optimised one.
* [AiBoss] "MoBA - Moonshot AIが提案した新しいアテンションメカニズム",
  section "MoBAの技術的原則" (causality design): a query never attends to a
  future block, and a causal mask is applied inside the current block.
  Section "MoBAの主な機能": seamless switching between full and sparse
  attention.

Readings where the pages are silent (each is listed in the design notes):

* R1 gate affinity: the score of block j for query q is ``q . mean(K_j)``,
  unscaled, no bias (a parameter-less gate).
* R2 the query's own block always counts as one of the top-k blocks; the
  remaining ``k-1`` are the best past blocks.
* R3 future blocks are never selected, so ``|Sel| = min(k, b+1)``.
* R4 ties in the gate score go to the lowest block index.
* R6 the gate only selects: the output is ONE softmax over the union of the
  selected keys (no gate weighting).
* R7 softmax scale ``1/sqrt(D)``, applied to attention only, never the gate.
* R8 GQA: query head h reads KV head ``h // (H/Hkv)``; every query head gates
  on its own.
* R9 the causal diagonal is inclusive (key t is visible to query i if t <= i).
* R10 queries are bottom-right aligned: query row r sits at position
  ``kv_len - q_len + r``.
* R11 a partial last block is averaged over the keys it holds.
* R15 training (the [MoBA card] "Highlighted Details" and the [Dev Tutorial]
  step 1 note: MoBA needs continued training; the pages give no backward
  pass): the top-k selection is piecewise constant and passes no gradient, so
  the gate and the block means receive none; the gradients are those of the
  softmax attention of every query over its fixed key set.

Layouts (one sequence): q ``[Lq, H, D]``, k and v ``[L, Hkv, D]``, all float64.
"""

from __future__ import annotations

import itertools
import math

import numpy as np

NEG_INF = -np.inf


# --------------------------------------------------------------------------
# Step 1: block partition and block-mean keys  ([MoBA card] "How It Works";
# [Dev Tutorial] step 1 "divide context into blocks"; reading R1, R11)
# --------------------------------------------------------------------------
def n_blocks(kv_len: int, block_size: int) -> int:
    return -(-kv_len // block_size)


def block_mean(k: np.ndarray, block_size: int) -> np.ndarray:
    """Mean key of every block: ``kbar[g, j] = mean_{t in block j} k[t, g]``.

    ``k`` is ``[L, Hkv, D]``; returns ``[Hkv, nb, D]`` float64.  A partial last
    block is averaged over the keys it actually holds (R11).
    """
    k = np.asarray(k, dtype=np.float64)
    L, hkv, d = k.shape
    nb = n_blocks(L, block_size)
    out = np.empty((hkv, nb, d), dtype=np.float64)
    for j in range(nb):
        lo, hi = j * block_size, min((j + 1) * block_size, L)
        out[:, j, :] = k[lo:hi].sum(axis=0) / (hi - lo)
    return out


# --------------------------------------------------------------------------
# Step 2: the parameter-less gate ([MoBA card] "How It Works": top-k gating
# for each query token; reading R1)
# --------------------------------------------------------------------------
def gate_scores(q_vec: np.ndarray, kbar_g: np.ndarray, own_block: int) -> np.ndarray:
    """Scores of the PAST blocks ``j < own_block``: ``s_j = q . kbar_j``."""
    return kbar_g[:own_block] @ np.asarray(q_vec, dtype=np.float64)


# --------------------------------------------------------------------------
# Step 3: top-k with the causal block rule ([AiBoss] causality design;
# readings R2, R3, R4)
# --------------------------------------------------------------------------
def select_blocks(scores_past: np.ndarray, own_block: int, topk: int):
    """Selected blocks of one query and the gate gap at the top-k boundary.

    The past blocks are ranked by (score descending, index ascending); the
    first ``min(topk-1, own_block)`` are kept and the own block is added.
    Returns ``(sel, gap)`` where ``sel`` is a tuple of length ``topk``,
    ascending, padded with -1, and ``gap`` is the difference between the last
    kept and the first dropped past score (``inf`` when nothing is dropped).
    """
    b = own_block
    n_keep = min(topk - 1, b)
    order = sorted(range(b), key=lambda j: (-float(scores_past[j]), j))
    kept = order[:n_keep]
    sel = sorted(kept + [b])
    sel = tuple(sel + [-1] * (topk - len(sel)))
    if n_keep >= 1 and b > n_keep:
        gap = float(scores_past[order[n_keep - 1]] - scores_past[order[n_keep]])
    else:
        gap = math.inf
    return sel, gap


def brute_force_select(scores_past: np.ndarray, own_block: int, topk: int):
    """Independent form of the selection for tiny inputs.

    Enumerates every subset of past blocks of size ``min(topk-1, b)``; a subset
    is a valid top set when its smallest score is >= the largest score left
    out.  Among valid subsets the lexicographically smallest sorted tuple is
    the lowest-index tie-break.  Returns ``sel`` like ``select_blocks``.
    """
    b = own_block
    n_keep = min(topk - 1, b)
    best = None
    for subset in itertools.combinations(range(b), n_keep):
        inside = [scores_past[j] for j in subset]
        outside = [scores_past[j] for j in range(b) if j not in subset]
        if inside and outside and min(inside) < max(outside):
            continue
        if best is None or subset < best:
            best = subset
    sel = sorted(list(best) + [b])
    return tuple(sel + [-1] * (topk - len(sel)))


def select_all(q, kbar, block_size, topk, q_offset=0, rows=None, positions=None):
    """Selection for many queries at once (same rule as ``select_blocks``).

    ``q`` is ``[Lq, H, D]``, ``kbar`` ``[Hkv, nb, D]``.  Uses a matmul for the
    scores and a stable argsort of the negated scores for the ranking (stable
    keeps the lower index first among equal scores, R4).  ``rows`` restricts
    the work to a subset of query rows; ``q_offset`` is the position of query
    row 0 (``kv_len - q_len``, R10).  ``positions`` instead gives the position
    of every row of ``q`` explicitly (for a sample of rows).  Returns ``sel [H, R, topk]`` (int64)
    and ``gap [H, R]``.
    """
    q = np.asarray(q, dtype=np.float64)
    lq, h_n, _ = q.shape
    hkv, nb, _ = kbar.shape
    group = h_n // hkv
    rows = np.arange(lq) if rows is None else np.asarray(rows)
    pos = q_offset + rows if positions is None else np.asarray(positions)[rows]
    own = pos // block_size
    n_keep = np.minimum(topk - 1, own)
    sel = np.full((h_n, rows.size, topk), -1, dtype=np.int64)
    gap = np.full((h_n, rows.size), np.inf)
    cols = np.arange(nb)
    kp = topk - 1
    big = np.iinfo(np.int64).max
    keep_mask = np.arange(kp)[None, :] < n_keep[:, None]           # [R, kp]
    has_gap = (n_keep >= 1) & (own > n_keep)
    for h in range(h_n):
        s = q[rows, h, :] @ kbar[h // group].T                # [R, nb]
        s = np.where(cols[None, :] < own[:, None], s, NEG_INF)  # past blocks only
        order = np.argsort(-s, axis=1, kind="stable")
        ranked = np.take_along_axis(s, order, axis=1)
        top = np.full((rows.size, kp), big, dtype=np.int64)
        w = min(kp, nb)
        top[:, :w] = order[:, :w]
        chosen = np.concatenate([np.where(keep_mask, top, big), own[:, None]], axis=1)
        chosen.sort(axis=1)
        sel[h] = np.where(chosen == big, -1, chosen)
        if kp >= 1:
            last = np.clip(n_keep - 1, 0, nb - 1)
            first_out = np.clip(n_keep, 0, nb - 1)
            with np.errstate(invalid="ignore"):   # -inf - -inf where no gap exists
                g = (np.take_along_axis(ranked, last[:, None], axis=1)[:, 0]
                     - np.take_along_axis(ranked, first_out[:, None], axis=1)[:, 0])
            gap[h] = np.where(has_gap, g, np.inf)
    return sel, gap


# --------------------------------------------------------------------------
# Step 4: softmax attention over the selected keys ([MoBA card] "How It
# Works"; [AiBoss] causal mask inside the own block; readings R6, R7, R9)
# --------------------------------------------------------------------------
def key_set(sel_row, position: int, block_size: int, kv_len: int) -> np.ndarray:
    """Keys a query attends: the selected past blocks whole, plus its own
    block up to and including its own position."""
    own = position // block_size
    keys = []
    for j in sel_row:
        if j < 0:
            continue
        if j < own:
            keys.extend(range(j * block_size, min((j + 1) * block_size, kv_len)))
        elif j == own:
            keys.extend(range(own * block_size, position + 1))
        else:  # a future block can never be attended
            raise AssertionError("future block in selection")
    return np.asarray(keys, dtype=np.int64)


def attend(q_vec, k_g, v_g, keys, scale):
    """``softmax(scale * K[keys] q) @ V[keys]`` for one query, in float64."""
    z = (k_g[keys] @ q_vec) * scale
    w = np.exp(z - z.max())
    return (w @ v_g[keys]) / w.sum()


def moba_reference(q, k, v, block_size, topk, q_offset=None, scale=None,
                   pairs=None, sel=None):
    """MoBA forward for one sequence, gather form.

    Returns ``(out [Lq, H, D], sel [H, Lq, topk], gap [H, Lq])``.  ``pairs``
    (an iterable of ``(h, r)``) restricts which outputs are computed; the
    others stay NaN.  ``sel`` may be given to evaluate the attention on a
    given selection (used for queries inside the gate's tie window).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    lq, h_n, d = q.shape
    L, hkv, _ = k.shape
    group = h_n // hkv
    if q_offset is None:
        q_offset = L - lq
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    kbar = block_mean(k, block_size)
    gap = None
    if sel is None:
        sel, gap = select_all(q, kbar, block_size, topk, q_offset=q_offset)
    out = np.full((lq, h_n, v.shape[2]), np.nan)
    if pairs is None:
        pairs = [(h, r) for h in range(h_n) for r in range(lq)]
    for h, r in pairs:
        g = h // group
        keys = key_set(sel[h, r], q_offset + r, block_size, L)
        out[r, h] = attend(q[r, h], k[:, g, :], v[:, g, :], keys, scale)
    return out, sel, gap


def attend_lse(q_vec, k_g, keys, scale):
    """Natural log of the softmax normaliser ``log sum_t exp(scale * k_t . q)``
    over ``keys`` (the max is taken out first)."""
    z = (k_g[keys] @ q_vec) * scale
    m = z.max()
    return m + np.log(np.exp(z - m).sum())


def moba_lse_reference(q, k, block_size, sel, q_offset=None, scale=None):
    """Log-sum-exp ``[H, Lq]`` of every query's logits over its key set (the
    statistic a forward keeps for the backward)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    lq, h_n, d = q.shape
    L, hkv, _ = k.shape
    group = h_n // hkv
    if q_offset is None:
        q_offset = L - lq
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    lse = np.empty((h_n, lq))
    for h in range(h_n):
        for r in range(lq):
            keys = key_set(sel[h, r], q_offset + r, block_size, L)
            lse[h, r] = attend_lse(q[r, h], k[:, h // group, :], keys, scale)
    return lse


# --------------------------------------------------------------------------
# Step 5 (training, reading R15): gradients of the attention over the fixed
# key sets.  Loss = sum(out * dout); for one query with key set T,
#   z_t = c k_t.q, p = softmax(z), o = sum_t p_t v_t,
#   dv_t += p_t dO,  dp_t = dO . v_t,  ds_t = p_t (dp_t - dO . o),
#   dq = c sum_t ds_t k_t,  dk_t += c ds_t q.
# --------------------------------------------------------------------------
def moba_backward_reference(q, k, v, dout, block_size, sel, q_offset=None, scale=None,
                            out=None, pairs=None):
    """Returns ``(dq [Lq, H, D], dk [L, Hkv, D], dv [L, Hkv, D])`` for the
    selection ``sel [H, Lq, topk]`` (held fixed).  GQA: a KV head's gradients
    sum over the query heads of its group (R8).

    ``out`` (optional, ``[Lq, H, D]``): a stored forward output that the term
    ``dO . o`` is to read instead of the exact output, as an algorithm that is
    handed the forward's (rounded) output computes it; None: exact.
    ``pairs`` (optional iterable of ``(h, r)``): only these query rows are
    processed (their dq rows; dk and dv then hold only their contributions)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    lq, h_n, d = q.shape
    L, hkv, _ = k.shape
    group = h_n // hkv
    if q_offset is None:
        q_offset = L - lq
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    if pairs is None:
        pairs = [(h, r) for h in range(h_n) for r in range(lq)]
    for h, r in pairs:
        g = h // group
        keys = key_set(sel[h, r], q_offset + r, block_size, L)
        kk, vv = k[keys, g, :], v[keys, g, :]
        z = (kk @ q[r, h]) * scale
        p = np.exp(z - z.max())
        p /= p.sum()
        o = p @ vv if out is None else np.asarray(out[r, h], dtype=np.float64)
        do = dout[r, h]
        dp = vv @ do
        ds = p * (dp - do @ o)
        dq[r, h] = scale * (ds @ kk)
        dk[keys, g, :] += scale * np.outer(ds, q[r, h])
        dv[keys, g, :] += np.outer(p, do)
    return dq, dk, dv


def full_reference(q, k, v, q_offset=None, scale=None, pairs=None):
    """Full causal attention (every key ``t <= position``), GQA as R8."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    lq, h_n, d = q.shape
    L, hkv, _ = k.shape
    group = h_n // hkv
    if q_offset is None:
        q_offset = L - lq
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.full((lq, h_n, v.shape[2]), np.nan)
    if pairs is None:
        pairs = [(h, r) for h in range(h_n) for r in range(lq)]
    for h, r in pairs:
        g = h // group
        keys = np.arange(q_offset + r + 1)
        out[r, h] = attend(q[r, h], k[:, g, :], v[:, g, :], keys, scale)
    return out


def naive_mask_reference(q, k, v, block_size, topk, q_offset=None, scale=None):
    """Second, independent form for small inputs: the mask formulation.

    ([Dev Tutorial] step 1 and [MoBA card] "Limitations & Caveats": the naive
    version builds the mask for analysis.)  For every query an ``[Lq, L]``
    boolean mask is built from the selection, masked logits are set to -inf,
    and a dense row softmax is applied.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    lq, h_n, d = q.shape
    L, hkv, _ = k.shape
    group = h_n // hkv
    if q_offset is None:
        q_offset = L - lq
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    kbar = block_mean(k, block_size)
    out = np.empty((lq, h_n, v.shape[2]))
    t = np.arange(L)
    blk = t // block_size
    for h in range(h_n):
        g = h // group
        mask = np.zeros((lq, L), dtype=bool)
        for r in range(lq):
            pos = q_offset + r
            own = pos // block_size
            sel, _ = select_blocks(gate_scores(q[r, h], kbar[g], own), own, topk)
            chosen = np.isin(blk, [j for j in sel if j >= 0])
            mask[r] = chosen & (t <= pos)
        logits = (q[:, h, :] @ k[:, g, :].T) * scale
        logits = np.where(mask, logits, NEG_INF)
        w = np.exp(logits - logits.max(axis=1, keepdims=True))
        w /= w.sum(axis=1, keepdims=True)
        out[:, h, :] = w @ v[:, g, :]
    return out


# --------------------------------------------------------------------------
# Dispatch view ([MoBA card] "How It Works": MoE principles, blocks act as
# experts; [AiBoss] "MoBAの主な機能": MoE-style optimisation)
# --------------------------------------------------------------------------
def routing_table(sel, n_kv_heads, n_blocks_, block_size, q_offset):
    """Regroup (query, selected PAST block) pairs by (KV head, block).

    ``sel`` is ``[batch, H, Lq, topk]`` (or ``[H, Lq, topk]`` for one
    sequence).  A routed entry is the pair (query row r of head h in sequence
    s, the s-th past block of its selection); its slot id is
    ``((s*H + h)*Lq + r)*(topk-1) + slot``.  Entries are bucketed by
    ``(s, h // G, block)`` in that order and listed by ascending slot id inside
    each bucket.  Returns ``(counts [batch*Hkv*nb], offsets [.. + 1],
    entries [E])`` as int64.
    """
    sel = np.asarray(sel)
    if sel.ndim == 3:
        sel = sel[None]
    batch, h_n, lq, topk = sel.shape
    group = h_n // n_kv_heads
    nb = n_blocks_
    if topk <= 1:
        counts = np.zeros(batch * n_kv_heads * nb, dtype=np.int64)
        return counts, np.zeros(counts.size + 1, dtype=np.int64), np.zeros(0, np.int64)
    kp = topk - 1
    own = (q_offset + np.arange(lq)) // block_size                 # [Lq]
    n_keep = np.minimum(kp, own)                                    # [Lq]
    past = sel[..., :kp]                                            # [S,H,Lq,kp]
    slot_of = np.arange(kp)
    valid = np.broadcast_to(slot_of[None, None, None, :] < n_keep[None, None, :, None],
                            past.shape)
    slot_ids = np.arange(batch * h_n * lq * kp, dtype=np.int64).reshape(past.shape)
    s_idx = np.arange(batch)[:, None, None, None]
    g_idx = (np.arange(h_n) // group)[None, :, None, None]
    bucket = (s_idx * n_kv_heads + g_idx) * nb + past
    bucket = np.broadcast_to(bucket, past.shape)[valid]
    slots = slot_ids[valid]                                          # ascending
    order = np.argsort(bucket, kind="stable")
    entries = slots[order]
    counts = np.bincount(bucket, minlength=batch * n_kv_heads * nb).astype(np.int64)
    offsets = np.zeros(counts.size + 1, dtype=np.int64)
    np.cumsum(counts, out=offsets[1:])
    return counts, offsets, entries


def moba_decode_reference(q, k, v, block_size, topk, scale=None):
    """Batched form: ``q [S, Lq, H, D]``, ``k, v [S, L, Hkv, D]``.

    Each sequence is handled as ``moba_reference`` with its queries at the end
    of its cache (R10).  Returns ``(out [S, Lq, H, D], sel [S, H, Lq, topk],
    gap [S, H, Lq])``.
    """
    outs, sels, gaps = [], [], []
    for s in range(q.shape[0]):
        o, sl, gp = moba_reference(q[s], k[s], v[s], block_size, topk, scale=scale)
        outs.append(o)
        sels.append(sl)
        gaps.append(gp)
    return np.stack(outs), np.stack(sels), np.stack(gaps)
