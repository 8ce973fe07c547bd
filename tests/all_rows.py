"""Every output row of a large prefill against a second reference: plain
PyTorch float32 on the GPU, attention over each query's selected blocks.

The CPU oracle evaluates a few hundred (head, query) rows of the 128K and 1M
prefills; this reference evaluates all of them (4.2M and 33.6M query-heads)
from the same definition (MoBA project card, "How It Works": each query
attends to the keys of its selected blocks, its own block causally), and is
itself compared with the oracle on the sampled rows, so its agreement
extends the oracle's evidence to every row.  It uses the GPU's selection,
which the selection check has already validated on every row.

Per KV group g: the routed (query-head, past block) pairs are sorted by
block; for each block j the pairs' query rows are gathered and their scores
against K_j, the softmax statistics and P V_j are taken in float32 and merged
into running (max, sum, output) accumulators per query-head (a query selects
a block at most once, so no two pairs of one block write the same row).  The
own block follows for every query block, with the causal mask.  No part of
it shares code with the library.
"""

from __future__ import annotations

import math

import torch


def _routed_pairs(sel, g, G, own, nb):
    """Routed pairs of KV group g: (local head, row, block) of every kept past
    block, sorted by block, and each block's [start, end) in that order."""
    sg = sel[g * G:(g + 1) * G].long()                           # [G, L, topk]
    past = (sg >= 0) & (sg < own[None, :, None])
    hl, ii, tt = past.nonzero(as_tuple=True)
    jj = sg[hl, ii, tt]
    del sg, past, tt
    order = torch.argsort(jj, stable=True)
    hl, ii, jj = hl[order], ii[order], jj[order]
    bounds = torch.searchsorted(jj, torch.arange(nb + 1, device=jj.device)).tolist()
    return hl, ii, bounds


@torch.no_grad()
def reference_all_rows(q, k, v, sel, block_size, chunk=1 << 16, with_lse=False):
    """q [L, H, D], k and v [L, Hkv, D] (bf16 or fp32, one sequence, queries at
    positions 0..L-1), sel [H, L, topk] int32 (-1 padded, own block included).

    Returns the float32 output [H, L, D] (and, with_lse, the natural
    log-sum-exp [H, L] of each row's scaled logits)."""
    assert torch.get_float32_matmul_precision() == "highest"  # full float32 products
    L, H, D = q.shape
    Hkv = k.shape[1]
    G = H // Hkv
    B = block_size
    nb = (L + B - 1) // B
    dev = q.device
    scale = 1.0 / math.sqrt(D)
    m = torch.full((H, L), -math.inf, dtype=torch.float32, device=dev)
    s = torch.zeros((H, L), dtype=torch.float32, device=dev)
    o = torch.zeros((H, L, D), dtype=torch.float32, device=dev)

    def merge(hh, ii, sc, vv):
        # sc [n, keys] scaled scores (-inf where masked), vv [keys, D]
        cm = sc.max(dim=1).values
        p = torch.exp(sc - cm[:, None])
        cs = p.sum(dim=1)
        co = p @ vv
        mo = m[hh, ii]
        mn = torch.maximum(mo, cm)
        a = torch.exp(mo - mn)
        b = torch.exp(cm - mn)
        s[hh, ii] = s[hh, ii] * a + cs * b
        o[hh, ii] = o[hh, ii] * a[:, None] + co * b[:, None]
        m[hh, ii] = mn

    own = torch.arange(L, device=dev) // B
    for g in range(Hkv):
        hl, ii, bounds = _routed_pairs(sel, g, G, own, nb)
        for j in range(nb):
            lo, hi = bounds[j], bounds[j + 1]
            if lo == hi:
                continue
            kj = k[j * B:(j + 1) * B, g].float()
            vj = v[j * B:(j + 1) * B, g].float()
            for c0 in range(lo, hi, chunk):
                c1 = min(c0 + chunk, hi)
                hh = hl[c0:c1] + g * G
                ri = ii[c0:c1]
                qq = q[ri, hh].float()
                merge(hh, ri, (qq @ kj.T) * scale, vj)
        del hl, ii
        # own block: keys from the block start up to the query
        for b in range(nb):
            r0, r1 = b * B, min((b + 1) * B, L)
            kb = k[r0:r1, g].float()
            vb = v[r0:r1, g].float()
            pos = torch.arange(r0, r1, device=dev)
            mask = pos[None, :] > pos[:, None]                  # [rows, keys]
            for h in range(g * G, (g + 1) * G):
                sc = (q[r0:r1, h].float() @ kb.T) * scale
                sc = sc.masked_fill(mask, -math.inf)
                merge(torch.full((r1 - r0,), h, device=dev, dtype=torch.long), pos, sc, vb)
    if with_lse:
        return o / s[..., None], m + torch.log(s)
    return o / s[..., None]


@torch.no_grad()
def reference_backward_all(q, k, v, out, dout, sel, block_size, chunk=1 << 15):
    """Gradients of the selected-block attention for every element, float32:
    with P = exp(q.k/sqrt(D) - lse) over each row's key set (lse from
    reference_all_rows) and delta = dO . out (the forward output the backward
    is handed), dS = P (dO . v - delta), dq = dS K / sqrt(D),
    dk = dS^T Q / sqrt(D), dv = P^T dO, summed over every (query-head, key)
    pair of the selection.  Shapes as reference_all_rows; out and dout
    [L, H, D].  Returns dq [L, H, D], dk and dv [L, Hkv, D] (float32)."""
    L, H, D = q.shape
    Hkv = k.shape[1]
    G = H // Hkv
    B = block_size
    nb = (L + B - 1) // B
    dev = q.device
    scale = 1.0 / math.sqrt(D)
    _, lse = reference_all_rows(q, k, v, sel, block_size, with_lse=True)
    delta = (dout.float() * out.float()).sum(dim=2).T.contiguous()   # [H, L]
    dq = torch.zeros((H, L, D), dtype=torch.float32, device=dev)
    dk = torch.zeros((L, Hkv, D), dtype=torch.float32, device=dev)
    dv = torch.zeros((L, Hkv, D), dtype=torch.float32, device=dev)

    def pairs(hh, ii, qq, dd, kb, vb, mask=None):
        # one (rows, key tile) product: returns dK and dV of the tile's keys
        sc = (qq @ kb.T) * scale
        p = torch.exp(sc - lse[hh, ii][:, None])
        if mask is not None:
            p = p.masked_fill(mask, 0.0)
        ds = p * (dd @ vb.T - delta[hh, ii][:, None])
        dq.index_put_((hh, ii), (ds @ kb) * scale, accumulate=True)
        return (ds.T @ qq) * scale, p.T @ dd

    own = torch.arange(L, device=dev) // B
    for g in range(Hkv):
        hl, ii, bounds = _routed_pairs(sel, g, G, own, nb)
        for j in range(nb):
            lo, hi = bounds[j], bounds[j + 1]
            if lo == hi:
                continue
            kj = k[j * B:(j + 1) * B, g].float()
            vj = v[j * B:(j + 1) * B, g].float()
            for c0 in range(lo, hi, chunk):
                c1 = min(c0 + chunk, hi)
                hh = hl[c0:c1] + g * G
                ri = ii[c0:c1]
                dkj, dvj = pairs(hh, ri, q[ri, hh].float(), dout[ri, hh].float(), kj, vj)
                dk[j * B:(j + 1) * B, g] += dkj
                dv[j * B:(j + 1) * B, g] += dvj
        del hl, ii
        for b in range(nb):
            r0, r1 = b * B, min((b + 1) * B, L)
            kb = k[r0:r1, g].float()
            vb = v[r0:r1, g].float()
            pos = torch.arange(r0, r1, device=dev)
            mask = pos[None, :] > pos[:, None]
            for h in range(g * G, (g + 1) * G):
                hh = torch.full((r1 - r0,), h, device=dev, dtype=torch.long)
                dkb, dvb = pairs(hh, pos, q[r0:r1, h].float(), dout[r0:r1, h].float(), kb, vb,
                                 mask)
                dk[r0:r1, g] += dkb
                dv[r0:r1, g] += dvb
    return dq.transpose(0, 1), dk, dv


def compare_grad_rows(name, got, ref, relrms):
    """Per-row (last axis) relative RMS error of a gradient for rows whose
    reference is not negligible; the others (keys no query attends: exactly
    zero) must stay within 1e-2 of the largest row norm."""
    got = got.reshape(-1, got.shape[-1]).float()
    ref = ref.reshape(-1, ref.shape[-1])
    nrm = ref.pow(2).mean(dim=1).sqrt()
    err = (got - ref).pow(2).mean(dim=1).sqrt()
    big = nrm > 1e-3 * nrm.max()
    rel = err[big] / nrm[big]
    small = (got[~big] - ref[~big]).abs().max().item() if bool((~big).any()) else 0.0
    worst = rel.max().item()
    assert worst <= relrms, f"{name}: relative RMS error {worst:.3e} > {relrms:.3e}"
    assert small <= 1e-2 * nrm.max().item(), f"{name}: near-zero rows off by {small:.2e}"
    return worst, rel.median().item(), int(big.sum()), small


def compare_all_rows(out, ref, tol_max, tol_mean, relrms):
    """out [L, H, D] from the library, ref [H, L, D] float32: max and mean
    absolute error, and every row's relative RMS error."""
    worst_abs = 0.0
    total_abs = 0.0
    worst_rel = 0.0
    n = 0
    H = ref.shape[0]
    for h in range(H):
        d = out[:, h].float() - ref[h]
        ad = d.abs()
        worst_abs = max(worst_abs, float(ad.max()))
        total_abs += float(ad.sum(dtype=torch.float64))
        n += ad.numel()
        rr = d.pow(2).mean(dim=1).sqrt() / ref[h].pow(2).mean(dim=1).sqrt().clamp_min(1e-30)
        worst_rel = max(worst_rel, float(rr.max()))
    mean_abs = total_abs / n
    assert worst_abs <= tol_max, f"max abs error {worst_abs:.3e} > {tol_max}"
    assert mean_abs <= tol_mean, f"mean abs error {mean_abs:.3e} > {tol_mean}"
    assert worst_rel <= relrms, f"relative RMS error {worst_rel:.3e} > {relrms:.3e}"
    return worst_abs, mean_abs, worst_rel
