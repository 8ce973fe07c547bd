#!/usr/bin/env python3
"""Benchmark of the MoBA forward on one MI355X (gfx950).

One step = one moba_forward_ex call over one batch of resident synthetic
inputs: block means, gate + top-k, routing, routed attention and the own-block
attention with the merge.  The workspace is allocated once, outside the timed
region.  Prints one JSON line.

  value        effective TFLOP/s of the MoBA forward on the 32K single-head
               shape (block 2048, top-k 3): only selected-block FLOPs count,
               F = 4 D sum_{h,i} (B |past blocks kept| + keys of the own block
               up to i).
  speedup      time of the library's own full causal attention at the same
               shape / time of the MoBA forward.
  also         the backward (moba_backward_ex) at 32K, 128K and 1M in effective
               TFLOP/s (five products per selected pair, 2.5 x the forward's
               FLOPs) with the dk/dv kernel's roofline; the same figures as
               above at the 128K Llama-layer prefill and the
               1M-token prefill (32/8 heads, block 4096, top-k 12), at 10M
               tokens with one head (block 4096, top-k 12; the full attention
               it is compared with runs once, about half a minute), and the
               batch-8 decode against a 1M-token cache in GB/s of algorithmic
               bytes against the HBM peak.
  roofline     the dominant kernel (routed attention): its algorithmic FLOPs
               per launch / its average launch time from HIP events recorded
               on the launch stream, against the 2.5 PFLOP/s bf16 dense MFMA
               peak.
  cpu_baseline the float64 CPU oracle on a bounded sample of the same
               workload, in the same unit.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoBA fwd effective TFLOP/s & speedup vs full attn at 32K and 1M tokens (1 GPU)"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ------------------------------------------------------------ HBM traffic
def sources_sha256(paths):
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(record_name):
    """HBM bytes per launch of a kernel from a committed counter record
    (profiles/<record_name>.json: FETCH_SIZE and WRITE_SIZE in KiB per
    dispatch from two rocprofv3 --pmc runs, each scaled by the factor the same
    counter reads for a plain copy of known size).  None when there is no
    record or the kernel's sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", record_name + ".json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    try:
        if rec["sources_sha256"] != sources_sha256(rec["sources"]):
            return None
        return (rec["fetch_kib_per_dispatch"] * rec["fetch_scale"]
                + rec["write_kib_per_dispatch"] * rec["write_scale"]) * 1024.0
    except (KeyError, OSError):
        return None


# ----------------------------------------------------------- work accounting
def prefill_flops(w):
    """(effective, routed, own, full) FLOPs of a prefill workload.

    Per query i of a head: the routed part attends B keys for each of its
    min(k-1, b(i)) kept past blocks; the own part attends i - b(i) B + 1 keys;
    2 FLOPs per multiply-add in Q K^T and in P V: 4 D per (query, key)."""
    N, B, k, D, H, S = w.q_len, w.block_size, w.topk, w.head_dim, w.n_heads, w.batch
    q_off = w.kv_len - w.q_len
    routed_keys = 0
    own_keys = 0
    full_keys = 0
    # closed form per block of positions
    for b in range((q_off + N - 1) // B + 1):
        lo = max(b * B, q_off)
        hi = min((b + 1) * B, q_off + N)
        if hi <= lo:
            continue
        cnt = hi - lo
        routed_keys += cnt * B * min(k - 1, b)
        # sum over positions p in [lo, hi) of (p - bB + 1)
        own_keys += (lo - b * B + 1 + hi - b * B) * cnt // 2
        full_keys += (lo + 1 + hi) * cnt // 2
    f = 4 * D * H * S
    return f * (routed_keys + own_keys), f * routed_keys, f * own_keys, f * full_keys


# ---------------------------------------------------------------- timing
# Untimed settling for short steps: after the warmup steps, a step shorter
# than SETTLE_MAX_STEP_S is repeated (untimed) for SETTLE_S, so that the timed
# steps run at the clock a continuous stream of such steps sees rather than at
# the one the GPU ramps up from after idling (the 32K step: 0.140 ms after 5
# warmup steps, 0.127 ms after 200).
SETTLE_S = 0.1
SETTLE_MAX_STEP_S = 0.005
last_settle_steps = 0


def time_region(fn, steps, warmup):
    import torch
    global last_settle_steps
    one = float("inf")  # wall time of the last warmup step
    for i in range(warmup):
        if i == warmup - 1:
            torch.cuda.synchronize()
            t = time.perf_counter()
        fn()
        if i == warmup - 1:
            torch.cuda.synchronize()
            one = time.perf_counter() - t
    torch.cuda.synchronize()
    last_settle_steps = 0
    if one < SETTLE_MAX_STEP_S:
        last_settle_steps = int(SETTLE_S / max(one, 1e-5))
        for _ in range(last_settle_steps):
            fn()
        torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(st)
    for _ in range(steps):
        fn()
    e1.record(st)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    return e0.elapsed_time(e1) / steps, wall * 1e3


def time_cold(fn, steps, flush_mib=512):
    """Median time of fn with a flush_mib MiB buffer written before every call
    (evicts the working set from the 256 MB Infinity Cache); each call is
    bracketed by its own events, the write is outside them."""
    import torch
    buf = torch.empty(flush_mib << 20, dtype=torch.uint8, device="cuda:0")
    st = torch.cuda.current_stream()
    times = []
    for _ in range(steps):
        buf.fill_(1)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(st)
        fn()
        e1.record(st)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    del buf
    times.sort()
    return times[len(times) // 2]


def kernel_breakdown(moba, fn, steps):
    """Per-kernel average launch time (ms) from the library's HIP events."""
    import torch
    torch.cuda.synchronize()
    moba.moba_profile_reset()
    moba.moba_profile_enable(True)
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    moba.moba_profile_enable(False)
    out = {}
    for name in moba.KERNEL_NAMES:
        ms, n = moba.moba_profile_read(name)
        if n:
            # per_step: launches of the kernel per call (a long prefill routes
            # in passes of KV heads, one routed launch per pass)
            out[name] = {"avg_ms": ms / n, "launches": n, "per_step": n / steps}
    moba.moba_profile_reset()
    return out


# largest workspace of the timed mask-based form (its dense matrices)
NAIVE_MAX_BYTES = 16 << 30


def run_prefill(moba, w, steps, warmup, full_steps, full_warmup, with_full=True, cold=False):
    import torch
    import moba_inputs
    log(f"[bench] {w.name}: generating inputs")
    q, k, v = moba_inputs.make_inputs(w, device="cuda:0")
    out = torch.empty_like(q)
    ws_bytes = moba.moba_workspace_size(q, k, v, w.block_size, w.topk)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    fwd = lambda: moba.moba_forward_ex(q, k, v, w.block_size, w.topk, out=out, workspace=ws)
    log(f"[bench] {w.name}: workspace {ws_bytes / 2**30:.2f} GiB; timing MoBA forward")
    ms, wall_ms = time_region(fwd, steps, warmup)
    settle = last_settle_steps
    kern = kernel_breakdown(moba, fwd, steps)
    eff, routed, own, full = prefill_flops(w)
    cold_ms = time_cold(fwd, steps) if cold else None
    res = {
        "workload": w.name, "ms": ms, "wall_ms": wall_ms,
        "effective_tflops": eff / (ms * 1e-3) / 1e12,
        "frac_of_bf16_peak": eff / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "effective_flop": eff, "routed_flop": routed, "own_flop": own,
        "untimed_settle_steps": settle,
        "kernels_ms": {k_: round(v_["avg_ms"], 4) for k_, v_ in kern.items()},
    }
    if cold_ms is not None:
        # inputs evicted from the Infinity Cache before every call (median)
        res["cold_ms"] = cold_ms
        res["cold_effective_tflops"] = eff / (cold_ms * 1e-3) / 1e12
    if "attn_routed" in kern:
        t = kern["attn_routed"]["avg_ms"] * 1e-3
        res["attn_routed_tflops"] = routed / (t * kern["attn_routed"]["per_step"]) / 1e12
        res["attn_routed_launches_per_step"] = kern["attn_routed"]["per_step"]
    if "attn_own_merge" in kern:
        t = kern["attn_own_merge"]["avg_ms"] * 1e-3
        res["attn_own_merge_tflops"] = own / (t * kern["attn_own_merge"]["per_step"]) / 1e12
    if with_full:
        fout = torch.empty_like(q)
        fws = torch.empty(max(moba.moba_full_workspace_size(q, k, v), 1), dtype=torch.uint8,
                          device=q.device)
        ffn = lambda: moba.moba_full_attention_ex(q, k, v, out=fout, workspace=fws)
        log(f"[bench] {w.name}: timing full attention")
        fms, _ = time_region(ffn, full_steps, full_warmup)
        fk = kernel_breakdown(moba, ffn, 1)
        res["full_ms"] = fms
        res["full_tflops"] = full / (fms * 1e-3) / 1e12
        res["full_frac_of_bf16_peak"] = res["full_tflops"] / PEAK_BF16_TFLOPS
        res["speedup_vs_full"] = fms / ms
        res["full_kernels_ms"] = {k_: round(v_["avg_ms"], 4) for k_, v_ in fk.items()}
        del fout, fws
    nbytes = moba.moba_naive_workspace_size(q, k, v, w.block_size, w.topk) if with_full else 0
    if 0 < nbytes <= NAIVE_MAX_BYTES:
        # the mask-based form (dense scores, block mask, softmax, P V): the
        # baseline of the pages' efficient-vs-naive ratio at this shape
        nout = torch.empty_like(q)
        nws = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
        nfn = lambda: moba.moba_naive_ex(q, k, v, w.block_size, w.topk, out=nout, workspace=nws)
        log(f"[bench] {w.name}: timing the mask-based (naive) form")
        nms, _ = time_region(nfn, min(steps, 5), min(warmup, 2))
        nk = kernel_breakdown(moba, nfn, 1)
        res["naive_ms"] = nms
        res["speedup_vs_naive"] = nms / ms
        res["naive_kernels_ms"] = {k_: round(v_["avg_ms"], 4) for k_, v_ in nk.items()}
        del nout, nws
    res["_roofline_src"] = kern
    del q, k, v, out, ws
    torch.cuda.empty_cache()
    return res


def run_backward(moba, w, steps, warmup):
    """One step = one moba_backward_ex call (the forward's selection and
    log-sum-exp precomputed, workspace preallocated).  Algorithmic work: five
    products per (query, selected key) pair (S, dP, dV, dK, dQ) = 2.5 x the
    forward's selected-block FLOPs; the dk/dv kernel does four of them."""
    import torch
    import moba_inputs  # noqa: F401
    log(f"[bench] {w.name}: backward inputs")
    q, k, v = moba_inputs.make_inputs(w, device="cuda:0")
    out, sel, lse = moba.moba_forward_ex(q, k, v, w.block_size, w.topk, return_selection=True,
                                         return_lse=True)
    g = torch.Generator(device="cuda:0").manual_seed(w.seed + 7)
    dout = torch.randn(q.shape, generator=g, device="cuda:0",
                       dtype=torch.float32).to(q.dtype)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(max(moba.moba_backward_workspace_size(q, k, v, w.block_size, w.topk), 1),
                     dtype=torch.uint8, device=q.device)
    bwd = lambda: moba.moba_backward_ex(q, k, v, out, dout, lse, sel, w.block_size, w.topk,
                                        dq=dq, dk=dk, dv=dv, workspace=ws)
    log(f"[bench] {w.name}: workspace {ws.numel() / 2**30:.2f} GiB; timing MoBA backward")
    ms, wall_ms = time_region(bwd, steps, warmup)
    kern = kernel_breakdown(moba, bwd, steps)
    eff, _, _, _ = prefill_flops(w)
    res = {"workload": w.name + "_backward", "ms": ms, "wall_ms": wall_ms,
           "effective_tflops": 2.5 * eff / (ms * 1e-3) / 1e12,
           "frac_of_bf16_peak": 2.5 * eff / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
           "effective_flop": 2.5 * eff,
           "kernels_ms": {k_: round(v_["avg_ms"], 4) for k_, v_ in kern.items()}}
    if "bwd_dkdv" in kern:
        t = kern["bwd_dkdv"]["avg_ms"] * 1e-3
        a = 2.0 * eff / t / 1e12
        res["roofline"] = {"bound": "mfma", "kernel": "bwd_dkdv", "achieved": a,
                           "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                           "frac": a / PEAK_BF16_TFLOPS,
                           "traffic": measured_traffic(f"bwd_dkdv_{w.name}_backward_bytes"),
                           "avg_launch_ms": kern["bwd_dkdv"]["avg_ms"]}
    del q, k, v, out, sel, lse, dout, dq, dk, dv, ws
    torch.cuda.empty_cache()
    return res


def run_decode(moba, w, steps, warmup, with_full=True):
    """Decode against a long cache: one moba_forward_ex call with the block
    means precomputed (untimed, as a decode loop reuses them).  Algorithmic
    bytes = every kept K/V block read once per (sequence, KV head) -- the
    union over the group's heads -- plus the block means, q and out."""
    import numpy as np
    import torch
    import moba_inputs
    log(f"[bench] {w.name}: generating the cache")
    q, k, v = moba_inputs.make_inputs(w, device="cuda:0")
    kbar = moba.moba_block_mean(k, w.block_size)
    S, Lq, H, D = q.shape
    L, Hkv = k.shape[1], k.shape[2]
    nb = L // w.block_size
    out = torch.empty_like(q)
    sel = torch.empty((S, H, Lq, w.topk), dtype=torch.int32, device=q.device)
    ws = torch.empty(max(moba.moba_workspace_size(q, k, v, w.block_size, w.topk, kbar, sel), 1),
                     dtype=torch.uint8, device=q.device)
    fwd = lambda: moba.moba_forward_ex(q, k, v, w.block_size, w.topk, out=out,
                                       k_block_mean=kbar, sel_out=sel, workspace=ws)
    log(f"[bench] {w.name}: timing MoBA decode")
    ms, wall_ms = time_region(fwd, steps, warmup)
    kern = kernel_breakdown(moba, fwd, steps)
    selh = sel.cpu().numpy()
    G = H // Hkv
    union = 0
    for s_ in range(S):
        for g in range(Hkv):
            blocks = selh[s_, g * G:(g + 1) * G, 0, :].ravel()
            union += np.unique(blocks[blocks >= 0]).size
    esz = q.element_size()
    kv_bytes = union * w.block_size * D * esz * 2
    alg = kv_bytes + S * Hkv * nb * D * 4 + 2 * q.numel() * esz
    res = {"workload": w.name, "ms": ms, "wall_ms": wall_ms, "algorithmic_bytes": alg,
           "union_blocks_per_seq_kvhead": union / (S * Hkv),
           "gbs": alg / (ms * 1e-3) / 1e9, "frac_of_hbm_peak": alg / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
           "kernels_ms": {k_: round(v_["avg_ms"], 4) for k_, v_ in kern.items()}}
    if "decode_attn" in kern:
        t = kern["decode_attn"]["avg_ms"] * 1e-3
        res["roofline"] = {"bound": "hbm", "kernel": "decode_attn", "achieved": kv_bytes / t / 1e9,
                           "peak": PEAK_HBM_GBS, "unit": "GB/s",
                           "frac": kv_bytes / t / 1e9 / PEAK_HBM_GBS,
                           "traffic": measured_traffic(f"decode_attn_{w.name}_bytes"),
                           "avg_launch_ms": kern["decode_attn"]["avg_ms"]}
    if with_full:
        fout = torch.empty_like(q)
        fws = torch.empty(max(moba.moba_full_workspace_size(q, k, v), 1), dtype=torch.uint8,
                          device=q.device)
        ffn = lambda: moba.moba_full_attention_ex(q, k, v, out=fout, workspace=fws)
        log(f"[bench] {w.name}: timing full-attention decode")
        fms, _ = time_region(ffn, max(1, steps // 2), max(1, warmup // 2))
        full_bytes = S * L * Hkv * D * esz * 2 + 2 * q.numel() * esz
        res["full_ms"] = fms
        res["full_gbs"] = full_bytes / (fms * 1e-3) / 1e9
        res["full_frac_of_hbm_peak"] = res["full_gbs"] / PEAK_HBM_GBS
        res["speedup_vs_full"] = fms / ms
        del fout, fws
    if with_full:
        # A batch whose sequences hold different numbers of tokens in the same
        # padded cache: one call with per-sequence cache lengths (kv_lens)
        # against one call per sequence on its own rows (same block means).
        gen = torch.Generator().manual_seed(w.seed + 1)
        lens = torch.randint(L // 4, L + 1, (S,), generator=gen, dtype=torch.int32)
        kv = lens.to(q.device)
        kws = torch.empty(max(moba.moba_workspace_size(q, k, v, w.block_size, w.topk, kbar, sel),
                              1), dtype=torch.uint8, device=q.device)
        kfn = lambda: moba.moba_forward_ex(q, k, v, w.block_size, w.topk, out=out,
                                           k_block_mean=kbar, sel_out=sel, workspace=kws,
                                           kv_lens=kv)
        per = []
        for s_ in range(S):
            Ls = int(lens[s_])
            nbs = -(-Ls // w.block_size)
            per.append((q[s_:s_ + 1], k[s_:s_ + 1, :Ls], v[s_:s_ + 1, :Ls],
                        kbar[s_:s_ + 1, :, :nbs].contiguous(), out[s_:s_ + 1]))
        # one workspace for every per-sequence call (they run in stream order)
        pws = torch.empty(max(max(moba.moba_workspace_size(a, b, c, w.block_size, w.topk, kb)
                                  for a, b, c, kb, _ in per), 1),
                          dtype=torch.uint8, device=q.device)
        pfn = lambda: [moba.moba_forward_ex(a, b, c, w.block_size, w.topk, out=o,
                                            k_block_mean=kb, workspace=pws)
                       for a, b, c, kb, o in per]
        log(f"[bench] {w.name}: timing per-sequence cache lengths (one call vs one per sequence)")
        kms, _ = time_region(kfn, steps, warmup)
        pms, _ = time_region(pfn, steps, warmup)
        res["kv_lens"] = {"lengths": [int(x) for x in lens], "one_call_ms": kms,
                          "per_sequence_calls_ms": pms, "speedup": pms / kms}
        del kws, per, pws
    del q, k, v, out, ws, kbar
    torch.cuda.empty_cache()
    return res


def roofline(res):
    kern = res["_roofline_src"]
    if "attn_routed" not in kern:
        return None
    t = kern["attn_routed"]["avg_ms"] * 1e-3
    # algorithmic FLOPs of one launch: 4 D B per routed entry, the entries of
    # one pass (all of them when the call routes in one pass)
    achieved = res["routed_flop"] / kern["attn_routed"]["per_step"] / t / 1e12
    return {"bound": "mfma", "kernel": "attn_routed", "achieved": achieved,
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
            "traffic": measured_traffic(f"attn_routed_{res['workload']}_bytes"),
            "avg_launch_ms": kern["attn_routed"]["avg_ms"]}


# ------------------------------------------------------------ CPU baseline
def cpu_baseline(w, budget_s):
    """The float64 oracle on a bounded sample of the workload: the gate and
    top-k for every query (one matmul + stable argsort per head) and the
    attention of uniformly drawn queries until ~budget_s of CPU time."""
    import numpy as np
    import torch
    import moba_inputs
    from oracle import moba_oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    q, k, v = moba_inputs.make_inputs(w, device="cuda:0")
    qh, kh, vh = (t.float().cpu().numpy().astype(np.float64) for t in (q, k, v))
    del q, k, v
    torch.cuda.empty_cache()
    N, D, B = qh.shape[0], qh.shape[2], w.block_size
    rng = np.random.default_rng(0)
    t0 = time.perf_counter()
    kbar = O.block_mean(kh, B)
    sel, _ = O.select_all(qh, kbar, B, w.topk)
    t_sel = time.perf_counter() - t0
    flop = 0
    nq = 0
    t1 = time.perf_counter()
    scale = 1.0 / math.sqrt(D)
    while time.perf_counter() - t1 < budget_s:
        r = int(rng.integers(0, N))
        h = int(rng.integers(0, qh.shape[1]))
        g = h // (qh.shape[1] // kh.shape[1])
        keys = O.key_set(sel[h, r], r, B, N)
        O.attend(qh[r, h], kh[:, g, :], vh[:, g, :], keys, scale)
        flop += 4 * D * keys.size
        nq += 1
    t_att = time.perf_counter() - t1
    # selection time attributed to the sampled queries pro rata
    t_total = t_att + t_sel * nq / (N * qh.shape[1])
    return {"value": flop / t_total / 1e12, "unit": "TFLOP/s", "cores": blas_threads,
            "kind": "oracle",
            "sample": (f"{nq} uniformly drawn (head, query) rows of {w.name} in {t_att:.1f} s "
                       f"(float64 NumPy attention over each row's selected keys) plus their "
                       f"share of the full-workload gate/top-k pass ({t_sel:.1f} s for all "
                       f"{N * qh.shape[1]} rows)"),
            "host_cpus": os.cpu_count(),
            "affinity_cpus": len(os.sched_getaffinity(0))}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--skip-1m", action="store_true", help="skip the 1M-token prefill")
    ap.add_argument("--skip-128k", action="store_true", help="skip the 128K Llama-layer prefill")
    ap.add_argument("--skip-decode", action="store_true", help="skip the 1M-cache decode")
    ap.add_argument("--skip-10m", action="store_true",
                    help="skip the 10M-token single-head prefill")
    ap.add_argument("--skip-backward", action="store_true",
                    help="skip the backward (32K, 128K and 1M)")
    ap.add_argument("--skip-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--workload", default=None,
                    help="time only this prefill workload's MoBA forward (profiling runs)")
    ap.add_argument("--no-full", action="store_true", help="with --workload: skip full attention")
    ap.add_argument("--backward", action="store_true",
                    help="with --workload: time the backward of that prefill workload")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="with --workload: also run a plain device copy of this many MiB "
                         "(reference for the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the library runs on one MI355X; multi-GPU execution is not implemented)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import block_sparse_attention_gate_amd as moba
    import moba_inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.workload:
        if args.calib_copy_mib:
            n = args.calib_copy_mib << 20
            src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
            dst = torch.empty_like(src)
            for _ in range(2):
                dst.copy_(src)
            torch.cuda.synchronize()
            log(f"[bench] calibration copy of {args.calib_copy_mib} MiB done")
            del src, dst
        w = moba_inputs.WORKLOADS[args.workload]
        if args.backward:
            r = run_backward(moba, w, args.steps, args.warmup)
        elif w.is_decode:
            r = run_decode(moba, w, args.steps, args.warmup, with_full=not args.no_full)
        else:
            r = run_prefill(moba, w, args.steps, args.warmup, full_steps=1, full_warmup=0,
                            with_full=not args.no_full)
            r["roofline"] = roofline(r)
            r.pop("_roofline_src")
        print(json.dumps({"workload": w.name, "steps": args.steps, "warmup": args.warmup,
                          "detail": r}), flush=True)
        return
    w = moba_inputs.WORKLOADS["micro_32k"]
    main_res = run_prefill(moba, w, args.steps, args.warmup, full_steps=args.steps,
                           full_warmup=args.warmup, cold=True)
    also = {}
    if not args.skip_128k:
        w3 = moba_inputs.WORKLOADS["llama8b_128k"]
        r3 = run_prefill(moba, w3, min(args.steps, 10), min(args.warmup, 2), full_steps=3,
                         full_warmup=1)
        r3["roofline"] = roofline(r3)
        r3.pop("_roofline_src")
        also["llama8b_128k"] = r3
    if not args.skip_1m:
        w1 = moba_inputs.WORKLOADS["prefill_1m"]
        r1 = run_prefill(moba, w1, min(args.steps, 3), min(args.warmup, 1), full_steps=1,
                         full_warmup=0)
        r1["roofline"] = roofline(r1)
        r1.pop("_roofline_src")
        also["prefill_1m"] = r1
    if not args.skip_10m:
        w10 = moba_inputs.WORKLOADS["prefill_10m"]
        r10 = run_prefill(moba, w10, min(args.steps, 3), min(args.warmup, 1), full_steps=1,
                          full_warmup=0)
        r10["roofline"] = roofline(r10)
        r10.pop("_roofline_src")
        also["prefill_10m"] = r10
    if not args.skip_backward:
        also["micro_32k_backward"] = run_backward(moba, w, args.steps, args.warmup)
        if not args.skip_128k:
            also["llama8b_128k_backward"] = run_backward(
                moba, moba_inputs.WORKLOADS["llama8b_128k"], min(args.steps, 3),
                min(args.warmup, 1))
        if not args.skip_1m:
            also["prefill_1m_backward"] = run_backward(
                moba, moba_inputs.WORKLOADS["prefill_1m"], 1, 1)
    if not args.skip_decode:
        also["decode_1m"] = run_decode(moba, moba_inputs.WORKLOADS["decode_1m"], args.steps,
                                       args.warmup)
    rl = roofline(main_res)
    main_res.pop("_roofline_src")
    cpu = None if args.skip_cpu else cpu_baseline(w, args.cpu_budget)
    line = {
        "metric": METRIC,
        "value": main_res["effective_tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "seq_len": w.q_len,
                   "n_heads": w.n_heads, "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim,
                   "block_size": w.block_size, "topk": w.topk, "parallelism": "single GPU"},
        "speedup_vs_full": main_res.get("speedup_vs_full"),
        "speedup_vs_naive": main_res.get("speedup_vs_naive"),
        "detail": main_res,
        "roofline": rl,
        "cpu_baseline": cpu,
        "also": also,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
