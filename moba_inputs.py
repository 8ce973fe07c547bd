"""Seeded synthetic inputs for the MoBA forward (data only).

This module holds none of the method's arithmetic.  It is the one piece that
both sides see: the HIP library's tests and benchmark feed its tensors to the
GPU, and the same bytes, copied to the host, to the CPU oracle.

Recipe (every workload):

* Q, V ~ N(0, 1).
* K[t, g, :] = z + o[g, t // B, :] with z ~ N(0, 1) and one offset vector
  o ~ N(0, 0.5^2) per (sequence, KV head, block), so the block means separate
  and the gate has something to choose between.
* Values are drawn in float32 with ``torch.Generator(device).manual_seed``
  and rounded to bfloat16 with round-to-nearest-even (float32 workloads stay
  float32).  Draw order: offsets, then Q, K noise, V, each in row chunks.

The named workloads mirror the five measured shapes: a tiny float32 case, the
32K single-head microbenchmark shape (block 2048, top-k 3), a Llama-3.1-8B
layer shape at 128K, the 1M-token prefill and a batch-8 decode against a
1M-token cache.
"""

from __future__ import annotations

import dataclasses

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str          # "f32" or "bf16"
    batch: int
    q_len: int
    kv_len: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    block_size: int
    topk: int
    seed: int

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def n_blocks(self):
        return -(-self.kv_len // self.block_size)

    @property
    def is_decode(self):
        return self.q_len < self.kv_len


WORKLOADS = {
    "tiny_f32_1k": Workload("tiny_f32_1k", "f32", 1, 1024, 1024, 1, 1, 64, 128, 3, 1001),
    "micro_32k": Workload("micro_32k", "bf16", 1, 32768, 32768, 1, 1, 128, 2048, 3, 1002),
    "llama8b_128k": Workload("llama8b_128k", "bf16", 1, 131072, 131072, 32, 8, 128, 4096, 12, 1003),
    "prefill_1m": Workload("prefill_1m", "bf16", 1, 1048576, 1048576, 32, 8, 128, 4096, 12, 1004),
    "decode_1m": Workload("decode_1m", "bf16", 8, 1, 1048576, 32, 8, 128, 4096, 12, 1005),
    # the 10M-token regime, one head (full attention at 32 heads would take minutes)
    "prefill_10m": Workload("prefill_10m", "bf16", 1, 10485760, 10485760, 1, 1, 128, 4096, 12,
                            1006),
}


def custom(name="custom", dtype="bf16", batch=1, q_len=256, kv_len=None, n_heads=1,
           n_kv_heads=1, head_dim=128, block_size=64, topk=3, seed=7) -> Workload:
    return Workload(name, dtype, batch, q_len, q_len if kv_len is None else kv_len,
                    n_heads, n_kv_heads, head_dim, block_size, topk, seed)


_CHUNK_ELEMS = 1 << 27  # float32 staging per draw: 512 MiB


def _normal_into(dst: torch.Tensor, gen: torch.Generator, scale: float = 1.0,
                 add=None):
    """Fill ``dst`` (any dtype, contiguous, leading dim = rows) chunk by chunk
    with N(0, scale^2) drawn in float32, optionally plus ``add(r0, r1)``."""
    rows = dst.shape[0]
    per_row = max(1, dst[0].numel())
    step = max(1, _CHUNK_ELEMS // per_row)
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        x = torch.randn((r1 - r0,) + tuple(dst.shape[1:]), generator=gen,
                        device=dst.device, dtype=torch.float32)
        if scale != 1.0:
            x.mul_(scale)
        if add is not None:
            x.add_(add(r0, r1))
        dst[r0:r1].copy_(x)  # float32 -> bfloat16 copy rounds to nearest even
        del x


def make_inputs(w: Workload, device="cpu"):
    """Return ``(q, k, v)``.

    Prefill (``q_len == kv_len`` and ``batch == 1``): q ``[L, H, D]``, k and v
    ``[L, Hkv, D]``.  Otherwise: q ``[S, Lq, H, D]``, k and v ``[S, L, Hkv, D]``.
    """
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed)
    dt = w.torch_dtype
    S, Lq, L = w.batch, w.q_len, w.kv_len
    H, G, D, B = w.n_heads, w.n_kv_heads, w.head_dim, w.block_size
    nb = w.n_blocks
    offsets = torch.randn((S, nb, G, D), generator=gen, device=device,
                          dtype=torch.float32).mul_(0.5)
    q = torch.empty((S, Lq, H, D), dtype=dt, device=device)
    k = torch.empty((S, L, G, D), dtype=dt, device=device)
    v = torch.empty((S, L, G, D), dtype=dt, device=device)
    for s in range(S):
        _normal_into(q[s], gen)

        def k_offset(r0, r1, s=s):
            blk = torch.arange(r0, r1, device=device) // B
            return offsets[s].index_select(0, blk)

        _normal_into(k[s], gen, add=k_offset)
        _normal_into(v[s], gen)
    del offsets
    if S == 1 and Lq == L:
        return q[0], k[0], v[0]
    return q, k, v
