"""C-ABI checks that need no GPU: the library loads, exports every function
include/moba.h declares, and rejects bad arguments before touching HIP."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "block_sparse_attention_gate_amd", "libmoba.so")
HEADER = os.path.join(ROOT, "include", "moba.h")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libmoba.so not built")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(moba_[a-z0-9_]+)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(LIB)
    names = _declared_functions()
    assert len(names) >= 13, names
    for n in names:
        assert hasattr(lib, n), f"{n} declared in moba.h but not exported"


def test_binding_covers_the_header():
    import block_sparse_attention_gate_amd as moba
    assert set(_declared_functions()) <= set(moba.EXPORTED)
    for n in _declared_functions():
        assert hasattr(moba, n), n


def test_version_and_status_strings():
    import block_sparse_attention_gate_amd as moba
    assert moba.moba_abi_version() == 4
    assert moba.moba_status_string(0) == "MOBA_OK"
    assert moba.moba_status_string(2) == "MOBA_ERR_UNSUPPORTED"
    assert moba.moba_status_string(99) == "MOBA_STATUS_UNKNOWN"


def _args(**kw):
    import block_sparse_attention_gate_amd as moba
    a = moba.MobaArgs()
    a.struct_size = ctypes.sizeof(moba.MobaArgs)
    fake = 1 << 40   # never dereferenced: every case fails validation first
    a.q = a.k = a.v = a.out = fake
    a.batch, a.n_heads, a.n_kv_heads, a.head_dim = 1, 32, 8, 128
    a.block_size, a.topk = 4096, 12
    a.q_len = a.kv_len = 1 << 20
    a.dtype = moba.MOBA_DTYPE_BF16
    for k_, v_ in kw.items():
        setattr(a, k_, v_)
    return a


@pytest.mark.parametrize("field,value,status", [
    ("q", 0, 1), ("head_dim", 96, 2), ("block_size", 100, 2), ("block_size", 0, 1),
    ("topk", 0, 1), ("topk", 18, 2), ("n_kv_heads", 5, 1), ("q_len", 0, 1),
    ("dtype", 7, 2), ("kv_len", (1 << 20) + 64, 1), ("struct_size", 8, 1),
])
def test_validation_rejects_before_any_launch(field, value, status):
    import block_sparse_attention_gate_amd as moba
    a = _args(**{field: value})
    if field == "kv_len":      # q_len > kv_len is invalid
        a.q_len = value + 64
    st = moba._lib.moba_forward_ex(ctypes.byref(a))
    assert st == status, (field, value, st, moba.moba_last_error())
    assert moba.moba_last_error()


def test_workspace_size_of_the_1m_prefill():
    """Workspace for 1M tokens, 32/8 heads, block 4096, top-k 12: V^T, block
    means, selection, routing tables and the routed partials (bf16 o + fp32
    lse + list entry per slot).  All 32 heads' partials would be ~94 GB, past
    the default 12 GiB routed limit, so the forward routes one KV head (four
    query heads, 11.9 GB of partials) at a time: the workspace holds one
    pass, under 16 GiB.  A limit above the whole problem's partials keeps
    them all."""
    import block_sparse_attention_gate_amd as moba
    L, slots_all = 1 << 20, 32 * (1 << 20) * 11
    vt, sel, counts = L * 8 * 128 * 2, 32 * L * 12 * 4, 8 * 256 * (4 * L // 128) * 4
    per_slot = 128 * 2 + 4 + 4
    a = _args()
    n = moba._lib.moba_workspace_size(ctypes.byref(a))
    expect_min = vt + sel + counts + (slots_all // 8) * per_slot
    assert expect_min <= n <= expect_min * 1.05, (n, expect_min)
    assert n < 16 << 30
    a.routed_bytes_limit = 128 << 30
    n_all = moba._lib.moba_workspace_size(ctypes.byref(a))
    expect_all = vt + sel + counts + slots_all * per_slot
    assert expect_all <= n_all <= expect_all * 1.05, (n_all, expect_all)
    bad = _args(head_dim=96)
    assert moba._lib.moba_workspace_size(ctypes.byref(bad)) == 0
    assert "head_dim" in moba.moba_last_error()


def test_workspace_size_of_the_32k_prefill():
    """Small problem (32K tokens, one head, block 2048, top-k 3): V^T, routed
    partials for 2 past blocks per query and the two own-block halves."""
    import block_sparse_attention_gate_amd as moba
    L = 1 << 15
    a = _args(n_heads=1, n_kv_heads=1, block_size=2048, topk=3, q_len=L, kv_len=L)
    n = moba._lib.moba_workspace_size(ctypes.byref(a))
    vt = L * 128 * 2
    routed = L * 2 * (128 * 2 + 4 + 4)     # partial o, lse, list entry per slot
    own = 2 * L * (128 * 2 + 4)            # two own-block halves
    expect_min = vt + routed + own
    assert expect_min <= n <= expect_min * 1.1, (n, expect_min)


def test_full_workspace_sizes():
    """Full attention: at 32K one head the rows run in 4096-key chunks (8
    partials per query); at 1M x 32 heads whole rows fill the chip (V^T only)."""
    import block_sparse_attention_gate_amd as moba
    L = 1 << 15
    a = _args(n_heads=1, n_kv_heads=1, q_len=L, kv_len=L)
    n = moba._lib.moba_full_workspace_size(ctypes.byref(a))
    expect_min = L * 128 * 2 + 8 * L * (128 * 2 + 4)
    assert expect_min <= n <= expect_min * 1.01, (n, expect_min)
    big = _args()
    n = moba._lib.moba_full_workspace_size(ctypes.byref(big))
    vt = (1 << 20) * 8 * 128 * 2
    assert vt <= n <= vt * 1.01, n


def test_naive_workspace_and_validation():
    """Mask-based form: the workspace holds fp32 scores and bf16
    probabilities for every (query, key) pair (kv_len rounded up to 64) on top
    of V^T; fp32 is refused, and so is a score matrix with 2^31 rows."""
    import block_sparse_attention_gate_amd as moba
    L = 1 << 15
    a = _args(n_heads=1, n_kv_heads=1, block_size=2048, topk=3, q_len=L, kv_len=L)
    n = moba._lib.moba_naive_workspace_size(ctypes.byref(a))
    expect_min = 6 * L * L + L * 128 * 2
    assert expect_min <= n <= expect_min * 1.01, (n, expect_min)
    ragged = _args(n_heads=2, n_kv_heads=1, block_size=128, topk=3, q_len=1000, kv_len=1000)
    n = moba._lib.moba_naive_workspace_size(ctypes.byref(ragged))
    assert n >= 6 * 2 * 1000 * 1024, n
    f32 = _args(n_heads=1, n_kv_heads=1, dtype=moba.MOBA_DTYPE_F32)
    assert moba._lib.moba_naive_workspace_size(ctypes.byref(f32)) == 0
    assert "bf16" in moba.moba_last_error()
    assert moba._lib.moba_naive_ex(ctypes.byref(f32)) == 2   # UNSUPPORTED, nothing enqueued
    rows = _args(n_heads=2048, n_kv_heads=1, topk=1, q_len=1 << 20, kv_len=1 << 20)
    assert moba._lib.moba_naive_workspace_size(ctypes.byref(rows)) == 0
    assert "too large" in moba.moba_last_error()


def test_ragged_lengths_are_accepted():
    """kv_len need not be a multiple of the block size or of 64: the bf16
    workspace then holds V^T padded to a multiple of 64 keys and the last,
    partial K tile of every sequence and KV head."""
    import block_sparse_attention_gate_amd as moba
    for L in (1000, 37, 4097):
        a = _args(n_heads=4, n_kv_heads=2, block_size=128, topk=3, q_len=L, kv_len=L)
        n = moba._lib.moba_workspace_size(ctypes.byref(a))
        lv = -(-L // 64) * 64
        assert n >= 2 * lv * 128 * 2 + 64 * 2 * 128 * 2, (L, n, moba.moba_last_error())
        assert moba._lib.moba_full_workspace_size(ctypes.byref(a)) >= 2 * lv * 128 * 2
    dec = _args(batch=2, q_len=1, kv_len=(1 << 20) + 5)
    assert moba._lib.moba_workspace_size(ctypes.byref(dec)) > 0, moba.moba_last_error()
    # the transposed V is addressed with 32-bit offsets in the bf16 prefill
    big = _args(n_heads=1, n_kv_heads=1, block_size=4096, topk=2, q_len=1 << 24,
                kv_len=1 << 24)
    assert moba._lib.moba_workspace_size(ctypes.byref(big)) == 0
    assert "2^31" in moba.moba_last_error()


def test_too_small_workspace_is_rejected():
    import block_sparse_attention_gate_amd as moba
    a = _args()
    a.workspace = 1 << 41
    a.workspace_bytes = 1024
    assert moba._lib.moba_forward_ex(ctypes.byref(a)) == moba.MOBA_ERR_INVALID_ARGUMENT
    assert "workspace too small" in moba.moba_last_error()


def test_python_binding_rejects_host_tensors():
    import torch
    import block_sparse_attention_gate_amd as moba
    q = torch.zeros(128, 1, 64)
    with pytest.raises(ValueError):
        moba.moba_forward(q, q, q, 64, 2)


def test_profile_names():
    import block_sparse_attention_gate_amd as moba
    for n in moba.KERNEL_NAMES:
        assert moba.moba_profile_read(n) == (0.0, 0)
    with pytest.raises(ValueError):
        moba.moba_profile_read("nope")


def test_version_one_struct_is_accepted():
    """A caller built against the version-1 header (moba_args without
    lse_out) passes the smaller struct_size; it is accepted and lse_out is
    taken as NULL."""
    import block_sparse_attention_gate_amd as moba
    a = _args()
    v1 = moba.MobaArgs.lse_out.offset
    a.struct_size = v1
    assert moba._lib.moba_workspace_size(ctypes.byref(a)) > 0, moba.moba_last_error()
    a.struct_size = v1 + 4
    assert moba._lib.moba_workspace_size(ctypes.byref(a)) == 0
    assert "struct_size" in moba.moba_last_error()


def test_grouped_workspace_of_the_128k_prefill():
    """128K tokens, 32/8 heads, block 4096, top-k 12: the routed partials of
    all heads (9.9 GB) fit the default limit (one pass); a 3 GiB limit gives
    passes of two KV heads (2.5 GB each), a 1-byte limit passes of one."""
    import block_sparse_attention_gate_amd as moba
    L = 1 << 17
    slots_kv = 4 * L * 11
    per_slot = 128 * 2 + 4 + 4
    a = _args(q_len=L, kv_len=L)
    sizes = []
    for limit in (0, 3 << 30, 1):
        a.routed_bytes_limit = limit
        sizes.append(moba._lib.moba_workspace_size(ctypes.byref(a)))
    assert sizes[0] - sizes[1] == pytest.approx(6 * slots_kv * per_slot, rel=0.01), sizes
    assert sizes[1] - sizes[2] == pytest.approx(slots_kv * per_slot, rel=0.01), sizes


def test_version_three_struct_is_accepted():
    """A version-3 struct (up to kv_lens) is accepted with routed_bytes_limit
    taken as 0 (the default limit); bytes past it are never read."""
    import block_sparse_attention_gate_amd as moba
    a = _args()
    n4 = moba._lib.moba_workspace_size(ctypes.byref(a))
    a.struct_size = moba.MobaArgs.routed_bytes_limit.offset
    a.routed_bytes_limit = 1 << 50      # past the version-3 struct: never read
    assert moba._lib.moba_workspace_size(ctypes.byref(a)) == n4, moba.moba_last_error()


def test_version_two_struct_and_kv_lens_validation():
    """A version-2 struct (up to lse_out) is accepted with kv_lens taken as
    NULL; kv_lens is refused off the decode path (q_len > 1, block size not
    a multiple of 512, the mask-based form) before any launch."""
    import block_sparse_attention_gate_amd as moba
    fake = 1 << 40
    a = _args(batch=8, q_len=1, kv_len=1 << 20)
    a.struct_size = moba.MobaArgs.kv_lens.offset
    a.kv_lens = 3   # past the version-2 struct: never read
    assert moba._lib.moba_workspace_size(ctypes.byref(a)) > 0, moba.moba_last_error()
    a.struct_size = ctypes.sizeof(moba.MobaArgs)
    a.kv_lens = fake
    assert moba._lib.moba_workspace_size(ctypes.byref(a)) > 0, moba.moba_last_error()
    a.kv_lens = fake + 2
    assert moba._lib.moba_workspace_size(ctypes.byref(a)) == 0
    assert "aligned" in moba.moba_last_error()
    a.kv_lens = fake
    a.q_len = 2
    assert moba._lib.moba_forward_ex(ctypes.byref(a)) == moba.MOBA_ERR_UNSUPPORTED
    assert "q_len 1" in moba.moba_last_error()
    a.q_len, a.block_size = 1, 256
    assert moba._lib.moba_forward_ex(ctypes.byref(a)) == moba.MOBA_ERR_UNSUPPORTED
    assert "decode kernels" in moba.moba_last_error()
    a.block_size = 4096
    assert moba._lib.moba_naive_workspace_size(ctypes.byref(a)) == 0
    assert "kv_lens" in moba.moba_last_error()
    full = _args(batch=8, q_len=1, kv_len=1 << 20, n_heads=64, n_kv_heads=2)
    full.kv_lens = fake
    assert moba._lib.moba_full_attention_ex(ctypes.byref(full)) == moba.MOBA_ERR_UNSUPPORTED


def test_plain_c_consumer_host_checks():
    """A C program built with gcc against include/moba.h and libmoba.so (no
    Python, no C++) checks the version, status strings and argument
    validation without a GPU."""
    import subprocess
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "moba_build", os.path.join(ROOT, "block_sparse_attention_gate_amd", "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    exe = b.CONSUMER_PATH if os.path.exists(b.CONSUMER_PATH) else b.build_consumer()
    res = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    print(res.stdout)
    assert res.returncode == 0 and res.stdout.strip().endswith("passed"), res.stdout + res.stderr


def _varlen(cu_q, cu_k, **kw):
    import block_sparse_attention_gate_amd as moba
    import numpy as np
    a = moba.MobaVarlenArgs()
    a.struct_size = ctypes.sizeof(moba.MobaVarlenArgs)
    fake = 1 << 40   # never dereferenced: sizes only
    a.q = a.k = a.v = a.out = fake
    cq = np.asarray(cu_q, dtype=np.int64)
    ck = np.asarray(cu_k, dtype=np.int64)
    a.cu_seqlens_q, a.cu_seqlens_k = cq.ctypes.data, ck.ctypes.data
    a.batch = len(cu_q) - 1
    a.n_heads, a.n_kv_heads, a.head_dim, a.block_size, a.topk = 4, 2, 128, 128, 3
    a.dtype = moba.MOBA_DTYPE_BF16
    for k_, v_ in kw.items():
        setattr(a, k_, v_)
    return a, (cq, ck)


def test_varlen_validation_before_any_launch():
    """Packed batches: every sequence is planned up front; lengths may be zero;
    decreasing offsets, a sequence with more queries than keys, or a bad
    sequence (head_dim) are refused with the sequence named."""
    import block_sparse_attention_gate_amd as moba
    a, keep = _varlen([0, 300, 300, 377, 1377], [0, 300, 300, 1534, 2534])
    assert moba._lib.moba_varlen_workspace_size(ctypes.byref(a), 0) > 0, moba.moba_last_error()
    a.dout = a.dq = a.dk = a.dv = a.sel = a.lse = 1 << 40
    assert moba._lib.moba_varlen_workspace_size(ctypes.byref(a), 1) > 0, moba.moba_last_error()
    a, keep = _varlen([0, 300, 200], [0, 300, 400])
    assert moba._lib.moba_varlen_workspace_size(ctypes.byref(a), 0) == 0
    assert "decrease" in moba.moba_last_error()
    a, keep = _varlen([0, 300, 700], [0, 300, 500])
    assert moba._lib.moba_varlen_workspace_size(ctypes.byref(a), 0) == 0
    assert "sequence 1" in moba.moba_last_error()
    a, keep = _varlen([0, 64], [0, 64], head_dim=96)
    assert moba._lib.moba_varlen_workspace_size(ctypes.byref(a), 0) == 0
    assert "sequence 0" in moba.moba_last_error() and "head_dim" in moba.moba_last_error()
    a, keep = _varlen([0, 64], [0, 64])   # backward without its inputs
    assert moba._lib.moba_backward_varlen(ctypes.byref(a)) == moba.MOBA_ERR_INVALID_ARGUMENT


def test_block_count_limit():
    """8192 blocks is the largest supported count (LDS histograms of the
    routing kernels); one more is refused before any launch."""
    import block_sparse_attention_gate_amd as moba
    a = _args(n_heads=1, n_kv_heads=1, head_dim=64, block_size=64, topk=3,
              q_len=8192 * 64, kv_len=8192 * 64)
    assert moba._lib.moba_workspace_size(ctypes.byref(a)) > 0, moba.moba_last_error()
    a.q_len = a.kv_len = 8192 * 64 + 1
    assert moba._lib.moba_workspace_size(ctypes.byref(a)) == 0
    assert "8192" in moba.moba_last_error()


def test_noalloc_refuses_a_problem_past_its_scratch():
    """moba_forward_noalloc holds a 64 MiB scratch array per GPU: a problem
    whose workspace is larger is UNSUPPORTED, refused before any launch (no
    GPU is touched), with the sizes in the message."""
    import block_sparse_attention_gate_amd as moba
    a = _args(q_len=1 << 17, kv_len=1 << 17)      # 128K tokens, 32/8 heads
    assert moba._lib.moba_workspace_size(ctypes.byref(a)) > 64 << 20
    assert moba._lib.moba_forward_noalloc(ctypes.byref(a)) == moba.MOBA_ERR_UNSUPPORTED
    assert "moba_forward_noalloc holds at most" in moba.moba_last_error()
    bad = _args(head_dim=96)
    assert moba._lib.moba_forward_noalloc(ctypes.byref(bad)) == moba.MOBA_ERR_UNSUPPORTED
    assert "head_dim" in moba.moba_last_error()
