"""lsh_sort_noalloc (the sort with the library's static scratch, for callers
that cannot allocate) against lsh_sort with a caller workspace, bit for bit,
through the C ABI: two calls in a row, the second on a smaller input, then the
same-bucket variant (window ids and the bucket ranks in the scratch)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import gpu_parity as GP
import lsh_attention_02_amd as lsh
from synthetic_inputs import Workload, make_inputs

pytestmark = pytest.mark.gpu


def _hash(w: Workload, flags: int = 0):
    x = make_inputs(w)
    cfg = GP.cfg_of(w, flags=flags)
    t = GP.upload(w, x)
    buckets = lsh.lsh_hash(cfg, t["qk"], t["R"])
    return cfg, buckets


def test_sort_noalloc_matches_sort():
    cases = [
        # the 64K-token workload's sort geometry at 16K tokens (8 rounds, tiles of 2048)
        (Workload("noalloc_a", batch=1, heads=8, seq_len=16384, d_head=128, dtype="bf16",
                  n_buckets=1024, n_rounds=8, chunk=64, causal=True, seed=170), 0),
        # a smaller one right after: the scratch holds the first call's counters
        (Workload("noalloc_b", batch=2, heads=3, seq_len=1344, d_head=64, dtype="bf16",
                  n_buckets=10, n_rounds=3, chunk=64, causal=True, seed=171), 0),
        # the same-bucket variant: bucket ranks in the scratch, window ids in cid
        (Workload("noalloc_c", batch=1, heads=4, seq_len=4096, d_head=64, dtype="bf16",
                  n_buckets=64, n_rounds=4, chunk=64, causal=False, seed=172),
         lsh.LSH_FLAG_SAME_BUCKET),
    ]
    for w, flags in cases:
        cfg, buckets = _hash(w, flags)
        perm_a, cid_a = lsh.lsh_sort(cfg, buckets)
        perm_b, cid_b = lsh.lsh_sort_noalloc(cfg, buckets)
        torch.cuda.synchronize()
        assert torch.equal(perm_a, perm_b), w.name
        assert torch.equal(cid_a, cid_b), w.name
        GP.log(f"[noalloc] {w.name} flags {flags}: perm and cid equal to lsh_sort "
               f"({perm_a.numel()} slots)")


def test_sort_noalloc_rejects_oversize():
    """A configuration whose counters exceed the static buffer is refused
    before anything is launched."""
    w = Workload("noalloc_big", batch=1, heads=64, seq_len=1 << 20, d_head=64, dtype="bf16",
                 n_buckets=16384, n_rounds=4, chunk=128, causal=True, seed=173)
    cfg = GP.cfg_of(w)
    assert lsh.lsh_sort_workspace_bytes(cfg) > lsh.SORT_NOALLOC_MAX_BYTES
    b = torch.zeros((1, 64, 4, 1 << 20), dtype=torch.int32, device="cuda:0")
    with pytest.raises(lsh.LSHError) as e:
        lsh.lsh_sort_noalloc(cfg, b)
    assert e.value.status == lsh.LSH_ERR_WORKSPACE
