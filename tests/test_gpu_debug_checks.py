"""The debug build's device-side bounds checks (liblsh_attention_debug.so).

On valid inputs the debug build gives the release build's results bit for bit
and counts no failed check.  Out-of-range positions in perm (chunk attention
and its backward) and out-of-range bucket ids (sort) are clamped or skipped by
the kernels of both builds, which then finish normally; the debug build counts
them.  Every call here goes through the C ABI of one of the two libraries."""
import pytest
import torch

import lsh_attention_02_amd as lsh
import lsh_attention_02_amd._binding as B
from synthetic_inputs import Workload, make_inputs

pytestmark = pytest.mark.gpu

CASES = {
    "bf16_d64_r4_causal": Workload("dbg_d64", batch=1, heads=2, seq_len=1024, d_head=64, dtype="bf16",
                                   n_buckets=32, n_rounds=4, chunk=64, causal=True, seed=11),
    "bf16_d128_r8": Workload("dbg_d128", batch=2, heads=2, seq_len=2048, d_head=128, dtype="bf16",
                             n_buckets=64, n_rounds=8, chunk=64, causal=False, seed=12),
    "f32_d64_chunk32_r3": Workload("dbg_f32", batch=1, heads=3, seq_len=960, d_head=64, dtype="f32",
                                   n_buckets=24, n_rounds=3, chunk=32, causal=True, seed=13),
}


@pytest.fixture(scope="module")
def dbg():
    lib = lsh.load_debug_library()
    lsh.debug_check_failures(lib, reset=True)
    return lib


def _cfg(w, flags=0):
    return lsh.LSHConfig(w.batch, w.heads, w.seq_len, w.d_head, w.n_buckets, w.n_rounds, w.chunk,
                         w.causal, dtype=w.dtype, flags=flags)


def _tensors(w):
    x = make_inputs(w)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    return {k: torch.from_numpy(x[k]).to("cuda:0").to(dt) for k in ("qk", "v", "R")}


def _run_forward_backward(w, flags=0):
    cfg = _cfg(w, flags)
    t = _tensors(w)
    out = lsh.forward(cfg, t["qk"], t["v"], t["R"], return_all=True)
    if w.dtype == "bf16" and w.chunk == 64:
        d_o = torch.randn(out["o"].shape, generator=torch.Generator().manual_seed(w.seed)).to(out["o"])
        out["d_qk"], out["d_v"] = lsh.lsh_attn_backward(cfg, t["qk"], t["v"], out["perm"], out["cid"],
                                                        out["lse"], out["o"], d_o)
    torch.cuda.synchronize()
    return {k: v.cpu() for k, v in out.items()}


@pytest.mark.parametrize("name", sorted(CASES))
def test_debug_build_matches_release_and_counts_nothing(name, dbg, monkeypatch):
    w = CASES[name]
    print(f"debug-check case {name}", flush=True)
    rel = _run_forward_backward(w)
    assert lsh.debug_check_failures() == 0          # the release build has no checks
    monkeypatch.setattr(B, "_lib", dbg)
    lsh.debug_check_failures(dbg, reset=True)
    got = _run_forward_backward(w)
    assert lsh.debug_check_failures(dbg, reset=True) == 0
    assert sorted(got) == sorted(rel)
    for k in rel:
        assert torch.equal(got[k], rel[k]), k


def test_debug_build_same_bucket_variant(dbg, monkeypatch):
    w = CASES["bf16_d64_r4_causal"]
    rel = _run_forward_backward(w, flags=lsh.LSH_FLAG_SAME_BUCKET)
    monkeypatch.setattr(B, "_lib", dbg)
    lsh.debug_check_failures(dbg, reset=True)
    got = _run_forward_backward(w, flags=lsh.LSH_FLAG_SAME_BUCKET)
    assert lsh.debug_check_failures(dbg, reset=True) == 0
    for k in rel:
        assert torch.equal(got[k], rel[k]), k


def test_out_of_range_positions_are_counted(dbg, monkeypatch):
    """perm entries outside [0, L) reach chunk attention and its backward: both
    clamp them to a valid row (so no access leaves the buffers) and the debug
    build counts them."""
    w = CASES["bf16_d64_r4_causal"]
    cfg = _cfg(w)
    t = _tensors(w)
    monkeypatch.setattr(B, "_lib", dbg)
    out = lsh.forward(cfg, t["qk"], t["v"], t["R"], return_all=True)
    torch.cuda.synchronize()
    assert lsh.debug_check_failures(dbg, reset=True) == 0
    perm = out["perm"].clone()
    perm[0, 0, 0, 0] = w.seq_len + 5
    perm[0, 1, 2, 77] = -3
    perm[0, 1, 3, w.seq_len - 1] = 1 << 30
    o_r, lse = lsh.lsh_chunk_attn(cfg, t["qk"], t["v"], perm, out["cid"])
    torch.cuda.synchronize()
    n_attn = lsh.debug_check_failures(dbg, reset=True)
    assert n_attn >= 3
    assert torch.isfinite(o_r.float()).all() and torch.isfinite(lse).all()
    d_o = torch.ones_like(out["o"])
    d_qk, d_v = lsh.lsh_attn_backward(cfg, t["qk"], t["v"], perm, out["cid"], lse, out["o"], d_o)
    torch.cuda.synchronize()
    assert lsh.debug_check_failures(dbg, reset=True) >= 3
    assert torch.isfinite(d_qk).all() and torch.isfinite(d_v).all()


@pytest.mark.parametrize("L,nb,nr", [(1024, 32, 2), (65536, 1024, 2), (4096, 2048, 2)])
def test_out_of_range_buckets_are_counted(L, nb, nr, dbg, monkeypatch):
    """Bucket ids outside [0, n_buckets) reach the sort (its counting and
    placement kernels for up to 1024 buckets, the LDS-table placement above):
    the positions are skipped and the debug build counts them; the valid
    positions are still placed."""
    cfg = lsh.LSHConfig(batch=1, heads=2, seq_len=L, d_head=64, n_buckets=nb, n_rounds=nr, chunk=64,
                        causal=True, dtype="bf16")
    g = torch.Generator().manual_seed(L + nb)
    b = torch.randint(0, nb, (1, 2, nr, L), generator=g, dtype=torch.int32)
    b[0, 0, 0, 3] = nb
    b[0, 1, nr - 1, L - 1] = -1
    b[0, 1, 0, L // 2] = 1 << 20
    monkeypatch.setattr(B, "_lib", dbg)
    lsh.debug_check_failures(dbg, reset=True)
    perm, cid = lsh.lsh_sort(cfg, b.cuda())
    torch.cuda.synchronize()
    assert lsh.debug_check_failures(dbg, reset=True) >= 3
    # an untouched segment is still sorted exactly
    seg = b[0, 0, nr - 1]
    want = torch.argsort(seg.long() * L + torch.arange(L), stable=True).to(torch.int32)
    assert torch.equal(perm[0, 0, nr - 1].cpu(), want)
