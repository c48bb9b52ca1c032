"""GPU parity of the four HIP steps (called through the C ABI) against the CPU oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import gpu_parity as GP
import lsh_attention_02_amd as lsh
import oracle.lsh_oracle as O
import reference_forms as RF
from synthetic_inputs import WORKLOADS, Workload, make_inputs

pytestmark = pytest.mark.gpu


def W(name, **kw) -> Workload:
    base = dict(batch=1, heads=1, seq_len=1024, d_head=64, dtype="bf16", n_buckets=32, n_rounds=2,
                chunk=64, causal=True, seed=100)
    base.update(kw)
    return Workload(name, **base)


# Small workloads the oracle finishes in seconds; several tiles of every kernel
# and ragged tails (L not a multiple of the hash workgroup's 512 tokens, chunk
# counts not a multiple of the attention run of 16 chunks, partial column tiles).
SMALL = {
    # runs of several chunks (the run length adapts to the problem size: these
    # have 2 and 3 chunks per run, with a ragged last run)
    "runs2_b2h8_L1344_r4": W("runs2", batch=2, heads=8, seq_len=1344, n_buckets=10, n_rounds=4,
                             seed=107),
    "runs3_b2h8_L4096_r3_d128": W("runs3", batch=2, heads=8, seq_len=4096, d_head=128,
                                  n_buckets=32, n_rounds=3, causal=False, seed=108),
    "tiny_f32": WORKLOADS["tiny_f32"],
    "short_4k": WORKLOADS["short_4k"],
    "ragged_b2h3_L1344_nb10_r3": W("ragged", batch=2, heads=3, seq_len=1344, n_buckets=10,
                                   n_rounds=3, seed=101),
    "d128_L2048_r4": W("d128", heads=2, seq_len=2048, d_head=128, n_buckets=64, n_rounds=4, seed=102),
    "chunk128_L2560": W("c128", heads=2, seq_len=2560, n_buckets=40, chunk=128, seed=103),
    "chunk128_d128_L2048_r3": W("c128d128", heads=2, seq_len=2048, d_head=128, n_buckets=32,
                                n_rounds=3, chunk=128, seed=113),
    # chunk 128 with 8 rounds (four packed chunk-id words) and several runs
    "chunk128_L4096_r8": W("c128r8", heads=2, seq_len=4096, n_buckets=32, n_rounds=8, chunk=128,
                           seed=114),
    "chunk32_noncausal_r5": W("c32", heads=2, seq_len=1056, n_buckets=16, n_rounds=5, chunk=32,
                              causal=False, seed=104),
    "f32_d128_r2_scale1": W("f32d128", seq_len=576, d_head=128, dtype="f32", n_buckets=16,
                            causal=True, seed=105),
    "f32_chunk128_d64": W("f32c128", seq_len=768, dtype="f32", n_buckets=24, n_rounds=3,
                          chunk=128, causal=False, seed=106),
    "clustered_b2h2_L4096": W("clu", batch=2, heads=2, seq_len=4096, n_buckets=256, n_rounds=4,
                              causal=False, clustered=True, seed=107),
    "rounds16_buckets1000": W("r16", seq_len=2048, n_buckets=1000, n_rounds=16, seed=108),
    # hash: 200 columns per round, one full and one partial group of 128 staged
    # columns (the bf16 path copies R into LDS and zeroes the columns past 200)
    "groups_d128_nb400_r3": W("grp128", heads=2, seq_len=2048, d_head=128, n_buckets=400,
                              n_rounds=3, seed=111),
    "groups_d64_nb400_r2": W("grp64", heads=2, seq_len=1536, n_buckets=400, n_rounds=2,
                             causal=False, seed=112),
    "one_chunk": W("one", seq_len=64, n_buckets=6, n_rounds=3, seed=109),
    "two_chunks_nb2": W("two", seq_len=128, n_buckets=2, n_rounds=1, seed=110),
}


@pytest.mark.parametrize("name", sorted(SMALL))
def test_full_parity(name):
    w = SMALL[name]
    scale = 1.0 if name == "f32_d128_r2_scale1" else None
    GP.full_parity(w, scale=scale)


# Variant flags: LSH_FLAG_NO_DUP_CORRECTION (1), LSH_FLAG_WRAP_LOOKBACK (2), both,
# LSH_FLAG_SAME_BUCKET (4) and 4 without the correction, on cases with several
# 16-chunk attention runs (the wrapped look-back of chunk 0 and of every later
# run), one chunk, 16 rounds, f32, d128 and bf16 chunk 128.
FLAG_CASES = {
    "short_4k": WORKLOADS["short_4k"],
    "ragged_b2h3_L1344_nb10_r3": SMALL["ragged_b2h3_L1344_nb10_r3"],
    "d128_L2048_r4": SMALL["d128_L2048_r4"],
    "chunk32_noncausal_r5": SMALL["chunk32_noncausal_r5"],
    "f32_chunk128_d64": SMALL["f32_chunk128_d64"],
    "chunk128_L2560": SMALL["chunk128_L2560"],
    "rounds16_buckets1000": SMALL["rounds16_buckets1000"],
    "one_chunk": SMALL["one_chunk"],
    "two_chunks_nb2": SMALL["two_chunks_nb2"],
}


@pytest.mark.parametrize("flags", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("name", sorted(FLAG_CASES))
def test_variant_parity(name, flags):
    GP.full_parity(FLAG_CASES[name], flags=flags)


@pytest.mark.parametrize("causal", [False, True])
def test_wrap_two_chunks_is_full_attention(causal):
    """With the wrapped look-back and two chunks, both chunks see the whole
    sequence in every round: textbook attention with the self-mask."""
    w = W("wrap2", seq_len=256, n_buckets=16, n_rounds=3, chunk=128, causal=causal,
          seed=121 + causal)
    x = make_inputs(w)
    _, _, g = GP.run_gpu(w, x, flags=lsh.LSH_FLAG_WRAP_LOOKBACK)
    ref = RF.full_attention_self_masked(x["qk"][0, 0], x["v"][0, 0], causal, 1 / np.sqrt(64))
    err = GP.rel_err(GP.to_np(g["o"])[0, 0], ref)
    assert err <= GP.GATE["bf16"], err


def test_maximum_sizes_sampled():
    """The largest chunk count (32767: chunk ids fill int16) and bucket count
    (32768) the boundary accepts, with two rounds at L = 32767 * 32."""
    w = W("max_sizes", seq_len=32767 * 32, chunk=32, n_buckets=32768, n_rounds=2, causal=True,
          seed=130)
    GP.sampled_parity(w, n_samples=256)


@pytest.mark.parametrize("flags", [lsh.LSH_FLAG_NO_DUP_CORRECTION | lsh.LSH_FLAG_WRAP_LOOKBACK,
                                   lsh.LSH_FLAG_SAME_BUCKET])
def test_full_size_sampled_variants(flags):
    """paper_64k with variant flags, in the benchmark's launch configuration."""
    GP.sampled_parity(WORKLOADS["paper_64k"], n_samples=512, flags=flags)


# The attention layer (projections around the four steps).  Ragged: 1344 rows
# and 192 output columns are not multiples of the 128 x 128 GEMM tile.
LAYER_CASES = {
    "b2_L512_dm256_h4_d64": (W("layer_a", batch=2, heads=4, seq_len=512, n_buckets=16, seed=140), 256),
    "L1024_dm512_h4_d128": (W("layer_b", heads=4, seq_len=1024, d_head=128, n_buckets=32,
                               n_rounds=4, seed=141), 512),
    "ragged_L1344_dm192_h3": (W("layer_c", heads=3, seq_len=1344, n_buckets=10, n_rounds=3,
                                causal=False, seed=142), 192),
}


@pytest.mark.parametrize("name", sorted(LAYER_CASES))
def test_layer_parity(name):
    w, d_model = LAYER_CASES[name]
    GP.layer_parity(w, d_model)


def test_layer_parity_paper_shape_same_bucket():
    """d_model 1024 and 8 heads of 128, as the pages' set-up, at L = 2048, with the
    same-bucket variant."""
    w = W("layer_paper", heads=8, seq_len=2048, d_head=128, n_buckets=64, n_rounds=4, seed=143)
    GP.layer_parity(w, 1024, flags=lsh.LSH_FLAG_SAME_BUCKET)


def test_native_library_is_loaded():
    lsh.load_library()
    with open("/proc/self/maps") as f:
        maps = f.read()
    assert "liblsh_attention.so" in maps


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_one_chunk_is_full_attention(causal, dtype):
    """chunk = L: every round's window is the whole sequence, so the GPU forward
    equals textbook softmax attention with the self-mask (2 buckets, as in the
    minimal case; any bucket count gives the same)."""
    w = W("full", seq_len=128, n_buckets=2, n_rounds=3, chunk=128, causal=causal, dtype=dtype,
          seed=111 + causal)
    x = make_inputs(w)
    _, _, g = GP.run_gpu(w, x)
    ref = RF.full_attention_self_masked(x["qk"][0, 0], x["v"][0, 0], causal, 1 / np.sqrt(64))
    err = GP.rel_err(GP.to_np(g["o"])[0, 0], ref)
    assert err <= GP.GATE[dtype], err


def test_zero_and_repeated_tokens():
    """Zero vectors hash to bucket 0; identical tokens tie everywhere.  The
    layered checks still hold (near-ties are excluded from the bucket gate)."""
    w = W("degenerate", heads=2, seq_len=1024, n_buckets=16, n_rounds=3, seed=112)
    x = make_inputs(w)
    x["qk"][0, 0, :100] = 0.0
    x["qk"][0, 1, 200:700] = x["qk"][0, 1, 50]
    rep = GP.full_parity(w, x=x)
    cfg, _, g = GP.run_gpu(w, x)
    assert np.all(GP.to_np(g["buckets"])[0, 0, :, :100] == 0)


def test_determinism():
    w = WORKLOADS["short_4k"]
    x = make_inputs(w)
    _, _, a = GP.run_gpu(w, x)
    _, _, b = GP.run_gpu(w, x)
    for k in a:
        assert torch.equal(a[k], b[k]), k


def test_clustered_16k_full():
    """The clustered workload at full size, every output against the oracle."""
    GP.full_parity(WORKLOADS["clustered_16k"])


# (batch row, head) slices checked row by row at full size: paper_64k with its
# hashes, long_1m fed the GPU's sort (a slice's hashes there are 2 TFLOP of fp64)
FULL_SIZE_SLICES = {"paper_64k": ([(0, 5)], True), "long_1m": ([(0, 2)], False)}


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["paper_64k", "long_1m"])
def test_full_size_sampled(name):
    """The benchmark's workloads at full size in its launch configuration:
    every sort output, 512 sampled hashes / rows / tokens, and every row of one
    (batch row, head) slice."""
    slices, with_hash = FULL_SIZE_SLICES[name]
    GP.sampled_parity(WORKLOADS[name], n_samples=512, slices=slices, slice_hash=with_hash)


# Full-tensor cases that reach the kernels the benchmark's workloads run:
# d 128 with 8 rounds (four chunk-id words, two gather register sets) and runs
# of 16 chunks, as paper_64k; bf16 d 64 with chunk 128, 4 rounds (two words) and
# runs of 16 chunks, as long_1m.  Every output of every step is compared.
HEADLINE_SHAPES = {
    "paper_path_L16384_r8_d128": W("paper_path", heads=8, seq_len=16384, d_head=128, n_buckets=256,
                                   n_rounds=8, chunk=64, causal=True, seed=144),
    "long_path_L65536_r4_c128": W("long_path", heads=8, seq_len=65536, d_head=64, n_buckets=1024,
                                  n_rounds=4, chunk=128, causal=True, seed=145),
}


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", sorted(HEADLINE_SHAPES))
def test_full_parity_headline_paths(name):
    GP.full_parity(HEADLINE_SHAPES[name])


def test_streams_and_preallocated_outputs():
    """Calls on a side stream with caller-owned outputs give the same result."""
    w = WORKLOADS["short_4k"]
    x = make_inputs(w)
    cfg, t, ref = GP.run_gpu(w, x)
    s = torch.cuda.Stream()
    outs = {k: torch.empty_like(v) for k, v in ref.items()}
    ws = lsh.sort_workspace(cfg, t["qk"].device)
    with torch.cuda.stream(s):
        lsh.lsh_hash(cfg, t["qk"], t["R"], outs["buckets"], stream=s)
        lsh.lsh_sort(cfg, outs["buckets"], outs["perm"], outs["cid"], ws, stream=s)
        lsh.lsh_chunk_attn(cfg, t["qk"], t["v"], outs["perm"], outs["cid"], outs["o_rounds"],
                           outs["lse"], stream=s)
        lsh.lsh_combine_rounds(cfg, outs["o_rounds"], outs["lse"], outs["o"], stream=s)
    s.synchronize()
    for k in ref:
        assert torch.equal(ref[k], outs[k]), k


def test_side_stream_with_library_allocations():
    """On a side stream, with every output, workspace and intermediate allocated
    by the binding (taken on that stream), forward() and the backward give the
    default stream's results."""
    w = WORKLOADS["short_4k"]
    x = make_inputs(w)
    cfg, t, ref = GP.run_gpu(w, x)
    d_o = torch.randn(ref["o"].shape, generator=torch.Generator().manual_seed(7)).to(
        device=ref["o"].device, dtype=ref["o"].dtype)
    g_ref = lsh.lsh_attn_backward(cfg, t["qk"], t["v"], ref["perm"], ref["cid"], ref["lse"],
                                  ref["o"], d_o)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        o = lsh.forward(cfg, t["qk"], t["v"], t["R"], stream=s)
        g = lsh.lsh_attn_backward(cfg, t["qk"], t["v"], ref["perm"], ref["cid"], ref["lse"],
                                  ref["o"], d_o, stream=s)
    s.synchronize()
    assert torch.equal(o, ref["o"])
    for a, b in zip(g, g_ref):
        assert torch.equal(a, b)


# (L, n_buckets, n_rounds, chunk): power-of-two and other bucket counts, tiles
# cut short by L (L not a multiple of the 2048-position tile), one bucket
# holding most positions, bucket counts where some lanes own no bucket in the
# placement's scan (nb not a multiple of 64) and where the tile is L itself; up
# to 1024 buckets the register placement runs, above it the LDS placement, and
# at 16384 buckets the per-segment scatter
SORT_SWEEP = [
    (2560, 40, 2, 128), (4096, 48, 3, 64), (6144, 100, 4, 32), (4096, 126, 1, 64),
    (4096, 128, 2, 64), (5000, 250, 5, 8), (2048, 2, 2, 64), (1344, 10, 3, 64),
    (8192, 1000, 8, 64), (4096, 1024, 2, 32), (12288, 2046, 2, 64), (6000, 4098, 3, 40),
    (32768, 16384, 2, 64),
    # 32K positions and more: the counting kernel splits each segment's buckets
    # over workgroups (4 ranges; 2 ranges with a ragged last tile; 4 ranges
    # feeding the placement kernel for more than 1024 buckets)
    (32768, 512, 2, 64), (36000, 36, 3, 40), (65536, 2048, 2, 64),
]


@pytest.mark.parametrize("L,nb,nr,chunk", SORT_SWEEP)
@pytest.mark.parametrize("flags", [0, lsh.LSH_FLAG_SAME_BUCKET])
def test_sort_sweep(L, nb, nr, chunk, flags):
    """perm and cid bit-exact against the oracle's stable sort on uniform and
    skewed bucket draws (the skewed ones put half the positions in bucket 0)."""
    rng = np.random.default_rng(L * 31 + nb * 7 + nr)
    cfg = lsh.LSHConfig(batch=1, heads=3, seq_len=L, d_head=64, n_buckets=nb, n_rounds=nr,
                        chunk=chunk, causal=True, dtype="bf16", flags=flags)
    for skew in (False, True):
        b = rng.integers(0, nb, (1, 3, nr, L)).astype(np.int32)
        if skew:
            b[rng.random(b.shape) < 0.5] = 0
        perm, cid = lsh.lsh_sort(cfg, torch.from_numpy(b).cuda())
        torch.cuda.synchronize()
        sp, sc_id = O.sort_rounds(b, nb, chunk)
        assert np.array_equal(perm.cpu().numpy(), sp), (L, nb, nr, chunk, flags, skew)
        gc = cid.cpu().numpy()
        want = GP.window_ids(sc_id, b, nb) if flags else sc_id.view(np.uint16)
        assert np.array_equal(gc.view(np.uint16), want), (L, nb, nr, chunk, flags, skew)


def test_workspace_too_small_is_rejected():
    w = WORKLOADS["short_4k"]
    cfg = GP.cfg_of(w)
    b = torch.zeros((1, 8, 2, 4096), dtype=torch.int32, device="cuda:0")
    ws = torch.empty(16, dtype=torch.uint8, device="cuda:0")
    with pytest.raises(lsh.LSHError) as e:
        lsh.lsh_sort(cfg, b, workspace=ws)
    assert e.value.status == lsh.LSH_ERR_WORKSPACE


# ---------------------------------------------------------------------- backward
# bf16, chunk 64; several runs of 16 chunks with a ragged last run, one chunk
# only, one round, an odd number of rounds, both head sizes, and the variant
# without the duplicate-count term.  Causal cases include positions whose
# windows hold only themselves.
BWD_CASES = {
    "b2h3_L1344_r3_d64_causal": (W("bwd_a", batch=2, heads=3, seq_len=1344, n_buckets=10,
                                   n_rounds=3, seed=150), 0),
    "L2048_r4_d128_noncausal": (W("bwd_b", heads=2, seq_len=2048, d_head=128, n_buckets=64,
                                  n_rounds=4, causal=False, seed=151), 0),
    "L64_single_chunk_r2": (W("bwd_c", heads=2, seq_len=64, n_buckets=4, seed=152), 0),
    "L1152_r1_d128": (W("bwd_d", seq_len=1152, d_head=128, n_buckets=16, n_rounds=1, seed=153), 0),
    "L1088_r5_d64_noncausal": (W("bwd_e", heads=2, seq_len=1088, n_buckets=16, n_rounds=5,
                                 causal=False, seed=154), 0),
    "L2048_r8_d128_causal": (W("bwd_f", seq_len=2048, d_head=128, n_buckets=32, n_rounds=8,
                               seed=155), 0),
    "no_dup_L1344_r3": (W("bwd_g", heads=2, seq_len=1344, n_buckets=10, n_rounds=3, seed=156),
                        lsh.LSH_FLAG_NO_DUP_CORRECTION),
    # wrap-around look-back: 21 chunks (odd: chunk 0 and its look-back share a
    # parity) over two runs; two chunks; one chunk
    "wrap_L1344_r3_causal": (W("bwd_h", heads=2, seq_len=1344, n_buckets=10, n_rounds=3, seed=157),
                             lsh.LSH_FLAG_WRAP_LOOKBACK),
    "wrap_L2048_r4_d128_noncausal": (W("bwd_i", seq_len=2048, d_head=128, n_buckets=32, n_rounds=4,
                                       causal=False, seed=158), lsh.LSH_FLAG_WRAP_LOOKBACK),
    "wrap_no_dup_L128_two_chunks": (W("bwd_j", heads=2, seq_len=128, n_buckets=4, n_rounds=3,
                                      causal=False, seed=159),
                                    lsh.LSH_FLAG_WRAP_LOOKBACK | lsh.LSH_FLAG_NO_DUP_CORRECTION),
    "wrap_L64_one_chunk": (W("bwd_k", heads=2, seq_len=64, n_buckets=4, seed=160),
                           lsh.LSH_FLAG_WRAP_LOOKBACK),
    # runs of 2 and 3 chunks (ragged last run): key gradients carried across tiles
    "runs2_b2h8_L1344_r4": (W("bwd_n", batch=2, heads=8, seq_len=1344, n_buckets=10, n_rounds=4,
                              seed=163), 0),
    "runs3_b2h8_L4096_r3_d128": (W("bwd_o", batch=2, heads=8, seq_len=4096, d_head=128,
                                   n_buckets=32, n_rounds=3, causal=False, seed=164), 0),
    "runs2_wrap_b2h8_L1344_r4": (W("bwd_p", batch=2, heads=8, seq_len=1344, n_buckets=10,
                                   n_rounds=4, seed=165), lsh.LSH_FLAG_WRAP_LOOKBACK),
    "same_bucket_L1344_r3": (W("bwd_l", batch=2, heads=2, seq_len=1344, n_buckets=10, n_rounds=3,
                               seed=161), lsh.LSH_FLAG_SAME_BUCKET),
    "same_bucket_no_dup_L2048_d128": (W("bwd_m", seq_len=2048, d_head=128, n_buckets=16, n_rounds=4,
                                        causal=False, seed=162),
                                      lsh.LSH_FLAG_SAME_BUCKET | lsh.LSH_FLAG_NO_DUP_CORRECTION),
}


@pytest.mark.parametrize("name", sorted(BWD_CASES))
def test_backward_parity(name):
    w, flags = BWD_CASES[name]
    GP.backward_parity(w, flags)


def test_backward_sampled_paper_64k():
    """The 64K-token, 8-head, 8-round workload at full size, sampled positions."""
    GP.sampled_backward(WORKLOADS["paper_64k"], n_samples=4)


def test_backward_short_4k():
    """The 4K-token, 8-head workload (d 64, causal), every gradient."""
    GP.backward_parity(WORKLOADS["short_4k"])


def test_backward_sampled_clustered_16k():
    """The clustered workload (batch 2, d 64, non-causal, 4 rounds), sampled positions."""
    GP.sampled_backward(WORKLOADS["clustered_16k"], n_samples=4)


# ---------------------------------------------------------------------- Reformer block
FFN_CASES = {
    "rows600_dm192_dff320_chunk256": (600, 192, 320, 256, 1.0, 170, False),
    "rows1000_dm128_dff512_chunk333_minus": (1000, 128, 512, 333, -1.0, 171, False),
    "rows4096_dm1024_dff4096_chunk1024": (4096, 1024, 4096, 1024, 1.0, 172, False),
    "rows700_in_place_one_chunk": (700, 256, 256, 4096, -1.0, 173, True),
}


@pytest.mark.parametrize("name", sorted(FFN_CASES))
def test_ffn_parity(name):
    GP.ffn_parity(*FFN_CASES[name])


BLOCK_CASES = {
    "L512_dm128_dff256_h2_chunkrows200": (W("block_a", heads=2, seq_len=512, n_buckets=16, seed=180),
                                          128, 256, 200),
    "paper_shape_L2048_dm1024_dff4096": (W("block_b", heads=8, seq_len=2048, d_head=128,
                                           n_buckets=64, n_rounds=2, seed=181), 1024, 4096, 512),
}


@pytest.mark.parametrize("name", sorted(BLOCK_CASES))
def test_block_parity(name):
    GP.block_parity(*BLOCK_CASES[name])


# ---------------------------------------------------------------------- large GEMM launches
# Sizes that take the 256 x 256 tiles (at least 256 such tiles per launch), with
# a ragged last row tile (16448 = 64 x 257 rows), checked on sampled rows.
def test_projections_big_tiles_sampled():
    GP.projections_sampled(W("proj_big", heads=8, seq_len=16448, d_head=128, n_buckets=64,
                             seed=190), 1024)


def test_projections_big_tiles_d64_sampled():
    GP.projections_sampled(W("proj_big64", batch=2, heads=16, seq_len=8256, d_head=64,
                             n_buckets=64, seed=191), 1024)


def test_ffn_big_tiles_sampled():
    GP.ffn_sampled(16448, 1024, 4096, 16448, 192)


def test_ffn_big_tiles_chunked_sampled():
    GP.ffn_sampled(40000, 1024, 4096, 16384, 193)


# ---------------------------------------------------------------------- HIP graph replay
def test_forward_graph_replay():
    """The four calls captured into one HIP graph (torch.cuda.CUDAGraph), replayed
    three times with eager work in between: every replay equals the eager
    result bit for bit (the kernels are deterministic and allocate nothing)."""
    w = WORKLOADS["short_4k"]
    x = make_inputs(w)
    cfg = GP.cfg_of(w)
    dev = "cuda:0"
    t = GP.upload(w, x, dev)
    eager = lsh.forward(cfg, t["qk"], t["v"], t["R"], return_all=True)
    torch.cuda.synchronize()
    B, H, L, d, nr = w.batch, w.heads, w.seq_len, w.d_head, w.n_rounds
    out = {k: torch.empty_like(eager[k]) for k in ("buckets", "perm", "cid", "o_rounds", "lse", "o")}
    ws = lsh.sort_workspace(cfg, dev)
    s = torch.cuda.Stream(device=dev)

    def step():
        lsh.lsh_hash(cfg, t["qk"], t["R"], out["buckets"], stream=s)
        lsh.lsh_sort(cfg, out["buckets"], out["perm"], out["cid"], ws, stream=s)
        lsh.lsh_chunk_attn(cfg, t["qk"], t["v"], out["perm"], out["cid"], out["o_rounds"], out["lse"],
                           stream=s)
        lsh.lsh_combine_rounds(cfg, out["o_rounds"], out["lse"], out["o"], stream=s)

    with torch.cuda.stream(s):
        step()                                   # warm-up outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    for rep in range(3):
        for k in out:                            # eager work between replays
            out[k].zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in out:
            assert torch.equal(out[k], eager[k]), (rep, k)
