"""Parity of the HIP path (through the C ABI) against the CPU oracle.

Layered checks, so that one near-tie hash flip cannot fail the later steps:
  hash     GPU buckets equal the oracle's wherever the oracle's fp64 top-2
           margin exceeds 1e-4; every mismatch is a near-tie (counted).
  sort     GPU perm/cid equal the oracle's stable counting sort of the GPU's
           own buckets (bit-exact).  At full size: the properties that define
           that sort uniquely (permutation, keys non-decreasing, equal keys in
           position order, cid = slot // chunk).
  attend   GPU o_rounds/lse against the oracle's attention fed the GPU's
           perm/cid.
  combine  GPU o against the oracle's combine fed the GPU's o_rounds/lse.
  forward  GPU o against the oracle's forward from scratch (whole heads whose
           buckets all agree).
Error metric for float outputs: max|gpu - ref| / max|ref| over the tensor
(or over the sampled rows).  Gates: 1e-5 for float32, 2e-2 for bfloat16.
lse gate: |gpu - ref| <= LSE_ATOL + 1e-6 |ref|; 1e-6 relative covers the fp32
rounding of the self-penalised scores, which sit near -1e5 (ulp 2^-7).
"""
from __future__ import annotations

import math
import sys
import time
from typing import Dict

import numpy as np
import torch

import lsh_attention_02_amd as lsh
import oracle.lsh_oracle as O
from synthetic_inputs import Workload, make_block_inputs, make_grad, make_inputs, make_layer_inputs

GATE = {"f32": 1e-5, "bf16": 2e-2}
LSE_ATOL = {"f32": 2e-5, "bf16": 1e-3}
LSE_RTOL = 1e-6


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def cfg_of(w: Workload, scale=None, flags=0) -> lsh.LSHConfig:
    return lsh.LSHConfig(w.batch, w.heads, w.seq_len, w.d_head, w.n_buckets, w.n_rounds, w.chunk,
                         w.causal, dtype=w.dtype, scale=scale, flags=flags)


def variant(flags: int) -> dict:
    """The oracle's switches for the library's LSH_FLAG_* bits (the same-bucket
    variant also needs the buckets, passed separately)."""
    return {"dup_correct": not (flags & lsh.LSH_FLAG_NO_DUP_CORRECTION),
            "wrap": bool(flags & lsh.LSH_FLAG_WRAP_LOOKBACK)}


def same_bucket(flags: int) -> bool:
    return bool(flags & lsh.LSH_FLAG_SAME_BUCKET)


def window_ids(chunk_ids: np.ndarray, buckets: np.ndarray, n_buckets: int) -> np.ndarray:
    """What lsh_sort writes into cid with LSH_FLAG_SAME_BUCKET (the header's
    definition): chunk id + 2 * number of non-empty buckets below the position's
    bucket in that round.  chunk_ids [B, H, L, n_r], buckets [B, H, n_r, L]."""
    B, H, n_r, L = buckets.shape
    out = chunk_ids.astype(np.int64).copy()
    for b in range(B):
        for h in range(H):
            for r in range(n_r):
                nonempty = np.bincount(buckets[b, h, r], minlength=n_buckets) > 0
                rank = np.cumsum(nonempty) - nonempty
                out[b, h, :, r] += 2 * rank[buckets[b, h, r]]
    return out


def upload(w: Workload, x: Dict[str, np.ndarray], device="cuda:0"):
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    # the arrays hold values exactly representable in dt, so the conversion is exact
    return {k: torch.from_numpy(x[k]).to(device).to(dt).contiguous() for k in ("qk", "v", "R")}


def run_gpu(w: Workload, x, scale=None, device="cuda:0", flags=0):
    cfg = cfg_of(w, scale, flags)
    t = upload(w, x, device)
    out = lsh.forward(cfg, t["qk"], t["v"], t["R"], return_all=True)
    torch.cuda.synchronize()
    return cfg, t, out


def to_np(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy()


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    den = float(np.max(np.abs(ref)))
    return float(np.max(np.abs(got.astype(np.float64) - ref))) / max(den, 1e-300)


def check_lse(got: np.ndarray, ref: np.ndarray, dtype: str, what: str) -> float:
    err = np.abs(got.astype(np.float64) - ref)
    bound = LSE_ATOL[dtype] + LSE_RTOL * np.abs(ref)
    worst = float(np.max(err - bound))
    assert worst <= 0, f"{what}: lse off by up to {float(np.max(err)):.3g} (excess {worst:.3g})"
    return float(np.max(err))


def check_hash(gpu_b: np.ndarray, ref_b: np.ndarray, margins: np.ndarray, what: str) -> dict:
    mism = gpu_b != ref_b
    near = margins <= O.NEAR_TIE_MARGIN
    bad = mism & ~near
    assert not bad.any(), f"{what}: {int(bad.sum())} bucket mismatches with margin > 1e-4"
    assert np.all((gpu_b >= 0)), what
    return {"near_ties": int(near.sum()), "near_tie_mismatches": int(mism.sum()), "hashes": int(mism.size)}


def full_parity(w: Workload, scale=None, x=None, flags=0) -> dict:
    """Every output of every step against the oracle (small workloads)."""
    t0 = time.time()
    x = make_inputs(w) if x is None else x
    cfg, _, g = run_gpu(w, x, scale, flags=flags)
    var = variant(flags)
    sc = cfg.score_scale
    qk = x["qk"].astype(np.float64)
    v = x["v"].astype(np.float64)
    R = x["R"].astype(np.float64)
    gb = to_np(g["buckets"])
    rep = {"workload": w.name, "flags": flags}
    # hash
    ob, om = O.hash_buckets(qk, R)
    rep.update(check_hash(gb, ob, om, w.name))
    # sort of the GPU's own buckets
    sp, sc_id = O.sort_rounds(gb, w.n_buckets, w.chunk)
    assert np.array_equal(to_np(g["perm"]), sp), f"{w.name}: perm differs from the stable sort"
    gcid = to_np(g["cid"])
    if same_bucket(flags):
        assert np.array_equal(gcid.view(np.uint16), window_ids(sc_id, gb, w.n_buckets)), \
            f"{w.name}: window ids differ"
    else:
        assert np.array_equal(gcid, sc_id), f"{w.name}: cid differs"
    # attention fed the GPU's perm (and its buckets for the same-bucket mask)
    o_r, lse = O.attention_rounds(qk, v, sp, sc_id, w.chunk, w.causal, sc, **var,
                                  buckets=gb if same_bucket(flags) else None)
    rep["o_rounds_err"] = rel_err(to_np(g["o_rounds"]), o_r)
    assert rep["o_rounds_err"] <= GATE[w.dtype], (w.name, "o_rounds", rep["o_rounds_err"])
    rep["lse_abs_err"] = check_lse(to_np(g["lse"]), lse, w.dtype, w.name)
    # combine fed the GPU's o_rounds/lse
    oc, _ = O.combine_rounds(to_np(g["o_rounds"]).astype(np.float64), to_np(g["lse"]).astype(np.float64))
    rep["combine_err"] = rel_err(to_np(g["o"]), oc)
    assert rep["combine_err"] <= GATE[w.dtype], (w.name, "combine", rep["combine_err"])
    # forward from scratch, on the heads whose buckets agree everywhere.  There
    # the oracle's own sort equals the sort of the GPU's buckets (asserted), so
    # its attention is the one computed above and only the combine remains.
    same = np.all(gb == ob, axis=(2, 3))
    rep["heads_bucket_exact"] = f"{int(same.sum())}/{same.size}"
    if same.any():
        pf, cf = O.sort_rounds(ob, w.n_buckets, w.chunk)
        assert np.array_equal(pf[same], sp[same]) and np.array_equal(cf[same], sc_id[same])
        of, _ = O.combine_rounds(o_r, lse)
        go = to_np(g["o"])
        rep["forward_err"] = rel_err(go[same], of[same])
        assert rep["forward_err"] <= GATE[w.dtype], (w.name, "forward", rep["forward_err"])
    rep["rows_compared"] = {"o_rounds": int(np.prod(o_r.shape[:-1])), "o": int(np.prod(oc.shape[:-1])),
                            "o_from_scratch": int(same.sum()) * w.seq_len}
    rep["seconds"] = round(time.time() - t0, 1)
    log(f"[parity] {rep}")
    return rep


# --------------------------------------------------------------------------- full-size, sampled
def sort_properties(gb: np.ndarray, gp: np.ndarray, gc: np.ndarray, chunk: int, what: str,
                    n_buckets: int = 0, flags: int = 0) -> np.ndarray:
    """The properties that determine the stable sort uniquely, checked on every
    segment.  Returns the chunk ids [B, H, L, n_r] (slot // chunk)."""
    B, H, n_r, L = gb.shape
    b2 = gb.reshape(-1, L).astype(np.int64)
    p2 = gp.reshape(-1, L).astype(np.int64)
    assert np.array_equal(np.sort(p2, axis=1), np.broadcast_to(np.arange(L), p2.shape)), \
        f"{what}: perm is not a permutation"
    keys = np.take_along_axis(b2, p2, axis=1)
    dk = np.diff(keys, axis=1)
    assert np.all(dk >= 0), f"{what}: buckets not sorted"
    assert np.all((dk > 0) | (np.diff(p2, axis=1) > 0)), f"{what}: equal buckets out of position order"
    slot = np.empty_like(p2)
    np.put_along_axis(slot, p2, np.broadcast_to(np.arange(L), p2.shape), axis=1)
    want = (slot // chunk).reshape(B, H, n_r, L).transpose(0, 1, 3, 2)
    if same_bucket(flags):
        assert np.array_equal(gc.view(np.uint16), window_ids(want, gb, n_buckets)), \
            f"{what}: window ids differ"
    else:
        assert np.array_equal(gc.astype(np.int64), want), f"{what}: cid differs from slot // chunk"
    return want


def sampled_parity(w: Workload, n_samples: int = 1024, seed: int = 0, flags: int = 0,
                   slices=(), slice_hash: bool = True) -> dict:
    """Full-size workload: every sort output, sampled hashes, rows and tokens;
    then every row of the (batch row, head) slices listed (see slice_checks)."""
    t0 = time.time()
    log(f"[sampled] {w.name} flags {flags}: generating inputs")
    x = make_inputs(w)
    log(f"[sampled] {w.name}: running the GPU path ({time.time() - t0:.1f}s)")
    cfg, t, g = run_gpu(w, x, flags=flags)
    var = variant(flags)
    sc = cfg.score_scale
    B, H, L, d, n_r = w.batch, w.heads, w.seq_len, w.d_head, w.n_rounds
    rng = np.random.default_rng(seed)
    rep = {"workload": w.name, "flags": flags}
    gb = to_np(g["buckets"])
    gp = to_np(g["perm"])
    gc = to_np(g["cid"])
    log(f"[sampled] {w.name}: sort properties ({time.time() - t0:.1f}s)")
    chunk_ids = sort_properties(gb, gp, gc, w.chunk, w.name, w.n_buckets, flags)
    # sampled hashes
    sb, sh, sr, si = (rng.integers(0, B, n_samples), rng.integers(0, H, n_samples),
                      rng.integers(0, n_r, n_samples), rng.integers(0, L, n_samples))
    ob = np.empty(n_samples, np.int64)
    om = np.empty(n_samples)
    for s in range(n_samples):
        ob[s], om[s] = O.hash_one(x["qk"][sb[s], sh[s], si[s]].astype(np.float64),
                                  x["R"][sr[s]].astype(np.float64))
    rep.update(check_hash(gb[sb, sh, sr, si], ob, om, w.name))
    # sampled attention rows, fed the GPU's perm/cid
    log(f"[sampled] {w.name}: attention rows ({time.time() - t0:.1f}s)")
    idx = torch.from_numpy(np.stack([sb, sh, sr, si])).to(t["qk"].device)
    g_or = to_np(g["o_rounds"][idx[0], idx[1], idx[2], idx[3]])
    g_lse = to_np(g["lse"][idx[0], idx[1], idx[2], idx[3]])
    ref_o = np.empty((n_samples, d))
    ref_l = np.empty(n_samples)
    for s in range(n_samples):
        b, h = sb[s], sh[s]
        ref_o[s], ref_l[s] = O.attention_one(x["qk"][b, h], x["v"][b, h], gp[b, h],
                                             chunk_ids[b, h], int(sr[s]), int(si[s]), w.chunk,
                                             w.causal, sc, **var,
                                             buckets_bh=gb[b, h] if same_bucket(flags) else None)
    rep["o_rounds_err"] = rel_err(g_or, ref_o)
    assert rep["o_rounds_err"] <= GATE[w.dtype], (w.name, "o_rounds", rep["o_rounds_err"])
    rep["lse_abs_err"] = check_lse(g_lse, ref_l, w.dtype, w.name)
    # sampled combine, fed the GPU's o_rounds/lse
    tok = torch.from_numpy(np.stack([sb, sh, si])).to(t["qk"].device)
    g_o = to_np(g["o"][tok[0], tok[1], tok[2]])
    g_orall = to_np(g["o_rounds"][tok[0], tok[1], :, tok[2]])      # [S, n_r, d]
    g_lall = to_np(g["lse"][tok[0], tok[1], :, tok[2]])            # [S, n_r]
    oc, _ = O.combine_rounds(g_orall[:, :, None, :].astype(np.float64),
                             g_lall[:, :, None].astype(np.float64))
    rep["combine_err"] = rel_err(g_o, oc[:, 0])
    assert rep["combine_err"] <= GATE[w.dtype], (w.name, "combine", rep["combine_err"])
    rep["seconds"] = round(time.time() - t0, 1)
    log(f"[sampled] {rep}")
    for b, h in slices:
        rep[f"slice_b{b}_h{h}"] = slice_checks(w, x, g, b, h, flags, slice_hash, sc, t0)
    return rep


def slice_checks(w: Workload, x, g, b: int, h: int, flags: int, with_hash: bool, sc: float,
                 t0: float) -> dict:
    """Every row of one (batch row, head) of a full-size run: its hashes in every
    round (with_hash), its perm/cid bit-exact against the oracle's stable sort
    of the GPU's buckets, every o_rounds row and lse fed the GPU's perm/cid,
    every combined row fed the GPU's o_rounds/lse, and the forward from scratch
    when all the slice's hashes agree with the oracle's."""
    var = variant(flags)
    rep = {}
    sl = (slice(b, b + 1), slice(h, h + 1))
    gb = to_np(g["buckets"][sl])
    qk = x["qk"][sl].astype(np.float64)
    v = x["v"][sl].astype(np.float64)
    ob = None
    if with_hash:
        log(f"[slice] {w.name} b {b} h {h}: hashes of {w.n_rounds} x {w.seq_len} ({time.time() - t0:.1f}s)")
        ob, om = O.hash_buckets(qk, x["R"].astype(np.float64))
        rep.update(check_hash(gb, ob, om, f"{w.name} slice"))
    log(f"[slice] {w.name} b {b} h {h}: sort ({time.time() - t0:.1f}s)")
    sp, sc_id = O.sort_rounds(gb, w.n_buckets, w.chunk)
    assert np.array_equal(to_np(g["perm"][sl]), sp), f"{w.name} slice: perm differs from the stable sort"
    gcid = to_np(g["cid"][sl])
    if same_bucket(flags):
        assert np.array_equal(gcid.view(np.uint16), window_ids(sc_id, gb, w.n_buckets))
    else:
        assert np.array_equal(gcid, sc_id), f"{w.name} slice: cid differs"
    log(f"[slice] {w.name} b {b} h {h}: attention, {w.n_rounds} rounds x {w.seq_len // w.chunk} "
        f"chunks ({time.time() - t0:.1f}s)")
    o_r, lse = O.attention_rounds(qk, v, sp, sc_id, w.chunk, w.causal, sc, **var,
                                  buckets=gb if same_bucket(flags) else None)
    g_or = to_np(g["o_rounds"][sl])
    g_lse = to_np(g["lse"][sl])
    rep["o_rounds_err"] = rel_err(g_or, o_r)
    assert rep["o_rounds_err"] <= GATE[w.dtype], (w.name, "slice o_rounds", rep["o_rounds_err"])
    rep["lse_abs_err"] = check_lse(g_lse, lse, w.dtype, f"{w.name} slice")
    oc, _ = O.combine_rounds(g_or.astype(np.float64), g_lse.astype(np.float64))
    go = to_np(g["o"][sl])
    rep["combine_err"] = rel_err(go, oc)
    assert rep["combine_err"] <= GATE[w.dtype], (w.name, "slice combine", rep["combine_err"])
    rep["rows_compared"] = {"o_rounds": w.n_rounds * w.seq_len, "o": w.seq_len}
    if ob is not None and np.array_equal(ob, gb):
        # the oracle's own sort of identical buckets is the one above
        of, _ = O.combine_rounds(o_r, lse)
        rep["forward_err"] = rel_err(go, of)
        assert rep["forward_err"] <= GATE[w.dtype], (w.name, "slice forward", rep["forward_err"])
        rep["rows_compared"]["o_from_scratch"] = w.seq_len
    log(f"[slice] {w.name} b {b} h {h}: {rep} ({time.time() - t0:.1f}s)")
    return rep


# --------------------------------------------------------------------------- the layer
GATE_PROJ = 1e-2     # bf16 outputs of fp32-accumulated products: rounding 2^-9 relative


def layer_parity(w: Workload, d_model: int, flags: int = 0) -> dict:
    """Layered: the GPU's projections against the oracle's on the same bf16
    inputs; the four steps on the GPU's qk and v (as in full_parity); the
    output projection of the GPU's o."""
    t0 = time.time()
    x = make_layer_inputs(w, d_model)
    dev = "cuda:0"
    t = {k: torch.from_numpy(a).to(dev).to(torch.bfloat16).contiguous() for k, a in x.items()}
    cfg = cfg_of(w, flags=flags)
    g = lsh.layer_forward(cfg, t["x"], t["w_qk"], t["w_v"], t["w_o"], t["R"], return_all=True)
    torch.cuda.synchronize()
    rep = {"workload": w.name, "d_model": d_model, "flags": flags}
    qk_ref, v_ref = O.project_in(x["x"], x["w_qk"], x["w_v"], w.heads)
    rep["qk_err"] = rel_err(to_np(g["qk"]), qk_ref)
    rep["v_err"] = rel_err(to_np(g["v"]), v_ref)
    assert rep["qk_err"] <= GATE_PROJ and rep["v_err"] <= GATE_PROJ, rep
    core = full_parity(w, x={"qk": to_np(g["qk"]), "v": to_np(g["v"]), "R": x["R"]}, flags=flags)
    rep["core_o_rounds_err"] = core["o_rounds_err"]
    y_ref = O.project_out(to_np(g["o"]).astype(np.float64), x["w_o"])
    rep["y_err"] = rel_err(to_np(g["y"]), y_ref)
    assert rep["y_err"] <= GATE_PROJ, rep
    rep["seconds"] = round(time.time() - t0, 1)
    log(f"[layer] {rep}")
    return rep


# --------------------------------------------------------------------------- backward
# d_qk and d_v are float32 sums of bf16-rounded partial products (P and dS are
# rounded to bf16 for the MFMA operands, each round's partial gradient is stored
# in bf16): the error is a few 2^-9 relative, so the bf16 gate applies.
GATE_BWD = GATE["bf16"]


def run_backward(w: Workload, x, d_o: np.ndarray, flags: int = 0, device="cuda:0"):
    cfg, t, g = run_gpu(w, x, flags=flags, device=device)
    do_t = torch.from_numpy(d_o).to(device).to(cfg.torch_dtype).contiguous()
    dqk, dv = lsh.lsh_attn_backward(cfg, t["qk"], t["v"], g["perm"], g["cid"], g["lse"], g["o"], do_t)
    torch.cuda.synchronize()
    return cfg, g, dqk, dv


def backward_parity(w: Workload, flags: int = 0) -> dict:
    """GPU d_qk, d_v against the oracle's backward fed the GPU's perm/cid (the
    sort itself is checked bit-exact in full_parity)."""
    t0 = time.time()
    x = make_inputs(w)
    d_o = make_grad(w)
    cfg, g, dqk, dv = run_backward(w, x, d_o, flags)
    gb = to_np(g["buckets"])
    sp, sc_id = O.sort_rounds(gb, w.n_buckets, w.chunk)
    assert np.array_equal(to_np(g["perm"]), sp), f"{w.name}: perm differs from the stable sort"
    ref = O.attention_backward(x["qk"].astype(np.float64), x["v"].astype(np.float64), sp, sc_id,
                               d_o.astype(np.float64), w.chunk, w.causal, cfg.score_scale,
                               **variant(flags), buckets=gb if same_bucket(flags) else None)
    rep = {"workload": w.name, "flags": flags}
    rep["dqk_err"] = rel_err(to_np(dqk), ref["dqk"])
    rep["dv_err"] = rel_err(to_np(dv), ref["dv"])
    assert rep["dqk_err"] <= GATE_BWD and rep["dv_err"] <= GATE_BWD, rep
    assert np.isfinite(to_np(dqk)).all() and np.isfinite(to_np(dv)).all()
    rep["seconds"] = round(time.time() - t0, 1)
    log(f"[backward] {rep}")
    return rep


def sampled_backward(w: Workload, n_samples: int = 6, seed: int = 0) -> dict:
    """Full-size workload: d_qk and d_v at sampled positions against the oracle's
    single-position gradients (fed the GPU's perm/cid, which sampled_parity
    checks against the sort's defining properties)."""
    t0 = time.time()
    log(f"[sampled-backward] {w.name}: generating inputs")
    x = make_inputs(w)
    d_o = make_grad(w)
    cfg, g, dqk, dv = run_backward(w, x, d_o)
    gp = to_np(g["perm"])
    gc = to_np(g["cid"])
    rng = np.random.default_rng(seed)
    B, H, L = w.batch, w.heads, w.seq_len
    sb, sh, si = rng.integers(0, B, n_samples), rng.integers(0, H, n_samples), rng.integers(0, L, n_samples)
    got_q = to_np(dqk[torch.from_numpy(sb), torch.from_numpy(sh), torch.from_numpy(si)])
    got_v = to_np(dv[torch.from_numpy(sb), torch.from_numpy(sh), torch.from_numpy(si)])
    ref_q = np.empty_like(got_q, dtype=np.float64)
    ref_v = np.empty_like(got_v, dtype=np.float64)
    for s in range(n_samples):
        b, h = sb[s], sh[s]
        log(f"[sampled-backward] sample {s}: b {b} h {h} pos {si[s]} ({time.time() - t0:.1f}s)")
        ref_q[s], ref_v[s] = O.attention_backward_one(
            x["qk"][b, h].astype(np.float64), x["v"][b, h].astype(np.float64),
            d_o[b, h].astype(np.float64), gp[b, h], gc[b, h], int(si[s]), w.chunk, w.causal,
            cfg.score_scale)
    rep = {"workload": w.name, "samples": n_samples}
    rep["dqk_err"] = rel_err(got_q, ref_q)
    rep["dv_err"] = rel_err(got_v, ref_v)
    assert rep["dqk_err"] <= GATE_BWD and rep["dv_err"] <= GATE_BWD, rep
    rep["seconds"] = round(time.time() - t0, 1)
    log(f"[sampled-backward] {rep}")
    return rep


# --------------------------------------------------------------------------- Reformer block
def ffn_parity(rows: int, d_model: int, d_ff: int, chunk_rows: int, sign: float, seed: int,
               in_place: bool = False) -> dict:
    """lsh_ffn against the oracle's feed-forward of the same bf16 inputs."""
    rng = np.random.default_rng(seed)
    bf = lambda a: torch.from_numpy(a.astype(np.float32)).to("cuda:0").to(torch.bfloat16).contiguous()
    x = bf(rng.standard_normal((rows, d_model)))
    w1 = bf(rng.standard_normal((d_ff, d_model)) / np.sqrt(d_model))
    b1 = bf(rng.standard_normal(d_ff) * 0.1)
    w2 = bf(rng.standard_normal((d_model, d_ff)) / np.sqrt(d_ff))
    b2 = bf(rng.standard_normal(d_model) * 0.1)
    res = bf(rng.standard_normal((rows, d_model)))
    res0 = to_np(res).astype(np.float64)
    y = lsh.lsh_ffn(x, w1, b1, w2, b2, res, sign, chunk_rows, y=res if in_place else None)
    torch.cuda.synchronize()
    ref = res0 + sign * O.feed_forward(to_np(x), to_np(w1), to_np(b1), to_np(w2), to_np(b2))
    rep = {"rows": rows, "d_model": d_model, "d_ff": d_ff, "chunk_rows": chunk_rows, "sign": sign,
           "in_place": in_place, "err": rel_err(to_np(y), ref)}
    assert rep["err"] <= GATE_PROJ, rep
    log(f"[ffn] {rep}")
    return rep


def block_parity(w: Workload, d_model: int, d_ff: int, chunk_rows: int) -> dict:
    """Layered: the block's forward halves against the oracle fed the GPU's
    intermediates, then the inverse likewise; the round trip x2 -> y2 -> x2 is
    exact up to bf16 rounding (no hashing on that path)."""
    t0 = time.time()
    x = make_block_inputs(w, d_model, d_ff)
    dev = "cuda:0"
    t = {k: torch.from_numpy(a).to(dev).to(torch.bfloat16).contiguous() for k, a in x.items()}
    cfg = cfg_of(w)
    wa = {k: t[k] for k in ("w_qk", "w_v", "w_o")}
    wf = {k: t[k] for k in ("w1", "b1", "w2", "b2")}
    f64 = lambda k: x[k].astype(np.float64)
    y1, y2 = lsh.block_forward(cfg, t["x1"], t["x2"], wa, wf, t["R"], chunk_rows)
    # the attention half: the GPU's own attention output of x2 (checked against
    # the oracle by the layer tests), projected and added by the oracle
    att = lsh.layer_forward(cfg, t["x2"], wa["w_qk"], wa["w_v"], wa["w_o"], t["R"], return_all=True)
    torch.cuda.synchronize()
    rep = {"workload": w.name, "d_model": d_model, "d_ff": d_ff, "chunk_rows": chunk_rows}
    ref1 = f64("x1") + O.project_out(to_np(att["o"]).astype(np.float64), f64("w_o"))
    rep["y1_err"] = rel_err(to_np(y1), ref1)
    ref2 = f64("x2") + O.feed_forward_chunked(to_np(y1), f64("w1"), f64("b1"), f64("w2"), f64("b2"),
                                              chunk_rows)
    rep["y2_err"] = rel_err(to_np(y2), ref2)
    assert rep["y1_err"] <= GATE_PROJ and rep["y2_err"] <= GATE_PROJ, rep
    # inverse, out of place and in place
    r1, r2 = lsh.block_inverse(cfg, y1, y2, wa, wf, t["R"], chunk_rows)
    att2 = lsh.layer_forward(cfg, r2, wa["w_qk"], wa["w_v"], wa["w_o"], t["R"], return_all=True)
    torch.cuda.synchronize()
    ref_r2 = to_np(y2).astype(np.float64) - O.feed_forward(to_np(y1), f64("w1"), f64("b1"), f64("w2"),
                                                           f64("b2"))
    rep["x2_inverse_err"] = rel_err(to_np(r2), ref_r2)
    ref_r1 = to_np(y1).astype(np.float64) - O.project_out(to_np(att2["o"]).astype(np.float64), f64("w_o"))
    rep["x1_inverse_err"] = rel_err(to_np(r1), ref_r1)
    assert rep["x2_inverse_err"] <= GATE_PROJ and rep["x1_inverse_err"] <= GATE_PROJ, rep
    rep["x2_round_trip_err"] = rel_err(to_np(r2), f64("x2"))
    assert rep["x2_round_trip_err"] <= GATE_PROJ, rep
    d1 = np.abs(to_np(r1).astype(np.float64) - f64("x1"))
    rep["x1_round_trip_median_err"] = float(np.median(d1) / np.max(np.abs(f64("x1"))))
    ip1, ip2 = y1.clone(), y2.clone()
    lsh.block_inverse(cfg, ip1, ip2, wa, wf, t["R"], chunk_rows, in_place=True)
    torch.cuda.synchronize()
    assert torch.equal(ip2, r2), "in-place inverse differs (x2)"
    assert torch.equal(ip1, r1), "in-place inverse differs (x1)"
    rep["seconds"] = round(time.time() - t0, 1)
    log(f"[block] {rep}")
    return rep


# --------------------------------------------------------------------------- large GEMM launches
def _sample_rows(n_rows: int, n: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    rows = rng.choice(n_rows, size=min(n, n_rows), replace=False)
    return np.sort(np.concatenate([rows, [0, n_rows - 1]]).astype(np.int64))


def projections_sampled(w: Workload, d_model: int, n_samples: int = 96) -> dict:
    """lsh_project_in / lsh_project_out / lsh_project_out_add at sizes that take the
    256 x 256 tiles, against the oracle on sampled rows (b, i)."""
    x = make_layer_inputs(w, d_model)
    dev = "cuda:0"
    t = {k: torch.from_numpy(a).to(dev).to(torch.bfloat16).contiguous() for k, a in x.items()}
    cfg = cfg_of(w)
    B, H, L, d = w.batch, w.heads, w.seq_len, w.d_head
    qk, v = lsh.lsh_project_in(cfg, d_model, t["x"], t["w_qk"], t["w_v"])
    rng = np.random.default_rng(7)
    o = torch.from_numpy(rng.standard_normal((B, H, L, d)).astype(np.float32)).to(dev).to(torch.bfloat16)
    res = torch.from_numpy(rng.standard_normal((B, L, d_model)).astype(np.float32)).to(dev).to(torch.bfloat16)
    y = lsh.lsh_project_out(cfg, d_model, o, t["w_o"])
    ya = lsh.lsh_project_out_add(cfg, d_model, o, t["w_o"], res, -1.0)
    torch.cuda.synchronize()
    rows = _sample_rows(B * L, n_samples, 11)
    bi, ii = rows // L, rows % L
    xs = x["x"][bi, ii].astype(np.float64)                                 # [S, d_model]
    ref_qk = (xs @ x["w_qk"].astype(np.float64).T).reshape(len(rows), H, d)
    ref_v = (xs @ x["w_v"].astype(np.float64).T).reshape(len(rows), H, d)
    got_qk = to_np(qk)[bi, :, ii]                                          # [S, H, d]
    got_v = to_np(v)[bi, :, ii]
    on = to_np(o)[bi, :, ii].reshape(len(rows), H * d).astype(np.float64)  # merge_heads of the rows
    ref_y = on @ x["w_o"].astype(np.float64).T
    ref_ya = to_np(res)[bi, ii].astype(np.float64) - ref_y
    rep = {"workload": w.name, "d_model": d_model, "rows": B * L,
           "qk_err": rel_err(got_qk, ref_qk), "v_err": rel_err(got_v, ref_v),
           "y_err": rel_err(to_np(y)[bi, ii], ref_y), "y_add_err": rel_err(to_np(ya)[bi, ii], ref_ya)}
    assert max(rep["qk_err"], rep["v_err"], rep["y_err"], rep["y_add_err"]) <= GATE_PROJ, rep
    log(f"[projections-sampled] {rep}")
    return rep


def ffn_sampled(rows: int, d_model: int, d_ff: int, chunk_rows: int, seed: int,
                n_samples: int = 96) -> dict:
    """lsh_ffn at sizes that take the 256 x 256 tiles, against the oracle on
    sampled rows."""
    rng = np.random.default_rng(seed)
    bf = lambda a: torch.from_numpy(a.astype(np.float32)).to("cuda:0").to(torch.bfloat16).contiguous()
    x = bf(rng.standard_normal((rows, d_model)))
    w1 = bf(rng.standard_normal((d_ff, d_model)) / np.sqrt(d_model))
    b1 = bf(rng.standard_normal(d_ff) * 0.1)
    w2 = bf(rng.standard_normal((d_model, d_ff)) / np.sqrt(d_ff))
    b2 = bf(rng.standard_normal(d_model) * 0.1)
    res = bf(rng.standard_normal((rows, d_model)))
    y = lsh.lsh_ffn(x, w1, b1, w2, b2, res, 1.0, chunk_rows)
    torch.cuda.synchronize()
    sel = _sample_rows(rows, n_samples, seed)
    ref = to_np(res)[sel].astype(np.float64) + O.feed_forward(to_np(x)[sel], to_np(w1), to_np(b1),
                                                              to_np(w2), to_np(b2))
    rep = {"rows": rows, "d_model": d_model, "d_ff": d_ff, "chunk_rows": chunk_rows,
           "err": rel_err(to_np(y)[sel], ref)}
    assert rep["err"] <= GATE_PROJ, rep
    log(f"[ffn-sampled] {rep}")
    return rep
