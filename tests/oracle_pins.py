"""Checks that pin the CPU oracle to facts outside itself.

Each check is a plain function that raises AssertionError on failure, so that
the mutation tests can plant a mistake in the oracle (on the CPU) and confirm
that some check catches it.  The oracle is always reached through the module
attribute ``O`` so that a monkeypatched function is the one that runs.

What pins what:
  hash   - the worked hashing example of the Ultralytics "Reformer" page
           (section on LSH attention): printed cosines and same-bucket shares;
         - bucket labels on axis-aligned inputs (x along column k of R lands in
           bucket k, -x in bucket k + n_buckets/2; exact ties go to the first
           index of [p, -p]);
         - the near-tie margin (top-1 minus top-2 of [p, -p]) on hand-built
           projections with known gaps: runner-up in either half, winner in
           the negated half, exact ties (margin 0), one column;
         - antipodal identity h(-x) = (h(x) + n_buckets/2) mod n_buckets;
         - scale invariance h(2^k x) = h(x);
         - with 2 buckets, the collision rate over random R is 1 - angle/pi
           (Charikar's SimHash; textbook, not on the pages).
  sort   - equals the library's stable sort (np.lexsort); chunk ids agree with
           the permutation.
  attend - one chunk spanning the sequence gives textbook full attention with
  +combine the self-mask (any bucket count, any number of rounds);
         - union brute force on L <= 64: the combined output equals plain
           softmax attention over the union of the rounds' windows;
         - constant values give constant outputs; one-hot values expose the
           weights (non-negative, sum 1, zero outside the round's window, zero
           on the query itself when it has company);
         - causal: position 0 returns its own value exactly;
         - combine: one round is the identity; equal lse gives the mean.
  variants - wrap-around look-back: union brute force with circular chunk
           distance; two chunks give full attention (without wrap they would
           not);
         - no duplicate correction: each round equals plain softmax over its
           brute-force window (o and lse); with one round the correction is
           a no-op;
         - same-bucket mask: union brute force and per-round brute force with
           windows restricted to the query's bucket.
  backward - the gradients of steps 3-4 against central finite differences of
           the oracle's own forward (fixed buckets), and against torch autograd
           of the union closed form (independent code); sum_j dv_j = sum_i d_o_i
           (the combined weights of each query sum to one).
  block  - the feed-forward layer against Python loops over its definition;
           chunking over positions (any chunk size, ragged last chunk) changes
           nothing; the reversible block's inverse recovers its inputs (round
           trip); zero output weights make the block the identity.
  layer  - both projections against Python loops over their definitions;
         - identity weights reduce the layer to the four steps on the input's
           head slices; permuting heads consistently changes nothing.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

import oracle.lsh_oracle as O
import reference_forms as RF
from synthetic_inputs import Workload, make_inputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# A round whose window holds only the query has lse near -SELF_PENALTY (1e5);
# the combine takes differences of such numbers, whose ulp is 1.5e-11, so the
# combined output is exact only to ~1e-10 on those rows.  Every other row is
# exact to ~1e-15.  A planted mistake moves outputs by far more than this.
TOL_COMBINED = 1e-9


def small_case(L=48, d=8, nb=6, n_r=3, chunk=8, causal=False, seed=11, dtype="f32"):
    w = Workload("pin", batch=1, heads=1, seq_len=L, d_head=d, dtype=dtype, n_buckets=nb,
                 n_rounds=n_r, chunk=chunk, causal=causal, seed=seed)
    x = make_inputs(w)
    return w, x["qk"].astype(np.float64), x["v"].astype(np.float64), x["R"].astype(np.float64)


# --------------------------------------------------------------------------- hash
def _draw_recipe(rc):
    """The named draws of a fixture recipe, in order, from torch's CPU generator
    (seeded 0): each is a standard-normal tensor of the listed shape, optionally
    scaled and added to an earlier draw.  Shapes name the recipe's sizes; "x/2"
    is half of size x."""
    import torch  # only to reproduce the page's random draws (CPU generator)

    def dim(s):
        name, _, div = s.partition("/")
        return rc["sizes"][name] // int(div or 1)

    out = {}
    state = torch.random.get_rng_state()
    try:
        torch.manual_seed(0)
        for dr in rc["draws"]:
            z = torch.randn(*[dim(s) for s in dr["shape"]]).numpy().astype(np.float64)
            if "scaled_by" in dr:
                # float32 arithmetic, as the draws themselves
                z = (np.float32(dr["scaled_by"]) * z.astype(np.float32)).astype(np.float64)
            if "added_to" in dr:
                z = (out[dr["added_to"]].astype(np.float32) + z.astype(np.float32)).astype(np.float64)
            out[dr["name"]] = z
    finally:
        torch.random.set_rng_state(state)
    return out


def check_hash_demo():
    """The Ultralytics page's hashing example: cosines and same-bucket shares of
    two vectors against a reference, over many rounds of random R."""
    with open(os.path.join(GOLDEN, "hash_demo.json")) as f:
        g = json.load(f)
    rc = g["recipe"]
    vals = _draw_recipe(rc)
    R = vals[rc["projection"]]
    ref = vals[rc["reference"]]
    ref_b = O.hash_buckets(ref[None, None, None, :], R)[0][0, 0, :, 0]
    for name in rc["compared"]:
        x = vals[name]
        xb = O.hash_buckets(x[None, None, None, :], R)[0][0, 0, :, 0]
        cos = float(ref @ x / (np.linalg.norm(ref) * np.linalg.norm(x)))
        # The page averages in single precision: 85/1000 is then 0.0850000009
        # and prints as 9%, where the double 0.085 would print 8%.
        share = float(np.float32(np.count_nonzero(xb == ref_b)) / np.float32(len(R)))
        got = {"cosine": f"{cos:.2f}", "same_bucket_percent": f"{share:.0%}"}
        assert got == g["printed"][name], (name, got, g["printed"][name])


def check_hash_labels():
    d, nb = 16, 12
    half = nb // 2
    R = np.zeros((d, half))
    R[np.arange(half), np.arange(half)] = 1.0         # p = x[:half] exactly
    for k in range(half):
        e = np.zeros(d)
        e[k] = 2.5
        assert O.hash_one(e, R)[0] == k
        assert O.hash_one(-e, R)[0] == k + half
    x = np.zeros(d)
    x[1], x[3] = 1.0, 1.0                              # exact tie between columns 1 and 3
    assert O.hash_one(x, R)[0] == 1
    x = np.zeros(d)
    x[1], x[3] = -1.0, 1.0                             # [p,-p] ties at index 3 and half+1
    assert O.hash_one(x, R)[0] == 3
    assert O.hash_one(np.zeros(d), R) == (0, 0.0)      # zero vector: bucket 0, margin 0


def check_hash_margin():
    """The near-tie margin: the gap between the largest and second-largest
    entries of [p, -p], on hand-built projections whose top two are known.
    Runner-up in the same half, runner-up in the negated half, the winner in
    the negated half, exact ties across and within halves (margin 0), and one
    column (n_buckets = 2, where the runner-up is the winner's own negation)."""
    cases = [
        # p                       bucket  margin
        ([1.0, 4.0, 3.5],           1,    0.5),    # runner-up p[2], same half
        ([3.0, 1.0, -2.5],          0,    0.5),    # runner-up -p[2], negated half
        ([-5.0, 1.0, 4.75],         3,    0.25),   # winner -p[0]; runner-up p[2]
        ([0.5, -6.0, 2.0, 5.0],     5,    1.0),    # winner -p[1]; runner-up p[3]
        ([2.0, -2.0],               0,    0.0),    # p[0] ties -p[1]: first index
        ([-1.0, 3.0, -3.0],         1,    0.0),    # p[1] ties -p[2]
        ([1.5, 1.5, -0.25],         0,    0.0),    # p[0] ties p[1], same half
        ([0.7],                     0,    1.4),    # one column: runner-up is -p[0]
        ([-0.2],                    1,    0.4),
        ([0.0, 0.0, 0.0],           0,    0.0),    # zero projection
    ]
    for p, bucket, margin in cases:
        b, m = O.bucket_from_projection(np.array([p]))
        assert int(b[0]) == bucket, (p, int(b[0]), bucket)
        assert abs(float(m[0]) - margin) < 1e-15, (p, float(m[0]), margin)
    # through the projection: R's columns pick coordinates of x, so p = x[:3]
    # exactly, and the margin is in projection units (linear in x)
    d = 8
    R = np.zeros((d, 3))
    R[np.arange(3), np.arange(3)] = 1.0
    x = np.zeros(d)
    x[:3] = [3.0, 1.0, -2.5]
    x[5] = 9.0                                        # outside R's columns: no effect
    for k in (1.0, 2.0, 0.125):
        assert O.hash_one(k * x, R) == (0, 0.5 * k)
    assert O.hash_one(-x, R) == (3, 0.5)


def check_hash_antipodal(seed=5):
    rng = np.random.default_rng(seed)
    for d, nb in ((64, 16), (128, 64), (8, 2), (16, 10)):
        x = rng.standard_normal((500, d))
        R = rng.standard_normal((d, nb // 2))
        b1, m1 = O.bucket_from_projection(O.project(x, R))
        b2, _ = O.bucket_from_projection(O.project(-x, R))
        ok = m1 > 0
        assert ok.mean() > 0.99
        assert np.array_equal(b2[ok], (b1[ok] + nb // 2) % nb)


def check_hash_scale_invariance(seed=6):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((400, 32))
    R = rng.standard_normal((32, 24))
    b0, _ = O.bucket_from_projection(O.project(x, R))
    for k in (-3, 1, 7):
        bk, _ = O.bucket_from_projection(O.project(x * 2.0 ** k, R))
        assert np.array_equal(bk, b0)


def check_simhash_rate(seed=7, rounds=20000):
    """n_buckets = 2: P[h(x) = h(y)] = 1 - angle(x, y)/pi over random R."""
    rng = np.random.default_rng(seed)
    d = 16
    R = rng.standard_normal((rounds, d, 1))
    x = rng.standard_normal(d)
    for target in (0.3, 1.2, 2.5):
        u = rng.standard_normal(d)
        u -= (u @ x) / (x @ x) * x
        u *= np.linalg.norm(x) / np.linalg.norm(u)
        y = math.cos(target) * x + math.sin(target) * u
        theta = math.acos(float(x @ y / (np.linalg.norm(x) * np.linalg.norm(y))))
        hx = np.array([O.hash_one(x, R[r])[0] for r in range(rounds)])
        hy = np.array([O.hash_one(y, R[r])[0] for r in range(rounds)])
        p = 1 - theta / math.pi
        rate = float(np.mean(hx == hy))
        sigma = math.sqrt(p * (1 - p) / rounds)
        assert abs(rate - p) < 5 * sigma, (theta, rate, p)


# --------------------------------------------------------------------------- sort
def check_sort_matches_library(seed=8):
    rng = np.random.default_rng(seed)
    cases = [rng.integers(0, 7, 1000), rng.integers(0, 1024, 5000), np.zeros(300, int),
             np.arange(200)[::-1].copy(), np.array([3]), rng.integers(0, 2, 64)]
    for keys in cases:
        nk = int(keys.max()) + 1
        got = O.stable_counting_sort(keys, nk)
        want = np.lexsort((np.arange(keys.size), keys))
        assert np.array_equal(got, want)


def check_sort_rounds_cid(seed=9):
    rng = np.random.default_rng(seed)
    B, H, n_r, L, nb, c = 2, 2, 3, 96, 10, 16
    buckets = rng.integers(0, nb, (B, H, n_r, L)).astype(np.int32)
    perm, cid = O.sort_rounds(buckets, nb, c)
    for b in range(B):
        for h in range(H):
            for r in range(n_r):
                want = np.lexsort((np.arange(L), buckets[b, h, r]))
                assert np.array_equal(perm[b, h, r], want)
                slots = np.arange(L)
                assert np.array_equal(cid[b, h, perm[b, h, r], r], slots // c)


# --------------------------------------------------------------------------- attention + combine
def _forward(w, qk, v, R, scale=None, **kw):
    out = O.forward(qk[None, None] if qk.ndim == 2 else qk, v[None, None] if v.ndim == 2 else v,
                    R, w.n_buckets, w.chunk, w.causal, scale=scale, **kw)
    return out


def check_full_attention(L=40, d=8, nb=6, n_r=3, causal=False, scale=None, seed=12):
    w, qk, v, R = small_case(L=L, d=d, nb=nb, n_r=n_r, chunk=L, causal=causal, seed=seed)
    sc = (1.0 / math.sqrt(d)) if scale is None else scale
    out = _forward(w, qk[0, 0], v[0, 0], R, scale=scale)
    ref = RF.full_attention_self_masked(qk[0, 0], v[0, 0], causal, sc)
    err = np.max(np.abs(out["o"][0, 0] - ref))
    assert err < TOL_COMBINED, err


def check_union(L=48, d=8, nb=6, n_r=3, chunk=8, causal=False, seed=13, dup_correct=True,
                wrap=False, same_bucket=False):
    w, qk, v, R = small_case(L=L, d=d, nb=nb, n_r=n_r, chunk=chunk, causal=causal, seed=seed)
    out = _forward(w, qk[0, 0], v[0, 0], R, dup_correct=dup_correct, wrap=wrap,
                   same_bucket=same_bucket)
    ref = RF.union_attention(qk[0, 0], v[0, 0], out["buckets"][0, 0], chunk, causal,
                             1.0 / math.sqrt(d), wrap=wrap, same_bucket=same_bucket)
    err = np.max(np.abs(out["o"][0, 0] - ref))
    assert err < TOL_COMBINED, err


def check_wrap_two_chunks(L=40, d=8, nb=6, n_r=3, causal=False, seed=18):
    """With wrap-around and two chunks, both chunks see the whole sequence in
    every round, so the forward is textbook full attention with the self-mask;
    without wrap the first chunk would see only itself."""
    w, qk, v, R = small_case(L=L, d=d, nb=nb, n_r=n_r, chunk=L // 2, causal=causal, seed=seed)
    out = _forward(w, qk[0, 0], v[0, 0], R, wrap=True)
    ref = RF.full_attention_self_masked(qk[0, 0], v[0, 0], causal, 1.0 / math.sqrt(d))
    err = np.max(np.abs(out["o"][0, 0] - ref))
    assert err < TOL_COMBINED, err


def check_rounds_without_correction(L=48, d=8, nb=6, n_r=3, chunk=8, causal=True, seed=19,
                                    wrap=False, same_bucket=False):
    """Without the duplicate-count term every round is plain softmax attention
    over that round's window (o_rounds and lse, round by round)."""
    w, qk, v, R = small_case(L=L, d=d, nb=nb, n_r=n_r, chunk=chunk, causal=causal, seed=seed)
    out = _forward(w, qk[0, 0], v[0, 0], R, dup_correct=False, wrap=wrap, same_bucket=same_bucket)
    W = RF.brute_windows(out["buckets"][0, 0], chunk, causal, wrap, same_bucket)
    for r in range(n_r):
        o, lse = RF.round_attention(qk[0, 0], v[0, 0], W[r], 1.0 / math.sqrt(d))
        assert np.max(np.abs(out["o_rounds"][0, 0, r] - o)) < 1e-12
        assert np.max(np.abs(out["lse"][0, 0, r] - lse) / np.maximum(1.0, np.abs(lse))) < 1e-13


def check_single_round_correction_free(seed=20):
    """With one round every duplicate count is 1, so the correction changes nothing."""
    w, qk, v, R = small_case(L=48, d=8, nb=6, n_r=1, chunk=8, causal=True, seed=seed)
    a = _forward(w, qk[0, 0], v[0, 0], R)
    b = _forward(w, qk[0, 0], v[0, 0], R, dup_correct=False)
    assert np.array_equal(a["o"], b["o"]) and np.array_equal(a["lse"], b["lse"])


def union_has_duplicates(L=48, d=8, nb=6, n_r=3, chunk=8, causal=False, seed=13) -> bool:
    """True if some query sees some other key in two or more rounds."""
    w, qk, v, R = small_case(L=L, d=d, nb=nb, n_r=n_r, chunk=chunk, causal=causal, seed=seed)
    buckets, _ = O.hash_buckets(qk, R)
    W = RF.brute_windows(buckets[0, 0], chunk, causal)
    for i in range(L):
        for j in range(L):
            if j != i and sum(j in Wr[i] for Wr in W) > 1:
                return True
    return False


def check_constant_values(seed=14):
    w, qk, v, R = small_case(L=64, d=8, nb=8, n_r=2, chunk=16, causal=True, seed=seed)
    ones = np.ones_like(v)
    out = _forward(w, qk, ones, R)
    assert np.max(np.abs(out["o_rounds"] - 1.0)) < 1e-12
    # rounds whose window holds only the query have lse near -SELF_PENALTY, whose
    # rounding (ulp 1.5e-11) bounds how exactly the combine weights sum to one
    assert np.max(np.abs(out["o"] - 1.0)) < TOL_COMBINED


def check_onehot_values(causal=True, seed=15):
    L, d = 32, 32
    w, qk, _, R = small_case(L=L, d=d, nb=6, n_r=2, chunk=8, causal=causal, seed=seed)
    v = np.eye(L, d)[None, None]
    out = _forward(w, qk, v, R)
    W = RF.brute_windows(out["buckets"][0, 0], w.chunk, causal)
    for r in range(w.n_rounds):
        wts = out["o_rounds"][0, 0, r]                 # row i = weights of query i over positions
        assert np.all(wts > -1e-15)
        assert np.max(np.abs(wts.sum(axis=1) - 1.0)) < 1e-12
        for i in range(L):
            outside = [j for j in range(L) if j not in W[r][i]]
            assert np.max(np.abs(wts[i, outside]), initial=0.0) < 1e-300
            if len(W[r][i]) > 1:
                assert wts[i, i] == 0.0


def check_causal_first_position(seed=16):
    w, qk, v, R = small_case(L=64, d=8, nb=8, n_r=3, chunk=16, causal=True, seed=seed)
    out = _forward(w, qk, v, R)
    assert np.array_equal(out["o_rounds"][0, 0, :, 0], np.repeat(v[0, 0, :1], 3, axis=0))
    # Every round's lse is about -SELF_PENALTY here, so lse - LSE carries the
    # rounding of numbers near 1e5 (ulp 1.5e-11): the combine is exact to ~1e-10.
    assert np.max(np.abs(out["o"][0, 0, 0] - v[0, 0, 0])) < TOL_COMBINED


def check_combine(seed=17):
    rng = np.random.default_rng(seed)
    o_r = rng.standard_normal((2, 1, 20, 4))
    lse = rng.standard_normal((2, 1, 20))
    o, LSE = O.combine_rounds(o_r, lse)
    assert np.array_equal(o, o_r[:, 0])
    assert np.array_equal(LSE, lse[:, 0])
    o_r = rng.standard_normal((3, 5, 20, 4))
    lse = np.full((3, 5, 20), 0.7)
    o, LSE = O.combine_rounds(o_r, lse)
    assert np.max(np.abs(o - o_r.mean(axis=1))) < 1e-14
    assert np.max(np.abs(LSE - (0.7 + math.log(5)))) < 1e-14


# --------------------------------------------------------------------------- the layer
def _layer_case(B=2, L=24, d_model=12, H=2, d=4, seed=28):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, L, d_model))
    w_qk = rng.standard_normal((H * d, d_model))
    w_v = rng.standard_normal((H * d, d_model))
    w_o = rng.standard_normal((d_model, H * d))
    return x, w_qk, w_v, w_o


def check_projections_brute_force():
    """Both projections against Python loops over the definitions (non-square
    weights, so a transposed operand fails)."""
    H, d = 2, 4
    x, w_qk, w_v, w_o = _layer_case(H=H, d=d)
    B, L, dm = x.shape
    qk, v = O.project_in(x, w_qk, w_v, H)
    o = np.random.default_rng(29).standard_normal((B, H, L, d))
    y = O.project_out(o, w_o)
    for b in range(B):
        for i in range(L):
            for h in range(H):
                for c in range(d):
                    ref_q = sum(x[b, i, k] * w_qk[h * d + c, k] for k in range(dm))
                    ref_v = sum(x[b, i, k] * w_v[h * d + c, k] for k in range(dm))
                    assert abs(qk[b, h, i, c] - ref_q) < 1e-12 and abs(v[b, h, i, c] - ref_v) < 1e-12
            for n in range(dm):
                ref_y = sum(o[b, h, i, c] * w_o[n, h * d + c] for h in range(H) for c in range(d))
                assert abs(y[b, i, n] - ref_y) < 1e-12


def check_identity_layer(seed=30):
    """With d_model = H*d and identity weights the layer is the four steps on the
    input's head slices (built here with loops) and their outputs side by side."""
    H, d, B, L = 2, 8, 1, 32
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, L, H * d))
    eye = np.eye(H * d)
    R = rng.standard_normal((3, d, 3))
    out = O.layer_forward(x, eye, eye, eye, R, H, 6, 8, True)
    heads = np.empty((B, H, L, d))
    for b in range(B):
        for h in range(H):
            for i in range(L):
                heads[b, h, i] = x[b, i, h * d:(h + 1) * d]
    ref = O.forward(heads, heads, R, 6, 8, True)
    for b in range(B):
        for i in range(L):
            for h in range(H):
                assert np.max(np.abs(out["y"][b, i, h * d:(h + 1) * d] - ref["o"][b, h, i])) < 1e-12


def check_head_permutation(seed=31):
    """Permuting the heads consistently in w_qk, w_v and w_o leaves the layer's
    output unchanged (heads are attended independently with the shared R)."""
    H, d = 3, 4
    x, w_qk, w_v, w_o = _layer_case(B=1, L=32, d_model=10, H=H, d=d, seed=seed)
    R = np.random.default_rng(seed + 1).standard_normal((2, d, 2))
    perm = [2, 0, 1]
    rows = np.concatenate([np.arange(h * d, (h + 1) * d) for h in perm])
    a = O.layer_forward(x, w_qk, w_v, w_o, R, H, 4, 8, False)
    b = O.layer_forward(x, w_qk[rows], w_v[rows], w_o[:, rows], R, H, 4, 8, False)
    assert np.max(np.abs(a["y"] - b["y"])) < 1e-12


# --------------------------------------------------------------------------- backward
def _bwd_case(L=16, d=3, n_r=2, nb=4, seed=40):
    rng = np.random.default_rng(seed)
    qk = rng.standard_normal((1, 1, L, d))
    v = rng.standard_normal((1, 1, L, d))
    d_o = rng.standard_normal((1, 1, L, d))
    buckets = rng.integers(0, nb, size=(1, 1, n_r, L))
    return qk, v, d_o, buckets


def _loss(qk, v, d_o, perm, cid, chunk, causal, scale, dup_correct, wrap=False, buckets=None):
    o_r, lse = O.attention_rounds(qk, v, perm, cid, chunk, causal, scale, dup_correct=dup_correct,
                                  wrap=wrap, buckets=buckets)
    o, _ = O.combine_rounds(o_r, lse)
    return float(np.sum(o * d_o))


def check_backward_finite_differences(causal=True, n_r=2, dup_correct=True, seed=40, wrap=False,
                                      same_bucket=False):
    """Central differences of sum(o * d_o) in every element of qk and v, with the
    buckets held fixed (they are piecewise constant in qk)."""
    L, d, nb, chunk = 16, 3, 4, 4
    qk, v, d_o, buckets = _bwd_case(L, d, n_r, nb, seed)
    perm, cid = O.sort_rounds(buckets, nb, chunk)
    scale = 0.7
    bk = buckets if same_bucket else None
    g = O.attention_backward(qk, v, perm, cid, d_o, chunk, causal, scale, dup_correct, wrap, bk)
    h = 1e-4
    for name, arr, grad in (("qk", qk, g["dqk"]), ("v", v, g["dv"])):
        fd = np.empty_like(arr)
        for idx in np.ndindex(arr.shape):
            a_p = arr.copy(); a_p[idx] += h
            a_m = arr.copy(); a_m[idx] -= h
            args_p = (a_p, v) if name == "qk" else (qk, a_p)
            args_m = (a_m, v) if name == "qk" else (qk, a_m)
            fd[idx] = (_loss(*args_p, d_o, perm, cid, chunk, causal, scale, dup_correct, wrap, bk)
                       - _loss(*args_m, d_o, perm, cid, chunk, causal, scale, dup_correct, wrap, bk)) / (2 * h)
        err = np.max(np.abs(grad - fd)) / np.max(np.abs(fd))
        assert err < 1e-6, f"d{name}: relative deviation {err:.3g} from finite differences"


def check_backward_union_autograd(causal=False, n_r=3, seed=41, wrap=False, same_bucket=False):
    """The oracle's gradients equal torch autograd of the union closed form
    (tests/reference_forms.py), which shares no code with the oracle."""
    import torch
    L, d, nb, chunk = 24, 4, 4, 4
    qk, v, d_o, buckets = _bwd_case(L, d, n_r, nb, seed)
    perm, cid = O.sort_rounds(buckets, nb, chunk)
    scale = 0.5
    g = O.attention_backward(qk, v, perm, cid, d_o, chunk, causal, scale, True, wrap,
                             buckets if same_bucket else None)
    W = RF.brute_windows(buckets[0, 0], chunk, causal, wrap, same_bucket)
    tq = torch.tensor(qk[0, 0], dtype=torch.float64, requires_grad=True)
    tv = torch.tensor(v[0, 0], dtype=torch.float64, requires_grad=True)
    out = RF.union_attention_torch(tq, tv, W, scale)
    (out * torch.tensor(d_o[0, 0])).sum().backward()
    for name, got, want in (("qk", g["dqk"][0, 0], tq.grad.numpy()), ("v", g["dv"][0, 0], tv.grad.numpy())):
        err = np.max(np.abs(got - want)) / np.max(np.abs(want))
        assert err < 1e-9, f"d{name}: relative deviation {err:.3g} from autograd of the union form"


def check_backward_dv_sum(seed=42):
    """Each query's combined weights sum to one, so sum_j dv_j = sum_i d_o_i."""
    L, d, nb, chunk = 32, 5, 8, 4
    qk, v, d_o, buckets = _bwd_case(L, d, 4, nb, seed)
    perm, cid = O.sort_rounds(buckets, nb, chunk)
    g = O.attention_backward(qk, v, perm, cid, d_o, chunk, True, 0.6)
    assert np.allclose(g["dv"].sum(axis=2), d_o.sum(axis=2), rtol=0, atol=1e-10)
    assert np.allclose(g["dqk_rounds"].sum(axis=2), g["dqk"], rtol=0, atol=1e-12)


def check_backward_one(seed=45):
    """The single-position gradients (used by the sampled GPU checks) equal the
    rows of the full backward."""
    L, d, nb, chunk = 48, 4, 4, 4
    for causal in (True, False):
        qk, v, d_o, buckets = _bwd_case(L, d, 3, nb, seed)
        perm, cid = O.sort_rounds(buckets, nb, chunk)
        g = O.attention_backward(qk, v, perm, cid, d_o, chunk, causal, 0.8)
        for pos in (0, 5, 17, 47):
            dq, dv = O.attention_backward_one(qk[0, 0], v[0, 0], d_o[0, 0], perm[0, 0], cid[0, 0],
                                              pos, chunk, causal, 0.8)
            assert np.allclose(dq, g["dqk"][0, 0, pos], rtol=0, atol=1e-9)
            assert np.allclose(dv, g["dv"][0, 0, pos], rtol=0, atol=1e-9)


# --------------------------------------------------------------------------- Reformer block
def _block_case(B=1, L=32, d_model=8, H=2, d=4, d_ff=12, seed=60):
    rng = np.random.default_rng(seed)
    hd = H * d
    wa = {"w_qk": rng.standard_normal((hd, d_model)) / np.sqrt(d_model),
          "w_v": rng.standard_normal((hd, d_model)) / np.sqrt(d_model),
          "w_o": rng.standard_normal((d_model, hd)) / np.sqrt(hd)}
    wf = {"w1": rng.standard_normal((d_ff, d_model)) / np.sqrt(d_model),
          "b1": rng.standard_normal(d_ff) * 0.5,
          "w2": rng.standard_normal((d_model, d_ff)) / np.sqrt(d_ff),
          "b2": rng.standard_normal(d_model) * 0.5}
    x1 = rng.standard_normal((B, L, d_model))
    x2 = rng.standard_normal((B, L, d_model))
    R = rng.standard_normal((2, d, 2))
    return x1, x2, wa, wf, R


def check_feed_forward_brute_force(seed=61):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((2, 5, 3))
    w1, b1 = rng.standard_normal((7, 3)), rng.standard_normal(7)
    w2, b2 = rng.standard_normal((3, 7)), rng.standard_normal(3)
    got = O.feed_forward(x, w1, b1, w2, b2)
    saw_negative = False
    for b in range(2):
        for i in range(5):
            h = []
            for f in range(7):
                a = b1[f] + sum(x[b, i, k] * w1[f, k] for k in range(3))
                saw_negative |= a < 0
                h.append(a if a > 0 else 0.0)
            for n in range(3):
                want = b2[n] + sum(h[f] * w2[n, f] for f in range(7))
                assert abs(got[b, i, n] - want) < 1e-12
    assert saw_negative      # the ReLU is exercised


def check_ffn_chunking(seed=62):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((2, 13, 6))
    w1, b1 = rng.standard_normal((10, 6)), rng.standard_normal(10)
    w2, b2 = rng.standard_normal((6, 10)), rng.standard_normal(6)
    full = O.feed_forward(x, w1, b1, w2, b2)
    for cr in (1, 3, 7, 26, 40):       # 26 rows in all: ragged last chunks, one chunk, larger
        assert np.allclose(O.feed_forward_chunked(x, w1, b1, w2, b2, cr), full, rtol=0, atol=1e-12)


def check_block_round_trip(seed=63):
    """inverse(forward(x)) = x: the reversible block recomputes its inputs."""
    for causal in (True, False):
        x1, x2, wa, wf, R = _block_case(seed=seed)
        y1, y2 = O.block_forward(x1, x2, wa, wf, R, 2, 4, 4, causal, chunk_rows=5)
        assert np.max(np.abs(y1 - x1)) > 0.1 and np.max(np.abs(y2 - x2)) > 0.1
        r1, r2 = O.block_inverse(y1, y2, wa, wf, R, 2, 4, 4, causal, chunk_rows=7)
        assert np.allclose(r1, x1, rtol=0, atol=1e-10) and np.allclose(r2, x2, rtol=0, atol=1e-10)


def check_block_zero_weights(seed=64):
    """Zero output weights make both branches vanish: the block is the identity."""
    x1, x2, wa, wf, R = _block_case(seed=seed)
    wa = dict(wa, w_o=np.zeros_like(wa["w_o"]))
    wf = dict(wf, w2=np.zeros_like(wf["w2"]), b2=np.zeros_like(wf["b2"]))
    y1, y2 = O.block_forward(x1, x2, wa, wf, R, 2, 4, 4, True, chunk_rows=8)
    assert np.array_equal(y1, x1) and np.array_equal(y2, x2)


ALL_CHECKS = {
    "hash_demo": check_hash_demo,
    "hash_labels": check_hash_labels,
    "hash_margin": check_hash_margin,
    "hash_antipodal": check_hash_antipodal,
    "hash_scale": check_hash_scale_invariance,
    "simhash": check_simhash_rate,
    "sort_library": check_sort_matches_library,
    "sort_cid": check_sort_rounds_cid,
    "full_attention": check_full_attention,
    "full_attention_causal": lambda: check_full_attention(causal=True, n_r=2, nb=2),
    "union": check_union,
    "union_causal": lambda: check_union(causal=True, n_r=4, nb=4, chunk=4, L=32),
    "constant_values": check_constant_values,
    "onehot_values": check_onehot_values,
    "causal_first": check_causal_first_position,
    "combine": check_combine,
    "union_wrap": lambda: check_union(wrap=True, nb=4, chunk=8, L=40, seed=21),
    "union_wrap_causal": lambda: check_union(wrap=True, causal=True, n_r=4, nb=4, chunk=4, L=32,
                                             seed=22),
    "wrap_two_chunks": check_wrap_two_chunks,
    "wrap_two_chunks_causal": lambda: check_wrap_two_chunks(causal=True, seed=23),
    "rounds_without_correction": check_rounds_without_correction,
    "rounds_without_correction_wrap": lambda: check_rounds_without_correction(wrap=True,
                                                                              causal=False, seed=24),
    "single_round_correction_free": check_single_round_correction_free,
    "union_same_bucket": lambda: check_union(same_bucket=True, nb=4, chunk=8, L=48, seed=25),
    "union_same_bucket_causal": lambda: check_union(same_bucket=True, causal=True, n_r=4, nb=4,
                                                    chunk=4, L=32, seed=26),
    "rounds_without_correction_same_bucket": lambda: check_rounds_without_correction(
        same_bucket=True, nb=4, seed=27),
    "projections_brute_force": check_projections_brute_force,
    "identity_layer": check_identity_layer,
    "head_permutation": check_head_permutation,
    "backward_finite_differences": check_backward_finite_differences,
    "backward_finite_differences_noncausal_no_correction": lambda: check_backward_finite_differences(
        causal=False, n_r=3, dup_correct=False, seed=43),
    "backward_finite_differences_wrap": lambda: check_backward_finite_differences(
        causal=False, n_r=3, seed=46, wrap=True),
    "backward_finite_differences_same_bucket": lambda: check_backward_finite_differences(
        causal=True, n_r=3, seed=47, same_bucket=True),
    "backward_union_autograd": check_backward_union_autograd,
    "backward_union_autograd_causal": lambda: check_backward_union_autograd(causal=True, n_r=2, seed=44),
    "backward_union_autograd_wrap": lambda: check_backward_union_autograd(causal=True, n_r=3, seed=48,
                                                                          wrap=True),
    "backward_union_autograd_same_bucket": lambda: check_backward_union_autograd(
        causal=False, n_r=3, seed=49, same_bucket=True),
    "backward_dv_sum": check_backward_dv_sum,
    "backward_one": check_backward_one,
    "feed_forward_brute_force": check_feed_forward_brute_force,
    "ffn_chunking": check_ffn_chunking,
    "block_round_trip": check_block_round_trip,
    "block_zero_weights": check_block_zero_weights,
}
