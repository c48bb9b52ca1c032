"""CPU tests of the oracle against its pins, and mutation tests showing that a
plausible mistake planted in the oracle (on the CPU) fails at least one pin."""
from __future__ import annotations

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle.lsh_oracle as O
import oracle_pins as P


@pytest.mark.parametrize("name", sorted(P.ALL_CHECKS))
def test_pin(name):
    P.ALL_CHECKS[name]()


@pytest.mark.parametrize("nb,n_r,causal,scale", [(2, 1, False, None), (2, 3, True, None),
                                                 (10, 4, False, 1.0), (16, 2, True, 0.3)])
def test_full_attention_any_buckets_and_rounds(nb, n_r, causal, scale):
    P.check_full_attention(L=32, d=8, nb=nb, n_r=n_r, causal=causal, scale=scale, seed=nb + n_r)


@settings(max_examples=40, deadline=None)
@given(L_chunks=st.integers(1, 8), chunk=st.sampled_from([1, 2, 4, 8]),
       nb_half=st.integers(1, 8), n_r=st.integers(1, 4), causal=st.booleans(),
       seed=st.integers(0, 10_000))
def test_union_bruteforce(L_chunks, chunk, nb_half, n_r, causal, seed):
    L = L_chunks * chunk
    if L > 64:
        return
    P.check_union(L=L, d=4, nb=2 * nb_half, n_r=n_r, chunk=chunk, causal=causal, seed=seed)


def test_union_negative_control():
    """Without the duplicate-count correction the union identity must fail."""
    kw = dict(L=48, d=8, nb=6, n_r=3, chunk=8, causal=False, seed=13)
    assert P.union_has_duplicates(**kw)
    P.check_union(**kw)
    with pytest.raises(AssertionError):
        P.check_union(dup_correct=False, **kw)


def test_oracle_shapes_and_dtypes():
    w, qk, v, R = P.small_case(L=64, d=8, nb=8, n_r=2, chunk=16, causal=True)
    out = O.forward(qk, v, R, w.n_buckets, w.chunk, w.causal)
    assert out["buckets"].shape == (1, 1, 2, 64) and out["buckets"].dtype == np.int32
    assert out["perm"].shape == (1, 1, 2, 64) and out["perm"].dtype == np.int32
    assert out["cid"].shape == (1, 1, 64, 2) and out["cid"].dtype == np.int16
    assert out["o_rounds"].shape == (1, 1, 2, 64, 8)
    assert out["lse"].shape == (1, 1, 2, 64)
    assert out["o"].shape == (1, 1, 64, 8)


def test_attention_one_matches_rounds():
    w, qk, v, R = P.small_case(L=64, d=8, nb=8, n_r=3, chunk=16, causal=True, seed=21)
    out = O.forward(qk, v, R, w.n_buckets, w.chunk, w.causal)
    sc = O.default_scale(8)
    for r in range(3):
        for pos in (0, 5, 17, 63):
            o, l = O.attention_one(qk[0, 0], v[0, 0], out["perm"][0, 0], out["cid"][0, 0], r, pos,
                                   w.chunk, w.causal, sc)
            assert np.max(np.abs(o - out["o_rounds"][0, 0, r, pos])) < 1e-14
            assert abs(l - out["lse"][0, 0, r, pos]) < 1e-12


# --------------------------------------------------------------------------- mutations
def _argmax_positive_half_only(p):
    p = np.asarray(p, dtype=np.float64)
    b = np.argmax(p, axis=-1).astype(np.int32)
    s = np.sort(p, axis=-1)
    m = s[:, -1] - (s[:, -2] if p.shape[1] > 1 else -np.inf)
    return b, m


def _argmin_labels(p):
    a = np.concatenate([p, -p], axis=-1)
    b = np.argmin(a, axis=-1).astype(np.int32)
    return b, np.ones(a.shape[0])


def _margin_over_p_only(p):
    """Bucket right, margin taken between the two largest entries of p alone."""
    p = np.asarray(p, dtype=np.float64)
    a = np.concatenate([p, -p], axis=-1)
    s = np.sort(p, axis=-1)
    m = s[:, -1] - s[:, -2] if p.shape[1] > 1 else np.abs(2 * s[:, -1])
    return np.argmax(a, axis=-1).astype(np.int32), m


def _margin_skips_negated_runner_up(p):
    """Bucket right; the runner-up is searched in the winner's own half only."""
    p = np.asarray(p, dtype=np.float64)
    a = np.concatenate([p, -p], axis=-1)
    b = np.argmax(a, axis=-1)
    half = p.shape[1]
    m = np.empty(p.shape[0])
    for i in range(p.shape[0]):
        side = a[i, :half] if b[i] < half else a[i, half:]
        s = np.sort(side)
        m[i] = s[-1] - s[-2] if half > 1 else 2 * abs(s[-1])
    return b.astype(np.int32), m


def _margin_absolute_values(p):
    """Bucket right; margin from the two largest |p| even with one column."""
    p = np.asarray(p, dtype=np.float64)
    a = np.concatenate([p, -p], axis=-1)
    s = np.sort(np.abs(p), axis=-1)
    m = s[:, -1] - (s[:, -2] if p.shape[1] > 1 else 0.0)
    return np.argmax(a, axis=-1).astype(np.int32), m


def _unstable_sort(keys, n_keys):
    keys = np.asarray(keys)
    return np.lexsort((-np.arange(keys.size), keys))


def _own_chunk_only(k, chunk, *_):
    return np.arange(k * chunk, (k + 1) * chunk)


def _two_back(k, chunk, *_):
    own = np.arange(k * chunk, (k + 1) * chunk)
    return own if k < 2 else np.concatenate([np.arange((k - 2) * chunk, (k - 1) * chunk), own])


def _mean_combine(o_r, lse):
    return np.asarray(o_r).mean(axis=-3), np.asarray(lse).max(axis=-2)


_DUP_ORIG = O.duplicate_counts


def _wrap(fn, transform):
    def inner(*a, **k):
        a, k = transform(list(a), dict(k))
        return fn(*a, **k)
    return inner


def _ignore_causal(a, k):
    a[6] = False
    return a, k


def _values_are_keys(a, k):
    a[1] = a[0]
    return a, k


def _correction_always_on(a, k):
    k["dup_correct"] = True
    return a, k


def _bucket_mask_ignored(a, k):
    k["bkt_bh"] = None
    return a, k


_WINDOW_CHUNKS_ORIG = O.window_chunks


def _weights_read_as_in_out(x, w_qk, w_v, heads):
    """The [out, in] weights' memory taken as [in, out] (a layout mix-up)."""
    x = np.asarray(x, dtype=np.float64)
    qk = x @ np.reshape(w_qk, (w_qk.shape[1], w_qk.shape[0]))
    v = x @ np.reshape(w_v, (w_v.shape[1], w_v.shape[0]))
    return O.split_heads(qk, heads), O.split_heads(v, heads)


_GRAD_ORIG = O.chunk_attention_grad


def _grad_without_delta(qk, v, do, LSE, delta, *a, **k):
    return _GRAD_ORIG(qk, v, do, LSE, np.zeros_like(delta), *a, **k)


def _grad_part_zeroed(part):
    def f(*a, **k):
        out = list(_GRAD_ORIG(*a, **k))
        out[part] = np.zeros_like(out[part])
        return tuple(out)
    return f


def _ffn_without_relu(x, w1, b1, w2, b2):
    x = np.asarray(x, dtype=np.float64)
    return (x @ w1.T + b1) @ w2.T + b2


def _chunked_drops_tail(x, w1, b1, w2, b2, chunk_rows):
    rows = np.asarray(x, dtype=np.float64).reshape(-1, x.shape[-1])
    out = np.zeros((rows.shape[0], w2.shape[0]))
    for r0 in range(0, rows.shape[0] - chunk_rows + 1, chunk_rows):
        out[r0:r0 + chunk_rows] = O.feed_forward(rows[r0:r0 + chunk_rows], w1, b1, w2, b2)
    return out.reshape(x.shape[:-1] + (out.shape[-1],))


def _inverse_wrong_order(y1, y2, wa, wf, R, heads, nb, chunk, causal, chunk_rows, scale=None, **v):
    # x1 first, from the output half y2 (not yet inverted): wrong
    x1 = y1 - O.attention_block(y2, wa, R, heads, nb, chunk, causal, scale, **v)
    x2 = y2 - O.feed_forward_chunked(y1, wf["w1"], wf["b1"], wf["w2"], wf["b2"], chunk_rows)
    return x1, x2


MUTATIONS = {
    "feed-forward without ReLU": ("feed_forward", _ffn_without_relu, "feed_forward_brute_force"),
    "chunked feed-forward drops the ragged tail": ("feed_forward_chunked", _chunked_drops_tail,
                                                   "ffn_chunking"),
    "block inverse in the wrong order": ("block_inverse", _inverse_wrong_order, "block_round_trip"),
    "backward drops Delta": ("chunk_attention_grad", _grad_without_delta, "backward_finite_differences"),
    "backward drops the key role": ("chunk_attention_grad", _grad_part_zeroed(3),
                                    "backward_union_autograd"),
    "backward drops the query role": ("chunk_attention_grad", _grad_part_zeroed(2),
                                      "backward_finite_differences"),
    "hash drops the negated half": ("bucket_from_projection", _argmax_positive_half_only, "hash_antipodal"),
    "hash takes argmin": ("bucket_from_projection", _argmin_labels, "hash_labels"),
    "margin over p only": ("bucket_from_projection", _margin_over_p_only, "hash_margin"),
    "margin skips the negated runner-up": ("bucket_from_projection", _margin_skips_negated_runner_up,
                                           "hash_margin"),
    "margin from |p| with one column": ("bucket_from_projection", _margin_absolute_values,
                                        "hash_margin"),
    "sort not stable": ("stable_counting_sort", _unstable_sort, "sort_library"),
    "no look-back chunk": ("window_slots", _own_chunk_only, "union"),
    "look-back two chunks": ("window_slots", _two_back, "union"),
    "duplicate counts dropped": ("duplicate_counts", lambda q, k, *_: np.ones((len(q), len(k))), "union"),
    "log of duplicate count dropped": ("duplicate_counts",
                                       lambda q, k, *a: np.exp(_DUP_ORIG(q, k, *a)),
                                       "union"),
    "no self penalty": ("SELF_PENALTY", 0.0, "full_attention"),
    "causal flag ignored": ("chunk_attention", "ignore_causal", "full_attention_causal"),
    "keys used as values": ("chunk_attention", "values_are_keys", "full_attention"),
    "scale dropped": ("default_scale", lambda d: 1.0, "full_attention"),
    "rounds averaged": ("combine_rounds", _mean_combine, "union"),
    "wrap-around ignored": ("window_chunks", lambda k, n, wrap=False: _WINDOW_CHUNKS_ORIG(k, n, False),
                            "wrap_two_chunks"),
    "wrap-around missing from the counts": ("duplicate_counts",
                                            lambda q, k, n=0, wrap=False, *b: _DUP_ORIG(q, k, n, False, *b),
                                            "union_wrap"),
    "correction applied when switched off": ("chunk_attention", "correction_always_on",
                                             "rounds_without_correction"),
    "same-bucket mask ignored": ("chunk_attention", "bucket_mask_ignored", "union_same_bucket"),
    "heads split in the wrong order": ("split_heads",
                                       lambda t, H: t.reshape(t.shape[0], t.shape[1], t.shape[2] // H, H)
                                       .transpose(0, 3, 1, 2), "identity_layer"),
    "projection weight read as [in, out]": ("project_in", _weights_read_as_in_out,
                                            "projections_brute_force"),
    "buckets missing from the counts": ("duplicate_counts",
                                        lambda q, k, n=0, wrap=False, *b: _DUP_ORIG(q, k, n, wrap),
                                        "union_same_bucket"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    attr, repl, check = MUTATIONS[name]
    orig = getattr(O, attr)
    if repl == "ignore_causal":
        repl = _wrap(orig, _ignore_causal)
    elif repl == "values_are_keys":
        repl = _wrap(orig, _values_are_keys)
    elif repl == "correction_always_on":
        repl = _wrap(orig, _correction_always_on)
    elif repl == "bucket_mask_ignored":
        repl = _wrap(orig, _bucket_mask_ignored)
    monkeypatch.setattr(O, attr, repl)
    with pytest.raises((AssertionError, IndexError, ValueError)):
        P.ALL_CHECKS[check]()


# --------------------------------------------------------------------------- pooled oracle
@pytest.mark.parametrize("kw", [dict(), dict(same_bucket=True), dict(wrap=True, dup_correct=False)])
def test_pooled_forward_equals_forward(kw):
    """The benchmark's process-pool driver (oracle/pool.py) splits the oracle's
    forward into per-(slice, round) jobs; the results are the same arrays."""
    from oracle.pool import OraclePool
    w, _, _, R = P.small_case(L=64, d=8, nb=8, n_r=3, chunk=8, causal=True, seed=33)
    rng = np.random.default_rng(34)
    qk = rng.standard_normal((2, 2, 64, 8)).astype(np.float32)
    v = rng.standard_normal((2, 2, 64, 8)).astype(np.float32)
    ref = O.forward(qk.astype(np.float64), v.astype(np.float64), R, 8, 8, True, **kw)
    with OraclePool(workers=3) as pool:
        got = pool.forward(qk, v, R, 8, 8, True, **kw)
    for k in ("buckets", "margins", "perm", "cid", "o_rounds", "lse", "o", "LSE"):
        assert np.array_equal(got[k], ref[k]), k
    assert set(got["seconds"]) == {"hash_sort", "attention", "combine", "total"}
