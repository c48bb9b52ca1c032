"""Plain fp64 CPU oracle for the forward pass of multi-round LSH attention with
shared query/key vectors (Reformer).

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import or run this module.  The HIP library and its Python
binding never import it, and it imports nothing from them: it shares no code,
table or constant with the GPU path.  Inputs arrive as NumPy arrays (the seeded
generator's float32 values, upcast here exactly to float64).

Sources (page title, section):
  [ULT] Ultralytics glossary "Reformer" (Spanish and Arabic editions), section
        "Atención LSH" / "الانتباه باستخدام LSH", with its hashing example and the
        result printed after it.
  [MOD] modulabs-hub notes on "Reformer: The Efficient Transformer", sections
        "Locality sensitive hashing", "LSH attention", "Multi-round LSH attention".
  [AIS] ai-scholar.tech article on Reformer, section "变形金刚有哪些问题？" (the
        scaled dot-product attention formula) and section "什么是本地敏感散列（LSH）？"
        (bucket, sort, equal chunks, attend to own and previous chunk); its
        experiment set-up (d_model 1024, 8 heads) sizes the layer around them.

The steps, in the pages' order:
  1. hash     bucket = first index of the maximum of [x R_r, -x R_r]      [ULT], [MOD]
  2. sort     positions sorted by bucket (stable, so ties keep position order),
              one sort per (batch row, head, round)                       [AIS], [ULT], [MOD]
  3. attend   sorted sequence cut into equal chunks; each query attends to its
              own chunk and the previous one, never to itself unless nothing
              else is there, optionally only to earlier positions          [AIS], [ULT], [MOD]
  4. combine  the rounds merged by logsumexp weights                      [ULT], [MOD]
Also the gradient of steps 3-4 with respect to qk and v (attention_backward),
by the chain rule through the steps above (the pages print no backward pass);
the attention layer around the steps (projections); and the Reformer block
built from it: reversible residual halves with a chunked feed-forward layer.

Readings taken where the pages leave a step open (each is argued in the design
notes):
  * scale is a parameter, default 1/sqrt(d_head) ([AIS] formula; [MOD] says the
    LSH form drops it, so scale = 1 is also accepted);
  * keys are the shared vectors themselves (no normalisation);
  * inside a window there is no same-bucket mask: the attended set of a round
    is the chunk window;
  * chunk 0 has no previous chunk (no wrap-around) and look-back stays inside
    a round; chunk must divide L.  The variant wrap=True gives chunk 0 the last
    chunk of its round as look-back (a window is a set of chunks, so a single
    chunk is attended once);
  * the self score carries a penalty of SELF_PENALTY score units in every
    round, so "self only if nothing else" is decided over all rounds together;
  * the score of key j for query i in a round is lowered by log N_ij, where
    N_ij is the number of rounds whose window for i contains j (duplicate-count
    correction); with it, the combined output equals attention over the union
    of the rounds' windows.  The variant dup_correct=False leaves it out;
  * inside a window every key is attended, whatever its bucket.  The variant
    same_bucket=True keeps only keys in the query's bucket of that round
    ([MOD] "LSH attention": the set P_i of keys hashed like the query), and
    N_ij then counts the rounds where j is in the window and in i's bucket;
  * R has shape [n_rounds, d, n_buckets/2] and is shared by every batch row and
    head, as in [ULT]'s example;
  * ties in the argmax go to the first index, as in [ULT]'s example.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

SELF_PENALTY = 1.0e5      # subtracted from the self score, in score units (after scaling)
NEAR_TIE_MARGIN = 1.0e-4  # a hash whose top-2 gap is at most this is a near-tie


# --------------------------------------------------------------------------- 1. hash
def project(x: np.ndarray, R_r: np.ndarray) -> np.ndarray:
    """Random projection p = x · R_r in float64.  x [n, d], R_r [d, n_buckets/2].

    [ULT]: multiply by a random matrix R (one per round).
    """
    return np.asarray(x, dtype=np.float64) @ np.asarray(R_r, dtype=np.float64)


def bucket_from_projection(p: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """bucket = first index of the maximum of [p, -p]; margin = top-1 minus top-2.

    [ULT], [MOD] "Locality sensitive hashing": half as many random columns as
    buckets, concatenated with their negation; the bucket is the position of the
    largest entry.  np.argmax returns the first index on exact ties, like the
    argmax of [ULT]'s example.  The margin is the gap between the largest and
    second-largest entries of [p, -p]; a zero vector has margin 0.
    """
    p = np.asarray(p, dtype=np.float64)
    a = np.concatenate([p, -p], axis=-1)
    bucket = np.argmax(a, axis=-1)
    rows = np.arange(a.shape[0])
    top = a[rows, bucket]
    rest = a.copy()
    rest[rows, bucket] = -np.inf
    margin = top - rest.max(axis=-1)
    return bucket.astype(np.int32), margin


def hash_buckets(qk: np.ndarray, R: np.ndarray, row_block: int = 16384):
    """Buckets and margins for every (batch row, head, round, position).

    qk [B, H, L, d], R [n_rounds, d, n_buckets/2]  ->
    buckets int32 [B, H, n_rounds, L], margins float64 [B, H, n_rounds, L].
    Rows are processed in blocks only to bound the size of the [p, -p] matrix.
    """
    B, H, L, _ = qk.shape
    n_r = R.shape[0]
    buckets = np.empty((B, H, n_r, L), dtype=np.int32)
    margins = np.empty((B, H, n_r, L), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for r in range(n_r):
                for s in range(0, L, row_block):
                    e = min(s + row_block, L)
                    bk, mg = bucket_from_projection(project(qk[b, h, s:e], R[r]))
                    buckets[b, h, r, s:e] = bk
                    margins[b, h, r, s:e] = mg
    return buckets, margins


def hash_one(qk_row: np.ndarray, R_r: np.ndarray) -> Tuple[int, float]:
    """Bucket and margin of a single vector under one round's R (for sampled checks)."""
    bk, mg = bucket_from_projection(project(np.asarray(qk_row)[None, :], R_r))
    return int(bk[0]), float(mg[0])


# --------------------------------------------------------------------------- 2. sort
def stable_counting_sort(keys: np.ndarray, n_keys: int) -> np.ndarray:
    """Positions sorted by key, equal keys kept in position order.

    Counting sort: histogram of the keys, exclusive prefix sum of the histogram
    (the first slot of each key), then every position, visited in increasing
    order, is written to the next free slot of its key.  [AIS], [MOD]: sort the
    tokens by bucket so that bucket-mates become neighbours.
    """
    keys = np.asarray(keys, dtype=np.int64)
    counts = np.bincount(keys, minlength=n_keys)
    first_slot = np.zeros(n_keys, dtype=np.int64)
    first_slot[1:] = np.cumsum(counts)[:-1]
    next_slot = first_slot.tolist()
    perm = [0] * keys.size
    for pos, k in enumerate(keys.tolist()):
        perm[next_slot[k]] = pos
        next_slot[k] += 1
    return np.asarray(perm, dtype=np.int64)


def sort_rounds(buckets: np.ndarray, n_buckets: int, chunk: int):
    """Sorted order and chunk ids for every (batch row, head, round).

    buckets [B, H, n_r, L] -> perm int32 [B, H, n_r, L] (perm[slot] = position)
    and cid int16 [B, H, L, n_r] (cid[position, r] = slot // chunk in round r).
    Sorting by (round, bucket, position) with one sort per round gives the same
    order as one sort over all rounds with the round in the key.
    """
    B, H, n_r, L = buckets.shape
    perm = np.empty((B, H, n_r, L), dtype=np.int32)
    cid = np.empty((B, H, L, n_r), dtype=np.int16)
    for b in range(B):
        for h in range(H):
            for r in range(n_r):
                p = stable_counting_sort(buckets[b, h, r], n_buckets)
                perm[b, h, r] = p
                slot = np.empty(L, dtype=np.int64)
                slot[p] = np.arange(L)
                cid[b, h, :, r] = slot // chunk
    return perm, cid


# --------------------------------------------------------------------------- 3. attend
def window_chunks(k: int, nchunks: int, wrap: bool = False):
    """Chunks attended by chunk k, in slot order: the previous chunk, then k.

    [AIS], [ULT]: the sorted sequence is cut into equal chunks and each chunk
    attends to itself and to the chunk before it.  Chunk 0 has no predecessor,
    unless wrap, where it is the last chunk of the round.  A window is a set:
    a chunk never appears twice (one chunk in all, with wrap).
    """
    if k >= 1:
        return [k - 1, k]
    if wrap and nchunks > 1:
        return [nchunks - 1, 0]
    return [0]


def window_slots(k: int, chunk: int, nchunks: int = 0, wrap: bool = False) -> np.ndarray:
    """Sorted slots of the chunks that chunk k attends to (see window_chunks)."""
    return np.concatenate([np.arange(c * chunk, (c + 1) * chunk)
                           for c in window_chunks(k, nchunks, wrap)])


def duplicate_counts(cid_q: np.ndarray, cid_k: np.ndarray, nchunks: int = 0,
                     wrap: bool = False, bkt_q: Optional[np.ndarray] = None,
                     bkt_k: Optional[np.ndarray] = None) -> np.ndarray:
    """N[i, j] = number of rounds whose window for query i contains key j.

    cid_q [nq, n_r], cid_k [nk, n_r] are chunk ids per round.  Key j lies in the
    window of query i in round r exactly when its chunk is the query's chunk or
    the one before it: cid_q[i, r] - cid_k[j, r] is 0 or 1; with wrap, the
    chunk before chunk 0 is the last one, so the difference is taken modulo
    the number of chunks.  With bucket ids (bkt_q [nq, n_r], bkt_k [nk, n_r])
    a round counts only when the two buckets are equal as well.
    """
    diff = cid_q[:, None, :].astype(np.int64) - cid_k[None, :, :].astype(np.int64)
    if wrap:
        diff = np.mod(diff, nchunks)
    inside = (diff == 0) | (diff == 1)
    if bkt_q is not None:
        inside &= bkt_q[:, None, :] == bkt_k[None, :, :]
    return inside.sum(axis=2)


def window_scores(qk_bh: np.ndarray, perm_r: np.ndarray, cid_bh: np.ndarray, k: int, chunk: int,
                  causal: bool, scale: float, query_slots: Optional[np.ndarray] = None,
                  dup_correct: bool = True, wrap: bool = False,
                  bkt_bh: Optional[np.ndarray] = None, r: int = 0):
    """One round's scores for the queries of sorted chunk k.

    qk_bh [L, d] (one batch row and head), perm_r [L] (this round's sorted
    order), cid_bh [L, n_r].  For query i and key j in the window of chunk k:
        s_ij = scale * <qk_i, qk_j> - log N_ij - SELF_PENALTY * [j == i],
    with s_ij = -inf for keys j > i when causal ([MOD] "LSH attention": only
    earlier positions; the query itself is penalised because shared QK makes it
    the most similar key).  query_slots restricts the queries to some sorted
    slots of chunk k.  The variants dup_correct=False (no log N_ij term) and
    wrap=True (chunk 0 looks back to the last chunk) change the window and its
    scores as described in window_chunks and duplicate_counts.  With bkt_bh
    [L, n_r] (bucket of every position in every round; r is this round) the
    window keeps only the keys in the query's bucket of round r (the
    same-bucket variant; the others get -inf).
    Returns (query positions qi [nq], key positions kj [nk], s [nq, nk]).
    """
    nchunks = len(perm_r) // chunk
    q_slots = np.arange(k * chunk, (k + 1) * chunk) if query_slots is None else np.asarray(query_slots)
    k_slots = window_slots(k, chunk, nchunks, wrap)
    qi = perm_r[q_slots].astype(np.int64)
    kj = perm_r[k_slots].astype(np.int64)
    q = np.asarray(qk_bh[qi], dtype=np.float64)
    kk = np.asarray(qk_bh[kj], dtype=np.float64)
    s = scale * (q @ kk.T)
    if bkt_bh is not None:
        s = np.where(bkt_bh[kj, r][None, :] != bkt_bh[qi, r][:, None], -np.inf, s)
    if dup_correct:
        bq = None if bkt_bh is None else bkt_bh[qi]
        bk = None if bkt_bh is None else bkt_bh[kj]
        N = duplicate_counts(cid_bh[qi], cid_bh[kj], nchunks, wrap, bq, bk)
        # N = 0 only for keys the bucket mask has already set to -inf
        s = s - np.log(np.maximum(N, 1))
    s = s - SELF_PENALTY * (qi[:, None] == kj[None, :])
    if causal:
        s = np.where(kj[None, :] > qi[:, None], -np.inf, s)
    return qi, kj, s


def chunk_attention(qk_bh: np.ndarray, v_bh: np.ndarray, perm_r: np.ndarray,
                    cid_bh: np.ndarray, k: int, chunk: int, causal: bool, scale: float,
                    query_slots: Optional[np.ndarray] = None, dup_correct: bool = True,
                    wrap: bool = False, bkt_bh: Optional[np.ndarray] = None, r: int = 0):
    """One round's attention for the queries of sorted chunk k, over the scores
    of window_scores (same arguments; v_bh [L, d]).  Returns (positions of the
    queries, o [nq, d], lse [nq]) with lse = logsumexp_j s_ij and
    o = sum_j softmax(s)_ij v_j ([AIS] formula).
    """
    qi, kj, s = window_scores(qk_bh, perm_r, cid_bh, k, chunk, causal, scale, query_slots,
                              dup_correct, wrap, bkt_bh, r)
    m = s.max(axis=1, keepdims=True)          # finite: the query itself is never dropped
    e = np.exp(s - m)
    z = e.sum(axis=1, keepdims=True)
    lse = (m + np.log(z))[:, 0]
    o = (e / z) @ np.asarray(v_bh[kj], dtype=np.float64)
    return qi, o, lse


def attention_rounds(qk: np.ndarray, v: np.ndarray, perm: np.ndarray, cid: np.ndarray,
                     chunk: int, causal: bool, scale: float, dup_correct: bool = True,
                     wrap: bool = False, buckets: Optional[np.ndarray] = None):
    """Every round's output in original position order.

    buckets [B, H, n_r, L] selects the same-bucket variant.
    -> o_r float64 [B, H, n_r, L, d], lse float64 [B, H, n_r, L].
    """
    B, H, L, d = qk.shape
    n_r = perm.shape[2]
    if L % chunk:
        raise ValueError("chunk must divide the sequence length")
    o_r = np.empty((B, H, n_r, L, d), dtype=np.float64)
    lse = np.empty((B, H, n_r, L), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            bkt = None if buckets is None else np.asarray(buckets[b, h]).T     # [L, n_r]
            for r in range(n_r):
                for k in range(L // chunk):
                    qi, o, l = chunk_attention(qk[b, h], v[b, h], perm[b, h, r], cid[b, h],
                                               k, chunk, causal, scale, dup_correct=dup_correct,
                                               wrap=wrap, bkt_bh=bkt, r=r)
                    o_r[b, h, r, qi] = o
                    lse[b, h, r, qi] = l
    return o_r, lse


def attention_one(qk_bh, v_bh, perm_bh, cid_bh, r: int, pos: int, chunk: int,
                  causal: bool, scale: float, dup_correct: bool = True, wrap: bool = False,
                  buckets_bh: Optional[np.ndarray] = None):
    """Round r's (o, lse) for the single query at position ``pos`` (sampled checks).
    buckets_bh [n_r, L] selects the same-bucket variant."""
    slot = int(cid_bh[pos, r]) * chunk
    seg = perm_bh[r]
    slot += int(np.nonzero(seg[slot:slot + chunk] == pos)[0][0])
    _, o, l = chunk_attention(qk_bh, v_bh, seg, cid_bh, slot // chunk, chunk, causal, scale,
                              query_slots=np.array([slot]), dup_correct=dup_correct, wrap=wrap,
                              bkt_bh=None if buckets_bh is None else np.asarray(buckets_bh).T, r=r)
    return o[0], float(l[0])


# --------------------------------------------------------------------------- 4. combine
def combine_rounds(o_r: np.ndarray, lse: np.ndarray):
    """Merge the rounds by logsumexp weights ([MOD] "Multi-round LSH attention").

    LSE = logsumexp_r lse_r;  o = sum_r exp(lse_r - LSE) * o_r.
    o_r [..., n_r, L, d], lse [..., n_r, L] -> (o [..., L, d], LSE [..., L]).
    """
    o_r = np.asarray(o_r, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    m = lse.max(axis=-2, keepdims=True)
    LSE = m + np.log(np.exp(lse - m).sum(axis=-2, keepdims=True))
    w = np.exp(lse - LSE)
    o = (w[..., None] * o_r).sum(axis=-3)
    return o, LSE[..., 0, :]


# --------------------------------------------------------------------------- forward
def default_scale(d_head: int) -> float:
    return 1.0 / np.sqrt(d_head)


def forward(qk: np.ndarray, v: np.ndarray, R: np.ndarray, n_buckets: int, chunk: int,
            causal: bool, scale: Optional[float] = None, dup_correct: bool = True,
            wrap: bool = False, same_bucket: bool = False):
    """All four steps.  Returns a dict with every intermediate (float64 / int)."""
    if scale is None:
        scale = default_scale(qk.shape[-1])
    buckets, margins = hash_buckets(qk, R)
    perm, cid = sort_rounds(buckets, n_buckets, chunk)
    o_r, lse = attention_rounds(qk, v, perm, cid, chunk, causal, scale, dup_correct=dup_correct,
                                wrap=wrap, buckets=buckets if same_bucket else None)
    o, LSE = combine_rounds(o_r, lse)
    return {"buckets": buckets, "margins": margins, "perm": perm, "cid": cid,
            "o_rounds": o_r, "lse": lse, "o": o, "LSE": LSE}


# --------------------------------------------------------------------------- backward
# The gradient of the forward above with respect to qk and v, for a loss whose
# gradient with respect to the combined output o is d_o.  The pages give no
# backward pass; this is the chain rule through the steps as defined here.  The
# buckets (hence perm and cid) are piecewise constant in qk and contribute no
# gradient.  Substituting the combine into the rounds gives
#     o_i = sum_r sum_{j in W_i^r} exp(s_ijr - LSE_i) v_j,   LSE_i = logsumexp_r lse_ir,
# one softmax over all (round, key) pairs of query i, so with
#     P_ijr = exp(s_ijr - LSE_i),  Delta_i = <d_o_i, o_i>,
#     dS_ijr = P_ijr (<d_o_i, v_j> - Delta_i):
#     dv_j  += P_ijr d_o_i
#     dqk_i += scale dS_ijr qk_j       (query role)
#     dqk_j += scale dS_ijr qk_i       (key role; both roles for j == i)
# The -log N_ij, self-penalty and causal terms are constants of the scores.
def chunk_attention_grad(qk_bh: np.ndarray, v_bh: np.ndarray, do_bh: np.ndarray,
                         LSE_bh: np.ndarray, delta_bh: np.ndarray, perm_r: np.ndarray,
                         cid_bh: np.ndarray, k: int, chunk: int, causal: bool, scale: float,
                         dup_correct: bool = True, wrap: bool = False,
                         bkt_bh: Optional[np.ndarray] = None, r: int = 0):
    """Round r's contributions to the gradients from the queries of sorted chunk
    k.  do_bh [L, d] is the gradient at the combined output, LSE_bh [L] the
    combined logsumexp, delta_bh [L] = <d_o_i, o_i>.  Returns (qi, kj, dq [nq, d]
    (query role), dk [nk, d] (key role), dv [nk, d])."""
    qi, kj, s = window_scores(qk_bh, perm_r, cid_bh, k, chunk, causal, scale, None,
                              dup_correct, wrap, bkt_bh, r)
    P = np.exp(s - np.asarray(LSE_bh, dtype=np.float64)[qi][:, None])
    do_q = np.asarray(do_bh[qi], dtype=np.float64)
    dP = do_q @ np.asarray(v_bh[kj], dtype=np.float64).T
    dS = P * (dP - np.asarray(delta_bh, dtype=np.float64)[qi][:, None])
    dq = scale * (dS @ np.asarray(qk_bh[kj], dtype=np.float64))
    dk = scale * (dS.T @ np.asarray(qk_bh[qi], dtype=np.float64))
    dv = P.T @ do_q
    return qi, kj, dq, dk, dv


def attention_backward(qk: np.ndarray, v: np.ndarray, perm: np.ndarray, cid: np.ndarray,
                       d_o: np.ndarray, chunk: int, causal: bool, scale: float,
                       dup_correct: bool = True, wrap: bool = False,
                       buckets: Optional[np.ndarray] = None):
    """Gradients of steps 3-4 for fixed perm/cid (the forward is recomputed).

    qk, v, d_o [B, H, L, d].  -> dict with dqk, dv [B, H, L, d] float64, the
    per-round contributions dqk_rounds, dv_rounds [B, H, n_r, L, d] (each
    round's share: a position's query- and key-role terms of that round), and
    the recomputed o, LSE and Delta.
    """
    B, H, L, d = qk.shape
    n_r = perm.shape[2]
    o_r, lse = attention_rounds(qk, v, perm, cid, chunk, causal, scale, dup_correct=dup_correct,
                                wrap=wrap, buckets=buckets)
    o, LSE = combine_rounds(o_r, lse)
    d_o = np.asarray(d_o, dtype=np.float64)
    delta = np.sum(d_o * o, axis=-1)
    dqk_r = np.zeros((B, H, n_r, L, d))
    dv_r = np.zeros((B, H, n_r, L, d))
    for b in range(B):
        for h in range(H):
            bkt = None if buckets is None else np.asarray(buckets[b, h]).T     # [L, n_r]
            for r in range(n_r):
                for k in range(L // chunk):
                    qi, kj, dq, dk, dv = chunk_attention_grad(
                        qk[b, h], v[b, h], d_o[b, h], LSE[b, h], delta[b, h], perm[b, h, r],
                        cid[b, h], k, chunk, causal, scale, dup_correct, wrap, bkt, r)
                    # positions are distinct within qi and within kj
                    dqk_r[b, h, r, qi] += dq
                    dqk_r[b, h, r, kj] += dk
                    dv_r[b, h, r, kj] += dv
    return {"dqk": dqk_r.sum(axis=2), "dv": dv_r.sum(axis=2), "dqk_rounds": dqk_r,
            "dv_rounds": dv_r, "o": o, "LSE": LSE, "delta": delta}


def attention_backward_one(qk_bh: np.ndarray, v_bh: np.ndarray, do_bh: np.ndarray,
                           perm_bh: np.ndarray, cid_bh: np.ndarray, pos: int, chunk: int,
                           causal: bool, scale: float, dup_correct: bool = True):
    """dqk[pos] and dv[pos] of one (batch row, head) (sampled checks): the terms
    of attention_backward that reach position pos.  In round r they come from
    the query chunks whose window holds pos, cid[pos, r] and the one after it;
    those queries' LSE and Delta are computed from their own rounds first."""
    n_r, L = perm_bh.shape
    nchunks = L // chunk
    need = set()
    for r in range(n_r):
        k = int(cid_bh[pos, r])
        for kk in (k, k + 1):
            if kk < nchunks:
                need.update(int(p) for p in perm_bh[r, kk * chunk:(kk + 1) * chunk])
    LSE = np.full(L, np.nan)
    delta = np.full(L, np.nan)
    do_bh = np.asarray(do_bh, dtype=np.float64)
    for q in sorted(need):
        o_q = np.empty((n_r, qk_bh.shape[1]))
        l_q = np.empty(n_r)
        for r in range(n_r):
            o_q[r], l_q[r] = attention_one(qk_bh, v_bh, perm_bh, cid_bh, r, q, chunk, causal, scale,
                                           dup_correct=dup_correct)
        o, lse_c = combine_rounds(o_q[:, None, :], l_q[:, None])
        LSE[q] = lse_c[0]
        delta[q] = float(do_bh[q] @ o[0])
    dqk = np.zeros(qk_bh.shape[1])
    dv = np.zeros(qk_bh.shape[1])
    for r in range(n_r):
        k = int(cid_bh[pos, r])
        for kk in (k, k + 1):
            if kk >= nchunks:
                continue
            qi, kj, dq, dk, dvv = chunk_attention_grad(qk_bh, v_bh, do_bh, LSE, delta, perm_bh[r],
                                                       cid_bh, kk, chunk, causal, scale,
                                                       dup_correct, False, None, r)
            dqk += dq[qi == pos].sum(axis=0) + dk[kj == pos].sum(axis=0)
            dv += dvv[kj == pos].sum(axis=0)
    return dqk, dv


def backward(qk: np.ndarray, v: np.ndarray, R: np.ndarray, d_o: np.ndarray, n_buckets: int,
             chunk: int, causal: bool, scale: Optional[float] = None, dup_correct: bool = True,
             wrap: bool = False, same_bucket: bool = False):
    """Hash and sort as in forward, then attention_backward."""
    if scale is None:
        scale = default_scale(qk.shape[-1])
    buckets, _ = hash_buckets(qk, R)
    perm, cid = sort_rounds(buckets, n_buckets, chunk)
    out = attention_backward(qk, v, perm, cid, d_o, chunk, causal, scale, dup_correct, wrap,
                             buckets if same_bucket else None)
    out.update({"buckets": buckets, "perm": perm, "cid": cid})
    return out


# --------------------------------------------------------------------------- the layer around it
# The attention layer ([MOD] "LSH attention": queries and keys come from one
# shared projection; [AIS] set-up: d_model 1024, 8 heads): x is projected to
# the shared qk and to v, split into heads (column h*d + c of the projection is
# element c of head h), attended head by head, the heads merged back and
# projected out.  Weights are [out, in] like a linear layer's.
def split_heads(t: np.ndarray, heads: int) -> np.ndarray:
    """[B, L, H*d] -> [B, H, L, d] (column h*d + c is element c of head h)."""
    B, L, hd = t.shape
    return t.reshape(B, L, heads, hd // heads).transpose(0, 2, 1, 3)


def merge_heads(t: np.ndarray) -> np.ndarray:
    """[B, H, L, d] -> [B, L, H*d], the inverse of split_heads."""
    B, H, L, d = t.shape
    return t.transpose(0, 2, 1, 3).reshape(B, L, H * d)


def project_in(x: np.ndarray, w_qk: np.ndarray, w_v: np.ndarray, heads: int):
    """qk = x w_qk^T and v = x w_v^T in float64, split into heads: [B, H, L, d] each."""
    x = np.asarray(x, dtype=np.float64)
    qk = x @ np.asarray(w_qk, dtype=np.float64).T
    v = x @ np.asarray(w_v, dtype=np.float64).T
    return split_heads(qk, heads), split_heads(v, heads)


def project_out(o: np.ndarray, w_o: np.ndarray) -> np.ndarray:
    """y = merge_heads(o) w_o^T in float64: [B, L, d_model]."""
    return merge_heads(np.asarray(o, dtype=np.float64)) @ np.asarray(w_o, dtype=np.float64).T


def layer_forward(x: np.ndarray, w_qk: np.ndarray, w_v: np.ndarray, w_o: np.ndarray,
                  R: np.ndarray, heads: int, n_buckets: int, chunk: int, causal: bool,
                  scale: Optional[float] = None, **variants):
    """The whole layer; returns the forward() dict plus qk, v and y."""
    qk, v = project_in(x, w_qk, w_v, heads)
    out = forward(qk, v, R, n_buckets, chunk, causal, scale=scale, **variants)
    out.update(qk=qk, v=v, y=project_out(out["o"], w_o))
    return out


# --------------------------------------------------------------------------- the Reformer block
# [ULT] "Capas reversibles y división en fragmentos" and [MOD] "Reversible
# Transformer", "Chunking": the activations are split into two halves (x1, x2);
# attention updates one half and the feed-forward layer the other,
#     y1 = x1 + Attention(x2),   y2 = x2 + FeedForward(y1),
# so the inputs can be recomputed from the outputs in the backward pass,
#     x2 = y2 - FeedForward(y1),  then  x1 = y1 - Attention(x2),
# and only the last layer's activations are stored.  The feed-forward layer acts
# on each position independently, so it is evaluated over chunks of positions
# (its hidden layer is several times wider than the model: d_ff 4096 at
# d_model 1024 in [AIS]'s set-up).  The pages do not write the feed-forward
# out; it is read here as the transformer's position-wise form
#     FeedForward(x) = relu(x w1^T + b1) w2^T + b2,
# weights [out, in] like a linear layer's.  Attention(x) is the attention layer
# above (projections, the four steps, output projection).
def feed_forward(x: np.ndarray, w1: np.ndarray, b1: np.ndarray, w2: np.ndarray,
                 b2: np.ndarray) -> np.ndarray:
    """relu(x w1^T + b1) w2^T + b2 in float64, on the last axis of x."""
    x = np.asarray(x, dtype=np.float64)
    h = np.maximum(x @ np.asarray(w1, dtype=np.float64).T + np.asarray(b1, dtype=np.float64), 0.0)
    return h @ np.asarray(w2, dtype=np.float64).T + np.asarray(b2, dtype=np.float64)


def feed_forward_chunked(x: np.ndarray, w1, b1, w2, b2, chunk_rows: int) -> np.ndarray:
    """feed_forward over chunks of chunk_rows positions of x [..., d_model] (rows
    flattened), one chunk's hidden activations at a time."""
    x = np.asarray(x, dtype=np.float64)
    rows = x.reshape(-1, x.shape[-1])
    out = np.empty((rows.shape[0], np.asarray(w2).shape[0]))
    for r0 in range(0, rows.shape[0], chunk_rows):
        out[r0:r0 + chunk_rows] = feed_forward(rows[r0:r0 + chunk_rows], w1, b1, w2, b2)
    return out.reshape(x.shape[:-1] + (out.shape[-1],))


def attention_block(x: np.ndarray, wa: dict, R: np.ndarray, heads: int, n_buckets: int,
                    chunk: int, causal: bool, scale: Optional[float] = None, **variants):
    """Attention(x): the attention layer's output y [B, L, d_model].  wa holds
    w_qk, w_v, w_o."""
    return layer_forward(x, wa["w_qk"], wa["w_v"], wa["w_o"], R, heads, n_buckets, chunk, causal,
                         scale=scale, **variants)["y"]


def block_forward(x1: np.ndarray, x2: np.ndarray, wa: dict, wf: dict, R: np.ndarray, heads: int,
                  n_buckets: int, chunk: int, causal: bool, chunk_rows: int,
                  scale: Optional[float] = None, **variants):
    """(y1, y2) = (x1 + Attention(x2), x2 + FeedForward(y1)).  wf holds w1, b1, w2, b2."""
    y1 = np.asarray(x1, dtype=np.float64) + attention_block(x2, wa, R, heads, n_buckets, chunk,
                                                            causal, scale, **variants)
    y2 = np.asarray(x2, dtype=np.float64) + feed_forward_chunked(y1, wf["w1"], wf["b1"], wf["w2"],
                                                                 wf["b2"], chunk_rows)
    return y1, y2


def block_inverse(y1: np.ndarray, y2: np.ndarray, wa: dict, wf: dict, R: np.ndarray, heads: int,
                  n_buckets: int, chunk: int, causal: bool, chunk_rows: int,
                  scale: Optional[float] = None, **variants):
    """The block's inputs recomputed from its outputs: x2 = y2 - FeedForward(y1),
    then x1 = y1 - Attention(x2)."""
    x2 = np.asarray(y2, dtype=np.float64) - feed_forward_chunked(y1, wf["w1"], wf["b1"], wf["w2"],
                                                                 wf["b2"], chunk_rows)
    x1 = np.asarray(y1, dtype=np.float64) - attention_block(x2, wa, R, heads, n_buckets, chunk,
                                                            causal, scale, **variants)
    return x1, x2
