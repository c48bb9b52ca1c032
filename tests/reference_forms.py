"""Independent closed forms the oracle must reduce to.

These are written from the definitions, not from the oracle: they share no
function with it.  Each is slow (Python loops) and meant for small inputs.

* full_attention_self_masked: textbook scaled dot-product attention
  softmax(scale * q k^T) v (ai-scholar Reformer article, section on the problems
  of the Transformer), over every key except the query itself (modulabs notes,
  section "LSH attention": the query is removed because with shared QK it is
  always its own best match), and over earlier positions only when causal.  A
  query left with no key returns its own value.  With one chunk spanning the
  whole sequence, every round's window is the whole sequence, so the LSH
  forward must equal this for any bucket count and any number of rounds.

* union_attention: for L <= 64, the windows of every round are enumerated by
  brute force (Python's sorted() on (bucket, position), then slot // chunk),
  and each query attends, with plain softmax weights, to the union of the keys
  its windows hold across rounds (minus itself unless nothing else is there).
  The duplicate-count corrected multi-round output must equal this.  With
  wrap, the chunk before the first is the last one; with the same-bucket
  mask, a window keeps only the keys in the query's bucket of that round.

* round_attention: one round without the duplicate-count term, plain softmax
  over the round's window; the variant without the correction must give it
  round by round.
"""
from __future__ import annotations

import numpy as np


def full_attention_self_masked(qk: np.ndarray, v: np.ndarray, causal: bool, scale: float) -> np.ndarray:
    qk = np.asarray(qk, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    L = qk.shape[0]
    out = np.empty_like(v)
    for i in range(L):
        js = [j for j in range(L) if j != i and (not causal or j <= i)]
        if not js:
            out[i] = v[i]
            continue
        s = scale * (qk[js] @ qk[i])
        w = np.exp(s - s.max())
        w /= w.sum()
        out[i] = w @ v[js]
    return out


def brute_chunk_of(buckets_r, chunk: int) -> list:
    """chunk_of[pos] for one round: sorted by (bucket, position), slot // chunk."""
    L = len(buckets_r)
    order = sorted(range(L), key=lambda i: (int(buckets_r[i]), i))
    chunk_of = [0] * L
    for slot, pos in enumerate(order):
        chunk_of[pos] = slot // chunk
    return chunk_of


def brute_windows(buckets: np.ndarray, chunk: int, causal: bool, wrap: bool = False,
                  same_bucket: bool = False):
    """W[r][i] = set of keys in query i's window in round r (after the causal cut).

    Key j is in the window when its chunk is the query's chunk or the one just
    before it; with wrap, the chunk before the first is the last, i.e. the
    chunk distance is counted around a circle of L / chunk chunks; with
    same_bucket, j must also share the query's bucket in that round.
    """
    n_r, L = buckets.shape
    nchunks = L // chunk
    W = []
    for r in range(n_r):
        c = brute_chunk_of(buckets[r], chunk)
        W.append([{j for j in range(L)
                   if ((c[i] - c[j]) % nchunks if wrap else c[i] - c[j]) in (0, 1)
                   and (not causal or j <= i)
                   and (not same_bucket or int(buckets[r][j]) == int(buckets[r][i]))}
                  for i in range(L)])
    return W


def round_attention(qk: np.ndarray, v: np.ndarray, window: list, scale: float):
    """One round without the duplicate-count term: query i attends with plain
    softmax weights to the keys of its window other than itself (to itself only
    when the window holds nothing else).  window[i] is a set of positions.
    Returns (o [L, d], lse [L]) with lse the log of the softmax denominator."""
    qk = np.asarray(qk, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    L = qk.shape[0]
    out = np.empty_like(v)
    lse = np.empty(L)
    for i in range(L):
        keys = sorted(window[i] - {i}) or [i]
        s = scale * (qk[keys] @ qk[i])
        if keys == [i]:
            s = s - 1.0e5            # the self penalty of the method, alone in the window
        m = s.max()
        w = np.exp(s - m)
        lse[i] = m + np.log(w.sum())
        out[i] = (w / w.sum()) @ v[keys]
    return out, lse


def union_attention(qk: np.ndarray, v: np.ndarray, buckets: np.ndarray, chunk: int,
                    causal: bool, scale: float, wrap: bool = False,
                    same_bucket: bool = False) -> np.ndarray:
    """buckets [n_r, L] of one (batch row, head)."""
    qk = np.asarray(qk, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    W = brute_windows(buckets, chunk, causal, wrap, same_bucket)
    L = qk.shape[0]
    out = np.empty_like(v)
    for i in range(L):
        union = set()
        for Wr in W:
            union |= Wr[i]
        others = sorted(union - {i})
        if not others:
            out[i] = v[i]
            continue
        s = scale * (qk[others] @ qk[i])
        w = np.exp(s - s.max())
        w /= w.sum()
        out[i] = w @ v[others]
    return out


def union_attention_torch(qk, v, windows: list, scale: float):
    """The union closed form above as differentiable float64 torch code (for
    gradient checks by autograd).  qk, v: torch tensors [L, d] (requires_grad as
    needed); windows: brute_windows(...) of one (batch row, head)."""
    import torch
    L = qk.shape[0]
    rows = []
    for i in range(L):
        union = set()
        for Wr in windows:
            union |= Wr[i]
        others = sorted(union - {i})
        if not others:
            rows.append(v[i])
            continue
        idx = torch.tensor(others, dtype=torch.long)
        s = scale * (qk[idx] @ qk[i])
        rows.append(torch.softmax(s, dim=0) @ v[idx])
    return torch.stack(rows)
