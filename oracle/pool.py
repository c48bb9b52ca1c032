"""The oracle's forward pass over many (batch row, head) slices in worker processes.

TEST INFRASTRUCTURE, like the oracle itself: the benchmark's CPU-baseline leg
and the CPU tests use it.  It adds no arithmetic of its own.  Every (batch row,
head) is independent through all four steps (R is shared, nothing else crosses
heads), and within a slice every round's hash and sort are independent, so the
work is split into jobs that call the oracle's own functions:
  phase A  (slice, round)         hash_buckets and sort_rounds of that round
  phase B  (slice, rounds group)  attention_rounds of those rounds, with the
                                  chunk ids of every round (duplicate counts)
  phase C  (slice)                combine_rounds
Inputs and outputs live in memory-mapped files under /dev/shm that every
worker maps, so only indices travel between processes.  Workers are spawned
processes limited to one BLAS thread each.  A process that has initialised a
GPU must not start them (spawning execs a new interpreter): the benchmark runs
this before its first GPU call.
"""
from __future__ import annotations

import concurrent.futures as cf
import multiprocessing as mp
import os
import shutil
import tempfile
import time
from typing import Dict, Optional

import numpy as np

from . import lsh_oracle as O

_BLAS_ENV = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "BLIS_NUM_THREADS")


# Worker processes are capped at the CPU share a one-GPU host gives this job.
MAX_WORKERS = 16


def host_cores() -> int:
    """Cores this process may run on (its affinity mask, not the machine's count)."""
    return len(os.sched_getaffinity(0))


def _one_blas_thread() -> None:
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # pragma: no cover - threadpoolctl is optional
        pass


def _noop(i):
    return i


def _maps(spec: dict) -> Dict[str, np.ndarray]:
    return {k: np.memmap(path, dtype=dt, mode="r+", shape=shape) for k, (path, dt, shape) in spec.items()}


def hash_sort_round(spec: dict, b: int, h: int, r: int, n_buckets: int, chunk: int) -> None:
    """Steps 1-2 of slice (b, h) in round r, into the shared buckets, margins,
    perm and cid."""
    m = _maps(spec)
    qk = np.asarray(m["qk"][b, h], dtype=np.float64)
    bk, mg = O.hash_buckets(qk[None, None], np.asarray(m["R"][r], dtype=np.float64)[None])
    p, c = O.sort_rounds(bk, n_buckets, chunk)
    m["buckets"][b, h, r] = bk[0, 0, 0]
    m["margins"][b, h, r] = mg[0, 0, 0]
    m["perm"][b, h, r] = p[0, 0, 0]
    m["cid"][b, h, :, r] = c[0, 0, :, 0]
    for a in m.values():
        a.flush()


def attention_some_rounds(spec: dict, b: int, h: int, rounds, chunk: int, causal: bool, scale: float,
                          dup_correct: bool = True, wrap: bool = False,
                          same_bucket: bool = False) -> None:
    """Step 3 of slice (b, h) for the listed rounds: attention_rounds on each
    round's sorted order, with every round's chunk ids (and buckets) reordered
    so that round r comes first (the duplicate counts sum over all rounds in
    any order; the same-bucket mask reads the first)."""
    m = _maps(spec)
    qk = np.asarray(m["qk"][b, h], dtype=np.float64)[None, None]
    v = np.asarray(m["v"][b, h], dtype=np.float64)[None, None]
    perm = np.asarray(m["perm"][b, h])
    cid = np.asarray(m["cid"][b, h])
    n_r = perm.shape[0]
    for r in rounds:
        order = [r] + [s for s in range(n_r) if s != r]
        bk = np.asarray(m["buckets"][b, h])[order][None, None] if same_bucket else None
        o_r, lse = O.attention_rounds(qk, v, perm[r][None, None, None], cid[:, order][None, None],
                                      chunk, causal, scale, dup_correct=dup_correct, wrap=wrap,
                                      buckets=bk)
        m["o_rounds"][b, h, r] = o_r[0, 0, 0]
        m["lse"][b, h, r] = lse[0, 0, 0]
    m["o_rounds"].flush()
    m["lse"].flush()


def combine_slice(spec: dict, b: int, h: int) -> None:
    """Step 4 of slice (b, h)."""
    m = _maps(spec)
    o, LSE = O.combine_rounds(np.asarray(m["o_rounds"][b, h]), np.asarray(m["lse"][b, h]))
    m["o"][b, h] = o
    m["LSE"][b, h] = LSE
    m["o"].flush()
    m["LSE"].flush()


class OraclePool:
    """A pool of spawned workers (one BLAS thread each), started and warmed up
    once so that timings exclude interpreter start-up."""

    def __init__(self, workers: int = 0):
        self.workers = min(workers or host_cores(), MAX_WORKERS)
        saved = {k: os.environ.get(k) for k in _BLAS_ENV}
        os.environ.update({k: "1" for k in _BLAS_ENV})      # inherited by the workers
        try:
            self.ex = cf.ProcessPoolExecutor(self.workers, mp_context=mp.get_context("spawn"),
                                             initializer=_one_blas_thread)
            list(self.ex.map(_noop, range(4 * self.workers)))
        finally:
            for k, v in saved.items():
                if v is None:
                    os.environ.pop(k, None)
                else:
                    os.environ[k] = v

    def close(self):
        self.ex.shutdown()

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def _run(self, fn, jobs):
        for f in [self.ex.submit(fn, *a) for a in jobs]:
            f.result()

    def forward(self, qk: np.ndarray, v: np.ndarray, R: np.ndarray, n_buckets: int, chunk: int,
                causal: bool, scale: Optional[float] = None, dup_correct: bool = True,
                wrap: bool = False, same_bucket: bool = False,
                keep=("buckets", "margins", "perm", "cid", "o_rounds", "lse", "o", "LSE")
                ) -> Dict[str, np.ndarray]:
        """The oracle's forward() of every (batch row, head), split into jobs.
        qk, v [B, H, L, d] (float32 holding the stored values, or float64),
        R [n_r, d, nb/2].  Returns the arrays named in `keep` among buckets,
        margins, perm, cid, o_rounds, lse, o and LSE, as forward() does, and
        "seconds": the wall-clock time of each phase and in total."""
        if scale is None:
            scale = O.default_scale(qk.shape[-1])
        B, H, L, d = qk.shape
        n_r = R.shape[0]
        shapes = {"qk": (qk.dtype, qk.shape), "v": (v.dtype, v.shape), "R": (np.float64, R.shape),
                  "buckets": (np.int32, (B, H, n_r, L)), "margins": (np.float64, (B, H, n_r, L)),
                  "perm": (np.int32, (B, H, n_r, L)), "cid": (np.int16, (B, H, L, n_r)),
                  "o_rounds": (np.float64, (B, H, n_r, L, d)), "lse": (np.float64, (B, H, n_r, L)),
                  "o": (np.float64, (B, H, L, d)), "LSE": (np.float64, (B, H, L))}
        tmp = tempfile.mkdtemp(prefix="lsh_oracle_", dir="/dev/shm" if os.path.isdir("/dev/shm") else None)
        try:
            spec = {k: (os.path.join(tmp, k), np.dtype(dt).str, tuple(sh)) for k, (dt, sh) in shapes.items()}
            for k, path in (("qk", qk), ("v", v), ("R", R)):
                mm = np.memmap(spec[k][0], dtype=spec[k][1], mode="w+", shape=spec[k][2])
                mm[...] = path
                mm.flush()
                del mm
            for k in shapes:
                if k not in ("qk", "v", "R"):
                    np.memmap(spec[k][0], dtype=spec[k][1], mode="w+", shape=spec[k][2]).flush()
            slices = [(b, h) for b in range(B) for h in range(H)]
            # rounds in groups, so that every worker has about one job per slice
            per = max(1, (len(slices) * n_r) // self.workers)
            groups = [list(range(r, min(r + per, n_r))) for r in range(0, n_r, per)]
            t = {}
            t0 = time.perf_counter()
            self._run(hash_sort_round, [(spec, b, h, r, n_buckets, chunk) for b, h in slices
                                        for r in range(n_r)])
            t1 = time.perf_counter()
            self._run(attention_some_rounds, [(spec, b, h, g, chunk, causal, scale, dup_correct, wrap,
                                               same_bucket) for b, h in slices for g in groups])
            t2 = time.perf_counter()
            self._run(combine_slice, [(spec, b, h) for b, h in slices])
            t3 = time.perf_counter()
            t = {"hash_sort": t1 - t0, "attention": t2 - t1, "combine": t3 - t2, "total": t3 - t0}
            m = _maps(spec)
            out = {k: np.array(m[k]) for k in keep}
            del m
        finally:
            shutil.rmtree(tmp, ignore_errors=True)
        out["seconds"] = t
        return out
