"""Seeded synthetic inputs for the multi-round shared-QK LSH-attention forward.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark.  It draws random numbers and rounds them to the storage dtype; it holds
no step of the method itself (no hashing, sorting, attention or combining).

Workloads
---------
The five workloads below carry the shapes of the Reformer pages' set-up:
shared query/key vectors of one projection, random rotations R with
n_buckets/2 columns per hash round, chunked attention, several hash rounds.
The pages train on enwik8-64k and imagenet64; those datasets are not used.
Standard-normal activations stand in for them (the pages do not give an
activation distribution).  "paper_64k" takes the experiment shape of the
ai-scholar Reformer article, section on results (d_model 1024 over 8 heads,
64K tokens, one GPU's share of batch 8); "long_1m" takes the ~1M-token
context claim of the Ultralytics "Reformer" glossary page (introduction).

Recipe (every workload):
  rng = numpy Generator(PCG64(seed)); draws in float32, in this order:
    qk  ~ N(0, 1), shape [B, H, L, d]  (clustered workload: see below)
    v   ~ N(0, 1), shape [B, H, L, d]
    R   ~ N(0, 1), shape [n_rounds, d, n_buckets // 2]  (one R per round,
          shared by every batch row and head)
  Clustered workload: 256 centroids ~ N(0, I_d), normalised to unit length;
  each (b, h, i) picks a centroid uniformly; qk = centroid + 0.3 * N(0, I_d).
  bf16 workloads then round qk, v and R to bfloat16 (round to nearest even);
  the arrays returned are float32 holding exactly those bf16 values, so the
  GPU side (which converts to torch.bfloat16 exactly) and the oracle (which
  upcasts to float64 exactly) see the same numbers.
"""
from __future__ import annotations

import dataclasses
from typing import Dict

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    seq_len: int
    d_head: int
    dtype: str          # "f32" or "bf16" (storage dtype; bf16 accumulates in fp32)
    n_buckets: int
    n_rounds: int
    chunk: int
    causal: bool
    seed: int
    clustered: bool = False
    n_centroids: int = 256
    noise: float = 0.3
    description: str = ""

    @property
    def tokens(self) -> int:
        return self.batch * self.seq_len

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads, in the order of their seeds 1..5.
WORKLOADS: Dict[str, Workload] = {
    "tiny_f32": Workload(
        "tiny_f32", batch=1, heads=1, seq_len=1024, d_head=64, dtype="f32",
        n_buckets=32, n_rounds=1, chunk=64, causal=False, seed=1,
        description="B1 H1 L1024 d64 fp32, 32 buckets, 1 round, chunk 64, non-causal"),
    "short_4k": Workload(
        "short_4k", batch=1, heads=8, seq_len=4096, d_head=64, dtype="bf16",
        n_buckets=64, n_rounds=2, chunk=64, causal=True, seed=2,
        description="B1 H8 L4096 d64 bf16, 64 buckets, 2 rounds, chunk 64, causal"),
    "paper_64k": Workload(
        "paper_64k", batch=1, heads=8, seq_len=65536, d_head=128, dtype="bf16",
        n_buckets=1024, n_rounds=8, chunk=64, causal=True, seed=3,
        description="B1 H8 L65536 d128 bf16, 1024 buckets, 8 rounds, chunk 64, causal "
                    "(d_model 1024 / 8 heads; one GPU's share of batch 8)"),
    "clustered_16k": Workload(
        "clustered_16k", batch=2, heads=8, seq_len=16384, d_head=64, dtype="bf16",
        n_buckets=256, n_rounds=4, chunk=64, causal=False, seed=4, clustered=True,
        description="B2 H8 L16384 d64 bf16, qk = one of 256 unit centroids + 0.3 N(0,I), "
                    "256 buckets, 4 rounds, chunk 64, non-causal"),
    "long_1m": Workload(
        "long_1m", batch=1, heads=8, seq_len=1 << 20, d_head=64, dtype="bf16",
        n_buckets=16384, n_rounds=4, chunk=128, causal=True, seed=5,
        description="B1 H8 L1048576 d64 bf16, 16384 buckets, 4 rounds, chunk 128, causal"),
}


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32.

    Storage conversion only.  Non-finite inputs are not expected here.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    rounded = (bits + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return rounded.view(np.float32)


def _storage(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return round_to_bf16(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def _normal(rng: np.random.Generator, shape, block: int = 1 << 26) -> np.ndarray:
    """float32 N(0,1) draws, filled in row-major order in blocks (bounded temporaries)."""
    out = np.empty(shape, dtype=np.float32)
    flat = out.reshape(-1)
    for s in range(0, flat.size, block):
        e = min(s + block, flat.size)
        rng.standard_normal(e - s, dtype=np.float32, out=flat[s:e])
    return out


def make_inputs(w: Workload, seed: int | None = None) -> Dict[str, np.ndarray]:
    """Draw qk, v and R for workload ``w`` (see the module docstring for the recipe).

    Returns float32 arrays: qk [B,H,L,d], v [B,H,L,d], R [n_rounds, d, n_buckets//2],
    with values exactly representable in ``w.dtype``.
    """
    if w.n_buckets % 2 or w.n_buckets < 2:
        raise ValueError("n_buckets must be even and >= 2")
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    B, H, L, d = w.batch, w.heads, w.seq_len, w.d_head
    if w.clustered:
        cent = rng.standard_normal((w.n_centroids, d)).astype(np.float64)
        cent /= np.linalg.norm(cent, axis=1, keepdims=True)
        cent = cent.astype(np.float32)
        assign = rng.integers(0, w.n_centroids, size=(B, H, L))
        qk = _normal(rng, (B, H, L, d))
        qk *= np.float32(w.noise)
        qk += cent[assign]
    else:
        qk = _normal(rng, (B, H, L, d))
    v = _normal(rng, (B, H, L, d))
    R = _normal(rng, (w.n_rounds, d, w.n_buckets // 2))
    return {"qk": _storage(qk, w.dtype), "v": _storage(v, w.dtype), "R": _storage(R, w.dtype)}


def make_layer_inputs(w: Workload, d_model: int, seed: int | None = None) -> Dict[str, np.ndarray]:
    """Draw the inputs of the attention layer around workload ``w``:
    x [B, L, d_model] ~ N(0, 1); the weights w_qk, w_v [H*d, d_model] and
    w_o [d_model, H*d] ~ N(0, 1/fan_in), so that the projections keep unit
    scale; R as in make_inputs.  Drawn in that order from PCG64(seed, default
    the workload's seed + 1000), rounded to ``w.dtype``; float32 arrays."""
    rng = np.random.Generator(np.random.PCG64((w.seed + 1000) if seed is None else seed))
    B, H, L, d = w.batch, w.heads, w.seq_len, w.d_head
    hd = H * d
    x = _normal(rng, (B, L, d_model))
    w_qk = _normal(rng, (hd, d_model)) * np.float32(1.0 / np.sqrt(d_model))
    w_v = _normal(rng, (hd, d_model)) * np.float32(1.0 / np.sqrt(d_model))
    w_o = _normal(rng, (d_model, hd)) * np.float32(1.0 / np.sqrt(hd))
    R = _normal(rng, (w.n_rounds, d, w.n_buckets // 2))
    return {k: _storage(a, w.dtype) for k, a in
            (("x", x), ("w_qk", w_qk), ("w_v", w_v), ("w_o", w_o), ("R", R))}


def make_grad(w: Workload, seed: int | None = None) -> np.ndarray:
    """A loss gradient at the combined output, d_o [B, H, L, d] ~ N(0, 1), drawn
    from PCG64(seed, default the workload's seed + 2000) and rounded to
    ``w.dtype``; float32 array."""
    rng = np.random.Generator(np.random.PCG64((w.seed + 2000) if seed is None else seed))
    return _storage(_normal(rng, (w.batch, w.heads, w.seq_len, w.d_head)), w.dtype)


def make_block_inputs(w: Workload, d_model: int, d_ff: int, seed: int | None = None) -> Dict[str, np.ndarray]:
    """Inputs of a Reformer block around workload ``w``: the halves x1, x2
    [B, L, d_model] ~ N(0, 1); the attention weights w_qk, w_v [H*d, d_model],
    w_o [d_model, H*d] and the feed-forward weights w1 [d_ff, d_model],
    w2 [d_model, d_ff] ~ N(0, 1/fan_in); biases b1 [d_ff], b2 [d_model] ~
    N(0, 0.01); R as in make_inputs.  Drawn in that order from PCG64(seed,
    default the workload's seed + 3000), rounded to ``w.dtype``; float32 arrays."""
    rng = np.random.Generator(np.random.PCG64((w.seed + 3000) if seed is None else seed))
    B, H, L, d = w.batch, w.heads, w.seq_len, w.d_head
    hd = H * d
    out = {"x1": _normal(rng, (B, L, d_model)), "x2": _normal(rng, (B, L, d_model)),
           "w_qk": _normal(rng, (hd, d_model)) * np.float32(1.0 / np.sqrt(d_model)),
           "w_v": _normal(rng, (hd, d_model)) * np.float32(1.0 / np.sqrt(d_model)),
           "w_o": _normal(rng, (d_model, hd)) * np.float32(1.0 / np.sqrt(hd)),
           "w1": _normal(rng, (d_ff, d_model)) * np.float32(1.0 / np.sqrt(d_model)),
           "b1": _normal(rng, (d_ff,)) * np.float32(0.1),
           "w2": _normal(rng, (d_model, d_ff)) * np.float32(1.0 / np.sqrt(d_ff)),
           "b2": _normal(rng, (d_model,)) * np.float32(0.1),
           "R": _normal(rng, (w.n_rounds, d, w.n_buckets // 2))}
    return {k: _storage(a, w.dtype) for k, a in out.items()}
