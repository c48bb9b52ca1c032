"""ctypes binding of liblsh_attention.so (declared in include/lsh_attention.h).

Argument marshalling only: every step of the forward pass runs in the HIP
kernels behind the C ABI.  torch provides device memory and streams.  The
wrappers check shapes, dtypes, devices and contiguity of the tensors on the
host, because the C ABI receives bare pointers and cannot.

There is no fallback: if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import functools
import dataclasses
import math
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblsh_attention.so")
# the same library with the device-side bounds checks compiled in (build --debug)
DEBUG_LIB_PATH = os.path.join(_PKG, "liblsh_attention_debug.so")

LSH_OK, LSH_ERR_INVALID_ARG, LSH_ERR_UNSUPPORTED, LSH_ERR_WORKSPACE, LSH_ERR_HIP = range(5)
LSH_F32, LSH_BF16 = 0, 1
# variant flags of lsh_config.flags (see include/lsh_attention.h)
LSH_FLAG_NO_DUP_CORRECTION, LSH_FLAG_WRAP_LOOKBACK, LSH_FLAG_SAME_BUCKET = 1, 2, 4

EXPORTED = ("lsh_hash", "lsh_sort_workspace_bytes", "lsh_sort", "lsh_sort_noalloc", "lsh_chunk_attn",
            "lsh_combine_rounds", "lsh_backward_workspace_bytes", "lsh_attn_backward",
            "lsh_project_in", "lsh_project_out", "lsh_project_out_add", "lsh_ffn_workspace_bytes",
            "lsh_ffn", "lsh_status_string", "lsh_last_error", "lsh_debug_check_failures")


class LSHError(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        super().__init__(f"{where}: {message} (status {status})")
        self.status = status


class CConfig(ctypes.Structure):
    """Mirror of struct lsh_config."""
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("seq_len", ctypes.c_int32), ("d_head", ctypes.c_int32),
                ("n_buckets", ctypes.c_int32), ("n_rounds", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("causal", ctypes.c_int32),
                ("scale", ctypes.c_float), ("dtype", ctypes.c_int32),
                ("flags", ctypes.c_int32)]


@dataclasses.dataclass(frozen=True)
class LSHConfig:
    batch: int
    heads: int
    seq_len: int
    d_head: int
    n_buckets: int
    n_rounds: int
    chunk: int
    causal: bool
    dtype: str = "bf16"            # "bf16" or "f32"
    scale: Optional[float] = None  # None: 1/sqrt(d_head)
    flags: int = 0                 # LSH_FLAG_* bits; 0 is the method as described

    @property
    def torch_dtype(self) -> torch.dtype:
        return {"bf16": torch.bfloat16, "f32": torch.float32}[self.dtype]

    @property
    def score_scale(self) -> float:
        return 1.0 / math.sqrt(self.d_head) if self.scale is None else float(self.scale)

    def to_c(self) -> CConfig:
        return CConfig(self.batch, self.heads, self.seq_len, self.d_head, self.n_buckets,
                       self.n_rounds, self.chunk, int(bool(self.causal)), self.score_scale,
                       {"bf16": LSH_BF16, "f32": LSH_F32}[self.dtype], self.flags)


_lib: Optional[ctypes.CDLL] = None


def load_library() -> ctypes.CDLL:
    """Load the in-tree HIP library (after torch, so both share one HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m lsh_attention_02_amd.build` (hipcc, gfx950)")
    _lib = _configure(ctypes.CDLL(LIB_PATH))
    return _lib


def load_debug_library() -> ctypes.CDLL:
    """The debug build (device-side bounds checks counted, see
    lsh_debug_check_failures), loaded beside the release one.  Assign it to
    this module's ``_lib`` to route the wrappers through it."""
    if not os.path.exists(DEBUG_LIB_PATH):
        raise RuntimeError(f"{DEBUG_LIB_PATH} is missing: build it with "
                           "`python -m lsh_attention_02_amd.build --debug` (hipcc, gfx950)")
    return _configure(ctypes.CDLL(DEBUG_LIB_PATH))


def debug_check_failures(lib: Optional[ctypes.CDLL] = None, reset: bool = False) -> int:
    """Failed device-side bounds checks counted by `lib` (default: the loaded
    library; always 0 for the release build) on the current device."""
    lib = lib if lib is not None else load_library()
    n = ctypes.c_ulonglong(0)
    st = lib.lsh_debug_check_failures(ctypes.byref(n), int(reset))
    if st != LSH_OK:
        raise LSHError(st, "lsh_debug_check_failures", lib.lsh_last_error().decode())
    return int(n.value)


def _configure(lib: ctypes.CDLL) -> ctypes.CDLL:
    P, CP, I32 = ctypes.c_void_p, ctypes.POINTER(CConfig), ctypes.c_int
    lib.lsh_hash.argtypes = [CP, P, P, P, P]
    lib.lsh_sort_workspace_bytes.argtypes = [CP]
    lib.lsh_sort_workspace_bytes.restype = ctypes.c_size_t
    lib.lsh_sort.argtypes = [CP, P, P, P, P, ctypes.c_size_t, P]
    lib.lsh_sort_noalloc.argtypes = [CP, P, P, P, P]
    lib.lsh_chunk_attn.argtypes = [CP, P, P, P, P, P, P, P]
    lib.lsh_combine_rounds.argtypes = [CP, P, P, P, P]
    lib.lsh_backward_workspace_bytes.argtypes = [CP]
    lib.lsh_backward_workspace_bytes.restype = ctypes.c_size_t
    lib.lsh_attn_backward.argtypes = [CP, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.lsh_project_in.argtypes = [CP, I32, P, P, P, P, P, P]
    lib.lsh_project_out.argtypes = [CP, I32, P, P, P, P]
    lib.lsh_project_out_add.argtypes = [CP, I32, P, P, P, ctypes.c_float, P, P]
    lib.lsh_ffn_workspace_bytes.argtypes = [ctypes.c_int64, I32, I32]
    lib.lsh_ffn_workspace_bytes.restype = ctypes.c_size_t
    lib.lsh_ffn.argtypes = [ctypes.c_int64, I32, I32, I32, P, P, P, P, P, P, ctypes.c_float, P, P,
                            ctypes.c_size_t, P]
    for f in ("lsh_hash", "lsh_sort", "lsh_sort_noalloc", "lsh_chunk_attn", "lsh_combine_rounds", "lsh_attn_backward",
              "lsh_project_in", "lsh_project_out", "lsh_project_out_add", "lsh_ffn"):
        getattr(lib, f).restype = I32
    lib.lsh_status_string.argtypes = [I32]
    lib.lsh_status_string.restype = ctypes.c_char_p
    lib.lsh_last_error.argtypes = []
    lib.lsh_last_error.restype = ctypes.c_char_p
    lib.lsh_debug_check_failures.argtypes = [ctypes.POINTER(ctypes.c_ulonglong), I32]
    lib.lsh_debug_check_failures.restype = I32
    return lib


def _check(status: int, where: str) -> None:
    if status != LSH_OK:
        lib = load_library()
        raise LSHError(status, where, lib.lsh_last_error().decode())


def _ptr(t: torch.Tensor) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device, stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream(device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _empty(shape, dtype: torch.dtype, device, stream=None) -> torch.Tensor:
    """torch.empty taken on `stream` (the current stream when None).  The caching
    allocator hands a block back out only in the order of the stream it was taken
    on, so a buffer the binding allocates for a call on a caller's stream (an
    output, a workspace, an intermediate that forward() drops) is not reused
    before that call's kernels have run."""
    if stream is None:
        return torch.empty(shape, dtype=dtype, device=device)
    with torch.cuda.stream(stream):
        return torch.empty(shape, dtype=dtype, device=device)


def _expect(t: torch.Tensor, name: str, shape, dtype: torch.dtype, device=None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device, got {t.device}")
    if device is not None and (t.get_device() != device.index if device.index is not None
                               else t.device != device):
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.shape != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


@functools.lru_cache(maxsize=256)
def _cconfig(cfg: LSHConfig) -> CConfig:
    """The C struct of a config, built once per config (the library only reads
    it), since a small step is bound by the host time of its calls."""
    return cfg.to_c()


@functools.lru_cache(maxsize=256)
def _shapes(cfg: LSHConfig):
    B, H, L, d, nr = cfg.batch, cfg.heads, cfg.seq_len, cfg.d_head, cfg.n_rounds
    return {"qk": (B, H, L, d), "v": (B, H, L, d), "R": (nr, d, cfg.n_buckets // 2),
            "buckets": (B, H, nr, L), "perm": (B, H, nr, L), "cid": (B, H, L, nr),
            "o_rounds": (B, H, nr, L, d), "lse": (B, H, nr, L), "o": (B, H, L, d)}


def lsh_hash(cfg: LSHConfig, qk: torch.Tensor, R: torch.Tensor,
             buckets: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Step 1: buckets [B, H, n_rounds, L] int32 (see lsh_hash in the header)."""
    lib = load_library()
    sh = _shapes(cfg)
    _expect(qk, "qk", sh["qk"], cfg.torch_dtype)
    _expect(R, "R", sh["R"], cfg.torch_dtype, qk.device)
    if buckets is None:
        buckets = _empty(sh["buckets"], torch.int32, qk.device, stream)
    _expect(buckets, "buckets", sh["buckets"], torch.int32, qk.device)
    c = _cconfig(cfg)
    _check(lib.lsh_hash(ctypes.byref(c), _ptr(qk), _ptr(R), _ptr(buckets),
                        _stream(qk.device, stream)), "lsh_hash")
    return buckets


def lsh_sort_workspace_bytes(cfg: LSHConfig) -> int:
    c = _cconfig(cfg)
    return int(load_library().lsh_sort_workspace_bytes(ctypes.byref(c)))


def sort_workspace(cfg: LSHConfig, device, stream=None) -> torch.Tensor:
    """A device buffer large enough for lsh_sort (at least 16 bytes), taken on
    `stream` (the current stream when None)."""
    n = max(16, lsh_sort_workspace_bytes(cfg))
    return _empty(n, torch.uint8, device, stream)


def lsh_sort(cfg: LSHConfig, buckets: torch.Tensor, perm: Optional[torch.Tensor] = None,
             cid: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
             stream=None):
    """Step 2: (perm [B, H, n_rounds, L] int32, cid [B, H, L, n_rounds] int16)."""
    lib = load_library()
    sh = _shapes(cfg)
    _expect(buckets, "buckets", sh["buckets"], torch.int32)
    dev = buckets.device
    if perm is None:
        perm = _empty(sh["perm"], torch.int32, dev, stream)
    if cid is None:
        cid = _empty(sh["cid"], torch.int16, dev, stream)
    if workspace is None:
        workspace = sort_workspace(cfg, dev, stream)
    _expect(perm, "perm", sh["perm"], torch.int32, dev)
    _expect(cid, "cid", sh["cid"], torch.int16, dev)
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous buffer on the same device")
    nbytes = workspace.numel() * workspace.element_size()
    c = _cconfig(cfg)
    _check(lib.lsh_sort(ctypes.byref(c), _ptr(buckets), _ptr(perm), _ptr(cid), _ptr(workspace),
                        ctypes.c_size_t(nbytes), _stream(dev, stream)), "lsh_sort")
    return perm, cid


# bytes of the static scratch array behind lsh_sort_noalloc (the header's
# LSH_SORT_NOALLOC_MAX_BYTES)
SORT_NOALLOC_MAX_BYTES = 64 << 20


def lsh_sort_noalloc(cfg: LSHConfig, buckets: torch.Tensor, perm: Optional[torch.Tensor] = None,
                     cid: Optional[torch.Tensor] = None, stream=None):
    """Step 2 with the library's static scratch instead of a workspace (see
    lsh_sort_noalloc in the header): (perm, cid).  Calls that overlap on one GPU
    share that scratch and race."""
    lib = load_library()
    sh = _shapes(cfg)
    _expect(buckets, "buckets", sh["buckets"], torch.int32)
    dev = buckets.device
    if perm is None:
        perm = _empty(sh["perm"], torch.int32, dev, stream)
    if cid is None:
        cid = _empty(sh["cid"], torch.int16, dev, stream)
    _expect(perm, "perm", sh["perm"], torch.int32, dev)
    _expect(cid, "cid", sh["cid"], torch.int16, dev)
    c = _cconfig(cfg)
    _check(lib.lsh_sort_noalloc(ctypes.byref(c), _ptr(buckets), _ptr(perm), _ptr(cid),
                                _stream(dev, stream)), "lsh_sort_noalloc")
    return perm, cid


def lsh_chunk_attn(cfg: LSHConfig, qk: torch.Tensor, v: torch.Tensor, perm: torch.Tensor,
                   cid: torch.Tensor, o_rounds: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None, stream=None):
    """Step 3: (o_rounds [B, H, n_rounds, L, d], lse [B, H, n_rounds, L] float32)."""
    lib = load_library()
    sh = _shapes(cfg)
    _expect(qk, "qk", sh["qk"], cfg.torch_dtype)
    dev = qk.device
    _expect(v, "v", sh["v"], cfg.torch_dtype, dev)
    _expect(perm, "perm", sh["perm"], torch.int32, dev)
    _expect(cid, "cid", sh["cid"], torch.int16, dev)
    if o_rounds is None:
        o_rounds = _empty(sh["o_rounds"], cfg.torch_dtype, dev, stream)
    if lse is None:
        lse = _empty(sh["lse"], torch.float32, dev, stream)
    _expect(o_rounds, "o_rounds", sh["o_rounds"], cfg.torch_dtype, dev)
    _expect(lse, "lse", sh["lse"], torch.float32, dev)
    c = _cconfig(cfg)
    _check(lib.lsh_chunk_attn(ctypes.byref(c), _ptr(qk), _ptr(v), _ptr(perm), _ptr(cid),
                              _ptr(o_rounds), _ptr(lse), _stream(dev, stream)), "lsh_chunk_attn")
    return o_rounds, lse


def lsh_combine_rounds(cfg: LSHConfig, o_rounds: torch.Tensor, lse: torch.Tensor,
                       o: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Step 4: o [B, H, L, d]."""
    lib = load_library()
    sh = _shapes(cfg)
    _expect(o_rounds, "o_rounds", sh["o_rounds"], cfg.torch_dtype)
    dev = o_rounds.device
    _expect(lse, "lse", sh["lse"], torch.float32, dev)
    if o is None:
        o = _empty(sh["o"], cfg.torch_dtype, dev, stream)
    _expect(o, "o", sh["o"], cfg.torch_dtype, dev)
    c = _cconfig(cfg)
    _check(lib.lsh_combine_rounds(ctypes.byref(c), _ptr(o_rounds), _ptr(lse), _ptr(o),
                                  _stream(dev, stream)), "lsh_combine_rounds")
    return o


def lsh_backward_workspace_bytes(cfg: LSHConfig) -> int:
    c = _cconfig(cfg)
    return int(load_library().lsh_backward_workspace_bytes(ctypes.byref(c)))


def backward_workspace(cfg: LSHConfig, device, stream=None) -> torch.Tensor:
    """A device buffer large enough for lsh_attn_backward (at least 16 bytes),
    taken on `stream` (the current stream when None)."""
    n = max(16, lsh_backward_workspace_bytes(cfg))
    return _empty(n, torch.uint8, device, stream)


def lsh_attn_backward(cfg: LSHConfig, qk: torch.Tensor, v: torch.Tensor, perm: torch.Tensor,
                      cid: torch.Tensor, lse: torch.Tensor, o: torch.Tensor, d_o: torch.Tensor,
                      d_qk: Optional[torch.Tensor] = None, d_v: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None, stream=None):
    """Backward of steps 3-4: (d_qk, d_v), each [B, H, L, d] float32."""
    lib = load_library()
    sh = _shapes(cfg)
    _expect(qk, "qk", sh["qk"], cfg.torch_dtype)
    dev = qk.device
    _expect(v, "v", sh["v"], cfg.torch_dtype, dev)
    _expect(perm, "perm", sh["perm"], torch.int32, dev)
    _expect(cid, "cid", sh["cid"], torch.int16, dev)
    _expect(lse, "lse", sh["lse"], torch.float32, dev)
    _expect(o, "o", sh["o"], cfg.torch_dtype, dev)
    _expect(d_o, "d_o", sh["o"], cfg.torch_dtype, dev)
    if d_qk is None:
        d_qk = _empty(sh["qk"], torch.float32, dev, stream)
    if d_v is None:
        d_v = _empty(sh["v"], torch.float32, dev, stream)
    _expect(d_qk, "d_qk", sh["qk"], torch.float32, dev)
    _expect(d_v, "d_v", sh["v"], torch.float32, dev)
    if workspace is None:
        workspace = backward_workspace(cfg, dev, stream)
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous buffer on the same device")
    nbytes = workspace.numel() * workspace.element_size()
    c = _cconfig(cfg)
    _check(lib.lsh_attn_backward(ctypes.byref(c), _ptr(qk), _ptr(v), _ptr(perm), _ptr(cid),
                                 _ptr(lse), _ptr(o), _ptr(d_o), _ptr(d_qk), _ptr(d_v),
                                 _ptr(workspace), ctypes.c_size_t(nbytes), _stream(dev, stream)),
           "lsh_attn_backward")
    return d_qk, d_v


def forward(cfg: LSHConfig, qk: torch.Tensor, v: torch.Tensor, R: torch.Tensor,
            workspace: Optional[torch.Tensor] = None, stream=None, return_all: bool = False):
    """All four steps on one stream; returns o (or a dict of every intermediate)."""
    buckets = lsh_hash(cfg, qk, R, stream=stream)
    perm, cid = lsh_sort(cfg, buckets, workspace=workspace, stream=stream)
    o_rounds, lse = lsh_chunk_attn(cfg, qk, v, perm, cid, stream=stream)
    o = lsh_combine_rounds(cfg, o_rounds, lse, stream=stream)
    if return_all:
        return {"buckets": buckets, "perm": perm, "cid": cid, "o_rounds": o_rounds,
                "lse": lse, "o": o}
    return o


def lsh_project_in(cfg: LSHConfig, d_model: int, x: torch.Tensor, w_qk: torch.Tensor,
                   w_v: torch.Tensor, qk: Optional[torch.Tensor] = None,
                   v: Optional[torch.Tensor] = None, stream=None):
    """Layer input projections: (qk, v), each [B, H, L, d] bf16, from x [B, L, d_model]
    and the weights w_qk, w_v [H*d, d_model] (see lsh_project_in in the header)."""
    lib = load_library()
    sh = _shapes(cfg)
    B, L, hd = cfg.batch, cfg.seq_len, cfg.heads * cfg.d_head
    _expect(x, "x", (B, L, d_model), cfg.torch_dtype)
    dev = x.device
    _expect(w_qk, "w_qk", (hd, d_model), cfg.torch_dtype, dev)
    _expect(w_v, "w_v", (hd, d_model), cfg.torch_dtype, dev)
    if qk is None:
        qk = _empty(sh["qk"], cfg.torch_dtype, dev, stream)
    if v is None:
        v = _empty(sh["v"], cfg.torch_dtype, dev, stream)
    _expect(qk, "qk", sh["qk"], cfg.torch_dtype, dev)
    _expect(v, "v", sh["v"], cfg.torch_dtype, dev)
    c = _cconfig(cfg)
    _check(lib.lsh_project_in(ctypes.byref(c), int(d_model), _ptr(x), _ptr(w_qk), _ptr(w_v),
                              _ptr(qk), _ptr(v), _stream(dev, stream)), "lsh_project_in")
    return qk, v


def lsh_project_out(cfg: LSHConfig, d_model: int, o: torch.Tensor, w_o: torch.Tensor,
                    y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Layer output projection: y [B, L, d_model] bf16 from o [B, H, L, d] and
    w_o [d_model, H*d] (see lsh_project_out in the header)."""
    lib = load_library()
    sh = _shapes(cfg)
    _expect(o, "o", sh["o"], cfg.torch_dtype)
    dev = o.device
    _expect(w_o, "w_o", (d_model, cfg.heads * cfg.d_head), cfg.torch_dtype, dev)
    if y is None:
        y = _empty((cfg.batch, cfg.seq_len, d_model), cfg.torch_dtype, dev, stream)
    _expect(y, "y", (cfg.batch, cfg.seq_len, d_model), cfg.torch_dtype, dev)
    c = _cconfig(cfg)
    _check(lib.lsh_project_out(ctypes.byref(c), int(d_model), _ptr(o), _ptr(w_o), _ptr(y),
                               _stream(dev, stream)), "lsh_project_out")
    return y


def lsh_project_out_add(cfg: LSHConfig, d_model: int, o: torch.Tensor, w_o: torch.Tensor,
                        residual: torch.Tensor, sign: float = 1.0, y: Optional[torch.Tensor] = None,
                        stream=None) -> torch.Tensor:
    """y = residual + sign * (lsh_project_out's product); y may be residual itself."""
    lib = load_library()
    sh = _shapes(cfg)
    _expect(o, "o", sh["o"], cfg.torch_dtype)
    dev = o.device
    shape = (cfg.batch, cfg.seq_len, d_model)
    _expect(w_o, "w_o", (d_model, cfg.heads * cfg.d_head), cfg.torch_dtype, dev)
    _expect(residual, "residual", shape, cfg.torch_dtype, dev)
    if y is None:
        y = _empty(shape, cfg.torch_dtype, dev, stream)
    _expect(y, "y", shape, cfg.torch_dtype, dev)
    c = _cconfig(cfg)
    _check(lib.lsh_project_out_add(ctypes.byref(c), int(d_model), _ptr(o), _ptr(w_o), _ptr(residual),
                                   ctypes.c_float(sign), _ptr(y), _stream(dev, stream)),
           "lsh_project_out_add")
    return y


def lsh_ffn_workspace_bytes(rows: int, d_ff: int, chunk_rows: int) -> int:
    return int(load_library().lsh_ffn_workspace_bytes(int(rows), int(d_ff), int(chunk_rows)))


def lsh_ffn(x: torch.Tensor, w1: torch.Tensor, b1: torch.Tensor, w2: torch.Tensor, b2: torch.Tensor,
            residual: torch.Tensor, sign: float = 1.0, chunk_rows: int = 8192,
            y: Optional[torch.Tensor] = None, hidden: Optional[torch.Tensor] = None,
            stream=None) -> torch.Tensor:
    """y = residual + sign * (relu(x w1^T + b1) w2^T + b2) over the rows of x
    [..., d_model] (bf16), chunk_rows rows at a time; y may be residual or x."""
    lib = load_library()
    d_ff, d_model = w1.shape
    dev = x.device
    if x.dtype != torch.bfloat16 or x.shape[-1] != d_model or not x.is_contiguous():
        raise ValueError(f"x must be a contiguous bf16 tensor [..., {d_model}]")
    rows = x.numel() // d_model
    for t, name, shape in ((w1, "w1", (d_ff, d_model)), (b1, "b1", (d_ff,)), (w2, "w2", (d_model, d_ff)),
                           (b2, "b2", (d_model,)), (residual, "residual", tuple(x.shape))):
        _expect(t, name, shape, torch.bfloat16, dev)
    if y is None:
        y = _empty(x.shape, x.dtype, dev, stream)
    _expect(y, "y", tuple(x.shape), torch.bfloat16, dev)
    need = lsh_ffn_workspace_bytes(rows, d_ff, chunk_rows)
    if hidden is None:
        hidden = _empty(max(16, need), torch.uint8, dev, stream)
    if hidden.device != dev or not hidden.is_contiguous():
        raise ValueError("hidden must be a contiguous buffer on the same device")
    _check(lib.lsh_ffn(int(rows), int(d_model), int(d_ff), int(chunk_rows), _ptr(x), _ptr(w1), _ptr(b1),
                       _ptr(w2), _ptr(b2), _ptr(residual), ctypes.c_float(sign), _ptr(y), _ptr(hidden),
                       ctypes.c_size_t(hidden.numel() * hidden.element_size()), _stream(dev, stream)),
           "lsh_ffn")
    return y


def _attention_into(cfg: LSHConfig, x: torch.Tensor, wa: dict, R: torch.Tensor, residual: torch.Tensor,
                    sign: float, y: torch.Tensor, workspace, stream):
    """y = residual + sign * Attention(x), Attention the attention layer."""
    d_model = x.shape[-1]
    qk, v = lsh_project_in(cfg, d_model, x, wa["w_qk"], wa["w_v"], stream=stream)
    o = forward(cfg, qk, v, R, workspace=workspace, stream=stream)
    return lsh_project_out_add(cfg, d_model, o, wa["w_o"], residual, sign, y, stream=stream)


def block_forward(cfg: LSHConfig, x1: torch.Tensor, x2: torch.Tensor, wa: dict, wf: dict,
                  R: torch.Tensor, chunk_rows: int = 8192, workspace=None, stream=None):
    """Reformer block: (y1, y2) = (x1 + Attention(x2), x2 + FeedForward(y1)).
    wa holds w_qk, w_v, w_o; wf holds w1, b1, w2, b2 (see the header)."""
    y1 = _attention_into(cfg, x2, wa, R, x1, 1.0, None, workspace, stream)
    y2 = lsh_ffn(y1, wf["w1"], wf["b1"], wf["w2"], wf["b2"], x2, 1.0, chunk_rows, stream=stream)
    return y1, y2


def block_inverse(cfg: LSHConfig, y1: torch.Tensor, y2: torch.Tensor, wa: dict, wf: dict,
                  R: torch.Tensor, chunk_rows: int = 8192, workspace=None, stream=None,
                  in_place: bool = False):
    """The block's inputs recomputed from its outputs: x2 = y2 - FeedForward(y1),
    then x1 = y1 - Attention(x2).  in_place overwrites y2 with x2 and y1 with x1."""
    x2 = lsh_ffn(y1, wf["w1"], wf["b1"], wf["w2"], wf["b2"], y2, -1.0, chunk_rows,
                 y=y2 if in_place else None, stream=stream)
    x1 = _attention_into(cfg, x2, wa, R, y1, -1.0, y1 if in_place else None, workspace, stream)
    return x1, x2


def layer_forward(cfg: LSHConfig, x: torch.Tensor, w_qk: torch.Tensor, w_v: torch.Tensor,
                  w_o: torch.Tensor, R: torch.Tensor, workspace: Optional[torch.Tensor] = None,
                  stream=None, return_all: bool = False):
    """The LSH-attention layer: projections in, the four steps, projection out.
    Returns y [B, L, d_model] (or a dict with every intermediate)."""
    d_model = x.shape[-1]
    qk, v = lsh_project_in(cfg, d_model, x, w_qk, w_v, stream=stream)
    out = forward(cfg, qk, v, R, workspace=workspace, stream=stream, return_all=True)
    y = lsh_project_out(cfg, d_model, out["o"], w_o, stream=stream)
    if return_all:
        return dict(out, qk=qk, v=v, y=y)
    return y
