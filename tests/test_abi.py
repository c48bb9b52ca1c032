"""CPU tests of the C ABI: the library loads, exports what the header declares,
and every argument check returns its status before any HIP call.  Nothing here
launches a kernel: every call fails validation first (fake pointers are only
used where an earlier check is certain to fail)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import lsh_attention_02_amd as lsh
from lsh_attention_02_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lsh_attention.h")


@pytest.fixture(scope="module")
def lib():
    import torch
    if torch.cuda.is_available():
        # These tests pass fake device pointers that validation must reject; a
        # mistake in a test would then reach a real GPU.  They run without one.
        pytest.skip("ABI validation tests run on hosts without a GPU")
    if not os.path.exists(B.LIB_PATH):
        from lsh_attention_02_amd.build import build
        build()
    return lsh.load_library()


def cfg(**kw):
    base = dict(batch=1, heads=8, seq_len=4096, d_head=64, n_buckets=64, n_rounds=2, chunk=64,
                causal=True, dtype="bf16")
    base.update(kw)
    return lsh.LSHConfig(**base).to_c()


def raw(c):
    return ctypes.byref(c)


FAKE = ctypes.c_void_p(1 << 20)      # aligned, never dereferenced (validation fails first)
NULL = ctypes.c_void_p(0)
MISALIGNED = ctypes.c_void_p((1 << 20) + 8)


def test_exports_match_header(lib):
    with open(HEADER) as f:
        text = f.read()
    declared = set(re.findall(r"^\w[\w\s\*]*?\b(lsh_\w+)\s*\(", text, flags=re.M))
    assert declared == set(B.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name


def test_flag_values_match_header():
    text = open(os.path.join(ROOT, "include", "lsh_attention.h")).read()
    vals = dict(re.findall(r"(LSH_FLAG_\w+)\s*=\s*(\d+)", text))
    assert vals == {"LSH_FLAG_NO_DUP_CORRECTION": str(B.LSH_FLAG_NO_DUP_CORRECTION),
                    "LSH_FLAG_WRAP_LOOKBACK": str(B.LSH_FLAG_WRAP_LOOKBACK),
                    "LSH_FLAG_SAME_BUCKET": str(B.LSH_FLAG_SAME_BUCKET)}


def test_struct_layout_matches_header():
    assert ctypes.sizeof(B.CConfig) == 11 * 4
    assert [f[0] for f in B.CConfig._fields_] == ["batch", "heads", "seq_len", "d_head", "n_buckets",
                                                  "n_rounds", "chunk", "causal", "scale", "dtype",
                                                  "flags"]


def test_status_strings(lib):
    for s in range(5):
        assert lib.lsh_status_string(s).decode().startswith(
            ["LSH_OK", "LSH_ERR_INVALID_ARG", "LSH_ERR_UNSUPPORTED", "LSH_ERR_WORKSPACE", "LSH_ERR_HIP"][s])
    assert b"unknown" in lib.lsh_status_string(99)


BAD_CONFIGS = [
    (dict(batch=0), B.LSH_ERR_INVALID_ARG, "positive"),
    (dict(heads=-1), B.LSH_ERR_INVALID_ARG, "positive"),
    (dict(n_buckets=63), B.LSH_ERR_INVALID_ARG, "even"),
    (dict(n_buckets=0), B.LSH_ERR_INVALID_ARG, "positive"),
    (dict(seq_len=4000), B.LSH_ERR_INVALID_ARG, "divide"),
    (dict(seq_len=32768 * 32, chunk=32), B.LSH_ERR_INVALID_ARG, "32767"),
    (dict(seq_len=(1 << 30) + (1 << 16), chunk=1 << 16), B.LSH_ERR_INVALID_ARG, "2^30"),
    (dict(scale=float("nan")), B.LSH_ERR_INVALID_ARG, "finite"),
    (dict(scale=float("inf")), B.LSH_ERR_INVALID_ARG, "finite"),
    (dict(d_head=96), B.LSH_ERR_UNSUPPORTED, "d_head"),
    (dict(n_buckets=65536), B.LSH_ERR_UNSUPPORTED, "32768"),
    (dict(n_rounds=17), B.LSH_ERR_UNSUPPORTED, "16"),
    (dict(flags=8), B.LSH_ERR_UNSUPPORTED, "flag"),
    (dict(flags=6), B.LSH_ERR_UNSUPPORTED, "WRAP"),
    (dict(flags=4, seq_len=32767 * 32, chunk=32, n_buckets=32768), B.LSH_ERR_UNSUPPORTED, "65534"),
    (dict(flags=-1), B.LSH_ERR_UNSUPPORTED, "flag"),
    # o_rounds = 2^20 * 2^10 * 16 * 2^20 * 128 float32 = 2^63 bytes
    (dict(batch=1 << 20, heads=1 << 10, seq_len=1 << 20, chunk=1024, n_rounds=16, d_head=128,
          dtype="f32"), B.LSH_ERR_INVALID_ARG, "2^62"),
]


@pytest.mark.parametrize("kw,status,msg", BAD_CONFIGS)
def test_bad_config_every_call(lib, kw, status, msg):
    c = cfg(**kw)
    calls = [
        lambda: lib.lsh_hash(raw(c), FAKE, FAKE, FAKE, NULL),
        lambda: lib.lsh_sort(raw(c), FAKE, FAKE, FAKE, FAKE, 1 << 40, NULL),
        lambda: lib.lsh_sort_noalloc(raw(c), FAKE, FAKE, FAKE, NULL),
        lambda: lib.lsh_chunk_attn(raw(c), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, NULL),
        lambda: lib.lsh_combine_rounds(raw(c), FAKE, FAKE, FAKE, NULL),
        lambda: lib.lsh_attn_backward(raw(c), *[FAKE] * 10, 1 << 40, NULL),
    ]
    for call in calls:
        assert call() == status
        assert msg in lib.lsh_last_error().decode()
    assert lib.lsh_sort_workspace_bytes(raw(c)) == 0
    assert lib.lsh_backward_workspace_bytes(raw(c)) == 0


def test_bad_dtype_and_causal(lib):
    c = cfg()
    c.dtype = 7
    assert lib.lsh_hash(raw(c), FAKE, FAKE, FAKE, NULL) == B.LSH_ERR_UNSUPPORTED
    c = cfg()
    c.causal = 2
    assert lib.lsh_hash(raw(c), FAKE, FAKE, FAKE, NULL) == B.LSH_ERR_INVALID_ARG


def test_null_config(lib):
    assert lib.lsh_hash(None, FAKE, FAKE, FAKE, NULL) == B.LSH_ERR_INVALID_ARG
    assert b"config" in lib.lsh_last_error()


@pytest.mark.parametrize("which", range(3))
def test_hash_pointer_checks(lib, which):
    c = cfg()
    for bad, word in ((NULL, "null"), (MISALIGNED, "aligned")):
        args = [FAKE, FAKE, FAKE]
        args[which] = bad
        assert lib.lsh_hash(raw(c), *args, NULL) == B.LSH_ERR_INVALID_ARG
        assert word in lib.lsh_last_error().decode()


@pytest.mark.parametrize("which", range(6))
def test_attn_pointer_checks(lib, which):
    c = cfg()
    args = [FAKE] * 6
    args[which] = NULL
    assert lib.lsh_chunk_attn(raw(c), *args, NULL) == B.LSH_ERR_INVALID_ARG


def test_attn_chunk_support(lib):
    for chunk in (16, 256):
        c = cfg(chunk=chunk, seq_len=4096)
        assert lib.lsh_chunk_attn(raw(c), NULL, NULL, NULL, NULL, NULL, NULL, NULL) == B.LSH_ERR_UNSUPPORTED
    c = cfg(dtype="f32", d_head=128, chunk=128)
    assert lib.lsh_chunk_attn(raw(c), NULL, NULL, NULL, NULL, NULL, NULL, NULL) == B.LSH_ERR_UNSUPPORTED


@pytest.mark.parametrize("which", range(5))
def test_project_in_pointer_checks(lib, which):
    c = cfg()
    args = [FAKE] * 5
    args[which] = NULL
    assert lib.lsh_project_in(raw(c), 512, *args, NULL) == B.LSH_ERR_INVALID_ARG
    args[which] = MISALIGNED
    assert lib.lsh_project_in(raw(c), 512, *args, NULL) == B.LSH_ERR_INVALID_ARG


@pytest.mark.parametrize("which", range(3))
def test_project_out_pointer_checks(lib, which):
    c = cfg()
    args = [FAKE] * 3
    args[which] = NULL
    assert lib.lsh_project_out(raw(c), 512, *args, NULL) == B.LSH_ERR_INVALID_ARG


def test_projection_config_checks(lib):
    c = cfg()
    for d_model in (0, -64, 96, 65600):
        assert lib.lsh_project_in(raw(c), d_model, FAKE, FAKE, FAKE, FAKE, FAKE, NULL) == B.LSH_ERR_INVALID_ARG
        assert "d_model" in lib.lsh_last_error().decode()
        assert lib.lsh_project_out(raw(c), d_model, FAKE, FAKE, FAKE, NULL) == B.LSH_ERR_INVALID_ARG
    c = cfg(dtype="f32")
    assert lib.lsh_project_in(raw(c), 512, FAKE, FAKE, FAKE, FAKE, FAKE, NULL) == B.LSH_ERR_UNSUPPORTED
    assert lib.lsh_project_out(raw(c), 512, FAKE, FAKE, FAKE, NULL) == B.LSH_ERR_UNSUPPORTED
    c = cfg(batch=1 << 12, seq_len=1 << 20, chunk=128)      # B * L = 2^32
    assert lib.lsh_project_in(raw(c), 512, FAKE, FAKE, FAKE, FAKE, FAKE, NULL) == B.LSH_ERR_INVALID_ARG
    assert "2^31" in lib.lsh_last_error().decode()


@pytest.mark.parametrize("which", range(10))
def test_backward_pointer_checks(lib, which):
    c = cfg()
    need = lib.lsh_backward_workspace_bytes(raw(c))
    for bad in (NULL, MISALIGNED):
        args = [FAKE] * 10
        args[which] = bad
        assert lib.lsh_attn_backward(raw(c), *args, need, NULL) == B.LSH_ERR_INVALID_ARG


def test_backward_support_and_workspace(lib):
    for kw in (dict(dtype="f32"), dict(chunk=32), dict(chunk=128)):
        c = cfg(**kw)
        assert lib.lsh_backward_workspace_bytes(raw(c)) == 0, kw
        assert lib.lsh_attn_backward(raw(c), *[FAKE] * 10, 1 << 40, NULL) == B.LSH_ERR_UNSUPPORTED, kw
    # combined lse and Delta (float32 per token-head), then three bf16 partials
    # [B, H, n_r, L, d], each part rounded up to 256 bytes
    def up(x):
        return (x + 255) // 256 * 256
    for kw in (dict(), dict(seq_len=65536, d_head=128, n_buckets=1024, n_rounds=8),
               dict(flags=B.LSH_FLAG_NO_DUP_CORRECTION, heads=3, seq_len=192),
               dict(flags=B.LSH_FLAG_WRAP_LOOKBACK), dict(flags=B.LSH_FLAG_SAME_BUCKET)):
        c = cfg(**kw)
        T = c.batch * c.heads * c.seq_len
        want = 2 * up(4 * T) + 3 * up(2 * T * c.n_rounds * c.d_head)
        assert lib.lsh_backward_workspace_bytes(raw(c)) == want, kw
        assert lib.lsh_attn_backward(raw(c), *[FAKE] * 10, want - 1, NULL) == B.LSH_ERR_WORKSPACE


def test_project_out_add_checks(lib):
    c = cfg()
    for which in range(4):
        args = [FAKE] * 4
        args[which] = NULL
        assert lib.lsh_project_out_add(raw(c), 512, args[0], args[1], args[2], ctypes.c_float(1.0),
                                       args[3], NULL) == B.LSH_ERR_INVALID_ARG
    assert lib.lsh_project_out_add(raw(c), 512, FAKE, FAKE, FAKE, ctypes.c_float(float("nan")), FAKE,
                                   NULL) == B.LSH_ERR_INVALID_ARG
    assert "sign" in lib.lsh_last_error().decode()
    assert lib.lsh_project_out_add(raw(c), 96, FAKE, FAKE, FAKE, ctypes.c_float(1.0), FAKE,
                                   NULL) == B.LSH_ERR_INVALID_ARG


def _ffn(lib, rows=4096, d_model=512, d_ff=2048, chunk=1024, ptrs=None, sign=1.0, hidden_bytes=1 << 40):
    p = [FAKE] * 8 if ptrs is None else ptrs
    return lib.lsh_ffn(rows, d_model, d_ff, chunk, p[0], p[1], p[2], p[3], p[4], p[5],
                       ctypes.c_float(sign), p[6], p[7], hidden_bytes, NULL)


def test_ffn_checks(lib):
    for kw in (dict(rows=0), dict(rows=1 << 31), dict(d_model=96), dict(d_ff=0), dict(d_ff=65600),
               dict(chunk=0), dict(sign=float("inf"))):
        assert _ffn(lib, **kw) == B.LSH_ERR_INVALID_ARG, kw
    for which in range(8):
        for bad in (NULL, MISALIGNED):
            ptrs = [FAKE] * 8
            ptrs[which] = bad
            assert _ffn(lib, ptrs=ptrs) == B.LSH_ERR_INVALID_ARG
    # one chunk's hidden activations in bf16 (fewer rows than a chunk: only those)
    assert lib.lsh_ffn_workspace_bytes(4096, 2048, 1024) == 1024 * 2048 * 2
    assert lib.lsh_ffn_workspace_bytes(300, 2048, 1024) == 300 * 2048 * 2
    assert lib.lsh_ffn_workspace_bytes(0, 2048, 1024) == 0
    assert _ffn(lib, hidden_bytes=1024 * 2048 * 2 - 1) == B.LSH_ERR_WORKSPACE


def test_sort_workspace(lib):
    # tile = smallest power of two >= max(2048, 2 * n_buckets) where a workgroup's
    # rounds fit in LDS, else >= max(2048, 4 * n_buckets); at most 65536, at most L.
    # With up to 1024 buckets the tile is then halved, down to max(64, 2 * n_buckets),
    # while the placement has fewer than 256 workgroups (one per (b, h, group of
    # rounds, tile); all rounds of a tile in one group at these sizes).
    # One int32 counter per (segment, tile, bucket).
    cases = [(dict(), 1 * 8 * 2 * 32 * 64),                          # tile 128: 8 x 32 workgroups
             (dict(seq_len=65536, d_head=128, n_buckets=1024, n_rounds=8), 8 * 8 * 32 * 1024),
             (dict(seq_len=1 << 20, n_buckets=16384, n_rounds=4, chunk=128), 8 * 4 * 16 * 16384),
             (dict(seq_len=1024, n_buckets=32, n_rounds=1, heads=1), 1 * 1 * 16 * 32)]   # tile 64
    # plus one int32 per (segment, bucket): the bucket totals (or, with the
    # same-bucket variant, possibly its bucket ranks)
    for flags in (0, B.LSH_FLAG_SAME_BUCKET):
        for kw, counters in cases:
            c = cfg(flags=flags, **kw)
            nseg = c.batch * c.heads * c.n_rounds
            assert lib.lsh_sort_workspace_bytes(raw(c)) == 4 * (counters + nseg * c.n_buckets), kw
    for flags in (0, B.LSH_FLAG_SAME_BUCKET):
        c = cfg(flags=flags)
        need = lib.lsh_sort_workspace_bytes(raw(c))
        assert lib.lsh_sort(raw(c), FAKE, FAKE, FAKE, FAKE, need - 1, NULL) == B.LSH_ERR_WORKSPACE


def test_binding_rejects_host_tensors(lib):
    import torch
    c = lsh.LSHConfig(1, 1, 128, 64, 8, 1, 64, False, dtype="f32")
    qk = torch.zeros(1, 1, 128, 64)
    R = torch.zeros(1, 64, 4)
    with pytest.raises(ValueError, match="GPU"):
        lsh.lsh_hash(c, qk, R)


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "LIB_PATH", "/nonexistent/liblsh_attention.so")
    with pytest.raises(RuntimeError, match="missing"):
        B.load_library()


def test_header_is_plain_c_with_hip_streams():
    """The header compiles as C99 host code, and every stream is a hipStream_t."""
    import shutil
    import subprocess
    text = open(HEADER).read()
    assert "void* stream" not in text
    assert len(re.findall(r"hipStream_t stream\)", text)) >= 9
    gcc = shutil.which("gcc")
    rocm_inc = "/opt/rocm/include"
    if gcc is None or not os.path.isdir(rocm_inc):
        pytest.skip("gcc or the ROCm headers are not installed")
    subprocess.run([gcc, "-x", "c", "-std=c99", "-fsyntax-only", "-Wall", "-Werror",
                    "-D__HIP_PLATFORM_AMD__", "-I" + rocm_inc, HEADER], check=True)


def test_sort_noalloc_checks(lib):
    """The entry point without a workspace checks its pointers, and rejects a
    configuration whose counters exceed the static scratch buffer, before any
    HIP call."""
    c = cfg()
    for which in range(3):
        for bad in (NULL, MISALIGNED):
            args = [FAKE] * 3
            args[which] = bad
            assert lib.lsh_sort_noalloc(raw(c), *args, NULL) == B.LSH_ERR_INVALID_ARG
    text = open(HEADER).read()
    m = re.search(r"#define LSH_SORT_NOALLOC_MAX_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == B.SORT_NOALLOC_MAX_BYTES
    big = cfg(heads=64, seq_len=1 << 20, n_buckets=16384, n_rounds=4, chunk=128)
    assert lib.lsh_sort_workspace_bytes(raw(big)) > B.SORT_NOALLOC_MAX_BYTES
    assert lib.lsh_sort_noalloc(raw(big), FAKE, FAKE, FAKE, NULL) == B.LSH_ERR_WORKSPACE
    assert "static buffer" in lib.lsh_last_error().decode()
    # the 1M-token workload fits
    long_1m = cfg(seq_len=1 << 20, n_buckets=16384, n_rounds=4, chunk=128)
    assert lib.lsh_sort_workspace_bytes(raw(long_1m)) <= B.SORT_NOALLOC_MAX_BYTES


def test_validation_under_host_asan():
    """The checks above, and more, in an AddressSanitizer build of the C ABI's
    host code (tests/abi_asan_check.c; built by the package build): every call
    fails validation before any HIP call, and ASan watches the message strings,
    the size arithmetic and the config reads."""
    import subprocess
    import torch
    from lsh_attention_02_amd import build as BLD
    if torch.cuda.is_available():
        pytest.skip("fake device pointers: runs on hosts without a GPU")
    if not os.path.exists(BLD.ASAN_CHECK):
        pytest.skip("ASan check not built (python -m lsh_attention_02_amd.build)")
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1")
    p = subprocess.run([BLD.ASAN_CHECK], stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       text=True, env=env, timeout=120)
    assert p.returncode == 0, p.stdout[-4000:]
    assert "ok: 0 failure(s)" in p.stdout


def test_debug_check_failures_release_build(lib):
    """The release library has no device-side checks: the count is 0, read
    without any HIP call; a null count is rejected."""
    n = ctypes.c_ulonglong(7)
    assert lib.lsh_debug_check_failures(ctypes.byref(n), 1) == B.LSH_OK
    assert n.value == 0
    assert lib.lsh_debug_check_failures(None, 0) == B.LSH_ERR_INVALID_ARG
    assert b"count" in lib.lsh_last_error()


def test_debug_library_exports(lib):
    """The debug build (device-side bounds checks) exports the same C ABI."""
    if not os.path.exists(B.DEBUG_LIB_PATH):
        from lsh_attention_02_amd.build import build
        build(debug=True)
    dbg = ctypes.CDLL(B.DEBUG_LIB_PATH)
    for name in B.EXPORTED:
        assert hasattr(dbg, name), name
    dbg.lsh_debug_check_failures.argtypes = [ctypes.c_void_p, ctypes.c_int]
    assert dbg.lsh_debug_check_failures(None, 0) == B.LSH_ERR_INVALID_ARG   # checked before any HIP call
