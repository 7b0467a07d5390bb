"""The C ABI library loads, exports every symbol include/attn.h declares, and rejects invalid
arguments on the host before any launch (CPU only: no call here reaches a kernel)."""
import ctypes
import os
import re

import pytest

import exact_attention_tiled_amd as eat
from exact_attention_tiled_amd import build as eat_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

OK, NULL_PTR, BAD_SHAPE, BAD_HEADS, BAD_DTYPE, BAD_MASK, WS_SMALL = 0, -1, -2, -3, -4, -5, -6
BAD_SCALE, BAD_PLAN, BAD_RANGE, BAD_DROPOUT, SCRATCH_SMALL = -9, -10, -11, -12, -13


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(eat_build.LIB_PATH):
        eat_build.build()
    return eat.load()


def header_functions():
    text = open(os.path.join(ROOT, "include", "attn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(attn_\w+)\s*\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported(lib):
    names = header_functions()
    assert len(names) >= 10, names
    for n in names:
        assert hasattr(lib, n), f"{n} missing from libattn.so"
    assert sorted(names) == sorted(eat.EXPORTS)


def test_version_and_status_strings(lib):
    assert eat.attn_version() == 110
    for code in (OK, NULL_PTR, BAD_SHAPE, BAD_HEADS, BAD_DTYPE, BAD_MASK, WS_SMALL, -7, -8,
                 BAD_SCALE, BAD_PLAN, BAD_RANGE, BAD_DROPOUT, SCRATCH_SMALL):
        s = eat.attn_status_string(code)
        assert s and s != "unknown status"
    assert eat.attn_status_string(12345) == "unknown status"


def _fwd(lib, **kw):
    a = dict(q=1, k=1, v=1, cu_q=1, cu_k=1, num_seqs=1, total_q=4, total_k=4, max_q=4, max_k=4,
             hq=2, hkv=1, d=64, dtype=0, scale=0.125, mode=1, window=0, path=0, splits=0,
             out=1, lse=1, ws=None, wsb=0, stream=None)
    a.update(kw)
    return lib.attn_fwd_ex(a["q"], a["k"], a["v"], a["cu_q"], a["cu_k"], a["num_seqs"],
                           a["total_q"], a["total_k"], a["max_q"], a["max_k"], a["hq"], a["hkv"],
                           a["d"], a["dtype"], a["scale"], a["mode"], a["window"], a["path"],
                           a["splits"], a["out"], a["lse"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(d=96), BAD_SHAPE), (dict(total_q=-1), BAD_SHAPE), (dict(max_q=5), BAD_SHAPE),
    (dict(hq=3, hkv=2), BAD_HEADS), (dict(hkv=0), BAD_HEADS), (dict(dtype=7), BAD_DTYPE),
    (dict(mode=3), BAD_MASK), (dict(mode=0, window=4), BAD_MASK),
    (dict(scale=float("inf")), BAD_SCALE), (dict(scale=float("nan")), BAD_SCALE),
    (dict(path=9), BAD_PLAN), (dict(path=2, max_q=4, hq=32, hkv=1), BAD_PLAN),
    (dict(path=2, max_q=1, dtype=1, d=128), BAD_PLAN),
    (dict(q=None), NULL_PTR), (dict(lse=None), NULL_PTR), (dict(cu_k=None), NULL_PTR),
])
def test_fwd_validation(lib, kw, code):
    assert _fwd(lib, **kw) == code


def test_fwd_empty_batch_is_noop(lib):
    assert _fwd(lib, num_seqs=0, total_q=0, total_k=0, max_q=0, max_k=0, q=None, k=None,
                v=None, out=None, lse=None, cu_q=None, cu_k=None) == OK


def test_fwd_workspace_checks(lib):
    # split-K needs workspace: too small -> error before any launch
    need = lib.attn_fwd_ex_workspace_size(2, 2, 4096, 1, 2048, 8, 2, 128, 0, 2, 0, 2, 0)
    assert need > 0
    assert _fwd(lib, num_seqs=2, total_q=2, total_k=4096, max_q=1, max_k=2048, hq=8, hkv=2,
                d=128, mode=2, path=2, ws=1, wsb=need - 1) == WS_SMALL
    # prefill of equal lengths needs none; unequal lengths one int32 per tile slot
    # (256 // 128 + 2 slots), rounded up to 256 bytes
    assert lib.attn_fwd_ex_workspace_size(2, 256, 256, 128, 128, 2, 2, 64, 1, 2, 0, 1, 0) == 0
    assert lib.attn_fwd_ex_workspace_size(2, 256, 300, 200, 200, 2, 2, 64, 0, 2, 0, 1, 0) == 256


def test_bwd_validation(lib):
    args = [1] * 8 + [1, 4, 4, 4, 4, 2, 1, 64, 0, ctypes.c_float(0.1), 1, 0, 1, 1, 1, None, 0, None]
    a = list(args)
    a[15] = 100   # head_dim
    assert lib.attn_bwd(*a) == BAD_SHAPE
    a = list(args)
    a[22] = None  # dk
    assert lib.attn_bwd(*a) == NULL_PTR
    a = list(args)
    assert lib.attn_bwd(*a) in (NULL_PTR, WS_SMALL)  # workspace missing
    need = lib.attn_bwd_workspace_size(1, 4, 4, 4, 4, 2, 1, 64, 0, 1, 0)
    assert need >= 2 * 4 * 2 * 4   # D and LSE (base 2) per (query, head), fp32


def test_bwd_accepts_both_dtypes(lib):
    """The backward takes bf16 and fp32 (the workspace size is the same two row vectors);
    any other dtype code is a validation error returned before any launch."""
    for dt in (0, 1):
        assert lib.attn_bwd_workspace_size(1, 4, 4, 4, 4, 2, 1, 64, dt, 1, 0) == 512
    args = [1] * 8 + [1, 4, 4, 4, 4, 2, 1, 64, 2, ctypes.c_float(0.1), 1, 0, 1, 1, 1, 1, 1 << 20,
                      None]
    assert lib.attn_bwd(*args) == BAD_DTYPE
    dargs = args[:5] + [None] + args[5:20] + [ctypes.c_float(0.1), ctypes.c_uint64(5)] + args[20:]
    assert lib.attn_bwd_dropout(*dargs) == BAD_DTYPE
    # the output residual exists for bf16 only
    dargs[17] = 1      # dtype ATTN_F32
    dargs[5] = 1       # out_residual
    assert lib.attn_bwd_dropout(*dargs) == BAD_DTYPE
    assert lib.attn_bwd_workspace_size(1, 4, 4, 4, 4, 2, 1, 64, 2, 1, 0) == 0


def test_mask_probe_validation(lib):
    assert lib.attn_mask_probe(1, 1, 1, 4, 4, 1, 0, 0, 5, 0, 4, 1, None) == BAD_RANGE
    assert lib.attn_mask_probe(1, 1, 1, 4, 4, 0, 3, 0, 4, 0, 4, 1, None) == BAD_MASK
    assert lib.attn_mask_probe(1, 1, 1, 4, 4, 1, 0, 0, 0, 0, 4, 1, None) == OK
    assert lib.attn_mask_probe(1, 1, 1, 4, 4, 1, 0, 0, 4, 0, 4, None, None) == NULL_PTR


def test_describe_plan(lib):
    buf = ctypes.create_string_buffer(256)
    assert lib.attn_describe_plan(4, 8192, 8192, 2048, 2048, 16, 16, 128, 0, 1, 0, 0, 0, buf, 256) == OK
    assert buf.value.startswith(b"path=prefill")
    assert lib.attn_describe_plan(16, 256, 524288, 16, 32768, 32, 8, 128, 0, 2, 0, 0, 0, buf, 256) == OK
    assert buf.value.startswith(b"path=splitk")
    assert lib.attn_describe_plan(16, 1024, 512, 64, 32, 32, 8, 128, 0, 2, 0, 0, 0, buf, 256) == OK
    assert buf.value.startswith(b"path=prefill")


def test_race_exposure_library_is_the_poisoned_build(lib):
    """lib/libattn_poison.so (compiled with ATTN_DEBUG_POISON_LDS) exports the same symbols
    and says so in its plan description; the release library does not."""
    if not os.path.exists(eat_build.POISON_LIB_PATH):
        eat_build.build(poison_lds=True)
    assert "-DATTN_DEBUG_POISON_LDS" in eat_build.compile_command("/tmp/x.so", poison_lds=True)
    assert "-DATTN_DEBUG_POISON_LDS" not in eat_build.compile_command("/tmp/x.so")
    poison = eat.load(eat_build.POISON_LIB_PATH)
    for n in header_functions():
        assert hasattr(poison, n), f"{n} missing from libattn_poison.so"
    buf = ctypes.create_string_buffer(256)
    for l in (poison, lib):
        assert l.attn_describe_plan(4, 8192, 8192, 2048, 2048, 16, 16, 128, 0, 1, 0, 0, 0,
                                    buf, 256) == OK
        assert buf.value.endswith(b" lds=poisoned") == (l is poison), buf.value
        assert l.attn_describe_plan(16, 256, 524288, 16, 32768, 32, 8, 128, 0, 2, 0, 0, 0,
                                    buf, 256) == OK
        assert buf.value.endswith(b" lds=poisoned") == (l is poison), buf.value


def test_build_command_targets_gfx950():
    cmd = eat_build.compile_command("/tmp/x.so")
    assert "--offload-arch=gfx950" in cmd
    assert "-packed-fp32-ops" in cmd


def test_dropout_validation(lib):
    """Dropout probabilities outside [0, 255.5/256) (or not finite) are rejected before any
    launch; the other arguments are validated as for attn_fwd / attn_bwd."""
    f = ctypes.c_float

    def fwd(p, **kw):
        a = dict(q=1, k=1, v=1, cu_q=1, cu_k=1, d=64, dtype=0, out=1, lse=1, res=None, ws=None,
                 wsb=0)
        a.update(kw)
        return lib.attn_fwd_dropout(a["q"], a["k"], a["v"], a["cu_q"], a["cu_k"], 1, 4, 4, 4, 4,
                                    2, 1, a["d"], a["dtype"], f(0.125), 1, 0, f(p), 12345,
                                    a["out"], a["lse"], a["res"], a["ws"], a["wsb"], None)

    for p in (1.0, -0.1, 255.6 / 256, float("nan"), float("inf")):
        assert fwd(p) == BAD_DROPOUT, p
    assert fwd(0.1, d=96) == BAD_SHAPE
    assert fwd(0.1, out=None) == NULL_PTR
    assert fwd(0.1, dtype=1, res=1) == BAD_DTYPE   # residual: bf16 only
    bargs = [1] * 9 + [1, 4, 4, 4, 4, 2, 1, 64, 0, f(0.1), 1, 0, f(1.5), 7, 1, 1, 1, None, 0,
                       None]
    assert lib.attn_bwd_dropout(*bargs) == BAD_DROPOUT
    bargs[21] = f(0.2)
    bargs[24] = None   # dk
    assert lib.attn_bwd_dropout(*bargs) == NULL_PTR
    assert lib.attn_fwd_dropout_workspace_size(1, 4, 4, 4, 4, 2, 1, 64, 0, 1, 0) == 0
    assert lib.attn_fwd_dropout_workspace_size(2, 9, 9, 5, 5, 2, 1, 64, 0, 1, 0) > 0  # ragged
    assert lib.attn_dropout_probe(0, 0, -1, 4, 0, 4, f(0.1), 1, None, None) == BAD_RANGE
    assert lib.attn_dropout_probe(0, 0, 0, 4, 0, 4, f(1.0), 1, None, None) == BAD_DROPOUT
    assert lib.attn_dropout_probe(0, 0, 0, 0, 0, 4, f(0.1), 1, None, None) == OK
    assert lib.attn_dropout_probe(0, 0, 0, 4, 0, 4, f(0.1), 1, None, None) == NULL_PTR
    big = 2**31 - 64
    assert lib.attn_dropout_probe(0, 0, big, 4, 0, 4, f(0.1), 1, None, None) == BAD_RANGE
    assert lib.attn_dropout_probe(0, 0, 0, 4, big, 4, f(0.1), 1, None, None) == BAD_RANGE
    assert lib.attn_dropout_probe(0, 0, 0, 32 * 65536, 0, 1, f(0.1), 1, None, None) == BAD_RANGE


def test_no_workspace_validation(lib):
    """attn_fwd_no_workspace validates like attn_fwd and refuses, before any launch, a plan
    whose workspace exceeds the fixed scratch (host only: these calls never reach a GPU)."""
    base = [1] * 5 + [1, 4, 4, 4, 4, 2, 1, 64, 0, ctypes.c_float(0.125), 1, 0, 1, 1, None]

    def call(**kw):
        a = list(base)
        for i, val in kw.items():
            a[int(i[1:])] = val
        return lib.attn_fwd_no_workspace(*a)

    assert call(a12=96) == BAD_SHAPE
    assert call(a10=3, a11=2) == BAD_HEADS
    assert call(a13=7) == BAD_DTYPE
    assert call(a15=0, a16=5) == BAD_MASK
    assert call(a14=ctypes.c_float(float("inf"))) == BAD_SCALE
    # split-K decode of 64 sequences x 64 query heads x 8 queries against 64k keys: the
    # partials need far more than the scratch
    big = dict(a5=64, a6=64 * 8, a7=64 * 65536, a8=8, a9=65536, a10=64, a11=8, a12=128, a15=2)
    need = lib.attn_fwd_workspace_size(64, 64 * 8, 64 * 65536, 8, 65536, 64, 8, 128, 0, 2, 0)
    assert need > (16 << 20)
    assert call(**big) == SCRATCH_SMALL
    assert call(a5=0) == OK           # empty batch: nothing to do


def test_mask_probe_ex_validation(lib):
    """Unknown units and split-K shapes the decode path does not take are refused on the
    host; so are heads outside [0, Hq) and windows outside the token ranges."""
    def call(unit, hq=8, hkv=2, max_q=4, max_k=300, head=0, q0=0, nq=4, k0=0, nk=300):
        return lib.attn_mask_probe_ex(1, 1, 1, 4, 300, max_q, max_k, hq, hkv, 2, 0, unit, head,
                                      0, q0, nq, k0, nk, 1, None)
    assert call(7) == BAD_PLAN
    assert call(-1) == BAD_PLAN
    assert call(2, hq=32, hkv=1) == BAD_PLAN   # 128 rows per K/V head: prefill only
    assert call(2, head=8) == BAD_RANGE
    assert call(0, nq=5) == BAD_RANGE
    assert call(3, k0=1) == BAD_RANGE
    assert call(2, hq=6, hkv=4) == BAD_HEADS


def test_check_seqlens_validation(lib):
    """Negative sizes and NULL arrays or word are refused on the host (nothing launched)."""
    def call(**kw):
        a = dict(cu_q=1, cu_k=1, n=1, tq=4, tk=4, mq=4, mk=4, word=1)
        a.update(kw)
        return lib.attn_check_seqlens(a["cu_q"], a["cu_k"], a["n"], a["tq"], a["tk"], a["mq"],
                                      a["mk"], a["word"], None)
    for k in ("n", "tq", "tk", "mq", "mk"):
        assert call(**{k: -1}) == BAD_SHAPE, k
    for k in ("cu_q", "cu_k", "word"):
        assert call(**{k: None}) == NULL_PTR, k


def test_seqlens_error_bits_match_the_header():
    """The binding's names of the error bits are the header's enum values."""
    text = open(os.path.join(ROOT, "include", "attn.h")).read()
    vals = dict(re.findall(r"(ATTN_SEQLENS_\w+) = (\d+)", text))
    assert sorted(int(v) for v in vals.values()) == sorted(eat.SEQLENS_ERRORS)
    assert vals["ATTN_SEQLENS_Q_START"] == "1" and vals["ATTN_SEQLENS_K_ABOVE_MAX"] == "128"
