"""The C ABI without a GPU: the library loads, exports every function the
header declares, and its host-only entry points (status strings, split policy,
workspace sizing, argument checks) behave as documented. No kernel runs."""
import ctypes
import math
import os
import re
import subprocess

import pytest

import gqa_attention_split_amd as mga
from gqa_attention_split_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mga_gqa.h")
A = 1 << 20  # a 16-byte-aligned fake device address; check_args never dereferences


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mga_\w+)\s*\(", text)))


def test_header_declares_the_documented_entry_points():
    assert header_functions() == sorted(_lib.SIGNATURES)


CITATION = re.compile(r"kaispace blog|Mirage documentation|Mirage docs")
# The one entry point outside the pages' passages names the callers it serves.
NO_ALLOC_CALLERS = re.compile(r"callers that cannot allocate")


def test_every_declaration_cites_its_passage():
    """The comment block in front of each declaration (the text since the
    previous declaration) names the page passage that defines the call."""
    text = open(HEADER).read()
    body = text[text.index("extern \"C\" {"):]
    starts = [(m.start(), m.group(1)) for m in re.finditer(r"^[a-z][\w\s\*]*\b(mga_\w+)\s*\(", body, re.M)]
    assert sorted(n for _, n in starts) == sorted(_lib.SIGNATURES)
    prev = 0
    for pos, name in starts:
        comments = " ".join(re.findall(r"/\*.*?\*/", body[prev:pos], flags=re.S))
        comments = re.sub(r"\s*\n\s*\*?\s*", " ", comments)  # join wrapped comment lines
        want = NO_ALLOC_CALLERS if name == "mga_gqa_forward_noalloc" else CITATION
        assert want.search(comments), f"{name}: no passage cited in the comment before it"
        prev = body.index(";", pos) + 1


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    for name in header_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in header_functions():
        assert name in exported, name


def test_status_strings():
    for code in range(7):
        s = mga.mga_status_string(code)
        assert s.startswith("MGA_"), s
    assert "unknown" in mga.mga_status_string(99)


def _check(B=2, M=256, N=4096, splits=0, q=A, k=A, v=A, o=A, ws=A, ws_bytes=None, D=64):
    if ws_bytes is None:
        ws_bytes = mga.mga_gqa_workspace_bytes(B, M, N, D, splits)
    return mga.mga_gqa_check_args(q, k, v, o, B, M, N, D, splits, ws, ws_bytes)


def test_check_args_codes():
    assert _check() == mga.MGA_OK
    assert _check(q=None) == mga.MGA_ERR_INVALID_VALUE
    assert _check(o=None) == mga.MGA_ERR_INVALID_VALUE
    assert _check(B=-1) == mga.MGA_ERR_INVALID_VALUE
    assert _check(M=-1) == mga.MGA_ERR_INVALID_VALUE
    assert _check(N=0) == mga.MGA_ERR_INVALID_VALUE
    assert _check(splits=-1) == mga.MGA_ERR_INVALID_VALUE
    assert _check(N=4100) == mga.MGA_OK                     # contiguous K, N % 8 != 0: repacked
    assert _check(N=4100, splits=1, ws=None, ws_bytes=0) == mga.MGA_ERR_WORKSPACE
    assert _check(k=A + 8) == mga.MGA_ERR_LAYOUT
    assert _check(o=A + 2) == mga.MGA_ERR_LAYOUT
    assert _check(splits=33) == mga.MGA_ERR_CONFIG          # ceil(4096/128) = 32
    assert _check(N=1 << 24, splits=1) == mga.MGA_ERR_CONFIG   # byte offsets exceed 32 bits
    assert _check(B=1 << 20, M=1 << 20, N=128) == mga.MGA_ERR_CONFIG
    assert _check(splits=4, ws=None) == mga.MGA_ERR_WORKSPACE
    assert _check(splits=4, ws_bytes=1024) == mga.MGA_ERR_WORKSPACE
    assert _check(splits=4, ws=A + 4) == mga.MGA_ERR_WORKSPACE
    # One split needs no workspace; empty batches or rows are no-ops.
    assert _check(splits=1, ws=None, ws_bytes=0) == mga.MGA_OK
    assert _check(B=0, q=None, k=None, v=None, o=None, ws=None, ws_bytes=0) == mga.MGA_OK
    assert _check(M=0, q=None, k=None, v=None, o=None, ws=None, ws_bytes=0) == mga.MGA_OK


def test_check_args_head_dim():
    assert _check(D=128) == mga.MGA_OK
    assert _check(D=128, splits=4) == mga.MGA_OK
    assert _check(D=128, splits=4, ws_bytes=mga.mga_gqa_workspace_bytes(2, 256, 4096, 64, 4)) == \
        mga.MGA_ERR_WORKSPACE                                 # sized for D = 64: too small
    for D in (0, -64, 32, 96, 256):
        assert _check(D=D) == mga.MGA_ERR_CONFIG, D
    # N * D * 2 bytes must stay below 2^31: N <= 2^23 - 1 at D = 128, 2^24 - 1 at D = 64
    assert _check(D=128, N=(1 << 23) - 8, splits=1) == mga.MGA_OK
    assert _check(D=128, N=1 << 23, splits=1) == mga.MGA_ERR_CONFIG
    assert _check(D=64, N=1 << 23, splits=1) == mga.MGA_OK
    assert _check(D=64, N=(1 << 24) - 8, splits=1) == mga.MGA_OK
    # B * M * D must stay below 2^31 elements
    assert _check(D=128, B=65535, M=256, N=8) == mga.MGA_OK
    assert _check(D=128, B=65536, M=256, N=8) == mga.MGA_ERR_CONFIG
    assert _check(D=64, B=65536, M=256, N=8) == mga.MGA_OK
    assert _check(D=64, B=65536, M=512, N=8) == mga.MGA_ERR_CONFIG


def test_forward_rejects_before_launching():
    # Errors come back before any HIP call, so this runs without a GPU.
    assert mga.mga_gqa_forward(A, A, A, A, 2, 256, 4100, 64, 0, None, 0, None) == mga.MGA_ERR_WORKSPACE
    assert mga.mga_gqa_forward(A + 2, A, A, A, 2, 256, 4096, 64, 0, None, 0, None) == mga.MGA_ERR_LAYOUT
    assert mga.mga_gqa_forward(A, A, A, A, 2, 256, 4096, 80, 1, None, 0, None) == mga.MGA_ERR_CONFIG
    assert mga.mga_gqa_partial(None, A, A, A, 2, 256, 4096, 128, 1, None, 0, None) == \
        mga.MGA_ERR_INVALID_VALUE
    assert mga.mga_gqa_combine(A, 2, 256, 4096, 64, 4, None, 0, None) == mga.MGA_ERR_WORKSPACE
    assert mga.mga_gqa_combine(A, 2, 256, 4096, 128, 4, A, 1024, None) == mga.MGA_ERR_WORKSPACE
    assert mga.mga_gqa_forward(None, None, None, None, 0, 256, 4096, 64, 0, None, 0, None) == \
        mga.MGA_OK


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("B,M,N", [(2, 256, 4096), (16, 256, 4096), (2, 256, 32768),
                                   (64, 8, 8192), (128, 256, 16384), (1, 1, 8), (3, 17, 136),
                                   (5, 100, 1000), (1, 300, 129 * 8), (64, 1, 4096)])
def test_split_policy_and_workspace(B, M, N, D):
    nblocks = math.ceil(N / mga.KEY_BLOCK)
    s = mga.mga_gqa_choose_splits(B, M, N, D)
    assert 1 <= s <= nblocks
    for req in sorted({r for r in (0, 1, 2, 3, 7, nblocks) if r <= nblocks}):
        eff = mga.mga_gqa_effective_splits(B, M, N, D, req)
        want = s if req == 0 else req
        chunk = math.ceil(nblocks / want)
        assert eff == math.ceil(nblocks / chunk)
        assert 1 <= eff <= want
        assert (eff - 1) * chunk < nblocks          # no empty split
        ws = mga.mga_gqa_workspace_bytes(B, M, N, D, req)
        rc, rows, eff2 = mga.mga_gqa_plan(B, M, N, D, req)
        assert rc == mga.MGA_OK and eff2 == eff and rows in ((32, 64, 128, 256) if D == 64 else (32,))
        if eff == 1:
            assert ws == 0
        else:
            o_bytes = -(-eff * B * M * D * 2 // 256) * 256   # fp16 partials, then fp32 denominators
            assert ws == -(-(o_bytes + eff * B * M * 4) // 256) * 256
    assert mga.mga_gqa_effective_splits(B, M, N, D, nblocks + 1) == -1
    assert mga.mga_gqa_plan(B, M, N, D, nblocks + 1)[0] == mga.MGA_ERR_CONFIG


@pytest.mark.parametrize("B,M,N,D,rows,splits", [
    (64, 1, 4096, 128, 32, 4),   # the head-dim-128 decode example: 4 splits fill 256 CUs
    (8, 32, 16384, 128, 32, 32),
    (1, 1, 8, 128, 32, 1),
    (256, 64, 1024, 128, 32, 1),
    (16, 256, 4096, 64, 64, 4),      # 64-row tiles, 4 splits fill 256 CUs
    (2, 256, 4096, 64, 32, 8),       # 64-row tiles would reach 64 workgroups at most: 32-row tiles
    (2, 256, 32768, 64, 64, 32),
    (64, 8, 8192, 64, 32, 8),        # decode-like rows: 32-row tiles, 4 waves, two workgroups per CU
    (128, 256, 16384, 64, 128, 1),   # 128-row tiles fill the chip unsplit
    (70, 300, 16384, 64, 256, 2),    # 256-row tiles fill the chip with two splits (128-row do not unsplit)
    (128, 130, 520, 64, 128, 1),     # 128-row tiles fill the chip unsplit
    (1024, 256, 1024, 64, 256, 1),   # 256-row tiles already fill the chip
])
def test_plan_policy(B, M, N, D, rows, splits):
    assert mga.mga_gqa_plan(B, M, N, D, 0) == (mga.MGA_OK, rows, splits)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(RuntimeError, match="no CPU fallback"):
        _lib.load()


# ---------------------------------------------------------------- strides --
_NAMES = ("q_b", "q_i", "k_b", "k_d", "k_n", "v_b", "v_n", "o_b", "o_i")


def _st(B, M, N, D, **kw):
    base = dict(q_b=M * D, q_i=D, k_b=D * N, k_d=N, k_n=1, v_b=N * D, v_n=D, o_b=M * D, o_i=D)
    base.update(kw)
    return [base[n] for n in _NAMES]


def _check_st(B=2, M=256, N=4096, D=64, splits=1, strides="default", **kw):
    st = _st(B, M, N, D, **kw) if strides == "default" else strides
    return mga.mga_gqa_check_args_strided(A, A, A, A, B, M, N, D, st, splits, None, 0)


def test_strided_layouts_accepted():
    assert _check_st() == mga.MGA_OK
    assert _check_st(strides=None) == mga.MGA_OK                      # NULL = contiguous
    for D in (64, 128):
        # K as the transpose of a (B, N, D) tensor: any N
        for N in (1, 13, 1001, 4096):
            assert _check_st(N=N, D=D, k_b=N * D, k_d=1, k_n=D) == mga.MGA_OK, (N, D)
        # head-dim-major K rows padded to a multiple of 8 keys
        assert _check_st(N=1001, D=D, k_b=D * 1008, k_d=1008) == mga.MGA_OK
        # K and V interleaved in one (B, N, 2, D) cache; Q and O inside wider rows
        assert _check_st(N=4096, D=D, k_b=4096 * 2 * D, k_d=1, k_n=2 * D, v_b=4096 * 2 * D,
                         v_n=2 * D, q_i=3 * D, q_b=256 * 3 * D, o_i=2 * D, o_b=256 * 2 * D) == mga.MGA_OK
    # K, V and Q shared by every batch (stride 0)
    assert _check_st(q_b=0, k_b=0, v_b=0) == mga.MGA_OK
    # O batches may sit anywhere when there is one batch
    assert _check_st(B=1, o_b=8) == mga.MGA_OK


def test_strided_layouts_rejected():
    # explicit head-dim-major strides need rows that start 16-byte aligned;
    # only the contiguous form (NULL strides) repacks K into the workspace
    assert _check_st(N=1001, k_b=64 * 1001, k_d=1001) == mga.MGA_ERR_LAYOUT
    assert _check_st(strides=None, N=1001) == mga.MGA_ERR_WORKSPACE
    assert _check_st(k_n=2) == mga.MGA_ERR_LAYOUT                      # no unit stride in K
    assert _check_st(k_d=1, k_n=56) == mga.MGA_ERR_LAYOUT              # key rows shorter than D
    assert _check_st(k_d=4088) == mga.MGA_ERR_LAYOUT                   # head-dim rows shorter than N
    assert _check_st(k_d=1, k_n=68) == mga.MGA_ERR_LAYOUT              # not a multiple of 8
    for name, val in (("q_i", 68), ("q_i", 56), ("v_n", 60), ("v_n", 56), ("o_i", 72 + 4),
                      ("o_i", 32), ("q_b", 4), ("k_b", 12), ("v_b", 2), ("o_b", 16384 + 4)):
        assert _check_st(**{name: val}) == mga.MGA_ERR_LAYOUT, (name, val)
    for name in _NAMES:
        assert _check_st(**{name: -8}) == mga.MGA_ERR_LAYOUT, name
    # O batches must not overlap: (M - 1) * o_i + D = 16384
    assert _check_st(o_b=16384) == mga.MGA_OK
    assert _check_st(o_b=16376) == mga.MGA_ERR_LAYOUT
    # byte extents behind one descriptor stay below 2^31
    assert _check_st(k_d=1, k_n=1 << 18, k_b=0) == mga.MGA_OK          # (4095 * 2^18 + 64) * 2 < 2^31
    assert _check_st(k_d=1, k_n=1 << 19, k_b=0) == mga.MGA_ERR_CONFIG
    assert _check_st(v_n=1 << 19) == mga.MGA_ERR_CONFIG
    rows = mga.mga_gqa_plan(2, 256, 4096, 64, 1)[1]                  # a workgroup's Q rows
    q_bad = next(1 << e for e in range(3, 31) if ((rows - 1) * (1 << e) + 64) * 2 >= 1 << 31)
    assert _check_st(q_i=q_bad) == mga.MGA_ERR_CONFIG
    assert _check_st(q_i=q_bad // 2) == mga.MGA_OK
    assert _check_st(o_i=(1 << 30) + 8) == mga.MGA_ERR_CONFIG
    assert _check_st(q_b=(1 << 48) + 8) == mga.MGA_ERR_CONFIG
    # a layout error comes back from the strided forward without launching
    assert mga.mga_gqa_forward_strided(A, A, A, A, 2, 256, 1001, 64, _st(2, 256, 1001, 64), 1,
                                       None, 0, None) == mga.MGA_ERR_LAYOUT


def test_plan_accepts_any_key_count():
    # the plan and workspace do not depend on the layout, so N % 8 != 0 is fine there
    rc, rows, eff = mga.mga_gqa_plan(2, 256, 1001, 64, 0)
    assert rc == mga.MGA_OK and eff == mga.mga_gqa_effective_splits(2, 256, 1001, 64, 0)
    assert mga.mga_gqa_workspace_bytes(2, 256, 1001, 64, 2) > 0


# --------------------------------------------------------- QK norm (host) --
def test_qknorm_plan_uses_private_ring_shapes():
    for (B, M, N, D, rows) in [(16, 256, 4096, 64, 64), (128, 256, 16384, 64, 64), (64, 8, 8192, 64, 32),
                               (64, 1, 4096, 128, 32), (2, 300, 1000, 64, 64)]:
        rc, r, eff = mga.mga_gqa_qknorm_plan(B, M, N, D, 0)
        assert rc == mga.MGA_OK and r == rows, (B, M, N, D, r)
        ws = mga.mga_gqa_qknorm_workspace_bytes(B, M, N, D, 0)
        if eff == 1:
            assert ws == 0
        else:
            o_bytes = -(-eff * B * M * D * 2 // 256) * 256
            assert ws == -(-(o_bytes + eff * B * M * 4) // 256) * 256


def test_qknorm_check_args():
    def chk(eps=1e-6, strides=None, **kw):
        a = dict(B=2, M=256, N=4096, D=64, splits=1)
        a.update(kw)
        return mga.mga_gqa_qknorm_check_args(A, A, A, A, a["B"], a["M"], a["N"], a["D"], eps, strides,
                                             a["splits"], None, 0)
    assert chk() == mga.MGA_OK
    assert chk(eps=0.0) == mga.MGA_OK
    for bad in (-1e-6, float("nan"), float("inf")):
        assert chk(eps=bad) == mga.MGA_ERR_INVALID_VALUE, bad
    assert chk(D=96) == mga.MGA_ERR_CONFIG
    assert chk(N=1001) == mga.MGA_ERR_WORKSPACE                       # contiguous K repack needs one
    assert chk(N=1001, strides=_st(2, 256, 1001, 64, k_b=1001 * 64, k_d=1, k_n=64)) == mga.MGA_OK
    assert chk(splits=4) == mga.MGA_ERR_WORKSPACE
    assert mga.mga_gqa_qknorm_forward(A, A, A, A, 2, 256, 4096, 64, -1.0, None, 1, None, 0,
                                      None) == mga.MGA_ERR_INVALID_VALUE


def test_repack_workspace_for_unaligned_contiguous_k():
    """Contiguous K with N % 8 != 0 is copied into the workspace with rows of
    ceil8(N) keys, after the partials (each part rounded up to 256 bytes)."""
    for (B, M, N, D) in [(2, 256, 1001, 64), (3, 40, 13, 128), (1, 1, 3, 64), (16, 256, 4095, 64)]:
        for splits in sorted({1, 0, 2} & set(range(math.ceil(N / mga.KEY_BLOCK) + 1))):
            eff = mga.mga_gqa_effective_splits(B, M, N, D, splits)
            part = 0
            if eff > 1:
                o_bytes = -(-eff * B * M * D * 2 // 256) * 256
                part = -(-(o_bytes + eff * B * M * 4) // 256) * 256
            n8 = -(-N // 8) * 8
            assert mga.mga_gqa_workspace_bytes(B, M, N, D, splits) == part + -(-B * D * n8 * 2 // 256) * 256
            assert mga.mga_gqa_check_args(A, A, A, A, B, M, N, D, splits, A,
                                          mga.mga_gqa_workspace_bytes(B, M, N, D, splits)) == mga.MGA_OK


def test_noalloc_refuses_plans_above_its_scratch_without_a_gpu():
    """The size check comes before any HIP call: a plan whose workspace is
    larger than the fixed scratch (here the K copy of a contiguous K with
    N % 8 != 0: 64*64*4104*2 bytes) is refused, as are invalid shapes."""
    need = mga.mga_gqa_workspace_bytes(64, 256, 4100, 64, 0)
    assert need > mga.NOALLOC_SCRATCH_BYTES
    assert mga.mga_gqa_forward_noalloc(A, A, A, A, 64, 256, 4100, 64, None, 0, None) == mga.MGA_ERR_SCRATCH
    assert mga.mga_gqa_forward_noalloc(A, A, A, A, 2, 256, 0, 64, None, 0, None) == mga.MGA_ERR_INVALID_VALUE
    assert mga.mga_gqa_forward_noalloc(A, A, A, A, 2, 256, 4096, 96, None, 0, None) == mga.MGA_ERR_CONFIG
    assert "16 MiB" in mga.mga_status_string(mga.MGA_ERR_SCRATCH)
