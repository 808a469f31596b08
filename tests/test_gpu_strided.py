"""Strided views and any key count through mga_gqa_forward_strided, against
the fp64 oracle (which always sees the logical, contiguous tensors) and, where
a contiguous counterpart exists, against mga_gqa_forward bit for bit.

Layouts covered: K as the transpose of a (B, N, D) tensor (key-major), K with
head-dim rows padded past N, K and V interleaved in one (B, N, 2, D) cache,
Q and O inside wider rows, K and V shared by every batch (stride 0). Memory
that the views do not cover (padding past N, cache rows past N, the rest of
O's rows) holds NaN or a sentinel, so a read of it or a write to it shows.
"""
from __future__ import annotations

import numpy as np
import pytest

import gqa_attention_split_amd as mga
import oracle
from gqa_attention_split_amd.inputs import make_qkv
from test_gpu_parity import assert_parity

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _t(x, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


def _key_major(k, dev, capacity=None):
    """K (B, D, N) as the transpose of a (B, capacity, D) cache whose rows past
    N are NaN."""
    import torch
    B, D, N = k.shape
    cap = capacity or N
    cache = torch.full((B, cap, D), float("nan"), dtype=torch.float16, device=dev)
    cache[:, :N] = _t(np.transpose(k, (0, 2, 1)), dev)
    return cache[:, :N].transpose(1, 2)


def _padded_rows(k, dev, pad):
    """K (B, D, N) inside (B, D, N + pad) rows, the padding NaN; N + pad is
    rounded up to a multiple of 8."""
    import torch
    B, D, N = k.shape
    width = -(-(N + pad) // 8) * 8
    buf = torch.full((B, D, width), float("nan"), dtype=torch.float16, device=dev)
    buf[:, :, :N] = _t(k, dev)
    return buf[:, :, :N]


def _run(q, k, v, splits=0, out=None):
    import torch
    o = mga.gqa_forward(q, k, v, out=out, splits=splits)
    torch.cuda.synchronize()
    return o


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("B,M,N", [(4, 256, 4096), (3, 100, 1000), (2, 33, 136)])
def test_other_k_layouts_equal_contiguous_bitwise(gpu, B, M, N, D):
    """Key-major K and padded head-dim-major K feed the same MFMA operands in
    the same order as contiguous K: the outputs are identical."""
    import torch
    q, k, v = make_qkv(B, M, N, seed=300 + N + D, qk_std=0.3 if D == 64 else 0.25, D=D)
    tq, tk, tv = _t(q, gpu), _t(k, gpu), _t(v, gpu)
    nblocks = -(-N // mga.KEY_BLOCK)
    for s in sorted({0, 1, 3, nblocks} & set(range(nblocks + 1))):
        ref = _run(tq, tk, tv, s)
        for name, kview in (("key-major", _key_major(k, gpu, capacity=N + 40)),
                            ("padded rows", _padded_rows(k, gpu, 24))):
            _say(f"[layout] B={B} M={M} N={N} D={D} splits={s} K {name} strides={tuple(kview.stride())}")
            o = _run(tq, kview, tv, s)
            assert torch.equal(o, ref), f"{name}: differs from the contiguous path"
    assert_parity(ref.cpu().numpy(), oracle.gqa_f64(q, k, v), q, k, v, f"D{D} B{B} M{M} N{N}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("N", [1, 3, 13, 100, 1001, 4099])
def test_any_key_count(gpu, N, D):
    """N not a multiple of 8 (or of the 32-key tile): the tail tile's keys past
    N are masked, whatever the padding behind them holds."""
    B, M = 3, 40
    q, k, v = make_qkv(B, M, N, seed=400 + N + D, qk_std=0.3 if D == 64 else 0.25, D=D)
    ref = oracle.gqa_f64(q, k, v)
    tq, tv = _t(q, gpu), _t(v, gpu)
    nblocks = -(-N // mga.KEY_BLOCK)
    for kname, kview in (("key-major", _key_major(k, gpu, capacity=N + 37)),
                         ("padded rows", _padded_rows(k, gpu, 5))):
        for s in sorted({0, 1, 2, nblocks} & set(range(nblocks + 1))):
            _say(f"[any N] N={N} D={D} K {kname} splits={s} "
                 f"(effective {mga.mga_gqa_effective_splits(B, M, N, D, s)})")
            o = _run(tq, kview, tv, s).cpu().numpy()
            assert_parity(o, ref, q, k, v, f"N{N} D{D} {kname} s{s}")


def test_any_key_count_structured(gpu):
    """Ones column and chunk-indicator V at N = 1001 (key-major K): a key past
    N that leaked into the sums, or a key lost at the tail, shows exactly."""
    B, M, N, D = 2, 70, 1001, 64
    q, k, v = make_qkv(B, M, N, seed=77, qk_std=0.3)
    kview = _key_major(k, gpu, capacity=N + 23)
    tq = _t(q, gpu)
    v1 = v.copy()
    v1[:, :, 5] = 1.0
    for s in (0, 1, 3, 8):
        o = _run(tq, kview, _t(v1, gpu), s).cpu().numpy()
        _say(f"[structured N=1001] ones column splits={s}")
        assert np.all(o[:, :, 5] == np.float16(1.0))
    r = -(-N // D)
    vi = np.zeros((B, N, D), np.float16)
    for n in range(N):
        vi[:, n, n // r] = 1.0
    ref = oracle.gqa_f64(q, k, vi)
    for s in (1, 5, 0):
        o = _run(tq, kview, _t(vi, gpu), s).cpu().numpy()
        assert_parity(o, ref, q, k, vi, f"chunk-indicator N=1001 s{s}")
        assert np.max(np.abs(o.astype(np.float64).sum(axis=2) - 1.0)) <= D * 2e-4


@pytest.mark.parametrize("D", [64, 128])
def test_interleaved_cache_and_wide_rows(gpu, D):
    """K and V interleaved in a (B, N, 2, D) cache, Q the middle third of
    (B, M, 3D) rows, O the first half of (B, M, 2D) rows whose second half must
    stay untouched."""
    import torch
    B, M, N = 4, 130, 2056
    q, k, v = make_qkv(B, M, N, seed=500 + D, qk_std=0.3 if D == 64 else 0.25, D=D)
    ref = oracle.gqa_f64(q, k, v)
    kv = torch.full((B, N + 8, 2, D), float("nan"), dtype=torch.float16, device=gpu)
    kv[:, :N, 0] = _t(np.transpose(k, (0, 2, 1)), gpu)
    kv[:, :N, 1] = _t(v, gpu)
    kview, vview = kv[:, :N, 0].transpose(1, 2), kv[:, :N, 1]
    qbig = torch.full((B, M, 3 * D), float("nan"), dtype=torch.float16, device=gpu)
    qbig[:, :, D:2 * D] = _t(q, gpu)
    qview = qbig[:, :, D:2 * D]
    for s in (0, 1, 4):
        obig = torch.full((B, M, 2 * D), -7.0, dtype=torch.float16, device=gpu)
        oview = obig[:, :, :D]
        _say(f"[interleaved] D={D} splits={s} strides q={tuple(qview.stride())} "
             f"k={tuple(kview.stride())} v={tuple(vview.stride())} o={tuple(oview.stride())}")
        _run(qview, kview, vview, s, out=oview)
        assert torch.all(obig[:, :, D:] == -7.0), "wrote outside the output view"
        assert_parity(oview.cpu().numpy(), ref, q, k, v, f"interleaved D{D} s{s}")


@pytest.mark.parametrize("D", [64, 128])
def test_kv_shared_by_every_batch(gpu, D):
    """K and V expanded over the batch axis (batch stride 0)."""
    import torch
    B, M, N = 6, 64, 1032
    q, k, v = make_qkv(B, M, N, seed=600 + D, qk_std=0.3 if D == 64 else 0.25, D=D)
    k1, v1 = k[:1], v[:1]
    kx, vx = _t(k1, gpu).expand(B, D, N), _t(v1, gpu).expand(B, N, D)
    kb, vb = np.repeat(k1, B, axis=0), np.repeat(v1, B, axis=0)
    ref = oracle.gqa_f64(q, kb, vb)
    for s in (0, 1, 3):
        _say(f"[shared kv] D={D} splits={s} k stride={tuple(kx.stride())}")
        o = _run(_t(q, gpu), kx, vx, s)
        assert_parity(o.cpu().numpy(), ref, q, kb, vb, f"shared kv D{D} s{s}")
        assert torch.equal(o, _run(_t(q, gpu), _t(kb, gpu), _t(vb, gpu), s))


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("N", [1, 3, 13, 1001, 4099])
def test_contiguous_k_with_unaligned_rows_is_repacked(gpu, N, D):
    """Contiguous K whose rows (N keys) do not start 16-byte aligned: the
    library copies it into the workspace with rows of ceil8(N) keys. The
    result equals the padded-row view's bit for bit (same kernel, same
    operands) and matches the oracle; the QK-normalised path takes the same
    copy."""
    import torch
    B, M = 3, 40
    q, k, v = make_qkv(B, M, N, seed=1100 + N + D, qk_std=0.3 if D == 64 else 0.25, D=D)
    tq, tk, tv = _t(q, gpu), _t(k, gpu), _t(v, gpu)
    ref = oracle.gqa_f64(q, k, v)
    nblocks = -(-N // mga.KEY_BLOCK)
    for s in sorted({0, 1, 2, nblocks} & set(range(nblocks + 1))):
        _say(f"[repack] N={N} D={D} splits={s} workspace={mga.mga_gqa_workspace_bytes(B, M, N, D, s)}")
        o = _run(tq, tk, tv, s)
        assert torch.equal(o, _run(tq, _padded_rows(k, gpu, 5), tv, s))
        assert_parity(o.cpu().numpy(), ref, q, k, v, f"repacked N{N} D{D} s{s}")
    o = mga.gqa_forward(tq, tk, tv, qk_norm=True)
    kview = _padded_rows(k, gpu, 11)
    o2 = mga.gqa_forward(tq, kview, tv, qk_norm=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)


def _random_views(n, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for _ in range(n):
        D = int(rng.choice([64, 128]))
        B = int(rng.integers(1, 9))
        M = int(rng.integers(1, 300))
        N = int(rng.integers(1, 3000))
        blocks = -(-N // mga.KEY_BLOCK)
        s = 0 if rng.random() < 0.5 else int(rng.integers(1, blocks + 1))
        pads = tuple(int(8 * rng.integers(0, 5)) for _ in range(5))  # q row, q batch rows, k, v row, o row
        km = bool(rng.random() < 0.5)
        out.append((B, M, N, D, s, km, pads))
    return out


@pytest.mark.parametrize("B,M,N,D,splits,key_major,pads", _random_views(24, 4242))
def test_random_strided_views_equal_contiguous(gpu, B, M, N, D, splits, key_major, pads):
    """Seeded shapes with every operand a strided view (Q and O inside wider
    rows, Q's batches further apart, K key-major from a longer cache or in
    padded head-dim-major rows, V inside wider rows), the memory outside the
    views NaN (inputs) or a sentinel (output): the result equals the
    contiguous path's bit for bit and nothing outside O's view is written."""
    import torch
    qpad, qrows, kpad, vpad, opad = pads
    q, k, v = make_qkv(B, M, N, seed=B * 7919 + M * 31 + N + D + splits, D=D)
    ref = _run(_t(q, gpu), _t(k, gpu), _t(v, gpu), splits)
    qb = torch.full((B, M + qrows, D + qpad), float("nan"), dtype=torch.float16, device=gpu)
    qb[:, :M, :D] = _t(q, gpu)
    qv = qb[:, :M, :D]
    kv = _key_major(k, gpu, capacity=N + kpad) if key_major else _padded_rows(k, gpu, kpad)
    vb = torch.full((B, N, D + vpad), float("nan"), dtype=torch.float16, device=gpu)
    vb[:, :, :D] = _t(v, gpu)
    vv = vb[:, :, :D]
    ob = torch.full((B, M, D + opad), 7.0, dtype=torch.float16, device=gpu)
    ov = ob[:, :, :D]
    _say(f"[random views] B={B} M={M} N={N} D={D} splits={splits} K {'key-major' if key_major else 'rows'} "
         f"q{tuple(qv.stride())} k{tuple(kv.stride())} v{tuple(vv.stride())} o{tuple(ov.stride())}")
    _run(qv, kv, vv, splits, out=ov)
    assert torch.equal(ov, ref), "strided views differ from the contiguous path"
    if opad:
        assert (ob[:, :, D:] == 7.0).all(), "a write outside O's view"
