"""HIP path vs the fp64 oracle, element by element, through the C ABI.

Contract tolerance (the target's stated bar), per element, no NaN/Inf:
    |o_gpu - o_ref| <= 1e-3 + 5e-3 * |o_ref|
Because |O| is only ~0.005-0.02 at the large shapes, that bar alone would let
a dropped key or block pass, so every case also asserts a tighter gate derived
from the kernel's arithmetic. The weights reach the second product as fp16
P = fp16(e_n) (relative error delta_n below 2^-10) and the row-sum is taken
from the same P, so the computed output is an exact convex combination with
perturbed weights: O' - O = sum_n (w'_n - w_n)(v_n - O), whose spread is about
2^-10/sqrt(12) * sqrt(sum_n w_n^2 (v_n - O)^2). Output rounding adds half an
fp16 ulp (<= 2^-11 |O|). The gate allows
    |o_gpu - o_ref| <= 2^-11 |o_ref| + 8 * 2^-10 * sqrt(sum_n w_n^2 (v_n - o_ref)^2) + 2e-6,
i.e. ~28 standard deviations of the weight-rounding term, with the weights
w_n recomputed here in float64. Structured inputs (ones column, Q = 0,
chunk-indicator V) expose missing or duplicated keys exactly.
"""
from __future__ import annotations

import numpy as np
import pytest

import gqa_attention_split_amd as mga
import oracle
from gqa_attention_split_amd.inputs import CONFIGS, CONFIG_ORDER, make_config, make_qkv

pytestmark = pytest.mark.gpu

CONTRACT_ATOL, CONTRACT_RTOL = 1e-3, 5e-3


def _say(msg):
    print(msg, flush=True)


def to_dev(x, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


def run_gpu(q, k, v, dev, splits=0):
    import torch
    tq, tk, tv = (to_dev(x, dev) for x in (q, k, v))
    out = mga.gqa_forward(tq, tk, tv, splits=splits)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def weight_spread(q, k, v, o_ref):
    """sqrt(sum_n w_n^2 (v_n - o_ref)^2) per output element, w = softmax(qk) in fp64."""
    a = np.matmul(q.astype(np.float64), k.astype(np.float64))
    a -= a.max(axis=2, keepdims=True)
    w = np.exp(a)
    w /= w.sum(axis=2, keepdims=True)
    w2 = w * w
    v64 = v.astype(np.float64)
    s = np.matmul(w2, v64 * v64) - 2 * o_ref * np.matmul(w2, v64) + \
        o_ref * o_ref * w2.sum(axis=2, keepdims=True)
    return np.sqrt(np.maximum(s, 0.0))


def assert_parity(o_gpu, o_ref, q, k, v, label="", extra=0.0):
    """q holds exactly the query rows that o_gpu / o_ref cover; `extra` is
    added to the gate (error terms a caller's path has beyond the plain one)."""
    o = o_gpu.astype(np.float64)
    assert np.isfinite(o).all(), f"{label}: non-finite output"
    err = np.abs(o - o_ref)
    bound = CONTRACT_ATOL + CONTRACT_RTOL * np.abs(o_ref)
    gate = 2.0 ** -11 * np.abs(o_ref) + 8 * 2.0 ** -10 * weight_spread(q, k, v, o_ref) + 2e-6 + extra
    rms = float(np.sqrt(np.mean(o_ref ** 2))) if o_ref.size else 0.0
    _say(f"  {label}: max|err|={err.max():.3e} max|err|/rms(ref)={err.max() / max(rms, 1e-30):.3e} "
         f"rms(ref)={rms:.3e} max(err/gate)={float((err / gate).max()):.3f}")
    assert (err <= bound).all(), f"{label}: contract tolerance violated, max err {err.max():.3e}"
    assert (err <= gate).all(), f"{label}: arithmetic gate violated, max err/gate {(err / gate).max():.3f}"


def sample_rows(M, n, seed):
    rows = {0, M - 1, M // 2}
    for t in (63, 64, 127, 128, 255):
        if t < M:
            rows.add(t)
    rng = np.random.Generator(np.random.PCG64(seed))
    rows.update(int(x) for x in rng.choice(M, size=min(n, M), replace=False))
    return np.array(sorted(rows))


# Full-size workloads, in the launch configuration the bench times (policy splits).
ROWS_PER_BATCH = {"gqa_b2_m256_n4096": 256, "gqa_b16_m256_n4096": 24, "gqa_b2_m256_n32768": 48,
                  "gqa_b64_m8_n8192": 8, "gqa_b128_m256_n16384": 6, "gqa_b64_m1_n4096_d128": 1}


@pytest.mark.parametrize("name", CONFIG_ORDER)
def test_full_size_workload_sampled_rows(gpu, name):
    cfg = CONFIGS[name]
    _say(f"[parity] {name} B={cfg.B} M={cfg.M} N={cfg.N} D={cfg.D} seed={cfg.seed} "
         f"splits={mga.mga_gqa_choose_splits(cfg.B, cfg.M, cfg.N, cfg.D)}")
    q, k, v = make_config(cfg)
    o = run_gpu(q, k, v, gpu)
    rows = sample_rows(cfg.M, ROWS_PER_BATCH[name], cfg.seed)
    qr = np.ascontiguousarray(q[:, rows])
    ref = oracle.gqa_f64(qr, k, v)
    assert_parity(o[:, rows], ref, qr, k, v, name)


SMALL = [(1, 1, 8), (1, 16, 8), (1, 8, 72), (2, 17, 136), (1, 64, 128), (2, 129, 256),
         (3, 255, 4104), (2, 300, 1000), (4, 65, 520), (1, 256, 2048)]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("B,M,N", SMALL)
def test_small_and_ragged_shapes_all_splits(gpu, B, M, N, D):
    q, k, v = make_qkv(B, M, N, seed=1000 + B * 7 + M * 3 + N + D, qk_std=0.3 if D == 64 else 0.25,
                       D=D)
    ref = oracle.gqa_f64(q, k, v)
    nblocks = -(-N // mga.KEY_BLOCK)
    for s in sorted({0, 1, 2, 3, 7, nblocks} & set(range(0, nblocks + 1))):
        _say(f"[parity] B={B} M={M} N={N} D={D} splits={s} "
             f"(effective {mga.mga_gqa_effective_splits(B, M, N, D, s)})")
        assert_parity(run_gpu(q, k, v, gpu, splits=s), ref, q, k, v, f"B{B} M{M} N{N} D{D} s{s}")


def _random_cases(n, seed):
    """Seeded shapes, both head dims, any N (contiguous K repacked when
    N % 8 != 0), splits 0 (policy) or 1..blocks, in three kinds: few batch
    rows (B up to 6, N up to 5000: 32-row tiles, long key streams); many (B
    up to 280, B*M*N up to 8M: the 128- and 256-row tiles on short key
    ranges); and between (B 8-40, M 129-300, N from 1024: 64-row tiles over
    split key ranges)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    cases = []
    for i in range(n):
        D = int(rng.choice([64, 128]))
        if i % 3 == 0:
            B = int(rng.integers(1, 7))
            M = int(rng.choice([int(rng.integers(1, 33)), int(rng.integers(33, 129)),
                                int(rng.integers(129, 301))]))
            N = int(rng.integers(1, 5001))
        elif i % 3 == 1:
            D = 64  # the 128- and 256-row tiles exist at D = 64
            B = int(rng.integers(8, 281))
            M = int(rng.integers(33, 301))
            N = int(rng.integers(1, max(2, min(700, 8_000_000 // (B * M)))))
        else:  # 64-row tiles over split key ranges (the shared ring)
            D = 64
            B = int(rng.integers(16, 41))
            M = int(rng.integers(129, 301))
            N = int(rng.integers(2048, max(2049, min(3000, 8_000_000 // (B * M)))))
        blocks = -(-N // 128)
        s = 0 if rng.random() < 0.5 else int(rng.integers(1, blocks + 1))
        cases.append((B, M, N, D, s))
    return cases


@pytest.mark.parametrize("B,M,N,D,splits", _random_cases(42, 2027))
def test_random_shapes_against_oracle(gpu, B, M, N, D, splits):
    q, k, v = make_qkv(B, M, N, seed=B * 100003 + M * 1009 + N * 7 + D + splits, D=D)
    _say(f"[random] B={B} M={M} N={N} D={D} splits={splits} "
         f"(effective {mga.mga_gqa_effective_splits(B, M, N, D, splits)}, "
         f"rows {mga.mga_gqa_plan(B, M, N, D, splits)[1]})")
    assert_parity(run_gpu(q, k, v, gpu, splits=splits), oracle.gqa_f64(q, k, v), q, k, v,
                  f"B{B} M{M} N{N} D{D} s{splits}")


def _quantized(shape, seed, scale):
    """Seeded uniform inputs on a 1/256 grid (exact in fp16), cheap to draw in bulk."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return (rng.integers(-128, 128, size=shape, dtype=np.int8).astype(np.float16) * np.float16(scale))


@pytest.mark.parametrize("D", [64, 128])
def test_largest_key_count(gpu, D):
    """N at the top of the supported range (2^30 / D - 8: 2^24 - 8 at D = 64,
    2^23 - 8 at D = 128): a batch's K and V byte offsets reach 2^31, the
    per-lane K offsets d*N*2 their maximum, and the last tile straddles N.
    Policy splits and one split per 128-key block."""
    import torch
    B, M, N = 1, 2, (1 << 30) // D - 8
    q = _quantized((B, M, D), 901, 1 / 256)             # |q| <= 0.5
    # |k| <= 16 / D: |score| <= D * 0.5 * 16 / D = 8 < ln 65504
    k = _quantized((B, D, N), 902, 1 / (8 * D))
    v = _quantized((B, N, D), 903, 1 / 64)              # |v| <= 2
    tq, tk, tv = (to_dev(x, gpu) for x in (q, k, v))
    ref = oracle.gqa_f64(q, k, v)
    nblocks = -(-N // mga.KEY_BLOCK)
    for s in (0, nblocks):
        _say(f"[max N] B={B} M={M} N={N} D={D} splits={s} "
             f"(effective {mga.mga_gqa_effective_splits(B, M, N, D, s)}, "
             f"workspace {mga.mga_gqa_workspace_bytes(B, M, N, D, s)} B)")
        o = mga.gqa_forward(tq, tk, tv, splits=s)
        torch.cuda.synchronize()
        assert_parity(o.cpu().numpy(), ref, q, k, v, f"max N D{D} s{s}")
    del tq, tk, tv
    torch.cuda.empty_cache()


@pytest.mark.parametrize("B,D", [(65536, 64), (65535, 128)])
def test_many_query_rows(gpu, B, D):
    """B batch rows x 256 queries over 8 keys, B * 256 * D just below 2^31
    elements (4 GiB of Q and of O): row and batch byte offsets past 2^31, a
    grid of 65536 (D = 64) or 524280 (D = 128) workgroups; checked on sampled
    rows of every 4096th batch."""
    import torch
    M, N = 256, 8
    q = _quantized((B, M, D), 911, 1 / 256)
    k = _quantized((B, D, N), 912, 1 / (4 * D))        # |k| <= 32 / D, as at D = 64 before
    v = _quantized((B, N, D), 913, 1 / 64)
    tq, tk, tv = (to_dev(x, gpu) for x in (q, k, v))
    _say(f"[many rows] B={B} M={M} N={N} D={D} plan={mga.mga_gqa_plan(B, M, N, D, 0)}")
    o = mga.gqa_forward(tq, tk, tv).cpu().numpy()
    torch.cuda.synchronize()
    bs = np.arange(0, B, 4096).tolist() + [B - 1]
    rows = sample_rows(M, 8, 5)
    qs = np.ascontiguousarray(q[bs][:, rows])
    ks, vs = np.ascontiguousarray(k[bs]), np.ascontiguousarray(v[bs])
    assert_parity(o[bs][:, rows], oracle.gqa_f64(qs, ks, vs), qs, ks, vs, f"many rows D{D}")
    del tq, tk, tv
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["gqa_b16_m256_n4096", "gqa_b64_m1_n4096_d128"])
def test_split_invariance_and_determinism(gpu, name):
    cfg = CONFIGS[name]
    q, k, v = make_config(cfg)
    rows = sample_rows(cfg.M, 16, 7)
    qr = np.ascontiguousarray(q[:, rows])
    ref = oracle.gqa_f64(qr, k, v)
    outs = {}
    for s in (1, 2, 3, 7, 16, 32):
        _say(f"[split-invariance] {name} splits={s}")
        o1 = run_gpu(q, k, v, gpu, splits=s)
        o2 = run_gpu(q, k, v, gpu, splits=s)
        assert o1.tobytes() == o2.tobytes(), f"splits={s}: run-to-run bits differ"
        assert_parity(o1[:, rows], ref, qr, k, v, f"splits={s}")
        outs[s] = o1
    base = outs[1].astype(np.float64)
    for s, o in outs.items():
        assert np.max(np.abs(o.astype(np.float64) - base)) <= 2e-4


@pytest.mark.parametrize("D", [64, 128])
def test_structured_inputs_expose_dropped_or_duplicated_keys(gpu, D):
    B, M, N = 3, 200, D * 37  # 2368 or 4736 keys: ragged last block
    q, k, v = make_qkv(B, M, N, seed=77, qk_std=0.3 if D == 64 else 0.25, D=D)
    v = v.copy()
    v[:, :, 7] = 1.0            # ones column: weights sum to 1 exactly in the kernel's sums
    for s in (1, 3, 0):
        o = run_gpu(q, k, v, gpu, splits=s)
        _say(f"[structured] ones column, splits={s}")
        assert np.all(o[:, :, 7] == np.float16(1.0))
    # Q = 0: every weight is equal, so O is the mean of V over all keys.
    q0 = np.zeros_like(q)
    o = run_gpu(q0, k, v, gpu)
    mean = np.broadcast_to(v.astype(np.float64).mean(axis=1, keepdims=True), o.shape)
    assert_parity(o, np.ascontiguousarray(mean), q0, k, v, "Q=0 mean")
    # Chunk-indicator V: column j is the weight mass of key range j.
    r = N // D
    vi = np.zeros((B, N, D), np.float16)
    for n in range(N):
        vi[:, n, n // r] = 1.0
    for s in (1, 5, 0):
        o = run_gpu(q, k, vi, gpu, splits=s)
        assert_parity(o, oracle.gqa_f64(q, k, vi), q, k, vi, f"chunk-indicator s{s}")
        assert np.max(np.abs(o.astype(np.float64).sum(axis=2) - 1.0)) <= D * 2e-4


@pytest.mark.parametrize("D", [64, 128])
def test_partial_then_combine_matches_forward(gpu, D):
    import torch
    B, M, N = 4, 256, 4096
    q, k, v = make_qkv(B, M, N, seed=5, qk_std=0.25, D=D)
    tq, tk, tv = (to_dev(x, gpu) for x in (q, k, v))
    for s in (1, 4):
        o_fwd = mga.gqa_forward(tq, tk, tv, splits=s)
        o = torch.empty_like(o_fwd)
        ws = mga.workspace_for(B, M, N, D, s, device=gpu)
        nb = 0 if ws is None else ws.numel()
        stream = torch.cuda.current_stream()
        assert mga.mga_gqa_partial(tq, tk, tv, o, B, M, N, D, s, ws, nb, stream) == mga.MGA_OK
        assert mga.mga_gqa_combine(o, B, M, N, D, s, ws, nb, stream) == mga.MGA_OK
        torch.cuda.synchronize()
        assert torch.equal(o, o_fwd)


@pytest.mark.parametrize("B,M,N,D", [(16, 256, 4096, 64), (64, 200, 520, 64), (64, 8, 8192, 64), (3, 100, 1000, 64),
                                     (128, 130, 520, 64), (128, 130, 264, 64),   # 128-row tiles: refilled / resident ring
                                     (256, 257, 520, 64), (256, 260, 136, 64),   # 256-row tiles: refilled / resident ring
                                     (64, 1, 4096, 128), (3, 33, 1000, 128)])    # head dim 128: 32-row tiles
def test_partial_then_combine_each_tile_shape(gpu, B, M, N, D):
    """Every query-tile shape the plan can pick (32, 64, 128 and 256 rows at
    head dim 64; 64 rows on the wave-private ring unsplit and on the shared
    ring when split; the shared ring both refilled and with the whole chunk
    resident; 32 rows at head dim 128): partial + combine equals forward bit
    for bit, and a reused workspace gives the same bits on every call."""
    import torch
    q, k, v = make_qkv(B, M, N, seed=31, qk_std=0.3 if D == 64 else 0.25, D=D)
    tq, tk, tv = (to_dev(x, gpu) for x in (q, k, v))
    nblocks = -(-N // mga.KEY_BLOCK)
    stream = torch.cuda.current_stream()
    for req in sorted({0, 2, 3, nblocks}):
        if req > nblocks:
            continue
        rc, rows, s = mga.mga_gqa_plan(B, M, N, D, req)
        assert rc == mga.MGA_OK
        ws = mga.workspace_for(B, M, N, D, req, device=gpu)
        nb = 0 if ws is None else ws.numel()
        ref = torch.empty((B, M, D), dtype=torch.float16, device=gpu)
        assert mga.mga_gqa_partial(tq, tk, tv, ref, B, M, N, D, req, ws, nb, stream) == mga.MGA_OK
        assert mga.mga_gqa_combine(ref, B, M, N, D, req, ws, nb, stream) == mga.MGA_OK
        for call in range(3):
            o = torch.full((B, M, D), float("nan"), dtype=torch.float16, device=gpu)
            assert mga.mga_gqa_forward(tq, tk, tv, o, B, M, N, D, req, ws, nb, stream) == mga.MGA_OK
            torch.cuda.synchronize()
            _say(f"[tile shapes] B={B} M={M} N={N} D={D} splits={s} rows={rows} call {call}")
            assert torch.equal(o, ref), f"forward differs from partial+combine (call {call})"
        assert_parity(ref.cpu().numpy(), oracle.gqa_f64(q, k, v), q, k, v, f"D{D} rows{rows} s{s}")


@pytest.mark.parametrize("D", [64, 128])
def test_non_default_stream_and_empty_shapes(gpu, D):
    import torch
    q, k, v = make_qkv(2, 40, 520, seed=9, D=D)
    ref = oracle.gqa_f64(q, k, v)
    tq, tk, tv = (to_dev(x, gpu) for x in (q, k, v))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out = mga.gqa_forward(tq, tk, tv)
    s.synchronize()
    assert_parity(out.cpu().numpy(), ref, q, k, v, "side stream")
    empty = torch.empty((2, 0, D), dtype=torch.float16, device=gpu)
    assert mga.gqa_forward(empty, tk, tv).shape == (2, 0, D)
    torch.cuda.synchronize()


def test_gpu_rejects_misaligned_pointer_without_launching(gpu):
    import torch
    buf = torch.zeros(2 * 8 * 64 + 8, dtype=torch.float16, device=gpu)
    k = torch.zeros((1, 64, 8), dtype=torch.float16, device=gpu)
    v = torch.zeros((1, 8, 64), dtype=torch.float16, device=gpu)
    o = torch.zeros((1, 8, 64), dtype=torch.float16, device=gpu)
    rc = mga.mga_gqa_forward(buf.data_ptr() + 2, k, v, o, 1, 8, 8, 64, 0, None, 0,
                             torch.cuda.current_stream())
    assert rc == mga.MGA_ERR_LAYOUT


@pytest.mark.parametrize("D,splits", [(64, 1), (64, 4), (128, 1), (128, 3)])
def test_row_whose_weights_all_underflow_is_nan(gpu, D, splits):
    """The documented underflow case: a row whose every score is below
    ln(2^-24) has P = fp16(e^a) = 0 for every key, so L = 0 and the output is
    0/0 = NaN, as the fp16 graph gives (the fp64 oracle, whose exp does not
    underflow there, returns a finite softmax). Every other row stays within
    the contract tolerance, including the rest of that batch (constant K:
    equal scores, the mean of V)."""
    B, M, N = 2, 40, 520
    q, k, v = make_qkv(B, M, N, seed=31, D=D)
    # row (1, 7): scores q.k = -(D/64) * 32 <= -32 for every key (K entries 0.5, Q -1)
    k = k.copy()
    k[1] = np.float16(0.5)
    q = q.copy()
    q[1, 7] = np.float16(-1.0)
    out = run_gpu(q, k, v, gpu, splits=splits)
    assert np.isnan(out[1, 7]).all(), "all-underflow row is not NaN"
    keep = np.ones((B, M), dtype=bool)
    keep[1, 7] = False
    assert np.isfinite(out[keep]).all()
    ref = oracle.gqa_f64(q, k, v)
    err = np.abs(out.astype(np.float64) - ref)[keep]
    assert (err <= CONTRACT_ATOL + CONTRACT_RTOL * np.abs(ref[keep])).all()
