"""QK-normalised path (mga_gqa_qknorm_forward) vs oracle.gqa_qknorm_f64,
element by element.

The gate of test_gpu_parity.assert_parity is applied with the normalised
operands (q-hat, k-hat in fp64), so the weights it derives its spread from are
those of the QK-normalised softmax. The path feeds raw Q and K to the first
product and scales the fp32 scores by both norms, so its per-score error is
that of the plain path; only the score scale differs (|A| up to D). That
scale makes the softmax sharp, and two error terms the plain gate never needs
appear, added per output column j with vmax_j = max_n |V[b,n,j]|:
  * each split's partial o_s is rounded to fp16 (at most 2^-11 |o_s| <= 2^-11
    vmax_j after the weighted combine), when there are several splits;
  * P = fp16(2^(a - m)) is subnormal below 2^-14 and flushes below 2^-24, so
    each key carries an absolute weight error up to 2^-25 / L with L >= 1:
    N 2^-24 vmax_j in all.

Inputs vary the raw magnitudes (rows and key vectors scaled by powers of two)
so that the normalisation does work, and include scores at the extremes
(+-D: a key equal to +-q) placed first and last in the key range, which moves
the running reference maximum both early and late.
"""
from __future__ import annotations

import numpy as np
import pytest

import gqa_attention_split_amd as mga
import oracle
from gqa_attention_split_amd.inputs import CONFIGS, make_config, make_qkv
from test_gpu_parity import assert_parity, sample_rows

pytestmark = pytest.mark.gpu

EPS = 1e-6


def _say(msg):
    print(msg, flush=True)


def _t(x, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


def _check(o, q, k, v, label, splits=1):
    ref = oracle.gqa_qknorm_f64(q, k, v, eps=EPS)
    qn, kn = oracle.rms_norm_f64(q, 2, EPS), oracle.rms_norm_f64(k, 1, EPS)
    N = k.shape[2]
    vmax = np.max(np.abs(v.astype(np.float64)), axis=1, keepdims=True)   # (B, 1, D)
    extra = (N * 2.0 ** -24 + (2.0 ** -11 if splits > 1 else 0.0)) * vmax
    assert_parity(o, ref, qn, kn, v, label, extra=extra)


def _eff(q, k, s):
    B, M, D = q.shape
    return mga.mga_gqa_qknorm_plan(B, M, k.shape[2], D, s)[2]


def _run(q, k, v, dev, splits=0):
    import torch
    o = mga.gqa_forward(_t(q, dev) if isinstance(q, np.ndarray) else q,
                        _t(k, dev) if isinstance(k, np.ndarray) else k,
                        _t(v, dev) if isinstance(v, np.ndarray) else v,
                        splits=splits, qk_norm=True, eps=EPS)
    torch.cuda.synchronize()
    return o.cpu().numpy()


def _rescaled(q, k, seed):
    """Scale every query row and key vector by 2^e, e in [-3, 3] (exact in fp16)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    B, M, D = q.shape
    N = k.shape[2]
    qs = q * np.exp2(rng.integers(-3, 4, size=(B, M, 1))).astype(np.float16)
    ks = k * np.exp2(rng.integers(-3, 4, size=(B, 1, N))).astype(np.float16)
    return qs.astype(np.float16), ks.astype(np.float16)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("B,M,N", [(1, 1, 8), (2, 17, 136), (2, 129, 256), (3, 255, 4104),
                                   (2, 300, 1000), (4, 65, 520)])
def test_qknorm_small_and_ragged(gpu, B, M, N, D):
    q, k, v = make_qkv(B, M, N, seed=700 + B + M + N + D, qk_std=1.0, D=D)
    q, k = _rescaled(q, k, N + D)
    nblocks = -(-N // mga.KEY_BLOCK)
    for s in sorted({0, 1, 2, 3, nblocks} & set(range(nblocks + 1))):
        _say(f"[qknorm] B={B} M={M} N={N} D={D} splits={s} plan={mga.mga_gqa_qknorm_plan(B, M, N, D, s)}")
        _check(_run(q, k, v, gpu, s), q, k, v, f"qknorm B{B} M{M} N{N} D{D} s{s}", _eff(q, k, s))


@pytest.mark.parametrize("name,rows", [("gqa_b16_m256_n4096", 16), ("gqa_b64_m1_n4096_d128", 1),
                                       ("gqa_b64_m8_n8192", 8), ("gqa_b2_m256_n32768", 24),
                                       ("gqa_b128_m256_n16384", 2)])
def test_qknorm_full_size_sampled_rows(gpu, name, rows):
    cfg = CONFIGS[name]
    q, k, v = make_config(cfg)
    _say(f"[qknorm full] {name} plan={mga.mga_gqa_qknorm_plan(cfg.B, cfg.M, cfg.N, cfg.D, 0)}")
    o = _run(q, k, v, gpu)
    r = sample_rows(cfg.M, rows, cfg.seed)
    qr = np.ascontiguousarray(q[:, r])
    _check(o[:, r], qr, k, v, f"qknorm {name}", _eff(q, k, 0))


@pytest.mark.parametrize("D", [64, 128])
def test_qknorm_extreme_scores_move_the_reference(gpu, D):
    """Key 0 = -q and key N-1 = +q for every query of batch 0 (M = 1): scores
    -D and +D; batch 1 has key 0 = +q: the largest score comes first."""
    B, M, N = 2, 1, 3000
    q, k, v = make_qkv(B, M, N, seed=800 + D, qk_std=1.0, D=D)
    k = k.copy()
    k[0, :, 0] = -q[0, 0]
    k[0, :, N - 1] = q[0, 0]
    k[1, :, 0] = q[1, 0] * np.float16(2.0)
    for s in (1, 0, 5, 24):
        _say(f"[qknorm extreme] D={D} splits={s}")
        o = _run(q, k, v, gpu, s)
        _check(o, q, k, v, f"extreme D{D} s{s}", _eff(q, k, s))


def test_qknorm_extreme_scores_on_the_shared_ring(gpu):
    """64 query rows with split keys run on the shared ring, whose two waves
    per SIMD take a tile's softmax before or after the previous tile's
    second product. Rows in both query waves (5 and 40) get keys at -q and
    +q first and last in the key range; row 45 gets its largest score
    first; the reference maximum then moves early and late in both phase
    orders."""
    B, M, N, D = 2, 64, 3000, 64
    q, k, v = make_qkv(B, M, N, seed=860, qk_std=1.0, D=D)
    k = k.copy()
    for b in range(B):
        k[b, :, 0] = -q[b, 5]
        k[b, :, N - 1] = q[b, 5]
        k[b, :, 1] = -q[b, 40]
        k[b, :, N - 2] = q[b, 40]
        k[b, :, 2] = q[b, 45] * np.float16(2.0)
    for s in (0, 2, 5, 23):
        plan = mga.mga_gqa_qknorm_plan(B, M, N, D, s)
        _say(f"[qknorm extreme shared] splits={s} plan={plan}")
        assert plan[1] == 64 and plan[2] > 1, plan  # 64-row tiles over split keys
        o = _run(q, k, v, gpu, s)
        _check(o, q, k, v, f"extreme shared s{s}", _eff(q, k, s))


def test_qknorm_strided_any_n_and_structured(gpu):
    import torch
    for D in (64, 128):
        B, M, N = 3, 40, 1001
        q, k, v = make_qkv(B, M, N, seed=900 + D, qk_std=1.0, D=D)
        cache = torch.full((B, N + 9, D), float("nan"), dtype=torch.float16, device=gpu)
        cache[:, :N] = _t(np.transpose(k, (0, 2, 1)), gpu)
        kview = cache[:, :N].transpose(1, 2)
        for s in (0, 1, 3):
            _say(f"[qknorm strided] D={D} N={N} splits={s}")
            o = _run(q, kview, v, gpu, s)
            _check(o, q, k, v, f"qknorm key-major D{D} s{s}", _eff(q, k, s))
        v1 = v.copy()
        v1[:, :, 3] = 1.0
        o = _run(q, kview, v1, gpu, 3)
        assert np.all(o[:, :, 3] == np.float16(1.0))


def test_qknorm_deterministic_and_split_consistent(gpu):
    B, M, N = 4, 64, 4096
    q, k, v = make_qkv(B, M, N, seed=950, qk_std=1.0)
    outs = {}
    for s in (1, 2, 4, 16, 32):
        a, b = _run(q, k, v, gpu, s), _run(q, k, v, gpu, s)
        assert a.tobytes() == b.tobytes(), f"splits={s}: run-to-run bits differ"
        outs[s] = a.astype(np.float64)
    for s, o in outs.items():
        assert np.max(np.abs(o - outs[1])) <= 2e-3, s
    _check(outs[4].astype(np.float16), q, k, v, "qknorm s4", 4)


def _random_qkn_cases(n, seed):
    """Seeded shapes for the QK-normalised path: few batch rows with long key
    ranges (M up to 32: 32-row tiles; more: 64-row tiles), and more batch
    rows with shorter ones (64-row tiles, on the shared ring once the keys
    are split), both head dims (D = 128: 32-row tiles), any N, policy or
    random splits."""
    rng = np.random.Generator(np.random.PCG64(seed))
    cases = []
    for i in range(n):
        D = int(rng.choice([64, 128]))
        if i % 2 == 0:
            M = int(rng.integers(1, 33)) if rng.random() < 0.5 else int(rng.integers(33, 300))
            B, N = int(rng.integers(1, 5)), int(rng.integers(1, 5000))
        else:
            B, M = int(rng.integers(8, 33)), int(rng.integers(65, 300))
            N = int(rng.integers(512, max(513, min(3000, 6_000_000 // (B * M)))))
        blocks = -(-N // mga.KEY_BLOCK)
        s = 0 if rng.random() < 0.5 else int(rng.integers(1, blocks + 1))
        cases.append((B, M, N, D, s))
    return cases


@pytest.mark.parametrize("B,M,N,D,splits", _random_qkn_cases(24, 5150))
def test_qknorm_random_shapes(gpu, B, M, N, D, splits):
    q, k, v = make_qkv(B, M, N, seed=B * 6007 + M * 17 + N + D + splits, qk_std=1.0, D=D)
    q, k = _rescaled(q, k, B + M + N)
    _say(f"[qknorm random] B={B} M={M} N={N} D={D} splits={splits} "
         f"plan={mga.mga_gqa_qknorm_plan(B, M, N, D, splits)}")
    _check(_run(q, k, v, gpu, splits), q, k, v, f"qknorm B{B} M{M} N{N} D{D} s{splits}",
           _eff(q, k, splits))
