"""Pins for the QK-normalised oracle (``oracle.gqa_qknorm_f64``).

The tutorial ("Implement QK Normalization and Optimize Attention Kernel in
Python" on the Mirage documentation pages) applies rms_norm to Q and to K and
then runs the GQA graph; it prints no output values. The pins therefore come
from the mathematics and from library routines:

* a library witness: torch.nn.functional.rms_norm (over the head dim, eps
  1e-6, no weight) on Q's rows and on K's key vectors, then
  scaled_dot_product_attention with scale 1, all in float64;
* a 50-digit brute force (Python ``decimal``) on tiny inputs;
* invariants that fix the axis reading: scaling a query row or a key vector
  by a positive factor leaves O unchanged (with eps = 0), while scaling one
  head-dim row of K (the same component of every key) changes it;
* a fixed point: inputs whose vectors already have unit root mean square
  give the plain graph's output (eps = 0);
* eps matters where the mean square is comparable to it.

``test_qknorm_mutant_is_caught`` plants plausible mistakes (norm over the
key axis, L2 instead of root-mean-square, eps outside the root, only Q or
only K normalised) and checks that each fails at least one pin.
"""
from __future__ import annotations

from decimal import Decimal, getcontext

import numpy as np
import pytest
import torch

import oracle
from gqa_attention_split_amd.inputs import make_qkv


def _rel_close(x, ref, rtol, atol=0.0):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    scale = max(float(np.max(np.abs(ref))) if ref.size else 0.0, 1e-300)
    err = float(np.max(np.abs(x - ref))) if ref.size else 0.0
    assert err <= atol + rtol * scale, f"max abs err {err:.3e} > {atol + rtol * scale:.3e}"


def pin_torch_witness(impl):
    for (B, M, N, D, std, seed) in [(2, 9, 300, 64, 0.3, 1), (3, 4, 130, 128, 0.25, 2),
                                    (1, 17, 64, 64, 1e-3, 3)]:     # last: mean square ~ eps
        q, k, v = make_qkv(B, M, N, seed=seed, qk_std=std, D=D)
        o = impl(q, k, v, 1e-6)
        tq = torch.from_numpy(q.astype(np.float64))
        tk = torch.from_numpy(np.ascontiguousarray(k.astype(np.float64).transpose(0, 2, 1)))
        tv = torch.from_numpy(v.astype(np.float64))
        qn = torch.nn.functional.rms_norm(tq, (D,), eps=1e-6)
        kn = torch.nn.functional.rms_norm(tk, (D,), eps=1e-6)
        ref = torch.nn.functional.scaled_dot_product_attention(qn, kn, tv, scale=1.0).numpy()
        _rel_close(o, ref, rtol=1e-10)


def pin_bruteforce_decimal(impl):
    getcontext().prec = 50
    for (B, M, N, D, seed) in [(1, 2, 3, 4, 11), (1, 1, 9, 16, 12), (2, 1, 2, 8, 13)]:
        q, k, v = make_qkv(B, M, N, seed=seed, qk_std=0.7, D=D)
        o = impl(q, k, v, 1e-6)
        eps = Decimal("1e-6")
        exact = np.zeros((B, M, D))
        for b in range(B):
            kn = []
            for n in range(N):
                col = [Decimal(float(k[b, d, n])) for d in range(D)]
                r = (sum(x * x for x in col) / D + eps).sqrt()
                kn.append([x / r for x in col])
            for i in range(M):
                row = [Decimal(float(q[b, i, d])) for d in range(D)]
                r = (sum(x * x for x in row) / D + eps).sqrt()
                qn = [x / r for x in row]
                e = [sum(qn[d] * kn[n][d] for d in range(D)).exp() for n in range(N)]
                s = sum(e)
                for j in range(D):
                    exact[b, i, j] = float(sum(e[n] / s * Decimal(float(v[b, n, j])) for n in range(N)))
        _rel_close(o, exact, rtol=1e-12)


def pin_scale_invariance_fixes_the_axis(impl):
    q, k, v = make_qkv(2, 6, 50, seed=21, qk_std=0.4)
    o = impl(q, k, v, 0.0)
    q2 = q.astype(np.float64)
    q2[:, 3, :] *= 8.0                     # one query row
    k2 = k.astype(np.float64)
    k2[:, :, 17] *= 0.125                  # one key vector
    _rel_close(impl(q2, k2, v, 0.0), o, rtol=1e-12)
    k3 = k.astype(np.float64)
    k3[:, 5, :] *= 4.0                     # one head-dim component of every key
    diff = np.max(np.abs(impl(q, k3, v, 0.0) - o))
    assert diff > 1e-3, f"scaling a head-dim row of K left O unchanged ({diff:.2e})"


def pin_unit_rms_fixed_point(impl):
    # Entries +-1 have root mean square exactly 1, so rms_norm (eps = 0) is
    # the identity and O is the plain graph's.
    rng = np.random.Generator(np.random.PCG64(31))
    B, M, N, D = 2, 5, 40, 64
    q = rng.choice(np.array([-1.0, 1.0], np.float16), size=(B, M, D))
    k = rng.choice(np.array([-1.0, 1.0], np.float16), size=(B, D, N))
    v = rng.standard_normal((B, N, D)).astype(np.float16)
    q /= np.float16(4.0)                    # rms 1/4 now: normalised back to +-1
    _rel_close(impl(q, k, v, 0.0), oracle.gqa_f64(q * np.float16(4.0), k, v), rtol=1e-12)


def pin_eps_inside_root(impl):
    # Mean square 1e-6 = eps: the root is sqrt(2e-6), not sqrt(1e-6) or 1e-3 + eps.
    B, M, N, D = 1, 1, 2, 4
    q = np.full((B, M, D), 1e-3)
    k = np.zeros((B, D, N))
    k[0, :, 0] = 1e-3
    k[0, :, 1] = -1e-3
    v = np.zeros((B, N, D))
    v[0, 0, 0] = 1.0
    # q_hat = k_hat(0) = 1/sqrt(2) per entry, k_hat(1) = -1/sqrt(2): scores +-2 -> weights logistic(4)
    w0 = 1.0 / (1.0 + np.exp(-4.0))
    o = impl(q, k, v, 1e-6)
    assert abs(o[0, 0, 0] - w0) <= 1e-12, (o[0, 0, 0], w0)


PINS = {f.__name__: f for f in [pin_torch_witness, pin_bruteforce_decimal,
                                pin_scale_invariance_fixes_the_axis, pin_unit_rms_fixed_point,
                                pin_eps_inside_root]}


@pytest.mark.parametrize("pin_name", list(PINS))
def test_qknorm_oracle_pin(pin_name):
    PINS[pin_name](lambda q, k, v, eps: oracle.gqa_qknorm_f64(q, k, v, eps=eps))


def test_rms_norm_rows_have_unit_mean_square():
    q, k, _ = make_qkv(3, 7, 33, seed=41, qk_std=0.6)
    qn = oracle.rms_norm_f64(q, axis=2, eps=0.0)
    kn = oracle.rms_norm_f64(k, axis=1, eps=0.0)
    assert np.max(np.abs(np.mean(qn * qn, axis=2) - 1.0)) <= 1e-14
    assert np.max(np.abs(np.mean(kn * kn, axis=1) - 1.0)) <= 1e-14


# ------------------------------------------------------------- mutants ----
def _norm(x, axis, eps, root=True, mean=True):
    x = np.asarray(x, np.float64)
    ss = np.sum(x * x, axis=axis, keepdims=True) / (x.shape[axis] if mean else 1)
    return x / (np.sqrt(ss + eps) if root else np.sqrt(ss) + eps)


def _mut_k_over_keys(q, k, v, eps):
    return oracle.gqa_f64(_norm(q, 2, eps), _norm(k, 2, eps), v)


def _mut_l2_not_rms(q, k, v, eps):
    return oracle.gqa_f64(_norm(q, 2, eps, mean=False), _norm(k, 1, eps, mean=False), v)


def _mut_eps_outside_root(q, k, v, eps):
    return oracle.gqa_f64(_norm(q, 2, eps, root=False), _norm(k, 1, eps, root=False), v)


def _mut_only_q(q, k, v, eps):
    return oracle.gqa_f64(_norm(q, 2, eps), k, v)


def _mut_only_k(q, k, v, eps):
    return oracle.gqa_f64(q, _norm(k, 1, eps), v)


MUTANTS = {f.__name__: f for f in [_mut_k_over_keys, _mut_l2_not_rms, _mut_eps_outside_root,
                                   _mut_only_q, _mut_only_k]}


@pytest.mark.parametrize("mutant", list(MUTANTS))
def test_qknorm_mutant_is_caught(mutant):
    failed = []
    for name, pin in PINS.items():
        if name == "pin_bruteforce_decimal":
            continue
        try:
            with np.errstate(all="ignore"):
                pin(MUTANTS[mutant])
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(name)
    assert failed, f"mutant {mutant} passed every pin"
