"""Pins for the CPU oracle: it is checked against things other than itself.

The pages print no output values for the GQA graph, so every pin comes from
the mathematics of the graph on the Mirage GQA tutorial page ("Mirage: Define
GQA Computation Graph": A = QK, E = exp(A), S = reduction(E, 2), D = E / S,
O = DV) or from library routines that compute textbook softmax attention:

* a high-precision brute force (Python ``decimal``, 60 digits) on tiny inputs;
* library witnesses: torch's scaled_dot_product_attention with scale 1 and
  scipy's softmax, both in float64 on the CPU;
* closed forms: Q = 0 or K = 0 gives the mean of V; N = 1 gives V's only row;
  N = 2 gives a logistic mix; scores (0, 1, 2) give e^j / (1 + e + e^2);
* invariants: rows are convex combinations of V rows (a ones column of V maps
  to exactly 1); a shared permutation of K's columns and V's rows changes
  nothing; adding a constant to a row's scores changes nothing; rows and
  batches are independent; a chunk-indicator V yields weight masses summing
  to 1.

``test_mutant_is_caught`` plants plausible mistakes (wrong reduction axis,
transposed operand, dropped key, missing exp, wrong sign, missing divide,
off-by-one key index) in a copy of the oracle's definition and checks that
each one fails at least one pin.
"""
from __future__ import annotations

import math
from decimal import Decimal, getcontext

import numpy as np
import pytest
import scipy.special
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


# ---------------------------------------------------------------- pins ----
# Each pin takes an implementation impl(q, k, v) -> O (float64) and raises
# AssertionError when the implementation disagrees with the pinned fact.

def pin_bruteforce_decimal(impl):
    getcontext().prec = 60
    for (B, M, N, D, seed) in [(1, 1, 1, 4, 1), (2, 3, 5, 8, 2), (1, 2, 17, 64, 3),
                               (2, 2, 2, 64, 4), (1, 1, 40, 16, 5)]:
        q, k, v = make_qkv(B, M, N, seed=seed, qk_std=0.5, D=D)
        o = impl(q, k, v)
        exact = np.zeros((B, M, D))
        for b in range(B):
            for i in range(M):
                a = [sum(Decimal(float(q[b, i, d])) * Decimal(float(k[b, d, n]))
                         for d in range(D)) for n in range(N)]
                e = [x.exp() for x in a]
                s = sum(e)
                for j in range(D):
                    exact[b, i, j] = float(sum(e[n] / s * Decimal(float(v[b, n, j]))
                                               for n in range(N)))
        _rel_close(o, exact, rtol=1e-13)


def pin_sdpa_witness(impl):
    for (B, M, N, D, std, seed) in [(3, 7, 301, 64, 0.3, 11), (2, 5, 1000, 16, 0.5, 12),
                                    (1, 33, 64, 64, 0.25, 13)]:
        q, k, v = make_qkv(B, M, N, seed=seed, qk_std=std, D=D)
        o = impl(q, k, v)
        tq = torch.from_numpy(q.astype(np.float64))
        tk = torch.from_numpy(np.ascontiguousarray(k.astype(np.float64).transpose(0, 2, 1)))
        tv = torch.from_numpy(v.astype(np.float64))
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=1.0).numpy()
        _rel_close(o, ref, rtol=1e-12)


def pin_scipy_softmax_witness(impl):
    q, k, v = make_qkv(2, 9, 130, seed=21, qk_std=0.4)
    o = impl(q, k, v)
    q64, k64, v64 = (x.astype(np.float64) for x in (q, k, v))
    scores = np.einsum("bid,bdn->bin", q64, k64)
    ref = np.einsum("bin,bnj->bij", scipy.special.softmax(scores, axis=-1), v64)
    _rel_close(o, ref, rtol=1e-12)


def pin_zero_q_or_k_gives_mean(impl):
    q, k, v = make_qkv(2, 4, 77, seed=31)
    mean = v.astype(np.float64).mean(axis=1, keepdims=True)
    expect = np.broadcast_to(mean, (2, 4, 64))
    _rel_close(impl(np.zeros_like(q), k, v), expect, rtol=1e-13)
    _rel_close(impl(q, np.zeros_like(k), v), expect, rtol=1e-13)


def pin_single_key(impl):
    q, k, v = make_qkv(3, 5, 1, seed=41, qk_std=1.0)
    expect = np.broadcast_to(v.astype(np.float64)[:, 0:1, :], (3, 5, 64))
    _rel_close(impl(q, k, v), expect, rtol=0, atol=1e-15)


def pin_two_keys_logistic(impl):
    q, k, v = make_qkv(2, 6, 2, seed=51, qk_std=0.5)
    o = impl(q, k, v)
    for b in range(2):
        for i in range(6):
            a0 = math.fsum(float(q[b, i, d]) * float(k[b, d, 0]) for d in range(64))
            a1 = math.fsum(float(q[b, i, d]) * float(k[b, d, 1]) for d in range(64))
            w0 = 1.0 / (1.0 + math.exp(a1 - a0))
            w1 = 1.0 / (1.0 + math.exp(a0 - a1))
            expect = w0 * v[b, 0].astype(np.float64) + w1 * v[b, 1].astype(np.float64)
            _rel_close(o[b, i], expect, rtol=1e-14)


def pin_softmax_of_0_1_2(impl):
    # Scores (0, 1, 2) for query row 0; V holds unit vectors, so O[0, j] is
    # the j-th softmax weight e^j / (1 + e + e^2).
    q = np.zeros((1, 1, 64), np.float16)
    q[0, 0, 0] = 1.0
    k = np.zeros((1, 64, 3), np.float16)
    k[0, 0, :] = [0.0, 1.0, 2.0]
    v = np.zeros((1, 3, 64), np.float16)
    for n in range(3):
        v[0, n, n] = 1.0
    denom = 1.0 + math.e + math.e ** 2
    expect = np.zeros((1, 1, 64))
    expect[0, 0, :3] = [1.0 / denom, math.e / denom, math.e ** 2 / denom]
    _rel_close(impl(q, k, v), expect, rtol=1e-15)


def pin_convex_and_ones_column(impl):
    q, k, v = make_qkv(2, 8, 200, seed=61, qk_std=0.5)
    v = v.copy()
    v[:, :, 5] = 1.0
    o = impl(q, k, v)
    v64 = v.astype(np.float64)
    lo = v64.min(axis=1, keepdims=True)
    hi = v64.max(axis=1, keepdims=True)
    assert np.all(o >= lo - 1e-14) and np.all(o <= hi + 1e-14)
    assert np.max(np.abs(o[:, :, 5] - 1.0)) <= 1e-14


def pin_key_permutation(impl):
    q, k, v = make_qkv(2, 5, 97, seed=71, qk_std=0.5)
    perm = np.random.Generator(np.random.PCG64(7)).permutation(97)
    o = impl(q, k, v)
    o_p = impl(q, np.ascontiguousarray(k[:, :, perm]), np.ascontiguousarray(v[:, perm, :]))
    _rel_close(o_p, o, rtol=1e-13)


def pin_row_shift(impl):
    # With K[b, d0, :] constant, Q[b, i, d0] only adds a constant to row i's
    # scores, which the normalisation removes.
    q, k, v = make_qkv(2, 4, 60, seed=81, qk_std=0.5)
    k = k.copy()
    k[:, 3, :] = 0.5
    q2 = q.copy()
    q2[:, :, 3] += np.float16(1.25)
    _rel_close(impl(q2, k, v), impl(q, k, v), rtol=1e-13)


def pin_row_and_batch_independence(impl):
    q, k, v = make_qkv(3, 6, 50, seed=91, qk_std=0.5)
    o = impl(q, k, v)
    _rel_close(impl(np.ascontiguousarray(q[:, 2:4]), k, v), o[:, 2:4], rtol=0, atol=0)
    _rel_close(impl(q[1:2], k[1:2], v[1:2]), o[1:2], rtol=0, atol=0)


def pin_chunk_indicator(impl):
    # V[b, n, j] = 1 iff key n lies in the j-th of 64 equal key ranges, so
    # O[b, i, j] is that range's weight mass and each row of O sums to 1.
    r = 3
    N = 64 * r
    q, k, _ = make_qkv(2, 4, N, seed=101, qk_std=0.5)
    v = np.zeros((2, N, 64), np.float16)
    for n in range(N):
        v[:, n, n // r] = 1.0
    o = impl(q, k, v)
    assert np.max(np.abs(o.sum(axis=2) - 1.0)) <= 1e-13
    o0 = impl(np.zeros_like(q), k, v)
    assert np.max(np.abs(o0 - r / N)) <= 1e-15


PINS = {f.__name__: f for f in [
    pin_bruteforce_decimal, pin_sdpa_witness, pin_scipy_softmax_witness,
    pin_zero_q_or_k_gives_mean, pin_single_key, pin_two_keys_logistic,
    pin_softmax_of_0_1_2, pin_convex_and_ones_column, pin_key_permutation,
    pin_row_shift, pin_row_and_batch_independence, pin_chunk_indicator]}

IMPLS = {"c_loops": oracle.gqa_f64, "numpy": oracle.gqa_numpy_f64}


@pytest.mark.parametrize("impl_name", list(IMPLS))
@pytest.mark.parametrize("pin_name", list(PINS))
def test_oracle_pin(impl_name, pin_name):
    PINS[pin_name](IMPLS[impl_name])


def test_c_and_numpy_twins_agree():
    q, k, v = make_qkv(3, 17, 515, seed=5, qk_std=0.3)
    _rel_close(oracle.gqa_f64(q, k, v), oracle.gqa_numpy_f64(q, k, v), rtol=1e-13)


def test_oracle_rejects_empty_keys_and_allows_empty_rows():
    q = np.zeros((1, 2, 64), np.float16)
    with pytest.raises(ValueError):
        oracle.gqa_f64(q, np.zeros((1, 64, 0), np.float16), np.zeros((1, 0, 64), np.float16))
    k = np.zeros((1, 64, 8), np.float16)
    v = np.zeros((1, 8, 64), np.float16)
    assert oracle.gqa_f64(np.zeros((1, 0, 64), np.float16), k, v).shape == (1, 0, 64)
    assert oracle.gqa_f64(np.zeros((0, 2, 64), np.float16), k[:0], v[:0]).shape == (0, 2, 64)


# ------------------------------------------------------------- mutants ----
def _f64(*xs):
    return [np.asarray(x, np.float64) for x in xs]


def _mut_axis(q, k, v):        # reduction over the query axis instead of keys
    q, k, v = _f64(q, k, v)
    E = np.exp(q @ k)
    return (E / E.sum(axis=1, keepdims=True)) @ v


def _mut_k_transposed(q, k, v):  # K read as (N, D) row-major
    q, k, v = _f64(q, k, v)
    B, D, N = k.shape
    E = np.exp(q @ k.reshape(B, N, D).transpose(0, 2, 1))
    return (E / E.sum(axis=2, keepdims=True)) @ v


def _mut_v_transposed(q, k, v):  # V read as (D, N) row-major
    q, k, v = _f64(q, k, v)
    B, N, D = v.shape
    E = np.exp(q @ k)
    return (E / E.sum(axis=2, keepdims=True)) @ v.reshape(B, D, N).transpose(0, 2, 1)


def _mut_drop_last_key_in_sum(q, k, v):
    q, k, v = _f64(q, k, v)
    E = np.exp(q @ k)
    return (E / E[:, :, :-1].sum(axis=2, keepdims=True)) @ v if E.shape[2] > 1 else \
        (E / (E.sum(axis=2, keepdims=True) * 2)) @ v


def _mut_no_exp(q, k, v):
    q, k, v = _f64(q, k, v)
    E = q @ k
    return (E / E.sum(axis=2, keepdims=True)) @ v


def _mut_negated_scores(q, k, v):
    q, k, v = _f64(q, k, v)
    E = np.exp(-(q @ k))
    return (E / E.sum(axis=2, keepdims=True)) @ v


def _mut_no_divide(q, k, v):
    q, k, v = _f64(q, k, v)
    return np.exp(q @ k) @ v


def _mut_key_off_by_one(q, k, v):  # scores of key n paired with V row n+1
    q, k, v = _f64(q, k, v)
    E = np.exp(q @ k)
    return (E / E.sum(axis=2, keepdims=True)) @ np.roll(v, 1, axis=1)


MUTANTS = {f.__name__: f for f in [
    _mut_axis, _mut_k_transposed, _mut_v_transposed, _mut_drop_last_key_in_sum,
    _mut_no_exp, _mut_negated_scores, _mut_no_divide, _mut_key_off_by_one]}


@pytest.mark.parametrize("mutant", list(MUTANTS))
def test_mutant_is_caught(mutant):
    impl = MUTANTS[mutant]
    failed = []
    for name, pin in PINS.items():
        if name == "pin_bruteforce_decimal":
            continue  # slowest pin; the cheaper ones must already catch every mutant
        try:
            with np.errstate(all="ignore"):
                pin(impl)
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(name)
    assert failed, f"mutant {mutant} passed every pin"
