"""Pins of the oracle's input decoding and temperature softmax.

The temperature softmax sigma_T(z)_i = exp(z_i / T) / sum_j exp(z_j / T) is the
one in "Speculative Decoding and Distillation", Part 2 "Loss (Hinton)"; it is
pinned against torch.softmax in float64 (a library routine), closed forms and
invariances. bf16 decoding is pinned exhaustively against torch's bfloat16.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth


def test_bf16_decode_exhaustive():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode_bf16(bits)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    np.testing.assert_array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan], ref[~nan])


def test_generator_bf16_rounding_matches_torch():
    x = np.random.default_rng(3).standard_normal(1 << 20).astype(np.float32) * 7
    x[:4] = [0.0, -0.0, 1.0 + 2.0**-8, 1.0 + 3 * 2.0**-8]  # ties to even
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(synth.to_bf16_bits(x), ref)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [1.0, 0.7, 0.05, 3.0])
def test_softmax_matches_torch_float64(dtype, T):
    rng = np.random.default_rng(7)
    V = 4099
    z32 = (rng.standard_normal((6, V)) * 3).astype(np.float32)
    z32[2, rng.choice(V, 50, replace=False)] = -np.inf
    store = synth.to_bf16_bits(z32) if dtype == "bf16" else z32
    zf = (synth.bf16_bits_to_f32(store) if dtype == "bf16" else store).astype(np.float64)
    Tf = float(np.float32(T))
    ref = torch.softmax(torch.from_numpy(zf) / Tf, dim=1).numpy()
    m, s, a, ok = oracle.row_stats(store, V, np.full(6, T, np.float32))
    assert ok.all()
    np.testing.assert_array_equal(m, zf.max(axis=1))
    np.testing.assert_array_equal(a, np.argmax(zf, axis=1))
    # S = sum exp((z - m)/T): torch's logsumexp gives log S + m/T
    lse = torch.logsumexp(torch.from_numpy(zf) / Tf, dim=1).numpy()
    np.testing.assert_allclose(np.log(s) + m / Tf, lse, rtol=0, atol=1e-12)
    for r in range(6):
        p = oracle.softmax_row(store, V, r, T)
        np.testing.assert_allclose(p, ref[r], rtol=1e-12, atol=1e-15)
        assert abs(p.sum() - 1.0) < 1e-12


def test_softmax_closed_forms():
    V = 8
    # equal logits -> uniform
    z = np.zeros((1, V), np.float32)
    np.testing.assert_array_equal(oracle.softmax_row(z, V, 0, 1.0), np.full(V, 1.0 / V))
    # two tokens: logistic sigma((a - b)/T)
    z = np.array([[1.25, -0.5]], np.float32)
    p = oracle.softmax_row(z, 2, 0, 0.5)
    want = 1.0 / (1.0 + math.exp(-(1.25 + 0.5) / 0.5))
    assert abs(p[0] - want) < 1e-15 and abs(p[1] - (1 - want)) < 1e-15
    # shift invariance, T scaling: softmax(z/T) == softmax((c*z)/(c*T))
    rng = np.random.default_rng(1)
    z = rng.standard_normal((1, 64)).astype(np.float32)
    p0 = oracle.softmax_row(z, 64, 0, 0.5)
    np.testing.assert_allclose(oracle.softmax_row(z + np.float32(3.0), 64, 0, 0.5), p0, rtol=1e-6)
    np.testing.assert_allclose(oracle.softmax_row(z * np.float32(2.0), 64, 0, 1.0), p0, rtol=1e-12)
    # masked tokens have probability exactly 0
    z = np.array([[0.0, -np.inf, 0.0, -np.inf]], np.float32)
    np.testing.assert_array_equal(oracle.softmax_row(z, 4, 0, 1.0), [0.5, 0.0, 0.5, 0.0])


def test_argmax_ties_lowest_index_and_validity():
    V = 6
    rows = np.array([[1, 3, 3, 0, 3, 2],
                     [-np.inf, -np.inf, 5, 5, -np.inf, 5],
                     [0, np.nan, 1, 2, 3, 4],
                     [0, 1, np.inf, 2, 3, 4],
                     [-np.inf] * 6,
                     [-0.0, 0.0, -0.0, 0.0, -1, -2]], np.float32)
    m, s, a, ok = oracle.row_stats(rows, V, np.zeros(6, np.float32))
    assert list(a[:2]) == [1, 2]
    assert list(ok) == [True, True, False, False, False, True]
    assert a[5] == 0  # -0.0 and +0.0 compare equal: lowest index wins
    assert np.isnan(s).all()  # greedy rows: no sum
