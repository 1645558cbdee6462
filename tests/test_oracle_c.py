"""Pins of the C form of the oracle (oracle/layer_ref.c through oracle.cref), the one the CPU
baseline times: against the pure-Python brute force (exact rational projections, correctly
rounded sums), against the numpy form on a larger case, against library dtype conversions for
the rounding, and against closed forms; its results do not depend on the thread count."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import brute, cref
from synth import Draw

DTYPES = ["f32", "f16", "bf16"]


@pytest.fixture(scope="module", autouse=True)
def _built():
    cref.build()


def _random_layer(seed, B, T, past, D, Hq, Hkv, d, dtype, cap=None):
    dr = Draw(seed)
    wq = dr.weights(D, Hq * d, dtype)
    wk = dr.weights(D, Hkv * d, dtype)
    wv = dr.weights(D, Hkv * d, dtype)
    x = dr.normal((B, T, D), 1.0, dtype)
    cap = cap or (max(past) + T + 3)
    kc = np.zeros((B, Hkv, cap, d), dtype=np.float32)
    vc = np.zeros((B, Hkv, cap, d), dtype=np.float32)
    for b in range(B):
        kc[b, :, :past[b]] = dr.normal((Hkv, past[b], d), 1.0, dtype)
        vc[b, :, :past[b]] = dr.normal((Hkv, past[b], d), 1.0, dtype)
    return x, wq, wk, wv, kc, vc, np.array(past, dtype=np.int32)


def _lists(*arrays):
    return [np.asarray(a, dtype=np.float64).tolist() for a in arrays]


@pytest.mark.parametrize("dtype", DTYPES)
def test_rounding_matches_exact_neighbour_search(dtype):
    """oref_round against brute.representable_round (exact rationals): random values over many
    binades, exact ties, subnormals, and values past the largest finite one."""
    dr = np.random.default_rng(3)
    p = {"f32": 24, "f16": 11, "bf16": 8}[dtype]
    vals = list(dr.standard_normal(300) * np.exp2(dr.integers(-30, 30, 300)))
    vals += [1.0 + 2.0 ** -p, 1.0 + 3 * 2.0 ** -p, -(1.0 + 2.0 ** -p), 2.0 ** -140, 3.3e-8, -6.1e-5,
             65519.0, 65520.0, 3.4e38, 3.5e38, 0.0]
    for v in vals:
        want = brute.representable_round(Fraction(float(v)), dtype)
        got = cref.round_to_dtype(v, dtype)
        assert got == float(want), (v, got, float(want))


def test_rounding_matches_library_casts():
    """f32 and f16 rounding against numpy's casts, bf16 against torch's (all ties to even)."""
    import torch
    v = np.random.default_rng(4).standard_normal(2000) * np.exp2(np.random.default_rng(5).integers(-20, 20, 2000))
    assert all(cref.round_to_dtype(a, "f32") == float(np.float32(a)) for a in v)
    assert all(cref.round_to_dtype(a, "f16") == float(np.float16(a)) for a in v[np.abs(v) < 6e4])
    bf = torch.from_numpy(v).to(torch.bfloat16).double().numpy()
    assert all(cref.round_to_dtype(a, "bf16") == b for a, b in zip(v, bf))


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("shape", [
    dict(B=2, T=3, past=[2, 5], D=8, Hq=4, Hkv=2, d=4),
    dict(B=1, T=5, past=[0], D=6, Hq=2, Hkv=2, d=8),
    dict(B=2, T=1, past=[7, 1], D=12, Hq=6, Hkv=3, d=4),
    dict(B=1, T=18, past=[3], D=8, Hq=2, Hkv=1, d=4),      # two blocks of query tokens
])
def test_c_oracle_matches_brute_force(dtype, shape):
    x, wq, wk, wv, kc, vc, past = _random_layer(17, shape["B"], shape["T"], shape["past"], shape["D"],
                                                shape["Hq"], shape["Hkv"], shape["d"], dtype)
    kb, vb = _lists(kc, vc)
    got = cref.layer_step(x, wq, wk, wv, kc, vc, past, shape["Hq"], dtype, threads=3)
    ref = brute.layer_step(*_lists(x, wq, wk, wv), kb, vb, [int(p) for p in past], shape["Hq"], dtype)
    np.testing.assert_allclose(got, np.array(ref), rtol=1e-12, atol=1e-13)
    assert np.array_equal(kc.astype(np.float64), np.array(kb))
    assert np.array_equal(vc.astype(np.float64), np.array(vb))


def test_c_oracle_matches_numpy_oracle_with_sampled_tokens():
    """A larger ragged GQA case (G = 4, d = 128), every token and a sample of tokens, against the
    numpy form of the oracle; the appended rows are the same bits."""
    x, wq, wk, wv, kc, vc, past = _random_layer(18, 3, 40, [0, 300, 77], 256, 8, 2, 128, "bf16")
    kn, vn = kc.copy(), vc.copy()
    ref = oracle.layer_step(x, wq, wk, wv, kn, vn, past, 8, "bf16")
    got = cref.layer_step(x, wq, wk, wv, kc, vc, past, 8, "bf16")
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)
    assert np.array_equal(kc, kn) and np.array_equal(vc, vn)
    ts = np.array([0, 17, 39])
    kc2, vc2 = _random_layer(18, 3, 40, [0, 300, 77], 256, 8, 2, 128, "bf16")[4:6]
    got_s = cref.layer_step(x, wq, wk, wv, kc2, vc2, past, 8, "bf16", t_index=ts)
    np.testing.assert_allclose(got_s, ref[:, ts], rtol=1e-12, atol=1e-13)


def test_results_do_not_depend_on_the_thread_count():
    x, wq, wk, wv, kc, vc, past = _random_layer(19, 2, 37, [5, 60], 64, 8, 2, 32, "f16")
    outs = []
    for th in (1, 3, 8):
        k, v = kc.copy(), vc.copy()
        outs.append((cref.layer_step(x, wq, wk, wv, k, v, past, 8, "f16", threads=th), k, v))
    for o, k, v in outs[1:]:
        assert np.array_equal(o, outs[0][0]) and np.array_equal(k, outs[0][1]) and np.array_equal(v, outs[0][2])


def test_closed_forms():
    """Equal keys give the mean of the visible value rows; the first token of an empty cache
    attends to itself only and returns its own (rounded) value row."""
    B, T, D, Hq, Hkv, d = 1, 6, 8, 2, 1, 4
    dr = Draw(20)
    x = dr.normal((B, T, D), 1.0, "f32")
    wq = dr.weights(D, Hq * d, "f32")
    wv = dr.weights(D, Hkv * d, "f32")
    wk = np.zeros((D, Hkv * d), dtype=np.float32)          # every new key is 0 -> all scores equal
    past = np.array([5], dtype=np.int32)
    kc = np.zeros((B, Hkv, 16, d), dtype=np.float32)
    vc = np.zeros_like(kc)
    vc[0, 0, :5] = dr.normal((5, d), 1.0, "f32")
    out = cref.layer_step(x, wq, wk, wv, kc, vc, past, Hq, "f32")
    for t in range(T):
        want = vc[0, 0, :5 + t + 1].astype(np.float64).mean(axis=0)
        for h in range(Hq):
            np.testing.assert_allclose(out[0, t, h], want, rtol=1e-13, atol=1e-14)
    kc0, vc0 = np.zeros((B, Hkv, 8, d), dtype=np.float32), np.zeros((B, Hkv, 8, d), dtype=np.float32)
    out0 = cref.layer_step(x, wq, dr.weights(D, Hkv * d, "f32"), wv, kc0, vc0, np.array([0], np.int32), Hq, "bf16")
    for h in range(Hq):
        assert np.array_equal(out0[0, 0, h], vc0[0, 0, 0].astype(np.float64))


def test_refuses_appends_past_capacity():
    x, wq, wk, wv, kc, vc, past = _random_layer(21, 1, 4, [2], 8, 2, 1, 4, "f32", cap=5)
    with pytest.raises(ValueError):
        cref.layer_step(x, wq, wk, wv, kc, vc, past, 2, "f32")
