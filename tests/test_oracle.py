"""Pins for the oracle: checks against facts that do not come from the oracle itself.

Each test names what fixes the expected value: a closed form, an invariant of softmax
attention, an exact-arithmetic construction, a library routine, or the independent
pure-Python brute force in oracle/brute.py.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import brute
import synth
from synth import Draw, quantize

DTYPES = ["f32", "f16", "bf16"]


# ---------------------------------------------------------------- rounding to storage

def _wide_doubles(n, seed):
    rng = np.random.default_rng(seed)
    mant = rng.uniform(-2.0, 2.0, n)
    exps = rng.integers(-160, 140, n)
    return np.ldexp(mant, exps)


@pytest.mark.parametrize("dtype,npdt", [("f16", np.float16), ("f32", np.float32)])
def test_round_matches_numpy_casts(dtype, npdt):
    """numpy's float64 -> float16/float32 casts are correctly rounded (ties to even)."""
    x = _wide_doubles(200000, 1)
    x = np.concatenate([x, [0.0, -0.0, 65504.0, 65520.0, 65519.99, 2.0 ** -24, 2.0 ** -25,
                            3 * 2.0 ** -26, 1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11,
                            np.inf, -np.inf, 3.4028235677973366e38, 3.4028235e38 * 1.0000001]])
    with np.errstate(over="ignore"):
        want = x.astype(npdt).astype(np.float64)
    got = oracle.round_to_dtype(x, dtype)
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))


def test_round_bf16_closed_forms():
    """Ties and edges of bfloat16 (8-bit significand, fp32 exponent range)."""
    cases = {
        1 + 2.0 ** -8: 1.0,                      # tie -> even significand (1.0000000)
        1 + 3 * 2.0 ** -8: 1 + 2.0 ** -6,        # tie -> even (1.0000010)
        1 + 2.0 ** -8 + 2.0 ** -30: 1 + 2.0 ** -7,
        2.0 ** -134: 0.0,                        # half of the smallest subnormal -> 0
        3 * 2.0 ** -134: 2.0 ** -132,            # tie between 1 and 2 quanta -> 2
        (2 - 2.0 ** -8) * 2.0 ** 127: math.inf,  # max + half ulp ties to the even 2^128
        (2 - 2.0 ** -7) * 2.0 ** 127: (2 - 2.0 ** -7) * 2.0 ** 127,
        -(1 + 2.0 ** -8): -1.0,
    }
    for x, want in cases.items():
        assert oracle.round_to_dtype(np.array([x]), "bf16")[0] == want, x


@pytest.mark.parametrize("dtype", DTYPES)
def test_round_matches_exact_search(dtype):
    """Against brute.representable_round, which searches neighbours in exact rationals."""
    x = _wide_doubles(3000, 2)
    got = oracle.round_to_dtype(x, dtype)
    for xi, gi in zip(x, got):
        want = brute.representable_round(Fraction(float(xi)), dtype)
        assert gi == float(want), (xi, gi, want)


def test_synth_inputs_are_representable():
    d = Draw(5)
    for dt in DTYPES:
        a = d.normal((1000,), 1.0, dt).astype(np.float64)
        assert np.array_equal(oracle.round_to_dtype(a, dt), a)


# ---------------------------------------------------------------- projection + append

def _exact_inputs(rng, B, T, D, ncols):
    """Integer X in [-8, 8]; W with at most 8 entries of +-1 per column. Every sum is an
    integer of magnitude <= 64, exact in every dtype and in any summation order."""
    x = rng.integers(-8, 9, size=(B, T, D)).astype(np.float64)
    w = np.zeros((D, ncols))
    for c in range(ncols):
        rows = rng.choice(D, size=min(8, D), replace=False)
        w[rows, c] = rng.choice([-1.0, 1.0], size=len(rows))
    return x, w


def test_projection_exact_against_rationals():
    rng = np.random.default_rng(3)
    x, w = _exact_inputs(rng, 2, 5, 40, 24)
    got = oracle.project(x, w)
    for b in range(2):
        for t in range(5):
            for c in range(24):
                want = sum(Fraction(int(x[b, t, k])) * Fraction(int(w[k, c])) for k in range(40))
                assert got[b, t, c] == float(want)


def test_projection_one_hot_rows_select_weight_rows():
    rng = np.random.default_rng(4)
    D, n = 16, 12
    w = rng.standard_normal((D, n))
    x = np.zeros((1, D, D))
    x[0, np.arange(D), rng.permutation(D)] = 1.0
    got = oracle.project(x, w)[0]
    for t in range(D):
        assert np.array_equal(got[t], w[np.argmax(x[0, t])])


@pytest.mark.parametrize("dtype", DTYPES)
def test_append_position_coded_with_canaries(dtype):
    """Row t of sequence b carries 100*b + t; every row outside the range stays NaN."""
    B, T, H, cap, d, D = 3, 4, 2, 16, 8, 4
    past = np.array([3, 0, 12], dtype=np.int32)
    x = np.zeros((B, T, D))
    for b in range(B):
        for t in range(T):
            x[b, t, 0] = 100 * b + t
    wk = np.zeros((D, H * d))
    wk[0, :] = 1.0                       # passes column 0 of X to every output
    cache = np.full((B, H, cap, d), np.nan, dtype=np.float32)
    oracle.append(cache, oracle.project(x, wk).reshape(B, T, H, d), past, dtype)
    for b in range(B):
        for g in range(H):
            for r in range(cap):
                if past[b] <= r < past[b] + T:
                    assert np.all(cache[b, g, r] == 100 * b + (r - past[b]))
                else:
                    assert np.all(np.isnan(cache[b, g, r]))


def test_append_rejects_overflowing_capacity():
    cache = np.zeros((1, 1, 8, 4), dtype=np.float32)
    with pytest.raises(ValueError):
        oracle.append(cache, np.zeros((1, 3, 1, 4)), [6], "f32")
    with pytest.raises(ValueError):
        oracle.append(cache, np.zeros((1, 1, 1, 4)), [-1], "f32")


@pytest.mark.parametrize("dtype", DTYPES)
def test_append_rounds_to_cache_dtype(dtype):
    rng = np.random.default_rng(6)
    rows = rng.standard_normal((1, 5, 2, 8))
    cache = np.zeros((1, 2, 8, 8))
    oracle.append(cache, rows, [1], dtype)
    for t in range(5):
        for g in range(2):
            for i in range(8):
                want = brute.representable_round(Fraction(float(rows[0, t, g, i])), dtype)
                assert cache[0, g, 1 + t, i] == float(want)


# ---------------------------------------------------------------- attention invariants

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


def test_two_key_closed_form():
    """Scores 0 and ln 3 give weights 1/4 and 3/4."""
    d = 4
    kc = np.zeros((1, 1, 4, d))
    vc = np.zeros((1, 1, 4, d))
    kc[0, 0, 1, 0] = 1.0                    # key 0 = 0, key 1 = e0
    vc[0, 0, 0] = [4.0, 0.0, -8.0, 1.0]
    vc[0, 0, 1] = [0.0, 8.0, 4.0, 1.0]
    q = np.zeros((1, 1, 1, d))
    q[0, 0, 0, 0] = 2.0 * math.log(3.0)     # s1 = q.e0 / sqrt(4) = ln 3
    out = oracle.attention(q, kc, vc, [1])
    want = 0.25 * vc[0, 0, 0] + 0.75 * vc[0, 0, 1]
    np.testing.assert_allclose(out[0, 0, 0], want, rtol=0, atol=1e-14)


@pytest.mark.parametrize("dtype", DTYPES)
def test_constant_values_return_the_constant(dtype):
    """softmax weights sum to one: V = c everywhere gives O = c for every query."""
    x, wq, wk, wv, kc, vc, past = _random_layer(7, 2, 6, [5, 9], 32, 4, 2, 16, dtype)
    wv = np.zeros_like(wv)
    c = 0.375
    vc[:] = c
    # with Wv = 0 the appended rows are 0, so make them c through a bias-free trick:
    # set X column 0 to 1 for every row and pass it through Wv scaled by c.
    x = x.copy()
    x[:, :, 0] = 1.0
    wv[0, :] = c
    out = oracle.layer_step(x, wq, wk, wv, kc, vc, past, 4, dtype)
    np.testing.assert_allclose(out, c, rtol=1e-15, atol=0)


@pytest.mark.parametrize("dtype", DTYPES)
def test_single_key_returns_its_value(dtype):
    """An empty cache and one new token: the only key is the token's own."""
    x, wq, wk, wv, kc, vc, past = _random_layer(8, 2, 1, [0, 0], 32, 4, 2, 16, dtype)
    out = oracle.layer_step(x, wq, wk, wv, kc, vc, past, 4, dtype)
    for b in range(2):
        for h in range(4):
            np.testing.assert_allclose(out[b, 0, h], vc[b, h // 2, 0], rtol=1e-15, atol=0)


def test_first_prefill_row_sees_only_itself():
    x, wq, wk, wv, kc, vc, past = _random_layer(9, 1, 7, [0], 32, 2, 1, 16, "bf16")
    out = oracle.layer_step(x, wq, wk, wv, kc, vc, past, 2, "bf16")
    np.testing.assert_allclose(out[0, 0, 0], vc[0, 0, 0], rtol=1e-15, atol=0)
    np.testing.assert_allclose(out[0, 0, 1], vc[0, 0, 0], rtol=1e-15, atol=0)


def test_zero_keys_give_the_prefix_mean():
    """Wk = 0 makes every score 0: query at position p returns mean(V[0..p])."""
    rng = np.random.default_rng(10)
    B, T, D, Hq, Hkv, d = 2, 5, 24, 4, 2, 8
    past = np.array([3, 6], dtype=np.int32)
    x, wv = _exact_inputs(rng, B, T, D, Hkv * d)
    wq = rng.standard_normal((D, Hq * d))
    wk = np.zeros((D, Hkv * d))
    cap = 12
    kc = np.zeros((B, Hkv, cap, d))
    vc = np.zeros((B, Hkv, cap, d))
    for b in range(B):
        vc[b, :, :past[b]] = rng.integers(-20, 21, size=(Hkv, past[b], d))
    out = oracle.layer_step(x, wq, wk, wv, kc, vc, past, Hq, "f32")
    for b in range(B):
        for t in range(T):
            p = past[b] + t
            for h in range(Hq):
                g = h // 2
                for i in range(d):
                    want = Fraction(sum(int(v) for v in vc[b, g, :p + 1, i]), p + 1)
                    assert abs(out[b, t, h, i] - float(want)) <= 1e-14 * max(1.0, abs(float(want)))


def test_gqa_equals_mha_with_repeated_kv_heads():
    rng = np.random.default_rng(11)
    B, n, Hq, Hkv, d, cap = 2, 3, 8, 2, 16, 20
    q = rng.standard_normal((B, n, Hq, d))
    kc = rng.standard_normal((B, Hkv, cap, d))
    vc = rng.standard_normal((B, Hkv, cap, d))
    past = [7, 12]
    gqa = oracle.attention(q, kc, vc, past)
    mha = oracle.attention(q, np.repeat(kc, Hq // Hkv, axis=1), np.repeat(vc, Hq // Hkv, axis=1), past)
    assert np.array_equal(gqa, mha)


def test_causal_perturbation_leaves_earlier_rows_bit_identical():
    args = _random_layer(12, 2, 9, [4, 0], 32, 4, 2, 16, "bf16")
    x, wq, wk, wv, kc, vc, past = args
    base = oracle.layer_step(x, wq, wk, wv, kc.copy(), vc.copy(), past, 4, "bf16")
    x2 = x.copy()
    x2[:, 5:, :] = quantize(np.random.default_rng(0).standard_normal(x2[:, 5:, :].shape), "bf16")
    pert = oracle.layer_step(x2, wq, wk, wv, kc.copy(), vc.copy(), past, 4, "bf16")
    assert np.array_equal(base[:, :5], pert[:, :5])
    assert not np.array_equal(base[:, 5:], pert[:, 5:])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_phase_consistency(dtype):
    """prefill(T) == prefill(T1) then prefill(T - T1) == T single-token steps."""
    x, wq, wk, wv, kc, vc, past = _random_layer(13, 2, 6, [3, 8], 32, 4, 2, 16, dtype)
    whole = oracle.layer_step(x, wq, wk, wv, kc.copy(), vc.copy(), past, 4, dtype)
    k2, v2 = kc.copy(), vc.copy()
    a = oracle.layer_step(x[:, :2], wq, wk, wv, k2, v2, past, 4, dtype)
    b = oracle.layer_step(x[:, 2:], wq, wk, wv, k2, v2, past + 2, 4, dtype)
    np.testing.assert_allclose(np.concatenate([a, b], axis=1), whole, rtol=1e-12, atol=1e-13)
    k3, v3 = kc.copy(), vc.copy()
    steps = [oracle.layer_step(x[:, t:t + 1], wq, wk, wv, k3, v3, past + t, 4, dtype) for t in range(6)]
    np.testing.assert_allclose(np.concatenate(steps, axis=1), whole, rtol=1e-12, atol=1e-13)
    assert np.array_equal(k2, k3) and np.array_equal(v2, v3)


def test_permuting_past_rows_leaves_decode_unchanged():
    """No positional encoding: past (K, V) rows can be permuted together."""
    x, wq, wk, wv, kc, vc, past = _random_layer(14, 1, 1, [11], 32, 4, 2, 16, "f32")
    base = oracle.layer_step(x, wq, wk, wv, kc.copy(), vc.copy(), past, 4, "f32")
    perm = np.random.default_rng(1).permutation(11)
    k2, v2 = kc.copy(), vc.copy()
    k2[:, :, :11] = kc[:, :, perm]
    v2[:, :, :11] = vc[:, :, perm]
    out = oracle.layer_step(x, wq, wk, wv, k2, v2, past, 4, "f32")
    np.testing.assert_allclose(out, base, rtol=1e-13, atol=1e-14)


def test_reciprocal_scaling_of_wq_and_wk_is_exact():
    """(4·Wq, Wk/4) leaves every score unchanged (powers of two scale exactly)."""
    x, wq, wk, wv, kc, vc, past = _random_layer(15, 2, 4, [6, 2], 32, 4, 2, 16, "f32")
    base = oracle.layer_step(x, wq, wk, wv, kc.copy(), vc.copy(), past, 4, "f32")
    k2 = kc.copy() / 4
    out = oracle.layer_step(x, wq * 4, wk / 4, wv, k2, vc.copy(), past, 4, "f32")
    assert np.array_equal(out, base)


def test_large_scores_stay_finite_and_match_brute_force():
    """Scores around 30x their usual size: no overflow, same as the brute force."""
    x, wq, wk, wv, kc, vc, past = _random_layer(16, 1, 3, [4], 8, 2, 1, 4, "f32")
    x = x * 30.0
    kc[:, :, :4] *= 30.0
    got = oracle.layer_step(x, wq, wk, wv, kc.copy(), vc.copy(), past, 2, "f32")
    assert np.all(np.isfinite(got))
    ref = brute.layer_step(x.tolist(), wq.tolist(), wk.tolist(), wv.tolist(),
                           kc.astype(np.float64).tolist(), vc.astype(np.float64).tolist(),
                           [int(p) for p in past], 2, "f32")
    np.testing.assert_allclose(got, np.array(ref), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("shape", [
    dict(B=2, T=3, past=[2, 5], D=8, Hq=4, Hkv=2, d=4),
    dict(B=1, T=5, past=[0], D=6, Hq=2, Hkv=2, d=8),
    dict(B=2, T=1, past=[7, 1], D=12, Hq=6, Hkv=3, d=4),
])
def test_whole_oracle_matches_brute_force(dtype, shape):
    x, wq, wk, wv, kc, vc, past = _random_layer(17, shape["B"], shape["T"], shape["past"],
                                                shape["D"], shape["Hq"], shape["Hkv"], shape["d"],
                                                dtype)
    kb, vb = kc.astype(np.float64).tolist(), vc.astype(np.float64).tolist()
    got = oracle.layer_step(x, wq, wk, wv, kc, vc, past, shape["Hq"], dtype)
    ref = brute.layer_step(x.tolist(), wq.tolist(), wk.tolist(), wv.tolist(), kb, vb,
                           [int(p) for p in past], shape["Hq"], dtype)
    np.testing.assert_allclose(got, np.array(ref), rtol=1e-12, atol=1e-13)
    # the appended cache rows are identical to the brute force's exact rounding
    assert np.array_equal(kc.astype(np.float64), np.array(kb))
    assert np.array_equal(vc.astype(np.float64), np.array(vb))


def test_empty_step_returns_nothing():
    x, wq, wk, wv, kc, vc, past = _random_layer(18, 1, 0, [3], 8, 2, 1, 4, "f32")
    before = kc.copy()
    out = oracle.layer_step(x, wq, wk, wv, kc, vc, past, 2, "f32")
    assert out.shape == (1, 0, 2, 4)
    assert np.array_equal(before, kc)


# ---- paged cache: gather_pages is the block-table mapping, pinned by construction and loops

def test_gather_pages_of_an_in_order_pool_is_the_contiguous_cache():
    # a contiguous cache cut into 16-row pages in order, table = identity
    rng = np.random.default_rng(40)
    H, d, n_pages = 3, 4, 5
    cache = rng.standard_normal((1, H, 16 * n_pages, d))
    pool = np.zeros((n_pages, H, 16, d))
    for p in range(n_pages):
        for g in range(H):
            for r in range(16):
                pool[p, g, r] = cache[0, g, 16 * p + r]
    got = oracle.gather_pages(pool, np.arange(n_pages)[None, :], [16 * n_pages])
    assert np.array_equal(got, cache)


def test_gather_pages_matches_loops_on_a_shuffled_table():
    rng = np.random.default_rng(41)
    H, d, n_pages, B, max_pages = 2, 3, 11, 3, 4
    pool = rng.standard_normal((n_pages, H, 16, d))
    perm = rng.permutation(n_pages)
    table = perm[: B * max_pages - 1].tolist() + [perm[0]]     # one page shared (read-only)
    table = np.array(table).reshape(B, max_pages)
    n_tokens = [37, 64, 1]
    got = oracle.gather_pages(pool, table, n_tokens)
    assert got.shape == (B, H, 64, d)
    for b in range(B):
        for g in range(H):
            for j in range(64):
                if j < n_tokens[b]:
                    page, row = table[b][j // 16], j % 16
                    assert np.array_equal(got[b, g, j], pool[page, g, row])
                else:
                    assert np.isnan(got[b, g, j]).all()


def test_paged_layer_step_equals_contiguous_layer_step():
    # the same logical cache as pages or contiguous gives the same layer step
    x, wq, wk, wv, kc, vc, past = _random_layer(42, 2, 3, [20, 33], 8, 4, 2, 4, "bf16")
    B, Hkv, cap, d = kc.shape
    n_lp = (cap + 15) // 16
    rng = np.random.default_rng(43)
    perm = rng.permutation(B * n_lp)
    table = perm.reshape(B, n_lp)
    pool_k = np.full((B * n_lp, Hkv, 16, d), np.nan)
    pool_v = np.full((B * n_lp, Hkv, 16, d), np.nan)
    for b in range(B):
        for j in range(cap):
            pool_k[table[b, j // 16], :, j % 16] = kc[b, :, j]
            pool_v[table[b, j // 16], :, j % 16] = vc[b, :, j]
    want = oracle.layer_step(x, wq, wk, wv, kc, vc, past, 4, "bf16")
    n_tok = [int(p) + 3 for p in past]
    kg = oracle.gather_pages(pool_k, table, [cap, cap])
    vg = oracle.gather_pages(pool_v, table, [cap, cap])
    got = oracle.layer_step(x, wq, wk, wv, kg, vg, past, 4, "bf16")
    assert np.array_equal(got, want)
    assert max(n_tok) <= cap


# ---- decoder-stack pieces around the layer (RMSNorm, SiLU/SwiGLU, the stack step)

def test_rmsnorm_closed_forms():
    # a constant row c·1 with unit weights: every output is c / sqrt(c^2 + eps)
    c, eps = -3.0, 1e-5
    out = oracle.rmsnorm(np.full((1, 8), c), np.ones(8), eps)
    np.testing.assert_allclose(out, c / np.sqrt(c * c + eps), rtol=1e-15)
    # eps = 0: scale invariant, unit mean square, and the weight multiplies elementwise
    rng = np.random.default_rng(50)
    x = rng.standard_normal((3, 16))
    g = rng.standard_normal(16)
    y = oracle.rmsnorm(x, np.ones(16), 0.0)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(oracle.rmsnorm(7.5 * x, g, 0.0), oracle.rmsnorm(x, g, 0.0), rtol=1e-14)
    np.testing.assert_allclose(oracle.rmsnorm(x, g, 0.0), y * g, rtol=1e-14)


def test_silu_and_swiglu_identities():
    z = np.linspace(-20.0, 20.0, 401)
    s = oracle.silu(z)
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(s - oracle.silu(-z), z, atol=1e-12)        # silu(z) - silu(-z) = z
    np.testing.assert_allclose(oracle.silu(np.array([40.0])), 40.0, rtol=1e-15)
    np.testing.assert_allclose(oracle.silu(np.array([np.log(3.0)])), np.log(3.0) * 0.75, rtol=1e-15)  # sigmoid(ln 3) = 3/4
    gate, up = z[:200].reshape(2, 100), z[200:400].reshape(2, 100)
    np.testing.assert_allclose(oracle.swiglu(np.concatenate([gate, up], -1)), oracle.silu(gate) * up, rtol=1e-15)


def _tiny_stack(seed, dtype, n_layers=2, B=2, D=16, Hq=4, Hkv=2, d=4, F=8, past=(3, 6)):
    dr = Draw(seed)
    layers = synth.stack_weights(dr, n_layers, D, Hq, Hkv, d, F, dtype)
    cap = max(past) + 2
    caches = []
    for _ in range(n_layers):
        kc = np.zeros((B, Hkv, cap, d), dtype=np.float32)
        vc = np.zeros((B, Hkv, cap, d), dtype=np.float32)
        synth.fill_past(dr, kc, vc, past, dtype)
        caches.append((kc, vc))
    h = dr.normal((B, D), 1.0, dtype)
    return layers, caches, h, np.array(past, dtype=np.int32)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_stack_step_matches_brute_force(dtype):
    layers, caches, h, past = _tiny_stack(51, dtype)
    bl = [{k: (v.astype(np.float64).tolist()) for k, v in lw.items()} for lw in layers]
    bc = [(kc.astype(np.float64).tolist(), vc.astype(np.float64).tolist()) for kc, vc in caches]
    got = oracle.decode_stack_step(h, layers, caches, past, 4, dtype, 1e-5)
    ref = np.array(brute.decode_stack_step(h.astype(np.float64).tolist(), bl, bc, [int(p) for p in past], 4,
                                           dtype, 1e-5))
    # both round every stored tensor to dtype; fp64 vs exact sums can only flip a rounding at a
    # tie-near boundary, which this seed does not hit
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)
    for (kc, vc), (bk, bv) in zip(caches, bc):           # both appended the same rows
        assert np.array_equal(kc.astype(np.float64), np.array(bk))
        assert np.array_equal(vc.astype(np.float64), np.array(bv))


def test_decode_stack_with_zero_output_weights_keeps_h():
    # Wo = W_down = 0: both residual branches add nothing, the caches still get the new row
    layers, caches, h, past = _tiny_stack(52, "f32", n_layers=1)
    layers[0]["wo"][:] = 0.0
    layers[0]["w_down"][:] = 0.0
    before = caches[0][0].copy()
    got = oracle.decode_stack_step(h, layers, caches, past, 4, "f32", 1e-5)
    assert np.array_equal(got, h.astype(np.float64))
    for b, L in enumerate(past):
        assert not np.array_equal(caches[0][0][b, :, L], before[b, :, L])


# ---------------------------------------------------------------- rotary position embedding

def _heads(seed, B=2, n=5, H=3, d=8):
    return np.random.default_rng(seed).standard_normal((B, n, H, d))


def test_rope_at_position_zero_is_the_identity():
    x = _heads(60)
    assert np.array_equal(oracle.rope(x, np.zeros((2, 5)), 10000.0), x)


def test_rope_turns_pairs_i_and_i_plus_half_only():
    """A vector with one nonzero component i < d/2 stays in the plane of components i and
    i + d/2; the first pair (frequency theta^0 = 1) turns by exactly p radians."""
    d, p = 8, 7.0
    for i in range(d // 2):
        x = np.zeros((1, 1, 1, d))
        x[..., i] = 1.0
        y = oracle.rope(x, np.array([[p]]), 500000.0)[0, 0, 0]
        others = [j for j in range(d) if j not in (i, i + d // 2)]
        assert np.all(y[others] == 0.0)
        np.testing.assert_allclose(y[i] ** 2 + y[i + d // 2] ** 2, 1.0, rtol=1e-15)
    x = np.zeros((1, 1, 1, d))
    x[..., 0] = 1.0
    y = oracle.rope(x, np.array([[p]]), 500000.0)[0, 0, 0]
    np.testing.assert_allclose([y[0], y[d // 2]], [math.cos(p), math.sin(p)], rtol=0, atol=1e-15)
    x = np.zeros((1, 1, 1, d))
    x[..., d // 2] = 1.0
    y = oracle.rope(x, np.array([[p]]), 500000.0)[0, 0, 0]
    np.testing.assert_allclose([y[0], y[d // 2]], [-math.sin(p), math.cos(p)], rtol=0, atol=1e-15)


def test_rope_frequencies_fall_geometrically():
    """At position 1 pair i turns by theta^(-2i/d): successive angles have the constant ratio
    theta^(-2/d), read back with atan2 from unit vectors (theta = 10000, d = 8: ratio 0.1)."""
    d = 8
    angles = []
    for i in range(d // 2):
        x = np.zeros((1, 1, 1, d))
        x[..., i] = 1.0
        y = oracle.rope(x, np.array([[1.0]]), 10000.0)[0, 0, 0]
        angles.append(math.atan2(y[i + d // 2], y[i]))
    np.testing.assert_allclose(angles[0], 1.0, rtol=1e-15)
    np.testing.assert_allclose(np.array(angles[1:]) / np.array(angles[:-1]), 0.1, rtol=1e-12)


def test_rope_composes_and_inverts():
    x = _heads(61)
    a = np.arange(10).reshape(2, 5) * 37.0
    b = np.arange(10).reshape(2, 5) * 11.0 + 3.0
    th = 500000.0
    np.testing.assert_allclose(oracle.rope(oracle.rope(x, a, th), b, th), oracle.rope(x, a + b, th), atol=1e-12)
    np.testing.assert_allclose(oracle.rope(oracle.rope(x, a, th), -a, th), x, atol=1e-12)


def test_rope_preserves_norms_and_depends_on_relative_position_only():
    q, k = _heads(62), _heads(63)
    th = 10000.0
    pq = np.array([[3, 50, 700, 9000, 131071]] * 2, dtype=np.float64)
    pk = pq - np.array([[0, 7, 1, 4096, 65536]] * 2)
    rq, rk = oracle.rope(q, pq, th), oracle.rope(k, pk, th)
    np.testing.assert_allclose(np.linalg.norm(rq, axis=-1), np.linalg.norm(q, axis=-1), rtol=1e-13)
    dot = np.einsum("bnhd,bnhd->bnh", rq, rk)
    for shift in (1.0, 12345.0):
        dot2 = np.einsum("bnhd,bnhd->bnh", oracle.rope(q, pq + shift, th), oracle.rope(k, pk + shift, th))
        np.testing.assert_allclose(dot2, dot, rtol=1e-9, atol=1e-9)


def _lists(*arrays):
    return [np.asarray(a, dtype=np.float64).tolist() for a in arrays]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_layer_with_rope_matches_brute_force(dtype):
    x, wq, wk, wv, kc, vc, past = _random_layer(64, 2, 3, [4, 9], 16, 4, 2, 8, dtype)
    bk, bv = _lists(kc, vc)
    got = oracle.layer_step(x, wq, wk, wv, kc, vc, past, 4, dtype, rope_theta=10000.0)
    ref = brute.layer_step(*_lists(x, wq, wk, wv), bk, bv, [int(p) for p in past], 4, dtype, rope_theta=10000.0)
    np.testing.assert_allclose(got, np.array(ref), rtol=1e-11, atol=1e-12)
    assert np.array_equal(kc.astype(np.float64), np.array(bk))   # the same rotated, rounded rows


def test_rope_layer_phase_consistency():
    """With RoPE the positions come from past_len: two prefill chunks give the single prefill's
    outputs and cache rows (fp64, within rounding order)."""
    x, wq, wk, wv, kc, vc, past = _random_layer(65, 1, 6, [5], 16, 4, 2, 8, "f32")
    kc1, vc1 = kc.copy(), vc.copy()
    o1 = oracle.layer_step(x, wq, wk, wv, kc1, vc1, past, 4, "f32", rope_theta=10000.0)
    kc2, vc2 = kc.copy(), vc.copy()
    a = oracle.layer_step(x[:, :2], wq, wk, wv, kc2, vc2, past, 4, "f32", rope_theta=10000.0)
    b = oracle.layer_step(x[:, 2:], wq, wk, wv, kc2, vc2, past + 2, 4, "f32", rope_theta=10000.0)
    np.testing.assert_allclose(np.concatenate([a, b], axis=1), o1, rtol=1e-12, atol=1e-13)
    assert np.array_equal(kc1, kc2)
