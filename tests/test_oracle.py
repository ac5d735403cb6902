"""Pins for the CPU oracle: it is checked against the pages' figures, a
hand-worked example, closed forms, invariants and brute force, never against
itself or the GPU library.  CPU only."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import nq_oracle as O
from tests.conftest import GOLDEN


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand_pm1(g, shape):
    return np.where(g.random(shape) < 0.5, -1, 1).astype(np.int64)


def _layer_from_pm1(U, V, s1, s2):
    """Pack +-1 integer matrices with the oracle's packer."""
    d_out, r = U.shape
    d_in = V.shape[0]
    return O.LRB(O.pack_ref(U.astype(np.float32)), O.pack_ref(V.T.astype(np.float32)),
                 s1, s2, d_out, d_in, r)


def _py_pack(M):
    """Independent packer: plain Python integers, one bit at a time."""
    n_out, n_red = len(M), len(M[0])
    nw = (n_red + 31) // 32
    out = [[0] * n_out for _ in range(nw)]
    for o in range(n_out):
        for e in range(n_red):
            if M[o][e] < 0:
                out[e // 32][o] |= 1 << (e % 32)
    return np.array(out, dtype=np.uint64).astype(np.uint32)


# --------------------------------------------------------------------------
# hand-worked example
# --------------------------------------------------------------------------


def test_hand_example():
    ex = _load("hand_example.json")
    U = np.array(ex["U"], dtype=np.float32)
    V = np.array(ex["V"], dtype=np.float32)
    assert np.array_equal(O.pack_ref(U), np.array(ex["u_words"], dtype=np.uint32))
    assert np.array_equal(O.pack_ref(V.T), np.array(ex["vt_words"], dtype=np.uint32))
    L = O.LRB(ex["u_words"], ex["vt_words"], ex["s1"], ex["s2"], ex["d_out"], ex["d_in"], ex["r"])
    assert np.array_equal(O.sign_product_ref(L), np.array(ex["UVt"], dtype=np.float64))
    assert np.array_equal(O.reconstruct_ref(L), np.array(ex["W"]))
    assert np.array_equal(O.reconstruct_expected_f32(L), np.array(ex["W"], dtype=np.float32))
    x = np.array(ex["x"], dtype=np.float32)
    assert np.array_equal(O.linear_ref(L, x), np.array(ex["y"]))
    assert np.array_equal(O.linear_factored_ref(L, x), np.array(ex["y"]))


# --------------------------------------------------------------------------
# packing layout: special cases, brute force, round trip
# --------------------------------------------------------------------------


@pytest.mark.parametrize("n_out,n_red", [(1, 1), (3, 31), (5, 32), (7, 33), (64, 100), (2, 257)])
def test_single_negative_sets_one_bit(n_out, n_red):
    g = np.random.default_rng(n_out * 1000 + n_red)
    for _ in range(5):
        o, e = int(g.integers(n_out)), int(g.integers(n_red))
        M = np.ones((n_out, n_red), dtype=np.float32)
        M[o, e] = -0.5
        W = O.pack_ref(M)
        assert W.shape == (O.n_words(n_red), n_out)
        expect = np.zeros_like(W)
        expect[e // 32, o] = np.uint32(1) << np.uint32(e % 32)
        assert np.array_equal(W, expect)


def test_all_positive_and_all_negative():
    M = np.abs(np.random.default_rng(1).standard_normal((9, 70))).astype(np.float32)
    assert not O.pack_ref(M).any()
    W = O.pack_ref(-M - 1)
    # full words are all ones, the last word holds 70-64 = 6 ones and zero padding
    assert np.all(W[0] == 0xFFFFFFFF) and np.all(W[1] == 0xFFFFFFFF)
    assert np.all(W[2] == 0x3F)


def test_sign_tie_breaks():
    vals = np.array([[0.0, -0.0, np.nan, -np.inf, np.inf, -1e-45, 1e-45, -np.nan]], dtype=np.float32)
    W = O.pack_ref(vals)
    # only -inf (bit 3) and the negative denormal (bit 5) encode -1
    assert int(W[0, 0]) == (1 << 3) | (1 << 5)


@pytest.mark.parametrize("n_out,n_red", [(1, 1), (4, 31), (6, 64), (3, 95), (33, 129)])
def test_pack_matches_bitwise_brute_force(n_out, n_red):
    M = np.random.default_rng(7 + n_red).standard_normal((n_out, n_red)).astype(np.float32)
    assert np.array_equal(O.pack_ref(M), _py_pack(M.tolist()))


def test_round_trip():
    g = np.random.default_rng(3)
    for n_out, n_red in [(1, 1), (10, 31), (17, 200), (64, 64)]:
        M = g.standard_normal((n_out, n_red)).astype(np.float32)
        S = O.unpack_ref(O.pack_ref(M), n_red)
        assert np.array_equal(S, np.where(M < 0, -1.0, 1.0))


def test_unpack_ignores_padding():
    W = np.full((2, 3), 0xFFFFFFFF, dtype=np.uint32)  # padding bits set on purpose
    S = O.unpack_ref(W, 40, n_out=2)
    assert S.shape == (2, 40) and np.all(S == -1.0)


# --------------------------------------------------------------------------
# storage formula against the pages
# --------------------------------------------------------------------------


@pytest.mark.parametrize("d_out,d_in,r", [(256, 256, 64), (4096, 4096, 2048), (11008, 4096, 2368),
                                          (96, 64, 32)])
def test_packed_sizes_match_storage_formula(d_out, d_in, r):
    # pack only shapes, not values: the buffers' bit counts + fp32 scales
    u_bits = O.n_words(r) * d_out * 32
    v_bits = O.n_words(d_in) * r * 32
    assert u_bits + v_bits + 32 * (d_out + d_in) == O.storage_bits_ref(d_out, d_in, r)


def test_small_pack_buffer_bits_equal_formula():
    U = np.random.default_rng(0).standard_normal((96, 32)).astype(np.float32)
    V = np.random.default_rng(1).standard_normal((64, 32)).astype(np.float32)
    bits = O.pack_ref(U).size * 32 + O.pack_ref(V.T).size * 32
    assert bits + 32 * (96 + 64) == O.storage_bits_ref(96, 64, 32)


def test_bits_per_weight_values():
    assert O.bits_per_weight_ref(256, 256, 64) == pytest.approx(0.75)
    assert O.bits_per_weight_ref(4096, 4096, 2048) == pytest.approx(1.015625)
    # the 7B MLP set at r = 2368: about the 0.8 bit/parameter the video quotes
    claims = _load("storage_claims.json")
    b = O.bits_per_weight_ref(11008, 4096, 2368)
    assert abs(b - claims["effective_bits_per_parameter"]["value"]) < 0.01


def test_70b_storage_matches_pages():
    """0.55-bit 70B linears + fp16 embeddings/head ~ 5.75 GB, ~24x (pages)."""
    claims = _load("storage_claims.json")
    layer = synth.llama2_70b_layer(0.55)
    lin_bits = 80 * sum(O.storage_bits_ref(s.d_out, s.d_in, s.r) for s in layer)
    embed_bits = 2 * 32000 * 8192 * 16  # Llama-2 vocabulary, fp16 embedding + lm_head
    total_gb = (lin_bits + embed_bits) / 8 / 1e9
    assert abs(total_gb - claims["compressed_70b_gb"]["value"]) < 0.03
    ratio = claims["fp16_70b_gb"]["value"] / total_gb
    assert abs(ratio - claims["compression_ratio_70b"]["value"]) < 0.6
    assert total_gb < claims["fits_consumer_gpu_gb"]["value"]


def test_rank_rule_values():
    assert [s.r for s in synth.llama2_70b_layer(1.0)] == [4096, 896, 896, 4096, 6336, 6336, 6336]
    assert [s.r for s in synth.llama2_70b_layer(0.55)] == [2240, 448, 448, 2240, 3456, 3456, 3456]


# --------------------------------------------------------------------------
# closed forms and invariants
# --------------------------------------------------------------------------


def test_rank1_all_ones_closed_form():
    g = np.random.default_rng(11)
    d_out, d_in = 7, 13
    s1 = synth.scales_halfnormal("t/s1", d_out)
    s2 = synth.scales_halfnormal("t/s2", d_in)
    L = _layer_from_pm1(np.ones((d_out, 1), np.int64), np.ones((d_in, 1), np.int64), s1, s2)
    W = O.reconstruct_ref(L)
    assert np.array_equal(W, np.outer(s1.astype(np.float64), s2.astype(np.float64)))
    x = g.standard_normal((3, d_in)).astype(np.float32)
    y = O.linear_ref(L, x)
    expect = s1.astype(np.float64)[None, :] * (x.astype(np.float64) @ s2.astype(np.float64))[:, None]
    np.testing.assert_allclose(y, expect, rtol=1e-14, atol=0)


def test_joint_flip_and_permutation_invariance():
    g = np.random.default_rng(5)
    d_out, d_in, r = 9, 40, 6
    U, V = _rand_pm1(g, (d_out, r)), _rand_pm1(g, (d_in, r))
    s1 = synth.scales_halfnormal("f/s1", d_out)
    s2 = synth.scales_halfnormal("f/s2", d_in)
    base = O.reconstruct_ref(_layer_from_pm1(U, V, s1, s2))
    for k in range(r):
        U2, V2 = U.copy(), V.copy()
        U2[:, k] *= -1
        V2[:, k] *= -1
        assert np.array_equal(O.reconstruct_ref(_layer_from_pm1(U2, V2, s1, s2)), base)
        # flipping only U's column k subtracts twice that rank-1 term
        M1 = O.sign_product_ref(_layer_from_pm1(U2, V, s1, s2))
        M0 = O.sign_product_ref(_layer_from_pm1(U, V, s1, s2))
        assert np.array_equal(M1, M0 - 2 * np.outer(U[:, k], V[:, k]))
    perm = g.permutation(r)
    assert np.array_equal(O.reconstruct_ref(_layer_from_pm1(U[:, perm], V[:, perm], s1, s2)), base)


def test_popcount_identity():
    """(U V^T)[i,j] = r - 2 popcount(u_i xor v_j) with rows packed along r."""
    g = np.random.default_rng(9)
    d_out, d_in, r = 6, 11, 45
    U, V = _rand_pm1(g, (d_out, r)), _rand_pm1(g, (d_in, r))
    M = O.sign_product_ref(_layer_from_pm1(U, V, np.ones(d_out, np.float32), np.ones(d_in, np.float32)))

    def row_int(v):
        return sum(1 << k for k in range(r) if v[k] < 0)

    for i in range(d_out):
        for j in range(d_in):
            m = r - 2 * bin(row_int(U[i]) ^ row_int(V[j])).count("1")
            assert M[i, j] == m
    assert np.all(np.abs(M) <= r) and np.all((M - r) % 2 == 0)


@pytest.mark.parametrize("d_out,d_in,r,T", [(1, 1, 1, 1), (3, 5, 2, 3), (5, 33, 31, 1), (33, 3, 33, 3),
                                            (5, 33, 33, 1)])
def test_brute_force_exact_fractions(d_out, d_in, r, T):
    g = np.random.default_rng(d_out * 100 + d_in * 10 + r)
    U, V = _rand_pm1(g, (d_out, r)), _rand_pm1(g, (d_in, r))
    s1 = synth.scales_lognormal(f"bf/s1/{d_out}", d_out)
    s2 = synth.scales_halfnormal(f"bf/s2/{d_in}", d_in)
    x = synth.round_bf16(g.standard_normal((T, d_in)).astype(np.float32))
    y = O.linear_ref(_layer_from_pm1(U, V, s1, s2), x)
    yf = O.linear_factored_ref(_layer_from_pm1(U, V, s1, s2), x)
    exact = np.zeros((T, d_out))
    for t in range(T):
        for i in range(d_out):
            acc = Fraction(0)
            for j in range(d_in):
                m = sum(int(U[i, k]) * int(V[j, k]) for k in range(r))
                acc += Fraction(float(s1[i])) * m * Fraction(float(s2[j])) * Fraction(float(x[t, j]))
            exact[t, i] = float(acc)
    assert O.rel_err(y, exact) <= 1e-12
    assert O.rel_err(yf, exact) <= 1e-12


def test_factored_equals_reconstructed():
    g = np.random.default_rng(21)
    d_out, d_in, r, T = 48, 80, 40, 4
    L = _layer_from_pm1(_rand_pm1(g, (d_out, r)), _rand_pm1(g, (d_in, r)),
                        synth.scales_halfnormal("fe/s1", d_out), synth.scales_halfnormal("fe/s2", d_in))
    x = g.standard_normal((T, d_in)).astype(np.float32)
    assert O.rel_err(O.linear_factored_ref(L, x), O.linear_ref(L, x)) <= 1e-12


def test_linearity():
    g = np.random.default_rng(22)
    d_out, d_in, r = 20, 30, 8
    U, V = _rand_pm1(g, (d_out, r)), _rand_pm1(g, (d_in, r))
    s1 = synth.scales_halfnormal("li/s1", d_out)
    s2 = synth.scales_halfnormal("li/s2", d_in)
    L = _layer_from_pm1(U, V, s1, s2)
    # small integers keep the combination exact in the oracle's fp32 input
    x1 = g.integers(-50, 50, (2, d_in)).astype(np.float32)
    x2 = g.integers(-50, 50, (2, d_in)).astype(np.float32)
    y = O.linear_ref(L, x1 * 2 + x2 * 0.5)
    np.testing.assert_allclose(y, 2 * O.linear_ref(L, x1) + 0.5 * O.linear_ref(L, x2), rtol=1e-12, atol=1e-14)
    y1 = O.linear_ref(_layer_from_pm1(U, V, s1 * np.float32(4), s2), x1)
    np.testing.assert_allclose(y1, 4 * O.linear_ref(L, x1), rtol=1e-14, atol=0)
    y2 = O.linear_ref(_layer_from_pm1(U, V, s1, s2 * np.float32(0.5)), x1)
    np.testing.assert_allclose(y2, 0.5 * O.linear_ref(L, x1), rtol=1e-14, atol=0)


def test_reconstruct_f32_rounding_emulation():
    """fl32(fl32(s1*m)*s2) checked with exact float64 products + one rounding each."""
    g = np.random.default_rng(4)
    d_out, d_in, r = 12, 37, 33
    U, V = _rand_pm1(g, (d_out, r)), _rand_pm1(g, (d_in, r))
    s1 = synth.scales_lognormal("rf/s1", d_out)
    s2 = synth.scales_lognormal("rf/s2", d_in)
    W = O.reconstruct_expected_f32(_layer_from_pm1(U, V, s1, s2))
    for i in range(d_out):
        for j in range(d_in):
            m = int(np.dot(U[i], V[j]))
            a = float(np.float32(float(s1[i]) * m))      # product exact in float64, one rounding
            w = np.float32(a * float(s2[j]))             # 24x24-bit product exact in float64
            assert W[i, j] == w and np.signbit(W[i, j]) == np.signbit(w)


@pytest.mark.parametrize("chunk", [48, 64, 4096])
def test_sampled_rows_match_full(chunk):
    g = np.random.default_rng(8)
    d_out, d_in, r, T = 40, 150, 70, 3
    L = _layer_from_pm1(_rand_pm1(g, (d_out, r)), _rand_pm1(g, (d_in, r)),
                        synth.scales_halfnormal("sr/s1", d_out), synth.scales_halfnormal("sr/s2", d_in))
    x = g.standard_normal((T, d_in)).astype(np.float32)
    rows = np.array([0, 7, 39, 12])
    full = O.linear_ref(L, x)
    np.testing.assert_allclose(O.sampled_linear_ref(L, x, rows, chunk=chunk), full[:, rows], rtol=1e-12, atol=1e-15)


def test_rel_err():
    a = np.array([3.0, 4.0])
    assert O.rel_err(a, a) == 0.0
    assert O.rel_err(a * 1.001, a) == pytest.approx(1e-3)


# --------------------------------------------------------------------------
# scale-only reconstruction: transposed packing and the gradients of s1, s2, x
# --------------------------------------------------------------------------


@pytest.mark.parametrize("n_out,n_red", [(1, 1), (5, 31), (33, 70), (64, 32), (40, 100)])
def test_transpose_bits_brute_force(n_out, n_red):
    g = np.random.default_rng(n_out * 1000 + n_red)
    M = np.where(g.random((n_out, n_red)) < 0.5, -1.0, 1.0)
    words = _py_pack(M.tolist())
    T_words = O.transpose_bits_ref(words, n_out, n_red)
    assert T_words.shape == ((n_out + 31) // 32, n_red)
    # element (e, o) of the transposed matrix is element (o, e) of M, bit by bit
    for e in range(n_red):
        for o in range(n_out):
            bit = (int(T_words[o // 32, e]) >> (o % 32)) & 1
            assert bit == (1 if M[o, e] < 0 else 0)
    # padding bits of the transposed words are 0
    if n_out % 32:
        assert np.all((T_words[-1].astype(np.uint64) >> np.uint64(n_out % 32)) == 0)


def _grads_case(seed, d_out, d_in, r, T):
    g = np.random.default_rng(seed)
    U, V = _rand_pm1(g, (d_out, r)), _rand_pm1(g, (d_in, r))
    s1 = synth.scales_lognormal(f"sg/s1/{seed}", d_out)
    s2 = synth.scales_halfnormal(f"sg/s2/{seed}", d_in)
    L = _layer_from_pm1(U, V, s1, s2)
    x = g.standard_normal((T, d_in)).astype(np.float32)
    gy = g.standard_normal((T, d_out)).astype(np.float32)
    return L, U, V, s1, s2, x, gy


def _loss(U, V, s1, s2, x, gy):
    """<g, W x> summed over tokens, by reconstruct-then-multiply."""
    return float(np.sum(gy.astype(np.float64) * O.linear_ref(_layer_from_pm1(U, V, s1, s2), x)))


@pytest.mark.parametrize("d_out,d_in,r,T", [(3, 5, 2, 1), (7, 11, 4, 3), (16, 9, 33, 2)])
def test_scale_grads_finite_differences(d_out, d_in, r, T):
    """The loss is linear in s1 and, separately, in s2 and in x: a step of
    delta in one value changes it by exactly delta times that value's gradient
    (up to float64 rounding).  The layer holds fp32 values, so each step is the
    difference of two fp32 numbers."""
    L, U, V, s1, s2, x, gy = _grads_case(d_out * 31 + d_in, d_out, d_in, r, T)
    dx, ds1, ds2 = O.scale_grads_ref(L, x, gy)
    base = _loss(U, V, s1, s2, x, gy)

    def stepped(v, idx):
        vp = v.copy()
        vp[idx] = np.float32(v[idx] + np.float32(1.0))
        return vp, float(vp[idx]) - float(v[idx])

    for i in range(d_out):
        s1p, delta = stepped(s1, i)
        d = _loss(U, V, s1p, s2, x, gy) - base
        assert abs(d - delta * ds1[i]) <= 1e-9 * (1 + abs(delta * ds1[i]) + abs(base))
    for j in range(d_in):
        s2p, delta = stepped(s2, j)
        d = _loss(U, V, s1, s2p, x, gy) - base
        assert abs(d - delta * ds2[j]) <= 1e-9 * (1 + abs(delta * ds2[j]) + abs(base))
    for t in range(T):
        for j in range(d_in):
            xp, delta = stepped(x, (t, j))
            d = _loss(U, V, s1, s2, xp, gy) - base
            assert abs(d - delta * dx[t, j]) <= 1e-9 * (1 + abs(delta * dx[t, j]) + abs(base))


def test_scale_grads_adjoint_and_euler_identities():
    """<g, W x> = <W^T g, x> = <s1, ds1> = <s2, ds2> (the loss is homogeneous of
    degree one in x, in s1 and in s2)."""
    L, U, V, s1, s2, x, gy = _grads_case(5, 40, 70, 24, 5)
    dx, ds1, ds2 = O.scale_grads_ref(L, x, gy)
    base = _loss(U, V, s1, s2, x, gy)
    for v in (np.sum(dx * x.astype(np.float64)), np.dot(ds1, s1.astype(np.float64)),
              np.dot(ds2, s2.astype(np.float64))):
        assert abs(v - base) <= 1e-10 * (abs(base) + 1)


def test_scale_grads_factored_equals_dense():
    L, U, V, s1, s2, x, gy = _grads_case(9, 48, 80, 40, 4)
    for a, b in zip(O.scale_grads_factored_ref(L, x, gy), O.scale_grads_ref(L, x, gy)):
        assert O.rel_err(a, b) <= 1e-12


# ---- magnitude balancing and scale extraction --------------------------------

def test_balance_hand_examples():
    """Hand-worked cases (tests/golden/balance_example.json), incl. the zero
    factor where the ratio of norms does not exist."""
    for c in _load("balance_example.json")["cases"]:
        U, V, s1, s2, eta = O.balance_ref(np.array(c["U_hat"], np.float32), np.array(c["V_hat"], np.float32))
        assert eta == pytest.approx(c["eta"], rel=1e-15)
        np.testing.assert_allclose(U, c["U"], rtol=1e-15, atol=0)
        np.testing.assert_allclose(V, c["V"], rtol=1e-15, atol=0)
        np.testing.assert_allclose(s1, c["s1"], rtol=1e-15, atol=0)
        np.testing.assert_allclose(s2, c["s2"], rtol=1e-15, atol=0)


def _latents(seed, d_out, d_in, r, su=1.0, sv=1.0):
    g = np.random.default_rng(seed)
    return ((g.standard_normal((d_out, r)) * su).astype(np.float32),
            (g.standard_normal((d_in, r)) * sv).astype(np.float32))


def test_balance_invariants():
    """Equal balanced norms; the product U V^T unchanged; signs unchanged;
    the result does not depend on how the latent scale is split between the
    factors (c U_hat, V_hat / c give the same U, V, s1, s2)."""
    Uh, Vh = _latents(1, 37, 53, 11, su=0.01, sv=30.0)
    U, V, s1, s2, eta = O.balance_ref(Uh, Vh)
    assert np.linalg.norm(U) == pytest.approx(np.linalg.norm(V), rel=1e-13)
    np.testing.assert_allclose(U @ V.T, Uh.astype(np.float64) @ Vh.astype(np.float64).T, rtol=1e-12, atol=1e-12)
    assert np.array_equal(np.signbit(U), np.signbit(Uh)) and np.array_equal(np.signbit(V), np.signbit(Vh))
    c = np.float32(8.0)  # a power of two keeps the rescaled latents exact in fp32
    U2, V2, s12, s22, eta2 = O.balance_ref(Uh * c, Vh / c)
    assert eta2 == pytest.approx(eta / 8.0, rel=1e-14)
    for a, b in ((U2, U), (V2, V), (s12, s1), (s22, s2)):
        np.testing.assert_allclose(a, b, rtol=1e-13, atol=0)


def test_balance_brute_force_exact():
    """Integer latents: eta^4 equals the exact ratio of squared norms, and the
    scales equal eta times (or 1/eta times) the exact mean of the row's
    absolute values (Fractions, plain loops)."""
    g = np.random.default_rng(3)
    Uh = g.integers(-9, 10, size=(4, 3)).astype(np.float32)
    Vh = g.integers(-9, 10, size=(5, 3)).astype(np.float32)
    U, V, s1, s2, eta = O.balance_ref(Uh, Vh)
    su = sum(Fraction(int(v)) ** 2 for v in Uh.ravel())
    sv = sum(Fraction(int(v)) ** 2 for v in Vh.ravel())
    assert eta ** 4 == pytest.approx(float(sv / su), rel=1e-14)
    for i in range(4):
        mean = sum(abs(Fraction(int(v))) for v in Uh[i]) / 3
        assert s1[i] == pytest.approx(eta * float(mean), rel=1e-15)
    for j in range(5):
        mean = sum(abs(Fraction(int(v))) for v in Vh[j]) / 3
        assert s2[j] == pytest.approx(float(mean) / eta, rel=1e-15)


def test_balance_already_balanced_is_identity():
    Uh, Vh = _latents(4, 16, 16, 8)
    Vh = (Vh * (np.linalg.norm(Uh.astype(np.float64)) / np.linalg.norm(Vh.astype(np.float64)))).astype(np.float32)
    U, V, s1, s2, eta = O.balance_ref(Uh, Vh)
    assert eta == pytest.approx(1.0, abs=1e-7)


# ---- refinement forward from latents -----------------------------------------

def test_linear_latent_equals_pack_then_linear():
    """The sign-of-latent forward against the packed route (bit packing, word
    unpacking and the factored product: no shared arithmetic)."""
    g = np.random.default_rng(11)
    d_out, d_in, r, T = 37, 70, 45, 3
    Ul = g.standard_normal((d_out, r)).astype(np.float32)
    Vl = g.standard_normal((d_in, r)).astype(np.float32)
    Ul[0, :5] = [0.0, -0.0, np.nan, -np.inf, np.inf]
    Vl[3, :3] = [-0.0, np.nan, 0.0]
    s1 = g.random(d_out).astype(np.float32)
    s2 = g.random(d_in).astype(np.float32)
    x = g.standard_normal((T, d_in)).astype(np.float32)
    L = O.LRB(O.pack_ref(Ul), O.pack_ref(Vl.T), s1, s2, d_out, d_in, r)
    got = O.linear_latent_ref(Ul, Vl, s1, s2, x)
    assert O.rel_err(got, O.linear_factored_ref(L, x)) <= 1e-13
    assert O.rel_err(got, O.linear_ref(L, x)) <= 1e-12


def test_linear_latent_hand_case():
    """d_out=2, d_in=2, r=1: sign(U) = [+1, -1] (the 0 packs as +1),
    sign(V) = [-1, +1]; W = s1 * [[-1, 1], [1, -1]] * s2."""
    U = np.array([[0.0], [-2.0]], np.float32)
    V = np.array([[-0.5], [3.0]], np.float32)
    s1 = np.array([2.0, 1.0], np.float32)
    s2 = np.array([1.0, 0.5], np.float32)
    x = np.array([[4.0, 2.0]], np.float32)
    # z = s2 x = [4, 1]; t = sign(V)^T z = -4 + 1 = -3; u = sign(U) t = [-3, 3]; y = s1 u
    np.testing.assert_array_equal(O.linear_latent_ref(U, V, s1, s2, x), [[-6.0, 3.0]])
