"""The output checks used by the parity tests and the benchmark, pinned on the
CPU: mistakes planted in the oracle's own output that the normwise bar alone
lets through are caught by the per-token and elementwise bars, and the
deterministic bound holds for a numpy model of each regime's rounding (no GPU)."""
import numpy as np
import pytest

import synth
from oracle import nq_oracle as O
from tests import checks as C
from tests import test_decode_numerics as D


def _layer(d_out, d_in, r, tag):
    cfg = synth.Config(tag, tag, [], (1,), "bf16")
    inp = synth.lrb_inputs(cfg, synth.LayerShape("w", d_out, d_in, r))
    return O.LRB(O.pack_ref(inp["U_latent"]), O.pack_ref(inp["V_latent"].T), inp["s1"], inp["s2"], d_out, d_in, r)


@pytest.fixture(scope="module")
def big_output():
    # 2048 tokens x 64 outputs: the size of the sampled 70B prefill checks
    L = _layer(64, 256, 48, "checks/big")
    x = synth.activations("checks/big/x", 2048, 256, "bf16")
    return L, x, O.linear_ref(L, x)


def test_exact_output_passes(big_output):
    L, x, y = big_output
    e = C.check(y.astype(np.float32), y, 2e-3, C.abs_terms(L, x), C.gamma(2048, "bf16", L.d_in, L.r))
    assert e["pass"], e


def test_one_element_off_by_half_is_caught(big_output):
    L, x, y = big_output
    bad = y.copy()
    rms = np.linalg.norm(y[1000]) / np.sqrt(y.shape[1])
    i = int(np.argmin(np.abs(np.abs(y[1000]) - rms)))  # an output of typical size
    bad[1000, i] *= 1.5
    assert O.rel_err(bad, y) <= 2e-3  # the normwise bar alone passes it
    e = C.check(bad, y, 2e-3)
    assert not e["pass"] and "elementwise_rms" in e["failed"], e


def test_small_element_off_by_half_is_caught(big_output):
    L, x, y = big_output
    bad = y.copy()
    rms = np.linalg.norm(y[7]) / np.sqrt(y.shape[1])
    i = int(np.argmin(np.abs(np.abs(y[7]) - 0.1 * rms)))  # an output at a tenth of the token's RMS
    bad[7, i] *= 1.5
    assert O.rel_err(bad, y) <= 2e-3
    assert "elementwise_rms" in C.check(bad, y, 2e-3)["failed"]


def test_one_token_off_by_one_percent_is_caught(big_output):
    L, x, y = big_output
    bad = y.copy()
    bad[5] *= 1.01
    assert O.rel_err(bad, y) <= 2e-3
    e = C.check(bad, y, 2e-3)
    assert "per_token" in e["failed"], e


def test_zero_token_must_be_exact():
    y_ref = np.zeros((2, 8))
    y_ref[0] = 1.0
    assert C.check(y_ref.copy(), y_ref, 1e-5)["pass"]
    bad = y_ref.copy()
    bad[1, 3] = 1e-30
    assert not C.check(bad, y_ref, 1e-5)["pass"]


def test_abs_terms_match_definition():
    # A[t,i] = |s1_i| sum_k |U_ik| sum_j |V_jk| |s2_j x_tj|, written out with the unpacked factors
    L = _layer(5, 7, 3, "checks/abs")
    x = synth.activations("checks/abs/x", 2, 7, "f32")
    U, Vt = np.abs(L.U()), np.abs(L.Vt())
    z = np.abs(x.astype(np.float64) * L.s2.astype(np.float64))
    want = np.abs(L.s1.astype(np.float64))[None, :] * ((z @ Vt.T) @ U.T)
    np.testing.assert_allclose(C.abs_terms(L, x), want, rtol=1e-14)
    np.testing.assert_allclose(C.abs_terms(L, x, [4, 1]), want[:, [4, 1]], rtol=1e-14)


def _f16_rows(a: np.ndarray, top: int) -> np.ndarray:
    """Round each row to fp16 after a power-of-two scale that puts its largest
    |value| in [2^(top-1), 2^top), then undo the scale (the GEMM regime's prep)."""
    out = np.zeros_like(a, dtype=np.float64)
    for t in range(a.shape[0]):
        m = np.max(np.abs(a[t]))
        if m == 0:
            continue
        e = top - (int(np.floor(np.log2(m))) + 1)
        out[t] = (a[t] * 2.0 ** e).astype(np.float16).astype(np.float64) * 2.0 ** -e
    return out


@pytest.mark.parametrize("kind", ["normal", "outliers", "spread"])
def test_bound_holds_for_modelled_gemm_rounding(kind):
    """fp16 rounding of each stage input (fp64 sums otherwise) stays inside gamma * A."""
    L = _layer(96, 384, 80, f"checks/gemm/{kind}")
    T = 64
    if kind == "normal":
        x = synth.activations(f"checks/gemm/x/{kind}", T, L.d_in, "bf16")
    elif kind == "outliers":
        x = synth.activations(f"checks/gemm/x/{kind}", T, L.d_in, "bf16", 0.02, 3000.0)
    else:
        g = synth.rng(f"checks/gemm/x/{kind}")
        x = synth.round_bf16((np.exp2(g.uniform(-30, 10, (T, L.d_in))) * np.sign(g.standard_normal((T, L.d_in))))
                             .astype(np.float32))
    z = x.astype(np.float64) * L.s2.astype(np.float64)
    t = _f16_rows(z, 11) @ L.Vt().T
    y = (_f16_rows(t, 11) @ L.U().T) * L.s1.astype(np.float64)
    e = C.check(y, O.linear_ref(L, x), 1.0, C.abs_terms(L, x), C.gamma(T, "bf16", L.d_in, L.r))
    assert "abs_bound" not in e["failed"], e
    assert e["bound_ratio_max"] < 0.5


def test_bound_holds_for_modelled_decode_pieces():
    """The fp8-piece model of the decode regime (per 1024-element chunk, both
    stages) stays inside gamma * A."""
    L = _layer(64, 2500, 1100, "checks/dec")
    T = 2
    x = synth.activations("checks/dec/x", T, L.d_in, "f32", 0.01, 1000.0)

    def pieces_of(v):
        out = np.zeros_like(v, dtype=np.float64)
        for tt in range(v.shape[0]):
            for c0 in range(0, v.shape[1], D.CHUNK):
                p, s = D.split_chunk(v[tt, c0:c0 + D.CHUNK].astype(np.float32))
                out[tt, c0:c0 + D.CHUNK] = D.reassemble(p, s)
        return out
    z = (x * L.s2).astype(np.float32)
    t = pieces_of(z) @ L.Vt().T
    y = (pieces_of(t.astype(np.float32)) @ L.U().T) * L.s1.astype(np.float64)
    e = C.check(y, O.linear_factored_ref(L, x), 1e-5, C.abs_terms(L, x), C.gamma(T, "f32", L.d_in, L.r))
    assert e["pass"], e
