"""CPU model of the decode regime's input pieces, and the bound they are
designed to meet (no GPU).

The decode kernels multiply the +-1 signs on the matrix cores by fp8 (e4m3)
pieces of each stage input v (z = s2 (.) x, or t).  Per 1024-element chunk and
token: s = min(133 - e, 107) with e the fp32 biased exponent of the chunk's
largest |v|, so that max|v| * 2^s lies in [64, 128) (s at most 115, so that
the E8M0 scale of the last piece stays in range); then four times: round
the scaled remainder to the nearest e4m3 value (ties to even); within each
group of eight elements that the matrix core adds together (elements of one
32-element word with the same index mod 4) keep only pieces whose e4m3
exponent field lies within 7 of the group's largest and is at least 1 (the
hardware adds a group in a window of about 13 binades); subtract and scale the
remainder by 16.  The claim: the pieces carry v to 2^-16 of the chunk's
largest |v|, for any data (a remainder of at most 4 fp8 quanta of the
scaled maximum after the fourth piece), and measured far closer (about
2^-20; the remainders alternate in sign).  This file re-derives that arithmetic from the
description above in numpy (it shares no code with the kernels) and checks
the bound on adversarial chunks: outliers, values spread over 50 binades,
ties, subnormals, all-zero and single-element chunks.
"""
import numpy as np
import pytest

import synth

CHUNK = 1024
PIECES = 4
MAX_SHIFT = 127 - 4 * (PIECES - 1)  # E8M0 scale of the last piece: 2^-(s + 4 (PIECES-1)) >= 2^-127


def e4m3_rne(x: np.ndarray) -> np.ndarray:
    """Nearest e4m3 value (ties to even); |x| stays far below the 448 maximum."""
    ax = np.abs(x)
    with np.errstate(divide="ignore"):
        E = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    E = np.maximum(E, -6.0)                 # subnormals share the quantum 2^-9
    q = np.exp2(E - 3.0)                    # 3 mantissa bits
    return np.sign(x) * np.round(ax / q) * q  # np.round: half to even


def e4m3_exponent_field(v: np.ndarray) -> np.ndarray:
    """Biased exponent field of e4m3 values (0 for zero and subnormals)."""
    av = np.abs(v)
    with np.errstate(divide="ignore"):
        E = np.floor(np.log2(np.where(av > 0, av, 1.0)))
    return np.where(av >= 2.0 ** -6, E + 7, 0).astype(np.int64)


def chunk_shift(m: np.float32) -> int:
    e = int((np.float32(m).view(np.uint32) >> 23) & 0xFF)
    return min(133 - e, MAX_SHIFT)


def split_chunk(v: np.ndarray):
    """(pieces [PIECES][n], s) for one chunk of fp32 values v (n <= 1024)."""
    v = np.asarray(v, dtype=np.float32)
    m = np.float32(np.max(np.abs(v))) if v.size else np.float32(0)
    s = chunk_shift(m)
    n = v.size
    pad = (-n) % 32
    r = np.concatenate([v.astype(np.float64) * 2.0 ** s, np.zeros(pad)])
    # group of an element: its word and its index mod 4
    idx = np.arange(r.size)
    group = (idx // 32) * 4 + idx % 4
    pieces = []
    for _ in range(PIECES):
        q = e4m3_rne(r)
        f = e4m3_exponent_field(q)
        gmax = np.zeros(group.max() + 1, dtype=np.int64)
        np.maximum.at(gmax, group, f)
        keep = f >= np.maximum(1, gmax[group] - 7)
        q = np.where(keep, q, 0.0)
        pieces.append(q[:n])
        r = (r - q) * 16.0
    return np.array(pieces), s


def reassemble(pieces: np.ndarray, s: int) -> np.ndarray:
    return sum(pieces[p] * 2.0 ** -(s + 4 * p) for p in range(PIECES))


def _adversarial(kind: str) -> np.ndarray:
    g = synth.rng(f"pieces/{kind}")
    if kind == "normal":
        return g.standard_normal(CHUNK).astype(np.float32)
    if kind == "outliers":  # 1 % at 3000 sigma
        v = g.standard_normal(CHUNK).astype(np.float32)
        v[g.choice(CHUNK, 10, replace=False)] = np.float32(3.0e3)
        return v
    if kind == "spread50":  # |v| log-uniform over 50 binades, random signs
        return (np.exp2(g.uniform(-40.0, 10.0, CHUNK)) * np.where(g.random(CHUNK) < 0.5, -1, 1)).astype(np.float32)
    if kind == "one_big_rest_tiny":  # one element per group of eight far above the rest
        v = (g.standard_normal(CHUNK) * 2.0 ** -15).astype(np.float32)
        v[::8] = np.float32(100.0)
        return v
    if kind == "ties":  # values halfway between e4m3 neighbours after scaling
        base = g.integers(8, 16, CHUNK).astype(np.float64) + 0.5   # x.5 on an 8-step grid: exact ties
        return (base * 2.0 ** -3 * np.where(g.random(CHUNK) < 0.5, -1, 1)).astype(np.float32)
    if kind == "subnormal_fp32":  # every element an fp32 subnormal (scale capped)
        return (g.integers(1, 1 << 20, CHUNK) * 2.0 ** -149).astype(np.float32)
    if kind == "huge":
        return (g.standard_normal(CHUNK) * 1e30).astype(np.float32)
    if kind == "single":
        v = np.zeros(CHUNK, np.float32)
        v[517] = np.float32(-3.25e-7)
        return v
    if kind == "zeros":
        return np.zeros(CHUNK, np.float32)
    if kind == "bf16_products":  # s2 * x with bf16 x and 0.02|N| scales, as in the workloads
        x = synth.round_bf16(g.standard_normal(CHUNK).astype(np.float32))
        s2 = (np.float32(0.02) * np.abs(g.standard_normal(CHUNK))).astype(np.float32)
        return (x * s2).astype(np.float32)
    raise ValueError(kind)


KINDS = ["normal", "outliers", "spread50", "one_big_rest_tiny", "ties", "subnormal_fp32", "huge", "single",
         "zeros", "bf16_products"]


def test_e4m3_rounding_model():
    # spot values of the e4m3 grid (OCP FP8 E4M3: bias 7, 3 mantissa bits)
    assert e4m3_rne(np.array([1.0, 1.0625, 1.1875, 100.0, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -10]))\
        .tolist() == [1.0, 1.0, 1.25, 96.0, 2.0 ** -9, 0.0, 2.0 ** -8]
    assert e4m3_exponent_field(np.array([1.0, 96.0, 2.0 ** -6, 2.0 ** -7, 0.0])).tolist() == [7, 13, 1, 0, 0]


@pytest.mark.parametrize("kind", KINDS)
def test_pieces_carry_chunk_to_2pow_minus16_of_its_max(kind):
    v = _adversarial(kind)
    pieces, s = split_chunk(v)
    m = float(np.max(np.abs(v.astype(np.float64))))
    err = np.abs(reassemble(pieces, s) - v.astype(np.float64))
    if m == 0.0:
        assert np.all(err == 0.0)
        return
    if 133 - int((np.float32(m).view(np.uint32) >> 23) & 0xFF) > MAX_SHIFT:
        # chunks whose largest |v| is below 2^-89 start below 64 after the
        # capped scale: they keep fewer bits, but the error stays below
        # 2^-16 of the largest value the scale could bring to 64
        assert np.max(err) <= 2.0 ** -16 * 2.0 ** -89 * 2
        return
    assert np.max(err) <= 2.0 ** -16 * m, (kind, np.max(err) / m)
    assert np.max(err) <= 2.0 ** -19 * m  # measured: about 2^-20
    # no piece exceeds the e4m3 range (no saturation) and the first holds the max
    assert np.max(np.abs(pieces)) < 448.0
    # the chunk's error total stays within 1024 * 2^-16 = 2^-6 of its sum of |v|
    assert err.sum() <= 2.0 ** -6 * np.abs(v.astype(np.float64)).sum() + 1e-300


def test_window_rule_is_what_keeps_the_bound():
    """Without the 7-binade window an element far below its group's largest is
    rounded into a piece whose bits the matrix core's 13-binade window would
    drop; with the rule it waits for a later piece.  Model both: the rule keeps
    every piece within 7 binades of its group's largest."""
    v = _adversarial("one_big_rest_tiny")
    pieces, _ = split_chunk(v)
    idx = np.arange(CHUNK)
    group = (idx // 32) * 4 + idx % 4
    for p in range(PIECES):
        f = e4m3_exponent_field(pieces[p])
        gmax = np.zeros(group.max() + 1, dtype=np.int64)
        np.maximum.at(gmax, group, f)
        nz = pieces[p] != 0
        assert np.all(f[nz] >= gmax[group[nz]] - 7)
        assert np.all(f[nz] >= 1)
