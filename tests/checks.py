"""Output checks of the layer against the oracle (test infrastructure).

Four bars, all taken on the same arrays:

* normwise:   ||y - y*||_F / ||y*||_F <= tol over the whole output (the bar the
  layer's acceptance is stated in);
* per token:  the same ratio for every token (row of y) on its own, so one bad
  token cannot hide among many good ones;
* elementwise, relative to the token's RMS: max_i |y - y*|[t,i] / rms(y*[t,:])
  <= k_elem * tol, so one bad element cannot hide among many good ones (a
  single output off by half its value fails it; the normwise bar alone lets
  that pass once an output has more than ~60 000 elements);
* elementwise, deterministic: |y - y*|[t,i] <= gamma * A[t,i] with
  A[t,i] = |s1_i| * sum_k |U_ik| * sum_j |V_jk| * |s2_j x_tj|
         = |s1_i| * r * sum_j |s2_j x_tj|           (U, V are +-1),
  the absolute-value product of the factored evaluation, and gamma derived
  from the arithmetic of the regime (`gamma`).  This holds for every input,
  including adversarial ranges where y* is small next to its terms.

y* and A come from the oracle (fp64); nothing here reads the GPU library.
"""
from __future__ import annotations

import numpy as np

from oracle import nq_oracle as O

U32 = 2.0 ** -24  # fp32 unit roundoff


def errors(y: np.ndarray, y_ref: np.ndarray) -> dict:
    """Normwise, worst per-token and worst RMS-relative elementwise errors."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    assert y.shape == y_ref.shape and y.ndim == 2, (y.shape, y_ref.shape)
    d = np.abs(y - y_ref)
    tok_ref = np.linalg.norm(y_ref, axis=1)
    tok_err = np.linalg.norm(y - y_ref, axis=1)
    zero = tok_ref == 0
    # tokens whose reference is exactly zero must come out exactly zero
    per_token = np.where(zero, np.where(tok_err == 0, 0.0, np.inf), tok_err / np.where(zero, 1.0, tok_ref))
    rms = tok_ref / np.sqrt(y.shape[1])
    elem = np.where(zero[:, None], np.where(d == 0, 0.0, np.inf), d / np.where(zero, 1.0, rms)[:, None])
    return {"normwise": O.rel_err(y, y_ref), "per_token_max": float(per_token.max()),
            "elem_rms_max": float(elem.max()), "abs_max": float(d.max())}


def abs_terms(ref: O.LRB, x: np.ndarray, rows=None) -> np.ndarray:
    """A[t, i] = |s1_i| * r * sum_j |s2_j x_tj| (float64), for the outputs `rows`."""
    x64 = np.abs(np.asarray(x, dtype=np.float32).astype(np.float64))
    s1 = np.abs(ref.s1.astype(np.float64))
    if rows is not None:
        s1 = s1[np.asarray(rows)]
    z = x64 @ np.abs(ref.s2.astype(np.float64))  # (T,)
    return ref.r * z[:, None] * s1[None, :]


def gamma(T: int, x_dtype: str, d_in: int, r: int) -> float:
    """Coefficient of the deterministic bound |y - y*| <= gamma * A.

    Each stage input v (z = s2 (.) x, then t) enters with a per-element error
    of at most u_in * sum |v| in total, and each stage's fp32 accumulation
    adds at most n * U32 * sum |terms| (n sequential additions); stage 2 sums
    r terms each bounded by sum_j |z_j|, which gives the factor r inside A.
      decode (T <= 8): a stage input is carried by fp8 pieces to 2^-16 of its
        1024-element chunk's largest value, so the chunk's errors add to at
        most 1024 * 2^-16 = 2^-6 of the chunk's sum of |v|; u_in = 2^-6 + U32
        (the s2 * x product); up to two roundings per 128-element step, plus
        the lane and span sums: n = 2 * ceil(n_red / 128) + 16.
      GEMM regime: activations rounded to fp16 after a power-of-two row scale
        (2^-11, plus 2^-20 for values that fall below the fp16 normal range);
        fp32 activations as two fp16 terms (2^-21); the operand encoding scales
        products by up to 12 before the accumulation and the correction sums
        add up to ~70 terms of up to 9 |a|: n = 16 * (ceil(n_red / 16) + 64).
    """
    def n_dec(n):
        return 2 * (-(-n // 128)) + 16

    def n_mfma(n):
        return 16 * (-(-n // 16) + 64)
    if T <= 8:
        u_in = 2.0 ** -6 + U32
        n = n_dec(d_in) + n_dec(r)
    else:
        u_in = (2.0 ** -11 + 2.0 ** -20) if x_dtype == "bf16" else 2.0 ** -21
        n = n_mfma(d_in) + n_mfma(r)
    return 2.0 * u_in + (n + 4) * U32


def latent_abs_terms(s1, s2, x, r: int) -> np.ndarray:
    """A[t, i] = |s1_i| * r * sum_j |s2_j x_tj| (float64) for a layer whose
    signs come from latents (the same form as abs_terms)."""
    z = np.abs(np.asarray(x, np.float32).astype(np.float64)) @ np.abs(np.asarray(s2, np.float64))
    return r * z[:, None] * np.abs(np.asarray(s1, np.float64))[None, :]


def gamma_latent(d_in: int, r: int) -> float:
    """Coefficient of |y - y*| <= gamma * A for the refinement forward at T <= 8
    (signs applied as the fp32 latents load): the s2 * x product (one rounding),
    then fp32 sums only.  Sequential additions per output: stage 1 at most 512
    rows of a span plus one per span (spans of at least 64 rows); stage 2 four
    per 256-element step of a span of at most 2048 elements, six across the
    wave's lanes and one per span (spans of at least 256 elements)."""
    n1 = 512 + -(-d_in // 64)
    n2 = 4 * (2048 // 256) + 6 + -(-r // 256)
    return 2.0 * U32 + (n1 + n2 + 4) * U32


def check(y, y_ref, tol: float, A=None, gam: float | None = None, k_elem: float = 8.0,
          token_bars: bool = True) -> dict:
    """All bars at once.  Returns the measured errors with a 'pass' flag and the
    names of the bars that failed.  token_bars=False skips the per-token and
    RMS-relative bars (tiny layers, where a token's few outputs can cancel to
    far below their terms; the normwise and deterministic bars still apply)."""
    e = errors(y, y_ref)
    failed = []
    if not e["normwise"] <= tol:
        failed.append("normwise")
    if token_bars and not e["per_token_max"] <= tol:
        failed.append("per_token")
    if token_bars and not e["elem_rms_max"] <= k_elem * tol:
        failed.append("elementwise_rms")
    if A is not None:
        bound = gam * np.asarray(A, dtype=np.float64)
        d = np.abs(np.asarray(y, np.float64) - np.asarray(y_ref, np.float64))
        e["bound_ratio_max"] = float(np.max(d / np.where(bound > 0, bound, np.inf), initial=0.0))
        if not np.all(d <= bound):  # NaN or inf anywhere fails too
            failed.append("abs_bound")
    e["tol"] = tol
    e["pass"] = not failed
    e["failed"] = failed
    return e


def splitmix_ref(cfg, shape, layer_idx: int) -> O.LRB:
    """The oracle's copy of a linear whose sign words are drawn with SplitMix64,
    regenerated on the host (never read back from the device)."""
    import synth
    inp = synth.lrb_inputs(cfg, shape, layer_idx)
    nwu, nwv = O.n_words(shape.r), O.n_words(shape.d_in)
    u = synth.random_words(inp["u_seed"], np.arange(nwu * shape.d_out, dtype=np.uint64)).reshape(nwu, shape.d_out)
    v = synth.random_words(inp["v_seed"], np.arange(nwv * shape.r, dtype=np.uint64)).reshape(nwv, shape.r)
    return O.LRB(u, v, inp["s1"], inp["s2"], shape.d_out, shape.d_in, shape.r)


def token_bars_apply(n_outputs: int, ref: O.LRB) -> bool:
    """Per-token and RMS-relative bars need enough outputs per token and
    reductions long enough that no token cancels to far below its terms."""
    return n_outputs >= 16 and min(ref.d_in, ref.r) >= 32


def sampled_check(y_rows: np.ndarray, ref: O.LRB, x: np.ndarray, rows, tol: float, x_dtype: str) -> dict:
    """check() on the outputs `rows` of every token (y_rows = y[:, rows])."""
    T = np.asarray(x).shape[0]
    y_ref = O.sampled_linear_ref(ref, x, rows)
    return check(y_rows, y_ref, tol, abs_terms(ref, x, rows), gamma(T, x_dtype, ref.d_in, ref.r),
                 token_bars=token_bars_apply(len(rows), ref))


def full_check(y: np.ndarray, ref: O.LRB, x: np.ndarray, tol: float, x_dtype: str, factored: bool = False) -> dict:
    """check() on every output."""
    T = np.asarray(x).shape[0]
    y_ref = O.linear_factored_ref(ref, x) if factored else O.linear_ref(ref, x)
    return check(y, y_ref, tol, abs_terms(ref, x), gamma(T, x_dtype, ref.d_in, ref.r),
                 token_bars=token_bars_apply(ref.d_out, ref))


def latent_ref(cfg, shape, layer_idx: int = 0) -> O.LRB:
    """The oracle's copy of a linear whose signs come from the config's fp32
    latents, packed by the oracle itself."""
    import synth
    inp = synth.lrb_inputs(cfg, shape, layer_idx)
    return O.LRB(O.pack_ref(inp["U_latent"]), O.pack_ref(inp["V_latent"].T), inp["s1"], inp["s2"],
                 shape.d_out, shape.d_in, shape.r)
