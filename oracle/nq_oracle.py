"""CPU oracle for the NanoQuant low-rank binary (LRB) linear layer.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke entry point and the
benchmark's CPU-baseline leg may import this module.  The GPU library never
imports, links or calls it, and this module imports nothing from the GPU
library: the two share no code.  Only the seeded input generators (module
`synth`) serve both sides.

Everything here is plain numpy, computed in float64 unless a function says
otherwise, written for a reader to check against the pages by eye:

* The representation (research.samsung.com blog "NanoQuant: Efficient Sub-1-Bit
  Quantization of Large Language Models", section 2 "Problem Formulation and
  Background", subsection "Low-Rank Binary Factorization", the factorization
  equation):  W ~= s1 (.) (U V^T) (.) s2^T, with U in {-1,+1}^(d_out x r),
  V in {-1,+1}^(d_in x r), s1 in R^d_out, s2 in R^d_in.  Read elementwise:
  W[i,j] = s1[i] * (sum_k U[i,k] V[j,k]) * s2[j]  (s1 scales output rows, s2
  scales input columns).
* Storage (same subsection, the sentence after the equation): r(d_out+d_in)
  binary values plus (d_out+d_in) floating-point values.
* The binary factors are the signs of real latent factors (section 3, "Step 3:
  Factorized Component Refinement": sign(U), sign(V)), frozen and packed into
  integer words before the final scale-only calibration (section 3, "Phase 3:
  Scale-Only Model Reconstruction").
* The layer output is y = W x for each token (the pages' inference kernels are a
  GEMV for token-by-token decoding and a GEMM for batches, section 4
  "Inference Performance").

Readings taken where the pages are silent (each is listed with its reason in the
design notes):
* sign(v) = -1 exactly when v < 0 under IEEE comparison; +0, -0 and NaN give +1.
* A stored bit of 1 encodes -1, a bit of 0 encodes +1.
* Word layout: for a stage with n_out outputs and a reduction of length n_red,
  words[w][o] (w < ceil(n_red/32), o < n_out, row stride ld >= n_out) holds the
  signs of elements (o, 32w .. 32w+31), element 32w+b in bit b (LSB first).
  Bits past n_red are 0.  U is packed with outputs i and reduction k
  (words along r); V is packed with outputs k and reduction j (words along
  d_in), i.e. as V^T.
* Scales are fp32; activations are fp32 or bf16; the output y is fp32 on the
  GPU and float64 here.
"""
from __future__ import annotations

import numpy as np

WORD_BITS = 32


def n_words(n_red: int) -> int:
    """Number of 32-bit words that hold n_red signs."""
    return (int(n_red) + WORD_BITS - 1) // WORD_BITS


# --------------------------------------------------------------------------
# storage (section 2, "Low-Rank Binary Factorization": r(d_out+d_in) binary
# values + (d_out+d_in) floating-point values)
# --------------------------------------------------------------------------


def storage_bits_ref(d_out: int, d_in: int, r: int, scale_bits: int = 32) -> int:
    """Bits to store one LRB matrix: r(d_out+d_in) signs + (d_out+d_in) scales."""
    return r * (d_out + d_in) + scale_bits * (d_out + d_in)


def bits_per_weight_ref(d_out: int, d_in: int, r: int, scale_bits: int = 32) -> float:
    return storage_bits_ref(d_out, d_in, r, scale_bits) / float(d_out * d_in)


# --------------------------------------------------------------------------
# packing (section 3, Phase 3: frozen binary factors packed into integer
# formats; the factors are sign(U), sign(V) of section 3, Step 3)
# --------------------------------------------------------------------------


def sign_bits_ref(M: np.ndarray) -> np.ndarray:
    """1 where sign(M) = -1 (M < 0), else 0.  NaN, +0 and -0 give 0."""
    return (np.asarray(M) < 0).astype(np.uint8)


def pack_ref(M: np.ndarray) -> np.ndarray:
    """Pack sign(M) for M of shape (n_out, n_red) into words of shape (nw, n_out).

    words[w][o] bit b = 1  <=>  M[o, 32w+b] < 0; bits past n_red are 0.
    """
    M = np.asarray(M)
    n_out, n_red = M.shape
    nw = n_words(n_red)
    B = np.zeros((n_out, nw * WORD_BITS), dtype=np.uint64)
    B[:, :n_red] = sign_bits_ref(M)
    B = B.reshape(n_out, nw, WORD_BITS)
    weights = np.uint64(1) << np.arange(WORD_BITS, dtype=np.uint64)
    words = (B * weights).sum(axis=2, dtype=np.uint64).astype(np.uint32)  # (n_out, nw)
    return np.ascontiguousarray(words.T)


def unpack_ref(words: np.ndarray, n_red: int, n_out: int | None = None) -> np.ndarray:
    """Inverse of pack_ref: float64 +-1 matrix of shape (n_out, n_red).

    Bit 1 -> -1.0, bit 0 -> +1.0; columns n_out.. of `words` (row padding) and
    bits past n_red are ignored.
    """
    words = np.asarray(words, dtype=np.uint32)
    if n_out is None:
        n_out = words.shape[1]
    nw = n_words(n_red)
    w = words[:nw, :n_out]
    shifts = np.arange(WORD_BITS, dtype=np.uint32)
    bits = (w[:, :, None] >> shifts) & np.uint32(1)  # (nw, n_out, 32)
    S = 1.0 - 2.0 * bits.astype(np.float64)
    S = S.transpose(1, 0, 2).reshape(n_out, nw * WORD_BITS)
    return np.ascontiguousarray(S[:, :n_red])


# --------------------------------------------------------------------------
# the layer (section 2 factorization equation; section 4 GEMV / GEMM)
# --------------------------------------------------------------------------


class LRB:
    """One packed LRB matrix: sign words of U and V^T plus fp32 scales."""

    def __init__(self, u_bits, vt_bits, s1, s2, d_out, d_in, r):
        self.u_bits = np.asarray(u_bits, dtype=np.uint32)    # (ceil(r/32), >= d_out)
        self.vt_bits = np.asarray(vt_bits, dtype=np.uint32)  # (ceil(d_in/32), >= r)
        self.s1 = np.asarray(s1, dtype=np.float32)
        self.s2 = np.asarray(s2, dtype=np.float32)
        self.d_out, self.d_in, self.r = int(d_out), int(d_in), int(r)

    def U(self) -> np.ndarray:
        """U as float64 +-1, shape (d_out, r)."""
        return unpack_ref(self.u_bits, self.r, self.d_out)

    def Vt(self) -> np.ndarray:
        """V^T as float64 +-1, shape (r, d_in)."""
        return unpack_ref(self.vt_bits, self.d_in, self.r)


def sign_product_ref(L: LRB) -> np.ndarray:
    """M = U V^T, exact integers in [-r, r] held in float64, shape (d_out, d_in)."""
    return L.U() @ L.Vt()


def reconstruct_ref(L: LRB) -> np.ndarray:
    """W[i,j] = s1[i] * (U V^T)[i,j] * s2[j] in float64, shape (d_out, d_in)."""
    M = sign_product_ref(L)
    s1 = L.s1.astype(np.float64)
    s2 = L.s2.astype(np.float64)
    return s1[:, None] * M * s2[None, :]


def reconstruct_expected_f32(L: LRB) -> np.ndarray:
    """The fp32 dense W the library must produce bit for bit.

    w[i,j] = fl32( fl32(s1[i] * m[i,j]) * s2[j] ) with m = (U V^T)[i,j] an exact
    integer (|m| <= r <= 2^24 is exact in fp32) and IEEE round-to-nearest-even
    for both products.  Two multiplies and no addition, so fused multiply-add
    contraction cannot change the result.
    """
    M = sign_product_ref(L).astype(np.float32)
    step = (L.s1[:, None] * M).astype(np.float32)
    return (step * L.s2[None, :]).astype(np.float32)


def linear_ref(L: LRB, x: np.ndarray) -> np.ndarray:
    """y[t,i] = sum_j W[i,j] x[t,j] in float64 (reconstruct, then multiply).

    x: (T, d_in) fp32 values (bf16 inputs are passed as their exact fp32 values).
    """
    x64 = np.asarray(x, dtype=np.float32).astype(np.float64)
    return x64 @ reconstruct_ref(L).T


def linear_factored_ref(L: LRB, x: np.ndarray) -> np.ndarray:
    """The same y evaluated in factored order s1 (.) U (V^T (s2 (.) x)), float64."""
    x64 = np.asarray(x, dtype=np.float32).astype(np.float64)
    z = x64 * L.s2.astype(np.float64)[None, :]      # (T, d_in)
    t = z @ L.Vt().T                                 # (T, r)
    u = t @ L.U().T                                  # (T, d_out)
    return u * L.s1.astype(np.float64)[None, :]


def sampled_linear_ref(L: LRB, x: np.ndarray, rows, chunk: int = 4096) -> np.ndarray:
    """y[:, rows] by reconstruct-then-multiply, restricted to the given outputs.

    W[rows, :] = s1[rows] * (U[rows] V^T) * s2 is built in column chunks of
    `chunk` inputs so that the 70B-shaped matrices fit in host memory.
    Returns float64 of shape (T, len(rows)).
    """
    rows = np.asarray(rows, dtype=np.int64)
    x64 = np.asarray(x, dtype=np.float32).astype(np.float64)
    Ur = unpack_ref(L.u_bits, L.r, L.d_out)[rows]     # (R, r)
    s1 = L.s1.astype(np.float64)[rows]
    s2 = L.s2.astype(np.float64)
    y = np.zeros((x64.shape[0], rows.size), dtype=np.float64)
    for j0 in range(0, L.d_in, chunk):
        j1 = min(L.d_in, j0 + chunk)
        # V^T columns j0..j1 need words covering those inputs
        w0, w1 = j0 // WORD_BITS, n_words(j1)
        Vt_c = unpack_ref(L.vt_bits[w0:w1], (w1 - w0) * WORD_BITS, L.r)
        Vt_c = Vt_c[:, j0 - w0 * WORD_BITS: j1 - w0 * WORD_BITS]  # (r, j1-j0)
        W_c = s1[:, None] * (Ur @ Vt_c) * s2[None, j0:j1]
        y += x64[:, j0:j1] @ W_c.T
    return y


# --------------------------------------------------------------------------
# scale-only reconstruction (section 3, "Phase 3: Scale-Only Model
# Reconstruction": with the binary factors frozen only s1 and s2 are tuned).
# For a loss whose gradient with respect to the layer output is g (T x d_out),
# the gradients with respect to s1, s2 and the input follow from the
# factorization equation by the chain rule.
# --------------------------------------------------------------------------


def transpose_bits_ref(words: np.ndarray, n_out: int, n_red: int) -> np.ndarray:
    """Sign words of the transposed sign matrix.

    The input holds an (n_out x n_red) sign matrix S in the word layout above;
    the result holds S^T (n_red outputs, reduction over the n_out positions),
    shape (ceil(n_out/32), n_red).
    """
    S = unpack_ref(words, n_red, n_out)  # (n_out, n_red), +-1
    return pack_ref(S.T)


def scale_grads_ref(L: LRB, x: np.ndarray, g: np.ndarray):
    """(dx, ds1, ds2) in float64 for y = W x with W[i,j] = s1[i] M[i,j] s2[j], M = U V^T.

    dx[t,j]  = sum_i W[i,j] g[t,i]                      (the input gradient)
    ds1[i]   = sum_t g[t,i] * sum_j M[i,j] s2[j] x[t,j]
    ds2[j]   = sum_t x[t,j] * sum_i g[t,i] s1[i] M[i,j]
    """
    x64 = np.asarray(x, dtype=np.float32).astype(np.float64)
    g64 = np.asarray(g, dtype=np.float32).astype(np.float64)
    M = sign_product_ref(L)
    s1 = L.s1.astype(np.float64)
    s2 = L.s2.astype(np.float64)
    dx = g64 @ reconstruct_ref(L)
    ds1 = np.sum(g64 * ((x64 * s2[None, :]) @ M.T), axis=0)
    ds2 = np.sum(x64 * ((g64 * s1[None, :]) @ M), axis=0)
    return dx, ds1, ds2


def scale_grads_factored_ref(L: LRB, x: np.ndarray, g: np.ndarray):
    """The same gradients in factored order (no d_out x d_in matrix), float64:
    u = U (V^T (s2 (.) x)), b = V (U^T (s1 (.) g)); dx = s2 (.) b,
    ds1 = sum_t g (.) u, ds2 = sum_t x (.) b."""
    x64 = np.asarray(x, dtype=np.float32).astype(np.float64)
    g64 = np.asarray(g, dtype=np.float32).astype(np.float64)
    s1 = L.s1.astype(np.float64)
    s2 = L.s2.astype(np.float64)
    U, Vt = L.U(), L.Vt()
    u = ((x64 * s2[None, :]) @ Vt.T) @ U.T
    b = ((g64 * s1[None, :]) @ U) @ Vt
    return b * s2[None, :], np.sum(g64 * u, axis=0), np.sum(x64 * b, axis=0)


# --------------------------------------------------------------------------
# refinement forward (section 3, "Step 3: Factorized Component Refinement"):
# the binary factors are the signs of real latents that the refinement keeps
# updating, so the forward pass takes sign() of the latents as it goes.
# --------------------------------------------------------------------------


def linear_latent_ref(U_lat: np.ndarray, V_lat: np.ndarray, s1, s2, x: np.ndarray) -> np.ndarray:
    """y = s1 (.) sign(U_lat) (sign(V_lat)^T (s2 (.) x)) in float64, for U_lat
    [d_out][r], V_lat [d_in][r], x [T][d_in]; sign(v) = -1 for v < 0, else +1
    (+0, -0 and NaN give +1)."""
    SU = np.where(np.asarray(U_lat, dtype=np.float32) < 0, -1.0, 1.0)
    SV = np.where(np.asarray(V_lat, dtype=np.float32) < 0, -1.0, 1.0)
    z = np.asarray(x, dtype=np.float32).astype(np.float64) * np.asarray(s2, dtype=np.float32).astype(np.float64)
    return ((z @ SV) @ SU.T) * np.asarray(s1, dtype=np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# magnitude balancing and scale extraction (section 3, "Magnitude Balancing
# and Scale Extraction"): after the ADMM step the continuous factors can be
# rescaled inversely without changing their product; the method fixes that
# freedom by equalising their Frobenius norms and reads the scale vectors off
# the balanced factors as per-row mean absolute values.
# --------------------------------------------------------------------------


def balance_ref(U_hat: np.ndarray, V_hat: np.ndarray):
    """(U, V, s1, s2, eta) in float64 for the latent factors U_hat [d_out][r]
    and V_hat [d_in][r]:
        eta = sqrt(||V_hat||_F / ||U_hat||_F),  U = eta U_hat,  V = V_hat / eta,
        s1[i] = mean_k |U[i, k]|,  s2[j] = mean_k |V[j, k]|.
    Reading where the section is silent: if either norm is 0 the product is 0
    and no ratio exists; eta is then 1 (the factors are left as they are)."""
    U_hat = np.asarray(U_hat, dtype=np.float32).astype(np.float64)
    V_hat = np.asarray(V_hat, dtype=np.float32).astype(np.float64)
    nu = np.linalg.norm(U_hat)
    nv = np.linalg.norm(V_hat)
    eta = float(np.sqrt(nv / nu)) if nu > 0 and nv > 0 else 1.0
    U = eta * U_hat
    V = V_hat / eta
    return U, V, np.mean(np.abs(U), axis=1), np.mean(np.abs(V), axis=1), eta


def rel_err(y: np.ndarray, y_ref: np.ndarray) -> float:
    """Normwise relative error ||y - y_ref||_F / ||y_ref||_F (float64)."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    den = np.linalg.norm(y_ref)
    num = np.linalg.norm(y - y_ref)
    return float(num / den) if den > 0 else float(num)
