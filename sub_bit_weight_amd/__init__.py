"""Python binding of libnq (NanoQuant low-rank binary linear layer on MI355X).

Argument marshalling only: every computation runs in the HIP kernels of
libnq.so.  torch provides device memory and the current HIP stream.  There is
no fallback: if libnq.so is missing or fails to load, every call raises.

Names follow the C ABI in include/nq.h:
  pack_signs, unpack_signs, lrb_linear, lrb_workspace_bytes, reconstruct,
  storage_bits, fill_random_words, Seq (nq_seq_*), transpose_signs,
  lrb_scale_grads (nq_lrb_scale_grads*), lrb_scale_grads_batch
  (nq_lrb_scale_grads_batch*), last_error.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# NQ_LIBRARY selects another build of the same library (the host-sanitized one)
LIB_PATH = os.environ.get("NQ_LIBRARY") or os.path.join(_HERE, "libnq.so")

NQ_OK, NQ_ERR_ARG, NQ_ERR_UNSUPPORTED, NQ_ERR_WORKSPACE, NQ_ERR_HIP = range(5)
NQ_F32, NQ_BF16 = 0, 1
STATUS_NAMES = {0: "NQ_OK", 1: "NQ_ERR_ARG", 2: "NQ_ERR_UNSUPPORTED", 3: "NQ_ERR_WORKSPACE", 4: "NQ_ERR_HIP"}

EXPORTED = [
    "nq_pack_signs", "nq_unpack_signs", "nq_lrb_workspace_bytes", "nq_lrb_linear", "nq_reconstruct",
    "nq_storage_bits", "nq_seq_create", "nq_seq_workspace_bytes", "nq_seq_run", "nq_seq_destroy",
    "nq_fill_random_words", "nq_last_error", "nq_version", "nq_transpose_signs",
    "nq_lrb_scale_grads_workspace_bytes", "nq_lrb_scale_grads", "nq_lrb_scale_grads_batch_workspace_bytes",
    "nq_lrb_scale_grads_batch", "nq_balance_workspace_bytes",
    "nq_balance_factors", "nq_lrb_latent_workspace_bytes", "nq_lrb_linear_latent", "nq_lrb_linear_noalloc",
]

# Size of the library's fixed per-GPU workspace array (NQ_NOALLOC_SCRATCH_BYTES in nq.h).
NOALLOC_SCRATCH_BYTES = 16 << 20


class NqError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class nq_lrb(ctypes.Structure):
    _fields_ = [
        ("d_out", ctypes.c_int64), ("d_in", ctypes.c_int64), ("r", ctypes.c_int64),
        ("u_bits", ctypes.c_void_p), ("ldu", ctypes.c_int64),
        ("vt_bits", ctypes.c_void_p), ("ldv", ctypes.c_int64),
        ("s1", ctypes.c_void_p), ("s2", ctypes.c_void_p),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libnq.so (once).  Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m sub_bit_weight_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    i64, vp, u64, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_size_t
    st = ctypes.c_int
    P = ctypes.POINTER
    L.nq_pack_signs.argtypes = [vp, i64, i64, i64, i64, vp, i64, vp]
    L.nq_pack_signs.restype = st
    L.nq_unpack_signs.argtypes = [vp, i64, i64, i64, vp, vp]
    L.nq_unpack_signs.restype = st
    L.nq_lrb_workspace_bytes.argtypes = [P(nq_lrb), i64]
    L.nq_lrb_workspace_bytes.restype = sz
    L.nq_lrb_linear.argtypes = [P(nq_lrb), vp, ctypes.c_int, i64, vp, vp, sz, vp]
    L.nq_lrb_linear.restype = st
    L.nq_lrb_linear_noalloc.argtypes = [P(nq_lrb), vp, ctypes.c_int, i64, vp, vp]
    L.nq_lrb_linear_noalloc.restype = st
    L.nq_reconstruct.argtypes = [P(nq_lrb), vp, vp]
    L.nq_reconstruct.restype = st
    L.nq_storage_bits.argtypes = [i64, i64, i64]
    L.nq_storage_bits.restype = u64
    L.nq_seq_create.argtypes = [P(nq_lrb), P(vp), P(vp), i64, ctypes.c_int, i64, P(vp)]
    L.nq_seq_create.restype = st
    L.nq_seq_workspace_bytes.argtypes = [vp]
    L.nq_seq_workspace_bytes.restype = sz
    L.nq_seq_run.argtypes = [vp, vp, sz, vp]
    L.nq_seq_run.restype = st
    L.nq_seq_destroy.argtypes = [vp]
    L.nq_seq_destroy.restype = None
    L.nq_fill_random_words.argtypes = [vp, i64, u64, vp]
    L.nq_fill_random_words.restype = st
    L.nq_transpose_signs.argtypes = [vp, i64, i64, i64, vp, i64, vp]
    L.nq_transpose_signs.restype = st
    L.nq_lrb_scale_grads_workspace_bytes.argtypes = [P(nq_lrb), i64]
    L.nq_lrb_scale_grads_workspace_bytes.restype = sz
    L.nq_lrb_scale_grads.argtypes = [P(nq_lrb), vp, i64, vp, i64, vp, ctypes.c_int, vp, ctypes.c_int, i64, vp, vp, vp,
                                     vp, sz, vp]
    L.nq_lrb_scale_grads.restype = st
    L.nq_lrb_scale_grads_batch_workspace_bytes.argtypes = [i64, P(nq_lrb), i64]
    L.nq_lrb_scale_grads_batch_workspace_bytes.restype = sz
    L.nq_lrb_scale_grads_batch.argtypes = [i64, P(nq_lrb), P(vp), P(i64), P(vp), P(i64), P(vp), ctypes.c_int, P(vp),
                                           ctypes.c_int, i64, P(vp), P(vp), P(vp), vp, sz, vp]
    L.nq_lrb_scale_grads_batch.restype = st
    L.nq_lrb_latent_workspace_bytes.argtypes = [i64, i64, i64, i64]
    L.nq_lrb_latent_workspace_bytes.restype = sz
    L.nq_lrb_linear_latent.argtypes = [vp, i64, vp, i64, i64, i64, i64, vp, vp, vp, ctypes.c_int, i64, vp, vp, sz, vp]
    L.nq_lrb_linear_latent.restype = st
    L.nq_balance_workspace_bytes.argtypes = [i64, i64]
    L.nq_balance_workspace_bytes.restype = sz
    L.nq_balance_factors.argtypes = [vp, i64, i64, vp, i64, i64, i64, vp, vp, vp, vp, vp, vp, sz, vp]
    L.nq_balance_factors.restype = st
    L.nq_last_error.argtypes = []
    L.nq_last_error.restype = ctypes.c_char_p
    L.nq_version.argtypes = []
    L.nq_version.restype = ctypes.c_char_p
    _lib = L
    return L


def last_error() -> str:
    return lib().nq_last_error().decode()


def _check(status: int) -> None:
    if status != NQ_OK:
        raise NqError(status, last_error())


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream=None, device: int | None = None) -> int:
    """The HIP stream handle: `stream`'s, else torch's current stream on
    `device` (default: the current device)."""
    if stream is None:
        if _raw_stream is not None and device is not None:
            return _raw_stream(device)  # no Stream object per call
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _on(stream):
    """Allocation context for a call on `stream`: buffers made for the call
    (outputs, workspace) belong to that stream in torch's caching allocator, so
    a workspace freed at return cannot be handed to work on another stream
    while the call's kernels still use it."""
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _dev(t: torch.Tensor, name: str) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def n_words(n: int) -> int:
    return (int(n) + 31) // 32


# ---------------------------------------------------------------- packing


def pack_signs(src: torch.Tensor, n_out: int, n_red: int, stride_out: int, stride_red: int,
               out: torch.Tensor | None = None, ld: int | None = None, stream=None) -> torch.Tensor:
    """Sign words [ceil(n_red/32)][ld] (int32 storage of uint32 words)."""
    _dev(src, "src")
    if src.dtype != torch.float32:
        raise ValueError("src must be float32")
    ld = n_out if ld is None else ld
    if out is None:
        with _on(stream):
            out = torch.zeros((n_words(n_red), ld), dtype=torch.int32, device=src.device)
    _check(lib().nq_pack_signs(_ptr(src), n_out, n_red, stride_out, stride_red, _ptr(out), ld, _stream(stream)))
    return out


def pack_u(U_latent: torch.Tensor, ld: int | None = None) -> torch.Tensor:
    """U latent [d_out][r] -> U words [ceil(r/32)][ld]."""
    d_out, r = U_latent.shape
    return pack_signs(U_latent, d_out, r, r, 1, ld=ld)


def pack_v(V_latent: torch.Tensor, ld: int | None = None) -> torch.Tensor:
    """V latent [d_in][r] -> V^T words [ceil(d_in/32)][ld]."""
    d_in, r = V_latent.shape
    return pack_signs(V_latent, r, d_in, 1, r, ld=ld)


def unpack_signs(bits: torch.Tensor, n_out: int, n_red: int, ld: int | None = None,
                 stream=None) -> torch.Tensor:
    _dev(bits, "bits")
    ld = bits.shape[1] if ld is None else ld
    with _on(stream):
        out = torch.empty((n_out, n_red), dtype=torch.float32, device=bits.device)
    _check(lib().nq_unpack_signs(_ptr(bits), n_out, n_red, ld, _ptr(out), _stream(stream)))
    return out


def fill_random_words(n: int, seed: int, device="cuda", out: torch.Tensor | None = None,
                      stream=None) -> torch.Tensor:
    """Synthetic sign words: low 32 bits of SplitMix64(seed, i) (an input generator)."""
    if out is None:
        with _on(stream):
            out = torch.empty(n, dtype=torch.int32, device=device)
    _check(lib().nq_fill_random_words(_ptr(out), n, seed & 0xFFFFFFFFFFFFFFFF, _stream(stream)))
    return out


# ---------------------------------------------------------------- layer


@dataclass
class Lrb:
    """One packed LRB matrix on the device (the tensors are kept alive here)."""
    d_out: int
    d_in: int
    r: int
    u_bits: torch.Tensor   # [ceil(r/32)][ldu] int32
    vt_bits: torch.Tensor  # [ceil(d_in/32)][ldv] int32
    s1: torch.Tensor       # [d_out] float32
    s2: torch.Tensor       # [d_in] float32

    def __setattr__(self, name, value):
        object.__setattr__(self, name, value)
        object.__setattr__(self, "_struct", None)  # any field change re-validates

    def struct(self) -> nq_lrb:
        """The C struct, after checking what the C ABI cannot see: dtypes,
        shapes and sizes of the tensors (a short buffer would otherwise be read
        past its end by the kernels).  Built once and kept until a field is
        assigned again; tensors must not be resized in place (resize_, set_)
        while the layer is in use."""
        cached = self.__dict__.get("_struct")
        if cached is not None:
            return cached
        for name in ("u_bits", "vt_bits", "s1", "s2"):
            _dev(getattr(self, name), name)
        if min(self.d_out, self.d_in, self.r) < 1:
            raise ValueError(f"sizes must be >= 1: {self.d_out}, {self.d_in}, {self.r}")
        for name, rows, cols in (("u_bits", n_words(self.r), self.d_out), ("vt_bits", n_words(self.d_in), self.r)):
            t = getattr(self, name)
            if t.dtype not in (torch.int32, torch.uint32) or t.dim() != 2:
                raise ValueError(f"{name} must be 2-D 32-bit words, got {t.dtype} {tuple(t.shape)}")
            if t.shape[0] < rows or t.shape[1] < cols:
                raise ValueError(f"{name} must be at least [{rows}][{cols}], got {tuple(t.shape)}")
        for name, n in (("s1", self.d_out), ("s2", self.d_in)):
            t = getattr(self, name)
            if t.dtype != torch.float32 or t.numel() < n:
                raise ValueError(f"{name} must be float32 with >= {n} elements, got {t.dtype} {t.numel()}")
        st = nq_lrb(self.d_out, self.d_in, self.r,
                    self.u_bits.data_ptr(), self.u_bits.shape[1],
                    self.vt_bits.data_ptr(), self.vt_bits.shape[1],
                    self.s1.data_ptr(), self.s2.data_ptr())
        object.__setattr__(self, "_struct", st)
        return st


def _x_dtype(x: torch.Tensor) -> int:
    if x.dtype == torch.float32:
        return NQ_F32
    if x.dtype == torch.bfloat16:
        return NQ_BF16
    raise ValueError(f"x dtype {x.dtype} not supported (float32 or bfloat16)")


def lrb_workspace_bytes(layer: Lrb, T: int) -> int:
    s = layer.struct()
    return int(lib().nq_lrb_workspace_bytes(ctypes.byref(s), T))


def lrb_linear(layer: Lrb, x: torch.Tensor, y: torch.Tensor | None = None,
               workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """y = s1 (.) U (V^T (s2 (.) x)); x [T][d_in] fp32/bf16 -> y [T][d_out] fp32."""
    _dev(x, "x")
    if x.dim() != 2 or x.shape[1] != layer.d_in:
        raise ValueError(f"x must be [T][{layer.d_in}], got {tuple(x.shape)}")
    T = x.shape[0]
    s = layer.struct()
    if y is None or workspace is None:
        with _on(stream):
            if y is None:
                y = torch.empty((T, layer.d_out), dtype=torch.float32, device=x.device)
            if workspace is None:
                need = int(lib().nq_lrb_workspace_bytes(ctypes.byref(s), T))
                workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    _check(lib().nq_lrb_linear(ctypes.byref(s), _ptr(x), _x_dtype(x), T, _ptr(y), _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _stream(stream, x.get_device())))
    return y


def lrb_linear_noalloc(layer: Lrb, x: torch.Tensor, y: torch.Tensor, stream=None) -> torch.Tensor:
    """lrb_linear with the library's fixed per-GPU workspace (nq_lrb_linear_noalloc):
    no device allocation at all, so y must be given.  Calls on one GPU must not
    overlap (they share the workspace)."""
    _dev(x, "x")
    _dev(y, "y")
    if x.dim() != 2 or x.shape[1] != layer.d_in:
        raise ValueError(f"x must be [T][{layer.d_in}], got {tuple(x.shape)}")
    T = x.shape[0]
    if tuple(y.shape) != (T, layer.d_out) or y.dtype != torch.float32:
        raise ValueError(f"y must be float32 [{T}][{layer.d_out}]")
    s = layer.struct()
    _check(lib().nq_lrb_linear_noalloc(ctypes.byref(s), _ptr(x), _x_dtype(x), T, _ptr(y),
                                       _stream(stream, x.get_device())))
    return y


def lrb_linear_latent(u_lat: torch.Tensor, v_lat: torch.Tensor, s1: torch.Tensor, s2: torch.Tensor,
                      x: torch.Tensor, r: int | None = None, y: torch.Tensor | None = None,
                      workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """y = s1 (.) sign(U)(sign(V)^T (s2 (.) x)) from fp32 latents u_lat [d_out][>= r],
    v_lat [d_in][>= r] (row stride = shape[1]); x [T][d_in] fp32/bf16 -> y fp32."""
    for t, n in ((u_lat, "u_lat"), (v_lat, "v_lat"), (s1, "s1"), (s2, "s2"), (x, "x")):
        _dev(t, n)
    for t, n in ((u_lat, "u_lat"), (v_lat, "v_lat")):
        if t.dtype != torch.float32 or t.dim() != 2 or t.stride(1) != 1:
            raise ValueError(f"{n} must be 2-D float32 with unit column stride")
    r = u_lat.shape[1] if r is None else r
    d_out, d_in = u_lat.shape[0], v_lat.shape[0]
    if x.dim() != 2 or x.shape[1] != d_in:
        raise ValueError(f"x must be [T][{d_in}], got {tuple(x.shape)}")
    T = x.shape[0]
    need = int(lib().nq_lrb_latent_workspace_bytes(d_out, d_in, r, T))
    with _on(stream):
        if y is None:
            y = torch.empty((T, d_out), dtype=torch.float32, device=x.device)
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    _check(lib().nq_lrb_linear_latent(_ptr(u_lat), u_lat.stride(0), _ptr(v_lat), v_lat.stride(0), d_out, d_in, r,
                                      _ptr(s1), _ptr(s2), _ptr(x), _x_dtype(x), T, _ptr(y), _ptr(workspace),
                                      workspace.numel() * workspace.element_size(), _stream(stream)))
    return y


def reconstruct(layer: Lrb, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    s = layer.struct()
    if out is None:
        with _on(stream):
            out = torch.empty((layer.d_out, layer.d_in), dtype=torch.float32, device=layer.s1.device)
    _check(lib().nq_reconstruct(ctypes.byref(s), _ptr(out), _stream(stream)))
    return out


def storage_bits(d_out: int, d_in: int, r: int) -> int:
    return int(lib().nq_storage_bits(d_out, d_in, r))


# ---------------------------------------------------------------- scale-only reconstruction


def transpose_signs(bits: torch.Tensor, n_out: int, n_red: int, ld: int | None = None,
                    out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Sign words of the transposed matrix: [ceil(n_out/32)][n_red] (int32 storage)."""
    _dev(bits, "bits")
    ld = bits.shape[1] if ld is None else ld
    if out is None:
        with _on(stream):
            out = torch.empty((n_words(n_out), n_red), dtype=torch.int32, device=bits.device)
    _check(lib().nq_transpose_signs(_ptr(bits), n_out, n_red, ld, _ptr(out), out.shape[1], _stream(stream)))
    return out


@dataclass
class Adjoint:
    """Sign words of a layer's transposed matrix W^T (from transpose_signs)."""
    ut_bits: torch.Tensor  # [ceil(d_out/32)][>= r]: U^T, outputs k < r, words along d_out
    v_bits: torch.Tensor   # [ceil(r/32)][>= d_in]: V, outputs j < d_in, words along r

    @staticmethod
    def of(layer: Lrb, stream=None) -> "Adjoint":
        return Adjoint(transpose_signs(layer.u_bits, layer.d_out, layer.r, stream=stream),
                       transpose_signs(layer.vt_bits, layer.r, layer.d_in, stream=stream))


def lrb_scale_grads_workspace_bytes(layer: Lrb, T: int) -> int:
    s = layer.struct()
    return int(lib().nq_lrb_scale_grads_workspace_bytes(ctypes.byref(s), T))


def lrb_scale_grads(layer: Lrb, adj: Adjoint, x: torch.Tensor, g: torch.Tensor,
                    workspace: torch.Tensor | None = None, stream=None):
    """(dx, ds1, ds2) for y = W x and g = dL/dy (fp32 or bf16): dx [T][d_in], ds1 [d_out], ds2 [d_in] (fp32)."""
    _dev(x, "x")
    _dev(g, "g")
    T = x.shape[0]
    if x.dim() != 2 or x.shape[1] != layer.d_in:
        raise ValueError(f"x must be [T][{layer.d_in}], got {tuple(x.shape)}")
    if tuple(g.shape) != (T, layer.d_out) or not g.is_contiguous():
        raise ValueError(f"g must be contiguous [{T}][{layer.d_out}]")
    s = layer.struct()
    need = int(lib().nq_lrb_scale_grads_workspace_bytes(ctypes.byref(s), T))
    with _on(stream):
        dx = torch.empty((T, layer.d_in), dtype=torch.float32, device=x.device)
        ds1 = torch.empty(layer.d_out, dtype=torch.float32, device=x.device)
        ds2 = torch.empty(layer.d_in, dtype=torch.float32, device=x.device)
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    _check(lib().nq_lrb_scale_grads(ctypes.byref(s), _ptr(adj.ut_bits), adj.ut_bits.shape[1], _ptr(adj.v_bits),
                                    adj.v_bits.shape[1], _ptr(x), _x_dtype(x), _ptr(g), _x_dtype(g), T, _ptr(dx), _ptr(ds1),
                                    _ptr(ds2), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                    _stream(stream)))
    return dx, ds1, ds2


def lrb_scale_grads_batch_workspace_bytes(layers, T: int) -> int:
    arr = (nq_lrb * len(layers))(*[L.struct() for L in layers])
    return int(lib().nq_lrb_scale_grads_batch_workspace_bytes(len(layers), arr, T))


def lrb_scale_grads_batch(layers, adjs, xs, gs, workspace: torch.Tensor | None = None, stream=None):
    """lrb_scale_grads for several independent linears in one call (same T and
    dtypes): a list of (dx, ds1, ds2), equal bit for bit to separate calls."""
    n = len(layers)
    if not (n == len(adjs) == len(xs) == len(gs)) or n < 1:
        raise ValueError("layers, adjs, xs and gs must be non-empty lists of one length")
    T = xs[0].shape[0]
    xd, gd = _x_dtype(xs[0]), _x_dtype(gs[0])
    for L, x, g in zip(layers, xs, gs):
        _dev(x, "x")
        _dev(g, "g")
        if x.dim() != 2 or tuple(x.shape) != (T, L.d_in) or _x_dtype(x) != xd:
            raise ValueError(f"every x must be [{T}][d_in] of one dtype, got {tuple(x.shape)}")
        if tuple(g.shape) != (T, L.d_out) or not g.is_contiguous() or _x_dtype(g) != gd:
            raise ValueError(f"every g must be contiguous [{T}][d_out] of one dtype, got {tuple(g.shape)}")
    arr = (nq_lrb * n)(*[L.struct() for L in layers])
    need = int(lib().nq_lrb_scale_grads_batch_workspace_bytes(n, arr, T))
    dev = xs[0].device
    with _on(stream):
        outs = [(torch.empty((T, L.d_in), dtype=torch.float32, device=dev),
                 torch.empty(L.d_out, dtype=torch.float32, device=dev),
                 torch.empty(L.d_in, dtype=torch.float32, device=dev)) for L in layers]
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)

    def ptrs(ts):
        return (ctypes.c_void_p * n)(*[_ptr(t) for t in ts])

    def lds(ts):
        return (ctypes.c_int64 * n)(*[t.shape[1] for t in ts])
    _check(lib().nq_lrb_scale_grads_batch(
        n, arr, ptrs([a.ut_bits for a in adjs]), lds([a.ut_bits for a in adjs]), ptrs([a.v_bits for a in adjs]),
        lds([a.v_bits for a in adjs]), ptrs(xs), xd, ptrs(gs), gd, T, ptrs([o[0] for o in outs]),
        ptrs([o[1] for o in outs]), ptrs([o[2] for o in outs]), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return outs


def balance_factors(u_hat: torch.Tensor, v_hat: torch.Tensor, r: int | None = None, balanced: bool = True,
                    inplace: bool = False, workspace: torch.Tensor | None = None, stream=None):
    """Magnitude balancing and scale extraction of latent factors u_hat
    [d_out][>= r] and v_hat [d_in][>= r] (fp32, row stride = shape[1]).
    Returns (U, V, s1, s2, eta): the balanced factors (None when balanced is
    False; the inputs themselves when inplace), the scales and eta ([1])."""
    _dev(u_hat, "u_hat")
    _dev(v_hat, "v_hat")
    for t, n in ((u_hat, "u_hat"), (v_hat, "v_hat")):
        if t.dtype != torch.float32 or t.dim() != 2 or t.stride(1) != 1:
            raise ValueError(f"{n} must be 2-D float32 with unit column stride")
    r = u_hat.shape[1] if r is None else r
    d_out, d_in = u_hat.shape[0], v_hat.shape[0]
    dev = u_hat.device
    need = int(lib().nq_balance_workspace_bytes(d_out, d_in))
    with _on(stream):
        if balanced:
            uo = u_hat if inplace else torch.empty_like(u_hat)
            vo = v_hat if inplace else torch.empty_like(v_hat)
        else:
            uo = vo = None
        s1 = torch.empty(d_out, dtype=torch.float32, device=dev)
        s2 = torch.empty(d_in, dtype=torch.float32, device=dev)
        eta = torch.empty(1, dtype=torch.float32, device=dev)
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check(lib().nq_balance_factors(_ptr(u_hat), d_out, u_hat.stride(0), _ptr(v_hat), d_in, v_hat.stride(0), r,
                                    None if uo is None else _ptr(uo), None if vo is None else _ptr(vo), _ptr(s1),
                                    _ptr(s2), _ptr(eta), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                    _stream(stream)))
    return uo, vo, s1, s2, eta


class Seq:
    """A planned sequence of independent LRB linears (nq_seq_*)."""

    def __init__(self, layers: list[Lrb], xs: list[torch.Tensor], ys: list[torch.Tensor]):
        if not (len(layers) == len(xs) == len(ys)) or not layers:
            raise ValueError("layers, xs, ys must be non-empty lists of equal length")
        T = xs[0].shape[0]
        xd = _x_dtype(xs[0])
        for x, y, L in zip(xs, ys, layers):
            _dev(x, "x")
            _dev(y, "y")
            if x.shape != (T, L.d_in) or _x_dtype(x) != xd or y.shape != (T, L.d_out) or y.dtype != torch.float32:
                raise ValueError("inconsistent x/y shapes or dtypes in sequence")
        n = len(layers)
        self.T = T
        self._keep = (layers, xs, ys)
        self._structs = (nq_lrb * n)(*[L.struct() for L in layers])
        self._xs = (ctypes.c_void_p * n)(*[x.data_ptr() for x in xs])
        self._ys = (ctypes.c_void_p * n)(*[y.data_ptr() for y in ys])
        h = ctypes.c_void_p()
        _check(lib().nq_seq_create(self._structs, self._xs, self._ys, n, xd, T, ctypes.byref(h)))
        self._h = h
        self.workspace_bytes = int(lib().nq_seq_workspace_bytes(h))
        self.workspace = torch.empty(max(self.workspace_bytes, 1), dtype=torch.uint8, device=xs[0].device)

    def run(self, stream=None) -> None:
        _check(lib().nq_seq_run(self._h, _ptr(self.workspace), self.workspace.numel(), _stream(stream)))

    def device_error(self) -> int:
        """The device error word (first 4 bytes of the workspace) after the last
        run: 0, or non-zero if a dependency wait gave up (synchronises)."""
        torch.cuda.synchronize()
        if self.T > 8:  # the matrix-core regime runs per-entry kernels without waits
            return 0
        return int(self.workspace[:4].view(torch.int32).item())

    def close(self) -> None:
        if getattr(self, "_h", None):
            lib().nq_seq_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
