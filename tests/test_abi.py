"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments on the host before any HIP call (no GPU needed)."""
import ctypes
import os
import re

import pytest

from tests.conftest import ROOT

nq = pytest.importorskip("sub_bit_weight_amd")

HEADER = os.path.join(ROOT, "include", "nq.h")

# Device pointers are never dereferenced by these tests: every call below fails
# host-side validation first.  A non-null, aligned dummy stands in for a buffer.
DUMMY = 0x100000


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(nq_[a-z0-9_]+)\s*\(", src)))


def test_library_builds_and_loads():
    assert os.path.exists(nq.LIB_PATH), "run `python -m sub_bit_weight_amd.build` first"
    L = nq.lib()
    assert b"gfx950" in L.nq_version()


def test_exports_every_declared_symbol():
    L = nq.lib()
    names = _declared()
    assert "nq_lrb_linear" in names and "nq_pack_signs" in names and "nq_reconstruct" in names
    for name in names:
        assert hasattr(L, name), name
    assert sorted(nq.EXPORTED) == names


def test_storage_bits_formula():
    L = nq.lib()
    assert L.nq_storage_bits(256, 256, 64) == 64 * 512 + 32 * 512
    assert L.nq_storage_bits(8192, 28672, 6336) == 6336 * (8192 + 28672) + 32 * (8192 + 28672)
    assert L.nq_storage_bits(0, 5, 5) == 0


def _layer(**kw):
    d = dict(d_out=64, d_in=64, r=32, u_bits=DUMMY, ldu=64, vt_bits=DUMMY, ldv=32, s1=DUMMY, s2=DUMMY)
    d.update(kw)
    return nq.nq_lrb(**d)


def _linear(layer, x=DUMMY, dtype=nq.NQ_BF16, T=1, y=DUMMY, ws=DUMMY, wsb=1 << 40):
    return nq.lib().nq_lrb_linear(ctypes.byref(layer), x, dtype, T, y, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(d_out=0), nq.NQ_ERR_ARG),
    (dict(r=-1), nq.NQ_ERR_ARG),
    (dict(ldu=63), nq.NQ_ERR_ARG),
    (dict(ldv=31), nq.NQ_ERR_ARG),
    (dict(u_bits=None), nq.NQ_ERR_ARG),
    (dict(vt_bits=DUMMY + 2), nq.NQ_ERR_ARG),
    (dict(s2=None), nq.NQ_ERR_ARG),
    (dict(r=(1 << 24) + 1, ldv=(1 << 24) + 1), nq.NQ_ERR_UNSUPPORTED),
])
def test_linear_rejects_bad_layer(kw, status):
    assert _linear(_layer(**kw)) == status
    assert nq.last_error() != ""


def test_linear_rejects_bad_io():
    L = _layer()
    assert _linear(L, T=0) == nq.NQ_ERR_ARG
    assert _linear(L, dtype=7) == nq.NQ_ERR_ARG
    assert _linear(L, x=None) == nq.NQ_ERR_ARG
    assert _linear(L, y=DUMMY + 2) == nq.NQ_ERR_ARG
    assert _linear(L, ws=None) == nq.NQ_ERR_WORKSPACE
    assert _linear(L, wsb=16) == nq.NQ_ERR_WORKSPACE
    assert "workspace" in nq.last_error()
    assert _linear(L, ws=DUMMY + 4) == nq.NQ_ERR_ARG  # not 256-byte aligned


def test_workspace_query():
    L = _layer()
    lib = nq.lib()
    assert lib.nq_lrb_workspace_bytes(ctypes.byref(L), 1) > 0
    assert lib.nq_lrb_workspace_bytes(ctypes.byref(L), 2048) >= 2048 * 32 * 4
    assert lib.nq_lrb_workspace_bytes(ctypes.byref(_layer(d_out=0)), 1) == 0
    assert lib.nq_lrb_workspace_bytes(ctypes.byref(L), 0) == 0


def test_pack_and_unpack_reject_bad_args():
    lib = nq.lib()
    assert lib.nq_pack_signs(None, 4, 4, 4, 1, DUMMY, 4, None) == nq.NQ_ERR_ARG
    assert lib.nq_pack_signs(DUMMY, 4, 4, 0, 1, DUMMY, 4, None) == nq.NQ_ERR_ARG
    assert lib.nq_pack_signs(DUMMY, 4, 4, 4, 1, DUMMY, 3, None) == nq.NQ_ERR_ARG
    assert lib.nq_pack_signs(DUMMY, 0, 4, 4, 1, DUMMY, 4, None) == nq.NQ_ERR_ARG
    assert lib.nq_unpack_signs(DUMMY, 4, 4, 3, DUMMY, None) == nq.NQ_ERR_ARG
    assert lib.nq_unpack_signs(DUMMY, 4, 4, 4, None, None) == nq.NQ_ERR_ARG
    assert lib.nq_fill_random_words(None, 4, 1, None) == nq.NQ_ERR_ARG
    assert lib.nq_fill_random_words(DUMMY, -1, 1, None) == nq.NQ_ERR_ARG


def test_reconstruct_rejects_bad_args():
    lib = nq.lib()
    assert lib.nq_reconstruct(ctypes.byref(_layer()), None, None) == nq.NQ_ERR_ARG
    assert lib.nq_reconstruct(ctypes.byref(_layer(ldu=1)), DUMMY, None) == nq.NQ_ERR_ARG


def test_seq_rejects_bad_entries():
    lib = nq.lib()
    layers = (nq.nq_lrb * 2)(_layer(), _layer(d_in=0))
    xs = (ctypes.c_void_p * 2)(DUMMY, DUMMY)
    ys = (ctypes.c_void_p * 2)(DUMMY, DUMMY)
    h = ctypes.c_void_p()
    assert lib.nq_seq_create(layers, xs, ys, 2, nq.NQ_BF16, 1, ctypes.byref(h)) == nq.NQ_ERR_ARG
    assert "[1]" in nq.last_error()
    assert lib.nq_seq_create(layers, xs, ys, 0, nq.NQ_BF16, 1, ctypes.byref(h)) == nq.NQ_ERR_ARG
    ok = (nq.nq_lrb * 1)(_layer())
    assert lib.nq_seq_create(ok, xs, ys, 1, nq.NQ_BF16, 1, ctypes.byref(h)) == nq.NQ_OK
    assert lib.nq_seq_workspace_bytes(h) > 0
    assert lib.nq_seq_run(h, None, 0, None) == nq.NQ_ERR_WORKSPACE
    lib.nq_seq_destroy(h)


def test_transpose_signs_rejects_bad_args():
    lib = nq.lib()
    assert lib.nq_transpose_signs(None, 4, 4, 4, DUMMY, 4, None) == nq.NQ_ERR_ARG
    assert lib.nq_transpose_signs(DUMMY, 4, 5, 3, DUMMY, 5, None) == nq.NQ_ERR_ARG    # ld < n_out
    assert lib.nq_transpose_signs(DUMMY, 4, 5, 4, DUMMY, 4, None) == nq.NQ_ERR_ARG    # ldt < n_red
    assert lib.nq_transpose_signs(DUMMY, 0, 5, 4, DUMMY, 5, None) == nq.NQ_ERR_ARG
    assert lib.nq_transpose_signs(DUMMY, 4, 5, 4, None, 5, None) == nq.NQ_ERR_ARG
    assert lib.nq_transpose_signs(DUMMY, 1 << 20, 1 << 20, 1 << 20, DUMMY, 1 << 20, None) == nq.NQ_ERR_UNSUPPORTED


def _grads(layer, ut=DUMMY, ldut=32, v=DUMMY, ldvv=64, x=DUMMY, dtype=nq.NQ_BF16, g=DUMMY, gdtype=nq.NQ_F32, T=1,
           dx=DUMMY, ds1=DUMMY, ds2=DUMMY, ws=DUMMY, wsb=1 << 40):
    return nq.lib().nq_lrb_scale_grads(ctypes.byref(layer), ut, ldut, v, ldvv, x, dtype, g, gdtype, T, dx, ds1, ds2,
                                       ws, wsb, None)


def test_scale_grads_rejects_bad_args():
    L = _layer()  # d_out = d_in = 64, r = 32: U^T words [2][>= 32], V words [1][>= 64]
    assert _grads(_layer(d_in=0)) == nq.NQ_ERR_ARG
    assert _grads(L, ut=None) == nq.NQ_ERR_ARG
    assert _grads(L, ldut=31) == nq.NQ_ERR_ARG
    assert _grads(L, ldvv=63) == nq.NQ_ERR_ARG
    assert _grads(L, v=DUMMY + 2) == nq.NQ_ERR_ARG
    assert _grads(L, g=None) == nq.NQ_ERR_ARG
    assert _grads(L, gdtype=5) == nq.NQ_ERR_ARG
    assert _grads(L, g=DUMMY + 2) == nq.NQ_ERR_ARG                  # fp32 g needs 4-byte alignment
    assert _grads(L, g=DUMMY + 1, gdtype=nq.NQ_BF16) == nq.NQ_ERR_ARG
    assert _grads(L, ds1=DUMMY + 1) == nq.NQ_ERR_ARG
    assert _grads(L, ds2=None) == nq.NQ_ERR_ARG
    assert _grads(L, dx=None) == nq.NQ_ERR_ARG
    assert _grads(L, T=0) == nq.NQ_ERR_ARG
    assert _grads(L, ws=None) == nq.NQ_ERR_WORKSPACE
    assert _grads(L, wsb=16) == nq.NQ_ERR_WORKSPACE
    assert _grads(L, ws=DUMMY + 4) == nq.NQ_ERR_ARG


def test_scale_grads_workspace_query():
    L = _layer()
    lib = nq.lib()
    need = lib.nq_lrb_scale_grads_workspace_bytes(ctypes.byref(L), 16)
    assert need >= 16 * (64 + 64) * 4 + lib.nq_lrb_workspace_bytes(ctypes.byref(L), 16)
    assert lib.nq_lrb_scale_grads_workspace_bytes(ctypes.byref(L), 0) == 0
    assert lib.nq_lrb_scale_grads_workspace_bytes(ctypes.byref(_layer(r=0)), 4) == 0


def _grads_batch(layers, n=None, ut=DUMMY, ldut=32, v=DUMMY, ldvv=64, x=DUMMY, dtype=nq.NQ_BF16, g=DUMMY,
                 gdtype=nq.NQ_F32, T=1, dx=DUMMY, ds1=DUMMY, ds2=DUMMY, ws=DUMMY, wsb=1 << 40):
    k = len(layers)
    arr = (nq.nq_lrb * k)(*layers)

    def ptrs(p):
        return (ctypes.c_void_p * k)(*([p] * k))

    def ints(i):
        return (ctypes.c_int64 * k)(*([i] * k))
    return nq.lib().nq_lrb_scale_grads_batch(k if n is None else n, arr, ptrs(ut), ints(ldut), ptrs(v), ints(ldvv),
                                             ptrs(x), dtype, ptrs(g), gdtype, T, ptrs(dx), ptrs(ds1), ptrs(ds2), ws,
                                             wsb, None)


def test_scale_grads_batch_rejects_bad_args():
    L = _layer()
    assert _grads_batch([L, L], n=0) == nq.NQ_ERR_ARG
    assert nq.lib().nq_lrb_scale_grads_batch(1, None, None, None, None, None, None, nq.NQ_BF16, None, nq.NQ_F32, 1,
                                             None, None, None, DUMMY, 1 << 40, None) == nq.NQ_ERR_ARG
    assert _grads_batch([L, L], ldut=31) == nq.NQ_ERR_ARG
    assert "linear 0" in nq.last_error()
    assert _grads_batch([L, _layer(d_in=0)]) == nq.NQ_ERR_ARG
    assert "linear 1" in nq.last_error()
    assert _grads_batch([L, L], gdtype=5) == nq.NQ_ERR_ARG
    assert _grads_batch([L, L], T=0) == nq.NQ_ERR_ARG
    assert _grads_batch([L, L], ws=None) == nq.NQ_ERR_WORKSPACE
    assert _grads_batch([L, L], wsb=16, T=64) == nq.NQ_ERR_WORKSPACE
    assert _grads_batch([L, L], ws=DUMMY + 4) == nq.NQ_ERR_ARG


def test_scale_grads_batch_workspace_query():
    L = _layer()
    lib = nq.lib()
    arr = (nq.nq_lrb * 2)(L, L)
    for T in (4, 64):
        single = lib.nq_lrb_scale_grads_workspace_bytes(ctypes.byref(L), T)
        assert lib.nq_lrb_scale_grads_batch_workspace_bytes(2, arr, T) >= single > 0
    # matrix-core regime: three streams, each with a linear workspace
    assert lib.nq_lrb_scale_grads_batch_workspace_bytes(2, arr, 64) >= 3 * lib.nq_lrb_workspace_bytes(ctypes.byref(L), 64)
    assert lib.nq_lrb_scale_grads_batch_workspace_bytes(0, arr, 64) == 0
    assert lib.nq_lrb_scale_grads_batch_workspace_bytes(2, arr, 0) == 0
    assert lib.nq_lrb_scale_grads_batch_workspace_bytes(2, (nq.nq_lrb * 2)(L, _layer(r=0)), 4) == 0


def _balance(u=DUMMY, d_out=8, ldu=4, v=DUMMY, d_in=5, ldv=4, r=4, uo=None, vo=None, s1=DUMMY, s2=DUMMY, eta=DUMMY,
             ws=DUMMY, wsb=1 << 20):
    return nq.lib().nq_balance_factors(u, d_out, ldu, v, d_in, ldv, r, uo, vo, s1, s2, eta, ws, wsb, None)


def test_balance_rejects_bad_args():
    """Every check runs on the host before any HIP call."""
    assert _balance(u=None) == nq.NQ_ERR_ARG
    assert _balance(v=None) == nq.NQ_ERR_ARG
    assert _balance(s1=None) == nq.NQ_ERR_ARG
    assert _balance(s2=None) == nq.NQ_ERR_ARG
    assert _balance(eta=None) == nq.NQ_ERR_ARG
    assert _balance(d_out=0) == nq.NQ_ERR_ARG
    assert _balance(d_in=0) == nq.NQ_ERR_ARG
    assert _balance(r=0) == nq.NQ_ERR_ARG
    assert _balance(ldu=3) == nq.NQ_ERR_ARG
    assert _balance(ldv=3) == nq.NQ_ERR_ARG
    assert _balance(uo=DUMMY) == nq.NQ_ERR_ARG          # only one of the outputs
    assert _balance(vo=DUMMY) == nq.NQ_ERR_ARG
    assert _balance(u=DUMMY + 2) == nq.NQ_ERR_ARG       # not 4-byte aligned
    assert _balance(uo=DUMMY + 1, vo=DUMMY) == nq.NQ_ERR_ARG
    assert _balance(ws=None) == nq.NQ_ERR_WORKSPACE
    assert _balance(wsb=16) == nq.NQ_ERR_WORKSPACE
    assert _balance(ws=DUMMY + 4) == nq.NQ_ERR_ARG      # not 256-byte aligned
    assert "nq_balance_factors" in nq.lib().nq_last_error().decode()


def test_balance_workspace_query():
    lib = nq.lib()
    assert lib.nq_balance_workspace_bytes(8, 5) >= 2 * 13 * 4
    assert lib.nq_balance_workspace_bytes(0, 5) == 0
    assert lib.nq_balance_workspace_bytes(8, 0) == 0


def _latent(u=DUMMY, ldu=8, v=DUMMY, ldv=8, d_out=16, d_in=24, r=8, s1=DUMMY, s2=DUMMY, x=DUMMY,
            dtype=nq.NQ_F32, T=1, y=DUMMY, ws=DUMMY, wsb=1 << 30):
    return nq.lib().nq_lrb_linear_latent(u, ldu, v, ldv, d_out, d_in, r, s1, s2, x, dtype, T, y, ws, wsb, None)


def test_linear_latent_rejects_bad_args():
    assert _latent(u=None) == nq.NQ_ERR_ARG
    assert _latent(v=None) == nq.NQ_ERR_ARG
    assert _latent(ldu=7) == nq.NQ_ERR_ARG
    assert _latent(ldv=7) == nq.NQ_ERR_ARG
    assert _latent(r=0) == nq.NQ_ERR_ARG
    assert _latent(d_out=0) == nq.NQ_ERR_ARG
    assert _latent(u=DUMMY + 2) == nq.NQ_ERR_ARG
    assert _latent(s1=None) == nq.NQ_ERR_ARG
    assert _latent(x=None) == nq.NQ_ERR_ARG
    assert _latent(T=0) == nq.NQ_ERR_ARG
    assert _latent(dtype=7) == nq.NQ_ERR_ARG
    assert _latent(ws=None) == nq.NQ_ERR_WORKSPACE
    assert _latent(wsb=64) == nq.NQ_ERR_WORKSPACE
    assert _latent(ws=DUMMY + 8) == nq.NQ_ERR_ARG
    assert "nq_lrb_linear_latent" in nq.lib().nq_last_error().decode()


def test_linear_latent_workspace_query():
    lib = nq.lib()
    need = lib.nq_lrb_latent_workspace_bytes(16, 24, 8, 1)
    assert need >= 8 * 4   # t at least (T <= 8: signs taken as the latents load)
    need9 = lib.nq_lrb_latent_workspace_bytes(16, 24, 8, 9)
    assert need9 >= 16 * 4 + 8 * 4   # T > 8: one word row of U and one of V^T at least
    assert lib.nq_lrb_latent_workspace_bytes(16, 24, 0, 1) == 0
    assert lib.nq_lrb_latent_workspace_bytes(16, 24, 8, 0) == 0


def test_noalloc_host_checks():
    """nq_lrb_linear_noalloc validates like nq_lrb_linear and refuses calls whose
    workspace exceeds the library's fixed array, all before any HIP call."""
    lib = nq.lib()

    def call(layer, T=1, dtype=nq.NQ_BF16, x=DUMMY, y=DUMMY):
        return lib.nq_lrb_linear_noalloc(ctypes.byref(layer), x, dtype, T, y, None)
    assert call(_layer(d_out=0)) == nq.NQ_ERR_ARG
    assert call(_layer(), T=0) == nq.NQ_ERR_ARG
    assert call(_layer(), dtype=5) == nq.NQ_ERR_ARG
    assert call(_layer(), y=None) == nq.NQ_ERR_ARG
    big = _layer(d_out=28672, d_in=8192, r=6336, ldu=28672, ldv=6336)
    assert lib.nq_lrb_workspace_bytes(ctypes.byref(big), 64) > nq.NOALLOC_SCRATCH_BYTES
    assert call(big, T=64) == nq.NQ_ERR_UNSUPPORTED
    assert "scratch" in nq.last_error()


# Shapes for the host planners: odd and tiny sizes, the 7B and 70B layer
# shapes, and the rank-sweep extremes.
PLAN_SHAPES = [(1, 1, 1), (33, 70, 3), (256, 256, 64), (320, 4096, 1088), (4096, 4096, 2048),
               (11008, 4096, 2368), (4096, 11008, 2368), (1024, 8192, 896), (28672, 8192, 6336),
               (8192, 28672, 6336), (8192, 8192, 12672)]
PLAN_T = [1, 2, 3, 4, 5, 7, 8, 9, 16, 63, 64, 65, 2048, 66000]


def _packed(d_out, d_in, r):
    return _layer(d_out=d_out, d_in=d_in, r=r, ldu=d_out, ldv=r)


def test_workspace_queries_over_shapes():
    """Every workspace query and sequence plan over a grid of shapes and token
    counts: no failure, sizes that grow with T, and a plan per T (the queries
    walk the tile and split planners, which run on the host alone)."""
    lib = nq.lib()
    for d_out, d_in, r in PLAN_SHAPES:
        L = _packed(d_out, d_in, r)
        prev = 0
        for T in PLAN_T:
            w = lib.nq_lrb_workspace_bytes(ctypes.byref(L), T)
            g = lib.nq_lrb_scale_grads_workspace_bytes(ctypes.byref(L), T)
            lat = lib.nq_lrb_latent_workspace_bytes(d_out, d_in, r, T)
            assert w > 0 and g >= w and lat > 0, (d_out, d_in, r, T)
            assert w < (1 << 40) and g < (1 << 40) and lat < (1 << 40)
            if T > 8:  # the matrix-core regime keeps per-token buffers
                assert w >= prev, (d_out, d_in, r, T)
                prev = w
        assert lib.nq_balance_workspace_bytes(d_out, d_in) > 0
    for T in PLAN_T:
        layers = (nq.nq_lrb * len(PLAN_SHAPES))(*[_packed(*s) for s in PLAN_SHAPES])
        xs = (ctypes.c_void_p * len(PLAN_SHAPES))(*([DUMMY] * len(PLAN_SHAPES)))
        ys = (ctypes.c_void_p * len(PLAN_SHAPES))(*([DUMMY] * len(PLAN_SHAPES)))
        h = ctypes.c_void_p()
        assert lib.nq_seq_create(layers, xs, ys, len(PLAN_SHAPES), nq.NQ_BF16, T, ctypes.byref(h)) == nq.NQ_OK, \
            (T, nq.last_error())
        assert 0 < lib.nq_seq_workspace_bytes(h) < (1 << 42)
        lib.nq_seq_destroy(h)


@pytest.mark.parametrize("dtype", [-1, 2, 7, 1 << 30, -(1 << 31)])
def test_every_dtype_value_is_checked(dtype):
    """Any 32-bit value in a dtype argument is either accepted or rejected on
    the host (the type is a plain int32, so out-of-range values are defined)."""
    lib = nq.lib()
    assert _linear(_layer(), dtype=dtype) == nq.NQ_ERR_ARG
    assert lib.nq_lrb_linear_noalloc(ctypes.byref(_layer()), DUMMY, dtype, 1, DUMMY, None) == nq.NQ_ERR_ARG
