"""nq_lrb_linear_noalloc (the entry point for callers that cannot allocate)
through the C ABI: the same y as nq_lrb_linear with a caller workspace, bit for
bit, on consecutive calls of different sizes that share the library's fixed
per-GPU workspace, and within the layer's bar of the oracle."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from oracle import nq_oracle as O
from tests import gpu_cases as G

pytestmark = pytest.mark.gpu

nq = pytest.importorskip("sub_bit_weight_amd")


def _noalloc(layer, x, y) -> int:
    s = layer.struct()
    dt = nq.NQ_BF16 if x.dtype == torch.bfloat16 else nq.NQ_F32
    return nq.lib().nq_lrb_linear_noalloc(ctypes.byref(s), x.data_ptr(), dt, x.shape[0], y.data_ptr(),
                                          torch.cuda.current_stream().cuda_stream)


def test_noalloc_matches_workspace_entry_point():
    cfg = synth.CONFIGS["70b_stack"]
    big_shape = next(s for s in cfg.layers if s.name == "gate")
    big, big_ref = G.splitmix_layer(cfg, big_shape, layer_idx=3)
    small_shape = synth.LayerShape("small", 300, 200, 64)
    small, small_ref, _ = G.latent_layer(G.tiny_config("noalloc"), small_shape, ld_pad=2)
    # (layer, oracle, T, x dtype): decode at the largest 70B shape, then a
    # smaller decode call and a smaller GEMM-regime call
    cases = [(big, big_ref, 8, "bf16"), (small, small_ref, 3, "f32"), (small, small_ref, 40, "bf16")]
    xs, want = [], []
    for i, (L, _, T, xd) in enumerate(cases):
        print(f"noalloc case {i}: {L.d_out}x{L.d_in} r{L.r} T{T} {xd}", flush=True)
        assert nq.lrb_workspace_bytes(L, T) <= nq.NOALLOC_SCRATCH_BYTES
        x_np = synth.activations(f"noalloc/x/{i}", T, L.d_in, xd)
        xs.append((x_np, G.to_device_x(x_np, xd)))
        want.append(nq.lrb_linear(L, xs[-1][1]))
    torch.cuda.synchronize()
    # two rounds of back-to-back calls into the shared array, no synchronisation between calls
    for rnd in range(2):
        ys = [torch.full((T, L.d_out), float("nan"), device=G.DEV) for L, _, T, _ in cases]
        for (L, _, T, _), (_, x), y in zip(cases, xs, ys):
            assert _noalloc(L, x, y) == nq.NQ_OK, nq.last_error()
        torch.cuda.synchronize()
        for i, ((L, ref, T, xd), (x_np, _), y, w) in enumerate(zip(cases, xs, ys, want)):
            assert torch.equal(y.view(torch.int32), w.view(torch.int32)), f"round {rnd} case {i}"
            if L is big:
                rows = np.sort(synth.rng("noalloc/rows").choice(L.d_out, 32, replace=False))
                err = O.rel_err(y.cpu().numpy()[:, rows], O.sampled_linear_ref(ref, x_np, rows))
            else:
                err = O.rel_err(y.cpu().numpy(), O.linear_ref(ref, x_np))
            assert err <= G.tol_for(T, xd), (rnd, i, err)


def test_noalloc_rejects_calls_beyond_the_array():
    cfg = synth.CONFIGS["70b_stack"]
    shape = next(s for s in cfg.layers if s.name == "gate")
    L, _ = G.splitmix_layer(cfg, shape)
    T = 64
    assert nq.lrb_workspace_bytes(L, T) > nq.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((T, L.d_in), dtype=torch.bfloat16, device=G.DEV)
    y = torch.full((T, L.d_out), 7.0, device=G.DEV)
    assert _noalloc(L, x, y) == nq.NQ_ERR_UNSUPPORTED
    assert "scratch" in nq.last_error()
    torch.cuda.synchronize()
    assert bool(torch.all(y == 7.0))  # nothing launched
