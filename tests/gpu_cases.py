"""Helpers for the GPU parity tests: build the same seeded layer twice, once on
the device through libnq and once on the host for the oracle.  The oracle's
copy is packed by the oracle itself (or regenerated with the host SplitMix64),
never read back from the device."""
from __future__ import annotations

import numpy as np
import torch

import sub_bit_weight_amd as nq
import synth
from oracle import nq_oracle as O

DEV = "cuda:0"


def tiny_config(key: str, x_dtype: str = "bf16", scale_kind: str = "halfnormal") -> synth.Config:
    return synth.Config(key, key, [], (1,), x_dtype, scale_kind=scale_kind)


def latent_layer(cfg: synth.Config, shape: synth.LayerShape, layer_idx: int = 0, ld_pad: int = 0):
    """(device Lrb, oracle LRB, host inputs) for a config whose signs come from fp32 latents."""
    inp = synth.lrb_inputs(cfg, shape, layer_idx)
    U = torch.from_numpy(inp["U_latent"]).to(DEV)
    V = torch.from_numpy(inp["V_latent"]).to(DEV)
    u_bits = nq.pack_u(U, ld=shape.d_out + ld_pad)
    vt_bits = nq.pack_v(V, ld=shape.r + ld_pad)
    dev = nq.Lrb(shape.d_out, shape.d_in, shape.r, u_bits, vt_bits,
                 torch.from_numpy(inp["s1"]).to(DEV), torch.from_numpy(inp["s2"]).to(DEV))
    ref = O.LRB(O.pack_ref(inp["U_latent"]), O.pack_ref(inp["V_latent"].T), inp["s1"], inp["s2"],
                shape.d_out, shape.d_in, shape.r)
    return dev, ref, inp


def splitmix_layer(cfg: synth.Config, shape: synth.LayerShape, layer_idx: int = 0):
    """(device Lrb, oracle LRB) for a config whose sign words are drawn directly."""
    inp = synth.lrb_inputs(cfg, shape, layer_idx)
    nwu, nwv = nq.n_words(shape.r), nq.n_words(shape.d_in)
    u_bits = nq.fill_random_words(nwu * shape.d_out, inp["u_seed"], DEV).view(nwu, shape.d_out)
    vt_bits = nq.fill_random_words(nwv * shape.r, inp["v_seed"], DEV).view(nwv, shape.r)
    dev = nq.Lrb(shape.d_out, shape.d_in, shape.r, u_bits, vt_bits,
                 torch.from_numpy(inp["s1"]).to(DEV), torch.from_numpy(inp["s2"]).to(DEV))
    host_u = synth.random_words(inp["u_seed"], np.arange(nwu * shape.d_out, dtype=np.uint64))
    host_v = synth.random_words(inp["v_seed"], np.arange(nwv * shape.r, dtype=np.uint64))
    ref = O.LRB(host_u.reshape(nwu, shape.d_out), host_v.reshape(nwv, shape.r), inp["s1"], inp["s2"],
                shape.d_out, shape.d_in, shape.r)
    return dev, ref


def to_device_x(x_np: np.ndarray, x_dtype: str) -> torch.Tensor:
    x = torch.from_numpy(np.ascontiguousarray(x_np)).to(DEV)
    return x.to(torch.bfloat16) if x_dtype == "bf16" else x


def words_to_host(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint32)


def decode_tol(x_dtype: str) -> float:
    # fp32 arithmetic throughout the decode regime: the fp32-path bar for both dtypes
    return 1e-5


def prefill_tol(x_dtype: str) -> float:
    # bf16 x: one fp16 rounding of each stage's input (measured ~3e-4); fp32 x:
    # two fp16 terms per stage input (~2^-22, measured ~6e-7)
    return 2e-3 if x_dtype == "bf16" else 1e-5


def tol_for(T: int, x_dtype: str) -> float:
    return decode_tol(x_dtype) if T <= 8 else prefill_tol(x_dtype)
