#!/usr/bin/env python3
"""Benchmark of the NanoQuant low-rank binary (LRB) linear on one MI355X.

Workload (one "step"): one decode token (T=1) through every linear of a
Llama-2-70B-shaped stack -- 80 layers x {q, k, v, o, gate, up, down} = 560 LRB
linears at ~1.0 bit/weight (r = d_out*d_in/(d_out+d_in) rounded down to a
multiple of 64), each y = s1 (.) U (V^T (s2 (.) x)) on its own bf16 input.
Sign words are drawn directly with SplitMix64 on the device; scales and inputs
come from the seeded host generators (module synth).  The same run also times
the 0.55-bit stack and the rank sweep (decode), a T=2048 pass over the
~1.0-bit stack (matrix cores), the single-linear configurations (256x256 r64;
7B attention; 7B MLP set at T=1 and 8), and the calibration legs.  Every timed
configuration is checked against the CPU oracle on sampled outputs after its
timing (through tests/checks.py).

Prints ONE JSON line.  value = decode tokens/s of the ~1.0-bit stack.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
F16_PEAK_TFLOPS = 2500.0       # MI355X dense fp16/bf16 matrix cores, TFLOP/s
WARM_MS = 100.0               # untimed GPU time before the secondary legs: launches after an idle gap run slower
DECODE_SRC = os.path.join(ROOT, "sub_bit_weight_amd", "csrc", "decode_mfma.hip")
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "decode_persistent_70b_stack_hbm_traffic.md")


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def algorithmic_bytes(shapes, T: int, x_bytes: int = 2) -> int:
    """Packed signs + fp32 scales + x + fp32 y, per pass over `shapes`."""
    tot = 0
    for s in shapes:
        tot += (s.r * s.d_in + 7) // 8 + (s.r * s.d_out + 7) // 8
        tot += 4 * (s.d_in + s.d_out) + T * s.d_in * x_bytes + T * s.d_out * 4
    return tot


def algorithmic_flops(shapes, T: int) -> int:
    return sum(2 * T * s.r * (s.d_in + s.d_out) for s in shapes)


class Stack:
    """All 560 linears of the 70B-shaped stack, resident in HBM."""

    def __init__(self, cfg, n_layers: int, device: str):
        import torch

        import sub_bit_weight_amd as nq
        import synth
        self.cfg, self.n_layers = cfg, n_layers
        self.shapes = []
        self.layers = []
        for l in range(n_layers):
            for s in cfg.layers:
                inp = synth.lrb_inputs(cfg, s, l)
                nwu, nwv = nq.n_words(s.r), nq.n_words(s.d_in)
                u = nq.fill_random_words(nwu * s.d_out, inp["u_seed"], device).view(nwu, s.d_out)
                v = nq.fill_random_words(nwv * s.r, inp["v_seed"], device).view(nwv, s.r)
                self.layers.append(nq.Lrb(s.d_out, s.d_in, s.r, u, v,
                                          torch.from_numpy(inp["s1"]).to(device),
                                          torch.from_numpy(inp["s2"]).to(device)))
                self.shapes.append(s)
        torch.cuda.synchronize()


PREFILL_SRC = os.path.join(ROOT, "sub_bit_weight_amd", "csrc", "prefill.hip")
PREFILL_COUNTERS = os.path.join(ROOT, "profiles", "prefill_gemm_70b_t2048_counters.md")


def summary_field(path: str, src: str, src_key: str, field: str):
    """A number from a committed counter summary, or None when the kernel
    source changed since the counters were taken (sha256 recorded there)."""
    import hashlib
    try:
        text = open(path).read()
    except OSError:
        return None
    fields = {k[2:].strip(): v.strip() for k, v in
              (line.split(":", 1) for line in text.splitlines() if ":" in line and line.startswith("- "))}
    if fields.get(src_key) != hashlib.sha256(open(src, "rb").read()).hexdigest():
        return None
    try:
        return float(fields[field])
    except (KeyError, ValueError):
        return None


def measured_traffic():
    """HBM bytes per decode launch from the committed rocprofv3 counter summary
    (FETCH_SIZE + WRITE_SIZE, calibrated against a copy of known size), or None
    when the decode kernel source changed since the counters were taken."""
    import hashlib
    try:
        text = open(TRAFFIC_SUMMARY).read()
    except OSError:
        return None
    fields = dict(line.split(":", 1) for line in text.splitlines() if ":" in line and line.startswith("- "))
    fields = {k[2:].strip(): v.strip() for k, v in fields.items()}
    src_hash = hashlib.sha256(open(DECODE_SRC, "rb").read()).hexdigest()
    if fields.get("decode_mfma.hip sha256") != src_hash:
        return None
    try:
        return float(fields["hbm bytes per launch"])
    except (KeyError, ValueError):
        return None


def time_decode(stack, T: int, steps: int, warmup: int, device: str, min_warm_ms: float = 0.0):
    """ms per step of one sequence plan over the stack, after `warmup` untimed
    steps (more if needed to fill `min_warm_ms`: launches after an idle gap run
    slower for ~30 ms)."""
    import torch

    import sub_bit_weight_amd as nq
    import synth
    xs_by_din = {d: torch.from_numpy(synth.x_for(stack.cfg, d, T)).to(device).to(torch.bfloat16)
                 for d in sorted({s.d_in for s in stack.shapes})}
    xs = [xs_by_din[s.d_in] for s in stack.shapes]
    ys = [torch.empty((T, s.d_out), dtype=torch.float32, device=device) for s in stack.shapes]
    seq = nq.Seq(stack.layers, xs, ys)
    warm = _warm(seq.run, warmup, min_warm_ms)
    for _ in range(warm):
        seq.run()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        seq.run()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    return ms, seq, xs, ys


def _warm(fn, n: int, min_ms: float) -> int:
    """Untimed calls still to make: n, or enough to fill min_ms of GPU time
    (one synchronized call measures the duration); the measuring call counts."""
    if min_ms <= 0:
        return n
    import time

    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    fn()
    torch.cuda.synchronize()
    ms = max((time.perf_counter() - t0) * 1e3, 1e-3)
    return max(n - 1, int(min_ms / ms))


def _summ(checks: list) -> dict:
    """Worst case over several tests/checks.py results."""
    keys = ("normwise", "per_token_max", "elem_rms_max", "bound_ratio_max")
    out = {k: max(c[k] for c in checks) for k in keys if all(k in c for c in checks)}
    out["tol"] = max(c["tol"] for c in checks)
    out["pass"] = all(c["pass"] for c in checks)
    return out


def stack_parity(stack, xs, ys, picks, rows_per: int = 16, x_dtype: str = "bf16") -> dict:
    """Oracle check of linears of a timed stack, on sampled output rows of every
    token: normwise, per-token, elementwise and deterministic bars (see
    tests/checks.py).  picks: (layer, linear name) pairs."""
    import numpy as np

    import synth
    from tests import checks as C
    per = len(stack.cfg.layers)
    names = [s.name for s in stack.cfg.layers]
    res, done = [], []
    for l, name in picks:
        l = min(l, stack.n_layers - 1)
        idx = l * per + names.index(name)
        s = stack.shapes[idx]
        T = xs[idx].shape[0]
        ref = C.splitmix_ref(stack.cfg, s, l)
        rows = np.sort(synth.rng(f"bench/rows/{stack.cfg.key}/{l}/{name}").choice(s.d_out, rows_per, replace=False))
        x = xs[idx].float().cpu().numpy()
        y = ys[idx].cpu().numpy()[:, rows]
        tol = 1e-5 if T <= 8 else 2e-3
        res.append(C.sampled_check(y, ref, x, rows, tol, x_dtype))
        done.append(f"{l}.{name}")
    out = _summ(res)
    out["checked"] = f"{', '.join(done)}: {rows_per} sampled rows x {xs[0].shape[0]} tokens each"
    return out


def time_prefill_serial(stack, T: int, device: str) -> float:
    """The same pass with one nq_lrb_linear call per linear on one stream
    (kernels never overlap: per-kernel durations in a trace are standalone)."""
    import torch

    import sub_bit_weight_amd as nq
    import synth
    per = len(stack.cfg.layers)
    xs_by_din = {d: torch.from_numpy(synth.x_for(stack.cfg, d, T)).to(device).to(torch.bfloat16)
                 for d in sorted({s.d_in for s in stack.shapes})}
    ys = [torch.empty((T, s.d_out), dtype=torch.float32, device=device) for s in stack.shapes[:per]]
    ws = torch.empty(max(nq.lrb_workspace_bytes(L, T) for L in stack.layers[:per]), dtype=torch.uint8,
                     device=device)
    for i in range(per):  # warm-up layer
        nq.lrb_linear(stack.layers[i], xs_by_din[stack.shapes[i].d_in], ys[i], ws)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for i, L in enumerate(stack.layers):
        nq.lrb_linear(L, xs_by_din[stack.shapes[i].d_in], ys[i % per], ws)
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1)


def time_prefill(stack, T: int, device: str, passes: int = 7):
    """T-token passes over every linear of the stack as one sequence plan
    (entries run round-robin on the plan's streams), each pass timed on its own
    with HIP events on the caller's stream (the plan forks from and joins back
    to it).  Returns (per-pass ms list, seq, xs, ys); each linear has its own
    output."""
    import torch

    import sub_bit_weight_amd as nq
    import synth
    xs_by_din = {d: torch.from_numpy(synth.x_for(stack.cfg, d, T)).to(device).to(torch.bfloat16)
                 for d in sorted({s.d_in for s in stack.shapes})}
    xs = [xs_by_din[s.d_in] for s in stack.shapes]
    ys = [torch.empty((T, s.d_out), dtype=torch.float32, device=device) for s in stack.shapes]
    seq = nq.Seq(stack.layers, xs, ys)
    seq.run()  # warm-up pass
    torch.cuda.synchronize()
    times = []
    for _ in range(passes):
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        seq.run()
        t1.record()
        torch.cuda.synchronize()
        times.append(t0.elapsed_time(t1))
    return times, seq, xs, ys


def time_scale_grads(stack, T: int, device: str, reps: int = 3, profile_passes: int = 0) -> dict:
    """The scale-only reconstruction step (gradients of s1, s2 and x for a given
    output gradient) over the linears of layer 0 at T tokens: the transposed
    sign words are made once (timed separately), then `reps` passes."""
    import numpy as np
    import torch

    import sub_bit_weight_amd as nq
    import synth
    from oracle import nq_oracle as O
    per = len(stack.cfg.layers)
    layers, shapes = stack.layers[:per], stack.shapes[:per]
    gen = torch.Generator(device=device).manual_seed(2048)
    xs = [torch.randn((T, s.d_in), generator=gen, device=device).to(torch.bfloat16) for s in shapes]
    gs = [torch.randn((T, s.d_out), generator=gen, device=device).to(torch.bfloat16) for s in shapes]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # transposed sign words: outputs allocated first, so only the kernels are timed
    outs = [(torch.empty((nq.n_words(L.d_out), L.r), dtype=torch.int32, device=device),
             torch.empty((nq.n_words(L.r), L.d_in), dtype=torch.int32, device=device)) for L in layers]

    def transpose_all():
        for L, (ut, v) in zip(layers, outs):
            nq.transpose_signs(L.u_bits, L.d_out, L.r, out=ut)
            nq.transpose_signs(L.vt_bits, L.r, L.d_in, out=v)
    for _ in range(_warm(transpose_all, 1, WARM_MS)):
        transpose_all()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        transpose_all()
    e1.record()
    torch.cuda.synchronize()
    t_ms = e0.elapsed_time(e1) / reps
    adjs = [nq.Adjoint(ut, v) for ut, v in outs]
    t_bytes = sum(2 * (L.u_bits.numel() + L.vt_bits.numel()) * 4 for L in layers)  # read + write
    ws = torch.empty(max(nq.lrb_scale_grads_workspace_bytes(L, T) for L in layers), dtype=torch.uint8, device=device)
    def grads_all():
        for L, a, x, g in zip(layers, adjs, xs, gs):
            nq.lrb_scale_grads(L, a, x, g, workspace=ws)
    wsb = torch.empty(nq.lrb_scale_grads_batch_workspace_bytes(layers, T), dtype=torch.uint8, device=device)
    if profile_passes:  # for a kernel trace: batched passes with an idle gap between them
        for _ in range(profile_passes):
            nq.lrb_scale_grads_batch(layers, adjs, xs, gs, workspace=wsb)
            torch.cuda.synchronize()
        return {}

    def grads_batch():
        return nq.lrb_scale_grads_batch(layers, adjs, xs, gs, workspace=wsb)

    def timed(fn):
        for _ in range(_warm(fn, 1, WARM_MS)):
            fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps
    ms_single = timed(grads_all)
    ms = timed(grads_batch)
    flops = sum(2 * 2 * T * s.r * (s.d_in + s.d_out) for s in shapes)  # forward + transposed product
    # parity of the timed call itself: layer 0's k at T tokens, every element
    # of dx, ds1 and ds2 against the factored float64 oracle
    from oracle import nq_oracle as O
    from tests import checks as C
    k = [s.name for s in shapes].index("k")
    ref = C.splitmix_ref(stack.cfg, shapes[k], 0)
    got = grads_batch()[k]
    single = nq.lrb_scale_grads(layers[k], adjs[k], xs[k], gs[k])
    want = O.scale_grads_factored_ref(ref, xs[k].float().cpu().numpy(), gs[k].float().cpu().numpy())
    checks = [C.check(got[0].cpu().numpy(), want[0], 2e-3)]
    checks += [C.check(g.cpu().numpy()[None, :], w[None, :], 2e-3) for g, w in zip(got[1:], want[1:])]
    par = _summ(checks)
    par["checked"] = f"layer 0 k, T={T}: every element of dx, ds1, ds2 of the batched call"
    par["batch_equals_single_calls"] = all(torch.equal(a.view(torch.int32), b.view(torch.int32))
                                           for a, b in zip(got, single))
    return {"T": T, "linears": f"layer 0 ({per} linears) in one batched call", "ms_per_layer": ms,
            "ms_per_layer_single_calls": ms_single,
            "tflops": flops / (ms * 1e-3) / 1e12, "frac_of_f16_peak": flops / (ms * 1e-3) / 1e12 / F16_PEAK_TFLOPS,
            "algorithmic_flop_per_layer": flops,
            "includes": "forward product without s1, transposed product without s2, token sums; x and g bf16",
            "transpose_ms_per_layer": t_ms, "transpose_gbs": t_bytes / (t_ms * 1e-3) / 1e9,
            "parity": par}


def time_balance(shapes, device: str, reps: int = 5) -> dict:
    """Magnitude balancing and scale extraction of the fp32 latent factors of
    layer 0's linears (U_hat [d_out][r], V_hat [d_in][r]), balanced factors
    written to separate buffers.  Algorithmic bytes: the latents read twice
    (row statistics, then scaling) and written once."""
    import torch

    import sub_bit_weight_amd as nq
    from oracle import nq_oracle as O
    gen = torch.Generator(device=device).manual_seed(55)
    lat = [(torch.randn((s.d_out, s.r), generator=gen, device=device) * 0.05,
            torch.randn((s.d_in, s.r), generator=gen, device=device) * 2.0) for s in shapes]
    outs = [(torch.empty_like(u), torch.empty_like(v)) for u, v in lat]
    sc = [(torch.empty(s.d_out, device=device), torch.empty(s.d_in, device=device), torch.empty(1, device=device))
          for s in shapes]
    ws = torch.empty(max(nq.lib().nq_balance_workspace_bytes(s.d_out, s.d_in) for s in shapes), dtype=torch.uint8,
                     device=device)
    lib = nq.lib()

    def run(balanced: bool):
        for s, (u, v), (uo, vo), (s1, s2, eta) in zip(shapes, lat, outs, sc):
            st = lib.nq_balance_factors(u.data_ptr(), s.d_out, s.r, v.data_ptr(), s.d_in, s.r, s.r,
                                        uo.data_ptr() if balanced else None, vo.data_ptr() if balanced else None,
                                        s1.data_ptr(), s2.data_ptr(), eta.data_ptr(), ws.data_ptr(), ws.numel(),
                                        torch.cuda.current_stream().cuda_stream)
            assert st == 0, lib.nq_last_error()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    res = {}
    lat_bytes = sum((s.d_out + s.d_in) * s.r * 4 for s in shapes)
    for balanced, nbytes in ((True, 3 * lat_bytes), (False, lat_bytes)):
        for _ in range(_warm(lambda: run(balanced), 1, WARM_MS)):
            run(balanced)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            run(balanced)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        res["balanced_factors" if balanced else "scales_only"] = {
            "ms_per_layer": ms, "gbs": nbytes / (ms * 1e-3) / 1e9, "frac_of_hbm_peak": nbytes / (ms * 1e-3) / 1e12 / 8.0,
            "algorithmic_bytes": nbytes}
    run(True)
    # parity on layer 0's first linear: scales and eta against the float64 oracle
    s0 = shapes[0]
    U0, V0, rs1, rs2, reta = O.balance_ref(lat[0][0].cpu().numpy(), lat[0][1].cpu().numpy())
    err = max(O.rel_err(sc[0][0].cpu().numpy(), rs1), O.rel_err(sc[0][1].cpu().numpy(), rs2),
              O.rel_err(outs[0][0].cpu().numpy(), U0), O.rel_err(outs[0][1].cpu().numpy(), V0),
              abs(float(sc[0][2].item()) / reta - 1))
    res.update({"linears": f"layer 0 ({len(shapes)} linears)", "latent_bytes": lat_bytes,
                "parity": {"rel_err_max": err, "tol": 1e-6, "pass": err <= 1e-6,
                           "checked": f"{s0.name} of the timed pass: every element of U, V, s1, s2 and eta"}})
    return res


def time_latent(shapes, device: str, reps: int = 5) -> dict:
    """The refinement forward from fp32 latent factors over layer 0's linears,
    at T=1 (signs applied as the latents load: GB/s counts the latent reads,
    the scales, x and y) and T=2048 (signs packed at the call, then the packed
    layer: the bytes add the packed words written and read back)."""
    import torch

    import sub_bit_weight_amd as nq
    gen = torch.Generator(device=device).manual_seed(77)
    lat = [(torch.randn((s.d_out, s.r), generator=gen, device=device),
            torch.randn((s.d_in, s.r), generator=gen, device=device),
            torch.rand(s.d_out, generator=gen, device=device), torch.rand(s.d_in, generator=gen, device=device))
           for s in shapes]
    res = {"linears": f"layer 0 ({len(shapes)} linears)"}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for T in (1, 2048):
        xs = [torch.randn((T, s.d_in), generator=gen, device=device).to(torch.bfloat16) for s in shapes]
        ys = [torch.empty((T, s.d_out), device=device) for s in shapes]
        ws = torch.empty(max(nq.lib().nq_lrb_latent_workspace_bytes(s.d_out, s.d_in, s.r, T) for s in shapes),
                         dtype=torch.uint8, device=device)

        def run():
            for (u, v, s1, s2), x, y in zip(lat, xs, ys):
                nq.lrb_linear_latent(u, v, s1, s2, x, y=y, workspace=ws)
        for _ in range(_warm(run, 1, WARM_MS)):
            run()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            run()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        # T > 8: the packed words are written and read back
        nbytes = sum((s.d_out + s.d_in) * s.r * 4 + (0 if T <= 8 else 2 * (s.d_out + s.d_in) * s.r // 8)
                     + 4 * (s.d_out + s.d_in) + T * (2 * s.d_in + 4 * s.d_out) for s in shapes)
        flops = sum(2 * T * s.r * (s.d_in + s.d_out) for s in shapes)
        # parity of the timed calls' outputs: the k linear (every output)
        from oracle import nq_oracle as O
        from tests import checks as C
        k = [s.name for s in shapes].index("k")
        u, v, s1, s2 = (t.cpu().numpy() for t in lat[k])
        want = O.linear_latent_ref(u, v, s1, s2, xs[k].float().cpu().numpy())
        par = C.check(ys[k].cpu().numpy(), want, 1e-5 if T <= 8 else 2e-3)
        res[f"T{T}"] = {"ms_per_layer": ms, "gbs": nbytes / (ms * 1e-3) / 1e9,
                        "frac_of_hbm_peak": nbytes / (ms * 1e-3) / 1e12 / 8.0, "tflops": flops / (ms * 1e-3) / 1e12,
                        "algorithmic_bytes": nbytes,
                        "parity": {kk: par[kk] for kk in ("normwise", "per_token_max", "elem_rms_max", "tol", "pass")}
                        | {"checked": f"layer 0 k, every output of the timed call, T={T}"}}
    return res


def time_single_configs(device: str, reps: int = 200) -> dict:
    """The single-linear configurations: 256x256 r64 (fp32 x, latency); the 7B
    attention projection 4096x4096 r2048 and the 7B MLP set (gate/up 11008x4096,
    down 4096x11008, r2368) at T=1 and T=8 (bf16 x).

    Copy 0 of each is packed from the config's fp32 latents (checked against
    the oracle on every output); the weights of a 7B layer (2.2 MB, 13.7 MB for
    the MLP set) sit in the 256 MB Infinity Cache, so HBM rates rotate over
    >= 1 GiB of distinct copies (copies 1.. drawn with SplitMix64 words, a
    sampled-row oracle check on the last one):
      single_call      -- nq_lrb_linear calls back to back, each on the next copy
                          (one call per linear; a decode-regime call is one
                          kernel launch);
      sequence         -- the same copies as one sequence plan (one persistent
                          launch for all of them): the HBM rate;
      cache_hot        -- calls back to back on copy 0 only (cache-resident);
      isolated_latency -- one call between two events, then synchronise
                          (median of 50)."""
    import statistics

    import numpy as np
    import torch

    import sub_bit_weight_amd as nq
    import synth
    from tests import checks as C

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def timed(fn, n):
        for _ in range(_warm(fn, 1, WARM_MS)):  # past the first ~30 ms after an idle gap
            fn()
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record()
        for _ in range(n):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    def isolated(fn, n=50):
        out = []
        for _ in range(n):
            torch.cuda.synchronize()
            a, b = ev(), ev()
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            out.append(a.elapsed_time(b))
        return statistics.median(out)

    def copies_for(cfg, n_copies):
        rot = synth.Config(f"{cfg.key}_rot", f"{cfg.description}, rotation copies", cfg.layers, cfg.T, cfg.x_dtype,
                           scale_kind=cfg.scale_kind, outlier_frac=cfg.outlier_frac, words="splitmix")
        sets = []
        inp0 = [synth.lrb_inputs(cfg, s) for s in cfg.layers]
        sets.append([nq.Lrb(s.d_out, s.d_in, s.r, nq.pack_u(torch.from_numpy(i["U_latent"]).to(device)),
                            nq.pack_v(torch.from_numpy(i["V_latent"]).to(device)),
                            torch.from_numpy(i["s1"]).to(device), torch.from_numpy(i["s2"]).to(device))
                     for s, i in zip(cfg.layers, inp0)])
        del inp0
        for c in range(1, n_copies):
            layer = []
            for s in cfg.layers:
                inp = synth.lrb_inputs(rot, s, c)
                nwu, nwv = nq.n_words(s.r), nq.n_words(s.d_in)
                layer.append(nq.Lrb(s.d_out, s.d_in, s.r,
                                    nq.fill_random_words(nwu * s.d_out, inp["u_seed"], device).view(nwu, s.d_out),
                                    nq.fill_random_words(nwv * s.r, inp["v_seed"], device).view(nwv, s.r),
                                    torch.from_numpy(inp["s1"]).to(device), torch.from_numpy(inp["s2"]).to(device)))
            sets.append(layer)
        torch.cuda.synchronize()
        return rot, sets

    out = {}
    # ---- 256 x 256, r 64, fp32 x, T=1: latency only (8 KB of data)
    cfg = synth.CONFIGS["single"]
    s0 = cfg.layers[0]
    _, sets = copies_for(cfg, 1)
    L = sets[0][0]
    x_np = synth.x_for(cfg, s0.d_in, 1)
    x = torch.from_numpy(x_np).to(device)
    y = torch.empty((1, s0.d_out), device=device)
    ws = torch.empty(max(nq.lrb_workspace_bytes(L, 1), 1), dtype=torch.uint8, device=device)
    per = timed(lambda: nq.lrb_linear(L, x, y, ws), reps)
    iso = isolated(lambda: nq.lrb_linear(L, x, y, ws))
    ya = torch.empty_like(y)
    per_na = timed(lambda: nq.lrb_linear_noalloc(L, x, ya), reps)
    torch.cuda.synchronize()
    par = C.full_check(y.cpu().numpy(), C.latent_ref(cfg, s0), x_np, 1e-5, "f32")
    out["single_256"] = {"config": "256x256, r=64, T=1, fp32 x", "back_to_back_us": per * 1e3,
                         "isolated_latency_us": iso * 1e3, "noalloc_back_to_back_us": per_na * 1e3,
                         "parity": _pick(par, "every output")}
    log(f"[bench] 256x256 r64: {per * 1e3:.1f} us per call back to back, {iso * 1e3:.1f} us isolated")

    # ---- 7B attention (505 copies) and 7B MLP set (79 copies) at T=1 and T=8
    for key, n_copies, Ts in (("7b_attn", 505, (1,)), ("7b_mlp", 79, (1, 8))):
        cfg = synth.CONFIGS[key]
        rot, sets = copies_for(cfg, n_copies)
        for T in Ts:
            xs = {d: synth.x_for(cfg, d, T) for d in sorted({s.d_in for s in cfg.layers})}
            xd = {d: torch.from_numpy(v).to(device).to(torch.bfloat16) for d, v in xs.items()}
            nbytes = algorithmic_bytes(cfg.layers, T)
            ws = torch.empty(max(nq.lrb_workspace_bytes(L, T) for L in sets[0]), dtype=torch.uint8, device=device)
            ybuf = {s.name: torch.empty((T, s.d_out), device=device) for s in cfg.layers}

            def call_set(layer):
                for L, s in zip(layer, cfg.layers):
                    nq.lrb_linear(L, xd[s.d_in], ybuf[s.name], ws)

            def rotate():
                for layer in sets:
                    call_set(layer)
            hot = timed(lambda: call_set(sets[0]), reps)
            rot_ms = timed(rotate, 3) / n_copies
            iso = isolated(lambda: call_set(sets[0]))
            # parity of copy 0's single-call outputs (every output)
            call_set(sets[0])
            torch.cuda.synchronize()
            par = [C.full_check(ybuf[s.name].cpu().numpy(), C.latent_ref(cfg, s), xs[s.d_in], 1e-5, "bf16",
                                factored=True) for s in cfg.layers]
            # the same copies as one sequence plan
            seq_layers = [L for layer in sets for L in layer]
            seq_shapes = [s for _ in sets for s in cfg.layers]
            ys = [torch.empty((T, s.d_out), device=device) for s in seq_shapes]
            seq = nq.Seq(seq_layers, [xd[s.d_in] for s in seq_shapes], ys)
            seq_ms = timed(seq.run, 50)
            assert seq.device_error() == 0
            nl = len(cfg.layers)
            par += [C.full_check(ys[i].cpu().numpy(), C.latent_ref(cfg, s), xs[s.d_in], 1e-5, "bf16", factored=True)
                    for i, s in enumerate(cfg.layers)]
            for i, s in enumerate(cfg.layers):  # the last copy, sampled rows
                rows = np.sort(synth.rng(f"bench/rot/{key}/{s.name}").choice(s.d_out, 64, replace=False))
                idx = (n_copies - 1) * nl + i
                par.append(C.sampled_check(ys[idx].cpu().numpy()[:, rows], C.splitmix_ref(rot, s, n_copies - 1),
                                           xs[s.d_in], rows, 1e-5, "bf16"))
            seq.close()
            del seq, ys
            res = {"config": f"{cfg.description}, T={T}, bf16 x", "copies": n_copies,
                   "distinct_bytes": nbytes * n_copies, "algorithmic_bytes_per_copy": nbytes,
                   "sequence": {"ms_per_copy": seq_ms / n_copies, "gbs": nbytes * n_copies / (seq_ms * 1e-3) / 1e9},
                   "single_call": {"us_per_copy": rot_ms * 1e3, "gbs": nbytes / (rot_ms * 1e-3) / 1e9},
                   "cache_hot": {"us_per_copy": hot * 1e3, "gbs": nbytes / (hot * 1e-3) / 1e9},
                   "isolated_latency_us": iso * 1e3,
                   "parity": _summ(par) | {"checked": "copy 0 every output (single call and sequence); "
                                                     "last copy 64 sampled rows (sequence)"}}
            res["sequence"]["frac_of_hbm_peak"] = res["sequence"]["gbs"] / HBM_PEAK_GBS
            out[f"{key}_T{T}"] = res
            log(f"[bench] {key} T={T}: sequence {res['sequence']['gbs']:.0f} GB/s over {n_copies} copies, "
                f"single calls {res['single_call']['gbs']:.0f} GB/s ({rot_ms * 1e3:.1f} us per copy), "
                f"cache-hot {res['cache_hot']['gbs']:.0f} GB/s, parity {'ok' if res['parity']['pass'] else 'FAIL'}")
        del sets
        torch.cuda.empty_cache()
    return out


def _pick(check: dict, what: str) -> dict:
    return {k: check[k] for k in ("normwise", "per_token_max", "elem_rms_max", "tol", "pass") if k in check} | {
        "checked": what}


def vendor_gemm_reference(shapes, T: int, device: str) -> dict:
    """Context for the matrix-core roofline: torch.matmul (hipBLASLt) on dense
    bf16 operands of the same GEMM shapes as the two LRB stages (M = T,
    N = r or d_out, K = d_in or r), TFLOP/s per distinct shape.  The LRB
    kernels read 1-bit B operands instead of bf16 ones."""
    import torch
    out = {}
    for s in shapes:
        for stage, (N, K) in (("stage1", (s.r, s.d_in)), ("stage2", (s.d_out, s.r))):
            key = f"{T}x{N}x{K}"
            if key in out:
                continue
            a = torch.randn(T, K, device=device, dtype=torch.bfloat16)
            b = torch.randn(K, N, device=device, dtype=torch.bfloat16)
            for _ in range(3):
                a @ b
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(10):
                a @ b
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / 10
            out[key] = round(2 * T * N * K / (ms * 1e-3) / 1e12, 1)
            del a, b
    return out


def cpu_baseline(cfg, min_s: float = 10.0) -> dict:
    """The oracle on the host cores, on a bounded sample of the decode step.

    Main line (value): the oracle's definition, reconstruct-then-multiply
    (oracle.reconstruct_ref, then the product with x), on the linears of layer
    0, 1, ... in stack order until at least `min_s` seconds are spent,
    extrapolated to the 560-linear T=1 step by flops (the 80 layers have
    identical shapes); reconstruct and apply are timed separately.  Second
    line: the oracle's factored fp64 evaluation (linear_factored_ref: the sign
    matrices unpacked to fp64, then two products), sampled the same way and
    extrapolated by the sign elements it unpacks.  Thread count and BLAS from
    threadpoolctl."""
    import numpy as np

    import synth
    from oracle import nq_oracle as O
    from tests import checks as C
    blas = {}
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if info:
            blas = {"blas": f"{info[0].get('internal_api')} {info[0].get('version')}",
                    "blas_threads": int(info[0].get("num_threads", 1))}
    except Exception:
        pass
    host_cpus = len(os.sched_getaffinity(0))

    def linears():
        for l in range(80):
            for s in cfg.layers:
                yield l, s

    # reconstruct-then-multiply
    t_rec = t_app = 0.0
    flops = 0
    done = []
    for l, s in linears():
        ref = C.splitmix_ref(cfg, s, l)
        x = synth.x_for(cfg, s.d_in, 1).astype(np.float64)
        t = time.perf_counter()
        W = O.reconstruct_ref(ref)
        t_rec += time.perf_counter() - t
        t = time.perf_counter()
        _ = x @ W.T
        t_app += time.perf_counter() - t
        del W
        flops += 2 * s.d_out * s.d_in * s.r + 2 * s.d_out * s.d_in
        done.append(f"{l}.{s.name}")
        if t_rec + t_app >= min_s:
            break
    step_flops = 80 * sum(2 * s.d_out * s.d_in * s.r + 2 * s.d_out * s.d_in for s in cfg.layers)
    scale = step_flops / flops
    step_s = (t_rec + t_app) * scale
    # factored fp64
    t_fac, elems, done_f = 0.0, 0, []
    for l, s in linears():
        ref = C.splitmix_ref(cfg, s, l)
        x = synth.x_for(cfg, s.d_in, 1)
        t = time.perf_counter()
        O.linear_factored_ref(ref, x)
        t_fac += time.perf_counter() - t
        elems += s.r * (s.d_in + s.d_out)
        done_f.append(f"{l}.{s.name}")
        if t_fac >= min_s:
            break
    step_elems = 80 * sum(s.r * (s.d_in + s.d_out) for s in cfg.layers)
    fac_s = t_fac * step_elems / elems
    return {"value": 1.0 / step_s, "unit": "tokens/s", "cores": int(blas.get("blas_threads", host_cpus)),
            "kind": "oracle",
            "sample": (f"oracle reconstruct-then-multiply in fp64, T=1, on {len(done)} linears ({done[0]} .. "
                       f"{done[-1]}, {t_rec + t_app:.1f} s), extrapolated by flops to the 560-linear step "
                       f"({step_s:.0f} s/token; identical layer shapes)"),
            "reconstruct_s_per_step": t_rec * scale, "apply_s_per_step": t_app * scale,
            "host_cpus": host_cpus, **blas,
            "factored": {"value": 1.0 / fac_s, "unit": "tokens/s", "s_per_step": fac_s,
                         "sample": (f"oracle factored fp64 evaluation (sign matrices unpacked to fp64, two "
                                    f"products) on {len(done_f)} linears ({done_f[0]} .. {done_f[-1]}, "
                                    f"{t_fac:.1f} s), extrapolated by unpacked sign elements")}}


STACK_PICKS = [(0, "q"), (0, "k"), (79, "gate"), (79, "down")]  # one linear of each distinct shape


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=40,
                    help="untimed steps first; launches after an idle gap run up to 40%% slower for ~30 ms")
    ap.add_argument("--layers", type=int, default=80, help="decoder layers in the stack (80 = Llama-2-70B)")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-055", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-grads", action="store_true", help="skip the scale-gradient (calibration) leg")
    ap.add_argument("--no-balance", action="store_true", help="skip the magnitude-balancing leg")
    ap.add_argument("--no-latent", action="store_true", help="skip the latent-factor forward leg")
    ap.add_argument("--no-single", action="store_true",
                    help="skip the single-linear configurations (256x256, 7B attention, 7B MLP set)")
    ap.add_argument("--no-lag7", action="store_true", help="skip the decode step with a one-layer stage lag")
    ap.add_argument("--no-rank-sweep", action="store_true",
                    help="skip decode at 0.25x .. 2x the 1-bit ranks (0.25 .. 2 bit/weight)")
    ap.add_argument("--prefill-serial", action="store_true",
                    help="also time the prefill pass as serial single-linear calls on one stream")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy 5 times (reference for HBM byte counters)")
    ap.add_argument("--grads-profile", type=int, default=0, metavar="N",
                    help="run layer 0's batched scale gradients at T=2048 N times, synchronising between "
                         "passes (for a kernel trace), and exit")
    ap.add_argument("--prefill-profile", type=int, default=0, metavar="N",
                    help="only run layer 0's seven T=2048 linears N times each, one after another, each as a "
                         "one-entry sequence plan (the kernels and tiles of the benchmarked pass, in a fixed "
                         "order: for profilers)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (see the design notes "
              "for how the layer would shard). Run with --gpus 1.", file=sys.stderr)
        return 2

    import statistics

    import torch

    import synth
    device = "cuda:0"
    torch.cuda.set_device(0)

    if args.copy_calibration:
        a = torch.ones(1 << 28, dtype=torch.int32, device=device)  # 1 GiB
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration": {"bytes_read_per_copy": a.numel() * 4,
                                               "bytes_written_per_copy": a.numel() * 4, "copies": 5}}))
        return 0

    if args.grads_profile:
        stack = Stack(synth.stack_config(1.0), 1, device)
        time_scale_grads(stack, 2048, device, profile_passes=args.grads_profile)
        log(f"[bench] profile: scale gradients, layer 0, T=2048 x{args.grads_profile}")
        return 0

    if args.prefill_profile:
        import sub_bit_weight_amd as nq
        stack = Stack(synth.CONFIGS["70b_prefill"], 1, device)
        Tp = 2048
        for L, s in zip(stack.layers, stack.shapes):
            x = torch.from_numpy(synth.x_for(stack.cfg, s.d_in, Tp)).to(device).to(torch.bfloat16)
            y = torch.empty((Tp, s.d_out), dtype=torch.float32, device=device)
            seq = nq.Seq([L], [x], [y])
            for _ in range(args.prefill_profile):
                seq.run()
            torch.cuda.synchronize()
            log(f"[bench] profile: {s.name} {s.d_out}x{s.d_in} r{s.r} T{Tp} x{args.prefill_profile}")
            seq.close()
        return 0

    cfg = synth.stack_config(1.0)
    log(f"[bench] building 70B stack (~1.0 bit), {args.layers} layers")
    stack = Stack(cfg, args.layers, device)
    T = 1
    log("[bench] decode T=1")
    ms, seq, xs, ys = time_decode(stack, T, args.steps, args.warmup, device)
    bytes_step = algorithmic_bytes(stack.shapes, T)
    import sub_bit_weight_amd as nq
    head_bits = (sum(nq.storage_bits(sh.d_out, sh.d_in, sh.r) for sh in stack.shapes)
                 / sum(sh.d_out * sh.d_in for sh in stack.shapes))
    gbs = bytes_step / (ms * 1e-3) / 1e9
    log(f"[bench] decode {ms:.3f} ms/step, {gbs:.0f} GB/s (one persistent-kernel launch per step)")
    parity = stack_parity(stack, xs, ys, STACK_PICKS)
    log(f"[bench] decode parity: normwise {parity['normwise']:.2e}, per-token {parity['per_token_max']:.2e}, "
        f"pass {parity['pass']}")
    del seq

    extra = {}
    if not args.no_lag7:
        # stage 2 of each linear right after stage 1 of the linear 7 places on
        # (one decoder layer): little overlap across layers
        os.environ["NQ_SEQ_LAG"] = "7"
        try:
            ms7, seq7, xs7, ys7 = time_decode(stack, T, args.steps, args.warmup, device, WARM_MS)
        finally:
            del os.environ["NQ_SEQ_LAG"]
        p7 = stack_parity(stack, xs7, ys7, STACK_PICKS[:2])
        extra["decode_lag7"] = {"ms_per_step": ms7, "tokens_per_s": 1000.0 / ms7,
                                "hbm_gbs": bytes_step / (ms7 * 1e-3) / 1e9,
                                "frac_of_hbm_peak": bytes_step / (ms7 * 1e-3) / 1e12 / 8.0,
                                "schedule": "stage 2 of each linear after stage 1 of the linear 7 places on "
                                            "(one decoder layer); the headline uses 320",
                                "parity": p7}
        log(f"[bench] decode lag 7: {ms7:.3f} ms/step, {extra['decode_lag7']['hbm_gbs']:.0f} GB/s")
        del seq7
    if not args.no_prefill:
        Tp = 2048
        log("[bench] prefill T=2048")
        ptimes, pseq, pxs, pys = time_prefill(stack, Tp, device)
        pms = statistics.median(ptimes)
        ppar = stack_parity(stack, pxs, pys, STACK_PICKS, rows_per=32)
        log(f"[bench] prefill parity: normwise {ppar['normwise']:.2e}, per-token {ppar['per_token_max']:.2e}, "
            f"pass {ppar['pass']}")
        del pseq, pys
        flops = algorithmic_flops(stack.shapes, Tp)
        tf = flops / (pms * 1e-3) / 1e12
        extra["prefill"] = {"T": Tp, "ms_per_pass": pms, "ms_per_pass_all": ptimes, "tflops": tf,
                            "frac_of_f16_peak": tf / F16_PEAK_TFLOPS,
                            "tokens_per_s": Tp / (pms * 1e-3), "algorithmic_flop": flops,
                            "roofline": {"bound": "mfma", "kernel": "gemm_kernel (whole pass incl. prep kernels)",
                                         "achieved": tf, "peak": F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                         "frac": tf / F16_PEAK_TFLOPS,
                                         "traffic": summary_field(PREFILL_COUNTERS, PREFILL_SRC, "prefill.hip sha256",
                                                                  "hbm bytes per pass"),
                                         "basis": f"median of {len(ptimes)} passes, HIP events on the caller's "
                                                  "stream around each pass"},
                            "operands": "fp16 (per-token power-of-two scaled) x +-1, fp32 accumulate",
                            "includes": "prep kernels (row scaling, fp16 conversion) and both GEMMs of all 560 linears",
                            "parity": ppar}
        log(f"[bench] prefill {pms:.1f} ms/pass (median of {len(ptimes)}), {tf:.0f} TFLOP/s")
        if args.prefill_serial:
            sms = time_prefill_serial(stack, Tp, device)
            extra["prefill"]["serial_ms_per_pass"] = sms
            extra["prefill"]["serial_tflops"] = flops / (sms * 1e-3) / 1e12
            log(f"[bench] prefill serial {sms:.1f} ms/pass")
        extra["prefill"]["vendor_dense_bf16_gemm_tflops"] = vendor_gemm_reference(stack.shapes[:len(cfg.layers)],
                                                                                  Tp, device)
    if not args.no_grads:
        log("[bench] scale gradients T=2048 (layer 0)")
        extra["scale_grads"] = time_scale_grads(stack, 2048, device)
        g = extra["scale_grads"]
        log(f"[bench] scale gradients {g['ms_per_layer']:.2f} ms/layer, {g['tflops']:.0f} TFLOP/s, "
            f"parity {g['parity']['pass']}")
    if not args.no_balance:
        log("[bench] magnitude balancing (layer 0 latents)")
        extra["balance"] = time_balance(stack.shapes[:len(cfg.layers)], device)
        b = extra["balance"]
        log(f"[bench] balancing {b['balanced_factors']['ms_per_layer']:.2f} ms/layer "
            f"({b['balanced_factors']['gbs']:.0f} GB/s), scales only {b['scales_only']['ms_per_layer']:.2f} ms "
            f"({b['scales_only']['gbs']:.0f} GB/s), parity {b['parity']['pass']}")
    if not args.no_latent:
        log("[bench] refinement forward from latents (layer 0)")
        extra["latent_forward"] = time_latent(stack.shapes[:len(cfg.layers)], device)
        lf = extra["latent_forward"]
        log(f"[bench] latent forward T=1 {lf['T1']['ms_per_layer']:.2f} ms/layer ({lf['T1']['gbs']:.0f} GB/s), "
            f"T=2048 {lf['T2048']['ms_per_layer']:.2f} ms/layer ({lf['T2048']['tflops']:.0f} TFLOP/s)")
    del stack
    torch.cuda.empty_cache()

    if not args.no_single:
        log("[bench] single-linear configurations")
        extra["single_configs"] = time_single_configs(device)
        torch.cuda.empty_cache()

    def stack_leg(frac, picks):
        cfgf = synth.stack_config(frac)
        stf = Stack(cfgf, args.layers, device)
        msf, seqf, xsf, ysf = time_decode(stf, 1, args.steps, args.warmup, device, WARM_MS)
        bf = algorithmic_bytes(stf.shapes, 1)
        weights = sum(sh.d_out * sh.d_in for sh in stf.shapes)
        import sub_bit_weight_amd as nq
        bits = sum(nq.storage_bits(sh.d_out, sh.d_in, sh.r) for sh in stf.shapes) / weights
        par = stack_parity(stf, xsf, ysf, picks)
        del seqf, stf
        torch.cuda.empty_cache()
        return {"rank_frac": frac, "bits_per_weight": bits, "ms_per_step": msf, "tokens_per_s": 1000.0 / msf,
                "hbm_gbs": bf / (msf * 1e-3) / 1e9, "frac_of_hbm_peak": bf / (msf * 1e-3) / 1e12 / 8.0,
                "algorithmic_bytes": bf, "parity": par}

    if not args.no_055:
        log("[bench] decode T=1, 0.55-bit stack")
        extra["decode_055bit"] = stack_leg(0.55, STACK_PICKS)
        d = extra["decode_055bit"]
        log(f"[bench] 0.55-bit: {d['ms_per_step']:.3f} ms/step, {d['hbm_gbs']:.0f} GB/s, parity {d['parity']['pass']}")

    if not args.no_rank_sweep:
        # the decode kernels across ranks: 0.25 .. 2.0 bit/weight of sign storage
        sweep = []
        for frac in (0.25, 0.5, 0.75, 1.0, 1.5, 2.0):
            if frac == 1.0:  # the headline stack
                sweep.append({"rank_frac": 1.0, "bits_per_weight": head_bits, "ms_per_step": ms,
                              "tokens_per_s": 1000.0 / ms, "hbm_gbs": gbs, "frac_of_hbm_peak": gbs / HBM_PEAK_GBS,
                              "algorithmic_bytes": bytes_step, "parity": parity, "note": "the headline run"})
                continue
            sweep.append(stack_leg(frac, [(0, "k"), (79, "down")]))
            w = sweep[-1]
            log(f"[bench] rank x{frac}: {w['bits_per_weight']:.3f} bit/weight, {w['ms_per_step']:.3f} ms/step, "
                f"{w['hbm_gbs']:.0f} GB/s, parity {w['parity']['pass']}")
        extra["rank_sweep"] = sweep

    out = {
        "metric": "decode tokens/s + HBM GB/s (T=1), prefill TFLOP/s (T=2048), 70B-shaped LRB layers",
        "value": T * 1000.0 / ms,
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp32", "data": "synthetic",
        "config": {"workload": f"Llama-2-70B-shaped LRB linear stack, {args.layers} layers x 7 linears, "
                               f"~1.0 bit/weight, T=1 decode, bf16 x, fp32 y",
                   "global_batch": T, "layers": args.layers, "parallelism": "single-gpu"},
        "hbm_gbs": gbs,
        "algorithmic_bytes_per_step": bytes_step,
        "roofline": {"bound": "hbm", "kernel": "dec_persistent_kernel<1> (one launch per step)",
                     "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": measured_traffic()},
        # The decode kernel's compute ceilings at 2.4 GHz: one 16x16x128
        # fp4 x fp8 MFMA (32 cycles) per 64 sign words and SIMD; 7 full-rate
        # VALU ops (2 cycles per wave64 op) per word expansion (the whole
        # kernel issues 9.7 VALU instructions per 64 words, MFMAs included).
        "decode_mfma_ceiling_gbs": 256 * 4 * 2.4e9 / 32 * 256 / 1e9,
        "decode_valu_ceiling_gbs": 256 * 4 * 2.4e9 / (7 * 2) * 256 / 1e9,
        "parity": parity,
    }
    out.update(extra)
    if not args.no_cpu:
        log("[bench] cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(cfg)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
