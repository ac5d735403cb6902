#!/usr/bin/env python3
"""Benchmark of the NanoQuant low-rank binary (LRB) linear on one MI355X.

Workload (one "step"): one decode token (T=1) through every linear of a
Llama-2-70B-shaped stack -- 80 layers x {q, k, v, o, gate, up, down} = 560 LRB
linears at ~1.0 bit/weight (r = d_out*d_in/(d_out+d_in) rounded down to a
multiple of 64), each y = s1 (.) U (V^T (s2 (.) x)) on its own bf16 input.
Sign words are drawn directly with SplitMix64 on the device; scales and inputs
come from the seeded host generators (module synth).  The same run also times
the 0.55-bit stack (decode) and a T=2048 prefill pass over the ~1.0-bit stack.

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


def time_decode(stack, T: int, steps: int, warmup: int, device: str):
    import torch

    import sub_bit_weight_amd as nq
    import synth
    xs_by_din = {d: torch.from_numpy(synth.x_for(stack.cfg, d, T)).to(device).to(torch.bfloat16)
                 for d in sorted({s.d_in for s in stack.shapes})}
    xs = [xs_by_din[s.d_in] for s in stack.shapes]
    ys = [torch.empty((T, s.d_out), dtype=torch.float32, device=device) for s in stack.shapes]
    seq = nq.Seq(stack.layers, xs, ys)
    for _ in range(warmup):
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


def parity_sample(stack, xs, ys, idx: int, n_rows: int = 16) -> float:
    """Oracle check of one linear of the stack on sampled output rows."""
    import numpy as np

    import synth
    from oracle import nq_oracle as O
    s = stack.shapes[idx]
    l = idx // len(stack.cfg.layers)
    inp = synth.lrb_inputs(stack.cfg, s, l)
    nwu, nwv = (s.r + 31) // 32, (s.d_in + 31) // 32
    ref = O.LRB(synth.random_words(inp["u_seed"], np.arange(nwu * s.d_out, dtype=np.uint64)).reshape(nwu, s.d_out),
                synth.random_words(inp["v_seed"], np.arange(nwv * s.r, dtype=np.uint64)).reshape(nwv, s.r),
                inp["s1"], inp["s2"], s.d_out, s.d_in, s.r)
    rows = np.sort(synth.rng(f"bench/rows/{idx}").choice(s.d_out, n_rows, replace=False))
    x = xs[idx].float().cpu().numpy()
    y = ys[idx].cpu().numpy()
    return O.rel_err(y[:, rows], O.sampled_linear_ref(ref, x, rows))


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


def time_prefill(stack, T: int, device: str):
    """One T-token pass over every linear of the stack as one sequence plan
    (entries run round-robin on the plan's streams).  Returns (ms, seq, xs,
    ys); each linear has its own output."""
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
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    seq.run()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1), seq, xs, ys


def time_scale_grads(stack, T: int, device: str, reps: int = 3) -> dict:
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
    for L, a, x, g in zip(layers, adjs, xs, gs):  # warm-up pass
        nq.lrb_scale_grads(L, a, x, g, workspace=ws)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        for L, a, x, g in zip(layers, adjs, xs, gs):
            nq.lrb_scale_grads(L, a, x, g, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    flops = sum(2 * 2 * T * s.r * (s.d_in + s.d_out) for s in shapes)  # forward + transposed product
    # parity on a few tokens of layer 0's k against the float64 oracle
    k = [s.name for s in shapes].index("k")
    s = shapes[k]
    inp = synth.lrb_inputs(stack.cfg, s, 0)
    nwu, nwv = (s.r + 31) // 32, (s.d_in + 31) // 32
    ref = O.LRB(synth.random_words(inp["u_seed"], np.arange(nwu * s.d_out, dtype=np.uint64)).reshape(nwu, s.d_out),
                synth.random_words(inp["v_seed"], np.arange(nwv * s.r, dtype=np.uint64)).reshape(nwv, s.r),
                inp["s1"], inp["s2"], s.d_out, s.d_in, s.r)
    xq, gq = xs[k][:4].contiguous(), gs[k][:4].contiguous()
    got = nq.lrb_scale_grads(layers[k], adjs[k], xq, gq)
    want = O.scale_grads_factored_ref(ref, xq.float().cpu().numpy(), gq.float().cpu().numpy())
    err = max(O.rel_err(a.cpu().numpy(), b) for a, b in zip(got, want))
    return {"T": T, "linears": f"layer 0 ({per} linears)", "ms_per_layer": ms,
            "tflops": flops / (ms * 1e-3) / 1e12, "frac_of_f16_peak": flops / (ms * 1e-3) / 1e12 / F16_PEAK_TFLOPS,
            "algorithmic_flop_per_layer": flops,
            "includes": "forward product without s1, transposed product without s2, token sums; x and g bf16",
            "transpose_ms_per_layer": t_ms, "transpose_gbs": t_bytes / (t_ms * 1e-3) / 1e9,
            "parity_rel_err": err, "parity_case": "layer 0 k, 4 tokens, max over dx, ds1, ds2"}


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
    res.update({"linears": f"layer 0 ({len(shapes)} linears)", "latent_bytes": lat_bytes, "parity_rel_err": err,
                "parity_case": f"{s0.name}: U, V, s1, s2, eta"})
    return res


def time_latent(shapes, device: str, reps: int = 5) -> dict:
    """The refinement forward from fp32 latent factors (signs packed at the
    call, then the packed layer) over layer 0's linears, at T=1 and T=2048
    (bf16 x).  At T=1 the latents dominate the bytes: GB/s counts the latent
    reads, the packed words written and read back, x and y."""
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
        run()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            run()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        nbytes = sum((s.d_out + s.d_in) * s.r * 4 + 2 * (s.d_out + s.d_in) * s.r // 8 + T * (2 * s.d_in + 4 * s.d_out)
                     for s in shapes)
        flops = sum(2 * T * s.r * (s.d_in + s.d_out) for s in shapes)
        res[f"T{T}"] = {"ms_per_layer": ms, "gbs": nbytes / (ms * 1e-3) / 1e9,
                        "frac_of_hbm_peak": nbytes / (ms * 1e-3) / 1e12 / 8.0, "tflops": flops / (ms * 1e-3) / 1e12,
                        "algorithmic_bytes": nbytes}
    return res


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
    """The oracle (reconstruct in fp64, then multiply) on the host cores, on a
    bounded sample of the decode step: the linears of layer 0, then layer 1,
    ... in stack order until at least `min_s` seconds of oracle work are done,
    extrapolated to the 560-linear step by reconstruction flops."""
    import numpy as np

    import synth
    from oracle import nq_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"),
                      default=1)
    except Exception:
        threads = len(os.sched_getaffinity(0))
    done, done_flops, elapsed = [], 0, 0.0
    for l in range(80):
        for s in cfg.layers:
            inp = synth.lrb_inputs(cfg, s, l)
            nwu, nwv = (s.r + 31) // 32, (s.d_in + 31) // 32
            ref = O.LRB(synth.random_words(inp["u_seed"], np.arange(nwu * s.d_out, dtype=np.uint64)).reshape(nwu, s.d_out),
                        synth.random_words(inp["v_seed"], np.arange(nwv * s.r, dtype=np.uint64)).reshape(nwv, s.r),
                        inp["s1"], inp["s2"], s.d_out, s.d_in, s.r)
            x = synth.x_for(cfg, s.d_in, 1)
            t = time.perf_counter()
            O.linear_ref(ref, x)
            elapsed += time.perf_counter() - t
            done_flops += 2 * s.d_out * s.d_in * s.r + 2 * s.d_out * s.d_in
            done.append(f"{l}.{s.name}")
            if elapsed >= min_s:
                break
        if elapsed >= min_s:
            break
    step_flops = 80 * sum(2 * s.d_out * s.d_in * s.r + 2 * s.d_out * s.d_in for s in cfg.layers)
    step_s = elapsed * step_flops / done_flops
    return {"value": 1.0 / step_s, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"oracle linear_ref (fp64 reconstruct-then-multiply, T=1) on {len(done)} linears "
                       f"({done[0]} .. {done[-1]}, {elapsed:.1f} s), extrapolated by reconstruction flops to "
                       f"the 560-linear T=1 step ({step_s:.0f} s/token)")}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", type=int, default=80, help="decoder layers in the stack (80 = Llama-2-70B)")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-055", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-grads", action="store_true", help="skip the scale-gradient (calibration) leg")
    ap.add_argument("--no-balance", action="store_true", help="skip the magnitude-balancing leg")
    ap.add_argument("--no-latent", action="store_true", help="skip the latent-factor forward leg")
    ap.add_argument("--no-rank-sweep", action="store_true",
                    help="skip decode at 0.25x .. 2x the 1-bit ranks (0.25 .. 2 bit/weight)")
    ap.add_argument("--prefill-serial", action="store_true",
                    help="also time the prefill pass as serial single-linear calls on one stream")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy 5 times (reference for HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (see the design notes "
              "for how the layer would shard). Run with --gpus 1.", file=sys.stderr)
        return 2

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

    cfg = synth.CONFIGS["70b_stack"]
    log(f"[bench] building 70B stack (~1.0 bit), {args.layers} layers")
    stack = Stack(cfg, args.layers, device)
    T = 1
    log("[bench] decode T=1")
    ms, seq, xs, ys = time_decode(stack, T, args.steps, args.warmup, device)
    bytes_step = algorithmic_bytes(stack.shapes, T)
    gbs = bytes_step / (ms * 1e-3) / 1e9
    log(f"[bench] decode {ms:.3f} ms/step, {gbs:.0f} GB/s (one persistent-kernel launch per step)")
    err = parity_sample(stack, xs, ys, idx=len(cfg.layers) - 1)
    log(f"[bench] parity (layer 0 down, 16 rows) rel err {err:.2e}")
    del seq

    extra = {}
    if not args.no_prefill:
        Tp = 2048
        log("[bench] prefill T=2048")
        pms, pseq, pxs, pys = time_prefill(stack, Tp, device)
        perr = parity_sample(stack, pxs, pys, idx=0)  # layer 0 q, 16 rows, all 2048 tokens
        log(f"[bench] prefill parity (layer 0 q, 16 rows) rel err {perr:.2e}")
        del pseq, pys
        flops = algorithmic_flops(stack.shapes, Tp)
        extra["prefill"] = {"T": Tp, "ms_per_pass": pms, "tflops": flops / (pms * 1e-3) / 1e12,
                            "frac_of_f16_peak": flops / (pms * 1e-3) / 1e12 / F16_PEAK_TFLOPS,
                            "tokens_per_s": Tp / (pms * 1e-3), "algorithmic_flop": flops,
                            "operands": "fp16 (per-token power-of-two scaled) x +-1, fp32 accumulate",
                            "includes": "prep kernels (row scaling, fp16 conversion) and both GEMMs of all 560 linears",
                            "parity_rel_err": perr}
        log(f"[bench] prefill {pms:.1f} ms/pass, {extra['prefill']['tflops']:.0f} TFLOP/s")
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
            f"parity {g['parity_rel_err']:.2e}")
    if not args.no_balance:
        log("[bench] magnitude balancing (layer 0 latents)")
        extra["balance"] = time_balance(stack.shapes[:len(cfg.layers)], device)
        b = extra["balance"]
        log(f"[bench] balancing {b['balanced_factors']['ms_per_layer']:.2f} ms/layer "
            f"({b['balanced_factors']['gbs']:.0f} GB/s), scales only {b['scales_only']['ms_per_layer']:.2f} ms "
            f"({b['scales_only']['gbs']:.0f} GB/s), parity {b['parity_rel_err']:.2e}")
    if not args.no_latent:
        log("[bench] refinement forward from latents (layer 0)")
        extra["latent_forward"] = time_latent(stack.shapes[:len(cfg.layers)], device)
        lf = extra["latent_forward"]
        log(f"[bench] latent forward T=1 {lf['T1']['ms_per_layer']:.2f} ms/layer ({lf['T1']['gbs']:.0f} GB/s), "
            f"T=2048 {lf['T2048']['ms_per_layer']:.2f} ms/layer ({lf['T2048']['tflops']:.0f} TFLOP/s)")
    del stack
    torch.cuda.empty_cache()

    if not args.no_055:
        cfg55 = synth.CONFIGS["70b_stack_055"]
        log("[bench] decode T=1, 0.55-bit stack")
        st55 = Stack(cfg55, args.layers, device)
        ms55, seq55, _, _ = time_decode(st55, 1, args.steps, args.warmup, device)
        b55 = algorithmic_bytes(st55.shapes, 1)
        extra["decode_055bit"] = {"ms_per_step": ms55, "tokens_per_s": 1000.0 / ms55,
                                  "hbm_gbs": b55 / (ms55 * 1e-3) / 1e9, "algorithmic_bytes": b55}
        del seq55, st55
        torch.cuda.empty_cache()

    if not args.no_rank_sweep:
        import sub_bit_weight_amd as nq
        # the decode kernels across ranks: 0.25 .. 2.0 bit/weight of sign storage
        sweep = []
        for frac in (0.25, 0.5, 0.75, 1.0, 1.5, 2.0):
            cfgf = synth.Config(f"70b_stack_{frac}", f"Llama-2-70B linear stack, {frac} x the 1-bit rank",
                                synth.llama2_70b_layer(frac), (1,), "bf16", n_layers=80, words="splitmix")
            stf = Stack(cfgf, args.layers, device)
            msf, seqf, _, _ = time_decode(stf, 1, args.steps, args.warmup, device)
            bf = algorithmic_bytes(stf.shapes, 1)
            weights = sum(sh.d_out * sh.d_in for sh in stf.shapes)
            bits = sum(nq.storage_bits(sh.d_out, sh.d_in, sh.r) for sh in stf.shapes) / weights
            sweep.append({"rank_frac": frac, "bits_per_weight": bits, "ms_per_step": msf,
                          "tokens_per_s": 1000.0 / msf, "hbm_gbs": bf / (msf * 1e-3) / 1e9,
                          "frac_of_hbm_peak": bf / (msf * 1e-3) / 1e12 / 8.0})
            log(f"[bench] rank x{frac}: {bits:.3f} bit/weight, {msf:.3f} ms/step, {sweep[-1]['hbm_gbs']:.0f} GB/s")
            del seqf, stf
            torch.cuda.empty_cache()
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
        # fp4 x fp8 MFMA (32 cycles) per 64 sign words and SIMD; 11 full-rate
        # VALU ops (2 cycles per wave64 op) per word expansion.
        "decode_mfma_ceiling_gbs": 256 * 4 * 2.4e9 / 32 * 256 / 1e9,
        "decode_valu_ceiling_gbs": 256 * 4 * 2.4e9 / (11 * 2) * 256 / 1e9,
        "parity_rel_err": err,
    }
    out.update(extra)
    if not args.no_cpu:
        log("[bench] cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(cfg)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
