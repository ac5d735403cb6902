"""Every configuration the benchmark times, against the oracle on the same
seeded inputs, through the C ABI: the 70B-shaped stacks at ~1.0 bit, 0.55 bit
and the rank-sweep extremes (0.25x and 2x the ~1-bit ranks), as single calls
and as sequence plans (the persistent decode schedule, also with a short
stage lag); the T=2048 matrix-core pass of one layer as a sequence plan and
gate/up as single calls; the 7B MLP set as a sequence; the scale-gradient and
latent-forward legs at a 70B shape.  Every check applies the normwise,
per-token, elementwise and deterministic bars of tests/checks.py."""
import numpy as np
import pytest
import torch

import synth
from oracle import nq_oracle as O
from tests import checks as C
from tests import gpu_cases as G

pytestmark = pytest.mark.gpu

nq = pytest.importorskip("sub_bit_weight_amd")

FRACS = [1.0, 0.55, 0.25, 2.0]


def _report(tag, e):
    print(f"{tag}: normwise {e['normwise']:.2e} per-token {e['per_token_max']:.2e} "
          f"elem/rms {e['elem_rms_max']:.2e} bound {e.get('bound_ratio_max', float('nan')):.2e}", flush=True)
    assert e["pass"], (tag, e)


def _rows(tag, n_out, n):
    return np.sort(synth.rng(f"timed/rows/{tag}").choice(n_out, min(n, n_out), replace=False))


# ---------------------------------------------------------------- decode stacks


@pytest.mark.parametrize("frac", FRACS)
@pytest.mark.parametrize("name", ["q", "k", "gate", "up", "down"])
def test_stack_single_call_decode(frac, name):
    cfg = synth.stack_config(frac)
    shape = next(s for s in cfg.layers if s.name == name)
    print(f"stack x{frac} {name} {shape.d_out}x{shape.d_in} r{shape.r} T1", flush=True)
    dev, _ = G.splitmix_layer(cfg, shape, layer_idx=0)
    ref = C.splitmix_ref(cfg, shape, 0)
    x = synth.x_for(cfg, shape.d_in, 1)
    y = nq.lrb_linear(dev, G.to_device_x(x, "bf16")).cpu().numpy()
    rows = _rows(f"{frac}/{name}", shape.d_out, 64)
    _report(f"x{frac} {name}", C.sampled_check(y[:, rows], ref, x, rows, G.decode_tol("bf16"), "bf16"))


def _stack_seq(cfg, layers, T, rows_per, tag):
    """Sequence plan over the given layers of a stack; checks sampled rows of every linear."""
    built, xs, ys, refs = [], [], [], []
    x_by_din = {}
    for l in layers:
        for s in cfg.layers:
            dev, _ = G.splitmix_layer(cfg, s, layer_idx=l)
            built.append((l, s, dev))
            if s.d_in not in x_by_din:
                x_np = synth.x_for(cfg, s.d_in, T)
                x_by_din[s.d_in] = (x_np, G.to_device_x(x_np, "bf16"))
            xs.append(x_by_din[s.d_in][1])
            ys.append(torch.full((T, s.d_out), float("nan"), device=G.DEV))
    seq = nq.Seq([b[2] for b in built], xs, ys)
    for _ in range(2):
        seq.run()
    assert seq.device_error() == 0
    for (l, s, _), y in zip(built, ys):
        rows = _rows(f"{tag}/{l}/{s.name}", s.d_out, rows_per)
        e = C.sampled_check(y.cpu().numpy()[:, rows], C.splitmix_ref(cfg, s, l), x_by_din[s.d_in][0], rows,
                            G.tol_for(T, "bf16"), "bf16")
        _report(f"{tag} layer {l} {s.name}", e)
    seq.close()


@pytest.mark.parametrize("frac", FRACS)
def test_stack_sequence_decode(frac):
    """Two layers (14 linears) through the persistent schedule, default stage lag."""
    cfg = synth.stack_config(frac)
    print(f"stack x{frac} sequence, layers 0-1", flush=True)
    _stack_seq(cfg, [0, 1], 1, 16, f"seq{frac}")


@pytest.mark.parametrize("frac", [1.0, 0.55])
def test_stack_sequence_decode_short_lag(frac, monkeypatch):
    """The same with stage 2 of each linear three linears after its stage 1, so
    most stage-2 tiles wait on their counters while other linears stream."""
    monkeypatch.setenv("NQ_SEQ_LAG", "3")
    cfg = synth.stack_config(frac)
    print(f"stack x{frac} sequence, lag 3", flush=True)
    _stack_seq(cfg, [0, 1], 1, 16, f"seqlag{frac}")


def test_stack_sequence_decode_t8():
    cfg = synth.stack_config(0.55)
    print("stack x0.55 sequence T8", flush=True)
    _stack_seq(cfg, [0], 8, 16, "seqt8")


# ---------------------------------------------------------------- matrix-core regime


def test_prefill_sequence_layer():
    """One layer's 7 linears at T=2048 as a sequence plan (the benchmarked pass:
    three streams, reductions never split)."""
    cfg = synth.CONFIGS["70b_prefill"]
    print("prefill sequence layer 0, T2048", flush=True)
    _stack_seq(cfg, [0], 2048, 16, "pfseq")


@pytest.mark.parametrize("name", ["gate", "up"])
def test_prefill_single_call_gate_up(name):
    cfg = synth.CONFIGS["70b_prefill"]
    shape = next(s for s in cfg.layers if s.name == name)
    print(f"prefill {name} T2048", flush=True)
    dev, _ = G.splitmix_layer(cfg, shape, layer_idx=0)
    x = synth.x_for(cfg, shape.d_in, 2048)
    y = nq.lrb_linear(dev, G.to_device_x(x, "bf16")).cpu().numpy()
    rows = _rows(f"pf/{name}", shape.d_out, 64)
    _report(f"prefill {name}", C.sampled_check(y[:, rows], C.splitmix_ref(cfg, shape, 0), x, rows, 2e-3, "bf16"))


# ---------------------------------------------------------------- 7B MLP set


@pytest.mark.parametrize("T", [1, 8])
def test_mlp_set_sequence(T):
    """The 7B MLP set (signs from latents) plus two SplitMix copies of it, as one
    sequence: the rotated-copies measurement's plan."""
    cfg = synth.CONFIGS["7b_mlp"]
    built = [G.latent_layer(cfg, s)[:2] for s in cfg.layers]
    rot = synth.Config("7b_mlp_rot", "7B MLP rotation copies", cfg.layers, (1, 8), "bf16",
                       scale_kind="lognormal", outlier_frac=0.01, words="splitmix")
    for c in (1, 2):
        built += [(G.splitmix_layer(rot, s, layer_idx=c)[0], C.splitmix_ref(rot, s, c)) for s in cfg.layers]
    x_np = {d: synth.x_for(cfg, d, T) for d in {s.d_in for s in cfg.layers}}
    xs = [G.to_device_x(x_np[d.d_in], "bf16") for d, _ in built]
    ys = [torch.full((T, d.d_out), float("nan"), device=G.DEV) for d, _ in built]
    seq = nq.Seq([d for d, _ in built], xs, ys)
    seq.run()
    assert seq.device_error() == 0
    for i, ((dev, ref), y) in enumerate(zip(built, ys)):
        x = x_np[dev.d_in]
        if i < 3:
            e = C.full_check(y.cpu().numpy(), ref, x, 1e-5, "bf16", factored=True)
        else:
            rows = _rows(f"mlprot/{i}", dev.d_out, 64)
            e = C.sampled_check(y.cpu().numpy()[:, rows], ref, x, rows, 1e-5, "bf16")
        _report(f"mlp set T{T} entry {i}", e)
    seq.close()


# ---------------------------------------------------------------- calibration legs at a 70B shape


def test_scale_grads_70b_k_t2048():
    """The scale-gradient leg's configuration: 70B k (1024 x 8192, r 896),
    T=2048, bf16 x and g, every gradient element against the factored oracle."""
    cfg = synth.CONFIGS["70b_stack"]
    shape = next(s for s in cfg.layers if s.name == "k")
    dev, _ = G.splitmix_layer(cfg, shape, layer_idx=0)
    ref = C.splitmix_ref(cfg, shape, 0)
    T = 2048
    x = synth.activations("timed/grads/x", T, shape.d_in, "bf16")
    g = synth.activations("timed/grads/g", T, shape.d_out, "bf16")
    dx, ds1, ds2 = nq.lrb_scale_grads(dev, nq.Adjoint.of(dev), G.to_device_x(x, "bf16"), G.to_device_x(g, "bf16"))
    rdx, rds1, rds2 = O.scale_grads_factored_ref(ref, x, g)
    _report("grads dx", C.check(dx.cpu().numpy(), rdx, 2e-3))
    for nm, got, want in (("ds1", ds1, rds1), ("ds2", ds2, rds2)):
        e = C.check(got.cpu().numpy()[None, :], want[None, :], 2e-3)
        _report(f"grads {nm}", e)


@pytest.mark.parametrize("T", [1, 2048])
def test_latent_forward_70b_k(T):
    """The latent-forward leg's configuration at the 70B k shape."""
    d_out, d_in, r = 1024, 8192, 896
    U = synth.normal_f32("timed/lat/U", (d_out, r))
    V = synth.normal_f32("timed/lat/V", (d_in, r))
    s1 = synth.scales_halfnormal("timed/lat/s1", d_out)
    s2 = synth.scales_halfnormal("timed/lat/s2", d_in)
    x = synth.activations(f"timed/lat/x/{T}", T, d_in, "bf16")
    y = nq.lrb_linear_latent(torch.from_numpy(U).to(G.DEV), torch.from_numpy(V).to(G.DEV),
                             torch.from_numpy(s1).to(G.DEV), torch.from_numpy(s2).to(G.DEV),
                             G.to_device_x(x, "bf16")).cpu().numpy()
    want = O.linear_latent_ref(U, V, s1, s2, x)
    _report(f"latent forward T{T}", C.check(y, want, G.tol_for(T, "bf16")))


# ---------------------------------------------------------------- caller streams


def test_calls_on_a_side_stream():
    """Calls on a stream other than torch's current one: the binding allocates
    its outputs and workspace for that stream, so allocations made right after
    on the current stream cannot take their memory while the kernels run."""
    shape = synth.LayerShape("side", 2048, 3072, 1024)
    dev, ref, _ = G.latent_layer(G.tiny_config("side"), shape)
    side = torch.cuda.Stream()
    for T in (1, 40):
        x_np = synth.activations(f"side/x/{T}", T, shape.d_in, "bf16")
        x = G.to_device_x(x_np, "bf16")
        side.wait_stream(torch.cuda.current_stream())
        y = nq.lrb_linear(dev, x, stream=side)
        g_np = synth.activations(f"side/g/{T}", T, shape.d_out, "bf16")
        g = G.to_device_x(g_np, "bf16")
        side.wait_stream(torch.cuda.current_stream())
        dx, ds1, ds2 = nq.lrb_scale_grads(dev, nq.Adjoint.of(dev, stream=side), x, g, stream=side)
        # churn the allocator on the current stream while the side stream runs
        junk = [torch.full((1 << 20,), 3.0, device=G.DEV) for _ in range(16)]
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        del junk
        _report(f"side stream linear T{T}", C.full_check(y.cpu().numpy(), ref, x_np, G.tol_for(T, "bf16"), "bf16"))
        for nm, got, want in zip(("dx", "ds1", "ds2"), (dx, ds1, ds2), O.scale_grads_factored_ref(ref, x_np, g_np)):
            w = want if want.ndim == 2 else want[None, :]
            gg = got.cpu().numpy()
            _report(f"side stream {nm} T{T}", C.check(gg if gg.ndim == 2 else gg[None, :], w, G.tol_for(T, "bf16")))


def test_layer_struct_validation():
    """Mis-sized or mistyped layer tensors are refused before any launch."""
    shape = synth.LayerShape("val", 100, 70, 40)
    good, _, _ = G.latent_layer(G.tiny_config("val"), shape)
    good.struct()
    bad = [
        dict(u_bits=good.u_bits[:1]),                     # too few word rows (needs ceil(40/32) = 2)
        dict(vt_bits=good.vt_bits[:, :39]),               # row stride below r
        dict(s1=good.s1[:99]),                            # s1 shorter than d_out
        dict(s2=good.s2.double()),                        # not fp32
        dict(u_bits=good.u_bits.float()),                 # not 32-bit words
        dict(vt_bits=good.vt_bits.cpu()),                 # not on the device
    ]
    for kw in bad:
        L = nq.Lrb(good.d_out, good.d_in, good.r, kw.get("u_bits", good.u_bits), kw.get("vt_bits", good.vt_bits),
                   kw.get("s1", good.s1), kw.get("s2", good.s2))
        with pytest.raises(ValueError):
            L.struct()
        with pytest.raises(ValueError):
            nq.lrb_linear(L, torch.zeros((1, shape.d_in), dtype=torch.bfloat16, device=G.DEV))
    # the checked struct is kept between calls; assigning a field checks again
    x = torch.zeros((1, shape.d_in), dtype=torch.bfloat16, device=G.DEV)
    nq.lrb_linear(good, x)
    s1 = good.s1
    good.s1 = s1[:99]
    with pytest.raises(ValueError):
        nq.lrb_linear(good, x)
    good.s1 = s1
    nq.lrb_linear(good, x)
    torch.cuda.synchronize()
