"""GPU parity: libnq (through its C ABI) against the CPU oracle on the same
seeded inputs.  Packing, the pack/unpack round trip, the word layout and the
dense reconstruction are bit-exact; nq_lrb_linear is within the normwise
relative-error bar (2e-3 for bf16 activations in the matrix-core regime,
1e-5 for fp32 arithmetic)."""
import os

import numpy as np
import pytest
import torch

import synth
from oracle import nq_oracle as O
from tests import checks as C
from tests import gpu_cases as G
from tests.conftest import GOLDEN

pytestmark = pytest.mark.gpu

nq = pytest.importorskip("sub_bit_weight_amd")

TINY = [  # (d_out, d_in, r): odd sizes, single elements, ragged words
    (1, 1, 1), (3, 5, 2), (33, 47, 5), (7, 1, 1), (1, 40, 33), (65, 129, 31), (100, 37, 64),
]


# ---------------------------------------------------------------- generator


@pytest.mark.parametrize("n,seed", [(1, 0), (1000, 1234567), ((1 << 20) + 13, 0xDEADBEEFCAFEF00D)])
def test_fill_words_matches_host_splitmix(n, seed):
    got = G.words_to_host(nq.fill_random_words(n, seed, G.DEV))
    assert np.array_equal(got, synth.random_words(seed, np.arange(n, dtype=np.uint64)))


# ---------------------------------------------------------------- packing


# the last case has more outputs than one launch's grid covers (more than
# 65535 x 16), so workgroups take a second group of outputs
@pytest.mark.parametrize("n_out,n_red,ld_pad", [(1, 1, 0), (5, 31, 3), (64, 64, 0), (33, 100, 1), (65, 129, 2),
                                                (68, 77, 0), (128, 1000, 3), (256, 256, 0), (300, 1000, 5), (4096, 2048, 0), (1_048_600, 3, 1)])
def test_pack_bit_exact(n_out, n_red, ld_pad):
    M = synth.normal_f32(f"pack/{n_out}/{n_red}", (n_out, n_red))
    ref = O.pack_ref(M)
    dev = torch.from_numpy(M).to(G.DEV)
    words = nq.pack_signs(dev, n_out, n_red, n_red, 1, ld=n_out + ld_pad)
    got = G.words_to_host(words)
    assert np.array_equal(got[:, :n_out], ref)
    assert not got[:, n_out:].any()  # columns past n_out untouched (zero-initialised)
    # the transposed source (V latent: stride_out = 1, stride_red = n_out)
    Mt = np.ascontiguousarray(M.T)
    words_t = nq.pack_signs(torch.from_numpy(Mt).to(G.DEV), n_out, n_red, 1, n_out)
    assert np.array_equal(G.words_to_host(words_t), ref)


def test_pack_special_values():
    vals = np.array([[0.0, -0.0, np.nan, -np.inf, np.inf, -1e-45, 1e-45, -1.0, 3.0] * 4], dtype=np.float32)
    words = nq.pack_signs(torch.from_numpy(vals).to(G.DEV), 1, vals.shape[1], vals.shape[1], 1)
    assert np.array_equal(G.words_to_host(words), O.pack_ref(vals))


@pytest.mark.parametrize("n_out,n_red", [(1, 1), (17, 45), (64, 96), (130, 257)])
def test_unpack_round_trip(n_out, n_red):
    M = synth.normal_f32(f"rt/{n_out}/{n_red}", (n_out, n_red))
    words = nq.pack_signs(torch.from_numpy(M).to(G.DEV), n_out, n_red, n_red, 1)
    S = nq.unpack_signs(words, n_out, n_red).cpu().numpy()
    assert np.array_equal(S, np.where(M < 0, -1.0, 1.0).astype(np.float32))
    assert np.array_equal(S.astype(np.float64), O.unpack_ref(G.words_to_host(words), n_red))


# ---------------------------------------------------------------- reconstruct


@pytest.mark.parametrize("shape", TINY + [(256, 256, 64), (96, 64, 1100)])
def test_reconstruct_bit_exact(shape):
    d_out, d_in, r = shape
    cfg = G.tiny_config(f"rec/{d_out}/{d_in}/{r}", scale_kind="lognormal")
    dev, ref, _ = G.latent_layer(cfg, synth.LayerShape("w", d_out, d_in, r), ld_pad=(3 if d_out > 50 else 0))
    W = nq.reconstruct(dev).cpu().numpy()
    expect = O.reconstruct_expected_f32(ref)
    assert np.array_equal(W.view(np.uint32), expect.view(np.uint32))


# ---------------------------------------------------------------- linear


def _linear_err(dev, ref, x_np, x_dtype, factored=False):
    """Normwise error of nq_lrb_linear against the oracle; the per-token,
    elementwise and deterministic bars of tests/checks.py must hold too."""
    y = nq.lrb_linear(dev, G.to_device_x(x_np, x_dtype)).cpu().numpy()
    assert np.all(np.isfinite(y))
    e = C.full_check(y, ref, x_np, G.tol_for(x_np.shape[0], x_dtype), x_dtype, factored)
    assert e["pass"], e
    return e["normwise"]


def test_config_single_lrb_fp32():
    cfg = synth.CONFIGS["single"]
    dev, ref, _ = G.latent_layer(cfg, cfg.layers[0])
    x = synth.x_for(cfg, 256, 1)
    err = _linear_err(dev, ref, x, "f32")
    print(f"single 256x256 r64 T1 fp32: rel err {err:.3e}")
    assert err <= 1e-5


def test_config_7b_attention():
    cfg = synth.CONFIGS["7b_attn"]
    dev, ref, _ = G.latent_layer(cfg, cfg.layers[0])
    x = synth.x_for(cfg, 4096, 1)
    err = _linear_err(dev, ref, x, "bf16")
    print(f"7b attn 4096x4096 r2048 T1: rel err {err:.3e}")
    assert err <= 2e-3
    assert err <= 1e-5  # decode arithmetic is fp32 throughout


@pytest.mark.parametrize("T", [1, 8])
def test_config_7b_mlp(T):
    cfg = synth.CONFIGS["7b_mlp"]
    for shape in cfg.layers:
        dev, ref, _ = G.latent_layer(cfg, shape)
        x = synth.x_for(cfg, shape.d_in, T)
        err = _linear_err(dev, ref, x, "bf16", factored=True)
        print(f"7b mlp {shape.name} {shape.d_out}x{shape.d_in} r{shape.r} T{T}: rel err {err:.3e}")
        assert err <= 1e-5


@pytest.mark.parametrize("x_dtype", ["bf16", "f32"])
@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 6, 7, 8, 9, 16, 63, 64, 65, 130])
def test_linear_token_sweep(T, x_dtype):
    shape = synth.LayerShape("sweep", 160, 200, 70)
    cfg = G.tiny_config(f"sweep/{x_dtype}", x_dtype=x_dtype)
    dev, ref, _ = G.latent_layer(cfg, shape, ld_pad=2)
    x = synth.activations(f"sweep/x/{T}/{x_dtype}", T, shape.d_in, x_dtype)
    err = _linear_err(dev, ref, x, x_dtype)
    assert err <= G.tol_for(T, x_dtype), err


@pytest.mark.parametrize("T", [1, 3, 9, 40])
@pytest.mark.parametrize("shape", TINY)
def test_linear_tiny_shapes(shape, T):
    d_out, d_in, r = shape
    cfg = G.tiny_config(f"tiny/{d_out}/{d_in}/{r}")
    dev, ref, _ = G.latent_layer(cfg, synth.LayerShape("w", d_out, d_in, r))
    x = synth.activations(f"tiny/x/{shape}/{T}", T, d_in, "bf16")
    err = _linear_err(dev, ref, x, "bf16")
    assert err <= G.tol_for(T, "bf16"), err


def test_linear_deterministic():
    shape = synth.LayerShape("det", 1024, 768, 256)
    dev, _, _ = G.latent_layer(G.tiny_config("det"), shape)
    for T in (1, 4, 100):
        x = G.to_device_x(synth.activations(f"det/x/{T}", T, shape.d_in, "bf16"), "bf16")
        y1 = nq.lrb_linear(dev, x).cpu()
        y2 = nq.lrb_linear(dev, x).cpu()
        assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))


def test_single_calls_on_two_streams_and_counter_fallback():
    """Single decode calls keep their dependency counters in a library slot per
    stream.  Calls on two streams at once, and layers with different counter
    counts one after another on each stream, give what the same calls give one
    at a time (bit for bit); a layer with more counters than a slot holds (1025
    stage-2 row blocks) keeps them in its workspace; all match the oracle."""
    cfg = G.tiny_config("slots")
    shapes = [synth.LayerShape("a", 1100, 2100, 300), synth.LayerShape("b", 4096, 1024, 1500)]
    layers = [G.latent_layer(cfg, s) for s in shapes]
    Ts = (1, 5)
    xs = {(T, i): synth.activations(f"slots/x/{s.name}/{T}", T, s.d_in, "bf16")
          for T in Ts for i, s in enumerate(shapes)}
    xd = {k: G.to_device_x(v, "bf16") for k, v in xs.items()}
    one_at_a_time = {}
    for (T, i), x in xd.items():
        one_at_a_time[T, i] = nq.lrb_linear(layers[i][0], x).cpu()
        torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]  # default priority
    outs = []
    for _ in range(20):
        for T, st in zip(Ts, streams):
            for i in range(len(shapes)):
                outs.append(((T, i), nq.lrb_linear(layers[i][0], xd[T, i], stream=st)))
    torch.cuda.synchronize()
    for key, y in outs:
        assert torch.equal(y.cpu().view(torch.int32), one_at_a_time[key].view(torch.int32)), key
    for (T, i), y in one_at_a_time.items():
        e = C.full_check(y.numpy(), layers[i][1], xs[T, i], G.decode_tol("bf16"), "bf16")
        assert e["pass"], ((T, i), e)
    big = synth.LayerShape("big", 524_800, 40, 33)
    dev, ref = G.splitmix_layer(synth.Config("slots/big", "slots/big", [], (1,), "bf16", words="splitmix"), big)
    for T in (2, 1):
        x = synth.activations(f"slots/big/x/{T}", T, big.d_in, "bf16")
        err = _linear_err(dev, ref, x, "bf16")
        assert err <= G.decode_tol("bf16"), err


def test_single_call_graph_replays():
    """A decode-regime single call captured into a graph (one kernel: its
    counters live in the capture stream's slot, no clearing launch) gives, on
    every replay, what an eager call gives on the same input, with eager calls
    on the default stream between the replays."""
    shape = synth.LayerShape("graph", 1100, 2100, 300)
    dev, ref, _ = G.latent_layer(G.tiny_config("graph"), shape)
    T = 3
    xs = [synth.activations(f"graph/x/{i}", T, shape.d_in, "bf16") for i in range(5)]
    x = G.to_device_x(xs[0], "bf16")
    y = torch.empty((T, shape.d_out), device=G.DEV)
    ws = torch.empty(nq.lrb_workspace_bytes(dev, T), dtype=torch.uint8, device=G.DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture
        nq.lrb_linear(dev, x, y, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        nq.lrb_linear(dev, x, y, ws)
    for i, x_np in enumerate(xs):
        x.copy_(G.to_device_x(x_np, "bf16"))
        g.replay()
        torch.cuda.synchronize()
        got = y.clone()
        eager = nq.lrb_linear(dev, G.to_device_x(x_np, "bf16"))
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int32), eager.view(torch.int32)), i
        e = C.full_check(got.cpu().numpy(), ref, x_np, G.decode_tol("bf16"), "bf16")
        assert e["pass"], (i, e)


TINY_PATH = [(256, 256, 64), (70, 100, 40), (1024, 2048, 512), (33, 1, 1), (1, 64, 33), (257, 96, 31)]


@pytest.mark.parametrize("x_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", TINY_PATH)
def test_tiny_path(shape, x_dtype, monkeypatch):
    """Small layers at T <= 8 run in one workgroup (z, t, y as fp32 sums in
    index order): against the oracle at every T the path takes, with padded
    words, and against the multi-workgroup decode kernels on the same inputs."""
    d_out, d_in, r = shape
    cfg = G.tiny_config(f"tinypath/{shape}/{x_dtype}", x_dtype=x_dtype)
    dev, ref, _ = G.latent_layer(cfg, synth.LayerShape("tp", d_out, d_in, r), ld_pad=3)
    ran = 0
    for T in range(1, 9):
        w32 = lambda n: -(-n // 32) * 32
        if not (T * w32(d_in) <= 2048 and T * w32(r) <= 512 and d_out <= 1024):
            continue
        x = synth.activations(f"tinypath/x/{shape}/{T}/{x_dtype}", T, d_in, x_dtype)
        err = _linear_err(dev, ref, x, x_dtype)
        assert err <= 1e-5, (T, err)
        y_tiny = nq.lrb_linear(dev, G.to_device_x(x, x_dtype)).cpu().numpy()
        monkeypatch.setenv("NQ_DECODE_TINY", "0")
        y_dec = nq.lrb_linear(dev, G.to_device_x(x, x_dtype)).cpu().numpy()
        monkeypatch.delenv("NQ_DECODE_TINY")
        assert C.errors(y_tiny, y_dec)["normwise"] <= 2e-5, T
        ran += 1
    assert ran >= 1


@pytest.mark.parametrize("T", [1, 2, 5, 8])
def test_decode_xor_variant(T, monkeypatch):
    """The per-weight sign-XOR decode kernels (kept for comparison) also match the oracle."""
    monkeypatch.setenv("NQ_DECODE_VARIANT", "xor")
    shape = synth.LayerShape("xor", 300, 200, 70)
    dev, ref, _ = G.latent_layer(G.tiny_config("xor"), shape, ld_pad=1)
    x = synth.activations(f"xor/x/{T}", T, shape.d_in, "bf16")
    assert _linear_err(dev, ref, x, "bf16") <= 1e-5


def test_sequence_matches_single_calls(monkeypatch):
    # single calls of these small layers would take the one-workgroup path;
    # the sequence runs the decode kernels, which single calls then match bit
    # for bit
    monkeypatch.setenv("NQ_DECODE_TINY", "0")
    cfg = G.tiny_config("seq")
    shapes = [synth.LayerShape("a", 300, 200, 64), synth.LayerShape("b", 96, 300, 40),
              synth.LayerShape("c", 200, 96, 33)]
    layers = [G.latent_layer(cfg, s, i)[0] for i, s in enumerate(shapes)]
    for T in (1, 8, 33):
        xs = [G.to_device_x(synth.activations(f"seq/x/{T}/{i}", T, s.d_in, "bf16"), "bf16")
              for i, s in enumerate(shapes)]
        ys = [torch.full((T, s.d_out), float("nan"), device=G.DEV) for s in shapes]
        seq = nq.Seq(layers, xs, ys)
        seq.run()
        seq.run()  # a second run reuses the uploaded schedule
        assert seq.device_error() == 0
        for L, x, y in zip(layers, xs, ys):
            assert torch.equal(y.view(torch.int32), nq.lrb_linear(L, x).view(torch.int32))
        seq.close()


def test_sequence_prefill_streams():
    # more entries than the plan's streams, shapes with and without split
    # reductions; inputs written and outputs read on the caller's stream right
    # before and after the run (the plan forks from and joins back to it)
    cfg = G.tiny_config("seqpf")
    shapes = [synth.LayerShape("a", 300, 200, 64), synth.LayerShape("b", 700, 800, 600),
              synth.LayerShape("c", 200, 96, 33), synth.LayerShape("d", 1024, 768, 256),
              synth.LayerShape("e", 96, 300, 40), synth.LayerShape("f", 512, 1024, 256),
              synth.LayerShape("g", 65, 129, 31)]
    built = [G.latent_layer(cfg, s, i) for i, s in enumerate(shapes)]
    T = 100
    x_np = [synth.activations(f"seqpf/x/{i}", T, s.d_in, "bf16") for i, s in enumerate(shapes)]
    src = [G.to_device_x(x, "bf16") for x in x_np]
    xs = [torch.zeros_like(x) for x in src]
    ys = [torch.full((T, s.d_out), float("nan"), device=G.DEV) for s in shapes]
    seq = nq.Seq([b[0] for b in built], xs, ys)
    first = None
    for rep in range(2):
        for x, x0 in zip(xs, src):
            x.copy_(x0 * (rep + 1))  # exact in bf16
        seq.run()
        got = [y.clone() for y in ys]
        torch.cuda.synchronize()
        for (dev, ref, _), x, g in zip(built, x_np, got):
            e = C.full_check(g.cpu().numpy(), ref, x * (rep + 1), G.tol_for(T, "bf16"), "bf16")
            assert e["pass"], e
        if rep == 0:
            first = got
    # run-to-run determinism of the plan (inputs doubled: outputs exactly doubled)
    for a, b in zip(first, got):
        assert torch.equal((a * 2).view(torch.int32), b.view(torch.int32))
    seq.close()


@pytest.mark.parametrize("T", [1, 3, 8])
def test_sequence_many_linears_parity(T):
    """A persistent schedule over many linears of mixed shapes (ragged row blocks,
    several reduction chunks) matches the oracle on every entry."""
    cfg = G.tiny_config(f"seqmany/{T}")
    shapes = [synth.LayerShape(f"m{i}", d_out, d_in, r) for i, (d_out, d_in, r) in enumerate(
        [(1000, 3000, 300), (64, 5000, 1100), (700, 33, 9), (257, 2500, 2100), (3, 3, 3), (1500, 700, 640)])]
    built = [G.latent_layer(cfg, s, i) for i, s in enumerate(shapes)]
    xs_np = [synth.activations(f"seqmany/x/{T}/{i}", T, s.d_in, "bf16") for i, s in enumerate(shapes)]
    xs = [G.to_device_x(x, "bf16") for x in xs_np]
    ys = [torch.full((T, s.d_out), float("nan"), device=G.DEV) for s in shapes]
    seq = nq.Seq([b[0] for b in built], xs, ys)
    for _ in range(3):
        seq.run()
    assert seq.device_error() == 0
    for (dev, ref, _), x, y in zip(built, xs_np, ys):
        assert O.rel_err(y.cpu().numpy(), O.linear_ref(ref, x)) <= 1e-5
    seq.close()


# ---------------------------------------------------------------- 70B shapes (sampled rows)


def _sampled_err(dev, ref, x_np, rows, x_dtype="bf16"):
    """Normwise error on sampled output rows (all tokens); the per-token,
    elementwise and deterministic bars must hold too."""
    y = nq.lrb_linear(dev, G.to_device_x(x_np, x_dtype)).cpu().numpy()
    assert np.all(np.isfinite(y))
    e = C.sampled_check(y[:, rows], ref, x_np, rows, G.tol_for(x_np.shape[0], x_dtype), x_dtype)
    print(f"  per-token max {e['per_token_max']:.2e}, elementwise/rms max {e['elem_rms_max']:.2e}, "
          f"bound ratio {e['bound_ratio_max']:.2e}")
    assert e["pass"], e
    return e["normwise"]


@pytest.mark.parametrize("name", ["k", "down"])
def test_70b_decode_sampled_rows(name):
    cfg = synth.CONFIGS["70b_stack"]
    shape = next(s for s in cfg.layers if s.name == name)
    dev, ref = G.splitmix_layer(cfg, shape, layer_idx=0)
    rows = np.sort(synth.rng(f"rows/{name}").choice(shape.d_out, 64, replace=False))
    x = synth.x_for(cfg, shape.d_in, 1)
    err = _sampled_err(dev, ref, x, rows)
    print(f"70b {name} T1 sampled 64 rows: rel err {err:.3e}")
    assert err <= 1e-5


# q: 256 output tiles (reduction split in two); k: few tiles (split eight ways in
# stage 1, two in stage 2); down: no split; q with fp32 x: two fp16 terms.
@pytest.mark.parametrize("name,x_dtype", [("q", "bf16"), ("k", "bf16"), ("down", "bf16"), ("q", "f32")])
def test_70b_prefill_sampled_rows(name, x_dtype):
    cfg = synth.CONFIGS["70b_prefill"]
    shape = next(s for s in cfg.layers if s.name == name)
    dev, ref = G.splitmix_layer(cfg, shape, layer_idx=0)
    rows = np.sort(synth.rng(f"rows/prefill/{name}").choice(shape.d_out, 64, replace=False))
    if x_dtype == "bf16":
        x = synth.x_for(cfg, shape.d_in, 2048)
    else:  # full fp32 mantissas, same distribution
        x = synth.activations(f"{cfg.key}/x32/{shape.d_in}/2048", 2048, shape.d_in, "f32", cfg.outlier_frac)
    err = _sampled_err(dev, ref, x, rows, x_dtype)
    print(f"70b {name} T2048 {x_dtype} sampled 64 rows: rel err {err:.3e}")
    assert err <= G.tol_for(2048, x_dtype)


# Reduction lengths that split unevenly: stage 1 has 13 tiles of 64 (pieces of
# 7 and 6), stage 2 has 10 (two pieces of 5); rows and outputs ragged too.
@pytest.mark.parametrize("x_dtype", ["bf16", "f32"])
def test_linear_uneven_split(x_dtype):
    shape = synth.LayerShape("split", 700, 800, 600)
    cfg = G.tiny_config(f"split/{x_dtype}", x_dtype=x_dtype)
    dev, ref, _ = G.latent_layer(cfg, shape)
    x = synth.activations(f"split/x/{x_dtype}", 200, shape.d_in, x_dtype)
    err = _linear_err(dev, ref, x, x_dtype)
    print(f"uneven split {x_dtype}: rel err {err:.3e}")
    assert err <= G.tol_for(200, x_dtype), err


# All-positive activations with a large mean: the matrix-core path's rotated
# operand encoding leaves a per-row correction sum that is then large next to
# the result (it must cancel exactly up to fp32 rounding).
@pytest.mark.parametrize("x_dtype", ["bf16", "f32"])
def test_linear_biased_inputs(x_dtype):
    shape = synth.LayerShape("biased", 512, 1024, 256)
    cfg = G.tiny_config(f"biased/{x_dtype}", x_dtype=x_dtype)
    dev, ref, _ = G.latent_layer(cfg, shape)
    x = np.abs(synth.activations(f"biased/x/{x_dtype}", 100, shape.d_in, "f32")) + np.float32(4.0)
    if x_dtype == "bf16":
        x = synth.round_bf16(x)
    err = _linear_err(dev, ref, x, x_dtype)
    print(f"biased inputs {x_dtype}: rel err {err:.3e}")
    assert err <= G.tol_for(100, x_dtype), err


# Decode on the matrix cores cuts each input into fp8 pieces per 1024-element
# chunk, scaled by the chunk's largest value; these cases stress that: strong
# outliers (wide dynamic range inside one group of 8 products), magnitudes
# spread over many binades, tiny and huge overall scales, all-zero chunks
# next to non-zero ones, and all-positive inputs.
def _decode_inputs(kind: str, T: int, d: int, x_dtype: str) -> np.ndarray:
    tag = f"decode-edge/{kind}/{T}/{d}/{x_dtype}"
    if kind == "outliers":
        x = synth.activations(tag, T, d, "f32", outlier_frac=0.01, outlier_mag=3.0e3)
    elif kind == "spread":  # |x| log-uniform over 2^-40 .. 2^10
        g = synth.rng(tag)
        x = (np.exp2(g.uniform(-40.0, 10.0, (T, d))) * np.where(g.random((T, d)) < 0.5, -1.0, 1.0)).astype(np.float32)
    elif kind == "tiny":
        x = synth.activations(tag, T, d, "f32") * np.float32(1e-20)
    elif kind == "huge":
        x = synth.activations(tag, T, d, "f32") * np.float32(1e12)
    elif kind == "zero_chunks":  # every other 1024-element chunk is zero
        x = synth.activations(tag, T, d, "f32")
        for c in range(0, d, 2048):
            x[:, c:c + 1024] = 0.0
    elif kind == "biased":
        x = np.abs(synth.activations(tag, T, d, "f32")) + np.float32(4.0)
    else:
        raise ValueError(kind)
    return synth.round_bf16(x) if x_dtype == "bf16" else x.astype(np.float32)


@pytest.mark.parametrize("kind", ["outliers", "spread", "tiny", "huge", "zero_chunks", "biased"])
# T = 4 and 7: a token's pieces straddle two MFMA column groups
@pytest.mark.parametrize("T,x_dtype", [(1, "bf16"), (1, "f32"), (2, "f32"), (4, "f32"), (7, "f32"), (8, "bf16")])
def test_decode_input_ranges(kind, T, x_dtype):
    shape = synth.LayerShape("ranges", 320, 4096, 1088)  # ragged rows and rank, 4 chunks of x, 2 of t
    cfg = G.tiny_config(f"ranges/{x_dtype}", x_dtype=x_dtype)
    dev, ref, _ = G.latent_layer(cfg, shape)
    x = _decode_inputs(kind, T, shape.d_in, x_dtype)
    err = _linear_err(dev, ref, x, x_dtype, factored=True)
    print(f"decode {kind} T{T} {x_dtype}: rel err {err:.3e}")
    assert err <= 1e-5, err


def test_decode_all_zero_input():
    shape = synth.LayerShape("zeros", 200, 3000, 300)
    cfg = G.tiny_config("zeros")
    dev, ref, _ = G.latent_layer(cfg, shape)
    y = nq.lrb_linear(dev, G.to_device_x(np.zeros((1, shape.d_in), np.float32), "bf16")).cpu().numpy()
    assert np.all(y == 0.0)


@pytest.mark.parametrize("bad", [np.nan, np.inf])
@pytest.mark.parametrize("T", [1, 6])
def test_decode_non_finite_input(bad, T):
    # one non-finite element of the last token reaches every output of that
    # token: the oracle's sums are NaN or +-inf; the decode result must not be
    # finite anywhere in that token, and the other tokens stay exact
    shape = synth.LayerShape("nonfinite", 256, 2048, 256)
    cfg = G.tiny_config("nonfinite")
    dev, ref, _ = G.latent_layer(cfg, shape)
    x = synth.activations("nonfinite/x", T, shape.d_in, "f32")
    x[T - 1, 1500] = bad
    y = nq.lrb_linear(dev, G.to_device_x(x, "f32")).cpu().numpy()
    y_ref = O.linear_factored_ref(ref, x)
    assert not np.any(np.isfinite(y_ref[T - 1]))
    assert not np.any(np.isfinite(y[T - 1]))
    if T > 1:
        assert O.rel_err(y[: T - 1], y_ref[: T - 1]) <= 1e-5


# ---------------------------------------------------------------- scale-only reconstruction


@pytest.mark.parametrize("n_out,n_red,ld_pad,ldt_pad", [(1, 1, 0, 0), (33, 70, 3, 1), (64, 32, 0, 0),
                                                        (100, 257, 5, 7), (512, 96, 0, 0), (31, 1000, 0, 2)])
def test_transpose_signs_bit_exact(n_out, n_red, ld_pad, ldt_pad):
    nw = nq.n_words(n_red)
    ld = n_out + ld_pad
    words = nq.fill_random_words(nw * ld, 77 + n_out, G.DEV).view(nw, ld)
    host = synth.random_words(77 + n_out, np.arange(nw * ld, dtype=np.uint64)).reshape(nw, ld)
    # the source's padding bits (past n_red) must be 0: clear them on both sides
    if n_red % 32:
        keep = np.uint32((1 << (n_red % 32)) - 1)
        host[-1] &= keep
        words[-1] &= int(np.array(keep).view(np.int32))
    out = torch.full((nq.n_words(n_out), n_red + ldt_pad), -1, dtype=torch.int32, device=G.DEV)
    nq.transpose_signs(words, n_out, n_red, ld=ld, out=out)
    got = G.words_to_host(out)
    want = O.transpose_bits_ref(host, n_out, n_red)
    np.testing.assert_array_equal(got[:, :n_red], want)
    assert np.all(got[:, n_red:] == np.uint32(0xFFFFFFFF))  # columns past n_red are not written


GRAD_SHAPES = [(33, 47, 5), (65, 129, 31), (100, 37, 64), (256, 320, 96)]


@pytest.mark.parametrize("shape", GRAD_SHAPES)
@pytest.mark.parametrize("T,x_dtype,g_dtype", [(1, "bf16", "f32"), (3, "f32", "f32"), (8, "bf16", "f32"),
                                               (9, "f32", "f32"), (64, "bf16", "f32"), (130, "f32", "f32"),
                                               (2, "f32", "bf16"), (96, "bf16", "bf16")])
def test_scale_grads_parity(shape, T, x_dtype, g_dtype):
    d_out, d_in, r = shape
    cfg = G.tiny_config(f"grads/{x_dtype}", x_dtype=x_dtype)
    dev, ref, _ = G.latent_layer(cfg, synth.LayerShape("grads", d_out, d_in, r))
    x = synth.activations(f"grads/x/{d_in}/{T}", T, d_in, x_dtype)
    g = synth.activations(f"grads/g/{d_out}/{T}", T, d_out, g_dtype)
    adj = nq.Adjoint.of(dev)
    dx, ds1, ds2 = nq.lrb_scale_grads(dev, adj, G.to_device_x(x, x_dtype), G.to_device_x(g, g_dtype))
    rdx, rds1, rds2 = O.scale_grads_factored_ref(ref, x, g)
    # dx and ds2 come from the transposed product of g, ds1 from the forward
    # product of x: each meets the bar of its own input's dtype and regime
    e = [O.rel_err(dx.cpu().numpy(), rdx), O.rel_err(ds1.cpu().numpy(), rds1), O.rel_err(ds2.cpu().numpy(), rds2)]
    print(f"grads {shape} T{T} x {x_dtype} g {g_dtype}: dx {e[0]:.2e} ds1 {e[1]:.2e} ds2 {e[2]:.2e}")
    assert e[0] <= G.tol_for(T, g_dtype) and e[2] <= G.tol_for(T, g_dtype)
    assert e[1] <= G.tol_for(T, x_dtype)


def test_scale_grads_padded_words_and_workspace_reuse():
    """Adjoint words with row padding, a shared workspace over two calls of
    different T, and the decode and GEMM regimes back to back."""
    shape = synth.LayerShape("gradspad", 96, 200, 40)
    cfg = G.tiny_config("gradspad", x_dtype="f32")
    dev, ref, _ = G.latent_layer(cfg, shape, ld_pad=3)
    ut = nq.transpose_signs(dev.u_bits, shape.d_out, shape.r,
                            out=torch.empty((nq.n_words(shape.d_out), shape.r + 5), dtype=torch.int32, device=G.DEV))
    v = nq.transpose_signs(dev.vt_bits, shape.r, shape.d_in,
                           out=torch.empty((nq.n_words(shape.r), shape.d_in + 2), dtype=torch.int32, device=G.DEV))
    adj = nq.Adjoint(ut, v)
    ws = torch.empty(nq.lrb_scale_grads_workspace_bytes(dev, 40), dtype=torch.uint8, device=G.DEV)
    for T in (40, 2):
        x = synth.activations(f"gradspad/x/{T}", T, shape.d_in, "f32")
        g = synth.activations(f"gradspad/g/{T}", T, shape.d_out, "f32")
        dx, ds1, ds2 = nq.lrb_scale_grads(dev, adj, G.to_device_x(x, "f32"), torch.from_numpy(g).to(G.DEV),
                                          workspace=ws)
        for got, want in zip((dx, ds1, ds2), O.scale_grads_factored_ref(ref, x, g)):
            assert O.rel_err(got.cpu().numpy(), want) <= 1e-5


def test_scale_grads_many_token_chunks():
    """T past the largest chunk count: the chunk length grows (66000 tokens
    in chunks of 65) and the last chunk is short."""
    shape = synth.LayerShape("gradslong", 33, 47, 5)
    cfg = G.tiny_config("gradslong", x_dtype="bf16")
    dev, ref, _ = G.latent_layer(cfg, shape)
    T = 66000
    x = synth.activations("gradslong/x", T, shape.d_in, "bf16")
    g = synth.activations("gradslong/g", T, shape.d_out, "bf16")
    dx, ds1, ds2 = nq.lrb_scale_grads(dev, nq.Adjoint.of(dev), G.to_device_x(x, "bf16"), G.to_device_x(g, "bf16"))
    for got, want in zip((dx, ds1, ds2), O.scale_grads_factored_ref(ref, x, g)):
        assert O.rel_err(got.cpu().numpy(), want) <= G.prefill_tol("bf16")


@pytest.mark.parametrize("T", [4, 200])
def test_scale_grads_batch_matches_single_calls(T):
    """nq_lrb_scale_grads_batch equals one nq_lrb_scale_grads call per linear bit
    for bit (decode regime: the calls in order; matrix-core regime: the product
    chains on the library's streams, with split reductions among them), and the
    factored oracle."""
    cfg = G.tiny_config(f"gbatch/{T}")
    shapes = [synth.LayerShape("a", 300, 200, 64), synth.LayerShape("b", 96, 300, 40),
              synth.LayerShape("c", 640, 512, 96), synth.LayerShape("d", 200, 96, 33)]
    built = [G.latent_layer(cfg, s, i) for i, s in enumerate(shapes)]
    layers = [b[0] for b in built]
    adjs = [nq.Adjoint.of(L) for L in layers]
    x_np = [synth.activations(f"gbatch/x/{T}/{i}", T, s.d_in, "bf16") for i, s in enumerate(shapes)]
    g_np = [synth.activations(f"gbatch/g/{T}/{i}", T, s.d_out, "bf16") for i, s in enumerate(shapes)]
    xs = [G.to_device_x(x, "bf16") for x in x_np]
    gs = [G.to_device_x(g, "bf16") for g in g_np]
    outs = nq.lrb_scale_grads_batch(layers, adjs, xs, gs)
    for i, (L, a, x, g) in enumerate(zip(layers, adjs, xs, gs)):
        want = nq.lrb_scale_grads(L, a, x, g)
        for nm, got, w in zip(("dx", "ds1", "ds2"), outs[i], want):
            assert torch.equal(got.view(torch.int32), w.view(torch.int32)), (i, nm)
    for i in range(len(shapes)):
        for got, want in zip(outs[i], O.scale_grads_factored_ref(built[i][1], x_np[i], g_np[i])):
            assert O.rel_err(got.cpu().numpy(), want) <= G.tol_for(T, "bf16"), i


# ---- magnitude balancing and scale extraction --------------------------------

# (d_out, d_in, r, row padding): the row stride r + pad decides between the
# float4 path (stride a multiple of 4) and the one-float path
BAL_CASES = [(1, 1, 1, 0), (2, 3, 2, 0), (37, 53, 11, 0), (64, 96, 64, 0), (300, 129, 257, 0),
             (33, 65, 100, 3), (40, 24, 61, 4), (130, 7, 1000, 0), (50, 70, 61, 3), (9, 5, 6, 2)]


@pytest.mark.parametrize("d_out,d_in,r,pad", BAL_CASES)
@pytest.mark.parametrize("mode", ["balanced", "scales", "inplace"])
def test_balance_parity(d_out, d_in, r, pad, mode):
    uh = np.full((d_out, r + pad), 1e6, np.float32)
    vh = np.full((d_in, r + pad), -1e6, np.float32)
    uh[:, :r] = synth.normal_f32(f"bal/u/{d_out}/{r}", (d_out, r)) * np.float32(0.02)
    vh[:, :r] = synth.normal_f32(f"bal/v/{d_in}/{r}", (d_in, r)) * np.float32(3.0)
    U0, V0, rs1, rs2, reta = O.balance_ref(uh[:, :r], vh[:, :r])
    du, dv = torch.from_numpy(uh).to(G.DEV), torch.from_numpy(vh).to(G.DEV)
    U, V, s1, s2, eta = nq.balance_factors(du, dv, r=r, balanced=mode != "scales", inplace=mode == "inplace")
    assert abs(float(eta.item()) / reta - 1) <= 1e-6
    assert O.rel_err(s1.cpu().numpy(), rs1) <= 1e-6 and O.rel_err(s2.cpu().numpy(), rs2) <= 1e-6
    if mode == "scales":
        assert U is None and V is None
        return
    if mode == "inplace":
        assert U is du and V is dv
    Uh, Vh = U.cpu().numpy(), V.cpu().numpy()
    assert O.rel_err(Uh[:, :r], U0) <= 1e-6 and O.rel_err(Vh[:, :r], V0) <= 1e-6
    # row padding (1e6 / -1e6) enters no sum (checked above) and is not written
    if mode == "inplace":
        assert np.all(Uh[:, r:] == np.float32(1e6)) and np.all(Vh[:, r:] == np.float32(-1e6))
    # eta > 0: the balanced factors pack to the same sign words
    a = nq.pack_signs(U, d_out, r, U.stride(0), 1)
    b = nq.pack_signs(torch.from_numpy(uh).to(G.DEV), d_out, r, r + pad, 1)
    assert torch.equal(a, b)


def test_balance_zero_factor_and_golden():
    """A zero factor (eta = 1 by the stated reading) and the hand-worked
    cases of tests/golden/balance_example.json through the library."""
    import json
    with open(os.path.join(GOLDEN, "balance_example.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        uh = torch.tensor(c["U_hat"], dtype=torch.float32, device=G.DEV)
        vh = torch.tensor(c["V_hat"], dtype=torch.float32, device=G.DEV)
        U, V, s1, s2, eta = nq.balance_factors(uh, vh)
        assert float(eta.item()) == pytest.approx(c["eta"], rel=1e-6)
        np.testing.assert_allclose(U.cpu().numpy(), c["U"], rtol=1e-6, atol=0)
        np.testing.assert_allclose(V.cpu().numpy(), c["V"], rtol=1e-6, atol=0)
        np.testing.assert_allclose(s1.cpu().numpy(), c["s1"], rtol=1e-6, atol=0)
        np.testing.assert_allclose(s2.cpu().numpy(), c["s2"], rtol=1e-6, atol=0)


def test_balance_llama_shape():
    """Latents of a 4096 x 11008 MLP projection at rank 2368, against the
    oracle on every element."""
    d_out, d_in, r = 11008, 4096, 2368
    uh = synth.normal_f32("bal/big/u", (d_out, r)) * np.float32(0.05)
    vh = synth.normal_f32("bal/big/v", (d_in, r)) * np.float32(2.0)
    U0, V0, rs1, rs2, reta = O.balance_ref(uh, vh)
    U, V, s1, s2, eta = nq.balance_factors(torch.from_numpy(uh).to(G.DEV), torch.from_numpy(vh).to(G.DEV))
    assert abs(float(eta.item()) / reta - 1) <= 1e-6
    for got, want in ((U, U0), (V, V0), (s1, rs1), (s2, rs2)):
        assert O.rel_err(got.cpu().numpy(), want) <= 1e-6


# ---- refinement forward from latent factors -----------------------------------

@pytest.mark.parametrize("shape", [(33, 47, 5), (100, 257, 64), (256, 320, 96)])
@pytest.mark.parametrize("T,x_dtype", [(1, "f32"), (5, "bf16"), (8, "f32"), (9, "bf16"), (64, "f32"), (130, "bf16")])
def test_linear_latent_parity(shape, T, x_dtype):
    """T > 8: bit-equal to nq_pack_signs + nq_lrb_linear; T <= 8 (signs taken
    as the latents load, fp32 throughout): within 1e-5 of the oracle, per
    token and element by element, and inside the deterministic bound of that
    arithmetic.  Latents with padded rows and +0, -0, NaN entries."""
    d_out, d_in, r = shape
    pad = 3
    Ul = np.full((d_out, r + pad), -7.0, np.float32)
    Vl = np.full((d_in, r + pad), -7.0, np.float32)
    Ul[:, :r] = synth.normal_f32(f"lat/u/{shape}", (d_out, r))
    Vl[:, :r] = synth.normal_f32(f"lat/v/{shape}", (d_in, r))
    Ul[0, :3] = [0.0, -0.0, np.nan]
    Vl[1, :3] = [np.nan, -0.0, 0.0]
    cfg = G.tiny_config(f"lat/{x_dtype}", x_dtype=x_dtype)
    s1 = synth.scales(cfg, f"lat/s1/{d_out}", d_out)
    s2 = synth.scales(cfg, f"lat/s2/{d_in}", d_in)
    x = synth.activations(f"lat/x/{d_in}/{T}", T, d_in, x_dtype)
    du, dv = torch.from_numpy(Ul).to(G.DEV), torch.from_numpy(Vl).to(G.DEV)
    ds1, ds2 = torch.from_numpy(s1).to(G.DEV), torch.from_numpy(s2).to(G.DEV)
    dx = G.to_device_x(x, x_dtype)
    y = nq.lrb_linear_latent(du, dv, ds1, ds2, dx, r=r)
    want = O.linear_latent_ref(Ul[:, :r], Vl[:, :r], s1, s2, x)
    if T > 8:
        # the packed route through the separate calls
        ub = nq.pack_signs(du, d_out, r, r + pad, 1)
        vb = nq.pack_signs(dv, r, d_in, 1, r + pad)
        layer = nq.Lrb(d_out, d_in, r, ub, vb, ds1, ds2)
        y2 = nq.lrb_linear(layer, dx)
        assert torch.equal(y, y2)
        assert O.rel_err(y.cpu().numpy(), want) <= G.tol_for(T, x_dtype)
        return
    A = C.latent_abs_terms(s1, s2, x, r)
    e = C.check(y.cpu().numpy(), want, 1e-5, A, C.gamma_latent(d_in, r), token_bars=min(d_in, r) >= 32)
    assert e["pass"], e


@pytest.mark.parametrize("shape,pad", [((64, 1500, 300), 0), ((40, 300, 4100), 0), ((24, 700, 4100), 1),
                                       ((3000, 64, 257), 4), ((50, 200, 258), 2)])
@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 6, 7, 8])
def test_linear_latent_sign_on_load(shape, pad, T):
    """The sign-on-load kernels (T <= 8) at every T, with reduction spans in
    both stages (stage 1: rows in spans of 64; stage 2: 4100 > one 2048-element
    span), ragged last column tiles, aligned rows (the float4 path, pad 0 or 4;
    with r = 258 and pad 2 the last float4 of a row takes two NaN padding
    entries, whose products are dropped) and unaligned ones (pad 1)."""
    d_out, d_in, r = shape
    Ul = np.full((d_out, r + pad), np.nan, np.float32)  # padding must not reach a sum
    Vl = np.full((d_in, r + pad), np.nan, np.float32)
    Ul[:, :r] = synth.normal_f32(f"lat2/u/{shape}", (d_out, r))
    Vl[:, :r] = synth.normal_f32(f"lat2/v/{shape}", (d_in, r))
    cfg = G.tiny_config("lat2/bf16", x_dtype="bf16")
    s1 = synth.scales(cfg, f"lat2/s1/{d_out}", d_out)
    s2 = synth.scales(cfg, f"lat2/s2/{d_in}", d_in)
    x = synth.activations(f"lat2/x/{d_in}/{T}", T, d_in, "bf16")
    y = nq.lrb_linear_latent(torch.from_numpy(Ul).to(G.DEV), torch.from_numpy(Vl).to(G.DEV),
                             torch.from_numpy(s1).to(G.DEV), torch.from_numpy(s2).to(G.DEV),
                             G.to_device_x(x, "bf16"), r=r).cpu().numpy()
    want = O.linear_latent_ref(Ul[:, :r], Vl[:, :r], s1, s2, x)
    e = C.check(y, want, 1e-5, C.latent_abs_terms(s1, s2, x, r), C.gamma_latent(d_in, r))
    assert e["pass"], e


@pytest.mark.parametrize("su,sv", [(1e20, 1e-25), (1e-25, 1e20), (3e19, 3e19), (1e-24, 1e-24)])
def test_balance_extreme_magnitudes(su, sv):
    """Latents whose squares leave the fp32 range (|v| above ~1.8e19 or below
    ~1e-23): the squared norms are accumulated in fp64, so eta, the scales and
    the balanced factors still match the oracle."""
    d_out, d_in, r = 70, 90, 100
    uh = (synth.normal_f32(f"balx/u/{su}", (d_out, r)) * np.float32(su)).astype(np.float32)
    vh = (synth.normal_f32(f"balx/v/{sv}", (d_in, r)) * np.float32(sv)).astype(np.float32)
    U0, V0, rs1, rs2, reta = O.balance_ref(uh, vh)
    U, V, s1, s2, eta = nq.balance_factors(torch.from_numpy(uh).to(G.DEV), torch.from_numpy(vh).to(G.DEV))
    print(f"balance |U|~{su:g} |V|~{sv:g}: eta {float(eta.item()):.4e} (oracle {reta:.4e})")
    assert abs(float(eta.item()) / reta - 1) <= 1e-6
    for got, want in ((s1, rs1), (s2, rs2), (U, U0), (V, V0)):
        g = got.cpu().numpy()
        assert np.all(np.isfinite(g))
        assert O.rel_err(g, want) <= 1e-6
