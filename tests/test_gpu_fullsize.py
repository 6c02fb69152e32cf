"""Full-size parity of one training step of the headline layer (12000 tokens,
5376 -> 7168, rotation block 128), run through the same layer object and
launch configuration the benchmark times, and of the transformer MLP's two
layers (8192 tokens, 4096 -> 14336 -> 4096) each on its own.

The oracle recomputes every per-row quantity from the seeded inputs itself
(weight prep, activation codes, both gradient quantizations) and compares
them in full.  The products are compared at outputs it computes one by one,
stratified over the 256 x 256 output tiles the kernels compute: at least 8
outputs of every tile of y and dW, and for the un-rotated dX a whole rotation
block of one row in every 128-column half of every tile.  Both the layer's
calls (which split the grid's last partial round of tiles along the
contraction) and the plain product calls are checked this way.  Whole rows
of dW feed the stochastic requant check.  Everything is bit-exact except the
bias gradient."""
import numpy as np
import pytest

import workloads
from tests.gpu_util import announce, assert_bitwise, dev, host, torch_cuda

pytestmark = pytest.mark.gpu


TILE = 256


def tile_samples(rng, R, C, per=8):
    """Positions (ii, jj) with `per` random outputs inside every TILE x TILE
    tile of an [R, C] output (fewer distinct ones in tiles smaller than that)."""
    ii, jj = [], []
    for r0 in range(0, R, TILE):
        for c0 in range(0, C, TILE):
            ii.append(rng.integers(r0, min(r0 + TILE, R), per))
            jj.append(rng.integers(c0, min(c0 + TILE, C), per))
    return np.concatenate(ii), np.concatenate(jj)


def block_samples(rng, R, C, blk):
    """(row, first column) of one blk-wide block of one random row in every
    128-column half of every TILE x TILE tile of an [R, C] output."""
    half = max(blk, 128)
    out = []
    for r0 in range(0, R, TILE):
        for c0 in range(0, C, half):
            m = int(rng.integers(r0, min(r0 + TILE, R)))
            b0 = c0 + int(rng.integers(0, min(half, C - c0) // blk)) * blk
            out.append((m, b0))
    return out


def _plain_products(layer, M, had):
    """The plain calls on the layer's saved operands (no grid balancing)."""
    from w8a8_integer_linear_amd import _native as Q
    y = Q.qlin_fwd(layer.qx, layer.sx, layer.qw, layer.sw, layer.bias)
    dx = Q.qlin_bwd_dx(layer._qg1[:M], layer._sg1[:M], layer.qw, had_block=had)
    dw = Q.qlin_bwd_dw(layer._qg2[:M], layer._sg2, layer.qx)
    return dict(y=host(y), dx=host(dx), dw=host(dw))


def _step(T, d, M, K, N, had, lr, seed, step):
    from w8a8_integer_linear_amd import LinearW8A8Training
    announce("layer step", M, K, N, had)
    layer = LinearW8A8Training(dev(d["w"]), bias=None if d["b"] is None else dev(d["b"]),
                               had_block=had, max_tokens=M)
    w0 = (host(layer.qw), host(layer.sw))
    y = layer.forward(dev(d["x"]))
    dx = layer.backward(dev(d["dy"]))
    got = dict(qw=w0[0], sw=w0[1], qx=host(layer.qx), sx=host(layer.sx), y=host(y),
               qg1=host(layer._qg1[:M]), sg1=host(layer._sg1[:M]), qg2=host(layer._qg2[:M]),
               sg2=host(layer._sg2), dx=host(dx), dw=host(layer.dw))
    if layer.db is not None:
        got["db"] = host(layer.db)
    got["plain"] = _plain_products(layer, M, had)
    layer.sgd_step(lr, seed, step)
    T.cuda.synchronize()
    got["qw1"], got["sw1"] = host(layer.qw), host(layer.sw)
    if layer.bias is not None:
        got["b1"] = host(layer.bias)
    return got


def _check_step(orc, d, got, M, K, N, had, lr, seed, step, n_samples, rng):
    qw, sw = orc.prepare_weight(d["w"], had_block=had)
    assert_bitwise(got["sw"], sw, "weight scales")
    assert_bitwise(got["qw"], qw, "weight codes")
    qx, sx = orc.quantize_rows(d["x"], had_block=had)
    assert_bitwise(got["sx"], sx, "activation scales")
    assert_bitwise(got["qx"], qx, "activation codes")
    ti, tj = tile_samples(rng, M, N)
    ii = np.concatenate([ti, rng.integers(0, M, n_samples)])
    jj = np.concatenate([tj, rng.integers(0, N, n_samples)])
    y_ref = orc.op_at(orc.OP_FWD, qx, sx, qw, sw, d["b"], M, N, K, ii, jj)
    for which, res in (("layer", got), ("plain", got["plain"])):
        assert_bitwise(res["y"][ii, jj], y_ref, f"y samples ({which})")
    qg1, sg1 = orc.quantize_rows(d["dy"], prescale=sw)
    assert_bitwise(got["sg1"], sg1, "dY row scales")
    assert_bitwise(got["qg1"], qg1, "dY row codes")
    qg2, sg2, db = orc.quantize_cols(d["dy"], prescale=sx, want_sum=True)
    assert_bitwise(got["sg2"], sg2, "dY column scales")
    assert_bitwise(got["qg2"], qg2, "dY column codes")
    # dX: whole blocks of the rotated-basis gradient, then the rotation back,
    # in every 128-column half of every tile.
    blk = had if had else 16
    picks = block_samples(rng, M, K, blk)
    mm = np.repeat([m for m, _ in picks], blk)
    cc = np.concatenate([np.arange(b0, b0 + blk) for _, b0 in picks])
    dxr = orc.op_at(orc.OP_DX, qg1, sg1, qw, None, None, M, N, K, mm, cc).reshape(-1, blk)
    ref = orc.hadamard(dxr, had) if had else dxr
    for which, res in (("layer", got), ("plain", got["plain"])):
        dx_got = res["dx"][mm, cc].reshape(-1, blk)
        assert_bitwise(dx_got, ref, f"dx blocks ({which}, {len(picks)} blocks)")
    # dW: 8 outputs of every tile, and whole rows (which the update reads).
    wi, wj = tile_samples(rng, N, K)
    dw_ref = orc.op_at(orc.OP_DW, qg2, sg2, qx, None, None, M, N, K, wi, wj)
    rows = np.sort(rng.choice(N, 4, replace=False))
    dw_rows = orc.bwd_dw_rows(qg2, sg2, qx, rows)
    for which, res in (("layer", got), ("plain", got["plain"])):
        assert_bitwise(res["dw"][wi, wj], dw_ref, f"dW tile samples ({which})")
        assert_bitwise(res["dw"][rows], dw_rows, f"dW rows ({which})")
    if "db" in got:
        xf = workloads.bf16_bits_to_f32(d["dy"]) if d["dy"].dtype == np.uint16 else d["dy"]
        bound = 1e-5 * np.abs(xf.astype(np.float64)).sum(axis=0)
        assert np.all(np.abs(got["db"].astype(np.float64) - db) <= bound)
        # bias update b - lr * db, with db known to the column-sum tolerance
        b_ref = d["b"].astype(np.float64) - np.float32(lr) * db.astype(np.float64)
        tol = lr * bound + 2.0 ** -23 * np.abs(b_ref)
        assert np.all(np.abs(got["b1"].astype(np.float64) - b_ref) <= tol)
    q1, s1, _ = orc.sgd_requant(qw[rows], sw[rows], dw_rows, lr, seed, step, row_ids=rows)
    assert_bitwise(got["sw1"][rows], s1, "updated scales")
    assert_bitwise(got["qw1"][rows], q1, "updated codes")


def test_tiny_train_step(orc):
    """The tiny workload end to end (64 x 256 -> 128, bias, no rotation)."""
    T = torch_cuda()
    d = workloads.tiny()
    got = _step(T, d, 64, 256, 128, 0, d["lr"], 0, 0)
    _check_step(orc, d, got, 64, 256, 128, 0, d["lr"], 0, 0, 2000, np.random.default_rng(1))


@pytest.mark.parametrize("M", [17, 2048])
def test_forward_width_step(orc, M):
    T = torch_cuda()
    d = workloads.linear(M, 5376, 7168, seed=0)
    got = _step(T, d, M, 5376, 7168, 128, 1e-3, 0, 3)
    _check_step(orc, d, got, M, 5376, 7168, 128, 1e-3, 0, 3, 2048, np.random.default_rng(2))


def test_headline_step(orc):
    """12000 x 5376 -> 7168, rotation 128: the benchmarked training step."""
    T = torch_cuda()
    d = workloads.linear(12000, 5376, 7168, seed=0)
    got = _step(T, d, 12000, 5376, 7168, 128, 1e-3, 0, 0)
    _check_step(orc, d, got, 12000, 5376, 7168, 128, 1e-3, 0, 0, 2048, np.random.default_rng(3))


def _random_layer_cases(n=8, seed=8801):
    """Seeded layer shapes away from the headline ones: any token count from
    17 (the tiled products) up, widths with a ragged last tile, rotation
    blocks 0, 16, 64 and 128, with and without bias, both input dtypes."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        had = [128, 0, 64, 16][i % 4]
        M = int(rng.integers(17, 4000))
        K = 128 * int(rng.integers(1, 24))
        N = 16 * int(rng.integers(1, 200))
        cases.append((i, M, K, N, had, bool(i % 2), bool(rng.integers(0, 2))))
    return cases


@pytest.mark.parametrize("i,M,K,N,had,bias,x_bf16", _random_layer_cases())
def test_layer_step_random_shapes(orc, i, M, K, N, had, bias, x_bf16):
    """One training step of the layer at a random shape, checked like the
    full-size steps: all codes and scales in full, the products at outputs of
    every tile (layer and plain calls), the updated rows bit for bit."""
    T = torch_cuda()
    d = workloads.linear(M, K, N, with_bias=bias, x_bf16=x_bf16, had_block=had, seed=50 + i)
    got = _step(T, d, M, K, N, had, 1e-3, 7, i)
    _check_step(orc, d, got, M, K, N, had, 1e-3, 7, i, 512, np.random.default_rng(60 + i))


@pytest.mark.parametrize("which", [1, 2])
def test_mlp_layer_step(orc, which):
    """The transformer MLP's layers at their own shapes (8192 tokens; fc1
    4096 -> 14336 with a bf16 input and fp32 gradient, fc2 14336 -> 4096 with
    an fp32 GELU-output input and bf16 gradient), rotation 128 on both."""
    T = torch_cuda()
    d = workloads.mlp_layer(which)
    N, K = d["w"].shape
    M = d["x"].shape[0]
    got = _step(T, d, M, K, N, 128, d["lr"], d["seed"], 0)
    _check_step(orc, d, got, M, K, N, 128, d["lr"], d["seed"], 0, 2048,
                np.random.default_rng(10 + which))


def _gelu64(h):
    from scipy.special import erf
    h = h.astype(np.float64)
    return 0.5 * h * (1.0 + erf(h / np.sqrt(2.0)))


def _gelu_grad64(h):
    from scipy.special import erf
    h = h.astype(np.float64)
    return 0.5 * (1.0 + erf(h / np.sqrt(2.0))) + h * np.exp(-0.5 * h * h) / np.sqrt(2 * np.pi)


def test_mlp_chain(orc):
    """The transformer MLP chained on the GPU (8192 tokens: fc1 4096 -> 14336,
    erf-GELU in fp32, fc2 14336 -> 4096; forward, backward to the input).  The
    output and the input gradient of each row depend only on that row, so the
    oracle recomputes 48 sampled rows from the seeded inputs, with the GELU in
    float64.  The GELU is outside the INT8 path (the GPU's fp32 erf and libm
    differ in the last bits), so rows are compared by a tight norm tolerance:
    a GELU ulp can only move a code across a rounding boundary."""
    import torch
    from w8a8_integer_linear_amd import LinearW8A8Training
    T = torch_cuda()
    d = workloads.mlp()
    announce("mlp chain", 8192)
    fc1 = LinearW8A8Training(dev(d["w1"]), had_block=128, max_tokens=8192)
    fc2 = LinearW8A8Training(dev(d["w2"]), had_block=128, max_tokens=8192)
    h = fc1.forward(dev(d["x"])).clone()
    a = torch.nn.functional.gelu(h)
    y = fc2.forward(a).clone()
    da = fc2.backward(dev(d["dy2"])).clone()
    hh = h.double()
    gp = 0.5 * (1 + torch.erf(hh / 2 ** 0.5)) + hh * torch.exp(-0.5 * hh * hh) / (2 * torch.pi) ** 0.5
    dh = (da.double() * gp).float()
    dx = fc1.backward(dh.contiguous())
    T.cuda.synchronize()
    rows = np.sort(np.random.default_rng(21).choice(8192, 48, replace=False))
    qw1, sw1 = orc.prepare_weight(d["w1"], had_block=128)
    qw2, sw2 = orc.prepare_weight(d["w2"], had_block=128)
    qx, sx = orc.quantize_rows(d["x"][rows], had_block=128)
    h_ref = orc.fwd(qx, sx, qw1, sw1)
    assert_bitwise(host(h)[rows], h_ref, "fc1 output")          # exact up to the GELU
    a_ref = _gelu64(h_ref).astype(np.float32)
    qa, sa = orc.quantize_rows(a_ref, had_block=128)
    y_ref = orc.fwd(qa, sa, qw2, sw2)
    qg, sg = orc.quantize_rows(d["dy2"][rows], prescale=sw2)
    da_ref = orc.hadamard(orc.bwd_dx(qg, sg, qw2), 128)
    assert_bitwise(host(da)[rows], da_ref, "fc2 input gradient")
    dh_ref = (da_ref.astype(np.float64) * _gelu_grad64(h_ref)).astype(np.float32)
    qg1, sg1 = orc.quantize_rows(dh_ref, prescale=sw1)
    dx_ref = orc.hadamard(orc.bwd_dx(qg1, sg1, qw1), 128)
    for name, got, ref in (("y", host(y)[rows], y_ref), ("dx", host(dx)[rows], dx_ref)):
        err = np.linalg.norm(got.astype(np.float64) - ref, axis=1)
        assert np.all(err <= 1e-3 * np.linalg.norm(ref.astype(np.float64), axis=1)), name


def test_deterministic(orc):
    """Two runs of the headline step give bitwise identical results."""
    T = torch_cuda()
    d = workloads.linear(2048, 5376, 7168, seed=5)
    a = _step(T, d, 2048, 5376, 7168, 128, 1e-3, 9, 1)
    b = _step(T, d, 2048, 5376, 7168, 128, 1e-3, 9, 1)
    for k in a:
        if k != "plain":
            assert_bitwise(a[k], b[k], k)


def test_graph_replay_of_step(orc):
    """One training step (2048 tokens, 5376 -> 7168, rotation 128: the dW
    product splits its last round) captured in a HIP graph and replayed three
    times from the same starting weight, with eager work between replays: each
    replay reproduces the eager step bit for bit (the calls allocate nothing,
    never synchronize, and the split counters return to zero)."""
    import torch
    from w8a8_integer_linear_amd import LinearW8A8Training
    T = torch_cuda()
    d = workloads.linear(2048, 5376, 7168, seed=4)
    announce("graph replay", 2048)
    layer = LinearW8A8Training(dev(d["w"]), had_block=128, max_tokens=2048)
    x, dy = dev(d["x"]), dev(d["dy"])

    def step():
        y = layer.forward(x)
        dx = layer.backward(dy)
        layer.sgd_step(1e-3, 7, 3)
        return y, dx

    step()                                   # first call: buffers and workspace
    q0, s0 = layer.qw.clone(), layer.sw.clone()
    y, dx = step()
    ref = [t.clone() for t in (y, dx, layer.qw, layer.sw)]
    layer.qw.copy_(q0)
    layer.sw.copy_(s0)
    T.cuda.synchronize()
    graph = T.cuda.CUDAGraph()
    with T.cuda.graph(graph):
        gy, gdx = step()
    for rep in range(3):
        layer.qw.copy_(q0)
        layer.sw.copy_(s0)
        junk = T.randn(1 << 20, device="cuda").sum()     # eager work between replays
        graph.replay()
        T.cuda.synchronize()
        for name, got, want in zip(("y", "dx", "qw", "sw"), (gy, gdx, layer.qw, layer.sw), ref):
            assert_bitwise(host(got), host(want), f"replay {rep}: {name}")
        del junk


def test_split_products_equal_plain_at_full_size(orc):
    """At 12000 x 5376 -> 7168 the forward (36 tiles in 3 pieces) and dW (76
    tiles in 2 pieces) products split their last round; over the whole output
    they equal the plain calls bit for bit, which the sampled oracle checks of
    the step pin.  dX (no split at this shape) goes through the same call."""
    import torch
    T = torch_cuda()
    from w8a8_integer_linear_amd import _native as Q
    M, K, N = 12000, 5376, 7168
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    codes = lambda shape: torch.randint(-127, 128, shape, generator=g, device="cuda",
                                        dtype=torch.int8)
    qx, qw, qg = codes((M, K)), codes((N, K)), codes((M, N))
    sx = torch.rand(M, generator=g, device="cuda") + 0.5
    sw = torch.rand(N, generator=g, device="cuda") * 1e-2
    s1 = torch.rand(M, generator=g, device="cuda") * 1e-3
    s2 = torch.rand(N, generator=g, device="cuda") * 1e-3
    bias = torch.randn(N, generator=g, device="cuda")
    assert Q.qlin_product_ws_bytes(0, M, N, K) > 0 and Q.qlin_product_ws_bytes(2, M, N, K) > 0
    announce("split vs plain at full size")
    pairs = [
        (Q.qlin_product_ws(0, qx, sx, qw, M, N, K, scol=sw, bias=bias),
         Q.qlin_fwd(qx, sx, qw, sw, bias)),
        (Q.qlin_product_ws(1, qg, s1, qw, M, N, K, had_block=128),
         Q.qlin_bwd_dx(qg, s1, qw, had_block=128)),
        (Q.qlin_product_ws(2, qg, s2, qx, M, N, K), Q.qlin_bwd_dw(qg, s2, qx)),
    ]
    T.cuda.synchronize()
    for name, (a, b) in zip(("y", "dx", "dw"), pairs):
        assert torch.equal(a, b), name


def test_weight_norm_step_at_full_size(orc):
    """Weight-normalized 5376 -> 7168 weight: preparation and two SGD steps on
    the whole weight; sampled rows against the oracle (rows key their own
    random streams)."""
    from w8a8_integer_linear_amd import _native as Q
    T = torch_cuda()
    N, K = 7168, 5376
    rng = np.random.default_rng(21)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    announce("wn full size", N, K)
    qd, sd = Q.qlin_quantize_rows(dev(w), had_block=128)
    gd, swd = Q.qlin_wn_init(qd, sd)
    rows = np.sort(rng.choice(N, 6, replace=False))
    q, s = host(qd)[rows], host(sd)[rows]
    g, sw = orc.wn_init(q, s)
    T.cuda.synchronize()
    assert_bitwise(host(gd)[rows], g, "g")
    assert_bitwise(host(swd)[rows], sw, "sw")
    for step in (1, 2):
        dw = (rng.standard_normal((N, K)) * 1e-3).astype(np.float32)
        Q.qlin_wn_sgd_requant(qd, sd, gd, swd, dev(dw), 0.05, seed=5, step=step)
        T.cuda.synchronize()
        q, s, g, sw, _ = orc.wn_sgd_requant(q, s, g, dw[rows], 0.05, 5, step, row_ids=rows)
        for got, ref, what in ((qd, q, "q"), (sd, s, "s"), (gd, g, "g"), (swd, sw, "sw")):
            assert_bitwise(host(got)[rows], ref, f"{what} after step {step}")


def test_weight_norm_layer_step(orc):
    """A layer built with weight_norm=True (tiny workload, no bias): forward,
    backward and the weight-normalized SGD step, every tensor bit for bit
    against the oracle's chain."""
    from w8a8_integer_linear_amd import LinearW8A8Training
    T = torch_cuda()
    d = workloads.tiny()
    M, K, N = 64, 256, 128
    announce("wn layer step")
    layer = LinearW8A8Training(dev(d["w"]), had_block=0, max_tokens=M, weight_norm=True)
    y = layer.forward(dev(d["x"]))
    dx = layer.backward(dev(d["dy"]))
    layer.sgd_step(0.05, 3, 1)
    T.cuda.synchronize()
    q, s = orc.quantize_rows(d["w"])
    g, sw = orc.wn_init(q, s)
    qx, sx = orc.quantize_rows(d["x"])
    assert_bitwise(host(y), orc.fwd(qx, sx, q, sw), "y")
    qg1, sg1 = orc.quantize_rows(d["dy"], prescale=sw)
    assert_bitwise(host(dx), orc.bwd_dx(qg1, sg1, q), "dx")
    qg2, sg2 = orc.quantize_cols(d["dy"], prescale=sx)[:2]
    dw = orc.bwd_dw(qg2, sg2, qx)
    assert_bitwise(host(layer.dw), dw, "dw")
    q1, s1, g1, sw1, _ = orc.wn_sgd_requant(q, s, g, dw, 0.05, 3, 1)
    for got, ref, what in ((layer.qw, q1, "q"), (layer.s, s1, "s"), (layer.g, g1, "g"),
                           (layer.sw, sw1, "sw")):
        assert_bitwise(host(got), ref, what)
