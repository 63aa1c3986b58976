"""GPU: the quantize + integer-scale GEMM path captured in a HIP graph.

A serving loop replays the captured launches instead of issuing them one by
one. The graph holds kernel nodes only (the entry points allocate nothing and
issue no memset), so every replay must give exactly the eager result. The
graph is replayed several times with new activations copied into its input
between replays and with eager launches and synchronizations in between; each
replay is compared bit-exactly with an eager run on the same input.
"""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def bgt():
    import bit_gemm_token_amd
    bit_gemm_token_amd.lib()
    return bit_gemm_token_amd


# M values cover the decode kernel (1, 17, 64) and the tiled kernel (300)
@pytest.mark.parametrize("float_scale", [False, True])
def test_graph_replays_match_eager(dev, bgt, float_scale):
    K, N = 1024, 2048
    Ms = (1, 17, 64, 300)
    print(f"graph replay: K={K} N={N} M={Ms} fs={float_scale}", flush=True)
    rng = np.random.default_rng(7)
    w = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    pw = bgt.pack_weights_int4(torch.from_numpy(w).to(dev), alpha=1024)
    xs = {M: torch.zeros((M, K), dtype=torch.float32, device=dev) for M in Ms}
    qs = {M: (torch.empty((M, K), dtype=torch.int8, device=dev),
              torch.empty(M, dtype=torch.float32, device=dev)) for M in Ms}
    ys = {M: torch.full((M, N), float("nan"), dtype=torch.float32, device=dev) for M in Ms}

    def run(M, y):
        q, s = qs[M]
        bgt.quantize_act(xs[M], q=q, scale=s)
        if float_scale:
            bgt.w4a8_gemm_fs(q, s, pw["packed"], pw["fscale"], N, y=y)
        else:
            bgt.w4a8_gemm_is(q, s, pw["packed"], pw["iscale"], pw["alpha"], N, y=y)

    # warm up on a side stream, as graph capture requires
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for M in Ms:
            run(M, ys[M])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for M in Ms:
            run(M, ys[M])

    for rep in range(4):
        for M in Ms:
            xs[M].copy_(torch.from_numpy(synth.activations(100 + rep, M, K)))
            ys[M].fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = {M: ys[M].cpu().numpy().copy() for M in Ms}
        for M in Ms:
            ref = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
            run(M, ref)
            torch.cuda.synchronize()
            r = ref.cpu().numpy()
            assert not np.isnan(got[M]).any(), f"replay {rep} M={M}: unwritten outputs"
            assert np.array_equal(got[M].view(np.int32), r.view(np.int32)), \
                f"replay {rep} M={M}: graph result differs from eager"
        print(f"  replay {rep}: all M equal to eager", flush=True)


def test_graph_replays_match_eager_w8a8(dev, bgt):
    M, K, N = 96, 1024, 1024
    print(f"graph replay w8a8: M={M} K={K} N={N}", flush=True)
    rng = np.random.default_rng(11)
    wt = torch.from_numpy((rng.standard_normal((N, K)) * 0.02).astype(np.float32)).to(dev)
    qw, sw, zw, cw = bgt.quantize_act(wt, mode="asym")
    x = torch.zeros((M, K), dtype=torch.float32, device=dev)
    qx = torch.empty((M, K), dtype=torch.uint8, device=dev)
    sx = torch.empty(M, dtype=torch.float32, device=dev)
    zx = torch.empty(M, dtype=torch.int32, device=dev)
    rx = torch.empty(M, dtype=torch.int32, device=dev)
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)

    def run(out):
        bgt.quantize_act(x, mode="asym", q=qx, scale=sx, zero=zx, rowsum=rx)
        bgt.w8a8_gemm_zp(qx, sx, zx, rx, qw, sw, zw, cw, y=out)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(y)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(y)
    for rep in range(4):
        x.copy_(torch.from_numpy(synth.activations(200 + rep, M, K, outlier_frac=0.0, mean=0.5)))
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = y.cpu().numpy().copy()
        ref = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
        run(ref)
        torch.cuda.synchronize()
        r = ref.cpu().numpy()
        assert not np.isnan(got).any(), f"replay {rep}: unwritten outputs"
        assert np.array_equal(got.view(np.int32), r.view(np.int32)), f"replay {rep}: graph differs from eager"
        print(f"  replay {rep}: equal to eager", flush=True)


def _replay_check(dev, run, outs, refill, reps=4):
    """Capture run() once, then for each replay refill the inputs, replay, and
    compare every output with an eager run on the same inputs."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(outs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(outs)
    for rep in range(reps):
        refill(rep)
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [o.cpu().numpy().copy() for o in outs]
        refs = [torch.full_like(o, float("nan")) for o in outs]
        run(refs)
        torch.cuda.synchronize()
        for a, r in zip(got, refs):
            r = r.cpu().numpy()
            assert not np.isnan(a).any(), f"replay {rep}: unwritten outputs"
            assert np.array_equal(a.view(np.int32), r.view(np.int32)), f"replay {rep}: differs from eager"
        print(f"  replay {rep}: equal to eager", flush=True)


def test_graph_replays_match_eager_w8a8_is(dev, bgt):
    # M = 3: one column tile per workgroup; M = 40: two tiles per workgroup over two parts of the
    # groups plus the reduction; M = 130: the 256 x 128 tile with K split, plus the reduction
    K, N = 4096, 512
    Ms = (3, 40, 130)
    print(f"graph replay w8a8_is: K={K} N={N} M={Ms}", flush=True)
    w = synth.weights(12, K, N, std=0.02, outlier_prob=0.001)
    pw = bgt.pack_weights_int8(torch.from_numpy(w).to(dev), alpha=1 << 16)
    xs = {M: torch.zeros((M, K), dtype=torch.float32, device=dev) for M in Ms}
    qs = {M: (torch.empty((M, K), dtype=torch.int8, device=dev),
              torch.empty(M, dtype=torch.float32, device=dev)) for M in Ms}
    outs = [torch.empty((M, N), dtype=torch.float32, device=dev) for M in Ms]

    def run(ys):
        for M, y in zip(Ms, ys):
            q, s = qs[M]
            bgt.quantize_act(xs[M], q=q, scale=s)
            bgt.w8a8_gemm_is(q, s, pw["qw"], pw["iscale"], pw["alpha"], N, y=y)

    def refill(rep):
        for M in Ms:
            xs[M].copy_(torch.from_numpy(synth.activations(300 + rep, M, K)))

    _replay_check(dev, run, outs, refill)


def test_graph_replays_match_eager_moe(dev, bgt):
    E, K, N = 8, 2048, 256
    Ts = (16, 100)
    print(f"graph replay moe: E={E} K={K} N={N} T={Ts}", flush=True)
    w = synth.expert_weights(13, E, K, N)
    packed = torch.empty((E, N * K // 2), dtype=torch.uint8, device=dev)
    isc = torch.empty((E, K // 128, N), dtype=torch.int32, device=dev)
    fsc = torch.empty((E, K // 128, N), dtype=torch.float32, device=dev)
    for e in range(E):
        bgt.pack_weights_int4(torch.from_numpy(w[e]).to(dev), alpha=1024, packed=packed[e],
                              fscale=fsc[e], iscale=isc[e])
    routes = {}
    for T in Ts:
        offs, tok = synth.route_by_expert(synth.moe_routing(T, T, E, 2), E)
        routes[T] = (torch.from_numpy(offs).to(dev), torch.from_numpy(tok).to(dev), len(tok))
    xs = {T: torch.zeros((T, K), dtype=torch.float32, device=dev) for T in Ts}
    qs = {T: (torch.empty((T, K), dtype=torch.int8, device=dev),
              torch.empty(T, dtype=torch.float32, device=dev)) for T in Ts}
    outs = [torch.empty((routes[T][2], N), dtype=torch.float32, device=dev) for T in Ts]

    def run(ys):
        for T, y in zip(Ts, ys):
            q, s = qs[T]
            offs, tok, _ = routes[T]
            bgt.quantize_act(xs[T], q=q, scale=s)
            bgt.w4a8_moe_gemm_is(q, s, offs, tok, packed, isc, 1024, N, y=y)

    def refill(rep):
        for T in Ts:
            xs[T].copy_(torch.from_numpy(synth.activations(400 + rep, T, K)))

    _replay_check(dev, run, outs, refill)


def test_graph_replays_match_eager_linear(dev, bgt):
    # the entry point the decode bench captures: fused quantization + GEMM for
    # M <= 4, quantizer + GEMM otherwise; 1-byte integer scales
    K, N = 4096, 1024
    Ms = (1, 4, 16)
    print(f"graph replay linear: K={K} N={N} M={Ms}", flush=True)
    w = synth.weights(14, K, N, std=0.02, outlier_prob=0.001)
    pw = bgt.pack_weights_int4(torch.from_numpy(w).to(dev), alpha=1024)
    isc = bgt.narrow_iscale(pw["iscale"], 1)
    xs = {M: torch.zeros((M, K), dtype=torch.float32, device=dev) for M in Ms}
    qs = {M: (torch.empty((M, K), dtype=torch.int8, device=dev),
              torch.empty(M, dtype=torch.float32, device=dev)) for M in Ms}
    outs = [torch.empty((M, N), dtype=torch.float32, device=dev) for M in Ms]
    assert bgt.w4a8_linear_fused(xs[1]) and not bgt.w4a8_linear_fused(xs[16])

    def run(ys):
        for M, y in zip(Ms, ys):
            q, s = qs[M]
            bgt.w4a8_linear_is(xs[M], pw["packed"], isc, pw["alpha"], N, qx=q, sx=s, y=y)

    def refill(rep):
        for M in Ms:
            xs[M].copy_(torch.from_numpy(synth.activations(500 + rep, M, K)))

    _replay_check(dev, run, outs, refill)
