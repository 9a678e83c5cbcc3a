"""GPU parity: every entry point of the C ABI against the CPU oracle on the same seeded
inputs.  Integer results (int8 codes, packed bytes, int32 accumulators) and the fp32
scales must be bit-exact; fp32 outputs within 1e-6 relative of the exact value; bf16
outputs within 1 ulp of the round-to-nearest-even of the exact value.

Inputs for a kernel under test come from the generators or from the oracle, never from
another HIP kernel, so each kernel is checked on its own; the chained tests then check
the whole path.  Run on an MI355X: pytest -m gpu.
"""
import numpy as np
import pytest
import torch

import oracle
import ternary_weight_linear_token_amd as bw
import workloads
from gpu_helpers import Problem, check_out, to_np

pytestmark = pytest.mark.gpu

DT = ["f32", "bf16", "i32"]


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


# ------------------------------------------------------------- activation quant


@pytest.mark.parametrize("M,K", [(4, 256), (1, 2560), (3, 260), (5, 4), (2, 28672), (7, 1028),
                                 (512, 2560), (64, 14336), (1, 8196), (3, 32772)])
def test_quant_act_matches_oracle(M, K):
    X = workloads.activations(M, K, seed=M * 7 + K)
    xq_ref, a_ref = oracle.act_quant(workloads.bf16_bits(X))
    xq, a = bw.quant_act(X.cuda())
    assert np.array_equal(to_np(a), a_ref)
    assert np.array_equal(to_np(xq), xq_ref)


def test_quant_act_special_rows():
    K = 64
    rows = torch.zeros((6, K), dtype=torch.float32)
    rows[1, :8] = torch.tensor([254, 125, 5, 1, -1, -3, 0, -254])  # exact half-way ties
    rows[2, 17] = -3.0                                            # a single nonzero
    rows[3] = torch.linspace(-1, 1, K)
    rows[3, 63] = 3.0e38                                          # huge maximum
    rows[4] = 1e-30                                               # below the eps clamp
    rows[5] = torch.arange(K) - 31.5
    X = rows.to(torch.bfloat16)
    xq_ref, a_ref = oracle.act_quant(workloads.bf16_bits(X))
    xq, a = bw.quant_act(X.cuda())
    assert np.array_equal(to_np(a), a_ref)
    assert np.array_equal(to_np(xq), xq_ref)
    assert to_np(xq)[1, :8].tolist() == [127, 62, 2, 0, 0, -2, 0, -127]


@pytest.mark.parametrize("M,K", [(1, 2560), (4, 256), (3, 260), (512, 2560), (7, 28672),
                                 (64, 14336), (2, 4), (300, 1028)])
def test_quant_act_per_tensor_matches_oracle(M, K):
    X = workloads.activations(M, K, seed=M * 13 + K)
    xq_ref, a_ref = oracle.act_quant_per_tensor(workloads.bf16_bits(X))
    xq, a = bw.quant_act_per_tensor(X.cuda())
    assert np.array_equal(to_np(a), a_ref)
    assert np.array_equal(to_np(xq), xq_ref)
    if M == 1:
        xq1, a1 = bw.quant_act(X.cuda())
        assert torch.equal(xq1, xq) and torch.equal(a1, a)


def test_per_tensor_scales_feed_the_products():
    """The product entry points take a per-tensor scale as M equal per-row scales."""
    M, N, K = 40, 300, 1024
    pb = Problem(M, N, K, seed=77)
    o = pb.oracle(full=False)
    xq_ref, a_ref = oracle.act_quant_per_tensor(pb.xbits)
    acc = oracle.accumulate(xq_ref, o["packed"], K)
    ref, _, _ = oracle.rescale(acc, a_ref, o["w_scale"])
    xq, a = bw.quant_act_per_tensor(pb.x_dev)
    for algo in ("tiled", "skinny"):
        out = bw.gemm(xq, a, dev(o["packed"]), dev(o["w_scale"]), "f32", algo=algo)
        check_out(to_np(out), acc, ref, "f32", f"per-tensor {algo}")


# ---------------------------------------------------------------- code tables


@pytest.mark.parametrize("N,K", [(1, 4), (3, 12), (129, 260), (640, 2560)])
def test_repack_codes_matches_oracle(N, K):
    rng = np.random.default_rng(N + K)
    raw = rng.integers(0, 256, size=(N, K // 4), dtype=np.uint8)  # includes unused codes
    for src, dst in ((bw.CODES_OFFSET, bw.CODES_SIGN), (bw.CODES_SIGN, bw.CODES_OFFSET),
                     (bw.CODES_OFFSET, bw.CODES_OFFSET)):
        ref, bad = oracle.repack(raw, K, src, dst)
        cnt = torch.zeros((1,), dtype=torch.int32, device="cuda")
        out = bw.repack_codes(dev(raw), K, src, dst, invalid_count=cnt)
        assert np.array_equal(to_np(out), ref), f"repack {src}->{dst} N={N} K={K}"
        assert int(cnt.item()) == bad
    # in place, and a round trip of valid weights restores them
    p, _ = oracle.pack_weights(workloads.latent_weights(N, K, seed=3).numpy())
    buf = dev(p)
    bw.repack_codes(buf, K, bw.CODES_OFFSET, bw.CODES_SIGN, out=buf)
    assert np.array_equal(to_np(buf), oracle.repack(p, K, 0, 1)[0])
    bw.repack_codes(buf, K, bw.CODES_SIGN, bw.CODES_OFFSET, out=buf)
    assert np.array_equal(to_np(buf), p)


# ---------------------------------------------------------------- weight packing


@pytest.mark.parametrize("N,K", [(128, 256), (33, 260), (1, 4), (640, 2560), (2560, 6912),
                                 (7, 28672)])
def test_pack_matches_oracle(N, K):
    W = workloads.latent_weights(N, K, seed=N + K)
    p_ref, s_ref = oracle.pack_weights(W.numpy())
    packed, scale = bw.pack_weights(W.cuda())
    assert np.array_equal(to_np(scale), s_ref)
    assert np.array_equal(to_np(packed), p_ref)
    codes = bw.unpack_weights(packed, K)
    assert np.array_equal(to_np(codes), oracle.unpack(p_ref, K))


def test_pack_special_rows():
    W = torch.zeros((5, 16))
    W[1] = 0.25
    W[2, :4] = torch.tensor([2.0, -2.0, 0.5, -0.5])
    W[3, :6] = torch.tensor([-0.3, 1.7, 0.0, -2.1, 0.8, -0.1])
    W[4] = -1e-8
    p_ref, s_ref = oracle.pack_weights(W.numpy())
    packed, scale = bw.pack_weights(W.cuda())
    assert np.array_equal(to_np(scale), s_ref)
    assert np.array_equal(to_np(packed), p_ref)


# --------------------------------------------------------- products (oracle inputs)


def product_inputs(pb: Problem):
    o = pb.oracle()
    return dev(o["xq"]), dev(o["a_scale"]), dev(o["packed"]), dev(o["w_scale"]), o


@pytest.mark.parametrize("M", [1, 2, 5, 16])
@pytest.mark.parametrize("N,K", [(16, 256), (37, 260), (300, 1024), (129, 2816), (64, 4),
                                 (33, 7168)])
def test_gemv_matches_oracle(M, N, K):
    pb = Problem(M, N, K, seed=M * 1000 + N + K)
    xq, a, packed, s, o = product_inputs(pb)
    for dt in DT:
        out = bw.gemv(xq, a, packed, s, dt)
        check_out(to_np(out), o["acc"], o["ref"], dt, f"gemv M={M} N={N} K={K} {dt}")


@pytest.mark.parametrize("M", [4, 8, 13, 16])
@pytest.mark.parametrize("N,K", [(300, 1024), (4097, 512), (50, 14336), (17, 64)])
def test_direct_and_staged_small_m_kernels_agree(M, N, K):
    # (also: the fused launch at 12+ tokens equals quant_act followed by the int8 product)
    """For a few tokens the int8 product reads the activations straight into the matrix
    cores (bitnet_w2a8_gemv routes there); the staged kernel (ALGO_SKINNY) must give the
    same bits, and both the oracle's result."""
    pb = Problem(M, N, K, seed=M * 19000 + N + K)
    xq, a, packed, s, o = product_inputs(pb)
    for dt in DT:
        direct = bw.gemv(xq, a, packed, s, dt)
        staged = bw.gemm(xq, a, packed, s, dt, algo="skinny")
        check_out(to_np(direct), o["acc"], o["ref"], dt, f"direct M={M} N={N} K={K} {dt}")
        assert np.array_equal(to_np(direct), to_np(staged)), f"direct != staged M={M} N={N} K={K} {dt}"
        fused, xq_f, a_f = bw.quant_gemv(pb.x_dev, packed, s, dt, return_quant=True)
        assert torch.equal(xq_f, xq) and torch.equal(a_f, a)
        assert np.array_equal(to_np(fused), to_np(direct)), f"fused != two-step M={M} N={N} K={K} {dt}"


@pytest.mark.parametrize("algo", ["tiled", "auto"])
@pytest.mark.parametrize("M", [1, 16, 17, 130, 300])
@pytest.mark.parametrize("N,K", [(64, 64), (200, 256), (130, 1000), (257, 320), (96, 2560)])
def test_gemm_matches_oracle(algo, M, N, K):
    pb = Problem(M, N, K, seed=M * 3000 + N + K)
    xq, a, packed, s, o = product_inputs(pb)
    for dt in DT:
        out = bw.gemm(xq, a, packed, s, dt, algo=algo)
        check_out(to_np(out), o["acc"], o["ref"], dt, f"gemm {algo} M={M} N={N} K={K} {dt}")


@pytest.mark.parametrize("M", [17, 24, 31, 32])
@pytest.mark.parametrize("N,K", [(37, 320), (300, 1024), (129, 6912), (2560, 2560), (64, 64)])
def test_auto_product_for_17_to_32_tokens(M, N, K):
    """17 to 32 tokens through ALGO_AUTO (the direct kernel's two token tiles when K % 64
    == 0): every output dtype against the oracle."""
    pb = Problem(M, N, K, seed=M * 7000 + N + K)
    xq, a, packed, s, o = product_inputs(pb)
    for dt in DT:
        out = bw.gemm(xq, a, packed, s, dt, algo="auto")
        check_out(to_np(out), o["acc"], o["ref"], dt, f"auto M={M} N={N} K={K} {dt}")


@pytest.mark.parametrize("M", [17, 31, 32, 33, 48, 64])
@pytest.mark.parametrize("N,K", [(37, 260), (300, 1024), (129, 6912), (16, 8448)])
def test_skinny_token_tiles_match_oracle(M, N, K):
    """17..64 tokens: two or four 16-row token tiles per chunk of weights, K in several
    LDS stages for the larger M."""
    pb = Problem(M, N, K, seed=M * 7000 + N + K)
    xq, a, packed, s, o = product_inputs(pb)
    for dt in DT:
        out = bw.gemm(xq, a, packed, s, dt, algo="skinny")
        check_out(to_np(out), o["acc"], o["ref"], dt, f"skinny M={M} N={N} K={K} {dt}")


@pytest.mark.parametrize("M", [1, 3, 12, 16])
@pytest.mark.parametrize("N,K", [(16, 256), (300, 1024), (37, 260), (50, 6912), (129, 14336)])
def test_quant_gemv_matches_oracle(M, N, K):
    pb = Problem(M, N, K, seed=M * 5000 + N + K)
    o = pb.oracle()
    packed, s = dev(o["packed"]), dev(o["w_scale"])
    for dt in DT:
        out, xq, a = bw.quant_gemv(pb.x_dev, packed, s, dt, return_quant=True)
        assert np.array_equal(to_np(a), o["a_scale"])
        assert np.array_equal(to_np(xq), o["xq"])
        check_out(to_np(out), o["acc"], o["ref"], dt, f"quant_gemv M={M} N={N} K={K} {dt}")


@pytest.mark.parametrize("M,N,K", [
    (3, 40, 14340),    # staged kernel, 8-byte scan loads (K % 8 != 0), one row per wave
    (6, 70, 14340),    # two K stages, waves with two rows
    (11, 33, 8200),    # 16-byte scan loads, three batches per row, odd batch counts
    (16, 50, 12292),   # 16 tokens on the staged kernel (K % 64 != 0)
    (13, 100, 14336),  # the direct kernel, four batches per row
    (16, 300, 4096),   # the direct kernel, one batch per row
])
def test_fused_scan_finds_each_rows_peak(M, N, K):
    """The fused launches scan every token's max |x| before they quantize: row m gets
    its largest magnitude at a position of its own (the last element for one row, the
    first for another), with a sign and size of its own, so a row mixed up with another
    or a batch left out changes a scale."""
    gen = torch.Generator().manual_seed(M * 31 + K)
    X = (torch.rand(M, K, generator=gen) * 2 - 1).to(torch.bfloat16)
    for m in range(M):
        pos = K - 1 if m == 1 else (0 if m == 2 else (m * 7919 + 13) % K)
        X[m, pos] = (-1) ** m * (4.0 + 0.75 * m)
    pb = Problem(M, N, K, seed=M + K, X=X)
    o = pb.oracle()
    packed, s = dev(o["packed"]), dev(o["w_scale"])
    for dt in DT:
        out, xq, a = bw.quant_gemv(pb.x_dev, packed, s, dt, return_quant=True)
        assert np.array_equal(to_np(a), o["a_scale"]), f"a_scale M={M} K={K}"
        assert np.array_equal(to_np(xq), o["xq"]), f"xq M={M} K={K}"
        check_out(to_np(out), o["acc"], o["ref"], dt, f"fused scan M={M} N={N} K={K} {dt}")


@pytest.mark.parametrize("K,Ns", [(512, [12304]), (256, [12312]), (256, [6912, 6912, 300]),
                                  (2560, [13824, 13830])])
def test_one_token_two_tile_blocks(K, Ns):
    """One token over 768+ row blocks runs blocks of two 16-row tiles: ragged ends where
    the second tile is partial or empty, grouped launches whose groups end mid-block,
    int8 and fused inputs."""
    pb = Problem(1, 1, K, seed=K + len(Ns))
    o1 = pb.oracle(full=False)
    xq, a = dev(o1["xq"]), dev(o1["a_scale"])
    packs, scales, refs = [], [], []
    for g, N in enumerate(Ns):
        W = workloads.latent_weights(N, K, seed=g + 5)
        p, s = oracle.pack_weights(W.numpy())
        acc = oracle.accumulate(o1["xq"], p, K)
        ref, _, _ = oracle.rescale(acc, o1["a_scale"], s)
        packs.append(dev(p)); scales.append(dev(s)); refs.append((acc, ref))
    for dt in DT:
        outs = (bw.quant_gemv_grouped(pb.x_dev, packs, scales, dt) if len(Ns) > 1
                else [bw.quant_gemv(pb.x_dev, packs[0], scales[0], dt)])
        for g, (out, (acc, ref)) in enumerate(zip(outs, refs)):
            check_out(to_np(out), acc, ref, dt, f"two-tile fused K={K} group {g} {dt}")
        if len(Ns) == 1:
            out = bw.gemv(xq, a, packs[0], scales[0], dt)
            check_out(to_np(out), refs[0][0], refs[0][1], dt, f"two-tile int8 K={K} {dt}")


@pytest.mark.parametrize("M", [1, 3, 16])
@pytest.mark.parametrize("K,Ns", [(1024, [300, 37, 16]), (2560, [640, 640, 2560]),
                                  (260, [129, 0, 50]), (256, [16]),
                                  (6912, [33, 64, 17, 200]), (28672, [7, 20])])
def test_quant_gemv_grouped_matches_oracle(M, K, Ns):
    """Several weight matrices against one activation matrix in one launch: each output
    matches the oracle and is bit-identical to the ungrouped launch."""
    X = workloads.activations(M, K, seed=M * 9000 + K)
    pbs = [Problem(M, n, K, seed=M * 9000 + K + 17 * g, X=X) for g, n in enumerate(Ns)]
    os_ = [pb.oracle() for pb in pbs]
    packed = [dev(o["packed"]) for o in os_]
    scales = [dev(o["w_scale"]) for o in os_]
    for dt in DT:
        outs, xq, a = bw.quant_gemv_grouped(pbs[0].x_dev, packed, scales, dt, return_quant=True)
        assert np.array_equal(to_np(a), os_[0]["a_scale"])
        assert np.array_equal(to_np(xq), os_[0]["xq"])
        for g, (o, out) in enumerate(zip(os_, outs)):
            assert tuple(out.shape) == (M, Ns[g])
            check_out(to_np(out), o["acc"], o["ref"], dt, f"grouped g={g} M={M} N={Ns[g]} K={K} {dt}")
            if Ns[g]:
                alone = bw.quant_gemv(pbs[0].x_dev, packed[g], scales[g], dt)
                assert torch.equal(out.view(torch.int32) if dt != "bf16" else out.view(torch.int16),
                                   alone.view(torch.int32) if dt != "bf16" else alone.view(torch.int16))


@pytest.mark.parametrize("M,K,Ns,dts", [
    # tile shape and k-stage chosen by the plan for each launch:
    (130, 320, [257, 64, 0, 96], DT),             # 64x128, 64-k, an empty group
    (512, 384, [2560, 640, 640], DT),             # q|k|v shapes: 64x128, 64-k
    (512, 2560, [2560, 640, 640], ("bf16", "i32")),  # q|k|v at full size: 64x128, 128-k
    (600, 256, [6912, 6912], ("bf16", "i32")),    # gate|up shapes: 128x128 one k-group, 128-k
    (500, 2048, [6000, 7000], ("f32", "i32")),    # 128x128 one k-group, 128-k
    (1024, 128, [4096, 1024, 1024, 300], ("f32", "i32")),  # 128x128 one k-group, 128-k
    (257, 320, [5000, 4000], ("bf16", "i32")),    # 128x128, 64-k
    (300, 384, [4100, 4100], ("bf16", "i32")),    # 128x128, 128-k
])
def test_gemm_grouped_matches_oracle(M, K, Ns, dts):
    """Several weight matrices against one int8 activation matrix in one tiled launch
    (the tile shape follows the launch's total tile count): each output matches the
    oracle and is bit-identical to the tiled launch on that matrix alone."""
    X = workloads.activations(M, K, seed=M * 13000 + K)
    pbs = [Problem(M, n, K, seed=M * 13000 + K + 23 * g, X=X) for g, n in enumerate(Ns)]
    os_ = [pb.oracle() for pb in pbs]
    xq, a = dev(os_[0]["xq"]), dev(os_[0]["a_scale"])
    packed = [dev(o["packed"]) for o in os_]
    scales = [dev(o["w_scale"]) for o in os_]
    for dt in dts:
        outs = bw.gemm_grouped(xq, a, packed, scales, dt)
        for g, (o, out) in enumerate(zip(os_, outs)):
            assert tuple(out.shape) == (M, Ns[g])
            check_out(to_np(out), o["acc"], o["ref"], dt, f"gemm grouped g={g} {M}x{Ns[g]}x{K} {dt}")
            if Ns[g]:
                alone = bw.gemm(xq, a, packed[g], scales[g], dt, algo="tiled")
                assert torch.equal(out.view(torch.int16), alone.view(torch.int16)), (g, dt)


def swiglu_tolerance(g_ref, u_ref, h_ref):
    """fp32 bound for h = silu(g) * u: g and u are each within 3 ulp of exact (see
    gpu_helpers); silu scales g's relative error by at most 1 + |g|; exp, the division
    and the two products add one rounding each.  An absolute floor of the smallest normal
    times |u| covers exp(-g) overflowing to inf for g < -88 (h then underflows to 0)."""
    return (12.0 + 6.0 * np.abs(g_ref)) * 2.0 ** -23 * np.abs(h_ref) + 2.0 ** -126 * np.abs(u_ref)


@pytest.mark.parametrize("M", [1, 3, 16])
@pytest.mark.parametrize("N,K", [(16, 256), (300, 1024), (37, 260), (129, 2560), (50, 6912),
                                 (20, 28672)])
def test_quant_gemv_swiglu_matches_oracle(M, N, K):
    """gate and up in one launch with h = silu(g) * u written out, against the oracle's
    swiglu of its exact products."""
    X = workloads.activations(M, K, seed=M * 11000 + N + K)
    pg = Problem(M, N, K, seed=M * 11000 + N + K + 1, X=X)
    pu = Problem(M, N, K, seed=M * 11000 + N + K + 2, X=X)
    og, ou = pg.oracle(), pu.oracle()
    h_ref = oracle.swiglu(og["ref"], ou["ref"])
    lim = swiglu_tolerance(og["ref"], ou["ref"], h_ref)
    pk_g, s_g, pk_u, s_u = dev(og["packed"]), dev(og["w_scale"]), dev(ou["packed"]), dev(ou["w_scale"])
    h, xq, a = bw.quant_gemv_swiglu(pg.x_dev, pk_g, s_g, pk_u, s_u, "f32", return_quant=True)
    assert np.array_equal(to_np(a), og["a_scale"]) and np.array_equal(to_np(xq), og["xq"])
    err = np.abs(to_np(h).astype(np.float64) - h_ref)
    bad = np.flatnonzero((err > lim).reshape(-1))
    assert bad.size == 0, f"swiglu M={M} N={N} K={K}: {bad.size} fp32 outputs beyond the bound"
    hb = to_np(bw.quant_gemv_swiglu(pg.x_dev, pk_g, s_g, pk_u, s_u, "bf16"))
    from gpu_helpers import bf16_key
    d = np.abs(bf16_key(hb) - bf16_key(oracle.f64_to_bf16(h_ref)))
    assert d.max(initial=0) <= 1, f"swiglu bf16 M={M} N={N} K={K}: off by {d.max()} ulp"


@pytest.mark.parametrize("M", [1, 2, 16])
@pytest.mark.parametrize("N,K", [(16, 64), (300, 1024), (37, 320), (129, 2560), (640, 6912),
                                 (20, 28672)])
def test_a16_gemv_matches_oracle(M, N, K):
    """bf16 activations times ternary weights: each product is exact, the fp32 sum of K
    terms is within (K + 2) 2^-24 sum|x w| of the exact sum (any order), times w_scale."""
    pb = Problem(M, N, K, seed=M * 17000 + N + K)
    o = pb.oracle(full=False)
    ref, sumabs = oracle.a16(pb.xbits, o["packed"], o["w_scale"], K)
    lim = (K + 2) * 2.0 ** -24 * sumabs
    packed, s = dev(o["packed"]), dev(o["w_scale"])
    out = to_np(bw.a16_gemv(pb.x_dev, packed, s, "f32")).astype(np.float64)
    bad = np.flatnonzero((np.abs(out - ref) > lim).reshape(-1))
    assert bad.size == 0, f"a16 M={M} N={N} K={K}: {bad.size} outputs beyond the bound"
    # the measured error sits far inside the worst-case bound
    assert np.max(np.abs(out - ref) / np.maximum(sumabs, 1e-30)) < 64 * 2.0 ** -24 * np.sqrt(K)
    outb = to_np(bw.a16_gemv(pb.x_dev, packed, s, "bf16"))
    fb = outb.astype(np.uint32) << 16
    vb = fb.view(np.float32).astype(np.float64)
    # bf16 adds one rounding of the fp32 value v: half an ulp, <= 2^-9 |v| <= 2^-9 (|ref| + lim)
    assert np.all(np.abs(vb - ref) <= (1 + 2.0 ** -8) * lim + 2.0 ** -8 * np.abs(ref)), \
        f"a16 bf16 M={M} N={N} K={K}"
    # integer-valued activations make every partial sum exact: then it is the int8 result
    xi = torch.randint(-127, 128, (M, K), generator=torch.Generator().manual_seed(K))
    xq = xi.to(torch.int8)
    acc = oracle.accumulate(xq.numpy(), o["packed"], K)
    exact, _, _ = oracle.rescale(acc, np.ones(M, np.float32), o["w_scale"])
    outi = to_np(bw.a16_gemv(xi.to(torch.bfloat16).cuda(), packed, s, "f32")).astype(np.float64)
    assert np.all(np.abs(outi - exact) <= 2.0 ** -24 * np.abs(exact)), f"a16 integer M={M} N={N} K={K}"


# ------------------------------------------------- five weights per byte (1.6 bits)


@pytest.mark.parametrize("N,K", [(1, 4), (3, 12), (129, 260), (640, 2560), (33, 8192),
                                 (7, 28672)])
def test_pack_b3_matches_oracle(N, K):
    rng = np.random.default_rng(N + K)
    # every 2-bit field value, the unused code 3 included (it becomes weight 0)
    packed = rng.integers(0, 256, size=(N, K // 4), dtype=np.uint8)
    cleared, _ = oracle.repack(packed, K, oracle.CODES_OFFSET, oracle.CODES_OFFSET)
    want = oracle.pack_b3(oracle.unpack(cleared, K))
    got = bw.pack_b3(dev(packed), K)
    assert np.array_equal(to_np(got), want)


@pytest.mark.parametrize("N,K", [(16, 256), (37, 264), (300, 1024), (129, 2560), (50, 6912),
                                 (33, 8192), (17, 30720), (1, 8), (640, 2560), (4100, 320)])
def test_quant_gemv_b3_matches_oracle(N, K):
    pb = Problem(1, N, K, seed=N * 7 + K)
    o = pb.oracle(full=False)
    q = oracle.unpack(o["packed"], K)
    b3 = oracle.pack_b3(q)
    acc = oracle.accumulate_b3(o["xq"], b3, K)
    ref, _, _ = oracle.rescale(acc, o["a_scale"], o["w_scale"])
    b3_dev, s = dev(b3), dev(o["w_scale"])
    for dt in DT:
        out = bw.quant_gemv_b3(pb.x_dev, b3_dev, s, dt)
        check_out(to_np(out), acc, ref, dt, f"b3 N={N} K={K} {dt}")
    # the same weights in the 2-bit format give the same exact accumulators
    two_bit = bw.quant_gemv(pb.x_dev, dev(o["packed"]), s, "i32")
    assert np.array_equal(to_np(two_bit), acc)


def test_b3_chain_from_latent_weights():
    # pack on the GPU (2-bit, then five per byte), then the product, against the oracle
    N, K = 515, 4096
    pb = Problem(1, N, K, seed=21)
    packed, s = bw.pack_weights(pb.w_dev)
    b3 = bw.pack_b3(packed, K)
    o = pb.oracle(full=False)
    assert np.array_equal(to_np(b3), oracle.pack_b3(oracle.unpack(o["packed"], K)))
    acc = oracle.accumulate_b3(o["xq"], to_np(b3), K)
    ref, _, _ = oracle.rescale(acc, o["a_scale"], o["w_scale"])
    check_out(to_np(bw.quant_gemv_b3(pb.x_dev, b3, s, "f32")), acc, ref, "f32", "b3 chain")


def test_extreme_accumulators():
    # every activation at +-127 and every weight +1 / -1: |acc| = 127 K, the largest sums
    M, N, K = 3, 40, 28672
    xq = np.full((M, K), 127, np.int8)
    xq[1] = -127
    xq[2, ::2] = -127
    q = np.ones((N, K), np.int8)
    q[1::2] = -1
    packed = oracle.pack(q)
    a = np.full((M,), 1.0, np.float32)
    s = np.linspace(0.5, 2.0, N).astype(np.float32)
    acc = oracle.accumulate(xq, packed, K)
    ref, _, _ = oracle.rescale(acc, a, s)
    for algo in ("skinny", "tiled"):
        for dt in DT:
            out = bw.gemm(dev(xq), dev(a), dev(packed), dev(s), dt, algo=algo)
            check_out(to_np(out), acc, ref, dt, f"extreme {algo} {dt}")


def test_unused_code_decodes_the_same_on_every_route():
    # Bytes with every 2-bit field value, 0b11 included (never written by the packing):
    # every int8 product route reads it as w = code - 1 = +2, like the oracle's decode,
    # and the bf16-activation product reads it as 0.
    rng = np.random.default_rng(33)
    K = 1024
    for M, N in ((1, 300), (5, 300), (16, 129), (17, 64), (40, 300), (130, 257)):
        packed_np = rng.integers(0, 256, size=(N, K // 4), dtype=np.uint8)
        assert np.any(((packed_np[..., None] >> np.array([0, 2, 4, 6], np.uint8)) & 3) == 3)
        X = workloads.activations(M, K, seed=M + N)
        xq_np, a_np = oracle.act_quant(workloads.bf16_bits(X))
        s_np = np.linspace(0.01, 0.03, N).astype(np.float32)
        acc = oracle.accumulate(xq_np, packed_np, K)
        ref, _, _ = oracle.rescale(acc, a_np, s_np)
        packed, s, xq, a = dev(packed_np), dev(s_np), dev(xq_np), dev(a_np)
        outs = {f"gemm {algo}": bw.gemm(xq, a, packed, s, "i32", algo=algo)
                for algo in ("tiled", "auto") + (("skinny",) if M <= 64 else ())}
        outs["grouped"] = bw.gemm_grouped(xq, a, [packed], [s], "i32")[0]
        if M <= bw.GEMV_MAX_M:
            outs["gemv"] = bw.gemv(xq, a, packed, s, "i32")
            outs["quant_gemv"] = bw.quant_gemv(X.cuda(), packed, s, "i32")
            outs["quant_gemv_grouped"] = bw.quant_gemv_grouped(X.cuda(), [packed], [s], "i32")[0]
        for route, out in outs.items():
            check_out(to_np(out), acc, ref, "i32", f"code 3, {route}, M={M} N={N}")
        if M <= bw.GEMV_MAX_M:
            as_zero, _ = oracle.repack(packed_np, K, oracle.CODES_OFFSET, oracle.CODES_OFFSET)
            ref16, sumabs = oracle.a16(workloads.bf16_bits(X), as_zero, s_np, K)
            out16 = to_np(bw.a16_gemv(X.cuda(), packed, s, "f32")).astype(np.float64)
            assert np.all(np.abs(out16 - ref16) <= (K + 2) * 2.0 ** -24 * sumabs), "code 3, a16"


def test_zero_rows_and_zero_weights():
    M, N, K = 4, 48, 512
    X = workloads.activations(M, K, seed=1)
    X[2] = 0
    W = workloads.latent_weights(N, K, seed=2)
    W[5] = 0
    W[17] = 1e-9
    pb = Problem(M, N, K, X=X, W=W)
    o = pb.oracle()
    packed, s = dev(o["packed"]), dev(o["w_scale"])
    for dt in DT:
        out = bw.quant_gemv(pb.x_dev, packed, s, dt)
        check_out(to_np(out), o["acc"], o["ref"], dt, f"zero rows {dt}")
        out2 = bw.gemm(dev(o["xq"]), dev(o["a_scale"]), packed, s, dt, algo="tiled")
        check_out(to_np(out2), o["acc"], o["ref"], dt, f"zero rows tiled {dt}")


def test_empty_problems_are_noops():
    xq = torch.zeros((0, 256), dtype=torch.int8, device="cuda")
    a = torch.zeros((0,), dtype=torch.float32, device="cuda")
    packed = torch.zeros((8, 64), dtype=torch.uint8, device="cuda")
    s = torch.ones((8,), dtype=torch.float32, device="cuda")
    out = bw.gemm(xq, a, packed, s, "f32")
    assert out.shape == (0, 8)
    out = bw.gemv(torch.zeros((1, 256), dtype=torch.int8, device="cuda"),
                  torch.ones((1,), device="cuda"), packed[:0], s[:0], "f32")
    assert out.shape == (1, 0)


def test_outputs_are_deterministic():
    pb = Problem(300, 257, 2560, seed=11)
    xq, a, packed, s, _ = product_inputs(pb)
    for algo in ("tiled",):
        o1 = bw.gemm(xq, a, packed, s, "f32", algo=algo)
        o2 = bw.gemm(xq, a, packed, s, "f32", algo=algo)
        assert torch.equal(o1.view(torch.int32), o2.view(torch.int32))
    x1 = bw.quant_gemv(pb.x_dev[:7], packed, s, "bf16")
    x2 = bw.quant_gemv(pb.x_dev[:7], packed, s, "bf16")
    assert torch.equal(x1.view(torch.int16), x2.view(torch.int16))


# ------------------------------------------------------------ chained GPU path


@pytest.mark.parametrize("dt", DT)
def test_tiny_workload_chain(dt):
    # The tiny workload end to end on the GPU: pack, quantize, product (both kernels).
    (name, N, K), = workloads.WORKLOADS["tiny"]["layer"]
    M = workloads.WORKLOADS["tiny"]["Ms"][0]
    pb = Problem(M, N, K, seed=0, outliers=False)
    o = pb.oracle()
    packed, s = bw.pack_weights(pb.w_dev)
    xq, a = bw.quant_act(pb.x_dev)
    assert np.array_equal(to_np(packed), o["packed"]) and np.array_equal(to_np(s), o["w_scale"])
    assert np.array_equal(to_np(xq), o["xq"]) and np.array_equal(to_np(a), o["a_scale"])
    for out in (bw.gemv(xq, a, packed, s, dt), bw.gemm(xq, a, packed, s, dt, algo="tiled"),
                bw.quant_gemv(pb.x_dev, packed, s, dt), bw.bitlinear(pb.x_dev, packed, s, dt)):
        check_out(to_np(out), o["acc"], o["ref"], dt, f"tiny chain {dt}")


@pytest.mark.parametrize("M", [1, 4, 5, 16, 17, 40, 64, 65, 200])
def test_bitlinear_every_route(M):
    # bitlinear picks the fused decode launch, or quantization plus the skinny or tiled
    # product, by M, N and K (a long row sends 4 tokens to the two-launch route); every
    # route must give the oracle's result.
    for N, K in ((300, 1024), (4096, 256), (64, 16384)):
        pb = Problem(M, N, K, seed=M * 11 + N)
        o = pb.oracle()
        packed, s = dev(o["packed"]), dev(o["w_scale"])
        for dt in DT:
            out = bw.bitlinear(pb.x_dev, packed, s, dt)
            check_out(to_np(out), o["acc"], o["ref"], dt, f"bitlinear M={M} N={N} K={K} {dt}")


def test_graph_replay_matches_eager():
    # The benchmark captures launches in HIP graphs: every replay, with eager work and
    # synchronizations in between, must reproduce the eager results bit for bit.
    pb = Problem(1, 640, 2560, seed=3)
    o = pb.oracle()
    packed, s = dev(o["packed"]), dev(o["w_scale"])
    pb2 = Problem(130, 200, 1024, seed=4)
    o2 = pb2.oracle()
    xq2, a2, packed2, s2 = dev(o2["xq"]), dev(o2["a_scale"]), dev(o2["packed"]), dev(o2["w_scale"])
    out = torch.empty((1, 640), dtype=torch.float32, device="cuda")
    out2 = torch.empty((130, 200), dtype=torch.bfloat16, device="cuda")
    xq_g = torch.empty((1, 2560), dtype=torch.int8, device="cuda")
    a_g = torch.empty((1,), dtype=torch.float32, device="cuda")

    def work():
        bw.quant_gemv(pb.x_dev, packed, s, "f32", out=out)
        bw.quant_act(pb.x_dev, xq=xq_g, a_scale=a_g)
        bw.gemm(xq2, a2, packed2, s2, "bf16", algo="tiled", out=out2)

    work()
    torch.cuda.synchronize()
    eager = (out.clone(), xq_g.clone(), out2.clone())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        work()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    for rep in range(4):
        out.zero_()
        out2.zero_()
        xq_g.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), eager[0].view(torch.int32)), rep
        assert torch.equal(xq_g, eager[1]), rep
        assert torch.equal(out2.view(torch.int16), eager[2].view(torch.int16)), rep
        bw.gemm(xq2, a2, packed2, s2, "f32", algo="tiled")  # unrelated eager work
    check_out(to_np(out), o["acc"], o["ref"], "f32", "graph replay gemv")
    check_out(to_np(out2), o2["acc"], o2["ref"], "bf16", "graph replay gemm")


def test_graph_replay_of_grouped_swiglu_and_a16_launches():
    # The same for the decode-step launches the benchmark captures: grouped q|k|v, the
    # SwiGLU pair, the bf16-activation product and the per-tensor quantization.
    X = workloads.activations(1, 1024, seed=21)
    pbs = [Problem(1, n, 1024, seed=30 + i, X=X) for i, n in enumerate((300, 64, 64))]
    os_ = [pb.oracle() for pb in pbs]
    pk = [dev(o["packed"]) for o in os_]
    sc = [dev(o["w_scale"]) for o in os_]
    x = pbs[0].x_dev
    outs = [torch.empty((1, pb.N), dtype=torch.float32, device="cuda") for pb in pbs]
    h = torch.empty((1, 64), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((1, 300), dtype=torch.float32, device="cuda")
    xq = torch.empty((1, 1024), dtype=torch.int8, device="cuda")
    a = torch.empty((1,), dtype=torch.float32, device="cuda")
    # a prefill-sized batch through the grouped tiled product
    xq64, a64 = bw.quant_act(workloads.activations(64, 1024, seed=22).cuda())
    gouts = [torch.empty((64, pb.N), dtype=torch.bfloat16, device="cuda") for pb in pbs]
    bufs = outs + [h, y, xq, a] + gouts

    def work():
        bw.quant_gemv_grouped(x, pk, sc, "f32", out=outs)
        bw.quant_gemv_swiglu(x, pk[1], sc[1], pk[2], sc[2], "bf16", out=h)
        bw.a16_gemv(x, pk[0], sc[0], "f32", out=y)
        bw.quant_act_per_tensor(x, xq=xq, a_scale=a)
        bw.gemm_grouped(xq64, a64, pk, sc, "bf16", out=gouts)

    work()
    torch.cuda.synchronize()
    eager = [b.clone() for b in bufs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        work()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    for rep in range(4):
        for b in bufs:
            b.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for b, e in zip(bufs, eager):
            assert torch.equal(b.view(torch.uint8), e.view(torch.uint8)), rep
        bw.quant_gemv(x, pk[0], sc[0], "f32")  # unrelated eager work
    for o, out, pb in zip(os_, outs, pbs):
        check_out(to_np(out), o["acc"], o["ref"], "f32", f"graph replay grouped N={pb.N}")


def test_gemm_small_and_large_tile_grids():
    # Shapes that select each unsplit tile configuration (64x128 with four k-groups,
    # 128x128 with two or one; 64-k and 128-k stages), including grids far smaller than
    # the CU count and ragged edges, with and without a workspace (with one, the small
    # grids split K across blocks)
    for (M, N, K) in [(300, 257, 2560), (512, 2560, 2560), (130, 640, 6912), (17, 1024, 4096),
                      (1024, 8192, 512), (600, 16384, 256), (257, 9000, 320), (520, 33000, 320),
                      (520, 33024, 128), (264, 65560, 192), (300, 8200, 384), (64, 4096, 1024)]:
        pb = Problem(M, N, K, seed=M + N + K)
        xq, a, packed, s, o = product_inputs(pb)
        out = bw.gemm(xq, a, packed, s, "i32", algo="tiled")
        check_out(to_np(out), o["acc"], o["ref"], "i32", f"tiles {M}x{N}x{K}")
        out = bw.gemm(xq, a, packed, s, "bf16", algo="tiled", workspace=False)
        check_out(to_np(out), o["acc"], o["ref"], "bf16", f"tiles {M}x{N}x{K} bf16")


# (M, N, K) whose tiled plan splits K across blocks (on 256 CUs): aligned and ragged N
# (vector and element-wise reduce), 64-k and 128-k stages, up to 16 slices; the last three
# reach the 256x128 (128-k and 64-k) and 256x256 tiles, which run only split
SPLIT_CASES = [(32, 8192, 4096), (64, 1024, 4096), (17, 300, 2560), (33, 1000, 6912),
               (96, 130, 8192), (5, 2000, 2048), (1, 640, 2560), (300, 257, 2560),
               (128, 512, 16384), (256, 4096, 14336),
               (400, 5000, 28672), (400, 3000, 20416), (600, 6912, 16320)]


@pytest.mark.parametrize("M,N,K", SPLIT_CASES)
def test_split_k_matches_oracle_and_unsplit(M, N, K):
    assert bw.gemm_plan(M, K, [N])[4] > 1, "shape no longer splits on this device"
    need = int(bw.lib().bitnet_w2a8_gemm_workspace_size(M, N, K))
    assert need > 0
    pb = Problem(M, N, K, seed=M * 3 + N + K)
    xq, a, packed, s, o = product_inputs(pb)
    ws = torch.full((need + 64,), 0x7F, dtype=torch.uint8, device="cuda")
    for dt in DT:
        split = bw.gemm(xq, a, packed, s, dt, algo="tiled", workspace=ws)
        check_out(to_np(split), o["acc"], o["ref"], dt, f"split {M}x{N}x{K} {dt}")
        whole = bw.gemm(xq, a, packed, s, dt, algo="tiled", workspace=False)
        assert torch.equal(split, whole), f"split and unsplit differ {M}x{N}x{K} {dt}"
        # a workspace one byte short of the plan's partials runs unsplit, same result
        short = bw.gemm(xq, a, packed, s, dt, algo="tiled", workspace=ws[:need - 16])
        assert torch.equal(short, whole), f"short workspace {M}x{N}x{K} {dt}"


def test_split_k_in_graph_replays():
    # the two launches of a split product (partials, then reduce) captured in a graph and
    # replayed several times with eager work in between, every replay checked
    M, N, K = 32, 8192, 4096
    pb = Problem(M, N, K, seed=5)
    xq, a, packed, s, o = product_inputs(pb)
    ws = torch.empty((int(bw.lib().bitnet_w2a8_gemm_workspace_size(M, N, K)),),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        bw.gemm(xq, a, packed, s, "f32", algo="tiled", out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        bw.gemm(xq, a, packed, s, "f32", algo="tiled", out=out, workspace=ws)
    for rep in range(4):
        out.zero_()
        ws.fill_(rep)
        g.replay()
        torch.cuda.synchronize()
        check_out(to_np(out), o["acc"], o["ref"], "f32", f"split graph replay {rep}")
