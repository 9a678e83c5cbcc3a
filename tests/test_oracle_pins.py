"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test names what it pins: a value printed on the pages (tests/golden/), a closed
form, an invariant of the definition, a special case that reduces to a library routine
(numpy matmul), or brute force on tiny inputs.  A plausible mistake anywhere in the
oracle (dropped term, wrong sign, swapped index, wrong rounding mode, transposed
operand, wrong constant) fails at least one of them.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def read_golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = line.split(":", 1)
            out[key.strip()] = val.split()
    return out


def bf16_row(values):
    t = torch.tensor(values, dtype=torch.float32)
    assert torch.equal(t.to(torch.bfloat16).float(), t), "pin values must be bf16-exact"
    return workloads.bf16_bits(t.to(torch.bfloat16))


# ----------------------------------------------------------------- O1 weight quant


def test_absmean_worked_example_from_page():
    g = read_golden("absmean_worked_example.txt")
    W = np.array([[float(v) for v in g["input"]]], np.float32)
    q, s = oracle.weight_quant(W)
    # scale printed to 4 decimals
    assert abs(float(s[0]) - float(g["scale"][0])) < 5e-5
    # values before the clamp, as printed: round(W / s) with half-to-even
    pre = np.rint(W[0] / s[0])
    assert pre.astype(int).tolist() == [int(v) for v in g["rounded_before_clamp"]]
    assert q[0].tolist() == [int(v) for v in g["codes"]]
    deq = q[0].astype(np.float64) * float(s[0])
    assert np.allclose(deq, [float(v) for v in g["dequant"]], atol=5e-5)


def test_weight_zero_fraction_gaussian_closed_form():
    # For a Gaussian latent of any sigma, the absmean scale is sigma*sqrt(2/pi), and the
    # code is 0 when |w| < scale/2: P = erf(0.5*sqrt(2/pi)/sqrt(2)) = erf(0.5/sqrt(pi)).
    N, K = 256, 4096
    W = workloads.latent_weights(N, K, seed=3).numpy()
    q, s = oracle.weight_quant(W)
    p0 = math.erf(0.5 / math.sqrt(math.pi))
    assert abs(p0 - 0.3101) < 1e-4
    frac0 = float(np.mean(q == 0))
    sigma = math.sqrt(p0 * (1 - p0) / q.size)
    assert abs(frac0 - p0) < 5 * sigma + 2e-3, frac0
    # symmetric distribution: +1 and -1 equally likely
    fp, fm = float(np.mean(q == 1)), float(np.mean(q == -1))
    assert abs(fp - fm) < 5 * math.sqrt(0.345 * 0.655 / q.size) * 1.5
    # the scale is close to sigma*sqrt(2/pi)
    assert abs(float(np.mean(s)) / (0.02 * math.sqrt(2 / math.pi)) - 1) < 2e-3


def test_weight_quant_invariants():
    rng = np.random.default_rng(7)
    W = (rng.standard_normal((37, 203)) * 0.05).astype(np.float32)
    q, s = oracle.weight_quant(W)
    # power-of-two scaling: codes unchanged, scale scaled exactly
    for e in (-4, 3):
        q2, s2 = oracle.weight_quant(W * np.float32(2.0 ** e))
        assert np.array_equal(q2, q)
        assert np.array_equal(s2, s * np.float32(2.0 ** e))
    # negation: codes negate, scale unchanged
    q3, s3 = oracle.weight_quant(-W)
    assert np.array_equal(q3, -q)
    assert np.array_equal(s3, s)
    assert set(np.unique(q).tolist()) <= {-1, 0, 1}


def test_weight_quant_special_rows():
    W = np.array([[0, 0, 0, 0],              # all zero: eps scale, codes 0
                  [0.25, 0.25, 0.25, 0.25],  # constant: scale = value, codes +1
                  [2, -2, 0.5, -0.5],        # mean|w| = 1.25: 1.6 -> 1, 0.4 -> 0
                  [1e-7, -1e-7, 0, 0]],      # tiny: scale clamps to 1e-5, codes 0
                 np.float32)
    q, s = oracle.weight_quant(W)
    assert s[0] == np.float32(1e-5) and q[0].tolist() == [0, 0, 0, 0]
    assert s[1] == np.float32(0.25) and q[1].tolist() == [1, 1, 1, 1]
    assert s[2] == np.float32(1.25) and q[2].tolist() == [1, -1, 0, 0]
    assert s[3] == np.float32(1e-5) and q[3].tolist() == [0, 0, 0, 0]


# ------------------------------------------------------------------- packing


def test_pack_bit_order_from_page():
    g = read_golden("pack_bit_order.txt")
    codes = np.array([[int(v) for v in g["codes"]]], np.int8)
    packed = oracle.pack(codes)
    assert packed[0].tolist() == [int(b, 16) for b in g["bytes_hex"]]
    assert np.array_equal(oracle.unpack(packed, 8), codes)


def test_pack_roundtrip_and_field_range():
    rng = np.random.default_rng(11)
    q = rng.integers(-1, 2, size=(19, 64), dtype=np.int8)
    packed = oracle.pack(q)
    assert packed.shape == (19, 16)
    assert np.array_equal(oracle.unpack(packed, 64), q)
    fields = np.stack([(packed >> (2 * i)) & 3 for i in range(4)])
    assert fields.max() <= 2  # the unused code 0b11 never appears
    # single-weight positions: weight k of a row lands in byte k//4, bits 2*(k%4)
    for k in range(8):
        one = np.zeros((1, 8), np.int8)
        one[0, k] = 1
        b = oracle.pack(one)[0]
        expect = [0x55, 0x55]
        expect[k // 4] += 1 << (2 * (k % 4))
        assert b.tolist() == expect
    with pytest.raises(oracle.OracleError):
        oracle.unpack(np.array([[0xFF]], np.uint8), 4)


# ---------------------------------------------------------------- O2 act quant


def test_act_quant_tie_case():
    g = read_golden("act_quant_tie_case.txt")
    x = bf16_row([[float(v) for v in g["x"]]])
    xq, a = oracle.act_quant(x)
    assert float(a[0]) == float(g["a_scale"][0])
    assert xq[0].tolist() == [int(v) for v in g["codes"]]


def test_act_quant_invariants():
    X = workloads.activations(9, 517, seed=5, outliers=True)
    xb = workloads.bf16_bits(X)
    xf = X.float().numpy().astype(np.float64)
    xq, a = oracle.act_quant(xb)
    amax = np.abs(xf).max(axis=1)
    # scale is 127 / max|x| to one rounding
    assert np.all(np.abs(a.astype(np.float64) * amax / 127.0 - 1) <= 2.0 ** -23)
    # the largest-magnitude element maps to +-127 with its sign
    arg = np.abs(xf).argmax(axis=1)
    for m in range(xf.shape[0]):
        assert xq[m, arg[m]] == 127 * np.sign(xf[m, arg[m]])
    # round to nearest: |x * a - xq| <= 1/2 (+ fp32 product rounding)
    err = np.abs(xf * a[:, None].astype(np.float64) - xq)
    assert err.max() <= 0.5 + 127 * 2.0 ** -23
    # codes within range, odd symmetry, power-of-two scale invariance
    assert xq.min() >= -127 and xq.max() <= 127
    xq_neg, a_neg = oracle.act_quant(workloads.bf16_bits(-X))
    assert np.array_equal(xq_neg, -xq) and np.array_equal(a_neg, a)
    for e in (-6, 4):
        xq_s, a_s = oracle.act_quant(workloads.bf16_bits(X * (2.0 ** e)))
        assert np.array_equal(xq_s, xq)
        assert np.array_equal(a_s, a / np.float32(2.0 ** e))
    # monotone within a row
    for m in range(xf.shape[0]):
        order = np.argsort(xf[m], kind="stable")
        assert np.all(np.diff(xq[m, order].astype(int)) >= 0)


def test_act_quant_position_equivariance():
    # Quantization is per token and elementwise given the token's max: permuting a row
    # permutes its codes.  Rotate every row so its largest |x| lands first, then last.
    X = workloads.activations(6, 300, seed=8, outliers=False)
    xb = workloads.bf16_bits(X)
    xq, a = oracle.act_quant(xb)
    arg = np.abs(X.float().numpy()).argmax(axis=1)
    for target in (0, xb.shape[1] - 1):
        rolled = np.stack([np.roll(xb[m], target - arg[m]) for m in range(xb.shape[0])])
        xq_r, a_r = oracle.act_quant(rolled)
        assert np.array_equal(a_r, a)
        for m in range(xb.shape[0]):
            assert np.array_equal(xq_r[m], np.roll(xq[m], target - arg[m]))
            assert abs(int(xq_r[m, target])) == 127


def test_act_quant_zero_row():
    xq, a = oracle.act_quant(np.zeros((2, 8), np.uint16))
    assert np.all(xq == 0)
    assert np.all(a == np.float32(127.0) / np.float32(1e-5))


# ------------------------------------------------------------- O3 accumulate


@pytest.mark.parametrize("seed", range(6))
def test_accumulate_matches_numpy_matmul_on_codes(seed):
    rng = np.random.default_rng(100 + seed)
    M = int(rng.integers(1, 18))
    N = int(rng.integers(1, 65))
    K = 4 * int(rng.integers(1, 65))
    xq = rng.integers(-127, 128, size=(M, K), dtype=np.int8)
    q = rng.integers(-1, 2, size=(N, K), dtype=np.int8)
    acc = oracle.accumulate(xq, oracle.pack(q), K)
    expect = xq.astype(np.int64) @ q.astype(np.int64).T
    assert np.array_equal(acc.astype(np.int64), expect)


def test_accumulate_special_cases():
    rng = np.random.default_rng(3)
    M, K = 5, 32
    xq = rng.integers(-127, 128, size=(M, K), dtype=np.int8)
    rowsum = xq.astype(np.int64).sum(axis=1)
    zeros = np.zeros((3, K), np.int8)
    assert np.all(oracle.accumulate(xq, oracle.pack(zeros), K) == 0)
    ones = np.ones((3, K), np.int8)
    assert np.array_equal(oracle.accumulate(xq, oracle.pack(ones), K), np.repeat(rowsum[:, None], 3, 1))
    assert np.array_equal(oracle.accumulate(xq, oracle.pack(-ones), K), -np.repeat(rowsum[:, None], 3, 1))
    eye = np.eye(K, dtype=np.int8)
    assert np.array_equal(oracle.accumulate(xq, oracle.pack(eye), K), xq.astype(np.int32))
    # extreme magnitudes: every product 127 * (+-1)
    big = np.full((1, 4096), 127, np.int8)
    acc = oracle.accumulate(big, oracle.pack(np.ones((1, 4096), np.int8)), 4096)
    assert acc[0, 0] == 127 * 4096


# ----------------------------------------------------------------- O4 rescale


@pytest.mark.parametrize("e", [0, 3, -2])
def test_rescale_reduces_to_float_linear_when_quant_is_lossless(e):
    # X integer-valued with max|x| = 127 * 2^-e in every row: the scale is exactly 2^e,
    # x * a is an integer, so xq * 2^-e == X exactly.  The layer output then equals the
    # float linear layer X @ (q * s)^T (numpy fp64 matmul, exact here), i.e. the page's
    # F.linear(x, w_q * scale).
    rng = np.random.default_rng(21 + e)
    M, N, K = 6, 24, 128
    Xi = rng.integers(-127, 128, size=(M, K)).astype(np.float64)
    Xi[:, 0] = 127.0
    X = Xi * 2.0 ** (-e)
    xb = workloads.bf16_bits(torch.tensor(X, dtype=torch.float32).to(torch.bfloat16))
    W = workloads.latent_weights(N, K, seed=4).numpy()
    out = oracle.bitlinear(xb, W)
    assert np.all(out["a_scale"] == np.float32(2.0 ** e))
    q = oracle.unpack(out["packed"], K).astype(np.float64)
    expect = X @ (q * out["w_scale"][:, None].astype(np.float64)).T
    assert np.array_equal(out["ref"], expect)
    assert np.array_equal(out["out_f32"], expect.astype(np.float32))


def test_bf16_rounding_pins():
    # values exact in fp32: must agree with torch's fp32 -> bf16 (round half even)
    rng = np.random.default_rng(5)
    v = np.concatenate([rng.standard_normal(1000) * 10.0 ** rng.integers(-20, 20, 1000),
                        [0.0, -0.0, 1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5, 3e38]])
    v32 = v.astype(np.float32)
    mine = oracle.f64_to_bf16(v32.astype(np.float64))
    theirs = workloads.bf16_bits(torch.tensor(v32).to(torch.bfloat16))
    assert np.array_equal(mine, theirs)
    # single rounding from fp64: 1 + 2^-8 + 2^-30 is above the tie -> 1 + 2^-7 (0x3F81);
    # rounding through fp32 first would land on the tie and give 1.0 (0x3F80).
    assert oracle.f64_to_bf16(np.array([1.0 + 2.0 ** -8 + 2.0 ** -30]))[0] == 0x3F81
    assert oracle.f64_to_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 0x3F80
    assert oracle.f64_to_bf16(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 0x3F82


def test_rescale_zero_and_sign():
    acc = np.array([[0, 5, -5]], np.int32)
    ref, f32, bf = oracle.rescale(acc, np.array([2.0], np.float32), np.array([1.0, 0.5, 0.5], np.float32))
    assert f32.tolist() == [[0.0, 1.25, -1.25]]
    assert bf[0, 0] == 0


# ---------------------------------------------------------------- tiny layer


def test_tiny_workload_end_to_end_brute_force():
    # Tiny workload (M=4, K=256, N=128): the whole forward against an independent
    # numpy/torch evaluation of the same definition on unpacked codes.
    X = workloads.activations(4, 256, seed=0, outliers=False)
    W = workloads.latent_weights(128, 256, seed=0).numpy()
    out = oracle.bitlinear(workloads.bf16_bits(X), W)
    q = oracle.unpack(out["packed"], 256)
    acc = out["xq"].astype(np.int64) @ q.astype(np.int64).T
    assert np.array_equal(out["acc"].astype(np.int64), acc)
    ref = acc * out["w_scale"][None, :].astype(np.float64) / out["a_scale"][:, None].astype(np.float64)
    assert np.allclose(out["ref"], ref, rtol=1e-15, atol=0)
    # the quantized layer tracks the float layer it approximates
    a64 = out["a_scale"][:, None].astype(np.float64)
    s64 = out["w_scale"][:, None].astype(np.float64)
    deq = (out["xq"] / a64) @ (q * s64).T
    assert np.allclose(out["ref"], deq, rtol=1e-12, atol=1e-12)
    frac0 = float(np.mean(q == 0))
    assert 0.25 < frac0 < 0.37


# ------------------------------------------------------------------- O5 swiglu


def test_swiglu_closed_forms():
    """silu(g) = g * sigmoid(g): sigmoid(ln 3) = 3/4 and sigmoid(-ln 3) = 1/4 exactly, so
    h(ln 3, u) = 0.75 ln 3 u and h(-ln 3, u) = -0.25 ln 3 u; the gate is the SiLU's
    argument (swapping g and u gives 2 sigmoid(2) ln 3, not 1.5 ln 3)."""
    L3 = math.log(3.0)
    h = oracle.swiglu(np.array([L3, -L3, L3, 0.0, 2.0]), np.array([1.0, 1.0, 2.0, 5.0, L3]))
    assert abs(h[0] - 0.75 * L3) <= 1e-15
    assert abs(h[1] + 0.25 * L3) <= 1e-15
    assert abs(h[2] - 1.5 * L3) <= 2e-15
    assert h[3] == 0.0
    assert abs(h[4] - 1.5 * L3) > 0.1


def test_swiglu_invariants():
    """silu(x) - silu(-x) = x; silu(x) -> x for large x and -> x e^x for very negative x;
    linear in u; odd in u."""
    rng = np.random.default_rng(5)
    x = rng.normal(0, 4, 1000)
    ones = np.ones_like(x)
    d = oracle.swiglu(x, ones) - oracle.swiglu(-x, ones)
    assert np.max(np.abs(d - x)) <= 1e-12
    big = np.array([40.0, 60.0])
    assert np.allclose(oracle.swiglu(big, np.ones(2)), big, rtol=1e-15, atol=0)
    neg = np.array([-40.0, -60.0])
    assert np.allclose(oracle.swiglu(neg, np.ones(2)), neg * np.exp(neg), rtol=1e-12, atol=0)
    u = rng.normal(0, 1, 1000)
    h1 = oracle.swiglu(x, u)
    assert np.max(np.abs(oracle.swiglu(x, 3.0 * u) - 3.0 * h1)) <= 1e-12 * np.max(np.abs(h1))
    assert np.array_equal(oracle.swiglu(x, -u), -h1)


# ------------------------------------------------ per-tensor activation scale


def _bits(rows):
    return workloads.bf16_bits(torch.tensor(rows, dtype=torch.float32).to(torch.bfloat16))


def test_act_quant_per_tensor_worked_values():
    """amax over the tensor is 8, so a = 127/8 = 15.875 for both rows: 1 -> 16 (15.875),
    -2 -> -32 (-31.75), 0.5 -> 8 (7.9375), 4 -> 64 (63.5, tie to even), 8 -> 127,
    -8 -> -127, 1 -> 16."""
    xq, a = oracle.act_quant_per_tensor(_bits([[1.0, -2.0, 0.5, 0.0], [4.0, 8.0, -8.0, 1.0]]))
    assert a.tolist() == [15.875, 15.875]
    assert xq.tolist() == [[16, -32, 8, 0], [64, 127, -127, 16]]


def test_act_quant_per_tensor_reduces_to_per_token_for_one_row():
    X = workloads.activations(1, 777 * 4, seed=3)
    b = workloads.bf16_bits(X)
    xq1, a1 = oracle.act_quant(b)
    xq2, a2 = oracle.act_quant_per_tensor(b)
    assert np.array_equal(xq1, xq2) and np.array_equal(a1, a2)


def test_act_quant_per_tensor_invariants():
    X = workloads.activations(6, 256, seed=9)
    b = workloads.bf16_bits(X)
    xq, a = oracle.act_quant_per_tensor(b)
    assert np.all(a == a[0])
    amax = np.max(np.abs(X.to(torch.bfloat16).to(torch.float32).numpy()))
    assert a[0] == np.float32(127.0) / np.float32(amax)
    perm = np.array([3, 0, 5, 1, 4, 2])
    xq_p, a_p = oracle.act_quant_per_tensor(b[perm])
    assert np.array_equal(xq_p, xq[perm]) and np.array_equal(a_p, a)
    # the row holding the tensor's max is coded exactly as by the per-token quantizer
    r = int(np.argmax(np.max(np.abs(X.to(torch.bfloat16).to(torch.float32).numpy()), axis=1)))
    xq_r, _ = oracle.act_quant(b[r:r + 1])
    assert np.array_equal(xq[r:r + 1], xq_r)


# ------------------------------------------------------------- code tables


def test_repack_page_table_example():
    """Weights (+1, 0, -1, +1): with code = w + 1 the byte is 10 00 01 10 (high to low
    field order 3..0) = 0x86; with the page's table (11 +1, 00 0, 01 -1) it is
    11 01 00 11 = 0xD3."""
    out, bad = oracle.repack(np.array([[0x86]], np.uint8), 4, oracle.CODES_OFFSET, oracle.CODES_SIGN)
    assert bad == 0 and out.tolist() == [[0xD3]]
    back, bad = oracle.repack(out, 4, oracle.CODES_SIGN, oracle.CODES_OFFSET)
    assert bad == 0 and back.tolist() == [[0x86]]


def test_repack_unused_codes_and_roundtrip():
    out, bad = oracle.repack(np.array([[0xFF, 0x55]], np.uint8), 8, oracle.CODES_OFFSET, oracle.CODES_SIGN)
    assert bad == 4 and out.tolist() == [[0x00, 0x00]]   # 11 unused -> weight 0; 01 = 0 -> 00
    out, bad = oracle.repack(np.array([[0xAA, 0x44]], np.uint8), 8, oracle.CODES_SIGN, oracle.CODES_OFFSET)
    # 10 unused -> 0 (offset code 01); 0x44 holds fields (00, 01, 00, 01) = (0, -1, 0, -1)
    # -> offset codes (01, 00, 01, 00) = 0x11
    assert bad == 4 and out.tolist() == [[0x55, 0x11]]
    p, _ = oracle.pack_weights(workloads.latent_weights(5, 64, seed=2).numpy())
    q, bad1 = oracle.repack(p, 64, oracle.CODES_OFFSET, oracle.CODES_SIGN)
    r, bad2 = oracle.repack(q, 64, oracle.CODES_SIGN, oracle.CODES_OFFSET)
    assert bad1 == 0 and bad2 == 0 and np.array_equal(r, p)
    assert not np.array_equal(q, p)


# ------------------------------------------------- O6 bf16 activations (W1.58A16)


def test_a16_hand_example():
    """x = (1, 2, 3, 4), w = (+1, 0, -1, +1), w_scale = 0.5: 0.5 * (1 - 3 + 4) = 1."""
    q = np.array([[1, 0, -1, 1]], np.int8)
    ref, sa = oracle.a16(_bits([[1.0, 2.0, 3.0, 4.0]]), oracle.pack(q), np.array([0.5], np.float32), 4)
    assert ref.tolist() == [[1.0]] and sa.tolist() == [[4.0]]


def test_a16_reduces_to_int8_path_for_integer_activations():
    """Integer activations |x| <= 127 are their own int8 codes: the product is then
    w_scale * acc from the pinned int8 accumulation (O3) with a unit activation scale."""
    rng = np.random.default_rng(12)
    M, N, K = 3, 17, 260
    xi = rng.integers(-127, 128, size=(M, K))
    p, s = oracle.pack_weights(workloads.latent_weights(N, K, seed=4).numpy())
    ref, sa = oracle.a16(_bits(xi.astype(np.float32).tolist()), p, s, K)
    acc = oracle.accumulate(xi.astype(np.int8), p, K)
    r2, _, _ = oracle.rescale(acc, np.ones(M, np.float32), s)
    assert np.array_equal(ref, r2)
    assert np.all(sa >= np.abs(ref))


def test_a16_linearity_and_zero_weights():
    X = workloads.activations(2, 64, seed=8).to(torch.bfloat16)
    p, s = oracle.pack_weights(workloads.latent_weights(5, 64, seed=1).numpy())
    r1, _ = oracle.a16(workloads.bf16_bits(X), p, s, 64)
    r2, _ = oracle.a16(workloads.bf16_bits(-X), p, s, 64)          # exact negation
    r4, _ = oracle.a16(workloads.bf16_bits(4 * X), p, s, 64)       # exact power-of-two scale
    assert np.array_equal(r2, -r1) and np.array_equal(r4, 4 * r1)
    zero = oracle.pack(np.zeros((5, 64), np.int8))
    rz, sz = oracle.a16(workloads.bf16_bits(X), zero, s, 64)
    assert not rz.any() and not sz.any()


# ------------------------------------------- five weights per byte (1.6 bits/weight)


def test_b3_hand_worked_bytes():
    # weights (+1, 0, -1, +1, 0) -> codes (2, 1, 0, 2, 1) -> v = 2*81 + 1*27 + 0*9 + 2*3 + 1
    # = 196 -> byte ceil(256 * 196 / 243) = ceil(206.49...) = 207; all zero weights: v =
    # 121 -> ceil(127.47...) = 128; all -1: v = 0 -> 0; all +1: v = 242 -> ceil(254.95) = 255
    rows = np.array([[1, 0, -1, 1, 0], [0, 0, 0, 0, 0], [-1] * 5, [1] * 5], np.int8)
    b = oracle.pack_b3(rows)
    assert b.shape == (4, 64)
    assert b[:, 0].tolist() == [207, 128, 0, 255]
    assert np.all(b[:, 1:] == 128)  # padding weights are 0
    assert np.array_equal(oracle.unpack_b3(b, 5), rows)


def test_b3_state_count_and_digit_extraction():
    # all 3^5 = 243 <= 256 digit patterns map to distinct bytes and back; the digits also
    # come out, first weight first, as the integer parts of repeated multiplication of
    # the byte by 3 (keeping the byte-wide fraction), which is what a decoder may use
    pats = np.array([[(p // 3 ** (4 - i)) % 3 - 1 for i in range(5)] for p in range(243)], np.int8)
    b = oracle.pack_b3(pats)[:, 0].astype(np.int64)
    assert len(set(b.tolist())) == 243 and b.max() <= 255
    assert np.array_equal(oracle.unpack_b3(oracle.pack_b3(pats), 5), pats)
    t = b.copy()
    for i in range(5):
        t = t * 3
        assert np.array_equal(t >> 8, pats[:, i].astype(np.int64) + 1)
        t &= 255


@pytest.mark.parametrize("N,K", [(37, 1000), (3, 320), (5, 4), (2, 641)])
def test_b3_round_trip_and_row_size(N, K):
    rng = np.random.default_rng(N * K)
    q = rng.integers(-1, 2, size=(N, K), dtype=np.int8)
    b = oracle.pack_b3(q)
    assert b.shape == (N, 64 * ((K + 319) // 320)) == (N, oracle.b3_row_bytes(K))
    assert np.array_equal(oracle.unpack_b3(b, K), q)
    if K % 320 == 0:
        assert b.size * 8 / q.size == 1.6


@pytest.mark.parametrize("M,N,K", [(3, 17, 640), (1, 40, 1000), (5, 9, 964)])
def test_b3_accumulate_matches_two_bit_path_and_matmul(M, N, K):
    rng = np.random.default_rng(M + N + K)
    q = rng.integers(-1, 2, size=(N, K), dtype=np.int8)
    xq = rng.integers(-127, 128, size=(M, K), dtype=np.int8)
    acc3 = oracle.accumulate_b3(xq, oracle.pack_b3(q), K)
    assert np.array_equal(acc3, oracle.accumulate(xq, oracle.pack(q), K))
    assert np.array_equal(acc3, xq.astype(np.int64) @ q.astype(np.int64).T)
