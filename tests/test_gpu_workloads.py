"""GPU parity at the full workload sizes, in the launch configuration the benchmark
times: packed weights and scales checked whole, quantized activations checked whole,
and every product output checked whole -- the int32 accumulators bit-exact against the
oracle's, the fp32 and bf16 outputs against the oracle's rescale of those accumulators.
Decode (M <= 16) runs the fused quant + GEMV entry point; larger M runs the separate
quantization kernel and then the GEMM entry point.

The oracle's scalar accumulation is the slow part: the largest shapes (70B gate / up /
down at M = 1024, 2.4e11 multiply-adds each) take tens of seconds on the host cores.
"""
import time

import numpy as np
import pytest
import torch

import oracle
import ternary_weight_linear_token_amd as bw
import workloads
from gpu_helpers import check_out, to_np

pytestmark = pytest.mark.gpu


def cases():
    out = []
    for wl, spec in workloads.WORKLOADS.items():
        if wl == "tiny":
            continue
        for name, N, K in workloads.distinct_shapes(spec["layer"]):
            out.append(pytest.param(wl, name, N, K, spec["Ms"], spec["outliers"],
                                    id=f"{wl}-{name}-{N}x{K}"))
    return out


@pytest.mark.parametrize("wl,name,N,K,Ms,outliers", cases())
def test_workload_shape(wl, name, N, K, Ms, outliers):
    assert torch.cuda.is_available()
    print(f"\n[{wl}] {name} N={N} K={K} Ms={Ms}", flush=True)
    W = workloads.latent_weights(N, K, seed=0)
    p_ref, s_ref = oracle.pack_weights(W.numpy())
    packed, w_scale = bw.pack_weights(W.cuda())
    del W
    assert np.array_equal(to_np(w_scale), s_ref), "w_scale"
    assert np.array_equal(to_np(packed), p_ref), "packed"
    for M in Ms:
        X = workloads.activations(M, K, seed=0, outliers=outliers)
        xq_ref, a_ref = oracle.act_quant(workloads.bf16_bits(X))
        x_dev = X.cuda()
        if M <= bw.GEMV_MAX_M:
            outs = {dt: bw.quant_gemv(x_dev, packed, w_scale, dt, return_quant=True)
                    for dt in ("f32", "bf16", "i32")}
            xq_dev, a_dev = outs["f32"][1], outs["f32"][2]
            outs = {dt: v[0] for dt, v in outs.items()}
        else:
            xq_dev, a_dev = bw.quant_act(x_dev)
            outs = {dt: bw.gemm(xq_dev, a_dev, packed, w_scale, dt) for dt in ("f32", "bf16", "i32")}
        outs = {dt: to_np(v) for dt, v in outs.items()}
        assert np.array_equal(to_np(a_dev), a_ref), f"a_scale M={M}"
        assert np.array_equal(to_np(xq_dev), xq_ref), f"xq M={M}"
        t0 = time.perf_counter()
        acc = oracle.accumulate(xq_ref, p_ref, K)
        ref, _, _ = oracle.rescale(acc, a_ref, s_ref)
        t_oracle = time.perf_counter() - t0
        for dt, out in outs.items():
            check_out(out, acc, ref, dt, f"{wl} {name} M={M} {dt} full")
        print(f"  M={M} ok (oracle {t_oracle:.1f} s)", flush=True)


def b3_cases():
    out = []
    for wl in ("2b_decode", "8b_sweep", "70b_chain"):
        for name, N, K in workloads.distinct_shapes(workloads.WORKLOADS[wl]["layer"]):
            out.append(pytest.param(N, K, id=f"{wl}-{name}-{N}x{K}"))
    return out


@pytest.mark.parametrize("N,K", b3_cases())
def test_b3_decode_shape(N, K):
    # the five-per-byte weights of every decode shape at M = 1, whole output compared
    print(f"\n[b3] N={N} K={K}", flush=True)
    W = workloads.latent_weights(N, K, seed=0)
    p_ref, s_ref = oracle.pack_weights(W.numpy())
    packed, w_scale = bw.pack_weights(W.cuda())
    del W
    b3 = bw.pack_b3(packed, K)
    b3_ref = oracle.pack_b3(oracle.unpack(p_ref, K))
    assert np.array_equal(to_np(b3), b3_ref), "b3 bytes"
    X = workloads.activations(1, K, seed=0, outliers=True)
    xq_ref, a_ref = oracle.act_quant(workloads.bf16_bits(X))
    acc = oracle.accumulate_b3(xq_ref, b3_ref, K)
    ref, _, _ = oracle.rescale(acc, a_ref, s_ref)
    for dt in ("f32", "bf16", "i32"):
        out = to_np(bw.quant_gemv_b3(X.cuda(), b3, w_scale, dt))
        check_out(out, acc, ref, dt, f"b3 {N}x{K} {dt}")
