"""Comparison helpers for the GPU parity tests (HIP path vs the CPU oracle)."""
import numpy as np
import torch

import oracle
import workloads

# fp32 outputs: relative error bound against the exact (fp64) value.  The kernels form
# (float)acc * w_scale * (1 / a_scale): (float)acc is exact (|acc| < 2^24), and the
# reciprocal and the two products are each one fp32 rounding, so the error is at most
# 3 * 2^-24 ~ 1.8e-7 relative; 1e-6 is the bar the product is held to.
F32_RTOL = 1e-6


def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def bf16_key(bits: np.ndarray) -> np.ndarray:
    """Map bf16 bit patterns onto a monotone integer line (ulp steps)."""
    b = bits.astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def check_out(out_gpu: np.ndarray, acc: np.ndarray, ref: np.ndarray, dtype: str, what: str):
    """Compare one output tensor with the oracle's acc (int32) and ref (fp64)."""
    if dtype == "i32":
        bad = np.flatnonzero(out_gpu.reshape(-1) != acc.reshape(-1))
        assert bad.size == 0, f"{what}: {bad.size} int32 mismatches, first at {bad[:5]}"
        return
    if dtype == "f32":
        g = out_gpu.astype(np.float64)
        err = np.abs(g - ref)
        lim = F32_RTOL * np.abs(ref)
        bad = np.flatnonzero((err > lim).reshape(-1))
        assert bad.size == 0, (f"{what}: {bad.size} fp32 outputs beyond rel {F32_RTOL}; "
                               f"worst rel {np.max(err / np.maximum(np.abs(ref), 1e-300)):.3g}")
        assert np.all(g[acc == 0] == 0.0), f"{what}: acc == 0 must give exactly 0"
        return
    if dtype == "bf16":
        expect = oracle.f64_to_bf16(ref)
        d = np.abs(bf16_key(out_gpu) - bf16_key(expect))
        assert d.max(initial=0) <= 1, f"{what}: bf16 off by {d.max()} ulp"
        assert np.all(out_gpu[acc == 0] & 0x7FFF == 0), f"{what}: acc == 0 must give 0"
        return
    raise ValueError(dtype)


class Problem:
    """One (M, N, K) BitLinear problem: seeded inputs, GPU tensors, oracle results."""

    def __init__(self, M, N, K, seed=0, outliers=True, device="cuda", X=None, W=None):
        self.M, self.N, self.K = M, N, K
        self.X = workloads.activations(M, K, seed=seed, outliers=outliers) if X is None else X
        self.W = workloads.latent_weights(N, K, seed=seed) if W is None else W
        self.xbits = workloads.bf16_bits(self.X)
        self.x_dev = self.X.to(device)
        self.w_dev = self.W.to(device)
        self._oracle = None

    def oracle(self, full=True):
        if self._oracle is None:
            o = {}
            o["packed"], o["w_scale"] = oracle.pack_weights(self.W.numpy())
            o["xq"], o["a_scale"] = oracle.act_quant(self.xbits)
            if full:
                o["acc"] = oracle.accumulate(o["xq"], o["packed"], self.K)
                o["ref"], _, _ = oracle.rescale(o["acc"], o["a_scale"], o["w_scale"])
            self._oracle = o
        return self._oracle
