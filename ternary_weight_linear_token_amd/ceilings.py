"""What this chip sustains, measured: the int8 matrix-core rate on register operands and
the streaming HBM read rate (libbitnet_probes.so), plus the vendor int8 GEMM
(hipBLASLt through torch._int_mm) at a given shape.  Context for the roofline
fractions; not part of the BitLinear path."""
from __future__ import annotations

import ctypes
import os

from . import build as _build

_lib = None


def _probes():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.PROBES_LIB):
            _build.build_probes()
        L = ctypes.CDLL(_build.PROBES_LIB)
        p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.bitnet_probe_mfma_i8.argtypes = [p, p, p, i32, i32, p]
        L.bitnet_probe_mfma_i8.restype = i32
        L.bitnet_probe_mfma_i8_ops.argtypes = [i32, i32]
        L.bitnet_probe_mfma_i8_ops.restype = ctypes.c_double
        L.bitnet_probe_wall_clock_hz.argtypes = []
        L.bitnet_probe_wall_clock_hz.restype = ctypes.c_double
        L.bitnet_probe_read.argtypes = [p, i64, p, i32, p]
        L.bitnet_probe_read.restype = i32
        _lib = L
    return _lib


def _time_us(torch, fn, reps):
    fn()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        fn()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) * 1e3 / reps


def mfma_i8_tops(torch, dev, blocks=2048, iters=2000, reps=5):
    """int8 MFMA throughput (TOPS) of a register-only loop, seeded random operands, and the
    core clock (GHz) the waves sustained during it (median over waves of core cycles per
    wall-counter tick times the wall counter's rate; None if the rate is unknown)."""
    L = _probes()
    g = torch.Generator().manual_seed(1)
    seed = torch.randint(-2**31, 2**31 - 1, (4096,), generator=g, dtype=torch.int64)
    seed = seed.to(torch.int32).to(dev)
    out = torch.empty((blocks * 256,), dtype=torch.int32, device=dev)
    clk = torch.zeros((blocks * 4 * 2,), dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream

    def run():
        rc = L.bitnet_probe_mfma_i8(seed.data_ptr(), out.data_ptr(), clk.data_ptr(), blocks,
                                    iters, stream)
        if rc:
            raise RuntimeError(f"bitnet_probe_mfma_i8: hip error {rc}")

    us = _time_us(torch, run, reps)
    c = clk.view(-1, 2).cpu().double()
    wall_hz = L.bitnet_probe_wall_clock_hz()
    ghz = None
    if wall_hz > 0 and bool((c[:, 1] > 0).all()):
        ghz = float((c[:, 0] / c[:, 1]).median()) * wall_hz / 1e9
    return L.bitnet_probe_mfma_i8_ops(blocks, iters) / us / 1e6, ghz


def hbm_read_gbs(torch, dev, nbytes=2 << 30, blocks=2048, reps=5):
    """Streaming read rate (GB/s) over an nbytes buffer (several times the 256 MB
    Infinity Cache, so the bytes come from HBM)."""
    L = _probes()
    buf = torch.ones((nbytes // 4,), dtype=torch.int32, device=dev)
    out = torch.empty((blocks * 256,), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream

    def run():
        rc = L.bitnet_probe_read(buf.data_ptr(), nbytes // 16, out.data_ptr(), blocks, stream)
        if rc:
            raise RuntimeError(f"bitnet_probe_read: hip error {rc}")

    us = _time_us(torch, run, reps)
    del buf
    return nbytes / us / 1e3


def same_grid_read_us(torch, dev, nbytes, blocks, graph_us, rotate_bytes=1 << 30):
    """Per-launch time (us) of the plain streaming read of nbytes with `blocks` blocks of
    256 threads (each block over its own contiguous share): the floor of any launch that
    reads those bytes with that grid.  Buffers rotate over rotate_bytes so the bytes come
    from HBM; graph_us(launch(r), R) times R back-to-back launches the way the product
    kernels are timed."""
    L = _probes()
    n16 = max(1, nbytes // 16)
    stride = n16 * 16
    R = max(4, min(256, rotate_bytes // stride))
    buf = torch.ones((R * stride // 4,), dtype=torch.int32, device=dev)
    out = torch.empty((blocks * 256,), dtype=torch.int32, device=dev)

    def launch(r):
        stream = torch.cuda.current_stream(dev).cuda_stream
        rc = L.bitnet_probe_read(buf.data_ptr() + (r % R) * stride, n16, out.data_ptr(),
                                 blocks, stream)
        if rc:
            raise RuntimeError(f"bitnet_probe_read: hip error {rc}")

    us = graph_us(launch, R)
    del buf
    return us


def vendor_int8_gemm_tops(torch, dev, M, N, K, reps=10):
    """hipBLASLt int8 GEMM (torch._int_mm) on dense int8 operands: xq (M, K) times
    codes^T with codes (N, K) in {-1, 0, 1}; TOPS, or None if unavailable."""
    g = torch.Generator().manual_seed(2)
    a = torch.randint(-127, 128, (M, K), generator=g, dtype=torch.int8).to(dev)
    b = torch.randint(-1, 2, (N, K), generator=g, dtype=torch.int8).to(dev)
    try:
        us = _time_us(torch, lambda: torch._int_mm(a, b.t()), reps)
    except RuntimeError:
        return None
    return 2.0 * M * N * K / us / 1e6
