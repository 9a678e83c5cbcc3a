"""The allocation-free product, bitnet_w2a8_gemm_noalloc, through the C ABI: on the GPU
its outputs must equal those of bitnet_w2a8_gemm (with its own workspace) bit for bit
and match the oracle to the usual bar (int32 exact, fp32 within 1e-6 relative, bf16
within 1 ulp), over consecutive calls that share the library's fixed scratch -- the
second one smaller than the first -- and over graph replays."""
import numpy as np
import pytest
import torch

import ternary_weight_linear_token_amd as bw
from gpu_helpers import Problem, check_out, to_np

pytestmark = pytest.mark.gpu

DT = ["f32", "bf16", "i32"]


def inputs(M, N, K, seed):
    pb = Problem(M, N, K, seed=seed)
    o = pb.oracle()
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return dev(o["xq"]), dev(o["a_scale"]), dev(o["packed"]), dev(o["w_scale"]), o


def test_noalloc_matches_gemm_on_consecutive_calls():
    # a product that splits K over 6 slices (6 MB of partials), then a smaller one that
    # splits over 10 and overwrites only the start of the scratch, then one that does
    # not split (the weight-streaming route of ALGO_AUTO)
    for M, N, K, algo in ((64, 4096, 14336, "tiled"), (17, 300, 2560, "tiled"),
                          (5, 2000, 2048, "auto")):
        if algo == "tiled":
            assert bw.gemm_plan(M, K, [N])[4] > 1, "expected a split plan"
        xq, a, packed, s, o = inputs(M, N, K, seed=M + N + K)
        for dt in DT:
            want = bw.gemm(xq, a, packed, s, dt, algo=algo)
            got = torch.full_like(want, 7)
            bw.gemm_noalloc(xq, a, packed, s, dt, algo=algo, out=got)
            torch.cuda.synchronize()
            assert torch.equal(got, want), f"noalloc differs from gemm {M}x{N}x{K} {dt}"
            check_out(to_np(got), o["acc"], o["ref"], dt, f"noalloc {M}x{N}x{K} {dt}")


def test_noalloc_in_graph_replays():
    # captured once (nothing is allocated inside the capture), replayed with eager work
    # in between; every replay is checked
    M, N, K = 32, 8192, 4096
    xq, a, packed, s, o = inputs(M, N, K, seed=9)
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        bw.gemm_noalloc(xq, a, packed, s, "bf16", algo="tiled", out=out)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        bw.gemm_noalloc(xq, a, packed, s, "bf16", algo="tiled", out=out)
    other = inputs(17, 300, 2560, seed=3)
    for rep in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        check_out(to_np(out), o["acc"], o["ref"], "bf16", f"noalloc graph replay {rep}")
        bw.gemm_noalloc(*other[:4], "f32", algo="tiled")  # eager use of the same scratch
        torch.cuda.synchronize()
