"""The arithmetic that the multi-GPU design relies on, checked on the CPU oracle (no
collectives run here: one GPU per box).

* Tensor parallel along N: each shard owns output rows and their weight scales; its
  outputs are the matching columns of the unsharded product, bit for bit.
* Tensor parallel along K: each shard owns a K slice (whole packed bytes, K/4 columns of
  the packed array).  With the per-token amax taken over the whole row (an all-reduce MAX
  of the shards' row maxima) every shard quantizes its slice to the same codes as the
  unsharded quantization, and the int32 sum of the shards' accumulators -- in any order,
  as a ring or a tree would add them -- is the unsharded accumulator exactly, so the
  rescaled outputs are bit-identical too.  Without the MAX exchange the codes differ.
"""
import numpy as np
import pytest

import oracle
import workloads

M, N, K = 4, 96, 1024


@pytest.fixture(scope="module")
def problem():
    X = workloads.activations(M, K, seed=7, outliers=True)
    W = workloads.latent_weights(N, K, seed=8).numpy()
    bits = workloads.bf16_bits(X)
    packed, w_scale = oracle.pack_weights(W)
    xq, a_scale = oracle.act_quant(bits)
    acc = oracle.accumulate(xq, packed, K)
    _, f32, bf16 = oracle.rescale(acc, a_scale, w_scale)
    return dict(bits=bits, packed=packed, w_scale=w_scale, xq=xq, a_scale=a_scale,
                acc=acc, f32=f32, bf16=bf16)


@pytest.mark.parametrize("shards", [2, 3, 8])
def test_tensor_parallel_along_n_is_a_column_split(problem, shards):
    bounds = np.linspace(0, N, shards + 1).astype(int)
    for n0, n1 in zip(bounds[:-1], bounds[1:]):
        acc = oracle.accumulate(problem["xq"], np.ascontiguousarray(problem["packed"][n0:n1]), K)
        assert np.array_equal(acc, problem["acc"][:, n0:n1])
        _, f32, _ = oracle.rescale(acc, problem["a_scale"], problem["w_scale"][n0:n1])
        assert np.array_equal(f32.view(np.uint32), problem["f32"][:, n0:n1].view(np.uint32))


def k_slices(shards):
    # shard boundaries on whole packed bytes (multiples of 4 weights), uneven on purpose
    cuts = sorted({4 * int(c) for c in np.linspace(0, K // 4, shards + 1)[1:-1] + 3})
    return list(zip([0] + cuts, cuts + [K]))


@pytest.mark.parametrize("shards", [2, 3, 8])
def test_tensor_parallel_along_k_is_exact_with_the_amax_exchange(problem, shards):
    bits, packed = problem["bits"], problem["packed"]
    slices = k_slices(shards)
    # each shard's row maxima of |x| (bf16 magnitude bits); the exchange takes their max
    local_max = [np.max(bits[:, k0:k1] & 0x7FFF, axis=1) for k0, k1 in slices]
    assert np.array_equal(np.maximum.reduce(local_max), np.max(bits & 0x7FFF, axis=1))
    partials = []
    for k0, k1 in slices:
        # the shard's codes under the global scale are the global codes of its slice
        xq_local = problem["xq"][:, k0:k1]
        pk = np.ascontiguousarray(packed[:, k0 // 4:k1 // 4])
        partials.append(oracle.accumulate(np.ascontiguousarray(xq_local), pk, k1 - k0))
    orders = [list(range(shards)), list(reversed(range(shards)))]
    for order in orders:
        total = np.zeros_like(problem["acc"])
        for i in order:
            total = total + partials[i]
        assert total.dtype == np.int32
        assert np.array_equal(total, problem["acc"])
    # a pairwise tree of sums
    level = list(partials)
    while len(level) > 1:
        level = [level[i] + level[i + 1] if i + 1 < len(level) else level[i]
                 for i in range(0, len(level), 2)]
    assert np.array_equal(level[0], problem["acc"])
    _, f32, bf16 = oracle.rescale(level[0], problem["a_scale"], problem["w_scale"])
    assert np.array_equal(f32.view(np.uint32), problem["f32"].view(np.uint32))
    assert np.array_equal(bf16, problem["bf16"])


def test_tensor_parallel_along_k_needs_the_amax_exchange(problem):
    # quantizing each slice with its own row maxima gives other codes on some rows: the
    # outlier channels sit in some slices only
    bits = problem["bits"]
    differs = False
    for k0, k1 in k_slices(2):
        xq_local, _ = oracle.act_quant(np.ascontiguousarray(bits[:, k0:k1]))
        differs |= not np.array_equal(xq_local, problem["xq"][:, k0:k1])
    assert differs
