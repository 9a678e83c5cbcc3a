"""CPU oracle for the BitNet b1.58 W2A8 BitLinear matmul -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``
may import this package.  The HIP library never imports, links or calls it, and it
never imports the HIP library: the two share no code.

The arithmetic lives in ``bitnet_oracle.c`` (plain C, scalar loops, each function
citing the page passage it follows).  This module only builds that file with gcc and
marshals numpy arrays into it with ctypes.

Functions and the pages they follow (page titles abbreviated):
  weight_quant  -- "BitNet 深度实战" (chenxutan.com) §2.4: per-row absmean scale, round,
                   clamp to {-1, 0, +1}.
  pack / unpack -- "BitNet-Triton" (zingnex.cn) 技术架构 §1: (N, K/4) uint8; "BitNet 深度实战"
                   §4.3: four weights per byte, first weight in bits 0-1.
  act_quant     -- "BitNet-Triton" 技术架构 §3 / "BitNet 1-bit LLM推理优化" (blog.hotdry.top)
                   §3.2: int8 activations, per-token absmax scale 127/max|x|.
  act_quant_per_tensor -- "BitNet 1-bit LLM推理优化" §2.2 / §3.2: one scale per tensor.
  repack        -- "BitNet 深度实战" §4.3: the page's 00/01/11 code table <-> code = w + 1.
  accumulate    -- "BitNet 深度实战" §4.4: int8 x ternary into int32.
  rescale       -- "BitNet 深度实战" §2.4 / §3.2: out = acc * w_scale / a_scale.
  swiglu        -- "BitNet 深度实战" §3.2: the MLP's silu(gate(x)) * up(x).
  a16           -- "将 BitNet 三元查找表集成到自定义 Triton 内核中" / "BitNet 深度实战" §2.2:
                   16-bit activations times ternary weights, no activation quantization.
  pack_b3 / unpack_b3 / accumulate_b3 -- "将 BitNet 三元查找表集成到自定义 Triton 内核中"
                   (4-5 ternary values per byte) / "BitNet 1-bit LLM推理优化" §2.1: five
                   weights per byte in base 3, 1.6 bits per weight.

Every function is pinned by tests/test_oracle_pins.py (worked example, closed forms,
invariants, library matmul on unpacked codes, brute force on tiny inputs).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bitnet_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

_lib = None
_lock = threading.Lock()


def build(force: bool = True) -> str:
    """Compile bitnet_oracle.c into liboracle.so with gcc (no fast-math, no contraction)."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
           "-fexcess-precision=standard", "-fopenmp", "-fPIC", "-shared",
           "-o", tmp, _SRC, "-lm"]
    subprocess.check_call(cmd)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        override = os.environ.get("BITNET_ORACLE_LIB")
        if override:
            # used only by tests/test_oracle_mutations.py to run the pins against a
            # deliberately broken copy of the oracle
            lib = ctypes.CDLL(override)
        else:
            stale = (not os.path.exists(_LIB_PATH)
                     or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC))
            if stale:
                build(force=True)
            lib = ctypes.CDLL(_LIB_PATH)
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        sig = {
            "oracle_weight_quant": [p, i64, i64, p, p],
            "oracle_pack": [p, i64, i64, p],
            "oracle_unpack": [p, i64, i64, p],
            "oracle_act_quant": [p, i64, i64, p, p],
            "oracle_accumulate": [p, p, i64, i64, i64, p],
            "oracle_rescale": [p, p, p, i64, i64, p, p, p],
            "oracle_f64_to_bf16": [p, i64, p],
            "oracle_swiglu": [p, p, i64, p],
            "oracle_act_quant_per_tensor": [p, i64, i64, p, p],
            "oracle_a16": [p, p, p, i64, i64, i64, p, p],
            "oracle_pack_b3": [p, i64, i64, p],
            "oracle_unpack_b3": [p, i64, i64, p],
            "oracle_accumulate_b3": [p, p, i64, i64, i64, p],
        }
        for name, args in sig.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int if name != "oracle_f64_to_bf16" else None
        lib.oracle_repack.argtypes = [p, i64, i64, ctypes.c_int, ctypes.c_int, p]
        lib.oracle_repack.restype = i64
        lib.oracle_b3_row_bytes.argtypes = [i64]
        lib.oracle_b3_row_bytes.restype = i64
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ctypes.c_int
        _lib = lib
        return lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return ctypes.c_void_p(a.ctypes.data)


class OracleError(RuntimeError):
    pass


def _check(rc: int, what: str):
    if rc != 0:
        raise OracleError(f"{what} returned {rc}")


def num_threads() -> int:
    return int(_load().oracle_num_threads())


# --------------------------------------------------------------------------- O1


def weight_quant(W: np.ndarray):
    """Per-row absmean ternarization. W: float32 (N, K), any K >= 1.

    Returns (q int8 (N, K) in {-1, 0, 1}, scale float32 (N,))."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    q = np.empty((N, K), np.int8)
    s = np.empty((N,), np.float32)
    _check(_load().oracle_weight_quant(_ptr(W), N, K, _ptr(q), _ptr(s)), "weight_quant")
    return q, s


def pack(q: np.ndarray) -> np.ndarray:
    """Ternary codes int8 (N, K) -> packed uint8 (N, K/4), code = w + 1, low bits first."""
    q = np.ascontiguousarray(q, dtype=np.int8)
    N, K = q.shape
    out = np.empty((N, K // 4), np.uint8)
    _check(_load().oracle_pack(_ptr(q), N, K, _ptr(out)), "pack")
    return out


def unpack(packed: np.ndarray, K: int) -> np.ndarray:
    """Packed uint8 (N, K/4) -> int8 (N, K).  Raises if a field holds the unused code."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    N = packed.shape[0]
    q = np.empty((N, K), np.int8)
    _check(_load().oracle_unpack(_ptr(packed), N, K, _ptr(q)), "unpack")
    return q


def pack_weights(W: np.ndarray):
    """O1 + pack: float32 (N, K) -> (packed uint8 (N, K/4), scale float32 (N,))."""
    q, s = weight_quant(W)
    return pack(q), s


# ------------------------------------------------ five weights per byte (1.6 bits)


def b3_row_bytes(K: int) -> int:
    """Bytes per row of the five-per-byte format: K padded to a multiple of 320, / 5."""
    r = int(_load().oracle_b3_row_bytes(int(K)))
    if r < 0:
        raise OracleError("b3_row_bytes: bad K")
    return r


def pack_b3(q: np.ndarray) -> np.ndarray:
    """Ternary codes int8 (N, K) -> (N, b3_row_bytes(K)) uint8, five weights per byte
    ("将 BitNet 三元查找表集成到自定义 Triton 内核中": 4-5 ternary values per byte;
    "BitNet 1-bit LLM推理优化" §2.1: below 2 bits per weight)."""
    q = np.ascontiguousarray(q, dtype=np.int8)
    N, K = q.shape
    out = np.empty((N, b3_row_bytes(K)), np.uint8)
    _check(_load().oracle_pack_b3(_ptr(q), N, K, _ptr(out)), "pack_b3")
    return out


def unpack_b3(b3: np.ndarray, K: int) -> np.ndarray:
    """Inverse of pack_b3 -> int8 (N, K); raises if a padding weight is not 0."""
    b3 = np.ascontiguousarray(b3, dtype=np.uint8)
    N = b3.shape[0]
    assert b3.shape[1] == b3_row_bytes(K)
    q = np.empty((N, K), np.int8)
    _check(_load().oracle_unpack_b3(_ptr(b3), N, K, _ptr(q)), "unpack_b3")
    return q


def accumulate_b3(xq: np.ndarray, b3: np.ndarray, K: int) -> np.ndarray:
    """acc[m, n] = sum_k xq[m, k] * w[n, k] with w decoded from the five-per-byte format."""
    xq = np.ascontiguousarray(xq, dtype=np.int8)
    b3 = np.ascontiguousarray(b3, dtype=np.uint8)
    M, N = xq.shape[0], b3.shape[0]
    assert xq.shape[1] == K and b3.shape[1] == b3_row_bytes(K)
    acc = np.empty((M, N), np.int32)
    _check(_load().oracle_accumulate_b3(_ptr(xq), _ptr(b3), M, N, K, _ptr(acc)), "accumulate_b3")
    return acc


# --------------------------------------------------------------------------- O2


def act_quant(x_bf16_bits: np.ndarray):
    """Per-token absmax int8 quantization.

    x_bf16_bits: uint16 (M, K) holding bf16 bit patterns.
    Returns (xq int8 (M, K), a_scale float32 (M,) = 127 / max|x|)."""
    x = np.ascontiguousarray(x_bf16_bits, dtype=np.uint16)
    M, K = x.shape
    xq = np.empty((M, K), np.int8)
    a = np.empty((M,), np.float32)
    rc = _load().oracle_act_quant(_ptr(x), M, K, _ptr(xq), _ptr(a))
    if rc == 1:
        raise OracleError("act_quant: the +-127 clamp fired, which the definition rules out")
    _check(rc, "act_quant")
    return xq, a


# --------------------------------------------------------------------------- O3


def act_quant_per_tensor(x_bf16_bits: np.ndarray):
    """One int8 scale for the whole (M, K) tensor ("BitNet 1-bit LLM推理优化" §2.2, §3.2).

    Returns (xq int8 (M, K), a_scale float32 (M,), every entry 127 / max|x|)."""
    x = np.ascontiguousarray(x_bf16_bits, dtype=np.uint16)
    M, K = x.shape
    xq = np.empty((M, K), np.int8)
    a = np.empty((M,), np.float32)
    rc = _load().oracle_act_quant_per_tensor(_ptr(x), M, K, _ptr(xq), _ptr(a))
    if rc == 1:
        raise OracleError("act_quant_per_tensor: the +-127 clamp fired, which the definition "
                          "rules out")
    _check(rc, "act_quant_per_tensor")
    return xq, a


CODES_OFFSET, CODES_SIGN = 0, 1


def repack(packed: np.ndarray, K: int, from_table: int, to_table: int):
    """Rewrite packed (N, K/4) bytes between the code tables ("BitNet 深度实战" §4.3).

    Returns (out uint8 (N, K/4), number of fields that held the source's unused code)."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    N = packed.shape[0]
    out = np.empty_like(packed)
    bad = _load().oracle_repack(_ptr(packed), N, K, int(from_table), int(to_table), _ptr(out))
    if bad < 0:
        raise OracleError("repack: bad arguments")
    return out, int(bad)


def accumulate(xq: np.ndarray, packed: np.ndarray, K: int) -> np.ndarray:
    """acc[m, n] = sum_k xq[m, k] * w[n, k] in exact integer arithmetic -> int32 (M, N)."""
    xq = np.ascontiguousarray(xq, dtype=np.int8)
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    M = xq.shape[0]
    N = packed.shape[0]
    assert xq.shape[1] == K and packed.shape[1] * 4 == K
    acc = np.empty((M, N), np.int32)
    _check(_load().oracle_accumulate(_ptr(xq), _ptr(packed), M, N, K, _ptr(acc)), "accumulate")
    return acc


# --------------------------------------------------------------------------- O4


def rescale(acc: np.ndarray, a_scale: np.ndarray, w_scale: np.ndarray):
    """Returns (ref float64, out_f32 float32, out_bf16 uint16 bit patterns), all (M, N)."""
    acc = np.ascontiguousarray(acc, dtype=np.int32)
    a_scale = np.ascontiguousarray(a_scale, dtype=np.float32)
    w_scale = np.ascontiguousarray(w_scale, dtype=np.float32)
    M, N = acc.shape
    ref = np.empty((M, N), np.float64)
    f32 = np.empty((M, N), np.float32)
    bf = np.empty((M, N), np.uint16)
    _check(_load().oracle_rescale(_ptr(acc), _ptr(a_scale), _ptr(w_scale), M, N, _ptr(ref),
                                  _ptr(f32), _ptr(bf)), "rescale")
    return ref, f32, bf


def a16(x_bf16_bits: np.ndarray, packed: np.ndarray, w_scale: np.ndarray, K: int):
    """O6: bf16 activations times the packed ternary weights, no activation quantization
    ("将 BitNet 三元查找表集成到自定义 Triton 内核中", mixed-precision serving; "BitNet 深度实战"
    §2.2).  Returns (ref fp64 (M, N) = w_scale[n] * sum_k x w, sumabs fp64 (M, N) =
    w_scale[n] * sum_k |x w|)."""
    x = np.ascontiguousarray(x_bf16_bits, dtype=np.uint16)
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    w_scale = np.ascontiguousarray(w_scale, dtype=np.float32)
    M = x.shape[0]
    N = packed.shape[0]
    ref = np.empty((M, N), np.float64)
    sa = np.empty((M, N), np.float64)
    _check(_load().oracle_a16(_ptr(x), _ptr(packed), _ptr(w_scale), M, N, K, _ptr(ref), _ptr(sa)),
           "a16")
    return ref, sa


def swiglu(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """O5: h = silu(g) * u = g / (1 + exp(-g)) * u in fp64, elementwise ("BitNet 深度实战"
    §3.2, the MLP's act_fn(gate(x)) * up(x) with act_fn = F.silu)."""
    g = np.ascontiguousarray(g, dtype=np.float64)
    u = np.ascontiguousarray(u, dtype=np.float64)
    if g.shape != u.shape:
        raise ValueError("g and u must have the same shape")
    h = np.empty(g.shape, np.float64)
    _check(_load().oracle_swiglu(_ptr(g), _ptr(u), g.size, _ptr(h)), "swiglu")
    return h


def f64_to_bf16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, np.uint16)
    _load().oracle_f64_to_bf16(_ptr(x), x.size, _ptr(out))
    return out


# ------------------------------------------------------------------ whole layer


def bitlinear(x_bf16_bits: np.ndarray, W: np.ndarray):
    """The whole forward: act quant, weight quant + pack, accumulate, rescale.

    Returns a dict with every intermediate the GPU path exposes."""
    packed, w_scale = pack_weights(W)
    xq, a_scale = act_quant(x_bf16_bits)
    K = W.shape[1]
    acc = accumulate(xq, packed, K)
    ref, f32, bf = rescale(acc, a_scale, w_scale)
    return dict(packed=packed, w_scale=w_scale, xq=xq, a_scale=a_scale, acc=acc, ref=ref,
                out_f32=f32, out_bf16=bf)
