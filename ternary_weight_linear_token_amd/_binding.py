"""ctypes binding of libbitnet_w2a8.so: names mirror the C ABI in include/bitnet_w2a8.h.

Marshalling only: tensors are checked (device, dtype, shape, contiguity) and their
device pointers and the current HIP stream are handed to the library.  Outputs are
allocated with torch unless passed in.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

from . import build as _build

OUT_F32, OUT_BF16, OUT_I32 = 0, 1, 2
ALGO_AUTO, ALGO_SKINNY, ALGO_TILED = 0, 1, 2
GEMV_MAX_M = 16
SKINNY_MAX_M = 64
MAX_GROUPS = 4

_OUT_TORCH = {OUT_F32: torch.float32, OUT_BF16: torch.bfloat16, OUT_I32: torch.int32}
_OUT_NAMES = {"f32": OUT_F32, "float32": OUT_F32, "bf16": OUT_BF16, "bfloat16": OUT_BF16,
              "i32": OUT_I32, "int32": OUT_I32}
_ALGO_NAMES = {"auto": ALGO_AUTO, "skinny": ALGO_SKINNY, "tiled": ALGO_TILED}

_lib = None
_lock = threading.Lock()


class BitnetError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        detail = status_str(status)
        if status == 4:
            detail += ": " + lib().bitnet_last_hip_error().decode()
        super().__init__(f"{what}: {detail} (status {status})")


def library_path() -> str:
    return _build.LIB_PATH


def lib():
    """Load libbitnet_w2a8.so, building it first if it is missing or out of date."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        override = os.environ.get("BITNET_LIBRARY")
        if override:
            # a differently built copy of the same sources (the sanitizer build of the
            # host-side validation layer, run by tests/test_sanitized_boundary.py)
            L = ctypes.CDLL(override)
        else:
            if not _build.is_current():
                _build.build()
            L = ctypes.CDLL(_build.LIB_PATH)
        p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        sigs = {
            "bitnet_abi_version": ([], i32),
            "bitnet_status_str": ([i32], ctypes.c_char_p),
            "bitnet_last_hip_error": ([], ctypes.c_char_p),
            "bitnet_pack_weights": ([p, i64, i64, p, p, p], i32),
            "bitnet_unpack_weights": ([p, i64, i64, p, p], i32),
            "bitnet_quant_act": ([p, i64, i64, p, p, p], i32),
            "bitnet_w2a8_gemv": ([p, p, p, p, i64, i64, i64, p, i32, p], i32),
            "bitnet_w2a8_gemm_workspace_size": ([i64, i64, i64], ctypes.c_size_t),
            "bitnet_w2a8_gemm": ([p, p, p, p, i64, i64, i64, p, i32, i32, p, ctypes.c_size_t, p], i32),
            "bitnet_quant_gemv": ([p, p, p, i64, i64, i64, p, i32, p, p, p], i32),
            "bitnet_quant_gemv_grouped": ([p, i64, i64, i64, p, p, p, p, i32, p, p, p], i32),
            "bitnet_w2a8_gemm_grouped": ([p, p, i64, i64, i64, p, p, p, p, i32, p], i32),
            "bitnet_w2a8_gemm_noalloc": ([p, p, p, p, i64, i64, i64, p, i32, i32, p], i32),
            "bitnet_w2a8_gemm_plan": ([i64, i64, i64, p, i64, p], i32),
            "bitnet_quant_gemv_swiglu": ([p, p, p, p, p, i64, i64, i64, p, i32, p, p, p], i32),
            "bitnet_quant_act_per_tensor": ([p, i64, i64, p, p, p], i32),
            "bitnet_a16_gemv": ([p, p, p, i64, i64, i64, p, i32, p], i32),
            "bitnet_repack_codes": ([p, i64, i64, i32, i32, p, p, p], i32),
            "bitnet_pack_b3": ([p, i64, i64, p, p], i32),
            "bitnet_quant_gemv_b3": ([p, p, p, i64, i64, i64, p, i32, p], i32),
        }
        for name, (args, res) in sigs.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
        return L


def abi_version() -> int:
    return int(lib().bitnet_abi_version())


def status_str(status: int) -> str:
    return lib().bitnet_status_str(int(status)).decode()


def _check(status: int, what: str):
    if status != 0:
        raise BitnetError(status, what)


def _out_code(out_dtype) -> int:
    if isinstance(out_dtype, int):
        return out_dtype
    if isinstance(out_dtype, torch.dtype):
        for k, v in _OUT_TORCH.items():
            if v == out_dtype:
                return k
    return _OUT_NAMES[str(out_dtype)]


def _tensor(t: torch.Tensor, dtype, name: str, shape=None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor (the library has no CPU path)")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr()


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _opt_ptr(t, dtype, name, shape):
    return None if t is None else _tensor(t, dtype, name, shape)


def pack_weights(w: torch.Tensor, packed: torch.Tensor | None = None,
                 w_scale: torch.Tensor | None = None):
    """fp32 (N, K) latent weights -> (packed uint8 (N, K/4), w_scale fp32 (N,))."""
    N, K = w.shape
    if packed is None:
        packed = torch.empty((N, K // 4), dtype=torch.uint8, device=w.device)
    if w_scale is None:
        w_scale = torch.empty((N,), dtype=torch.float32, device=w.device)
    _check(lib().bitnet_pack_weights(_tensor(w, torch.float32, "w", (N, K)), N, K,
                                     _tensor(packed, torch.uint8, "packed", (N, K // 4)),
                                     _tensor(w_scale, torch.float32, "w_scale", (N,)), _stream(w)),
           "bitnet_pack_weights")
    return packed, w_scale


def unpack_weights(packed: torch.Tensor, K: int, codes: torch.Tensor | None = None):
    """packed uint8 (N, K/4) -> int8 codes (N, K) in {-1, 0, 1}."""
    N = packed.shape[0]
    if codes is None:
        codes = torch.empty((N, K), dtype=torch.int8, device=packed.device)
    _check(lib().bitnet_unpack_weights(_tensor(packed, torch.uint8, "packed", (N, K // 4)), N, K,
                                       _tensor(codes, torch.int8, "codes", (N, K)), _stream(packed)),
           "bitnet_unpack_weights")
    return codes


def quant_act(x: torch.Tensor, xq: torch.Tensor | None = None,
              a_scale: torch.Tensor | None = None):
    """bf16 (M, K) -> (xq int8 (M, K), a_scale fp32 (M,) = 127 / max|x|)."""
    M, K = x.shape
    if xq is None:
        xq = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if a_scale is None:
        a_scale = torch.empty((M,), dtype=torch.float32, device=x.device)
    _check(lib().bitnet_quant_act(_tensor(x, torch.bfloat16, "x", (M, K)), M, K,
                                  _tensor(xq, torch.int8, "xq", (M, K)),
                                  _tensor(a_scale, torch.float32, "a_scale", (M,)), _stream(x)),
           "bitnet_quant_act")
    return xq, a_scale


def quant_act_per_tensor(x: torch.Tensor, xq: torch.Tensor | None = None,
                         a_scale: torch.Tensor | None = None):
    """bf16 (M, K) -> (int8 (M, K), fp32 (M,)) with one scale for the whole tensor."""
    M, K = x.shape
    if xq is None:
        xq = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if a_scale is None:
        a_scale = torch.empty((M,), dtype=torch.float32, device=x.device)
    _check(lib().bitnet_quant_act_per_tensor(_tensor(x, torch.bfloat16, "x", (M, K)), M, K,
                                             _tensor(xq, torch.int8, "xq", (M, K)),
                                             _tensor(a_scale, torch.float32, "a_scale", (M,)),
                                             _stream(x)),
           "bitnet_quant_act_per_tensor")
    return xq, a_scale


CODES_OFFSET, CODES_SIGN = 0, 1


def repack_codes(packed: torch.Tensor, K: int, from_table: int, to_table: int,
                 out: torch.Tensor | None = None, invalid_count: torch.Tensor | None = None):
    """Rewrite a packed (N, K/4) array from one 2-bit code table to the other."""
    N = packed.shape[0]
    if out is None:
        out = torch.empty_like(packed)
    _check(lib().bitnet_repack_codes(_tensor(packed, torch.uint8, "packed", (N, K // 4)), N, K,
                                     int(from_table), int(to_table),
                                     _tensor(out, torch.uint8, "out", (N, K // 4)),
                                     _opt_ptr(invalid_count, torch.int32, "invalid_count", (1,)),
                                     _stream(packed)),
           "bitnet_repack_codes")
    return out


def _alloc_out(out, M, N, code, device):
    if out is None:
        out = torch.empty((M, N), dtype=_OUT_TORCH[code], device=device)
    return out


def gemv(xq, a_scale, packed, w_scale, out_dtype="f32", out=None):
    """Decode-sized product (M <= 16): int8 xq x packed ternary -> (M, N)."""
    M, K = xq.shape
    N = packed.shape[0]
    code = _out_code(out_dtype)
    out = _alloc_out(out, M, N, code, xq.device)
    _check(lib().bitnet_w2a8_gemv(_tensor(xq, torch.int8, "xq", (M, K)),
                                  _tensor(a_scale, torch.float32, "a_scale", (M,)),
                                  _tensor(packed, torch.uint8, "packed", (N, K // 4)),
                                  _tensor(w_scale, torch.float32, "w_scale", (N,)), M, N, K,
                                  _tensor(out, _OUT_TORCH[code], "out", (M, N)), code, _stream(xq)),
           "bitnet_w2a8_gemv")
    return out


def gemm(xq, a_scale, packed, w_scale, out_dtype="f32", algo="auto", out=None, workspace=None):
    """Product for any M: int8 xq x packed ternary -> (M, N).

    workspace: a uint8 device tensor the call may use to split K across blocks (int32
    partial sums); by default one of the size the library asks for
    (bitnet_w2a8_gemm_workspace_size) is allocated when that size is not 0.  Pass
    workspace=False to run without one (unsplit; the same result)."""
    M, K = xq.shape
    N = packed.shape[0]
    code = _out_code(out_dtype)
    algo_code = _ALGO_NAMES[algo] if isinstance(algo, str) else int(algo)
    out = _alloc_out(out, M, N, code, xq.device)
    stream = _stream(xq)
    if workspace is None:
        ws_need = int(lib().bitnet_w2a8_gemm_workspace_size(M, N, K))
        if ws_need:
            workspace = torch.empty((ws_need,), dtype=torch.uint8, device=xq.device)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None and workspace is not False:
        ws_ptr = _tensor(workspace, torch.uint8, "workspace")
        ws_bytes = workspace.numel()
    _check(lib().bitnet_w2a8_gemm(_tensor(xq, torch.int8, "xq", (M, K)),
                                  _tensor(a_scale, torch.float32, "a_scale", (M,)),
                                  _tensor(packed, torch.uint8, "packed", (N, K // 4)),
                                  _tensor(w_scale, torch.float32, "w_scale", (N,)), M, N, K,
                                  _tensor(out, _OUT_TORCH[code], "out", (M, N)), code, algo_code,
                                  ws_ptr, ws_bytes, stream),
           "bitnet_w2a8_gemm")
    return out


def gemm_noalloc(xq, a_scale, packed, w_scale, out_dtype="f32", algo="auto", out=None):
    """gemm through the entry point that allocates nothing: split-K partials go to the
    library's fixed device scratch (calls on one GPU must not overlap).  Pass `out` to
    keep the call free of torch allocations as well."""
    M, K = xq.shape
    N = packed.shape[0]
    code = _out_code(out_dtype)
    algo_code = _ALGO_NAMES[algo] if isinstance(algo, str) else int(algo)
    out = _alloc_out(out, M, N, code, xq.device)
    _check(lib().bitnet_w2a8_gemm_noalloc(_tensor(xq, torch.int8, "xq", (M, K)),
                                          _tensor(a_scale, torch.float32, "a_scale", (M,)),
                                          _tensor(packed, torch.uint8, "packed", (N, K // 4)),
                                          _tensor(w_scale, torch.float32, "w_scale", (N,)), M, N,
                                          K, _tensor(out, _OUT_TORCH[code], "out", (M, N)), code,
                                          algo_code, _stream(xq)),
           "bitnet_w2a8_gemm_noalloc")
    return out


def gemm_grouped(xq, a_scale, packed, w_scale, out_dtype="f32", out=None):
    """Tiled product for up to MAX_GROUPS weight matrices that read the same xq, one launch.

    packed / w_scale: sequences of equal length; returns the list of (M, N_g) outputs."""
    M, K = xq.shape
    G = len(packed)
    if len(w_scale) != G:
        raise ValueError("packed and w_scale must have the same length")
    code = _out_code(out_dtype)
    Ns = [int(pk.shape[0]) for pk in packed]
    outs = list(out) if out is not None else [None] * G
    if len(outs) != G:
        raise ValueError("out must have one tensor per group")
    outs = [_alloc_out(o, M, n, code, xq.device) for o, n in zip(outs, Ns)]
    P = (ctypes.c_void_p * max(G, 1))(*[_tensor(pk, torch.uint8, f"packed[{g}]", (Ns[g], K // 4))
                                        for g, pk in enumerate(packed)])
    S = (ctypes.c_void_p * max(G, 1))(*[_tensor(sc, torch.float32, f"w_scale[{g}]", (Ns[g],))
                                        for g, sc in enumerate(w_scale)])
    O = (ctypes.c_void_p * max(G, 1))(*[_tensor(o, _OUT_TORCH[code], f"out[{g}]", (M, Ns[g]))
                                        for g, o in enumerate(outs)])
    NN = (ctypes.c_int64 * max(G, 1))(*Ns)
    _check(lib().bitnet_w2a8_gemm_grouped(_tensor(xq, torch.int8, "xq", (M, K)),
                                          _tensor(a_scale, torch.float32, "a_scale", (M,)), M, K,
                                          G, ctypes.cast(P, ctypes.c_void_p),
                                          ctypes.cast(S, ctypes.c_void_p),
                                          ctypes.cast(NN, ctypes.c_void_p),
                                          ctypes.cast(O, ctypes.c_void_p), code, _stream(xq)),
           "bitnet_w2a8_gemm_grouped")
    return outs


def gemm_plan(M, K, Ns, cus=0):
    """Tile plan (block rows, block columns, k-groups, k per stage, K slices) of a tiled
    launch over weight matrices of Ns rows (one matrix: gemm with its workspace; several:
    gemm_grouped, never split); host-only."""
    G = len(Ns)
    NN = (ctypes.c_int64 * max(G, 1))(*[int(n) for n in Ns])
    out = (ctypes.c_int32 * 5)()
    _check(lib().bitnet_w2a8_gemm_plan(int(M), int(K), G, ctypes.cast(NN, ctypes.c_void_p),
                                       int(cus), ctypes.cast(out, ctypes.c_void_p)),
           "bitnet_w2a8_gemm_plan")
    return tuple(int(v) for v in out)


def quant_gemv(x, packed, w_scale, out_dtype="f32", out=None, return_quant=False):
    """Fused per-token int8 quantization + decode product (M <= 16) in one launch."""
    M, K = x.shape
    N = packed.shape[0]
    code = _out_code(out_dtype)
    out = _alloc_out(out, M, N, code, x.device)
    xq = a_scale = None
    if return_quant:
        xq = torch.empty((M, K), dtype=torch.int8, device=x.device)
        a_scale = torch.empty((M,), dtype=torch.float32, device=x.device)
    _check(lib().bitnet_quant_gemv(_tensor(x, torch.bfloat16, "x", (M, K)),
                                   _tensor(packed, torch.uint8, "packed", (N, K // 4)),
                                   _tensor(w_scale, torch.float32, "w_scale", (N,)), M, N, K,
                                   _tensor(out, _OUT_TORCH[code], "out", (M, N)), code,
                                   _opt_ptr(xq, torch.int8, "xq_out", (M, K)),
                                   _opt_ptr(a_scale, torch.float32, "a_scale_out", (M,)), _stream(x)),
           "bitnet_quant_gemv")
    return (out, xq, a_scale) if return_quant else out


def quant_gemv_grouped(x, packed, w_scale, out_dtype="f32", out=None, return_quant=False):
    """quant_gemv for up to MAX_GROUPS weight matrices that read the same x, one launch.

    packed / w_scale: sequences of equal length; returns the list of (M, N_g) outputs."""
    M, K = x.shape
    G = len(packed)
    if len(w_scale) != G:
        raise ValueError("packed and w_scale must have the same length")
    code = _out_code(out_dtype)
    Ns = [int(pk.shape[0]) for pk in packed]
    outs = list(out) if out is not None else [None] * G
    if len(outs) != G:
        raise ValueError("out must have one tensor per group")
    outs = [_alloc_out(o, M, n, code, x.device) for o, n in zip(outs, Ns)]
    P = (ctypes.c_void_p * max(G, 1))(*[_tensor(pk, torch.uint8, f"packed[{g}]", (Ns[g], K // 4))
                                        for g, pk in enumerate(packed)])
    S = (ctypes.c_void_p * max(G, 1))(*[_tensor(sc, torch.float32, f"w_scale[{g}]", (Ns[g],))
                                        for g, sc in enumerate(w_scale)])
    O = (ctypes.c_void_p * max(G, 1))(*[_tensor(o, _OUT_TORCH[code], f"out[{g}]", (M, Ns[g]))
                                        for g, o in enumerate(outs)])
    NN = (ctypes.c_int64 * max(G, 1))(*Ns)
    xq = a_scale = None
    if return_quant:
        xq = torch.empty((M, K), dtype=torch.int8, device=x.device)
        a_scale = torch.empty((M,), dtype=torch.float32, device=x.device)
    _check(lib().bitnet_quant_gemv_grouped(_tensor(x, torch.bfloat16, "x", (M, K)), M, K, G,
                                           ctypes.cast(P, ctypes.c_void_p),
                                           ctypes.cast(S, ctypes.c_void_p),
                                           ctypes.cast(NN, ctypes.c_void_p),
                                           ctypes.cast(O, ctypes.c_void_p), code,
                                           _opt_ptr(xq, torch.int8, "xq_out", (M, K)),
                                           _opt_ptr(a_scale, torch.float32, "a_scale_out", (M,)),
                                           _stream(x)),
           "bitnet_quant_gemv_grouped")
    return (outs, xq, a_scale) if return_quant else outs


def quant_gemv_swiglu(x, packed_gate, w_scale_gate, packed_up, w_scale_up, out_dtype="bf16",
                      out=None, return_quant=False):
    """silu(x W_gate^T) * (x W_up^T) for M <= 16 in one launch (fused quantization)."""
    M, K = x.shape
    N = packed_gate.shape[0]
    code = _out_code(out_dtype)
    if code == OUT_I32:
        raise ValueError("the SwiGLU output is fp32 or bf16")
    out = _alloc_out(out, M, N, code, x.device)
    xq = a_scale = None
    if return_quant:
        xq = torch.empty((M, K), dtype=torch.int8, device=x.device)
        a_scale = torch.empty((M,), dtype=torch.float32, device=x.device)
    _check(lib().bitnet_quant_gemv_swiglu(
        _tensor(x, torch.bfloat16, "x", (M, K)),
        _tensor(packed_gate, torch.uint8, "packed_gate", (N, K // 4)),
        _tensor(w_scale_gate, torch.float32, "w_scale_gate", (N,)),
        _tensor(packed_up, torch.uint8, "packed_up", (N, K // 4)),
        _tensor(w_scale_up, torch.float32, "w_scale_up", (N,)), M, N, K,
        _tensor(out, _OUT_TORCH[code], "out", (M, N)), code,
        _opt_ptr(xq, torch.int8, "xq_out", (M, K)),
        _opt_ptr(a_scale, torch.float32, "a_scale_out", (M,)), _stream(x)),
        "bitnet_quant_gemv_swiglu")
    return (out, xq, a_scale) if return_quant else out


def a16_gemv(x, packed, w_scale, out_dtype="f32", out=None):
    """bf16 activations (M <= 16) times the packed ternary weights, no activation
    quantization, fp32 accumulation."""
    M, K = x.shape
    N = packed.shape[0]
    code = _out_code(out_dtype)
    if code == OUT_I32:
        raise ValueError("the bf16-activation product is fp32 or bf16")
    out = _alloc_out(out, M, N, code, x.device)
    _check(lib().bitnet_a16_gemv(_tensor(x, torch.bfloat16, "x", (M, K)),
                                 _tensor(packed, torch.uint8, "packed", (N, K // 4)),
                                 _tensor(w_scale, torch.float32, "w_scale", (N,)), M, N, K,
                                 _tensor(out, _OUT_TORCH[code], "out", (M, N)), code, _stream(x)),
           "bitnet_a16_gemv")
    return out


def b3_row_bytes(K: int) -> int:
    """Bytes per row of the five-per-byte (1.6-bit) weight format."""
    return 64 * ((int(K) + 319) // 320)


def pack_b3(packed: torch.Tensor, K: int, out: torch.Tensor | None = None):
    """2-bit packed (N, K/4) -> five-per-byte (N, b3_row_bytes(K)) uint8."""
    N = packed.shape[0]
    RB = b3_row_bytes(K)
    if out is None:
        out = torch.empty((N, RB), dtype=torch.uint8, device=packed.device)
    _check(lib().bitnet_pack_b3(_tensor(packed, torch.uint8, "packed", (N, K // 4)), N, K,
                                _tensor(out, torch.uint8, "b3", (N, RB)), _stream(packed)),
           "bitnet_pack_b3")
    return out


def quant_gemv_b3(x, b3, w_scale, out_dtype="f32", out=None):
    """Fused int8 quantization + product for one token with five-per-byte weights."""
    M, K = x.shape
    N = b3.shape[0]
    code = _out_code(out_dtype)
    out = _alloc_out(out, M, N, code, x.device)
    _check(lib().bitnet_quant_gemv_b3(_tensor(x, torch.bfloat16, "x", (M, K)),
                                      _tensor(b3, torch.uint8, "b3", (N, b3_row_bytes(K))),
                                      _tensor(w_scale, torch.float32, "w_scale", (N,)), M, N, K,
                                      _tensor(out, _OUT_TORCH[code], "out", (M, N)), code,
                                      _stream(x)),
           "bitnet_quant_gemv_b3")
    return out


# The fused launch quantizes the activations in every block of 16 output rows, so its
# cost grows with the bf16 bytes each block re-reads (M * K); past these limits one
# quantization launch followed by the int8 product is faster.
FUSED_MAX_M = 4
FUSED_MAX_MK = 32768


def bitlinear(x, packed, w_scale, out_dtype="f32"):
    """One BitLinear forward: fused quant+GEMV for one token, or a few tokens of a short
    row, else quant + GEMM."""
    M, K = x.shape
    if M == 1 or (M <= FUSED_MAX_M and M * K <= FUSED_MAX_MK):
        return quant_gemv(x, packed, w_scale, out_dtype)
    xq, a_scale = quant_act(x)
    return gemm(xq, a_scale, packed, w_scale, out_dtype)
