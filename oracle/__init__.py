"""CPU oracle for the small-M 8-bit quantized GEMM (numpy front end).

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import this package.  The GPU library
(bit_quantized_gemm_token_amd) never imports it, and the two share no code:
the arithmetic lives in oracle/w8_oracle.c, written from its definitions, and
this module only marshals numpy arrays into it.

Definitions follow ai-radar.it, "Helion nel backend vLLM: un solo GEMM, tuning
per forma e guadagni fino al 10%": paragraph 1 names the formats FP8_Dynamic,
W8A8_INT8 and Block_FP8; paragraph 2 says Standard, Split-K and Swap-AB
compute the same GEMM.  The page fixes no granularity, dtype or rounding rule;
the header of w8_oracle.c states the readings used.

Pins: every function here is pinned in tests/test_oracle_*.py against values
the mathematics fixes (exhaustive codec closed forms, Fraction brute force,
numpy integer matmul, closed-form GEMMs).  None is "parity unpinned".
"""
import ctypes
import os

import numpy as np

FP8_DYNAMIC = 0
W8A8_INT8 = 1
BLOCK_FP8 = 2
FORMATS = {"FP8_Dynamic": FP8_DYNAMIC, "W8A8_INT8": W8A8_INT8, "Block_FP8": BLOCK_FP8}
GROUP = 128

_HERE = os.path.dirname(os.path.abspath(__file__))
# W8_ORACLE_LIBRARY: another build of the oracle to load (the host-sanitizer
# build of build.build_sanitized(), for the CPU tests)
_LIB_PATH = os.environ.get("W8_ORACLE_LIBRARY") or os.path.join(_HERE, "_build", "libw8oracle.so")
_lib = None


class OracleError(RuntimeError):
    pass


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    u8p = ctypes.POINTER(ctypes.c_uint8)
    i8p = ctypes.POINTER(ctypes.c_int8)
    f32p = ctypes.POINTER(ctypes.c_float)
    f64p = ctypes.POINTER(ctypes.c_double)
    i64p = ctypes.POINTER(ctypes.c_int64)
    u16p = ctypes.POINTER(ctypes.c_uint16)
    i64 = ctypes.c_int64
    c_int = ctypes.c_int
    lib.or_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.or_e4m3_decode.restype = ctypes.c_double
    lib.or_e4m3_encode.argtypes = [ctypes.c_float]
    lib.or_e4m3_encode.restype = ctypes.c_uint8
    lib.or_int8_encode.argtypes = [ctypes.c_float]
    lib.or_int8_encode.restype = ctypes.c_int8
    lib.or_e4m3_encode_n.argtypes = [f32p, i64, u8p]
    lib.or_e4m3_encode_n.restype = None
    lib.or_int8_encode_n.argtypes = [f32p, i64, i8p]
    lib.or_int8_encode_n.restype = None
    lib.or_quantize_group.argtypes = [f32p, i64, c_int, u8p, f32p]
    lib.or_quantize_group.restype = c_int
    lib.or_quantize_act.argtypes = [c_int, c_int, c_int, u16p, i64, u8p, i64, f32p]
    lib.or_quantize_act.restype = c_int
    lib.or_quantize_weight.argtypes = [c_int, c_int, c_int, f32p, i64, u8p, i64, f32p]
    lib.or_quantize_weight.restype = c_int
    lib.or_acc_int8.argtypes = [c_int, c_int, c_int, c_int, i8p, i64, i8p, i64, i64p]
    lib.or_acc_int8.restype = c_int
    lib.or_acc_fp8.argtypes = [c_int, c_int, c_int, c_int, u8p, i64, u8p, i64, f64p]
    lib.or_acc_fp8.restype = c_int
    lib.or_gemm.argtypes = [c_int, c_int, c_int, c_int, u8p, i64, f32p, u8p, i64, f32p, f64p]
    lib.or_gemm.restype = c_int
    lib.or_num_threads.argtypes = []
    lib.or_num_threads.restype = c_int
    lib.or_set_threads.argtypes = [c_int]
    lib.or_set_threads.restype = None
    _lib = lib
    return lib


def _ptr(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _check(rc, what):
    if rc != 0:
        raise OracleError(f"{what}: oracle status {rc}")


def _fmt(fmt):
    return FORMATS[fmt] if isinstance(fmt, str) else int(fmt)


def num_threads() -> int:
    return _load().or_num_threads()


def set_threads(n: int) -> None:
    """OpenMP threads of the oracle's loops (timing only: results do not
    depend on it)."""
    _load().or_set_threads(int(n))


# ---------------------------------------------------------------- codecs ----
def e4m3_decode(codes) -> np.ndarray:
    """OCP E4M3FN decode of uint8 codes to float64 (NaN for 0x7F/0xFF)."""
    lib = _load()
    c = np.asarray(codes, dtype=np.uint8)
    table = np.array([lib.or_e4m3_decode(i) for i in range(256)], dtype=np.float64)
    return table[c]


def e4m3_encode(values) -> np.ndarray:
    """Saturating round-to-nearest-even encode of float32 values to E4M3FN."""
    lib = _load()
    v = np.ascontiguousarray(values, dtype=np.float32)
    out = np.zeros(v.shape, dtype=np.uint8)
    lib.or_e4m3_encode_n(_ptr(v, ctypes.c_float), v.size, _ptr(out, ctypes.c_uint8))
    return out


def int8_encode(values) -> np.ndarray:
    lib = _load()
    v = np.ascontiguousarray(values, dtype=np.float32)
    out = np.zeros(v.shape, dtype=np.int8)
    lib.or_int8_encode_n(_ptr(v, ctypes.c_float), v.size, _ptr(out, ctypes.c_int8))
    return out


def quantize_group(x, is_int8: bool):
    """One quantization group of fp32 values -> (codes uint8, scale float32)."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float32).ravel()
    q = np.zeros(x.size, dtype=np.uint8)
    s = np.zeros(1, dtype=np.float32)
    _check(lib.or_quantize_group(_ptr(x, ctypes.c_float), x.size, int(bool(is_int8)),
                                 _ptr(q, ctypes.c_uint8), _ptr(s, ctypes.c_float)),
           "quantize_group")
    return q, s[0]


# ---------------------------------------------------------- quantizers ----
def quantize_act(fmt, x_bf16_bits):
    """Dynamic activation quantization of bf16 X [M, K] (given as uint16 bits).

    Returns (xq uint8 [M, K], sx float32 [M] or [M, K/128]).
    """
    lib = _load()
    f = _fmt(fmt)
    x = np.ascontiguousarray(x_bf16_bits, dtype=np.uint16)
    M, K = x.shape
    xq = np.zeros((M, K), dtype=np.uint8)
    sx = np.zeros((M, K // GROUP) if f == BLOCK_FP8 else (M,), dtype=np.float32)
    _check(lib.or_quantize_act(f, M, K, _ptr(x, ctypes.c_uint16), K,
                               _ptr(xq, ctypes.c_uint8), K, _ptr(sx, ctypes.c_float)),
           "quantize_act")
    return xq, sx


def quantize_weight(fmt, w_fp32):
    """Offline E4M3FN weight quantization of fp32 W [N, K].

    FP8_Dynamic: sw float32 [N]; Block_FP8: sw float32 [ceil(N/128), ceil(K/128)].
    """
    lib = _load()
    f = _fmt(fmt)
    w = np.ascontiguousarray(w_fp32, dtype=np.float32)
    N, K = w.shape
    wq = np.zeros((N, K), dtype=np.uint8)
    if f == BLOCK_FP8:
        sw = np.zeros(((N + GROUP - 1) // GROUP, (K + GROUP - 1) // GROUP), dtype=np.float32)
    else:
        sw = np.zeros((N,), dtype=np.float32)
    _check(lib.or_quantize_weight(f, N, K, _ptr(w, ctypes.c_float), K,
                                  _ptr(wq, ctypes.c_uint8), K, _ptr(sw, ctypes.c_float)),
           "quantize_weight")
    return wq, sw


# -------------------------------------------------------------- GEMM ----
def acc_int8(xq, wq, k0=0, k1=None) -> np.ndarray:
    """Exact int64 accumulator C[m, n] = sum_k xq[m,k] wq[n,k] over [k0, k1)."""
    lib = _load()
    x = np.ascontiguousarray(xq).view(np.int8)
    w = np.ascontiguousarray(wq).view(np.int8)
    M, K = x.shape
    N = w.shape[0]
    k1 = K if k1 is None else k1
    C = np.zeros((M, N), dtype=np.int64)
    _check(lib.or_acc_int8(M, N, k0, k1, _ptr(x, ctypes.c_int8), K,
                           _ptr(w, ctypes.c_int8), w.shape[1], _ptr(C, ctypes.c_int64)),
           "acc_int8")
    return C


def acc_fp8(xq, wq, k0=0, k1=None) -> np.ndarray:
    """Exact E4M3FN dot products over [k0, k1), as float64."""
    lib = _load()
    x = np.ascontiguousarray(xq, dtype=np.uint8)
    w = np.ascontiguousarray(wq, dtype=np.uint8)
    M, K = x.shape
    N = w.shape[0]
    k1 = K if k1 is None else k1
    D = np.zeros((M, N), dtype=np.float64)
    _check(lib.or_acc_fp8(M, N, k0, k1, _ptr(x, ctypes.c_uint8), K,
                          _ptr(w, ctypes.c_uint8), w.shape[1], _ptr(D, ctypes.c_double)),
           "acc_fp8")
    return D


def gemm(fmt, xq, sx, wq, sw) -> np.ndarray:
    """Y = dequant(Xq) . dequant(Wq)^T in float64, [M, N] (not rounded to bf16)."""
    lib = _load()
    f = _fmt(fmt)
    x = np.ascontiguousarray(xq).view(np.uint8)
    w = np.ascontiguousarray(wq).view(np.uint8)
    sxa = np.ascontiguousarray(sx, dtype=np.float32)
    swa = np.ascontiguousarray(sw, dtype=np.float32)
    M, K = x.shape
    N = w.shape[0]
    Y = np.zeros((M, N), dtype=np.float64)
    _check(lib.or_gemm(f, M, N, K, _ptr(x, ctypes.c_uint8), K, _ptr(sxa, ctypes.c_float),
                       _ptr(w, ctypes.c_uint8), w.shape[1], _ptr(swa, ctypes.c_float),
                       _ptr(Y, ctypes.c_double)), "gemm")
    return Y


def forward(fmt, x_bf16_bits, wq, sw):
    """The whole path: quantize the activations, then the GEMM.

    Returns (Y float64 [M, N], xq, sx).
    """
    xq, sx = quantize_act(fmt, x_bf16_bits)
    return gemm(fmt, xq, sx, wq, sw), xq, sx


def moe_gemm(fmt, xq, sx, offsets, rows, wq, sw) -> np.ndarray:
    """MoE grouped GEMM (the pages' next target: MoE models, ai-radar.it,
    "Helion nel backend vLLM", paragraph 9).  E experts, each with its own
    weights wq[e] [N, K] and scales sw[e]; the routed entries of expert e are
    i in [offsets[e], offsets[e+1]), entry i reading token row rows[i] of the
    quantized activations.  Y[i] = the GEMM of that token row with expert e's
    weights, so Y[offsets[e]:offsets[e+1]] = gemm(fmt, xq[rows_e], sx[rows_e],
    wq[e], sw[e]).  Returns float64 [offsets[E], N]."""
    offsets = np.asarray(offsets, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    E = len(offsets) - 1
    N = wq.shape[1]
    Y = np.zeros((int(offsets[E]), N), dtype=np.float64)
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            r = rows[a:b]
            Y[a:b] = gemm(fmt, xq[r], sx[r], wq[e], sw[e])
    return Y
