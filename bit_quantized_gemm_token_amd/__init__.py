"""Small-M 8-bit quantized linear-layer GEMM for MI355X (gfx950).

    Y[M, N] = dequant(Xq) . dequant(Wq)^T,  1 <= M <= 32,
    formats FP8_Dynamic, W8A8_INT8 and Block_FP8.

Python face of the C-ABI in include/w8gemm.h (libw8gemm.so, built in-tree).
This module only marshals arguments: it takes torch tensors for device memory
and the current HIP stream, checks dtypes and layouts, and calls the library;
every step of the computation runs in the library's HIP kernels.  Importing it
fails when the library is not built.

Method: ai-radar.it, "Helion nel backend vLLM: un solo GEMM, tuning per forma e
guadagni fino al 10%" -- paragraph 1 (formats), 2-3 (Standard, Split-K,
Swap-AB as tunables of one GEMM; split_k a power of two up to 256),
4 (M <= 32 under graph replay), 6-7 (per-shape config table with a default).
"""
import ctypes
import os

import torch

from . import _capi
from ._capi import (ABI_VERSION, FORMATS, FORMAT_NAMES, GROUP, MAX_M, MAX_SPLIT_K, OPS, Config,
                    TuneOpts, TuneStats)

_lib = _capi.load()
LIB_PATH = _capi.LIB_PATH
DEFAULT_TABLE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "configs", "gfx950.tbl")

__all__ = ["Config", "W8Error", "UnsupportedShape", "Workspace", "PackedWeight", "quantize_act",
           "quantize_weight", "pack_weight", "gemm_w8a8", "gemm_w8a8_acc", "linear",
           "workspace_size",
           "validate_config", "default_config", "resolve_config", "lookup_config",
           "set_config", "load_config_table", "save_config_table", "clear_config_table",
           "config_table_size", "config_table_foreign", "tune_shape", "rank_configs",
           "profile_configs", "model_config", "moe_gemm", "moe_config", "moe_tune",
           "moe_workspace_size", "moe_linear", "moe_linear_config",
           "pack_experts", "PackedExperts", "read_floor", "FORMATS", "MAX_M",
           "MAX_SPLIT_K", "GROUP", "ABI_VERSION"]


class W8Error(RuntimeError):
    def __init__(self, status, message):
        self.status = status
        self.status_name = _capi.STATUS.get(status, str(status))
        super().__init__(f"{self.status_name}: {message}")


class UnsupportedShape(W8Error):
    """M is outside the small-M window; the caller should use another backend."""


def _check(status):
    if status != 0:
        msg = _lib.w8_last_error().decode(errors="replace")
        if status == 2:
            raise UnsupportedShape(status, msg)
        raise W8Error(status, msg)


def _fmt(fmt):
    if isinstance(fmt, str):
        if fmt not in FORMATS:
            raise ValueError(f"unknown format {fmt!r}; expected one of {list(FORMATS)}")
        return FORMATS[fmt]
    return int(fmt)


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dev_ptr(t, name, dtype=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _row_major(t, name):
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D tensor with unit inner stride")
    return t.stride(0)


def _cfg_ptr(cfg):
    if cfg is None:
        return None
    if isinstance(cfg, dict):
        cfg = Config.make(**cfg)
    return ctypes.byref(cfg)


def _op(op):
    if isinstance(op, str):
        if op not in OPS:
            raise ValueError(f"unknown op {op!r}; expected one of {list(OPS)}")
        return OPS[op]
    return int(op)


def _codes_dtype(fmt):
    return torch.int8 if _fmt(fmt) == FORMATS["W8A8_INT8"] else torch.float8_e4m3fn


def _act_scales(f, M, K):
    """Element count of the activation scales: [M] or, Block_FP8, [M, K/128]."""
    return M * (K // GROUP) if f == FORMATS["Block_FP8"] else M


def _weight_scales(f, N, K):
    """Element count of the weight scales: [N] or, Block_FP8, [ceil(N/128), ceil(K/128)]."""
    if f == FORMATS["Block_FP8"]:
        return ((N + GROUP - 1) // GROUP) * ((K + GROUP - 1) // GROUP)
    return N


def _check_scales(t, n, name):
    """The kernels read n contiguous fp32 scales from t's first element."""
    if not t.is_contiguous() or t.numel() != n:
        raise ValueError(f"{name} must be a contiguous tensor of {n} elements, got shape "
                         f"{tuple(t.shape)}")


def _check_out(t, M, N, name):
    if t.dim() != 2 or t.shape[0] != M or t.shape[1] != N:
        raise ValueError(f"{name} must be [{M}, {N}], got {tuple(t.shape)}")


# ----------------------------------------------------------------- quantize --
def quantize_act(fmt, x, xq=None, sx=None, stream=None):
    """Dynamic activation quantization of bf16 x [M, K] on the GPU.

    Returns (xq, sx): codes [M, K] (float8_e4m3fn or int8) and fp32 scales,
    [M] for the per-token formats or [M, K/128] for Block_FP8.
    """
    f = _fmt(fmt)
    ldx = _row_major(x, "x")
    M, K = x.shape
    if xq is None:
        xq = torch.empty((M, K), dtype=_codes_dtype(f), device=x.device)
    if sx is None:
        shape = (M, K // GROUP) if f == FORMATS["Block_FP8"] else (M,)
        sx = torch.empty(shape, dtype=torch.float32, device=x.device)
    _check_out(xq, M, K, "xq")
    if xq.element_size() != 1:
        raise TypeError("xq must hold 1-byte codes")
    _check_scales(sx, _act_scales(f, M, K), "sx")
    ldq = _row_major(xq, "xq")
    _check(_lib.w8_quantize_act(f, M, K, _dev_ptr(x, "x", torch.bfloat16), ldx,
                                _dev_ptr(xq, "xq"), ldq * xq.element_size(),
                                _dev_ptr(sx, "sx", torch.float32), _stream(stream, x.device)))
    return xq, sx


def quantize_weight(fmt, w, wq=None, sw=None, stream=None):
    """Offline E4M3FN quantization of fp32 weights w [N, K] on the GPU.

    FP8_Dynamic: sw [N]; Block_FP8: sw [ceil(N/128), ceil(K/128)].
    """
    f = _fmt(fmt)
    ldw = _row_major(w, "w")
    N, K = w.shape
    if wq is None:
        wq = torch.empty((N, K), dtype=torch.float8_e4m3fn, device=w.device)
    if sw is None:
        shape = ((N + GROUP - 1) // GROUP, (K + GROUP - 1) // GROUP) \
            if f == FORMATS["Block_FP8"] else (N,)
        sw = torch.empty(shape, dtype=torch.float32, device=w.device)
    ldq = _row_major(wq, "wq")
    _check(_lib.w8_quantize_weight(f, N, K, _dev_ptr(w, "w", torch.float32), ldw,
                                   _dev_ptr(wq, "wq"), ldq * wq.element_size(),
                                   _dev_ptr(sw, "sw", torch.float32), _stream(stream, w.device)))
    return wq, sw


# ------------------------------------------------------------- weight layout --
# Weight layout codes: 0 row-major, 1 packed (MFMA-native, 16-row blocks),
# 2/4/8 K-segmented packed (that many K-steps per MFMA, 16/T-row blocks).
LAYOUTS = {"row": 0, "packed": 1, "seg2": 2, "seg4": 4, "seg8": 8}
LAYOUT_NAMES = {v: k for k, v in LAYOUTS.items()}


def _layout(packed):
    """Layout code of a `packed` argument: False/True, 0/1/2/4/8 or a name."""
    if isinstance(packed, str):
        if packed not in LAYOUTS:
            raise ValueError(f"unknown weight layout {packed!r}")
        return LAYOUTS[packed]
    v = int(packed)
    if v not in LAYOUT_NAMES:
        raise ValueError(f"weight layout must be one of {sorted(LAYOUT_NAMES)}, got {packed!r}")
    return v


class PackedWeight:
    """Weight codes in a packed layout (1: MFMA-native; 2, 4, 8: K-segmented).

    Produced by pack_weight(); pass it to gemm_w8a8() in place of the
    row-major [N, K] code tensor.  `data` is the 1-D uint8 device buffer.
    """

    def __init__(self, fmt, N, K, data, layout=1):
        self.fmt, self.N, self.K, self.data = _fmt(fmt), int(N), int(K), data
        self.layout = _layout(layout)
        if self.layout == 0:
            raise ValueError("a PackedWeight holds a packed layout (1, 2, 4 or 8)")
        self.shape = (self.N, self.K)
        self.device = data.device


def packed_weight_size(fmt, N, K, layout=1):
    n = ctypes.c_size_t(0)
    _check(_lib.w8_packed_weight_size(_fmt(fmt), N, K, _layout(layout), ctypes.byref(n)))
    return n.value


def pack_weight(fmt, wq, stream=None, layout=1):
    """Pack row-major codes [N, K] into packed layout `layout` (offline, on the GPU)."""
    f = _fmt(fmt)
    lay = _layout(layout)
    ldw = _row_major(wq, "wq") * wq.element_size()
    N, K = wq.shape
    out = torch.empty(packed_weight_size(f, N, K, lay), dtype=torch.uint8, device=wq.device)
    _check(_lib.w8_pack_weight(f, N, K, _dev_ptr(wq, "wq"), ldw, _dev_ptr(out, "out"), lay,
                               _stream(stream, wq.device)))
    return PackedWeight(f, N, K, out, lay)


# --------------------------------------------------------------------- GEMM --
def workspace_size(fmt, M, N, K, cfg=None, packed=False, op="gemm"):
    n = ctypes.c_size_t(0)
    _check(_lib.w8_workspace_size(_fmt(fmt), _op(op), M, N, K, _layout(packed), _cfg_ptr(cfg),
                                  ctypes.byref(n)))
    return n.value


class Workspace:
    """Device workspace for split-K and the linear op's quantize launch.

    Zero-filled when (re)allocated; the GEMM leaves its arrival counters at
    multiples of 256 after each call (which is all a call needs of them), so
    one Workspace can serve any sequence of calls on one stream
    (calls that overlap on several streams race).

    Under HIP graph capture the workspace cannot grow: the fill would be
    recorded into the graph and a buffer given back to the allocator could
    be handed out again while the graph still writes to it.  Size it
    beforehand (Workspace(device, nbytes), or call reserve() before the
    capture).  A buffer that a larger one replaces is kept alive for the
    Workspace's lifetime, because a graph captured earlier may still use it;
    release_retired() drops those once no such graph remains.
    """

    def __init__(self, device=None, nbytes=0):
        self.device = torch.device(device or "cuda")
        self.buf = None
        self._retired = []
        if nbytes:
            self.reserve(nbytes)

    def reserve(self, nbytes, stream=None):
        """The buffer, grown to at least nbytes (zero-filled on `stream`,
        default the current stream, before any later work on it)."""
        if self.buf is not None and self.buf.numel() >= nbytes:
            return self.buf
        if torch.cuda.is_current_stream_capturing():
            raise RuntimeError(
                f"the workspace would grow to {int(nbytes)} bytes during graph capture; "
                f"size it before capturing (Workspace(device, nbytes) or reserve())")
        if self.buf is not None:
            self._retired.append(self.buf)
        s = stream if stream is not None else torch.cuda.current_stream(self.device)
        if not isinstance(s, torch.cuda.Stream):
            s = torch.cuda.ExternalStream(int(s), device=self.device)
        with torch.cuda.stream(s):
            buf = torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=self.device)
            buf.zero_()
        self.buf = buf
        return self.buf

    def release_retired(self):
        """Drops the buffers that larger ones replaced (call only when no
        captured graph that used them will be replayed)."""
        self._retired.clear()

    def for_call(self, fmt, M, N, K, cfg=None, packed=False, op="gemm", stream=None):
        need = workspace_size(fmt, M, N, K, cfg, packed, op)
        if need == 0:
            return None, 0
        buf = self.reserve(need, stream)
        return ctypes.c_void_p(buf.data_ptr()), buf.numel()


def _weights(f, wq):
    """(N, K, ldw, device tensor, layout) of row-major codes or a PackedWeight
    (ldw 0 for layout 1, -T for the K-segmented layouts)."""
    if isinstance(wq, PackedWeight):
        if wq.fmt != f:
            raise ValueError("packed weights were packed for another format")
        return wq.N, wq.K, (0 if wq.layout == 1 else -wq.layout), wq.data, wq.layout
    if wq.element_size() != 1:
        raise TypeError("wq must hold 1-byte codes")
    N, wk = wq.shape
    return N, wk, _row_major(wq, "wq") * wq.element_size(), wq, 0


def _gemm(entry, fmt, xq, sx, wq, sw, out, cfg, workspace, stream):
    f = _fmt(fmt)
    ldq = _row_major(xq, "xq") * xq.element_size()
    ldo = _row_major(out, "out")
    M, K = xq.shape
    N, wk, ldw, wptr, packed = _weights(f, wq)
    if wk != K:
        raise ValueError(f"K mismatch: xq {tuple(xq.shape)} vs weights {(N, wk)}")
    if xq.element_size() != 1:
        raise TypeError("xq must hold 1-byte codes")
    _check_scales(sx, _act_scales(f, M, K), "sx")
    _check_scales(sw, _weight_scales(f, N, K), "sw")
    _check_out(out, M, N, "out")
    if workspace is None:
        workspace = _default_workspace(xq.device)
    ws_ptr, ws_bytes = workspace.for_call(f, M, N, K, cfg, packed, "gemm", stream)
    _check(entry(f, M, N, K, _dev_ptr(xq, "xq"), ldq, _dev_ptr(sx, "sx", torch.float32),
                 _dev_ptr(wptr, "wq"), ldw, _dev_ptr(sw, "sw", torch.float32),
                 _dev_ptr(out, "out"), ldo, _cfg_ptr(cfg), ws_ptr, ws_bytes,
                 _stream(stream, xq.device)))
    return out


_workspaces = {}


def _default_workspace(device):
    key = str(device)
    if key not in _workspaces:
        _workspaces[key] = Workspace(device)
    return _workspaces[key]


def gemm_w8a8(fmt, xq, sx, wq, sw, cfg=None, y=None, workspace=None, stream=None):
    """Y = dequant(xq) . dequant(wq)^T as bf16 [M, N].

    wq: row-major codes [N, K] or a PackedWeight.  cfg: a Config (or dict of
    its fields); None uses the config table entry for the shape and weight
    layout, else the default config.
    """
    M, N = xq.shape[0], wq.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=xq.device)
    elif y.dtype != torch.bfloat16:
        raise TypeError("y must be bfloat16")
    return _gemm(_lib.w8_gemm_w8a8, fmt, xq, sx, wq, sw, y, cfg, workspace, stream)


def gemm_w8a8_acc(fmt, xq, sx, wq, sw, cfg=None, out=None, workspace=None, stream=None):
    """Test hook: raw accumulators [M, N] (int32 for W8A8_INT8, else fp32)."""
    M, N = xq.shape[0], wq.shape[0]
    dt = torch.int32 if _fmt(fmt) == FORMATS["W8A8_INT8"] else torch.float32
    if out is None:
        out = torch.empty((M, N), dtype=dt, device=xq.device)
    elif out.dtype != dt:
        raise TypeError(f"out must be {dt}")
    return _gemm(_lib.w8_gemm_w8a8_acc, fmt, xq, sx, wq, sw, out, cfg, workspace, stream)


def linear(fmt, x, wq, sw, cfg=None, y=None, workspace=None, stream=None, fused=False):
    """The whole hot path on bf16 activations x [M, K].

    fused=False: quantize_act, then gemm_w8a8 (two calls; cfg is the GEMM
    config).  fused=True: the single entry point w8_linear with a linear-op
    config (None = the table's "linear" entry): cfg.quant_launch = 0 fuses the
    quantization into the GEMM (one launch; needs x_lds=1), 1 runs the
    quantize kernel into the workspace and then the GEMM.  All give the same Y
    for the same tile config.  wq: row-major codes [N, K] or a PackedWeight."""
    if not fused:
        xq, sx = quantize_act(fmt, x, stream=stream)
        return gemm_w8a8(fmt, xq, sx, wq, sw, cfg=cfg, y=y, workspace=workspace, stream=stream)
    f = _fmt(fmt)
    if x.dtype != torch.bfloat16:
        raise TypeError("x must be bfloat16")
    ldx = _row_major(x, "x")
    M, K = x.shape
    N, wk, ldw, wptr, packed = _weights(f, wq)
    if wk != K:
        raise ValueError(f"K mismatch: x {tuple(x.shape)} vs weights {(N, wk)}")
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    elif y.dtype != torch.bfloat16:
        raise TypeError("y must be bfloat16")
    _check_out(y, M, N, "y")
    _check_scales(sw, _weight_scales(f, N, K), "sw")
    if workspace is None:
        workspace = _default_workspace(x.device)
    ws_ptr, ws_bytes = workspace.for_call(f, M, N, K, cfg, packed, "linear", stream)
    _check(_lib.w8_linear(f, M, N, K, _dev_ptr(x, "x"), ldx, _dev_ptr(wptr, "wq"), ldw,
                          _dev_ptr(sw, "sw", torch.float32), _dev_ptr(y, "y"), _row_major(y, "y"),
                          _cfg_ptr(cfg), ws_ptr, ws_bytes, _stream(stream, x.device)))
    return y


# ---------------------------------------------------------------------- MoE --
class PackedExperts:
    """Every expert's weight codes in the packed layout, one expert per row of
    the 2-D uint8 device buffer `data` [E, packed_weight_size(fmt, N, K)]."""

    def __init__(self, fmt, N, K, data):
        self.fmt, self.N, self.K, self.data = _fmt(fmt), int(N), int(K), data
        self.E = data.shape[0]
        self.device = data.device


def pack_experts(fmt, wq, stream=None):
    """Pack row-major expert codes [E, N, K] (offline, on the GPU)."""
    f = _fmt(fmt)
    E, N, K = wq.shape
    out = torch.empty((E, packed_weight_size(f, N, K)), dtype=torch.uint8, device=wq.device)
    for e in range(E):
        w = wq[e]
        _check(_lib.w8_pack_weight(f, N, K, _dev_ptr(w, "wq"), _row_major(w, "wq"),
                                   _dev_ptr(out[e], "out"), 1, _stream(stream, wq.device)))
    return PackedExperts(f, N, K, out)


def _experts(f, wq):
    """(E, N, K, ldw, w_stride, pointer, packed) of [E, N, K] codes or PackedExperts."""
    if isinstance(wq, PackedExperts):
        if wq.fmt != f:
            raise ValueError("experts were packed for another format")
        return wq.E, wq.N, wq.K, 0, wq.data.stride(0), _dev_ptr(wq.data, "wq"), True
    if wq.dim() != 3 or wq.element_size() != 1 or wq.stride(2) != 1:
        raise ValueError("wq must be [E, N, K] 1-byte codes with unit inner stride")
    E, N, K = wq.shape
    return E, N, K, wq.stride(1), wq.stride(0), _dev_ptr(wq, "wq"), False


def moe_config(fmt, E, T, N, K, max_m=32, packed=False):
    """(config moe_gemm uses when cfg is None, 1 if it is the table's "moe"
    entry for (T, N, K) else 0)."""
    c = Config()
    hit = ctypes.c_int(0)
    _check(_lib.w8_moe_config(_fmt(fmt), E, T, N, K, max_m, _layout(packed), ctypes.byref(c),
                              ctypes.byref(hit)))
    return c, hit.value


def moe_linear_config(fmt, E, T, N, K, max_m=32, packed=False):
    """(config moe_linear uses when cfg is None, 1 if it is the table's
    "moe_linear" entry for (T, N, K) else 0)."""
    c = Config()
    hit = ctypes.c_int(0)
    _check(_lib.w8_moe_linear_config(_fmt(fmt), E, T, N, K, max_m, _layout(packed),
                                     ctypes.byref(c), ctypes.byref(hit)))
    return c, hit.value


def moe_tune(fmt, E, T, N, K, topk, warmup=2, replays=5, bank2_top=5, rotate_bytes=512 << 20,
             max_split_k=MAX_SPLIT_K, insert=True, fail_candidate=-1, packed=False, fused=False):
    """Ahead-of-time tuning of the grouped GEMM for E experts of (N, K) at T
    tokens routed top-k (seeded uniform routings); fused=True tunes
    moe_linear (quantization fused) instead of moe_gemm.  The winner becomes
    the table's "moe" (or "moe_linear") entry for (T, N, K) when insert.
    Returns (Config, stats dict).  Synchronizes the device."""
    o = _tune_opts(warmup, replays, bank2_top, rotate_bytes, max_split_k, insert,
                   fail_candidate, packed, False, "linear" if fused else "gemm", 0)
    best = Config()
    stats = TuneStats()
    _check(_lib.w8_moe_tune(_fmt(fmt), E, T, N, K, topk, ctypes.byref(o), ctypes.byref(best),
                            ctypes.byref(stats)))
    return best, stats.as_dict()


def moe_workspace_size(fmt, E, T, N, K, max_m=32, cfg=None, packed=False):
    n = ctypes.c_size_t(0)
    _check(_lib.w8_moe_workspace_size(_fmt(fmt), E, T, N, K, max_m, _layout(packed),
                                      _cfg_ptr(cfg), ctypes.byref(n)))
    return n.value


def moe_gemm(fmt, xq, sx, offsets, rows, wq, sw, max_m=32, cfg=None, y=None, workspace=None,
             stream=None):
    """MoE grouped GEMM: for routed entry i of expert e (offsets[e] <= i <
    offsets[e+1]), Y[i] = dequant(xq[rows[i]]) . dequant(Wq_e)^T, bf16
    [len(rows), N].  xq, sx: the T quantized token rows (quantize_act);
    offsets int32 [E + 1], rows int32 (device); wq: [E, N, K] codes or
    PackedExperts; sw: [E, ...] scales in the format's per-expert layout;
    every expert's count <= max_m <= 32.  One launch, no host sync."""
    f = _fmt(fmt)
    ldq = _row_major(xq, "xq") * xq.element_size()
    T, K = xq.shape
    E, N, wk, ldw, w_stride, wptr, packed = _experts(f, wq)
    if wk != K:
        raise ValueError(f"K mismatch: xq {tuple(xq.shape)} vs experts' K {wk}")
    if offsets.numel() != E + 1:
        raise ValueError("offsets must hold E + 1 entries")
    if sw.shape[0] != E or not sw.is_contiguous() or sw.numel() != E * _weight_scales(f, N, K):
        raise ValueError(f"sw must be a contiguous [E, {_weight_scales(f, N, K)}] tensor")
    _check_scales(sx, _act_scales(f, T, K), "sx")
    if y is None:
        y = torch.empty((rows.numel(), N), dtype=torch.bfloat16, device=xq.device)
    elif y.dtype != torch.bfloat16:
        raise TypeError("y must be bfloat16")
    elif y.shape[0] < rows.numel() or y.shape[1] != N:
        raise ValueError(f"y must be [{rows.numel()}, {N}]")
    if workspace is None:
        workspace = _default_workspace(xq.device)
    need = moe_workspace_size(f, E, T, N, K, max_m, cfg, packed)
    ws_ptr, ws_bytes = (None, 0)
    if need:
        buf = workspace.reserve(need, stream)
        ws_ptr, ws_bytes = ctypes.c_void_p(buf.data_ptr()), buf.numel()
    _check(_lib.w8_moe_gemm(f, E, T, N, K, max_m, _dev_ptr(xq, "xq"), ldq,
                            _dev_ptr(sx, "sx", torch.float32),
                            _dev_ptr(offsets, "offsets", torch.int32),
                            _dev_ptr(rows, "rows", torch.int32), rows.numel(), wptr, ldw,
                            w_stride,
                            _dev_ptr(sw, "sw", torch.float32), sw.stride(0),
                            _dev_ptr(y, "y"), _row_major(y, "y"), _cfg_ptr(cfg), ws_ptr, ws_bytes,
                            _stream(stream, xq.device)))
    return y


def moe_linear(fmt, x, offsets, rows, wq, sw, max_m=32, cfg=None, y=None, workspace=None,
               stream=None):
    """MoE grouped GEMM on bf16 tokens x [T, K] with the activation
    quantization fused into the grouped kernel: equals quantize_act(x) then
    moe_gemm with the same config, bit for bit.  cfg: a grouped config with
    x_lds=1 and waves_k <= 4, or None (moe_linear_config).  Other arguments as
    for moe_gemm.  One launch, no host sync."""
    f = _fmt(fmt)
    if x.dtype != torch.bfloat16:
        raise TypeError("x must be bfloat16")
    ldx = _row_major(x, "x")
    T, K = x.shape
    E, N, wk, ldw, w_stride, wptr, packed = _experts(f, wq)
    if wk != K:
        raise ValueError(f"K mismatch: x {tuple(x.shape)} vs experts' K {wk}")
    if offsets.numel() != E + 1:
        raise ValueError("offsets must hold E + 1 entries")
    if sw.shape[0] != E or not sw.is_contiguous() or sw.numel() != E * _weight_scales(f, N, K):
        raise ValueError(f"sw must be a contiguous [E, {_weight_scales(f, N, K)}] tensor")
    if y is None:
        y = torch.empty((rows.numel(), N), dtype=torch.bfloat16, device=x.device)
    elif y.dtype != torch.bfloat16:
        raise TypeError("y must be bfloat16")
    elif y.shape[0] < rows.numel() or y.shape[1] != N:
        raise ValueError(f"y must be [{rows.numel()}, {N}]")
    if cfg is None:
        cfg = moe_linear_config(f, E, T, N, K, max_m, packed)[0]
    if workspace is None:
        workspace = _default_workspace(x.device)
    need = moe_workspace_size(f, E, T, N, K, max_m, cfg, packed)
    ws_ptr, ws_bytes = (None, 0)
    if need:
        buf = workspace.reserve(need, stream)
        ws_ptr, ws_bytes = ctypes.c_void_p(buf.data_ptr()), buf.numel()
    _check(_lib.w8_moe_linear(f, E, T, N, K, max_m, _dev_ptr(x, "x"), ldx,
                              _dev_ptr(offsets, "offsets", torch.int32),
                              _dev_ptr(rows, "rows", torch.int32), rows.numel(), wptr, ldw,
                              w_stride, _dev_ptr(sw, "sw", torch.float32), sw.stride(0),
                              _dev_ptr(y, "y"), _row_major(y, "y"), _cfg_ptr(cfg), ws_ptr,
                              ws_bytes, _stream(stream, x.device)))
    return y


# ------------------------------------------------------------------- config --
# op: "gemm" (gemm_w8a8) or "linear" (linear(..., fused=True)).
def validate_config(fmt, M, N, K, cfg, op="gemm", packed=False):
    """Raises W8Error unless cfg is valid for op and the shape on weights of
    layout `packed` (False/True, 0/1/2/4/8 or a LAYOUTS name)."""
    _check(_lib.w8_validate_config(_fmt(fmt), _op(op), M, N, K, _layout(packed), _cfg_ptr(cfg)))


def default_config(fmt, M, N, K, op="gemm", packed=False):
    c = Config()
    _check(_lib.w8_default_config(_fmt(fmt), _op(op), M, N, K, _layout(packed), ctypes.byref(c)))
    return c


def resolve_config(fmt, M, N, K, packed=False, op="gemm"):
    """(Config, source) that the op uses when cfg is None; source is 1 for
    the table entry of the shape, 2 for an entry of the same N, K and
    floor(log2 M) bucket, 0 for the cost model's pick."""
    c = Config()
    hit = ctypes.c_int(0)
    _check(_lib.w8_resolve_config(_fmt(fmt), _op(op), M, N, K, _layout(packed),
                                  ctypes.byref(c), ctypes.byref(hit)))
    return c, hit.value


def model_config(fmt, M, N, K, packed=False, op="gemm"):
    """The cost model's top-1 config (what an untuned shape runs)."""
    c = Config()
    _check(_lib.w8_model_config(_fmt(fmt), _op(op), M, N, K, _layout(packed), ctypes.byref(c)))
    return c


class PredictBatch:
    """Rows (fmt, op, layout, M, N, K, cfg) packed once for the library's
    cost model (w8_predict_us); run(params) returns the predicted us per call
    of every row as a numpy array, with the compiled constants (params None)
    or 13 trial constants.  Host only."""

    def __init__(self, rows):
        import numpy as np
        n = len(rows)
        self.n = n
        arr = lambda vals: (ctypes.c_int * max(n, 1))(*vals)
        self._fmt = arr([_fmt(r[0]) for r in rows])
        self._op = arr([_op(r[1]) for r in rows])
        self._layout = arr([_layout(r[2]) for r in rows])
        self._M, self._N, self._K = (arr([int(r[i]) for r in rows]) for i in (3, 4, 5))
        self._cfgs = (Config * max(n, 1))(*[c if isinstance(c, Config) else Config.make(**c)
                                            for c in (r[6] for r in rows)])
        self._out = np.zeros(max(n, 1), dtype=np.float64)

    def run(self, params=None):
        dp = ctypes.POINTER(ctypes.c_double)
        if params is None:
            pp, npar = None, 0
        else:
            pv = (ctypes.c_double * len(params))(*[float(v) for v in params])
            pp, npar = ctypes.cast(pv, dp), len(params)
        _check(_lib.w8_predict_us(self.n, self._fmt, self._op, self._layout, self._M, self._N,
                                  self._K, self._cfgs, pp, npar,
                                  self._out.ctypes.data_as(dp)))
        return self._out[:self.n].copy()


def predict_us(rows, params=None):
    """The cost model's predicted us per call of each (fmt, op, layout, M, N,
    K, cfg) row (cfg a Config or a dict of its fields)."""
    return list(PredictBatch(rows).run(params))


def lookup_config(fmt, M, N, K, packed=False, with_time=False, op="gemm"):
    """Exact table entry for the op, shape and weight layout, or None.

    with_time=True returns (Config, us_per_call) instead of the Config.
    """
    c = Config()
    us = ctypes.c_double(0.0)
    st = _lib.w8_lookup_config(_fmt(fmt), _op(op), M, N, K, _layout(packed), ctypes.byref(c),
                               ctypes.byref(us))
    if st == 8:
        return None
    _check(st)
    return (c, us.value) if with_time else c


def best_layout(fmt, M, N, K, op="gemm", layouts=(0, 1, 2, 4, 8)):
    """The layout code (of `layouts`) whose table entry for this op and
    shape has the lowest time per call; 0 (row-major) when none has one."""
    best, best_us = 0, None
    for lay in layouts:
        e = lookup_config(fmt, M, N, K, packed=lay, with_time=True, op=op)
        if e is not None and (best_us is None or e[1] < best_us):
            best, best_us = _layout(lay), e[1]
    return best


def set_config(fmt, M, N, K, cfg, us_per_gemm=0.0, packed=False, op="gemm"):
    if isinstance(cfg, dict):
        cfg = Config.make(**cfg)
    _check(_lib.w8_set_config(_fmt(fmt), _op(op), M, N, K, _layout(packed), ctypes.byref(cfg),
                              float(us_per_gemm)))


def load_config_table(path):
    _check(_lib.w8_load_config_table(os.fsencode(path)))


def save_config_table(path):
    _check(_lib.w8_save_config_table(os.fsencode(path)))


def clear_config_table():
    _lib.w8_clear_config_table()


def config_table_size():
    return _lib.w8_config_table_size()


def config_table_foreign():
    return _lib.w8_config_table_foreign()


def load_default_table():
    """Load the shipped gfx950 table if present; returns True if loaded."""
    if os.path.exists(DEFAULT_TABLE):
        load_config_table(DEFAULT_TABLE)
        return True
    return False


# -------------------------------------------------------------------- tuner --
def _tune_opts(warmup=2, replays=5, bank2_top=5, rotate_bytes=512 << 20,
               max_split_k=MAX_SPLIT_K, insert=True, fail_candidate=-1, packed=False,
               stream_k=False, op="gemm", top_n=0):
    o = TuneOpts()
    _lib.w8_tune_default_opts(ctypes.byref(o))
    o.warmup, o.replays, o.bank2_top = warmup, replays, bank2_top
    o.rotate_bytes, o.max_split_k = rotate_bytes, max_split_k
    o.insert, o.fail_candidate = int(bool(insert)), fail_candidate
    o.packed = _layout(packed)
    o.stream_k = int(bool(stream_k))
    o.op = _op(op)
    o.top_n = int(top_n)
    # the caller's current stream: the tuners refuse to run while it is being
    # captured into a graph
    if torch.cuda.is_available():
        o.stream = torch.cuda.current_stream().cuda_stream
    return o


def rank_configs(fmt, M, N, K, packed=False, op="gemm", max_split_k=MAX_SPLIT_K,
                 stream_k=False):
    """The tuner's candidate set ranked by the cost model: [(predicted_us, Config)],
    fastest first.  Host only."""
    o = _tune_opts(packed=packed, op=op, max_split_k=max_split_k, stream_k=stream_k)
    n = ctypes.c_int(0)
    _check(_lib.w8_rank_configs(_fmt(fmt), M, N, K, ctypes.byref(o), None, None, 0,
                                ctypes.byref(n)))
    cfgs = (Config * max(n.value, 1))()
    us = (ctypes.c_double * max(n.value, 1))()
    _check(_lib.w8_rank_configs(_fmt(fmt), M, N, K, ctypes.byref(o), cfgs, us, n.value,
                                ctypes.byref(n)))
    return [(us[i], cfgs[i]) for i in range(n.value)]


def profile_configs(fmt, M, N, K, cfgs, packed=False, op="gemm", warmup=2, replays=5,
                    rotate_bytes=512 << 20):
    """Times configs with the tuner's harness (bank 1, no table insert):
    [us or None when the config's output failed validation].  Synchronizes."""
    o = _tune_opts(warmup=warmup, replays=replays, rotate_bytes=rotate_bytes, packed=packed,
                   op=op, insert=False)
    n = len(cfgs)
    arr = (Config * max(n, 1))(*cfgs)
    us = (ctypes.c_double * max(n, 1))()
    valid = (ctypes.c_int * max(n, 1))()
    _check(_lib.w8_profile_configs(_fmt(fmt), M, N, K, ctypes.byref(o), arr, n, us, valid))
    return [us[i] if valid[i] else None for i in range(n)]


def tune_shape(fmt, M, N, K, warmup=2, replays=5, bank2_top=5, rotate_bytes=512 << 20,
               max_split_k=MAX_SPLIT_K, insert=True, fail_candidate=-1, packed=False,
               stream_k=False, op="gemm", top_n=0):
    """Ahead-of-time tuning of one shape and weight layout on the current device
    (top_n > 0: only the cost model's top_n candidates are timed).

    Returns (Config, stats dict).  Synchronizes the device.
    """
    o = _tune_opts(warmup, replays, bank2_top, rotate_bytes, max_split_k, insert,
                   fail_candidate, packed, stream_k, op, top_n)
    best = Config()
    stats = TuneStats()
    _check(_lib.w8_tune_shape(_fmt(fmt), M, N, K, ctypes.byref(o), ctypes.byref(best),
                              ctypes.byref(stats)))
    return best, stats.as_dict()


def algorithmic_bytes(fmt, M, N, K):
    """Bytes the GEMM must move: weights, activations, scales and bf16 output."""
    if _fmt(fmt) == FORMATS["Block_FP8"]:
        G = (K + GROUP - 1) // GROUP
        return N * K + M * K + 2 * M * N + 4 * ((N + GROUP - 1) // GROUP) * G + 4 * M * G
    return N * K + M * K + 2 * M * N + 4 * N + 4 * M


load_default_table()


# -------------------------------------------------------------- measurement --
def read_floor(src, nbytes, sink, grid=512, waves=4, depth=4, stream=None):
    """One launch of the read-floor kernel: streams nbytes (a multiple of
    1024) of the device tensor src once, writing grid * waves words to the
    uint32/int32 device tensor sink.  Measurement only (w8_read_floor)."""
    if src.numel() * src.element_size() < nbytes:
        raise ValueError("src holds fewer than nbytes bytes")
    _check(_lib.w8_read_floor(_dev_ptr(src, "src"), nbytes, _dev_ptr(sink, "sink"),
                              sink.numel() * sink.element_size(), grid, waves, depth,
                              _stream(stream, src.device)))
