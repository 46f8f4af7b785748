"""ctypes declarations of the C-ABI in include/w8gemm.h."""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# W8_LIBRARY: another build of the library to load (the host-sanitizer
# build of build.build_sanitized(), for the CPU tests)
LIB_PATH = os.environ.get("W8_LIBRARY") or os.path.join(_HERE, "libw8gemm.so")

ABI_VERSION = 5
MAX_M = 32
MAX_SPLIT_K = 256
GROUP = 128

FORMATS = {"FP8_Dynamic": 0, "W8A8_INT8": 1, "Block_FP8": 2}
OPS = {"gemm": 0, "linear": 1, "moe": 2, "moe_linear": 3}
FORMAT_NAMES = {v: k for k, v in FORMATS.items()}

STATUS = {0: "W8_OK", 1: "W8_E_INVALID", 2: "W8_E_UNSUPPORTED", 3: "W8_E_WORKSPACE",
          4: "W8_E_TABLE_FORMAT", 5: "W8_E_IO", 6: "W8_E_HIP", 7: "W8_E_VALIDATION",
          8: "W8_E_NOT_FOUND"}

# Every symbol include/w8gemm.h declares.
EXPORTS = ("w8_abi_version", "w8_status_string", "w8_last_error", "w8_quantize_act",
           "w8_quantize_weight", "w8_packed_weight_size", "w8_pack_weight",
           "w8_workspace_size", "w8_gemm_w8a8", "w8_gemm_w8a8_acc", "w8_linear",
           "w8_validate_config", "w8_default_config", "w8_resolve_config",
           "w8_load_config_table", "w8_save_config_table", "w8_clear_config_table",
           "w8_config_table_size", "w8_config_table_foreign", "w8_set_config",
           "w8_lookup_config", "w8_tune_shape", "w8_tune_default_opts", "w8_model_config",
           "w8_rank_configs", "w8_profile_configs", "w8_moe_gemm", "w8_moe_workspace_size",
           "w8_moe_validate_config", "w8_moe_config", "w8_moe_tune", "w8_moe_linear",
           "w8_moe_linear_config", "w8_read_floor", "w8_gemm_w8a8_noalloc", "w8_predict_us")


class Config(ctypes.Structure):
    """w8_cfg: one configuration of the GEMM family."""
    _fields_ = [("abi_version", ctypes.c_int32), ("tile_n", ctypes.c_int32),
                ("waves_k", ctypes.c_int32), ("waves_n", ctypes.c_int32),
                ("unroll", ctypes.c_int32), ("split_k", ctypes.c_int32),
                ("grid", ctypes.c_int32), ("swap_ab", ctypes.c_int32),
                ("x_lds", ctypes.c_int32), ("quant_launch", ctypes.c_int32),
                ("reserved", ctypes.c_int32 * 1)]

    KEYS = ("tile_n", "waves_k", "waves_n", "unroll", "split_k", "grid", "swap_ab", "x_lds",
            "quant_launch")

    @classmethod
    def make(cls, tile_n=16, waves_k=4, unroll=2, split_k=1, swap_ab=0, waves_n=1, grid=0,
             x_lds=None, quant_launch=0):
        if x_lds is None:
            x_lds = 1 if waves_n > 1 else 0
        return cls(ABI_VERSION, tile_n, waves_k, waves_n, unroll, split_k, grid, int(swap_ab),
                   int(x_lds), int(quant_launch))

    def as_dict(self):
        return {k: int(getattr(self, k)) for k in self.KEYS}

    def __repr__(self):
        return "Config(" + ", ".join(f"{k}={v}" for k, v in self.as_dict().items()) + ")"

    def __eq__(self, other):
        return isinstance(other, Config) and self.as_dict() == other.as_dict()


class TuneOpts(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_int32), ("warmup", ctypes.c_int32),
                ("replays", ctypes.c_int32), ("bank2_top", ctypes.c_int32),
                ("rotate_bytes", ctypes.c_int64), ("max_split_k", ctypes.c_int32),
                ("insert", ctypes.c_int32), ("fail_candidate", ctypes.c_int32),
                ("packed", ctypes.c_int32), ("stream_k", ctypes.c_int32),
                ("op", ctypes.c_int32), ("top_n", ctypes.c_int32), ("stream", ctypes.c_void_p)]


class TuneStats(ctypes.Structure):
    _fields_ = [("candidates", ctypes.c_int32), ("validated", ctypes.c_int32),
                ("rejected", ctypes.c_int32), ("best_index", ctypes.c_int32),
                ("best_us_bank1", ctypes.c_double), ("best_us_bank2", ctypes.c_double),
                ("default_us_bank2", ctypes.c_double), ("best_gbps", ctypes.c_double),
                ("tune_seconds", ctypes.c_double), ("best_us_bank2_min", ctypes.c_double),
                ("best_us_bank2_p90", ctypes.c_double)]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


def load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; build it with "
            "`python -c 'import __graft_entry__ as g; g.build()'` from the repository root")
    lib = ctypes.CDLL(LIB_PATH)
    c_int, i64, vp, f32p = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p
    cfgp = ctypes.POINTER(Config)
    st = ctypes.c_int
    lib.w8_abi_version.restype = c_int
    lib.w8_read_floor.argtypes = [vp, ctypes.c_size_t, vp, ctypes.c_size_t, c_int, c_int, c_int,
                                  vp]
    lib.w8_read_floor.restype = st
    lib.w8_status_string.argtypes = [st]
    lib.w8_status_string.restype = ctypes.c_char_p
    lib.w8_last_error.restype = ctypes.c_char_p
    lib.w8_quantize_act.argtypes = [c_int, c_int, c_int, vp, i64, vp, i64, f32p, vp]
    lib.w8_quantize_act.restype = st
    lib.w8_quantize_weight.argtypes = [c_int, c_int, c_int, f32p, i64, vp, i64, f32p, vp]
    lib.w8_quantize_weight.restype = st
    lib.w8_workspace_size.argtypes = [c_int, c_int, c_int, c_int, c_int, c_int, cfgp,
                                      ctypes.POINTER(ctypes.c_size_t)]
    lib.w8_workspace_size.restype = st
    lib.w8_packed_weight_size.argtypes = [c_int, c_int, c_int, c_int,
                                          ctypes.POINTER(ctypes.c_size_t)]
    lib.w8_packed_weight_size.restype = st
    lib.w8_pack_weight.argtypes = [c_int, c_int, c_int, vp, i64, vp, c_int, vp]
    lib.w8_pack_weight.restype = st
    gemm_args = [c_int, c_int, c_int, c_int, vp, i64, f32p, vp, i64, f32p, vp, i64, cfgp, vp,
                 ctypes.c_size_t, vp]
    lib.w8_gemm_w8a8.argtypes = gemm_args
    lib.w8_gemm_w8a8.restype = st
    lib.w8_gemm_w8a8_acc.argtypes = gemm_args
    lib.w8_gemm_w8a8_acc.restype = st
    lib.w8_gemm_w8a8_noalloc.argtypes = [c_int, c_int, c_int, c_int, vp, i64, f32p, vp, i64, f32p,
                                         vp, i64, cfgp, vp]
    lib.w8_gemm_w8a8_noalloc.restype = st
    lib.w8_linear.argtypes = [c_int, c_int, c_int, c_int, vp, i64, vp, i64, f32p, vp, i64, cfgp,
                              vp, ctypes.c_size_t, vp]
    lib.w8_linear.restype = st
    lib.w8_validate_config.argtypes = [c_int, c_int, c_int, c_int, c_int, c_int, cfgp]
    lib.w8_validate_config.restype = st
    lib.w8_default_config.argtypes = [c_int, c_int, c_int, c_int, c_int, c_int, cfgp]
    lib.w8_default_config.restype = st
    lib.w8_resolve_config.argtypes = [c_int, c_int, c_int, c_int, c_int, c_int, cfgp,
                                      ctypes.POINTER(c_int)]
    lib.w8_resolve_config.restype = st
    lib.w8_load_config_table.argtypes = [ctypes.c_char_p]
    lib.w8_load_config_table.restype = st
    lib.w8_save_config_table.argtypes = [ctypes.c_char_p]
    lib.w8_save_config_table.restype = st
    lib.w8_clear_config_table.restype = None
    lib.w8_config_table_size.restype = c_int
    lib.w8_config_table_foreign.restype = c_int
    lib.w8_set_config.argtypes = [c_int, c_int, c_int, c_int, c_int, c_int, cfgp, ctypes.c_double]
    lib.w8_set_config.restype = st
    lib.w8_lookup_config.argtypes = [c_int, c_int, c_int, c_int, c_int, c_int, cfgp,
                                     ctypes.POINTER(ctypes.c_double)]
    lib.w8_lookup_config.restype = st
    lib.w8_tune_shape.argtypes = [c_int, c_int, c_int, c_int, ctypes.POINTER(TuneOpts), cfgp,
                                  ctypes.POINTER(TuneStats)]
    lib.w8_tune_shape.restype = st
    lib.w8_tune_default_opts.argtypes = [ctypes.POINTER(TuneOpts)]
    lib.w8_tune_default_opts.restype = None
    lib.w8_model_config.argtypes = [c_int, c_int, c_int, c_int, c_int, c_int, cfgp]
    lib.w8_model_config.restype = st
    ip = ctypes.POINTER(c_int)
    lib.w8_predict_us.argtypes = [c_int, ip, ip, ip, ip, ip, ip, cfgp,
                                  ctypes.POINTER(ctypes.c_double), c_int,
                                  ctypes.POINTER(ctypes.c_double)]
    lib.w8_predict_us.restype = st
    dp = ctypes.POINTER(ctypes.c_double)
    lib.w8_rank_configs.argtypes = [c_int, c_int, c_int, c_int, ctypes.POINTER(TuneOpts), cfgp,
                                    dp, c_int, ctypes.POINTER(c_int)]
    lib.w8_rank_configs.restype = st
    lib.w8_profile_configs.argtypes = [c_int, c_int, c_int, c_int, ctypes.POINTER(TuneOpts),
                                       cfgp, c_int, dp, ctypes.POINTER(c_int)]
    lib.w8_profile_configs.restype = st
    lib.w8_moe_gemm.argtypes = [c_int, c_int, c_int, c_int, c_int, c_int, vp, i64, f32p, vp, vp,
                                c_int, vp, i64, i64, f32p, i64, vp, i64, cfgp, vp,
                                ctypes.c_size_t, vp]
    lib.w8_moe_gemm.restype = st
    lib.w8_moe_workspace_size.argtypes = [c_int, c_int, c_int, c_int, c_int, c_int, c_int, cfgp,
                                          ctypes.POINTER(ctypes.c_size_t)]
    lib.w8_moe_workspace_size.restype = st
    lib.w8_moe_validate_config.argtypes = [c_int, c_int, c_int, c_int, c_int, c_int, cfgp]
    lib.w8_moe_validate_config.restype = st
    lib.w8_moe_config.argtypes = [c_int, c_int, c_int, c_int, c_int, c_int, c_int, cfgp,
                                  ctypes.POINTER(c_int)]
    lib.w8_moe_config.restype = st
    lib.w8_moe_tune.argtypes = [c_int, c_int, c_int, c_int, c_int, c_int,
                                ctypes.POINTER(TuneOpts), cfgp, ctypes.POINTER(TuneStats)]
    lib.w8_moe_tune.restype = st
    lib.w8_moe_linear.argtypes = [c_int, c_int, c_int, c_int, c_int, c_int, vp, i64, vp, vp,
                                  c_int, vp, i64, i64, f32p, i64, vp, i64, cfgp, vp,
                                  ctypes.c_size_t, vp]
    lib.w8_moe_linear.restype = st
    lib.w8_moe_linear_config.argtypes = [c_int, c_int, c_int, c_int, c_int, c_int, c_int, cfgp,
                                         ctypes.POINTER(c_int)]
    lib.w8_moe_linear_config.restype = st
    return lib
