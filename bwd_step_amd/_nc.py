"""ctypes binding of the C ABI in include/nc.h (argument marshalling only).

Every function here forwards to the shared library ``bwd_step_amd/libnc.so``;
all compute happens in its HIP kernels.  Loading fails loudly if the library
has not been built: there is no fallback path.
"""

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libnc.so")

NC_OK = 0
NC_BF16 = 0
NC_FP32 = 1
DECODE_SCRATCH_BYTES = 32 << 20  # NC_DECODE_SCRATCH_BYTES in include/nc.h
STATUS = {
    0: "NC_OK", 1: "NC_ERR_CONFIG", 2: "NC_ERR_NULL", 3: "NC_ERR_WORKSPACE",
    4: "NC_ERR_TOKEN_RANGE", 5: "NC_ERR_NONFINITE", 6: "NC_ERR_HIP",
    7: "NC_ERR_UNSUPPORTED", 8: "NC_ERR_ARG",
}

# Every symbol include/nc.h declares, with (restype, argtypes).
_vp, _i, _u64, _f = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64, ctypes.c_float


class NcConfig(ctypes.Structure):
    _fields_ = [
        ("depth", ctypes.c_int32), ("d_model", ctypes.c_int32), ("n_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("d_ff", ctypes.c_int32), ("vocab", ctypes.c_int32),
        ("seq_len", ctypes.c_int32), ("max_batch", ctypes.c_int32),
        ("rope_base", ctypes.c_float), ("norm_eps", ctypes.c_float), ("dtype", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
    ]


class NcTensorDesc(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("offset", ctypes.c_uint64),
                ("rows", ctypes.c_int32), ("cols", ctypes.c_int32)]


class NcOptimConfig(ctypes.Structure):
    _fields_ = [
        ("lr_adamw", ctypes.c_float), ("lr_muon", ctypes.c_float), ("beta1", ctypes.c_float),
        ("beta2", ctypes.c_float), ("eps", ctypes.c_float), ("momentum", ctypes.c_float),
        ("weight_decay", ctypes.c_float), ("clip", ctypes.c_float), ("final_frac", ctypes.c_float),
        ("warmup_steps", ctypes.c_int32), ("total_steps", ctypes.c_int32), ("ns_steps", ctypes.c_int32),
    ]


class NcProfEntry(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", ctypes.c_int64), ("ms", ctypes.c_double),
                ("flops", ctypes.c_double), ("bytes", ctypes.c_double)]


SIGNATURES = {
    "nc_strerror": (ctypes.c_char_p, [_i]),
    "nc_init": (_i, [ctypes.POINTER(NcConfig), _vp, ctypes.POINTER(_vp)]),
    "nc_destroy": (None, [_vp]),
    "nc_get_config": (_i, [_vp, ctypes.POINTER(NcConfig)]),
    "nc_set_stream": (_i, [_vp, _vp]),
    "nc_param_count": (_u64, [_vp]),
    "nc_param_layout": (_i, [_vp, ctypes.POINTER(NcTensorDesc), _i]),
    "nc_workspace_bytes": (_u64, [_vp, _i]),
    "nc_set_workspace": (_i, [_vp, _vp, _u64]),
    "nc_forward_backward": (_i, [_vp, _vp, _vp, _vp, _i, _vp, _vp, _i]),
    "nc_forward_backward_accum": (_i, [_vp, _vp, _vp, _vp, _i, _i, _vp, _vp]),
    "nc_forward_logits": (_i, [_vp, _vp, _vp, _i, _vp]),
    "nc_kv_cache_bytes": (_u64, [_vp, _i, _i]),
    "nc_decode_workspace_bytes": (_u64, [_vp, _i, _i]),
    "nc_prefill": (_i, [_vp, _vp, _vp, _i, _i, _vp, _i, _i, _i, _vp]),
    "nc_decode": (_i, [_vp, _vp, _vp, _vp, _i, _vp, _i, _vp, _u64, _vp]),
    "nc_decode_static": (_i, [_vp, _vp, _vp, _vp, _i, _vp, _i, _vp, _vp]),
    "nc_check": (_i, [_vp]),
    "nc_debug_poison_workspace": (_i, [_vp, _i]),
    "nc_set_residual_fp32": (_i, [_vp, _i]),
    "nc_profile_enable": (_i, [_vp, _i]),
    "nc_profile_read": (_i, [_vp, ctypes.POINTER(NcProfEntry), _i]),
    "nc_attention_workspace_bytes": (_u64, [_i, _i, _i, _i, _i]),
    "nc_attention_fwd_bwd": (_i, [_vp] * 8 + [_i, _i, _i, _i, _f, _f, _i, _vp, _u64, _vp]),
    "nc_lmhead_ce_workspace_bytes": (_u64, [_i, _i, _i, _i]),
    "nc_lmhead_ce_fwd_bwd": (_i, [_vp, _vp, _vp, _i, _i, _i, _vp, _vp, _vp, _i, _vp, _u64, _vp]),
    "nc_op_status": (_i, [_vp, _vp]),
    "nc_rmsnorm_fwd": (_i, [_vp, _vp, _vp, _i, _i, _f, _i, _vp]),
    "nc_rmsnorm_bwd": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp]),
    "nc_embedding_fwd": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _vp, _vp]),
    "nc_embedding_bwd_workspace_bytes": (_u64, [_i, _i, _i]),
    "nc_embedding_bwd": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _vp, _u64, _vp]),
    "nc_gemm_workspace_bytes": (_u64, [_i, _i, _i, _i]),
    "nc_gemm": (_i, [_vp, _i, _i, _vp, _i, _i, _vp, _i, _i, _i, _i, _i, _i, _vp, _u64, _vp]),
    "nc_optim_state_bytes": (_u64, [_vp]),
    "nc_optim_workspace_bytes": (_u64, [_vp]),
    "nc_optim_init": (_i, [_vp, _vp, _vp]),
    "nc_optim_step": (_i, [_vp, ctypes.POINTER(NcOptimConfig), _i, _vp, _vp, _vp, _vp, _u64, _vp]),
}

_lib = None


class NcError(RuntimeError):
    def __init__(self, code, where=""):
        self.code = code
        super().__init__(f"{where}: {STATUS.get(code, code)} ({strerror(code)})")


def lib():
    """Load libnc.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        # torch first: its HIP runtime must be the one libnc.so binds to, or the
        # streams and memory torch hands over belong to another runtime
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with bwd_step_amd/build.py "
                              "(or __graft_entry__.build())")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


def strerror(code):
    try:
        return lib().nc_strerror(code).decode()
    except ImportError:
        return "?"


def check(code, where=""):
    if code != NC_OK:
        raise NcError(code, where)
    return code
