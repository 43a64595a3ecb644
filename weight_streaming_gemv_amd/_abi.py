"""ctypes declarations of the C ABI in ``include/wsg.h`` (argument marshalling only).

Every function here has the same name and argument order as its C entry
point.  Nothing computes on the host: the calls go straight to
``libwsg.so``, and importing this module fails loudly if the library has
not been built.
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libwsg.so")

WSG_OK, WSG_ERR_INVALID_ARG, WSG_ERR_OUT_OF_RANGE, WSG_ERR_STATE, WSG_ERR_HIP, WSG_ERR_UNSUPPORTED = 0, -1, -2, -3, -4, -5
WSG_F32, WSG_F16 = 0, 1
WSG_W_DENSE, WSG_W_Q4G64 = 0, 1
WSG_OPT_USE_GRAPH, WSG_OPT_TIMED_STAGE = 1, 2
WSG_OPT_FUSE_ATTN_O, WSG_OPT_ROWS_ATTN_O = 3, 15
WSG_OPT_HEAD_WAVES = 16
WSG_OPT_SPLIT_DOWN = 17
WSG_OPT_FOR_TWO_TOKEN = 0x100
WSG_OPT_ROWS = {"qkv": 10, "o": 11, "gateup": 12, "down": 13, "head": 14}
WSG_OPT_GRID = {"qkv": 20, "o": 21, "gateup": 22, "down": 23, "head": 24}
WSG_STAGE_QKV, WSG_STAGE_ATTN, WSG_STAGE_O, WSG_STAGE_GATEUP, WSG_STAGE_DOWN, WSG_STAGE_HEAD = range(6)
WSG_GEMV_NONTEMPORAL = 1
WSG_GEMV_SPLIT2 = 2

STATUS_NAMES = {0: "WSG_OK", -1: "WSG_ERR_INVALID_ARG", -2: "WSG_ERR_OUT_OF_RANGE", -3: "WSG_ERR_STATE",
                -4: "WSG_ERR_HIP", -5: "WSG_ERR_UNSUPPORTED"}


class wsg_config(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("hidden", C.c_int32), ("intermediate", C.c_int32),
                ("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("vocab", C.c_int32), ("max_context", C.c_int32), ("prefill_chunk", C.c_int32),
                ("rms_eps", C.c_float), ("rope_theta", C.c_float), ("dtype", C.c_int32),
                ("lossless_pack", C.c_int32), ("weight_format", C.c_int32)]


_PP = C.POINTER(C.c_void_p)


class wsg_host_weights(C.Structure):
    _fields_ = [("embed", C.c_void_p), ("final_norm", C.c_void_p), ("in_norm", _PP), ("wq", _PP),
                ("wk", _PP), ("wv", _PP), ("q_norm", _PP), ("k_norm", _PP), ("wo", _PP),
                ("post_norm", _PP), ("wg", _PP), ("wu", _PP), ("wd", _PP)]


class wsg_q4_matrix(C.Structure):
    _fields_ = [("words", C.c_void_p), ("scales", C.c_void_p)]


_PQ = C.POINTER(wsg_q4_matrix)


class wsg_host_q4_weights(C.Structure):
    _fields_ = [("embed", wsg_q4_matrix), ("wq", _PQ), ("wk", _PQ), ("wv", _PQ), ("wo", _PQ), ("wg", _PQ),
                ("wu", _PQ), ("wd", _PQ)]


class WsgError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


_lib = None

# name -> (restype, argtypes)
_SIGS = {
    "wsg_packed_weight_bytes": (C.c_int, [C.POINTER(wsg_config), C.POINTER(C.c_size_t)]),
    "wsg_pack_weights": (C.c_int, [C.POINTER(wsg_config), C.POINTER(wsg_host_weights), C.c_void_p, C.c_size_t]),
    "wsg_pack_weights_q4": (C.c_int, [C.POINTER(wsg_config), C.POINTER(wsg_host_weights),
                                      C.POINTER(wsg_host_q4_weights), C.c_void_p, C.c_size_t]),
    "wsg_workspace_bytes": (C.c_int, [C.POINTER(wsg_config), C.POINTER(C.c_size_t)]),
    "wsg_model_create": (C.c_int, [C.POINTER(wsg_config), C.c_void_p, C.c_size_t, C.c_void_p, C.c_size_t,
                                   C.c_void_p, C.POINTER(C.c_void_p)]),
    "wsg_model_destroy": (None, [C.c_void_p]),
    "wsg_reset_cache": (C.c_int, [C.c_void_p]),
    "wsg_prefill": (C.c_int, [C.c_void_p, C.POINTER(C.c_int32), C.c_int32, C.POINTER(C.c_int32),
                              C.POINTER(C.c_void_p)]),
    "wsg_step": (C.c_int, [C.c_void_p, C.c_int32, C.POINTER(C.c_int32), C.POINTER(C.c_void_p)]),
    "wsg_generate": (C.c_int, [C.c_void_p, C.c_int32, C.POINTER(C.c_int32)]),
    "wsg_step2": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.POINTER(C.c_int32), C.POINTER(C.c_int32),
                            C.POINTER(C.c_void_p)]),
    "wsg_position": (C.c_int32, [C.c_void_p]),
    "wsg_kv_view": (C.c_int, [C.c_void_p, C.c_int32, C.POINTER(C.c_void_p), C.POINTER(C.c_void_p),
                              C.POINTER(C.c_int32), C.POINTER(C.c_int64)]),
    "wsg_set_prefill_chunk": (C.c_int, [C.c_void_p, C.c_int32]),
    "wsg_set_option": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32]),
    "wsg_stage_time": (C.c_int, [C.c_void_p, C.POINTER(C.c_double), C.POINTER(C.c_int64),
                                 C.POINTER(C.c_int64)]),
    "wsg_gemv": (C.c_int, [C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p,
                           C.c_void_p, C.c_void_p]),
    "wsg_gemv_ex": (C.c_int, [C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                              C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p]),
    "wsg_gemv_q4g64": (C.c_int, [C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p,
                                 C.c_void_p, C.c_void_p, C.c_void_p]),
    "wsg_gemv_q4g64_ex": (C.c_int, [C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                                    C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p]),
    "wsg_gemm_nt_f32": (C.c_int, [C.c_int32, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p,
                                  C.c_int32, C.c_void_p]),
    "wsg_gemm_swiglu_f32": (C.c_int, [C.c_int32, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p,
                                      C.c_void_p]),
    "wsg_stream_read": (C.c_int, [C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p]),
    "wsg_argmax_workspace_bytes": (C.c_int, [C.c_int32, C.c_int32, C.POINTER(C.c_size_t)]),
    "wsg_argmax": (C.c_int, [C.c_int32, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t,
                             C.c_void_p]),
    "wsg_argmax_noalloc": (C.c_int, [C.c_int32, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p]),
    "wsg_rewind": (C.c_int, [C.c_void_p, C.c_int32]),
    "wsg_weight_storage": (C.c_int, [C.c_void_p, C.POINTER(C.c_int32), C.POINTER(C.c_int32),
                                     C.POINTER(C.c_int64)]),
    "wsg_describe": (C.c_int, [C.c_void_p, C.c_char_p, C.c_size_t, C.POINTER(C.c_size_t)]),
    "wsg_time_stage": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.POINTER(C.c_double), C.POINTER(C.c_int64)]),
    "wsg_last_error": (C.c_char_p, []),
    "wsg_version": (C.c_char_p, []),
}

EXPORTED = tuple(_SIGS)


def lib() -> C.CDLL:
    """The loaded ``libwsg.so``; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                              "(python -m weight_streaming_gemv_amd.build)")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def check(status: int) -> None:
    if status != WSG_OK:
        raise WsgError(status, lib().wsg_last_error().decode())


def _call(name):
    def f(*args):
        return getattr(lib(), name)(*args)
    f.__name__ = name
    return f


# Thin same-name wrappers (raw status codes returned, nothing converted).
for _n in _SIGS:
    globals()[_n] = _call(_n)
