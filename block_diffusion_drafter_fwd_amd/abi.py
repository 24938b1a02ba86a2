"""ctypes mirror of include/dflash.h and the loader of the native libraries.

Argument marshalling only: every step of the drafter runs in libdflash.so.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int, c_int32, c_int64, c_size_t, c_uint64, c_void_p

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_HIP = os.path.join(HERE, "libdflash.so")
LIB_HOST = os.path.join(HERE, "libdflash_host.so")

OK = 0
E_ARG, E_CONFIG, E_SHAPE, E_CONTEXT_GAP, E_CAPACITY, E_STATE, E_HIP = -1, -2, -3, -4, -5, -6, -7
FP32, BF16 = 0, 1


class Config(ctypes.Structure):
    _fields_ = [(n, c_int32) for n in (
        "dtype", "hidden", "layers", "q_heads", "kv_heads", "head_dim", "taps", "target_hidden",
        "vocab", "block_size", "mask_id", "window", "intermediate", "causal", "qk_norm", "gate",
        "aux_norms", "ctx_input_norm", "fused_qkv", "attention_bias", "flush_rows")] + [
        ("rope_theta", c_float), ("rms_eps", c_float), ("sel_candidates", c_int32), ("sel_dim", c_int32)]


class Tensor(ctypes.Structure):
    _fields_ = [("data", c_void_p), ("ndim", c_int32), ("shape", c_int64 * 2)]


LAYER_FIELDS = ("input_layernorm", "post_attention_layernorm", "q_proj", "k_proj", "v_proj", "qkv_proj",
                "q_norm", "k_norm", "g_proj", "o_proj", "gate_proj", "up_proj", "down_proj")


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, Tensor) for n in LAYER_FIELDS]


class Weights(ctypes.Structure):
    _fields_ = [("embed", Tensor), ("lm_head", Tensor), ("fc", Tensor), ("hidden_norm", Tensor),
                ("norm", Tensor), ("aux_norms", Tensor), ("layers", POINTER(LayerWeights)),
                ("sel_prev", Tensor), ("sel_next", Tensor)]


class SampleParams(ctypes.Structure):
    _fields_ = [("temperature", c_float), ("rep_penalty", c_float), ("history", c_int32), ("round", c_int32)]


class SelectParams(ctypes.Structure):
    _fields_ = [("temperature", c_float), ("round", c_int32)]


class VerifyParams(ctypes.Structure):
    _fields_ = [("temperature", c_float), ("round", c_int32)]


SYMBOLS = {
    "dflash_last_error": (c_char_p, []),
    "dflash_create": (c_int, [POINTER(Config), POINTER(Weights), POINTER(c_void_p)]),
    "dflash_destroy": (None, [c_void_p]),
    "dflash_draft_limit": (c_int, [c_void_p]),
    "dflash_session_bytes": (c_size_t, [c_void_p, c_int32]),
    "dflash_workspace_bytes": (c_size_t, [c_void_p, c_int32]),
    "dflash_session_open": (c_int, [c_void_p, c_void_p, c_size_t, c_int32, c_void_p, c_size_t, c_int32,
                                    c_int32, c_uint64, c_uint64, c_void_p, POINTER(c_void_p)]),
    "dflash_session_close": (c_int, [c_void_p]),
    "dflash_committed": (c_int, [c_void_p, POINTER(c_int32), c_void_p, c_int32, c_int32]),
    "dflash_flush": (c_int, [c_void_p]),
    "dflash_flush_batch": (c_int, [POINTER(c_void_p), c_int32]),
    "dflash_committed_batch": (c_int, [POINTER(c_void_p), c_int32, POINTER(c_int32), POINTER(c_int32),
                                        POINTER(c_void_p), POINTER(c_int32)]),
    "dflash_commit_block": (c_int, [c_void_p]),
    "dflash_propose": (c_int, [c_void_p, c_int32, c_int32, c_void_p, c_void_p, POINTER(c_int32)]),
    "dflash_propose_batch": (c_int, [POINTER(c_void_p), c_int32, POINTER(c_int32), POINTER(c_int32),
                                     c_void_p, POINTER(c_int32)]),
    "dflash_sample": (c_int, [POINTER(c_void_p), c_int32, POINTER(c_int32), c_void_p,
                              POINTER(SampleParams), c_void_p, c_void_p]),
    "dflash_select": (c_int, [POINTER(c_void_p), c_int32, POINTER(c_int32), c_void_p, POINTER(c_int32),
                              POINTER(SelectParams), c_void_p, c_void_p, c_void_p, c_void_p]),
    "dflash_verify": (c_int, [POINTER(c_void_p), c_int32, POINTER(c_int32), c_void_p, c_void_p, c_void_p,
                              POINTER(VerifyParams), c_void_p, c_void_p]),
    "dflash_verify_noalloc": (c_int, [POINTER(c_void_p), c_int32, POINTER(c_int32), c_void_p, c_void_p, c_void_p,
                                      POINTER(VerifyParams), c_void_p, c_void_p]),
    "dflash_width_policy_create": (c_int, [c_int32, c_float, c_float, c_float, c_float, c_float,
                                           POINTER(c_void_p)]),
    "dflash_width_policy_observe": (c_int, [c_void_p, c_int32, c_int32]),
    "dflash_width_policy_choose": (c_int, [c_void_p]),
    "dflash_width_policy_rates": (c_int, [c_void_p, POINTER(c_float)]),
    "dflash_width_policy_destroy": (None, [c_void_p]),
    "dflash_session_state": (c_int, [c_void_p, POINTER(c_int32), POINTER(c_int32), POINTER(c_int32),
                                     POINTER(c_int32), POINTER(c_int64)]),
    "dflash_cache_read": (c_int, [c_void_p, c_int32, c_int32, c_int32, c_void_p, c_void_p]),
    "dflash_profile_begin": (c_int, [c_void_p, c_char_p]),
    "dflash_profile_end": (c_int, [c_void_p, POINTER(ctypes.c_double), POINTER(c_int32)]),
}

_libs = {}


def load(kind: str = "hip") -> ctypes.CDLL:
    """Load libdflash.so ("hip") or the host-only trace build ("host").

    Raises if the library has not been built: there is no fallback.
    """
    if kind in _libs:
        return _libs[kind]
    path = LIB_HIP if kind == "hip" else LIB_HOST
    if not os.path.exists(path):
        raise RuntimeError(f"{os.path.basename(path)} is not built; run "
                           "python -m block_diffusion_drafter_fwd_amd.build")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SYMBOLS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _libs[kind] = lib
    return lib


class DFlashError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"dflash error {code}: {msg}")
        self.code = code


class ContextGap(DFlashError):
    pass


def check(lib, rc: int):
    if rc != 0:
        msg = lib.dflash_last_error().decode(errors="replace")
        raise (ContextGap if rc == E_CONTEXT_GAP else DFlashError)(rc, msg)
    return rc
