"""ctypes view of libdflash.so (the C ABI declared in include/dflash.h).

Argument marshalling only: every step of the drafter runs in the HIP library.
Importing this module never falls back to anything else; if the library is
missing it raises, telling the caller to build it.
"""
from __future__ import annotations

import ctypes as C
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libdflash.so")

F32, BF16, FP8_E4M3 = 0, 1, 2
DTYPES = {"f32": F32, "bf16": BF16, "fp8": FP8_E4M3}

OK, EINVAL, ERANGE, EUNSUPPORTED, EHIP, ESTATE = 0, -1, -2, -3, -4, -5
STAGE_QKV, STAGE_O, STAGE_GATE_UP, STAGE_DOWN = 0, 1, 2, 3
PATH_AUTO, PATH_KERNELS, PATH_PERSISTENT = 0, 1, 2


class Config(C.Structure):
    _fields_ = [
        ("n_layer", C.c_int32), ("n_embd", C.c_int32), ("n_head", C.c_int32), ("n_head_kv", C.c_int32),
        ("head_dim", C.c_int32), ("n_ff", C.c_int32), ("window", C.c_int32), ("block", C.c_int32),
        ("n_vocab", C.c_int32), ("n_capture", C.c_int32), ("target_hidden", C.c_int32), ("mask_id", C.c_int32),
        ("max_batch", C.c_int32), ("max_inject", C.c_int32), ("rms_eps", C.c_float), ("rope_base", C.c_double),
        ("weight_dtype", C.c_int32), ("aux_dtype", C.c_int32), ("ring_dtype", C.c_int32),
        ("feature_dtype", C.c_int32),
    ]


class LayerWeights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("attn_norm", "wq", "wk", "wv", "wo", "q_norm", "k_norm", "ffn_norm",
                                            "w_gate", "w_up", "w_down")] + \
               [(n, C.c_void_p) for n in ("s_q", "s_k", "s_v", "s_o", "s_gate", "s_up", "s_down")]


class Weights(C.Structure):
    _fields_ = [("tok_embd", C.c_void_p), ("lm_head", C.c_void_p), ("fc", C.c_void_p),
                ("hidden_norm", C.c_void_p), ("output_norm", C.c_void_p), ("s_lm_head", C.c_void_p),
                ("layers", C.POINTER(LayerWeights))]


SYMBOLS = {
    "dflash_workspace_bytes": (C.c_size_t, [C.POINTER(Config)]),
    "dflash_ring_bytes": (C.c_size_t, [C.POINTER(Config)]),
    "dflash_create": (C.c_int, [C.POINTER(Config), C.POINTER(Weights), C.c_void_p, C.c_size_t, C.c_void_p,
                                C.POINTER(C.c_void_p)]),
    "dflash_destroy": (None, [C.c_void_p]),
    "dflash_ring_reset": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p]),
    "dflash_encode": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p]),
    "dflash_encode_static": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p]),
    "dflash_inject": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p]),
    "dflash_inject_batch": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p,
                                      C.c_int32, C.c_void_p]),
    "dflash_block_step": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p,
                                    C.c_void_p, C.c_void_p]),
    "dflash_block_step_accept": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p,
                                           C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p]),
    "dflash_block_forward": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p,
                                       C.c_void_p, C.c_void_p]),
    "dflash_accept": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p]),
    "dflash_accept_bonus": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p,
                                      C.c_void_p]),
    "dflash_step_graph_create": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p,
                                           C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                           C.POINTER(C.c_void_p)]),
    "dflash_step_graph_launch": (C.c_int, [C.c_void_p, C.c_void_p]),
    "dflash_graph_destroy": (None, [C.c_void_p]),
    "dflash_replay_stage": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.c_void_p]),
    "dflash_quantize_fp8_rows": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p]),
    "dflash_set_path": (C.c_int, [C.c_void_p, C.c_int32]),
    "dflash_set_block_width": (C.c_int, [C.c_void_p, C.c_int32]),
    "dflash_block_width": (C.c_int32, [C.c_void_p]),
    "dflash_set_sampling": (C.c_int, [C.c_void_p, C.c_float, C.c_uint64]),
    "dflash_page_bytes": (C.c_size_t, [C.c_void_p]),
    "dflash_set_paged_pool": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int32]),
    "dflash_pages_reset": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.c_void_p]),
    "dflash_step_path": (C.c_int32, [C.c_void_p, C.c_int32]),
    "dflash_check_device": (C.c_int, [C.c_void_p, C.c_void_p]),
    "dflash_set_wait_limit": (C.c_int, [C.c_void_p, C.c_int64, C.c_void_p]),
    "dflash_last_error": (C.c_char_p, []),
}

_lib = None


class DFlashError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"dflash error {code}: {msg}")
        self.code = code


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(or python -m block_diffusion_drafter_02_amd.build)")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in SYMBOLS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def check(rc: int) -> None:
    if rc != OK:
        raise DFlashError(rc, lib().dflash_last_error().decode())


def make_config(shape, weight_dtype: str, ring_dtype: str, feature_dtype: str, max_batch: int = 1,
                max_inject: int = 64, aux_dtype: str | None = None) -> Config:
    if aux_dtype is None:
        aux_dtype = "f32" if weight_dtype == "f32" else "bf16"
    return Config(
        n_layer=shape.n_layer, n_embd=shape.n_embd, n_head=shape.n_head, n_head_kv=shape.n_head_kv,
        head_dim=shape.head_dim, n_ff=shape.n_ff, window=shape.window, block=shape.block, n_vocab=shape.n_vocab,
        n_capture=shape.n_capture, target_hidden=shape.target_hidden, mask_id=shape.mask_id,
        max_batch=max_batch, max_inject=max_inject, rms_eps=shape.rms_eps, rope_base=shape.rope_base,
        weight_dtype=DTYPES[weight_dtype], aux_dtype=DTYPES[aux_dtype], ring_dtype=DTYPES[ring_dtype],
        feature_dtype=DTYPES[feature_dtype],
    )
