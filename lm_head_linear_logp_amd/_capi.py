"""ctypes mirror of include/llp.h (structs, constants, function signatures)."""
from __future__ import annotations

import ctypes as C
import os

LLP_OK = 0
LLP_ERR_UNAVAILABLE = 1
LLP_ERR_INVALID_ARGUMENT = 2
LLP_ERR_UNSUPPORTED = 3
LLP_ERR_HIP = 4
LLP_ERR_INTERNAL = 5
STATUS_NAMES = {0: "OK", 1: "UNAVAILABLE", 2: "INVALID_ARGUMENT", 3: "UNSUPPORTED", 4: "HIP",
                5: "INTERNAL"}

LLP_STATUS_TARGET_OUT_OF_RANGE = 1
LLP_STATUS_TARGET_NOT_FOUND = 2
LLP_STATUS_REPLAY_ID_INVALID = 4
LLP_STATUS_LAYOUT_INVALID = 8

LLP_DTYPE_BF16 = 1
LLP_DTYPE_F32 = 2
LLP_OP_FORWARD = 1
LLP_OP_BACKWARD = 2
LLP_FLAG_WANT_ENTROPY = 1
LLP_FLAG_OVERWRITE_GRADS = 2
LLP_FLAG_G_SLABS = 4
LLP_G_SLAB_COLUMNS = 32768
LLP_MAX_REPLAY_IDS = 64
LLP_MAX_WORLD = 64

vp = C.c_void_p


class llp_info(C.Structure):
    _fields_ = [("name", C.c_char * 32), ("version", C.c_char * 16), ("arch", C.c_char * 32),
                ("route", C.c_char * 128), ("max_replay_ids", C.c_int32),
                ("num_cus", C.c_int32), ("device", C.c_int32), ("reserved", C.c_int32)]


class llp_projection(C.Structure):
    _fields_ = [("hidden", vp), ("hidden_stride", C.c_int64), ("weight", vp),
                ("weight_stride", C.c_int64), ("bias", vp), ("bias_dtype", C.c_int32),
                ("reserved", C.c_int32), ("hidden_size", C.c_int64)]


class llp_vocab_partition(C.Structure):
    _fields_ = [("offset", C.c_int64), ("local_size", C.c_int64), ("real_vocab", C.c_int64),
                ("padded_vocab", C.c_int64), ("rank", C.c_int32), ("world", C.c_int32)]


class llp_token_layout(C.Structure):
    _fields_ = [("num_tokens", C.c_int64), ("num_seqs", C.c_int32), ("reserved", C.c_int32),
                ("cu_seqlens", vp), ("loss_mask", vp)]


class llp_request(C.Structure):
    _fields_ = [("proj", llp_projection), ("vocab", llp_vocab_partition),
                ("layout", llp_token_layout), ("target_ids", vp), ("temperature", C.c_float),
                ("flags", C.c_uint32), ("status_word", vp)]


class llp_partials(C.Structure):
    _fields_ = [("target_logit", vp), ("in_range", vp), ("lse", vp), ("entropy", vp),
                ("logp", vp)]


class llp_final_out(C.Structure):
    _fields_ = [("logp", vp), ("lse", vp), ("entropy", vp)]


class llp_bwd_in(C.Structure):
    _fields_ = [("lse", vp), ("dlogp", vp), ("dentropy", vp), ("entropy", vp)]


class llp_bwd_out(C.Structure):
    _fields_ = [("dhidden", vp), ("dhidden_stride", C.c_int64), ("dweight", vp),
                ("dweight_stride", C.c_int64), ("dbias", vp)]


class llp_topp_request(C.Structure):
    _fields_ = [("logits", vp), ("logits_dtype", C.c_int32), ("num_replay", C.c_int32),
                ("logits_stride", C.c_int64), ("num_tokens", C.c_int64),
                ("vocab", llp_vocab_partition), ("replay_ids", vp), ("replay_stride", C.c_int64),
                ("target_ids", vp), ("loss_mask", vp), ("temperature", C.c_float),
                ("processed_logprobs", C.c_int32), ("status_word", vp)]


class llp_logits_request(C.Structure):
    _fields_ = [("logits", vp), ("logits_dtype", C.c_int32), ("reserved", C.c_int32),
                ("logits_stride", C.c_int64), ("vocab", llp_vocab_partition),
                ("layout", llp_token_layout), ("target_ids", vp), ("temperature", C.c_float),
                ("flags", C.c_uint32), ("status_word", vp)]


class llp_keep_mask_request(C.Structure):
    _fields_ = [("logits", vp), ("logits_dtype", C.c_int32), ("processed_logprobs", C.c_int32),
                ("logits_stride", C.c_int64), ("keep_mask", vp), ("keep_stride", C.c_int64),
                ("num_tokens", C.c_int64), ("vocab", llp_vocab_partition), ("target_ids", vp),
                ("loss_mask", vp), ("temperature", C.c_float), ("reserved", C.c_int32),
                ("status_word", vp)]


SIGNATURES = {
    "llp_open": (C.c_int, [C.c_int32, C.POINTER(llp_info)]),
    "llp_workspace_bytes": (C.c_int, [C.POINTER(llp_request), C.c_int32, C.POINTER(C.c_size_t)]),
    "llp_forward": (C.c_int, [C.POINTER(llp_request), C.POINTER(llp_partials), vp, C.c_size_t, vp]),
    "llp_forward_noalloc": (C.c_int, [C.POINTER(llp_request), C.POINTER(llp_partials), vp]),
    "llp_merge": (C.c_int, [C.c_int32, C.POINTER(llp_partials), C.c_int64, vp,
                            C.POINTER(llp_final_out), vp, vp]),
    "llp_backward": (C.c_int, [C.POINTER(llp_request), C.POINTER(llp_bwd_in),
                               C.POINTER(llp_bwd_out), vp, C.c_size_t, vp]),
    "llp_top_p_replay": (C.c_int, [C.POINTER(llp_topp_request), C.POINTER(llp_partials), vp]),
    "llp_forward_logits": (C.c_int, [C.POINTER(llp_logits_request), C.POINTER(llp_partials), vp]),
    "llp_keep_mask_replay": (C.c_int, [C.POINTER(llp_keep_mask_request), C.POINTER(llp_partials),
                                       vp]),
    "llp_last_error": (C.c_char_p, []),
}

# The in-tree build; LLP_LIBRARY may name another build of the same sources.
LIB_PATH = os.environ.get("LLP_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libllp.so")
_lib = None


def load() -> C.CDLL:
    """Load the in-tree HIP library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing "
                           "(python -m lm_head_linear_logp_amd.build)")
    lib = C.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib
