"""ctypes loader for ``libdrafter_attn.so`` (the C ABI of include/drafter_attn.h)."""
import ctypes
import os
import threading

_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdrafter_attn.so")
_lock = threading.Lock()
_lib = None

c_i32, c_i64, c_f32, c_sz, c_vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p
c_i32p = ctypes.POINTER(ctypes.c_int32)


class DaYarn(ctypes.Structure):
    """struct da_yarn of the header (YaRN rotary scaling parameters, passed by host pointer)."""
    _fields_ = [("factor", ctypes.c_float), ("original_max_position", ctypes.c_int32),
                ("alpha", ctypes.c_float), ("beta", ctypes.c_float),
                ("ramp", ctypes.c_int32), ("mscale", ctypes.c_float)]


YARN_RAMPS = {"turns": 0, "index": 1, "index_unrounded": 2}  # DA_YARN_RAMP_* of the header


c_yarnp = ctypes.POINTER(DaYarn)

# name -> (restype, argtypes), in the header's order
SIGNATURES = {
    "drafter_attn_workspace_bytes": (c_sz, [c_i32, c_i32, c_i32, c_i32, c_i32, c_i32]),
    "drafter_attn_plan": (ctypes.c_int, [c_i32, c_i32, c_i32, c_i32p, c_i32p]),
    "drafter_attn": (ctypes.c_int, [
        c_vp, c_i64,                  # qkv, qkv_row_stride
        c_vp, c_vp, c_i64, c_i32,     # k_pool, v_pool, pool_page_stride, num_pages
        c_vp, c_i32,                  # page_table, page_table_stride
        c_vp, c_vp,                   # context_lens, block_lens
        c_i32, c_i32, c_i32, c_i32,   # R, T, Hq, Hkv
        c_i32, c_i32,                 # head_dim, page_size
        c_f32,                        # scale
        c_vp, c_sz,                   # workspace, workspace_bytes
        c_vp, c_i64,                  # out, out_row_stride
        c_vp, c_vp,                   # status_word, stream
    ]),
    "drafter_attn_qknorm": (ctypes.c_int, [
        c_vp, c_i64,
        c_vp, c_vp, c_i64, c_i32,
        c_vp, c_i32,
        c_vp, c_vp,
        c_i32, c_i32, c_i32, c_i32,
        c_i32, c_i32,
        c_f32,
        c_vp, c_i32,                  # positions, positions_dtype
        c_vp, c_vp,                   # q_norm_weight, k_norm_weight
        c_f32, c_f32,                 # eps, rope_base
        c_vp, c_sz,
        c_vp, c_i64,
        c_vp, c_vp,
    ]),
    "drafter_attn_qknorm_yarn": (ctypes.c_int, [
        c_vp, c_i64,
        c_vp, c_vp, c_i64, c_i32,
        c_vp, c_i32,
        c_vp, c_vp,
        c_i32, c_i32, c_i32, c_i32,
        c_i32, c_i32,
        c_f32,
        c_vp, c_i32,
        c_vp, c_vp,
        c_f32, c_f32, c_yarnp,        # eps, rope_base, yarn (host struct)
        c_vp, c_sz,
        c_vp, c_i64,
        c_vp, c_vp,
    ]),
    "drafter_attn_qknorm_noalloc": (ctypes.c_int, [
        c_vp, c_i64,
        c_vp, c_vp, c_i64, c_i32,
        c_vp, c_i32,
        c_vp, c_vp,
        c_i32, c_i32, c_i32, c_i32,
        c_i32, c_i32,
        c_f32,
        c_vp, c_i32,
        c_vp, c_vp,
        c_f32, c_f32,
        c_vp, c_i64,                  # out, out_row_stride (no workspace: the library's scratch)
        c_vp, c_vp,
    ]),
    "drafter_qk_norm_rope": (ctypes.c_int, [
        c_vp, c_i64, c_i32,           # qkv, qkv_row_stride, num_tokens
        c_i32, c_i32, c_i32,          # Hq, Hkv, head_dim
        c_vp, c_i32,                  # positions, positions_dtype
        c_vp, c_vp,                   # q_norm_weight, k_norm_weight
        c_f32, c_f32,                 # eps, rope_base
        c_vp,                         # stream
    ]),
    "drafter_qk_norm_rope_yarn": (ctypes.c_int, [
        c_vp, c_i64, c_i32,
        c_i32, c_i32, c_i32,
        c_vp, c_i32,
        c_vp, c_vp,
        c_f32, c_f32, c_yarnp,        # eps, rope_base, yarn (host struct)
        c_vp,
    ]),
    "drafter_kv_append": (ctypes.c_int, [
        c_vp, c_i64,                  # qkv, qkv_row_stride
        c_vp, c_vp, c_i64, c_i32,     # k_pool, v_pool, pool_page_stride, num_pages
        c_vp, c_i32,                  # page_table, page_table_stride
        c_vp, c_vp,                   # context_lens, block_lens
        c_i32, c_i32, c_i32, c_i32,   # R, T, Hq, Hkv
        c_i32, c_i32,                 # head_dim, page_size
        c_vp, c_vp,                   # status_word, stream
    ]),
    "drafter_paged_attn": (ctypes.c_int, [
        c_vp, c_i64,
        c_vp, c_vp, c_i64, c_i32,
        c_vp, c_i32,
        c_vp, c_vp,                   # kv_lens, block_lens
        c_i32, c_i32, c_i32, c_i32,
        c_i32, c_i32,
        c_f32,
        c_vp, c_sz,
        c_vp, c_i64,
        c_vp, c_vp,
    ]),
    "drafter_attn_last_error": (ctypes.c_char_p, []),
}


def library_path() -> str:
    return _PATH


def load():
    """Load the HIP library once; raise ImportError if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_PATH):
            raise ImportError(
                f"{_PATH} is missing: build it with `python -m speculative_decoding_drafter_amd.build` "
                "(there is no fallback path)")
        lib = ctypes.CDLL(_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def last_error() -> str:
    return load().drafter_attn_last_error().decode()
