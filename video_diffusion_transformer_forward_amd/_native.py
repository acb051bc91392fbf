"""ctypes view of include/wan.h and include/wan_vae.h.  Loads the in-tree libwan.so; no fallback."""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libwan.so")

WAN_OK = 0
WAN_E_NULL = -1
WAN_E_SHAPE = -2
WAN_E_MODE = -3
WAN_E_ALIGN = -4
WAN_E_WORKSPACE = -5
WAN_E_HIP = -6
WAN_E_ENTRY = -7
WAN_E_SCRATCH = -8
NOALLOC_SCRATCH_BYTES = 64 << 20   # WAN_NOALLOC_SCRATCH_BYTES

WAN_BF16 = 0
WAN_FP32 = 1
WAN_BF16_QK8 = 2
WAN_FP8 = 3

ENTRY_PATCHIFY = 0
ENTRY_BLOCK = 1
ENTRY_STEP = 2
ENTRY_TIME_EMBED = 3
ENTRY_HEAD = 4

EXPORTS = ("wan_status_str", "wan_workspace_bytes", "wan_patchify", "wan_time_embed",
           "wan_dit_block_forward", "wan_dit_block_forward_noalloc", "wan_head", "wan_denoise_step", "wan_cache_bytes",
           "wan_denoise_step_cached", "wan_timing_enable", "wan_timing_read",
           "wan_stream_workspace_bytes", "wan_stream_tick",
           "wan_vae_param_count", "wan_vae_param_info", "wan_vae_blob_elems", "wan_vae_workspace_bytes",
           "wan_vae_cache_bytes", "wan_vae_decode")

CACHE_STORE = 1
CACHE_REUSE_ATTN = 2
CACHE_REUSE_UNCOND = 4

KERNEL_SELF_ATTENTION = 0
KERNEL_CROSS_ATTENTION = 1
KERNEL_GEMM = 2
KERNEL_ELEMENTWISE = 3


class WanShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in ("batch", "in_ch", "out_ch", "frames", "height", "width", "dim",
                                           "heads", "ffn_dim", "txt_len", "img_len", "mode")]


_vp = ctypes.c_void_p


class WanVaeShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in ("frames", "height", "width", "z_ch", "base", "n_res", "chunk")]


class WanVaeParam(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("kind", ctypes.c_int), ("dims", ctypes.c_int * 5),
                ("offset", ctypes.c_size_t), ("count", ctypes.c_size_t)]


class WanBlockWeights(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("qkv_w", "qkv_b", "o_w", "o_b", "cq_w", "cq_b", "ckv_w", "ckv_b",
                                   "ikv_w", "ikv_b", "co_w", "co_b", "ff1_w", "ff1_b", "ff2_w", "ff2_b")]


class WanModelWeights(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("pe_w", "pe_b", "t1_w", "t1_b", "t2_w", "t2_b", "m_w", "m_b",
                                   "hd_w", "hd_b")] + [("n_blocks", ctypes.c_int),
                                                       ("blocks", ctypes.POINTER(WanBlockWeights))]


class WanError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{msg} (status {code})")
        self.code = code


_lib = None


def load(path: str = LIB_PATH):
    """Load libwan.so once.  Raises if it is missing: there is no other implementation."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run video_diffusion_transformer_forward_amd.build.build()")
    try:  # share torch's HIP runtime when torch is present (same soname, loaded first)
        import torch  # noqa: F401
    except Exception:
        pass
    lib = ctypes.CDLL(path)
    lib.wan_status_str.restype = ctypes.c_char_p
    lib.wan_status_str.argtypes = [ctypes.c_int]
    lib.wan_workspace_bytes.restype = ctypes.c_size_t
    lib.wan_workspace_bytes.argtypes = [ctypes.POINTER(WanShape), ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
    sp = ctypes.POINTER(WanShape)
    lib.wan_patchify.restype = ctypes.c_int
    lib.wan_patchify.argtypes = [sp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
    lib.wan_time_embed.restype = ctypes.c_int
    lib.wan_time_embed.argtypes = [sp, ctypes.POINTER(WanModelWeights), ctypes.c_float, _vp, _vp, ctypes.c_size_t,
                                   _vp]
    lib.wan_dit_block_forward.restype = ctypes.c_int
    lib.wan_dit_block_forward.argtypes = [sp, ctypes.POINTER(WanBlockWeights), _vp, _vp, ctypes.c_longlong, _vp,
                                          _vp, ctypes.c_size_t, _vp]
    lib.wan_dit_block_forward_noalloc.restype = ctypes.c_int
    lib.wan_dit_block_forward_noalloc.argtypes = [sp, ctypes.POINTER(WanBlockWeights), _vp, _vp, ctypes.c_longlong,
                                                  _vp, _vp]
    lib.wan_head.restype = ctypes.c_int
    lib.wan_head.argtypes = [sp, ctypes.POINTER(WanModelWeights), _vp, _vp, _vp, ctypes.c_size_t, _vp]
    lib.wan_denoise_step.restype = ctypes.c_int
    lib.wan_denoise_step.argtypes = [sp, ctypes.POINTER(WanModelWeights), _vp, _vp, _vp, _vp, ctypes.c_float,
                                     ctypes.c_float, ctypes.c_float, _vp, ctypes.c_size_t, _vp]
    lib.wan_cache_bytes.restype = ctypes.c_size_t
    lib.wan_cache_bytes.argtypes = [sp, ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
    lib.wan_denoise_step_cached.restype = ctypes.c_int
    lib.wan_denoise_step_cached.argtypes = [sp, ctypes.POINTER(WanModelWeights), _vp, _vp, _vp, _vp, ctypes.c_float,
                                            ctypes.c_float, ctypes.c_float, ctypes.c_int, _vp, ctypes.c_size_t, _vp,
                                            ctypes.c_size_t, _vp]
    lib.wan_timing_enable.restype = ctypes.c_int
    lib.wan_timing_enable.argtypes = [ctypes.c_int]
    lib.wan_timing_read.restype = ctypes.c_int
    lib.wan_timing_read.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_double),
                                    ctypes.POINTER(ctypes.c_longlong), ctypes.c_int]
    lib.wan_stream_workspace_bytes.restype = ctypes.c_size_t
    lib.wan_stream_workspace_bytes.argtypes = [sp, ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
    lib.wan_stream_tick.restype = ctypes.c_int
    lib.wan_stream_tick.argtypes = [sp, ctypes.POINTER(WanModelWeights), _vp, _vp, _vp, _vp, ctypes.c_int, _vp, _vp,
                                    _vp, ctypes.c_size_t, _vp]
    vs = ctypes.POINTER(WanVaeShape)
    ip = ctypes.POINTER(ctypes.c_int)
    lib.wan_vae_param_count.restype = ctypes.c_int
    lib.wan_vae_param_count.argtypes = [vs, ip]
    lib.wan_vae_param_info.restype = ctypes.c_int
    lib.wan_vae_param_info.argtypes = [vs, ctypes.c_int, ctypes.POINTER(WanVaeParam)]
    lib.wan_vae_blob_elems.restype = ctypes.c_size_t
    lib.wan_vae_blob_elems.argtypes = [vs, ctypes.c_int, ip]
    lib.wan_vae_workspace_bytes.restype = ctypes.c_size_t
    lib.wan_vae_workspace_bytes.argtypes = [vs, ip]
    lib.wan_vae_cache_bytes.restype = ctypes.c_size_t
    lib.wan_vae_cache_bytes.argtypes = [vs, ip]
    lib.wan_vae_decode.restype = ctypes.c_int
    lib.wan_vae_decode.argtypes = [vs, _vp, _vp, _vp, ctypes.c_int, ctypes.c_int, _vp, ctypes.c_size_t, _vp, _vp,
                                   ctypes.c_size_t, _vp]
    _lib = lib
    return lib


def check(code: int):
    if code != WAN_OK:
        raise WanError(code, load().wan_status_str(code).decode())
    return code
