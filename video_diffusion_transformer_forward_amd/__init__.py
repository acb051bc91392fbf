"""Wan2.1 DiT block and CFG/Euler denoise step on MI355X (gfx950).

Thin torch-facing binding of libwan.so (include/wan.h): every function below
only marshals tensor pointers, shapes and the current HIP stream into the C ABI.
All computation runs in the library's HIP kernels; there is no other path.
PyTorch provides device memory and streams.
"""
from __future__ import annotations

import ctypes

from . import _native as N
from ._native import WanError  # noqa: F401
from .synth import WanConfig

__all__ = ["shape_of", "DeviceBlock", "DeviceModel", "workspace", "workspace_bytes", "patchify", "time_embed",
           "cache_bytes", "diffusion_cache", "denoise_step_cached",
           "dit_block_forward", "dit_block_forward_noalloc", "head", "denoise_step", "timing_enable", "timing_read",
           "WanError",
           "vae_shape_of", "vae_param_table", "VaeDevice", "vae_workspace", "vae_cache", "vae_decode",
           "stream_workspace", "stream_tick"]


def _torch():
    import torch
    return torch


def elem_dtype(cfg: WanConfig):
    torch = _torch()
    return torch.bfloat16 if cfg.mode == "bf16" else torch.float32


def shape_of(cfg: WanConfig) -> N.WanShape:
    return N.WanShape(cfg.batch, cfg.in_ch, cfg.out_ch, cfg.frames, cfg.height, cfg.width, cfg.dim, cfg.heads,
                      cfg.ffn_dim, cfg.txt_len, cfg.img_len, _mode_id(cfg))


def _mode_id(cfg: WanConfig) -> int:
    if cfg.mode == "bf16":
        if cfg.fp8:
            return N.WAN_FP8
        return N.WAN_BF16_QK8 if cfg.qk8 else N.WAN_BF16
    if cfg.qk8 or cfg.fp8:
        raise ValueError("the 8-bit forms need mode 'bf16'")
    return N.WAN_FP32


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def workspace_bytes(cfg: WanConfig, entry: int) -> int:
    lib = N.load()
    st = ctypes.c_int(0)
    sh = shape_of(cfg)
    n = lib.wan_workspace_bytes(ctypes.byref(sh), entry, ctypes.byref(st))
    N.check(st.value)
    return int(n)


def workspace(cfg: WanConfig, entry: int, device="cuda"):
    torch = _torch()
    n = workspace_bytes(cfg, entry)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def _dev(a, dtype, device):
    torch = _torch()
    return torch.as_tensor(a).to(device=device, dtype=dtype).contiguous()


class DeviceBlock:
    """One block's weights resident on the device, plus the ABI struct pointing at them."""

    def __init__(self, cfg: WanConfig, w: dict, device="cuda"):
        torch = _torch()
        et = elem_dtype(cfg)
        self.t = {k: _dev(v, torch.float32 if k.endswith("_b") else et, device) for k, v in w.items()}
        f = {k: _ptr(v) for k, v in self.t.items()}
        self.struct = N.WanBlockWeights(*[f.get(n) for n, _ in N.WanBlockWeights._fields_])


class DeviceModel:
    """Model-level weights (patch embedding, time MLP, head) and a list of DeviceBlock."""

    def __init__(self, cfg: WanConfig, mw: dict, blocks=(), device="cuda"):
        torch = _torch()
        et = elem_dtype(cfg)
        self.t = {k: _dev(v, torch.float32 if k.endswith("_b") else et, device) for k, v in mw.items()}
        self.blocks = list(blocks)
        self._arr = (N.WanBlockWeights * max(1, len(self.blocks)))(*[b.struct for b in self.blocks])
        f = {k: _ptr(v) for k, v in self.t.items()}
        vals = [f.get(n) for n, _ in N.WanModelWeights._fields_[:10]]
        self.struct = N.WanModelWeights(*vals, len(self.blocks),
                                        ctypes.cast(self._arr, ctypes.POINTER(N.WanBlockWeights)))


def patchify(cfg, z, cond, pe_w, pe_b, x, stream=None):
    """wan_patchify: x (B, L, D) float32 <- (1,2,2) patch embedding of [z ; cond]."""
    lib = N.load()
    sh = shape_of(cfg)
    N.check(lib.wan_patchify(ctypes.byref(sh), _ptr(z), _ptr(cond), _ptr(pe_w), _ptr(pe_b), _ptr(x), None, 0,
                             _stream(stream)))
    return x


def time_embed(cfg, model: DeviceModel, timestep: float, mod, ws, stream=None):
    """wan_time_embed: mod (6, D) float32 from the timestep."""
    lib = N.load()
    sh = shape_of(cfg)
    N.check(lib.wan_time_embed(ctypes.byref(sh), ctypes.byref(model.struct), float(timestep), _ptr(mod), _ptr(ws),
                               ws.numel(), _stream(stream)))
    return mod


def dit_block_forward(cfg, block: DeviceBlock, x, mod, ctx, ws, mod_batch_stride=None, stream=None):
    """wan_dit_block_forward: one block in place on x (B, L, D) float32."""
    lib = N.load()
    sh = shape_of(cfg)
    if mod_batch_stride is None:
        mod_batch_stride = 6 * cfg.dim if mod.dim() == 3 else 0
    N.check(lib.wan_dit_block_forward(ctypes.byref(sh), ctypes.byref(block.struct), _ptr(x), _ptr(mod),
                                      int(mod_batch_stride), _ptr(ctx), _ptr(ws), ws.numel(), _stream(stream)))
    return x


def dit_block_forward_noalloc(cfg, block: DeviceBlock, x, mod, ctx, mod_batch_stride=None, stream=None):
    """wan_dit_block_forward_noalloc: one block in place on x, on the library's fixed device scratch
    (no workspace argument; WanError WAN_E_SCRATCH when the shape needs more than it holds)."""
    lib = N.load()
    sh = shape_of(cfg)
    if mod_batch_stride is None:
        mod_batch_stride = 6 * cfg.dim if mod.dim() == 3 else 0
    N.check(lib.wan_dit_block_forward_noalloc(ctypes.byref(sh), ctypes.byref(block.struct), _ptr(x), _ptr(mod),
                                              int(mod_batch_stride), _ptr(ctx), _stream(stream)))
    return x


def head(cfg, model: DeviceModel, x, v, ws, stream=None):
    """wan_head: v (B, 16, F, H, W) float32 from the residual stream x."""
    lib = N.load()
    sh = shape_of(cfg)
    N.check(lib.wan_head(ctypes.byref(sh), ctypes.byref(model.struct), _ptr(x), _ptr(v), _ptr(ws), ws.numel(),
                         _stream(stream)))
    return v


def timing_enable(on: bool = True):
    """Bracket library kernel launches with HIP events (measurement only)."""
    N.check(N.load().wan_timing_enable(1 if on else 0))


def timing_read(kernel_class: int, reset: bool = True):
    """(total ms, launches) of one kernel class since the last reset; waits for its events."""
    ms = ctypes.c_double(0)
    n = ctypes.c_longlong(0)
    N.check(N.load().wan_timing_read(kernel_class, ctypes.byref(ms), ctypes.byref(n), 1 if reset else 0))
    return ms.value, n.value


def cache_bytes(cfg: WanConfig, n_blocks: int) -> int:
    """wan_cache_bytes: device bytes of the diffusion cache for cfg's shape and n_blocks blocks."""
    lib = N.load()
    sh = shape_of(cfg)
    st = ctypes.c_int(0)
    n = lib.wan_cache_bytes(ctypes.byref(sh), int(n_blocks), ctypes.byref(st))
    N.check(st.value)
    return int(n)


def diffusion_cache(cfg: WanConfig, n_blocks: int, device="cuda"):
    torch = _torch()
    return torch.empty(cache_bytes(cfg, n_blocks), dtype=torch.uint8, device=device)


def denoise_step_cached(cfg, model: DeviceModel, z, cond, ctx_cond, ctx_null, timestep, dt, guide_scale, mode,
                        cache, ws, stream=None):
    """wan_denoise_step_cached: one CFG + Euler step under a diffusion-cache mode (CACHE_*)."""
    lib = N.load()
    sh = shape_of(cfg)
    N.check(lib.wan_denoise_step_cached(ctypes.byref(sh), ctypes.byref(model.struct), _ptr(z), _ptr(cond),
                                        _ptr(ctx_cond), _ptr(ctx_null), float(timestep), float(dt),
                                        float(guide_scale), int(mode), _ptr(cache), cache.numel(), _ptr(ws),
                                        ws.numel(), _stream(stream)))
    return z


def denoise_step(cfg, model: DeviceModel, z, cond, ctx_cond, ctx_null, timestep, dt, guide_scale, ws, stream=None):
    """wan_denoise_step: one CFG + Euler step in place on z (B, 16, F, H, W) float32."""
    lib = N.load()
    sh = shape_of(cfg)
    N.check(lib.wan_denoise_step(ctypes.byref(sh), ctypes.byref(model.struct), _ptr(z), _ptr(cond), _ptr(ctx_cond),
                                 _ptr(ctx_null), float(timestep), float(dt), float(guide_scale), _ptr(ws),
                                 ws.numel(), _stream(stream)))
    return z


# ----------------------------------------------------------------------------- Wan-VAE decoder
def vae_shape_of(cfg, chunk=None) -> N.WanVaeShape:
    """wan_vae_shape of a VaeConfig; chunk: most latent frames per call (default: all)."""
    return N.WanVaeShape(cfg.frames, cfg.height, cfg.width, cfg.z_ch, cfg.base, cfg.n_res,
                         cfg.frames if chunk is None else int(chunk))


def vae_param_table(sh: N.WanVaeShape):
    """[(name, kind, dims, offset, count)] from wan_vae_param_info."""
    lib = N.load()
    st = ctypes.c_int(0)
    n = lib.wan_vae_param_count(ctypes.byref(sh), ctypes.byref(st))
    N.check(st.value)
    out = []
    info = N.WanVaeParam()
    for i in range(n):
        N.check(lib.wan_vae_param_info(ctypes.byref(sh), i, ctypes.byref(info)))
        k = info.kind
        out.append((info.name.decode(), k, tuple(info.dims[:5 if k == 0 else 1]), int(info.offset), int(info.count)))
    return out


class VaeDevice:
    """The decoder's parameters in the library's two device blobs (bf16 weights, float
    biases and norm scales), placed by wan_vae_param_info."""

    def __init__(self, sh: N.WanVaeShape, params: dict, device="cuda"):
        import numpy as np
        from .synth import bf16_bits, round_bf16
        torch = _torch()
        lib = N.load()
        st = ctypes.c_int(0)
        nw = lib.wan_vae_blob_elems(ctypes.byref(sh), 0, ctypes.byref(st))
        N.check(st.value)
        nf = lib.wan_vae_blob_elems(ctypes.byref(sh), 1, ctypes.byref(st))
        N.check(st.value)
        wb = np.zeros(max(nw, 64), np.uint16)
        fb = np.zeros(max(nf, 64), np.float32)
        for name, kind, dims, off, cnt in vae_param_table(sh):
            a = np.asarray(params[name], np.float32).reshape(-1)
            if a.size != cnt:
                raise ValueError(f"{name}: {a.size} values, the library expects {cnt}")
            if kind == 0:
                # nearest bf16 value, ties to even (the conversion the DiT weights get)
                wb[off:off + cnt] = bf16_bits(round_bf16(a))
            else:
                fb[off:off + cnt] = a
        self.weights = torch.from_numpy(wb.view(np.int16)).to(device)
        self.fparams = torch.from_numpy(fb).to(device)


def vae_workspace(sh: N.WanVaeShape, device="cuda"):
    torch = _torch()
    st = ctypes.c_int(0)
    n = N.load().wan_vae_workspace_bytes(ctypes.byref(sh), ctypes.byref(st))
    N.check(st.value)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def vae_cache(sh: N.WanVaeShape, device="cuda"):
    torch = _torch()
    st = ctypes.c_int(0)
    n = N.load().wan_vae_cache_bytes(ctypes.byref(sh), ctypes.byref(st))
    N.check(st.value)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def vae_decode(sh: N.WanVaeShape, dev: VaeDevice, z, t0: int, n: int, cache, video, ws, stream=None):
    """wan_vae_decode: latent frames [t0, t0 + n) of z (z_ch, n, H, W) float32 -> video
    (3, n_out, 8H, 8W) float32."""
    lib = N.load()
    N.check(lib.wan_vae_decode(ctypes.byref(sh), _ptr(dev.weights), _ptr(dev.fparams), _ptr(z), int(t0), int(n),
                               _ptr(cache), cache.numel(), _ptr(video), _ptr(ws), ws.numel(), _stream(stream)))


# ----------------------------------------------------------------------------- streaming queue
def stream_workspace(cfg, group: int, device="cuda"):
    torch = _torch()
    st = ctypes.c_int(0)
    sh = shape_of(cfg)
    n = N.load().wan_stream_workspace_bytes(ctypes.byref(sh), int(group), ctypes.byref(st))
    N.check(st.value)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def stream_tick(cfg, model: DeviceModel, window, ctx, taus, dts, group: int, noise_in, frames_out, ws, stream=None):
    """wan_stream_tick: one tick of the streaming denoise queue (window updated in place)."""
    lib = N.load()
    sh = shape_of(cfg)
    k = len(taus)
    ta = (ctypes.c_float * k)(*[float(t) for t in taus])
    da = (ctypes.c_float * k)(*[float(t) for t in dts])
    N.check(lib.wan_stream_tick(ctypes.byref(sh), ctypes.byref(model.struct), _ptr(window), _ptr(ctx),
                                ctypes.cast(ta, ctypes.c_void_p), ctypes.cast(da, ctypes.c_void_p), int(group),
                                _ptr(noise_in), _ptr(frames_out), _ptr(ws), ws.numel(), _stream(stream)))
