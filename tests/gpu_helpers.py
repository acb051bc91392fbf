"""Shared helpers of the GPU parity tests: run the HIP library through its C ABI
and the float64 oracle on the same seeded inputs, and compare."""
from __future__ import annotations

import numpy as np

from oracle import wan_oracle as O
from video_diffusion_transformer_forward_amd import synth as S

# normwise relative error bars: bf16 operands with float32 accumulation, and float32 throughout
TOL = {"bf16": 1e-2, "fp32": 1e-5}


def rel_err(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(got - ref) / np.linalg.norm(ref))


def inc_err(got_out, ref_out, x_in) -> float:
    """Relative error of the increment x_out - x_in.

    The library stores x_out (and z) in float32, so the reference increment is
    taken from the exact result rounded to float32: what an exact computation
    would return through the same output format.  Without that rounding the
    increment of a sublayer that changes x by ~1e-2 relative carries ~1e-5 of
    pure storage error."""
    ref32 = np.asarray(ref_out, np.float32).astype(np.float64)
    x_in = np.asarray(x_in, np.float64)
    return rel_err(np.asarray(got_out, np.float64) - x_in, ref32 - x_in)


def announce(msg: str):
    print(f"[gpu-case] {msg}", flush=True)


def W():
    import video_diffusion_transformer_forward_amd as lib
    return lib


def native():
    from video_diffusion_transformer_forward_amd import _native
    return _native


def torch():
    import torch as t
    return t


def to_dev(a, dtype=None):
    t = torch()
    x = t.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        x = x.to(dtype)
    return x.cuda()


def ctx_dev(cfg, ctx):
    return to_dev(ctx, W().elem_dtype(cfg))


def gpu_block(cfg, w, x, mod, ctx, mod_stride=None):
    """Run wan_dit_block_forward; returns the updated residual stream (numpy float32)."""
    lib = W()
    t = torch()
    blk = lib.DeviceBlock(cfg, w)
    xd = to_dev(x)
    md = to_dev(mod)
    cd = ctx_dev(cfg, ctx)
    ws = lib.workspace(cfg, native().ENTRY_BLOCK)
    lib.dit_block_forward(cfg, blk, xd, md, cd, ws, mod_batch_stride=mod_stride)
    t.cuda.synchronize()
    return xd.cpu().numpy()


def oracle_block(cfg, w, x, mod, ctx, rows=None):
    return O.dit_block(x, mod, ctx, w, cfg.heads, cfg.grid, cfg.img_len, rows=rows, qk8=cfg.qk8, fp8=cfg.fp8)


def block_case(cfg, zero_co=False):
    w = S.block_weights(cfg, 0, zero_co=zero_co)
    x = S.block_inputs(cfg)
    mod = S.modulation(cfg)
    ctx = S.context(cfg, "cond")
    return w, x, mod, ctx


def device_model(cfg, mw, blocks_w):
    lib = W()
    blocks = [lib.DeviceBlock(cfg, b) for b in blocks_w]
    return lib.DeviceModel(cfg, mw, blocks)


def gpu_step(cfg, mw, blocks_w, z, cond, ctx_c, ctx_n, tau, dt, g, model=None):
    lib = W()
    t = torch()
    model = model or device_model(cfg, mw, blocks_w)
    zd = to_dev(z)
    cd = to_dev(cond) if cond is not None else None
    ws = lib.workspace(cfg, native().ENTRY_STEP)
    lib.denoise_step(cfg, model, zd, cd, ctx_dev(cfg, ctx_c), ctx_dev(cfg, ctx_n), tau, dt, g, ws)
    t.cuda.synchronize()
    return zd.cpu().numpy()


def token_pixels(cfg, rows):
    """Index arrays (c, f, y, x) of the latent pixels covered by each token in rows: (n, 16, 4)."""
    F, Hh, Ww = cfg.grid
    out = []
    for l in rows:
        f, rem = divmod(int(l), Hh * Ww)
        i, j = divmod(rem, Ww)
        out.append((f, i, j))
    return out


def sample_rows(L, n, seed=0):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(L, size=min(n, L), replace=False).tolist())
    rows.update([0, L - 1])
    return sorted(rows)


def self_attention_only(cfg, w, mod):
    """Block weights and modulation under which the block adds only its self-attention sublayer,
    with b_v = 0 (the output is pure weighting): cross-attention output projection and FFN gate zero."""
    w = dict(w)
    w["qkv_b"] = w["qkv_b"].copy()
    w["qkv_b"][2 * cfg.dim:] = 0.0
    w["co_w"] = np.zeros_like(w["co_w"])
    w["co_b"] = np.zeros_like(w["co_b"])
    m = mod.copy()
    m[:, 5] = 0.0
    return w, m
