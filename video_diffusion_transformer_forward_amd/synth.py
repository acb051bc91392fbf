"""Seeded synthetic inputs for the Wan2.1 DiT block and denoise step.

This module holds shapes, seeds and random draws only: none of the method's
arithmetic lives here.  Both sides of every parity check (the HIP library and
the CPU oracle) take their inputs from these generators, so both see the same
values.  Matrices are drawn in float32 and, in bf16 mode, rounded once to the
nearest bfloat16 (ties to even); the rounded values are returned as float32
arrays, which hold them exactly.  Biases and every activation tensor that the
library takes in float32 (latents, condition channels, modulation) are never
rounded.

Seeds: numpy PCG64 with seed = 1000 * config.seed_base + tensor id
(0 latent z, 1 cond text context, 2 null text context, 3 condition latent z_c,
4 modulation, 10 model-level weights, 100 + b block b).
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

WEIGHT_STD = 0.02


@dataclass(frozen=True)
class WanConfig:
    name: str
    seed_base: int
    batch: int = 1
    in_ch: int = 16          # 16 text-to-video, 36 image-to-video (16 + 4 mask + 16 cond)
    out_ch: int = 16
    frames: int = 2          # latent frames F'
    height: int = 16         # latent height H'
    width: int = 16          # latent width W'
    dim: int = 256
    heads: int = 4
    ffn_dim: int = 1024
    txt_len: int = 32
    img_len: int = 0
    n_blocks: int = 1
    mode: str = "fp32"       # "fp32" or "bf16"
    qk8: bool = False        # bf16 only: self-attention scores from 8-bit q and k
    fp8: bool = False        # bf16 only: 8-bit projections (q/k/v, cross q, FFN) plus qk8
    timestep: float = 500.0
    dt: float = 0.05
    guide_scale: float = 5.0
    mod_std: float = 0.1     # std of the directly drawn modulation (block-level tests)
    qk_std: float = WEIGHT_STD  # std of the q/k rows of the fused qkv weight

    @property
    def head_dim(self) -> int:
        return self.dim // self.heads

    @property
    def grid(self):
        return (self.frames, self.height // 2, self.width // 2)

    @property
    def seq_len(self) -> int:
        f, h, w = self.grid
        return f * h * w

    @property
    def ctx_len(self) -> int:
        return self.img_len + self.txt_len

    @property
    def patch_k(self) -> int:
        return self.in_ch * 4

    def with_(self, **kw) -> "WanConfig":
        return replace(self, **kw)


# The five workloads: a toy fp32 block, the 1.3B block and step at 480p x 81
# frames, a 14B block at 720p and a 14B image-to-video block at 480p.
CONFIGS = {
    "toy": WanConfig("toy", 1, frames=2, height=16, width=16, dim=256, heads=4,
                     ffn_dim=1024, txt_len=32, mode="fp32"),
    "wan13b_block": WanConfig("wan13b_block", 2, frames=21, height=60, width=104,
                              dim=1536, heads=12, ffn_dim=8960, txt_len=512, mode="bf16"),
    "wan13b_step": WanConfig("wan13b_step", 3, frames=21, height=60, width=104,
                             dim=1536, heads=12, ffn_dim=8960, txt_len=512,
                             n_blocks=30, mode="bf16"),
    "wan14b_720p_block": WanConfig("wan14b_720p_block", 4, frames=21, height=90, width=160,
                                   dim=5120, heads=40, ffn_dim=13824, txt_len=512, mode="bf16"),
    "wan14b_i2v_block": WanConfig("wan14b_i2v_block", 5, in_ch=36, frames=21, height=60,
                                  width=104, dim=5120, heads=40, ffn_dim=13824,
                                  txt_len=512, img_len=257, mode="bf16"),
}

# Small shapes for parity runs that the oracle finishes in seconds.  They span
# several tiles and end in ragged tails (L = 351 = 2*128 + 95; 257 image tokens).
TEST_CONFIGS = {
    "mid_bf16": WanConfig("mid_bf16", 11, frames=3, height=18, width=26, dim=256, heads=2,
                          ffn_dim=768, txt_len=40, mode="bf16"),
    "mid_fp32": WanConfig("mid_fp32", 12, frames=3, height=18, width=26, dim=256, heads=2,
                          ffn_dim=768, txt_len=40, mode="fp32"),
    "mid_i2v_bf16": WanConfig("mid_i2v_bf16", 13, in_ch=36, frames=3, height=14, width=22,
                              dim=512, heads=4, ffn_dim=1024, txt_len=64, img_len=257,
                              mode="bf16"),
    "mid_b2_bf16": WanConfig("mid_b2_bf16", 14, batch=2, frames=2, height=20, width=22,
                             dim=256, heads=2, ffn_dim=512, txt_len=24, mode="bf16"),
    "toy_step": WanConfig("toy_step", 15, frames=2, height=16, width=16, dim=256, heads=4,
                          ffn_dim=1024, txt_len=32, n_blocks=3, mode="fp32"),
    "mid_step_bf16": WanConfig("mid_step_bf16", 16, frames=3, height=12, width=20, dim=256,
                               heads=2, ffn_dim=512, txt_len=24, n_blocks=4, mode="bf16"),
    "toy_i2v_fp32": WanConfig("toy_i2v_fp32", 17, in_ch=36, frames=2, height=10, width=12,
                              dim=256, heads=4, ffn_dim=512, txt_len=16, img_len=9,
                              mode="fp32"),
}


def get_config(name: str) -> WanConfig:
    if name in CONFIGS:
        return CONFIGS[name]
    return TEST_CONFIGS[name]


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    # 32-bit arithmetic: finite values never carry past bit 31 (only NaN payloads could)
    r = (u >> np.uint32(16)) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r &= np.uint32(0xFFFF0000)
    return r.view(np.float32).reshape(a.shape)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16-exact."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def _rng(cfg: WanConfig, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(1000 * cfg.seed_base + tensor_id))


def _normal(rng, shape, std=1.0):
    return (rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def _mat(cfg, rng, shape, std=WEIGHT_STD):
    w = _normal(rng, shape, std)
    return round_bf16(w) if cfg.mode == "bf16" else w


def block_weights(cfg: WanConfig, b: int, *, zero_co: bool = False) -> dict:
    """Weights of block b: PyTorch Linear layout [out][in]; biases float32."""
    rng = _rng(cfg, 100 + b)
    d, f = cfg.dim, cfg.ffn_dim
    w = {}
    qkv = _normal(rng, (3 * d, d), WEIGHT_STD)
    if cfg.qk_std != WEIGHT_STD:
        qkv[: 2 * d] *= np.float32(cfg.qk_std / WEIGHT_STD)
    w["qkv_w"] = round_bf16(qkv) if cfg.mode == "bf16" else qkv
    w["qkv_b"] = _normal(rng, (3 * d,), WEIGHT_STD)
    w["o_w"] = _mat(cfg, rng, (d, d))
    w["o_b"] = _normal(rng, (d,), WEIGHT_STD)
    w["cq_w"] = _mat(cfg, rng, (d, d))
    w["cq_b"] = _normal(rng, (d,), WEIGHT_STD)
    w["ckv_w"] = _mat(cfg, rng, (2 * d, d))
    w["ckv_b"] = _normal(rng, (2 * d,), WEIGHT_STD)
    if cfg.img_len > 0:
        w["ikv_w"] = _mat(cfg, rng, (2 * d, d))
        w["ikv_b"] = _normal(rng, (2 * d,), WEIGHT_STD)
    w["co_w"] = _mat(cfg, rng, (d, d))
    w["co_b"] = _normal(rng, (d,), WEIGHT_STD)
    w["ff1_w"] = _mat(cfg, rng, (f, d))
    w["ff1_b"] = _normal(rng, (f,), WEIGHT_STD)
    w["ff2_w"] = _mat(cfg, rng, (d, f))
    w["ff2_b"] = _normal(rng, (d,), WEIGHT_STD)
    if zero_co:
        w["co_w"] = np.zeros_like(w["co_w"])
        w["co_b"] = np.zeros_like(w["co_b"])
    return w


def model_weights(cfg: WanConfig) -> dict:
    """Patch embedding, time MLP and head weights (the per-block weights are separate)."""
    rng = _rng(cfg, 10)
    d = cfg.dim
    w = {}
    w["pe_w"] = _mat(cfg, rng, (d, cfg.patch_k))
    w["pe_b"] = _normal(rng, (d,), WEIGHT_STD)
    w["t1_w"] = _mat(cfg, rng, (d, 256))
    w["t1_b"] = _normal(rng, (d,), WEIGHT_STD)
    w["t2_w"] = _mat(cfg, rng, (d, d))
    w["t2_b"] = _normal(rng, (d,), WEIGHT_STD)
    w["m_w"] = _mat(cfg, rng, (6 * d, d))
    w["m_b"] = _normal(rng, (6 * d,), WEIGHT_STD)
    w["hd_w"] = _mat(cfg, rng, (cfg.out_ch * 4, d))
    w["hd_b"] = _normal(rng, (cfg.out_ch * 4,), WEIGHT_STD)
    return w


def latent(cfg: WanConfig) -> np.ndarray:
    """Noisy latent z: (B, 16, F', H', W') float32, N(0, 1)."""
    return _normal(_rng(cfg, 0), (cfg.batch, cfg.out_ch, cfg.frames, cfg.height, cfg.width))


def condition(cfg: WanConfig):
    """Image-to-video condition channels (B, 20, F', H', W') = [mask(4); z_c(16)], or None.

    The mask is 1 on latent frame 0 (the given image) and 0 on every other frame;
    z_c is N(0, 1)."""
    if cfg.in_ch == 16:
        return None
    extra = cfg.in_ch - 16
    n_mask = extra - 16
    shp = (cfg.batch, 16, cfg.frames, cfg.height, cfg.width)
    zc = _normal(_rng(cfg, 3), shp)
    mask = np.zeros((cfg.batch, n_mask, cfg.frames, cfg.height, cfg.width), np.float32)
    mask[:, :, 0] = 1.0
    return np.concatenate([mask, zc], axis=1)


def context(cfg: WanConfig, which: str = "cond") -> np.ndarray:
    """Context tokens (B, L_img + L_txt, D): image tokens first, N(0, 1)."""
    tid = 1 if which == "cond" else 2
    c = _normal(_rng(cfg, tid), (cfg.batch, cfg.ctx_len, cfg.dim))
    return round_bf16(c) if cfg.mode == "bf16" else c


def modulation(cfg: WanConfig) -> np.ndarray:
    """Directly drawn modulation (B, 6, D) float32 for block-level runs.

    Order: shift1, scale1, gate1 (self-attention), shift2, scale2, gate2 (FFN)."""
    return _normal(_rng(cfg, 4), (cfg.batch, 6, cfg.dim), cfg.mod_std)


def block_inputs(cfg: WanConfig) -> dict:
    """Residual stream x (B, L, D) float32 for block-level runs, N(0, 1)."""
    rng = _rng(cfg, 5)
    return _normal(rng, (cfg.batch, cfg.seq_len, cfg.dim))
