"""Seeded synthetic inputs for the Wan-VAE decoder: configurations, the list of
parameter tensors (names and shapes) and their random draws.

Like `synth`, this module holds shapes, seeds and random draws only; the
decoder's arithmetic lives in the library and, separately, in the oracle.

Parameter list (execution order).  Convolution weights are [C_out][k_t][k_h][k_w][C_in]
(taps outer, input channels inner), with a float32 bias of C_out; RMSNorm scales
are float32 vectors of C.  Names:
  conv_in                              z_ch -> d0, 3x3x3 causal
  mid.{0,1}.*                          residual blocks d0 -> d0
  up.{i}.res.{j}.*                     residual blocks of stage i (the first changes the width)
  up.{i}.time_conv                     (stages 0, 1) 3x1x1 causal, C -> 2C (temporal x2)
  up.{i}.space_conv                    (stages 0, 1, 2) 1x3x3, C -> C after nearest x2 in space
  head.norm, head.conv                 RMSNorm, then 3x3x3 causal d4 -> 3
A residual block has norm_a, conv_a (3x3x3), norm_b, conv_b (3x3x3) and, when
the width changes, skip (1x1x1).

Seeds: numpy PCG64 with seed = 1000 * seed_base + tensor id (0 latent,
10 + layer index parameters).  Convolution weights are N(0, 1/fan_in) rounded
once to bfloat16, biases N(0, 0.02^2), norm scales 1 + N(0, 0.1^2); the latent
is N(0, 1) float32.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

from .synth import round_bf16


@dataclass(frozen=True)
class VaeConfig:
    name: str
    seed_base: int
    frames: int = 3      # latent frames T
    height: int = 4      # latent height
    width: int = 6       # latent width
    z_ch: int = 16
    base: int = 32       # stage widths (4b, 4b, 4b, 2b, b)
    n_res: int = 2       # residual blocks per stage

    @property
    def dims(self):
        b = self.base
        return (4 * b, 4 * b, 4 * b, 2 * b, b)

    @property
    def out_frames(self) -> int:
        return 1 + 4 * (self.frames - 1)

    @property
    def out_height(self) -> int:
        return 8 * self.height

    @property
    def out_width(self) -> int:
        return 8 * self.width

    def with_(self, **kw) -> "VaeConfig":
        return replace(self, **kw)


VAE_CONFIGS = {
    # 81 frames at 480x832 from the 21 x 60 x 104 latent
    "vae_480p": VaeConfig("vae_480p", 31, frames=21, height=60, width=104, base=96),
    # small shapes for parity runs
    "vae_tiny": VaeConfig("vae_tiny", 32, frames=3, height=4, width=6, base=32),
    "vae_small": VaeConfig("vae_small", 33, frames=5, height=6, width=10, base=32),
    "vae_w96": VaeConfig("vae_w96", 34, frames=4, height=5, width=7, base=96),
}


def get_vae_config(name: str) -> VaeConfig:
    return VAE_CONFIGS[name]


def _res_shapes(prefix, cin, cout):
    out = [(prefix + ".norm_a", (cin,)), (prefix + ".conv_a", (cout, 3, 3, 3, cin)),
           (prefix + ".norm_b", (cout,)), (prefix + ".conv_b", (cout, 3, 3, 3, cout))]
    if cin != cout:
        out.append((prefix + ".skip", (cout, 1, 1, 1, cin)))
    return out


def vae_param_shapes(cfg: VaeConfig):
    """[(name, shape)] of every parameter tensor in execution order (bias of a
    convolution `name` is `name + '.bias'`, shape (C_out,))."""
    d = cfg.dims
    shapes = [("conv_in", (d[0], 3, 3, 3, cfg.z_ch))]
    for i in range(2):
        shapes += _res_shapes(f"mid.{i}", d[0], d[0])
    for s in range(4):
        cin, cout = d[s], d[s + 1]
        for j in range(cfg.n_res):
            shapes += _res_shapes(f"up.{s}.res.{j}", cin if j == 0 else cout, cout)
        if s < 2:
            shapes.append((f"up.{s}.time_conv", (2 * cout, 3, 1, 1, cout)))
        if s < 3:
            shapes.append((f"up.{s}.space_conv", (cout, 1, 3, 3, cout)))
    shapes += [("head.norm", (d[4],)), ("head.conv", (3, 3, 3, 3, d[4]))]
    return shapes


def _rng(cfg: VaeConfig, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(1000 * cfg.seed_base + tensor_id))


def vae_params(cfg: VaeConfig) -> dict:
    """Every parameter tensor (float32 arrays; convolution weights bf16-exact)."""
    p = {}
    for idx, (name, shape) in enumerate(vae_param_shapes(cfg)):
        rng = _rng(cfg, 10 + idx)
        if len(shape) == 1:
            p[name] = (1.0 + 0.1 * rng.standard_normal(shape, dtype=np.float32)).astype(np.float32)
        else:
            fan_in = int(np.prod(shape[1:]))
            w = rng.standard_normal(shape, dtype=np.float32) * np.float32(1.0 / np.sqrt(fan_in))
            p[name] = round_bf16(w)
            p[name + ".bias"] = (0.02 * rng.standard_normal(shape[0], dtype=np.float32)).astype(np.float32)
    return p


def vae_latent(cfg: VaeConfig) -> np.ndarray:
    """Latent (z_ch, T, H, W) float32, N(0, 1)."""
    return _rng(cfg, 0).standard_normal((cfg.z_ch, cfg.frames, cfg.height, cfg.width), dtype=np.float32)
