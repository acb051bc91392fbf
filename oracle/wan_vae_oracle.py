"""Plain float64 CPU oracle for the Wan-VAE decoder (latent -> RGB video).

TEST INFRASTRUCTURE ONLY.  Only the test suite and the benchmark's CPU
baseline may import this module; the product path never calls it and shares
no code with it.

Source: [P2] hyper.ai summary of the Wan technical report, section "方法"
(method), the Wan-VAE paragraphs: a 3D causal VAE compressing time x height x
width by 4 x 8 x 8 ([1+T, H, W, 3] <-> [1+T/4, H/8, W/8, C]); 3D causal
convolutions; the first frame compressed only in space, the others in space and
time; every GroupNorm replaced by RMSNorm so that a feature cache can carry the
frame-level features of earlier chunks, which lets arbitrarily long videos be
decoded chunk by chunk.

The pages give no layer list.  Readings taken (listed with the design notes):
stage widths (4b, 4b, 4b, 2b, b); a 3x3x3 causal input convolution; two
residual blocks in the middle and per stage, each RMSNorm -> SiLU -> 3x3x3
causal conv, twice, plus the input (through a 1x1x1 convolution when the width
changes); stages 0 and 1 double time (a 3x1x1 causal convolution to 2C whose
halves become two consecutive frames; the video's first frame passes through
undoubled) then space; stage 2 doubles space only; spatial doubling is nearest
neighbour followed by a 1x3x3 convolution; the head is RMSNorm -> SiLU ->
3x3x3 causal convolution to RGB.  Causal convolutions pad time with the two
previous frames of their input (zeros before the first frame) and space with
zeros.  RMSNorm: x / sqrt(mean_c x^2 + 1e-6) * gamma over the channels.

Tensors are channels-last (T, H, W, C) float64 inside; the interface takes the
latent as (z_ch, T, H, W) and returns the video as (3, T_out, H_out, W_out).
"""
from __future__ import annotations

import numpy as np

RMS_EPS = 1e-6


def f64(a):
    return np.asarray(a, dtype=np.float64)


def causal_conv3d(x, w, b, cache=None):
    """Causal 3D convolution, channels-last.

    x (T, H, W, Cin); w (Cout, kt, kh, kw, Cin); b (Cout,).  The kt-1 frames
    before x are `cache` (the previous frames of this layer's input, a feature
    cache) or zeros; space is zero-padded by (k-1)/2 on each side.  Output
    frame t sees input frames t-kt+1 .. t.  Returns (out (T, H, W, Cout), the
    kt-1 last frames of the padded input: the cache for the next chunk)."""
    x, w = f64(x), f64(w)
    T, H, W, C = x.shape
    cout, kt, kh, kw, cin = w.shape
    assert cin == C
    prev = np.zeros((kt - 1, H, W, C)) if cache is None else f64(cache)
    xp = np.concatenate([prev, x], axis=0)
    ph, pw = (kh - 1) // 2, (kw - 1) // 2
    xp = np.pad(xp, ((0, 0), (ph, ph), (pw, pw), (0, 0)))
    out = np.zeros((T, H, W, cout))
    for dt in range(kt):
        for dh in range(kh):
            for dw in range(kw):
                out += xp[dt:dt + T, dh:dh + H, dw:dw + W, :] @ w[:, dt, dh, dw, :].T
    out += f64(b)
    new_cache = xp[T:, ph:ph + H, pw:pw + W, :] if kt > 1 else None
    return out, new_cache


def rms_norm(x, g):
    x = f64(x)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + RMS_EPS) * f64(g)


def silu(x):
    return x / (1.0 + np.exp(-x))


def upsample_space(x):
    """Nearest-neighbour doubling of height and width."""
    return np.repeat(np.repeat(x, 2, axis=1), 2, axis=2)


class VaeDecoder:
    """The decoder with its feature cache.  `decode(z_chunk)` takes the next
    latent frames (z_ch, n, H, W) and returns their video frames
    (3, n_out, 8H, 8W); the first call's first latent frame yields one video
    frame, every other latent frame four."""

    def __init__(self, params, dims, n_res=2):
        self.p = {k: f64(v) for k, v in params.items()}
        self.d = dims
        self.n_res = n_res
        self.cache = {}
        self.first = True

    def _conv(self, name, x):
        out, c = causal_conv3d(x, self.p[name], self.p[name + ".bias"], self.cache.get(name))
        if c is not None:
            self.cache[name] = c
        return out

    def _res(self, prefix, x):
        h = self._conv(prefix + ".conv_a", silu(rms_norm(x, self.p[prefix + ".norm_a"])))
        h = self._conv(prefix + ".conv_b", silu(rms_norm(h, self.p[prefix + ".norm_b"])))
        skip = self._conv(prefix + ".skip", x) if prefix + ".skip" in self.p else x
        return h + skip

    def _time_up(self, name, x):
        """3x1x1 causal conv to 2C; the halves of frame t become frames 2t, 2t+1.
        The video's first frame is kept as it is (no doubling)."""
        y = self._conv(name, x)
        T, H, W, C2 = y.shape
        C = C2 // 2
        doubled = y.reshape(T, H, W, 2, C).transpose(0, 3, 1, 2, 4).reshape(2 * T, H, W, C)
        if self.first:
            return np.concatenate([x[:1], doubled[2:]], axis=0)
        return doubled

    def decode(self, z):
        x = f64(z).transpose(1, 2, 3, 0)            # (n, H, W, z_ch)
        x = self._conv("conv_in", x)
        for i in range(2):
            x = self._res(f"mid.{i}", x)
        for s in range(4):
            for j in range(self.n_res):
                x = self._res(f"up.{s}.res.{j}", x)
            if s < 2:
                x = self._time_up(f"up.{s}.time_conv", x)
            if s < 3:
                x = self._conv(f"up.{s}.space_conv", upsample_space(x))
        x = self._conv("head.conv", silu(rms_norm(x, self.p["head.norm"])))
        self.first = False
        return x.transpose(3, 0, 1, 2)               # (3, n_out, H_out, W_out)


def vae_decode(z, params, dims, n_res=2, chunks=None):
    """Decode the latent (z_ch, T, H, W).  chunks: latent frame counts of the
    successive calls (default: all frames at once)."""
    dec = VaeDecoder(params, dims, n_res)
    T = np.asarray(z).shape[1]
    chunks = chunks or [T]
    assert sum(chunks) == T
    outs, t = [], 0
    for n in chunks:
        outs.append(dec.decode(np.asarray(z)[:, t:t + n]))
        t += n
    return np.concatenate(outs, axis=1)
