"""CPU pins of the Wan-VAE decoder oracle: library routines, brute force, causality,
chunked decoding with the feature cache, and closed forms."""
import numpy as np
import pytest
import torch

from oracle import wan_vae_oracle as V
from video_diffusion_transformer_forward_amd import vae_synth as VS

rng = np.random.default_rng(7)


def _torch_conv(x, w, b):
    """Causal conv3d through torch (float64): time padded in front with kt-1 zeros."""
    cout, kt, kh, kw, cin = w.shape
    xt = torch.from_numpy(np.ascontiguousarray(x.transpose(3, 0, 1, 2)))[None]      # (1, C, T, H, W)
    xt = torch.nn.functional.pad(xt, ((kw - 1) // 2, (kw - 1) // 2, (kh - 1) // 2, (kh - 1) // 2, kt - 1, 0))
    wt = torch.from_numpy(np.ascontiguousarray(w.transpose(0, 4, 1, 2, 3)))
    y = torch.nn.functional.conv3d(xt, wt, torch.from_numpy(b))
    return y[0].numpy().transpose(1, 2, 3, 0)


@pytest.mark.parametrize("k", [(3, 3, 3), (3, 1, 1), (1, 3, 3), (1, 1, 1)])
def test_causal_conv_matches_torch(k):
    x = rng.standard_normal((4, 5, 6, 7))
    w = rng.standard_normal((3,) + k + (7,))
    b = rng.standard_normal(3)
    out, _ = V.causal_conv3d(x, w, b)
    np.testing.assert_allclose(out, _torch_conv(x, w, b), rtol=1e-12, atol=1e-12)


def test_causal_conv_brute_force():
    x = rng.standard_normal((3, 3, 4, 2))
    w = rng.standard_normal((2, 3, 3, 3, 2))
    b = rng.standard_normal(2)
    out, _ = V.causal_conv3d(x, w, b)
    T, H, W, C = x.shape
    for t in range(T):
        for h in range(H):
            for ww in range(W):
                for o in range(2):
                    s = b[o]
                    for dt in range(3):
                        for dh in range(3):
                            for dw in range(3):
                                ti, hi, wi = t - 2 + dt, h - 1 + dh, ww - 1 + dw
                                if ti < 0 or not (0 <= hi < H) or not (0 <= wi < W):
                                    continue
                                s += np.dot(w[o, dt, dh, dw], x[ti, hi, wi])
                    assert abs(out[t, h, ww, o] - s) < 1e-12


def test_conv_cache_is_the_previous_frames():
    """Two calls with the returned cache equal one call over the concatenated frames."""
    x = rng.standard_normal((5, 4, 4, 3))
    w = rng.standard_normal((2, 3, 3, 3, 3))
    b = rng.standard_normal(2)
    whole, _ = V.causal_conv3d(x, w, b)
    a, c = V.causal_conv3d(x[:2], w, b)
    bb, _ = V.causal_conv3d(x[2:], w, b, c)
    np.testing.assert_allclose(np.concatenate([a, bb]), whole, rtol=1e-12, atol=1e-12)
    a, c = V.causal_conv3d(x[:1], w, b)          # a one-frame chunk: the cache keeps a zero frame
    np.testing.assert_array_equal(c[0], 0.0)


def test_rms_norm_closed_forms():
    x = rng.standard_normal((3, 8))
    g = rng.standard_normal(8)
    np.testing.assert_allclose(V.rms_norm(5.0 * x, g), V.rms_norm(x, g), rtol=2e-6)   # up to the eps term
    c = np.full((1, 8), 3.0)
    np.testing.assert_allclose(V.rms_norm(c, g), g[None] * 3.0 / np.sqrt(9.0 + V.RMS_EPS), rtol=1e-14)
    r = V.rms_norm(x, np.ones(8))
    np.testing.assert_allclose(np.mean(r * r, axis=-1), np.mean(x * x, -1) / (np.mean(x * x, -1) + V.RMS_EPS))


def test_upsample_space_nearest():
    x = rng.standard_normal((2, 3, 4, 5))
    u = V.upsample_space(x)
    assert u.shape == (2, 6, 8, 5)
    for a in range(2):
        for b in range(2):
            np.testing.assert_array_equal(u[:, a::2, b::2], x)


def test_time_doubling_copies_with_identity_taps_and_keeps_the_first_frame():
    C = 3
    dec = V.VaeDecoder({}, (C,) * 5)
    w = np.zeros((2 * C, 3, 1, 1, C))
    w[:C, 2, 0, 0] = np.eye(C)          # first half: the current frame
    w[C:, 2, 0, 0] = 2 * np.eye(C)      # second half: twice the current frame
    dec.p["tc"], dec.p["tc.bias"] = w, np.zeros(2 * C)
    x = rng.standard_normal((3, 2, 2, C))
    y = dec._time_up("tc", x)
    assert y.shape[0] == 5
    np.testing.assert_array_equal(y[0], x[0])
    for t in (1, 2):
        np.testing.assert_array_equal(y[2 * t - 1], x[t])
        np.testing.assert_array_equal(y[2 * t], 2 * x[t])
    dec.first = False
    assert dec._time_up("tc", x).shape[0] == 6


def test_residual_block_identity_with_zero_second_conv():
    cfg = VS.get_vae_config("vae_tiny")
    p = VS.vae_params(cfg)
    p["mid.0.conv_b"] = np.zeros_like(p["mid.0.conv_b"])
    p["mid.0.conv_b.bias"] = np.zeros_like(p["mid.0.conv_b.bias"])
    dec = V.VaeDecoder(p, cfg.dims, cfg.n_res)
    x = rng.standard_normal((2, 3, 3, cfg.dims[0]))
    np.testing.assert_array_equal(dec._res("mid.0", x), x)


def test_decoder_shapes_chunking_and_causality():
    cfg = VS.get_vae_config("vae_tiny")
    p = VS.vae_params(cfg)
    z = VS.vae_latent(cfg)
    whole = V.vae_decode(z, p, cfg.dims, cfg.n_res)
    assert whole.shape == (3, cfg.out_frames, cfg.out_height, cfg.out_width)
    assert np.all(np.isfinite(whole))
    for chunks in ([1, 2], [1, 1, 1], [2, 1]):
        np.testing.assert_allclose(V.vae_decode(z, p, cfg.dims, cfg.n_res, chunks), whole, rtol=1e-10, atol=1e-10)
    # latent frame 2 only reaches video frames 1 + 4 * 1 = 5 onward
    z2 = z.copy()
    z2[:, 2] += 1.0
    moved = V.vae_decode(z2, p, cfg.dims, cfg.n_res)
    np.testing.assert_array_equal(moved[:, :5], whole[:, :5])
    assert np.max(np.abs(moved[:, 5:] - whole[:, 5:])) > 1e-3


def test_param_list_covers_the_decoder():
    """Every parameter drawn for a configuration is used by the decoder, and the widths
    follow (4b, 4b, 4b, 2b, b)."""
    cfg = VS.get_vae_config("vae_tiny")
    p = VS.vae_params(cfg)
    used = set()

    class Spy(dict):
        def __getitem__(self, k):
            used.add(k)
            return dict.__getitem__(self, k)

    dec = V.VaeDecoder(p, cfg.dims, cfg.n_res)
    dec.p = Spy(dec.p)
    dec.decode(VS.vae_latent(cfg))
    assert used == set(p)
    assert cfg.dims == (128, 128, 128, 64, 32)


def test_silu_matches_torch_and_hand_values():
    """The decoder's SiLU(x) = x * sigmoid(x): torch float64 over both signs, hand values."""
    import math
    x = np.concatenate([np.linspace(-40.0, 40.0, 801), rng.standard_normal(300) * 4, [-300.0, 300.0]])
    np.testing.assert_allclose(V.silu(x), torch.nn.functional.silu(torch.from_numpy(x)).numpy(), rtol=1e-14,
                               atol=1e-300)
    assert V.silu(np.float64(1.0)) == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), rel=1e-15)
    assert V.silu(np.float64(-1.0)) == pytest.approx(-1.0 / (1.0 + math.e), rel=1e-15)
    assert V.silu(np.float64(0.0)) == 0.0
    np.testing.assert_allclose(V.silu(x) - V.silu(-x), x, rtol=1e-12, atol=1e-12)


def test_decoding_a_latent_crop_gives_the_whole_decode_inside_the_reach():
    """The decoder's spatial reach is 13.5 latent pixels (nine 3x3 convolutions at the latent
    resolution, five at x2, five at x4, six at x8): decoding a crop of the latent reproduces the
    whole decode exactly wherever the output lies 14 or more latent pixels inside the crop, and
    not where it lies closer to the crop's edge (zero padding reaches it there)."""
    cfg = VS.get_vae_config("vae_tiny").with_(frames=2, height=34, width=36)
    p = VS.vae_params(cfg)
    z = VS.vae_latent(cfg)
    whole = V.vae_decode(z, p, cfg.dims, cfg.n_res)
    r0, c0, n, mg = 15, 17, 3, 14
    zc = z[:, :, r0 - mg:r0 + n + mg, c0 - mg:c0 + n + mg]
    crop = V.vae_decode(zc, p, cfg.dims, cfg.n_res)
    inner = crop[:, :, 8 * mg:8 * (mg + n), 8 * mg:8 * (mg + n)]
    np.testing.assert_allclose(inner, whole[:, :, 8 * r0:8 * (r0 + n), 8 * c0:8 * (c0 + n)], rtol=1e-11, atol=1e-11)
    # one latent pixel closer to the edge is not exact any more
    m2 = mg - 1
    edge = crop[:, :, 8 * m2:8 * m2 + 8, 8 * mg:8 * (mg + n)]
    assert np.abs(edge - whole[:, :, 8 * (r0 - 1):8 * r0, 8 * c0:8 * (c0 + n)]).max() > 1e-9
