"""GPU parity of the Wan-VAE decoder (wan_vae_decode) against the float64 oracle.

bf16 convolution operands with float32 accumulation and bf16 activations
between layers.  The bar is derived from that arithmetic: the decoder stores
about thirty activation tensors in sequence, each rounded to bf16; the oracle
alone, with every convolution and RMSNorm-SiLU output and the latent rounded to
bf16 (nearest even), moves 7.6e-3 (vae_tiny) and 8.4e-3 (vae_small) away from
the exact decode.  The bar is 2e-2 normwise on the video.  Chunked
decoding through the feature cache must reproduce the whole-video decode
bit for bit (every output voxel sums the same products in the same order).
"""
import numpy as np
import pytest

from oracle import wan_vae_oracle as V
from video_diffusion_transformer_forward_amd import vae_synth as VS

from gpu_helpers import announce, rel_err, torch, W

pytestmark = pytest.mark.gpu

TOL_VAE = 2e-2
# spatial reach of the decoder, in latent pixels, rounded up: 9 3x3 convolutions at the
# latent resolution, 5 at x2, 5 at x4 and 6 at x8 (one pixel each)
VAE_REACH = 14


def _gpu_decode(cfg, params, z, chunks=None, chunk_cap=None):
    lib, t = W(), torch()
    chunks = chunks or [cfg.frames]
    sh = lib.vae_shape_of(cfg, chunk_cap or max(chunks))
    dev = lib.VaeDevice(sh, params)
    ws = lib.vae_workspace(sh)
    cache = lib.vae_cache(sh)
    outs, t0 = [], 0
    for n in chunks:
        zc = t.from_numpy(np.ascontiguousarray(z[:, t0:t0 + n])).cuda()
        n_out = 4 * n - 3 if t0 == 0 else 4 * n
        video = t.empty((3, n_out, cfg.out_height, cfg.out_width), dtype=t.float32, device="cuda")
        lib.vae_decode(sh, dev, zc, t0, n, cache, video, ws)
        outs.append(video)
        t0 += n
    t.cuda.synchronize()
    return np.concatenate([o.cpu().numpy() for o in outs], axis=1)


@pytest.mark.parametrize("name", ["vae_tiny", "vae_small", "vae_w96"])
def test_vae_decode_small(name):
    cfg = VS.get_vae_config(name)
    announce(f"vae decode {name}")
    p = VS.vae_params(cfg)
    z = VS.vae_latent(cfg)
    got = _gpu_decode(cfg, p, z)
    assert got.shape == (3, cfg.out_frames, cfg.out_height, cfg.out_width)
    assert np.all(np.isfinite(got))
    ref = V.vae_decode(z, p, cfg.dims, cfg.n_res)
    err = rel_err(got, ref)
    print(f"{name}: rel err {err:.3e}")
    assert err <= TOL_VAE


@pytest.mark.parametrize("name,chunks", [("vae_tiny", [1, 2]), ("vae_tiny", [1, 1, 1]), ("vae_small", [2, 3]),
                                         ("vae_w96", [1, 3])])
def test_vae_chunked_equals_whole(name, chunks):
    cfg = VS.get_vae_config(name)
    announce(f"vae chunked {name} {chunks}")
    p = VS.vae_params(cfg)
    z = VS.vae_latent(cfg)
    whole = _gpu_decode(cfg, p, z)
    part = _gpu_decode(cfg, p, z, chunks)
    np.testing.assert_array_equal(part, whole)


def test_vae_single_latent_frame():
    cfg = VS.get_vae_config("vae_tiny").with_(frames=1)
    announce("vae single latent frame")
    p = VS.vae_params(cfg)
    z = VS.vae_latent(cfg)
    got = _gpu_decode(cfg, p, z)
    assert got.shape[1] == 1
    assert rel_err(got, V.vae_decode(z, p, cfg.dims, cfg.n_res)) <= TOL_VAE


def test_vae_480p_full_size():
    """The 480p x 81-frame decode (21 x 60 x 104 latent, widths 384/384/384/192/96): video frame 0
    against the oracle's decode of latent frame 0 alone (by causality the same frame), the
    whole decode against a chunked one, bit for bit, over the first latent frames, and video
    frames 0-4 over a window against the oracle's decode of a latent crop."""
    cfg = VS.get_vae_config("vae_480p")
    announce("vae 480p full size")
    p = VS.vae_params(cfg)
    z = VS.vae_latent(cfg)
    got = _gpu_decode(cfg, p, z)
    assert got.shape == (3, 81, 480, 832)
    assert np.all(np.isfinite(got))
    ref0 = V.vae_decode(z[:, :1], p, cfg.dims, cfg.n_res)
    err = rel_err(got[:, :1], ref0)
    print(f"480p frame 0: rel err {err:.3e}")
    assert err <= TOL_VAE
    part = _gpu_decode(cfg, p, z[:, :3], [1, 2], chunk_cap=2)
    np.testing.assert_array_equal(part, got[:, :part.shape[1]])
    # video frames 0-4 (latent frames 0 and 1: frames 1-4 come out of both time doublings)
    # over a window of 8 x 8 latent pixels: the decoder reaches 13.5 latent pixels in space,
    # so the oracle's decode of a latent crop with a 14-pixel margin holds the whole decode's
    # values inside the margin (the CPU pins check this on a small decoder)
    r0, c0, n, mg = 26, 48, 8, VAE_REACH
    zc = z[:, :2, r0 - mg:r0 + n + mg, c0 - mg:c0 + n + mg]
    refc = V.vae_decode(zc, p, cfg.dims, cfg.n_res)[:, :, 8 * mg:8 * (mg + n), 8 * mg:8 * (mg + n)]
    err = rel_err(got[:, :5, 8 * r0:8 * (r0 + n), 8 * c0:8 * (c0 + n)], refc)
    print(f"480p frames 0-4, 64 x 64 pixel window: rel err {err:.3e}")
    assert err <= TOL_VAE
