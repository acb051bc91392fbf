"""GPU parity of the streaming denoise queue (wan_stream_tick) against the oracle's tick.

The Euler increment of a tick (frames_out - window slot 0, and the shifted window's
increments) is compared, as the block results are: the latent itself dominates
the values.  Several ticks in a row are compared on the emitted frames.
"""
import numpy as np
import pytest

from oracle import wan_oracle as O
from video_diffusion_transformer_forward_amd import synth as S

from gpu_helpers import TOL, announce, ctx_dev, device_model, inc_err, rel_err, to_dev, torch, W

pytestmark = pytest.mark.gpu

CASES = {
    "bf16_k4": (S.WanConfig("stream_bf16", 41, frames=4, height=12, width=20, dim=256, heads=2, ffn_dim=512,
                            txt_len=24, n_blocks=2, mode="bf16"), 1),
    "fp32_k2": (S.WanConfig("stream_fp32", 42, frames=4, height=8, width=8, dim=256, heads=4, ffn_dim=512,
                            txt_len=16, n_blocks=2, mode="fp32"), 2),
    "qk8_k4": (S.WanConfig("stream_qk8", 43, frames=4, height=12, width=20, dim=256, heads=2, ffn_dim=512,
                           txt_len=24, n_blocks=2, mode="bf16", qk8=True), 1),
}


def _levels(K):
    """Slot k at t = (K - 1 - k) / K of the flow (t = 0 noise), one step of 1/K per tick."""
    taus = [1000.0 * (1.0 - (K - 1 - k) / K) for k in range(K)]
    return taus, [1.0 / K] * K


def _noise(cfg, group, tick):
    rng = np.random.default_rng(1000 + tick)
    return rng.standard_normal((1, 16, group, cfg.height, cfg.width)).astype(np.float32)


def _run(cfg, group, ticks):
    mw = S.model_weights(cfg)
    bw = [S.block_weights(cfg, b) for b in range(cfg.n_blocks)]
    z0 = S.latent(cfg)
    ctx = S.context(cfg, "cond")
    K = cfg.frames // group
    taus, dts = _levels(K)
    lib, t = W(), torch()
    model = device_model(cfg, mw, bw)
    ws = lib.stream_workspace(cfg, group)
    win = to_dev(z0)
    cd = ctx_dev(cfg, ctx)
    got = []
    for i in range(ticks):
        out = t.empty((1, 16, group, cfg.height, cfg.width), dtype=t.float32, device="cuda")
        lib.stream_tick(cfg, model, win, cd, taus, dts, group, to_dev(_noise(cfg, group, i)), out, ws)
        got.append(out)
    t.cuda.synchronize()
    got = [g.cpu().numpy() for g in got]
    ref, w_ref = [], z0
    for i in range(ticks):
        w_ref, o = O.stream_tick(w_ref, ctx, mw, bw, cfg.heads, taus, dts, group, _noise(cfg, group, i),
                                 qk8=cfg.qk8)
        ref.append(o)
    return z0, got, win.cpu().numpy(), ref, w_ref


@pytest.mark.parametrize("case", sorted(CASES))
def test_stream_one_tick(case):
    cfg, group = CASES[case]
    announce(f"stream one tick {case}")
    z0, got, win, ref, w_ref = _run(cfg, group, 1)
    tol = TOL[cfg.mode]
    e_out = inc_err(got[0], ref[0], z0[:, :, :group])
    e_win = inc_err(win[:, :, :-group], w_ref[:, :, :-group], z0[:, :, group:])
    print(f"{case}: emitted {e_out:.3e}, window {e_win:.3e}")
    assert e_out <= tol and e_win <= tol
    np.testing.assert_array_equal(win[:, :, -group:], _noise(cfg, group, 0))


@pytest.mark.parametrize("case", ["bf16_k4", "fp32_k2"])
def test_stream_several_ticks(case):
    cfg, group = CASES[case]
    announce(f"stream five ticks {case}")
    z0, got, win, ref, w_ref = _run(cfg, group, 5)
    tol = TOL[cfg.mode]
    for i, (g, r) in enumerate(zip(got, ref)):
        err = rel_err(g, r)
        print(f"{case} tick {i}: emitted {err:.3e}")
        assert err <= tol
    assert rel_err(win, w_ref) <= tol


def test_stream_full_shape_one_block():
    """The bench's streaming shape (480p latent 60 x 104, 4 slots of one frame, L = 6240, 1.3B widths)
    with one block: one tick against the oracle's tick."""
    cfg = S.get_config("wan13b_step").with_(frames=4, n_blocks=1, batch=1)
    announce("stream full shape one block")
    z0, got, win, ref, w_ref = _run(cfg, 1, 1)
    e_out = inc_err(got[0], ref[0], z0[:, :, :1])
    e_win = inc_err(win[:, :, :-1], w_ref[:, :, :-1], z0[:, :, 1:])
    print(f"full shape: emitted {e_out:.3e}, window {e_win:.3e}")
    assert e_out <= TOL["bf16"] and e_win <= TOL["bf16"]
