"""GPU parity of the 8-bit-score self-attention mode (WAN_BF16_QK8) against the
oracle's 8-bit reading: q and k rows (per token and head) given power-of-two
scales and rounded to e4m3, scores from the rounded rows, everything else as
in bf16 mode.

Besides the usual bar, the peaked-softmax cases check that the library follows
the 8-bit reading and not the plain one: there the two oracles differ by several
times the bar, and the library must sit much closer to the 8-bit one.
"""
import numpy as np
import pytest

from oracle import wan_oracle as O
from video_diffusion_transformer_forward_amd import synth as S

from gpu_helpers import (TOL, announce, inc_err, block_case, gpu_block, gpu_step, oracle_block, sample_rows)

pytestmark = pytest.mark.gpu


def _sa_only(cfg, w, mod):
    """Self-attention sublayer alone: FFN gate and cross-attention output projection zero."""
    m = mod.copy()
    m[:, 5] = 0.0
    ww = dict(w)
    ww["co_w"] = np.zeros_like(w["co_w"])
    ww["co_b"] = np.zeros_like(w["co_b"])
    return ww, m


@pytest.mark.parametrize("name", ["mid_bf16", "mid_b2_bf16", "mid_i2v_bf16"])
def test_qk8_block_small(name):
    cfg = S.get_config(name).with_(qk8=True)
    announce(f"qk8 block {name}")
    w, x, mod, ctx = block_case(cfg)
    got = gpu_block(cfg, w, x, mod, ctx)
    ref = oracle_block(cfg, w, x, mod, ctx)
    err = inc_err(got, ref, x)
    print(f"{name} qk8: rel err of the increment {err:.3e}")
    assert np.all(np.isfinite(got))
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("name", ["mid_bf16", "mid_b2_bf16"])
def test_qk8_follows_the_8bit_reading(name):
    """Peaked softmax (logit std ~4, b_v = 0), self-attention only."""
    base = S.get_config(name)
    cfg = base.with_(qk_std=float(np.sqrt(4.0 / base.dim)), qk8=True)
    announce(f"qk8 peaked {name}")
    w, x, mod, ctx = block_case(cfg)
    w["qkv_b"][2 * cfg.dim:] = 0.0
    ww, m = _sa_only(cfg, w, mod)
    got = gpu_block(cfg, ww, x, m, ctx)
    ref8 = oracle_block(cfg, ww, x, m, ctx)
    ref16 = oracle_block(cfg.with_(qk8=False), ww, x, m, ctx)
    err = inc_err(got, ref8, x)
    gap = inc_err(ref16, ref8, x)
    print(f"{name}: vs 8-bit oracle {err:.3e}, 8-bit vs plain oracle {gap:.3e}")
    assert gap > 2 * TOL["bf16"]          # the case separates the two readings
    assert err <= TOL["bf16"]
    assert err < 0.2 * gap


def test_qk8_single_token():
    cfg = S.WanConfig("tiny", 21, frames=1, height=2, width=2, dim=256, heads=2, ffn_dim=256, txt_len=1,
                      mode="bf16", qk8=True)
    announce("qk8 block single token")
    w, x, mod, ctx = block_case(cfg)
    got = gpu_block(cfg, w, x, mod, ctx)
    ref = oracle_block(cfg, w, x, mod, ctx)
    assert inc_err(got, ref, x) <= TOL["bf16"]


def test_qk8_zero_rows():
    """q and k rows that are all zero (zero q/k weights and biases): scale byte 127, scores 0,
    so the self-attention output is the mean of v."""
    cfg = S.get_config("mid_bf16").with_(qk8=True)
    announce("qk8 zero q/k")
    w, x, mod, ctx = block_case(cfg)
    w["qkv_w"] = w["qkv_w"].copy()
    w["qkv_b"] = w["qkv_b"].copy()
    w["qkv_w"][: 2 * cfg.dim] = 0.0
    w["qkv_b"][: 2 * cfg.dim] = 0.0
    ww, m = _sa_only(cfg, w, mod)
    got = gpu_block(cfg, ww, x, m, ctx)
    ref = oracle_block(cfg, ww, x, m, ctx)
    assert inc_err(got, ref, x) <= TOL["bf16"]


def test_qk8_deterministic():
    cfg = S.get_config("mid_bf16").with_(qk8=True)
    announce("qk8 determinism")
    w, x, mod, ctx = block_case(cfg)
    np.testing.assert_array_equal(gpu_block(cfg, w, x, mod, ctx), gpu_block(cfg, w, x, mod, ctx))


def test_qk8_step_small():
    cfg = S.get_config("mid_step_bf16").with_(qk8=True)
    announce("qk8 step mid_step_bf16")
    mw = S.model_weights(cfg)
    bw = [S.block_weights(cfg, b) for b in range(cfg.n_blocks)]
    z = S.latent(cfg)
    cond = S.condition(cfg)
    cc, cn = S.context(cfg, "cond"), S.context(cfg, "null")
    got = gpu_step(cfg, mw, bw, z, cond, cc, cn, cfg.timestep, cfg.dt, cfg.guide_scale)
    ref = O.denoise_step(z, cond, cc, cn, mw, bw, cfg.heads, cfg.timestep, cfg.dt, cfg.guide_scale, cfg.img_len,
                         qk8=True)
    err = inc_err(got, ref, z)
    print(f"qk8 step: rel err of dt*v {err:.3e}")
    assert err <= TOL["bf16"]


def test_qk8_block_wan13b_full_size_sampled_rows():
    """The 1.3B block at 480p x 81 frames (L = 32760) in 8-bit-score mode: sampled rows."""
    cfg = S.get_config("wan13b_block").with_(qk8=True)
    announce("qk8 block wan13b full size")
    w, x, mod, ctx = block_case(cfg)
    got = gpu_block(cfg, w, x, mod, ctx)
    assert np.all(np.isfinite(got))
    rows = sample_rows(cfg.seq_len, 32, seed=7)
    ref = oracle_block(cfg, w, x, mod, ctx, rows=rows)
    err = inc_err(got[:, rows], ref, x[:, rows])
    print(f"wan13b qk8 sampled rows: rel err {err:.3e}")
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("name,peaked", [("mid_bf16", False), ("mid_b2_bf16", False), ("mid_i2v_bf16", False),
                                         ("mid_bf16", True), ("mid_b2_bf16", True)])
def test_qk8_against_the_unrounded_8bit_reading(name, peaked):
    """The library against the 8-bit reading taken on q and k projected from the exact
    (unrounded) modulated input.  The library's projection operand is bf16, which moves
    about 6% of the e4m3 codes of q and k by one step against that reading, so the bar is
    derived from the oracle alone: 1e-2 plus the distance d between the two 8-bit readings
    (decision on bf16 m / on exact m) on the same case.  On peaked softmax inputs the
    library must also sit well inside the gap between the unrounded 8-bit reading and the
    plain (non-8-bit) one, i.e. it follows the 8-bit decision."""
    base = S.get_config(name)
    cfg = base.with_(qk8=True)
    if peaked:
        cfg = cfg.with_(qk_std=float(np.sqrt(4.0 / base.dim)))
    announce(f"qk8 unrounded reading {name} peaked={peaked}")
    w, x, mod, ctx = block_case(cfg)
    if peaked:
        w["qkv_b"][2 * cfg.dim:] = 0.0
        w, mod = _sa_only(cfg, w, mod)
    got = gpu_block(cfg, w, x, mod, ctx)
    exact8 = O.dit_block(x, mod, ctx, w, cfg.heads, cfg.grid, cfg.img_len, qk8=True, qk8_exact=True)
    round8 = O.dit_block(x, mod, ctx, w, cfg.heads, cfg.grid, cfg.img_len, qk8=True)
    plain = O.dit_block(x, mod, ctx, w, cfg.heads, cfg.grid, cfg.img_len)
    d = inc_err(round8, exact8, x)
    bar = TOL["bf16"] + d
    err = inc_err(got, exact8, x)
    gap = inc_err(plain, exact8, x)
    print(f"{name} peaked={peaked}: vs unrounded 8-bit {err:.3e} (bar {bar:.3e}, readings apart {d:.3e}); "
          f"vs bf16-decided 8-bit {inc_err(got, round8, x):.3e}; unrounded 8-bit vs plain {gap:.3e}")
    assert err <= bar
    if peaked:
        assert gap > 2 * TOL["bf16"]
        assert err < 0.5 * gap


def test_qk8_wan13b_full_size_against_the_unrounded_reading():
    """1.3B block at L = 32760, sampled rows, against the 8-bit reading decided on exact m."""
    cfg = S.get_config("wan13b_block").with_(qk8=True)
    announce("qk8 wan13b full size, unrounded reading")
    w, x, mod, ctx = block_case(cfg)
    got = gpu_block(cfg, w, x, mod, ctx)
    rows = sample_rows(cfg.seq_len, 16, seed=11)
    exact8 = O.dit_block(x, mod, ctx, w, cfg.heads, cfg.grid, 0, rows=rows, qk8=True, qk8_exact=True)
    round8 = O.dit_block(x, mod, ctx, w, cfg.heads, cfg.grid, 0, rows=rows, qk8=True)
    d = inc_err(round8, exact8, x[:, rows])
    err = inc_err(got[:, rows], exact8, x[:, rows])
    print(f"wan13b qk8 vs unrounded reading {err:.3e} (readings apart {d:.3e})")
    assert err <= TOL["bf16"] + d
