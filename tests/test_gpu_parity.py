"""GPU parity: the HIP library (through its C ABI) against the float64 oracle.

Every case prints its name before touching the GPU.  Errors are normwise
relative errors; the bar is 1e-2 for bf16 operands with float32 accumulation
and 1e-5 for the float32 mode.  Block results are compared on the increment
x_out - x_in (the residual dominates x_out itself).
"""
import numpy as np
import pytest

from oracle import wan_oracle as O
from video_diffusion_transformer_forward_amd import synth as S

from gpu_helpers import (TOL, announce, inc_err, block_case, ctx_dev, device_model, gpu_block, gpu_step, native,
                         oracle_block, rel_err, sample_rows, to_dev, torch, W)

pytestmark = pytest.mark.gpu

SMALL_BLOCK = ["toy", "mid_fp32", "mid_bf16", "mid_i2v_bf16", "mid_b2_bf16", "toy_i2v_fp32"]


# ----------------------------------------------------------------------------- patchify
@pytest.mark.parametrize("name", ["toy", "mid_bf16", "mid_i2v_bf16", "toy_i2v_fp32", "wan13b_block",
                                  "wan14b_i2v_block"])
def test_patchify(name):
    cfg = S.get_config(name)
    announce(f"patchify {name}")
    mw = S.model_weights(cfg)
    z = S.latent(cfg)
    cond = S.condition(cfg)
    lib = W()
    et = lib.elem_dtype(cfg)
    t = torch()
    x = t.empty((cfg.batch, cfg.seq_len, cfg.dim), dtype=t.float32, device="cuda")
    lib.patchify(cfg, to_dev(z), to_dev(cond) if cond is not None else None, to_dev(mw["pe_w"], et),
                 to_dev(mw["pe_b"]), x)
    t.cuda.synchronize()
    got = x.cpu().numpy()
    # the GPU takes the latent as bf16 operands in bf16 mode; the oracle sees the float32 latent
    ref = O.patchify(z, cond, mw["pe_w"], mw["pe_b"])
    err = rel_err(got, ref)
    print(f"{name}: rel err {err:.3e}")
    assert err <= TOL[cfg.mode]


# ----------------------------------------------------------------------------- time modulation
@pytest.mark.parametrize("name,tau", [("toy", 500.0), ("toy", 0.0), ("mid_bf16", 999.0), ("wan13b_block", 500.0)])
def test_time_embed(name, tau):
    cfg = S.get_config(name)
    announce(f"time_embed {name} tau={tau}")
    mw = S.model_weights(cfg)
    lib = W()
    t = torch()
    model = device_model(cfg, mw, [])
    mod = t.empty((6, cfg.dim), dtype=t.float32, device="cuda")
    ws = lib.workspace(cfg, native().ENTRY_TIME_EMBED)
    lib.time_embed(cfg, model, tau, mod, ws)
    t.cuda.synchronize()
    ref = O.time_modulation(tau, mw["t1_w"], mw["t1_b"], mw["t2_w"], mw["t2_b"], mw["m_w"], mw["m_b"])
    err = rel_err(mod.cpu().numpy(), ref)
    print(f"{name}: rel err {err:.3e}")
    # weights are exact inputs in both modes; the GEMVs accumulate in float32
    assert err <= 1e-5


# ----------------------------------------------------------------------------- block
@pytest.mark.parametrize("name", SMALL_BLOCK)
def test_block_small(name):
    cfg = S.get_config(name)
    announce(f"block {name}")
    w, x, mod, ctx = block_case(cfg)
    got = gpu_block(cfg, w, x, mod, ctx)
    ref = oracle_block(cfg, w, x, mod, ctx)
    err = inc_err(got, ref, x)
    print(f"{name}: rel err of the increment {err:.3e}")
    assert np.all(np.isfinite(got))
    assert err <= TOL[cfg.mode]


@pytest.mark.parametrize("name", ["toy", "mid_bf16"])
def test_block_shared_modulation(name):
    """mod given once as (6, D) with batch stride 0."""
    cfg = S.get_config(name).with_(batch=2)
    announce(f"block shared-mod {name}")
    w, x, mod, ctx = block_case(cfg)
    m1 = mod[0]
    got = gpu_block(cfg, w, x, m1, ctx, mod_stride=0)
    ref = oracle_block(cfg, w, x, m1, ctx)
    assert inc_err(got, ref, x) <= TOL[cfg.mode]


@pytest.mark.parametrize("name", ["toy", "mid_bf16"])
def test_block_sublayer_isolation(name):
    """Each sublayer alone: the other two switched off through gates / W_co."""
    cfg = S.get_config(name)
    w, x, mod, ctx = block_case(cfg)
    cases = {
        "self-attention": dict(zero=[5], zero_co=True),
        "cross-attention": dict(zero=[2, 5], zero_co=False),
        "ffn": dict(zero=[2], zero_co=True),
    }
    for label, c in cases.items():
        announce(f"block {name} isolation {label}")
        m = mod.copy()
        for i in c["zero"]:
            m[:, i] = 0.0
        ww = dict(w)
        if c["zero_co"]:
            ww["co_w"] = np.zeros_like(w["co_w"])
            ww["co_b"] = np.zeros_like(w["co_b"])
        got = gpu_block(cfg, ww, x, m, ctx)
        ref = oracle_block(cfg, ww, x, m, ctx)
        err = inc_err(got, ref, x)
        print(f"{name} {label}: {err:.3e}")
        assert err <= TOL[cfg.mode], label


@pytest.mark.parametrize("name", ["toy", "mid_bf16", "mid_i2v_bf16"])
def test_block_identity_when_gates_zero(name):
    cfg = S.get_config(name)
    announce(f"block identity {name}")
    w, x, mod, ctx = block_case(cfg, zero_co=True)
    mod[:, 2] = 0.0
    mod[:, 5] = 0.0
    got = gpu_block(cfg, w, x, mod, ctx)
    np.testing.assert_array_equal(got, x)


@pytest.mark.parametrize("name", ["mid_bf16", "mid_fp32"])
def test_block_attention_stress(name):
    """Peaked softmax: q/k weights scaled so the logits have std ~4, and b_v = 0."""
    base = S.get_config(name)
    cfg = base.with_(qk_std=float(np.sqrt(4.0 / base.dim)))
    announce(f"block stress {name}")
    w, x, mod, ctx = block_case(cfg)
    w["qkv_b"][2 * cfg.dim:] = 0.0      # b_v = 0: the output is all weighting
    m = mod.copy()
    m[:, 5] = 0.0
    w["co_w"] = np.zeros_like(w["co_w"])
    w["co_b"] = np.zeros_like(w["co_b"])
    got = gpu_block(cfg, w, x, m, ctx)
    ref = oracle_block(cfg, w, x, m, ctx)
    err = inc_err(got, ref, x)
    print(f"{name} stress: {err:.3e}")
    assert err <= TOL[cfg.mode]


@pytest.mark.parametrize("mode", ["fp32", "bf16"])
def test_block_degenerate_single_token(mode):
    """L = 1 token, one text token: every tile is a ragged tail."""
    cfg = S.WanConfig("tiny", 21, frames=1, height=2, width=2, dim=256, heads=2, ffn_dim=256, txt_len=1,
                      mode=mode)
    announce(f"block single token {mode}")
    w, x, mod, ctx = block_case(cfg)
    got = gpu_block(cfg, w, x, mod, ctx)
    ref = oracle_block(cfg, w, x, mod, ctx)
    assert inc_err(got, ref, x) <= TOL[mode]


def test_block_deterministic():
    cfg = S.get_config("mid_bf16")
    announce("block determinism")
    w, x, mod, ctx = block_case(cfg)
    a = gpu_block(cfg, w, x, mod, ctx)
    b = gpu_block(cfg, w, x, mod, ctx)
    np.testing.assert_array_equal(a, b)


def test_block_wan13b_full_size_sampled_rows():
    """The 1.3B block at 480p x 81 frames (L = 32760): sampled token rows against the oracle."""
    cfg = S.get_config("wan13b_block")
    announce("block wan13b full size")
    w, x, mod, ctx = block_case(cfg)
    got = gpu_block(cfg, w, x, mod, ctx)
    assert np.all(np.isfinite(got))
    rows = sample_rows(cfg.seq_len, 48, seed=3)
    ref = oracle_block(cfg, w, x, mod, ctx, rows=rows)
    err = inc_err(got[:, rows], ref, x[:, rows])
    print(f"wan13b sampled rows: rel err {err:.3e}")
    assert err <= TOL["bf16"]


@pytest.mark.slow
@pytest.mark.parametrize("name", ["wan14b_720p_block", "wan14b_i2v_block"])
def test_block_14b_full_size_sampled_rows(name):
    """The 14B block at full size: 720p x 81 frames (L = 75600, 40 heads of 128) and I2V at
    480p (L = 32760, context of 257 image + 512 text tokens, two-source cross-attention):
    sampled token rows against the oracle, whose keys and values cover every token."""
    cfg = S.get_config(name)
    announce(f"block {name} full size")
    w, x, mod, ctx = block_case(cfg)
    got = gpu_block(cfg, w, x, mod, ctx)
    assert np.all(np.isfinite(got))
    rows = sample_rows(cfg.seq_len, 12, seed=4)
    ref = oracle_block(cfg, w, x, mod, ctx, rows=rows)
    err = inc_err(got[:, rows], ref, x[:, rows])
    print(f"{name} sampled rows: rel err {err:.3e}")
    assert err <= TOL["bf16"]


def test_block_14b_i2v_two_videos_equal_single_video_runs():
    """The 14B I2V block over two videos at once (the CFG batch of a step) against two one-video
    calls on the same inputs: bit for bit (every output sums the same products in the same order
    whatever the tile it falls in).  With two videos the text and image K / V projections have
    160 tiles of 256x256 and take the 16x16 packing form without a q section, which no one-video
    shape reaches."""
    cfg = S.get_config("wan14b_i2v_block").with_(batch=2)
    announce("block wan14b_i2v two videos against one-video runs")
    w, x, mod, ctx = block_case(cfg)
    both = gpu_block(cfg, w, x, mod, ctx)
    assert np.all(np.isfinite(both))
    one = cfg.with_(batch=1)
    for b in range(2):
        single = gpu_block(one, w, x[b:b + 1], mod[b:b + 1], ctx[b:b + 1])
        same = np.array_equal(single[0], both[b])
        print(f"video {b}: two-video call equals the one-video call bitwise: {same}")
        assert same


# ----------------------------------------------------------------------------- head
@pytest.mark.parametrize("name", ["toy", "mid_bf16"])
def test_head(name):
    cfg = S.get_config(name)
    announce(f"head {name}")
    mw = S.model_weights(cfg)
    x = S.block_inputs(cfg)
    lib = W()
    t = torch()
    model = device_model(cfg, mw, [])
    v = t.empty((cfg.batch, 16, cfg.frames, cfg.height, cfg.width), dtype=t.float32, device="cuda")
    ws = lib.workspace(cfg, native().ENTRY_HEAD)
    lib.head(cfg, model, to_dev(x), v, ws)
    t.cuda.synchronize()
    ref = O.patch_scatter(O.head(x, mw["hd_w"], mw["hd_b"]), cfg.frames, cfg.height, cfg.width)
    err = rel_err(v.cpu().numpy(), ref)
    print(f"{name}: {err:.3e}")
    assert err <= TOL[cfg.mode]


# ----------------------------------------------------------------------------- denoise step
@pytest.mark.parametrize("name", ["toy_step", "mid_step_bf16"])
def test_step_small(name):
    cfg = S.get_config(name)
    announce(f"step {name}")
    mw = S.model_weights(cfg)
    bw = [S.block_weights(cfg, b) for b in range(cfg.n_blocks)]
    z = S.latent(cfg)
    cond = S.condition(cfg)
    cc, cn = S.context(cfg, "cond"), S.context(cfg, "null")
    got = gpu_step(cfg, mw, bw, z, cond, cc, cn, cfg.timestep, cfg.dt, cfg.guide_scale)
    ref = O.denoise_step(z, cond, cc, cn, mw, bw, cfg.heads, cfg.timestep, cfg.dt, cfg.guide_scale, cfg.img_len)
    err = inc_err(got, ref, z)
    print(f"{name}: rel err of dt*v {err:.3e}")
    assert err <= TOL[cfg.mode]


def test_step_i2v_small():
    cfg = S.get_config("toy_i2v_fp32").with_(n_blocks=2)
    announce("step toy_i2v_fp32")
    mw = S.model_weights(cfg)
    bw = [S.block_weights(cfg, b) for b in range(cfg.n_blocks)]
    z, cond = S.latent(cfg), S.condition(cfg)
    cc, cn = S.context(cfg, "cond"), S.context(cfg, "null")
    got = gpu_step(cfg, mw, bw, z, cond, cc, cn, 250.0, 0.05, 5.0)
    ref = O.denoise_step(z, cond, cc, cn, mw, bw, cfg.heads, 250.0, 0.05, 5.0, cfg.img_len)
    assert inc_err(got, ref, z) <= TOL["fp32"]


def test_step_wan13b_one_block_sampled():
    """The 1.3B step shape (CFG batch 2, L = 32760) with one block: sampled tokens against the oracle."""
    cfg = S.get_config("wan13b_step").with_(n_blocks=1)
    announce("step wan13b one block")
    mw = S.model_weights(cfg)
    bw = [S.block_weights(cfg, 0)]
    z = S.latent(cfg)
    cc, cn = S.context(cfg, "cond"), S.context(cfg, "null")
    got = gpu_step(cfg, mw, bw, z, None, cc, cn, cfg.timestep, cfg.dt, cfg.guide_scale)
    rows = sample_rows(cfg.seq_len, 24, seed=5)
    x = O.patchify(z, None, mw["pe_w"], mw["pe_b"])
    mod = O.time_modulation(cfg.timestep, mw["t1_w"], mw["t1_b"], mw["t2_w"], mw["t2_b"], mw["m_w"], mw["m_b"])
    v = []
    for ctx in (cc, cn):
        xr = O.dit_block(x, mod, ctx, bw[0], cfg.heads, cfg.grid, 0, rows=rows)
        v.append(O.head(xr, mw["hd_w"], mw["hd_b"]))       # (1, n, 64)
    vv = O.cfg_combine(v[0], v[1], cfg.guide_scale)[0]
    F, Hh, Ww = cfg.grid
    g_out, r_out, z_in = [], [], []
    for n, l in enumerate(rows):
        f, rem = divmod(l, Hh * Ww)
        i, j = divmod(rem, Ww)
        for c in range(16):
            for a in range(2):
                for b in range(2):
                    zv = float(z[0, c, f, 2 * i + a, 2 * j + b])
                    z_in.append(zv)
                    g_out.append(got[0, c, f, 2 * i + a, 2 * j + b])
                    r_out.append(zv + cfg.dt * vv[n, c * 4 + a * 2 + b])
    err = inc_err(g_out, r_out, z_in)
    print(f"wan13b step one block sampled: {err:.3e}")
    assert err <= TOL["bf16"]


def test_step_wan13b_30_blocks_properties():
    """Full 30-block 1.3B step: guidance linearity and identity blocks, at full size."""
    cfg = S.get_config("wan13b_step")
    announce("step wan13b 30 blocks properties")
    mw = S.model_weights(cfg)
    bw = [S.block_weights(cfg, b) for b in range(cfg.n_blocks)]
    z = S.latent(cfg)
    cc, cn = S.context(cfg, "cond"), S.context(cfg, "null")
    model = device_model(cfg, mw, bw)
    zs = {g: gpu_step(cfg, mw, bw, z, None, cc, cn, cfg.timestep, cfg.dt, g, model=model) for g in (0.0, 1.0, 5.0)}
    for g in zs.values():
        assert np.all(np.isfinite(g))
    d1 = zs[1.0].astype(np.float64) - zs[0.0]
    d5 = zs[5.0].astype(np.float64) - zs[0.0]
    err = rel_err(d5, 5 * d1)
    print(f"guidance linearity: {err:.3e}")
    assert err <= 1e-3
    # identity blocks: both gates and the cross-attention output projection zero
    mw0 = dict(mw)
    D = cfg.dim
    mw0["m_w"] = mw["m_w"].copy()
    mw0["m_b"] = mw["m_b"].copy()
    for r in (2, 5):
        mw0["m_w"][r * D:(r + 1) * D] = 0.0
        mw0["m_b"][r * D:(r + 1) * D] = 0.0
    bw0 = []
    for b in bw:
        b0 = dict(b)
        b0["co_w"] = np.zeros_like(b["co_w"])
        b0["co_b"] = np.zeros_like(b["co_b"])
        bw0.append(b0)
    del model
    got = gpu_step(cfg, mw0, bw0, z, None, cc, cn, cfg.timestep, cfg.dt, cfg.guide_scale)
    v = O.patch_scatter(O.head(O.patchify(z, None, mw["pe_w"], mw["pe_b"]), mw["hd_w"], mw["hd_b"]),
                        cfg.frames, cfg.height, cfg.width)
    err = inc_err(got, z + cfg.dt * v, z)
    print(f"identity-block step: {err:.3e}")
    assert err <= TOL["bf16"]


# ----------------------------------------------------------------------------- diffusion cache
def _cache_run(cfg, model, steps, z0, cond, cc, cn, g=5.0):
    """Run (mode, tau) steps through wan_denoise_step_cached; returns the final latent."""
    lib, t = W(), torch()
    cache = lib.diffusion_cache(cfg, cfg.n_blocks)
    ws = lib.workspace(cfg, native().ENTRY_STEP)
    zd = to_dev(z0)
    cd = to_dev(cond) if cond is not None else None
    ccd, cnd = ctx_dev(cfg, cc), ctx_dev(cfg, cn)
    for mode, tau in steps:
        if mode == 0:
            lib.denoise_step(cfg, model, zd, cd, ccd, cnd, tau, 0.05, g, ws)
        else:
            lib.denoise_step_cached(cfg, model, zd, cd, ccd, cnd, tau, 0.05, g, mode, cache, ws)
    t.cuda.synchronize()
    return zd.cpu().numpy()


def _cache_case(name):
    cfg = S.get_config(name)
    mw = S.model_weights(cfg)
    bw = [S.block_weights(cfg, b) for b in range(cfg.n_blocks)]
    return cfg, mw, bw, S.latent(cfg), S.condition(cfg), S.context(cfg, "cond"), S.context(cfg, "null")


@pytest.mark.parametrize("name", ["toy_step", "mid_step_bf16"])
def test_cache_store_and_same_state_reuse_match_the_plain_step(name):
    cfg, mw, bw, z, cond, cc, cn = _cache_case(name)
    announce(f"cache same-state {name}")
    model = device_model(cfg, mw, bw)
    plain = _cache_run(cfg, model, [(0, 500.0)], z, cond, cc, cn)
    stored = _cache_run(cfg, model, [(native().CACHE_STORE, 500.0)], z, cond, cc, cn)
    np.testing.assert_array_equal(stored, plain)
    # reusing what was stored at the very same state reproduces the step
    for mode in (native().CACHE_REUSE_ATTN, native().CACHE_REUSE_UNCOND,
                 native().CACHE_REUSE_ATTN | native().CACHE_REUSE_UNCOND):
        lib, t = W(), torch()
        cache = lib.diffusion_cache(cfg, cfg.n_blocks)
        ws = lib.workspace(cfg, native().ENTRY_STEP)
        ccd, cnd = ctx_dev(cfg, cc), ctx_dev(cfg, cn)
        cd = to_dev(cond) if cond is not None else None
        z1 = to_dev(z)
        lib.denoise_step_cached(cfg, model, z1, cd, ccd, cnd, 500.0, 0.05, 5.0, native().CACHE_STORE, cache, ws)
        z2 = to_dev(z)
        lib.denoise_step_cached(cfg, model, z2, cd, ccd, cnd, 500.0, 0.05, 5.0, mode, cache, ws)
        t.cuda.synchronize()
        err = rel_err(z2.cpu().numpy() - z, plain - z)
        print(f"{name} mode {mode} same state: {err:.3e}")
        assert err <= 1e-6


@pytest.mark.parametrize("name", ["toy_step", "mid_step_bf16"])
@pytest.mark.parametrize("mode", [2, 4, 6])
def test_cache_store_then_reuse_matches_oracle(name, mode):
    """A store step then a reuse step at a later time, against the oracle's own cache."""
    cfg, mw, bw, z, cond, cc, cn = _cache_case(name)
    announce(f"cache store+reuse {name} mode {mode}")
    model = device_model(cfg, mw, bw)
    got = _cache_run(cfg, model, [(native().CACHE_STORE, 500.0), (mode, 450.0)], z, cond, cc, cn)
    cache = {}
    z1 = O.denoise_step_cached(z, cond, cc, cn, mw, bw, cfg.heads, 500.0, 0.05, 5.0, O.CACHE_STORE, cache,
                               cfg.img_len)
    z2 = O.denoise_step_cached(z1, cond, cc, cn, mw, bw, cfg.heads, 450.0, 0.05, 5.0, mode, cache, cfg.img_len)
    err = inc_err(got, z2, z)
    print(f"{name} store+reuse mode {mode}: rel err of the two-step increment {err:.3e}")
    assert err <= TOL[cfg.mode]


@pytest.mark.parametrize("name,batch", [("toy_i2v_fp32", 1), ("mid_step_bf16", 2)])
def test_cache_i2v_and_two_videos(name, batch):
    """The cached step with image conditioning (two-source cross-attention) and with two videos per
    call (CFG batch 4), store then reuse of both the attention and the unconditional velocity."""
    cfg = S.get_config(name).with_(batch=batch, n_blocks=2)
    announce(f"cache {name} batch {batch}")
    mw = S.model_weights(cfg)
    bw = [S.block_weights(cfg, b) for b in range(cfg.n_blocks)]
    z, cond = S.latent(cfg), S.condition(cfg)
    cc, cn = S.context(cfg, "cond"), S.context(cfg, "null")
    model = device_model(cfg, mw, bw)
    both = native().CACHE_REUSE_ATTN | native().CACHE_REUSE_UNCOND
    got = _cache_run(cfg, model, [(native().CACHE_STORE, 500.0), (both, 450.0)], z, cond, cc, cn)
    cache = {}
    z1 = O.denoise_step_cached(z, cond, cc, cn, mw, bw, cfg.heads, 500.0, 0.05, 5.0, O.CACHE_STORE, cache,
                               cfg.img_len)
    z2 = O.denoise_step_cached(z1, cond, cc, cn, mw, bw, cfg.heads, 450.0, 0.05, 5.0, both, cache, cfg.img_len)
    err = inc_err(got, z2, z)
    print(f"{name} batch {batch} store+reuse: {err:.3e}")
    assert err <= TOL[cfg.mode]


def test_step_two_videos():
    """One plain step over two videos at once (CFG batch 4) against the oracle."""
    cfg = S.get_config("mid_step_bf16").with_(batch=2, n_blocks=2)
    announce("step two videos")
    mw = S.model_weights(cfg)
    bw = [S.block_weights(cfg, b) for b in range(cfg.n_blocks)]
    z = S.latent(cfg)
    cc, cn = S.context(cfg, "cond"), S.context(cfg, "null")
    got = gpu_step(cfg, mw, bw, z, None, cc, cn, 300.0, 0.05, 5.0)
    ref = O.denoise_step(z, None, cc, cn, mw, bw, cfg.heads, 300.0, 0.05, 5.0)
    assert inc_err(got, ref, z) <= TOL["bf16"]


# ----------------------------------------------------------------------------- depth of the step
def _depth_sweep(base, depths, rows_fn=None):
    mw = S.model_weights(base)
    bw_all = [S.block_weights(base, b) for b in range(max(depths))]
    z = S.latent(base)
    cc, cn = S.context(base, "cond"), S.context(base, "null")
    errs = {}
    for n in depths:
        cfg = base.with_(n_blocks=n)
        announce(f"step {base.name} depth {n}")
        got = gpu_step(cfg, mw, bw_all[:n], z, None, cc, cn, cfg.timestep, cfg.dt, cfg.guide_scale)
        ref = O.denoise_step(z, None, cc, cn, mw, bw_all[:n], cfg.heads, cfg.timestep, cfg.dt, cfg.guide_scale)
        errs[n] = inc_err(got, ref, z)
        print(f"{base.name} depth {n:2d}: rel err of dt*v {errs[n]:.3e}", flush=True)
    return errs


@pytest.mark.slow
@pytest.mark.parametrize("i2v", [False, True], ids=["t2v", "i2v"])
def test_step_14b_width_short_sequence_fp32(i2v):
    """A CFG step at the 14B width (D = 5120, 40 heads of 128, FFN 13824, 512 text tokens; I2V: 36
    input channels and 257 image tokens, decoupled cross-attention) over a short latent (grid
    (2, 8, 12), L = 192), two blocks, in the float32 mode against the oracle over the whole output.
    In bf16 this input sits beyond the 1e-2 bar for any bf16-operand computation: rounding every
    GEMM and attention operand of the float64 oracle to bf16, and nothing else, moves the step by
    1.05e-2 (the synthetic N(0, 0.02) weights give logits of std about 2 at this width), and the
    bf16 library measures 1.02-1.16e-2 here.  The bf16 form of the K / V-only packing GEMM this
    shape reaches is checked bit for bit by test_block_14b_i2v_two_videos_equal_single_video_runs."""
    extra = {"in_ch": 36, "img_len": 257} if i2v else {}
    cfg = S.get_config("wan13b_step").with_(name="wan14b_step_short", seed_base=61, dim=5120, heads=40,
                                            ffn_dim=13824, frames=2, height=16, width=24, n_blocks=2, mode="fp32",
                                            **extra)
    announce(f"step 14B width short sequence fp32 i2v={i2v}")
    mw = S.model_weights(cfg)
    bw = [S.block_weights(cfg, b) for b in range(cfg.n_blocks)]
    z, cond = S.latent(cfg), S.condition(cfg)
    cc, cn = S.context(cfg, "cond"), S.context(cfg, "null")
    got = gpu_step(cfg, mw, bw, z, cond, cc, cn, cfg.timestep, cfg.dt, cfg.guide_scale)
    ref = O.denoise_step(z, cond, cc, cn, mw, bw, cfg.heads, cfg.timestep, cfg.dt, cfg.guide_scale, cfg.img_len)
    err = inc_err(got, ref, z)
    print(f"14B-width step fp32 i2v={i2v}: rel err of dt*v {err:.3e}")
    assert err <= TOL["fp32"]


def test_step_30_blocks_against_oracle_by_depth():
    """The CFG step with 30 distinct blocks (the 1.3B model's depth) at the mid shape
    (L = 180, D = 256, head dim 128) against the oracle, and how the bf16 error grows
    with depth (1, 2, 4, 8, 16, 30 blocks)."""
    errs = _depth_sweep(S.get_config("mid_step_bf16"), [1, 2, 4, 8, 16, 30])
    assert max(errs.values()) <= TOL["bf16"]


@pytest.mark.slow
def test_step_30_blocks_13b_width_short_sequence():
    """The 1.3B model itself (30 blocks, D = 1536, 12 heads of 128, FFN 8960, 512 text
    tokens, CFG batch 2, g = 5) over a short latent (grid (2, 8, 12), L = 192) against the
    oracle over the whole output, at depths 1, 10 and 30."""
    base = S.get_config("wan13b_step").with_(name="wan13b_step_short", frames=2, height=16, width=24)
    errs = _depth_sweep(base, [1, 10, 30])
    assert max(errs.values()) <= TOL["bf16"]
