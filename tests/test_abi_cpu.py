"""The C ABI without a GPU: the library loads, exports every declared entry point,
and rejects invalid arguments with the documented codes before any HIP call."""
import ctypes
import os
import re

import pytest

from video_diffusion_transformer_forward_amd import _native as N
from video_diffusion_transformer_forward_amd import shape_of, workspace_bytes
from video_diffusion_transformer_forward_amd.synth import CONFIGS, TEST_CONFIGS, get_config

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for h in ("wan.h", "wan_vae.h"):
        src = open(os.path.join(ROOT, "include", h)).read()
        names |= set(re.findall(r"^\s*(?:const\s+)?[a-z_]+\s*\*?\s*(wan_[a-z_]+)\s*\(", src, re.M))
    return sorted(names)


def test_library_exports_every_declared_function():
    lib = N.load()
    names = declared_functions()
    assert set(names) == set(N.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    lib = N.load()
    for code in range(0, -9, -1):
        assert lib.wan_status_str(code)
        assert lib.wan_status_str(code) != lib.wan_status_str(42)
    assert b"unknown" in lib.wan_status_str(42)


@pytest.mark.parametrize("name", list(CONFIGS) + list(TEST_CONFIGS))
def test_workspace_sizes(name):
    cfg = get_config(name)
    for entry in (N.ENTRY_BLOCK, N.ENTRY_STEP, N.ENTRY_HEAD, N.ENTRY_TIME_EMBED):
        assert workspace_bytes(cfg, entry) > 0
    assert workspace_bytes(cfg, N.ENTRY_PATCHIFY) == 0
    # the step holds a CFG batch of two plus the residual stream: more than one block
    assert workspace_bytes(cfg, N.ENTRY_STEP) > workspace_bytes(cfg, N.ENTRY_BLOCK)


def _ws_status(**kw):
    lib = N.load()
    cfg = get_config("toy").with_(**kw)
    sh = shape_of(cfg)
    st = ctypes.c_int(99)
    n = lib.wan_workspace_bytes(ctypes.byref(sh), N.ENTRY_BLOCK, ctypes.byref(st))
    return st.value, n


@pytest.mark.parametrize("kw,code", [
    (dict(height=15), N.WAN_E_SHAPE), (dict(width=0), N.WAN_E_SHAPE), (dict(heads=3), N.WAN_E_SHAPE),
    (dict(dim=384, heads=4), N.WAN_E_SHAPE), (dict(heads=2, dim=192), N.WAN_E_SHAPE),
    (dict(in_ch=20), N.WAN_E_SHAPE), (dict(txt_len=0), N.WAN_E_SHAPE), (dict(ffn_dim=1000), N.WAN_E_SHAPE),
    (dict(mode="fp32"), N.WAN_OK), (dict(batch=0), N.WAN_E_SHAPE), (dict(img_len=-1), N.WAN_E_SHAPE),
    (dict(dim=6144, heads=48), N.WAN_E_SHAPE),
])
def test_shape_validation(kw, code):
    st, n = _ws_status(**kw)
    assert st == code
    assert (n > 0) == (code == N.WAN_OK)


def test_mode_and_entry_validation():
    lib = N.load()
    sh = shape_of(get_config("toy"))
    sh.mode = 7
    st = ctypes.c_int(0)
    assert lib.wan_workspace_bytes(ctypes.byref(sh), N.ENTRY_BLOCK, ctypes.byref(st)) == 0
    assert st.value == N.WAN_E_MODE
    sh.mode = N.WAN_FP32
    assert lib.wan_workspace_bytes(ctypes.byref(sh), 99, ctypes.byref(st)) == 0
    assert st.value == N.WAN_E_ENTRY
    assert lib.wan_workspace_bytes(None, N.ENTRY_BLOCK, ctypes.byref(st)) == 0
    assert st.value == N.WAN_E_NULL


FAKE = 0x100000  # an aligned address that is never dereferenced: validation fails first or no device is found


def _block_call(x=FAKE, mod=FAKE, ctx=FAKE, ws=FAKE, ws_bytes=1 << 40, stride=0, weights=None, cfg="toy"):
    lib = N.load()
    sh = shape_of(get_config(cfg))
    bw = weights or N.WanBlockWeights(*([FAKE] * 16))
    return lib.wan_dit_block_forward(ctypes.byref(sh), ctypes.byref(bw), x, mod, stride, ctx, ws, ws_bytes, None)


def test_block_argument_errors_before_any_hip_call():
    assert _block_call(x=None) == N.WAN_E_NULL
    assert _block_call(ctx=None) == N.WAN_E_NULL
    assert _block_call(x=FAKE + 4) == N.WAN_E_ALIGN
    assert _block_call(ws=None) == N.WAN_E_WORKSPACE
    assert _block_call(ws_bytes=1024) == N.WAN_E_WORKSPACE
    assert _block_call(stride=5) == N.WAN_E_SHAPE
    w = N.WanBlockWeights(*([FAKE] * 16))
    w.ff2_w = None
    assert _block_call(weights=w) == N.WAN_E_NULL
    # image tokens need their own K/V projection
    lib = N.load()
    cfg = get_config("toy_i2v_fp32")
    sh = shape_of(cfg)
    w = N.WanBlockWeights(*([FAKE] * 16))
    w.ikv_w = None
    assert lib.wan_dit_block_forward(ctypes.byref(sh), ctypes.byref(w), FAKE, FAKE, 0, FAKE, FAKE, 1 << 40,
                                     None) == N.WAN_E_NULL


def test_step_argument_errors():
    lib = N.load()
    cfg = get_config("toy_step")
    sh = shape_of(cfg)
    blocks = (N.WanBlockWeights * 2)(N.WanBlockWeights(*([FAKE] * 16)), N.WanBlockWeights(*([FAKE] * 16)))
    mw = N.WanModelWeights(*([FAKE] * 10), 2, ctypes.cast(blocks, ctypes.POINTER(N.WanBlockWeights)))
    call = lambda **k: lib.wan_denoise_step(ctypes.byref(sh), ctypes.byref(mw), k.get("z", FAKE), None, FAKE, FAKE,
                                            500.0, k.get("dt", 0.05), 5.0, FAKE, k.get("wsb", 1 << 40), None)
    assert call(z=None) == N.WAN_E_NULL
    assert call(dt=float("nan")) == N.WAN_E_SHAPE
    assert call(wsb=16) == N.WAN_E_WORKSPACE
    blocks[1].qkv_w = None
    assert call() == N.WAN_E_NULL


def test_cache_sizes_and_argument_errors():
    lib = N.load()
    cfg = get_config("toy_step")
    sh = shape_of(cfg)
    st = ctypes.c_int(0)
    one = lib.wan_cache_bytes(ctypes.byref(sh), 1, ctypes.byref(st))
    assert st.value == N.WAN_OK and one > 0
    # n_blocks attention slots (2B, L, D) in the mode's type, then (B, L, 64) float32
    L, D = cfg.seq_len, cfg.dim
    slot = 2 * cfg.batch * L * D * 4
    assert lib.wan_cache_bytes(ctypes.byref(sh), 3, ctypes.byref(st)) - one >= 2 * slot
    assert lib.wan_cache_bytes(ctypes.byref(sh), 0, ctypes.byref(st)) == 0 and st.value == N.WAN_E_SHAPE
    blocks = (N.WanBlockWeights * 2)(N.WanBlockWeights(*([FAKE] * 16)), N.WanBlockWeights(*([FAKE] * 16)))
    mw = N.WanModelWeights(*([FAKE] * 10), 2, ctypes.cast(blocks, ctypes.POINTER(N.WanBlockWeights)))
    need = lib.wan_cache_bytes(ctypes.byref(sh), 2, ctypes.byref(st))
    call = lambda mode=N.CACHE_STORE, cache=FAKE, cb=need: lib.wan_denoise_step_cached(
        ctypes.byref(sh), ctypes.byref(mw), FAKE, None, FAKE, FAKE, 500.0, 0.05, 5.0, mode, cache, cb, FAKE,
        1 << 40, None)
    for bad in (0, 3, 5, 7, 8, -1):
        assert call(mode=bad) == N.WAN_E_MODE
    assert call(cache=None) == N.WAN_E_NULL
    assert call(cache=FAKE + 4) == N.WAN_E_ALIGN
    assert call(cb=need - 1) == N.WAN_E_WORKSPACE


def test_no_device_reported_as_hip_error():
    """With valid arguments the first HIP query fails on a host without a gfx950 GPU."""
    try:
        import torch
        if torch.cuda.is_available():
            pytest.skip("a GPU is present")
    except ImportError:
        pass
    assert _block_call() == N.WAN_E_HIP


def test_qk8_mode_shapes():
    """8-bit-score mode: same workspace as bf16 for 128-wide heads, WAN_E_SHAPE for 64-wide heads."""
    lib = N.load()
    st = ctypes.c_int(0)
    for name in ("mid_bf16", "wan13b_step"):
        cfg = get_config(name)
        sizes = []
        for qk8 in (False, True):
            sh = shape_of(cfg.with_(qk8=qk8))
            sizes.append(lib.wan_workspace_bytes(ctypes.byref(sh), N.ENTRY_STEP, ctypes.byref(st)))
            assert st.value == N.WAN_OK
        assert sizes[0] == sizes[1] > 0
    sh = shape_of(get_config("toy").with_(mode="bf16", qk8=True))   # dim 256, 4 heads of 64
    assert lib.wan_workspace_bytes(ctypes.byref(sh), N.ENTRY_BLOCK, ctypes.byref(st)) == 0
    assert st.value == N.WAN_E_SHAPE
    with pytest.raises(ValueError):
        shape_of(get_config("toy").with_(qk8=True))                    # fp32 has no 8-bit form


def test_fp8_mode_shapes():
    """8-bit GEMM mode: a larger workspace than bf16 (e4m3 activations, weights and scales) for
    128-wide heads, WAN_E_SHAPE for 64-wide heads."""
    lib = N.load()
    st = ctypes.c_int(0)
    cfg = get_config("wan13b_step")
    sizes = {}
    for k, kw in (("bf16", {}), ("fp8", dict(fp8=True))):
        sh = shape_of(cfg.with_(**kw))
        sizes[k] = lib.wan_workspace_bytes(ctypes.byref(sh), N.ENTRY_STEP, ctypes.byref(st))
        assert st.value == N.WAN_OK
    D, F, L = cfg.dim, cfg.ffn_dim, cfg.seq_len
    assert sizes["fp8"] - sizes["bf16"] >= 2 * L * F + 4 * D * D + 2 * F * D
    sh = shape_of(get_config("toy").with_(mode="bf16", fp8=True))
    assert lib.wan_workspace_bytes(ctypes.byref(sh), N.ENTRY_BLOCK, ctypes.byref(st)) == 0
    assert st.value == N.WAN_E_SHAPE


def test_vae_shapes_and_argument_errors():
    """VAE decoder: parameter table against the input generator's list, workspace sizes, and
    argument errors reported before any device work."""
    from video_diffusion_transformer_forward_amd import vae_synth as VS
    import video_diffusion_transformer_forward_amd as W
    lib = N.load()
    st = ctypes.c_int(0)
    cfg = VS.get_vae_config("vae_w96")
    sh = W.vae_shape_of(cfg)
    tab = W.vae_param_table(sh)
    assert [t[0] for t in tab if t[1] != 1] == [n for n, _ in VS.vae_param_shapes(cfg)]
    assert all(t[3] % 64 == 0 for t in tab)
    assert lib.wan_vae_workspace_bytes(ctypes.byref(sh), ctypes.byref(st)) > 0 and st.value == N.WAN_OK
    assert lib.wan_vae_cache_bytes(ctypes.byref(sh), ctypes.byref(st)) > 0
    for bad in (dict(base=48), dict(base=0), dict(z_ch=40), dict(n_res=0), dict(frames=0)):
        b = W.vae_shape_of(cfg.with_(**bad)) if "frames" not in bad else N.WanVaeShape(0, 5, 7, 16, 96, 2, 1)
        assert lib.wan_vae_workspace_bytes(ctypes.byref(b), ctypes.byref(st)) == 0
        assert st.value == N.WAN_E_SHAPE
    big = N.WanVaeShape(21, 600, 1040, 16, 96, 2, 21)
    assert lib.wan_vae_workspace_bytes(ctypes.byref(big), ctypes.byref(st)) == 0 and st.value == N.WAN_E_SHAPE
    F = FAKE
    dec = lambda t0, n, ws_bytes=1 << 40, cb=1 << 40, z=F: lib.wan_vae_decode(
        ctypes.byref(sh), F, F, z, t0, n, F, cb, F, F, ws_bytes, None)
    assert dec(0, 5) == N.WAN_E_SHAPE          # t0 + n > frames
    assert dec(-1, 1) == N.WAN_E_SHAPE
    assert dec(0, 0) == N.WAN_E_SHAPE
    assert dec(0, 1, ws_bytes=1024) == N.WAN_E_WORKSPACE
    assert dec(0, 1, cb=16) == N.WAN_E_WORKSPACE
    assert dec(0, 1, z=None) == N.WAN_E_NULL
    assert dec(0, 1, z=F + 4) == N.WAN_E_ALIGN


def test_vae_device_rounds_weights_to_nearest_even():
    """VaeDevice converts float32 weights that are not bf16-exact to the nearest bf16 value,
    ties to even (the DiT weights' conversion), and keeps biases and scales in float32."""
    import numpy as np
    import torch
    from video_diffusion_transformer_forward_amd import vae_synth as VS
    import video_diffusion_transformer_forward_amd as W
    cfg = VS.get_vae_config("vae_tiny")
    sh = W.vae_shape_of(cfg)
    params = VS.vae_params(cfg)
    rng = np.random.default_rng(7)
    noisy = {}
    for k, v in params.items():
        a = np.asarray(v, np.float32)
        # add sub-bf16 bits so the float32 values are not bf16-exact
        noisy[k] = (a * (1.0 + rng.uniform(-3e-3, 3e-3, a.shape))).astype(np.float32)
    name, kind, dims, off, cnt = next(t for t in W.vae_param_table(sh) if t[1] == 0)
    a = noisy[name].reshape(-1)
    # plant exact ties: the lower 16 bits 0x8000, once with an even and once with an odd upper half
    u = a.view(np.uint32)
    u[0] = np.uint32(0x3F808000)   # 1.00390625: halfway between 0x3F80 and 0x3F81 -> even 0x3F80
    u[1] = np.uint32(0x3F818000)   # halfway between 0x3F81 and 0x3F82 -> even 0x3F82
    u[2] = np.uint32(0x3F80C000)   # above the midpoint -> 0x3F81
    dev = W.VaeDevice(sh, noisy, device="cpu")
    got = dev.weights.numpy().view(np.uint16)[off:off + cnt]
    want = (torch.from_numpy(a.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
    np.testing.assert_array_equal(got, want)
    assert got[0] == 0x3F80 and got[1] == 0x3F82 and got[2] == 0x3F81
    # truncation would differ on a sizeable share of these values
    assert np.mean(got != (a.view(np.uint32) >> 16).astype(np.uint16)) > 0.2
    fname, _, _, foff, fcnt = next(t for t in W.vae_param_table(sh) if t[1] != 0)
    np.testing.assert_array_equal(dev.fparams.numpy()[foff:foff + fcnt], noisy[fname].reshape(-1))


def _noalloc_call(cfg="toy", x=FAKE, mod=FAKE, ctx=FAKE, stride=0, weights=None, **kw):
    lib = N.load()
    sh = shape_of(get_config(cfg).with_(**kw))
    bw = weights or N.WanBlockWeights(*([FAKE] * 16))
    return lib.wan_dit_block_forward_noalloc(ctypes.byref(sh), ctypes.byref(bw), x, mod, stride, ctx, None)


def test_noalloc_block_rejects_shapes_beyond_its_scratch_before_any_hip_call():
    """The no-allocation block entry point takes shapes whose block workspace fits its fixed
    64 MiB device array and rejects the others with WAN_E_SCRATCH before touching a device."""
    assert N.NOALLOC_SCRATCH_BYTES == 64 << 20
    for name in ("wan13b_block", "wan14b_720p_block", "wan14b_i2v_block"):
        assert workspace_bytes(get_config(name), N.ENTRY_BLOCK) > N.NOALLOC_SCRATCH_BYTES
        assert _noalloc_call(name) == N.WAN_E_SCRATCH
    # the 1.3B width over one 480p latent frame (L = 1560) fits; four frames (L = 6240) do not
    one = get_config("wan13b_block").with_(frames=1)
    assert workspace_bytes(one, N.ENTRY_BLOCK) <= N.NOALLOC_SCRATCH_BYTES
    assert workspace_bytes(one.with_(frames=4), N.ENTRY_BLOCK) > N.NOALLOC_SCRATCH_BYTES
    assert _noalloc_call("wan13b_block", frames=4) == N.WAN_E_SCRATCH
    for name in TEST_CONFIGS:
        assert workspace_bytes(get_config(name), N.ENTRY_BLOCK) <= N.NOALLOC_SCRATCH_BYTES
    assert _noalloc_call(x=None) == N.WAN_E_NULL
    assert _noalloc_call(ctx=FAKE + 4) == N.WAN_E_ALIGN
    assert _noalloc_call(stride=5) == N.WAN_E_SHAPE
    assert _noalloc_call(heads=3) == N.WAN_E_SHAPE
    w = N.WanBlockWeights(*([FAKE] * 16))
    w.o_w = None
    assert _noalloc_call(weights=w) == N.WAN_E_NULL


def test_noalloc_block_without_device_is_a_hip_error():
    try:
        import torch
        if torch.cuda.is_available():
            pytest.skip("a GPU is present")
    except ImportError:
        pass
    assert _noalloc_call() == N.WAN_E_HIP
    assert _noalloc_call("wan13b_block", frames=1) == N.WAN_E_HIP
