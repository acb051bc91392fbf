"""HIP graph capture of the denoise step and of the no-allocation block entry point.

wan_denoise_step and wan_dit_block_forward_noalloc enqueue only kernels and device-to-device
copies on the caller's stream, and allocate and synchronise nothing, so a caller can capture
them into a HIP graph (here through torch.cuda.CUDAGraph) and replay it.  Each replay starts
from a reset input, with eager library work on the same buffers (workspace, fixed scratch)
and device synchronisations between the replays, and must equal the eager result bit for bit
(the same kernels run on the same values)."""
import numpy as np
import pytest

from video_diffusion_transformer_forward_amd import synth as S

from gpu_helpers import announce, block_case, ctx_dev, device_model, native, to_dev, torch, W

pytestmark = pytest.mark.gpu

REPLAYS = 3


def test_step_graph_replays_equal_the_eager_step():
    lib, t = W(), torch()
    cfg = S.get_config("mid_step_bf16").with_(n_blocks=2)
    mw = S.model_weights(cfg)
    bw = [S.block_weights(cfg, b) for b in range(cfg.n_blocks)]
    model = device_model(cfg, mw, bw)
    z0 = to_dev(S.latent(cfg))
    cc, cn = ctx_dev(cfg, S.context(cfg, "cond")), ctx_dev(cfg, S.context(cfg, "null"))
    ws = lib.workspace(cfg, native().ENTRY_STEP)
    args = (cfg.timestep, cfg.dt, cfg.guide_scale, ws)

    announce("graph: eager step (reference)")
    z = z0.clone()
    lib.denoise_step(cfg, model, z, None, cc, cn, *args)
    t.cuda.synchronize()
    ref = z.cpu().numpy()
    # eager work between replays: a step on other values through the same workspace
    z_other = (2.0 * z0).contiguous()

    announce("graph: capture the step")
    zg = z0.clone()
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        lib.denoise_step(cfg, model, zg, None, cc, cn, *args)
    for r in range(REPLAYS):
        zg.copy_(z0)
        announce(f"graph: step replay {r}")
        g.replay()
        t.cuda.synchronize()
        got = zg.cpu().numpy()
        assert np.all(np.isfinite(got))
        assert np.array_equal(got, ref), f"replay {r} differs from the eager step"
        zo = z_other.clone()
        lib.denoise_step(cfg, model, zo, None, cc, cn, *args)
        t.cuda.synchronize()
    del g


def test_noalloc_block_graph_replays_equal_the_eager_call():
    lib, t = W(), torch()
    cfg = S.get_config("mid_bf16")
    w, x, mod, ctx = block_case(cfg)
    blk = lib.DeviceBlock(cfg, w)
    md, cd = to_dev(mod), to_dev(ctx, lib.elem_dtype(cfg))
    x0 = to_dev(x)

    announce("graph: eager no-allocation block (reference)")
    xe = x0.clone()
    lib.dit_block_forward_noalloc(cfg, blk, xe, md, cd)  # also looks up the scratch address
    t.cuda.synchronize()
    ref = xe.cpu().numpy()

    announce("graph: capture the no-allocation block")
    xg = x0.clone()
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        lib.dit_block_forward_noalloc(cfg, blk, xg, md, cd)
    for r in range(REPLAYS):
        xg.copy_(x0)
        announce(f"graph: block replay {r}")
        g.replay()
        t.cuda.synchronize()
        got = xg.cpu().numpy()
        assert np.all(np.isfinite(got))
        assert np.array_equal(got, ref), f"replay {r} differs from the eager call"
        # eager work on the same fixed scratch: the block on other values
        xo = (2.0 * x0).contiguous()
        lib.dit_block_forward_noalloc(cfg, blk, xo, md, cd)
        t.cuda.synchronize()
    del g
