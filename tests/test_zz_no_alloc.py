"""The no-allocation block entry point (wan_dit_block_forward_noalloc, workspace in the
library's fixed device array) against wan_dit_block_forward with a caller workspace.

Three no-allocation calls run in a row on the same array, each with a smaller workspace
than the one before (bf16 at L = 351, the float32 toy block at L = 128, bf16 at L = 234),
so later calls find the earlier calls' values in the array.  Each must equal the workspace entry point's
result on the same inputs: within the parity bar on the block increment, and bit for bit
(the same kernels run on the same values)."""
import numpy as np
import pytest

from video_diffusion_transformer_forward_amd import synth as S

from gpu_helpers import TOL, announce, block_case, gpu_block, inc_err, native, to_dev, torch, W

pytestmark = pytest.mark.gpu

CASES = [S.get_config("mid_bf16"), S.get_config("toy"), S.get_config("mid_bf16").with_(frames=2)]


def test_noalloc_block_matches_the_workspace_entry_point():
    lib, t = W(), torch()
    sizes = [lib.workspace_bytes(c, native().ENTRY_BLOCK) for c in CASES]
    assert sizes == sorted(sizes, reverse=True) and sizes[0] <= native().NOALLOC_SCRATCH_BYTES
    inputs = [block_case(c) for c in CASES]
    refs = []
    for cfg, (w, x, mod, ctx) in zip(CASES, inputs):
        announce(f"no-alloc reference {cfg.name} L={cfg.seq_len} (workspace entry point)")
        refs.append(gpu_block(cfg, w, x, mod, ctx))
    outs = []
    for cfg, (w, x, mod, ctx) in zip(CASES, inputs):
        announce(f"no-alloc block {cfg.name} L={cfg.seq_len} (fixed scratch, {lib.workspace_bytes(cfg, 1)} bytes)")
        blk = lib.DeviceBlock(cfg, w)
        xd = to_dev(x)
        lib.dit_block_forward_noalloc(cfg, blk, xd, to_dev(mod), to_dev(ctx, lib.elem_dtype(cfg)))
        t.cuda.synchronize()
        outs.append(xd.cpu().numpy())
    for cfg, (w, x, mod, ctx), ref, got in zip(CASES, inputs, refs, outs):
        err = inc_err(got, ref, x)
        same = np.array_equal(got, ref)
        print(f"{cfg.name} L={cfg.seq_len}: no-alloc vs workspace entry point {err:.3e}, bitwise equal {same}")
        assert np.all(np.isfinite(got))
        assert err <= TOL[cfg.mode]
        assert same


def test_noalloc_block_rejects_a_shape_beyond_the_scratch():
    lib, t = W(), torch()
    cfg = S.get_config("wan13b_block").with_(frames=4)
    announce("no-alloc block beyond the scratch (host-side rejection)")
    sh = lib.shape_of(cfg)
    import ctypes
    fake = native().WanBlockWeights(*([0x100000] * 16))
    rc = native().load().wan_dit_block_forward_noalloc(ctypes.byref(sh), ctypes.byref(fake), 0x100000, 0x100000, 0,
                                                       0x100000, None)
    assert rc == native().WAN_E_SCRATCH
