"""Self-attention parity over ragged sequence lengths at the 1.3B width (D = 1536, 12 heads of 128, one video).

The bf16 path picks its kernel by the number of 256-query workgroups: from 512 of them
(L > 10752 at 12 heads and one video) the 8-wave form, below it the 4-wave form of 128
queries.  These lengths sit on both sides of that switch and give every remainder class of
the 64-key tile (the keys past L masked in the last tile) and of the 256-query tile (the
queries past L neither loaded nor stored):
  10000 = (1, 100, 100): 4-wave form, 16 keys in the last tile;
  10961 = (1, 97, 113): 17 keys; 11000 = (1, 100, 110): 56 keys, 248 queries in the last tile;
  11008 = (2, 43, 128): whole tiles; 11021 = (1, 107, 103): 13 keys, 13 queries in the last tile.
Logits of std about 4 (q / k weights of std sqrt(4/D)), b_v = 0 and only the self-attention
sublayer, so the output is all weighting and the online-softmax rescale fires late; bf16 and
8-bit-score modes, sampled query rows (always the first and the last) against the oracle at
the bf16 bar.
"""
import numpy as np
import pytest

from oracle import wan_oracle as O
from video_diffusion_transformer_forward_amd import synth as S

from gpu_helpers import TOL, announce, block_case, gpu_block, inc_err, sample_rows, self_attention_only

pytestmark = pytest.mark.gpu

GRIDS = {10000: (1, 100, 100), 10961: (1, 97, 113), 11000: (1, 100, 110), 11008: (2, 43, 128),
         11021: (1, 107, 103)}


@pytest.mark.parametrize("qk8", [False, True], ids=["bf16", "qk8"])
@pytest.mark.parametrize("L", sorted(GRIDS))
def test_self_attention_ragged_lengths(L, qk8):
    f, h, w_ = GRIDS[L]
    base = S.get_config("wan13b_block")
    cfg = base.with_(name=f"wan13b_L{L}", seed_base=40 + L % 17, frames=f, height=2 * h, width=2 * w_, qk8=qk8,
                     qk_std=float(np.sqrt(4.0 / base.dim)))
    assert cfg.seq_len == L and cfg.batch == 1
    announce(f"self-attention ragged L={L} grid={cfg.grid} qk8={qk8}")
    w, x, mod, ctx = block_case(cfg)
    w, mod = self_attention_only(cfg, w, mod)
    last_q = (L - 1) // 256 * 256
    rows = sorted(set(sample_rows(L, 12, seed=L) + [last_q, min(last_q + 1, L - 1), L - 2]))
    got = gpu_block(cfg, w, x, mod, ctx)
    assert np.all(np.isfinite(got))
    ref = O.dit_block(x, mod, ctx, w, cfg.heads, cfg.grid, 0, rows=rows, qk8=qk8)
    err = inc_err(got[:, rows], ref, x[:, rows])
    print(f"L={L} qk8={qk8}: rel err {err:.3e} over {len(rows)} rows")
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("qk8", [False, True], ids=["bf16", "qk8"])
def test_self_attention_static_offset_fallback(qk8):
    """The 256-query bf16 kernel offsets every exponent by |q| max_k |k|, which bounds the scores
    from above; when that bound overshoots a row's largest score by more than 64 in base 2 the
    workgroup is recomputed with the running maximum.  Here one token's key in head 0 carries a
    component of about 800 along feature d-1 (the slowest-turning RoPE pair): the bound of
    every head-0 query is then hundreds of powers of two above its scores, so all of head 0 takes
    the recomputation, while the other heads stay on the static offset.  Half of the head-0
    queries (q_{d-1} > 0) are dominated by that key, the others ignore it.  Both the bf16 kernel
    and the 8-bit-score kernel (against the oracle's 8-bit reading) take this path."""
    f, h, w_ = GRIDS[11000]
    base = S.get_config("wan13b_block")
    cfg = base.with_(name="wan13b_L11000_fb", seed_base=77, frames=f, height=2 * h, width=2 * w_, qk8=qk8)
    L = cfg.seq_len
    announce(f"self-attention static-offset fallback L={L} qk8={qk8}")
    w, x, mod, ctx = block_case(cfg)
    w, mod = self_attention_only(cfg, w, mod)
    D, d = cfg.dim, cfg.head_dim
    tok, j = 4321, 777
    qkv_w = w["qkv_w"].copy()
    qkv_w[D + 0 * d + d - 1, j] += 20.0
    w["qkv_w"] = S.round_bf16(qkv_w)
    x[:, tok, j] = 1000.0
    rows = sorted(set(sample_rows(L, 16, seed=5) + [tok, tok + 1]))
    got = gpu_block(cfg, w, x, mod, ctx)
    assert np.all(np.isfinite(got))
    ref = O.dit_block(x, mod, ctx, w, cfg.heads, cfg.grid, 0, rows=rows, qk8=qk8)
    err = inc_err(got[:, rows], ref, x[:, rows])
    print(f"L={L} planted large-norm key qk8={qk8}: rel err {err:.3e} over {len(rows)} rows")
    assert err <= TOL["bf16"]


# Short sequences reach the static-offset kernel through the batch: 43 videos x 12 heads give 516
# 256-query workgroups at one query tile each.  That kernel's three-stage K / V^T rings then hold
# more stages than there are key tiles (the copies past the last tile are clamped to it and the
# scores past L masked, the next tile's first K fragments read from a clamped stage):
#   64 = (1, 8, 8): one key tile; 130 = (2, 5, 13): three tiles, 2 keys in the last;
#   195 = (3, 5, 13): four tiles, 3 keys in the last.
SHORT = {64: (1, 8, 8), 130: (2, 5, 13), 195: (3, 5, 13)}


@pytest.mark.parametrize("L", sorted(SHORT))
def test_self_attention_few_key_tiles_static_offset(L):
    f, h, w_ = SHORT[L]
    base = S.get_config("wan13b_block")
    cfg = base.with_(name=f"wan13b_b43_L{L}", seed_base=90 + L % 11, batch=43, frames=f, height=2 * h,
                     width=2 * w_, qk_std=float(np.sqrt(4.0 / base.dim)))
    assert cfg.seq_len == L and (L + 255) // 256 * cfg.heads * cfg.batch >= 512
    announce(f"self-attention few key tiles L={L} batch={cfg.batch} grid={cfg.grid}")
    w, x, mod, ctx = block_case(cfg)
    w, mod = self_attention_only(cfg, w, mod)
    rows = sample_rows(L, 10, seed=L)
    got = gpu_block(cfg, w, x, mod, ctx)
    assert np.all(np.isfinite(got))
    ref = O.dit_block(x, mod, ctx, w, cfg.heads, cfg.grid, 0, rows=rows)
    err = inc_err(got[:, rows], ref, x[:, rows])
    print(f"L={L} batch {cfg.batch}: rel err {err:.3e} over {len(rows)} rows of every video")
    assert err <= TOL["bf16"]
