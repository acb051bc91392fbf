"""Plain float64 CPU oracle for the Wan2.1 DiT block and CFG/Euler denoise step.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this module; the product path never
calls it and shares no code with it.

Every function computes the plain definition of one step, in float64 numpy
(a BLAS matmul serves as the contraction), with no blocking, fusion or
reordering beyond what the definition states.  Inputs are the very values the
GPU library receives (bf16-exact where the library takes bf16), upcast to
float64; nothing here emulates GPU rounding.

Sources (the pages the method is described on):
  [P2] hyper.ai summary of the Wan technical report (arXiv 2503.20314),
       section "方法" (method): patchify / blocks / unpatchify, the time MLP
       predicting six modulation parameters, flow matching velocity.
  [P3] zizhi168.cn, "阿里Wan 2.1视频生成模型深度剖析", section "核心代码实现亮点":
       the classifier-free guidance combine, the image-context concatenation,
       RoPE applied to q and k before attention.
  [P1] CSDN "wan2.1 论文精读二", section 1.1 (I2V input channels and mask),
       section 5 (camera adapter, the (gamma + 1) * f + beta modulation form).
  [P4] kwkr.cn "单流DiT与Flow Matching架构解析", sections 3.2 and 4.4
       (Euler integration of the predicted velocity; text garbled there).

Where the pages are silent the readings used are listed in the design notes;
each function names the reading it takes.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf

LN_EPS = 1e-6
ROPE_THETA = 10000.0
TIME_FREQ_DIM = 256


def f64(a):
    return np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------------- patchify
def patch_gather(u):
    """Cut the latent into (1, 2, 2) patches.

    [P2] method: a 3D convolution with kernel (1, 2, 2) turns the latent into a
    (B, L, D) sequence.  With kernel == stride the convolution is a linear map
    of each non-overlapping patch; this function lists the patches.

    u: (B, C, F, H, W).  Returns (B, L, C*4) with token l = (f*(H/2) + i)*(W/2) + j
    and feature k = c*4 + a*2 + b holding u[c, f, 2i+a, 2j+b].
    """
    u = f64(u)
    B, C, F, H, W = u.shape
    t = u.reshape(B, C, F, H // 2, 2, W // 2, 2)          # b c f i a j b'
    t = t.transpose(0, 2, 3, 5, 1, 4, 6)                   # b f i j c a b'
    return t.reshape(B, F * (H // 2) * (W // 2), C * 4)


def patch_scatter(p, F, H, W):
    """Inverse of patch_gather: (B, L, C*4) -> (B, C, F, H, W)."""
    p = f64(p)
    B, L, K = p.shape
    C = K // 4
    t = p.reshape(B, F, H // 2, W // 2, C, 2, 2)           # b f i j c a b'
    t = t.transpose(0, 4, 1, 2, 5, 3, 6)                   # b c f i a j b'
    return t.reshape(B, C, F, H, W)


def patchify(z, cond, pe_w, pe_b):
    """Patch embedding x = W_pe u + b_pe per (1,2,2) patch.

    z: (B, 16, F, H, W); cond: None or (B, 20, F, H, W) = [mask(4); z_c(16)]
    ([P1] 1.1: noisy latent, mask and condition latent joined on the channel
    axis; channel order taken as [z_t; mask; z_c]).  pe_w: (D, C_in*4) which is
    the (D, C_in, 1, 2, 2) convolution weight flattened row-major.
    """
    u = f64(z) if cond is None else np.concatenate([f64(z), f64(cond)], axis=1)
    return patch_gather(u) @ f64(pe_w).T + f64(pe_b)


# --------------------------------------------------------------------------- time MLP
def timestep_sinusoid(tau, n=TIME_FREQ_DIM):
    """Sinusoidal timestep features s = [cos(tau*w_k) ; sin(tau*w_k)], w_k = 10000^(-k/(n/2)).

    The pages name a time embedding processed by an MLP ([P2] method) but not
    its feature map; the standard transformer sinusoid is taken.
    """
    half = n // 2
    k = np.arange(half, dtype=np.float64)
    w = ROPE_THETA ** (-k / half)
    a = float(tau) * w
    return np.concatenate([np.cos(a), np.sin(a)])


def silu(x):
    x = f64(x)
    return x / (1.0 + np.exp(-x))


def time_modulation(tau, t1_w, t1_b, t2_w, t2_b, m_w, m_b):
    """Six modulation vectors shared by every block.

    [P2] method: an MLP of a Linear and a SiLU layer processes the time
    embedding and predicts six modulation parameters; [P2] experiments: the
    AdaLN is fully shared by all blocks.  The embedding
    before it is the two-layer DiT timestep embedder:
        e   = W_t2 SiLU(W_t1 s + b_t1) + b_t2
        mod = W_m SiLU(e) + b_m                     -> (6, D)
    Order of the six: shift1, scale1, gate1, shift2, scale2, gate2.
    """
    s = timestep_sinusoid(tau)
    e = f64(t2_w) @ silu(f64(t1_w) @ s + f64(t1_b)) + f64(t2_b)
    mod = f64(m_w) @ silu(e) + f64(m_b)
    return mod.reshape(6, -1)


# --------------------------------------------------------------------------- norms
def layer_norm(x, eps=LN_EPS):
    """LayerNorm over the last axis, biased variance, no affine."""
    x = f64(x)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps)


def modulate(xn, shift, scale):
    """AdaLN modulation xn * (1 + scale) + shift.

    [P1] section 5 writes the adaptive normalisation as (gamma + 1) * f + beta;
    the block uses the same form with (scale, shift) from the time MLP.
    """
    return f64(xn) * (1.0 + f64(scale)) + f64(shift)


def gelu(x):
    """Exact GELU: x/2 * (1 + erf(x / sqrt 2))."""
    x = f64(x)
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


# --------------------------------------------------------------------------- RoPE
def rope_sections(d):
    """Split of a head's d features over (frame, row, column): (d - 4*(d//6), 2*(d//6), 2*(d//6))."""
    ds = 2 * (d // 6)
    return (d - 2 * ds, ds, ds)


def grid_positions(grid):
    """(L, 3) 0-based (frame, row, column) index of each token, row-major over the grid."""
    F, Hh, Ww = grid
    f, i, j = np.meshgrid(np.arange(F), np.arange(Hh), np.arange(Ww), indexing="ij")
    return np.stack([f.ravel(), i.ravel(), j.ravel()], axis=1).astype(np.float64)


def rope_apply(x, grid, rows=None):
    """3D rotary position embedding of q or k.

    [P3] core code: rope_apply(q, grid_sizes, freqs) rotates q and k (not v)
    before attention.  Reading taken: the head dimension is split over the
    (frame, row, column) axes as rope_sections(d); within an axis segment of
    size d_a, the adjacent pair (2r, 2r+1) is rotated by angle
    pos * 10000^(-2r/d_a).

    x: (B, n, H, d) for the tokens `rows` of the grid (all tokens if None).
    Returns the rotated copy.
    """
    x = f64(x)
    B, n, H, d = x.shape
    pos = grid_positions(grid)
    if rows is not None:
        pos = pos[np.asarray(rows)]
    assert pos.shape[0] == n
    out = x.copy()
    off = 0
    for axis, da in enumerate(rope_sections(d)):
        r = np.arange(da // 2, dtype=np.float64)
        theta = ROPE_THETA ** (-2.0 * r / da)
        phi = pos[:, axis][:, None] * theta[None, :]          # (n, da/2)
        c = np.cos(phi)[None, :, None, :]
        s = np.sin(phi)[None, :, None, :]
        u0 = x[..., off + 0:off + da:2]
        u1 = x[..., off + 1:off + da:2]
        out[..., off + 0:off + da:2] = u0 * c - u1 * s
        out[..., off + 1:off + da:2] = u0 * s + u1 * c
        off += da
    return out


# --------------------------------------------------------------------------- attention
def attention(q, k, v, chunk=4096):
    """softmax(q k^T / sqrt(d)) v for one head, full (no mask, no window).

    q: (Lq, d), k: (Lk, d), v: (Lk, d).  Two-pass, max-subtracted softmax,
    evaluated over blocks of query rows to bound memory.
    """
    q, k, v = f64(q), f64(k), f64(v)
    d = q.shape[-1]
    out = np.empty((q.shape[0], v.shape[1]))
    for r0 in range(0, q.shape[0], chunk):
        s = q[r0:r0 + chunk] @ k.T / math.sqrt(d)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        out[r0:r0 + chunk] = p @ v
    return out


# --------------------------------------------------------------------------- 8-bit Q K^T
E4M3_MAX = 448.0


def e4m3_round(x):
    """Nearest float8 e4m3 value (4 exponent bits with bias 7, 3 mantissa bits,
    subnormal spacing 2^-9, largest finite value 448), ties to the even code.
    Inputs must satisfy |x| <= 448."""
    x = f64(x)
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    e = np.maximum(e, -6.0)           # below 2^-6 the spacing stays 2^-9 (subnormals)
    step = np.exp2(e - 3.0)
    return np.sign(x) * np.round(ax / step) * step   # np.round: half to even


def quantize_rows_e4m3(x):
    """8-bit form of q or k ([P2] method: FP8 GEMM and 8-bit FlashAttention at
    inference; the scaling rule is this build's reading): every row (one token of
    one head) is rounded to float32, given the power-of-two scale 2^e with the
    smallest e such that max|row| / 2^e <= 448 (clamped to [-127, 127]), and
    rounded to e4m3 in that scale.
    Returns the dequantized rows (float64) and the exponents e."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    amax = np.abs(x32).max(axis=-1)
    mant, ex = np.frexp(amax)           # amax = mant * 2^ex, mant in [0.5, 1)
    e = np.where(amax > 0, ex - 9 + (mant > 0.875), 0).astype(np.int64)
    e = np.clip(e, -127, 127)            # the range of an 8-bit power-of-two scale (exponent + 127)
    scale = np.exp2(e.astype(np.float64))[..., None]
    return e4m3_round(x32 / scale) * scale, e


def round_bf16_rne(a):
    """Nearest bfloat16 value of float32(a), ties to even (bfloat16 is the upper
    half of a float32: 8 exponent bits, 7 mantissa bits)."""
    u = np.asarray(a, dtype=np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


FP8_BLOCK = 128


def quantize_blocks_e4m3(x, block=FP8_BLOCK):
    """8-bit form of a GEMM operand ([P2] method: FP8 GEMMs at inference; the
    scaling rule is this build's reading): each row is cut into blocks of
    `block` consecutive elements along the contraction axis, and every block is
    quantised as one row of quantize_rows_e4m3 (its own power-of-two scale,
    e4m3 values).  Returns the dequantised operand (float64)."""
    x = f64(x)
    shp = x.shape
    q, _ = quantize_rows_e4m3(x.reshape(shp[:-1] + (shp[-1] // block, block)))
    return q.reshape(shp)


def linear_fp8(x, w, b):
    """x W^T + b with both operands in their 8-bit form (blocks of 128 along the
    contraction axis: per token for x, per output feature for W)."""
    return quantize_blocks_e4m3(x) @ quantize_blocks_e4m3(w).T + f64(b)


def attention_qk8(q, k, v, chunk=4096):
    """attention() with q and k in their 8-bit form (quantize_rows_e4m3, per token);
    the probabilities and v stay exact."""
    return attention(quantize_rows_e4m3(q)[0], quantize_rows_e4m3(k)[0], v, chunk)


def multihead_attention(q, k, v, heads, qk8=False):
    """q: (B, Lq, D), k/v: (B, Lk, D); head h uses features [h*d, (h+1)*d).
    qk8: q and k of every head in their 8-bit form (attention_qk8)."""
    q, k, v = f64(q), f64(k), f64(v)
    B, Lq, D = q.shape
    d = D // heads
    out = np.empty((B, Lq, D))
    for b in range(B):
        for h in range(heads):
            sl = slice(h * d, (h + 1) * d)
            att = attention_qk8 if qk8 else attention
            out[b, :, sl] = att(q[b, :, sl], k[b, :, sl], v[b, :, sl])
    return out


# --------------------------------------------------------------------------- block
def _lin(x, w, b):
    return f64(x) @ f64(w).T + f64(b)


def self_attention(m_all, w, heads, grid, rows=None, attn=None, record=None, qk8=False, fp8=False,
                   qk8_exact=False):
    """Self-attention sublayer output (before its gate).

    q, k, v = m W_qkv^T + b_qkv (rows of W_qkv ordered [q; k; v]); RoPE on q and
    k ([P3] core code); full attention over every token; output projection W_o.
    m_all: the modulated input of every token (source of keys and values);
    rows: token indices whose outputs are wanted (None = all).
    attn: a cached attention output (B, L, D) (heads concatenated, before W_o)
    used instead of computing q, k, v and the attention (the diffusion cache);
    record: a list that receives the attention output computed here;
    qk8: the scores from q and k in their 8-bit form (attention_qk8).  The 8-bit
    rounding is a decision taken on q and k, so it is taken on the values the
    library decides on: q and k projected from the bfloat16 form of m (the
    operand precision of the projection in bf16 mode), see round_bf16_rne.
    fp8: the q, k, v projection is an 8-bit GEMM (linear_fp8); q and k are then
    decided on as that GEMM gives them (implies qk8).
    qk8_exact: take the 8-bit decision on q and k projected from the exact m
    instead (the plain reading, with no rounding of the projection input).
    """
    qk8 = qk8 or fp8
    if attn is not None:
        a = f64(attn) if rows is None else f64(attn)[:, rows]
        return _lin(a, w["o_w"], w["o_b"])
    B, L, D = m_all.shape
    d = D // heads
    wq, wk, wv = np.split(f64(w["qkv_w"]), 3, axis=0)
    bq, bk, bv = np.split(f64(w["qkv_b"]), 3)
    lin = linear_fp8 if fp8 else _lin
    m_qk = round_bf16_rne(m_all) if qk8 and not fp8 and not qk8_exact else m_all
    k = rope_apply(lin(m_qk, wk, bk).reshape(B, L, heads, d), grid).reshape(B, L, D)
    v = lin(m_all, wv, bv)
    mq = m_qk if rows is None else m_qk[:, rows]
    n = mq.shape[1]
    q = rope_apply(lin(mq, wq, bq).reshape(B, n, heads, d), grid, rows).reshape(B, n, D)
    a = multihead_attention(q, k, v, heads, qk8)
    if record is not None:
        record.append(a)
    return _lin(a, w["o_w"], w["o_b"])


def cross_attention(xn, ctx, w, heads, img_len, fp8=False):
    """Cross-attention to the context tokens (ungated, un-modulated).

    [P2] method: text conditions enter through cross-attention.  [P3] core code:
    for image-to-video the image tokens are placed before the text tokens in
    the context.  [P1] 1.1 names it decoupled cross-attention; reading taken:
    one shared query projection, separate K/V projections and separate softmax
    for the image tokens and the text tokens, the two results summed before the
    shared output projection.
    fp8: the query projection is an 8-bit GEMM (linear_fp8); the context K / V
    projections and the output projection stay exact.
    """
    q = (linear_fp8 if fp8 else _lin)(xn, w["cq_w"], w["cq_b"])
    ctx = f64(ctx)
    D = ctx.shape[-1]
    ctx_img, ctx_txt = ctx[:, :img_len], ctx[:, img_len:]
    kv = _lin(ctx_txt, w["ckv_w"], w["ckv_b"])
    a = multihead_attention(q, kv[..., :D], kv[..., D:], heads)
    if img_len > 0:
        kvi = _lin(ctx_img, w["ikv_w"], w["ikv_b"])
        a = a + multihead_attention(q, kvi[..., :D], kvi[..., D:], heads)
    return _lin(a, w["co_w"], w["co_b"])


def ffn(xm, w, fp8=False):
    """GELU feed-forward: W2 GELU(W1 m + b1) + b2 (fp8: both as 8-bit GEMMs, linear_fp8)."""
    lin = linear_fp8 if fp8 else _lin
    return lin(gelu(lin(xm, w["ff1_w"], w["ff1_b"])), w["ff2_w"], w["ff2_b"])


def dit_block(x, mod, ctx, w, heads, grid, img_len=0, rows=None, attn=None, record=None, qk8=False, fp8=False,
              qk8_exact=False):
    """One DiT block, residual stream in float64.

        x <- x + g1 * SA(LN(x) (1 + sc1) + sh1)
        x <- x + CA(LN(x), ctx)
        x <- x + g2 * FFN(LN(x) (1 + sc2) + sh2)

    x: (B, L, D); mod: (B, 6, D) or (6, D) (shift1, scale1, gate1, shift2,
    scale2, gate2), or (B, L, 6, D) for a modulation per token (the streaming
    queue's per-frame noise levels); ctx: (B, L_img + L_txt, D).
    rows: if given, return only those tokens' outputs (the keys and values of
    self-attention still come from every token) -> (B, len(rows), D).
    attn / record: see self_attention (diffusion cache); qk8: 8-bit q k^T in self-attention;
    fp8: the q/k/v, cross-attention query and both FFN projections as 8-bit GEMMs, plus qk8;
    qk8_exact: see self_attention.
    """
    x = f64(x)
    mod = f64(mod)
    if mod.ndim == 2:
        mod = mod[None]
    if mod.ndim == 4:                      # per token: (B, L, 6, D)
        sh1, sc1, g1, sh2, sc2, g2 = [mod[:, :, i] for i in range(6)]
    else:
        sh1, sc1, g1, sh2, sc2, g2 = [mod[:, i][:, None, :] for i in range(6)]
    m_all = modulate(layer_norm(x), sh1, sc1)
    if mod.ndim == 4 and rows is not None:
        g1, sh2, sc2, g2 = [a[:, rows] for a in (g1, sh2, sc2, g2)]
    xr = x if rows is None else x[:, rows]
    xr = xr + g1 * self_attention(m_all, w, heads, grid, rows, attn, record, qk8, fp8, qk8_exact)
    xr = xr + cross_attention(layer_norm(xr), ctx, w, heads, img_len, fp8)
    xr = xr + g2 * ffn(modulate(layer_norm(xr), sh2, sc2), w, fp8)
    return xr


# --------------------------------------------------------------------------- head + sampler
def head(x, hd_w, hd_b):
    """Output head: LN (no affine) then Linear D -> out_ch*4 per token."""
    return _lin(layer_norm(x), hd_w, hd_b)


def cfg_combine(v_cond, v_null, guide_scale):
    """Classifier-free guidance ([P3] core code): v = v_null + g (v_cond - v_null)."""
    v_cond, v_null = f64(v_cond), f64(v_null)
    return v_null + guide_scale * (v_cond - v_null)


def euler_update(z, v, dt):
    """Flow-matching Euler step z <- z + dt * v.

    [P2] method: the model predicts the velocity of the straight path from
    noise x0 to data x1; [P4] 4.4: each sampling step updates the state with
    the predicted velocity times the step size.
    """
    return f64(z) + dt * f64(v)


def dit_forward(z, cond, ctx, model_w, blocks_w, heads, tau, img_len=0, attn_cache=None, record=None, qk8=False,
                fp8=False):
    """Velocity prediction of the whole DiT for one context: (B, 16, F, H, W).

    attn_cache: per-block cached self-attention outputs to use instead of
    computing them; record: a list that receives each block's attention output.
    """
    B, _, F, H, W = np.shape(z)
    grid = (F, H // 2, W // 2)
    x = patchify(z, cond, model_w["pe_w"], model_w["pe_b"])
    mod = time_modulation(tau, model_w["t1_w"], model_w["t1_b"], model_w["t2_w"],
                          model_w["t2_b"], model_w["m_w"], model_w["m_b"])
    for i, w in enumerate(blocks_w):
        x = dit_block(x, mod, ctx, w, heads, grid, img_len,
                      attn=None if attn_cache is None else attn_cache[i], record=record, qk8=qk8, fp8=fp8)
    p = head(x, model_w["hd_w"], model_w["hd_b"])
    return patch_scatter(p, F, H, W)


def denoise_step(z, cond, ctx_cond, ctx_null, model_w, blocks_w, heads, tau, dt,
                 guide_scale, img_len=0, qk8=False, fp8=False):
    """One CFG denoise step: both branches, guidance combine, Euler update."""
    v_c = dit_forward(z, cond, ctx_cond, model_w, blocks_w, heads, tau, img_len, qk8=qk8, fp8=fp8)
    v_u = dit_forward(z, cond, ctx_null, model_w, blocks_w, heads, tau, img_len, qk8=qk8, fp8=fp8)
    return euler_update(z, cfg_combine(v_c, v_u, guide_scale), dt)


# --------------------------------------------------------------------------- diffusion cache
CACHE_STORE = 1
CACHE_REUSE_ATTN = 2
CACHE_REUSE_UNCOND = 4


def denoise_step_cached(z, cond, ctx_cond, ctx_null, model_w, blocks_w, heads, tau, dt,
                        guide_scale, mode, cache, img_len=0, qk8=False, fp8=False):
    """One CFG denoise step with the diffusion cache ([P2] method: inference reuses
    the similarity of attention between sampling steps and of the two CFG
    branches; the pages give no further rule, the reading taken is):

      CACHE_STORE         the full step; keeps every block's self-attention output
                          of both branches and the unconditional velocity;
      CACHE_REUSE_ATTN    every block takes its self-attention output (before the
                          output projection) from the cache instead of computing it;
      CACHE_REUSE_UNCOND  only the conditional branch runs; the unconditional
                          velocity comes from the cache.

    cache: a dict filled by a CACHE_STORE step ("attn_c", "attn_u": per-block
    arrays; "v_u": the unconditional velocity).  Returns the new latent.
    """
    if mode == CACHE_STORE:
        rec_c, rec_u = [], []
        v_c = dit_forward(z, cond, ctx_cond, model_w, blocks_w, heads, tau, img_len, record=rec_c,
                          qk8=qk8, fp8=fp8)
        v_u = dit_forward(z, cond, ctx_null, model_w, blocks_w, heads, tau, img_len, record=rec_u,
                          qk8=qk8, fp8=fp8)
        cache["attn_c"], cache["attn_u"], cache["v_u"] = rec_c, rec_u, v_u
    else:
        if mode & ~(CACHE_REUSE_ATTN | CACHE_REUSE_UNCOND) or mode == 0:
            raise ValueError(f"cache mode {mode}")
        reuse_attn = bool(mode & CACHE_REUSE_ATTN)
        v_c = dit_forward(z, cond, ctx_cond, model_w, blocks_w, heads, tau, img_len,
                          attn_cache=cache["attn_c"] if reuse_attn else None, qk8=qk8, fp8=fp8)
        if mode & CACHE_REUSE_UNCOND:
            v_u = cache["v_u"]
        else:
            v_u = dit_forward(z, cond, ctx_null, model_w, blocks_w, heads, tau, img_len,
                              attn_cache=cache["attn_u"] if reuse_attn else None, qk8=qk8, fp8=fp8)
    return euler_update(z, cfg_combine(v_c, v_u, guide_scale), dt)


# --------------------------------------------------------------------------- streaming queue
def stream_tick(window, ctx, model_w, blocks_w, heads, taus, dts, group, noise_in, qk8=False):
    """One tick of the streaming denoise queue ([P1] 6.2 Streamer: a sliding
    temporal window makes arbitrarily long videos; 6.3: with a distilled
    consistency model the classifier-free guidance is folded into the model and
    a frame needs four sampling steps).  Reading taken: the window holds K slots
    of `group` latent frames each, slot 0 the oldest; slot k sits at noise level
    taus[k] (its own time modulation, the same for all of its tokens) and moves by
    dts[k] in one Euler step of the conditional velocity (no guidance); the
    whole window attends as one video (RoPE positions are window positions).
    After the step slot 0 leaves the queue and `noise_in` enters as the newest
    slot.

    window (1, 16, K*group, H, W); noise_in (1, 16, group, H, W).
    Returns (new window, emitted frames (1, 16, group, H, W))."""
    window = f64(window)
    B, C, F, H, W = window.shape
    K = len(taus)
    assert B == 1 and F == K * group and len(dts) == K
    grid = (F, H // 2, W // 2)
    per_frame = (H // 2) * (W // 2)
    mods = [time_modulation(t, model_w["t1_w"], model_w["t1_b"], model_w["t2_w"], model_w["t2_b"],
                            model_w["m_w"], model_w["m_b"]) for t in taus]          # K x (6, D)
    mod_tok = np.stack([mods[f // group] for f in range(F) for _ in range(per_frame)])[None]   # (1, L, 6, D)
    x = patchify(window, None, model_w["pe_w"], model_w["pe_b"])
    for w in blocks_w:
        x = dit_block(x, mod_tok, ctx, w, heads, grid, 0, qk8=qk8)
    v = patch_scatter(head(x, model_w["hd_w"], model_w["hd_b"]), F, H, W)
    dt_frame = np.repeat(f64(dts), group)[None, None, :, None, None]
    z = window + dt_frame * v
    out = z[:, :, :group]
    new = np.concatenate([z[:, :, group:], f64(noise_in)], axis=2)
    return new, out
