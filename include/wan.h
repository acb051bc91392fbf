/*
 * wan.h -- C ABI of the MI355X (gfx950) Wan2.1 DiT block and denoise-step library.
 *
 * The library computes the forward pass of a Wan2.1 diffusion-transformer (DiT)
 * block over the patchified spatio-temporal latent, and one classifier-free
 * guided flow-matching Euler step built from such blocks, as described in:
 *   [P2] hyper.ai summary of the Wan technical report (arXiv 2503.20314),
 *        section "方法" (method);
 *   [P3] zizhi168.cn, "阿里Wan 2.1视频生成模型深度剖析", section "核心代码实现亮点";
 *   [P1] CSDN, "wan2.1 论文精读二 | 模型设计与加速", sections 1.1 and 5;
 *   [P4] kwkr.cn, "Wan2.1视频生成模型实战：单流DiT与Flow Matching架构解析", section 4.4.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every tensor pointer is DEVICE memory owned by the caller.  The library
 *   never allocates, frees or keeps a pointer after a call returns.  Every
 *   tensor pointer must be 16-byte aligned.
 * - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL = the
 *   null stream) and the call returns without synchronising.  Faults of the
 *   enqueued kernels surface at the caller's next synchronisation.
 * - Apart from a one-time device check and kernel attribute setup on the first
 *   call on a device, a call enqueues only kernel launches and device-to-device
 *   copies (and, while the measurement hook is enabled, its event pairs): once
 *   an entry point has run eagerly it can be captured into a HIP graph, which
 *   replays it with the scalars of the capture (timestep, step size, guide
 *   scale).
 * - Every argument is validated before anything is enqueued; a call that
 *   returns an error has no side effect.
 * - Weight matrices use the Linear layout [out][in], row-major, in the mode's
 *   element type (bf16 in WAN_BF16 mode, float in WAN_FP32 mode).  Biases are
 *   always float32.  The residual stream x, the latent z, the condition
 *   channels and the modulation are always float32.  Context tokens use the
 *   mode's element type.
 * - Results are bitwise reproducible run to run (no floating-point atomics).
 * - Calls that use distinct workspaces and outputs may run concurrently.
 */
#ifndef WAN_H_
#define WAN_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define WAN_OK 0
#define WAN_E_NULL (-1)      /* a required pointer is NULL */
#define WAN_E_SHAPE (-2)     /* unsupported or inconsistent shape */
#define WAN_E_MODE (-3)      /* unknown precision mode */
#define WAN_E_ALIGN (-4)     /* a pointer is not 16-byte aligned */
#define WAN_E_WORKSPACE (-5) /* workspace missing or smaller than wan_workspace_bytes() */
#define WAN_E_HIP (-6)       /* no usable gfx950 device, or a launch failed */
#define WAN_E_ENTRY (-7)     /* unknown entry id passed to wan_workspace_bytes */
#define WAN_E_SCRATCH (-8)   /* the shape needs more than WAN_NOALLOC_SCRATCH_BYTES of scratch */

/* precision modes */
#define WAN_BF16 0 /* bf16 GEMM/attention operands, float32 accumulation */
#define WAN_FP32 1 /* float32 everywhere */
/* As WAN_BF16 (same weights, context and workspace sizes), except that every
 * self-attention takes its scores from q and k in 8-bit form ([P2] method:
 * inference runs FP8 GEMMs and an 8-bit FlashAttention; which operands go to
 * 8 bits and how they are scaled is this library's reading): each
 * (token, head) row of q and of k (after RoPE) is given the power-of-two scale
 * 2^e with the smallest e (clamped to [-127, 127]) that brings its largest
 * magnitude to 448 or below, and is rounded to the nearest float8 e4m3 value
 * (ties to even) in that scale; q k^T is then taken from the rounded rows.  The
 * probabilities and v stay bf16, cross-attention is unchanged.  Needs
 * dim / heads == 128 (WAN_E_SHAPE otherwise). */
#define WAN_BF16_QK8 2
/* As WAN_BF16_QK8, and the q/k/v projection, the cross-attention query
 * projection and both FFN projections are 8-bit GEMMs ([P2] method: FP8 GEMMs
 * at inference; the scaling rule is this library's reading): both operands
 * are cut into blocks of 128 consecutive elements along the contraction axis
 * (per token for the activation, per output feature for the weight), each
 * block gets the power-of-two scale and e4m3 rounding of WAN_BF16_QK8, and the
 * products accumulate in float32.  The weights stay bf16 at the interface and
 * are quantised inside each call.  The self- and cross-attention output
 * projections and the context K / V projections stay bf16.  Needs
 * dim / heads == 128 (WAN_E_SHAPE otherwise); the workspace is larger than in
 * bf16 mode (wan_workspace_bytes). */
#define WAN_FP8 3

/* entry ids for wan_workspace_bytes */
#define WAN_ENTRY_PATCHIFY 0
#define WAN_ENTRY_BLOCK 1
#define WAN_ENTRY_STEP 2
#define WAN_ENTRY_TIME_EMBED 3
#define WAN_ENTRY_HEAD 4

/*
 * Problem shape.  The latent is (batch, 16, frames, height, width) with even
 * height and width; the (1,2,2) patchify ([P2] method) makes
 * L = frames * (height/2) * (width/2) tokens of width `dim`.
 *   in_ch    16 (text-to-video) or 36 (image-to-video: 16 noisy + 4 mask +
 *            16 condition-latent channels, [P1] 1.1)
 *   out_ch   16 (the velocity has the latent's channels)
 *   heads    dim / heads must be 64 or 128
 *   ffn_dim  FFN hidden width
 *   txt_len  text tokens (>= 1); img_len image tokens (0 unless in_ch == 36
 *            is wanted with decoupled image cross-attention, [P1] 1.1 / [P3])
 * Limits: dim % 256 == 0, ffn_dim % 256 == 0, 1 <= L, ctx lengths <= 65536.
 */
typedef struct wan_shape {
  int batch;
  int in_ch;
  int out_ch;
  int frames;
  int height;
  int width;
  int dim;
  int heads;
  int ffn_dim;
  int txt_len;
  int img_len;
  int mode;
} wan_shape;

/* Device pointers of one block's weights (a host struct).  Shapes with D = dim,
 * F = ffn_dim: qkv_w [3D][D] (rows ordered q, k, v), o_w [D][D], cq_w [D][D],
 * ckv_w [2D][D] (rows k then v, text tokens), ikv_w [2D][D] (image tokens;
 * NULL when img_len == 0), co_w [D][D], ff1_w [F][D], ff2_w [D][F];
 * each *_b is the float32 bias of its matrix's output width. */
typedef struct wan_block_weights {
  const void* qkv_w; const float* qkv_b;
  const void* o_w;   const float* o_b;
  const void* cq_w;  const float* cq_b;
  const void* ckv_w; const float* ckv_b;
  const void* ikv_w; const float* ikv_b;
  const void* co_w;  const float* co_b;
  const void* ff1_w; const float* ff1_b;
  const void* ff2_w; const float* ff2_b;
} wan_block_weights;

/* Device pointers of the model-level weights plus a HOST array of blocks.
 * pe_w [D][in_ch*4] (the (D, in_ch, 1, 2, 2) patch convolution flattened),
 * t1_w [D][256], t2_w [D][D], m_w [6D][D], hd_w [out_ch*4][D]. */
typedef struct wan_model_weights {
  const void* pe_w; const float* pe_b;
  const void* t1_w; const float* t1_b;
  const void* t2_w; const float* t2_b;
  const void* m_w;  const float* m_b;
  const void* hd_w; const float* hd_b;
  int n_blocks;
  const wan_block_weights* blocks;
} wan_model_weights;

/* Human-readable text of a status code (static storage). */
const char* wan_status_str(int code);

/* Bytes of device workspace the entry `entry` (WAN_ENTRY_*) needs for shape
 * `s`; 0 when the entry needs none.  Pure host function.  Returns 0 and sets
 * *status (if non-NULL) to a negative code when the shape is invalid. */
size_t wan_workspace_bytes(const wan_shape* s, int entry, int* status);

/*
 * Patch embedding ([P2] method: 3D convolution with kernel (1,2,2) giving a
 * (B, L, D) sequence).
 *   z     (B, 16, F, H, W) float32
 *   cond  (B, in_ch - 16, F, H, W) float32 = [mask ; z_c], or NULL when in_ch == 16
 *   x     out: (B, L, D) float32, token l = (f*(H/2) + i)*(W/2) + j
 * Patch feature k = c*4 + a*2 + b holds channel c at (2i+a, 2j+b).
 */
int wan_patchify(const wan_shape* s, const float* z, const float* cond, const void* pe_w,
                 const float* pe_b, float* x, void* ws, size_t ws_bytes, void* stream);

/*
 * Time modulation ([P2] method: an MLP of Linear and SiLU layers on the time
 * embedding predicts six modulation parameters, shared by every block):
 *   s = [cos(tau w_k) ; sin(tau w_k)], w_k = 10000^(-k/128), k < 128
 *   e = t2_w SiLU(t1_w s + t1_b) + t2_b;  mod = m_w SiLU(e) + m_b
 *   mod  out: (6, D) float32, rows (shift1, scale1, gate1, shift2, scale2, gate2)
 */
int wan_time_embed(const wan_shape* s, const wan_model_weights* w, float timestep, float* mod,
                   void* ws, size_t ws_bytes, void* stream);

/*
 * One DiT block, in place on the float32 residual stream x (B, L, D):
 *   x += g1 * SelfAttn(RoPE; LN(x)(1+sc1)+sh1)        [P2] method, [P3] core code
 *   x += CrossAttn(LN(x), ctx)                          [P2] method, [P1] 1.1 / [P3]
 *   x += g2 * FFN_GELU(LN(x)(1+sc2)+sh2)
 * LN has eps 1e-6 and no affine.  mod is (B, 6, D) float32; mod_batch_stride
 * is the element stride between batch items (6*D, or 0 to share one (6, D)).
 * ctx is (B, img_len + txt_len, D) in the mode's type, image tokens first; the
 * image tokens use their own K/V projection and softmax and the two attention
 * results are summed before the shared output projection.
 */
int wan_dit_block_forward(const wan_shape* s, const wan_block_weights* w, float* x,
                          const float* mod, long long mod_batch_stride, const void* ctx,
                          void* ws, size_t ws_bytes, void* stream);

/*
 * wan_dit_block_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, kernels and results as
 * wan_dit_block_forward, except that the workspace is a fixed device array
 * of WAN_NOALLOC_SCRATCH_BYTES inside the library (one copy per GPU, held
 * from the library's load until the process ends).  The call allocates and
 * frees nothing.
 *   Returns WAN_E_SCRATCH when wan_workspace_bytes(s, WAN_ENTRY_BLOCK, ...)
 *   exceeds WAN_NOALLOC_SCRATCH_BYTES (checked before anything is enqueued);
 *   otherwise as wan_dit_block_forward.
 * Every call on one GPU uses that GPU's single array, which keeps what the
 * last call left in it; no result depends on those contents (the block
 * overwrites every value it uses), so nothing needs clearing between calls.
 * Calls that may overlap on one GPU (other host threads, or concurrent
 * streams) race on the array and must be serialised by the caller.
 */
#define WAN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int wan_dit_block_forward_noalloc(const wan_shape* s, const wan_block_weights* w, float* x, const float* mod,
                                  long long mod_batch_stride, const void* ctx, void* stream);

/*
 * Output head: per token LN(x) (no affine) then Linear D -> out_ch*4, and the
 * inverse of the patch permutation ([P2] method, unpatchify module).
 *   x  (B, L, D) float32;  v out: (B, out_ch, F, H, W) float32
 */
int wan_head(const wan_shape* s, const wan_model_weights* w, const float* x, float* v,
             void* ws, size_t ws_bytes, void* stream);

/*
 * One classifier-free-guided flow-matching Euler step, in place on z:
 *   v_c = DiT(z, ctx_cond), v_u = DiT(z, ctx_null)         (batched as 2B)
 *   z  += dt * (v_u + guide_scale * (v_c - v_u))          [P3] core code, [P4] 4.4
 * DiT = patchify, time modulation at `timestep`, n_blocks blocks, head.
 *   z (B, 16, F, H, W) float32 in/out; cond as in wan_patchify;
 *   ctx_cond, ctx_null (B, img_len + txt_len, D) in the mode's type.
 */
int wan_denoise_step(const wan_shape* s, const wan_model_weights* w, float* z, const float* cond,
                     const void* ctx_cond, const void* ctx_null, float timestep, float dt,
                     float guide_scale, void* ws, size_t ws_bytes, void* stream);

/*
 * Diffusion cache ([P2] method: inference exploits the similarity of attention
 * between sampling steps and of the two CFG branches; [P2] experiments: 1.62x).
 * One step as wan_denoise_step, under one of these modes:
 *   WAN_CACHE_STORE         the full step; also writes every block's self-attention
 *                           output of both branches (before the output projection)
 *                           and the unconditional head output into `cache`;
 *   WAN_CACHE_REUSE_ATTN    every block takes its self-attention output from the
 *                           cache: the q/k/v projection and the attention are skipped;
 *   WAN_CACHE_REUSE_UNCOND  only the conditional branch runs (batch B instead of 2B);
 *                           the unconditional head output comes from the cache.
 * The two REUSE flags combine.  A REUSE step reads what the last STORE step on
 * the same shape and cache wrote; the cache is not checked for that (a REUSE
 * step on a cache no STORE step has filled reads undefined values).
 * cache: caller-owned device memory of wan_cache_bytes(s) bytes, laid out as
 *   n_blocks x (2B, L, D) attention outputs in the mode's type (conditional
 *   batch items first), then (B, L, out_ch*4) float32 unconditional head output.
 * Returns WAN_E_MODE for any other mode value, WAN_E_WORKSPACE when cache_bytes
 * is below wan_cache_bytes(s); otherwise as wan_denoise_step.
 */
#define WAN_CACHE_STORE 1
#define WAN_CACHE_REUSE_ATTN 2
#define WAN_CACHE_REUSE_UNCOND 4
size_t wan_cache_bytes(const wan_shape* s, int n_blocks, int* status);
int wan_denoise_step_cached(const wan_shape* s, const wan_model_weights* w, float* z, const float* cond,
                            const void* ctx_cond, const void* ctx_null, float timestep, float dt,
                            float guide_scale, int cache_mode, void* cache, size_t cache_bytes,
                            void* ws, size_t ws_bytes, void* stream);

/*
 * Kernel timing (measurement support, not part of the computation).
 * While enabled, the library brackets every launch of the kernel classes below
 * with a pair of hipEvents recorded on the launch stream.  wan_timing_read
 * waits for the recorded events, returns the summed elapsed milliseconds and
 * the launch count of one class since the last reset, and with reset != 0
 * clears that class.  Enabling adds two event records per launch.
 */
/* Streaming denoise queue ([P1] 6.2 Streamer: a sliding temporal window
 * generates videos of any length; 6.3: a distilled consistency model folds the
 * guidance into the model and needs four sampling steps per frame).  Reading
 * taken: the latent window (1, 16, frames, height, width) holds K = frames / group
 * slots of `group` latent frames, slot 0 the oldest.  One tick runs the DiT once
 * over the whole window with the conditional context only (no guidance), every
 * token modulated with its slot's time modulation at timestep taus[k]; each
 * slot's frames then take an Euler step of dts[k] along the predicted
 * velocity.  The first slot's updated frames are written to frames_out
 * (1, 16, group, height, width); the window shifts down by one slot (in place)
 * and noise_in (1, 16, group, height, width) becomes its newest slot.
 * taus and dts are HOST arrays of K floats.  Shape: batch 1, in_ch 16,
 * img_len 0, 1 <= K <= 64; mode WAN_BF16, WAN_FP32 or WAN_BF16_QK8
 * (WAN_E_MODE for WAN_FP8).  RoPE positions are window positions. */
size_t wan_stream_workspace_bytes(const wan_shape* s, int group, int* status);
int wan_stream_tick(const wan_shape* s, const wan_model_weights* w, float* window, const void* ctx, const float* taus,
                    const float* dts, int group, const float* noise_in, float* frames_out, void* ws, size_t ws_bytes,
                    void* stream);

#define WAN_KERNEL_SELF_ATTENTION 0
#define WAN_KERNEL_CROSS_ATTENTION 1
#define WAN_KERNEL_GEMM 2
#define WAN_KERNEL_ELEMENTWISE 3
int wan_timing_enable(int on);
int wan_timing_read(int kernel_class, double* ms_total, long long* launches, int reset);

#ifdef __cplusplus
}
#endif

#endif /* WAN_H_ */
