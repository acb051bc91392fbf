/*
 * wan_vae.h -- C ABI of the Wan-VAE decoder (latent -> RGB video) in the same
 * library as wan.h (libwan.so); the status codes are wan.h's WAN_* codes.
 *
 * [P2] hyper.ai summary of the Wan technical report, section "方法" (method),
 * the Wan-VAE paragraphs: a 3D causal VAE that compresses time, height and width
 * by 4, 8 and 8 ([1+T, H, W, 3] <-> [1+T/4, H/8, W/8, C]); 3D causal
 * convolutions; the first frame compressed only in space; RMSNorm in place of
 * GroupNorm so that a feature cache of earlier frames lets a video of any length
 * be decoded chunk by chunk.  The layer list is this library's reading (the
 * pages give none):
 *   conv_in (3x3x3 causal, z_ch -> 4b); two residual blocks of width 4b;
 *   four stages of widths 4b, 4b, 2b, b with n_res residual blocks each (the
 *   first block of a stage takes the previous width, with a 1x1x1 convolution
 *   on its shortcut when the width changes); after stages 0 and 1 a time
 *   doubling (3x1x1 causal convolution to 2C, whose two halves become two
 *   consecutive frames; the video's first frame passes through undoubled) and,
 *   after stages 0, 1 and 2, a space doubling (nearest neighbour, then a 1x3x3
 *   convolution); head: RMSNorm, SiLU, 3x3x3 causal convolution to RGB.
 *   A residual block is RMSNorm -> SiLU -> conv -> RMSNorm -> SiLU -> conv,
 *   plus its input.  RMSNorm: x / sqrt(mean_c x^2 + 1e-6) * gamma.  Causal
 *   convolutions see the two previous frames of their input (zeros before the
 *   video's first frame) and zero spatial padding.
 *
 * Conventions: as in wan.h (caller-owned device memory, 16-byte aligned
 * pointers, validation before any launch, work enqueued on `stream`).
 * Arithmetic: bf16 convolution operands with float32 accumulation, float32
 * RMSNorm, bf16 activations between layers, float32 video.
 */
#ifndef WAN_VAE_H_
#define WAN_VAE_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Decoder shape.  frames, height, width: the latent video (frames >= 1);
 * z_ch: latent channels (1..32, 16 for Wan); base: width unit b (stage widths
 * 4b, 4b, 4b, 2b, b; b a multiple of 32, at most 128); n_res: residual blocks
 * per stage (1..4); chunk: the most latent frames one wan_vae_decode call takes
 * (sizes the workspace).  Limit: 256 * chunk * height * width < 2^31. */
typedef struct wan_vae_shape {
  int frames;
  int height;
  int width;
  int z_ch;
  int base;
  int n_res;
  int chunk;
} wan_vae_shape;

/* One parameter tensor.  kind 0: convolution weight [dims[0] = C_out][dims[1] = k_t]
 * [dims[2] = k_h][dims[3] = k_w][dims[4] = C_in], bf16, at element `offset` of the
 * weight blob; kind 1: its bias (C_out floats) and kind 2: an RMSNorm scale
 * (C floats), at element `offset` of the float blob (a multiple of 64). */
typedef struct wan_vae_param {
  char name[48];
  int kind;
  int dims[5];
  size_t offset;
  size_t count;
} wan_vae_param;

/* Number of parameter tensors (execution order; a convolution's bias follows
 * its weight).  0 and *status set on an invalid shape. */
int wan_vae_param_count(const wan_vae_shape* s, int* status);
/* Description of parameter `index` (0 <= index < count) into *out. */
int wan_vae_param_info(const wan_vae_shape* s, int index, wan_vae_param* out);
/* Elements of the bf16 weight blob (which = 0) or of the float blob (which = 1). */
size_t wan_vae_blob_elems(const wan_vae_shape* s, int which, int* status);

/* Device workspace and feature-cache bytes for shape s (0 and *status on error). */
size_t wan_vae_workspace_bytes(const wan_vae_shape* s, int* status);
size_t wan_vae_cache_bytes(const wan_vae_shape* s, int* status);

/* Decode latent frames [t0, t0 + n) of the video, 1 <= n <= s->chunk,
 * t0 + n <= s->frames.
 *   weights  bf16 weight blob, fparams float blob (wan_vae_param_info layout)
 *   z        (z_ch, n, height, width) float32: this call's latent frames
 *   cache    feature cache (wan_vae_cache_bytes): the decoder state after frames
 *            [0, t0); reset by a call with t0 == 0, updated by every call
 *   video    (3, n_out, 8 height, 8 width) float32 output of this call's frames,
 *            n_out = 4n - 3 when t0 == 0, else 4n
 * Successive calls over consecutive ranges decode the same video as one call
 * over all frames.  Calls sharing a cache must be ordered on one stream. */
int wan_vae_decode(const wan_vae_shape* s, const void* weights, const float* fparams, const float* z, int t0, int n,
                   void* cache, size_t cache_bytes, float* video, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* WAN_VAE_H_ */
