// Internal launchers of the gfx950 kernels (host side).  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wan {

// LOAD_FP8 (T = bf16 output type): A and W are e4m3 bytes with one power-of-two
// scale byte (exponent + 127) per 128-element block along K: A scales at
// a_scale[blk * a_sld + r] for GEMM row r, W scales at w_scale[blk * N + n]
// LOAD_CONV (bf16): implicit GEMM of a convolution over a padded channels-last
// buffer [frames][cv_hp][cv_wp][lda]: row r is output voxel (t, h, w) of a
// (cv_h x cv_w) frame, t = r / (cv_h cv_w); column k = tap * (cv_kpt * 32) + c reads
// A + ((t + cv_t0) * cv_hp + h) * cv_wp + w) * lda + tap_off[tap] + c
enum Loader { LOAD_PLAIN = 0, LOAD_PATCH = 1, LOAD_FP8 = 2, LOAD_CONV = 3 };
// EPI_STORE_GELU8: GELU, then e4m3 bytes at C + r * ldc + n with one scale byte per
// (row, 128-column block) at c_scale[(n / 128) * c_sld + r]
// EPI_CONV (LOAD_CONV): bf16 into a padded channels-last buffer with two leading
// cache frames: voxel (t, h, w), column n -> frame cv_of0 + cv_ofs * t (+1 for
// n >= cv_split, channel n - cv_split), stored at
// C + (((frame + 2) * cv_hp + h + 1) * cv_wp + w + 1) * ldc + channel, plus cv_res
// (same layout) when non-null.  EPI_CONV_VIDEO: float32 video planes
// C[n][cv_of0 + t][h][w] (plane stride ldc) for n < cv_nout.
enum Epi { EPI_STORE = 0, EPI_STORE_GELU = 1, EPI_STORE_F32 = 2, EPI_RESID = 3, EPI_PACK = 4, EPI_PACK8 = 5,
           EPI_STORE_GELU8 = 6, EPI_CONV = 7, EPI_CONV_VIDEO = 8 };

constexpr int CONV_MAX_TAPS = 27;

// C[M][N] = A[M][K] * W[N][K]^T + bias, with an epilogue selected by `epi`.
struct GemmArgs {
  int M = 0, N = 0, K = 0;
  // A operand (LOAD_PLAIN): row r lives at A + (r / a_rpb) * a_bstride + (r % a_rpb) * lda;
  // with a_valid > 0, rows r % a_rpb >= a_valid (padding of a padded row pitch) read row a_valid-1
  const void* A = nullptr;
  long long lda = 0, a_bstride = 0;
  int a_rpb = 1;
  int a_valid = 0;
  // LOAD_FP8 scale bytes (blocks of 128 along K)
  const unsigned char* a_scale = nullptr;
  long long a_sld = 0;
  const unsigned char* w_scale = nullptr;
  // LOAD_CONV / EPI_CONV geometry
  int cv_h = 0, cv_w = 0, cv_hp = 0, cv_wp = 0, cv_t0 = 0, cv_kpt = 1;
  int cv_of0 = 0, cv_ofs = 1, cv_split = 1 << 30, cv_nout = 0;
  const void* cv_res = nullptr;
  long long tap_off[CONV_MAX_TAPS] = {};
  // A operand (LOAD_PATCH): (1,2,2) patches of [z ; cond], token rows of `zb_count` videos
  const float* z = nullptr;
  const float* cond = nullptr;
  int z_batch = 1;          // videos held by z / cond (row batch b reads video b % z_batch)
  int in_ch = 16, F = 1, H = 2, W = 2;
  // weights
  const void* Wt = nullptr;
  long long ldw = 0;
  const float* bias = nullptr;
  // rows of C belong to batch b = r / c_rpb, token t = r % c_rpb; with c_valid > 0
  // (EPI_PACK*, EPI_RESID) tokens t >= c_valid are padding and not stored
  int c_rpb = 1;
  int c_valid = 0;
  // EPI_STORE*: C + r * ldc + n
  void* C = nullptr;
  long long ldc = 0;
  unsigned char* c_scale = nullptr;  // EPI_STORE_GELU8
  long long c_sld = 0;
  // EPI_RESID: x[xr * ldx + n] += gate[b * gate_bstride + n] * (acc + bias); gate NULL -> 1;
  // xr = r, or b * c_valid + t when c_valid > 0
  float* x = nullptr;
  long long ldx = 0;
  const float* gate = nullptr;
  long long gate_bstride = 0;
  // EPI_PACK: columns [0, nq) -> q, [nq, nq+nk) -> k, rest -> v^T; all head-major.
  // EPI_PACK8 (bf16, hd == 128): q and k as e4m3 bytes [B][H][Lp][hd] plus one
  // scale byte per (batch, head, token) in qs / ks [B][H][Lp]; v^T as EPI_PACK
  void* q = nullptr;
  void* k = nullptr;
  void* vt = nullptr;
  unsigned char* qs = nullptr;
  unsigned char* ks = nullptr;
  int nq = 0, nk = 0;
  int heads = 1, hd = 128, Lp = 64;
  const float2* rope = nullptr;  // per-token (cos, sin) table [token][hd/2], or NULL for no rotation
  // EPI_PACK / EPI_PACK8 with 128-wide heads: when set, every wave of a k-section tile writes the largest
  // |k|^2 of the stored k rows it handled to kpart[(b * heads + h) * kpart_n + tile * waves + wave]
  // (tile = the 256-row tile's index inside batch item b; kpart_n = tiles per item x waves)
  float* kpart = nullptr;
  int kpart_n = 0;
  float q_scale = 1.0f;  // EPI_PACK / EPI_PACK8: the q section is multiplied by this after RoPE
};

template <typename T> hipError_t launch_gemm(const GemmArgs& g, int loader, int epi, hipStream_t st);

// Flash attention over head-major q [B][H][Lqp][hd], k [B][H][Lkp][hd],
// v^T [B][H][hd][Lkp] (keys permuted inside each 16-key group), one or two
// key/value sources summed after their own softmax.  Output o (B, Lq, H*hd).
struct AttnArgs {
  const void* q = nullptr;
  int Lq = 0, Lqp = 0;
  const void* k[2] = {nullptr, nullptr};
  const void* vt[2] = {nullptr, nullptr};
  int Lk[2] = {0, 0}, Lkp[2] = {0, 0};
  int nsrc = 1;
  int self = 0;  // 1: self-attention (selects the kernel symbol; the computation is the same)
  // qk8 (bf16, self, hd == 128): q and k are e4m3 bytes with per-row scale bytes qs [B][H][Lqp]
  // and ks [B][H][Lkp] (power-of-two exponent + 127), as EPI_PACK8 writes them
  int qk8 = 0;
  const unsigned char* qs = nullptr;
  const unsigned char* ks = nullptr;
  void* o = nullptr;
  int B = 1, heads = 1, hd = 128;
  float scale_log2 = 0.f;
  // bf16 self-attention with 256-query workgroups: with kpart ([B][heads][kpart_n] partial
  // maxima of |k|^2 over the keys, as the QKV epilogue writes them) and fallback
  // ([attn_wide_flags] ints, any contents) the probabilities take the static offset
  // |q| max|k| (no running maximum); the workgroups that flag an under-flowing row are then
  // recomputed with the running maximum.  The bf16 kernel takes this path with q already
  // multiplied by log2(e)/sqrt(hd) and scale_log2 == 1; the 8-bit-score kernel with q as
  // projected and scale_log2 == log2(e)/sqrt(hd)
  const float* kpart = nullptr;
  int kpart_n = 0;
  int* fallback = nullptr;
  const int* only = nullptr;  // set internally: run only the workgroups flagged here
};
template <typename T> hipError_t launch_attention(const AttnArgs& a, hipStream_t st);
// whether launch_attention takes a 256-query (static-offset capable) self-attention path: the
// bf16 kernel at full length, or the 8-bit-score kernel
bool attn_static_offset_path(int hd, int Lq, int heads, int B, bool bf16, bool qk8);
int attn_wide_flags(int Lq, int heads, int B);

// out[r] = T( LN(x[r]) * (1 + scale[b]) + shift[b] ), rows of length D; shift/scale NULL -> plain LN
template <typename T>
hipError_t launch_ln_mod(const float* x, void* out, int rows, int D, int rows_per_batch, const float* shift,
                         const float* scale, long long mod_bstride, hipStream_t st);

// As launch_ln_mod, with e4m3 output bytes out8 [rows][D] and one scale byte per
// (row, 128-column block) at sc[(col / 128) * sc_ld + b * pitch + t], row = b * rows_per_batch + t
hipError_t launch_ln_mod8(const float* x, unsigned char* out8, unsigned char* sc, long long sc_ld, int pitch, int rows,
                          int D, int rows_per_batch, const float* shift, const float* scale, long long mod_bstride,
                          hipStream_t st);

// bf16 weights W [N][K] -> e4m3 bytes W8 [N][K] and scale bytes sc [K/128][N] (blocks of 128 along K)
hipError_t launch_quant_weights(const void* W, unsigned char* W8, unsigned char* sc, int N, int K, hipStream_t st);

// (cos, sin) RoPE table for head dim hd over grid (F, Hh, Ww), computed in double: the
// frame segment, then the row and column segments, one entry per (position, pair).
hipError_t launch_rope_table(float2* tab, int hd, int F, int Hh, int Ww, hipStream_t st);
// Per-token table [F*Hh*Ww][hd/2] gathered from the segment table above.
hipError_t launch_rope_tokens(float2* tok, const float2* tab, int hd, int F, int Hh, int Ww, hipStream_t st);

// zero the key padding [L, Lp) of a v^T buffer [BH][hd][Lp]
template <typename T> hipError_t launch_zero_vt_pad(void* vt, int BH, int hd, int L, int Lp, hipStream_t st);

// y[n] = sum_k W[n][k] * act(x[k]) + b[n]; act = SiLU when silu_in, x float32 of length K.
// When x is NULL the input is the 256-wide timestep sinusoid of `tau` (computed in double).
template <typename T>
hipError_t launch_gemv(const void* Wt, const float* bias, const float* x, float tau, float* y, int N, int K,
                       int silu_in, hipStream_t st);

// Unpatchify the head output p (rows of out_ch*4) and either store it (dt == 0 && !step)
// or apply guidance + Euler to z.  With `step`, p rows [0, B*L) are the conditional
// branch and p_null (default: p rows [B*L, 2*B*L)) the unconditional one.
hipError_t launch_unpatch(const float* p, float* out, int B, int C, int F, int H, int W, int step, float dt,
                          float guide, hipStream_t st, const float* p_null = nullptr);

// Wan-VAE decoder helpers over padded channels-last bf16 frame buffers
// [2 + frames][H + 2][W + 2][Cs] (two leading cache frames, one-voxel zero border)
hipError_t launch_vae_latent(const float* z, void* buf, int zc, int n, int H, int W, int Cs, hipStream_t st);
hipError_t launch_vae_rms_silu(const void* in, void* out, const float* g, int C, int Cs, int n, int H, int W,
                               hipStream_t st);
hipError_t launch_vae_up_space(const void* in, void* out, int n, int H, int W, int Cs, hipStream_t st);
hipError_t launch_vae_border(void* buf, int frames, int Hp, int Wp, int Cs, hipStream_t st);
hipError_t launch_vae_pad_weight(const void* W, const float* b, void* Wp, float* bp, int Cout, int N, int taps, int Cin,
                                 int Cink, hipStream_t st);

// Streaming denoise queue: z (C, F = K * group, H, W) += dts[f / group] * v (v from the head
// rows p); frames [0, group) -> out (C, group, H, W); the rest shifted down by group into nz,
// whose last group frames are `noise`.  dts is a host array of K <= STREAM_MAX_SLOTS values.
constexpr int STREAM_MAX_SLOTS = 64;
hipError_t launch_stream_update(const float* p, const float* z, const float* noise, float* nz, float* out, int C,
                                int F, int H, int W, int group, const float* dts, int K, hipStream_t st);

// copy helper (device to device, on the stream)
hipError_t copy_async(void* dst, const void* src, size_t bytes, hipStream_t st);

}  // namespace wan
