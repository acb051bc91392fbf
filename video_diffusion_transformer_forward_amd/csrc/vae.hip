// Wan-VAE decoder kernels for gfx950 (the convolutions run on the GEMM kernel
// with its convolution loader): latent intake, RMSNorm + SiLU, nearest-neighbour
// space doubling, border clearing and weight padding.
//
// Activations are channels-last bf16 in padded frame buffers
// [2 + frames][H + 2][W + 2][Cs]: two leading frames hold the causal
// convolution's previous frames (the feature cache, or zeros), a one-voxel zero
// border gives the 3x3 spatial taps their padding, and the channel stride Cs is
// a multiple of 32 (channels past the true width C are never read as data).
#include "common.h"
#include "kernels.h"

namespace wan {

namespace {

constexpr float VAE_RMS_EPS = 1e-6f;

__device__ __forceinline__ long long vox_off(int t, int h, int w, int Hp, int Wp, int Cs) {
  return (((long long)(t + 2) * Hp + h + 1) * Wp + w + 1) * Cs;
}

// latent (zc, n, H, W) float32 -> frames 2.. of buf, channels zc..Cs-1 zero
__global__ __launch_bounds__(256) void vae_latent_kernel(const float* __restrict__ z, bf16* __restrict__ buf, int zc,
                                                         int n, int H, int W, int Cs) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long total = (long long)n * H * W * Cs;
  if (i >= total) return;
  const int c = (int)(i % Cs);
  const long long v = i / Cs;
  const int w = (int)(v % W);
  const int h = (int)((v / W) % H);
  const int t = (int)(v / ((long long)W * H));
  const float x = c < zc ? z[(((long long)c * n + t) * H + h) * W + w] : 0.f;
  buf[vox_off(t, h, w, H + 2, W + 2, Cs) + c] = to_bf16(x);
}

// y = SiLU(x / sqrt(mean_c x^2 + eps) * g) over the C channels of every voxel;
// G lanes per voxel, 8 channels per lane
template <int G>
__global__ __launch_bounds__(256) void vae_rms_silu_kernel(const bf16* __restrict__ in, bf16* __restrict__ out,
                                                           const float* __restrict__ g, int C, int Cs, int n, int H,
                                                           int W) {
  const long long vox = (long long)blockIdx.x * (256 / G) + threadIdx.x / G;
  const int lg = threadIdx.x % G;
  if (vox >= (long long)n * H * W) return;  // a whole group of G lanes leaves together
  const int w = (int)(vox % W);
  const int h = (int)((vox / W) % H);
  const int t = (int)(vox / ((long long)W * H));
  const long long off = vox_off(t, h, w, H + 2, W + 2, Cs);
  const int c0 = lg * 8;
  const bool act = c0 < C;
  float x[8];
  if (act) {
    Chunk<bf16> c;
    c.load(in + off + c0);
    const bf16x8 v = as_bf16x8(c.v);
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = (float)v[u];
  } else {
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = 0.f;
  }
  float ss = 0.f;
#pragma unroll
  for (int u = 0; u < 8; ++u) ss += x[u] * x[u];
#pragma unroll
  for (int o = 1; o < G; o <<= 1) ss += __shfl_xor(ss, o, 64);
  const float inv = 1.0f / sqrtf(ss / C + VAE_RMS_EPS);
  if (act) {
    const float4 g0 = *reinterpret_cast<const float4*>(g + c0);
    const float4 g1 = *reinterpret_cast<const float4*>(g + c0 + 4);
    const float gg[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    // SiLU as r / (1 + 2^(-r log2 e)) with the hardware exp2 and reciprocal (about
    // 1 ulp each, far below the bf16 rounding of the result); r -> -inf gives -0
    float y[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float r = x[u] * inv * gg[u];
      y[u] = r * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(r * -1.4426950408889634f));
    }
    Chunk<bf16> c;
    pack8(c, y);
    c.store(out + off + c0);
  }
}

// The same for widths C = 24 G (96, 192 and 384 here): G lanes per voxel with three 8-channel
// chunks each (chunk j G + lane, so no lane idles and a wave's loads stay contiguous), and
// V voxels per lane group whose loads all go out before any arithmetic: one 16-byte load
// per lane left too few bytes in flight per CU to cover the memory latency.
template <int G, int V>
__global__ __launch_bounds__(256) void vae_rms_silu24_kernel(const bf16* __restrict__ in, bf16* __restrict__ out,
                                                             const float* __restrict__ g, int Cs, int n, int H,
                                                             int W) {
  constexpr int NC = 3, C = 24 * G;
  const long long nvox = (long long)n * H * W;
  const long long v0 = ((long long)blockIdx.x * (256 / G) + threadIdx.x / G) * V;
  const int lg = threadIdx.x % G;
  if (v0 >= nvox) return;  // a whole group of G lanes leaves together
  long long off[V];
  Chunk<bf16> raw[V][NC];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const long long vox = v0 + v < nvox ? v0 + v : nvox - 1;
    const int w = (int)(vox % W);
    const int h = (int)((vox / W) % H);
    const int t = (int)(vox / ((long long)W * H));
    off[v] = vox_off(t, h, w, H + 2, W + 2, Cs);
#pragma unroll
    for (int j = 0; j < NC; ++j) raw[v][j].load(in + off[v] + (j * G + lg) * 8);
  }
  float gg[NC][8];
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const float4 g0 = *reinterpret_cast<const float4*>(g + (j * G + lg) * 8);
    const float4 g1 = *reinterpret_cast<const float4*>(g + (j * G + lg) * 8 + 4);
    gg[j][0] = g0.x; gg[j][1] = g0.y; gg[j][2] = g0.z; gg[j][3] = g0.w;
    gg[j][4] = g1.x; gg[j][5] = g1.y; gg[j][6] = g1.z; gg[j][7] = g1.w;
  }
#pragma unroll
  for (int v = 0; v < V; ++v) {
    float x[NC][8];
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const bf16x8 b = as_bf16x8(raw[v][j].v);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        x[j][u] = (float)b[u];
        ss += x[j][u] * x[j][u];
      }
    }
#pragma unroll
    for (int o = 1; o < G; o <<= 1) ss += __shfl_xor(ss, o, 64);
    const float inv = 1.0f / sqrtf(ss / C + VAE_RMS_EPS);
    if (v0 + v < nvox) {
#pragma unroll
      for (int j = 0; j < NC; ++j) {
        float y[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float r = x[j][u] * inv * gg[j][u];
          y[u] = r * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(r * -1.4426950408889634f));
        }
        Chunk<bf16> c;
        pack8(c, y);
        c.store(out + off[v] + (j * G + lg) * 8);
      }
    }
  }
}

// out (2H x 2W) frame t = nearest doubling of in (H x W) frame t, 16-byte chunks
__global__ __launch_bounds__(256) void vae_up_space_kernel(const bf16* __restrict__ in, bf16* __restrict__ out, int n,
                                                           int H, int W, int Cs) {
  // one input chunk per lane, written to its 2 x 2 output voxels (each input byte read once)
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  const int cpv = Cs / 8;
  const long long total = (long long)n * H * W * cpv;
  if (i >= total) return;
  const int c8 = (int)(i % cpv) * 8;
  const long long v = i / cpv;
  const int w = (int)(v % W);
  const int h = (int)((v / W) % H);
  const int t = (int)(v / ((long long)W * H));
  Chunk<bf16> c;
  c.load(in + vox_off(t, h, w, H + 2, W + 2, Cs) + c8);
#pragma unroll
  for (int dh = 0; dh < 2; ++dh) {
    bf16* o = out + vox_off(t, 2 * h + dh, 2 * w, 2 * H + 2, 2 * W + 2, Cs) + c8;
    c.store(o);
    c.store(o + Cs);
  }
}

// zero the one-voxel spatial border of frames [0, frames) of a padded buffer
__global__ __launch_bounds__(256) void vae_border_kernel(bf16* __restrict__ buf, int frames, int Hp, int Wp, int Cs) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  const int cpv = Cs / 8;
  const int per_frame = 2 * Wp + 2 * (Hp - 2);  // border voxels of a frame
  const long long total = (long long)frames * per_frame * cpv;
  if (i >= total) return;
  const int c8 = (int)(i % cpv) * 8;
  const long long v = i / cpv;
  const int f = (int)(v / per_frame);
  const int b = (int)(v % per_frame);
  int h, w;
  if (b < Wp) {
    h = 0;
    w = b;
  } else if (b < 2 * Wp) {
    h = Hp - 1;
    w = b - Wp;
  } else {
    const int k = b - 2 * Wp;
    h = 1 + k / 2;
    w = (k & 1) ? Wp - 1 : 0;
  }
  Chunk<bf16> z;
  z.zero();
  z.store(buf + (((long long)f * Hp + h) * Wp + w) * Cs + c8);
}

// W [Cout][taps][Cin] -> Wp [N][taps][Cink] and bias -> bias_p [N], zero-filled
__global__ __launch_bounds__(256) void vae_pad_weight_kernel(const bf16* __restrict__ W, const float* __restrict__ b,
                                                             bf16* __restrict__ Wp, float* __restrict__ bp, int Cout,
                                                             int N, int taps, int Cin, int Cink) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long total = (long long)N * taps * Cink;
  if (i < N) bp[i] = i < Cout ? b[i] : 0.f;
  if (i >= total) return;
  const int c = (int)(i % Cink);
  const long long r = i / Cink;
  const int tap = (int)(r % taps);
  const int o = (int)(r / taps);
  Wp[i] = (o < Cout && c < Cin) ? W[((long long)o * taps + tap) * Cin + c] : to_bf16(0.f);
}

unsigned blocks_for(long long n) { return (unsigned)((n + 255) / 256); }

}  // namespace

hipError_t launch_vae_latent(const float* z, void* buf, int zc, int n, int H, int W, int Cs, hipStream_t st) {
  const long long total = (long long)n * H * W * Cs;
  if (total <= 0) return hipSuccess;
  if (zc > Cs) return hipErrorInvalidValue;
  hipLaunchKernelGGL(vae_latent_kernel, dim3(blocks_for(total)), dim3(256), 0, st, z, reinterpret_cast<bf16*>(buf), zc,
                     n, H, W, Cs);
  return hipGetLastError();
}

hipError_t launch_vae_rms_silu(const void* in, void* out, const float* g, int C, int Cs, int n, int H, int W,
                               hipStream_t st) {
  const long long vox = (long long)n * H * W;
  if (vox <= 0) return hipSuccess;
  if (C % 8 != 0 || C > Cs || C > 512) return hipErrorInvalidValue;
  const bf16* i = reinterpret_cast<const bf16*>(in);
  bf16* o = reinterpret_cast<bf16*>(out);
  constexpr int V = 4;  // voxels per lane group
  const long long groups = (vox + V - 1) / V;
  if (C == 96)
    hipLaunchKernelGGL((vae_rms_silu24_kernel<4, V>), dim3(blocks_for(groups * 4)), dim3(256), 0, st, i, o, g, Cs, n, H, W);
  else if (C == 192)
    hipLaunchKernelGGL((vae_rms_silu24_kernel<8, V>), dim3(blocks_for(groups * 8)), dim3(256), 0, st, i, o, g, Cs, n, H, W);
  else if (C == 384)
    hipLaunchKernelGGL((vae_rms_silu24_kernel<16, V>), dim3(blocks_for(groups * 16)), dim3(256), 0, st, i, o, g, Cs, n, H, W);
  else if (C <= 128)
    hipLaunchKernelGGL(vae_rms_silu_kernel<16>, dim3(blocks_for(vox * 16)), dim3(256), 0, st, i, o, g, C, Cs, n, H, W);
  else if (C <= 256)
    hipLaunchKernelGGL(vae_rms_silu_kernel<32>, dim3(blocks_for(vox * 32)), dim3(256), 0, st, i, o, g, C, Cs, n, H, W);
  else
    hipLaunchKernelGGL(vae_rms_silu_kernel<64>, dim3(blocks_for(vox * 64)), dim3(256), 0, st, i, o, g, C, Cs, n, H, W);
  return hipGetLastError();
}

hipError_t launch_vae_up_space(const void* in, void* out, int n, int H, int W, int Cs, hipStream_t st) {
  const long long total = (long long)n * H * W * (Cs / 8);
  if (total <= 0) return hipSuccess;
  if (Cs % 8 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(vae_up_space_kernel, dim3(blocks_for(total)), dim3(256), 0, st, reinterpret_cast<const bf16*>(in),
                     reinterpret_cast<bf16*>(out), n, H, W, Cs);
  return hipGetLastError();
}

hipError_t launch_vae_border(void* buf, int frames, int Hp, int Wp, int Cs, hipStream_t st) {
  const long long total = (long long)frames * (2 * Wp + 2 * (Hp - 2)) * (Cs / 8);
  if (total <= 0) return hipSuccess;
  if (Cs % 8 != 0 || Hp < 3 || Wp < 3) return hipErrorInvalidValue;
  hipLaunchKernelGGL(vae_border_kernel, dim3(blocks_for(total)), dim3(256), 0, st, reinterpret_cast<bf16*>(buf),
                     frames, Hp, Wp, Cs);
  return hipGetLastError();
}

hipError_t launch_vae_pad_weight(const void* W, const float* b, void* Wp, float* bp, int Cout, int N, int taps, int Cin,
                                 int Cink, hipStream_t st) {
  const long long total = (long long)N * taps * Cink;
  if (total <= 0 || N < Cout || Cink < Cin) return hipErrorInvalidValue;
  hipLaunchKernelGGL(vae_pad_weight_kernel, dim3(blocks_for(total > N ? total : N)), dim3(256), 0, st,
                     reinterpret_cast<const bf16*>(W), b, reinterpret_cast<bf16*>(Wp), bp, Cout, N, taps, Cin, Cink);
  return hipGetLastError();
}

}  // namespace wan
