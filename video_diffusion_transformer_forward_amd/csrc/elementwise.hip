// Bandwidth-bound kernels: fused LayerNorm + AdaLN modulation, the RoPE
// cos/sin table, the time-embedding GEMVs, v^T key-padding fill, and the fused
// unpatchify + classifier-free guidance + Euler update.
#include "common.h"
#include "kernels.h"

namespace wan {

namespace {

constexpr int LN_MAX_V4 = 20;  // up to D = 5120 per wave (20 float4 per lane)

// One wave per row: the row stays in registers between the mean, the variance
// and the output pass (two-pass statistics, biased variance, eps 1e-6).
// Narrow rows (D = 256*NV up to 2048): one wave walks R consecutive rows, the
// next row's loads in flight while the current one is reduced, and keeps the
// modulation vectors of its batch item in registers instead of re-reading them
// for every row.
// 8-bit output of the LayerNorm kernels: e4m3 bytes [rows][D] and one scale byte per
// (row, 128-column block) at sc[(col / 128) * sc_ld + b * pitch + t] for row = b * rows_per_batch + t
struct LnQ8 {
  unsigned char* out = nullptr;
  unsigned char* sc = nullptr;
  long long sc_ld = 0;
  int pitch = 0;
};

// the four values of a lane at column col (a 128-column block is 32 lanes: half a wave)
__device__ __forceinline__ void ln_store_q8(const LnQ8& q8, const float (&r)[4], int row, int col, int lane, int D,
                                            int rows_per_batch) {
  float am = __builtin_elementwise_maximum(__builtin_elementwise_maximum(fabsf(r[0]), fabsf(r[1])),
                                           __builtin_elementwise_maximum(fabsf(r[2]), fabsf(r[3])));
#pragma unroll
  for (int o = 1; o < 32; o <<= 1) am = __builtin_elementwise_maximum(am, __shfl_xor(am, o, 64));
  const int ex = e8_exponent(am);
  const float inv = __uint_as_float((unsigned)(127 - ex) << 23);
  unsigned w = __builtin_amdgcn_cvt_pk_fp8_f32(r[0] * inv, r[1] * inv, 0u, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(r[2] * inv, r[3] * inv, w, true);
  *reinterpret_cast<unsigned*>(q8.out + (long long)row * D + col) = w;
  if ((lane & 31) == 0) {
    const int b = row / rows_per_batch, t = row - b * rows_per_batch;
    q8.sc[(long long)(col >> 7) * q8.sc_ld + (long long)b * q8.pitch + t] = (unsigned char)(ex + 127);
  }
}

template <typename T, int NV, bool Q8 = false>
__global__ __launch_bounds__(256) void ln_mod_rows_kernel(const float* __restrict__ x, T* __restrict__ out, int rows,
                                                          int R, int rows_per_batch, const float* __restrict__ shift,
                                                          const float* __restrict__ scale, long long mod_bstride,
                                                          LnQ8 q8 = LnQ8()) {
  constexpr int D = NV * 256;
  const int lane = threadIdx.x & 63;
  const int r0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * R;
  if (r0 >= rows) return;
  const int r1 = min(r0 + R, rows);
  float4 v[NV], nx[NV], sc4[NV], sh4[NV];
  int bcur = -1;
  auto load_row = [&](float4 (&dst)[NV], int row) {
    const float4* xr = reinterpret_cast<const float4*>(x + (long long)row * D);
#pragma unroll
    for (int i = 0; i < NV; ++i) dst[i] = xr[i * 64 + lane];
  };
  load_row(v, r0);
  for (int row = r0; row < r1; ++row) {
    if (row + 1 < r1) load_row(nx, row + 1);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) s += (v[i].x + v[i].y) + (v[i].z + v[i].w);
    const float mean = wave_sum(s) * (1.0f / D);
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const float a0 = v[i].x - mean, a1 = v[i].y - mean, a2 = v[i].z - mean, a3 = v[i].w - mean;
      q += (a0 * a0 + a1 * a1) + (a2 * a2 + a3 * a3);
    }
    const float rstd = 1.0f / sqrtf(wave_sum(q) * (1.0f / D) + 1e-6f);
    if (scale) {
      const int b = row / rows_per_batch;
      if (b != bcur) {
        bcur = b;
        const float4* sc = reinterpret_cast<const float4*>(scale + (long long)b * mod_bstride);
        const float4* sh = reinterpret_cast<const float4*>(shift + (long long)b * mod_bstride);
#pragma unroll
        for (int i = 0; i < NV; ++i) {
          sc4[i] = sc[i * 64 + lane];
          sh4[i] = sh[i * 64 + lane];
        }
      }
    }
    T* orow = out + (long long)row * D;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int col = (i * 64 + lane) * 4;
      float r[4] = {(v[i].x - mean) * rstd, (v[i].y - mean) * rstd, (v[i].z - mean) * rstd, (v[i].w - mean) * rstd};
      if (scale) {
        r[0] = r[0] * (1.f + sc4[i].x) + sh4[i].x;
        r[1] = r[1] * (1.f + sc4[i].y) + sh4[i].y;
        r[2] = r[2] * (1.f + sc4[i].z) + sh4[i].z;
        r[3] = r[3] * (1.f + sc4[i].w) + sh4[i].w;
      }
      if constexpr (Q8) {
        ln_store_q8(q8, r, row, col, lane, D, rows_per_batch);
      } else if constexpr (sizeof(T) == 2) {
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        bf16x4 o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = to_bf16(r[e]);
        *reinterpret_cast<bf16x4*>(orow + col) = o4;
      } else {
        *reinterpret_cast<float4*>(orow + col) = make_float4(r[0], r[1], r[2], r[3]);
      }
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i] = nx[i];
  }
}

template <typename T, bool Q8 = false>
__global__ __launch_bounds__(256) void ln_mod_kernel(const float* __restrict__ x, T* __restrict__ out, int rows,
                                                     int D, int rows_per_batch, const float* __restrict__ shift,
                                                     const float* __restrict__ scale, long long mod_bstride,
                                                     LnQ8 q8 = LnQ8()) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int nv = D / 256;  // float4 per lane
  const float4* xr = reinterpret_cast<const float4*>(x + (long long)row * D);
  float4 v[LN_MAX_V4];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < LN_MAX_V4; ++i) {
    if (i < nv) {
      v[i] = xr[i * 64 + lane];
      s += (v[i].x + v[i].y) + (v[i].z + v[i].w);
    }
  }
  const float mean = wave_sum(s) / D;
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < LN_MAX_V4; ++i) {
    if (i < nv) {
      float a0 = v[i].x - mean, a1 = v[i].y - mean, a2 = v[i].z - mean, a3 = v[i].w - mean;
      q += (a0 * a0 + a1 * a1) + (a2 * a2 + a3 * a3);
    }
  }
  const float var = wave_sum(q) / D;
  const float rstd = 1.0f / sqrtf(var + 1e-6f);
  const int b = row / rows_per_batch;
  const float* sh = shift ? shift + (long long)b * mod_bstride : nullptr;
  const float* sc = scale ? scale + (long long)b * mod_bstride : nullptr;
  T* orow = out + (long long)row * D;
#pragma unroll
  for (int i = 0; i < LN_MAX_V4; ++i) {
    if (i < nv) {
      const int col = (i * 64 + lane) * 4;
      float r[4] = {(v[i].x - mean) * rstd, (v[i].y - mean) * rstd, (v[i].z - mean) * rstd,
                    (v[i].w - mean) * rstd};
      if (sc) {
        const float4 s4 = *reinterpret_cast<const float4*>(sc + col);
        const float4 h4 = *reinterpret_cast<const float4*>(sh + col);
        r[0] = r[0] * (1.f + s4.x) + h4.x;
        r[1] = r[1] * (1.f + s4.y) + h4.y;
        r[2] = r[2] * (1.f + s4.z) + h4.z;
        r[3] = r[3] * (1.f + s4.w) + h4.w;
      }
      if constexpr (Q8) {
        ln_store_q8(q8, r, row, col, lane, D, rows_per_batch);
      } else if (sizeof(T) == 2) {
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        bf16x4 o4;
        o4[0] = to_bf16(r[0]);
        o4[1] = to_bf16(r[1]);
        o4[2] = to_bf16(r[2]);
        o4[3] = to_bf16(r[3]);
        *reinterpret_cast<bf16x4*>(orow + col) = o4;
      } else {
        *reinterpret_cast<float4*>(orow + col) = make_float4(r[0], r[1], r[2], r[3]);
      }
    }
  }
}

// (cos, sin) of pos * 10000^(-2r/d_axis) for the three axes, in double.
__global__ void rope_table_kernel(float2* tab, int hd, int F, int Hh, int Ww) {
  const int ds = 2 * (hd / 6);
  const int df = hd - 2 * ds;
  const int n0 = F * (df / 2), n1 = Hh * (ds / 2), n2 = Ww * (ds / 2);
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n0 + n1 + n2) return;
  int pos, r, da;
  if (idx < n0) {
    pos = idx / (df / 2);
    r = idx % (df / 2);
    da = df;
  } else if (idx < n0 + n1) {
    pos = (idx - n0) / (ds / 2);
    r = (idx - n0) % (ds / 2);
    da = ds;
  } else {
    pos = (idx - n0 - n1) / (ds / 2);
    r = (idx - n0 - n1) % (ds / 2);
    da = ds;
  }
  const double theta = pow(10000.0, -2.0 * r / (double)da);
  const double phi = pos * theta;
  tab[idx] = make_float2((float)cos(phi), (float)sin(phi));
}

// tok[t][j] = the segment-table entry of pair j at token t's grid position
__global__ void rope_tokens_kernel(float2* __restrict__ tok, const float2* __restrict__ tab, int hd, int F, int Hh,
                                   int Ww) {
  const int ds = 2 * (hd / 6);
  const int df = hd - 2 * ds;
  const int hp = hd / 2;
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long n = (long long)F * Hh * Ww * hp;
  if (idx >= n) return;
  const int t = (int)(idx / hp), j = (int)(idx - (long long)t * hp);
  const int hw = Hh * Ww;
  const int f = t / hw, rem = t - f * hw;
  const int yy = rem / Ww, xx = rem - yy * Ww;
  int k;
  if (j < df / 2)
    k = f * (df / 2) + j;
  else if (j < df / 2 + ds / 2)
    k = F * (df / 2) + yy * (ds / 2) + (j - df / 2);
  else
    k = F * (df / 2) + Hh * (ds / 2) + xx * (ds / 2) + (j - df / 2 - ds / 2);
  tok[idx] = tab[k];
}

__device__ __forceinline__ int vt_perm_e(int t) { return (t & ~0xC) | (((t >> 2) & 1) << 3) | (((t >> 3) & 1) << 2); }

template <typename T>
__global__ void zero_vt_pad_kernel(T* vt, int rows, int L, int Lp) {
  const int pad = Lp - L;
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long long)rows * pad) return;
  const long long row = idx / pad;
  const int t = L + (int)(idx - row * pad);
  vt[row * Lp + vt_perm_e(t)] = from_f<T>(0.f);
}

// One wave per output: y[n] = sum_k W[n][k] act(x[k]) + b[n].  The input
// vector (K <= 8192) is staged once per workgroup in LDS.
template <typename T>
__global__ __launch_bounds__(256) void gemv_kernel(const T* __restrict__ Wt, const float* __restrict__ bias,
                                                   const float* __restrict__ x, float tau, float* __restrict__ y,
                                                   int N, int K, int silu_in) {
  __shared__ float xs[8192];
  for (int k = threadIdx.x; k < K; k += 256) {
    float v;
    if (x) {
      v = x[k];
    } else {
      // timestep sinusoid: [cos(tau w_i) ; sin(tau w_i)], w_i = 10000^(-i/half)
      const int half = K / 2;
      const int i = k < half ? k : k - half;
      const double w = pow(10000.0, -(double)i / half);
      const double arg = (double)tau * w;
      v = (float)(k < half ? cos(arg) : sin(arg));
    }
    xs[k] = silu_in ? silu(v) : v;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= N) return;
  const T* wr = Wt + (long long)n * K;
  float acc = 0.f;
  for (int k = lane * 8; k < K; k += 64 * 8) {
    Chunk<T> c;
    c.load(wr + k);
    const T* e = reinterpret_cast<const T*>(&c);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += to_f<T>(e[u]) * xs[k + u];
  }
  acc = wave_sum(acc);
  if (lane == 0) y[n] = acc + (bias ? bias[n] : 0.f);
}

// out[b][c][f][y][x] from the head rows p[(b, token)][c*4 + (y%2)*2 + x%2].
// step: out holds z; z += dt * (p_null + g (p_cond - p_null)), p_null rows (b, token) of `pn`.
__global__ void unpatch_kernel(const float* __restrict__ p, const float* __restrict__ pn, float* __restrict__ out,
                               int B, int C, int F, int H, int W, int step, float dt, float guide) {
  const long long n = (long long)B * C * F * H * W;
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n) return;
  long long r = idx;
  const int xw = (int)(r % W); r /= W;
  const int yh = (int)(r % H); r /= H;
  const int f = (int)(r % F); r /= F;
  const int c = (int)(r % C); r /= C;
  const int b = (int)r;
  const int Hh = H / 2, Ww = W / 2;
  const long long L = (long long)F * Hh * Ww;
  const long long tok = ((long long)f * Hh + yh / 2) * Ww + xw / 2;
  const int k = c * 4 + (yh & 1) * 2 + (xw & 1);
  const int K = C * 4;
  const float pc = p[((long long)b * L + tok) * K + k];
  if (!step) {
    out[idx] = pc;
  } else {
    const float pu = pn[((long long)b * L + tok) * K + k];
    const float v = pu + guide * (pc - pu);
    out[idx] = out[idx] + dt * v;
  }
}

// Streaming queue update of one video window z (C, F, H, W): every frame moves by
// its slot's step along the head velocity p (rows = tokens, as unpatch_kernel);
// the first `group` frames go to `out`, the others shift down by `group` into
// `nz`, whose last `group` frames are the new noise frames.
struct StreamDts {
  float v[STREAM_MAX_SLOTS];
};
__global__ void stream_update_kernel(const float* __restrict__ p, const float* __restrict__ z,
                                     const float* __restrict__ noise, float* __restrict__ nz, float* __restrict__ out,
                                     int C, int F, int H, int W, int group, StreamDts dts) {
  const long long n = (long long)C * F * H * W;
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n) return;
  long long r = idx;
  const int xw = (int)(r % W); r /= W;
  const int yh = (int)(r % H); r /= H;
  const int f = (int)(r % F); r /= F;
  const int c = (int)r;
  const int Hh = H / 2, Ww = W / 2;
  const long long tok = ((long long)f * Hh + yh / 2) * Ww + xw / 2;
  const float v = p[tok * (C * 4) + c * 4 + (yh & 1) * 2 + (xw & 1)];
  const float zn = z[idx] + dts.v[f / group] * v;
  const long long plane = (long long)H * W;
  const long long in_frame = (long long)yh * W + xw;
  if (f < group) {
    out[((long long)c * group + f) * plane + in_frame] = zn;
    nz[((long long)c * F + (F - group + f)) * plane + in_frame] = noise[((long long)c * group + f) * plane + in_frame];
  } else {
    nz[((long long)c * F + (f - group)) * plane + in_frame] = zn;
  }
}

// W [N][K] bf16 -> e4m3 bytes [N][K] plus one scale byte per (row, 128-block) at
// sc[blk * N + n]; one wave per block, two elements per lane
__global__ __launch_bounds__(256) void quant_w_kernel(const bf16* __restrict__ W, unsigned char* __restrict__ W8,
                                                      unsigned char* __restrict__ sc, int N, int K) {
  const int nkb = K >> 7;
  const long long wid = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid >= (long long)N * nkb) return;
  const int lane = threadIdx.x & 63;
  const int n = (int)(wid / nkb), kb = (int)(wid - (long long)n * nkb);
  const long long off = (long long)n * K + kb * 128 + 2 * lane;
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 p = *reinterpret_cast<const bf16x2*>(W + off);
  const float a = (float)p[0], b = (float)p[1];
  float am = __builtin_elementwise_maximum(fabsf(a), fabsf(b));
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) am = __builtin_elementwise_maximum(am, __shfl_xor(am, o, 64));
  const int ex = e8_exponent(am);
  const float inv = __uint_as_float((unsigned)(127 - ex) << 23);
  const unsigned w = __builtin_amdgcn_cvt_pk_fp8_f32(a * inv, b * inv, 0u, false);
  *reinterpret_cast<unsigned short*>(W8 + off) = (unsigned short)(w & 0xFFFFu);
  if (lane == 0) sc[(long long)kb * N + n] = (unsigned char)(ex + 127);
}

}  // namespace

hipError_t launch_quant_weights(const void* W, unsigned char* W8, unsigned char* sc, int N, int K, hipStream_t st) {
  if (N <= 0) return hipSuccess;
  if (K % 128 != 0) return hipErrorInvalidValue;
  const long long waves = (long long)N * (K / 128);
  hipLaunchKernelGGL(quant_w_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, st,
                     reinterpret_cast<const bf16*>(W), W8, sc, N, K);
  return hipGetLastError();
}

hipError_t launch_ln_mod8(const float* x, unsigned char* out8, unsigned char* sc, long long sc_ld, int pitch, int rows,
                          int D, int rows_per_batch, const float* shift, const float* scale, long long mod_bstride,
                          hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  if (D % 256 != 0 || D / 256 > LN_MAX_V4 || pitch < rows_per_batch) return hipErrorInvalidValue;
  if ((shift == nullptr) != (scale == nullptr)) return hipErrorInvalidValue;
  LnQ8 q8;
  q8.out = out8;
  q8.sc = sc;
  q8.sc_ld = sc_ld;
  q8.pitch = pitch;
  constexpr int R = 2;  // rows per wave, as in launch_ln_mod
  const dim3 grid_r((rows + 4 * R - 1) / (4 * R));
  bf16* o = nullptr;
  switch (D / 256) {
    case 1: hipLaunchKernelGGL((ln_mod_rows_kernel<bf16, 1, true>), grid_r, dim3(256), 0, st, x, o, rows, R, rows_per_batch, shift, scale, mod_bstride, q8); break;
    case 2: hipLaunchKernelGGL((ln_mod_rows_kernel<bf16, 2, true>), grid_r, dim3(256), 0, st, x, o, rows, R, rows_per_batch, shift, scale, mod_bstride, q8); break;
    case 6: hipLaunchKernelGGL((ln_mod_rows_kernel<bf16, 6, true>), grid_r, dim3(256), 0, st, x, o, rows, R, rows_per_batch, shift, scale, mod_bstride, q8); break;
    default:
      hipLaunchKernelGGL((ln_mod_kernel<bf16, true>), dim3((rows + 3) / 4), dim3(256), 0, st, x, o, rows, D,
                         rows_per_batch, shift, scale, mod_bstride, q8);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_ln_mod(const float* x, void* out, int rows, int D, int rows_per_batch, const float* shift,
                         const float* scale, long long mod_bstride, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  if (D % 256 != 0 || D / 256 > LN_MAX_V4) return hipErrorInvalidValue;
  if ((shift == nullptr) != (scale == nullptr)) return hipErrorInvalidValue;
  constexpr int R = 2;  // rows per wave in the narrow-row kernel (2: 4x the workgroups of 8, a shorter last round; 6% faster)
  const dim3 grid_r((rows + 4 * R - 1) / (4 * R));
  T* o = reinterpret_cast<T*>(out);
  switch (D / 256) {
    case 1: hipLaunchKernelGGL((ln_mod_rows_kernel<T, 1>), grid_r, dim3(256), 0, st, x, o, rows, R, rows_per_batch, shift, scale, mod_bstride); break;
    case 2: hipLaunchKernelGGL((ln_mod_rows_kernel<T, 2>), grid_r, dim3(256), 0, st, x, o, rows, R, rows_per_batch, shift, scale, mod_bstride); break;
    case 6: hipLaunchKernelGGL((ln_mod_rows_kernel<T, 6>), grid_r, dim3(256), 0, st, x, o, rows, R, rows_per_batch, shift, scale, mod_bstride); break;
    default:
      hipLaunchKernelGGL(ln_mod_kernel<T>, dim3((rows + 3) / 4), dim3(256), 0, st, x, o, rows, D, rows_per_batch,
                         shift, scale, mod_bstride);
  }
  return hipGetLastError();
}

hipError_t launch_rope_table(float2* tab, int hd, int F, int Hh, int Ww, hipStream_t st) {
  const int ds = 2 * (hd / 6);
  const int df = hd - 2 * ds;
  const int n = F * (df / 2) + Hh * (ds / 2) + Ww * (ds / 2);
  hipLaunchKernelGGL(rope_table_kernel, dim3((n + 255) / 256), dim3(256), 0, st, tab, hd, F, Hh, Ww);
  return hipGetLastError();
}

hipError_t launch_rope_tokens(float2* tok, const float2* tab, int hd, int F, int Hh, int Ww, hipStream_t st) {
  const long long n = (long long)F * Hh * Ww * (hd / 2);
  hipLaunchKernelGGL(rope_tokens_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, tok, tab, hd, F, Hh, Ww);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_zero_vt_pad(void* vt, int BH, int hd, int L, int Lp, hipStream_t st) {
  const long long n = (long long)BH * hd * (Lp - L);
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_vt_pad_kernel<T>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                     reinterpret_cast<T*>(vt), BH * hd, L, Lp);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_gemv(const void* Wt, const float* bias, const float* x, float tau, float* y, int N, int K,
                       int silu_in, hipStream_t st) {
  if (K > 8192 || K % 8 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gemv_kernel<T>, dim3((N + 3) / 4), dim3(256), 0, st, reinterpret_cast<const T*>(Wt), bias, x,
                     tau, y, N, K, silu_in);
  return hipGetLastError();
}

hipError_t launch_unpatch(const float* p, float* out, int B, int C, int F, int H, int W, int step, float dt,
                          float guide, hipStream_t st, const float* p_null) {
  const long long n = (long long)B * C * F * H * W;
  if (n <= 0) return hipSuccess;
  const long long L = (long long)F * (H / 2) * (W / 2);
  if (!p_null) p_null = p + (long long)B * L * C * 4;
  hipLaunchKernelGGL(unpatch_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, p_null, out, B, C, F,
                     H, W, step, dt, guide);
  return hipGetLastError();
}

hipError_t launch_stream_update(const float* p, const float* z, const float* noise, float* nz, float* out, int C,
                                int F, int H, int W, int group, const float* dts, int K, hipStream_t st) {
  const long long n = (long long)C * F * H * W;
  if (n <= 0) return hipSuccess;
  if (K < 1 || K > STREAM_MAX_SLOTS || group < 1 || F != K * group) return hipErrorInvalidValue;
  StreamDts d;
  for (int k = 0; k < STREAM_MAX_SLOTS; ++k) d.v[k] = k < K ? dts[k] : 0.f;
  hipLaunchKernelGGL(stream_update_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, z, noise, nz, out,
                     C, F, H, W, group, d);
  return hipGetLastError();
}

hipError_t copy_async(void* dst, const void* src, size_t bytes, hipStream_t st) {
  return hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, st);
}

template hipError_t launch_ln_mod<bf16>(const float*, void*, int, int, int, const float*, const float*, long long,
                                        hipStream_t);
template hipError_t launch_ln_mod<float>(const float*, void*, int, int, int, const float*, const float*, long long,
                                         hipStream_t);
template hipError_t launch_zero_vt_pad<bf16>(void*, int, int, int, int, hipStream_t);
template hipError_t launch_zero_vt_pad<float>(void*, int, int, int, int, hipStream_t);
template hipError_t launch_gemv<bf16>(const void*, const float*, const float*, float, float*, int, int, int,
                                      hipStream_t);
template hipError_t launch_gemv<float>(const void*, const float*, const float*, float, float*, int, int, int,
                                       hipStream_t);

}  // namespace wan
