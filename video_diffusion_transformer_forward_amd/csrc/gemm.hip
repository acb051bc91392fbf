// LDS-tiled MFMA GEMM for gfx950: C = A W^T + bias with fused epilogues.
//
// 256 threads (4 waves) per workgroup, a BM x BN tile, BK-deep k-steps, two
// LDS stages.  Global loads of step k+1 are issued before the MFMAs of step k
// and written to the idle LDS stage afterwards, one barrier per step.  LDS rows
// hold 8-element chunks XOR-swizzled by row so that the 32 rows one MFMA
// operand reads land on distinct banks.  Tiles are ordered in groups of 8
// M-tiles and the hardware workgroup order is remapped so that each XCD (with
// its own L2) works on one contiguous group of tiles.
#include "common.h"
#include "kernels.h"

namespace wan {

namespace {

template <typename T, int BM, int BN, int WM, int WN, int LOADER, int EPI>
struct Gemm {
  static constexpr int BK = sizeof(T) == 2 ? 64 : 32;
  static constexpr int CPR = BK / 8;  // chunks per tile row
  static constexpr int TM = BM / WM / 32;
  static constexpr int TN = BN / WN / 32;
  static constexpr int A_PT = BM * CPR / 256;
  static constexpr int B_PT = BN * CPR / 256;
  static constexpr int STAGE = (BM + BN) * CPR;  // chunks per stage
  static constexpr size_t PIPE_BYTES = 2 * STAGE * sizeof(Chunk<T>);
  // epilogue slab: the whole tile when it fits the pipeline's LDS, else one wave column
  static constexpr int SW = ((size_t)BM * (BN + 4) * 4 <= PIPE_BYTES) ? BN : BN / WN;
  static constexpr int SWP = SW + 4;
  static constexpr size_t SLAB_BYTES = (size_t)BM * SWP * 4;
  static constexpr size_t LDS_BYTES = PIPE_BYTES > SLAB_BYTES ? PIPE_BYTES : SLAB_BYTES;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
  static_assert(BN % SW == 0 && SW % 8 == 0, "slab");
  static_assert(WM * WN == 4, "4 waves");
  static_assert(TM >= 1 && TN >= 1, "wave tile");
  static_assert((BM * CPR) % 256 == 0 && (BN * CPR) % 256 == 0, "load split");
};

// Load the 8 patch features [k0, k0+8) of token row (b, t): two channels x (2x2).
template <typename T>
__device__ __forceinline__ void load_patch_chunk(Chunk<T>& out, const GemmArgs& g, int zb, int f, int i, int j,
                                                 int k0) {
  float v[8];
  const long long HW = (long long)g.H * g.W;
#pragma unroll
  for (int cc = 0; cc < 2; ++cc) {
    int ch = k0 / 4 + cc;
    const float* src;
    if (ch < 16)
      src = g.z + (((long long)zb * 16 + ch) * g.F + f) * HW;
    else
      src = g.cond + (((long long)zb * (g.in_ch - 16) + (ch - 16)) * g.F + f) * HW;
    const float2 r0 = *reinterpret_cast<const float2*>(src + (long long)(2 * i) * g.W + 2 * j);
    const float2 r1 = *reinterpret_cast<const float2*>(src + (long long)(2 * i + 1) * g.W + 2 * j);
    v[cc * 4 + 0] = r0.x;
    v[cc * 4 + 1] = r0.y;
    v[cc * 4 + 2] = r1.x;
    v[cc * 4 + 3] = r1.y;
  }
  pack8(out, v);
}

__device__ __forceinline__ int vt_perm(int t) {
  // keys are stored with 4-key runs 1 and 2 of every 16-key group swapped, the
  // order in which one 32x32 MFMA of P^T consumes them
  return (t & ~0xC) | (((t >> 2) & 1) << 3) | (((t >> 3) & 1) << 2);
}

template <typename T, int BM, int BN, int WM, int WN, int LOADER, int EPI>
__global__ __launch_bounds__(256) void gemm_kernel(const GemmArgs g) {
  using C = Gemm<T, BM, BN, WM, WN, LOADER, EPI>;
  constexpr int BK = C::BK, CPR = C::CPR, TM = C::TM, TN = C::TN;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  Chunk<T>* smem = reinterpret_cast<Chunk<T>*>(smem_raw);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g2 = lane >> 5;  // lane group: which 8-chunk of a 16-wide k step
  const int l32 = lane & 31;

  // ---- tile coordinates: XCD-contiguous ranges, groups of 8 M-tiles
  const int nm = (g.M + BM - 1) / BM;
  const int nn = g.N / BN;
  const int ntiles = nm * nn;
  const int lid = xcd_remap(blockIdx.x, ntiles);
  constexpr int GM = 8;
  const int group = lid / (GM * nn);
  const int first_m = group * GM;
  const int gsize = min(nm - first_m, GM);
  const int in_group = lid - group * GM * nn;
  const int tm = first_m + in_group % gsize;
  const int tn = in_group / gsize;
  const int m0 = tm * BM;
  const int n0 = tn * BN;

  // ---- per-thread load rows (fixed across k-steps)
  const T* a_ptr[C::A_PT];
  int pf[C::A_PT], pi[C::A_PT], pj[C::A_PT], pzb[C::A_PT];
#pragma unroll
  for (int u = 0; u < C::A_PT; ++u) {
    int idx = tid + 256 * u;
    int r = m0 + idx / CPR;
    r = min(r, g.M - 1);
    if (LOADER == LOAD_PLAIN) {
      int b = r / g.a_rpb, t = r - b * g.a_rpb;
      a_ptr[u] = reinterpret_cast<const T*>(g.A) + (long long)b * g.a_bstride + (long long)t * g.lda;
    } else {
      int b = r / g.c_rpb, t = r - b * g.c_rpb;
      int hh = g.H / 2, ww = g.W / 2;
      pf[u] = t / (hh * ww);
      int rem = t - pf[u] * hh * ww;
      pi[u] = rem / ww;
      pj[u] = rem - pi[u] * ww;
      pzb[u] = b % g.z_batch;
    }
  }
  const T* b_ptr[C::B_PT];
#pragma unroll
  for (int u = 0; u < C::B_PT; ++u) {
    int idx = tid + 256 * u;
    b_ptr[u] = reinterpret_cast<const T*>(g.Wt) + (long long)(n0 + idx / CPR) * g.ldw;
  }

  Chunk<T> ra[C::A_PT], rb[C::B_PT];
  auto load_tile = [&](int kt) {
    const int kb = kt * BK;
#pragma unroll
    for (int u = 0; u < C::A_PT; ++u) {
      int c = (tid + 256 * u) % CPR;
      int k0 = kb + c * 8;
      if (k0 < g.K) {
        if (LOADER == LOAD_PLAIN)
          ra[u].load(a_ptr[u] + k0);
        else
          load_patch_chunk<T>(ra[u], g, pzb[u], pf[u], pi[u], pj[u], k0);
      } else {
        ra[u].zero();
      }
    }
#pragma unroll
    for (int u = 0; u < C::B_PT; ++u) {
      int c = (tid + 256 * u) % CPR;
      int k0 = kb + c * 8;
      if (k0 < g.K)
        rb[u].load(b_ptr[u] + k0);
      else
        rb[u].zero();
    }
  };
  auto store_tile = [&](int stage) {
    Chunk<T>* sa = smem + stage * C::STAGE;
    Chunk<T>* sb = sa + BM * CPR;
#pragma unroll
    for (int u = 0; u < C::A_PT; ++u) {
      int idx = tid + 256 * u;
      int r = idx / CPR, c = idx % CPR;
      ra[u].store(&sa[r * CPR + (c ^ (r & (CPR - 1)))]);
    }
#pragma unroll
    for (int u = 0; u < C::B_PT; ++u) {
      int idx = tid + 256 * u;
      int r = idx / CPR, c = idx % CPR;
      rb[u].store(&sb[r * CPR + (c ^ (r & (CPR - 1)))]);
    }
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int wm = wave / WN, wn = wave % WN;
  const int arow0 = wm * (BM / WM);
  const int brow0 = wn * (BN / WN);

  const int nk = (g.K + BK - 1) / BK;
  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_tile(kt + 1);
    const Chunk<T>* sa = smem + cur * C::STAGE;
    const Chunk<T>* sb = sa + BM * CPR;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int c = 2 * ks + g2;
      Chunk<T> fa[TM], fb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        int r = arow0 + 32 * i + l32;
        fa[i].load(&sa[r * CPR + (c ^ (r & (CPR - 1)))]);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        int r = brow0 + 32 * j + l32;
        fb[j].load(&sb[r * CPR + (c ^ (r & (CPR - 1)))]);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) mma32(acc[i][j], fa[i], fb[j]);
    }
    if (kt + 1 < nk) store_tile(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue.  The fp32 tile goes through LDS in column slabs (phase 1:
  // lane writes its column l32, rows 8*(r/4) + 4*g2 + r%4 of each 32x32 block);
  // phase 2 walks the slab in 8-element chunks and writes 16-byte pieces.
  float* slab = reinterpret_cast<float*>(smem_raw);
  constexpr int SW = C::SW, SWP = C::SWP;
#pragma unroll
  for (int s0 = 0; s0 < BN; s0 += SW) {
    // phase 1
    if (brow0 + BN / WN > s0 && brow0 < s0 + SW) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int col = brow0 + 32 * j + l32 - s0;
        if (col < 0 || col >= SW) continue;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = arow0 + 32 * i + 8 * (r / 4) + 4 * g2 + (r % 4);
            slab[row * SWP + col] = acc[i][j][r];
          }
      }
    }
    __syncthreads();
    // phase 2
    const int nbase = n0 + s0;
    int sec = 0;
    if (EPI == EPI_PACK) sec = nbase < g.nq ? 0 : (nbase < g.nq + g.nk ? 1 : 2);
    if (EPI == EPI_PACK && sec == 2) {
      // v^T: a chunk is 8 consecutive tokens of one feature column
      const int nv0 = nbase - g.nq - g.nk;
      for (int idx = tid; idx < SW * (BM / 8); idx += 256) {
        const int col = idx % SW;
        const int r8 = (idx / SW) * 8;
        const int nvc = nv0 + col;
        const int hh = nvc / g.hd, e = nvc - hh * g.hd;
        const float bn = g.bias[nbase + col];
        const int row0 = m0 + r8;
        if (row0 >= g.M) continue;
        const int b0 = row0 / g.c_rpb, t0 = row0 - b0 * g.c_rpb;
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = slab[(r8 + u) * SWP + col] + bn;
        T* vrow = reinterpret_cast<T*>(g.vt) + (((long long)b0 * g.heads + hh) * g.hd + e) * g.Lp;
        if ((t0 & 7) == 0 && t0 + 8 <= g.c_rpb && row0 + 8 <= g.M) {
          // 8 aligned tokens: two runs of 4 that stay contiguous under the key permutation
#pragma unroll
          for (int u = 0; u < 8; ++u) vrow[vt_perm(t0 + u)] = from_f<T>(v[u]);
        } else {
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int rr = row0 + u;
            if (rr >= g.M) break;
            const int b = rr / g.c_rpb, t = rr - b * g.c_rpb;
            reinterpret_cast<T*>(g.vt)[(((long long)b * g.heads + hh) * g.hd + e) * g.Lp + vt_perm(t)] =
                from_f<T>(v[u]);
          }
        }
      }
    } else {
      for (int idx = tid; idx < BM * (SW / 8); idx += 256) {
        const int lrow = idx / (SW / 8);
        const int c8 = (idx % (SW / 8)) * 8;
        const int row = m0 + lrow;
        if (row >= g.M) continue;
        const int n = nbase + c8;
        float v[8];
        const f32x4 lo = *reinterpret_cast<const f32x4*>(&slab[lrow * SWP + c8]);
        const f32x4 hi = *reinterpret_cast<const f32x4*>(&slab[lrow * SWP + c8 + 4]);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          v[u] = lo[u];
          v[4 + u] = hi[u];
        }
        if (g.bias) {
          const f32x4 b0 = *reinterpret_cast<const f32x4*>(g.bias + n);
          const f32x4 b1 = *reinterpret_cast<const f32x4*>(g.bias + n + 4);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            v[u] += b0[u];
            v[4 + u] += b1[u];
          }
        }
        if (EPI == EPI_STORE || EPI == EPI_STORE_GELU) {
          if (EPI == EPI_STORE_GELU) {
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = gelu_erf(v[u]);
          }
          Chunk<T> c;
          pack8(c, v);
          c.store(reinterpret_cast<T*>(g.C) + (long long)row * g.ldc + n);
        } else if (EPI == EPI_STORE_F32) {
          Chunk<float> c;
          pack8(c, v);
          c.store(reinterpret_cast<float*>(g.C) + (long long)row * g.ldc + n);
        } else if (EPI == EPI_RESID) {
          float* xp = g.x + (long long)row * g.ldx + n;
          f32x4 x0 = *reinterpret_cast<const f32x4*>(xp);
          f32x4 x1 = *reinterpret_cast<const f32x4*>(xp + 4);
          if (g.gate) {
            const int b = row / g.c_rpb;
            const float* gp = g.gate + (long long)b * g.gate_bstride + n;
            const f32x4 g0 = *reinterpret_cast<const f32x4*>(gp);
            const f32x4 g1 = *reinterpret_cast<const f32x4*>(gp + 4);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              x0[u] += g0[u] * v[u];
              x1[u] += g1[u] * v[4 + u];
            }
          } else {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              x0[u] += v[u];
              x1[u] += v[4 + u];
            }
          }
          *reinterpret_cast<f32x4*>(xp) = x0;
          *reinterpret_cast<f32x4*>(xp + 4) = x1;
        } else if (EPI == EPI_PACK) {
          // q or k, with optional RoPE on the adjacent pairs of the chunk
          const int nsec = n - (sec == 0 ? 0 : g.nq);
          const int hh = nsec / g.hd, e0 = nsec - hh * g.hd;
          const int b = row / g.c_rpb, t = row - b * g.c_rpb;
          if (g.rope) {
            const int hw = g.gH * g.gW;
            const int f = t / hw;
            const int rem = t - f * hw;
            const int yy = rem / g.gW;
            const int xx = rem - yy * g.gW;
            const int ds = 2 * (g.hd / 6);
            const int df = g.hd - 2 * ds;
#pragma unroll
            for (int u = 0; u < 8; u += 2) {
              const int e = e0 + u;
              float2 cs;
              if (e < df)
                cs = g.rope[f * (df / 2) + e / 2];
              else if (e < df + ds)
                cs = g.rope[g.gF * (df / 2) + yy * (ds / 2) + (e - df) / 2];
              else
                cs = g.rope[g.gF * (df / 2) + g.gH * (ds / 2) + xx * (ds / 2) + (e - df - ds) / 2];
              const float u0 = v[u], u1 = v[u + 1];
              v[u] = u0 * cs.x - u1 * cs.y;
              v[u + 1] = u0 * cs.y + u1 * cs.x;
            }
          }
          Chunk<T> c;
          pack8(c, v);
          T* base = reinterpret_cast<T*>(sec == 0 ? g.q : g.k);
          c.store(base + (((long long)b * g.heads + hh) * g.Lp + t) * g.hd + e0);
        }
      }
    }
    __syncthreads();
  }
}

template <typename T, int BM, int BN, int WM, int WN, int LOADER, int EPI>
hipError_t launch_cfg(const GemmArgs& g, hipStream_t st) {
  using C = Gemm<T, BM, BN, WM, WN, LOADER, EPI>;
  if (g.N % BN != 0) return hipErrorInvalidValue;
  auto kern = gemm_kernel<T, BM, BN, WM, WN, LOADER, EPI>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::LDS_BYTES);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int nm = (g.M + BM - 1) / BM;
  const int nt = nm * (g.N / BN);
  hipLaunchKernelGGL(kern, dim3(nt), dim3(256), C::LDS_BYTES, st, g);
  return hipGetLastError();
}

template <typename T, int LOADER, int EPI>
hipError_t launch_by_n(const GemmArgs& g, hipStream_t st) {
  if constexpr (sizeof(T) == 2) {
    if (g.N % 256 == 0) return launch_cfg<T, 256, 256, 2, 2, LOADER, EPI>(g, st);
    if (g.N % 64 == 0) return launch_cfg<T, 128, 64, 4, 1, LOADER, EPI>(g, st);
  } else {
    if (g.N % 128 == 0) return launch_cfg<T, 128, 128, 2, 2, LOADER, EPI>(g, st);
    if (g.N % 64 == 0) return launch_cfg<T, 128, 64, 4, 1, LOADER, EPI>(g, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

template <typename T>
hipError_t launch_gemm(const GemmArgs& g, int loader, int epi, hipStream_t st) {
  if (g.M <= 0) return hipSuccess;
  if (loader == LOAD_PATCH) {
    if (epi == EPI_STORE_F32) return launch_by_n<T, LOAD_PATCH, EPI_STORE_F32>(g, st);
    return hipErrorInvalidValue;
  }
  switch (epi) {
    case EPI_STORE: return launch_by_n<T, LOAD_PLAIN, EPI_STORE>(g, st);
    case EPI_STORE_GELU: return launch_by_n<T, LOAD_PLAIN, EPI_STORE_GELU>(g, st);
    case EPI_STORE_F32: return launch_by_n<T, LOAD_PLAIN, EPI_STORE_F32>(g, st);
    case EPI_RESID: return launch_by_n<T, LOAD_PLAIN, EPI_RESID>(g, st);
    case EPI_PACK: return launch_by_n<T, LOAD_PLAIN, EPI_PACK>(g, st);
  }
  return hipErrorInvalidValue;
}

template hipError_t launch_gemm<bf16>(const GemmArgs&, int, int, hipStream_t);
template hipError_t launch_gemm<float>(const GemmArgs&, int, int, hipStream_t);

}  // namespace wan
