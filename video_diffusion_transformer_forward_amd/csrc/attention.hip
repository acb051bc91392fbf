// Flash attention for gfx950: softmax(q k^T / sqrt(d)) v without storing the
// score matrix, for self-attention (one key/value source) and decoupled
// cross-attention (two sources, each with its own softmax, results summed).
//
// Work split: a workgroup of 4 waves owns 4*32*QB queries of one (batch, head);
// each wave keeps its 32*QB query rows in registers as the B operand of
// S^T = K Q^T (32x32x16 MFMA, keys on the row axis, queries on the column
// axis).  The softmax statistics of a query live in the two lanes l and l^32
// that hold its column, so a row max needs a single cross-lane exchange.  The
// probabilities go straight from the S^T accumulators into the B operand of
// O^T = V^T P^T; v is stored transposed with 4-key runs permuted inside every
// 16-key group so that each lane's eight keys are one 16-byte LDS read.
// K and V^T tiles of 64 keys are double-buffered in LDS (XOR-swizzled rows),
// the next tile's global loads overlapping the current tile's MFMAs.
// The running max is only moved (and the accumulators rescaled) when it grows
// by more than 2^8: the probabilities then stay below 256, and numerator and
// denominator share the same stale max, so the result is unchanged.
#include "common.h"
#include "kernels.h"

namespace wan {

namespace {

constexpr int ATT_BN = 64;
constexpr float RESCALE_LOG2 = 8.0f;  // move the running max only when it grows by > 2^8

typedef __attribute__((address_space(3))) void lds_void;

template <typename T, int HD>
struct AttCfg {
  static constexpr int HC = HD / 8;                       // chunks per K row
  static constexpr int KCH = ATT_BN * HC;                 // chunks per K tile
  static constexpr int VCH = HD * (ATT_BN / 8);           // chunks per V^T tile
  static constexpr int STAGE = KCH + VCH;                 // chunks per pipeline stage
  static constexpr int SPC = (int)sizeof(Chunk<T>) / 16;  // 16-byte pieces per chunk
  static constexpr int K_DMA = KCH * SPC / 256;           // 16-byte LDS-DMA loads per thread per K tile
  static constexpr int V_DMA = VCH * SPC / 256;
  static constexpr size_t LDS_BYTES = 2 * STAGE * sizeof(Chunk<T>);
};

template <typename T, int HD, int NSRC>
__device__ __forceinline__ void attn_body(const AttnArgs& a) {
  using Cfg = AttCfg<T, HD>;
  constexpr int HC = Cfg::HC;
  constexpr int SPC = Cfg::SPC;
  constexpr int BMQ = 128;      // queries per workgroup: 4 waves x 32
  constexpr int ND = HD / 32;   // 32-row blocks of d in O^T
  constexpr int NS = HD / 16;   // 16-deep k steps of S^T
  extern __shared__ __align__(16) unsigned char smem_raw[];
  Chunk<T>* smem = reinterpret_cast<Chunk<T>*>(smem_raw);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g2 = lane >> 5;
  const int l32 = lane & 31;

  const int nqt = (a.Lq + BMQ - 1) / BMQ;
  const int G = nqt * a.heads * a.B;
  const int id = xcd_remap(blockIdx.x, G);
  const int qt = id % nqt;
  const int bh = id / nqt;
  const int b = bh / a.heads;
  const int h = bh - b * a.heads;
  const int q0 = qt * BMQ + wave * 32;
  const float c = a.scale_log2;

  // queries of this wave: B operand chunks (query l32, d chunk 2s + g2)
  Chunk<T> qf[NS];
  {
    const int qrow = q0 + l32;
    const T* qp = reinterpret_cast<const T*>(a.q) + ((long long)bh * a.Lqp + qrow) * HD;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (qrow < a.Lq)
        qf[s].load(qp + (2 * s + g2) * 8);
      else
        qf[s].zero();
    }
  }

  // K / V^T tiles go global -> LDS directly; each wave instruction fills 1 KB of LDS,
  // lane l the l-th 16 bytes, so the swizzle is applied on the global side.
  auto issue_tile = [&](const T* Kp, const T* Vp, int Lkp, int j, int stage) {
    unsigned char* kst = smem_raw + (size_t)stage * Cfg::STAGE * sizeof(Chunk<T>);
    unsigned char* vst = kst + (size_t)Cfg::KCH * sizeof(Chunk<T>);
#pragma unroll
    for (int i = 0; i < Cfg::K_DMA; ++i) {
      const int P = (wave * Cfg::K_DMA + i) * 64 + lane;   // 16-byte piece in the tile
      const int pc = P / SPC, sub = P % SPC;               // physical chunk, piece within it
      const int r = pc / HC, pcol = pc % HC;
      const int lc = pcol ^ (r & 7);                       // logical chunk stored there
      const T* src = Kp + (long long)(j * ATT_BN + r) * HD + lc * 8 + sub * (8 / SPC);
      __builtin_amdgcn_global_load_lds(src, (lds_void*)(kst + (size_t)(wave * Cfg::K_DMA + i) * 1024), 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < Cfg::V_DMA; ++i) {
      const int P = (wave * Cfg::V_DMA + i) * 64 + lane;
      const int pc = P / SPC, sub = P % SPC;
      const int r = pc / 8, pcol = pc % 8;
      const int lc = pcol ^ (r & 7);
      const T* src = Vp + (long long)r * Lkp + j * ATT_BN + lc * 8 + sub * (8 / SPC);
      __builtin_amdgcn_global_load_lds(src, (lds_void*)(vst + (size_t)(wave * Cfg::V_DMA + i) * 1024), 16, 0, 0);
    }
  };

  f32x16 o[ND];
  f32x16 o_prev[NSRC == 2 ? ND : 1];

  for (int src = 0; src < NSRC; ++src) {
    const int Lk = a.Lk[src];
    const int Lkp = a.Lkp[src];
    const T* Kp = reinterpret_cast<const T*>(a.k[src]) + (long long)bh * Lkp * HD;
    const T* Vp = reinterpret_cast<const T*>(a.vt[src]) + (long long)bh * HD * Lkp;
    const int nkt = (Lk + ATT_BN - 1) / ATT_BN;

    float m = -INFINITY, l = 0.f;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] = 0.f;

    issue_tile(Kp, Vp, Lkp, 0, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    for (int j = 0; j < nkt; ++j) {
      const int cur = j & 1;
      if (j + 1 < nkt) issue_tile(Kp, Vp, Lkp, j + 1, cur ^ 1);
      const Chunk<T>* ks = smem + cur * Cfg::STAGE;
      const Chunk<T>* vs = ks + Cfg::KCH;

      // S^T = K Q^T for the 64 keys of the tile (two 32-key blocks)
      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int row = 32 * kb + l32;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          Chunk<T> ka;
          ka.load(&ks[row * HC + ((2 * s + g2) ^ (row & 7))]);
          if (s == 0) {
            f32x16 zero = {};
            sacc[kb] = zero;
          }
          mma32(sacc[kb], ka, qf[s]);
        }
      }

      // online softmax in base 2; the scale enters through one FMA per score
      float mx = -INFINITY;
      if ((j + 1) * ATT_BN > Lk) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = j * ATT_BN + 32 * kb + 8 * (r / 4) + 4 * g2 + (r % 4);
            if (key >= Lk) sacc[kb][r] = -INFINITY;
          }
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) mx = fmaxf(mx, fmaxf(sacc[kb][r], sacc[kb][r + 1]));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mnew = fmaxf(m, mx);
      if (__ballot((mnew - m) * c > RESCALE_LOG2) != 0) {
        const float alpha = __builtin_amdgcn_exp2f((m - mnew) * c);
        m = mnew;
        l *= alpha;
#pragma unroll
        for (int db = 0; db < ND; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      }
      const float nmc = -m * c;
      Chunk<T> pf[4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          float p[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][8 * half + e], c, nmc));
            l += p[e];
          }
          pack8(pf[2 * kb + half], p);
        }

      // O^T += V^T P^T, four 16-key steps
#pragma unroll
      for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int db = 0; db < ND; ++db) {
          const int row = 32 * db + l32;
          Chunk<T> va;
          va.load(&vs[row * 8 + ((2 * u + g2) ^ (row & 7))]);
          mma32(o[db], va, pf[u]);
        }
      }

      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    }

    // normalise this source
    const float inv = 1.0f / (l + __shfl_xor(l, 32, 64));
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v = o[db][r] * inv;
        if (NSRC == 2) {
          if (src == 0)
            o_prev[db % (NSRC == 2 ? ND : 1)][r] = v;
          else
            v += o_prev[db % (NSRC == 2 ? ND : 1)][r];
        }
        o[db][r] = v;
      }
  }

  // ---- epilogue: stage the wave's rows in LDS as [query][d], then 16-byte row stores
  T* st = reinterpret_cast<T*>(smem_raw) + wave * (32 * HD);
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int d = 32 * db + 8 * (r / 4) + 4 * g2 + (r % 4);
      st[l32 * HD + d] = from_f<T>(o[db][r]);
    }
  __syncthreads();
  const int ld = a.heads * HD;
#pragma unroll
  for (int u = 0; u < (32 * HC) / 64; ++u) {
    const int idx = lane + 64 * u;
    const int qr = idx / HC, cc = idx % HC;
    const int q = q0 + qr;
    if (q < a.Lq) {
      Chunk<T> v;
      v.load(st + qr * HD + cc * 8);
      v.store(reinterpret_cast<T*>(a.o) + ((long long)b * a.Lq + q) * ld + h * HD + cc * 8);
    }
  }
}

// one key/value source: two workgroups per CU (at most 256 registers per lane)
template <typename T, int HD>
__global__ __launch_bounds__(256, 2) void attn_kernel_1src(const AttnArgs a) {
  attn_body<T, HD, 1>(a);
}
// image + text sources keep a second accumulator: one workgroup per CU
template <typename T, int HD>
__global__ __launch_bounds__(256, 1) void attn_kernel_2src(const AttnArgs a) {
  attn_body<T, HD, 2>(a);
}

template <typename T, int HD, int NSRC>
hipError_t launch_attn_cfg(const AttnArgs& a, hipStream_t st) {
  using Cfg = AttCfg<T, HD>;
  auto kern = NSRC == 1 ? attn_kernel_1src<T, HD> : attn_kernel_2src<T, HD>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)Cfg::LDS_BYTES);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int nqt = (a.Lq + 127) / 128;
  const int G = nqt * a.heads * a.B;
  hipLaunchKernelGGL(kern, dim3(G), dim3(256), Cfg::LDS_BYTES, st, a);
  return hipGetLastError();
}

}  // namespace

template <typename T>
hipError_t launch_attention(const AttnArgs& a, hipStream_t st) {
  if (a.Lq <= 0) return hipSuccess;
  if (a.hd == 128) {
    if (a.nsrc == 1) return launch_attn_cfg<T, 128, 1>(a, st);
    return launch_attn_cfg<T, 128, 2>(a, st);
  }
  if (a.hd == 64) {
    if (a.nsrc == 1) return launch_attn_cfg<T, 64, 1>(a, st);
    return launch_attn_cfg<T, 64, 2>(a, st);
  }
  return hipErrorInvalidValue;
}

template hipError_t launch_attention<bf16>(const AttnArgs&, hipStream_t);
template hipError_t launch_attention<float>(const AttnArgs&, hipStream_t);

}  // namespace wan
