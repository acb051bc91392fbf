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
constexpr float RESCALE_THRESHOLD = 8.0f;

template <typename T, int HD>
struct AttCfg {
  static constexpr int HC = HD / 8;                 // chunks per K row
  static constexpr int KCH = ATT_BN * HC;           // chunks per K tile
  static constexpr int VCH = HD * (ATT_BN / 8);     // chunks per V^T tile
  static constexpr int STAGE = KCH + VCH;
  static constexpr int KPT = KCH / 256;             // K chunks loaded per thread
  static constexpr int VPT = VCH / 256;
  static constexpr size_t LDS_BYTES = 2 * STAGE * sizeof(Chunk<T>);
};

template <typename T, int HD, int QB, int NSRC>
__global__ __launch_bounds__(256) void attn_kernel(const AttnArgs a) {
  using Cfg = AttCfg<T, HD>;
  constexpr int HC = Cfg::HC;
  constexpr int BMQ = 4 * 32 * QB;
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
  const int q0 = qt * BMQ + wave * 32 * QB;

  // ---- queries of this wave: B operand chunks
  Chunk<T> qf[QB][NS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qrow = q0 + 32 * qb + l32;
    const T* qp = reinterpret_cast<const T*>(a.q) + ((long long)bh * a.Lqp + qrow) * HD;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (qrow < a.Lq)
        qf[qb][s].load(qp + (2 * s + g2) * 8);
      else
        qf[qb][s].zero();
    }
  }

  Chunk<T> rk[Cfg::KPT], rv[Cfg::VPT];
  auto load_tile = [&](const T* Kp, const T* Vp, int Lkp, int j) {
#pragma unroll
    for (int u = 0; u < Cfg::KPT; ++u) {
      int idx = tid + 256 * u;
      int row = idx / HC, c = idx % HC;
      rk[u].load(Kp + (long long)(j * ATT_BN + row) * HD + c * 8);
    }
#pragma unroll
    for (int u = 0; u < Cfg::VPT; ++u) {
      int idx = tid + 256 * u;
      int row = idx / 8, c = idx % 8;
      rv[u].load(Vp + (long long)row * Lkp + j * ATT_BN + c * 8);
    }
  };
  auto store_tile = [&](int stage) {
    Chunk<T>* ks = smem + stage * Cfg::STAGE;
    Chunk<T>* vs = ks + Cfg::KCH;
#pragma unroll
    for (int u = 0; u < Cfg::KPT; ++u) {
      int idx = tid + 256 * u;
      int row = idx / HC, c = idx % HC;
      rk[u].store(&ks[row * HC + (c ^ (row & 7))]);
    }
#pragma unroll
    for (int u = 0; u < Cfg::VPT; ++u) {
      int idx = tid + 256 * u;
      int row = idx / 8, c = idx % 8;
      rv[u].store(&vs[row * 8 + (c ^ (row & 7))]);
    }
  };

  f32x16 o[QB][ND];
  f32x16 o_prev[QB][NSRC == 2 ? ND : 1];

  for (int src = 0; src < NSRC; ++src) {
    const int Lk = a.Lk[src];
    const int Lkp = a.Lkp[src];
    const T* Kp = reinterpret_cast<const T*>(a.k[src]) + (long long)bh * Lkp * HD;
    const T* Vp = reinterpret_cast<const T*>(a.vt[src]) + (long long)bh * HD * Lkp;
    const int nkt = (Lk + ATT_BN - 1) / ATT_BN;

    float m[QB], l[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      m[qb] = -INFINITY;
      l[qb] = 0.f;
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[qb][db][r] = 0.f;
    }

    load_tile(Kp, Vp, Lkp, 0);
    store_tile(0);
    __syncthreads();

    for (int j = 0; j < nkt; ++j) {
      const int cur = j & 1;
      if (j + 1 < nkt) load_tile(Kp, Vp, Lkp, j + 1);
      const Chunk<T>* ks = smem + cur * Cfg::STAGE;
      const Chunk<T>* vs = ks + Cfg::KCH;

      // S^T = K Q^T for the 64 keys of the tile (two 32-key blocks)
      f32x16 sacc[QB][2];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[qb][kb][r] = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int row = 32 * kb + l32;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          Chunk<T> ka;
          ka.load(&ks[row * HC + ((2 * s + g2) ^ (row & 7))]);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) mma32(sacc[qb][kb], ka, qf[qb][s]);
        }
      }

      // online softmax (base 2, scale folded in)
      const bool tail = (j + 1) * ATT_BN > Lk;
      Chunk<T> pf[QB][4];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float sv = sacc[qb][kb][r] * a.scale_log2;
            if (tail) {
              int key = j * ATT_BN + 32 * kb + 8 * (r / 4) + 4 * g2 + (r % 4);
              if (key >= Lk) sv = -INFINITY;
            }
            sacc[qb][kb][r] = sv;
            mx = fmaxf(mx, sv);
          }
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float mnew = fmaxf(m[qb], mx);
        const bool need = mnew > m[qb] + RESCALE_THRESHOLD;
        if (__ballot(need) != 0) {
          const float alpha = __builtin_amdgcn_exp2f(m[qb] - mnew);
          m[qb] = mnew;
          l[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < ND; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[qb][db][r] *= alpha;
        }
        float ls = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            float p[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              p[e] = __builtin_amdgcn_exp2f(sacc[qb][kb][8 * half + e] - m[qb]);
              ls += p[e];
            }
            pack8(pf[qb][2 * kb + half], p);
          }
        l[qb] += ls;
      }

      // O^T += V^T P^T, four 16-key steps
#pragma unroll
      for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int db = 0; db < ND; ++db) {
          const int row = 32 * db + l32;
          Chunk<T> va;
          va.load(&vs[row * 8 + ((2 * u + g2) ^ (row & 7))]);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) mma32(o[qb][db], va, pf[qb][u]);
        }
      }

      if (j + 1 < nkt) store_tile(cur ^ 1);
      __syncthreads();
    }

    // normalise this source
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float lt = l[qb] + __shfl_xor(l[qb], 32, 64);
      const float inv = 1.0f / lt;
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float v = o[qb][db][r] * inv;
          if (NSRC == 2) {
            if (src == 0)
              o_prev[qb][db % (NSRC == 2 ? ND : 1)][r] = v;
            else
              v += o_prev[qb][db % (NSRC == 2 ? ND : 1)][r];
          }
          o[qb][db][r] = v;
        }
    }
  }

  // ---- epilogue: stage the wave's rows in LDS as [query][d], then 16-byte row stores
  T* st = reinterpret_cast<T*>(smem_raw) + wave * (32 * QB * HD);
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int d = 32 * db + 8 * (r / 4) + 4 * g2 + (r % 4);
        st[(32 * qb + l32) * HD + d] = from_f<T>(o[qb][db][r]);
      }
  __syncthreads();
  const int ld = a.heads * HD;
#pragma unroll
  for (int u = 0; u < (32 * QB * HC) / 64; ++u) {
    const int idx = lane + 64 * u;
    const int qr = idx / HC, c = idx % HC;
    const int q = q0 + qr;
    if (q < a.Lq) {
      Chunk<T> v;
      v.load(st + qr * HD + c * 8);
      v.store(reinterpret_cast<T*>(a.o) + ((long long)b * a.Lq + q) * ld + h * HD + c * 8);
    }
  }
}

template <typename T, int HD, int QB, int NSRC>
hipError_t launch_attn_cfg(const AttnArgs& a, hipStream_t st) {
  using Cfg = AttCfg<T, HD>;
  auto kern = attn_kernel<T, HD, QB, NSRC>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)Cfg::LDS_BYTES);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  constexpr int BMQ = 4 * 32 * QB;
  const int nqt = (a.Lq + BMQ - 1) / BMQ;
  const int G = nqt * a.heads * a.B;
  hipLaunchKernelGGL(kern, dim3(G), dim3(256), Cfg::LDS_BYTES, st, a);
  return hipGetLastError();
}

}  // namespace

template <typename T>
hipError_t launch_attention(const AttnArgs& a, hipStream_t st) {
  if (a.Lq <= 0) return hipSuccess;
  if (a.hd == 128) {
    if (a.nsrc == 1) return launch_attn_cfg<T, 128, 1, 1>(a, st);
    return launch_attn_cfg<T, 128, 1, 2>(a, st);
  }
  if (a.hd == 64) {
    if (a.nsrc == 1) return launch_attn_cfg<T, 64, 1, 1>(a, st);
    return launch_attn_cfg<T, 64, 1, 2>(a, st);
  }
  return hipErrorInvalidValue;
}

template hipError_t launch_attention<bf16>(const AttnArgs&, hipStream_t);
template hipError_t launch_attention<float>(const AttnArgs&, hipStream_t);

}  // namespace wan
