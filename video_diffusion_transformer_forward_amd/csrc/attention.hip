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
// K and V^T tiles of 64 keys are double-buffered in LDS (XOR-swizzled rows, so
// the 16 rows one 16-lane group of a wide LDS read touches hit distinct banks),
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

// Position of 16-byte chunk c in LDS row r.  A wave-wide 16-byte LDS read is
// served 16 lanes at a time: the 16 rows those lanes touch must land on 16
// distinct 16-byte bank groups (64 banks x 4 bytes = 256 bytes).
// CPR is the number of chunks (8 elements each) per row.
template <typename T, int CPR>
__device__ __forceinline__ int att_swz(int r, int c) {
  if constexpr (CPR >= 16)
    return c ^ (r & 15);                   // 256-byte (or longer) rows all start on bank 0
  else if constexpr (sizeof(T) == 2)
    return c ^ ((r >> 1) & 7);             // 128-byte rows: two rows per bank line
  else
    return c ^ (r & 7);                    // float, 8 chunks of 32 bytes
}

// Write a lane's share of O^T (query `row`; d = 32 db + 8 r4 + 4 g2 + 0..3) into
// the LDS rows [query][d] as 4-element stores, each at the swizzled 8-element
// chunk of its row, so that the 32 rows one store instruction touches spread over
// the banks (unswizzled, rows of 128 bf16 all start on bank 0: a 32-way conflict).
template <typename T, int HD>
__device__ __forceinline__ void stage_o_rows(T* stg, int row, int g2, const f32x16* o, float inv) {
  constexpr int HC = HD / 8;
#pragma unroll
  for (int db = 0; db < HD / 32; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      T* dst = stg + row * HD + att_swz<T, HC>(row, 4 * db + r4) * 8 + 4 * g2;
      const float v0 = o[db][4 * r4] * inv, v1 = o[db][4 * r4 + 1] * inv;
      const float v2 = o[db][4 * r4 + 2] * inv, v3 = o[db][4 * r4 + 3] * inv;
      if constexpr (sizeof(T) == 2)
        *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
      else
        *reinterpret_cast<f32x4*>(dst) = (f32x4){v0, v1, v2, v3};
    }
}

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

template <typename T, int HD, int NSRC, int KIND>
__device__ __forceinline__ void attn_body(const AttnArgs& a) {
  using Cfg = AttCfg<T, HD>;
  constexpr int HC = Cfg::HC;
  constexpr int SPC = Cfg::SPC;
  constexpr int CB = (int)sizeof(Chunk<T>);              // bytes per chunk
  constexpr int BMQ = 128;                               // queries per workgroup: 4 waves x 32
  constexpr int ND = HD / 32;                            // 32-row blocks of d in O^T
  constexpr int NS = HD / 16;                            // 16-deep k steps of S^T
  constexpr int STAGE_B = Cfg::STAGE * CB;               // bytes per LDS stage
  constexpr int KBLK_B = 32 * HC * CB;                   // bytes of 32 K rows
  constexpr int VBLK_B = 32 * 8 * CB;                    // bytes of 32 V^T rows
  extern __shared__ __align__(16) unsigned char smem_raw[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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

  // Per-lane LDS byte offsets of the MFMA operands.  The swizzle of row
  // 32*blk + l32 does not depend on blk, so the block and the stage enter as
  // immediate offsets of the LDS reads.
  int koff[NS], voff[4];
#pragma unroll
  for (int s = 0; s < NS; ++s) koff[s] = (l32 * HC + att_swz<T, HC>(l32, 2 * s + g2)) * CB;
#pragma unroll
  for (int u = 0; u < 4; ++u) voff[u] = Cfg::KCH * CB + (l32 * 8 + att_swz<T, 8>(l32, 2 * u + g2)) * CB;

  // Per-lane element offsets of the global -> LDS copies inside one tile.  Each
  // wave instruction fills 1 KB of LDS, lane l the l-th 16 bytes, so the XOR
  // swizzle of the chunk position is applied to the global address.
  int kdo[Cfg::K_DMA], vdo[Cfg::V_DMA];
#pragma unroll
  for (int i = 0; i < Cfg::K_DMA; ++i) {
    const int P = (wave * Cfg::K_DMA + i) * 64 + lane;
    const int pc = P / SPC, sub = P % SPC;
    const int r = pc / HC;
    kdo[i] = r * HD + att_swz<T, HC>(r, pc % HC) * 8 + sub * (8 / SPC);
  }

  f32x16 o[ND];
  f32x16 o_prev[NSRC == 2 ? ND : 1];

  for (int src = 0; src < NSRC; ++src) {
    const int Lk = a.Lk[src];
    const int Lkp = a.Lkp[src];
    const T* Kp = reinterpret_cast<const T*>(a.k[src]) + (long long)bh * Lkp * HD;
    const T* Vp = reinterpret_cast<const T*>(a.vt[src]) + (long long)bh * HD * Lkp;
    const int nkt = (Lk + ATT_BN - 1) / ATT_BN;
#pragma unroll
    for (int i = 0; i < Cfg::V_DMA; ++i) {
      const int P = (wave * Cfg::V_DMA + i) * 64 + lane;
      const int pc = P / SPC, sub = P % SPC;
      const int r = pc / 8;
      vdo[i] = r * Lkp + att_swz<T, 8>(r, pc % 8) * 8 + sub * (8 / SPC);
    }

    // copies through buffer resources based at this source's K and V^T of (batch item, head), so
    // that the waits for LDS operand reads stay counted (see the 256-query kernel below)
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)Kp, (short)0, -1, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)Vp, (short)0, -1, 0x00020000);
    auto issue = [&](int j, int stage) {
      unsigned char* kst = smem_raw + stage * STAGE_B;
#pragma unroll
      for (int i = 0; i < Cfg::K_DMA; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(kst + (wave * Cfg::K_DMA + i) * 1024), 16,
                                                 (unsigned)kdo[i] * (unsigned)sizeof(T),
                                                 j * ATT_BN * HD * (int)sizeof(T), 0, 0);
      unsigned char* vst = kst + Cfg::KCH * CB;
#pragma unroll
      for (int i = 0; i < Cfg::V_DMA; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(vst + (wave * Cfg::V_DMA + i) * 1024), 16,
                                                 (unsigned)vdo[i] * (unsigned)sizeof(T), j * ATT_BN * (int)sizeof(T),
                                                 0, 0);
    };

    float m = -INFINITY, l = 0.f;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] = 0.f;

    // one 64-key tile held in LDS stage `stage` (a literal after inlining)
    auto tile = [&](int j, int stage) {
      const unsigned char* sbase = smem_raw + stage * STAGE_B;
      // S^T = K Q^T for the 64 keys of the tile (two 32-key blocks)
      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          Chunk<T> ka;
          ka.load(sbase + kb * KBLK_B + koff[s]);
          if (s == 0) {
            f32x16 zero = {};
            sacc[kb] = zero;
          }
          mma32(sacc[kb], ka, qf[s]);
        }
      }
      // keys at or past Lk get -inf (only ever the last tile)
      if ((j + 1) * ATT_BN > Lk) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = j * ATT_BN + 32 * kb + 8 * (r / 4) + 4 * g2 + (r % 4);
            if (key >= Lk) sacc[kb][r] = -INFINITY;
          }
      }
      // online softmax in base 2; the scale enters through one FMA per score
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2)
          mx = __builtin_elementwise_maximum(mx, __builtin_elementwise_maximum(sacc[kb][r], sacc[kb][r + 1]));
      mx = __builtin_elementwise_maximum(mx, __shfl_xor(mx, 32, 64));
      const float mnew = __builtin_elementwise_maximum(m, mx);
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
          Chunk<T> va;
          va.load(sbase + db * VBLK_B + voff[u]);
          mma32(o[db], va, pf[u]);
        }
      }
    };

    issue(0, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    for (int j = 0; j < nkt; j += 2) {
      if (j + 1 < nkt) issue(j + 1, 1);
      tile(j, 0);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (j + 1 < nkt) {
        if (j + 2 < nkt) issue(j + 2, 0);
        tile(j + 1, 1);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
      }
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
  stage_o_rows<T, HD>(st, l32, g2, o, 1.0f);
  __syncthreads();
  const int ld = a.heads * HD;
#pragma unroll
  for (int u = 0; u < (32 * HC) / 64; ++u) {
    const int idx = lane + 64 * u;
    const int qr = idx / HC, cc = idx % HC;
    const int q = q0 + qr;
    if (q < a.Lq) {
      Chunk<T> v;
      v.load(st + qr * HD + att_swz<T, HC>(qr, cc) * 8);
      v.store(reinterpret_cast<T*>(a.o) + ((long long)b * a.Lq + q) * ld + h * HD + cc * 8);
    }
  }
}

// ---------------------------------------------------------------------------
// Self-attention in bf16, software-pipelined.
//
// A workgroup of NW waves owns NW*32*QB queries of one (batch, head) and shares
// every K / V^T tile among them (with NW = 8, two waves per SIMD and one
// workgroup per CU); a wave holds QB 32-query blocks, so each K or V^T fragment
// read from LDS feeds QB MFMAs.  The key-tile loop is software-pipelined inside
// the wave: while the matrix core computes the scores S(t+1) of the next tile,
// the VALU runs the softmax of tile t, and the P V products of tile t overlap
// the rest of it and the row maxima of S(t+1).  Since the scores of tile t+1
// and the values of tile t are read in the same iteration, K and V^T tiles live
// in two separate LDS rings of NR stages each.
constexpr int WIDE_NW = 8;  // waves per workgroup
constexpr int WIDE_QB = 1;  // 32-query blocks per wave
constexpr int WIDE_NR = 2;  // stages per K / V^T ring
constexpr int WIDE_NR_SM = 3;  // the static-offset kernel: three stages, barrier at slot 24

template <int HD, int NR, int QB, int NW>
struct WideCfg {
  static constexpr int WQ = 32 * QB;    // queries per wave
  static constexpr int BMQ = NW * WQ;   // queries per workgroup
  static constexpr int KT_B = ATT_BN * HD * 2;  // bytes per K tile
  static constexpr int VT_B = HD * ATT_BN * 2;  // bytes per V^T tile
  static constexpr int K_DMA = KT_B / (16 * 64 * NW);  // 16-byte loads per thread per tile
  static constexpr int V_DMA = VT_B / (16 * 64 * NW);
  static constexpr size_t RING_BYTES = (size_t)NR * (KT_B + VT_B);
  static constexpr size_t EPI_BYTES = (size_t)BMQ * HD * 2;
  static constexpr size_t LDS_BYTES = RING_BYTES > EPI_BYTES ? RING_BYTES : EPI_BYTES;
  static_assert(K_DMA * 16 * 64 * NW == KT_B && V_DMA * 16 * 64 * NW == VT_B, "DMA split");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

// s_waitcnt vmcnt(N) only (gfx9 encoding; the other counters at their maximum)
template <int N>
__device__ __forceinline__ void att_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier that waits for this wave's LDS reads but leaves its global
// loads in flight.
__device__ __forceinline__ void att_barrier_lds() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// SM (static offset): every query's exponent offset is fixed before the key sweep at
// m_q = |q| max_k |k| (by Cauchy-Schwarz no score exceeds it, so every probability is at
// most 1), which removes the per-tile row maxima, the running-max update and the
// rescaling of the accumulators.  q arrives multiplied by log2(e)/sqrt(d) (scale_log2 is 1),
// so the scores are in base-2 units, and the score accumulators start at -m_q: a
// probability is exp2 of the accumulator, with no per-score multiply-add.  The result is the same softmax; only its scale
// differs, and exactness needs the largest probability of a row to stay far above
// the smallest normal float: a workgroup with a row sum below 2^-64 (the offset
// overshot the true maximum by more than 64 in base 2) flags itself in a.fallback (one
// flag per wave, written whether set or not), and a second launch of the running-max
// kernel recomputes exactly those.
template <int HD, int NR, int QB, int NW, bool SM = false>
__device__ __forceinline__ void attn_wide_body(const AttnArgs& a) {
  using T = bf16;
  using Cfg = WideCfg<HD, NR, QB, NW>;
  constexpr int WQ = Cfg::WQ, BMQ = Cfg::BMQ;
  constexpr int HC = HD / 8;        // chunks per K row
  constexpr int CB = 16;            // bytes per chunk
  constexpr int ND = HD / 32;       // 32-row blocks of d in O^T
  constexpr int NS = HD / 16;       // 16-deep k steps of S^T
  constexpr int KBLK_B = 32 * HC * CB;
  constexpr int VBLK_B = 32 * 8 * CB;
  constexpr int VRING = NR * Cfg::KT_B;  // byte offset of the V^T ring
  constexpr int INFLIGHT = (NR - 2) * (Cfg::K_DMA + Cfg::V_DMA);
  static_assert(NR >= 2, "ring");
  extern __shared__ __align__(16) unsigned char smem_raw[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g2 = lane >> 5;
  const int l32 = lane & 31;

  const int nqt = (a.Lq + BMQ - 1) / BMQ;
  const int G = nqt * a.heads * a.B;
  const int id = xcd_remap(blockIdx.x, G);
  const int qt = id % nqt;
  const int bh = id / nqt;
  const int b = bh / a.heads;
  const int h = bh - b * a.heads;
  // second pass after the static-offset kernel: only the workgroups it flagged (one flag per wave)
  if (!SM && a.only) {
    int any = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) any |= a.only[id * NW + w];
    if (any == 0) return;
  }
  const int q0 = qt * BMQ + wave * WQ;
  const float c = a.scale_log2;
  const int Lk = a.Lk[0];
  const int Lkp = a.Lkp[0];
  const int n = (Lk + ATT_BN - 1) / ATT_BN;

  // queries of this wave, two 32-query blocks: B operand chunks (query l32, d chunk 2s + g2)
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

  // per-lane LDS byte offsets of the MFMA operands within a K tile / V^T tile
  int koff[NS], voff[4];
#pragma unroll
  for (int s = 0; s < NS; ++s) koff[s] = (l32 * HC + att_swz<T, HC>(l32, 2 * s + g2)) * CB;
#pragma unroll
  for (int u = 0; u < 4; ++u) voff[u] = (l32 * 8 + att_swz<T, 8>(l32, 2 * u + g2)) * CB;

  // per-lane byte offsets of the global -> LDS copies inside one tile (lane l of
  // a wave instruction fills the l-th 16 bytes of a 1 KB LDS block)
  unsigned kdo[Cfg::K_DMA], vdo[Cfg::V_DMA];
#pragma unroll
  for (int i = 0; i < Cfg::K_DMA; ++i) {
    const int P = (wave * Cfg::K_DMA + i) * 64 + lane;
    const int r = P / HC;
    kdo[i] = (unsigned)(r * HD + att_swz<T, HC>(r, P % HC) * 8) * 2u;
  }
#pragma unroll
  for (int i = 0; i < Cfg::V_DMA; ++i) {
    const int P = (wave * Cfg::V_DMA + i) * 64 + lane;
    const int r = P / 8;
    vdo[i] = (unsigned)(r * Lkp + att_swz<T, 8>(r, P % 8) * 8) * 2u;
  }
  // The copies go through buffer resources based at this (batch item, head)'s K and V^T (the
  // tile offset in the scalar offset).  Global-address LDS copies would count as both a memory
  // and an LDS access, and every later wait for an LDS operand read would then have to drain
  // all reads in flight (lgkmcnt(0)) instead of only the one it needs.
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(reinterpret_cast<const unsigned char*>(a.k[0]) + (long long)bh * Lkp * HD * 2), (short)0, -1, 0x00020000);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(reinterpret_cast<const unsigned char*>(a.vt[0]) + (long long)bh * HD * Lkp * 2), (short)0, -1, 0x00020000);

  auto issue_k = [&](int j, int stage) {
    unsigned char* dst = smem_raw + stage * Cfg::KT_B;
#pragma unroll
    for (int i = 0; i < Cfg::K_DMA; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(dst + (wave * Cfg::K_DMA + i) * 1024), 16, kdo[i],
                                               j * Cfg::KT_B, 0, 0);
  };
  auto issue_v = [&](int j, int stage) {
    unsigned char* dst = smem_raw + VRING + stage * Cfg::VT_B;
#pragma unroll
    for (int i = 0; i < Cfg::V_DMA; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(dst + (wave * Cfg::V_DMA + i) * 1024), 16, vdo[i],
                                               j * ATT_BN * 2, 0, 0);
  };

  f32x16 sinit[QB];  // initial score accumulators (set below, once the offsets are known)
  // S^T of one 32-key block kb of the K tile in stage kst, for both query blocks
  auto scores = [&](f32x16 (&s)[QB][2], int kst, int kb) {
    const unsigned char* kbase = smem_raw + kst * Cfg::KT_B + kb * KBLK_B;
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      Chunk<T> ka;
      ka.load(kbase + koff[st]);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        if (st == 0) s[qb][kb] = sinit[qb];
        mma32(s[qb][kb], ka, qf[qb][st]);
      }
    }
  };
  // keys at or past Lk get -inf (only ever the last tile)
  auto mask = [&](f32x16 (&s)[QB][2], int j) {
    if ((j + 1) * ATT_BN > Lk) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = j * ATT_BN + 32 * kb + 8 * (r / 4) + 4 * g2 + (r % 4);
            if (key >= Lk) s[qb][kb][r] = -INFINITY;
          }
    }
  };
  // row maxima of both query blocks (the two lanes of a query exchange theirs)
  auto rowmax = [&](const f32x16 (&s)[QB][2], float (&mx)[QB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float v = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2)
          v = __builtin_elementwise_maximum(v, __builtin_elementwise_maximum(s[qb][kb][r], s[qb][kb][r + 1]));
      mx[qb] = __builtin_elementwise_maximum(v, __shfl_xor(v, 32, 64));
    }
  };

  f32x16 o[QB][ND];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[qb][db][r] = 0.f;
  float m[QB], l[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m[qb] = -INFINITY;
    l[qb] = 0.f;
  }
  if constexpr (SM) {
    // m_q = |q| max_k |k|: |q| from the bf16 values the MFMAs multiply, max |k| from the keys
    // before their rounding to bf16 (which moves a norm by at most 2^-9 of itself); the
    // factor 1 + 2^-8 covers that and the float32 rounding of the norms and score sums
    float k2 = 0.f;
    for (int i = lane; i < a.kpart_n; i += 64) k2 = __builtin_elementwise_maximum(k2, a.kpart[(long long)bh * a.kpart_n + i]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) k2 = __builtin_elementwise_maximum(k2, __shfl_xor(k2, o, 64));
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float q2 = 0.f;
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        const bf16x8 e = as_bf16x8(qf[qb][st].v);
#pragma unroll
        for (int u = 0; u < 8; ++u) q2 = __builtin_fmaf((float)e[u], (float)e[u], q2);
      }
      q2 += __shfl_xor(q2, 32, 64);
      m[qb] = sqrtf(q2 * k2) * (1.0f + 1.0f / 256.0f);
    }
  }
  // score accumulators start at 0, or (static offset, q pre-scaled by log2(e)/sqrt(d)) at -m_q,
  // so that the probability is exp2 of the accumulator itself
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int r = 0; r < 16; ++r) sinit[qb][r] = SM ? -m[qb] : 0.f;

  // Lazy running max: a query's max moves only when its tile max exceeds it by
  // more than 2^8; its sum is then scaled by alpha at once, the accumulators
  // (only when some lane of the wave moved) once the pending P V products are in.
  float alpha[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) alpha[qb] = 1.0f;
  auto new_max = [&](const float (&mx)[QB]) {
    bool moved = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float mnew = __builtin_elementwise_maximum(m[qb], mx[qb]);
      const bool mv = (mnew - m[qb]) * c > RESCALE_LOG2;
      const float al = __builtin_amdgcn_exp2f((m[qb] - mnew) * c);
      alpha[qb] = mv ? al : 1.0f;
      m[qb] = mv ? mnew : m[qb];
      l[qb] *= alpha[qb];
      moved = moved || mv;
    }
    return __ballot(moved) != 0;
  };
  auto scale_o = [&]() {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[qb][db][r] *= alpha[qb];
  };
  // probabilities of 32-key block kb for both query blocks -> B operand chunks pf[qb][2kb], pf[qb][2kb+1]
  auto probs = [&](const f32x16 (&s)[QB][2], int kb, Chunk<T> (&pf)[QB][4]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float nmc = -m[qb] * c;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = SM ? __builtin_amdgcn_exp2f(s[qb][kb][8 * half + e])
                    : __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][kb][8 * half + e], c, nmc));
          l[qb] += p[e];
        }
        pack8(pf[qb][2 * kb + half], p);
      }
    }
  };
  // O^T += V^T P^T over 16-key steps u0, u0+1 of the V^T tile in stage vst
  auto pv = [&](int vst, int u0, const Chunk<T> (&pf)[QB][4]) {
    const unsigned char* vbase = smem_raw + VRING + vst * Cfg::VT_B;
#pragma unroll
    for (int u = u0; u < u0 + 2; ++u)
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        Chunk<T> va;
        va.load(vbase + db * VBLK_B + voff[u]);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) mma32(o[qb][db], va, pf[qb][u]);
      }
  };

  // Values computed in one phase and consumed in a later one are pinned where
  // they are produced (an empty asm that takes them in registers); otherwise the
  // compiler sinks their arithmetic next to the consuming MFMAs and the phases
  // no longer overlap VALU work with matrix work.

  // ---- prologue: K_0..K_{NR-1} and V_0..V_{NR-2} in flight; S(0), its maxima and
  // the probabilities of its first 32 keys
#pragma unroll
  for (int j = 0; j < NR; ++j) issue_k(min(j, n - 1), j);
#pragma unroll
  for (int j = 0; j < NR - 1; ++j) issue_v(min(j, n - 1), j);
  att_wait_vmcnt<0>();
  __syncthreads();
  f32x16 S[QB][2];
  Chunk<T> pf[QB][4];
  float mx[QB];
  auto pin_probs = [&](int kb) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) asm volatile("" : "+v"(pf[qb][2 * kb].v), "+v"(pf[qb][2 * kb + 1].v));
  };
  auto pin_stats = [&]() {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) asm volatile("" : "+v"(m[qb]), "+v"(l[qb]), "+v"(alpha[qb]), "+v"(mx[qb]));
  };
  scores(S, 0, 0);
  scores(S, 0, 1);
  mask(S, 0);
  if constexpr (!SM) {
    rowmax(S, mx);
    new_max(mx);  // first tile: the max moves from -inf, sums and accumulators are still zero
  }
  probs(S, 0, pf);
  // MB (static offset, three-stage rings): the workgroup barrier sits at slot 24 of an
  // iteration, and slots 24..31 already read the first 8 operands of the next iteration
  // (K_{t+2}, keys 0..31) into `carry`; here the prologue reads those of iteration 0
  constexpr bool MB = SM && NR == 3;
  Chunk<T> carry[8];
  if constexpr (MB) {
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8) carry[s8].load(smem_raw + 1 * Cfg::KT_B + koff[s8]);
  }
  att_barrier_lds();  // K stage 0 is refilled by the first iteration

  // One iteration, entered with the scores S(t) of tile t in S and the
  // probabilities of its first 32 keys in pf[.][0..1].  The MFMAs of a
  // wave run as 32 slots (QB MFMAs each, one per query block), each issuing the
  // LDS read of the operand needed 8 slots later and a share of the VALU work:
  //   slots  0..7   S(t+1), keys 0..31    | probabilities of tile t, keys 32..63
  //   slots  8..15  S(t+1), keys 32..63   | masking and row maxima of S(t+1), keys 0..31
  //   slots 16..23  O += P V, keys 0..31  | masking and row maxima, keys 32..63; new max
  //   slots 24..31  O += P V, keys 32..63 | probabilities of tile t+1, keys 0..31
  // K_{t+1} sits in K stage (t+1)%NR, V_t in V stage t%NR.  The loads issued here
  // refill the stages read in the previous iteration: K_{t+NR} and V_{t+NR-1}
  // (indices clamped at the last tile; those copies are never read).  Past the
  // last tile S(n) is computed from a stale stage but masked out entirely.
  // `ph` = t % NR, a literal after inlining, so every LDS offset is an immediate.
  // A scheduling barrier closes every slot; values consumed in a later slot are
  // pinned where they are produced.  The static-offset form orders its slots
  // differently (see the slot loop) and, with three-stage rings, synchronises the
  // workgroup at slot 24 instead of at the end of the iteration.
  auto iter = [&](int t, int ph) {
    const int kst = (ph + 1) % NR, vst = ph;
    issue_k(min(t + NR, n - 1), ph);
    issue_v(min(t + NR - 1, n - 1), (ph + NR - 1) % NR);
    const unsigned char* kbase = smem_raw + kst * Cfg::KT_B;
    const unsigned char* vbase = smem_raw + VRING + vst * Cfg::VT_B;
    // operand of slot i: K block i/8 step i%8, then V^T 16-key step (i-16)/4, d block (i-16)%4.
    // With the static offset the slots alternate instead: K block 0, V^T keys 0..31, K block 1,
    // V^T keys 32..63 (see the slot loop below)
    auto raddr = [&](int i) -> const unsigned char* {
      if constexpr (SM) {
        if ((i & 8) == 0) return kbase + (i / 16) * KBLK_B + koff[i % 8];
        const int v = (i / 16) * 8 + (i % 8);
        return vbase + (v % 4) * VBLK_B + voff[v / 4];
      }
      if (i < 16) return kbase + (i / 8) * KBLK_B + koff[i % 8];
      return vbase + ((i - 16) % 4) * VBLK_B + voff[(i - 16) / 4];
    };
    constexpr int AHEAD = 8;
    static_assert(!MB || AHEAD == 8, "carry holds the 8 reads issued in slots 24..31");
    Chunk<T> rf[32];
#pragma unroll
    for (int i = 0; i < AHEAD; ++i) {
      if constexpr (MB)
        rf[i] = carry[i];
      else
        rf[i].load(raddr(i));
    }
    const unsigned char* knext = smem_raw + ((ph + 2) % NR) * Cfg::KT_B;  // K_{t+2} (MB only)
    const bool mask_next = (t + 2) * ATT_BN > Lk;
    float nmc[QB], vmax[QB], pbuf[QB][8];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      nmc[qb] = -m[qb] * c;
      vmax[qb] = -INFINITY;
    }
    bool moved = false;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if constexpr (MB) {
        if (i == 24) {
          // K_{t+2} and V_{t+1} (copied during the previous iteration) have landed; after the
          // barrier every wave has finished its reads of K_{t+1} (last used in slot 23) and
          // of V_t (its reads for slots 24..31 were issued by slot 23 and are waited here),
          // the stages the next iteration refills
          att_wait_vmcnt<INFLIGHT>();
          att_barrier_lds();
        }
        if (i + AHEAD < 32)
          rf[i + AHEAD].load(raddr(i + AHEAD));
        else
          carry[i + AHEAD - 32].load(knext + koff[i + AHEAD - 32]);
      } else {
        if (i + AHEAD < 32) rf[i + AHEAD].load(raddr(i + AHEAD));
      }
      if constexpr (SM) {
        // Static offset: no row maxima, so the only VALU work is one exp2 (and its sum) per
        // score, spread over every slot.  The two waves of a SIMD start each tile together
        // (one barrier per tile); with the exp2 work in half of the slots both waves issued
        // it at once while the other half had none.
        //   slots  0..7   S(t+1), keys 0..31    | probabilities of tile t, keys 32..63 (1st half)
        //   slots  8..15  O += P V, keys 0..31  | probabilities of tile t, keys 32..63 (2nd half)
        //   slots 16..23  S(t+1), keys 32..63   | masking of S(t+1) keys 0..31 at 16; probabilities of
        //   slots 24..31  O += P V, keys 32..63 |   tile t+1, keys 0..31 (masking of its keys 32..63 at 24)
        // S(t) keys 32..63 are read in slots 0..15, before the MFMAs of slots 16..23 overwrite
        // them; P(t) keys 0..31 are read by slots 8..15, before slot 23 repacks them for t+1.
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          if ((i & 8) == 0) {
            const int kb = i / 16, st = i % 8;
            if (st == 0) S[qb][kb] = sinit[qb];
            mma32(S[qb][kb], rf[i], qf[qb][st]);
          } else {
            const int v = (i / 16) * 8 + (i % 8);
            mma32(o[qb][v % 4], rf[i], pf[qb][v / 4]);
          }
        }
        if ((i == 16 || i == 24) && mask_next) {
          const int kb = i == 16 ? 0 : 1;
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = (t + 1) * ATT_BN + 32 * kb + 8 * (r / 4) + 4 * g2 + (r % 4);
              if (key >= Lk) S[qb][kb][r] = -INFINITY;
            }
        }
        {
          const int kb = i < 16 ? 1 : 0, e = i % 16;
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            pbuf[qb][e % 8] = __builtin_amdgcn_exp2f(S[qb][kb][e]);
            l[qb] += pbuf[qb][e % 8];
            if (e % 8 == 7) {
              const int c8 = (kb == 1 ? 2 : 0) + e / 8;
              pack8(pf[qb][c8], pbuf[qb]);
              asm volatile("" : "+v"(pf[qb][c8].v), "+v"(l[qb]));
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        continue;
      }
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        if (i < 16) {
          const int kb = i / 8, st = i % 8;
          if (st == 0) S[qb][kb] = sinit[qb];
          mma32(S[qb][kb], rf[i], qf[qb][st]);
        } else {
          const int u = (i - 16) / 4, db = (i - 16) % 4;
          mma32(o[qb][db], rf[i], pf[qb][u]);
        }
      }
      if (i < 8) {
        // probabilities of tile t, keys 32..63: elements 2i, 2i+1 of S(t) block 1
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
          for (int e = 2 * i; e < 2 * i + 2; ++e) {
            pbuf[qb][e % 8] = SM ? __builtin_amdgcn_exp2f(S[qb][1][e])
                                 : __builtin_amdgcn_exp2f(__builtin_fmaf(S[qb][1][e], c, nmc[qb]));
            l[qb] += pbuf[qb][e % 8];
          }
          if (i % 4 == 3) {
            pack8(pf[qb][2 + i / 4], pbuf[qb]);
            asm volatile("" : "+v"(pf[qb][2 + i / 4].v), "+v"(l[qb]));
          }
        }
      } else if (i < 24) {
        // row maxima of S(t+1): block 0 in slots 8..15, block 1 in slots 16..23
        const int kb = (i - 8) / 8, k = (i - 8) % 8;
        if (k == 0 && mask_next) {
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = (t + 1) * ATT_BN + 32 * kb + 8 * (r / 4) + 4 * g2 + (r % 4);
              if (key >= Lk) S[qb][kb][r] = -INFINITY;
            }
        }
        if constexpr (!SM) {
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            vmax[qb] = __builtin_elementwise_maximum(
                vmax[qb], __builtin_elementwise_maximum(S[qb][kb][2 * k], S[qb][kb][2 * k + 1]));
            asm volatile("" : "+v"(vmax[qb]));
          }
          if (i == 23) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) mx[qb] = __builtin_elementwise_maximum(vmax[qb], __shfl_xor(vmax[qb], 32, 64));
            moved = new_max(mx);
            pin_stats();
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
              nmc[qb] = -m[qb] * c;
              asm volatile("" : "+v"(nmc[qb]));
            }
          }
        }
      } else {
        // probabilities of tile t+1, keys 0..31: elements 2(i-24), +1 of S(t+1) block 0
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
          for (int e = 2 * (i - 24); e < 2 * (i - 24) + 2; ++e) {
            pbuf[qb][e % 8] = SM ? __builtin_amdgcn_exp2f(S[qb][0][e])
                                 : __builtin_amdgcn_exp2f(__builtin_fmaf(S[qb][0][e], c, nmc[qb]));
            l[qb] += pbuf[qb][e % 8];
          }
          if (i % 4 == 3) {
            pack8(pf[qb][(i - 24) / 4], pbuf[qb]);
            asm volatile("" : "+v"(pf[qb][(i - 24) / 4].v), "+v"(l[qb]));
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (moved) scale_o();
    if constexpr (!MB) {
      att_wait_vmcnt<INFLIGHT>();  // K_{t+2} and V_{t+1} have landed
      att_barrier_lds();
    }
  };
  static_assert(NR == 2 || NR == 4 || (NR == 3 && SM), "ring depth");
  for (int t = 0; t < n; t += NR) {
    iter(t, 0);
    if (t + 1 < n) iter(t + 1, 1);
    if constexpr (NR >= 3) {
      if (t + 2 < n) iter(t + 2, 2);
    }
    if constexpr (NR == 4) {
      if (t + 3 < n) iter(t + 3, 3);
    }
  }
  att_wait_vmcnt<0>();
  __syncthreads();
  if constexpr (SM) {
    // a row sum below 2^-64: the static offset overshot this row's largest score by more
    // than 64 in base 2, so its terms may have fallen below the normal floats
    bool low = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) low = low || (l[qb] + __shfl_xor(l[qb], 32, 64)) < 0x1p-64f;
    const int flag = __ballot(low) != 0 ? 1 : 0;
    if (lane == 0) a.fallback[id * NW + wave] = flag;  // written every time: no clearing needed
  }

  // ---- epilogue: normalise, stage the wave's 64 rows in LDS as [query][d], 16-byte row stores
  T* stg = reinterpret_cast<T*>(smem_raw) + wave * (WQ * HD);
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float inv = 1.0f / (l[qb] + __shfl_xor(l[qb], 32, 64));
    stage_o_rows<T, HD>(stg, 32 * qb + l32, g2, o[qb], inv);
  }
  __syncthreads();
  const int ld = a.heads * HD;
#pragma unroll
  for (int u = 0; u < (WQ * HC) / 64; ++u) {
    const int idx = lane + 64 * u;
    const int qr = idx / HC, cc = idx % HC;
    const int q = q0 + qr;
    if (q < a.Lq) {
      Chunk<T> v;
      v.load(stg + qr * HD + att_swz<T, HC>(qr, cc) * 8);
      v.store(reinterpret_cast<T*>(a.o) + ((long long)b * a.Lq + q) * ld + h * HD + cc * 8);
    }
  }
}

// ---- self-attention with 8-bit scores
//
// q and k arrive as e4m3 bytes with one power-of-two scale per (token, head)
// (an E8M0 byte, exponent + 127).  S^T = K Q^T runs on the scaled fp8 MFMA
// (32x32x64), which multiplies in the key's and the query's scale itself, so
// the scores are those of the dequantised rows up to float32 summation.  A
// 32-key block of S over the 128-wide head is two such MFMAs (64 cycles each,
// against eight bf16 MFMAs of 32 cycles), so a 64-key tile costs 256 matrix
// cycles for S and 512 for the bf16 P V products.  The rest follows the bf16
// kernel above: 8 waves of 32 queries share K / V^T rings in LDS, the
// softmax of tile t overlaps the scores of tile t+1 and the P V products.
// Both halves of a lane pair (l, l+32) pass the same scale byte, so the scale
// covers the whole head whatever k-order the MFMA gives its operand bytes.
template <int NR, int NW>
struct Wide8Cfg {
  static constexpr int HD = 128;
  static constexpr int BMQ = NW * 32;                 // queries per workgroup
  static constexpr int KT_B = ATT_BN * HD;            // bytes per fp8 K tile
  static constexpr int VT_B = HD * ATT_BN * 2;        // bytes per bf16 V^T tile
  static constexpr int KS_B = 256;                    // key-scale bytes per stage (64 used)
  static constexpr int K_DMA = KT_B / (16 * 64 * NW);
  static constexpr int V_DMA = VT_B / (16 * 64 * NW);
  static constexpr int VRING = NR * KT_B;
  static constexpr int SRING = VRING + NR * VT_B;
  static constexpr size_t RING_BYTES = (size_t)SRING + NR * KS_B;
  static constexpr size_t EPI_BYTES = (size_t)BMQ * HD * 2;
  static constexpr size_t LDS_BYTES = RING_BYTES > EPI_BYTES ? RING_BYTES : EPI_BYTES;
  static_assert(K_DMA * 16 * 64 * NW == KT_B && V_DMA * 16 * 64 * NW == VT_B, "DMA split");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

typedef int i32x8 __attribute__((ext_vector_type(8)));

// 32 operand bytes from two 16-byte LDS / global reads
__device__ __forceinline__ i32x8 load32(const unsigned char* lo, const unsigned char* hi) {
  const u32x4 a = *reinterpret_cast<const u32x4*>(lo);
  const u32x4 b = *reinterpret_cast<const u32x4*>(hi);
  return __builtin_bit_cast(i32x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// S^T(32 keys x 32 queries) += K8 Q8^T over 64 head features, scales per key row / query column
__device__ __forceinline__ void mma8(f32x16& acc, const i32x8& k, const i32x8& q, int kscale, int qscale) {
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(k, q, acc, 0, 0, 0, kscale, 0, qscale);
}

// SM: the static offset of the bf16 kernel above, with the dequantised q (e4m3 bytes times
// their power-of-two scale) and max |k| taken before the e4m3 rounding of k, whose relative
// error (at most 2^-4 per element, far less on the norm of a 128-wide row scaled to its
// maximum) the factor 1 + 2^-3 covers.  q is rounded to e4m3 as projected (a prior scaling
// by log2(e)/sqrt(d) would change its rounded bytes), so the offset is in score units and
// each probability is exp2(c S) with S seeded at -m_q: one multiply per score.
template <int NR, int NW, bool SM = false>
__device__ __forceinline__ void attn_wide8_body(const AttnArgs& a) {
  using T = bf16;
  using Cfg = Wide8Cfg<NR, NW>;
  constexpr int HD = Cfg::HD, BMQ = Cfg::BMQ;
  constexpr int ND = HD / 32;              // 32-row blocks of d in O^T
  constexpr int KBLK_B = 32 * HD;          // bytes per 32-key block of a K tile
  constexpr int VBLK_B = 32 * 8 * 16;      // bytes per 32-row block of a V^T tile
  static_assert(NR == 2, "ring depth");
  extern __shared__ __align__(16) unsigned char smem_raw[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g2 = lane >> 5;
  const int l32 = lane & 31;

  const int nqt = (a.Lq + BMQ - 1) / BMQ;
  const int G = nqt * a.heads * a.B;
  const int id = xcd_remap(blockIdx.x, G);
  const int qt = id % nqt;
  const int bh = id / nqt;
  const int b = bh / a.heads;
  const int h = bh - b * a.heads;
  // second pass after the static-offset kernel: only the workgroups it flagged (one flag per wave)
  if (!SM && a.only) {
    int any = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) any |= a.only[id * NW + w];
    if (any == 0) return;
  }
  const int q0 = qt * BMQ + wave * 32;
  const float c = a.scale_log2;
  const int Lk = a.Lk[0];
  const int Lkp = a.Lkp[0];
  const int n = (Lk + ATT_BN - 1) / ATT_BN;

  // the wave's 32 queries: operand of MFMA s = bytes [64s + 32 g2, +32) of query l32, and its scale
  i32x8 qf[2];
  int qsc = 127;
  {
    const int qrow = q0 + l32;
    if (qrow < a.Lq) {
      const unsigned char* qp = reinterpret_cast<const unsigned char*>(a.q) + ((long long)bh * a.Lqp + qrow) * HD;
#pragma unroll
      for (int s = 0; s < 2; ++s) qf[s] = load32(qp + 64 * s + 32 * g2, qp + 64 * s + 32 * g2 + 16);
      qsc = a.qs[(long long)bh * a.Lqp + qrow];
    } else {
      const i32x8 zero = {};
      qf[0] = zero;
      qf[1] = zero;
    }
  }

  // LDS offsets: K rows are 128 bytes (8 chunks, swizzled as 128-byte bf16 rows)
  int koff[2][2], voff[4];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) koff[s][hf] = (l32 * 8 + att_swz<T, 8>(l32, 4 * s + 2 * g2 + hf)) * 16;
#pragma unroll
  for (int u = 0; u < 4; ++u) voff[u] = (l32 * 8 + att_swz<T, 8>(l32, 2 * u + g2)) * 16;

  unsigned kdo[Cfg::K_DMA], vdo[Cfg::V_DMA];
#pragma unroll
  for (int i = 0; i < Cfg::K_DMA; ++i) {
    const int P = (wave * Cfg::K_DMA + i) * 64 + lane;
    const int r = P / 8;
    kdo[i] = (unsigned)(r * HD + att_swz<T, 8>(r, P % 8) * 16);
  }
#pragma unroll
  for (int i = 0; i < Cfg::V_DMA; ++i) {
    const int P = (wave * Cfg::V_DMA + i) * 64 + lane;
    const int r = P / 8;
    vdo[i] = (unsigned)(r * Lkp + att_swz<T, 8>(r, P % 8) * 8) * 2u;
  }
  // buffer-resource copies, as in the bf16 kernel (the waits for LDS operand reads stay counted)
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(reinterpret_cast<const unsigned char*>(a.k[0]) + (long long)bh * Lkp * HD), (short)0, -1, 0x00020000);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(reinterpret_cast<const unsigned char*>(a.vt[0]) + (long long)bh * HD * Lkp * 2), (short)0, -1, 0x00020000);
  // key scales: wave 0 copies a tile's 64 bytes (lanes past 15 repeat the last word)
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)(a.ks + (long long)bh * Lkp), (short)0, -1,
                                                                      0x00020000);
  const unsigned sdo = 4u * (unsigned)(lane < 16 ? lane : 15);

  auto issue_k = [&](int j, int stage) {
    unsigned char* dst = smem_raw + stage * Cfg::KT_B;
#pragma unroll
    for (int i = 0; i < Cfg::K_DMA; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(dst + (wave * Cfg::K_DMA + i) * 1024), 16, kdo[i],
                                               j * Cfg::KT_B, 0, 0);
    if (wave == 0)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(smem_raw + Cfg::SRING + stage * Cfg::KS_B), 4, sdo,
                                               j * ATT_BN, 0, 0);
  };
  auto issue_v = [&](int j, int stage) {
    unsigned char* dst = smem_raw + Cfg::VRING + stage * Cfg::VT_B;
#pragma unroll
    for (int i = 0; i < Cfg::V_DMA; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(dst + (wave * Cfg::V_DMA + i) * 1024), 16, vdo[i],
                                               j * ATT_BN * 2, 0, 0);
  };
  auto kscale = [&](int kst, int kb) -> int { return smem_raw[Cfg::SRING + kst * Cfg::KS_B + 32 * kb + l32]; };

  f32x16 o[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  float m = -INFINITY, l = 0.f, alpha = 1.f;
  if constexpr (SM) {
    float k2 = 0.f;
    for (int i = lane; i < a.kpart_n; i += 64) k2 = __builtin_elementwise_maximum(k2, a.kpart[(long long)bh * a.kpart_n + i]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) k2 = __builtin_elementwise_maximum(k2, __shfl_xor(k2, o, 64));
    // |q|^2 of the dequantised query: this lane's 64 e4m3 bytes, the other half from lane ^ 32
    float q2 = 0.f;
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const int word = qf[s][w];
        const float e0 = __builtin_amdgcn_cvt_f32_fp8(word, 0), e1 = __builtin_amdgcn_cvt_f32_fp8(word, 1);
        const float e2 = __builtin_amdgcn_cvt_f32_fp8(word, 2), e3 = __builtin_amdgcn_cvt_f32_fp8(word, 3);
        q2 = __builtin_fmaf(e0, e0, __builtin_fmaf(e1, e1, __builtin_fmaf(e2, e2, __builtin_fmaf(e3, e3, q2))));
      }
    q2 += __shfl_xor(q2, 32, 64);
    const float qs = __uint_as_float((unsigned)qsc << 23);  // 2^(qsc - 127)
    m = sqrtf(q2 * k2) * qs * (1.0f + 1.0f / 8.0f);
  }
  // score accumulators start at 0, or (static offset, in score units) at -m_q
  f32x16 sinit;
#pragma unroll
  for (int r = 0; r < 16; ++r) sinit[r] = SM ? -m : 0.f;

  // lazy running max, as in the bf16 kernel
  auto new_max = [&](float mx) {
    const float mnew = __builtin_elementwise_maximum(m, mx);
    const bool mv = (mnew - m) * c > RESCALE_LOG2;
    const float al = __builtin_amdgcn_exp2f((m - mnew) * c);
    alpha = mv ? al : 1.0f;
    m = mv ? mnew : m;
    l *= alpha;
    return __ballot(mv) != 0;
  };
  auto mask_block = [&](f32x16& s, int j, int kb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = j * ATT_BN + 32 * kb + 8 * (r / 4) + 4 * g2 + (r % 4);
      if (key >= Lk) s[r] = -INFINITY;
    }
  };

  // S(t) lives in S0 (keys 0..31) and S1[t % 2] (keys 32..63): the probabilities
  // of keys 32..63 of tile t are taken while S(t+1) is computed
  f32x16 S0, S1[2];
  Chunk<T> pf[4];

  // ---- prologue
#pragma unroll
  for (int j = 0; j < NR; ++j) issue_k(min(j, n - 1), j);
#pragma unroll
  for (int j = 0; j < NR - 1; ++j) issue_v(min(j, n - 1), j);
  att_wait_vmcnt<0>();
  __syncthreads();
  {
    S0 = sinit;
    S1[0] = sinit;
    const int ks0 = kscale(0, 0), ks1 = kscale(0, 1);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      mma8(S0, load32(smem_raw + koff[s][0], smem_raw + koff[s][1]), qf[s], ks0, qsc);
      mma8(S1[0], load32(smem_raw + KBLK_B + koff[s][0], smem_raw + KBLK_B + koff[s][1]), qf[s], ks1, qsc);
    }
    if (ATT_BN > Lk) {
      mask_block(S0, 0, 0);
      mask_block(S1[0], 0, 1);
    }
    if constexpr (!SM) {
      float v = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) v = __builtin_elementwise_maximum(v, __builtin_elementwise_maximum(S0[r], S1[0][r]));
      new_max(__builtin_elementwise_maximum(v, __shfl_xor(v, 32, 64)));
    }
    const float nmc = -m * c;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = SM ? __builtin_amdgcn_exp2f(S0[8 * half + e] * c) : __builtin_amdgcn_exp2f(__builtin_fmaf(S0[8 * half + e], c, nmc));
        l += p[e];
      }
      pack8(pf[half], p);
    }
  }
  att_barrier_lds();

  // One iteration, entered with S(t) and the probabilities of its keys 0..31 in
  // pf[0..1].  20 MFMA slots, each issuing the LDS read of the operand needed 6
  // slots later and a share of the VALU work:
  //   slots  0..3   S(t+1) (4 fp8 MFMAs)  | probabilities of tile t, keys 32..47
  //   slots  4..11  O += P V, keys 0..31  | probabilities of keys 48..63 (4..7);
  //                                         masking and row maxima of S(t+1) (8..11), new max
  //   slots 12..19  O += P V, keys 32..63 | probabilities of tile t+1, keys 0..31
  // K_{t+1} (and its scales) sit in K stage (t+1)%2, V_t in V stage t%2; the
  // loads issued here refill the stages read in the previous iteration.
  auto iter = [&](int t, int ph) {
    const int kst = (ph + 1) % NR, vst = ph;
    issue_k(min(t + NR, n - 1), ph);
    issue_v(min(t + NR - 1, n - 1), (ph + NR - 1) % NR);
    const unsigned char* kbase = smem_raw + kst * Cfg::KT_B;
    const unsigned char* vbase = smem_raw + Cfg::VRING + vst * Cfg::VT_B;
    f32x16& Sc = S1[ph];       // S(t), keys 32..63
    f32x16& Sn = S1[ph ^ 1];   // S(t+1), keys 32..63
    constexpr int AHEAD = 6;
    i32x8 kf[4];
    Chunk<T> vf[20];
    auto rd = [&](int i) {
      if (i < 4)
        kf[i] = load32(kbase + (i / 2) * KBLK_B + koff[i % 2][0], kbase + (i / 2) * KBLK_B + koff[i % 2][1]);
      else
        vf[i].load(vbase + ((i - 4) % 4) * VBLK_B + voff[(i - 4) / 4]);
    };
#pragma unroll
    for (int i = 0; i < AHEAD; ++i) rd(i);
    const int ks0 = kscale(kst, 0), ks1 = kscale(kst, 1);
    const bool mask_next = (t + 2) * ATT_BN > Lk;
    float nmc = -m * c, vmax = -INFINITY, pbuf[8];
    bool moved = false;
#pragma unroll
    for (int i = 0; i < 20; ++i) {
      if (i + AHEAD < 20) rd(i + AHEAD);
      if (i < 4) {
        const int kb = i / 2, s = i % 2;
        if (s == 0) {
          if (kb == 0) S0 = sinit; else Sn = sinit;
        }
        if (kb == 0) mma8(S0, kf[i], qf[s], ks0, qsc);
        else mma8(Sn, kf[i], qf[s], ks1, qsc);
      } else {
        const int u = (i - 4) / 4, db = (i - 4) % 4;
        mma32(o[db], vf[i], pf[u]);
      }
      if (i < 8) {
        // probabilities of tile t, keys 32..63: elements 2i, 2i+1 of Sc
#pragma unroll
        for (int e = 2 * i; e < 2 * i + 2; ++e) {
          pbuf[e % 8] = SM ? __builtin_amdgcn_exp2f(Sc[e] * c) : __builtin_amdgcn_exp2f(__builtin_fmaf(Sc[e], c, nmc));
          l += pbuf[e % 8];
        }
        if (i % 4 == 3) {
          pack8(pf[2 + i / 4], pbuf);
          asm volatile("" : "+v"(pf[2 + i / 4].v), "+v"(l));
        }
      } else if (i < 12) {
        // row maxima of S(t+1): keys 0..31 in slots 8, 9; keys 32..63 in slots 10, 11
        const int kb = (i - 8) / 2, k = (i - 8) % 2;
        f32x16& Sb = kb == 0 ? S0 : Sn;
        if (k == 0 && mask_next) mask_block(Sb, t + 1, kb);
        if constexpr (!SM) {
#pragma unroll
          for (int r = 8 * k; r < 8 * k + 8; r += 2)
            vmax = __builtin_elementwise_maximum(vmax, __builtin_elementwise_maximum(Sb[r], Sb[r + 1]));
          asm volatile("" : "+v"(vmax));
          if (i == 11) {
            moved = new_max(__builtin_elementwise_maximum(vmax, __shfl_xor(vmax, 32, 64)));
            nmc = -m * c;
            asm volatile("" : "+v"(m), "+v"(l), "+v"(alpha), "+v"(nmc));
          }
        }
      } else {
        // probabilities of tile t+1, keys 0..31: elements 2(i-12), +1 of S0
#pragma unroll
        for (int e = 2 * (i - 12); e < 2 * (i - 12) + 2; ++e) {
          pbuf[e % 8] = SM ? __builtin_amdgcn_exp2f(S0[e] * c) : __builtin_amdgcn_exp2f(__builtin_fmaf(S0[e], c, nmc));
          l += pbuf[e % 8];
        }
        if (i % 4 == 3) {
          pack8(pf[(i - 12) / 4], pbuf);
          asm volatile("" : "+v"(pf[(i - 12) / 4].v), "+v"(l));
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (moved) {
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
    }
    att_wait_vmcnt<0>();  // K_{t+2} (with scales) and V_{t+1} have landed
    att_barrier_lds();
  };
  for (int t = 0; t < n; t += 2) {
    iter(t, 0);
    if (t + 1 < n) iter(t + 1, 1);
  }
  att_wait_vmcnt<0>();
  __syncthreads();
  if constexpr (SM) {
    const int flag = __ballot((l + __shfl_xor(l, 32, 64)) < 0x1p-64f) != 0 ? 1 : 0;
    if (lane == 0) a.fallback[id * NW + wave] = flag;
  }

  // ---- epilogue: normalise, stage the wave's 32 rows in LDS as [query][d], 16-byte row stores
  constexpr int HC = HD / 8;
  T* stg = reinterpret_cast<T*>(smem_raw) + wave * (32 * HD);
  {
    const float inv = 1.0f / (l + __shfl_xor(l, 32, 64));
    stage_o_rows<T, HD>(stg, l32, g2, o, inv);
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
      v.load(stg + qr * HD + att_swz<T, HC>(qr, cc) * 8);
      v.store(reinterpret_cast<T*>(a.o) + ((long long)b * a.Lq + q) * ld + h * HD + cc * 8);
    }
  }
}

// Kernel entry points (thin wrappers: the host pass only sees these).  Self- and
// text cross-attention run the same body under two symbols so that traces
// separate them; KIND only keeps the instantiations apart.
// One key/value source: two workgroups per CU (at most 256 registers per lane).
template <typename T, int HD>
__global__ __launch_bounds__(256, 2) void attn_self_kernel(const AttnArgs a) {
  attn_body<T, HD, 1, 0>(a);
}
template <typename T, int HD>
__global__ __launch_bounds__(256, 2) void attn_cross_kernel(const AttnArgs a) {
  attn_body<T, HD, 1, 1>(a);
}
// bf16 self-attention: 8 waves of 32 queries (or 4 waves of 32*QB) per workgroup
template <int HD, int NR, int QB, int NW, bool SM>
__global__ __launch_bounds__(64 * NW, (NW == 4 && QB == 1) ? 2 : 1) void attn_self_wide_kernel(const AttnArgs a) {
  attn_wide_body<HD, NR, QB, NW, SM>(a);
}
// bf16 self-attention with 8-bit scores: 8 waves of 32 queries, one workgroup per CU
template <int NR, int NW, bool SM>
__global__ __launch_bounds__(64 * NW, 1) void attn_self_qk8_kernel(const AttnArgs a) {
  attn_wide8_body<NR, NW, SM>(a);
}
// image + text sources keep a second accumulator: one workgroup per CU
template <typename T, int HD>
__global__ __launch_bounds__(256, 1) void attn_cross2_kernel(const AttnArgs a) {
  attn_body<T, HD, 2, 2>(a);
}

template <typename T, int HD, int NSRC>
hipError_t launch_attn_cfg(const AttnArgs& a, hipStream_t st) {
  using Cfg = AttCfg<T, HD>;
  auto kern = NSRC == 2 ? attn_cross2_kernel<T, HD> : (a.self ? attn_self_kernel<T, HD> : attn_cross_kernel<T, HD>);
  static bool attr_set[2] = {false, false};
  const int which = a.self ? 1 : 0;
  if (!attr_set[which]) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)Cfg::LDS_BYTES);
    if (e != hipSuccess) return e;
    attr_set[which] = true;
  }
  const int nqt = (a.Lq + 127) / 128;
  const int G = nqt * a.heads * a.B;
  hipLaunchKernelGGL(kern, dim3(G), dim3(256), Cfg::LDS_BYTES, st, a);
  return hipGetLastError();
}

}  // namespace

template <int HD, int NR, int QB, int NW, bool SM = false>
hipError_t launch_attn_wide(const AttnArgs& a, hipStream_t st) {
  using Cfg = WideCfg<HD, NR, QB, NW>;
  auto kern = attn_self_wide_kernel<HD, NR, QB, NW, SM>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)Cfg::LDS_BYTES);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int nqt = (a.Lq + Cfg::BMQ - 1) / Cfg::BMQ;
  const int G = nqt * a.heads * a.B;
  hipLaunchKernelGGL(kern, dim3(G), dim3(64 * NW), Cfg::LDS_BYTES, st, a);
  return hipGetLastError();
}

template <int NR, int NW, bool SM = false>
hipError_t launch_attn_qk8(const AttnArgs& a, hipStream_t st) {
  using Cfg = Wide8Cfg<NR, NW>;
  auto kern = attn_self_qk8_kernel<NR, NW, SM>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)Cfg::LDS_BYTES);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int nqt = (a.Lq + Cfg::BMQ - 1) / Cfg::BMQ;
  const int G = nqt * a.heads * a.B;
  hipLaunchKernelGGL(kern, dim3(G), dim3(64 * NW), Cfg::LDS_BYTES, st, a);
  return hipGetLastError();
}

bool attn_static_offset_path(int hd, int Lq, int heads, int B, bool bf16, bool qk8) {
  // the 8-bit-score kernel always runs 256-query workgroups
  if (qk8) return bf16 && hd == 128;
  const long long g8 = (long long)((Lq + 255) / 256) * heads * B;
  return bf16 && hd == 128 && g8 >= 512;
}
int attn_wide_flags(int Lq, int heads, int B) { return ((Lq + 255) / 256) * heads * B * WIDE_NW; }

template <typename T>
hipError_t launch_attention(const AttnArgs& a, hipStream_t st) {
  if (a.Lq <= 0) return hipSuccess;
  if (a.qk8) {
    // 8-bit scores: bf16 V, one key source, 128-wide heads, padded key rows
    if (sizeof(T) != 2 || a.hd != 128 || a.nsrc != 1 || !a.qs || !a.ks || a.Lk[0] < 1 || a.Lkp[0] % ATT_BN != 0 ||
        a.Lkp[0] < a.Lk[0])
      return hipErrorInvalidValue;
    if constexpr (sizeof(T) == 2) {
      if (a.kpart && a.fallback) {
        // static offset, then the running-maximum kernel on the workgroups it flagged
        hipError_t e = launch_attn_qk8<2, 8, true>(a, st);
        if (e != hipSuccess) return e;
        AttnArgs b = a;
        b.only = a.fallback;
        return launch_attn_qk8<2, 8>(b, st);
      }
      return launch_attn_qk8<2, 8>(a, st);
    }
  }
  if constexpr (sizeof(T) == 2) {
    if (a.hd == 128 && a.nsrc == 1 && a.self) {
      // Fewer 256-query workgroups than two rounds of the 256 CUs (short sequences):
      // 128-query workgroups of 4 waves, two per CU, so the last round runs on
      // finer pieces (at full length the 8-wave form is about 7% faster).
      if (!attn_static_offset_path(a.hd, a.Lq, a.heads, a.B, true, false))
        return launch_attn_wide<128, WIDE_NR, 1, 4>(a, st);
      if (a.kpart && a.fallback && a.scale_log2 == 1.0f) {
        // static offset, then the running-maximum kernel on the workgroups it flagged
        hipError_t e = launch_attn_wide<128, WIDE_NR_SM, WIDE_QB, WIDE_NW, true>(a, st);
        if (e != hipSuccess) return e;
        AttnArgs b = a;
        b.only = a.fallback;
        return launch_attn_wide<128, WIDE_NR, WIDE_QB, WIDE_NW>(b, st);
      }
      return launch_attn_wide<128, WIDE_NR, WIDE_QB, WIDE_NW>(a, st);
    }
  }
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
