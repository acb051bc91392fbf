// LDS-tiled MFMA GEMM for gfx950: C = A W^T + bias with fused epilogues.
//
// WM x WN waves per workgroup (4, 6 or 8) compute a BM x BN tile in BK-deep
// k-tiles.  Operand tiles stream global -> LDS through the 16-byte LDS-DMA
// path, so the loads of a k-tile are issued tiles ahead of its MFMAs; one
// barrier per k-tile.  Two ring layouts:
//  - 128-byte tile rows (64-deep bf16 or 128-deep e4m3 k-tiles): split rings,
//    NST A stages and two W stages, refilled by buffer loads spread over the
//    MFMA slots of the tile (the bf16 projections, the e4m3 projections and the
//    convolutions with 64-channel taps);
//  - 64-byte tile rows: one NST-stage ring of (A, W) stages (fp32 operands, the
//    patch gather, convolutions with 32- or 96-channel taps).
// An LDS-DMA instruction moves about twice the bytes per cycle over 128-byte
// row pieces as over 64-byte ones, which is why the wider rows are preferred.
// Inside a k-tile the MFMA operand fragments of the next 16-deep step are read
// while the current step's MFMAs run.  Tile rows hold 16-byte chunks whose
// position is XOR-swizzled with low row bits, which puts the 16 rows one
// wave-wide operand read touches on distinct banks.  Tiles are ordered in groups
// of 8 (or 4) M-tiles and the hardware workgroup order is remapped so that each XCD
// (with its own L2) works through one contiguous range.  The epilogue stages
// the fp32 tile in LDS and writes 16-byte pieces.
#include "common.h"
#include "kernels.h"

namespace wan {

namespace {

typedef __attribute__((address_space(3))) void lds_void;

template <typename T, int BM, int BN, int WM, int WN, int NST_, int RB, int LOADER, int EPI, int MI = 32>
struct Gemm {
  static constexpr bool F8 = LOADER == LOAD_FP8;       // e4m3 operands (T: output type)
  static constexpr int BK = F8 ? RB : RB / (int)sizeof(T);  // k-tile depth
  static constexpr int CPR = F8 ? RB / 16 : BK / 8;    // chunks per tile row (16-byte chunks for e4m3)
  static constexpr int PPR = RB / 16;                  // 16-byte pieces per tile row
  static constexpr int RPD = 64 / PPR;                 // tile rows per LDS-DMA wave instruction
  static constexpr int NST = NST_;                     // LDS ring stages
  static constexpr int TM = BM / WM / 32;
  static constexpr int TN = BN / WN / 32;
  static constexpr int STAGE = (BM + BN) * CPR;  // chunks per stage
  // e4m3: per stage, the scale bytes of the tile's A and W rows (64 rows per wave, 256-byte slots)
  static constexpr int SC_STAGE = (F8 && RB == 64) ? 256 * WM * WN : 0;
  // 128-byte rows of bf16 operands (64-deep k-tiles) use split rings: NST A
  // stages and two W stages; otherwise one ring of NST (A, W) stages
  static constexpr bool SPLIT = RB == 128 && (((LOADER == LOAD_PLAIN || LOADER == LOAD_CONV) && sizeof(T) == 2) || F8);
  // MI == 16: the bf16 split-ring main loop on 16x16x32 MFMAs (256x256 tiles; with 4 waves,
  // 128x128 per wave, one wave per SIMD, accumulators in AGPRs)
  static constexpr bool MI16 = MI == 16 && SPLIT && !F8 && LOADER == LOAD_PLAIN && BM == 256 && BN == 256;
  static_assert(MI == 32 || MI16, "16x16x32 MFMAs only on the bf16 split-ring path with 256x256 tiles");
  static constexpr size_t DATA_BYTES =
      SPLIT ? (size_t)NST * BM * RB + 2 * (size_t)BN * RB : (size_t)NST * STAGE * sizeof(Chunk<T>);
  static constexpr size_t PIPE_BYTES = DATA_BYTES + (size_t)NST * SC_STAGE;
  // DMA instructions per wave per k-tile: each covers RPD rows
  static constexpr int NW = WM * WN;                   // waves per workgroup
  static constexpr int NT = 64 * NW;                   // threads per workgroup
  static constexpr int NA = BM / RPD / NW, NB = BN / RPD / NW;
  // register-staged (gathered) path: chunks per thread per k-tile
  static constexpr int A_PT = (BM * CPR + NT - 1) / NT;
  static constexpr int B_PT = (BN * CPR + NT - 1) / NT;
  // epilogue slab: the whole tile when it fits the pipeline's LDS, else one wave column
  static constexpr int SW = ((size_t)BM * (BN + 4) * 4 <= PIPE_BYTES) ? BN : BN / WN;
  static constexpr int SWP = SW + 4;
  static constexpr size_t SLAB_BYTES = (size_t)BM * SWP * 4;
  // the v^T section of a packing GEMM stages its slab transposed ([column][row])
  static constexpr int SWPT = BM + 8;
  static constexpr bool PACK = EPI == EPI_PACK || EPI == EPI_PACK8;
  static constexpr size_t SLABT_BYTES = PACK ? (size_t)SW * SWPT * 4 : 0;
  static constexpr size_t SLAB_MAX = SLAB_BYTES > SLABT_BYTES ? SLAB_BYTES : SLABT_BYTES;
  static constexpr size_t LDS_BYTES = PIPE_BYTES > SLAB_MAX ? PIPE_BYTES : SLAB_MAX;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
  static_assert(BN % SW == 0 && SW % 8 == 0, "slab");
  static_assert(NW == 4 || NW == 8 || NW == 6, "4, 6 or 8 waves");
  static_assert(TM >= 1 && TN >= 1, "wave tile");
  static_assert(NA * RPD * NW == BM && NB * RPD * NW == BN, "DMA split");
  static_assert(RB == 64 || RB == 128, "64- or 128-byte rows");
  static_assert(NST >= 2 && NST <= 4, "ring depth");
  static_assert(!F8 || (BM == 256 && BN == 256 && WM * WN == 8 && sizeof(T) == 2),
                "e4m3 operands: 256x256 tiles of 8 waves, bf16 output");
};

// Physical chunk position of logical chunk c in tile row r (RB-byte rows).  A
// wave-wide 16-byte LDS read is served 16 lanes at a time; those lanes read 16
// consecutive rows at one chunk, which must land on 16 distinct 16-byte bank
// groups of the 256-byte bank line: 64-byte rows put 4 rows on a line and XOR
// the chunk with row bits 2..3, 128-byte rows put 2 rows on a line and XOR the
// 16-byte piece with row bits 1..3.
template <int RB, int CPR>
__device__ __forceinline__ int swz(int r, int c) {
  if constexpr (RB == 64)
    return c ^ ((r >> 2) & (CPR - 1));
  else
    return c ^ ((r >> 1) & (CPR - 1));
}

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

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] and [15:14], expcnt[6:4],
// lgkmcnt[11:8]); a field at its maximum does not wait.  Issued through the
// builtin so that the compiler's own wait insertion accounts for them.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier that waits for this wave's LDS reads only.  __syncthreads()
// would also drain every outstanding global load (vmcnt(0)), i.e. the k-tiles
// prefetched into the ring; the vmcnt wait for the tile needed next is explicit.
// The empty asm statements keep the compiler from moving memory accesses across.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <typename T, int BM, int BN, int WM, int WN, int NST_, int RB, int LOADER, int EPI, int MI = 32>
__device__ __forceinline__ void gemm_body(const GemmArgs& g) {
  using C = Gemm<T, BM, BN, WM, WN, NST_, RB, LOADER, EPI, MI>;
  constexpr int BK = C::BK, CPR = C::CPR, TM = C::TM, TN = C::TN, NST = C::NST, NT = C::NT;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  Chunk<T>* smem = reinterpret_cast<Chunk<T>*>(smem_raw);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS-DMA targets stay scalar
  const int g2 = lane >> 5;  // lane group: which 8-chunk of a 16-wide k step
  const int l32 = lane & 31;

  // ---- tile coordinates: XCD-contiguous ranges, groups of 8 or 4 M-tiles
  const int nm = (g.M + BM - 1) / BM;
  const int nn = g.N / BN;
  const int ntiles = nm * nn;
  const int lid = xcd_remap(blockIdx.x, ntiles);
  int tm, tn;
  if (nn <= 8) {
    // few N-tiles: all of them run side by side on one XCD, so every A row panel
    // is fetched from HBM once while each N-tile consumes it
    tm = lid / nn;
    tn = lid - tm * nn;
  } else {
    // groups of GM M-tiles walk all N-tiles, M fastest.  Eight 256-row bf16 A
    // panels of K <= 2048 (up to 1 MB each) overflow one XCD's 4 MB L2 while four
    // fit; with many N-tiles (the FFN1 shape: 35) the smaller group reuses its A
    // panels from L2 (5% faster there; 8 stays better for fewer N-tiles)
    const int GM = (LOADER == LOAD_PLAIN && sizeof(T) == 2 && nn >= 32 && g.K <= 2048) ? 4 : 8;
    const int group = lid / (GM * nn);
    const int first_m = group * GM;
    const int gsize = min(nm - first_m, GM);
    const int in_group = lid - group * GM * nn;
    tm = first_m + in_group % gsize;
    tn = in_group / gsize;
  }
  const int m0 = tm * BM;
  const int n0 = tn * BN;

  f32x16 acc[TM][TN];
  // 16x16 form: 16-row blocks of the wave's A rows and W rows
  constexpr int TR16 = C::MI16 ? (BM / WM) / 16 : 1, TC16 = C::MI16 ? (BN / WN) / 16 : 1;
  f32x4 acc16[TR16][TC16];
  if constexpr (C::MI16) {
    // each zero accumulator is materialised in its own AGPRs: left to the compiler, the zeros
    // share registers and every k-tile iteration then copies 60 accumulator registers around
#pragma unroll
    for (int i = 0; i < TR16; ++i)
#pragma unroll
      for (int j = 0; j < TC16; ++j) {
        acc16[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};
        if constexpr (WM * WN == 4) asm volatile("" : "+a"(acc16[i][j]));  // AGPRs at one wave per SIMD
      }
  } else {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  }

  const int wm = wave / WN, wn = wave % WN;
  const int arow0 = wm * (BM / WM);
  const int brow0 = wn * (BN / WN);
  const int nk = (g.K + BK - 1) / BK;
  constexpr int KS = BK / 16;

  // MFMA operand fragments of one 16-deep k step, double-buffered
  Chunk<T> fa[2][TM], fb[2][TN];
  auto load_frags = [&](int stage, int ks, int buf) {
    const Chunk<T>* sa = smem + stage * C::STAGE;
    const Chunk<T>* sb = sa + BM * CPR;
    const int c = 2 * ks + g2;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int r = arow0 + 32 * i + l32;
      fa[buf][i].load(&sa[r * CPR + swz<RB, CPR>(r, c)]);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int r = brow0 + 32 * j + l32;
      fb[buf][j].load(&sb[r * CPR + swz<RB, CPR>(r, c)]);
    }
  };
  auto mma_step = [&](int buf) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) mma32(acc[i][j], fb[buf][j], fa[buf][i]);
  };

  if constexpr (LOADER == LOAD_FP8 && RB == 128) {
    // ---- e4m3 operands in split rings: 128-byte rows = 128-deep k-tiles, one
    // scale block each, in the ring layout and schedule of the bf16 split path
    // below (A: NST stages, W: 2, buffer-load refills spread over the tile).
    // Each k-tile is two scaled 32x32x64 MFMA steps.  The scale bytes of a lane's
    // rows (A: row operand of scale_b, W: of scale_a) are loaded straight into
    // registers one tile ahead, ahead of the W refill, so the tile-end wait
    // covers them.  MFMA row operand = W rows, column operand = A rows.
    constexpr int NA = C::NA, NB = C::NB, DPT = NA + NB, RPD = C::RPD, PPR = C::PPR;
    constexpr int NM = TM * TN, NR = TM + TN;
    constexpr int K8 = BK / 64;  // scaled k steps per tile
    constexpr int SYNC_SLOT = 1;
    constexpr int A_SB = BM * RB, B_SB = BN * RB;
    static_assert(K8 == 2 && NST >= 3 && NM >= NR && SYNC_SLOT <= TM - 1, "e4m3 split rings");
    const int pp = lane % PPR;
    const int rlow = lane / PPR;
    const unsigned char* a_tile;
    {
      const int bb = m0 / g.a_rpb;
      int t = m0 - bb * g.a_rpb;
      if (g.a_valid > 0) t = min(t, g.a_valid - 1);
      a_tile = reinterpret_cast<const unsigned char*>(g.A) + (long long)bb * g.a_bstride + (long long)t * g.lda;
    }
    const unsigned char* w_tile = reinterpret_cast<const unsigned char*>(g.Wt) + (long long)n0 * g.ldw;
    unsigned a_vo[NA], b_vo[NB];
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int rt = (wave * NA + i) * RPD + rlow;
      const int r = min(m0 + rt, g.M - 1);
      const int bb = r / g.a_rpb;
      int t = r - bb * g.a_rpb;
      if (g.a_valid > 0) t = min(t, g.a_valid - 1);
      a_vo[i] = (unsigned)((long long)bb * g.a_bstride + (long long)t * g.lda - (a_tile - reinterpret_cast<const unsigned char*>(g.A)) +
                           swz<RB, CPR>(rt, pp) * 16);
    }
    // W rows of piece i differ from those of piece i % 2 by a multiple of 2 RPD rows and share
    // its swizzle (row bits 1..3 depend on i only through i % 2): two lane offsets serve all
    // pieces, the rest of the row offset goes into the scalar offset
    static_assert(NB % 2 == 0 && RPD == 8, "W lane offsets by piece parity");
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int rt = (wave * NB + i) * RPD + rlow;
      b_vo[i] = (unsigned)((long long)rt * g.ldw + swz<RB, CPR>(rt, pp) * 16);
    }
    const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc((void*)a_tile, (short)0, -1, 0x00020000);
    const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc((void*)w_tile, (short)0, -1, 0x00020000);
    unsigned char* a_ring = smem_raw;
    unsigned char* b_ring = smem_raw + NST * A_SB;
    auto dma_a = [&](int t, int d) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_void*)(a_ring + (t % NST) * A_SB + (wave * NA + d) * 1024), 16,
                                               a_vo[d], t * BK, 0, 0);
    };
    auto dma_b = [&](int t, int d) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lds_void*)(b_ring + (t % 2) * B_SB + (wave * NB + d) * 1024), 16,
                                               b_vo[d % 2], t * BK + (d / 2) * 2 * RPD * (int)g.ldw, 0, 0);
    };
    auto refill = [&](int kt, int d) {
      if (d < NB)
        dma_b(min(kt + 1, nk - 1), d);
      else
        dma_a(min(kt + NST - 1, nk - 1), d - NB);
    };
    // scale bytes of this lane's rows for k-block t: buffer loads at lane offset
    // l32 + 32 i from a scalar base (descriptor at the tile's rows, k-block offset scalar)
    const __amdgpu_buffer_rsrc_t rca = __builtin_amdgcn_make_buffer_rsrc((void*)(g.a_scale + m0 + arow0), (short)0, -1,
                                                                         0x00020000);
    const __amdgpu_buffer_rsrc_t rcb = __builtin_amdgcn_make_buffer_rsrc((void*)(g.w_scale + n0 + brow0), (short)0, -1,
                                                                         0x00020000);
    // the current tile's scales are packed, one byte per fragment (the MFMA's op_sel picks the
    // byte: W fragment j, A fragment i); the next tile's arrive one byte per register
    int sa8p = 0, sb8p = 0, nsa[TM], nsb[TN];
    static_assert(TM == 2 && TN == 4, "one scale byte per fragment in a 32-bit register (op_sel cases below)");
    auto pack_scales = [&]() {
      sa8p = 0;
      sb8p = 0;
#pragma unroll
      for (int i = 0; i < TM; ++i) sa8p |= (nsa[i] & 0xFF) << (8 * i);
#pragma unroll
      for (int j = 0; j < TN; ++j) sb8p |= (nsb[j] & 0xFF) << (8 * j);
    };
    auto load_scales = [&](int t, int (&xa)[TM], int (&xb)[TN]) {
#pragma unroll
      for (int i = 0; i < TM; ++i) xa[i] = __builtin_amdgcn_raw_buffer_load_b8(rca, l32 + 32 * i, t * g.a_sld, 0);
#pragma unroll
      for (int j = 0; j < TN; ++j) xb[j] = __builtin_amdgcn_raw_buffer_load_b8(rcb, l32 + 32 * j, t * g.N, 0);
    };
    // Fragments are single-buffered: the MFMAs of a step run W-fragment-major,
    // (i, j) at slot j * TM + i, so W fragment j is dead after slot j * TM + TM - 1
    // and A fragment i after slot (TN - 1) * TM + i; the next step's copy of each is
    // read in the slot where it dies.
    typedef int i32x8 __attribute__((ext_vector_type(8)));
    i32x8 fa8[TM], fb8[TN];
    auto read_frag = [&](int t, int ks, const unsigned char* base, int row) {
      const int p0 = 4 * ks + 2 * g2;
      const unsigned char* rowp = base + row * RB;
      const u32x4 lo = *reinterpret_cast<const u32x4*>(rowp + swz<RB, CPR>(row, p0) * 16);
      const u32x4 hi = *reinterpret_cast<const u32x4*>(rowp + swz<RB, CPR>(row, p0 + 1) * 16);
      return __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    auto read_a = [&](int t, int ks, int i) {
      fa8[i] = read_frag(t, ks, a_ring + (t % NST) * A_SB, arow0 + 32 * i + l32);
    };
    auto read_b = [&](int t, int ks, int j) {
      fb8[j] = read_frag(t, ks, b_ring + (t % 2) * B_SB, brow0 + 32 * j + l32);
    };
#pragma unroll
    for (int d = 0; d < NB; ++d) dma_b(0, d);
#pragma unroll
    for (int s0 = 0; s0 < NST - 1; ++s0)
#pragma unroll
      for (int d = 0; d < NA; ++d) dma_a(min(s0, nk - 1), d);
    load_scales(0, nsa, nsb);
    wait_vmcnt<0>();
    barrier_lds();
    pack_scales();
#pragma unroll
    for (int i = 0; i < TM; ++i) read_a(0, 0, i);
#pragma unroll
    for (int j = 0; j < TN; ++j) read_b(0, 0, j);
    for (int kt = 0; kt < nk; ++kt) {
#pragma unroll
      for (int ks = 0; ks < K8; ++ks) {
        const bool last = ks + 1 == K8;
        const int tn = last ? kt + 1 : kt;   // tile and step of the fragments read in this step
        const int kn = last ? 0 : ks + 1;
#pragma unroll
        for (int q = 0; q < NM; ++q) {
          if (ks == 0 && q == 0) load_scales(min(kt + 1, nk - 1), nsa, nsb);
          const int i = q % TM, j = q / TM;
          // op_sel must be an immediate: one case per (W fragment, A fragment), resolved at compile time
          switch (j * 4 + i) {
#define WAN_MMA8(J, I)                                                                                          \
  case J * 4 + I:                                                                                                \
    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb8[j], fa8[i], acc[i][j], 0, 0, J, sb8p, I, sa8p); \
    break;
            WAN_MMA8(0, 0) WAN_MMA8(0, 1) WAN_MMA8(1, 0) WAN_MMA8(1, 1)
            WAN_MMA8(2, 0) WAN_MMA8(2, 1) WAN_MMA8(3, 0) WAN_MMA8(3, 1)
#undef WAN_MMA8
          }
          if (last && q == SYNC_SLOT) {
            wait_vmcnt<NA>();  // scales, W and A of tile kt+1 have landed
            barrier_lds();
          }
          if (j == TN - 1) read_a(tn, kn, i);  // A fragment i is dead from here
          if (i == TM - 1) read_b(tn, kn, j);  // W fragment j is dead from here
          {
            // refill piece d at slot d * SPAN / DPT: all of them before the tile-end wait
            constexpr int SPAN = (K8 - 1) * NM + SYNC_SLOT;
            const int gs = ks * NM + q;
#pragma unroll
            for (int d = 0; d < DPT; ++d)
              if ((d * SPAN) / DPT == gs) refill(kt, d);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      pack_scales();
    }
    wait_vmcnt<0>();
    __syncthreads();
  } else if constexpr (LOADER == LOAD_FP8) {
    // ---- e4m3 operands: the LDS-DMA ring of the bf16 path with 64-byte k-tiles
    // (64 elements, one scaled 32x32x64 MFMA step) plus, per stage, the scale
    // bytes of the tile's 256 A rows (waves 0-3) and 256 W rows (waves 4-7) for
    // the k-tile's 128-block.  MFMA row operand = W rows (scale_a), column operand
    // = A rows (scale_b), as in the bf16 path.
    constexpr int NA = C::NA, NB = C::NB, DPT = NA + NB + 1, RPD = C::RPD, PPR = C::PPR;
    const int pp = lane % PPR;
    const int rlow = lane / PPR;
    const unsigned char* a_src[NA];
    const unsigned char* b_src[NB];
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int rt = (wave * NA + i) * RPD + rlow;
      const int r = min(m0 + rt, g.M - 1);
      const int bb = r / g.a_rpb;
      int t = r - bb * g.a_rpb;
      if (g.a_valid > 0) t = min(t, g.a_valid - 1);
      a_src[i] = reinterpret_cast<const unsigned char*>(g.A) + (long long)bb * g.a_bstride + (long long)t * g.lda +
                 swz<RB, CPR>(rt, pp) * 16;
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int rt = (wave * NB + i) * RPD + rlow;
      b_src[i] = reinterpret_cast<const unsigned char*>(g.Wt) + (long long)(n0 + rt) * g.ldw + swz<RB, CPR>(rt, pp) * 16;
    }
    // scale rows: a 64-byte run per wave, lanes past 15 repeat the last word into the slot's tail
    const bool sc_a = wave < 4;
    const unsigned char* sc_src = (sc_a ? g.a_scale + m0 + 64 * wave : g.w_scale + n0 + 64 * (wave - 4)) +
                                  4 * (lane < 16 ? lane : 15);
    const long long sc_ld = sc_a ? g.a_sld : (long long)g.N;
    auto issue = [&](int kt) {
      const int st = kt % NST;
      unsigned char* base = smem_raw + (size_t)st * C::STAGE * sizeof(Chunk<T>);
      const int koff = kt * BK;
#pragma unroll
      for (int i = 0; i < NA; ++i)
        __builtin_amdgcn_global_load_lds(a_src[i] + koff, (lds_void*)(base + (size_t)(wave * NA + i) * 1024), 16,
                                         0, 0);
      unsigned char* bbase = base + (size_t)BM * RB;
#pragma unroll
      for (int i = 0; i < NB; ++i)
        __builtin_amdgcn_global_load_lds(b_src[i] + koff, (lds_void*)(bbase + (size_t)(wave * NB + i) * 1024), 16,
                                         0, 0);
      __builtin_amdgcn_global_load_lds(sc_src + (long long)(koff / 128) * sc_ld,
                                       (lds_void*)(smem_raw + C::DATA_BYTES + (size_t)st * C::SC_STAGE + wave * 256),
                                       4, 0, 0);
    };
    constexpr int INFLIGHT = (NST - 2) * DPT;
    auto issue_c = [&](int kt) { issue(min(kt, nk - 1)); };
    typedef int i32x8 __attribute__((ext_vector_type(8)));
    i32x8 fa[TM], fb[TN];
    int sa8[TM], sb8[TN];
    auto load_frags8 = [&](int st) {
      const unsigned char* sa = smem_raw + (size_t)st * C::STAGE * sizeof(Chunk<T>);
      const unsigned char* sb = sa + (size_t)BM * RB;
      const unsigned char* sc = smem_raw + C::DATA_BYTES + (size_t)st * C::SC_STAGE;
      auto rd32 = [&](const unsigned char* rowp, int r) {
        const u32x4 lo = *reinterpret_cast<const u32x4*>(rowp + swz<RB, CPR>(r, 2 * g2) * 16);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(rowp + swz<RB, CPR>(r, 2 * g2 + 1) * 16);
        return __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      };
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int r = brow0 + 32 * j + l32;
        fb[j] = rd32(sb + r * RB, r);
        sb8[j] = sc[(4 + r / 64) * 256 + r % 64];
      }
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = arow0 + 32 * i + l32;
        fa[i] = rd32(sa + r * RB, r);
        sa8[i] = sc[(r / 64) * 256 + r % 64];
      }
    };
#pragma unroll
    for (int s0 = 0; s0 < NST - 1; ++s0) issue_c(s0);
    wait_vmcnt<INFLIGHT>();
    barrier_lds();
    load_frags8(0);
    for (int kt = 0; kt < nk; ++kt) {
      issue_c(kt + NST - 1);
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int i = 0; i < TM; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[j], fa[i], acc[i][j], 0, 0, 0, sb8[j], 0,
                                                                      sa8[i]);
      wait_vmcnt<INFLIGHT>();  // k-tile kt+1 (and its scales) have landed
      barrier_lds();
      load_frags8((kt + 1) % NST);
    }
    wait_vmcnt<0>();
    __syncthreads();
  } else if constexpr (C::MI16) {
    // ---- split rings as below, 4 waves of 128x128 on 16x16x32 MFMAs: per 32-deep k step a
    // wave reads 8 A and 8 W fragments (lane l: row l%16 of a 16-row block, 16-byte chunk
    // 4 ks + l/16 of the 64-deep tile row) and runs 64 MFMAs.  The next step's 16
    // fragments are read over the first 32 slots; in a tile's last step the wave waits for
    // the refills and synchronises at slot SYNC16, then reads the next tile's first fragments.
    constexpr int NA = C::NA, NB = C::NB, DPT = NA + NB, RPD = C::RPD, PPR = C::PPR;
    constexpr int KS2 = BK / 32;
    constexpr int NS16 = TR16 * TC16;   // MFMA slots per k step
    constexpr int NR16 = TR16 + TC16;   // fragment reads per k step
    constexpr int SYNC16 = NS16 - 2 * NR16 - 8 > 0 ? NS16 - 2 * NR16 - 8 : 0;
    constexpr int SPAN = (KS2 - 1) * NS16 + SYNC16;
    constexpr int A_SB = BM * RB, B_SB = BN * RB;
    static_assert(KS2 == 2 && NST >= 3 && SYNC16 + NR16 < NS16 && 2 * NR16 <= NS16, "16x16 split rings");
    const int pp = lane % PPR;
    const int rlow = lane / PPR;
    const T* a_tile;
    {
      const int bb = m0 / g.a_rpb;
      int t = m0 - bb * g.a_rpb;
      if (g.a_valid > 0) t = min(t, g.a_valid - 1);
      a_tile = reinterpret_cast<const T*>(g.A) + (long long)bb * g.a_bstride + (long long)t * g.lda;
    }
    unsigned a_vo[NA];
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int rt = (wave * NA + i) * RPD + rlow;
      const int r = min(m0 + rt, g.M - 1);
      const int bb = r / g.a_rpb;
      int t = r - bb * g.a_rpb;
      if (g.a_valid > 0) t = min(t, g.a_valid - 1);
      const T* src = reinterpret_cast<const T*>(g.A) + (long long)bb * g.a_bstride + (long long)t * g.lda +
                     swz<RB, CPR>(rt, pp) * 8;
      a_vo[i] = (unsigned)((src - a_tile) * (long long)sizeof(T));
    }
    const T* w_tile = reinterpret_cast<const T*>(g.Wt) + (long long)n0 * g.ldw;
    unsigned b_vo[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int rt = (wave * NB + i) * RPD + rlow;
      b_vo[i] = (unsigned)(((long long)rt * g.ldw + swz<RB, CPR>(rt, pp) * 8) * (long long)sizeof(T));
    }
    const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc((void*)a_tile, (short)0, -1, 0x00020000);
    const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc((void*)w_tile, (short)0, -1, 0x00020000);
    unsigned char* a_ring = smem_raw;
    unsigned char* b_ring = smem_raw + NST * A_SB;
    auto dma_a = [&](int t, int d) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_void*)(a_ring + (t % NST) * A_SB + (wave * NA + d) * 1024), 16,
                                               a_vo[d], t * BK * (int)sizeof(T), 0, 0);
    };
    auto dma_b = [&](int t, int d) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lds_void*)(b_ring + (t % 2) * B_SB + (wave * NB + d) * 1024), 16,
                                               b_vo[d], t * BK * (int)sizeof(T), 0, 0);
    };
    auto refill = [&](int kt, int d) {
      if (d < NB)
        dma_b(min(kt + 1, nk - 1), d);
      else
        dma_a(min(kt + NST - 1, nk - 1), d - NB);
    };
    Chunk<T> f16a[2][TR16], f16b[2][TC16];
    const int r16 = lane & 15, c16 = lane >> 4;
    auto read16 = [&](int t, int ks, int buf, int r) {
      const int c = 4 * ks + c16;
      if (r < TR16) {
        const Chunk<T>* sa = reinterpret_cast<const Chunk<T>*>(a_ring + (t % NST) * A_SB);
        const int row = arow0 + 16 * r + r16;
        f16a[buf][r].load(&sa[row * CPR + swz<RB, CPR>(row, c)]);
      } else {
        const Chunk<T>* sb = reinterpret_cast<const Chunk<T>*>(b_ring + (t % 2) * B_SB);
        const int row = brow0 + 16 * (r - TR16) + r16;
        f16b[buf][r - TR16].load(&sb[row * CPR + swz<RB, CPR>(row, c)]);
      }
    };
#pragma unroll
    for (int d = 0; d < NB; ++d) dma_b(0, d);
#pragma unroll
    for (int s0 = 0; s0 < NST - 1; ++s0)
#pragma unroll
      for (int d = 0; d < NA; ++d) dma_a(min(s0, nk - 1), d);
    wait_vmcnt<(NST - 2) * NA>();
    barrier_lds();
#pragma unroll
    for (int r = 0; r < NR16; ++r) read16(0, 0, 0, r);
    for (int kt = 0; kt < nk; ++kt) {
#pragma unroll
      for (int ks = 0; ks < KS2; ++ks) {
        const int buf = ks & 1;
#pragma unroll
        for (int q = 0; q < NS16; ++q) {
          {
            const int i = q / TC16, j = q % TC16;
            acc16[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(f16b[buf][j].v),
                                                                  as_bf16x8(f16a[buf][i].v), acc16[i][j], 0, 0, 0);
          }
          if (ks + 1 < KS2) {
            if ((q & 1) == 0 && q / 2 < NR16) read16(kt, ks + 1, buf ^ 1, q / 2);
          } else {
            if (q == SYNC16) {
              wait_vmcnt<NA>();
              barrier_lds();
            }
            if (q > SYNC16 && q - SYNC16 - 1 < NR16) read16(kt + 1, 0, buf ^ 1, q - SYNC16 - 1);
          }
          {
            const int gs = ks * NS16 + q;
#pragma unroll
            for (int d = 0; d < DPT; ++d)
              if ((d * SPAN) / DPT == gs) refill(kt, d);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    wait_vmcnt<0>();
    __syncthreads();
  } else if constexpr (C::SPLIT) {
    // ---- split LDS-DMA rings, 128-byte rows.  An LDS-DMA instruction over 64-byte
    // row pieces moves about half the bytes per cycle of one over 128-byte pieces,
    // so the k-tile is 64 deep; a 256x256 tile then needs 64 KB per stage, and the
    // 160 KB of LDS hold NST = 3 A stages (32 KB each) and 2 W stages.  At the top
    // of tile kt the W slice of tile kt+1 goes out first, then the A slice of tile
    // kt+2, spread over the MFMA slots before the tile-end wait, which lets only
    // that A slice stay in flight.  The copies are buffer loads (one descriptor per
    // operand based at the tile's first row, 32-bit lane offsets, the k offset (for
    // the convolution, the tap offset plus the k offset) as the scalar offset: no
    // vector ALU per refill).  Global-address LDS copies would also make every wait
    // for a fragment read drain all LDS reads in flight.
    // The tile runs as KS k steps of TM*TN slots, one MFMA each, closed by a
    // scheduling barrier: a step reads the fragments of the next step in its first
    // TM+TN slots; the last step waits and synchronises after SYNC_SLOT + 1 MFMAs
    // and then reads the next tile's first fragments.
    constexpr int NA = C::NA, NB = C::NB, DPT = NA + NB, RPD = C::RPD, PPR = C::PPR;
    constexpr int NM = TM * TN, NR = TM + TN;
    constexpr int SYNC_SLOT = NM - NR - 1 > 0 ? NM - NR - 1 : 0;
    constexpr int SPAN = (KS - 1) * NM + SYNC_SLOT;  // slots before the wait: the refills go out over them
    constexpr int A_SB = BM * RB, B_SB = BN * RB;  // stage bytes
    static_assert(KS % 2 == 0 && NST >= 3 && NM >= NR, "split rings: even k steps, 3+ A stages");
    const int pp = lane % PPR;
    const int rlow = lane / PPR;
    // A rows: token rows of the plain loader, or output voxels of the convolution
    // loader (the A row of a voxel is the front-top-left corner of its window in the
    // padded buffer; later rows of a tile lie further on, and the tap offsets, added
    // per k-tile, are non-negative; a tap's channels span kpt 64-deep k-tiles)
    const T* a_tile = reinterpret_cast<const T*>(g.A);
    unsigned a_vo[NA];  // byte offsets from the tile's first row (the host bounds them below 2^32)
    const int kpt = LOADER == LOAD_CONV ? g.cv_kpt / 2 : 1;
    if constexpr (LOADER == LOAD_CONV) {
      const int hw = g.cv_h * g.cv_w;
      auto voxel_row = [&](int r) {
        const int tv = r / hw, rem = r - tv * hw;
        const int hv = rem / g.cv_w, wv = rem - hv * g.cv_w;
        return reinterpret_cast<const T*>(g.A) + (((long long)(tv + g.cv_t0) * g.cv_hp + hv) * g.cv_wp + wv) * g.lda;
      };
      a_tile = voxel_row(m0);
#pragma unroll
      for (int i = 0; i < NA; ++i) {
        const int rt = (wave * NA + i) * RPD + rlow;
        const T* src = voxel_row(min(m0 + rt, g.M - 1)) + swz<RB, CPR>(rt, pp) * 8;
        a_vo[i] = (unsigned)((src - a_tile) * (long long)sizeof(T));
      }
    } else {
      {
        const int bb = m0 / g.a_rpb;
        int t = m0 - bb * g.a_rpb;
        if (g.a_valid > 0) t = min(t, g.a_valid - 1);
        a_tile = reinterpret_cast<const T*>(g.A) + (long long)bb * g.a_bstride + (long long)t * g.lda;
      }
#pragma unroll
      for (int i = 0; i < NA; ++i) {
        const int rt = (wave * NA + i) * RPD + rlow;
        const int r = min(m0 + rt, g.M - 1);
        const int bb = r / g.a_rpb;
        int t = r - bb * g.a_rpb;
        if (g.a_valid > 0) t = min(t, g.a_valid - 1);
        const T* src = reinterpret_cast<const T*>(g.A) + (long long)bb * g.a_bstride + (long long)t * g.lda +
                       swz<RB, CPR>(rt, pp) * 8;
        a_vo[i] = (unsigned)((src - a_tile) * (long long)sizeof(T));
      }
    }
    const T* w_tile = reinterpret_cast<const T*>(g.Wt) + (long long)n0 * g.ldw;
    unsigned b_vo[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int rt = (wave * NB + i) * RPD + rlow;
      b_vo[i] = (unsigned)(((long long)rt * g.ldw + swz<RB, CPR>(rt, pp) * 8) * (long long)sizeof(T));
    }
    const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc((void*)a_tile, (short)0, -1, 0x00020000);
    const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc((void*)w_tile, (short)0, -1, 0x00020000);
    unsigned char* a_ring = smem_raw;
    unsigned char* b_ring = smem_raw + NST * A_SB;
    auto dma_a = [&](int t, int d) {
      lds_void* dst = (lds_void*)(a_ring + (t % NST) * A_SB + (wave * NA + d) * 1024);
      if constexpr (LOADER == LOAD_CONV) {
        const int tap = t / kpt;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rsa, dst, 16, a_vo[d], (int)((g.tap_off[tap] + (long long)(t - tap * kpt) * BK) * (long long)sizeof(T)), 0,
            0);
      } else {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, dst, 16, a_vo[d], t * BK * (int)sizeof(T), 0, 0);
      }
    };
    auto dma_b = [&](int t, int d) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lds_void*)(b_ring + (t % 2) * B_SB + (wave * NB + d) * 1024), 16,
                                               b_vo[d], t * BK * (int)sizeof(T), 0, 0);
    };
    // refill piece d of tile kt's iteration (indices clamped at the end: the
    // redundant copies rewrite a stage with the bytes it already holds)
    auto refill = [&](int kt, int d) {
      if (d < NB)
        dma_b(min(kt + 1, nk - 1), d);
      else
        dma_a(min(kt + NST - 1, nk - 1), d - NB);
    };
    auto read_one = [&](int t, int ks, int buf, int r) {
      const int c = 2 * ks + g2;
      if (r < TM) {
        const Chunk<T>* sa = reinterpret_cast<const Chunk<T>*>(a_ring + (t % NST) * A_SB);
        const int row = arow0 + 32 * r + l32;
        fa[buf][r].load(&sa[row * CPR + swz<RB, CPR>(row, c)]);
      } else {
        const Chunk<T>* sb = reinterpret_cast<const Chunk<T>*>(b_ring + (t % 2) * B_SB);
        const int row = brow0 + 32 * (r - TM) + l32;
        fb[buf][r - TM].load(&sb[row * CPR + swz<RB, CPR>(row, c)]);
      }
    };
    // prologue: W tile 0, A tiles 0 .. NST-2
#pragma unroll
    for (int d = 0; d < NB; ++d) dma_b(0, d);
#pragma unroll
    for (int s0 = 0; s0 < NST - 1; ++s0)
#pragma unroll
      for (int d = 0; d < NA; ++d) dma_a(min(s0, nk - 1), d);
    wait_vmcnt<(NST - 2) * NA>();
    barrier_lds();
#pragma unroll
    for (int r = 0; r < NR; ++r) read_one(0, 0, 0, r);
    for (int kt = 0; kt < nk; ++kt) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int buf = ks & 1;
#pragma unroll
        for (int q = 0; q < NM; ++q) {
          {
            const int i = q / TN, j = q % TN;
            mma32(acc[i][j], fb[buf][j], fa[buf][i]);
          }
          if (ks + 1 < KS) {
            if (q < NR) read_one(kt, ks + 1, buf ^ 1, q);
          } else {
            if (q == SYNC_SLOT) {
              wait_vmcnt<NA>();  // W and A of tile kt+1 have landed; A of tile kt+NST-1 may be out
              barrier_lds();
            }
            if (q > SYNC_SLOT && q - SYNC_SLOT - 1 < NR) read_one(kt + 1, 0, buf ^ 1, q - SYNC_SLOT - 1);
            if (q == NM - 1) {
#pragma unroll
              for (int r = NM - SYNC_SLOT - 1; r < NR; ++r) read_one(kt + 1, 0, buf ^ 1, r);
            }
          }
          {
            // refill piece d at slot d * SPAN / DPT, all before the tile-end wait
            const int gs = ks * NM + q;
#pragma unroll
            for (int d = 0; d < DPT; ++d)
              if ((d * SPAN) / DPT == gs) refill(kt, d);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    wait_vmcnt<0>();
    __syncthreads();
  } else if constexpr (LOADER == LOAD_PLAIN || LOADER == LOAD_CONV) {
    // ---- LDS-DMA ring.  One wave instruction fills 1 KB = RPD tile rows; lane
    // l writes the l-th 16 bytes, so the chunk swizzle is applied to the global
    // address each lane reads.
    constexpr int SPC = (int)sizeof(Chunk<T>) / 16;
    constexpr int NA = C::NA, NB = C::NB, DPT = NA + NB, RPD = C::RPD, PPR = C::PPR;
    const int pp = lane % PPR;   // 16-byte piece within the tile row
    const int rlow = lane / PPR; // row within the instruction's RPD rows
    auto col_off = [&](int r) { return swz<RB, CPR>(r, pp / SPC) * 8 + (pp % SPC) * (8 / SPC); };
    // The plain loader copies from 64-bit lane addresses (this path also serves operands
    // whose tile-relative offsets need more than 32 bits).  The convolution loader copies
    // through buffer resources based at the tile's first output voxel and first W row
    // (32-bit lane offsets, the tap and k offsets as the scalar offset; the host bounds
    // them), so that the waits for fragment reads stay counted.
    constexpr bool CONV = LOADER == LOAD_CONV;
    const T* a_src[CONV ? 1 : NA];
    const T* b_src[CONV ? 1 : NB];
    unsigned a_vo[CONV ? NA : 1], b_vo[CONV ? NB : 1];
    const T* a_tile = reinterpret_cast<const T*>(g.A);
    const T* w_tile = reinterpret_cast<const T*>(g.Wt) + (long long)n0 * g.ldw;
    if constexpr (CONV) {
      // output voxel (t, h, w) of the chunk: the front-top-left corner of its window
      const int hw = g.cv_h * g.cv_w;
      auto voxel_row = [&](int r) {
        const int tv = r / hw, rem = r - tv * hw;
        const int hv = rem / g.cv_w, wv = rem - hv * g.cv_w;
        return reinterpret_cast<const T*>(g.A) + (((long long)(tv + g.cv_t0) * g.cv_hp + hv) * g.cv_wp + wv) * g.lda;
      };
      a_tile = voxel_row(m0);
#pragma unroll
      for (int i = 0; i < NA; ++i) {
        const int rt = (wave * NA + i) * RPD + rlow;  // row within the tile
        const T* src = voxel_row(min(m0 + rt, g.M - 1)) + col_off(rt);
        a_vo[i] = (unsigned)((src - a_tile) * (long long)sizeof(T));
      }
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int rt = (wave * NB + i) * RPD + rlow;
        b_vo[i] = (unsigned)(((long long)rt * g.ldw + col_off(rt)) * (long long)sizeof(T));
      }
    } else {
#pragma unroll
      for (int i = 0; i < NA; ++i) {
        const int rt = (wave * NA + i) * RPD + rlow;  // row within the tile
        const int r = min(m0 + rt, g.M - 1);
        const int bb = r / g.a_rpb;
        int t = r - bb * g.a_rpb;
        if (g.a_valid > 0) t = min(t, g.a_valid - 1);  // padding rows of a padded row pitch
        a_src[i] = reinterpret_cast<const T*>(g.A) + (long long)bb * g.a_bstride + (long long)t * g.lda + col_off(rt);
      }
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int rt = (wave * NB + i) * RPD + rlow;
        b_src[i] = w_tile + (long long)rt * g.ldw + col_off(rt);
      }
    }
    const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc((void*)a_tile, (short)0, -1, 0x00020000);
    const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc((void*)w_tile, (short)0, -1, 0x00020000);
    auto issue = [&](int kt) {
      unsigned char* base = smem_raw + (size_t)(kt % NST) * C::STAGE * sizeof(Chunk<T>);
      unsigned char* bbase = base + (size_t)BM * CPR * sizeof(Chunk<T>);
      const int koff = kt * BK;
      if constexpr (CONV) {
        const int tap = kt / g.cv_kpt;
        const int aoff = (int)((g.tap_off[tap] + (long long)(kt - tap * g.cv_kpt) * BK) * (long long)sizeof(T));
#pragma unroll
        for (int i = 0; i < NA; ++i)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_void*)(base + (size_t)(wave * NA + i) * 1024), 16, a_vo[i],
                                                   aoff, 0, 0);
#pragma unroll
        for (int i = 0; i < NB; ++i)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lds_void*)(bbase + (size_t)(wave * NB + i) * 1024), 16,
                                                   b_vo[i], koff * (int)sizeof(T), 0, 0);
      } else {
#pragma unroll
        for (int i = 0; i < NA; ++i)
          __builtin_amdgcn_global_load_lds(a_src[i] + koff, (lds_void*)(base + (size_t)(wave * NA + i) * 1024), 16,
                                           0, 0);
#pragma unroll
        for (int i = 0; i < NB; ++i)
          __builtin_amdgcn_global_load_lds(b_src[i] + koff, (lds_void*)(bbase + (size_t)(wave * NB + i) * 1024), 16,
                                           0, 0);
      }
    };
    static_assert(KS == 1 || KS % 2 == 0, "one or an even number of k steps per tile");
    // Every iteration first refills the stage of k-tile kt-1 (its last reads
    // preceded the previous barrier) with k-tile kt+NST-1 (the index clamped at
    // the end, the redundant copies landing in stages nobody reads again), so
    // exactly NST-2 tiles may stay in flight when tile kt+1 is needed.
    constexpr int INFLIGHT = (NST - 2) * DPT;
    auto issue_c = [&](int kt) { issue(min(kt, nk - 1)); };
    // the LDS reads of the next fragments interleaved with the MFMAs of this step
    auto interleave = [&]() {
#pragma unroll
      for (int q = 0; q < TM + TN; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, (TM * TN) / (TM + TN), 0);  // MFMAs
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one DS read
      }
    };

#pragma unroll
    for (int s0 = 0; s0 < NST - 1; ++s0) issue_c(s0);
    wait_vmcnt<NST == 2 ? 0 : INFLIGHT>();
    barrier_lds();
    load_frags(0, 0, 0);
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt % NST;
      issue_c(kt + NST - 1);
      if constexpr (KS >= 2) {
        // k steps 0 .. KS-2 with the fragments of the next step loading meanwhile
#pragma unroll
        for (int ks = 0; ks + 1 < KS; ++ks) {
          load_frags(cur, ks + 1, (ks + 1) & 1);
          mma_step(ks & 1);
          interleave();
        }
        wait_vmcnt<INFLIGHT>();  // k-tile kt+1 has landed
        barrier_lds();
        load_frags((kt + 1) % NST, 0, 0);
        mma_step((KS - 1) & 1);
        interleave();
      } else {
        mma_step(0);
        wait_vmcnt<INFLIGHT>();
        barrier_lds();
        load_frags((kt + 1) % NST, 0, 0);
      }
    }
    wait_vmcnt<0>();
    __syncthreads();
  } else {
    // ---- gathered A (patch embedding): global -> registers -> LDS, zero-filled K tail,
    // two ring stages
    int pf[C::A_PT], pi[C::A_PT], pj[C::A_PT], pzb[C::A_PT];
#pragma unroll
    for (int u = 0; u < C::A_PT; ++u) {
      int idx = min(tid + NT * u, BM * CPR - 1);
      int r = m0 + idx / CPR;
      r = min(r, g.M - 1);
      int b = r / g.c_rpb, t = r - b * g.c_rpb;
      int hh = g.H / 2, ww = g.W / 2;
      pf[u] = t / (hh * ww);
      int rem = t - pf[u] * hh * ww;
      pi[u] = rem / ww;
      pj[u] = rem - pi[u] * ww;
      pzb[u] = b % g.z_batch;
    }
    const T* b_ptr[C::B_PT];
#pragma unroll
    for (int u = 0; u < C::B_PT; ++u) {
      int idx = min(tid + NT * u, BN * CPR - 1);
      b_ptr[u] = reinterpret_cast<const T*>(g.Wt) + (long long)(n0 + idx / CPR) * g.ldw;
    }
    Chunk<T> ra[C::A_PT], rb[C::B_PT];
    auto load_tile = [&](int kt) {
      const int kb = kt * BK;
#pragma unroll
      for (int u = 0; u < C::A_PT; ++u) {
        int c = (tid + NT * u) % CPR;
        int k0 = kb + c * 8;
        if (k0 < g.K)
          load_patch_chunk<T>(ra[u], g, pzb[u], pf[u], pi[u], pj[u], k0);
        else
          ra[u].zero();
      }
#pragma unroll
      for (int u = 0; u < C::B_PT; ++u) {
        int c = (tid + NT * u) % CPR;
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
        int idx = tid + NT * u;
        if (idx >= BM * CPR) break;
        int r = idx / CPR, c = idx % CPR;
        ra[u].store(&sa[r * CPR + swz<RB, CPR>(r, c)]);
      }
#pragma unroll
      for (int u = 0; u < C::B_PT; ++u) {
        int idx = tid + NT * u;
        if (idx >= BN * CPR) break;
        int r = idx / CPR, c = idx % CPR;
        rb[u].store(&sb[r * CPR + swz<RB, CPR>(r, c)]);
      }
    };
    load_tile(0);
    store_tile(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      if (kt + 1 < nk) load_tile(kt + 1);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        load_frags(cur, ks, 0);
        mma_step(0);
      }
      if (kt + 1 < nk) store_tile(cur ^ 1);
      __syncthreads();
    }
  }

  if constexpr (C::MI16 && (EPI == EPI_STORE || EPI == EPI_STORE_GELU)) {
    // bf16 store epilogues of the 16x16 form: bias (and GELU) on the accumulators, then
    // the whole tile staged once in LDS as bf16 (half the bytes of the float32 slabs, one
    // barrier) and written as 16-byte row pieces; each sum sees the same float32
    // operations as in the general path, so the outputs are the same bits.
    // A staged row is 32 bytes past a multiple of 256: the 16 rows of one 8-byte write
    // instruction (32 bytes each) share the 8 bank groups of 32 bytes two by two.
    constexpr int SP = BN + 16;
    static_assert((size_t)BM * SP * sizeof(T) <= C::LDS_BYTES, "bf16 staging");
    T* stage16 = reinterpret_cast<T*>(smem_raw);
#pragma unroll
    for (int j = 0; j < TC16; ++j) {
      const int col = brow0 + 16 * j + 4 * (lane >> 4);
      f32x4 bj = {0.f, 0.f, 0.f, 0.f};
      if (g.bias) bj = *reinterpret_cast<const f32x4*>(g.bias + n0 + col);
#pragma unroll
      for (int i = 0; i < TR16; ++i) {
        const int row = arow0 + 16 * i + (lane & 15);
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = acc16[i][j][e] + bj[e];
          if constexpr (EPI == EPI_STORE_GELU) v[e] = gelu_erf(v[e]);
        }
        *reinterpret_cast<uint2*>(stage16 + row * SP + col) =
            make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
      }
    }
    __syncthreads();
    constexpr int CPR16 = BN / 8, IT16 = BM * CPR16 / NT;
    static_assert(IT16 * NT == BM * CPR16, "whole 16-byte pieces per thread");
#pragma unroll
    for (int it = 0; it < IT16; ++it) {
      const int idx = tid + it * NT;
      const int lrow = idx / CPR16, c8 = (idx % CPR16) * 8;
      const int row = m0 + lrow;
      if (row < g.M) {
        Chunk<T> c;
        c.load(stage16 + lrow * SP + c8);
        c.store(reinterpret_cast<T*>(g.C) + (long long)row * g.ldc + n0 + c8);
      }
    }
    return;
  }

  if constexpr (C::MI16 && EPI == EPI_PACK && sizeof(T) == 2 && BN / WN == 128) {
    // q / k tiles of the 16x16 form: a lane holds four consecutive features of one token
    // per accumulator block, i.e. two whole RoPE pairs, and each wave's 128 columns are
    // one head.  Bias, rotation, q scale and the k-row norms are applied to the
    // accumulators; the tile is then staged once as bf16 (like the store epilogues) and
    // written as 16-byte pieces of head-major rows.  v^T tiles take the general path.
    const int sec0 = n0 < g.nq ? 0 : g.nq;
    const int sec_end = n0 < g.nq ? g.nq : g.nq + g.nk;
    if (n0 < g.nq + g.nk && n0 + BN <= sec_end && g.hd == 128 && (n0 - sec0) % 128 == 0 &&
        g.c_rpb % BM == 0) {
      constexpr int SP = BN + 16;
      static_assert((size_t)BM * SP * sizeof(T) <= C::LDS_BYTES, "bf16 staging");
      T* stage16 = reinterpret_cast<T*>(smem_raw);
      const bool is_k = n0 >= g.nq;  // (a K / V-only packing GEMM has nq = 0)
      const int b = m0 / g.c_rpb, t0 = m0 - b * g.c_rpb;
      const int valid = g.c_valid > 0 ? g.c_valid : g.c_rpb;
      const float qsc = is_k ? 1.0f : g.q_scale;
      const bool kmax_on = is_k && g.kpart != nullptr;
      f32x4 bj[TC16];
#pragma unroll
      for (int j = 0; j < TC16; ++j) {
        bj[j] = (f32x4){0.f, 0.f, 0.f, 0.f};
        if (g.bias) bj[j] = *reinterpret_cast<const f32x4*>(g.bias + n0 + brow0 + 16 * j + 4 * (lane >> 4));
      }
      float kacc = 0.f;  // largest |k|^2 over this lane's rows
#pragma unroll
      for (int i = 0; i < TR16; ++i) {
        const int row = arow0 + 16 * i + (lane & 15);
        const int t = t0 + row;
        const bool live = t < valid && m0 + row < g.M;
        // (cos, sin) of the lane's two pairs in each block; padding rows read the last token's
        const float2* rrow = g.rope ? g.rope + (long long)min(t, valid - 1) * 64 : nullptr;
        f32x4 cs[TC16];
        if (rrow) {
#pragma unroll
          for (int j = 0; j < TC16; ++j) cs[j] = *reinterpret_cast<const f32x4*>(rrow + 8 * j + 2 * (lane >> 4));
        }
        float sq = 0.f;
#pragma unroll
        for (int j = 0; j < TC16; ++j) {
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc16[i][j][e] + bj[j][e];
          if (rrow) {
#pragma unroll
            for (int u = 0; u < 4; u += 2) {
              const float u0 = v[u], u1 = v[u + 1], c = cs[j][u], s = cs[j][u + 1];
              v[u] = u0 * c - u1 * s;
              v[u + 1] = u0 * s + u1 * c;
            }
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] *= qsc;
          if (kmax_on) {
#pragma unroll
            for (int e = 0; e < 4; ++e) sq = __builtin_fmaf(v[e], v[e], sq);
          }
          *reinterpret_cast<uint2*>(stage16 + row * SP + brow0 + 16 * j + 4 * (lane >> 4)) =
              make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        }
        if (kmax_on) {
          // the row's |k|^2 before the bf16 rounding (rounding to nearest moves a norm by at most
          // 2^-9 of itself; the attention's margin covers that): four lanes of 32 features each
          sq += __shfl_xor(sq, 16, 64);
          sq += __shfl_xor(sq, 32, 64);
          if (live) kacc = __builtin_elementwise_maximum(kacc, sq);
        }
      }
      if (kmax_on) {
        // one partial maximum per wave; the head's 256-row tile has 8 slots and WM waves
        // cover it, so each wave fills 8 / WM of them (the attention takes the maximum)
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) kacc = __builtin_elementwise_maximum(kacc, __shfl_xor(kacc, o, 64));
        if (lane == 0) {
          const int hh = (n0 + brow0 - g.nq) / 128, mt = t0 / BM;
          float* kp = g.kpart + ((long long)b * g.heads + hh) * g.kpart_n + mt * 8 + (8 / WM) * wm;
#pragma unroll
          for (int s = 0; s < 8 / WM; ++s) kp[s] = kacc;
        }
      }
      __syncthreads();
      constexpr int CPR16 = BN / 8, IT16 = BM * CPR16 / NT;
      static_assert(IT16 * NT == BM * CPR16, "whole 16-byte pieces per thread");
      T* base = reinterpret_cast<T*>(is_k ? g.k : g.q);
#pragma unroll
      for (int it = 0; it < IT16; ++it) {
        const int idx = tid + it * NT;
        const int lrow = idx / CPR16, c8 = (idx % CPR16) * 8;
        const int t = t0 + lrow;
        if (t < valid && m0 + lrow < g.M) {
          const int nsec = n0 - sec0 + c8;
          const long long rowidx = ((long long)b * g.heads + (nsec >> 7)) * g.Lp + t;
          Chunk<T> c;
          c.load(stage16 + lrow * SP + c8);
          c.store(base + rowidx * 128 + (nsec & 127));
        }
      }
      return;
    }
  }
  // ---- epilogue.  The fp32 tile goes through LDS in column slabs; phase 2
  // walks a slab in 8-element chunks and writes 16-byte pieces.
  float* slab = reinterpret_cast<float*>(smem_raw);
  constexpr int SW = C::SW, SWP = C::SWP, SWPT = C::SWPT;
  // v^T tiles of a packing GEMM whose rows lie in one batch item (row pitch a
  // multiple of BM): the slab is staged transposed, so that a lane reads 8
  // tokens of one feature column as two 16-byte LDS reads and writes them as
  // one 16-byte store
  constexpr bool PACK = C::PACK;
  // 8-bit q / k: the 16 lanes that hold one token row of a slab hold one whole head
  static_assert(EPI != EPI_PACK8 || SW % 128 == 0, "8-bit q / k need head-aligned slabs");
  const bool vt_tile = PACK && n0 >= g.nq + g.nk && g.c_rpb % BM == 0;
  // Phase 2 item it of a thread is chunk idx = tid + it * NT of the slab (row
  // idx / CPRS, columns 8 * (idx % CPRS) ..+7).  When NT is a multiple of CPRS the
  // chunk's columns are the same in every item, so the bias (and the gate of a
  // residual) is fetched once per slab.
  constexpr int CPRS = SW / 8, TOT = BM * CPRS, IT = (TOT + NT - 1) / NT;
  constexpr bool FIXC = NT % CPRS == 0;
  // batch items a residual tile's rows span: two gate rows cover the tile when the
  // items are at least a tile long
  const int gb_lo = m0 / g.c_rpb, gb_hi = min(m0 + BM - 1, g.M - 1) / g.c_rpb;
  const bool gate2 = FIXC && gb_hi - gb_lo <= 1;
  // residual epilogue without global loads in phase 2: the thread's chunk columns
  // are fixed (bias and gates fetched once per slab) and the residual rows are
  // fetched in two batches
  const bool fast_x = EPI == EPI_RESID && FIXC && (gate2 || !g.gate);
#pragma unroll
  for (int s0 = 0; s0 < BN; s0 += SW) {
    const int nbase = n0 + s0;
    int sec = 0;
    if (PACK) sec = nbase < g.nq ? 0 : (nbase < g.nq + g.nk ? 1 : 2);
    // Global inputs of this thread's phase-2 items (residual rows, gates, bias)
    // are fetched before the slab is staged, so their latency overlaps
    // the LDS staging and the barrier: an item waiting for its own load puts one
    // HBM round trip per item on the tile's critical path (one workgroup per CU
    // leaves nothing else to run meanwhile).
    // residual rows: registers for half the items (the other half is fetched in
    // one batch once the first half is done), which keeps the tile's accumulators
    // of the next slab and these rows within the register budget
    constexpr int NPX = EPI == EPI_RESID ? (IT + 1) / 2 : 1;
    f32x4 pre[NPX][2];
    auto load_x = [&](int it, int slot) {
      const int idx = tid + it * NT;
      const int lrow = idx / CPRS, row = m0 + lrow;
      if (idx >= TOT || row >= g.M) return;
      long long xrow = row;
      if (g.c_valid > 0) {
        const int b = row / g.c_rpb, t = row - b * g.c_rpb;
        if (t >= g.c_valid) return;
        xrow = (long long)b * g.c_valid + t;
      }
      const float* xp = g.x + xrow * g.ldx + nbase + (idx % CPRS) * 8;
      pre[slot][0] = *reinterpret_cast<const f32x4*>(xp);
      pre[slot][1] = *reinterpret_cast<const f32x4*>(xp + 4);
    };
    f32x4 pbias[2], pgate[2][2];
    const int c8f = (tid % CPRS) * 8;
    if (FIXC && g.bias && !(PACK && vt_tile)) {
      pbias[0] = *reinterpret_cast<const f32x4*>(g.bias + nbase + c8f);
      pbias[1] = *reinterpret_cast<const f32x4*>(g.bias + nbase + c8f + 4);
    }
    if (fast_x) {
      if (g.gate) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float* gp = g.gate + (long long)(h ? gb_hi : gb_lo) * g.gate_bstride + nbase + c8f;
          pgate[h][0] = *reinterpret_cast<const f32x4*>(gp);
          pgate[h][1] = *reinterpret_cast<const f32x4*>(gp + 4);
        }
      }
#pragma unroll
      for (int it = 0; it < NPX; ++it) load_x(it, it);
    }
    // phase 1: the accumulators hold C^T (the weight fragment is the MFMA row
    // operand), so element r of lane l is column 8*(r/4) + 4*g2 + r%4, row l32 of
    // its 32x32 block: four consecutive columns per lane, one 16-byte LDS write
    // (four 4-byte writes down four columns for a transposed slab)
    if constexpr (C::MI16) {
      // 16x16 blocks: element e of lane l is column 4*(l/16) + e, row l%16 of its block
      if (brow0 + BN / WN > s0 && brow0 < s0 + SW) {
#pragma unroll
        for (int j = 0; j < TC16; ++j) {
          const int col = brow0 + 16 * j + 4 * (lane >> 4) - s0;
          if (col < 0 || col >= SW) continue;
#pragma unroll
          for (int i = 0; i < TR16; ++i) {
            const int row = arow0 + 16 * i + (lane & 15);
            if (PACK && vt_tile) {
#pragma unroll
              for (int e = 0; e < 4; ++e) slab[(col + e) * SWPT + row] = acc16[i][j][e];
            } else {
              *reinterpret_cast<f32x4*>(&slab[row * SWP + col]) = acc16[i][j];
            }
          }
        }
      }
    } else if (brow0 + BN / WN > s0 && brow0 < s0 + SW) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int col = brow0 + 32 * j + 8 * rq + 4 * g2 - s0;
          if (col < 0 || col >= SW) continue;
#pragma unroll
          for (int i = 0; i < TM; ++i) {
            const int row = arow0 + 32 * i + l32;
            if (PACK && vt_tile) {
#pragma unroll
              for (int e = 0; e < 4; ++e) slab[(col + e) * SWPT + row] = acc[i][j][4 * rq + e];
            } else {
              const f32x4 q4 = {acc[i][j][4 * rq], acc[i][j][4 * rq + 1], acc[i][j][4 * rq + 2],
                                acc[i][j][4 * rq + 3]};
              *reinterpret_cast<f32x4*>(&slab[row * SWP + col]) = q4;
            }
          }
        }
      }
    }
    __syncthreads();
    // phase 2
    if (PACK && vt_tile) {
      // v^T from the transposed slab.  Lane work item (column, 16-token group,
      // half hf): tokens 4hf..4hf+3 and 8+4hf..8+4hf+3 of the group, which the
      // key permutation stores at positions 8hf..8hf+7 -- one 16-byte store;
      // 32 consecutive items cover 512 contiguous bytes of one v^T row.
      const int nv0 = nbase - g.nq - g.nk;
      const int b0 = m0 / g.c_rpb, t0 = m0 - b0 * g.c_rpb;
      const int valid = g.c_valid > 0 ? g.c_valid : g.c_rpb;
      constexpr int NG = BM / 16;
      for (int idx = tid; idx < SW * NG * 2; idx += NT) {
        const int hf = idx & 1;
        const int grp = (idx >> 1) % NG;
        const int col = (idx >> 1) / NG;
        const float* sp = slab + col * SWPT + 16 * grp + 4 * hf;
        const f32x4 lo = *reinterpret_cast<const f32x4*>(sp);
        const f32x4 hi = *reinterpret_cast<const f32x4*>(sp + 8);
        const float bn = g.bias[nbase + col];
        float v[8];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          v[u] = lo[u] + bn;
          v[4 + u] = hi[u] + bn;
        }
        const int nvc = nv0 + col;
        const int hh = nvc / g.hd, e = nvc - hh * g.hd;
        T* vrow = reinterpret_cast<T*>(g.vt) + (((long long)b0 * g.heads + hh) * g.hd + e) * g.Lp;
        const int tb = t0 + 16 * grp;
        if (tb + 16 <= valid) {
          Chunk<T> c;
          pack8(c, v);
          c.store(vrow + tb + 8 * hf);
        } else {
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int tok = tb + 4 * hf + (u < 4 ? u : u + 4);
            if (tok < valid) vrow[vt_perm(tok)] = from_f<T>(v[u]);
          }
        }
      }
    } else if (PACK && sec == 2) {
      // v^T: a chunk is 8 consecutive tokens of one feature column
      const int nv0 = nbase - g.nq - g.nk;
      for (int idx = tid; idx < SW * (BM / 8); idx += NT) {
        const int col = idx % SW;
        const int r8 = (idx / SW) * 8;
        const int nvc = nv0 + col;
        const int hh = nvc / g.hd, e = nvc - hh * g.hd;
        const float bn = g.bias[nbase + col];
        const int row0 = m0 + r8;
        if (row0 >= g.M) continue;
        const int b0 = row0 / g.c_rpb, t0 = row0 - b0 * g.c_rpb;
        const int valid = g.c_valid > 0 ? g.c_valid : g.c_rpb;
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = slab[(r8 + u) * SWP + col] + bn;
        T* vrow = reinterpret_cast<T*>(g.vt) + (((long long)b0 * g.heads + hh) * g.hd + e) * g.Lp;
        if ((t0 & 7) == 0 && t0 + 8 <= valid && row0 + 8 <= g.M) {
          // 8 aligned tokens: two runs of 4 that stay contiguous under the key permutation
#pragma unroll
          for (int u = 0; u < 8; ++u) vrow[vt_perm(t0 + u)] = from_f<T>(v[u]);
        } else {
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int rr = row0 + u;
            if (rr >= g.M) break;
            const int b = rr / g.c_rpb, t = rr - b * g.c_rpb;
            if (t >= valid) continue;
            reinterpret_cast<T*>(g.vt)[(((long long)b * g.heads + hh) * g.hd + e) * g.Lp + vt_perm(t)] =
                from_f<T>(v[u]);
          }
        }
      }
    } else if (EPI == EPI_RESID && fast_x) {
#pragma unroll
      for (int it = 0; it < IT; ++it) {
        if (it == NPX) {
#pragma unroll
          for (int i2 = NPX; i2 < IT; ++i2) load_x(i2, i2 - NPX);
        }
        const int idx = tid + it * NT;
        if (idx >= TOT) break;
        const int lrow = idx / CPRS, row = m0 + lrow;
        const f32x4 lo = *reinterpret_cast<const f32x4*>(&slab[lrow * SWP + c8f]);
        const f32x4 hi = *reinterpret_cast<const f32x4*>(&slab[lrow * SWP + c8f + 4]);
        f32x4 y0 = lo, y1 = hi;
        if (g.bias) {
          y0 += pbias[0];
          y1 += pbias[1];
        }
        f32x4 x0 = pre[it % NPX][0], x1 = pre[it % NPX][1];
        const int b = row / g.c_rpb, t = row - b * g.c_rpb;
        if (g.gate) {
          const bool h = b != gb_lo;
          const f32x4 g0 = h ? pgate[1][0] : pgate[0][0];
          const f32x4 g1 = h ? pgate[1][1] : pgate[0][1];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            x0[u] += g0[u] * y0[u];
            x1[u] += g1[u] * y1[u];
          }
        } else {
          x0 += y0;
          x1 += y1;
        }
        if (row < g.M && (g.c_valid <= 0 || t < g.c_valid)) {
          const long long xrow = g.c_valid > 0 ? (long long)b * g.c_valid + t : (long long)row;
          float* xp = g.x + xrow * g.ldx + nbase + c8f;
          *reinterpret_cast<f32x4*>(xp) = x0;
          *reinterpret_cast<f32x4*>(xp + 4) = x1;
        }
      }
    } else {
      // k rows of a packing GEMM with kpart: each (row, head) of a 128-column slab sits in 16
      // consecutive lanes (one 8-column chunk each); a thread keeps the largest |k|^2 it saw
      constexpr bool KMAX = (EPI == EPI_PACK || EPI == EPI_PACK8) && SW == 128 && NT % 16 == 0;
      const bool kmax_on = KMAX && g.kpart && sec == 1;
      float ksq[KMAX ? IT : 1];  // this thread's chunk of each item's row: sum of 8 squares
#pragma unroll
      for (int it = 0; it < (KMAX ? IT : 1); ++it) ksq[it] = 0.f;
#pragma unroll
      for (int it = 0; it < IT; ++it) {
        const int idx = tid + it * NT;
        if (idx >= TOT) break;
        const int lrow = idx / CPRS;
        const int c8 = (idx % CPRS) * 8;
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
          f32x4 b0, b1;
          if constexpr (FIXC) {
            b0 = pbias[0];
            b1 = pbias[1];
          } else {
            b0 = *reinterpret_cast<const f32x4*>(g.bias + n);
            b1 = *reinterpret_cast<const f32x4*>(g.bias + n + 4);
          }
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            v[u] += b0[u];
            v[4 + u] += b1[u];
          }
        }
        if constexpr (EPI == EPI_CONV || EPI == EPI_CONV_VIDEO) {
          const int hw = g.cv_h * g.cv_w;
          const int tv = row / hw, rem = row - tv * hw;
          const int hv = rem / g.cv_w, wv = rem - hv * g.cv_w;
          if constexpr (EPI == EPI_CONV) {
            int ch = n, fr = g.cv_of0 + g.cv_ofs * tv;
            if (n >= g.cv_split) {
              ch = n - g.cv_split;
              fr += 1;
            }
            const long long off = (((long long)(fr + 2) * g.cv_hp + hv + 1) * g.cv_wp + wv + 1) * g.ldc + ch;
            if (g.cv_res) {
              Chunk<T> rc;
              rc.load(reinterpret_cast<const T*>(g.cv_res) + off);
              const bf16x8 r8 = as_bf16x8(rc.v);
#pragma unroll
              for (int u = 0; u < 8; ++u) v[u] += (float)r8[u];
            }
            Chunk<T> c;
            pack8(c, v);
            c.store(reinterpret_cast<T*>(g.C) + off);
          } else {
            const long long px = (long long)(g.cv_of0 + tv) * hw + rem;
#pragma unroll
            for (int u = 0; u < 8; ++u)
              if (n + u < g.cv_nout) reinterpret_cast<float*>(g.C)[(long long)(n + u) * g.ldc + px] = v[u];
          }
        } else if constexpr (EPI == EPI_STORE_GELU8) {
          // GELU, then e4m3 with one power-of-two scale per (row, 128-column block):
          // the 16 lanes of this row within the 128-column slab hold the block
#pragma unroll
          for (int u = 0; u < 8; ++u) v[u] = gelu_erf(v[u]);
          float am = 0.f;
#pragma unroll
          for (int u = 0; u < 8; ++u) am = __builtin_elementwise_maximum(am, fabsf(v[u]));
#pragma unroll
          for (int o = 1; o < 16; o <<= 1) am = __builtin_elementwise_maximum(am, __shfl_xor(am, o, 64));
          const int ex = e8_exponent(am);
          const float inv = __uint_as_float((unsigned)(127 - ex) << 23);
          *reinterpret_cast<uint2*>(reinterpret_cast<unsigned char*>(g.C) + (long long)row * g.ldc + n) =
              e4m3_pack8(v, inv);
          if ((n & 127) == 0) g.c_scale[(long long)(n >> 7) * g.c_sld + row] = (unsigned char)(ex + 127);
        } else if (EPI == EPI_STORE || EPI == EPI_STORE_GELU) {
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
          long long xrow = row;
          if (g.c_valid > 0) {
            // padded row pitch: token t of batch item b is residual row b * c_valid + t
            const int b = row / g.c_rpb, t = row - b * g.c_rpb;
            if (t >= g.c_valid) continue;
            xrow = (long long)b * g.c_valid + t;
          }
          float* xp = g.x + xrow * g.ldx + n;
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
        } else if (PACK) {
          // q or k, with optional RoPE on the adjacent pairs of the chunk
          const int nsec = n - (sec == 0 ? 0 : g.nq);
          const int hh = nsec / g.hd, e0 = nsec - hh * g.hd;
          const int b = row / g.c_rpb, t = row - b * g.c_rpb;
          if (g.c_valid > 0 && t >= g.c_valid) continue;  // padding row
          if (g.rope) {
            // per-token (cos, sin) of the four pairs (e0, e0+1) .. (e0+6, e0+7)
            const f32x4* rp = reinterpret_cast<const f32x4*>(g.rope + (long long)t * (g.hd / 2) + e0 / 2);
            const f32x4 c01 = rp[0], c23 = rp[1];
            const float cs[8] = {c01[0], c01[1], c01[2], c01[3], c23[0], c23[1], c23[2], c23[3]};
#pragma unroll
            for (int u = 0; u < 8; u += 2) {
              const float u0 = v[u], u1 = v[u + 1];
              v[u] = u0 * cs[u] - u1 * cs[u + 1];
              v[u + 1] = u0 * cs[u + 1] + u1 * cs[u];
            }
          }
          const long long rowidx = ((long long)b * g.heads + hh) * g.Lp + t;
          if (sec == 0 && g.q_scale != 1.0f) {
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] *= g.q_scale;
          }
          if constexpr (EPI == EPI_PACK8) {
            // e4m3 with one power-of-two scale per (token, head), stored as the
            // byte e + 127 (e8_exponent); max|row| gathers over the 16 lanes of the head
            float am = 0.f;
#pragma unroll
            for (int u = 0; u < 8; ++u) am = __builtin_elementwise_maximum(am, fabsf(v[u]));
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) am = __builtin_elementwise_maximum(am, __shfl_xor(am, o, 64));
            const int ex = e8_exponent(am);
            const float inv = __uint_as_float((unsigned)(127 - ex) << 23);  // 2^-e, exact scaling
            unsigned char* base = reinterpret_cast<unsigned char*>(sec == 0 ? g.q : g.k);
            *reinterpret_cast<uint2*>(base + rowidx * g.hd + e0) = e4m3_pack8(v, inv);
            if (e0 == 0) (sec == 0 ? g.qs : g.ks)[rowidx] = (unsigned char)(ex + 127);
            if constexpr (KMAX) {
              if (kmax_on) {
                // |k|^2 before the e4m3 rounding, this chunk's share (the attention's margin
                // covers the rounding)
                float sq = 0.f;
#pragma unroll
                for (int u = 0; u < 8; ++u) sq = __builtin_fmaf(v[u], v[u], sq);
                ksq[it] = sq;
              }
            }
          } else {
            Chunk<T> c;
            pack8(c, v);
            T* base = reinterpret_cast<T*>(sec == 0 ? g.q : g.k);
            c.store(base + rowidx * g.hd + e0);
            if constexpr (KMAX) {
              if (kmax_on) {
                // |k|^2 of the row before its rounding to bf16, this chunk's share (rounding
                // to nearest moves a norm by at most 2^-9 of itself; the attention's margin
                // covers that)
                float sq = 0.f;
#pragma unroll
                for (int u = 0; u < 8; ++u) sq = __builtin_fmaf(v[u], v[u], sq);
                ksq[it] = sq;
              }
            }
          }
        }
      }
      if constexpr (KMAX) {
        if (kmax_on) {
          // row sums over each row's 16 lanes (skipped rows hold zeros), the largest of this
          // thread's rows, the wave's four row groups, then one partial maximum per wave (no
          // atomics: the attention kernel reduces the partials of its (batch item, head))
          float kacc = 0.f;
#pragma unroll
          for (int it = 0; it < IT; ++it) kacc = __builtin_elementwise_maximum(kacc, row16_sum(ksq[it]));
          kacc = __builtin_elementwise_maximum(kacc, __shfl_xor(kacc, 16, 64));
          kacc = __builtin_elementwise_maximum(kacc, __shfl_xor(kacc, 32, 64));
          if (lane == 0) {
            const int hh = (nbase - g.nq) / g.hd;
            const int b = m0 / g.c_rpb, mt = (m0 - b * g.c_rpb) / BM;
            g.kpart[((long long)b * g.heads + hh) * g.kpart_n + mt * C::NW + wave] = kacc;
          }
        }
      }
    }
    __syncthreads();
  }
}

// The kernel body lives in a device function: the host pass only sees this wrapper.
// OCC workgroups share a CU (it bounds the registers per wave).
template <typename T, int BM, int BN, int WM, int WN, int NST, int RB, int OCC, int LOADER, int EPI, int MI = 32>
__global__ __launch_bounds__(64 * WM * WN, OCC) void gemm_kernel(const GemmArgs g) {
  gemm_body<T, BM, BN, WM, WN, NST, RB, LOADER, EPI, MI>(g);
}

template <typename T, int BM, int BN, int WM, int WN, int NST, int RB, int OCC, int LOADER, int EPI, int MI = 32>
hipError_t launch_cfg(const GemmArgs& g, hipStream_t st) {
  using C = Gemm<T, BM, BN, WM, WN, NST, RB, LOADER, EPI, MI>;
  static_assert(OCC * C::LDS_BYTES <= 160 * 1024, "occupancy exceeds the LDS");
  if (g.N % BN != 0) return hipErrorInvalidValue;
  if ((LOADER == LOAD_PLAIN || LOADER == LOAD_FP8 || LOADER == LOAD_CONV) && g.K % C::BK != 0)
    return hipErrorInvalidValue;
  // the k-row norms need one 128-wide head per 128-column slab, and tiles inside one batch item
  if (g.kpart && !((EPI == EPI_PACK || EPI == EPI_PACK8) && C::SW == 128 && C::NT % 16 == 0 && g.hd == 128 && g.c_rpb % BM == 0 &&
                   g.nq % 128 == 0 && g.kpart_n == g.c_rpb / BM * (C::MI16 ? 8 : C::NW)))
    return hipErrorInvalidValue;
  auto kern = gemm_kernel<T, BM, BN, WM, WN, NST, RB, OCC, LOADER, EPI, MI>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::LDS_BYTES);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int nm = (g.M + BM - 1) / BM;
  const int nt = nm * (g.N / BN);
  hipLaunchKernelGGL(kern, dim3(nt), dim3(C::NT), C::LDS_BYTES, st, g);
  return hipGetLastError();
}

// The split-ring path addresses each operand from its tile's first row with
// 32-bit byte offsets: rows of one tile may span a batch boundary of A.
// Elements from a tile's first A row to the end of its last k-slice: a tile of
// 256 rows spans at most 256 / a_rpb + 1 batch items.
inline long long split_a_span(const GemmArgs& g) {
  const long long items = g.a_rpb < g.M ? 256LL / g.a_rpb + 1 : 0LL;
  return items * g.a_bstride + 256LL * g.lda + g.K;
}

// The convolution loader addresses A from the tile's first output voxel: lane offsets
// cover the frames a tile's 256 voxels can touch, the scalar offset the largest tap
// offset plus one tap's channels; W from the tile's first row.  Both must stay below
// 2^31 bytes, and no tap may point before the voxel's row.
inline bool conv_offsets_fit(const GemmArgs& g) {
  const long long hw = (long long)g.cv_h * g.cv_w;
  const long long lane_span = (256 / hw + 2) * g.cv_hp * g.cv_wp * g.lda;
  long long tap_max = 0;
  for (int i = 0; i < CONV_MAX_TAPS; ++i) {
    if (g.tap_off[i] < 0) return false;
    tap_max = tap_max > g.tap_off[i] ? tap_max : g.tap_off[i];
  }
  const long long w_span = 256LL * g.ldw + g.K;
  return (lane_span + tap_max + g.K) * 2 < (1LL << 31) && w_span * 2 < (1LL << 31);
}

template <typename T>
bool split_offsets_fit(const GemmArgs& g) {
  const long long w_span = 256LL * g.ldw + g.K;
  return g.a_bstride >= 0 && split_a_span(g) * (long long)sizeof(T) < (1LL << 32) &&
         w_span * (long long)sizeof(T) < (1LL << 32);
}

template <typename T, int LOADER, int EPI>
hipError_t launch_by_n(const GemmArgs& g, hipStream_t st) {
  if constexpr (sizeof(T) == 2) {
    // 256x256 tiles of 8 waves over 64-deep k-tiles in split rings (the
    // refill moves 128-byte row pieces); the configurations below serve K not a
    // multiple of 64 and the other loaders.
    // Fewer tiles than CUs (short sequences): 256x192 tiles (64x96 per wave) when
    // N allows, a third more of them; fewer than 128 tiles (the context K / V
    // projections): 128x64 tiles instead.
    const long long big_tiles = (long long)((g.M + 255) / 256) * (g.N / 256);
    if constexpr (LOADER == LOAD_PLAIN)
      if (g.N % 256 == 0 && g.K % 64 == 0 && big_tiles >= 128 && split_offsets_fit<T>(g)) {
        if (big_tiles < 256 && g.N % 192 == 0) return launch_cfg<T, 256, 192, 4, 2, 3, 128, 1, LOADER, EPI>(g, st);
        // 16x16x32 MFMAs (measured on the 1.3B step shapes, same box): the packing epilogue
        // gains 10% on 8 waves (4 waves spill its v^T staging); FFN1+GELU and a long-K residual
        // GEMM (FFN2, K = 8960) run best on 4 waves of 128x128 (two thirds of the LDS fragment
        // reads per MFMA), while the short-K residual GEMMs (K = 1536), whose epilogue
        // dominates, stay on 8 waves of 32x32x16 (the 4-wave and the 8-wave 16x16 forms are
        // 2% and 1% slower there)
        if constexpr (EPI == EPI_PACK)
          return launch_cfg<T, 256, 256, 4, 2, 3, 128, 1, LOADER, EPI, 16>(g, st);
        if constexpr (EPI == EPI_STORE_GELU)
          return launch_cfg<T, 256, 256, 2, 2, 3, 128, 1, LOADER, EPI, 16>(g, st);
        if constexpr (EPI == EPI_RESID)
          if (g.K >= 4096) return launch_cfg<T, 256, 256, 2, 2, 3, 128, 1, LOADER, EPI, 16>(g, st);
        return launch_cfg<T, 256, 256, 4, 2, 3, 128, 1, LOADER, EPI>(g, st);
      }
    if constexpr (LOADER == LOAD_PLAIN)
      if (big_tiles < 128 && g.N % 64 == 0) return launch_cfg<T, 128, 64, 4, 1, 4, 64, 1, LOADER, EPI>(g, st);
    // Fallbacks on 64-byte rows (K not a multiple of 64, lane offsets beyond 32
    // bits, N not a multiple of 256).  Short-K GEMMs with a heavy epilogue (GELU,
    // residual read-modify-write): 256x128 tiles of 4 waves and a three-stage
    // ring (72 KB) give two workgroups per CU, so one workgroup's epilogue
    // overlaps the other's main loop.  Otherwise 256x256 tiles of 8 waves (two
    // per SIMD, 64x128 each) and a four-stage ring, or 128x64 tiles.
    constexpr bool heavy_epi = EPI == EPI_STORE_GELU || EPI == EPI_RESID;
    if (heavy_epi && g.K <= 2048 && g.N % 128 == 0) return launch_cfg<T, 256, 128, 2, 2, 3, 64, 2, LOADER, EPI>(g, st);
    if (g.N % 256 == 0) return launch_cfg<T, 256, 256, 4, 2, 4, 64, 1, LOADER, EPI>(g, st);
    if (g.N % 64 == 0) return launch_cfg<T, 128, 64, 4, 1, 4, 64, 1, LOADER, EPI>(g, st);
  } else {
    if (g.N % 128 == 0) return launch_cfg<T, 128, 128, 2, 2, 4, 64, 1, LOADER, EPI>(g, st);
    if (g.N % 64 == 0) return launch_cfg<T, 128, 64, 4, 1, 4, 64, 1, LOADER, EPI>(g, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

template <typename T>
hipError_t launch_gemm(const GemmArgs& g, int loader, int epi, hipStream_t st) {
  if (g.M <= 0) return hipSuccess;
  // the LDS-DMA path streams whole k-tiles: K must be a multiple of the k-tile depth
  constexpr int BK = sizeof(T) == 2 ? 32 : 16;
  if (loader == LOAD_FP8 && epi != EPI_PACK && epi != EPI_PACK8 && epi != EPI_STORE_GELU8 && epi != EPI_RESID)
    return hipErrorInvalidValue;
  if (loader == LOAD_PLAIN && g.K % BK != 0) return hipErrorInvalidValue;
  if (loader == LOAD_PATCH) {
    if (epi == EPI_STORE_F32) return launch_by_n<T, LOAD_PATCH, EPI_STORE_F32>(g, st);
    return hipErrorInvalidValue;
  }
  if (loader == LOAD_CONV) {
    // bf16 convolutions: whole 32-channel k-tiles per tap
    if constexpr (sizeof(T) == 2) {
      if (g.K % 32 != 0 || g.cv_kpt < 1 || g.K / 32 > g.cv_kpt * CONV_MAX_TAPS || g.K % (32 * g.cv_kpt) != 0 ||
          g.cv_h < 1 || g.cv_w < 1 || !conv_offsets_fit(g))
        return hipErrorInvalidValue;
      if (epi == EPI_CONV) {
        // a small chunk (fewer than 128 tiles of 256 rows, e.g. one latent frame at the
        // lowest level): 128x64 tiles, so that most CUs get work
        const long long rows256 = (g.M + 255) / 256;
        const long long tiles = rows256 * (g.N % 256 == 0 ? g.N / 256 : g.N % 192 == 0 ? g.N / 192 : g.N / 128);
        if (tiles < 128 && g.N % 64 == 0) return launch_cfg<T, 128, 64, 4, 1, 4, 64, 1, LOAD_CONV, EPI_CONV>(g, st);
        // taps of whole 64-channel k-tiles: split rings, 256x256 or 256x192 tiles (64x96 per wave)
        if (g.cv_kpt % 2 == 0) {
          if (g.N % 256 == 0) return launch_cfg<T, 256, 256, 4, 2, 3, 128, 1, LOAD_CONV, EPI_CONV>(g, st);
          if (g.N % 192 == 0) return launch_cfg<T, 256, 192, 4, 2, 3, 128, 1, LOAD_CONV, EPI_CONV>(g, st);
        }
        if (g.N % 256 == 0) return launch_cfg<T, 256, 256, 4, 2, 4, 64, 1, LOAD_CONV, EPI_CONV>(g, st);
        if (g.N % 128 == 0) return launch_cfg<T, 256, 128, 2, 2, 3, 64, 2, LOAD_CONV, EPI_CONV>(g, st);
        // 192-wide outputs: 128x192 tiles of 4 waves (64x96 each), two workgroups per CU
        if (g.N % 192 == 0) return launch_cfg<T, 128, 192, 2, 2, 4, 64, 2, LOAD_CONV, EPI_CONV>(g, st);
        if (g.N % 64 == 0) return launch_cfg<T, 128, 64, 4, 1, 4, 64, 1, LOAD_CONV, EPI_CONV>(g, st);
        // 96-wide outputs: 192x96 tiles of 6 waves (32x96 each), two workgroups per CU
        if (g.N % 96 == 0) return launch_cfg<T, 192, 96, 6, 1, 4, 64, 2, LOAD_CONV, EPI_CONV>(g, st);
      } else if (epi == EPI_CONV_VIDEO) {
        if (g.N % 64 == 0) return launch_cfg<T, 128, 64, 4, 1, 4, 64, 1, LOAD_CONV, EPI_CONV_VIDEO>(g, st);
      }
    }
    return hipErrorInvalidValue;
  }
  if (loader == LOAD_FP8) {
    // e4m3 operands: 256x256 tiles of 8 waves; M a whole number of tiles (the scale
    // rows of a tile are read as one 256-byte run), K whole 128-blocks
    if constexpr (sizeof(T) == 2) {
      if (g.N % 256 != 0 || g.K % 128 != 0 || g.M % 256 != 0 || !g.a_scale || !g.w_scale || g.a_sld < g.M)
        return hipErrorInvalidValue;
      // split rings of 128-deep k-tiles when the tile-relative byte offsets fit 32 bits
      const bool split = split_offsets_fit<unsigned char>(g);  // e4m3: one byte per element
      switch (epi) {
        case EPI_PACK:
          if (split) return launch_cfg<T, 256, 256, 4, 2, 3, 128, 1, LOAD_FP8, EPI_PACK>(g, st);
          return launch_cfg<T, 256, 256, 4, 2, 4, 64, 1, LOAD_FP8, EPI_PACK>(g, st);
        case EPI_PACK8:
          if (g.hd != 128 || !g.qs || !g.ks) return hipErrorInvalidValue;
          if (split) return launch_cfg<T, 256, 256, 4, 2, 3, 128, 1, LOAD_FP8, EPI_PACK8>(g, st);
          return launch_cfg<T, 256, 256, 4, 2, 4, 64, 1, LOAD_FP8, EPI_PACK8>(g, st);
        case EPI_STORE_GELU8:
          if (!g.c_scale || g.c_sld < g.M) return hipErrorInvalidValue;
          if (split) return launch_cfg<T, 256, 256, 4, 2, 3, 128, 1, LOAD_FP8, EPI_STORE_GELU8>(g, st);
          return launch_cfg<T, 256, 256, 4, 2, 4, 64, 1, LOAD_FP8, EPI_STORE_GELU8>(g, st);
        case EPI_RESID:
          if (split) return launch_cfg<T, 256, 256, 4, 2, 3, 128, 1, LOAD_FP8, EPI_RESID>(g, st);
          return launch_cfg<T, 256, 256, 4, 2, 4, 64, 1, LOAD_FP8, EPI_RESID>(g, st);
      }
    }
    return hipErrorInvalidValue;
  }
  switch (epi) {
    case EPI_STORE: return launch_by_n<T, LOAD_PLAIN, EPI_STORE>(g, st);
    case EPI_STORE_GELU: return launch_by_n<T, LOAD_PLAIN, EPI_STORE_GELU>(g, st);
    case EPI_STORE_F32: return launch_by_n<T, LOAD_PLAIN, EPI_STORE_F32>(g, st);
    case EPI_RESID: return launch_by_n<T, LOAD_PLAIN, EPI_RESID>(g, st);
    case EPI_PACK: return launch_by_n<T, LOAD_PLAIN, EPI_PACK>(g, st);
    case EPI_PACK8:
      // 8-bit q / k need whole heads of 128 in one 128-column slab: 256x256 tiles only
      if constexpr (sizeof(T) == 2) {
        if (g.N % 256 != 0 || g.hd != 128 || !g.qs || !g.ks) return hipErrorInvalidValue;
        if (g.K % 64 == 0 && split_offsets_fit<T>(g))
          return launch_cfg<T, 256, 256, 4, 2, 3, 128, 1, LOAD_PLAIN, EPI_PACK8>(g, st);
        return launch_cfg<T, 256, 256, 4, 2, 4, 64, 1, LOAD_PLAIN, EPI_PACK8>(g, st);
      }
      return hipErrorInvalidValue;
  }
  return hipErrorInvalidValue;
}

template hipError_t launch_gemm<bf16>(const GemmArgs&, int, int, hipStream_t);
template hipError_t launch_gemm<float>(const GemmArgs&, int, int, hipStream_t);

}  // namespace wan
