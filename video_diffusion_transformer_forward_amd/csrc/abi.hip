// C ABI: argument validation, workspace planning and the launch sequences of
// the patchify, time-modulation, block, head and denoise-step entry points.
#include <math.h>
#include <string.h>

#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "../../include/wan.h"
#include "../../include/wan_vae.h"
#include "common.h"
#include "kernels.h"

namespace wan {
namespace {

constexpr size_t ALIGN = 256;
constexpr int MAX_DIM = 5120;  // the LayerNorm kernel keeps one row in a wave's registers
constexpr int MAX_CTX = 65536;
constexpr int MAX_TOKENS = 1 << 20;
constexpr int MAX_BLOCKS = 1024;
constexpr int TIME_DIM = 256;

size_t al(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }
int pad64(int x) { return (x + 63) / 64 * 64; }
// row pitch of the packing GEMMs: every 256-row tile lies inside one batch item
int pad256(int x) { return (x + 255) / 256 * 256; }

struct Dims {
  int B, Cin, F, H, W, Hh, Ww, L, Lp, D, heads, hd, Ff, Lt, Li, Lc, Ltp, Lip, mode;
  bool qk8;  // self-attention scores from 8-bit q and k (WAN_BF16_QK8, WAN_FP8)
  bool fp8;  // 8-bit projections (WAN_FP8)
  size_t es;
};

int check_shape(const wan_shape* s, Dims* d) {
  if (!s) return WAN_E_NULL;
  if (s->mode != WAN_BF16 && s->mode != WAN_FP32 && s->mode != WAN_BF16_QK8 && s->mode != WAN_FP8) return WAN_E_MODE;
  if (s->batch < 1 || (s->in_ch != 16 && s->in_ch != 36) || s->out_ch != 16) return WAN_E_SHAPE;
  if (s->frames < 1 || s->height < 2 || s->width < 2 || (s->height & 1) || (s->width & 1)) return WAN_E_SHAPE;
  if (s->dim < 256 || s->dim % 256 != 0 || s->dim > MAX_DIM) return WAN_E_SHAPE;
  if (s->heads < 1 || s->dim % s->heads != 0) return WAN_E_SHAPE;
  const int hd = s->dim / s->heads;
  if (hd != 64 && hd != 128) return WAN_E_SHAPE;
  if ((s->mode == WAN_BF16_QK8 || s->mode == WAN_FP8) && hd != 128) return WAN_E_SHAPE;
  if (s->ffn_dim < 256 || s->ffn_dim % 256 != 0 || s->ffn_dim > (1 << 16)) return WAN_E_SHAPE;
  if (s->txt_len < 1 || s->img_len < 0 || s->txt_len + s->img_len > MAX_CTX) return WAN_E_SHAPE;
  const long long L = (long long)s->frames * (s->height / 2) * (s->width / 2);
  if (L > MAX_TOKENS || (long long)s->batch * L * 2 > (1LL << 30)) return WAN_E_SHAPE;
  if (s->batch > 64) return WAN_E_SHAPE;
  if (d) {
    d->B = s->batch;
    d->Cin = s->in_ch;
    d->F = s->frames;
    d->H = s->height;
    d->W = s->width;
    d->Hh = s->height / 2;
    d->Ww = s->width / 2;
    d->L = (int)L;
    d->Lp = pad64((int)L);
    d->D = s->dim;
    d->heads = s->heads;
    d->hd = hd;
    d->Ff = s->ffn_dim;
    d->Lt = s->txt_len;
    d->Li = s->img_len;
    d->Lc = s->txt_len + s->img_len;
    d->Ltp = pad64(s->txt_len);
    d->Lip = pad64(s->img_len);
    d->mode = s->mode == WAN_FP32 ? WAN_FP32 : WAN_BF16;  // element type of the operands
    d->qk8 = s->mode == WAN_BF16_QK8 || s->mode == WAN_FP8;
    d->fp8 = s->mode == WAN_FP8;
    d->es = d->mode == WAN_BF16 ? 2 : 4;
  }
  return WAN_OK;
}

// Offsets (bytes) inside the workspace of one block run over Bb batch rows.
struct BlockPlan {
  size_t m, r1, q, k, vt, o, ck, cvt, ik, ivt, rope, ropet;
  // static-offset self-attention: partial maxima of |k|^2 per (batch item, head, 256-row
  // tile, wave of the QKV GEMM) and the per-workgroup fallback flags
  size_t kmax, aflag;
  // WAN_FP8: e4m3 LayerNorm outputs and their scales, e4m3 FFN hidden and its
  // scales, the block's e4m3 projection weights and their scales
  size_t m8, msc, h8, hsc, w8, wsc;
  size_t total;
};

// offsets of the four 8-bit weight matrices inside BlockPlan::w8 / ::wsc
struct W8Plan {
  size_t qkv, cq, ff1, ff2;       // bytes into w8
  size_t sqkv, scq, sff1, sff2;   // bytes into wsc
  size_t w_bytes, s_bytes;
};
W8Plan plan_w8(const Dims& d) {
  W8Plan w;
  const size_t D = d.D, F = d.Ff;
  w.qkv = 0;
  w.cq = 3 * D * D;
  w.ff1 = 4 * D * D;
  w.ff2 = 4 * D * D + F * D;
  w.w_bytes = 4 * D * D + 2 * F * D;
  w.sqkv = 0;
  w.scq = (D / 128) * 3 * D;
  w.sff1 = (D / 128) * 4 * D;
  w.sff2 = (D / 128) * (4 * D + F);
  w.s_bytes = (D / 128) * (4 * D + F) + (F / 128) * D;
  return w;
}

size_t rope_entries(const Dims& d) {
  const int ds = 2 * (d.hd / 6), df = d.hd - 2 * ds;
  return (size_t)d.F * (df / 2) + (size_t)d.Hh * (ds / 2) + (size_t)d.Ww * (ds / 2);
}

BlockPlan plan_block(const Dims& d, int Bb, size_t base) {
  BlockPlan p;
  const size_t es = d.es;
  size_t off = base;
  p.m = off;
  off += al((size_t)Bb * d.L * d.D * es);
  const size_t qkv1 = al((size_t)Bb * d.heads * d.Lp * d.hd * es);
  const size_t hbytes = al((size_t)Bb * d.L * d.Ff * es);
  p.r1 = off;
  p.q = off;
  p.k = off + qkv1;
  p.vt = off + 2 * qkv1;
  off += (3 * qkv1 > hbytes ? 3 * qkv1 : hbytes);
  p.o = off;
  off += al((size_t)Bb * d.L * d.D * es);
  p.ck = off;
  off += al((size_t)Bb * d.heads * d.Ltp * d.hd * es);
  p.cvt = off;
  off += al((size_t)Bb * d.heads * d.Ltp * d.hd * es);
  p.ik = off;
  p.ivt = off;
  if (d.Li > 0) {
    off += al((size_t)Bb * d.heads * d.Lip * d.hd * es);
    p.ivt = off;
    off += al((size_t)Bb * d.heads * d.Lip * d.hd * es);
  }
  p.rope = off;
  off += al(rope_entries(d) * sizeof(float2));
  p.ropet = off;
  off += al((size_t)d.L * (d.hd / 2) * sizeof(float2));
  p.kmax = off;
  off += al((size_t)Bb * d.heads * (pad256(d.L) / 256) * 8 * sizeof(float));
  p.aflag = off;
  off += al((size_t)attn_wide_flags(d.L, d.heads, Bb) * sizeof(int));
  p.m8 = p.msc = p.h8 = p.hsc = p.w8 = p.wsc = off;
  if (d.fp8) {
    const size_t rows_p = (size_t)Bb * pad256(d.L);  // padded token rows of the 8-bit GEMMs
    const W8Plan w8 = plan_w8(d);
    p.m8 = off;
    off += al((size_t)Bb * d.L * d.D);
    p.msc = off;
    off += al((size_t)(d.D / 128) * rows_p);
    p.h8 = off;
    off += al(rows_p * d.Ff);
    p.hsc = off;
    off += al((size_t)(d.Ff / 128) * rows_p);
    p.w8 = off;
    off += al(w8.w_bytes);
    p.wsc = off;
    off += al(w8.s_bytes);
  }
  p.total = off;
  return p;
}

struct StepPlan {
  size_t x, mod, t1, t2, p, ctx;
  BlockPlan blk;
  size_t total;
};

StepPlan plan_step(const Dims& d) {
  StepPlan p;
  size_t off = 0;
  const int B2 = 2 * d.B;
  p.x = off;
  off += al((size_t)B2 * d.L * d.D * 4);
  p.mod = off;
  off += al((size_t)6 * d.D * 4);
  p.t1 = off;
  off += al((size_t)d.D * 4);
  p.t2 = off;
  off += al((size_t)d.D * 4);
  p.p = off;
  off += al((size_t)B2 * d.L * 64 * 4);
  p.ctx = off;
  off += al((size_t)B2 * d.Lc * d.D * d.es);
  p.blk = plan_block(d, B2, off);
  p.total = p.blk.total;
  return p;
}

size_t head_bytes(const Dims& d) { return al((size_t)d.B * d.L * d.D * d.es) + al((size_t)d.B * d.L * 64 * 4); }
size_t time_bytes(const Dims& d) { return 2 * al((size_t)d.D * 4); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

int check_ptrs(std::initializer_list<const void*> ps) {
  for (const void* p : ps) {
    if (!p) return WAN_E_NULL;
    if (!aligned16(p)) return WAN_E_ALIGN;
  }
  return WAN_OK;
}

int check_block_weights(const wan_block_weights* w, const Dims& d) {
  if (!w) return WAN_E_NULL;
  int rc = check_ptrs({w->qkv_w, w->qkv_b, w->o_w, w->o_b, w->cq_w, w->cq_b, w->ckv_w, w->ckv_b, w->co_w, w->co_b,
                       w->ff1_w, w->ff1_b, w->ff2_w, w->ff2_b});
  if (rc) return rc;
  if (d.Li > 0) return check_ptrs({w->ikv_w, w->ikv_b});
  return WAN_OK;
}

int check_model_weights(const wan_model_weights* w, const Dims& d, bool blocks) {
  if (!w) return WAN_E_NULL;
  int rc = check_ptrs({w->pe_w, w->pe_b, w->t1_w, w->t1_b, w->t2_w, w->t2_b, w->m_w, w->m_b, w->hd_w, w->hd_b});
  if (rc) return rc;
  if (blocks) {
    if (w->n_blocks < 0 || w->n_blocks > MAX_BLOCKS) return WAN_E_SHAPE;
    if (w->n_blocks > 0 && !w->blocks) return WAN_E_NULL;
    for (int i = 0; i < w->n_blocks; ++i) {
      rc = check_block_weights(&w->blocks[i], d);
      if (rc) return rc;
    }
  }
  return WAN_OK;
}

int check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return WAN_OK;
  if (!ws || ws_bytes < need) return WAN_E_WORKSPACE;
  if (!aligned16(ws)) return WAN_E_ALIGN;
  return WAN_OK;
}

// A gfx950 device must be current; the answer is cached per device.
int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return WAN_E_HIP;
  static std::mutex mu;
  static int known[64] = {0};  // 0 unknown, 1 ok, -1 unusable
  if (dev >= 64) return WAN_E_HIP;
  std::lock_guard<std::mutex> lock(mu);
  if (known[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return WAN_E_HIP;
    known[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
  }
  return known[dev] == 1 ? WAN_OK : WAN_E_HIP;
}

#define HIP_TRY(expr)                          \
  do {                                         \
    if ((expr) != hipSuccess) return WAN_E_HIP; \
  } while (0)

// ---- optional event timing of kernel classes
constexpr int N_CLASSES = 4;
struct Timing {
  std::mutex mu;
  bool on = false;
  std::vector<hipEvent_t> pool;                                // free events
  std::vector<std::pair<hipEvent_t, hipEvent_t>> pending[N_CLASSES];
  double ms[N_CLASSES] = {0, 0, 0, 0};
  long long n[N_CLASSES] = {0, 0, 0, 0};
};
Timing& timing() {
  static Timing t;
  return t;
}
hipEvent_t take_event(Timing& t) {
  if (!t.pool.empty()) {
    hipEvent_t e = t.pool.back();
    t.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Run `launch` (returning hipError_t), bracketed by events when timing is on.
template <typename F>
hipError_t timed(int cls, hipStream_t st, F&& launch) {
  Timing& t = timing();
  hipEvent_t a = nullptr, b = nullptr;
  {
    std::lock_guard<std::mutex> lock(t.mu);
    if (t.on) {
      a = take_event(t);
      b = take_event(t);
    }
  }
  if (a && b) {
    if (hipEventRecord(a, st) != hipSuccess) return hipErrorUnknown;
  }
  hipError_t e = launch();
  if (a && b) {
    if (hipEventRecord(b, st) != hipSuccess) return hipErrorUnknown;
    std::lock_guard<std::mutex> lock(t.mu);
    t.pending[cls].emplace_back(a, b);
  }
  return e;
}

char* at(void* ws, size_t off) { return static_cast<char*>(ws) + off; }

// bytes of e4m3 q (or k) of Bb batch rows; the scale bytes follow them inside
// the bf16 q (k) region, which is twice as large
size_t qk8_bytes(const Dims& d, int Bb) { return al((size_t)Bb * d.heads * d.Lp * d.hd); }

// Self-attention output handling of one block run (diffusion cache)
enum AttnMode { ATTN_COMPUTE = 0, ATTN_STORE = 1, ATTN_REUSE = 2 };

template <typename T>
int run_block(const Dims& d, int Bb, const wan_block_weights* w, float* x, const float* mod, long long mbs,
              const void* ctx, void* ws, const BlockPlan& p, bool rope_ready, hipStream_t st,
              int attn_mode = ATTN_COMPUTE, void* attn_io = nullptr, int lm = 0) {
  const int M = Bb * d.L;
  // tokens per modulation vector: a batch item's tokens, or (streaming queue) one slot's tokens
  if (lm <= 0) lm = d.L;
  T* m = reinterpret_cast<T*>(at(ws, p.m));
  T* o = reinterpret_cast<T*>(at(ws, p.o));
  float2* rope = reinterpret_cast<float2*>(at(ws, p.rope));
  float2* ropet = reinterpret_cast<float2*>(at(ws, p.ropet));
  const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)d.hd));
  const int P = pad256(d.L);  // padded row pitch of the token-row packing GEMMs

  if (!rope_ready) {
    HIP_TRY(launch_rope_table(rope, d.hd, d.F, d.Hh, d.Ww, st));
    HIP_TRY(launch_rope_tokens(ropet, rope, d.hd, d.F, d.Hh, d.Ww, st));
  }

  // WAN_FP8: the 8-bit projections take e4m3 operands with scales per 128-block;
  // the weights are quantised here, the activations by the kernels producing them
  unsigned char* m8 = reinterpret_cast<unsigned char*>(at(ws, p.m8));
  unsigned char* msc = reinterpret_cast<unsigned char*>(at(ws, p.msc));
  const long long rows_p = (long long)Bb * P;
  const W8Plan w8p = plan_w8(d);
  unsigned char* w8 = reinterpret_cast<unsigned char*>(at(ws, p.w8));
  unsigned char* wsc = reinterpret_cast<unsigned char*>(at(ws, p.wsc));
  if (d.fp8) {
    if (attn_mode != ATTN_REUSE)
      HIP_TRY(timed(WAN_KERNEL_ELEMENTWISE, st, [&] { return launch_quant_weights(w->qkv_w, w8 + w8p.qkv, wsc + w8p.sqkv, 3 * d.D, d.D, st); }));
    HIP_TRY(timed(WAN_KERNEL_ELEMENTWISE, st, [&] { return launch_quant_weights(w->cq_w, w8 + w8p.cq, wsc + w8p.scq, d.D, d.D, st); }));
    HIP_TRY(timed(WAN_KERNEL_ELEMENTWISE, st, [&] { return launch_quant_weights(w->ff1_w, w8 + w8p.ff1, wsc + w8p.sff1, d.Ff, d.D, st); }));
    HIP_TRY(timed(WAN_KERNEL_ELEMENTWISE, st, [&] { return launch_quant_weights(w->ff2_w, w8 + w8p.ff2, wsc + w8p.sff2, d.D, d.Ff, st); }));
  }
  // LayerNorm (+ modulation) of x into m, or into m8 / msc for an 8-bit projection
  auto ln = [&](const float* shift, const float* scale) {
    if (d.fp8)
      return timed(WAN_KERNEL_ELEMENTWISE, st, [&] {
        return launch_ln_mod8(x, m8, msc, rows_p, P, M, d.D, d.L, shift, scale, shift ? mbs : 0, st);
      });
    return timed(WAN_KERNEL_ELEMENTWISE, st, [&] { return launch_ln_mod<T>(x, m, M, d.D, lm, shift, scale, shift ? mbs : 0, st); });
  };
  // A operand of a projection whose input is the LayerNorm output
  auto ln_operand = [&](GemmArgs& g, size_t w8_off, size_t ws_off) {
    if (d.fp8) {
      g.A = m8; g.a_scale = msc; g.a_sld = rows_p;
      g.Wt = w8 + w8_off; g.w_scale = wsc + ws_off;
    }
  };
  const int ld_loader = d.fp8 ? LOAD_FP8 : LOAD_PLAIN;

  // self-attention sublayer (its attention output optionally written to, or
  // taken from, the diffusion cache)
  T* a_out = attn_mode == ATTN_COMPUTE ? o : reinterpret_cast<T*>(attn_io);
  // self-attention at full length (bf16, or 8-bit scores): the static-offset path (the QKV
  // epilogue gathers max |k|^2 per batch row and head; flagged workgroups are recomputed)
  const bool static_off = attn_static_offset_path(d.hd, d.L, d.heads, Bb, sizeof(T) == 2, d.qk8);
  float* kpart = reinterpret_cast<float*>(at(ws, p.kmax));
  const int kpart_n = P / 256 * 8;  // 256-row tiles per batch item x the QKV GEMM's 8 waves
  int* aflag = reinterpret_cast<int*>(at(ws, p.aflag));
  if (attn_mode != ATTN_REUSE) {
  HIP_TRY(ln(mod + 0 * d.D, mod + 1 * d.D));
  HIP_TRY(launch_zero_vt_pad<T>(at(ws, p.vt), Bb * d.heads, d.hd, d.L, d.Lp, st));
  {
    GemmArgs g;
    g.M = Bb * P; g.N = 3 * d.D; g.K = d.D;
    g.A = m; g.lda = d.D; g.a_rpb = P; g.a_bstride = (long long)d.L * d.D; g.a_valid = d.L;
    g.Wt = w->qkv_w; g.ldw = d.D; g.bias = w->qkv_b;
    g.c_rpb = P; g.c_valid = d.L;
    g.q = at(ws, p.q); g.k = at(ws, p.k); g.vt = at(ws, p.vt);
    g.nq = d.D; g.nk = d.D; g.heads = d.heads; g.hd = d.hd; g.Lp = d.Lp;
    g.rope = ropet;
    if (static_off) {
      g.kpart = kpart;
      g.kpart_n = kpart_n;
      // bf16 q leaves the epilogue in base-2 score units; 8-bit q keeps its projected values
      // (its e4m3 rounding is taken on q as projected), the attention scales its scores
      if (!d.qk8) g.q_scale = scale_log2;
    }
    if (d.qk8) {
      // e4m3 q / k take the first half of their bf16 regions, the scale bytes follow
      g.qs = reinterpret_cast<unsigned char*>(at(ws, p.q + qk8_bytes(d, Bb)));
      g.ks = reinterpret_cast<unsigned char*>(at(ws, p.k + qk8_bytes(d, Bb)));
    }
    ln_operand(g, w8p.qkv, w8p.sqkv);
    HIP_TRY(timed(WAN_KERNEL_GEMM, st, [&] { return launch_gemm<T>(g, ld_loader, d.qk8 ? EPI_PACK8 : EPI_PACK, st); }));
  }
  {
    AttnArgs a;
    a.q = at(ws, p.q); a.Lq = d.L; a.Lqp = d.Lp;
    a.k[0] = at(ws, p.k); a.vt[0] = at(ws, p.vt); a.Lk[0] = d.L; a.Lkp[0] = d.Lp; a.nsrc = 1; a.self = 1;
    a.o = a_out; a.B = Bb; a.heads = d.heads; a.hd = d.hd; a.scale_log2 = scale_log2;
    if (static_off) {
      a.kpart = kpart;
      a.kpart_n = kpart_n;
      a.fallback = aflag;
      if (!d.qk8) a.scale_log2 = 1.0f;  // q carries log2(e)/sqrt(hd) already
    }
    if (d.qk8) {
      a.qk8 = 1;
      a.qs = reinterpret_cast<const unsigned char*>(at(ws, p.q + qk8_bytes(d, Bb)));
      a.ks = reinterpret_cast<const unsigned char*>(at(ws, p.k + qk8_bytes(d, Bb)));
    }
    HIP_TRY(timed(WAN_KERNEL_SELF_ATTENTION, st, [&] { return launch_attention<T>(a, st); }));
  }
  }
  {
    GemmArgs g;
    g.M = M; g.N = d.D; g.K = d.D;
    g.A = a_out; g.lda = d.D; g.a_rpb = M;
    g.Wt = w->o_w; g.ldw = d.D; g.bias = w->o_b;
    g.c_rpb = lm; g.x = x; g.ldx = d.D; g.gate = mod + 2 * d.D; g.gate_bstride = mbs;
    HIP_TRY(timed(WAN_KERNEL_GEMM, st, [&] { return launch_gemm<T>(g, LOAD_PLAIN, EPI_RESID, st); }));
  }

  // cross-attention sublayer (ungated)
  HIP_TRY(ln(nullptr, nullptr));
  {
    GemmArgs g;
    g.M = Bb * P; g.N = d.D; g.K = d.D;
    g.A = m; g.lda = d.D; g.a_rpb = P; g.a_bstride = (long long)d.L * d.D; g.a_valid = d.L;
    g.Wt = w->cq_w; g.ldw = d.D; g.bias = w->cq_b;
    g.c_rpb = P; g.c_valid = d.L; g.q = at(ws, p.q); g.nq = d.D; g.nk = 0;
    g.heads = d.heads; g.hd = d.hd; g.Lp = d.Lp;
    ln_operand(g, w8p.cq, w8p.scq);
    HIP_TRY(timed(WAN_KERNEL_GEMM, st, [&] { return launch_gemm<T>(g, ld_loader, EPI_PACK, st); }));
  }
  {
    GemmArgs g;
    const int Pt = pad256(d.Lt);
    g.M = Bb * Pt; g.N = 2 * d.D; g.K = d.D;
    g.A = static_cast<const char*>(ctx) + (size_t)d.Li * d.D * d.es;
    g.lda = d.D; g.a_rpb = Pt; g.a_bstride = (long long)d.Lc * d.D; g.a_valid = d.Lt;
    g.Wt = w->ckv_w; g.ldw = d.D; g.bias = w->ckv_b;
    g.c_rpb = Pt; g.c_valid = d.Lt; g.k = at(ws, p.ck); g.vt = at(ws, p.cvt); g.nq = 0; g.nk = d.D;
    g.heads = d.heads; g.hd = d.hd; g.Lp = d.Ltp;
    HIP_TRY(launch_zero_vt_pad<T>(at(ws, p.cvt), Bb * d.heads, d.hd, d.Lt, d.Ltp, st));
    HIP_TRY(timed(WAN_KERNEL_GEMM, st, [&] { return launch_gemm<T>(g, LOAD_PLAIN, EPI_PACK, st); }));
  }
  if (d.Li > 0) {
    GemmArgs g;
    const int Pi = pad256(d.Li);
    g.M = Bb * Pi; g.N = 2 * d.D; g.K = d.D;
    g.A = ctx; g.lda = d.D; g.a_rpb = Pi; g.a_bstride = (long long)d.Lc * d.D; g.a_valid = d.Li;
    g.Wt = w->ikv_w; g.ldw = d.D; g.bias = w->ikv_b;
    g.c_rpb = Pi; g.c_valid = d.Li; g.k = at(ws, p.ik); g.vt = at(ws, p.ivt); g.nq = 0; g.nk = d.D;
    g.heads = d.heads; g.hd = d.hd; g.Lp = d.Lip;
    HIP_TRY(launch_zero_vt_pad<T>(at(ws, p.ivt), Bb * d.heads, d.hd, d.Li, d.Lip, st));
    HIP_TRY(timed(WAN_KERNEL_GEMM, st, [&] { return launch_gemm<T>(g, LOAD_PLAIN, EPI_PACK, st); }));
  }
  {
    AttnArgs a;
    a.q = at(ws, p.q); a.Lq = d.L; a.Lqp = d.Lp;
    a.k[0] = at(ws, p.ck); a.vt[0] = at(ws, p.cvt); a.Lk[0] = d.Lt; a.Lkp[0] = d.Ltp;
    a.nsrc = 1;
    if (d.Li > 0) {
      a.k[1] = at(ws, p.ik); a.vt[1] = at(ws, p.ivt); a.Lk[1] = d.Li; a.Lkp[1] = d.Lip; a.nsrc = 2;
    }
    a.o = o; a.B = Bb; a.heads = d.heads; a.hd = d.hd; a.scale_log2 = scale_log2;
    HIP_TRY(timed(WAN_KERNEL_CROSS_ATTENTION, st, [&] { return launch_attention<T>(a, st); }));
  }
  {
    GemmArgs g;
    g.M = M; g.N = d.D; g.K = d.D;
    g.A = o; g.lda = d.D; g.a_rpb = M;
    g.Wt = w->co_w; g.ldw = d.D; g.bias = w->co_b;
    g.c_rpb = d.L; g.x = x; g.ldx = d.D; g.gate = nullptr;
    HIP_TRY(timed(WAN_KERNEL_GEMM, st, [&] { return launch_gemm<T>(g, LOAD_PLAIN, EPI_RESID, st); }));
  }

  // FFN sublayer
  HIP_TRY(ln(mod + 3 * d.D, mod + 4 * d.D));
  if (d.fp8) {
    // FFN1 + GELU writes e4m3 rows (padded pitch) with scales per 128 columns; FFN2 reads them
    unsigned char* h8 = reinterpret_cast<unsigned char*>(at(ws, p.h8));
    unsigned char* hsc = reinterpret_cast<unsigned char*>(at(ws, p.hsc));
    {
      GemmArgs g;
      g.M = (int)rows_p; g.N = d.Ff; g.K = d.D;
      g.lda = d.D; g.a_rpb = P; g.a_bstride = (long long)d.L * d.D; g.a_valid = d.L;
      g.ldw = d.D; g.bias = w->ff1_b;
      ln_operand(g, w8p.ff1, w8p.sff1);
      g.c_rpb = P; g.C = h8; g.ldc = d.Ff; g.c_scale = hsc; g.c_sld = rows_p;
      HIP_TRY(timed(WAN_KERNEL_GEMM, st, [&] { return launch_gemm<T>(g, LOAD_FP8, EPI_STORE_GELU8, st); }));
    }
    {
      GemmArgs g;
      g.M = (int)rows_p; g.N = d.D; g.K = d.Ff;
      g.A = h8; g.lda = d.Ff; g.a_rpb = (int)rows_p; g.a_scale = hsc; g.a_sld = rows_p;
      g.Wt = w8 + w8p.ff2; g.w_scale = wsc + w8p.sff2; g.ldw = d.Ff; g.bias = w->ff2_b;
      g.c_rpb = P; g.c_valid = d.L; g.x = x; g.ldx = d.D; g.gate = mod + 5 * d.D; g.gate_bstride = mbs;
      HIP_TRY(timed(WAN_KERNEL_GEMM, st, [&] { return launch_gemm<T>(g, LOAD_FP8, EPI_RESID, st); }));
    }
    return WAN_OK;
  }
  T* hbuf = reinterpret_cast<T*>(at(ws, p.r1));
  {
    GemmArgs g;
    g.M = M; g.N = d.Ff; g.K = d.D;
    g.A = m; g.lda = d.D; g.a_rpb = M;
    g.Wt = w->ff1_w; g.ldw = d.D; g.bias = w->ff1_b;
    g.c_rpb = d.L; g.C = hbuf; g.ldc = d.Ff;
    HIP_TRY(timed(WAN_KERNEL_GEMM, st, [&] { return launch_gemm<T>(g, LOAD_PLAIN, EPI_STORE_GELU, st); }));
  }
  {
    GemmArgs g;
    g.M = M; g.N = d.D; g.K = d.Ff;
    g.A = hbuf; g.lda = d.Ff; g.a_rpb = M;
    g.Wt = w->ff2_w; g.ldw = d.Ff; g.bias = w->ff2_b;
    g.c_rpb = lm; g.x = x; g.ldx = d.D; g.gate = mod + 5 * d.D; g.gate_bstride = mbs;
    HIP_TRY(timed(WAN_KERNEL_GEMM, st, [&] { return launch_gemm<T>(g, LOAD_PLAIN, EPI_RESID, st); }));
  }
  return WAN_OK;
}

template <typename T>
int run_patchify(const Dims& d, int Bout, const float* z, const float* cond, const void* pe_w, const float* pe_b,
                 float* x, hipStream_t st) {
  GemmArgs g;
  g.M = Bout * d.L; g.N = d.D; g.K = d.Cin * 4;
  g.z = z; g.cond = cond; g.z_batch = d.B; g.in_ch = d.Cin; g.F = d.F; g.H = d.H; g.W = d.W;
  g.Wt = pe_w; g.ldw = d.Cin * 4; g.bias = pe_b;
  g.c_rpb = d.L; g.C = x; g.ldc = d.D;
  HIP_TRY(timed(WAN_KERNEL_GEMM, st, [&] { return launch_gemm<T>(g, LOAD_PATCH, EPI_STORE_F32, st); }));
  return WAN_OK;
}

template <typename T>
int run_time(const Dims& d, const wan_model_weights* w, float tau, float* mod, float* t1, float* t2, hipStream_t st) {
  HIP_TRY(launch_gemv<T>(w->t1_w, w->t1_b, nullptr, tau, t1, d.D, TIME_DIM, 0, st));
  HIP_TRY(launch_gemv<T>(w->t2_w, w->t2_b, t1, 0.f, t2, d.D, d.D, 1, st));
  HIP_TRY(launch_gemv<T>(w->m_w, w->m_b, t2, 0.f, mod, 6 * d.D, d.D, 1, st));
  return WAN_OK;
}

template <typename T>
int run_head(const Dims& d, int Bb, const wan_model_weights* w, const float* x, void* mbuf, float* p, hipStream_t st) {
  HIP_TRY(timed(WAN_KERNEL_ELEMENTWISE, st, [&] { return launch_ln_mod<T>(x, mbuf, Bb * d.L, d.D, d.L, nullptr, nullptr, 0, st); }));
  GemmArgs g;
  g.M = Bb * d.L; g.N = 64; g.K = d.D;
  g.A = mbuf; g.lda = d.D; g.a_rpb = g.M;
  g.Wt = w->hd_w; g.ldw = d.D; g.bias = w->hd_b;
  g.c_rpb = d.L; g.C = p; g.ldc = 64;
  HIP_TRY(timed(WAN_KERNEL_GEMM, st, [&] { return launch_gemm<T>(g, LOAD_PLAIN, EPI_STORE_F32, st); }));
  return WAN_OK;
}


// ======================================================================= streaming queue
struct StreamPlan {
  size_t x, mod, t1, t2, p, nz;
  BlockPlan blk;
  size_t total;
};

StreamPlan plan_stream(const Dims& d, int K) {
  StreamPlan p;
  size_t off = 0;
  p.x = off;
  off += al((size_t)d.L * d.D * 4);
  p.mod = off;
  off += al((size_t)K * 6 * d.D * 4);
  p.t1 = off;
  off += al((size_t)d.D * 4);
  p.t2 = off;
  off += al((size_t)d.D * 4);
  p.p = off;
  off += al((size_t)d.L * 64 * 4);
  p.nz = off;
  off += al((size_t)16 * d.F * d.H * d.W * 4);
  p.blk = plan_block(d, 1, off);
  p.total = p.blk.total;
  return p;
}

template <typename T>
int run_stream(const Dims& d, const wan_model_weights* w, float* window, const void* ctx, const float* taus,
               const float* dts, int K, int group, const float* noise, float* out, void* ws, const StreamPlan& p,
               hipStream_t st) {
  float* x = reinterpret_cast<float*>(at(ws, p.x));
  float* mod = reinterpret_cast<float*>(at(ws, p.mod));
  float* pbuf = reinterpret_cast<float*>(at(ws, p.p));
  int rc;
  for (int k = 0; k < K; ++k)
    if ((rc = run_time<T>(d, w, taus[k], mod + (size_t)k * 6 * d.D, reinterpret_cast<float*>(at(ws, p.t1)),
                          reinterpret_cast<float*>(at(ws, p.t2)), st)))
      return rc;
  if ((rc = run_patchify<T>(d, 1, window, nullptr, w->pe_w, w->pe_b, x, st))) return rc;
  const int lm = group * d.Hh * d.Ww;  // tokens of one slot
  for (int i = 0; i < w->n_blocks; ++i)
    if ((rc = run_block<T>(d, 1, &w->blocks[i], x, mod, 6LL * d.D, ctx, ws, p.blk, i > 0, st, ATTN_COMPUTE, nullptr,
                           lm)))
      return rc;
  if ((rc = run_head<T>(d, 1, w, x, at(ws, p.blk.m), pbuf, st))) return rc;
  float* nz = reinterpret_cast<float*>(at(ws, p.nz));
  HIP_TRY(timed(WAN_KERNEL_ELEMENTWISE, st, [&] {
    return launch_stream_update(pbuf, window, noise, nz, out, 16, d.F, d.H, d.W, group, dts, K, st);
  }));
  HIP_TRY(copy_async(window, nz, (size_t)16 * d.F * d.H * d.W * 4, st));
  return WAN_OK;
}

// ======================================================================= Wan-VAE decoder
// Layer list, parameter table, workspace plan and the launch sequence.

struct VaeDims {
  int T, H, W, zc, b, n_res, chunk;
  int d[5];  // stage widths 4b, 4b, 4b, 2b, b
};

int vae_check(const wan_vae_shape* s, VaeDims* d) {
  if (!s) return WAN_E_NULL;
  if (s->frames < 1 || s->height < 1 || s->width < 1 || s->z_ch < 1 || s->z_ch > 32) return WAN_E_SHAPE;
  if (s->base < 32 || s->base > 128 || s->base % 32 != 0 || s->n_res < 1 || s->n_res > 4) return WAN_E_SHAPE;
  if (s->chunk < 1 || s->chunk > s->frames) return WAN_E_SHAPE;
  if (256LL * s->chunk * s->height * s->width >= (1LL << 31)) return WAN_E_SHAPE;
  if (d) {
    d->T = s->frames;
    d->H = s->height;
    d->W = s->width;
    d->zc = s->z_ch;
    d->b = s->base;
    d->n_res = s->n_res;
    d->chunk = s->chunk;
    const int b = s->base;
    const int w[5] = {4 * b, 4 * b, 4 * b, 2 * b, b};
    for (int i = 0; i < 5; ++i) d->d[i] = w[i];
  }
  return WAN_OK;
}

// channel stride of a buffer holding c channels, and the GEMM width of a convolution
// producing them: c itself when a tile width divides it (multiples of 64 or 96), else
// c rounded up to 64 (zero weights in the padding)
int vcs(int c) { return (c % 64 == 0 || c % 96 == 0) ? c : (c + 63) / 64 * 64; }

struct VaeConvInfo {
  int cout, kt, kh, kw, cin;
  int level, in_cs;
  size_t w_off, b_off;       // into the caller's blobs
  int n_pad, cin_k;          // GEMM N and per-tap K (padded)
  long long cache_off;       // into the feature cache, -1 without one
  long long pad_off;         // padded weights (bf16) + bias (float) in the workspace, -1 if not padded
};

struct VaeTable {
  std::vector<wan_vae_param> params;
  std::vector<VaeConvInfo> convs;  // execution order
  std::vector<size_t> norm_off;    // float-blob offsets of the RMSNorm scales, execution order
  size_t w_elems = 0, f_elems = 0, cache_bytes = 0, pad_bytes = 0;
};

VaeTable vae_table(const VaeDims& d) {
  VaeTable t;
  auto lvl_hw = [&](int l, int& hp, int& wp) {
    hp = (d.H << l) + 2;
    wp = (d.W << l) + 2;
  };
  auto add_param = [&](const char* name, int kind, std::initializer_list<int> dims, size_t count) {
    wan_vae_param p;
    memset(&p, 0, sizeof(p));
    strncpy(p.name, name, sizeof(p.name) - 1);
    p.kind = kind;
    int i = 0;
    for (int v : dims) p.dims[i++] = v;
    size_t& off = kind == 0 ? t.w_elems : t.f_elems;
    off = (off + 63) / 64 * 64;
    p.offset = off;
    p.count = count;
    off += count;
    t.params.push_back(p);
    return p.offset;
  };
  auto add_norm = [&](const std::string& name, int c) {
    t.norm_off.push_back(add_param(name.c_str(), 2, {c}, (size_t)c));
  };
  auto add_conv = [&](const std::string& name, int cout, int kt, int kh, int kw, int cin, int level, int in_cs) {
    VaeConvInfo c;
    c.cout = cout; c.kt = kt; c.kh = kh; c.kw = kw; c.cin = cin; c.level = level; c.in_cs = in_cs;
    c.w_off = add_param(name.c_str(), 0, {cout, kt, kh, kw, cin}, (size_t)cout * kt * kh * kw * cin);
    c.b_off = add_param((name + ".bias").c_str(), 1, {cout}, (size_t)cout);
    c.n_pad = vcs(cout);
    c.cin_k = (cin + 31) / 32 * 32;
    c.cache_off = -1;
    if (kt > 1) {
      int hp, wp;
      lvl_hw(level, hp, wp);
      c.cache_off = (long long)t.cache_bytes;
      t.cache_bytes += al((size_t)(kt - 1) * hp * wp * in_cs * 2);
    }
    c.pad_off = -1;
    if (c.n_pad != cout || c.cin_k != cin) {
      c.pad_off = (long long)t.pad_bytes;
      t.pad_bytes += al((size_t)c.n_pad * kt * kh * kw * c.cin_k * 2) + al((size_t)c.n_pad * 4);
    }
    t.convs.push_back(c);
  };
  auto add_res = [&](const std::string& pre, int cin, int cout, int level) {
    add_norm(pre + ".norm_a", cin);
    add_conv(pre + ".conv_a", cout, 3, 3, 3, cin, level, vcs(cin));
    add_norm(pre + ".norm_b", cout);
    add_conv(pre + ".conv_b", cout, 3, 3, 3, cout, level, vcs(cout));
    if (cin != cout) add_conv(pre + ".skip", cout, 1, 1, 1, cin, level, vcs(cin));
  };
  add_conv("conv_in", d.d[0], 3, 3, 3, d.zc, 0, 32);
  for (int i = 0; i < 2; ++i) add_res("mid." + std::to_string(i), d.d[0], d.d[0], 0);
  for (int s = 0; s < 4; ++s) {
    const int cin = d.d[s], cout = d.d[s + 1];
    for (int j = 0; j < d.n_res; ++j)
      add_res("up." + std::to_string(s) + ".res." + std::to_string(j), j == 0 ? cin : cout, cout, s);
    if (s < 2) add_conv("up." + std::to_string(s) + ".time_conv", 2 * cout, 3, 1, 1, cout, s, vcs(cout));
    if (s < 3) add_conv("up." + std::to_string(s) + ".space_conv", cout, 1, 3, 3, cout, s + 1, vcs(cout));
  }
  add_norm("head.norm", d.d[4]);
  add_conv("head.conv", 3, 3, 3, 3, d.d[4], 3, vcs(d.d[4]));
  return t;
}

// Frames held per level for a call of n latent frames: level 0 also holds the
// time-doubled frames of stage 0, level 1 those of stage 1.
void vae_frames(int n, bool first, int f[4]) {
  const int f1 = first ? 2 * n - 1 : 2 * n;
  const int f2 = first ? 4 * n - 3 : 4 * n;
  f[0] = n;
  f[1] = f1;
  f[2] = f2;
  f[3] = f2;
}

struct VaePlan {
  size_t buf[4][4];     // four buffers per level
  size_t buf_bytes[4];
  int cap[4], cs[4];    // frame capacity (with the two cache frames) and channel stride per level
  size_t pad;           // padded weights
  size_t total;
};

VaePlan vae_plan(const VaeDims& d, const VaeTable& t) {
  VaePlan p;
  const int capf[4] = {2 * d.chunk, 4 * d.chunk, 4 * d.chunk, 4 * d.chunk};
  const int cs[4] = {vcs(d.d[0]), vcs(d.d[1]), vcs(d.d[2]), vcs(d.d[3]) > vcs(d.d[4]) ? vcs(d.d[3]) : vcs(d.d[4])};
  size_t off = 0;
  for (int l = 0; l < 4; ++l) {
    p.cap[l] = capf[l] + 2;
    p.cs[l] = l == 0 && cs[0] < 32 ? 32 : cs[l];
    const size_t hp = (size_t)(d.H << l) + 2, wp = (size_t)(d.W << l) + 2;
    p.buf_bytes[l] = al((size_t)p.cap[l] * hp * wp * p.cs[l] * 2);
    for (int k = 0; k < 4; ++k) {
      p.buf[l][k] = off;
      off += p.buf_bytes[l];
    }
  }
  p.pad = off;
  off += t.pad_bytes;
  p.total = off;
  return p;
}

struct VaeAct {
  int l, k;    // level, buffer index
  int c, cs;   // channels, channel stride
  int nf;      // frames
};

int vae_run(const VaeDims& d, const VaeTable& tab, const VaePlan& pl, const void* wblob, const float* fblob,
            const float* z, int t0, int n, char* cache, float* video, char* ws, hipStream_t st) {
  const bool first = t0 == 0;
  const bf16* W = static_cast<const bf16*>(wblob);
  auto buf = [&](int l, int k) { return ws + pl.buf[l][k]; };
  auto hp = [&](int l) { return (d.H << l) + 2; };
  auto wp = [&](int l) { return (d.W << l) + 2; };
  auto frame_bytes = [&](int l, int cs) { return (size_t)hp(l) * wp(l) * cs * 2; };

  // padded weights
  for (const VaeConvInfo& c : tab.convs) {
    if (c.pad_off < 0) continue;
    const int taps = c.kt * c.kh * c.kw;
    char* wp_ = ws + pl.pad + c.pad_off;
    float* bp = reinterpret_cast<float*>(wp_ + al((size_t)c.n_pad * taps * c.cin_k * 2));
    HIP_TRY(launch_vae_pad_weight(W + c.w_off, fblob + c.b_off, wp_, bp, c.cout, c.n_pad, taps, c.cin, c.cin_k, st));
  }
  if (first) HIP_TRY(hipMemsetAsync(cache, 0, tab.cache_bytes, st));

  size_t conv_i = 0, norm_i = 0;
  // one convolution: in (level l, stride in.cs, in.nf frames); rows of frames [t_in0, t_in0 + rows_f)
  auto conv = [&](const VaeAct& in, int rows_f, int t_in0, void* out, int out_cs, int of0, int ofs, int split,
                  const void* res, int epi, long long plane) -> int {
    const VaeConvInfo& c = tab.convs[conv_i++];
    const int l = in.l;
    char* ib = buf(l, in.k);
    // the spatial taps read the one-voxel border of the input frames as zero padding: a
    // buffer holds other tensors (and strides) earlier in the call, so clear it here; the
    // two leading frames come from the cache, whose frames were saved with clear borders
    HIP_TRY(launch_vae_border(ib + 2 * frame_bytes(l, in.cs), in.nf, hp(l), wp(l), in.cs, st));
    if (c.cache_off >= 0) HIP_TRY(copy_async(ib, cache + c.cache_off, 2 * frame_bytes(l, in.cs), st));
    const int taps = c.kt * c.kh * c.kw;
    GemmArgs g;
    g.M = rows_f * (d.H << l) * (d.W << l);
    g.N = c.n_pad;
    g.K = taps * c.cin_k;
    g.A = ib;
    g.lda = in.cs;
    if (c.pad_off >= 0) {
      char* wp_ = ws + pl.pad + c.pad_off;
      g.Wt = wp_;
      g.bias = reinterpret_cast<const float*>(wp_ + al((size_t)c.n_pad * taps * c.cin_k * 2));
    } else {
      g.Wt = W + c.w_off;
      g.bias = fblob + c.b_off;
    }
    g.ldw = g.K;
    g.cv_h = d.H << l;
    g.cv_w = d.W << l;
    g.cv_hp = hp(l);
    g.cv_wp = wp(l);
    g.cv_t0 = t_in0;
    g.cv_kpt = c.cin_k / 32;
    for (int dt = 0; dt < c.kt; ++dt)
      for (int dh = 0; dh < c.kh; ++dh)
        for (int dw = 0; dw < c.kw; ++dw) {
          const int ft = dt + (3 - c.kt), fh = dh + (3 - c.kh) / 2, fw = dw + (3 - c.kw) / 2;
          g.tap_off[(dt * c.kh + dh) * c.kw + dw] = (((long long)ft * hp(l) + fh) * wp(l) + fw) * in.cs;
        }
    g.cv_of0 = of0;
    g.cv_ofs = ofs;
    if (split > 0) g.cv_split = split;
    g.cv_res = res;
    g.cv_nout = 3;
    g.C = out;
    g.ldc = epi == EPI_CONV_VIDEO ? plane : out_cs;
    HIP_TRY(timed(WAN_KERNEL_GEMM, st, [&] { return launch_gemm<bf16>(g, LOAD_CONV, epi, st); }));
    if (c.cache_off >= 0)
      HIP_TRY(copy_async(cache + c.cache_off, ib + (size_t)in.nf * frame_bytes(l, in.cs), 2 * frame_bytes(l, in.cs), st));
    return WAN_OK;
  };
  auto norm = [&](const VaeAct& in, int k_out) -> int {
    const float* gsc = fblob + tab.norm_off[norm_i++];
    const int l = in.l;
    HIP_TRY(timed(WAN_KERNEL_ELEMENTWISE, st, [&] {
      return launch_vae_rms_silu(buf(l, in.k), buf(l, k_out), gsc, in.c, in.cs, in.nf, d.H << l, d.W << l, st);
    }));
    return WAN_OK;
  };
  auto free_buf = [&](int a, int b = -1, int c = -1) {
    for (int k = 0; k < 4; ++k)
      if (k != a && k != b && k != c) return k;
    return -1;
  };
  int rc;
  // residual block: x -> (in place, or into a new buffer when the width changes)
  auto res = [&](VaeAct& x, int cout) -> int {
    const int l = x.l;
    const int kn = free_buf(x.k), kh = free_buf(x.k, kn), ks = free_buf(x.k, kn, kh);
    if ((rc = norm(x, kn))) return rc;
    VaeAct nv{l, kn, x.c, x.cs, x.nf};
    if ((rc = conv(nv, x.nf, 0, buf(l, kh), vcs(cout), 0, 1, 0, nullptr, EPI_CONV, 0))) return rc;
    VaeAct hv{l, kh, cout, vcs(cout), x.nf};
    if ((rc = norm(hv, kn))) return rc;
    VaeAct n2{l, kn, cout, vcs(cout), x.nf};
    if (x.c == cout) {
      if ((rc = conv(n2, x.nf, 0, buf(l, x.k), x.cs, 0, 1, 0, buf(l, x.k), EPI_CONV, 0))) return rc;
    } else {
      // the block's second convolution comes before its shortcut in execution order
      const size_t conv_b = conv_i;
      conv_i = conv_b + 1;  // shortcut first, into ks
      if ((rc = conv(x, x.nf, 0, buf(l, ks), vcs(cout), 0, 1, 0, nullptr, EPI_CONV, 0))) return rc;
      const size_t after = conv_i;
      conv_i = conv_b;
      if ((rc = conv(n2, x.nf, 0, buf(l, ks), vcs(cout), 0, 1, 0, buf(l, ks), EPI_CONV, 0))) return rc;
      conv_i = after;
      x.k = ks;
      x.c = cout;
      x.cs = vcs(cout);
    }
    return WAN_OK;
  };

  int f[4];
  vae_frames(n, first, f);
  VaeAct x{0, 0, d.zc, 32, n};
  HIP_TRY(launch_vae_latent(z, buf(0, 0), d.zc, n, d.H, d.W, 32, st));
  {
    const int k = free_buf(0);
    if ((rc = conv(x, n, 0, buf(0, k), vcs(d.d[0]), 0, 1, 0, nullptr, EPI_CONV, 0))) return rc;
    x = VaeAct{0, k, d.d[0], vcs(d.d[0]), n};
  }
  for (int i = 0; i < 2; ++i)
    if ((rc = res(x, d.d[0]))) return rc;
  for (int s = 0; s < 4; ++s) {
    for (int j = 0; j < d.n_res; ++j)
      if ((rc = res(x, d.d[s + 1]))) return rc;
    if (s < 2) {
      // time doubling at this level's resolution: frames t >= (first ? 1 : 0) -> two frames each
      const int l = x.l, kt_ = free_buf(x.k);
      const int t0r = first ? 1 : 0;
      if ((rc = conv(x, x.nf - t0r, t0r, buf(l, kt_), x.cs, t0r, 2, x.c, nullptr, EPI_CONV, 0))) return rc;
      if (first) HIP_TRY(copy_async(buf(l, kt_) + 2 * frame_bytes(l, x.cs), buf(l, x.k) + 2 * frame_bytes(l, x.cs),
                                    frame_bytes(l, x.cs), st));
      x.k = kt_;
      x.nf = f[s + 1];
    }
    if (s < 3) {
      const int l = x.l, ku = 0, kv = 1;
      HIP_TRY(timed(WAN_KERNEL_ELEMENTWISE, st, [&] {
        return launch_vae_up_space(buf(l, x.k), buf(l + 1, ku), x.nf, d.H << l, d.W << l, x.cs, st);
      }));
      VaeAct u{l + 1, ku, x.c, x.cs, x.nf};
      if ((rc = conv(u, x.nf, 0, buf(l + 1, kv), x.cs, 0, 1, 0, nullptr, EPI_CONV, 0))) return rc;
      x = VaeAct{l + 1, kv, x.c, x.cs, x.nf};
    }
  }
  // head
  {
    const int kn = free_buf(x.k);
    if ((rc = norm(x, kn))) return rc;
    VaeAct nv{3, kn, x.c, x.cs, x.nf};
    const long long plane = (long long)x.nf * (d.H << 3) * (d.W << 3);
    if ((rc = conv(nv, x.nf, 0, video, 0, 0, 1, 0, nullptr, EPI_CONV_VIDEO, plane))) return rc;
  }
  return conv_i == tab.convs.size() && norm_i == tab.norm_off.size() ? WAN_OK : WAN_E_SHAPE;
}
}  // namespace
}  // namespace wan

using namespace wan;

// Diffusion cache layout: n_blocks self-attention outputs (2B, L, D), then the
// unconditional head output (B, L, out_ch*4) float32.
size_t cache_attn_slot(const Dims& d) { return al((size_t)2 * d.B * d.L * d.D * d.es); }
size_t cache_bytes(const Dims& d, int n_blocks) {
  return (size_t)n_blocks * cache_attn_slot(d) + al((size_t)d.B * d.L * 64 * 4);
}

// One CFG Euler step; mode 0 = plain, else a WAN_CACHE_* mode with `cache`.
template <typename T>
int run_step(const Dims& d, const wan_model_weights* w, float* z, const float* cnd, const void* ctx_cond,
             const void* ctx_null, float timestep, float dt, float guide_scale, int mode, char* cache,
             void* ws, const StepPlan& p, hipStream_t st) {
  const bool uncond_cached = (mode & WAN_CACHE_REUSE_UNCOND) != 0;
  const int nb = uncond_cached ? d.B : 2 * d.B;  // batch rows: cond videos, then null videos
  float* x = reinterpret_cast<float*>(at(ws, p.x));
  float* mod = reinterpret_cast<float*>(at(ws, p.mod));
  float* pbuf = reinterpret_cast<float*>(at(ws, p.p));
  void* ctx2 = at(ws, p.ctx);
  const size_t ctx_bytes = (size_t)d.B * d.Lc * d.D * d.es;
  HIP_TRY(copy_async(ctx2, ctx_cond, ctx_bytes, st));
  if (!uncond_cached) HIP_TRY(copy_async(static_cast<char*>(ctx2) + ctx_bytes, ctx_null, ctx_bytes, st));
  int rc;
  if ((rc = run_time<T>(d, w, timestep, mod, (float*)at(ws, p.t1), (float*)at(ws, p.t2), st))) return rc;
  if ((rc = run_patchify<T>(d, nb, z, cnd, w->pe_w, w->pe_b, x, st))) return rc;
  const int amode = mode == WAN_CACHE_STORE ? ATTN_STORE : ((mode & WAN_CACHE_REUSE_ATTN) ? ATTN_REUSE : ATTN_COMPUTE);
  for (int i = 0; i < w->n_blocks; ++i) {
    void* aio = cache ? cache + (size_t)i * cache_attn_slot(d) : nullptr;
    if ((rc = run_block<T>(d, nb, &w->blocks[i], x, mod, 0, ctx2, ws, p.blk, i > 0, st, amode, aio))) return rc;
  }
  if ((rc = run_head<T>(d, nb, w, x, at(ws, p.blk.m), pbuf, st))) return rc;
  const size_t pu_rows = (size_t)d.B * d.L * 64;
  float* cache_pu = cache ? reinterpret_cast<float*>(cache + (size_t)w->n_blocks * cache_attn_slot(d)) : nullptr;
  if (mode == WAN_CACHE_STORE) HIP_TRY(copy_async(cache_pu, pbuf + pu_rows, pu_rows * sizeof(float), st));
  HIP_TRY(timed(WAN_KERNEL_ELEMENTWISE, st, [&] {
    return launch_unpatch(pbuf, z, d.B, 16, d.F, d.H, d.W, 1, dt, guide_scale, st, uncond_cached ? cache_pu : nullptr);
  }));
  return WAN_OK;
}

int step_entry(const wan_shape* s, const wan_model_weights* w, float* z, const float* cond, const void* ctx_cond,
               const void* ctx_null, float timestep, float dt, float guide_scale, int mode, void* cache,
               size_t cache_size, void* ws, size_t ws_bytes, void* stream) {
  Dims d;
  int rc = check_shape(s, &d);
  if (rc) return rc;
  if ((rc = check_model_weights(w, d, true))) return rc;
  if ((rc = check_ptrs({z, ctx_cond, ctx_null}))) return rc;
  if (d.Cin == 36 && (rc = check_ptrs({cond}))) return rc;
  if (!isfinite(timestep) || !isfinite(dt) || !isfinite(guide_scale)) return WAN_E_SHAPE;
  if (mode) {
    if ((rc = check_ptrs({cache}))) return rc;
    if (cache_size < cache_bytes(d, w->n_blocks)) return WAN_E_WORKSPACE;
  }
  const StepPlan p = plan_step(d);
  if ((rc = check_ws(ws, ws_bytes, p.total))) return rc;
  if ((rc = check_device())) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const float* cnd = d.Cin == 36 ? cond : nullptr;
  char* c = static_cast<char*>(cache);
  return d.mode == WAN_BF16
             ? run_step<bf16>(d, w, z, cnd, ctx_cond, ctx_null, timestep, dt, guide_scale, mode, c, ws, p, st)
             : run_step<float>(d, w, z, cnd, ctx_cond, ctx_null, timestep, dt, guide_scale, mode, c, ws, p, st);
}

// Workspace of wan_dit_block_forward_noalloc: a fixed array in device memory,
// one copy per GPU (allocated by the runtime when the library's code object is
// loaded on that GPU).  Host code never uses the name itself, which is a
// host-side stand-in: the device address comes from noalloc_scratch().
static __device__ __align__(256) unsigned char scratch[WAN_NOALLOC_SCRATCH_BYTES];

namespace wan {
namespace {
// Device address of `scratch` on the current device, looked up on the first
// call on each device (with that device current) and kept; NULL on failure.
void* noalloc_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  static std::mutex mu;
  static void* ptr[64] = {};
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    ptr[dev] = p;
  }
  return ptr[dev];
}
}  // namespace
}  // namespace wan

extern "C" {

const char* wan_status_str(int code) {
  switch (code) {
    case WAN_OK: return "ok";
    case WAN_E_NULL: return "a required pointer is NULL";
    case WAN_E_SHAPE: return "unsupported or inconsistent shape";
    case WAN_E_MODE: return "unknown precision mode";
    case WAN_E_ALIGN: return "a pointer is not 16-byte aligned";
    case WAN_E_WORKSPACE: return "workspace missing or too small";
    case WAN_E_HIP: return "no usable gfx950 device, or a HIP launch failed";
    case WAN_E_ENTRY: return "unknown entry id";
    case WAN_E_SCRATCH: return "the shape needs more scratch than the no-allocation entry point holds";
  }
  return "unknown status code";
}

size_t wan_workspace_bytes(const wan_shape* s, int entry, int* status) {
  Dims d;
  int rc = check_shape(s, &d);
  size_t n = 0;
  if (rc == WAN_OK) {
    switch (entry) {
      case WAN_ENTRY_PATCHIFY: n = 0; break;
      case WAN_ENTRY_BLOCK: n = plan_block(d, d.B, 0).total; break;
      case WAN_ENTRY_STEP: n = plan_step(d).total; break;
      case WAN_ENTRY_TIME_EMBED: n = time_bytes(d); break;
      case WAN_ENTRY_HEAD: n = head_bytes(d); break;
      default: rc = WAN_E_ENTRY;
    }
  }
  if (status) *status = rc;
  return rc == WAN_OK ? n : 0;
}

int wan_patchify(const wan_shape* s, const float* z, const float* cond, const void* pe_w, const float* pe_b,
                 float* x, void* ws, size_t ws_bytes, void* stream) {
  Dims d;
  int rc = check_shape(s, &d);
  if (rc) return rc;
  if ((rc = check_ptrs({z, pe_w, pe_b, x}))) return rc;
  if (d.Cin == 36 && (rc = check_ptrs({cond}))) return rc;
  (void)ws;
  (void)ws_bytes;
  if ((rc = check_device())) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return d.mode == WAN_BF16 ? run_patchify<bf16>(d, d.B, z, d.Cin == 36 ? cond : nullptr, pe_w, pe_b, x, st)
                            : run_patchify<float>(d, d.B, z, d.Cin == 36 ? cond : nullptr, pe_w, pe_b, x, st);
}

int wan_time_embed(const wan_shape* s, const wan_model_weights* w, float timestep, float* mod, void* ws,
                   size_t ws_bytes, void* stream) {
  Dims d;
  int rc = check_shape(s, &d);
  if (rc) return rc;
  if ((rc = check_model_weights(w, d, false))) return rc;
  if ((rc = check_ptrs({mod}))) return rc;
  if ((rc = check_ws(ws, ws_bytes, time_bytes(d)))) return rc;
  if (!isfinite(timestep)) return WAN_E_SHAPE;
  if ((rc = check_device())) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  float* t1 = reinterpret_cast<float*>(at(ws, 0));
  float* t2 = reinterpret_cast<float*>(at(ws, al((size_t)d.D * 4)));
  return d.mode == WAN_BF16 ? run_time<bf16>(d, w, timestep, mod, t1, t2, st)
                            : run_time<float>(d, w, timestep, mod, t1, t2, st);
}

int wan_dit_block_forward(const wan_shape* s, const wan_block_weights* w, float* x, const float* mod,
                          long long mod_batch_stride, const void* ctx, void* ws, size_t ws_bytes, void* stream) {
  Dims d;
  int rc = check_shape(s, &d);
  if (rc) return rc;
  if ((rc = check_block_weights(w, d))) return rc;
  if ((rc = check_ptrs({x, mod, ctx}))) return rc;
  if (mod_batch_stride != 0 && mod_batch_stride != 6LL * d.D) return WAN_E_SHAPE;
  const BlockPlan p = plan_block(d, d.B, 0);
  if ((rc = check_ws(ws, ws_bytes, p.total))) return rc;
  if ((rc = check_device())) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return d.mode == WAN_BF16 ? run_block<bf16>(d, d.B, w, x, mod, mod_batch_stride, ctx, ws, p, false, st)
                            : run_block<float>(d, d.B, w, x, mod, mod_batch_stride, ctx, ws, p, false, st);
}

int wan_dit_block_forward_noalloc(const wan_shape* s, const wan_block_weights* w, float* x, const float* mod,
                                  long long mod_batch_stride, const void* ctx, void* stream) {
  Dims d;
  int rc = check_shape(s, &d);
  if (rc) return rc;
  if ((rc = check_block_weights(w, d))) return rc;
  if ((rc = check_ptrs({x, mod, ctx}))) return rc;
  if (mod_batch_stride != 0 && mod_batch_stride != 6LL * d.D) return WAN_E_SHAPE;
  const BlockPlan p = plan_block(d, d.B, 0);
  if (p.total > WAN_NOALLOC_SCRATCH_BYTES) return WAN_E_SCRATCH;
  if ((rc = check_device())) return rc;
  void* ws = noalloc_scratch();
  if (!ws) return WAN_E_HIP;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // no result depends on what the array held before (the block overwrites every
  // workspace value it uses; padded key rows are masked by assignment), so the
  // array is not cleared
  return d.mode == WAN_BF16 ? run_block<bf16>(d, d.B, w, x, mod, mod_batch_stride, ctx, ws, p, false, st)
                            : run_block<float>(d, d.B, w, x, mod, mod_batch_stride, ctx, ws, p, false, st);
}

int wan_head(const wan_shape* s, const wan_model_weights* w, const float* x, float* v, void* ws, size_t ws_bytes,
             void* stream) {
  Dims d;
  int rc = check_shape(s, &d);
  if (rc) return rc;
  if ((rc = check_model_weights(w, d, false))) return rc;
  if ((rc = check_ptrs({x, v}))) return rc;
  if ((rc = check_ws(ws, ws_bytes, head_bytes(d)))) return rc;
  if ((rc = check_device())) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  void* mbuf = at(ws, 0);
  float* p = reinterpret_cast<float*>(at(ws, al((size_t)d.B * d.L * d.D * d.es)));
  rc = d.mode == WAN_BF16 ? run_head<bf16>(d, d.B, w, x, mbuf, p, st) : run_head<float>(d, d.B, w, x, mbuf, p, st);
  if (rc) return rc;
  HIP_TRY(launch_unpatch(p, v, d.B, 16, d.F, d.H, d.W, 0, 0.f, 0.f, st));
  return WAN_OK;
}

int wan_denoise_step(const wan_shape* s, const wan_model_weights* w, float* z, const float* cond,
                     const void* ctx_cond, const void* ctx_null, float timestep, float dt, float guide_scale,
                     void* ws, size_t ws_bytes, void* stream) {
  return step_entry(s, w, z, cond, ctx_cond, ctx_null, timestep, dt, guide_scale, 0, nullptr, 0, ws, ws_bytes,
                    stream);
}

size_t wan_cache_bytes(const wan_shape* s, int n_blocks, int* status) {
  Dims d;
  int rc = check_shape(s, &d);
  if (rc == WAN_OK && (n_blocks < 1 || n_blocks > MAX_BLOCKS)) rc = WAN_E_SHAPE;
  if (status) *status = rc;
  return rc == WAN_OK ? cache_bytes(d, n_blocks) : 0;
}

int wan_denoise_step_cached(const wan_shape* s, const wan_model_weights* w, float* z, const float* cond,
                            const void* ctx_cond, const void* ctx_null, float timestep, float dt, float guide_scale,
                            int cache_mode, void* cache, size_t cache_bytes_, void* ws, size_t ws_bytes,
                            void* stream) {
  if (cache_mode != WAN_CACHE_STORE && cache_mode != WAN_CACHE_REUSE_ATTN && cache_mode != WAN_CACHE_REUSE_UNCOND &&
      cache_mode != (WAN_CACHE_REUSE_ATTN | WAN_CACHE_REUSE_UNCOND))
    return WAN_E_MODE;
  if (!cache) return WAN_E_NULL;
  return step_entry(s, w, z, cond, ctx_cond, ctx_null, timestep, dt, guide_scale, cache_mode, cache, cache_bytes_,
                    ws, ws_bytes, stream);
}

size_t wan_stream_workspace_bytes(const wan_shape* s, int group, int* status) {
  Dims d;
  int rc = check_shape(s, &d);
  if (rc == WAN_OK && (d.B != 1 || d.Cin != 16 || d.Li != 0 || d.fp8 || group < 1 || d.F % group != 0 ||
                       d.F / group > STREAM_MAX_SLOTS))
    rc = WAN_E_SHAPE;
  if (status) *status = rc;
  return rc == WAN_OK ? plan_stream(d, d.F / group).total : 0;
}

int wan_stream_tick(const wan_shape* s, const wan_model_weights* w, float* window, const void* ctx, const float* taus,
                    const float* dts, int group, const float* noise_in, float* frames_out, void* ws, size_t ws_bytes,
                    void* stream) {
  Dims d;
  int rc = check_shape(s, &d);
  if (rc) return rc;
  if (d.fp8) return WAN_E_MODE;
  if (d.B != 1 || d.Cin != 16 || d.Li != 0 || group < 1 || d.F % group != 0 || d.F / group > STREAM_MAX_SLOTS)
    return WAN_E_SHAPE;
  const int K = d.F / group;
  if (!taus || !dts) return WAN_E_NULL;
  for (int k = 0; k < K; ++k)
    if (!isfinite(taus[k]) || !isfinite(dts[k])) return WAN_E_SHAPE;
  if ((rc = check_model_weights(w, d, true))) return rc;
  if ((rc = check_ptrs({window, ctx, noise_in, frames_out}))) return rc;
  const StreamPlan p = plan_stream(d, K);
  if ((rc = check_ws(ws, ws_bytes, p.total))) return rc;
  if ((rc = check_device())) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return d.mode == WAN_BF16 ? run_stream<bf16>(d, w, window, ctx, taus, dts, K, group, noise_in, frames_out, ws, p, st)
                            : run_stream<float>(d, w, window, ctx, taus, dts, K, group, noise_in, frames_out, ws, p, st);
}

int wan_vae_param_count(const wan_vae_shape* s, int* status) {
  VaeDims d;
  const int rc = vae_check(s, &d);
  if (status) *status = rc;
  return rc == WAN_OK ? (int)vae_table(d).params.size() : 0;
}

int wan_vae_param_info(const wan_vae_shape* s, int index, wan_vae_param* out) {
  VaeDims d;
  int rc = vae_check(s, &d);
  if (rc) return rc;
  if (!out) return WAN_E_NULL;
  const VaeTable t = vae_table(d);
  if (index < 0 || index >= (int)t.params.size()) return WAN_E_ENTRY;
  *out = t.params[index];
  return WAN_OK;
}

size_t wan_vae_blob_elems(const wan_vae_shape* s, int which, int* status) {
  VaeDims d;
  int rc = vae_check(s, &d);
  if (rc == WAN_OK && which != 0 && which != 1) rc = WAN_E_ENTRY;
  if (status) *status = rc;
  if (rc) return 0;
  const VaeTable t = vae_table(d);
  return which == 0 ? t.w_elems : t.f_elems;
}

size_t wan_vae_workspace_bytes(const wan_vae_shape* s, int* status) {
  VaeDims d;
  const int rc = vae_check(s, &d);
  if (status) *status = rc;
  if (rc) return 0;
  const VaeTable t = vae_table(d);
  return vae_plan(d, t).total;
}

size_t wan_vae_cache_bytes(const wan_vae_shape* s, int* status) {
  VaeDims d;
  const int rc = vae_check(s, &d);
  if (status) *status = rc;
  return rc == WAN_OK ? vae_table(d).cache_bytes : 0;
}

int wan_vae_decode(const wan_vae_shape* s, const void* weights, const float* fparams, const float* z, int t0, int n,
                   void* cache, size_t cache_bytes_, float* video, void* ws, size_t ws_bytes, void* stream) {
  VaeDims d;
  int rc = vae_check(s, &d);
  if (rc) return rc;
  if ((rc = check_ptrs({weights, fparams, z, cache, video}))) return rc;
  if (n < 1 || n > d.chunk || t0 < 0 || t0 + n > d.T) return WAN_E_SHAPE;
  const VaeTable t = vae_table(d);
  const VaePlan p = vae_plan(d, t);
  if (cache_bytes_ < t.cache_bytes) return WAN_E_WORKSPACE;
  if ((rc = check_ws(ws, ws_bytes, p.total))) return rc;
  if ((rc = check_device())) return rc;
  return vae_run(d, t, p, weights, fparams, z, t0, n, static_cast<char*>(cache), video, static_cast<char*>(ws),
                 static_cast<hipStream_t>(stream));
}

int wan_timing_enable(int on) {
  Timing& t = timing();
  std::lock_guard<std::mutex> lock(t.mu);
  t.on = on != 0;
  return WAN_OK;
}

int wan_timing_read(int kernel_class, double* ms_total, long long* launches, int reset) {
  if (kernel_class < 0 || kernel_class >= N_CLASSES) return WAN_E_ENTRY;
  if (!ms_total || !launches) return WAN_E_NULL;
  Timing& t = timing();
  std::lock_guard<std::mutex> lock(t.mu);
  for (auto& pr : t.pending[kernel_class]) {
    if (hipEventSynchronize(pr.second) != hipSuccess) return WAN_E_HIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, pr.first, pr.second) != hipSuccess) return WAN_E_HIP;
    t.ms[kernel_class] += ms;
    t.n[kernel_class] += 1;
    t.pool.push_back(pr.first);
    t.pool.push_back(pr.second);
  }
  t.pending[kernel_class].clear();
  *ms_total = t.ms[kernel_class];
  *launches = t.n[kernel_class];
  if (reset) {
    t.ms[kernel_class] = 0;
    t.n[kernel_class] = 0;
  }
  return WAN_OK;
}

}  // extern "C"
