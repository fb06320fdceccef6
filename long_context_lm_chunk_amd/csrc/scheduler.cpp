// Chunk scheduler and C ABI of the TTT-E2E inner loop.
//
// Per context (ttt_prefill):
//   phase A  for a block of whole chunks (prefill_block tokens): embed, then
//            every frozen block 0 .. L-q-1 and the attention half of block
//            L-q, batched over the whole block.  None of this depends on the
//            fast weights: only the MLPs of the last q blocks are updated
//            (podcast 6:36 and 7:08), and attention/embeddings stay static.
//   phase B  for each chunk of the block, sequentially (the next chunk needs
//            the weights updated by this one): forward of the top q blocks
//            with the current fast weights, fused head + next-token
//            cross-entropy (NVIDIA blog, "Our method": the loss at the end of
//            the network), backward into the fast MLPs only, fused SGD in the
//            weight-gradient epilogue (forum post TL;DR: mini-gradient
//            descent on the context during inference).
// Keys/values are written to per-layer rings when a position is read and
// are never recomputed, so attention memory stays bounded by the window.
//
// Everything stays resident in the caller's workspace; the host only
// enqueues kernels on one stream and reads back an error flag.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "kernels.hpp"
#include "../../include/ttt.h"

using namespace ttt;

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

#define HIPCHK(x)                                                                 \
  do {                                                                            \
    hipError_t e_ = (x);                                                          \
    if (e_ != hipSuccess) return fail(TTT_ERR_HIP, std::string(#x) + ": " + hipGetErrorString(e_)); \
  } while (0)

constexpr int NCLS = 8;
constexpr int kMaxSplit = 8;   // key-range splits of the per-chunk attention launches

struct Timing {
  bool on = false;
  std::vector<hipEvent_t> ev;   // pairs
  size_t used = 0;
  int64_t launches = 0;
  double flops = 0.0;
};

// Bump allocator over the workspace (base == nullptr computes the size).
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <typename P> P* take(size_t bytes) {
    off = (off + 255) & ~size_t(255);
    P* p = base ? reinterpret_cast<P*>(base + off) : nullptr;
    off += bytes;
    return p;
  }
};

// A fast MLP is held as W0 + delta: W0 is the loaded matrix (exact, in the
// storage type), delta the accumulated SGD updates.  delta's fp32 master takes
// the updates; its copy in the storage type (the master itself in fp32 mode)
// feeds the products, which run over W0 and delta in one fp32 accumulation.
// Updates of lr*g ~ 1e-8 are far below a bf16 ulp of W (~1e-4), so rounding
// W0 + delta to bf16 would erase them; delta's own ulp scales with delta.
//
// The input-gradient products of the backward pass only need the current
// weights to working precision, so they read one rounded copy
// round(W0 + delta), kept transposed (ct_up / ct_dn: the products then take
// both operands k-contiguous) and rewritten by the SGD epilogue.
struct FastLayer {
  float* m_up = nullptr;  // fp32 delta master [F2][d]
  float* m_dn = nullptr;  // fp32 delta master [d][F]
  void* s_up = nullptr;   // delta in the storage type (== master in fp32 mode)
  void* s_dn = nullptr;
  void* ct_up = nullptr;  // round(W0 + delta) in the storage type, transposed: [d][F2]
  void* ct_dn = nullptr;  // [F][d] (k-contiguous operands of the input-gradient products)
};

struct Layer {
  void* wqkv = nullptr;  // [3d][d]  out-major
  void* wo = nullptr;    // [d][d]
  void* wup = nullptr;   // [F2][d] (SwiGLU: gate/up interleaved in 16-row blocks)
  void* wdn = nullptr;   // [d][F]
  void* kring = nullptr; void* vring = nullptr;  // [cap][d]
  void* vtring = nullptr;                          // [d][cap]: V transposed, key-permuted (forward)
  void* ktring = nullptr;                          // [d][cap]: K transposed, key-permuted (fast blocks: dQ)
  void* wqkvT = nullptr;  // [d][3d] and [d][d]: transposed copies for the input-gradient
  void* woT = nullptr;    // products (fast blocks above the first)
  // frozen second MLP of a fast block (static_mlp): forward layout like
  // wup / wdn, and transposed copies for the input-gradient products
  void* swup = nullptr; void* swdn = nullptr;    // [F2][d], [d][F]
  void* swupT = nullptr; void* swdnT = nullptr;  // [d][F2], [F][d]
  int64_t cap = 0;
};

struct PB {  // phase-B buffers of one fast layer (chunk rows)
  float* xin = nullptr; float* x2 = nullptr;
  float* mean1 = nullptr; float* rstd1 = nullptr; float* mean2 = nullptr; float* rstd2 = nullptr;
  void* a = nullptr; void* q = nullptr; void* o = nullptr; float* lse = nullptr;
  void* b = nullptr; void* z = nullptr; void* act = nullptr;
  // frozen second MLP: its input (the residual after the fast MLP), LayerNorm
  // statistics and pre-activations (for the activation backward)
  float* xm = nullptr; float* mean3 = nullptr; float* rstd3 = nullptr; void* z2 = nullptr;
};

}  // namespace

struct ttt_model {
  ttt_config c{};
  bool bf = true;
  size_t es = 2;          // element size of weights/activations
  int d = 0, F = 0, F2 = 0, V = 0, L = 0, q = 0, f0 = 0, H = 0, hd = 0, W = 0, Cmax = 0, MA = 0;
  int nparts = 0;
  void* E = nullptr; void* U = nullptr;
  void* UT = nullptr;                   // head transposed [d][V] (input gradient of the head)
  std::vector<Layer> layers;
  std::vector<FastLayer> fast;
  double* theta = nullptr;
  float2* csA = nullptr; float2* csB = nullptr;   // rotary cos/sin of a phase-A block / a chunk
  // phase A
  // phase A runs on its own stream, one block ahead of phase B; its output
  // block is double-buffered (hAb[block % 2]); hA = hAb[0] also serves as the
  // phase-B input of a decode chunk
  float* hAb[2] = {nullptr, nullptr};
  float* hA = nullptr; void* aA = nullptr; void* qkvA = nullptr; void* qA = nullptr; void* oA = nullptr;
  hipStream_t sa = nullptr;
  hipEvent_t ev0 = nullptr, evA[2] = {nullptr, nullptr}, evB[2] = {nullptr, nullptr};
  void* actA = nullptr;
  // phase B
  std::vector<PB> pb;
  float* xL = nullptr; float* meanf = nullptr; float* rstdf = nullptr; void* fN = nullptr;
  void* qkvB = nullptr;
  float* pmax = nullptr; float* psum = nullptr; float* tlog = nullptr; float* lse_ce = nullptr;
  float* zce = nullptr;                 // the chunk's logits [C][V] fp32 (head statistics pass)
  void* cS = nullptr; void* actS = nullptr; void* dzS = nullptr;   // second-MLP temporaries [C][..]
  void* G = nullptr;
  float* dh = nullptr; void* dh_lo = nullptr; void* dz = nullptr;
  // transposed operands of the weight-gradient products, one set per fast
  // block (the updates run on their own stream, concurrently with the rest
  // of the backward pass): [features][Cp]
  struct TOps { void* dhT = nullptr; void* actT = nullptr; void* dzT = nullptr; void* bT = nullptr; };
  std::vector<TOps> tops;
  int64_t Cp = 0;                       // their row stride
  hipStream_t sc = nullptr;             // fast-weight updates (SGD products)
  std::vector<hipEvent_t> evT1, evT2;   // per fast block: update operands ready
  std::vector<hipEvent_t> evR1, evR2;   // per fast block: dh_lo / dz read by the update stream
  hipEvent_t evC = nullptr;             // all updates of the chunk done
  // Within a prefill the chain does not wait for the chunk's updates at its
  // end: the next chunk's forward waits for the first fast block's up
  // update (evR1[0]) before that block's up product (for the transposes of
  // its operands (evR2[0]) before the LayerNorm feeding it) and for its down
  // update (evC) before the down product.  sgd_defer asks chunk_step for that; sgd_open
  // says such waits are owed.
  bool sgd_defer = false, sgd_open = false;
  hipStream_t sk = nullptr;             // dK/dV of the attention backward, beside dQ
  hipStream_t sb = nullptr;             // the chunk chain when several contexts run at once
  hipEvent_t evOut = nullptr;           // end of this context's work in such a run
  hipEvent_t evK0 = nullptr, evK1 = nullptr;
  float* dtmp = nullptr; void* dout = nullptr; void* dqkv = nullptr; float* Dattn = nullptr;
  float* attn_part = nullptr; float* attn_ml = nullptr;   // key-range split partials
  // Q and dO of the chunk transposed for dK/dV: [d][Cq], Cq = the chunk
  // capacity rounded up to a multiple of 64, columns permuted in groups of 16
  void* qT = nullptr; void* gT = nullptr; int64_t Cq = 0;
  float* split_ws = nullptr; int64_t split_cap = 0;         // split-K partials of the GEMMs
  // decode
  float* xd = nullptr; void* qd = nullptr; void* od = nullptr;
  void* actd = nullptr; float* logits = nullptr; float* attn_ws = nullptr;
  int32_t* hist = nullptr; int32_t* cur_tok = nullptr;
  int64_t* dstate = nullptr;            // decode state on the device: {pos, ci}
  float* amax = nullptr;                // per-block (max, index) pairs of the head product
  hipGraphExec_t dec_exec = nullptr;    // one decode token, captured once
  int* err = nullptr;
  float* nanv = nullptr;
  // state
  int64_t pos = 0;        // next position to read
  int64_t dchunk0 = 0;    // first position of the current decode chunk
  int64_t logit_rows = 0; // rows of the chunk logits kept in zce (the last chunk read by chunk_step)
  bool prefilled = false;
  bool no_update = false; // read by ttt_forward: decode makes no updates
  float lr = 0.f; int steps = 1; int chunk = 1;
  Timing tm[NCLS];
  int static_dev = -1;    // device whose static workspace holds this model (ttt_model_load_static)
};

namespace {

size_t esz(const ttt_config& c) { return c.dtype == TTT_BF16 ? 2 : 4; }

int check_config(const ttt_config* c) {
  if (!c) return fail(TTT_ERR_ARG, "config is NULL");
  if (c->dtype != TTT_BF16 && c->dtype != TTT_FP32) return fail(TTT_ERR_CONFIG, "dtype must be TTT_BF16 or TTT_FP32");
  if (c->mlp != TTT_MLP_GELU && c->mlp != TTT_MLP_SWIGLU) return fail(TTT_ERR_CONFIG, "mlp must be GELU or SwiGLU");
  const int hd = c->head_dim;
  if (!(hd == 16 || hd == 32 || hd == 64 || hd == 96 || hd == 128)) return fail(TTT_ERR_CONFIG, "head_dim must be 16, 32, 64, 96 or 128");
  if (c->n_heads <= 0 || c->n_heads * hd != c->d_model) return fail(TTT_ERR_CONFIG, "n_heads * head_dim must equal d_model");
  if (c->d_model % 16 || c->d_ff % 16 || c->d_ff <= 0) return fail(TTT_ERR_CONFIG, "d_model and d_ff must be positive multiples of 16");
  if (c->vocab <= 0 || c->vocab % 8) return fail(TTT_ERR_CONFIG, "vocab must be a positive multiple of 8");
  if (c->n_layers <= 0 || c->n_fast < 1 || c->n_fast > c->n_layers) return fail(TTT_ERR_CONFIG, "need 1 <= n_fast <= n_layers");
  if (c->window < 1 || c->window > (1 << 22)) return fail(TTT_ERR_CONFIG, "window must be in [1, 4194304]");
  {
    const int kmax = c->dtype == TTT_BF16 ? 16384 : 8192;   // decode input vector held in LDS
    if (c->d_model > kmax || c->d_ff > kmax)
      return fail(TTT_ERR_CONFIG, "d_model and d_ff must be <= 16384 (bf16) or 8192 (fp32)");
  }
  if (c->max_chunk < 1 || c->max_chunk > (1 << 16)) return fail(TTT_ERR_CONFIG, "max_chunk must be in [1, 65536]");
  if (c->prefill_block < 0) return fail(TTT_ERR_CONFIG, "prefill_block must be >= 0");
  if (c->static_mlp != 0 && c->static_mlp != 1) return fail(TTT_ERR_CONFIG, "static_mlp must be 0 or 1");
  if (!(c->ln_eps > 0.f) || !(c->rope_base > 1.f)) return fail(TTT_ERR_CONFIG, "ln_eps > 0 and rope_base > 1 required");
  {
    // Every operand of a matrix product is read through a buffer resource
    // (32-bit byte offsets): none may span more than 2^31 - 1 bytes.  Rows x
    // row length of each operand: phase-A blocks (MA rows), chunk rows (C),
    // the weights and the transposed activations of the weight gradients.
    const int64_t es = esz(*c), d = c->d_model, F = c->d_ff, V = c->vocab;
    const int64_t F2 = c->mlp == TTT_MLP_SWIGLU ? 2 * F : F;
    const int64_t C = c->max_chunk;
    const int64_t MA = std::max<int64_t>(c->prefill_block > 0 ? c->prefill_block : 8192, C);
    const int64_t Cp = (C + 7) / 8 * 8;
    const int64_t rows_x_len[] = {MA * d, MA * F, C * V, C * F2, C * 3 * d, V * d, F2 * d, 3 * d * d,
                                  F2 * Cp, F * Cp};
    for (const int64_t e : rows_x_len)
      if (e * es > GEMM_MAX_OPERAND_BYTES)
        return fail(TTT_ERR_CONFIG, "a matrix-product operand would span more than 2^31 - 1 bytes "
                                    "(bound vocab * max_chunk, prefill_block * d_ff, max_chunk * d_ff, "
                                    "vocab * d_model)");
  }
  return TTT_OK;
}

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Lay the model out in the workspace (m->... pointers); returns bytes used.
size_t layout(ttt_model* m, void* base) {
  Carver cv(base);
  const ttt_config& c = m->c;
  const size_t es = m->es;
  const int d = m->d, F = m->F, F2 = m->F2, V = m->V, C = m->Cmax, MA = m->MA, H = m->H;
  m->E = cv.take<void>((size_t)V * d * es);
  m->U = cv.take<void>((size_t)V * d * es);
  m->layers.assign(m->L, Layer());
  const int64_t capA = round_up((int64_t)m->W + MA, 64);
  const int64_t capB = round_up((int64_t)m->W + C, 64);
  for (int l = 0; l < m->L; ++l) {
    Layer& ly = m->layers[l];
    ly.wqkv = cv.take<void>((size_t)3 * d * d * es);
    ly.wo = cv.take<void>((size_t)d * d * es);
    ly.wup = cv.take<void>((size_t)F2 * d * es);
    ly.wdn = cv.take<void>((size_t)d * F * es);
    ly.cap = (l <= m->f0) ? capA : capB;
    ly.kring = cv.take<void>((size_t)ly.cap * d * es);
    ly.vring = cv.take<void>((size_t)ly.cap * d * es);
    ly.vtring = cv.take<void>((size_t)ly.cap * d * es);
    ly.ktring = (l > m->f0) ? cv.take<void>((size_t)ly.cap * d * es) : nullptr;
    if (l > m->f0) {
      ly.wqkvT = cv.take<void>((size_t)3 * d * d * es);
      ly.woT = cv.take<void>((size_t)d * d * es);
    }
    if (m->c.static_mlp && l >= m->f0) {
      ly.swup = cv.take<void>((size_t)F2 * d * es);
      ly.swdn = cv.take<void>((size_t)d * F * es);
      ly.swupT = cv.take<void>((size_t)F2 * d * es);
      ly.swdnT = cv.take<void>((size_t)d * F * es);
    }
  }
  m->UT = cv.take<void>((size_t)V * d * es);
  m->fast.assign(m->q, FastLayer());
  for (int j = 0; j < m->q; ++j) {
    FastLayer& f = m->fast[j];
    f.m_up = cv.take<float>((size_t)F2 * d * 4);
    f.m_dn = cv.take<float>((size_t)d * F * 4);
    if (m->bf) {
      f.s_up = cv.take<void>((size_t)F2 * d * es);
      f.s_dn = cv.take<void>((size_t)d * F * es);
    } else {
      f.s_up = f.m_up;
      f.s_dn = f.m_dn;
    }
    f.ct_up = cv.take<void>((size_t)F2 * d * es);
    f.ct_dn = cv.take<void>((size_t)d * F * es);
  }
  m->theta = cv.take<double>((size_t)(m->hd / 2) * 8);
  m->csA = cv.take<float2>((size_t)MA * (m->hd / 2) * 8);
  m->csB = cv.take<float2>((size_t)C * (m->hd / 2) * 8);
  // phase A
  m->hAb[0] = cv.take<float>((size_t)MA * d * 4);
  m->hAb[1] = cv.take<float>((size_t)MA * d * 4);
  m->hA = m->hAb[0];
  m->aA = cv.take<void>((size_t)MA * d * es);
  m->qkvA = cv.take<void>((size_t)MA * 3 * d * es);
  m->qA = cv.take<void>((size_t)MA * d * es);
  m->oA = cv.take<void>((size_t)MA * d * es);
  m->actA = cv.take<void>((size_t)MA * F * es);
  // phase B
  m->pb.assign(m->q, PB());
  for (int j = 0; j < m->q; ++j) {
    PB& b = m->pb[j];
    if (j > 0) {
      b.xin = cv.take<float>((size_t)C * d * 4);
      b.x2 = cv.take<float>((size_t)C * d * 4);
      b.mean1 = cv.take<float>((size_t)C * 4);
      b.rstd1 = cv.take<float>((size_t)C * 4);
      b.a = cv.take<void>((size_t)C * d * es);
      b.q = cv.take<void>((size_t)C * d * es);
      b.o = cv.take<void>((size_t)C * d * es);
      b.lse = cv.take<float>((size_t)H * C * 4);
    }
    b.mean2 = cv.take<float>((size_t)C * 4);
    b.rstd2 = cv.take<float>((size_t)C * 4);
    b.b = cv.take<void>((size_t)C * d * es);
    b.z = cv.take<void>((size_t)C * F2 * es);
    b.act = cv.take<void>((size_t)C * F * es);
    if (m->c.static_mlp) {
      b.xm = cv.take<float>((size_t)C * d * 4);
      b.mean3 = cv.take<float>((size_t)C * 4);
      b.rstd3 = cv.take<float>((size_t)C * 4);
      b.z2 = cv.take<void>((size_t)C * F2 * es);
    }
  }
  if (m->c.static_mlp) {
    m->cS = cv.take<void>((size_t)C * d * es);
    m->actS = cv.take<void>((size_t)C * F * es);
    m->dzS = cv.take<void>((size_t)C * F2 * es);
  }
  m->xL = cv.take<float>((size_t)C * d * 4);
  m->meanf = cv.take<float>((size_t)C * 4);
  m->rstdf = cv.take<float>((size_t)C * 4);
  m->fN = cv.take<void>((size_t)C * d * es);
  m->qkvB = cv.take<void>((size_t)C * 3 * d * es);
  m->nparts = 2 * ((V + 127) / 128);
  m->pmax = cv.take<float>((size_t)m->nparts * C * 4);
  m->psum = cv.take<float>((size_t)m->nparts * C * 4);
  m->tlog = cv.take<float>((size_t)C * 4);
  m->lse_ce = cv.take<float>((size_t)2 * C * 4);
  m->G = cv.take<void>((size_t)C * V * es);
  m->zce = cv.take<float>((size_t)C * V * 4);
  m->dh = cv.take<float>((size_t)C * d * 4);
  m->dh_lo = cv.take<void>((size_t)C * d * es);
  // transposed operands of the weight-gradient products: [features][Cp],
  // Cp = the chunk capacity rounded up to a multiple of 8 (zero padded)
  m->Cp = round_up((int64_t)C, 8);
  m->tops.assign(m->q, ttt_model::TOps());
  for (int j = 0; j < m->q; ++j) {
    ttt_model::TOps& t = m->tops[j];
    t.dhT = cv.take<void>((size_t)m->Cp * d * es);
    t.actT = cv.take<void>((size_t)m->Cp * F * es);
    t.dzT = cv.take<void>((size_t)m->Cp * F2 * es);
    t.bT = cv.take<void>((size_t)m->Cp * d * es);
  }
  m->dz = cv.take<void>((size_t)C * F2 * es);
  m->dtmp = cv.take<float>((size_t)C * d * 4);
  m->dout = cv.take<void>((size_t)C * d * es);
  m->dqkv = cv.take<void>((size_t)C * 3 * d * es);
  m->Dattn = cv.take<float>((size_t)H * C * 4);
  m->attn_part = cv.take<float>((size_t)kMaxSplit * C * d * 4);
  m->attn_ml = cv.take<float>((size_t)kMaxSplit * H * C * 2 * 4);
  m->Cq = round_up((int64_t)C, 64);
  m->qT = cv.take<void>((size_t)m->Cq * d * es);
  m->gT = cv.take<void>((size_t)m->Cq * d * es);
  m->split_cap = (int64_t)4 * C * std::max(d, 3 * d);
  m->split_ws = cv.take<float>((size_t)m->split_cap * 4);
  // decode
  m->xd = cv.take<float>((size_t)d * 4);
  m->qd = cv.take<void>((size_t)d * es);
  m->od = cv.take<void>((size_t)d * es);
  m->actd = cv.take<void>((size_t)F * es);
  m->logits = cv.take<float>((size_t)V * 4);
  const int64_t nsplit = (m->W + 255) / 256 + 1;
  m->attn_ws = cv.take<float>((size_t)H * nsplit * (2 + m->hd) * 4);
  m->hist = cv.take<int32_t>((size_t)(C + 2) * 4);
  m->cur_tok = cv.take<int32_t>(4);
  m->dstate = cv.take<int64_t>(16);
  m->amax = cv.take<float>((size_t)2 * dgemv_blocks(m->V) * 4);
  m->err = cv.take<int>(4);
  m->nanv = cv.take<float>(4);
  (void)c;
  return cv.off + 256;
}

void init_dims(ttt_model* m, const ttt_config& c) {
  m->c = c;
  m->bf = c.dtype == TTT_BF16;
  m->es = esz(c);
  m->d = c.d_model; m->F = c.d_ff; m->F2 = c.mlp == TTT_MLP_SWIGLU ? 2 * c.d_ff : c.d_ff;
  m->V = c.vocab; m->L = c.n_layers; m->q = c.n_fast; m->f0 = c.n_layers - c.n_fast;
  m->H = c.n_heads; m->hd = c.head_dim; m->W = c.window; m->Cmax = c.max_chunk;
  int ma = c.prefill_block > 0 ? c.prefill_block : 8192;
  if (ma < c.max_chunk) ma = c.max_chunk;
  m->MA = ma;
}

// ---------------------------------------------------------------- timing
struct Scope {
  ttt_model* m; int cls; hipStream_t s; bool on;
  Scope(ttt_model* m_, int cls_, hipStream_t s_, double flops) : m(m_), cls(cls_), s(s_) {
    on = m->tm[cls].on;
    if (!on) return;
    Timing& t = m->tm[cls];
    if (t.used + 2 > t.ev.size()) {
      for (int i = 0; i < 256; ++i) {
        hipEvent_t e;
        if (hipEventCreate(&e) == hipSuccess) t.ev.push_back(e);
      }
    }
    if (t.used + 2 > t.ev.size()) { on = false; return; }
    hipEventRecord(t.ev[t.used], s);
    t.launches += 1;
    t.flops += flops;
  }
  ~Scope() {
    if (!on) return;
    Timing& t = m->tm[cls];
    hipEventRecord(t.ev[t.used + 1], s);
    t.used += 2;
  }
};

enum { CLS_GEMM = 0, CLS_ATTN_FWD = 1, CLS_ATTN_BWD = 2, CLS_CE = 3, CLS_SGD = 4, CLS_MLP_UP = 5 };

int gemm_fail(int rc) {
  if (rc == GEMM_TOO_LARGE) return fail(TTT_ERR_CONFIG, "a GEMM operand spans more than 2^31 - 1 bytes");
  return fail(TTT_ERR_CONFIG, "internal: GEMM variant not built");
}

int run_gemm(ttt_model* m, const GemmParams& p0, bool a_kc, bool b_kc, int epi, bool out_f32,
             hipStream_t s, bool allow_split = true) {
  GemmParams p = p0;
  // the split-K scratch belongs to the phase-B stream; phase A (large M)
  // runs unsplit so the two streams never share it
  p.split_ws = allow_split ? m->split_ws : nullptr;
  p.split_cap = allow_split ? m->split_cap : 0;
  const double fl = 2.0 * p.M * (double)p.N * p.K;
  int rc;
  {
    Scope t0(m, CLS_GEMM, s, fl);
    // class 5 is one kernel symbol: the up-projection with a single B over a
    // whole block of rows (the frozen blocks, unsplit); the fast blocks'
    // two-B launches and the chunk-sized second-MLP launches are other kernels
    const bool up1 = (epi == EPI_GELU || epi == EPI_SWIGLU) && p.B2 == nullptr && !allow_split;
    Scope t4(m, epi == EPI_SGD ? CLS_SGD : up1 ? CLS_MLP_UP : NCLS - 1, s,
             (epi == EPI_SGD || up1) ? fl : 0.0);
    rc = gemm(p, m->bf, a_kc, b_kc, epi, out_f32, s);
  }
  return rc == 0 ? TTT_OK : gemm_fail(rc);
}

// Algorithmic attention work: the number of (query, key) pairs inside the
// window for queries at positions [p0, p0+n), i.e. sum_t min(t+1, W), and
// (inchunk) the pairs whose key is >= kmin = p0.
double window_sum(int64_t a, int64_t b, int64_t W) {   // sum_{t=a}^{b-1} min(t+1, W)
  if (b <= a) return 0.0;
  const int64_t e = std::min<int64_t>(b, W - 1);        // t < W-1 contributes t+1
  double s = 0.0;
  if (e > a) s += 0.5 * (double)(e - a) * (double)(a + 1 + e);
  const int64_t f = std::max<int64_t>(a, W - 1);
  if (b > f) s += (double)W * (double)(b - f);
  return s;
}
double pairs(int64_t p0, int n, int64_t W, int64_t kmin, double* inchunk) {
  if (inchunk) *inchunk = window_sum(p0 - kmin, p0 - kmin + n, W);
  return window_sum(p0, p0 + n, W);
}

// --------------------------------------------------------------- phase A
// One pre-LN block with its loaded weights over nb rows of the residual
// stream x (fp32 [nb][d], positions pos0 .. pos0+nb-1, updated in place):
// LN1 -> QKV -> RoPE (K/V to the layer's rings) -> attention -> O + residual,
// then, when `mlp`, LN2 -> up + activation -> down + residual.  cs holds the
// rotary table rows of these positions.  Its temporaries are the phase-A
// buffers, so it runs on one stream at a time.
int block_fwd(ttt_model* m, int l, int64_t pos0, int nb, float* x, const float2* cs, bool mlp,
              hipStream_t s) {
  const int d = m->d, F = m->F, F2 = m->F2;
  const bool bf = m->bf;
  Layer& ly = m->layers[l];
  layernorm_fwd(x, d, nb, d, m->c.ln_eps, m->aA, d, nullptr, nullptr, bf, s);
  GemmParams g;
  g.A = m->aA; g.lda = d; g.B = ly.wqkv; g.ldb = d; g.M = nb; g.N = 3 * d; g.K = d;
  g.C = m->qkvA; g.ldc = 3 * d;
  int rc = run_gemm(m, g, true, true, EPI_STORE, false, s, false); if (rc) return rc;
  qkv_rope(m->qkvA, nb, m->H, m->hd, pos0, cs, m->qA, ly.kring, ly.vring, ly.vtring, nullptr, ly.cap,
           bf, s);
  AttnParams ap;
  ap.q = m->qA; ap.ldq = d; ap.kring = ly.kring; ap.vring = ly.vring; ap.vtring = ly.vtring; ap.cap = ly.cap;
  ap.n = nb; ap.H = m->H; ap.hd = m->hd; ap.window = m->W; ap.pos0 = pos0; ap.o = m->oA; ap.ldo = d;
  {
    Scope t(m, CLS_ATTN_FWD, s, 4.0 * d * pairs(pos0, nb, m->W, 0, nullptr));
    swa_fwd(ap, bf, s);
  }
  GemmParams go;
  go.A = m->oA; go.lda = d; go.B = ly.wo; go.ldb = d; go.M = nb; go.N = d; go.K = d;
  go.C = x; go.ldc = d; go.R = x; go.ldr = d;
  rc = run_gemm(m, go, true, true, EPI_RESID, true, s, false); if (rc) return rc;
  if (!mlp) return TTT_OK;
  layernorm_fwd(x, d, nb, d, m->c.ln_eps, m->aA, d, nullptr, nullptr, bf, s);
  GemmParams gu;
  gu.A = m->aA; gu.lda = d; gu.B = ly.wup; gu.ldb = d; gu.M = nb; gu.N = F2; gu.K = d;
  gu.C2 = m->actA; gu.ldc2 = F;     // no backward here: the pre-activations are not kept
  rc = run_gemm(m, gu, true, true, m->c.mlp == TTT_MLP_SWIGLU ? EPI_SWIGLU : EPI_GELU, false, s, false);
  if (rc) return rc;
  GemmParams gd;
  gd.A = m->actA; gd.lda = F; gd.B = ly.wdn; gd.ldb = F; gd.M = nb; gd.N = d; gd.K = F;
  gd.C = x; gd.ldc = d; gd.R = x; gd.ldr = d;
  rc = run_gemm(m, gd, true, true, EPI_RESID, true, s, false);
  if (rc || !ly.swup) return rc;
  // the frozen second MLP of a fast block: LN3 -> up + activation -> down + residual
  layernorm_fwd(x, d, nb, d, m->c.ln_eps, m->aA, d, nullptr, nullptr, bf, s);
  gu.B = ly.swup;
  rc = run_gemm(m, gu, true, true, m->c.mlp == TTT_MLP_SWIGLU ? EPI_SWIGLU : EPI_GELU, false, s, false);
  if (rc) return rc;
  gd.B = ly.swdn;
  return run_gemm(m, gd, true, true, EPI_RESID, true, s, false);
}

// Phase A of one block of positions [B0, B0+nb): embedding, every frozen
// block and the attention half of the first fast block.
int phase_a(ttt_model* m, const int32_t* tokens, int64_t B0, int nb, float* hA, hipStream_t s) {
  embed(tokens + B0, nb, m->E, m->d, m->V, m->bf, hA, m->err, s);
  rope_table(B0, nb, m->hd / 2, m->theta, m->csA, s);
  for (int l = 0; l <= m->f0; ++l) {
    const int rc = block_fwd(m, l, B0, nb, hA, m->csA, l < m->f0, s);
    if (rc) return rc;
  }
  return TTT_OK;
}

// --------------------------------------------------------------- phase B
// One step on one chunk: positions [p0, p0+n), x2_0 = residual stream after
// the attention of the first fast block ([n][d] fp32), targets tgt[0..n_tgt).
int chunk_step(ttt_model* m, int64_t p0, int n, const float* x2_0, const int32_t* tgt, int n_tgt,
               float lr, float* loss_out, hipStream_t s) {
  const int d = m->d, F = m->F, F2 = m->F2, V = m->V, q = m->q;
  const bool bf = m->bf;
  const float eps = m->c.ln_eps;
  const int upepi = m->c.mlp == TTT_MLP_SWIGLU ? EPI_SWIGLU : EPI_GELU;
  int rc;
  rope_table(p0, n, m->hd / 2, m->theta, m->csB, s);
  m->logit_rows = n;
  // ---------------- forward of the fast blocks
  // The QKV, output and down products of a chunk leave their K-split
  // partial slabs (when split) for their consumer to sum: the RoPE pass for
  // QKV, the next LayerNorm (which adds the residual and stores the sum) for
  // the others; pend / pend_r: a down product still owed to the residual.
  int pend = 1;
  const float* pend_r = nullptr;
  for (int j = 0; j < q; ++j) {
    const int l = m->f0 + j;
    Layer& ly = m->layers[l];
    PB& b = m->pb[j];
    const float* x2 = x2_0;
    int npo = 1;                                     // slabs of the output product
    if (j > 0) {
      if (pend > 1) layernorm_fwd_resid(m->split_ws, pend, pend_r, b.xin, n, d, eps, b.a, d, b.mean1, b.rstd1, bf, s);
      else layernorm_fwd(b.xin, d, n, d, eps, b.a, d, b.mean1, b.rstd1, bf, s);
      pend = 1;
      GemmParams g;
      int nq = 1;
      g.A = b.a; g.lda = d; g.B = ly.wqkv; g.ldb = d; g.M = n; g.N = 3 * d; g.K = d;
      g.C = m->qkvB; g.ldc = 3 * d; g.split_defer = &nq;
      rc = run_gemm(m, g, true, true, EPI_STORE, false, s); if (rc) return rc;
      qkv_rope(m->qkvB, n, m->H, m->hd, p0, m->csB, b.q, ly.kring, ly.vring, ly.vtring, ly.ktring, ly.cap,
               bf, s, nq > 1 ? m->split_ws : nullptr, nq);
      AttnParams ap;
      ap.q = b.q; ap.ldq = d; ap.kring = ly.kring; ap.vring = ly.vring; ap.vtring = ly.vtring; ap.cap = ly.cap;
      ap.n = n; ap.H = m->H; ap.hd = m->hd; ap.window = m->W; ap.pos0 = p0; ap.o = b.o; ap.ldo = d;
      ap.lse = b.lse;
      ap.part = m->attn_part; ap.part_ml = m->attn_ml; ap.max_split = kMaxSplit;
      {
        Scope t(m, CLS_ATTN_FWD, s, 4.0 * d * pairs(p0, n, m->W, 0, nullptr));
        swa_fwd(ap, bf, s);
      }
      GemmParams go;
      go.A = b.o; go.lda = d; go.B = ly.wo; go.ldb = d; go.M = n; go.N = d; go.K = d;
      go.C = b.x2; go.ldc = d; go.R = b.xin; go.ldr = d; go.split_defer = &npo;
      rc = run_gemm(m, go, true, true, EPI_RESID, true, s); if (rc) return rc;
      x2 = b.x2;
    }
    // the previous chunk's updates of block 0 (up, then down; every other
    // block's ran before them on the in-order update stream)
    // The LayerNorm only rewrites b, which the up update's operand
    // transposes have read (evR2[0]), so it runs beside that update; the up
    // product needs the updated matrix and act read by the down update's
    // transposes (evR1[0]).
    const bool owed = j == 0 && m->sgd_open;
    if (owed) HIPCHK(hipStreamWaitEvent(s, m->evR2[0], 0));   // b read
    if (npo > 1) layernorm_fwd_resid(m->split_ws, npo, b.xin, b.x2, n, d, eps, b.b, d, b.mean2, b.rstd2, bf, s);
    else layernorm_fwd(x2, d, n, d, eps, b.b, d, b.mean2, b.rstd2, bf, s);
    if (owed) HIPCHK(hipStreamWaitEvent(s, m->evR1[0], 0));   // up updated, act read
    GemmParams gu;
    gu.A = b.b; gu.lda = d; gu.B = ly.wup; gu.B2 = m->fast[j].s_up; gu.ldb = d; gu.M = n; gu.N = F2; gu.K = d;
    gu.C = b.z; gu.ldc = F2; gu.C2 = b.act; gu.ldc2 = F;
    rc = run_gemm(m, gu, true, true, upepi, false, s); if (rc) return rc;
    float* xout = (j + 1 < q) ? m->pb[j + 1].xin : m->xL;
    if (owed) {
      HIPCHK(hipStreamWaitEvent(s, m->evC, 0));                // down updated
      m->sgd_open = false;
    }
    GemmParams gd;
    int nd = 1;
    gd.A = b.act; gd.lda = F; gd.B = ly.wdn; gd.B2 = m->fast[j].s_dn; gd.ldb = F; gd.M = n; gd.N = d; gd.K = F;
    gd.C = ly.swup ? b.xm : xout; gd.ldc = d; gd.R = x2; gd.ldr = d;
    if (!ly.swup) gd.split_defer = &nd;
    rc = run_gemm(m, gd, true, true, EPI_RESID, true, s); if (rc) return rc;
    if (nd > 1) { pend = nd; pend_r = x2; }
    if (ly.swup) {
      // frozen second MLP: LN3 -> up + activation (pre-activations kept for
      // the backward) -> down + residual
      layernorm_fwd(b.xm, d, n, d, eps, m->cS, d, b.mean3, b.rstd3, bf, s);
      GemmParams su;
      su.A = m->cS; su.lda = d; su.B = ly.swup; su.ldb = d; su.M = n; su.N = F2; su.K = d;
      su.C = b.z2; su.ldc = F2; su.C2 = m->actS; su.ldc2 = F;
      rc = run_gemm(m, su, true, true, upepi, false, s); if (rc) return rc;
      GemmParams sd;
      sd.A = m->actS; sd.lda = F; sd.B = ly.swdn; sd.ldb = F; sd.M = n; sd.N = d; sd.K = F;
      sd.C = xout; sd.ldc = d; sd.R = b.xm; sd.ldr = d;
      rc = run_gemm(m, sd, true, true, EPI_RESID, true, s); if (rc) return rc;
    }
  }
  if (pend > 1) layernorm_fwd_resid(m->split_ws, pend, pend_r, m->xL, n, d, eps, m->fN, d, m->meanf, m->rstdf, bf, s);
  else layernorm_fwd(m->xL, d, n, d, eps, m->fN, d, m->meanf, m->rstdf, bf, s);

  // ---------------- fused head + cross-entropy
  {
    Scope t(m, CLS_CE, s, 2.0 * n * (double)d * V);
    GemmParams gs;
    gs.A = m->fN; gs.lda = d; gs.B = m->U; gs.ldb = d; gs.M = n; gs.N = V; gs.K = d;
    gs.tgt = tgt; gs.n_tgt = n_tgt; gs.part_max = m->pmax; gs.part_sum = m->psum;
    gs.ldpart = m->Cmax; gs.tgt_logit = m->tlog;
    gs.C = m->zce; gs.ldc = V;      // logits kept for the gradient pass
    if (const int rg = gemm(gs, bf, true, true, EPI_CESTAT, true, s)) return gemm_fail(rg);
    ce_finish(m->pmax, m->psum, m->nparts, m->Cmax, m->tlog, n, n_tgt, m->lse_ce, loss_out, m->err, s);
  }
  if (n_tgt <= 0) return TTT_OK;   // nothing to learn from this chunk
  // The products feeding a LayerNorm backward (d = G.U, db, da) leave their
  // K-split partial slabs in the split scratch; the LayerNorm backward sums
  // them (nsl slabs) instead of a separate reduction pass.
  int nsl = 1;
  auto dy_of = [&]() -> const float* { return nsl > 1 ? m->split_ws : m->dtmp; };
  {
    Scope t(m, CLS_CE, s, 2.0 * n * (double)d * V);
    // G = (softmax - onehot) / n_targets from the stored logits (a stream
    // over C x V instead of recomputing the logits product)
    ce_grad(m->zce, V, m->lse_ce, tgt, n, n_tgt, V, 1.f / (float)n_tgt, m->G, V, bf, s);
    GemmParams gx;   // dHf = G . U  (through U^T [d][V], k-contiguous over the vocabulary)
    gx.A = m->G; gx.lda = V; gx.B = m->UT; gx.ldb = V; gx.M = n; gx.N = d; gx.K = V;
    gx.C = m->dtmp; gx.ldc = d;
    gx.split_ws = m->split_ws; gx.split_cap = m->split_cap; gx.split_defer = &nsl;
    if (const int rg = gemm(gx, bf, true, true, EPI_STORE, true, s)) return gemm_fail(rg);
  }
  fill_f32(m->dh, (int64_t)n * d, 0.f, s);
  layernorm_bwd_acc(dy_of(), m->xL, m->meanf, m->rstdf, n, d, m->dh, m->dh_lo, bf, s, nsl, (int64_t)n * d);

  // ---------------- backward through the fast blocks, SGD fused
  for (int j = q - 1; j >= 0; --j) {
    const int l = m->f0 + j;
    Layer& ly = m->layers[l];
    PB& b = m->pb[j];
    FastLayer& fw = m->fast[j];
    const float* x2 = (j > 0) ? b.x2 : x2_0;
    // Every product below runs with both operands k-contiguous: the weights
    // through their transposed copies, the activations of the weight
    // gradients transposed to [features][tokens] (tokens padded to a multiple
    // of 8 with zeros, which add nothing to the reduction).
    const int np = (n + 7) & ~7;
    if (ly.swup) {
      // back through the frozen second MLP (no weight gradient): dz2 =
      // act'(z2) (dh . Wdn2), dc = dz2 . Wup2, dh += LN3_backward(dc)
      GemmParams sa2;
      sa2.A = m->dh_lo; sa2.lda = d; sa2.B = ly.swdnT; sa2.ldb = d; sa2.M = n; sa2.N = F; sa2.K = d;
      sa2.C = m->dzS; sa2.ldc = F2; sa2.Z = b.z2; sa2.ldz = F2; sa2.act_swiglu = m->c.mlp == TTT_MLP_SWIGLU;
      rc = run_gemm(m, sa2, true, true, EPI_ACTBWD, false, s); if (rc) return rc;
      GemmParams sb2;
      sb2.A = m->dzS; sb2.lda = F2; sb2.B = ly.swupT; sb2.ldb = F2; sb2.M = n; sb2.N = d; sb2.K = F2;
      sb2.C = m->dtmp; sb2.ldc = d; sb2.split_defer = &nsl;
      nsl = 1;
      rc = run_gemm(m, sb2, true, true, EPI_STORE, true, s); if (rc) return rc;
      layernorm_bwd_acc(dy_of(), b.xm, b.mean3, b.rstd3, n, d, m->dh, m->dh_lo, bf, s, nsl, (int64_t)n * d);
    }
    // dz = act'(z) (dh . Wdn): the activation backward runs in the product's
    // epilogue (the product reads the weights before their update: Wdn^T
    // [F][d]).  dz is rewritten here: the update stream must have read the
    // block above's.
    if (j + 1 < q) HIPCHK(hipStreamWaitEvent(s, m->evR2[j + 1], 0));
    ttt_model::TOps& to = m->tops[j];
    // The update stream's pieces: operand transposes, then the SGD products.
    auto trans_dn = [&]() {               // operands of the down update
      transpose(m->dh_lo, n, d, d, to.dhT, m->Cp, np, bf, m->sc);
      transpose(b.act, n, F, F, to.actT, m->Cp, np, bf, m->sc);
    };
    // Wdn -= lr * dh^T act   ([d][F], reduction over the chunk's tokens)
    auto sgd_dn = [&]() -> int {
      GemmParams gw;
      gw.A = to.dhT; gw.lda = m->Cp; gw.B = to.actT; gw.ldb = m->Cp; gw.M = d; gw.N = F; gw.K = np;
      gw.C = fw.m_dn; gw.ldc = F; gw.C2 = bf ? fw.s_dn : nullptr; gw.ldc2 = F; gw.alpha = lr;
      gw.C3 = fw.ct_dn; gw.ldc3 = d; gw.W0 = ly.wdn;
      return run_gemm(m, gw, true, true, EPI_SGD, true, m->sc);
    };
    // Wup -= lr * dz^T b
    auto sgd_up = [&]() -> int {
      GemmParams gw2;
      gw2.A = to.dzT; gw2.lda = m->Cp; gw2.B = to.bT; gw2.ldb = m->Cp; gw2.M = F2; gw2.N = d; gw2.K = np;
      gw2.C = fw.m_up; gw2.ldc = d; gw2.C2 = bf ? fw.s_up : nullptr; gw2.ldc2 = d; gw2.alpha = lr;
      gw2.C3 = fw.ct_up; gw2.ldc3 = F2; gw2.W0 = ly.wup;
      return run_gemm(m, gw2, true, true, EPI_SGD, true, m->sc);
    };
    if (j == 0) {
      // Block 0's update operands other than dz (dh_lo, act, b) are final
      // here: they are transposed on the update stream while ga runs, so
      // that only dz's transpose and the up update stand between ga and
      // the next chunk's up product.
      HIPCHK(hipEventRecord(m->evT1[0], s));
      HIPCHK(hipStreamWaitEvent(m->sc, m->evT1[0], 0));
      trans_dn();
      transpose(b.b, n, d, d, to.bT, m->Cp, np, bf, m->sc);
    }
    // dz = act'(z) (dh . Wdn): the activation backward runs in the product's
    // epilogue (the product reads the weights before their update: Wdn^T
    // [F][d]).  dz is rewritten here: the update stream must have read the
    // block above's.
    GemmParams ga;
    ga.A = m->dh_lo; ga.lda = d; ga.B = fw.ct_dn; ga.ldb = d; ga.M = n; ga.N = F; ga.K = d;
    ga.C = m->dz; ga.ldc = F2; ga.Z = b.z; ga.ldz = F2; ga.act_swiglu = m->c.mlp == TTT_MLP_SWIGLU;
    rc = run_gemm(m, ga, true, true, EPI_ACTBWD, false, s); if (rc) return rc;
    // The updates run on the update stream, after ga has read the old
    // weights; the chain goes on at once.
    if (j == 0) {
      // block 0 is the last to be updated and the first the next chunk
      // reads, up matrix first: up, then down, so that the next chunk's up
      // product can run beside the down update
      HIPCHK(hipEventRecord(m->evT2[0], s));
      HIPCHK(hipStreamWaitEvent(m->sc, m->evT2[0], 0));
      transpose(m->dz, n, F2, F2, to.dzT, m->Cp, np, bf, m->sc);
      HIPCHK(hipEventRecord(m->evR2[0], m->sc));      // dz and b read
      rc = sgd_up(); if (rc) return rc;
      HIPCHK(hipEventRecord(m->evR1[0], m->sc));      // up updated; dh_lo and act read
      rc = sgd_dn(); if (rc) return rc;
      break;   // no gradient below the first fast MLP
    }
    auto update_dn = [&]() -> int {
      HIPCHK(hipEventRecord(m->evT1[j], s));
      HIPCHK(hipStreamWaitEvent(m->sc, m->evT1[j], 0));
      trans_dn();
      HIPCHK(hipEventRecord(m->evR1[j], m->sc));      // dh_lo and act read
      return sgd_dn();
    };
    // (after gb has read the old up weights)
    auto update_up = [&]() -> int {
      HIPCHK(hipEventRecord(m->evT2[j], s));
      HIPCHK(hipStreamWaitEvent(m->sc, m->evT2[j], 0));
      transpose(m->dz, n, F2, F2, to.dzT, m->Cp, np, bf, m->sc);
      transpose(b.b, n, d, d, to.bT, m->Cp, np, bf, m->sc);
      HIPCHK(hipEventRecord(m->evR2[j], m->sc));      // dz and b read
      return sgd_up();
    };
    rc = update_dn(); if (rc) return rc;
    {
      GemmParams gb;   // db = dz . Wup (before its update: Wup^T [d][F2])
      gb.A = m->dz; gb.lda = F2; gb.B = fw.ct_up; gb.ldb = F2; gb.M = n; gb.N = d; gb.K = F2;
      gb.C = m->dtmp; gb.ldc = d; gb.split_defer = &nsl;
      nsl = 1;
      rc = run_gemm(m, gb, true, true, EPI_STORE, true, s); if (rc) return rc;
    }
    rc = update_up(); if (rc) return rc;
    HIPCHK(hipStreamWaitEvent(s, m->evR1[j], 0));   // dh_lo is rewritten below
    layernorm_bwd_acc(dy_of(), x2, b.mean2, b.rstd2, n, d, m->dh, m->dh_lo, bf, s, nsl, (int64_t)n * d);
    GemmParams gdo;   // dO = dh . Wo  (Wo^T [d][d])
    gdo.A = m->dh_lo; gdo.lda = d; gdo.B = ly.woT; gdo.ldb = d; gdo.M = n; gdo.N = d; gdo.K = d;
    gdo.C = m->dout; gdo.ldc = d;
    // D = rowsum(O * dO) per head: in the split product's reduction pass
    // when it has one, else by its own pass
    int rd_done = 0;
    gdo.rd_o = b.o; gdo.rd_D = m->Dattn; gdo.rd_hd = m->hd; gdo.rd_done = &rd_done;
    rc = run_gemm(m, gdo, true, true, EPI_STORE, false, s); if (rc) return rc;
    if (!rd_done) attn_rowdot(b.o, m->dout, n, m->H, m->hd, m->Dattn, bf, s);
    AttnParams ap;
    ap.q = b.q; ap.ldq = d; ap.kring = ly.kring; ap.vring = ly.vring; ap.cap = ly.cap;
    ap.n = n; ap.H = m->H; ap.hd = m->hd; ap.window = m->W; ap.pos0 = p0;
    ap.lse = b.lse; ap.dout = m->dout; ap.lddo = d; ap.D = m->Dattn;
    ap.ktring = ly.ktring;
    ap.part = m->attn_part; ap.part_ml = m->attn_ml; ap.max_split = kMaxSplit;
    ap.dq = m->dqkv; ap.dk = static_cast<char*>(m->dqkv) + (size_t)d * m->es;
    ap.dv = static_cast<char*>(m->dqkv) + (size_t)2 * d * m->es; ap.ldg = 3 * d; ap.kmin = p0;
    ap.rope_cs = m->csB;                             // RoPE^-1 inside the kernels where they can
    int rotated = 0;
    {
      double in = 0;
      const double tot = pairs(p0, n, m->W, p0, &in);
      Scope t(m, CLS_ATTN_BWD, s, 4.0 * d * (tot + in));
      HIPCHK(hipEventRecord(m->evK0, s));            // inputs of dK/dV ready
      HIPCHK(hipStreamWaitEvent(m->sk, m->evK0, 0));
      if (swa_bwd_reads_transposes(m->hd, bf)) {
        const int npad = (int)round_up((int64_t)n, 64);
        transpose(b.q, n, d, d, m->qT, m->Cq, npad, bf, m->sk, true);
        transpose(m->dout, n, d, d, m->gT, m->Cq, npad, bf, m->sk, true);
        ap.qtr = m->qT; ap.gtr = m->gT; ap.ldtr = m->Cq;
      }
      rotated = swa_bwd(ap, bf, s, m->sk);
      HIPCHK(hipEventRecord(m->evK1, m->sk));
      HIPCHK(hipStreamWaitEvent(s, m->evK1, 0));     // dK/dV in place for the RoPE backward
    }
    rope_bwd(m->dqkv, n, m->H, m->hd, m->csB, bf, s, 3 & ~rotated);
    GemmParams gq;   // da = dqkv . Wqkv  (Wqkv^T [d][3d])
    gq.A = m->dqkv; gq.lda = 3 * d; gq.B = ly.wqkvT; gq.ldb = 3 * d; gq.M = n; gq.N = d; gq.K = 3 * d;
    gq.C = m->dtmp; gq.ldc = d; gq.split_defer = &nsl;
    nsl = 1;
    rc = run_gemm(m, gq, true, true, EPI_STORE, true, s); if (rc) return rc;
    layernorm_bwd_acc(dy_of(), b.xin, b.mean1, b.rstd1, n, d, m->dh, m->dh_lo, bf, s, nsl, (int64_t)n * d);
  }
  // every update of this chunk lands before the next chunk's forward reads
  // the new weights: here, or (within a prefill) at block 0's MLP of that
  // forward
  HIPCHK(hipEventRecord(m->evC, m->sc));
  if (m->sgd_defer) m->sgd_open = true;
  else HIPCHK(hipStreamWaitEvent(s, m->evC, 0));
  return TTT_OK;
}

// ------------------------------------------------------- forward only
// One block of positions [B0, B0+nb) read with the loaded weights and no
// update: every block batched over the rows (the fast blocks too, since
// their MLPs keep their initial values), then the final LayerNorm and the
// fused head + cross-entropy statistics per chunk.  The fast blocks' rings
// hold window + max_chunk positions, so their layers run over sub-blocks
// that never overwrite a key a later query of the block still reads.
int forward_block(ttt_model* m, const int32_t* tokens, int64_t T, int64_t B0, int nb, int chunk,
                  float* losses, hipStream_t s) {
  const int d = m->d, half = m->hd / 2;
  const bool bf = m->bf;
  float* x = m->hAb[0];
  embed(tokens + B0, nb, m->E, d, m->V, bf, x, m->err, s);
  rope_table(B0, nb, half, m->theta, m->csA, s);
  for (int l = 0; l < m->L; ++l) {
    for (int o = 0; o < nb;) {
      // rows [p, p+sb) write sb ring slots and read keys back to
      // max(0, p - W + 1): all distinct modulo cap while the span fits;
      // whole 64-row groups where possible
      const int64_t p = B0 + o;
      int64_t room = m->layers[l].cap - std::min<int64_t>(p, m->W - 1);
      if (room >= 64) room -= room % 64;
      const int sb = (int)std::min<int64_t>(nb - o, room);
      const int rc = block_fwd(m, l, p, sb, x + (int64_t)o * d, m->csA + (int64_t)o * half, true, s);
      if (rc) return rc;
      o += sb;
    }
  }
  for (int64_t c0 = B0; c0 < B0 + nb; c0 += chunk) {
    const int n = (int)std::min<int64_t>(chunk, T - c0);
    const int n_tgt = (int)std::min<int64_t>(n, T - 1 - c0);
    layernorm_fwd(x + (c0 - B0) * d, d, n, d, m->c.ln_eps, m->fN, d, nullptr, nullptr, bf, s);
    {
      Scope t(m, CLS_CE, s, 2.0 * n * (double)d * m->V);
      GemmParams gs;
      gs.A = m->fN; gs.lda = d; gs.B = m->U; gs.ldb = d; gs.M = n; gs.N = m->V; gs.K = d;
      gs.tgt = tokens + c0 + 1; gs.n_tgt = n_tgt; gs.part_max = m->pmax; gs.part_sum = m->psum;
      gs.ldpart = m->Cmax; gs.tgt_logit = m->tlog;
      if (const int rg = gemm(gs, bf, true, true, EPI_CESTAT, true, s)) return gemm_fail(rg);
      ce_finish(m->pmax, m->psum, m->nparts, m->Cmax, m->tlog, n, n_tgt, m->lse_ce,
                losses + (c0 / chunk), m->err, s);
    }
    if (c0 + n == T) {   // first decode token: argmax of the last position's logits
      const char* frow = static_cast<const char*>(m->fN) + (size_t)(n - 1) * d * m->es;
      dgemv_vec(m->U, nullptr, m->V, d, frow, m->logits, nullptr, nullptr, nullptr, m->amax, bf, s);
      argmax_part(m->amax, dgemv_blocks(m->V), m->cur_tok, nullptr, nullptr, false, s);
      dec_set(m->dstate, T, 0, s);
    }
  }
  return TTT_OK;
}

// One decode token: read the current token at position dstate[0], append
// its K/V to every ring, and leave the next greedy token in cur_tok.  No
// argument depends on the position, so the launches can be captured once.
void decode_body(ttt_model* m, hipStream_t s) {
  const int d = m->d, F = m->F, V = m->V;
  const bool bf = m->bf;
  const float eps = m->c.ln_eps;
  const bool sw = m->c.mlp == TTT_MLP_SWIGLU;
  dec_embed(m->cur_tok, m->dstate, m->hist, m->E, d, V, m->xd, m->err, bf, s);
  for (int l = 0; l < m->L; ++l) {
    Layer& ly = m->layers[l];
    const int j = l - m->f0;
    // LN1 -> qkv -> RoPE -> rings
    dgemv_ln_rope(ly.wqkv, d, m->xd, eps, m->H, m->hd, m->theta, m->dstate, m->qd, ly.kring,
                  ly.vring, ly.cap, bf, s);
    swa_decode(m->qd, ly.kring, ly.vring, ly.cap, m->H, m->hd, m->W, m->dstate, m->od, m->attn_ws,
               bf, s);
    // x += o Wo; the first fast block's input row is also kept for the
    // decode-chunk update
    dgemv_vec(ly.wo, nullptr, d, d, m->od, m->xd, m->xd, j == 0 ? m->hA : nullptr, m->dstate,
              nullptr, bf, s);
    const void* dup = j >= 0 ? m->fast[j].s_up : nullptr;
    const void* ddn = j >= 0 ? m->fast[j].s_dn : nullptr;
    dgemv_ln_act(ly.wup, dup, F, d, m->xd, eps, sw, m->actd, bf, s);   // LN2 -> up -> act
    dgemv_vec(ly.wdn, ddn, d, F, m->actd, m->xd, m->xd, nullptr, nullptr, nullptr, bf, s);
    if (ly.swup) {   // frozen second MLP
      dgemv_ln_act(ly.swup, nullptr, F, d, m->xd, eps, sw, m->actd, bf, s);
      dgemv_vec(ly.swdn, nullptr, d, F, m->actd, m->xd, m->xd, nullptr, nullptr, nullptr, bf, s);
    }
  }
  dgemv_ln_head(m->U, V, d, m->xd, eps, m->logits, m->amax, bf, s);
  argmax_part(m->amax, dgemv_blocks(V), m->cur_tok, m->hist, m->dstate, true, s);
}

int sync_and_check(ttt_model* m, hipStream_t s) {
  HIPCHK(hipStreamSynchronize(s));
  int e = 0;
  HIPCHK(hipMemcpy(&e, m->err, sizeof(int), hipMemcpyDeviceToHost));
  if (e & 1) return fail(TTT_ERR_TOKEN, "a token id outside [0, vocab) was read");
  if (e & 2) return fail(TTT_ERR_NONFINITE, "a chunk loss was not finite");
  return TTT_OK;
}

int reset_state(ttt_model* m, hipStream_t s) {
  const int d = m->d, F = m->F, F2 = m->F2;
  for (int j = 0; j < m->q; ++j) {
    Layer& ly = m->layers[m->f0 + j];
    FastLayer& f = m->fast[j];
    fill_f32(f.m_up, (int64_t)F2 * d, 0.f, s);
    fill_f32(f.m_dn, (int64_t)d * F, 0.f, s);
    if (m->bf) {   // zero bits are 0 in bf16 too
      fill_f32(static_cast<float*>(f.s_up), (int64_t)F2 * d * (int64_t)m->es / 4, 0.f, s);
      fill_f32(static_cast<float*>(f.s_dn), (int64_t)d * F * (int64_t)m->es / 4, 0.f, s);
    }
    transpose(ly.wup, F2, d, d, f.ct_up, F2, F2, m->bf, s);   // W0^T: no update yet
    transpose(ly.wdn, d, F, F, f.ct_dn, d, d, m->bf, s);
  }
  for (int l = 0; l < m->L; ++l) {
    Layer& ly = m->layers[l];
    const int64_t n = ly.cap * d * (int64_t)m->es / 4;
    fill_f32(static_cast<float*>(ly.kring), n, 0.f, s);
    fill_f32(static_cast<float*>(ly.vring), n, 0.f, s);
    fill_f32(static_cast<float*>(ly.vtring), n, 0.f, s);
    if (ly.ktring) fill_f32(static_cast<float*>(ly.ktring), n, 0.f, s);
  }
  fill_f32(reinterpret_cast<float*>(m->err), 1, 0.f, s);
  m->pos = 0;
  m->dchunk0 = 0;
  m->prefilled = false;
  m->no_update = false;
  return TTT_OK;
}

// ------------------------------------------------------------ prefill run
// One context's prefill as a sequence of enqueue steps (one chunk and all
// its steps at a time), so that several contexts can be interleaved.
struct PrefillRun {
  ttt_model* m = nullptr;
  const int32_t* tokens = nullptr;
  int64_t T = 0;
  int chunk = 1;
  float lr = 0.f;
  int steps = 1;
  float* losses = nullptr;
  hipStream_t s = nullptr;     // the chunk chain's stream
  int64_t blk = 0, nblocks = 0;
  int64_t b = 0, c0 = 0, k = 0;   // current block, next chunk start, its index
};

int prefill_check(ttt_model* m, const int32_t* tokens, int64_t T, int32_t chunk, float lr, int32_t steps,
                  float* chunk_losses) {
  if (!m || !tokens || !chunk_losses) return fail(TTT_ERR_ARG, "NULL argument");
  if (T < 2) return fail(TTT_ERR_ARG, "T must be >= 2");
  if (chunk < 1 || chunk > m->Cmax) return fail(TTT_ERR_ARG, "chunk must be in [1, max_chunk]");
  if (steps < 1) return fail(TTT_ERR_ARG, "steps must be >= 1");
  if (!std::isfinite(lr)) return fail(TTT_ERR_ARG, "lr must be finite");
  return TTT_OK;
}

// Phase A of block b+1 (frozen layers, independent of the fast weights)
// runs on m->sa while phase B of block b runs on the chain stream.
// evA[b%2]: block b's phase-A output is ready; evB[b%2]: phase B is done
// reading it, so the buffer can take block b+2.
int prefill_launch_a(PrefillRun& r, int64_t b) {
  ttt_model* m = r.m;
  const int64_t B0 = b * r.blk;
  const int nb = (int)std::min<int64_t>(r.blk, r.T - B0);
  if (b >= 2) HIPCHK(hipStreamWaitEvent(m->sa, m->evB[b % 2], 0));
  const int rc = phase_a(m, r.tokens, B0, nb, m->hAb[b % 2], m->sa);
  if (rc) return rc;
  HIPCHK(hipEventRecord(m->evA[b % 2], m->sa));
  return TTT_OK;
}

int prefill_begin(PrefillRun& r) {
  ttt_model* m = r.m;
  int rc = reset_state(m, r.s);
  if (rc) return rc;
  m->sgd_open = false;
  m->lr = r.lr;
  m->steps = r.steps;
  m->chunk = r.chunk;
  r.blk = std::max<int64_t>(r.chunk, (m->MA / r.chunk) * (int64_t)r.chunk);
  r.nblocks = (r.T + r.blk - 1) / r.blk;
  r.b = r.c0 = r.k = 0;
  HIPCHK(hipEventRecord(m->ev0, r.s));
  HIPCHK(hipStreamWaitEvent(m->sa, m->ev0, 0));
  return prefill_launch_a(r, 0);
}

// Enqueue the next chunk (with all its steps).
int prefill_next(PrefillRun& r) {
  ttt_model* m = r.m;
  const int d = m->d;
  const int64_t B0 = r.b * r.blk;
  const int nb = (int)std::min<int64_t>(r.blk, r.T - B0);
  if (r.c0 == B0) {   // the block's first chunk
    if (r.b + 1 < r.nblocks) {
      const int rc = prefill_launch_a(r, r.b + 1);
      if (rc) return rc;
    }
    HIPCHK(hipStreamWaitEvent(r.s, m->evA[r.b % 2], 0));
  }
  const float* hAblk = m->hAb[r.b % 2];
  const int64_t c0 = r.c0;
  const int n = (int)std::min<int64_t>(r.chunk, r.T - c0);
  const int n_tgt = (int)std::min<int64_t>(n, r.T - 1 - c0);
  for (int st = 0; st < r.steps; ++st) {
    // the last step of the last chunk joins its updates before returning
    m->sgd_defer = c0 + n < r.T || st + 1 < r.steps;
    const int rc = chunk_step(m, c0, n, hAblk + (c0 - B0) * (int64_t)d, r.tokens + c0 + 1, n_tgt, r.lr,
                              r.losses + r.k * r.steps + st, r.s);
    m->sgd_defer = false;
    if (rc) return rc;
  }
  if (c0 + n == r.T) {
    // first decode token: argmax of the last position's logits from this
    // chunk's last read
    const char* frow = static_cast<const char*>(m->fN) + (size_t)(n - 1) * d * m->es;
    dgemv_vec(m->U, nullptr, m->V, d, frow, m->logits, nullptr, nullptr, nullptr, m->amax, m->bf, r.s);
    argmax_part(m->amax, dgemv_blocks(m->V), m->cur_tok, nullptr, nullptr, false, r.s);
    dec_set(m->dstate, r.T, 0, r.s);
  }
  r.c0 += n;
  r.k += 1;
  if (r.c0 >= B0 + nb) {   // the block is done: its phase-A buffer may be refilled
    HIPCHK(hipEventRecord(m->evB[r.b % 2], r.s));
    r.b += 1;
  }
  return TTT_OK;
}

// After a failed enqueue: wait for what the model's own streams still hold,
// so that a later call cannot race with it (the caller's stream orders the
// rest).
void drain(ttt_model* m) {
  for (hipStream_t q : {m->sa, m->sc, m->sk, m->sb})
    if (q) (void)hipStreamSynchronize(q);
}

int prefill_finish(PrefillRun& r, hipStream_t s) {
  ttt_model* m = r.m;
  const int rc = sync_and_check(m, s);
  if (rc) return rc;
  m->pos = r.T;
  m->dchunk0 = r.T;
  m->prefilled = true;
  return TTT_OK;
}

}  // namespace

// ======================================================================= ABI
extern "C" {

int ttt_workspace_bytes(const ttt_config* cfg, size_t* bytes) {
  int rc = check_config(cfg);
  if (rc) return rc;
  if (!bytes) return fail(TTT_ERR_ARG, "bytes is NULL");
  ttt_model tmp;
  init_dims(&tmp, *cfg);
  *bytes = layout(&tmp, nullptr);
  return TTT_OK;
}

// ------------------------------------------------------- static workspace
// Device state of a model loaded by ttt_model_load_static, for callers that
// cannot allocate device memory: a file-scope device array, of which every
// GPU the library runs on holds its own copy until the process ends.  In
// host code `scratch` only names the symbol (passing it to a kernel would
// hand the kernel a host address); its address on each device is taken once
// with hipGetSymbolAddress, with that device current, and kept per device.
constexpr size_t kStaticWorkspaceBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kStaticWorkspaceBytes];

namespace {

struct StaticWorkspace {
  void* ptr = nullptr;          // device address of `scratch` on this device
  ttt_model* owner = nullptr;   // the model whose state lives there, if any
};
std::mutex g_static_mu;
std::vector<StaticWorkspace> g_static;   // indexed by device ordinal

int load_impl(const ttt_config* cfg, const void* const* weights, int32_t n_weights, void* workspace,
              size_t ws_bytes, void* stream, ttt_model** out);

}  // namespace

int ttt_model_load(const ttt_config* cfg, const void* const* weights, int32_t n_weights,
                   void* workspace, size_t ws_bytes, void* stream, ttt_model** out) {
  return load_impl(cfg, weights, n_weights, workspace, ws_bytes, stream, out);
}

int ttt_model_load_static(const ttt_config* cfg, const void* const* weights, int32_t n_weights, void* stream,
                          ttt_model** out) {
  if (!out) return fail(TTT_ERR_ARG, "out is NULL");
  *out = nullptr;
  int rc = check_config(cfg);
  if (rc) return rc;
  {
    ttt_model probe;
    init_dims(&probe, *cfg);
    const size_t need = layout(&probe, nullptr);
    if (need > kStaticWorkspaceBytes)
      return fail(TTT_ERR_WORKSPACE, "the configuration needs " + std::to_string(need) +
                                         " bytes of device state; the static workspace holds " +
                                         std::to_string(kStaticWorkspaceBytes));
  }
  int dev = 0;
  HIPCHK(hipGetDevice(&dev));
  std::lock_guard<std::mutex> lk(g_static_mu);
  if ((int)g_static.size() <= dev) g_static.resize(dev + 1);
  StaticWorkspace& sw = g_static[dev];
  if (!sw.ptr) {
    void* p = nullptr;
    HIPCHK(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p || (reinterpret_cast<uintptr_t>(p) & 255)) return fail(TTT_ERR_HIP, "static workspace address");
    sw.ptr = p;
  }
  if (sw.owner) return fail(TTT_ERR_STATE, "the static workspace of this device holds another model");
  rc = load_impl(cfg, weights, n_weights, sw.ptr, kStaticWorkspaceBytes, stream, out);
  if (rc) return rc;
  (*out)->static_dev = dev;
  sw.owner = *out;
  return TTT_OK;
}

namespace {
int load_impl(const ttt_config* cfg, const void* const* weights, int32_t n_weights, void* workspace,
              size_t ws_bytes, void* stream, ttt_model** out) {
  int rc = check_config(cfg);
  if (rc) return rc;
  if (!out) return fail(TTT_ERR_ARG, "out is NULL");
  *out = nullptr;
  const int nm = cfg->mlp == TTT_MLP_SWIGLU ? 3 : 2;
  const int per = 4 + nm;
  if (!weights || n_weights != 2 + cfg->n_layers * per + (cfg->static_mlp ? cfg->n_fast * nm : 0))
    return fail(TTT_ERR_ARG, "n_weights must be 2 + n_layers * (4 + mlp matrices) "
                             "(+ n_fast * mlp matrices with static_mlp)");
  for (int i = 0; i < n_weights; ++i)
    if (!weights[i]) return fail(TTT_ERR_ARG, "a weight pointer is NULL");
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255))
    return fail(TTT_ERR_WORKSPACE, "workspace must be non-NULL and 256-byte aligned");
  ttt_model* m = new ttt_model();
  init_dims(m, *cfg);
  const size_t need = layout(m, workspace);
  if (ws_bytes < need) {
    delete m;
    return fail(TTT_ERR_WORKSPACE, "workspace too small: need " + std::to_string(need) + " bytes");
  }
  {
    hipError_t e1 = hipStreamCreateWithFlags(&m->sa, hipStreamNonBlocking);
    if (e1 == hipSuccess) e1 = hipStreamCreateWithFlags(&m->sc, hipStreamNonBlocking);
    if (e1 == hipSuccess) e1 = hipStreamCreateWithFlags(&m->sk, hipStreamNonBlocking);
    if (e1 == hipSuccess) e1 = hipStreamCreateWithFlags(&m->sb, hipStreamNonBlocking);
    m->evT1.assign(m->q, nullptr);
    m->evT2.assign(m->q, nullptr);
    m->evR1.assign(m->q, nullptr);
    m->evR2.assign(m->q, nullptr);
    std::vector<hipEvent_t*> evs = {&m->ev0, &m->evA[0], &m->evA[1], &m->evB[0], &m->evB[1], &m->evC,
                                    &m->evK0, &m->evK1, &m->evOut};
    for (int j = 0; j < m->q; ++j) {
      evs.push_back(&m->evT1[j]); evs.push_back(&m->evT2[j]);
      evs.push_back(&m->evR1[j]); evs.push_back(&m->evR2[j]);
    }
    for (auto* e : evs)
      if (e1 == hipSuccess) e1 = hipEventCreateWithFlags(e, hipEventDisableTiming);
    if (e1 != hipSuccess) {
      ttt_model_free(m);
      return fail(TTT_ERR_HIP, std::string("stream/event creation: ") + hipGetErrorString(e1));
    }
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int d = m->d, F = m->F, V = m->V;
  const bool bf = m->bf;
  // E [V][d] stays as is; U canonical [d][V] -> [V][d]
  convert_weight(weights[0], V, d, false, -1, m->E, bf, s);
  convert_weight(weights[n_weights - 1], d, V, true, -1, m->U, bf, s);
  auto load_mlp = [&](const void* const* w, void* up, void* dn) {
    if (cfg->mlp == TTT_MLP_SWIGLU) {
      convert_weight(w[0], d, F, true, 0, up, bf, s);
      convert_weight(w[1], d, F, true, 1, up, bf, s);
      convert_weight(w[2], F, d, true, -1, dn, bf, s);
    } else {
      convert_weight(w[0], d, F, true, -1, up, bf, s);
      convert_weight(w[1], F, d, true, -1, dn, bf, s);
    }
  };
  const void* const* w = weights + 1;
  for (int l = 0; l < m->L; ++l, w += per) {
    Layer& ly = m->layers[l];
    char* qkv = static_cast<char*>(ly.wqkv);
    for (int p = 0; p < 3; ++p)   // Wq, Wk, Wv [d][d] -> rows p*d.. of [3d][d]
      convert_weight(w[p], d, d, true, -1, qkv + (size_t)p * d * d * m->es, bf, s);
    convert_weight(w[3], d, d, true, -1, ly.wo, bf, s);
    load_mlp(w + 4, ly.wup, ly.wdn);
    if (ly.swup) {   // the frozen second MLP follows the layer's own matrices
      w += nm;
      load_mlp(w + 4, ly.swup, ly.swdn);
      transpose(ly.swup, m->F2, d, d, ly.swupT, m->F2, m->F2, bf, s);
      transpose(ly.swdn, d, F, F, ly.swdnT, d, d, bf, s);
    }
  }
  // transposed copies read by the input-gradient products
  transpose(m->U, V, d, d, m->UT, V, V, bf, s);
  for (int l = m->f0 + 1; l < m->L; ++l) {
    Layer& ly = m->layers[l];
    transpose(ly.wqkv, 3 * d, d, d, ly.wqkvT, 3 * d, 3 * d, bf, s);
    transpose(ly.wo, d, d, d, ly.woT, d, d, bf, s);
  }
  // RoPE frequencies theta_i = base^(-2i/hd), float64 on the host
  std::vector<double> th(m->hd / 2);
  for (int i = 0; i < m->hd / 2; ++i) th[i] = std::pow((double)cfg->rope_base, -2.0 * i / m->hd);
  hipError_t e = hipMemcpyAsync(m->theta, th.data(), th.size() * 8, hipMemcpyHostToDevice, s);
  if (e != hipSuccess) { ttt_model_free(m); return fail(TTT_ERR_HIP, hipGetErrorString(e)); }
  float nan = NAN;
  e = hipMemcpyAsync(m->nanv, &nan, 4, hipMemcpyHostToDevice, s);
  if (e != hipSuccess) { ttt_model_free(m); return fail(TTT_ERR_HIP, hipGetErrorString(e)); }
  rc = reset_state(m, s);
  if (!rc) {
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) rc = fail(TTT_ERR_HIP, hipGetErrorString(e));
  }
  if (rc) { ttt_model_free(m); return rc; }
  *out = m;
  return TTT_OK;
}
}  // namespace

int ttt_prefill(ttt_model* m, const int32_t* tokens, int64_t T, int32_t chunk, float lr,
                int32_t steps, float* chunk_losses, void* stream) {
  int rc = prefill_check(m, tokens, T, chunk, lr, steps, chunk_losses);
  if (rc) return rc;
  PrefillRun r;
  r.m = m; r.tokens = tokens; r.T = T; r.chunk = chunk; r.lr = lr; r.steps = steps;
  r.losses = chunk_losses; r.s = static_cast<hipStream_t>(stream);
  rc = prefill_begin(r);
  while (!rc && r.b < r.nblocks) rc = prefill_next(r);
  if (rc) {
    drain(m);
    return rc;
  }
  return prefill_finish(r, r.s);
}

int ttt_prefill_many(ttt_model* const* models, int32_t n, const int32_t* const* tokens, int64_t T,
                     int32_t chunk, float lr, int32_t steps, float* const* chunk_losses, void* stream) {
  if (!models || !tokens || !chunk_losses || n < 1) return fail(TTT_ERR_ARG, "NULL argument or n < 1");
  for (int i = 0; i < n; ++i) {
    for (int j = 0; j < i; ++j)
      if (models[i] == models[j]) return fail(TTT_ERR_ARG, "a model handle appears twice");
    const int rc = prefill_check(models[i], tokens[i], T, chunk, lr, steps, chunk_losses[i]);
    if (rc) return rc;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  // every context's chain runs on its own stream (its phase A, updates and
  // dK/dV on theirs), enqueued chunk by chunk in turn, so the contexts'
  // kernels fill the GPU together; the caller's stream joins them at the end
  HIPCHK(hipEventRecord(models[0]->evOut, s));
  std::vector<PrefillRun> runs(n);
  for (int i = 0; i < n; ++i) {
    HIPCHK(hipStreamWaitEvent(models[i]->sb, models[0]->evOut, 0));
    PrefillRun& r = runs[i];
    r.m = models[i]; r.tokens = tokens[i]; r.T = T; r.chunk = chunk; r.lr = lr; r.steps = steps;
    r.losses = chunk_losses[i]; r.s = models[i]->sb;
  }
  auto fail_all = [&](int rc) {
    for (int i = 0; i < n; ++i) drain(models[i]);
    return rc;
  };
  for (int i = 0; i < n; ++i) {
    const int rc = prefill_begin(runs[i]);
    if (rc) return fail_all(rc);
  }
  for (bool more = true; more;) {
    more = false;
    for (int i = 0; i < n; ++i) {
      if (runs[i].b >= runs[i].nblocks) continue;
      const int rc = prefill_next(runs[i]);
      if (rc) return fail_all(rc);
      more = more || runs[i].b < runs[i].nblocks;
    }
  }
  for (int i = 0; i < n; ++i) {
    HIPCHK(hipEventRecord(models[i]->evOut, models[i]->sb));
    HIPCHK(hipStreamWaitEvent(s, models[i]->evOut, 0));
  }
  int first = TTT_OK;
  for (int i = 0; i < n; ++i) {
    const int rc = prefill_finish(runs[i], s);
    if (rc && !first) first = rc;
  }
  return first;
}

int ttt_forward(ttt_model* m, const int32_t* tokens, int64_t T, int32_t chunk, float* chunk_losses,
                void* stream) {
  if (!m || !tokens || !chunk_losses) return fail(TTT_ERR_ARG, "NULL argument");
  if (T < 2) return fail(TTT_ERR_ARG, "T must be >= 2");
  if (chunk < 1 || chunk > m->Cmax) return fail(TTT_ERR_ARG, "chunk must be in [1, max_chunk]");
  hipStream_t s = static_cast<hipStream_t>(stream);
  int rc = reset_state(m, s);
  if (rc) return rc;
  m->lr = 0.f;
  m->steps = 1;
  m->chunk = chunk;
  const int64_t blk = std::max<int64_t>(chunk, (m->MA / chunk) * (int64_t)chunk);
  for (int64_t B0 = 0; B0 < T; B0 += blk) {
    rc = forward_block(m, tokens, T, B0, (int)std::min<int64_t>(blk, T - B0), chunk, chunk_losses, s);
    if (rc) return rc;
  }
  rc = sync_and_check(m, s);
  if (rc) return rc;
  m->pos = T;
  m->dchunk0 = T;
  m->prefilled = true;
  m->no_update = true;
  return TTT_OK;
}

namespace {
int export_fast(ttt_model* m, int32_t fast_idx, int32_t mat, float* dst, int64_t n, bool delta_only,
                void* stream) {
  if (!m || !dst) return fail(TTT_ERR_ARG, "NULL argument");
  if (fast_idx < 0 || fast_idx >= m->q) return fail(TTT_ERR_ARG, "fast_idx out of range");
  const bool sw = m->c.mlp == TTT_MLP_SWIGLU;
  const int nmat = sw ? 3 : 2;
  if (mat < 0 || mat >= nmat) return fail(TTT_ERR_ARG, "mat out of range");
  const int d = m->d, F = m->F;
  if (n != (int64_t)d * F) return fail(TTT_ERR_ARG, "n must equal d_model * d_ff");
  hipStream_t s = static_cast<hipStream_t>(stream);
  FastLayer& f = m->fast[fast_idx];
  Layer& ly = m->layers[m->f0 + fast_idx];
  if (mat == nmat - 1) export_weight(delta_only ? nullptr : ly.wdn, f.m_dn, d, F, 0, 0, dst, m->bf, s);  // [F][d]
  else export_weight(delta_only ? nullptr : ly.wup, f.m_up, F, d, sw ? 1 : 0, mat, dst, m->bf, s);       // [d][F]
  return TTT_OK;
}
}  // namespace

int ttt_fast_weight(ttt_model* m, int32_t fast_idx, int32_t mat, float* dst, int64_t n,
                    void* stream) {
  return export_fast(m, fast_idx, mat, dst, n, false, stream);
}

int ttt_fast_weight_delta(ttt_model* m, int32_t fast_idx, int32_t mat, float* dst, int64_t n,
                          void* stream) {
  return export_fast(m, fast_idx, mat, dst, n, true, stream);
}

int ttt_decode_step(ttt_model* m, int32_t* next_token, float* logits_out, float* update_loss,
                    void* stream) {
  if (!m || !next_token) return fail(TTT_ERR_ARG, "NULL argument");
  if (!m->prefilled) return fail(TTT_ERR_STATE, "decode needs a prefill first");
  hipStream_t s = static_cast<hipStream_t>(stream);
  copy_i32(m->cur_tok, next_token, s);   // the token this call emits (and reads)
  if (!m->dec_exec) {
    // Capture one token's launches once (on the library's own stream: the
    // caller's may be the legacy default stream, which cannot be captured);
    // every launch reads the position from the device-side state.
    HIPCHK(hipStreamSynchronize(m->sa));
    HIPCHK(hipStreamBeginCapture(m->sa, hipStreamCaptureModeThreadLocal));
    decode_body(m, m->sa);
    hipGraph_t g = nullptr;
    HIPCHK(hipStreamEndCapture(m->sa, &g));
    const hipError_t e = hipGraphInstantiate(&m->dec_exec, g, nullptr, nullptr, 0);
    (void)hipGraphDestroy(g);
    if (e != hipSuccess) {
      m->dec_exec = nullptr;
      return fail(TTT_ERR_HIP, std::string("decode graph: ") + hipGetErrorString(e));
    }
  }
  HIPCHK(hipGraphLaunch(m->dec_exec, s));
  if (logits_out) copy_f32(m->logits, logits_out, m->V, s);
  m->pos += 1;
  bool updated = false;
  if (m->pos - m->dchunk0 == m->chunk && m->no_update) {
    // after ttt_forward: the chunk bookkeeping restarts, no update is made
    m->dchunk0 = m->pos;
    dec_set(m->dstate, m->pos, 0, s);
  } else if (m->pos - m->dchunk0 == m->chunk) {
    // the decode chunk is complete: its targets are known, make the update
    const int n = m->chunk;
    for (int st = 0; st < m->steps; ++st) {
      int rc = chunk_step(m, m->dchunk0, n, m->hA, m->hist + 1, n, m->lr,
                          update_loss ? update_loss : m->dtmp, s);
      if (rc) return rc;
    }
    m->dchunk0 = m->pos;
    dec_set(m->dstate, m->pos, 0, s);
    updated = true;
  }
  if (update_loss && !updated) copy_f32(m->nanv, update_loss, 1, s);
  return TTT_OK;
}

int ttt_reset(ttt_model* m, void* stream) {
  if (!m) return fail(TTT_ERR_ARG, "NULL model");
  return reset_state(m, static_cast<hipStream_t>(stream));
}

void ttt_model_free(ttt_model* m) {
  if (!m) return;
  if (m->sa) (void)hipStreamSynchronize(m->sa);
  if (m->dec_exec) (void)hipGraphExecDestroy(m->dec_exec);
  for (auto& t : m->tm)
    for (auto e : t.ev) (void)hipEventDestroy(e);
  if (m->sc) (void)hipStreamSynchronize(m->sc);
  if (m->sk) (void)hipStreamSynchronize(m->sk);
  if (m->sb) (void)hipStreamSynchronize(m->sb);
  std::vector<hipEvent_t> evs = {m->ev0, m->evA[0], m->evA[1], m->evB[0], m->evB[1], m->evC,
                                 m->evK0, m->evK1, m->evOut};
  for (auto* v : {&m->evT1, &m->evT2, &m->evR1, &m->evR2}) evs.insert(evs.end(), v->begin(), v->end());
  for (auto e : evs)
    if (e) (void)hipEventDestroy(e);
  if (m->sa) (void)hipStreamDestroy(m->sa);
  if (m->sc) (void)hipStreamDestroy(m->sc);
  if (m->sk) (void)hipStreamDestroy(m->sk);
  if (m->sb) (void)hipStreamDestroy(m->sb);
  if (m->static_dev >= 0) {   // the device's static workspace is free again
    std::lock_guard<std::mutex> lk(g_static_mu);
    if (g_static[m->static_dev].owner == m) g_static[m->static_dev].owner = nullptr;
  }
  delete m;
}

const char* ttt_status_str(int st) {
  switch (st) {
    case TTT_OK: return "ok";
    case TTT_ERR_ARG: return "invalid argument";
    case TTT_ERR_CONFIG: return "unsupported configuration";
    case TTT_ERR_HIP: return "HIP runtime error";
    case TTT_ERR_TOKEN: return "token id out of range";
    case TTT_ERR_NONFINITE: return "non-finite loss";
    case TTT_ERR_STATE: return "call out of order";
    case TTT_ERR_WORKSPACE: return "workspace missing or too small";
    default: return "unknown status";
  }
}

const char* ttt_last_error(void) { return g_err.c_str(); }

int ttt_timing_enable(ttt_model* m, int32_t cls, int32_t on) {
  if (!m || cls < 0 || cls >= NCLS - 1) return fail(TTT_ERR_ARG, "bad timing class");
  Timing& t = m->tm[cls];
  t.on = on != 0;
  t.used = 0;
  t.launches = 0;
  t.flops = 0;
  return TTT_OK;
}

int ttt_timing_read(ttt_model* m, int32_t cls, double* total_ms, int64_t* launches, double* flops) {
  if (!m || cls < 0 || cls >= NCLS - 1 || !total_ms) return fail(TTT_ERR_ARG, "bad timing read");
  Timing& t = m->tm[cls];
  double tot = 0;
  for (size_t i = 0; i + 1 < t.used; i += 2) {
    HIPCHK(hipEventSynchronize(t.ev[i + 1]));
    float ms = 0.f;
    HIPCHK(hipEventElapsedTime(&ms, t.ev[i], t.ev[i + 1]));
    tot += ms;
  }
  *total_ms = tot;
  if (launches) *launches = t.launches;
  if (flops) *flops = t.flops;
  return TTT_OK;
}

int ttt_diag_gemm(int32_t dtype, int32_t a_kc, int32_t b_kc, int32_t M, int32_t N, int32_t K,
                  const void* A, int64_t lda, const void* B, int64_t ldb, float* C, int64_t ldc,
                  void* stream) {
  if (!A || !B || !C || M < 0 || N < 0 || K < 0) return fail(TTT_ERR_ARG, "bad GEMM arguments");
  if (dtype != TTT_BF16 && dtype != TTT_FP32) return fail(TTT_ERR_ARG, "bad dtype");
  const int vec = dtype == TTT_BF16 ? 8 : 4;
  if (lda % vec || ldb % vec || (!a_kc && M % vec) || (!b_kc && N % vec) || ((a_kc || b_kc) && K % vec))
    return fail(TTT_ERR_ARG, "strides / vector dims must be multiples of 16 bytes");
  if (N % 4 || ldc % 4 || ldc < N)
    return fail(TTT_ERR_ARG, "N and ldc must be multiples of 4 with ldc >= N (4-wide output groups)");
  GemmParams p;
  p.A = A; p.lda = lda; p.B = B; p.ldb = ldb; p.M = M; p.N = N; p.K = K; p.C = C; p.ldc = ldc;
  int epi = EPI_STORE;
  if (!a_kc && !b_kc) { epi = EPI_SGD; p.alpha = -1.f; }
  else if (!a_kc) return fail(TTT_ERR_ARG, "layout (0,1) is not used by the inner loop");
  const int rg = gemm(p, dtype == TTT_BF16, a_kc != 0, b_kc != 0, epi, true, static_cast<hipStream_t>(stream));
  if (rg == GEMM_TOO_LARGE) return fail(TTT_ERR_ARG, "a GEMM operand spans more than 2^31 - 1 bytes");
  if (rg) return fail(TTT_ERR_ARG, "GEMM variant not built");
  return TTT_OK;
}

int ttt_diag_sgd(int32_t dtype, int32_t M, int32_t N, int32_t K, const void* A, int64_t lda, const void* B,
                 int64_t ldb, float lr, float* master, void* copy, const void* w0, void* cur_t, void* stream) {
  if (!A || !B || !master || !w0 || !cur_t || M <= 0 || N <= 0 || K <= 0)
    return fail(TTT_ERR_ARG, "bad SGD arguments");
  if (dtype != TTT_BF16 && dtype != TTT_FP32) return fail(TTT_ERR_ARG, "bad dtype");
  if (dtype == TTT_BF16 && !copy) return fail(TTT_ERR_ARG, "bf16 needs the copy output");
  const int vec = dtype == TTT_BF16 ? 8 : 4;
  if (lda % vec || ldb % vec || K % vec || lda < K || ldb < K)
    return fail(TTT_ERR_ARG, "K and the row strides must be multiples of 16 bytes, strides >= K");
  if (M % 4 || N % 4) return fail(TTT_ERR_ARG, "M and N must be multiples of 4");
  if (!std::isfinite(lr)) return fail(TTT_ERR_ARG, "lr must be finite");
  GemmParams p;
  p.A = A; p.lda = lda; p.B = B; p.ldb = ldb; p.M = M; p.N = N; p.K = K;
  p.C = master; p.ldc = N; p.alpha = lr;
  p.C2 = dtype == TTT_BF16 ? copy : nullptr; p.ldc2 = N;
  p.C3 = cur_t; p.ldc3 = M; p.W0 = w0;
  const int rg = gemm(p, dtype == TTT_BF16, true, true, EPI_SGD, true, static_cast<hipStream_t>(stream));
  if (rg == GEMM_TOO_LARGE) return fail(TTT_ERR_ARG, "a GEMM operand spans more than 2^31 - 1 bytes");
  if (rg) return fail(TTT_ERR_ARG, "GEMM variant not built");
  return TTT_OK;
}

int ttt_diag_chunk_logits(ttt_model* m, float* dst, int64_t n, void* stream) {
  if (!m || !dst) return fail(TTT_ERR_ARG, "NULL argument");
  if (m->logit_rows <= 0) return fail(TTT_ERR_STATE, "no chunk has been read with updates yet");
  if (n != m->logit_rows * m->V) return fail(TTT_ERR_ARG, "n must equal rows * vocab of the last chunk");
  HIPCHK(hipMemcpyAsync(dst, m->zce, (size_t)n * 4, hipMemcpyDeviceToDevice, static_cast<hipStream_t>(stream)));
  return TTT_OK;
}

int64_t ttt_diag_chunk_logit_rows(const ttt_model* m) { return m ? m->logit_rows : 0; }

int ttt_diag_gemm_core(int32_t mode) { return gemm_core(mode); }

int ttt_diag_mfma_peak(float* scratch, int64_t* clk, double* tflops, double* clock_mhz, void* stream) {
  if (!scratch || !clk || !tflops || !clock_mhz) return fail(TTT_ERR_ARG, "NULL argument");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int blocks = 2048, iters = 4096;
  mfma_peak(blocks, 64, scratch, clk, s);   // warm-up (clocks ramp)
  hipEvent_t e0 = nullptr, e1 = nullptr;
  HIPCHK(hipEventCreate(&e0));
  HIPCHK(hipEventCreate(&e1));
  HIPCHK(hipEventRecord(e0, s));
  mfma_peak(blocks, iters, scratch, clk, s);
  HIPCHK(hipEventRecord(e1, s));
  HIPCHK(hipEventSynchronize(e1));
  float ms = 0.f;
  const hipError_t e = hipEventElapsedTime(&ms, e0, e1);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (e != hipSuccess) return fail(TTT_ERR_HIP, hipGetErrorString(e));
  int64_t t[2] = {0, 0};
  HIPCHK(hipMemcpy(t, clk, sizeof(t), hipMemcpyDeviceToHost));
  const double flops = (double)blocks * 4 * iters * 8 * 2.0 * 32 * 32 * 16;
  *tflops = flops / (ms * 1e-3) / 1e12;
  *clock_mhz = t[1] > 0 ? (double)t[0] / (double)t[1] * 100.0 : 0.0;
  return TTT_OK;
}

}  // extern "C"
