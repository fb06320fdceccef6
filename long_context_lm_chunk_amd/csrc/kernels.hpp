// Host-side launchers of the HIP kernels (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ttt {

enum Epi { EPI_STORE = 0, EPI_RESID, EPI_GELU, EPI_SWIGLU, EPI_SGD, EPI_CESTAT, EPI_CEGRAD, EPI_ACTBWD };

struct GemmParams {
  const void* A = nullptr; int64_t lda = 0;  // k-contiguous [M][K] or m-contiguous [K][M]
  const void* B = nullptr; int64_t ldb = 0;  // k-contiguous [N][K] or n-contiguous [K][N]
  const void* B2 = nullptr;                  // optional second B (same layout): C = A.(B + B2)
  int M = 0, N = 0, K = 0;
  void* C = nullptr; int64_t ldc = 0;        // primary output (GELU/SWIGLU: pre-activations, optional)
  const float* R = nullptr; int64_t ldr = 0; // residual input (RESID)
  void* C2 = nullptr; int64_t ldc2 = 0;      // act (GELU/SWIGLU), delta copy (SGD)
  void* C3 = nullptr; const void* W0 = nullptr;  // SGD: C3 = round(W0 + delta), written
  int64_t ldc3 = 0;                              // transposed: C3[col][row], row stride ldc3
  float alpha = 0.f;                         // SGD: lr; CEGRAD: 1/n_targets
  // cross-entropy epilogues
  const int* tgt = nullptr; int n_tgt = 0;
  float* part_max = nullptr; float* part_sum = nullptr; int64_t ldpart = 0;
  float* tgt_logit = nullptr; const float* lse = nullptr;
  // ACTBWD: the product is d(act); Z holds the saved pre-activations (row
  // stride ldz; SwiGLU gate/up interleaved in blocks of 16, else GELU) and C
  // receives d(pre-activation) in Z's layout (row stride ldc)
  const void* Z = nullptr; int64_t ldz = 0; int act_swiglu = 0;
  // split-K scratch (optional; STORE/RESID launches with too few tiles):
  // split_ws holds up to split_cap floats
  float* split_ws = nullptr; int64_t split_cap = 0;
  // STORE or RESID: when set, a split launch leaves its nz partial slabs in
  // split_ws ([nz][M][N], summed by the consumer in slab order, then the
  // residual added, then rounded to C's type) instead of reducing them into
  // C; *split_defer receives nz (1 when the launch was not split and C holds
  // the result)
  int* split_defer = nullptr;
  // STORE, when the launch is split and reduced into C: the reduction pass
  // also writes rd_D[h][row] = sum over the rd_hd columns of head h of
  // rd_o (bf16 or fp32 as C, row stride ldc) times C as stored (the
  // attention backward's rowsum(O * dO)), and sets *rd_done = 1; it is left
  // alone otherwise (rd_hd / 4 a power of two <= 64 dividing N / 4)
  const void* rd_o = nullptr; float* rd_D = nullptr; int rd_hd = 0; int* rd_done = nullptr;
};

// Returns 0, or -1 for an epilogue/layout combination that is not built.
// core selection for the bf16 k-contiguous products (diagnostics): returns
// the previous mode
enum { GEMM_CORE_AUTO = 0, GEMM_CORE_BIG = 1, GEMM_CORE_SMALL = 2 };
int gemm_core(int mode);
// matrix-core throughput probe: blocks x 256 threads, each wave iters x 8
// bf16 32x32x16 products; out [blocks*256] floats, clk[2] = shader-clock and
// 100 MHz real-time ticks of one wave's loop
void mfma_peak(int blocks, int iters, float* out, int64_t* clk, hipStream_t s);
// Returns 0, -1 for a variant that is not built, or GEMM_TOO_LARGE when an
// operand spans more than 2^31 - 1 bytes (nothing is launched then).
constexpr int GEMM_TOO_LARGE = -2;
constexpr int64_t GEMM_MAX_OPERAND_BYTES = 0x7fffffff;
int gemm(const GemmParams& p, bool bf16_operands, bool a_kc, bool b_kc, int epi, bool out_f32,
         hipStream_t s);

// ---- elementwise (elementwise.hip); T is bf16 when bf16 != 0, else float
// dst[c][r] = src[r][c] (r < rows, c < cols); rows..rows_pad-1 written as 0;
// with perm16 the columns of dst are permuted by kperm (rows_pad % 16 == 0)
void transpose(const void* src, int rows, int cols, int64_t ld_src, void* dst, int64_t ld_dst,
               int rows_pad, bool bf16, hipStream_t s, bool perm16 = false);
void embed(const int32_t* tok, int n, const void* E, int d, int V, bool bf16, float* out, int* err,
           hipStream_t s);
void layernorm_fwd(const float* x, int64_t ldx, int n, int d, float eps, void* y, int64_t ldy,
                   float* mean, float* rstd, bool bf16, hipStream_t s);
// x_out = R + (sum of the nsl fp32 K-split slabs [nsl][n][d] of a product,
// in slab order), then the LayerNorm of x_out as layernorm_fwd
void layernorm_fwd_resid(const float* slabs, int nsl, const float* R, float* x_out, int n, int d, float eps,
                         void* y, int64_t ldy, float* mean, float* rstd, bool bf16, hipStream_t s);
// acc += LN_backward(dy) ; optionally acc_lo = low-precision copy of the new acc.
// dy may be nslab partial slabs (row r of slab z at dy + z*slab_stride +
// r*d), summed in slab order.
void layernorm_bwd_acc(const float* dy, const float* x, const float* mean, const float* rstd, int n,
                       int d, float* acc, void* acc_lo, bool bf16, hipStream_t s, int nslab = 1,
                       int64_t slab_stride = 0);
// acc_lo = low-precision copy of acc
void cast_rows(const float* src, void* dst, int64_t n, bool bf16, hipStream_t s);
// cs[t][i] = (cos, sin) of (pos0 + t) * theta[i], angle in float64, t < n, i < half
void rope_table(int64_t pos0, int n, int half, const double* theta, float2* cs, hipStream_t s);
// q (rotated) -> q_out [n][H*hd]; k (rotated), v -> rings at slot
// (pos0 + t) mod cap; v and (when ktring is set) k also to the transposed
// rings [H*hd][cap], column kperm(slot); cs from rope_table(pos0, n, hd/2).
// hd <= 128, hd % 16 == 0, cap % 16 == 0
// (slabs, nsl > 1: the QKV product was left as nsl fp32 K-split slabs
// [nsl][n][3*H*hd], read instead of qkv)
void qkv_rope(const void* qkv, int n, int H, int hd, int64_t pos0, const float2* cs, void* q_out,
              void* kring, void* vring, void* vtring, void* ktring, int64_t cap, bool bf16, hipStream_t s,
              const float* slabs = nullptr, int nsl = 1);
// the rotation's transpose applied to dQ (parts bit 0) and dK (bit 1) inside
// dqkv [n][3*H*hd]
void rope_bwd(void* dqkv, int n, int H, int hd, const float2* cs, bool bf16, hipStream_t s, int parts = 3);
void convert_weight(const void* src, int rows, int cols, bool transpose, int interleave16_half,
                    void* dst, bool bf16, hipStream_t s);
// dst (canonical [in][out] fp32) = W0 + delta (delta alone when w0 is null), from the
// internal [out][in] layout
void export_weight(const void* w0, const float* delta, int out_dim, int in_dim, int interleave_half,
                   int which, float* dst, bool bf16, hipStream_t s);
void widen(const void* src, float* dst, int64_t n, bool bf16, hipStream_t s);
void copy_cast_from_f32(const float* src, void* dst, int64_t n, bool bf16, hipStream_t s);
void fill_f32(float* p, int64_t n, float v, hipStream_t s);
void ce_finish(const float* part_max, const float* part_sum, int nparts, int64_t ldpart,
               const float* tgt_logit, int n_rows, int n_tgt, float* lse, float* loss_out,
               int* err, hipStream_t s);
void attn_rowdot(const void* o, const void* dout, int n, int H, int hd, float* D, bool bf16,
                 hipStream_t s);
// g = (exp(z - lse) - onehot(tgt)) * alpha on rows < n_tgt, 0 on the other
// rows < n_rows; z fp32 logits [n_rows][ldz], g [n_rows][ldg], V % 4 == 0
void ce_grad(const float* z, int64_t ldz, const float* lse, const int* tgt, int n_rows, int n_tgt,
             int V, float alpha, void* g, int64_t ldg, bool bf16, hipStream_t s);

// ---- attention (attention.hip)
struct AttnParams {
  const void* q = nullptr;   // [n][H*hd], row stride ldq
  int64_t ldq = 0;
  const void* kring = nullptr; const void* vring = nullptr;  // [cap][H*hd]
  // [H*hd][cap] transposed copies, columns permuted by kperm (written by qkv_rope)
  const void* vtring = nullptr;                               // V (forward)
  const void* ktring = nullptr;                               // K (dQ)
  int64_t cap = 0;
  int n = 0, H = 0, hd = 0, window = 0;
  int64_t pos0 = 0;          // absolute position of query row 0
  void* o = nullptr; int64_t ldo = 0;
  float* lse = nullptr;      // [H][n] natural-log LSE (may be null)
  // backward
  const void* dout = nullptr; int64_t lddo = 0;
  const float* D = nullptr;  // [H][n] rowsum(dO*O)
  void* dq = nullptr; void* dk = nullptr; void* dv = nullptr; int64_t ldg = 0;
  int64_t kmin = 0;          // smallest key position that receives dK/dV (chunk start)
  // Q and dO transposed, [H*hd][ldtr], columns permuted by kperm and zero
  // up to a multiple of 64 (optional: the staged dK/dV kernel reads them)
  const void* qtr = nullptr; const void* gtr = nullptr; int64_t ldtr = 0;
  // key-range split scratch (optional): part [max_split][n][H*hd] fp32,
  // part_ml [max_split][H][n][2]
  float* part = nullptr; float* part_ml = nullptr; int max_split = 1;
  // optional: (cos, sin) of each row's rotary angles, [n][hd/2] (rope_table):
  // the backward then applies the rotation's transpose to dQ and dK where its
  // kernels can (swa_bwd's return value says which)
  const float2* rope_cs = nullptr;
};
void swa_fwd(const AttnParams& p, bool bf16, hipStream_t s);
// dQ on s, dK/dV on s_kv (the two are independent; the caller orders s_kv
// after the inputs and joins it before using dK/dV; s_kv may equal s).
// Returns which gradients left rotated back when rope_cs is set: bit 0 dQ
// (the staged dQ kernel or the split combine), bit 1 dK (the staged dK/dV
// kernel); the caller applies rope_bwd to the others.
int swa_bwd(const AttnParams& p, bool bf16, hipStream_t s, hipStream_t s_kv);
// whether swa_bwd takes its staged dK/dV path (which reads qtr / gtr) for
// this head size and type
bool swa_bwd_reads_transposes(int hd, bool bf16);

// ---- decode (decode.hip)
// Every decode kernel reads the position from dstate = {pos, ci} on the
// device, so one token's launches can be captured once and replayed.
// Matrix-vector products (W [N][K] k-contiguous, W2 of the same shape added
// when non-null); LN(x) is the LayerNorm of the fp32 row x, fused:
//   dgemv_ln_rope: LN(x) -> Wqkv; RoPE on q and k, q to `q`, k and v to the
//                  rings at slot pos % cap (the transposed copies are made
//                  by the chunk forward of the update that reads them)
//   dgemv_ln_act:  LN(x) -> up-projection; act = silu(gate) * up (SwiGLU,
//                  rows interleaved in blocks of 16) or gelu, storage type
//   dgemv_vec:     y = (W + W2) x (+ resid; y may alias resid); optionally y
//                  also to rows[dstate[1]][.] and per-block argmax pairs
//   dgemv_ln_head: logits = U LN(x), per-block argmax pairs in amax
// amax holds 2 floats per block; dgemv_blocks(units) gives the block count.
void dgemv_ln_rope(const void* Wqkv, int d, const float* x, float eps, int H, int hd,
                   const double* theta, const int64_t* dstate, void* q, void* kring, void* vring,
                   int64_t cap, bool bf16, hipStream_t s);
void dgemv_ln_act(const void* Wup, const void* Wup2, int F, int d, const float* x, float eps,
                  bool swiglu, void* act, bool bf16, hipStream_t s);
void dgemv_vec(const void* W, const void* W2, int N, int K, const void* x, float* y,
               const float* resid, float* rows, const int64_t* dstate, float* amax, bool bf16,
               hipStream_t s);
void dgemv_ln_head(const void* U, int V, int d, const float* x, float eps, float* logits,
                   float* amax, bool bf16, hipStream_t s);
int dgemv_blocks(int units);
// split-key attention of the new query over the window + per-head combine
void swa_decode(const void* q, const void* kring, const void* vring, int64_t cap, int H, int hd,
                int window, const int64_t* dstate, void* o, float* ws, bool bf16, hipStream_t s);
// x = E[*cur] (fp32) and hist[ci] = *cur
void dec_embed(const int32_t* cur, const int64_t* dstate, int32_t* hist, const void* E, int d, int V,
               float* x, int* err, bool bf16, hipStream_t s);
// greedy token from per-block argmax pairs; hist[ci + 1] = token when hist is
// set; dstate advanced by one position when `advance`
void argmax_part(const float* part, int nb, int32_t* out_tok, int32_t* hist, int64_t* dstate,
                 bool advance, hipStream_t s);
void dec_set(int64_t* dstate, int64_t pos, int64_t ci, hipStream_t s);
void copy_i32(const int32_t* a, int32_t* b, hipStream_t s);
void copy_f32(const float* a, float* b, int n, hipStream_t s);

}  // namespace ttt
