/*
 * ttt.h -- C ABI of the MI355X (gfx950) TTT-E2E test-time inner loop.
 *
 * The method (End-to-End Test-Time Training for Long Context): a standard
 * decoder-only Transformer with sliding-window attention reads its context
 * in chunks ("mini-batches", ~1K tokens at the 3B operating point, podcast
 * 6:36) and, for each chunk, runs the forward pass, takes the next-token
 * cross-entropy at the end of the network (NVIDIA blog, "Our method"),
 * back-propagates into the MLP weights of the last quarter of the blocks
 * only (podcast 6:36 and 7:08; forum post TL;DR "Inner Loop") and applies a
 * plain SGD step before the next chunk.  Generation afterwards has constant
 * per-token cost (paper summary "Key claims"; blog Figure 1 caption).
 *
 * Conventions for every call:
 *  - Every function returns TTT_OK (0) or a negative ttt_status; nothing
 *    throws, aborts or exits.  ttt_last_error() gives a message for the
 *    last failure on the calling thread.
 *  - Pointers documented "device" are HIP device memory owned by the
 *    caller; they must stay valid until the stream has executed the call.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls enqueue
 *    work and return; outputs are valid after the stream is synchronised.
 *    Calls that must report a device-detected error (bad token, non-finite
 *    loss) synchronise the stream before returning.
 *  - A model handle is not thread-safe; separate handles are independent.
 *  - The library performs no device allocation of its own: all device
 *    state lives in the caller's workspace (ttt_workspace_bytes).
 */
#ifndef TTT_H
#define TTT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TTT_OK = 0,
  TTT_ERR_ARG = -1,        /* invalid argument (NULL, size out of range, non-finite lr) */
  TTT_ERR_CONFIG = -2,     /* configuration not supported (see ttt_config) */
  TTT_ERR_HIP = -3,        /* a HIP runtime call failed */
  TTT_ERR_TOKEN = -4,      /* a token id outside [0, vocab) was read */
  TTT_ERR_NONFINITE = -5,  /* a chunk loss was not finite */
  TTT_ERR_STATE = -6,      /* call out of order (decode before prefill) */
  TTT_ERR_WORKSPACE = -7   /* workspace missing, misaligned or too small */
} ttt_status;

enum { TTT_MLP_GELU = 0, TTT_MLP_SWIGLU = 1 };
enum { TTT_FP32 = 0, TTT_BF16 = 1 };

/*
 * Model shape and capacity.  Architecture readings (where the pages are
 * silent): pre-LN blocks, LayerNorm without affine parameters (eps ln_eps),
 * final LayerNorm before an untied head, no biases, multi-head attention,
 * rotate-half RoPE on absolute positions (base rope_base, float64 angles),
 * window = number of keys a query sees (itself included).
 *
 * Supported: head_dim in {16, 32, 64, 96, 128}; n_heads * head_dim ==
 * d_model; d_model % 16 == 0; d_ff % 16 == 0; vocab % 8 == 0;
 * d_model, d_ff <= 16384 (bf16) or 8192 (fp32); 1 <= n_fast <= n_layers;
 * 1 <= window <= 4194304 (the K/V rings hold window + prefill_block
 * positions per layer, so memory bounds it in practice); 1 <= max_chunk <= 65536.
 */
typedef struct {
  int32_t n_layers, d_model, n_heads, head_dim, d_ff, vocab, window;
  int32_t n_fast;        /* the last n_fast blocks' MLPs are the fast weights */
  int32_t mlp;           /* TTT_MLP_GELU (exact erf) or TTT_MLP_SWIGLU */
  int32_t dtype;         /* TTT_BF16: bf16 weights/activations, fp32 accumulate,
                            fp32 master of the fast weights; TTT_FP32: check mode */
  float rope_base;       /* 10000 */
  float ln_eps;          /* 1e-5 */
  int32_t max_chunk;     /* largest chunk a prefill call may use */
  int32_t prefill_block; /* tokens per frozen-layer block; 0 = default (8192) */
  int32_t static_mlp;    /* 1: every fast block also has a frozen second MLP (podcast
                            7:08: pre-trained knowledge kept static beside the updated
                            MLP), a pre-LN residual sublayer of the same shape and
                            activation after the fast MLP; 0: none */
} ttt_config;

/* Workspace bytes needed for `cfg` (device memory, 256-byte aligned). */
int ttt_workspace_bytes(const ttt_config* cfg, size_t* bytes);

/*
 * Create a model.  `weights` is a host array of `n_weights` device pointers
 * in canonical order and layout, element type bf16 (TTT_BF16) or float
 * (TTT_FP32):
 *   E [vocab][d_model];
 *   for each layer: Wq, Wk, Wv, Wo [d_model][d_model], then
 *     GELU:   W1 [d_model][d_ff], W2 [d_ff][d_model]
 *     SwiGLU: Wg [d_model][d_ff], Wu [d_model][d_ff], Wd [d_ff][d_model],
 *     and, in each of the last n_fast layers when static_mlp = 1, the
 *     frozen second MLP's matrices in the same order and shapes;
 *   U [d_model][vocab].
 * Every matrix is [in][out] row-major (a layer computes y = x W).  The
 * weights are copied into the workspace (in the library's own layout), so
 * the caller may free them after the stream has executed the call.
 * `workspace` (device, ws_bytes >= ttt_workspace_bytes) is owned by the
 * caller and must outlive the model.  On success *out receives a handle in
 * the reset state.
 */
int ttt_model_load(const ttt_config* cfg, const void* const* weights, int32_t n_weights,
                   void* workspace, size_t ws_bytes, void* stream, struct ttt_model** out);

/*
 * ttt_model_load without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops and
 * harnesses that forbid hipMalloc): the model's device state lives in a
 * static array of the library, 64 MiB on every GPU it runs on (held until
 * the process ends), on the device current at the call.  It allocates no
 * device memory.  Arguments and results otherwise as ttt_model_load.
 * Errors: TTT_ERR_WORKSPACE when ttt_workspace_bytes(cfg) exceeds 64 MiB
 * (the tiny and small configurations fit; the 125M shape does not);
 * TTT_ERR_STATE while another model loaded this way on the same device is
 * alive (one at a time per device; ttt_model_free releases it).  The array
 * keeps the last model's contents; loading clears what must start at zero.
 * Calls on the two models of the same device that overlap in time would
 * race on it, which the ownership check rules out.
 */
int ttt_model_load_static(const ttt_config* cfg, const void* const* weights, int32_t n_weights, void* stream,
                          struct ttt_model** out);

/*
 * The inner loop over a whole context (forum post TL;DR "Inner Loop": the
 * model keeps learning at test time by mini-gradient descent on the context,
 * updating specific MLP layers; podcast 6:36 and 7:08: mini-batches of about
 * 1,000 tokens, only the MLPs of the last quarter of the blocks updated;
 * NVIDIA blog "Our method": the next-token loss taken at the end of the
 * network).  Resets the model (fast weights back
 * to their loaded values, empty K/V rings), then for each chunk k of
 * positions [k*chunk, min((k+1)*chunk, T)) and each of `steps` steps:
 * forward with the current fast weights (attention over the window of
 * earlier positions, whose K/V are kept as computed when read), mean
 * next-token cross-entropy over the chunk's targets (position t predicts
 * tokens[t+1]; the last position has none), gradient into the fast MLP
 * weights only, SGD phi <- phi - lr * g.
 *   tokens       device int32 [T], 2 <= T
 *   chunk        1 <= chunk <= max_chunk
 *   lr           finite
 *   steps        >= 1
 *   chunk_losses device float [ceil(T/chunk) * steps], the loss of each
 *                step before its update (natural log); a chunk with no
 *                target reports 0 and makes no update.
 * Errors: TTT_ERR_TOKEN (a token outside [0, vocab)), TTT_ERR_NONFINITE;
 * both are detected on the device and reported after a stream sync.
 */
int ttt_prefill(struct ttt_model* m, const int32_t* tokens, int64_t T, int32_t chunk, float lr,
                int32_t steps, float* chunk_losses, void* stream);

/*
 * Several independent contexts at once, one model handle each (every
 * context has its own fast weights and K/V rings; the handles may share a
 * configuration and weights or not): the same inner loop as ttt_prefill for
 * every context, with one T, chunk, lr and steps.  Each context's chunk
 * chain runs on a stream of its own handle, and the contexts' chunks are
 * enqueued in turn, so their kernels occupy the GPU together (independent
 * contexts are the data-parallel unit of the method: each keeps its own
 * fast weights).  The caller's stream waits for every context.
 *   models        host array of n distinct handles
 *   tokens        host array of n device int32 [T] pointers
 *   chunk_losses  host array of n device float [ceil(T/chunk) * steps]
 * The result of each context equals that of ttt_prefill on it.  Errors:
 * as ttt_prefill (the first context's error is returned after every
 * context has run); TTT_ERR_ARG for a repeated handle.
 */
int ttt_prefill_many(struct ttt_model* const* models, int32_t n, const int32_t* const* tokens, int64_t T,
                     int32_t chunk, float lr, int32_t steps, float* const* chunk_losses, void* stream);

/*
 * The same context read without test-time training: the static-weight
 * model whose latency the pages set against TTT-E2E (blog Figure 1, right
 * panel; paper abstract: constant latency versus full attention, whose
 * per-token cost grows with the context).  Resets the model, then every
 * block, the fast ones with their loaded MLP weights, reads the positions in
 * batches of whole chunks (prefill_block tokens); no gradient, no update.
 * chunk_losses[k] is the mean next-token cross-entropy of chunk k
 * (positions [k*chunk, min((k+1)*chunk, T))), i.e. what ttt_prefill returns
 * at lr = 0.  With window >= T this is a plain full-attention Transformer.
 *   tokens       device int32 [T], 2 <= T
 *   chunk        1 <= chunk <= max_chunk (only groups the losses)
 *   chunk_losses device float [ceil(T/chunk)]
 * Decode steps may follow; they make no updates.  Errors as ttt_prefill.
 */
int ttt_forward(struct ttt_model* m, const int32_t* tokens, int64_t T, int32_t chunk,
                float* chunk_losses, void* stream);

/*
 * Copy fast-weight matrix `mat` of fast layer `fast_idx` (0 = the first
 * fast layer) as float32 in canonical [in][out] layout into `dst` (device,
 * n floats, n == rows*cols): the MLP weights as updated so far by the inner
 * loop (forum post TL;DR "Inner Loop"; podcast 7:08: only the MLP layers of
 * the last quarter of the blocks change).  mat: GELU 0 = W1, 1 = W2;
 * SwiGLU 0 = Wg, 1 = Wu, 2 = Wd.  Errors: TTT_ERR_ARG for a NULL handle or
 * dst, an index out of range or n != rows*cols (nothing is copied).
 * Asynchronous on `stream`.
 */
int ttt_fast_weight(struct ttt_model* m, int32_t fast_idx, int32_t mat, float* dst, int64_t n,
                    void* stream);

/*
 * The same matrix's change since loading, phi - phi0 (the sum of the SGD
 * steps, forum post TL;DR "Inner Loop"), as float32 in the same layout and
 * with the same arguments and errors.  It is read from the float32 master of
 * the update, so it is exact where the difference of two ttt_fast_weight
 * exports would round at the magnitude of the weights (at lr = 1e-4 the
 * change per chunk is ~1e-8, below a float32 ulp of a weight of ~0.02).
 */
int ttt_fast_weight_delta(struct ttt_model* m, int32_t fast_idx, int32_t mat, float* dst, int64_t n,
                          void* stream);

/*
 * One greedy decode step after ttt_prefill or ttt_forward (or a previous
 * decode step).  Generation after reading the context costs the same per
 * token whatever the context length (paper summary "Key claims": constant
 * inference latency; blog Figure 1, right panel caption): attention reads
 * the window's K/V rings, the fast weights carry the rest of the context.
 * The first call emits argmax of the last prefill position's logits; every
 * call then reads the emitted token at the next position (its K/V join the
 * rings) and prepares the next argmax (lowest id on ties).  When `chunk`
 * decode positions are complete, that chunk makes the same update as a
 * prefill chunk.
 *   next_token  device int32 [1]: the token emitted by this call
 *   logits      device float [vocab] or NULL: logits of the position read
 *               by this call (whose argmax the next call emits)
 *   update_loss device float [1] or NULL: loss of the update made by this
 *               call, NaN when none was made
 */
int ttt_decode_step(struct ttt_model* m, int32_t* next_token, float* logits, float* update_loss,
                    void* stream);

/* Back to the loaded state (fast weights, empty rings, position 0). */
int ttt_reset(struct ttt_model* m, void* stream);

/* Destroy the handle (the caller's workspace is not touched). */
void ttt_model_free(struct ttt_model* m);

/* Message for a status code, and for the last failure on this thread. */
const char* ttt_status_str(int status);
const char* ttt_last_error(void);

/*
 * Kernel timing (measurement aid).  When enabled, every launch of the
 * kernel class `cls` is bracketed by HIP events on its stream:
 *   cls 0 = all matrix-core GEMM launches of the inner loop
 *   cls 1 = sliding-window attention forward
 *   cls 2 = sliding-window attention backward
 *   cls 3 = fused head + cross-entropy (statistics, gradient, input grad)
 *   cls 4 = the weight-gradient GEMMs with the fused SGD update
 *   cls 5 = the MLP up-projection GEMM of the frozen blocks (one kernel)
 * ttt_timing_read synchronises the stream and returns the summed event time
 * (ms), the number of launches and the algorithmic FLOPs of those launches.
 */
int ttt_timing_enable(struct ttt_model* m, int32_t cls, int32_t on);
int ttt_timing_read(struct ttt_model* m, int32_t cls, double* total_ms, int64_t* launches,
                    double* flops);

/*
 * Diagnostic access to the inner loop's matrix-core GEMM kernel, for
 * kernel-level parity tests.  Computes C[M][N] (device float, row stride
 * ldc) = sum_k A[m,k] * B[n,k] with element type bf16 (dtype TTT_BF16) or
 * float (TTT_FP32), fp32 accumulation:
 *   a_kc = 1: A is [M][K] (row stride lda); 0: A is [K][M]
 *   b_kc = 1: B is [N][K] (row stride ldb); 0: B is [K][N]
 * Layouts (a_kc, b_kc) = (1,1), (1,0) overwrite C; (0,0) is the weight-
 * gradient kernel and ADDS the product to C (its SGD epilogue run with
 * lr = -1).  Row strides must be multiples of 8 elements, pointers 16-byte
 * aligned; N and ldc multiples of 4 with ldc >= N (the output is written in
 * groups of 4 columns).  Otherwise TTT_ERR_ARG and nothing is launched.
 */
int ttt_diag_gemm(int32_t dtype, int32_t a_kc, int32_t b_kc, int32_t M, int32_t N, int32_t K,
                  const void* A, int64_t lda, const void* B, int64_t ldb, float* C, int64_t ldc,
                  void* stream);

/*
 * Diagnostic access to the fused weight-gradient + SGD product that updates
 * the fast weights (forum post TL;DR "Inner Loop": a gradient step per
 * mini-batch), the same kernels and epilogue the inner loop launches:
 *   G[m][n]      = sum_k A[m][k] * B[n][k]      A [M][K], B [N][K] (row strides lda, ldb)
 *   master[m][n] -= lr * G[m][n]                float [M][N], read and written
 *   copy[m][n]    = master[m][n] rounded         bf16 [M][N] (TTT_BF16 only; NULL for TTT_FP32)
 *   cur_t[n][m]   = w0[m][n] + master[m][n]      [N][M] (transposed), rounded to the element type
 * A, B, w0, copy and cur_t have the element type of dtype (bf16 or float);
 * master is always float.  All pointers are device memory owned by the
 * caller.  K and the row strides must be multiples of 16 bytes (lda, ldb >=
 * K), M and N multiples of 4, lr finite; otherwise TTT_ERR_ARG and nothing
 * is launched.  The GEMM core is chosen as in the inner loop (see
 * ttt_diag_gemm_core).  Asynchronous on `stream`.
 */
int ttt_diag_sgd(int32_t dtype, int32_t M, int32_t N, int32_t K, const void* A, int64_t lda, const void* B,
                 int64_t ldb, float lr, float* master, void* copy, const void* w0, void* cur_t, void* stream);

/*
 * Diagnostic: the logits (float32, [rows][vocab]) of every position of the
 * last chunk read with updates (by ttt_prefill, or by the update of a
 * completed decode chunk), as the fused head kept them between its
 * statistics and gradient passes.  ttt_diag_chunk_logit_rows gives rows (0
 * before any such chunk).  n must equal rows * vocab (TTT_ERR_ARG); before
 * any chunk TTT_ERR_STATE.  Asynchronous on `stream`.
 */
int ttt_diag_chunk_logits(struct ttt_model* m, float* dst, int64_t n, void* stream);
int64_t ttt_diag_chunk_logit_rows(const struct ttt_model* m);

/*
 * Diagnostic choice of the GEMM core for the bf16 products whose operands
 * are both k-contiguous (forward products, head): mode 0 = the default
 * (the 256x256 core for every epilogue it has, the 128x128 core for the
 * rest), 1 = the 256x256 core wherever it applies (the same today), 2 = the
 * 128x128 core only.  Process-wide; returns the previous mode, or the
 * current one unchanged for any other value.  For parity tests that must
 * reach a core the default would not pick at their sizes.
 */
int ttt_diag_gemm_core(int32_t mode);

/*
 * Diagnostic: the matrix-core throughput this GPU reaches on bf16 32x32x16
 * products fed from registers (no memory traffic), and the shader clock they
 * ran at, for reporting utilisation against a measured peak beside the
 * specified one.  scratch: device float [2048 * 256]; clk: device int64 [2].
 * Synchronises the stream; *tflops and *clock_mhz are host outputs.
 */
int ttt_diag_mfma_peak(float* scratch, int64_t* clk, double* tflops, double* clock_mhz, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TTT_H */
