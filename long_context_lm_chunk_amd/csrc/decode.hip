// One-token decode kernels: HBM-bound matrix-vector products, split-key
// sliding-window attention over the ring, and the greedy argmax.  Per-token
// cost is bounded by the window and the weights, not by the context length
// (the constant-latency claim of the paper summary, "Key claims", and of the
// NVIDIA blog's Figure 1 caption).
#include "common.hpp"
#include "kernels.hpp"

namespace ttt {
namespace {

// y[n] = sum_k W[n][k] x[k] (+ resid[n]); W [N][K] k-contiguous.
// One wave per output row, 16-byte loads along k.
template <typename T, typename X>
__global__ __launch_bounds__(256) void gemv_k(const T* __restrict__ W, const T* __restrict__ W2,
                                              int N, int K, const X* __restrict__ x,
                                              float* __restrict__ y, const float* __restrict__ resid) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= N) return;
  constexpr int V = Vec16<T>::N;
  float s = 0.f;
  // 4 independent 16-byte loads in flight per lane per step
  for (int pass = 0; pass < (W2 ? 2 : 1); ++pass) {   // fast weights: W0 + delta, one fp32 sum
    const T* w = (pass ? W2 : W) + (int64_t)row * K;
    int k = lane * V;
    for (; k + 3 * 64 * V < K; k += 4 * 64 * V) {
      U128 wv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) wv[u] = ld128(w + k + u * 64 * V);
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < V; ++e) s += to_f32(elem<T>(wv[u], e)) * to_f32(x[k + u * 64 * V + e]);
    }
    for (; k < K; k += 64 * V) {
      const U128 wv = ld128(w + k);
#pragma unroll
      for (int e = 0; e < V; ++e) s += to_f32(elem<T>(wv, e)) * to_f32(x[k + e]);
    }
  }
  s = wave_sum(s);
  if (lane == 0) y[row] = s + (resid ? resid[row] : 0.f);
}

template <typename T>
__global__ void swiglu_vec_k(const float* __restrict__ z, int F, T* __restrict__ act) {
  const int f = blockIdx.x * blockDim.x + threadIdx.x;
  if (f >= F) return;
  const int c = (f / 16) * 32 + (f % 16);
  const float g = z[c], u = z[c + 16];
  act[f] = from_f32<T>(g / (1.f + __expf(-g)) * u);
}
template <typename T>
__global__ void gelu_vec_k(const float* __restrict__ z, int F, T* __restrict__ act) {
  const int f = blockIdx.x * blockDim.x + threadIdx.x;
  if (f >= F) return;
  const float v = z[f];
  act[f] = from_f32<T>(0.5f * v * (1.f + erff(v * 0.70710678118654752f)));
}

constexpr int DK = 256;   // keys per split

// Partial attention of one query over keys [lo + split*DK, ...) of head h,
// bandwidth-bound.  Lanes work in groups of G = hd/8 (16 for hd = 128):
// a group covers one key's row with one 16-byte load per lane, so a wave
// reads 64/G whole rows per instruction.  ws per (h, split): m, l, o[hd].
template <typename T, int hd>
__global__ __launch_bounds__(256) void swa_decode_part_k(const T* __restrict__ q,
                                                         const T* __restrict__ kr,
                                                         const T* __restrict__ vr, int64_t cap,
                                                         int H, int window,
                                                         const int64_t* __restrict__ dstate,
                                                         float* __restrict__ ws, int nsplit) {
  // position of this token from the device-side decode state (so a captured
  // graph replays unchanged); splits past the window write empty partials
  const int64_t pos = dstate[0];
  int64_t lo = pos - window + 1;
  if (lo < 0) lo = 0;
  constexpr int V = Vec16<T>::N;
  __shared__ float ps[DK];
  __shared__ float red[8];
  __shared__ float oacc[4][128];
  const int h = blockIdx.y, sp = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int d = H * hd;
  // lanes per key row: hd/V rounded up to a power of two
  constexpr int G = (hd / V <= 1) ? 1 : (hd / V <= 2) ? 2 : (hd / V <= 4) ? 4 : (hd / V <= 8) ? 8
                  : (hd / V <= 16) ? 16 : (hd / V <= 32) ? 32 : 64;
  constexpr int KPW = 64 / G;              // keys per wave instruction
  const int gi = lane % G, kg = lane / G;  // lane's vector within the row, key slot
  const bool live = gi * V < hd;           // hd = 96: 12 of every 16 lanes carry data
  const int64_t kbase = lo + (int64_t)sp * DK;
  float qv[V];
  {
    const U128 qq = live ? ld128(q + h * hd + gi * V) : zero128();
#pragma unroll
    for (int e = 0; e < V; ++e) qv[e] = to_f32(elem<T>(qq, e));
  }
  const float scale = 1.f / sqrtf((float)hd);
  // scores: each wave takes keys wave*64 .. wave*64+63 of the split
#pragma unroll
  for (int k0 = wave * 64; k0 < wave * 64 + 64; k0 += KPW) {
    const int kk = k0 + kg;
    const int64_t kp = kbase + kk;
    float sacc = 0.f;
    if (live && kp <= pos) {
      const U128 kv = ld128(kr + (kp % cap) * d + h * hd + gi * V);
#pragma unroll
      for (int e = 0; e < V; ++e) sacc += to_f32(elem<T>(kv, e)) * qv[e];
    }
#pragma unroll
    for (int o = 1; o < G; o <<= 1) sacc += __shfl_xor(sacc, o, 64);
    if (gi == 0 && kk < DK) ps[kk] = (kp <= pos) ? sacc * scale : -INFINITY;
  }
  __syncthreads();
  // max and sum over the split's 256 scores
  float mx = wave_max(ps[tid]);
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  const float m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float e = (ps[tid] == -INFINITY) ? 0.f : __expf(ps[tid] - m);
  float sm = wave_sum(e);
  __syncthreads();
  ps[tid] = e;
  if (lane == 0) red[4 + wave] = sm;
  __syncthreads();
  const float l = red[4] + red[5] + red[6] + red[7];
  // o = sum_k p_k v_k: same lane grouping, each lane accumulates its V
  // elements over the keys of its slot, then slots and waves are summed
  float o[V];
#pragma unroll
  for (int e2 = 0; e2 < V; ++e2) o[e2] = 0.f;
#pragma unroll
  for (int k0 = wave * 64; k0 < wave * 64 + 64; k0 += KPW) {
    const int kk = k0 + kg;
    const int64_t kp = kbase + kk;
    if (live && kk < DK && kp <= pos) {
      const float pk = ps[kk];
      const U128 vv = ld128(vr + (kp % cap) * d + h * hd + gi * V);
#pragma unroll
      for (int e2 = 0; e2 < V; ++e2) o[e2] += pk * to_f32(elem<T>(vv, e2));
    }
  }
  // reduce over key slots (lanes gi + G*kg) within the wave
  for (int off = G; off < 64; off <<= 1)
#pragma unroll
    for (int e2 = 0; e2 < V; ++e2) o[e2] += __shfl_xor(o[e2], off, 64);
  if (kg == 0 && live) {
#pragma unroll
    for (int e2 = 0; e2 < V; ++e2) oacc[wave][gi * V + e2] = o[e2];
  }
  __syncthreads();
  float* w = ws + ((int64_t)h * nsplit + sp) * (2 + hd);
  if (tid < hd) w[2 + tid] = oacc[0][tid] + oacc[1][tid] + oacc[2][tid] + oacc[3][tid];
  if (tid == 0) { w[0] = m; w[1] = l; }
}

template <typename T>
__global__ void swa_decode_combine_k(const float* __restrict__ ws, int nsplit, int H, int hd,
                                     T* __restrict__ o) {
  // (every split writes its partial, possibly empty: m = -inf, l = 0)
  __shared__ float fs[64];
  __shared__ float Ls;
  const int h = blockIdx.x, j = threadIdx.x;
  if (j < 64) {
    float mv = -INFINITY;
    if (j < nsplit) mv = ws[((int64_t)h * nsplit + j) * (2 + hd)];
    const float M = wave_max(mv);
    const float f = (j < nsplit && mv != -INFINITY) ? __expf(mv - M) : 0.f;
    fs[j] = f;
    const float lv = (j < nsplit) ? ws[((int64_t)h * nsplit + j) * (2 + hd) + 1] * f : 0.f;
    const float L = wave_sum(lv);
    if (j == 0) Ls = L;
  }
  __syncthreads();
  if (j >= hd) return;
  float acc = 0.f;
  for (int sp = 0; sp < nsplit; ++sp) acc += ws[((int64_t)h * nsplit + sp) * (2 + hd) + 2 + j] * fs[sp];
  o[h * hd + j] = from_f32<T>(acc / Ls);
}

// Decode bookkeeping kernels (graph-safe: no memcpy/memset nodes).
// dstate = {pos, ci}: position being read, index within the decode chunk.
__global__ void dec_begin_k(const int32_t* __restrict__ cur, const int64_t* __restrict__ dstate,
                            int32_t* __restrict__ hist) {
  if (threadIdx.x == 0) hist[dstate[1]] = *cur;
}
__global__ void dec_end_k(int64_t* __restrict__ dstate) {
  if (threadIdx.x == 0) { dstate[0] += 1; dstate[1] += 1; }
}
__global__ void dec_row_k(const float* __restrict__ x, int d, const int64_t* __restrict__ dstate,
                          float* __restrict__ rows) {
  const int64_t ci = dstate[1];
  for (int i = threadIdx.x; i < d; i += blockDim.x) rows[ci * d + i] = x[i];
}
__global__ void dec_set_k(int64_t* __restrict__ dstate, int64_t pos, int64_t ci) {
  if (threadIdx.x == 0) { dstate[0] = pos; dstate[1] = ci; }
}
__global__ void copy_i32_k(const int32_t* __restrict__ a, int32_t* __restrict__ b) {
  if (threadIdx.x == 0) *b = *a;
}
__global__ void copy_f32_k(const float* __restrict__ a, float* __restrict__ b, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) b[i] = a[i];
}

// Greedy choice: largest logit, lowest id on ties.  The chosen id also goes
// to hist[ci + 1] (the target of the position just read).
__global__ void argmax_k(const float* __restrict__ z, int V, int32_t* __restrict__ out,
                         int32_t* __restrict__ hist, const int64_t* __restrict__ dstate) {
  __shared__ float bv[1024];
  __shared__ int bi[1024];
  float best = -INFINITY;
  int idx = 0x7fffffff;
  for (int i = threadIdx.x; i < V; i += blockDim.x) {
    const float v = z[i];
    if (v > best || (v == best && i < idx)) { best = v; idx = i; }
  }
  bv[threadIdx.x] = best;
  bi[threadIdx.x] = idx;
  __syncthreads();
  for (int o = blockDim.x / 2; o > 0; o >>= 1) {
    if (threadIdx.x < o) {
      const float v2 = bv[threadIdx.x + o];
      const int i2 = bi[threadIdx.x + o];
      if (v2 > bv[threadIdx.x] || (v2 == bv[threadIdx.x] && i2 < bi[threadIdx.x])) {
        bv[threadIdx.x] = v2;
        bi[threadIdx.x] = i2;
      }
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const int r = bi[0] == 0x7fffffff ? 0 : bi[0];
    *out = r;
    if (hist) hist[dstate ? dstate[1] + 1 : 0] = r;
  }
}

}  // namespace

void gemv(const void* W, const void* W2, int N, int K, const void* x, bool x_f32, float* y,
          const float* resid, bool bf, hipStream_t s) {
  dim3 grid((N + 3) / 4);
  if (bf) {
    if (x_f32) hipLaunchKernelGGL((gemv_k<bf16, float>), grid, dim3(256), 0, s, (const bf16*)W, (const bf16*)W2, N, K, (const float*)x, y, resid);
    else hipLaunchKernelGGL((gemv_k<bf16, bf16>), grid, dim3(256), 0, s, (const bf16*)W, (const bf16*)W2, N, K, (const bf16*)x, y, resid);
  } else {
    hipLaunchKernelGGL((gemv_k<float, float>), grid, dim3(256), 0, s, (const float*)W, (const float*)W2, N, K, (const float*)x, y, resid);
  }
}

void swiglu_vec(const float* z, int F, void* act, bool bf, hipStream_t s) {
  if (bf) hipLaunchKernelGGL(swiglu_vec_k<bf16>, dim3((F + 255) / 256), dim3(256), 0, s, z, F, (bf16*)act);
  else hipLaunchKernelGGL(swiglu_vec_k<float>, dim3((F + 255) / 256), dim3(256), 0, s, z, F, (float*)act);
}
void gelu_vec(const float* z, int F, void* act, bool bf, hipStream_t s) {
  if (bf) hipLaunchKernelGGL(gelu_vec_k<bf16>, dim3((F + 255) / 256), dim3(256), 0, s, z, F, (bf16*)act);
  else hipLaunchKernelGGL(gelu_vec_k<float>, dim3((F + 255) / 256), dim3(256), 0, s, z, F, (float*)act);
}

template <typename T>
void swa_decode_t(const void* q, const void* kring, const void* vring, int64_t cap, int H, int hd,
                  int window, const int64_t* dstate, void* o, float* ws, hipStream_t s) {
  const int nsplit = (window + DK - 1) / DK;   // covers a full window
  dim3 grid(nsplit, H);
  switch (hd) {
#define CASE(HDV) case HDV: hipLaunchKernelGGL((swa_decode_part_k<T, HDV>), grid, dim3(256), 0, s, \
      (const T*)q, (const T*)kring, (const T*)vring, cap, H, window, dstate, ws, nsplit); break;
    CASE(16) CASE(32) CASE(64) CASE(96) CASE(128)
#undef CASE
    default: return;
  }
  // nsplit <= 64 for windows up to 16384 keys
  hipLaunchKernelGGL(swa_decode_combine_k<T>, dim3(H), dim3(128), 0, s, ws, nsplit, H, hd, (T*)o);
}

void swa_decode(const void* q, const void* kring, const void* vring, int64_t cap, int H, int hd,
                int window, const int64_t* dstate, void* o, float* ws, bool bf, hipStream_t s) {
  if (bf) swa_decode_t<bf16>(q, kring, vring, cap, H, hd, window, dstate, o, ws, s);
  else swa_decode_t<float>(q, kring, vring, cap, H, hd, window, dstate, o, ws, s);
}

void dec_begin(const int32_t* cur, const int64_t* dstate, int32_t* hist, hipStream_t s) {
  hipLaunchKernelGGL(dec_begin_k, dim3(1), dim3(64), 0, s, cur, dstate, hist);
}
void dec_end(int64_t* dstate, hipStream_t s) { hipLaunchKernelGGL(dec_end_k, dim3(1), dim3(64), 0, s, dstate); }
void dec_row(const float* x, int d, const int64_t* dstate, float* rows, hipStream_t s) {
  hipLaunchKernelGGL(dec_row_k, dim3(1), dim3(256), 0, s, x, d, dstate, rows);
}
void dec_set(int64_t* dstate, int64_t pos, int64_t ci, hipStream_t s) {
  hipLaunchKernelGGL(dec_set_k, dim3(1), dim3(64), 0, s, dstate, pos, ci);
}
void copy_i32(const int32_t* a, int32_t* b, hipStream_t s) { hipLaunchKernelGGL(copy_i32_k, dim3(1), dim3(64), 0, s, a, b); }
void copy_f32(const float* a, float* b, int n, hipStream_t s) {
  hipLaunchKernelGGL(copy_f32_k, dim3((n + 255) / 256 > 1024 ? 1024 : (n + 255) / 256), dim3(256), 0, s, a, b, n);
}

void argmax_tok(const float* logits, int V, int32_t* out_tok, int32_t* tok_hist, const int64_t* dstate,
                hipStream_t s) {
  hipLaunchKernelGGL(argmax_k, dim3(1), dim3(1024), 0, s, logits, V, out_tok, tok_hist, dstate);
}

}  // namespace ttt
