// One-token decode kernels: HBM-bound matrix-vector products with the
// LayerNorm, activation, RoPE and residual steps fused into them, split-key
// sliding-window attention over the ring, and the greedy argmax.  Per-token cost is bounded by the window and the weights,
// not by the context length (the constant-latency claim of the paper
// summary, "Key claims", and of the NVIDIA blog's Figure 1 caption).
#include "common.hpp"
#include "kernels.hpp"

namespace ttt {
namespace {

// ---------------------------------------------------------------------------
// Matrix-vector products.  W [N][K] is k-contiguous (the library's weight
// layout).  One wave owns one output "unit" (one row, or a pair of rows whose
// results its epilogue combines) and streams its rows with 16-byte loads, up
// to sixteen in flight per lane; the input vector is read straight from
// global memory (it is small and stays in L1/L2), so there is no prologue
// and no barrier.
//
// LayerNorm of the input is fused algebraically: with c = x[0] as a shift
// (against cancellation), mu' = mean(x - c) and rs = 1/sqrt(var(x) + eps),
//   W . LN(x) = rs * (W . (x - c) - mu' * sum_k W[k]),
// and every wave gathers sum(x - c), sum((x - c)^2) and the row sums in the
// same pass as the dot product (the wave covers all of K).
struct DecGemv {
  const void* W; const void* W2;   // W2 (same shape) is added to W when set
  int N, K;
  const void* x; float eps;        // LN: fp32 row to normalise; else storage-type vector
  float* y; const float* resid;    // OUT_F32: y = W x (+ resid); y may alias resid
  float* rows; const int64_t* dstate;   // OUT_F32: y also to rows[dstate[1]][.] when set
  float* amax;                     // OUT_F32: per-block (max, index) pairs when set
  void* act;                       // OUT_SWIGLU / OUT_GELU: activation vector, storage type
  int H, hd; const double* theta;  // OUT_ROPE
  void* q; void* kr; void* vr; int64_t cap;
};

enum { OUT_F32 = 0, OUT_SWIGLU = 1, OUT_GELU = 2, OUT_ROPE = 3 };

template <int OUT> struct Units;
// one row
template <> struct Units<OUT_F32> {
  static constexpr int R = 1;
  DEVI static int count(const DecGemv& a) { return a.N; }
  DEVI static void rows(const DecGemv&, int u, int* r) { r[0] = u; }
};
template <> struct Units<OUT_GELU> : Units<OUT_F32> {};
// SwiGLU: gate and up rows of activation f (interleaved in blocks of 16)
template <> struct Units<OUT_SWIGLU> {
  static constexpr int R = 2;
  DEVI static int count(const DecGemv& a) { return a.N / 2; }
  DEVI static void rows(const DecGemv&, int u, int* r) {
    r[0] = (u / 16) * 32 + (u % 16);
    r[1] = r[0] + 16;
  }
};
// RoPE: rows i and i + hd/2 of one head in the q, k or v part
template <> struct Units<OUT_ROPE> {
  static constexpr int R = 2;
  DEVI static int count(const DecGemv& a) { return a.N / 2; }
  DEVI static void rows(const DecGemv& a, int u, int* r) {
    const int d = a.H * a.hd, half = a.hd >> 1, per = d >> 1;
    const int part = u / per, idx = u - part * per;
    const int h = idx / half, i = idx - h * half;
    r[0] = part * d + h * a.hd + i;
    r[1] = r[0] + half;
  }
};

// V consecutive input elements as floats (x of storage type T, or fp32)
template <typename T, bool XF32> DEVI void load_x(const void* x, int k, float* xv) {
  constexpr int V = Vec16<T>::N;
  if constexpr (XF32) {
#pragma unroll
    for (int h = 0; h < V; h += 4) {
      const float4 f = *reinterpret_cast<const float4*>(static_cast<const float*>(x) + k + h);
      xv[h] = f.x; xv[h + 1] = f.y; xv[h + 2] = f.z; xv[h + 3] = f.w;
    }
  } else {
    const U128 u = ld128(static_cast<const T*>(x) + k);
#pragma unroll
    for (int e = 0; e < V; ++e) xv[e] = to_f32(elem<T>(u, e));
  }
}

// UN = k-steps (16-byte loads per row) in flight per lane; KS = waves that
// split one unit's k range (steps interleaved), reduced through LDS.
template <typename T, bool LN, int OUT, bool DUAL, int UN, int KS>
__global__ __launch_bounds__(256) void dgemv_k(DecGemv a) {
  using U = Units<OUT>;
  constexpr int R = U::R;
  constexpr int P = DUAL ? 2 : 1;
  constexpr int V = Vec16<T>::N;
  constexpr int UPB = 4 / KS;                // units per block
  constexpr int NP = 2 * R + 2;              // partials per wave
  __shared__ float part[4][NP];
  __shared__ float bestv[UPB];
  __shared__ int besti[UPB];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ks = wave % KS, ul = wave / KS;
  const int K = a.K;
  const int u = blockIdx.x * UPB + ul;
  const bool active = u < U::count(a);
  float acc[R], rsum[R];
#pragma unroll
  for (int j = 0; j < R; ++j) { acc[j] = 0.f; rsum[j] = 0.f; }
  float sx = 0.f, sxx = 0.f;
  float c = 0.f;
  if constexpr (LN) c = static_cast<const float*>(a.x)[0];
  if (active) {
    int r[2] = {0, 0};
    U::rows(a, u, r);
    const T* wr[R][P];
#pragma unroll
    for (int j = 0; j < R; ++j) {
      wr[j][0] = static_cast<const T*>(a.W) + (int64_t)r[j] * K;
      if constexpr (DUAL) wr[j][1] = static_cast<const T*>(a.W2) + (int64_t)r[j] * K;
    }
    // k-step t of this wave covers elements ((t * KS + ks) * 64 + lane) * V
    constexpr int SK = KS * 64 * V;          // elements between a wave's steps
    int k = (ks * 64 + lane) * V;
    for (; k + (UN - 1) * SK < K; k += UN * SK) {
      U128 w[UN][R][P];
#pragma unroll
      for (int s2 = 0; s2 < UN; ++s2)
#pragma unroll
        for (int j = 0; j < R; ++j)
#pragma unroll
          for (int p = 0; p < P; ++p) w[s2][j][p] = ld128(wr[j][p] + k + s2 * SK);
#pragma unroll
      for (int s2 = 0; s2 < UN; ++s2) {
        float xv[V];
        load_x<T, LN>(a.x, k + s2 * SK, xv);
#pragma unroll
        for (int e = 0; e < V; ++e) {
          const float xe = xv[e] - c;
          if constexpr (LN) { sx += xe; sxx += xe * xe; }
#pragma unroll
          for (int j = 0; j < R; ++j)
#pragma unroll
            for (int p = 0; p < P; ++p) {
              const float we = to_f32(elem<T>(w[s2][j][p], e));
              acc[j] += we * xe;
              if constexpr (LN) rsum[j] += we;
            }
        }
      }
    }
    for (; k < K; k += SK) {
      U128 w[R][P];
#pragma unroll
      for (int j = 0; j < R; ++j)
#pragma unroll
        for (int p = 0; p < P; ++p) w[j][p] = ld128(wr[j][p] + k);
      float xv[V];
      load_x<T, LN>(a.x, k, xv);
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const float xe = xv[e] - c;
        if constexpr (LN) { sx += xe; sxx += xe * xe; }
#pragma unroll
        for (int j = 0; j < R; ++j)
#pragma unroll
          for (int p = 0; p < P; ++p) {
            const float we = to_f32(elem<T>(w[j][p], e));
            acc[j] += we * xe;
            if constexpr (LN) rsum[j] += we;
          }
      }
    }
#pragma unroll
    for (int j = 0; j < R; ++j) {
      acc[j] = wave_sum(acc[j]);
      if constexpr (LN) rsum[j] = wave_sum(rsum[j]);
    }
    if constexpr (LN) {
      sx = wave_sum(sx);
      sxx = wave_sum(sxx);
    }
  }
  if constexpr (KS > 1) {
    if (lane == 0) {
#pragma unroll
      for (int j = 0; j < R; ++j) { part[wave][j] = acc[j]; part[wave][R + j] = rsum[j]; }
      part[wave][2 * R] = sx;
      part[wave][2 * R + 1] = sxx;
    }
    __syncthreads();
    if (ks == 0 && lane == 0) {
      for (int t = 1; t < KS; ++t) {
#pragma unroll
        for (int j = 0; j < R; ++j) { acc[j] += part[wave + t][j]; rsum[j] += part[wave + t][R + j]; }
        sx += part[wave + t][2 * R];
        sxx += part[wave + t][2 * R + 1];
      }
    }
  }
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  if (active && ks == 0 && lane == 0) {
    if constexpr (LN) {
      const float mu = sx / K;                              // mean of x - c
      const float var = fmaxf(sxx / K - mu * mu, 0.f);
      const float rs = rsqrtf(var + a.eps);
#pragma unroll
      for (int j = 0; j < R; ++j) acc[j] = rs * (acc[j] - mu * rsum[j]);
    }
    if constexpr (OUT == OUT_F32) {
      const float v = acc[0] + (a.resid ? a.resid[u] : 0.f);
      a.y[u] = v;
      if (a.rows) a.rows[a.dstate[1] * a.N + u] = v;
      bv = v;
      bi = u;
    } else if constexpr (OUT == OUT_GELU) {
      const float v = acc[0];
      static_cast<T*>(a.act)[u] = from_f32<T>(0.5f * v * (1.f + erff(v * 0.70710678118654752f)));
    } else if constexpr (OUT == OUT_SWIGLU) {
      const float g = acc[0], up = acc[1];
      static_cast<T*>(a.act)[u] = from_f32<T>(g / (1.f + __expf(-g)) * up);
    } else {
      const int d = a.H * a.hd, half = a.hd >> 1, per = d >> 1;
      const int part_ = u / per, idx = u - part_ * per;
      const int h = idx / half, i = idx - h * half;
      const int j1 = h * a.hd + i, j2 = j1 + half;
      const int64_t pos = a.dstate[0];
      const int64_t slot = pos % a.cap;
      float v1 = acc[0], v2 = acc[1];
      if (part_ < 2) {
        float cs, sn;
        rope_cs(pos, a.theta, i, cs, sn);
        const float r1 = v1 * cs - v2 * sn, r2 = v2 * cs + v1 * sn;
        v1 = r1;
        v2 = r2;
      }
      if (part_ == 0) {
        static_cast<T*>(a.q)[j1] = from_f32<T>(v1);
        static_cast<T*>(a.q)[j2] = from_f32<T>(v2);
      } else if (part_ == 1) {
        static_cast<T*>(a.kr)[slot * d + j1] = from_f32<T>(v1);
        static_cast<T*>(a.kr)[slot * d + j2] = from_f32<T>(v2);
      } else {
        static_cast<T*>(a.vr)[slot * d + j1] = from_f32<T>(v1);
        static_cast<T*>(a.vr)[slot * d + j2] = from_f32<T>(v2);
      }
    }
  }
  if constexpr (OUT == OUT_F32) {
    if (a.amax) {   // uniform over the block: per-block greedy candidate
      if (ks == 0 && lane == 0) { bestv[ul] = bv; besti[ul] = bi; }
      __syncthreads();
      if (threadIdx.x == 0) {
        float b = bestv[0];
        int ib = besti[0];
        for (int w2 = 1; w2 < UPB; ++w2)
          if (bestv[w2] > b || (bestv[w2] == b && besti[w2] < ib)) { b = bestv[w2]; ib = besti[w2]; }
        a.amax[2 * blockIdx.x] = b;
        a.amax[2 * blockIdx.x + 1] = __int_as_float(ib);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Split-key attention of the one new query over the window.

constexpr int DK = 256;   // keys per split

// Partial attention of one query over keys [lo + split*DK, ...) of head h,
// bandwidth-bound.  Lanes work in groups of G = hd/8 (16 for hd = 128): a
// group covers one key's row with one 16-byte load per lane, so a wave reads
// 64/G whole rows per instruction.  Each wave takes 64 keys on its own: a
// lane's group reduces the score of each of its keys by shuffles, so every
// lane already holds the scores of exactly the keys whose V elements it
// accumulates; the wave's softmax statistics come from wave reductions and
// the four waves meet once, in LDS, at the end.  The V loads are issued as
// soon as the K rows are consumed, so they overlap the softmax.
// ws per (h, split): m, l, o[hd].
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
  __shared__ float wml[4][2];
  __shared__ float wo[4][hd];
  const int h = blockIdx.y, sp = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int d = H * hd;
  // lanes per key row: hd/V rounded up to a power of two
  constexpr int G = (hd / V <= 1) ? 1 : (hd / V <= 2) ? 2 : (hd / V <= 4) ? 4 : (hd / V <= 8) ? 8
                  : (hd / V <= 16) ? 16 : (hd / V <= 32) ? 32 : 64;
  constexpr int KPW = 64 / G;              // keys per wave instruction
  constexpr int NI = 64 / KPW;             // instructions per wave (64 keys)
  const int gi = lane % G, kg = lane / G;  // lane's vector within the row, key slot
  const bool live = gi * V < hd;           // hd = 96: 12 of every 16 lanes carry data
  const int64_t kbase = lo + (int64_t)sp * DK;
  // ring slot of the split's first key; every key read is < window <= cap
  // past it, so one conditional subtraction replaces a 64-bit modulo
  const int64_t s0 = kbase % cap;
  float qv[V];
  {
    const U128 qq = live ? ld128(q + h * hd + gi * V) : zero128();
    const float scale = 1.f / sqrtf((float)hd);
#pragma unroll
    for (int e = 0; e < V; ++e) qv[e] = to_f32(elem<T>(qq, e)) * scale;
  }
  int64_t off[NI];
  bool ok[NI];
  U128 kv[NI];
#pragma unroll
  for (int it = 0; it < NI; ++it) {
    const int kk = wave * 64 + it * KPW + kg;
    int64_t slot = s0 + kk;
    if (slot >= cap) slot -= cap;
    off[it] = slot * d + h * hd + gi * V;
    ok[it] = kbase + kk <= pos;
    kv[it] = (live && ok[it]) ? ld128(kr + off[it]) : zero128();
  }
  float sc[NI];
  float mx = -INFINITY;
#pragma unroll
  for (int it = 0; it < NI; ++it) {
    float a = 0.f;
#pragma unroll
    for (int e = 0; e < V; ++e) a += to_f32(elem<T>(kv[it], e)) * qv[e];
#pragma unroll
    for (int o = 1; o < G; o <<= 1) a += __shfl_xor(a, o, 64);
    sc[it] = ok[it] ? a : -INFINITY;
    mx = fmaxf(mx, sc[it]);
  }
  U128 vv[NI];
#pragma unroll
  for (int it = 0; it < NI; ++it) vv[it] = (live && ok[it]) ? ld128(vr + off[it]) : zero128();
  const float m = wave_max(mx);
  float l = 0.f;
#pragma unroll
  for (int it = 0; it < NI; ++it) {
    sc[it] = (sc[it] == -INFINITY) ? 0.f : __expf(sc[it] - m);
    l += sc[it];
  }
  // every lane of a group holds the same scores: count each key once
  l = wave_sum(gi == 0 ? l : 0.f);
  float o[V];
#pragma unroll
  for (int e = 0; e < V; ++e) o[e] = 0.f;
#pragma unroll
  for (int it = 0; it < NI; ++it)
#pragma unroll
    for (int e = 0; e < V; ++e) o[e] += sc[it] * to_f32(elem<T>(vv[it], e));
  // reduce over key slots (lanes gi + G*kg) within the wave
  for (int offs = G; offs < 64; offs <<= 1)
#pragma unroll
    for (int e = 0; e < V; ++e) o[e] += __shfl_xor(o[e], offs, 64);
  if (kg == 0 && live) {
#pragma unroll
    for (int e = 0; e < V; ++e) wo[wave][gi * V + e] = o[e];
  }
  if (lane == 0) { wml[wave][0] = m; wml[wave][1] = l; }
  __syncthreads();
  // merge the four waves (a wave with no key in range has m = -inf, l = 0)
  const float M = fmaxf(fmaxf(wml[0][0], wml[1][0]), fmaxf(wml[2][0], wml[3][0]));
  float f[4];
#pragma unroll
  for (int w2 = 0; w2 < 4; ++w2) f[w2] = (wml[w2][0] == -INFINITY) ? 0.f : __expf(wml[w2][0] - M);
  float* w = ws + ((int64_t)h * nsplit + sp) * (2 + hd);
  if (tid < hd) w[2 + tid] = wo[0][tid] * f[0] + wo[1][tid] * f[1] + wo[2][tid] * f[2] + wo[3][tid] * f[3];
  if (tid == 0) {
    w[0] = M;
    w[1] = wml[0][1] * f[0] + wml[1][1] * f[1] + wml[2][1] * f[2] + wml[3][1] * f[3];
  }
}

// ---------------------------------------------------------------------------
// Decode bookkeeping kernels (graph-safe: no memcpy/memset nodes).
// dstate = {pos, ci}: position being read, index within the decode chunk.

// x = E[cur] as fp32, and the token read at this position into hist[ci].
template <typename T>
__global__ void dec_embed_k(const int32_t* __restrict__ cur, const int64_t* __restrict__ dstate,
                            int32_t* __restrict__ hist, const T* __restrict__ E, int d, int V,
                            float* __restrict__ x, int* __restrict__ err) {
  int id = *cur;
  if (threadIdx.x == 0) hist[dstate[1]] = id;
  if (id < 0 || id >= V) {
    if (threadIdx.x == 0) atomicOr(err, 1);
    id = 0;
  }
  for (int i = threadIdx.x; i < d; i += blockDim.x) x[i] = to_f32(E[(int64_t)id * d + i]);
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

// Greedy choice over the per-block (max, index) pairs of the head product:
// largest logit, lowest id on ties (a NaN logit is never chosen).  The id
// goes to *out and, when hist is set, to hist[ci + 1] (the target of the
// position just read); with advance set the decode state moves on by one.
DEVI void better(float& bv, int& bi, float v, int i) {
  if (v > bv || (v == bv && i < bi)) { bv = v; bi = i; }
}
__global__ __launch_bounds__(1024) void argmax_part_k(const float2* __restrict__ part, int nb,
                                                      int32_t* __restrict__ out,
                                                      int32_t* __restrict__ hist,
                                                      int64_t* __restrict__ dstate, int advance) {
  __shared__ float wv[16];
  __shared__ int wi[16];
  float best = -INFINITY;
  int idx = 0x7fffffff;
  // eight independent loads per thread per round (8192 pairs in one round)
  for (int b0 = threadIdx.x; b0 < nb; b0 += 8 * 1024) {
    float2 p[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int b = b0 + u * 1024;
      p[u] = b < nb ? part[b] : make_float2(-INFINITY, __int_as_float(0x7fffffff));
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) better(best, idx, p[u].x, __float_as_int(p[u].y));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float v2 = __shfl_xor(best, o, 64);
    const int i2 = __shfl_xor(idx, o, 64);
    better(best, idx, v2, i2);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) { wv[wave] = best; wi[wave] = idx; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 16; ++w) better(best, idx, wv[w], wi[w]);
    const int r = idx == 0x7fffffff ? 0 : idx;
    *out = r;
    if (hist) hist[dstate[1] + 1] = r;
    if (advance) { dstate[0] += 1; dstate[1] += 1; }
  }
}

// Combine the splits of head h = blockIdx.x for 16 output columns starting
// at 16 * blockIdx.y: o = sum_s e^(m_s - M) o_s / sum_s e^(m_s - M) l_s,
// M = max_s m_s (a split with no key wrote m = -inf, l = 0).  Thread t takes
// column t % 16 of the splits t / 16, t / 16 + 16, ...; the 16 groups meet in
// LDS in a fixed order.  Any number of splits, so long windows (full
// attention) spread their combine over H * hd / 16 workgroups.
template <typename T>
__global__ __launch_bounds__(256) void swa_decode_combine_k(const float* __restrict__ ws, int nsplit,
                                                            int hd, T* __restrict__ o) {
  __shared__ float sacc[16][17];
  __shared__ float sl[16];
  __shared__ float wm[4];
  const int h = blockIdx.x, col = blockIdx.y * 16 + (threadIdx.x & 15), g = threadIdx.x >> 4;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float* wh = ws + (int64_t)h * nsplit * (2 + hd);
  float mv = -INFINITY;
  for (int sp = g; sp < nsplit; sp += 16) mv = fmaxf(mv, wh[(int64_t)sp * (2 + hd)]);
  mv = wave_max(mv);
  if (lane == 0) wm[wave] = mv;
  __syncthreads();
  const float M = fmaxf(fmaxf(wm[0], wm[1]), fmaxf(wm[2], wm[3]));
  const bool live = col < hd;
  float acc = 0.f, lp = 0.f;
  for (int sp = g; sp < nsplit; sp += 16) {
    const float* w = wh + (int64_t)sp * (2 + hd);
    const float m = w[0];
    const float f = (m == -INFINITY) ? 0.f : __expf(m - M);
    lp += w[1] * f;
    if (live) acc += w[2 + col] * f;
  }
  sacc[g][threadIdx.x & 15] = acc;
  if ((threadIdx.x & 15) == 0) sl[g] = lp;
  __syncthreads();
  if (threadIdx.x < 16 && live) {
    float A = 0.f, L = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) { A += sacc[i][threadIdx.x]; L += sl[i]; }
    o[h * hd + col] = from_f32<T>(A / L);
  }
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
  hipLaunchKernelGGL(swa_decode_combine_k<T>, dim3(H, (hd + 15) / 16), dim3(256), 0, s, ws, nsplit, hd, (T*)o);
}

template <typename T, bool LN, int OUT, bool DUAL, int UN = 4, int KS = 1>
void dgemv_launch(const DecGemv& a, hipStream_t s) {
  const int units = (OUT == OUT_SWIGLU || OUT == OUT_ROPE) ? a.N / 2 : a.N;
  const int upb = 4 / KS;
  hipLaunchKernelGGL((dgemv_k<T, LN, OUT, DUAL, UN, KS>), dim3((units + upb - 1) / upb), dim3(256), 0, s, a);
}

// Launch shapes from a sweep on MI355X (bf16, 3B shapes): two loads in flight
// with the k range split over the block's four waves is best or within a
// few per cent for the LayerNorm and down products; the 32000-row head
// prefers one row per wave, the 3072-square output product UN = 2, KS = 1,
// and the LayerNorm + QKV + RoPE product (4608 row pairs) two row pairs per
// block with the k range split over two waves (half as many workgroups:
// about one round of resident blocks instead of two and a quarter; decode
// 0.5-1% faster than with the four-wave split).
enum { SHAPE_SPLIT = 0, SHAPE_ROWS = 1, SHAPE_ROWS2 = 2, SHAPE_SPLIT2 = 3 };
template <typename T, bool LN, int OUT, bool DUAL>
void dgemv_shaped(const DecGemv& a, int shape, hipStream_t s) {
  if (shape == SHAPE_ROWS) dgemv_launch<T, LN, OUT, DUAL, 1, 1>(a, s);
  else if (shape == SHAPE_ROWS2) dgemv_launch<T, LN, OUT, DUAL, 2, 1>(a, s);
  else if (shape == SHAPE_SPLIT2) dgemv_launch<T, LN, OUT, DUAL, 2, 2>(a, s);
  else dgemv_launch<T, LN, OUT, DUAL, 2, 4>(a, s);
}

template <typename T>
void dgemv_t(const DecGemv& a, bool ln, int out, int shape, hipStream_t s) {
  const bool dual = a.W2 != nullptr;
  if (ln) {
    switch (out) {
      case OUT_ROPE: dgemv_shaped<T, true, OUT_ROPE, false>(a, shape, s); break;
      case OUT_SWIGLU: dual ? dgemv_shaped<T, true, OUT_SWIGLU, true>(a, shape, s)
                            : dgemv_shaped<T, true, OUT_SWIGLU, false>(a, shape, s); break;
      case OUT_GELU: dual ? dgemv_shaped<T, true, OUT_GELU, true>(a, shape, s)
                          : dgemv_shaped<T, true, OUT_GELU, false>(a, shape, s); break;
      default: dgemv_shaped<T, true, OUT_F32, false>(a, shape, s); break;
    }
  } else {
    dual ? dgemv_shaped<T, false, OUT_F32, true>(a, shape, s)
         : dgemv_shaped<T, false, OUT_F32, false>(a, shape, s);
  }
}

}  // namespace

void swa_decode(const void* q, const void* kring, const void* vring, int64_t cap, int H, int hd,
                int window, const int64_t* dstate, void* o, float* ws, bool bf, hipStream_t s) {
  if (bf) swa_decode_t<bf16>(q, kring, vring, cap, H, hd, window, dstate, o, ws, s);
  else swa_decode_t<float>(q, kring, vring, cap, H, hd, window, dstate, o, ws, s);
}

void dgemv_ln_rope(const void* Wqkv, int d, const float* x, float eps, int H, int hd,
                   const double* theta, const int64_t* dstate, void* q, void* kring, void* vring,
                   int64_t cap, bool bf, hipStream_t s) {
  DecGemv a{};
  a.W = Wqkv; a.N = 3 * d; a.K = d; a.x = x; a.eps = eps;
  a.H = H; a.hd = hd; a.theta = theta; a.dstate = dstate;
  a.q = q; a.kr = kring; a.vr = vring; a.cap = cap;
  if (bf) dgemv_t<bf16>(a, true, OUT_ROPE, SHAPE_SPLIT2, s);
  else dgemv_t<float>(a, true, OUT_ROPE, SHAPE_SPLIT, s);
}

void dgemv_ln_act(const void* Wup, const void* Wup2, int F, int d, const float* x, float eps,
                  bool swiglu, void* act, bool bf, hipStream_t s) {
  DecGemv a{};
  a.W = Wup; a.W2 = Wup2; a.N = swiglu ? 2 * F : F; a.K = d; a.x = x; a.eps = eps; a.act = act;
  const int out = swiglu ? OUT_SWIGLU : OUT_GELU;
  if (bf) dgemv_t<bf16>(a, true, out, SHAPE_SPLIT, s);
  else dgemv_t<float>(a, true, out, SHAPE_SPLIT, s);
}

void dgemv_vec(const void* W, const void* W2, int N, int K, const void* x, float* y,
               const float* resid, float* rows, const int64_t* dstate, float* amax, bool bf,
               hipStream_t s) {
  DecGemv a{};
  a.W = W; a.W2 = W2; a.N = N; a.K = K; a.x = x; a.y = y; a.resid = resid;
  a.rows = rows; a.dstate = dstate; a.amax = amax;
  // amax pairs are per block: with them, one row per wave (4 rows per block)
  const int shape = amax ? SHAPE_ROWS : (K < 4096 && !W2) ? SHAPE_ROWS2 : SHAPE_SPLIT;
  if (bf) dgemv_t<bf16>(a, false, OUT_F32, shape, s);
  else dgemv_t<float>(a, false, OUT_F32, shape, s);
}

void dgemv_ln_head(const void* U, int V, int d, const float* x, float eps, float* logits,
                   float* amax, bool bf, hipStream_t s) {
  DecGemv a{};
  a.W = U; a.N = V; a.K = d; a.x = x; a.eps = eps; a.y = logits; a.amax = amax;
  if (bf) dgemv_t<bf16>(a, true, OUT_F32, SHAPE_ROWS, s);
  else dgemv_t<float>(a, true, OUT_F32, SHAPE_ROWS, s);
}

int dgemv_blocks(int units) { return (units + 3) / 4; }   // SHAPE_ROWS: 4 rows per block

void dec_embed(const int32_t* cur, const int64_t* dstate, int32_t* hist, const void* E, int d, int V,
               float* x, int* err, bool bf, hipStream_t s) {
  if (bf) hipLaunchKernelGGL(dec_embed_k<bf16>, dim3(1), dim3(256), 0, s, cur, dstate, hist, (const bf16*)E, d, V, x, err);
  else hipLaunchKernelGGL(dec_embed_k<float>, dim3(1), dim3(256), 0, s, cur, dstate, hist, (const float*)E, d, V, x, err);
}
void dec_set(int64_t* dstate, int64_t pos, int64_t ci, hipStream_t s) {
  hipLaunchKernelGGL(dec_set_k, dim3(1), dim3(64), 0, s, dstate, pos, ci);
}
void copy_i32(const int32_t* a, int32_t* b, hipStream_t s) { hipLaunchKernelGGL(copy_i32_k, dim3(1), dim3(64), 0, s, a, b); }
void copy_f32(const float* a, float* b, int n, hipStream_t s) {
  hipLaunchKernelGGL(copy_f32_k, dim3((n + 255) / 256 > 1024 ? 1024 : (n + 255) / 256), dim3(256), 0, s, a, b, n);
}
void argmax_part(const float* part, int nb, int32_t* out_tok, int32_t* hist, int64_t* dstate,
                 bool advance, hipStream_t s) {
  hipLaunchKernelGGL(argmax_part_k, dim3(1), dim3(1024), 0, s, reinterpret_cast<const float2*>(part), nb,
                     out_tok, hist, dstate, (int)advance);
}

}  // namespace ttt
