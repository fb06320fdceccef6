// Banded-causal ("sliding window") flash attention for gfx950.
//
// Query at absolute position t attends to keys at positions j with
// t - W < j <= t (W keys, itself included), the short-term memory of the
// method (NVIDIA blog "Our method"; podcast 4:41 and 6:36 on the ~8K window).
// Keys and values live in a per-layer ring buffer, row (position mod cap),
// so the memory is bounded by the window whatever the context length.
//
// Layout of the work: a workgroup = 4 waves = 64 queries (forward, dQ) or 64
// keys (dK/dV) of one head; K/V (or Q/dO) tiles of 64 positions are staged
// in LDS, once k-contiguous and, where a product reduces over positions,
// once transposed.  Scores are computed transposed (S^T = K Q^T) so that each
// lane owns one query column; the accumulator layout of S^T is then exactly
// the operand layout that the P.V product needs, and the online softmax
// rescaling stays inside the lane.
#include "common.hpp"
#include "kernels.hpp"

namespace ttt {
namespace {

constexpr int TQ = 64;     // positions per tile
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

template <typename T, int HD> struct AttnCfg {
  static constexpr int KS = (HD + 31) / 32;          // 32-wide k steps over head_dim
  static constexpr int HDP = KS * 32;                // head_dim padded with zeros
  static constexpr int HB = HD / 16;                 // 16-row blocks of head_dim
  static constexpr int PAD = 16 / sizeof(T);
  static constexpr int LSN = HDP + PAD;              // natural tile row stride [pos][hd]
  static constexpr int LST = TQ + PAD;               // transposed tile row stride [hd][pos]
};

// Load a 64-position tile of one head from a ring ([cap][ld]) in natural
// layout (positions >= nvalid zero-filled, hd >= HD zero-filled).
template <typename T, int HD>
DEVI void load_nat(T* lds, const T* base, int64_t ld, int nvalid, int tid) {
  using C = AttnCfg<T, HD>;
  tile_copy_rows<T, TQ, C::HDP, C::LSN, 256>(lds, base, ld, nvalid, HD, tid);
}
template <typename T, int HD>
DEVI void load_tr(T* lds, const T* base, int64_t ld, int nvalid, int tid) {
  using C = AttnCfg<T, HD>;
  tile_copy_transpose<T, TQ, HD, C::LST, 256>(lds, base, ld, nvalid, HD, tid);
}

// operand fragment (8 k-slots over head_dim) of row r from a natural tile
template <typename T, int HD>
DEVI typename Frag<T>::type nat_frag(const T* lds, int r, int ks, int lane) {
  using C = AttnCfg<T, HD>;
  return lds_frag8<T>(lds + r * C::LSN + ks * 32 + 8 * (lane >> 4));
}
// operand fragment of head-dim row r from a transposed tile, k-slots = 32
// positions of pair pp laid out as two accumulator blocks (see header).
template <typename T, int HD>
DEVI typename Frag<T>::type tr_frag(const T* lds, int r, int pp, int lane) {
  using C = AttnCfg<T, HD>;
  const T* row = lds + r * C::LST + 4 * (lane >> 4);
  return lds_frag4x2<T>(row + (2 * pp) * 16, row + (2 * pp + 1) * 16);
}
// operand fragment built from two accumulator blocks (values per lane: 4 + 4)
template <typename T>
DEVI typename Frag<T>::type acc_frag(const f32x4& a, const f32x4& b) {
  float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return pack8<T>(v);
}

// register fragments of 16 rows (one per lane, row = l%16) of a [n][ld] matrix
template <typename T, int HD>
DEVI void row_frags(typename Frag<T>::type* f, const T* base, int64_t ld,
                    bool row_ok, int lane) {
#pragma unroll
  for (int ks = 0; ks < AttnCfg<T, HD>::KS; ++ks) {
    const int c = ks * 32 + 8 * (lane >> 4);
    f[ks] = g_frag8<T>(base + c, row_ok && c < HD);
  }
}

// ------------------------------------------------------------------ forward
// Each wave owns QB blocks of 16 queries, so every K / V^T fragment read
// from LDS feeds QB matrix-core products; K/V tiles are double-buffered
// (global reads for tile t+1 are in flight while tile t is consumed); only
// tiles that straddle the band edges evaluate the mask.
template <typename T, int HD, int QB>
__global__ __launch_bounds__(256) void swa_fwd_k(AttnParams p) {
  using C = AttnCfg<T, HD>;
  constexpr int QW = 16 * QB;
  constexpr int QT = 4 * QW;
  __shared__ __attribute__((aligned(16))) T Ks[2][TQ * C::LSN];
  __shared__ __attribute__((aligned(16))) T Vt[2][HD * C::LST];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.y;
  const int qs = blockIdx.x * QT;
  const int d = p.H * HD;
  const T* Q = static_cast<const T*>(p.q);
  const T* KR = static_cast<const T*>(p.kring);
  const T* VR = static_cast<const T*>(p.vring);

  typename Frag<T>::type qf[QB][C::KS];
  float m[QB], l[QB];
  f32x4 oacc[QB][C::HB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = qs + wave * QW + qb * 16 + (lane & 15);
    row_frags<T, HD>(qf[qb], Q + (int64_t)row * p.ldq + h * HD, p.ldq, row < p.n, lane);
    m[qb] = -INFINITY;
    l[qb] = 0.f;
#pragma unroll
    for (int b = 0; b < C::HB; ++b) oacc[qb][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float sc = LOG2E / sqrtf((float)HD);

  const int64_t first = p.pos0 + qs;
  const int64_t last = p.pos0 + min(qs + QT, p.n) - 1;
  int64_t lo = first - p.window + 1;
  if (lo < 0) lo = 0;
  const int64_t kt0 = (lo / TQ) * TQ;
  const int ntile = (int)((last - kt0) / TQ) + 1;

  StagedRows<T, TQ, C::HDP, C::LSN, 256> lk;
  StagedTrans<T, TQ, HD, C::LST, 256> lv;
  {
    const int nv = (int)min<int64_t>(TQ, last - kt0 + 1);
    const int64_t slot = kt0 % p.cap;
    lk.load(KR + slot * d + h * HD, d, nv, HD, tid);
    lv.load(VR + slot * d + h * HD, d, nv, HD, tid);
    lk.store(Ks[0], tid);
    lv.store(Vt[0], tid);
  }
  __syncthreads();

  for (int it = 0; it < ntile; ++it) {
    const int cur = it & 1;
    const int64_t kt = kt0 + (int64_t)it * TQ;
    if (it + 1 < ntile) {
      const int64_t kn = kt + TQ;
      const int nv = (int)min<int64_t>(TQ, last - kn + 1);
      const int64_t slot = kn % p.cap;
      lk.load(KR + slot * d + h * HD, d, nv, HD, tid);
      lv.load(VR + slot * d + h * HD, d, nv, HD, tid);
    }
    const bool interior = (kt + TQ - 1 <= first) && (kt > last - p.window);
    const int kq0 = (int)(kt - first);   // key offset relative to the first query
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      f32x4 s[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks)
          mma16x16x32(nat_frag<T, HD>(Ks[cur], kb * 16 + (lane & 15), ks, lane), qf[qb][ks], s[kb]);
      }
      if (!interior) {
        const int qoff = wave * QW + qb * 16 + (lane & 15);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int rel = kq0 + kb * 16 + 4 * (lane >> 4) + i - qoff;   // key - query
            if (!(rel <= 0 && rel > -p.window)) s[kb][i] = -INFINITY;
          }
      }
      float tmax = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        tmax = fmaxf(fmaxf(tmax, fmaxf(s[kb][0], s[kb][1])), fmaxf(s[kb][2], s[kb][3]));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      tmax *= sc;   // scores enter the exponent as s * sc (log2 units)
      // Lazy rescaling: the reference maximum only moves when the tile's
      // maximum exceeds it by more than 8 (log2 units), so probabilities stay
      // below 2^8 (harmless in fp32 sums and in bf16) and the accumulator
      // rescale is skipped on almost every tile.  The result does not depend
      // on the reference, so this is exact.
      const bool bump = tmax > m[qb] + 8.f;
      if (__any(bump)) {
        const float mn = bump ? tmax : m[qb];
        const float alpha = (m[qb] == -INFINITY) ? 0.f : fast_exp2(m[qb] - mn);
        l[qb] *= alpha;
#pragma unroll
        for (int b = 0; b < C::HB; ++b) oacc[qb][b] *= alpha;
        m[qb] = mn;
      }
      const float mref = (m[qb] == -INFINITY) ? 0.f : m[qb];
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = fast_exp2(fmaf(s[kb][i], sc, -mref));   // -inf -> 0
          s[kb][i] = e;
          rs += e;
        }
      rs += __shfl_xor(rs, 16, 64);
      rs += __shfl_xor(rs, 32, 64);
      l[qb] += rs;
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        const typename Frag<T>::type pf = acc_frag<T>(s[2 * pp], s[2 * pp + 1]);
#pragma unroll
        for (int b = 0; b < C::HB; ++b)
          mma16x16x32(tr_frag<T, HD>(Vt[cur], b * 16 + (lane & 15), pp, lane), pf, oacc[qb][b]);
      }
    }
    if (it + 1 < ntile) {
      lk.store(Ks[cur ^ 1], tid);
      lv.store(Vt[cur ^ 1], tid);
    }
    __syncthreads();
  }

#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = qs + wave * QW + qb * 16 + (lane & 15);
    if (row >= p.n) continue;
    const float inv = l[qb] > 0.f ? 1.f / l[qb] : 0.f;
    T* O = static_cast<T*>(p.o) + (int64_t)row * p.ldo + h * HD;
#pragma unroll
    for (int b = 0; b < C::HB; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) O[b * 16 + 4 * (lane >> 4) + i] = from_f32<T>(oacc[qb][b][i] * inv);
    if (p.lse && (lane >> 4) == 0) p.lse[(int64_t)h * p.n + row] = (m[qb] + log2f(l[qb])) * LN2;
  }
}

// ------------------------------------------- forward, 32x32 matrix cores
// Each wave owns 32 queries.  Scores are formed transposed, Sᵀ[32 keys x 32
// queries] = K·Qᵀ with the 32x32x16 step, so a lane holds 16 keys of one
// query and the row max/sum need one cross-half exchange only.  Eight
// consecutive accumulator values of a lane are exactly the k-slots of the
// next P·V step (keys 16h..16h+15 of a 32-key block), so probabilities go
// from accumulator to operand without leaving registers.  V is read from
// its transposed ring copy ([H*hd][cap]), so both tiles are plain copies.
template <typename T, int HD> struct Attn32 {
  static constexpr int KS = HD / 16;              // 16-wide k steps of Qᵀ
  static constexpr int HB = (HD + 31) / 32;       // 32-row blocks of Oᵀ
  static constexpr int HDR = HB * 32;             // Vᵀ tile rows (zero beyond HD)
  static constexpr int PAD = 16 / sizeof(T);
  static constexpr int LSN = HD + PAD;            // K tile pitch  [key][hd]
  static constexpr int LSV = TQ + PAD;            // Vᵀ tile pitch [hd][key]
};

template <typename T, int HD>
__global__ __launch_bounds__(256) void swa_fwd32_k(AttnParams p) {
  using C = Attn32<T, HD>;
  constexpr int QT = 128;
  __shared__ __attribute__((aligned(16))) T Ks[2][TQ * C::LSN];
  __shared__ __attribute__((aligned(16))) T Vt[2][C::HDR * C::LSV];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, ql = lane & 31;
  const int h = blockIdx.y;
  const int qs = blockIdx.x * QT;
  const int d = p.H * HD;
  const T* Q = static_cast<const T*>(p.q);
  const T* KR = static_cast<const T*>(p.kring);
  const T* VT = static_cast<const T*>(p.vtring) + (int64_t)h * HD * p.cap;

  const int qrow = qs + wave * 32 + ql;
  typename Frag<T>::type qf[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks)
    qf[ks] = g_frag8<T>(Q + (int64_t)qrow * p.ldq + h * HD + ks * 16 + 8 * hl, qrow < p.n);
  float m = -INFINITY, l = 0.f;
  f32x16 oacc[C::HB];
#pragma unroll
  for (int b = 0; b < C::HB; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[b][r] = 0.f;
  const float sc = LOG2E / sqrtf((float)HD);

  const int64_t first = p.pos0 + qs;
  const int64_t last = p.pos0 + min(qs + QT, p.n) - 1;
  int64_t lo = first - p.window + 1;
  if (lo < 0) lo = 0;
  const int64_t kt0 = (lo / TQ) * TQ;
  const int ntile = (int)((last - kt0) / TQ) + 1;

  // Whole tiles are copied (the ring rows exist for every slot); keys past
  // the last query are masked by causality.
  StagedRows<T, TQ, HD, C::LSN, 256> lk;
  StagedRows<T, C::HDR, TQ, C::LSV, 256> lv;
  {
    const int64_t slot = kt0 % p.cap;
    lk.load(KR + slot * d + h * HD, d, TQ, HD, tid);
    lv.load(VT + slot, p.cap, HD, TQ, tid);
    lk.store(Ks[0], tid);
    lv.store(Vt[0], tid);
  }
  __syncthreads();

  for (int it = 0; it < ntile; ++it) {
    const int cur = it & 1;
    const int64_t kt = kt0 + (int64_t)it * TQ;
    if (it + 1 < ntile) {
      const int64_t slot = (kt + TQ) % p.cap;
      lk.load(KR + slot * d + h * HD, d, TQ, HD, tid);
      lv.load(VT + slot, p.cap, HD, TQ, tid);
    }
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks)
        mma32x32x16(lds_frag8<T>(Ks[cur] + (kb * 32 + ql) * C::LSN + ks * 16 + 8 * hl), qf[ks], s[kb]);
    }
    const bool interior = (kt + TQ - 1 <= first) && (kt > last - p.window);
    if (!interior) {
      const int kq0 = (int)(kt - first) - (wave * 32 + ql);   // key - query of s[0][0]
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rel = kq0 + kb * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
          if (!(rel <= 0 && rel > -p.window)) s[kb][r] = -INFINITY;
        }
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) tmax = fmaxf(tmax, fmaxf(s[kb][r], s[kb][r + 1]));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64)) * sc;
    // lazy rescaling (see the 16x16 kernel above): exact, rarely taken
    const bool bump = tmax > m + 8.f;
    if (__any(bump)) {
      const float mn = bump ? tmax : m;
      const float alpha = (m == -INFINITY) ? 0.f : fast_exp2(m - mn);
      l *= alpha;
#pragma unroll
      for (int b = 0; b < C::HB; ++b) oacc[b] *= alpha;
      m = mn;
    }
    const float mref = (m == -INFINITY) ? 0.f : m;
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = fast_exp2(fmaf(s[kb][r], sc, -mref));
        s[kb][r] = e;
        rs += e;
      }
    l += rs + __shfl_xor(rs, 32, 64);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        float pv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) pv[j] = s[kb][8 * hf + j];
        const typename Frag<T>::type pf = pack8<T>(pv);
        const int koff = kb * 32 + 16 * hf + 4 * hl;
#pragma unroll
        for (int b = 0; b < C::HB; ++b) {
          const T* row = Vt[cur] + (b * 32 + ql) * C::LSV + koff;
          mma32x32x16(lds_frag4x2<T>(row, row + 8), pf, oacc[b]);
        }
      }
    if (it + 1 < ntile) {
      lk.store(Ks[cur ^ 1], tid);
      lv.store(Vt[cur ^ 1], tid);
    }
    __syncthreads();
  }

  if (qrow < p.n) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    T* O = static_cast<T*>(p.o) + (int64_t)qrow * p.ldo + h * HD;
#pragma unroll
    for (int b = 0; b < C::HB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int c = b * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
        if (c < HD) O[c] = from_f32<T>(oacc[b][r] * inv);
      }
    if (p.lse && hl == 0) p.lse[(int64_t)h * p.n + qrow] = (m + log2f(l)) * LN2;
  }
}

// Vᵀ ring copy: rows h*hd + i, column (position mod cap); one block per 64
// positions of one head, transposed through LDS so both sides coalesce.
template <typename T>
__global__ __launch_bounds__(256) void ring_vt_k(const T* __restrict__ qkv, int n, int H, int hd,
                                                 int64_t pos0, T* __restrict__ vt, int64_t cap) {
  __shared__ T tile[64][128 + 2];
  const int h = blockIdx.y, t0 = blockIdx.x * 64, tid = threadIdx.x;
  const int d = H * hd;
  for (int idx = tid; idx < 64 * hd; idx += 256) {
    const int t = idx / hd, i = idx % hd;
    tile[t][i] = (t0 + t < n) ? qkv[(int64_t)(t0 + t) * 3 * d + 2 * d + h * hd + i] : from_f32<T>(0.f);
  }
  __syncthreads();
  for (int idx = tid; idx < hd * 64; idx += 256) {
    const int i = idx / 64, t = idx % 64;
    if (t0 + t < n) vt[(int64_t)(h * hd + i) * cap + (pos0 + t0 + t) % cap] = tile[t][i];
  }
}

// ------------------------------------------------------------ backward dQ
template <typename T, int HD>
__global__ __launch_bounds__(256) void swa_bwd_dq_k(AttnParams p) {
  using C = AttnCfg<T, HD>;
  __shared__ __attribute__((aligned(16))) T Ks[TQ * C::LSN];
  __shared__ __attribute__((aligned(16))) T Vs[TQ * C::LSN];
  __shared__ __attribute__((aligned(16))) T Kt[HD * C::LST];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.y;
  const int qs = blockIdx.x * TQ;
  const int d = p.H * HD;
  const T* KR = static_cast<const T*>(p.kring);
  const T* VR = static_cast<const T*>(p.vring);

  const int qrow = qs + wave * 16 + (lane & 15);
  const bool qok = qrow < p.n;
  const int64_t qpos = p.pos0 + qrow;
  typename Frag<T>::type qf[C::KS], gf[C::KS];
  row_frags<T, HD>(qf, static_cast<const T*>(p.q) + (int64_t)qrow * p.ldq + h * HD, p.ldq, qok, lane);
  row_frags<T, HD>(gf, static_cast<const T*>(p.dout) + (int64_t)qrow * p.lddo + h * HD, p.lddo, qok, lane);
  const float lse2 = qok ? p.lse[(int64_t)h * p.n + qrow] * LOG2E : 0.f;
  const float Dq = qok ? p.D[(int64_t)h * p.n + qrow] : 0.f;
  const float sc = LOG2E / sqrtf((float)HD);

  f32x4 dacc[C::HB];
#pragma unroll
  for (int b = 0; b < C::HB; ++b) dacc[b] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int64_t first = p.pos0 + qs;
  const int64_t last = p.pos0 + min(qs + TQ, p.n) - 1;
  int64_t lo = first - p.window + 1;
  if (lo < 0) lo = 0;
  for (int64_t kt = (lo / TQ) * TQ; kt <= last; kt += TQ) {
    const int nvalid = (int)min<int64_t>(TQ, last - kt + 1);
    const int64_t slot = kt % p.cap;
    __syncthreads();
    load_nat<T, HD>(Ks, KR + slot * d + h * HD, d, nvalid, tid);
    load_nat<T, HD>(Vs, VR + slot * d + h * HD, d, nvalid, tid);
    load_tr<T, HD>(Kt, KR + slot * d + h * HD, d, nvalid, tid);
    __syncthreads();

    f32x4 s[4], dp[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
      dp[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        mma16x16x32(nat_frag<T, HD>(Ks, kb * 16 + (lane & 15), ks, lane), qf[ks], s[kb]);
        mma16x16x32(nat_frag<T, HD>(Vs, kb * 16 + (lane & 15), ks, lane), gf[ks], dp[kb]);
      }
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t kp = kt + kb * 16 + 4 * (lane >> 4) + i;
        const bool ok = qok && kp <= qpos && kp > qpos - p.window;
        const float pr = ok ? fast_exp2(fmaf(s[kb][i], sc, -lse2)) : 0.f;
        s[kb][i] = pr * (dp[kb][i] - Dq);   // dS^T
      }
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      const typename Frag<T>::type df = acc_frag<T>(s[2 * pp], s[2 * pp + 1]);
#pragma unroll
      for (int b = 0; b < C::HB; ++b)
        mma16x16x32(tr_frag<T, HD>(Kt, b * 16 + (lane & 15), pp, lane), df, dacc[b]);
    }
  }
  if (qok) {
    const float scale = 1.f / sqrtf((float)HD);
    T* G = static_cast<T*>(p.dq) + (int64_t)qrow * p.ldg + h * HD;
#pragma unroll
    for (int b = 0; b < C::HB; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) G[b * 16 + 4 * (lane >> 4) + i] = from_f32<T>(dacc[b][i] * scale);
  }
}

// --------------------------------------------------------- backward dK, dV
// Keys are the in-chunk positions (query rows of this chunk); cached keys
// of earlier chunks are constants and receive no gradient.
template <typename T, int HD>
__global__ __launch_bounds__(256) void swa_bwd_dkdv_k(AttnParams p) {
  using C = AttnCfg<T, HD>;
  __shared__ __attribute__((aligned(16))) T Qs[TQ * C::LSN];
  __shared__ __attribute__((aligned(16))) T Gs[TQ * C::LSN];
  __shared__ __attribute__((aligned(16))) T Qt[HD * C::LST];
  __shared__ __attribute__((aligned(16))) T Gt[HD * C::LST];
  __shared__ float lse_s[TQ], D_s[TQ];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.y;
  const int ks0 = blockIdx.x * TQ;
  const int d = p.H * HD;
  const T* Q = static_cast<const T*>(p.q);
  const T* G = static_cast<const T*>(p.dout);
  const T* KR = static_cast<const T*>(p.kring);
  const T* VR = static_cast<const T*>(p.vring);

  const int krow = ks0 + wave * 16 + (lane & 15);     // chunk-relative key index
  const bool kok = krow < p.n;
  const int64_t kpos = p.pos0 + krow;
  const int64_t kslot = (kok ? kpos : p.pos0) % p.cap;
  typename Frag<T>::type kf[C::KS], vf[C::KS];
  row_frags<T, HD>(kf, KR + kslot * d + h * HD, d, kok, lane);
  row_frags<T, HD>(vf, VR + kslot * d + h * HD, d, kok, lane);
  const float sc = LOG2E / sqrtf((float)HD);

  f32x4 dk[C::HB], dv[C::HB];
#pragma unroll
  for (int b = 0; b < C::HB; ++b) { dk[b] = f32x4{0.f, 0.f, 0.f, 0.f}; dv[b] = f32x4{0.f, 0.f, 0.f, 0.f}; }

  const int kmax = min(ks0 + TQ, p.n) - 1;
  const int64_t qend = min<int64_t>((int64_t)p.n - 1, (int64_t)kmax + p.window - 1);
  for (int qt = ks0; qt <= qend; qt += TQ) {
    const int nvalid = min(TQ, p.n - qt);
    __syncthreads();
    load_nat<T, HD>(Qs, Q + (int64_t)qt * p.ldq + h * HD, p.ldq, nvalid, tid);
    load_nat<T, HD>(Gs, G + (int64_t)qt * p.lddo + h * HD, p.lddo, nvalid, tid);
    load_tr<T, HD>(Qt, Q + (int64_t)qt * p.ldq + h * HD, p.ldq, nvalid, tid);
    load_tr<T, HD>(Gt, G + (int64_t)qt * p.lddo + h * HD, p.lddo, nvalid, tid);
    if (tid < TQ) {
      const bool ok = tid < nvalid;
      lse_s[tid] = ok ? p.lse[(int64_t)h * p.n + qt + tid] * LOG2E : 0.f;
      D_s[tid] = ok ? p.D[(int64_t)h * p.n + qt + tid] : 0.f;
    }
    __syncthreads();

    f32x4 s[4], dp[4];
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      s[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
      dp[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        mma16x16x32(nat_frag<T, HD>(Qs, qb * 16 + (lane & 15), ks, lane), kf[ks], s[qb]);
        mma16x16x32(nat_frag<T, HD>(Gs, qb * 16 + (lane & 15), ks, lane), vf[ks], dp[qb]);
      }
    }
#pragma unroll
    for (int qb = 0; qb < 4; ++qb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int qi = qb * 16 + 4 * (lane >> 4) + i;
        const int64_t qp = p.pos0 + qt + qi;
        const bool ok = kok && (qt + qi < p.n) && kpos <= qp && kpos > qp - p.window;
        const float pr = ok ? fast_exp2(fmaf(s[qb][i], sc, -lse_s[qi])) : 0.f;
        s[qb][i] = pr;                              // P
        dp[qb][i] = pr * (dp[qb][i] - D_s[qi]);     // dS
      }
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      const typename Frag<T>::type pf = acc_frag<T>(s[2 * pp], s[2 * pp + 1]);
      const typename Frag<T>::type df = acc_frag<T>(dp[2 * pp], dp[2 * pp + 1]);
#pragma unroll
      for (int b = 0; b < C::HB; ++b) {
        mma16x16x32(tr_frag<T, HD>(Gt, b * 16 + (lane & 15), pp, lane), pf, dv[b]);
        mma16x16x32(tr_frag<T, HD>(Qt, b * 16 + (lane & 15), pp, lane), df, dk[b]);
      }
    }
  }
  if (kok) {
    const float scale = 1.f / sqrtf((float)HD);
    T* DK = static_cast<T*>(p.dk) + (int64_t)krow * p.ldg + h * HD;
    T* DV = static_cast<T*>(p.dv) + (int64_t)krow * p.ldg + h * HD;
#pragma unroll
    for (int b = 0; b < C::HB; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        DK[b * 16 + 4 * (lane >> 4) + i] = from_f32<T>(dk[b][i] * scale);
        DV[b * 16 + 4 * (lane >> 4) + i] = from_f32<T>(dv[b][i]);
      }
  }
}

template <typename T, template <typename, int> class K> struct HdDispatch;

template <typename T>
void fwd_t(const AttnParams& p, hipStream_t s) {
  dim3 grid((p.n + 127) / 128, p.H);
  switch (p.hd) {
    case 16: hipLaunchKernelGGL((swa_fwd32_k<T, 16>), grid, dim3(256), 0, s, p); break;
    case 32: hipLaunchKernelGGL((swa_fwd32_k<T, 32>), grid, dim3(256), 0, s, p); break;
    case 64: hipLaunchKernelGGL((swa_fwd32_k<T, 64>), grid, dim3(256), 0, s, p); break;
    case 96: hipLaunchKernelGGL((swa_fwd32_k<T, 96>), grid, dim3(256), 0, s, p); break;
    case 128: hipLaunchKernelGGL((swa_fwd32_k<T, 128>), grid, dim3(256), 0, s, p); break;
    default: break;
  }
}
template <typename T>
void bwd_t(const AttnParams& p, hipStream_t s) {
  dim3 grid((p.n + TQ - 1) / TQ, p.H);
  switch (p.hd) {
#define CASE(HDV) case HDV: \
    hipLaunchKernelGGL((swa_bwd_dq_k<T, HDV>), grid, dim3(256), 0, s, p); \
    hipLaunchKernelGGL((swa_bwd_dkdv_k<T, HDV>), grid, dim3(256), 0, s, p); break;
    CASE(16) CASE(32) CASE(64) CASE(96) CASE(128)
#undef CASE
    default: break;
  }
}

}  // namespace

void swa_fwd(const AttnParams& p, bool bf, hipStream_t s) {
  if (p.n <= 0) return;
  if (bf) fwd_t<bf16>(p, s); else fwd_t<float>(p, s);
}
void ring_write_vt(const void* qkv, int n, int H, int hd, int64_t pos0, void* vt, int64_t cap, bool bf,
                   hipStream_t s) {
  if (n <= 0) return;
  dim3 grid((n + 63) / 64, H);
  if (bf) hipLaunchKernelGGL(ring_vt_k<bf16>, grid, dim3(256), 0, s, (const bf16*)qkv, n, H, hd, pos0, (bf16*)vt, cap);
  else hipLaunchKernelGGL(ring_vt_k<float>, grid, dim3(256), 0, s, (const float*)qkv, n, H, hd, pos0, (float*)vt, cap);
}

void swa_bwd(const AttnParams& p, bool bf, hipStream_t s) {
  if (p.n <= 0) return;
  if (bf) bwd_t<bf16>(p, s); else bwd_t<float>(p, s);
}

}  // namespace ttt
