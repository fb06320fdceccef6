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
#include <algorithm>
#include <type_traits>

namespace ttt {
namespace {

// Workgroups are dealt to the 8 XCDs round-robin by linear id, and the
// query tiles of one head are consecutive ids: left as is, every XCD would
// hold one tile of every head and its L2 would fetch every head's keys.
// Renumber so that each XCD holds a contiguous run of logical ids (whole
// heads, all their query tiles), which then share K/V lines in that L2.
DEVI void attn_block(int& bx, int& by, int& bz) {
  const int gx = gridDim.x, gy = gridDim.y;
  const int total = gx * gy * (int)gridDim.z;
  const int b = blockIdx.x + gx * (blockIdx.y + gy * blockIdx.z);
  const int x = b & 7, y = b >> 3, q8 = total >> 3, r8 = total & 7;
  const int L = x * q8 + min(x, r8) + y;
  bx = L % gx;
  const int r = L / gx;
  by = r % gy;
  bz = r / gy;
}


constexpr int TQ = 64;     // positions per tile
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// ------------------------------------------- forward, 32x32 matrix cores
// Each wave owns 32 queries.  Scores are formed transposed, Sᵀ[32 keys x 32
// queries] = K·Qᵀ with the 32x32x16 step, so a lane holds 16 keys of one
// query and the row max/sum need one cross-half exchange only.  Eight
// consecutive accumulator values of a lane are exactly the k-slots of the
// next P·V step (keys 16h..16h+15 of a 32-key block), so probabilities go
// from accumulator to operand without leaving registers.  V is read from
// its key-permuted transposed ring copy ([H*hd][cap], see kperm), so both
// tiles are plain copies and each P.V operand fragment is one 16-byte read.
template <typename T, int HD> struct Attn32 {
  static constexpr int KS = HD / 16;              // 16-wide k steps of Qᵀ
  static constexpr int HB = (HD + 31) / 32;       // 32-row blocks of Oᵀ
  static constexpr int HDR = HB * 32;             // Vᵀ tile rows (zero beyond HD)
  static constexpr int PAD = 16 / sizeof(T);
  static constexpr int LSN = HD + PAD;            // K tile pitch  [key][hd]
  static constexpr int LSV = TQ + PAD;            // Vᵀ tile pitch [hd][key]
};

template <typename T, int HD>
__global__ __launch_bounds__(256, 2) void swa_fwd32_k(AttnParams p) {
  using C = Attn32<T, HD>;
  constexpr int QT = 128;
  __shared__ __attribute__((aligned(16))) T Ks[2][TQ * C::LSN];
  __shared__ __attribute__((aligned(16))) T Vt[2][C::HDR * C::LSV];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, ql = lane & 31;
  int bx, h, bz;
  attn_block(bx, h, bz);
  const int qs = bx * QT;
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
  // split z of gridDim.z takes a contiguous run of the key tiles
  const int64_t ktA = (lo / TQ) * TQ;
  const int nall = (int)((last - ktA) / TQ) + 1;
  const int per = (nall + (int)gridDim.z - 1) / (int)gridDim.z;
  const int tb = min(nall, bz * per), te = min(nall, tb + per);
  const int64_t kt0 = ktA + (int64_t)tb * TQ;
  const int ntile = te - tb;

  // Whole tiles are copied (the ring rows exist for every slot); keys past
  // the last query are masked by causality.
  StagedRows<T, TQ, HD, C::LSN, 256> lk;
  StagedRows<T, C::HDR, TQ, C::LSV, 256> lv;
  if (ntile > 0) {
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
    // lazy rescaling: the reference max m is raised only when a tile's max
    // exceeds it by more than 2^8, so exponents stay below 2^8; exact, since
    // l and O share the reference, and rarely taken
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
        // the 8 keys of this lane's k-slots: one run of the key-permuted V^T row
        const int koff = kb * 32 + 16 * hf + 8 * hl;
#pragma unroll
        for (int b = 0; b < C::HB; ++b)
          mma32x32x16(lds_frag8<T>(Vt[cur] + (b * 32 + ql) * C::LSV + koff), pf, oacc[b]);
      }
    if (it + 1 < ntile) {
      lk.store(Ks[cur ^ 1], tid);
      lv.store(Vt[cur ^ 1], tid);
    }
    __syncthreads();
  }

  if (qrow < p.n) {
    if (gridDim.z == 1) {
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
    } else {
      // unnormalised partial of this key range, combined by swa_combine_k
      float* O = p.part + ((int64_t)bz * p.n + qrow) * d + h * HD;
#pragma unroll
      for (int b = 0; b < C::HB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = b * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
          if (c < HD) O[c] = oacc[b][r];
        }
      if (hl == 0) {
        float* ml = p.part_ml + ((int64_t)bz * p.H + h) * p.n * 2;
        ml[2 * qrow] = m;
        ml[2 * qrow + 1] = l;
      }
    }
  }
}

// Combine key-range partials: O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
template <typename T>
__global__ void swa_combine_k(AttnParams p, int nsplit) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;   // over n * H * hd
  const int d = p.H * p.hd;
  if (idx >= p.n * d) return;
  const int row = idx / d, c = idx % d, h = c / p.hd;
  float M = -INFINITY;
  for (int z = 0; z < nsplit; ++z) M = fmaxf(M, p.part_ml[(((int64_t)z * p.H + h) * p.n + row) * 2]);
  float L = 0.f, acc = 0.f;
  for (int z = 0; z < nsplit; ++z) {
    const float* ml = p.part_ml + (((int64_t)z * p.H + h) * p.n + row) * 2;
    const float f = (ml[0] == -INFINITY) ? 0.f : fast_exp2(ml[0] - M);
    L += ml[1] * f;
    acc += p.part[((int64_t)z * p.n + row) * d + c] * f;
  }
  static_cast<T*>(p.o)[(int64_t)row * p.ldo + c] = from_f32<T>(L > 0.f ? acc / L : 0.f);
  if (p.lse && c % p.hd == 0) p.lse[(int64_t)h * p.n + row] = (M + log2f(L)) * LN2;
}



// ------------------------------------------------------------ backward dQ
// dQ = scale * sum_keys dS K with dS = P (dP - D), P = exp(S - LSE),
// dP = dO Vᵀ, over every key of the window (cached keys included).  Lanes
// own queries as in the forward; Sᵀ and dPᵀ come from K and V tiles, the dQᵀ
// product from the transposed K ring copy.  Single-buffered tiles; two
// workgroups share a CU.
template <typename T, int HD>
__global__ __launch_bounds__(256, 2) void swa_bwd_dq32_k(AttnParams p) {
  using C = Attn32<T, HD>;
  constexpr int QT = 128;
  __shared__ __attribute__((aligned(16))) T Ks[TQ * C::LSN];
  __shared__ __attribute__((aligned(16))) T Vs[TQ * C::LSN];
  __shared__ __attribute__((aligned(16))) T Kt[C::HDR * C::LSV];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, ql = lane & 31;
  int bx, h, bz;
  attn_block(bx, h, bz);
  const int qs = bx * QT;
  const int d = p.H * HD;
  const T* KR = static_cast<const T*>(p.kring);
  const T* VR = static_cast<const T*>(p.vring);
  const T* KT = static_cast<const T*>(p.ktring) + (int64_t)h * HD * p.cap;

  const int qrow = qs + wave * 32 + ql;
  const bool qok = qrow < p.n;
  typename Frag<T>::type qf[C::KS], gf[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    qf[ks] = g_frag8<T>(static_cast<const T*>(p.q) + (int64_t)qrow * p.ldq + h * HD + ks * 16 + 8 * hl, qok);
    gf[ks] = g_frag8<T>(static_cast<const T*>(p.dout) + (int64_t)qrow * p.lddo + h * HD + ks * 16 + 8 * hl, qok);
  }
  const float lse2 = qok ? p.lse[(int64_t)h * p.n + qrow] * LOG2E : 0.f;
  const float Dq = qok ? p.D[(int64_t)h * p.n + qrow] : 0.f;
  const float sc = LOG2E / sqrtf((float)HD);
  f32x16 dacc[C::HB];
#pragma unroll
  for (int b = 0; b < C::HB; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) dacc[b][r] = 0.f;

  const int64_t first = p.pos0 + qs;
  const int64_t last = p.pos0 + min(qs + QT, p.n) - 1;
  int64_t lo = first - p.window + 1;
  if (lo < 0) lo = 0;
  const int64_t ktA = (lo / TQ) * TQ;
  const int nall = (int)((last - ktA) / TQ) + 1;
  const int per = (nall + (int)gridDim.z - 1) / (int)gridDim.z;
  const int tb = min(nall, bz * per), te = min(nall, tb + per);
  for (int it = tb; it < te; ++it) {
    const int64_t kt = ktA + (int64_t)it * TQ;
    const int64_t slot = kt % p.cap;
    __syncthreads();
    tile_copy_rows<T, TQ, HD, C::LSN, 256>(Ks, KR + slot * d + h * HD, d, TQ, HD, tid);
    tile_copy_rows<T, TQ, HD, C::LSN, 256>(Vs, VR + slot * d + h * HD, d, TQ, HD, tid);
    tile_copy_rows<T, C::HDR, TQ, C::LSV, 256>(Kt, KT + slot, p.cap, HD, TQ, tid);
    __syncthreads();
    f32x16 s[2], dp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) { s[kb][r] = 0.f; dp[kb][r] = 0.f; }
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        mma32x32x16(lds_frag8<T>(Ks + (kb * 32 + ql) * C::LSN + ks * 16 + 8 * hl), qf[ks], s[kb]);
        mma32x32x16(lds_frag8<T>(Vs + (kb * 32 + ql) * C::LSN + ks * 16 + 8 * hl), gf[ks], dp[kb]);
      }
    }
    const bool interior = (kt + TQ - 1 <= first) && (kt > last - p.window);
    const int kq0 = (int)(kt - first) - (wave * 32 + ql);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rel = kq0 + kb * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
        const bool ok = qok && (interior || (rel <= 0 && rel > -p.window));
        const float pr = ok ? fast_exp2(fmaf(s[kb][r], sc, -lse2)) : 0.f;
        s[kb][r] = pr * (dp[kb][r] - Dq);   // dSᵀ
      }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        float dv8[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) dv8[j] = s[kb][8 * hf + j];
        const typename Frag<T>::type df = pack8<T>(dv8);
        // the 8 keys of this lane's k-slots, one 16-byte run of the
        // key-permuted transposed K copy
        const int koff = kb * 32 + 16 * hf + 8 * hl;
#pragma unroll
        for (int b = 0; b < C::HB; ++b)
          mma32x32x16(lds_frag8<T>(Kt + (b * 32 + ql) * C::LSV + koff), df, dacc[b]);
      }
  }
  if (qok) {
    const float scale = 1.f / sqrtf((float)HD);
    if (gridDim.z == 1) {
      T* G = static_cast<T*>(p.dq) + (int64_t)qrow * p.ldg + h * HD;
#pragma unroll
      for (int b = 0; b < C::HB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = b * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
          if (c < HD) G[c] = from_f32<T>(dacc[b][r] * scale);
        }
    } else {
      float* G = p.part + ((int64_t)bz * p.n + qrow) * d + h * HD;
#pragma unroll
      for (int b = 0; b < C::HB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = b * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
          if (c < HD) G[c] = dacc[b][r] * scale;
        }
    }
  }
}

template <typename T>
__global__ void dq_combine_k(AttnParams p, int nsplit) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  const int d = p.H * p.hd;
  if (!p.rope_cs) {
    if (idx >= p.n * d) return;
    const int row = idx / d, c = idx % d;
    float acc = 0.f;
    for (int z = 0; z < nsplit; ++z) acc += p.part[((int64_t)z * p.n + row) * d + c];
    static_cast<T*>(p.dq)[(int64_t)row * p.ldg + c] = from_f32<T>(acc);
    return;
  }
  // with RoPE^-1: one thread per pair (i, i + hd/2) of a head, each summed
  // and rounded to T, then turned back by the row's angle and rounded again
  const int half = p.hd / 2;
  if (idx >= p.n * (d / 2)) return;
  const int row = idx / (d / 2), r = idx % (d / 2), h = r / half, i = r % half;
  const int c = h * p.hd + i;
  float a = 0.f, b = 0.f;
  for (int z = 0; z < nsplit; ++z) {
    const float* pz = p.part + ((int64_t)z * p.n + row) * d + c;
    a += pz[0];
    b += pz[half];
  }
  a = to_f32(from_f32<T>(a));
  b = to_f32(from_f32<T>(b));
  const float2 w = p.rope_cs[(int64_t)row * half + i];
  T* o = static_cast<T*>(p.dq) + (int64_t)row * p.ldg + c;
  o[0] = from_f32<T>(a * w.x + b * w.y);
  o[half] = from_f32<T>(b * w.x - a * w.y);
}

// ------------------------------------------------ backward dQ, bf16, hd 128
// The same product as swa_bwd_dq32_k for the bf16 / head_dim 128 case,
// organised for throughput: a workgroup of 8 waves holds 256 queries (32 per
// wave, two waves per SIMD so one's exponentials overlap the other's matrix
// steps), and the 64-key tiles of K, V (natural, [key][hd]) and of the
// key-permuted K^T copy ([hd][key]) are brought in by direct global->LDS
// 16-byte loads into two stages, the next tile's loads in flight while the
// current one is multiplied; each tile is loaded once for 256 queries.  LDS
// rows are XOR-swizzled at 16-byte granularity (K/V rows of 256 B: slot
// c ^ (row & 15); K^T rows of 128 B: slot c ^ ((row >> 1) & 7)) so the
// fragment reads are conflict-free.
namespace stg {
constexpr int HD = 128, KT = 64, NW = 8, QT = 32 * NW, NTHR = 64 * NW;
constexpr int ROWK = HD * 2;                 // bytes of a K/V row (one key)
constexpr int TILE_K = KT * ROWK;            // 16 KB
constexpr int ROWT = KT * 2;                 // bytes of a K^T row (one head dim)
constexpr int TILE_T = HD * ROWT;            // 16 KB
constexpr int STAGE = 2 * TILE_K + TILE_T;   // dQ: K, V, K^T (48 KB)
constexpr int LDS_BYTES = 2 * STAGE;         // 96 KB: one workgroup per CU
constexpr int STAGE_F = TILE_K + TILE_T;     // forward: K, V^T (32 KB)
constexpr int LDS_F = 2 * STAGE_F;           // 64 KB
constexpr int PER = 16 / NW;                 // 1 KB load instructions per wave and array
// dK/dV: 4 waves x 32 keys; per 64-query tile Q and dO ([query][hd], rows
// of 256 B), their transposes ([hd][query], rows of 128 B) and the tile's
// LSE and D (256 B each)
constexpr int KWAVES = 4, KB_ = 32 * KWAVES, QTL = 64;
constexpr int TILE_Q = QTL * ROWK;           // 16 KB
constexpr int TILE_QT = HD * QTL * 2;        // 16 KB
constexpr int STAGE_B = 2 * TILE_Q + 2 * TILE_QT + 2 * QTL * 4;
constexpr int LDS_B = 2 * STAGE_B;           // 129 KB
typedef __attribute__((address_space(3))) void lds_void;
DEVI __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
  const int nb = bytes > 0x7fffffff ? 0x7fffffff : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nb, 0x00020000);
}
}  // namespace stg

// RoPE^-1 of one row of a head-dim-128 gradient held in 32x32 accumulator
// blocks (block b has dims b*32 + 8g + 4*hl + e): the gradient is scaled and
// rounded to bf16 first, then each pair (i, i + 64) is turned back by the
// row's angle (cs[i] = (cos, sin)) and rounded again, as the separate RoPE
// backward pass does on the stored gradient.
DEVI void store_rope_bwd(bf16* dst, const f32x16 (&acc)[4], float scale, const float2* cs, int hl) {
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int c = b * 32 + 8 * g + 4 * hl;
      bf16x4 oa, ob;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float a = static_cast<float>(static_cast<bf16>(acc[b][4 * g + e] * scale));
        const float bb = static_cast<float>(static_cast<bf16>(acc[b + 2][4 * g + e] * scale));
        const float2 w = cs[c + e];
        oa[e] = static_cast<bf16>(a * w.x + bb * w.y);
        ob[e] = static_cast<bf16>(bb * w.x - a * w.y);
      }
      *reinterpret_cast<bf16x4*>(dst + c) = oa;
      *reinterpret_cast<bf16x4*>(dst + c + 64) = ob;
    }
}

__global__ __launch_bounds__(stg::NTHR, 1) void swa_bwd_dq_bf16_128_k(AttnParams p) {
  using namespace stg;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5, ql = lane & 31;
  int bx, h, bz;
  attn_block(bx, h, bz);
  const int qs = bx * QT;
  const int d = p.H * HD;
  const bf16* Q = static_cast<const bf16*>(p.q);
  const bf16* G = static_cast<const bf16*>(p.dout);

  // this lane's query and its operand fragments
  const int qrow = qs + wave * 32 + ql;
  const bool qok = qrow < p.n;
  bf16x8 qf[8], gf[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    qf[ks] = g_frag8<bf16>(Q + (int64_t)qrow * p.ldq + h * HD + ks * 16 + 8 * hl, qok);
    gf[ks] = g_frag8<bf16>(G + (int64_t)qrow * p.lddo + h * HD + ks * 16 + 8 * hl, qok);
  }
  // a row past the end gets P = exp2(. - inf) = 0
  const float lse2 = qok ? p.lse[(int64_t)h * p.n + qrow] * LOG2E : INFINITY;
  const float Dq = qok ? p.D[(int64_t)h * p.n + qrow] : 0.f;
  const uint32_t wlen = (uint32_t)p.window;
  const float sc = LOG2E / sqrtf((float)HD);
  f32x16 dacc[4];
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) dacc[b][r] = 0.f;

  // key tiles of the window of this workgroup's queries, split z's run
  const int64_t first = p.pos0 + qs;
  const int64_t last = p.pos0 + min(qs + QT, p.n) - 1;
  int64_t lo = first - p.window + 1;
  if (lo < 0) lo = 0;
  const int64_t ktA = (lo / KT) * KT;
  const int nall = (int)((last - ktA) / KT) + 1;
  const int per = (nall + (int)gridDim.z - 1) / (int)gridDim.z;
  const int tb = min(nall, bz * per), te = min(nall, tb + per);

  const __amdgpu_buffer_rsrc_t rk = rsrc(p.kring, p.cap * d * 2);
  const __amdgpu_buffer_rsrc_t rv = rsrc(p.vring, p.cap * d * 2);
  const __amdgpu_buffer_rsrc_t rt = rsrc(p.ktring, (int64_t)d * p.cap * 2);
  // ring slot of the next tile to load, advanced by one tile per issue
  // (tiles never wrap: cap % 64 == 0)
  // (32-bit offsets: the launch admits rings of at most 2^31 - 1 bytes)
  uint32_t slot_next = (uint32_t)((ktA + (int64_t)tb * KT) % p.cap);
  const uint32_t ucap = (uint32_t)p.cap, ud = (uint32_t)d;
  // the next tile's buffer offsets, computed under the current tile's
  // products (prep) and used by its loads after the barrier (fire)
  uint32_t offk[PER], offt[PER];
  auto prep = [&]() {
    const uint32_t slot0 = slot_next;
    slot_next = slot_next + KT == ucap ? 0u : slot_next + KT;
    // K and V: 16 instructions of 4 rows (1 KB) each per tile
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int q = wave * PER + i;
      const int row = q * 4 + (lane >> 4), pc = lane & 15;
      const int c = pc ^ (row & 15);
      offk[i] = ((slot0 + row) * ud + h * HD + 8 * c) * 2u;
    }
    // K^T: 16 instructions of 8 rows (head dims) each
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int q = wave * PER + i;
      const int row = q * 8 + (lane >> 3), pc = lane & 7;
      const int c = pc ^ ((row >> 1) & 7);
      offt[i] = ((uint32_t)(h * HD + row) * ucap + slot0 + 8 * c) * 2u;
    }
  };
  auto fire = [&](int stage) {
    char* st = smem + stage * STAGE;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int q = wave * PER + i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(st + q * 1024), 16, offk[i], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(st + TILE_K + q * 1024), 16, offk[i], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < PER; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rt, (lds_void*)(st + 2 * TILE_K + (wave * PER + i) * 1024), 16,
                                               offt[i], 0, 0, 0);
  };

  if (tb < te) {
    prep();
    fire(0);
    prep();                                // offsets of tile tb + 1
  }
  for (int it = tb; it < te; ++it) {
    const int stage = (it - tb) & 1;
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0x0F70);    // vmcnt(0): this wave's loads of tile it
    __syncthreads();                       // every wave's; the other stage is free
    if (it + 1 < te) fire(stage ^ 1);
    const char* Ks = smem + stage * STAGE;
    const char* Vs = Ks + TILE_K;
    const char* Ts = Ks + 2 * TILE_K;
    const int64_t kt = ktA + (int64_t)it * KT;
    const bool interior = (kt + KT - 1 <= first) && (kt > last - p.window);
    // key - query of element r = 0 of this lane (key half 0)
    const int kq0 = (int)(kt - first) - (wave * 32 + ql) + 4 * hl;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 s, dp;
      const f32x16 zero = {};
      const int krow = kb * 32 + ql;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const int slot = ((2 * ks + hl) ^ (krow & 15)) * 16;
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(Ks + krow * ROWK + slot);
        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(Vs + krow * ROWK + slot);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], ks ? s : zero, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, gf[ks], ks ? dp : zero, 0, 0, 0);
      }
      // the K^T fragments of this half's dQ products: their reads run under
      // the exponentials
      bf16x8 tf[2][4];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int c = 4 * kb + 2 * hf + hl, trow = b * 32 + ql;
          tf[hf][b] = *reinterpret_cast<const bf16x8*>(Ts + trow * ROWT + ((c ^ ((trow >> 1) & 7)) * 16));
        }
      __builtin_amdgcn_sched_barrier(0);
      // outside the band S = -inf (wave-uniform test: most tiles are inside)
      if (!interior) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rel = kq0 + 32 * kb + 8 * (r >> 2) + (r & 3);
          s[r] = (uint32_t)(-rel) < wlen ? s[r] : -INFINITY;
        }
      }
      // dS^T = P (dP - D), P = exp(S - LSE)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = fast_exp2(fmaf(s[r], sc, -lse2)) * (dp[r] - Dq);
      // dQ^T += K^T dS^T: the lane's 8 k-slots of half hf are one 16-byte run
      // of the key-permuted K^T row
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        float v8[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v8[j] = s[8 * hf + j];
        const bf16x8 df = pack8<bf16>(v8);
#pragma unroll
        for (int b = 0; b < 4; ++b) mma32x32x16(tf[hf][b], df, dacc[b]);
      }
    }
    if (it + 2 < te) prep();               // offsets of tile it + 2, under these products
  }

  if (!qok) return;
  const float scale = 1.f / sqrtf((float)HD);
  if (gridDim.z == 1) {
    bf16* dst = static_cast<bf16*>(p.dq) + (int64_t)qrow * p.ldg + h * HD;
    if (p.rope_cs) {
      // dims c and c + 64 (blocks b and b + 2) are the lane's own pairs
      store_rope_bwd(dst, dacc, scale, p.rope_cs + (int64_t)qrow * (HD / 2), hl);
    } else {
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          bf16x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = static_cast<bf16>(dacc[b][4 * g + e] * scale);
          *reinterpret_cast<bf16x4*>(dst + b * 32 + 8 * g + 4 * hl) = o;
        }
    }
    return;
  }
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int c = b * 32 + 8 * g + 4 * hl;      // 4 consecutive head dims
      float4 v;
      v.x = dacc[b][4 * g] * scale; v.y = dacc[b][4 * g + 1] * scale;
      v.z = dacc[b][4 * g + 2] * scale; v.w = dacc[b][4 * g + 3] * scale;
      *reinterpret_cast<float4*>(p.part + ((int64_t)bz * p.n + qrow) * d + h * HD + c) = v;
    }
}

// --------------------------------------------- forward, bf16, head_dim 128
// The forward of swa_fwd32_k for the bf16 / head_dim 128 case with the
// staging of the dQ kernel above: 8 waves x 32 queries per workgroup, the
// 64-key tiles of K ([key][hd], rows of 256 B) and of the key-permuted V^T
// copy ([hd][key], rows of 128 B) by direct global->LDS loads into two
// stages, swizzled as there.
__global__ __launch_bounds__(stg::NTHR, 1) void swa_fwd_bf16_128_k(AttnParams p) {
  using namespace stg;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5, ql = lane & 31;
  int bx, h, bz;
  attn_block(bx, h, bz);
  const int qs = bx * QT;
  const int d = p.H * HD;
  const bf16* Q = static_cast<const bf16*>(p.q);

  const int qrow = qs + wave * 32 + ql;
  const bool qok = qrow < p.n;
  bf16x8 qf[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
    qf[ks] = g_frag8<bf16>(Q + (int64_t)qrow * p.ldq + h * HD + ks * 16 + 8 * hl, qok);
  float m = -INFINITY, l = 0.f;
  f32x16 oacc[4];
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[b][r] = 0.f;
  const uint32_t wlen = (uint32_t)p.window;
  const float sc = LOG2E / sqrtf((float)HD);

  const int64_t first = p.pos0 + qs;
  const int64_t last = p.pos0 + min(qs + QT, p.n) - 1;
  int64_t lo = first - p.window + 1;
  if (lo < 0) lo = 0;
  const int64_t ktA = (lo / KT) * KT;
  const int nall = (int)((last - ktA) / KT) + 1;
  const int per = (nall + (int)gridDim.z - 1) / (int)gridDim.z;
  const int tb = min(nall, bz * per), te = min(nall, tb + per);

  const __amdgpu_buffer_rsrc_t rk = rsrc(p.kring, p.cap * d * 2);
  const __amdgpu_buffer_rsrc_t rt = rsrc(p.vtring, (int64_t)d * p.cap * 2);
  // ring slot of the next tile to load, advanced by one tile per issue
  // (tiles never wrap: cap % 64 == 0)
  // (32-bit offsets: the launch admits rings of at most 2^31 - 1 bytes)
  uint32_t slot_next = (uint32_t)((ktA + (int64_t)tb * KT) % p.cap);
  const uint32_t ucap = (uint32_t)p.cap, ud = (uint32_t)d;
  // the next tile's buffer offsets, computed under the current tile's
  // products (prep) and used by its loads after the barrier (fire)
  uint32_t offk[PER], offt[PER];
  auto prep = [&]() {
    const uint32_t slot0 = slot_next;
    slot_next = slot_next + KT == ucap ? 0u : slot_next + KT;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int q = wave * PER + i;
      const int row = q * 4 + (lane >> 4), pc = lane & 15;
      const int c = pc ^ (row & 15);
      offk[i] = ((slot0 + row) * ud + h * HD + 8 * c) * 2u;
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int q = wave * PER + i;
      const int row = q * 8 + (lane >> 3), pc = lane & 7;
      const int c = pc ^ ((row >> 1) & 7);
      offt[i] = ((uint32_t)(h * HD + row) * ucap + slot0 + 8 * c) * 2u;
    }
  };
  auto fire = [&](int stage) {
    char* st = smem + stage * STAGE_F;
#pragma unroll
    for (int i = 0; i < PER; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(st + (wave * PER + i) * 1024), 16, offk[i], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < PER; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rt, (lds_void*)(st + TILE_K + (wave * PER + i) * 1024), 16, offt[i],
                                               0, 0, 0);
  };

  // the lane's fragment offsets within a stage: K fragment ks of key half kb
  // at ka[ks] + kb * 32 rows, V^T fragment (kb, hf) of head-dim block b at
  // va[2 * kb + hf] + b * 32 rows (the swizzle depends on the lane only)
  uint32_t ka[8], va[4];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) ka[ks] = ql * ROWK + (((2 * ks + hl) ^ (ql & 15)) * 16);
#pragma unroll
  for (int kh = 0; kh < 4; ++kh) va[kh] = TILE_K + ql * ROWT + (((2 * kh + hl) ^ ((ql >> 1) & 7)) * 16);

  if (tb < te) {
    prep();
    fire(0);
    prep();                                // offsets of tile tb + 1
  }
  for (int it = tb; it < te; ++it) {
    const int stage = (it - tb) & 1;
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0x0F70);    // vmcnt(0): this wave's loads of tile it
    __syncthreads();                       // every wave's; the other stage is free
    if (it + 1 < te) fire(stage ^ 1);
    const char* Ks = smem + stage * STAGE_F;
    const int64_t kt = ktA + (int64_t)it * KT;
    // all 16 K fragments of the tile first, then the 16 score products;
    // the registers then take the 16 V^T fragments, whose reads run under
    // the softmax arithmetic
    bf16x8 fr[16];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        fr[kb * 8 + ks] = *reinterpret_cast<const bf16x8*>(Ks + ka[ks] + kb * 32 * ROWK);
    __builtin_amdgcn_sched_barrier(0);
    f32x16 s[2];
    const f32x16 zero = {};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[kb * 8 + ks], qf[ks], ks ? s[kb] : zero, 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int b = 0; b < 4; ++b)
          fr[kb * 8 + hf * 4 + b] = *reinterpret_cast<const bf16x8*>(Ks + va[2 * kb + hf] + b * 32 * ROWT);
    __builtin_amdgcn_sched_barrier(0);
    const bool interior = (kt + KT - 1 <= first) && (kt > last - p.window);
    if (!interior) {
      const int kq0 = (int)(kt - first) - (wave * 32 + ql) + 4 * hl;   // key - query of s[0][0]
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rel = kq0 + 32 * kb + 8 * (r >> 2) + (r & 3);
          s[kb][r] = (uint32_t)(-rel) < wlen ? s[kb][r] : -INFINITY;
        }
    }
    // (IEEE maximum: one three-input instruction per two scores, and no
    // quieting of the products' outputs first, which maxnum needs)
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2)
        tmax = __builtin_elementwise_maximum(tmax, __builtin_elementwise_maximum(s[kb][r], s[kb][r + 1]));
    tmax = __builtin_elementwise_maximum(tmax, __shfl_xor(tmax, 32, 64)) * sc;
    // lazy rescaling as in swa_fwd32_k
    const bool bump = tmax > m + 8.f;
    if (__any(bump)) {
      const float mn = bump ? tmax : m;
      const float alpha = (m == -INFINITY) ? 0.f : fast_exp2(m - mn);
      l *= alpha;
#pragma unroll
      for (int b = 0; b < 4; ++b) oacc[b] *= alpha;
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
        const bf16x8 pf = pack8<bf16>(pv);
#pragma unroll
        for (int b = 0; b < 4; ++b) mma32x32x16(fr[kb * 8 + hf * 4 + b], pf, oacc[b]);
      }
    if (it + 2 < te) prep();               // offsets of tile it + 2, under these products
  }

  if (!qok) return;
  if (gridDim.z == 1) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    bf16* O = static_cast<bf16*>(p.o) + (int64_t)qrow * p.ldo + h * HD;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = static_cast<bf16>(oacc[b][4 * g + j] * inv);
        *reinterpret_cast<bf16x4*>(O + b * 32 + 8 * g + 4 * hl) = o;
      }
    if (p.lse && hl == 0) p.lse[(int64_t)h * p.n + qrow] = (m + log2f(l)) * LN2;
  } else {
    // unnormalised partial of this key range, combined by swa_combine_k
    float* O = p.part + ((int64_t)bz * p.n + qrow) * d + h * HD;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float4 v;
        v.x = oacc[b][4 * g]; v.y = oacc[b][4 * g + 1]; v.z = oacc[b][4 * g + 2]; v.w = oacc[b][4 * g + 3];
        *reinterpret_cast<float4*>(O + b * 32 + 8 * g + 4 * hl) = v;
      }
    if (hl == 0) {
      float* ml = p.part_ml + ((int64_t)bz * p.H + h) * p.n * 2;
      ml[2 * qrow] = m;
      ml[2 * qrow + 1] = l;
    }
  }
}

// --------------------------------------------------------- backward dK, dV
// Keys are the in-chunk positions; cached keys of earlier chunks are
// constants and receive no gradient.  Each wave owns 32 keys (lane = key);
// per 64-query tile: S = Q Kᵀ, dP = dO Vᵀ, then dVᵀ += dOᵀ P and dKᵀ += Qᵀ dS
// with the probabilities fed from the accumulators.
template <typename T, int HD>
__global__ __launch_bounds__(256) void swa_bwd_dkdv32_k(AttnParams p) {
  using C = Attn32<T, HD>;
  constexpr int KT_ = 128;
  __shared__ __attribute__((aligned(16))) T Qs[TQ * C::LSN];
  __shared__ __attribute__((aligned(16))) T Gs[TQ * C::LSN];
  __shared__ __attribute__((aligned(16))) T Qt[C::HDR * C::LSV];
  __shared__ __attribute__((aligned(16))) T Gt[C::HDR * C::LSV];
  __shared__ float lse_s[TQ], D_s[TQ];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, ql = lane & 31;
  int bx, h, bz;
  attn_block(bx, h, bz);
  const int ks0 = bx * KT_;
  const int d = p.H * HD;
  const T* Q = static_cast<const T*>(p.q);
  const T* G = static_cast<const T*>(p.dout);
  const T* KR = static_cast<const T*>(p.kring);
  const T* VR = static_cast<const T*>(p.vring);

  const int krow = ks0 + wave * 32 + ql;
  const bool kok = krow < p.n;
  const int64_t kpos = p.pos0 + krow;
  const int64_t kslot = (kok ? kpos : p.pos0) % p.cap;
  typename Frag<T>::type kf[C::KS], vf[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    kf[ks] = g_frag8<T>(KR + kslot * d + h * HD + ks * 16 + 8 * hl, kok);
    vf[ks] = g_frag8<T>(VR + kslot * d + h * HD + ks * 16 + 8 * hl, kok);
  }
  const float sc = LOG2E / sqrtf((float)HD);
  f32x16 dk[C::HB], dv[C::HB];
#pragma unroll
  for (int b = 0; b < C::HB; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) { dk[b][r] = 0.f; dv[b][r] = 0.f; }

  const int kmax = min(ks0 + KT_, p.n) - 1;
  const int64_t qend = min<int64_t>((int64_t)p.n - 1, (int64_t)kmax + p.window - 1);
  for (int qt = (ks0 / TQ) * TQ; qt <= qend; qt += TQ) {
    const int nvalid = min(TQ, p.n - qt);
    __syncthreads();
    tile_copy_rows<T, TQ, HD, C::LSN, 256>(Qs, Q + (int64_t)qt * p.ldq + h * HD, p.ldq, nvalid, HD, tid);
    tile_copy_rows<T, TQ, HD, C::LSN, 256>(Gs, G + (int64_t)qt * p.lddo + h * HD, p.lddo, nvalid, HD, tid);
    tile_copy_transpose<T, TQ, HD, C::LSV, 256>(Qt, Q + (int64_t)qt * p.ldq + h * HD, p.ldq, nvalid, HD, tid);
    tile_copy_transpose<T, TQ, HD, C::LSV, 256>(Gt, G + (int64_t)qt * p.lddo + h * HD, p.lddo, nvalid, HD, tid);
    if (tid < TQ) {
      const bool ok = tid < nvalid;
      lse_s[tid] = ok ? p.lse[(int64_t)h * p.n + qt + tid] * LOG2E : 0.f;
      D_s[tid] = ok ? p.D[(int64_t)h * p.n + qt + tid] : 0.f;
    }
    __syncthreads();
    f32x16 s[2], dp[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) { s[qb][r] = 0.f; dp[qb][r] = 0.f; }
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        mma32x32x16(lds_frag8<T>(Qs + (qb * 32 + ql) * C::LSN + ks * 16 + 8 * hl), kf[ks], s[qb]);
        mma32x32x16(lds_frag8<T>(Gs + (qb * 32 + ql) * C::LSN + ks * 16 + 8 * hl), vf[ks], dp[qb]);
      }
    }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qi = qb * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
        const int64_t qp = p.pos0 + qt + qi;
        const bool ok = kok && (qt + qi < p.n) && kpos <= qp && kpos > qp - p.window;
        const float pr = ok ? fast_exp2(fmaf(s[qb][r], sc, -lse_s[qi])) : 0.f;
        s[qb][r] = pr;                                 // P
        dp[qb][r] = pr * (dp[qb][r] - D_s[qi]);        // dS
      }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        float a8[8], b8[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) { a8[j] = s[qb][8 * hf + j]; b8[j] = dp[qb][8 * hf + j]; }
        const typename Frag<T>::type pf = pack8<T>(a8);
        const typename Frag<T>::type df = pack8<T>(b8);
        const int qoff = qb * 32 + 16 * hf + 4 * hl;
#pragma unroll
        for (int b = 0; b < C::HB; ++b) {
          const T* grow = Gt + (b * 32 + ql) * C::LSV + qoff;
          const T* qrow_ = Qt + (b * 32 + ql) * C::LSV + qoff;
          mma32x32x16(lds_frag4x2<T>(grow, grow + 8), pf, dv[b]);
          mma32x32x16(lds_frag4x2<T>(qrow_, qrow_ + 8), df, dk[b]);
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
      for (int r = 0; r < 16; ++r) {
        const int c = b * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
        if (c < HD) {
          DK[c] = from_f32<T>(dk[b][r] * scale);
          DV[c] = from_f32<T>(dv[b][r]);
        }
      }
  }
}

// ------------------------------------------- backward dK, dV, bf16, hd 128
// swa_bwd_dkdv32_k for the bf16 / head_dim 128 case, staged: the keys of a
// workgroup (4 waves x 32, lane = key) keep their K and V fragments in
// registers; per 64-query tile, Q and dO, their query-permuted transposes
// and the tile's LSE and D arrive by direct global->LDS loads into two
// stages (the next tile's in flight while the current one is multiplied).
// S = Q K^T and dP = dO V^T come out with lane = key, so P and dS feed
// dV^T += dO^T P and dK^T += Q^T dS straight from the accumulators, each
// transposed operand fragment one 16-byte read.
__global__ __launch_bounds__(256, 1) void swa_bwd_dkdv_bf16_128_k(AttnParams p) {
  using namespace stg;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5, ql = lane & 31;
  int bx, h, bz;
  attn_block(bx, h, bz);
  const int ks0 = bx * KB_;
  const int d = p.H * HD;
  const bf16* KR = static_cast<const bf16*>(p.kring);
  const bf16* VR = static_cast<const bf16*>(p.vring);

  const int kw = ks0 + wave * 32;              // this wave's first key (chunk row)
  const int krow = kw + ql;
  const bool kok = krow < p.n;
  const int64_t kslot = (p.pos0 + (kok ? krow : 0)) % p.cap;
  bf16x8 kf[8], vf[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    kf[ks] = g_frag8<bf16>(KR + kslot * d + h * HD + ks * 16 + 8 * hl, kok);
    vf[ks] = g_frag8<bf16>(VR + kslot * d + h * HD + ks * 16 + 8 * hl, kok);
  }
  const float sc = LOG2E / sqrtf((float)HD);
  const uint32_t wlen = (uint32_t)p.window;
  f32x16 dk[4], dv[4];
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) { dk[b][r] = 0.f; dv[b][r] = 0.f; }

  // query tiles: from the first key on, up to the last query the last key
  // reaches (chunk rows; the window may end before the chunk does)
  const int kmax = min(ks0 + KB_, p.n) - 1;
  const int qend = (int)min<int64_t>((int64_t)p.n - 1, (int64_t)kmax + p.window - 1);
  const int qt0 = (ks0 / QTL) * QTL;
  const int ntile = qend >= qt0 ? (qend - qt0) / QTL + 1 : 0;

  const __amdgpu_buffer_rsrc_t rq = rsrc(p.q, (int64_t)p.n * p.ldq * 2);
  const __amdgpu_buffer_rsrc_t rg = rsrc(p.dout, (int64_t)p.n * p.lddo * 2);
  const __amdgpu_buffer_rsrc_t rqt = rsrc(p.qtr, (int64_t)d * p.ldtr * 2);
  const __amdgpu_buffer_rsrc_t rgt = rsrc(p.gtr, (int64_t)d * p.ldtr * 2);
  const __amdgpu_buffer_rsrc_t rl = rsrc(p.lse + (int64_t)h * p.n, (int64_t)p.n * 4);
  const __amdgpu_buffer_rsrc_t rd = rsrc(p.D + (int64_t)h * p.n, (int64_t)p.n * 4);
  auto issue = [&](int t, int stage) {
    const int qt = qt0 + t * QTL;
    char* st = smem + stage * STAGE_B;
    // Q, dO: 16 instructions of 4 rows each, 4 per wave; rows past n read 0
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = wave * 4 + i;
      const int row = q * 4 + (lane >> 4), pc = lane & 15;
      const int c = pc ^ (row & 15);
      const uint32_t oq = (uint32_t)(((int64_t)(qt + row) * p.ldq + h * HD + 8 * c) * 2);
      const uint32_t og = (uint32_t)(((int64_t)(qt + row) * p.lddo + h * HD + 8 * c) * 2);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (lds_void*)(st + q * 1024), 16, oq, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rg, (lds_void*)(st + TILE_Q + q * 1024), 16, og, 0, 0, 0);
    }
    // Q^T, dO^T: 16 instructions of 8 rows (head dims) each, 4 per wave
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = wave * 4 + i;
      const int row = q * 8 + (lane >> 3), pc = lane & 7;
      const int c = pc ^ ((row >> 1) & 7);
      const uint32_t off = (uint32_t)((((int64_t)(h * HD + row)) * p.ldtr + qt + 8 * c) * 2);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rqt, (lds_void*)(st + 2 * TILE_Q + q * 1024), 16, off, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rgt, (lds_void*)(st + 2 * TILE_Q + TILE_QT + q * 1024), 16, off, 0, 0, 0);
    }
    // LSE and D of the tile (4 bytes per lane); past n they read 0
    char* ld = st + 2 * TILE_Q + 2 * TILE_QT;
    if (wave == 0) __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (lds_void*)ld, 4, (uint32_t)(qt + lane) * 4u, 0, 0, 0);
    if (wave == 1) __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (lds_void*)(ld + QTL * 4), 4, (uint32_t)(qt + lane) * 4u, 0, 0, 0);
  };

  if (ntile > 0) issue(0, 0);
  for (int t = 0; t < ntile; ++t) {
    const int stage = t & 1;
    __builtin_amdgcn_s_waitcnt(0x0F70);    // vmcnt(0): this wave's loads of tile t
    __syncthreads();                       // every wave's; the other stage is free
    if (t + 1 < ntile) issue(t + 1, stage ^ 1);
    const char* Qs = smem + stage * STAGE_B;
    const char* Gs = Qs + TILE_Q;
    const char* Qts = Qs + 2 * TILE_Q;
    const char* Gts = Qts + TILE_QT;
    const float* lse_s = reinterpret_cast<const float*>(Qts + 2 * TILE_QT);
    const float* D_s = lse_s + QTL;
    const int qt = qt0 + t * QTL;
    // every (query, key) pair of the tile inside the band, every query < n
    const bool interior = qt + QTL - 1 < p.n && qt >= kw + 31 && qt + QTL - 1 - kw < p.window;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      f32x16 s, dp;
      const f32x16 zero = {};
      const int qr = qb * 32 + ql;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const int slot = ((2 * ks + hl) ^ (qr & 15)) * 16;
        const bf16x8 qf = *reinterpret_cast<const bf16x8*>(Qs + qr * ROWK + slot);
        const bf16x8 gf = *reinterpret_cast<const bf16x8*>(Gs + qr * ROWK + slot);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf, kf[ks], ks ? s : zero, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(gf, vf[ks], ks ? dp : zero, 0, 0, 0);
      }
      // element r: query qb*32 + 8(r/4) + 4hl + r%4 of the tile, key krow
      if (!interior) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qi = qb * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
          const int rel = qt + qi - krow;                       // query - key
          const bool ok = (uint32_t)rel < wlen && qt + qi < p.n;
          s[r] = ok ? s[r] : -INFINITY;
        }
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 l4 = *reinterpret_cast<const float4*>(lse_s + qb * 32 + 8 * g + 4 * hl);
        const float4 d4 = *reinterpret_cast<const float4*>(D_s + qb * 32 + 8 * g + 4 * hl);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          const float pr = fast_exp2(fmaf(s[r], sc, -lv[e] * LOG2E));
          s[r] = pr;                                   // P
          dp[r] = pr * (dp[r] - dv4[e]);               // dS
        }
      }
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        float a8[8], b8[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) { a8[j] = s[8 * hf + j]; b8[j] = dp[8 * hf + j]; }
        const bf16x8 pf = pack8<bf16>(a8);
        const bf16x8 df = pack8<bf16>(b8);
        const int c = 4 * qb + 2 * hf + hl;    // the lane's 8 queries in the permuted rows
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int trow = b * 32 + ql;
          const int off = trow * (QTL * 2) + ((c ^ ((trow >> 1) & 7)) * 16);
          const bf16x8 gt = *reinterpret_cast<const bf16x8*>(Gts + off);
          const bf16x8 qtf = *reinterpret_cast<const bf16x8*>(Qts + off);
          dv[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(gt, pf, dv[b], 0, 0, 0);
          dk[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qtf, df, dk[b], 0, 0, 0);
        }
      }
    }
  }
  if (!kok) return;
  const float scale = 1.f / sqrtf((float)HD);
  bf16* DK = static_cast<bf16*>(p.dk) + (int64_t)krow * p.ldg + h * HD;
  bf16* DV = static_cast<bf16*>(p.dv) + (int64_t)krow * p.ldg + h * HD;
  if (p.rope_cs) store_rope_bwd(DK, dk, scale, p.rope_cs + (int64_t)krow * (HD / 2), hl);
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int c = b * 32 + 8 * g + 4 * hl;        // 4 consecutive head dims
      bf16x4 ok4, ov4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ok4[e] = static_cast<bf16>(dk[b][4 * g + e] * scale);
        ov4[e] = static_cast<bf16>(dv[b][4 * g + e]);
      }
      if (!p.rope_cs) *reinterpret_cast<bf16x4*>(DK + c) = ok4;
      *reinterpret_cast<bf16x4*>(DV + c) = ov4;
    }
}

// Key-range splits for launches too small to fill the GPU (the per-chunk
// calls).  The GPU runs 512 of these workgroups at once (two per CU), so a
// launch of wgs * z workgroups takes ceil(wgs * z / 512) rounds for 1/z of
// the work each: pick z in [1, zmax] with the fewest rounds per unit of
// work, the smaller z on ties (each split adds a combine pass).  Measured on
// the 3B chunk shape (192 workgroups): dQ 527 us at z = 3, 372 us at z = 8;
// the forward 208 us at z = 3, 179 us at z = 2.
inline int pick_split(const AttnParams& p, int wgs, int zmax) {
  if (!p.part || !p.part_ml) return 1;
  if (zmax > p.max_split) zmax = p.max_split;
  int best = 1;
  double cost = 1e30;
  for (int z = 1; z <= zmax; ++z) {
    const double c = (double)((wgs * z + 511) / 512) / z;
    if (c < cost - 1e-9) { cost = c; best = z; }
  }
  return best;
}

// Key-range split of the staged kernels (one resident workgroup per CU, 256
// slots).  A run of t key tiles costs about t + 4 tile-times (fragment loads
// and pipeline fill), rounds of resident workgroups add up, and each split
// beyond the first adds a combine pass over the fp32 partials of about 4
// tile-times (measured on 1024-query chunks, 24 heads, window 8192).  The
// run length is that of the last workgroup, which spans the most keys.
inline int pick_split_staged(const AttnParams& p) {
  if (!p.part || !p.part_ml) return 1;
  const int wgs = ((p.n + stg::QT - 1) / stg::QT) * p.H;
  const int64_t qlast = p.pos0 + p.n - 1;
  const int64_t qfirst = std::max<int64_t>(p.pos0, qlast - stg::QT + 1);
  const int64_t klo = std::max<int64_t>(0, qfirst - p.window + 1);
  const double tiles = (double)((qlast - (klo / stg::KT) * stg::KT) / stg::KT + 1);
  int best = 1;
  double cost = 1e30;
  for (int z = 1; z <= p.max_split && z <= 8; ++z) {
    const double c = (double)((wgs * z + 255) / 256) * (tiles / z + 4.0) + (z > 1 ? 4.0 * z : 0.0);
    if (c < cost - 1e-9) { cost = c; best = z; }
  }
  return best;
}
// bf16, head_dim 128, ring of whole 64-slot tiles addressable by 32-bit
// buffer offsets: the staged kernels
template <typename T>
bool staged_ok(const AttnParams& p) {
  return std::is_same<T, bf16>::value && p.hd == 128 && p.cap % 64 == 0 &&
         (int64_t)p.cap * p.H * p.hd * 2 <= 0x7fffffff;
}

template <typename T>
void fwd_t(const AttnParams& p, hipStream_t s) {
  if (staged_ok<T>(p)) {
    const int nz = pick_split_staged(p);
    static bool attr = false;
    if (!attr) {
      (void)hipFuncSetAttribute((const void*)swa_fwd_bf16_128_k, hipFuncAttributeMaxDynamicSharedMemorySize,
                                stg::LDS_F);
      attr = true;
    }
    hipLaunchKernelGGL(swa_fwd_bf16_128_k, dim3((p.n + stg::QT - 1) / stg::QT, p.H, nz), dim3(stg::NTHR),
                       stg::LDS_F, s, p);
    if (nz > 1) {
      const int tot = p.n * p.H * p.hd;
      hipLaunchKernelGGL(swa_combine_k<T>, dim3((tot + 255) / 256), dim3(256), 0, s, p, nz);
    }
    return;
  }
  const int nz = pick_split(p, ((p.n + 127) / 128) * p.H, 4);
  dim3 grid((p.n + 127) / 128, p.H, nz);
  switch (p.hd) {
    case 16: hipLaunchKernelGGL((swa_fwd32_k<T, 16>), grid, dim3(256), 0, s, p); break;
    case 32: hipLaunchKernelGGL((swa_fwd32_k<T, 32>), grid, dim3(256), 0, s, p); break;
    case 64: hipLaunchKernelGGL((swa_fwd32_k<T, 64>), grid, dim3(256), 0, s, p); break;
    case 96: hipLaunchKernelGGL((swa_fwd32_k<T, 96>), grid, dim3(256), 0, s, p); break;
    case 128: hipLaunchKernelGGL((swa_fwd32_k<T, 128>), grid, dim3(256), 0, s, p); break;
    default: return;
  }
  if (nz > 1) {
    const int tot = p.n * p.H * p.hd;
    hipLaunchKernelGGL(swa_combine_k<T>, dim3((tot + 255) / 256), dim3(256), 0, s, p, nz);
  }
}
template <typename T>
int bwd_t(const AttnParams& p, hipStream_t s, hipStream_t s2) {
  // bf16 / head_dim 128 / 64-aligned ring: the staged 256-query dQ kernel
  // (one workgroup per CU: 256 resident workgroups); otherwise the general one
  const bool wide = staged_ok<T>(p);
  int nz;
  if (wide) {
    nz = pick_split_staged(p);
    static bool attr = false;
    if (!attr) {
      (void)hipFuncSetAttribute((const void*)swa_bwd_dq_bf16_128_k, hipFuncAttributeMaxDynamicSharedMemorySize,
                                stg::LDS_BYTES);
      attr = true;
    }
    hipLaunchKernelGGL(swa_bwd_dq_bf16_128_k, dim3((p.n + stg::QT - 1) / stg::QT, p.H, nz), dim3(stg::NTHR),
                       stg::LDS_BYTES, s, p);
  } else {
    nz = pick_split(p, ((p.n + 127) / 128) * p.H, 8);
  }
  dim3 gq((p.n + 127) / 128, p.H, nz);
  dim3 gk((p.n + 127) / 128, p.H);
  // the staged dK/dV kernel also needs the transposed Q and dO
  const bool wide_kv = wide && p.qtr && p.gtr && p.ldtr % 64 == 0 && p.ldtr >= ((p.n + 63) / 64) * 64 &&
                       (int64_t)(p.n + 64) * std::max(p.ldq, p.lddo) * 2 <= 0x7fffffff &&
                       (int64_t)p.H * p.hd * p.ldtr * 2 <= 0x7fffffff;
  if (wide_kv) {
    static bool attr = false;
    if (!attr) {
      (void)hipFuncSetAttribute((const void*)swa_bwd_dkdv_bf16_128_k, hipFuncAttributeMaxDynamicSharedMemorySize,
                                stg::LDS_B);
      attr = true;
    }
    hipLaunchKernelGGL(swa_bwd_dkdv_bf16_128_k, dim3((p.n + stg::KB_ - 1) / stg::KB_, p.H), dim3(256),
                       stg::LDS_B, s2, p);
  }
  switch (p.hd) {
#define CASE(HDV) case HDV: \
    if (!wide) hipLaunchKernelGGL((swa_bwd_dq32_k<T, HDV>), gq, dim3(256), 0, s, p); \
    if (!wide_kv) hipLaunchKernelGGL((swa_bwd_dkdv32_k<T, HDV>), gk, dim3(256), 0, s2, p); break;
    CASE(16) CASE(32) CASE(64) CASE(96) CASE(128)
#undef CASE
    default: return 0;
  }
  int rotated = 0;
  if (nz > 1) {
    const int tot = p.n * p.H * p.hd / (p.rope_cs ? 2 : 1);
    hipLaunchKernelGGL(dq_combine_k<T>, dim3((tot + 255) / 256), dim3(256), 0, s, p, nz);
    if (p.rope_cs) rotated |= 1;
  } else if (wide && p.rope_cs) {
    rotated |= 1;
  }
  if (wide_kv && p.rope_cs) rotated |= 2;
  return rotated;
}

}  // namespace

void swa_fwd(const AttnParams& p, bool bf, hipStream_t s) {
  if (p.n <= 0) return;
  if (bf) fwd_t<bf16>(p, s); else fwd_t<float>(p, s);
}

int swa_bwd(const AttnParams& p, bool bf, hipStream_t s, hipStream_t s_kv) {
  if (p.n <= 0) return 0;
  return bf ? bwd_t<bf16>(p, s, s_kv) : bwd_t<float>(p, s, s_kv);
}

bool swa_bwd_reads_transposes(int hd, bool bf) { return bf && hd == stg::HD; }

}  // namespace ttt
