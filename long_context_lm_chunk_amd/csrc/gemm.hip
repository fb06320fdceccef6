// Tiled matrix-core GEMM for gfx950 with fused epilogues.
//
//   C[M,N] = sum_k A[m,k] * B[n,k]
//
// A is given either k-contiguous ([M][K] row-major) or m-contiguous
// ([K][M] row-major); B either k-contiguous ([N][K]) or n-contiguous
// ([K][N]).  Both are staged in LDS k-contiguous, so one compute loop serves
// the forward products (y = x W), the input-gradient products (dx = dy W^T)
// and the weight-gradient products (dW = x^T dy, reduction over tokens).
//
// Workgroup tile 128x128, 4 waves in 2x2, each wave 64x64 = 4x4 blocks of
// 16x16 matrix-core accumulators; K staged 128 bytes per step (64 bf16 or
// 32 fp32) with a double-buffered LDS tile and register prefetch.
//
// Epilogues (fused so that intermediate products never round-trip HBM):
//   STORE   out = acc                              (T or fp32)
//   RESID   out_f32 = resid_f32 + acc              (residual stream)
//   GELU    z = acc, act = gelu_erf(acc)
//   SWIGLU  columns come in blocks of 16 gate / 16 up; z = acc,
//           act = silu(gate) * up
//   SGD     delta_f32 -= lr * acc ; delta copy = round(delta) ;
//           current = round(W0 + delta)                    (fast weights)
//   CESTAT  per-row partial max / sum(exp) of the logits and the target logit;
//           with C set, also the logits (fp32)
//   CEGRAD  g = (softmax - onehot(target)) / n_targets, rows without a target 0
//   ACTBWD  d(pre-activation) from the product d(act) and the saved Z
#include "common.hpp"
#include "kernels.hpp"
#include <type_traits>

namespace ttt {

namespace {

constexpr int BM = 128, BN = 128, NT = 256;

template <typename T> struct GemmCfg {
  static constexpr int BK = 128 / sizeof(T);      // 64 bf16, 32 fp32
  static constexpr int PAD = 16 / sizeof(T);
  static constexpr int LS = BK + PAD;             // LDS row stride (elements)
  static constexpr int V = Vec16<T>::N;
};

// Register-staged loader for one operand tile (rows x BK), reading through
// a buffer resource: 32-bit offsets instead of 64-bit addresses, and
// elements outside the matrix get an out-of-range offset, for which the
// hardware returns zero (no branches around the loads).
constexpr uint32_t OOB = 0x80000000u;

DEVI __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes > 0x7fffffff ? 0x7fffffff : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}
DEVI U128 bload(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  U128 u; u.w[0] = v[0]; u.w[1] = v[1]; u.w[2] = v[2]; u.w[3] = v[3];
  return u;
}

template <typename T, bool KC, int ROWS> struct TileLoader {
  using C = GemmCfg<T>;
  static constexpr int V = C::V;
  // k-contiguous: ROWS*BK/V vectors; m-contiguous: (ROWS/V)*(BK/4) groups of 4 vectors
  static constexpr int NV = KC ? (ROWS * C::BK / V) / NT : 4 * ((ROWS / V) * (C::BK / 4)) / NT;
  U128 r[NV];

  DEVI void load(__amdgpu_buffer_rsrc_t rs, int64_t ld, int row0, int row_lim, int k0, int K, int tid) {
    const uint32_t ldb = (uint32_t)ld * (uint32_t)sizeof(T);
    if constexpr (KC) {
      constexpr int VPR = C::BK / V;
#pragma unroll
      for (int it = 0; it < NV; ++it) {
        int idx = it * NT + tid;
        int rr = idx / VPR, c = (idx % VPR) * V;
        bool ok = (row0 + rr < row_lim) && (k0 + c < K);
        const uint32_t off = (uint32_t)(row0 + rr) * ldb + (uint32_t)(k0 + c) * (uint32_t)sizeof(T);
        r[it] = bload(rs, ok ? off : OOB);
      }
    } else {
      constexpr int KB = C::BK / 4;
#pragma unroll
      for (int it = 0; it < NV / 4; ++it) {
        int idx = it * NT + tid;
        int kb = idx % KB, mv = idx / KB;
        int m = row0 + mv * V, k = k0 + kb * 4;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          bool ok = (k + q < K) && (m < row_lim);
          const uint32_t off = (uint32_t)(k + q) * ldb + (uint32_t)m * (uint32_t)sizeof(T);
          r[it * 4 + q] = bload(rs, ok ? off : OOB);
        }
      }
    }
  }

  DEVI void store(T* __restrict__ lds, int tid) const {
    if constexpr (KC) {
      constexpr int VPR = C::BK / V;
#pragma unroll
      for (int it = 0; it < NV; ++it) {
        int idx = it * NT + tid;
        int rr = idx / VPR, c = (idx % VPR) * V;
        st128(lds + rr * C::LS + c, r[it]);
      }
    } else {
      // k-groups fastest across lanes: a wave's transposed 8-byte LDS
      // writes then spread over the banks instead of colliding 8 ways
      constexpr int KB = C::BK / 4;
#pragma unroll
      for (int it = 0; it < NV / 4; ++it) {
        int idx = it * NT + tid;
        int kb = idx % KB, mv = idx / KB;
        int m0 = mv * V, k0 = kb * 4;
#pragma unroll
        for (int e = 0; e < V; ++e) {
          T t4[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) t4[q] = elem<T>(r[it * 4 + q], e);
          T* dst = lds + (m0 + e) * C::LS + k0;
          if constexpr (sizeof(T) == 2) {
            uint2 w;
            w.x = (uint32_t)__builtin_bit_cast(uint16_t, t4[0]) | ((uint32_t)__builtin_bit_cast(uint16_t, t4[1]) << 16);
            w.y = (uint32_t)__builtin_bit_cast(uint16_t, t4[2]) | ((uint32_t)__builtin_bit_cast(uint16_t, t4[3]) << 16);
            *reinterpret_cast<uint2*>(dst) = w;
          } else {
            float4 w; w.x = t4[0]; w.y = t4[1]; w.z = t4[2]; w.w = t4[3];
            *reinterpret_cast<float4*>(dst) = w;
          }
        }
      }
    }
  }
};

template <typename T> DEVI void store4(T* p, const float4& v);
template <> DEVI void store4<float>(float* p, const float4& v) { *reinterpret_cast<float4*>(p) = v; }
template <> DEVI void store4<bf16>(bf16* p, const float4& v) {
  bf16x4 b;
  b[0] = static_cast<bf16>(v.x); b[1] = static_cast<bf16>(v.y);
  b[2] = static_cast<bf16>(v.z); b[3] = static_cast<bf16>(v.w);
  *reinterpret_cast<bf16x4*>(p) = b;
}
// The same with the non-temporal hint, for data that no kernel reads again
// soon (the residual stream's read-modify-write, the fast weights' master,
// copies and transposed copies rewritten by the SGD epilogue): the caches
// keep the products' operand tiles instead (+1.2% prefill against plain
// accesses everywhere; plain stores are kept for outputs the next kernel
// reads, where the hint on every store gained only a quarter of that).
template <typename T> DEVI void store4nt(T* p, const float4& v);
template <> DEVI void store4nt<float>(float* p, const float4& v) {
  const f32x4 t = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(t, reinterpret_cast<f32x4*>(p));
}
template <> DEVI void store4nt<bf16>(bf16* p, const float4& v) {
  bf16x4 b;
  b[0] = static_cast<bf16>(v.x); b[1] = static_cast<bf16>(v.y);
  b[2] = static_cast<bf16>(v.z); b[3] = static_cast<bf16>(v.w);
  __builtin_nontemporal_store(b, reinterpret_cast<bf16x4*>(p));
}
template <typename T> DEVI float4 load4nt(const T* p);
template <> DEVI float4 load4nt<float>(const float* p) {
  const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  return make_float4(t.x, t.y, t.z, t.w);
}
template <> DEVI float4 load4nt<bf16>(const bf16* p) {
  const bf16x4 b = __builtin_nontemporal_load(reinterpret_cast<const bf16x4*>(p));
  return make_float4(static_cast<float>(b[0]), static_cast<float>(b[1]), static_cast<float>(b[2]),
                     static_cast<float>(b[3]));
}
template <typename T> DEVI float4 load4(const T* p);
template <> DEVI float4 load4<float>(const float* p) { return *reinterpret_cast<const float4*>(p); }
template <> DEVI float4 load4<bf16>(const bf16* p) {
  const bf16x4 b = *reinterpret_cast<const bf16x4*>(p);
  float4 v; v.x = static_cast<float>(b[0]); v.y = static_cast<float>(b[1]);
  v.z = static_cast<float>(b[2]); v.w = static_cast<float>(b[3]);
  return v;
}

DEVI float gelu_erf(float z) { return 0.5f * z * (1.f + erff(z * 0.70710678118654752f)); }
DEVI float silu(float z) { return z / (1.f + __expf(-z)); }

// Epilogue over an fp32 tile staged in LDS: rows [0, nr) x cols [0, nc) of
// st (row pitch ES floats) are output rows row0.. and columns n0.. .  Every
// thread takes runs of 4 consecutive columns (16-byte fp32 / 8-byte bf16
// vector accesses).  With a K split (gridDim.z > 1) the raw partial goes to
// slab z of split_ws instead.
template <int EPI, typename TO>
DEVI void epi_apply(const GemmParams& p, float* st, int ES, int nr, int nc, int row0, int n0,
                    int tid, int nthr) {
  if (gridDim.z > 1) {
    float* slab = p.split_ws + (int64_t)blockIdx.z * p.M * p.N;
#pragma unroll 4
    for (int g = tid; g < nr * (nc / 4); g += nthr) {
      const int r = g / (nc / 4), c = (g % (nc / 4)) * 4;
      const int row = row0 + r, col = n0 + c;
      if (row >= p.M || col >= p.N) continue;
      *reinterpret_cast<float4*>(slab + (int64_t)row * p.N + col) =
          *reinterpret_cast<const float4*>(st + r * ES + c);
    }
    return;
  }
  if constexpr (EPI == EPI_SGD) {
    // delta -= lr * acc (fp32 master C, row-major), its storage-type copy C2;
    // the current weight W0 + delta goes back into the staged tile and then
    // out transposed to C3[col][row] in runs of 4 rows (the input-gradient
    // products read it as a k-contiguous operand).  Groups are taken four at
    // a time with every load issued before any store (the stores to the
    // master could otherwise alias the next group's loads and serialise them).
    constexpr int U = 4;
    const int total = nr * (nc / 4);
    for (int g0 = tid; g0 < total; g0 += U * nthr) {
      float4 v[U], w[U], w0[U];
      int64_t ci[U];
      bool ok[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int g = g0 + u * nthr;
        const int r = g / (nc / 4), c = (g % (nc / 4)) * 4;
        const int row = row0 + r, col = n0 + c;
        ok[u] = g < total && row < p.M && col < p.N;
        ci[u] = (int64_t)row * p.ldc + col;
        if (ok[u]) {
          v[u] = *reinterpret_cast<const float4*>(st + r * ES + c);
          w[u] = *reinterpret_cast<const float4*>(static_cast<const float*>(p.C) + ci[u]);
          if (p.C3) w0[u] = load4<TO>(static_cast<const TO*>(p.W0) + ci[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (!ok[u]) continue;
        const int g = g0 + u * nthr;
        const int r = g / (nc / 4), c = (g % (nc / 4)) * 4;
        const int row = row0 + r, col = n0 + c;
        float4 x = w[u];
        x.x -= p.alpha * v[u].x; x.y -= p.alpha * v[u].y; x.z -= p.alpha * v[u].z; x.w -= p.alpha * v[u].w;
        *reinterpret_cast<float4*>(static_cast<float*>(p.C) + ci[u]) = x;
        if (p.C2) store4<TO>(static_cast<TO*>(p.C2) + (int64_t)row * p.ldc2 + col, x);
        if (p.C3) {
          float4 cur;
          cur.x = w0[u].x + x.x; cur.y = w0[u].y + x.y; cur.z = w0[u].z + x.z; cur.w = w0[u].w + x.w;
          *reinterpret_cast<float4*>(st + r * ES + c) = cur;
        }
      }
    }
    if (p.C3) {
      __syncthreads();
  #pragma unroll 4
    for (int g = tid; g < nc * (nr / 4); g += nthr) {
        const int c = g / (nr / 4), r = (g % (nr / 4)) * 4;
        const int row = row0 + r, col = n0 + c;
        if (row >= p.M || col >= p.N) continue;
        TO* dst = static_cast<TO*>(p.C3) + (int64_t)col * p.ldc3 + row;
        if (row + 3 < p.M) {
          float4 v;
          v.x = st[r * ES + c]; v.y = st[(r + 1) * ES + c]; v.z = st[(r + 2) * ES + c]; v.w = st[(r + 3) * ES + c];
          store4<TO>(dst, v);
        } else {
          for (int e = 0; row + e < p.M; ++e) dst[e] = from_f32<TO>(st[(r + e) * ES + c]);
        }
      }
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    // columns: gate block 32c..32c+15, up block 32c+16..32c+31 -> act 16c..16c+15
#pragma unroll 4
    for (int g = tid; g < nr * (nc / 8); g += nthr) {
      const int r = g / (nc / 8), q = g % (nc / 8);      // q: 4-wide group of act columns
      const int row = row0 + r;
      const int cg = (q / 4) * 32 + (q % 4) * 4;          // gate column in the tile
      if (row >= p.M || n0 + cg >= p.N) continue;   // N % 32 == 0: gate in => up in
      const float4 gv = *reinterpret_cast<const float4*>(st + r * ES + cg);
      const float4 uv = *reinterpret_cast<const float4*>(st + r * ES + cg + 16);
      if (p.C) {                                    // pre-activations kept (for a backward)
        TO* z = static_cast<TO*>(p.C) + (int64_t)row * p.ldc + n0;
        store4<TO>(z + cg, gv);
        store4<TO>(z + cg + 16, uv);
      }
      float4 a;
      a.x = silu(gv.x) * uv.x; a.y = silu(gv.y) * uv.y; a.z = silu(gv.z) * uv.z; a.w = silu(gv.w) * uv.w;
      store4<TO>(static_cast<TO*>(p.C2) + (int64_t)row * p.ldc2 + n0 / 2 + (q / 4) * 16 + (q % 4) * 4, a);
    }
  } else {
#pragma unroll 4
    for (int g = tid; g < nr * (nc / 4); g += nthr) {
      const int r = g / (nc / 4), c = (g % (nc / 4)) * 4;
      const int row = row0 + r, col = n0 + c;
      if (row >= p.M || col >= p.N) continue;         // N is a multiple of 4
      const float4 v = *reinterpret_cast<const float4*>(st + r * ES + c);
      const int64_t ci = (int64_t)row * p.ldc + col;
      if constexpr (EPI == EPI_STORE) {
        store4<TO>(static_cast<TO*>(p.C) + ci, v);
      } else if constexpr (EPI == EPI_RESID) {
        const float4 rr = load4nt<float>(p.R + (int64_t)row * p.ldr + col);
        float4 o; o.x = rr.x + v.x; o.y = rr.y + v.y; o.z = rr.z + v.z; o.w = rr.w + v.w;
        store4nt<float>(static_cast<float*>(p.C) + ci, o);
      } else if constexpr (EPI == EPI_GELU) {
        if (p.C) store4<TO>(static_cast<TO*>(p.C) + ci, v);   // pre-activations kept (for a backward)
        float4 a; a.x = gelu_erf(v.x); a.y = gelu_erf(v.y); a.z = gelu_erf(v.z); a.w = gelu_erf(v.w);
        store4<TO>(static_cast<TO*>(p.C2) + (int64_t)row * p.ldc2 + col, a);
      } else if constexpr (EPI == EPI_ACTBWD) {
        // v = d(act) of activations col..col+3 (four of one 16-block)
        const TO* z = static_cast<const TO*>(p.Z) + (int64_t)row * p.ldz;
        TO* dz = static_cast<TO*>(p.C) + (int64_t)row * p.ldc;
        if (p.act_swiglu) {
          const int cg = (col / 16) * 32 + (col % 16);
          const float4 g = load4<TO>(z + cg), u = load4<TO>(z + cg + 16);
          float4 dg, du;
          swiglu_bwd(v.x, g.x, u.x, dg.x, du.x);
          swiglu_bwd(v.y, g.y, u.y, dg.y, du.y);
          swiglu_bwd(v.z, g.z, u.z, dg.z, du.z);
          swiglu_bwd(v.w, g.w, u.w, dg.w, du.w);
          store4<TO>(dz + cg, dg);
          store4<TO>(dz + cg + 16, du);
        } else {
          const float4 zz = load4<TO>(z + col);
          float4 o;
          o.x = gelu_bwd(zz.x, v.x); o.y = gelu_bwd(zz.y, v.y); o.z = gelu_bwd(zz.z, v.z); o.w = gelu_bwd(zz.w, v.w);
          store4<TO>(dz + col, o);
        }
      } else if constexpr (EPI == EPI_CEGRAD) {
        float4 gq = {0.f, 0.f, 0.f, 0.f};
        if (row < p.n_tgt) {
          const float l = p.lse[row];
          const int t = p.tgt[row];
          gq.x = __expf(v.x - l) - (col == t ? 1.f : 0.f);
          gq.y = __expf(v.y - l) - (col + 1 == t ? 1.f : 0.f);
          gq.z = __expf(v.z - l) - (col + 2 == t ? 1.f : 0.f);
          gq.w = __expf(v.w - l) - (col + 3 == t ? 1.f : 0.f);
          gq.x *= p.alpha; gq.y *= p.alpha; gq.z *= p.alpha; gq.w *= p.alpha;
        }
        store4<TO>(static_cast<TO*>(p.C) + ci, gq);
      }
    }
  }
}

template <typename T, bool A_KC, bool B_KC, int EPI, typename TO, bool DUAL>
__global__ __launch_bounds__(NT, 2) void gemm_kernel(GemmParams p) {
  using C = GemmCfg<T>;
  __shared__ __attribute__((aligned(16))) T lds[2][(BM + BN) * C::LS];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const T* __restrict__ A = static_cast<const T*>(p.A);
  const T* __restrict__ B = static_cast<const T*>(p.B);

  TileLoader<T, A_KC, BM> la;
  TileLoader<T, B_KC, BN> lb;

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // With DUAL the reduction runs twice over K, against B then B2: the fast
  // weights are applied as W0 + delta without rounding their sum.  With a
  // split (gridDim.z > 1) this workgroup takes one contiguous run of the
  // k-tiles and writes an fp32 partial for gemm_reduce_k.
  const int nk1 = (p.K + C::BK - 1) / C::BK;
  const int ntot = DUAL ? 2 * nk1 : nk1;
  const int per = (ntot + (int)gridDim.z - 1) / (int)gridDim.z;
  const int kt_begin = min(ntot, (int)blockIdx.z * per);
  const int kt_end = min(ntot, kt_begin + per);
  const T* __restrict__ B2 = static_cast<const T*>(p.B2);
  // matrix extents in bytes for the buffer resources
  const int64_t abytes = (A_KC ? (int64_t)p.M * p.lda : (int64_t)p.K * p.lda) * (int64_t)sizeof(T);
  const int64_t bbytes = (B_KC ? (int64_t)p.N * p.ldb : (int64_t)p.K * p.ldb) * (int64_t)sizeof(T);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, abytes);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(B, bbytes);
  const __amdgpu_buffer_rsrc_t rb2 = make_rsrc(DUAL ? (const void*)B2 : (const void*)B, bbytes);
  auto load = [&](int t) {
    const bool second = DUAL && t >= nk1;
    const int k0 = (second ? t - nk1 : t) * C::BK;
    la.load(ra, p.lda, m0, p.M, k0, p.K, tid);
    lb.load(second ? rb2 : rb, p.ldb, n0, p.N, k0, p.K, tid);
  };
  if (kt_begin < kt_end) {
    load(kt_begin);
    la.store(lds[0], tid);
    lb.store(lds[0] + BM * C::LS, tid);
  }
  __syncthreads();

  for (int kt = kt_begin; kt < kt_end; ++kt) {
    const int cur = (kt - kt_begin) & 1;
    if (kt + 1 < kt_end) load(kt + 1);
    const T* As = lds[cur];
    const T* Bs = lds[cur] + BM * C::LS;
    // fragments of k-step ks + 1 read between the products of k-step ks
    typename Frag<T>::type af[2][4], bfr[2][4];
    auto rd = [&](int ks, int b) {
      const int kk = ks * 32 + 8 * (lane >> 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) af[b][i] = lds_frag8<T>(As + (wm * 64 + i * 16 + (lane & 15)) * C::LS + kk);
#pragma unroll
      for (int j = 0; j < 4; ++j) bfr[b][j] = lds_frag8<T>(Bs + (wn * 64 + j * 16 + (lane & 15)) * C::LS + kk);
    };
    rd(0, 0);
#pragma unroll
    for (int ks = 0; ks < C::BK / 32; ++ks) {
      const int b = ks & 1;
      if (ks + 1 < C::BK / 32) rd(ks + 1, b ^ 1);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) mma16x16x32(af[b][i], bfr[b][j], acc[i][j]);
      if (ks + 1 < C::BK / 32) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (kt + 1 < kt_end) {
      la.store(lds[cur ^ 1], tid);
      lb.store(lds[cur ^ 1] + BM * C::LS, tid);
    }
    __syncthreads();
  }

  // ---------------------------------------------------------------- epilogue
  const int rbase = m0 + wm * 64 + 4 * (lane >> 4);
  const int cbase = n0 + wn * 64 + (lane & 15);

  if constexpr (EPI == EPI_CESTAT) {
    // rows = tokens, cols = vocab; partial (max, sumexp) of this wave's 64
    // columns, plus the target logit where the target falls in them.
    const int* tgt = p.tgt;
    const int part = blockIdx.x * 2 + wn;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = rbase + i * 16 + e;
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = cbase + j * 16;
          if (col < p.N) mx = fmaxf(mx, acc[i][j][e]);
        }
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
        float s = 0.f;
        float tv = 0.f;
        bool has = false;
        const int t = (row < p.n_tgt) ? tgt[row] : -1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = cbase + j * 16;
          if (col < p.N) s += __expf(acc[i][j][e] - mx);
          if (col == t) { tv = acc[i][j][e]; has = true; }
          // the logits themselves, for the gradient pass (optional)
          if (p.C && row < p.M && col < p.N) static_cast<float*>(p.C)[(int64_t)row * p.ldc + col] = acc[i][j][e];
        }
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) s += __shfl_xor(s, o, 64);
        if (row < p.M) {
          if ((lane & 15) == 0) {
            p.part_max[(int64_t)part * p.ldpart + row] = mx;
            p.part_sum[(int64_t)part * p.ldpart + row] = s;
          }
          if (has) p.tgt_logit[row] = tv;
        }
      }
    }
    return;
  } else {
    // Stage the 128x128 fp32 tile through LDS (the operand buffers are free
    // after the last barrier of the main loop), then let every thread apply
    // the epilogue to runs of 4 consecutive columns with 16-byte (fp32) or
    // 8-byte (bf16) vector accesses instead of the scattered per-element
    // stores of the matrix-core layout.
    constexpr int ES = BN + 4;                         // fp32 row pitch in LDS
    static_assert(BM * ES * 4 <= 2 * (BM + BN) * C::LS * (int)sizeof(T), "epilogue tile fits");
    float* st = reinterpret_cast<float*>(&lds[0][0]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          st[(wm * 64 + i * 16 + 4 * (lane >> 4) + e) * ES + wn * 64 + j * 16 + (lane & 15)] = acc[i][j][e];
    __syncthreads();
    epi_apply<EPI, TO>(p, st, ES, BM, BN, m0, n0, tid, NT);
  }
}

// Sum of the split-K slabs in a fixed order (deterministic), then the
// STORE or RESID epilogue.
template <int EPI, typename TO>
__global__ void gemm_reduce_k(GemmParams p, int nz) {
  const int64_t g = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;   // 4-column groups
  const int64_t total = (int64_t)p.M * (p.N / 4);
  if (g >= total) return;
  const int row = (int)(g / (p.N / 4)), col = (int)(g % (p.N / 4)) * 4;
  float4 v = *reinterpret_cast<const float4*>(p.split_ws + (int64_t)row * p.N + col);
  for (int z = 1; z < nz; ++z) {
    const float4 w = load4nt<float>(p.split_ws + ((int64_t)z * p.M + row) * p.N + col);
    v.x += w.x; v.y += w.y; v.z += w.z; v.w += w.w;
  }
  const int64_t ci = (int64_t)row * p.ldc + col;
  if constexpr (EPI == EPI_RESID) {
    const float4 r = *reinterpret_cast<const float4*>(p.R + (int64_t)row * p.ldr + col);
    v.x += r.x; v.y += r.y; v.z += r.z; v.w += r.w;
    *reinterpret_cast<float4*>(static_cast<float*>(p.C) + ci) = v;
  } else {
    store4<TO>(static_cast<TO*>(p.C) + ci, v);
    if (p.rd_D) {
      // rowsum over a head of rd_o times the stored values: the head's
      // rd_hd / 4 threads are consecutive lanes of one wave
      const float4 o = load4<TO>(static_cast<const TO*>(p.rd_o) + ci);
      float t = o.x * to_f32(from_f32<TO>(v.x)) + o.y * to_f32(from_f32<TO>(v.y)) +
                o.z * to_f32(from_f32<TO>(v.z)) + o.w * to_f32(from_f32<TO>(v.w));
      const int lanes = p.rd_hd / 4;
      for (int m = lanes / 2; m > 0; m >>= 1) t += __shfl_xor(t, m, 64);
      if (((col / 4) & (lanes - 1)) == 0) p.rd_D[(int64_t)(col / p.rd_hd) * p.M + row] = t;
    }
  }
}

// ---------------------------------------------------------------------------
// Large-tile core for bf16 operands that are both k-contiguous (the forward
// products and everything else of the form C = A B^T with A [M][K], B [N][K]).
//
// Workgroup tile 256x256, eight waves in 2x4 (two per SIMD, so one wave's
// barrier and load issue hide behind the other's products), each wave
// 128x64 = 4x2 blocks of 32x32 accumulators (v_mfma_f32_32x32x16_bf16).
// K advances 64 per stage through two 64 KB stages filled by direct
// global->LDS 16-byte loads (buffer_load ... lds: no staging registers;
// out-of-range rows and columns read as zero).  A 1 KB wave load covers 8
// rows of 128 contiguous bytes, whole cache lines: with 32-wide stages
// (64-byte row pieces, four 32 KB stages) the same bytes took twice the
// address work, the vector-memory address and command queues were full
// most of the time (rocprof's SQ_VMEM_TA_ADDR_FIFO_FULL 27x hipBLASLt's on
// the same product) and the products ran 4-8% slower on the 3B shapes
// (2.4% in the prefill).
// Every stage slot issues the same number of loads (past the end of K they
// read zeros into a slot nobody uses), so the wait for a stage is a fixed
// vmcnt.  LDS rows are 128 bytes; 16-byte chunk c of row r sits at slot
// c ^ ((r >> 1) & 7): the 16 lanes of one LDS read pass (16 consecutive
// rows, one chunk) then hit 16 distinct 16-byte bank groups.
namespace big {
constexpr int BM = 256, BN = 256, BK = 64, NS = 2;   // two 64-wide k stages
constexpr int WM = 2, WN = 4, NW = WM * WN, NT = 64 * NW;   // 8 waves, 2 per SIMD
constexpr int TM = BM / WM, TN = BN / WN;    // wave tile 128 x 64
constexpr int FI = TM / 32, FJ = TN / 32;    // 32x32 accumulator blocks per wave (4 x 2)
constexpr int ROWB = BK * 2;                 // bytes per LDS row
constexpr int STAGE_A = BM * ROWB;
constexpr int STAGE = (BM + BN) * ROWB;
constexpr int LDS_BYTES = NS * STAGE;        // 128 KB of the 160 KB per CU
constexpr int CHUNKS = ROWB / 16;            // 16-byte chunks per LDS row
constexpr int RPL = 64 / CHUNKS;             // rows per 1 KB wave load
constexpr int SLAB_LOADS = BM / RPL / NW;    // 1 KB loads per wave per operand slab
constexpr int LOADS = 2 * SLAB_LOADS;        // per wave per stage
static_assert(NW * 32 * (BN / WN + 4) * 4 <= LDS_BYTES, "per-wave epilogue areas fit");
// slot of 16-byte chunk c of row r: c ^ swz(r), so that the 16 lanes of one
// LDS read pass (16 consecutive rows, one chunk) hit 16 distinct 16-byte
// bank groups
DEVI int swz(int r) { return (r >> 1) & 7; }
// s_waitcnt immediates with vmcnt n (expcnt and lgkmcnt not waited for)
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }
static_assert((NS - 1) * LOADS < 64, "vmcnt range");
typedef __attribute__((address_space(3))) void lds_void;

// The loads of one 256-row operand slab (rows row0.., k k0..k0+BK-1) into
// LDS: wave instructions of 1 KB (RPL rows), SLAB_LOADS per wave.  The
// buffer offsets are computed first (slab_offsets, out of OOB past the
// operand's rows or K) and the loads issued later (slab_fire), so that the
// address arithmetic can run under the products before the stage barrier.
DEVI void slab_offsets(uint32_t ldb, int row0, int rows, int k0, int K, int wave, int lane,
                       uint32_t (&off)[SLAB_LOADS]) {
  const int rl = lane / CHUNKS, p = lane % CHUNKS;
#pragma unroll
  for (int i = 0; i < SLAB_LOADS; ++i) {
    const int blk = wave * SLAB_LOADS + i;              // RPL-row block of the slab
    const int r = blk * RPL + rl;                       // row within the slab
    const int c = p ^ swz(r);                           // logical chunk at slot p
    const int k = k0 + 8 * c;
    const bool ok = row0 + r < rows && k < K;
    off[i] = ok ? (uint32_t)(row0 + r) * ldb + (uint32_t)k * 2u : OOB;
  }
}
DEVI void slab_fire(__amdgpu_buffer_rsrc_t rs, const uint32_t (&off)[SLAB_LOADS], char* dst, int wave) {
#pragma unroll
  for (int i = 0; i < SLAB_LOADS; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + (wave * SLAB_LOADS + i) * 1024), 16, off[i],
                                             0, 0, 0);
}
}  // namespace big

template <int EPI, typename TO, bool DUAL>
__global__ __launch_bounds__(big::NT, 1) void gemm256_kernel(GemmParams p) {
  constexpr int BM = big::BM, BN = big::BN, BK = big::BK, NT = big::NT, NS = big::NS, ROWB = big::ROWB;
  constexpr int STAGE_A = big::STAGE_A, STAGE = big::STAGE;
  constexpr int TM = big::TM, TN = big::TN, FI = big::FI, FJ = big::FJ, WN = big::WN;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  // Workgroups are dealt to the 8 XCDs round-robin; give each XCD a
  // contiguous run of tiles, walked in groups of GM tile rows (column-major
  // inside a group), so the ~32 workgroups an XCD runs at once cover a
  // 4 x 8 patch of tiles and share 4 A slabs and 8 B slabs in its L2.
  constexpr int GM = 4;
  const int tm = (p.M + BM - 1) / BM, tn = (p.N + BN - 1) / BN, ntile = tm * tn;
  const int b = blockIdx.x, x = b & 7, y = b >> 3;
  const int q8 = ntile >> 3, r8 = ntile & 7;
  const int t = x * q8 + min(x, r8) + y;
  const int grp = t / (GM * tn), first = grp * GM, gm = min(tm - first, GM);
  const int tl = t - grp * GM * tn;
  const int m0 = (first + tl % gm) * BM, n0 = (tl / gm) * BN;

  f32x16 acc[FI][FJ];
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int nk1 = (p.K + BK - 1) / BK;
  const int ntot = DUAL ? 2 * nk1 : nk1;
  const int per = (ntot + (int)gridDim.z - 1) / (int)gridDim.z;
  const int kt_begin = min(ntot, (int)blockIdx.z * per);
  const int kt_end = min(ntot, kt_begin + per);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A, (int64_t)p.M * p.lda * 2);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.B, (int64_t)p.N * p.ldb * 2);
  const __amdgpu_buffer_rsrc_t rb2 = make_rsrc(DUAL ? p.B2 : p.B, (int64_t)p.N * p.ldb * 2);
  const uint32_t lda = (uint32_t)p.lda * 2u, ldb = (uint32_t)p.ldb * 2u;
  // k-tile kt into ring slot kt % NS; past kt_end the loads read zeros
  typedef uint32_t Offs[big::SLAB_LOADS];
  auto prep = [&](int kt, Offs& oa, Offs& ob) {
    const bool live = kt < kt_end;
    const bool second = DUAL && kt >= nk1;
    const int k0 = live ? (second ? kt - nk1 : kt) * BK : p.K;
    big::slab_offsets(lda, m0, p.M, k0, p.K, wave, lane, oa);
    big::slab_offsets(ldb, n0, p.N, k0, p.K, wave, lane, ob);
  };
  auto fire = [&](int kt, const Offs& oa, const Offs& ob) {
    const bool second = DUAL && kt >= nk1;
    char* st = smem + ((unsigned)(kt - kt_begin) % NS) * STAGE;
    big::slab_fire(ra, oa, st, wave);
    big::slab_fire(second ? rb2 : rb, ob, st + STAGE_A, wave);
  };
  auto fire_a = [&](int kt, const Offs& oa) {
    big::slab_fire(ra, oa, smem + ((unsigned)(kt - kt_begin) % NS) * STAGE, wave);
  };
  auto fire_b = [&](int kt, const Offs& ob) {
    const bool second = DUAL && kt >= nk1;
    big::slab_fire(second ? rb2 : rb, ob, smem + ((unsigned)(kt - kt_begin) % NS) * STAGE + STAGE_A, wave);
  };
  auto issue = [&](int kt) {
    Offs oa, ob;
    prep(kt, oa, ob);
    fire(kt, oa, ob);
  };
  // fragment addressing: lane reads row (l & 31) of a 32-row block, logical
  // chunk 2*ks + (l >> 5), at slot chunk ^ ((row >> 2) & 3) = chunk ^ ((l >> 2) & 3)
  const int frow = lane & 31, fsw = big::swz(frow), fhi = lane >> 5;
  const int abase = (wm * TM + frow) * ROWB, bbase = STAGE_A + (wn * TN + frow) * ROWB;
  auto frags = [&](int kt, int ks, bf16x8 (&a)[FI], bf16x8 (&b)[FJ]) {
    const char* st = smem + ((unsigned)(kt - kt_begin) % NS) * STAGE;
    const int slot = ((2 * ks + fhi) ^ fsw) * 16;
#pragma unroll
    for (int i = 0; i < FI; ++i) a[i] = *reinterpret_cast<const bf16x8*>(st + abase + i * 32 * ROWB + slot);
#pragma unroll
    for (int j = 0; j < FJ; ++j) b[j] = *reinterpret_cast<const bf16x8*>(st + bbase + j * 32 * ROWB + slot);
  };
  bf16x8 fa0[FI], fb0[FJ], fa1[FI], fb1[FJ];
  // products of one k-step on (a, b) with the fragment reads of the next
  // (issued by the caller just before) interleaved one per product, and the
  // VL vector loads of a later stage among the first products
  auto kstep = [&](const bf16x8 (&a)[FI], const bf16x8 (&b)[FJ], auto vl) {
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
      for (int j = 0; j < FJ; ++j) mma32x32x16(a[i], b[j], acc[i][j]);
#pragma unroll
    for (int u = 0; u < FI + FJ; ++u) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (u < decltype(vl)::value) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, FI * FJ - (FI + FJ), 0);
    __builtin_amdgcn_sched_barrier(0);
  };
  using none = std::integral_constant<int, 0>;
  using all = std::integral_constant<int, big::LOADS>;
  using half = std::integral_constant<int, big::SLAB_LOADS>;
  // Two 64-wide stages, four k-steps each.  Fragments run one k-step
  // ahead of the products, across the stage border: the reads of
  // (kt + 1, 0) go out during the products of (kt, 3).  So before that
  // k-step stage kt + 1 must be complete in LDS (this wave's loads:
  // vmcnt 0; every wave's: the barrier), and every wave must be done
  // reading stage kt (lgkmcnt 0, then the barrier), whose slot then takes
  // stage kt + 2: its A slab's loads go out between the products of
  // (kt, 3), its B slab's between those of (kt + 1, 0), so that the
  // vector-memory queues see them spread over two k-steps (with all eight
  // loads in one k-step, the address queue was full 10-15% of the time;
  // spread, the products run 1-6% faster on the 3B shapes and the prefill
  // 1.8%), and both have landed by the barrier of stage kt + 1.
  // Each 1 KB load covers 8 rows of 128 contiguous bytes (whole cache
  // lines: half the address work per byte of 64-byte rows), and one
  // barrier serves four k-steps.
  if (kt_begin < kt_end) {
    issue(kt_begin);
    issue(kt_begin + 1);
    __builtin_amdgcn_s_waitcnt(big::vmcnt_imm(big::LOADS));     // stage kt_begin
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    frags(kt_begin, 0, fa0, fb0);
  }
  Offs obp;                              // B offsets of the stage whose B loads are still to go out
  bool bpend = false;
  for (int kt = kt_begin; kt < kt_end; ++kt) {
    Offs oa, ob;
    prep(kt + 2, oa, ob);                // address arithmetic under these products
    frags(kt, 1, fa1, fb1);
    if (bpend) {
      fire_b(kt + 1, obp);
      kstep(fa0, fb0, half());
    } else {
      kstep(fa0, fb0, none());
    }
    frags(kt, 2, fa0, fb0);
    kstep(fa1, fb1, none());
    frags(kt, 3, fa1, fb1);
    kstep(fa0, fb0, none());
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0): stage kt + 1 in, stage kt read
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    fire_a(kt + 2, oa);
    frags(kt + 1, 0, fa0, fb0);          // past the end: zeros, unused
    kstep(fa1, fb1, half());
#pragma unroll
    for (int i = 0; i < big::SLAB_LOADS; ++i) obp[i] = ob[i];
    bpend = true;
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);      // vmcnt(0): the zero-fill loads past the end
  __syncthreads();                         // all waves done with the operand stages

  if constexpr (EPI == EPI_SGD) {
    // Each wave updates its own 128 x 64 block, 32 rows at a time, through a
    // private LDS area: no workgroup barrier, every load of a 32-row part in
    // flight at once, and the accumulators of a part are free once staged.
    constexpr int P = TN + 4;                          // row pitch (floats)
    float* ws = reinterpret_cast<float*>(smem) + wave * 32 * P;
    const int cbase = n0 + wn * TN;
#pragma unroll
    for (int i = 0; i < FI; ++i) {
      const int rbase = m0 + wm * TM + i * 32;
#pragma unroll
      for (int j = 0; j < FJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) ws[(8 * (r >> 2) + 4 * fhi + (r & 3)) * P + j * 32 + frow] = acc[i][j][r];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // 32 rows x 16 groups of 4 columns = 512 groups, 8 per lane, all loaded first
      float4 v[8], w[8], w0[8];
      bool ok[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int g = u * 64 + lane, r = g >> 4, c = (g & 15) * 4;
        const int row = rbase + r, col = cbase + c;
        ok[u] = row < p.M && col < p.N;
        if (ok[u]) {
          const int64_t ci = (int64_t)row * p.ldc + col;
          v[u] = *reinterpret_cast<const float4*>(ws + r * P + c);
          w[u] = load4nt<float>(static_cast<const float*>(p.C) + ci);
          w0[u] = load4nt<TO>(static_cast<const TO*>(p.W0) + ci);
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (!ok[u]) continue;
        const int g = u * 64 + lane, r = g >> 4, c = (g & 15) * 4;
        const int row = rbase + r, col = cbase + c;
        const int64_t ci = (int64_t)row * p.ldc + col;
        float4 x = w[u];
        x.x -= p.alpha * v[u].x; x.y -= p.alpha * v[u].y; x.z -= p.alpha * v[u].z; x.w -= p.alpha * v[u].w;
        store4nt<float>(static_cast<float*>(p.C) + ci, x);
        if (p.C2) store4nt<TO>(static_cast<TO*>(p.C2) + (int64_t)row * p.ldc2 + col, x);
        float4 cur;
        cur.x = w0[u].x + x.x; cur.y = w0[u].y + x.y; cur.z = w0[u].z + x.z; cur.w = w0[u].w + x.w;
        *reinterpret_cast<float4*>(ws + r * P + c) = cur;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // transposed current weights: 64 columns x 8 groups of 4 rows, 8 per lane
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int g = u * 64 + lane, c = g >> 3, r = (g & 7) * 4;
        const int row = rbase + r, col = cbase + c;
        if (row >= p.M || col >= p.N) continue;
        TO* dst = static_cast<TO*>(p.C3) + (int64_t)col * p.ldc3 + row;
        if (row + 3 < p.M) {
          float4 t;
          t.x = ws[r * P + c]; t.y = ws[(r + 1) * P + c]; t.z = ws[(r + 2) * P + c]; t.w = ws[(r + 3) * P + c];
          store4nt<TO>(dst, t);
        } else {
          for (int e = 0; row + e < p.M; ++e) dst[e] = from_f32<TO>(ws[(r + e) * P + c]);
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  } else if constexpr (EPI == EPI_CESTAT) {
    // rows = tokens, cols = vocab: per row the (max, sum of exp) of each
    // 64-column group (partial index col / 64, as in the 128x128 core), the
    // target logit where the target falls in the group, and (when C is set)
    // the logits themselves for the gradient pass.  Each wave stages its
    // 128 x 64 block 32 rows at a time; two lanes per row then take 32
    // columns each.
    constexpr int P = TN + 4;
    float* ws = reinterpret_cast<float*>(smem) + wave * 32 * P;
    const int cb = n0 + wn * TN;
    const int part = cb / 64;
    const int sr = lane >> 1, sh = lane & 1;
#pragma unroll
    for (int i = 0; i < FI; ++i) {
      const int rbase = m0 + wm * TM + i * 32;
#pragma unroll
      for (int j = 0; j < FJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) ws[(8 * (r >> 2) + 4 * fhi + (r & 3)) * P + j * 32 + frow] = acc[i][j][r];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      if (p.C) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int g = u * 64 + lane, r = g >> 4, c = (g & 15) * 4;
          const int row = rbase + r, col = cb + c;
          if (row >= p.M || col >= p.N) continue;
          float* dst = static_cast<float*>(p.C) + (int64_t)row * p.ldc + col;
          const float4 v = *reinterpret_cast<const float4*>(ws + r * P + c);
          if (col + 3 < p.N) {
            *reinterpret_cast<float4*>(dst) = v;
          } else {
            dst[0] = v.x;
            if (col + 1 < p.N) dst[1] = v.y;
            if (col + 2 < p.N) dst[2] = v.z;
          }
        }
      }
      const int row = rbase + sr;
      const float* wr = ws + sr * P + sh * 32;
      const int c1 = cb + sh * 32;
      float mx = -INFINITY;
#pragma unroll
      for (int c = 0; c < 32; ++c)
        if (c1 + c < p.N) mx = fmaxf(mx, wr[c]);
      mx = fmaxf(mx, __shfl_xor(mx, 1, 64));
      float sm = 0.f;
      const int t = (row < p.n_tgt) ? p.tgt[row] : -1;
#pragma unroll
      for (int c = 0; c < 32; ++c)
        if (c1 + c < p.N) sm += __expf(wr[c] - mx);
      sm += __shfl_xor(sm, 1, 64);
      if (row < p.M) {
        // the partial arrays hold 2 * ceil(N / 128) groups (the 128x128
        // core's count): the groups past N up to there read (-inf, 0)
        if (sh == 0 && part < 2 * ((p.N + 127) / 128)) {
          p.part_max[(int64_t)part * p.ldpart + row] = mx;
          p.part_sum[(int64_t)part * p.ldpart + row] = sm;
        }
        if (t >= c1 && t < c1 + 32 && t < p.N) p.tgt_logit[row] = wr[t - c1];
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  } else {
    // The other epilogues the same way: each wave applies it to its own
    // 128 x 64 block, 32 rows at a time, staged in a private LDS area.
    constexpr int P = TN + 4;
    float* ws = reinterpret_cast<float*>(smem) + wave * 32 * P;
#pragma unroll
    for (int i = 0; i < FI; ++i) {
#pragma unroll
      for (int j = 0; j < FJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) ws[(8 * (r >> 2) + 4 * fhi + (r & 3)) * P + j * 32 + frow] = acc[i][j][r];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      epi_apply<EPI, TO>(p, ws, P, 32, TN, m0 + wm * TM + i * 32, n0 + wn * TN, lane, 64);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
}

// The reduction pass's parameters: its rowsum option (rd_D) is kept for a
// STORE whose head lane groups line up, and then reported done.
template <int EPI>
GemmParams reduce_params(const GemmParams& p) {
  GemmParams q = p;
  const int lanes = p.rd_hd / 4;
  const bool ok = EPI == EPI_STORE && p.rd_D && p.rd_o && lanes > 0 && lanes <= 64 &&
                  (lanes & (lanes - 1)) == 0 && (p.N / 4) % lanes == 0;
  if (!ok) q.rd_D = nullptr;
  else if (p.rd_done) *p.rd_done = 1;
  return q;
}

// A split STORE or RESID whose caller takes the partial slabs itself
// (split_defer set): report the slab count, skip the reduction.
template <int EPI, typename TO>
bool defer_split(const GemmParams& p, int nz) {
  if ((EPI != EPI_STORE && EPI != EPI_RESID) || !p.split_defer) return false;
  *p.split_defer = nz;
  return true;
}

// The 256x256 core takes bf16 A [M][K] and B [N][K] with 16-byte aligned
// rows; split K when there are too few tiles for the 256 CUs.
template <int EPI, typename TO>
bool launch_big(const GemmParams& p, hipStream_t s) {
  if (p.K % 8 || p.lda % 8 || p.ldb % 8) return false;
  if ((int64_t)p.M * p.lda * 2 > 0x7fffffff || (int64_t)p.N * p.ldb * 2 > 0x7fffffff) return false;
  const int tiles = ((p.N + big::BN - 1) / big::BN) * ((p.M + big::BM - 1) / big::BM);
  int nz = 1;
  if constexpr (EPI == EPI_STORE || EPI == EPI_RESID) {
    const int ktiles = ((p.K + big::BK - 1) / big::BK) * (p.B2 ? 2 : 1);
    if (p.split_ws && tiles < 192 && ktiles >= 8) {
      nz = (256 + tiles - 1) / tiles;
      if (nz > ktiles / 4) nz = ktiles / 4;
      if (nz > 4) nz = 4;
      if ((int64_t)nz * p.M * p.N > p.split_cap || p.N % 4) nz = 1;
    }
  }
  static bool attr_done[2][8][2] = {};
  auto go = [&](auto kern, bool dual) {
    bool& done = attr_done[dual][EPI][sizeof(TO) == 4];
    if (!done) {
      (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, big::LDS_BYTES);
      done = true;
    }
    hipLaunchKernelGGL(kern, dim3(tiles, 1, nz), dim3(big::NT), big::LDS_BYTES, s, p);
  };
  if (p.B2) go(gemm256_kernel<EPI, TO, true>, true);
  else go(gemm256_kernel<EPI, TO, false>, false);
  if constexpr (EPI == EPI_STORE || EPI == EPI_RESID) {
    if (defer_split<EPI, TO>(p, nz)) return true;
    if (nz > 1) {
      const int64_t groups = (int64_t)p.M * (p.N / 4);
      hipLaunchKernelGGL((gemm_reduce_k<EPI, TO>), dim3((unsigned)((groups + 255) / 256)), dim3(256), 0, s,
                         reduce_params<EPI>(p), nz);
    }
  }
  return true;
}

// Which core runs the bf16 k-contiguous products: the 256x256 core, for
// every epilogue it has.  Alone, on grids of fewer than ~1024 of its tiles
// with short reductions, the 128x128 core (two workgroups per CU) fills
// the CUs more evenly and is as fast or faster; in a prefill, where the
// products of several streams share the GPU, the larger tiles' fewer
// operand re-reads per flop win (measured against the 128x128 core for
// those products: +0.5%, and +0.06% more for the activation-backward
// products, +0.5% for the cross-entropy statistics).  The 128x128 core
// keeps the fp32 products and the other operand layouts.
int g_gemm_core = GEMM_CORE_AUTO;

template <typename T, bool AK, bool BK_, int EPI, typename TO>
void launch_t(const GemmParams& p, hipStream_t s) {
  if constexpr (std::is_same<T, bf16>::value && AK && BK_ &&
                (EPI == EPI_STORE || EPI == EPI_RESID || EPI == EPI_GELU || EPI == EPI_SWIGLU ||
                 EPI == EPI_SGD || EPI == EPI_ACTBWD || EPI == EPI_CESTAT)) {
    const bool want = g_gemm_core != GEMM_CORE_SMALL;
    if (want && launch_big<EPI, TO>(p, s)) return;
  }
  const int tiles = ((p.N + BN - 1) / BN) * ((p.M + BM - 1) / BM);
  int nz = 1;
  if constexpr (EPI == EPI_STORE || EPI == EPI_RESID) {
    // Too few tiles to give every CU two workgroups, and a long reduction:
    // split K so that ~2 workgroups per CU run, each with >= 8 k-tiles.
    const int ktiles = ((p.K + GemmCfg<T>::BK - 1) / GemmCfg<T>::BK) * (p.B2 ? 2 : 1);
    if (p.split_ws && tiles < 256 && ktiles >= 16) {
      nz = (512 + tiles - 1) / tiles;
      if (nz > ktiles / 8) nz = ktiles / 8;
      if (nz > 4) nz = 4;
      if ((int64_t)nz * p.M * p.N > p.split_cap || p.N % 4) nz = 1;
    }
  }
  dim3 grid((p.N + BN - 1) / BN, (p.M + BM - 1) / BM, nz);
  if (p.B2) hipLaunchKernelGGL((gemm_kernel<T, AK, BK_, EPI, TO, true>), grid, dim3(NT), 0, s, p);
  else hipLaunchKernelGGL((gemm_kernel<T, AK, BK_, EPI, TO, false>), grid, dim3(NT), 0, s, p);
  if constexpr (EPI == EPI_STORE || EPI == EPI_RESID) {
    if (defer_split<EPI, TO>(p, nz)) return;
  }
  if constexpr (EPI == EPI_STORE || EPI == EPI_RESID) {
    if (nz > 1) {
      const int64_t groups = (int64_t)p.M * (p.N / 4);
      hipLaunchKernelGGL((gemm_reduce_k<EPI, TO>), dim3((unsigned)((groups + 255) / 256)), dim3(256), 0, s,
                         reduce_params<EPI>(p), nz);
    }
  }
}

template <typename T>
int dispatch(const GemmParams& p, bool a_kc, bool b_kc, int epi, bool out_f32, hipStream_t s) {
  // The instantiations used by the inner loop.
  if (a_kc && b_kc) {
    switch (epi) {
      case EPI_STORE:
        if (out_f32) launch_t<T, true, true, EPI_STORE, float>(p, s);
        else launch_t<T, true, true, EPI_STORE, T>(p, s);
        return 0;
      case EPI_RESID: launch_t<T, true, true, EPI_RESID, float>(p, s); return 0;
      case EPI_GELU: launch_t<T, true, true, EPI_GELU, T>(p, s); return 0;
      case EPI_SWIGLU: launch_t<T, true, true, EPI_SWIGLU, T>(p, s); return 0;
      case EPI_CESTAT: launch_t<T, true, true, EPI_CESTAT, float>(p, s); return 0;
      case EPI_CEGRAD: launch_t<T, true, true, EPI_CEGRAD, T>(p, s); return 0;
      case EPI_ACTBWD: launch_t<T, true, true, EPI_ACTBWD, T>(p, s); return 0;
      case EPI_SGD: if (p.B2) return -1; launch_t<T, true, true, EPI_SGD, T>(p, s); return 0;
      default: return -1;
    }
  }
  if (a_kc && !b_kc) {
    if (epi != EPI_STORE) return -1;
    if (out_f32) launch_t<T, true, false, EPI_STORE, float>(p, s);
    else launch_t<T, true, false, EPI_STORE, T>(p, s);
    return 0;
  }
  if (!a_kc && !b_kc) {
    if (epi != EPI_SGD || p.B2) return -1;
    launch_t<T, false, false, EPI_SGD, T>(p, s);
    return 0;
  }
  return -1;
}

// Matrix-core throughput probe: every wave issues `iters` rounds of eight
// independent 32x32x16 bf16 products on register operands (no memory
// traffic), then writes its accumulators so nothing is optimised away.
// Wave 0 of block 0 also reads the shader-clock and the 100 MHz real-time
// counters around its loop, giving the clock the products ran at.
__global__ __launch_bounds__(256) void mfma_peak_k(int iters, float* out, int64_t* clk) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = static_cast<bf16>(0.001f * (float)(lane + j));
    b[j] = static_cast<bf16>(0.002f * (float)(lane - j));
  }
  f32x16 acc[8];
#pragma unroll
  for (int u = 0; u < 8; ++u)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[u][r] = 0.f;
  const bool timer = blockIdx.x == 0 && threadIdx.x == 0;
  int64_t t0 = 0, r0 = 0;
  if (timer) { t0 = __builtin_amdgcn_s_memtime(); r0 = __builtin_amdgcn_s_memrealtime(); }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[u], 0, 0, 0);
  }
  float sum = 0.f;
#pragma unroll
  for (int u = 0; u < 8; ++u)
#pragma unroll
    for (int r = 0; r < 16; ++r) sum += acc[u][r];
  out[blockIdx.x * blockDim.x + threadIdx.x] = sum;
  if (timer) {
    const int64_t t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
    clk[0] = t1 - t0;
    clk[1] = r1 - r0;
  }
}

}  // namespace

int gemm_core(int mode) {
  const int prev = g_gemm_core;
  if (mode == GEMM_CORE_AUTO || mode == GEMM_CORE_BIG || mode == GEMM_CORE_SMALL) g_gemm_core = mode;
  return prev;
}

void mfma_peak(int blocks, int iters, float* out, int64_t* clk, hipStream_t s) {
  hipLaunchKernelGGL(mfma_peak_k, dim3(blocks), dim3(256), 0, s, iters, out, clk);
}

int gemm(const GemmParams& p, bool bf16_operands, bool a_kc, bool b_kc, int epi, bool out_f32,
         hipStream_t s) {
  if (p.M <= 0 || p.N <= 0) return 0;
  // Operands are read through buffer resources (32-bit byte offsets, range
  // at most 2^31 - 1 bytes): refuse larger ones instead of reading zeros.
  const int64_t es = bf16_operands ? 2 : 4;
  const int64_t abytes = (a_kc ? (int64_t)p.M : (int64_t)p.K) * p.lda * es;
  const int64_t bbytes = (b_kc ? (int64_t)p.N : (int64_t)p.K) * p.ldb * es;
  if (abytes > 0x7fffffff || bbytes > 0x7fffffff) return GEMM_TOO_LARGE;
  return bf16_operands ? dispatch<bf16>(p, a_kc, b_kc, epi, out_f32, s)
                       : dispatch<float>(p, a_kc, b_kc, epi, out_f32, s);
}

}  // namespace ttt
