// Shared device-side building blocks for the gfx950 (CDNA4) kernels.
//
// Matrix-core convention used by every kernel here: one "16x16x32 step"
// C[16x16] += A[16x32] * B[32x16] executed by one 64-lane wavefront.
//   lane l holds A[row = l%16][kslot = 8*(l/16) + j], j = 0..7
//   lane l holds B[kslot = 8*(l/16) + j][col = l%16]
//   accumulator c[i] = C[row = 4*(l/16) + i][col = l%16], i = 0..3
// bf16 operands map to one v_mfma_f32_16x16x32_bf16; fp32 operands (the
// float32 check mode) map to eight v_mfma_f32_16x16x4_f32, sub-step j taking
// k-slot 8*(l/16)+j from lane group l/16.  Because the reduction runs over
// all k-slots, any consistent assignment of k indices to k-slots in A and B
// gives the same product; the kernels use that freedom to feed softmax
// probabilities straight from an accumulator into the next product.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

#define DEVI __device__ __forceinline__

template <typename T> struct Frag;
template <> struct Frag<bf16> { typedef bf16x8 type; };
template <> struct Frag<float> { typedef f32x8 type; };

DEVI void mma16x16x32(const bf16x8& a, const bf16x8& b, f32x4& c) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
DEVI void mma16x16x32(const f32x8& a, const f32x8& b, f32x4& c) {
#pragma unroll
  for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], c, 0, 0, 0);
}

// 32x32x16 step: lane l holds A[row l%32][kslot 8*(l/32)+j], B[kslot
// 8*(l/32)+j][col l%32]; accumulator c[r] = C[8*(r/4) + 4*(l/32) + r%4][l%32].
typedef float f32x16 __attribute__((ext_vector_type(16)));
DEVI void mma32x32x16(const bf16x8& a, const bf16x8& b, f32x16& c) {
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
DEVI void mma32x32x16(const f32x8& a, const f32x8& b, f32x16& c) {
#pragma unroll
  for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[j], b[j], c, 0, 0, 0);
}

template <typename T> DEVI T from_f32(float x);
template <> DEVI float from_f32<float>(float x) { return x; }
template <> DEVI bf16 from_f32<bf16>(float x) { return static_cast<bf16>(x); }
DEVI float to_f32(float x) { return x; }
DEVI float to_f32(bf16 x) { return static_cast<float>(x); }

// 16-byte vector of T
template <typename T> struct Vec16 { static constexpr int N = 16 / sizeof(T); };

struct alignas(16) U128 { uint32_t w[4]; };

DEVI U128 ld128(const void* p) { return *reinterpret_cast<const U128*>(p); }
DEVI void st128(void* p, const U128& v) { *reinterpret_cast<U128*>(p) = v; }
DEVI U128 zero128() { U128 z; z.w[0] = z.w[1] = z.w[2] = z.w[3] = 0; return z; }

template <typename T> DEVI T elem(const U128& v, int i) {
  return reinterpret_cast<const T*>(&v)[i];
}

// wave-level reductions (64 lanes)
DEVI float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
DEVI float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Copy a [ROWS x COLS] tile whose COLS are contiguous in global memory into
// an LDS tile with the same orientation (row stride LDS_STRIDE elements).
// Rows >= row_lim or columns >= col_lim are zero-filled; col_lim must be a
// multiple of the 16-byte vector width.
template <typename T, int ROWS, int COLS, int LDS_STRIDE, int NTHREADS>
DEVI void tile_copy_rows(T* __restrict__ lds, const T* __restrict__ g, int64_t ld, int row_lim,
                         int col_lim, int tid) {
  constexpr int V = Vec16<T>::N;
  constexpr int VPR = COLS / V;  // vectors per row
  constexpr int TOTAL = ROWS * VPR;
#pragma unroll
  for (int it = 0; it < (TOTAL + NTHREADS - 1) / NTHREADS; ++it) {
    int idx = it * NTHREADS + tid;
    if (TOTAL % NTHREADS == 0 || idx < TOTAL) {
      int r = idx / VPR, c = (idx % VPR) * V;
      U128 v = (r < row_lim && c < col_lim) ? ld128(g + (int64_t)r * ld + c) : zero128();
      st128(lds + r * LDS_STRIDE + c, v);
    }
  }
}

// Load a tile stored in global memory as [KR rows][MC cols] (MC contiguous)
// and store it transposed into LDS as [MC rows][KR cols] (row stride
// LDS_STRIDE).  Each thread moves 4 consecutive k-rows x one 16-byte vector
// of m, transposing in registers, so LDS is written 4 elements at a time.
// Global rows >= k_lim or columns >= m_lim are zero-filled (m_lim a multiple
// of the vector width).
template <typename T, int KR, int MC, int LDS_STRIDE, int NTHREADS>
DEVI void tile_copy_transpose(T* __restrict__ lds, const T* __restrict__ g, int64_t ld, int k_lim,
                              int m_lim, int tid) {
  constexpr int V = Vec16<T>::N;
  constexpr int MV = MC / V;          // vectors along m
  constexpr int KB = KR / 4;          // 4-row groups along k
  constexpr int TOTAL = MV * KB;
  static_assert(KR % 4 == 0, "k rows in groups of 4");
#pragma unroll
  for (int it = 0; it < (TOTAL + NTHREADS - 1) / NTHREADS; ++it) {
    int idx = it * NTHREADS + tid;
    if (TOTAL % NTHREADS == 0 || idx < TOTAL) {
      int kb = idx % KB, mv = idx / KB;   // k-groups fastest (bank conflicts)
      int m0 = mv * V, k0 = kb * 4;
      U128 r[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        r[q] = (k0 + q < k_lim && m0 < m_lim) ? ld128(g + (int64_t)(k0 + q) * ld + m0) : zero128();
#pragma unroll
      for (int e = 0; e < V; ++e) {
        T t4[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) t4[q] = elem<T>(r[q], e);
        T* dst = lds + (m0 + e) * LDS_STRIDE + k0;
        if constexpr (sizeof(T) == 2) {
          uint32_t lo = (uint32_t)__builtin_bit_cast(uint16_t, t4[0]) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, t4[1]) << 16);
          uint32_t hi = (uint32_t)__builtin_bit_cast(uint16_t, t4[2]) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, t4[3]) << 16);
          uint2 w; w.x = lo; w.y = hi;
          *reinterpret_cast<uint2*>(dst) = w;
        } else {
          float4 w; w.x = t4[0]; w.y = t4[1]; w.z = t4[2]; w.w = t4[3];
          *reinterpret_cast<float4*>(dst) = w;
        }
      }
    }
  }
}

// Register-staged versions of the two tile copies above: load() issues the
// global reads (so they can overlap compute on the other LDS buffer),
// store() writes LDS.
template <typename T, int ROWS, int COLS, int LDS_STRIDE, int NTHREADS>
struct StagedRows {
  static constexpr int V = Vec16<T>::N;
  static constexpr int VPR = COLS / V;
  static constexpr int TOTAL = ROWS * VPR;
  static constexpr int IT = (TOTAL + NTHREADS - 1) / NTHREADS;
  U128 r[IT];
  DEVI void load(const T* __restrict__ g, int64_t ld, int row_lim, int col_lim, int tid) {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int idx = it * NTHREADS + tid;
      const int rr = idx / VPR, c = (idx % VPR) * V;
      const bool ok = (TOTAL % NTHREADS == 0 || idx < TOTAL) && rr < row_lim && c < col_lim;
      r[it] = ok ? ld128(g + (int64_t)rr * ld + c) : zero128();
    }
  }
  DEVI void store(T* __restrict__ lds, int tid) const {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int idx = it * NTHREADS + tid;
      if (TOTAL % NTHREADS == 0 || idx < TOTAL) {
        const int rr = idx / VPR, c = (idx % VPR) * V;
        st128(lds + rr * LDS_STRIDE + c, r[it]);
      }
    }
  }
};

template <typename T, int KR, int MC, int LDS_STRIDE, int NTHREADS>
struct StagedTrans {
  static constexpr int V = Vec16<T>::N;
  static constexpr int MV = MC / V;
  static constexpr int KB = KR / 4;
  static constexpr int TOTAL = MV * KB;
  static constexpr int IT = (TOTAL + NTHREADS - 1) / NTHREADS;
  U128 r[IT][4];
  DEVI void load(const T* __restrict__ g, int64_t ld, int k_lim, int m_lim, int tid) {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int idx = it * NTHREADS + tid;
      const int kb = idx % KB, mv = idx / KB;   // k-groups fastest: see store()
      const int m0 = mv * V, k0 = kb * 4;
      const bool live = TOTAL % NTHREADS == 0 || idx < TOTAL;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        r[it][q] = (live && k0 + q < k_lim && m0 < m_lim) ? ld128(g + (int64_t)(k0 + q) * ld + m0) : zero128();
    }
  }
  DEVI void store(T* __restrict__ lds, int tid) const {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int idx = it * NTHREADS + tid;
      if (!(TOTAL % NTHREADS == 0 || idx < TOTAL)) continue;
      // Lanes of a wave differ mostly in kb, i.e. in the column of the
      // transposed row they write; with the usual row pitch of (multiple of
      // 64) + 16 bytes this keeps a wave's 8-byte writes at most 2-way
      // bank-conflicted (m-fastest lanes would hit the same bank 8 ways).
      const int kb = idx % KB, mv = idx / KB;
      const int m0 = mv * V, k0 = kb * 4;
#pragma unroll
      for (int e = 0; e < V; ++e) {
        T t4[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) t4[q] = elem<T>(r[it][q], e);
        T* dst = lds + (m0 + e) * LDS_STRIDE + k0;
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
};

// Read an 8-element operand fragment from an LDS row (k contiguous).
template <typename T> DEVI typename Frag<T>::type lds_frag8(const T* p);
template <> DEVI bf16x8 lds_frag8<bf16>(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
template <> DEVI f32x8 lds_frag8<float>(const float* p) {
  f32x8 r;
  float4 a = *reinterpret_cast<const float4*>(p);
  float4 b = *reinterpret_cast<const float4*>(p + 4);
  r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w; r[4] = b.x; r[5] = b.y; r[6] = b.z; r[7] = b.w;
  return r;
}
// Two 4-element halves from two LDS locations (k-slots 0..3 and 4..7).
template <typename T> DEVI typename Frag<T>::type lds_frag4x2(const T* p0, const T* p1);
template <> DEVI bf16x8 lds_frag4x2<bf16>(const bf16* p0, const bf16* p1) {
  bf16x4 a = *reinterpret_cast<const bf16x4*>(p0);
  bf16x4 b = *reinterpret_cast<const bf16x4*>(p1);
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3]; r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}
template <> DEVI f32x8 lds_frag4x2<float>(const float* p0, const float* p1) {
  float4 a = *reinterpret_cast<const float4*>(p0);
  float4 b = *reinterpret_cast<const float4*>(p1);
  f32x8 r;
  r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w; r[4] = b.x; r[5] = b.y; r[6] = b.z; r[7] = b.w;
  return r;
}
// Global-memory fragment: 8 contiguous elements, zero beyond `lim` elements.
template <typename T> DEVI typename Frag<T>::type g_frag8(const T* p, bool ok);
template <> DEVI bf16x8 g_frag8<bf16>(const bf16* p, bool ok) {
  if (ok) return *reinterpret_cast<const bf16x8*>(p);
  bf16x8 z; for (int i = 0; i < 8; ++i) z[i] = static_cast<bf16>(0.f); return z;
}
template <> DEVI f32x8 g_frag8<float>(const float* p, bool ok) {
  f32x8 r;
  if (ok) {
    float4 a = *reinterpret_cast<const float4*>(p);
    float4 b = *reinterpret_cast<const float4*>(p + 4);
    r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w; r[4] = b.x; r[5] = b.y; r[6] = b.z; r[7] = b.w;
  } else {
    for (int i = 0; i < 8; ++i) r[i] = 0.f;
  }
  return r;
}
// Pack 8 floats into an operand fragment of T.
template <typename T> DEVI typename Frag<T>::type pack8(const float* v);
template <> DEVI bf16x8 pack8<bf16>(const float* v) {
  bf16x8 r; for (int i = 0; i < 8; ++i) r[i] = static_cast<bf16>(v[i]); return r;
}
template <> DEVI f32x8 pack8<float>(const float* v) {
  f32x8 r; for (int i = 0; i < 8; ++i) r[i] = v[i]; return r;
}

// Column of position slot s in a position-permuted transposed copy (of K,
// V, Q or dO: [H*hd][slots]): inside every aligned group of 16 slots the
// middle two quads are swapped (offsets 4..7 and 8..11), so the 8 positions
// {4h..4h+3, 8+4h..8+4h+3} of a group, which one lane holds in a 32x32
// accumulator of scores, sit in one 16-byte run (offsets 8h..8h+7).
DEVI int64_t kperm(int64_t s) {
  const int o = (int)(s & 15);
  return (s & ~(int64_t)15) | (o < 4 || o >= 12 ? o : (o < 8 ? o + 4 : o - 4));
}

// Activation backward, shared by the standalone and the GEMM-epilogue forms:
// SwiGLU act = silu(g) * u -> (d/dg, d/du); GELU (erf) -> d/dv.
DEVI void swiglu_bwd(float da, float g, float u, float& dg, float& du) {
  const float sg = 1.f / (1.f + __expf(-g));
  dg = da * u * sg * (1.f + g * (1.f - sg));
  du = da * g * sg;
}
DEVI float gelu_bwd(float v, float d) {
  const float cdf = 0.5f * (1.f + erff(v * 0.70710678118654752f));
  const float pdf = 0.39894228040143268f * __expf(-0.5f * v * v);
  return d * (cdf + v * pdf);
}

// 2^x with the hardware instruction (no denormal range fix-up; the inputs
// here are <= 8 and results below 2^-126 may flush to zero).
DEVI float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// RoPE angle of pair i at position pos, in float64, reduced before the
// float rotation (positions reach 5e5, where a float angle would be off by
// 0.03).
DEVI void rope_cs(int64_t pos, const double* theta, int i, float& c, float& s) {
  const double a = (double)pos * theta[i];
  double sd, cd;
  sincos(a, &sd, &cd);
  c = (float)cd;
  s = (float)sd;
}
