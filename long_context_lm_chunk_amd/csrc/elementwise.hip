// Bandwidth-bound kernels of the inner loop: embedding gather, LayerNorm
// forward/backward (fp32 statistics), RoPE with float64 angles written
// straight into the K/V ring, activation backward, weight layout conversion
// and the cross-entropy row combine.
#include "common.hpp"
#include "kernels.hpp"

namespace ttt {
namespace {

// 16-byte load with the non-temporal hint, for intermediates read once (the
// K-split partial slabs, the head's kept logits, the transposes' sources),
// so that the caches keep what the products read again.
DEVI float4 ldnt4(const float4* p) {
  const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  return make_float4(t.x, t.y, t.z, t.w);
}
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));

// 4 consecutive values to T (16 bytes of fp32 or 8 of bf16)
template <typename T> DEVI void store4v(T* p, const float4& v);
template <> DEVI void store4v<float>(float* p, const float4& v) { *reinterpret_cast<float4*>(p) = v; }
template <> DEVI void store4v<bf16>(bf16* p, const float4& v) {
  bf16x4 b;
  b[0] = static_cast<bf16>(v.x); b[1] = static_cast<bf16>(v.y);
  b[2] = static_cast<bf16>(v.z); b[3] = static_cast<bf16>(v.w);
  *reinterpret_cast<bf16x4*>(p) = b;
}
template <typename T> DEVI float4 load4v(const T* p);
template <> DEVI float4 load4v<float>(const float* p) { return *reinterpret_cast<const float4*>(p); }
template <> DEVI float4 load4v<bf16>(const bf16* p) {
  const bf16x4 b = *reinterpret_cast<const bf16x4*>(p);
  return make_float4(static_cast<float>(b[0]), static_cast<float>(b[1]), static_cast<float>(b[2]),
                     static_cast<float>(b[3]));
}


template <typename T>
__global__ void embed_k(const int32_t* __restrict__ tok, int n, const T* __restrict__ E, int d, int V,
                        float* __restrict__ out, int* __restrict__ err) {
  const int t = blockIdx.x;
  if (t >= n) return;
  int id = tok[t];
  if (id < 0 || id >= V) {
    if (threadIdx.x == 0) atomicOr(err, 1);
    id = 0;
  }
  for (int i = threadIdx.x; i < d; i += blockDim.x)
    out[(int64_t)t * d + i] = to_f32(E[(int64_t)id * d + i]);
}

// One wave per row.  y = (x - mean) * rstd, biased variance.
template <typename T>
__global__ void ln_fwd_k(const float* __restrict__ x, int64_t ldx, int n, int d, float eps,
                         T* __restrict__ y, int64_t ldy, float* __restrict__ mean,
                         float* __restrict__ rstd) {
  const int row = blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= n) return;
  const float* xr = x + (int64_t)row * ldx;
  float s = 0.f;
  for (int i = lane; i < d; i += 64) s += xr[i];
  const float mu = wave_sum(s) / d;
  float v = 0.f;
  for (int i = lane; i < d; i += 64) { const float c = xr[i] - mu; v += c * c; }
  const float rs = rsqrtf(wave_sum(v) / d + eps);
  T* yr = y + (int64_t)row * ldy;
  for (int i = lane; i < d; i += 64) yr[i] = from_f32<T>((xr[i] - mu) * rs);
  if (lane == 0) {
    if (mean) mean[row] = mu;
    if (rstd) rstd[row] = rs;
  }
}

// Few rows (decode): one 256-thread block per row, two-level reduction, so a
// single row costs a few microseconds instead of one wave's serial passes.
template <typename T>
__global__ __launch_bounds__(256) void ln_fwd_row_k(const float* __restrict__ x, int64_t ldx, int d,
                                                    float eps, T* __restrict__ y, int64_t ldy,
                                                    float* __restrict__ mean, float* __restrict__ rstd) {
  __shared__ float red[8];
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* xr = x + (int64_t)row * ldx;
  float s = 0.f;
  for (int i = tid; i < d; i += 256) s += xr[i];
  s = wave_sum(s);
  if (lane == 0) red[wave] = s;
  __syncthreads();
  const float mu = (red[0] + red[1] + red[2] + red[3]) / d;
  float v = 0.f;
  for (int i = tid; i < d; i += 256) { const float c = xr[i] - mu; v += c * c; }
  v = wave_sum(v);
  if (lane == 0) red[4 + wave] = v;
  __syncthreads();
  const float rs = rsqrtf((red[4] + red[5] + red[6] + red[7]) / d + eps);
  T* yr = y + (int64_t)row * ldy;
  for (int i = tid; i < d; i += 256) yr[i] = from_f32<T>((xr[i] - mu) * rs);
  if (tid == 0) {
    if (mean) mean[row] = mu;
    if (rstd) rstd[row] = rs;
  }
}

// acc += rstd * (dy - mean(dy) - yhat * mean(dy * yhat)); acc_lo = round(acc)
template <typename T>
__global__ void ln_bwd_k(const float* __restrict__ dy, const float* __restrict__ x,
                         const float* __restrict__ mean, const float* __restrict__ rstd, int n, int d,
                         float* __restrict__ acc, T* __restrict__ acc_lo, int nslab, int64_t slab_stride) {
  const int row = blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= n) return;
  const float* g = dy + (int64_t)row * d;
  // dy of column i, the partial slabs of a K-split product summed in slab order
  auto gval = [&](int i) {
    float v = g[i];
    for (int z = 1; z < nslab; ++z) v += g[z * slab_stride + i];
    return v;
  };
  const float* xr = x + (int64_t)row * d;
  const float mu = mean[row], rs = rstd[row];
  float s1 = 0.f, s2 = 0.f;
  for (int i = lane; i < d; i += 64) {
    const float yh = (xr[i] - mu) * rs;
    const float gi = gval(i);
    s1 += gi;
    s2 += gi * yh;
  }
  const float m1 = wave_sum(s1) / d, m2 = wave_sum(s2) / d;
  float* a = acc + (int64_t)row * d;
  for (int i = lane; i < d; i += 64) {
    const float yh = (xr[i] - mu) * rs;
    const float nv = a[i] + rs * (gval(i) - m1 - yh * m2);
    a[i] = nv;
    if (acc_lo) acc_lo[(int64_t)row * d + i] = from_f32<T>(nv);
  }
}

// Register-resident LayerNorm, d = 256 * NV: a lane holds NV float4 of its
// row, all loaded at once, so the row is read from memory a single time and
// every load of the wave is in flight together (the loop versions above
// re-read the row per pass with one 4-byte load per lane per step).
template <typename T, int NV>
__global__ __launch_bounds__(256) void ln_fwd_reg_k(const float* __restrict__ x, int64_t ldx, int n,
                                                    float eps, T* __restrict__ y, int64_t ldy,
                                                    float* __restrict__ mean, float* __restrict__ rstd,
                                                    const float* __restrict__ sl, int nsl, int64_t sls,
                                                    float* __restrict__ xo) {
  constexpr int D = 256 * NV;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= n) return;
  const float4* xr = reinterpret_cast<const float4*>(x + (int64_t)row * ldx);
  float4 v[NV];
  if (sl) {
    // the row is the residual x plus a product left as nsl K-split slabs
    // (rows of D floats): summed in slab order, then x added, as the
    // reduction pass would have done; the sum is stored to xo
    const float4* s0 = reinterpret_cast<const float4*>(sl + (int64_t)row * D);
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i] = ldnt4(s0 + lane + 64 * i);
    for (int z = 1; z < nsl; ++z) {
      const float4* sz = reinterpret_cast<const float4*>(sl + z * sls + (int64_t)row * D);
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const float4 w = ldnt4(sz + lane + 64 * i);
        v[i].x += w.x; v[i].y += w.y; v[i].z += w.z; v[i].w += w.w;
      }
    }
    float4* xw = reinterpret_cast<float4*>(xo + (int64_t)row * D);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const float4 r = xr[lane + 64 * i];
      v[i].x += r.x; v[i].y += r.y; v[i].z += r.z; v[i].w += r.w;
      xw[lane + 64 * i] = v[i];
    }
  } else {
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i] = xr[lane + 64 * i];
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) s += (v[i].x + v[i].y) + (v[i].z + v[i].w);
  const float mu = wave_sum(s) / D;
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const float a = v[i].x - mu, b = v[i].y - mu, c = v[i].z - mu, e = v[i].w - mu;
    q += (a * a + b * b) + (c * c + e * e);
  }
  const float rs = rsqrtf(wave_sum(q) / D + eps);
  T* yr = y + (int64_t)row * ldy;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    float4 o;
    o.x = (v[i].x - mu) * rs; o.y = (v[i].y - mu) * rs; o.z = (v[i].z - mu) * rs; o.w = (v[i].w - mu) * rs;
    store4v<T>(yr + 4 * (lane + 64 * i), o);
  }
  if (lane == 0) {
    if (mean) mean[row] = mu;
    if (rstd) rstd[row] = rs;
  }
}

// The same with one 256-thread block per row (d = 1024 * NQ): each thread
// holds NQ float4 of every array, the K-split slabs (up to 4) are loaded
// together with the row, and the two row sums meet through LDS, so a chunk
// of rows keeps 16 waves per CU busy instead of 4.
template <typename T, int NQ>
__global__ __launch_bounds__(256) void ln_bwd_blk_k(const float* __restrict__ dy, const float* __restrict__ x,
                                                    const float* __restrict__ mean,
                                                    const float* __restrict__ rstd, int n,
                                                    float* __restrict__ acc, T* __restrict__ acc_lo,
                                                    int nslab, int64_t slab_stride) {
  constexpr int D = 1024 * NQ;
  __shared__ float red[8];
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (row >= n) return;
  const float4* g = reinterpret_cast<const float4*>(dy + (int64_t)row * D);
  const float4* xr = reinterpret_cast<const float4*>(x + (int64_t)row * D);
  float4* a = reinterpret_cast<float4*>(acc + (int64_t)row * D);
  const float mu = mean[row], rs = rstd[row];
  float4 gv[NQ], yh[NQ], av[NQ], gz[3][NQ];
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    gv[i] = g[tid + 256 * i];
    yh[i] = xr[tid + 256 * i];
    av[i] = a[tid + 256 * i];
  }
#pragma unroll
  for (int z = 0; z < 3; ++z)
    if (z + 1 < nslab) {
      const float4* gs = reinterpret_cast<const float4*>(dy + (z + 1) * slab_stride + (int64_t)row * D);
#pragma unroll
      for (int i = 0; i < NQ; ++i) gz[z][i] = ldnt4(gs + tid + 256 * i);
    }
  // partial slabs of a K-split product, summed in slab order
#pragma unroll
  for (int z = 0; z < 3; ++z)
    if (z + 1 < nslab) {
#pragma unroll
      for (int i = 0; i < NQ; ++i) {
        gv[i].x += gz[z][i].x; gv[i].y += gz[z][i].y; gv[i].z += gz[z][i].z; gv[i].w += gz[z][i].w;
      }
    }
  float s1 = 0.f, s2 = 0.f;
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    yh[i].x = (yh[i].x - mu) * rs; yh[i].y = (yh[i].y - mu) * rs;
    yh[i].z = (yh[i].z - mu) * rs; yh[i].w = (yh[i].w - mu) * rs;
    s1 += (gv[i].x + gv[i].y) + (gv[i].z + gv[i].w);
    s2 += (gv[i].x * yh[i].x + gv[i].y * yh[i].y) + (gv[i].z * yh[i].z + gv[i].w * yh[i].w);
  }
  s1 = wave_sum(s1);
  s2 = wave_sum(s2);
  if (lane == 0) { red[wave] = s1; red[4 + wave] = s2; }
  __syncthreads();
  const float m1 = ((red[0] + red[1]) + (red[2] + red[3])) / D;
  const float m2 = ((red[4] + red[5]) + (red[6] + red[7])) / D;
  T* lo = acc_lo ? acc_lo + (int64_t)row * D : nullptr;
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    float4 nv;
    nv.x = av[i].x + rs * (gv[i].x - m1 - yh[i].x * m2);
    nv.y = av[i].y + rs * (gv[i].y - m1 - yh[i].y * m2);
    nv.z = av[i].z + rs * (gv[i].z - m1 - yh[i].z * m2);
    nv.w = av[i].w + rs * (gv[i].w - m1 - yh[i].w * m2);
    a[tid + 256 * i] = nv;
    if (lo) store4v<T>(lo + 4 * (tid + 256 * i), nv);
  }
}

template <typename T, int NV>
__global__ __launch_bounds__(256) void ln_bwd_reg_k(const float* __restrict__ dy, const float* __restrict__ x,
                                                    const float* __restrict__ mean,
                                                    const float* __restrict__ rstd, int n,
                                                    float* __restrict__ acc, T* __restrict__ acc_lo,
                                                    int nslab, int64_t slab_stride) {
  constexpr int D = 256 * NV;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= n) return;
  const float4* g = reinterpret_cast<const float4*>(dy + (int64_t)row * D);
  const float4* xr = reinterpret_cast<const float4*>(x + (int64_t)row * D);
  float4* a = reinterpret_cast<float4*>(acc + (int64_t)row * D);
  const float mu = mean[row], rs = rstd[row];
  float4 gv[NV], yh[NV], av[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    gv[i] = g[lane + 64 * i];
    yh[i] = xr[lane + 64 * i];
    av[i] = a[lane + 64 * i];
  }
  // partial slabs of a K-split product, summed in slab order
  for (int z = 1; z < nslab; ++z) {
    const float4* gz = reinterpret_cast<const float4*>(dy + z * slab_stride + (int64_t)row * D);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const float4 w = gz[lane + 64 * i];
      gv[i].x += w.x; gv[i].y += w.y; gv[i].z += w.z; gv[i].w += w.w;
    }
  }
  float s1 = 0.f, s2 = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    yh[i].x = (yh[i].x - mu) * rs; yh[i].y = (yh[i].y - mu) * rs;
    yh[i].z = (yh[i].z - mu) * rs; yh[i].w = (yh[i].w - mu) * rs;
    s1 += (gv[i].x + gv[i].y) + (gv[i].z + gv[i].w);
    s2 += (gv[i].x * yh[i].x + gv[i].y * yh[i].y) + (gv[i].z * yh[i].z + gv[i].w * yh[i].w);
  }
  const float m1 = wave_sum(s1) / D, m2 = wave_sum(s2) / D;
  T* lo = acc_lo ? acc_lo + (int64_t)row * D : nullptr;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    float4 nv;
    nv.x = av[i].x + rs * (gv[i].x - m1 - yh[i].x * m2);
    nv.y = av[i].y + rs * (gv[i].y - m1 - yh[i].y * m2);
    nv.z = av[i].z + rs * (gv[i].z - m1 - yh[i].z * m2);
    nv.w = av[i].w + rs * (gv[i].w - m1 - yh[i].w * m2);
    a[lane + 64 * i] = nv;
    if (lo) store4v<T>(lo + 4 * (lane + 64 * i), nv);
  }
}

template <typename T>
__global__ void cast_k(const float* __restrict__ s, T* __restrict__ d, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    d[i] = from_f32<T>(s[i]);
}

template <typename T>
__global__ void widen_k(const T* __restrict__ s, float* __restrict__ d, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    d[i] = to_f32(s[i]);
}

__global__ void fill_k(float* __restrict__ p, int64_t n, float v) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}


// cos / sin of the rotary angle (pos0 + t) * theta_i for t < n, i < half,
// formed in float64 (rope_cs) once per block of positions and shared by
// every layer and head that reads those positions.
__global__ void rope_table_k(int64_t pos0, int n, int half, const double* __restrict__ theta,
                             float2* __restrict__ cs) {
  const int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (idx >= (int64_t)n * half) return;
  const int t = (int)(idx / half), i = (int)(idx % half);
  float c, s;
  rope_cs(pos0 + t, theta, i, c, s);
  cs[idx] = make_float2(c, s);
}

template <typename T> DEVI void ld8(const T* p, float* v);
template <> DEVI void ld8<bf16>(const bf16* p, float* v) {
  const bf16x8 x = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = static_cast<float>(x[j]);
}
template <> DEVI void ld8<float>(const float* p, float* v) {
  const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
// 8 consecutive outputs of a product at element off: read from src (T), or,
// when the product left nsl > 1 fp32 K-split slabs (slab stride sls), their
// sum in slab order rounded to T, as the reduction pass would have stored it
template <typename T>
DEVI void ld8_out(const T* src, const float* sl, int nsl, int64_t sls, int64_t off, float* v) {
  if (nsl <= 1) {
    ld8<T>(src + off, v);
    return;
  }
  float4 a = ldnt4(reinterpret_cast<const float4*>(sl + off));
  float4 b = ldnt4(reinterpret_cast<const float4*>(sl + off + 4));
  for (int z = 1; z < nsl; ++z) {
    const float4 c = ldnt4(reinterpret_cast<const float4*>(sl + z * sls + off));
    const float4 e = ldnt4(reinterpret_cast<const float4*>(sl + z * sls + off + 4));
    a.x += c.x; a.y += c.y; a.z += c.z; a.w += c.w;
    b.x += e.x; b.y += e.y; b.z += e.z; b.w += e.w;
  }
  const float w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = to_f32(from_f32<T>(w[j]));
}
template <typename T> DEVI void st8(T* p, const float* v);
template <> DEVI void st8<bf16>(bf16* p, const float* v) {
  bf16x8 x;
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = static_cast<bf16>(v[j]);
  *reinterpret_cast<bf16x8*>(p) = x;
}
template <> DEVI void st8<float>(float* p, const float* v) {
  reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
}

// Rotary embedding of 64 positions of one head, in work items of 8 rotation
// pairs with 16-byte (bf16) accesses: q -> q_out [n][H*hd]; k (rotated) and
// v -> ring row (pos0 + t) mod cap; then, through one LDS tile, v and (when
// kt is set) k -> the position-permuted transposed rings [H*hd][cap] (the
// column of a slot is kperm(slot)).  qkv [n][3*H*hd]; hd <= 128, hd % 16 == 0.
template <typename T>
__global__ __launch_bounds__(256) void qkv_rope_k(const T* __restrict__ qkv, const float* __restrict__ sl,
                                                  int nsl, int64_t sls, int n, int H, int hd,
                                                  int64_t pos0, const float2* __restrict__ cs,
                                                  T* __restrict__ qo, T* __restrict__ kr, T* __restrict__ vr,
                                                  T* __restrict__ vt, T* __restrict__ kt, int64_t cap) {
  constexpr int NI = 2;                        // work items per thread (64 positions x <= 8 chunks)
  __shared__ T tile[64][128 + 2];
  const int h = blockIdx.y, t0 = blockIdx.x * 64, tid = threadIdx.x;
  const int half = hd >> 1, nc = half / 8, d = H * hd;
  float kv[NI][16];
#pragma unroll
  for (int u = 0; u < NI; ++u) {
    const int it = tid + 256 * u;
    const int t = it / nc, c = it % nc, i0 = 8 * c;
    if (it >= 64 * nc || t0 + t >= n) continue;
    const int64_t slot = (pos0 + t0 + t) % cap;
    const int64_t row = (int64_t)(t0 + t) * 3 * d + h * hd;
    const float2* e = cs + (int64_t)(t0 + t) * half + i0;
    float a[8], b[8], ra[8], rb[8];
    ld8_out<T>(qkv, sl, nsl, sls, row + i0, a);
    ld8_out<T>(qkv, sl, nsl, sls, row + half + i0, b);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float2 w = e[j];
      ra[j] = a[j] * w.x - b[j] * w.y;
      rb[j] = b[j] * w.x + a[j] * w.y;
    }
    T* qr = qo + (int64_t)(t0 + t) * d + h * hd;
    st8<T>(qr + i0, ra);
    st8<T>(qr + half + i0, rb);
    ld8_out<T>(qkv, sl, nsl, sls, row + d + i0, a);
    ld8_out<T>(qkv, sl, nsl, sls, row + d + half + i0, b);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float2 w = e[j];
      kv[u][j] = a[j] * w.x - b[j] * w.y;
      kv[u][8 + j] = b[j] * w.x + a[j] * w.y;
    }
    T* krow = kr + slot * d + h * hd;
    st8<T>(krow + i0, kv[u]);
    st8<T>(krow + half + i0, kv[u] + 8);
    ld8_out<T>(qkv, sl, nsl, sls, row + 2 * d + i0, a);
    ld8_out<T>(qkv, sl, nsl, sls, row + 2 * d + half + i0, b);
    T* vrow = vr + slot * d + h * hd;
    st8<T>(vrow + i0, a);
    st8<T>(vrow + half + i0, b);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      tile[t][i0 + j] = from_f32<T>(a[j]);
      tile[t][half + i0 + j] = from_f32<T>(b[j]);
    }
  }
  __syncthreads();
  for (int idx = tid; idx < hd * 64; idx += 256) {
    const int i = idx / 64, t = idx % 64;
    if (t0 + t < n) vt[(int64_t)(h * hd + i) * cap + kperm((pos0 + t0 + t) % cap)] = tile[t][i];
  }
  if (!kt) return;
  __syncthreads();
#pragma unroll
  for (int u = 0; u < NI; ++u) {
    const int it = tid + 256 * u;
    const int t = it / nc, c = it % nc, i0 = 8 * c;
    if (it >= 64 * nc || t0 + t >= n) continue;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      tile[t][i0 + j] = from_f32<T>(kv[u][j]);
      tile[t][half + i0 + j] = from_f32<T>(kv[u][8 + j]);
    }
  }
  __syncthreads();
  for (int idx = tid; idx < hd * 64; idx += 256) {
    const int i = idx / 64, t = idx % 64;
    if (t0 + t < n) kt[(int64_t)(h * hd + i) * cap + kperm((pos0 + t0 + t) % cap)] = tile[t][i];
  }
}

// Transposed rotation of dQ and dK inside dqkv [n][3d] (the rotation's
// transpose), 8 pairs per thread with 16-byte accesses, angles from the table.
template <typename T>
__global__ void rope_bwd_tab_k(T* __restrict__ g, int n, int H, int hd, const float2* __restrict__ cs,
                               int parts) {
  const int half = hd >> 1, nc = half / 8;
  const int64_t total = (int64_t)n * H * nc;
  const int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int c = (int)(idx % nc), h = (int)((idx / nc) % H), t = (int)(idx / ((int64_t)nc * H));
  const int d = H * hd, i0 = 8 * c;
  const float2* e = cs + (int64_t)t * half + i0;
#pragma unroll
  for (int part = 0; part < 2; ++part) {
    if (!((parts >> part) & 1)) continue;
    T* r = g + (int64_t)t * 3 * d + part * d + h * hd;
    float a[8], b[8], ra[8], rb[8];
    ld8<T>(r + i0, a);
    ld8<T>(r + half + i0, b);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float2 w = e[j];
      ra[j] = a[j] * w.x + b[j] * w.y;
      rb[j] = b[j] * w.x - a[j] * w.y;
    }
    st8<T>(r + i0, ra);
    st8<T>(r + half + i0, rb);
  }
}

// dst[c][r] = src[r][c] for r < rows, c < cols; rows rows..rows_pad-1 of
// dst's columns are written as zero (so that a reduction over r can run in
// whole 16-byte vectors).  64x64 tiles through LDS: coalesced reads along c,
// coalesced writes along r.
template <typename T>
__global__ __launch_bounds__(256) void transpose_k(const T* __restrict__ src, int rows, int cols,
                                                   int64_t lds_, T* __restrict__ dst, int64_t ldd,
                                                   int rows_pad, int perm, int vec_in, int vec_out) {
  // 64 x 64 tile: 16-byte loads along the source rows (V elements), then
  // runs of 4 source rows written as one 4-element store per output row
  // (with perm, kperm moves aligned runs of 4 as a whole)
  constexpr int V = 16 / (int)sizeof(T);
  __shared__ T tile[64][65];
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int t = threadIdx.x;
#pragma unroll
  for (int idx = t; idx < 64 * (64 / V); idx += 256) {
    const int row = idx / (64 / V), cv = (idx % (64 / V)) * V;
    const int r = r0 + row, c = c0 + cv;
    T v[V];
    if (vec_in && r < rows && c + V <= cols) {
      *reinterpret_cast<u32x4v*>(v) =
          __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(src + (int64_t)r * lds_ + c));
    } else {
#pragma unroll
      for (int e = 0; e < V; ++e) v[e] = (r < rows && c + e < cols) ? src[(int64_t)r * lds_ + c + e] : from_f32<T>(0.f);
    }
#pragma unroll
    for (int e = 0; e < V; ++e) tile[row][cv + e] = v[e];
  }
  __syncthreads();
#pragma unroll
  for (int idx = t; idx < 64 * 16; idx += 256) {
    const int j = idx / 16, rg = (idx % 16) * 4;
    const int c = c0 + j, r = r0 + rg;
    if (c >= cols || r >= rows_pad) continue;
    T w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = tile[rg + e][j];
    T* drow = dst + (int64_t)c * ldd;
    if (vec_out && r + 3 < rows_pad) {
      T* d4 = drow + (perm ? kperm(r) : r);
      if constexpr (sizeof(T) == 2) *reinterpret_cast<uint2*>(d4) = *reinterpret_cast<const uint2*>(w);
      else *reinterpret_cast<uint4*>(d4) = *reinterpret_cast<const uint4*>(w);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (r + e < rows_pad) drow[perm ? kperm(r + e) : r + e] = w[e];
    }
  }
}



// Canonical [rows=in][cols=out] -> internal [out][in] (transpose), optionally
// into the gate (half 0) or up (half 1) rows of a block-16 interleaved matrix.
template <typename T>
__global__ void convert_k(const T* __restrict__ src, int rows, int cols, int transpose, int ilv,
                          T* __restrict__ dst) {
  __shared__ T tile[32][33];
  const int bx = blockIdx.x * 32, by = blockIdx.y * 32;  // bx over cols, by over rows of src
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5; // 256 threads: 32 x 8
  if (!transpose) {
    for (int r = ty; r < 32; r += 8) {
      const int rr = by + r, cc = bx + tx;
      if (rr < rows && cc < cols) dst[(int64_t)rr * cols + cc] = src[(int64_t)rr * cols + cc];
    }
    return;
  }
  for (int r = ty; r < 32; r += 8) {
    const int rr = by + r, cc = bx + tx;
    if (rr < rows && cc < cols) tile[r][tx] = src[(int64_t)rr * cols + cc];
  }
  __syncthreads();
  for (int c = ty; c < 32; c += 8) {
    const int oc = bx + c;   // output row (= src col)
    const int orr = by + tx; // output col (= src row)
    if (oc < cols && orr < rows) {
      int64_t drow = oc;
      if (ilv >= 0) drow = (int64_t)(oc / 16) * 32 + ilv * 16 + (oc % 16);
      dst[drow * rows + orr] = tile[tx][c];
    }
  }
}

// Internal [out][in] W0 (optionally interleaved, taking half `which`) plus
// the fp32 delta -> canonical fp32 [in][out].
template <typename T>
__global__ void export_k(const T* __restrict__ w0, const float* __restrict__ dm, int out_dim,
                         int in_dim, int ilv, int which, float* __restrict__ dst) {
  const int64_t total = (int64_t)out_dim * in_dim;
  const int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int f = idx % out_dim;          // output column (out index)
  const int j = idx / out_dim;          // input row
  int64_t r = f;
  if (ilv) r = (int64_t)(f / 16) * 32 + which * 16 + (f % 16);
  dst[idx] = (w0 ? to_f32(w0[r * in_dim + j]) : 0.f) + dm[r * in_dim + j];   // no w0: the delta
}

// One wave per row: combine the per-part (max, sumexp) into the row LSE and
// the row loss (natural log).
__global__ void ce_rows_k(const float* __restrict__ pmax, const float* __restrict__ psum, int nparts,
                          int64_t ldp, const float* __restrict__ tl, int n_rows, int n_tgt,
                          float* __restrict__ lse, float* __restrict__ rowloss) {
  const int row = blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= n_rows) return;
  float m = -INFINITY;
  for (int p = lane; p < nparts; p += 64) m = fmaxf(m, pmax[(int64_t)p * ldp + row]);
  m = wave_max(m);
  float s = 0.f;
  for (int p = lane; p < nparts; p += 64) s += psum[(int64_t)p * ldp + row] * __expf(pmax[(int64_t)p * ldp + row] - m);
  s = wave_sum(s);
  if (lane == 0) {
    const float l = m + __logf(s);
    lse[row] = l;
    rowloss[row] = row < n_tgt ? l - tl[row] : 0.f;
  }
}

// Gradient of the mean CE with respect to the logits, from stored fp32
// logits: g = (exp(z - lse) - onehot(target)) / n_tgt on target rows, 0 on
// the others; four columns per thread (V % 4 == 0).
template <typename T>
__global__ void ce_grad_k(const float* __restrict__ z, int64_t ldz, const float* __restrict__ lse,
                          const int* __restrict__ tgt, int n_rows, int n_tgt, int V, float alpha,
                          T* __restrict__ g, int64_t ldg) {
  const int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;   // 4-column groups
  const int64_t total = (int64_t)n_rows * (V / 4);
  if (idx >= total) return;
  const int row = (int)(idx / (V / 4)), col = (int)(idx % (V / 4)) * 4;
  float4 o = {0.f, 0.f, 0.f, 0.f};
  if (row < n_tgt) {
    const float4 v = ldnt4(reinterpret_cast<const float4*>(z + (int64_t)row * ldz + col));
    const float l = lse[row];
    const int t = tgt[row];
    o.x = (__expf(v.x - l) - (col == t ? 1.f : 0.f)) * alpha;
    o.y = (__expf(v.y - l) - (col + 1 == t ? 1.f : 0.f)) * alpha;
    o.z = (__expf(v.z - l) - (col + 2 == t ? 1.f : 0.f)) * alpha;
    o.w = (__expf(v.w - l) - (col + 3 == t ? 1.f : 0.f)) * alpha;
  }
  store4v<T>(g + (int64_t)row * ldg + col, o);
}

// Deterministic mean over the target rows; flags a non-finite loss.
__global__ void ce_mean_k(const float* __restrict__ rowloss, int n_tgt, float* __restrict__ out,
                          int* __restrict__ err) {
  __shared__ float red[1024];
  float s = 0.f;
  for (int i = threadIdx.x; i < n_tgt; i += blockDim.x) s += rowloss[i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int o = blockDim.x / 2; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const float v = n_tgt > 0 ? red[0] / n_tgt : 0.f;
    *out = v;
    if (!isfinite(v)) atomicOr(err, 2);
  }
}

// D[h][t] = sum_i dO[t][h,i] * O[t][h,i]; one wave per (t, h)
template <typename T>
__global__ void rowdot_k(const T* __restrict__ o, const T* __restrict__ g, int n, int H, int hd,
                         float* __restrict__ D) {
  const int w = blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (w >= n * H) return;
  const int t = w / H, h = w % H;
  const int64_t base = (int64_t)t * H * hd + h * hd;
  float s = 0.f;
  for (int i = lane; i < hd; i += 64) s += to_f32(o[base + i]) * to_f32(g[base + i]);
  s = wave_sum(s);
  if (lane == 0) D[(int64_t)h * n + t] = s;
}

// x_out = (sum of nsl K-split slabs in slab order) + R, 4 floats per thread
// (rows of d floats, d % 4 == 0): the reduction pass of a split product with
// a residual, for the LayerNorm paths that do not take the slabs themselves
__global__ void resid_slabs_k(const float* __restrict__ sl, int nsl, int64_t sls, const float* __restrict__ R,
                              float* __restrict__ xo, int64_t groups) {
  const int64_t g = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (g >= groups) return;
  float4 v = ldnt4(reinterpret_cast<const float4*>(sl) + g);
  for (int z = 1; z < nsl; ++z) {
    const float4 w = ldnt4(reinterpret_cast<const float4*>(sl + z * sls) + g);
    v.x += w.x; v.y += w.y; v.z += w.z; v.w += w.w;
  }
  const float4 r = reinterpret_cast<const float4*>(R)[g];
  v.x += r.x; v.y += r.y; v.z += r.z; v.w += r.w;
  reinterpret_cast<float4*>(xo)[g] = v;
}

inline unsigned nblk(int64_t n, int b) { return (unsigned)((n + b - 1) / b); }
inline unsigned gs_blocks(int64_t n) { int64_t b = (n + 255) / 256; return (unsigned)(b > 65536 ? 65536 : (b < 1 ? 1 : b)); }

}  // namespace

#define TSEL(bf, call_bf, call_f) do { if (bf) { call_bf; } else { call_f; } } while (0)

void embed(const int32_t* tok, int n, const void* E, int d, int V, bool bf, float* out, int* err,
           hipStream_t s) {
  if (n <= 0) return;
  TSEL(bf, hipLaunchKernelGGL(embed_k<bf16>, dim3(n), dim3(256), 0, s, tok, n, (const bf16*)E, d, V, out, err),
       hipLaunchKernelGGL(embed_k<float>, dim3(n), dim3(256), 0, s, tok, n, (const float*)E, d, V, out, err));
}

void layernorm_fwd(const float* x, int64_t ldx, int n, int d, float eps, void* y, int64_t ldy,
                   float* mean, float* rstd, bool bf, hipStream_t s) {
  if (n <= 0) return;
  if (n < 64) {
    TSEL(bf, hipLaunchKernelGGL(ln_fwd_row_k<bf16>, dim3(n), dim3(256), 0, s, x, ldx, d, eps, (bf16*)y, ldy, mean, rstd),
         hipLaunchKernelGGL(ln_fwd_row_k<float>, dim3(n), dim3(256), 0, s, x, ldx, d, eps, (float*)y, ldy, mean, rstd));
    return;
  }
  if (d % 256 == 0 && d <= 4096 && ldx % 4 == 0 && ldy % 4 == 0) {
    switch (d / 256) {
#define LNF(NV) case NV: TSEL(bf, hipLaunchKernelGGL((ln_fwd_reg_k<bf16, NV>), dim3(nblk(n, 4)), dim3(256), 0, s, x, ldx, n, eps, (bf16*)y, ldy, mean, rstd, nullptr, 0, (int64_t)0, nullptr), \
                               hipLaunchKernelGGL((ln_fwd_reg_k<float, NV>), dim3(nblk(n, 4)), dim3(256), 0, s, x, ldx, n, eps, (float*)y, ldy, mean, rstd, nullptr, 0, (int64_t)0, nullptr)); return;
      LNF(1) LNF(2) LNF(3) LNF(4) LNF(5) LNF(6) LNF(7) LNF(8) LNF(9) LNF(10) LNF(11) LNF(12)
      LNF(13) LNF(14) LNF(15) LNF(16)
#undef LNF
      default: break;
    }
  }
  TSEL(bf, hipLaunchKernelGGL(ln_fwd_k<bf16>, dim3(nblk(n, 4)), dim3(256), 0, s, x, ldx, n, d, eps, (bf16*)y, ldy, mean, rstd),
       hipLaunchKernelGGL(ln_fwd_k<float>, dim3(nblk(n, 4)), dim3(256), 0, s, x, ldx, n, d, eps, (float*)y, ldy, mean, rstd));
}

void layernorm_fwd_resid(const float* slabs, int nsl, const float* R, float* x_out, int n, int d, float eps,
                         void* y, int64_t ldy, float* mean, float* rstd, bool bf, hipStream_t s) {
  if (n <= 0) return;
  const int64_t sls = (int64_t)n * d;
  if (n >= 64 && d % 256 == 0 && d <= 4096 && ldy % 4 == 0) {
    switch (d / 256) {
#define LNF(NV) case NV: TSEL(bf, hipLaunchKernelGGL((ln_fwd_reg_k<bf16, NV>), dim3(nblk(n, 4)), dim3(256), 0, s, R, (int64_t)d, n, eps, (bf16*)y, ldy, mean, rstd, slabs, nsl, sls, x_out), \
                               hipLaunchKernelGGL((ln_fwd_reg_k<float, NV>), dim3(nblk(n, 4)), dim3(256), 0, s, R, (int64_t)d, n, eps, (float*)y, ldy, mean, rstd, slabs, nsl, sls, x_out)); return;
      LNF(1) LNF(2) LNF(3) LNF(4) LNF(5) LNF(6) LNF(7) LNF(8) LNF(9) LNF(10) LNF(11) LNF(12)
      LNF(13) LNF(14) LNF(15) LNF(16)
#undef LNF
      default: break;
    }
  }
  const int64_t groups = (int64_t)n * (d / 4);
  hipLaunchKernelGGL(resid_slabs_k, dim3(nblk(groups, 256)), dim3(256), 0, s, slabs, nsl, sls, R, x_out, groups);
  layernorm_fwd(x_out, d, n, d, eps, y, ldy, mean, rstd, bf, s);
}

void layernorm_bwd_acc(const float* dy, const float* x, const float* mean, const float* rstd, int n,
                       int d, float* acc, void* acc_lo, bool bf, hipStream_t s, int nslab,
                       int64_t slab_stride) {
  if (n <= 0) return;
  if (d % 1024 == 0 && d <= 4096 && nslab <= 4) {
    switch (d / 1024) {
#define LNQ(NQ) case NQ: TSEL(bf, hipLaunchKernelGGL((ln_bwd_blk_k<bf16, NQ>), dim3(n), dim3(256), 0, s, dy, x, mean, rstd, n, acc, (bf16*)acc_lo, nslab, slab_stride), \
                               hipLaunchKernelGGL((ln_bwd_blk_k<float, NQ>), dim3(n), dim3(256), 0, s, dy, x, mean, rstd, n, acc, (float*)acc_lo, nslab, slab_stride)); return;
      LNQ(1) LNQ(2) LNQ(3) LNQ(4)
#undef LNQ
      default: break;
    }
  }
  if (d % 256 == 0 && d <= 4096) {
    switch (d / 256) {
#define LNB(NV) case NV: TSEL(bf, hipLaunchKernelGGL((ln_bwd_reg_k<bf16, NV>), dim3(nblk(n, 4)), dim3(256), 0, s, dy, x, mean, rstd, n, acc, (bf16*)acc_lo, nslab, slab_stride), \
                               hipLaunchKernelGGL((ln_bwd_reg_k<float, NV>), dim3(nblk(n, 4)), dim3(256), 0, s, dy, x, mean, rstd, n, acc, (float*)acc_lo, nslab, slab_stride)); return;
      LNB(1) LNB(2) LNB(3) LNB(4) LNB(5) LNB(6) LNB(7) LNB(8) LNB(9) LNB(10) LNB(11) LNB(12)
      LNB(13) LNB(14) LNB(15) LNB(16)
#undef LNB
      default: break;
    }
  }
  TSEL(bf, hipLaunchKernelGGL(ln_bwd_k<bf16>, dim3(nblk(n, 4)), dim3(256), 0, s, dy, x, mean, rstd, n, d, acc, (bf16*)acc_lo, nslab, slab_stride),
       hipLaunchKernelGGL(ln_bwd_k<float>, dim3(nblk(n, 4)), dim3(256), 0, s, dy, x, mean, rstd, n, d, acc, (float*)acc_lo, nslab, slab_stride));
}

void cast_rows(const float* src, void* dst, int64_t n, bool bf, hipStream_t s) {
  copy_cast_from_f32(src, dst, n, bf, s);
}

void copy_cast_from_f32(const float* src, void* dst, int64_t n, bool bf, hipStream_t s) {
  if (n <= 0) return;
  TSEL(bf, hipLaunchKernelGGL(cast_k<bf16>, dim3(gs_blocks(n)), dim3(256), 0, s, src, (bf16*)dst, n),
       hipLaunchKernelGGL(cast_k<float>, dim3(gs_blocks(n)), dim3(256), 0, s, src, (float*)dst, n));
}

void widen(const void* src, float* dst, int64_t n, bool bf, hipStream_t s) {
  if (n <= 0) return;
  TSEL(bf, hipLaunchKernelGGL(widen_k<bf16>, dim3(gs_blocks(n)), dim3(256), 0, s, (const bf16*)src, dst, n),
       hipLaunchKernelGGL(widen_k<float>, dim3(gs_blocks(n)), dim3(256), 0, s, (const float*)src, dst, n));
}

void fill_f32(float* p, int64_t n, float v, hipStream_t s) {
  if (n <= 0) return;
  hipLaunchKernelGGL(fill_k, dim3(gs_blocks(n)), dim3(256), 0, s, p, n, v);
}

void rope_table(int64_t pos0, int n, int half, const double* theta, float2* cs, hipStream_t s) {
  const int64_t total = (int64_t)n * half;
  if (total <= 0) return;
  hipLaunchKernelGGL(rope_table_k, dim3(nblk(total, 256)), dim3(256), 0, s, pos0, n, half, theta, cs);
}

void qkv_rope(const void* qkv, int n, int H, int hd, int64_t pos0, const float2* cs, void* q_out,
              void* kring, void* vring, void* vtring, void* ktring, int64_t cap, bool bf, hipStream_t s,
              const float* slabs, int nsl) {
  if (n <= 0) return;
  dim3 grid((n + 63) / 64, H);
  const int64_t sls = (int64_t)n * 3 * H * hd;
  TSEL(bf, hipLaunchKernelGGL(qkv_rope_k<bf16>, grid, dim3(256), 0, s, (const bf16*)qkv, slabs, nsl, sls, n, H, hd, pos0, cs, (bf16*)q_out, (bf16*)kring, (bf16*)vring, (bf16*)vtring, (bf16*)ktring, cap),
       hipLaunchKernelGGL(qkv_rope_k<float>, grid, dim3(256), 0, s, (const float*)qkv, slabs, nsl, sls, n, H, hd, pos0, cs, (float*)q_out, (float*)kring, (float*)vring, (float*)vtring, (float*)ktring, cap));
}

void transpose(const void* src, int rows, int cols, int64_t lds_, void* dst, int64_t ldd, int rows_pad,
               bool bf, hipStream_t s, bool perm16) {
  if (rows_pad < rows) rows_pad = rows;
  if (rows_pad <= 0 || cols <= 0) return;
  dim3 grid((cols + 63) / 64, (rows_pad + 63) / 64);
  const int pm = perm16 ? 1 : 0;
  const int es = bf ? 2 : 4;
  // 16-byte loads need 16-byte aligned source rows, 4-element stores
  // 4-element aligned destination rows
  const int vin = (lds_ * es) % 16 == 0 && reinterpret_cast<uintptr_t>(src) % 16 == 0;
  const int vout = ldd % 4 == 0 && reinterpret_cast<uintptr_t>(dst) % (4 * es) == 0;
  TSEL(bf, hipLaunchKernelGGL(transpose_k<bf16>, grid, dim3(256), 0, s, (const bf16*)src, rows, cols, lds_, (bf16*)dst, ldd, rows_pad, pm, vin, vout),
       hipLaunchKernelGGL(transpose_k<float>, grid, dim3(256), 0, s, (const float*)src, rows, cols, lds_, (float*)dst, ldd, rows_pad, pm, vin, vout));
}

void rope_bwd(void* dqkv, int n, int H, int hd, const float2* cs, bool bf, hipStream_t s, int parts) {
  const int64_t total = (int64_t)n * H * (hd / 16);
  if (total <= 0 || !(parts & 3)) return;
  TSEL(bf, hipLaunchKernelGGL(rope_bwd_tab_k<bf16>, dim3(nblk(total, 256)), dim3(256), 0, s, (bf16*)dqkv, n, H, hd, cs, parts),
       hipLaunchKernelGGL(rope_bwd_tab_k<float>, dim3(nblk(total, 256)), dim3(256), 0, s, (float*)dqkv, n, H, hd, cs, parts));
}


void convert_weight(const void* src, int rows, int cols, bool transpose, int ilv, void* dst, bool bf,
                    hipStream_t s) {
  dim3 grid(nblk(cols, 32), nblk(rows, 32));
  TSEL(bf, hipLaunchKernelGGL(convert_k<bf16>, grid, dim3(256), 0, s, (const bf16*)src, rows, cols, (int)transpose, ilv, (bf16*)dst),
       hipLaunchKernelGGL(convert_k<float>, grid, dim3(256), 0, s, (const float*)src, rows, cols, (int)transpose, ilv, (float*)dst));
}

void export_weight(const void* w0, const float* delta, int out_dim, int in_dim, int ilv, int which,
                   float* dst, bool bf, hipStream_t s) {
  const int64_t total = (int64_t)out_dim * in_dim;
  TSEL(bf, hipLaunchKernelGGL(export_k<bf16>, dim3(nblk(total, 256)), dim3(256), 0, s, (const bf16*)w0, delta, out_dim, in_dim, ilv, which, dst),
       hipLaunchKernelGGL(export_k<float>, dim3(nblk(total, 256)), dim3(256), 0, s, (const float*)w0, delta, out_dim, in_dim, ilv, which, dst));
}

void ce_finish(const float* part_max, const float* part_sum, int nparts, int64_t ldpart,
               const float* tgt_logit, int n_rows, int n_tgt, float* lse, float* loss_out, int* err,
               hipStream_t s) {
  // rowloss reuses the tail of lse's buffer region provided by the caller:
  // lse has room for 2*n_rows floats.
  float* rowloss = lse + n_rows;
  hipLaunchKernelGGL(ce_rows_k, dim3(nblk(n_rows, 4)), dim3(256), 0, s, part_max, part_sum, nparts, ldpart,
                     tgt_logit, n_rows, n_tgt, lse, rowloss);
  hipLaunchKernelGGL(ce_mean_k, dim3(1), dim3(1024), 0, s, rowloss, n_tgt, loss_out, err);
}

void ce_grad(const float* z, int64_t ldz, const float* lse, const int* tgt, int n_rows, int n_tgt,
             int V, float alpha, void* g, int64_t ldg, bool bf, hipStream_t s) {
  const int64_t total = (int64_t)n_rows * (V / 4);
  if (total <= 0) return;
  TSEL(bf, hipLaunchKernelGGL(ce_grad_k<bf16>, dim3((unsigned)nblk(total, 256)), dim3(256), 0, s, z, ldz, lse, tgt, n_rows, n_tgt, V, alpha, (bf16*)g, ldg),
       hipLaunchKernelGGL(ce_grad_k<float>, dim3((unsigned)nblk(total, 256)), dim3(256), 0, s, z, ldz, lse, tgt, n_rows, n_tgt, V, alpha, (float*)g, ldg));
}

void attn_rowdot(const void* o, const void* dout, int n, int H, int hd, float* D, bool bf,
                 hipStream_t s) {
  const int waves = n * H;
  if (waves <= 0) return;
  TSEL(bf, hipLaunchKernelGGL(rowdot_k<bf16>, dim3(nblk(waves, 4)), dim3(256), 0, s, (const bf16*)o, (const bf16*)dout, n, H, hd, D),
       hipLaunchKernelGGL(rowdot_k<float>, dim3(nblk(waves, 4)), dim3(256), 0, s, (const float*)o, (const float*)dout, n, H, hd, D));
}

}  // namespace ttt
