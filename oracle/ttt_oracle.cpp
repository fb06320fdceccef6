// Plain C++ float64 CPU oracle of the TTT-E2E test-time inner loop.
//
// TEST INFRASTRUCTURE ONLY.  Nothing in the product path may load, call or
// link this file or the library built from it: only the tests, the package
// smoke check and the benchmark's CPU-baseline leg do.  It shares no code with
// the HIP path (no header, helper, table or kernel), and none with the numpy
// oracle beside it either: it is a second, independent statement of the same
// computation, written as loops over the textbook definitions.
//
// What it computes (End-to-End Test-Time Training for Long Context):
//  * a decoder-only Transformer whose self-attention is sliding-window
//    attention (paper summary page, "Method"; arXiv abstract);
//  * at test time the model keeps training on its context with next-token
//    cross-entropy measured at the end of the network (NVIDIA blog, "Our
//    method: compressing context into weights"), one gradient step per
//    mini-batch (chunk) of tokens (forum post, TL;DR "Inner Loop");
//  * only the MLPs of the last quarter of the blocks are updated; attention,
//    embeddings and the other blocks stay as loaded (podcast 6:36, 7:08);
//  * optionally each updated block also carries a frozen second MLP that
//    keeps pre-trained knowledge (podcast 7:08), read as a pre-LN residual
//    sublayer after the fast MLP.
//
// Readings where the pages are silent (the same ones the numpy oracle and the
// kernels take): pre-LN blocks; LayerNorm with biased variance, eps from the
// configuration, no affine parameters; a final LayerNorm before an untied
// head; no biases; RoPE on queries and keys with rotate-half pairs
// (i, i + hd/2) and theta_i = base^(-2i/hd), absolute positions, angles in
// float64; attention scale 1/sqrt(hd), query t sees keys j with
// t - W < j <= t; exact erf GELU; chunks cut by input position, position t
// predicts token t+1, the chunk loss is the mean over the chunk's targets and
// is measured before the chunk's update; keys and values of earlier chunks
// are cached as computed when read and are constants for the gradient; with
// several steps the chunk is re-read each step and the last read's keys and
// values are kept; a chunk without targets is read and cached, makes no
// update and reports loss 0; greedy decoding takes the lowest id on ties,
// continues the chunk grid and a completed decode chunk makes the same update.
//
// Layout: every projection is [in][out] row-major (y = x W), the canonical
// order of the seeded weight generator: E [V][d]; per layer Wq, Wk, Wv, Wo
// [d][d], then W1 [d][F], W2 [F][d] (GELU) or Wg, Wu [d][F], Wd [F][d]
// (SwiGLU), then the frozen second MLP of a fast layer when configured; U
// [d][V] last.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <deque>
#include <string>
#include <vector>

namespace {

using Vec = std::vector<double>;

constexpr double kPi = 3.14159265358979323846;

struct Config {
  int n_layers, d, H, hd, F, V, W, n_fast, swiglu, static_mlp;
  double rope_base, ln_eps;
};

// ---------------------------------------------------------------- products
// C[n][m] = A[n][k] B[k][m]
Vec mm(const Vec& A, const Vec& B, int n, int k, int m) {
  Vec C((size_t)n * m, 0.0);
#pragma omp parallel for schedule(static)
  for (int i = 0; i < n; ++i) {
    double* c = &C[(size_t)i * m];
    for (int p = 0; p < k; ++p) {
      const double a = A[(size_t)i * k + p];
      const double* b = &B[(size_t)p * m];
      for (int j = 0; j < m; ++j) c[j] += a * b[j];
    }
  }
  return C;
}

// C[n][m] = A[n][k] B[m][k]^T  (B given [m][k])
Vec mm_bt(const Vec& A, const Vec& B, int n, int k, int m) {
  Vec C((size_t)n * m, 0.0);
#pragma omp parallel for schedule(static)
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < m; ++j) {
      double s = 0.0;
      for (int p = 0; p < k; ++p) s += A[(size_t)i * k + p] * B[(size_t)j * k + p];
      C[(size_t)i * m + j] = s;
    }
  return C;
}

// C[k][m] = A[n][k]^T B[n][m]  (the weight gradient of y = x W: x^T dy)
Vec mm_at(const Vec& A, const Vec& B, int n, int k, int m) {
  Vec C((size_t)k * m, 0.0);
#pragma omp parallel for schedule(static)
  for (int p = 0; p < k; ++p) {
    double* c = &C[(size_t)p * m];
    for (int i = 0; i < n; ++i) {
      const double a = A[(size_t)i * k + p];
      const double* b = &B[(size_t)i * m];
      for (int j = 0; j < m; ++j) c[j] += a * b[j];
    }
  }
  return C;
}

void add_into(Vec& a, const Vec& b) {
  for (size_t i = 0; i < a.size(); ++i) a[i] += b[i];
}

// ------------------------------------------------------------- LayerNorm
// y = (x - mean) / sqrt(var + eps) per row (biased variance, no affine)
void layer_norm(const Vec& x, int n, int d, double eps, Vec& y, Vec& rstd) {
  y.assign((size_t)n * d, 0.0);
  rstd.assign(n, 0.0);
  for (int i = 0; i < n; ++i) {
    const double* r = &x[(size_t)i * d];
    double mu = 0.0;
    for (int j = 0; j < d; ++j) mu += r[j];
    mu /= d;
    double var = 0.0;
    for (int j = 0; j < d; ++j) var += (r[j] - mu) * (r[j] - mu);
    var /= d;
    const double rs = 1.0 / std::sqrt(var + eps);
    rstd[i] = rs;
    for (int j = 0; j < d; ++j) y[(size_t)i * d + j] = (r[j] - mu) * rs;
  }
}

// dx = rstd (dy - mean(dy) - y mean(dy y)) per row
Vec layer_norm_bwd(const Vec& dy, const Vec& y, const Vec& rstd, int n, int d) {
  Vec dx((size_t)n * d);
  for (int i = 0; i < n; ++i) {
    double m1 = 0.0, m2 = 0.0;
    for (int j = 0; j < d; ++j) {
      m1 += dy[(size_t)i * d + j];
      m2 += dy[(size_t)i * d + j] * y[(size_t)i * d + j];
    }
    m1 /= d;
    m2 /= d;
    for (int j = 0; j < d; ++j)
      dx[(size_t)i * d + j] = rstd[i] * (dy[(size_t)i * d + j] - m1 - y[(size_t)i * d + j] * m2);
  }
  return dx;
}

// ------------------------------------------------------------------ RoPE
// x [n][H*hd], row i at position pos[i]; pair (c, c + hd/2) of each head is
// rotated by pos * base^(-2c/hd) (sign = +1) or by its negative (sign = -1,
// the transpose, used by the backward pass).
void rope(Vec& x, int n, int H, int hd, const int64_t* pos, double base, int sign) {
  const int half = hd / 2;
  for (int i = 0; i < n; ++i)
    for (int c = 0; c < half; ++c) {
      const double theta = std::pow(base, -2.0 * c / hd);
      const double ang = (double)pos[i] * theta;
      const double cs = std::cos(ang), sn = sign * std::sin(ang);
      for (int h = 0; h < H; ++h) {
        double* v = &x[(size_t)i * H * hd + (size_t)h * hd];
        const double a = v[c], b = v[c + half];
        v[c] = a * cs - b * sn;
        v[c + half] = b * cs + a * sn;
      }
    }
}

// ----------------------------------------------------------- activations
double gelu(double z) { return 0.5 * z * (1.0 + std::erf(z / std::sqrt(2.0))); }
double gelu_d(double z) {
  return 0.5 * (1.0 + std::erf(z / std::sqrt(2.0))) + z * std::exp(-0.5 * z * z) / std::sqrt(2.0 * kPi);
}
double sigm(double z) { return 1.0 / (1.0 + std::exp(-z)); }

// ------------------------------------------------------------- attention
// Banded causal attention of nq queries over nk keys (positions qpos, kpos):
// P[h][t][j] = softmax_j(q_t . k_j / sqrt(hd)) over t - W < pos_j <= pos_t,
// o_t = sum_j P v_j.  P is returned dense (zeros outside the band).
void attention(const Vec& q, const Vec& k, const Vec& v, int nq, int nk, int H, int hd,
               const int64_t* qpos, const int64_t* kpos, int64_t W, Vec& o, Vec& P) {
  const int D = H * hd;
  const double scale = 1.0 / std::sqrt((double)hd);
  o.assign((size_t)nq * D, 0.0);
  P.assign((size_t)H * nq * nk, 0.0);
#pragma omp parallel for collapse(2) schedule(static)
  for (int h = 0; h < H; ++h)
    for (int t = 0; t < nq; ++t) {
      double* p = &P[((size_t)h * nq + t) * nk];
      double mx = -INFINITY;
      for (int j = 0; j < nk; ++j) {
        if (!(kpos[j] <= qpos[t] && kpos[j] > qpos[t] - W)) continue;
        double s = 0.0;
        for (int c = 0; c < hd; ++c) s += q[(size_t)t * D + h * hd + c] * k[(size_t)j * D + h * hd + c];
        p[j] = s * scale;
        if (p[j] > mx) mx = p[j];
      }
      double sum = 0.0;
      for (int j = 0; j < nk; ++j) {
        if (!(kpos[j] <= qpos[t] && kpos[j] > qpos[t] - W)) continue;
        p[j] = std::exp(p[j] - mx);
        sum += p[j];
      }
      for (int j = 0; j < nk; ++j) p[j] /= sum;
      for (int j = 0; j < nk; ++j) {
        if (p[j] == 0.0) continue;
        for (int c = 0; c < hd; ++c) o[(size_t)t * D + h * hd + c] += p[j] * v[(size_t)j * D + h * hd + c];
      }
    }
}

// Gradients of o = P V with P = softmax(q k^T / sqrt(hd)) (masked entries
// have P = 0): dV = P^T dO, dP = dO V^T, dS = P (dP - rowsum(P dP)),
// dQ = dS K / sqrt(hd), dK = dS^T Q / sqrt(hd).
void attention_bwd(const Vec& dO, const Vec& q, const Vec& k, const Vec& v, const Vec& P, int nq,
                   int nk, int H, int hd, Vec& dq, Vec& dk, Vec& dv) {
  const int D = H * hd;
  const double scale = 1.0 / std::sqrt((double)hd);
  dq.assign((size_t)nq * D, 0.0);
  dk.assign((size_t)nk * D, 0.0);
  dv.assign((size_t)nk * D, 0.0);
#pragma omp parallel for schedule(static)
  for (int h = 0; h < H; ++h) {
    Vec ds(nk);
    for (int t = 0; t < nq; ++t) {
      const double* p = &P[((size_t)h * nq + t) * nk];
      double rs = 0.0;
      for (int j = 0; j < nk; ++j) {
        double dp = 0.0;
        for (int c = 0; c < hd; ++c) dp += dO[(size_t)t * D + h * hd + c] * v[(size_t)j * D + h * hd + c];
        ds[j] = dp;
        rs += p[j] * dp;
      }
      for (int j = 0; j < nk; ++j) {
        const double s = p[j] * (ds[j] - rs);
        for (int c = 0; c < hd; ++c) {
          dv[(size_t)j * D + h * hd + c] += p[j] * dO[(size_t)t * D + h * hd + c];
          dq[(size_t)t * D + h * hd + c] += s * k[(size_t)j * D + h * hd + c] * scale;
          dk[(size_t)j * D + h * hd + c] += s * q[(size_t)t * D + h * hd + c] * scale;
        }
      }
    }
  }
}

// ------------------------------------------------------------------ MLPs
struct MLP {
  Vec m[3];  // GELU: W1 [d][F], W2 [F][d]; SwiGLU: Wg, Wu [d][F], Wd [F][d]
};

struct MLPAct {
  Vec z, u, a;  // pre-activations (GELU: z; SwiGLU: gate z and up u) and the product input a
};

Vec mlp_fwd(const Config& c, const MLP& w, const Vec& b, int n, MLPAct& act) {
  if (!c.swiglu) {
    act.z = mm(b, w.m[0], n, c.d, c.F);
    act.a.resize(act.z.size());
    for (size_t i = 0; i < act.z.size(); ++i) act.a[i] = gelu(act.z[i]);
    return mm(act.a, w.m[1], n, c.F, c.d);
  }
  act.z = mm(b, w.m[0], n, c.d, c.F);
  act.u = mm(b, w.m[1], n, c.d, c.F);
  act.a.resize(act.z.size());
  for (size_t i = 0; i < act.z.size(); ++i) act.a[i] = act.z[i] * sigm(act.z[i]) * act.u[i];
  return mm(act.a, w.m[2], n, c.F, c.d);
}

// Backward of y = mlp(b): weight gradients (if grads != nullptr) and, if
// asked, the input gradient db.
void mlp_bwd(const Config& c, const MLP& w, const Vec& b, const MLPAct& act, const Vec& dy, int n,
             MLP* grads, Vec* db) {
  const int nm = c.swiglu ? 3 : 2;
  const Vec& Wout = w.m[nm - 1];
  if (grads) grads->m[nm - 1] = mm_at(act.a, dy, n, c.F, c.d);
  Vec da = mm_bt(dy, Wout, n, c.d, c.F);
  if (!c.swiglu) {
    Vec dz(da.size());
    for (size_t i = 0; i < da.size(); ++i) dz[i] = da[i] * gelu_d(act.z[i]);
    if (grads) grads->m[0] = mm_at(b, dz, n, c.d, c.F);
    if (db) *db = mm_bt(dz, w.m[0], n, c.F, c.d);
    return;
  }
  Vec dg(da.size()), du(da.size());
  for (size_t i = 0; i < da.size(); ++i) {
    const double g = act.z[i], s = sigm(g);
    dg[i] = da[i] * act.u[i] * s * (1.0 + g * (1.0 - s));
    du[i] = da[i] * g * s;
  }
  if (grads) {
    grads->m[0] = mm_at(b, dg, n, c.d, c.F);
    grads->m[1] = mm_at(b, du, n, c.d, c.F);
  }
  if (db) {
    *db = mm_bt(dg, w.m[0], n, c.F, c.d);
    add_into(*db, mm_bt(du, w.m[1], n, c.F, c.d));
  }
}

// ----------------------------------------------------------------- model
struct Layer {
  Vec Wq, Wk, Wv, Wo;
  MLP mlp;
  MLP stat;  // frozen second MLP (fast layers with static_mlp)
};

struct KV {  // one layer's cached keys (post-RoPE) and values, oldest first
  std::deque<int64_t> pos;
  std::deque<Vec> k, v;
};

struct LayerAct {  // what a chunk's forward keeps of one layer
  Vec k, v;                       // new keys (post-RoPE) and values: the cache
  Vec h, a, r1, q, kall, vall, h2; // attention of fast layers above the first
  std::vector<int64_t> kpos;
  int ncache = 0;
  Vec P;
  Vec b, r2;                      // MLP input of fast layers
  MLPAct mact;
  Vec cst, r3;                    // frozen second MLP's input
  MLPAct mact2;
};

struct Fwd {
  std::vector<LayerAct> L;
  Vec f, rf, logits;
  std::vector<int64_t> pos;
};

struct Model {
  Config c;
  Vec E, U;
  std::vector<Layer> layers;
  std::vector<MLP> fast;  // current fast weights (float64) of layers L - n_fast .. L-1
  std::vector<KV> cache;
  int64_t T = 0;          // positions read so far (decode continues from here)
  int64_t pos_offset = 0;
  int chunk = 0, steps = 1;
  double lr = 0.0;
  Vec last_logits;
  std::string err;
};

int first_fast(const Config& c) { return c.n_layers - c.n_fast; }
int n_mlp(const Config& c) { return c.swiglu ? 3 : 2; }

// Forward of n tokens at positions pos0.. through every layer with the
// current fast weights; attention reads the given cache plus the chunk's own
// keys (causal).
Fwd forward(const Model& M, const std::vector<MLP>& fast, const std::vector<KV>& cache,
            const int32_t* tok, int n, int64_t pos0) {
  const Config& c = M.c;
  const int d = c.d;
  Fwd fw;
  fw.L.resize(c.n_layers);
  fw.pos.resize(n);
  for (int i = 0; i < n; ++i) fw.pos[i] = pos0 + i;
  Vec h((size_t)n * d);
  for (int i = 0; i < n; ++i)
    std::memcpy(&h[(size_t)i * d], &M.E[(size_t)tok[i] * d], sizeof(double) * d);
  for (int l = 0; l < c.n_layers; ++l) {
    const Layer& Wl = M.layers[l];
    const int fl = l - first_fast(c);
    LayerAct& A = fw.L[l];
    Vec a, r1;
    layer_norm(h, n, d, c.ln_eps, a, r1);
    Vec q = mm(a, Wl.Wq, n, d, d), k = mm(a, Wl.Wk, n, d, d), v = mm(a, Wl.Wv, n, d, d);
    rope(q, n, c.H, c.hd, fw.pos.data(), c.rope_base, +1);
    rope(k, n, c.H, c.hd, fw.pos.data(), c.rope_base, +1);
    const KV& kv = cache[l];
    const int nc = (int)kv.pos.size(), nk = nc + n;
    Vec kall((size_t)nk * d), vall((size_t)nk * d);
    std::vector<int64_t> kpos(nk);
    for (int j = 0; j < nc; ++j) {
      std::memcpy(&kall[(size_t)j * d], kv.k[j].data(), sizeof(double) * d);
      std::memcpy(&vall[(size_t)j * d], kv.v[j].data(), sizeof(double) * d);
      kpos[j] = kv.pos[j];
    }
    std::memcpy(&kall[(size_t)nc * d], k.data(), sizeof(double) * n * d);
    std::memcpy(&vall[(size_t)nc * d], v.data(), sizeof(double) * n * d);
    for (int i = 0; i < n; ++i) kpos[nc + i] = fw.pos[i];
    Vec o, P;
    attention(q, kall, vall, n, nk, c.H, c.hd, fw.pos.data(), kpos.data(), c.W, o, P);
    Vec h2 = mm(o, Wl.Wo, n, d, d);
    add_into(h2, h);
    Vec b, r2;
    layer_norm(h2, n, d, c.ln_eps, b, r2);
    MLPAct mact;
    Vec m = mlp_fwd(c, fl >= 0 ? fast[fl] : Wl.mlp, b, n, mact);
    A.k = k;
    A.v = v;
    if (fl >= 0) {
      A.b = b;
      A.r2 = r2;
      A.mact = std::move(mact);
    }
    if (fl > 0) {
      A.h = h;
      A.a = a;
      A.r1 = r1;
      A.q = q;
      A.kall = std::move(kall);
      A.vall = std::move(vall);
      A.kpos = kpos;
      A.ncache = nc;
      A.P = std::move(P);
      A.h2 = h2;
    }
    h = h2;
    add_into(h, m);
    if (fl >= 0 && c.static_mlp) {
      layer_norm(h, n, d, c.ln_eps, A.cst, A.r3);
      Vec m2 = mlp_fwd(c, Wl.stat, A.cst, n, A.mact2);
      add_into(h, m2);
    }
  }
  layer_norm(h, n, d, c.ln_eps, fw.f, fw.rf);
  fw.logits = mm(fw.f, M.U, n, d, c.V);
  return fw;
}

// Mean next-token CE over the first m rows (rows past m have no target) and
// its gradient with respect to the logits.
double cross_entropy(const Vec& logits, int n, int V, const int32_t* tgt, int m, Vec& dlog) {
  dlog.assign((size_t)n * V, 0.0);
  if (m == 0) return 0.0;
  double total = 0.0;
  for (int i = 0; i < m; ++i) {
    const double* z = &logits[(size_t)i * V];
    double mx = z[0];
    for (int j = 1; j < V; ++j) mx = z[j] > mx ? z[j] : mx;
    double s = 0.0;
    for (int j = 0; j < V; ++j) s += std::exp(z[j] - mx);
    const double lse = mx + std::log(s);
    total += lse - z[tgt[i]];
    for (int j = 0; j < V; ++j) dlog[(size_t)i * V + j] = std::exp(z[j] - lse) / m;
    dlog[(size_t)i * V + tgt[i]] -= 1.0 / m;
  }
  return total / m;
}

// Gradient of the chunk loss with respect to the fast weights only; the
// pass stops at the lowest fast MLP and cached keys/values are constants.
std::vector<MLP> backward(const Model& M, const std::vector<MLP>& fast, const Fwd& fw,
                          const Vec& dlog) {
  const Config& c = M.c;
  const int d = c.d, n = (int)fw.pos.size();
  std::vector<MLP> grads(c.n_fast);
  Vec df = mm_bt(dlog, M.U, n, c.V, d);
  Vec dh = layer_norm_bwd(df, fw.f, fw.rf, n, d);
  for (int l = c.n_layers - 1; l >= first_fast(c); --l) {
    const LayerAct& A = fw.L[l];
    const Layer& Wl = M.layers[l];
    const int fl = l - first_fast(c);
    const bool need = l > first_fast(c);
    if (c.static_mlp) {
      Vec dcst;
      mlp_bwd(c, Wl.stat, A.cst, A.mact2, dh, n, nullptr, &dcst);
      add_into(dh, layer_norm_bwd(dcst, A.cst, A.r3, n, d));
    }
    Vec db;
    mlp_bwd(c, fast[fl], A.b, A.mact, dh, n, &grads[fl], need ? &db : nullptr);
    if (!need) break;
    Vec dh2 = dh;
    add_into(dh2, layer_norm_bwd(db, A.b, A.r2, n, d));
    Vec dO = mm_bt(dh2, Wl.Wo, n, d, d);
    const int nk = (int)A.kpos.size();
    Vec dq, dkall, dvall;
    attention_bwd(dO, A.q, A.kall, A.vall, A.P, n, nk, c.H, c.hd, dq, dkall, dvall);
    // the cached rows (the first ncache keys) get no gradient
    Vec dk(dkall.begin() + (size_t)A.ncache * d, dkall.end());
    Vec dv(dvall.begin() + (size_t)A.ncache * d, dvall.end());
    rope(dq, n, c.H, c.hd, fw.pos.data(), c.rope_base, -1);
    rope(dk, n, c.H, c.hd, fw.pos.data(), c.rope_base, -1);
    Vec da = mm_bt(dq, Wl.Wq, n, d, d);
    add_into(da, mm_bt(dk, Wl.Wk, n, d, d));
    add_into(da, mm_bt(dv, Wl.Wv, n, d, d));
    dh = dh2;
    add_into(dh, layer_norm_bwd(da, A.a, A.r1, n, d));
  }
  return grads;
}

void sgd(const Config& c, std::vector<MLP>& fast, const std::vector<MLP>& grads, double lr) {
  for (int f = 0; f < c.n_fast; ++f)
    for (int j = 0; j < n_mlp(c); ++j)
      for (size_t i = 0; i < fast[f].m[j].size(); ++i) fast[f].m[j][i] -= lr * grads[f].m[j][i];
}

// Append the chunk's keys/values (its last read) to every layer's cache,
// keeping the newest `keep` positions.
void commit(const Config& c, std::vector<KV>& cache, const Fwd& fw, int64_t keep) {
  const int n = (int)fw.pos.size(), d = c.d;
  for (int l = 0; l < c.n_layers; ++l) {
    KV& kv = cache[l];
    for (int i = 0; i < n; ++i) {
      kv.pos.push_back(fw.pos[i]);
      kv.k.emplace_back(fw.L[l].k.begin() + (size_t)i * d, fw.L[l].k.begin() + (size_t)(i + 1) * d);
      kv.v.emplace_back(fw.L[l].v.begin() + (size_t)i * d, fw.L[l].v.begin() + (size_t)(i + 1) * d);
    }
    while ((int64_t)kv.pos.size() > keep) {
      kv.pos.pop_front();
      kv.k.pop_front();
      kv.v.pop_front();
    }
  }
}

std::vector<MLP> initial_fast(const Model& M) {
  std::vector<MLP> f;
  for (int l = first_fast(M.c); l < M.c.n_layers; ++l) f.push_back(M.layers[l].mlp);
  return f;
}

int argmax_lowest(const double* z, int V) {
  int best = 0;
  for (int j = 1; j < V; ++j)
    if (z[j] > z[best]) best = j;
  return best;
}

}  // namespace

// ======================================================================
// C ABI (ctypes)
// ======================================================================
extern "C" {

struct orc_config {
  int32_t n_layers, d_model, n_heads, head_dim, d_ff, vocab, window, n_fast, swiglu, static_mlp;
  double rope_base, ln_eps;
};

// Number of weight matrices the configuration takes (canonical order).
int orc_n_weights(const orc_config* cfg) {
  const int nm = cfg->swiglu ? 3 : 2;
  return 2 + cfg->n_layers * (4 + nm) + (cfg->static_mlp ? cfg->n_fast * nm : 0);
}

// New model from float64 weights in canonical order and [in][out] layout
// (the pointers are read once; the model keeps its own copies).
void* orc_model_new(const orc_config* cfg, const double* const* w) {
  Model* M = new Model();
  Config& c = M->c;
  c = Config{cfg->n_layers, cfg->d_model, cfg->n_heads, cfg->head_dim, cfg->d_ff, cfg->vocab,
             cfg->window, cfg->n_fast, cfg->swiglu, cfg->static_mlp, cfg->rope_base, cfg->ln_eps};
  const int d = c.d, F = c.F, V = c.V, nm = n_mlp(c);
  auto take = [&](const double* p, size_t n) { return Vec(p, p + n); };
  int i = 0;
  M->E = take(w[i++], (size_t)V * d);
  M->layers.resize(c.n_layers);
  for (int l = 0; l < c.n_layers; ++l) {
    Layer& L = M->layers[l];
    L.Wq = take(w[i++], (size_t)d * d);
    L.Wk = take(w[i++], (size_t)d * d);
    L.Wv = take(w[i++], (size_t)d * d);
    L.Wo = take(w[i++], (size_t)d * d);
    for (int j = 0; j < nm; ++j) L.mlp.m[j] = take(w[i++], (size_t)d * F);
    if (c.static_mlp && l >= first_fast(c))
      for (int j = 0; j < nm; ++j) L.stat.m[j] = take(w[i++], (size_t)d * F);
  }
  M->U = take(w[i++], (size_t)d * V);
  M->fast = initial_fast(*M);
  M->cache.assign(c.n_layers, KV());
  return M;
}

void orc_model_free(void* m) { delete static_cast<Model*>(m); }

// The inner loop over a whole context, from the initial fast weights and an
// empty cache.  losses gets n_chunks * steps values (every step's loss,
// measured before its update); last_logits (may be null) the logits of the
// context's last position.  The model keeps the state for orc_decode.
int orc_prefill(void* m, const int32_t* tok, int64_t T, int32_t chunk, double lr, int32_t steps,
                int64_t pos_offset, double* losses, double* last_logits) {
  Model& M = *static_cast<Model*>(m);
  const Config& c = M.c;
  if (chunk < 1 || steps < 1 || T < 1) return 1;
  M.fast = initial_fast(M);
  M.cache.assign(c.n_layers, KV());
  M.chunk = chunk;
  M.steps = steps;
  M.lr = lr;
  M.pos_offset = pos_offset;
  const int64_t keep = (int64_t)c.W + chunk;
  const int64_t nch = (T + chunk - 1) / chunk;
  int64_t li = 0;
  Fwd fw;
  for (int64_t kk = 0; kk < nch; ++kk) {
    const int64_t p0 = kk * chunk, p1 = std::min<int64_t>(p0 + chunk, T);
    const int n = (int)(p1 - p0);
    const int mt = (int)(std::min<int64_t>(p1 + 1, T) - (p0 + 1));
    for (int s = 0; s < steps; ++s) {
      fw = forward(M, M.fast, M.cache, tok + p0, n, p0 + pos_offset);
      Vec dl;
      losses[li++] = cross_entropy(fw.logits, n, c.V, tok + p0 + 1, mt, dl);
      if (mt > 0) sgd(c, M.fast, backward(M, M.fast, fw, dl), lr);
    }
    commit(c, M.cache, fw, keep);
    if (kk == nch - 1) M.last_logits.assign(fw.logits.end() - c.V, fw.logits.end());
  }
  if (last_logits) std::memcpy(last_logits, M.last_logits.data(), sizeof(double) * c.V);
  M.T = T;
  return 0;
}

// Greedy decode of n tokens after orc_prefill: position T + i is read with
// the current fast weights and its keys/values join the cache; the next token
// is the argmax of its logits (lowest id on ties) unless forced (n entries,
// or null) gives it.  When the decode positions of a chunk are complete the
// chunk is re-read from the cache as it stood before it and makes the
// prefill's update; its losses go to update_losses (n_updates counts them).
int orc_decode(void* m, int32_t n, const int32_t* forced, int32_t* out_tok, double* out_logits,
               double* update_losses, int32_t* n_updates) {
  Model& M = *static_cast<Model*>(m);
  const Config& c = M.c;
  const int C = M.chunk;
  if (C < 1 || M.last_logits.empty()) return 1;
  const int64_t keep = (int64_t)c.W + C, T0 = M.T, off = M.pos_offset;
  int nxt = forced ? forced[0] : argmax_lowest(M.last_logits.data(), c.V);
  std::vector<int32_t> ctoks;
  int nu = 0;
  for (int i = 0; i < n; ++i) {
    const int64_t p = T0 + i;
    const int32_t tk = nxt;
    out_tok[i] = tk;
    ctoks.push_back(tk);
    Fwd fw = forward(M, M.fast, M.cache, &tk, 1, p + off);
    commit(c, M.cache, fw, keep);
    std::memcpy(out_logits + (size_t)i * c.V, fw.logits.data(), sizeof(double) * c.V);
    nxt = (forced && i + 1 < n) ? forced[i + 1] : argmax_lowest(fw.logits.data(), c.V);
    if ((i + 1) % C == 0) {
      const int64_t c0 = p + 1 - C;
      std::vector<int32_t> tgt(ctoks.begin() + 1, ctoks.end());
      tgt.push_back(nxt);
      std::vector<KV> before(c.n_layers);
      for (int l = 0; l < c.n_layers; ++l)
        for (size_t j = 0; j < M.cache[l].pos.size(); ++j)
          if (M.cache[l].pos[j] < c0 + off) {
            before[l].pos.push_back(M.cache[l].pos[j]);
            before[l].k.push_back(M.cache[l].k[j]);
            before[l].v.push_back(M.cache[l].v[j]);
          }
      Fwd fwc;
      for (int s = 0; s < M.steps; ++s) {
        fwc = forward(M, M.fast, before, ctoks.data(), C, c0 + off);
        Vec dl;
        update_losses[nu++] = cross_entropy(fwc.logits, C, c.V, tgt.data(), C, dl);
        sgd(c, M.fast, backward(M, M.fast, fwc, dl), M.lr);
      }
      commit(c, before, fwc, keep);
      M.cache = std::move(before);
      ctoks.clear();
    }
  }
  M.T = T0 + n;
  M.last_logits.clear();
  if (n_updates) *n_updates = nu;
  return 0;
}

// Current fast matrix j (canonical MLP order) of fast layer f, [in][out].
int orc_fast_weight(void* m, int32_t f, int32_t j, double* out) {
  Model& M = *static_cast<Model*>(m);
  if (f < 0 || f >= M.c.n_fast || j < 0 || j >= n_mlp(M.c)) return 1;
  std::memcpy(out, M.fast[f].m[j].data(), sizeof(double) * M.fast[f].m[j].size());
  return 0;
}

int orc_set_fast_weight(void* m, int32_t f, int32_t j, const double* in) {
  Model& M = *static_cast<Model*>(m);
  if (f < 0 || f >= M.c.n_fast || j < 0 || j >= n_mlp(M.c)) return 1;
  std::memcpy(M.fast[f].m[j].data(), in, sizeof(double) * M.fast[f].m[j].size());
  return 0;
}

// Loss of n tokens at pos0.. (targets: the first mt rows) over the current
// cache and fast weights, and its fast-weight gradient (grads: per fast
// layer, per matrix, concatenated; may be null).  Changes nothing.
double orc_chunk_loss_grad(void* m, const int32_t* tok, int32_t n, const int32_t* tgt, int32_t mt,
                           int64_t pos0, double* grads) {
  Model& M = *static_cast<Model*>(m);
  Fwd fw = forward(M, M.fast, M.cache, tok, n, pos0);
  Vec dl;
  const double loss = cross_entropy(fw.logits, n, M.c.V, tgt, mt, dl);
  if (grads) {
    std::vector<MLP> g = backward(M, M.fast, fw, dl);
    size_t o = 0;
    for (int f = 0; f < M.c.n_fast; ++f)
      for (int j = 0; j < n_mlp(M.c); ++j) {
        std::memcpy(grads + o, g[f].m[j].data(), sizeof(double) * g[f].m[j].size());
        o += g[f].m[j].size();
      }
  }
  return loss;
}

// Read n tokens at pos0.. into the cache without any update (the state a
// finite-difference check starts from).
int orc_read(void* m, const int32_t* tok, int32_t n, int64_t pos0, int32_t keep_extra) {
  Model& M = *static_cast<Model*>(m);
  Fwd fw = forward(M, M.fast, M.cache, tok, n, pos0);
  commit(M.c, M.cache, fw, (int64_t)M.c.W + keep_extra);
  return 0;
}

// Elementary pieces exposed for their own pins.
void orc_rope(double* x, int32_t n, int32_t H, int32_t hd, const int64_t* pos, double base,
              int32_t sign) {
  Vec v(x, x + (size_t)n * H * hd);
  rope(v, n, H, hd, pos, base, sign);
  std::memcpy(x, v.data(), sizeof(double) * v.size());
}

void orc_layer_norm(const double* x, int32_t n, int32_t d, double eps, double* y) {
  Vec xv(x, x + (size_t)n * d), yv, r;
  layer_norm(xv, n, d, eps, yv, r);
  std::memcpy(y, yv.data(), sizeof(double) * yv.size());
}

void orc_attention(const double* q, const double* k, const double* v, int32_t nq, int32_t nk,
                   int32_t H, int32_t hd, const int64_t* qpos, const int64_t* kpos, int64_t W,
                   double* o) {
  const size_t D = (size_t)H * hd;
  Vec qv(q, q + nq * D), kv(k, k + nk * D), vv(v, v + nk * D), ov, P;
  attention(qv, kv, vv, nq, nk, H, hd, qpos, kpos, W, ov, P);
  std::memcpy(o, ov.data(), sizeof(double) * ov.size());
}

}  // extern "C"
