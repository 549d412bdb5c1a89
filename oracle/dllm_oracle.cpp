// Plain CPU oracle of one token-skipping denoising step, in C++17. TEST INFRASTRUCTURE ONLY.
//
// Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may load or call this
// library (through oracle/cpp.py). The HIP library never routes through it; the two share no
// code, header, table or helper. Built by __graft_entry__.build() with the host compiler.
//
// Arithmetic is float64 with the plain definitions, in the order the pages state them:
//   saliency       ES-dLLM (German summary page) §2.A, importance-score equation:
//                  I = alpha * c + (1 - alpha) * ||H^t - H^(t-1)||_1 / (sqrt(d) ||H^(t-1)||_2);
//                  DyLLM (French summary page) §2.A cosine rule (as 1 - cos); relative L2.
//                  c = the largest softmax probability of the previous step's logits.
//   select         ES-dLLM (German page) §2.B top-k positions proceed; DyLLM §2.A threshold;
//                  DyLLM §2.C: excluded positions (response-only steps) are never candidates.
//   qkv / ffn      ES-dLLM (German page) §2.B: only selected positions are computed; their K/V
//                  and hidden-state cache entries are overwritten in place, the rest reused.
//   attention      DyLLM (French page) §2.B: a salient token's attention row is recomputed
//                  exactly against every cached key; §1: bidirectional, no mask.
//   context        DyLLM (French page) §2.B both paths: the context of every token is the
//                  attention of the query cache (selected rows replaced) against the updated
//                  cache; §2.C: unselected positions before q_first keep their old context.
//   commit         SlowFast (German summary page) "Der SlowFast-Algorithmus" item 2: threshold
//                  commit in the active block, a top-k update when too few pass.
// Readings where the pages are silent (listed with the design notes): pre-norm block with
// RMSNorm, fused QKV rows ordered Q | K | V, kv head = h / (H / Hkv), scale given by the caller
// (1/sqrt(hd)), no positional rotation, SwiGLU FFN with silu(x) = x / (1 + e^-x), residual adds
// around attention and FFN; top-k by (score descending, position ascending), NaN below every
// number, -0 == +0; threshold strict (score > tau) in float32.
//
// Storage: every tensor argument comes with a type code (0 float32, 1 bfloat16 bit patterns,
// 2 float64). The tensors the library stores in its own type -- q rows, K/V cache rows,
// attention outputs, hidden-state rows -- are rounded to the type `store` names (0 float32,
// 1 bfloat16 round-to-nearest-even, 2 float64 = no rounding) and written as float64 values; no
// other value is rounded, except the score, which is the float32 array selection decides on.
//
// Work is split over std::thread workers by independent rows (or (row, head) pairs); each
// result is computed by one worker in a fixed order, so results do not depend on the count.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <thread>
#include <vector>

namespace {

int g_threads = 0;  // 0: OMP_NUM_THREADS when set (the host's CPU share), else every hardware thread

int workers() {
  if (g_threads > 0) return g_threads;
  const unsigned hw = std::thread::hardware_concurrency();
  const int h = hw ? (int)hw : 1;
  if (const char* env = std::getenv("OMP_NUM_THREADS")) {
    const int n = std::atoi(env);
    if (n > 0) return std::min(n, h);
  }
  return h;
}

// f(i) for every i in [0, n), the range cut into one contiguous block per worker
template <class F>
void parallel_for(int64_t n, F f) {
  const int64_t T = std::min<int64_t>(workers(), n);
  if (T <= 1) {
    for (int64_t i = 0; i < n; ++i) f(i);
    return;
  }
  std::vector<std::thread> pool;
  pool.reserve(T);
  for (int64_t t = 0; t < T; ++t)
    pool.emplace_back([=, &f] {
      for (int64_t i = n * t / T; i < n * (t + 1) / T; ++i) f(i);
    });
  for (auto& th : pool) th.join();
}

// ------------------------------------------------------------------ number formats
// bfloat16 = the upper 16 bits of an IEEE binary32 (1 sign, 8 exponent, 7 fraction bits)
double bf16_to_f64(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return (double)f;
}

// nearest bfloat16 value of x, ties to even, from the format's definition: the spacing of
// bfloat16 numbers in the binade of x is 2^(E - 7) (E = unbiased exponent, at least -126, the
// subnormal range sharing the spacing 2^-133); x / spacing is rounded to an integer with ties
// to even (rint in the default rounding mode) and scaled back. Both scalings are by powers of
// two, so they are exact; overflow past the largest finite value gives infinity.
double round_bf16(double x) {
  if (std::isnan(x) || std::isinf(x) || x == 0.0) return x;
  int e;
  std::frexp(std::fabs(x), &e);  // |x| = f 2^e, f in [0.5, 1): unbiased exponent e - 1
  const int E = std::max(e - 1, -126);
  const double q = std::ldexp(1.0, E - 7);
  const double y = std::rint(x / q) * q;
  const double max_bf16 = std::ldexp(255.0, 120);  // (2 - 2^-7) 2^127
  if (std::fabs(y) > max_bf16) return std::copysign(INFINITY, x);
  return y;
}

double store_round(double x, int store) {
  if (store == 0) return (double)(float)x;  // C++ conversion: round to nearest even
  if (store == 1) return round_bf16(x);
  return x;
}

// element i of a typed input array
struct In {
  const void* p;
  int dt;
  double operator[](int64_t i) const {
    if (dt == 1) return bf16_to_f64(static_cast<const uint16_t*>(p)[i]);
    if (dt == 0) return (double)static_cast<const float*>(p)[i];
    return static_cast<const double*>(p)[i];
  }
};

struct Dims {
  int32_t B, S, d, H, Hkv, hd, F;
};

// ------------------------------------------------------------------ building blocks
// sum_k x[k] w[n0 + k]  (x float64, w typed), k ascending
double dot(const double* x, const In& w, int64_t n0, int K) {
  double acc = 0.0;
  for (int k = 0; k < K; ++k) acc += x[k] * w[n0 + k];
  return acc;
}

// y[n] = sum_k x[k] W[n, k] for n in [0, N): one row of x W^T, W stored [N, K]
void row_times_wt(const double* x, const In& W, int N, int K, double* y) {
  for (int n = 0; n < N; ++n) y[n] = dot(x, W, (int64_t)n * K, K);
}

// x / sqrt(mean(x^2) + eps) * g
void rms_norm_row(const double* x, const In& g, int d, double eps, double* out) {
  double ss = 0.0;
  for (int i = 0; i < d; ++i) ss += x[i] * x[i];
  const double r = 1.0 / std::sqrt(ss / d + eps);
  for (int i = 0; i < d; ++i) out[i] = x[i] * r * g[i];
}

double silu(double x) { return x / (1.0 + std::exp(-x)); }

// softmax-weighted sum over keys t of v_t, weights exp(scale q.k_t) normalised; returns the
// log-sum-exp of the scaled scores
double attend(const double* q, const double* k, const double* v, int S, int hd, double scale,
              double* o) {
  std::vector<double> s(S);
  double m = -INFINITY;
  for (int t = 0; t < S; ++t) {
    double a = 0.0;
    for (int e = 0; e < hd; ++e) a += q[e] * k[(int64_t)t * hd + e];
    s[t] = a * scale;
    m = std::max(m, s[t]);
  }
  double l = 0.0;
  for (int t = 0; t < S; ++t) {
    s[t] = std::exp(s[t] - m);
    l += s[t];
  }
  for (int e = 0; e < hd; ++e) o[e] = 0.0;
  for (int t = 0; t < S; ++t) {
    const double p = s[t] / l;
    for (int e = 0; e < hd; ++e) o[e] += p * v[(int64_t)t * hd + e];
  }
  return m + std::log(l);
}

// 1 / sum_v exp(z_v - max z): the largest softmax probability of one logit row; also the
// index of the (first) largest logit
double confidence_row(const In& z, int64_t off, int64_t V, int64_t* arg) {
  double m = -INFINITY;
  int64_t a = 0;
  for (int64_t v = 0; v < V; ++v) {
    const double x = z[off + v];
    if (x > m) {
      m = x;
      a = v;
    }
  }
  double l = 0.0;
  for (int64_t v = 0; v < V; ++v) l += std::exp(z[off + v] - m);
  if (arg) *arg = a;
  return 1.0 / l;
}

}  // namespace

extern "C" {

int ora_version(void) { return 100; }
void ora_set_threads(int n) { g_threads = n > 0 ? n : 0; }
int ora_threads(void) { return workers(); }

double ora_round_bf16(double x) { return round_bf16(x); }

// ------------------------------------------------------------------ (1) saliency
// per token: L1N ||x - y||_1 / (sqrt(d) ||y||_2), COS 1 - <x,y> / (||x|| ||y||), L2R ||x-y|| / ||y||
void ora_delta(int64_t ntok, int d, int kind, const void* x, int x_dt, const void* y, int y_dt,
               double* out) {
  const In X{x, x_dt}, Y{y, y_dt};
  parallel_for(ntok, [&](int64_t r) {
    const int64_t o = r * d;
    double s1 = 0, s2 = 0, sx = 0, sy = 0, sxy = 0;
    for (int i = 0; i < d; ++i) {
      const double a = X[o + i], b = Y[o + i];
      s1 += std::fabs(a - b);
      s2 += (a - b) * (a - b);
      sx += a * a;
      sy += b * b;
      sxy += a * b;
    }
    if (kind == 0) out[r] = s1 / (std::sqrt((double)d) * std::sqrt(sy));
    else if (kind == 1) out[r] = 1.0 - sxy / (std::sqrt(sx) * std::sqrt(sy));
    else out[r] = std::sqrt(s2) / std::sqrt(sy);
  });
}

void ora_confidence(int64_t ntok, int64_t V, const void* z, int z_dt, double* conf,
                    int64_t* arg) {
  const In Z{z, z_dt};
  parallel_for(ntok, [&](int64_t r) {
    conf[r] = confidence_row(Z, r * V, V, arg ? arg + r : nullptr);
  });
}

// score = alpha c + (1 - alpha) v, rounded to float32. c from the logits (or conf_in when no
// logits are given; 0 when neither), v from h_cur / h_prev (0 when they are NULL).
void ora_saliency(int64_t ntok, int d, int64_t V, int kind, double alpha, const void* h_cur,
                  int hc_dt, const void* h_prev, int hp_dt, const void* logits, int lg_dt,
                  const double* conf_in, float* score, double* conf_out, double* delta_out) {
  std::vector<double> c(ntok, 0.0), v(ntok, 0.0);
  if (logits) ora_confidence(ntok, V, logits, lg_dt, c.data(), nullptr);
  else if (conf_in) std::copy(conf_in, conf_in + ntok, c.begin());
  if (h_cur) ora_delta(ntok, d, kind, h_cur, hc_dt, h_prev, hp_dt, v.data());
  for (int64_t r = 0; r < ntok; ++r) {
    score[r] = (float)(alpha * c[r] + (1.0 - alpha) * v[r]);
    if (conf_out) conf_out[r] = c[r];
    if (delta_out) delta_out[r] = v[r];
  }
}

// ------------------------------------------------------------------ (2) selection
// flags: bit 0 forced; else bit 1 excluded; else a candidate (NULL: all candidates).
// mode 1 top-k by (score descending, position ascending; NaN last), mode 0 score > tau.
void ora_select(int B, int S, int mode, float tau, int k, const float* score,
                const uint8_t* flags, int32_t* sel, int32_t* rp) {
  int32_t n = 0;
  rp[0] = 0;
  for (int b = 0; b < B; ++b) {
    const float* sc = score + (int64_t)b * S;
    std::vector<char> take(S, 0);
    std::vector<int> cand;
    for (int s = 0; s < S; ++s) {
      const int f = flags ? flags[(int64_t)b * S + s] : 0;
      if (f & 1) take[s] = 1;
      else if (!(f & 2)) cand.push_back(s);
    }
    if (mode == 1) {
      std::stable_sort(cand.begin(), cand.end(), [&](int a, int c) {
        const bool na = std::isnan(sc[a]), nc = std::isnan(sc[c]);
        if (na != nc) return nc;          // numbers before NaN
        if (na) return a < c;
        if (sc[a] != sc[c]) return sc[a] > sc[c];
        return a < c;
      });
      const int kk = std::min<int>(std::max(k, 0), (int)cand.size());
      for (int i = 0; i < kk; ++i) take[cand[i]] = 1;
    } else {
      for (int s : cand)
        if (sc[s] > tau) take[s] = 1;
    }
    for (int s = 0; s < S; ++s)
      if (take[s]) sel[n++] = b * S + s;
    rp[b + 1] = n;
  }
}

// rows restricted to an earlier selection: listed positions keep bit 0 of `force` (or become
// candidates), every other position is excluded (flag 2)
void ora_flags_from_rows(int B, int S, const uint8_t* force, const int32_t* sel,
                         const int32_t* rp, uint8_t* flags) {
  for (int64_t i = 0; i < (int64_t)B * S; ++i) flags[i] = 2;
  for (int32_t j = 0; j < rp[B]; ++j) flags[sel[j]] = force ? (force[sel[j]] & 1) : 0;
}

// ------------------------------------------------------------------ helpers for the pins
void ora_rms_norm(int64_t rows, int d, const double* x, const double* g, double eps,
                  double* out) {
  const In G{g, 2};
  parallel_for(rows, [&](int64_t r) { rms_norm_row(x + r * d, G, d, eps, out + r * d); });
}

void ora_silu(int64_t n, const double* x, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = silu(x[i]);
}

// ------------------------------------------------------------------ (3) QKV + K/V scatter
// selected row j = (b, s) = (sel[j] / S, sel[j] % S):
//   qkv = RMSNorm(h_in[b, s]) g_attn W_qkv^T; q -> q_sel[j]; k, v -> cache[b, hk, s, :]
void ora_qkv(const Dims* dm, double eps, int store, const void* h_in, int h_dt,
             const void* g_attn, int g_dt, const void* w_qkv, int w_dt, const int32_t* sel,
             const int32_t* rp, double* q_sel, double* k_cache, double* v_cache) {
  const Dims D = *dm;
  const int Nq = D.H * D.hd, Nkv = D.Hkv * D.hd, N = Nq + 2 * Nkv;
  const int32_t M = rp[D.B];
  const In Hin{h_in, h_dt}, G{g_attn, g_dt}, W{w_qkv, w_dt};
  parallel_for(M, [&](int64_t j) {
    const int b = sel[j] / D.S, s = sel[j] % D.S;
    std::vector<double> x(D.d), xn(D.d), y(N);
    for (int i = 0; i < D.d; ++i) x[i] = Hin[((int64_t)b * D.S + s) * D.d + i];
    rms_norm_row(x.data(), G, D.d, eps, xn.data());
    row_times_wt(xn.data(), W, N, D.d, y.data());
    for (int n = 0; n < Nq; ++n) q_sel[j * Nq + n] = store_round(y[n], store);
    for (int hk = 0; hk < D.Hkv; ++hk)
      for (int e = 0; e < D.hd; ++e) {
        const int64_t c = (((int64_t)b * D.Hkv + hk) * D.S + s) * D.hd + e;
        k_cache[c] = store_round(y[Nq + hk * D.hd + e], store);
        v_cache[c] = store_round(y[Nq + Nkv + hk * D.hd + e], store);
      }
  });
}

// ------------------------------------------------------------------ (4) partial attention
// selected row j of sequence b, head h (kv head h / (H / Hkv)): softmax over every key t of
// scale q.k_t, weighted sum of v_t
void ora_attn(const Dims* dm, double scale, int store, const double* q_sel,
              const double* k_cache, const double* v_cache, const int32_t* sel,
              const int32_t* rp, double* o_sel) {
  const Dims D = *dm;
  const int Nq = D.H * D.hd, G = D.H / D.Hkv;
  const int32_t M = rp[D.B];
  parallel_for((int64_t)M * D.H, [&](int64_t jh) {
    const int64_t j = jh / D.H;
    const int h = (int)(jh % D.H), hk = h / G;
    const int b = sel[j] / D.S;
    const int64_t panel = ((int64_t)b * D.Hkv + hk) * D.S * D.hd;
    std::vector<double> o(D.hd);
    attend(q_sel + j * Nq + (int64_t)h * D.hd, k_cache + panel, v_cache + panel, D.S, D.hd,
           scale, o.data());
    for (int e = 0; e < D.hd; ++e) o_sel[j * Nq + (int64_t)h * D.hd + e] = store_round(o[e], store);
  });
}

// ------------------------------------------------------------------ (5) FFN + hidden scatter
// h = h_in[b, s] + o_sel[j] W_o^T; hn = RMSNorm(h) g_ffn;
// h_out[b, s] = h + (silu(hn W_gate^T) * (hn W_up^T)) W_down^T
void ora_ffn(const Dims* dm, double eps, int store, const void* h_in, int h_dt,
             const double* o_sel, const void* w_o, const void* g_ffn, int g_dt,
             const void* w_gate, const void* w_up, const void* w_down, int w_dt,
             const int32_t* sel, const int32_t* rp, double* h_out) {
  const Dims D = *dm;
  const int Nq = D.H * D.hd;
  const int32_t M = rp[D.B];
  const In Hin{h_in, h_dt}, Wo{w_o, w_dt}, G{g_ffn, g_dt}, Wg{w_gate, w_dt}, Wu{w_up, w_dt},
      Wd{w_down, w_dt};
  parallel_for(M, [&](int64_t j) {
    const int64_t row = sel[j];
    std::vector<double> h(D.d), hn(D.d), g(D.F), u(D.F), z(D.F), y(D.d);
    row_times_wt(o_sel + j * Nq, Wo, D.d, Nq, h.data());
    for (int i = 0; i < D.d; ++i) h[i] += Hin[row * D.d + i];
    rms_norm_row(h.data(), G, D.d, eps, hn.data());
    row_times_wt(hn.data(), Wg, D.F, D.d, g.data());
    row_times_wt(hn.data(), Wu, D.F, D.d, u.data());
    for (int f = 0; f < D.F; ++f) z[f] = silu(g[f]) * u[f];
    row_times_wt(z.data(), Wd, D.d, D.F, y.data());
    for (int i = 0; i < D.d; ++i) h_out[row * D.d + i] = store_round(h[i] + y[i], store);
  });
}

// ------------------------------------------------------------------ dense reference block
// The same pre-norm block on every token with full attention, written without selection or
// gathers (pins "select every token == full recompute"). No rounding.
void ora_dense_layer(const Dims* dm, double eps, double scale, const double* h,
                     const double* g_attn, const double* w_qkv, const double* w_o,
                     const double* g_ffn, const double* w_gate, const double* w_up,
                     const double* w_down, double* k_out, double* v_out, double* h_out) {
  const Dims D = *dm;
  const int Nq = D.H * D.hd, Nkv = D.Hkv * D.hd, N = Nq + 2 * Nkv, G = D.H / D.Hkv;
  const int64_t T = (int64_t)D.B * D.S;
  std::vector<double> q(T * Nq), o(T * Nq);
  const In Ga{g_attn, 2}, Wqkv{w_qkv, 2};
  parallel_for(T, [&](int64_t r) {           // projections of every token
    const int b = (int)(r / D.S), s = (int)(r % D.S);
    std::vector<double> xn(D.d), y(N);
    rms_norm_row(h + r * D.d, Ga, D.d, eps, xn.data());
    row_times_wt(xn.data(), Wqkv, N, D.d, y.data());
    for (int n = 0; n < Nq; ++n) q[r * Nq + n] = y[n];
    for (int hk = 0; hk < D.Hkv; ++hk)
      for (int e = 0; e < D.hd; ++e) {
        const int64_t c = (((int64_t)b * D.Hkv + hk) * D.S + s) * D.hd + e;
        k_out[c] = y[Nq + hk * D.hd + e];
        v_out[c] = y[Nq + Nkv + hk * D.hd + e];
      }
  });
  parallel_for(T * D.H, [&](int64_t rh) {     // attention of every token and head
    const int64_t r = rh / D.H;
    const int h = (int)(rh % D.H), b = (int)(r / D.S);
    const int64_t panel = ((int64_t)b * D.Hkv + h / G) * D.S * D.hd;
    attend(q.data() + r * Nq + (int64_t)h * D.hd, k_out + panel, v_out + panel, D.S, D.hd, scale,
           o.data() + r * Nq + (int64_t)h * D.hd);
  });
  const In Wo{w_o, 2}, Gf{g_ffn, 2}, Wg{w_gate, 2}, Wu{w_up, 2}, Wd{w_down, 2};
  parallel_for(T, [&](int64_t r) {           // output projection and FFN of every token
    std::vector<double> a(D.d), hn(D.d), g(D.F), u(D.F), z(D.F), y(D.d);
    row_times_wt(o.data() + r * Nq, Wo, D.d, Nq, a.data());
    for (int i = 0; i < D.d; ++i) a[i] += h[r * D.d + i];
    rms_norm_row(a.data(), Gf, D.d, eps, hn.data());
    row_times_wt(hn.data(), Wg, D.F, D.d, g.data());
    row_times_wt(hn.data(), Wu, D.F, D.d, u.data());
    for (int f = 0; f < D.F; ++f) z[f] = g[f] / (1.0 + std::exp(-g[f])) * u[f];
    row_times_wt(z.data(), Wd, D.d, D.F, y.data());
    for (int i = 0; i < D.d; ++i) h_out[r * D.d + i] = a[i] + y[i];
  });
}

// ------------------------------------------------------------------ context of every token
// copies of the K/V rows at the selected positions: rows[j, hk, :] = cache[b, hk, s, :]
void ora_gather_kv_rows(const Dims* dm, const double* k_cache, const double* v_cache,
                        const int32_t* sel, const int32_t* rp, double* k_rows, double* v_rows) {
  const Dims D = *dm;
  for (int32_t j = 0; j < rp[D.B]; ++j) {
    const int b = sel[j] / D.S, s = sel[j] % D.S;
    for (int hk = 0; hk < D.Hkv; ++hk)
      for (int e = 0; e < D.hd; ++e) {
        const int64_t c = (((int64_t)b * D.Hkv + hk) * D.S + s) * D.hd + e;
        k_rows[((int64_t)j * D.Hkv + hk) * D.hd + e] = k_cache[c];
        v_rows[((int64_t)j * D.Hkv + hk) * D.hd + e] = v_cache[c];
      }
  }
}

// attention of every token's query against every key: o [B, S, H hd], lse [B, S, H]
void ora_context_all(const Dims* dm, double scale, const double* q_all, const double* k_cache,
                     const double* v_cache, double* o, double* lse) {
  const Dims D = *dm;
  const int Nq = D.H * D.hd, G = D.H / D.Hkv;
  parallel_for((int64_t)D.B * D.S * D.H, [&](int64_t rh) {
    const int64_t r = rh / D.H;
    const int h = (int)(rh % D.H), b = (int)(r / D.S);
    const int64_t panel = ((int64_t)b * D.Hkv + h / G) * D.S * D.hd;
    lse[rh] = attend(q_all + r * Nq + (int64_t)h * D.hd, k_cache + panel, v_cache + panel, D.S,
                     D.hd, scale, o + r * Nq + (int64_t)h * D.hd);
  });
}

// DyLLM §2.B / §2.C: the query cache takes the selected rows' new queries; the context of every
// token is its query against the updated cache, except unselected positions s < q_first, which
// keep o_prev / lse_prev. q_all is updated in place; o and lse receive the contexts.
void ora_salient_attention(const Dims* dm, double scale, const double* q_sel, double* q_all,
                           const double* k_cache, const double* v_cache, const int32_t* sel,
                           const int32_t* rp, int q_first, const double* o_prev,
                           const double* lse_prev, double* o, double* lse) {
  const Dims D = *dm;
  const int Nq = D.H * D.hd;
  const int32_t M = rp[D.B];
  std::vector<char> selected((int64_t)D.B * D.S, 0);
  for (int32_t j = 0; j < M; ++j) {
    selected[sel[j]] = 1;
    std::copy(q_sel + (int64_t)j * Nq, q_sel + (int64_t)(j + 1) * Nq, q_all + (int64_t)sel[j] * Nq);
  }
  ora_context_all(dm, scale, q_all, k_cache, v_cache, o, lse);
  if (q_first > 0)
    for (int b = 0; b < D.B; ++b)
      for (int s = 0; s < q_first; ++s) {
        const int64_t p = (int64_t)b * D.S + s;
        if (selected[p]) continue;
        std::copy(o_prev + p * Nq, o_prev + (p + 1) * Nq, o + p * Nq);
        std::copy(lse_prev + p * D.H, lse_prev + (p + 1) * D.H, lse + p * D.H);
      }
}

// ------------------------------------------------------------------ decode loop
// conf and arg of one logit row (largest softmax probability; index of the first largest logit)
void ora_confidence_argmax(int64_t V, const void* z, int z_dt, double* conf, int64_t* arg) {
  const In Z{z, z_dt};
  *conf = confidence_row(Z, 0, V, arg);
}

// SlowFast §2 item 2: per sequence, in the active block [P + blk L, P + (blk + 1) L) (clipped
// to S), the masked positions (tok < 0) commit the n best by (conf descending, position
// ascending), n = max(#{conf > tau}, min(k_min, #masked)), conf compared as float32; a block
// with no masked position left advances blk. flags = 1 over the (new) active block.
// row_of (optional): position b S + s -> row of `logits` holding its logits (NULL: that same
// index), so a caller may pass only the rows of the active blocks.
void ora_commit(int B, int S, int64_t V, const void* logits, int lg_dt, const int32_t* row_of,
                int P, int L, float tau, int k_min, int32_t* tok, int32_t* blk, int32_t* cidx,
                int32_t* crp, uint8_t* flags) {
  const In Z{logits, lg_dt};
  const int nblk = (S - P + L - 1) / L;
  int32_t n_out = 0;
  crp[0] = 0;
  std::memset(flags, 0, (size_t)B * S);
  for (int b = 0; b < B; ++b) {
    if (blk[b] < nblk) {
      const int lo = P + blk[b] * L, hi = std::min(S, lo + L);
      std::vector<int> masked;
      for (int s = lo; s < hi; ++s)
        if (tok[(int64_t)b * S + s] < 0) masked.push_back(s);
      std::vector<float> conf(masked.size());
      std::vector<int64_t> arg(masked.size());
      for (size_t i = 0; i < masked.size(); ++i) {
        const int64_t p = (int64_t)b * S + masked[i];
        conf[i] = (float)confidence_row(Z, (row_of ? row_of[p] : p) * V, V, &arg[i]);
      }
      int above = 0;
      for (float c : conf) above += c > tau;
      const int n = std::max(above, std::min(k_min, (int)masked.size()));
      std::vector<int> order(masked.size());
      for (size_t i = 0; i < order.size(); ++i) order[i] = (int)i;
      std::stable_sort(order.begin(), order.end(), [&](int a, int c) {
        if (conf[a] != conf[c]) return conf[a] > conf[c];
        return masked[a] < masked[c];
      });
      std::vector<int> chosen(order.begin(), order.begin() + n);
      std::sort(chosen.begin(), chosen.end());  // ascending positions (masked is ascending)
      for (int i : chosen) {
        tok[(int64_t)b * S + masked[i]] = (int32_t)arg[i];
        cidx[n_out++] = b * S + masked[i];
      }
      bool done = true;
      for (int s = lo; s < hi; ++s) done = done && tok[(int64_t)b * S + s] >= 0;
      if (done) blk[b] += 1;
    }
    crp[b + 1] = n_out;
    if (blk[b] < nblk) {
      const int lo = P + blk[b] * L, hi = std::min(S, lo + L);
      for (int s = lo; s < hi; ++s) flags[(int64_t)b * S + s] = 1;
    }
  }
}

// x[b, s] = emb[tok[b, s]] for a committed token, mask_emb for a masked one, at listed positions
void ora_embed_rows(int B, int /*S*/, int d, const void* emb, int emb_dt, const void* mask_emb,
                    int mask_dt, const int32_t* tok, const int32_t* sel, const int32_t* rp,
                    double* x) {
  const In E{emb, emb_dt}, Mk{mask_emb, mask_dt};
  for (int32_t j = 0; j < rp[B]; ++j) {
    const int64_t p = sel[j];
    const int32_t t = tok[p];
    for (int i = 0; i < d; ++i) x[p * d + i] = t >= 0 ? E[(int64_t)t * d + i] : Mk[i];
  }
}

}  // extern "C"
