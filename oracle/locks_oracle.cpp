// Plain fp64 CPU oracle for the Locks decode-step path.
//
// TEST INFRASTRUCTURE ONLY. Nothing in the product path may load, call or link
// this file: only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline
// leg use it. It shares no code, header, table or helper with the HIP library.
//
// Source of every formula: "Locks: Page-Local Compact Key Summaries for
// Efficient Long-Context Decoding" (J. Hwang, arXiv 2607.24555), cited below
// as [Locks] with the section / equation it follows.
//
// Everything is written for clarity, not speed: plain loops in double
// precision, no BLAS, no blocking, no fusion. Inputs are the stored values
// (bf16 or fp32) already widened exactly to double by the caller.
//
// Layout conventions (all row-major, contiguous):
//   keys  [n_pages][P][d]      one page = P consecutive tokens
//   mu    [n_pages][d]         page centroid
//   vt    [n_pages][r][d]      row rho = basis vector phi_rho (column rho of V)
//   coef  [n_pages][P][r]      row i = c_i = V^T (k_i - mu)
//   q     [G][d]               the G query heads sharing one KV head
//
// Readings where the paper leaves a step open (each one restated where used):
//   * eigenvector sign: the largest-magnitude entry of each basis vector is
//     made positive (lowest index on ties); equal eigenvalues keep index order.
//   * the sink page is logical page 0; the "most recent page" is page J-1,
//     the page that holds the newest token (it may be partial).
//   * only complete pages carry a summary; the partial page is never a
//     candidate and is not part of the per-head normaliser.
//   * ties in the ranking key go to the lower page id.

#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>
#include <algorithm>

namespace {

// Cyclic Jacobi eigen-decomposition of a symmetric n x n matrix `a`
// (destroyed). On return a[i][i] are the eigenvalues and column j of `phi`
// is the eigenvector for a[j][j]. Each rotation zeroes one off-diagonal
// entry: J = [[c, s], [-s, c]] on (p, q), A <- J^T A J, Phi <- Phi J, with
// t = s/c the smaller root of t^2 + 2 theta t - 1 = 0, theta =
// (a_qq - a_pp) / (2 a_pq). Sweeps stop once the off-diagonal Frobenius norm
// is at most 1e-14 of the whole matrix's.
int jacobi_eigen(int n, std::vector<double>& a, std::vector<double>& phi) {
  phi.assign((size_t)n * n, 0.0);
  for (int i = 0; i < n; ++i) phi[(size_t)i * n + i] = 1.0;
  double fro = 0.0;
  for (size_t i = 0; i < a.size(); ++i) fro += a[i] * a[i];
  fro = std::sqrt(fro);
  if (fro == 0.0) return 0;
  int sweep = 0;
  for (; sweep < 100; ++sweep) {
    double off = 0.0;
    for (int p = 0; p < n; ++p)
      for (int q = 0; q < n; ++q)
        if (p != q) off += a[(size_t)p * n + q] * a[(size_t)p * n + q];
    if (std::sqrt(off) <= 1e-14 * fro) break;
    for (int p = 0; p < n - 1; ++p) {
      for (int q = p + 1; q < n; ++q) {
        const double apq = a[(size_t)p * n + q];
        if (apq == 0.0) continue;
        const double app = a[(size_t)p * n + p];
        const double aqq = a[(size_t)q * n + q];
        const double theta = (aqq - app) / (2.0 * apq);
        const double t = (theta >= 0.0 ? 1.0 : -1.0) /
                         (std::fabs(theta) + std::sqrt(theta * theta + 1.0));
        const double c = 1.0 / std::sqrt(t * t + 1.0);
        const double s = t * c;
        // columns p, q of A <- A J
        for (int k = 0; k < n; ++k) {
          const double akp = a[(size_t)k * n + p];
          const double akq = a[(size_t)k * n + q];
          a[(size_t)k * n + p] = c * akp - s * akq;
          a[(size_t)k * n + q] = s * akp + c * akq;
        }
        // rows p, q of A <- J^T A
        for (int k = 0; k < n; ++k) {
          const double apk = a[(size_t)p * n + k];
          const double aqk = a[(size_t)q * n + k];
          a[(size_t)p * n + k] = c * apk - s * aqk;
          a[(size_t)q * n + k] = s * apk + c * aqk;
        }
        a[(size_t)p * n + q] = 0.0;
        a[(size_t)q * n + p] = 0.0;
        for (int k = 0; k < n; ++k) {
          const double fkp = phi[(size_t)k * n + p];
          const double fkq = phi[(size_t)k * n + q];
          phi[(size_t)k * n + p] = c * fkp - s * fkq;
          phi[(size_t)k * n + q] = s * fkp + c * fkq;
        }
      }
    }
  }
  return sweep;
}

// Summary of one page, [Locks] §3 (centroid and scatter H_j) and §4
// (D_j, V_j = top-r eigenvectors of H_j = top-r right singular vectors of
// D_j, C_j = D_j V_j).
void build_one(int P, int d, int r, const double* k, double* mu, double* vt,
               double* coef, double* evals, int* sweeps) {
  for (int a = 0; a < d; ++a) {
    double s = 0.0;
    for (int i = 0; i < P; ++i) s += k[(size_t)i * d + a];
    mu[a] = s / P;
  }
  std::vector<double> D((size_t)P * d);
  for (int i = 0; i < P; ++i)
    for (int a = 0; a < d; ++a) D[(size_t)i * d + a] = k[(size_t)i * d + a] - mu[a];
  std::vector<double> H((size_t)d * d, 0.0);
  for (int a = 0; a < d; ++a)
    for (int b = 0; b < d; ++b) {
      double s = 0.0;
      for (int i = 0; i < P; ++i) s += D[(size_t)i * d + a] * D[(size_t)i * d + b];
      H[(size_t)a * d + b] = s;
    }
  std::vector<double> phi;
  const int sw = jacobi_eigen(d, H, phi);
  if (sweeps) *sweeps = sw;
  std::vector<int> order(d);
  for (int j = 0; j < d; ++j) order[j] = j;
  std::stable_sort(order.begin(), order.end(), [&](int x, int y) {
    return H[(size_t)x * d + x] > H[(size_t)y * d + y];
  });
  if (evals)
    for (int j = 0; j < d; ++j) evals[j] = H[(size_t)order[j] * d + order[j]];
  for (int rho = 0; rho < r; ++rho) {
    const int col = order[rho];
    int arg = 0;
    double best = -1.0;
    for (int a = 0; a < d; ++a) {
      const double m = std::fabs(phi[(size_t)a * d + col]);
      if (m > best) { best = m; arg = a; }
    }
    const double sgn = phi[(size_t)arg * d + col] < 0.0 ? -1.0 : 1.0;
    for (int a = 0; a < d; ++a) vt[(size_t)rho * d + a] = sgn * phi[(size_t)a * d + col];
  }
  for (int i = 0; i < P; ++i)
    for (int rho = 0; rho < r; ++rho) {
      double s = 0.0;
      for (int a = 0; a < d; ++a) s += D[(size_t)i * d + a] * vt[(size_t)rho * d + a];
      coef[(size_t)i * r + rho] = s;
    }
}

double log_sum_exp(const double* x, int n) {
  double m = -INFINITY;
  for (int i = 0; i < n; ++i) m = std::max(m, x[i]);
  if (m == -INFINITY) return -INFINITY;
  double s = 0.0;
  for (int i = 0; i < n; ++i) s += std::exp(x[i] - m);
  return m + std::log(s);
}

}  // namespace

extern "C" {

int lo_version(void) { return 1; }

// Fit (mu, V, C) for each of n_pages pages, [Locks] §3-§4. evals (may be
// NULL) receives all d eigenvalues of H_j in descending order, sweeps (may be
// NULL) the Jacobi sweep count. Pages are independent and are split over
// n_threads plain threads.
int lo_build_pages(int n_pages, int P, int d, int r, const double* keys,
                   double* mu, double* vt, double* coef, double* evals,
                   int* sweeps, int n_threads) {
  if (n_pages < 0 || P < 1 || d < 1 || r < 1 || r > d || !keys || !mu || !vt || !coef)
    return -1;
  if (n_threads < 1) n_threads = 1;
  auto work = [&](int t) {
    for (int j = t; j < n_pages; j += n_threads)
      build_one(P, d, r, keys + (size_t)j * P * d, mu + (size_t)j * d,
                vt + (size_t)j * r * d, coef + (size_t)j * P * r,
                evals ? evals + (size_t)j * d : nullptr, sweeps ? sweeps + j : nullptr);
  };
  std::vector<std::thread> pool;
  for (int t = 1; t < n_threads; ++t) pool.emplace_back(work, t);
  work(0);
  for (auto& th : pool) th.join();
  return 0;
}

// Round-to-nearest-even onto the bfloat16 grid (8 significant bits, fp32
// exponent range), computed from the binary64 value directly. Values beyond
// the largest finite bf16 go to +-inf; subnormal bf16 results are kept.
void lo_round_bf16(const double* x, long n, double* y) {
  for (long i = 0; i < n; ++i) {
    const double v = x[i];
    if (!std::isfinite(v) || v == 0.0) { y[i] = v; continue; }
    int e;
    std::frexp(std::fabs(v), &e);  // |v| = m * 2^e, m in [0.5, 1)
    // bf16 spacing at this binade is 2^(e-8); below the normal range the
    // spacing stays at the subnormal step 2^-133.
    int ex = e - 8;
    if (ex < -133) ex = -133;
    const double step = std::ldexp(1.0, ex);
    const double qv = std::nearbyint(v / step) * step;  // ties-to-even (default mode)
    const double maxbf = std::ldexp(255.0, 120);        // (2 - 2^-7) * 2^127
    y[i] = std::fabs(qv) > maxbf ? std::copysign(INFINITY, v) : qv;
  }
}

// Reconstructed page log-sum-exp, [Locks] §4 Eq. (2):
//   shat_j(q) = q.mu_j * scale + log sum_i exp(((V_j^T q) . c_i) * scale)
// out[g][j] for each of the G heads and n_pages pages.
int lo_page_scores(int G, int d, int r, int P, int n_pages, const double* q,
                   const double* mu, const double* vt, const double* coef,
                   double scale, double* out) {
  if (G < 1 || d < 1 || r < 1 || P < 1 || n_pages < 0) return -1;
  std::vector<double> w(r), z(P);
  for (int g = 0; g < G; ++g) {
    const double* qg = q + (size_t)g * d;
    for (int j = 0; j < n_pages; ++j) {
      const double* m = mu + (size_t)j * d;
      const double* v = vt + (size_t)j * r * d;
      const double* c = coef + (size_t)j * P * r;
      double qm = 0.0;
      for (int a = 0; a < d; ++a) qm += qg[a] * m[a];
      for (int rho = 0; rho < r; ++rho) {
        double s = 0.0;
        for (int a = 0; a < d; ++a) s += v[(size_t)rho * d + a] * qg[a];
        w[rho] = s;
      }
      for (int i = 0; i < P; ++i) {
        double s = 0.0;
        for (int rho = 0; rho < r; ++rho) s += w[rho] * c[(size_t)i * r + rho];
        z[i] = s * scale;
      }
      out[(size_t)g * n_pages + j] = qm * scale + log_sum_exp(z.data(), P);
    }
  }
  return 0;
}

// Exact page log-sum-exp, [Locks] §2 Eq. (1): s_j(q) = log sum_{i in P_j}
// exp(q.k_i * scale). n_valid[j] (NULL = all P) limits page j to its first
// tokens, for a partial last page.
int lo_exact_page_lse(int G, int d, int P, int n_pages, const int* n_valid,
                      const double* q, const double* keys, double scale, double* out) {
  if (G < 1 || d < 1 || P < 1 || n_pages < 0) return -1;
  std::vector<double> z(P);
  for (int g = 0; g < G; ++g) {
    const double* qg = q + (size_t)g * d;
    for (int j = 0; j < n_pages; ++j) {
      const int nv = n_valid ? n_valid[j] : P;
      const double* k = keys + (size_t)j * P * d;
      for (int i = 0; i < nv; ++i) {
        double s = 0.0;
        for (int a = 0; a < d; ++a) s += qg[a] * k[(size_t)i * d + a];
        z[i] = s * scale;
      }
      out[(size_t)g * n_pages + j] = log_sum_exp(z.data(), nv);
    }
  }
  return 0;
}

// Share-average combine, [Locks] §4: per head the page shares
// m_g(j) = exp(s_j,g) / sum_j' exp(s_j',g); the group score is
// mbar_j = (1/G) sum_g m_g(j). Written in the log domain:
//   logz[g]  = log sum_j exp(s[g][j])
//   sigma[j] = log mbar_j = log sum_g exp(s[g][j] - logz[g]) - log G
// s is [G][n] over the n summarised (complete) pages.
int lo_combine(int G, int n, const double* s, double* logz, double* sigma) {
  if (G < 1 || n < 0) return -1;
  std::vector<double> t(G);
  for (int g = 0; g < G; ++g) logz[g] = log_sum_exp(s + (size_t)g * n, n);
  for (int j = 0; j < n; ++j) {
    for (int g = 0; g < G; ++g) t[g] = s[(size_t)g * n + j] - logz[g];
    sigma[j] = log_sum_exp(t.data(), G) - std::log((double)G);
  }
  return 0;
}

// Page selection, [Locks] §2 and §4: with J pages in the sequence and k page
// slots, J <= k keeps every page. Otherwise the sink page 0 and the most
// recent page J-1 are always kept and the other k-2 slots go to the
// highest-scoring remaining complete pages. sigma[n_complete] holds the
// ranking key of each complete page; ties go to the lower page id.
// sel[k] receives the chosen logical page ids in ascending order, padded
// with -1. Returns the number chosen, or -1 on bad arguments.
int lo_select(int n_complete, int J, int k, const double* sigma, int* sel) {
  if (k < 2 || J < 0 || n_complete < 0 || n_complete > J || J - n_complete > 1) return -1;
  for (int i = 0; i < k; ++i) sel[i] = -1;
  if (J <= k) {
    for (int j = 0; j < J; ++j) sel[j] = j;
    return J;
  }
  std::vector<int> cand;
  for (int j = 1; j < n_complete; ++j)
    if (j != J - 1) cand.push_back(j);
  std::stable_sort(cand.begin(), cand.end(), [&](int x, int y) {
    if (sigma[x] != sigma[y]) return sigma[x] > sigma[y];
    return x < y;
  });
  const int take = std::min<int>(k - 2, (int)cand.size());
  std::vector<int> S = {0, J - 1};
  for (int i = 0; i < take; ++i) S.push_back(cand[i]);
  std::sort(S.begin(), S.end());
  for (size_t i = 0; i < S.size(); ++i) sel[i] = S[i];
  return (int)S.size();
}

// Attention restricted to a token set, [Locks] §2: with the softmax
// renormalised over the n_tok given tokens,
//   alpha_i = exp(q.k_i * scale) / sum_i' exp(q.k_i' * scale)
//   o = sum_i alpha_i v_i,   lse = log sum_i exp(q.k_i * scale)
// keys/vals [n_tok][d], out [G][d], lse [G]. With every token given this is
// dense decode attention.
int lo_attend(int G, int d, int n_tok, const double* q, const double* keys,
              const double* vals, double scale, double* out, double* lse) {
  if (G < 1 || d < 1 || n_tok < 0) return -1;
  std::vector<double> z(n_tok);
  for (int g = 0; g < G; ++g) {
    const double* qg = q + (size_t)g * d;
    for (int i = 0; i < n_tok; ++i) {
      double s = 0.0;
      for (int a = 0; a < d; ++a) s += qg[a] * keys[(size_t)i * d + a];
      z[i] = s * scale;
    }
    const double l = log_sum_exp(z.data(), n_tok);
    if (lse) lse[g] = l;
    for (int a = 0; a < d; ++a) out[(size_t)g * d + a] = 0.0;
    for (int i = 0; i < n_tok; ++i) {
      const double alpha = std::exp(z[i] - l);
      for (int a = 0; a < d; ++a) out[(size_t)g * d + a] += alpha * vals[(size_t)i * d + a];
    }
  }
  return 0;
}


// Quantized summary storage, [Locks] §4 (the "i4" variants) and App. C.7:
// the basis V_j in 4-bit integers, the centroid mu_j and the coefficients
// C_j in 8-bit integers, with bfloat16 scales. The pages give the widths and
// the byte count only (d*r/2 + B*r + d bytes before scales; 818 / 490 / 326
// bytes with scales at B = 16, d = 128, r = 8 / 4 / 2). Reading taken here:
//   * symmetric codes, one scale per group, the groups being each basis
//     vector (d entries), each token's coefficient row (r entries) and the
//     centroid (d entries): r + B + 1 scales, the count that reproduces the
//     printed totals;
//   * scale = bf16(max|x| / L) with L = 7 (4-bit) or 127 (8-bit), code =
//     round-half-even(x / scale), clamped to [-L, L]; a group of zeros has
//     scale 0 and codes 0;
//   * every step in double precision like the rest of this file: the maximum,
//     the division by L (then one rounding to bf16) and the division by the
//     scale. For values held in fp32 or below, the double quotient x / scale
//     sits on a half-integer only when the exact quotient does, so the
//     round-half-even decision is the exact one.
// The three parts are quantized independently from the full-precision fit.
static void quantize_group(const double* x, long n, long stride, int L, int* code, long cstride,
                           double* scale) {
  double amax = 0.0;
  for (long i = 0; i < n; ++i) amax = std::max(amax, std::fabs(x[i * stride]));
  const double s64 = amax / (double)L;
  double sb = 0.0;
  lo_round_bf16(&s64, 1, &sb);
  *scale = sb;
  for (long i = 0; i < n; ++i) {
    int c = 0;
    if (sb > 0.0) {
      c = (int)std::nearbyint(x[i * stride] / sb);  // ties to even in the default rounding mode
      c = std::min(L, std::max(-L, c));
    }
    code[i * cstride] = c;
  }
}

// n_pages summaries (mu [n][d], vt [n][r][d], coef [n][P][r], full precision)
// -> signed codes of the same shapes and scales mu_scale [n], vt_scale [n][r]
// (one per basis vector), coef_scale [n][P] (one per token).
int lo_quantize_summaries(int n_pages, int d, int P, int r, const double* mu, const double* vt,
                          const double* coef, int* mu_code, int* vt_code, int* coef_code,
                          double* mu_scale, double* vt_scale, double* coef_scale) {
  if (n_pages < 0 || d < 1 || P < 1 || r < 1) return -1;
  for (int j = 0; j < n_pages; ++j) {
    quantize_group(mu + (size_t)j * d, d, 1, 127, mu_code + (size_t)j * d, 1, mu_scale + j);
    for (int rho = 0; rho < r; ++rho) {
      const size_t o = ((size_t)j * r + rho) * d;
      quantize_group(vt + o, d, 1, 7, vt_code + o, 1, vt_scale + (size_t)j * r + rho);
    }
    for (int i = 0; i < P; ++i) {
      const size_t o = ((size_t)j * P + i) * r;
      quantize_group(coef + o, r, 1, 127, coef_code + o, 1, coef_scale + (size_t)j * P + i);
    }
  }
  return 0;
}

}  // extern "C"
