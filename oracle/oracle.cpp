// Reference oracle for the verify-and-resample step of speculative sampling.
//
// TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, single-threaded,
// double-precision statement of what the step computes.  Only the test suite,
// the smoke check and the CPU-baseline leg of the benchmark may load it.  It
// shares no code, header, table or helper with the GPU library, and it never
// includes anything from the package directory.
//
// Sources it follows (the pages of the method; no GPU design is taken from
// them):
//   * "Accelerating Large Language Model Decoding with Speculative Sampling"
//     (FDE Interviews breakdown, section 01 "The paper in one minute" and its
//     figure "The idea, visually"): keep draft token d_t with probability
//     min(1, q(d_t)/p(d_t)), q = target, p = draft; at the first rejection draw
//     a replacement from the normalised positive part of q - p and discard the
//     rest; if all K survive, the target's last logit set yields one more
//     token; temperature, top-k, nucleus and greedy are all covered.
//   * paperlayer.ai summary of arXiv 2302.01318, sections "Auto-regressive
//     Sampling" (K+1 target-logit sets) and "Modified Rejection Sampling"
//     (sampling controls are applied before the rejection step; at least one
//     token per loop, one extra when the draft is fully accepted).
//   * roadtointelligence.com "Speculative Decoding", section "Draft, then
//     verify" (same rule with the letters swapped: there p = target).
//
// Readings where the pages are silent (each is also listed in the design
// notes of the repository):
//   R1  letters: q = target, p = draft.
//   R2  accept test is u * p(d) < q(d) with u on a 24-bit grid in [0, 1).
//   R3  temperature first, then one filter per row, applied to the target and
//       the draft independently.
//   R4  top-k keeps every token whose raw logit is >= the k-th largest raw
//       logit (ties at the boundary are all kept).
//   R5  nucleus: tokens are grouped by equal logit value and visited in
//       descending order; a group is kept iff the mass of the groups before
//       it is < top_p.  The first group is always kept; top_p >= 1 keeps
//       every token with non-zero probability (plain sampling).
//   R6  greedy: one-hot at the lowest index among the maximal raw logits;
//       temperature is ignored.
//   R7  inverse-CDF draws walk the vocabulary in index order.
//   R8  a residual with zero mass (rounding only) falls back to q_n and sets
//       status bit 3.
//   R9  p(d) = 0: the test u*0 < q(d) accepts iff q(d) > 0; status bit 4.
//   R10 K_b = 0 is allowed: the step is then one draw from the filtered q_0.
//   R11 target position t scores draft slot t; position K_b is the bonus;
//       ragged rows use the padded K_max stride.
//   R12 random numbers: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11,
//       "Parallel Random Numbers: As Easy as 1, 2, 3"), key = seed,
//       counter = (g lo, t, purpose, g hi), u = (word0 >> 8) * 2^-24.
//   R13 logits that are NaN or +inf in a used row, a draft token outside
//       [0, V), an all -inf row or an invalid per-row parameter make the row
//       an error row: accepted = -1 and every emitted token is -1.
//
// A decision is "near its boundary" (flag bits, oracle only) when a uniform
// or a nucleus cumulative mass lies within 1e-6 of the value it is compared
// with; those rows are the only ones where an fp32 implementation may
// legitimately disagree.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <numeric>
#include <vector>

#include "oracle.h"

namespace {

// ---------------------------------------------------------------- Philox ---
// Philox4x32 with 10 rounds, written from the published description: each
// round multiplies counter words 0 and 2 by two fixed odd constants, takes
// the 64-bit products apart into high and low halves, and recombines them
// with the other two counter words and the round key by xor; the key is
// advanced between rounds by two Weyl constants.
const uint32_t kMulA = 0xD2511F53u;
const uint32_t kMulB = 0xCD9E8D57u;
const uint32_t kWeylA = 0x9E3779B9u;
const uint32_t kWeylB = 0xBB67AE85u;

void philox_round(uint32_t c[4], const uint32_t k[2]) {
  uint64_t pa = (uint64_t)kMulA * (uint64_t)c[0];
  uint64_t pb = (uint64_t)kMulB * (uint64_t)c[2];
  uint32_t a_hi = (uint32_t)(pa >> 32), a_lo = (uint32_t)pa;
  uint32_t b_hi = (uint32_t)(pb >> 32), b_lo = (uint32_t)pb;
  uint32_t n0 = b_hi ^ c[1] ^ k[0];
  uint32_t n1 = b_lo;
  uint32_t n2 = a_hi ^ c[3] ^ k[1];
  uint32_t n3 = a_lo;
  c[0] = n0; c[1] = n1; c[2] = n2; c[3] = n3;
}

void philox10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  uint32_t c[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
  uint32_t k[2] = {key[0], key[1]};
  for (int r = 0; r < 10; ++r) {
    if (r > 0) { k[0] += kWeylA; k[1] += kWeylB; }
    philox_round(c, k);
  }
  for (int i = 0; i < 4; ++i) out[i] = c[i];
}

uint32_t draw_word(uint64_t seed, uint64_t g, uint32_t t, uint32_t purpose) {
  uint32_t ctr[4] = {(uint32_t)g, t, purpose, (uint32_t)(g >> 32)};
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t out[4];
  philox10(ctr, key, out);
  return out[0];
}

double draw_uniform(uint64_t seed, uint64_t g, uint32_t t, uint32_t purpose) {
  return (double)(draw_word(seed, g, t, purpose) >> 8) * (1.0 / 16777216.0);
}

// ------------------------------------------------------------- decoding ---
double decode(const void* base, int dtype, size_t i) {
  if (dtype == ORACLE_BF16) {
    uint16_t h = static_cast<const uint16_t*>(base)[i];
    uint32_t bits = (uint32_t)h << 16;
    float f;
    std::memcpy(&f, &bits, 4);
    return (double)f;
  }
  return (double)static_cast<const float*>(base)[i];
}

const double kInf = std::numeric_limits<double>::infinity();

// ------------------------------------------------------------ transform ---
// Turns one row of raw logits into the "adjusted distribution" the step
// samples from (temperature and a filter applied before the rejection step).
// Returns the status bits of the row (bit 1: NaN or +inf, bit 2: every logit
// is -inf).  *margin receives the distance of the nucleus cut from top_p
// (infinity when the mode has no floating-point cut).
struct RowResult {
  std::vector<double> pi;
  uint32_t status = 0;
  double topp_margin = kInf;
  int n_keep = 0;
};

RowResult transform_row(const std::vector<double>& x, int mode, double tau,
                        int top_k, double top_p) {
  RowResult r;
  const int V = (int)x.size();
  r.pi.assign(V, 0.0);
  bool any_not_neg_inf = false;
  for (int v = 0; v < V; ++v) {
    if (std::isnan(x[v]) || x[v] == kInf) r.status |= ORACLE_ST_NONFINITE;
    if (x[v] != -kInf) any_not_neg_inf = true;
  }
  if (r.status) return r;
  if (!any_not_neg_inf) { r.status |= ORACLE_ST_EMPTY; return r; }

  double M = -kInf;
  for (int v = 0; v < V; ++v) M = std::max(M, x[v]);

  if (mode == ORACLE_GREEDY) {
    int gidx = 0;
    while (x[gidx] != M) ++gidx;  // lowest index among the maxima
    r.pi[gidx] = 1.0;
    r.n_keep = 1;
    return r;
  }
  if (mode == ORACLE_TOPP && top_p >= 1.0) mode = ORACLE_PLAIN;

  // e_v = exp((x_v - M) / tau): the softmax numerator after temperature.
  std::vector<double> e(V);
  for (int v = 0; v < V; ++v) e[v] = std::exp((x[v] - M) / tau);

  std::vector<char> keep(V, 0);
  if (mode == ORACLE_PLAIN) {
    for (int v = 0; v < V; ++v) keep[v] = (x[v] != -kInf);
  } else if (mode == ORACLE_TOPK) {
    std::vector<double> sorted(x);
    std::sort(sorted.begin(), sorted.end(), std::greater<double>());
    double kth = sorted[top_k - 1];  // counted with multiplicity
    for (int v = 0; v < V; ++v) keep[v] = (x[v] >= kth);
  } else {  // ORACLE_TOPP
    double Z = 0.0;
    for (int v = 0; v < V; ++v) Z += e[v];
    std::vector<int> order(V);
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(),
                     [&](int a, int b) { return x[a] > x[b]; });
    double before = 0.0;  // mass of all groups visited so far
    double margin = kInf;
    int i = 0;
    while (i < V) {
      int j = i;
      double group_mass = 0.0;
      while (j < V && x[order[j]] == x[order[i]]) {
        group_mass += e[order[j]] / Z;
        ++j;
      }
      margin = std::min(margin, std::fabs(before - top_p));
      bool kept = (i == 0) || (before < top_p);
      if (kept)
        for (int m = i; m < j; ++m) keep[order[m]] = 1;
      before += group_mass;
      i = j;
    }
    r.topp_margin = margin;
  }
  double Zs = 0.0;
  for (int v = 0; v < V; ++v)
    if (keep[v]) { Zs += e[v]; ++r.n_keep; }
  for (int v = 0; v < V; ++v) r.pi[v] = keep[v] ? e[v] / Zs : 0.0;
  return r;
}

// Inverse CDF in vocabulary order: the smallest v with C_v > u * S, where
// C_v is the running sum of w.  Falls back to the last v with w_v > 0 when
// rounding leaves none.  *lo / *hi receive C_{y-1}/S and C_y/S for the
// boundary check; *interior_lo / *interior_hi say whether those boundaries
// are computed values (a non-zero weight lies on the other side).
int inverse_cdf(const std::vector<double>& w, double S, double u, double* lo,
                double* hi, bool* interior_lo, bool* interior_hi) {
  const int V = (int)w.size();
  double target = u * S;
  double c = 0.0;
  int y = -1;
  double c_before = 0.0;
  for (int v = 0; v < V; ++v) {
    double c_next = c + w[v];
    if (c_next > target && w[v] > 0.0) {
      y = v;
      c_before = c;
      c = c_next;
      break;
    }
    c = c_next;
  }
  if (y < 0) {
    for (int v = V - 1; v >= 0; --v)
      if (w[v] > 0.0) { y = v; break; }
    c = S;
    c_before = S - w[y];
  }
  *lo = c_before / S;
  *hi = c / S;
  bool any_before = false, any_after = false;
  for (int v = 0; v < y; ++v) any_before |= (w[v] > 0.0);
  for (int v = y + 1; v < V; ++v) any_after |= (w[v] > 0.0);
  *interior_lo = any_before;
  *interior_hi = any_after;
  return y;
}

struct RowParams {
  int Kb, mode, top_k;
  double tau, top_p;
  bool valid;
};

RowParams read_params(const OracleArgs* a, int b) {
  RowParams p;
  p.Kb = a->k_per_row ? a->k_per_row[b] : a->K_max;
  p.mode = a->mode ? (int)a->mode[b] : a->default_mode;
  p.tau = a->temperature ? (double)a->temperature[b] : (double)a->default_temperature;
  p.top_k = a->top_k ? a->top_k[b] : a->default_top_k;
  p.top_p = a->top_p ? (double)a->top_p[b] : (double)a->default_top_p;
  bool ok = p.Kb >= 0 && p.Kb <= a->K_max && p.mode >= 0 && p.mode <= 3;
  if (ok && p.mode != ORACLE_GREEDY) ok = std::isfinite(p.tau) && p.tau > 0.0;
  if (ok && p.mode == ORACLE_TOPK) ok = p.top_k >= 1 && p.top_k <= a->V;
  if (ok && p.mode == ORACLE_TOPP) ok = p.top_p > 0.0 && p.top_p <= 1.0;
  p.valid = ok;
  return p;
}

const double kWindow = 1e-6;

}  // namespace

extern "C" {

void oracle_philox4x32_10(const uint32_t* ctr, const uint32_t* key, uint32_t* out) {
  philox10(ctr, key, out);
}

void oracle_philox_words(uint64_t seed, uint64_t n, const uint64_t* g,
                         const uint32_t* t, const uint32_t* purpose,
                         uint32_t* out_words) {
  for (uint64_t i = 0; i < n; ++i) out_words[i] = draw_word(seed, g[i], t[i], purpose[i]);
}

double oracle_uniform(uint64_t seed, uint64_t g, uint32_t t, uint32_t purpose) {
  return draw_uniform(seed, g, t, purpose);
}

uint32_t oracle_row_probs(const void* logits, int dtype, int V, int mode,
                          float tau, int top_k, float top_p, double* pi_out,
                          double* topp_margin, int* n_keep) {
  std::vector<double> x(V);
  for (int v = 0; v < V; ++v) x[v] = decode(logits, dtype, v);
  RowResult r = transform_row(x, mode, (double)tau, top_k, (double)top_p);
  if (pi_out) for (int v = 0; v < V; ++v) pi_out[v] = r.pi[v];
  if (topp_margin) *topp_margin = r.topp_margin;
  if (n_keep) *n_keep = r.n_keep;
  return r.status;
}

int oracle_verify(const OracleArgs* a) {
  if (!a || a->B < 0 || a->K_max < 0 || a->V <= 0) return -1;
  const int B = a->B, KM = a->K_max, V = a->V;
  const size_t Vs = (size_t)V;
  for (int b = 0; b < B; ++b) {
    const uint64_t g = a->row_offset + (uint64_t)b;
    RowParams prm = read_params(a, b);
    uint32_t status = 0, flags = 0;
    int32_t* toks = a->out_tokens + (size_t)b * (KM + 1);
    for (int i = 0; i <= KM; ++i) toks[i] = -1;
    if (a->diag)
      for (int i = 0; i < 2 * KM; ++i) a->diag[(size_t)b * 2 * KM + i] = std::nan("");
    if (a->resid_mass) a->resid_mass[b] = std::nan("");

    if (!prm.valid) {
      a->accepted[b] = -1;
      a->row_status[b] = ORACLE_ST_PARAM;
      if (a->flags) a->flags[b] = 0;
      continue;
    }
    const int Kb = prm.Kb;
    const int32_t* d = a->draft_tokens + (size_t)b * KM;
    for (int t = 0; t < Kb; ++t)
      if (d[t] < 0 || d[t] >= V) status |= ORACLE_ST_TOKEN;

    // Target rows t = 0..Kb and draft rows t = 0..Kb-1 of sequence b.
    std::vector<RowResult> tq(Kb + 1), dp(Kb);
    for (int t = 0; t <= Kb; ++t) {
      std::vector<double> x(V);
      size_t base = ((size_t)b * (KM + 1) + t) * Vs;
      for (int v = 0; v < V; ++v) x[v] = decode(a->target_logits, a->dtype, base + v);
      tq[t] = transform_row(x, prm.mode, prm.tau, prm.top_k, prm.top_p);
      status |= tq[t].status;
    }
    for (int t = 0; t < Kb; ++t) {
      std::vector<double> x(V);
      size_t base = ((size_t)b * KM + t) * Vs;
      for (int v = 0; v < V; ++v) x[v] = decode(a->draft_logits, a->dtype, base + v);
      dp[t] = transform_row(x, prm.mode, prm.tau, prm.top_k, prm.top_p);
      status |= dp[t].status;
    }
    if (status & ORACLE_ST_ERRORS) {
      a->accepted[b] = -1;
      a->row_status[b] = status;
      if (a->flags) a->flags[b] = 0;
      continue;
    }
    for (int t = 0; t <= Kb; ++t)
      if (tq[t].topp_margin < kWindow) flags |= ORACLE_FL_TOPP;
    for (int t = 0; t < Kb; ++t)
      if (dp[t].topp_margin < kWindow) flags |= ORACLE_FL_TOPP;

    // Accept loop: left to right, stop at the first rejection.
    int n = Kb;
    for (int t = 0; t < Kb; ++t) {
      double q = tq[t].pi[d[t]], p = dp[t].pi[d[t]];
      if (a->diag) {
        a->diag[((size_t)b * KM + t) * 2 + 0] = q;
        a->diag[((size_t)b * KM + t) * 2 + 1] = p;
      }
      double u = draw_uniform(a->seed, g, (uint32_t)t, ORACLE_PURPOSE_ACCEPT);
      if (p == 0.0) status |= ORACLE_ST_PZERO;
      bool accept = u * p < q;
      if (p > 0.0) {
        double ratio = q / p;
        if (ratio < 1.0 + kWindow && std::fabs(u - ratio) < kWindow) flags |= ORACLE_FL_ACCEPT;
      }
      if (!accept) { n = t; break; }
    }
    // Diagnostics of positions after the stop are still reported.
    if (a->diag)
      for (int t = n + 1; t < Kb; ++t) {
        a->diag[((size_t)b * KM + t) * 2 + 0] = tq[t].pi[d[t]];
        a->diag[((size_t)b * KM + t) * 2 + 1] = dp[t].pi[d[t]];
      }

    // Resample from normalize((q_n - p_n)+) or draw the bonus from q_Kb.
    std::vector<double> w(V);
    double u;
    if (n < Kb) {
      for (int v = 0; v < V; ++v) w[v] = std::max(0.0, tq[n].pi[v] - dp[n].pi[v]);
      u = draw_uniform(a->seed, g, (uint32_t)n, ORACLE_PURPOSE_RESAMPLE);
    } else {
      for (int v = 0; v < V; ++v) w[v] = tq[Kb].pi[v];
      u = draw_uniform(a->seed, g, (uint32_t)Kb, ORACLE_PURPOSE_BONUS);
    }
    double S = 0.0;
    for (int v = 0; v < V; ++v) S += w[v];
    if (!(S > 0.0)) {
      for (int v = 0; v < V; ++v) w[v] = tq[n].pi[v];
      S = 0.0;
      for (int v = 0; v < V; ++v) S += w[v];
      status |= ORACLE_ST_ZERO_RESIDUAL;
    }
    if (a->resid_mass) a->resid_mass[b] = S;
    double lo, hi;
    bool ilo, ihi;
    int y = inverse_cdf(w, S, u, &lo, &hi, &ilo, &ihi);
    if ((ilo && u - lo < kWindow) || (ihi && hi - u < kWindow)) flags |= ORACLE_FL_CDF;

    for (int t = 0; t < n; ++t) toks[t] = d[t];
    toks[n] = y;
    a->accepted[b] = n;
    a->row_status[b] = status;
    if (a->flags) a->flags[b] = flags;
  }
  return 0;
}

}  // extern "C"
