// Host producers of libsfa: rung bases, scaled offsets, per-layer schedules,
// Christoffel offsets, power-law edge lists and the rotary table.  Pure,
// synchronous, deterministic; no HIP calls.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <numeric>
#include <vector>

#include "sfa_internal.h"

namespace sfa {

static thread_local char g_err[512];

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

void clear_error() { g_err[0] = 0; }

}  // namespace sfa

using sfa::fail;

extern "C" const char* sfa_last_error(void) { return sfa::g_err; }

extern "C" int sfa_version(void) { return 1; }

// Fibonacci rungs of "Depth-Staggered Fibonacci Spacing for Sparse
// Attention", fib equation: f_1 = 1, f_2 = 2, f_{k+2} = f_{k+1} + f_k, K = 15.
extern "C" int sfa_base_fib(int32_t* base, int cap) {
  if (!base) return fail(SFA_ERR_ARG, "sfa_base_fib: base is NULL");
  if (cap < 15) return fail(SFA_ERR_CAPACITY, "sfa_base_fib: need 15 entries");
  int32_t a = 1, b = 2;
  for (int k = 0; k < 15; ++k) {
    base[k] = a;
    int32_t c = a + b;
    a = b;
    b = c;
  }
  return 15;
}

// Same page, power-of-2 control: 2^0 .. 2^10 (reach 1024 ~ 987).
extern "C" int sfa_base_pow2(int32_t* base, int cap) {
  if (!base) return fail(SFA_ERR_ARG, "sfa_base_pow2: base is NULL");
  if (cap < 11) return fail(SFA_ERR_CAPACITY, "sfa_base_pow2: need 11 entries");
  for (int k = 0; k < 11; ++k) base[k] = int32_t(1) << k;
  return 11;
}

// Same page, gather paragraph: d = alpha * f, rows floor(d) and floor(d)+1.
extern "C" int sfa_offsets_scaled(const int32_t* base, int k_count,
                                  double alpha, int32_t* lo, float* frac) {
  if (k_count < 0) return fail(SFA_ERR_ARG, "sfa_offsets_scaled: k_count < 0");
  if (k_count > 0 && (!base || !lo || !frac))
    return fail(SFA_ERR_ARG, "sfa_offsets_scaled: NULL buffer");
  if (!std::isfinite(alpha) || !(alpha > 0.0))
    return fail(SFA_ERR_ARG, "sfa_offsets_scaled: alpha must be finite and > 0");
  for (int k = 0; k < k_count; ++k) {
    if (base[k] < 0) return fail(SFA_ERR_ARG, "sfa_offsets_scaled: base[%d] < 0", k);
    const double d = alpha * double(base[k]);
    if (!(d < 1073741824.0))
      return fail(SFA_ERR_ARG, "sfa_offsets_scaled: distance %d too large", k);
  }
  for (int k = 0; k < k_count; ++k) {
    const double d = alpha * double(base[k]);  // one rounding
    const double fl = std::floor(d);
    lo[k] = int32_t(fl);
    frac[k] = float(d - fl);                   // exact difference, then float
  }
  return k_count;
}

extern "C" int sfa_offsets_fib(double alpha, int32_t* lo, float* frac, int cap) {
  if (cap < 15) return fail(SFA_ERR_CAPACITY, "sfa_offsets_fib: need 15 entries");
  int32_t base[15];
  sfa_base_fib(base, 15);
  return sfa_offsets_scaled(base, 15, alpha, lo, frac);
}

extern "C" int sfa_offsets_pow2(double alpha, int32_t* lo, float* frac, int cap) {
  if (cap < 11) return fail(SFA_ERR_CAPACITY, "sfa_offsets_pow2: need 11 entries");
  int32_t base[11];
  sfa_base_pow2(base, 11);
  return sfa_offsets_scaled(base, 11, alpha, lo, frac);
}

// Same page, schedule list.  The ramp value 0.5 + s/(L-1) is one correctly
// rounded division of small integers, (2s + L - 1) / (2(L - 1)), so every
// floor of alpha * f matches the exact rational.
extern "C" int sfa_stagger_alpha(int schedule, int layer, int L, int S,
                                 double* alpha) {
  if (!alpha) return fail(SFA_ERR_ARG, "sfa_stagger_alpha: alpha is NULL");
  if (L < 2 || layer < 0 || layer >= L)
    return fail(SFA_ERR_ARG, "sfa_stagger_alpha: need L >= 2 and 0 <= layer < L");
  int s;
  switch (schedule) {
    case SFA_SCHEDULE_FIXED:
      *alpha = 1.0;
      return SFA_OK;
    case SFA_SCHEDULE_LINEAR:
      s = layer;
      break;
    case SFA_SCHEDULE_COPRIME:
      if (S <= 0 || std::gcd(S, L) != 1)
        return fail(SFA_ERR_ARG, "sfa_stagger_alpha: stride must be coprime with L");
      s = int((int64_t(S) * layer) % L);
      break;
    default:
      return fail(SFA_ERR_ARG, "sfa_stagger_alpha: unknown schedule %d", schedule);
  }
  *alpha = double(2 * s + L - 1) / double(2 * (L - 1));
  return SFA_OK;
}

// Same page, alpha parameterisation.
extern "C" int sfa_alpha_of_theta(double theta, double* alpha, double* dadt) {
  if (!std::isfinite(theta)) return fail(SFA_ERR_ARG, "sfa_alpha_of_theta: theta not finite");
  const double a = 0.5 + 1.0 / (1.0 + std::exp(-theta));
  if (alpha) *alpha = a;
  if (dadt) *dadt = (a - 0.5) * (1.5 - a);
  return SFA_OK;
}

// "Christoffel-Balanced Sparse Attention", construction: the carry word in
// exact integer arithmetic, then the positions of its ones.
extern "C" int sfa_offsets_christoffel(int m, int k, int32_t* offsets, int cap) {
  if (k < 1 || k > (1 << 24) || m < 0 || m > k)
    return fail(SFA_ERR_ARG, "sfa_offsets_christoffel: need 1 <= k <= 2^24, 0 <= m <= k");
  if (m > 0 && !offsets) return fail(SFA_ERR_ARG, "sfa_offsets_christoffel: offsets is NULL");
  if (cap < m) return fail(SFA_ERR_CAPACITY, "sfa_offsets_christoffel: need %d entries", m);
  int w = 0;
  int64_t prev = 0;  // floor(j m / k)
  for (int64_t j = 0; j < k; ++j) {
    const int64_t next = ((j + 1) * int64_t(m)) / k;
    if (next - prev == 1) offsets[w++] = int32_t(j);
    prev = next;
  }
  return w;
}

// Bidirectional form by signed offsets ("Christoffel-Balanced Sparse
// Attention", integration paragraph): -O then +O, ascending.
extern "C" int sfa_offsets_christoffel_signed(int m, int k, int32_t* offsets, int cap) {
  if (k < 1 || k > (1 << 24) || m < 0 || m > k)
    return fail(SFA_ERR_ARG, "sfa_offsets_christoffel_signed: need 1 <= k <= 2^24, 0 <= m <= k");
  if (m > 0 && !offsets) return fail(SFA_ERR_ARG, "sfa_offsets_christoffel_signed: offsets is NULL");
  if (cap < 2 * m) return fail(SFA_ERR_CAPACITY, "sfa_offsets_christoffel_signed: need %d entries", 2 * m);
  const int w = sfa_offsets_christoffel(m, k, offsets + m, m);
  if (w < 0) return w;
  for (int t = 0; t < m; ++t) offsets[t] = -offsets[2 * m - 1 - t];
  return 2 * m;
}

// "Critical power-law sparse attention", items 1-2, with SplitMix64 as the
// generator (Steele, Lea and Flood 2014).
namespace {

inline uint64_t splitmix(uint64_t x) {
  uint64_t z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

}  // namespace

extern "C" int sfa_edges_powerlaw(int n, int r, double sigma, int draws,
                                  int width, uint64_t seed, int32_t* edges,
                                  int32_t* count) {
  if (n < 2 || r < 0 || draws < 0 || width < 1 || width > SFA_MAX_EDGE_WIDTH)
    return fail(SFA_ERR_ARG, "sfa_edges_powerlaw: bad n/r/draws/width");
  if (!std::isfinite(sigma) || !(sigma > -1.0))
    return fail(SFA_ERR_ARG, "sfa_edges_powerlaw: sigma must be finite and > -1");
  if (!edges || !count) return fail(SFA_ERR_ARG, "sfa_edges_powerlaw: NULL buffer");
  const int half = n / 2;
  const double expo = -(1.0 + sigma);
  // Weights in increasing d, their sum, then the normalised running sums.
  std::vector<double> cdf(half);
  double z = 0.0;
  for (int d = 1; d <= half; ++d) z += std::pow(double(d), expo);
  double acc = 0.0;
  for (int d = 1; d <= half; ++d) {
    acc += std::pow(double(d), expo);
    cdf[d - 1] = acc / z;
  }
  cdf[half - 1] = 1.0;
  std::vector<int32_t> row;
  row.reserve(size_t(2 * r + 1 + draws));
  int maxc = 0;
  for (int i = 0; i < n; ++i) {
    row.clear();
    for (int j = std::max(0, i - r); j <= std::min(n - 1, i + r); ++j) row.push_back(j);
    const uint64_t key = splitmix(seed ^ splitmix(uint64_t(i)));
    for (int t = 0; t < draws; ++t) {
      const uint64_t a = splitmix(key + 2ull * uint64_t(t));
      const uint64_t b = splitmix(key + 2ull * uint64_t(t) + 1ull);
      const double u = double(a >> 11) * 0x1.0p-53;
      // smallest d with u < cdf[d-1]
      const int d = int(std::upper_bound(cdf.begin(), cdf.end(), u) - cdf.begin()) + 1;
      const int64_t s = (b >> 63) ? -1 : 1;
      int64_t j = (int64_t(i) + s * d) % n;
      if (j < 0) j += n;
      row.push_back(int32_t(j));
    }
    std::sort(row.begin(), row.end());
    row.erase(std::unique(row.begin(), row.end()), row.end());
    if (int(row.size()) > width)
      return fail(SFA_ERR_CAPACITY, "sfa_edges_powerlaw: query %d has %zu keys > width %d",
                  i, row.size(), width);
    int32_t* e = edges + size_t(i) * size_t(width);
    for (int t = 0; t < width; ++t) e[t] = t < int(row.size()) ? row[t] : -1;
    count[i] = int32_t(row.size());
    maxc = std::max(maxc, int(row.size()));
  }
  return maxc;
}

// Inverted edge table for the key-side gather of the edge-list backward
// (training with the per-query masks of "Critical power-law sparse
// attention", item 4, and "Christoffel-Balanced Sparse Attention"): for
// every key j the slots s = i * width + t with edges[i][t] = j, ascending.
extern "C" int sfa_edges_transpose(int n, int width, const int32_t* edges, const int32_t* count, int cap,
                                   int32_t* inv, int32_t* inv_count) {
  if (n < 0 || width < 1 || width > SFA_MAX_EDGE_WIDTH)
    return fail(SFA_ERR_ARG, "sfa_edges_transpose: bad n/width");
  if (n > 0 && (!edges || !count)) return fail(SFA_ERR_ARG, "sfa_edges_transpose: NULL edges or count");
  if (int64_t(n) * width > (int64_t(1) << 31) - 1)
    return fail(SFA_ERR_ARG, "sfa_edges_transpose: n * width exceeds int32 slot indices");
  std::vector<int32_t> deg(size_t(n), 0);
  for (int i = 0; i < n; ++i) {
    if (count[i] < 0 || count[i] > width)
      return fail(SFA_ERR_ARG, "sfa_edges_transpose: count[%d] = %d not in [0, width]", i, count[i]);
    for (int t = 0; t < count[i]; ++t) {
      const int32_t j = edges[size_t(i) * size_t(width) + t];
      if (j < 0 || j >= n) return fail(SFA_ERR_ARG, "sfa_edges_transpose: edges[%d][%d] = %d out of range", i, t, j);
      ++deg[size_t(j)];
    }
  }
  int need = 1;
  for (int j = 0; j < n; ++j) need = std::max(need, int(deg[size_t(j)]));
  if (!inv) return need;  // size query
  if (!inv_count) return fail(SFA_ERR_ARG, "sfa_edges_transpose: inv_count is NULL");
  if (cap < need) return fail(SFA_ERR_CAPACITY, "sfa_edges_transpose: needs cap >= %d, got %d", need, cap);
  for (int j = 0; j < n; ++j) {
    inv_count[j] = 0;
    for (int u = 0; u < cap; ++u) inv[size_t(j) * size_t(cap) + u] = -1;
  }
  for (int i = 0; i < n; ++i)
    for (int t = 0; t < count[i]; ++t) {
      const int32_t j = edges[size_t(i) * size_t(width) + t];
      inv[size_t(j) * size_t(cap) + size_t(inv_count[j]++)] = i * width + t;
    }
  return need;
}

// Rotary table: "Depth-Staggered Fibonacci Spacing for Sparse Attention",
// gather paragraph (rotation at true positions before the gather) and
// architecture paragraph (base 1e4); rotation of interleaved pairs.
extern "C" int sfa_rope_table(int n, int head_dim, double theta, float* table) {
  if (n < 1 || head_dim < 2 || (head_dim & 1))
    return fail(SFA_ERR_ARG, "sfa_rope_table: need n >= 1 and even head_dim >= 2");
  if (!std::isfinite(theta) || !(theta > 0.0))
    return fail(SFA_ERR_ARG, "sfa_rope_table: theta must be finite and > 0");
  if (!table) return fail(SFA_ERR_ARG, "sfa_rope_table: table is NULL");
  const int half = head_dim / 2;
  for (int p = 0; p < half; ++p) {
    const double inv = std::pow(theta, -2.0 * double(p) / double(head_dim));
    for (int m = 0; m < n; ++m) {
      const double ang = double(m) * inv;
      float* t = table + (size_t(m) * half + p) * 2;
      t[0] = float(std::cos(ang));
      t[1] = float(std::sin(ang));
    }
  }
  return SFA_OK;
}
