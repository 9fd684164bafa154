// Host-side batch planning: the length-bucket batch sampler, dual-constraint
// batch sizing and the step-cost fit.
//
// "LingBot-VA packing" report, section 2.1 (LengthBucketBatchSampler, pad
// collate): per epoch, a shuffle seeded with seed + epoch, a round-robin shard
// over the ranks with the tail padded so every rank gets the same number of
// batches, pools of episodes sorted by length and cut into batches, and a
// shuffled batch order; a batch is padded to round_up(max frames, multiple).
// AdaptiveLoad summary, section 2A: a bucket of sequence length S gets the
// batch size max(1, min(floor(M_mem / S), floor(M_comp / S^p))), with p and
// M_comp taken from a fit of step time ~ a + b * B * S^p to measured shapes.
//
// The shuffles use SplitMix64 (Steele, Lea and Flood, 2014) and Fisher-Yates
// with j = high 64 bits of next() * (i + 1), so a plan is reproducible from
// (seed, epoch) on any host.
#include <stdint.h>

#include <algorithm>
#include <cmath>
#include <vector>

#include "packattn.h"

namespace {

struct SplitMix64 {
  uint64_t s;
  uint64_t next() {
    s += 0x9E3779B97F4A7C15ull;
    uint64_t z = s;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
  uint64_t below(uint64_t bound) {
    return (uint64_t)(((unsigned __int128)next() * bound) >> 64);
  }
};

template <typename V>
void shuffle(std::vector<V>& v, SplitMix64& g) {
  for (size_t i = v.size(); i-- > 1;) std::swap(v[i], v[g.below(i + 1)]);
}

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

int32_t batch_size_for(double seq_len, double m_mem, double m_comp, double p) {
  const double a = std::floor(m_mem / seq_len), b = std::floor(m_comp / std::pow(seq_len, p));
  const double v = std::min(a, b);
  if (!(v >= 1.0)) return 1;
  return v > 2147483647.0 ? 2147483647 : (int32_t)v;
}

}  // namespace

extern "C" size_t length_bucket_rank_size(int32_t n, int32_t world_size) {
  if (n < 0 || world_size < 1) return 0;
  return (size_t)((n + world_size - 1) / world_size);
}

extern "C" int32_t dual_constraint_batch(double seq_len, double m_mem, double m_comp, double p) {
  if (!(seq_len > 0) || !(m_mem > 0) || !(m_comp > 0) || !std::isfinite(p)) return PA_ERR_SHAPE;
  return batch_size_for(seq_len, m_mem, m_comp, p);
}

extern "C" int32_t length_bucket_batches(const int32_t* frames, int32_t n, uint64_t seed,
                                         int32_t epoch, int32_t pool_size, int32_t pad_multiple,
                                         int32_t batch_size, const pa_dual_constraint* dual,
                                         int32_t rank, int32_t world_size, int32_t* episodes,
                                         int32_t* batch_ptr, int32_t* batch_frames,
                                         int32_t* n_batches) {
  if (n < 0 || pool_size < 1 || pad_multiple < 1 || batch_size < 0 || world_size < 1 ||
      rank < 0 || rank >= world_size)
    return PA_ERR_SHAPE;
  if (!n_batches || (n > 0 && (!frames || !episodes || !batch_ptr || !batch_frames)))
    return PA_ERR_NULL;
  if (batch_size == 0) {
    if (!dual) return PA_ERR_NULL;
    if (!(dual->m_mem > 0) || !(dual->m_comp > 0) || !std::isfinite(dual->p) ||
        dual->tokens_per_frame < 1)
      return PA_ERR_SHAPE;
  }
  for (int32_t i = 0; i < n; ++i)
    if (frames[i] < 0) return PA_ERR_SHAPE;
  SplitMix64 g{seed + (uint64_t)(int64_t)epoch};
  std::vector<int32_t> order(n);
  for (int32_t i = 0; i < n; ++i) order[i] = i;
  shuffle(order, g);
  *n_batches = 0;
  if (n == 0) return PA_OK;
  const int64_t total = (int64_t)(n + world_size - 1) / world_size * world_size;
  std::vector<int32_t> mine;
  for (int64_t i = rank; i < total; i += world_size) mine.push_back(order[i % n]);
  std::vector<std::vector<int32_t>> batches;
  const auto shorter = [&](int32_t a, int32_t b) { return frames[a] < frames[b]; };
  for (size_t p0 = 0; p0 < mine.size(); p0 += (size_t)pool_size) {
    std::vector<int32_t> pool(mine.begin() + p0,
                              mine.begin() + std::min(mine.size(), p0 + (size_t)pool_size));
    std::stable_sort(pool.begin(), pool.end(), shorter);
    if (batch_size > 0) {
      for (size_t b0 = 0; b0 < pool.size(); b0 += (size_t)batch_size)
        batches.emplace_back(pool.begin() + b0,
                             pool.begin() + std::min(pool.size(), b0 + (size_t)batch_size));
    } else {
      // ascending lengths: a batch grows while its size fits the bound of its
      // padded sequence length (the bound only shrinks as the batch grows)
      std::vector<int32_t> cur;
      for (int32_t e : pool) {
        const int64_t s = round_up(frames[e], pad_multiple) * dual->tokens_per_frame;
        const int32_t cap = batch_size_for((double)s, dual->m_mem, dual->m_comp, dual->p);
        if (!cur.empty() && (int64_t)cur.size() + 1 > cap) {
          batches.push_back(cur);
          cur.clear();
        }
        cur.push_back(e);
      }
      if (!cur.empty()) batches.push_back(cur);
    }
  }
  shuffle(batches, g);
  int32_t pos = 0;
  batch_ptr[0] = 0;
  for (size_t b = 0; b < batches.size(); ++b) {
    int32_t mx = 0;
    for (int32_t e : batches[b]) {
      episodes[pos++] = e;
      mx = std::max(mx, frames[e]);
    }
    batch_ptr[b + 1] = pos;
    batch_frames[b] = (int32_t)round_up(mx, pad_multiple);
  }
  *n_batches = (int32_t)batches.size();
  return PA_OK;
}

extern "C" int32_t fit_step_cost(const double* B, const double* S, const double* t, int32_t m,
                                 double p_lo, double p_hi, double* out) {
  if (m < 2 || !(p_lo < p_hi) || !std::isfinite(p_lo) || !std::isfinite(p_hi))
    return PA_ERR_SHAPE;
  if (!B || !S || !t || !out) return PA_ERR_NULL;
  for (int32_t i = 0; i < m; ++i)
    if (!(B[i] > 0) || !(S[i] > 0) || !std::isfinite(t[i])) return PA_ERR_SHAPE;
  // for a fixed p, a and b are the least-squares line of t against u = B * S^p
  // (centred, with u scaled by its maximum for conditioning)
  const auto solve = [&](double p, double* a, double* b) {
    std::vector<double> u(m);
    double umax = 0;
    for (int32_t i = 0; i < m; ++i) umax = std::max(umax, u[i] = B[i] * std::pow(S[i], p));
    double um = 0, tm = 0;
    for (int32_t i = 0; i < m; ++i) {
      u[i] /= umax;
      um += u[i];
      tm += t[i];
    }
    um /= m;
    tm /= m;
    double sxy = 0, sxx = 0;
    for (int32_t i = 0; i < m; ++i) {
      sxy += (u[i] - um) * (t[i] - tm);
      sxx += (u[i] - um) * (u[i] - um);
    }
    const double bs = sxx > 0 ? sxy / sxx : 0.0;
    const double as = tm - bs * um;
    double rss = 0;
    for (int32_t i = 0; i < m; ++i) {
      const double r = as + bs * u[i] - t[i];
      rss += r * r;
    }
    if (a) *a = as;
    if (b) *b = bs / umax;
    return rss;
  };
  // golden-section search of the residual over p
  const double gr = 0.5 * (std::sqrt(5.0) - 1.0);
  double lo = p_lo, hi = p_hi;
  double x1 = hi - gr * (hi - lo), x2 = lo + gr * (hi - lo);
  double f1 = solve(x1, nullptr, nullptr), f2 = solve(x2, nullptr, nullptr);
  for (int it = 0; it < 200 && hi - lo > 1e-13; ++it) {
    if (f1 <= f2) {
      hi = x2;
      x2 = x1;
      f2 = f1;
      x1 = hi - gr * (hi - lo);
      f1 = solve(x1, nullptr, nullptr);
    } else {
      lo = x1;
      x1 = x2;
      f1 = f2;
      x2 = lo + gr * (hi - lo);
      f2 = solve(x2, nullptr, nullptr);
    }
  }
  const double p = 0.5 * (lo + hi);
  solve(p, &out[0], &out[1]);
  out[2] = p;
  return PA_OK;
}
