// NF4 codebook of the library, built once on the host.
//
// Levels: quantiles of a standard normal distribution ([P1] "QLoRA" bullets,
// "NF4 instead of a uniform grid"; [P2] "QLoRA" s1 "Key Innovation: NF4"):
// 16 levels, equal probability steps on each side, 8 positive levels and 7
// negative ones, an exact zero, normalised so the outermost levels are -1 and
// +1. The outermost levels sit at the centre of the outermost equal-probability
// bin (1 - 1/32 for 16 bins, 1 - 1/30 for 15 bins); one shared probability,
// their mean, keeps both ends at exactly +-1.
//
// The normal CDF here is its own series (no libm erf/erfc) and the inverse is
// Newton's method; the construction is checked at first use (see build()).
#include <cmath>
#include <cstring>
#include <mutex>

#include "../../include/qlora_amd.h"
#include "internal.h"

namespace qlora {
namespace {

double normal_pdf(double t) { return std::exp(-0.5 * t * t) / std::sqrt(2.0 * M_PI); }

// Phi(t) = 1/2 + pdf(t) * (t + t^3/3 + t^5/(3*5) + t^7/(3*5*7) + ...), a series
// that converges for every t and is accurate to a few ulps for |t| < 3.
double normal_cdf(double t) {
  const double t2 = t * t;
  double term = t, sum = t;
  for (int k = 1; k < 1000; ++k) {
    term *= t2 / (2.0 * k + 1.0);
    const double next = sum + term;
    if (next == sum) break;
    sum = next;
  }
  return 0.5 + normal_pdf(t) * sum;
}

// Inverse CDF for p in [1/2, 1) by Newton's method from t = 0. The CDF is
// concave on t > 0, so the iterates rise monotonically to the root.
double normal_quantile_upper(double p) {
  double t = 0.0;
  for (int it = 0; it < 400; ++it) {
    const double next = t - (normal_cdf(t) - p) / normal_pdf(t);
    if (!(next > t)) break;  // converged (or a last-ulp wobble)
    t = next;
  }
  return t;
}

uint32_t fnv1a(uint32_t h, const void* data, size_t n) {
  const unsigned char* p = static_cast<const unsigned char*>(data);
  for (size_t i = 0; i < n; ++i) {
    h ^= p[i];
    h *= 16777619u;
  }
  return h;
}

// Identifier of a quantization setup: the level-bit hash extended by the
// layout constants and the second level's top code value (127, 255 or 448,
// one per format). The default format's identifier is the codebook id.
uint32_t setup_hash(uint32_t level_hash, int dq_format) {
  const uint32_t top = dq_format == kDqInt8 ? 127u : dq_format == kDqUint8 ? 255u : 448u;
  const uint32_t meta[5] = {(uint32_t)kBlock, (uint32_t)kGroup, 1u /* even index in low nibble */,
                            top, QLORA_FORMAT_VERSION};
  return fnv1a(level_hash, meta, sizeof meta);
}

// Quotient threshold of decision threshold t (see Codebook::thr_q). A
// quotient of two normal bf16 numbers is q = a 2^j / b with significands a, b
// in [128, 255]. Every such q of t's sign within a factor of four of t is
// compared, exactly in integers (values in units of 2^-61), against t and
// against its fp32 successor s, and the result set against RN(q) > t, which
// holds when q is above the midpoint of t and s, or on it with s even (ties
// round to the even neighbour). The first candidate that agrees for every q
// is taken; false if neither does.
bool quotient_threshold(float t, float* out) {
  if (!(std::fabs(t) >= 0x1p-20f && std::fabs(t) < 1.0f)) return false;
  const float s = std::nextafter(t, INFINITY);
  const int64_t T = (int64_t)std::ldexp((double)t, 61), S = (int64_t)std::ldexp((double)s, 61);
  const int64_t mid = (T + S) / 2;  // T and S are even: t's last bit is 2^-43 or above
  uint32_t sbits;
  std::memcpy(&sbits, &s, 4);
  const bool tie_up = (sbits & 1u) == 0;
  const int sg = t < 0.0f ? -1 : 1;
  int e;
  std::frexp(std::fabs((double)t), &e);  // |t| in [2^(e-1), 2^e)
  bool t_ok = true, s_ok = true;
  for (int j = e - 3; j <= e + 1; ++j)
    for (int a = 128; a < 256; ++a) {
      const __int128 qs = (__int128)(sg * a) * ((__int128)1 << (j + 61));  // q * b * 2^61
      for (int b = 128; b < 256; ++b) {
        auto cmp = [&](int64_t X) {
          const __int128 r = (__int128)X * b;
          return (qs > r) - (qs < r);
        };
        const int cm = cmp(mid);
        const bool above = cm > 0 || (cm == 0 && tie_up);
        t_ok = t_ok && (cmp(T) > 0) == above;
        s_ok = s_ok && (cmp(S) > 0) == above;
      }
    }
  if (t_ok)
    *out = t;
  else if (s_ok)
    *out = s;
  return t_ok || s_ok;
}

struct State {
  Codebook cb{};
  uint32_t level_hash = 0;
  uint32_t id = 0;
  int status = QLORA_ERR_INTERNAL;
};

State build() {
  State s;
  const double pmax = 1.0 - (1.0 / 32.0 + 1.0 / 30.0) / 2.0;
  const double zmax = normal_quantile_upper(pmax);
  double lv[16];
  for (int i = 0; i < 7; ++i) {  // negative side, 7 levels
    const double p = 0.5 + (pmax - 0.5) * (double)(7 - i) / 7.0;
    lv[i] = -normal_quantile_upper(p) / zmax;
  }
  lv[7] = 0.0;
  for (int j = 0; j < 8; ++j) {  // positive side, 8 levels
    const double p = 0.5 + (pmax - 0.5) * (double)(j + 1) / 8.0;
    lv[8 + j] = normal_quantile_upper(p) / zmax;
  }
  lv[0] = -1.0;
  lv[15] = 1.0;
  for (int i = 0; i < 16; ++i) s.cb.level[i] = (float)lv[i];
  for (int i = 0; i < 15; ++i) {
    // Midpoint of two fp32 levels (exact in double), rounded toward -inf:
    // then "x > thr" for an fp32 x means x is above the true midpoint.
    const double m = 0.5 * ((double)s.cb.level[i] + (double)s.cb.level[i + 1]);
    float t = (float)m;
    if ((double)t > m) t = std::nextafter(t, -INFINITY);
    s.cb.thr[i] = t;
  }
  // Self-checks the quantize kernel relies on: strictly increasing levels,
  // interleaved thresholds, at most one threshold per 1/32-wide bucket of
  // [-1,1], no threshold within 2^-20 of a bucket edge nor in the last 1/16
  // of its bucket (the bf16 path's bucket index rounds to nearest and may
  // move such values up one bucket), and a quotient threshold for each.
  bool ok = s.cb.level[0] == -1.0f && s.cb.level[7] == 0.0f && s.cb.level[15] == 1.0f;
  for (int i = 0; i < 15; ++i) {
    ok = ok && s.cb.level[i] < s.cb.thr[i] && s.cb.thr[i] < s.cb.level[i + 1];
    const double pos = ((double)s.cb.thr[i] + 1.0) * 32.0;
    ok = ok && std::fabs(pos - std::nearbyint(pos)) > 32.0 * std::ldexp(1.0, -20);
    ok = ok && pos - std::floor(pos) < 15.0 / 16.0 - std::ldexp(1.0, -10);
    if (i > 0) ok = ok && std::floor(pos) != std::floor(((double)s.cb.thr[i - 1] + 1.0) * 32.0);
    ok = ok && quotient_threshold(s.cb.thr[i], &s.cb.thr_q[i]);
  }
  if (!ok) return s;
  uint32_t h = 2166136261u;
  for (int i = 0; i < 16; ++i) {
    uint32_t bits;
    std::memcpy(&bits, &s.cb.level[i], 4);
    h = fnv1a(h, &bits, 4);
  }
  s.level_hash = h;
  s.cb.dq_format = kDqInt8;
  s.id = setup_hash(h, kDqInt8);
  s.status = QLORA_OK;
  return s;
}

const State& state() {
  static std::once_flag once;
  static State st;
  std::call_once(once, [] { st = build(); });
  return st;
}

}  // namespace

int get_codebook(const Codebook** cb, uint32_t* id) {
  const State& st = state();
  if (st.status != QLORA_OK) return st.status;
  if (cb) *cb = &st.cb;
  if (id) *id = st.id;
  return QLORA_OK;
}

uint32_t setup_id(int dq_format) {
  const State& st = state();
  if (st.status != QLORA_OK) return 0u;
  if (dq_format != kDqInt8 && dq_format != kDqUint8 && dq_format != kDqE4m3) return 0u;
  return setup_hash(st.level_hash, dq_format);
}

}  // namespace qlora
