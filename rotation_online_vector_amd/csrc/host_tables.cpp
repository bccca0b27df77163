// Host-side plan tables: Philox4x32-10 randomness, fp64 Box-Muller -> bf16, and the
// Lloyd-Max codebook for the rotated-coordinate law.  Independent of any test code.
//
// Randomness (TurboQuant technical overview, intelliparadigm.com, §2.1.2 and §2.3.2:
// rotation signs and the QJL projection come from a seeded pseudo-random generator
// rather than stored matrices).  Generator: Philox4x32-10 as defined in Salmon, Moraes,
// Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11).
//   key = (seed lo, seed hi); counter = (block lo, block hi, domain, 0)
//   domain = purpose << 24 | subset << 16 | round << 8
//   purpose 1: rotation signs (rounds 0..2), purpose 2: QJL Gaussian (round 0)
//
// Codebook (same page, §1.2.2 and §2.2): Lloyd-Max for the density
// (1 - t^2)^a, a = (D-3)/2, on [-1, 1].  Cell masses use J_a(t) = int_0^t (1-s^2)^a ds
// from the integration-by-parts recurrence (2a+1) J_a = t (1-t^2)^a + 2a J_{a-1},
// started at J_0 = t (integer a) or J_{-1/2} = asin t (half-integer a).
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#include "tq_internal.h"

namespace tq {

// ---------------------------------------------------------------- Philox4x32-10

static inline void philox_round(uint32_t c[4], uint32_t k0, uint32_t k1) {
  const uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
  const uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
  const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
  const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
  const uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
  c[0] = n0; c[1] = lo1; c[2] = n2; c[3] = lo0;
}

void philox4x32_10(uint64_t block, uint32_t domain, uint64_t seed, uint32_t out[4]) {
  uint32_t c[4] = {(uint32_t)block, (uint32_t)(block >> 32), domain, 0u};
  uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
    philox_round(c, k0, k1);
  }
  memcpy(out, c, sizeof(c));
}

static inline uint32_t domain_word(int purpose, int subset, int round) {
  return ((uint32_t)purpose << 24) | ((uint32_t)subset << 16) | ((uint32_t)round << 8);
}

void sign_words(uint64_t seed, int subset, int D, uint32_t* words /* [3][D/32] */) {
  const int nw = D / 32;
  for (int r = 0; r < 3; ++r) {
    const uint32_t dom = domain_word(1, subset, r);
    for (int b = 0; 4 * b < nw; ++b) {
      uint32_t o[4];
      philox4x32_10((uint64_t)b, dom, seed, o);
      for (int t = 0; t < 4 && 4 * b + t < nw; ++t) words[r * nw + 4 * b + t] = o[t];
    }
  }
}

// fp64 -> bf16 bits, round to nearest, ties to even, directly from the double's bits.
uint16_t bf16_rne_from_double(double x) {
  uint64_t u;
  memcpy(&u, &x, 8);
  const uint64_t sign = u >> 63;
  int64_t e = (int64_t)((u >> 52) & 0x7FF);
  uint64_t m = u & ((1ull << 52) - 1);
  if (e == 0) return (uint16_t)(sign << 15);          // zero / fp64 subnormal -> signed zero
  // keep 7 fraction bits of 52: round at bit 45
  const uint64_t keep = m >> 45, rest = m & ((1ull << 45) - 1), half = 1ull << 44;
  uint64_t mant = keep;
  if (rest > half || (rest == half && (keep & 1))) mant += 1;
  if (mant == 128) { mant = 0; e += 1; }
  const int64_t eb = e - 1023 + 127;                  // bf16 shares fp32's exponent
  if (eb >= 255) return (uint16_t)((sign << 15) | 0x7F80);
  if (eb <= 0) return (uint16_t)(sign << 15);          // below fp32 normal range: not reached
  return (uint16_t)((sign << 15) | ((uint64_t)eb << 7) | mant);
}

void qjl_matrix_bf16(uint64_t seed, int subset, int k, int D, uint16_t* S) {
  const uint64_t count = (uint64_t)k * (uint64_t)D;
  const uint32_t dom = domain_word(2, subset, 0);
  const double two_pi = 2.0 * M_PI;
  for (uint64_t b = 0; 4 * b < count; ++b) {
    uint32_t o[4];
    philox4x32_10(b, dom, seed, o);
    double g[4];
    for (int p = 0; p < 2; ++p) {
      const double u1 = ((double)o[2 * p] + 0.5) * 0x1p-32;
      const double u2 = ((double)o[2 * p + 1] + 0.5) * 0x1p-32;
      const double rho = std::sqrt(-2.0 * std::log(u1));
      const double th = two_pi * u2;
      g[2 * p] = rho * std::cos(th);
      g[2 * p + 1] = rho * std::sin(th);
    }
    for (int t = 0; t < 4 && 4 * b + t < count; ++t) S[4 * b + t] = bf16_rne_from_double(g[t]);
  }
}

// ---------------------------------------------------------------- Lloyd-Max codebook

namespace {

// J_a(t) = int_0^t (1 - s^2)^a ds for a = a0 + j, a0 in {0, -1/2}, by the upward recurrence.
struct BetaLaw {
  int D;
  double a;
  bool half;     // a is a half-integer
  double norm;   // 2 J_a(1): total mass of (1 - s^2)^a on [-1, 1]

  explicit BetaLaw(int D_) : D(D_), a((D_ - 3) / 2.0), half((D_ % 2) == 0) { norm = 2.0 * J(1.0); }

  double J(double t) const {
    const double s = std::max(0.0, 1.0 - t * t);
    double aa, Jv;
    if (half) { aa = -0.5; Jv = std::asin(t); } else { aa = 0.0; Jv = t; }
    double pw = half ? std::sqrt(s) : s;   // s^(aa+1) for the first step
    while (aa < a - 0.25) {
      aa += 1.0;
      Jv = (t * pw + 2.0 * aa * Jv) / (2.0 * aa + 1.0);
      pw *= s;
    }
    return Jv;
  }
  // int_lo^hi s (1-s^2)^a ds = [(1-lo^2)^(a+1) - (1-hi^2)^(a+1)] / (2 (a+1))
  double moment1(double lo, double hi) const {
    const double sl = std::max(0.0, 1.0 - lo * lo), sh = std::max(0.0, 1.0 - hi * hi);
    return (std::pow(sl, a + 1.0) - std::pow(sh, a + 1.0)) / (2.0 * (a + 1.0));
  }
};

}  // namespace

int solve_codebook(int D, int R, double* levels, double* thresholds) {
  const int L = 1 << R;
  const BetaLaw law(D);
  const double sd = 1.0 / std::sqrt((double)D);
  const double span = std::min(4.0 * sd, 0.999);
  std::vector<double> t(L + 1), c(L), Jt(L + 1);
  t[0] = -1.0; t[L] = 1.0;
  for (int j = 1; j < L; ++j) t[j] = -span + 2.0 * span * j / L;
  // Stop when the thresholds move by less than 2e-15/sqrt(D), or once the moves stop
  // shrinking at the rounding-noise floor (below 1e-12/sqrt(D)).
  const double tol = 2e-15 * sd;
  double best = 1e300;
  int stall = 0;
  for (int it = 0; it < 1000000; ++it) {
    for (int j = 0; j <= L; ++j) Jt[j] = law.J(t[j]);
    for (int l = 0; l < L; ++l) c[l] = law.moment1(t[l], t[l + 1]) / (Jt[l + 1] - Jt[l]);
    // exact symmetry of the law: mirror the upper half onto the lower half
    for (int l = 0; l < L / 2; ++l) {
      const double v = 0.5 * (c[L - 1 - l] - c[l]);
      c[L - 1 - l] = v; c[l] = -v;
    }
    double moved = 0.0;
    for (int j = 1; j < L; ++j) {
      const double nt = (j == L / 2) ? 0.0 : 0.5 * (c[j - 1] + c[j]);
      moved = std::max(moved, std::fabs(nt - t[j]));
      t[j] = nt;
    }
    if (moved <= tol) break;
    if (moved < best) { best = moved; stall = 0; } else if (moved < 1e-12 * sd && ++stall > 50) break;
  }
  for (int j = 0; j <= L; ++j) Jt[j] = law.J(t[j]);
  for (int l = 0; l < L; ++l) c[l] = law.moment1(t[l], t[l + 1]) / (Jt[l + 1] - Jt[l]);
  for (int l = 0; l < L / 2; ++l) {
    const double v = 0.5 * (c[L - 1 - l] - c[l]);
    c[L - 1 - l] = v; c[l] = -v;
  }
  for (int l = 0; l < L; ++l) levels[l] = c[l];
  for (int j = 1; j < L; ++j) thresholds[j - 1] = t[j];
  return 0;
}

}  // namespace tq
