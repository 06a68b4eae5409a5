// Host restatement of the NVFP4 row encoder's arithmetic
// (precision_rl_amd/csrc/quantize.hip), checked against the direct rounding.
//
// Per block the encoder needs the E4M3 scale code d = RNE_E4M3(b / (6 g)) of
// the block's bf16 maximum b (g = RN_f32(a / 2688) from the row maximum a) and
// the E2M1 code RNE_E2M1(|x| / (d g)) of every element (miniTE Technical
// Report, section 5.1, block-scale equation).  Directly: one correctly
// rounded FP64 division for d, and the exact FP64 products mu_j d g for the
// seven E2M1 midpoints.  The kernel instead takes
//   scale:  b * RN64(1 / (6 g)) rounded to float, with an exact check when
//           that float is an E4M3 rounding midpoint;
//   codes:  the hardware conversion (round to nearest even onto E2M1,
//           modelled here as that) of RN32(x ilo) and RN32(x ihi), the
//           reciprocal of RN32(d g) nudged by 1 -+ 2^-19; where the two codes
//           differ, the element against the exact product mu d g of the
//           midpoint between them.
// Part A runs the scale code over every pair (row maximum, block maximum <=
// row maximum) of finite bf16 magnitudes -- the whole input domain of that
// step.  Part B runs the codes of the elements next to every midpoint (the
// bf16 values just below and above mu d g, and one further on each side),
// where a rounding error could move a code, for sampled pairs, with the
// hardware reciprocal taken as the correctly rounded one and one float ulp
// either side of it.  Any difference is reported.
// Arithmetic: IEEE binary32/binary64 round-to-nearest and fused multiply-add,
// as on the GPU (built without contraction).
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <thread>

namespace {

uint32_t bits_of(float f) { uint32_t u; std::memcpy(&u, &f, 4); return u; }
float float_of(uint32_t u) { float f; std::memcpy(&f, &u, 4); return f; }
float bf16_value(uint32_t b) { return float_of(b << 16); }

// ---------------------------------------------------------------- direct
uint32_t e4m3_rne(double q, double* val) {
  if (!(q > 0.0)) { *val = 0.0; return 0u; }
  if (q >= 448.0) { *val = 448.0; return 0x7Eu; }
  int ex;
  std::frexp(q, &ex);
  int e = std::max(ex - 1, -6);
  const double v = std::ldexp(std::rint(std::ldexp(q, 3 - e)), e - 3);
  *val = v;
  if (v == 0.0) return 0u;
  std::frexp(v, &ex);
  const int e2 = ex - 1;
  if (e2 < -6) return static_cast<uint32_t>(std::ldexp(v, 9));
  return static_cast<uint32_t>(((e2 + 7) << 3) | (static_cast<int>(std::ldexp(v, 3 - e2)) - 8));
}

// Value of an E4M3FN code: subnormal m 2^-9, normal (8 + m) 2^(e - 10).
double e4m3_value(uint32_t c) {
  const uint32_t e = c >> 3, m = c & 7u;
  return e == 0u ? static_cast<double>(m) * 0x1p-9 : std::ldexp(static_cast<double>(8u + m), static_cast<int>(e) - 10);
}

const double kMu[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};

// E2M1 magnitude code of |x| / D by the exact products: midpoint j separates
// codes j and j + 1, and a tie goes to the even code (crossing odd j takes
// |x| >= mu_j D, even j |x| > mu_j D).
uint32_t e2m1_direct(double xm, double D) {
  uint32_t c = 0;
  for (int j = 0; j < 7; ++j) {
    const double t = kMu[j] * D;
    c += (j & 1) ? (xm >= t ? 1u : 0u) : (xm > t ? 1u : 0u);
  }
  return c;
}

// Round to nearest even onto E2M1 magnitudes, saturating at 6 (the hardware
// conversion's rounding).
uint32_t e2m1_rne(float q) {
  const double m = std::fabs(static_cast<double>(q));
  uint32_t c = 0;
  for (int j = 0; j < 7; ++j) c += (j & 1) ? (m >= kMu[j] ? 1u : 0u) : (m > kMu[j] ? 1u : 0u);
  return c;
}

// ------------------------------------------------------------ the kernel's
uint32_t e4m3_code_fast(uint32_t b, double inv6g, double g6) {
  const double ab = static_cast<double>(bf16_value(b));
  const float q = static_cast<float>(ab * inv6g);
  const uint32_t qb = bits_of(q);
  const float qs = q * 512.0f;
  const bool sub = q < 0x1p-6f;
  uint32_t c = sub ? static_cast<uint32_t>(std::rint(qs)) : ((qb + 0x7FFFFu + ((qb >> 20) & 1u)) >> 20) - 960u;
  const bool mid = sub ? (qs - std::floor(qs)) == 0.5f : (qb & 0xFFFFFu) == 0x80000u;
  if (mid) {
    const double m = g6 * static_cast<double>(q);
    const uint32_t lo = sub ? static_cast<uint32_t>(std::floor(qs)) : (qb >> 20) - 960u;
    if (ab > m) c = lo + 1u;
    else if (ab < m) c = lo;
  }
  return std::min(c, 0x7Eu);
}

float e4m3_float(uint32_t c) {
  return c >= 8u ? float_of((c << 20) + (120u << 23)) : static_cast<float>(c) * 0x1p-9f;
}

// The code of element magnitude xm (a bf16 value) as the kernel forms it,
// with reciprocal `inv` of RN32(d g); *open is set where the bracket left it
// to the exact check.
uint32_t e2m1_kernel(float xm, float inv, uint32_t d, float g, bool* open) {
  volatile float lo_scale = inv * (1.0f - 0x1p-19f);   // plain products, not fused
  volatile float hi_scale = inv * (1.0f + 0x1p-19f);
  const float ilo = lo_scale, ihi = hi_scale;
  volatile float plo = xm * ilo, phi = xm * ihi;
  const uint32_t clo = e2m1_rne(plo), chi = e2m1_rne(phi);
  *open = clo != chi;
  if (clo == chi) return clo;
  const double t = kMu[clo] * (e4m3_value(d) * static_cast<double>(g));
  const double x = static_cast<double>(xm);
  return clo + ((x > t || (x == t && (clo & 1u))) ? 1u : 0u);
}

}  // namespace

int main() {
  // the decoded value of every code is the value the direct rounding returns
  for (uint32_t c = 0; c <= 0x7Eu; ++c) {
    double v;
    const double q = c == 0 ? 0.0 : e4m3_value(c);
    if (e4m3_rne(q, &v) != c || v != q) { std::printf("e4m3 value mismatch at code %02x\n", c); return 1; }
    if (c > 0 && static_cast<double>(e4m3_float(c)) != q) { std::printf("e4m3 float mismatch at code %02x\n", c); return 1; }
  }
  std::atomic<long> pairs{0}, scale_bad{0}, on_midpoint{0}, near_ties{0};
  std::atomic<long> elems{0}, code_bad{0}, opened{0}, ties{0};
  auto work = [&](uint32_t first, uint32_t step) {
    long n = 0, bad = 0, mids = 0, near = 0, ne = 0, cbad = 0, nopen = 0, ntie = 0;
    for (uint32_t a = first; a < 0x7F80u; a += step) {
      const float g = static_cast<float>(static_cast<double>(bf16_value(a)) / 2688.0);
      const bool fast = g == 0.0f || (g >= 0x1p-100f && g <= 0x1p100f);
      if (!fast) continue;
      const double g6 = 6.0 * static_cast<double>(g);
      const double inv6g = g > 0.0f ? 1.0 / g6 : 0.0;
      const bool sample = a % 7u == 0u;
      for (uint32_t b = 0; b <= a; ++b) {
        // part A: the scale code
        double dv = 0.0;
        const uint32_t d0 = g > 0.0f ? e4m3_rne(static_cast<double>(bf16_value(b)) / g6, &dv) : 0u;
        const uint32_t d1 = g > 0.0f ? e4m3_code_fast(b, inv6g, g6) : 0u;
        ++n;
        if (d0 != d1) {
          if (bad < 4) std::printf("scale mismatch: row max %04x block max %04x: %02x vs %02x\n", a, b, d0, d1);
          ++bad;
        }
        if (g > 0.0f) {
          const double ab = static_cast<double>(bf16_value(b));
          const float q = static_cast<float>(ab * inv6g);
          const float qs = q * 512.0f;
          const bool mid = q < 0x1p-6f ? (qs - std::floor(qs)) == 0.5f : (bits_of(q) & 0xFFFFFu) == 0x80000u;
          if (mid) { ++mids; if (g6 * static_cast<double>(q) != ab) ++near; }
        }
        // part B: the codes next to every midpoint, sampled pairs
        if (!sample || d0 == 0u || (b % 29u != 0u && b != a)) continue;
        const double D = e4m3_value(d0) * static_cast<double>(g);       // exact
        volatile float D32 = e4m3_float(d0) * g;
        const float r = 1.0f / D32;                                     // correctly rounded
        const float invs[3] = {r, std::nextafter(r, 0.0f), std::nextafter(r, INFINITY)};
        for (int j = 0; j < 7; ++j) {
          const double t = kMu[j] * D;
          const float tf = static_cast<float>(t);
          const uint32_t hb = bits_of(tf) >> 16;
          for (int dlt = -2; dlt <= 2; ++dlt) {
            const uint32_t xb = hb + static_cast<uint32_t>(dlt);
            if (xb == 0u || xb >= 0x7F80u) continue;
            const float xm = bf16_value(xb);
            const uint32_t want = e2m1_direct(static_cast<double>(xm), D);
            if (static_cast<double>(xm) == t) ++ntie;
            for (float inv : invs) {
              bool op = false;
              const uint32_t got = e2m1_kernel(xm, inv, d0, g, &op);
              ++ne;
              nopen += op ? 1 : 0;
              if (got != want) {
                if (cbad < 4) std::printf("code mismatch: row max %04x block scale %02x element %04x: %u vs %u\n", a, d0, xb, got, want);
                ++cbad;
              }
            }
          }
        }
      }
    }
    pairs += n; scale_bad += bad; on_midpoint += mids; near_ties += near;
    elems += ne; code_bad += cbad; opened += nopen; ties += ntie;
  };
  const unsigned n_threads = std::max(1u, std::min(16u, std::thread::hardware_concurrency()));
  std::thread pool[16];
  for (unsigned t = 0; t < n_threads; ++t) pool[t] = std::thread(work, t, n_threads);
  for (unsigned t = 0; t < n_threads; ++t) pool[t].join();
  std::printf("pairs %ld scale_mismatches %ld midpoint %ld near_ties %ld\n", pairs.load(), scale_bad.load(),
              on_midpoint.load(), near_ties.load());
  std::printf("elements %ld code_mismatches %ld open %ld exact_ties %ld\n", elems.load(), code_bad.load(),
              opened.load(), ties.load());
  return scale_bad.load() == 0 && code_bad.load() == 0 ? 0 : 1;
}
