// 2^(t/64) in fp64 for t <= 0: the sampling kernels' softmax weights
// exp((z - max) / T) = 2^(t/64) with t = (z - max) * (64 / (T ln2)).  Own
// implementation, table-driven:
//   t = 64 k + j + f, with 64 k + j = n the integer nearest t, 0 <= j < 64
//   and |f| <= 1/2 (f = t - n is exact);
//   2^(t/64) = 2^k * 2^(j/64) * e^(f c),  c = ln2 / 64,
//   e^(f c) - 1 = sum_{i=1..5} (f c)^i / i!   (the omitted terms are below
//   3.5e-17 relative, as |f c| <= 0.0055).
// kExp2Frac[j] is 2^(j/64) correctly rounded to fp64 (from a 60-digit decimal
// evaluation), and the series coefficients c^i / i! likewise.  t below
// -69300 (2^(t/64) < 2^-1082) gives +0.  Within 2 ulp of 2^(t/64) for the t
// given; t itself carries the rounding of its own computation (relative
// 2^-52 or so, i.e. an absolute error of about |x| 2^-52 in the exponent x
// of e^x), as the argument of any fp64 exp would.  About 12 fp64
// instructions and one table read (from LDS in the kernels), against about
// 45 for the general library exp.
#pragma once

#if defined(__HIPCC__)
#define ORTHRUS_HD __host__ __device__
#else
#define ORTHRUS_HD
#endif

#include <cmath>

namespace orthrus {

constexpr double kExp2Frac[64] = {
    0x1.0000000000000p+0, 0x1.02c9a3e778061p+0, 0x1.059b0d3158574p+0, 0x1.0874518759bc8p+0,
    0x1.0b5586cf9890fp+0, 0x1.0e3ec32d3d1a2p+0, 0x1.11301d0125b51p+0, 0x1.1429aaea92de0p+0,
    0x1.172b83c7d517bp+0, 0x1.1a35beb6fcb75p+0, 0x1.1d4873168b9aap+0, 0x1.2063b88628cd6p+0,
    0x1.2387a6e756238p+0, 0x1.26b4565e27cddp+0, 0x1.29e9df51fdee1p+0, 0x1.2d285a6e4030bp+0,
    0x1.306fe0a31b715p+0, 0x1.33c08b26416ffp+0, 0x1.371a7373aa9cbp+0, 0x1.3a7db34e59ff7p+0,
    0x1.3dea64c123422p+0, 0x1.4160a21f72e2ap+0, 0x1.44e086061892dp+0, 0x1.486a2b5c13cd0p+0,
    0x1.4bfdad5362a27p+0, 0x1.4f9b2769d2ca7p+0, 0x1.5342b569d4f82p+0, 0x1.56f4736b527dap+0,
    0x1.5ab07dd485429p+0, 0x1.5e76f15ad2148p+0, 0x1.6247eb03a5585p+0, 0x1.6623882552225p+0,
    0x1.6a09e667f3bcdp+0, 0x1.6dfb23c651a2fp+0, 0x1.71f75e8ec5f74p+0, 0x1.75feb564267c9p+0,
    0x1.7a11473eb0187p+0, 0x1.7e2f336cf4e62p+0, 0x1.82589994cce13p+0, 0x1.868d99b4492edp+0,
    0x1.8ace5422aa0dbp+0, 0x1.8f1ae99157736p+0, 0x1.93737b0cdc5e5p+0, 0x1.97d829fde4e50p+0,
    0x1.9c49182a3f090p+0, 0x1.a0c667b5de565p+0, 0x1.a5503b23e255dp+0, 0x1.a9e6b5579fdbfp+0,
    0x1.ae89f995ad3adp+0, 0x1.b33a2b84f15fbp+0, 0x1.b7f76f2fb5e47p+0, 0x1.bcc1e904bc1d2p+0,
    0x1.c199bdd85529cp+0, 0x1.c67f12e57d14bp+0, 0x1.cb720dcef9069p+0, 0x1.d072d4a07897cp+0,
    0x1.d5818dcfba487p+0, 0x1.da9e603db3285p+0, 0x1.dfc97337b9b5fp+0, 0x1.e502ee78b3ff6p+0,
    0x1.ea4afa2a490dap+0, 0x1.efa1bee615a27p+0, 0x1.f50765b6e4540p+0, 0x1.fa7c1819e90d8p+0};

// 64 / ln2: t = x * kExp2Scale turns e^x into 2^(t/64)
constexpr double kExp2Scale = 0x1.71547652b82fep+6;

// tab: kExp2Frac or a copy of it (the kernels keep one in LDS)
ORTHRUS_HD inline double exp2_64(double t, const double* tab) {
  t = t < -69300.0 ? -69300.0 : t;
  const double n = std::rint(t);
  const double f = t - n;
  const int ni = static_cast<int>(n);
  const int j = ni & 63;                        // n = 64 k + j, k = floor(n / 64)
  const int k = ni >> 6;
  double p = std::fma(f, 0x1.5d87fe78a6731p-40, 0x1.3b2ab6fba4e77p-31);
  p = std::fma(p, f, 0x1.c6b08d704a0c0p-23);
  p = std::fma(p, f, 0x1.ebfbdff82c58fp-15);
  p = std::fma(p, f, 0x1.62e42fefa39efp-7);
  p = p * f;                                    // e^(f c) - 1
  return std::ldexp(std::fma(tab[j], p, tab[j]), k);
}

}  // namespace orthrus
