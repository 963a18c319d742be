// e^x in fp64 for the non-positive arguments of the sampling kernels
// (softmax weights exp((z - max) / T)).  Own implementation, table-driven:
//   x = (64 k + j) ln2 / 64 + r, with 64 k + j the integer nearest 64 x / ln2,
//   0 <= j < 64 and |r| <= ln2 / 128;
//   e^x = 2^k * 2^(j/64) * e^r,  e^r = 1 + r + r^2/2 + r^3/6 + r^4/24 + r^5/120
//   (the omitted terms are below 3.5e-17 relative).
// The reduction is Cody-Waite: ln2 / 64 = kC1 + kC2 with kC1 rounded to 36
// significant bits, so n * kC1 is exact for |n| < 2^17 (all x >= -750).
// kExp2Frac[j] is 2^(j/64) correctly rounded to fp64 (from a 60-digit decimal
// evaluation).  Arguments below -750 give +0 (e^x < 2^-1075 rounds to zero
// anyway); elsewhere the result is within 2 ulp of the exact value.  About 13
// fp64 instructions and one table read (from LDS in the kernels), against
// about 45 instructions for the general library exp.
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

// tab: kExp2Frac or a copy of it (the kernels keep one in LDS)
ORTHRUS_HD inline double exp_nonpos(double x, const double* tab) {
  const double k64OverLn2 = 0x1.71547652b82fep+6;
  const double kC1 = 0x1.62e42fefa0000p-7;     // ln2 / 64 to 36 bits
  const double kC2 = 0x1.cf79abc9e3b3ap-46;    // ln2 / 64 - kC1
  x = x < -750.0 ? -750.0 : x;
  const double t = std::rint(x * k64OverLn2);
  double r = std::fma(-t, kC1, x);
  r = std::fma(-t, kC2, r);
  const int n = static_cast<int>(t);
  const int j = n & 63;                         // n = 64 k + j, k = floor(n / 64)
  const int k = n >> 6;
  double p = std::fma(r, 0x1.1111111111111p-7, 0x1.5555555555555p-5);   // 1/120, 1/24
  p = std::fma(p, r, 0x1.5555555555555p-3);                             // 1/6
  p = std::fma(p, r, 0.5);
  p = std::fma(p, r, 1.0);
  p = p * r;                                                            // e^r - 1
  return std::ldexp(std::fma(tab[j], p, tab[j]), k);
}

}  // namespace orthrus
