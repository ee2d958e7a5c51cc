// sv_exp64.hpp -- float64 exponential of the float64 draw (sv_draw.hip):
// table-driven argument reduction after P. T. P. Tang, "Table-driven
// implementation of the exponential function in IEEE floating-point
// arithmetic", ACM Trans. Math. Software 15(2), 1989.
//
// x = n ln2/64 + r with n = rint(64 x / ln2) and |r| <= ln2/128 (plus the
// rounding of the product); with n = 64 m + j, j in [0, 64),
// exp(x) = 2^m 2^(j/64) e^r.  2^(j/64) is read from a table of the 64 values
// rounded to nearest; e^r is its Taylor polynomial of degree 5, whose
// truncation is below (ln2/128)^6 / 720 < 4e-17 relative.  r is reduced in
// two fused steps against a two-part ln2/64 (hi + lo), so it carries one
// rounding of a number below 0.0055.  Error: about 2 ulp (table entry 0.5,
// polynomial about 1, final product 0.5) for x in [-745, 709]; exactly 0
// below -745.2 (exp underflows to 0 there) and for -inf; NaN for NaN.
// Used for arguments x <= 0; its cost is about half that of the library
// exp (about 13 float64 operations), and it needs no polynomial constants
// in vector registers beyond the table.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace sv {

constexpr int kExp64Table = 64;
constexpr double kExp64Scale = 0x1.71547652b82fep+6;  // 64 / ln 2
constexpr double kExp64Hi = 0x1.62e42fefa39efp-7;     // ln2 / 64, rounded
constexpr double kExp64Lo = 0x1.abc9e3b39803fp-62;    // ln2 / 64 - kExp64Hi, rounded
constexpr double kExp64C3 = 0x1.5555555555555p-3;     // 1/6
constexpr double kExp64C4 = 0x1.5555555555555p-5;     // 1/24
constexpr double kExp64C5 = 0x1.1111111111111p-7;     // 1/120

// 2^(j/64), j = 0 .. 63, rounded to nearest.
constexpr double kExp2Frac[kExp64Table] = {
    0x1.0000000000000p+0, 0x1.02c9a3e778061p+0, 0x1.059b0d3158574p+0,
    0x1.0874518759bc8p+0, 0x1.0b5586cf9890fp+0, 0x1.0e3ec32d3d1a2p+0,
    0x1.11301d0125b51p+0, 0x1.1429aaea92de0p+0, 0x1.172b83c7d517bp+0,
    0x1.1a35beb6fcb75p+0, 0x1.1d4873168b9aap+0, 0x1.2063b88628cd6p+0,
    0x1.2387a6e756238p+0, 0x1.26b4565e27cddp+0, 0x1.29e9df51fdee1p+0,
    0x1.2d285a6e4030bp+0, 0x1.306fe0a31b715p+0, 0x1.33c08b26416ffp+0,
    0x1.371a7373aa9cbp+0, 0x1.3a7db34e59ff7p+0, 0x1.3dea64c123422p+0,
    0x1.4160a21f72e2ap+0, 0x1.44e086061892dp+0, 0x1.486a2b5c13cd0p+0,
    0x1.4bfdad5362a27p+0, 0x1.4f9b2769d2ca7p+0, 0x1.5342b569d4f82p+0,
    0x1.56f4736b527dap+0, 0x1.5ab07dd485429p+0, 0x1.5e76f15ad2148p+0,
    0x1.6247eb03a5585p+0, 0x1.6623882552225p+0, 0x1.6a09e667f3bcdp+0,
    0x1.6dfb23c651a2fp+0, 0x1.71f75e8ec5f74p+0, 0x1.75feb564267c9p+0,
    0x1.7a11473eb0187p+0, 0x1.7e2f336cf4e62p+0, 0x1.82589994cce13p+0,
    0x1.868d99b4492edp+0, 0x1.8ace5422aa0dbp+0, 0x1.8f1ae99157736p+0,
    0x1.93737b0cdc5e5p+0, 0x1.97d829fde4e50p+0, 0x1.9c49182a3f090p+0,
    0x1.a0c667b5de565p+0, 0x1.a5503b23e255dp+0, 0x1.a9e6b5579fdbfp+0,
    0x1.ae89f995ad3adp+0, 0x1.b33a2b84f15fbp+0, 0x1.b7f76f2fb5e47p+0,
    0x1.bcc1e904bc1d2p+0, 0x1.c199bdd85529cp+0, 0x1.c67f12e57d14bp+0,
    0x1.cb720dcef9069p+0, 0x1.d072d4a07897cp+0, 0x1.d5818dcfba487p+0,
    0x1.da9e603db3285p+0, 0x1.dfc97337b9b5fp+0, 0x1.e502ee78b3ff6p+0,
    0x1.ea4afa2a490dap+0, 0x1.efa1bee615a27p+0, 0x1.f50765b6e4540p+0,
    0x1.fa7c1819e90d8p+0,
};

// exp(x) with the table `tab` (kExp2Frac, or a copy of it in LDS).
__host__ __device__ __forceinline__ double exp64_tab(double x, const double* tab) {
  // clamp before the integer conversion (x = -inf, or far below underflow)
  const double n = fmax(rint(x * kExp64Scale), -70000.0);
  double r = fma(-n, kExp64Hi, x);
  r = fma(-n, kExp64Lo, r);
  double q = fma(r, kExp64C5, kExp64C4);
  q = fma(q, r, kExp64C3);
  q = fma(q, r, 0.5);
  q = fma(q, r, 1.0);
  q = fma(q, r, 1.0);
  const int ni = (int)n;
  const double y = ldexp(tab[ni & (kExp64Table - 1)] * q, ni >> 6);
  return x < -745.2 ? 0.0 : y;
}

}  // namespace sv
