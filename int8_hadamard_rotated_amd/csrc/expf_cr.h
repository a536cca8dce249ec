// exp of a binary32 argument, correctly rounded to binary32 (round to
// nearest, ties to even), for the gated activations SiLU and Sigmoid ahead of
// the quantizer (page "ggml operator extensions", section "sd.cpp
// integration": SiLU/Sigmoid -> Mul -> ConvRot, SwiGLU -> ConvRot).  The
// quantizer's codes are decisions on these values, so the exp must be the one
// exact function, not an approximation that differs from other
// implementations in the last bit.
//
// Method: argument reduction x = k ln2 + r with a three-part ln2 (its first
// part short enough that k * part is exact), |r| <= ln2 / 2, then
//   fast path: a degree-10 polynomial in binary64 with fused multiply-adds,
//     scaled by 2^k.  The polynomial is the Chebyshev series of exp on
//     [-0.3466, 0.3466] truncated after degree 10 (its coefficients are twice
//     the modified Bessel values I_j(0.3466), I_0 once), rewritten in powers of
//     r and rounded to binary64: relative error 2^-51.3 before evaluation,
//     below 2^-50 with the evaluation's rounding, so within the 2^-49 window
//     below (the Taylor series needs degree 13 for the same bound).  Its
//     binary32 rounding is returned unless the binary64 value lies within
//     2^-49 (relative) of a binary32 rounding boundary: for binary32-normal
//     results, unless the 29 bits of the binary64 significand below binary32
//     precision are within 16 of the halfway pattern (a table-driven
//     reduction to a shorter series measured slower: its per-element table
//     gathers cost more than the multiply-adds they save);
//   slow path (a few dozen of the 2^31 arguments in range): the same series
//     in double-double arithmetic (error far below 2^-90) and an exact
//     rounding of the double-double sum.
// Checked against exp rounded once from x87 extended precision on every
// binary32 argument in [-104, 89] (tests/test_expf_host.py builds this header
// for the host); below -104 the result is 0, above 89 it is +inf.
//
// Binary64 operations here must not be contracted: compile with
// -ffp-contract=off (the fused multiply-adds are explicit).
#pragma once
#include <cstdint>

#ifndef CONVROT_HD
#define CONVROT_HD __host__ __device__
#endif
#ifndef CONVROT_NOINLINE
#define CONVROT_NOINLINE __attribute__((noinline))
#endif

namespace convrot_expf {

constexpr double kInvLn2 = 1.4426950408889634;
constexpr double kLn2Hi = 0x1.62e42fefa3800p-1;    // 42 significant bits
constexpr double kLn2Lo = 0x1.ef35793c76730p-45;
constexpr double kLn2Lo2 = 0x1.f97b57a079a19p-103;
constexpr double kOverflow = 0x1.fffffep127 + 0x1p103;   // FLT_MAX + half its ulp

CONVROT_HD inline double fma_d(double a, double b, double c) { return __builtin_fma(a, b, c); }

// A constant the device keeps in a scalar register pair, so that a binary64
// multiply-add takes it as an operand instead of rebuilding it per use.
CONVROT_HD inline double uniform(double c)
{
#if defined(__HIP_DEVICE_COMPILE__)
    asm("" : "+s"(c));
#endif
    return c;
}

// 2^k * v for -150 <= k <= 130 as two scalings by powers of two, each exact
// because every value involved stays a normal binary64 number.
CONVROT_HD inline double scale2(double v, int k)
{
    const int k1 = k / 2, k2 = k - k1;
    const double s1 = __builtin_bit_cast(double, (uint64_t)(1023 + k1) << 52);
    const double s2 = __builtin_bit_cast(double, (uint64_t)(1023 + k2) << 52);
    return (v * s1) * s2;
}

// ---- double-double helpers (value hi + lo, |lo| <= half an ulp of hi)
struct dd {
    double hi, lo;
};
CONVROT_HD inline dd two_sum(double a, double b)
{
    const double s = a + b, bb = s - a;
    return {s, (a - (s - bb)) + (b - bb)};
}
CONVROT_HD inline dd fast_two_sum(double a, double b)
{
    const double s = a + b;
    return {s, b - (s - a)};
}
CONVROT_HD inline dd dd_add(dd a, dd b)
{
    dd s = two_sum(a.hi, b.hi);
    s.lo += a.lo + b.lo;
    return fast_two_sum(s.hi, s.lo);
}
CONVROT_HD inline dd dd_mul(dd a, dd b)
{
    const double p = a.hi * b.hi;
    double e = fma_d(a.hi, b.hi, -p);
    e += a.hi * b.lo + a.lo * b.hi;
    return fast_two_sum(p, e);
}
CONVROT_HD inline dd dd_div(dd a, double b)
{
    const double q = a.hi / b;
    double r = fma_d(-q, b, a.hi);
    r += a.lo;
    return fast_two_sum(q, r / b);
}

// The neighbour of a positive binary32 f: one up or one down.
CONVROT_HD inline float next_up(float f) { return __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, f) + 1u); }
CONVROT_HD inline float next_down(float f) { return __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, f) - 1u); }

// exp(x) in double-double, relative error far below 2^-90.
CONVROT_HD inline dd exp_dd(float xf)
{
    const double x = xf;
    const double k = __builtin_rint(x * kInvLn2);
    dd r = two_sum(x, -(k * kLn2Hi));                     // k * kLn2Hi is exact
    const double q = k * kLn2Lo;
    r = dd_add(r, dd{-q, -fma_d(k, kLn2Lo, -q)});
    r = dd_add(r, dd{-(k * kLn2Lo2), 0.0});
    dd sum = {1.0, 0.0}, term = {1.0, 0.0};
    for (int n = 1; n <= 30; ++n) {
        term = dd_div(dd_mul(term, r), (double)n);
        sum = dd_add(sum, term);
    }
    return dd{scale2(sum.hi, (int)k), scale2(sum.lo, (int)k)};
}

// Round a positive double-double to binary32: (float)hi, unless hi lies
// exactly halfway between two binary32 values, where lo decides.  (If the
// exact value were across a midpoint from hi, that midpoint, a binary64
// value, would be nearer to it than hi, which is the rounded sum.)
CONVROT_HD inline float round_dd(dd v)
{
    const float f = (float)v.hi;
    const double fd = f;
    if (fd == v.hi || v.lo == 0.0)
        return f;
    const float nb = v.hi > fd ? next_up(f) : next_down(f);
    if (v.hi != 0.5 * (fd + (double)nb))
        return f;
    const bool above = v.lo > 0.0;                        // the exact value vs the midpoint
    if (v.hi > fd)
        return above ? nb : f;
    return above ? f : nb;
}

CONVROT_HD CONVROT_NOINLINE inline float expf_slow(float x) { return round_dd(exp_dd(x)); }

CONVROT_HD inline float expf_cr(float x)
{
    if (x > 89.0f)
        return __builtin_huge_valf();
    if (x < -104.0f)
        return 0.0f;
    const double xd = x;
    const double k = __builtin_rint(xd * uniform(kInvLn2));
    double r = fma_d(-k, uniform(kLn2Hi), xd);
    r = fma_d(-k, uniform(kLn2Lo), r);
    // the degree-10 polynomial of the fast path (see the header comment)
    double p = uniform(0x1.28b40e50912c4p-22);
    p = fma_d(p, r, uniform(0x1.72fafc8b35748p-19));
    p = fma_d(p, r, uniform(0x1.a01991a2e8693p-16));
    p = fma_d(p, r, uniform(0x1.a01978baa91ffp-13));
    p = fma_d(p, r, uniform(0x1.6c16c187ff82fp-10));
    p = fma_d(p, r, uniform(0x1.1111112dda5a8p-7));
    p = fma_d(p, r, uniform(0x1.555555554f0bdp-5));
    p = fma_d(p, r, uniform(0x1.555555554b73ap-3));
    p = fma_d(p, r, uniform(0x1.0000000000011p-1));
    p = fma_d(p, r, uniform(0x1.000000000001ep+0));
    p = fma_d(p, r, 1.0);
    // |k| <= 150, so 2^k and p * 2^k are normal binary64 numbers: exact
    const double y = __builtin_ldexp(p, (int)k);
    const float f = (float)y;
    if (y >= 0x1p-126 && y < 0x1.fffffep127) {
        const uint32_t low = (uint32_t)(__builtin_bit_cast(uint64_t, y) & 0x1FFFFFFFu);
        if (low > 0x10000000u + 16u || low < 0x10000000u - 16u)
            return f;
        return expf_slow(x);
    }
    // results below the binary32 normal range or at its top: the rounding
    // boundaries next to f (the overflow threshold above FLT_MAX)
    const uint32_t fb = __builtin_bit_cast(uint32_t, f);
    const double fd = f;
    const bool is_inf = fb >= 0x7F800000u;
    const double up = is_inf ? 0.0 : (fb == 0x7F7FFFFFu ? kOverflow : 0.5 * (fd + (double)next_up(f)));
    const double dn = is_inf ? kOverflow : (fb == 0u ? 0.0 : 0.5 * (fd + (double)next_down(f)));
    const double tol = y * 0x1p-49;
    if ((is_inf || up - y > tol) && (fb == 0u || y - dn > tol))
        return f;
    return expf_slow(x);
}

}  // namespace convrot_expf
