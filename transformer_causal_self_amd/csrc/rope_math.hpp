// rope_math.hpp -- the rotation of one RoPE channel pair, shared by every
// kernel that rotates (the RoPE pass, the decode-step preparation and the
// prefill kernel's query load), so they all produce the same bits.
//
// A pair (x1, x2) turns by the angle whose float32 cosine and sine are
// (c, s): [[c, -s], [s, c]] ("Transformer" (ai-notes) -- RoPE; "The
// Transformer architecture" -- Now: RoPE).  Written with explicit fused
// multiply-adds so that no kernel's compiler contracts it differently.
#pragma once

namespace rocattn {

__device__ inline void rope_turn(float x1, float x2, float c, float s, float& y1, float& y2) {
    y1 = fmaf(x1, c, -(x2 * s));
    y2 = fmaf(x1, s, x2 * c);
}

// sin and cos of a RoPE angle x (|x| < 2^31) in double precision, for the
// float32 (cos, sin) the rotations use.  Cody and Waite's argument
// reduction (W. J. Cody and W. Waite, Software Manual for the Elementary
// Functions, 1980): x = k (pi/2) + r with k the nearest integer to x / (pi/2)
// and pi/2 split into three doubles P1 + P2 + P3, each product k Pi exact
// inside a fused multiply-add, so |r| <= pi/4 carries no cancellation loss.
// Then the Taylor series of sin and cos at r, whose coefficients are
// (-1)^n / n! (terms through r^17 and r^18: the remainders, below 1e-19,
// sit under half an ulp), and the quadrant k mod 4 picks and signs them.
__device__ inline void rope_sincos(double x, double& s, double& c) {
    constexpr double P1 = 0x1.921fb54442d18p+0;     // pi/2 rounded to a double
    constexpr double P2 = 0x1.1a62633145c07p-54;    // pi/2 - P1 rounded
    constexpr double P3 = -0x1.f1976b7ed8fbcp-110;  // pi/2 - P1 - P2 rounded
    constexpr double TWO_OVER_PI = 0x1.45f306dc9c883p-1;
    const double k = rint(x * TWO_OVER_PI);
    double r = fma(-k, P1, x);
    r = fma(-k, P2, r);
    r = fma(-k, P3, r);
    const double z = r * r;
    // sin r = r + r z (-1/3! + z (1/5! - z (1/7! - ...))), Horner in z
    double ps = 1.0 / 355687428096000.0;                 // 1/17!
    ps = fma(z, ps, -1.0 / 1307674368000.0);            // 1/15!
    ps = fma(z, ps, 1.0 / 6227020800.0);                // 1/13!
    ps = fma(z, ps, -1.0 / 39916800.0);                 // 1/11!
    ps = fma(z, ps, 1.0 / 362880.0);                    // 1/9!
    ps = fma(z, ps, -1.0 / 5040.0);                     // 1/7!
    ps = fma(z, ps, 1.0 / 120.0);                       // 1/5!
    ps = fma(z, ps, -1.0 / 6.0);                        // 1/3!
    // cos r = 1 + z (-1/2! + z (1/4! - z (1/6! - ...)))
    double pc = -1.0 / 6402373705728000.0;              // 1/18!
    pc = fma(z, pc, 1.0 / 20922789888000.0);            // 1/16!
    pc = fma(z, pc, -1.0 / 87178291200.0);              // 1/14!
    pc = fma(z, pc, 1.0 / 479001600.0);                 // 1/12!
    pc = fma(z, pc, -1.0 / 3628800.0);                  // 1/10!
    pc = fma(z, pc, 1.0 / 40320.0);                     // 1/8!
    pc = fma(z, pc, -1.0 / 720.0);                      // 1/6!
    pc = fma(z, pc, 1.0 / 24.0);                        // 1/4!
    pc = fma(z, pc, -0.5);                              // 1/2!
    const double sr = fma(r * z, ps, r);
    const double cr = fma(z, pc, 1.0);
    const int q = (int)((long long)k & 3);
    const double a = (q & 1) ? cr : sr;   // sin x up to sign
    const double b = (q & 1) ? sr : cr;   // cos x up to sign
    s = (q & 2) ? -a : a;
    c = ((q + 1) & 2) ? -b : b;
}

}  // namespace rocattn
