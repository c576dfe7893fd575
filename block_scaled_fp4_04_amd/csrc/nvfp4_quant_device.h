// nvfp4_quant_device.h -- device functions of the NVFP4 quantisation rule,
// shared by the quantiser kernel and the GEMM kernel that quantises its
// activations on the fly (so that both produce the same bytes).
//
// Per 16-element block (the format of "Peeling the Kernel Onion", section
// "The Benchmark Design"):
//   scale byte = E4M3 value nearest to fp32(amax / 6), ties to the even byte,
//                saturating at 448;
//   code       = E2M1 magnitude nearest to fp32(x / scale), ties to the even
//                code, saturating at 6, with the sign bit of x; a block whose
//                scale is 0 keeps only the sign bits.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

// E4M3 byte (0x00..0x7E) nearest to t >= 0, ties to the even byte,
// saturating at 448.  E4M3: subnormals f * 2^-9 (bytes 0..7), normals
// (1 + f/8) * 2^(e-7) (byte (e << 3) | f, e = 1..15, largest finite 0x7E).
// Branch-free: both ranges are computed and the right one selected.
__device__ __forceinline__ uint32_t e4m3_nearest(float t) {
    // below 2^-6 the spacing is 2^-9: exact scaling, round to nearest even
    // (a result of 8 is byte 0x08 = 2^-6)
    const uint32_t sub = (uint32_t)__builtin_rintf(__builtin_fminf(t, 0.015625f) * 512.0f);
    const uint32_t bits = __builtin_bit_cast(uint32_t, t);
    const uint32_t e = ((bits >> 23) & 0xFFu) - 120u;      // E4M3 exponent field
    const uint32_t mant = bits & 0x7FFFFFu;
    const uint32_t f = mant >> 20;                          // 3 kept mantissa bits
    const uint32_t rest = mant & 0xFFFFFu;                  // 20 dropped bits
    const uint32_t up = (rest > 0x80000u || (rest == 0x80000u && (f & 1u))) ? 1u : 0u;
    const uint32_t normal = ((e << 3) | f) + up;            // a carry out of f bumps e
    const uint32_t r = t < 0.015625f ? sub : normal;
    return t < 448.0f ? r : 0x7Eu;                          // at or past 448 (and NaN)
}

// Value of a non-negative E4M3 byte as fp32 (exact).
__device__ __forceinline__ float e4m3_value(uint32_t b) {
    const uint32_t e = b >> 3, f = b & 7u;
    const float sub = (float)f * 0.001953125f;                          // f * 2^-9
    const float nrm = __builtin_bit_cast(float, ((e + 120u) << 23) | (f << 20));
    return e == 0 ? sub : nrm;
}

// E2M1 magnitude code of y = fp32(ax / s) for ax >= 0, s > 0 an E4M3
// value: nearest E2M1 magnitude, ties to the even code, past 6 saturating.
// The code counts the rounding boundaries T = 0.25, 0.75, 1.25, 1.75, 2.5,
// 3.5, 5 that y passes: y > T where the tie at T goes down (to the even
// code below), y >= T where it goes up.  These are decided exactly without
// dividing: with P = T * s (exact in fp32: T has at most 3 significant bits,
// s at most 4),
//   y > T   <=>  ax / s > T + u/2  <=>  ax > P     (u = ulp of T in fp32)
//   y >= T  <=>  ax / s >= T - u/2  <=>  ax >= P
// because (u/2) * s is smaller than the fp32 spacing at P (at most 3/4 of
// it), so the quotient's rounding boundary lies strictly between P and the
// neighbouring fp32 value, where no ax can fall; and P is never a power of
// two for the ">=" boundaries (0.75, 1.75 and 3.5 have a factor 3 or 7), so
// the spacing below P is the same.  Each comparison's bit is the sign of a
// comparison of fp32 values, done on their bit patterns.
// The seven boundaries as fp32 bit patterns (non-negative floats order like
// their bits), the ">=" ones minus 1 so that every test is "bits(ax) > b".
struct E2m1Search {
    uint32_t p0, p1m, p2, p3m, p4, p5m, p6;
};
__device__ __forceinline__ uint32_t fbits(float x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ E2m1Search e2m1_search(float s) {
    E2m1Search q{fbits(0.25f * s), fbits(0.75f * s) - 1u, fbits(1.25f * s),
                 fbits(1.75f * s) - 1u, fbits(2.5f * s), fbits(3.5f * s) - 1u, fbits(5.0f * s)};
    // opaque to the optimiser: otherwise it moves the selects of the search
    // in front of these multiplications and redoes them for every element
    asm volatile("" : "+v"(q.p0), "+v"(q.p1m), "+v"(q.p2), "+v"(q.p3m), "+v"(q.p4), "+v"(q.p5m),
                 "+v"(q.p6));
    return q;
}
// The code is the number of boundaries below A (A and the boundaries are
// fp32 bit patterns of non-negative values, so they order as integers, and
// the boundaries increase -- but for a zero scale, whose codes are masked
// off).  A three-level binary search finds it: A against the middle
// boundary, then against the middle of the half that selects, then against
// the one boundary left, the three bits summed (about 10 instructions per
// element; counting all seven boundaries through a borrow chain took 14:
// 16384 x 8192 bfloat16 rows 85 -> 80 us, fp32 rows 136 -> 134 us).
__device__ __forceinline__ uint32_t e2m1_code(uint32_t A, const E2m1Search& q) {
    const bool s0 = A > q.p3m;
    const uint32_t mid = s0 ? q.p5m : q.p1m;
    const uint32_t lo = s0 ? q.p4 : q.p0, hi = s0 ? q.p6 : q.p2;
    const bool s1 = A > mid;
    const uint32_t last = s1 ? hi : lo;
    return (s0 ? 4u : 0u) + (s1 ? 2u : 0u) + (A > last ? 1u : 0u);
}

// Code word (8 codes, element i in bits 4i+3:4i) of 8 values of one block
// whose scale search is q (keep: 7, or 0 for a block whose scale is 0).
__device__ __forceinline__ uint32_t e2m1_word(const float (&v)[8], const E2m1Search& q,
                                              uint32_t keep) {
    uint32_t w = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t b = fbits(v[i]);
        w |= (((b >> 28) & 8u) | (e2m1_code(b & 0x7FFFFFFFu, q) & keep)) << (4 * i);
    }
    return w;
}

}  // namespace nvfp4
