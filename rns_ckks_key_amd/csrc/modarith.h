// 32-bit modular arithmetic for odd primes q < 2^32 (gfx950 device code).
//
// Residues are canonical, in [0, q), at every kernel boundary.  The primes of a
// 2^16-point chain all exceed 2^31, so a + b can carry out of 32 bits and the
// lazy [0, 2q) forms do not fit a word: add_mod and sub_mod reduce fully.  The
// forward transforms instead carry any 32-bit representative (lazy_add,
// lazy_sub) and make it canonical once at the end (canon).  Multiplication by a constant w uses Montgomery's REDC with R = 2^32
// on a precomputed pair (w~ = w*R mod q, w~ * q^-1 mod R); a sum of up to ~2^31
// 64-bit products is kept exactly in three words and brought back to [0, q) by
// two word-steps of REDC (result carries a factor R^-2 that callers fold into a
// later constant).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ckks {

__host__ __device__ __forceinline__ uint32_t umulhi32(uint32_t a, uint32_t b) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __umulhi(a, b);
#else
  return (uint32_t)(((uint64_t)a * b) >> 32);
#endif
}

struct Mod {
  uint32_t q;     // the prime
  uint32_t qinv;  // q^-1 mod 2^32
};

// a - b mod q for a, b in [0, q): the borrow of the 32-bit subtraction selects a - b + q.
__host__ __device__ __forceinline__ uint32_t sub_mod(uint32_t a, uint32_t b, uint32_t q) {
  uint32_t d;
  const bool borrow = __builtin_sub_overflow(a, b, &d);
  return borrow ? d + q : d;
}

// a + b mod q for a, b in [0, q): a + b when a < q - b, else a - (q - b) (no 33-bit sum needed).
__host__ __device__ __forceinline__ uint32_t add_mod(uint32_t a, uint32_t b, uint32_t q) {
  uint32_t d;
  const bool borrow = __builtin_sub_overflow(a, q - b, &d);
  return borrow ? a + b : d;
}

// Lazy forms, used inside the forward transforms: a value there is any 32-bit
// representative of its residue (possibly >= q).  For t in [0, q), a + t and a - t
// stay in [0, 2^32) without a comparison with q: a carry out of a + t is taken back
// by adding 2^32 - q (giving a + t - q), a borrow of a - t by subtracting it (giving
// a - t + q).  Valid for every q < 2^32.
__host__ __device__ __forceinline__ uint32_t lazy_add(uint32_t a, uint32_t t, uint32_t q) {
  uint32_t s;
  const bool carry = __builtin_add_overflow(a, t, &s);
  return carry ? s + (0u - q) : s;
}
__host__ __device__ __forceinline__ uint32_t lazy_sub(uint32_t a, uint32_t t, uint32_t q) {
  uint32_t d;
  const bool borrow = __builtin_sub_overflow(a, t, &d);
  return borrow ? d - (0u - q) : d;
}

// a * w mod q, where (wm, wmq) = (w*2^32 mod q, wm*qinv mod 2^32); any a < 2^32.
// REDC(a*wm) with the borrow form: (a*wm - m*q)/2^32 = hi(a*wm) - hi(m*q), m = lo(a*wm)*qinv.
__host__ __device__ __forceinline__ uint32_t mul_const(uint32_t a, uint32_t wm, uint32_t wmq, uint32_t q) {
  uint32_t hi = umulhi32(a, wm);
  uint32_t m = a * wmq;
  uint32_t t = umulhi32(m, q);
  return sub_mod(hi, t, q);
}

// a * b * 2^-32 mod q for b < q and any a < 2^32 (REDC of the full product, subtract
// form; a * b < q * 2^32 keeps both high words below q).
__host__ __device__ __forceinline__ uint32_t mont_mul(uint32_t a, uint32_t b, Mod md) {
  const uint32_t lo = a * b;
  const uint32_t hi = umulhi32(a, b);
  const uint32_t t = umulhi32(lo * md.qinv, md.q);
  return sub_mod(hi, t, md.q);
}

// a - b*c*2^-32 (mod q) for any 32-bit a and b and c < q, as a 32-bit representative
// (a lazy value).  The Montgomery product's two reduction cases fold into the
// subtraction's: with u = t - hi (hi - t is the unreduced product, in (-q, q)), the
// word sum a + u is corrected by +q if u wrapped and by -q (adding nq = 2^32 - q)
// if the sum carried.  nq is an argument so that a caller can keep the compiler
// from turning the second correction into a subtraction (three-operand add).
__host__ __device__ __forceinline__ uint32_t lazy_sub_mont(uint32_t a, uint32_t b, uint32_t c, Mod md,
                                                           uint32_t nq) {
  const uint32_t lo = b * c;
  const uint32_t hi = umulhi32(b, c);
  const uint32_t t = umulhi32(lo * md.qinv, md.q);
  uint32_t u, s;
  const bool neg = __builtin_sub_overflow(t, hi, &u);
  const bool carry = __builtin_add_overflow(a, u, &s);
  return s + (neg ? md.q : 0u) + (carry ? nq : 0u);
}

// a + b*c*2^-32 (mod q), the same way: u = hi - t, corrected as in lazy_sub_mont.
__host__ __device__ __forceinline__ uint32_t lazy_add_mont(uint32_t a, uint32_t b, uint32_t c, Mod md,
                                                           uint32_t nq) {
  const uint32_t lo = b * c;
  const uint32_t hi = umulhi32(b, c);
  const uint32_t t = umulhi32(lo * md.qinv, md.q);
  uint32_t u, s;
  const bool neg = __builtin_sub_overflow(hi, t, &u);
  const bool carry = __builtin_add_overflow(a, u, &s);
  return s + (neg ? md.q : 0u) + (carry ? nq : 0u);
}

// Canonical residue of a 32-bit representative x.  For q > 2^31, x < 2q and one
// conditional subtraction does it (min(x, x - q): x - q wraps above x when x < q);
// otherwise x is multiplied by one = (2^32 mod q, companion), i.e. reduced by REDC.
__host__ __device__ __forceinline__ uint32_t canon(uint32_t x, uint32_t q, uint32_t one_wm, uint32_t one_wmq) {
  if (q >> 31) {
    const uint32_t d = x - q;
    return d < x ? d : x;
  }
  return mul_const(x, one_wm, one_wmq, q);
}

// Companion of a Montgomery-form constant: wm * q^-1 mod 2^32.
__host__ __device__ __forceinline__ uint32_t companion(uint32_t wm, uint32_t qinv) { return wm * qinv; }

// Exact three-word accumulator of 64-bit products.
struct Acc96 {
  uint64_t lo;  // low 64 bits
  uint32_t hi;  // carries out of the low 64 bits
};

__host__ __device__ __forceinline__ void acc_zero(Acc96& a) {
  a.lo = 0;
  a.hi = 0;
}

__host__ __device__ __forceinline__ void acc_mac(Acc96& a, uint32_t x, uint32_t y) {
  uint64_t p = (uint64_t)x * (uint64_t)y;
  uint64_t s = a.lo + p;
  a.hi += (s < p) ? 1u : 0u;
  a.lo = s;
}

// S * 2^-64 mod q for the accumulated S = hi*2^64 + lo, valid while hi + 2 < q.
// Two word-steps of REDC in the subtract form: with m = w*q^-1 mod 2^32 for the
// low word w, S - m*q has a zero low word, so (S - m*q)/2^32 = (S >> 32) - hi(m*q).
// After the first step the value lies in (-q, (hi+1)*2^32); after the second in
// [-q, hi+1], so one conditional add of q makes it canonical.
__host__ __device__ __forceinline__ uint32_t acc_redc2(const Acc96& a, Mod md) {
  const uint32_t a1 = umulhi32((uint32_t)a.lo * md.qinv, md.q);
  const uint64_t s1 = (((uint64_t)a.hi << 32) | (a.lo >> 32)) - a1;  // two's complement if negative
  const int32_t h1 = (int32_t)(uint32_t)(s1 >> 32);
  const uint32_t a2 = umulhi32((uint32_t)s1 * md.qinv, md.q);
  const int64_t r = (int64_t)h1 - (int64_t)a2;
  return (uint32_t)(r < 0 ? r + md.q : r);
}

}  // namespace ckks
