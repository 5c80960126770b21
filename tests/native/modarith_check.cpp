// Host-side check of the library's modular-arithmetic core (modarith.h compiled
// for the CPU) against 128-bit integer arithmetic.  Prints "ok <count>" or the
// first failing case and exits non-zero.
#include <cstdio>
#include <cstdint>
#include <random>
#include "../../rns_ckks_key_amd/csrc/modarith.h"

using namespace ckks;
typedef unsigned __int128 u128;

static uint32_t inv2_32(uint32_t q) { uint32_t x = q; for (int i = 0; i < 5; ++i) x *= 2 - q * x; return x; }

int main() {
  std::mt19937_64 rng(12345);
  const uint32_t primes[] = {4293918721u, 4233756673u, 1073692673u, 1073479681u, 65537u, 4294967291u, 3221225473u};
  long count = 0;
  for (uint32_t q : primes) {
    const uint32_t qinv = inv2_32(q);
    if (q * qinv != 1u) { printf("bad qinv %u\n", q); return 1; }
    const Mod md{q, qinv};
    const uint32_t edge[] = {0u, 1u, 2u, q - 1, q - 2, q / 2, q / 2 + 1};
    for (int it = 0; it < 200000; ++it) {
      uint32_t a = it < 49 ? edge[it % 7] : (uint32_t)(rng() % q);
      uint32_t b = it < 49 ? edge[it / 7] : (uint32_t)(rng() % q);
      if (add_mod(a, b, q) != (uint32_t)(((uint64_t)a + b) % q)) { printf("add %u %u %u\n", a, b, q); return 1; }
      if (sub_mod(a, b, q) != (uint32_t)(((uint64_t)a + q - b) % q)) { printf("sub %u %u %u\n", a, b, q); return 1; }
      // lazy add/subtract of a canonical t to any 32-bit representative, and canonicalisation
      {
        const uint32_t x = (uint32_t)rng(), t = b;
        const uint32_t one_wm = (uint32_t)((((uint64_t)1) << 32) % q);
        if ((uint64_t)lazy_add(x, t, q) % q != ((uint64_t)x + t) % q) { printf("lazy_add %u %u %u\n", x, t, q); return 1; }
        if ((uint64_t)lazy_sub(x, t, q) % q != ((uint64_t)x % q + q - t) % q) { printf("lazy_sub %u %u %u\n", x, t, q); return 1; }
        if (canon(x, q, one_wm, one_wm * qinv) != x % q) { printf("canon %u %u\n", x, q); return 1; }
        if (canon(a, q, one_wm, one_wm * qinv) != a) { printf("canon canonical %u %u\n", a, q); return 1; }
        // Montgomery product with a full 32-bit left operand: x * t * 2^-32 mod q
        const uint32_t mm = mont_mul(x, t, md);
        if (mm >= q || (u128)mm * (((u128)1 << 32) % q) % q != (u128)x * t % q) { printf("mont_mul %u %u %u\n", x, t, q); return 1; }
        // the accumulation step of the final inner-product pass, x - y * t * 2^-32 for any
        // 32-bit x and y: ls * 2^32 = x * 2^32 - y * t (mod q), word edges included
        const uint32_t wedge[] = {0u, 1u, q - 1, q, q + 1, 0xffffffffu, 0x80000000u};
        const uint32_t xs = it < 49 ? wedge[it % 7] : x, ys = it < 49 ? wedge[it / 7] : (uint32_t)rng();
        const uint32_t ls = lazy_sub_mont(xs, ys, t, md, 0u - q);
        const u128 r32 = ((u128)1 << 32) % q;
        if (((u128)ls * r32 + (u128)ys * t) % q != (u128)xs * r32 % q) {
          printf("lazy_sub_mont %u %u %u %u\n", xs, ys, t, q);
          return 1;
        }
        const uint32_t la = lazy_add_mont(xs, ys, t, md, 0u - q);  // la * 2^32 = x * 2^32 + y * t
        if (((u128)la * r32) % q != ((u128)xs * r32 + (u128)ys * t) % q) {
          printf("lazy_add_mont %u %u %u %u\n", xs, ys, t, q);
          return 1;
        }
        count += 6;
      }
      // constant multiply, any a < 2^32
      uint32_t araw = it & 1 ? (uint32_t)rng() : a;
      uint32_t wm = (uint32_t)(((uint64_t)b << 32) % q);
      if (mul_const(araw, wm, wm * qinv, q) != (uint32_t)((uint64_t)araw % q * b % q)) {
        printf("mul_const %u %u %u\n", araw, b, q); return 1;
      }
      // accumulate up to 40 products and reduce: result * 2^64 = S mod q
      int nt = 1 + (int)(rng() % 40);
      Acc96 acc; acc_zero(acc);
      u128 s = 0;
      for (int k = 0; k < nt; ++k) {
        uint32_t x = it < 49 ? q - 1 : (uint32_t)(rng() % q), y = it < 49 ? q - 1 : (uint32_t)(rng() % q);
        if (k == 0 && it % 5 == 0) { x = (uint32_t)rng(); y = (uint32_t)rng(); }  // full 32-bit operands
        acc_mac(acc, x, y);
        s += (u128)x * y;
      }
      u128 got = acc_redc2(acc, md);
      u128 r64 = ((u128)1 << 64) % q;
      if (got >= q || (got * r64) % q != s % q) { printf("redc2 q=%u n=%d\n", q, nt); return 1; }
      count += 4;
    }
  }
  printf("ok %ld\n", count);
  return 0;
}
