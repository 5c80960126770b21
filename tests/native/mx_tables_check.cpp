// Host check of the matrix-core conversion's operand tables (no GPU).
//
// The library's host code is compiled in (api.cpp; the launchers and the no-alloc
// scratch are stubbed out by launch_stubs.h).  For the N = 2^16, 36 + 12 prime
// chain it builds the tables, then emulates what the
// conversion kernel computes from them: the int8 product of a constant tile (A) and
// the 7-bit digits of 32 coefficients' source values (B), in the lane layout of
// v_mfma_i32_32x32x32_i8 (lane l holds row l % 32 of A and column l % 32 of B with
// K slice 16*(l / 32) + i; register r of D in lane l is row 8*(r/4) + 4*(l/32) + r%4,
// column l % 32), the recombination sum_e D_e * W_e and the Montgomery reduction.
// Every result must equal sum_s y_s * c_s mod q_t with the fast-base-conversion
// constants recomputed here from the primes: c_s = prod of the other primes of the
// digit (ModUp) or of the special part (ModDown) mod q_t, times 2^-32 for the
// key-switch ModDown, whose sums carry that factor.  Source values past the digit's
// size are random (the kernel leaves stale values there; their constants are zero).
#include "../../rns_ckks_key_amd/csrc/api.cpp"

#include <cstdio>
#include <random>

#include "launch_stubs.h"

namespace {

uint32_t prod_mod_except(const std::vector<uint32_t>& primes, uint32_t skip, uint32_t q) {
  uint64_t v = 1;
  for (uint32_t p : primes)
    if (p != skip) v = v * (p % q) % q;
  return (uint32_t)v;
}

struct Checker {
  const Host& h;
  std::mt19937_64 rng{2024};
  long checked = 0, bad = 0;

  // tile: 2048 bytes for target pair (2mt, 2mt+1); tp(e): absolute prime of target e or
  // -1; cst(e, s): the plain constant for target e and source s; scale: extra factor
  void run(const uint8_t* tile, uint32_t mt, uint32_t ns, const std::function<int(uint32_t)>& tp,
           const std::function<uint32_t(uint32_t, uint32_t)>& cst, const std::function<uint32_t(uint32_t)>& scale) {
    uint32_t y[32][12];
    for (auto& row : y)
      for (auto& v : row) v = (uint32_t)rng();
    for (uint32_t l = 0; l < 64; ++l) {
      const uint32_t n = l & 31, e = 2 * mt + (l >> 5);
      int64_t d[16];
      for (uint32_t r = 0; r < 16; ++r) {
        const uint32_t m = 8 * (r / 4) + 4 * (l / 32) + r % 4;
        int64_t acc = 0;
        for (uint32_t kap = 0; kap < 2; ++kap)
          for (uint32_t hh = 0; hh < 2; ++hh)
            for (uint32_t i = 0; i < 16; ++i) {
              const int8_t av = (int8_t)tile[(kap * 64 + m + 32 * hh) * 16 + i];
              const uint32_t g = 16 * kap + i;
              const uint32_t bv = g < 30 ? (y[n][6 * hh + g / 5] >> (7 * (g % 5))) & 127u : 0u;
              acc += (int64_t)av * (int8_t)bv;
            }
        d[r] = acc;
      }
      const int t = tp(e);
      if (t < 0) continue;
      const uint32_t q = h.q[t];
      for (uint32_t r = 9; r < 16; ++r) bad += d[r] != 0;
      uint64_t x = 0;
      for (uint32_t r = 0; r < 9; ++r) {
        if (d[r] < 0 || d[r] >= (1 << 20)) ++bad;
        x += (uint64_t)d[r] * h.mx_w[(size_t)t * 12 + r];
      }
      const uint32_t xl = (uint32_t)x, xh = (uint32_t)(x >> 32);
      const uint32_t u = (uint32_t)(((uint64_t)(xl * h.qinv[t]) * q) >> 32);
      const uint32_t got = xh < u ? xh - u + q : xh - u;
      unsigned __int128 want = 0;
      for (uint32_t s = 0; s < ns; ++s) want += (unsigned __int128)y[n][s] * cst(e, s);
      const uint32_t w = mulmod((uint32_t)(want % q), scale(t), q);
      ++checked;
      if (got != w) {
        if (bad < 5) std::printf("tile %u lane %u target %u: got %u want %u\n", mt, l, e, got, w);
        ++bad;
      }
    }
  }
};

}  // namespace

int main() {
  Host h;
  h.log_n = 16;
  h.n = 1u << 16;
  h.L = 36;
  h.K = 12;
  h.dnum = 3;
  h.alpha = 12;
  h.q.resize(48);
  if (ckks_chain_primes(16, 32, 48, h.q.data()) != CKKS_OK) return std::printf("chain failed\n"), 1;
  build_tables(h);
  if (!h.mx_ok) return std::printf("tables not built\n"), 1;
  const uint32_t L = h.L, K = h.K, E = L + K, A = h.alpha, D = h.dnum, T = ckks::kMxTiles;
  std::vector<uint32_t> special(h.q.begin() + L, h.q.end());
  Checker ck{h};
  auto one = [](uint32_t) { return 1u; };
  for (uint32_t l : {36u, 35u, 25u, 24u, 13u, 12u, 2u, 1u}) {
    const uint32_t d = (l + A - 1) / A;
    for (uint32_t j = 0; j < d; ++j) {
      const uint32_t lo = j * A, ns = std::min(lo + A, l) - lo, nt = l + K - ns;
      std::vector<uint32_t> digit(h.q.begin() + lo, h.q.begin() + lo + ns);
      auto tp = [&](uint32_t e) -> int {
        if (e >= nt) return -1;
        const uint32_t dl = e < lo ? e : e + ns;
        return (int)(dl < l ? dl : L + (dl - l));
      };
      auto cst = [&](uint32_t e, uint32_t s) { return prod_mod_except(digit, digit[s], h.q[tp(e)]); };
      for (uint32_t mt = 0; 2 * mt < nt; ++mt)
        ck.run(&h.mx_up[(((size_t)l * D + j) * T + mt) * 2048], mt, ns, tp, cst, one);
    }
  }
  auto tp_md = [&](uint32_t e) -> int { return e < L ? (int)e : -1; };
  auto cst_md = [&](uint32_t e, uint32_t s) { return prod_mod_except(special, special[s], h.q[e]); };
  auto inv32 = [&](uint32_t t) { return invmod(r32(h.q[t]), h.q[t]); };
  for (uint32_t mt = 0; 2 * mt < L; ++mt) {
    ck.run(&h.mx_md_pl[(size_t)mt * 2048], mt, K, tp_md, cst_md, one);
    ck.run(&h.mx_md_ks[(size_t)mt * 2048], mt, K, tp_md, cst_md, inv32);
  }
  (void)E;
  if (ck.bad || ck.checked < 10000) return std::printf("FAIL: %ld of %ld\n", ck.bad, ck.checked), 1;
  std::printf("ok %ld\n", ck.checked);
  return 0;
}
