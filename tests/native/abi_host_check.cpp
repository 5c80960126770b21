// The library's host half under AddressSanitizer and UndefinedBehaviorSanitizer
// (no GPU).  api.cpp is compiled in with the launchers stubbed out, and every path
// that runs without a device is driven through the C-ABI:
//  - the prime chains of every workload shape, each checked for q = 1 mod 2N;
//  - host-only contexts on those chains (every table the device would get is built),
//    with each context's minimal 2N-th roots checked (psi^N = -1 mod q);
//  - rejected parameters of ckks_ctx_create;
//  - every entry point's argument checks, which must return their status before any
//    launch (a call that got through would reach a stub and return CKKS_EHIP).
// Prints "ok <checks>" when every expectation holds.
#include "../../rns_ckks_key_amd/csrc/api.cpp"

#include <cstdio>
#include <cstring>
#include <vector>

#include "launch_stubs.h"

namespace {

int checks = 0, fails = 0;

void expect(bool cond, const char* what, int line) {
  ++checks;
  if (!cond) {
    ++fails;
    std::printf("FAIL line %d: %s (last error: %s)\n", line, what, ckks_last_error());
  }
}
#define EXPECT(c) expect((c), #c, __LINE__)

uint32_t pow_mod(uint64_t b, uint64_t e, uint64_t q) {
  uint64_t r = 1;
  b %= q;
  while (e) {
    if (e & 1) r = r * b % q;
    b = b * b % q;
    e >>= 1;
  }
  return (uint32_t)r;
}

bool last_error_has(const char* s) { return std::strstr(ckks_last_error(), s) != nullptr; }

template <class T>
T* fake(uintptr_t a) {
  return reinterpret_cast<T*>(a);  // never dereferenced: every call below stops at its checks
}

struct Shape {
  uint32_t log_n, L, K, dnum, bits;
};

void check_context(const Shape& s) {
  const uint32_t E = s.L + s.K, n = 1u << s.log_n;
  std::vector<uint32_t> primes(E), roots(E);
  EXPECT(ckks_chain_primes(s.log_n, s.bits, E, primes.data()) == CKKS_OK);
  for (uint32_t i = 0; i < E; ++i) {
    EXPECT(primes[i] % (2 * n) == 1);
    EXPECT(s.bits == 32 || primes[i] < (1u << s.bits));
    if (i) EXPECT(primes[i] < primes[i - 1]);
  }
  ckks_ctx* ctx = nullptr;
  EXPECT(ckks_ctx_create(&ctx, s.log_n, s.L, s.K, s.dnum, primes.data(), 0) == CKKS_OK);
  if (!ctx) return;
  uint32_t nn = 0, nq = 0, np = 0, dnum = 0, alpha = 0, mb = 7;
  uint64_t ws = 1;
  EXPECT(ckks_ctx_info(ctx, &nn, &nq, &np, &dnum, &alpha, &mb, &ws, roots.data()) == CKKS_OK);
  EXPECT(nn == n && nq == s.L && np == s.K && dnum == s.dnum && mb == 0 && ws == 0);
  EXPECT(alpha == (s.L + s.dnum - 1) / s.dnum);
  for (uint32_t i = 0; i < E; ++i) EXPECT(pow_mod(roots[i], n, primes[i]) == primes[i] - 1);

  // every compute entry point stops at its checks on a host-only context
  const uint32_t L = s.L;
  uint32_t* ct = fake<uint32_t>(0x1000);
  uint32_t* far = fake<uint32_t>(0x40000000);
  const uint32_t* kb = fake<const uint32_t>(0x70000000);
  uint8_t seed[32] = {};
  EXPECT(ckks_keyswitch(ctx, ct, 0, kb, seed, nullptr, 5, far, 1, nullptr) == CKKS_ERANGE);
  EXPECT(ckks_keyswitch(ctx, ct, L + 1, kb, seed, nullptr, 5, far, 1, nullptr) == CKKS_ERANGE);
  EXPECT(ckks_keyswitch(ctx, ct, L, kb, seed, nullptr, 4, far, 1, nullptr) == CKKS_ERANGE);
  EXPECT(ckks_keyswitch(ctx, ct, L, kb, seed, nullptr, 2 * n + 1, far, 1, nullptr) == CKKS_ERANGE);
  EXPECT(ckks_keyswitch(ctx, ct, L, kb, seed, nullptr, 5, far, 0, nullptr) == CKKS_ERANGE);
  EXPECT(ckks_keyswitch(ctx, nullptr, L, kb, seed, nullptr, 5, far, 1, nullptr) == CKKS_EINVAL);
  EXPECT(ckks_keyswitch(ctx, ct, L, kb, nullptr, nullptr, 5, far, 1, nullptr) == CKKS_EINVAL);
  EXPECT(ckks_keyswitch(ctx, ct, L, kb, seed, nullptr, 5, ct + 1, 1, nullptr) == CKKS_EINVAL);
  EXPECT(last_error_has("overlaps ct"));
  EXPECT(ckks_keyswitch(ctx, ct, L, kb, seed, nullptr, 5, far, 1, nullptr) == CKKS_EINVAL);
  EXPECT(last_error_has("host-only"));
  EXPECT(ckks_keyswitch_noalloc(ctx, ct, L, kb, seed, nullptr, 5, far, 0, nullptr) == CKKS_ERANGE);
  EXPECT(ckks_ntt_fwd(ctx, ct, E, 1, 1, nullptr) == CKKS_ERANGE);
  EXPECT(ckks_ntt_fwd(ctx, nullptr, 0, 1, 1, nullptr) == CKKS_EINVAL);
  EXPECT(ckks_ntt_inv(ctx, ct, 0, 0, 1, nullptr) == CKKS_ERANGE);
  EXPECT(ckks_ntt_fwd(ctx, ct, 0, E, 1, nullptr) == CKKS_EINVAL && last_error_has("host-only"));
  EXPECT(ckks_modup(ctx, ct, L + 1, far, 1, nullptr) == CKKS_ERANGE);
  EXPECT(ckks_modup(ctx, ct, L, ct + n, 1, nullptr) == CKKS_EINVAL && last_error_has("overlaps"));
  EXPECT(ckks_moddown(ctx, ct, 0, far, 1, nullptr) == CKKS_ERANGE);
  EXPECT(ckks_moddown(ctx, ct, L, far, 1, nullptr) == CKKS_EINVAL && last_error_has("host-only"));
  EXPECT(ckks_rescale(ctx, ct, 1, far, 1, nullptr) == CKKS_ERANGE);
  EXPECT(ckks_rescale(ctx, ct, L, ct, 1, nullptr) == CKKS_EINVAL && last_error_has("overlaps"));
  EXPECT(ckks_mul_relin_rescale(ctx, ct, ct, 1, kb, seed, nullptr, far, 1, nullptr) == CKKS_ERANGE);
  EXPECT(ckks_mul_relin_rescale(ctx, ct, ct, L, kb, nullptr, nullptr, far, 1, nullptr) == CKKS_EINVAL);
  EXPECT(ckks_expand_a(ctx, nullptr, far, nullptr) == CKKS_EINVAL);

  const uint32_t* keys[2] = {kb, kb};
  uint8_t seeds[64] = {};  // two keys' seeds, 32 bytes each
  uint32_t gal[2] = {5, 25};
  EXPECT(ckks_keyswitch_hoisted(ctx, ct, L, 0, keys, seeds, nullptr, gal, far, nullptr) == CKKS_ERANGE);
  gal[1] = 6;
  EXPECT(ckks_keyswitch_hoisted(ctx, ct, L, 2, keys, seeds, nullptr, gal, far, nullptr) == CKKS_ERANGE);
  gal[1] = 25;
  EXPECT(ckks_keyswitch_hoisted(ctx, ct, L, 2, keys, seeds, nullptr, gal, far, nullptr) == CKKS_EINVAL);
  EXPECT(last_error_has("host-only"));

  ckks_ks_item items[2] = {};
  const uint64_t span = 2ull * L * n;  // words of one ciphertext
  for (int i = 0; i < 2; ++i) {
    items[i].ct = ct + 2 * i * span;
    items[i].out = far + 2 * i * span;
    items[i].key_b = kb;
    items[i].level = L;
    items[i].galois_elt = 5;
  }
  EXPECT(ckks_keyswitch_multi(ctx, 0, nullptr, nullptr) == CKKS_OK);
  EXPECT(ckks_keyswitch_multi(ctx, 2, nullptr, nullptr) == CKKS_EINVAL);
  items[1].level = L + 1;
  EXPECT(ckks_keyswitch_multi(ctx, 2, items, nullptr) == CKKS_ERANGE && last_error_has("item 1"));
  items[1].level = L;
  items[1].out = far + span / 2;  // overlaps item 0's output
  EXPECT(ckks_keyswitch_multi(ctx, 2, items, nullptr) == CKKS_EINVAL);
  items[1].out = far + 2 * span;
  EXPECT(ckks_keyswitch_multi(ctx, 2, items, nullptr) == CKKS_EINVAL && last_error_has("host-only"));

  ckks_rot_key rk[2] = {};
  rk[0].key_b = rk[1].key_b = kb;
  rk[0].galois_elt = 5;
  rk[1].galois_elt = 25;
  const uint32_t* diags = fake<const uint32_t>(0x7000);
  EXPECT(ckks_linear_transform_bsgs(ctx, ct, L, 0, 2, rk, rk, diags, far, nullptr) == CKKS_ERANGE);
  EXPECT(ckks_linear_transform_bsgs(ctx, ct, L, 17, 2, rk, rk, diags, far, nullptr) == CKKS_ERANGE);
  EXPECT(ckks_linear_transform_bsgs(ctx, ct, L, 2, 9, rk, rk, diags, far, nullptr) == CKKS_ERANGE);
  EXPECT(ckks_linear_transform_bsgs(ctx, ct, L, 2, 2, rk, rk, nullptr, far, nullptr) == CKKS_EINVAL);
  EXPECT(ckks_linear_transform_bsgs(ctx, ct, L, 2, 2, rk, rk, diags, far, nullptr) == CKKS_EINVAL);
  EXPECT(last_error_has("host-only"));

  EXPECT(ckks_ctx_set_regen_blocks(ctx, 63) == CKKS_ERANGE);
  EXPECT(ckks_ctx_set_regen_blocks(ctx, 64) == CKKS_OK);
  EXPECT(ckks_ctx_set_fused(ctx, 0) == CKKS_EINVAL);
  double ms[8];
  uint32_t launches[8];
  EXPECT(ckks_profile_read(ctx, ms, launches, 8) == CKKS_EINVAL);
  ckks_ctx_destroy(ctx);
}

}  // namespace

int main() {
  // the five workload shapes' chains, a six-prime-digit chain, and the smaller ring
  const Shape shapes[] = {{12, 4, 2, 2, 30}, {16, 36, 12, 3, 32}, {16, 36, 6, 6, 32}, {15, 20, 7, 3, 32},
                          {13, 9, 4, 3, 31}, {14, 13, 5, 3, 32}};
  for (const Shape& s : shapes) check_context(s);

  // rejected parameters
  std::vector<uint32_t> qs(6);
  EXPECT(ckks_chain_primes(12, 30, 6, qs.data()) == CKKS_OK);
  ckks_ctx* ctx = nullptr;
  EXPECT(ckks_ctx_create(&ctx, 12, 4, 2, 2, nullptr, 0) == CKKS_EINVAL);
  EXPECT(ckks_ctx_create(nullptr, 12, 4, 2, 2, qs.data(), 0) == CKKS_EINVAL);
  EXPECT(ckks_ctx_create(&ctx, 17, 4, 2, 2, qs.data(), 0) == CKKS_EUNSUPPORTED);
  std::vector<uint32_t> bad = qs;
  bad[2] = 8193;  // 1 mod 2N but 3 * 2731
  EXPECT(ckks_ctx_create(&ctx, 12, 4, 2, 2, bad.data(), 0) == CKKS_ERANGE);
  bad = qs;
  bad[5] = qs[0];  // repeated prime
  EXPECT(ckks_ctx_create(&ctx, 12, 4, 2, 2, bad.data(), 0) == CKKS_ERANGE);
  EXPECT(ckks_ctx_create(&ctx, 12, 4, 1, 2, qs.data(), 0) == CKKS_ERANGE);  // special modulus < a digit
  EXPECT(ckks_ctx_create(&ctx, 12, 4, 2, 0, qs.data(), 0) == CKKS_ERANGE);
  EXPECT(ckks_chain_primes(12, 19, 4, qs.data()) == CKKS_ERANGE);
  EXPECT(ckks_chain_primes(12, 30, 4, nullptr) == CKKS_EINVAL);
  EXPECT(ckks_keyswitch(nullptr, nullptr, 1, nullptr, nullptr, nullptr, 5, nullptr, 1, nullptr) == CKKS_EINVAL);
  ckks_ctx_destroy(nullptr);

  if (fails) {
    std::printf("%d of %d checks failed\n", fails, checks);
    return 1;
  }
  std::printf("ok %d\n", checks);
  return 0;
}
