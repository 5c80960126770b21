// C-ABI of the key-switching library: argument checks, host precompute of the
// constant tables, device workspace, and the launch sequence of each call.
//
// Launch sequence of one key-switch of `batch` ciphertexts at level l (all on
// the caller's stream, no host synchronisation):
//   1. k_row  (inverse)   c1 -> rowtmp           row half of INTT(c1)
//   2. k_conv (ModUp)     rowtmp -> ext          column INTT, scale, conversion, column NTT
//   3. k_ip   (special)   ext, key -> tmpP       row NTT, sigma_g, inner product, row INTT
//   4. k_conv (ModDown)   tmpP -> conv           column INTT, scale, P->Q conversion, column NTT
//   5. k_ip   (final)     ext, c1, c0, conv, key -> out
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <iterator>
#include <string>
#include <vector>

#include "../../include/ckks_ks.h"
#include "ckks_internal.h"

using ckks::DevTables;

namespace {

thread_local std::string g_err;

ckks_status fail(ckks_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
ckks_status fail(ckks_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

ckks_status ok() {
  g_err.clear();
  return CKKS_OK;
}

// ---------------------------------------------------------------- number theory (host)

uint32_t mulmod(uint32_t a, uint32_t b, uint32_t m) { return (uint32_t)((uint64_t)a * b % m); }

uint32_t powmod(uint32_t b, uint64_t e, uint32_t m) {
  uint64_t r = 1 % m, x = b % m;
  while (e) {
    if (e & 1) r = r * x % m;
    x = x * x % m;
    e >>= 1;
  }
  return (uint32_t)r;
}

uint32_t invmod(uint32_t a, uint32_t p) { return powmod(a, p - 2, p); }  // p prime

// Deterministic Miller-Rabin for n < 2^32 with bases 2, 7, 61.
bool is_prime32(uint32_t n) {
  if (n < 2) return false;
  for (uint32_t p : {2u, 3u, 5u, 7u, 11u, 13u, 61u})
    if (n % p == 0) return n == p;
  uint32_t d = n - 1, s = 0;
  while (!(d & 1)) { d >>= 1; ++s; }
  for (uint32_t a : {2u, 7u, 61u}) {
    uint64_t x = powmod(a, d, n);
    if (x == 1 || x == n - 1) continue;
    bool comp = true;
    for (uint32_t r = 1; r < s; ++r) {
      x = x * x % n;
      if (x == n - 1) { comp = false; break; }
    }
    if (comp) return false;
  }
  return true;
}

// Smallest x with x^n = -1 mod q: the minimum over all primitive 2n-th roots (odd powers of one).
uint32_t min_root(uint32_t q, uint32_t n) {
  uint32_t w = 0;
  for (uint32_t h = 2;; ++h) {
    w = powmod(h, (q - 1) / (2 * (uint64_t)n), q);
    if (powmod(w, n, q) == q - 1) break;
  }
  const uint32_t w2 = mulmod(w, w, q);
  uint32_t best = w, x = w;
  for (uint32_t k = 1; k < n; ++k) {
    x = mulmod(x, w2, q);
    best = std::min(best, x);
  }
  return best;
}

uint32_t brv(uint32_t x, uint32_t bits) {
  uint32_t r = 0;
  for (uint32_t i = 0; i < bits; ++i) { r = (r << 1) | (x & 1); x >>= 1; }
  return r;
}

uint32_t inv2_32(uint32_t q) {  // q^-1 mod 2^32 by Newton iteration
  uint32_t x = q;
  for (int i = 0; i < 5; ++i) x *= 2 - q * x;
  return x;
}

uint2 mont(uint32_t w, uint32_t q) {  // (w*2^32 mod q, companion)
  uint32_t wm = (uint32_t)(((uint64_t)(w % q) << 32) % q);
  return make_uint2(wm, wm * inv2_32(q));
}

uint32_t r32(uint32_t q) { return (uint32_t)((1ull << 32) % q); }  // 2^32 mod q

uint32_t r64(uint32_t q) {  // 2^64 mod q
  uint32_t r32 = (uint32_t)((1ull << 32) % q);
  return mulmod(r32, r32, q);
}

struct Host {
  uint32_t log_n = 0, n = 0, L = 0, K = 0, dnum = 0, alpha = 0;
  std::vector<uint32_t> q, qinv, psi;
  std::vector<uint32_t> tw, itw;
  std::vector<uint2> ninv, mu_scale, md_scale_ks, md_scale_pl, md_fin_ks, md_fin_pl, one, r2, rs_inv, p_mod;
  std::vector<uint32_t> mu_conv, md_conv, md_conv64, bound, r64tab;
  // matrix-core conversion operands (ring 2^16 with 9..12 sources per conversion)
  bool mx_ok = false;
  std::vector<uint32_t> mx_w;                     // [L+K][12]
  std::vector<uint8_t> mx_up, mx_md_ks, mx_md_pl; // tiles of 2048 bytes
};

// One matrix-core operand tile (two K steps x 64 lanes x 16 bytes) for the target
// pair (2mt, 2mt+1) of a conversion.  Lane l holds row m = l & 31, i.e. pair member
// p = (m >> 2) & 1 and digit position e = 4(m >> 3) + (m & 3), and K half h = l >> 5.
// Byte i of K step kappa is g = 16 kappa + i: source s = 6h + g/5, source digit
// a = g % 5 (g < 30).  Its value is 7-bit digit e - a of the constant cst(p, s) when
// 0 <= e - a <= 4, else 0 (cst returns 0 for a missing target).
template <class F>
void mx_tile(uint8_t* out, uint32_t ns, F cst) {
  for (uint32_t kap = 0; kap < 2; ++kap)
    for (uint32_t l = 0; l < 64; ++l) {
      const uint32_t m = l & 31, h = l >> 5, p = (m >> 2) & 1, e = 4 * (m >> 3) + (m & 3);
      for (uint32_t i = 0; i < 16; ++i) {
        const uint32_t g = 16 * kap + i;
        uint8_t b = 0;
        if (g < 30) {
          const uint32_t src = 6 * h + g / 5, a = g % 5;
          if (src < ns && e >= a && e - a <= 4) b = (uint8_t)((cst(p, src) >> (7 * (e - a))) & 127u);
        }
        out[(kap * 64 + l) * 16 + i] = b;
      }
    }
}

// Operand tables of the matrix-core conversion.  The vector path multiplies by
// constants c' carrying 2^64 and reduces by 2^-64; the effective constant is
// c' * 2^-64 mod q, whose digits go into the tiles, so both paths give the same residue.
void build_mx_tables(Host& h) {
  const uint32_t L = h.L, K = h.K, E = L + K, A = h.alpha, D = h.dnum, T = ckks::kMxTiles;
  h.mx_ok = h.log_n == 16 && A >= 9 && A <= 12 && K >= 9 && K <= 12 && E <= 2 * T;
  if (!h.mx_ok) return;
  std::vector<uint32_t> inv64(E);
  for (uint32_t t = 0; t < E; ++t) inv64[t] = invmod(r64(h.q[t]), h.q[t]);
  h.mx_w.assign((size_t)E * 12, 0);
  for (uint32_t t = 0; t < E; ++t)
    for (uint32_t e = 0; e < 9; ++e) h.mx_w[(size_t)t * 12 + e] = mulmod(powmod(2, 7 * e, h.q[t]), r32(h.q[t]), h.q[t]);
  const size_t tile = 2048;
  h.mx_up.assign((size_t)(L + 1) * D * T * tile, 0);
  for (uint32_t l = 1; l <= L; ++l) {
    const uint32_t d = (l + A - 1) / A;
    for (uint32_t j = 0; j < d; ++j) {
      const uint32_t lo = j * A, ns = std::min(lo + A, l) - lo, nt = l + K - ns;
      for (uint32_t mt = 0; 2 * mt < nt; ++mt) {
        auto cst = [&](uint32_t p, uint32_t src) -> uint32_t {
          const uint32_t e = 2 * mt + p;
          if (e >= nt) return 0;
          const uint32_t dl = e < lo ? e : e + ns, tp = dl < l ? dl : L + (dl - l);
          const uint32_t c = h.mu_conv[(((size_t)l * D + j) * A + src) * E + tp];
          return mulmod(c, inv64[tp], h.q[tp]);
        };
        mx_tile(&h.mx_up[(((size_t)l * D + j) * T + mt) * tile], ns, cst);
      }
    }
  }
  h.mx_md_ks.assign((size_t)T * tile, 0);
  h.mx_md_pl.assign((size_t)T * tile, 0);
  for (uint32_t mt = 0; 2 * mt < L; ++mt) {
    auto ks = [&](uint32_t p, uint32_t src) -> uint32_t {
      const uint32_t e = 2 * mt + p;
      return e < L ? mulmod(h.md_conv[(size_t)src * L + e], inv64[e], h.q[e]) : 0u;
    };
    auto pl = [&](uint32_t p, uint32_t src) -> uint32_t {
      const uint32_t e = 2 * mt + p;
      return e < L ? mulmod(h.md_conv64[(size_t)src * L + e], inv64[e], h.q[e]) : 0u;
    };
    mx_tile(&h.mx_md_ks[(size_t)mt * tile], K, ks);
    mx_tile(&h.mx_md_pl[(size_t)mt * tile], K, pl);
  }
}

void build_tables(Host& h) {
  const uint32_t n = h.n, E = h.L + h.K, L = h.L, K = h.K, A = h.alpha;
  h.qinv.resize(E);
  h.psi.resize(E);
  h.tw.resize((size_t)E * n);
  h.itw.resize((size_t)E * n);
  h.ninv.resize(E);
  h.bound.resize(E);
  h.one.resize(E);
  h.r2.resize(E);
  h.r64tab.resize(E);
  for (uint32_t t = 0; t < E; ++t) {
    const uint32_t q = h.q[t];
    h.qinv[t] = inv2_32(q);
    h.psi[t] = min_root(q, n);
    const uint32_t pinv = invmod(h.psi[t], q);
    std::vector<uint32_t> pw(n), ipw(n);
    pw[0] = ipw[0] = 1;
    for (uint32_t k = 1; k < n; ++k) {
      pw[k] = mulmod(pw[k - 1], h.psi[t], q);
      ipw[k] = mulmod(ipw[k - 1], pinv, q);
    }
    for (uint32_t k = 0; k < n; ++k) {
      const uint32_t r = brv(k, h.log_n);
      h.tw[(size_t)t * n + k] = mont(pw[r], q).x;
      h.itw[(size_t)t * n + k] = mont(ipw[r], q).x;
    }
    h.ninv[t] = mont(invmod(n % q, q), q);
    h.bound[t] = (uint32_t)(((1ull << 32) / q) * q);
    h.one[t] = mont(1, q);
    h.r2[t] = mont(r32(q), q);
    h.r64tab[t] = r64(q);
  }
  // rescale at level l: q_{l-1}^-1 mod q_i for i < l-1
  h.rs_inv.assign((size_t)(L + 1) * L, make_uint2(0, 0));
  for (uint32_t l = 2; l <= L; ++l)
    for (uint32_t i = 0; i + 1 < l; ++i)
      h.rs_inv[(size_t)l * L + i] = mont(invmod(h.q[l - 1] % h.q[i], h.q[i]), h.q[i]);
  // ModUp: per level l, digit j, source prime i of the digit, target prime t
  h.mu_scale.assign((size_t)(L + 1) * L, make_uint2(0, 0));
  h.mu_conv.assign((size_t)(L + 1) * h.dnum * A * E, 0);
  for (uint32_t l = 1; l <= L; ++l) {
    const uint32_t d = (l + A - 1) / A;
    for (uint32_t j = 0; j < d; ++j) {
      const uint32_t lo = j * A, hi = std::min(lo + A, l);
      for (uint32_t i = lo; i < hi; ++i) {
        // [Qd/q_i]_{q_i} and its inverse, times N^-1
        uint32_t qh = 1;
        for (uint32_t i2 = lo; i2 < hi; ++i2)
          if (i2 != i) qh = mulmod(qh, h.q[i2] % h.q[i], h.q[i]);
        const uint32_t sc = mulmod(invmod(qh, h.q[i]), invmod(n % h.q[i], h.q[i]), h.q[i]);
        h.mu_scale[(size_t)l * L + i] = mont(sc, h.q[i]);
        for (uint32_t t = 0; t < E; ++t) {
          const uint32_t qt = h.q[t];
          uint32_t v = 1;
          for (uint32_t i2 = lo; i2 < hi; ++i2)
            if (i2 != i) v = mulmod(v, h.q[i2] % qt, qt);
          h.mu_conv[(((size_t)l * h.dnum + j) * A + (i - lo)) * E + t] = mulmod(v, r64(qt), qt);
        }
      }
    }
  }
  // ModDown
  h.md_scale_ks.resize(K);
  h.md_scale_pl.resize(K);
  h.md_conv.resize((size_t)K * L);
  h.md_conv64.resize((size_t)K * L);
  h.md_fin_ks.resize(L);
  h.md_fin_pl.resize(L);
  h.p_mod.resize(L);
  for (uint32_t k = 0; k < K; ++k) {
    const uint32_t pk = h.q[L + k];
    uint32_t ph = 1;
    for (uint32_t k2 = 0; k2 < K; ++k2)
      if (k2 != k) ph = mulmod(ph, h.q[L + k2] % pk, pk);
    const uint32_t base = mulmod(invmod(ph, pk), invmod(n % pk, pk), pk);
    h.md_scale_pl[k] = mont(base, pk);
    h.md_scale_ks[k] = mont(mulmod(base, r32(pk), pk), pk);
    for (uint32_t i = 0; i < L; ++i) {
      const uint32_t qi = h.q[i];
      uint32_t v = 1;
      for (uint32_t k2 = 0; k2 < K; ++k2)
        if (k2 != k) v = mulmod(v, h.q[L + k2] % qi, qi);
      h.md_conv[(size_t)k * L + i] = mulmod(v, r32(qi), qi);
      h.md_conv64[(size_t)k * L + i] = mulmod(v, r64(qi), qi);
    }
  }
  for (uint32_t i = 0; i < L; ++i) {
    const uint32_t qi = h.q[i];
    uint32_t p = 1;
    for (uint32_t k = 0; k < K; ++k) p = mulmod(p, h.q[L + k] % qi, qi);
    const uint32_t pinv = invmod(p, qi);
    h.md_fin_pl[i] = mont(pinv, qi);
    h.p_mod[i] = mont(p, qi);
    h.md_fin_ks[i] = mont(mulmod(pinv, r32(qi), qi), qi);
  }
  build_mx_tables(h);
}

}  // namespace

struct ckks_ctx {
  Host h;
  DevTables d{};
  void* dev_tables = nullptr;
  uint32_t max_batch = 0;
  int device = -1;
  uint32_t regen_blocks = ckks::kDefaultRegenBlocks;
  // matrix-core conversion: operand tables on the device, and whether calls use them
  const uint4* mx_up = nullptr;
  const uint4* mx_md_ks = nullptr;
  const uint4* mx_md_pl = nullptr;
  bool conv_mfma = false;
  // ckks_keyswitch with the inner product and ModDown as separate launches
  bool unfused = false;
  // workspace (items = max_batch)
  void* ws = nullptr;
  uint64_t ws_bytes = 0;
  uint32_t* rowtmp = nullptr;  // [B][max(L,K)][N]
  uint32_t* ext = nullptr;     // [B][dnum][L+K][N]
  uint32_t* tmpP = nullptr;    // [B][2][K][N]
  uint32_t* conv = nullptr;    // [B][2][L][N]
  uint32_t* tens = nullptr;    // [B][3][L][N]: relinearised pair of a multiply; R and S buffers of a transform
  // ckks_keyswitch_multi: side streams (default priority, created on first use) and
  // one event per launch sequence of a call
  std::vector<hipStream_t> side;
  std::vector<hipEvent_t> task_ev;
  // per-launch event timer (measurement aid)
  bool prof_on = false;
  std::vector<hipEvent_t> prof_ev;     // pool: 2 events per record
  std::vector<int> prof_cls;           // class of each record
};

namespace {

constexpr size_t kProfMax = 8192;
// streams a multi-item key-switch spreads its launch sequences over (the caller's
// included); four matches the hardware queues HIP gives a process by default
constexpr uint32_t kMultiStreams = 4;

// Brackets one launch with events on `s` when the context's timer is on.
struct ProfScope {
  ckks_ctx* c;
  hipStream_t s;
  size_t rec;
  ProfScope(ckks_ctx* ctx, int cls, hipStream_t st) : c(ctx), s(st), rec(SIZE_MAX) {
    if (!c->prof_on || c->prof_cls.size() >= kProfMax) return;
    rec = c->prof_cls.size();
    c->prof_cls.push_back(cls);
    (void)hipEventRecord(c->prof_ev[2 * rec], s);
  }
  ~ProfScope() {
    if (rec != SIZE_MAX) (void)hipEventRecord(c->prof_ev[2 * rec + 1], s);
  }
};

}  // namespace

namespace {

template <typename T>
size_t bytes_of(const std::vector<T>& v) { return v.size() * sizeof(T); }

ckks_status upload_tables(ckks_ctx* c) {
  Host& h = c->h;
  struct Part { const void* src; size_t bytes; const void** dst; };
  DevTables& d = c->d;
  std::vector<Part> parts = {
      {h.q.data(), bytes_of(h.q), (const void**)&d.q},
      {h.qinv.data(), bytes_of(h.qinv), (const void**)&d.qinv},
      {h.tw.data(), bytes_of(h.tw), (const void**)&d.tw},
      {h.itw.data(), bytes_of(h.itw), (const void**)&d.itw},
      {h.ninv.data(), bytes_of(h.ninv), (const void**)&d.ninv},
      {h.mu_scale.data(), bytes_of(h.mu_scale), (const void**)&d.mu_scale},
      {h.mu_conv.data(), bytes_of(h.mu_conv), (const void**)&d.mu_conv},
      {h.md_scale_ks.data(), bytes_of(h.md_scale_ks), (const void**)&d.md_scale_ks},
      {h.md_scale_pl.data(), bytes_of(h.md_scale_pl), (const void**)&d.md_scale_pl},
      {h.md_conv.data(), bytes_of(h.md_conv), (const void**)&d.md_conv},
      {h.md_conv64.data(), bytes_of(h.md_conv64), (const void**)&d.md_conv64},
      {h.md_fin_ks.data(), bytes_of(h.md_fin_ks), (const void**)&d.md_fin_ks},
      {h.md_fin_pl.data(), bytes_of(h.md_fin_pl), (const void**)&d.md_fin_pl},
      {h.bound.data(), bytes_of(h.bound), (const void**)&d.bound},
      {h.one.data(), bytes_of(h.one), (const void**)&d.one},
      {h.r2.data(), bytes_of(h.r2), (const void**)&d.r2},
      {h.r64tab.data(), bytes_of(h.r64tab), (const void**)&d.r64},
      {h.rs_inv.data(), bytes_of(h.rs_inv), (const void**)&d.rs_inv},
      {h.p_mod.data(), bytes_of(h.p_mod), (const void**)&d.p_mod},
  };
  if (h.mx_ok) {
    parts.push_back({h.mx_w.data(), bytes_of(h.mx_w), (const void**)&d.mx_w});
    parts.push_back({h.mx_up.data(), bytes_of(h.mx_up), (const void**)&c->mx_up});
    parts.push_back({h.mx_md_ks.data(), bytes_of(h.mx_md_ks), (const void**)&c->mx_md_ks});
    parts.push_back({h.mx_md_pl.data(), bytes_of(h.mx_md_pl), (const void**)&c->mx_md_pl});
  }
  size_t total = 0;
  for (auto& p : parts) total += (p.bytes + 255) & ~size_t(255);
  if (hipMalloc(&c->dev_tables, total) != hipSuccess)
    return fail(CKKS_ENOMEM, "hipMalloc of %zu bytes of constant tables failed", total);
  size_t off = 0;
  for (auto& p : parts) {
    char* dst = (char*)c->dev_tables + off;
    if (hipMemcpy(dst, p.src, p.bytes, hipMemcpyHostToDevice) != hipSuccess)
      return fail(CKKS_EHIP, "hipMemcpy of constant tables failed");
    *p.dst = dst;
    off += (p.bytes + 255) & ~size_t(255);
  }
  // the matrix-core operand tiles are only read on the device
  std::vector<uint8_t>().swap(h.mx_up);
  std::vector<uint8_t>().swap(h.mx_md_ks);
  std::vector<uint8_t>().swap(h.mx_md_pl);
  return CKKS_OK;
}

ckks_status check_ctx(const ckks_ctx* c) {
  if (!c) return fail(CKKS_EINVAL, "ctx is NULL");
  return CKKS_OK;
}

// Last check of every compute call, after all argument checks: a host-only context stops here.
ckks_status check_device(const ckks_ctx* c) {
  if (c->max_batch == 0) return fail(CKKS_EINVAL, "host-only context (max_batch = 0) cannot run device calls");
  return CKKS_OK;
}

ckks_status check_level(const ckks_ctx* c, uint32_t level) {
  if (level < 1 || level > c->h.L) return fail(CKKS_ERANGE, "level %u outside 1..%u", level, c->h.L);
  return CKKS_OK;
}

ckks_status check_batch(const ckks_ctx* c, uint32_t batch) {
  const uint32_t lim = c->max_batch ? c->max_batch : 4096;  // host-only contexts check the shape only
  if (batch < 1 || batch > lim) return fail(CKKS_ERANGE, "batch %u outside 1..%u (context max_batch)", batch, lim);
  return CKKS_OK;
}

ckks_status check_galois(const ckks_ctx* c, uint32_t g) {
  if (g % 2 == 0 || g >= 2 * c->h.n)
    return fail(CKKS_ERANGE, "Galois element %u must be odd and below 2N = %u", g, 2 * c->h.n);
  return CKKS_OK;
}

// Whether word ranges [a, a + na) and [b, b + nb) overlap (a NULL range never does).
bool overlaps(const uint32_t* a, uint64_t na, const uint32_t* b, uint64_t nb) {
  return a && b && a < b + nb && b < a + na;
}

// A key-switch's output (out_words words) overlaps neither its ciphertexts
// ct[batch][2][level][N] nor the key halves [dnum][L+K][N] (the kernels read
// them after the first outputs are written).
ckks_status check_keyswitch_out(const ckks_ctx* c, const uint32_t* ct, uint32_t level, uint32_t batch,
                                const uint32_t* key_b, const uint32_t* key_a, const uint32_t* out,
                                uint64_t out_words) {
  const uint64_t N = c->h.n, key_words = (uint64_t)c->h.dnum * (c->h.L + c->h.K) * N;
  if (overlaps(ct, (uint64_t)batch * 2 * level * N, out, out_words)) return fail(CKKS_EINVAL, "out overlaps ct");
  if (overlaps(key_b, key_words, out, out_words)) return fail(CKKS_EINVAL, "out overlaps key_b");
  if (overlaps(key_a, key_words, out, out_words)) return fail(CKKS_EINVAL, "out overlaps key_a");
  return CKKS_OK;
}

ckks_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(CKKS_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

void seed_words(const uint8_t* seed, uint32_t out[8]) {
  for (int i = 0; i < 8; ++i)
    out[i] = (uint32_t)seed[4 * i] | ((uint32_t)seed[4 * i + 1] << 8) | ((uint32_t)seed[4 * i + 2] << 16) |
             ((uint32_t)seed[4 * i + 3] << 24);
}

uint32_t digits_at(const Host& h, uint32_t level) { return (level + h.alpha - 1) / h.alpha; }

// Shifts the context's workspace pointers to start at workspace item `pos` for its
// lifetime, so that launch sequences on different streams use disjoint item ranges.
struct WsView {
  ckks_ctx* c;
  uint32_t *rowtmp, *ext, *tmpP, *conv;
  WsView(ckks_ctx* ctx, uint32_t pos) : c(ctx), rowtmp(ctx->rowtmp), ext(ctx->ext), tmpP(ctx->tmpP), conv(ctx->conv) {
    const Host& h = c->h;
    const uint64_t N = h.n, p = pos;
    c->rowtmp += p * std::max(std::max(h.L, h.K), 2u) * N;
    c->ext += p * h.dnum * (h.L + h.K) * N;
    c->tmpP += p * 2 * h.K * N;
    c->conv += p * 2 * h.L * N;
  }
  ~WsView() {
    c->rowtmp = rowtmp;
    c->ext = ext;
    c->tmpP = tmpP;
    c->conv = conv;
  }
};

// Workspace of one key-switch launch sequence: c1 after the row half of INTT
// (rowtmp, item stride level*N), the extended digits (ext, item stride ext_item),
// the special part after the row INTT (tmpP, item stride 2K*N) and the converted
// special part (conv, item stride 2*level*N).  By default the context's own.
struct Ws {
  uint32_t *rowtmp, *ext, *tmpP, *conv;
  uint64_t ext_item;
};

Ws ctx_ws(const ckks_ctx* c) {
  return Ws{c->rowtmp, c->ext, c->tmpP, c->conv, (uint64_t)c->h.dnum * (c->h.L + c->h.K) * c->h.n};
}

// Steps 1-2: INTT row half of c1 and the fused ModUp conversion into the workspace's ext.
// c1b (optional): c1 is the elementwise product c1 * c1b, formed in the row pass.
hipError_t run_modup(ckks_ctx* c, const uint32_t* c1, uint64_t c1_item_stride, uint32_t level, uint32_t items,
                     hipStream_t s, const uint32_t* const* c1_items = nullptr, const uint32_t* c1b = nullptr,
                     const Ws* wsp = nullptr) {
  const Host& h = c->h;
  const uint64_t N = h.n;
  const Ws w = wsp ? *wsp : ctx_ws(c);
  ckks::RowArgs r{};
  r.src = c1;
  if (c1_items) {  // one pointer per item (at most kMaxGroup)
    r.use_srcs = 1;
    for (uint32_t i = 0; i < items; ++i) r.srcs[i] = c1_items[i];
  }
  r.dst = w.rowtmp;
  r.src2 = c1b;
  r.src_item_stride = c1_item_stride;
  r.dst_item_stride = (uint64_t)level * N;
  r.prime0 = 0;
  r.n_limbs = level;
  r.own_lo = r.own_n = 0;
  r.level = 0;
  hipError_t e;
  {
    ProfScope p(c, CKKS_K_ROW, s);
    e = ckks::launch_row(c->d, r, false, items, s);
  }
  if (e != hipSuccess) return e;
  ckks::ConvArgs a{};
  a.src = w.rowtmp;
  a.src_item = (uint64_t)level * N;
  a.src_y = (uint64_t)h.alpha * N;
  a.dst = w.ext;
  a.dst_item = w.ext_item;
  a.dst_y = (uint64_t)(h.L + h.K) * N;
  a.src_prime0 = 0;
  a.src_prime_step = h.alpha;
  a.ns_max = h.alpha;
  a.ns_limit = level;
  a.scale = c->d.mu_scale + (size_t)level * h.L;
  a.scale_y = h.alpha;
  a.conv = c->d.mu_conv + (size_t)level * h.dnum * h.alpha * (h.L + h.K);
  a.conv_y = h.alpha * (h.L + h.K);
  a.conv_s = h.L + h.K;
  a.conv_by_abs = 1;
  a.skip = 1;
  a.level = level;
  a.n_targets = 0;  // per digit: level + K - (digit size), computed in the kernel
  if (c->conv_mfma) {
    a.mx = c->mx_up + (size_t)level * h.dnum * ckks::kMxTiles * 128;
    a.mx_y = ckks::kMxTiles * 128;
  }
  ProfScope p(c, CKKS_K_MODUP_CONV, s);
  return ckks::launch_conv(c->d, a, digits_at(h, level), items, s);
}

// Steps 3-5 for `n_keys` key groups of `n_ct` ciphertexts each (the workspace's ext already
// filled; ciphertext c's digits at ext + c * ext_stride).
hipError_t run_ip_moddown(ckks_ctx* c, const uint32_t* ct, uint64_t ct_stride, uint64_t ext_stride,
                          uint32_t level, uint32_t n_ct, uint32_t n_keys, const ckks::KeyRef* keys, uint32_t* out,
                          bool digits_ntt, hipStream_t s, bool per_group = false,
                          const uint32_t* ty = nullptr, const Ws* wsp = nullptr) {
  const Host& h = c->h;
  const uint64_t N = h.n;
  const Ws w = wsp ? *wsp : ctx_ws(c);
  ckks::IpArgs ip{};
  ip.level = level;
  ip.nd = digits_at(h, level);
  ip.n_ct = n_ct;
  ip.ext = w.ext;
  ip.ext_ct_stride = ext_stride;
  ip.ct = ct;
  ip.ct_ct_stride = ct_stride;
  ip.tmpP = w.tmpP;
  ip.conv = w.conv;
  ip.out = out;
  ip.regen_blocks = c->regen_blocks;
  ip.digits_ntt = digits_ntt ? 1u : 0u;
  ip.per_group = per_group ? 1u : 0u;
  ip.n_keys = n_keys;
  for (uint32_t k = 0; k < n_keys; ++k) ip.key[k] = keys[k];
  ip.ty = ty;
  hipError_t e;
  {
    ProfScope p(c, CKKS_K_IP_SPECIAL, s);
    e = ckks::launch_ip(c->d, ip, false, h.K, s);
  }
  if (e != hipSuccess) return e;
  ckks::ConvArgs a{};
  a.src = w.tmpP;
  a.src_item = 2ull * h.K * N;
  a.src_y = (uint64_t)h.K * N;
  a.dst = w.conv;
  a.dst_item = 2ull * level * N;
  a.dst_y = (uint64_t)level * N;
  a.src_prime0 = h.L;
  a.src_prime_step = 0;
  a.ns_max = h.K;
  a.ns_limit = h.K;
  a.scale = c->d.md_scale_ks;
  a.scale_y = 0;
  a.conv = c->d.md_conv;
  a.conv_y = 0;
  a.conv_s = h.L;
  a.conv_by_abs = 0;
  a.n_targets = level;
  a.skip = 0;
  a.level = level;
  if (c->conv_mfma) a.mx = c->mx_md_ks;
  {
    ProfScope p(c, CKKS_K_MODDOWN_CONV, s);
    e = ckks::launch_conv(c->d, a, 2, n_ct * n_keys, s);
  }
  if (e != hipSuccess) return e;
  ProfScope p(c, CKKS_K_IP_FINAL, s);
  return ckks::launch_ip(c->d, ip, true, level, s);
}

// ModUp of one ciphertext ct [2][level][N] into ctx->ext with the digits' NTT finished
// (row half; own limbs copied from c1): the shared start of every hoisted call.
hipError_t run_hoisted_digits(ckks_ctx* c, const uint32_t* ct, uint32_t level, hipStream_t s) {
  const Host& h = c->h;
  const uint64_t N = h.n;
  hipError_t e = run_modup(c, ct + (uint64_t)level * N, 0, level, 1, s);
  if (e != hipSuccess) return e;
  for (uint32_t j = 0; j < digits_at(h, level); ++j) {
    ckks::RowArgs r{};
    r.src = c->ext + (uint64_t)j * (h.L + h.K) * N;
    r.dst = c->ext + (uint64_t)j * (h.L + h.K) * N;
    r.src_item_stride = r.dst_item_stride = 0;
    r.prime0 = 0;
    r.n_limbs = level + h.K;
    r.own_lo = j * h.alpha;
    r.own_n = std::min(h.alpha, level - j * h.alpha);
    r.own_src = ct + (uint64_t)level * N;
    r.own_item_stride = 0;
    r.level = level;
    ProfScope p(c, CKKS_K_ROW, s);
    e = ckks::launch_row(c->d, r, true, 1, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// ModDown of `items` extended polynomials x [level+K][N] (stride x_item) into out
// [level][N] (stride out_item).  Uses ctx->rowtmp and ctx->conv.
hipError_t run_moddown(ckks_ctx* c, const uint32_t* x, uint64_t x_item, uint32_t level, uint32_t* out,
                       uint64_t out_item, uint32_t items, hipStream_t s) {
  const Host& h = c->h;
  const uint64_t N = h.n;
  ckks::RowArgs r{};
  r.src = x + (uint64_t)level * N;
  r.src_item_stride = x_item;
  r.dst = c->rowtmp;
  r.dst_item_stride = (uint64_t)h.K * N;
  r.prime0 = h.L;
  r.n_limbs = h.K;
  hipError_t e;
  {
    ProfScope p(c, CKKS_K_MODDOWN_ROW, s);
    e = ckks::launch_row(c->d, r, false, items, s);
  }
  if (e != hipSuccess) return e;
  ckks::ConvArgs a{};
  a.src = c->rowtmp;
  a.src_item = (uint64_t)h.K * N;
  a.src_y = 0;
  a.dst = c->conv;
  a.dst_item = (uint64_t)level * N;
  a.dst_y = 0;
  a.src_prime0 = h.L;
  a.src_prime_step = 0;
  a.ns_max = h.K;
  a.ns_limit = h.K;
  a.scale = c->d.md_scale_pl;
  a.scale_y = 0;
  a.conv = c->d.md_conv64;
  a.conv_y = 0;
  a.conv_s = h.L;
  a.conv_by_abs = 0;
  a.n_targets = level;
  a.skip = 0;
  a.level = level;
  if (c->conv_mfma) a.mx = c->mx_md_pl;
  {
    ProfScope p(c, CKKS_K_MODDOWN_CONV, s);
    e = ckks::launch_conv(c->d, a, 1, items, s);
  }
  if (e != hipSuccess) return e;
  // row NTT fused with (x_i - .) * P^-1
  ckks::RowArgs f{};
  f.src = c->conv;
  f.src_item_stride = (uint64_t)level * N;
  f.dst = out;
  f.dst_item_stride = out_item;
  f.prime0 = 0;
  f.n_limbs = level;
  f.cmb = x;
  f.cmb_item_stride = x_item;
  f.cmb_factor = c->d.md_fin_pl;
  ProfScope p(c, CKKS_K_MODDOWN_FINAL, s);
  return ckks::launch_row(c->d, f, true, items, s);
}

// Argument checks of a key-switch call other than the batch limit and the device.
ckks_status check_keyswitch_args(const ckks_ctx* c, const uint32_t* ct, uint32_t level, const uint32_t* key_b,
                                 const uint8_t* key_seed, const uint32_t* key_a, uint32_t galois_elt,
                                 const uint32_t* out, uint32_t batch) {
  ckks_status st;
  if (!ct || !key_b || !out) return fail(CKKS_EINVAL, "ct, key_b or out is NULL");
  if (!key_a && !key_seed) return fail(CKKS_EINVAL, "need key_a or key_seed");
  if ((st = check_level(c, level)) || (st = check_galois(c, galois_elt))) return st;
  return check_keyswitch_out(c, ct, level, batch, key_b, key_a, out, (uint64_t)batch * 2 * level * c->h.n);
}

// A batched key-switch with the inner product and ModDown as separate launches (the
// fusion knob off): ModUp, the digits' row NTT (own limbs copied from c1), the
// extended-basis inner product with P*sigma(c0) on the ciphertext primes, and
// ModDown of both halves.  ModUp runs once for the batch; the rest in groups of
// items that fit the pairs buffer (tens) and ModDown's row buffer.
ckks_status keyswitch_unfused(ckks_ctx* c, const uint32_t* ct, uint32_t level, const uint32_t* key_b,
                              const uint8_t* key_seed, const uint32_t* key_a, uint32_t galois_elt, uint32_t* out,
                              uint32_t batch, hipStream_t s) {
  const Host& h = c->h;
  const uint64_t N = h.n, E = h.L + h.K, El = level + h.K, B = c->max_batch;
  const uint64_t ext_item = (uint64_t)h.dnum * E * N;
  const uint64_t group = std::min<uint64_t>(
      {(uint64_t)batch, B * 3 * h.L / (2 * El), B * std::max(std::max(h.L, h.K), 2u) / (2 * h.K)});
  if (group == 0)
    return fail(CKKS_ERANGE, "the unfused key-switch at level %u needs a context with a larger max_batch", level);
  hipError_t e = run_modup(c, ct + (uint64_t)level * N, 2ull * level * N, level, batch, s);
  if (e != hipSuccess) return hip_status(e, "ModUp");
  const uint32_t nd = digits_at(h, level);
  for (uint32_t j = 0; j < nd; ++j) {
    ckks::RowArgs r{};
    r.src = r.dst = c->ext + (uint64_t)j * E * N;
    r.src_item_stride = r.dst_item_stride = ext_item;
    r.prime0 = 0;
    r.n_limbs = (uint32_t)El;
    r.own_lo = j * h.alpha;
    r.own_n = std::min(h.alpha, level - j * h.alpha);
    r.own_src = ct + (uint64_t)level * N;
    r.own_item_stride = 2ull * level * N;
    r.level = level;
    ProfScope p(c, CKKS_K_DIGIT_NTT, s);
    e = ckks::launch_row(c->d, r, true, batch, s);
    if (e != hipSuccess) return hip_status(e, "digit NTT");
  }
  for (uint64_t i0 = 0; i0 < batch; i0 += group) {
    const uint32_t items = (uint32_t)std::min<uint64_t>(group, batch - i0);
    ckks::ExtArgs a{};
    a.level = level;
    a.nd = nd;
    a.ext = c->ext + i0 * ext_item;
    a.c0 = ct + i0 * 2 * level * N;
    a.out = c->tens;
    a.regen_blocks = c->regen_blocks;
    a.n_keys = 1;
    a.items = items;
    a.ext_item = ext_item;
    a.c0_item = 2ull * level * N;
    a.out_item = 2 * El * N;
    a.key[0] = ckks::KeyRef{};
    a.key[0].b = key_b;
    a.key[0].a = key_a;
    if (!key_a) seed_words(key_seed, a.key[0].seed);
    a.key[0].galois = galois_elt;
    {
      ProfScope p(c, CKKS_K_IP_EXT, s);
      e = ckks::launch_rot_ext(c->d, a, s);
    }
    if (e != hipSuccess) return hip_status(e, "inner product");
    e = run_moddown(c, c->tens, El * N, level, out + i0 * 2 * level * N, (uint64_t)level * N, 2 * items, s);
    if (e != hipSuccess) return hip_status(e, "ModDown");
  }
  return ok();
}

// The launch sequence of one batched key-switch, in the workspace `wsp` (the
// context's when NULL).
ckks_status keyswitch_run(ckks_ctx* c, const uint32_t* ct, uint32_t level, const uint32_t* key_b,
                          const uint8_t* key_seed, const uint32_t* key_a, uint32_t galois_elt, uint32_t* out,
                          uint32_t batch, hipStream_t s, const Ws* wsp) {
  const uint64_t N = c->h.n;
  if (c->unfused && !wsp) return keyswitch_unfused(c, ct, level, key_b, key_seed, key_a, galois_elt, out, batch, s);
  const Ws w = wsp ? *wsp : ctx_ws(c);
  hipError_t e = run_modup(c, ct + (uint64_t)level * N, 2ull * level * N, level, batch, s, nullptr, nullptr, &w);
  if (e != hipSuccess) return hip_status(e, "ModUp");
  ckks::KeyRef k{};
  k.b = key_b;
  k.a = key_a;
  if (!key_a) seed_words(key_seed, k.seed);
  k.galois = galois_elt;
  e = run_ip_moddown(c, ct, 2ull * level * N, w.ext_item, level, batch, 1, &k, out, false, s, false, nullptr, &w);
  return hip_status(e, "inner product / ModDown");
}

}  // namespace

extern "C" {

const char* ckks_last_error(void) { return g_err.c_str(); }

ckks_status ckks_chain_primes(uint32_t log_n, uint32_t bits, uint32_t count, uint32_t* out_host) {
  if (!out_host) return fail(CKKS_EINVAL, "out_host is NULL");
  if (bits < 20 || bits > 32) return fail(CKKS_ERANGE, "bits %u outside 20..32", bits);
  if (log_n < 1 || log_n + 1 >= bits) return fail(CKKS_ERANGE, "log_n %u out of range for %u-bit primes", log_n, bits);
  const uint64_t step = 2ull << log_n;
  uint64_t cand = (1ull << bits) - step + 1;
  uint32_t found = 0;
  while (found < count) {
    if (cand <= step) return fail(CKKS_ERANGE, "fewer than %u qualifying primes below 2^%u", count, bits);
    if (is_prime32((uint32_t)cand)) out_host[found++] = (uint32_t)cand;
    cand -= step;
  }
  return ok();
}

ckks_status ckks_ctx_create(ckks_ctx** out, uint32_t log_n, uint32_t num_q, uint32_t num_p, uint32_t dnum,
                            const uint32_t* primes, uint32_t max_batch) {
  if (!out) return fail(CKKS_EINVAL, "out is NULL");
  *out = nullptr;
  if (!primes) return fail(CKKS_EINVAL, "primes is NULL");
  if (log_n < 12 || log_n > 16) return fail(CKKS_EUNSUPPORTED, "log_n %u: this build implements 12..16", log_n);
  if (num_q < 1 || num_p < 1 || num_q + num_p > 256) return fail(CKKS_ERANGE, "num_q %u / num_p %u out of range", num_q, num_p);
  if (dnum < 1 || dnum > ckks::kMaxDnum || dnum > num_q) return fail(CKKS_ERANGE, "dnum %u outside 1..min(%u, num_q)", dnum, ckks::kMaxDnum);
  const uint32_t alpha = (num_q + dnum - 1) / dnum;
  if (num_p < alpha) return fail(CKKS_ERANGE, "num_p %u below the digit width %u", num_p, alpha);
  if (alpha > 16 || num_p > 16) return fail(CKKS_EUNSUPPORTED, "digit width %u / num_p %u above 16", alpha, num_p);
  const uint32_t n = 1u << log_n;
  for (uint32_t t = 0; t < num_q + num_p; ++t) {
    const uint32_t q = primes[t];
    if (q % (2 * n) != 1 || !is_prime32(q))
      return fail(CKKS_ERANGE, "primes[%u] = %u is not a prime = 1 mod 2N", t, q);
    for (uint32_t u = 0; u < t; ++u)
      if (primes[u] == q) return fail(CKKS_ERANGE, "primes[%u] repeats primes[%u]", t, u);
  }
  if (max_batch > 4096) return fail(CKKS_ERANGE, "max_batch %u above 4096", max_batch);
  ckks_ctx* c = new ckks_ctx();
  Host& h = c->h;
  h.log_n = log_n;
  h.n = n;
  h.L = num_q;
  h.K = num_p;
  h.dnum = dnum;
  h.alpha = alpha;
  h.q.assign(primes, primes + num_q + num_p);
  build_tables(h);
  c->max_batch = max_batch;
  c->d.log_n = log_n;
  c->d.n = n;
  c->d.L = num_q;
  c->d.K = num_p;
  c->d.dnum = dnum;
  c->d.alpha = alpha;
  c->d.all_big = 1;
  for (uint32_t t = 0; t < num_q + num_p; ++t) c->d.all_big &= primes[t] >> 31;
  if (max_batch == 0) {
    *out = c;
    return ok();
  }
  if (const hipError_t e = hipGetDevice(&c->device); e != hipSuccess) {
    delete c;
    return fail(CKKS_EHIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  }
  // device address of the static scratch array of ckks_keyswitch_noalloc (once per
  // device, with that device current); a failure only disables that call
  (void)ckks::scratch_setup(c->device);
  ckks_status st = upload_tables(c);
  if (st != CKKS_OK) {
    std::string msg = g_err;
    ckks_ctx_destroy(c);
    g_err = msg;
    return st;
  }
  const uint64_t N = n, E = num_q + num_p, B = max_batch;
  const uint64_t rowtmp = B * std::max(std::max(num_q, num_p), 2u) * N, ext = B * dnum * E * N,
                 tmpP = B * 2 * num_p * N, conv = B * 2 * num_q * N, tens = B * 3 * num_q * N;
  c->ws_bytes = (rowtmp + ext + tmpP + conv + tens) * sizeof(uint32_t);
  if (hipMalloc(&c->ws, c->ws_bytes) != hipSuccess) {
    uint64_t b = c->ws_bytes;
    ckks_ctx_destroy(c);
    return fail(CKKS_ENOMEM, "hipMalloc of %llu workspace bytes failed", (unsigned long long)b);
  }
  c->rowtmp = (uint32_t*)c->ws;
  c->ext = c->rowtmp + rowtmp;
  c->tmpP = c->ext + ext;
  c->conv = c->tmpP + tmpP;
  c->tens = c->conv + conv;
  *out = c;
  return ok();
}

void ckks_ctx_destroy(ckks_ctx* c) {
  if (!c) return;
  for (hipEvent_t e : c->prof_ev) (void)hipEventDestroy(e);
  for (hipEvent_t e : c->task_ev) (void)hipEventDestroy(e);
  for (hipStream_t st : c->side) (void)hipStreamDestroy(st);
  if (c->ws) (void)hipFree(c->ws);
  if (c->dev_tables) (void)hipFree(c->dev_tables);
  delete c;
}

ckks_status ckks_ctx_info(const ckks_ctx* c, uint32_t* n_out, uint32_t* num_q_out, uint32_t* num_p_out,
                          uint32_t* dnum_out, uint32_t* alpha_out, uint32_t* max_batch_out,
                          uint64_t* workspace_bytes_out, uint32_t* roots_out) {
  if (!c) return fail(CKKS_EINVAL, "ctx is NULL");
  if (n_out) *n_out = c->h.n;
  if (num_q_out) *num_q_out = c->h.L;
  if (num_p_out) *num_p_out = c->h.K;
  if (dnum_out) *dnum_out = c->h.dnum;
  if (alpha_out) *alpha_out = c->h.alpha;
  if (max_batch_out) *max_batch_out = c->max_batch;
  if (workspace_bytes_out) *workspace_bytes_out = c->ws_bytes;
  if (roots_out) std::copy(c->h.psi.begin(), c->h.psi.end(), roots_out);
  return ok();
}

ckks_status ckks_ctx_set_regen_blocks(ckks_ctx* c, uint32_t blocks) {
  if (!c) return fail(CKKS_EINVAL, "ctx is NULL");
  if (blocks < ckks::kRow / 16 || blocks > ckks::kMaxRegenBlocks)
    return fail(CKKS_ERANGE, "regen blocks %u outside %u..%u", blocks, ckks::kRow / 16, ckks::kMaxRegenBlocks);
  c->regen_blocks = blocks;
  return ok();
}

ckks_status ckks_ctx_set_fused(ckks_ctx* c, uint32_t fused) {
  ckks_status st = check_ctx(c);
  if (st) return st;
  if (!c->max_batch) return fail(CKKS_EINVAL, "host-only context");
  c->unfused = !fused;
  return ok();
}

ckks_status ckks_ctx_set_conv_mfma(ckks_ctx* c, uint32_t on) {
  if (!c) return fail(CKKS_EINVAL, "ctx is NULL");
  if (on && !c->h.mx_ok)
    return fail(CKKS_EUNSUPPORTED, "matrix-core conversion needs N = 2^16 and 9..12 primes per digit and special part");
  if (on && c->max_batch == 0) return fail(CKKS_EINVAL, "host-only context (max_batch = 0) has no device tables");
  c->conv_mfma = on != 0;
  return ok();
}

static ckks_status ntt_common(const ckks_ctx* c, uint32_t* data, uint32_t first, uint32_t n_limbs, uint32_t batch) {
  ckks_status st = check_ctx(c);
  if (st) return st;
  if (!data) return fail(CKKS_EINVAL, "data is NULL");
  if (n_limbs == 0 || batch == 0) return fail(CKKS_ERANGE, "n_limbs and batch must be positive");
  if ((uint64_t)first + n_limbs > c->h.L + c->h.K)
    return fail(CKKS_ERANGE, "limbs %u..%u beyond the chain of %u primes", first, first + n_limbs - 1, c->h.L + c->h.K);
  if (batch > 65535 || n_limbs > 65535) return fail(CKKS_ERANGE, "batch / n_limbs above 65535");
  return check_device(c);
}

ckks_status ckks_ntt_fwd(const ckks_ctx* c, uint32_t* data, uint32_t first_prime, uint32_t n_limbs, uint32_t batch,
                         void* stream) {
  ckks_status st = ntt_common(c, data, first_prime, n_limbs, batch);
  if (st) return st;
  hipStream_t s = (hipStream_t)stream;
  const uint64_t N = c->h.n;
  ckks::ColArgs ca{data, (uint64_t)n_limbs * N, first_prime, n_limbs};
  ckks_ctx* cm = const_cast<ckks_ctx*>(c);
  hipError_t e;
  {
    ProfScope p(cm, CKKS_K_COL, s);
    e = ckks::launch_col(c->d, ca, true, false, batch, s);
  }
  if (e != hipSuccess) return hip_status(e, "column pass");
  ckks::RowArgs r{};
  r.src = data;
  r.dst = data;
  r.src_item_stride = r.dst_item_stride = (uint64_t)n_limbs * N;
  r.prime0 = first_prime;
  r.n_limbs = n_limbs;
  ProfScope p(cm, CKKS_K_ROW, s);
  return hip_status(ckks::launch_row(c->d, r, true, batch, s), "row pass");
}

ckks_status ckks_ntt_inv(const ckks_ctx* c, uint32_t* data, uint32_t first_prime, uint32_t n_limbs, uint32_t batch,
                         void* stream) {
  ckks_status st = ntt_common(c, data, first_prime, n_limbs, batch);
  if (st) return st;
  hipStream_t s = (hipStream_t)stream;
  const uint64_t N = c->h.n;
  ckks::RowArgs r{};
  r.src = data;
  r.dst = data;
  r.src_item_stride = r.dst_item_stride = (uint64_t)n_limbs * N;
  r.prime0 = first_prime;
  r.n_limbs = n_limbs;
  ckks_ctx* cm = const_cast<ckks_ctx*>(c);
  hipError_t e;
  {
    ProfScope p(cm, CKKS_K_ROW, s);
    e = ckks::launch_row(c->d, r, false, batch, s);
  }
  if (e != hipSuccess) return hip_status(e, "row pass");
  ckks::ColArgs ca{data, (uint64_t)n_limbs * N, first_prime, n_limbs};
  ProfScope p(cm, CKKS_K_COL, s);
  return hip_status(ckks::launch_col(c->d, ca, false, true, batch, s), "column pass");
}

ckks_status ckks_modup(const ckks_ctx* cc, const uint32_t* c1, uint32_t level, uint32_t* digits, uint32_t batch,
                       void* stream) {
  ckks_ctx* c = const_cast<ckks_ctx*>(cc);
  ckks_status st = check_ctx(c);
  if (st) return st;
  if (!c1 || !digits) return fail(CKKS_EINVAL, "c1 or digits is NULL");
  if ((st = check_level(c, level)) || (st = check_batch(c, batch))) return st;
  const Host& h = c->h;
  const uint64_t N = h.n, El = level + h.K;
  if (overlaps(c1, (uint64_t)batch * level * N, digits, (uint64_t)batch * digits_at(h, level) * El * N))
    return fail(CKKS_EINVAL, "digits overlaps c1");
  if ((st = check_device(c))) return st;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = run_modup(c, c1, (uint64_t)level * N, level, batch, s);
  if (e != hipSuccess) return hip_status(e, "ModUp");
  const uint32_t d = digits_at(h, level);
  for (uint32_t j = 0; j < d; ++j) {
    ckks::RowArgs r{};
    r.src = c->ext + (uint64_t)j * (h.L + h.K) * N;
    r.src_item_stride = (uint64_t)h.dnum * (h.L + h.K) * N;
    r.dst = digits + (uint64_t)j * El * N;
    r.dst_item_stride = (uint64_t)d * El * N;
    r.prime0 = 0;
    r.n_limbs = (uint32_t)El;
    r.own_lo = j * h.alpha;
    r.own_n = std::min(h.alpha, level - j * h.alpha);
    r.own_src = c1;
    r.own_item_stride = (uint64_t)level * N;
    r.level = level;
    {
      ProfScope p(c, CKKS_K_ROW, s);
      e = ckks::launch_row(c->d, r, true, batch, s);
    }
    if (e != hipSuccess) return hip_status(e, "ModUp row pass");
  }
  return ok();
}

ckks_status ckks_moddown(const ckks_ctx* cc, const uint32_t* x, uint32_t level, uint32_t* out, uint32_t batch,
                         void* stream) {
  ckks_ctx* c = const_cast<ckks_ctx*>(cc);
  ckks_status st = check_ctx(c);
  if (st) return st;
  if (!x || !out) return fail(CKKS_EINVAL, "x or out is NULL");
  if ((st = check_level(c, level)) || (st = check_batch(c, batch))) return st;
  const uint64_t N = c->h.n;
  if (overlaps(x, (uint64_t)batch * (level + c->h.K) * N, out, (uint64_t)batch * level * N))
    return fail(CKKS_EINVAL, "out overlaps x");
  if ((st = check_device(c))) return st;
  return hip_status(run_moddown(c, x, (uint64_t)(level + c->h.K) * N, level, out, (uint64_t)level * N, batch,
                                (hipStream_t)stream),
                    "ModDown");
}

ckks_status ckks_keyswitch(const ckks_ctx* cc, const uint32_t* ct, uint32_t level, const uint32_t* key_b,
                           const uint8_t* key_seed, const uint32_t* key_a, uint32_t galois_elt, uint32_t* out,
                           uint32_t batch, void* stream) {
  ckks_ctx* c = const_cast<ckks_ctx*>(cc);
  ckks_status st = check_ctx(c);
  if (st) return st;
  if ((st = check_keyswitch_args(c, ct, level, key_b, key_seed, key_a, galois_elt, out, batch)) ||
      (st = check_batch(c, batch)) || (st = check_device(c)))
    return st;
  return keyswitch_run(c, ct, level, key_b, key_seed, key_a, galois_elt, out, batch, (hipStream_t)stream, nullptr);
}

ckks_status ckks_keyswitch_noalloc(const ckks_ctx* cc, const uint32_t* ct, uint32_t level, const uint32_t* key_b,
                                   const uint8_t* key_seed, const uint32_t* key_a, uint32_t galois_elt,
                                   uint32_t* out, uint32_t batch, void* stream) {
  ckks_ctx* c = const_cast<ckks_ctx*>(cc);
  ckks_status st = check_ctx(c);
  if (st) return st;
  if ((st = check_keyswitch_args(c, ct, level, key_b, key_seed, key_a, galois_elt, out, batch))) return st;
  if (batch < 1) return fail(CKKS_ERANGE, "batch must be positive");
  const Host& h = c->h;
  const uint64_t N = h.n, d = digits_at(h, level), E = h.L + h.K;
  // per ciphertext: rowtmp level limbs, ext d_l * (L+K), tmpP 2K, conv 2 * level
  const uint64_t per_item = (level + d * E + 2ull * h.K + 2ull * level) * N;
  const uint64_t need = per_item * batch * sizeof(uint32_t);
  if (need > ckks::kScratchBytes)
    return fail(CKKS_ERANGE, "batch %u at level %u needs %llu bytes of scratch, above the %llu-byte maximum", batch,
                level, (unsigned long long)need, (unsigned long long)ckks::kScratchBytes);
  if ((st = check_device(c))) return st;
  uint32_t* sp = ckks::scratch_ptr(c->device);
  if (!sp) return fail(CKKS_EHIP, "the static scratch array has no device address on device %d: %s", c->device,
                       ckks::scratch_error(c->device));
  Ws w{};
  w.rowtmp = sp;
  w.ext = w.rowtmp + (uint64_t)batch * level * N;
  w.ext_item = d * E * N;
  w.tmpP = w.ext + (uint64_t)batch * w.ext_item;
  w.conv = w.tmpP + (uint64_t)batch * 2 * h.K * N;
  return keyswitch_run(c, ct, level, key_b, key_seed, key_a, galois_elt, out, batch, (hipStream_t)stream, &w);
}

}  // extern "C"

namespace {

// Rescale of `items` polynomials [level][N] (NTT domain), consecutive at stride level*N,
// into out [level-1][N] at stride (level-1)*N: INTT of limb level-1 (row pass and
// column pass), its coefficients reduced modulo each q_i and column-transformed
// under q_i (one broadcast column pass), then the row NTT fused with
// (c_i - .) * q_{level-1}^-1.  Uses ctx->rowtmp and ctx->conv.
hipError_t run_rescale(ckks_ctx* c, const uint32_t* src, uint32_t level, uint32_t* out, uint32_t items,
                       hipStream_t s) {
  const Host& h = c->h;
  const uint64_t N = h.n;
  ckks::RowArgs r{};
  r.src = src + (uint64_t)(level - 1) * N;
  r.src_item_stride = (uint64_t)level * N;
  r.dst = c->rowtmp;
  r.dst_item_stride = N;
  r.prime0 = level - 1;
  r.n_limbs = 1;
  hipError_t e;
  {
    ProfScope p(c, CKKS_K_ROW, s);
    e = ckks::launch_row(c->d, r, false, items, s);
  }
  if (e != hipSuccess) return e;
  {  // column INTT (with N^-1) of the dropped limb: rowtmp now holds its coefficients
    ckks::ColArgs ca{c->rowtmp, N, level - 1, 1, nullptr, 0};
    ProfScope p(c, CKKS_K_RESCALE_CONV, s);
    e = ckks::launch_col(c->d, ca, false, true, items, s);
  }
  if (e != hipSuccess) return e;
  {  // those coefficients modulo each q_i, column NTT under q_i
    ckks::ColArgs cb{c->conv, (uint64_t)(level - 1) * N, 0, level - 1, c->rowtmp, N};
    ProfScope p(c, CKKS_K_RESCALE_CONV, s);
    e = ckks::launch_col(c->d, cb, true, false, items, s);
  }
  if (e != hipSuccess) return e;
  ckks::RowArgs f{};
  f.src = c->conv;
  f.src_item_stride = (uint64_t)(level - 1) * N;
  f.dst = out;
  f.dst_item_stride = (uint64_t)(level - 1) * N;
  f.prime0 = 0;
  f.n_limbs = level - 1;
  f.cmb = src;
  f.cmb_item_stride = (uint64_t)level * N;
  f.cmb_factor = c->d.rs_inv + (size_t)level * h.L;
  ProfScope p(c, CKKS_K_RESCALE_FINAL, s);
  return ckks::launch_row(c->d, f, true, items, s);
}


}  // namespace

extern "C" {

ckks_status ckks_rescale(const ckks_ctx* cc, const uint32_t* ct, uint32_t level, uint32_t* out, uint32_t batch,
                         void* stream) {
  ckks_ctx* c = const_cast<ckks_ctx*>(cc);
  ckks_status st = check_ctx(c);
  if (st) return st;
  if (!ct || !out) return fail(CKKS_EINVAL, "ct or out is NULL");
  if ((st = check_level(c, level)) || (st = check_batch(c, batch))) return st;
  if (level < 2) return fail(CKKS_ERANGE, "rescale needs level >= 2 (got %u)", level);
  const uint64_t N = c->h.n;
  if (overlaps(ct, (uint64_t)batch * 2 * level * N, out, (uint64_t)batch * 2 * (level - 1) * N))
    return fail(CKKS_EINVAL, "out overlaps ct");
  if ((st = check_device(c))) return st;
  return hip_status(run_rescale(c, ct, level, out, 2 * batch, (hipStream_t)stream), "rescale");
}

ckks_status ckks_mul_relin_rescale(const ckks_ctx* cc, const uint32_t* x, const uint32_t* y, uint32_t level,
                                   const uint32_t* key_b, const uint8_t* key_seed, const uint32_t* key_a,
                                   uint32_t* out, uint32_t batch, void* stream) {
  ckks_ctx* c = const_cast<ckks_ctx*>(cc);
  ckks_status st = check_ctx(c);
  if (st) return st;
  if (!x || !y || !key_b || !out) return fail(CKKS_EINVAL, "x, y, key_b or out is NULL");
  if (!key_a && !key_seed) return fail(CKKS_EINVAL, "need key_a or key_seed");
  if ((st = check_level(c, level)) || (st = check_batch(c, batch))) return st;
  if (level < 2) return fail(CKKS_ERANGE, "rescale needs level >= 2 (got %u)", level);
  if ((st = check_device(c))) return st;
  hipStream_t s = (hipStream_t)stream;
  const uint64_t N = c->h.n, ln = (uint64_t)level * N;
  uint32_t* pair = c->tens;  // [B][2][l][N]: the relinearised (e0, e1)
  // The tensor product (d0, d1, d2) = (x0 y0, x0 y1 + x1 y0, x1 y1) is never stored:
  // ModUp's row pass forms d2, the final inner-product pass forms d0, d1 and d2's own limbs.
  hipError_t e = run_modup(c, x + ln, 2 * ln, level, batch, s, nullptr, y + ln);
  if (e != hipSuccess) return hip_status(e, "ModUp");
  ckks::KeyRef k{};
  k.b = key_b;
  k.a = key_a;
  if (!key_a) seed_words(key_seed, k.seed);
  k.galois = 1;
  e = run_ip_moddown(c, x, 2 * ln, (uint64_t)c->h.dnum * (c->h.L + c->h.K) * N, level, batch, 1, &k, pair, false,
                     s, false, y);
  if (e != hipSuccess) return hip_status(e, "relinearisation");
  return hip_status(run_rescale(c, pair, level, out, 2 * batch, s), "rescale");
}

ckks_status ckks_linear_transform_bsgs(const ckks_ctx* cc, const uint32_t* ct, uint32_t level, uint32_t n1,
                                       uint32_t n2, const ckks_rot_key* baby, const ckks_rot_key* giant,
                                       const uint32_t* diags, uint32_t* out, void* stream) {
  ckks_ctx* c = const_cast<ckks_ctx*>(cc);
  ckks_status st = check_ctx(c);
  if (st) return st;
  if (!ct || !diags || !out) return fail(CKKS_EINVAL, "ct, diags or out is NULL");
  if ((st = check_level(c, level))) return st;
  if (n1 < 1 || n1 > ckks::kMaxGroup) return fail(CKKS_ERANGE, "n1 %u outside 1..%u", n1, ckks::kMaxGroup);
  if (n2 < 1 || n2 > ckks::kMaxGiant) return fail(CKKS_ERANGE, "n2 %u outside 1..%u", n2, ckks::kMaxGiant);
  if ((n1 > 1 && !baby) || (n2 > 1 && !giant)) return fail(CKKS_EINVAL, "baby or giant key array is NULL");
  for (uint32_t k = 0; k + 1 < n1 + n2 - 1; ++k) {
    const ckks_rot_key& key = k + 1 < n1 ? baby[k] : giant[k + 1 - n1];
    if (!key.key_b) return fail(CKKS_EINVAL, "key %u has no key_b", k);
    if ((st = check_galois(c, key.galois_elt))) return st;
  }
  const Host& h = c->h;
  const uint64_t N = h.n, El = level + h.K;
  // workspace: R (baby steps) and S (diagonal sums) in ctx->tens, then the giant-step
  // inputs over R, the giant-step outputs over S
  const uint64_t r_words = (uint64_t)(n1 - 1) * 2 * El * N, s_words = (uint64_t)n2 * 2 * El * N,
                 ct_words = (uint64_t)n2 * 2 * level * N;
  const uint64_t B = c->max_batch ? c->max_batch : 4096;
  if (std::max(r_words, ct_words) + s_words > B * 3 * h.L * N || 2 * n2 * h.K > B * std::max(std::max(h.L, h.K), 2u) ||
      n2 > B)
    return fail(CKKS_ERANGE, "a %u x %u transform needs a larger context (max_batch %u)", n1, n2, c->max_batch);
  if ((st = check_device(c))) return st;
  hipStream_t s = (hipStream_t)stream;
  uint32_t* rbuf = c->tens;
  uint32_t* sbuf = c->tens + std::max(r_words, ct_words);
  uint32_t* ctbuf = c->tens;
  hipError_t e;
  if (n1 > 1) {
    e = run_hoisted_digits(c, ct, level, s);
    if (e != hipSuccess) return hip_status(e, "hoisted ModUp");
    ckks::ExtArgs a{};
    a.level = level;
    a.nd = digits_at(h, level);
    a.ext = c->ext;
    a.c0 = ct;
    a.out = rbuf;
    a.regen_blocks = c->regen_blocks;
    a.n_keys = n1 - 1;
    a.items = 1;
    for (uint32_t k = 0; k + 1 < n1; ++k) {
      a.key[k] = ckks::KeyRef{};
      a.key[k].b = baby[k].key_b;
      a.key[k].a = baby[k].key_a;
      if (!baby[k].key_a) seed_words(baby[k].key_seed, a.key[k].seed);
      a.key[k].galois = baby[k].galois_elt;
    }
    ProfScope p(c, CKKS_K_BABY, s);
    e = ckks::launch_rot_ext(c->d, a, s);
    if (e != hipSuccess) return hip_status(e, "baby steps");
  }
  {
    ckks::DiagArgs d{level, n1, n2, ct, rbuf, diags, sbuf};
    ProfScope p(c, CKKS_K_DIAG, s);
    e = ckks::launch_diag_acc(c->d, d, s);
  }
  if (e != hipSuccess) return hip_status(e, "diagonal sums");
  if (n2 == 1) return hip_status(run_moddown(c, sbuf, El * N, level, out, (uint64_t)level * N, 2, s), "ModDown");
  e = run_moddown(c, sbuf, El * N, level, ctbuf, (uint64_t)level * N, 2 * n2, s);
  if (e != hipSuccess) return hip_status(e, "ModDown");
  ckks::SumArgs sum{};
  sum.n_src = n2;
  sum.words = 2ull * level * N;
  sum.src[0] = ctbuf;
  // giant steps 1..n2-1: key-switches of ModDown(S_j), each with its own key, in one
  // ModUp batch and one group of key-using launches; outputs over S
  ckks::KeyRef keys[ckks::kMaxGroup];
  for (uint32_t j = 1; j < n2; ++j) {
    ckks::KeyRef& k = keys[j - 1];
    k = ckks::KeyRef{};
    k.b = giant[j - 1].key_b;
    k.a = giant[j - 1].key_a;
    if (!k.a) seed_words(giant[j - 1].key_seed, k.seed);
    k.galois = giant[j - 1].galois_elt;
    k.ct = ctbuf + (uint64_t)j * 2 * level * N;
    k.out = sbuf + (uint64_t)j * 2 * level * N;
    sum.src[j] = k.out;
  }
  e = run_modup(c, ctbuf + 2ull * level * N + (uint64_t)level * N, 2ull * level * N, level, n2 - 1, s);
  if (e != hipSuccess) return hip_status(e, "giant-step ModUp");
  e = run_ip_moddown(c, nullptr, 0, (uint64_t)h.dnum * (h.L + h.K) * N, level, 1, n2 - 1, keys, nullptr, false, s,
                     true);
  if (e != hipSuccess) return hip_status(e, "giant-step key-switches");
  ProfScope p(c, CKKS_K_DIAG, s);
  return hip_status(ckks::launch_sum(c->d, sum, out, level, s), "sum of giant steps");
}

ckks_status ckks_keyswitch_hoisted(const ckks_ctx* cc, const uint32_t* ct, uint32_t level, uint32_t n_keys,
                                   const uint32_t* const* key_b, const uint8_t* key_seeds,
                                   const uint32_t* const* key_a, const uint32_t* galois_elts, uint32_t* out,
                                   void* stream) {
  ckks_ctx* c = const_cast<ckks_ctx*>(cc);
  ckks_status st = check_ctx(c);
  if (st) return st;
  if (!ct || !key_b || !galois_elts || !out) return fail(CKKS_EINVAL, "ct, key_b, galois_elts or out is NULL");
  if ((st = check_level(c, level))) return st;
  if (n_keys < 1 || n_keys > ckks::kMaxHoist) return fail(CKKS_ERANGE, "n_keys %u outside 1..%u", n_keys, ckks::kMaxHoist);
  for (uint32_t k = 0; k < n_keys; ++k) {
    if (!key_b[k]) return fail(CKKS_EINVAL, "key_b[%u] is NULL", k);
    if ((!key_a || !key_a[k]) && !key_seeds) return fail(CKKS_EINVAL, "key %u has neither key_a nor a seed", k);
    if ((st = check_galois(c, galois_elts[k]))) return st;
  }
  for (uint32_t k = 0; k < n_keys; ++k)
    if ((st = check_keyswitch_out(c, ct, level, 1, key_b[k], key_a ? key_a[k] : nullptr, out,
                                  (uint64_t)n_keys * 2 * level * c->h.n)))
      return st;
  if ((st = check_device(c))) return st;
  hipStream_t s = (hipStream_t)stream;
  const uint64_t N = c->h.n;
  hipError_t e = run_hoisted_digits(c, ct, level, s);
  if (e != hipSuccess) return hip_status(e, "hoisted ModUp");
  const uint32_t chunk = std::min<uint32_t>(c->max_batch, ckks::kMaxGroup);
  for (uint32_t k0 = 0; k0 < n_keys; k0 += chunk) {
    const uint32_t nk = std::min(chunk, n_keys - k0);
    ckks::KeyRef keys[ckks::kMaxGroup];
    for (uint32_t k = 0; k < nk; ++k) {
      keys[k] = ckks::KeyRef{};
      keys[k].b = key_b[k0 + k];
      keys[k].a = key_a ? key_a[k0 + k] : nullptr;
      if (!keys[k].a) seed_words(key_seeds + 32 * (k0 + k), keys[k].seed);
      keys[k].galois = galois_elts[k0 + k];
    }
    e = run_ip_moddown(c, ct, 0, 0, level, 1, nk, keys, out + (uint64_t)k0 * 2 * level * N, true, s);
    if (e != hipSuccess) return hip_status(e, "inner product / ModDown");
  }
  return ok();
}

ckks_status ckks_keyswitch_multi(const ckks_ctx* cc, uint32_t n_items, const ckks_ks_item* items, void* stream) {
  ckks_ctx* c = const_cast<ckks_ctx*>(cc);
  ckks_status st = check_ctx(c);
  if (st) return st;
  if (n_items == 0) return ok();
  if (!items) return fail(CKKS_EINVAL, "items is NULL");
  for (uint32_t i = 0; i < n_items; ++i) {
    const ckks_ks_item& it = items[i];
    if (!it.ct || !it.out || !it.key_b) return fail(CKKS_EINVAL, "item %u: ct, out or key_b is NULL", i);
    if ((st = check_level(c, it.level)) || (st = check_galois(c, it.galois_elt))) {
      std::string m = g_err;
      return fail(st, "item %u: %s", i, m.c_str());
    }
  }
  {  // outputs overlap neither each other nor any input (the items run concurrently)
    const uint64_t nb = 2ull * c->h.n * sizeof(uint32_t);
    std::vector<std::pair<uintptr_t, uintptr_t>> outs(n_items);
    for (uint32_t i = 0; i < n_items; ++i)
      outs[i] = {(uintptr_t)items[i].out, (uintptr_t)items[i].out + nb * items[i].level};
    std::sort(outs.begin(), outs.end());
    for (uint32_t i = 1; i < n_items; ++i)
      if (outs[i].first < outs[i - 1].second) return fail(CKKS_EINVAL, "the outputs of two items overlap");
    for (uint32_t i = 0; i < n_items; ++i) {
      const uintptr_t lo = (uintptr_t)items[i].ct, hi = lo + nb * items[i].level;
      auto it = std::lower_bound(outs.begin(), outs.end(), std::make_pair(hi, (uintptr_t)0));
      if (it != outs.begin() && std::prev(it)->second > lo)
        return fail(CKKS_EINVAL, "item %u: ct overlaps an item's out", i);
    }
  }
  if ((st = check_device(c))) return st;
  hipStream_t s = (hipStream_t)stream;
  const Host& h = c->h;
  const uint64_t N = h.n;
  const uint32_t B = c->max_batch, chunk = std::min<uint32_t>(B, ckks::kMaxGroup);
  // Launch sequences: items of equal level, in chunks of at most `chunk`, in the
  // order of each level's first item.
  struct Task {
    uint32_t level, m, idx[ckks::kMaxGroup];
  };
  std::vector<Task> tasks;
  {
    std::vector<bool> done(n_items, false);
    for (uint32_t i0 = 0; i0 < n_items; ++i0) {
      if (done[i0]) continue;
      Task t{};
      t.level = items[i0].level;
      for (uint32_t i = i0; i < n_items; ++i) {
        if (done[i] || items[i].level != t.level) continue;
        done[i] = true;
        t.idx[t.m++] = i;
        if (t.m == chunk) {
          tasks.push_back(t);
          t.m = 0;
        }
      }
      if (t.m) tasks.push_back(t);
    }
  }
  // The sequences are independent apart from the workspace.  They take item ranges
  // of the workspace in turn (wrapping round) and are dealt out to the caller's
  // stream and the side streams in turn; a sequence whose range was last used by a
  // sequence on another stream waits for that sequence's event.  The caller's
  // stream finally waits for every side stream, so later calls on it are ordered
  // after the whole call.
  const uint32_t S = tasks.size() > 1 && B > 1 ? std::min<uint32_t>(kMultiStreams, (uint32_t)tasks.size()) : 1;
  if (S > 1 && (c->side.size() + 1 < S || c->task_ev.size() < tasks.size() + 1)) {
    // created on the context's device, whichever is current
    int cur = c->device;
    if (hipGetDevice(&cur) != hipSuccess || (cur != c->device && hipSetDevice(c->device) != hipSuccess))
      return fail(CKKS_EHIP, "cannot select the context's device");
    hipError_t ce = hipSuccess;
    while (c->side.size() + 1 < S && ce == hipSuccess) {
      hipStream_t st;
      if ((ce = hipStreamCreateWithFlags(&st, hipStreamNonBlocking)) == hipSuccess) c->side.push_back(st);
    }
    while (c->task_ev.size() < tasks.size() + 1 && ce == hipSuccess) {
      hipEvent_t ev;
      if ((ce = hipEventCreateWithFlags(&ev, hipEventDisableTiming)) == hipSuccess) c->task_ev.push_back(ev);
    }
    if (cur != c->device) (void)hipSetDevice(cur);
    if (ce != hipSuccess) return hip_status(ce, "creating the side streams and events");
  }
  auto stream_of = [&](uint32_t k) { return k == 0 ? s : c->side[k - 1]; };
  hipError_t e = hipSuccess;
  if (S > 1) {  // fork: side streams start after the caller's earlier work
    hipEvent_t fork = c->task_ev[tasks.size()];
    if ((e = hipEventRecord(fork, s)) != hipSuccess) return hip_status(e, "hipEventRecord");
    for (uint32_t k = 1; k < S; ++k)
      if ((e = hipStreamWaitEvent(stream_of(k), fork, 0)) != hipSuccess) return hip_status(e, "hipStreamWaitEvent");
  }
  std::vector<int> owner(B, -1);  // last sequence that used each workspace item
  uint32_t pos = 0;
  ckks_status bad = CKKS_OK;
  for (uint32_t ti = 0; ti < tasks.size() && bad == CKKS_OK; ++ti) {
    const Task& t = tasks[ti];
    const uint32_t k = ti % S, level = t.level, m = t.m;
    hipStream_t st = stream_of(k);
    if (pos + m > B) pos = 0;
    if (S > 1) {
      int last[kMultiStreams];  // newest earlier sequence per other stream on this range
      for (uint32_t j = 0; j < S; ++j) last[j] = -1;
      for (uint32_t w = pos; w < pos + m; ++w)
        if (owner[w] >= 0 && (uint32_t)owner[w] % S != k)
          last[owner[w] % S] = std::max(last[owner[w] % S], owner[w]);
      for (uint32_t j = 0; j < S; ++j)
        if (last[j] >= 0 && (e = hipStreamWaitEvent(st, c->task_ev[last[j]], 0)) != hipSuccess) break;
      if (e != hipSuccess) {
        bad = hip_status(e, "hipStreamWaitEvent");
        break;
      }
    }
    const uint32_t* c1s[ckks::kMaxGroup];
    ckks::KeyRef keys[ckks::kMaxGroup];
    for (uint32_t j = 0; j < m; ++j) {
      const ckks_ks_item& it = items[t.idx[j]];
      c1s[j] = it.ct + (uint64_t)level * N;
      keys[j] = ckks::KeyRef{};
      keys[j].b = it.key_b;
      keys[j].a = it.key_a;
      if (!it.key_a) seed_words(it.key_seed, keys[j].seed);
      keys[j].galois = it.galois_elt;
      keys[j].ct = it.ct;
      keys[j].out = it.out;
    }
    {
      WsView view(c, pos);
      if ((e = run_modup(c, nullptr, 0, level, m, st, c1s)) != hipSuccess) {
        bad = hip_status(e, "ModUp");
      } else if ((e = run_ip_moddown(c, nullptr, 0, (uint64_t)h.dnum * (h.L + h.K) * N, level, 1, m, keys, nullptr,
                                     false, st, true)) != hipSuccess) {
        bad = hip_status(e, "inner product / ModDown");
      }
    }
    // recorded after a failed launch too, so that the join below stays well formed
    if (S > 1 && (e = hipEventRecord(c->task_ev[ti], st)) != hipSuccess && bad == CKKS_OK)
      bad = hip_status(e, "hipEventRecord");
    for (uint32_t w = pos; w < pos + m; ++w) owner[w] = (int)ti;
    pos += m;
  }
  if (bad != CKKS_OK) {  // keep the message of the first failure
    std::string msg = g_err;
    for (uint32_t k = 1; k < S; ++k) (void)hipStreamSynchronize(stream_of(k));
    g_err = msg;
    return bad;
  }
  // join: the newest sequence of each side stream
  for (uint32_t k = 1; k < S; ++k) {
    uint32_t ti = (uint32_t)tasks.size() - 1;
    while (ti % S != k) --ti;
    if ((e = hipStreamWaitEvent(s, c->task_ev[ti], 0)) != hipSuccess) return hip_status(e, "hipStreamWaitEvent");
  }
  return ok();
}

ckks_status ckks_expand_a(const ckks_ctx* c, const uint8_t* key_seed, uint32_t* key_a, void* stream) {
  ckks_status st = check_ctx(c);
  if (st) return st;
  if (!key_seed || !key_a) return fail(CKKS_EINVAL, "key_seed or key_a is NULL");
  if ((st = check_device(c))) return st;
  uint32_t w[8];
  seed_words(key_seed, w);
  ProfScope p(const_cast<ckks_ctx*>(c), CKKS_K_EXPAND, (hipStream_t)stream);
  return hip_status(ckks::launch_expand(c->d, w, key_a, c->regen_blocks, (hipStream_t)stream), "expand");
}

ckks_status ckks_profile_enable(ckks_ctx* c, int enable) {
  ckks_status st = check_ctx(c);
  if (st || (st = check_device(c))) return st;
  if (enable) {
    if (c->prof_ev.empty()) {
      c->prof_ev.resize(2 * kProfMax);
      for (auto& e : c->prof_ev)
        if (hipEventCreate(&e) != hipSuccess) return fail(CKKS_EHIP, "hipEventCreate failed");
    }
    c->prof_cls.clear();
  }
  c->prof_on = enable != 0;
  return ok();
}

ckks_status ckks_profile_read(ckks_ctx* c, double* ms_out, uint32_t* launches_out, uint32_t n_classes) {
  ckks_status st = check_ctx(c);
  if (st || (st = check_device(c))) return st;
  if (!ms_out) return fail(CKKS_EINVAL, "ms_out is NULL");
  for (uint32_t k = 0; k < n_classes; ++k) {
    ms_out[k] = 0.0;
    if (launches_out) launches_out[k] = 0;
  }
  for (size_t r = 0; r < c->prof_cls.size(); ++r) {
    const int k = c->prof_cls[r];
    if (hipEventSynchronize(c->prof_ev[2 * r + 1]) != hipSuccess) return fail(CKKS_EHIP, "hipEventSynchronize failed");
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, c->prof_ev[2 * r], c->prof_ev[2 * r + 1]) != hipSuccess)
      return fail(CKKS_EHIP, "hipEventElapsedTime failed");
    if ((uint32_t)k < n_classes) {
      ms_out[k] += ms;
      if (launches_out) launches_out[k] += 1;
    }
  }
  return ok();
}

}  // extern "C"
