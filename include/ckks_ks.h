/* ckks_ks.h - RNS-CKKS hybrid key-switching on one AMD Instinct MI355X (gfx950).
 *
 * The method: one half of a key-switching key is uniformly random, so only its
 * 32-byte seed is kept and the kernels that consume the key rebuild that half
 * with ChaCha12 in counter mode, which cuts the key's memory in two; the chain is
 * RNS CKKS over 32-bit primes (Perseus summary on ai4snews, "Interpretation"
 * paragraph 2; the Perseus abstract names this in-kernel key regeneration as its
 * backend-level change).  The rest of the path is textbook hybrid key-switching
 * (Han and Ki, CT-RSA 2020) with fast base conversion (Bajard et al., SAC 2016)
 * and merged-twist negacyclic NTTs (Longa and Naehrig 2016).
 *
 * Conventions shared by every call
 *  - Pointers are DEVICE pointers unless marked (host).  Every residue array is
 *    uint32_t, limb-major: [.. ][limb][N], coefficient n of limb i at i*N + n.
 *  - Residues are canonical, in [0, q), on input and output.  Polynomials are in
 *    the NTT domain (bit-reversed evaluation order: entry j holds the value at
 *    psi^(2*brv(j)+1), psi the smallest primitive 2N-th root mod q) except the
 *    output of ckks_ntt_inv and the input of ckks_ntt_fwd.
 *  - The chain is q_0..q_{L-1} (ciphertext primes) then p_0..p_{K-1} (special
 *    primes); absolute prime index t runs over all L+K.  Level l means the
 *    ciphertext primes q_0..q_{l-1} are active.  Digit width alpha = ceil(L/dnum);
 *    digit j at level l holds primes j*alpha .. min((j+1)*alpha, l)-1 and there
 *    are d_l = ceil(l/alpha) digits.
 *  - Keys: key_b and key_a are [dnum][L+K][N], row (j, t) for digit j and
 *    absolute prime t, so one key serves every level.  The a-half is exactly the
 *    ChaCha12 expansion of the key's 32-byte seed (see ckks_expand_a).
 *  - Every call is asynchronous on `stream` (a hipStream_t passed as void*; NULL
 *    is the default stream) and never synchronises the host (the one exception:
 *    ckks_keyswitch_multi waits for its internal streams when a launch fails
 *    part-way, before it returns the error).  Calls on one
 *    context share its workspace: calls on different streams must not overlap
 *    (use one context per stream).  Output buffers must not alias inputs.
 *  - Arguments are validated before anything is launched; on failure nothing is
 *    launched and the status says why (ckks_last_error() holds a message for the
 *    calling thread).  The library never allocates device memory outside
 *    ckks_ctx_create.
 */
#ifndef CKKS_KS_H
#define CKKS_KS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ckks_ctx ckks_ctx;

typedef enum {
  CKKS_OK = 0,
  CKKS_EINVAL = -1,        /* NULL pointer, bad enum, inconsistent sizes */
  CKKS_ERANGE = -2,        /* level, batch, Galois element or prime out of range */
  CKKS_ENOMEM = -3,        /* device allocation failed in ckks_ctx_create */
  CKKS_EHIP = -4,          /* a HIP runtime call or kernel launch failed */
  CKKS_EUNSUPPORTED = -5   /* parameters this build does not implement */
} ckks_status;

/* Thread-local description of the last failure on the calling thread ("" if none). */
const char *ckks_last_error(void);

/* Build identity, for callers that must not run a stale library: the first 16
 * hex digits of the sha256 of the sources the library was compiled from (the
 * kernel, host and header files, by name and content), fixed at build time.  The
 * Python binding compares it with the sources beside it and refuses a mismatch.
 * A static string; never fails. */
const char *ckks_build_id(void);

/* The `count` largest primes q < 2^bits with q = 1 mod 2^(log_n+1), in descending
 * order, written to out_host[0..count) (host).  This is the chain reading used
 * throughout: the pages fix only "a 32-bit RNS CKKS chain".  bits in 20..32. */
ckks_status ckks_chain_primes(uint32_t log_n, uint32_t bits, uint32_t count, uint32_t *out_host);

/* Create a context for ring degree N = 2^log_n (12 <= log_n <= 16), chain
 * primes[0..num_q+num_p) (host; ciphertext primes first), dnum digits, and a
 * workspace for up to max_batch ciphertexts (or hoisted keys) per call at level
 * num_q.  Every prime must be prime, < 2^32, = 1 mod 2N, and all distinct;
 * num_p >= ceil(num_q/dnum) is required (the special modulus covers a digit).
 * max_batch = 0 creates a host-only context: every table is computed and every
 * argument check works, but no HIP call is made and compute calls return
 * CKKS_EINVAL.  Errors: EINVAL (NULL), ERANGE (sizes, non-qualifying prime),
 * EUNSUPPORTED (log_n outside 12..16), ENOMEM/EHIP (device setup). */
ckks_status ckks_ctx_create(ckks_ctx **out, uint32_t log_n, uint32_t num_q, uint32_t num_p,
                            uint32_t dnum, const uint32_t *primes, uint32_t max_batch);
void ckks_ctx_destroy(ckks_ctx *ctx);

/* Host copies of what the context derived: the minimal 2N-th root psi_t of every
 * prime (roots_out[L+K]) and the context's sizes. Any output pointer may be NULL. */
ckks_status ckks_ctx_info(const ckks_ctx *ctx, uint32_t *n_out, uint32_t *num_q_out, uint32_t *num_p_out,
                          uint32_t *dnum_out, uint32_t *alpha_out, uint32_t *max_batch_out,
                          uint64_t *workspace_bytes_out, uint32_t *roots_out);

/* Forward negacyclic NTT, in place, of data[batch][n_limbs][N] (coefficients in
 * natural order in, NTT domain out); limb i of each item is taken modulo chain
 * prime first_prime + i.  The pages name the key-switching key and a 32-bit RNS
 * chain (Perseus summary on ai4snews, "Interpretation" paragraph 2) but fix no
 * transform; the reading taken is the textbook one: entry j of the output is the
 * input polynomial evaluated at psi^(2*brv(j)+1), psi the smallest x >= 2 with
 * x^N = -1 mod q (merged-twist Cooley-Tukey, Longa and Naehrig 2016).  data is
 * caller-owned and is overwritten.  Errors: EINVAL (NULL ctx or data, host-only
 * context), ERANGE if first_prime + n_limbs > L+K, or batch or n_limbs is 0. */
ckks_status ckks_ntt_fwd(const ckks_ctx *ctx, uint32_t *data, uint32_t first_prime, uint32_t n_limbs,
                         uint32_t batch, void *stream);
/* Inverse of ckks_ntt_fwd, in place (Gentleman-Sande, includes the factor N^-1):
 * NTT domain in, coefficients out.  Same reading, ownership and errors. */
ckks_status ckks_ntt_inv(const ckks_ctx *ctx, uint32_t *data, uint32_t first_prime, uint32_t n_limbs,
                         uint32_t batch, void *stream);

/* ModUp: extended digits of c1[batch][level][N] (NTT domain).  digits is
 * [batch][d_l][level+K][N]: limb e of digit j is over prime e (e < level) or
 * p_{e-level}; for a prime of digit j it is c1's own limb, otherwise the NTT of
 * the fast base conversion of digit j's coefficients.  The pages give no steps
 * for key-switching beyond its key (Perseus summary on ai4snews, "Interpretation"
 * paragraph 2); the reading taken is hybrid key-switching's ModUp (Han and Ki,
 * CT-RSA 2020) with fast base conversion without overflow correction (Bajard et
 * al., SAC 2016): the multiple u*Q_j (0 <= u < digit size) stays in, and cancels
 * against the key's gadget.  Caller-owned buffers; digits must not overlap c1.
 * Errors: EINVAL (NULL, overlap, host-only context), ERANGE for level outside
 * 1..L or batch outside 1..max_batch. */
ckks_status ckks_modup(const ckks_ctx *ctx, const uint32_t *c1, uint32_t level, uint32_t *digits,
                       uint32_t batch, void *stream);

/* ModDown: out[batch][level][N] = (x_i - NTT(conv_{P->q_i}(INTT(x_P)))) * P^-1 mod q_i for
 * x[batch][level+K][N] (level ciphertext limbs then K special limbs, NTT domain).
 * Reading taken (the pages give no steps): floor-type ModDown of hybrid
 * key-switching (Han and Ki, CT-RSA 2020): no P/2 offset, and the conversion's
 * overflow v*P (0 <= v < K) left in.  out must not overlap x.  Errors: EINVAL
 * (NULL, overlap, host-only context), ERANGE (level, batch). */
ckks_status ckks_moddown(const ckks_ctx *ctx, const uint32_t *x, uint32_t level, uint32_t *out,
                         uint32_t batch, void *stream);

/* Key-switch of ct[batch][2][level][N] (c0 then c1) under one key with Galois
 * element galois_elt (odd, < 2N; 1 = no automorphism):
 *   out = (sigma(c0) + ModDown(sum_j sigma(d_j) * b_j), ModDown(sum_j sigma(d_j) * a_j))
 * with d_j the ModUp digits of c1 and sigma applied in the NTT domain after ModUp.
 * key_a == NULL: the a-half is regenerated in-kernel from key_seed (host, 32
 * bytes); otherwise key_a is the stored a-half and key_seed is ignored (may be
 * NULL).  out must not overlap ct, key_b or key_a.  Errors: EINVAL (NULL
 * ct/key_b/out, both key_a and key_seed NULL, an overlap, host-only context),
 * ERANGE (level, batch, even or out-of-range galois_elt). */
ckks_status ckks_keyswitch(const ckks_ctx *ctx, const uint32_t *ct, uint32_t level, const uint32_t *key_b,
                           const uint8_t *key_seed, const uint32_t *key_a, uint32_t galois_elt,
                           uint32_t *out, uint32_t batch, void *stream);

/* The key-switch of ckks_keyswitch for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): same arguments, same launches, bit-identical results, but
 * its workspace is a static device array of the library (96 MiB per GPU,
 * reserved on each GPU when the first context is created there and held until
 * the process ends) instead of the context's; no call allocates or frees memory.
 * The batch is limited by that array, not by max_batch: batch * (3*level +
 * d_l*(L+K) + 2K) * N * 4 bytes must fit in it (one ciphertext at N = 2^16 with
 * 36 + 12 primes at any level; more at lower levels and smaller rings).  Every
 * call on one GPU uses the same array, so calls that overlap in time on one GPU
 * (other streams, other threads, other contexts) race: serialise them.  No part
 * of the array needs to start at zero; it keeps the last call's contents.
 * Errors: as ckks_keyswitch, ERANGE when the batch does not fit the array, EHIP
 * when the array has no address on the context's device. */
ckks_status ckks_keyswitch_noalloc(const ckks_ctx *ctx, const uint32_t *ct, uint32_t level, const uint32_t *key_b,
                                   const uint8_t *key_seed, const uint32_t *key_a, uint32_t galois_elt,
                                   uint32_t *out, uint32_t batch, void *stream);

/* Hoisted key-switch: one ModUp of ct[2][level][N], then for every key k an
 * inner product and ModDown with (key_b[k], key_a[k] or key_seeds[k], galois_elts[k]);
 * out is [n_keys][2][level][N], bit-identical to n_keys calls of ckks_keyswitch.
 * key_b, galois_elts and key_seeds are host arrays (key_b holds device
 * pointers; key_seeds is 32*n_keys bytes); key_a is NULL (all regenerated) or a
 * host array of device pointers whose NULL entries are regenerated.
 * 1 <= n_keys <= 64; out must not overlap ct or any key.  Errors as ckks_keyswitch. */
ckks_status ckks_keyswitch_hoisted(const ckks_ctx *ctx, const uint32_t *ct, uint32_t level, uint32_t n_keys,
                                   const uint32_t *const *key_b, const uint8_t *key_seeds,
                                   const uint32_t *const *key_a, const uint32_t *galois_elts,
                                   uint32_t *out, void *stream);

/* One ciphertext of a multi-item call: its own level, key and Galois element. */
typedef struct {
  const uint32_t *ct;        /* [2][level][N], NTT domain (device) */
  uint32_t *out;             /* [2][level][N] (device), must not alias any input */
  const uint32_t *key_b;     /* [dnum][L+K][N] (device) */
  const uint32_t *key_a;     /* stored a-half (device) or NULL: regenerate from key_seed */
  uint8_t key_seed[32];      /* ChaCha12 seed of the a-half, used when key_a is NULL */
  uint32_t level;            /* 1..L */
  uint32_t galois_elt;       /* odd, < 2N */
} ckks_ks_item;

/* A stream of independent key-switches (different levels, keys and Galois
 * elements), bit-identical to one ckks_keyswitch call per item with batch 1.
 * Items of equal level are processed together, up to min(16, max_batch) per
 * launch sequence, so a decode-shaped stream does not pay one small launch
 * sequence per ciphertext.  The sequences run concurrently on `stream` and up to
 * three internal streams of the context (default priority, created on the first
 * call that has more than one sequence), each in its own part of the workspace;
 * `stream` waits for all of them before the call returns, so work queued on it
 * afterwards sees every output.  The items must therefore be independent: no
 * item's out may overlap another item's ct or out.  items is a host array.
 * Errors: EINVAL (NULL pointers), ERANGE (an item's level or Galois element),
 * with the item index in ckks_last_error(); nothing is launched if any item is
 * invalid. */
ckks_status ckks_keyswitch_multi(const ckks_ctx *ctx, uint32_t n_items, const ckks_ks_item *items, void *stream);

/* The a-half [dnum][L+K][N] that key_seed (host, 32 bytes) regenerates: the stored
 * variant of a key.  Stream layout: one ChaCha12 sub-stream per (digit j,
 * absolute prime t, tile tau of 1024 coefficients); state = "expand 32-byte k",
 * the seed as 8 little-endian words, block counter from 0, then j, t, tau; words
 * in counter then word order; a word w is accepted iff w < floor(2^32/q_t)*q_t
 * and gives w mod q_t; the k-th accepted word is coefficient tau*1024 + k. */
ckks_status ckks_expand_a(const ckks_ctx *ctx, const uint8_t *key_seed, uint32_t *key_a, void *stream);

/* Rescale by the last active prime: out[batch][2][level-1][N] from
 * ct[batch][2][level][N], both NTT domain, level >= 2.  With the floor convention
 * of ModDown: c_i <- (c_i - NTT_i([INTT_{q_{l-1}}(c_{l-1})] mod q_i)) * q_{l-1}^-1
 * mod q_i for i < l-1, so a coefficient C in [0, Q_l) becomes floor(C / q_{l-1}).
 * The pages name rescaling only as the multiplication depth a CKKS ciphertext
 * spends (EncryptedLLM summary on lpnh, "Core problem" paragraph); the RNS steps
 * are those of Cheon et al., SAC 2018.  out must not overlap ct.
 * Errors: EINVAL (NULL, overlap), ERANGE (level outside 2..L, batch). */
ckks_status ckks_rescale(const ckks_ctx *ctx, const uint32_t *ct, uint32_t level, uint32_t *out, uint32_t batch,
                         void *stream);

/* Multiply, relinearise and rescale: out[batch][2][level-1][N] =
 * Rescale(e0, e1) with (d0, d1, d2) = x (x) y, the NTT-domain tensor product
 * (d0 = x0*y0, d1 = x0*y1 + x1*y0, d2 = x1*y1 mod q_i), and (e0, e1) =
 * (d0 + ModDown(acc_b), d1 + ModDown(acc_a)) the key-switch of d2 (ModUp, inner
 * product, ModDown exactly as ckks_keyswitch with Galois element 1).  The key
 * (key_b, and key_a or key_seed as in ckks_keyswitch) switches from s^2 to s.
 * x, y: [batch][2][level][N]; level >= 2.  Relinearisation is one of the
 * key-switches whose key the pages regenerate in-kernel (Perseus summary on
 * ai4snews, "Interpretation" paragraph 2).  The tensor product is never stored:
 * ModUp's inverse row pass forms d2, the final inner-product pass forms d0, d1 and
 * the own-digit limbs of d2 from x and y.  Uses the context's workspace (the
 * relinearised pair takes 2*batch*level*N words of it).  out may alias x or y.
 * Errors: EINVAL (NULL, no key_a or seed), ERANGE (level outside 2..L, batch). */
ckks_status ckks_mul_relin_rescale(const ckks_ctx *ctx, const uint32_t *x, const uint32_t *y, uint32_t level,
                                   const uint32_t *key_b, const uint8_t *key_seed, const uint32_t *key_a,
                                   uint32_t *out, uint32_t batch, void *stream);

/* One rotation key of a linear transform: key_b and, if key_a is NULL, the seed of
 * its a-half (as in ckks_keyswitch), with its Galois element. */
typedef struct {
  const uint32_t *key_b;   /* [dnum][L+K][N] */
  const uint32_t *key_a;   /* stored a-half [dnum][L+K][N], or NULL */
  uint8_t key_seed[32];    /* used when key_a is NULL */
  uint32_t galois_elt;     /* odd, < 2N */
} ckks_rot_key;

/* Baby-step/giant-step linear transform with both hoists: out[2][level][N] =
 * sum_{j<n2} Rot_j(ModDown(S_j)), S_j = sum_{k<n1} D[j][k] * R_k in the extended
 * basis, where R_0 = P*ct and R_k (k >= 1) = (P*sigma_k(c0) + acc_b^k, acc_a^k) is
 * baby key k's inner product with ct's digits (one ModUp serves every baby step;
 * one ModDown per giant step), and Rot_0 is the identity, Rot_j (j >= 1) the full
 * key-switch with giant key j.  diags: D[n2][n1][level+K][N], NTT domain over
 * q_0..q_{level-1}, p_0..p_{K-1}.  baby: n1-1 keys (host array), giant: n2-1 keys
 * (host array).  1 <= n1 <= 16, 1 <= n2 <= 8; out may alias ct.  The pages name
 * bootstrapping, whose linear transforms these are, as the cost centre (Perseus
 * summary on ai4snews, "Synopsis"); the two hoists are those of Bossuat et al.,
 * Eurocrypt 2021.  Uses the context's workspace: needs max_batch large enough
 * for 2*n2 ModDown items and the R and S buffers.
 * Errors: EINVAL (NULL), ERANGE (level, n1, n2, Galois element, workspace). */
ckks_status ckks_linear_transform_bsgs(const ckks_ctx *ctx, const uint32_t *ct, uint32_t level, uint32_t n1,
                                       uint32_t n2, const ckks_rot_key *baby, const ckks_rot_key *giant,
                                       const uint32_t *diags, uint32_t *out, void *stream);

/* Test knob: number of ChaCha blocks generated per 1024-word tile before the
 * rare continuation path runs (default 68, at least 64).  64 sends every tile
 * with a rejected word through the continuation path. */
ckks_status ckks_ctx_set_regen_blocks(ckks_ctx *ctx, uint32_t blocks);

/* Base conversion on the matrix cores.  on = 1: ModUp and ModDown conversions
 * (every call that uses them) run the fused conversion kernel whose sums over
 * sources are exact int8 matrix products (v_mfma_i32_32x32x32_i8 on 7-bit digits of
 * the scaled source values and of the conversion constants), recombined and reduced
 * on the vector unit; on = 0 (the default): the vector-unit kernel.  Both give
 * bit-identical results (the conversion of Han and Ki, 2020, is exact integer
 * arithmetic either way).  Available for N = 2^16 with 9..12 primes per digit and
 * in the special part; the operand tables are built at context creation.
 * Calls already enqueued are not affected.
 * Errors: EINVAL (NULL ctx, host-only context), EUNSUPPORTED (on = 1 for another shape). */
ckks_status ckks_ctx_set_conv_mfma(ckks_ctx *ctx, uint32_t on);

/* Fusion of the inner product with ModDown in ckks_keyswitch.  fused = 1 (the
 * default): the inner product runs in two kernels, one over the special primes (with
 * the row INTT of ModDown) and one over the ciphertext primes (with the end of
 * ModDown and sigma(c0)).  fused = 0: the same arithmetic as separate launches, so
 * that each step can be timed on its own: ModUp, the row NTT of the raised digits
 * (CKKS_K_DIGIT_NTT), the inner product over all level+K primes into an
 * extended-basis pair with P*sigma(c0) added on the ciphertext primes
 * (CKKS_K_IP_EXT), then ckks_moddown's three launches on both halves.  Both give
 * bit-identical results (the ModDown of Han and Ki, 2020, of P*sigma(c0) + acc is
 * sigma(c0) + ModDown(acc) exactly).  The unfused route moves more data through the
 * workspace and is slower; it processes the batch in as many groups as the
 * workspace needs (a context of max_batch B holds 3*B*L*N words for the pairs).
 * Affects ckks_keyswitch only (not the no-alloc, hoisted or multi-item calls).
 * Errors: EINVAL (NULL ctx, host-only context). */
ckks_status ckks_ctx_set_fused(ckks_ctx *ctx, uint32_t fused);

/* Kernel classes of the per-kernel event timer. */
typedef enum {
  CKKS_K_ROW = 0,          /* row pass of an NTT/INTT (1024-coefficient blocks) */
  CKKS_K_COL = 1,          /* column pass of an NTT/INTT */
  CKKS_K_MODUP_CONV = 2,   /* fused column INTT + ModUp conversion + column NTT */
  CKKS_K_IP_SPECIAL = 3,   /* inner product over the special primes (+ row INTT) */
  CKKS_K_MODDOWN_CONV = 4, /* fused column INTT + P->Q conversion + column NTT */
  CKKS_K_IP_FINAL = 5,     /* inner product over the ciphertext primes + end of ModDown */
  CKKS_K_EXPAND = 6,       /* standalone a-half expansion */
  CKKS_K_MODDOWN_FINAL = 7,/* end of a standalone ModDown: row NTT fused with (x - .) * P^-1 */
  CKKS_K_RESCALE_CONV = 8, /* rescale column passes: INTT of the dropped limb; its reduction and NTT per q_i */
  CKKS_K_RESCALE_FINAL = 9,/* row NTT fused with the rescale's subtraction and q_{l-1}^-1 */
  CKKS_K_BABY = 10,        /* baby steps of a linear transform in the extended basis */
  CKKS_K_DIAG = 11,        /* diagonal sums of a linear transform, and the sum of its giant steps */
  CKKS_K_DIGIT_NTT = 12,   /* unfused key-switch: row NTT of the raised digits */
  CKKS_K_IP_EXT = 13,      /* unfused key-switch: inner product over all level+K primes, P*sigma(c0) added */
  CKKS_K_MODDOWN_ROW = 14, /* row INTT of the special part at the start of a standalone ModDown */
  CKKS_K_CLASSES = 15
} ckks_kernel_class;

/* Measurement aid: while enabled, every launch of this context is bracketed by
 * two HIP events recorded on the stream it is launched on (the call's stream, or
 * an internal one of ckks_keyswitch_multi; at most 8192 launches are kept;
 * later ones are not timed).  Enabling clears earlier records; disabling keeps
 * them for ckks_profile_read.  Errors: EINVAL (NULL or host-only context). */
ckks_status ckks_profile_enable(ckks_ctx *ctx, int enable);

/* Waits for the recorded events and writes, for each kernel class c <
 * n_classes, the summed kernel time in milliseconds (ms_out[c], host) and the
 * number of timed launches (launches_out[c], host; may be NULL). */
ckks_status ckks_profile_read(ckks_ctx *ctx, double *ms_out, uint32_t *launches_out, uint32_t n_classes);

#ifdef __cplusplus
}
#endif
#endif /* CKKS_KS_H */
