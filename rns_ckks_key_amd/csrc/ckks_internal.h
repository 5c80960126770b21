// Internal interface between the host orchestration (api.cpp) and the gfx950
// kernels (kernels.hip).  Nothing here crosses the C-ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ckks {

constexpr uint32_t kRow = 1024;         // row-pass block = ChaCha tile = 2^10 coefficients
constexpr uint32_t kMaxHoist = 64;      // keys per hoisted call
constexpr uint32_t kMaxDnum = 8;
constexpr uint32_t kDefaultRegenBlocks = 68;
constexpr uint32_t kMaxRegenBlocks = 256;

// Device-resident constant tables of one context.  Pairs (wm, wmq) are a
// constant w in Montgomery form wm = w*2^32 mod q and its companion wm*q^-1 mod 2^32.
struct DevTables {
  uint32_t log_n, n, L, K, dnum, alpha;
  uint32_t all_big;         // 1: every prime of the chain exceeds 2^31
  const uint32_t* q;        // [L+K]
  const uint32_t* qinv;     // [L+K] q^-1 mod 2^32
  const uint32_t* tw;       // [L+K][N]  psi^brv(k) * 2^32 mod q (companion computed on use)
  const uint32_t* itw;      // [L+K][N]  psi^-brv(k) * 2^32 mod q
  const uint2* ninv;        // [L+K]     N^-1
  const uint2* mu_scale;    // [L+1][L]  N^-1 * (Qd/q_i)^-1 mod q_i for i's digit at level l
  const uint32_t* mu_conv;  // [L+1][dnum][alpha][L+K]  (Qd/q_i) * 2^64 mod q_t (plain)
  const uint2* md_scale_ks; // [K] N^-1 * (P/p_k)^-1 * 2^32 mod p_k (inner-product sums carry 2^-32)
  const uint2* md_scale_pl; // [K] N^-1 * (P/p_k)^-1 mod p_k
  const uint32_t* md_conv;  // [K][L] (P/p_k) * 2^32 mod q_i (plain; REDC2 leaves z * 2^-32)
  const uint32_t* md_conv64;// [K][L] (P/p_k) * 2^64 mod q_i (plain)
  const uint2* md_fin_ks;   // [L] 2^32 * P^-1 mod q_i
  const uint2* md_fin_pl;   // [L] P^-1 mod q_i
  const uint32_t* bound;    // [L+K] floor(2^32/q)*q
  const uint2* one;         // [L+K] 1 (i.e. 2^32 mod q) for w mod q
  const uint2* r2;          // [L+K] multiplier 2^32 mod q (undoes a Montgomery product's 2^-32)
  const uint32_t* r64;      // [L+K] 2^64 mod q (plain): constant of a one-source reduction
  const uint2* rs_inv;      // [L+1][L] q_{l-1}^-1 mod q_i (rescale at level l)
  const uint2* p_mod;       // [L] P mod q_i
  const uint4* mx_w;        // [L+K][3] 2^(7e+32) mod q, e = 0..8 (then zeros): matrix-core conversion
};

// Row pass over limbs: blocks of 1024 coefficients, one wave per block.
constexpr uint32_t kMaxGroup = 16;     // items whose pointers travel in kernel arguments

struct RowArgs {
  const uint32_t* src;
  uint32_t* dst;
  uint64_t src_item_stride, dst_item_stride;   // words between items
  const uint32_t* srcs[kMaxGroup];             // per-item sources (when use_srcs)
  uint32_t use_srcs;
  uint32_t prime0;           // absolute prime of limb 0
  uint32_t n_limbs;
  // ModUp finish mode: limbs [own_lo, own_lo+own_n) are copied from `own_src` untransformed
  // and the transformed limbs come from src limb index y (y < own_lo) or y - own_n.
  uint32_t own_lo, own_n;
  const uint32_t* own_src;
  uint64_t own_item_stride;
  // ext-basis prime mapping (limb y -> absolute prime): y < level ? prime0 + y : L + (y - level)
  uint32_t level;            // 0: plain mapping prime0 + y
  // forward pass only, when cmb != nullptr: dst = (cmb - NTT(src)) * cmb_factor[y]
  const uint32_t* cmb;
  uint64_t cmb_item_stride;
  // inverse pass only, when src2 != nullptr: the source limb is src * src2 (elementwise,
  // same layout and item stride as src), the x1 y1 part of a tensor product
  const uint32_t* src2;
  const uint2* cmb_factor;
};

// Column pass over limbs (in place): one thread per column of 2^(log_n-10) coefficients.
struct ColArgs {
  uint32_t* data;
  uint64_t item_stride;
  uint32_t prime0, n_limbs;
  // forward pass only, when bsrc != nullptr: every limb starts from bsrc[item] (one
  // polynomial of values < 2^32) reduced modulo its prime, instead of its own data
  const uint32_t* bsrc;
  uint64_t bsrc_item_stride;
};

// Fused column INTT + scale + fast base conversion + column NTT.
struct ConvArgs {
  const uint32_t* src;       // source limbs: src + item*src_item + y*src_y + s*N
  uint64_t src_item, src_y;
  uint32_t* dst;             // dst + item*dst_item + y*dst_y + dlimb*N
  uint64_t dst_item, dst_y;
  uint32_t src_prime0, src_prime_step;   // absolute prime of source limb s of group y: prime0 + y*step + s
  uint32_t ns_max, ns_limit;             // ns = min(ns_max, ns_limit - y*src_prime_step)
  const uint2* scale;        // + y*scale_y + s
  uint32_t scale_y;
  const uint32_t* conv;      // + y*conv_y + s*conv_s + abs target prime (or target limb)
  uint32_t conv_y, conv_s;
  uint32_t conv_by_abs;      // 1: index conv by absolute target prime, 0: by target limb
  uint32_t n_targets;        // targets e; dst limb = e < skip_lo ? e : e + ns; abs prime via level map
  uint32_t skip;             // 1: skip the source limbs' own range in the destination limbs
  uint32_t level;            // ext mapping: dlimb < level ? dlimb : L + dlimb - level (level=0: dlimb)
  uint32_t tchunks;          // targets split over this many workgroups (set by the launcher)
  // Matrix-core conversion (ring 2^16, 9..12 sources): int8 A operands of target pair
  // tiles, [group y][tile][K step][lane] uint4 from mx + y*mx_y; nullptr = vector path.
  const uint4* mx;
  uint32_t mx_y;
};

// Target-pair tiles per conversion group in the matrix-core operand tables.
constexpr uint32_t kMxTiles = 32;

struct KeyRef {
  const uint32_t* b;         // [dnum][L+K][N]
  const uint32_t* a;         // stored a-half or nullptr
  uint32_t seed[8];
  uint32_t galois;
  const uint32_t* ct;        // per-group ciphertext [2][level][N] (per_group mode)
  uint32_t* out;             // per-group output [2][level][N] (per_group mode)
};

// Inner product (+ fused ModDown pieces).  Grid: x = limb, y = 1024-block, z = key group.
struct IpArgs {
  uint32_t level, nd;        // level and its digit count
  uint32_t n_ct;             // ciphertexts per key group
  const uint32_t* ext;       // [ext item][dnum][L+K][N]
  uint64_t ext_ct_stride;    // words between ciphertexts (0 when hoisted: one shared ModUp)
  const uint32_t* ct;        // [ct][2][level][N]
  uint64_t ct_ct_stride;     // 0 when hoisted
  uint32_t* tmpP;            // special output [item][2][K][N]
  const uint32_t* conv;      // final input   [item][2][level][N] (row pass pending)
  uint32_t* out;             // final output  [item][2][level][N]
  uint32_t regen_blocks;
  uint32_t digits_ntt;       // 1: ext holds fully transformed digits, own limbs included (hoisted calls)
  uint32_t per_group;        // 1: key group g has its own ciphertext key[g].ct, output key[g].out and
                             //    digits at ext + g * ext_ct_stride (n_ct = 1)
  uint32_t n_keys;
  KeyRef key[kMaxGroup];     // per key group (grid z)
  // Relinearisation: the ciphertext is the tensor product of ct (x) and ty (y), both
  // [ct][2][level][N] with stride ct_ct_stride, formed in the final pass (Galois element 1).
  const uint32_t* ty;
};

hipError_t launch_row(const DevTables& T, const RowArgs& a, bool fwd, uint32_t items, hipStream_t s);
hipError_t launch_col(const DevTables& T, const ColArgs& a, bool fwd, bool scale_ninv, uint32_t items, hipStream_t s);
hipError_t launch_conv(const DevTables& T, const ConvArgs& a, uint32_t groups, uint32_t items, hipStream_t s);
hipError_t launch_ip(const DevTables& T, const IpArgs& a, bool final_pass, uint32_t n_limbs, hipStream_t s);
// Baby steps of a linear transform in the extended basis (NTT domain), one per key
// group: R_k = (P*sigma_k(c0) + acc_b, acc_a) over limbs e < level + K (the c0 term
// only on ciphertext primes), from fully transformed hoisted digits.
struct ExtArgs {
  uint32_t level, nd;
  const uint32_t* ext;       // digits [dnum][L+K][N], row NTT done, own limbs included
  const uint32_t* c0;        // [level][N]
  uint32_t* out;             // R [key group][2][level+K][N]
  uint32_t regen_blocks;
  uint32_t n_keys;
  // items sharing the keys: item i reads ext + i*ext_item and c0 + i*c0_item and
  // writes out + i*out_item (a workgroup regenerates its a-tile once for all of them)
  uint32_t items;
  uint64_t ext_item, c0_item, out_item;
  KeyRef key[kMaxGroup];
};

// Diagonal sums S_j = sum_k D[j][k] * R_k over the extended basis, R_0 = P*ct.
constexpr uint32_t kMaxGiant = 8;
struct DiagArgs {
  uint32_t level, n1, n2;
  const uint32_t* ct;        // [2][level][N]
  const uint32_t* r;         // R_1.. [n1-1][2][level+K][N]
  const uint32_t* diags;     // [n2][n1][level+K][N]
  uint32_t* s;               // [n2][2][level+K][N]
};

// out [2][level][N] = sum of n_src polynomials of the same shape.
struct SumArgs {
  uint32_t n_src;
  uint64_t words;            // 2 * level * N
  const uint32_t* src[kMaxGroup];
};

hipError_t launch_rot_ext(const DevTables& T, const ExtArgs& a, hipStream_t s);
hipError_t launch_diag_acc(const DevTables& T, const DiagArgs& a, hipStream_t s);
hipError_t launch_sum(const DevTables& T, const SumArgs& a, uint32_t* out, uint32_t level, hipStream_t s);
hipError_t launch_expand(const DevTables& T, const uint32_t seed[8], uint32_t* key_a, uint32_t regen_blocks,
                         hipStream_t s);

// Static scratch of the key-switch that allocates nothing (noalloc.hip): 96 MiB per
// GPU, the workspace of one ciphertext at N = 2^16 with 36 + 12 primes at any level.
constexpr uint64_t kScratchBytes = 96ull << 20;
// Looks up the array's device address on `device`, which must be current (once per
// device; later calls return the first result).
hipError_t scratch_setup(int device);
// The array's device address on `device`, or nullptr if scratch_setup has not
// succeeded there; scratch_error says why.
uint32_t* scratch_ptr(int device);
const char* scratch_error(int device);

}  // namespace ckks
