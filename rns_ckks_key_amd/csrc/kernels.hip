// gfx950 kernels of the key-switching path.
//
// Transform split.  An N = C * 1024 point negacyclic NTT (merged twist,
// Cooley-Tukey, natural order in, bit-reversed out; Longa-Naehrig 2016) is done
// as two passes: a column pass over the C elements {c + 1024k} of each column c
// (the stages whose butterfly distance is >= 1024; all columns share twiddles),
// and a row pass over each contiguous 1024-element block (distances 512..1).
// The inverse (Gentleman-Sande) runs the row pass first.  A column lives in one
// thread's registers; a block lives in one wave (16 values per lane) and moves
// between three register layouts through wave-private LDS:
//   layout A: x[k]        <-> r = lane + 64k          (stages 512..64)
//   layout B: x[k]        <-> r = 64*(lane>>2) + 4k + (lane&3)   (stages 32..4)
//   layout C: x[4g + k2]  <-> r = 4*lane + 256g + k2  (stages 2, 1)
// Global loads/stores use layout A (64 lanes x 4 B contiguous) or C (16-byte
// vectors, 1 KB contiguous per instruction).
//
// Key-switch kernels.  The conversions of ModUp and ModDown are per-coefficient,
// so they are fused into the column pass (k_conv).  The inner product and the
// automorphism are fused into the row pass, and the ChaCha12 tile of 1024
// a-half coefficients coincides with a row block, so the two kernels that use
// the key (k_ip: special primes, and the ciphertext primes together with the
// end of ModDown) regenerate each tile once per workgroup and reuse it for
// every ciphertext of the batch (Perseus summary on ai4snews, "Interpretation"
// paragraph 2: the random half of the key is rebuilt from a seed with ChaCha12
// in counter mode by the kernels that consume the key).  k_conv_mx is the conversion with its
// sums over sources as int8 matrix-core products (selected per context).  A
// relinearisation never stores its tensor product: the inverse row pass forms
// x1*y1 (k_row MUL) and the final inner-product pass the other products (TENSOR).
#include <type_traits>
#include <utility>

#include "ckks_internal.h"
#include "modarith.h"

namespace ckks {

// Compile-time loop: f(std::integral_constant<int, i>) for i = 0..N-1, as
// straight-line code (register arrays indexed by i stay in registers).
template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// ------------------------------------------------------------------ helpers

// A scalar zero the optimiser cannot see through.  A row transform inside a loop
// takes `lane + opaque_zero()` as its lane index: its per-lane twiddle and LDS
// addresses are then computed in the loop, where they are used, instead of being
// hoisted out of it and held in (64-bit) registers for the whole kernel, which
// costs a wave per SIMD of occupancy.
__device__ __forceinline__ uint32_t opaque_zero() {
  uint32_t z;
  asm volatile("s_mov_b32 %0, 0" : "=s"(z));
  return z;
}

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Workgroups are dealt to the 8 XCDs round robin by linear id.  Remaps the
// linear id so that each XCD gets one contiguous run of the logical order
// (whose slowest index is a prime), so an XCD's L2 holds the twiddles of few
// primes.  XCD x holds the ids w = x, x+8, ... < total, i.e. total/8 + (x <
// total%8) of them; they take the logical ids from x*(total/8) + min(x, total%8)
// on, so the map is a bijection onto [0, total) for every total.
constexpr uint32_t kXcds = 8;
__device__ __forceinline__ uint32_t xcd_logical_id() {
  const uint32_t total = gridDim.x * gridDim.y * gridDim.z;
  const uint32_t w = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  const uint32_t x = w % kXcds, base = total / kXcds, extra = total % kXcds;
  return __builtin_amdgcn_readfirstlane(x * base + min(x, extra) + w / kXcds);
}

// LDS position of coefficient r of a 1024-word block: 4 pad words after every
// 64.  16-byte aligned for layout C, and free of bank conflicts within each
// half-wave for layouts A, B and C.  For a lane below 64 the position of each
// layout's register k is a per-lane base plus a constant (the pad count depends
// on k and the lane's high bits only), written out below so that every LDS
// instruction takes an immediate offset even where the lane index is opaque to
// the compiler:
//   A: r = lane + 64k              -> lane + 68k
//   B: r = 64(lane/4) + lane%4 + 4k -> 68(lane/4) + lane%4 + 4k
//   C: r = 4 lane + 256g           -> 4 lane + 4(lane/16) + 272g
constexpr uint32_t kRowPad = kRow + kRow / 16;
__device__ __forceinline__ uint32_t swz(uint32_t r) { return r + ((r >> 6) << 2); }
__device__ __forceinline__ uint32_t lds_base_B(uint32_t lane) { return 68 * (lane >> 2) + (lane & 3); }
__device__ __forceinline__ uint32_t lds_base_C(uint32_t lane) { return 4 * lane + 4 * (lane >> 4); }

// Twiddles are stored as w*2^32 mod q only; the Montgomery companion w*q^-1 mod 2^32
// is one multiply (a scalar one when the twiddle is wave-uniform).
// Forward butterfly.  LAZY: a, b and the results are any 32-bit representatives
// (t = b*w is canonical, so a + t and a - t each take one carry-selected
// correction); otherwise all are canonical.
template <bool LAZY = true>
__device__ __forceinline__ void ct_bfly_c(uint32_t& a, uint32_t& b, uint2 w, uint32_t q) {
  const uint32_t t = mul_const(b, w.x, w.y, q);
  if constexpr (LAZY) {
    b = lazy_sub(a, t, q);
    a = lazy_add(a, t, q);
  } else {
    b = sub_mod(a, t, q);
    a = add_mod(a, t, q);
  }
}
template <bool LAZY = true>
__device__ __forceinline__ void ct_bfly(uint32_t& a, uint32_t& b, uint32_t w, uint32_t qinv, uint32_t q) {
  ct_bfly_c<LAZY>(a, b, make_uint2(w, w * qinv), q);
}

// Canonical residues of lazy values for q > 2^31 (x < 2q): min(x, x - q).
template <int R>
__device__ __forceinline__ void canon_big(uint32_t (&v)[R], uint32_t q) {
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const uint32_t d = v[i] - q;
    v[i] = d < v[i] ? d : v[i];
  }
}

// Canonical product a*b mod q: a Montgomery product (factor 2^-32), then times 2^32.
__device__ __forceinline__ uint32_t prod_mod(uint32_t a, uint32_t b, const Mod& md, uint2 r2) {
  return mul_const(mont_mul(a, b, md), r2.x, r2.y, md.q);
}

__device__ __forceinline__ void gs_bfly_c(uint32_t& a, uint32_t& b, uint2 w, uint32_t q) {
  uint32_t s = add_mod(a, b, q);
  uint32_t d = sub_mod(a, b, q);
  a = s;
  b = mul_const(d, w.x, w.y, q);
}
__device__ __forceinline__ void gs_bfly(uint32_t& a, uint32_t& b, uint32_t w, uint32_t qinv, uint32_t q) {
  gs_bfly_c(a, b, make_uint2(w, w * qinv), q);
}

// Twiddle i of a row transform with its Montgomery companion: from a limb's table of
// w*2^32 mod q (companion computed, on the scalar unit when i is wave-uniform), or
// from a block's staged copy that holds both.
__device__ __forceinline__ uint2 twc(const uint32_t* __restrict__ tw, uint32_t i, uint32_t qinv) {
  const uint32_t w = tw[i];
  return make_uint2(w, w * qinv);
}
__device__ __forceinline__ uint2 twc(const uint2* __restrict__ tw, uint32_t i, uint32_t) { return tw[i]; }

__device__ __forceinline__ void load_A(uint32_t (&x)[16], const uint32_t* __restrict__ p, uint32_t lane) {
#pragma unroll
  for (int k = 0; k < 16; ++k) x[k] = p[lane + 64 * k];
}
__device__ __forceinline__ void store_A(uint32_t* __restrict__ p, const uint32_t (&x)[16], uint32_t lane) {
#pragma unroll
  for (int k = 0; k < 16; ++k) p[lane + 64 * k] = x[k];
}
__device__ __forceinline__ void load_C(uint32_t (&x)[16], const uint32_t* __restrict__ p, uint32_t lane) {
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    uint4 v = *reinterpret_cast<const uint4*>(p + 4 * lane + 256 * g);
    x[4 * g] = v.x; x[4 * g + 1] = v.y; x[4 * g + 2] = v.z; x[4 * g + 3] = v.w;
  }
}
__device__ __forceinline__ void store_C(uint32_t* __restrict__ p, const uint32_t (&x)[16], uint32_t lane) {
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    uint4 v = make_uint4(x[4 * g], x[4 * g + 1], x[4 * g + 2], x[4 * g + 3]);
    *reinterpret_cast<uint4*>(p + 4 * lane + 256 * g) = v;
  }
}
// layout C registers -> LDS block in natural (swizzled) order, and back
__device__ __forceinline__ void lds_put_C(uint32_t* lds, const uint32_t (&x)[16], uint32_t lane) {
  uint32_t* p = lds + lds_base_C(lane);
#pragma unroll
  for (int g = 0; g < 4; ++g)
    *reinterpret_cast<uint4*>(p + 272 * g) = make_uint4(x[4 * g], x[4 * g + 1], x[4 * g + 2], x[4 * g + 3]);
}
__device__ __forceinline__ void lds_get_C(uint32_t (&x)[16], const uint32_t* lds, uint32_t lane) {
  const uint32_t* p = lds + lds_base_C(lane);
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    uint4 v = *reinterpret_cast<const uint4*>(p + 272 * g);
    x[4 * g] = v.x; x[4 * g + 1] = v.y; x[4 * g + 2] = v.z; x[4 * g + 3] = v.w;
  }
}
__device__ __forceinline__ void lds_put_A(uint32_t* lds, const uint32_t (&x)[16], uint32_t lane) {
  uint32_t* p = lds + lane;
#pragma unroll
  for (int k = 0; k < 16; ++k) p[68 * k] = x[k];
}
__device__ __forceinline__ void lds_get_A(uint32_t (&x)[16], const uint32_t* lds, uint32_t lane) {
  const uint32_t* p = lds + lane;
#pragma unroll
  for (int k = 0; k < 16; ++k) x[k] = p[68 * k];
}
__device__ __forceinline__ void lds_put_B(uint32_t* lds, const uint32_t (&x)[16], uint32_t lane) {
  uint32_t* p = lds + lds_base_B(lane);
#pragma unroll
  for (int k = 0; k < 16; ++k) p[4 * k] = x[k];
}
__device__ __forceinline__ void lds_get_B(uint32_t (&x)[16], const uint32_t* lds, uint32_t lane) {
  const uint32_t* p = lds + lds_base_B(lane);
#pragma unroll
  for (int k = 0; k < 16; ++k) x[k] = p[4 * k];
}

// ------------------------------------------------------------------ row pass

// Forward stages 512..1 of one 1024-block of a limb: layout A in, layout C out.
// A stage of half distance t has m = 512/t twiddle groups in a block; group i of
// block blk uses tw[N/(2t) + blk*m + i] = tw[m*(N/1024 + blk) + i].  The caller
// passes `off`: N/1024 + blk with the limb's table, or 1 with a block's own copy
// (entry m + i, as staged in LDS by stage_block_twiddles).  The butterflies carry
// lazy values; CANON makes the outputs canonical (callers that only multiply them
// by constants skip it).  BIG: the prime exceeds 2^31, known at compile time, so
// canonical is one conditional subtraction with no branch on q.
template <bool CANON = true, bool BIG = false, class Tw>
__device__ __forceinline__ void row_fwd(uint32_t (&x)[16], uint32_t lane, uint32_t off, const Tw* __restrict__ tw,
                                        uint32_t q, uint32_t qinv, uint32_t* lds, uint2 one) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int h = 8 >> s;
    const uint32_t m = 1u << s;
#pragma unroll
    for (int grp = 0; grp < 8 / h; ++grp) {
      const uint2 w = twc(tw, m * off + grp, qinv);
#pragma unroll
      for (int kk = 0; kk < h; ++kk) ct_bfly_c(x[2 * grp * h + kk], x[2 * grp * h + kk + h], w, q);
    }
  }
  lds_put_A(lds, x, lane);
  wave_sync();
  lds_get_B(x, lds, lane);
  wave_sync();
  const uint32_t hb = lane >> 2;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int h = 8 >> s;
    const uint32_t m = 16u << s;
    const uint32_t base = m * off + 8 * hb / h;
#pragma unroll
    for (int grp = 0; grp < 8 / h; ++grp) {
      const uint2 w = twc(tw, base + grp, qinv);
#pragma unroll
      for (int kk = 0; kk < h; ++kk) ct_bfly_c(x[2 * grp * h + kk], x[2 * grp * h + kk + h], w, q);
    }
  }
  lds_put_B(lds, x, lane);
  wave_sync();
  lds_get_C(x, lds, lane);
  wave_sync();
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const uint2 w = twc(tw, 256 * off + lane + 64 * g, qinv);
    ct_bfly_c(x[4 * g], x[4 * g + 2], w, q);
    ct_bfly_c(x[4 * g + 1], x[4 * g + 3], w, q);
    const uint32_t i1 = 512 * off + 2 * lane + 128 * g;
    const uint2 w0 = twc(tw, i1, qinv), w1 = twc(tw, i1 + 1, qinv);
    ct_bfly_c(x[4 * g], x[4 * g + 1], w0, q);
    ct_bfly_c(x[4 * g + 2], x[4 * g + 3], w1, q);
  }
  if constexpr (CANON && BIG) {
    canon_big(x, q);
  } else if constexpr (CANON) {
#pragma unroll
    for (int k = 0; k < 16; ++k) x[k] = canon(x[k], q, one.x, one.y);
  }
}

// Inverse stages 1..512 of one 1024-block: layout C in, layout A out (no N^-1).
// Twiddles indexed as in row_fwd (off = N/1024 + blk, or 1 with a block's copy).
template <class Tw>
__device__ __forceinline__ void row_inv(uint32_t (&x)[16], uint32_t lane, uint32_t off, const Tw* __restrict__ itw,
                                        uint32_t q, uint32_t qinv, uint32_t* lds) {
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const uint32_t i1 = 512 * off + 2 * lane + 128 * g;
    const uint2 w0 = twc(itw, i1, qinv), w1 = twc(itw, i1 + 1, qinv);
    gs_bfly_c(x[4 * g], x[4 * g + 1], w0, q);
    gs_bfly_c(x[4 * g + 2], x[4 * g + 3], w1, q);
    const uint2 w = twc(itw, 256 * off + lane + 64 * g, qinv);
    gs_bfly_c(x[4 * g], x[4 * g + 2], w, q);
    gs_bfly_c(x[4 * g + 1], x[4 * g + 3], w, q);
  }
  lds_put_C(lds, x, lane);
  wave_sync();
  lds_get_B(x, lds, lane);
  wave_sync();
  const uint32_t hb = lane >> 2;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int h = 1 << s;
    const uint32_t m = 128u >> s;
    const uint32_t base = m * off + 8 * hb / h;
#pragma unroll
    for (int grp = 0; grp < 8 / h; ++grp) {
      const uint2 w = twc(itw, base + grp, qinv);
#pragma unroll
      for (int kk = 0; kk < h; ++kk) gs_bfly_c(x[2 * grp * h + kk], x[2 * grp * h + kk + h], w, q);
    }
  }
  lds_put_B(lds, x, lane);
  wave_sync();
  lds_get_A(x, lds, lane);
  wave_sync();
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int h = 1 << s;
    const uint32_t m = 8u >> s;
#pragma unroll
    for (int grp = 0; grp < 8 / h; ++grp) {
      const uint2 w = twc(itw, m * off + grp, qinv);
#pragma unroll
      for (int kk = 0; kk < h; ++kk) gs_bfly_c(x[2 * grp * h + kk], x[2 * grp * h + kk + h], w, q);
    }
  }
}

// Copies the twiddles of block blk of a limb (entries m*(N/1024 + blk) + i of its
// table, m = 1, 2, ..., 512, i < m) to dst[m + i]: the 1023 twiddles a row pass over
// that block uses.  Every thread of the workgroup may take part (no barrier here).
__device__ __forceinline__ void stage_block_twiddles(uint32_t* dst, const uint32_t* __restrict__ tw, uint32_t off) {
  for (uint32_t k = threadIdx.x + 1; k < kRow; k += blockDim.x) {
    const uint32_t m = 1u << (31 - __builtin_clz(k));  // the stage of entry k: m <= k < 2m
    dst[k] = tw[m * off + (k - m)];
  }
}
// The same copy with each twiddle's Montgomery companion beside it.
__device__ __forceinline__ void stage_block_twiddles(uint2* dst, const uint32_t* __restrict__ tw, uint32_t off,
                                                     uint32_t qinv) {
  for (uint32_t k = threadIdx.x + 1; k < kRow; k += blockDim.x) {
    const uint32_t m = 1u << (31 - __builtin_clz(k));
    const uint32_t w = tw[m * off + (k - m)];
    dst[k] = make_uint2(w, w * qinv);
  }
}

// ------------------------------------------------------------------ column pass

// Forward stages N/2..1024 on one column v[k] <-> e = 1024k + c (twiddles tw[1..C-1], shared by all columns).
// LAZY: outputs are 32-bit representatives, which callers make canonical.
template <int LOGC, bool LAZY>
__device__ __forceinline__ void col_fwd(uint32_t (&v)[1 << LOGC], const uint32_t* __restrict__ tw, uint32_t q,
                                        uint32_t qinv) {
  constexpr int C = 1 << LOGC;
#pragma unroll
  for (int s = 0; s < LOGC; ++s) {
    const int m = 1 << s;
    const int h = C >> (s + 1);
#pragma unroll
    for (int i = 0; i < m; ++i) {
      const uint32_t w = tw[m + i];
#pragma unroll
      for (int k = 0; k < h; ++k) ct_bfly<LAZY>(v[2 * i * h + k], v[2 * i * h + k + h], w, qinv, q);
    }
  }
}

template <int LOGC>
__device__ __forceinline__ void col_inv(uint32_t (&v)[1 << LOGC], const uint32_t* __restrict__ itw, uint32_t q,
                                        uint32_t qinv) {
  constexpr int C = 1 << LOGC;
#pragma unroll
  for (int s = LOGC - 1; s >= 0; --s) {
    const int m = 1 << s;
    const int h = C >> (s + 1);
#pragma unroll
    for (int i = 0; i < m; ++i) {
      const uint32_t w = itw[m + i];
#pragma unroll
      for (int k = 0; k < h; ++k) gs_bfly(v[2 * i * h + k], v[2 * i * h + k + h], w, qinv, q);
    }
  }
}

// col_inv, then every output times the constant sc (w*2^32 mod q, companion), with
// that multiplication folded into the last stage: its sums are multiplied by sc and
// its differences by w*sc (w the stage's one twiddle), instead of the differences by
// w and then all outputs by sc.  The results are the same residues, canonical.
template <int LOGC>
__device__ __forceinline__ void col_inv_scaled(uint32_t (&v)[1 << LOGC], const uint32_t* __restrict__ itw,
                                               uint32_t q, uint32_t qinv, uint2 sc) {
  constexpr int C = 1 << LOGC;
#pragma unroll
  for (int s = LOGC - 1; s >= 1; --s) {
    const int m = 1 << s;
    const int h = C >> (s + 1);
#pragma unroll
    for (int i = 0; i < m; ++i) {
      const uint32_t w = itw[m + i];
#pragma unroll
      for (int k = 0; k < h; ++k) gs_bfly(v[2 * i * h + k], v[2 * i * h + k + h], w, qinv, q);
    }
  }
  const uint32_t wsc = mont_mul(itw[1], sc.x, Mod{q, qinv});  // (w * scale) in Montgomery form
  const uint32_t wscq = wsc * qinv;
#pragma unroll
  for (int k = 0; k < C / 2; ++k) {
    const uint32_t a = v[k], b = v[k + C / 2];  // canonical: outputs of the stages above
    v[k] = mul_const(lazy_add(a, b, q), sc.x, sc.y, q);
    v[k + C / 2] = mul_const(lazy_sub(a, b, q), wsc, wscq, q);
  }
}

// col_inv_scaled on two lanes per column: lane z of an aligned lane pair holds rows
// z*C/2 .. z*C/2 + C/2 - 1.  Every stage but the last stays in the lane (the lane's
// half of the column holds whole butterfly groups); the last pairs the two lanes, the
// sums landing in lane 0 (times sc) and the differences in lane 1 (times w*sc).
template <int LOGC>
__device__ __forceinline__ void col_inv_scaled_pair(uint32_t (&v)[(1 << LOGC) / 2], uint32_t z,
                                                    const uint32_t* __restrict__ itw, uint32_t q, uint32_t qinv,
                                                    uint2 sc) {
  constexpr int C = 1 << LOGC, H = C / 2;
#pragma unroll
  for (int s = LOGC - 1; s >= 1; --s) {
    const int m = 1 << s;
    const int h = C >> (s + 1);
#pragma unroll
    for (int i = 0; i < m / 2; ++i) {
      const uint32_t w = itw[m + z * (m / 2) + i];
#pragma unroll
      for (int k = 0; k < h; ++k) gs_bfly(v[2 * i * h + k], v[2 * i * h + k + h], w, qinv, q);
    }
  }
  const uint32_t wsc = mont_mul(itw[1], sc.x, Mod{q, qinv});
  const uint32_t cx = z ? wsc : sc.x, cy = z ? wsc * qinv : sc.y;
#pragma unroll
  for (int k = 0; k < H; ++k) {
    const uint32_t own = v[k];
    const uint32_t other = __builtin_amdgcn_mov_dpp(own, 0xB1, 0xf, 0xf, true);  // the pair's other lane
    const uint32_t sum = lazy_add(own, other, q), dif = lazy_sub(other, own, q);
    v[k] = mul_const(z ? dif : sum, cx, cy, q);
  }
}

// ------------------------------------------------------------------ ChaCha12

// ChaCha block function (Bernstein 2008) with 12 rounds: state = constant
// "expand 32-byte k", 8 seed words, counter, then words 13..15; output = state
// after 6 double rounds plus the initial state.
#define CK_QR(a, b, c, d)                 \
  a += b; d ^= a; d = __builtin_rotateleft32(d, 16); \
  c += d; b ^= c; b = __builtin_rotateleft32(b, 12); \
  a += b; d ^= a; d = __builtin_rotateleft32(d, 8);  \
  c += d; b ^= c; b = __builtin_rotateleft32(b, 7);

__device__ __forceinline__ void chacha12_block(const uint32_t* __restrict__ key, uint32_t ctr, uint32_t w13,
                                               uint32_t w14, uint32_t w15, uint32_t (&o)[16]) {
  uint32_t x0 = 0x61707865u, x1 = 0x3320646eu, x2 = 0x79622d32u, x3 = 0x6b206574u;
  uint32_t x4 = key[0], x5 = key[1], x6 = key[2], x7 = key[3];
  uint32_t x8 = key[4], x9 = key[5], x10 = key[6], x11 = key[7];
  uint32_t x12 = ctr, x13 = w13, x14 = w14, x15 = w15;
#pragma unroll
  for (int r = 0; r < 6; ++r) {
    CK_QR(x0, x4, x8, x12) CK_QR(x1, x5, x9, x13) CK_QR(x2, x6, x10, x14) CK_QR(x3, x7, x11, x15)
    CK_QR(x0, x5, x10, x15) CK_QR(x1, x6, x11, x12) CK_QR(x2, x7, x8, x13) CK_QR(x3, x4, x9, x14)
  }
  o[0] = x0 + 0x61707865u; o[1] = x1 + 0x3320646eu; o[2] = x2 + 0x79622d32u; o[3] = x3 + 0x6b206574u;
  o[4] = x4 + key[0]; o[5] = x5 + key[1]; o[6] = x6 + key[2]; o[7] = x7 + key[3];
  o[8] = x8 + key[4]; o[9] = x9 + key[5]; o[10] = x10 + key[6]; o[11] = x11 + key[7];
  o[12] = x12 + ctr; o[13] = x13 + w13; o[14] = x14 + w14; o[15] = x15 + w15;
}
#undef CK_QR

// Exclusive prefix sum of v over the workgroup's threads, in thread order, and the
// workgroup total.  wsum: 16 words of LDS scratch.  blockDim.x must be a multiple of
// 64; every thread must call this (two workgroup barriers).
__device__ __forceinline__ uint2 block_scan(uint32_t v, uint32_t* wsum) {
  const uint32_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  uint32_t incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = __shfl_up(incl, d, 64);
    if (lane >= (uint32_t)d) incl += y;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  uint32_t before = 0, total = 0;
  for (uint32_t w = 0; w < nw; ++w) {
    const uint32_t sw = wsum[w];
    before += w < wave ? sw : 0u;
    total += sw;
  }
  __syncthreads();
  return make_uint2(before + incl - v, total);
}

// Places one block's 16 words: word i goes to tile position pos (then pos + 1) if it
// is accepted and pos < 1024; every other word is written to this thread's own
// scratch word instead, so the stores need no branch.  With bound == q (primes above
// 2^31) an accepted word is already its residue; otherwise it is reduced mod q by a
// Montgomery multiply with `one` (2^32 mod q, companion).
__device__ __forceinline__ void place_block(const uint32_t (&w)[16], uint32_t pos, uint32_t bound, uint32_t q,
                                            uint2 one, uint32_t* tile, uint32_t* trash) {
  if (bound == q) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const bool ok = w[i] < bound;
      *((ok && pos < kRow) ? tile + pos : trash) = w[i];
      pos += ok ? 1u : 0u;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const bool ok = w[i] < bound;
      *((ok && pos < kRow) ? tile + pos : trash) = mul_const(w[i], one.x, one.y, q);
      pos += ok ? 1u : 0u;
    }
  }
}

// Regenerates `ntiles` tiles of the a-half, tile T = (digit j0+T, prime t, tile tau),
// into dst[T*1024 .. +1024) (LDS).  Rejection sampling: word w is accepted iff
// w < bound and becomes w mod q; the k-th accepted word of a sub-stream lands at
// coefficient k.  The first `nb` blocks of every tile are generated together by
// all threads (block j of tile T by job T*nb + j); a workgroup prefix sum of the
// accepted counts places each block's words.  The rare tile still short of 1024
// words continues with blockDim.x more blocks at a time.  cnt: LDS scratch of
// 2*ntiles + 16 + 64 words (the last 64: one sink word per lane, shared by the
// waves, as only lanes of one instruction write at once).  Every thread of the
// workgroup must call this (it contains workgroup barriers).
__device__ void regen_tiles(const uint32_t* __restrict__ seed, uint32_t j0, uint32_t ntiles, uint32_t t,
                            uint32_t tau, uint32_t q, uint32_t bound, uint2 one, uint32_t nb, uint32_t* dst,
                            uint32_t* cnt) {
  const uint32_t tid = threadIdx.x, nth = blockDim.x;
  const uint32_t jobs = ntiles * nb;
  uint32_t* tstart = cnt;             // [ntiles] accepted words before each tile's first block
  uint32_t* tot = cnt + ntiles;       // [ntiles] accepted words of the first nb blocks of each tile
  uint32_t* wsum = cnt + 2 * ntiles;  // [16] scan scratch
  uint32_t* trash = cnt + 2 * ntiles + 16 + (tid & 63);  // this lane's sink for words that land nowhere
  uint32_t carry = 0;                 // accepted words of all earlier passes (uniform)
  for (uint32_t r0 = 0; r0 < jobs; r0 += nth) {
    const uint32_t x = r0 + tid;
    uint32_t w[16];
    uint32_t mask = 0;
    uint32_t tile = 0, bc = 0;
    if (x < jobs) {
      tile = x / nb;
      bc = x - tile * nb;
      chacha12_block(seed, bc, j0 + tile, t, tau, w);
#pragma unroll
      for (int i = 0; i < 16; ++i) mask |= (w[i] < bound ? 1u : 0u) << i;
    }
    const uint32_t c = __popc(mask);
    const uint2 sc = block_scan(c, wsum);
    const uint32_t before = carry + sc.x;
    if (x < jobs && bc == 0) tstart[tile] = before;
    carry += sc.y;
    __syncthreads();
    if (x < jobs) {
      const uint32_t off = before - tstart[tile];
      if (bc == nb - 1) tot[tile] = off + c;
      place_block(w, off, bound, q, one, dst + tile * kRow, trash);
    }
    __syncthreads();
  }
  // continuation for tiles that are still short (uniform control flow)
  for (uint32_t tile = 0; tile < ntiles; ++tile) {
    uint32_t filled = tot[tile];
    uint32_t ctr0 = nb;
    while (filled < kRow) {
      uint32_t w[16];
      uint32_t mask = 0;
      chacha12_block(seed, ctr0 + tid, j0 + tile, t, tau, w);
#pragma unroll
      for (int i = 0; i < 16; ++i) mask |= (w[i] < bound ? 1u : 0u) << i;
      const uint2 sc = block_scan(__popc(mask), wsum);
      place_block(w, filled + sc.x, bound, q, one, dst + tile * kRow, trash);
      filled += sc.y;
      ctr0 += nth;
    }
  }
}

// ------------------------------------------------------------------ kernels

// MUL (inverse only): the source limb is the product of src and src2 (same layout), the
// x1*y1 part of a tensor product formed where the relinearisation's ModUp reads it.
// BIG (forward only): every prime of the chain exceeds 2^31.
template <bool FWD, bool MUL = false, bool BIG = false>
__global__ __launch_bounds__(256) void k_row(DevTables T, RowArgs a) {
  __shared__ uint32_t lds[4][kRowPad];
  const uint32_t wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint32_t n = T.n;
  const uint32_t u = xcd_logical_id();
  if (u >= gridDim.x * gridDim.y * gridDim.z) return;  // guard (the map is a bijection)
  const uint32_t bx = __builtin_amdgcn_readfirstlane(u % gridDim.x);
  const uint32_t item = __builtin_amdgcn_readfirstlane((u / gridDim.x) % gridDim.z);
  const uint32_t y = __builtin_amdgcn_readfirstlane(u / (gridDim.x * gridDim.z));
  const uint32_t blk = bx * 4 + wave;
  if (blk >= n / kRow) return;
  uint32_t* dst = a.dst + item * a.dst_item_stride + (uint64_t)y * n + blk * kRow;
  if (y >= a.own_lo && y < a.own_lo + a.own_n) {
    const uint32_t* s = a.own_src + item * a.own_item_stride + (uint64_t)y * n + blk * kRow;
    uint32_t x[16];
    load_C(x, s, lane);
    store_C(dst, x, lane);
    return;
  }
  const uint32_t tp = a.level ? (y < a.level ? a.prime0 + y : T.L + (y - a.level)) : a.prime0 + y;
  const uint32_t q = T.q[tp];
  const uint32_t* src = (a.use_srcs ? a.srcs[item] : a.src + item * a.src_item_stride) + (uint64_t)y * n + blk * kRow;
  uint32_t x[16];
  if (FWD) {
    load_A(x, src, lane);
    row_fwd<true, BIG>(x, lane, n / kRow + blk, T.tw + (uint64_t)tp * n, q, T.qinv[tp], lds[wave], T.one[tp]);
    if (a.cmb) {
      const uint2 f = a.cmb_factor[y];
      uint32_t c[16];
      load_C(c, a.cmb + item * a.cmb_item_stride + (uint64_t)y * n + blk * kRow, lane);
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] = mul_const(sub_mod(c[r], x[r], q), f.x, f.y, q);
    }
    store_C(dst, x, lane);
  } else {
    load_C(x, src, lane);
    if constexpr (MUL) {
      const Mod md{q, T.qinv[tp]};
      const uint2 r2 = T.r2[tp];
      const uint32_t* src2 = a.src2 + item * a.src_item_stride + (uint64_t)y * n + blk * kRow;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint4 v = *reinterpret_cast<const uint4*>(src2 + 4 * lane + 256 * g);
        x[4 * g] = prod_mod(x[4 * g], v.x, md, r2);
        x[4 * g + 1] = prod_mod(x[4 * g + 1], v.y, md, r2);
        x[4 * g + 2] = prod_mod(x[4 * g + 2], v.z, md, r2);
        x[4 * g + 3] = prod_mod(x[4 * g + 3], v.w, md, r2);
      }
    }
    row_inv(x, lane, n / kRow + blk, T.itw + (uint64_t)tp * n, q, T.qinv[tp], lds[wave]);
    store_A(dst, x, lane);
  }
}

// BCAST: every limb y starts from the same coefficients a.bsrc (one polynomial per
// item, any values < 2^32), reduced modulo its prime, instead of its own data.
// BIG (forward only): every prime of the chain exceeds 2^31, so the butterflies run on
// lazy values with one correction at the end.
template <bool FWD, int LOGC, bool BCAST = false, bool BIG = false>
__global__ __launch_bounds__(64) void k_col(DevTables T, ColArgs a, uint32_t scale) {
  constexpr int C = 1 << LOGC;
  const uint32_t c = blockIdx.x * 64 + threadIdx.x;
  const uint32_t y = blockIdx.y, item = blockIdx.z;
  const uint32_t n = T.n;
  const uint32_t tp = a.prime0 + y;
  const uint32_t q = T.q[tp];
  uint32_t* p = a.data + item * a.item_stride + (uint64_t)y * n + c;
  uint32_t v[C];
  if constexpr (BCAST) {
    const uint32_t* b = a.bsrc + item * a.bsrc_item_stride + c;
    const uint2 one = T.one[tp];
#pragma unroll
    for (int k = 0; k < C; ++k) v[k] = mul_const(b[k * kRow], one.x, one.y, q);
  } else {
#pragma unroll
    for (int k = 0; k < C; ++k) v[k] = p[k * kRow];
  }
  if constexpr (FWD && BIG) {
    col_fwd<LOGC, true>(v, T.tw + (uint64_t)tp * n, q, T.qinv[tp]);
    canon_big(v, q);
  } else if constexpr (FWD) {
    col_fwd<LOGC, false>(v, T.tw + (uint64_t)tp * n, q, T.qinv[tp]);
  }
  if constexpr (!FWD) col_inv<LOGC>(v, T.itw + (uint64_t)tp * n, q, T.qinv[tp]);
  if (scale) {
    const uint2 s = T.ninv[tp];
#pragma unroll
    for (int k = 0; k < C; ++k) v[k] = mul_const(v[k], s.x, s.y, q);
  }
#pragma unroll
  for (int k = 0; k < C; ++k) p[k * kRow] = v[k];
}

// Forward column NTT (stages N/2..1024) of one column held by G consecutive lanes
// (G = 1, 2 or 4): lane z holds rows z + G*i.  Stages of half-distance h >= G stay
// in the lane (their twiddles are the same for all G lanes); the last log2(G)
// stages pair lanes z and z ^ h and exchange values by lane shuffles.  All G lanes
// of a column must be active.  LAZY as in ct_bfly.
template <int LOGC, int G, bool LAZY>
__device__ __forceinline__ void col_fwd_lanes_body(uint32_t (&v)[(1 << LOGC) / G], const uint32_t* __restrict__ tw,
                                                   const Mod& md, uint32_t z) {
  constexpr int C = 1 << LOGC, R = C / G;
  static_assert(G == 1 || G == 2 || G == 4, "lanes per column");
  const uint32_t q = md.q;
  if constexpr (G == 1) {
    col_fwd<LOGC, LAZY>(v, tw, q, md.qinv);
  } else {
#pragma unroll
    for (int s = 0; s < LOGC; ++s) {
      const int m = 1 << s, h = C >> (s + 1);
      if (h >= G) {  // butterflies (i, i + h/G) within the lane
        const int hi = h / G;
#pragma unroll
        for (int ig = 0; ig < m; ++ig) {
          const uint32_t w = tw[m + ig];
#pragma unroll
          for (int t = 0; t < hi; ++t) ct_bfly<LAZY>(v[2 * hi * ig + t], v[2 * hi * ig + t + hi], w, md.qinv, q);
        }
      } else {  // rows z + G*i and its partner in lane z ^ h; group (G*i)/(2h) + (z >> log2(2h))
        const bool lo = (z & (uint32_t)h) == 0;
#pragma unroll
        for (int i = 0; i < R; ++i) {
          const int g0 = G * i / (2 * h);
          uint32_t w = tw[m + g0];
          if (2 * h < G) w = (z & (uint32_t)(2 * h)) ? tw[m + g0 + 1] : w;  // G = 4, h = 1
          const uint32_t other = __shfl_xor(v[i], h);
          const uint32_t t = mul_const(lo ? other : v[i], w, w * md.qinv, q);
          if constexpr (LAZY) v[i] = lo ? lazy_add(v[i], t, q) : lazy_sub(other, t, q);
          else v[i] = lo ? add_mod(v[i], t, q) : sub_mod(other, t, q);
        }
      }
    }
  }
}

// The same with canonical outputs: lazy butterflies and one final correction when
// q > 2^31 (a lazy value is then below 2q), canonical butterflies otherwise.
template <int LOGC, int G>
__device__ __forceinline__ void col_fwd_lanes(uint32_t (&v)[(1 << LOGC) / G], const uint32_t* __restrict__ tw,
                                              const Mod& md, uint32_t z) {
  if (md.q >> 31) {
    col_fwd_lanes_body<LOGC, G, true>(v, tw, md, z);
    canon_big(v, md.q);
  } else {
    col_fwd_lanes_body<LOGC, G, false>(v, tw, md, z);
  }
}

// One (target, column) task of the conversion's second phase: the target limb's
// values on the column's C rows (sum over sources of y_s * c_s, reduced), then its
// column NTT, stored.  G consecutive lanes (G = 1, 2 or 4) share the task: lane z
// holds rows z + G*i.
// The target of a task: its destination limb, prime, and the conversion constants
// of every source split into 16-bit halves (zero past the last source).
template <int MAXS>
struct ConvTarget {
  uint32_t cl[MAXS], ch[MAXS];
  Mod md;
  uint32_t dl, tp;
};

template <int MAXS>
__device__ __forceinline__ ConvTarget<MAXS> conv_target(const DevTables& T, const ConvArgs& a, uint32_t e, uint32_t ns,
                                                        uint32_t skip_lo, uint32_t y) {
  ConvTarget<MAXS> k;
  k.dl = (a.skip && e >= skip_lo) ? e + ns : e;
  k.tp = a.level ? (k.dl < a.level ? k.dl : T.L + (k.dl - a.level)) : k.dl;
  k.md = Mod{T.q[k.tp], T.qinv[k.tp]};
  const uint32_t* cv = a.conv + y * a.conv_y + (a.conv_by_abs ? k.tp : k.dl);
#pragma unroll
  for (int s = 0; s < MAXS; ++s) {
    const uint32_t w = (uint32_t)s < ns ? cv[s * a.conv_s] : 0u;  // zero weight past the last source
    k.cl[s] = w & 0xffffu;
    k.ch[s] = w >> 16;
  }
  return k;
}

template <int LOGC, int CW, int MAXS, int G, bool BIG>
__device__ __forceinline__ void conv_task(const DevTables& T, const ConvArgs& a, const uint32_t* ys, uint32_t* dst,
                                          const ConvTarget<MAXS>& k, uint32_t c, uint32_t z, uint32_t col0) {
  constexpr int C = 1 << LOGC, R = C / G;
  const uint32_t n = T.n;
  const uint32_t dl = k.dl, tp = k.tp;
  const Mod md = k.md;
  const uint32_t* cl = k.cl;
  const uint32_t* ch = k.ch;
  uint32_t v[R];
  static_for<R>([&](auto kc) {
    constexpr int i = decltype(kc)::value;
    const uint32_t* yr = ys + ((z + G * i) * CW + c) * MAXS;
    uint64_t A = 0, B = 0;
    static_for<MAXS / 4>([&](auto sc4) {
      constexpr int s4 = decltype(sc4)::value;
      const uint4 y4 = *reinterpret_cast<const uint4*>(yr + 4 * s4);
      A += (uint64_t)y4.x * ch[4 * s4] + (uint64_t)y4.y * ch[4 * s4 + 1];
      A += (uint64_t)y4.z * ch[4 * s4 + 2] + (uint64_t)y4.w * ch[4 * s4 + 3];
      B += (uint64_t)y4.x * cl[4 * s4] + (uint64_t)y4.y * cl[4 * s4 + 1];
      B += (uint64_t)y4.z * cl[4 * s4 + 2] + (uint64_t)y4.w * cl[4 * s4 + 3];
    });
    Acc96 acc;
    acc.lo = B + (A << 16);
    acc.hi = (uint32_t)(A >> 48) + (acc.lo < B ? 1u : 0u);
    v[i] = acc_redc2(acc, md);
  });
  if constexpr (BIG) {  // every prime above 2^31: lazy butterflies, one final correction
    col_fwd_lanes_body<LOGC, G, true>(v, T.tw + (uint64_t)tp * n, md, z);
    canon_big(v, md.q);
  } else {
    col_fwd_lanes_body<LOGC, G, false>(v, T.tw + (uint64_t)tp * n, md, z);
  }
  uint32_t* pd = dst + (uint64_t)dl * n + col0 + c;
#pragma unroll
  for (int i = 0; i < R; ++i) pd[(z + G * i) * kRow] = v[i];
}

// Fused: column INTT of each source limb, scale, fast base conversion to every
// target limb, column NTT of each target.  Grid: x = column tile (CW columns),
// y = source group (digit or ModDown part), z = item.  Phase 1 leaves the scaled
// source values in LDS as ys[row][column][s] (s fastest, MAXS per slot) so that
// phase 2 reads one row of all sources with 16-byte loads.  Each conversion
// constant c < 2^32 is split as c = ch*2^16 + cl and the products are summed in
// two carry-free 64-bit accumulators (each term < 2^48): S = A*2^16 + B.
// BIG: every prime of the chain exceeds 2^31, so the column NTTs run on lazy values.
// NTH: threads per workgroup (256 or 512; chosen per launch from the task count).
template <int LOGC, int CW, int MAXS, bool BIG, int NTH>
__global__ __launch_bounds__(NTH) __attribute__((amdgpu_waves_per_eu(4, 8))) void k_conv(DevTables T, ConvArgs a) {
  constexpr int C = 1 << LOGC;
  extern __shared__ uint32_t ys[];  // [C][CW][MAXS]
  const uint32_t col0 = blockIdx.x * CW, y = blockIdx.y / a.tchunks, chunk = blockIdx.y % a.tchunks;
  const uint32_t item = blockIdx.z;
  const uint32_t n = T.n;
  const uint32_t p0 = a.src_prime0 + y * a.src_prime_step;
  const uint32_t ns = min(a.ns_max, a.ns_limit - y * a.src_prime_step);
  const uint32_t* src = a.src + item * a.src_item + y * a.src_y;
  // ModUp: the digit's own limbs [p0, p0 + ns) of the extended basis are not targets
  const uint32_t skip_lo = p0;
  const uint32_t n_targets = a.skip ? a.level + T.K - ns : a.n_targets;
  const uint32_t per = (n_targets + a.tchunks - 1) / a.tchunks;
  const uint32_t e0 = chunk * per, e1 = min(n_targets, e0 + per);
  // (target, column) tasks: whole rounds of one task per thread, then a last partial
  // round spread over the first rem*G threads, G = 4 or 2 per task, when it fits
  const uint32_t ntask = (e1 > e0 ? e1 - e0 : 0u) * CW, nth = blockDim.x;
  const uint32_t full = ntask / nth * nth, rem = ntask - full;
  const uint32_t G = (LOGC >= 4 && rem) ? (nth >= 4 * rem ? 4u : nth >= 2 * rem ? 2u : 1u) : 1u;
  const bool coop = G > 1;
  const uint32_t nfirst = coop ? full : ntask;
  // Phase 1: one (source, column) task per thread (ns * CW <= 256 <= NTH).  The
  // threads without one load the constants of their first phase-2 task meanwhile,
  // so that latency passes during phase 1 (on the phase-1 path they are not live).
  static_assert(16 * CW <= NTH, "one phase-1 task per thread");
  const bool has_first = threadIdx.x < nfirst;
  ConvTarget<MAXS> first;
  const uint32_t task1 = threadIdx.x;
  // two lanes per (source, column) when the workgroup has the threads for it
  const bool pair = 2 * ns * CW <= nth;
  if (task1 >= (pair ? 2 : 1) * ns * CW) {
    if (has_first) first = conv_target<MAXS>(T, a, e0 + threadIdx.x / CW, ns, skip_lo, y);
  } else if (pair) {
    __builtin_amdgcn_s_setprio(2);
    const uint32_t pt = task1 >> 1, z = task1 & 1;
    const uint32_t s = pt / CW, c = pt - s * CW;
    const uint32_t tp = p0 + s;
    const uint32_t q = T.q[tp];
    constexpr int H = C / 2;
    uint32_t v[H];
    const uint32_t* ps = src + (uint64_t)s * n + col0 + c + (uint64_t)z * H * kRow;
#pragma unroll
    for (int k = 0; k < H; ++k) v[k] = ps[k * kRow];
    col_inv_scaled_pair<LOGC>(v, z, T.itw + (uint64_t)tp * n, q, T.qinv[tp], a.scale[y * a.scale_y + s]);
#pragma unroll
    for (int k = 0; k < H; ++k) ys[((z * H + k) * CW + c) * MAXS + s] = v[k];
    if (has_first) first = conv_target<MAXS>(T, a, e0 + threadIdx.x / CW, ns, skip_lo, y);
    __builtin_amdgcn_s_setprio(0);
  } else {
    // The rest of the workgroup waits at the barrier for these waves, while the other
    // workgroup on the CU competes for the SIMDs: raise their issue priority meanwhile.
    __builtin_amdgcn_s_setprio(2);
    const uint32_t task = task1;
    const uint32_t s = task / CW, c = task - s * CW;
    const uint32_t tp = p0 + s;
    const uint32_t q = T.q[tp];
    uint32_t v[C];
    const uint32_t* ps = src + (uint64_t)s * n + col0 + c;
#pragma unroll
    for (int k = 0; k < C; ++k) v[k] = ps[k * kRow];
    col_inv_scaled<LOGC>(v, T.itw + (uint64_t)tp * n, q, T.qinv[tp], a.scale[y * a.scale_y + s]);
#pragma unroll
    for (int k = 0; k < C; ++k) ys[(k * CW + c) * MAXS + s] = v[k];
    if (has_first) first = conv_target<MAXS>(T, a, e0 + threadIdx.x / CW, ns, skip_lo, y);
    __builtin_amdgcn_s_setprio(0);
  }
  __syncthreads();
  uint32_t* dst = a.dst + item * a.dst_item + y * a.dst_y;
  if (has_first) conv_task<LOGC, CW, MAXS, 1, BIG>(T, a, ys, dst, first, threadIdx.x % CW, 0, col0);
  for (uint32_t task = threadIdx.x + nth; task < nfirst; task += nth)
    conv_task<LOGC, CW, MAXS, 1, BIG>(T, a, ys, dst, conv_target<MAXS>(T, a, e0 + task / CW, ns, skip_lo, y),
                                      task % CW, 0, col0);
  if constexpr (LOGC >= 4) {
    if (coop && threadIdx.x < rem * G) {  // whole groups of G lanes: G divides 64
      const uint32_t task = full + threadIdx.x / G, z = threadIdx.x % G;
      const ConvTarget<MAXS> k = conv_target<MAXS>(T, a, e0 + task / CW, ns, skip_lo, y);
      if (G == 2) conv_task<LOGC, CW, MAXS, 2, BIG>(T, a, ys, dst, k, task % CW, z, col0);
      else conv_task<LOGC, CW, MAXS, 4, BIG>(T, a, ys, dst, k, task % CW, z, col0);
    }
  }
}

// ------------------------------------------------------------------ conversion on the matrix cores

typedef int mx_v4 __attribute__((ext_vector_type(4)));
typedef int mx_v16 __attribute__((ext_vector_type(16)));

// x * 2^-32 mod q for x < q * 2^32 (subtract-form Montgomery reduction).
__device__ __forceinline__ uint32_t redc64(uint64_t x, const Mod& md) {
  const uint32_t xl = (uint32_t)x, xh = (uint32_t)(x >> 32);
  const uint32_t u = __umulhi(xl * md.qinv, md.q);  // x - m*q vanishes mod 2^32 for m = xl * q^-1
  const uint32_t r = xh - u;
  return xh < u ? r + md.q : r;
}

// Column NTTs of the staged targets tl < ng (staging stg[tl][row][column], kStg words
// per target), G lanes per (target, column), stored to the target limbs.
template <int G>
__device__ __forceinline__ void mx_ntt_store(const DevTables& T, const ConvArgs& a, const uint32_t* stg,
                                             uint32_t kStg, uint32_t* dst, uint32_t g0, uint32_t ng, uint32_t ns,
                                             uint32_t skip_lo, uint32_t col0) {
  constexpr int LOGC = 6, C = 64, CW = 16, R = C / G;
  const uint32_t slot = threadIdx.x / G, z = threadIdx.x % G;
  const uint32_t tl = slot / CW, c = slot % CW;
  if (tl >= ng) return;  // all G lanes of a slot leave together
  const uint32_t e = g0 + tl;
  const uint32_t dl = (a.skip && e >= skip_lo) ? e + ns : e;
  const uint32_t tp = a.level ? (dl < a.level ? dl : T.L + (dl - a.level)) : dl;
  const Mod md{T.q[tp], T.qinv[tp]};
  uint32_t v[R];
  const uint32_t* sp = stg + tl * kStg + z * CW + c;
#pragma unroll
  for (int i = 0; i < R; ++i) v[i] = sp[G * i * CW];
  col_fwd_lanes<LOGC, G>(v, T.tw + (uint64_t)tp * T.n, md, z);
  uint32_t* pd = dst + (uint64_t)dl * T.n + col0 + c;
#pragma unroll
  for (int i = 0; i < R; ++i) pd[(z + G * i) * kRow] = v[i];
}

// The fused conversion of k_conv (ring 2^16, 16 columns, up to 12 sources) with the
// sums over sources on the matrix cores.  Every scaled source value y < 2^32 and
// every constant c < 2^32 is cut into five 7-bit digits, so that for each target
//   sum_s y_s c_s = sum_{e=0..8} 2^(7e) D_e,   D_e = sum_s sum_{a+b=e} y_{s,a} c_{s,b} < 2^20,
// and the D_e of two targets and 32 coefficients are one exact int8 product
// (v_mfma_i32_32x32x32_i8, two K steps of 32) of a constant tile A (rows: target
// pair x digit position e, from the operand table) and the coefficients' digits B.
// The sum is then sum_e D_e W_e with W_e = 2^(7e+32) mod q (nine 64-bit multiply-adds)
// and one Montgomery reduction, bit-identical to the vector path's result.
// K layout (the same in A and B): lane half h, K step kappa, byte i hold source
// s = 6h + g/5 and digit a = g%5 of g = 16*kappa + i (g = 30, 31 are zero).
// Wave w owns coefficients of rows 16w..16w+15 (eight tiles of 32: rows 16w + 2j and
// 16w + 2j + 1, all 16 columns), keeps their digits in registers, and runs all target
// tiles; D's layout puts digit position e in register e of a lane, target (l >> 5) of
// the pair and coefficient l & 31.  Targets go in groups of 8 through an LDS staging
// area (over the source values, no longer needed) to the column NTTs, 2 or 4 lanes per
// (target, column).
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 8))) void k_conv_mx(DevTables T, ConvArgs a) {
  constexpr int LOGC = 6, C = 64, CW = 16, MAXS = 12;
  constexpr uint32_t kStg = C * CW + 32;  // staging words per target (the pad spreads target pairs over banks)
  extern __shared__ uint32_t ys[];        // [C][CW][MAXS], then staging [8][kStg]
  const uint32_t col0 = blockIdx.x * CW, y = blockIdx.y / a.tchunks, chunk = blockIdx.y % a.tchunks;
  const uint32_t item = blockIdx.z;
  const uint32_t n = T.n;
  const uint32_t p0 = a.src_prime0 + y * a.src_prime_step;
  const uint32_t ns = min(a.ns_max, a.ns_limit - y * a.src_prime_step);
  const uint32_t* src = a.src + item * a.src_item + y * a.src_y;
  for (uint32_t task = threadIdx.x; task < ns * CW; task += blockDim.x) {
    const uint32_t s = task / CW, c = task - s * CW;
    const uint32_t tp = p0 + s;
    const uint32_t q = T.q[tp];
    uint32_t v[C];
    const uint32_t* ps = src + (uint64_t)s * n + col0 + c;
#pragma unroll
    for (int k = 0; k < C; ++k) v[k] = ps[k * kRow];
    col_inv_scaled<LOGC>(v, T.itw + (uint64_t)tp * n, q, T.qinv[tp], a.scale[y * a.scale_y + s]);
#pragma unroll
    for (int k = 0; k < C; ++k) ys[(k * CW + c) * MAXS + s] = v[k];
  }
  __syncthreads();
  // B operands: the digits of this wave's eight coefficient tiles (sources past ns hold
  // stale values; their constants in A are zero)
  const uint32_t wave = threadIdx.x >> 6, lane = threadIdx.x & 63, n32 = lane & 31, hh = lane >> 5;
  mx_v4 bop[8][2];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t row = 16 * wave + 2 * j + (n32 >> 4), col = n32 & 15;
    const uint32_t* yp = ys + (row * CW + col) * MAXS + 6 * hh;
    uint32_t yv[6];
#pragma unroll
    for (int s = 0; s < 6; s += 2) {
      const uint2 t2 = *reinterpret_cast<const uint2*>(yp + s);
      yv[s] = t2.x;
      yv[s + 1] = t2.y;
    }
    uint32_t dg[32];
#pragma unroll
    for (int g = 0; g < 32; ++g) dg[g] = g < 30 ? (yv[g / 5] >> (7 * (g % 5))) & 127u : 0u;
#pragma unroll
    for (int kap = 0; kap < 2; ++kap) {
      uint32_t wd[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int g = 16 * kap + 4 * u;
        wd[u] = dg[g] | (dg[g + 1] << 8) | (dg[g + 2] << 16) | (dg[g + 3] << 24);
      }
      bop[j][kap] = mx_v4{(int)wd[0], (int)wd[1], (int)wd[2], (int)wd[3]};
    }
  }
  __syncthreads();  // the source values' LDS becomes the staging area
  uint32_t* stg = ys;
  uint32_t* dst = a.dst + item * a.dst_item + y * a.dst_y;
  const uint32_t skip_lo = p0;
  const uint32_t n_targets = a.skip ? a.level + T.K - ns : a.n_targets;
  // chunks start on an even target, so target pairs match the operand table's tiles
  const uint32_t per = (((n_targets + a.tchunks - 1) / a.tchunks) + 1) & ~1u;
  const uint32_t e0 = min(n_targets, chunk * per), e1 = min(n_targets, e0 + per);
  const mx_v4* atab = reinterpret_cast<const mx_v4*>(a.mx) + (uint64_t)y * a.mx_y + lane;
  uint32_t* srow = stg + hh * kStg + (16 * wave + (n32 >> 4)) * CW + (n32 & 15);
  for (uint32_t g0 = e0; g0 < e1; g0 += 8) {
    const uint32_t ng = min(8u, e1 - g0);
    for (uint32_t mt = 0; 2 * mt < ng; ++mt) {
      const uint32_t ea = g0 + 2 * mt;  // even: tile ea / 2 of the table
      const mx_v4 a0 = atab[(ea / 2) * 128], a1 = atab[(ea / 2) * 128 + 64];
      // this lane's target; a pair's missing second target borrows the first's
      // prime (its sums are staged but never stored)
      const uint32_t e = min(ea + hh, e1 - 1);
      const uint32_t dl = (a.skip && e >= skip_lo) ? e + ns : e;
      const uint32_t tp = a.level ? (dl < a.level ? dl : T.L + (dl - a.level)) : dl;
      const Mod md{T.q[tp], T.qinv[tp]};
      const uint4 w0 = T.mx_w[3 * tp], w1 = T.mx_w[3 * tp + 1], w2 = T.mx_w[3 * tp + 2];
      const uint32_t W[9] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w, w2.x};
      uint32_t* sp = srow + 2 * mt * kStg;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        mx_v16 d = {};
        d = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, bop[j][0], d, 0, 0, 0);
        d = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, bop[j][1], d, 0, 0, 0);
        uint64_t acc = 0;
#pragma unroll
        for (int r = 0; r < 9; ++r) acc += (uint64_t)(uint32_t)d[r] * W[r];
        sp[2 * j * CW] = redc64(acc, md);
      }
    }
    __syncthreads();
    // 4 lanes per (target, column): 64 columns per pass of the workgroup
    mx_ntt_store<4>(T, a, stg, kStg, dst, g0, min(ng, 4u), ns, skip_lo, col0);
    if (ng > 4) mx_ntt_store<4>(T, a, stg + 4 * kStg, kStg, dst, g0 + 4, ng - 4, ns, skip_lo, col0);
    __syncthreads();
  }
}

// NTT-domain Galois permutation: position j holds the value at psi^(2 brv(j)+1);
// sigma_g(a)[j] = a[pi(j)] with 2 brv(pi(j)) + 1 = (2 brv(j) + 1) g mod 2N.
__device__ __forceinline__ uint32_t galois_src(uint32_t j, uint32_t g, uint32_t log_n) {
  const uint32_t sh = 32 - log_n;
  const uint32_t e = 2 * (__brev(j) >> sh) + 1;
  const uint32_t e2 = (e * g) & ((2u << log_n) - 1);
  return __brev((e2 - 1) >> 1) >> sh;
}

// The two kernels that use the key.  FINAL = false: special primes p_k; the
// inner product is followed by the row INTT of ModDown and written to tmpP.
// FINAL = true: ciphertext primes q_i; the inner product meets the converted
// special part (conv, row NTT pending) and c0:
//   out_b = (acc_b - conv_b) * P^-1 + sigma(c0),  out_a = (acc_a - conv_a) * P^-1.
// Grid: x = limb, y = 1024-block, z = key group; waves take ciphertexts in turn.
// The row transforms take `lane + opaque_zero()`: their per-lane addresses are
// recomputed in the loops, which keeps these kernels within 128 VGPRs.
// TENSOR (final pass of a relinearisation): the ciphertext is the tensor product
// (x0 y0, x0 y1 + x1 y0, x1 y1) of ct = x and a.ty = y, formed here from x and y:
// x0 y0 is the c0 term, x1 y1 the own digit, and x0 y1 + x1 y0 is added to the a-half.
// BIG: every prime of the chain exceeds 2^31 (the canonical form of conv's transform
// then needs no branch on q).
template <bool FINAL, int WAVES, bool TENSOR = false, bool BIG = false>
__device__ __forceinline__ void ip_body(const DevTables& T, const IpArgs& a) {
  extern __shared__ uint32_t smem[];
  const uint32_t wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint32_t u = xcd_logical_id();
  if (u >= gridDim.x * gridDim.y * gridDim.z) return;  // guard (the map is a bijection)
  // wave-uniform indices (the divisions run on the vector unit; keep the results scalar)
  const uint32_t blk = __builtin_amdgcn_readfirstlane(u % gridDim.y);
  const uint32_t kg = __builtin_amdgcn_readfirstlane((u / gridDim.y) % gridDim.z);
  const uint32_t limb = __builtin_amdgcn_readfirstlane(u / (gridDim.y * gridDim.z));
  const uint32_t n = T.n, L = T.L, K = T.K, E = T.L + T.K, nd = a.nd, level = a.level;
  const uint32_t tabs = FINAL ? limb : L + limb;
  const uint32_t elimb = FINAL ? limb : level + limb;
  const uint32_t q = T.q[tabs];
  const Mod md{q, T.qinv[tabs]};
  const uint32_t* tw = T.tw + (uint64_t)tabs * n;
  const KeyRef& key = a.key[kg];
  // Key rows of this (prime, block).  Several waves share them: staged in LDS.
  // One wave: b (and a stored a) read straight from memory; only a regenerated
  // a-half lives in LDS (which keeps single-wave workgroups small).
  constexpr bool kStage = WAVES > 1;
  const bool a_in_lds = kStage || !key.a;
  const uint32_t tile_words = (a_in_lds ? nd * kRow : 0u) + (kStage ? nd * kRow : 0u);
  uint32_t* Atile = smem;                                   // a rows [nd][1024]
  uint32_t* Btile = smem + nd * kRow;                       // b rows [nd][1024] (staged only)
  // Several waves also share the twiddles of this prime's blocks: the final pass's
  // conv transform uses block blk, the digits' transforms block sblk (their source
  // under sigma_g), the special pass's inverse transform block blk.  Staged in LDS
  // (two tables of 1024 entries), they replace per-lane loads from the limb's table
  // in the middle of each transform.  With eight waves each entry also carries its
  // Montgomery companion (8 KB a table), which saves the transforms a multiply per
  // twiddle; the four-wave kernel keeps 4 KB tables, so that three of its workgroups
  // still fit a CU.
  constexpr bool kTwc = WAVES == 8;
  using TwT = std::conditional_t<kTwc, uint2, uint32_t>;
  TwT* twA = reinterpret_cast<TwT*>(smem + tile_words);     // sblk's forward twiddles (staged only)
  TwT* twB = twA + kRow;                                    // blk's forward (FINAL) or inverse twiddles
  const uint32_t stw = kStage ? (kTwc ? 4 : 2) * kRow : 0u;
  uint32_t* priv = smem + tile_words + stw + wave * kRowPad;  // wave-private block
  uint32_t* cnt = smem + tile_words + stw + WAVES * kRowPad;  // expander scratch
  const uint32_t sblk = galois_src(blk * kRow, key.galois, T.log_n) >> 10;

  if (kStage) {
    for (uint32_t i = threadIdx.x; i < nd * (kRow / 4); i += blockDim.x) {
      const uint32_t j = i / (kRow / 4), w4 = i - j * (kRow / 4);
      const uint64_t off = ((uint64_t)j * E + tabs) * n + blk * kRow + 4 * w4;
      *reinterpret_cast<uint4*>(Btile + j * kRow + 4 * w4) = *reinterpret_cast<const uint4*>(key.b + off);
      if (key.a) *reinterpret_cast<uint4*>(Atile + j * kRow + 4 * w4) = *reinterpret_cast<const uint4*>(key.a + off);
    }
    if constexpr (kTwc) {
      stage_block_twiddles(twA, tw, n / kRow + sblk, md.qinv);
      stage_block_twiddles(twB, FINAL ? tw : T.itw + (uint64_t)tabs * n, n / kRow + blk, md.qinv);
    } else {
      stage_block_twiddles(twA, tw, n / kRow + sblk);
      stage_block_twiddles(twB, FINAL ? tw : T.itw + (uint64_t)tabs * n, n / kRow + blk);
    }
  }
  if (!key.a) {
    uint32_t seed[8];
    for (int i = 0; i < 8; ++i) seed[i] = key.seed[i];
    regen_tiles(seed, 0, nd, tabs, blk, q, T.bound[tabs], T.one[tabs], a.regen_blocks, Atile, cnt);
  }
  __syncthreads();
  // twiddle sources and offsets of the three kinds of row transform
  const TwT* tw_dig;
  const TwT* tw_blk;
  uint32_t off_dig, off_blk;
  if constexpr (kStage) {
    tw_dig = twA;
    tw_blk = twB;
    off_dig = off_blk = 1u;
  } else {
    tw_dig = tw;
    tw_blk = FINAL ? tw : T.itw + (uint64_t)tabs * n;
    off_dig = n / kRow + sblk;
    off_blk = n / kRow + blk;
  }
  const uint32_t* kb_row = kStage ? Btile : key.b + (uint64_t)tabs * n + blk * kRow;
  const uint32_t* ka_row = a_in_lds ? Atile : key.a + (uint64_t)tabs * n + blk * kRow;
  const uint64_t bstride = kStage ? kRow : (uint64_t)E * n;   // digit stride of kb_row
  const uint64_t kstride = a_in_lds ? kRow : (uint64_t)E * n; // digit stride of ka_row

  // this lane's 16 output positions (layout C) and their sources under sigma_g
  uint32_t sidx[16];  // padded LDS position of each output's source within block sblk
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const uint32_t rout = 4 * lane + 256 * (r >> 2) + (r & 3);
    sidx[r] = swz(galois_src(blk * kRow + rout, key.galois, T.log_n) & (kRow - 1));
  }
  const uint32_t own_digit = FINAL ? limb / T.alpha : 0xffffffffu;
  const uint32_t nq = WAVES == 8 ? (0u - q) + opaque_zero() : 0u;  // 2^32 - q, opaque: see lazy_sub_mont

#pragma unroll 1
  for (uint32_t c = wave; c < a.n_ct; c += WAVES) {
    const uint32_t item = kg * a.n_ct + c;
    const uint32_t* ext = a.ext + (a.per_group ? kg : c) * a.ext_ct_stride;
    const uint32_t* ct = a.per_group ? key.ct : a.ct + c * a.ct_ct_stride;
    const uint32_t* cy = TENSOR ? a.ty + c * a.ct_ct_stride : nullptr;  // y of a tensor product
    uint32_t* out = a.per_group ? key.out : a.out + (uint64_t)item * 2 * level * n;
    // inner product: sum_j sigma(d_j) * key_j, each product Montgomery-reduced (factor 2^-32).
    // FINAL: the accumulators start from conv (its row NTT done first), so no extra block is
    // live next to both, and the products are subtracted: they end as conv - sum (lazy
    // values, only multiplied afterwards), and the final constant is negated.  The
    // multi-wave kernels keep conv's transform canonical: skipping that step there let
    // the compiler schedule the two transforms in a way that ran the kernel 17% slower,
    // while the single-wave kernel gains from skipping it.
    uint32_t rb[16], ra[16];
    if constexpr (FINAL) {
      load_A(rb, a.conv + (((uint64_t)item * 2 + 0) * level + limb) * n + blk * kRow, lane);
      row_fwd<(WAVES > 1), BIG>(rb, lane + opaque_zero(), off_blk, tw_blk, q, md.qinv, priv, T.one[tabs]);
      load_A(ra, a.conv + (((uint64_t)item * 2 + 1) * level + limb) * n + blk * kRow, lane);
      row_fwd<(WAVES > 1), BIG>(ra, lane + opaque_zero(), off_blk, tw_blk, q, md.qinv, priv, T.one[tabs]);
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) { rb[r] = 0; ra[r] = 0; }
    }
#pragma unroll 1
    for (uint32_t j = 0; j < nd; ++j) {
      uint32_t x[16];
      if (a.digits_ntt) {
        load_C(x, ext + ((uint64_t)j * E + elimb) * n + sblk * kRow, lane);
      } else if (FINAL && j == own_digit) {
        load_C(x, ct + ((uint64_t)level + limb) * n + sblk * kRow, lane);
        if constexpr (TENSOR) {  // c1 = x1 y1
          const uint2 r2 = T.r2[tabs];
          const uint32_t* py = cy + ((uint64_t)level + limb) * n + sblk * kRow;
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const uint4 v = *reinterpret_cast<const uint4*>(py + 4 * lane + 256 * g);
            x[4 * g] = prod_mod(x[4 * g], v.x, md, r2);
            x[4 * g + 1] = prod_mod(x[4 * g + 1], v.y, md, r2);
            x[4 * g + 2] = prod_mod(x[4 * g + 2], v.z, md, r2);
            x[4 * g + 3] = prod_mod(x[4 * g + 3], v.w, md, r2);
          }
        }
      } else {
        load_A(x, ext + ((uint64_t)j * E + elimb) * n + sblk * kRow, lane);
        row_fwd<false>(x, lane + opaque_zero(), off_dig, tw_dig, q, md.qinv, priv, T.one[tabs]);  // lazy: only multiplied
      }
      lds_put_C(priv, x, lane);
      wave_sync();
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint32_t rout = 4 * lane + 256 * g;
        const uint4 kb = *reinterpret_cast<const uint4*>(kb_row + j * bstride + rout);
        const uint4 ka = *reinterpret_cast<const uint4*>(ka_row + j * kstride + rout);
        const uint32_t kbv[4] = {kb.x, kb.y, kb.z, kb.w}, kav[4] = {ka.x, ka.y, ka.z, ka.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int r = 4 * g + u;
          const uint32_t v = priv[sidx[r]];
          if constexpr (FINAL) {  // lazy accumulators (only multiplied afterwards)
            if constexpr (WAVES == 8) {  // (in the smaller kernels this form cost registers)
              rb[r] = lazy_sub_mont(rb[r], v, kbv[u], md, nq);
              ra[r] = lazy_sub_mont(ra[r], v, kav[u], md, nq);
            } else {
              rb[r] = lazy_sub(rb[r], mont_mul(v, kbv[u], md), q);
              ra[r] = lazy_sub(ra[r], mont_mul(v, kav[u], md), q);
            }
          } else {  // canonical: the row INTT follows
            rb[r] = add_mod(rb[r], mont_mul(v, kbv[u], md), q);
            ra[r] = add_mod(ra[r], mont_mul(v, kav[u], md), q);
          }
        }
      }
      wave_sync();
    }
    if (!FINAL) {
      row_inv(rb, lane + opaque_zero(), off_blk, tw_blk, q, md.qinv, priv);
      store_A(a.tmpP + (((uint64_t)item * 2 + 0) * K + limb) * n + blk * kRow, rb, lane);
      __builtin_amdgcn_sched_barrier(0);
      row_inv(ra, lane + opaque_zero(), off_blk, tw_blk, q, md.qinv, priv);
      store_A(a.tmpP + (((uint64_t)item * 2 + 1) * K + limb) * n + blk * kRow, ra, lane);
    } else {
      // -(2^32 P^-1) in Montgomery form: the accumulators hold conv - sum
      const uint32_t fn = T.md_fin_ks[limb].x ? q - T.md_fin_ks[limb].x : 0u;
      const uint2 fin = make_uint2(fn, fn * md.qinv);
#pragma unroll
      for (int r = 0; r < 16; ++r) rb[r] = mul_const(rb[r], fin.x, fin.y, q);
      // sigma(c0): its source block, staged through LDS like the digits
      uint32_t cv[16];
      load_C(cv, ct + (uint64_t)limb * n + sblk * kRow, lane);
      if constexpr (TENSOR) {  // c0 = x0 y0
        const uint2 r2 = T.r2[tabs];
        const uint32_t* py = cy + (uint64_t)limb * n + sblk * kRow;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const uint4 v = *reinterpret_cast<const uint4*>(py + 4 * lane + 256 * g);
          cv[4 * g] = prod_mod(cv[4 * g], v.x, md, r2);
          cv[4 * g + 1] = prod_mod(cv[4 * g + 1], v.y, md, r2);
          cv[4 * g + 2] = prod_mod(cv[4 * g + 2], v.z, md, r2);
          cv[4 * g + 3] = prod_mod(cv[4 * g + 3], v.w, md, r2);
        }
      }
      lds_put_C(priv, cv, lane);
      wave_sync();
#pragma unroll
      for (int r = 0; r < 16; ++r) rb[r] = add_mod(rb[r], priv[sidx[r]], q);
      wave_sync();
      store_C(out + ((uint64_t)0 * level + limb) * n + blk * kRow, rb, lane);
#pragma unroll
      for (int r = 0; r < 16; ++r) ra[r] = mul_const(ra[r], fin.x, fin.y, q);
      if constexpr (TENSOR) {  // the a-half gains d1 = x0 y1 + x1 y0 (Galois element 1: block blk)
        const uint2 r2 = T.r2[tabs];
        const uint64_t o0 = (uint64_t)limb * n + blk * kRow, o1 = ((uint64_t)level + limb) * n + blk * kRow;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const uint32_t w = 4 * lane + 256 * g;
          const uint4 x0 = *reinterpret_cast<const uint4*>(ct + o0 + w), x1 = *reinterpret_cast<const uint4*>(ct + o1 + w);
          const uint4 y0 = *reinterpret_cast<const uint4*>(cy + o0 + w), y1 = *reinterpret_cast<const uint4*>(cy + o1 + w);
          const uint32_t a0[4] = {x0.x, x0.y, x0.z, x0.w}, a1[4] = {x1.x, x1.y, x1.z, x1.w};
          const uint32_t b0[4] = {y0.x, y0.y, y0.z, y0.w}, b1[4] = {y1.x, y1.y, y1.z, y1.w};
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const uint32_t m = add_mod(mont_mul(a0[k], b1[k], md), mont_mul(a1[k], b0[k], md), q);
            ra[4 * g + k] = add_mod(ra[4 * g + k], mul_const(m, r2.x, r2.y, q), q);
          }
        }
      }
      store_C(out + ((uint64_t)1 * level + limb) * n + blk * kRow, ra, lane);
    }
  }
}

// A batch sharing one key, whose tiles are staged once in LDS per workgroup.
// Eight waves, at most 128 VGPRs: the tiles' LDS is shared by eight waves, so two
// workgroups (four waves per SIMD) fit a CU.
template <bool FINAL, bool TENSOR = false, bool BIG = false>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4, 8))) void k_ip8(DevTables T, IpArgs a) {
  ip_body<FINAL, 8, TENSOR, BIG>(T, a);
}
// Four waves (batches of 4..7): LDS allows three workgroups per CU.
template <bool FINAL, bool TENSOR = false, bool BIG = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 8))) void k_ip4(DevTables T, IpArgs a) {
  ip_body<FINAL, 4, TENSOR, BIG>(T, a);
}
// One wave per workgroup (hoisted keys, multi-item groups, small batches).  At
// least two waves per SIMD: the register budget that keeps the single-wave shapes
// fastest when every key is used once.
template <bool FINAL, bool TENSOR = false>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 8))) void k_ip1(DevTables T, IpArgs a) {
  ip_body<FINAL, 1, TENSOR>(T, a);
}

// Inner product in the extended basis: for key group kg and limb e (prime t),
// R = (P*sigma(c0) + sum_j sigma(d_j)*b_j, sum_j sigma(d_j)*a_j) on block blk, from
// digits that are already fully transformed, for each of a.items ciphertexts in turn
// (the baby steps of a linear transform: one hoisted ciphertext, several keys; the
// unfused key-switch: a batch, one key).  One wave per workgroup; a regenerated
// a-half lives in LDS, built once for all items.  Grid: x = limb, y = block, z = key.
__global__ __launch_bounds__(64) void k_rot_ext(DevTables T, ExtArgs a) {
  extern __shared__ uint32_t smem[];
  const uint32_t lane = threadIdx.x;
  const uint32_t u = xcd_logical_id();
  if (u >= gridDim.x * gridDim.y * gridDim.z) return;  // guard (the map is a bijection)
  const uint32_t blk = __builtin_amdgcn_readfirstlane(u % gridDim.y);
  const uint32_t kg = __builtin_amdgcn_readfirstlane((u / gridDim.y) % gridDim.z);
  const uint32_t e = __builtin_amdgcn_readfirstlane(u / (gridDim.y * gridDim.z));
  const uint32_t n = T.n, E = T.L + T.K, nd = a.nd, level = a.level, El = level + T.K;
  const uint32_t t = e < level ? e : T.L + (e - level);
  const uint32_t q = T.q[t];
  const Mod md{q, T.qinv[t]};
  const KeyRef& key = a.key[kg];
  uint32_t* Atile = smem;                                   // regenerated a rows [nd][1024]
  const uint32_t tiles = key.a ? 0u : nd * kRow;
  uint32_t* priv = smem + tiles;                            // gather block
  uint32_t* cnt = priv + kRowPad;                           // expander scratch
  if (!key.a) {
    uint32_t seed[8];
    for (int i = 0; i < 8; ++i) seed[i] = key.seed[i];
    regen_tiles(seed, 0, nd, t, blk, q, T.bound[t], T.one[t], a.regen_blocks, Atile, cnt);
  }
  __syncthreads();
  const uint32_t sblk = galois_src(blk * kRow, key.galois, T.log_n) >> 10;
  uint32_t sidx[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const uint32_t rout = 4 * lane + 256 * (r >> 2) + (r & 3);
    sidx[r] = swz(galois_src(blk * kRow + rout, key.galois, T.log_n) & (kRow - 1));
  }
  const uint32_t nq = (0u - q) + opaque_zero();  // 2^32 - q, opaque: see lazy_sub_mont
#pragma unroll 1
  for (uint32_t item = 0; item < a.items; ++item) {
    const uint32_t* ext = a.ext + item * a.ext_item;
    uint32_t rb[16], ra[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) { rb[r] = 0; ra[r] = 0; }
#pragma unroll 1
    for (uint32_t j = 0; j < nd; ++j) {
      uint32_t x[16];
      load_C(x, ext + ((uint64_t)j * E + e) * n + sblk * kRow, lane);
      lds_put_C(priv, x, lane);
      wave_sync();
      const uint32_t* kb = key.b + ((uint64_t)j * E + t) * n + blk * kRow;
      const uint32_t* ka = key.a ? key.a + ((uint64_t)j * E + t) * n + blk * kRow : Atile + j * kRow;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint32_t rout = 4 * lane + 256 * g;
        const uint4 b4 = *reinterpret_cast<const uint4*>(kb + rout);
        const uint4 a4 = *reinterpret_cast<const uint4*>(ka + rout);
        const uint32_t bv[4] = {b4.x, b4.y, b4.z, b4.w}, av[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int r = 4 * g + v;
          const uint32_t d = priv[sidx[r]];
          rb[r] = lazy_add_mont(rb[r], d, bv[v], md, nq);  // lazy: only multiplied afterwards
          ra[r] = lazy_add_mont(ra[r], d, av[v], md, nq);
        }
      }
      wave_sync();
    }
    const uint2 r2 = T.r2[t];  // the Montgomery products carry 2^-32
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      rb[r] = mul_const(rb[r], r2.x, r2.y, q);
      ra[r] = mul_const(ra[r], r2.x, r2.y, q);
    }
    if (e < level) {  // + P*sigma(c0) on the ciphertext primes
      uint32_t c[16];
      load_C(c, a.c0 + item * a.c0_item + (uint64_t)e * n + sblk * kRow, lane);
      lds_put_C(priv, c, lane);
      wave_sync();
      const uint2 pm = T.p_mod[e];
#pragma unroll
      for (int r = 0; r < 16; ++r) rb[r] = add_mod(rb[r], mul_const(priv[sidx[r]], pm.x, pm.y, q), q);
      wave_sync();
    }
    uint32_t* out = a.out + item * a.out_item + (uint64_t)kg * 2 * El * n + (uint64_t)e * n + blk * kRow;
    store_C(out, rb, lane);
    store_C(out + (uint64_t)El * n, ra, lane);
  }
}

// S_j = sum_k D[j][k] * R_k for every giant step j, on 4 coefficients per thread of
// limb e; R_0 = P*ct on the ciphertext primes and 0 on the special ones.  The sums
// of Montgomery products are multiplied by 2^32 once, at the end.
// Grid: x = 1024-coefficient chunk, y = limb.
__global__ __launch_bounds__(256) void k_diag_acc(DevTables T, DiagArgs a) {
  const uint32_t n = T.n, e = blockIdx.y, level = a.level, El = level + T.K;
  const uint32_t t = e < level ? e : T.L + (e - level);
  const uint32_t q = T.q[t];
  const Mod md{q, T.qinv[t]};
  const uint64_t col = 4 * (blockIdx.x * blockDim.x + threadIdx.x);
  const uint64_t le = (uint64_t)El * n;
  uint32_t acc[kMaxGiant][2][4];
#pragma unroll
  for (uint32_t j = 0; j < kMaxGiant; ++j)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[j][c][v] = 0;
  for (uint32_t k = 0; k < a.n1; ++k) {
    uint32_t rv[2][4];
    if (k == 0) {
      if (e < level) {
        const uint2 pm = T.p_mod[e];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const uint4 x = *reinterpret_cast<const uint4*>(a.ct + ((uint64_t)c * level + e) * n + col);
          const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
          for (int v = 0; v < 4; ++v) rv[c][v] = mul_const(xs[v], pm.x, pm.y, q);
        }
      } else {
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int v = 0; v < 4; ++v) rv[c][v] = 0;
      }
    } else {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const uint4 x = *reinterpret_cast<const uint4*>(a.r + (uint64_t)(k - 1) * 2 * le + c * le + (uint64_t)e * n + col);
        rv[c][0] = x.x; rv[c][1] = x.y; rv[c][2] = x.z; rv[c][3] = x.w;
      }
    }
#pragma unroll
    for (uint32_t j = 0; j < kMaxGiant; ++j) {
      if (j >= a.n2) break;
      const uint4 d4 = *reinterpret_cast<const uint4*>(a.diags + ((uint64_t)j * a.n1 + k) * le + (uint64_t)e * n + col);
      const uint32_t dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[j][c][v] = add_mod(acc[j][c][v], mont_mul(dv[v], rv[c][v], md), q);
    }
  }
  const uint2 r2 = T.r2[t];  // the Montgomery products carry 2^-32
#pragma unroll
  for (uint32_t j = 0; j < kMaxGiant; ++j) {
    if (j >= a.n2) break;
#pragma unroll
    for (int c = 0; c < 2; ++c)
      *reinterpret_cast<uint4*>(a.s + ((uint64_t)j * 2 + c) * le + (uint64_t)e * n + col) =
          make_uint4(mul_const(acc[j][c][0], r2.x, r2.y, q), mul_const(acc[j][c][1], r2.x, r2.y, q),
                     mul_const(acc[j][c][2], r2.x, r2.y, q), mul_const(acc[j][c][3], r2.x, r2.y, q));
  }
}

// out = sum of the n_src sources, element by element (limb of element w: (w / N) % level).
__global__ __launch_bounds__(256) void k_sum(DevTables T, SumArgs a, uint32_t* __restrict__ out, uint32_t level) {
  const uint64_t w = 4 * ((uint64_t)blockIdx.x * blockDim.x + threadIdx.x);
  if (w >= a.words) return;
  const uint32_t q = T.q[(uint32_t)((w / T.n) % level)];
  uint4 acc = *reinterpret_cast<const uint4*>(a.src[0] + w);
  for (uint32_t i = 1; i < a.n_src; ++i) {
    const uint4 x = *reinterpret_cast<const uint4*>(a.src[i] + w);
    acc = make_uint4(add_mod(acc.x, x.x, q), add_mod(acc.y, x.y, q), add_mod(acc.z, x.z, q), add_mod(acc.w, x.w, q));
  }
  *reinterpret_cast<uint4*>(out + w) = acc;
}

// Standalone expansion of the a-half: grid x = tile, y = prime, z = digit.
__global__ __launch_bounds__(64) void k_expand(DevTables T, KeyRef key, uint32_t* key_a, uint32_t nb) {
  __shared__ uint32_t tile[kRow];
  __shared__ uint32_t cnt[2 + 16 + 64];  // regen_tiles scratch for one tile
  const uint32_t tau = blockIdx.x, t = blockIdx.y, j = blockIdx.z;
  uint32_t seed[8];
  for (int i = 0; i < 8; ++i) seed[i] = key.seed[i];
  regen_tiles(seed, j, 1, t, tau, T.q[t], T.bound[t], T.one[t], nb, tile, cnt);
  __syncthreads();
  uint32_t* dst = key_a + ((uint64_t)j * (T.L + T.K) + t) * T.n + tau * kRow;
  for (uint32_t i = threadIdx.x; i < kRow; i += blockDim.x) dst[i] = tile[i];
}


// ------------------------------------------------------------------ launchers

hipError_t launch_rot_ext(const DevTables& T, const ExtArgs& a, hipStream_t s) {
  dim3 grid(a.level + T.K, T.n / kRow, a.n_keys);
  bool regen = false;
  for (uint32_t k = 0; k < a.n_keys; ++k) regen |= a.key[k].a == nullptr;
  const size_t shm = ((regen ? (size_t)a.nd * kRow + 2 * a.nd + 16 + 64 : 0) + kRowPad) * sizeof(uint32_t);
  hipLaunchKernelGGL(k_rot_ext, grid, dim3(64), shm, s, T, a);
  return hipGetLastError();
}

hipError_t launch_diag_acc(const DevTables& T, const DiagArgs& a, hipStream_t s) {
  if (a.n2 < 1 || a.n2 > kMaxGiant) return hipErrorInvalidValue;
  dim3 grid(T.n / 1024, a.level + T.K, 1);
  hipLaunchKernelGGL(k_diag_acc, grid, dim3(256), 0, s, T, a);
  return hipGetLastError();
}

hipError_t launch_sum(const DevTables& T, const SumArgs& a, uint32_t* out, uint32_t level, hipStream_t s) {
  const uint64_t threads = a.words / 4;
  dim3 grid((uint32_t)((threads + 255) / 256));
  hipLaunchKernelGGL(k_sum, grid, dim3(256), 0, s, T, a, out, level);
  return hipGetLastError();
}

hipError_t launch_row(const DevTables& T, const RowArgs& a, bool fwd, uint32_t items, hipStream_t s) {
  const uint32_t nblk = T.n / kRow;
  dim3 grid((nblk + 3) / 4, a.n_limbs, items);
  if (a.src2 && (fwd || a.use_srcs || a.own_n)) return hipErrorInvalidValue;  // products: plain inverse only
  if (fwd && T.all_big) hipLaunchKernelGGL((k_row<true, false, true>), grid, dim3(256), 0, s, T, a);
  else if (fwd) hipLaunchKernelGGL(k_row<true>, grid, dim3(256), 0, s, T, a);
  else if (a.src2) hipLaunchKernelGGL((k_row<false, true>), grid, dim3(256), 0, s, T, a);
  else hipLaunchKernelGGL(k_row<false>, grid, dim3(256), 0, s, T, a);
  return hipGetLastError();
}

template <bool FWD, bool BCAST = false>
static hipError_t col_dispatch(const DevTables& T, const ColArgs& a, uint32_t scale, uint32_t items, hipStream_t s) {
  dim3 grid(kRow / 64, a.n_limbs, items);
  switch (T.log_n) {
    case 12: hipLaunchKernelGGL((k_col<FWD, 2, BCAST>), grid, dim3(64), 0, s, T, a, scale); break;
    case 13: hipLaunchKernelGGL((k_col<FWD, 3, BCAST>), grid, dim3(64), 0, s, T, a, scale); break;
    case 14: hipLaunchKernelGGL((k_col<FWD, 4, BCAST>), grid, dim3(64), 0, s, T, a, scale); break;
    case 15:
      if (FWD && T.all_big) hipLaunchKernelGGL((k_col<FWD, 5, BCAST, true>), grid, dim3(64), 0, s, T, a, scale);
      else hipLaunchKernelGGL((k_col<FWD, 5, BCAST>), grid, dim3(64), 0, s, T, a, scale);
      break;
    case 16:
      if (FWD && T.all_big) hipLaunchKernelGGL((k_col<FWD, 6, BCAST, true>), grid, dim3(64), 0, s, T, a, scale);
      else hipLaunchKernelGGL((k_col<FWD, 6, BCAST>), grid, dim3(64), 0, s, T, a, scale);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_col(const DevTables& T, const ColArgs& a, bool fwd, bool scale_ninv, uint32_t items,
                      hipStream_t s) {
  if (a.bsrc) return fwd ? col_dispatch<true, true>(T, a, scale_ninv ? 1u : 0u, items, s) : hipErrorInvalidValue;
  return fwd ? col_dispatch<true>(T, a, scale_ninv ? 1u : 0u, items, s)
             : col_dispatch<false>(T, a, scale_ninv ? 1u : 0u, items, s);
}

// Columns per workgroup (16).  A workgroup has 16 or 32 threads per column, 256 or 512
// threads.  256: 4 waves, and its 48 KB of LDS allows three per CU (12 waves).  512:
// 8 waves, and registers (at most 128 per lane) allow two per CU (16 waves).  A
// launch takes 512 when a workgroup has at least 512 (target, column) tasks, as the
// 36 targets x 16 columns of a key-switch at level 36 do.  Those tasks are then one
// round plus 64 tasks on 4 lanes each, and batch 8 is whole rounds of workgroups
// (1,536 for ModUp, 1,024 for ModDown).  With 256 threads that ModDown is 1 1/3 rounds
// and both conversions take 6-10% longer.  Fewer tasks keep 256 threads: 384 tasks on
// 512 threads would leave a quarter of the lanes idle.  (12 threads per column were
// slower, and 20 or 24 did not divide the tasks.)
constexpr int kConvCW = 16;

template <int LOGC, int MAXS>
static void conv_go(const DevTables& T, const ConvArgs& a, dim3 grid, bool wide, hipStream_t s) {
  const size_t shm = (size_t)(1 << LOGC) * kConvCW * MAXS * sizeof(uint32_t);
  if constexpr (LOGC >= 5) {  // the large rings get a lazy-butterfly instantiation for chains above 2^31
    if (T.all_big) {
      if (wide) hipLaunchKernelGGL((k_conv<LOGC, kConvCW, MAXS, true, 512>), grid, dim3(512), shm, s, T, a);
      else hipLaunchKernelGGL((k_conv<LOGC, kConvCW, MAXS, true, 256>), grid, dim3(256), shm, s, T, a);
      return;
    }
    if (wide) {
      hipLaunchKernelGGL((k_conv<LOGC, kConvCW, MAXS, false, 512>), grid, dim3(512), shm, s, T, a);
      return;
    }
  }
  hipLaunchKernelGGL((k_conv<LOGC, kConvCW, MAXS, false, 256>), grid, dim3(256), shm, s, T, a);
}

template <int LOGC>
static hipError_t conv_maxs(const DevTables& T, const ConvArgs& a, dim3 grid, bool wide, hipStream_t s) {
  if (a.ns_max <= 4) conv_go<LOGC, 4>(T, a, grid, wide, s);
  else if (a.ns_max <= 8) conv_go<LOGC, 8>(T, a, grid, wide, s);
  else if (a.ns_max <= 12) conv_go<LOGC, 12>(T, a, grid, wide, s);
  else if (a.ns_max <= 16) conv_go<LOGC, 16>(T, a, grid, wide, s);
  else return hipErrorInvalidValue;
  return hipSuccess;
}

hipError_t launch_conv(const DevTables& T, const ConvArgs& a0, uint32_t groups, uint32_t items, hipStream_t s) {
  // small launches (few items) split the targets so that every CU gets work
  ConvArgs a = a0;
  const uint32_t wgs = (kRow / kConvCW) * groups * items;
  a.tchunks = wgs >= 512 ? 1u : min(4u, (512 + wgs - 1) / wgs);
  dim3 grid(kRow / kConvCW, groups * a.tchunks, items);
  if (a.mx) {  // matrix-core path: ring 2^16, 9..12 sources, 16-column tiles
    if (T.log_n != 16 || a.ns_max < 9 || a.ns_max > 12 || kConvCW != 16 || !T.mx_w) return hipErrorInvalidValue;
    const size_t shm = (size_t)64 * 16 * 12 * sizeof(uint32_t);
    hipLaunchKernelGGL(k_conv_mx, grid, dim3(256), shm, s, T, a);
    return hipGetLastError();
  }
  // (target, column) tasks of one workgroup: the targets of digit 0 (or of the
  // special part) in one chunk, times the columns
  const uint32_t ns0 = min(a.ns_max, a.ns_limit);
  const uint32_t targets = a.skip ? a.level + T.K - ns0 : a.n_targets;
  const bool wide = (targets + a.tchunks - 1) / a.tchunks * kConvCW >= 512;
  hipError_t e;
  switch (T.log_n) {
    case 12: e = conv_maxs<2>(T, a, grid, wide, s); break;
    case 13: e = conv_maxs<3>(T, a, grid, wide, s); break;
    case 14: e = conv_maxs<4>(T, a, grid, wide, s); break;
    case 15: e = conv_maxs<5>(T, a, grid, wide, s); break;
    case 16: e = conv_maxs<6>(T, a, grid, wide, s); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

hipError_t launch_ip(const DevTables& T, const IpArgs& a, bool final_pass, uint32_t n_limbs, hipStream_t s) {
  dim3 grid(n_limbs, T.n / kRow, a.n_keys);
  const uint32_t waves = a.n_ct >= 8 ? 8 : a.n_ct >= 4 ? 4 : 1;
  const uint32_t nth = 64 * waves;
  bool regen = false;
  for (uint32_t k = 0; k < a.n_keys; ++k) regen |= a.key[k].a == nullptr;
  // staged key rows and two block twiddle tables (multi-wave), or a regenerated a-half
  // (the eight-wave kernels' twiddle tables hold companions too: 2 words an entry)
  const size_t tw_words = waves == 8 ? 4 * kRow : 2 * kRow;
  const size_t tiles = (waves > 1 ? 2 * (size_t)a.nd * kRow + tw_words : (regen ? (size_t)a.nd * kRow : 0));
  const size_t shm = (tiles + waves * kRowPad + (regen ? 2 * a.nd + 16 + 64 : 0)) * sizeof(uint32_t);
  const bool big = T.all_big;  // the multi-wave final passes canonicalise conv's transform without a branch on q
  if (final_pass) {
    if (a.ty) {  // relinearisation of the tensor product of ct and ty
      if (waves == 8 && big) hipLaunchKernelGGL((k_ip8<true, true, true>), grid, dim3(nth), shm, s, T, a);
      else if (waves == 8) hipLaunchKernelGGL((k_ip8<true, true>), grid, dim3(nth), shm, s, T, a);
      else if (waves == 4 && big) hipLaunchKernelGGL((k_ip4<true, true, true>), grid, dim3(nth), shm, s, T, a);
      else if (waves == 4) hipLaunchKernelGGL((k_ip4<true, true>), grid, dim3(nth), shm, s, T, a);
      else hipLaunchKernelGGL((k_ip1<true, true>), grid, dim3(nth), shm, s, T, a);
    } else if (waves == 8 && big) hipLaunchKernelGGL((k_ip8<true, false, true>), grid, dim3(nth), shm, s, T, a);
    else if (waves == 8) hipLaunchKernelGGL((k_ip8<true>), grid, dim3(nth), shm, s, T, a);
    else if (waves == 4 && big) hipLaunchKernelGGL((k_ip4<true, false, true>), grid, dim3(nth), shm, s, T, a);
    else if (waves == 4) hipLaunchKernelGGL((k_ip4<true>), grid, dim3(nth), shm, s, T, a);
    else hipLaunchKernelGGL((k_ip1<true>), grid, dim3(nth), shm, s, T, a);
  } else {
    if (waves == 8) hipLaunchKernelGGL((k_ip8<false>), grid, dim3(nth), shm, s, T, a);
    else if (waves == 4) hipLaunchKernelGGL((k_ip4<false>), grid, dim3(nth), shm, s, T, a);
    else hipLaunchKernelGGL((k_ip1<false>), grid, dim3(nth), shm, s, T, a);
  }
  return hipGetLastError();
}

hipError_t launch_expand(const DevTables& T, const uint32_t seed[8], uint32_t* key_a, uint32_t regen_blocks,
                         hipStream_t s) {
  KeyRef k{};
  for (int i = 0; i < 8; ++i) k.seed[i] = seed[i];
  dim3 grid(T.n / kRow, T.L + T.K, T.dnum);
  hipLaunchKernelGGL(k_expand, grid, dim3(64), 0, s, T, k, key_a, regen_blocks);
  return hipGetLastError();
}


}  // namespace ckks
