// Throughput of the gfx950 vector integer instructions the key-switching
// kernels are built from: the measured ceilings behind the vector-ALU roofline.
//
// Each kernel runs one instruction kind in 8 independent dependency chains per
// lane (so latency is hidden within a wave), 16 rounds per loop iteration, on a
// grid that fills every SIMD with 8 waves.  The instructions are written as
// inline assembly so that exactly the named instruction is issued (no folding,
// no strength reduction); none of them touches memory.  Lane-ops per second =
// threads x iterations x 16 x 8 / kernel time (HIP events around one launch).
// Built as its own small shared object; measurement only.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "modarith.h"

namespace {

enum Op : int {
  kMulLo = 0,   // v_mul_lo_u32
  kMulHi = 1,   // v_mul_hi_u32
  kMad64 = 2,   // v_mad_u64_u32 (64-bit accumulate, carry to an SGPR pair)
  kAdd = 3,     // v_add_u32 (no carry)
  kAddCo = 4,   // v_add_co_u32 (carry to VCC)
  kSubCo = 5,   // v_sub_co_u32 (borrow to VCC)
  kXor = 6,     // v_xor_b32
  kCndmask = 7, // v_cndmask_b32 (lane select by VCC, which no instruction of the loop writes)
  kAdd3 = 8,    // v_add3_u32 (three operands)
  kSub = 9,     // v_sub_u32 (no borrow)
  kMin = 10,    // v_min_u32
  kCmp = 11,    // v_cmp_gt_u32 (to VCC)
  kMul24 = 12,  // v_mul_u32_u24
  kMad24 = 13,  // v_mad_u32_u24
  kAlign = 14,  // v_alignbit_b32 (a rotate)
  kAdd64 = 15,  // v_lshl_add_u64 (64-bit add)
  kBfly = 16,   // the path's lazy forward butterfly (modarith.h), counted in butterflies
  kOps = 17
};

template <int OP>
__device__ __forceinline__ void step(uint32_t& a, uint64_t& w, uint32_t b) {
  if constexpr (OP == kMulLo) {
    asm volatile("v_mul_lo_u32 %0, %0, %1" : "+v"(a) : "v"(b));
  } else if constexpr (OP == kMulHi) {
    asm volatile("v_mul_hi_u32 %0, %0, %1" : "+v"(a) : "v"(b));
  } else if constexpr (OP == kMad64) {
    uint64_t c;
    asm volatile("v_mad_u64_u32 %0, %1, %2, %3, %0" : "+v"(w), "=s"(c) : "v"(a), "v"(b));
  } else if constexpr (OP == kAdd) {
    asm volatile("v_add_u32 %0, %0, %1" : "+v"(a) : "v"(b));
  } else if constexpr (OP == kAddCo) {
    asm volatile("v_add_co_u32 %0, vcc, %0, %1" : "+v"(a) : "v"(b) : "vcc");
  } else if constexpr (OP == kSubCo) {
    asm volatile("v_sub_co_u32 %0, vcc, %0, %1" : "+v"(a) : "v"(b) : "vcc");
  } else if constexpr (OP == kXor) {
    asm volatile("v_xor_b32 %0, %0, %1" : "+v"(a) : "v"(b));
  } else if constexpr (OP == kCndmask) {
    asm volatile("v_cndmask_b32 %0, %0, %1, vcc" : "+v"(a) : "v"(b));
  } else if constexpr (OP == kAdd3) {
    asm volatile("v_add3_u32 %0, %0, %1, %0" : "+v"(a) : "v"(b));
  } else if constexpr (OP == kSub) {
    asm volatile("v_sub_u32 %0, %0, %1" : "+v"(a) : "v"(b));
  } else if constexpr (OP == kMin) {
    asm volatile("v_min_u32 %0, %0, %1" : "+v"(a) : "v"(b));
  } else if constexpr (OP == kCmp) {
    asm volatile("v_cmp_gt_u32 vcc, %0, %1" : : "v"(a), "v"(b) : "vcc");
    asm volatile("v_xor_b32 %0, %0, %1" : "+v"(a) : "v"(b));  // keeps the chain live (counted separately)
  } else if constexpr (OP == kMul24) {
    asm volatile("v_mul_u32_u24 %0, %0, %1" : "+v"(a) : "v"(b));
  } else if constexpr (OP == kMad24) {
    asm volatile("v_mad_u32_u24 %0, %0, %1, %0" : "+v"(a) : "v"(b));
  } else if constexpr (OP == kAlign) {
    asm volatile("v_alignbit_b32 %0, %0, %0, 7" : "+v"(a));
  } else {
    asm volatile("v_lshl_add_u64 %0, %0, 0, %0" : "+v"(w));
  }
}

template <int OP>
__global__ __launch_bounds__(256) void k_rate(uint32_t* __restrict__ out, uint32_t iters, uint32_t seed) {
  const uint32_t tid = blockIdx.x * blockDim.x + threadIdx.x;
  const uint32_t b = (seed ^ (tid * 2654435761u)) | 1u;
  uint32_t a[8];
  uint64_t w[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = tid * (2 * i + 3) + seed;
    w[i] = a[i];
  }
  if constexpr (OP == kCndmask) asm volatile("v_cmp_gt_u32 vcc, %0, %1" : : "v"(a[0]), "v"(b) : "vcc");
  if constexpr (OP == kBfly) {
    // 4 independent butterfly pairs per lane (a[2i], a[2i+1]), lazy values, a 32-bit prime > 2^31
    const uint32_t q = 4293918721u;
    uint32_t qinv = q;  // q^-1 mod 2^32 by Newton's iteration
    for (int i = 0; i < 5; ++i) qinv *= 2u - q * qinv;
    const uint32_t wm = (b % q), wq = wm * qinv;
    for (uint32_t it = 0; it < iters; ++it) {
#pragma unroll
      for (int r = 0; r < 32; ++r) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t t = ckks::mul_const(a[2 * i + 1], wm, wq, q);
          a[2 * i + 1] = ckks::lazy_sub(a[2 * i], t, q);
          a[2 * i] = ckks::lazy_add(a[2 * i], t, q);
        }
      }
    }
    uint32_t x = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) x ^= a[i];
    out[tid] = x;
    return;
  }
  for (uint32_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
#pragma unroll
      for (int i = 0; i < 8; ++i) step<OP>(a[i], w[i], b);
    }
  }
  uint32_t x = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) x ^= a[i] ^ (uint32_t)w[i] ^ (uint32_t)(w[i] >> 32);
  out[tid] = x;
}

template <int OP>
hipError_t launch(uint32_t blocks, uint32_t* out, uint32_t iters, hipStream_t s) {
  hipLaunchKernelGGL(k_rate<OP>, dim3(blocks), dim3(256), 0, s, out, iters, 12345u);
  return hipGetLastError();
}

hipError_t launch_op(int op, uint32_t blocks, uint32_t* out, uint32_t iters, hipStream_t s) {
  switch (op) {
    case kMulLo: return launch<kMulLo>(blocks, out, iters, s);
    case kMulHi: return launch<kMulHi>(blocks, out, iters, s);
    case kMad64: return launch<kMad64>(blocks, out, iters, s);
    case kAdd: return launch<kAdd>(blocks, out, iters, s);
    case kAddCo: return launch<kAddCo>(blocks, out, iters, s);
    case kSubCo: return launch<kSubCo>(blocks, out, iters, s);
    case kXor: return launch<kXor>(blocks, out, iters, s);
    case kCndmask: return launch<kCndmask>(blocks, out, iters, s);
    case kAdd3: return launch<kAdd3>(blocks, out, iters, s);
    case kSub: return launch<kSub>(blocks, out, iters, s);
    case kMin: return launch<kMin>(blocks, out, iters, s);
    case kCmp: return launch<kCmp>(blocks, out, iters, s);
    case kMul24: return launch<kMul24>(blocks, out, iters, s);
    case kMad24: return launch<kMad24>(blocks, out, iters, s);
    case kAlign: return launch<kAlign>(blocks, out, iters, s);
    case kAdd64: return launch<kAdd64>(blocks, out, iters, s);
    case kBfly: return launch<kBfly>(blocks, out, iters, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

extern "C" {

// Number of instruction kinds and the name of kind `op` ("" if out of range).
int ckks_valu_rate_ops(void) { return kOps; }
const char* ckks_valu_rate_name(int op) {
  static const char* names[kOps] = {"v_mul_lo_u32",  "v_mul_hi_u32",  "v_mad_u64_u32",  "v_add_u32",
                                    "v_add_co_u32",  "v_sub_co_u32",  "v_xor_b32",      "v_cndmask_b32",
                                    "v_add3_u32",    "v_sub_u32",     "v_min_u32",      "v_cmp_gt_u32+v_xor_b32",
                                    "v_mul_u32_u24", "v_mad_u32_u24", "v_alignbit_b32", "v_lshl_add_u64",
                                    "lazy_butterfly"};
  return op >= 0 && op < kOps ? names[op] : "";
}

// Lane-ops per second (x 1e12) of instruction kind `op` on the current device
// (for the butterfly kind: butterflies per second; for the compare kind: pairs),
// best of `reps` launches of `blocks` workgroups of 256 threads with `iters`
// loop iterations (128 instructions per thread each).  Returns 0 on success.
int ckks_valu_rate(int op, uint32_t blocks, uint32_t iters, int reps, double* tera_per_s) {
  if (!tera_per_s || op < 0 || op >= kOps || blocks == 0 || iters == 0 || reps < 1) return -1;
  uint32_t* out = nullptr;
  if (hipMalloc(&out, (size_t)blocks * 256 * sizeof(uint32_t)) != hipSuccess) return -3;
  hipEvent_t e0, e1;
  (void)hipEventCreate(&e0);
  (void)hipEventCreate(&e1);
  int rc = 0;
  float best = 0.f;
  if (launch_op(op, blocks, out, iters, nullptr) != hipSuccess) rc = -4;  // warm-up
  for (int r = 0; r < reps && rc == 0; ++r) {
    (void)hipEventRecord(e0, nullptr);
    if (launch_op(op, blocks, out, iters, nullptr) != hipSuccess) rc = -4;
    (void)hipEventRecord(e1, nullptr);
    if (hipEventSynchronize(e1) != hipSuccess) rc = -4;
    float ms = 0.f;
    (void)hipEventElapsedTime(&ms, e0, e1);
    if (rc == 0 && (best == 0.f || ms < best)) best = ms;
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  (void)hipFree(out);
  if (rc) return rc;
  // every kind runs 128 instructions (or, for the butterfly, 128 butterflies) per thread and iteration
  const double ops = (double)blocks * 256 * iters * 16 * 8;
  *tera_per_s = ops / (best * 1e-3) / 1e12;
  return 0;
}

}  // extern "C"
