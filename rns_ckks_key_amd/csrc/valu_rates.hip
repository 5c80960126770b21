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

namespace {

enum Op : int {
  kMulLo = 0,   // v_mul_lo_u32
  kMulHi = 1,   // v_mul_hi_u32
  kMad64 = 2,   // v_mad_u64_u32 (64-bit accumulate, carry to an SGPR pair)
  kAdd = 3,     // v_add_u32 (no carry)
  kAddCo = 4,   // v_add_co_u32 (carry to VCC)
  kSubCo = 5,   // v_sub_co_u32 (borrow to VCC)
  kXor = 6,     // v_xor_b32
  kCndmask = 7, // v_cndmask_b32 (lane select by VCC)
  kAdd3 = 8,    // v_add3_u32 (three operands)
  kOps = 9
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
    asm volatile("v_cndmask_b32 %0, %0, %1, vcc" : "+v"(a) : "v"(b) : "vcc");
  } else {
    asm volatile("v_add3_u32 %0, %0, %1, %0" : "+v"(a) : "v"(b));
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
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

extern "C" {

// Number of instruction kinds and the name of kind `op` ("" if out of range).
int ckks_valu_rate_ops(void) { return kOps; }
const char* ckks_valu_rate_name(int op) {
  static const char* names[kOps] = {"v_mul_lo_u32", "v_mul_hi_u32", "v_mad_u64_u32", "v_add_u32", "v_add_co_u32",
                                    "v_sub_co_u32", "v_xor_b32",    "v_cndmask_b32", "v_add3_u32"};
  return op >= 0 && op < kOps ? names[op] : "";
}

// Lane-ops per second (x 1e12) of instruction kind `op` on the current device,
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
  const double ops = (double)blocks * 256 * iters * 16 * 8;
  *tera_per_s = ops / (best * 1e-3) / 1e12;
  return 0;
}

}  // extern "C"
