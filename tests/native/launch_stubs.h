// Stand-ins for what the library's host code calls in its device half: every
// launcher and the no-alloc key-switch's static-array set-up.  Host checks that
// compile api.cpp in (no GPU, no device code) link against these; each returns a
// HIP error, so a compute call that got past its argument checks would fail loudly.
#pragma once

namespace ckks {
hipError_t launch_row(const DevTables&, const RowArgs&, bool, uint32_t, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_col(const DevTables&, const ColArgs&, bool, bool, uint32_t, hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_conv(const DevTables&, const ConvArgs&, uint32_t, uint32_t, hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_ip(const DevTables&, const IpArgs&, bool, uint32_t, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_rot_ext(const DevTables&, const ExtArgs&, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_diag_acc(const DevTables&, const DiagArgs&, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_sum(const DevTables&, const SumArgs&, uint32_t*, uint32_t, hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_expand(const DevTables&, const uint32_t*, uint32_t*, uint32_t, hipStream_t) {
  return hipErrorInvalidValue;
}
// the no-alloc key-switch's static array lives in device code, not compiled here
hipError_t scratch_setup(int) { return hipErrorInvalidValue; }
uint32_t* scratch_ptr(int) { return nullptr; }
const char* scratch_error(int) { return "not built into the host check"; }
}  // namespace ckks
