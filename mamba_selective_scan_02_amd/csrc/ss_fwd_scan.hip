// Instantiations of the general forward scan (ss_fwd_scan.h, N > 64) for one
// I/O type per object.  The library build compiles this file three times, with
// SS_SCAN_IO = 0 (f32), 1 (f16) and 2 (bf16): each type instantiates the kernel
// for every (G, EXACT, HAS_Z, MODE), and the three objects compile in
// parallel.
#include "ss_fwd_scan.h"

#ifndef SS_SCAN_IO
#error "compile with -DSS_SCAN_IO=0 (f32), 1 (f16) or 2 (bf16)"
#endif

namespace ss {

// EXACT (N fills the bucket, or B / C were copied into padded rows) reads
// whole B / C rows; for 16-bit types that needs 4-byte aligned rows: 4-byte
// aligned B and C and even row strides.
template <typename T, int NS, int G>
static hipError_t launch_fwd_e(const FwdArgs& a, hipStream_t s) {
  const bool rows_ok = sizeof(T) == 4 || ((reinterpret_cast<uintptr_t>(a.B) % 4 == 0) &&
                                          (reinterpret_cast<uintptr_t>(a.C) % 4 == 0) &&
                                          a.ldb % 2 == 0 && a.ldc % 2 == 0);
  const bool padded = a.b_pad != nullptr && a.B == a.b_pad;
  const bool exact = (a.N == (int64_t)NS * G || padded) && rows_ok;
  if (a.z != nullptr)
    return exact ? launch_fwd_t<T, NS, G, true, true>(a, s) : launch_fwd_t<T, NS, G, false, true>(a, s);
  return exact ? launch_fwd_t<T, NS, G, true, false>(a, s) : launch_fwd_t<T, NS, G, false, false>(a, s);
}

// G = 8 (N <= 128) or 16 lanes per channel, 16 states per lane.
template <typename T>
static hipError_t launch_fwd_ty(const FwdArgs& a, int ns, int gl, hipStream_t s) {
  if (ns == 16 && gl == 8) return launch_fwd_e<T, 16, 8>(a, s);
  if (ns == 16 && gl == 16) return launch_fwd_e<T, 16, 16>(a, s);
  return hipErrorInvalidValue;
}

#if SS_SCAN_IO == 0
hipError_t launch_fwd_scan_f32(const FwdArgs& a, int ns, int gl, hipStream_t s) {
  return launch_fwd_ty<float>(a, ns, gl, s);
}
#elif SS_SCAN_IO == 1
hipError_t launch_fwd_scan_f16(const FwdArgs& a, int ns, int gl, hipStream_t s) {
  return launch_fwd_ty<f16_t>(a, ns, gl, s);
}
#elif SS_SCAN_IO == 2
hipError_t launch_fwd_scan_bf16(const FwdArgs& a, int ns, int gl, hipStream_t s) {
  return launch_fwd_ty<bf16_t>(a, ns, gl, s);
}
#else
#error "SS_SCAN_IO must be 0, 1 or 2"
#endif

}  // namespace ss
