// Instantiations of the general forward scan (N > 32) for float I/O.
#include "ss_fwd_scan.h"

namespace ss {

hipError_t launch_fwd_scan_f32(const FwdArgs& a, int ns, int gl, hipStream_t s) {
  return launch_fwd_ty<float>(a, ns, gl, s);
}

}  // namespace ss
