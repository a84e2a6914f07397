// Instantiations of the general forward scan (N > 32) for bf16_t I/O.
#include "ss_fwd_scan.h"

namespace ss {

hipError_t launch_fwd_scan_bf16(const FwdArgs& a, int ns, int gl, hipStream_t s) {
  return launch_fwd_ty<bf16_t>(a, ns, gl, s);
}

}  // namespace ss
