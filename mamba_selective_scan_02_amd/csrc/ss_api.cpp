// C entry points of libss: validation, schedule planning and launches.
//
// Validation follows the baracuda-kernels page "src/attention/selective_scan.rs"
// (SelectiveScanPlan::select / can_implement and the backward plan's run):
// negative extents are an invalid problem, dstate above 256 and dtypes outside
// {f32, f16, bf16} are unsupported, a workspace smaller than the query is
// WorkspaceTooSmall, the optional-input / gradient pairs of the backward must
// be both given or both omitted, and empty problems (B * L * D = 0) return
// success without launching.  Raw pointers carry no shapes, so shape checks
// become descriptor checks; null and misaligned pointers are rejected here.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/ss.h"
#include "ss_device.h"
#include "ss_plan.h"
#include "ss_plan_complex.h"

namespace ss {
hipError_t launch_fwd(const FwdArgs& a, int io_dtype, int ns, int gl, hipStream_t s);
hipError_t launch_zero_param(void* p, int64_t n, int dtype, hipStream_t s);
hipError_t launch_copy_param(void* dst, const void* src, int64_t n, int dtype, hipStream_t s);
hipError_t launch_bwd(const BwdArgs& a, const Plan& p, int io_dtype, hipStream_t s);
hipError_t launch_fwd_complex(const FwdArgs& a, int io_dtype, int ns, int gl, hipStream_t s);
hipError_t launch_bwd_complex(const BwdArgs& a, const Plan& p, int io_dtype, hipStream_t s);
}  // namespace ss

namespace {

thread_local char g_err[512];

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int64_t dtype_size(int32_t dt) { return dt == SS_F32 ? 4 : 2; }

bool aligned(const void* p, int64_t a) { return (reinterpret_cast<uintptr_t>(p) % (uintptr_t)a) == 0; }

// Descriptor checks shared by forward and backward.
int check_desc(const ss_desc* d, const char* who) {
  if (!d) return fail(SS_ERR_INVALID_PROBLEM, "%s: descriptor is NULL", who);
  if (d->batch < 0 || d->seqlen < 0 || d->dim < 0 || d->dstate < 0)
    return fail(SS_ERR_INVALID_PROBLEM, "%s: extents must be non-negative", who);
  if (d->dstate > 256)
    return fail(SS_ERR_UNSUPPORTED, "%s: dstate must be <= 256 (got %d)", who, d->dstate);
  if (d->io_dtype != SS_F32 && d->io_dtype != SS_F16 && d->io_dtype != SS_BF16)
    return fail(SS_ERR_UNSUPPORTED, "%s: io_dtype must be f32, f16 or bf16", who);
  if (d->param_dtype != SS_F32 && d->param_dtype != d->io_dtype)
    return fail(SS_ERR_UNSUPPORTED, "%s: param_dtype must be f32 or equal to io_dtype", who);
  if (d->delta_softplus != 0 && d->delta_softplus != 1)
    return fail(SS_ERR_INVALID_PROBLEM, "%s: delta_softplus must be 0 or 1", who);
  if (d->chunk_len < 0)
    return fail(SS_ERR_INVALID_PROBLEM, "%s: chunk_len must be >= 0", who);
  return SS_OK;
}

struct PtrCheck {
  const char* who;
  int status = SS_OK;
  void need(const void* p, const char* name, int64_t elem) {
    if (status != SS_OK) return;
    if (!p) status = fail(SS_ERR_INVALID_PROBLEM, "%s: %s is NULL", who, name);
    else if (!aligned(p, elem))
      status = fail(SS_ERR_INVALID_PROBLEM, "%s: %s is not aligned to its element size", who, name);
  }
  void opt(const void* p, const char* name, int64_t elem) {
    if (status != SS_OK || !p) return;
    if (!aligned(p, elem))
      status = fail(SS_ERR_INVALID_PROBLEM, "%s: %s is not aligned to its element size", who, name);
  }
};

int check_workspace(size_t need, void* ws, size_t ws_bytes, const char* who) {
  if (ws_bytes < need)
    return fail(SS_ERR_WORKSPACE_TOO_SMALL, "%s: workspace too small (need %zu bytes, got %zu)",
                who, need, ws_bytes);
  if (need > 0 && !ws) return fail(SS_ERR_INVALID_PROBLEM, "%s: workspace is NULL", who);
  if (need > 0 && !aligned(ws, 256))
    return fail(SS_ERR_INVALID_PROBLEM, "%s: workspace must be 256-byte aligned", who);
  return SS_OK;
}

// [p, p + bytes) and [q, q + bytes) share at least one byte
bool overlap(const void* p, const void* q, int64_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
  return bytes > 0 && a < b + (uintptr_t)bytes && b < a + (uintptr_t)bytes;
}

// Row strides of B / C (0 = N, the packed layout): at least N, and within
// the 32-bit byte offsets that the tile kernels take inside one chunk
// (rows_per_chunk rows, 0 for kernels with 64-bit addressing).
int check_ld(int64_t* ldb, int64_t* ldc, int64_t N, int64_t es, int64_t rows_per_chunk,
             const char* who) {
  if (*ldb == 0) *ldb = N;
  if (*ldc == 0) *ldc = N;
  if (*ldb < N || *ldc < N)
    return fail(SS_ERR_INVALID_PROBLEM, "%s: B / C row strides must be 0 or >= dstate", who);
  const int64_t ld = *ldb > *ldc ? *ldb : *ldc;
  if (rows_per_chunk > 0 && (rows_per_chunk + ss::GL_MAX_TILE) * ld * es > 0x7fffffffLL)
    return fail(SS_ERR_UNSUPPORTED, "%s: B / C row stride %lld is too large for chunks of "
                "%lld steps (set a shorter desc->chunk_len)", who, (long long)ld,
                (long long)rows_per_chunk);
  return SS_OK;
}

int hip_status(hipError_t e, const char* who) {
  if (e == hipSuccess) return SS_OK;
  return fail(SS_ERR_HIP, "%s: launch failed: %s", who, hipGetErrorString(e));
}

}  // namespace

extern "C" {

size_t ss_workspace_size(const ss_desc* d, int32_t backward) {
  if (check_desc(d, "ss_workspace_size") != SS_OK) return 0;
  return ss::make_plan(*d, backward != 0).ws_bytes;
}

int ss_plan_query(const ss_desc* d, int32_t backward, ss_plan* out) {
  g_err[0] = 0;
  int st = check_desc(d, "ss_plan_query");
  if (st != SS_OK) return st;
  if (!out) return fail(SS_ERR_INVALID_PROBLEM, "ss_plan_query: out is NULL");
  const ss::Plan p = ss::make_plan(*d, backward != 0);
  out->chunk_len = (int32_t)p.chunk_len;
  out->n_chunks = (int32_t)p.K;
  out->states_per_lane = p.NS;
  out->lanes_per_channel = p.G;
  out->n_launches = p.n_launches;
  return SS_OK;
}

int ss_fwd(const ss_desc* d, const void* u, const void* delta, const void* A, const void* B,
           const void* C, const void* Dskip, const void* z, const void* delta_bias, void* y,
           void* last_state, void* workspace, size_t workspace_bytes, void* stream) {
  return ss_fwd_h0(d, u, delta, A, B, C, Dskip, z, delta_bias, nullptr, y, last_state,
                   workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

// Forward of a dense problem (cu = NULL: B sequences of L steps) or of a packed
// variable-length one (cu = cu_seqlens on the device, B sequences of at most
// L steps in `total` rows).
int fwd_impl(const char* who, const ss_desc* d, const int32_t* cu, int64_t total,
             int64_t ldb, int64_t ldc, const void* u, const void* delta, const void* A, const void* B, const void* C,
             const void* Dskip, const void* z, const void* delta_bias, const void* h0, void* y,
             void* last_state, void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  int st = check_desc(d, who);
  if (st != SS_OK) return st;
  const int64_t Bn = d->batch, L = d->seqlen, D = d->dim, N = d->dstate;
  if (cu && total < 0) return fail(SS_ERR_INVALID_PROBLEM, "%s: total_len must be >= 0", who);
  if (cu && !aligned(cu, 4))
    return fail(SS_ERR_INVALID_PROBLEM, "%s: cu_seqlens is not 4-byte aligned", who);
  if (cu && total > (int64_t)d->batch * d->seqlen)
    return fail(SS_ERR_INVALID_PROBLEM, "%s: total_len exceeds batch * seqlen", who);
  const int64_t rows = cu ? total : Bn * L;          // rows of the [rows, D] tensors
  const int64_t io = dtype_size(d->io_dtype), pa = dtype_size(d->param_dtype);
  hipStream_t s = static_cast<hipStream_t>(stream);
  PtrCheck pc{who};
  pc.opt(last_state, "last_state", pa);
  if (Bn * D * N > 0) pc.opt(h0, "h0", pa);
  if (pc.status != SS_OK) return pc.status;
  const int64_t state_bytes = Bn * D * N * pa;
  const bool in_place = h0 && last_state == h0 && state_bytes > 0;
  if (h0 && last_state && !in_place && overlap(h0, last_state, state_bytes))
    return fail(SS_ERR_INVALID_PROBLEM, "%s: h0 and last_state must be the same buffer or "
                "not overlap", who);
  if (rows * D == 0 || Bn == 0) {
    // Nothing to scan.  An empty sequence leaves the initial state (h0 or 0).
    if (rows == 0 && last_state && state_bytes > 0)
      return hip_status(h0 ? ss::launch_copy_param(last_state, h0, Bn * D * N, d->param_dtype, s)
                           : ss::launch_zero_param(last_state, Bn * D * N, d->param_dtype, s),
                        who);
    return SS_OK;
  }
  pc.need(u, "u", io);
  pc.need(delta, "delta", io);
  pc.need(y, "y", io);
  if (N > 0) {
    pc.need(A, "A", pa);
    pc.need(B, "B", io);
    pc.need(C, "C", io);
  }
  pc.opt(Dskip, "D", pa);
  pc.opt(z, "z", io);
  pc.opt(delta_bias, "delta_bias", pa);
  if (pc.status != SS_OK) return pc.status;
  // In place (last_state == h0): one chunk, so that the only reader of h0 is
  // the lane that later writes the same elements of last_state.
  ss_desc dd = *d;
  if (in_place) dd.chunk_len = d->seqlen;
  const ss::Plan p = ss::make_plan(dd, false);
  if (in_place && p.K > 1)
    return fail(SS_ERR_UNSUPPORTED, "%s: an in-place state update (last_state == h0) needs a "
                "single chunk, and this shape's rows exceed one chunk's 32-bit range", who);
  st = check_ld(&ldb, &ldc, N, io, p.G == 8 && p.NS <= 8 ? p.chunk_len : 0, who);
  if (st != SS_OK) return st;
  st = check_workspace(p.ws_bytes, workspace, workspace_bytes, who);
  if (st != SS_OK) return st;

  ss::FwdArgs a{};
  a.u = u; a.delta = delta; a.A = A; a.B = B; a.C = C;
  a.Dskip = Dskip; a.z = z; a.bias = delta_bias; a.y = y; a.last_state = last_state;
  a.h0 = N > 0 ? h0 : nullptr;
  char* ws = static_cast<char*>(workspace);
  a.chunk_dsum = p.K > 1 ? reinterpret_cast<float*>(ws + p.off_dsum) : nullptr;
  a.chunk_state = p.K > 1 ? reinterpret_cast<float*>(ws + p.off_state) : nullptr;
  a.b_pad = p.pad_rows ? ws + p.off_bpad : nullptr;
  a.c_pad = p.pad_rows ? ws + p.off_cpad : nullptr;
  a.Bn = Bn; a.L = L; a.D = D; a.N = N;
  a.chunk_len = p.chunk_len; a.K = p.K;
  a.cu = cu; a.Lt = rows;
  a.ldb = ldb; a.ldc = ldc;
  a.softplus = d->delta_softplus;
  a.param_dtype = d->param_dtype;
  return hip_status(ss::launch_fwd(a, d->io_dtype, p.NS, p.G, s), who);
}

}  // namespace

extern "C" {

int ss_fwd_h0(const ss_desc* d, const void* u, const void* delta, const void* A, const void* B,
              const void* C, const void* Dskip, const void* z, const void* delta_bias,
              const void* h0, void* y, void* last_state, void* workspace,
              size_t workspace_bytes, void* stream) {
  return fwd_impl(h0 ? "ss_fwd_h0" : "ss_fwd", d, nullptr, 0, 0, 0, u, delta, A, B, C, Dskip, z,
                  delta_bias, h0, y, last_state, workspace, workspace_bytes, stream);
}

int ss_fwd_varlen(const ss_desc* d, const int32_t* cu_seqlens, int64_t total_len,
                  const void* u, const void* delta, const void* A, const void* B, const void* C,
                  const void* Dskip, const void* z, const void* delta_bias, const void* h0,
                  void* y, void* last_state, void* workspace, size_t workspace_bytes,
                  void* stream) {
  if (!cu_seqlens) {
    g_err[0] = 0;
    return fail(SS_ERR_INVALID_PROBLEM, "ss_fwd_varlen: cu_seqlens is NULL");
  }
  return fwd_impl("ss_fwd_varlen", d, cu_seqlens, total_len, 0, 0, u, delta, A, B, C, Dskip, z,
                  delta_bias, h0, y, last_state, workspace, workspace_bytes, stream);
}

int ss_bwd(const ss_desc* d, const void* u, const void* delta, const void* A, const void* B,
           const void* C, const void* Dskip, const void* z, const void* delta_bias,
           const void* dy, void* du, void* ddelta, void* dA, void* dB, void* dC, void* dD,
           void* dz, void* ddelta_bias, void* workspace, size_t workspace_bytes, void* stream) {
  return ss_bwd_h0(d, u, delta, A, B, C, Dskip, z, delta_bias, nullptr, dy, du, ddelta, dA, dB,
                   dC, dD, dz, ddelta_bias, nullptr, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

// Backward of a dense (cu = NULL) or packed variable-length problem.
int bwd_impl(const char* who, const ss_desc* d, const int32_t* cu, int64_t total,
             int64_t ldb, int64_t ldc, const void* u, const void* delta, const void* A, const void* B, const void* C,
             const void* Dskip, const void* z, const void* delta_bias, const void* h0,
             const void* dy, void* du, void* ddelta, void* dA, void* dB, void* dC, void* dD,
             void* dz, void* ddelta_bias, void* dh0, void* workspace, size_t workspace_bytes,
             void* stream) {
  g_err[0] = 0;
  int st = check_desc(d, who);
  if (st != SS_OK) return st;
  if (cu && total < 0) return fail(SS_ERR_INVALID_PROBLEM, "%s: total_len must be >= 0", who);
  if (cu && !aligned(cu, 4))
    return fail(SS_ERR_INVALID_PROBLEM, "%s: cu_seqlens is not 4-byte aligned", who);
  // The dB / dC partials are sized for batch * seqlen rows; sequences of at
  // most seqlen steps cannot hold more.
  if (cu && total > (int64_t)d->batch * d->seqlen)
    return fail(SS_ERR_INVALID_PROBLEM, "%s: total_len exceeds batch * seqlen", who);
  if ((h0 == nullptr) != (dh0 == nullptr))
    return fail(SS_ERR_INVALID_PROBLEM, "%s: h0 and dh0 must be both given or both omitted", who);
  if ((Dskip == nullptr) != (dD == nullptr))
    return fail(SS_ERR_INVALID_PROBLEM, "%s: D and dD must be both given or both omitted", who);
  if ((z == nullptr) != (dz == nullptr))
    return fail(SS_ERR_INVALID_PROBLEM, "%s: z and dz must be both given or both omitted", who);
  if ((delta_bias == nullptr) != (ddelta_bias == nullptr))
    return fail(SS_ERR_INVALID_PROBLEM,
                "%s: delta_bias and ddelta_bias must be both given or both omitted", who);
  const int64_t Bn = d->batch, L = d->seqlen, D = d->dim, N = d->dstate;
  const int64_t rows = cu ? total : Bn * L;          // rows of the [rows, D] tensors
  const int64_t io = dtype_size(d->io_dtype), pa = dtype_size(d->param_dtype);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const ss::Plan p = ss::make_plan(*d, true);
  PtrCheck pc{who};
  if (rows * D > 0) {
    pc.need(u, "u", io); pc.need(delta, "delta", io); pc.need(dy, "dy", io);
    pc.need(du, "du", io); pc.need(ddelta, "ddelta", io);
    if (N > 0) {
      pc.need(A, "A", pa); pc.need(B, "B", io); pc.need(C, "C", io);
    }
    pc.opt(z, "z", io); pc.opt(dz, "dz", io);
  }
  if (D * N > 0) pc.need(dA, "dA", pa);
  if (rows * N > 0) { pc.need(dB, "dB", io); pc.need(dC, "dC", io); }
  pc.opt(Dskip, "D", pa); pc.opt(dD, "dD", pa);
  pc.opt(delta_bias, "delta_bias", pa); pc.opt(ddelta_bias, "ddelta_bias", pa);
  if (Bn * D * N > 0) { pc.opt(h0, "h0", pa); pc.opt(dh0, "dh0", pa); }
  if (pc.status != SS_OK) return pc.status;
  if (h0 && overlap(h0, dh0, Bn * D * N * pa))
    return fail(SS_ERR_INVALID_PROBLEM, "%s: dh0 must not overlap h0", who);
  st = check_ld(&ldb, &ldc, N, io, p.bwd_tile ? p.chunk_len : 0, who);
  if (st != SS_OK) return st;
  st = check_workspace(p.ws_bytes, workspace, workspace_bytes, who);
  if (st != SS_OK) return st;
  if (rows * D == 0 && D * N == 0 && rows * N == 0 && D == 0) return SS_OK;
  const bool has_state = h0 && Bn * D * N > 0;

  ss::BwdArgs a{};
  a.u = u; a.delta = delta; a.A = A; a.B = B; a.C = C;
  a.Dskip = Dskip; a.z = z; a.bias = delta_bias; a.dy = dy;
  a.du = du; a.ddelta = ddelta; a.dA = dA; a.dB = dB; a.dC = dC;
  a.dD = dD; a.dz = dz; a.dbias = ddelta_bias;
  a.h0 = has_state ? h0 : nullptr;
  a.dh0 = has_state ? dh0 : nullptr;
  a.ws = static_cast<char*>(workspace);
  a.Bn = Bn; a.L = L; a.D = D; a.N = N;
  a.chunk_len = p.chunk_len; a.K = p.K;
  a.cu = cu; a.Lt = rows;
  a.ldb = ldb; a.ldc = ldc;
  a.softplus = d->delta_softplus;
  a.param_dtype = d->param_dtype;
  a.io_dtype = d->io_dtype;
  return hip_status(ss::launch_bwd(a, p, d->io_dtype, s), who);
}

}  // namespace

extern "C" {

int ss_bwd_h0(const ss_desc* d, const void* u, const void* delta, const void* A, const void* B,
              const void* C, const void* Dskip, const void* z, const void* delta_bias,
              const void* h0, const void* dy, void* du, void* ddelta, void* dA, void* dB,
              void* dC, void* dD, void* dz, void* ddelta_bias, void* dh0, void* workspace,
              size_t workspace_bytes, void* stream) {
  return bwd_impl(h0 ? "ss_bwd_h0" : "ss_bwd", d, nullptr, 0, 0, 0, u, delta, A, B, C, Dskip, z,
                  delta_bias, h0, dy, du, ddelta, dA, dB, dC, dD, dz, ddelta_bias, dh0,
                  workspace, workspace_bytes, stream);
}

}  // extern "C"

// Scratch of ss_bwd_noalloc: the workspace of callers that cannot allocate.
// Each GPU the library runs on holds its own copy until the process ends; in
// host code `scratch` only names the symbol, and its device address is looked
// up once per device with hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[SS_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the device the work is enqueued on (the
// stream's device, or the current one for the NULL stream).
int scratch_address(hipStream_t s, void** out, const char* who) {
  int cur = 0, dev = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e == hipSuccess) {
    dev = cur;
    if (s) e = hipStreamGetDevice(s, &dev);
  }
  if (e != hipSuccess) return fail(SS_ERR_HIP, "%s: no device: %s", who, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(SS_ERR_UNSUPPORTED, "%s: device %d is beyond the %d the scratch table holds",
                who, dev, kMaxDevices);
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess)
        return fail(SS_ERR_HIP, "%s: cannot select device %d: %s", who, dev, hipGetErrorString(e));
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (dev != cur) (void)hipSetDevice(cur);
      if (e != hipSuccess || !p)
        return fail(SS_ERR_HIP, "%s: no address for the static scratch on device %d: %s", who,
                    dev, hipGetErrorString(e));
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return SS_OK;
}

}  // namespace

extern "C" {

int ss_bwd_noalloc(const ss_desc* d, const void* u, const void* delta, const void* A,
                   const void* B, const void* C, const void* Dskip, const void* z,
                   const void* delta_bias, const void* h0, const void* dy, void* du,
                   void* ddelta, void* dA, void* dB, void* dC, void* dD, void* dz,
                   void* ddelta_bias, void* dh0, void* stream) {
  const char* who = "ss_bwd_noalloc";
  g_err[0] = 0;
  int st = check_desc(d, who);
  if (st != SS_OK) return st;
  const size_t need = ss::make_plan(*d, true).ws_bytes;
  if (need > (size_t)SS_NOALLOC_SCRATCH_BYTES)
    return fail(SS_ERR_UNSUPPORTED, "%s: this problem needs %zu bytes of scratch, above the %zu "
                "of the static scratch (call ss_bwd_h0 with a workspace instead)", who, need,
                (size_t)SS_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (need > 0) {
    st = scratch_address(static_cast<hipStream_t>(stream), &ws, who);
    if (st != SS_OK) return st;
  }
  return bwd_impl(who, d, nullptr, 0, 0, 0, u, delta, A, B, C, Dskip, z, delta_bias, h0, dy, du,
                  ddelta, dA, dB, dC, dD, dz, ddelta_bias, dh0, ws,
                  need > 0 ? (size_t)SS_NOALLOC_SCRATCH_BYTES : 0, stream);
}

int ss_bwd_varlen(const ss_desc* d, const int32_t* cu_seqlens, int64_t total_len,
                  const void* u, const void* delta, const void* A, const void* B, const void* C,
                  const void* Dskip, const void* z, const void* delta_bias, const void* h0,
                  const void* dy, void* du, void* ddelta, void* dA, void* dB, void* dC,
                  void* dD, void* dz, void* ddelta_bias, void* dh0, void* workspace,
                  size_t workspace_bytes, void* stream) {
  if (!cu_seqlens) {
    g_err[0] = 0;
    return fail(SS_ERR_INVALID_PROBLEM, "ss_bwd_varlen: cu_seqlens is NULL");
  }
  return bwd_impl("ss_bwd_varlen", d, cu_seqlens, total_len, 0, 0, u, delta, A, B, C, Dskip, z,
                  delta_bias, h0, dy, du, ddelta, dA, dB, dC, dD, dz, ddelta_bias, dh0,
                  workspace, workspace_bytes, stream);
}

int ss_fwd_strided(const ss_desc* d, const int32_t* cu_seqlens, int64_t total_len,
                   int64_t ldb, int64_t ldc, const void* u, const void* delta, const void* A,
                   const void* B, const void* C, const void* Dskip, const void* z,
                   const void* delta_bias, const void* h0, void* y, void* last_state,
                   void* workspace, size_t workspace_bytes, void* stream) {
  return fwd_impl("ss_fwd_strided", d, cu_seqlens, total_len, ldb, ldc, u, delta, A, B, C,
                  Dskip, z, delta_bias, h0, y, last_state, workspace, workspace_bytes, stream);
}

int ss_bwd_strided(const ss_desc* d, const int32_t* cu_seqlens, int64_t total_len,
                   int64_t ldb, int64_t ldc, const void* u, const void* delta, const void* A,
                   const void* B, const void* C, const void* Dskip, const void* z,
                   const void* delta_bias, const void* h0, const void* dy, void* du,
                   void* ddelta, void* dA, void* dB, void* dC, void* dD, void* dz,
                   void* ddelta_bias, void* dh0, void* workspace, size_t workspace_bytes,
                   void* stream) {
  return bwd_impl("ss_bwd_strided", d, cu_seqlens, total_len, ldb, ldc, u, delta, A, B, C,
                  Dskip, z, delta_bias, h0, dy, du, ddelta, dA, dB, dC, dD, dz, ddelta_bias,
                  dh0, workspace, workspace_bytes, stream);
}

size_t ss_workspace_size_complex(const ss_desc* d, int32_t backward) {
  if (check_desc(d, "ss_workspace_size_complex") != SS_OK) return 0;
  return ss::make_plan_complex(*d, backward != 0).ws_bytes;
}

int ss_fwd_complex(const ss_desc* d, const void* u, const void* delta, const void* A,
                   const void* B, const void* C, const void* Dskip, const void* z,
                   const void* delta_bias, const void* h0, void* y, void* last_state,
                   void* workspace, size_t workspace_bytes, void* stream) {
  const char* who = "ss_fwd_complex";
  g_err[0] = 0;
  int st = check_desc(d, who);
  if (st != SS_OK) return st;
  const int64_t Bn = d->batch, L = d->seqlen, D = d->dim, N = d->dstate;
  const int64_t io = dtype_size(d->io_dtype), pa = dtype_size(d->param_dtype);
  hipStream_t s = static_cast<hipStream_t>(stream);
  PtrCheck pc{who};
  pc.opt(last_state, "last_state", pa);
  if (Bn * D * N > 0) pc.opt(h0, "h0", pa);
  if (pc.status != SS_OK) return pc.status;
  const int64_t state_elems = 2 * Bn * D * N;   // (re, im) pairs
  const int64_t state_bytes = state_elems * pa;
  const bool in_place = h0 && last_state == h0 && state_bytes > 0;
  if (h0 && last_state && !in_place && overlap(h0, last_state, state_bytes))
    return fail(SS_ERR_INVALID_PROBLEM, "%s: h0 and last_state must be the same buffer or "
                "not overlap", who);
  if (Bn * L * D == 0) {
    if (L == 0 && last_state && state_bytes > 0)
      return hip_status(h0 ? ss::launch_copy_param(last_state, h0, state_elems, d->param_dtype, s)
                           : ss::launch_zero_param(last_state, state_elems, d->param_dtype, s),
                        who);
    return SS_OK;
  }
  pc.need(u, "u", io);
  pc.need(delta, "delta", io);
  pc.need(y, "y", io);
  if (N > 0) {
    pc.need(A, "A", pa);
    pc.need(B, "B", io);
    pc.need(C, "C", io);
  }
  pc.opt(Dskip, "D", pa);
  pc.opt(z, "z", io);
  pc.opt(delta_bias, "delta_bias", pa);
  if (pc.status != SS_OK) return pc.status;
  // In place (last_state == h0): one chunk, so that the only reader of an h0
  // element is the lane that writes the same last_state element at its end.
  ss_desc dd = *d;
  if (in_place) dd.chunk_len = d->seqlen;
  const ss::Plan p = ss::make_plan_complex(dd, false);
  st = check_workspace(p.ws_bytes, workspace, workspace_bytes, who);
  if (st != SS_OK) return st;
  ss::FwdArgs a{};
  a.u = u; a.delta = delta; a.A = A; a.B = B; a.C = C;
  a.Dskip = Dskip; a.z = z; a.bias = delta_bias; a.y = y; a.last_state = last_state;
  a.h0 = N > 0 ? h0 : nullptr;
  char* ws = static_cast<char*>(workspace);
  a.chunk_state = p.K > 1 && N > 0 ? reinterpret_cast<float*>(ws + p.off_state) : nullptr;
  a.Bn = Bn; a.L = L; a.D = D; a.N = N;
  a.chunk_len = p.chunk_len; a.K = p.K;
  a.Lt = Bn * L; a.ldb = 2 * N; a.ldc = 2 * N;
  a.softplus = d->delta_softplus;
  a.param_dtype = d->param_dtype;
  return hip_status(ss::launch_fwd_complex(a, d->io_dtype, p.NS, p.G, s), who);
}

int ss_bwd_complex(const ss_desc* d, const void* u, const void* delta, const void* A,
                   const void* B, const void* C, const void* Dskip, const void* z,
                   const void* delta_bias, const void* h0, const void* dy, void* du,
                   void* ddelta, void* dA, void* dB, void* dC, void* dD, void* dz,
                   void* ddelta_bias, void* dh0, void* workspace, size_t workspace_bytes,
                   void* stream) {
  const char* who = "ss_bwd_complex";
  g_err[0] = 0;
  int st = check_desc(d, who);
  if (st != SS_OK) return st;
  if ((h0 == nullptr) != (dh0 == nullptr))
    return fail(SS_ERR_INVALID_PROBLEM, "%s: h0 and dh0 must be both given or both omitted", who);
  if ((Dskip == nullptr) != (dD == nullptr))
    return fail(SS_ERR_INVALID_PROBLEM, "%s: D and dD must be both given or both omitted", who);
  if ((z == nullptr) != (dz == nullptr))
    return fail(SS_ERR_INVALID_PROBLEM, "%s: z and dz must be both given or both omitted", who);
  if ((delta_bias == nullptr) != (ddelta_bias == nullptr))
    return fail(SS_ERR_INVALID_PROBLEM,
                "%s: delta_bias and ddelta_bias must be both given or both omitted", who);
  const int64_t Bn = d->batch, L = d->seqlen, D = d->dim, N = d->dstate;
  const int64_t io = dtype_size(d->io_dtype), pa = dtype_size(d->param_dtype);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const ss::Plan p = ss::make_plan_complex(*d, true);
  PtrCheck pc{who};
  if (Bn * L * D > 0) {
    pc.need(u, "u", io); pc.need(delta, "delta", io); pc.need(dy, "dy", io);
    pc.need(du, "du", io); pc.need(ddelta, "ddelta", io);
    if (N > 0) {
      pc.need(A, "A", pa); pc.need(B, "B", io); pc.need(C, "C", io);
    }
    pc.opt(z, "z", io); pc.opt(dz, "dz", io);
  }
  if (D * N > 0) pc.need(dA, "dA", pa);
  if (Bn * L * N > 0) { pc.need(dB, "dB", io); pc.need(dC, "dC", io); }
  pc.opt(Dskip, "D", pa); pc.opt(dD, "dD", pa);
  pc.opt(delta_bias, "delta_bias", pa); pc.opt(ddelta_bias, "ddelta_bias", pa);
  if (Bn * D * N > 0) { pc.opt(h0, "h0", pa); pc.opt(dh0, "dh0", pa); }
  if (pc.status != SS_OK) return pc.status;
  if (h0 && overlap(h0, dh0, 2 * Bn * D * N * pa))
    return fail(SS_ERR_INVALID_PROBLEM, "%s: dh0 must not overlap h0", who);
  st = check_workspace(p.ws_bytes, workspace, workspace_bytes, who);
  if (st != SS_OK) return st;
  if (Bn * L * D == 0 && D * N == 0 && Bn * L * N == 0 && D == 0) return SS_OK;
  const bool has_state = h0 && Bn * D * N > 0;
  ss::BwdArgs a{};
  a.u = u; a.delta = delta; a.A = A; a.B = B; a.C = C;
  a.Dskip = Dskip; a.z = z; a.bias = delta_bias; a.dy = dy;
  a.du = du; a.ddelta = ddelta; a.dA = dA; a.dB = dB; a.dC = dC;
  a.dD = dD; a.dz = dz; a.dbias = ddelta_bias;
  a.h0 = has_state ? h0 : nullptr;
  a.dh0 = has_state ? dh0 : nullptr;
  a.ws = static_cast<char*>(workspace);
  a.Bn = Bn; a.L = L; a.D = D; a.N = N;
  a.chunk_len = p.chunk_len; a.K = p.K;
  a.Lt = Bn * L; a.ldb = 2 * N; a.ldc = 2 * N;
  a.softplus = d->delta_softplus;
  a.param_dtype = d->param_dtype;
  a.io_dtype = d->io_dtype;
  return hip_status(ss::launch_bwd_complex(a, p, d->io_dtype, s), who);
}

const char* ss_status_string(int status) {
  switch (status) {
    case SS_OK: return "success";
    case SS_ERR_INVALID_PROBLEM: return "invalid problem";
    case SS_ERR_UNSUPPORTED: return "unsupported";
    case SS_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case SS_ERR_HIP: return "HIP launch error";
  }
  return "unknown status";
}

const char* ss_last_error(void) { return g_err; }

}  // extern "C"
