/* Mamba-1 selective scan for AMD Instinct MI355X (gfx950): C ABI.
 *
 * Operation (baracuda-kernels page "src/attention/selective_scan.rs", module
 * docs, section "Algorithm summary"), per batch b, channel d and state n:
 *
 *     x        = delta[b,t,d] + delta_bias[d]            (bias optional)
 *     dt       = softplus(x) = log(1 + e^x)  if delta_softplus, else x
 *     a        = exp(dt * A[d,n])
 *     h[n]     = a * h[n] + dt * B[b,t,n] * u[b,t,d]     (h = h0[b,d,n], or 0, before t = 0)
 *     o        = sum_n C[b,t,n] * h[n] + D[d] * u[b,t,d] (D optional)
 *     y[b,t,d] = o * z * sigmoid(z), z = z[b,t,d]       (z optional)
 *     last_state[b,d,n] = h[n] after t = L-1            (optional)
 *
 * Layouts (same page, "Shape contract"): every tensor is contiguous
 * row-major; u, delta, z, y, dy, du, ddelta, dz are [B, L, D]; A and dA are
 * [D, N]; B, C, dB, dC are [B, L, N]; D, delta_bias, dD, ddelta_bias are
 * [D]; last_state, h0 and dh0 are [B, D, N].
 *
 * Conventions shared by every entry point:
 *  - Pointers are DEVICE pointers owned by the caller (workspace included).
 *    The library allocates no memory, keeps no state between calls (two
 *    exceptions, both stated where they are declared: the per-thread message
 *    of ss_last_error, and the static scratch of ss_bwd_noalloc), is
 *    reentrant, enqueues work only on the given stream (a hipStream_t; NULL
 *    means the default stream) and never synchronises.  Calls return after
 *    enqueueing; results are ready when the stream reaches that point.
 *  - Validation happens before anything is enqueued; on any error nothing is
 *    written.  Status codes follow the page's error variants
 *    (InvalidProblem, Unsupported, WorkspaceTooSmall); SS_ERR_HIP reports a
 *    failed kernel launch.  ss_last_error() gives a message for the calling
 *    thread's last failed call.
 *  - Outputs are overwritten (never accumulated into).
 *  - Arithmetic and state accumulation are f32.  io-dtype outputs are rounded
 *    to nearest even.  All reductions run in a fixed order without atomics,
 *    so every output is bitwise reproducible run to run on one device.
 */
#ifndef SS_H
#define SS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types.  Ids follow the page's workspace query (f32 = 0, f16 = 1,
 * bf16 = 2). */
typedef enum { SS_F32 = 0, SS_F16 = 1, SS_BF16 = 2 } ss_dtype;

typedef enum {
  SS_OK = 0,
  SS_ERR_INVALID_PROBLEM = 1,     /* bad extents, null or misaligned pointer, presence mismatch */
  SS_ERR_UNSUPPORTED = 2,         /* dstate > 256, dtype outside {f32, f16, bf16} */
  SS_ERR_WORKSPACE_TOO_SMALL = 3, /* workspace_bytes < ss_workspace_size() */
  SS_ERR_HIP = 4                  /* a launch failed (e.g. no gfx950 code for the device) */
} ss_status;

/* Problem descriptor (the page's SelectiveScanDescriptor, plus a separate
 * parameter dtype and a schedule override). */
typedef struct ss_desc {
  int32_t batch;          /* B >= 0 */
  int32_t seqlen;         /* L >= 0 */
  int32_t dim;            /* D >= 0 (channels) */
  int32_t dstate;         /* N, 0 <= N <= 256 */
  int32_t delta_softplus; /* 0 or 1 */
  int32_t io_dtype;       /* ss_dtype of u, delta, B, C, z, y, dy, du, ddelta, dB, dC, dz */
  int32_t param_dtype;    /* ss_dtype of A, D, delta_bias, last_state, dA, dD, ddelta_bias:
                             SS_F32 or equal to io_dtype */
  int32_t chunk_len;      /* 0: the library picks the time-chunk length from the shape
                             (the normal setting).  > 0: force chunks of this many steps
                             (for testing the chunked schedule); >= L means one chunk. */
} ss_desc;

/* Workspace bytes that ss_fwd (backward = 0) or ss_bwd (backward = 1) needs
 * for this descriptor: pure arithmetic, no device access.  Returns 0 for an
 * invalid descriptor (ss_fwd / ss_bwd then report the error).  This is the
 * query the scan page asks callers to make before a launch (module docs,
 * "Workspace"; SelectiveScanPlan::workspace_size and
 * SelectiveScanBackwardPlan::workspace_size).  The sizes differ from the
 * page's: its forward needs none and its backward records every state,
 * B*D*L*N elements.  Here a single-pass forward needs none, a forward cut
 * into time chunks needs the chunk summaries, and the backward needs f32
 * chunk checkpoints, carried adjoints and fixed-order reduction partials
 * (each sub-buffer 256-byte aligned). */
size_t ss_workspace_size(const ss_desc* desc, int32_t backward);

/* Forward.  u, delta, A, B, C, y are required; Dskip, z, delta_bias and
 * last_state may be NULL (absent).  A, B, C may be NULL only when N = 0.
 * workspace must be 256-byte aligned and hold ss_workspace_size(desc, 0)
 * bytes (it may be NULL when that size is 0).  Empty problems (B*L*D = 0)
 * return SS_OK; if L = 0 and last_state is given, last_state is set to 0
 * (the state before the first step). */
int ss_fwd(const ss_desc* desc, const void* u, const void* delta, const void* A,
           const void* B, const void* C, const void* Dskip, const void* z,
           const void* delta_bias, void* y, void* last_state, void* workspace,
           size_t workspace_bytes, void* stream);

/* Backward (BPTT) of the forward above for the loss sum(dy * y): the
 * gradient set of the page's SelectiveScanBackwardArgs.  Saved forward
 * inputs plus dy are read; du, ddelta, dA, dB, dC are required outputs; dD,
 * dz, ddelta_bias must be given exactly when Dskip, z, delta_bias are
 * (otherwise SS_ERR_INVALID_PROBLEM).  ddelta is the gradient with respect to
 * the raw delta input (through the bias and the softplus); dA is with respect
 * to A.  workspace: ss_workspace_size(desc, 1) bytes, 256-byte aligned. */
int ss_bwd(const ss_desc* desc, const void* u, const void* delta, const void* A,
           const void* B, const void* C, const void* Dskip, const void* z,
           const void* delta_bias, const void* dy, void* du, void* ddelta, void* dA,
           void* dB, void* dC, void* dD, void* dz, void* ddelta_bias, void* workspace,
           size_t workspace_bytes, void* stream);

/* Forward from a given initial state h0 [B, D, N] (param dtype; NULL means
 * zero, i.e. ss_fwd).  This is the state carried from one call to the next:
 * the mamba-rs page "mamba_ssm/gpu/backward.rs" runs its SSM forward from
 * per-layer states carried between calls (module docs, forward pipeline;
 * ssm_states [B*n_layers*d_inner*d_state] of its target-forward scratch).
 * With seqlen = 1 it is one decode step.  last_state may be the same buffer
 * as h0 (an in-place state update); the call then runs as a single chunk and
 * returns SS_ERR_UNSUPPORTED if one chunk's rows would exceed 2^31 bytes.
 * h0 and last_state must otherwise not overlap.  If L = 0, last_state = h0.
 * Everything else as ss_fwd. */
int ss_fwd_h0(const ss_desc* desc, const void* u, const void* delta, const void* A,
              const void* B, const void* C, const void* Dskip, const void* z,
              const void* delta_bias, const void* h0, void* y, void* last_state,
              void* workspace, size_t workspace_bytes, void* stream);

/* Backward of ss_fwd_h0: as ss_bwd, plus dh0 [B, D, N] (param dtype), the
 * gradient with respect to h0, which must be given exactly when h0 is
 * (otherwise SS_ERR_INVALID_PROBLEM) and must not overlap h0.  If L = 0,
 * dh0 = 0.  Same workspace as ss_bwd. */
int ss_bwd_h0(const ss_desc* desc, const void* u, const void* delta, const void* A,
              const void* B, const void* C, const void* Dskip, const void* z,
              const void* delta_bias, const void* h0, const void* dy, void* du, void* ddelta,
              void* dA, void* dB, void* dC, void* dD, void* dz, void* ddelta_bias, void* dh0,
              void* workspace, size_t workspace_bytes, void* stream);

/* Forward over packed variable-length sequences.  The scan page leaves
 * variable-length sequences (cu_seqlens) out of its scope (module docs,
 * "Trailblazer scope"); this is the usual packed layout.  desc->batch is the
 * number of sequences S and desc->seqlen an upper bound on every sequence's
 * length; cu_seqlens is a DEVICE array of S + 1 int32 row offsets
 * (cu_seqlens[0] = 0, non-decreasing, cu_seqlens[S] = total_len).  Sequence s
 * occupies rows cu_seqlens[s] .. cu_seqlens[s+1] - 1 of u, delta, z, y
 * ([total_len, D]) and of B, C ([total_len, N]); each sequence is scanned
 * independently from h0[s] (or 0), and last_state[s] is its final state
 * ([S, D, N]).  The offsets are read on the device and not validated there
 * beyond clamping into [0, total_len] and lengths to desc->seqlen: rows no
 * sequence covers are not written (their backward gradients are unspecified).
 * total_len > batch * seqlen is SS_ERR_INVALID_PROBLEM.  Workspace:
 * ss_workspace_size(desc, 0) with the same desc.  Everything else as
 * ss_fwd_h0. */
int ss_fwd_varlen(const ss_desc* desc, const int32_t* cu_seqlens, int64_t total_len,
                  const void* u, const void* delta, const void* A, const void* B, const void* C,
                  const void* Dskip, const void* z, const void* delta_bias, const void* h0,
                  void* y, void* last_state, void* workspace, size_t workspace_bytes,
                  void* stream);

/* Backward of ss_fwd_varlen: as ss_bwd_h0 with the packed layout (du,
 * ddelta, dz, dy [total_len, D]; dB, dC [total_len, N]; h0 / dh0 [S, D, N]).
 * Workspace: ss_workspace_size(desc, 1) with the same desc. */
int ss_bwd_varlen(const ss_desc* desc, const int32_t* cu_seqlens, int64_t total_len,
                  const void* u, const void* delta, const void* A, const void* B, const void* C,
                  const void* Dskip, const void* z, const void* delta_bias, const void* h0,
                  const void* dy, void* du, void* ddelta, void* dA, void* dB, void* dC,
                  void* dD, void* dz, void* ddelta_bias, void* dh0, void* workspace,
                  size_t workspace_bytes, void* stream);

/* Forward and backward with B and C read as row-strided column slices.  The
 * scan page restricts itself to contiguous layouts (module docs,
 * "Trailblazer scope"); the mamba-rs page "mamba_ssm/gpu/backward.rs" keeps
 * B and C as column ranges of the x-projection output xdbl (row width
 * dt_rank + 2N, B at column dt_rank, C at dt_rank + N), gathers them into
 * contiguous buffers before its SSM backward and scatters dB / dC back into
 * the matching columns of d_xdbl afterwards (section "B3: SSM BPTT +
 * reductions").  Here row t of B (and of dB) starts ldb elements after row
 * t - 1, and likewise C / dC with ldc, so B = xdbl + dt_rank, C = xdbl +
 * dt_rank + N, ldb = ldc = dt_rank + 2N read and write those columns in
 * place.  ldb / ldc = 0 means N (packed); otherwise each must be >= N.  Only
 * the first N elements of each dB / dC row are written; the elements between
 * rows are not touched, so they may hold other data (e.g. the dt columns of
 * d_xdbl), but they must not overlap any other argument.  cu_seqlens = NULL
 * gives the dense layout of ss_fwd_h0 / ss_bwd_h0 (total_len is then
 * ignored), otherwise the packed layout of ss_fwd_varlen / ss_bwd_varlen.
 * With the tile kernels (dstate <= 32), a stride whose byte extent over one
 * chunk exceeds 2^31 is SS_ERR_UNSUPPORTED (a shorter desc->chunk_len
 * lifts that).  Everything else, workspace included, as those entry points. */
int ss_fwd_strided(const ss_desc* desc, const int32_t* cu_seqlens, int64_t total_len,
                   int64_t ldb, int64_t ldc, const void* u, const void* delta, const void* A,
                   const void* B, const void* C, const void* Dskip, const void* z,
                   const void* delta_bias, const void* h0, void* y, void* last_state,
                   void* workspace, size_t workspace_bytes, void* stream);
int ss_bwd_strided(const ss_desc* desc, const int32_t* cu_seqlens, int64_t total_len,
                   int64_t ldb, int64_t ldc, const void* u, const void* delta, const void* A,
                   const void* B, const void* C, const void* Dskip, const void* z,
                   const void* delta_bias, const void* h0, const void* dy, void* du,
                   void* ddelta, void* dA, void* dB, void* dC, void* dD, void* dz,
                   void* ddelta_bias, void* dh0, void* workspace, size_t workspace_bytes,
                   void* stream);

/* Complex-valued variant.  The scan page reserves complex variants without
 * defining them (module docs, "Trailblazer scope"); here the recurrence of
 * its "Algorithm summary" runs with A, B, C and the state complex and the
 * rest real:
 *     a = exp(dt * A[d,n])                      (complex; dt as above)
 *     h = a * h + dt * u[b,t,d] * B[b,t,n]      (h = h0[b,d,n], or 0, before t = 0)
 *     o = Re(sum_n C[b,t,n] * h[n]) + D[d] * u[b,t,d],   y = o * silu(z)
 * Complex tensors are (re, im) pairs in a trailing axis of 2: A [D, N, 2] and
 * h0 / last_state [B, D, N, 2] in param_dtype, B, C [B, L, N, 2] in io_dtype;
 * the gradients dA, dB, dC, dh0 have the same layouts and hold
 * (dL/dRe, dL/dIm) of each element.  Real tensors are as for ss_fwd_h0 /
 * ss_bwd_h0.  A convention that keeps one state of each conjugate pair and
 * doubles the real part is this operation with C scaled by 2.  The layouts
 * are dense and packed (no cu_seqlens, no strides).  Workspace:
 * ss_workspace_size_complex(desc, backward).  Validation, ownership,
 * streams, determinism and the in-place state update (last_state == h0) are
 * as for the real entry points. */
size_t ss_workspace_size_complex(const ss_desc* desc, int32_t backward);
int ss_fwd_complex(const ss_desc* desc, const void* u, const void* delta, const void* A,
                   const void* B, const void* C, const void* Dskip, const void* z,
                   const void* delta_bias, const void* h0, void* y, void* last_state,
                   void* workspace, size_t workspace_bytes, void* stream);
int ss_bwd_complex(const ss_desc* desc, const void* u, const void* delta, const void* A,
                   const void* B, const void* C, const void* Dskip, const void* z,
                   const void* delta_bias, const void* h0, const void* dy, void* du,
                   void* ddelta, void* dA, void* dB, void* dC, void* dD, void* dz,
                   void* ddelta_bias, void* dh0, void* workspace, size_t workspace_bytes,
                   void* stream);

/* Backward for callers that cannot allocate (code under HIP graph capture,
 * tight serving or training loops, harnesses that forbid hipMalloc): ss_bwd_h0
 * without the workspace arguments.  Its scratch is a static device array of
 * SS_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held from the
 * first call on that GPU until the process ends; the call itself allocates
 * nothing.  A problem whose ss_workspace_size(desc, 1) exceeds
 * SS_NOALLOC_SCRATCH_BYTES returns SS_ERR_UNSUPPORTED before anything is
 * enqueued (the backward workload B=2, L=2048, D=2048, N=16 needs 57.5 MiB).
 * Every call on one GPU shares that GPU's array: calls that overlap in time
 * on one GPU (other streams, other threads, other host processes' contexts
 * excepted) race and give undefined results; serialise them on one stream.
 * The first call on a GPU looks the array's address up (a mutex guards that
 * lookup).  Everything else, including the results bit for bit, as ss_bwd_h0. */
#define SS_NOALLOC_SCRATCH_BYTES (64u << 20)
int ss_bwd_noalloc(const ss_desc* desc, const void* u, const void* delta, const void* A,
                   const void* B, const void* C, const void* Dskip, const void* z,
                   const void* delta_bias, const void* h0, const void* dy, void* du,
                   void* ddelta, void* dA, void* dB, void* dC, void* dD, void* dz,
                   void* ddelta_bias, void* dh0, void* stream);

/* The schedule the library would use for a descriptor (informational). */
typedef struct ss_plan {
  int32_t chunk_len;          /* time steps per chunk */
  int32_t n_chunks;           /* chunks along L (1 = single pass) */
  int32_t states_per_lane;    /* state registers per lane (>= N / lanes_per_channel) */
  int32_t lanes_per_channel;  /* lanes sharing one channel's states */
  int32_t n_launches;         /* kernels enqueued per call */
} ss_plan;

/* Fills *out for ss_fwd (backward = 0) or ss_bwd (backward = 1).  Returns a
 * status like the entry points (no device access). */
int ss_plan_query(const ss_desc* desc, int32_t backward, ss_plan* out);

/* Static text for a status code, naming the scan page's error
 * variants (Error::InvalidProblem, Error::Unsupported,
 * Error::WorkspaceTooSmall, returned by SelectiveScanPlan::select /
 * can_implement and the backward plan's run) and of a failed launch, which
 * the page maps from the kernel's return code (map_status).  Unknown codes
 * give "unknown status".  Never NULL; the text is static. */
const char* ss_status_string(int status);

/* Message describing the calling thread's most recent failed call ("" if
 * none): which entry point, which argument and why.  This is the library's
 * one piece of per-thread state: a thread-local buffer of 512 bytes that
 * every entry point clears on entry and fills on failure.  The pointer stays
 * valid until the same thread's next call into the library. */
const char* ss_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SS_H */
