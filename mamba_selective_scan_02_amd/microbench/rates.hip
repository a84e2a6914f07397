// Hardware rates that bound the selective scan on this GPU (gfx950).
//
// Prints the measured HBM read and copy bandwidth, then the issue cost of the
// instruction kinds a state update is made of, at 1 to 8 resident waves per
// SIMD:
//
//   fma        16 independent chains of v_fma_f32 (VGPR operands)
//   exp        16 independent chains of v_exp_f32
//   fma+exp    16 FMA chains and 4 exp chains with no data flow between them:
//              its time against fma's and exp's says whether the
//              transcendental unit issues beside the FP32 VALU (time near the
//              larger of the two parts) or takes VALU issue slots (near their
//              sum)
//   update     the scan's own state update on 4 states x 4 steps per
//              iteration: a = exp2(dt * A), h = a * h + x * B, o += C * h
//              (4 FP32 VALU + 1 exp per update), B and C in VGPRs
//   update_s   the same with B and C wave-uniform (SGPR operands)
//   upd_nexp   the update without its exp (a = dt * A), for the VALU share
//   upd_clust  the update with its 16 exps issued back to back (empty asm
//              fences order: 16 dt*A products, 16 exps, then the 48 other
//              operations), against the compiler's interleaved order
//   perm32     8 v_permlane32_swap per iteration (8 independent pairs) plus
//              16 FMAs; perm16 the same with v_permlane16_swap; dpp_add 16
//              v_add_f32 with a DPP row rotation plus 16 FMAs: the cross-lane
//              steps of the readout's sum over a channel's lanes
//
// Each line gives ns and shader-clock cycles per wave-instruction per SIMD
// (the SIMD's issue cost of one 64-lane instruction), the clock the kernel
// ran at (s_memtime cycles over elapsed time), and for the update kernels
// the state updates per second of the whole chip.
//
//   hipcc --offload-arch=gfx950 -O3 -Xclang -target-feature -Xclang -packed-fp32-ops \
//     rates.hip -o rates && ./rates
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdint>

#define CK(x)                                                                       \
  do {                                                                              \
    hipError_t e_ = (x);                                                            \
    if (e_ != hipSuccess) {                                                         \
      printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);         \
      return 1;                                                                     \
    }                                                                               \
  } while (0)

__global__ void copy_k(const float4* __restrict__ in, float4* __restrict__ out, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    out[i] = in[i];
}

__global__ void read_k(const float4* __restrict__ in, float* __restrict__ out, size_t n) {
  float4 acc = {0, 0, 0, 0};
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x) {
    const float4 v = in[i];
    acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
  }
  out[blockIdx.x * (size_t)blockDim.x + threadIdx.x] = acc.x + acc.y + acc.z + acc.w;
}

enum { M_FMA = 0, M_EXP, M_MIX, M_UPD, M_UPD_S, M_UPD_NEXP, M_UPD_CL, M_PERM32, M_PERM16,
       M_DPP, M_COUNT };
static const char* kModeName[M_COUNT] = {"fma", "exp", "fma+exp", "update", "update_s",
                                         "upd_nexp", "upd_clust", "perm32", "perm16", "dpp_add"};
// counted wave-instructions per iteration of each mode
static const int kInstr[M_COUNT] = {16, 16, 20, 80, 80, 64, 80, 24, 24, 32};
// state updates per lane per iteration (update kernels)
static const int kUpd[M_COUNT] = {0, 0, 0, 16, 16, 16, 16, 0, 0, 0};

// Keeps v in a VGPR and opaque to the optimiser without emitting code.
#define OPAQUE(v) __asm__ volatile("" : "+v"(v))

// The dynamic LDS request sets how many 256-lane workgroups (one wave per
// SIMD each) fit on a CU, i.e. the resident waves per SIMD.
template <int MODE>
__global__ __launch_bounds__(256, 8) void alu_k(float* __restrict__ out, long long* __restrict__ clk,
                                             const float* __restrict__ uni, int iters) {
  extern __shared__ float pad[];
  const int tid = threadIdx.x;
  const float f = 1.0f + 1e-7f * (tid & 63);
  float x[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) x[j] = (0.5f + 0.001f * j) * f;
  float c0 = 0.999f * f, c1 = 0.001f * f;
  OPAQUE(c0);
  OPAQUE(c1);
  // update kernels: 4 steps (dt, x), 4 states (A2, h, B, C)
  float dt[4], xu[4], A2[4], h[4], o[4], Bv[4], Cv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    dt[i] = (0.1f + 0.05f * i) * f;
    xu[i] = (0.3f - 0.02f * i) * f;
    A2[i] = -(1.0f + i) * 1.4426950408889634f * f;
    h[i] = 0.0f;
    o[i] = 0.0f;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (MODE == M_UPD_S) {
      Bv[j] = uni[j];
      Cv[j] = uni[16 + j];
    } else {
      Bv[j] = (0.5f - 0.03f * j) * f;
      Cv[j] = (0.25f + 0.01f * j) * f;
    }
  }
  const long long t_start = clock64();
  for (int it = 0; it < iters; ++it) {
    if (MODE == M_FMA || MODE == M_MIX) {
#pragma unroll
      for (int j = 0; j < 16; ++j) x[j] = __builtin_fmaf(x[j], c0, c1);
    }
    if (MODE == M_EXP) {
#pragma unroll
      for (int j = 0; j < 16; ++j) x[j] = __builtin_amdgcn_exp2f(-x[j]);
    }
    if (MODE == M_MIX) {
      // 4 exp chains on their own registers: no data flow to or from the FMAs
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = __builtin_amdgcn_exp2f(-o[j]);
    }
    if (MODE == M_PERM32 || MODE == M_PERM16) {
      // 8 pairs (x[2k], x[2k+1]) swapped across lanes, then each pair summed back
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const auto r = MODE == M_PERM32
            ? __builtin_amdgcn_permlane32_swap(__float_as_uint(x[2 * k]),
                                               __float_as_uint(x[2 * k + 1]), false, false)
            : __builtin_amdgcn_permlane16_swap(__float_as_uint(x[2 * k]),
                                               __float_as_uint(x[2 * k + 1]), false, false);
        const unsigned r0 = r[0], r1 = r[1];
        x[2 * k] = __builtin_fmaf(__uint_as_float(r0), c0, c1);
        x[2 * k + 1] = __builtin_fmaf(__uint_as_float(r1), c0, c1);
      }
    }
    if (MODE == M_DPP) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float d = __builtin_bit_cast(
            float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x[j]), 0x128, 0xf, 0xf, true));
        x[j] = __builtin_fmaf(d + x[j], c0, c1);
      }
    }
    if (MODE == M_UPD_CL) {
      float e[16];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        OPAQUE(dt[i]);
        OPAQUE(xu[i]);
      }
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i) e[4 * s + i] = dt[s] * A2[i];
#pragma unroll
      for (int j = 0; j < 16; ++j) OPAQUE(e[j]);
#pragma unroll
      for (int j = 0; j < 16; ++j) e[j] = __builtin_amdgcn_exp2f(e[j]);
      // the other operations read xu, B, C only after this fence
#pragma unroll
      for (int j = 0; j < 16; ++j) OPAQUE(e[j]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        OPAQUE(xu[i]);
        OPAQUE(Bv[i]);
        OPAQUE(Cv[i]);
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        float acc = o[s];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          h[i] = __builtin_fmaf(e[4 * s + i], h[i], xu[s] * Bv[i]);
          acc = __builtin_fmaf(Cv[i], h[i], acc);
        }
        o[s] = acc;
      }
    }
    if (MODE == M_UPD || MODE == M_UPD_S || MODE == M_UPD_NEXP) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        OPAQUE(dt[i]);
        OPAQUE(xu[i]);
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        float acc = o[s];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float arg = dt[s] * A2[i];
          const float a = (MODE == M_UPD_NEXP) ? arg : __builtin_amdgcn_exp2f(arg);
          h[i] = __builtin_fmaf(a, h[i], xu[s] * Bv[i]);
          acc = __builtin_fmaf(Cv[i], h[i], acc);
        }
        o[s] = acc;
      }
    }
  }
  const long long t_end = clock64();
  float s = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) s += x[j];
#pragma unroll
  for (int i = 0; i < 4; ++i) s += h[i] + o[i];
  pad[tid] = s;
  __syncthreads();
  s += pad[(tid + 1) & 255];
  out[blockIdx.x * 256 + tid] = s;
  if ((tid & 63) == 0) clk[blockIdx.x * 4 + (tid >> 6)] = t_end - t_start;
}

struct Timing { double ms, cycles; };

template <int MODE>
static Timing time_alu(float* out, long long* clk, const float* uni, int blocks, int lds,
                       int iters) {
  hipEvent_t a, b;
  (void)hipEventCreate(&a);
  (void)hipEventCreate(&b);
  alu_k<MODE><<<blocks, 256, lds>>>(out, clk, uni, iters);
  (void)hipEventRecord(a);
  const int reps = 3;
  for (int r = 0; r < reps; ++r) alu_k<MODE><<<blocks, 256, lds>>>(out, clk, uni, iters);
  (void)hipEventRecord(b);
  (void)hipEventSynchronize(b);
  float ms = 0;
  (void)hipEventElapsedTime(&ms, a, b);
  (void)hipEventDestroy(a);
  (void)hipEventDestroy(b);
  static long long host[16384 * 4];
  (void)hipMemcpy(host, clk, sizeof(long long) * blocks * 4, hipMemcpyDeviceToHost);
  double sum = 0;
  for (int i = 0; i < blocks * 4; ++i) sum += (double)host[i];
  return {ms / reps, sum / (blocks * 4)};
}

template <int MODE>
static void report(float* out, long long* clk, const float* uni, int wps, int lds, int iters) {
  const int blocks = 256 * wps;  // wps workgroups per CU: wps waves on each SIMD
  const Timing t = time_alu<MODE>(out, clk, uni, blocks, lds, iters);
  const double instr_per_simd = (double)iters * wps * kInstr[MODE];
  const double ns = t.ms * 1e6 / instr_per_simd;
  // one wave's measured cycles cover the instructions of all wps waves sharing its SIMD
  const double cyc = t.cycles / ((double)iters * kInstr[MODE]) / wps;
  const double ghz = t.cycles / (t.ms * 1e6);
  printf("waves/SIMD %d  %-9s %7.3f ns  %6.2f cycles per wave-instruction per SIMD  (clock %.2f GHz",
         wps, kModeName[MODE], ns, cyc, ghz);
  if (kUpd[MODE]) {
    const double upd = (double)blocks * 256 * iters * kUpd[MODE];
    printf(", %.3g state-updates/s", upd / (t.ms * 1e-3));
  }
  printf(")\n");
  fflush(stdout);
}

int main() {
  hipDeviceProp_t p;
  CK(hipGetDeviceProperties(&p, 0));
  printf("device %s, %d CUs, clock %d kHz, LDS per CU %zu bytes\n", p.gcnArchName,
         p.multiProcessorCount, p.clockRate, (size_t)p.maxSharedMemoryPerMultiProcessor);
  const size_t bytes = 1ull << 30, n4 = bytes / 16;
  float4 *in, *outp;
  CK(hipMalloc(&in, bytes));
  CK(hipMalloc(&outp, bytes));
  float* red;
  CK(hipMalloc(&red, sizeof(float) * 16384 * 256));  // >= largest grid * 256
  CK(hipMemset(in, 0, bytes));
  hipEvent_t a, b;
  CK(hipEventCreate(&a));
  CK(hipEventCreate(&b));
  for (int grid : {2048, 8192}) {
    copy_k<<<grid, 256>>>(in, outp, n4);
    CK(hipDeviceSynchronize());
    CK(hipEventRecord(a));
    for (int r = 0; r < 10; ++r) copy_k<<<grid, 256>>>(in, outp, n4);
    CK(hipEventRecord(b));
    CK(hipEventSynchronize(b));
    float ms = 0;
    CK(hipEventElapsedTime(&ms, a, b));
    printf("copy 1 GiB (grid %d): %.1f GB/s read+write\n", grid, 2.0 * bytes / (ms / 10) / 1e6);
    read_k<<<grid, 256>>>(in, red, n4);
    CK(hipDeviceSynchronize());
    CK(hipEventRecord(a));
    for (int r = 0; r < 10; ++r) read_k<<<grid, 256>>>(in, red, n4);
    CK(hipEventRecord(b));
    CK(hipEventSynchronize(b));
    CK(hipEventElapsedTime(&ms, a, b));
    printf("read 1 GiB (grid %d): %.1f GB/s\n", grid, 1.0 * bytes / (ms / 10) / 1e6);
    fflush(stdout);
  }
  CK(hipFree(in));
  CK(hipFree(outp));
  long long* clk;
  CK(hipMalloc(&clk, sizeof(long long) * 16384 * 4));
  float* uni;
  CK(hipMalloc(&uni, sizeof(float) * 32));
  float huni[32];
  for (int j = 0; j < 16; ++j) {
    huni[j] = 0.5f - 0.03f * j;
    huni[16 + j] = 0.25f + 0.01f * j;
  }
  CK(hipMemcpy(uni, huni, sizeof(huni), hipMemcpyHostToDevice));
  const int lds_cu = (int)p.maxSharedMemoryPerMultiProcessor;  // 160 KiB on gfx950
  const int max_lds = (int)p.sharedMemPerBlock;                // a workgroup may take all of it
  CK(hipFuncSetAttribute((const void*)alu_k<M_FMA>, hipFuncAttributeMaxDynamicSharedMemorySize, max_lds));
  CK(hipFuncSetAttribute((const void*)alu_k<M_EXP>, hipFuncAttributeMaxDynamicSharedMemorySize, max_lds));
  CK(hipFuncSetAttribute((const void*)alu_k<M_MIX>, hipFuncAttributeMaxDynamicSharedMemorySize, max_lds));
  CK(hipFuncSetAttribute((const void*)alu_k<M_UPD>, hipFuncAttributeMaxDynamicSharedMemorySize, max_lds));
  CK(hipFuncSetAttribute((const void*)alu_k<M_UPD_S>, hipFuncAttributeMaxDynamicSharedMemorySize, max_lds));
  CK(hipFuncSetAttribute((const void*)alu_k<M_UPD_NEXP>, hipFuncAttributeMaxDynamicSharedMemorySize, max_lds));
  CK(hipFuncSetAttribute((const void*)alu_k<M_UPD_CL>, hipFuncAttributeMaxDynamicSharedMemorySize, max_lds));
  CK(hipFuncSetAttribute((const void*)alu_k<M_PERM32>, hipFuncAttributeMaxDynamicSharedMemorySize, max_lds));
  CK(hipFuncSetAttribute((const void*)alu_k<M_PERM16>, hipFuncAttributeMaxDynamicSharedMemorySize, max_lds));
  CK(hipFuncSetAttribute((const void*)alu_k<M_DPP>, hipFuncAttributeMaxDynamicSharedMemorySize, max_lds));
  const int iters = 2048;
  for (int wps : {1, 2, 3, 4, 5, 6, 8}) {
    // the largest 1 KiB multiple that lets wps workgroups, but not wps + 1, share a CU
    int lds = (lds_cu / wps) / 1024 * 1024;
    if (lds > max_lds) lds = max_lds;
    report<M_FMA>(red, clk, uni, wps, lds, iters);
    report<M_EXP>(red, clk, uni, wps, lds, iters);
    report<M_MIX>(red, clk, uni, wps, lds, iters);
    report<M_UPD>(red, clk, uni, wps, lds, iters);
    report<M_UPD_S>(red, clk, uni, wps, lds, iters);
    report<M_UPD_NEXP>(red, clk, uni, wps, lds, iters);
    report<M_UPD_CL>(red, clk, uni, wps, lds, iters);
    report<M_PERM32>(red, clk, uni, wps, lds, iters);
    report<M_PERM16>(red, clk, uni, wps, lds, iters);
    report<M_DPP>(red, clk, uni, wps, lds, iters);
  }
  CK(hipDeviceSynchronize());
  CK(hipFree(red));
  CK(hipFree(clk));
  CK(hipFree(uni));
  printf("rates done\n");
  return 0;
}
