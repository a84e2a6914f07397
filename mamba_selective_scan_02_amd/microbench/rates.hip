// Hardware rates that bound the selective scan on this GPU (gfx950).
//
// Prints, per line: the measured HBM read and copy bandwidth, and the issue
// cost of the instruction kinds the scan is made of (FP32 FMA, v_exp_f32 and
// SALU) at 1, 2 and 4 waves per SIMD.  These set the ALU roofline the scan
// is measured against (a state update is one v_exp_f32 plus four FP32 VALU
// operations).
//
//   hipcc --offload-arch=gfx950 -O3 -Xclang -target-feature -Xclang -packed-fp32-ops \
//     rates.hip -o rates && ./rates
#include <hip/hip_runtime.h>

#include <cstdio>

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

// MODE 0: 16 FMA per iteration. 1: 16 FMA + 4 v_exp_f32. 2: 16 FMA + 8 SALU.
// LDSB pads LDS so that only 160 KiB / LDSB workgroups fit on a CU, i.e. sets
// the waves per SIMD (a 256-thread workgroup is one wave on each SIMD).
template <int MODE, int LDSB>
__global__ __launch_bounds__(256) void alu_k(float* __restrict__ out, int iters) {
  __shared__ float pad[LDSB / 4];
  float x[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) x[j] = 0.5f + 0.01f * (threadIdx.x & 7) + 0.001f * j;
  uint32_t su = __builtin_amdgcn_readfirstlane(blockIdx.x + 12345u);
  uint32_t sv = __builtin_amdgcn_readfirstlane(blockIdx.x * 7u + 3u);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 16; ++j) x[j] = __builtin_fmaf(x[j], 0.999f, 0.001f);
    if (MODE == 1) {
#pragma unroll
      for (int j = 0; j < 4; ++j) x[j] = __builtin_amdgcn_exp2f(-x[j]);
    }
    if (MODE == 2) {
#pragma unroll
      for (int j = 0; j < 4; ++j) { su = (su << 1) ^ sv; sv = (sv & 0xffff0000u) | (su >> 7); }
    }
  }
  float s = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) s += x[j];
  pad[threadIdx.x % (LDSB / 4)] = s;
  __syncthreads();
  s += pad[(threadIdx.x + 1) % (LDSB / 4)];
  out[blockIdx.x * 256 + threadIdx.x] = s + (float)(su ^ sv) * 1e-30f;
}

template <int MODE, int LDSB>
static float time_alu(float* out, int blocks, int iters) {
  hipEvent_t a, b;
  (void)hipEventCreate(&a);
  (void)hipEventCreate(&b);
  alu_k<MODE, LDSB><<<blocks, 256>>>(out, iters);
  (void)hipEventRecord(a);
  for (int r = 0; r < 3; ++r) alu_k<MODE, LDSB><<<blocks, 256>>>(out, iters);
  (void)hipEventRecord(b);
  (void)hipEventSynchronize(b);
  float ms = 0;
  (void)hipEventElapsedTime(&ms, a, b);
  return ms / 3;
}

template <int LDSB>
static void alu_rates(float* out, int wps, int iters) {
  const int blocks = 256 * wps;
  const float t0 = time_alu<0, LDSB>(out, blocks, iters);
  const float t1 = time_alu<1, LDSB>(out, blocks, iters);
  const float t2 = time_alu<2, LDSB>(out, blocks, iters);
  // ns of SIMD time per wave-instruction: each SIMD runs wps waves x iters iterations
  const double per_iter = 1e6 / ((double)iters * wps);
  const double fma_ns = t0 * per_iter / 16;
  const double exp_ns = (t1 - t0) * per_iter / 4;
  const double salu_ns = (t2 - t0) * per_iter / 20;  // 5 SALU ops x 4 per iteration
  printf("waves/SIMD %d: FMA %.3f ns, v_exp_f32 %.3f ns, SALU %.3f ns per wave-instruction "
         "per SIMD  (FMA lane rate %.1f T/s)\n",
         wps, fma_ns, exp_ns, salu_ns, 64.0 * 1024 / fma_ns / 1e3);
  fflush(stdout);
}

int main() {
  hipDeviceProp_t p;
  CK(hipGetDeviceProperties(&p, 0));
  printf("device %s, %d CUs, clock %d kHz\n", p.gcnArchName, p.multiProcessorCount, p.clockRate);
  const size_t bytes = 1ull << 30, n4 = bytes / 16;
  float4 *in, *outp;
  float* red;
  CK(hipMalloc(&in, bytes));
  CK(hipMalloc(&outp, bytes));
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
  const int iters = 4096;
  alu_rates<100 * 1024>(red, 1, iters);
  alu_rates<64 * 1024>(red, 2, iters);
  alu_rates<32 * 1024>(red, 4, iters);
  CK(hipDeviceSynchronize());
  CK(hipFree(red));
  printf("rates done\n");
  return 0;
}
