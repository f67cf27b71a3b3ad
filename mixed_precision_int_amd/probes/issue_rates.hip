// Issue-rate probe for gfx950: how fast one CU sustains the long-prompt
// GEMM's instruction mix with no global-memory traffic.
//
// Each wave runs chains of v_mfma_i32_32x32x32_i8 (four k-steps per 32 x 32
// fragment, eight fragments per pass) and, depending on the mode:
//   mfma         : the MFMAs alone;
//   +rescale     : the eq. 19 rescale of the previous fragment's INT32
//                  products into FP32 sums (one convert and one FMA per
//                  element: 8 vector-ALU instructions per MFMA), the ratio of
//                  the GEMM's inner loop at b_K = 128;
//   +rescale+lds : the same plus one 16-byte LDS fragment read per MFMA;
//   +lds         : MFMAs and LDS reads, no rescale;
//   rescale-only : the vector-ALU work alone, reported as the MFMA rate it
//                  would allow.
// at 1, 2 and 4 waves per SIMD (one workgroup per CU: 100 KB of LDS each).
// Rates are INT8 TOPS over the whole GPU (2 ops per multiply-add), timed
// with HIP events; the dense INT8 peak of an MI355X is 5000 TOPS.
//
// Build: hipcc --offload-arch=gfx950 -O3 -std=c++17 -Xclang -target-feature
//        -Xclang -packed-fp32-ops -mllvm -amdgpu-mfma-vgpr-form=1
//        issue_rates.hip -o issue_rates   (mixed_precision_int_amd/build.py)
#include <hip/hip_runtime.h>

#include <cstdio>

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

enum { kMfma = 0, kRescale = 1, kRescaleLds = 2, kLds = 3, kRescaleOnly = 4 };

template <int WPS, int MODE, int NF>
__global__ __launch_bounds__(256 * WPS, 1) void probe(int iters, float *out, int seed) {
  __shared__ __attribute__((aligned(1024))) int8_t lds[102400];  // one workgroup per CU
  const int lane = threadIdx.x & 63;
  for (int i = threadIdx.x; i < 65536 / 4; i += blockDim.x)
    reinterpret_cast<int *>(lds)[i] = (int)(i * 2654435761u) + seed;
  __syncthreads();
  v4i fa[4], fb[2];
  for (int u = 0; u < 4; ++u) fa[u] = v4i{lane + u, seed, lane ^ u, 3};
  for (int u = 0; u < 2; ++u) fb[u] = v4i{lane * 7 + u, 1, seed, lane};
  float F[NF][16];
  for (int f = 0; f < NF; ++f)
    for (int e = 0; e < 16; ++e) F[f][e] = 0.f;
  v16i acc[2] = {v16i{0}, v16i{0}};
  const float sc = 1.0f + lane * 1e-3f;
  const int base = ((threadIdx.x >> 6) * 2048 + lane * 16) & 65535;
  for (int it = 0; it < iters; ++it) {
    // the operands are opaque to the compiler, so no MFMA is hoisted
    asm volatile("" : "+v"(fa[0]), "+v"(fa[1]), "+v"(fa[2]), "+v"(fa[3]), "+v"(fb[0]), "+v"(fb[1]));
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      const int p = f & 1;
      if (MODE == kRescaleLds || MODE == kLds) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
          fa[u] = *reinterpret_cast<const v4i *>(lds + ((base + f * 4096 + u * 1024) & 65535));
      }
      if (MODE != kRescaleOnly) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
          acc[p] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[u], fb[u & 1], acc[p], 0, 0, 0);
      } else {
        asm volatile("" : "+v"(acc[p]));
      }
      if (MODE == kRescale || MODE == kRescaleLds || MODE == kRescaleOnly) {
        const int q = (f + 7) % NF;
#pragma unroll
        for (int e = 0; e < 16; ++e) F[q][e] = fmaf((float)acc[p ^ 1][e], sc, F[q][e]);
      }
    }
  }
  float s = 0.f;
  for (int f = 0; f < NF; ++f)
    for (int e = 0; e < 16; ++e) s += F[f][e];
  s += (float)(acc[0][0] + acc[1][3]);
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

static bool ok(hipError_t e) {
  if (e != hipSuccess) std::fprintf(stderr, "HIP error: %s\n", hipGetErrorString(e));
  return e == hipSuccess;
}

template <int WPS, int MODE, int NF>
double rate(int cus, float *out) {
  constexpr int iters = 2000;
  hipEvent_t a, b;
  if (!ok(hipEventCreate(&a)) || !ok(hipEventCreate(&b))) return -1;
  hipLaunchKernelGGL((probe<WPS, MODE, NF>), dim3(cus), dim3(256 * WPS), 0, 0, 4, out, 1);  // warm-up
  if (!ok(hipEventRecord(a, 0))) return -1;
  hipLaunchKernelGGL((probe<WPS, MODE, NF>), dim3(cus), dim3(256 * WPS), 0, 0, iters, out, 1);
  if (!ok(hipEventRecord(b, 0)) || !ok(hipEventSynchronize(b))) return -1;
  float ms = 0;
  if (!ok(hipEventElapsedTime(&ms, a, b))) return -1;
  (void)hipEventDestroy(a);
  (void)hipEventDestroy(b);
  const double ops = (double)cus * 4 * WPS * iters * 8 * 4 * 65536.0;
  return ops / (ms * 1e-3) / 1e12;
}

template <int WPS, int NF>
void row(int cus, float *out) {
  std::printf("| %d | %.0f | %.0f | %.0f | %.0f | %.0f |\n", WPS, rate<WPS, kMfma, NF>(cus, out),
              rate<WPS, kRescale, NF>(cus, out), rate<WPS, kRescaleLds, NF>(cus, out),
              rate<WPS, kLds, NF>(cus, out), rate<WPS, kRescaleOnly, NF>(cus, out));
}

int main() {
  int dev = 0, cus = 0;
  if (!ok(hipGetDevice(&dev)) ||
      !ok(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)))
    return 1;
  float *out = nullptr;
  if (!ok(hipMalloc(&out, (size_t)cus * 1024 * sizeof(float)))) return 1;
  std::printf("| waves per SIMD | mfma TOPS | +rescale | +rescale+lds | +lds | rescale-only (as MFMA TOPS) |\n");
  std::printf("|---|---|---|---|---|---|\n");
  row<1, 4>(cus, out);
  row<2, 4>(cus, out);
  row<4, 2>(cus, out);
  const bool good = ok(hipDeviceSynchronize());
  (void)hipFree(out);
  return good ? 0 : 1;
}
