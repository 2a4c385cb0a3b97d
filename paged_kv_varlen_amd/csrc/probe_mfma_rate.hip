// Dense matrix-core throughput of v_mfma_f32_32x32x16_f16 on operands of a
// chosen distribution: a measurement tool for the prefill roofline, not part
// of the library.
//
// Every wave runs four independent accumulator chains back to back (no
// vector-ALU work, no memory traffic in the loop), so the matrix cores are the
// only busy unit.  The operand values decide how many bits toggle per product
// and therefore the power drawn; under load the chip lowers its clock to stay
// within its power limit, so the rate reached on random data is the ceiling
// that an attention kernel fed with N(0, 1) fp16 data can approach, below
// the published peak (which constant operands reach).
//
//   probe_mfma_rate            prints one line per (distribution, waves per CU)
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kIters = 4096;            // loop trips; 16 products each
constexpr double kFlopPerMfma = 32768;  // 2 * 32 * 32 * 16

__device__ inline uint32_t mix(uint32_t x) {  // 32-bit integer hash (xor-shift-multiply)
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// KIND 0: zeros; 1: the constant 1; 2: zero-mean, unit-variance values (the
// sum of two uniform variates, a triangular distribution, scaled)
template <int KIND>
__device__ inline _Float16 operand(uint32_t i) {
  if (KIND == 0) return static_cast<_Float16>(0.f);
  if (KIND == 1) return static_cast<_Float16>(1.f);
  const uint32_t h = mix(i);
  const float u = static_cast<float>((h & 0xffffu) + (h >> 16)) * (1.f / 65536.f) - 1.f;  // in (-1, 1)
  return static_cast<_Float16>(u * 2.449489743f);  // variance 1/6 -> 1
}

template <int KIND, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void mfma_rate(float* out) {
  const uint32_t tid = threadIdx.x;
  half8_t a[4], b[4];
  for (int j = 0; j < 4; ++j)
    for (int e = 0; e < 8; ++e) {
      a[j][e] = operand<KIND>(blockIdx.x * 1000003u + tid * 97u + j * 8u + e);
      b[j][e] = operand<KIND>(blockIdx.x * 7919u + tid * 131u + j * 8u + e + 55555u);
    }
  f32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < kIters; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[j], b[j], c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[j], b[(j + 1) & 3], c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[(j + 2) & 3], b[j], c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[(j + 3) & 3], b[(j + 2) & 3], c3, 0, 0, 0);
    }
    asm volatile("" ::"v"(a[0]), "v"(b[0]));  // keeps every trip's products in the loop
  }
  float s = 0.f;
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  out[blockIdx.x * 64 * WAVES + tid] = s;  // grid * 64 * WAVES floats
}

bool check(hipError_t e, const char* what) {
  if (e == hipSuccess) return true;
  std::fprintf(stderr, "probe_mfma_rate: %s: %s\n", what, hipGetErrorString(e));
  return false;
}

template <int KIND, int WAVES>
bool run(const char* name, float* out, int grid) {
  hipLaunchKernelGGL((mfma_rate<KIND, WAVES>), dim3(grid), dim3(64 * WAVES), 0, 0, out);  // warm-up
  hipEvent_t e0, e1;
  if (!check(hipEventCreate(&e0), "event") || !check(hipEventCreate(&e1), "event")) return false;
  if (!check(hipEventRecord(e0), "record")) return false;
  hipLaunchKernelGGL((mfma_rate<KIND, WAVES>), dim3(grid), dim3(64 * WAVES), 0, 0, out);
  if (!check(hipGetLastError(), "launch") || !check(hipEventRecord(e1), "record")) return false;
  if (!check(hipEventSynchronize(e1), "synchronize")) return false;
  float ms = 0.f;
  if (!check(hipEventElapsedTime(&ms, e0, e1), "elapsed")) return false;
  const double flops = static_cast<double>(grid) * WAVES * kIters * 16 * kFlopPerMfma;
  std::printf("%-24s %d waves/CU: %9.1f us  %7.1f TFLOP/s\n", name, WAVES, ms * 1e3, flops / (ms * 1e-3) / 1e12);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  return true;
}

}  // namespace

int main() {
  int dev = 0, cus = 0;
  if (!check(hipGetDevice(&dev), "device") ||
      !check(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev), "attribute"))
    return 1;
  const int grid = cus;  // one workgroup per compute unit
  float* out = nullptr;
  if (!check(hipMalloc(&out, static_cast<size_t>(grid) * 64 * 8 * sizeof(float)), "malloc")) return 1;
  std::printf("v_mfma_f32_32x32x16_f16, %d workgroups, %d products per wave\n", grid, kIters * 16);
  const bool ok = run<0, 8>("zeros", out, grid) && run<1, 8>("constant 1", out, grid) &&
                  run<2, 8>("random, unit variance", out, grid) && run<0, 4>("zeros", out, grid) &&
                  run<1, 4>("constant 1", out, grid) && run<2, 4>("random, unit variance", out, grid);
  (void)hipFree(out);
  return ok ? 0 : 1;
}
