// Test support (not part of libswinattn): fills the LDS of every compute
// unit with seeded pseudo-random words.  The LDS a workgroup receives is not
// cleared between kernels, so a kernel launched right after this one on the
// same stream starts from these words; a kernel that reads LDS it has not
// written then gives results that change with the seed.  The race test runs
// each kernel after two different seeds and requires identical bits.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
constexpr int kLdsBytes = 160 * 1024;  // the whole LDS of a gfx950 compute unit

__device__ __forceinline__ uint32_t mix(uint32_t x) {
  // a 32-bit integer hash (xorshift-multiply rounds)
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

__global__ __launch_bounds__(kThreads) void lds_scrub_kernel(uint32_t seed) {
  extern __shared__ uint32_t lds[];
  // volatile (in the LDS address space): the stores are kept although
  // nothing reads them here
  typedef __attribute__((address_space(3))) volatile uint32_t lds_u32;
  lds_u32* v = (lds_u32*)(__attribute__((address_space(3))) uint32_t*)lds;
  const uint32_t base = mix(seed ^ mix(blockIdx.x * 0x9e3779b9u));
  for (int i = threadIdx.x; i < kLdsBytes / 4; i += kThreads) v[i] = mix(base + (uint32_t)i);
}

}  // namespace

extern "C" int lds_scrub(uint32_t seed, int blocks, void* stream) {
  if (blocks <= 0) return -1;
  hipLaunchKernelGGL(lds_scrub_kernel, dim3((unsigned)blocks), dim3(kThreads), kLdsBytes,
                     static_cast<hipStream_t>(stream), seed);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}
