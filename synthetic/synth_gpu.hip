// Seeded, counter-based synthetic input generator (device side).
//
// Same definition as synth.c, element for element: SplitMix64 draws
// (Steele, Lea & Flood, OOPSLA 2014) -> two exact uniforms in [-1,1) ->
// Marsaglia's polar method with an ln() made of IEEE basic operations ->
// optional |z| <= 2 truncation -> (float)(z*std) -> optional bf16 RNE.
// It exists so that a weight bank of ~100 GB can be written straight into
// HBM; the host generator remains the definition, and the tests compare the
// two on sampled slices.  Compiled with floating-point contraction off.
// It holds none of the Switch layer's arithmetic.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

__device__ double synth_ln(double s) {
  uint64_t b = (uint64_t)__double_as_longlong(s);
  int e = (int)((b >> 52) & 0x7ff) - 1023;
  double m = __longlong_as_double((long long)((b & 0x000FFFFFFFFFFFFFULL) | 0x3FF0000000000000ULL));
  if (m > 1.4142135623730951) { m = m * 0.5; e += 1; }
  double t = (m - 1.0) / (m + 1.0);
  double t2 = t * t;
  double p = 1.0 / 25.0;
  p = p * t2 + 1.0 / 23.0;
  p = p * t2 + 1.0 / 21.0;
  p = p * t2 + 1.0 / 19.0;
  p = p * t2 + 1.0 / 17.0;
  p = p * t2 + 1.0 / 15.0;
  p = p * t2 + 1.0 / 13.0;
  p = p * t2 + 1.0 / 11.0;
  p = p * t2 + 1.0 / 9.0;
  p = p * t2 + 1.0 / 7.0;
  p = p * t2 + 1.0 / 5.0;
  p = p * t2 + 1.0 / 3.0;
  p = p * t2 + 1.0;
  return (double)e * 0.6931471805599453 + 2.0 * t * p;
}

__device__ __forceinline__ double synth_uniform(uint64_t stream, uint64_t n) {
  uint64_t r = mix64(stream + (n + 1ULL) * 0x9E3779B97F4A7C15ULL);
  return (double)(r >> 11) * (1.0 / 4503599627370496.0) - 1.0;
}

__device__ double synth_normal(uint64_t stream, int truncated, uint64_t index) {
  for (uint64_t a = 0; a < 64; ++a) {
    uint64_t n = (index * 64ULL + a) * 2ULL;
    double u0 = synth_uniform(stream, n);
    double u1 = synth_uniform(stream, n + 1ULL);
    double s = u0 * u0 + u1 * u1;
    if (s >= 1.0 || s == 0.0) continue;
    double z = u0 * __builtin_sqrt(-2.0 * synth_ln(s) / s);
    if (truncated && (z > 2.0 || z < -2.0)) continue;
    return z;
  }
  return 0.0;
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__global__ void fill_bf16_kernel(uint64_t stream, int truncated, double std, uint64_t start,
                                 uint64_t count, uint16_t* __restrict__ out) {
  uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (; i < count; i += stride)
    out[i] = f32_to_bf16_rne((float)(synth_normal(stream, truncated, start + i) * std));
}

__global__ void fill_f32_kernel(uint64_t stream, int truncated, double std, uint64_t start,
                                uint64_t count, float* __restrict__ out) {
  uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (; i < count; i += stride)
    out[i] = (float)(synth_normal(stream, truncated, start + i) * std);
}

uint64_t host_mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

}  // namespace

// Returns 0 on success, otherwise the hipError_t of the launch.
extern "C" int synth_gpu_fill(uint64_t seed, uint32_t tensor_id, int truncated, double std,
                              uint64_t start, uint64_t count, int is_bf16, void* out, void* stream) {
  if (count == 0) return 0;
  uint64_t s = host_mix64(seed * 256ULL + (uint64_t)tensor_id + 1ULL);
  const int threads = 256;
  uint64_t blocks = (count + threads - 1) / threads;
  if (blocks > 65536) blocks = 65536;
  hipStream_t st = (hipStream_t)stream;
  if (is_bf16)
    hipLaunchKernelGGL(fill_bf16_kernel, dim3((unsigned)blocks), dim3(threads), 0, st, s, truncated,
                       std, start, count, (uint16_t*)out);
  else
    hipLaunchKernelGGL(fill_f32_kernel, dim3((unsigned)blocks), dim3(threads), 0, st, s, truncated,
                       std, start, count, (float*)out);
  return (int)hipGetLastError();
}
