// Attainable-peak probes for the measurement (MI355X, gfx950): what a plain
// bf16 MFMA loop and plain HBM streams reach on the box, so that kernel
// fractions can be stated against measured peaks as well as the published
// ones.  Built into libswitch_peaks.so, separate from the layer library; the
// caller times each launch with events on the stream it passes.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

// Every wave runs `iters` rounds of four independent v_mfma_f32_32x32x16_bf16
// chains (32 x 32 x 16 x 2 = 32768 flops each) on register operands; one
// value per wave leaves so the loop is not removed.
__global__ __launch_bounds__(256) void mfma_loop_kernel(float* __restrict__ sink, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)(lane + i));
    b[i] = (__bf16)(0.002f * (float)(lane - i));
  }
  floatx16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  if (lane == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
}

// The streams give XCD k (block b runs on XCD b % 8) its own contiguous eighth
// of the buffer, which its blocks stride over; with every block striding over
// the whole buffer instead, reads reach about 15% less on MI355X.
struct Window {
  int64_t base, n, i, stride;
};
__device__ __forceinline__ Window xcd_window(int64_t n) {
  const int k = (int)(blockIdx.x & 7);
  const int64_t per = (int64_t)(gridDim.x >> 3) * blockDim.x;
  const int64_t w = n >> 3;
  Window r;
  r.base = k * w;
  r.n = k == 7 ? n - 7 * w : w;
  r.i = (int64_t)(blockIdx.x >> 3) * blockDim.x + threadIdx.x;
  r.stride = per;
  return r;
}

// Read n 16-byte pieces; one word per thread block leaves.
__global__ __launch_bounds__(256) void read_kernel(const uint4* __restrict__ src, int64_t n,
                                                   uint32_t* __restrict__ sink) {
  const Window w = xcd_window(n);
  const uint4* p = src + w.base;
  uint32_t acc = 0;
  for (int64_t i = w.i; i < w.n; i += w.stride) {
    const uint4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  __shared__ uint32_t red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int j = 0; j < 256; ++j) r ^= red[j];
    sink[blockIdx.x] = r;
  }
}

__global__ __launch_bounds__(256) void write_kernel(uint4* __restrict__ dst, int64_t n,
                                                    uint32_t v) {
  const Window w = xcd_window(n);
  uint4* p = dst + w.base;
  for (int64_t i = w.i; i < w.n; i += w.stride) p[i] = make_uint4(v, v + 1, v + 2, v + 3);
}

__global__ __launch_bounds__(256) void copy_kernel(const uint4* __restrict__ src,
                                                   uint4* __restrict__ dst, int64_t n) {
  const Window w = xcd_window(n);
  const uint4* s = src + w.base;
  uint4* d = dst + w.base;
  const int64_t stride = w.stride;
  int64_t i = w.i;
  for (; i + stride < w.n; i += 2 * stride) {
    const uint4 v0 = s[i], v1 = s[i + stride];
    d[i] = v0;
    d[i + stride] = v1;
  }
  for (; i < w.n; i += stride) d[i] = s[i];
}

// Streams: 8 blocks of 256 threads per compute unit.
unsigned stream_blocks() {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  return ((unsigned)cus * 8 + 7) & ~7u;  // a whole number of blocks per XCD
}

}  // namespace

extern "C" {

// MFMA loop: blocks of 4 waves; sink holds 4 floats per block.  Flops of one
// launch: blocks * 4 * iters * 4 * 32768.  Returns 0, or -1 on a launch error.
int peak_mfma_bf16(float* sink, int blocks, int iters, void* stream) {
  if (!sink || blocks <= 0 || iters <= 0) return -1;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                     sink, iters);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Number of sink words peak_hbm_read writes (one per block).
int peak_stream_blocks(void) { return (int)stream_blocks(); }

// HBM read of `bytes` (a multiple of 16) from src; sink: peak_stream_blocks() words.
int peak_hbm_read(const void* src, int64_t bytes, uint32_t* sink, void* stream) {
  if (!src || !sink || bytes <= 0 || bytes % 16) return -1;
  hipLaunchKernelGGL(read_kernel, dim3(stream_blocks()), dim3(256), 0, (hipStream_t)stream,
                     (const uint4*)src, bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// HBM write of `bytes` (a multiple of 16) to dst.
int peak_hbm_write(void* dst, int64_t bytes, void* stream) {
  if (!dst || bytes <= 0 || bytes % 16) return -1;
  hipLaunchKernelGGL(write_kernel, dim3(stream_blocks()), dim3(256), 0, (hipStream_t)stream,
                     (uint4*)dst, bytes / 16, 1u);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// HBM copy of `bytes` (a multiple of 16): reads and writes `bytes` each.
int peak_hbm_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  if (!src || !dst || bytes <= 0 || bytes % 16) return -1;
  hipLaunchKernelGGL(copy_kernel, dim3(stream_blocks()), dim3(256), 0, (hipStream_t)stream,
                     (const uint4*)src, (uint4*)dst, bytes / 16);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // extern "C"
