// Device helpers shared by the Switch-layer kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swl {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // 16-byte moves

// bf16 is carried as its 16-bit pattern in memory.
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

// fp32 -> bf16 with round-to-nearest-even: the conversion instruction of
// gfx950 (v_cvt_pk_bf16_f32, IEEE rounding in the default mode), no branches.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Two fp32 values to a packed pair of bf16 (first value in the low half).
__device__ __forceinline__ uint32_t f32x2_to_bf16x2_bits(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float floatx2 __attribute__((ext_vector_type(2)));
  const floatx2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// ReLU on a packed pair of bf16 values: as 16-bit integers, exactly the
// values with the sign bit set (negatives and -0) become +0.
__device__ __forceinline__ uint32_t relu_bf16x2_bits(uint32_t p) {
  typedef short shortx2 __attribute__((ext_vector_type(2)));
  const shortx2 v = __builtin_bit_cast(shortx2, p);
  const shortx2 z = {0, 0};
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(v, z));
}

// out = x + g * y on eight bf16 values (16 bytes): fp32 fused multiply-add,
// rounded to nearest even.  y is the expert output already rounded to bf16.
__device__ __forceinline__ u32x4 combine_vec_bf16(u32x4 xv, u32x4 yv, float g) {
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float x0 = __uint_as_float(xv[i] << 16), x1 = __uint_as_float(xv[i] & 0xFFFF0000u);
    const float y0 = __uint_as_float(yv[i] << 16), y1 = __uint_as_float(yv[i] & 0xFFFF0000u);
    o[i] = f32x2_to_bf16x2_bits(fmaf(g, y0, x0), fmaf(g, y1, x1));
  }
  return o;
}

// Element access for the two activation types.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p, int64_t i) { return p[i]; }
  static __device__ __forceinline__ void store(float* p, int64_t i, float v) { p[i] = v; }
};
template <> struct Elem<uint16_t> {
  static __device__ __forceinline__ float load(const uint16_t* p, int64_t i) { return bf16_bits_to_f32(p[i]); }
  static __device__ __forceinline__ void store(uint16_t* p, int64_t i, float v) { p[i] = f32_to_bf16_bits(v); }
};

__device__ __forceinline__ double shfl_xor_f64(double v, int m) {
  int lo = __double2loint(v), hi = __double2hiint(v);
  lo = __shfl_xor(lo, m, kWave);
  hi = __shfl_xor(hi, m, kWave);
  return __hiloint2double(hi, lo);
}

// xor-shuffle of a double inside groups of `width` lanes
__device__ __forceinline__ double shfl_xor_f64_w(double v, int m, int width) {
  int lo = __double2loint(v), hi = __double2hiint(v);
  lo = __shfl_xor(lo, m, width);
  hi = __shfl_xor(hi, m, width);
  return __hiloint2double(hi, lo);
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += shfl_xor_f64(v, m);
  return v;
}

// Wave-wide max with the lowest index among equal maxima.
__device__ __forceinline__ void wave_argmax(float& v, int& idx) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    float ov = __shfl_xor(v, m, kWave);
    int oi = __shfl_xor(idx, m, kWave);
    if (ov > v || (ov == v && oi < idx)) { v = ov; idx = oi; }
  }
}

// tile_start[e] = sum over e' < e of ceil(n_kept[e'] / tile_rows), and
// tile_start[N] the total: the compact tile list of the grouped matmuls.  The
// whole block calls it; each thread takes a contiguous run of experts.  s_run:
// blockDim.x ints of LDS.
__device__ __forceinline__ void tile_prefix_block(const int32_t* __restrict__ n_kept, int N, int tile_rows,
                                  int32_t* __restrict__ tile_start, int32_t* s_run) {
  const int tid = threadIdx.x;
  const int nthr = (int)blockDim.x;
  const int per = (N + nthr - 1) / nthr;
  const int used = (N + per - 1) / per;             // threads that own experts
  const int e0 = tid * per, e1 = (e0 + per < N) ? e0 + per : N;
  int32_t sum = 0;
  for (int e = e0; e < e1; ++e) sum += (n_kept[e] + tile_rows - 1) / tile_rows;
  s_run[tid] = sum;
  __syncthreads();
  for (int off = 1; off < used; off <<= 1) {
    const int32_t v = tid >= off ? s_run[tid - off] : 0;
    __syncthreads();
    s_run[tid] += v;
    __syncthreads();
  }
  int32_t run = s_run[tid] - sum;
  for (int e = e0; e < e1; ++e) {
    tile_start[e] = run;
    run += (n_kept[e] + tile_rows - 1) / tile_rows;
  }
  if (tid == used - 1) tile_start[N] = s_run[tid];
}

// K-outer LDS tiles ([k][columns], columns innermost): rows of R + KO_PAD
// elements.  A pitch of 32 mod 128 elements puts the four rows of a
// transposing read 16 banks apart.
constexpr int KO_PAD = 32;

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

// MFMA fragment (v_mfma_f32_32x32x16_bf16 operand) of the 32 columns starting at
// col of a K-outer LDS tile, K sub-step ks: lane l receives column col + l % 32,
// rows 16 ks + 8 (l / 32) .. +7.  ds_read_b64_tr_b16: in each group of 16 lanes,
// source lane 4 q + p addresses row q and columns 4 p .. 4 p + 3 of a 4 x 16
// block and lane i receives column i of rows 0..3, so two such reads give a
// lane its column's 8 consecutive k.
__device__ __forceinline__ bf16x8 frag_kouter(const uint16_t* tile, int pitch, int ks, int col,
                                              int lane) {
  const int g = lane >> 4, j = lane & 15;
  const int row = ks * 16 + 8 * (g >> 1) + (j >> 2);
  const int c = col + 16 * (g & 1) + 4 * (j & 3);
  const uint16_t* p0 = tile + row * pitch + c;
  const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)p0);
  const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(p0 + 4 * pitch));
  typedef short shortx8 __attribute__((ext_vector_type(8)));
  const shortx8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

}  // namespace swl
