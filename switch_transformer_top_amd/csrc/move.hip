// Dispatch gather and combine scatter.
//
// On one device the dispatcher and combiner are memory moves (kasblo explainer,
// section "tokenをExpertへ送って戻すforward pass": grouping tokens per expert
// and returning them to token order is a gather/scatter in memory).
//   dispatch: Xbuf[e, p, :] = x[t, :] for every kept token t (e = e_t, p = position_t)
//   combine:  out[t] = x[t] + gate[t] * Ybuf[e_t, position_t]  (kept)
//             out[t] = x[t] bit for bit                         (dropped: passed
//             through on the residual, llm-papers-study section 3.4; "Switch
//             Transformer by Hand" step 13)
// The gate multiply is the paper's y = p_{i*}(x) E_{i*}(x) (llm-papers-study
// section 3.2); the residual add sits inside the layer as in its part 六 diagram.
#include "common.hpp"
#include "kernels.hpp"

namespace swl {

// One thread per 16-byte piece of a row: every row's index loads and data
// moves run concurrently across the grid instead of row after row.
// row_vec16 = bytes of one row / 16 (rows are a multiple of 16 bytes).

// Dispatch also finalises the routing: position = chunk offset + in-chunk
// rank, drop = position >= C; kept rows are copied to their expert slot.
__global__ __launch_bounds__(256) void dispatch_kernel(const uint4* __restrict__ x, int64_t T,
                                                       int row_vec16,
                                                       const int32_t* __restrict__ expert_idx,
                                                       const int32_t* __restrict__ rank_local,
                                                       const int32_t* __restrict__ offsets, int N,
                                                       int64_t chunk, int64_t C,
                                                       int32_t* __restrict__ position,
                                                       uint8_t* __restrict__ drop_mask,
                                                       uint4* __restrict__ Xbuf) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t t = gid / row_vec16;
  const int c = (int)(gid - t * row_vec16);
  if (t >= T) return;
  const int32_t e = expert_idx[t];
  const int32_t pos = offsets[(t / chunk) * N + e] + rank_local[t];
  const bool dropped = (int64_t)pos >= C;
  if (c == 0) {
    position[t] = pos;
    drop_mask[t] = dropped ? 1 : 0;
  }
  if (!dropped) Xbuf[((int64_t)e * C + pos) * row_vec16 + c] = x[t * row_vec16 + c];
}

__device__ __forceinline__ uint4 combine_vec_f32(uint4 xv, uint4 yv, float g) {
  float4 a = *reinterpret_cast<float4*>(&xv), b = *reinterpret_cast<float4*>(&yv);
  float4 o = make_float4(fmaf(g, b.x, a.x), fmaf(g, b.y, a.y), fmaf(g, b.z, a.z), fmaf(g, b.w, a.w));
  return *reinterpret_cast<uint4*>(&o);
}

template <bool BF16>
__global__ __launch_bounds__(256) void combine_kernel(const uint4* __restrict__ x, int64_t T,
                                                      int row_vec16,
                                                      const int32_t* __restrict__ expert_idx,
                                                      const int32_t* __restrict__ position,
                                                      const uint8_t* __restrict__ drop_mask,
                                                      const float* __restrict__ gate, int64_t C,
                                                      const uint4* __restrict__ Ybuf,
                                                      uint4* __restrict__ out) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t t = gid / row_vec16;
  const int c = (int)(gid - t * row_vec16);
  if (t >= T) return;
  const uint4 xv = x[t * row_vec16 + c];
  if (drop_mask[t]) {
    out[t * row_vec16 + c] = xv;
    return;
  }
  const float g = gate[t];
  const uint4 yv = Ybuf[((int64_t)expert_idx[t] * C + position[t]) * row_vec16 + c];
  if (BF16) {
    const u32x4 o = combine_vec_bf16(u32x4{xv.x, xv.y, xv.z, xv.w}, u32x4{yv.x, yv.y, yv.z, yv.w}, g);
    out[t * row_vec16 + c] = make_uint4(o.x, o.y, o.z, o.w);
  } else {
    out[t * row_vec16 + c] = combine_vec_f32(xv, yv, g);
  }
}

// Dispatch by index (bf16 path): the expert matmuls read the rows of x in
// place, so dispatch only finalises the routing and records, for every kept
// token, which token sits in slot (e, position): tok[e * C + position] = t.
// A dropped token leaves the layer unchanged: its row of x is copied to out
// here, and the fused combine never touches it.
__global__ __launch_bounds__(256) void dispatch_index_kernel(const uint4* __restrict__ x, int64_t T,
                                                             int row_vec16,
                                                             const int32_t* __restrict__ expert_idx,
                                                             const int32_t* __restrict__ rank_local,
                                                             const int32_t* __restrict__ offsets,
                                                             int N, int64_t chunk, int64_t C,
                                                             int32_t* __restrict__ position,
                                                             uint8_t* __restrict__ drop_mask,
                                                             int32_t* __restrict__ tok,
                                                             uint4* __restrict__ out) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t t = gid / row_vec16;
  const int c = (int)(gid - t * row_vec16);
  if (t >= T) return;
  const int32_t e = expert_idx[t];
  const int32_t pos = offsets[(t / chunk) * N + e] + rank_local[t];
  const bool dropped = (int64_t)pos >= C;
  if (c == 0) {
    position[t] = pos;
    drop_mask[t] = dropped ? 1 : 0;
    if (!dropped) tok[(int64_t)e * C + pos] = (int32_t)t;
  }
  if (dropped) out[t * row_vec16 + c] = x[t * row_vec16 + c];
}

// Copy of the expert outputs for the debug entry point: rows p < n_kept[e].
__global__ __launch_bounds__(256) void copy_expert_rows_kernel(const uint4* __restrict__ Ybuf,
                                                               const int32_t* __restrict__ n_kept,
                                                               int64_t C, int row_vec16,
                                                               uint4* __restrict__ dst) {
  const int e = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int64_t p = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (p >= n_kept[e]) return;
  const int64_t row = (int64_t)e * C + p;
  for (int c = lane; c < row_vec16; c += kWave) dst[row * row_vec16 + c] = Ybuf[row * row_vec16 + c];
}

// ------------------------------------------------------------------ launchers

static unsigned move_blocks(int64_t T, int row_bytes) {
  const int64_t threads = T * (row_bytes / 16);
  return (unsigned)((threads + 255) / 256);
}

void launch_dispatch(const void* x, int64_t T, int row_bytes, const int32_t* expert_idx,
                     const int32_t* rank_local, const int32_t* offsets, int N, int64_t chunk,
                     int64_t C, int32_t* position, uint8_t* drop_mask, void* Xbuf, hipStream_t s) {
  if (T == 0) return;
  hipLaunchKernelGGL(dispatch_kernel, dim3(move_blocks(T, row_bytes)), dim3(256), 0, s, (const uint4*)x, T,
                     row_bytes / 16, expert_idx, rank_local, offsets, N, chunk, C, position,
                     drop_mask, (uint4*)Xbuf);
}

void launch_dispatch_index(const void* x, int64_t T, int row_bytes, const int32_t* expert_idx,
                           const int32_t* rank_local, const int32_t* offsets, int N, int64_t chunk,
                           int64_t C, int32_t* position, uint8_t* drop_mask, int32_t* tok,
                           void* out, hipStream_t s) {
  if (T == 0) return;
  hipLaunchKernelGGL(dispatch_index_kernel, dim3(move_blocks(T, row_bytes)), dim3(256), 0, s,
                     (const uint4*)x, T, row_bytes / 16, expert_idx, rank_local, offsets, N, chunk,
                     C, position, drop_mask, tok, (uint4*)out);
}

void launch_combine(const void* x, bool bf16, int64_t T, int row_bytes, const int32_t* expert_idx,
                    const int32_t* position, const uint8_t* drop_mask, const float* gate,
                    int64_t C, const void* Ybuf, void* out, hipStream_t s) {
  if (T == 0) return;
  if (bf16)
    hipLaunchKernelGGL(combine_kernel<true>, dim3(move_blocks(T, row_bytes)), dim3(256), 0, s,
                       (const uint4*)x, T, row_bytes / 16, expert_idx, position, drop_mask, gate,
                       C, (const uint4*)Ybuf, (uint4*)out);
  else
    hipLaunchKernelGGL(combine_kernel<false>, dim3(move_blocks(T, row_bytes)), dim3(256), 0, s,
                       (const uint4*)x, T, row_bytes / 16, expert_idx, position, drop_mask, gate,
                       C, (const uint4*)Ybuf, (uint4*)out);
}

void launch_copy_expert_rows(const void* Ybuf, const int32_t* n_kept, int N, int64_t C,
                             int row_bytes, void* dst, hipStream_t s) {
  if (C == 0 || N == 0) return;
  hipLaunchKernelGGL(copy_expert_rows_kernel, dim3((unsigned)((C + 3) / 4), (unsigned)N),
                     dim3(256), 0, s, (const uint4*)Ybuf, n_kept, C, row_bytes / 16, (uint4*)dst);
}

}  // namespace swl
