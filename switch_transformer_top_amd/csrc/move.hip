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

// row_vec16 = bytes of one row / 16 (rows are a multiple of 16 bytes).

// Row gather of the fp32 path (into Xbuf), one thread per 16-byte piece of a
// row.  Dispatch also finalises the routing: position = chunk offset + in-chunk
// rank, drop = position >= C; kept rows are copied to their expert slot.  With
// k choices per token, assignment a = t * k + j goes to expert_idx[a]; thread
// c < k of a token finalises choice c, and every thread copies its piece of the
// row for each kept choice.
__global__ __launch_bounds__(256) void dispatch_kernel(const uint4* __restrict__ x, int64_t T,
                                                       int k, int row_vec16,
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
  for (int j = 0; j < k; ++j) {
    const int64_t a = t * k + j;
    const int32_t e = expert_idx[a];
    const int32_t pos = offsets[(t / chunk) * N + e] + rank_local[a];
    const bool dropped = (int64_t)pos >= C;
    if (c == j) {
      position[a] = pos;
      drop_mask[a] = dropped ? 1 : 0;
    }
    if (!dropped) Xbuf[((int64_t)e * C + pos) * row_vec16 + c] = x[t * row_vec16 + c];
  }
}

// Lanes per row of the row-wise kernels below: a power of two, at most a wave,
// no more than the row's 16-byte pieces need.
__host__ __device__ constexpr int lanes_per_row(int row_vec16) {
  return row_vec16 >= 64 ? 64 : row_vec16 >= 32 ? 32 : row_vec16 >= 16 ? 16 : row_vec16 >= 8 ? 8
         : row_vec16 >= 4 ? 4 : row_vec16 >= 2 ? 2 : 1;
}

// out[t] = x[t] + sum over kept choices j of gate[t, j] * Y[e_tj, position_tj]:
// fp32 fused multiply-adds in choice order, then one rounding (bf16 layers).
// A token with no kept choice leaves bit for bit.  R = lanes_per_row lanes own
// a row: they read the token's routing once (the same addresses, one request
// per wave) and move its 16-byte pieces c, c + R, ...; rows t, t + rows in
// flight, ... in a grid-stride loop.
template <bool BF16>
__global__ __launch_bounds__(256) void combine_kernel(const uint4* __restrict__ x, int64_t T,
                                                      int k, int row_vec16,
                                                      const int32_t* __restrict__ expert_idx,
                                                      const int32_t* __restrict__ position,
                                                      const uint8_t* __restrict__ drop_mask,
                                                      const float* __restrict__ gate, int64_t C,
                                                      const uint4* __restrict__ Ybuf,
                                                      uint4* __restrict__ out) {
  const int R = lanes_per_row(row_vec16);
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int sub = (int)(gid % R);
  const int64_t stride = (int64_t)gridDim.x * blockDim.x / R;
  constexpr int NV = BF16 ? 8 : 4;   // values per 16-byte piece
  for (int64_t t = gid / R; t < T; t += stride) {
    const uint4* xr = x + t * row_vec16;
    uint4* orow = out + t * row_vec16;
    // the token's kept choices (at most kMaxTopK): gate and source row in Ybuf
    float g[kMaxTopK];
    const uint4* yr[kMaxTopK];
    int nk = 0;
    for (int j = 0; j < k; ++j) {
      const int64_t a = t * k + j;
      if (drop_mask[a]) continue;
      g[nk] = gate[a];
      yr[nk] = Ybuf + ((int64_t)expert_idx[a] * C + position[a]) * row_vec16;
      ++nk;
    }
    for (int c = sub; c < row_vec16; c += R) {
      const uint4 xv = xr[c];
      if (nk == 0) {
        orow[c] = xv;
        continue;
      }
      float acc[NV];
      const uint32_t xs[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (BF16) {
          acc[2 * i] = __uint_as_float(xs[i] << 16);
          acc[2 * i + 1] = __uint_as_float(xs[i] & 0xFFFF0000u);
        } else {
          acc[i] = __uint_as_float(xs[i]);
        }
      }
      for (int j = 0; j < nk; ++j) {
        const uint4 yv = yr[j][c];
        const uint32_t ys[4] = {yv.x, yv.y, yv.z, yv.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (BF16) {
            acc[2 * i] = fmaf(g[j], __uint_as_float(ys[i] << 16), acc[2 * i]);
            acc[2 * i + 1] = fmaf(g[j], __uint_as_float(ys[i] & 0xFFFF0000u), acc[2 * i + 1]);
          } else {
            acc[i] = fmaf(g[j], __uint_as_float(ys[i]), acc[i]);
          }
        }
      }
      uint32_t o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        o[i] = BF16 ? f32x2_to_bf16x2_bits(acc[2 * i], acc[2 * i + 1]) : __float_as_uint(acc[i]);
      orow[c] = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
}

// Dispatch by index (bf16 path): the expert matmuls read the rows of x in
// place, so dispatch only finalises the routing and records, for every kept
// assignment, which token sits in slot (e, position): tok[e * C + position] = t.
// A block of four waves takes 64 assignments: in wave 0 lane i derives
// assignment 64 b + i (position = chunk offset + in-chunk rank, drop =
// position >= C) and stores the results.  With the fused combine (k = 1) a
// dropped token leaves the layer unchanged: wave 0 leaves the block's drop
// mask in LDS, and the r-th dropped row of the 64 is copied from x to out by
// wave r % 4, in 16-byte pieces spread over the lanes; the combine never
// touches it.  (Every wave deriving the mask itself took four times the
// gathers of chunk offsets.)
__global__ __launch_bounds__(256) void dispatch_index_kernel(const uint4* __restrict__ x, int64_t T,
                                                             int k, int row_vec16,
                                                             const int32_t* __restrict__ expert_idx,
                                                             const int32_t* __restrict__ rank_local,
                                                             const int32_t* __restrict__ offsets,
                                                             int N, int64_t chunk, int64_t C,
                                                             int32_t* __restrict__ position,
                                                             uint8_t* __restrict__ drop_mask,
                                                             int32_t* __restrict__ tok,
                                                             bool copy_dropped,
                                                             uint4* __restrict__ out) {
  __shared__ uint64_t s_drops;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t a0 = (int64_t)blockIdx.x * kWave;
  const int64_t a = a0 + lane;
  if (w > 0 && !copy_dropped) return;   // uniform: only wave 0 has work then
  if (w == 0) {
    bool dropped = false;
    if (a < T * k) {
      const int64_t t = a / k;
      const int32_t e = expert_idx[a];
      const int32_t pos = offsets[(t / chunk) * N + e] + rank_local[a];
      dropped = (int64_t)pos >= C;
      position[a] = pos;
      drop_mask[a] = dropped ? 1 : 0;
      if (!dropped) tok[(int64_t)e * C + pos] = (int32_t)t;
    }
    const uint64_t m0 = __ballot(dropped);
    if (lane == 0) s_drops = m0;
  }
  if (!copy_dropped) return;   // uniform; k = 1 from here on: assignment a is token a
  __syncthreads();
  uint64_t m = s_drops;
  for (int r = 0; m; ++r) {
    const int64_t t = a0 + __builtin_ctzll(m);
    m &= m - 1;
    if ((r & 3) != w) continue;
    const uint4* src = x + t * row_vec16;
    uint4* dst = out + t * row_vec16;
#pragma unroll 4
    for (int c = lane; c < row_vec16; c += kWave) dst[c] = src[c];
  }
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

void launch_dispatch(const void* x, int64_t T, int k, int row_bytes, const int32_t* expert_idx,
                     const int32_t* rank_local, const int32_t* offsets, int N, int64_t chunk,
                     int64_t C, int32_t* position, uint8_t* drop_mask, void* Xbuf, hipStream_t s) {
  if (T == 0) return;
  launch_k(dispatch_kernel, dim3(move_blocks(T, row_bytes)), dim3(256), 0, s,
                     (const uint4*)x, T, k, row_bytes / 16, expert_idx, rank_local, offsets, N,
                     chunk, C, position, drop_mask, (uint4*)Xbuf);
}

void launch_dispatch_index(const void* x, int64_t T, int k, int row_bytes,
                           const int32_t* expert_idx, const int32_t* rank_local,
                           const int32_t* offsets, int N, int64_t chunk, int64_t C,
                           int32_t* position, uint8_t* drop_mask, int32_t* tok, bool copy_dropped,
                           void* out, hipStream_t s) {
  if (T == 0) return;
  const int64_t groups = (T * k + kWave - 1) / kWave;   // 64 assignments per block
  launch_k(dispatch_index_kernel, dim3((unsigned)groups), dim3(256), 0, s,
                     (const uint4*)x, T, k, row_bytes / 16, expert_idx, rank_local, offsets, N,
                     chunk, C, position, drop_mask, tok, copy_dropped && k == 1, (uint4*)out);
}

void launch_combine(const void* x, bool bf16, int64_t T, int k, int row_bytes,
                    const int32_t* expert_idx, const int32_t* position, const uint8_t* drop_mask,
                    const float* gate, int64_t C, const void* Ybuf, void* out, hipStream_t s) {
  if (T == 0) return;
  // one row per R lanes, up to 8 rows per 256-thread block in each pass; the
  // grid-stride loop takes the rest (about 16 blocks per compute unit)
  const int64_t R = lanes_per_row(row_bytes / 16);
  const int64_t want = (T * R + 255) / 256;
  const unsigned grid = (unsigned)(want < 4096 ? want : 4096);
  if (bf16)
    launch_k(combine_kernel<true>, dim3(grid), dim3(256), 0, s,
                       (const uint4*)x, T, k, row_bytes / 16, expert_idx, position, drop_mask,
                       gate, C, (const uint4*)Ybuf, (uint4*)out);
  else
    launch_k(combine_kernel<false>, dim3(grid), dim3(256), 0, s,
                       (const uint4*)x, T, k, row_bytes / 16, expert_idx, position, drop_mask,
                       gate, C, (const uint4*)Ybuf, (uint4*)out);
}

void launch_copy_expert_rows(const void* Ybuf, const int32_t* n_kept, int N, int64_t C,
                             int row_bytes, void* dst, hipStream_t s) {
  if (C == 0 || N == 0) return;
  launch_k(copy_expert_rows_kernel, dim3((unsigned)((C + 3) / 4), (unsigned)N),
                     dim3(256), 0, s, (const uint4*)Ybuf, n_kept, C, row_bytes / 16, (uint4*)dst);
}

}  // namespace swl
