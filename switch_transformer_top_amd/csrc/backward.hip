// Backward pass of the top-1 Switch layer: the kernels around the grouped
// matmuls.
//
// The expert choice and the capacity cut are piecewise constant and carry no
// gradient; the gradient reaches the router through the continuous gate
// p_{i*}(x) that scales the chosen expert's output (kasblo explainer, section
// "argmaxは離散なのに、Routerはなぜ学習できるのか"), and through P_i of the
// load-balancing loss, f_i being a count (llm-papers-study close reading,
// section 3.3).  With G = dL/dout and g_aux = dL/daux:
//   kept t (expert e, slot p, gate g):  Gs[e, p] = g G_t,
//     dU = (Gs W_out[e]) * [H > 0],  dX[e, p] = dU W_in[e],
//     dW_out[e] = Gs^T H,  dW_in[e] = dU^T X  (sums over the expert's rows),
//     dg_t = G_t . Y[e, p];
//   every t:  dp_i = [i = e_t, kept] dg_t + g_aux alpha N load_i / T^2,
//     dh = p * (dp - p . dp),  dW_r = dh^T x,  db = sum_t dh,
//     dx_t = G_t + dX[e_t, p_t] + W_r^T dh_t.
// The matmuls are the grouped bf16 kernels of gemm.hip (fp32 accumulation),
// which read the weights and the per-slot activations as stored; this file
// holds the slot/scale pass, the gather of the token rows with K (the expert's
// rows) innermost for dW_in, the router backward and the assembly of dx.
#include "common.hpp"
#include "kernels.hpp"

namespace swl {

// n_kept[e] = min(load[e], C) (the forward's per-expert loads), and the
// compact list of tile_rows-row tiles over them (one block).
__global__ __launch_bounds__(1024) void bwd_rows_kernel(const int32_t* __restrict__ load, int N,
                                                        int64_t C, int32_t* __restrict__ n_kept,
                                                        int32_t* __restrict__ tile_start,
                                                        int tile_rows) {
  __shared__ int32_t s_run[1024];
  for (int e = threadIdx.x; e < N; e += blockDim.x)
    n_kept[e] = (int32_t)((int64_t)load[e] < C ? (int64_t)load[e] : C);
  __syncthreads();
  if (tile_start) tile_prefix_block(n_kept, N, tile_rows, tile_start, s_run);
}

// Slot table and scaled output gradient of every kept assignment (t, j):
// tok[e * C + p] = t and Gs[e, p, :] = bf16(gate_tj * G_t) (fp32 product,
// rounded to nearest even).  One thread per 16-byte piece of a row.
__global__ __launch_bounds__(256) void bwd_slots_kernel(const u32x4* __restrict__ G, int64_t T,
                                                        int topk, int row_vec16,
                                                        const int32_t* __restrict__ expert_idx,
                                                        const int32_t* __restrict__ position,
                                                        const uint8_t* __restrict__ drop_mask,
                                                        const float* __restrict__ gate, int64_t C,
                                                        int32_t* __restrict__ tok,
                                                        u32x4* __restrict__ Gs) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t a = gid / row_vec16;  // assignment (token t, choice j): a = t topk + j
  const int c = (int)(gid - a * row_vec16);
  if (a >= T * topk || drop_mask[a]) return;
  const int64_t t = a / topk;
  const int64_t slot = (int64_t)expert_idx[a] * C + position[a];
  if (c == 0) tok[slot] = (int32_t)t;
  const float g = gate[a];
  const u32x4 v = G[t * row_vec16 + c];
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = f32x2_to_bf16x2_bits(g * __uint_as_float(v[i] << 16),
                                g * __uint_as_float(v[i] & 0xFFFF0000u));
  Gs[slot * row_vec16 + c] = o;
}

// Per-expert transpose of a bf16 matrix block src[e] [R, Ccols] (row stride
// ld) into dst[e] [Ccols, Rpad]: dst[c][r] = src[r][c] for r < rows_e, 0 for
// rows_e <= r < Rpad.  rows_e = valid[e], or R when valid is NULL.  With tok,
// row r of expert e is row tok[e * R + r] of src (a gathered row of x).
// 64 x 64 tiles through LDS (rows of 72 bf16); every global access moves 16
// bytes: a thread loads 8 consecutive columns of a source row and stores 8
// consecutive rows of a destination row.  Ccols, ld and Rpad are multiples of
// 8 (Rpad of 64); grid (ceil(Ccols / 64), Rpad / 64, N).
__global__ __launch_bounds__(256) void transpose_kernel(const uint16_t* __restrict__ src,
                                                        int64_t src_estride, int ld, int R,
                                                        int Ccols,
                                                        const int32_t* __restrict__ valid,
                                                        const int32_t* __restrict__ tok,
                                                        uint16_t* __restrict__ dst,
                                                        int64_t dst_estride, int Rpad) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[64][72];
  const int e = blockIdx.z;
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
  const int rows_e = valid ? valid[e] : R;
  const uint16_t* se = src + (tok ? 0 : (int64_t)e * src_estride);
  const int32_t* te = tok ? tok + (int64_t)e * R : nullptr;
  const int lr = threadIdx.x >> 3, lc = (threadIdx.x & 7) * 8;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int i = lr + 32 * j;
    const int r = r0 + i, c = c0 + lc;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r < rows_e && c < Ccols) {
      const int64_t row = te ? (int64_t)te[r] : (int64_t)r;
      v = *reinterpret_cast<const u32x4*>(se + row * ld + c);
    }
    *reinterpret_cast<u32x4*>(&tile[i][lc]) = v;
  }
  __syncthreads();
  uint16_t* de = dst + (int64_t)e * dst_estride;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int cc = lr + 32 * j;          // destination row (source column)
    const int c = c0 + cc, r = r0 + lc;
    if (c >= Ccols) continue;
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      o[q] = (uint32_t)tile[lc + 2 * q][cc] | ((uint32_t)tile[lc + 2 * q + 1][cc] << 16);
    *reinterpret_cast<u32x4*>(de + (int64_t)c * Rpad + r) = o;
  }
}

// Router backward, one wave per token: dg_j = G_t . Y[e_j, p_j] for each kept
// choice j, p = softmax(h_t) (fp32 exponentials, fp64 sums as in the forward),
// dp, and dh_t = p * (dp - p . dp) written to dh [T, N] (fp32).
__global__ __launch_bounds__(256) void router_bwd_kernel(const float* __restrict__ h, int64_t T,
                                                         int N, int d, int topk,
                                                         const uint16_t* __restrict__ G,
                                                         const uint16_t* __restrict__ Ybuf,
                                                         int64_t C,
                                                         const int32_t* __restrict__ expert_idx,
                                                         const int32_t* __restrict__ position,
                                                         const uint8_t* __restrict__ drop_mask,
                                                         const int32_t* __restrict__ load,
                                                         float loss_scale,
                                                         float* __restrict__ dh) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int ej[kMaxTopK];
  bool kj[kMaxTopK];
  double dg[kMaxTopK];
  // dg_j = <G[t], Y[e_j, position]> in fp64 over 16-byte pieces (d is a
  // multiple of 128, so rows are whole pieces); bf16 products are exact
  const u32x4* gt = reinterpret_cast<const u32x4*>(G + t * d);
  const int nv = d / 8;
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    const int64_t a = t * topk + j;
    ej[j] = j < topk ? expert_idx[a] : -1;
    kj[j] = j < topk && drop_mask[a] == 0;
    dg[j] = 0.0;
    if (kj[j]) {
      const u32x4* yt =
          reinterpret_cast<const u32x4*>(Ybuf + ((int64_t)ej[j] * C + position[a]) * d);
      double acc = 0.0;
      for (int q = lane; q < nv; q += kWave) {
        const u32x4 gv = gt[q], yv = yt[q];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc += (double)__uint_as_float(gv[i] << 16) * (double)__uint_as_float(yv[i] << 16);
          acc += (double)__uint_as_float(gv[i] & 0xFFFF0000u) *
                 (double)__uint_as_float(yv[i] & 0xFFFF0000u);
        }
      }
      dg[j] = wave_sum_f64(acc);
    }
  }
  const float* ht = h + t * N;
  float m = -__builtin_huge_valf();
  for (int i = lane; i < N; i += kWave) m = fmaxf(m, ht[i]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
  double S = 0.0;
  for (int i = lane; i < N; i += kWave) S += (double)expf(ht[i] - m);
  S = wave_sum_f64(S);
  const double inv = 1.0 / S;
  // dp_i = sum_j [i = e_j, kept] dg_j + loss_scale * load_i,
  // loss_scale = g_aux alpha N / (k T^2)
  auto dp_of = [&](int i) {
    double dp = (double)loss_scale * (double)load[i];
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j)
      if (kj[j] && i == ej[j]) dp += dg[j];
    return dp;
  };
  double pdp = 0.0;
  for (int i = lane; i < N; i += kWave) pdp += (double)expf(ht[i] - m) * inv * dp_of(i);
  pdp = wave_sum_f64(pdp);
  for (int i = lane; i < N; i += kWave) {
    const double p = (double)expf(ht[i] - m) * inv;
    dh[t * N + i] = (float)(p * (dp_of(i) - pdp));
  }
}

// dW_r[i, k] = sum_t dh[t, i] x[t, k] and db[i] = sum_t dh[t, i] (fp32).
// Block (k tile, i tile, s): 64 experts x 64 columns over the tokens of slice
// s (RW_SLICE consecutive tokens), 256 threads each 4 x 4 outputs, the slice
// in steps of 32 tokens through LDS.  Each slice writes its partial sums to
// part[s] ([N, d], and part_b[s] [N] from the k-tile-0 blocks);
// router_wgrad_reduce adds the slices in slice order.  Fixed order throughout.
constexpr int RW_SLICE = 256;

__global__ __launch_bounds__(256) void router_wgrad_kernel(const float* __restrict__ dh,
                                                           const uint16_t* __restrict__ x,
                                                           int64_t T, int N, int d,
                                                           float* __restrict__ part,
                                                           float* __restrict__ part_b) {
  __shared__ float Ds[32][68];
  __shared__ float Xs[32][68];
  const int i0 = blockIdx.y * 64, k0 = blockIdx.x * 64;
  const int64_t ts = (int64_t)blockIdx.z * RW_SLICE;
  const int64_t te = ts + RW_SLICE < T ? ts + RW_SLICE : T;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float acc[4][4] = {};
  float bacc = 0.f;
  for (int64_t t0 = ts; t0 < te; t0 += 32) {
    for (int idx = threadIdx.x; idx < 32 * 64; idx += 256) {
      const int r = idx >> 6, c = idx & 63;
      const int64_t t = t0 + r;
      Ds[r][c] = (t < te && i0 + c < N) ? dh[t * N + i0 + c] : 0.f;
      Xs[r][c] = (t < te && k0 + c < d) ? bf16_bits_to_f32(x[t * d + k0 + c]) : 0.f;
    }
    __syncthreads();
#pragma unroll 4
    for (int r = 0; r < 32; ++r) {
      float a[4], b[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) { a[q] = Ds[r][ty + 16 * q]; b[q] = Xs[r][tx + 16 * q]; }
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int w = 0; w < 4; ++w) acc[q][w] = fmaf(a[q], b[w], acc[q][w]);
      if (blockIdx.x == 0 && threadIdx.x < 64) bacc += Ds[r][threadIdx.x];
    }
    __syncthreads();
  }
  float* ps = part + (int64_t)blockIdx.z * N * d;
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int i = i0 + ty + 16 * q, k = k0 + tx + 16 * w;
      if (i < N && k < d) ps[(int64_t)i * d + k] = acc[q][w];
    }
  if (blockIdx.x == 0 && threadIdx.x < 64 && i0 + threadIdx.x < N)
    part_b[(int64_t)blockIdx.z * N + i0 + threadIdx.x] = bacc;
}

// Few experts (N <= 32): one wave per (256-column block, token slice); lane l
// owns columns 4 l .. 4 l + 3 of the block and every expert, so one 8-byte
// load of x feeds 4 NP fused multiply-adds.  The slice's dh rows pass through
// LDS in steps of RS_TOK tokens and are read back as broadcasts.  Partial sums
// go to part[s] like the general kernel's; the reduction is the same.
constexpr int RS_TOK = 32;

template <int NP>
__global__ __launch_bounds__(64) void router_wgrad_small_kernel(const float* __restrict__ dh,
                                                               const uint16_t* __restrict__ x,
                                                               int64_t T, int N, int d,
                                                               int64_t slice,
                                                               float* __restrict__ part,
                                                               float* __restrict__ part_b) {
  __shared__ __attribute__((aligned(16))) float Dh[RS_TOK * NP];
  const int lane = threadIdx.x;
  const int c0 = blockIdx.x * 256 + lane * 4;
  const bool has_cols = c0 < d;
  const int64_t ts = (int64_t)blockIdx.y * slice;
  const int64_t te = ts + slice < T ? ts + slice : T;
  float acc[NP][4];
#pragma unroll
  for (int i = 0; i < NP; ++i)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[i][c] = 0.f;
  float bacc = 0.f;
  for (int64_t t0 = ts; t0 < te; t0 += RS_TOK) {
    const int nt = (int)(te - t0 < RS_TOK ? te - t0 : RS_TOK);
    for (int idx = lane; idx < RS_TOK * NP; idx += kWave) {
      const int r = idx / NP, i = idx - r * NP;
      Dh[idx] = (r < nt && i < N) ? dh[(t0 + r) * N + i] : 0.f;
    }
    __syncthreads();
    // rows of x eight at a time, all eight in flight at once (rows past the
    // slice read as 0)
#pragma unroll 1
    for (int rb = 0; rb < RS_TOK; rb += 8) {
      uint2 xr[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        xr[u] = (has_cols && rb + u < nt)
                    ? *reinterpret_cast<const uint2*>(x + (t0 + rb + u) * d + c0)
                    : make_uint2(0u, 0u);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int r = rb + u;
        const uint2 v = xr[u];
        const float xv[4] = {__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xFFFF0000u),
                             __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xFFFF0000u)};
#pragma unroll
        for (int i4 = 0; i4 < NP / 4; ++i4) {
          const float4 w = *reinterpret_cast<const float4*>(&Dh[r * NP + 4 * i4]);
          const float wv[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[4 * i4 + q][c] = fmaf(wv[q], xv[c], acc[4 * i4 + q][c]);
        }
        if (blockIdx.x == 0 && lane < N && r < nt) bacc += Dh[r * NP + lane];
      }
    }
    __syncthreads();
  }
  float* ps = part + (int64_t)blockIdx.y * N * d;
  if (has_cols) {
#pragma unroll
    for (int i = 0; i < NP; ++i)
      if (i < N)
        *reinterpret_cast<float4*>(ps + (int64_t)i * d + c0) =
            make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
  }
  if (blockIdx.x == 0 && lane < N) part_b[(int64_t)blockIdx.y * N + lane] = bacc;
}

// dW_r = sum over slices of part[s]; db likewise (when db != NULL).  A block
// takes 64 consecutive outputs; its four waves add every fourth slice (wave w:
// slices w, w + 4, ...) in slice order, and the four partial sums are added in
// wave order.  Fixed order throughout.
__global__ __launch_bounds__(256) void router_wgrad_reduce(const float* __restrict__ part,
                                                           const float* __restrict__ part_b,
                                                           int slices, int N, int d,
                                                           float* __restrict__ dW_r,
                                                           float* __restrict__ db) {
  __shared__ float red[4][64];
  const int64_t n = (int64_t)N * d;
  const int o = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t i = (int64_t)blockIdx.x * 64 + o;
  float acc = 0.f;
  if (i < n) {
#pragma unroll 8
    for (int sl = w; sl < slices; sl += 4) acc += part[(int64_t)sl * n + i];
  } else if (i < n + N && db) {
    const int64_t j = i - n;
#pragma unroll 8
    for (int sl = w; sl < slices; sl += 4) acc += part_b[(int64_t)sl * N + j];
  }
  red[w][o] = acc;
  __syncthreads();
  if (w == 0) {
    const float v = ((red[0][o] + red[1][o]) + red[2][o]) + red[3][o];
    if (i < n) dW_r[i] = v;
    else if (i < n + N && db) db[i - n] = v;
  }
}

// dx_t = G_t + sum over kept choices j of dX[e_tj, p_tj] + sum_i dh[t, i] W_r[i, :],
// fp32 then one rounding to bf16.  Block: 64 tokens x 64 columns; the router part is a
// small matmul with K = N, in steps of 32 experts through LDS; thread (ty, tx)
// owns tokens ty + 16 q and the four columns 4 tx .. 4 tx + 3.
__global__ __launch_bounds__(256) void grad_x_kernel(const uint16_t* __restrict__ G, int64_t T,
                                                     int d, int topk,
                                                     const int32_t* __restrict__ expert_idx,
                                                     const int32_t* __restrict__ position,
                                                     const uint8_t* __restrict__ drop_mask,
                                                     int64_t C, const uint16_t* __restrict__ dXe,
                                                     const float* __restrict__ dh,
                                                     const float* __restrict__ W_r, int N,
                                                     uint16_t* __restrict__ dx) {
  __shared__ float Ds[64][33];
  __shared__ float Ws[32][68];
  const int64_t t0 = (int64_t)blockIdx.y * 64;
  const int k0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float acc[4][4] = {};
  for (int i0 = 0; i0 < N; i0 += 32) {
    for (int idx = threadIdx.x; idx < 64 * 32; idx += 256) {
      const int r = idx >> 5, c = idx & 31;
      const int64_t t = t0 + r;
      Ds[r][c] = (t < T && i0 + c < N) ? dh[t * N + i0 + c] : 0.f;
    }
    for (int idx = threadIdx.x; idx < 32 * 64; idx += 256) {
      const int r = idx >> 6, c = idx & 63;
      Ws[r][c] = (i0 + r < N && k0 + c < d) ? W_r[(int64_t)(i0 + r) * d + k0 + c] : 0.f;
    }
    __syncthreads();
#pragma unroll 4
    for (int i = 0; i < 32; ++i) {
      float w[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) w[c] = Ws[i][4 * tx + c];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float a = Ds[ty + 16 * q][i];
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[q][c] = fmaf(a, w[c], acc[q][c]);
      }
    }
    __syncthreads();
  }
  const int k = k0 + 4 * tx;
  if (k >= d) return;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t t = t0 + ty + 16 * q;
    if (t >= T) continue;
    const uint2 gv = *reinterpret_cast<const uint2*>(G + t * d + k);
    float v[4] = {__uint_as_float(gv.x << 16), __uint_as_float(gv.x & 0xFFFF0000u),
                  __uint_as_float(gv.y << 16), __uint_as_float(gv.y & 0xFFFF0000u)};
    for (int j = 0; j < topk; ++j) {  // the kept choices' expert parts, in choice order
      const int64_t a = t * topk + j;
      if (drop_mask[a]) continue;
      const uint2 xv = *reinterpret_cast<const uint2*>(
          dXe + ((int64_t)expert_idx[a] * C + position[a]) * d + k);
      v[0] += __uint_as_float(xv.x << 16);
      v[1] += __uint_as_float(xv.x & 0xFFFF0000u);
      v[2] += __uint_as_float(xv.y << 16);
      v[3] += __uint_as_float(xv.y & 0xFFFF0000u);
    }
    const uint2 o = make_uint2(f32x2_to_bf16x2_bits(v[0] + acc[q][0], v[1] + acc[q][1]),
                               f32x2_to_bf16x2_bits(v[2] + acc[q][2], v[3] + acc[q][3]));
    *reinterpret_cast<uint2*>(dx + t * d + k) = o;
  }
}

// Zero fill (16-byte stores; bytes a multiple of 16).
__global__ __launch_bounds__(256) void fill_zero_kernel(u32x4* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = u32x4{0u, 0u, 0u, 0u};
}

// ------------------------------------------------------------------ launchers

void launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
  const int64_t n = (int64_t)(bytes / 16);
  if (n == 0) return;
  const int64_t blocks = (n + 255) / 256;
  launch_k(fill_zero_kernel, dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(256),
                     0, s, (u32x4*)p, n);
}

void launch_bwd_rows(const int32_t* load, int N, int64_t C, int32_t* n_kept,
                     int32_t* tile_start, hipStream_t s) {
  launch_k(bwd_rows_kernel, dim3(1), dim3(1024), 0, s, load, N, C, n_kept, tile_start,
                     kWideTileRows);
}

void launch_bwd_slots(const void* G, int64_t T, int d, int k, const int32_t* expert_idx,
                      const int32_t* position, const uint8_t* drop_mask, const float* gate,
                      int64_t C, int32_t* tok, void* Gs, hipStream_t s) {
  if (T == 0) return;
  const int rv = d / 8;
  launch_k(bwd_slots_kernel, dim3((unsigned)((T * k * rv + 255) / 256)), dim3(256), 0,
                     s, (const u32x4*)G, T, k, rv, expert_idx, position, drop_mask, gate, C, tok,
                     (u32x4*)Gs);
}

void launch_transpose(const void* src, int64_t src_estride, int ld, int R, int Ccols,
                      const int32_t* valid, const int32_t* tok, void* dst, int64_t dst_estride,
                      int Rpad, int n_experts, hipStream_t s) {
  if (Ccols == 0 || Rpad == 0 || n_experts == 0) return;
  const dim3 grid((unsigned)((Ccols + 63) / 64), (unsigned)(Rpad / 64), (unsigned)n_experts);
  launch_k(transpose_kernel, grid, dim3(256), 0, s, (const uint16_t*)src, src_estride,
                     ld, R, Ccols, valid, tok, (uint16_t*)dst, dst_estride, Rpad);
}

void launch_router_bwd(const float* h, int64_t T, int N, int d, int k, const void* G,
                       const void* Ybuf, int64_t C, const int32_t* expert_idx,
                       const int32_t* position, const uint8_t* drop_mask, const int32_t* load,
                       float loss_scale, float* dh, hipStream_t s) {
  if (T == 0) return;
  launch_k(router_bwd_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, h, T, N,
                     d, k, (const uint16_t*)G, (const uint16_t*)Ybuf, C, expert_idx, position,
                     drop_mask, load, loss_scale, dh);
}

// Tokens per slice of the few-expert kernel: at least RS_TOK, and at most 256
// slices in all (bounds the partial sums at 256 N d floats).
static int64_t small_slice(int64_t T) {
  int64_t sl = (T + 255) / 256;
  sl = (sl + RS_TOK - 1) / RS_TOK * RS_TOK;
  return sl < RS_TOK ? RS_TOK : sl;
}

int64_t router_wgrad_slices(int64_t T, int N) {
  if (T <= 0) return 0;
  if (N <= 32) return (T + small_slice(T) - 1) / small_slice(T);
  return (T + RW_SLICE - 1) / RW_SLICE;
}

void launch_router_wgrad(const float* dh, const void* x, int64_t T, int N, int d, float* part,
                         float* part_b, float* dW_r, float* db, hipStream_t s) {
  const int64_t slices = router_wgrad_slices(T, N);
  if (slices > 0 && N <= 32) {
    const dim3 grid((unsigned)((d + 255) / 256), (unsigned)slices);
    const int64_t sl = small_slice(T);
    if (N <= 8)
      launch_k(router_wgrad_small_kernel<8>, grid, dim3(64), 0, s, dh,
                         (const uint16_t*)x, T, N, d, sl, part, part_b);
    else if (N <= 16)
      launch_k(router_wgrad_small_kernel<16>, grid, dim3(64), 0, s, dh,
                         (const uint16_t*)x, T, N, d, sl, part, part_b);
    else
      launch_k(router_wgrad_small_kernel<32>, grid, dim3(64), 0, s, dh,
                         (const uint16_t*)x, T, N, d, sl, part, part_b);
  } else if (slices > 0) {
    const dim3 grid((unsigned)((d + 63) / 64), (unsigned)((N + 63) / 64), (unsigned)slices);
    launch_k(router_wgrad_kernel, grid, dim3(256), 0, s, dh, (const uint16_t*)x, T, N,
                       d, part, part_b);
  }
  const int64_t n = (int64_t)N * d + N;
  launch_k(router_wgrad_reduce, dim3((unsigned)((n + 63) / 64)), dim3(256), 0, s, part,
                     part_b, (int)slices, N, d, dW_r, db);
}

void launch_grad_x(const void* G, int64_t T, int d, int k, const int32_t* expert_idx,
                   const int32_t* position, const uint8_t* drop_mask, int64_t C, const void* dXe,
                   const float* dh, const float* W_r, int N, void* dx, hipStream_t s) {
  if (T == 0) return;
  const dim3 grid((unsigned)((d + 63) / 64), (unsigned)((T + 63) / 64));
  launch_k(grad_x_kernel, grid, dim3(256), 0, s, (const uint16_t*)G, T, d, k,
                     expert_idx, position, drop_mask, C, (const uint16_t*)dXe, dh, W_r, N,
                     (uint16_t*)dx);
}

}  // namespace swl
