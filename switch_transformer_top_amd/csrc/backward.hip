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

// Slot table and scaled output gradient of every kept assignment (t, j):
// tok[e * C + p] = t and Gs[e, p, :] = bf16(gate_tj * G_t) (fp32 product,
// rounded to nearest even).  One thread per 16-byte piece of a row.  The last
// block instead writes n_kept[e] = min(load[e], C) (the forward's per-expert
// loads) and the compact list of tile_rows-row tiles over them.
__global__ __launch_bounds__(256) void bwd_slots_kernel(const u32x4* __restrict__ G, int64_t T,
                                                        int topk, int row_vec16,
                                                        const int32_t* __restrict__ expert_idx,
                                                        const int32_t* __restrict__ position,
                                                        const uint8_t* __restrict__ drop_mask,
                                                        const float* __restrict__ gate, int64_t C,
                                                        int32_t* __restrict__ tok,
                                                        u32x4* __restrict__ Gs,
                                                        const int32_t* __restrict__ load, int N,
                                                        int32_t* __restrict__ n_kept,
                                                        int32_t* __restrict__ tile_start,
                                                        int tile_rows) {
  if (blockIdx.x == gridDim.x - 1) {
    __shared__ int32_t s_run[256];
    for (int e = threadIdx.x; e < N; e += blockDim.x)
      n_kept[e] = (int32_t)((int64_t)load[e] < C ? (int64_t)load[e] : C);
    __syncthreads();
    if (tile_start) tile_prefix_block(n_kept, N, tile_rows, tile_start, s_run);
    return;
  }
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
                                                         const uint16_t* __restrict__ Yfwd,
                                                         const int32_t* __restrict__ yflag,
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
  // Y from the forward's buffer when that call kept it, else as recomputed
  const uint16_t* __restrict__ Y = (yflag && *yflag != 0) ? Yfwd : Ybuf;
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
          reinterpret_cast<const u32x4*>(Y + ((int64_t)ej[j] * C + position[a]) * d);
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

// dW_r[i, k] = sum_t dh[t, i] x[t, k] and db[i] = sum_t dh[t, i], for more
// than 32 experts, on bf16 MFMA (v_mfma_f32_32x32x16_bf16, fp32 accumulation):
// each dh value is split into three bf16 planes, hi = bf16(v), mid =
// bf16(v - hi), lo = bf16(v - hi - mid), which hold its 24 significant bits (the
// forward router splits W_r the same way), and x is exact in bf16, so
// dW_r = sum over the planes of plane^T x.  Both operands are token-major (the
// contraction runs over tokens): they are staged in LDS as stored, [32
// tokens][128 + KO_PAD], and read with the transposing fragment read.  Block
// (128-column tile, 128-expert tile, token slice s): four waves of 64 experts x
// 64 columns (2 x 2 MFMA tiles); the slice in steps of 32 tokens, one LDS
// buffer, the next step's loads in registers while the current one is
// multiplied.  db sums the fp32 dh values, each thread over its row group's
// tokens, then the eight groups in order.  Each slice writes its
// partial sums to part[s] ([N, d]; part_b[s] [N] from the column-tile-0
// blocks); wgrad_reduce_block adds the slices in slice order (the dx kernel's
// last blocks, or router_wgrad_reduce when there are no tokens).
constexpr int RW_TOK = 32, RW_PITCH = 128 + KO_PAD;

// dh rows t0 .. t0 + 32 of experts i0 .. i0 + 128 (thread: column quad tid % 32,
// tokens tid / 32 + 8 u) and x rows (16-byte pieces tid + 256 u)
__device__ __forceinline__ void rw_load(const float* __restrict__ dh,
                                        const uint16_t* __restrict__ x, int64_t ts, int64_t te,
                                        int N, int d, int i0, int k0, bool vec4,
                                        float4 (&dv)[4], u32x4 (&xv)[2]) {
  const int tid = threadIdx.x, c = i0 + 4 * (tid & 31);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t t = ts + (tid >> 5) + 8 * u;
    const float* row = dh + t * N + c;
    if (t >= te) {
      dv[u] = make_float4(0.f, 0.f, 0.f, 0.f);
    } else if (vec4 && c + 3 < N) {
      dv[u] = *reinterpret_cast<const float4*>(row);
    } else {
      dv[u] = make_float4(c < N ? row[0] : 0.f, c + 1 < N ? row[1] : 0.f,
                          c + 2 < N ? row[2] : 0.f, c + 3 < N ? row[3] : 0.f);
    }
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int idx = threadIdx.x + 256 * u, r = idx >> 4, cc = (idx & 15) * 8;
    const int64_t t = ts + r;
    xv[u] = t < te ? *reinterpret_cast<const u32x4*>(x + t * d + k0 + cc)
                   : u32x4{0u, 0u, 0u, 0u};
  }
}

__device__ __forceinline__ void rw_store(uint16_t (*Ps)[RW_TOK * RW_PITCH], uint16_t* Xs,
                                         const float4 (&dv)[4], const u32x4 (&xv)[2]) {
  const int tid = threadIdx.x, c = 4 * (tid & 31);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int r = (tid >> 5) + 8 * u;
    const float w[4] = {dv[u].x, dv[u].y, dv[u].z, dv[u].w};
    uint16_t hb[4], mb[4], lb[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      hb[q] = f32_to_bf16_bits(w[q]);
      const float r1 = w[q] - bf16_bits_to_f32(hb[q]);
      mb[q] = f32_to_bf16_bits(r1);
      lb[q] = f32_to_bf16_bits(r1 - bf16_bits_to_f32(mb[q]));
    }
    const int off = r * RW_PITCH + c;
    *reinterpret_cast<uint2*>(&Ps[0][off]) =
        make_uint2(hb[0] | ((uint32_t)hb[1] << 16), hb[2] | ((uint32_t)hb[3] << 16));
    *reinterpret_cast<uint2*>(&Ps[1][off]) =
        make_uint2(mb[0] | ((uint32_t)mb[1] << 16), mb[2] | ((uint32_t)mb[3] << 16));
    *reinterpret_cast<uint2*>(&Ps[2][off]) =
        make_uint2(lb[0] | ((uint32_t)lb[1] << 16), lb[2] | ((uint32_t)lb[3] << 16));
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int idx = tid + 256 * u;
    *reinterpret_cast<u32x4*>(&Xs[(idx >> 4) * RW_PITCH + (idx & 15) * 8]) = xv[u];
  }
}

__global__ __launch_bounds__(256, 2) void router_wgrad_kernel(const float* __restrict__ dh,
                                                              const uint16_t* __restrict__ x,
                                                              int64_t T, int N, int d,
                                                              int64_t slice,
                                                              float* __restrict__ part,
                                                              float* __restrict__ part_b) {
  __shared__ __attribute__((aligned(16))) uint16_t Ps[3][RW_TOK * RW_PITCH];
  __shared__ __attribute__((aligned(16))) uint16_t Xs[RW_TOK * RW_PITCH];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1, col = lane & 31, kh = lane >> 5;
  const int k0 = blockIdx.x * 128, i0 = blockIdx.y * 128;
  const int64_t ts = (int64_t)blockIdx.z * slice;
  const int64_t te = ts + slice < T ? ts + slice : T;
  const int steps = (int)((te - ts + RW_TOK - 1) / RW_TOK);
  const bool bias = blockIdx.x == 0;
  const bool vec4 = (N & 3) == 0;

  floatx16 acc[2][2];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[m][n][v] = 0.f;
  // db: this thread's column quad over its row group's tokens (see the end)
  float4 bacc = make_float4(0.f, 0.f, 0.f, 0.f);

  float4 dv[4];
  u32x4 xv[2];
  rw_load(dh, x, ts, te, N, d, i0, k0, vec4, dv, xv);
  for (int st = 0; st < steps; ++st) {
    if (st > 0) __syncthreads();  // the previous step's fragments are read
    rw_store(Ps, Xs, dv, xv);
    if (bias) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        bacc.x += dv[u].x;
        bacc.y += dv[u].y;
        bacc.z += dv[u].z;
        bacc.w += dv[u].w;
      }
    }
    __syncthreads();
    if (st + 1 < steps)
      rw_load(dh, x, ts + (int64_t)(st + 1) * RW_TOK, te, N, d, i0, k0, vec4, dv, xv);
#pragma unroll
    for (int ks = 0; ks < RW_TOK / 16; ++ks) {
      bf16x8 a[2][3], b[2];
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int p = 0; p < 3; ++p) a[m][p] = frag_kouter(Ps[p], RW_PITCH, ks, 64 * wm + 32 * m, lane);
#pragma unroll
      for (int n = 0; n < 2; ++n) b[n] = frag_kouter(Xs, RW_PITCH, ks, 64 * wn + 32 * n, lane);
#pragma unroll
      for (int p = 2; p >= 0; --p)  // small planes first
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int n = 0; n < 2; ++n)
            acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[m][p], b[n], acc[m][n], 0, 0, 0);
    }
  }
  // acc[m][n][v]: expert i0 + 64 wm + 32 m + 8 (v / 4) + 4 kh + v % 4,
  // column k0 + 64 wn + 32 n + col
  float* ps = part + (int64_t)blockIdx.z * N * d;
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int i = i0 + 64 * wm + 32 * m + 8 * (v >> 2) + 4 * kh + (v & 3);
      if (i < N) {
#pragma unroll
        for (int n = 0; n < 2; ++n) ps[(int64_t)i * d + k0 + 64 * wn + 32 * n + col] = acc[m][n][v];
      }
    }
  if (bias) {
    // thread (g, q) = (tid / 32, tid % 32) summed columns 4 q .. 4 q + 3 over the
    // tokens 32 st + g + 8 u; the eight row groups are added in group order
    __shared__ float s_g[8][128];
    const int q = tid & 31, g = tid >> 5;
    s_g[g][4 * q] = bacc.x;
    s_g[g][4 * q + 1] = bacc.y;
    s_g[g][4 * q + 2] = bacc.z;
    s_g[g][4 * q + 3] = bacc.w;
    __syncthreads();
    if (tid < 128 && i0 + tid < N) {
      float v = 0.f;
#pragma unroll
      for (int gg = 0; gg < 8; ++gg) v += s_g[gg][tid];
      part_b[(int64_t)blockIdx.z * N + i0 + tid] = v;
    }
  }
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

// dW_r = sum over slices of part[s]; db likewise (when db != NULL).  Block
// number blk (256 threads) takes the 64 consecutive outputs from 64 blk; its
// four waves add every fourth slice (wave w: slices w, w + 4, ...) in slice
// order, and the four partial sums are added in wave order.  Fixed order
// throughout.  Runs as its own kernel (no tokens) or as the last blocks of the
// dx kernel.
struct WgradSums {
  const float* part;
  const float* part_b;
  int slices;
  float* dW_r;
  float* db;
};

__device__ __forceinline__ void wgrad_reduce_block(const WgradSums& ws, int N, int d,
                                                   int64_t blk) {
  __shared__ float red[4][64];
  const float* __restrict__ part = ws.part;
  const float* __restrict__ part_b = ws.part_b;
  const int slices = ws.slices;
  float* __restrict__ dW_r = ws.dW_r;
  float* __restrict__ db = ws.db;
  const int64_t n = (int64_t)N * d;
  const int o = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t i = blk * 64 + o;
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

__global__ __launch_bounds__(256) void router_wgrad_reduce(WgradSums ws, int N, int d) {
  wgrad_reduce_block(ws, N, d, blockIdx.x);
}

// dx_t = G_t + sum over kept choices j of dX[e_tj, p_tj] + sum_i dh[t, i] W_r[i, :],
// fp32 then one rounding to bf16.  Block: 64 tokens x 128 columns.  The router
// part D[k][t] = sum_i W_r[i][k] dh[t][i] runs on bf16 MFMA
// (v_mfma_f32_32x32x16_bf16, fp32 accumulation) with both operands split into
// two bf16 planes, v = hi + mid + r, |r| <= 2^-16 |v|, as
// hi(W) hi(dh) + hi(W) mid(dh) + mid(W) hi(dh), which leaves out mid * mid and
// the rests: at most 3.1 * 2^-16 of sum_i |W_r[i][k] dh[t][i]|, far below the
// final bf16 rounding of dx (unit roundoff 2^-8).
// Steps of 32 experts (two 16-deep sub-steps; experts past N read as 0): the W_r
// planes staged as stored, [32 experts][128 + KO_PAD] (read with the transposing
// fragment read), the dh planes as [64 tokens][32 + 8] (experts innermost, read
// directly); one LDS buffer, the next step's loads in registers.  Wave w owns
// columns 64 (w & 1) .. +64 (two 32-column MFMA tiles) and tokens
// 32 (w >> 1) .. +32.  The sums go through LDS as a [64][128] fp32 tile, and G,
// the dX rows and dx move in 16-byte row pieces (thread: pieces tid + 256 u,
// token tid / 16 + 16 u).  The block rows past the token tiles add the dW_r
// slices (wgrad_reduce_block) instead.
constexpr int GX_TOK = 64, GX_EXP = 32, GX_WP = 128 + KO_PAD, GX_DP = GX_EXP + 8,
              GX_YLD = 132;

// W_r rows i0 .. i0 + 32, columns k0 .. k0 + 128 (thread: float4 pieces tid + 256 u)
// and dh experts i0 .. i0 + 32 of tokens t0 .. t0 + 64 (thread: token tid / 4,
// experts 8 (tid % 4) .. +7)
__device__ __forceinline__ void gx_load(const float* __restrict__ dh,
                                        const float* __restrict__ W_r, int64_t T, int N, int d,
                                        int64_t t0, int k0, int i0, bool vec4, float4 (&wv)[4],
                                        float (&dv)[8]) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int idx = tid + 256 * u, r = idx >> 5, c = (idx & 31) * 4;
    wv[u] = i0 + r < N ? *reinterpret_cast<const float4*>(W_r + (int64_t)(i0 + r) * d + k0 + c)
                       : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  const int64_t t = t0 + (tid >> 2);
  const int c = i0 + 8 * (tid & 3);
  const float* row = dh + t * N + c;
  if (t < T && vec4 && c + 7 < N) {
    const float4 a = *reinterpret_cast<const float4*>(row);
    const float4 b = *reinterpret_cast<const float4*>(row + 4);
    dv[0] = a.x; dv[1] = a.y; dv[2] = a.z; dv[3] = a.w;
    dv[4] = b.x; dv[5] = b.y; dv[6] = b.z; dv[7] = b.w;
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) dv[j] = (t < T && c + j < N) ? row[j] : 0.f;
  }
}

// hi = bf16(v), mid = bf16(v - hi)
__device__ __forceinline__ void split2(float v, uint16_t& hi, uint16_t& mid) {
  hi = f32_to_bf16_bits(v);
  mid = f32_to_bf16_bits(v - bf16_bits_to_f32(hi));
}

__device__ __forceinline__ void gx_store(uint16_t (*Wp)[GX_EXP * GX_WP],
                                         uint16_t (*Dp)[GX_TOK * GX_DP], const float4 (&wv)[4],
                                         const float (&dv)[8]) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int idx = tid + 256 * u, r = idx >> 5, c = (idx & 31) * 4;
    const float w[4] = {wv[u].x, wv[u].y, wv[u].z, wv[u].w};
    uint16_t h[4], m[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) split2(w[q], h[q], m[q]);
    *reinterpret_cast<uint2*>(&Wp[0][r * GX_WP + c]) =
        make_uint2(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16));
    *reinterpret_cast<uint2*>(&Wp[1][r * GX_WP + c]) =
        make_uint2(m[0] | ((uint32_t)m[1] << 16), m[2] | ((uint32_t)m[3] << 16));
  }
  uint16_t h[8], m[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) split2(dv[j], h[j], m[j]);
  const int off = (tid >> 2) * GX_DP + 8 * (tid & 3);
  *reinterpret_cast<u32x4*>(&Dp[0][off]) =
      u32x4{h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16),
            h[4] | ((uint32_t)h[5] << 16), h[6] | ((uint32_t)h[7] << 16)};
  *reinterpret_cast<u32x4*>(&Dp[1][off]) =
      u32x4{m[0] | ((uint32_t)m[1] << 16), m[2] | ((uint32_t)m[3] << 16),
            m[4] | ((uint32_t)m[5] << 16), m[6] | ((uint32_t)m[7] << 16)};
}

__global__ __launch_bounds__(256) void grad_x_kernel(const uint16_t* __restrict__ G, int64_t T,
                                                     int d, int topk,
                                                     const int32_t* __restrict__ expert_idx,
                                                     const int32_t* __restrict__ position,
                                                     const uint8_t* __restrict__ drop_mask,
                                                     int64_t C, const uint16_t* __restrict__ dXe,
                                                     const float* __restrict__ dh,
                                                     const float* __restrict__ W_r, int N,
                                                     uint16_t* __restrict__ dx, int tok_tiles,
                                                     WgradSums wsum) {
  if ((int)blockIdx.y >= tok_tiles) {  // the blocks past the token tiles add the dW_r slices
    wgrad_reduce_block(wsum, N, d, (int64_t)(blockIdx.y - tok_tiles) * gridDim.x + blockIdx.x);
    return;
  }
  // the operand planes during the products, then the [64][GX_YLD] fp32 sum tile
  constexpr int PLANES = (2 * GX_EXP * GX_WP + 2 * GX_TOK * GX_DP) * 2, SUMS = GX_TOK * GX_YLD * 4;
  __shared__ __attribute__((aligned(16))) unsigned char raw[PLANES > SUMS ? PLANES : SUMS];
  typedef uint16_t WArr[GX_EXP * GX_WP];
  typedef uint16_t DArr[GX_TOK * GX_DP];
  WArr* Wp = reinterpret_cast<WArr*>(raw);
  DArr* Dp = reinterpret_cast<DArr*>(raw + 2 * GX_EXP * GX_WP * 2);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1, col = lane & 31, kh = lane >> 5;
  const int64_t t0 = (int64_t)blockIdx.y * GX_TOK;
  const int k0 = blockIdx.x * 128;
  const int pc = k0 + 8 * (tid & 15);  // the thread's piece columns
  const bool vec4 = (N & 3) == 0;

  floatx16 acc[2];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[m][v] = 0.f;
  const int steps = (N + GX_EXP - 1) / GX_EXP;
  float4 wv[4];
  float dv[8];
  gx_load(dh, W_r, T, N, d, t0, k0, 0, vec4, wv, dv);
  for (int st = 0; st < steps; ++st) {
    const int i0 = st * GX_EXP;
    if (st > 0) __syncthreads();  // the previous step's fragments are read
    gx_store(Wp, Dp, wv, dv);
    __syncthreads();
    if (st + 1 < steps) gx_load(dh, W_r, T, N, d, t0, k0, i0 + GX_EXP, vec4, wv, dv);
    const int left = N - i0 < GX_EXP ? N - i0 : GX_EXP;
    const int nsub = (left + 15) >> 4;  // 16-deep sub-steps holding experts
    for (int ks = 0; ks < nsub; ++ks) {
      bf16x8 a[2][2], b[2];
#pragma unroll
      for (int p = 0; p < 2; ++p) {
#pragma unroll
        for (int m = 0; m < 2; ++m) a[p][m] = frag_kouter(Wp[p], GX_WP, ks, 64 * wm + 32 * m, lane);
        b[p] = *reinterpret_cast<const bf16x8*>(&Dp[p][(32 * wn + col) * GX_DP + 16 * ks + 8 * kh]);
      }
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1][m], b[0], acc[m], 0, 0, 0);
        acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0][m], b[1], acc[m], 0, 0, 0);
        acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0][m], b[0], acc[m], 0, 0, 0);
      }
    }
  }
  __syncthreads();  // the planes are read: the sum tile takes their place
  // G and the kept choices' dX rows of the thread's pieces
  u32x4 gin[4];
  u32x4 xin[kMaxTopK][4];
  bool kept[kMaxTopK][4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t t = t0 + (tid >> 4) + 16 * u;
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) kept[j][u] = false;
    if (t >= T) continue;
    gin[u] = *reinterpret_cast<const u32x4*>(G + t * d + pc);
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      if (j >= topk) break;
      const int64_t a = t * topk + j;
      kept[j][u] = drop_mask[a] == 0;
      if (kept[j][u])
        xin[j][u] = *reinterpret_cast<const u32x4*>(
            dXe + ((int64_t)expert_idx[a] * C + position[a]) * d + pc);
    }
  }

  // acc[m][4 b + q]: column 64 wm + 32 m + 8 b + 4 kh + q of token 32 wn + col
  float (*Ys)[GX_YLD] = reinterpret_cast<float (*)[GX_YLD]>(raw);
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int b = 0; b < 4; ++b)
      *reinterpret_cast<float4*>(&Ys[32 * wn + col][64 * wm + 32 * m + 8 * b + 4 * kh]) =
          make_float4(acc[m][4 * b], acc[m][4 * b + 1], acc[m][4 * b + 2], acc[m][4 * b + 3]);
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int r = (tid >> 4) + 16 * u;
    const int64_t t = t0 + r;
    if (t >= T) continue;
    const u32x4 gv = gin[u];
    float v[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(gv[i] << 16);
      v[2 * i + 1] = __uint_as_float(gv[i] & 0xFFFF0000u);
    }
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {  // the kept choices' expert parts, in choice order
      if (!kept[j][u]) continue;
      const u32x4 xv = xin[j][u];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] += __uint_as_float(xv[i] << 16);
        v[2 * i + 1] += __uint_as_float(xv[i] & 0xFFFF0000u);
      }
    }
    const float4 s0 = *reinterpret_cast<const float4*>(&Ys[r][8 * (tid & 15)]);
    const float4 s1 = *reinterpret_cast<const float4*>(&Ys[r][8 * (tid & 15) + 4]);
    const u32x4 o = {f32x2_to_bf16x2_bits(v[0] + s0.x, v[1] + s0.y),
                     f32x2_to_bf16x2_bits(v[2] + s0.z, v[3] + s0.w),
                     f32x2_to_bf16x2_bits(v[4] + s1.x, v[5] + s1.y),
                     f32x2_to_bf16x2_bits(v[6] + s1.z, v[7] + s1.w)};
    *reinterpret_cast<u32x4*>(dx + t * d + pc) = o;
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

void launch_bwd_slots(const void* G, int64_t T, int d, int k, const int32_t* expert_idx,
                      const int32_t* position, const uint8_t* drop_mask, const float* gate,
                      int64_t C, int32_t* tok, void* Gs, const int32_t* load, int N,
                      int32_t* n_kept, int32_t* tile_start, hipStream_t s) {
  const int rv = d / 8;
  // the slot blocks, then the block for n_kept and the tile list
  const int64_t nb = (T * k * rv + 255) / 256 + 1;
  launch_k(bwd_slots_kernel, dim3((unsigned)nb), dim3(256), 0, s, (const u32x4*)G, T, k, rv,
           expert_idx, position, drop_mask, gate, C, tok, (u32x4*)Gs, load, N, n_kept,
           tile_start, kWideTileRows);
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
                       const void* Ybuf, const void* Yfwd, const int32_t* yflag, int64_t C,
                       const int32_t* expert_idx,
                       const int32_t* position, const uint8_t* drop_mask, const int32_t* load,
                       float loss_scale, float* dh, hipStream_t s) {
  if (T == 0) return;
  launch_k(router_bwd_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, h, T, N,
                     d, k, (const uint16_t*)G, (const uint16_t*)Ybuf,
                     (const uint16_t*)Yfwd, yflag, C, expert_idx, position,
                     drop_mask, load, loss_scale, dh);
}

// Tokens per slice of the few-expert kernel: at least RS_TOK, and at most 256
// slices in all (bounds the partial sums at 256 N d floats).
static int64_t small_slice(int64_t T) {
  int64_t sl = (T + 255) / 256;
  sl = (sl + RS_TOK - 1) / RS_TOK * RS_TOK;
  return sl < RS_TOK ? RS_TOK : sl;
}

// Tokens per slice of the MFMA kernel: about 512 blocks over the
// (128-column, 128-expert) tiles, slices of whole 32-token steps.
static int64_t mfma_slice(int64_t T, int N, int d) {
  const int64_t tiles = (int64_t)((d + 127) / 128) * ((N + 127) / 128);
  const int64_t most = (T + RW_TOK - 1) / RW_TOK;
  int64_t want = (512 + tiles - 1) / tiles;
  want = want < most ? want : most;
  const int64_t sl = (T + want - 1) / want;
  return (sl + RW_TOK - 1) / RW_TOK * RW_TOK;
}

int64_t router_wgrad_slices(int64_t T, int N, int d) {
  if (T <= 0) return 0;
  const int64_t sl = N <= 32 ? small_slice(T) : mfma_slice(T, N, d);
  return (T + sl - 1) / sl;
}

void launch_router_wgrad(const float* dh, const void* x, int64_t T, int N, int d, float* part,
                         float* part_b, float* dW_r, float* db, bool reduce, hipStream_t s) {
  const int64_t slices = router_wgrad_slices(T, N, d);
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
    // d is a multiple of 128 (bf16 layers): whole column tiles
    const dim3 grid((unsigned)(d / 128), (unsigned)((N + 127) / 128), (unsigned)slices);
    launch_k(router_wgrad_kernel, grid, dim3(256), 0, s, dh, (const uint16_t*)x, T, N,
                       d, mfma_slice(T, N, d), part, part_b);
  }
  if (!reduce) return;  // the dx kernel's last blocks add the slices
  const int64_t n = (int64_t)N * d + N;
  launch_k(router_wgrad_reduce, dim3((unsigned)((n + 63) / 64)), dim3(256), 0, s,
           WgradSums{part, part_b, (int)slices, dW_r, db}, N, d);
}

void launch_grad_x(const void* G, int64_t T, int d, int k, const int32_t* expert_idx,
                   const int32_t* position, const uint8_t* drop_mask, int64_t C, const void* dXe,
                   const float* dh, const float* W_r, int N, void* dx, const float* part,
                   const float* part_b, float* dW_r, float* db, hipStream_t s) {
  if (T == 0) return;
  // d is a multiple of 128 (bf16 layers): whole column tiles; then enough rows of
  // blocks for the router weight-gradient sums (64 outputs each)
  const int64_t tok_tiles = (T + GX_TOK - 1) / GX_TOK;
  const int64_t n = (int64_t)N * d + N, sum_blocks = (n + 63) / 64;
  const int64_t sum_rows = (sum_blocks + d / 128 - 1) / (d / 128);
  const dim3 grid((unsigned)(d / 128), (unsigned)(tok_tiles + sum_rows));
  const WgradSums ws{part, part_b, (int)router_wgrad_slices(T, N, d), dW_r, db};
  launch_k(grad_x_kernel, grid, dim3(256), 0, s, (const uint16_t*)G, T, d, k, expert_idx,
           position, drop_mask, C, (const uint16_t*)dXe, dh, W_r, N, (uint16_t*)dx,
           (int)tok_tiles, ws);
}

}  // namespace swl
