// Router: logits h = x W_r^T + b in fp32, then per-token softmax statistics,
// top-1 choice, gate and the per-block sums of router probabilities.
//
// The router runs in fp32 (kasblo explainer, section "Routerだけfloat32で計算する
// Selective Precision"): bf16 tokens widen exactly, products and sums are fp32.
// Logits h(x) = W_r x and p_i = softmax(h)_i follow the llm-papers-study close
// reading, section 3.1; top-1 and the gate p_{i*} follow its section 3.2.
#include "common.hpp"
#include "kernels.hpp"

namespace swl {

// ---------------------------------------------------------------------------
// h[T, N] = x[T, d] . W_r[N, d]^T + b_r[N]     (fp32 FMA, tiled through LDS)
//
// Block: 256 threads computing a 64-token x 64-expert tile; K in steps of 32.
// Thread (ty, tx) of a 16 x 16 grid owns tokens ty + 16 i and experts tx + 16 j
// (i, j < 4), which keeps LDS reads of one instruction on distinct banks.
// d must be a multiple of 8 (validated by the host).
// ---------------------------------------------------------------------------
constexpr int RT_BT = 64, RT_BE = 64, RT_BK = 32;

template <typename XT>
__device__ __forceinline__ void load8(const XT* p, float* v);
template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float* v) {
  uint4 q = *reinterpret_cast<const uint4*>(p);
  uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float* v) {
  float4 a = *reinterpret_cast<const float4*>(p);
  float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

template <typename XT>
__global__ __launch_bounds__(256) void router_logits_kernel(const XT* __restrict__ x,
                                                            const float* __restrict__ W_r,
                                                            const float* __restrict__ b_r,
                                                            float* __restrict__ h, int64_t T,
                                                            int d, int N) {
  __shared__ float Xs[RT_BK][RT_BT + 4];
  __shared__ float Ws[RT_BK][RT_BE + 4];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int64_t t0 = (int64_t)blockIdx.x * RT_BT;
  const int e0 = blockIdx.y * RT_BE;

  // loader mapping: one 8-wide k chunk of one row per thread (64 rows x 4 chunks)
  const int lrow = tid >> 2, lchunk = (tid & 3) * 8;

  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;

  for (int k0 = 0; k0 < d; k0 += RT_BK) {
    float xv[8], wv[8];
    const int kk = k0 + lchunk;
    const int64_t tr = t0 + lrow;
    if (tr < T && kk < d) load8<XT>(x + tr * d + kk, xv);
    else {
#pragma unroll
      for (int i = 0; i < 8; ++i) xv[i] = 0.f;
    }
    const int er = e0 + lrow;
    if (er < N && kk < d) load8<float>(W_r + (int64_t)er * d + kk, wv);
    else {
#pragma unroll
      for (int i = 0; i < 8; ++i) wv[i] = 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      Xs[lchunk + i][lrow] = xv[i];
      Ws[lchunk + i][lrow] = wv[i];
    }
    __syncthreads();
#pragma unroll 8
    for (int k = 0; k < RT_BK; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = Xs[k][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Ws[k][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t t = t0 + ty + 16 * i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + tx + 16 * j;
      if (e < N) h[t * N + e] = acc[i][j] + (b_r ? b_r[e] : 0.f);
    }
  }
}

// ---------------------------------------------------------------------------
// Routing statistics shared by both router variants.  Tokens are grouped in
// chunks (consecutive tokens, one chunk per routing block); for every chunk c
//   hist[c, e]      tokens of the chunk routed to expert e
//   P_part[c, e]    sum over the chunk's tokens of p_e(t)
//   rank_local[t]   tokens before t in its chunk that chose the same expert
// The final position of t is the exclusive prefix of hist over earlier chunks
// plus rank_local[t] (route_scan_kernel, then finalize in the dispatch pass),
// i.e. the token-order rank; nothing depends on the order threads run in.
// ---------------------------------------------------------------------------

// Rank of every lane's expert among lower lanes with the same expert, and
// whether the lane is the last one holding its expert (e < 0: inactive lane).
__device__ __forceinline__ void wave_rank(int32_t e, int& rank, bool& last) {
  int r = 0, after = 0;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < kWave; ++j) {
    const int32_t ej = __builtin_amdgcn_readlane(e, j);
    const bool same = (ej == e);
    r += (same && j < lane) ? 1 : 0;
    after += (same && j > lane) ? 1 : 0;
  }
  rank = r;
  last = after == 0;
}

// Writes rank_local and the chunk's histogram row from the chunk's experts
// held one per lane (lanes >= n are inactive).  cnt: LDS scratch of N ints;
// the whole block must call this (it synchronises).
__device__ __forceinline__ void chunk_hist_rank(int32_t e, int n, int64_t t, int N, int32_t* cnt,
                                                int32_t* __restrict__ hist_row,
                                                int32_t* __restrict__ rank_local) {
  for (int i = threadIdx.x; i < N; i += blockDim.x) cnt[i] = 0;
  __syncthreads();
  if (threadIdx.x < kWave) {
    const bool active = (int)threadIdx.x < n;
    int rank;
    bool last;
    wave_rank(active ? e : -1, rank, last);
    if (active) {
      rank_local[t] = rank;
      if (last) cnt[e] = rank + 1;
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < N; i += blockDim.x) hist_row[i] = cnt[i];
}

// ---------------------------------------------------------------------------
// Fused router for bf16 tokens and up to 256 experts, one wave per block.
//
// Logits on MFMA with fp32 semantics: x is bf16 (exact), and each fp32 router
// weight is split exactly into three bf16 pieces w = hi + mid + lo (8 + 8 + 8
// significant bits; each piece is the round-to-nearest bf16 of what the
// earlier ones leave).  Every product x * piece is exact in fp32 and the MFMA
// accumulates in fp32, so h is an fp32 dot product of the exact values over 3d
// terms (smallest pieces first).  v_mfma_f32_16x16x32_bf16 layout per lane l:
// A row (token) l % 16 and B column (expert) l % 16 with k = 8 (l / 16) .. +8;
// result rows 4 (l / 16) + i, i < 4, column l % 16.
//
// A block owns 16 * ROWT consecutive tokens (one chunk) and all NPAD >= N
// experts (padded columns get -inf).  After the K loop the wave has whole
// logit rows spread over the 16 lanes of each lane group, so softmax, top-1
// (lowest index on ties), gate = 1 / sum_i exp(h_i - max) and the chunk sums
// of p_i are shuffle reductions; then the chunk histogram and ranks.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint16_t bf16_rne_bits(float f) { return f32_to_bf16_bits(f); }

__device__ __forceinline__ void split3(const float* w, bf16x8& hi, bf16x8& mid, bf16x8& lo) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint16_t h = bf16_rne_bits(w[i]);
    const float r1 = w[i] - bf16_bits_to_f32(h);
    const uint16_t m = bf16_rne_bits(r1);
    const float r2 = r1 - bf16_bits_to_f32(m);
    const uint16_t l = bf16_rne_bits(r2);
    hi[i] = __builtin_bit_cast(__bf16, h);
    mid[i] = __builtin_bit_cast(__bf16, m);
    lo[i] = __builtin_bit_cast(__bf16, l);
  }
}

template <int NPAD, int ROWT>
__global__ __launch_bounds__(256) void router_mfma_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ W_r, const float* __restrict__ b_r,
    int64_t T, int d, int N, float* __restrict__ logits, int32_t* __restrict__ expert_idx,
    float* __restrict__ gate, float* __restrict__ P_part, int32_t* __restrict__ hist,
    int32_t* __restrict__ rank_local) {
  constexpr int NJ = NPAD / 16;
  constexpr int BT = 16 * ROWT;
  constexpr int NACC = ROWT * NJ * 4;  // accumulator floats per lane
  __shared__ int32_t s_idx[BT];
  __shared__ int32_t cnt[NPAD];
  __shared__ float red[3][NACC][kWave];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * BT;
  const int n_tok = (int)((T - t0) < BT ? (T - t0) : BT);
  const int fr = lane & 15, fk = (lane >> 4) * 8;

  floatx4 acc[ROWT][NJ];
#pragma unroll
  for (int r = 0; r < ROWT; ++r)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[r][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  // the four waves take consecutive quarters of K (d is a multiple of 128)
  const int kq = d / 4;
  const int kbeg = wave * kq;
  const uint16_t* xrow[ROWT];
#pragma unroll
  for (int r = 0; r < ROWT; ++r) {
    int64_t t = t0 + 16 * r + fr;
    t = t < T ? t : T - 1;  // rows past T: any valid row, never stored
    xrow[r] = x + t * d + kbeg + fk;
  }
  const float* wrow[NJ];
  bool wvalid[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = 16 * j + fr;
    wvalid[j] = e < N;
    wrow[j] = W_r + (int64_t)(e < N ? e : 0) * d + kbeg + fk;
  }

  // register double buffer: operands of step k + 32 load while step k runs
  bf16x8 a_nx[ROWT];
  float4 w_nx[NJ][2];
  auto load_step = [&](int k) {
#pragma unroll
    for (int r = 0; r < ROWT; ++r) a_nx[r] = *reinterpret_cast<const bf16x8*>(xrow[r] + k);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      w_nx[j][0] = *reinterpret_cast<const float4*>(wrow[j] + k);
      w_nx[j][1] = *reinterpret_cast<const float4*>(wrow[j] + k + 4);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  load_step(0);
  for (int k0 = 0; k0 < kq; k0 += 32) {
    bf16x8 a[ROWT];
    float4 wv[NJ][2];
#pragma unroll
    for (int r = 0; r < ROWT; ++r) a[r] = a_nx[r];
#pragma unroll
    for (int j = 0; j < NJ; ++j) { wv[j][0] = w_nx[j][0]; wv[j][1] = w_nx[j][1]; }
    load_step(k0 + 32 < kq ? k0 + 32 : k0);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      float w[8] = {wv[j][0].x, wv[j][0].y, wv[j][0].z, wv[j][0].w,
                    wv[j][1].x, wv[j][1].y, wv[j][1].z, wv[j][1].w};
      if (!wvalid[j]) {
#pragma unroll
        for (int i = 0; i < 8; ++i) w[i] = 0.f;
      }
      bf16x8 hi, mid, lo;
      split3(w, hi, mid, lo);
#pragma unroll
      for (int r = 0; r < ROWT; ++r) {
        acc[r][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[r], lo, acc[r][j], 0, 0, 0);
        acc[r][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[r], mid, acc[r][j], 0, 0, 0);
        acc[r][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[r], hi, acc[r][j], 0, 0, 0);
      }
    }
  }

  // partial sums of the K quarters meet in wave 0, added in wave order
  if (wave > 0) {
#pragma unroll
    for (int r = 0; r < ROWT; ++r)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wave - 1][(r * NJ + j) * 4 + i][lane] = acc[r][j][i];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int w = 0; w < 3; ++w)
#pragma unroll
      for (int r = 0; r < ROWT; ++r)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[r][j][i] += red[w][(r * NJ + j) * 4 + i][lane];

    // logits (+ bias), padded experts at -inf
    const int g = lane >> 4;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int e = 16 * j + fr;
      const float bias = (e < N && b_r) ? b_r[e] : 0.f;
#pragma unroll
      for (int r = 0; r < ROWT; ++r)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v = acc[r][j][i] + bias;
          acc[r][j][i] = e < N ? v : -__builtin_huge_valf();
          const int64_t t = t0 + 16 * r + 4 * g + i;
          if (logits && e < N && t < T) logits[t * N + e] = v;
        }
    }

    // per token: max with lowest index, sum of exp, gate; chunk sums of p
    float psum[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) psum[j] = 0.f;
#pragma unroll
    for (int r = 0; r < ROWT; ++r) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float m = acc[r][0][i];
        int mi = fr;
#pragma unroll
        for (int j = 1; j < NJ; ++j)
          if (acc[r][j][i] > m) { m = acc[r][j][i]; mi = 16 * j + fr; }
#pragma unroll
        for (int o = 8; o >= 1; o >>= 1) {
          const float om = __shfl_xor(m, o, 16);
          const int oi = __shfl_xor(mi, o, 16);
          if (om > m || (om == m && oi < mi)) { m = om; mi = oi; }
        }
        double ssum = 0.0;
#pragma unroll
        for (int j = 0; j < NJ; ++j) ssum += (double)expf(acc[r][j][i] - m);
#pragma unroll
        for (int o = 8; o >= 1; o >>= 1) ssum += shfl_xor_f64_w(ssum, o, 16);
        const double inv = 1.0 / ssum;
        const int tl = 16 * r + 4 * g + i;
        const int64_t t = t0 + tl;
        if (t < T) {
#pragma unroll
          for (int j = 0; j < NJ; ++j) psum[j] += (float)((double)expf(acc[r][j][i] - m) * inv);
          if (fr == 0) {
            expert_idx[t] = mi;
            gate[t] = (float)inv;
            s_idx[tl] = mi;
          }
        }
      }
    }
    // column sums over the 4 lane groups, then one lane per expert writes
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      psum[j] += __shfl_xor(psum[j], 16, 64);
      psum[j] += __shfl_xor(psum[j], 32, 64);
      const int e = 16 * j + fr;
      if (g == 0 && e < N) P_part[(int64_t)blockIdx.x * N + e] = psum[j];
    }
  }
  __syncthreads();
  const int32_t my_e = (wave == 0 && lane < n_tok) ? s_idx[lane] : -1;
  chunk_hist_rank(my_e, n_tok, t0 + lane, N, cnt, hist + (int64_t)blockIdx.x * N, rank_local);
}

// ---------------------------------------------------------------------------
// Routing statistics from logits in memory (fp32 routers, N > 256, and the
// test entry point that takes logits).  Block: 256 threads, one chunk of 64
// tokens.  Each wave takes 16 tokens: lanes stride over the N logits of a row;
// shuffle reductions give the max with its lowest index and S = sum exp(h - m)
// in fp64; gate = exp(0) / S = 1 / S.  Then every thread owns experts
// i = tid, tid + 256, ... and sums p_i(t) = exp(h_ti - m_t) / S_t over the
// chunk in token order (fp64), and wave 0 ranks the chunk.
// ---------------------------------------------------------------------------
constexpr int RR_ROWS = 64;

__global__ __launch_bounds__(256) void route_rows_kernel(const float* __restrict__ h, int64_t T,
                                                         int N, int32_t* __restrict__ expert_idx,
                                                         float* __restrict__ gate,
                                                         float* __restrict__ P_part,
                                                         int32_t* __restrict__ hist,
                                                         int32_t* __restrict__ rank_local) {
  extern __shared__ int32_t cnt[];
  __shared__ float s_m[RR_ROWS];
  __shared__ double s_inv[RR_ROWS];
  __shared__ int32_t s_idx[RR_ROWS];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * RR_ROWS;
  const int rows = (int)((T - t0) < RR_ROWS ? (T - t0) : RR_ROWS);

  for (int r = wave; r < rows; r += 4) {
    const float* row = h + (t0 + r) * N;
    float m = -__builtin_huge_valf();
    int mi = 0x7fffffff;
    if (lane < N) { m = row[lane]; mi = lane; }
    for (int i = lane + kWave; i < N; i += kWave) {
      float v = row[i];
      if (v > m) { m = v; mi = i; }  // first (lowest) index wins within a lane
    }
    wave_argmax(m, mi);
    double s = 0.0;
    for (int i = lane; i < N; i += kWave) s += (double)expf(row[i] - m);
    s = wave_sum_f64(s);
    if (lane == 0) {
      expert_idx[t0 + r] = mi;
      gate[t0 + r] = (float)(1.0 / s);
      s_m[r] = m;
      s_inv[r] = 1.0 / s;
      s_idx[r] = mi;
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < N; i += blockDim.x) {
    double acc = 0.0;
    for (int r = 0; r < rows; ++r) acc += (double)expf(h[(t0 + r) * N + i] - s_m[r]) * s_inv[r];
    P_part[(int64_t)blockIdx.x * N + i] = (float)acc;
  }
  const int32_t my_e = (wave == 0 && lane < rows) ? s_idx[lane] : -1;
  chunk_hist_rank(my_e, rows, t0 + lane, N, cnt, hist + (int64_t)blockIdx.x * N, rank_local);
}

// ------------------------------------------------------------------ launchers

bool router_fused_ok(bool x_bf16, int N) { return x_bf16 && N <= 256; }

int64_t route_chunk_tokens(bool x_bf16, int N) {
  if (!router_fused_ok(x_bf16, N)) return RR_ROWS;
  return 16;
}

void launch_router_logits(const void* x, bool x_bf16, const float* W_r, const float* b_r,
                          float* h, int64_t T, int d, int N, hipStream_t s) {
  if (T == 0) return;
  dim3 grid((unsigned)((T + RT_BT - 1) / RT_BT), (unsigned)((N + RT_BE - 1) / RT_BE));
  if (x_bf16)
    hipLaunchKernelGGL(router_logits_kernel<uint16_t>, grid, dim3(256), 0, s,
                       (const uint16_t*)x, W_r, b_r, h, T, d, N);
  else
    hipLaunchKernelGGL(router_logits_kernel<float>, grid, dim3(256), 0, s, (const float*)x, W_r,
                       b_r, h, T, d, N);
}

void launch_router_fused(const uint16_t* x, const float* W_r, const float* b_r, int64_t T, int d,
                         int N, float* logits, int32_t* expert_idx, float* gate, float* P_part,
                         int32_t* hist, int32_t* rank_local, hipStream_t s) {
  if (T == 0) return;
  const int64_t ch = route_chunk_tokens(true, N);
  const dim3 grid((unsigned)((T + ch - 1) / ch));
#define SWL_ROUTER(NP, RT)                                                                       \
  hipLaunchKernelGGL((router_mfma_kernel<NP, RT>), grid, dim3(256), 0, s, x, W_r, b_r, T, d, N,  \
                     logits, expert_idx, gate, P_part, hist, rank_local)
  if (N <= 16) SWL_ROUTER(16, 1);
  else if (N <= 32) SWL_ROUTER(32, 1);
  else if (N <= 64) SWL_ROUTER(64, 1);
  else if (N <= 128) SWL_ROUTER(128, 1);
  else SWL_ROUTER(256, 1);
#undef SWL_ROUTER
}

void launch_route_rows(const float* h, int64_t T, int N, int32_t* expert_idx, float* gate,
                       float* P_part, int32_t* hist, int32_t* rank_local, hipStream_t s) {
  if (T == 0) return;
  hipLaunchKernelGGL(route_rows_kernel, dim3((unsigned)((T + RR_ROWS - 1) / RR_ROWS)), dim3(256),
                     sizeof(int32_t) * (size_t)N, s, h, T, N, expert_idx, gate, P_part, hist,
                     rank_local);
}

}  // namespace swl
