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
// Routing statistics shared by the router variants.  Tokens are grouped in
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

// Ranks and histogram of one chunk from its experts s_idx[0..n) (LDS), one
// entry per assignment in (token, choice) order starting at assignment a0 of
// the call (a0 = t0 * k).  Wave 0 walks the chunk 64 assignments at a time; cnt (LDS, N ints) holds the running
// count per expert, which ends as the chunk's histogram.  The whole block must
// call this (it synchronises).
__device__ __forceinline__ void chunk_hist_rank(const int32_t* s_idx, int n, int64_t a0, int N,
                                                int32_t* cnt, int32_t* __restrict__ hist_row,
                                                int32_t* __restrict__ rank_local) {
  for (int i = threadIdx.x; i < N; i += blockDim.x) cnt[i] = 0;
  __syncthreads();
  if (threadIdx.x < kWave) {
    for (int base = 0; base < n; base += kWave) {
      const int i = base + (int)threadIdx.x;
      const bool active = i < n;
      const int32_t e = active ? s_idx[i] : -1;
      int rank;
      bool last;
      wave_rank(e, rank, last);
      if (active) {
        const int32_t r = cnt[e] + rank;  // every lane reads before any lane writes
        rank_local[a0 + i] = r;
        if (last) cnt[e] = r + 1;
      }
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < N; i += blockDim.x) hist_row[i] = cnt[i];
}

// The three-piece split of the routers below (w = hi + mid + lo, each piece the
// round-to-nearest bf16 of what the earlier ones leave) for a pair of weights,
// with the packed conversion (two values per v_cvt_pk_bf16_f32): the pieces as
// packed bf16 pairs (first value in the low half)
__device__ __forceinline__ void split3x2(float a, float b, uint32_t& hi, uint32_t& mid,
                                         uint32_t& lo) {
  hi = f32x2_to_bf16x2_bits(a, b);
  const float ra = a - __uint_as_float(hi << 16), rb = b - __uint_as_float(hi & 0xFFFF0000u);
  mid = f32x2_to_bf16x2_bits(ra, rb);
  const float qa = ra - __uint_as_float(mid << 16), qb = rb - __uint_as_float(mid & 0xFFFF0000u);
  lo = f32x2_to_bf16x2_bits(qa, qb);
}

// ---------------------------------------------------------------------------
// bf16 routers on MFMA with fp32 semantics.  x is bf16 (exact), and each fp32
// router weight is split exactly into three bf16 pieces w = hi + mid + lo
// (8 + 8 + 8 significant bits; each piece is the round-to-nearest bf16 of what
// the earlier ones leave).  Every product x * piece is exact in fp32 and the
// MFMA accumulates in fp32, so h is an fp32 dot product of the exact values
// over 3d terms (smallest pieces first).  v_mfma_f32_16x16x32_bf16 layout per
// lane l: A row (token) l % 16 and B column (expert) l % 16 with k = 8 (l / 16)
// .. +8; result rows 4 (l / 16) + i, i < 4, column l % 16.
//
// After the K loop a wave holds whole logit rows spread over the 16 lanes of
// each lane group, so softmax, top-1 (lowest index on ties), gate = 1 / sum_i
// exp(h_i - max) and the sums of p_i over the wave's tokens are shuffle
// reductions (row_stats below).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void split3(const float* w, bf16x8& hi, bf16x8& mid, bf16x8& lo) {
  uint32_t h4[4], m4[4], l4[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) split3x2(w[2 * i], w[2 * i + 1], h4[i], m4[i], l4[i]);
  hi = __builtin_bit_cast(bf16x8, u32x4{h4[0], h4[1], h4[2], h4[3]});
  mid = __builtin_bit_cast(bf16x8, u32x4{m4[0], m4[1], m4[2], m4[3]});
  lo = __builtin_bit_cast(bf16x8, u32x4{l4[0], l4[1], l4[2], l4[3]});
}

// Routing statistics of a block's logit tile st[BT][LD] (LDS, fp32, bias
// added, padded experts at -inf), tokens t0 .. t0 + n_tok.  A few consecutive
// threads share a token row (TPR = blockDim / BT): max with the lowest index,
// S = sum_i exp(h_i - max) (fp64), gate = 1 / S; with k = 2 also the best of
// the other experts (lowest index on ties) and its probability
// exp(h - max) / S.  Choices go to expert_idx / gate [t * k + j] and s_idx
// [row * k + j].  Then thread e owns expert e and sums p_e over the chunk's
// tokens in token order (fp64) for P_part (with at most 128 experts two
// threads share an expert, each summing half of the tokens in order, and the
// halves are added first + second); the logits leave in full coalesced rows
// when requested.  Synchronises the block.
//
// With s_term (LDS, BT x NPAD doubles) each thread also stores its terms
// exp(h_e - max) * (1 / S) there, so the P_part sums read them back instead of
// evaluating the exponentials again (the same values, added in the same order).
template <int BT, int NPAD, int LD>
__device__ __forceinline__ void block_stats(const float* st, int N, int k, int64_t t0, int n_tok,
                                            float* __restrict__ logits,
                                            int32_t* __restrict__ expert_idx,
                                            float* __restrict__ gate,
                                            float* __restrict__ P_row, int32_t* s_idx,
                                            float* s_m, double* s_inv,
                                            double* s_term = nullptr) {
  constexpr int TPR = 256 / BT;          // threads per token row
  constexpr int SPAN = NPAD / TPR;       // experts per thread
  static_assert(TPR >= 1 && TPR <= 16 && SPAN >= 1, "row split");
  const int tid = threadIdx.x;
  const int row = tid / TPR, part = tid % TPR;
  const float* rp = st + row * LD + part * SPAN;
  float m = rp[0];
  int mi = part * SPAN;
#pragma unroll 8
  for (int i = 1; i < SPAN; ++i)
    if (rp[i] > m) { m = rp[i]; mi = part * SPAN + i; }
#pragma unroll
  for (int o = TPR / 2; o >= 1; o >>= 1) {
    const float om = __shfl_xor(m, o, TPR);
    const int oi = __shfl_xor(mi, o, TPR);
    if (om > m || (om == m && oi < mi)) { m = om; mi = oi; }
  }
  double ssum = 0.0;
#pragma unroll 8
  for (int i = 0; i < SPAN; ++i) ssum += (double)expf(rp[i] - m);
#pragma unroll
  for (int o = TPR / 2; o >= 1; o >>= 1) ssum += shfl_xor_f64_w(ssum, o, TPR);
  if (s_term) {
    // every thread of the row holds the same sum after the butterfly
    const double rinv = 1.0 / ssum;
#pragma unroll 8
    for (int i = 0; i < SPAN; ++i)
      s_term[row * NPAD + part * SPAN + i] = (double)expf(rp[i] - m) * rinv;
  }
  // second choice: the largest logit among the other experts (real ones only)
  float m2 = -__builtin_huge_valf();
  int mi2 = 0x7fffffff;
  if (k > 1) {
#pragma unroll 8
    for (int i = 0; i < SPAN; ++i) {
      const int e = part * SPAN + i;
      if (e != mi && e < N && (rp[i] > m2 || mi2 == 0x7fffffff)) { m2 = rp[i]; mi2 = e; }
    }
#pragma unroll
    for (int o = TPR / 2; o >= 1; o >>= 1) {
      const float om = __shfl_xor(m2, o, TPR);
      const int oi = __shfl_xor(mi2, o, TPR);
      if (oi != 0x7fffffff && (mi2 == 0x7fffffff || om > m2 || (om == m2 && oi < mi2))) {
        m2 = om;
        mi2 = oi;
      }
    }
  }
  if (part == 0 && row < n_tok) {
    const double inv = 1.0 / ssum;
    s_m[row] = m;
    s_inv[row] = inv;
    s_idx[row * k] = mi;
    expert_idx[(t0 + row) * k] = mi;
    gate[(t0 + row) * k] = (float)inv;
    if (k > 1) {
      s_idx[row * k + 1] = mi2;
      expert_idx[(t0 + row) * k + 1] = mi2;
      gate[(t0 + row) * k + 1] = (float)((double)expf(m2 - m) * inv);
    }
  }
  if (logits) {
    for (int idx = tid; idx < n_tok * N; idx += 256) {
      const int r = idx / N, e = idx - r * N;
      logits[(t0 + r) * N + e] = st[r * LD + e];
    }
  }
  __syncthreads();
  if (!s_term && 2 * N <= 256) {
    // two adjacent threads per expert, each over half of the rows in token
    // order; the halves are added first + second
    const int e = tid >> 1, g = tid & 1;
    const int half = (n_tok + 1) >> 1;
    const int r0 = g ? half : 0, r1 = g ? n_tok : half;
    double acc = 0.0;
    if (e < N) {
#pragma unroll 4
      for (int r = r0; r < r1; ++r) acc += (double)expf(st[r * LD + e] - s_m[r]) * s_inv[r];
    }
    const double other = shfl_xor_f64_w(acc, 1, 2);
    if (e < N && g == 0) P_row[e] = (float)(acc + other);
    return;
  }
  for (int e = tid; e < N; e += 256) {
    double acc = 0.0;
    if (s_term) {
      for (int r = 0; r < n_tok; ++r) acc += s_term[r * NPAD + e];
    } else {
#pragma unroll 4
      for (int r = 0; r < n_tok; ++r) acc += (double)expf(st[r * LD + e] - s_m[r]) * s_inv[r];
    }
    P_row[e] = (float)acc;
  }
}

// Ranks and histogram of a chunk of at most 64 assignments over at most 64
// experts, by one wave (threads 64..127 of the block, so that it runs beside
// wave 0's P_part sums): for each expert a ballot of the lanes holding it;
// a lane's rank is the number of set bits below it (mbcnt), the histogram
// entry the population count.  Same results as chunk_hist_rank.
__device__ __forceinline__ void chunk_hist_rank_wave(const int32_t* s_idx, int n, int64_t a0,
                                                     int N, int32_t* __restrict__ hist_row,
                                                     int32_t* __restrict__ rank_local) {
  const int lane = threadIdx.x & 63;
  const int32_t e = lane < n ? s_idx[lane] : -1;
  for (int i = 0; i < N; ++i) {
    const uint64_t m = __ballot(e == i);
    if (e == i)
      rank_local[a0 + lane] = (int32_t)__builtin_amdgcn_mbcnt_hi(
          (uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    if (lane == 0) hist_row[i] = (int32_t)__popcll(m);
  }
}

// Few experts (N <= 32): a block owns 16 tokens (one chunk) and its four waves
// take consecutive quarters of K, with every K step of the quarter loaded up
// front (8 at a time) so the loads' latency is paid once.  The partial sums of
// the quarters meet in wave 0, added in wave order.
template <int NPAD>
__global__ __launch_bounds__(256) void router_small_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ W_r, const float* __restrict__ b_r,
    int64_t T, int d, int N, int k, float* __restrict__ logits, int32_t* __restrict__ expert_idx,
    float* __restrict__ gate, float* __restrict__ P_part, int32_t* __restrict__ hist,
    int32_t* __restrict__ rank_local) {
  constexpr int NJ = NPAD / 16, BT = 16, NACC = NJ * 4, GRP = 8, LD = NPAD + 4;
  __shared__ int32_t s_idx[BT * kMaxTopK];
  __shared__ double s_term[BT * NPAD];
  __shared__ float red[3][NACC][kWave];
  __shared__ float st[BT * LD];
  __shared__ float s_m[BT];
  __shared__ double s_inv[BT];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * BT;
  const int n_tok = (int)((T - t0) < BT ? (T - t0) : BT);
  const int fr = lane & 15, fk = (lane >> 4) * 8;

  floatx4 acc[1][NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) acc[0][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int kq = d / 4, kbeg = wave * kq;
  int64_t t = t0 + fr;
  t = t < T ? t : T - 1;  // rows past T: any valid row, never stored
  const uint16_t* xrow = x + t * d + kbeg + fk;
  const float* wrow[NJ];
  bool wvalid[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = 16 * j + fr;
    wvalid[j] = e < N;
    wrow[j] = W_r + (int64_t)(e < N ? e : 0) * d + kbeg + fk;
  }

  for (int kg = 0; kg < kq; kg += GRP * 32) {
    bf16x8 a[GRP];
    float4 wv[GRP][NJ][2];
#pragma unroll
    for (int s = 0; s < GRP; ++s) {
      int k = kg + 32 * s;
      k = k < kq ? k : kq - 32;  // past the quarter: reload its last step, never used
      a[s] = *reinterpret_cast<const bf16x8*>(xrow + k);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        wv[s][j][0] = *reinterpret_cast<const float4*>(wrow[j] + k);
        wv[s][j][1] = *reinterpret_cast<const float4*>(wrow[j] + k + 4);
      }
    }
#pragma unroll
    for (int s = 0; s < GRP; ++s) {
      if (kg + 32 * s >= kq) break;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        float w[8] = {wv[s][j][0].x, wv[s][j][0].y, wv[s][j][0].z, wv[s][j][0].w,
                      wv[s][j][1].x, wv[s][j][1].y, wv[s][j][1].z, wv[s][j][1].w};
        if (!wvalid[j]) {
#pragma unroll
          for (int i = 0; i < 8; ++i) w[i] = 0.f;
        }
        bf16x8 hi, mid, lo;
        split3(w, hi, mid, lo);
        acc[0][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s], lo, acc[0][j], 0, 0, 0);
        acc[0][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s], mid, acc[0][j], 0, 0, 0);
        acc[0][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s], hi, acc[0][j], 0, 0, 0);
      }
    }
  }

  if (wave > 0) {
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave - 1][j * 4 + i][lane] = acc[0][j][i];
  }
  __syncthreads();
  if (wave == 0) {
    const int g = lane >> 4;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int e = 16 * j + fr;
      const float bias = (e < N && b_r) ? b_r[e] : 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = acc[0][j][i];
#pragma unroll
        for (int w = 0; w < 3; ++w) v += red[w][j * 4 + i][lane];
        st[(4 * g + i) * LD + e] = e < N ? v + bias : -__builtin_huge_valf();
      }
    }
  }
  __syncthreads();
  block_stats<BT, NPAD, LD>(&st[0], N, k, t0, n_tok, logits, expert_idx, gate,
                            P_part + (int64_t)blockIdx.x * N, s_idx, s_m, s_inv, s_term);
  static_assert(BT * kMaxTopK <= kWave && NPAD <= kWave, "one wave ranks the chunk");
  if (threadIdx.x >= kWave && threadIdx.x < 2 * kWave)
    chunk_hist_rank_wave(s_idx, n_tok * k, t0 * k, N, hist + (int64_t)blockIdx.x * N,
                         rank_local);
}


// More experts (32 < N): a block of WAVES waves owns 16 * ROWT * WAVES tokens
// and NPAD experts starting at e0 = blockIdx.y * NPAD; each wave takes
// 16 * ROWT of the tokens and the whole K.  Every 32-wide K chunk of W_r is
// loaded once per block, split into its three bf16 planes and stored in LDS
// (double buffered, rows of 40 bf16), where all the waves read their B
// fragments; the next chunk is loaded into registers while the current one is
// multiplied.  Each block streams its NPAD rows of W_r once, so more tokens per
// block mean less weight traffic.
// FUSED (N <= NPAD, one expert tile, four waves): routing statistics and the
// chunk histogram / ranks follow; otherwise only the logits are written, the
// tile staged through LDS a group of four waves at a time.
template <int NPAD, int ROWT, bool FUSED, int WAVES = 4>
__global__ __launch_bounds__(64 * WAVES) void router_tok_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ W_r, const float* __restrict__ b_r,
    int64_t T, int d, int N, int k, float* __restrict__ logits, int32_t* __restrict__ expert_idx,
    float* __restrict__ gate, float* __restrict__ P_part, int32_t* __restrict__ hist,
    int32_t* __restrict__ rank_local) {
  constexpr int NTHR = 64 * WAVES, NJ = NPAD / 16, BT = 16 * ROWT * WAVES, WLD = 40,
                LD = NPAD + 4;
  constexpr int WL = NPAD * 8 / NTHR;  // float4 loads per thread per K chunk
  constexpr int WROWS = NTHR / 8;      // W_r rows per loader pass
  static_assert(WL >= 1 && WL * WROWS == NPAD, "whole loader passes over the expert rows");
  static_assert(!FUSED || WAVES == 4, "the statistics take a four-wave block");
  static_assert(WAVES % 4 == 0, "groups of four waves");
  constexpr int GROUPS = WAVES / 4;    // the logit tile goes through LDS a group at a time
  // the weight planes during the K loop, then a group's logit tile
  constexpr int PLANES = 2 * 3 * NPAD * WLD * 2, TILE = (BT / GROUPS) * LD * 4;
  __shared__ __attribute__((aligned(16))) unsigned char raw[PLANES > TILE ? PLANES : TILE];
  typedef uint16_t PlaneArr[3][NPAD * WLD];
  PlaneArr* wpl = reinterpret_cast<PlaneArr*>(raw);
  float* st = reinterpret_cast<float*>(raw);
  __shared__ int32_t s_idx[FUSED ? BT * kMaxTopK : 1];
  __shared__ int32_t cnt[FUSED ? NPAD : 1];
  __shared__ float s_m[FUSED ? BT : 1];
  __shared__ double s_inv[FUSED ? BT : 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * BT;
  const int e0 = blockIdx.y * NPAD;
  const int n_tok = (int)((T - t0) < BT ? (T - t0) : BT);
  const int fr = lane & 15, fk = (lane >> 4) * 8;
  const int64_t tw0 = t0 + wave * 16 * ROWT;

  floatx4 acc[ROWT][NJ];
#pragma unroll
  for (int r = 0; r < ROWT; ++r)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[r][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  const uint16_t* xrow[ROWT];
#pragma unroll
  for (int r = 0; r < ROWT; ++r) {
    int64_t t = tw0 + 16 * r + fr;
    t = t < T ? t : T - 1;  // rows past T: any valid row, never stored
    xrow[r] = x + t * d + fk;
  }
  // W loader: thread covers expert row (tid / 8) + WROWS q and k offset 4 (tid % 8)
  const int wr = tid >> 3, wk = (tid & 7) * 4;
  const float* wsrc[WL];
  bool wok[WL];
#pragma unroll
  for (int q = 0; q < WL; ++q) {
    const int e = e0 + wr + WROWS * q;
    wok[q] = e < N;
    wsrc[q] = W_r + (int64_t)(e < N ? e : 0) * d + wk;
  }
  // PF register stages: K chunks kc+1 .. kc+PF are in flight while kc runs
  constexpr int PF = 3;
  float4 wreg[PF][WL];
  bf16x8 xa[PF][ROWT];
  const int nk = d / 32;
  auto load_chunk = [&](int st, int kc) {
    const int k = (kc < nk ? kc : nk - 1) * 32;
#pragma unroll
    for (int q = 0; q < WL; ++q) wreg[st][q] = *reinterpret_cast<const float4*>(wsrc[q] + k);
#pragma unroll
    for (int r = 0; r < ROWT; ++r) xa[st][r] = *reinterpret_cast<const bf16x8*>(xrow[r] + k);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto store_planes = [&](int st, int buf) {
#pragma unroll
    for (int q = 0; q < WL; ++q) {
      const float4 wq = wreg[st][q];
      const float w4[4] = {wok[q] ? wq.x : 0.f, wok[q] ? wq.y : 0.f, wok[q] ? wq.z : 0.f,
                           wok[q] ? wq.w : 0.f};
      uint32_t hv[2], mv[2], lv[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) split3x2(w4[2 * h], w4[2 * h + 1], hv[h], mv[h], lv[h]);
      const int off = (wr + WROWS * q) * WLD + wk;
      *reinterpret_cast<uint2*>(&wpl[buf][0][off]) = make_uint2(hv[0], hv[1]);
      *reinterpret_cast<uint2*>(&wpl[buf][1][off]) = make_uint2(mv[0], mv[1]);
      *reinterpret_cast<uint2*>(&wpl[buf][2][off]) = make_uint2(lv[0], lv[1]);
    }
  };
  auto compute = [&](int st, int buf) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int off = (16 * j + fr) * WLD + fk;
      const bf16x8 lo = *reinterpret_cast<const bf16x8*>(&wpl[buf][2][off]);
      const bf16x8 mid = *reinterpret_cast<const bf16x8*>(&wpl[buf][1][off]);
      const bf16x8 hi = *reinterpret_cast<const bf16x8*>(&wpl[buf][0][off]);
#pragma unroll
      for (int r = 0; r < ROWT; ++r) {
        acc[r][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[st][r], lo, acc[r][j], 0, 0, 0);
        acc[r][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[st][r], mid, acc[r][j], 0, 0, 0);
        acc[r][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[st][r], hi, acc[r][j], 0, 0, 0);
      }
    }
  };

#pragma unroll
  for (int st = 0; st < PF; ++st) load_chunk(st, st);
  // chunk kc lives in register stage kc % PF and LDS buffer kc % 2; after its
  // planes are stored and multiplied, the stage is refilled with chunk kc + PF
  for (int kc0 = 0; kc0 < nk; kc0 += PF) {
#pragma unroll
    for (int st = 0; st < PF; ++st) {
      const int kc = kc0 + st;
      if (kc < nk) {
        const int buf = kc & 1;
        store_planes(st, buf);
        __syncthreads();
        compute(st, buf);
        load_chunk(st, kc + PF);
      }
    }
  }

  // logit tile (+ bias, padded experts at -inf) into LDS over the weight planes,
  // one group of four waves (64 ROWT tokens) at a time
  constexpr int GT = BT / GROUPS;
  const int grp = wave >> 2;
#pragma unroll 1
  for (int gi = 0; gi < GROUPS; ++gi) {
    __syncthreads();
    if (grp == gi) {
      const int g = lane >> 4;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int e = e0 + 16 * j + fr;
        const float bias = (e < N && b_r) ? b_r[e] : 0.f;
#pragma unroll
        for (int r = 0; r < ROWT; ++r)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            st[((wave & 3) * 16 * ROWT + 16 * r + 4 * g + i) * LD + 16 * j + fr] =
                e < N ? acc[r][j][i] + bias : -__builtin_huge_valf();
      }
    }
    __syncthreads();
    if (!FUSED) {
      // logits only, in full rows of the group's tokens; statistics come from
      // route_rows_kernel
      const int ne = (N - e0) < NPAD ? (N - e0) : NPAD;
      const int r0 = gi * GT;
      const int nr = n_tok - r0 < GT ? n_tok - r0 : GT;
      for (int idx = tid; idx < nr * ne; idx += NTHR) {
        const int r = idx / ne, e = idx - r * ne;
        logits[(t0 + r0 + r) * N + e0 + e] = st[r * LD + e];
      }
    }
  }
  if (!FUSED) return;
  block_stats<BT, NPAD, LD>(st, N, k, t0, n_tok, logits, expert_idx, gate,
                            P_part + (int64_t)blockIdx.x * N, s_idx, s_m, s_inv);
  chunk_hist_rank(s_idx, n_tok * k, t0 * k, N, cnt, hist + (int64_t)blockIdx.x * N, rank_local);
}

// ---------------------------------------------------------------------------
// Logits of many experts (N > 256, bf16 tokens): a dense fp32-exact GEMM
// h[T, N] = x W_r^T + b on bf16 MFMA over the three-plane split of W_r (see
// split3), written to memory for the statistics kernel below.  A pre-pass
// writes hi, mid and lo of every W_r row (split3x2) to planes [3][N][d] bf16
// once per call, and the logits kernel moves its x and plane tiles from memory
// straight into LDS (global_load_lds_dwordx4: no registers and no VALU on the
// way), so the data path of a step is eight load instructions per wave.
//
// Block: 512 threads = 8 waves, tile 256 tokens x 256 experts; waves in a
// 2 x 4 grid (token half, expert quarter), each 128 tokens x 64 experts = 4 x 2
// tiles of v_mfma_f32_32x32x16_bf16 with the weight plane as the first operand,
// so lane l ends up holding token (l % 32) of a tile and 16 of its 32 experts:
// rows 8 (v / 4) + 4 (l / 32) + (v % 4), which leave as four 16-byte stores.
// Every x fragment serves three MFMAs (one per plane) and every plane fragment
// four token tiles.  K steps of 32; the tiles are [rows][32] bf16 (64-byte
// rows): x tiles (16 KB) in a ring of four, the three plane tiles of a step
// (48 KB) in a ring of two, 160 KB in all.  Tile order: block b takes expert
// tile b % n_et and token tile b / n_et, so with 8 expert tiles XCD k (b % 8)
// keeps its 256 experts' planes (3 MB) in its L2 and the planes are fetched one
// step ahead; the x tiles come from beyond L2 (every XCD reads all of x once)
// and are fetched three steps ahead.  Every load instruction fills 1 KB of LDS
// (16 rows) with lane l writing bytes 16 l .. 16 l + 15, so the rows cannot be
// padded; instead the 16-byte chunk c of row r sits at position
// c ^ ((r >> 2) & 3) of its row, which puts the 16 rows one fragment read
// touches (one chunk each) on 16 distinct groups of four banks (the counters
// read no bank conflicts).  A lane of a load instruction therefore fetches row
// R + l / 4, chunk (l % 4) ^ swizzle(row).
// ---------------------------------------------------------------------------
constexpr int RD_BT = 256, RD_BE = 256, RD_BK = 32;
constexpr int RD_XB = RD_BT * RD_BK * 2;          // bytes of the x tile
constexpr int RD_PB = RD_BE * RD_BK * 2;          // bytes of one plane tile
constexpr int RD_XRING = 4, RD_PRING = 2;         // x and plane stages
constexpr int RD_POFF = RD_XRING * RD_XB;         // plane ring offset
constexpr size_t kRouterDmaLds = (size_t)RD_POFF + RD_PRING * 3 * (size_t)RD_PB;  // 160 KiB

typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(1))) void* global_void_ptr;

// byte offset of logical 16-byte chunk c (0..3) of row r in a [rows][32] tile
__device__ __forceinline__ int rd_at(int r, int c) { return r * 64 + ((c ^ ((r >> 2) & 3)) << 4); }

// planes[p][e][k] (p = 0 hi, 1 mid, 2 lo) of W_r [N][d]; n8 = N d / 8.
__global__ __launch_bounds__(256) void router_planes_kernel(const float* __restrict__ W_r,
                                                            uint16_t* __restrict__ planes,
                                                            int64_t n8) {
  const int64_t plane = n8 * 8;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8;
       i += (int64_t)gridDim.x * blockDim.x) {
    const float4 a = reinterpret_cast<const float4*>(W_r)[2 * i];
    const float4 b = reinterpret_cast<const float4*>(W_r)[2 * i + 1];
    const float w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    uint32_t h4[4], m4[4], l4[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) split3x2(w[2 * j], w[2 * j + 1], h4[j], m4[j], l4[j]);
    *reinterpret_cast<u32x4*>(planes + 8 * i) = u32x4{h4[0], h4[1], h4[2], h4[3]};
    *reinterpret_cast<u32x4*>(planes + plane + 8 * i) = u32x4{m4[0], m4[1], m4[2], m4[3]};
    *reinterpret_cast<u32x4*>(planes + 2 * plane + 8 * i) = u32x4{l4[0], l4[1], l4[2], l4[3]};
  }
}

__global__ __launch_bounds__(512, 1) void router_gemm_dma_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ planes,
    const float* __restrict__ b_r, float* __restrict__ h, int64_t T, int d, int N, int n_et,
    bool vec) {
  extern __shared__ __attribute__((aligned(16))) uint16_t rlds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wt = wave >> 2, we = wave & 3;
  const int et = (int)(blockIdx.x % (unsigned)n_et);
  const int64_t t0 = (int64_t)(blockIdx.x / (unsigned)n_et) * RD_BT;
  const int e0 = et * RD_BE;

  // wave w moves rows 32 w .. 32 w + 31 of the x tile (two instructions) and
  // rows 96 w .. 96 w + 95 of the 768 plane rows [3][256] (six); token rows
  // past T read row T - 1 and expert rows past N read row 0 (never stored)
  const int lr = lane >> 2, pc = lane & 3;
  const uint16_t* src[8];
  int dst[8];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = 32 * wave + 16 * j + lr;
    int64_t tr = t0 + row;
    tr = tr < T ? tr : T - 1;
    src[j] = x + tr * d + ((pc ^ ((row >> 2) & 3)) << 3);
    dst[j] = (32 * wave + 16 * j) * 64;  // within an x stage
  }
#pragma unroll
  for (int j = 0; j < 6; ++j) {
    const int prow = 96 * wave + 16 * j + lr;
    const int p = prow >> 8, r = prow & 255;
    const int e = e0 + r < N ? e0 + r : 0;
    src[2 + j] = planes + ((int64_t)p * N + e) * d + ((pc ^ ((r >> 2) & 3)) << 3);
    dst[2 + j] = (96 * wave + 16 * j) * 64;  // within a plane stage
  }
  char* lds_bytes = reinterpret_cast<char*>(rlds);
  auto dma_x = [&](int kc) {
    char* stage = lds_bytes + (kc & (RD_XRING - 1)) * RD_XB;
#pragma unroll
    for (int j = 0; j < 2; ++j)
      __builtin_amdgcn_global_load_lds((global_void_ptr)(src[j] + kc * RD_BK),
                                       (lds_void_ptr)(stage + dst[j]), 16, 0, 0);
  };
  auto dma_planes = [&](int kc) {
    char* stage = lds_bytes + RD_POFF + (kc & (RD_PRING - 1)) * 3 * RD_PB;
#pragma unroll
    for (int j = 2; j < 8; ++j)
      __builtin_amdgcn_global_load_lds((global_void_ptr)(src[j] + kc * RD_BK),
                                       (lds_void_ptr)(stage + dst[j]), 16, 0, 0);
  };

  floatx16 acc[2][4];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[j][i][v] = 0.f;
  const int fr = lane & 31, fc = lane >> 5;
  // fragments of K sub-step s (16 k): x of the wave's four token tiles and,
  // per plane, its two expert tiles
  struct Frags {
    bf16x8 x[4], w[3][2];
  };
  auto read_x = [&](Frags& f, const char* xst, int s) {
    const int c = 2 * s + fc;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      f.x[i] = *reinterpret_cast<const bf16x8*>(xst + rd_at(wt * 128 + i * 32 + fr, c));
  };
  auto read_w = [&](Frags& f, const char* pst, int s) {
    const int c = 2 * s + fc;
#pragma unroll
    for (int p = 2; p >= 0; --p)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        f.w[p][j] = *reinterpret_cast<const bf16x8*>(pst + p * RD_PB +
                                                     rd_at(we * 64 + j * 32 + fr, c));
  };
  // the 24 MFMAs of a sub-step, smallest plane first
  auto mfmas = [&](const Frags& f) {
#pragma unroll
    for (int p = 2; p >= 0; --p)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.w[p][j], f.x[i], acc[j][i], 0, 0, 0);
  };

  // Issue order: x 0, x 1, planes 0, x 2, then in step t planes t + 1 and
  // x t + 3.  At the top of step t the last two load instructions of this wave
  // are those of x t + 2 (while it exists), so waiting until at most two are
  // outstanding completes x t, x t + 1 and planes t (the counter retires loads
  // in issue order); the barrier then covers every wave's loads, and every
  // wave has finished step t - 1, whose stages steps t + 1 and t + 3 refill.
  // (A plain __syncthreads would wait for all outstanding loads.)
  const int nk = d / RD_BK;
  dma_x(0);
  if (nk > 1) dma_x(1);
  dma_planes(0);
  if (nk > 2) dma_x(2);
  auto xstage = [&](int kc) { return lds_bytes + (kc & (RD_XRING - 1)) * RD_XB; };
  auto pstage = [&](int kc) { return lds_bytes + RD_POFF + (kc & (RD_PRING - 1)) * 3 * RD_PB; };
  // The wait before step t's barrier also completes this wave's fragment
  // reads (lgkmcnt 0): the loads issued after the barrier refill the stages
  // that step t - 1 read.
  auto step_barrier = [&](int t) {
    if (t + 2 < nk) asm volatile("s_waitcnt vmcnt(2) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };
  // MFMAs of `f` with the ten fragment reads of `g` (sub-step s of step kc)
  // spread between them, one read after every two MFMAs
  auto mfmas_reading = [&](const Frags& f, Frags& g, int kc, int s) {
    mfmas(f);
    read_x(g, xstage(kc), s);
    read_w(g, pstage(kc), s);
#pragma unroll
    for (int i = 0; i < 10; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    __builtin_amdgcn_sched_barrier(0);
  };
  // Software pipeline across the barrier: after step t's barrier the MFMAs of
  // step t - 1's second sub-step (its fragments already in registers) run
  // while step t's first fragments arrive, then step t's first sub-step runs
  // while its second sub-step's fragments arrive.
  Frags f0, f1;
  step_barrier(0);
  if (nk > 1) dma_planes(1);
  if (nk > 3) dma_x(3);
  read_x(f0, xstage(0), 0);
  read_w(f0, pstage(0), 0);
  __builtin_amdgcn_sched_barrier(0);
  mfmas_reading(f0, f1, 0, 1);
  // Each wave raises its issue priority for its MFMA and fragment-read section and
  // drops it before the next barrier, so that on a SIMD a wave in that section
  // issues ahead of one between sections (1% faster at the 2048-expert share,
  // same process).
  for (int t = 1; t < nk; ++t) {
    step_barrier(t);
    if (t + 1 < nk) dma_planes(t + 1);
    if (t + 3 < nk) dma_x(t + 3);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(1);
    mfmas_reading(f1, f0, t, 0);
    mfmas_reading(f0, f1, t, 1);
    __builtin_amdgcn_s_setprio(0);
  }
  mfmas(f1);

  // Epilogue: each wave stages two of its four 32-token tiles at a time in its
  // own 20 KB of the (now free) LDS, rows of 64 logits padded to 68, and reads
  // them back row-major, so that every store instruction writes four whole
  // 256-byte row pieces (the accumulator layout alone gives 32-byte pieces of
  // 32 rows, whose lines can be written back before they are complete).
  __syncthreads();  // every wave is done with the operand rings
  constexpr int SP = 68;                                 // staged row pitch (floats)
  float* wst = reinterpret_cast<float*>(rlds) + wave * (20480 / 4);
  const int rc = lane & 15, rr = lane >> 4;              // read-back: chunk, row within 4
  const int eb = e0 + we * 64 + 4 * rc;                  // first expert of the lane's chunk
  float bias[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) bias[u] = (b_r && eb + u < N) ? b_r[eb + u] : 0.f;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
      const int i = 2 * half + ii;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<float4*>(wst + (ii * 32 + fr) * SP + j * 32 + 8 * q + 4 * fc) =
              make_float4(acc[j][i][4 * q], acc[j][i][4 * q + 1], acc[j][i][4 * q + 2],
                          acc[j][i][4 * q + 3]);
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 16; ++it) {
      const int row = 4 * it + rr;                       // 0..63: two token tiles
      const int64_t t = t0 + wt * 128 + half * 64 + row;
      const float4 v4 = *reinterpret_cast<const float4*>(wst + row * SP + 4 * rc);
      if (t >= T) continue;
      float v[4] = {v4.x + bias[0], v4.y + bias[1], v4.z + bias[2], v4.w + bias[3]};
      float* hrow = h + t * N;
      if (vec && eb + 3 < N) {
        *reinterpret_cast<float4*>(hrow + eb) = make_float4(v[0], v[1], v[2], v[3]);
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (eb + u < N) hrow[eb + u] = v[u];
      }
    }
    __syncthreads();  // the second half reuses the staging rows
  }
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

// e^x for x <= 0 (or -inf) as 2^(x log2 e) on the hardware exp2 (v_exp_f32, about
// 1 ulp): the product x log2 e is rounded to t, and what the rounding and the
// fp32 value of log2 e leave out, dt = (x L - t) + x L_lo (fma keeps x L exact),
// is put back to first order, 2^(t + dt) = 2^t (1 + dt ln 2) with |dt| < 2^-16.
// Inputs below -104 give 0 (e^-104 is below the smallest fp32 denormal).  The
// statistics kernels below, which read logits from memory, take every
// exponential from here: within about 2 ulp (a library expf: about 1), in seven
// instructions instead of twelve.
__device__ __forceinline__ float exp_nonpos(float x) {
  constexpr float kLog2e = 1.44269502f;             // fp32(log2 e)
  constexpr float kLog2eLo = 1.92596299e-8f;        // log2 e - fp32(log2 e)
  constexpr float kLn2 = 0.693147182f;
  x = fmaxf(x, -104.0f);
  const float t = x * kLog2e;
  const float dt = fmaf(x, kLog2eLo, fmaf(x, kLog2e, -t));
  const float r = __builtin_amdgcn_exp2f(t);
  return fmaf(r, dt * kLn2, r);
}

__global__ __launch_bounds__(256) void route_rows_kernel(const float* __restrict__ h, int64_t T,
                                                         int N, int k,
                                                         int32_t* __restrict__ expert_idx,
                                                         float* __restrict__ gate,
                                                         float* __restrict__ P_part,
                                                         int32_t* __restrict__ hist,
                                                         int32_t* __restrict__ rank_local) {
  extern __shared__ int32_t cnt[];
  __shared__ float s_m[RR_ROWS];
  __shared__ double s_inv[RR_ROWS];
  __shared__ int32_t s_idx[RR_ROWS * kMaxTopK];
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
    for (int i = lane; i < N; i += kWave) s += (double)exp_nonpos(row[i] - m);
    s = wave_sum_f64(s);
    // second choice (k = 2): the best of the other experts, lowest index on ties
    float m2 = -__builtin_huge_valf();
    int mi2 = 0x7fffffff;
    if (k > 1) {
      for (int i = lane; i < N; i += kWave) {
        const float v = row[i];
        if (i != mi && (v > m2 || mi2 == 0x7fffffff)) { m2 = v; mi2 = i; }
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const float om = __shfl_xor(m2, o, kWave);
        const int oi = __shfl_xor(mi2, o, kWave);
        if (oi != 0x7fffffff && (mi2 == 0x7fffffff || om > m2 || (om == m2 && oi < mi2))) {
          m2 = om;
          mi2 = oi;
        }
      }
    }
    if (lane == 0) {
      expert_idx[(t0 + r) * k] = mi;
      gate[(t0 + r) * k] = (float)(1.0 / s);
      s_m[r] = m;
      s_inv[r] = 1.0 / s;
      s_idx[r * k] = mi;
      if (k > 1) {
        expert_idx[(t0 + r) * k + 1] = mi2;
        gate[(t0 + r) * k + 1] = (float)((double)exp_nonpos(m2 - m) * (1.0 / s));
        s_idx[r * k + 1] = mi2;
      }
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < N; i += blockDim.x) {
    double acc = 0.0;
    for (int r = 0; r < rows; ++r) acc += (double)exp_nonpos(h[(t0 + r) * N + i] - s_m[r]) * s_inv[r];
    P_part[(int64_t)blockIdx.x * N + i] = (float)acc;
  }
  chunk_hist_rank(s_idx, rows * k, t0 * k, N, cnt, hist + (int64_t)blockIdx.x * N, rank_local);
}

// Statistics from logits with each row read once (N <= 64 NPL): a wave takes
// rows w, w + 4, ... of the block's 64; lane l holds experts l + 64 i of the row
// in registers for the max, the sum, the second choice and its own running
// sums of p over the wave's 16 rows (fp32: at most 16 terms of at most 1).
// The four waves' sums are then added in fp64 as (w0 + w2) + (w1 + w3) through
// two LDS rows of N doubles, which the chunk's counts reuse afterwards.  Same statistics as route_rows_kernel; the P sums
// are the same terms added in another fixed order.  K (choices per token) and
// FULL (N == 64 NPL: no padded experts) are compile-time, so that no per-expert
// masks or indices stay live: with at most 128 registers four blocks share a
// CU (32 KB of LDS each at N = 2048), twice the waves of the register-bound
// form, which hides the row loads behind the other waves' arithmetic.
// word 3 of a raw buffer resource on gfx9-family parts: 32-bit data format,
// offsets checked against the record count
constexpr int kBufferRsrcWord3 = 0x00020000;

template <int NPL, int K, bool FULL>
__global__ __launch_bounds__(256, 4) void route_rows_reg_kernel(const float* __restrict__ h,
                                                                int64_t T, int N,
                                                                int32_t* __restrict__ expert_idx,
                                                                float* __restrict__ gate,
                                                                float* __restrict__ P_part,
                                                                int32_t* __restrict__ hist,
                                                                int32_t* __restrict__ rank_local) {
  extern __shared__ double rr_red[];  // [2][N] partial sums, later N ints of counts
  __shared__ int32_t s_idx[RR_ROWS * kMaxTopK];
  int32_t* cnt = reinterpret_cast<int32_t*>(rr_red);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: row bases in SGPRs
  const int64_t t0 = (int64_t)blockIdx.x * RR_ROWS;
  const int rows = (int)((T - t0) < RR_ROWS ? (T - t0) : RR_ROWS);
  float pacc[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) pacc[i] = 0.0f;

  // row r + 4 is loaded while row r is worked on: two register buffers, the loop
  // taken twice per pass so that no copy between them waits for the loads
  auto load_row = [&](float (&v)[NPL], int r) {
    // buffer loads over the one row: a uniform base, one lane offset, and reads
    // past the row's N values return 0 without touching memory
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(h + (t0 + r) * N), (short)0, N * 4, kBufferRsrcWord3);
    // the lane's byte offset, kept opaque so that the compiler folds each
    // element's 256 i into the instruction instead of holding NPL offsets live
    int off = lane * 4;
    asm volatile("" : "+v"(off));
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      v[i] = __builtin_bit_cast(
          float, __builtin_amdgcn_raw_buffer_load_b32(rs, off + 256 * (i & 15), 4096 * (i >> 4), 0));
  };
  auto do_row = [&](float (&v)[NPL], float (&vn)[NPL], int r) {
    load_row(vn, r + 4 < rows ? r + 4 : r);  // the last one reads its own row again
    // experts past N (read as 0) out of every choice and sum; done here, not at
    // the load, so that only this row's loads are waited for
    if (!FULL) {
#pragma unroll
      for (int i = 0; i < NPL; ++i)
        if (lane + kWave * i >= N) v[i] = -__builtin_huge_valf();
    }
    // lane maximum, the first (lowest) index among equals: a strict > over
    // ascending i; a lane with no expert (lane >= N) offers -inf at index lane,
    // which loses to every expert's index on a tie
    float m = v[0];
    int mi = 0;
#pragma unroll
    for (int i = 1; i < NPL; ++i)
      if (v[i] > m) {
        m = v[i];
        mi = i;
      }
    mi = lane + kWave * mi;
    wave_argmax(m, mi);
    float m2 = -__builtin_huge_valf();
    int mi2 = 0x7fffffff;
    if (K > 1) {
#pragma unroll
      for (int i = 0; i < NPL; ++i) {
        const int e = lane + kWave * i;
        if ((FULL || e < N) && e != mi && (v[i] > m2 || mi2 == 0x7fffffff)) {
          m2 = v[i];
          mi2 = e;
        }
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const float om = __shfl_xor(m2, o, kWave);
        const int oi = __shfl_xor(mi2, o, kWave);
        if (oi != 0x7fffffff && (mi2 == 0x7fffffff || om > m2 || (om == m2 && oi < mi2))) {
          m2 = om;
          mi2 = oi;
        }
      }
    }
    // each exponential once: the terms replace the logits (the same values, added
    // in the same order, as evaluating them again for the sums of p)
    double sum = 0.0;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      v[i] = exp_nonpos(v[i] - m);
      sum += (double)v[i];
    }
    sum = wave_sum_f64(sum);
    const double inv = 1.0 / sum;
    const float invf = (float)inv;
#pragma unroll
    for (int i = 0; i < NPL; ++i) pacc[i] = fmaf(v[i], invf, pacc[i]);
    if (lane == 0) {
      expert_idx[(t0 + r) * K] = mi;
      gate[(t0 + r) * K] = (float)inv;
      s_idx[r * K] = mi;
      if (K > 1) {
        expert_idx[(t0 + r) * K + 1] = mi2;
        gate[(t0 + r) * K + 1] = (float)((double)exp_nonpos(m2 - m) * inv);
        s_idx[r * K + 1] = mi2;
      }
    }
  };
  float va[NPL], vb[NPL];
  if (wave < rows) load_row(va, wave);
  for (int r = wave; r < rows; r += 8) {
    do_row(va, vb, r);
    if (r + 4 >= rows) break;
    do_row(vb, va, r + 4);
  }
  // (w0 + w2) + (w1 + w3) in fp64: waves 2 and 3 leave their sums in two LDS
  // rows, waves 0 and 1 add theirs in place, then wave 0 adds the two rows
  if (wave >= 2) {
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if (FULL || lane + kWave * i < N) rr_red[(wave - 2) * N + lane + kWave * i] = (double)pacc[i];
  }
  __syncthreads();
  if (wave < 2) {
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if (FULL || lane + kWave * i < N) rr_red[wave * N + lane + kWave * i] += (double)pacc[i];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int e = lane + kWave * i;
      if (FULL || e < N) P_part[(int64_t)blockIdx.x * N + e] = (float)(rr_red[e] + rr_red[N + e]);
    }
  }
  __syncthreads();  // the counts below reuse the rows
  chunk_hist_rank(s_idx, rows * K, t0 * K, N, cnt, hist + (int64_t)blockIdx.x * N, rank_local);
}

// ------------------------------------------------------------------ launchers

constexpr int kTokRowt = 2;                 // router_tok_kernel: 128 tokens per block

bool router_fused_ok(bool x_bf16, int N) { return x_bf16 && N <= 256; }

int64_t route_chunk_tokens(bool x_bf16, int N) {
  if (!router_fused_ok(x_bf16, N)) return RR_ROWS;
  return N <= 32 ? 16 : 64 * kTokRowt;
}

void launch_router_logits(const void* x, bool x_bf16, const float* W_r, const float* b_r,
                          float* h, int64_t T, int d, int N, uint16_t* planes, hipStream_t s) {
  if (T == 0) return;
  if (x_bf16) {
    // the weight planes once per call, then MFMA logits in 256 x 256 tiles;
    // statistics by route_rows_kernel
    static uint64_t set_on = 0;
    int dev = 0;
    (void)hipGetDevice(&dev);
    if (dev < 64 && !(set_on >> dev & 1)) {
      (void)hipFuncSetAttribute((const void*)router_gemm_dma_kernel,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)kRouterDmaLds);
      set_on |= 1ull << dev;
    }
    const int64_t n8 = (int64_t)N * d / 8;
    const int64_t pb = (n8 + 255) / 256;
    launch_k(router_planes_kernel, dim3((unsigned)(pb < 4096 ? pb : 4096)), dim3(256), 0, s, W_r,
             planes, n8);
    const int n_et = (N + RD_BE - 1) / RD_BE;
    const int64_t n_tt = (T + RD_BT - 1) / RD_BT;
    const bool vec = (N & 3) == 0 && ((uintptr_t)h & 15) == 0;
    launch_k(router_gemm_dma_kernel, dim3((unsigned)(n_tt * n_et)), dim3(512), kRouterDmaLds, s,
             (const uint16_t*)x, (const uint16_t*)planes, b_r, h, T, d, N, n_et, vec);
    return;
  }
  dim3 grid((unsigned)((T + RT_BT - 1) / RT_BT), (unsigned)((N + RT_BE - 1) / RT_BE));
  launch_k(router_logits_kernel<float>, grid, dim3(256), 0, s, (const float*)x, W_r,
                     b_r, h, T, d, N);
}

void launch_router_fused(const uint16_t* x, const float* W_r, const float* b_r, int64_t T, int d,
                         int N, int k, float* logits, int32_t* expert_idx, float* gate,
                         float* P_part, int32_t* hist, int32_t* rank_local, hipStream_t s) {
  if (T == 0) return;
  const int64_t ch = route_chunk_tokens(true, N);
  const dim3 grid((unsigned)((T + ch - 1) / ch));
#define SWL_SMALL(NP)                                                                           \
  launch_k((router_small_kernel<NP>), grid, dim3(256), 0, s, x, W_r, b_r, T, d, N, k, \
                     logits, expert_idx, gate, P_part, hist, rank_local)
#define SWL_TOK(NP)                                                                             \
  launch_k((router_tok_kernel<NP, kTokRowt, true>), grid, dim3(256), 0, s, x, W_r,    \
                     b_r, T, d, N, k, logits, expert_idx, gate, P_part, hist, rank_local)
  if (N <= 16) SWL_SMALL(16);
  else if (N <= 32) SWL_SMALL(32);
  else if (N <= 64) SWL_TOK(64);
  else if (N <= 128) SWL_TOK(128);
  else SWL_TOK(256);
#undef SWL_SMALL
#undef SWL_TOK
}

void launch_route_rows(const float* h, int64_t T, int N, int k, int32_t* expert_idx, float* gate,
                       float* P_part, int32_t* hist, int32_t* rank_local, hipStream_t s) {
  if (T == 0) return;
  const dim3 grid((unsigned)((T + RR_ROWS - 1) / RR_ROWS));
  const size_t lds = 2 * sizeof(double) * (size_t)N;
#define SWL_RR3(NPL, K, FULL)                                                                    \
  launch_k((route_rows_reg_kernel<NPL, K, FULL>), grid, dim3(256), lds, s, h, T, N, expert_idx, \
           gate, P_part, hist, rank_local)
#define SWL_RR(NPL)                                                                              \
  do {                                                                                           \
    const bool full = N == kWave * NPL;                                                          \
    if (k == 1 && full) SWL_RR3(NPL, 1, true);                                                   \
    else if (k == 1) SWL_RR3(NPL, 1, false);                                                     \
    else if (full) SWL_RR3(NPL, 2, true);                                                        \
    else SWL_RR3(NPL, 2, false);                                                                 \
  } while (0)
  if (N <= 4 * kWave) SWL_RR(4);
  else if (N <= 8 * kWave) SWL_RR(8);
  else if (N <= 16 * kWave) SWL_RR(16);
  else if (N <= 32 * kWave) SWL_RR(32);
  else
    launch_k(route_rows_kernel, grid, dim3(256), sizeof(int32_t) * (size_t)N, s, h, T,
                       N, k, expert_idx, gate, P_part, hist, rank_local);
#undef SWL_RR
#undef SWL_RR3
}

}  // namespace swl
