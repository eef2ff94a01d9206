// Capacity assignment and the load-balancing loss.
//
// position[t] = number of earlier tokens (in flattened token order) routed to
// the same expert; a token whose position reaches the capacity C overflows and
// is dropped.  The token-order rule follows the Incredible.AI blog's "MoE Layer"
// section (an expert keeps the first `capacity` tokens routed to it) and the
// kasblo explainer's "16 token、4 Expertで考える"; the overflow token of
// "Switch Transformer by Hand" (step 7) is the third token routed to a full
// expert.  All of it is integer work on per-chunk counts and is deterministic:
// the router leaves hist[c, e] and in-chunk ranks; this kernel turns hist into
// exclusive prefixes over chunks; the dispatch pass adds the two.
//
// Load-balancing loss (llm-papers-study close reading, section 3.3):
// aux = alpha N sum_i f_i P_i, f_i = load_i / T, P_i = (1/T) sum_t p_i(t), with
// load_i counted before the capacity cut.  With k choices per token load_i
// counts assignments and f_i = load_i / (k T).
#include "common.hpp"
#include "kernels.hpp"

namespace swl {

// tile_start[e] = sum over e' < e of ceil(n_kept[e'] / tile_rows), and
// tile_start[N] the total: the compact tile list of the grouped matmuls.  One
// block of 1024 threads; each thread takes a contiguous run of experts.
__device__ void tile_prefix_block(const int32_t* __restrict__ n_kept, int N, int tile_rows,
                                  int32_t* __restrict__ tile_start, int32_t* s_run) {
  const int tid = threadIdx.x;
  const int per = (N + 1023) / 1024;
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

// Chunk scan.  A block of 1024 threads takes EG consecutive experts (EG a power
// of two: N rounded up when one block covers all experts, 64 otherwise); the
// G = 1024 / EG threads of an expert split the chunk range into contiguous
// pieces.  Each thread sums its piece (counts and
// probability sums); a log-step scan over the pieces (in LDS) gives each
// piece's start, and the thread rewrites its piece of hist[:, e] as exclusive
// prefixes.  Probability sums of the pieces add in a fixed pairwise tree
// (fp64).  Every result is independent of timing.  With more than one block
// the loss terms load_e * Psum_e go to `terms` for aux_kernel; with one block
// the loss is finished here.
__global__ __launch_bounds__(1024) void route_scan_kernel(int32_t* __restrict__ hist,
                                                          const float* __restrict__ P_part,
                                                          int64_t nc, int N, int EG, int64_t T,
                                                          int k, int64_t C, float alpha,
                                                          int32_t* __restrict__ load,
                                                          int32_t* __restrict__ n_kept,
                                                          double* __restrict__ terms,
                                                          float* __restrict__ aux,
                                                          int32_t* __restrict__ tile_start,
                                                          int tile_rows) {
  __shared__ int32_t s_cnt[1024];
  __shared__ double s_p[1024];
  const int tid = threadIdx.x;
  const int G = 1024 / EG;
  const int el = tid % EG, g = tid / EG;
  const int64_t per = (nc + G - 1) / G;
  const int64_t c0 = (int64_t)g * per;
  const int64_t c1 = (c0 + per < nc) ? c0 + per : nc;
  const int e = blockIdx.x * EG + el;
  const bool valid = e < N;

  int32_t cnt = 0;
  double p = 0.0;
  if (valid) {
#pragma unroll 8
    for (int64_t c = c0; c < c1; ++c) {
      cnt += hist[c * N + e];
      p += (double)P_part[c * N + e];
    }
  }
  s_cnt[tid] = cnt;
  s_p[tid] = p;
  __syncthreads();
  // inclusive scan of the pieces' counts along g (Hillis-Steele)
  for (int off = 1; off < G; off <<= 1) {
    const int32_t v = g >= off ? s_cnt[tid - off * EG] : 0;
    __syncthreads();
    s_cnt[tid] += v;
    __syncthreads();
  }
  // pairwise sum of the pieces' probability sums along g
  for (int half = G >> 1; half >= 1; half >>= 1) {
    if (g < half) s_p[tid] += s_p[tid + half * EG];
    __syncthreads();
  }
  if (valid) {
    int32_t run = s_cnt[tid] - cnt;  // exclusive start of this piece
#pragma unroll 8
    for (int64_t c = c0; c < c1; ++c) {
      const int32_t v = hist[c * N + e];
      hist[c * N + e] = run;
      run += v;
    }
  }
  double term = 0.0;
  if (g == G - 1 && valid) {
    const int32_t total = s_cnt[tid];
    load[e] = total;
    n_kept[e] = (int32_t)((int64_t)total < C ? (int64_t)total : C);
    term = (double)total * s_p[el];
    if (terms) terms[e] = term;
  }
  if (terms) return;
  // the EG loss terms sit in the last EG threads: a fixed pairwise tree over them
  __syncthreads();
  if (g == G - 1) s_p[el] = term;
  __syncthreads();
  for (int s = EG >> 1; s >= 1; s >>= 1) {
    if (tid < s) s_p[tid] += s_p[tid + s];
    __syncthreads();
  }
  if (tid == 0) {
    double v = 0.0;
    if (T > 0) v = (double)alpha * (double)N * (s_p[0] / ((double)k * (double)T * (double)T));
    *aux = (float)v;
  }
  // n_kept of every expert was written by this block above
  if (tile_start) tile_prefix_block(n_kept, N, tile_rows, tile_start, s_cnt);
}

// aux = alpha N sum_e terms[e] / T^2, summed in a fixed tree (fp64).
__global__ __launch_bounds__(1024) void aux_kernel(const double* __restrict__ terms, int N,
                                                   int64_t T, int k, float alpha,
                                                   float* __restrict__ aux,
                                                   const int32_t* __restrict__ n_kept,
                                                   int32_t* __restrict__ tile_start,
                                                   int tile_rows) {
  __shared__ double red[1024];
  __shared__ int32_t s_run[1024];
  double acc = 0.0;
  for (int i = threadIdx.x; i < N; i += 1024) acc += terms[i];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int s = 512; s >= 1; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    double v = 0.0;
    if (T > 0) v = (double)alpha * (double)N * (red[0] / ((double)k * (double)T * (double)T));
    *aux = (float)v;
  }
  if (tile_start) tile_prefix_block(n_kept, N, tile_rows, tile_start, s_run);
}

// position = chunk offset + in-chunk rank; drop when it reaches C (route only:
// no data moves).  One thread per assignment a = t * k + j.
__global__ __launch_bounds__(256) void finalize_positions_kernel(
    int64_t T, int k, const int32_t* __restrict__ expert_idx,
    const int32_t* __restrict__ rank_local, const int32_t* __restrict__ offsets, int N,
    int64_t chunk, int64_t C, int32_t* __restrict__ position, uint8_t* __restrict__ drop_mask) {
  const int64_t a = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (a >= T * k) return;
  const int64_t t = a / k;
  const int32_t pos = offsets[(t / chunk) * N + expert_idx[a]] + rank_local[a];
  position[a] = pos;
  drop_mask[a] = (int64_t)pos >= C ? 1 : 0;
}

// ------------------------------------------------------------------ launchers

void launch_route_scan(int32_t* hist, const float* P_part, int64_t nc, int N, int64_t T, int k,
                       int64_t C, float alpha, int32_t* load, int32_t* n_kept, double* terms,
                       float* aux, int32_t* tile_start, int tile_rows, hipStream_t s) {
  if (N <= 1024) {
    int EG = 1;
    while (EG < N) EG <<= 1;
    hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(1024), 0, s, hist, P_part, nc, N, EG, T,
                       k, C, alpha, load, n_kept, nullptr, aux, tile_start, tile_rows);
    return;
  }
  constexpr int EG = 64;
  hipLaunchKernelGGL(route_scan_kernel, dim3((unsigned)((N + EG - 1) / EG)), dim3(1024), 0, s,
                     hist, P_part, nc, N, EG, T, k, C, alpha, load, n_kept, terms, aux, nullptr,
                     tile_rows);
  hipLaunchKernelGGL(aux_kernel, dim3(1), dim3(1024), 0, s, terms, N, T, k, alpha, aux, n_kept,
                     tile_start, tile_rows);
}

void launch_finalize_positions(int64_t T, int k, const int32_t* expert_idx,
                               const int32_t* rank_local, const int32_t* offsets, int N,
                               int64_t chunk, int64_t C, int32_t* position, uint8_t* drop_mask,
                               hipStream_t s) {
  if (T == 0) return;
  const int64_t n = T * k;
  hipLaunchKernelGGL(finalize_positions_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                     s, T, k, expert_idx, rank_local, offsets, N, chunk, C, position, drop_mask);
}

}  // namespace swl
