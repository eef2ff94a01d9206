// Capacity assignment and the load-balancing loss.
//
// position[t] = number of earlier tokens (in flattened token order) routed to
// the same expert; a token whose position reaches the capacity C overflows and
// is dropped.  The token-order rule follows the Incredible.AI blog's "MoE Layer"
// section (an expert keeps the first `capacity` tokens routed to it) and the
// kasblo explainer's "16 token、4 Expertで考える"; the overflow token of
// "Switch Transformer by Hand" (step 7) is the third token routed to a full
// expert.  All of it is integer work on per-chunk counts and is deterministic:
// the router leaves hist[c, e] and in-chunk ranks; position = the exclusive
// prefix of hist over earlier chunks + the rank.  assign_kernel does it all in
// one launch; for large count tables route_scan_kernel rewrites hist into the
// prefixes and the dispatch pass adds the two.
//
// Load-balancing loss (llm-papers-study close reading, section 3.3):
// aux = alpha N sum_i f_i P_i, f_i = load_i / T, P_i = (1/T) sum_t p_i(t), with
// load_i counted before the capacity cut.  With k choices per token load_i
// counts assignments and f_i = load_i / (k T).
#include "common.hpp"
#include "kernels.hpp"

namespace swl {

// Chunk scan.  A block of 1024 threads takes EG consecutive experts (EG a power
// of two: N rounded up when one block covers all experts, 32 otherwise); the
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

// ---------------------------------------------------------------------------
// One-launch capacity assignment for moderate sizes (assign_one_launch_ok):
// the chunk scan and the finalisation of the two-kernel path in one grid.
// Blocks 1 .. nb own AS_TOK consecutive tokens each.  Such a block adds up
// hist over every chunk before its first one (integer sums: the order does not
// matter), walks its own chunks for their exclusive offsets, and finalises its
// assignments as the dispatch passes do: position = offset + rank in chunk,
// drop when position >= C, the slot table tok[e * C + position] = t, and the
// row copies of the mode (dropped rows of x to out for the fused top-1
// combine; kept rows of x to Xbuf for the fp32 path).  Block 0 computes the
// per-expert totals (load, n_kept), the loss and the compact tile list, with
// its own fixed summation tree for the probability sums.
// ---------------------------------------------------------------------------
constexpr int AS_TOK = 64;
constexpr int AS_MAXCH = AS_TOK / 16 + 1;  // chunks a block can touch (chunk >= 16)

__global__ __launch_bounds__(256) void assign_kernel(
    const int32_t* __restrict__ hist, const float* __restrict__ P_part, int64_t nc, int N,
    int64_t T, int k, int64_t chunk, int64_t C, float alpha,
    const int32_t* __restrict__ expert_idx, const int32_t* __restrict__ rank_local,
    int32_t* __restrict__ load, int32_t* __restrict__ n_kept, float* __restrict__ aux,
    int32_t* __restrict__ tile_start, int tile_rows, int32_t* __restrict__ position,
    uint8_t* __restrict__ drop_mask, int32_t* __restrict__ tok, int copy_mode, int row_vec16,
    const uint4* __restrict__ x, uint4* __restrict__ dst) {
  __shared__ int32_t s_off[AS_MAXCH * 256];
  __shared__ int32_t s_e[AS_TOK * kMaxTopK];
  __shared__ int32_t s_pos[AS_TOK * kMaxTopK];
  __shared__ double s_p[256];
  const int tid = threadIdx.x;
  int EG = 1;
  while (EG < N) EG <<= 1;
  const int G = 256 / EG, el = tid % EG, g = tid / EG;
  const int64_t nb = (T + AS_TOK - 1) / AS_TOK;

  (void)nb;
  if (blockIdx.x == 0) {
    // totals: G pieces of the chunk range per expert, pieces added in a fixed tree
    int32_t* s_cnt = s_off;
    const int64_t per = (nc + G - 1) / G;
    const int64_t c0 = (int64_t)g * per;
    const int64_t c1 = c0 + per < nc ? c0 + per : nc;
    int32_t cnt = 0;
    double p = 0.0;
    if (el < N)
      for (int64_t c = c0; c < c1; ++c) {
        cnt += hist[c * N + el];
        p += (double)P_part[c * N + el];
      }
    s_cnt[tid] = cnt;
    s_p[tid] = p;
    __syncthreads();
    for (int half = G >> 1; half >= 1; half >>= 1) {
      if (g < half) {
        s_cnt[tid] += s_cnt[tid + half * EG];
        s_p[tid] += s_p[tid + half * EG];
      }
      __syncthreads();
    }
    // thread el < EG now holds expert el's totals; terms and tile counts go to
    // slots 256 .. 256 + EG and 512 .. 512 + EG of s_off
    int32_t* s_nt = s_off + 512;
    double term = 0.0;
    int32_t nt = 0;
    if (tid < EG && tid < N) {
      const int32_t total = s_cnt[tid];
      const int32_t nk = (int32_t)((int64_t)total < C ? (int64_t)total : C);
      load[tid] = total;
      n_kept[tid] = nk;
      term = (double)total * s_p[tid];
      nt = (nk + tile_rows - 1) / tile_rows;
    }
    __syncthreads();
    if (tid < EG) {
      s_p[tid] = term;
      s_nt[tid] = nt;
    }
    __syncthreads();
    for (int half = EG >> 1; half >= 1; half >>= 1) {
      if (tid < half) s_p[tid] += s_p[tid + half];
      __syncthreads();
    }
    if (tid == 0) {
      double v = 0.0;
      if (T > 0) v = (double)alpha * (double)N * (s_p[0] / ((double)k * (double)T * (double)T));
      *aux = (float)v;
    }
    if (tile_start) {
      // inclusive scan of the tile counts over EG entries (Hillis-Steele)
      for (int off = 1; off < EG; off <<= 1) {
        const int32_t v = (tid < EG && tid >= off) ? s_nt[tid - off] : 0;
        __syncthreads();
        if (tid < EG) s_nt[tid] += v;
        __syncthreads();
      }
      if (tid < N) tile_start[tid] = s_nt[tid] - nt;
      if (tid == EG - 1) tile_start[N] = s_nt[tid];
    }
    return;
  }

  const int64_t t0 = (int64_t)(blockIdx.x - 1) * AS_TOK;
  const int64_t t1 = t0 + AS_TOK < T ? t0 + AS_TOK : T;
  const int64_t cb0 = t0 / chunk, cb1 = (t1 - 1) / chunk;
  const int ncb = (int)(cb1 - cb0 + 1);
  const int na = (int)(t1 - t0) * k;
  // every global read of the block is issued before the first barrier: the
  // block's assignments, its own chunks' counts, and the counts before cb0
  int32_t e_a = 0, r_a = 0;
  if (tid < na) {
    e_a = expert_idx[t0 * k + tid];
    r_a = rank_local[t0 * k + tid];
  }
  int32_t own[AS_MAXCH];
#pragma unroll
  for (int j = 0; j < AS_MAXCH; ++j)
    own[j] = (tid < N && j < ncb) ? hist[(cb0 + j) * N + tid] : 0;
  int32_t acc = 0;
  if (el < N) {
#pragma unroll 4
    for (int64_t c = g; c < cb0; c += G) acc += hist[c * N + el];
  }
  // tokens routed to each expert in the chunks before cb0
  int32_t* s_base = s_off + (AS_MAXCH - 1) * 256;  // reused once the walk has read it
  if (tid < N) s_base[tid] = 0;
  __syncthreads();
  if (el < N && acc) atomicAdd(&s_base[el], acc);
  __syncthreads();
  int32_t run = 0;
  if (tid < N) run = s_base[tid];
  __syncthreads();
  if (tid < N) {
#pragma unroll
    for (int j = 0; j < AS_MAXCH; ++j) {
      if (j < ncb) s_off[j * 256 + tid] = run;
      run += own[j];
    }
  }
  __syncthreads();
  if (tid < na) {
    const int64_t a = t0 * k + tid;
    const int64_t t = a / k;
    const int32_t pos = s_off[(int)(t / chunk - cb0) * 256 + e_a] + r_a;
    const bool dropped = (int64_t)pos >= C;
    position[a] = pos;
    drop_mask[a] = dropped ? 1 : 0;
    if (!dropped && tok) tok[(int64_t)e_a * C + pos] = (int32_t)t;
    s_e[tid] = e_a;
    s_pos[tid] = pos;
  }
  if (copy_mode == 0) return;
  __syncthreads();
  if (copy_mode == 1) {
    // top-1: a dropped token leaves the layer unchanged
    for (int idx = tid; idx < na * row_vec16; idx += 256) {
      const int i = idx / row_vec16, c = idx - i * row_vec16;
      if ((int64_t)s_pos[i] >= C) dst[(t0 + i) * row_vec16 + c] = x[(t0 + i) * row_vec16 + c];
    }
  } else {
    // kept assignments: the token's row into its expert slot
    for (int idx = tid; idx < na * row_vec16; idx += 256) {
      const int i = idx / row_vec16, c = idx - i * row_vec16;
      if ((int64_t)s_pos[i] < C)
        dst[((int64_t)s_e[i] * C + s_pos[i]) * row_vec16 + c] = x[(t0 + i / k) * row_vec16 + c];
    }
  }
}

// ------------------------------------------------------------------ launchers

void launch_route_scan(int32_t* hist, const float* P_part, int64_t nc, int N, int64_t T, int k,
                       int64_t C, float alpha, int32_t* load, int32_t* n_kept, double* terms,
                       float* aux, int32_t* tile_start, int tile_rows, hipStream_t s) {
  if (N <= 1024) {
    int EG = 1;
    while (EG < N) EG <<= 1;
    launch_k(route_scan_kernel, dim3(1), dim3(1024), 0, s, hist, P_part, nc, N, EG, T,
                       k, C, alpha, load, n_kept, nullptr, aux, tile_start, tile_rows);
    return;
  }
  // 32 experts per block: each row piece a thread group reads and rewrites is
  // one whole 128-byte line, with twice the blocks of 64 (64 at N = 2048)
  constexpr int EG = 32;
  launch_k(route_scan_kernel, dim3((unsigned)((N + EG - 1) / EG)), dim3(1024), 0, s,
                     hist, P_part, nc, N, EG, T, k, C, alpha, load, n_kept, terms, aux, nullptr,
                     tile_rows);
  launch_k(aux_kernel, dim3(1), dim3(1024), 0, s, terms, N, T, k, alpha, aux, n_kept,
                     tile_start, tile_rows);
}

void launch_finalize_positions(int64_t T, int k, const int32_t* expert_idx,
                               const int32_t* rank_local, const int32_t* offsets, int N,
                               int64_t chunk, int64_t C, int32_t* position, uint8_t* drop_mask,
                               hipStream_t s) {
  if (T == 0) return;
  const int64_t n = T * k;
  launch_k(finalize_positions_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                     s, T, k, expert_idx, rank_local, offsets, N, chunk, C, position, drop_mask);
}


bool assign_one_launch_ok(int N, int64_t nc, int64_t chunk) {
  return N >= 1 && N <= 256 && chunk >= 16 && nc * (int64_t)N <= kAssignMaxCells;
}

void launch_assign(const int32_t* hist, const float* P_part, int64_t nc, int N, int64_t T, int k,
                   int64_t chunk, int64_t C, float alpha, const int32_t* expert_idx,
                   const int32_t* rank_local, int32_t* load, int32_t* n_kept, float* aux,
                   int32_t* tile_start, int tile_rows, int32_t* position, uint8_t* drop_mask,
                   int32_t* tok, int copy_mode, int row_bytes, const void* x, void* dst,
                   hipStream_t s) {
  const int64_t nb = (T + AS_TOK - 1) / AS_TOK;
  launch_k(assign_kernel, dim3((unsigned)(nb + 1)), dim3(256), 0, s, hist, P_part, nc,
                     N, T, k, chunk, C, alpha, expert_idx, rank_local, load, n_kept, aux,
                     tile_start, tile_rows, position, drop_mask, tok, copy_mode, row_bytes / 16,
                     (const uint4*)x, (uint4*)dst);
}

}  // namespace swl
