// Grouped expert FFN matmuls.
//
// Each expert is the dense FFN it replaces (kasblo explainer, section
// "TransformerのどこへSwitch layerが入るのか"), here relu(x W_in^T) W_out^T with
// no biases; every expert multiplies the block of tokens gathered for it
// (section "tokenをExpertへ送って戻すforward pass").  Both matmuls have the
// same shape class, C[m, n] = sum_k A[m, k] B[n, k] with A and B K-contiguous:
//   GEMM1: A = Xbuf[e] [rows, d],  B = W_in[e]  [F, d] -> Hbuf[e] [rows, F], relu
//   GEMM2: A = Hbuf[e] [rows, F],  B = W_out[e] [d, F] -> Ybuf[e] [rows, d]
// The number of rows of expert e, n_kept[e], is read on the device: tiles past
// it return at once, so the host never waits for the routing result.
//
// On the bf16 path the token rows never move: GEMM1 reads the A rows of
// expert e straight from x through the slot table tok[e * C + m] (the dispatch
// of the kasblo explainer's forward pass becomes an indexed load), and GEMM2
// combines its output rows into out[t] = x[t] + gate[t] * y (the combine, with
// the gate multiply of llm-papers-study section 3.2 and the residual of its
// part 六 diagram) in its epilogue.
//
// bf16 path: CDNA4 MFMA v_mfma_f32_32x32x16_bf16, fp32 accumulation, the
// result rounded to bf16 (after the ReLU for GEMM1).  fp32 path: plain FMA.
#include <type_traits>

#include "epilogue.hpp"

namespace swl {

// Tile order: the grid is 1-D.  Workgroups are handed to the 8 XCDs round
// robin (block b runs on XCD b % 8), so block b takes tile
// (b % 8) * ceil(tiles / 8) + b / 8: each XCD walks a contiguous stretch of the
// tile list, whose order is expert, then N tile, then M tile.  The tiles of one
// expert (its gathered rows and its weights) therefore share one XCD's L2, and
// consecutive M tiles reuse the same weight tile.
//
// Block: 256 threads = 4 waves in a 2 x 2 grid; each wave owns a
// (BM/2) x (BN/2) sub-tile made of 32 x 32 MFMA tiles.  The launch bound asks
// for three waves per SIMD (three blocks per CU share the LDS and MFMA pipes).  K advances BK at a
// time through one padded LDS buffer per operand; the next K tile is fetched
// into registers (unconditionally: the last step re-reads its own tile) while
// the current one is multiplied.  BK is 128 for 64 x 128 tiles, which stream
// weights with few rows to reuse them: twice the bytes in flight per block
// (three blocks and 144 KB per CU) and 256 contiguous bytes of every weight
// row per step; 64 x 256 tiles (BKT = 64) move the same bytes per step over
// twice the columns, and 128-row tiles keep BK = 64 (their registers would not
// allow three blocks per CU at 128).  K is a multiple of 128 (the layer
// accepts bf16 shapes with d and F multiples of 128 only).
//
// MFMA 32x32x16 operand layout (per lane l): first operand row (l % 32) with 8
// consecutive k, second operand column (l % 32) with the same 8 k; the k group
// is (l / 32).  Result: lane l holds column (l % 32) and rows
// 8 (v / 4) + 4 (l / 32) + (v % 4), v < 16.  The first operand is the weight
// fragment, so those result rows are output columns (see stage_tile_bf16).
template <int BM, int BN, bool RELU, int MODE, bool NTW = false, int BKT = 0>
__global__ __launch_bounds__(256, 3) void gemm_bf16_kernel(const uint16_t* __restrict__ A,
                                                        int64_t strideA,
                                                        const uint16_t* __restrict__ B,
                                                        int64_t strideB,
                                                        uint16_t* __restrict__ Cout,
                                                        int64_t strideC,
                                                        const int32_t* __restrict__ rows, int K,
                                                        int Nout, int m_tiles, int n_tiles,
                                                        int tiles, GemmIO io, int64_t C) {
  if (y_prologue(io)) return;
  constexpr int BK = BKT ? BKT : (BM == 64 ? 128 : 64);
  constexpr int LDK = BK + GB_PAD;            // LDS row stride (bf16 elements)
  constexpr int TPR = BK / 8;                 // threads per row of a K tile (16 bytes each)
  constexpr int RP = 256 / TPR;               // rows per load pass
  constexpr int LA = BM / RP, LB = BN / RP;   // 16-byte loads per thread per operand
  constexpr int TI = BM / 64, TJ = BN / 64;   // MFMA tiles per wave
  // one buffer holding the A rows then the B rows; reused by the epilogue
  __shared__ __attribute__((aligned(16))) uint16_t lds[(BM + BN) * LDK];
  static_assert(4 * (BM / 2) * (BN / 2 + 8) <= (BM + BN) * LDK, "epilogue staging fits");
  uint16_t* As = lds;
  uint16_t* Bs = lds + BM * LDK;

  const int per_xcd = (tiles + 7) >> 3;
  const int tile = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (tile >= tiles) return;
  const int mt = tile % m_tiles;
  const int nt = (tile / m_tiles) % n_tiles;
  const int e = tile / (m_tiles * n_tiles);
  const int rows_e = rows ? rows[e] : (int)C;
  const int m0 = mt * BM;
  if (m0 >= rows_e) return;
  const int n0 = nt * BN;

  // GATHER: A is x itself and the rows come from the slot table
  const uint16_t* Ae = MODE == kRowsGather ? io.x : A + (int64_t)e * strideA;
  const uint16_t* Be = B + (int64_t)e * strideB + (int64_t)n0 * K;
  uint16_t* Ce = Cout + (int64_t)e * strideC;
  const int32_t* tok_e = MODE == kRowsDense ? nullptr : io.tok + (int64_t)e * C;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lrow = tid / TPR, lcol = (tid % TPR) * 8;

  int64_t a_off[LA], b_off[LB];
  u32x4 ra[LA], rb[LB];
  // the first K step's weight rows are requested before the slot-table reads
  // that the gathered A rows wait on
#pragma unroll
  for (int j = 0; j < LB; ++j) b_off[j] = (int64_t)(lrow + RP * j) * K + lcol;
#pragma unroll
  for (int j = 0; j < LB; ++j)
    rb[j] = NTW ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Be + b_off[j]))
                : *reinterpret_cast<const u32x4*>(Be + b_off[j]);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < LA; ++j) {
    int r = m0 + lrow + RP * j;
    r = r < rows_e ? r : rows_e - 1;  // rows past n_kept: any valid row, never stored
    const int64_t src = MODE == kRowsGather ? (int64_t)tok_e[r] : (int64_t)r;
    a_off[j] = src * K + lcol;
  }

  floatx16 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int last = K - BK;
  // The scheduling barrier keeps the prefetch loads ahead of the MFMAs that
  // follow; without it the compiler sinks them to the end of the loop body,
  // where nothing is left to hide their latency.
  auto fetch = [&](int k) {
    k = k < last ? k : last;
#pragma unroll
    for (int j = 0; j < LA; ++j) ra[j] = *reinterpret_cast<const u32x4*>(Ae + a_off[j] + k);
#pragma unroll
    for (int j = 0; j < LB; ++j)
      rb[j] = NTW ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Be + b_off[j] + k))
                  : *reinterpret_cast<const u32x4*>(Be + b_off[j] + k);
    __builtin_amdgcn_sched_barrier(0);
  };
  const int fr = lane & 31, fk = (lane >> 5) * 8;

  // the K loop for a wave whose first TV row tiles of 32 hold kept rows (the
  // MFMAs of row tiles wholly past n_kept are left out; every wave still loads
  // and stores its share of the operand tiles)
  auto kloop = [&](auto tv_const) {
    constexpr int TV = decltype(tv_const)::value;
#pragma unroll
    for (int j = 0; j < LA; ++j) ra[j] = *reinterpret_cast<const u32x4*>(Ae + a_off[j]);
    __builtin_amdgcn_sched_barrier(0);  // (rb holds step 0 already)
    for (int k0 = 0; k0 < K; k0 += BK) {
      __syncthreads();
#pragma unroll
      for (int j = 0; j < LA; ++j)
        *reinterpret_cast<u32x4*>(&As[(lrow + RP * j) * LDK + lcol]) = ra[j];
#pragma unroll
      for (int j = 0; j < LB; ++j)
        *reinterpret_cast<u32x4*>(&Bs[(lrow + RP * j) * LDK + lcol]) = rb[j];
      __syncthreads();
      fetch(k0 + BK);
      if (TV == 0) continue;
#pragma unroll
      for (int ks = 0; ks < BK; ks += 16) {
        bf16x8 a[TI], b[TJ];
#pragma unroll
        for (int i = 0; i < TV; ++i)
          a[i] = *reinterpret_cast<const bf16x8*>(
              &As[(wm * (BM / 2) + i * 32 + fr) * LDK + ks + fk]);
#pragma unroll
        for (int j = 0; j < TJ; ++j)
          b[j] = *reinterpret_cast<const bf16x8*>(
              &Bs[(wn * (BN / 2) + j * 32 + fr) * LDK + ks + fk]);
#pragma unroll
        for (int i = 0; i < TV; ++i)
#pragma unroll
          for (int j = 0; j < TJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], a[i], acc[i][j], 0, 0, 0);
      }
    }
  };
  int tv = (rows_e - (m0 + wm * (BM / 2)) + 31) / 32;
  tv = tv < 0 ? 0 : (tv > TI ? TI : tv);
  static_assert(TI == 1 || TI == 2, "row tiles per wave");
  if (tv >= TI) kloop(std::integral_constant<int, TI>{});
  else if (TI == 2 && tv == 1) kloop(std::integral_constant<int, (TI == 2 ? 1 : 0)>{});
  else kloop(std::integral_constant<int, 0>{});

  __syncthreads();  // every wave is done with the LDS operand tiles
  if (MODE == kRowsCombine)
    store_tile_combine<TI, TJ>(acc, lds + wave * (BM / 2) * (BN / 2 + 8), tok_e, io.x, io.gate,
                               io.out, m0 + wm * (BM / 2), n0 + wn * (BN / 2), rows_e, Nout, lane,
                               ykeep_at(io, e, C, m0 + wm * (BM / 2), n0 + wn * (BN / 2), Nout));
  else if (MODE == kRowsMask)
    store_tile_bf16<TI, TJ, false, true>(acc, lds + wave * (BM / 2) * (BN / 2 + 8), Ce,
                                         m0 + wm * (BM / 2), n0 + wn * (BN / 2), rows_e, Nout,
                                         lane, io.mask + (int64_t)e * strideC);
  else
    store_tile_bf16<TI, TJ, RELU>(acc, lds + wave * (BM / 2) * (BN / 2 + 8), Ce,
                                  m0 + wm * (BM / 2), n0 + wn * (BN / 2), rows_e, Nout, lane);
}

// Wide variant for experts with many rows (the Switch-Base shape, about 512
// rows per expert): a 256 x 256 tile, 8 waves in a 2 x 4 grid, each wave
// 128 x 64 (4 x 2 MFMA tiles).  Against 128 x 128 it halves the operand bytes
// each CU must load per MFMA, which is what bounds these grouped matmuls.
// Two padded LDS buffers (one barrier per K step of 64); the loads of step
// k + 2 and the LDS stores of step k + 1 are spread over the MFMAs of step k.
// Tiles come from the compact list io.tile_start (prefix over experts of their
// 256-row M tiles, from the routing scan): block b takes list entry
// (b % 8) * ceil(total / 8) + b / 8, so each XCD walks one stretch of the list
// (order expert, N tile, M tile), and a grid sized for full capacity leaves
// its extra blocks idle.  No XCD gets more tiles than its share.  Without a
// list every expert has the full count of M tiles (the weight-gradient
// matmuls, whose rows are all valid).  Epilogue modes: plain (optional ReLU)
// and the ReLU-derivative mask of the backward pass.
// Issue order inside a K sub-step of the wide kernel: each of the first six
// MFMAs is followed by one fragment read for the next sub-step, the last two
// by this sub-step's NW LDS stores and NL global loads (about 3% faster than
// leaving the order to the compiler within each sub-step).
template <int NW, int NL>
__device__ __forceinline__ void sched_substep() {
#pragma unroll
  for (int i = 0; i < 6; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x200, (NW + 1) / 2, 0);  // LDS write
  __builtin_amdgcn_sched_group_barrier(0x020, (NL + 1) / 2, 0);  // global load
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x200, NW / 2, 0);
  __builtin_amdgcn_sched_group_barrier(0x020, NL / 2, 0);
  __builtin_amdgcn_sched_barrier(0);
}

// The same interleave for a wave that multiplies only part of its row tiles
// (NM MFMAs and NR fragment reads per K sub-step): MFMA / read pairs while both
// last, then the stores and loads split over the last two MFMAs.
template <int NM, int NR, int NW, int NL>
__device__ __forceinline__ void sched_substep_n() {
  constexpr int P = NM - 2 < NR ? NM - 2 : NR;
#pragma unroll
  for (int i = 0; i < P; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
  }
  if (NM >= 2) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x200, (NW + 1) / 2, 0);  // LDS write
    __builtin_amdgcn_sched_group_barrier(0x020, (NL + 1) / 2, 0);  // global load
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x200, NW / 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x020, NL / 2, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// After a K step's barrier: the previous sub-step's MFMAs with this step's
// first fragment reads (TV + 2 of them) between them.
template <int TV>
__device__ __forceinline__ void sched_tail_tv() {
  constexpr int NM = 2 * TV, NR = TV > 0 ? TV + 2 : 0;
#pragma unroll
  for (int i = 0; i < (NM < NR ? NM : NR); ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
  }
  __builtin_amdgcn_sched_barrier(0);
}

template <int TV, int NW, int NL>
__device__ __forceinline__ void sched_substep_tv() {
  if constexpr (TV == 4) sched_substep<NW, NL>();
  else sched_substep_n<2 * TV, (TV > 0 ? TV + 2 : 0), NW, NL>();
}

constexpr int GW_BM = 256, GW_BN = 256;
constexpr size_t kWideLds = (size_t)2 * (GW_BM + GW_BN) * GB_LDK * sizeof(uint16_t);

template <bool RELU, int MODE>
__global__ __launch_bounds__(512, 1) void gemm_bf16_wide_kernel(
    const uint16_t* __restrict__ A, int64_t strideA, const uint16_t* __restrict__ B,
    int64_t strideB, uint16_t* __restrict__ Cout, int64_t strideC,
    const int32_t* __restrict__ rows, int K, int Nout, int m_tiles, int n_tiles, int tiles,
    GemmIO io, int64_t C, int n_exp) {
  if (y_prologue(io)) return;
  constexpr int BM = GW_BM, BN = GW_BN, BK = GB_BK, LDK = GB_LDK;
  constexpr int TI = 4, TJ = 2;
  constexpr int STAGE = (BM + BN) * LDK;
  constexpr int NL = 8;  // 16-byte loads per thread per K step: 4 of A, 4 of B
  static_assert(8 * 128 * (64 + 8) * sizeof(uint16_t) <= kWideLds, "epilogue staging fits");
  extern __shared__ __attribute__((aligned(16))) uint16_t wlds[];
  (void)m_tiles;
  (void)tiles;

  const int32_t* ts = io.tile_start;
  int e, me, local, tile;
  if (ts) {
    const int total = ts[n_exp] * n_tiles;
    const int per_xcd = (total + 7) >> 3;
    tile = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if ((int)(blockIdx.x >> 3) >= per_xcd || tile >= total) return;
    // expert: the last e with ts[e] * n_tiles <= tile (it has M tiles)
    int lo = 0, hi = n_exp - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (ts[mid] * n_tiles <= tile) lo = mid; else hi = mid - 1;
    }
    e = lo;
    me = ts[e + 1] - ts[e];
    local = tile - ts[e] * n_tiles;
  } else {
    // no tile list: every expert has m_tiles M tiles (rows past its count return)
    const int per_xcd = (tiles + 7) >> 3;
    tile = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if (tile >= tiles) return;
    me = m_tiles;
    e = tile / (m_tiles * n_tiles);
    local = tile - e * m_tiles * n_tiles;
  }
  const int nt = local / me;
  const int mt = local - nt * me;
  const int rows_e = rows ? rows[e] : (int)C;
  const int m0 = mt * BM;
  if (m0 >= rows_e) return;
  const int n0 = nt * BN;

  const uint16_t* Ae = MODE == kRowsGather ? io.x : A + (int64_t)e * strideA;
  const uint16_t* Be = B + (int64_t)e * strideB + (int64_t)n0 * K;
  uint16_t* Ce = Cout + (int64_t)e * strideC;
  const int32_t* tok_e =
      MODE == kRowsGather || MODE == kRowsCombine ? io.tok + (int64_t)e * C : nullptr;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int lrow = tid >> 3, lcol = (tid & 7) * 8;  // 64 rows per pass of 512 threads

  int64_t go[NL];  // element offsets: A rows (j < 4) from Ae, B rows (j >= 4) from Be
  u32x4 g[NL];
  // the first K step's weight rows are requested before the slot-table reads
  // that the gathered A rows wait on (1-4% off the matmuls at the Switch-Base
  // and Switch-Large shapes, same bits)
#pragma unroll
  for (int j = 0; j < 4; ++j) go[4 + j] = (int64_t)(lrow + 64 * j) * K + lcol;
#pragma unroll
  for (int j = 4; j < NL; ++j) g[j] = *reinterpret_cast<const u32x4*>(Be + go[j]);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int r = m0 + lrow + 64 * j;
    r = r < rows_e ? r : rows_e - 1;  // rows past n_kept: any valid row, never stored
    const int64_t src = MODE == kRowsGather ? (int64_t)tok_e[r] : (int64_t)r;
    go[j] = src * K + lcol;
  }
  const int lbase = lrow * LDK + lcol;
  const int nk = K / BK;
  auto gload = [&](int j0, int j1, int t) {
    t = t < nk ? t : nk - 1;
    const int k = t * BK;
#pragma unroll
    for (int j = j0; j < j1; ++j)
      g[j] = *reinterpret_cast<const u32x4*>((j < 4 ? Ae : Be) + go[j] + k);
  };
  auto gstore = [&](int j0, int j1, int buf) {
#pragma unroll
    for (int j = j0; j < j1; ++j)
      *reinterpret_cast<u32x4*>(
          &wlds[buf * STAGE + lbase + ((j & 3) * 64 + (j < 4 ? 0 : BM)) * LDK]) = g[j];
  };
  floatx16 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  const int fr = lane & 31, fk = (lane >> 5) * 8;
  bf16x8 fa[2][TI], fb[2][TJ];

  // The K loop for a wave whose first TV row tiles of 32 hold kept rows: the
  // MFMAs (and fragment reads) of row tiles wholly past n_kept are left out, so
  // the short last M tile of an expert costs MFMA time for its kept rows only;
  // every wave still loads and stores its share of the operand tiles and meets
  // every barrier.
  auto kloop = [&](auto tv_const) {
    constexpr int TV = decltype(tv_const)::value;
    auto frags = [&](int f, int buf, int ks) {
      if (TV == 0) return;
#pragma unroll
      for (int i = 0; i < TV; ++i)
        fa[f][i] = *reinterpret_cast<const bf16x8*>(
            &wlds[buf * STAGE + (wm * 128 + i * 32 + fr) * LDK + ks * 16 + fk]);
#pragma unroll
      for (int j = 0; j < TJ; ++j)
        fb[f][j] = *reinterpret_cast<const bf16x8*>(
            &wlds[buf * STAGE + (BM + wn * 64 + j * 32 + fr) * LDK + ks * 16 + fk]);
    };
    auto mfmas = [&](int f) {
#pragma unroll
      for (int i = 0; i < TV; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
          acc[i][j] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[f][j], fa[f][i], acc[i][j], 0, 0, 0);
    };

    gload(0, 4, 0);  // the weight rows of step 0 are already on their way
    gstore(0, NL, 0);
    gload(0, NL, 1);
    __syncthreads();
    frags(0, 0, 0);
    for (int t = 0; t < nk; ++t) {
      const int cur = t & 1, nxt = cur ^ 1;
      // buffer nxt was last read in step t - 1, before the barrier that ended it
      frags(1, cur, 1);
      gstore(0, 3, nxt);
      gload(0, 3, t + 2);
      mfmas(0);
      sched_substep_tv<TV, 3, 3>();
      frags(0, cur, 2);
      gstore(3, 6, nxt);
      gload(3, 6, t + 2);
      mfmas(1);
      sched_substep_tv<TV, 3, 3>();
      frags(1, cur, 3);
      gstore(6, 8, nxt);
      gload(6, 8, t + 2);
      mfmas(0);
      sched_substep_tv<TV, 2, 2>();
      // the last sub-step's MFMAs go after the barrier (their fragments are in
      // registers), so the matrix pipe has work while the next step's first
      // fragments arrive
      __syncthreads();
      frags(0, nxt, 0);
      mfmas(1);
      sched_tail_tv<TV>();
    }
  };
  int tv = (rows_e - (m0 + wm * 128) + 31) / 32;
  tv = tv < 0 ? 0 : (tv > TI ? TI : tv);
  static_assert(TI == 4, "row tiles per wave");
  switch (tv) {
    case 4: kloop(std::integral_constant<int, 4>{}); break;
    case 3: kloop(std::integral_constant<int, 3>{}); break;
    case 2: kloop(std::integral_constant<int, 2>{}); break;
    case 1: kloop(std::integral_constant<int, 1>{}); break;
    default: kloop(std::integral_constant<int, 0>{}); break;
  }

  __syncthreads();  // every wave is done with the LDS operand buffers
  uint16_t* stage = wlds + wave * 128 * (64 + 8);
  if (MODE == kRowsCombine) {
    // the accumulators go to LDS first, so the residual rows and gates fetched
    // next do not have to share the registers with them
    stage_tile_bf16<TI, TJ, CombineRows<TI, TJ>::LD, false>(acc, stage, lane);
    CombineRows<TI, TJ> cr;
    combine_prefetch<TI, TJ>(cr, tok_e, io.x, io.gate, m0 + wm * 128, n0 + wn * 64, rows_e,
                             Nout, lane);
    combine_from_stage<TI, TJ>(stage, cr, io.out, lane,
                               ykeep_at(io, e, C, m0 + wm * 128, n0 + wn * 64, Nout), Nout);
  } else if (MODE == kRowsMask)
    store_tile_bf16<TI, TJ, false, true>(acc, stage, Ce, m0 + wm * 128, n0 + wn * 64, rows_e,
                                         Nout, lane, io.mask + (int64_t)e * strideC);
  else
    store_tile_bf16<TI, TJ, RELU>(acc, stage, Ce, m0 + wm * 128, n0 + wn * 64, rows_e, Nout,
                                  lane);
}


template <int R, int NTHR, bool KOUTER>
struct OpLayout {
  static constexpr int PITCH = KOUTER ? R + KO_PAD : GB_LDK;      // LDS row pitch (elements)
  static constexpr int ELEMS = KOUTER ? GB_BK * PITCH : R * GB_LDK;
  static constexpr int P = R * GB_BK / 8 / NTHR;                   // 16-byte pieces per thread
  // K-contiguous: thread -> (row, 8-wide k chunk); K-outer: (k row, 8-wide column chunk)
  static constexpr int CPR = KOUTER ? R / 8 : GB_BK / 8;          // chunks per LDS row
  static constexpr int RPP = NTHR / CPR;                           // LDS rows per pass
  static_assert(P * NTHR * 8 == R * GB_BK && RPP * CPR == NTHR, "whole passes");
};


// Split-K variant of the 128 x 128 tile for launches with no more tiles than
// CUs (the Switch-Base GEMM2 shape: about 240 tiles, K = 3072), where one
// four-wave block per CU leaves the MFMA pipes idle while each wave waits on
// LDS and barriers.  Eight waves, two per SIMD: waves 0-3 and 4-7 form two
// groups owning the same 2 x 2 grid of 64 x 64 wave tiles; in every 64-wide K
// step group 0 multiplies K sub-steps 0 and 1, group 1 sub-steps 2 and 3.  Two
// LDS operand buffers, one barrier per step, the loads of step t + 2 in flight
// during step t.  At the end the groups exchange halves of their fp32 partial
// sums through LDS and each finishes half of the rows (epilogue included).
// BKO: B stored K-outer ([K][Nout] per expert, pitch io.ldb; the backward's
// dX = dU W_in[e]).
constexpr size_t kSplitRed = (size_t)8 * 8 * 64 * 16;              // bytes of partial sums
constexpr size_t kSplitLds = kSplitRed + (size_t)8 * 32 * (64 + 8) * sizeof(uint16_t);

template <bool RELU, int MODE, bool BKO = false>
__global__ __launch_bounds__(512, 1) void gemm_bf16_split_kernel(
    const uint16_t* __restrict__ A, int64_t strideA, const uint16_t* __restrict__ B,
    int64_t strideB, uint16_t* __restrict__ Cout, int64_t strideC,
    const int32_t* __restrict__ rows, int K, int Nout, int m_tiles, int n_tiles, int tiles,
    GemmIO io, int64_t C) {
  if (y_prologue(io)) return;
  constexpr int BM = 128, BN = 128, BK = GB_BK, LDK = GB_LDK, TI = 2, TJ = 2;
  using LB = OpLayout<BN, 512, BKO>;
  constexpr int GS_STAGE = BM * GB_LDK + LB::ELEMS;                 // elements per buffer
  static_assert(2 * GS_STAGE * sizeof(uint16_t) <= kSplitLds, "operand buffers fit");
  static_assert(kSplitRed <= 2 * GS_STAGE * sizeof(uint16_t), "partial sums reuse the buffers");
  extern __shared__ __attribute__((aligned(16))) uint16_t slds[];

  const int per_xcd = (tiles + 7) >> 3;
  const int tile = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (tile >= tiles) return;
  const int mt = tile % m_tiles;
  const int nt = (tile / m_tiles) % n_tiles;
  const int e = tile / (m_tiles * n_tiles);
  const int rows_e = rows ? rows[e] : (int)C;
  const int m0 = mt * BM;
  if (m0 >= rows_e) return;
  const int n0 = nt * BN;

  const uint16_t* Ae = MODE == kRowsGather ? io.x : A + (int64_t)e * strideA;
  const uint16_t* Be = B + (int64_t)e * strideB + (BKO ? (int64_t)n0 : (int64_t)n0 * K);
  uint16_t* Ce = Cout + (int64_t)e * strideC;
  const int32_t* tok_e = MODE == kRowsDense ? nullptr : io.tok + (int64_t)e * C;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int grp = wave >> 2, wq = wave & 3, wm = wq >> 1, wn = wq & 1;
  const int lrow = tid >> 3, lcol = (tid & 7) * 8;  // 64 rows per pass of 512 threads

  // element offsets: A rows (j < 2) from Ae, B pieces (j >= 2) from Be; LDS offsets
  int64_t go[4];
  int lo_[4];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    int r = m0 + lrow + 64 * j;
    r = r < rows_e ? r : rows_e - 1;  // rows past n_kept: any valid row, never stored
    const int64_t src = MODE == kRowsGather ? (int64_t)tok_e[r] : (int64_t)r;
    go[j] = src * K + lcol;
    lo_[j] = (lrow + 64 * j) * LDK + lcol;
    if (BKO) {
      // K-outer B: k row tid / 16 + 32 j, columns 8 (tid % 16) .. + 7
      const int kr = tid / LB::CPR + LB::RPP * j, c = (tid % LB::CPR) * 8;
      go[2 + j] = (int64_t)kr * io.ldb + c;
      lo_[2 + j] = BM * LDK + kr * LB::PITCH + c;
    } else {
      go[2 + j] = (int64_t)(lrow + 64 * j) * K + lcol;
      lo_[2 + j] = BM * LDK + (lrow + 64 * j) * LDK + lcol;
    }
  }
  static_assert(LB::P == 2, "two B pieces per thread");
  const int nk = K / BK;
  const int64_t b_step = BKO ? (int64_t)BK * io.ldb : BK;
  u32x4 g[4];
  auto gload = [&](int t) {
    t = t < nk ? t : nk - 1;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      g[j] = j < 2 ? *reinterpret_cast<const u32x4*>(Ae + go[j] + (int64_t)t * BK)
                   : *reinterpret_cast<const u32x4*>(Be + go[j] + t * b_step);
  };
  auto gstore = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<u32x4*>(&slds[buf * GS_STAGE + lo_[j]]) = g[j];
  };
  floatx16 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  const int fr = lane & 31, fk = (lane >> 5) * 8;
  bf16x8 fa[2][TI], fb[2][TJ];
  auto frags = [&](int f, int buf, int ks) {
#pragma unroll
    for (int i = 0; i < TI; ++i)
      fa[f][i] = *reinterpret_cast<const bf16x8*>(
          &slds[buf * GS_STAGE + (wm * 64 + i * 32 + fr) * LDK + ks * 16 + fk]);
#pragma unroll
    for (int j = 0; j < TJ; ++j)
      fb[f][j] = BKO ? frag_kouter(slds + buf * GS_STAGE + BM * LDK, LB::PITCH, ks,
                                   wn * 64 + j * 32, lane)
                     : *reinterpret_cast<const bf16x8*>(
                           &slds[buf * GS_STAGE + (BM + wn * 64 + j * 32 + fr) * LDK + ks * 16 +
                                 fk]);
  };
  auto mfmas = [&](int f) {
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[f][j], fa[f][i], acc[i][j], 0, 0, 0);
  };

  const int ks0 = 2 * grp;
  gload(0);
  gstore(0);
  gload(1);
  __syncthreads();
  for (int t = 0; t < nk; ++t) {
    const int cur = t & 1, nxt = cur ^ 1;
    // buffer nxt was last read in step t - 1, before the barrier that ended it
    frags(0, cur, ks0);
    frags(1, cur, ks0 + 1);
    // all eight MFMAs go out before the waits for the LDS stores: the first
    // sub-step's fragment reads, then MFMAs each followed by reads of the
    // second sub-step, then MFMAs each followed by one LDS store and one load
    // (the compiler's own order waited on the loads after three MFMAs; this
    // one is 4% faster at the Switch-Base GEMM2 and 8% at the backward's dX).
    // A fragment of a K-outer B takes two transposing reads.
    constexpr int RF = TI + (BKO ? 2 : 1) * TJ;  // LDS reads per sub-step
    mfmas(0);
    mfmas(1);
    gstore(nxt);
    gload(t + 2);
    __builtin_amdgcn_sched_group_barrier(0x100, RF, 0);  // LDS read
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, (RF + 3) / 4, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, (RF + 2) / 4, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, (RF + 1) / 4, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, RF / 4, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // LDS write
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // global load
    }
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
  }

  // The two groups finish one half of the tile each: group 0 the first MFMA
  // row tile (i = 0) of its wave tile, group 1 the second.  Each hands the
  // other half of its partial sums over through LDS, laid out
  // [wave][j][q][lane][4 floats] so that every 16-byte LDS access of a wave
  // covers consecutive addresses, and adds the half it receives to its own
  // (fp32 addition commutes, so the sum is the same whichever group adds).
  float* red = reinterpret_cast<float*>(slds);
  auto send = [&](const floatx16 (&a)[TJ]) {
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 v = {a[j][4 * q], a[j][4 * q + 1], a[j][4 * q + 2], a[j][4 * q + 3]};
        *reinterpret_cast<float4*>(red + ((wave * TJ * 4 + j * 4 + q) * 64 + lane) * 4) = v;
      }
  };
  // group g's partner wave is wave ^ 4 (same wave tile, other group)
  auto take = [&](floatx16 (&a)[TJ]) {
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 v = *reinterpret_cast<const float4*>(
            red + (((wave ^ 4) * TJ * 4 + j * 4 + q) * 64 + lane) * 4);
        a[j][4 * q] += v.x;
        a[j][4 * q + 1] += v.y;
        a[j][4 * q + 2] += v.z;
        a[j][4 * q + 3] += v.w;
      }
  };
  static_assert((size_t)8 * TJ * 4 * 64 * 16 <= kSplitRed, "partial sums fit");
  // the combine's reads go out before the exchange
  const int rh = m0 + wm * 64 + grp * 32, ch0 = n0 + wn * 64;
  CombineRows<1, TJ> cr;
  if (MODE == kRowsCombine)
    combine_prefetch<1, TJ>(cr, tok_e, io.x, io.gate, rh, ch0, rows_e, Nout, lane);
  if (grp == 0) send(acc[1]); else send(acc[0]);
  __syncthreads();
  // epilogue staging lies past the partial sums: 32 rows of 64 + 8 bf16 per wave
  uint16_t* stage = slds + kSplitRed / sizeof(uint16_t) + wave * 32 * (64 + 8);
  auto finish = [&](floatx16 (&a)[TJ], int half) {
    take(a);
    floatx16 (&t)[1][TJ] = *reinterpret_cast<floatx16 (*)[1][TJ]>(&a);
    const int r0 = m0 + wm * 64 + half * 32, c0 = n0 + wn * 64;
    if (MODE == kRowsCombine)
      store_tile_combine<1, TJ>(t, stage, cr, io.out, lane, ykeep_at(io, e, C, r0, c0, Nout),
                                Nout);
    else if (MODE == kRowsMask)
      store_tile_bf16<1, TJ, false, true>(t, stage, Ce, r0, c0, rows_e, Nout, lane,
                                          io.mask + (int64_t)e * strideC);
    else
      store_tile_bf16<1, TJ, RELU>(t, stage, Ce, r0, c0, rows_e, Nout, lane);
  };
  if (grp == 0) finish(acc[0], 0); else finish(acc[1], 1);
}

// ---------------------------------------------------------------------------
// Grouped matmul with operands in either layout, for the backward pass, where
// the products contract over a dimension that is not innermost in memory:
// dU = Gs W_out[e] and dX = dU W_in[e] read the weights as stored ([K][N], N
// innermost), dW_out = Gs^T H and dW_in = dU^T X read activations [rows][*]
// with the rows as K.  A K-outer operand tile is staged in LDS as stored
// ([64 k][R + 8] per K step, 16-byte row pieces) and its MFMA fragments come
// from ds_read_b64_tr_b16: in each group of 16 lanes, source lane 4 q + p
// addresses row q and columns 4 p .. 4 p + 3 of a 4 x 16 block and lane i
// receives column i of rows 0..3, so two such reads give a lane its column's
// 8 consecutive k.  K-contiguous operands are staged as in the kernels above.
//
// Tile BM x BN with BN / 64 x 2 waves, each (BM / 2) x 64; at 256 x 256 two
// LDS operand buffers, one barrier per K step, the loads of step t + 2 in
// flight during step t (at 128 x 128 see t_buffers); tile order as the wide
// kernel (compact list, or every expert at full capacity). Rows of a K-outer
// operand at or past io.krows[e] read as zero (the expert's rows beyond its
// kept count).
// ---------------------------------------------------------------------------

// The 128 x 128 form stages through one LDS buffer (two barriers per K step,
// the next step's loads in registers) so that three blocks fit on a CU.
template <int BM, int BN>
constexpr int t_buffers() { return BM == 128 ? 1 : 2; }

template <int BM, int BN, bool AKO, bool BKO, bool RELU, int MODE>
__global__ __launch_bounds__(BN * 2, BM == 128 ? 3 : 1) void gemm_bf16_t_kernel(
    const uint16_t* __restrict__ A, int64_t strideA, const uint16_t* __restrict__ B,
    int64_t strideB, uint16_t* __restrict__ Cout, int64_t strideC,
    const int32_t* __restrict__ rows, int K, int Nout, int m_tiles, int n_tiles, int tiles,
    GemmIO io, int64_t C, int n_exp) {
  constexpr int NTHR = BN * 2, WN = BN / 64, TI = BM / 64, TJ = 2;
  using LA = OpLayout<BM, NTHR, AKO>;
  using LB = OpLayout<BN, NTHR, BKO>;
  constexpr int STAGE = LA::ELEMS + LB::ELEMS;
  static_assert(MODE == kRowsDense || MODE == kRowsMask, "plain or masked epilogue");
  extern __shared__ __attribute__((aligned(16))) uint16_t tlds[];

  const int32_t* ts = io.tile_start;
  int e, me, local, tile;
  if (ts) {
    const int total = ts[n_exp] * n_tiles;
    const int per_xcd = (total + 7) >> 3;
    tile = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if ((int)(blockIdx.x >> 3) >= per_xcd || tile >= total) return;
    int lo = 0, hi = n_exp - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (ts[mid] * n_tiles <= tile) lo = mid; else hi = mid - 1;
    }
    e = lo;
    me = ts[e + 1] - ts[e];
    local = tile - ts[e] * n_tiles;
  } else {
    const int per_xcd = (tiles + 7) >> 3;
    tile = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if (tile >= tiles) return;
    me = m_tiles;
    e = tile / (m_tiles * n_tiles);
    local = tile - e * m_tiles * n_tiles;
  }
  const int nt = local / me;
  const int mt = local - nt * me;
  const int rows_e = rows ? rows[e] : (int)C;
  const int m0 = mt * BM;
  if (m0 >= rows_e) return;
  const int n0 = nt * BN;
  const int krows = io.krows ? io.krows[e] : K;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int nk = K / GB_BK;

  // global element offsets of this thread's pieces at K step 0 and their LDS
  // offsets; a K-outer piece also records its k row (for the krows test)
  const uint16_t* Ae = A + (int64_t)e * strideA;
  const uint16_t* Be = B + (int64_t)e * strideB;
  int64_t ga[LA::P], gb[LB::P];
  int la[LA::P], lb[LB::P], ka[LA::P], kb[LB::P];
  const int64_t a_step = AKO ? (int64_t)GB_BK * io.lda : GB_BK;
  const int64_t b_step = BKO ? (int64_t)GB_BK * io.ldb : GB_BK;
#pragma unroll
  for (int j = 0; j < LA::P; ++j) {
    const int r = tid / LA::CPR + LA::RPP * j, c = (tid % LA::CPR) * 8;
    if (AKO) {
      ga[j] = (int64_t)r * io.lda + m0 + c;
      ka[j] = r;
    } else {
      int row = m0 + r;
      row = row < rows_e ? row : rows_e - 1;  // rows past the count: any valid row, never stored
      ga[j] = (int64_t)row * K + c;
      ka[j] = 0;
    }
    la[j] = r * LA::PITCH + c;
  }
#pragma unroll
  for (int j = 0; j < LB::P; ++j) {
    const int r = tid / LB::CPR + LB::RPP * j, c = (tid % LB::CPR) * 8;
    if (BKO) {
      gb[j] = (int64_t)r * io.ldb + n0 + c;
      kb[j] = r;
    } else {
      gb[j] = (int64_t)(n0 + r) * K + c;
      kb[j] = 0;
    }
    lb[j] = r * LB::PITCH + c;
  }
  u32x4 ra[LA::P], rb[LB::P];
  auto gload = [&](int t) {
    t = t < nk ? t : nk - 1;
#pragma unroll
    for (int j = 0; j < LA::P; ++j)
      ra[j] = (!AKO || t * GB_BK + ka[j] < krows)
                  ? *reinterpret_cast<const u32x4*>(Ae + ga[j] + t * a_step)
                  : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < LB::P; ++j)
      rb[j] = (!BKO || t * GB_BK + kb[j] < krows)
                  ? *reinterpret_cast<const u32x4*>(Be + gb[j] + t * b_step)
                  : u32x4{0u, 0u, 0u, 0u};
  };
  auto gstore = [&](int buf) {
#pragma unroll
    for (int j = 0; j < LA::P; ++j)
      *reinterpret_cast<u32x4*>(&tlds[buf * STAGE + la[j]]) = ra[j];
#pragma unroll
    for (int j = 0; j < LB::P; ++j)
      *reinterpret_cast<u32x4*>(&tlds[buf * STAGE + LA::ELEMS + lb[j]]) = rb[j];
  };
  floatx16 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  const int fr = lane & 31, fk = (lane >> 5) * 8;
  auto step = [&](int buf) {
    const uint16_t* At = tlds + buf * STAGE;
    const uint16_t* Bt = At + LA::ELEMS;
#pragma unroll
    for (int ks = 0; ks < GB_BK / 16; ++ks) {
      bf16x8 a[TI], b[TJ];
#pragma unroll
      for (int i = 0; i < TI; ++i)
        a[i] = AKO ? frag_kouter(At, LA::PITCH, ks, wm * (BM / 2) + i * 32, lane)
                   : *reinterpret_cast<const bf16x8*>(
                         &At[(wm * (BM / 2) + i * 32 + fr) * LA::PITCH + ks * 16 + fk]);
#pragma unroll
      for (int j = 0; j < TJ; ++j)
        b[j] = BKO ? frag_kouter(Bt, LB::PITCH, ks, wn * 64 + j * 32, lane)
                   : *reinterpret_cast<const bf16x8*>(
                         &Bt[(wn * 64 + j * 32 + fr) * LB::PITCH + ks * 16 + fk]);
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], a[i], acc[i][j], 0, 0, 0);
    }
  };

  if (t_buffers<BM, BN>() == 1) {
    gload(0);
    for (int t = 0; t < nk; ++t) {
      __syncthreads();  // every wave is done with step t - 1's tile
      gstore(0);
      __syncthreads();
      gload(t + 1);
      step(0);
    }
    __syncthreads();
  } else {
    gload(0);
    gstore(0);
    gload(1);
    __syncthreads();
    for (int t = 0; t < nk; ++t) {
      const int cur = t & 1, nxt = cur ^ 1;
      // buffer nxt was last read in step t - 1, before the barrier that ended it
      gstore(nxt);
      gload(t + 2);
      step(cur);
      __syncthreads();
    }
  }

  uint16_t* stage = tlds + wave * (BM / 2) * (64 + 8);
  uint16_t* Ce = Cout + (int64_t)e * strideC;
  if (MODE == kRowsMask)
    store_tile_bf16<TI, TJ, false, true>(acc, stage, Ce, m0 + wm * (BM / 2), n0 + wn * 64, rows_e,
                                         Nout, lane, io.mask + (int64_t)e * strideC);
  else
    store_tile_bf16<TI, TJ, RELU>(acc, stage, Ce, m0 + wm * (BM / 2), n0 + wn * 64, rows_e, Nout,
                                  lane);
}

template <int BM, int BN, bool AKO, bool BKO>
constexpr size_t t_kernel_lds() {
  constexpr size_t ops = (size_t)t_buffers<BM, BN>() *
                         (OpLayout<BM, BN * 2, AKO>::ELEMS + OpLayout<BN, BN * 2, BKO>::ELEMS);
  constexpr size_t epi = (size_t)(BN / 64) * 2 * (BM / 2) * (64 + 8);
  return (ops > epi ? ops : epi) * sizeof(uint16_t);
}

// fp32 path (parity-sized fp32 layers): 32 x 32 tile, K in steps of 32, each
// of 256 threads owns 4 rows of one column.  Any sizes (bounds-checked).
template <bool RELU>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A, int64_t strideA,
                                                       const float* __restrict__ B, int64_t strideB,
                                                       float* __restrict__ Cout, int64_t strideC,
                                                       const int32_t* __restrict__ rows, int K,
                                                       int Nout) {
  __shared__ float As[32][33];
  __shared__ float Bs[32][33];
  const int e = blockIdx.z;
  const int rows_e = rows[e];
  const int m0 = blockIdx.y * 32;
  if (m0 >= rows_e) return;
  const int n0 = blockIdx.x * 32;
  const float* Ae = A + (int64_t)e * strideA;
  const float* Be = B + (int64_t)e * strideB;
  float* Ce = Cout + (int64_t)e * strideC;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < K; k0 += 32) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int idx = threadIdx.x + 256 * j;
      const int r = idx >> 5, k = idx & 31;
      const int gk = k0 + k;
      As[r][k] = (m0 + r < rows_e && gk < K) ? Ae[(int64_t)(m0 + r) * K + gk] : 0.f;
      Bs[r][k] = (n0 + r < Nout && gk < K) ? Be[(int64_t)(n0 + r) * K + gk] : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int k = 0; k < 32; ++k) {
      const float b = Bs[tx][k];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = fmaf(As[ty + 8 * i][k], b, acc[i]);
    }
    __syncthreads();
  }
  const int c = n0 + tx;
  if (c >= Nout) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = m0 + ty + 8 * i;
    if (r < rows_e) {
      float v = acc[i];
      if (RELU) v = v > 0.f ? v : 0.f;
      Ce[(int64_t)r * Nout + c] = v;
    }
  }
}

// ------------------------------------------------------------------ launchers

namespace {

// Compute units of the current device (cached per device).
int device_cus() {
  static int cus[64] = {};
  int dev = 0;
  (void)hipGetDevice(&dev);
  if (dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

// The wide tile pays off when N splits into 256-column tiles and the experts
// hold at least two of its M tiles; without a compact tile list (every expert
// at full capacity) also only with tiles for at least two rounds of CUs.
// one_tile (the forward-layout products): with the tile list, one full M tile
// of capacity suffices when the experts' tiles at full capacity would fill the
// CUs (at the Switch-Large shape, 188-320 rows per expert, both matmuls beat
// 128-row tiles despite the padding of the second M tile; at the Switch-Base
// second matmul, 72 tiles, the split-K kernel wins), while the backward's
// masked K-outer product is slower on them.
bool use_wide(int64_t C, int Nout, int n_experts, const GemmIO& io, bool one_tile = false) {
  static_assert(GW_BM == kWideTileRows, "tile list and kernel agree");
  const int64_t tiles = (C + GW_BM - 1) / GW_BM * (Nout / GW_BN) * n_experts;
  if (Nout % GW_BN != 0) return false;
  if (io.tile_start && one_tile) return C >= GW_BM && tiles >= device_cus();
  if (io.tile_start) return C >= 2 * GW_BM;
  return C >= 2 * GW_BM && tiles >= 2 * device_cus();
}

template <bool RELU, int MODE>
void launch_wide(const uint16_t* a, int64_t strideA, const uint16_t* b, int64_t strideB,
                 uint16_t* c, int64_t strideC, const int32_t* rows, int n_experts, int64_t C,
                 int K, int Nout, const GemmIO& io, hipStream_t s) {
  // kernels above 64 KiB of LDS must say so once per device
  static uint64_t set_on = 0;
  int dev = 0;
  (void)hipGetDevice(&dev);
  if (dev < 64 && !(set_on >> dev & 1)) {
    (void)hipFuncSetAttribute((const void*)gemm_bf16_wide_kernel<RELU, MODE>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)kWideLds);
    set_on |= 1ull << dev;
  }
  const int mt = (int)((C + GW_BM - 1) / GW_BM), nt = Nout / GW_BN;
  const int tiles = mt * nt * n_experts;
  const unsigned grid = (unsigned)(((tiles + 7) / 8) * 8);
  launch_k((gemm_bf16_wide_kernel<RELU, MODE>), dim3(grid), dim3(512), kWideLds, s, a,
                     strideA, b, strideB, c, strideC, rows, K, Nout, mt, nt, tiles, io, C,
                     n_experts);
}

template <bool RELU, int MODE, bool BKO = false>
void launch_split(unsigned grid, const uint16_t* a, int64_t strideA, const uint16_t* b,
                  int64_t strideB, uint16_t* c, int64_t strideC, const int32_t* rows, int K,
                  int Nout, int mt, int nt, int tiles, const GemmIO& io, int64_t C,
                  hipStream_t s) {
  static uint64_t set_on = 0;
  int dev = 0;
  (void)hipGetDevice(&dev);
  if (dev < 64 && !(set_on >> dev & 1)) {
    (void)hipFuncSetAttribute((const void*)gemm_bf16_split_kernel<RELU, MODE, BKO>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)kSplitLds);
    set_on |= 1ull << dev;
  }
  launch_k((gemm_bf16_split_kernel<RELU, MODE, BKO>), dim3(grid), dim3(512), kSplitLds,
                     s, a, strideA, b, strideB, c, strideC, rows, K, Nout, mt, nt, tiles, io, C);
}

template <int BM, int BN, bool AKO, bool BKO, bool RELU, int MODE>
void launch_t(const uint16_t* a, int64_t strideA, const uint16_t* b, int64_t strideB,
              uint16_t* c, int64_t strideC, const int32_t* rows, int n_experts, int64_t C, int K,
              int Nout, const GemmIO& io, hipStream_t s) {
  constexpr size_t lds = t_kernel_lds<BM, BN, AKO, BKO>();
  auto kern = gemm_bf16_t_kernel<BM, BN, AKO, BKO, RELU, MODE>;
  static uint64_t set_on = 0;
  int dev = 0;
  (void)hipGetDevice(&dev);
  if (lds > 65536 && dev < 64 && !(set_on >> dev & 1)) {
    (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)lds);
    set_on |= 1ull << dev;
  }
  const int mt = (int)((C + BM - 1) / BM), nt = Nout / BN;
  const int tiles = mt * nt * n_experts;
  const unsigned grid = (unsigned)(((tiles + 7) / 8) * 8);
  launch_k(kern, dim3(grid), dim3(BN * 2), lds, s, a, strideA, b, strideB, c, strideC,
                     rows, K, Nout, mt, nt, tiles, io, C, n_experts);
}

template <int BM, int BN>
void launch_t_sized(GemmRows mode, bool relu, bool a_ko, bool b_ko, const uint16_t* a,
                    int64_t strideA, const uint16_t* b, int64_t strideB, uint16_t* c,
                    int64_t strideC, const int32_t* rows, int n_experts, int64_t C, int K,
                    int Nout, const GemmIO& io, hipStream_t s) {
#define SWL_T(AK, BK, RL, MD)                                                                    \
  launch_t<BM, BN, AK, BK, RL, MD>(a, strideA, b, strideB, c, strideC, rows, n_experts, C, K, \
                                   Nout, io, s)
  if (mode == kRowsMask && !a_ko && b_ko) SWL_T(false, true, false, kRowsMask);
  else if (mode == kRowsDense && !relu && !a_ko && b_ko) SWL_T(false, true, false, kRowsDense);
  else if (mode == kRowsDense && !relu && a_ko && b_ko) SWL_T(true, true, false, kRowsDense);
  else if (mode == kRowsDense && !relu && a_ko && !b_ko) SWL_T(true, false, false, kRowsDense);
#undef SWL_T
}

// The 4-wave tile for launches with more tiles than CUs.  Experts of at most
// 64 rows take 64-row tiles: the same weight traffic as 128 rows with half the
// LDS, registers and MFMA work, so more blocks share a CU and more loads are in
// flight (at the 2048-expert share, capacity 64, the two matmuls stream their
// weights 7-16% faster).  Where the output width splits into 256-column tiles
// they are 64 x 256 with 64-wide K steps: half the tiles (half the prologues)
// and half the re-reads of the A rows of 64 x 128 with 128-wide steps, with the
// same 40 KB of operands in flight and three blocks per CU (at the 2048-expert
// share: GEMM2 with the combine 2.4% and GEMM1 0.7% faster, same process).
template <int BM, int BN, int BKT>
void launch_plain_tiles(GemmRows mode, bool relu, const uint16_t* a, int64_t strideA,
                        const uint16_t* b, int64_t strideB, uint16_t* c, int64_t strideC,
                        const int32_t* rows, int n_experts, int64_t C, int K, int Nout,
                        const GemmIO& io, hipStream_t s) {
  const int mt = (int)((C + BM - 1) / BM), nt = Nout / BN;
  const int tiles = mt * nt * n_experts;
  const unsigned grid = (unsigned)(((tiles + 7) / 8) * 8);
#define SWL_PLAIN(RL, MD, NT)                                                                  \
  launch_k((gemm_bf16_kernel<BM, BN, RL, MD, NT, BKT>), dim3(grid), dim3(256), 0, s, a,       \
           strideA, b, strideB, c, strideC, rows, K, Nout, mt, nt, tiles, io, C)
  if (mode == kRowsGather && relu) SWL_PLAIN(true, kRowsGather, false);
  // every expert's weights are read once: non-temporal loads keep them from
  // pushing H (read by all N tiles of an expert) out of L2
  else if (mode == kRowsCombine && mt == 1) SWL_PLAIN(false, kRowsCombine, true);
  else if (mode == kRowsCombine) SWL_PLAIN(false, kRowsCombine, false);
  else if (mode == kRowsMask) SWL_PLAIN(false, kRowsMask, false);
  else if (relu) SWL_PLAIN(true, kRowsDense, false);
  else SWL_PLAIN(false, kRowsDense, false);
#undef SWL_PLAIN
}

template <int BM>
void launch_plain(GemmRows mode, bool relu, const uint16_t* a, int64_t strideA,
                  const uint16_t* b, int64_t strideB, uint16_t* c, int64_t strideC,
                  const int32_t* rows, int n_experts, int64_t C, int K, int Nout,
                  const GemmIO& io, hipStream_t s) {
  if constexpr (BM == 64) {
    if (Nout % 256 == 0) {
      launch_plain_tiles<64, 256, 64>(mode, relu, a, strideA, b, strideB, c, strideC, rows,
                                      n_experts, C, K, Nout, io, s);
      return;
    }
  }
  launch_plain_tiles<BM, 128, 0>(mode, relu, a, strideA, b, strideB, c, strideC, rows,
                                 n_experts, C, K, Nout, io, s);
}

}  // namespace

void launch_expert_gemm_bf16_t(GemmRows mode, bool relu, bool a_kouter, bool b_kouter,
                               const void* A, int64_t strideA, const void* B, int64_t strideB,
                               void* Cout, int64_t strideC, const int32_t* rows, int n_experts,
                               int64_t C, int K, int Nout, const GemmIO& io, hipStream_t s) {
  if (C == 0 || n_experts == 0) return;
  // a K-outer A is read in whole column tiles of the M range
  const bool wide = use_wide(C, Nout, n_experts, io) && (!a_kouter || C % GW_BM == 0);
  const int tiles128 = (int)((C + 127) / 128) * (Nout / 128) * n_experts;
  if (!wide && !a_kouter && b_kouter && !relu && tiles128 <= device_cus()) {
    const unsigned grid = (unsigned)(((tiles128 + 7) / 8) * 8);
    GemmIO plain = io;
    plain.tile_start = nullptr;
    if (mode == kRowsMask)
      launch_split<false, kRowsMask, true>(grid, (const uint16_t*)A, strideA, (const uint16_t*)B,
                                           strideB, (uint16_t*)Cout, strideC, rows, K, Nout,
                                           (int)((C + 127) / 128), Nout / 128, tiles128, plain,
                                           C, s);
    else
      launch_split<false, kRowsDense, true>(grid, (const uint16_t*)A, strideA,
                                            (const uint16_t*)B, strideB, (uint16_t*)Cout,
                                            strideC, rows, K, Nout, (int)((C + 127) / 128),
                                            Nout / 128, tiles128, plain, C, s);
    return;
  }
  if (wide) {
    launch_t_sized<GW_BM, GW_BN>(mode, relu, a_kouter, b_kouter, (const uint16_t*)A, strideA,
                                 (const uint16_t*)B, strideB, (uint16_t*)Cout, strideC, rows,
                                 n_experts, C, K, Nout, io, s);
  } else {
    GemmIO plain = io;  // a tile list counts 256-row tiles
    plain.tile_start = nullptr;
    launch_t_sized<128, 128>(mode, relu, a_kouter, b_kouter, (const uint16_t*)A, strideA,
                             (const uint16_t*)B, strideB, (uint16_t*)Cout, strideC, rows,
                             n_experts, C, K, Nout, plain, s);
  }
}

void launch_expert_gemm_bf16(GemmRows mode, bool relu, const void* A, int64_t strideA,
                             const void* B, int64_t strideB, void* Cout, int64_t strideC,
                             const int32_t* rows, int n_experts, int64_t C, int K, int Nout,
                             const GemmIO& io, hipStream_t s) {
  if (C == 0 || n_experts == 0) return;
  const uint16_t* a = (const uint16_t*)A;
  const uint16_t* b = (const uint16_t*)B;
  uint16_t* c = (uint16_t*)Cout;
  if (use_wide(C, Nout, n_experts, io, true)) {
    if (mode == kRowsCombine)
      launch_wide<false, kRowsCombine>(a, strideA, b, strideB, c, strideC, rows, n_experts, C, K,
                                       Nout, io, s);
    else if (mode == kRowsGather && relu)
      launch_wide<true, kRowsGather>(a, strideA, b, strideB, c, strideC, rows, n_experts, C, K,
                                     Nout, io, s);
    else if (mode == kRowsMask)
      launch_wide<false, kRowsMask>(a, strideA, b, strideB, c, strideC, rows, n_experts, C, K,
                                    Nout, io, s);
    else if (mode == kRowsDense && !relu)
      launch_wide<false, kRowsDense>(a, strideA, b, strideB, c, strideC, rows, n_experts, C, K,
                                     Nout, io, s);
    else
      launch_wide<true, kRowsDense>(a, strideA, b, strideB, c, strideC, rows, n_experts, C, K,
                                    Nout, io, s);
    return;
  }
  constexpr int BM = 128, BN = 128;
  const int mt = (int)((C + BM - 1) / BM), nt = Nout / BN;
  const int tiles = mt * nt * n_experts;
  const unsigned grid = (unsigned)(((tiles + 7) / 8) * 8);
  if (tiles <= device_cus()) {
    if (mode == kRowsGather && relu)
      launch_split<true, kRowsGather>(grid, a, strideA, b, strideB, c, strideC, rows, K, Nout, mt,
                                      nt, tiles, io, C, s);
    else if (mode == kRowsCombine)
      launch_split<false, kRowsCombine>(grid, a, strideA, b, strideB, c, strideC, rows, K, Nout,
                                        mt, nt, tiles, io, C, s);
    else if (mode == kRowsMask)
      launch_split<false, kRowsMask>(grid, a, strideA, b, strideB, c, strideC, rows, K, Nout, mt,
                                     nt, tiles, io, C, s);
    else if (relu)
      launch_split<true, kRowsDense>(grid, a, strideA, b, strideB, c, strideC, rows, K, Nout, mt,
                                     nt, tiles, io, C, s);
    else
      launch_split<false, kRowsDense>(grid, a, strideA, b, strideB, c, strideC, rows, K, Nout, mt,
                                      nt, tiles, io, C, s);
    return;
  }
  if (C <= 64)
    launch_plain<64>(mode, relu, a, strideA, b, strideB, c, strideC, rows, n_experts, C, K, Nout,
                     io, s);
  else
    launch_plain<128>(mode, relu, a, strideA, b, strideB, c, strideC, rows, n_experts, C, K, Nout,
                      io, s);
}

void launch_expert_gemm(bool bf16, bool relu, const void* A, int64_t strideA, const void* B,
                        int64_t strideB, void* Cout, int64_t strideC, const int32_t* rows,
                        int n_experts, int64_t C, int K, int Nout, hipStream_t s) {
  if (C == 0 || n_experts == 0) return;
  if (bf16) {
    launch_expert_gemm_bf16(kRowsDense, relu, A, strideA, B, strideB, Cout, strideC, rows,
                            n_experts, C, K, Nout, GemmIO{}, s);
  } else {
    dim3 grid((unsigned)((Nout + 31) / 32), (unsigned)((C + 31) / 32), (unsigned)n_experts);
    if (relu)
      launch_k(gemm_f32_kernel<true>, grid, dim3(256), 0, s, (const float*)A, strideA,
                         (const float*)B, strideB, (float*)Cout, strideC, rows, K, Nout);
    else
      launch_k(gemm_f32_kernel<false>, grid, dim3(256), 0, s, (const float*)A, strideA,
                         (const float*)B, strideB, (float*)Cout, strideC, rows, K, Nout);
  }
}

bool expert_gemm_shape_ok(bool bf16, int d, int F) {
  if (!bf16) return true;
  return d % 128 == 0 && F % 128 == 0;
}

}  // namespace swl
