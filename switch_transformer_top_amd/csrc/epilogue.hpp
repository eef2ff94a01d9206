// Epilogues shared by the expert matmul kernels (gemm.hip) and the fused
// expert FFN (ffn.hip): MFMA accumulators rounded to bf16 and staged through
// LDS, then stored in 16-byte row pieces, or combined into the layer output.
#pragma once
#include "common.hpp"
#include "kernels.hpp"

namespace swl {

constexpr int GB_BK = 64, GB_PAD = 8;
constexpr int GB_LDK = GB_BK + GB_PAD;  // LDS row stride in bf16 elements (144 bytes)

// The MFMAs take the weight fragment as their first operand and the token
// fragment as the second, so a 32 x 32 accumulator tile holds the transpose of
// the output tile: lane l has output row (l % 32) and, for q < 4, the four
// consecutive output columns 8 q + 4 (l / 32) .. + 3 in elements 4 q .. 4 q + 3.
// A lane therefore rounds its values in pairs (v_cvt_pk_bf16_f32) and writes
// 8 bytes of one row at a time.
template <int TI, int TJ, int LD, bool RELU>
__device__ __forceinline__ void stage_tile_bf16(const floatx16 (&acc)[TI][TJ], uint16_t* stage,
                                                int lane) {
  const int fr = lane & 31, g = lane >> 5;
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t lo = f32x2_to_bf16x2_bits(acc[i][j][4 * q], acc[i][j][4 * q + 1]);
        uint32_t hi = f32x2_to_bf16x2_bits(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
        if (RELU) {
          lo = relu_bf16x2_bits(lo);
          hi = relu_bf16x2_bits(hi);
        }
        *reinterpret_cast<uint2*>(stage + (i * 32 + fr) * LD + j * 32 + 8 * q + 4 * g) =
            make_uint2(lo, hi);
      }
}

// Epilogue shared by the bf16 kernels: a wave's TI x TJ grid of 32 x 32 fp32
// accumulators goes through LDS (rows of TJ * 32 + 8 bf16, after the optional
// ReLU and round-to-nearest-even) and then out in 16-byte row pieces, instead
// of one 2-byte store per accumulator.  Rows at or past rows_e are not stored.
template <int TI, int TJ, bool RELU, bool MASK = false>
__device__ __forceinline__ void store_tile_bf16(const floatx16 (&acc)[TI][TJ], uint16_t* stage,
                                                uint16_t* __restrict__ Ce, int r0, int c0,
                                                int rows_e, int Nout, int lane,
                                                const uint16_t* __restrict__ Me = nullptr) {
  constexpr int W = TJ * 32, LD = W + 8, CPR = W / 8;
  stage_tile_bf16<TI, TJ, LD, RELU>(acc, stage, lane);
#pragma unroll 4
  for (int idx = lane; idx < TI * 32 * CPR; idx += kWave) {
    const int row = idx / CPR, ch = idx - row * CPR;
    if (r0 + row < rows_e) {
      const int64_t at = (int64_t)(r0 + row) * Nout + c0 + ch * 8;
      u32x4 v = *reinterpret_cast<const u32x4*>(stage + row * LD + ch * 8);
      if (MASK) {
        // keep a value where the matching activation is positive (bf16 sign bit
        // clear and not zero), zero it elsewhere
        const u32x4 m = *reinterpret_cast<const u32x4*>(Me + at);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t lo = (m[i] & 0x8000u) == 0 && (m[i] & 0x7FFFu) != 0 ? 0xFFFFu : 0u;
          const uint32_t hi = (m[i] & 0x80000000u) == 0 && (m[i] & 0x7FFF0000u) != 0
                                  ? 0xFFFF0000u : 0u;
          v[i] &= lo | hi;
        }
      }
      *reinterpret_cast<u32x4*>(Ce + at) = v;
    }
  }
}

// Combine epilogue: like store_tile_bf16 (no ReLU), but each 16-byte piece of
// output row m goes to token t = tok_e[m]: out[t] = x[t] + gate[t] * y, with y
// the expert output rounded to bf16 first (the same arithmetic as a separate
// combine pass over a stored expert output).  The reads it needs (slot table,
// gates, residual rows) are issued by combine_prefetch, which a kernel may call
// early so that their latency overlaps other work.
template <int TI, int TJ>
struct CombineRows {
  static constexpr int W = TJ * 32, LD = W + 8, CPR = W / 8;
  static constexpr int NR = (TI * 32 + kWave - 1) / kWave;   // rows per lane
  static constexpr int IT = TI * 32 * CPR / kWave;            // 16-byte pieces per lane
  static constexpr int RPI = kWave / CPR;                     // rows per piece round
  int64_t at[IT];   // element offset of each piece in x and out (-1: row not stored)
  float g[IT];
  u32x4 xv[IT];
};

template <int TI, int TJ>
__device__ __forceinline__ void combine_prefetch(CombineRows<TI, TJ>& cr,
                                                 const int32_t* __restrict__ tok_e,
                                                 const uint16_t* __restrict__ x,
                                                 const float* __restrict__ gate, int r0, int c0,
                                                 int rows_e, int d, int lane) {
  using CR = CombineRows<TI, TJ>;
  // lane l fetches the token and gate of rows l, l + 64, ...; the pieces take
  // them with a lane shuffle
  int tl[CR::NR];
  float gl[CR::NR];
#pragma unroll
  for (int q = 0; q < CR::NR; ++q) {
    const int r = r0 + q * kWave + lane;
    const bool ok = q * kWave + lane < TI * 32 && r < rows_e;
    tl[q] = ok ? tok_e[r] : 0;
    gl[q] = ok ? gate[tl[q]] : 0.f;
  }
#pragma unroll
  for (int it = 0; it < CR::IT; ++it) {
    const int idx = it * kWave + lane;
    const int row = idx / CR::CPR, ch = idx - row * CR::CPR;
    const int q = it * CR::RPI / kWave;              // register holding this row
    const int64_t t = __shfl(tl[q], row & (kWave - 1), kWave);
    cr.g[it] = __shfl(gl[q], row & (kWave - 1), kWave);
    cr.at[it] = r0 + row < rows_e ? t * d + c0 + ch * 8 : -1;
    cr.xv[it] = cr.at[it] >= 0 ? *reinterpret_cast<const u32x4*>(x + cr.at[it]) : u32x4{0, 0, 0, 0};
  }
}

// The combine of a tile already staged in LDS (stage_tile_bf16 with CR::LD).
template <int TI, int TJ>
// With yk (the tile's first row and column in the kept Y buffer, row pitch
// ld_y) the staged Y rows are stored there too.
__device__ __forceinline__ void combine_from_stage(const uint16_t* stage,
                                                   const CombineRows<TI, TJ>& cr,
                                                   uint16_t* __restrict__ out, int lane,
                                                   uint16_t* __restrict__ yk = nullptr,
                                                   int ld_y = 0) {
  using CR = CombineRows<TI, TJ>;
#pragma unroll
  for (int it = 0; it < CR::IT; ++it) {
    const int idx = it * kWave + lane;
    const int row = idx / CR::CPR, ch = idx - row * CR::CPR;
    if (cr.at[it] >= 0) {
      const u32x4 yv = *reinterpret_cast<const u32x4*>(stage + row * CR::LD + ch * 8);
      *reinterpret_cast<u32x4*>(out + cr.at[it]) = combine_vec_bf16(cr.xv[it], yv, cr.g[it]);
      if (yk) *reinterpret_cast<u32x4*>(yk + (int64_t)row * ld_y + ch * 8) = yv;
    }
  }
}

template <int TI, int TJ>
__device__ __forceinline__ void store_tile_combine(const floatx16 (&acc)[TI][TJ], uint16_t* stage,
                                                   const CombineRows<TI, TJ>& cr,
                                                   uint16_t* __restrict__ out, int lane,
                                                   uint16_t* __restrict__ yk = nullptr,
                                                   int ld_y = 0) {
  stage_tile_bf16<TI, TJ, CombineRows<TI, TJ>::LD, false>(acc, stage, lane);
  combine_from_stage<TI, TJ>(stage, cr, out, lane, yk, ld_y);
}

template <int TI, int TJ>
__device__ __forceinline__ void store_tile_combine(const floatx16 (&acc)[TI][TJ], uint16_t* stage,
                                                   const int32_t* __restrict__ tok_e,
                                                   const uint16_t* __restrict__ x,
                                                   const float* __restrict__ gate,
                                                   uint16_t* __restrict__ out, int r0, int c0,
                                                   int rows_e, int d, int lane,
                                                   uint16_t* __restrict__ yk = nullptr) {
  CombineRows<TI, TJ> cr;
  combine_prefetch<TI, TJ>(cr, tok_e, x, gate, r0, c0, rows_e, d, lane);
  store_tile_combine<TI, TJ>(acc, stage, cr, out, lane, yk, d);
}

// The kept-Y origin of a combine tile (rows r0.., columns c0.. of expert e), or
// NULL when the forward keeps no Y.
__device__ __forceinline__ uint16_t* ykeep_at(const GemmIO& io, int e, int64_t C, int r0, int c0,
                                              int Nout) {
  return io.ykeep ? io.ykeep + ((int64_t)e * C + r0) * Nout + c0 : nullptr;
}

// First statements of the forward's second matmul and the backward's Y
// recomputation: block 0 records whether Y is kept; a recomputation whose Y is
// already kept exits.  True: the block returns.
__device__ __forceinline__ bool y_prologue(const GemmIO& io) {
  if (io.yflag && blockIdx.x == 0 && threadIdx.x == 0) *io.yflag = io.yflag_value;
  return io.yskip && *io.yskip != 0;
}

}  // namespace swl
