// Fused expert FFN: the first matmul, the ReLU, the second matmul and the
// combine in one launch, with the hidden activations H kept on chip.
//
// Each expert is the dense FFN it replaces (kasblo explainer, section
// "TransformerのどこへSwitch layerが入るのか"), relu(x W_in^T) W_out^T, applied
// to the tokens routed to it; the result returns to token order scaled by the
// gate (section "tokenをExpertへ送って戻すforward pass"; llm-papers-study
// section 3.2, y = p_{i*} E_{i*}(x)) and is added to the residual.  The
// unfused path writes H [rows, F] to memory between two launches; here a block
// owns 64 rows of one expert and walks F in chunks of 256 hidden units:
//   phase A  H_c = relu(X W_in[e][chunk]^T)   (K = d), rounded to bf16 into LDS
//   phase B  Y  += H_c W_out[e][:, chunk]^T   (K = 256), fp32 in registers
// so H never leaves the CU.  The same roundings as the unfused path: H is
// rounded to bf16 after the ReLU, Y to bf16 before the fp32 combine.
//
// Block: 512 threads = 8 waves, one block per CU.  Phase A: wave w owns hidden
// units 32 w .. 32 w + 31 of the chunk for both 32-row halves of the tile (two
// v_mfma_f32_32x32x16_bf16 tiles, the W_in fragment first).  Phase B: wave w
// owns output columns w * 32 NT .. + 32 NT - 1 (NT tiles of 32, d = 256 NT) for
// both halves: 2 NT accumulator tiles that live across all chunks.
//
// Both phases are one stream of equal steps: a step loads one 64-byte piece per
// lane of a weight fragment (phase A: rows of W_in over a 64-wide K step;
// phase B: 32 output rows of W_out over 64 hidden units) and runs 8 MFMAs
// (2 row tiles x 4 K sub-steps).  K is permuted inside a step the same way for
// both operands: lane group g = l / 32 takes the 32 consecutive k of its half
// of the 64, sub-step s the 8 of them at 8 s, so a lane's weight piece is 64
// contiguous bytes.  Weights ride a ring of two register slots (step i + 2 is
// loaded while step i runs).
//
// X (the gathered token rows) goes through LDS in [64][64] K tiles, double
// buffered, one barrier per phase-A step; H_c in a [64][256] tile.
#include "epilogue.hpp"

namespace swl {

constexpr int FF_BM = 64;    // token rows per block
constexpr int FF_FC = 256;   // hidden units per chunk
// LDS rows are padded by one 16-byte chunk: X tile rows of 64 + 8 elements (9
// chunks) and H tile rows of 256 + 8 (33 chunks), odd chunk counts, so the 16
// rows one fragment read touches fall on 16 distinct 16-byte bank groups and a
// lane's fragments of successive K sub-steps sit at constant offsets.
constexpr int FF_XP = 64 + 8, FF_HP = FF_FC + 8;   // row pitches (elements)
constexpr int FF_XE = FF_BM * FF_XP;    // elements of one X K tile
constexpr int FF_HE = FF_BM * FF_HP;    // elements of the H tile

// element offset of 16-byte chunk c of row r
__device__ __forceinline__ int ffx_at(int r, int c) { return r * FF_XP + 8 * c; }
__device__ __forceinline__ int ffh_at(int r, int c) { return r * FF_HP + 8 * c; }

template <int NT>
constexpr size_t ffn_lds_bytes() {
  constexpr size_t ops = (size_t)(2 * FF_XE + FF_HE) * sizeof(uint16_t);
  constexpr size_t epi = (size_t)8 * FF_BM * (32 * NT + 8) * sizeof(uint16_t);
  return ops > epi ? ops : epi;
}

template <int NT>
__global__ __launch_bounds__(512, 1) void ffn_fused_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ W_in,
    const uint16_t* __restrict__ W_out, const int32_t* __restrict__ n_kept,
    const int32_t* __restrict__ tile_start, const int32_t* __restrict__ tok,
    const float* __restrict__ gate, uint16_t* __restrict__ out, int F, int64_t C, int n_exp,
    int32_t* __restrict__ yflag, int32_t* __restrict__ hflag) {
  constexpr int d = 256 * NT;
  constexpr int NKA = d / 64;              // phase-A steps per chunk (even)
  constexpr int NKB = 4 * NT;              // phase-B steps per chunk (even)
  constexpr int SPC = NKA + NKB;           // steps per chunk
  extern __shared__ __attribute__((aligned(16))) uint16_t flds[];
  uint16_t* Xs = flds;                     // [2][64][64]
  uint16_t* Hs = flds + 2 * FF_XE;         // [64][256]

  if (blockIdx.x == 0 && threadIdx.x == 0) {
    if (yflag) *yflag = 0;   // this path keeps neither Y nor H in the workspace
    if (hflag) *hflag = 0;
  }
  // tile from the compact list of 64-row tiles, each XCD one stretch of it
  const int total = tile_start[n_exp];
  const int per_xcd = (total + 7) >> 3;
  const int tile = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if ((int)(blockIdx.x >> 3) >= per_xcd || tile >= total) return;
  int lo = 0, hi = n_exp - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tile_start[mid] <= tile) lo = mid; else hi = mid - 1;
  }
  const int e = lo;
  const int m0 = (tile - tile_start[e]) * FF_BM;
  const int rows_e = n_kept[e];
  const int32_t* tok_e = tok + (int64_t)e * C;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int fr = lane & 31, g = lane >> 5;
  const int nchunks = F / FF_FC;

  // weight rows of this lane: phase A row 32 w + fr of each chunk of W_in[e];
  // phase B rows w * 32 NT + 32 j + fr of W_out[e]; the lane's 64-byte piece
  // starts 32 g elements into each 64-wide step.  Addresses are a wave-uniform
  // base (scalar registers) plus one 32-bit lane offset per matrix.
  const uint16_t* win_e = W_in + (int64_t)e * F * d;
  const uint16_t* wout_e = W_out + (int64_t)e * d * F;
  const uint32_t off_a = (uint32_t)(((32 * w + fr) * d + 32 * g) * 2);
  const uint32_t off_b = (uint32_t)(((w * 32 * NT + fr) * F + 32 * g) * 2);
  const int64_t jstride = (int64_t)32 * F;   // between the output tiles of a wave

  // X loader: thread -> row tid / 8 of the tile, 16-byte chunk tid % 8 of each
  // [64][64] K tile; X tile a (a = c NKA + t over the whole call) is K tile t
  const int xrow = tid >> 3, xch = tid & 7;
  int mr = m0 + xrow;
  mr = mr < rows_e ? mr : rows_e - 1;   // rows past n_kept: any valid row, never stored
  const uint16_t* xsrc = x + (int64_t)tok_e[mr] * d + 8 * xch;
  const int xdst = ffx_at(xrow, xch);

  u32x4 ring[2][4];
  u32x4 xr[2];
  // step r (a constant of the unrolled chunk body) of chunk c into ring slot
  // `slot`: r < NKA phase A K step r; r >= NKA phase B, hidden units 64 G of
  // the chunk and output tile j with r - NKA = G NT + j; r >= SPC is step
  // r - SPC of chunk c + 1 (nothing past the last chunk)
  auto wload = [&](int slot, int c, int r) {
    if (r >= SPC) {
      r -= SPC;
      ++c;
      if (c >= nchunks) return;
    }
    const char* p;
    if (r < NKA) {
      p = reinterpret_cast<const char*>(win_e + (int64_t)c * FF_FC * d + 64 * r) + off_a;
    } else {
      const int q = r - NKA, G = q / NT, j = q - G * NT;
      p = reinterpret_cast<const char*>(wout_e + j * jstride + c * FF_FC + 64 * G) + off_b;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) ring[slot][u] = *reinterpret_cast<const u32x4*>(p + 16 * u);
  };
  // X K tile t of the next chunk when t >= NKA (nothing past the last chunk).
  // xoff is 0, passed through an empty asm statement once per chunk: the tiles
  // are the same for every chunk, and without it the compiler would hoist all
  // of them out of the chunk loop into registers.
  int xoff = 0;
  auto xload = [&](int k, int c, int t) {
    if (t >= NKA) {
      t -= NKA;
      if (c + 1 >= nchunks) return;
    }
    xr[k] = *reinterpret_cast<const u32x4*>(xsrc + xoff + 64 * t);
  };

  floatx16 accy[2][NT];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) accy[i][j][v] = 0.f;
  floatx16 acch[2];

  // prologue: weight steps 0 and 1; X tile 0 into LDS, tiles 1 and 2 into registers
  wload(0, 0, 0);
  wload(1, 0, 1);
  xload(0, 0, 0);
  *reinterpret_cast<u32x4*>(Xs + xdst) = xr[0];
  xload(1, 0, 1);
  xload(0, 0, 2);
  __syncthreads();

  // fragments of a step's four K sub-steps come from LDS one sub-step ahead of
  // the MFMAs that use them
  const int xfrag = ffx_at(fr, 4 * g);
  auto mfma_step = [&](floatx16 (&acc)[2], const u32x4 (&wp)[4], const uint16_t* tile, int pitch,
                       int base) {
    bf16x8 fb[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
      fb[0][i] = *reinterpret_cast<const bf16x8*>(tile + base + 32 * i * pitch);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s < 3) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
          fb[(s + 1) & 1][i] =
              *reinterpret_cast<const bf16x8*>(tile + base + 32 * i * pitch + 8 * (s + 1));
      }
      const bf16x8 wv = __builtin_bit_cast(bf16x8, wp[s]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wv, fb[s & 1][i], acc[i], 0, 0, 0);
    }
  };

  for (int c = 0; c < nchunks; ++c) {
    asm volatile("" : "+v"(xoff));
    // ---- phase A: H_c = X W_in[e][chunk]^T over K = d
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) acch[i][v] = 0.f;
#pragma unroll
    for (int t = 0; t < NKA; ++t) {
      // step c SPC + t (SPC even: slot t & 1); X tile c NKA + t (NKA even: its
      // buffer is t & 1)
      const int slot = t & 1;
      mfma_step(acch, ring[slot], Xs + (t & 1) * FF_XE, FF_XP, xfrag);
      wload(slot, c, t + 2);
      // X tile + 1 (registers (t + 1) & 1) into the other buffer, last read in the
      // step before this one; then tile + 3 into the registers it leaves
      if (t + 1 < NKA || c + 1 < nchunks)
        *reinterpret_cast<u32x4*>(Xs + ((t + 1) & 1) * FF_XE + xdst) = xr[(t + 1) & 1];
      xload((t + 1) & 1, c, t + 3);
      __syncthreads();
    }
    // H_c: ReLU, bf16, into LDS (last read in the previous chunk's phase B,
    // NKA barriers ago); lane (row 32 i + fr, half g) holds hidden units
    // 32 w + 8 q + 4 g .. + 3 of the chunk
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t p0 =
            relu_bf16x2_bits(f32x2_to_bf16x2_bits(acch[i][4 * q], acch[i][4 * q + 1]));
        const uint32_t p1 =
            relu_bf16x2_bits(f32x2_to_bf16x2_bits(acch[i][4 * q + 2], acch[i][4 * q + 3]));
        *reinterpret_cast<uint2*>(Hs + ffh_at(32 * i + fr, 4 * w + q) + 4 * g) =
            make_uint2(p0, p1);
      }
    __syncthreads();
    // ---- phase B: Y += H_c W_out[e][:, chunk]^T, hidden units 64 G .. + 63,
    // output tile j (no barrier: H_c is read only)
#pragma unroll
    for (int G = 0; G < 4; ++G)
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int r = NKA + G * NT + j;
        const int slot = r & 1;
        floatx16 acc2[2] = {accy[0][j], accy[1][j]};
        mfma_step(acc2, ring[slot], Hs, FF_HP, ffh_at(fr, 8 * G + 4 * g));
        accy[0][j] = acc2[0];
        accy[1][j] = acc2[1];
        wload(slot, c, r + 2);
      }
  }

  // epilogue: Y rounded to bf16 and staged in LDS per wave (64 rows x 32 NT
  // columns), then out[t] = x[t] + gate[t] * y for the tile's kept rows
  __syncthreads();   // every wave is done with X and H_c
  uint16_t* stage = flds + w * FF_BM * (32 * NT + 8);
  stage_tile_bf16<2, NT, CombineRows<2, NT>::LD, false>(accy, stage, lane);
  CombineRows<2, NT> cr;
  combine_prefetch<2, NT>(cr, tok_e, x, gate, m0, w * 32 * NT, rows_e, d, lane);
  combine_from_stage<2, NT>(stage, cr, out, lane);
}

bool ffn_fused_shape_ok(int d, int F) {
  return d % 256 == 0 && d >= 256 && d <= 1024 && F % FF_FC == 0;
}

void launch_ffn_fused(const void* x, const void* W_in, const void* W_out, const int32_t* n_kept,
                      const int32_t* tile_start, const int32_t* tok, const float* gate,
                      void* out, int d, int F, int64_t C, int n_exp, int32_t* yflag,
                      int32_t* hflag, hipStream_t s) {
  if (C == 0 || n_exp == 0) return;
  const int64_t tiles = (C + FF_BM - 1) / FF_BM * (int64_t)n_exp;   // upper bound
  const unsigned grid = (unsigned)((tiles + 7) / 8 * 8);
#define SWL_FFN(NT_)                                                                          \
  do {                                                                                        \
    constexpr size_t lds = ffn_lds_bytes<NT_>();                                              \
    static uint64_t set_on = 0;                                                               \
    int dev = 0;                                                                              \
    (void)hipGetDevice(&dev);                                                                 \
    if (lds > 65536 && dev < 64 && !(set_on >> dev & 1)) {                                    \
      (void)hipFuncSetAttribute((const void*)ffn_fused_kernel<NT_>,                           \
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);        \
      set_on |= 1ull << dev;                                                                  \
    }                                                                                         \
    launch_k(ffn_fused_kernel<NT_>, dim3(grid), dim3(512), lds, s, (const uint16_t*)x,        \
             (const uint16_t*)W_in, (const uint16_t*)W_out, n_kept, tile_start, tok, gate,    \
             (uint16_t*)out, F, C, n_exp, yflag, hflag);                                      \
  } while (0)
  switch (d / 256) {
    case 1: SWL_FFN(1); break;
    case 2: SWL_FFN(2); break;
    case 3: SWL_FFN(3); break;
    default: SWL_FFN(4); break;
  }
#undef SWL_FFN
}

}  // namespace swl
