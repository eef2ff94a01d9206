// Launchers of the Switch-layer kernels (host side) and the per-stage event
// profiler used for measurement.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swl {

// Per-stage timing of a call, for measurement.  While a profiled call runs,
// the first kernel a stage launches records the stage's start event and every
// kernel its stop event on the dispatch itself (hipExtLaunchKernel), so a
// stage's time is its kernels' execution from the first start to the last end,
// with no event packets of their own on the stream.  Up to max_calls calls are
// recorded; nothing synchronises.
struct StageEvents {
  hipEvent_t start = nullptr, stop = nullptr;
  bool launched = false;
};
// the open stage of the profiled call in progress on this thread, or NULL
extern thread_local StageEvents* g_stage;

struct Profiler {
  static constexpr int kMax = 24;   // stages per call
  bool on = false;
  int max_calls = 0;
  int calls = 0;                    // calls recorded so far
  int n = 0;                        // stages of the call being (or last) recorded
  bool active = false;              // the current call is being recorded
  hipEvent_t* ev = nullptr;         // max_calls * kMax * 2: start and stop per stage
  const char* names[kMax];
  StageEvents cur;                  // the stage open now
};

// A stage that launched no kernel gets both events recorded where it ends.
inline void prof_close(Profiler* p, hipStream_t s) {
  if (g_stage != &p->cur) return;
  if (!p->cur.launched) {
    (void)hipEventRecord(p->cur.start, s);
    (void)hipEventRecord(p->cur.stop, s);
  }
  g_stage = nullptr;
}
inline void prof_begin(Profiler* p) {
  g_stage = nullptr;
  if (!p || !p->on) return;
  p->active = p->calls < p->max_calls;
  if (p->active) p->n = 0;  // calls past the recorded ones keep the recorded stage count
}
inline void prof_mark(Profiler* p, hipStream_t s, const char* name) {
  if (!p || !p->on || !p->active || p->n >= Profiler::kMax) return;
  prof_close(p, s);
  p->names[p->n] = name;
  hipEvent_t* e = p->ev + 2 * (p->calls * Profiler::kMax + p->n);
  p->cur.start = e[0];
  p->cur.stop = e[1];
  p->cur.launched = false;
  g_stage = &p->cur;
  p->n += 1;
}
inline void prof_end(Profiler* p, hipStream_t s) {
  if (!p || !p->on || !p->active || p->n == 0) {
    g_stage = nullptr;
    return;
  }
  prof_close(p, s);
  p->calls += 1;
  p->active = false;
}

// Every kernel of the library is launched through here.
template <typename F, typename... Args>
inline void launch_k(F kernel, const dim3& grid, const dim3& block, uint32_t lds, hipStream_t s,
                     Args... args) {
  StageEvents* st = g_stage;
  if (st) {
    hipExtLaunchKernelGGL(kernel, grid, block, lds, s, st->launched ? nullptr : st->start,
                          st->stop, 0, args...);
    st->launched = true;
  } else {
    hipLaunchKernelGGL(kernel, grid, block, lds, s, args...);
  }
}

// Experts per token: 1 (the Switch layer) or 2 (classic top-2 MoE routing).
// Per-token outputs are laid out [T, k]; assignment a = t * k + j.
constexpr int kMaxTopK = 2;

// router.hip
bool router_fused_ok(bool x_bf16, int N);
int64_t route_chunk_tokens(bool x_bf16, int N);
// planes: workspace of 3 N d bf16 for the weight planes (bf16 x only)
void launch_router_logits(const void* x, bool x_bf16, const float* W_r, const float* b_r,
                          float* h, int64_t T, int d, int N, uint16_t* planes, hipStream_t s);
void launch_router_fused(const uint16_t* x, const float* W_r, const float* b_r, int64_t T, int d,
                         int N, int k, float* logits, int32_t* expert_idx, float* gate,
                         float* P_part, int32_t* hist, int32_t* rank_local, hipStream_t s);
void launch_route_rows(const float* h, int64_t T, int N, int k, int32_t* expert_idx, float* gate,
                       float* P_part, int32_t* hist, int32_t* rank_local, hipStream_t s);

// assign.hip
// tile_start (optional, N + 1 entries): exclusive prefix over experts of
// ceil(n_kept / tile_rows), with the total last.
// k: assignments per token (the loss divides load by k T).
void launch_route_scan(int32_t* hist, const float* P_part, int64_t nc, int N, int64_t T, int k,
                       int64_t C, float alpha, int32_t* load, int32_t* n_kept, double* terms,
                       float* aux, int32_t* tile_start, int tile_rows, hipStream_t s);
// One launch for the chunk scan, the loss and the finalisation (N <= 256,
// chunks of at least 16 tokens, nc * N <= kAssignMaxCells).  copy_mode 0: no
// rows move; 1: rows of dropped tokens from x to dst (= out, top-1); 2: rows of
// kept assignments from x to dst (= Xbuf [N, C, row]).  tok may be NULL.
constexpr int64_t kAssignMaxCells = 8192;  // every block re-reads up to nc * N counts
bool assign_one_launch_ok(int N, int64_t nc, int64_t chunk);
void launch_assign(const int32_t* hist, const float* P_part, int64_t nc, int N, int64_t T, int k,
                   int64_t chunk, int64_t C, float alpha, const int32_t* expert_idx,
                   const int32_t* rank_local, int32_t* load, int32_t* n_kept, float* aux,
                   int32_t* tile_start, int tile_rows, int32_t* position, uint8_t* drop_mask,
                   int32_t* tok, int copy_mode, int row_bytes, const void* x, void* dst,
                   hipStream_t s);
void launch_finalize_positions(int64_t T, int k, const int32_t* expert_idx,
                               const int32_t* rank_local, const int32_t* offsets, int N,
                               int64_t chunk, int64_t C, int32_t* position, uint8_t* drop_mask,
                               hipStream_t s);

// move.hip
void launch_dispatch(const void* x, int64_t T, int k, int row_bytes, const int32_t* expert_idx,
                     const int32_t* rank_local, const int32_t* offsets, int N, int64_t chunk,
                     int64_t C, int32_t* position, uint8_t* drop_mask, void* Xbuf, hipStream_t s);
// copy_dropped: copy the rows of dropped tokens to out (k = 1 with the fused combine)
void launch_dispatch_index(const void* x, int64_t T, int k, int row_bytes,
                           const int32_t* expert_idx, const int32_t* rank_local,
                           const int32_t* offsets, int N, int64_t chunk, int64_t C,
                           int32_t* position, uint8_t* drop_mask, int32_t* tok, bool copy_dropped,
                           void* out, hipStream_t s);
void launch_combine(const void* x, bool bf16, int64_t T, int k, int row_bytes,
                    const int32_t* expert_idx, const int32_t* position, const uint8_t* drop_mask,
                    const float* gate, int64_t C, const void* Ybuf, void* out, hipStream_t s);
void launch_copy_expert_rows(const void* Ybuf, const int32_t* n_kept, int N, int64_t C,
                             int row_bytes, void* dst, hipStream_t s);

// gemm.hip
// Row routing of the bf16 expert matmuls.  GATHER: the A rows of expert e are
// rows tok[e * C + m] of x (K = d_model).  COMBINE: output row m of expert e is
// combined into out[tok[e * C + m]] = x + gate * y instead of being stored.
// MASK: the stored result is zeroed where io.mask (same layout as the output,
// bf16) is not positive -- the ReLU derivative of the backward pass.
// rows == NULL: every expert has C valid rows (dense weight-gradient matmuls).
enum GemmRows { kRowsDense = 0, kRowsGather = 1, kRowsCombine = 2, kRowsMask = 3 };
struct GemmIO {
  const int32_t* tile_start = nullptr;  // compact tile list of the wide kernel
  const uint16_t* mask = nullptr;       // kRowsMask: the forward activation H
  const int32_t* tok = nullptr;
  const uint16_t* x = nullptr;
  const float* gate = nullptr;
  uint16_t* out = nullptr;
  // K-outer operands (launch_expert_gemm_bf16_t): row pitch in elements, and
  // per-expert count of valid K rows (NULL: all K rows are valid)
  int64_t lda = 0, ldb = 0;
  const int32_t* krows = nullptr;
  // expert output kept by a training forward: the combine also stores Y into
  // ykeep ([experts][C][Nout], the dense layout), and block 0 of a forward's
  // second matmul writes yflag_value to *yflag (1: Y is in the forward's Y
  // buffer).  yskip: the kernel exits at once when *yskip is nonzero (the
  // backward's recomputation of Y, when the forward kept it).
  uint16_t* ykeep = nullptr;
  int32_t* yflag = nullptr;
  int32_t yflag_value = 0;
  const int32_t* yskip = nullptr;
};
void launch_expert_gemm_bf16(GemmRows mode, bool relu, const void* A, int64_t strideA,
                             const void* B, int64_t strideB, void* Cout, int64_t strideC,
                             const int32_t* rows, int n_experts, int64_t C, int K, int Nout,
                             const GemmIO& io, hipStream_t s);
void launch_expert_gemm(bool bf16, bool relu, const void* A, int64_t strideA, const void* B,
                        int64_t strideB, void* Cout, int64_t strideC, const int32_t* rows,
                        int n_experts, int64_t C, int K, int Nout, hipStream_t s);
// The same products with either operand stored K-outer (a_kouter: A is
// [K][rows] per expert with pitch io.lda, the tile's M range a column range;
// b_kouter: B is [K][Nout] with pitch io.ldb).  Modes kRowsDense (optional
// ReLU) and kRowsMask.  K must be a multiple of 64.
void launch_expert_gemm_bf16_t(GemmRows mode, bool relu, bool a_kouter, bool b_kouter,
                               const void* A, int64_t strideA, const void* B, int64_t strideB,
                               void* Cout, int64_t strideC, const int32_t* rows, int n_experts,
                               int64_t C, int K, int Nout, const GemmIO& io, hipStream_t s);
bool expert_gemm_shape_ok(bool bf16, int d, int F);
constexpr int kWideTileRows = 256;   // M tile of the wide bf16 kernel

// ffn.hip: the fused expert FFN (both matmuls, the ReLU and the combine, H
// kept on chip) over the compact list of kFfnTileRows-row tiles; d a multiple
// of 256 up to 1024, F a multiple of 256, bf16, top-1.  Block 0 writes 0 to
// *yflag and *hflag (neither Y nor H is left in the workspace).
constexpr int kFfnTileRows = 64;
bool ffn_fused_shape_ok(int d, int F);
void launch_ffn_fused(const void* x, const void* W_in, const void* W_out, const int32_t* n_kept,
                      const int32_t* tile_start, const int32_t* tok, const float* gate,
                      void* out, int d, int F, int64_t C, int n_exp, int32_t* yflag,
                      int32_t* hflag, hipStream_t s);

// backward.hip
// n_kept = min(load, C) and the compact tile list of kWideTileRows-row tiles
// (tile_start may be NULL)
void launch_bwd_slots(const void* G, int64_t T, int d, int k, const int32_t* expert_idx,
                      const int32_t* position, const uint8_t* drop_mask, const float* gate,
                      int64_t C, int32_t* tok, void* Gs, const int32_t* load, int N,
                      int32_t* n_kept, int32_t* tile_start, hipStream_t s);
void launch_transpose(const void* src, int64_t src_estride, int ld, int R, int Ccols,
                      const int32_t* valid, const int32_t* tok, void* dst, int64_t dst_estride,
                      int Rpad, int n_experts, hipStream_t s);
// Y from Yfwd when *yflag is nonzero (yflag may be NULL), else from Ybuf
void launch_router_bwd(const float* h, int64_t T, int N, int d, int k, const void* G,
                       const void* Ybuf, const void* Yfwd, const int32_t* yflag, int64_t C,
                       const int32_t* expert_idx,
                       const int32_t* position, const uint8_t* drop_mask, const int32_t* load,
                       float loss_scale, float* dh, hipStream_t s);
// part [slices, N, d] and part_b [slices, N] fp32 scratch, slices = router_wgrad_slices(T, N, d)
int64_t router_wgrad_slices(int64_t T, int N, int d);
// reduce = false leaves the slice sums to launch_grad_x (called later with the
// same part, part_b, T, N and d)
void launch_router_wgrad(const float* dh, const void* x, int64_t T, int N, int d, float* part,
                         float* part_b, float* dW_r, float* db, bool reduce, hipStream_t s);
void launch_grad_x(const void* G, int64_t T, int d, int k, const int32_t* expert_idx,
                   const int32_t* position, const uint8_t* drop_mask, int64_t C, const void* dXe,
                   const float* dh, const float* W_r, int N, void* dx, const float* part,
                   const float* part_b, float* dW_r, float* db, hipStream_t s);
void launch_fill_zero(void* p, size_t bytes, hipStream_t s);

}  // namespace swl
