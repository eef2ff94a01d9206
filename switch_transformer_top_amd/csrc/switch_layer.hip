// Host side of the C ABI declared in include/switch_layer.h: argument
// validation, workspace layout and the launch sequence of one Switch FFN
// forward pass.  Every step runs in the kernels of this directory; the host
// only enqueues them on the caller's stream and never waits for them.
#include <math.h>
#include <string.h>

#include <mutex>
#include <new>

#include "kernels.hpp"
#include "switch_layer.h"

struct switch_layer {
  switch_config cfg;
  const float* W_r;
  const float* b_r;
  const void* W_in;
  const void* W_out;
  int device;
  swl::Profiler prof;
  int keep_y = 0;  // forward: also store the expert outputs for switch_backward
  int ffn_mode = SWITCH_FFN_AUTO;  // fused or two-launch expert FFN (switch_set_ffn_mode)
  void* scratch = nullptr;  // this device's copy of `scratch` (switch_forward_noalloc)
};

// Scratch of switch_forward_noalloc, for callers that cannot allocate: one copy
// per GPU, in the code object's data, resolved once per device by scratch_on.
// In host code the name is only a stand-in; kernels get the device address.
static __device__ __align__(256) unsigned char scratch[SWITCH_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

size_t dtype_size(int32_t dt) { return dt == SWITCH_BF16 ? 2 : 4; }

// Experts per token (the stored config has 0 replaced by 1).
int top_k(const switch_config& c) { return c.top_k; }

// Capacity C = ceil(k * c * T / N) in double, or the override.  Buffers hold
// min(C, T) rows per expert: the k choices of a token are distinct experts, so
// a position is always below T; a capacity above T drops nothing and a
// capacity of min(C, T) keeps exactly the same assignments.
int64_t capacity_of(const switch_config& c, int64_t T) {
  if (c.capacity_override > 0) return c.capacity_override;
  double v = ceil(((double)top_k(c) * c.capacity_factor * (double)T) / (double)c.n_experts);
  if (!(v >= 0.0)) return 0;
  if (v > 9.0e18) v = 9.0e18;
  return (int64_t)v;
}

int64_t buffer_rows(const switch_config& c, int64_t T) {
  int64_t C = capacity_of(c, T);
  return C < T ? C : T;
}

struct Layout {
  size_t logits, planes, ppart, hist, rank, load, nkept, terms, tiles, tok, xbuf, hbuf, ybuf, yflag,
      hflag, total;
};

// Chunks of the routing statistics: the fused router uses small chunks, the
// logits-based path 64 tokens; the workspace is sized for the smaller one.
int64_t chunk_tokens(const switch_config& c) {
  return swl::route_chunk_tokens(c.act_dtype == SWITCH_BF16, c.n_experts);
}
constexpr int64_t kRowsChunk = 64;  // chunk of the logits-based path

Layout layout_of(const switch_layer* L, int64_t T) {
  const switch_config& c = L->cfg;
  const int64_t N = c.n_experts, Cb = buffer_rows(c, T);
  // the smallest chunk any entry point may use sets the number of chunk rows
  const int64_t ch = chunk_tokens(c) < kRowsChunk ? chunk_tokens(c) : kRowsChunk;
  const int64_t nc = (T + ch - 1) / ch;
  const size_t es = dtype_size(c.act_dtype);
  Layout lo;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t at = off; off += align_up(bytes); return at; };
  lo.logits = take(sizeof(float) * (size_t)T * (size_t)N);
  // the bf16 logits router of many experts splits W_r into three bf16 planes
  const bool planes = c.act_dtype == SWITCH_BF16 && !swl::router_fused_ok(true, (int)N);
  lo.planes = take(planes ? 3 * sizeof(uint16_t) * (size_t)N * (size_t)c.d_model : 0);
  lo.ppart = take(sizeof(float) * (size_t)nc * (size_t)N);
  lo.hist = take(sizeof(int32_t) * (size_t)nc * (size_t)N);
  lo.rank = take(sizeof(int32_t) * (size_t)T * (size_t)top_k(c));
  lo.load = take(sizeof(int32_t) * (size_t)N);
  lo.nkept = take(sizeof(int32_t) * (size_t)N);
  lo.terms = take(sizeof(double) * (size_t)N);
  lo.tiles = take(sizeof(int32_t) * (size_t)(N + 1));
  lo.tok = take(sizeof(int32_t) * (size_t)N * (size_t)Cb);
  // the bf16 path reads token rows in place; only the fp32 path gathers them
  const bool gather_copy = c.act_dtype != SWITCH_BF16;
  lo.xbuf = take(gather_copy ? es * (size_t)N * (size_t)Cb * (size_t)c.d_model : 0);
  lo.hbuf = take(es * (size_t)N * (size_t)Cb * (size_t)c.d_ff);
  lo.ybuf = take(es * (size_t)N * (size_t)Cb * (size_t)c.d_model);
  lo.yflag = take(sizeof(int32_t));  // 1: ybuf holds this call's expert outputs
  lo.hflag = take(sizeof(int32_t));  // 1: hbuf holds this call's hidden activations
  lo.total = off;
  return lo;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Device address of the current device's copy of `scratch`, looked up once per
// device (hipGetSymbolAddress with that device current); NULL if the lookup
// failed.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];
bool g_scratch_done[kMaxDevices];

void* scratch_on(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_done[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) {
      p = nullptr;
      (void)hipGetLastError();  // reported by switch_forward_noalloc as SWITCH_E_HIP
    }
    g_scratch_ptr[dev] = p;
    g_scratch_done[dev] = true;
  }
  return g_scratch_ptr[dev];
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return na && nb && x < y + nb && y < x + na;
}

switch_status check_device(const switch_layer* L) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return SWITCH_E_HIP;
  return dev == L->device ? SWITCH_OK : SWITCH_E_INVALID;
}

// Common validation of the routing outputs and the workspace.
switch_status check_route_args(const switch_layer* L, int64_t T, const int32_t* expert_idx,
                               const float* gate, const int32_t* position,
                               const uint8_t* drop_mask, const float* aux_loss, void* ws,
                               size_t ws_bytes) {
  if (!L) return SWITCH_E_INVALID;
  if (T < 0 || T > L->cfg.t_max) return SWITCH_E_INVALID;
  if (!aux_loss || !aligned(aux_loss, 4)) return SWITCH_E_INVALID;
  if (T > 0 && (!expert_idx || !gate || !position || !drop_mask)) return SWITCH_E_INVALID;
  if (!aligned(expert_idx, 4) || !aligned(gate, 4) || !aligned(position, 4))
    return SWITCH_E_INVALID;
  if (!ws || !aligned(ws, 16)) return SWITCH_E_INVALID;
  if (ws_bytes < layout_of(L, T).total) return SWITCH_E_INVALID;
  return SWITCH_OK;
}

struct Routed {
  int32_t* load;
  int32_t* nkept;
  int32_t* tile_start;
  int32_t* offsets;
  int32_t* rank;
  int64_t chunk;
  int64_t Cb;
  // set when the scan is left to the one-launch assignment (finish_assignment)
  bool one_launch = false;
  int64_t nc = 0;
  float* ppart = nullptr;
  float* aux = nullptr;
  const int32_t* expert_idx = nullptr;
  int tile_rows = swl::kWideTileRows;  // rows per tile of the compact tile list
};

// Routing stage (logits, softmax / top-1 / gate, chunk statistics, scan and
// the load-balancing loss).  `x` may be NULL when `given_logits` holds the
// logits.  Positions and drops are finalised later: by dispatch in a forward
// call, by finalize_positions otherwise.
Routed enqueue_routing(switch_layer* L, const void* x, const float* given_logits, int64_t T,
                       float* logits_out, int32_t* expert_idx, float* gate, float* aux_loss,
                       int32_t* load, char* ws, const Layout& lo, hipStream_t s,
                       int tile_rows = swl::kWideTileRows) {
  const switch_config& c = L->cfg;
  const int N = c.n_experts;
  const bool bf16 = c.act_dtype == SWITCH_BF16;
  swl::Profiler* P = &L->prof;
  Routed r;
  r.Cb = buffer_rows(c, T);
  r.load = load ? load : (int32_t*)(ws + lo.load);
  r.nkept = (int32_t*)(ws + lo.nkept);
  r.tile_start = (int32_t*)(ws + lo.tiles);
  r.offsets = (int32_t*)(ws + lo.hist);
  r.rank = (int32_t*)(ws + lo.rank);
  float* ppart = (float*)(ws + lo.ppart);
  const bool fused = !given_logits && swl::router_fused_ok(bf16, N);
  r.chunk = fused ? chunk_tokens(c) : kRowsChunk;
  if (T > 0) {
    if (fused) {
      swl::prof_mark(P, s, "router");
      swl::launch_router_fused((const uint16_t*)x, L->W_r, L->b_r, T, c.d_model, N, top_k(c),
                               logits_out, expert_idx, gate, ppart, r.offsets, r.rank, s);
    } else {
      const float* h = given_logits;
      if (!h) {
        float* hw = logits_out ? logits_out : (float*)(ws + lo.logits);
        swl::prof_mark(P, s, "router_logits");
        swl::launch_router_logits(x, bf16, L->W_r, L->b_r, hw, T, c.d_model, N,
                                  (uint16_t*)(ws + lo.planes), s);
        h = hw;
      }
      swl::prof_mark(P, s, "route_rows");
      swl::launch_route_rows(h, T, N, top_k(c), expert_idx, gate, ppart, r.offsets, r.rank, s);
    }
  }
  const int64_t nc = (T + r.chunk - 1) / r.chunk;
  r.nc = nc;
  r.ppart = ppart;
  r.aux = aux_loss;
  r.expert_idx = expert_idx;
  r.one_launch = T > 0 && swl::assign_one_launch_ok(N, nc, r.chunk);
  r.tile_rows = tile_rows;
  if (!r.one_launch) {
    swl::prof_mark(P, s, "route_scan");
    swl::launch_route_scan(r.offsets, ppart, nc, N, T, top_k(c), r.Cb, c.alpha, r.load, r.nkept,
                           (double*)(ws + lo.terms), aux_loss, r.tile_start, tile_rows, s);
  }
  return r;
}

// With the one-launch assignment: scan, loss, positions, drops, the slot
// table (tok, may be NULL) and the row copies of copy_mode in one kernel.
void finish_assignment(switch_layer* L, const Routed& r, int64_t T, int32_t* position,
                       uint8_t* drop_mask, int32_t* tok, int copy_mode, const void* x, void* dst,
                       hipStream_t s) {
  const switch_config& c = L->cfg;
  swl::prof_mark(&L->prof, s, "assign");
  swl::launch_assign(r.offsets, r.ppart, r.nc, c.n_experts, T, top_k(c), r.chunk, r.Cb, c.alpha,
                     r.expert_idx, r.rank, r.load, r.nkept, r.aux, r.tile_start,
                     r.tile_rows, position, drop_mask, tok, copy_mode,
                     (int)(dtype_size(c.act_dtype) * (size_t)c.d_model), x, dst, s);
}

// Whether a forward call runs the fused expert FFN (H kept on chip): bf16 top-1
// layers of a shape the kernel takes, when the caller wants neither the expert
// outputs (debug hook) nor Y kept for a backward, and the layer asks for it.
// The automatic mode keeps the two-launch matmuls: on every workload measured
// (Switch-Base, Zipf overflow, Switch-Large shapes) they are faster.
bool fused_ffn(const switch_layer* L, int64_t T, bool want_y) {
  const switch_config& c = L->cfg;
  (void)T;
  if (c.act_dtype != SWITCH_BF16 || top_k(c) != 1 || want_y || L->keep_y) return false;
  if (!swl::ffn_fused_shape_ok(c.d_model, c.d_ff)) return false;
  return L->ffn_mode == SWITCH_FFN_FUSED;
}

switch_status forward_impl(switch_layer* L, const void* x, int64_t T, void* out,
                           int32_t* expert_idx, float* gate, int32_t* position,
                           uint8_t* drop_mask, float* aux_loss, float* logits, int32_t* load,
                           void* ws, size_t ws_bytes, void* expert_out, hipStream_t s) {
  switch_status st = check_route_args(L, T, expert_idx, gate, position, drop_mask, aux_loss, ws,
                                      ws_bytes);
  if (st != SWITCH_OK) return st;
  const switch_config& c = L->cfg;
  const size_t es = dtype_size(c.act_dtype);
  const size_t xbytes = es * (size_t)T * (size_t)c.d_model;
  if (T > 0 && (!x || !out)) return SWITCH_E_INVALID;
  if (!aligned(x, 16) || !aligned(out, 16) || !aligned(logits, 4) || !aligned(load, 4) ||
      !aligned(expert_out, 16))
    return SWITCH_E_INVALID;
  if (overlaps(x, xbytes, out, xbytes)) return SWITCH_E_INVALID;
  if ((st = check_device(L)) != SWITCH_OK) return st;

  const Layout lo = layout_of(L, T);
  char* w = (char*)ws;
  const int N = c.n_experts, d = c.d_model, F = c.d_ff;
  const bool bf16 = c.act_dtype == SWITCH_BF16;
  swl::Profiler* P = &L->prof;
  swl::prof_begin(P);

  const bool ffn1 = T > 0 && fused_ffn(L, T, expert_out != nullptr);
  Routed r = enqueue_routing(L, x, nullptr, T, logits, expert_idx, gate, aux_loss, load, w, lo, s,
                             ffn1 ? swl::kFfnTileRows : swl::kWideTileRows);
  const int64_t Cb = r.Cb;
  void* xbuf = w + lo.xbuf;
  void* hbuf = w + lo.hbuf;
  void* ybuf = w + lo.ybuf;
  const int k = top_k(c);
  if (T > 0 && bf16) {
    // rows stay in place: dispatch records the slot table, GEMM1 gathers
    // through it, GEMM2 combines into out (top-1 without a copy of the expert
    // output), or stores the expert output for the combine pass (top-2, where
    // two experts add into one row, or when the caller asks for it)
    int32_t* tok = (int32_t*)(w + lo.tok);
    swl::GemmIO io;
    io.tile_start = r.tile_start;
    io.tok = tok;
    io.x = (const uint16_t*)x;
    io.gate = gate;
    io.out = (uint16_t*)out;
    const bool fused = !expert_out && k == 1;
    if (r.one_launch) {
      finish_assignment(L, r, T, position, drop_mask, tok, fused ? 1 : 0, x, out, s);
    } else {
      swl::prof_mark(P, s, "dispatch");
      swl::launch_dispatch_index(x, T, k, (int)(es * d), expert_idx, r.rank, r.offsets, N,
                                 r.chunk, Cb, position, drop_mask, tok, fused, out, s);
    }
    if (ffn1) {
      // both matmuls, the ReLU and the combine in one launch, H on chip
      swl::prof_mark(P, s, "ffn_fused");
      swl::launch_ffn_fused(x, L->W_in, L->W_out, r.nkept, r.tile_start, tok, gate, out, d, F,
                            Cb, N, (int32_t*)(w + lo.yflag), (int32_t*)(w + lo.hflag), s);
      swl::prof_end(P, s);
      return hipGetLastError() == hipSuccess ? SWITCH_OK : SWITCH_E_HIP;
    }
    // the first matmul records in the workspace that hbuf holds H
    swl::GemmIO io1 = io;
    io1.yflag = (int32_t*)(w + lo.hflag);
    io1.yflag_value = 1;
    swl::prof_mark(P, s, "gemm1_relu");
    swl::launch_expert_gemm_bf16(swl::kRowsGather, true, nullptr, 0, L->W_in, (int64_t)F * d,
                                 hbuf, Cb * F, r.nkept, N, Cb, d, F, io1, s);
    // GEMM2 runs on the same tiles with or without the fused combine, so both
    // paths give the same expert outputs (the tile list of 256-row tiles
    // applies when the wide kernel is chosen)
    // the second matmul records in the workspace whether ybuf holds Y: always
    // on the dense path, on the fused path when the layer keeps it
    swl::GemmIO io2 = io;
    io2.yflag = (int32_t*)(w + lo.yflag);
    if (fused) {
      swl::prof_mark(P, s, "gemm2_combine");
      io2.yflag_value = L->keep_y ? 1 : 0;
      io2.ykeep = L->keep_y ? (uint16_t*)ybuf : nullptr;
      swl::launch_expert_gemm_bf16(swl::kRowsCombine, false, hbuf, Cb * F, L->W_out,
                                   (int64_t)d * F, nullptr, 0, r.nkept, N, Cb, F, d, io2, s);
    } else {
      swl::prof_mark(P, s, "gemm2");
      io2.yflag_value = 1;
      swl::launch_expert_gemm_bf16(swl::kRowsDense, false, hbuf, Cb * F, L->W_out, (int64_t)d * F,
                                   ybuf, Cb * d, r.nkept, N, Cb, F, d, io2, s);
      swl::prof_mark(P, s, "combine");
      swl::launch_combine(x, bf16, T, k, (int)(es * d), expert_idx, position, drop_mask, gate, Cb,
                          ybuf, out, s);
      if (expert_out) {
        swl::prof_mark(P, s, "copy_expert_rows");
        swl::launch_copy_expert_rows(ybuf, r.nkept, N, Cb, (int)(es * d), expert_out, s);
      }
    }
  } else if (T > 0) {
    if (r.one_launch) {
      finish_assignment(L, r, T, position, drop_mask, nullptr, 2, x, xbuf, s);
    } else {
      swl::prof_mark(P, s, "dispatch");
      swl::launch_dispatch(x, T, k, (int)(es * d), expert_idx, r.rank, r.offsets, N, r.chunk, Cb,
                           position, drop_mask, xbuf, s);
    }
    swl::prof_mark(P, s, "gemm1_relu");
    swl::launch_expert_gemm(bf16, true, xbuf, Cb * d, L->W_in, (int64_t)F * d, hbuf, Cb * F,
                            r.nkept, N, Cb, d, F, s);
    swl::prof_mark(P, s, "gemm2");
    swl::launch_expert_gemm(bf16, false, hbuf, Cb * F, L->W_out, (int64_t)d * F, ybuf, Cb * d,
                            r.nkept, N, Cb, F, d, s);
    swl::prof_mark(P, s, "combine");
    swl::launch_combine(x, bf16, T, k, (int)(es * d), expert_idx, position, drop_mask, gate, Cb,
                        ybuf, out, s);
    if (expert_out) {
      swl::prof_mark(P, s, "copy_expert_rows");
      swl::launch_copy_expert_rows(ybuf, r.nkept, N, Cb, (int)(es * d), expert_out, s);
    }
  }
  swl::prof_end(P, s);
  return hipGetLastError() == hipSuccess ? SWITCH_OK : SWITCH_E_HIP;
}

switch_status route_impl(switch_layer* L, const void* x, const float* given_logits, int64_t T,
                         float* logits_out, int32_t* expert_idx, float* gate, int32_t* position,
                         uint8_t* drop_mask, float* aux_loss, int32_t* load, void* ws,
                         hipStream_t s) {
  const Layout lo = layout_of(L, T);
  swl::prof_begin(&L->prof);
  Routed r = enqueue_routing(L, x, given_logits, T, logits_out, expert_idx, gate, aux_loss, load,
                             (char*)ws, lo, s);
  if (r.one_launch) {
    finish_assignment(L, r, T, position, drop_mask, nullptr, 0, nullptr, nullptr, s);
  } else if (T > 0) {
    swl::prof_mark(&L->prof, s, "finalize");
    swl::launch_finalize_positions(T, top_k(L->cfg), expert_idx, r.rank, r.offsets,
                                   L->cfg.n_experts, r.chunk, r.Cb, position, drop_mask, s);
  }
  swl::prof_end(&L->prof, s);
  return hipGetLastError() == hipSuccess ? SWITCH_OK : SWITCH_E_HIP;
}

// Workspace of the backward pass (bf16 layers, top-1).  Cbp = Cb rounded up
// to 64: the weight-gradient matmuls run over the expert's rows as their K
// dimension, zero-padded to whole K steps.
struct BwdLayout {
  size_t nkept, tiles, tok, gs, hbuf, ybuf, du, dxe, xT, dh, wpart, bpart, total;
  int64_t Cb, Cbp;
};

BwdLayout bwd_layout_of(const switch_layer* L, int64_t T) {
  const switch_config& c = L->cfg;
  const size_t N = (size_t)c.n_experts, d = (size_t)c.d_model, F = (size_t)c.d_ff;
  BwdLayout lo;
  lo.Cb = buffer_rows(c, T);
  lo.Cbp = (lo.Cb + 63) / 64 * 64;
  const size_t Cb = (size_t)lo.Cb, Cbp = (size_t)lo.Cbp;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t at = off; off += align_up(bytes); return at; };
  lo.nkept = take(4 * N);
  lo.tiles = take(4 * (N + 1));
  lo.tok = take(4 * N * Cb);
  lo.gs = take(2 * N * Cb * d);
  lo.hbuf = take(2 * N * Cb * F);
  lo.ybuf = take(2 * N * Cb * d);
  lo.du = take(2 * N * Cb * F);
  lo.dxe = take(2 * N * Cb * d);
  lo.xT = take(2 * N * d * Cbp);
  lo.dh = take(4 * (size_t)T * N);
  const size_t slices = (size_t)swl::router_wgrad_slices(T, (int)N, (int)d);
  lo.wpart = take(4 * slices * N * d);
  lo.bpart = take(4 * slices * N);
  lo.total = off;
  return lo;
}

switch_status backward_impl(switch_layer* L, const void* x, int64_t T, const void* grad_out,
                            float grad_aux, const float* logits, const int32_t* expert_idx,
                            const float* gate, const int32_t* position, const uint8_t* drop_mask,
                            const int32_t* load, void* grad_x, float* grad_W_r, float* grad_b_r,
                            void* grad_W_in, void* grad_W_out, void* ws, void* fwd_ws,
                            hipStream_t s) {
  const switch_config& c = L->cfg;
  const int N = c.n_experts, d = c.d_model, F = c.d_ff;
  const BwdLayout lo = bwd_layout_of(L, T);
  const int64_t Cb = lo.Cb, Cbp = lo.Cbp;
  char* w = (char*)ws;
  int32_t* nkept = (int32_t*)(w + lo.nkept);
  int32_t* tok = (int32_t*)(w + lo.tok);
  void* gs = w + lo.gs;
  // the forward call's H when its workspace is given (the same tiles computed
  // it, so it equals the recomputation bit for bit); else recomputed here.  A
  // forward that ran the fused FFN left no H: its flag word says so, and the
  // recomputation then writes H into that workspace (decided on the device)
  const bool have_h = fwd_ws != nullptr;
  void* hbuf = have_h ? (void*)((char*)fwd_ws + layout_of(L, T).hbuf) : (void*)(w + lo.hbuf);
  const int32_t* hflag_fwd = have_h ? (const int32_t*)((const char*)fwd_ws + layout_of(L, T).hflag)
                                    : nullptr;
  void* ybuf = w + lo.ybuf;
  // its expert outputs too, when it kept them (decided on the device: the flag
  // word the forward's second matmul wrote)
  const Layout flo = layout_of(L, T);
  const int32_t* yflag_fwd = have_h ? (const int32_t*)((const char*)fwd_ws + flo.yflag) : nullptr;
  const void* ybuf_fwd = have_h ? (const void*)((const char*)fwd_ws + flo.ybuf) : nullptr;
  void* du = w + lo.du;
  void* dxe = w + lo.dxe;
  float* dh = (float*)(w + lo.dh);
  swl::Profiler* P = &L->prof;
  swl::prof_begin(P);
  if (T > 0) {
    swl::prof_mark(P, s, "bwd_slots");
    int32_t* tiles = (int32_t*)(w + lo.tiles);
    const int k = top_k(c);
    swl::launch_bwd_slots(grad_out, T, d, k, expert_idx, position, drop_mask, gate, Cb, tok, gs,
                          load, N, nkept, tiles, s);
    // io_rows: products over the experts' token rows with F columns (the tile
    // list of 256-row tiles applies); io: the rest
    swl::GemmIO io;
    io.tok = tok;
    io.x = (const uint16_t*)x;
    swl::GemmIO io_rows = io;
    io_rows.tile_start = tiles;
    if (Cb > 0) {
      swl::prof_mark(P, s, "recompute_h");
      swl::GemmIO ioh = io_rows;
      ioh.yskip = hflag_fwd;   // the forward stored H: the blocks exit at once
      swl::launch_expert_gemm_bf16(swl::kRowsGather, true, nullptr, 0, L->W_in, (int64_t)F * d,
                                   hbuf, Cb * F, nkept, N, Cb, d, F, ioh, s);
      // Y again, unless the forward call whose workspace is given kept it (its
      // flag word; the kernel's blocks then exit at once)
      swl::prof_mark(P, s, "recompute_y");
      swl::GemmIO ioy = io;
      ioy.yskip = yflag_fwd;
      swl::launch_expert_gemm_bf16(swl::kRowsDense, false, hbuf, Cb * F, L->W_out,
                                   (int64_t)d * F, ybuf, Cb * d, nkept, N, Cb, F, d, ioy, s);
    }
    swl::prof_mark(P, s, "router_bwd");
    // d aux / d p_i(t) = alpha N f_i / T with f_i = load_i / (k T)
    const float loss_scale = (float)((double)grad_aux * (double)c.alpha * (double)N /
                                     ((double)k * (double)T * (double)T));
    swl::launch_router_bwd(logits, T, N, d, k, grad_out, ybuf, ybuf_fwd, yflag_fwd, Cb,
                           expert_idx, position, drop_mask, load, loss_scale, dh, s);
    // the slices' partial sums; launch_grad_x adds them into grad_W_r and grad_b_r
    swl::launch_router_wgrad(dh, x, T, N, d, (float*)(w + lo.wpart), (float*)(w + lo.bpart),
                             grad_W_r, grad_b_r, false, s);
    if (Cb > 0) {
      // dU = (Gs W_out[e]) * [H > 0], W_out[e] read as stored ([d][F], K = d outer)
      swl::prof_mark(P, s, "grad_h");
      io_rows.mask = (const uint16_t*)hbuf;
      io_rows.ldb = F;
      swl::launch_expert_gemm_bf16_t(swl::kRowsMask, false, false, true, gs, Cb * d, L->W_out,
                                     (int64_t)d * F, du, Cb * F, nkept, N, Cb, d, F, io_rows, s);
      // dX = dU W_in[e], W_in[e] read as stored ([F][d], K = F outer)
      swl::prof_mark(P, s, "grad_x_expert");
      swl::GemmIO io_w = io;
      io_w.ldb = d;
      swl::launch_expert_gemm_bf16_t(swl::kRowsDense, false, false, true, du, Cb * F, L->W_in,
                                     (int64_t)F * d, dxe, Cb * d, nkept, N, Cb, F, d, io_w, s);
      // the gathered token rows, K (the expert's rows) innermost, zero past n_kept
      swl::prof_mark(P, s, "x_transpose");
      void* xT = w + lo.xT;
      swl::launch_transpose(x, 0, d, (int)Cb, d, nkept, tok, xT, (int64_t)d * Cbp, (int)Cbp, N,
                            s);
      // dW_out[e] = Gs^T H and dW_in[e] = dU^T X over the expert's rows (K = Cbp,
      // rows at or past n_kept read as zero): Gs, H and dU read as stored
      swl::GemmIO io_g = io;
      io_g.krows = nkept;
      swl::prof_mark(P, s, "grad_w_out");
      io_g.lda = d;
      io_g.ldb = F;
      swl::launch_expert_gemm_bf16_t(swl::kRowsDense, false, true, true, gs, Cb * d, hbuf, Cb * F,
                                     grad_W_out, (int64_t)d * F, nullptr, N, d, (int)Cbp, F, io_g,
                                     s);
      swl::prof_mark(P, s, "grad_w_in");
      io_g.lda = F;
      io_g.ldb = 0;
      swl::launch_expert_gemm_bf16_t(swl::kRowsDense, false, true, false, du, Cb * F, xT,
                                     (int64_t)d * Cbp, grad_W_in, (int64_t)F * d, nullptr, N, F,
                                     (int)Cbp, d, io_g, s);
    }
    swl::prof_mark(P, s, "grad_x");
    swl::launch_grad_x(grad_out, T, d, k, expert_idx, position, drop_mask, Cb, dxe, dh, L->W_r, N,
                       grad_x, (const float*)(w + lo.wpart), (const float*)(w + lo.bpart),
                       grad_W_r, grad_b_r, s);
  }
  if (T == 0 || Cb == 0) {
    // no token reached an expert: the expert weights get no gradient
    swl::launch_fill_zero(grad_W_in, (size_t)N * F * d * 2, s);
    swl::launch_fill_zero(grad_W_out, (size_t)N * d * F * 2, s);
  }
  if (T == 0) {
    // no tokens: the router gradient sums are empty (the kernel writes zeros)
    swl::launch_router_wgrad(dh, x, 0, N, d, (float*)(w + lo.wpart), (float*)(w + lo.bpart),
                             grad_W_r, grad_b_r, true, s);
  }
  swl::prof_end(P, s);
  return hipGetLastError() == hipSuccess ? SWITCH_OK : SWITCH_E_HIP;
}

}  // namespace

namespace swl {
thread_local StageEvents* g_stage = nullptr;
}

extern "C" {

switch_status switch_layer_create(const switch_config* cfg, const float* W_r, const float* b_r,
                                  const void* W_in, const void* W_out, switch_layer** out) {
  if (!cfg || !out) return SWITCH_E_INVALID;
  *out = nullptr;
  const switch_config& c = *cfg;
  if (c.n_experts < 1 || c.n_experts > 8192) return SWITCH_E_INVALID;
  if (c.d_model < 8 || c.d_model % 8 != 0 || c.d_ff < 8 || c.d_ff % 8 != 0)
    return SWITCH_E_INVALID;
  if (c.t_max < 0 || c.t_max > 0x7fffffff) return SWITCH_E_INVALID;
  if (!(c.capacity_factor >= 0.0) || !isfinite(c.capacity_factor)) return SWITCH_E_INVALID;
  if (c.capacity_override < 0 || !isfinite(c.alpha)) return SWITCH_E_INVALID;
  const int k = c.top_k == 0 ? 1 : c.top_k;
  if (k < 1 || k > swl::kMaxTopK || k > c.n_experts) return SWITCH_E_INVALID;
  if ((c.act_dtype != SWITCH_F32 && c.act_dtype != SWITCH_BF16) ||
      (c.expert_dtype != SWITCH_F32 && c.expert_dtype != SWITCH_BF16))
    return SWITCH_E_INVALID;
  if (!W_r || !W_in || !W_out) return SWITCH_E_INVALID;
  if (!aligned(W_r, 16) || !aligned(W_in, 16) || !aligned(W_out, 16) || !aligned(b_r, 4))
    return SWITCH_E_INVALID;
  if (c.act_dtype != c.expert_dtype) return SWITCH_E_UNSUPPORTED;
  if (!swl::expert_gemm_shape_ok(c.act_dtype == SWITCH_BF16, c.d_model, c.d_ff))
    return SWITCH_E_UNSUPPORTED;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return SWITCH_E_HIP;
  switch_layer* L = new (std::nothrow) switch_layer();
  if (!L) return SWITCH_E_INVALID;
  L->cfg = c;
  L->cfg.top_k = k;
  L->W_r = W_r;
  L->b_r = b_r;
  L->W_in = W_in;
  L->W_out = W_out;
  L->device = dev;
  L->scratch = scratch_on(dev);
  *out = L;
  return SWITCH_OK;
}

void switch_layer_destroy(switch_layer* L) {
  if (!L) return;
  (void)switch_profile_enable(L, 0);
  delete L;
}

int64_t switch_capacity(const switch_layer* L, int64_t T) {
  if (!L || T < 0) return -1;
  return capacity_of(L->cfg, T);
}

size_t switch_workspace_bytes(const switch_layer* L, int64_t T) {
  if (!L || T < 0 || T > L->cfg.t_max) return 0;
  return layout_of(L, T).total;
}

switch_status switch_route(switch_layer* L, const void* x, int64_t T, float* logits,
                           int32_t* expert_idx, float* gate, int32_t* position,
                           uint8_t* drop_mask, float* aux_loss, int32_t* load, void* ws,
                           size_t ws_bytes, void* stream) {
  switch_status st = check_route_args(L, T, expert_idx, gate, position, drop_mask, aux_loss, ws,
                                      ws_bytes);
  if (st != SWITCH_OK) return st;
  if (T > 0 && !x) return SWITCH_E_INVALID;
  if (!aligned(x, 16) || !aligned(logits, 4) || !aligned(load, 4)) return SWITCH_E_INVALID;
  if ((st = check_device(L)) != SWITCH_OK) return st;
  return route_impl(L, x, nullptr, T, logits, expert_idx, gate, position, drop_mask, aux_loss,
                    load, ws, (hipStream_t)stream);
}

switch_status switch_route_from_logits(switch_layer* L, const float* logits, int64_t T,
                                       int32_t* expert_idx, float* gate, int32_t* position,
                                       uint8_t* drop_mask, float* aux_loss, int32_t* load,
                                       void* ws, size_t ws_bytes, void* stream) {
  switch_status st = check_route_args(L, T, expert_idx, gate, position, drop_mask, aux_loss, ws,
                                      ws_bytes);
  if (st != SWITCH_OK) return st;
  if ((T > 0 && !logits) || !aligned(logits, 4) || !aligned(load, 4)) return SWITCH_E_INVALID;
  if ((st = check_device(L)) != SWITCH_OK) return st;
  return route_impl(L, nullptr, logits, T, nullptr, expert_idx, gate, position, drop_mask,
                    aux_loss, load, ws, (hipStream_t)stream);
}

switch_status switch_forward(switch_layer* L, const void* x, int64_t T, void* out,
                             int32_t* expert_idx, float* gate, int32_t* position,
                             uint8_t* drop_mask, float* aux_loss, float* logits, int32_t* load,
                             void* ws, size_t ws_bytes, void* stream) {
  return forward_impl(L, x, T, out, expert_idx, gate, position, drop_mask, aux_loss, logits, load,
                      ws, ws_bytes, nullptr, (hipStream_t)stream);
}

switch_status switch_forward_noalloc(switch_layer* L, const void* x, int64_t T, void* out,
                                     int32_t* expert_idx, float* gate, int32_t* position,
                                     uint8_t* drop_mask, float* aux_loss, float* logits,
                                     int32_t* load, void* stream) {
  if (!L || T < 0 || T > L->cfg.t_max) return SWITCH_E_INVALID;
  if (layout_of(L, T).total > SWITCH_NOALLOC_SCRATCH_BYTES) return SWITCH_E_TOO_LARGE;
  switch_status st = check_device(L);
  if (st != SWITCH_OK) return st;
  if (!L->scratch) return SWITCH_E_HIP;
  return forward_impl(L, x, T, out, expert_idx, gate, position, drop_mask, aux_loss, logits, load,
                      L->scratch, SWITCH_NOALLOC_SCRATCH_BYTES, nullptr, (hipStream_t)stream);
}

switch_status switch_forward_debug(switch_layer* L, const void* x, int64_t T, void* out,
                                   int32_t* expert_idx, float* gate, int32_t* position,
                                   uint8_t* drop_mask, float* aux_loss, float* logits,
                                   int32_t* load, void* ws, size_t ws_bytes, void* expert_out,
                                   void* stream) {
  // an empty expert buffer (capacity 0 or T = 0) may come as NULL
  if (!L || (!expert_out && T >= 0 && T <= L->cfg.t_max && buffer_rows(L->cfg, T) > 0))
    return SWITCH_E_INVALID;
  return forward_impl(L, x, T, out, expert_idx, gate, position, drop_mask, aux_loss, logits, load,
                      ws, ws_bytes, expert_out, (hipStream_t)stream);
}

size_t switch_backward_workspace_bytes(const switch_layer* L, int64_t T) {
  if (!L || T < 0 || T > L->cfg.t_max) return 0;
  return bwd_layout_of(L, T).total;
}

switch_status switch_backward(switch_layer* L, const void* x, int64_t T, const void* grad_out,
                              float grad_aux, const float* logits, const int32_t* expert_idx,
                              const float* gate, const int32_t* position,
                              const uint8_t* drop_mask, const int32_t* load, void* grad_x,
                              float* grad_W_r, float* grad_b_r, void* grad_W_in,
                              void* grad_W_out, void* ws, size_t ws_bytes, void* fwd_ws,
                              size_t fwd_ws_bytes, void* stream) {
  if (!L || T < 0 || T > L->cfg.t_max) return SWITCH_E_INVALID;
  const switch_config& c = L->cfg;
  if (c.act_dtype != SWITCH_BF16) return SWITCH_E_UNSUPPORTED;
  if (!isfinite(grad_aux)) return SWITCH_E_INVALID;
  if (T > 0 && (!x || !grad_out || !logits || !expert_idx || !gate || !position || !drop_mask ||
                !grad_x))
    return SWITCH_E_INVALID;
  if (!load || !grad_W_r || !grad_W_in || !grad_W_out || !ws) return SWITCH_E_INVALID;
  if (!aligned(x, 16) || !aligned(grad_out, 16) || !aligned(grad_x, 16) || !aligned(logits, 4) ||
      !aligned(expert_idx, 4) || !aligned(gate, 4) || !aligned(position, 4) ||
      !aligned(load, 4) || !aligned(grad_W_r, 16) || !aligned(grad_b_r, 16) ||
      !aligned(grad_W_in, 16) || !aligned(grad_W_out, 16) || !aligned(ws, 16))
    return SWITCH_E_INVALID;
  if (ws_bytes < bwd_layout_of(L, T).total) return SWITCH_E_INVALID;
  if (fwd_ws && (!aligned(fwd_ws, 16) || fwd_ws_bytes < layout_of(L, T).total))
    return SWITCH_E_INVALID;
  const size_t xbytes = (size_t)T * (size_t)c.d_model * 2;
  if (overlaps(grad_x, xbytes, x, xbytes) || overlaps(grad_x, xbytes, grad_out, xbytes))
    return SWITCH_E_INVALID;
  switch_status st = check_device(L);
  if (st != SWITCH_OK) return st;
  return backward_impl(L, x, T, grad_out, grad_aux, logits, expert_idx, gate, position, drop_mask,
                       load, grad_x, grad_W_r, grad_b_r, grad_W_in, grad_W_out, ws, fwd_ws,
                       (hipStream_t)stream);
}

switch_status switch_set_ffn_mode(switch_layer* L, int mode) {
  if (!L || (mode != SWITCH_FFN_AUTO && mode != SWITCH_FFN_UNFUSED && mode != SWITCH_FFN_FUSED))
    return SWITCH_E_INVALID;
  if (mode == SWITCH_FFN_FUSED &&
      (L->cfg.act_dtype != SWITCH_BF16 || top_k(L->cfg) != 1 ||
       !swl::ffn_fused_shape_ok(L->cfg.d_model, L->cfg.d_ff)))
    return SWITCH_E_UNSUPPORTED;
  L->ffn_mode = mode;
  return SWITCH_OK;
}

switch_status switch_set_keep_expert_out(switch_layer* L, int keep) {
  if (!L || (keep != 0 && keep != 1)) return SWITCH_E_INVALID;
  L->keep_y = keep;
  return SWITCH_OK;
}

switch_status switch_profile_enable(switch_layer* L, int max_calls) {
  if (!L || max_calls < 0) return SWITCH_E_INVALID;
  swl::Profiler& P = L->prof;
  if (swl::g_stage == &P.cur) swl::g_stage = nullptr;
  if (P.ev) {
    for (int i = 0; i < P.max_calls * swl::Profiler::kMax * 2; ++i) (void)hipEventDestroy(P.ev[i]);
    delete[] P.ev;
    P.ev = nullptr;
  }
  P.on = false;
  P.max_calls = 0;
  P.calls = 0;
  P.n = 0;
  if (max_calls == 0) return SWITCH_OK;
  const int count = max_calls * swl::Profiler::kMax * 2;
  P.ev = new (std::nothrow) hipEvent_t[count];
  if (!P.ev) return SWITCH_E_INVALID;
  for (int i = 0; i < count; ++i) {
    if (hipEventCreate(&P.ev[i]) != hipSuccess) {
      for (int j = 0; j < i; ++j) (void)hipEventDestroy(P.ev[j]);
      delete[] P.ev;
      P.ev = nullptr;
      return SWITCH_E_HIP;
    }
  }
  P.max_calls = max_calls;
  P.on = true;
  return SWITCH_OK;
}

int switch_profile_read(switch_layer* L, float* ms, const char** names, int cap) {
  if (!L || !L->prof.ev || cap < 0) return -1;
  swl::Profiler& P = L->prof;
  if (P.calls == 0) return 0;
  const int stride = swl::Profiler::kMax * 2;
  // every recorded call of this session has the same stages (the last one's)
  const int n = P.n;
  if (hipEventSynchronize(P.ev[(P.calls - 1) * stride + 2 * (n - 1) + 1]) != hipSuccess) return -1;
  for (int i = 0; i < n && i < cap; ++i) {
    double sum = 0.0;
    for (int c = 0; c < P.calls; ++c) {
      float t = 0.f;
      const hipEvent_t* e = P.ev + c * stride + 2 * i;
      if (hipEventElapsedTime(&t, e[0], e[1]) != hipSuccess) return -1;
      sum += t;
    }
    if (ms) ms[i] = (float)(sum / P.calls);
    if (names) names[i] = P.names[i];
  }
  return n;
}

const char* switch_status_string(switch_status s) {
  switch (s) {
    case SWITCH_OK: return "SWITCH_OK";
    case SWITCH_E_INVALID: return "SWITCH_E_INVALID: invalid argument";
    case SWITCH_E_UNSUPPORTED: return "SWITCH_E_UNSUPPORTED: unsupported dtype or shape";
    case SWITCH_E_HIP: return "SWITCH_E_HIP: HIP runtime error";
    case SWITCH_E_TOO_LARGE:
      return "SWITCH_E_TOO_LARGE: the call needs more than the no-allocation scratch array";
  }
  return "unknown switch_status";
}

switch_status switch_last_async_error(switch_layer* L, void* stream) {
  if (!L) return SWITCH_E_INVALID;
  const switch_status st = check_device(L);
  if (st != SWITCH_OK) return st;
  const hipError_t launch = hipGetLastError();
  const hipError_t q = hipStreamQuery((hipStream_t)stream);
  if (launch != hipSuccess || (q != hipSuccess && q != hipErrorNotReady)) return SWITCH_E_HIP;
  return SWITCH_OK;
}

}  // extern "C"
