// Internal definitions shared by the library's translation units.
// Not part of the ABI (include/mok.h is).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <vector>

#include "mok.h"

namespace mok {

// ---------------------------------------------------------------------------
// Schedule buffer
// ---------------------------------------------------------------------------
enum HeaderField : int {
  HDR_T = 0,
  HDR_K = 1,
  HDR_E = 2,
  HDR_C = 3,
  HDR_P = 4,
  HDR_ROWS_CAP = 5,
  HDR_NMB = 6,
  HDR_MB = 7,
  HDR_DROPPED = 8,
  HDR_INVALID = 9,
  HDR_ROWS_TOTAL = 10,
  HDR_HASH = 11,
  HDR_INTS = 16
};

// Tile heights whose per-expert tile prefix sums the schedule carries.
constexpr int kNumTileBMs = 4;
constexpr int kTileBM[kNumTileBMs] = {32, 64, 128, 256};
__host__ __device__ constexpr int tile_bm_index(int bm) { return bm == 32 ? 0 : bm == 64 ? 1 : bm == 128 ? 2 : 3; }

struct Layout {
  size_t header, counts, kept, offsets, mb_offsets, row_src, slot_row, tiles, total;
  int64_t rows_cap_max, n_mb_max;
};

int64_t capacity(int64_t T, float mult);
int64_t rows_cap(const mok_config& c, int64_t T);
int64_t n_minibatches(const mok_config& c, int64_t T);
// The forward streams the batch through a token ring (0 < macrobatch_size < max_tokens).
bool ring(const mok_config& c);
// Tokens per schedule sub-offset step: minibatch_size, else the macrobatch in ring mode (0 = none).
int64_t sub_offset_tokens(const mok_config& c);
Layout schedule_layout(const mok_config& c);
uint32_t config_hash(const mok_config& c);

// Device view of a schedule buffer (all int32).
struct SchedView {
  int32_t* header;
  int32_t* counts;
  int32_t* kept;
  int32_t* offsets;     // [E+1]
  int32_t* mb_offsets;  // [(n_mb_max+1)*E]
  int32_t* row_src;     // [rows_cap_max]
  int32_t* slot_row;    // [T_max*k]
  int32_t* tiles;       // [4][E+2]
  // not part of the buffer: the hash of the configuration the reading
  // launches expect in header[HDR_HASH], and where they count a mismatch
  int hash = 0;
  int32_t* status = nullptr;
};
SchedView sched_view(void* base, const Layout& L);

// ---------------------------------------------------------------------------
// Workspace
// ---------------------------------------------------------------------------
struct TimedLaunch {
  int kernel;
  hipEvent_t start, stop;
};

// Transposed operands of the weight-gradient GEMMs (bf16 elements, or MXFP8
// codes quantized in 32-row blocks with their scales). Expert e's block of an
// array with `cols` columns starts at element kofs_e * cols (kofs_e = 128 *
// the expert's first 128-row tile) and is [cols, K_e] with K_e = 128 * its
// 128-row tile count (rows past the segment are zero); MXFP8 scales start at
// kofs_e / 32 * cols and are [cols, K_e / 32]. The shared expert's block sits
// at K offset kr_cap (a static bound on the routed total).
struct TqArrays {
  uint8_t* x;       // cols H: x rows of the expert (shared: all tokens)
  uint8_t* dy;      // cols H: w * grad_out rows
  uint8_t* h;       // cols I (shared: I_s): h rows (dequantized forward codes)
  uint8_t* dg;      // cols I: dG rows
  uint8_t* du;      // cols I: dU rows
  uint8_t* xs;      // scales of each
  uint8_t* dys;
  uint8_t* hs;
  uint8_t* dgs;
  uint8_t* dus;
  int64_t kr_cap;   // K offset of the shared expert's blocks (multiple of 128)
};

// Device scratch of the backward, sized for the configuration. The MXFP8
// backward's buffers are carved from the same regions as the BF16 ones
// (a backward runs in one mode at a time).
struct BwdScratch {
  uint16_t* wdT = nullptr;  // [E, I, H] transposed routed down weights
  uint16_t* wgT = nullptr;  // [E, H, I]
  uint16_t* wuT = nullptr;
  uint16_t* sdT = nullptr;  // [I_s, H]
  uint16_t* sgT = nullptr;  // [H, I_s]
  uint16_t* suT = nullptr;
  uint16_t* dg = nullptr;   // dG, dU: routed [rows_cap_max, I] then shared [T_max, I_s]
  uint16_t* du = nullptr;
  uint16_t* hw = nullptr;   // (the MXFP8 backward keeps dU's codes at the start of the region)
  float* dw_part = nullptr;      // [rows_cap_max + T_max, dw_parts(cfg)]
  // MXFP8: transposed weights quantized along their new rows (codes, scales)
  uint8_t *wdTq = nullptr, *wgTq = nullptr, *wuTq = nullptr, *sdTq = nullptr, *sgTq = nullptr, *suTq = nullptr;
  uint8_t *wdTs = nullptr, *wgTs = nullptr, *wuTs = nullptr, *sdTs = nullptr, *sgTs = nullptr, *suTs = nullptr;
  // MXFP8: dU quantized along I (dG uses the workspace's hq buffer)
  uint8_t* duq = nullptr;
  uint8_t* duq_scale = nullptr;
  // operands of the weight-gradient GEMMs: MXFP8 (tq) and bf16 (tq16)
  TqArrays tq{};
  TqArrays tq16{};
  bool mxfp8_ready = false;  // the configuration admits the MXFP8 backward and its buffers exist
};

}  // namespace mok

struct mok_workspace {
  mok_config cfg;
  int device;
  int num_cus;
  mok::Layout layout;
  // scratch
  char* scratch = nullptr;
  size_t scratch_bytes = 0;
  int32_t* chunk_hist = nullptr;   // [n_chunks_max * E]
  int64_t n_chunks_max = 0;
  void* hbuf = nullptr;            // h (bf16) or MXFP8 h codes + scales when no context is kept
  size_t hbuf_bytes = 0;
  void* ybuf = nullptr;            // bf16 [(rows_cap_max + T_max) * H]
  uint8_t* xq = nullptr;           // E4M3 [T_max * H]
  uint8_t* xq_scale = nullptr;     // [T_max * H/32]
  uint8_t* hq = nullptr;           // E4M3 h (routed rows then shared rows)
  uint8_t* hq_scale = nullptr;     // its E8M0 scales, one per 32 along I
  // backward scratch
  mok::BwdScratch bwd;
  // minibatch pipeline of the down GEMM: per-minibatch finished-tile
  // counters; status words: [0] mover waits that ran out of time, [1]
  // launches that found a schedule of another configuration
  int32_t* pipe_cnt = nullptr;     // [n_mb_max]
  int32_t* status = nullptr;       // [2]
  // token ring (0 < macrobatch_size < max_tokens): one macrobatch's schedule
  void* pass_sched = nullptr;
  // timing
  uint32_t timing_mask = 0;  // bit k: time launches of kernel id k
  std::vector<mok::TimedLaunch> launches;
  std::vector<hipEvent_t> event_pool;
};

namespace mok {

// Event bracket around one launch when timing is enabled.
struct LaunchTimer {
  mok_workspace* ws;
  int kernel;
  hipStream_t stream;
  hipEvent_t a = nullptr, b = nullptr;
  LaunchTimer(mok_workspace* w, int k, hipStream_t s);
  ~LaunchTimer();
};

// ---------------------------------------------------------------------------
// Launchers (each returns hipSuccess or the launch error)
// ---------------------------------------------------------------------------
hipError_t launch_schedule(mok_workspace* ws, const int64_t* top, int64_t T, void* sched, hipStream_t s);
// One macrobatch of the token ring: its schedule, in the pass layout
// (pass_config), cut out of the whole batch's.
mok_config pass_config(const mok_config& c);
hipError_t launch_sched_slice(mok_workspace* ws, const void* sched, int pass, void* pass_sched, hipStream_t s);

hipError_t launch_quantize(const void* src, int src_is_fp32, int64_t rows, int64_t cols, int64_t ld_src, int axis,
                           uint8_t* dst, int64_t ld_dst, uint8_t* dst_scale, hipStream_t s);

struct FwdArgs {
  const mok_weights* w;
  const void* x;              // bf16 [T,H]
  const float* router_w;      // [T,k]
  void* out;                  // bf16 [T,H]
  void* ctx_g;                // routed [rows_cap_max, I] then shared [T_max, I_s] (bf16; fp32 in MXFP8); null = not kept
  void* ctx_u;
  void* h;                    // h (routed rows then shared rows): bf16, or MXFP8 codes + scales
  void* y;                    // bf16 [(rows_cap_max + T_max), H]
  int mxfp8;
};
// One forward over the schedule `sched` (layout L) of configuration c: the
// workspace's own, or one pass of its token ring.
hipError_t launch_forward(mok_workspace* ws, const mok_config& c, const Layout& L, const void* sched,
                          const FwdArgs& a, hipStream_t s);

// Transposed MXFP8 quantization of bf16 matrices [B][R][C] -> [B][C][R]
// codes with [B][C][R/32] scales (R % 128 == 0, C % 64 == 0).
hipError_t launch_quantize_t_matrix(const void* src, int64_t batches, int64_t R, int64_t C, uint8_t* dst,
                                    uint8_t* dst_scale, int grid_cap, hipStream_t s);
// The weight-gradient GEMM operands (TqArrays layout; bf16 elements without
// scales when out_bf16, kinds 0-2 only) from one source:
// src_kind 0 = x token rows, 1 = router weight times grad_out token rows,
// 2 = schedule-row bf16 rows, 3 = schedule-row MXFP8 rows (h).
hipError_t launch_quantize_t_rows(int src_kind, const SchedView& v, const void* src, const uint8_t* src_codes,
                                  const uint8_t* src_scale, const float* router_w, int E, int k, int cols_r, int cols_s,
                                  int64_t rows_cap_max, int64_t kr_cap, uint8_t* dst, uint8_t* dst_scale, int grid,
                                  hipStream_t s, bool out_bf16 = false);

// Axis-1 MXFP8 quantization of a bf16 [T, cols] tensor whose row count T is
// read on the device from a schedule header; the grid covers max_rows.
hipError_t launch_quantize_rows_dev(const void* src, const SchedView& v, int64_t max_rows, int64_t cols, uint8_t* dst,
                                    uint8_t* dst_scale, hipStream_t s);

struct BwdArgs {
  const mok_weights* w;
  const void* x;
  const void* grad_out;
  const float* router_w;
  const void* ctx_g;
  const void* ctx_u;
  const void* ctx_h;
  const mok_grads* g;
  int mxfp8;
  int weights_t;  // MXFP8: `w` holds the weights transposed and quantized (mok_mxfp8_quantize_transposed)
};
hipError_t launch_backward(mok_workspace* ws, const void* sched, const BwdArgs& a, hipStream_t s);

// The SwiGLU input limit the kernels apply: +inf (no clamp) unless the
// configuration sets a positive finite limit.
inline float swiglu_lim(const mok_config& c) {
  return (c.swiglu_limit > 0.0f && c.swiglu_limit < __builtin_inff()) ? c.swiglu_limit : __builtin_inff();
}

// Host-side checks shared by the entry points (api.hip).
bool mxfp8_shapes_ok(const mok_config& c);
mok_status check_weights(const mok_config& c, mok_mode mode, const mok_weights* w, bool need_scales);

// Start of every launch that reads a schedule: false when the schedule's
// header carries another configuration's hash (the launch then does
// nothing; one thread of workgroup 0 counts it in status[1]).
__device__ __forceinline__ bool sched_matches(const int32_t* hdr, int hash, int32_t* status) {
  if (hdr[HDR_HASH] == hash) return true;
  if (status && blockIdx.x == 0 && threadIdx.x == 0)
    __hip_atomic_fetch_add(status + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return false;
}

// Columns of the per-row partial router-weight gradients.
int dw_parts(const mok_config& c);

// Context layout: G, U, h, each [rows_cap_max*I + T_max*I_s] elements
// (routed rows, then shared rows). BF16: G, U and h in bf16. MXFP8: G and U
// in fp32 (the backward's SwiGLU derivative then starts from the values the
// forward's h came from), h as E4M3 codes followed by one E8M0 scale per 32.
inline size_t ctx_elems(const mok_config& c, const Layout& L) {
  return (size_t)L.rows_cap_max * c.intermediate + (size_t)c.max_tokens * c.shared_intermediate;
}
struct CtxLayout {
  size_t g, u, h, total;  // byte offsets of G, U, h and the total size
};
inline CtxLayout ctx_layout(const mok_config& c, const Layout& L, bool mxfp8) {
  const size_t ce = ctx_elems(c, L);
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  CtxLayout r;
  const size_t gu = al(ce * (mxfp8 ? 4 : 2));
  r.g = 0;
  r.u = gu;
  r.h = 2 * gu;
  r.total = 2 * gu + (mxfp8 ? al(ce) + al(ce / 32) : al(ce * 2));
  return r;
}

}  // namespace mok

#define MOK_HIP_TRY(expr)                   \
  do {                                      \
    hipError_t e_ = (expr);                 \
    if (e_ != hipSuccess) return e_;        \
  } while (0)
