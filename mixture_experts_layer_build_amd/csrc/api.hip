// Host side of the C ABI declared in include/mok.h: configuration checks,
// schedule/context sizing, workspace allocation, launch sequencing.
//
// "Mixture-of-Kittens: a deterministic MoE megakernel for NVL72 racks",
// section "The two API layers and the schedule object": a workspace is
// allocated once and reused; the schedule is built once per layer and step
// and passed to both forward and backward. Every check below happens before
// anything is enqueued, and no call reads device memory on the host.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <new>

#include "mok_internal.h"

namespace mok {

int64_t capacity(int64_t T, float mult) {
  // C = min(T, ceil(mult * T)), the float32 multiplier evaluated in float64.
  const double c = std::ceil((double)mult * (double)T);
  const int64_t ci = c < 0 ? 0 : (int64_t)c;
  return std::min<int64_t>(T, ci);
}

int64_t rows_cap(const mok_config& c, int64_t T) {
  const int64_t C = capacity(T, c.capacity_multiplier);
  return std::min<int64_t>(T * c.topk, (int64_t)c.num_experts * C) + (int64_t)c.num_experts * (c.expert_pad - 1);
}

bool ring(const mok_config& c) { return c.macrobatch_size > 0 && (int64_t)c.macrobatch_size < c.max_tokens; }

int64_t sub_offset_tokens(const mok_config& c) {
  if (c.minibatch_size > 0) return c.minibatch_size;
  return ring(c) ? c.macrobatch_size : 0;
}

int64_t n_minibatches(const mok_config& c, int64_t T) {
  const int64_t g = sub_offset_tokens(c);
  if (g <= 0 || T <= 0) return 1;
  return std::max<int64_t>(1, (T + g - 1) / g);
}

static size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

Layout schedule_layout(const mok_config& c) {
  Layout L{};
  const int64_t E = c.num_experts;
  L.rows_cap_max = rows_cap(c, c.max_tokens);
  L.n_mb_max = n_minibatches(c, c.max_tokens);
  size_t off = 0;
  auto take = [&](size_t ints) {
    const size_t o = off;
    off = align_up(off + ints * sizeof(int32_t), 256);
    return o;
  };
  L.header = take(HDR_INTS);
  L.counts = take(E);
  L.kept = take(E);
  L.offsets = take(E + 1);
  L.mb_offsets = take((L.n_mb_max + 1) * E);
  L.row_src = take(L.rows_cap_max);
  L.slot_row = take((size_t)c.max_tokens * c.topk);
  L.tiles = take((size_t)kNumTileBMs * (E + 2));
  L.total = off;
  return L;
}

uint32_t config_hash(const mok_config& c) {
  // FNV-1a over the fields that shape a schedule.
  uint32_t h = 2166136261u;
  auto mix = [&](const void* p, size_t n) {
    const unsigned char* b = (const unsigned char*)p;
    for (size_t i = 0; i < n; ++i) h = (h ^ b[i]) * 16777619u;
  };
  mix(&c.num_experts, 4);
  mix(&c.topk, 4);
  mix(&c.max_tokens, 8);
  mix(&c.capacity_multiplier, 4);
  mix(&c.expert_pad, 4);
  mix(&c.minibatch_size, 4);
  mix(&c.macrobatch_size, 4);
  return h & 0x7FFFFFFFu;
}

SchedView sched_view(void* base, const Layout& L) {
  char* b = (char*)base;
  SchedView v;
  v.header = (int32_t*)(b + L.header);
  v.counts = (int32_t*)(b + L.counts);
  v.kept = (int32_t*)(b + L.kept);
  v.offsets = (int32_t*)(b + L.offsets);
  v.mb_offsets = (int32_t*)(b + L.mb_offsets);
  v.row_src = (int32_t*)(b + L.row_src);
  v.slot_row = (int32_t*)(b + L.slot_row);
  v.tiles = (int32_t*)(b + L.tiles);
  return v;
}

LaunchTimer::LaunchTimer(mok_workspace* w, int k, hipStream_t s) : ws(w), kernel(k), stream(s) {
  if (!ws || k < 0 || k >= 32 || !((ws->timing_mask >> k) & 1u)) return;
  auto get = [&]() {
    hipEvent_t e = nullptr;
    if (!ws->event_pool.empty()) {
      e = ws->event_pool.back();
      ws->event_pool.pop_back();
    } else if (hipEventCreate(&e) != hipSuccess) {
      e = nullptr;
    }
    return e;
  };
  a = get();
  b = get();
  if (a) (void)hipEventRecord(a, stream);
}

LaunchTimer::~LaunchTimer() {
  if (!ws || !a || !b) return;
  (void)hipEventRecord(b, stream);
  ws->launches.push_back(TimedLaunch{kernel, a, b});
}

// Restores the caller's current device when a call switches to the
// workspace's device.
struct DeviceGuard {
  int prev = -1;
  bool ok = true;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    if (prev != dev) ok = hipSetDevice(dev) == hipSuccess;
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

// Scratch parts, in allocation order.
enum ScratchPart : int {
  SP_SCHED = 0,  // schedule chunk histograms
  SP_H,          // h when no context is kept (bf16 or MXFP8 codes)
  SP_Y,          // y rows (bf16), reused for the backward's dA rows
  SP_XQ,         // x in MXFP8 (+ scales)
  SP_HQ,         // h in MXFP8 (+ scales) when no context is kept
  SP_WT,         // transposed weights for the backward (routed + shared)
  SP_DGUH,       // dG, dU, w*h (3 x context-sized)
  SP_DWP,        // partial router-weight gradients
  SP_ROWS,       // transposed operands of the weight-gradient GEMMs
  SP_PIPE,       // the minibatch pipeline's counters and its status word
  SP_PASS,       // the token ring: one macrobatch's schedule
  SP_COUNT
};

// MXFP8 GEMMs load one dword of E8M0 scales (4 blocks of 32) per row and
// two K steps, so every contraction length must be a multiple of 128.
bool mxfp8_shapes_ok(const mok_config& c) {
  return c.hidden % 128 == 0 && c.intermediate % 128 == 0 && c.shared_intermediate % 128 == 0;
}

// The MXFP8 backward's buffers, placed inside the BF16 backward's regions.
// kr_cap bounds the routed K of the weight-gradient operands (each segment
// rounded up to 128 rows: at most rows_cap + 127 E), ks_cap the shared K.
struct Fp8BwdPlan {
  size_t w_c, w_s, sw_c, sw_s;     // routed / shared weight codes and scales (each of 3)
  int64_t kr_cap, ks_cap;
  size_t xc, xs, ic, is;           // H-column and I-column operand codes / scales (each array)
  size_t wt, dguh, rows;           // bytes needed in the WT, DGUH and ROWS regions
};

Fp8BwdPlan fp8_bwd_plan(const mok_config& c, const Layout& L) {
  const int64_t Tm = c.max_tokens, H = c.hidden, E = c.num_experts, I = c.intermediate, Is = c.shared_intermediate;
  const size_t ce = ctx_elems(c, L);
  Fp8BwdPlan f{};
  f.w_c = align_up((size_t)E * I * H, 256);
  f.w_s = align_up((size_t)E * I * H / 32, 256);
  f.sw_c = align_up((size_t)Is * H, 256);
  f.sw_s = align_up((size_t)Is * H / 32, 256);
  f.kr_cap = (int64_t)align_up((size_t)(L.rows_cap_max + 128 * E), 128);
  f.ks_cap = Is > 0 ? (int64_t)align_up((size_t)Tm, 128) : 0;
  f.xc = align_up((size_t)H * (f.kr_cap + f.ks_cap), 256);
  f.xs = align_up((size_t)H * (f.kr_cap + f.ks_cap) / 32, 256);
  f.ic = align_up((size_t)I * f.kr_cap + (size_t)Is * f.ks_cap, 256);
  f.is = align_up(((size_t)I * f.kr_cap + (size_t)Is * f.ks_cap) / 32, 256);
  f.wt = 3 * (f.w_c + f.w_s) + 3 * (f.sw_c + f.sw_s);
  f.dguh = align_up(ce, 256) + align_up(ce / 32, 256);
  f.rows = 2 * (f.xc + f.xs) + 3 * (f.ic + f.is);
  return f;
}

// bf16 operands of the BF16 weight-gradient GEMMs (the TqArrays layout
// without scales), in the ROWS region.
struct Bf16DwPlan {
  int64_t kr_cap, ks_cap;
  size_t xc, ic, rows;
};

Bf16DwPlan bf16_dw_plan(const mok_config& c, const Layout& L) {
  const int64_t Tm = c.max_tokens, H = c.hidden, E = c.num_experts, I = c.intermediate, Is = c.shared_intermediate;
  Bf16DwPlan f{};
  f.kr_cap = (int64_t)align_up((size_t)(L.rows_cap_max + 128 * E), 128);
  f.ks_cap = Is > 0 ? (int64_t)align_up((size_t)Tm, 128) : 0;
  f.xc = align_up((size_t)H * (f.kr_cap + f.ks_cap) * 2, 256);
  f.ic = align_up(((size_t)I * f.kr_cap + (size_t)Is * f.ks_cap) * 2, 256);
  f.rows = 2 * f.xc + 3 * f.ic;
  return f;
}

// One pass of the token ring: macrobatch_size tokens, every expert able to
// take all of them (capacity 1: the whole batch's capacity decided which
// assignments are kept), one minibatch, no pipeline.
mok_config pass_config(const mok_config& c) {
  mok_config q = c;
  q.max_tokens = c.macrobatch_size;
  q.capacity_multiplier = 1.0f;
  q.minibatch_size = 0;
  q.num_mover_wgs = 0;
  q.macrobatch_size = 0;
  q.forward_only = 1;
  return q;
}

size_t workspace_bytes(const mok_config& c, const Layout& L, size_t* parts) {
  const int64_t Tm = c.max_tokens, H = c.hidden, E = c.num_experts, I = c.intermediate, Is = c.shared_intermediate;
  const int64_t rowsR = L.rows_cap_max;
  const int64_t n_chunks_max = std::max<int64_t>(1, 24 * 1024 / c.num_experts);
  const size_t ce = ctx_elems(c, L);
  // the forward's token-sized scratch holds one macrobatch in ring mode
  const bool rg = ring(c);
  const mok_config fc = rg ? pass_config(c) : c;
  const Layout FL = rg ? schedule_layout(fc) : L;
  const size_t fce = ctx_elems(fc, FL);
  const int64_t fT = fc.max_tokens;
  size_t p[SP_COUNT] = {
      (size_t)n_chunks_max * E * 4,
      fce * 2,
      (size_t)(FL.rows_cap_max + fT) * H * 2,
      (size_t)fT * H + (size_t)fT * (H / 32),
      fce + fce / 32,
      3 * align_up((size_t)E * I * H * 2, 256) + 3 * align_up((size_t)Is * H * 2, 256),
      3 * align_up(ce * 2, 256),
      (size_t)(rowsR + Tm) * dw_parts(c) * 4,
      bf16_dw_plan(c, L).rows,
      (size_t)(L.n_mb_max + 64) * 4,
      rg ? FL.total : 0};
  if (c.forward_only) p[SP_WT] = p[SP_DGUH] = p[SP_DWP] = p[SP_ROWS] = 0;  // no backward
  if (mxfp8_shapes_ok(c) && !c.forward_only) {
    const Fp8BwdPlan f = fp8_bwd_plan(c, L);
    p[SP_WT] = std::max(p[SP_WT], f.wt);
    p[SP_DGUH] = std::max(p[SP_DGUH], f.dguh);
    p[SP_ROWS] = std::max(p[SP_ROWS], f.rows);
  }
  size_t total = 0;
  for (int i = 0; i < SP_COUNT; ++i) {
    if (parts) parts[i] = align_up(p[i], 256);
    total += align_up(p[i], 256);
  }
  return total;
}

}  // namespace mok

using namespace mok;

static mok_status to_status(hipError_t e) {
  if (e == hipSuccess) return MOK_OK;
  if (e == hipErrorNotSupported) return MOK_ERR_UNSUPPORTED;
  return MOK_ERR_HIP;
}

// ------------------------------------------------------------------------
// Pure host queries
// ------------------------------------------------------------------------
extern "C" const char* mok_status_string(mok_status s) {
  switch (s) {
    case MOK_OK: return "MOK_OK";
    case MOK_ERR_INVALID_ARGUMENT: return "MOK_ERR_INVALID_ARGUMENT";
    case MOK_ERR_UNSUPPORTED: return "MOK_ERR_UNSUPPORTED";
    case MOK_ERR_CONFIG_MISMATCH: return "MOK_ERR_CONFIG_MISMATCH";
    case MOK_ERR_BUFFER_TOO_SMALL: return "MOK_ERR_BUFFER_TOO_SMALL";
    case MOK_ERR_HIP: return "MOK_ERR_HIP";
  }
  return "MOK_ERR_UNKNOWN";
}

extern "C" mok_status mok_validate_config(const mok_config* c) {
  if (!c) return MOK_ERR_INVALID_ARGUMENT;
  if (c->struct_size != sizeof(mok_config)) return MOK_ERR_INVALID_ARGUMENT;
  if (c->hidden <= 0 || c->intermediate <= 0 || c->num_experts <= 0 || c->topk <= 0 || c->max_tokens <= 0 ||
      c->shared_intermediate < 0 || c->expert_pad <= 0 || c->minibatch_size < 0 || c->num_mover_wgs < 0)
    return MOK_ERR_INVALID_ARGUMENT;
  if (!(c->capacity_multiplier > 0.0f) || !std::isfinite(c->capacity_multiplier)) return MOK_ERR_INVALID_ARGUMENT;
  if (!(c->swiglu_limit >= 0.0f)) return MOK_ERR_INVALID_ARGUMENT;  // negative or NaN
  if (c->macrobatch_size < 0 || (c->forward_only != 0 && c->forward_only != 1)) return MOK_ERR_INVALID_ARGUMENT;
  // the ring: inference only; passes made of whole minibatches; E >= k, so
  // that a pass's kept rows (at most M k, repeated ids included) fit the
  // pass layout's min(M k, E M)
  if (ring(*c) && (!c->forward_only || c->num_experts < c->topk ||
                   (c->minibatch_size > 0 && c->macrobatch_size % c->minibatch_size != 0)))
    return MOK_ERR_UNSUPPORTED;
  if (c->hidden % 128 != 0 || c->intermediate % 64 != 0 || c->shared_intermediate % 64 != 0)
    return MOK_ERR_UNSUPPORTED;
  if (c->num_experts > 1024 || c->topk > 64 || c->expert_pad % 32 != 0) return MOK_ERR_UNSUPPORTED;
  if (c->max_tokens * (int64_t)c->topk >= (int64_t)1 << 31) return MOK_ERR_UNSUPPORTED;
  const Layout L = schedule_layout(*c);
  if (L.rows_cap_max + c->max_tokens >= (int64_t)1 << 31) return MOK_ERR_UNSUPPORTED;
  // Operands are read through one buffer range each, with offsets below
  // 2 GiB (the kernels' out-of-range marker sits at 2 GiB):
  //  - token-indexed operands: max_tokens rows of H, I or I_s bf16 elements
  //    (an expert may receive every token, and the weight gradients read its
  //    rows transposed, [I or H][rows rounded up to 128]), and a
  //    weight-gradient tile's 256 rows of that expert's rounded row count;
  //  - one expert's weight matrix, I x H or I_s x H bf16 elements.
  const int64_t widest = std::max({(int64_t)c->hidden, (int64_t)c->intermediate,
                                   (int64_t)c->shared_intermediate, (int64_t)256});
  if ((c->max_tokens + 127) * widest * 2 >= (int64_t)1 << 31) return MOK_ERR_UNSUPPORTED;
  if ((int64_t)c->intermediate * c->hidden * 2 >= (int64_t)1 << 31 ||
      (int64_t)c->shared_intermediate * c->hidden * 2 >= (int64_t)1 << 31)
    return MOK_ERR_UNSUPPORTED;
  return MOK_OK;
}

extern "C" size_t mok_schedule_bytes(const mok_config* c) {
  if (mok_validate_config(c) != MOK_OK) return 0;
  return schedule_layout(*c).total;
}

extern "C" mok_status mok_schedule_layout_query(const mok_config* c, mok_schedule_layout* out) {
  const mok_status st = mok_validate_config(c);
  if (st != MOK_OK) return st;
  if (!out) return MOK_ERR_INVALID_ARGUMENT;
  const Layout L = schedule_layout(*c);
  out->total_bytes = L.total;
  out->header = L.header;
  out->counts = L.counts;
  out->kept = L.kept;
  out->offsets = L.offsets;
  out->mb_offsets = L.mb_offsets;
  out->row_src = L.row_src;
  out->slot_row = L.slot_row;
  out->tiles = L.tiles;
  out->rows_cap_max = L.rows_cap_max;
  out->n_mb_max = L.n_mb_max;
  return MOK_OK;
}

extern "C" size_t mok_context_bytes(const mok_config* c, mok_mode mode) {
  if (mok_validate_config(c) != MOK_OK) return 0;
  if (mode != MOK_MODE_BF16 && mode != MOK_MODE_MXFP8) return 0;
  const Layout L = schedule_layout(*c);
  return ctx_layout(*c, L, mode == MOK_MODE_MXFP8).total;
}

extern "C" size_t mok_workspace_bytes(const mok_config* c) {
  if (mok_validate_config(c) != MOK_OK) return 0;
  return workspace_bytes(*c, schedule_layout(*c), nullptr);
}

// ------------------------------------------------------------------------
// Workspace
// ------------------------------------------------------------------------
extern "C" mok_status mok_workspace_create(const mok_config* c, int device, mok_workspace** out) {
  if (!out) return MOK_ERR_INVALID_ARGUMENT;
  *out = nullptr;
  const mok_status st = mok_validate_config(c);
  if (st != MOK_OK) return st;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess) return MOK_ERR_HIP;
  if (device < 0 || device >= ndev) return MOK_ERR_INVALID_ARGUMENT;
  DeviceGuard g(device);
  if (!g.ok) return MOK_ERR_HIP;
  mok_workspace* ws = new (std::nothrow) mok_workspace();
  if (!ws) return MOK_ERR_HIP;
  ws->cfg = *c;
  ws->device = device;
  ws->layout = schedule_layout(*c);
  if (hipDeviceGetAttribute(&ws->num_cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess ||
      ws->num_cus <= 0) {
    delete ws;
    return MOK_ERR_HIP;
  }
  size_t parts[SP_COUNT];
  ws->scratch_bytes = workspace_bytes(*c, ws->layout, parts);
  if (hipMalloc((void**)&ws->scratch, ws->scratch_bytes) != hipSuccess) {
    delete ws;
    return MOK_ERR_HIP;
  }
  char* p = ws->scratch;
  ws->n_chunks_max = std::max<int64_t>(1, 24 * 1024 / c->num_experts);
  ws->chunk_hist = (int32_t*)p;
  p += parts[SP_SCHED];
  ws->hbuf = p;
  ws->hbuf_bytes = parts[SP_H];
  p += parts[SP_H];
  ws->ybuf = p;
  p += parts[SP_Y];
  // (in ring mode these four are sized for one macrobatch: pass_config)
  const mok_config fc = ring(*c) ? pass_config(*c) : *c;
  const size_t fce = ctx_elems(fc, ring(*c) ? schedule_layout(fc) : ws->layout);
  ws->xq = (uint8_t*)p;
  ws->xq_scale = (uint8_t*)p + (size_t)fc.max_tokens * c->hidden;
  p += parts[SP_XQ];
  ws->hq = (uint8_t*)p;
  ws->hq_scale = (uint8_t*)p + fce;
  p += parts[SP_HQ];
  const size_t ce = ctx_elems(*c, ws->layout);
  if (!c->forward_only) {
    char* bp = p;  // the backward regions: WT, DGUH, DWP, ROWS
    const size_t wr = align_up((size_t)c->num_experts * c->intermediate * c->hidden * 2, 256);
    const size_t wsh = align_up((size_t)c->shared_intermediate * c->hidden * 2, 256);
    BwdScratch& b = ws->bwd;
    b.wdT = (uint16_t*)bp;
    b.wgT = (uint16_t*)(bp + wr);
    b.wuT = (uint16_t*)(bp + 2 * wr);
    b.sdT = (uint16_t*)(bp + 3 * wr);
    b.sgT = (uint16_t*)(bp + 3 * wr + wsh);
    b.suT = (uint16_t*)(bp + 3 * wr + 2 * wsh);
    bp += parts[SP_WT];
    const size_t cb = align_up(ce * 2, 256);
    b.dg = (uint16_t*)bp;
    b.du = (uint16_t*)(bp + cb);
    b.hw = (uint16_t*)(bp + 2 * cb);
    bp += parts[SP_DGUH];
    b.dw_part = (float*)bp;
    bp += parts[SP_DWP];
    {
      const Bf16DwPlan f = bf16_dw_plan(*c, ws->layout);
      uint8_t* r = (uint8_t*)bp;  // start of the ROWS region
      TqArrays& q = b.tq16;
      q.x = r;
      q.dy = r + f.xc;
      q.h = r + 2 * f.xc;
      q.dg = r + 2 * f.xc + f.ic;
      q.du = r + 2 * f.xc + 2 * f.ic;
      q.kr_cap = f.kr_cap;
    }
    if (mxfp8_shapes_ok(*c) && !c->forward_only) {
      const Fp8BwdPlan f = fp8_bwd_plan(*c, ws->layout);
      uint8_t* w = (uint8_t*)b.wdT;  // start of the WT region
      uint8_t** wc[6] = {&b.wdTq, &b.wgTq, &b.wuTq, &b.sdTq, &b.sgTq, &b.suTq};
      uint8_t** wsc[6] = {&b.wdTs, &b.wgTs, &b.wuTs, &b.sdTs, &b.sgTs, &b.suTs};
      for (int i = 0; i < 6; ++i) {
        *wc[i] = w;
        w += i < 3 ? f.w_c : f.sw_c;
        *wsc[i] = w;
        w += i < 3 ? f.w_s : f.sw_s;
      }
      // DGUH region: dU's MXFP8 codes and scales along I
      b.duq = (uint8_t*)b.dg;
      b.duq_scale = b.duq + align_up(ce, 256);
      uint8_t* r = b.tq16.x;  // start of the ROWS region
      TqArrays& q = b.tq;
      q.x = r;
      q.xs = r + f.xc;
      r += f.xc + f.xs;
      q.dy = r;
      q.dys = r + f.xc;
      r += f.xc + f.xs;
      q.h = r;
      q.hs = r + f.ic;
      r += f.ic + f.is;
      q.dg = r;
      q.dgs = r + f.ic;
      r += f.ic + f.is;
      q.du = r;
      q.dus = r + f.ic;
      q.kr_cap = f.kr_cap;
      b.mxfp8_ready = true;
    }
  }
  p += parts[SP_WT] + parts[SP_DGUH] + parts[SP_DWP] + parts[SP_ROWS];
  ws->pass_sched = parts[SP_PASS] ? p + parts[SP_PIPE] : nullptr;
  ws->status = (int32_t*)p;  // status words first, then the counters
  ws->pipe_cnt = (int32_t*)p + 64;
  if (hipMemset(p, 0, parts[SP_PIPE]) != hipSuccess) {
    (void)mok_workspace_destroy(ws);
    return MOK_ERR_HIP;
  }
  p += parts[SP_PIPE];
  *out = ws;
  return MOK_OK;
}

extern "C" mok_status mok_workspace_destroy(mok_workspace* ws) {
  if (!ws) return MOK_OK;
  mok_status st = MOK_OK;
  {
    DeviceGuard g(ws->device);
    if (hipDeviceSynchronize() != hipSuccess) st = MOK_ERR_HIP;
    for (auto& l : ws->launches) {
      (void)hipEventDestroy(l.start);
      (void)hipEventDestroy(l.stop);
    }
    for (auto e : ws->event_pool) (void)hipEventDestroy(e);
    if (ws->scratch && hipFree(ws->scratch) != hipSuccess) st = MOK_ERR_HIP;
  }
  delete ws;
  return st;
}

// ------------------------------------------------------------------------
// Hot path
// ------------------------------------------------------------------------
extern "C" mok_status mok_build_schedule(mok_workspace* ws, const int64_t* top_experts, int64_t T, void* schedule,
                                         size_t schedule_bytes, void* stream) {
  if (!ws || !schedule) return MOK_ERR_INVALID_ARGUMENT;
  if (T < 0 || T > ws->cfg.max_tokens) return MOK_ERR_INVALID_ARGUMENT;
  if (T > 0 && !top_experts) return MOK_ERR_INVALID_ARGUMENT;
  if (schedule_bytes < ws->layout.total) return MOK_ERR_BUFFER_TOO_SMALL;
  DeviceGuard g(ws->device);
  if (!g.ok) return MOK_ERR_HIP;
  return launch_schedule(ws, top_experts, T, schedule, (hipStream_t)stream) == hipSuccess ? MOK_OK : MOK_ERR_HIP;
}

namespace mok {
mok_status check_weights(const mok_config& c, mok_mode mode, const mok_weights* w, bool need_scales) {
  if (!w || !w->routed_gate || !w->routed_up || !w->routed_down) return MOK_ERR_INVALID_ARGUMENT;
  const bool sh = c.shared_intermediate > 0;
  if (sh != (w->shared_gate != nullptr) || sh != (w->shared_up != nullptr) || sh != (w->shared_down != nullptr))
    return MOK_ERR_INVALID_ARGUMENT;
  if (mode == MOK_MODE_MXFP8 && need_scales) {
    if (!w->routed_gate_scale || !w->routed_up_scale || !w->routed_down_scale) return MOK_ERR_INVALID_ARGUMENT;
    if (sh && (!w->shared_gate_scale || !w->shared_up_scale || !w->shared_down_scale))
      return MOK_ERR_INVALID_ARGUMENT;
  }
  return MOK_OK;
}
}  // namespace mok

extern "C" mok_status mok_forward(mok_workspace* ws, mok_mode mode, const void* schedule, size_t schedule_bytes,
                                  const void* x, const float* router_weights, const mok_weights* weights, void* out,
                                  void* context, size_t context_bytes, void* stream) {
  if (!ws || !schedule || !x || !router_weights || !out) return MOK_ERR_INVALID_ARGUMENT;
  if (mode != MOK_MODE_BF16 && mode != MOK_MODE_MXFP8) return MOK_ERR_INVALID_ARGUMENT;
  if (schedule_bytes < ws->layout.total) return MOK_ERR_BUFFER_TOO_SMALL;
  mok_status st = check_weights(ws->cfg, mode, weights, true);
  if (st != MOK_OK) return st;
  if (mode == MOK_MODE_MXFP8 && !mxfp8_shapes_ok(ws->cfg)) return MOK_ERR_UNSUPPORTED;
  if (context && ws->cfg.forward_only) return MOK_ERR_UNSUPPORTED;
  if (context && context_bytes < mok_context_bytes(&ws->cfg, mode)) return MOK_ERR_BUFFER_TOO_SMALL;
  DeviceGuard g(ws->device);
  if (!g.ok) return MOK_ERR_HIP;
  FwdArgs a{};
  a.w = weights;
  a.x = x;
  a.router_w = router_weights;
  a.out = out;
  a.mxfp8 = mode == MOK_MODE_MXFP8;
  if (context) {
    char* cb = (char*)context;
    const CtxLayout cl = ctx_layout(ws->cfg, ws->layout, a.mxfp8 != 0);
    a.ctx_g = cb + cl.g;
    a.ctx_u = cb + cl.u;
    a.h = cb + cl.h;
  } else {
    a.h = ws->hbuf;
  }
  a.y = ws->ybuf;
  const hipStream_t s = (hipStream_t)stream;
  if (!ring(ws->cfg)) return to_status(launch_forward(ws, ws->cfg, ws->layout, schedule, a, s));
  // Token ring: the batch goes through the scratch macrobatch by macrobatch.
  // T is only known on the device, so every pass that max_tokens allows is
  // enqueued; a pass past T has no tokens and its launches return at once.
  // Pass p cuts its own schedule out of the whole batch's (capacity and drops
  // stay the whole batch's) and runs the one-pass launches on tokens
  // [p*M, p*M + M) through pointers offset by p*M tokens; the row sums of the
  // combine do not depend on the pass, so the output bits are those of one
  // pass.
  const mok_config qc = pass_config(ws->cfg);
  const Layout QL = schedule_layout(qc);
  const int64_t M = ws->cfg.macrobatch_size, H = ws->cfg.hidden, k = ws->cfg.topk;
  const int64_t passes = (ws->cfg.max_tokens + M - 1) / M;
  for (int64_t pass = 0; pass < passes; ++pass) {
    hipError_t e = launch_sched_slice(ws, schedule, (int)pass, ws->pass_sched, s);
    if (e != hipSuccess) return to_status(e);
    FwdArgs b = a;
    b.x = (const uint16_t*)x + pass * M * H;
    b.router_w = router_weights + pass * M * k;
    b.out = (uint16_t*)out + pass * M * H;
    e = launch_forward(ws, qc, QL, ws->pass_sched, b, s);
    if (e != hipSuccess) return to_status(e);
  }
  return MOK_OK;
}

extern "C" mok_status mok_backward(mok_workspace* ws, mok_mode mode, const void* schedule, size_t schedule_bytes,
                                   const void* context, size_t context_bytes, const void* grad_out, const void* x,
                                   const float* router_weights, const mok_weights* weights, const mok_grads* grads,
                                   void* stream) {
  if (!ws || !schedule || !context || !grad_out || !x || !router_weights || !grads) return MOK_ERR_INVALID_ARGUMENT;
  if (mode != MOK_MODE_BF16 && mode != MOK_MODE_MXFP8) return MOK_ERR_INVALID_ARGUMENT;
  if (ws->cfg.forward_only) return MOK_ERR_UNSUPPORTED;
  if (schedule_bytes < ws->layout.total) return MOK_ERR_BUFFER_TOO_SMALL;
  if (context_bytes < mok_context_bytes(&ws->cfg, mode)) return MOK_ERR_BUFFER_TOO_SMALL;
  mok_status st = check_weights(ws->cfg, mode, weights, false);
  if (st != MOK_OK) return st;
  if (mode == MOK_MODE_MXFP8 && (!mxfp8_shapes_ok(ws->cfg) || !ws->bwd.mxfp8_ready)) return MOK_ERR_UNSUPPORTED;
  // MXFP8: the scale pointers say whether the weights come transposed and
  // quantized (all set) or in BF16 (none set)
  const bool sh_w = ws->cfg.shared_intermediate > 0;
  const int n_scales = (weights->routed_gate_scale != nullptr) + (weights->routed_up_scale != nullptr) +
                       (weights->routed_down_scale != nullptr) + (weights->shared_gate_scale != nullptr) +
                       (weights->shared_up_scale != nullptr) + (weights->shared_down_scale != nullptr);
  const bool weights_t = mode == MOK_MODE_MXFP8 && n_scales > 0;
  if (weights_t && n_scales != (sh_w ? 6 : 3)) return MOK_ERR_INVALID_ARGUMENT;
  const bool sh = ws->cfg.shared_intermediate > 0;
  if (!grads->dx || !grads->d_router_weights || !grads->d_routed_gate || !grads->d_routed_up ||
      !grads->d_routed_down)
    return MOK_ERR_INVALID_ARGUMENT;
  if (sh != (grads->d_shared_gate != nullptr) || sh != (grads->d_shared_up != nullptr) ||
      sh != (grads->d_shared_down != nullptr))
    return MOK_ERR_INVALID_ARGUMENT;
  DeviceGuard g(ws->device);
  if (!g.ok) return MOK_ERR_HIP;
  const CtxLayout cl = ctx_layout(ws->cfg, ws->layout, mode == MOK_MODE_MXFP8);
  BwdArgs a{};
  a.w = weights;
  a.x = x;
  a.grad_out = grad_out;
  a.router_w = router_weights;
  a.ctx_g = (const char*)context + cl.g;
  a.ctx_u = (const char*)context + cl.u;
  a.ctx_h = (const char*)context + cl.h;
  a.g = grads;
  a.mxfp8 = mode == MOK_MODE_MXFP8;
  a.weights_t = weights_t;
  return to_status(launch_backward(ws, schedule, a, (hipStream_t)stream));
}

extern "C" mok_status mok_mxfp8_quantize(const void* src, int src_is_fp32, int64_t rows, int64_t cols,
                                         int64_t ld_src, int axis, uint8_t* dst, int64_t ld_dst,
                                         uint8_t* dst_scale, void* stream) {
  if (rows < 0 || cols < 0 || (axis != 0 && axis != 1) || (src_is_fp32 != 0 && src_is_fp32 != 1))
    return MOK_ERR_INVALID_ARGUMENT;
  if (rows == 0 || cols == 0) return MOK_OK;
  if (!src || !dst || !dst_scale) return MOK_ERR_INVALID_ARGUMENT;
  if (ld_src < cols || ld_dst < cols) return MOK_ERR_INVALID_ARGUMENT;
  if (cols % 8 != 0 || ld_dst % 8 != 0 || ld_src % 8 != 0) return MOK_ERR_UNSUPPORTED;
  if (axis == 1 && cols % 32 != 0) return MOK_ERR_UNSUPPORTED;
  if (axis == 0 && rows % 32 != 0) return MOK_ERR_UNSUPPORTED;
  if (axis == 1 && !src_is_fp32 && rows > ((int64_t)1 << 24)) return MOK_ERR_UNSUPPORTED;  // one workgroup per row
  if ((((uintptr_t)src) & 15) || (((uintptr_t)dst) & 7)) return MOK_ERR_UNSUPPORTED;
  if (axis == 0 && (((uintptr_t)dst_scale) & 7)) return MOK_ERR_UNSUPPORTED;
  return launch_quantize(src, src_is_fp32, rows, cols, ld_src, axis, dst, ld_dst, dst_scale, (hipStream_t)stream) ==
                 hipSuccess
             ? MOK_OK
             : MOK_ERR_HIP;
}

extern "C" mok_status mok_mxfp8_quantize_transposed(const void* src, int64_t batches, int64_t rows, int64_t cols,
                                                    uint8_t* dst, uint8_t* dst_scale, void* stream) {
  if (batches < 0 || rows < 0 || cols < 0) return MOK_ERR_INVALID_ARGUMENT;
  if (batches == 0 || rows == 0 || cols == 0) return MOK_OK;
  if (!src || !dst || !dst_scale) return MOK_ERR_INVALID_ARGUMENT;
  if (rows % 128 != 0 || cols % 64 != 0) return MOK_ERR_UNSUPPORTED;
  if ((((uintptr_t)src) & 15) || (((uintptr_t)dst) & 15) || (((uintptr_t)dst_scale) & 3)) return MOK_ERR_UNSUPPORTED;
  int dev = -1, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return MOK_ERR_HIP;
  return launch_quantize_t_matrix(src, batches, rows, cols, dst, dst_scale, cus * 4, (hipStream_t)stream) ==
                 hipSuccess
             ? MOK_OK
             : MOK_ERR_HIP;
}

// ------------------------------------------------------------------------
// Diagnostics
// ------------------------------------------------------------------------
extern "C" const char* mok_kernel_name(int id) {
  static const char* names[MOK_K_COUNT] = {
      "sched_count", "sched_scan", "sched_scatter", "sched_minibatch", "quant_x",      "gate_up",
      "down",        "combine",    "bwd_transpose", "bwd_gather",      "bwd_dh",       "bwd_dw_reduce",
      "bwd_dx_rows", "bwd_dx_sum", "bwd_dw",        "bwd_quant",       "sched_slice"};
  if (id < 0 || id >= MOK_K_COUNT) return "unknown";
  return names[id];
}

extern "C" mok_status mok_workspace_set_timing(mok_workspace* ws, int enable) {
  if (!ws) return MOK_ERR_INVALID_ARGUMENT;
  ws->timing_mask = enable != 0 ? (1u << MOK_K_COUNT) - 1u : 0u;
  return MOK_OK;
}

static_assert(MOK_K_COUNT <= 32, "one mask bit per kernel id");

extern "C" mok_status mok_workspace_set_timing_mask(mok_workspace* ws, uint32_t kernel_mask) {
  if (!ws) return MOK_ERR_INVALID_ARGUMENT;
  ws->timing_mask = kernel_mask & ((1u << MOK_K_COUNT) - 1u);
  return MOK_OK;
}

extern "C" mok_status mok_workspace_read_status(mok_workspace* ws, int32_t* pipeline_timeouts,
                                                int32_t* schedule_mismatches) {
  if (!ws) return MOK_ERR_INVALID_ARGUMENT;
  DeviceGuard g(ws->device);
  if (!g.ok) return MOK_ERR_HIP;
  int32_t st[2] = {0, 0};
  if (hipDeviceSynchronize() != hipSuccess) return MOK_ERR_HIP;
  if (hipMemcpy(st, ws->status, sizeof(st), hipMemcpyDeviceToHost) != hipSuccess) return MOK_ERR_HIP;
  if (hipMemset(ws->status, 0, sizeof(st)) != hipSuccess) return MOK_ERR_HIP;
  if (pipeline_timeouts) *pipeline_timeouts = st[0];
  if (schedule_mismatches) *schedule_mismatches = st[1];
  return st[1] > 0 ? MOK_ERR_CONFIG_MISMATCH : MOK_OK;
}

extern "C" mok_status mok_workspace_read_timing(mok_workspace* ws, float* total_ms, int64_t* launches, int n) {
  if (!ws || n < 0 || (n > 0 && (!total_ms || !launches))) return MOK_ERR_INVALID_ARGUMENT;
  for (int i = 0; i < n; ++i) {
    total_ms[i] = 0.f;
    launches[i] = 0;
  }
  DeviceGuard g(ws->device);
  mok_status st = MOK_OK;
  for (auto& l : ws->launches) {
    float ms = 0.f;
    if (hipEventSynchronize(l.stop) != hipSuccess || hipEventElapsedTime(&ms, l.start, l.stop) != hipSuccess)
      st = MOK_ERR_HIP;
    if (l.kernel >= 0 && l.kernel < n) {
      total_ms[l.kernel] += ms;
      launches[l.kernel] += 1;
    }
    ws->event_pool.push_back(l.start);
    ws->event_pool.push_back(l.stop);
  }
  ws->launches.clear();
  return st;
}
