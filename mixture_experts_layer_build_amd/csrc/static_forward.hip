// mok_forward_static: the forward (inference, no context) of mok_forward
// with its scratch in a fixed device array instead of a workspace, for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc).
//
// The array below is the scratch: h (bf16, or MXFP8 codes and scales), the
// weighted down rows y, and in MXFP8 mode the codes and scales of x. Each
// GPU the library runs on holds its own copy until the process ends. Host
// code never uses the array's name as an address (on the host it is only a
// stand-in): the first call on a device, with that device current, takes the
// device address with hipGetSymbolAddress and keeps it for that device.
// Nothing in the scratch needs to start at zero (every kernel writes what it
// reads later in the same call). Calls that overlap on one GPU share the
// array and race.
#include <mutex>

#include "mok_internal.h"

namespace mok {
namespace {

constexpr size_t kStaticScratchBytes = size_t(128) << 20;  // 128 MiB
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
uint8_t* g_scratch[kMaxDevices];  // device address of `scratch` on each device, once taken
int g_cus[kMaxDevices];

size_t al256(size_t v) { return (v + 255) / 256 * 256; }

// Byte offsets of the forward's scratch parts inside the array.
struct StaticPlan {
  size_t h, y, xq, total;
};

StaticPlan static_plan(const mok_config& c, const Layout& L, bool mxfp8) {
  const size_t ce = ctx_elems(c, L);
  StaticPlan p{};
  p.h = 0;
  const size_t hb = mxfp8 ? al256(ce) + al256(ce / 32) : al256(ce * 2);  // codes, then scales at + ce
  p.y = p.h + hb;
  const size_t yb = al256((size_t)(L.rows_cap_max + c.max_tokens) * c.hidden * 2);
  p.xq = p.y + yb;
  const size_t tx = (size_t)c.max_tokens * c.hidden;
  p.total = p.xq + (mxfp8 ? al256(tx) + al256(tx / 32) : 0);
  return p;
}

}  // namespace
}  // namespace mok

using namespace mok;

extern "C" mok_status mok_forward_static(const mok_config* cfg, mok_mode mode, const void* schedule,
                                         size_t schedule_bytes, const void* x, const float* router_weights,
                                         const mok_weights* weights, void* out, void* stream) {
  mok_status st = mok_validate_config(cfg);
  if (st != MOK_OK) return st;
  if (mode != MOK_MODE_BF16 && mode != MOK_MODE_MXFP8) return MOK_ERR_INVALID_ARGUMENT;
  if (!schedule || !x || !router_weights || !out) return MOK_ERR_INVALID_ARGUMENT;
  const Layout L = schedule_layout(*cfg);
  if (schedule_bytes < L.total) return MOK_ERR_BUFFER_TOO_SMALL;
  st = check_weights(*cfg, mode, weights, true);
  if (st != MOK_OK) return st;
  const bool mx = mode == MOK_MODE_MXFP8;
  if (mx && !mxfp8_shapes_ok(*cfg)) return MOK_ERR_UNSUPPORTED;
  const StaticPlan plan = static_plan(*cfg, L, mx);
  if (plan.total > kStaticScratchBytes) return MOK_ERR_UNSUPPORTED;  // beyond the fixed scratch
  // set-up, once per device, with that device current
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MOK_ERR_HIP;
  if (dev >= kMaxDevices) return MOK_ERR_UNSUPPORTED;
  uint8_t* base = nullptr;
  int cus = 0;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_scratch[dev]) {
      void* ptr = nullptr;
      if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return MOK_ERR_HIP;
      int n = 0;
      if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        return MOK_ERR_HIP;
      g_cus[dev] = n;
      g_scratch[dev] = (uint8_t*)ptr;
    }
    base = g_scratch[dev];
    cus = g_cus[dev];
  }
  // a workspace view of the scratch (no auxiliary stream: no minibatch
  // pipeline; no timing); it owns nothing
  mok_workspace ws;
  ws.cfg = *cfg;
  ws.cfg.num_mover_wgs = 0;
  ws.device = dev;
  ws.num_cus = cus;
  ws.layout = L;
  const size_t ce = ctx_elems(*cfg, L);
  ws.hbuf = base + plan.h;
  ws.hq = base + plan.h;
  ws.hq_scale = base + plan.h + ce;
  ws.ybuf = base + plan.y;
  ws.xq = base + plan.xq;
  ws.xq_scale = base + plan.xq + (size_t)cfg->max_tokens * cfg->hidden;
  FwdArgs a{};
  a.w = weights;
  a.x = x;
  a.router_w = router_weights;
  a.out = out;
  a.mxfp8 = mx;
  a.h = ws.hbuf;
  a.y = ws.ybuf;
  const hipError_t e = launch_forward(&ws, ws.cfg, ws.layout, schedule, a, (hipStream_t)stream);
  return e == hipSuccess ? MOK_OK : MOK_ERR_HIP;
}
