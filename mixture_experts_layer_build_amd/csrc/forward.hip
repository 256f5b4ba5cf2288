// Forward of the grouped SwiGLU expert MLP and the router-weighted combine,
// in BF16 and in MXFP8.
//
// "nemo_automodel.components.moe.mok_experts", GroupedExpertsMoK.forward and
// _MoKRuntime.forward: fused shared and routed SwiGLU experts; routed
// gate/up [E, I, H], down [E, H, I]; shared gate/up [I_s, H], down [H, I_s];
// no expert bias. "Mixture-of-Kittens: a deterministic MoE megakernel for
// NVL72 racks", section "The two API layers and the schedule object": the
// schedule drives both dispatch (here a gather of token rows into the
// expert-contiguous order) and combine (a gather-sum back to token order);
// section "Tuning the five hyperparameters before production": in MXFP8 mode
// the activations enter in BF16 and are quantized here, the weights arrive
// pre-quantized.
//
// Launch sequence (all stream-ordered, no host synchronisation; every grid
// is sized from the configuration, the real counts are read on the device):
//   [MXFP8: quantize x along H into E4M3 + E8M0]
//   gate_up : grouped GEMM, epilogue h = silu(g) * u (bf16, or MXFP8 along I)
//   down    : grouped GEMM, epilogue y = w_r * acc (bf16)
//   combine : out[t] = bf16(sum over j in slot order of y[slot_row[t, j]]
//             + y_shared[t]), fp32 accumulation, no atomics.
#include "device_common.h"
#include "combine.h"
#include "gemm_nt.h"
#include "mok_internal.h"

namespace mok {

static void fill_schedule(nt::Params& p, const mok_config& c, const Layout& L, const SchedView& v) {
  p.hdr = v.header;
  p.offsets = v.offsets;
  p.kept = v.kept;
  p.tiles = v.tiles + tile_bm_index(nt::BM) * (c.num_experts + 2);
  p.row_src = v.row_src;
  p.mb_offsets = v.mb_offsets;
  p.E = c.num_experts;
  p.k = c.topk;
  p.H = c.hidden;
  p.I = c.intermediate;
  p.Is = c.shared_intermediate;
  p.rows_cap_max = L.rows_cap_max;
  p.swiglu_lim = swiglu_lim(c);
  p.cfg_hash = v.hash;
  p.status = v.status;
}

// Mover workgroups of the minibatch pipeline (0 = no pipeline):
// num_mover_wgs rounded down to a multiple of the XCD count, leaving at
// least four XCD rounds of compute workgroups; the pipeline needs the tile
// tables in LDS and more than one minibatch.
int mover_units(const mok_workspace* ws, const mok_config& c) {
  if (c.minibatch_size <= 0 || c.num_mover_wgs <= 0 || c.num_experts > nt::kMaxLdsE) return 0;
  if ((int64_t)c.minibatch_size >= c.max_tokens || ws->pipe_cnt == nullptr) return 0;
  const int m = c.num_mover_wgs / nt::kNumXcd * nt::kNumXcd;
  return std::min(m, ws->num_cus - 4 * nt::kNumXcd);
}

hipError_t launch_forward(mok_workspace* ws, const mok_config& c, const Layout& L, const void* sched,
                          const FwdArgs& a, hipStream_t s) {
  SchedView v = sched_view(const_cast<void*>(sched), L);
  v.hash = (int)config_hash(c);
  v.status = ws->status;
  const int grid = ws->num_cus;  // one 512-thread workgroup per compute unit
  const size_t ce = ctx_elems(c, L);
  nt::Params p{};
  fill_schedule(p, c, L, v);
  p.router_w = a.router_w;
  p.ctx_g = a.ctx_g;
  p.ctx_u = a.ctx_u;
  // h: bf16 in BF16 mode; E4M3 codes then E8M0 scales in MXFP8 mode (in the
  // context's h region when a context is kept, else in the workspace).
  uint8_t* hq = nullptr;
  uint8_t* hq_scale = nullptr;
  if (a.mxfp8) {
    hq = a.ctx_g ? (uint8_t*)a.h : ws->hq;
    hq_scale = a.ctx_g ? (uint8_t*)a.h + ce : ws->hq_scale;
    LaunchTimer tm(ws, MOK_K_QUANT_X, s);
    MOK_HIP_TRY(launch_quantize_rows_dev(a.x, v, c.max_tokens, c.hidden, ws->xq, ws->xq_scale, s));
  }
  // gate/up
  if (a.mxfp8) {
    p.a_tok = ws->xq;
    p.a_tok_scale = ws->xq_scale;
    p.out = hq;
    p.out_scale = hq_scale;
    p.b0s = a.w->routed_gate_scale;
    p.b1s = a.w->routed_up_scale;
    p.sb0s = a.w->shared_gate_scale;
    p.sb1s = a.w->shared_up_scale;
  } else {
    p.a_tok = a.x;
    p.out = a.h;
  }
  p.b0 = a.w->routed_gate;
  p.b1 = a.w->routed_up;
  p.sb0 = a.w->shared_gate;
  p.sb1 = a.w->shared_up;
  if (mover_units(ws, c) > 0) {  // the pipeline's tile counters start at zero in every forward
    p.mb_done = ws->pipe_cnt;
    p.n_done = (int)L.n_mb_max;
  }
  {
    LaunchTimer tm(ws, MOK_K_GATE_UP, s);
    if (a.mxfp8)
      nt::grouped_gemm_nt<nt::GATE_UP, true><<<grid, nt::NTHR, 0, s>>>(p);
    else
      nt::grouped_gemm_nt<nt::GATE_UP, false><<<grid, nt::NTHR, 0, s>>>(p);
    MOK_HIP_TRY(hipGetLastError());
  }
  // down
  nt::Params d{};
  fill_schedule(d, c, L, v);
  d.router_w = a.router_w;
  d.a_row = a.mxfp8 ? (const void*)hq : a.h;
  d.a_row_scale = hq_scale;
  d.b0 = a.w->routed_down;
  d.sb0 = a.w->shared_down;
  d.b0s = a.w->routed_down_scale;
  d.sb0s = a.w->shared_down_scale;
  d.out = a.y;
  const uint16_t* y = (const uint16_t*)a.y;
  const uint16_t* ys = c.shared_intermediate > 0 ? y + L.rows_cap_max * c.hidden : nullptr;
  const int cgrid = (int)std::min<int64_t>(c.max_tokens, (int64_t)ws->num_cus * 8);
  const int movers = mover_units(ws, c);
  if (movers == 0) {
    {
      LaunchTimer tm(ws, MOK_K_DOWN, s);
      if (a.mxfp8)
        nt::grouped_gemm_nt<nt::DOWN, true><<<grid, nt::NTHR, 0, s>>>(d);
      else
        nt::grouped_gemm_nt<nt::DOWN, false><<<grid, nt::NTHR, 0, s>>>(d);
      MOK_HIP_TRY(hipGetLastError());
    }
    LaunchTimer tm(ws, MOK_K_COMBINE, s);
    sum_slot_rows<<<cgrid, 256, 0, s>>>(v.header, v.hash, v.status, v.slot_row, y, ys, (uint16_t*)a.out, c.hidden,
                                        c.topk);
    MOK_HIP_TRY(hipGetLastError());
    return hipSuccess;
  }
  // Minibatch pipeline in one launch ("Tuning the five hyperparameters before
  // production": minibatch_size sets the granularity of the overlap, a set of
  // SMs serves the exchange): one workgroup per compute unit; the compute
  // workgroups run the down tiles minibatch by minibatch and count each
  // finished tile in mb_done[b] (zeroed by the gate/up launch above); the last
  // `movers` workgroups combine minibatch b as soon as its count is complete,
  // while the tiles of later minibatches run. Each output row is summed by
  // the same arithmetic as the stand-alone combine, so the bits do not depend
  // on minibatch_size or num_mover_wgs.
  d.mb = c.minibatch_size;
  d.mb_done = ws->pipe_cnt;

  d.n_movers = movers;
  d.slot_row = v.slot_row;
  d.comb_out = (uint16_t*)a.out;
  LaunchTimer tm(ws, MOK_K_DOWN, s);
  if (a.mxfp8)
    nt::grouped_gemm_nt<nt::DOWN, true, true><<<grid, nt::NTHR, 0, s>>>(d);
  else
    nt::grouped_gemm_nt<nt::DOWN, false, true><<<grid, nt::NTHR, 0, s>>>(d);
  return hipGetLastError();
}

}  // namespace mok
