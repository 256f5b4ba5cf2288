// BF16 backward of the grouped SwiGLU expert MLP.
//
// "nemo_automodel.components.moe.mok_experts", _MoKRuntime.backward: one
// gradient per float input of the forward (x, router weights, the three
// routed and the three shared weight tensors), reusing the forward's
// schedule and saved context; the integer expert ids get none.
// "Mixture-of-Kittens: a deterministic MoE megakernel for NVL72 racks",
// section "The two API layers and the schedule object": backward takes the
// same schedule object as forward.
//
// Per kept row r (token t, expert e, router weight w), with G, U, h saved by
// the forward and y = W_d h the unweighted expert output:
//   dh_hat = W_d^T dOut[t]                 d_router_weight = <dh_hat, h> = <dOut[t], y>
//   dh = w * dh_hat                        dG = dh * U * s * (1 + G (1 - s)), s = sigmoid(G)
//   dU = dh * silu(G)                      dA_r = W_g^T dG + W_u^T dU
//   dx[t] = sum over t's kept rows of dA_r (+ the shared expert's row)
//   dW_d[e] += dOut[t] (w h)^T,  dW_g[e] += dG x_t^T,  dW_u[e] += dU x_t^T
// and the same for the shared expert with w = 1 (no router-weight gradient).
//
// Launch sequence (stream-ordered, no host synchronisation):
//   transpose : W_d^T [E, I, H], W_g^T and W_u^T [E, H, I] (and shared)
//   bwd_dh    : NT grouped GEMM of grad_out rows (gathered by token in the
//               operand loads) x W_d^T; epilogue writes dG, dU and per-tile
//               partial sums of d_router_weight
//   dw reduce : d_router_weights[t, j] = fixed-order sum of the partials
//   bwd_dx    : NT grouped GEMM [dG | dU] x [W_g^T | W_u^T] -> dA rows
//   dx        : fixed-order gather-sum of dA rows back to token order
//   dW operands: x rows, w * grad_out rows, h, dG, dU written transposed
//               per expert ([cols, K_e], K_e = its rows rounded up to 128)
//   bwd_dw    : the same NT grouped GEMM (mode BWD_DW), the three weight
//               gradients per expert, contracting over the expert's rows
#include "device_common.h"
#include "combine.h"
#include "gemm_nt.h"
#include "mok_internal.h"

namespace mok {
namespace {

// out[b][c][r] = in[b][r][c] for bf16 [nb][R][C]; R, C multiples of 64.
__global__ void __launch_bounds__(256) transpose_bf16(const uint16_t* __restrict__ in, uint16_t* __restrict__ out,
                                                      int R, int C) {
  __shared__ uint16_t tile[64][64 + 2];
  const int tiles_c = C / 64;
  const int tr = blockIdx.x / tiles_c, tc = blockIdx.x - tr * tiles_c;
  const int64_t b = blockIdx.y;
  const uint16_t* src = in + b * (int64_t)R * C;
  uint16_t* dst = out + b * (int64_t)R * C;
  const int t = threadIdx.x;
  // load 64 rows x 64 columns: 8 threads per row, 8 elements each, 2 passes
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int r = pass * 32 + (t >> 3), c = (t & 7) * 8;
    const uint4 v = *reinterpret_cast<const uint4*>(src + (int64_t)(tr * 64 + r) * C + tc * 64 + c);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      tile[r][c + 2 * q] = (uint16_t)(w[q] & 0xFFFFu);
      tile[r][c + 2 * q + 1] = (uint16_t)(w[q] >> 16);
    }
  }
  __syncthreads();
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int c = pass * 32 + (t >> 3), r = (t & 7) * 8;  // output row c, columns r .. r+7
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) w[q] = (uint32_t)tile[r + 2 * q][c] | ((uint32_t)tile[r + 2 * q + 1][c] << 16);
    *reinterpret_cast<uint4*>(dst + (int64_t)(tc * 64 + c) * R + tr * 64 + r) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// d_router_weights[a] = sum over parts (fixed order) of dw_part[slot_row[a]],
// 0 for dropped or invalid assignments.
__global__ void __launch_bounds__(256) reduce_dw(const int32_t* __restrict__ hdr, int hash, int32_t* status,
                                                 const int32_t* __restrict__ slot_row,
                                                 const float* __restrict__ dw_part, int parts, int n_parts_used, int k,
                                                 float* __restrict__ dwr) {
  if (!sched_matches(hdr, hash, status)) return;
  const int64_t n = (int64_t)hdr[HDR_T] * k;
  for (int64_t a = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; a < n; a += (int64_t)gridDim.x * blockDim.x) {
    const int row = slot_row[a];
    float s = 0.f;
    if (row >= 0)
      for (int q = 0; q < n_parts_used; ++q) s += dw_part[(int64_t)row * parts + q];
    dwr[a] = s;
  }
}


hipError_t transpose(const void* in, void* out, int nb, int R, int C, hipStream_t s) {
  if (nb == 0) return hipSuccess;
  dim3 grid((unsigned)((R / 64) * (C / 64)), (unsigned)nb);
  transpose_bf16<<<grid, 256, 0, s>>>((const uint16_t*)in, (uint16_t*)out, R, C);
  return hipGetLastError();
}

}  // namespace

int dw_parts(const mok_config& c) {
  const int Imax = c.intermediate > c.shared_intermediate ? c.intermediate : c.shared_intermediate;
  return nt::kDwPartsPerNTile * ((Imax + nt::BN - 1) / nt::BN);
}

// MXFP8 backward: every GEMM operand quantized along that GEMM's own
// contraction dimension (blocks of 32, E8M0 scales), fp32 accumulation.
//   dh_hat = Q_H(grad_out rows) Q_H(W_down)            -> dG, dU (fp32), partial dw
//   (one pass over dG, dU: Q_r for the weight gradients and Q_I for dA)
//   dA     = Q_I(dG) Q_I(W_gate) + Q_I(dU) Q_I(W_up)   -> dx (fixed-order sum)
//   dW_down = Q_r(w grad_out rows)^T Q_r(h),  dW_gate = Q_r(dG)^T Q_r(x rows),  dW_up likewise
// with Q_r in 32-row blocks of each expert's segment and h the forward's
// MXFP8 h. dw = <dh_hat, h>.
static hipError_t launch_backward_mxfp8(mok_workspace* ws, const void* sched, const BwdArgs& a, hipStream_t s) {
  const mok_config& c = ws->cfg;
  const int E = c.num_experts, H = c.hidden, I = c.intermediate, Is = c.shared_intermediate, k = c.topk;
  SchedView v = sched_view(const_cast<void*>(sched), ws->layout);
  v.hash = (int)config_hash(ws->cfg);
  v.status = ws->status;
  const int64_t rcm = ws->layout.rows_cap_max;
  const size_t ce = ctx_elems(c, ws->layout);
  const mok_weights* w = a.w;
  const mok_grads* g = a.g;
  BwdScratch& b = ws->bwd;
  const int qgrid = ws->num_cus * 4;
  // The weights transposed and quantized along each backward GEMM's
  // contraction: W_down [E,H,I] -> [E,I,H] along H; W_gate / W_up [E,I,H] ->
  // [E,H,I] along I. Either given so by the caller (scale pointers set,
  // from mok_mxfp8_quantize_transposed) or made here from the BF16 weights.
  struct Wt {
    const uint8_t *c, *s;
  } wd{b.wdTq, b.wdTs}, wg{b.wgTq, b.wgTs}, wu{b.wuTq, b.wuTs}, sd{b.sdTq, b.sdTs}, sg{b.sgTq, b.sgTs},
      su{b.suTq, b.suTs};
  if (a.weights_t) {
    wd = {(const uint8_t*)w->routed_down, w->routed_down_scale};
    wg = {(const uint8_t*)w->routed_gate, w->routed_gate_scale};
    wu = {(const uint8_t*)w->routed_up, w->routed_up_scale};
    sd = {(const uint8_t*)w->shared_down, w->shared_down_scale};
    sg = {(const uint8_t*)w->shared_gate, w->shared_gate_scale};
    su = {(const uint8_t*)w->shared_up, w->shared_up_scale};
  } else {
    LaunchTimer tm(ws, MOK_K_BWD_TRANSPOSE, s);
    MOK_HIP_TRY(launch_quantize_t_matrix(w->routed_down, E, H, I, b.wdTq, b.wdTs, qgrid, s));
    MOK_HIP_TRY(launch_quantize_t_matrix(w->routed_gate, E, I, H, b.wgTq, b.wgTs, qgrid, s));
    MOK_HIP_TRY(launch_quantize_t_matrix(w->routed_up, E, I, H, b.wuTq, b.wuTs, qgrid, s));
    if (Is > 0) {
      MOK_HIP_TRY(launch_quantize_t_matrix(w->shared_down, 1, H, Is, b.sdTq, b.sdTs, qgrid, s));
      MOK_HIP_TRY(launch_quantize_t_matrix(w->shared_gate, 1, Is, H, b.sgTq, b.sgTs, qgrid, s));
      MOK_HIP_TRY(launch_quantize_t_matrix(w->shared_up, 1, Is, H, b.suTq, b.suTs, qgrid, s));
    }
  }
  {
    LaunchTimer tm(ws, MOK_K_BWD_QUANT, s);
    MOK_HIP_TRY(launch_quantize_rows_dev(a.grad_out, v, c.max_tokens, H, ws->xq, ws->xq_scale, s));
  }
  const int grid = ws->num_cus;
  auto sched_params = [&](nt::Params& p, int bm) {
    p.hdr = v.header;
    p.offsets = v.offsets;
    p.kept = v.kept;
    p.tiles = v.tiles + tile_bm_index(bm) * (E + 2);
    p.row_src = v.row_src;
    p.E = E;
    p.k = k;
    p.H = H;
    p.I = I;
    p.Is = Is;
    p.rows_cap_max = rcm;
    p.swiglu_lim = swiglu_lim(c);
    p.cfg_hash = v.hash;
    p.status = v.status;
  };
  {
    nt::Params p{};
    sched_params(p, nt::BM);
    p.router_w = a.router_w;
    p.a_tok = ws->xq;
    p.a_tok_scale = ws->xq_scale;
    p.b0 = wd.c;
    p.b0s = wd.s;
    p.sb0 = sd.c;
    p.sb0s = sd.s;
    p.g_in = a.ctx_g;
    p.u_in = a.ctx_u;
    p.hq_in = (const uint8_t*)a.ctx_h;
    p.hq_scale_in = (const uint8_t*)a.ctx_h + ce;
    // dG and dU quantized in the epilogue: along I for dA (dG into the
    // workspace's hq buffer, dU into duq), along rows for the weight gradients
    p.rq_g = ws->hq;
    p.rq_gs = ws->hq_scale;
    p.rq_u = b.duq;
    p.rq_us = b.duq_scale;
    p.tq = b.tq;
    p.tiles128 = v.tiles + tile_bm_index(128) * (E + 2);
    p.dw_part = b.dw_part;
    p.dw_parts = dw_parts(c);
    LaunchTimer tm(ws, MOK_K_BWD_DH, s);
    nt::grouped_gemm_nt<nt::BWD_DH, true><<<grid, nt::NTHR, 0, s>>>(p);
    MOK_HIP_TRY(hipGetLastError());
  }
  {
    LaunchTimer tm(ws, MOK_K_BWD_DW_REDUCE, s);
    const int n_used = nt::kDwPartsPerNTile * ((I + nt::BN - 1) / nt::BN);
    const int64_t n = c.max_tokens * k;
    const int rgrid = (int)std::min<int64_t>((n + 255) / 256, (int64_t)ws->num_cus * 16);
    reduce_dw<<<rgrid, 256, 0, s>>>(v.header, v.hash, v.status, v.slot_row, b.dw_part, dw_parts(c), n_used, k,
                                    g->d_router_weights);
    MOK_HIP_TRY(hipGetLastError());
  }
  {
    nt::Params p{};
    sched_params(p, nt::BM);
    p.a_row = ws->hq;
    p.a_row_scale = ws->hq_scale;
    p.a_row2 = b.duq;
    p.a_row2_scale = b.duq_scale;
    p.b0 = wg.c;
    p.b0s = wg.s;
    p.b1 = wu.c;
    p.b1s = wu.s;
    p.sb0 = sg.c;
    p.sb0s = sg.s;
    p.sb1 = su.c;
    p.sb1s = su.s;
    p.out = ws->ybuf;
    LaunchTimer tm(ws, MOK_K_BWD_DX_ROWS, s);
    nt::grouped_gemm_nt<nt::BWD_DX, true><<<grid, nt::NTHR, 0, s>>>(p);
    MOK_HIP_TRY(hipGetLastError());
  }
  {
    LaunchTimer tm(ws, MOK_K_BWD_DX_SUM, s);
    const int cgrid = (int)std::min<int64_t>(c.max_tokens, (int64_t)ws->num_cus * 8);
    const uint16_t* y = (const uint16_t*)ws->ybuf;
    sum_slot_rows<<<cgrid, 256, 0, s>>>(v.header, v.hash, v.status, v.slot_row, y, Is > 0 ? y + rcm * H : nullptr,
                                        (uint16_t*)g->dx, H, k);
    MOK_HIP_TRY(hipGetLastError());
  }
  {
    LaunchTimer tm(ws, MOK_K_BWD_QUANT, s);
    const TqArrays& q = b.tq;
    const uint8_t* hq = (const uint8_t*)a.ctx_h;
    MOK_HIP_TRY(launch_quantize_t_rows(0, v, a.x, nullptr, nullptr, nullptr, E, k, H, H, rcm, q.kr_cap, q.x, q.xs,
                                       qgrid, s));
    MOK_HIP_TRY(launch_quantize_t_rows(1, v, a.grad_out, nullptr, nullptr, a.router_w, E, k, H, H, rcm, q.kr_cap,
                                       q.dy, q.dys, qgrid, s));
    MOK_HIP_TRY(launch_quantize_t_rows(3, v, nullptr, hq, hq + ce, nullptr, E, k, I, Is, rcm, q.kr_cap, q.h, q.hs,
                                       qgrid, s));
  }
  {
    nt::Params p{};
    sched_params(p, 128);  // the 128-row tile table gives each expert's K offset and length
    p.tq = b.tq;
    p.d_wd = (uint16_t*)g->d_routed_down;
    p.d_wg = (uint16_t*)g->d_routed_gate;
    p.d_wu = (uint16_t*)g->d_routed_up;
    p.d_sd = (uint16_t*)g->d_shared_down;
    p.d_sg = (uint16_t*)g->d_shared_gate;
    p.d_su = (uint16_t*)g->d_shared_up;
    LaunchTimer tm(ws, MOK_K_BWD_DW, s);
    nt::grouped_gemm_nt<nt::BWD_DW, true><<<grid, nt::NTHR, 0, s>>>(p);
    MOK_HIP_TRY(hipGetLastError());
  }
  return hipSuccess;
}

hipError_t launch_backward(mok_workspace* ws, const void* sched, const BwdArgs& a, hipStream_t s) {
  if (a.mxfp8) return launch_backward_mxfp8(ws, sched, a, s);
  const mok_config& c = ws->cfg;
  const int E = c.num_experts, H = c.hidden, I = c.intermediate, Is = c.shared_intermediate, k = c.topk;
  SchedView v = sched_view(const_cast<void*>(sched), ws->layout);
  v.hash = (int)config_hash(ws->cfg);
  v.status = ws->status;
  const int64_t rcm = ws->layout.rows_cap_max;
  const mok_weights* w = a.w;
  const mok_grads* g = a.g;
  BwdScratch& b = ws->bwd;
  {
    LaunchTimer tm(ws, MOK_K_BWD_TRANSPOSE, s);
    MOK_HIP_TRY(transpose(w->routed_down, b.wdT, E, H, I, s));  // [E,H,I] -> [E,I,H]
    MOK_HIP_TRY(transpose(w->routed_gate, b.wgT, E, I, H, s));  // [E,I,H] -> [E,H,I]
    MOK_HIP_TRY(transpose(w->routed_up, b.wuT, E, I, H, s));
    if (Is > 0) {
      MOK_HIP_TRY(transpose(w->shared_down, b.sdT, 1, H, Is, s));
      MOK_HIP_TRY(transpose(w->shared_gate, b.sgT, 1, Is, H, s));
      MOK_HIP_TRY(transpose(w->shared_up, b.suT, 1, Is, H, s));
    }
  }
  const int grid = ws->num_cus;  // one 512-thread workgroup per compute unit
  auto sched_params = [&](nt::Params& p) {
    p.hdr = v.header;
    p.offsets = v.offsets;
    p.kept = v.kept;
    p.tiles = v.tiles + tile_bm_index(nt::BM) * (E + 2);
    p.row_src = v.row_src;
    p.E = E;
    p.k = k;
    p.H = H;
    p.I = I;
    p.Is = Is;
    p.rows_cap_max = rcm;
    p.swiglu_lim = swiglu_lim(c);
    p.cfg_hash = v.hash;
    p.status = v.status;
  };
  {
    nt::Params p{};
    sched_params(p);
    p.router_w = a.router_w;
    p.a_tok = a.grad_out;
    p.b0 = b.wdT;
    p.sb0 = b.sdT;
    p.g_in = a.ctx_g;
    p.u_in = a.ctx_u;
    p.h_in = (const uint16_t*)a.ctx_h;
    p.dg_out = b.dg;
    p.du_out = b.du;
    p.dw_part = b.dw_part;
    p.dw_parts = dw_parts(c);
    LaunchTimer tm(ws, MOK_K_BWD_DH, s);
    nt::grouped_gemm_nt<nt::BWD_DH, false><<<grid, nt::NTHR, 0, s>>>(p);
    MOK_HIP_TRY(hipGetLastError());
  }
  {
    LaunchTimer tm(ws, MOK_K_BWD_DW_REDUCE, s);
    const int n_used = nt::kDwPartsPerNTile * ((I + nt::BN - 1) / nt::BN);
    const int64_t n = c.max_tokens * k;
    const int rgrid = (int)std::min<int64_t>((n + 255) / 256, (int64_t)ws->num_cus * 16);
    reduce_dw<<<rgrid, 256, 0, s>>>(v.header, v.hash, v.status, v.slot_row, b.dw_part, dw_parts(c), n_used, k,
                                    g->d_router_weights);
    MOK_HIP_TRY(hipGetLastError());
  }
  {
    nt::Params p{};
    sched_params(p);
    p.a_row = b.dg;
    p.a_row2 = b.du;
    p.b0 = b.wgT;
    p.b1 = b.wuT;
    p.sb0 = b.sgT;
    p.sb1 = b.suT;
    p.out = ws->ybuf;
    LaunchTimer tm(ws, MOK_K_BWD_DX_ROWS, s);
    nt::grouped_gemm_nt<nt::BWD_DX, false><<<grid, nt::NTHR, 0, s>>>(p);
    MOK_HIP_TRY(hipGetLastError());
  }
  {
    LaunchTimer tm(ws, MOK_K_BWD_DX_SUM, s);
    const int cgrid = (int)std::min<int64_t>(c.max_tokens, (int64_t)ws->num_cus * 8);
    const uint16_t* y = (const uint16_t*)ws->ybuf;
    sum_slot_rows<<<cgrid, 256, 0, s>>>(v.header, v.hash, v.status, v.slot_row, y, Is > 0 ? y + rcm * H : nullptr,
                                        (uint16_t*)g->dx, H, k);
    MOK_HIP_TRY(hipGetLastError());
  }
  {
    // weight-gradient operands, transposed per expert ([cols, K_e] bf16):
    // x rows, router weight times grad_out rows, h, dG, dU
    LaunchTimer tm(ws, MOK_K_BWD_GATHER, s);
    const TqArrays& q = b.tq16;
    const int qgrid = ws->num_cus * 4;
    MOK_HIP_TRY(launch_quantize_t_rows(0, v, a.x, nullptr, nullptr, nullptr, E, k, H, H, rcm, q.kr_cap, q.x, nullptr,
                                       qgrid, s, true));
    MOK_HIP_TRY(launch_quantize_t_rows(1, v, a.grad_out, nullptr, nullptr, a.router_w, E, k, H, H, rcm, q.kr_cap, q.dy,
                                       nullptr, qgrid, s, true));
    MOK_HIP_TRY(launch_quantize_t_rows(2, v, a.ctx_h, nullptr, nullptr, nullptr, E, k, I, Is, rcm, q.kr_cap, q.h, nullptr,
                                       qgrid, s, true));
    MOK_HIP_TRY(launch_quantize_t_rows(2, v, b.dg, nullptr, nullptr, nullptr, E, k, I, Is, rcm, q.kr_cap, q.dg, nullptr,
                                       qgrid, s, true));
    MOK_HIP_TRY(launch_quantize_t_rows(2, v, b.du, nullptr, nullptr, nullptr, E, k, I, Is, rcm, q.kr_cap, q.du, nullptr,
                                       qgrid, s, true));
  }
  {
    nt::Params p{};
    sched_params(p);
    p.tiles = v.tiles + tile_bm_index(128) * (E + 2);  // each expert's K offset and length
    p.tq = b.tq16;
    p.d_wd = (uint16_t*)g->d_routed_down;
    p.d_wg = (uint16_t*)g->d_routed_gate;
    p.d_wu = (uint16_t*)g->d_routed_up;
    p.d_sd = (uint16_t*)g->d_shared_down;
    p.d_sg = (uint16_t*)g->d_shared_gate;
    p.d_su = (uint16_t*)g->d_shared_up;
    LaunchTimer tm(ws, MOK_K_BWD_DW, s);
    nt::grouped_gemm_nt<nt::BWD_DW, false><<<grid, nt::NTHR, 0, s>>>(p);
    MOK_HIP_TRY(hipGetLastError());
  }
  return hipSuccess;
}

}  // namespace mok
