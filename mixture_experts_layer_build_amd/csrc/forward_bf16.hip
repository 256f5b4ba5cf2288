// BF16 forward of the grouped SwiGLU expert MLP and the router-weighted
// combine.
//
// "nemo_automodel.components.moe.mok_experts", GroupedExpertsMoK.forward and
// _MoKRuntime.forward: fused shared and routed SwiGLU experts; routed
// gate/up [E, I, H], down [E, H, I]; shared gate/up [I_s, H], down [H, I_s];
// no expert bias. "Mixture-of-Kittens: a deterministic MoE megakernel for
// NVL72 racks", section "The two API layers and the schedule object": the
// schedule drives both dispatch (here a gather of token rows into the
// expert-contiguous order) and combine (a gather-sum back to token order).
//
// Kernels (all persistent: one workgroup per compute unit, a tile loop read
// from the schedule on the device, so no host ever needs the counts):
//   gate_up : per expert segment, [rows, H] x [H, I] for gate and up in one
//             tile (A rows gathered from x through the schedule's row map),
//             epilogue h = silu(g) * u in fp32 -> bf16 (g, u saved for
//             backward when a context is given).
//   down    : per segment, h [rows, I] x [I, H], epilogue y = w_r * acc in
//             fp32 -> bf16 (w_r the router weight of the row's assignment,
//             1 for the shared expert).
//   combine : out[t] = bf16(sum over j in slot order of y[slot_row[t, j]]
//             + y_shared[t]), fp32 accumulation, no atomics.
//
// GEMM tiling for gfx950: 256 threads (4 wave64), output tile 128 rows x
// 256 B-rows, K step 64, double-buffered LDS with rows padded to 144 bytes
// (16-byte operand reads of 32 consecutive rows fall in distinct banks),
// v_mfma_f32_32x32x16_bf16 with each wave owning a 64 x 128 block (2 x 4
// MFMA tiles, 128 fp32 accumulators per lane). Workgroup b runs on XCD
// b % 8; tile ids are split into 8 contiguous ranges so the tiles of one
// expert (which share its weights) run on one XCD and hit its L2.
#include "device_common.h"
#include "mok_internal.h"

namespace mok {
namespace {

constexpr int BM = 128, BN = 256, BK = 64, LDK = BK + 8, NTHR = 256;
constexpr int A_ELEMS = BM * LDK, B_ELEMS = BN * LDK;
constexpr int STAGE_ELEMS = A_ELEMS + B_ELEMS;
constexpr int kNumXcd = 8;

struct GemmParams {
  // schedule
  const int32_t* hdr;
  const int32_t* offsets;
  const int32_t* kept;
  const int32_t* tiles;    // per-expert prefix sums of 128-row tiles; [E] routed total, [E+1] with shared
  const int32_t* row_src;
  int E, k;
  int H, I, Is;
  int64_t rows_cap_max;
  // gate/up operands
  const uint16_t* x;
  const uint16_t* wg;
  const uint16_t* wu;
  const uint16_t* sg;
  const uint16_t* su;
  // down operands
  const uint16_t* wd;
  const uint16_t* sd;
  const float* router_w;
  // buffers
  uint16_t* h;       // routed [rows_cap_max, I] then shared [T_max, Is]
  uint16_t* ctx_g;   // same layout as h, or null
  uint16_t* ctx_u;
  uint16_t* y;       // routed [rows_cap_max, H] then shared [T_max, H]
};

struct Tile {
  int e;        // expert, or -1 for the shared expert
  int m0;       // first row (schedule row, or token for the shared expert)
  int m_end;    // one past the last valid row
  int nt;       // N tile
};

// Tile id -> (expert, rows, N tile). Routed tiles first (M tile major, N
// fastest), then the shared expert's.
__device__ __forceinline__ Tile decode_tile(const GemmParams& p, int id, int nt_r, int nt_s, int n_routed_mt, int T) {
  Tile t;
  const int n_routed = n_routed_mt * nt_r;
  if (id < n_routed) {
    const int mt = id / nt_r;
    t.nt = id - mt * nt_r;
    int lo = 0, hi = p.E;  // largest e with tiles[e] <= mt
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (p.tiles[mid] <= mt)
        lo = mid;
      else
        hi = mid;
    }
    t.e = lo;
    const int base = p.offsets[lo];
    t.m0 = base + (mt - p.tiles[lo]) * BM;
    t.m_end = base + p.kept[lo];
  } else {
    const int sid = id - n_routed;
    const int mt = sid / nt_s;
    t.nt = sid - mt * nt_s;
    t.e = -1;
    t.m0 = mt * BM;
    t.m_end = T;
  }
  return t;
}

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + __expf(-g)); }

// MODE 0: gate/up + SwiGLU epilogue. MODE 1: down + router-weight epilogue.
template <int MODE>
__global__ void __launch_bounds__(NTHR) __attribute__((amdgpu_waves_per_eu(1, 1)))
grouped_gemm_bf16(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * STAGE_ELEMS];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, lh = lane >> 5;
  const int T = p.hdr[HDR_T];
  const int n_routed_mt = p.tiles[p.E];
  const int n_all_mt = p.tiles[p.E + 1];
  const int nt_r = MODE == 0 ? (p.I + 127) / 128 : (p.H + BN - 1) / BN;
  const int nt_s = MODE == 0 ? (p.Is + 127) / 128 : nt_r;
  const int ntiles = n_routed_mt * nt_r + (n_all_mt - n_routed_mt) * nt_s;

  // XCD-aware split of the tile range.
  int start, stop, step, first;
  if ((gridDim.x % kNumXcd) == 0) {
    const int xcd = blockIdx.x % kNumXcd, slots = gridDim.x / kNumXcd;
    const int chunk = (ntiles + kNumXcd - 1) / kNumXcd;
    start = xcd * chunk;
    stop = min(ntiles, start + chunk);
    step = slots;
    first = start + (int)(blockIdx.x / kNumXcd);
  } else {
    start = 0;
    stop = ntiles;
    step = gridDim.x;
    first = blockIdx.x;
  }
  (void)start;

  const int ld_c = tid & 7;   // 16-byte chunk of a 128-byte K slice
  const int ld_r = tid >> 3;  // 0..31

  for (int id = first; id < stop; id += step) {
    const Tile t = decode_tile(p, id, nt_r, nt_s, n_routed_mt, T);
    const bool shared = t.e < 0;
    const int K = MODE == 0 ? p.H : (shared ? p.Is : p.I);
    const int Nd = MODE == 0 ? (shared ? p.Is : p.I) : p.H;  // valid output columns

    // Row sources for this thread's 4 A rows and 8 B rows.
    const uint16_t* a_src[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = t.m0 + ld_r + 32 * i;
      a_src[i] = nullptr;
      if (r < t.m_end) {
        if (MODE == 0) {
          const int tok = shared ? r : p.row_src[r] / p.k;
          a_src[i] = p.x + (int64_t)tok * p.H;
        } else {
          a_src[i] = shared ? p.h + p.rows_cap_max * p.I + (int64_t)r * p.Is : p.h + (int64_t)r * p.I;
        }
      }
    }
    const uint16_t* b_src[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int lb = ld_r + 32 * i;
      b_src[i] = nullptr;
      if (MODE == 0) {
        const bool up = lb >= 128;
        const int n = t.nt * 128 + (lb & 127);
        if (n < Nd) {
          const uint16_t* base = shared ? (up ? p.su : p.sg) : (up ? p.wu : p.wg) + (int64_t)t.e * p.I * p.H;
          b_src[i] = base + (int64_t)n * p.H;
        }
      } else {
        const int n = t.nt * BN + lb;
        if (n < Nd) b_src[i] = shared ? p.sd + (int64_t)n * p.Is : p.wd + ((int64_t)t.e * p.H + n) * p.I;
      }
    }

    f32x16 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    uint4 ra[4], rb[8];
    auto gload = [&](int k0) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        ra[i] = a_src[i] ? *reinterpret_cast<const uint4*>(a_src[i] + k0 + ld_c * 8) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        rb[i] = b_src[i] ? *reinterpret_cast<const uint4*>(b_src[i] + k0 + ld_c * 8) : make_uint4(0, 0, 0, 0);
    };
    auto lstore = [&](int stage) {
      uint16_t* As = lds + stage * STAGE_ELEMS;
      uint16_t* Bs = As + A_ELEMS;
#pragma unroll
      for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(As + (ld_r + 32 * i) * LDK + ld_c * 8) = ra[i];
#pragma unroll
      for (int i = 0; i < 8; ++i) *reinterpret_cast<uint4*>(Bs + (ld_r + 32 * i) * LDK + ld_c * 8) = rb[i];
    };

    const int nk = K / BK;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      if (kt + 1 < nk) gload((kt + 1) * BK);
      const uint16_t* As = lds + cur * STAGE_ELEMS;
      const uint16_t* Bs = As + A_ELEMS;
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        bf16x8 af[2], bfr[4];
#pragma unroll
        for (int i = 0; i < 2; ++i)
          af[i] = *reinterpret_cast<const bf16x8*>(As + (wm * 64 + i * 32 + lr) * LDK + ks * 16 + lh * 8);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int br = MODE == 0 ? ((j < 2) ? wn * 64 + j * 32 : 128 + wn * 64 + (j - 2) * 32) : wn * 128 + j * 32;
          bfr[j] = *reinterpret_cast<const bf16x8*>(Bs + (br + lr) * LDK + ks * 16 + lh * 8);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
      if (kt + 1 < nk) lstore(cur ^ 1);
      __syncthreads();
    }

    // Epilogue. Accumulator element r of lane (lr, lh) in a 32x32 MFMA tile
    // is row 8*(r/4) + 4*lh + r%4, column lr.
    if (MODE == 0) {
      uint16_t* hb = shared ? p.h + p.rows_cap_max * p.I : p.h;
      uint16_t* gb = p.ctx_g ? (shared ? p.ctx_g + p.rows_cap_max * p.I : p.ctx_g) : nullptr;
      uint16_t* ub = p.ctx_u ? (shared ? p.ctx_u + p.rows_cap_max * p.I : p.ctx_u) : nullptr;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jg = 0; jg < 2; ++jg) {
          const int col = t.nt * 128 + wn * 64 + jg * 32 + lr;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = t.m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
            if (row < t.m_end && col < Nd) {
              const float g = acc[i][jg][r], u = acc[i][jg + 2][r];
              const int64_t o = (int64_t)row * Nd + col;
              hb[o] = f32_to_bf16(silu_f(g) * u);
              if (gb) {
                gb[o] = f32_to_bf16(g);
                ub[o] = f32_to_bf16(u);
              }
            }
          }
        }
    } else {
      uint16_t* yb = shared ? p.y + p.rows_cap_max * p.H : p.y;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = t.m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
          if (row < t.m_end) {
            const float w = shared ? 1.0f : p.router_w[p.row_src[row]];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int col = t.nt * BN + wn * 128 + j * 32 + lr;
              if (col < Nd) yb[(int64_t)row * p.H + col] = f32_to_bf16(w * acc[i][j][r]);
            }
          }
        }
    }
  }
}

// out[t] = bf16(sum_j y[slot_row[t*k + j]] (kept slots, slot order) + y_shared[t]).
__global__ void __launch_bounds__(256) combine_bf16(const int32_t* __restrict__ hdr, const int32_t* __restrict__ slot_row,
                                                    const uint16_t* __restrict__ y, const uint16_t* __restrict__ y_shared,
                                                    uint16_t* __restrict__ out, int H, int k) {
  const int T = hdr[HDR_T];
  const int nchunk = H / 8;
  for (int t = blockIdx.x; t < T; t += gridDim.x) {
    const int32_t* sl = slot_row + (int64_t)t * k;
    for (int c = threadIdx.x; c < nchunk; c += blockDim.x) {
      float acc[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = 0.f;
      for (int j = 0; j < k; ++j) {
        const int row = sl[j];
        if (row < 0) continue;
        const uint4 v = *reinterpret_cast<const uint4*>(y + (int64_t)row * H + c * 8);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * q] += u2f(w[q] << 16);
          acc[2 * q + 1] += u2f(w[q] & 0xFFFF0000u);
        }
      }
      if (y_shared) {
        const uint4 v = *reinterpret_cast<const uint4*>(y_shared + (int64_t)t * H + c * 8);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * q] += u2f(w[q] << 16);
          acc[2 * q + 1] += u2f(w[q] & 0xFFFF0000u);
        }
      }
      uint4 o;
      o.x = pack_bf16x2(acc[0], acc[1]);
      o.y = pack_bf16x2(acc[2], acc[3]);
      o.z = pack_bf16x2(acc[4], acc[5]);
      o.w = pack_bf16x2(acc[6], acc[7]);
      *reinterpret_cast<uint4*>(out + (int64_t)t * H + c * 8) = o;
    }
  }
}

}  // namespace

hipError_t launch_forward_bf16(mok_workspace* ws, const void* sched, const FwdArgs& a, hipStream_t s) {
  const mok_config& c = ws->cfg;
  const SchedView v = sched_view(const_cast<void*>(sched), ws->layout);
  GemmParams p{};
  p.hdr = v.header;
  p.offsets = v.offsets;
  p.kept = v.kept;
  p.tiles = v.tiles + tile_bm_index(BM) * (c.num_experts + 2);
  p.row_src = v.row_src;
  p.E = c.num_experts;
  p.k = c.topk;
  p.H = c.hidden;
  p.I = c.intermediate;
  p.Is = c.shared_intermediate;
  p.rows_cap_max = ws->layout.rows_cap_max;
  p.x = (const uint16_t*)a.x;
  p.wg = (const uint16_t*)a.w->routed_gate;
  p.wu = (const uint16_t*)a.w->routed_up;
  p.wd = (const uint16_t*)a.w->routed_down;
  p.sg = (const uint16_t*)a.w->shared_gate;
  p.su = (const uint16_t*)a.w->shared_up;
  p.sd = (const uint16_t*)a.w->shared_down;
  p.router_w = a.router_w;
  p.h = (uint16_t*)a.h;
  p.ctx_g = (uint16_t*)a.ctx_g;
  p.ctx_u = (uint16_t*)a.ctx_u;
  p.y = (uint16_t*)a.y;
  const int grid = ws->num_cus;
  {
    LaunchTimer tm(ws, MOK_K_GATE_UP, s);
    grouped_gemm_bf16<0><<<grid, NTHR, 0, s>>>(p);
    MOK_HIP_TRY(hipGetLastError());
  }
  {
    LaunchTimer tm(ws, MOK_K_DOWN, s);
    grouped_gemm_bf16<1><<<grid, NTHR, 0, s>>>(p);
    MOK_HIP_TRY(hipGetLastError());
  }
  {
    LaunchTimer tm(ws, MOK_K_COMBINE, s);
    const int cgrid = (int)std::min<int64_t>(c.max_tokens, (int64_t)ws->num_cus * 8);
    const uint16_t* ys = c.shared_intermediate > 0 ? p.y + p.rows_cap_max * p.H : nullptr;
    combine_bf16<<<cgrid, 256, 0, s>>>(v.header, v.slot_row, p.y, ys, (uint16_t*)a.out, c.hidden, c.topk);
    MOK_HIP_TRY(hipGetLastError());
  }
  return hipSuccess;
}

hipError_t launch_forward(mok_workspace* ws, const void* sched, const FwdArgs& a, hipStream_t s) {
  if (a.mxfp8) return launch_forward_mxfp8(ws, sched, a, s);
  return launch_forward_bf16(ws, sched, a, s);
}

}  // namespace mok
