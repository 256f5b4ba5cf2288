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
// 256 B-rows, K step 32 (64-byte rows). Operands stream global -> LDS with
// 16-byte LDS-DMA loads into a 3-stage ring of XOR-swizzled rows (two K
// steps in flight while the MFMAs consume the third; no staging registers,
// no LDS write instructions). v_mfma_f32_32x32x16_bf16 with each wave
// owning a 64 x 128 block (2 x 4 MFMA tiles, 128 fp32 accumulators per
// lane). Two workgroups share each compute unit (77 KiB of LDS and at most
// 256 registers per lane each), so one workgroup's MFMAs run while the
// other waits at a barrier, on LDS, or in its tile prologue/epilogue.
// Workgroup b runs on XCD b % 8; tile ids are split into 8 contiguous
// ranges so the tiles of one expert (which share its weights) run on one
// XCD and hit its L2.
#include "device_common.h"
#include "gemm_common.h"
#include "mok_internal.h"

namespace mok {
namespace {

constexpr int BM = 128, BN = 256, BK = 32, NTHR = 256, NSTAGE = 3;
constexpr int A_ELEMS = BM * BK, B_ELEMS = BN * BK;
constexpr int STAGE_ELEMS = A_ELEMS + B_ELEMS;  // 24 KiB of bf16 per stage
constexpr int kBlocksPerCu = 2;
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

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + __expf(-g)); }

// Per-block LDS besides the A/B stages: the schedule's tile table, offsets
// and kept counts (so decoding a tile id costs no global round trip), and
// per-row metadata of the current tile.
constexpr int kMaxE = 1024;

struct alignas(16) GemmLds {
  uint16_t stage[NSTAGE * STAGE_ELEMS];  // A/B ring
  int32_t tiles[kMaxE + 2];
  int32_t row_src[BM];              // per tile row: source row (token of x, or row of h), -1 = none
  float row_w[BM];                  // per tile row: router weight (down GEMM)
};

// Decode using the LDS copies of the schedule tables.
__device__ __forceinline__ Tile decode_tile_lds(const GemmLds& L, const int32_t* __restrict__ offsets,
                                                const int32_t* __restrict__ kept, int E, int id, int nt_r, int nt_s,
                                                int n_routed_mt, int T) {
  Tile t;
  const int n_routed = n_routed_mt * nt_r;
  if (id < n_routed) {
    const int mt = id / nt_r;
    t.nt = id - mt * nt_r;
    int lo = 0, hi = E;  // largest e with tiles[e] <= mt
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (L.tiles[mid] <= mt)
        lo = mid;
      else
        hi = mid;
    }
    t.e = __builtin_amdgcn_readfirstlane(lo);
    const int base = offsets[t.e];
    t.m0 = base + (mt - L.tiles[t.e]) * BM;
    t.m_end = base + kept[t.e];
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

// MODE 0: gate/up + SwiGLU epilogue. MODE 1: down + router-weight epilogue.
//
// The MFMA is issued with the weight tile as its first operand, so each
// accumulator is a 32 (output columns) x 32 (rows) block: element r of lane
// (lr, lh) is output column 8*(r/4) + 4*lh + r%4, row lr. Each lane thus
// holds runs of 4 consecutive output columns of one row, which pack into
// 8-byte LDS writes when the tile is staged for 16-byte global stores.
template <int MODE>
__global__ void __launch_bounds__(NTHR) __attribute__((amdgpu_waves_per_eu(kBlocksPerCu, kBlocksPerCu)))
grouped_gemm_bf16(GemmParams p) {
  __shared__ GemmLds L;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, lh = lane >> 5;
  const int E = p.E;

  for (int i = tid; i < E + 2; i += NTHR) L.tiles[i] = p.tiles[i];
  const int T = p.hdr[HDR_T];
  __syncthreads();
  const int n_routed_mt = L.tiles[E];
  const int n_all_mt = L.tiles[E + 1];
  const int nt_r = MODE == 0 ? (p.I + 127) / 128 : (p.H + BN - 1) / BN;
  const int nt_s = MODE == 0 ? (p.Is + 127) / 128 : nt_r;
  const int ntiles = n_routed_mt * nt_r + (n_all_mt - n_routed_mt) * nt_s;

  // XCD-aware split of the tile range: workgroup b runs on XCD b % 8.
  int stop, step, first;
  if ((gridDim.x % kNumXcd) == 0) {
    const int xcd = blockIdx.x % kNumXcd, slots = gridDim.x / kNumXcd;
    const int chunk = (ntiles + kNumXcd - 1) / kNumXcd;
    const int start = xcd * chunk;
    stop = min(ntiles, start + chunk);
    step = slots;
    first = start + (int)(blockIdx.x / kNumXcd);
  } else {
    stop = ntiles;
    step = gridDim.x;
    first = blockIdx.x;
  }

  const int ld_c = tid & 7;   // 16-byte chunk of a 128-byte K slice
  const int ld_r = tid >> 3;  // 0..31

  for (int id = first; id < stop; id += step) {
    Tile t = decode_tile_lds(L, p.offsets, p.kept, E, id, nt_r, nt_s, n_routed_mt, T);
    t.e = __builtin_amdgcn_readfirstlane(t.e);
    t.m0 = __builtin_amdgcn_readfirstlane(t.m0);
    t.m_end = __builtin_amdgcn_readfirstlane(t.m_end);
    t.nt = __builtin_amdgcn_readfirstlane(t.nt);
    const bool shared = t.e < 0;
    const int K = MODE == 0 ? p.H : (shared ? p.Is : p.I);
    const int Nd = MODE == 0 ? (shared ? p.Is : p.I) : p.H;  // valid output columns

    // Row metadata, one thread per tile row.
    if (tid < BM) {
      const int r = t.m0 + tid;
      int src = -1;
      float w = 0.f;
      if (r < t.m_end) {
        if (shared) {
          src = r;
          w = 1.f;
        } else {
          const int a = p.row_src[r];
          src = MODE == 0 ? a / p.k : r;
          if (MODE == 1) w = p.router_w[a];
        }
      }
      L.row_src[tid] = src;
      L.row_w[tid] = w;
    }
    __syncthreads();

    // Operand rows as 32-bit byte offsets into per-tile buffer resources;
    // rows outside the tile's valid range get an offset past the
    // resource's size (the hardware returns zeros; those output rows or
    // columns are never stored).
    constexpr uint32_t kOff = 0x80000000u;
    const uint16_t* a_base;
    uint32_t a_bytes;
    if (MODE == 0) {
      a_base = p.x;
      a_bytes = (uint32_t)((int64_t)T * p.H * 2);
    } else {
      a_base = shared ? p.h + p.rows_cap_max * p.I : p.h;
      a_bytes = (uint32_t)(shared ? (int64_t)T * p.Is * 2 : p.rows_cap_max * p.I * 2);
    }
    const int a_ld = MODE == 0 ? p.H : (shared ? p.Is : p.I);
    const i32x4v rs_a = rsrc(a_base, a_bytes);
    // This wave's LDS-DMA rows (one instruction = 16 rows of 64 bytes):
    // A rows 32*wave + 16*i + lane/4 (i < 2), B rows 64*wave + 16*i + lane/4
    // (i < 4); lane % 4 is the physical 16-byte chunk of the row.
    const int dr = lane >> 2, dp = lane & 3;
    uint32_t a_off[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = 32 * wave + 16 * i + dr;
      const int src = L.row_src[row];
      a_off[i] = src >= 0 ? (uint32_t)src * (uint32_t)a_ld * 2u + 16u * (uint32_t)(dp ^ swz64(row)) : kOff;
    }
    const uint16_t* b_base;
    uint32_t b_bytes;
    if (MODE == 0) {
      // waves 0-1 load gate rows, waves 2-3 the matching up rows
      const bool up = wave >= 2;
      b_base = shared ? (up ? p.su : p.sg) : (up ? p.wu : p.wg) + (int64_t)t.e * p.I * p.H;
      b_bytes = (uint32_t)Nd * (uint32_t)p.H * 2u;
    } else {
      b_base = shared ? p.sd : p.wd + (int64_t)t.e * p.H * p.I;
      b_bytes = (uint32_t)p.H * (uint32_t)K * 2u;
    }
    const i32x4v rs_b = rsrc(b_base, b_bytes);
    uint32_t b_off[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int lb = 64 * wave + 16 * i + dr;
      const int n = MODE == 0 ? t.nt * 128 + (lb & 127) : t.nt * BN + lb;
      b_off[i] = n < Nd ? (uint32_t)n * (uint32_t)K * 2u + 16u * (uint32_t)(dp ^ swz64(lb)) : kOff;
    }
    const uint32_t lds0 = lds_addr(L.stage);
    // One K step: 6 LDS-DMA loads per lane.
    auto issue = [&](int stage, int k0) {
      const uint32_t sbase = lds0 + (uint32_t)stage * STAGE_ELEMS * 2u;
      const uint32_t kb = (uint32_t)k0 * 2u;
#pragma unroll
      for (int i = 0; i < 2; ++i) lds_dma16(rs_a, a_off[i], kb, sbase + (uint32_t)(32 * wave + 16 * i) * 64u);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        lds_dma16(rs_b, b_off[i], kb, sbase + (uint32_t)A_ELEMS * 2u + (uint32_t)(64 * wave + 16 * i) * 64u);
    };

    f32x16 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int sw = swz64(lr);  // rows read by this lane are lr mod 32
    // Fragments of K sub-step ks (16 wide) are read into one of two register
    // sets while the MFMAs consume the other.
    bf16x8 fa[2][2], fb[2][4];
    auto read_frags = [&](int set, int stage, int ks) {
      const uint16_t* As = L.stage + stage * STAGE_ELEMS;
      const uint16_t* Bs = As + A_ELEMS;
      const int pc = ((2 * ks + lh) ^ sw) * 8;
#pragma unroll
      for (int i = 0; i < 2; ++i) fa[set][i] = *reinterpret_cast<const bf16x8*>(As + (wm * 64 + i * 32 + lr) * BK + pc);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int br = MODE == 0 ? ((j < 2) ? wn * 64 + j * 32 : 128 + wn * 64 + (j - 2) * 32) : wn * 128 + j * 32;
        fb[set][j] = *reinterpret_cast<const bf16x8*>(Bs + (br + lr) * BK + pc);
      }
    };
    auto mfmas = [&](int set) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[set][j], fa[set][i], acc[i][j], 0, 0, 0);
    };

    // 3-stage ring: K steps kt+1 and kt+2 are in flight (6 loads per lane
    // each) while step kt is consumed.
    const int nk = K / BK;
    wait_vmcnt<0>();  // stores of the previous tile's epilogue are older than these loads
    issue(0, 0);
    if (nk > 1) issue(1, BK);
    for (int kt = 0; kt < nk; ++kt) {
      if (kt + 1 < nk)
        wait_vmcnt<6>();
      else
        wait_vmcnt<0>();
      __syncthreads();  // every wave's loads of step kt landed; step kt-1's stage is free
      if (kt + 2 < nk) issue((kt + 2) % NSTAGE, (kt + 2) * BK);
      const int st = kt % NSTAGE;
      read_frags(0, st, 0);
      read_frags(1, st, 1);
      __builtin_amdgcn_sched_barrier(0);
      mfmas(0);
      mfmas(1);
    }

    // Epilogue: each wave stages its sub-tile in LDS (the stages are free
    // after this barrier), then writes whole row segments with 16-byte
    // stores (one instruction covers 4 or 8 contiguous row segments instead
    // of 32 rows of 16 bytes each).
    __syncthreads();
    const int rows_here = t.m_end - t.m0;
    if (MODE == 0) {
      constexpr int SW = 64 + 8;  // staged row stride (bf16): 144 bytes
      uint16_t* reg = L.stage + wave * 64 * SW;
      uint16_t* outs[3] = {shared ? p.h + p.rows_cap_max * p.I : p.h,
                           p.ctx_g ? (shared ? p.ctx_g + p.rows_cap_max * p.I : p.ctx_g) : nullptr,
                           p.ctx_u ? (shared ? p.ctx_u + p.rows_cap_max * p.I : p.ctx_u) : nullptr};
      const int nout = p.ctx_g ? 3 : 1;
      for (int b = 0; b < nout; ++b) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int jg = 0; jg < 2; ++jg)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              float v[4];
#pragma unroll
              for (int c = 0; c < 4; ++c) {
                const float g = acc[i][jg][4 * q + c], u = acc[i][jg + 2][4 * q + c];
                v[c] = b == 0 ? silu_f(g) * u : (b == 1 ? g : u);
              }
              *reinterpret_cast<uint2*>(reg + (i * 32 + lr) * SW + jg * 32 + 8 * q + 4 * lh) =
                  make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
            }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        // 64 rows x 8 chunks of 16 bytes: 8 rows per instruction
        const int col = t.nt * 128 + wn * 64 + (lane & 7) * 8;
#pragma unroll
        for (int it = 0; it < 8; ++it) {
          const int r = it * 8 + (lane >> 3);
          const int ml = wm * 64 + r;
          const u32x4 v = *reinterpret_cast<const u32x4*>(reg + r * SW + (lane & 7) * 8);
          if (ml < rows_here && col < Nd)
            *reinterpret_cast<u32x4*>(outs[b] + (int64_t)(t.m0 + ml) * Nd + col) = v;
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      }
    } else {
      constexpr int SW = 128 + 8;  // 272 bytes
      uint16_t* reg = L.stage + wave * 64 * SW;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const float w = L.row_w[wm * 64 + i * 32 + lr];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            *reinterpret_cast<uint2*>(reg + (i * 32 + lr) * SW + j * 32 + 8 * q + 4 * lh) =
                make_uint2(pack_bf16x2(w * acc[i][j][4 * q], w * acc[i][j][4 * q + 1]),
                           pack_bf16x2(w * acc[i][j][4 * q + 2], w * acc[i][j][4 * q + 3]));
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      uint16_t* yb = shared ? p.y + p.rows_cap_max * p.H : p.y;
      const int col = t.nt * BN + wn * 128 + (lane & 15) * 8;
      // 64 rows x 16 chunks of 16 bytes: 4 rows per instruction
#pragma unroll
      for (int it = 0; it < 16; ++it) {
        const int r = it * 4 + (lane >> 4);
        const int ml = wm * 64 + r;
        const u32x4 v = *reinterpret_cast<const u32x4*>(reg + r * SW + (lane & 15) * 8);
        if (ml < rows_here && col < Nd) *reinterpret_cast<u32x4*>(yb + (int64_t)(t.m0 + ml) * p.H + col) = v;
      }
    }
    __syncthreads();  // row metadata and LDS stages are reused by the next tile
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
  const int grid = ws->num_cus * kBlocksPerCu;
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
