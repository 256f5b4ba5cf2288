// Persistent grouped GEMM over the schedule's expert segments, both
// operands K-contiguous ("NT": C[m, n] = sum_k A[m, k] * B[n, k]), on
// gfx950 MFMA. One kernel template serves the forward (gate/up with the
// SwiGLU epilogue, down with the router-weight epilogue) and the backward
// GEMMs whose contraction runs along a row (grad rows times the transposed
// down weights, and [dG | dU] rows times the transposed gate/up weights).
//
// Tiling: one workgroup of 512 threads (8 wave64, two per SIMD) per compute
// unit, output tile 256 rows x 256 B-rows, one K step = one 128-byte cache
// line of every A and B row (64 bf16 or 128 E4M3 elements). Operands stream
// global -> LDS with 16-byte LDS-DMA loads (a wave instruction fetches 8
// whole lines) into two 64 KiB stages of XOR-swizzled rows; in MXFP8 mode
// the step's E8M0 block scales (one dword per row) follow with 4-byte
// LDS-DMA loads. Wave (wm = wave / 4, wn = wave % 4) owns 128 rows x 64
// B-rows: 4 x 2 MFMA tiles of 32 x 32 (v_mfma_f32_32x32x16_bf16, or
// v_mfma_scale_f32_32x32x64_f8f6f4 with per-lane E8M0 scales), 128 fp32
// accumulators per lane. In an expert's ragged last tile a wave runs only
// the 32-row blocks that hold valid rows (the K loop is instantiated per
// count of live blocks): a tile with 32 valid rows issues 1/8 of a full
// tile's MFMAs and A-fragment reads, and a wave with no valid rows only
// loads and waits, so its SIMD runs the partner wave at full rate. Workgroup b runs on XCD b % 8; tile ids are
// split into 8 contiguous ranges so the tiles of one expert (which share
// its weights) run on one XCD and hit its L2.
//
// The MFMA takes the B (weight) fragment as its first operand, so
// accumulator element r of lane (lr = lane % 32, lh = lane / 32) in an MFMA
// tile is output column 8*(r/4) + 4*lh + r%4 and row lr: every lane holds
// runs of 4 consecutive columns of one row.
#pragma once

#include <type_traits>

#include "device_common.h"
#include "gemm_common.h"
#include "mok_internal.h"

namespace mok {
namespace nt {

constexpr int BM = 256, BN = 256, NTHR = 512, NSTAGE = 2;
constexpr int ROWB = 128;                                     // bytes of one row per K step
constexpr int A_BYTES = BM * ROWB, B_BYTES = BN * ROWB;       // 32 KiB + 32 KiB
constexpr int SA_BYTES = BM * 4, SB_BYTES = BN * 4;           // E8M0 scale dwords of a K step (MXFP8)
constexpr int kNumXcd = 8;
constexpr int kMaxLdsE = 256;  // schedules with more experts search the tile table in global memory
constexpr int kGroupM = 4;  // BWD_DW tile order: 4 M tiles per group
constexpr int kDwPartsPerNTile = 4;  // partial router-weight gradients per N tile (one per wave column)
constexpr uint32_t kOff = 0x80000000u;  // offset past every resource: loads return 0
// Short tiles (at most SHORT_ROWS valid rows: an expert's ragged last tile)
// run their K loop on a ring of three compact stages, A SHORT_ROWS rows then
// B BN rows each (and their MXFP8 scale dwords), so that two steps are in
// flight instead of one.
constexpr int SHORT_ROWS = 64;
constexpr int SHORT_SLOT = (SHORT_ROWS + BN) * ROWB;  // 40 KiB
constexpr int SHORT_SSLOT = (SHORT_ROWS + BN) * 4;    // 1280 bytes of scales
static_assert(3 * SHORT_SLOT <= NSTAGE * (A_BYTES + B_BYTES), "three short stages fit the two full ones");
static_assert(3 * SHORT_SSLOT <= NSTAGE * (SA_BYTES + SB_BYTES), "and their scales the two full ones'");

enum Mode : int {
  GATE_UP = 0,  // A = tokens of x, B = gate | up rows, epilogue h = silu(g) * u
  DOWN = 1,     // A = h rows, B = down rows, epilogue y = w * acc
  BWD_DH = 2,   // A = tokens of grad_out, B = rows of down^T, epilogue dG, dU, w*h, partial dw
  BWD_DX = 3,   // A = [dG | dU] rows, B = rows of [gate^T | up^T], epilogue dA rows
  BWD_DW = 4    // per expert, K = its rows: dW_down = dY^T h, dW_gate = dG^T X, dW_up = dU^T X, the
                // operands stored transposed, [cols, K_e] (bf16, or MXFP8 quantized in 32-row blocks)
};

struct Params {
  // schedule
  const int32_t* hdr;
  const int32_t* offsets;
  const int32_t* kept;
  const int32_t* tiles;    // prefix sums of 256-row tiles per expert; [E] routed total, [E+1] with shared
  const int32_t* row_src;
  const int32_t* mb_offsets;    // per (minibatch, expert) first rows, [(n_mb + 1) * E]
  int mb;                       // DOWN: tokens per minibatch of the pipeline (0 = no pipeline: one pass over every row)
  // DOWN minibatch pipeline (mb > 0): the last n_movers workgroups combine
  // minibatch b once mb_done[b] counts all of its tiles, while the others
  // run the tiles of later minibatches
  int32_t* mb_done;             // per-minibatch finished-tile counters (zeroed by the gate/up launch)
  int n_done;                   // GATE_UP: how many counters it zeroes
  int32_t* status;              // [0]: a mover's wait that ran out of time adds 1; [1]: schedule mismatches
  int cfg_hash;                 // the configuration hash the schedule's header must carry
  int n_movers;
  const int32_t* slot_row;      // [T*k] the row of each assignment (combine)
  uint16_t* comb_out;           // the layer output [T, H] bf16 (combine)
  int E, k, H, I, Is;
  int64_t rows_cap_max;
  // SwiGLU input limit L: h = silu(min(g, L)) * clamp(u, -L, L); +inf = none
  float swiglu_lim;
  // A operand
  const void* a_tok;            // token-indexed rows [T, K] (x, x codes, grad_out)
  const uint8_t* a_tok_scale;   // their E8M0 scales [T, K/32]
  const void* a_row;            // schedule-row-indexed rows: routed [rows_cap_max, K], shared after it
  const uint8_t* a_row_scale;
  const void* a_row2;           // second half of K (dU) for BWD_DX
  const uint8_t* a_row2_scale;
  // B operand: routed [E, N, K] and shared [N, K]; b1 = up (GATE_UP) or up^T (BWD_DX)
  const void *b0, *b1, *sb0, *sb1;
  const uint8_t *b0s, *b1s, *sb0s, *sb1s;
  const float* router_w;
  // outputs (row layouts as a_row: routed rows, then shared rows at rows_cap_max)
  void* out;                    // h (GATE_UP), y (DOWN), dA (BWD_DX)
  uint8_t* out_scale;           // h scales (GATE_UP, MXFP8)
  void* ctx_g;                  // G, U saved for backward (GATE_UP): bf16, fp32 in MXFP8 mode
  void* ctx_u;
  // BWD_DH epilogue
  const void* g_in;             // the saved G, U: bf16, fp32 in MXFP8 mode
  const void* u_in;
  const uint16_t* h_in;
  uint16_t* dg_out;
  uint16_t* du_out;
  // MXFP8: dG and dU quantized in the epilogue, along I (row-major codes
  // and scales, the layout of the forward's h codes: the dA GEMM's A
  // operands) and along rows (p.tq.dg/dgs, p.tq.du/dus: the weight
  // gradients' operands, [cols, K_e] per expert at 128 * tiles128[e] * I)
  uint8_t* rq_g;
  uint8_t* rq_gs;
  uint8_t* rq_u;
  uint8_t* rq_us;
  const int32_t* tiles128;      // prefix sums of 128-row tiles per expert, [E] routed, [E+1] with shared
  uint16_t* hw_out;
  const uint8_t* hq_in;         // MXFP8: h codes and scales saved by the forward (instead of h_in)
  const uint8_t* hq_scale_in;
  float* dw_part;               // [rows_cap_max + T_max, dw_parts]
  int dw_parts;
  // BWD_DW
  TqArrays tq;
  uint16_t* d_wd;               // routed weight gradients [E, H, I], [E, I, H], [E, I, H]
  uint16_t* d_wg;
  uint16_t* d_wu;
  uint16_t* d_sd;               // shared [H, I_s], [I_s, H], [I_s, H]
  uint16_t* d_sg;
  uint16_t* d_su;
};

struct Tile {
  int e;      // expert, -1 = shared expert
  int m0;     // first row (schedule row, or token for the shared expert)
  int m_end;  // one past the last valid row
  int nt;     // N tile
  int job;    // BWD_DW: 0 = dW_down, 1 = dW_gate, 2 = dW_up
  int kdim;   // BWD_DW: the expert's K (rows, a multiple of 128)
  int kofs;   // BWD_DW: the expert's K offset in the transposed arrays
};

// LDS past the stages that the MXFP8 dh_hat epilogue stages through with
// them (two padded 32 x 64 fp32 buffers per wave)
constexpr int kEpiExtra = NTHR / 64 * 2 * 32 * (64 + 4) * 4 - NSTAGE * (A_BYTES + B_BYTES);

struct alignas(16) Lds {
  uint8_t stage[NSTAGE][A_BYTES + B_BYTES];
  uint8_t epi_extra[kEpiExtra];  // (contiguous with the stages)
  uint8_t scale[NSTAGE][SA_BYTES + SB_BYTES];  // used in MXFP8 mode
  int32_t tiles[kMaxLdsE + 2];
  int32_t fullp[kMaxLdsE + 2];  // exclusive prefix over experts (shared last) of full M tiles
  int32_t tailp[kMaxLdsE + 2];  // ... and of tail M tiles (a segment's last tile with <= 128 rows)
  int32_t offs[kMaxLdsE];       // per expert: first row and row count of this launch's segment
  int32_t keptl[kMaxLdsE];
  int32_t wsum[2][NTHR / 64];   // per-wave partial sums of the two scans
  int32_t row_src[BM];  // per tile row: source row (token, or tile-local row), -1 = none
  float row_w[BM];      // per tile row: router weight (1 for the shared expert)
};

// SiLU and the logistic function with the hardware reciprocal (1 ulp): the
// results are rounded to bf16 or E4M3 right after.
__device__ __forceinline__ float sigmoid_f(float g) { return __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }
__device__ __forceinline__ float silu_f(float g) { return g * sigmoid_f(g); }
// SwiGLU with its inputs limited: the gate from above at L, the up
// projection to [-L, L] (L = +inf leaves both unchanged).
__device__ __forceinline__ float swiglu_f(float g, float u, float L) {
  return silu_f(__builtin_fminf(g, L)) * __builtin_fminf(__builtin_fmaxf(u, -L), L);
}
// G and U as saved for the backward: an input that the limit clamped is
// saved as +-inf, so the backward knows the forward's clamp decision exactly
// (a bf16-rounded value near L would not tell), and reads the clamped value
// back as min(g, L), clamp(u, -L, L).
__device__ __forceinline__ float saved_gate(float g, float L) { return g > L ? __builtin_inff() : g; }
__device__ __forceinline__ float saved_up(float u, float L) {
  return u > L ? __builtin_inff() : (u < -L ? -__builtin_inff() : u);
}

template <int MODE>
__device__ __forceinline__ int n_tile_width() {
  return MODE == GATE_UP ? 128 : BN;  // GATE_UP tiles pair 128 gate rows with the 128 matching up rows
}

template <int MODE>
__device__ __forceinline__ int k_of(const Params& p, bool shared) {
  const int Iv = shared ? p.Is : p.I;
  return MODE == GATE_UP ? p.H : MODE == DOWN ? Iv : MODE == BWD_DH ? p.H : 2 * Iv;
}

template <int MODE>
__device__ __forceinline__ int n_of(const Params& p, bool shared) {
  const int Iv = shared ? p.Is : p.I;
  return (MODE == GATE_UP || MODE == BWD_DH) ? Iv : p.H;
}

// Down tiles of minibatch b of the pipeline: per expert, its rows of
// tokens in [b mb, (b + 1) mb) in 256-row tiles, times the N tiles; plus the
// shared expert's rows of those tokens. Every thread of the workgroup gets
// the total (a workgroup reduction through L.wsum).
__device__ __forceinline__ int pipe_tiles_of(const Params& p, Lds& L, int b, int T) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = p.E, nt = (p.H + BN - 1) / BN;  // down's N tiles: the same for routed and shared rows
  int cnt = 0;
  for (int e = tid; e < E; e += NTHR)
    cnt += (p.mb_offsets[(b + 1) * E + e] - p.mb_offsets[b * E + e] + BM - 1) / BM * nt;
  if (tid == 0 && p.Is > 0) {
    const int t0 = min(T, b * p.mb), t1 = min(T, t0 + p.mb);
    cnt += (t1 - t0 + BM - 1) / BM * nt;
  }
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) cnt += __shfl_xor(cnt, d);
  __syncthreads();  // L.wsum is free (a previous read has completed)
  if (lane == 0) L.wsum[0][wave] = cnt;
  __syncthreads();
  int total = 0;
#pragma unroll
  for (int w = 0; w < NTHR / 64; ++w) total += L.wsum[0][w];
  return total;
}

// A mover workgroup of the down GEMM's minibatch pipeline. For each
// minibatch b in order: wait (bounded) until the compute workgroups have
// counted all of b's down tiles in mb_done[b], then combine b's tokens:
// out[t] = bf16(sum over j in slot order of y[slot_row[t, j]], then + the
// shared row), fp32 adds, as the stand-alone combine does, so the bits do
// not depend on the split. The y rows come from other XCDs' L2s: they were
// stored, and are loaded here, at agent scope (sc1), and a tile is counted
// only after all of its stores completed. A wait that runs out of time adds
// 1 to status[0] and gives up on the remaining waits (the kernel always
// ends; the host reads the flag).
__device__ __forceinline__ void pipe_mover(const Params& p, Lds& L, int T) {
  constexpr int kSleepsPerWait = 1 << 20;   // s_sleep 64 (~2 us each): about 2 s in all
  const int tid = threadIdx.x;
  const int n_mb = p.hdr[HDR_NMB];
  const int mover = (int)blockIdx.x - ((int)gridDim.x - p.n_movers);
  const int H = p.H, k = p.k, nchunk = H / 8;
  const uint16_t* y = (const uint16_t*)p.out;
  const uint16_t* ys = p.Is > 0 ? y + p.rows_cap_max * (int64_t)H : nullptr;
  int budget = kSleepsPerWait;  // shared by every wait of this workgroup (thread 0's copy counts)
  for (int b = 0; b < n_mb; ++b) {
    const int target = pipe_tiles_of(p, L, b, T);
    if (tid == 0) {
      int seen = __hip_atomic_load(p.mb_done + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      while (seen < target && budget > 0) {
        __builtin_amdgcn_s_sleep(64);
        --budget;
        seen = __hip_atomic_load(p.mb_done + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      if (seen < target) {
        budget = 0;
        __hip_atomic_fetch_add(p.status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __syncthreads();  // the wait is over for every thread; no load below moves above it
    asm volatile("" ::: "memory");
    const int t0 = min(T, b * p.mb), t1 = min(T, t0 + p.mb);
    // two tokens at a time (one per half workgroup), 16 bytes of a row per thread
    for (int t = t0 + 2 * mover + (tid >> 8); t < t1; t += 2 * p.n_movers) {
      const int32_t* sl = p.slot_row + (int64_t)t * k;
      for (int c = tid & 255; c < nchunk; c += 256) {
        float acc[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = 0.f;
        auto add = [&](uint64_t lo, uint64_t hi) {
          const uint32_t w[4] = {(uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32)};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc[2 * q] += u2f(w[q] << 16);
            acc[2 * q + 1] += u2f(w[q] & 0xFFFF0000u);
          }
        };
        for (int j0 = 0; j0 < k; j0 += 8) {
          int row[8];
          uint64_t lo[8], hi[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            row[u] = j0 + u < k ? sl[j0 + u] : -1;
            lo[u] = hi[u] = 0;
            if (row[u] >= 0) {
              const uint64_t* src = reinterpret_cast<const uint64_t*>(y + (int64_t)row[u] * H + c * 8);
              lo[u] = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              hi[u] = __hip_atomic_load(src + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
          }
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (row[u] >= 0) add(lo[u], hi[u]);
        }
        if (ys) {
          const uint64_t* src = reinterpret_cast<const uint64_t*>(ys + (int64_t)t * H + c * 8);
          add(__hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
              __hip_atomic_load(src + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        }
        u32x4 o;
        o[0] = pack_bf16x2(acc[0], acc[1]);
        o[1] = pack_bf16x2(acc[2], acc[3]);
        o[2] = pack_bf16x2(acc[4], acc[5]);
        o[3] = pack_bf16x2(acc[6], acc[7]);
        *reinterpret_cast<u32x4*>(p.comb_out + (int64_t)t * H + c * 8) = o;
      }
    }
  }
}

// PIPE (MODE == DOWN only): the minibatch pipeline, movers included.
template <int MODE, bool FP8, bool PIPE = false>
__global__ void __launch_bounds__(NTHR) __attribute__((amdgpu_waves_per_eu(2, 2)))
grouped_gemm_nt(Params p) {
  static_assert(!PIPE || MODE == DOWN, "the pipeline is the down GEMM's");
  __shared__ Lds L;
  constexpr int ES = FP8 ? 1 : 2;           // element size in bytes
  constexpr int KS = ROWB / ES;             // K elements per step
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int lr = lane & 31, lh = lane >> 5;
  const int E = p.E;

  if (!sched_matches(p.hdr, p.cfg_hash, p.status)) return;  // before any barrier: the whole grid returns
  const bool lds_tiles = E <= kMaxLdsE;
  if (lds_tiles) {
    for (int i = tid; i < E + 2; i += NTHR) L.tiles[i] = p.tiles[i];
    for (int i = tid; i < E; i += NTHR) {
      L.offs[i] = p.offsets[i];
      L.keptl[i] = p.kept[i];
    }
  }
  const int T = p.hdr[HDR_T];
  if (MODE == GATE_UP && p.mb_done && blockIdx.x == 0)  // for the pipelined down launch that follows
    for (int i = tid; i < p.n_done; i += NTHR) p.mb_done[i] = 0;
  __syncthreads();
  // the down GEMM's minibatch pipeline (one launch): movers combine, the
  // other workgroups run the tiles minibatch by minibatch
  constexpr bool pipe = PIPE;
  if (pipe && (int)blockIdx.x >= (int)gridDim.x - p.n_movers) {
    pipe_mover(p, L, T);
    return;
  }
  const int n_pass = pipe ? p.hdr[HDR_NMB] : 1;  // (1 at compile time without the pipeline)
  for (int pass = 0; pass < n_pass; ++pass) {
  // shared-expert rows of this pass: every token, or one minibatch's tokens
  int sh0 = 0, sh1 = T;
  if (pipe) {
    // minibatch b = pass: only its rows, expert e's being rows
    // [mb_offsets[b][e], mb_offsets[b+1][e]) of its segment. The tile table
    // of these row ranges is built here (the launcher keeps E <= kMaxLdsE).
    const int b = pass;
    sh0 = min(T, b * p.mb);
    sh1 = min(T, sh0 + p.mb);
    int cnt = 0;
    __syncthreads();  // the previous pass's tables are no longer read
    if (tid < E) {
      const int lo = p.mb_offsets[b * E + tid];
      const int hi = p.mb_offsets[(b + 1) * E + tid];
      L.offs[tid] = lo;
      L.keptl[tid] = hi - lo;
      cnt = (hi - lo + BM - 1) / BM;
    } else if (tid == E) {
      cnt = p.Is > 0 ? (sh1 - sh0 + BM - 1) / BM : 0;
    }
    int sc = cnt;
#pragma unroll
    for (int dd = 1; dd < 64; dd <<= 1) {
      const int av = __shfl_up(sc, dd);
      if (lane >= dd) sc += av;
    }
    if (lane == 63) L.wsum[0][wave] = sc;
    __syncthreads();
    int bs = 0;
    for (int w = 0; w < wave; ++w) bs += L.wsum[0][w];
    if (tid <= E + 1) L.tiles[tid] = bs + sc - cnt;  // exclusive prefix; [E + 1] = total with the shared expert
    __syncthreads();
  }
  auto tile_at = [&](int e) { return lds_tiles ? L.tiles[e] : p.tiles[e]; };
  auto offset_at = [&](int e) { return lds_tiles ? L.offs[e] : p.offsets[e]; };
  auto kept_at = [&](int e) { return lds_tiles ? L.keptl[e] : p.kept[e]; };
  const int n_routed_mt = tile_at(E);
  const int n_all_mt = tile_at(E + 1);
  const int ntw = n_tile_width<MODE>();
  const int nt_r = (n_of<MODE>(p, false) + ntw - 1) / ntw;
  const int nt_s = p.Is > 0 ? (n_of<MODE>(p, true) + ntw - 1) / ntw : 1;
  // BWD_DW: per expert (the shared expert first) 3 jobs of tpj 256 x 256 tiles
  const int hb = (p.H + BM - 1) / BM;
  const int tpj_r = hb * ((p.I + BN - 1) / BN);
  const int tpj_s = hb * ((p.Is + BN - 1) / BN);
  const int ntiles = MODE == BWD_DW ? E * 3 * tpj_r + (p.Is > 0 ? 3 * tpj_s : 0)
                                    : n_routed_mt * nt_r + (n_all_mt - n_routed_mt) * nt_s;

  // ---- work lists ----
  // Workgroup b runs on XCD b % 8 and works through that XCD's list of
  // tiles, taking positions slot, slot + slots, ... (slot = b / 8), so the
  // tiles of one expert, which share its weights, run together on one XCD and
  // hit its L2. The modes whose A rows are gathered tokens (gate/up and the
  // backward's grad_out GEMM) order each list longest first: the XCD's share
  // of the full M tiles (more than 128 valid rows), then its share of the
  // tail tiles (a segment's last M tile, at most 128 rows, whose MFMAs the
  // idle wave half skips), which then fill the last round. The other modes
  // keep the natural order (an expert's tiles together, its tail tile right
  // after its full ones), which reads each expert's weights once.
  const int ncomp = (int)gridDim.x - (pipe ? p.n_movers : 0);  // compute workgroups (the movers are the last)
  const int nq = (ncomp % kNumXcd) == 0 ? kNumXcd : 1;
  const int xq = blockIdx.x % nq;
  const int slot = blockIdx.x / nq, slots = ncomp / nq;
  // experts with at least kGroupM M tiles on average
  const bool deep = n_routed_mt >= kGroupM * E;
  // longest-first lists: always for gate/up and dh; for down (not in a
  // minibatch launch, whose rows are a minibatch's share) and dA when
  // experts are deep, where the ragged tail tiles otherwise end the kernel
  // unevenly (at shallow experts the natural order measured faster for them)
  const bool lpt = lds_tiles && (MODE == GATE_UP || MODE == BWD_DH ||
                                 (deep && (MODE == BWD_DX || (MODE == DOWN && !pipe))));
  int TFr = 0, TF = 0, TTr = 0, TT = 0, f0 = 0, nf = 0, u0 = 0, qlen = 0, id0 = 0;
  if (lpt) {
    // counts of full and tail M tiles per expert (index E = shared expert),
    // exclusive scans across the workgroup (waves scan with shuffles)
    int cf = 0, ct = 0;
    if (tid <= E) {
      const int nm = L.tiles[tid + 1] - L.tiles[tid];
      const int rows = tid < E ? p.kept[tid] : (p.Is > 0 ? T : 0);
      const int tail = (nm > 0 && rows - BM * (nm - 1) <= BM / 2) ? 1 : 0;
      cf = nm - tail;
      ct = tail;
    }
    int sf = cf, st = ct;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int af = __shfl_up(sf, d), at = __shfl_up(st, d);
      if (lane >= d) {
        sf += af;
        st += at;
      }
    }
    if (lane == 63) {
      L.wsum[0][wave] = sf;
      L.wsum[1][wave] = st;
    }
    __syncthreads();
    int bf = 0, bt = 0;
    for (int w = 0; w < wave; ++w) {
      bf += L.wsum[0][w];
      bt += L.wsum[1][w];
    }
    if (tid <= E + 1) {
      L.fullp[tid] = bf + sf - cf;  // exclusive
      L.tailp[tid] = bt + st - ct;
    }
    __syncthreads();
    TFr = L.fullp[E] * nt_r;
    TF = TFr + (L.fullp[E + 1] - L.fullp[E]) * nt_s;
    TTr = L.tailp[E] * nt_r;
    TT = TTr + (L.tailp[E + 1] - L.tailp[E]) * nt_s;
    const int cfq = (TF + nq - 1) / nq, ctq = (TT + nq - 1) / nq;
    f0 = min(TF, xq * cfq);
    nf = min(TF, f0 + cfq) - f0;
    u0 = min(TT, xq * ctq);
    qlen = nf + min(TT, u0 + ctq) - u0;
  } else if (MODE == BWD_DW) {
    // A weight-gradient tile's work is its K: its expert's rows (the shared
    // expert's are every token, several times a routed expert's). Ids run
    // over the shared expert's tiles first (the longest ones start first),
    // then the routed experts'; XCD xq takes the ids whose work starts in
    // [xq W / nq, (xq + 1) W / nq), W = the total work, in 128-row blocks.
    const int64_t units_r = 3LL * tpj_r;                 // tiles per routed expert
    const int64_t sh_tiles = p.Is > 0 ? 3LL * tpj_s : 0;
    const int64_t ks = tile_at(E + 1) - tile_at(E);     // the shared expert's K blocks
    const int64_t Wsh = sh_tiles * ks;
    const int64_t W = Wsh + units_r * tile_at(E);
    // smallest id whose work starts at or after wpos (ntiles if none)
    auto first_id = [&](int64_t wpos) -> int {
      if (wpos <= 0) return 0;
      if (wpos <= Wsh - ks) return (int)((wpos + ks - 1) / ks);  // a shared tile (ks > 0 here)
      const int64_t wr = wpos - Wsh;
      // routed expert e's last tile starts at units_r * tiles[e + 1] - kd(e),
      // which does not decrease with e: the first e where that is >= wr
      int lo = 0, hi = E;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        const int64_t kd = tile_at(mid + 1) - tile_at(mid);
        if (units_r * tile_at(mid + 1) - kd >= wr)
          hi = mid;
        else
          lo = mid + 1;
      }
      if (lo >= E) return ntiles;
      const int64_t kd = tile_at(lo + 1) - tile_at(lo);
      const int64_t rel = wr - units_r * tile_at(lo);
      const int64_t local = (kd == 0 || rel <= 0) ? 0 : (rel + kd - 1) / kd;
      return (int)(sh_tiles + lo * units_r + local);
    };
    id0 = first_id(W * xq / nq);
    qlen = (xq == nq - 1 ? ntiles : first_id(W * (xq + 1) / nq)) - id0;
  } else {
    const int chunk = (ntiles + nq - 1) / nq;
    id0 = min(ntiles, xq * chunk);
    qlen = min(ntiles, id0 + chunk) - id0;
  }
  auto search = [&](const int32_t* pre, int v) {  // largest e in [0, E) with pre[e] <= v
    int lo = 0, hi = E;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (pre[mid] <= v)
        lo = mid;
      else
        hi = mid;
    }
    return lo;
  };

  // When experts have many M tiles (at least kGroupM on average), tiles go
  // in runs of kGroupM M tiles x all N tiles, M fastest: the tiles in flight
  // together on one XCD share both operands' rows in its L2 (N fastest
  // streams each weight N-tile once per M tile). With few M tiles per expert
  // an XCD's round already spans whole experts and the natural order (N
  // fastest) measured faster; the grad-out GEMM keeps it too (slower
  // grouped at 32768 tokens). The weight gradients are always grouped.
  const bool grp_order = MODE == BWD_DW || (MODE != BWD_DH && deep);
  auto grouped = [&](int v, int n_m, int n_n, int& mi, int& ni) {
    if (!grp_order) {
      mi = v / n_n;
      ni = v - mi * n_n;
      return;
    }
    const int grp = v / (kGroupM * n_n);
    const int base = grp * kGroupM;
    const int gm = min(kGroupM, n_m - base);
    const int r = v - grp * kGroupM * n_n;
    mi = base + r % gm;
    ni = r / gm;
  };

  // Gate/up's and dh's lists are longest first and end with their cheapest
  // tiles, so after the complete rounds the last slots are the least loaded
  // (they took tail tiles earliest): the last, partial round goes to them,
  // slot slots - 1 first. BF16 only: in MXFP8 the extra index arithmetic
  // cost more than the balance gained (gate/up measured slower), and other
  // modes keep plain round-robin.
  constexpr bool kRevLast = !FP8 && (MODE == GATE_UP || MODE == BWD_DH);
  const int q_base = kRevLast ? qlen / slots * slots : 0;  // first position of the partial round
  const int q_stop = kRevLast && lpt ? q_base + (slot >= slots - (qlen - q_base) ? slots : 0) : qlen;
  for (int q0 = slot; q0 < q_stop; q0 += slots) {
    const int q = (kRevLast && lpt && q0 >= q_base) ? q_base + slots - 1 - slot : q0;
    // ---- decode the tile ----
    Tile t;
    const int id = id0 + q;  // natural-order id (BWD_DW, or more experts than the LDS tables hold)
    if (lpt) {
      const bool full = q < nf;
      const int v = full ? f0 + q : u0 + (q - nf);
      const int vr = full ? TFr : TTr;
      if (v < vr) {
        int mi, ni;
        grouped(v, full ? L.fullp[E] : L.tailp[E], nt_r, mi, ni);
        t.nt = ni;
        const int e = __builtin_amdgcn_readfirstlane(search(full ? L.fullp : L.tailp, mi));
        t.e = e;
        const int base = offset_at(e);
        const int mt = full ? mi - L.fullp[e] : L.tiles[e + 1] - L.tiles[e] - 1;
        t.m0 = base + mt * BM;
        t.m_end = base + kept_at(e);
      } else {
        int mi, ni;
        grouped(v - vr, full ? L.fullp[E + 1] - L.fullp[E] : L.tailp[E + 1] - L.tailp[E], nt_s, mi, ni);
        t.nt = ni;
        t.e = -1;
        t.m0 = sh0 + (full ? mi : L.tiles[E + 1] - L.tiles[E] - 1) * BM;
        t.m_end = sh1;
      }
      t.m0 = __builtin_amdgcn_readfirstlane(t.m0);
      t.m_end = __builtin_amdgcn_readfirstlane(t.m_end);
      t.nt = __builtin_amdgcn_readfirstlane(t.nt);
    } else if constexpr (MODE == BWD_DW) {
      const int n_shared = p.Is > 0 ? 3 * tpj_s : 0;  // the shared expert's tiles come first
      const bool sh = id < n_shared;
      const int tpj = sh ? tpj_s : tpj_r;
      const int rem0 = sh ? id : (id - n_shared) % (3 * tpj_r);
      t.e = sh ? -1 : (id - n_shared) / (3 * tpj_r);
      t.job = rem0 / tpj;
      const int tt = rem0 - t.job * tpj;
      const int Ivt = sh ? p.Is : p.I;
      const int nn = t.job == 0 ? (Ivt + BN - 1) / BN : hb;  // N tiles of the job
      const int nm = t.job == 0 ? hb : (Ivt + BM - 1) / BM;  // M tiles of the job
      int mt, ni;
      grouped(tt, nm, nn, mt, ni);
      t.nt = ni;
      t.m0 = mt * BM;
      t.m_end = t.job == 0 ? p.H : Ivt;
      const int k0t = sh ? tile_at(E) : tile_at(t.e);
      const int k1t = sh ? tile_at(E + 1) : tile_at(t.e + 1);
      t.kdim = 128 * (k1t - k0t);
      t.kofs = sh ? 0 : 128 * k0t;
      t.e = __builtin_amdgcn_readfirstlane(t.e);
      t.job = __builtin_amdgcn_readfirstlane(t.job);
      t.m0 = __builtin_amdgcn_readfirstlane(t.m0);
      t.m_end = __builtin_amdgcn_readfirstlane(t.m_end);
      t.nt = __builtin_amdgcn_readfirstlane(t.nt);
      t.kdim = __builtin_amdgcn_readfirstlane(t.kdim);
      t.kofs = __builtin_amdgcn_readfirstlane(t.kofs);
    } else {
      const int n_routed = n_routed_mt * nt_r;
      if (id < n_routed) {
        int mt, ni;
        grouped(id, n_routed_mt, nt_r, mt, ni);
        t.nt = ni;
        int lo = 0, hi = E;  // largest e with tiles[e] <= mt
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (tile_at(mid) <= mt)
            lo = mid;
          else
            hi = mid;
        }
        t.e = __builtin_amdgcn_readfirstlane(lo);
        const int base = offset_at(t.e);
        t.m0 = base + (mt - tile_at(t.e)) * BM;
        t.m_end = base + kept_at(t.e);
      } else {
        int mt, ni;
        grouped(id - n_routed, n_all_mt - n_routed_mt, nt_s, mt, ni);
        t.nt = ni;
        t.e = -1;
        t.m0 = sh0 + mt * BM;
        t.m_end = sh1;
      }
      t.m0 = __builtin_amdgcn_readfirstlane(t.m0);
      t.m_end = __builtin_amdgcn_readfirstlane(t.m_end);
      t.nt = __builtin_amdgcn_readfirstlane(t.nt);
    }
    const bool shared = t.e < 0;
    const int Iv = shared ? p.Is : p.I;
    const int K = MODE == BWD_DW ? t.kdim : k_of<MODE>(p, shared);
    const int Nd = MODE == BWD_DW ? (t.job == 0 ? Iv : p.H) : n_of<MODE>(p, shared);  // valid output columns
    const int rows_here = t.m_end - t.m0;
    // a tile without a valid row (the schedule counts tiles from kept rows,
    // so none is listed; kept as a guard) would turn the byte counts of its
    // buffer resources negative: skip it, the same decision in every wave
    if (rows_here <= 0) {
      if (pipe && tid == 0) __hip_atomic_fetch_add(p.mb_done + pass, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      continue;
    }
    // 32-row MFMA blocks of this wave's 128 rows that hold valid rows
    // (uniform across the wave): 4 except in a segment's last tile
    const int live_blocks = min(4, max(0, (rows_here - wm * 128 + 31) / 32));

    // ---- row metadata, one thread per tile row ----
    // Down's A rows are tile-local, so its loads do not need this table: its
    // router weights are read while the first K step is in flight (below).
    constexpr bool kLateMeta = MODE == DOWN;
    if (!kLateMeta && tid < BM) {
      const int r = t.m0 + tid;
      int src = -1;
      float w = 0.f;
      if (r < t.m_end) {
        if (MODE == BWD_DW) {
          src = tid;  // tile-local row of the transposed operand
        } else if (shared) {
          src = (MODE == GATE_UP || MODE == BWD_DH) ? r : tid;
          w = 1.f;
        } else {
          const int a = p.row_src[r];
          src = (MODE == GATE_UP || MODE == BWD_DH) ? a / p.k : tid;  // token, or tile-local row
          if (MODE == DOWN || MODE == BWD_DH) w = p.router_w[a];
        }
      }
      L.row_src[tid] = src;
      L.row_w[tid] = w;
    }
    if constexpr (!kLateMeta) __syncthreads();

    // ---- operand resources and per-lane DMA offsets ----
    const bool a_by_token = MODE == GATE_UP || MODE == BWD_DH;
    const int a_k = MODE == BWD_DX ? Iv : K;  // row length of the A array(s)
    const uint8_t* a_base;
    const uint8_t* a_base2 = nullptr;
    uint32_t a_bytes;
    // BWD_DW: the job's transposed arrays (A = [M, K_e], B = [N, K_e]) and
    // the routed column count that places the shared expert's blocks
    const uint8_t *dw_a = nullptr, *dw_as = nullptr, *dw_b = nullptr, *dw_bs = nullptr;
    int64_t dw_a_blk = 0, dw_as_blk = 0, dw_b_blk = 0, dw_bs_blk = 0;
    if constexpr (MODE == BWD_DW) {
      const int Mc = t.m_end;  // M columns of the job's A array
      const int colsA_r = t.job == 0 ? p.H : p.I, colsB_r = t.job == 0 ? p.I : p.H;
      dw_a = t.job == 0 ? p.tq.dy : t.job == 1 ? p.tq.dg : p.tq.du;
      dw_as = t.job == 0 ? p.tq.dys : t.job == 1 ? p.tq.dgs : p.tq.dus;  // MXFP8 only
      dw_b = t.job == 0 ? p.tq.h : p.tq.x;
      dw_bs = t.job == 0 ? p.tq.hs : p.tq.xs;
      dw_a_blk = shared ? p.tq.kr_cap * colsA_r : (int64_t)t.kofs * Mc;
      dw_as_blk = shared ? p.tq.kr_cap / 32 * colsA_r : (int64_t)(t.kofs / 32) * Mc;
      dw_b_blk = shared ? p.tq.kr_cap * colsB_r : (int64_t)t.kofs * Nd;
      dw_bs_blk = shared ? p.tq.kr_cap / 32 * colsB_r : (int64_t)(t.kofs / 32) * Nd;
      a_base = dw_a + (dw_a_blk + (int64_t)t.m0 * K) * ES;
      a_bytes = (uint32_t)((int64_t)rows_here * K * ES);
    } else if (a_by_token) {
      a_base = (const uint8_t*)p.a_tok;
      a_bytes = (uint32_t)((int64_t)T * K * ES);
    } else {
      // based at the tile's first row (rows are tile-local), so the buffer
      // ranges stay small whatever the total row count
      const int64_t off0 = (shared ? p.rows_cap_max * p.I * ES : 0) + (int64_t)t.m0 * a_k * ES;
      a_base = (const uint8_t*)p.a_row + off0;
      if (MODE == BWD_DX) a_base2 = (const uint8_t*)p.a_row2 + off0;
      a_bytes = (uint32_t)((int64_t)rows_here * a_k * ES);
    }
    const i32x4v rs_a = rsrc(a_base, a_bytes);
    const i32x4v rs_a2 = rsrc(MODE == BWD_DX ? a_base2 : a_base, a_bytes);
    // B: GATE_UP waves 0-3 load the 128 gate rows, waves 4-7 the matching up rows.
    const uint8_t *b_base, *b_base2 = nullptr;
    uint32_t b_bytes;
    const int b_k = MODE == BWD_DX ? Iv : K;
    if constexpr (MODE == BWD_DW) {
      b_base = dw_b + dw_b_blk * ES;
      b_bytes = (uint32_t)((int64_t)Nd * K * ES);
    } else {
      const int64_t estride = (int64_t)Nd * b_k * ES;
      const void* r0 = (MODE == GATE_UP && wave >= 4) ? p.b1 : p.b0;
      const void* s0 = (MODE == GATE_UP && wave >= 4) ? p.sb1 : p.sb0;
      b_base = shared ? (const uint8_t*)s0 : (const uint8_t*)r0 + (int64_t)t.e * estride;
      if (MODE == BWD_DX) b_base2 = shared ? (const uint8_t*)p.sb1 : (const uint8_t*)p.b1 + (int64_t)t.e * estride;
      b_bytes = (uint32_t)estride;
    }
    const i32x4v rs_b = rsrc(b_base, b_bytes);
    const i32x4v rs_b2 = rsrc(MODE == BWD_DX ? b_base2 : b_base, b_bytes);

    // This wave's LDS-DMA rows (one 16-byte instruction = 8 rows of 128
    // bytes): A and B rows 32*wave + 8*i + lane/8 (i < 4); lane % 8 is the
    // physical 16-byte chunk, which holds logical chunk (lane % 8) ^ swz.
    const int dr = lane >> 3, dp = lane & 7;
    const uint32_t a_row_bytes = (uint32_t)a_k * ES;
    uint32_t a_off[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 32 * wave + 8 * i + dr;
      const int src = kLateMeta ? (row < rows_here ? row : -1) : L.row_src[row];
      a_off[i] = src >= 0 ? (uint32_t)src * a_row_bytes + 16u * (uint32_t)(dp ^ swz(row)) : kOff;
    }
    const uint32_t b_row_bytes = (uint32_t)b_k * ES;
    uint32_t b_off[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int lb = 32 * wave + 8 * i + dr;
      const int n = MODE == GATE_UP ? t.nt * 128 + (lb & 127) : t.nt * BN + lb;
      b_off[i] = n < Nd ? (uint32_t)n * b_row_bytes + 16u * (uint32_t)(dp ^ swz(lb)) : kOff;
    }
    // MXFP8 scales: one dword per row holds the E8M0 scales of the step's 4
    // blocks of 32. Waves 0-3 load A rows 64*wave + lane, waves 4-7 load B
    // rows 64*(wave-4) + lane (GATE_UP: waves 4-5 gate rows, 6-7 up rows).
    // BWD_DX: the dG / gate^T scales serve the first half of K, the dU / up^T
    // scales (rs_s2) the second; each has Iv / 32 scale bytes per row.
    i32x4v rs_s = rs_a, rs_s2 = rs_a;
    uint32_t s_off = kOff;
    if (FP8) {
      const int kb = (MODE == BWD_DX ? Iv : K) / 32;
      if (wave < 4) {
        const uint8_t* sa_base;
        const uint8_t* sa_base2 = nullptr;
        uint32_t sa_bytes = (uint32_t)(rows_here * kb);
        if (MODE == BWD_DW) {
          sa_base = dw_as + dw_as_blk + (int64_t)t.m0 * kb;
        } else if (a_by_token) {
          sa_base = p.a_tok_scale;
          sa_bytes = (uint32_t)T * kb;
        } else {
          const int64_t so = (shared ? p.rows_cap_max * (p.I / 32) : 0) + (int64_t)t.m0 * kb;
          sa_base = p.a_row_scale + so;
          if (MODE == BWD_DX) sa_base2 = p.a_row2_scale + so;
        }
        rs_s = rsrc(sa_base, sa_bytes);
        rs_s2 = rsrc(MODE == BWD_DX ? sa_base2 : sa_base, sa_bytes);
        const int src = kLateMeta ? (64 * wave + lane < rows_here ? 64 * wave + lane : -1) : L.row_src[64 * wave + lane];
        if (src >= 0) s_off = (uint32_t)src * kb;
      } else {
        const int lb = 64 * (wave - 4) + lane;
        const bool up = MODE == GATE_UP && wave >= 6;
        const uint8_t* bsb;
        const uint8_t* bsb2 = nullptr;
        if (MODE == BWD_DW) {
          bsb = dw_bs + dw_bs_blk;
        } else {
          bsb = shared ? (up ? p.sb1s : p.sb0s) : (up ? p.b1s : p.b0s) + (int64_t)t.e * Nd * kb;
          if (MODE == BWD_DX) bsb2 = shared ? p.sb1s : p.b1s + (int64_t)t.e * Nd * kb;
        }
        rs_s = rsrc(bsb, (uint32_t)Nd * kb);
        rs_s2 = rsrc(MODE == BWD_DX ? bsb2 : bsb, (uint32_t)Nd * kb);
        const int n = MODE == GATE_UP ? t.nt * 128 + (lb & 127) : t.nt * BN + lb;
        s_off = n < Nd ? (uint32_t)n * kb : kOff;
      }
    }

    const uint32_t lds0 = lds_addr(&L.stage[0][0]);
    const uint32_t ldss0 = lds_addr(&L.scale[0][0]);
    auto issue = [&](int stage, int kstep) {
      const int k0 = kstep * KS;
      const bool second = MODE == BWD_DX && k0 >= Iv;  // dU / up^T half of K
      const uint32_t kb = (uint32_t)(second ? k0 - Iv : k0) * ES;
      const uint32_t sbase = lds0 + (uint32_t)stage * (A_BYTES + B_BYTES);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        lds_dma16(second ? rs_a2 : rs_a, a_off[i], kb, sbase + (uint32_t)(32 * wave + 8 * i) * ROWB);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        lds_dma16(second ? rs_b2 : rs_b, b_off[i], kb, sbase + A_BYTES + (uint32_t)(32 * wave + 8 * i) * ROWB);
      if (FP8) {
        const uint32_t sb = ldss0 + (uint32_t)stage * (SA_BYTES + SB_BYTES);
        lds_dma4(second ? rs_s2 : rs_s, s_off, (uint32_t)((second ? k0 - Iv : k0) / 32), sb + (uint32_t)(64 * wave) * 4u);
      }
    };

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int sw = swz(lr);  // rows read by this lane are lr mod 32
    auto b_row = [&](int j) { return MODE == GATE_UP ? j * 128 + wn * 32 : wn * 64 + j * 32; };
    // NI = live 32-row blocks (compile time, so that a ragged tile's wave
    // runs only its valid blocks' LDS reads and MFMAs without a per-block
    // branch in the unrolled step)
    // As, Bs: the stage's A and B rows; Sa, Sb: their MXFP8 scale dwords
    // pre(ks): called in BF16 sub-step ks before its MFMAs (the staggered load issue below)
    auto compute = [&](auto ni_c, const uint8_t* As, const uint8_t* Bs, const uint8_t* Sa, const uint8_t* Sb, auto&& pre) {
      constexpr int NI = decltype(ni_c)::value;
      if constexpr (!FP8 && MODE == BWD_DH) {
        // (the dh epilogue leaves no registers for a second fragment set)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int pc = ((2 * ks + lh) ^ sw) * 16;
          bf16x8 fa[NI > 0 ? NI : 1], fb[2];
#pragma unroll
          for (int i = 0; i < NI; ++i)
            fa[i] = *reinterpret_cast<const bf16x8*>(As + (wm * 128 + i * 32 + lr) * ROWB + pc);
#pragma unroll
          for (int j = 0; j < 2; ++j) fb[j] = *reinterpret_cast<const bf16x8*>(Bs + (b_row(j) + lr) * ROWB + pc);
          pre(ks);
#pragma unroll
          for (int i = 0; i < NI; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
        }
      } else if constexpr (!FP8) {
        // Fragments are double-buffered: sub-step ks + 1's LDS reads are
        // issued before sub-step ks's MFMAs (the scheduling barriers keep
        // that order), so the reads' latency overlaps the matrix work
        // instead of stalling the wave between them.
        bf16x8 fa[2][NI > 0 ? NI : 1], fb[2][2];
        auto load_frags = [&](int ks, int buf) {
          const int pc = ((2 * ks + lh) ^ sw) * 16;
#pragma unroll
          for (int i = 0; i < NI; ++i)
            fa[buf][i] = *reinterpret_cast<const bf16x8*>(As + (wm * 128 + i * 32 + lr) * ROWB + pc);
#pragma unroll
          for (int j = 0; j < 2; ++j) fb[buf][j] = *reinterpret_cast<const bf16x8*>(Bs + (b_row(j) + lr) * ROWB + pc);
        };
        load_frags(0, 0);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          if (ks + 1 < 4) load_frags(ks + 1, (ks + 1) & 1);
          pre(ks);
          __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of this sub-step's MFMAs
#pragma unroll
          for (int i = 0; i < NI; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[ks & 1][j], fa[ks & 1][i], acc[i][j], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
        // MFMA sub-step ks covers K bytes [64 ks, 64 ks + 64): lane bytes
        // 0-15 are chunk 4 ks + lh (block 2 ks), bytes 16-31 chunk
        // 4 ks + 2 + lh (block 2 ks + 1); the lane's scale operand is block
        // 2 ks + lh of its row (that byte of the row's scale dword).
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int p0 = ((4 * ks + lh) ^ sw) * 16, p1 = ((4 * ks + 2 + lh) ^ sw) * 16;
          i32x8 fa[NI], fb[2];
          int sa[NI], sbv[2];
#pragma unroll
          for (int i = 0; i < NI; ++i) {
            const int row = wm * 128 + i * 32 + lr;
            const i32x4 lo = *reinterpret_cast<const i32x4*>(As + row * ROWB + p0);
            const i32x4 hi = *reinterpret_cast<const i32x4*>(As + row * ROWB + p1);
            fa[i] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            sa[i] = Sa[row * 4 + 2 * ks + lh];
          }
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int row = b_row(j) + lr;
            const i32x4 lo = *reinterpret_cast<const i32x4*>(Bs + row * ROWB + p0);
            const i32x4 hi = *reinterpret_cast<const i32x4*>(Bs + row * ROWB + p1);
            fb[j] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            sbv[j] = Sb[row * 4 + 2 * ks + lh];
          }
#pragma unroll
          for (int i = 0; i < NI; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[j], fa[i], acc[i][j], 0, 0, 0, sbv[j],
                                                                           0, sa[i]);
        }
      }
    };

    // ---- main loop: two stages, step kt+1 in flight while kt is consumed ----
    const int nk = K / KS;
    // Down: the assignment of row m0 + tid is loaded ahead of the first
    // step's loads (inline, so that the compiler's own wait for it cannot
    // also cover them); its router weight then goes straight into the row
    // table by LDS-DMA (zero past the segment), landing with the step.
    auto k_loop = [&](auto ni_c) {
      if constexpr (kLateMeta) {
        const int r = t.m0 + tid;
        const bool routed_row = tid < BM && r < t.m_end && !shared;
        int a = 0;
        if (routed_row) asm volatile("global_load_dword %0, %1, off" : "=v"(a) : "v"(p.row_src + r) : "memory");
        if (nk > 0) issue(0, 0);
        // the assignment is older than this wave's FP8 ? 9 : 8 loads of the step
        if constexpr (FP8)
          asm volatile("s_waitcnt vmcnt(9)" : "+v"(a) : : "memory");
        else
          asm volatile("s_waitcnt vmcnt(8)" : "+v"(a) : : "memory");
        if (tid < BM) {
          if (shared)
            L.row_w[tid] = r < t.m_end ? 1.f : 0.f;
          else
            lds_dma4(rsrc(p.router_w, (uint32_t)T * p.k * 4u), routed_row ? (uint32_t)a * 4u : kOff, 0u,
                     lds_addr(&L.row_w[64 * wave]));
        }
      } else {
        wait_vmcnt<0>();  // stores of the previous tile's epilogue are older than these loads
        if (nk > 0) issue(0, 0);
      }
      for (int kt = 0; kt < nk; ++kt) {
        wait_vmcnt<0>();
        __syncthreads();  // every wave's loads of step kt landed; step kt-1's stage is free
        // BF16: the two waves of a SIMD issue the next step's loads at
        // different times (waves 0-3 here, waves 4-7 after their first
        // sub-step's MFMAs), so that while one waits to issue its loads at
        // the CU's load unit the other's MFMAs keep the matrix pipe busy.
        // (MXFP8: issued here by all; the later issue point spills its
        // fragments.)
        constexpr bool kStagger = !FP8 && decltype(ni_c)::value > 0;
        if ((!kStagger || wave < 4) && kt + 1 < nk) issue((kt + 1) & 1, kt + 1);
        if constexpr (decltype(ni_c)::value > 0) {
          const uint8_t* As = &L.stage[kt & 1][0];
          const uint8_t* Sa = &L.scale[kt & 1][0];
          compute(ni_c, As, As + A_BYTES, Sa, Sa + SA_BYTES, [&](int i) {
            if (kStagger && wave >= 4 && i == 1 && kt + 1 < nk) issue((kt + 1) & 1, kt + 1);
          });
        }
      }
    };
    // Short tiles: three compact stages, steps kt+1 and kt+2 in flight while
    // kt is consumed. Each wave loads 8 of the SHORT_ROWS A rows and its 32 B
    // rows (5 instructions a step; in MXFP8 wave 0 adds the A rows' scale
    // dwords and waves 4-7 the B rows'), so step kt has landed once at most 5
    // of the wave's loads are outstanding: at least 5 of step kt+1's are
    // younger.
    constexpr bool kShortRing = MODE == GATE_UP;
    auto k_loop_short = [&](auto ni_c) {
      const int arow = 8 * wave + dr;
      const int asrc = L.row_src[arow];
      const uint32_t a_off_s = asrc >= 0 ? (uint32_t)asrc * a_row_bytes + 16u * (uint32_t)(dp ^ swz(arow)) : kOff;
      auto issue_s = [&](int slot, int kstep) {
        const uint32_t kb = (uint32_t)(kstep * KS) * ES;
        const uint32_t sbase = lds0 + (uint32_t)slot * SHORT_SLOT;
        lds_dma16(rs_a, a_off_s, kb, sbase + (uint32_t)(8 * wave) * ROWB);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          lds_dma16(rs_b, b_off[i], kb, sbase + SHORT_ROWS * ROWB + (uint32_t)(32 * wave + 8 * i) * ROWB);
        if (FP8 && (wave == 0 || wave >= 4)) {
          const uint32_t ss = ldss0 + (uint32_t)slot * SHORT_SSLOT +
                              (wave == 0 ? 0u : (uint32_t)(SHORT_ROWS + 64 * (wave - 4)) * 4u);
          lds_dma4(rs_s, s_off, (uint32_t)(kstep * KS / 32), ss);
        }
      };
      wait_vmcnt<0>();  // stores of the previous tile's epilogue are older than these loads
      if (nk > 0) issue_s(0, 0);
      if (nk > 1) issue_s(1, 1);
      int slot = 0;
      for (int kt = 0; kt < nk; ++kt) {
        if (kt + 1 < nk)
          wait_vmcnt<5>();
        else
          wait_vmcnt<0>();
        __syncthreads();  // every wave's loads of step kt landed; step kt-1's stage is free
        if (kt + 2 < nk) issue_s(slot == 0 ? 2 : slot - 1, kt + 2);
        if constexpr (decltype(ni_c)::value > 0) {
          const uint8_t* As = &L.stage[0][0] + slot * SHORT_SLOT;
          const uint8_t* Sa = &L.scale[0][0] + slot * SHORT_SSLOT;
          compute(ni_c, As, As + SHORT_ROWS * ROWB, Sa, Sa + SHORT_ROWS * 4, [](int) {});
        }
        slot = slot == 2 ? 0 : slot + 1;
      }
    };
    // every wave runs the same loads and barriers; only its MFMA blocks differ
    if (kShortRing && rows_here <= SHORT_ROWS) {
      // wave rows 0-127 hold at most 2 live blocks, rows 128-255 none
      switch (live_blocks) {
        case 2: k_loop_short(std::integral_constant<int, 2>{}); break;
        case 1: k_loop_short(std::integral_constant<int, 1>{}); break;
        default: k_loop_short(std::integral_constant<int, 0>{}); break;
      }
    } else {
      switch (live_blocks) {
        case 4: k_loop(std::integral_constant<int, 4>{}); break;
        case 3: k_loop(std::integral_constant<int, 3>{}); break;
        case 2: k_loop(std::integral_constant<int, 2>{}); break;
        case 1: k_loop(std::integral_constant<int, 1>{}); break;
        default: k_loop(std::integral_constant<int, 0>{}); break;
      }
    }

    // ---- epilogue ----
    __syncthreads();  // the stages are free: stage output tiles per wave
    if constexpr (MODE == GATE_UP) {
      // wave columns: h columns nt*128 + wn*32 .. +32 (gate tile j = 0 and up
      // tile j = 1 hold the same columns)
      const int64_t sh = shared ? p.rows_cap_max * p.I : 0;  // element offset of the shared rows
      const int col0 = t.nt * 128 + wn * 32;
      if constexpr (!FP8) {
        constexpr int SW = 32 + 8;  // staged row stride (bf16): 80 bytes
        uint16_t* reg = reinterpret_cast<uint16_t*>(&L.stage[0][0]) + wave * 128 * SW;
        // output sel: 0 = h, 1 = G, 2 = U (G and U only when a context is kept)
        auto store_out = [&](uint16_t* ob, auto sel_c) {
          constexpr int SEL = decltype(sel_c)::value;
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              float v[4];
#pragma unroll
              for (int c = 0; c < 4; ++c) {
                const float g = acc[i][0][4 * q + c], u = acc[i][1][4 * q + c];
                v[c] = SEL == 0 ? swiglu_f(g, u, p.swiglu_lim)
                                : (SEL == 1 ? saved_gate(g, p.swiglu_lim) : saved_up(u, p.swiglu_lim));
              }
              *reinterpret_cast<uint2*>(reg + (i * 32 + lr) * SW + 8 * q + 4 * lh) =
                  make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
            }
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
          const int col = col0 + (lane & 3) * 8;
#pragma unroll
          for (int it = 0; it < 8; ++it) {  // 128 rows x 4 chunks of 16 bytes, 16 rows per instruction
            const int r = it * 16 + (lane >> 2);
            const int ml = wm * 128 + r;
            const u32x4 v = *reinterpret_cast<const u32x4*>(reg + r * SW + (lane & 3) * 8);
            if (ml < rows_here && col < Nd) *reinterpret_cast<u32x4*>(ob + (int64_t)(t.m0 + ml) * Nd + col) = v;
          }
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        };
        store_out((uint16_t*)p.out + sh, std::integral_constant<int, 0>{});
        if (p.ctx_g) {
          store_out((uint16_t*)p.ctx_g + sh, std::integral_constant<int, 1>{});
          store_out((uint16_t*)p.ctx_u + sh, std::integral_constant<int, 2>{});
        }
      } else {
        // h = silu(g) * u in fp32, quantized along I in blocks of 32: the
        // block is this wave's 32 columns, split between lanes lh = 0 and 1
        // of the same row, so the block maximum takes one cross-lane max.
        constexpr int SW = 32 + 16;  // staged row stride (bytes)
        uint8_t* reg = &L.stage[0][0] + wave * 128 * SW;
        uint8_t* hq = (uint8_t*)p.out + sh;
        uint8_t* hs = p.out_scale + (shared ? p.rows_cap_max * (p.I / 32) : 0);
        const int nb = Nd / 32;
        const int blk = col0 / 32;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float hv[16];
          uint32_t amax = 0;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            hv[r] = swiglu_f(acc[i][0][r], acc[i][1][r], p.swiglu_lim);
            amax = max(amax, f2u(hv[r]) & 0x7FFFFFFFu);
          }
          amax = max(amax, (uint32_t)__shfl_xor((int)amax, 32));
          const int X = mx_block_exponent(amax);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t w = e4m3x4_encode_scaled(hv[4 * q], hv[4 * q + 1], hv[4 * q + 2], hv[4 * q + 3], X);
            *reinterpret_cast<uint32_t*>(reg + (i * 32 + lr) * SW + 8 * q + 4 * lh) = w;
          }
          const int ml = wm * 128 + i * 32 + lr;
          if (lh == 0 && ml < rows_here && blk < nb) hs[(int64_t)(t.m0 + ml) * nb + blk] = (uint8_t)(X + 127);
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        const int col = col0 + (lane & 1) * 16;
#pragma unroll
        for (int it = 0; it < 4; ++it) {  // 128 rows x 2 chunks of 16 bytes, 32 rows per instruction
          const int r = it * 32 + (lane >> 1);
          const int ml = wm * 128 + r;
          const u32x4 v = *reinterpret_cast<const u32x4*>(reg + r * SW + (lane & 1) * 16);
          if (ml < rows_here && col < Nd) *reinterpret_cast<u32x4*>(hq + (int64_t)(t.m0 + ml) * Nd + col) = v;
        }
        if (p.ctx_g) {
          // G and U for the backward, fp32 as accumulated. Staged through
          // LDS 64 rows at a time, so that each store instruction writes
          // whole 128-byte lines (8 lanes per row: the wave's 32 columns),
          // non-temporal: they are read only by the backward, and streaming
          // them past L2 keeps the operands' lines there.
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
          constexpr int SWC = 32 + 4;  // staged row stride (floats)
          // (past the 8 waves' h staging areas, so no wave waits for another)
          float* regc = reinterpret_cast<float*>(&L.stage[0][0] + NTHR / 64 * 128 * SW) + wave * 64 * SWC;
          static_assert(NTHR / 64 * (128 * SW + 64 * SWC * 4) <= NSTAGE * (A_BYTES + B_BYTES), "ctx staging fits");
          const float L = p.swiglu_lim;
          const int col = col0 + (lane & 7) * 4;
#pragma unroll
          for (int gu = 0; gu < 2; ++gu) {
            float* dst = gu ? (float*)p.ctx_u : (float*)p.ctx_g;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
#pragma unroll
              for (int ii = 0; ii < 2; ++ii) {
                const int i = 2 * half + ii;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                  const float a0 = acc[i][gu][4 * q], a1 = acc[i][gu][4 * q + 1], a2 = acc[i][gu][4 * q + 2],
                              a3 = acc[i][gu][4 * q + 3];
                  *reinterpret_cast<float4*>(regc + (ii * 32 + lr) * SWC + 8 * q + 4 * lh) =
                      gu ? make_float4(saved_up(a0, L), saved_up(a1, L), saved_up(a2, L), saved_up(a3, L))
                         : make_float4(saved_gate(a0, L), saved_gate(a1, L), saved_gate(a2, L), saved_gate(a3, L));
                }
              }
              asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
              for (int it = 0; it < 8; ++it) {  // 64 rows x 8 chunks of 16 bytes, 8 rows per instruction
                const int r = it * 8 + (lane >> 3);
                const int ml = wm * 128 + half * 64 + r;
                const u32x4 v = *reinterpret_cast<const u32x4*>(regc + r * SWC + (lane & 7) * 4);
                if (ml < rows_here && col < Nd)
                  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst + sh + (int64_t)(t.m0 + ml) * Nd + col));
              }
              asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            }
          }
        }
      }
    } else if constexpr (MODE == DOWN || MODE == BWD_DX || MODE == BWD_DW) {
      // wave tile: 128 rows x 64 columns, staged 64 rows at a time
      constexpr int SW = 64 + 8;  // 144 bytes
      uint16_t* reg = reinterpret_cast<uint16_t*>(&L.stage[0][0]) + wave * 64 * SW;
      uint16_t* ob;
      int64_t ldo = p.H;  // output row stride (elements)
      if constexpr (MODE == BWD_DW) {
        // the job's weight gradient: dW_down [H, Iv], dW_gate / dW_up [Iv, H]
        ldo = Nd;
        const int64_t eo = (int64_t)t.e * p.H * p.I;
        ob = t.job == 0 ? (shared ? p.d_sd : p.d_wd + eo) : t.job == 1 ? (shared ? p.d_sg : p.d_wg + eo)
                                                                      : (shared ? p.d_su : p.d_wu + eo);
      } else {
        ob = (uint16_t*)p.out + (shared ? p.rows_cap_max * p.H : 0);
      }
      const int col = t.nt * BN + wn * 64 + (lane & 7) * 8;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
          const int i = 2 * half + ii;
          const float w = MODE == DOWN ? L.row_w[wm * 128 + i * 32 + lr] : 1.0f;
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
              *reinterpret_cast<uint2*>(reg + (ii * 32 + lr) * SW + j * 32 + 8 * q + 4 * lh) =
                  make_uint2(pack_bf16x2(w * acc[i][j][4 * q], w * acc[i][j][4 * q + 1]),
                             pack_bf16x2(w * acc[i][j][4 * q + 2], w * acc[i][j][4 * q + 3]));
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int it = 0; it < 8; ++it) {  // 64 rows x 8 chunks of 16 bytes, 8 rows per instruction
          const int r = it * 8 + (lane >> 3);
          const int ml = wm * 128 + half * 64 + r;
          const u32x4 v = *reinterpret_cast<const u32x4*>(reg + r * SW + (lane & 7) * 8);
          if (ml < rows_here && col < Nd) {
            if (pipe) {  // read by movers on other XCDs within this launch: stored at agent scope
              uint64_t* d8 = reinterpret_cast<uint64_t*>(ob + (int64_t)(t.m0 + ml) * ldo + col);
              __hip_atomic_store(d8, (uint64_t)v[0] | ((uint64_t)v[1] << 32), __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
              __hip_atomic_store(d8 + 1, (uint64_t)v[2] | ((uint64_t)v[3] << 32), __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
            } else {
              // non-temporal: the rows are read back by a later launch (or
              // the caller), so streaming them past L2 keeps the operands'
              // lines there. Each instruction writes whole 128-byte lines (8
              // lanes per row); partial-line stores marked this way were
              // slower.
              __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(ob + (int64_t)(t.m0 + ml) * ldo + col));
            }
          }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      }
    } else {  // BWD_DH
      // dh_hat[row, col] = acc (fp32). With the saved G, U, h of the row:
      //   dw partial += dh_hat * h,   dh = w * dh_hat,
      //   dG = dh * u * s * (1 + g * (1 - s)) (s = sigmoid(g)),  dU = dh * silu(g),
      //   hw = w * h (the down-weight gradient's right operand; BF16 only).
      // The wave's 128 x 64 tile is staged through LDS one 32-row block at a
      // time (fp32), so that each lane then takes 8 consecutive columns of
      // one row: the saved G, U, h reads and the dG, dU, hw writes of a wave
      // instruction cover whole 128-byte lines of 8 rows.
      constexpr int SWF = 64 + 4;  // staged row stride (floats)
      float* reg = reinterpret_cast<float*>(&L.stage[0][0]) + wave * 32 * SWF;
      const int64_t sh = shared ? p.rows_cap_max * p.I : 0;
      const int rr = lane >> 3, cc = (lane & 7) * 8;  // read-back: rows rr + 8 it, columns cc .. cc + 7
      const int n = t.nt * BN + wn * 64 + cc;        // Nd is a multiple of 64: all 8 columns valid or none
      auto stage_block = [&](int i) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            *reinterpret_cast<float4*>(reg + lr * SWF + j * 32 + 8 * q + 4 * lh) =
                make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      };
      auto store_part = [&](float part, bool row_live, int ml) {  // the row's 64 columns of this wave: 8 lanes
        part += __shfl_xor(part, 1);
        part += __shfl_xor(part, 2);
        part += __shfl_xor(part, 4);
        if (row_live && (lane & 7) == 0) {
          const int64_t prow = shared ? p.rows_cap_max + t.m0 + ml : t.m0 + ml;
          p.dw_part[prow * p.dw_parts + t.nt * kDwPartsPerNTile + wn] = part;
        }
      };
      if constexpr (!FP8) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          stage_block(i);
#pragma unroll 2
          for (int it = 0; it < 4; ++it) {
            const int r = it * 8 + rr;
            const int ml = wm * 128 + i * 32 + r;
            const bool row_live = ml < rows_here;
            float part = 0.f;
            if (row_live && n < Nd) {
              const float w = L.row_w[ml];
              const int64_t rowo = sh + (int64_t)(t.m0 + ml) * Nd + n;
              const float4 d0 = *reinterpret_cast<const float4*>(reg + r * SWF + cc);
              const float4 d1 = *reinterpret_cast<const float4*>(reg + r * SWF + cc + 4);
              const float d[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
              // saved G and U: bf16 pairs
              const uint4 gv = *reinterpret_cast<const uint4*>((const uint16_t*)p.g_in + rowo);
              const uint4 uv = *reinterpret_cast<const uint4*>((const uint16_t*)p.u_in + rowo);
              const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w}, uw[4] = {uv.x, uv.y, uv.z, uv.w};
              const uint4 hv = *reinterpret_cast<const uint4*>(p.h_in + rowo);
              const uint32_t hw4[4] = {hv.x, hv.y, hv.z, hv.w};
              float h[8];
#pragma unroll
              for (int c = 0; c < 8; ++c) h[c] = (c & 1) ? u2f(hw4[c >> 1] & 0xFFFF0000u) : u2f(hw4[c >> 1] << 16);
#pragma unroll
              for (int hh = 0; hh < 2; ++hh) {  // two halves of 4 columns: fewer live registers
                float dg[4], du[4], hwv[4];
#pragma unroll
                for (int c4 = 0; c4 < 4; ++c4) {
                  const int c = 4 * hh + c4;
                  const float g = (c & 1) ? u2f(gw[c >> 1] & 0xFFFF0000u) : u2f(gw[c >> 1] << 16);
                  const float u = (c & 1) ? u2f(uw[c >> 1] & 0xFFFF0000u) : u2f(uw[c >> 1] << 16);
                  part += d[c] * h[c];
                  const float dh = w * d[c];
                  // through the limit: the clamped inputs, and no gradient where the
                  // forward clamped (saved as +-inf)
                  const float L = p.swiglu_lim;
                  const float gc = __builtin_fminf(g, L), uc = __builtin_fminf(__builtin_fmaxf(u, -L), L);
                  const float sg = sigmoid_f(gc);
                  // (both products computed, then selected: as conditional
                  // expressions the compiler branched around them per value)
                  const float dgv = dh * uc * sg * (1.0f + gc * (1.0f - sg)), duv = dh * gc * sg;
                  dg[c4] = g < __builtin_inff() ? dgv : 0.0f;
                  du[c4] = __builtin_fabsf(u) < __builtin_inff() ? duv : 0.0f;
                  hwv[c4] = w * h[c];
                }
                *reinterpret_cast<uint2*>(p.dg_out + rowo + 4 * hh) =
                    make_uint2(pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3]));
                *reinterpret_cast<uint2*>(p.du_out + rowo + 4 * hh) =
                    make_uint2(pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3]));
                if (p.hw_out)
                  *reinterpret_cast<uint2*>(p.hw_out + rowo + 4 * hh) =
                      make_uint2(pack_bf16x2(hwv[0], hwv[1]), pack_bf16x2(hwv[2], hwv[3]));
              }
            }
            store_part(part, row_live, ml);
          }
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        }
      } else {
        // MXFP8: h is the forward's E4M3 h (codes and block scales). dG and
        // dU (fp32) are quantized here, from the values as computed:
        //  - along I for dA: a row's block of 32 columns is 4 lanes x 8;
        //  - along rows for the weight gradients: a staged block holds 32
        //    rows of the expert's segment (tiles start at segment offsets,
        //    which are multiples of 32). dG replaces dh_hat in the wave's
        //    first LDS buffer and dU goes to its second; then lane c reduces
        //    column c's 32 rows of each and writes its 32 codes, one
        //    contiguous run of the transposed operand [cols, K_e]. Rows past
        //    the kept rows are zeros, up to K_e (the segment's rows rounded
        //    up to 128), as the weight gradients' K loop reads them.
        // The two buffers per wave (rows padded as above) take the stages
        // and the LDS right after them.
        static_assert(NTHR / 64 * 2 * 32 * SWF * 4 == NSTAGE * (A_BYTES + B_BYTES) + kEpiExtra, "staging size");
        float* bufg = reinterpret_cast<float*>(&L.stage[0][0]) + wave * 2 * 32 * SWF;
        float* bufu = bufg + 32 * SWF;
        auto at = [](int r, int c) { return r * SWF + c; };
        const int e_t = shared ? E : t.e;
        const int k0 = p.tiles128[e_t];
        const int Kseg = 128 * (p.tiles128[e_t + 1] - k0);  // the segment's K
        const int seg0 = shared ? 0 : offset_at(t.e);        // its first row
        const int64_t tb = shared ? p.tq.kr_cap * p.I : (int64_t)128 * k0 * p.I;      // the segment's codes
        const int64_t tbs = shared ? p.tq.kr_cap / 32 * p.I : (int64_t)4 * k0 * p.I;  // and scales
        const int64_t rqs = shared ? p.rows_cap_max * (p.I / 32) : 0;
        const int nw = t.nt * BN + wn * 64;  // the wave's first column
        const bool cols_live = nw < Nd;      // (the same for the whole wave)
        // the wave's 4 blocks are all below K_e or all past it (K_e and the
        // wave's first row are multiples of 128): their 4 scale bytes per
        // column are adjacent, and go out as one dword after the last block
        const int kl0 = (t.m0 - seg0) + wm * 128;
        const bool blocks_live = kl0 < Kseg;
        uint32_t sc_g = 0, sc_u = 0;
        auto col_pass = [&](const float* buf, uint8_t* tq, uint32_t& sc, int kl, int i) {
          float v[32];
          uint32_t amax = 0;
#pragma unroll
          for (int r2 = 0; r2 < 32; ++r2) {
            v[r2] = buf[r2 * SWF + lane];
            amax = max(amax, f2u(v[r2]) & 0x7FFFFFFFu);
          }
          const int X = mx_block_exponent(amax);
          uint32_t w[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) w[q] = e4m3x4_encode_scaled(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3], X);
          uint8_t* o = tq + tb + (int64_t)(nw + lane) * Kseg + kl;
          *reinterpret_cast<uint4*>(o) = make_uint4(w[0], w[1], w[2], w[3]);
          *reinterpret_cast<uint4*>(o + 16) = make_uint4(w[4], w[5], w[6], w[7]);
          sc |= (uint32_t)(X + 127) << (8 * i);
        };
        if (cols_live) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
              for (int q = 0; q < 4; ++q)
                *reinterpret_cast<float4*>(bufg + at(lr, j * 32 + 8 * q + 4 * lh)) =
                    make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll 2
            for (int it = 0; it < 4; ++it) {
              const int r = it * 8 + rr;
              const int ml = wm * 128 + i * 32 + r;
              const bool row_live = ml < rows_here;
              const int rowi = t.m0 + ml;
              float part = 0.f;
              if (row_live) {
                const float w = L.row_w[ml];
                const int64_t rowo = sh + (int64_t)rowi * Nd + n;
                const float4 d0 = *reinterpret_cast<const float4*>(bufg + at(r, cc));
                const float4 d1 = *reinterpret_cast<const float4*>(bufg + at(r, cc + 4));
                const float d[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
                // the forward's MXFP8 h: 8 codes, all in one block of 32
                const uint2 hc = *reinterpret_cast<const uint2*>(p.hq_in + rowo);
                const float hs =
                    __builtin_ldexpf(1.0f, (int)p.hq_scale_in[rqs + (int64_t)rowi * (Nd / 32) + n / 32] - 127);
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {  // two halves of 4 columns: fewer live registers
                  // saved G and U: fp32, as accumulated
                  const float4 g4 = *reinterpret_cast<const float4*>((const float*)p.g_in + rowo + 4 * hh);
                  const float4 u4 = *reinterpret_cast<const float4*>((const float*)p.u_in + rowo + 4 * hh);
                  const float gs[4] = {g4.x, g4.y, g4.z, g4.w}, us[4] = {u4.x, u4.y, u4.z, u4.w};
                  float dg[4], du[4];
#pragma unroll
                  for (int c4 = 0; c4 < 4; ++c4) {
                    const int c = 4 * hh + c4;
                    const float g = gs[c4], u = us[c4];
                    const float hval = e4m3_decode_byte_scaled(hh ? hc.y : hc.x, c4, hs);
                    part += d[c] * hval;
                    const float dh = w * d[c];
                    const float L = p.swiglu_lim;
                    const float gc = __builtin_fminf(g, L), uc = __builtin_fminf(__builtin_fmaxf(u, -L), L);
                    const float sg = sigmoid_f(gc);
                    const float dgv = dh * uc * sg * (1.0f + gc * (1.0f - sg)), duv = dh * gc * sg;
                    dg[c4] = g < __builtin_inff() ? dgv : 0.0f;
                    du[c4] = __builtin_fabsf(u) < __builtin_inff() ? duv : 0.0f;
                  }
                  // dG takes these dh_hat values' place; dU the same place in
                  // the second buffer
                  *reinterpret_cast<float4*>(bufg + at(r, cc + 4 * hh)) = make_float4(dg[0], dg[1], dg[2], dg[3]);
                  *reinterpret_cast<float4*>(bufu + at(r, cc + 4 * hh)) = make_float4(du[0], du[1], du[2], du[3]);
                }
              } else {  // zeros on rows past the kept rows
                const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
                *reinterpret_cast<float4*>(bufg + at(r, cc)) = z;
                *reinterpret_cast<float4*>(bufg + at(r, cc + 4)) = z;
                *reinterpret_cast<float4*>(bufu + at(r, cc)) = z;
                *reinterpret_cast<float4*>(bufu + at(r, cc + 4)) = z;
              }
              store_part(part, row_live, ml);
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            // along I: the same lanes read their 8 values of dG, then of dU, back
#pragma unroll 1
            for (int it = 0; it < 4; ++it) {
              const int r = it * 8 + rr;
              const int ml = wm * 128 + i * 32 + r;
              const int rowi = t.m0 + ml;
#pragma unroll
              for (int gu = 0; gu < 2; ++gu) {
                const float* buf = gu ? bufu : bufg;
                const float4 v0 = *reinterpret_cast<const float4*>(buf + at(r, cc));
                const float4 v1 = *reinterpret_cast<const float4*>(buf + at(r, cc + 4));
                uint32_t am = max(max(max(f2u(v0.x) & 0x7FFFFFFFu, f2u(v0.y) & 0x7FFFFFFFu),
                                      max(f2u(v0.z) & 0x7FFFFFFFu, f2u(v0.w) & 0x7FFFFFFFu)),
                                  max(max(f2u(v1.x) & 0x7FFFFFFFu, f2u(v1.y) & 0x7FFFFFFFu),
                                      max(f2u(v1.z) & 0x7FFFFFFFu, f2u(v1.w) & 0x7FFFFFFFu)));
                am = max(am, (uint32_t)__shfl_xor((int)am, 1));
                am = max(am, (uint32_t)__shfl_xor((int)am, 2));
                if (ml < rows_here) {
                  const int X = mx_block_exponent(am);
                  const int64_t qo = sh + (int64_t)rowi * Nd + n;
                  *reinterpret_cast<uint2*>((gu ? p.rq_u : p.rq_g) + qo) =
                      make_uint2(e4m3x4_encode_scaled(v0.x, v0.y, v0.z, v0.w, X),
                                 e4m3x4_encode_scaled(v1.x, v1.y, v1.z, v1.w, X));
                  if ((lane & 3) == 0) (gu ? p.rq_us : p.rq_gs)[rqs + (int64_t)rowi * (Nd / 32) + n / 32] = (uint8_t)(X + 127);
                }
              }
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            if (blocks_live) {
              const int kl = kl0 + i * 32;  // the block's first row in the segment
              col_pass(bufg, p.tq.dg, sc_g, kl, i);
              col_pass(bufu, p.tq.du, sc_u, kl, i);
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
          }
          if (blocks_live) {
            const int64_t so = tbs + (int64_t)(nw + lane) * (Kseg / 32) + kl0 / 32;
            *reinterpret_cast<uint32_t*>(p.tq.dgs + so) = sc_g;
            *reinterpret_cast<uint32_t*>(p.tq.dus + so) = sc_u;
          }
        }
      }
    }
    if (pipe) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this thread's y stores are complete
    __syncthreads();  // row metadata and LDS stages are reused by the next tile
    if (pipe && tid == 0)  // every thread's stores of the tile completed: count it
      __hip_atomic_fetch_add(p.mb_done + pass, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  }  // pass
}

}  // namespace nt
}  // namespace mok
