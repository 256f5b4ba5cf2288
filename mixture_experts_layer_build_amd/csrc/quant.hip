// MXFP8 quantization: E4M3 elements with one E8M0 scale per 32 elements.
//
// "Mixture-of-Kittens: a deterministic MoE megakernel for NVL72 racks",
// section "Tuning the five hyperparameters before production": in MXFP8
// mode weights are quantized ahead of time by a separate call, activations
// enter in BF16. Block rule (OCP MX v1.0): X = clamp(floor(log2 amax) - 8,
// -127, 127), scale byte X + 127, elements round-to-nearest-even of v / 2^X
// on the E4M3 grid, saturating at 448, sign kept.
//
// HBM-bound streaming kernels: 16-byte loads per lane, consecutive lanes on
// consecutive 16-byte chunks, the block maximum reduced across the lanes that
// share a block with cross-lane shuffles. Codes of a block come from the
// hardware scaled conversion (e4m3x4_encode_scaled), bit-identical to the
// integer encoder, which the axis-0 kernel (a scale per column) keeps.
#include <algorithm>

#include "device_common.h"
#include "mok_internal.h"

namespace mok {
namespace {

// axis = 1, bf16 source: one workgroup per row, 4 lanes per 32-element
// block, 8 elements (16 bytes) per lane, lanes on consecutive chunks, each
// lane with up to 4 chunks' loads in flight. A row has nchunk = cols / 8
// chunks, a multiple of 4, and the workgroup size is a multiple of 4, so the
// 4 lanes of a block are always active together.
__device__ __forceinline__ void quant_chunk_bf16(const uint4 raw, uint8_t* __restrict__ d, uint8_t* __restrict__ sc,
                                                 int c) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = (w[i] << 16) & 0x7FFFFFFFu, hi = w[i] & 0x7FFF0000u;
    amax = max(amax, max(lo, hi));
  }
  amax = max(amax, (uint32_t)__shfl_xor((int)amax, 1));
  amax = max(amax, (uint32_t)__shfl_xor((int)amax, 2));
  const int X = mx_block_exponent(amax);
  uint32_t q[2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
    q[h] = e4m3x4_encode_scaled(u2f(w[2 * h] << 16), u2f(w[2 * h] & 0xFFFF0000u), u2f(w[2 * h + 1] << 16),
                                u2f(w[2 * h + 1] & 0xFFFF0000u), X);
  *reinterpret_cast<uint2*>(d + (int64_t)c * 8) = make_uint2(q[0], q[1]);
  if ((c & 3) == 0) sc[c >> 2] = (uint8_t)(X + 127);
}

__device__ __forceinline__ void quant_row_bf16(const uint16_t* __restrict__ s, uint8_t* __restrict__ d,
                                               uint8_t* __restrict__ sc, int nchunk) {
  constexpr int kU = 4;
  const int bd = blockDim.x;
  for (int c0 = threadIdx.x; c0 < nchunk; c0 += kU * bd) {
    uint4 raw[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u)
      raw[u] = c0 + u * bd < nchunk ? *reinterpret_cast<const uint4*>(s + (int64_t)(c0 + u * bd) * 8)
                                    : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (c0 + u * bd < nchunk) quant_chunk_bf16(raw[u], d, sc, c0 + u * bd);
  }
}

__global__ void __launch_bounds__(256) quant_axis1_bf16(const uint16_t* __restrict__ src, int64_t cols,
                                                        int64_t ld_src, uint8_t* __restrict__ dst, int64_t ld_dst,
                                                        uint8_t* __restrict__ scale) {
  const int64_t row = blockIdx.x;
  quant_row_bf16(src + row * ld_src, dst + row * ld_dst, scale + row * (cols >> 5), (int)(cols >> 3));
}

// The same with the row count read on the device (the schedule header's
// token count), over a grid sized for max_rows.
__global__ void __launch_bounds__(256) quant_rows_dev_bf16(const uint16_t* __restrict__ src, const int32_t* __restrict__ hdr,
                                                           int hash, int32_t* status, int64_t cols,
                                                           uint8_t* __restrict__ dst, uint8_t* __restrict__ scale) {
  if (!sched_matches(hdr, hash, status)) return;
  const int64_t row = blockIdx.x;
  if (row >= hdr[HDR_T]) return;
  quant_row_bf16(src + row * cols, dst + row * cols, scale + row * (cols >> 5), (int)(cols >> 3));
}

// axis = 1, fp32 source: 8 lanes per block, 4 elements per lane.
__global__ void __launch_bounds__(256) quant_axis1_f32(const float* __restrict__ src, int64_t rows, int64_t cols,
                                                       int64_t ld_src, uint8_t* __restrict__ dst, int64_t ld_dst,
                                                       uint8_t* __restrict__ scale) {
  const int64_t nblk_row = cols >> 5;
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t b = g >> 3;
  const int part = (int)(g & 7);
  const bool live = b < rows * nblk_row;
  int64_t row = 0, blk = 0;
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  if (live) {
    row = b / nblk_row;
    blk = b - row * nblk_row;
    v = *reinterpret_cast<const float4*>(src + row * ld_src + blk * 32 + part * 4);
  }
  uint32_t amax = max(max(f2u(v.x) & 0x7FFFFFFFu, f2u(v.y) & 0x7FFFFFFFu),
                      max(f2u(v.z) & 0x7FFFFFFFu, f2u(v.w) & 0x7FFFFFFFu));
  amax = max(amax, (uint32_t)__shfl_xor((int)amax, 1));
  amax = max(amax, (uint32_t)__shfl_xor((int)amax, 2));
  amax = max(amax, (uint32_t)__shfl_xor((int)amax, 4));
  if (!live) return;
  const int X = mx_block_exponent(amax);
  const uint32_t c = e4m3x4_encode_scaled(v.x, v.y, v.z, v.w, X);
  *reinterpret_cast<uint32_t*>(dst + row * ld_dst + blk * 32 + part * 4) = c;
  if (part == 0) scale[row * nblk_row + blk] = (uint8_t)(X + 127);
}

// axis = 0: one lane owns 16 bytes of columns (8 bf16 or 4 fp32) of one
// 32-row block; it reads the 32 rows to reduce each column's maximum, then
// reads them again (from cache) to write the 32 code rows, and writes the
// block's scale bytes (two passes: holding all 32 rows spilled).
template <typename T>
__global__ void __launch_bounds__(256) quant_axis0(const T* __restrict__ src, int64_t rows, int64_t cols,
                                                   int64_t ld_src, uint8_t* __restrict__ dst, int64_t ld_dst,
                                                   uint8_t* __restrict__ scale) {
  constexpr int CW = 16 / sizeof(T);  // columns per lane
  const int64_t ngrp = cols / CW;
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= (rows >> 5) * ngrp) return;
  const int64_t rb = g / ngrp;
  const int64_t col = (g - rb * ngrp) * CW;
  const T* p = src + rb * 32 * ld_src + col;
  auto bits_of = [](const uint4& v, int c) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    return sizeof(T) == 2 ? ((c & 1) ? (w[c >> 1] & 0xFFFF0000u) : (w[c >> 1] << 16)) : w[c];
  };
  uint32_t amax[CW];
#pragma unroll
  for (int c = 0; c < CW; ++c) amax[c] = 0;
#pragma unroll 8
  for (int r = 0; r < 32; ++r) {
    const uint4 v = *reinterpret_cast<const uint4*>(p + r * ld_src);
#pragma unroll
    for (int c = 0; c < CW; ++c) amax[c] = max(amax[c], bits_of(v, c) & 0x7FFFFFFFu);
  }
  int X[CW];
#pragma unroll
  for (int c = 0; c < CW; ++c) X[c] = mx_block_exponent(amax[c]);
#pragma unroll 8
  for (int r = 0; r < 32; ++r) {
    const uint4 v = *reinterpret_cast<const uint4*>(p + r * ld_src);
    uint32_t code[2] = {0, 0};
#pragma unroll
    for (int c = 0; c < CW; ++c) code[c >> 2] |= e4m3_encode_scaled(u2f(bits_of(v, c)), X[c]) << ((c & 3) * 8);
    uint8_t* q = dst + (rb * 32 + r) * ld_dst + col;
    if (CW == 8)
      *reinterpret_cast<uint2*>(q) = make_uint2(code[0], code[1]);
    else
      *reinterpret_cast<uint32_t*>(q) = code[0];
  }
  uint32_t sc[2] = {0, 0};
#pragma unroll
  for (int c = 0; c < CW; ++c) sc[c >> 2] |= (uint32_t)(X[c] + 127) << ((c & 3) * 8);
  uint8_t* s = scale + rb * cols + col;
  if (CW == 8)
    *reinterpret_cast<uint2*>(s) = make_uint2(sc[0], sc[1]);
  else
    *reinterpret_cast<uint32_t*>(s) = sc[0];
}

// ---- transposed quantization (blocks of 32 along the source's rows) ----
//
// A workgroup of 256 threads takes a tile of 128 source rows x 64 columns:
// each thread loads 32 consecutive values of one row into LDS (fp32), then
// thread (column c = tid / 4, block b = tid % 4) reduces rows 32b .. 32b+31
// of column c and writes their 32 codes as one contiguous run of the output
// row c (4 threads fill one 128-byte line) plus the block's scale byte.

constexpr int kTqRows = 128, kTqCols = 64, kTqLd = kTqCols + 1;

// LDS column of (row, col) in the quantizers' 128 x 64 fp32 tile: the
// column is XORed with 16 times the row's 32-row block, so that the column
// reads of tq_store (4 lanes of a column in 4 different blocks) fall in
// distinct banks; the row-wise staging writes (one 32-row block per wave)
// stay conflict-free.
__device__ __forceinline__ int tq_col(int row, int col) { return col ^ ((row >> 5) << 4); }

__device__ __forceinline__ void tq_store(const float (*tile)[kTqLd], uint8_t* out_row, uint8_t* scale_row) {
  const int c = threadIdx.x >> 2, b = threadIdx.x & 3;
  float v[32];
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    v[i] = tile[32 * b + i][c ^ (b << 4)];  // tq_col(32 b + i, c)
    amax = max(amax, f2u(v[i]) & 0x7FFFFFFFu);
  }
  const int X = mx_block_exponent(amax);
  uint32_t w[8];
#pragma unroll
  for (int q = 0; q < 8; ++q)
    w[q] = e4m3x4_encode_scaled(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3], X);
  // out_row / scale_row: the output row of this thread's column c, at the tile's first block
  *reinterpret_cast<uint4*>(out_row + 32 * b) = make_uint4(w[0], w[1], w[2], w[3]);
  *reinterpret_cast<uint4*>(out_row + 32 * b + 16) = make_uint4(w[4], w[5], w[6], w[7]);
  scale_row[b] = (uint8_t)(X + 127);
}

// Weights: src [B][R][C] bf16 -> dst codes [B][C][R], scales [B][C][R/32]
// (R % 128 == 0, C % 64 == 0). The next unit's rows are loaded into
// registers while the current unit is quantized and stored.
__global__ void __launch_bounds__(256) quant_t_matrix(const uint16_t* __restrict__ src, int64_t B, int64_t R, int64_t C,
                                                      uint8_t* __restrict__ dst, uint8_t* __restrict__ dst_scale) {
  __shared__ float tile[kTqRows][kTqLd];
  const int64_t nkb = R / kTqRows, ncc = C / kTqCols;
  const int64_t units = B * nkb * ncc;
  const int r = threadIdx.x >> 1, half = threadIdx.x & 1;
  auto fetch = [&](int64_t u, uint4 (&raw)[4]) {
    const int64_t b = u / (nkb * ncc);
    const int64_t rem = u - b * nkb * ncc;
    const int64_t kb = rem / ncc, cc = rem - kb * ncc;
    const uint16_t* s = src + b * R * C + (kb * kTqRows + r) * C + cc * kTqCols + 32 * half;
#pragma unroll
    for (int q = 0; q < 4; ++q) raw[q] = *reinterpret_cast<const uint4*>(s + 8 * q);
  };
  uint4 raw[4];
  int64_t u = blockIdx.x;
  if (u < units) fetch(u, raw);
  for (; u < units; u += gridDim.x) {
    float* trow = &tile[r][0];  // column (32 half + k) at tq_col(r, 32 half + k)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t w[4] = {raw[q].x, raw[q].y, raw[q].z, raw[q].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        trow[tq_col(r, 32 * half + 8 * q + 2 * j)] = u2f(w[j] << 16);
        trow[tq_col(r, 32 * half + 8 * q + 2 * j + 1)] = u2f(w[j] & 0xFFFF0000u);
      }
    }
    __syncthreads();
    if (u + gridDim.x < units) fetch(u + gridDim.x, raw);
    const int64_t b = u / (nkb * ncc);
    const int64_t rem = u - b * nkb * ncc;
    const int64_t kb = rem / ncc, cc = rem - kb * ncc;
    const int64_t c = cc * kTqCols + (threadIdx.x >> 2);
    tq_store(tile, dst + b * C * R + c * R + kb * kTqRows, dst_scale + b * C * (R / 32) + c * (R / 32) + kb * 4);
    __syncthreads();
  }
}

enum TqSrc : int {
  TQ_X = 0,     // x rows of the segment's tokens (bf16)
  TQ_DY = 1,    // router weight times grad_out rows (bf16 source, fp32 product)
  TQ_ROWS = 2,  // schedule-row-indexed bf16 rows (dG, dU)
  TQ_MX = 3     // schedule-row-indexed MXFP8 rows (the forward's h codes and scales)
};

constexpr int kMaxT128 = 1024 + 2;  // experts + 2 entries of a workspace's largest tile table

struct TqParams {
  int hash;             // the configuration hash the schedule's header must carry
  int32_t* status;      // where a mismatch is counted
  const int32_t* hdr;
  const int32_t* offsets;
  const int32_t* kept;
  const int32_t* tiles128;  // prefix sums of 128-row tiles per expert, [E] routed, [E+1] with shared
  const int32_t* row_src;
  const float* router_w;
  int E, k, cols_r, cols_s;
  int64_t rows_cap_max, kr_cap;
  const uint16_t* src;       // TQ_X / TQ_DY: token rows [T, cols]; TQ_ROWS: routed rows then shared rows
  const uint8_t* src_codes;  // TQ_MX
  const uint8_t* src_scale;
  uint8_t* dst;
  uint8_t* dst_scale;
};

// The weight-gradient GEMMs' operands: for expert e, rows of its segment in
// 128-row blocks (rows past kept[e] are zero) -> [cols, K_e] elements at
// 128 * tiles128[e] * cols_r, quantized to MXFP8 along the rows (with
// scales); the shared expert's all-token segment -> [cols_s, K_s] at
// kr_cap * cols_r.
template <int SRC>
__global__ void __launch_bounds__(256) quant_t_rows(TqParams p) {
  __shared__ float tile[kTqRows][kTqLd];
  __shared__ int32_t t128[kMaxT128];  // the per-expert 128-row tile prefix sums, searched per unit
  if (!sched_matches(p.hdr, p.hash, p.status)) return;  // before any barrier
  const int E = p.E;
  const int T = p.hdr[HDR_T];
  for (int i = threadIdx.x; i <= E + 1; i += blockDim.x) t128[i] = p.tiles128[i];
  __syncthreads();
  const int nkb = t128[E + 1];
  const int ncc = (max(p.cols_r, p.cols_s) + kTqCols - 1) / kTqCols;
  const int64_t units = (int64_t)nkb * ncc;
  const int r = threadIdx.x >> 1, half = threadIdx.x & 1;
  // A unit (128-row block x 64 columns): its expert (E = the shared
  // expert), column chunk and block inside the segment; live is false for a
  // chunk past the expert's columns (uniform across the workgroup).
  struct Unit {
    int e, cc, kl, cols;
    bool live;
  };
  auto place = [&](int64_t u) {
    Unit w;
    const int kb = (int)(u / ncc);
    w.cc = (int)(u - (int64_t)kb * ncc);
    int e = E;
    if (kb < t128[E]) {
      int lo = 0, hi = E;  // largest e with tiles128[e] <= kb
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (t128[mid] <= kb) lo = mid; else hi = mid;
      }
      e = lo;
    }
    w.e = e;
    w.cols = e == E ? p.cols_s : p.cols_r;
    w.live = w.cc * kTqCols < w.cols;
    w.kl = kb - t128[e];
    return w;
  };
  // The thread's 32 source values of its row (row r of the block, columns
  // 32 * half ..), held as loaded so that the next unit's loads are in
  // flight while the current unit is quantized and stored.
  constexpr int NV = SRC == TQ_MX ? 2 : 4;  // 16-byte loads
  uint4 raw[NV];
  float mul = 1.0f;
  int X = 0;
  bool have = false;
  auto fetch = [&](const Unit& w) {
    have = false;
    mul = 1.0f;
    if (!w.live) return;
    const bool shared = w.e == E;
    const int lr = w.kl * kTqRows + r;  // row inside the segment
    const int c0 = w.cc * kTqCols + 32 * half;
    const int nrows = shared ? T : p.kept[w.e];
    if (lr >= nrows) return;  // zero row past the segment's end
    const int64_t row = shared ? lr : p.offsets[w.e] + (int64_t)lr;
    if constexpr (SRC == TQ_MX) {
      const int64_t code0 = shared ? p.rows_cap_max * p.cols_r + row * w.cols : row * w.cols;
      const int64_t sc0 = shared ? p.rows_cap_max * (p.cols_r / 32) + row * (w.cols / 32) : row * (w.cols / 32);
      X = (int)p.src_scale[sc0 + c0 / 32] - 127;
      raw[0] = *reinterpret_cast<const uint4*>(p.src_codes + code0 + c0);
      raw[1] = *reinterpret_cast<const uint4*>(p.src_codes + code0 + c0 + 16);
    } else {
      const uint16_t* s;
      if (shared) {
        s = SRC == TQ_ROWS ? p.src + p.rows_cap_max * p.cols_r + row * w.cols + c0 : p.src + row * w.cols + c0;
      } else if (SRC == TQ_ROWS) {
        s = p.src + row * w.cols + c0;
      } else {
        const int a = p.row_src[row];
        s = p.src + (int64_t)(a / p.k) * w.cols + c0;
        if (SRC == TQ_DY) mul = p.router_w[a];
      }
#pragma unroll
      for (int q = 0; q < NV; ++q) raw[q] = *reinterpret_cast<const uint4*>(s + 8 * q);
    }
    have = true;
  };
  // raw values -> fp32 in the LDS tile (zeros for a row past the segment)
  auto stage = [&]() {
    float* trow = &tile[r][0];  // column (32 half + k) at tq_col(r, 32 half + k)
    if (!have) {
#pragma unroll
      for (int i = 0; i < 32; ++i) trow[tq_col(r, 32 * half + i)] = 0.f;
      return;
    }
    const float xs = SRC == TQ_MX ? __builtin_ldexpf(1.0f, X) : 1.0f;  // the h block's scale 2^X
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      const uint32_t w[4] = {raw[q].x, raw[q].y, raw[q].z, raw[q].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (SRC == TQ_MX) {
#pragma unroll
          for (int b = 0; b < 4; ++b) trow[tq_col(r, 32 * half + 16 * q + 4 * j + b)] = e4m3_decode_byte_scaled(w[j], b, xs);
        } else {
          trow[tq_col(r, 32 * half + 8 * q + 2 * j)] = mul * u2f(w[j] << 16);
          trow[tq_col(r, 32 * half + 8 * q + 2 * j + 1)] = mul * u2f(w[j] & 0xFFFF0000u);
        }
      }
    }
  };
  int64_t u = blockIdx.x;
  Unit cur{};
  if (u < units) {
    cur = place(u);
    fetch(cur);
  }
  for (; u < units; u += gridDim.x) {
    if (cur.live) stage();
    __syncthreads();
    Unit nxt{};
    if (u + gridDim.x < units) {
      nxt = place(u + gridDim.x);
      fetch(nxt);
    }
    if (cur.live) {
      const bool shared = cur.e == E;
      const int64_t Kp = 128 * (int64_t)(shared ? nkb - t128[E] : t128[cur.e + 1] - t128[cur.e]);
      const int64_t kofs = shared ? 0 : 128 * (int64_t)t128[cur.e];
      const int64_t base = shared ? p.kr_cap * p.cols_r : kofs * cur.cols;
      const int64_t sbase = shared ? p.kr_cap / 32 * p.cols_r : kofs / 32 * cur.cols;
      const int64_t c = cur.cc * kTqCols + (threadIdx.x >> 2);
      tq_store(tile, p.dst + base + c * Kp + (int64_t)cur.kl * kTqRows,
               p.dst_scale + sbase + c * (Kp / 32) + cur.kl * 4);
    }
    __syncthreads();
    cur = nxt;
  }
}

// The BF16 weight gradients' operands: the same per-expert transposes
// without quantization, as pure data movement. Tile: 128 segment rows x 128
// columns. A thread loads 16 bytes (8 columns) from each of two adjacent
// rows, for 4 row pairs (8 loads in flight); 16 lanes cover 256 contiguous
// bytes of a row. LDS holds the tile column-major as dwords that pair rows
// 2j and 2j + 1 (65 dwords per column: the writes are at most 2-way bank
// conflicts, the reads none). A thread then writes 16 bytes (8 rows) of one
// output row, 16 lanes per 256-byte run of it.
constexpr int kTbRows = 128, kTbCols = 128, kTbLd = kTbRows / 2 + 1;

template <int SRC>
__global__ void __launch_bounds__(256) transpose_rows_bf16(TqParams p) {
  __shared__ uint32_t tile[kTbCols][kTbLd];
  __shared__ int32_t t128[kMaxT128];  // the per-expert 128-row tile prefix sums, searched per unit
  if (!sched_matches(p.hdr, p.hash, p.status)) return;  // before any barrier
  const int E = p.E;
  const int T = p.hdr[HDR_T];
  for (int i = threadIdx.x; i <= E + 1; i += blockDim.x) t128[i] = p.tiles128[i];
  __syncthreads();
  const int nkb = t128[E + 1];
  const int ncc = (max(p.cols_r, p.cols_s) + kTbCols - 1) / kTbCols;
  const int64_t units = (int64_t)nkb * ncc;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int cch = lane & 15, jq = lane >> 4;  // load phase: 8-column chunk, row pair within the wave's 4
  const int m = threadIdx.x & 15;             // store phase: output rows' 8-element chunk
  for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {
    const int kb = (int)(u / ncc), cc = (int)(u - (int64_t)kb * ncc);
    const bool shared = kb >= t128[E];
    int e = E;
    if (!shared) {
      int lo = 0, hi = E;  // largest e with tiles128[e] <= kb
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (t128[mid] <= kb) lo = mid; else hi = mid;
      }
      e = lo;
    }
    const int cols = shared ? p.cols_s : p.cols_r;
    if (cc * kTbCols >= cols) continue;  // uniform across the workgroup
    const int kl = kb - t128[e];   // block index inside the segment
    const int nrows = shared ? T : p.kept[e];
    const int64_t row0 = shared ? 0 : p.offsets[e];
    const int c0 = cc * kTbCols + 8 * cch;
    const bool col_ok = c0 < cols;  // cols is a multiple of 64: a chunk is all in or all out
    // source of segment row lr (nullptr: a zero row past the segment's end)
    auto row_ptr = [&](int lr, float& mul) -> const uint16_t* {
      mul = 1.0f;
      if (lr >= nrows) return nullptr;
      if (shared) return SRC == TQ_ROWS ? p.src + p.rows_cap_max * p.cols_r + (int64_t)lr * cols : p.src + (int64_t)lr * cols;
      const int64_t row = row0 + lr;
      if (SRC == TQ_ROWS) return p.src + row * cols;
      const int a = p.row_src[row];
      if (SRC == TQ_DY) mul = p.router_w[a];
      return p.src + (int64_t)(a / p.k) * cols;
    };
    uint4 va[4], vb[4];
    float ma[4], mb[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int j = it * 16 + wave * 4 + jq;  // row pair
      const uint16_t* s0 = row_ptr(kl * kTbRows + 2 * j, ma[it]);
      const uint16_t* s1 = row_ptr(kl * kTbRows + 2 * j + 1, mb[it]);
      va[it] = (s0 && col_ok) ? *reinterpret_cast<const uint4*>(s0 + c0) : make_uint4(0, 0, 0, 0);
      vb[it] = (s1 && col_ok) ? *reinterpret_cast<const uint4*>(s1 + c0) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int j = it * 16 + wave * 4 + jq;
      const uint32_t a[4] = {va[it].x, va[it].y, va[it].z, va[it].w};
      const uint32_t b[4] = {vb[it].x, vb[it].y, vb[it].z, vb[it].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {  // columns 8 cch + 2q and 8 cch + 2q + 1
        uint32_t a0 = a[q] & 0xFFFFu, a1 = a[q] >> 16, b0 = b[q] & 0xFFFFu, b1 = b[q] >> 16;
        if (SRC == TQ_DY) {  // router weight times grad_out, rounded to bf16 (nearest even)
          a0 = f32_to_bf16(ma[it] * bf16_to_f32((uint16_t)a0));
          a1 = f32_to_bf16(ma[it] * bf16_to_f32((uint16_t)a1));
          b0 = f32_to_bf16(mb[it] * bf16_to_f32((uint16_t)b0));
          b1 = f32_to_bf16(mb[it] * bf16_to_f32((uint16_t)b1));
        }
        tile[8 * cch + 2 * q][j] = a0 | (b0 << 16);
        tile[8 * cch + 2 * q + 1][j] = a1 | (b1 << 16);
      }
    }
    __syncthreads();
    const int64_t Kp = 128 * (int64_t)(shared ? nkb - t128[E] : t128[e + 1] - t128[e]);
    const int64_t kofs = shared ? 0 : 128 * (int64_t)t128[e];
    uint16_t* dst = reinterpret_cast<uint16_t*>(p.dst) + (shared ? p.kr_cap * p.cols_r : kofs * cols);
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int cl = it * 16 + (threadIdx.x >> 4);  // output row (source column) within the tile
      const int cg = cc * kTbCols + cl;
      const uint32_t* src = &tile[cl][4 * m];
      if (cg < cols)
        *reinterpret_cast<uint4*>(dst + (int64_t)cg * Kp + (int64_t)kl * kTbRows + 8 * m) =
            make_uint4(src[0], src[1], src[2], src[3]);
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_quantize_t_matrix(const void* src, int64_t batches, int64_t R, int64_t C, uint8_t* dst,
                                    uint8_t* dst_scale, int grid_cap, hipStream_t s) {
  const int64_t units = batches * (R / kTqRows) * (C / kTqCols);
  if (units == 0) return hipSuccess;
  const int grid = (int)std::min<int64_t>(units, grid_cap);
  quant_t_matrix<<<grid, 256, 0, s>>>((const uint16_t*)src, batches, R, C, dst, dst_scale);
  return hipGetLastError();
}

hipError_t launch_quantize_t_rows(int src_kind, const SchedView& v, const void* src, const uint8_t* src_codes,
                                  const uint8_t* src_scale, const float* router_w, int E, int k, int cols_r, int cols_s,
                                  int64_t rows_cap_max, int64_t kr_cap, uint8_t* dst, uint8_t* dst_scale, int grid,
                                  hipStream_t s, bool out_bf16) {
  TqParams p{};
  p.hdr = v.header;
  p.hash = v.hash;
  p.status = v.status;
  p.offsets = v.offsets;
  p.kept = v.kept;
  p.tiles128 = v.tiles + tile_bm_index(128) * (E + 2);
  p.row_src = v.row_src;
  p.router_w = router_w;
  p.E = E;
  p.k = k;
  p.cols_r = cols_r;
  p.cols_s = cols_s;
  p.rows_cap_max = rows_cap_max;
  p.kr_cap = kr_cap;
  p.src = (const uint16_t*)src;
  p.src_codes = src_codes;
  p.src_scale = src_scale;
  p.dst = dst;
  p.dst_scale = dst_scale;
  if (out_bf16) {
    switch (src_kind) {
      case TQ_X: transpose_rows_bf16<TQ_X><<<grid, 256, 0, s>>>(p); break;
      case TQ_DY: transpose_rows_bf16<TQ_DY><<<grid, 256, 0, s>>>(p); break;
      case TQ_ROWS: transpose_rows_bf16<TQ_ROWS><<<grid, 256, 0, s>>>(p); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (src_kind) {
      case TQ_X: quant_t_rows<TQ_X><<<grid, 256, 0, s>>>(p); break;
      case TQ_DY: quant_t_rows<TQ_DY><<<grid, 256, 0, s>>>(p); break;
      case TQ_ROWS: quant_t_rows<TQ_ROWS><<<grid, 256, 0, s>>>(p); break;
      default: quant_t_rows<TQ_MX><<<grid, 256, 0, s>>>(p); break;
    }
  }
  return hipGetLastError();
}

// threads per row-quantizer workgroup: a quarter of the row's 16-byte
// chunks, rounded up to whole waves, at most 256
static int row_threads(int64_t cols) {
  const int64_t nchunk = cols >> 3;
  return (int)std::min<int64_t>(256, std::max<int64_t>(64, (nchunk / 4 + 63) / 64 * 64));
}

hipError_t launch_quantize_rows_dev(const void* src, const SchedView& v, int64_t max_rows, int64_t cols, uint8_t* dst,
                                    uint8_t* dst_scale, hipStream_t s) {
  if (max_rows == 0 || cols == 0) return hipSuccess;
  quant_rows_dev_bf16<<<dim3((unsigned)max_rows), dim3(row_threads(cols)), 0, s>>>((const uint16_t*)src, v.header, v.hash, v.status, cols,
                                                                                  dst, dst_scale);
  return hipGetLastError();
}

hipError_t launch_quantize(const void* src, int src_is_fp32, int64_t rows, int64_t cols, int64_t ld_src, int axis,
                           uint8_t* dst, int64_t ld_dst, uint8_t* dst_scale, hipStream_t s) {
  if (rows == 0 || cols == 0) return hipSuccess;
  const int threads = 256;
  if (axis == 1) {
    const int64_t lanes = rows * (cols >> 5) * (src_is_fp32 ? 8 : 4);
    const int64_t grid = (lanes + threads - 1) / threads;
    if (src_is_fp32)
      quant_axis1_f32<<<dim3((unsigned)grid), dim3(threads), 0, s>>>((const float*)src, rows, cols, ld_src, dst,
                                                                    ld_dst, dst_scale);
    else
      quant_axis1_bf16<<<dim3((unsigned)rows), dim3(row_threads(cols)), 0, s>>>((const uint16_t*)src, cols, ld_src,
                                                                               dst, ld_dst, dst_scale);
  } else {
    const int64_t lanes = (rows >> 5) * (cols / (src_is_fp32 ? 4 : 8));
    const int64_t grid = (lanes + threads - 1) / threads;
    if (src_is_fp32)
      quant_axis0<float><<<dim3((unsigned)grid), dim3(threads), 0, s>>>((const float*)src, rows, cols, ld_src, dst,
                                                                       ld_dst, dst_scale);
    else
      quant_axis0<uint16_t><<<dim3((unsigned)grid), dim3(threads), 0, s>>>((const uint16_t*)src, rows, cols,
                                                                          ld_src, dst, ld_dst, dst_scale);
  }
  return hipGetLastError();
}

}  // namespace mok
