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
// share a block with cross-lane shuffles.
#include "device_common.h"
#include "mok_internal.h"

namespace mok {
namespace {

// axis = 1, bf16 source: 4 lanes per 32-element block, 8 elements per lane.
__global__ void __launch_bounds__(256) quant_axis1_bf16(const uint16_t* __restrict__ src, int64_t rows,
                                                        int64_t cols, int64_t ld_src, uint8_t* __restrict__ dst,
                                                        int64_t ld_dst, uint8_t* __restrict__ scale) {
  const int64_t nblk_row = cols >> 5;
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t b = g >> 2;
  const int part = (int)(g & 3);
  const bool live = b < rows * nblk_row;
  int64_t row = 0, blk = 0;
  uint4 raw = make_uint4(0, 0, 0, 0);
  if (live) {
    row = b / nblk_row;
    blk = b - row * nblk_row;
    raw = *reinterpret_cast<const uint4*>(src + row * ld_src + blk * 32 + part * 8);
  }
  uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t lo = (w[i] << 16) & 0x7FFFFFFFu, hi = w[i] & 0x7FFF0000u;
    amax = max(amax, max(lo, hi));
  }
  amax = max(amax, (uint32_t)__shfl_xor((int)amax, 1));
  amax = max(amax, (uint32_t)__shfl_xor((int)amax, 2));
  if (!live) return;
  const int X = mx_block_exponent(amax);
  uint32_t c[2] = {0, 0};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t e0 = e4m3_encode_scaled(u2f(w[i] << 16), X);
    uint32_t e1 = e4m3_encode_scaled(u2f(w[i] & 0xFFFF0000u), X);
    c[i >> 1] |= (e0 | (e1 << 8)) << ((i & 1) * 16);
  }
  *reinterpret_cast<uint2*>(dst + row * ld_dst + blk * 32 + part * 8) = make_uint2(c[0], c[1]);
  if (part == 0) scale[row * nblk_row + blk] = (uint8_t)(X + 127);
}

// axis = 1, bf16 source with the row count read on the device (the
// schedule header's token count), over a grid sized for max_rows.
__global__ void __launch_bounds__(256) quant_rows_dev_bf16(const uint16_t* __restrict__ src, const int32_t* __restrict__ hdr,
                                                           int64_t cols, uint8_t* __restrict__ dst,
                                                           uint8_t* __restrict__ scale) {
  const int64_t rows = hdr[HDR_T];
  const int64_t nblk_row = cols >> 5;
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t b = g >> 2;
  const int part = (int)(g & 3);
  const bool live = b < rows * nblk_row;
  int64_t row = 0, blk = 0;
  uint4 raw = make_uint4(0, 0, 0, 0);
  if (live) {
    row = b / nblk_row;
    blk = b - row * nblk_row;
    raw = *reinterpret_cast<const uint4*>(src + row * cols + blk * 32 + part * 8);
  }
  uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t lo = (w[i] << 16) & 0x7FFFFFFFu, hi = w[i] & 0x7FFF0000u;
    amax = max(amax, max(lo, hi));
  }
  amax = max(amax, (uint32_t)__shfl_xor((int)amax, 1));
  amax = max(amax, (uint32_t)__shfl_xor((int)amax, 2));
  if (!live) return;
  const int X = mx_block_exponent(amax);
  uint32_t c[2] = {0, 0};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t e0 = e4m3_encode_scaled(u2f(w[i] << 16), X);
    uint32_t e1 = e4m3_encode_scaled(u2f(w[i] & 0xFFFF0000u), X);
    c[i >> 1] |= (e0 | (e1 << 8)) << ((i & 1) * 16);
  }
  *reinterpret_cast<uint2*>(dst + row * cols + blk * 32 + part * 8) = make_uint2(c[0], c[1]);
  if (part == 0) scale[row * nblk_row + blk] = (uint8_t)(X + 127);
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
  uint32_t c = e4m3_encode_scaled(v.x, X) | (e4m3_encode_scaled(v.y, X) << 8) |
               (e4m3_encode_scaled(v.z, X) << 16) | (e4m3_encode_scaled(v.w, X) << 24);
  *reinterpret_cast<uint32_t*>(dst + row * ld_dst + blk * 32 + part * 4) = c;
  if (part == 0) scale[row * nblk_row + blk] = (uint8_t)(X + 127);
}

// axis = 0: one lane owns 16 bytes of columns (8 bf16 or 4 fp32) of one
// 32-row block; it reads the 32 rows, reduces each column's maximum and
// writes the 32 code rows and the block's scale bytes.
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
  uint4 raw[32];
  const T* p = src + rb * 32 * ld_src + col;
#pragma unroll
  for (int r = 0; r < 32; ++r) raw[r] = *reinterpret_cast<const uint4*>(p + r * ld_src);
  float vals[CW];
  uint32_t amax[CW];
#pragma unroll
  for (int c = 0; c < CW; ++c) amax[c] = 0;
#pragma unroll
  for (int r = 0; r < 32; ++r) {
    const uint32_t w[4] = {raw[r].x, raw[r].y, raw[r].z, raw[r].w};
#pragma unroll
    for (int c = 0; c < CW; ++c) {
      uint32_t bits = sizeof(T) == 2 ? ((c & 1) ? (w[c >> 1] & 0xFFFF0000u) : (w[c >> 1] << 16)) : w[c];
      amax[c] = max(amax[c], bits & 0x7FFFFFFFu);
    }
  }
  int X[CW];
#pragma unroll
  for (int c = 0; c < CW; ++c) X[c] = mx_block_exponent(amax[c]);
#pragma unroll
  for (int r = 0; r < 32; ++r) {
    const uint32_t w[4] = {raw[r].x, raw[r].y, raw[r].z, raw[r].w};
    uint32_t code[2] = {0, 0};
#pragma unroll
    for (int c = 0; c < CW; ++c) {
      uint32_t bits = sizeof(T) == 2 ? ((c & 1) ? (w[c >> 1] & 0xFFFF0000u) : (w[c >> 1] << 16)) : w[c];
      vals[c] = u2f(bits);
      code[c >> 2] |= e4m3_encode_scaled(vals[c], X[c]) << ((c & 3) * 8);
    }
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

}  // namespace

hipError_t launch_quantize_rows_dev(const void* src, const int32_t* hdr, int64_t max_rows, int64_t cols, uint8_t* dst,
                                    uint8_t* dst_scale, hipStream_t s) {
  const int64_t lanes = max_rows * (cols >> 5) * 4;
  const int64_t grid = (lanes + 255) / 256;
  if (grid == 0) return hipSuccess;
  quant_rows_dev_bf16<<<dim3((unsigned)grid), dim3(256), 0, s>>>((const uint16_t*)src, hdr, cols, dst, dst_scale);
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
      quant_axis1_bf16<<<dim3((unsigned)grid), dim3(threads), 0, s>>>((const uint16_t*)src, rows, cols, ld_src,
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
