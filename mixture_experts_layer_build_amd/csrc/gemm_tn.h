// Persistent grouped GEMM contracting over an expert's rows ("TN":
// C[m, n] = sum_r A[r, m] * B[r, n], both operands row-major with the
// contraction along rows), on gfx950 MFMA. It computes the weight gradients
// of the expert MLP: for each expert (and the shared expert) and each of
//   type 0: dW_down[h, i] = sum_r dOut_rows[r, h] * (w_r h_r)[i]
//   type 1: dW_gate[i, h] = sum_r dG[r, i] * x_rows[r, h]
//   type 2: dW_up[i, h]   = sum_r dU[r, i] * x_rows[r, h]
// the whole sum over the expert's rows runs inside one output tile, in a
// fixed order: deterministic, no atomics. Rows past the expert's kept rows
// (segment padding, the ragged tail of the shared expert's tokens) are read
// with an out-of-range offset, which the LDS-DMA turns into zeros.
//
// Tiling mirrors the NT kernel: 256 threads, output tile 128 (M) x 256 (N),
// each wave 64 x 128 with 2 x 4 v_mfma_f32_32x32x16_bf16 tiles; one K step =
// 32 rows. The LDS holds each K step as rows of the contraction index:
// A [32][128] (256-byte rows) and B [32][256] (512-byte rows), filled by
// 16-byte LDS-DMA loads, 16-byte chunks XOR-swizzled by row. MFMA operands
// (8 consecutive K values of one M or N index) come from two
// ds_read_b64_tr_b16 per fragment: in a group of 16 lanes, lane i supplies
// the address of 4 consecutive M values at K row i / 4, and lane j receives
// M value j at the 4 K rows.
#pragma once

#include "device_common.h"
#include "gemm_common.h"
#include "mok_internal.h"

namespace mok {
namespace tn {

constexpr int BM = 128, BN = 256, BKR = 32, NTHR = 256, NSTAGE = 3;
constexpr int A_BYTES = BKR * BM * 2, B_BYTES = BKR * BN * 2;  // 8 KiB + 16 KiB per step
constexpr int kBlocksPerCu = 2;
constexpr int kNumXcd = 8;
constexpr uint32_t kOff = 0x80000000u;

struct Params {
  // schedule
  const int32_t* offsets;
  const int32_t* kept;
  const int32_t* hdr;
  int E, H, I, Is;
  int64_t rows_cap_max;
  // row-indexed operands: routed rows [rows_cap_max, .] then shared rows
  const uint16_t* dout_rows;  // [rows_cap_max, H] grad_out gathered in schedule order
  const uint16_t* x_rows;     // [rows_cap_max, H] x gathered in schedule order
  const uint16_t* dout;       // [T, H] (shared expert rows = tokens)
  const uint16_t* x;          // [T, H]
  const uint16_t* hw;         // w * h: routed [rows_cap_max, I], shared [T_max, Is]
  const uint16_t* dg;
  const uint16_t* du;
  // outputs
  uint16_t* d_wd;  // [E, H, I]
  uint16_t* d_wg;  // [E, I, H]
  uint16_t* d_wu;
  uint16_t* d_sd;  // [H, Is]
  uint16_t* d_sg;  // [Is, H]
  uint16_t* d_su;
};

struct alignas(16) Lds {
  uint8_t stage[NSTAGE][A_BYTES + B_BYTES];
};

// Chunk swizzle of a K row: 16-byte reads of 4 rows x 2 chunks (one 16-lane
// group of ds_read_b64_tr_b16) hit distinct bank groups with 32 banks, and 4
// rows x 4 chunks (two groups) with 64 banks.
__device__ __forceinline__ int kswz(int krow) { return (0xCA60 >> ((krow & 3) * 4)) & 0xF; }  // 0, 6, 10, 12

struct Job {
  int type;   // 0 dW_down, 1 dW_gate, 2 dW_up
  int e;      // expert, -1 = shared
  int mt, nt; // output tile
  int M, N;   // output shape
  int rows;   // contraction length (valid rows)
  int r0;     // first row (schedule row; 0 for the shared expert)
  int nk;     // K steps
};

__device__ __forceinline__ void job_dims(const Params& p, int type, bool shared, int& M, int& N) {
  const int Iv = shared ? p.Is : p.I;
  M = type == 0 ? p.H : Iv;
  N = type == 0 ? Iv : p.H;
}

__device__ __forceinline__ int tiles_of(int M, int N) { return ((M + BM - 1) / BM) * ((N + BN - 1) / BN); }

__global__ void __launch_bounds__(NTHR) __attribute__((amdgpu_waves_per_eu(kBlocksPerCu, kBlocksPerCu)))
grouped_gemm_tn(Params p) {
  __shared__ Lds L;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int T = p.hdr[HDR_T];
  const bool has_shared = p.Is > 0;
  // tile counts per expert (routed) and for the shared expert
  int per_e = 0, per_s = 0;
#pragma unroll
  for (int ty = 0; ty < 3; ++ty) {
    int M, N;
    job_dims(p, ty, false, M, N);
    per_e += tiles_of(M, N);
    if (has_shared) {
      job_dims(p, ty, true, M, N);
      per_s += tiles_of(M, N);
    }
  }
  const int ntiles = p.E * per_e + per_s;

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

  const uint32_t lds0 = lds_addr(&L.stage[0][0]);
  for (int id = first; id < stop; id += step) {
    Job j;
    {
      int rem;
      bool shared;
      if (id < p.E * per_e) {
        j.e = id / per_e;
        rem = id - j.e * per_e;
        shared = false;
      } else {
        j.e = -1;
        rem = id - p.E * per_e;
        shared = true;
      }
      j.type = 0;
      for (;;) {
        job_dims(p, j.type, shared, j.M, j.N);
        const int nt_ = tiles_of(j.M, j.N);
        if (rem < nt_ || j.type == 2) break;
        rem -= nt_;
        ++j.type;
      }
      const int ntn = (j.N + BN - 1) / BN;
      j.mt = rem / ntn;
      j.nt = rem - j.mt * ntn;
      if (shared) {
        j.r0 = 0;
        j.rows = T;
      } else {
        j.r0 = p.offsets[j.e];
        j.rows = p.kept[j.e];
      }
      j.nk = (j.rows + BKR - 1) / BKR;
      j.type = __builtin_amdgcn_readfirstlane(j.type);
      j.e = __builtin_amdgcn_readfirstlane(j.e);
      j.mt = __builtin_amdgcn_readfirstlane(j.mt);
      j.nt = __builtin_amdgcn_readfirstlane(j.nt);
      j.r0 = __builtin_amdgcn_readfirstlane(j.r0);
      j.rows = __builtin_amdgcn_readfirstlane(j.rows);
      j.nk = __builtin_amdgcn_readfirstlane(j.nk);
    }
    const bool shared = j.e < 0;
    const int Iv = shared ? p.Is : p.I;
    // operand arrays (row-major, rows = contraction index), based at the
    // job's first row so every buffer range stays far below 2 GiB
    const uint16_t *A, *B;
    int lda, ldb;  // row lengths (elements)
    if (j.type == 0) {
      A = shared ? p.dout : p.dout_rows;
      lda = p.H;
      B = shared ? p.hw + p.rows_cap_max * p.I : p.hw;
      ldb = Iv;
    } else {
      A = shared ? (j.type == 1 ? p.dg : p.du) + p.rows_cap_max * p.I : (j.type == 1 ? p.dg : p.du);
      lda = Iv;
      B = shared ? p.x : p.x_rows;
      ldb = p.H;
    }
    const i32x4v rs_a = rsrc(A + (int64_t)j.r0 * lda, (uint32_t)((int64_t)j.rows * lda * 2));
    const i32x4v rs_b = rsrc(B + (int64_t)j.r0 * ldb, (uint32_t)((int64_t)j.rows * ldb * 2));
    const int m0 = j.mt * BM, n0 = j.nt * BN;

    // DMA lanes: A instruction i (i < 2) of wave w covers K rows
    // 8w + 4i + lane/16, physical chunk lane % 16 (256-byte rows);
    // B instruction i (i < 4) covers K rows 8w + 2i + lane/32, physical
    // chunk lane % 32 (512-byte rows).
    uint32_t a_col[2], b_col[4];
    int a_kr[2], b_kr[4];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int kr = 8 * wave + 4 * i + (lane >> 4);
      const int c = (lane & 15) ^ kswz(kr);
      const int m = m0 + c * 8;
      a_kr[i] = kr;
      a_col[i] = m < j.M ? (uint32_t)m * 2u : kOff;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kr = 8 * wave + 2 * i + (lane >> 5);
      const int c = (lane & 31) ^ kswz(kr);
      const int n = n0 + c * 8;
      b_kr[i] = kr;
      b_col[i] = n < j.N ? (uint32_t)n * 2u : kOff;
    }
    auto issue = [&](int stage, int kstep) {
      const uint32_t sbase = lds0 + (uint32_t)stage * (A_BYTES + B_BYTES);
      const int rbase = kstep * BKR;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = rbase + a_kr[i];
        const uint32_t off = (r < j.rows && a_col[i] != kOff) ? (uint32_t)r * (uint32_t)lda * 2u + a_col[i] : kOff;
        lds_dma16(rs_a, off, 0u, sbase + (uint32_t)(8 * wave + 4 * i) * (BM * 2));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = rbase + b_kr[i];
        const uint32_t off = (r < j.rows && b_col[i] != kOff) ? (uint32_t)r * (uint32_t)ldb * 2u + b_col[i] : kOff;
        lds_dma16(rs_b, off, 0u, sbase + A_BYTES + (uint32_t)(8 * wave + 2 * i) * (BN * 2));
      }
    };

    f32x16 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][jj][r] = 0.f;

    // Transposed fragment reads: lane (g = lane/16, i16 = lane%16) supplies
    // the address of K row ks*16 + (g/2)*8 + 4h + i16/4, M (or N) values
    // base + 16*(g%2) + 4*(i16%4) .. +3.
    const int g = (lane >> 4) & 3, i16 = lane & 15;
    auto tr_read = [&](const uint8_t* base, int row_bytes, int ks, int h, int mbase) {
      const int kr = ks * 16 + (g >> 1) * 8 + 4 * h + (i16 >> 2);
      const int m = mbase + 16 * (g & 1) + 4 * (i16 & 3);
      const int pc = ((m >> 3) ^ kswz(kr)) * 16 + (m & 7) * 2;
      return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4v*)(base + kr * row_bytes + pc));
    };
    auto frag = [&](const uint8_t* base, int row_bytes, int ks, int mbase) {
      const i16x4v lo = tr_read(base, row_bytes, ks, 0, mbase);
      const i16x4v hi = tr_read(base, row_bytes, ks, 1, mbase);
      const i16x8v v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      return __builtin_bit_cast(bf16x8, v);
    };
    auto compute = [&](int stage) {
      const uint8_t* As = &L.stage[stage][0];
      const uint8_t* Bs = As + A_BYTES;
      bf16x8 fa[2][2], fb[2][4];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int i = 0; i < 2; ++i) fa[ks][i] = frag(As, BM * 2, ks, wm * 64 + i * 32);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) fb[ks][jj] = frag(Bs, BN * 2, ks, wn * 128 + jj * 32);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[ks][jj], fa[ks][i], acc[i][jj], 0, 0, 0);
    };

    const int nk = j.nk;
    wait_vmcnt<0>();
    if (nk > 0) issue(0, 0);
    if (nk > 1) issue(1, 1);
    for (int kt = 0; kt < nk; ++kt) {
      if (kt + 1 < nk)
        wait_vmcnt<6>();
      else
        wait_vmcnt<0>();
      __syncthreads();
      if (kt + 2 < nk) issue((kt + 2) % NSTAGE, kt + 2);
      compute(kt % NSTAGE);
    }

    // Epilogue: the accumulator of lane (lr, lh) in MFMA tile (i, jj) is
    // output row m0 + wm*64 + i*32 + lr, columns n0 + wn*128 + jj*32 +
    // 8*(r/4) + 4*lh + r%4. Staged per wave, written as 16-byte row chunks.
    __syncthreads();
    uint16_t* out;
    if (j.type == 0)
      out = shared ? p.d_sd : p.d_wd + (int64_t)j.e * p.H * p.I;
    else if (j.type == 1)
      out = shared ? p.d_sg : p.d_wg + (int64_t)j.e * p.I * p.H;
    else
      out = shared ? p.d_su : p.d_wu + (int64_t)j.e * p.I * p.H;
    constexpr int SW = 128 + 8;
    const int lr = lane & 31, lh = lane >> 5;
    uint16_t* reg = reinterpret_cast<uint16_t*>(&L.stage[0][0]) + wave * 64 * SW;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<uint2*>(reg + (i * 32 + lr) * SW + jj * 32 + 8 * q + 4 * lh) =
              make_uint2(pack_bf16x2(acc[i][jj][4 * q], acc[i][jj][4 * q + 1]),
                         pack_bf16x2(acc[i][jj][4 * q + 2], acc[i][jj][4 * q + 3]));
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const int col = n0 + wn * 128 + (lane & 15) * 8;
#pragma unroll
    for (int it = 0; it < 16; ++it) {
      const int r = it * 4 + (lane >> 4);
      const int m = m0 + wm * 64 + r;
      const u32x4 v = *reinterpret_cast<const u32x4*>(reg + r * SW + (lane & 15) * 8);
      if (m < j.M && col < j.N) *reinterpret_cast<u32x4*>(out + (int64_t)m * j.N + col) = v;
    }
    __syncthreads();
  }
}

}  // namespace tn
}  // namespace mok
