// The combine ("Mixture-of-Kittens: a deterministic MoE megakernel for NVL72
// racks", "The two API layers and the schedule object": the dispatch and
// combine schedule): out[t] = bf16( sum over j = 0 .. k-1 with
// slot_row[t, j] >= 0 of rows[slot_row[t, j]], then + rows_shared[t] ), the
// fp32 adds in exactly that order, so the result does not depend on timing.
// The forward sums the weighted down rows y into out; the backward sums the
// dA rows into dx.
//
// One workgroup per token at a time; a thread owns 8 consecutive columns
// (16 bytes) and issues the loads of up to 8 slots before adding them, so a
// token costs one memory round trip per 8 slots, not one per slot. Each row
// is read once: the loads are non-temporal, so they stream past L2 instead
// of evicting lines that later launches read (measured 5 % faster).
#pragma once

#include "device_common.h"
#include "mok_internal.h"

namespace mok {
namespace {

__device__ __forceinline__ uint4 load_once16(const uint16_t* p) {
  const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(x[0], x[1], x[2], x[3]);
}

__global__ void __launch_bounds__(256) sum_slot_rows(const int32_t* __restrict__ hdr, int hash, int32_t* status,
                                                     const int32_t* __restrict__ slot_row,
                                                     const uint16_t* __restrict__ rows,
                                                     const uint16_t* __restrict__ rows_shared, uint16_t* __restrict__ out,
                                                     int H, int k) {
  constexpr int kBatch = 8;
  if (!sched_matches(hdr, hash, status)) return;
  const int T = hdr[HDR_T];
  const int nchunk = H / 8;
  for (int t = (int)blockIdx.x; t < T; t += gridDim.x) {
    const int32_t* sl = slot_row + (int64_t)t * k;
    for (int c = threadIdx.x; c < nchunk; c += blockDim.x) {
      float acc[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = 0.f;
      auto add = [&](const uint4& v) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * q] += u2f(w[q] << 16);
          acc[2 * q + 1] += u2f(w[q] & 0xFFFF0000u);
        }
      };
      for (int j0 = 0; j0 < k; j0 += kBatch) {
        int row[kBatch];
        uint4 v[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          row[u] = j0 + u < k ? sl[j0 + u] : -1;
          v[u] = row[u] >= 0 ? load_once16(rows + (int64_t)row[u] * H + c * 8) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
          if (row[u] >= 0) add(v[u]);
      }
      if (rows_shared) add(load_once16(rows_shared + (int64_t)t * H + c * 8));
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
}  // namespace mok
