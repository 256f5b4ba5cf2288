// Deterministic dispatch/combine schedule.
//
// "Mixture-of-Kittens: a deterministic MoE megakernel for NVL72 racks":
//  - "The two API layers and the schedule object": routing decisions are
//    materialised before any expert kernel runs, and the same schedule feeds
//    forward and backward; it is sized for the worst case through the
//    capacity multiplier.
//  - "Tuning the five hyperparameters before production": capacity
//    multiplier (worst-case share of tokens per destination, 1.0 = all) and
//    expert padding.
// Single-GPU reading: every expert is local, so the capacity caps each
// expert at C = min(T, ceil(mult*T)) assignments; the first C in flat order
// a = t*k + j are kept, later ones dropped; rows of an expert are in
// ascending a; segments are padded to P rows.
//
// Two launches, each a streaming pass (no atomics on global memory, so the
// bytes are identical from run to run):
//   1. count+scan: one workgroup. All threads count the assignments into
//      per-chunk histograms in LDS (LDS atomics: counts do not depend on
//      order), then per-expert exclusive scans over chunks (chunk bases),
//      counts, kept, padded offsets, tile prefix sums, header, padding rows.
//   2. scatter: one wave per chunk: stable rank of each assignment inside its
//      expert from a wave ballot match plus the chunk base, then the
//      permutation (row_src) and its inverse (slot_row).
// (3. minibatch sub-offsets: binary search per (minibatch, expert); only
//     when the schedule has more than one minibatch.)
#include "device_common.h"
#include "mok_internal.h"

namespace mok {
namespace {

constexpr int kWaves = 4;        // waves per workgroup in the scatter kernel
constexpr int kMaxE = 1024;      // the largest expert count a workspace accepts
constexpr int kCountBatch = 16;  // loads in flight per thread while counting
constexpr int kScatterBatch = 8; // 64-assignment rounds loaded ahead per wave (divides iters)

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_inclusive_scan(int x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x;
}

__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

struct SchedParams {
  const int64_t* top;
  int64_t n;          // T*k assignments
  int T, k, E, C, P;
  int iters;          // 64-assignment rounds per chunk (a power of two >= kScatterBatch)
  int chunk_shift;    // log2(iters * 64)
  int scan_group;     // chunk runs per expert in the chunk scan: a power of two <= 64, scan_group * E <= 1024
  int n_chunks;
  int rows_cap;       // rows_cap(T)
  int n_mb, mb;
  int hash;
  int shared_rows;    // T if the shared expert exists, else 0
  SchedView v;
  int32_t* chunk_hist;  // [n_chunks][E] chunk bases for the scatter
};

// One workgroup of 1024 threads.
__global__ void __launch_bounds__(1024) sched_count_scan(SchedParams p) {
  extern __shared__ int32_t lds[];  // [n_chunks * E] per-chunk histograms, then chunk bases
  __shared__ int32_t s_wtot[kNumTileBMs + 3][16];  // per-wave totals: scans, invalid, dropped
  __shared__ int32_t s_tot[kNumTileBMs + 3];
  __shared__ int32_t s_part[1024];  // chunk-run totals of the per-expert scan
  __shared__ int32_t s_cnt[kMaxE];
  __shared__ int32_t s_kept[kMaxE];
  __shared__ int32_t s_off[kMaxE + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = p.E, NC = p.n_chunks;
  int32_t* h = lds;
  for (int i = tid; i < NC * E; i += 1024) h[i] = 0;
  __syncthreads();
  // count: thread tid takes assignments tid + 1024 j, kCountBatch loads ahead
  int invalid = 0;
  for (int64_t a0 = tid; a0 < p.n; a0 += (int64_t)1024 * kCountBatch) {
    int64_t ev[kCountBatch];
#pragma unroll
    for (int u = 0; u < kCountBatch; ++u) {
      const int64_t a = a0 + (int64_t)1024 * u;
      ev[u] = a < p.n ? p.top[a] : 0;
    }
#pragma unroll
    for (int u = 0; u < kCountBatch; ++u) {
      const int64_t a = a0 + (int64_t)1024 * u;
      if (a < p.n) {
        if (ev[u] >= 0 && ev[u] < E)
          atomicAdd(&h[(int)(a >> p.chunk_shift) * E + (int)ev[u]], 1);
        else
          ++invalid;
      }
    }
  }
  // per-expert exclusive scan over chunks (in LDS): G = p.scan_group runs of
  // contiguous chunks per expert, run q of expert e on thread q * E + e (so a
  // wave's lanes read consecutive experts of one chunk: no bank conflicts);
  // the run totals, summed in order, give each run its base.
  __syncthreads();
  {
    const int G = p.scan_group, part = tid / E, ge = tid - part * E;
    const bool act = part < G;
    const int per = (NC + G - 1) / G;
    const int c0 = min(NC, part * per), c1 = min(NC, c0 + per);
    int run = 0;
    if (act)
      for (int c = c0; c < c1; ++c) run += h[c * E + ge];
    s_part[tid] = run;
    __syncthreads();
    if (act) {
      int base = 0;
      for (int q = 0; q < part; ++q) base += s_part[q * E + ge];
      if (part == G - 1) s_cnt[ge] = base + run;
      for (int c = c0; c < c1; ++c) {
        const int v = h[c * E + ge];
        h[c * E + ge] = base;
        base += v;
      }
    }
  }
  __syncthreads();
  // totals and kept, one expert per thread (E <= 1024)
  const int e = tid;
  int kept = 0, dropped = 0;
  if (e < E) {
    const int run = s_cnt[e];
    kept = run < p.C ? run : p.C;
    p.v.counts[e] = run;
    p.v.kept[e] = kept;
    s_kept[e] = kept;
    dropped = run - kept;
  }
  // exclusive scans over experts: padded rows, then tiles for each BM; plus
  // the invalid and dropped totals. Wave scans, then one pass over the 16
  // wave totals.
  const int padded = (kept + p.P - 1) / p.P * p.P;
  int val[1 + kNumTileBMs], incl[1 + kNumTileBMs];
#pragma unroll
  for (int q = 0; q < 1 + kNumTileBMs; ++q) {
    val[q] = q == 0 ? padded : (padded + kTileBM[q - 1] - 1) / kTileBM[q - 1];
    incl[q] = wave_inclusive_scan(val[q], lane);
  }
  const int inv_w = wave_sum(invalid), drop_w = wave_sum(dropped);
  if (lane == 63) {
#pragma unroll
    for (int q = 0; q < 1 + kNumTileBMs; ++q) s_wtot[q][wave] = incl[q];
    s_wtot[1 + kNumTileBMs][wave] = inv_w;
    s_wtot[2 + kNumTileBMs][wave] = drop_w;
  }
  __syncthreads();
  for (int i = tid; i < NC * E; i += 1024) p.chunk_hist[i] = h[i];  // chunk bases for the scatter pass
#pragma unroll
  for (int q = 0; q < 1 + kNumTileBMs; ++q) {
    int before = 0;
    for (int w = 0; w < wave; ++w) before += s_wtot[q][w];
    const int excl = before + incl[q] - val[q];
    if (e < E) {
      if (q == 0) {
        p.v.offsets[e] = excl;
        s_off[e] = excl;
      } else {
        p.v.tiles[(q - 1) * (E + 2) + e] = excl;
      }
    }
  }
  if (tid == 0) {
#pragma unroll
    for (int q = 0; q < 3 + kNumTileBMs; ++q) {
      int tot = 0;
      for (int w = 0; w < 16; ++w) tot += s_wtot[q][w];
      s_tot[q] = tot;
    }
  }
  __syncthreads();
  const int invalid_total = s_tot[1 + kNumTileBMs], dropped_total = s_tot[2 + kNumTileBMs];
  const int total_rows = s_tot[0];
  if (tid == 0) {
    s_off[E] = total_rows;
    p.v.offsets[E] = total_rows;
    for (int q = 0; q < kNumTileBMs; ++q) {
      const int bm = kTileBM[q];
      p.v.tiles[q * (E + 2) + E] = s_tot[q + 1];
      p.v.tiles[q * (E + 2) + E + 1] = s_tot[q + 1] + (p.shared_rows + bm - 1) / bm;
    }
    int32_t* hd = p.v.header;
    hd[HDR_T] = p.T;
    hd[HDR_K] = p.k;
    hd[HDR_E] = E;
    hd[HDR_C] = p.C;
    hd[HDR_P] = p.P;
    hd[HDR_ROWS_CAP] = p.rows_cap;
    hd[HDR_NMB] = p.n_mb;
    hd[HDR_MB] = p.mb;
    hd[HDR_DROPPED] = dropped_total;
    hd[HDR_INVALID] = invalid_total;
    hd[HDR_ROWS_TOTAL] = total_rows;
    hd[HDR_HASH] = p.hash;
    for (int i = HDR_HASH + 1; i < HDR_INTS; ++i) hd[i] = 0;
  }
  __syncthreads();
  // padding rows of every segment, and unused rows up to rows_cap(T), get -1
  if (e < E) {
    const int lo = s_off[e] + s_kept[e], hi = s_off[e + 1];
    for (int r = lo; r < hi; ++r) p.v.row_src[r] = -1;
  }
  for (int r = total_rows + tid; r < p.rows_cap; r += 1024) p.v.row_src[r] = -1;
  // single-minibatch sub-offsets: [offsets, offsets + kept]
  if (p.n_mb == 1 && e < E) {
    p.v.mb_offsets[e] = s_off[e];
    p.v.mb_offsets[E + e] = s_off[e] + s_kept[e];
  }
}

__global__ void __launch_bounds__(256) sched_scatter(SchedParams p, int nbits) {
  extern __shared__ int32_t lds[];  // [E] segment offsets, then [kWaves][E] running rank per expert
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int chunk = blockIdx.x * kWaves + wave;
  int32_t* offs = lds;
  int32_t* run = lds + p.E + wave * p.E;
  for (int e = threadIdx.x; e < p.E; e += 256) offs[e] = p.v.offsets[e];
  if (chunk < p.n_chunks)
    for (int e = lane; e < p.E; e += 64) run[e] = p.chunk_hist[(int64_t)chunk * p.E + e];
  __syncthreads();
  if (chunk >= p.n_chunks) return;  // whole waves exit together; no block barrier below
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int64_t base = (int64_t)chunk * p.iters * 64;
  for (int it0 = 0; it0 < p.iters; it0 += kScatterBatch) {
    int ev[kScatterBatch];
#pragma unroll
    for (int u = 0; u < kScatterBatch; ++u) {
      const int64_t a = base + (int64_t)(it0 + u) * 64 + lane;
      const int64_t v = a < p.n ? p.top[a] : -1;
      ev[u] = (v >= 0 && v < p.E) ? (int)v : -1;
    }
#pragma unroll
    for (int u = 0; u < kScatterBatch; ++u) {
      const int64_t a = base + (int64_t)(it0 + u) * 64 + lane;
      const int e = ev[u];
      const bool valid = e >= 0;
      // lanes holding the same expert id: intersect ballots bit by bit
      uint64_t same = ballot64(valid);
      for (int b = 0; b < nbits; ++b) {
        const bool bit = valid && ((e >> b) & 1);
        const uint64_t m = ballot64(bit);
        same &= bit ? m : ~m;
      }
      int q = 0;
      if (valid) q = run[e] + __popcll(same & lt_mask);
      __builtin_amdgcn_wave_barrier();
      // the highest lane of each group advances that expert's running count
      const bool last = valid && ((same >> lane) == 1ull);
      if (last) run[e] = q + 1;
      __builtin_amdgcn_s_waitcnt(0);
      __builtin_amdgcn_wave_barrier();
      if (a < p.n) {
        int slot = -1;
        if (valid && q < p.C) {
          const int row = offs[e] + q;
          p.v.row_src[row] = (int32_t)a;
          slot = row;
        }
        p.v.slot_row[a] = slot;
      }
    }
  }
}

// mb_offsets[b][e] = first row of expert e whose token >= b*mb (binary
// search over the token-ordered segment).
__global__ void __launch_bounds__(256) sched_minibatch(SchedParams p) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (p.n_mb + 1) * p.E) return;
  const int b = idx / p.E, e = idx - b * p.E;
  const int64_t bound = (int64_t)b * p.mb < p.T ? (int64_t)b * p.mb : p.T;
  int lo = p.v.offsets[e], hi = lo + p.v.kept[e];
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if ((int64_t)(p.v.row_src[mid] / p.k) < bound)
      lo = mid + 1;
    else
      hi = mid;
  }
  p.v.mb_offsets[idx] = lo;
}

}  // namespace

hipError_t launch_schedule(mok_workspace* ws, const int64_t* top, int64_t T, void* sched, hipStream_t s) {
  const mok_config& c = ws->cfg;
  SchedParams p;
  p.top = top;
  p.k = c.topk;
  p.E = c.num_experts;
  p.T = (int)T;
  p.n = T * c.topk;
  p.C = (int)capacity(T, c.capacity_multiplier);
  p.P = c.expert_pad;
  p.rows_cap = (int)rows_cap(c, T);
  p.n_mb = (int)n_minibatches(c, T);
  p.mb = c.minibatch_size > 0 ? c.minibatch_size : (int)T;
  p.hash = (int)config_hash(c);
  p.shared_rows = c.shared_intermediate > 0 ? (int)T : 0;
  p.v = sched_view(sched, ws->layout);
  p.chunk_hist = ws->chunk_hist;
  // chunk size: keep n_chunks * E within the count+scan kernel's LDS budget
  const int64_t lds_ints = 24 * 1024;
  int iters = kScatterBatch;
  while ((p.n + iters * 64 - 1) / (iters * 64) * (int64_t)p.E > lds_ints) iters *= 2;
  p.iters = iters;
  p.chunk_shift = 6;
  while ((1 << p.chunk_shift) < iters * 64) ++p.chunk_shift;
  p.n_chunks = (int)((p.n + iters * 64 - 1) / (iters * 64));
  if (p.n_chunks > ws->n_chunks_max) return hipErrorInvalidValue;  // sized at workspace creation
  if (p.E > kMaxE) return hipErrorInvalidValue;
  p.scan_group = 1;
  while (p.scan_group < 64 && p.scan_group * 2 * p.E <= 1024) p.scan_group *= 2;
  int nbits = 0;
  while ((1 << nbits) < p.E) ++nbits;
  {
    LaunchTimer t(ws, MOK_K_SCHED_SCAN, s);
    sched_count_scan<<<1, 1024, (size_t)p.n_chunks * p.E * sizeof(int32_t), s>>>(p);
    MOK_HIP_TRY(hipGetLastError());
  }
  if (p.n_chunks > 0) {
    LaunchTimer t(ws, MOK_K_SCHED_SCATTER, s);
    const int grid_w = (p.n_chunks + kWaves - 1) / kWaves;
    sched_scatter<<<grid_w, 256, (size_t)(kWaves + 1) * p.E * sizeof(int32_t), s>>>(p, nbits);
    MOK_HIP_TRY(hipGetLastError());
  }
  if (p.n_mb > 1) {
    LaunchTimer t(ws, MOK_K_SCHED_MINIBATCH, s);
    const int n = (p.n_mb + 1) * p.E;
    sched_minibatch<<<(n + 255) / 256, 256, 0, s>>>(p);
    MOK_HIP_TRY(hipGetLastError());
  }
  return hipSuccess;
}

}  // namespace mok
