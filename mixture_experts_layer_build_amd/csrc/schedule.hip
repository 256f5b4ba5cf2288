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
// Three launches, each a streaming pass (no atomics on global memory, so the
// bytes are identical from run to run):
//   1. count:   one wave per chunk of assignments -> per-chunk histograms.
//   2. scan:    one workgroup: per-expert exclusive scan over chunks (chunk
//               bases), counts, kept, padded offsets, tile prefix sums,
//               header, padding rows.
//   3. scatter: one wave per chunk: stable rank of each assignment inside its
//               expert from a wave ballot match plus the chunk base, then the
//               permutation (row_src) and its inverse (slot_row).
// (4. minibatch sub-offsets: binary search per (minibatch, expert); only
//     when the schedule has more than one minibatch.)
#include "device_common.h"
#include "mok_internal.h"

namespace mok {
namespace {

constexpr int kWaves = 4;  // waves per workgroup in the count/scatter kernels

struct SchedParams {
  const int64_t* top;
  int64_t n;          // T*k assignments
  int T, k, E, C, P;
  int iters;          // 64-assignment rounds per chunk
  int n_chunks;
  int rows_cap;       // rows_cap(T)
  int n_mb, mb;
  int hash;
  int shared_rows;    // T if the shared expert exists, else 0
  SchedView v;
  int32_t* chunk_hist;
  int32_t* chunk_invalid;
};

__global__ void __launch_bounds__(256) sched_count(SchedParams p) {
  extern __shared__ int32_t lds_hist[];  // [kWaves][E]
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int32_t* hist = lds_hist + wave * p.E;
  for (int e = lane; e < p.E; e += 64) hist[e] = 0;
  __syncthreads();
  const int chunk = blockIdx.x * kWaves + wave;
  int invalid = 0;
  if (chunk < p.n_chunks) {
    const int64_t base = (int64_t)chunk * p.iters * 64;
    for (int it = 0; it < p.iters; ++it) {
      const int64_t a = base + (int64_t)it * 64 + lane;
      if (a < p.n) {
        const int64_t e = p.top[a];
        if (e >= 0 && e < p.E)
          atomicAdd(&hist[e], 1);  // LDS atomics: counts do not depend on order
        else
          ++invalid;
      }
    }
  }
  // wave reduction of the invalid count
  for (int off = 32; off > 0; off >>= 1) invalid += __shfl_xor(invalid, off);
  __syncthreads();
  if (chunk < p.n_chunks) {
    for (int e = lane; e < p.E; e += 64) p.chunk_hist[(int64_t)chunk * p.E + e] = hist[e];
    if (lane == 0) p.chunk_invalid[chunk] = invalid;
  }
}

// One workgroup of 1024 threads.
__global__ void __launch_bounds__(1024) sched_scan(SchedParams p) {
  extern __shared__ int32_t lds[];  // [n_chunks * E] histogram copy, then scratch
  __shared__ int32_t s_pad[1024];
  __shared__ int32_t s_tot[kNumTileBMs + 3];
  const int tid = threadIdx.x;
  const int E = p.E, NC = p.n_chunks;
  int32_t* h = lds;
  for (int i = tid; i < NC * E; i += 1024) h[i] = p.chunk_hist[i];
  __syncthreads();
  // per-expert exclusive scan over chunks (in LDS), then totals
  for (int e = tid; e < E; e += 1024) {
    int run = 0;
    for (int c = 0; c < NC; ++c) {
      const int v = h[c * E + e];
      h[c * E + e] = run;
      run += v;
    }
    p.v.counts[e] = run;
    const int kept = run < p.C ? run : p.C;
    p.v.kept[e] = kept;
  }
  __syncthreads();
  for (int i = tid; i < NC * E; i += 1024) p.chunk_hist[i] = h[i];  // chunk bases for the scatter pass
  // exclusive scan of padded sizes over experts (sequential in chunks of 1024)
  if (tid < kNumTileBMs + 3) s_tot[tid] = 0;
  __syncthreads();
  for (int e0 = 0; e0 < E; e0 += 1024) {
    const int e = e0 + tid;
    int kept = 0, cnt = 0;
    if (e < E) {
      kept = p.v.kept[e];
      cnt = p.v.counts[e];
    }
    const int padded = (kept + p.P - 1) / p.P * p.P;
    // scans: padded rows, then tiles for each BM
    for (int q = 0; q < 1 + kNumTileBMs; ++q) {
      const int val = q == 0 ? padded : (padded + kTileBM[q - 1] - 1) / kTileBM[q - 1];
      s_pad[tid] = val;
      __syncthreads();
      for (int off = 1; off < 1024; off <<= 1) {
        const int t = tid >= off ? s_pad[tid - off] : 0;
        __syncthreads();
        s_pad[tid] += t;
        __syncthreads();
      }
      const int excl = s_pad[tid] - val + s_tot[q];
      if (e < E) {
        if (q == 0)
          p.v.offsets[e] = excl;
        else
          p.v.tiles[(q - 1) * (E + 2) + e] = excl;
      }
      __syncthreads();
      if (tid == 1023) s_tot[q] = excl + val;
      __syncthreads();
    }
    // dropped = sum(count - kept)
    s_pad[tid] = cnt - kept;
    __syncthreads();
    for (int off = 512; off > 0; off >>= 1) {
      if (tid < off) s_pad[tid] += s_pad[tid + off];
      __syncthreads();
    }
    if (tid == 0) s_tot[kNumTileBMs + 1] += s_pad[0];
    __syncthreads();
  }
  // invalid = sum over chunks
  s_pad[tid] = 0;
  for (int c = tid; c < NC; c += 1024) s_pad[tid] += p.chunk_invalid[c];
  __syncthreads();
  for (int off = 512; off > 0; off >>= 1) {
    if (tid < off) s_pad[tid] += s_pad[tid + off];
    __syncthreads();
  }
  const int total_rows = s_tot[0];
  if (tid == 0) {
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
    hd[HDR_DROPPED] = s_tot[kNumTileBMs + 1];
    hd[HDR_INVALID] = s_pad[0];
    hd[HDR_ROWS_TOTAL] = total_rows;
    hd[HDR_HASH] = p.hash;
    for (int i = HDR_HASH + 1; i < HDR_INTS; ++i) hd[i] = 0;
  }
  __syncthreads();
  // padding rows of every segment, and unused rows up to rows_cap(T), get -1
  for (int e = tid; e < E; e += 1024) {
    const int lo = p.v.offsets[e] + p.v.kept[e], hi = p.v.offsets[e + 1];
    for (int r = lo; r < hi; ++r) p.v.row_src[r] = -1;
  }
  for (int r = total_rows + tid; r < p.rows_cap; r += 1024) p.v.row_src[r] = -1;
  // single-minibatch sub-offsets: [offsets, offsets + kept]
  if (p.n_mb == 1) {
    for (int e = tid; e < E; e += 1024) {
      p.v.mb_offsets[e] = p.v.offsets[e];
      p.v.mb_offsets[E + e] = p.v.offsets[e] + p.v.kept[e];
    }
  }
}

__global__ void __launch_bounds__(256) sched_scatter(SchedParams p, int nbits) {
  extern __shared__ int32_t lds_run[];  // [kWaves][E] running rank per expert
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int chunk = blockIdx.x * kWaves + wave;
  if (chunk >= p.n_chunks) return;  // whole waves exit together; no block barrier below
  int32_t* run = lds_run + wave * p.E;
  for (int e = lane; e < p.E; e += 64) run[e] = p.chunk_hist[(int64_t)chunk * p.E + e];
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int64_t base = (int64_t)chunk * p.iters * 64;
  for (int it = 0; it < p.iters; ++it) {
    const int64_t a = base + (int64_t)it * 64 + lane;
    int e = -1;
    if (a < p.n) {
      const int64_t ev = p.top[a];
      e = (ev >= 0 && ev < p.E) ? (int)ev : -1;
    }
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
        const int row = p.v.offsets[e] + q;
        p.v.row_src[row] = (int32_t)a;
        slot = row;
      }
      p.v.slot_row[a] = slot;
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
  p.chunk_invalid = ws->chunk_invalid;
  // chunk size: keep n_chunks * E within the scan kernel's LDS budget
  const int64_t lds_ints = 24 * 1024;
  int iters = 16;
  while ((p.n + iters * 64 - 1) / (iters * 64) * (int64_t)p.E > lds_ints) iters *= 2;
  p.iters = iters;
  p.n_chunks = (int)((p.n + iters * 64 - 1) / (iters * 64));
  if (p.n_chunks > ws->n_chunks_max) return hipErrorInvalidValue;  // sized at workspace creation
  int nbits = 0;
  while ((1 << nbits) < p.E) ++nbits;
  const int grid_w = (p.n_chunks + kWaves - 1) / kWaves;
  const size_t lds_waves = (size_t)kWaves * p.E * sizeof(int32_t);
  if (p.n_chunks > 0) {
    LaunchTimer t(ws, MOK_K_SCHED_COUNT, s);
    sched_count<<<grid_w, 256, lds_waves, s>>>(p);
    MOK_HIP_TRY(hipGetLastError());
  }
  {
    LaunchTimer t(ws, MOK_K_SCHED_SCAN, s);
    sched_scan<<<1, 1024, (size_t)p.n_chunks * p.E * sizeof(int32_t), s>>>(p);
    MOK_HIP_TRY(hipGetLastError());
  }
  if (p.n_chunks > 0) {
    LaunchTimer t(ws, MOK_K_SCHED_SCATTER, s);
    sched_scatter<<<grid_w, 256, lds_waves, s>>>(p, nbits);
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
