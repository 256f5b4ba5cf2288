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
// Two launches (no atomics on global memory, so the bytes are identical from
// run to run):
//   1. count: workgroup b counts the assignments of chunks [16 b, 16 b + 16)
//      into per-chunk expert histograms in LDS (LDS atomics: counts do not
//      depend on the order of the adds) and stores them.
//   2. scan + scatter: every workgroup reads the whole chunk x expert table,
//      derives per-expert totals, kept counts, padded offsets and the rank
//      base of each of its 16 chunks itself (no grid-wide wait), then one
//      wave per chunk ranks each assignment inside its expert from a wave
//      ballot match plus that base and writes the permutation (row_src) and
//      its inverse (slot_row). Workgroup 0 also writes counts, kept, offsets,
//      tile prefix sums and the header; the padding rows are split over all
//      workgroups.
// (3. minibatch sub-offsets: binary search per (minibatch, expert); only
//     when the schedule has more than one minibatch.)
#include "device_common.h"
#include "mok_internal.h"

namespace mok {
namespace {

constexpr int kWaves = 16;       // waves per workgroup in both passes
constexpr int kThreads = kWaves * 64;
constexpr int kCountChunks = 16; // chunks per workgroup in the count pass
constexpr int kScatterChunks = 4;  // chunks per workgroup in the scatter pass: one wave each, one per SIMD
constexpr int kMaxE = 1024;      // the largest expert count a workspace accepts
constexpr int kCountBatch = 8;   // loads in flight per thread while counting
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
  int32_t* chunk_hist;  // [n_chunks][E] per-chunk expert counts
};

// Pass 1. Workgroup b: histograms of chunks [kCountChunks b, kCountChunks (b + 1)).
__global__ void __launch_bounds__(kThreads) sched_count(SchedParams p) {
  extern __shared__ int32_t lds[];  // [kCountChunks][E]
  const int tid = threadIdx.x, E = p.E;
  const int c0 = blockIdx.x * kCountChunks;
  const int nc = min(kCountChunks, p.n_chunks - c0);
  for (int i = tid; i < nc * E; i += kThreads) lds[i] = 0;
  __syncthreads();
  const int64_t a_lo = (int64_t)c0 << p.chunk_shift;
  const int64_t a_hi = min(p.n, (int64_t)(c0 + nc) << p.chunk_shift);
  for (int64_t a0 = a_lo + tid; a0 < a_hi; a0 += (int64_t)kThreads * kCountBatch) {
    int64_t ev[kCountBatch];
#pragma unroll
    for (int u = 0; u < kCountBatch; ++u) {
      const int64_t a = a0 + (int64_t)kThreads * u;
      ev[u] = a < a_hi ? p.top[a] : -1;
    }
#pragma unroll
    for (int u = 0; u < kCountBatch; ++u) {
      const int64_t a = a0 + (int64_t)kThreads * u;
      if (a < a_hi && ev[u] >= 0 && ev[u] < E) atomicAdd(&lds[(int)((a - a_lo) >> p.chunk_shift) * E + (int)ev[u]], 1);
    }
  }
  __syncthreads();
  for (int i = tid; i < nc * E; i += kThreads) p.chunk_hist[(int64_t)c0 * E + i] = lds[i];
}

// Pass 2. Workgroup b: the scans (every workgroup, all its waves), then the
// scatter of chunks [kScatterChunks b, kScatterChunks (b + 1)), wave w < kScatterChunks
// taking chunk kScatterChunks b + w (one scatter wave per SIMD).
__global__ void __launch_bounds__(kThreads) sched_scan_scatter(SchedParams p, int nbits) {
  extern __shared__ int32_t lds[];  // [E] segment offsets, then [kScatterChunks][E] running rank per expert
  __shared__ int32_t s_part[kThreads];  // per chunk run: all chunks
  __shared__ int32_t s_pre[kThreads];   // per chunk run: chunks before this workgroup's first
  __shared__ int32_t s_cnt[kMaxE];
  __shared__ int32_t s_base[kMaxE];
  __shared__ int32_t s_wtot[kNumTileBMs + 3][kWaves];  // per-wave totals: scans, counts, dropped
  __shared__ int32_t s_tot[kNumTileBMs + 3];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = p.E, NC = p.n_chunks;
  const int c_first = blockIdx.x * kScatterChunks;
  int32_t* offs = lds;
  int32_t* run_all = lds + E;
  // this workgroup's own chunk counts of expert tid (E <= kThreads), loaded
  // first so that their latency overlaps the scan's loads
  int own[kScatterChunks];
#pragma unroll
  for (int w = 0; w < kScatterChunks; ++w)
    own[w] = (tid < E && c_first + w < NC) ? p.chunk_hist[(int64_t)(c_first + w) * E + tid] : 0;
  // per-expert totals over all chunks and over the chunks before c_first:
  // G = p.scan_group runs of contiguous chunks per expert, run q of expert e
  // on thread q * E + e (a wave's lanes read consecutive experts of a chunk)
  {
    constexpr int kB = 8;  // loads in flight per thread
    const int G = p.scan_group, part = tid / E, ge = tid - part * E;
    const int per = (NC + G - 1) / G;
    const int r0 = min(NC, part * per), r1 = part < G ? min(NC, r0 + per) : r0;
    int tot = 0, pre = 0;
    for (int c = r0; c < r1; c += kB) {
      int v[kB];
#pragma unroll
      for (int u = 0; u < kB; ++u) v[u] = c + u < r1 ? p.chunk_hist[(int64_t)(c + u) * E + ge] : 0;
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        tot += v[u];
        pre += c + u < c_first ? v[u] : 0;
      }
    }
    s_part[tid] = tot;
    s_pre[tid] = pre;
    __syncthreads();
    for (int e = tid; e < E; e += kThreads) {
      int t = 0, b = 0;
      for (int q = 0; q < G; ++q) {
        t += s_part[q * E + e];
        b += s_pre[q * E + e];
      }
      s_cnt[e] = t;
      s_base[e] = b;
    }
  }
  __syncthreads();
  // running rank of each expert at the start of each of this workgroup's chunks
  if (tid < E) {
    int acc = s_base[tid];
#pragma unroll
    for (int w = 0; w < kScatterChunks; ++w) {
      run_all[w * E + tid] = acc;
      acc += own[w];
    }
  }
  // kept, padded rows and tile counts per expert (one expert per thread,
  // E <= 1024), exclusive scans over experts: wave scans, then one pass over
  // the wave totals
  const int e = tid;
  int cnt = 0, kept = 0;
  if (e < E) {
    cnt = s_cnt[e];
    kept = cnt < p.C ? cnt : p.C;
  }
  const int padded = (kept + p.P - 1) / p.P * p.P;
  // GEMM tiles cover the kept rows only: counted from the padded length, a
  // pad that does not divide the tile height (P = 96: 250 kept rows, 288
  // padded) would give a last tile with no valid row
  int val[1 + kNumTileBMs], incl[1 + kNumTileBMs];
#pragma unroll
  for (int q = 0; q < 1 + kNumTileBMs; ++q) {
    val[q] = q == 0 ? padded : (kept + kTileBM[q - 1] - 1) / kTileBM[q - 1];
    incl[q] = wave_inclusive_scan(val[q], lane);
  }
  const int cnt_w = wave_sum(cnt), drop_w = wave_sum(cnt - kept);
  if (lane == 63) {
#pragma unroll
    for (int q = 0; q < 1 + kNumTileBMs; ++q) s_wtot[q][wave] = incl[q];
    s_wtot[1 + kNumTileBMs][wave] = cnt_w;
    s_wtot[2 + kNumTileBMs][wave] = drop_w;
  }
  __syncthreads();
  const bool writer = blockIdx.x == 0;
#pragma unroll
  for (int q = 0; q < 1 + kNumTileBMs; ++q) {
    int before = 0;
    for (int w = 0; w < wave; ++w) before += s_wtot[q][w];
    const int excl = before + incl[q] - val[q];
    if (e < E) {
      if (q == 0) {
        offs[e] = excl;
        if (writer) p.v.offsets[e] = excl;
      } else if (writer) {
        p.v.tiles[(q - 1) * (E + 2) + e] = excl;
      }
    }
  }
  if (tid == 0) {
#pragma unroll
    for (int q = 0; q < 3 + kNumTileBMs; ++q) {
      int tot = 0;
      for (int w = 0; w < kWaves; ++w) tot += s_wtot[q][w];
      s_tot[q] = tot;
    }
  }
  __syncthreads();
  const int total_rows = s_tot[0];
  if (writer) {
    if (e < E) {
      p.v.counts[e] = cnt;
      p.v.kept[e] = kept;
      if (p.n_mb == 1) {  // single-minibatch sub-offsets: [offsets, offsets + kept]
        p.v.mb_offsets[e] = offs[e];
        p.v.mb_offsets[E + e] = offs[e] + kept;
      }
    }
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
      hd[HDR_DROPPED] = s_tot[2 + kNumTileBMs];
      hd[HDR_INVALID] = (int)(p.n - s_tot[1 + kNumTileBMs]);  // assignments no expert counted
      hd[HDR_ROWS_TOTAL] = total_rows;
      hd[HDR_HASH] = p.hash;
      for (int i = HDR_HASH + 1; i < HDR_INTS; ++i) hd[i] = 0;
    }
  }
  // padding rows of every segment (experts split over the workgroups), and
  // unused rows up to rows_cap(T), get -1
  if (e < E && e % gridDim.x == blockIdx.x) {
    const int hi = e + 1 < E ? offs[e + 1] : total_rows;
    for (int r = offs[e] + kept; r < hi; ++r) p.v.row_src[r] = -1;
  }
  for (int r = total_rows + blockIdx.x * kThreads + tid; r < p.rows_cap; r += gridDim.x * kThreads)
    p.v.row_src[r] = -1;
  // scatter: wave w ranks chunk c_first + w
  const int chunk = c_first + wave;
  if (wave >= kScatterChunks || chunk >= NC) return;  // whole waves exit; no barrier below
  int32_t* run = run_all + wave * E;
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
      const int ex = ev[u];
      const bool valid = ex >= 0;
      // lanes holding the same expert id: intersect ballots bit by bit
      uint64_t same = ballot64(valid);
      for (int b = 0; b < nbits; ++b) {
        const bool bit = valid && ((ex >> b) & 1);
        const uint64_t m = ballot64(bit);
        same &= bit ? m : ~m;
      }
      int q = 0;
      if (valid) q = run[ex] + __popcll(same & lt_mask);
      __builtin_amdgcn_wave_barrier();
      // the highest lane of each group advances that expert's running count
      const bool last = valid && ((same >> lane) == 1ull);
      if (last) run[ex] = q + 1;
      __builtin_amdgcn_s_waitcnt(0);
      __builtin_amdgcn_wave_barrier();
      if (a < p.n) {
        int slot = -1;
        if (valid && q < p.C) {
          const int row = offs[ex] + q;
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

// One pass of the token ring: the schedule of the tokens [t0, t0 + T_p),
// t0 = pass * M, cut out of the whole batch's schedule, with its rows
// packed. Expert e keeps the rows of those tokens that the whole batch kept,
// rows [lo_e, hi_e) of its segment (the sub-offsets at the pass's
// boundaries), in the same order; they become rows [offq_e, offq_e + n_e)
// of the pass, segments padded to P. Assignment ids and slot indices are
// made relative to t0, so that the pass runs with x, the router weights and
// the output offset by t0 tokens. Every workgroup derives the per-expert
// tables itself; workgroup 0 writes them; all share the rows and slots.
struct SliceParams {
  SchedView g;        // the whole batch's schedule
  SchedView q;        // the pass's
  int E, k, P, M;
  int steps;          // sub-offset steps per pass
  int pass;
  int rows_cap_q;     // rows of the pass layout
  int hash_q;         // the pass configuration's hash
  int shared;         // 1 with a shared expert
};

__global__ void __launch_bounds__(kThreads) sched_slice(SliceParams p) {
  __shared__ int32_t lo[kMaxE], kp[kMaxE], offq[kMaxE + 1], goff[kMaxE + 1];
  __shared__ int32_t s_wtot[1 + kNumTileBMs][kWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = p.E, k = p.k;
  if (!sched_matches(p.g.header, p.g.hash, p.g.status)) {
    // a foreign schedule: the pass's header gets a hash no launch expects,
    // so that the pass's launches return too
    if (blockIdx.x == 0 && tid == 0) p.q.header[HDR_HASH] = p.hash_q ^ 0x40000000;
    return;
  }
  const int T = p.g.header[HDR_T], n_mb = p.g.header[HDR_NMB];
  const int t0 = min(T, p.pass * p.M);
  const int Tp = min(p.M, T - t0);
  const int i0 = min(p.pass * p.steps, n_mb), i1 = min((p.pass + 1) * p.steps, n_mb);
  int n = 0;
  if (tid < E) {
    const int l = p.g.mb_offsets[i0 * E + tid];
    n = p.g.mb_offsets[i1 * E + tid] - l;
    lo[tid] = l;
    kp[tid] = n;
  }
  if (tid <= E) goff[tid] = p.g.offsets[tid];
  // exclusive scans over experts: padded rows, and the 32/64/128/256-row tiles
  const int padded = (n + p.P - 1) / p.P * p.P;
  int val[1 + kNumTileBMs], incl[1 + kNumTileBMs];
#pragma unroll
  for (int t = 0; t < 1 + kNumTileBMs; ++t) {
    val[t] = t == 0 ? padded : (n + kTileBM[t - 1] - 1) / kTileBM[t - 1];
    incl[t] = wave_inclusive_scan(val[t], lane);
  }
  if (lane == 63) {
#pragma unroll
    for (int t = 0; t < 1 + kNumTileBMs; ++t) s_wtot[t][wave] = incl[t];
  }
  __syncthreads();
  int tot[1 + kNumTileBMs];
#pragma unroll
  for (int t = 0; t < 1 + kNumTileBMs; ++t) {
    int before = 0, all = 0;
    for (int w = 0; w < kWaves; ++w) {
      before += w < wave ? s_wtot[t][w] : 0;
      all += s_wtot[t][w];
    }
    tot[t] = all;
    const int excl = before + incl[t] - val[t];
    if (tid < E) {
      if (t == 0) offq[tid] = excl;
      else if (blockIdx.x == 0) p.q.tiles[(t - 1) * (E + 2) + tid] = excl;
    }
  }
  if (tid == 0) offq[E] = tot[0];
  __syncthreads();
  const int rows_total = tot[0];
  if (blockIdx.x == 0) {
    if (tid < E) {
      p.q.counts[tid] = kp[tid];
      p.q.kept[tid] = kp[tid];
      p.q.offsets[tid] = offq[tid];
      p.q.mb_offsets[tid] = offq[tid];
      p.q.mb_offsets[E + tid] = offq[tid] + kp[tid];
    }
    if (tid == 0) {
      p.q.offsets[E] = rows_total;
#pragma unroll
      for (int t = 0; t < kNumTileBMs; ++t) {
        const int bm = kTileBM[t];
        p.q.tiles[t * (E + 2) + E] = tot[t + 1];
        p.q.tiles[t * (E + 2) + E + 1] = tot[t + 1] + (p.shared ? (Tp + bm - 1) / bm : 0);
      }
      int32_t* hd = p.q.header;
      hd[HDR_T] = Tp;
      hd[HDR_K] = k;
      hd[HDR_E] = E;
      hd[HDR_C] = p.M;
      hd[HDR_P] = p.P;
      hd[HDR_ROWS_CAP] = min(Tp * k, E * Tp) + E * (p.P - 1);
      hd[HDR_NMB] = 1;
      hd[HDR_MB] = Tp;
      hd[HDR_DROPPED] = 0;
      hd[HDR_INVALID] = 0;
      hd[HDR_ROWS_TOTAL] = rows_total;
      hd[HDR_HASH] = p.hash_q;
      for (int i = HDR_HASH + 1; i < HDR_INTS; ++i) hd[i] = 0;
    }
  }
  // largest e with a[e] <= v (segments that start at the same row: the last,
  // the only one that can hold it)
  auto search = [&](const int32_t* a, int v) {
    int l = 0, h = E;
    while (h - l > 1) {
      const int mid = (l + h) >> 1;
      if (a[mid] <= v) l = mid; else h = mid;
    }
    return l;
  };
  const int stride = gridDim.x * kThreads;
  for (int r = blockIdx.x * kThreads + tid; r < p.rows_cap_q; r += stride) {
    int src = -1;
    if (r < rows_total) {
      const int e = search(offq, r);
      const int i = r - offq[e];
      if (i < kp[e]) src = p.g.row_src[lo[e] + i] - t0 * k;
    }
    p.q.row_src[r] = src;
  }
  for (int a = blockIdx.x * kThreads + tid; a < Tp * k; a += stride) {
    const int r = p.g.slot_row[(int64_t)t0 * k + a];
    int s = -1;
    if (r >= 0) {
      const int e = search(goff, r);
      s = offq[e] + (r - lo[e]);
    }
    p.q.slot_row[a] = s;
  }
}

}  // namespace

hipError_t launch_sched_slice(mok_workspace* ws, const void* sched, int pass, void* pass_sched, hipStream_t s) {
  const mok_config& c = ws->cfg;
  const mok_config qc = pass_config(c);
  const Layout QL = schedule_layout(qc);
  SliceParams p;
  p.g = sched_view(const_cast<void*>(sched), ws->layout);
  p.g.hash = (int)config_hash(c);
  p.g.status = ws->status;
  p.q = sched_view(pass_sched, QL);
  p.E = c.num_experts;
  p.k = c.topk;
  p.P = c.expert_pad;
  p.M = c.macrobatch_size;
  p.steps = (int)(c.macrobatch_size / sub_offset_tokens(c));
  p.pass = pass;
  p.rows_cap_q = (int)QL.rows_cap_max;
  p.hash_q = (int)config_hash(qc);
  p.shared = c.shared_intermediate > 0;
  if (p.E > kMaxE) return hipErrorInvalidValue;
  const int64_t work = std::max<int64_t>(QL.rows_cap_max, (int64_t)c.macrobatch_size * c.topk);
  const int grid = (int)std::min<int64_t>((work + kThreads - 1) / kThreads, 256);
  LaunchTimer t(ws, MOK_K_SCHED_SLICE, s);
  sched_slice<<<grid, kThreads, 0, s>>>(p);
  return hipGetLastError();
}

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
  p.mb = sub_offset_tokens(c) > 0 ? (int)sub_offset_tokens(c) : (int)T;
  p.hash = (int)config_hash(c);
  p.shared_rows = c.shared_intermediate > 0 ? (int)T : 0;
  p.v = sched_view(sched, ws->layout);
  p.chunk_hist = ws->chunk_hist;
  // chunk size: n_chunks * E within the workspace's chunk table (and each
  // scan thread's share of it small)
  const int64_t table_ints = 24 * 1024;
  int iters = kScatterBatch;
  while ((p.n + iters * 64 - 1) / (iters * 64) * (int64_t)p.E > table_ints) iters *= 2;
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
  const int count_groups = (p.n_chunks + kCountChunks - 1) / kCountChunks;
  const int scatter_groups = (p.n_chunks + kScatterChunks - 1) / kScatterChunks;
  if (count_groups > 0) {
    LaunchTimer t(ws, MOK_K_SCHED_COUNT, s);
    sched_count<<<count_groups, kThreads, (size_t)kCountChunks * p.E * sizeof(int32_t), s>>>(p);
    MOK_HIP_TRY(hipGetLastError());
  }
  {
    // at least one workgroup: an empty batch still gets its header
    LaunchTimer t(ws, MOK_K_SCHED_SCATTER, s);
    sched_scan_scatter<<<scatter_groups > 0 ? scatter_groups : 1, kThreads,
                         (size_t)(kScatterChunks + 1) * p.E * sizeof(int32_t), s>>>(p, nbits);
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
