/*
 * mok.h -- C ABI of the MoE-layer hot path for AMD Instinct MI355X (gfx950).
 *
 * One GPU's share of a mixture-of-experts layer: a deterministic schedule
 * built from top-k routing, a grouped SwiGLU expert MLP with an always-on
 * shared expert, and a router-weighted combine back to token order, forward
 * and backward, in BF16 and in MXFP8 (E4M3 elements, one E8M0 scale per 32
 * elements along the contraction dimension).
 *
 * Pages this interface follows (titles as published):
 *   [R] "Mixture-of-Kittens: a deterministic MoE megakernel for NVL72 racks"
 *   [A] "nemo_automodel.components.moe.mok_experts" (NeMo AutoModel API docs)
 *   [B] the moses-y.github.io review "mixture-of-kittens"
 *
 * Conventions for every call:
 *   - Pointers named as device pointers must point to device memory of the
 *     workspace's device; every tensor is dense and row-major ("contiguous",
 *     [A] _MoKRuntime.forward parameters). bf16 tensors are passed as raw
 *     16-bit patterns (void*).
 *   - `stream` is a hipStream_t (NULL = the default stream). Calls that take a
 *     stream only enqueue work: they never synchronise with the host and never
 *     read device data on the host ([B] "What This Does": no CPU-GPU
 *     synchronization; [R] "What Mixture-of-Kittens solves").
 *   - Argument, shape and configuration errors are detected on the host
 *     before anything is enqueued and returned synchronously; nothing is
 *     enqueued when a call returns an error. A failed HIP launch returns
 *     MOK_ERR_HIP.
 *   - The library touches no device when it is loaded; a device is first used
 *     by mok_workspace_create ([A] _load_mok_functional: loading the extension
 *     before the process has picked its GPU leaves a stray context).
 *   - A workspace may be used by one stream at a time; calls that overlap on
 *     one workspace race on its scratch memory.
 */
#ifndef MOK_H_
#define MOK_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOK_VERSION_MAJOR 0
#define MOK_VERSION_MINOR 1

typedef enum mok_status {
  MOK_OK = 0,
  MOK_ERR_INVALID_ARGUMENT = 1, /* null pointer, negative or inconsistent size */
  MOK_ERR_UNSUPPORTED = 2,      /* shape outside the kernels' contract ([A] _validate_model_mok_config) */
  MOK_ERR_CONFIG_MISMATCH = 3,  /* schedule/context built for another config or token count */
  MOK_ERR_BUFFER_TOO_SMALL = 4, /* caller buffer smaller than the *_bytes query says */
  MOK_ERR_HIP = 5               /* a HIP runtime call or launch failed */
} mok_status;

typedef enum mok_mode {
  MOK_MODE_BF16 = 0,  /* bf16 operands, fp32 accumulation */
  MOK_MODE_MXFP8 = 1  /* E4M3 operands with E8M0 block scales, fp32 accumulation ([R] "Tuning the five hyperparameters before production") */
} mok_mode;

/*
 * Layer configuration: the single-GPU reading of the pages' MoKConfig
 * ([R] "The two API layers and the schedule object", "Tuning the five
 * hyperparameters before production"). Set struct_size = sizeof(mok_config).
 *
 * Contract (MOK_ERR_UNSUPPORTED otherwise, MOK_ERR_INVALID_ARGUMENT for
 * negative sizes): hidden % 128 == 0;
 * intermediate % 64 == 0 and shared_intermediate % 64 == 0 (0 = no shared
 * expert); 1 <= num_experts <= 1024; 1 <= topk <= 64; expert_pad a positive
 * multiple of 32 (MXFP8 backward needs 32-row blocks inside one expert);
 * max_tokens >= 1 with max_tokens * topk < 2^31. Every operand a kernel
 * reads stays below 2 GiB: (max_tokens + 127) * max(hidden, intermediate,
 * shared_intermediate, 256) * 2 < 2^31, intermediate * hidden * 2 < 2^31 and
 * shared_intermediate * hidden * 2 < 2^31; and the schedule's row bound
 * rows_cap_max + max_tokens < 2^31.
 */
typedef struct mok_config {
  uint32_t struct_size;
  int32_t hidden;               /* H */
  int32_t intermediate;         /* I: routed expert intermediate size */
  int32_t num_experts;          /* E: local experts (all experts, on one GPU) */
  int32_t topk;                 /* k */
  int32_t shared_intermediate;  /* I_s: shared expert intermediate size, 0 = none */
  int64_t max_tokens;           /* T_max: sizes every buffer for the worst case */
  float capacity_multiplier;    /* per-expert capacity C = min(T, ceil(mult * T)) ([R] "Tuning...": schedule_capacity_multiplier) */
  int32_t expert_pad;           /* P: each expert segment padded to a multiple of P rows ([R] "Tuning...": expert padding) */
  int32_t minibatch_size;       /* tokens per minibatch: the schedule's sub-offsets, and the granularity of the
                                   forward's minibatch pipeline; 0 = one minibatch ([R] "Tuning...": minibatch_size) */
  int32_t num_mover_wgs;        /* mover workgroups of the forward's minibatch pipeline (rounded down to a multiple
                                   of 8, at most the compute units less 32); 0 = no pipeline. With 0 <
                                   minibatch_size < max_tokens, num_mover_wgs >= 8 and num_experts <= 256, the down
                                   GEMM and the combine run as one launch of one workgroup per compute unit: the
                                   others run the down tiles minibatch by minibatch and count each finished tile,
                                   and these combine minibatch b as soon as its count is complete, while the tiles
                                   of later minibatches run ([R] "Tuning...": fwd_num_comm_sms, minibatch_size).
                                   A mover's wait is bounded (about 2 s in all); one that runs out of time is
                                   counted in mok_workspace_read_status. The result bits do not depend on either
                                   value. */
  float swiglu_limit;           /* SwiGLU input limit L ([A] _MoKRuntime(mok_config, swiglu_limit); the pages give
                                   no formula): L > 0 computes h = silu(min(g, L)) * clamp(u, -L, L), and the
                                   backward passes no gradient where a clamp is active (g > L, |u| > L);
                                   0 or +inf = no limit. Negative or NaN: MOK_ERR_INVALID_ARGUMENT. */
  int32_t macrobatch_size;      /* tokens per pass of the workspace's token ring ([R] "Tuning...": macrobatch_size, the
                                   token ring buffer; a size at least max_tokens means the ring is used once).
                                   0 or >= max_tokens: one pass. Otherwise mok_forward streams the batch through
                                   scratch sized for macrobatch_size tokens, macrobatch by macrobatch, with the
                                   whole batch's schedule (capacity and drops as in one pass): the output bits are
                                   those of one pass. Requires forward_only = 1 (a backward contracts each expert's
                                   weight gradient over the whole batch), num_experts >= topk and, when
                                   minibatch_size > 0, a multiple of it (MOK_ERR_UNSUPPORTED otherwise). Each pass
                                   adds one small kernel (its schedule) and runs without the minibatch pipeline. */
  int32_t forward_only;         /* 1: an inference workspace, with no backward scratch (mok_backward returns
                                   MOK_ERR_UNSUPPORTED, mok_forward takes no context); 0: training */
} mok_config;

/* Routed and shared expert weights, layouts of [A] _MoKRuntime.forward:
 * gate/up [E, I, H], down [E, H, I], shared gate/up [I_s, H], shared down
 * [H, I_s]. In BF16 mode the data pointers are bf16 and the scale pointers
 * are ignored. In MXFP8 mode the data pointers are E4M3 bytes of the same
 * shapes and the scales are E8M0 bytes with one scale per 32 elements along
 * the last dimension (the contraction dimension of the forward GEMMs), as
 * written by mok_mxfp8_quantize(axis = 1): gate/up scales [E*I, H/32], down
 * [E*H, I/32], shared gate/up [I_s, H/32], shared down [H, I_s/32]. Shared
 * pointers must be NULL iff shared_intermediate == 0. */
typedef struct mok_weights {
  const void* routed_gate;
  const void* routed_up;
  const void* routed_down;
  const void* shared_gate;
  const void* shared_up;
  const void* shared_down;
  const uint8_t* routed_gate_scale;
  const uint8_t* routed_up_scale;
  const uint8_t* routed_down_scale;
  const uint8_t* shared_gate_scale;
  const uint8_t* shared_up_scale;
  const uint8_t* shared_down_scale;
} mok_weights;

/* Gradients written by mok_backward ([A] _MoKRuntime.backward: one gradient
 * per float input; the integer expert ids get none). dx bf16 [T, H];
 * d_router_weights fp32 [T, k] (0 for dropped or invalid assignments);
 * d_routed_gate/up bf16 [E, I, H]; d_routed_down bf16 [E, H, I];
 * d_shared_gate/up bf16 [I_s, H]; d_shared_down bf16 [H, I_s] (NULL iff
 * shared_intermediate == 0). Every element is written (experts that receive
 * no rows get zero weight gradients). */
typedef struct mok_grads {
  void* dx;
  float* d_router_weights;
  void* d_routed_gate;
  void* d_routed_up;
  void* d_routed_down;
  void* d_shared_gate;
  void* d_shared_up;
  void* d_shared_down;
} mok_grads;

/* Byte offsets of the schedule's fields inside the caller's schedule buffer
 * (every field int32, little endian). The schedule is the pages' "schedule
 * object": built once per layer and step from routing, before any expert
 * math, and passed unchanged to forward and backward ([R] "The two API
 * layers and the schedule object"). Fields (this call's token count T):
 *   header[16]: [0] T, [1] k, [2] E, [3] C, [4] P, [5] rows_cap(T),
 *               [6] n_mb, [7] minibatch size, [8] dropped, [9] invalid,
 *               [10] total padded rows = offsets[E], [11] config hash,
 *               [12..15] reserved
 *   counts[E]     valid assignments per expert
 *   kept[E]       min(counts, C)
 *   offsets[E+1]  exclusive prefix sum of kept rounded up to P
 *   mb_offsets[(n_mb_max+1)*E]  row where minibatch b of expert e starts
 *   row_src[rows_cap_max]  flat assignment a = t*k + j feeding each row, -1 for
 *                          padding and unused rows (valid up to rows_cap(T))
 *   slot_row[T_max*k]      row of assignment a, -1 if dropped or invalid
 *   tiles[4][E+2]          internal GEMM tile prefix sums (not part of the
 *                          method's result) */
typedef struct mok_schedule_layout {
  size_t total_bytes;
  size_t header;
  size_t counts;
  size_t kept;
  size_t offsets;
  size_t mb_offsets;
  size_t row_src;
  size_t slot_row;
  size_t tiles;
  int64_t rows_cap_max;
  int64_t n_mb_max;
} mok_schedule_layout;

typedef struct mok_workspace mok_workspace;  /* opaque; owns device scratch only */

/* ---- pure host queries (no device, no HIP call) ---------------------- */

/* Name of a status code. Never NULL. */
const char* mok_status_string(mok_status status);

/* Checks a configuration against the contract above. */
mok_status mok_validate_config(const mok_config* cfg);

/* Bytes of the caller-owned schedule buffer for this config; 0 if invalid.
 * "At most a few megabytes" at production shapes ([R] "Tuning..."). */
size_t mok_schedule_bytes(const mok_config* cfg);

/* Fills *out with the schedule buffer's field offsets. */
mok_status mok_schedule_layout_query(const mok_config* cfg, mok_schedule_layout* out);

/* Bytes of the caller-owned forward context (saved activations for
 * backward: G, U and h of every routed and shared row); 0 if invalid.
 * BF16 mode: G, U and h in bf16. MXFP8 mode: G and U in fp32 as the
 * forward accumulated them (the backward's SwiGLU derivative starts from the
 * values h came from) and h as the E4M3 codes and E8M0 scales the down GEMM
 * read; about twice the BF16 size. A context is read only by a backward of
 * the mode that wrote it. */
size_t mok_context_bytes(const mok_config* cfg, mok_mode mode);

/* Device scratch a workspace of this config allocates, in bytes. */
size_t mok_workspace_bytes(const mok_config* cfg);

/* ---- workspace ------------------------------------------------------- */

/* Allocates the workspace's scratch once on `device` ([R] "The two API
 * layers and the schedule object": one workspace per model, reused across
 * layers and steps). The config is copied. Writes NULL to *out on error. */
mok_status mok_workspace_create(const mok_config* cfg, int device, mok_workspace** out);

/* Frees the scratch (waits for the device). NULL is accepted. */
mok_status mok_workspace_destroy(mok_workspace* ws);

/* ---- the hot path ---------------------------------------------------- */

/*
 * Builds the schedule for T tokens from top_experts (device int64 [T, k],
 * expert ids; ids outside [0, E) are counted as invalid and never
 * dispatched). Per expert: counts, capacity C = min(T, ceil(mult*T)),
 * kept = first C assignments in flat order a = t*k + j (the rest are
 * dropped and counted), segments padded to P rows, exclusive prefix-sum
 * offsets, a stable permutation (rows of an expert in ascending a) and its
 * inverse, and per-minibatch sub-offsets. Deterministic: the same ids give
 * the same bytes ([R] "How MoK differs from a general MoE kernel library").
 * `schedule` is a device buffer of at least mok_schedule_bytes(cfg) bytes;
 * 0 <= T <= max_tokens. Runs 2 small kernels (3 with more than one minibatch).
 */
mok_status mok_build_schedule(mok_workspace* ws, const int64_t* top_experts, int64_t T,
                              void* schedule, size_t schedule_bytes, void* stream);

/*
 * Forward ([A] _MoKRuntime.forward; [A] GroupedExpertsMoK.forward): for each
 * token t, out[t] = sum over its kept assignments j of
 * w[t,j] * W_d[e] (silu(W_g[e] x_t) * (W_u[e] x_t)) + the shared expert's
 * S_d (silu(S_g x_t) * (S_u x_t)), with fp32 accumulation, summed in fixed
 * slot order (deterministic). x bf16 [T, H] (device); router_weights fp32
 * [T, k] (device); out bf16 [T, H] (device). T is taken from the schedule.
 * In MXFP8 mode x is quantized on the device inside this call and the
 * weights must be pre-quantized ([R] "Tuning...": MXFP8 workflow); h is
 * quantized along I before the down projection.
 * `context` (device, nullable, at least mok_context_bytes) receives the
 * activations mok_backward needs; pass NULL for inference.
 * x, router_weights and out must be non-NULL even for an empty batch (the
 * host cannot see T): with T = 0 they are never read or written, so any
 * device address will do.
 */
mok_status mok_forward(mok_workspace* ws, mok_mode mode, const void* schedule, size_t schedule_bytes,
                       const void* x, const float* router_weights, const mok_weights* weights,
                       void* out, void* context, size_t context_bytes, void* stream);

/*
 * Backward ([A] _MoKRuntime.backward): gradients of sum(grad_out * out) for
 * every float input, reusing the forward's schedule and context. grad_out,
 * x bf16 [T, H]; router_weights fp32 [T, k]. In BF16 mode `weights` are the
 * BF16 weights (scale pointers ignored). In MXFP8 mode every backward GEMM
 * operand is quantized along that GEMM's own contraction dimension (grad_out
 * rows along H; dG, dU along I; the weight gradients' operands in 32-row
 * blocks of each expert's rows), the context must come from an MXFP8 forward
 * of the same schedule, and `weights` is either
 *   - the BF16 weights with every scale pointer NULL: they are transposed
 *     and quantized on the device in this call, or
 *   - the weights already transposed and quantized by
 *     mok_mxfp8_quantize_transposed, with every scale pointer set (the
 *     pages' workflow of weights pre-quantized by a separate call, [R]
 *     "Tuning the five hyperparameters before production"): routed_down
 *     [E, I, H] codes with [E*I, H/32] scales (W_d^T, blocks along H);
 *     routed_gate / routed_up [E, H, I] with [E*H, I/32] (blocks along I);
 *     shared_down [I_s, H] with [I_s, H/32]; shared_gate / shared_up
 *     [H, I_s] with [H, I_s/32].
 *   Some but not all scale pointers set: MOK_ERR_INVALID_ARGUMENT.
 * MXFP8 mode returns MOK_ERR_UNSUPPORTED unless H, I and I_s are multiples
 * of 128. Uses only the workspace's scratch (no allocation). Every weight
 * gradient is written in full (zero for experts with no kept rows, and for
 * all of them when T = 0); as in mok_forward, the token-sized pointers must
 * be non-NULL even when T = 0.
 */
mok_status mok_backward(mok_workspace* ws, mok_mode mode, const void* schedule, size_t schedule_bytes,
                        const void* context, size_t context_bytes, const void* grad_out, const void* x,
                        const float* router_weights, const mok_weights* weights, const mok_grads* grads,
                        void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the
 * inference forward of mok_forward (context = NULL) without a workspace.
 * Its scratch (h, the weighted down rows y, and x's MXFP8 codes) is a fixed
 * device array of the library, 128 MiB per GPU, held from the first call on
 * a GPU until the process ends; the call allocates nothing. Scratch needed,
 * with n = rows_cap_max * I + max_tokens * I_s (rows_cap_max from
 * mok_schedule_layout_query) and each part rounded up to 256 bytes: h, 2n
 * bytes (BF16) or n + n/32 (MXFP8); y, (rows_cap_max + max_tokens) * H * 2;
 * in MXFP8 also x's codes and scales, m + m/32 with m = max_tokens * H. A
 * config that needs more returns MOK_ERR_UNSUPPORTED before anything is
 * enqueued. cfg is the config of the workspace whose
 * mok_build_schedule wrote `schedule` (minibatch pipeline and token ring
 * fields are ignored: one pass, no pipeline; the bits are the same). Runs on the current device (`stream` must belong
 * to it). Arguments and results otherwise as mok_forward. Calls on one GPU
 * share the array: calls that overlap on one GPU race.
 */
mok_status mok_forward_static(const mok_config* cfg, mok_mode mode, const void* schedule, size_t schedule_bytes,
                              const void* x, const float* router_weights, const mok_weights* weights, void* out,
                              void* stream);

/*
 * MXFP8 quantization ([R] "Tuning the five hyperparameters before
 * production": the separate quantize call for pre-quantizing weights).
 * src: device [rows, cols] with row stride ld_src elements, bf16
 * (src_is_fp32 = 0) or fp32 (src_is_fp32 = 1).
 * axis = 1: blocks of 32 consecutive elements along a row (cols % 32 == 0);
 *           scales [rows, cols/32], row stride cols/32.
 * axis = 0: blocks of 32 consecutive rows in a column (rows % 32 == 0);
 *           scales [rows/32, cols], row stride cols.
 * dst: E4M3 bytes [rows, cols] with row stride ld_dst (cols % 8 == 0 and
 * ld_dst % 8 == 0, ld_src % 8 == 0). Per block: X = clamp(floor(log2 amax)
 * - 8, -127, 127) (X = -127 for an all-zero block), scale byte X + 127,
 * element = round-to-nearest-even of v / 2^X on the E4M3 grid, saturating
 * at +-448, sign kept. Inputs must be finite. The codes are exact: the
 * hardware scaled conversion gives the same bytes as the rule above.
 * MOK_ERR_UNSUPPORTED for bf16 sources along axis 1 with more than 2^24 rows
 * (one workgroup per row).
 */
mok_status mok_mxfp8_quantize(const void* src, int src_is_fp32, int64_t rows, int64_t cols, int64_t ld_src,
                              int axis, uint8_t* dst, int64_t ld_dst, uint8_t* dst_scale, void* stream);

/*
 * Transposed MXFP8 quantization of a batch of bf16 matrices, the weights'
 * form for the MXFP8 backward ([R] "Tuning the five hyperparameters before
 * production": weights are quantized by a separate call). src: device bf16
 * [batches, rows, cols], dense. dst: E4M3 [batches, cols, rows] (the
 * transpose), quantized in blocks of 32 consecutive elements along its rows
 * (the source's `rows` dimension, which is the backward GEMM's contraction);
 * dst_scale: E8M0 [batches, cols, rows/32]. Codes and scales follow the rule
 * of mok_mxfp8_quantize. rows % 128 == 0 and cols % 64 == 0, src and dst
 * 16-byte aligned, dst_scale 4-byte aligned (MOK_ERR_UNSUPPORTED otherwise).
 * Runs on the current device. For W_d [E, H, I]: batches E, rows H, cols I;
 * W_g / W_u [E, I, H]: rows I, cols H; the shared weights with batches 1.
 */
mok_status mok_mxfp8_quantize_transposed(const void* src, int64_t batches, int64_t rows, int64_t cols, uint8_t* dst,
                                         uint8_t* dst_scale, void* stream);

/* ---- diagnostics (these synchronise; never on the hot path) ---------- */

/* Per-kernel event timing inside a workspace: when enabled, every launch
 * the workspace makes is bracketed by HIP events on the launch stream. */
typedef enum mok_kernel_id {
  MOK_K_SCHED_COUNT = 0, /* per-chunk expert histograms */
  MOK_K_SCHED_SCAN,      /* reserved: the scans run inside the scatter kernel */
  MOK_K_SCHED_SCATTER,   /* scans, ranks and permutation */
  MOK_K_SCHED_MINIBATCH,
  MOK_K_QUANT_X,
  MOK_K_GATE_UP,
  MOK_K_DOWN,
  MOK_K_COMBINE,
  MOK_K_BWD_TRANSPOSE,
  MOK_K_BWD_GATHER,
  MOK_K_BWD_DH,
  MOK_K_BWD_DW_REDUCE,
  MOK_K_BWD_DX_ROWS,
  MOK_K_BWD_DX_SUM,
  MOK_K_BWD_DW,
  MOK_K_BWD_QUANT,
  MOK_K_SCHED_SLICE,     /* token ring: one pass's schedule */
  MOK_K_COUNT
} mok_kernel_id;

const char* mok_kernel_name(int kernel_id);
/* Waits for the device, then returns (and resets) two counts since the last
 * call: *pipeline_timeouts, mover waits of the forward's minibatch pipeline
 * that ran out of time (their minibatches' outputs are then incomplete; 0 in
 * normal operation), and *schedule_mismatches, launches of this workspace
 * that were given a schedule whose header carries another configuration's
 * hash (such a launch does nothing: its outputs are not written). Either
 * pointer may be NULL. Returns MOK_ERR_CONFIG_MISMATCH when
 * schedule_mismatches is non-zero. */
mok_status mok_workspace_read_status(mok_workspace* ws, int32_t* pipeline_timeouts, int32_t* schedule_mismatches);
/* enable != 0: time every kernel; 0: none. */
mok_status mok_workspace_set_timing(mok_workspace* ws, int enable);
/* Time only the kernels whose bit (1 << mok_kernel_id) is set; 0 = none.
 * Each timed launch records two events on its stream, a few microseconds
 * each, so a measurement of the whole step times only what it needs. */
mok_status mok_workspace_set_timing_mask(mok_workspace* ws, uint32_t kernel_mask);
/* Waits for recorded events and returns, per kernel id, the summed
 * milliseconds and number of launches since the last reset; then resets. */
mok_status mok_workspace_read_timing(mok_workspace* ws, float* total_ms, int64_t* launches, int n);

#ifdef __cplusplus
}
#endif

#endif /* MOK_H_ */
