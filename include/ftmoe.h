/*
 * ftmoe.h -- C ABI of the offloaded Mixture-of-Experts layer for AMD MI355X
 * (gfx950).
 *
 * The layer keeps every routed expert of every layer in pinned host RAM and a
 * least-recently-used pool of expert slots in GPU memory, one pool shared by
 * all layers.  Per call: a router picks the top-k experts of each token; each
 * chosen expert is looked up in the pool (a hit runs in place, a miss is
 * streamed from host RAM over PCIe, or, in the hybrid strategy, part of the
 * step's misses is computed on host cores); tokens are grouped by expert, run
 * through a block-scaled 4-bit or 8-bit SwiGLU expert and combined with their
 * routing weights.  Prefill chunks instead stream every expert of a layer,
 * double buffered so that layer N+1 copies while layer N computes.
 *
 * Where the behaviour comes from (FreeToken pages, by title and section):
 *   - offload strategy, LRU cache of expert slots, hit at GPU speed, miss over
 *     PCIe, hybrid split of a step's misses, one global LRU pool:
 *     devpik "FreeToken: Run Frontier MoE Models on Your Own GPU, and the RAM
 *     It Takes", section "Why a Huge MoE Model Fits on One Consumer GPU";
 *     byteiota "FreeToken: Run a 290B MoE Model on One Gaming GPU", sections
 *     "VRAM Is Not the Bottleneck You Think It Is", "The Bandwidth-Adaptive
 *     Runtime".
 *   - prefill: all experts of a layer copied per chunk, layer N+1 copied while
 *     N computes, a warning when the cache cannot hold the two staging layers:
 *     devpik article, section "Long Prompts Are the Bottleneck".
 *   - formats MXFP4, NVFP4 (an 8-bit scale per 16 weights), FP8: devpik
 *     article, "The Real Requirement Is System RAM".
 *   - expert-cache hit rate and cache fullness as statistics: devpik article,
 *     "What to Watch Out For" (--moe-collect-stats); mindstudio "FreeToken
 *     Explained", section "Is FreeToken worth using...?" (FT shell stats).
 *
 * Conventions: every call returns an int status (FT_OK = 0, > 0 warnings,
 * < 0 errors) and never lets a C++ exception cross the ABI; the message of the
 * last error of the calling thread is returned by ft_moe_last_error().
 * "dev" pointers are HIP device addresses on the pool's device; "host"
 * pointers are ordinary host memory.  A pool is not thread safe: drive each
 * pool from one host thread.
 */
#ifndef FTMOE_H
#define FTMOE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ft_moe_pool ft_moe_pool; /* opaque; owned by the library */

enum {
  FT_OK = 0,
  FT_WARN_STAGING_SMALL = 1, /* init: pool cannot hold two full layers (prefill disabled) */
  FT_E_INVALID = -1,         /* bad argument, shape or pointer */
  FT_E_OOM_DEVICE = -2,      /* device allocation failed */
  FT_E_OOM_PINNED = -3,      /* pinned host allocation failed */
  FT_E_HIP = -4,             /* a HIP runtime call failed (message has details) */
  FT_E_STATE = -5            /* call out of order (prefill layers must run 0,1,...,L-1) */
};

enum { FT_FMT_MXFP4 = 1, FT_FMT_NVFP4 = 2, FT_FMT_FP8_B128 = 3 };

enum {
  FT_FWD_DECODE = 0,         /* resolve against the LRU pool */
  FT_FWD_PREFILL_STAGED = 1, /* stream all experts of the layer into staging half (layer % 2) */
  FT_FWD_MODE_MASK = 0xF,
  FT_ACT_BF16 = 0 << 4,      /* expert inputs used as given (bf16) */
  /* MX activation modes: prefill calls on MXFP4-weight layers only (else
   * FT_E_INVALID).  x and h are quantised per 32-element block as the OCP MX
   * v1.0 conversion defines (power-of-two scale from the block's amax,
   * nearest-even, saturating) and both products run on the block-scaled MFMA. */
  FT_ACT_MXFP8 = 1 << 4,     /* x and h as MXFP8 (E4M3) */
  FT_ACT_MXFP4 = 2 << 4,     /* x and h as MXFP4 (E2M1) */
  FT_ACT_MASK = 0xF << 4,
  /* Prefill option (devpik "FreeToken: Run Frontier MoE Models on Your Own
   * GPU, and the RAM It Takes", section "Long Prompts Are the Bottleneck":
   * skip experts already in the GPU cache so only misses cross PCIe).  An
   * expert of the layer resident in the pool outside the staging region
   * [0, 2E) is not copied: its pairs are FT_PAIR_HIT and read the weights
   * in its pool slot; the others stream into the staging half as usual.
   * Residency is read once, at layer 0 of the chunk (the device is
   * synchronised then), and the pool outside the staging region does not
   * change during a chunk.  Every call of a chunk must carry the same
   * option (else FT_E_STATE).  The copied experts become residents of
   * their staging slots (until a later call clears that half, so after a
   * chunk the last two layers stay cached), and each call updates the LRU
   * order like one decode wave over its pairs: copies that no token selects
   * take the first clock ticks (expert order), then every selected expert
   * the clock of its last pair.  Counters: pair hits count the pairs of
   * resident experts, expert hits the resident experts of the layer, and
   * bytes H2D the experts copied. */
  FT_FWD_PREFILL_HIT_D2D = 1 << 8
};

enum { FT_PAIR_HIT = 0, FT_PAIR_MISS_STREAM = 1, FT_PAIR_MISS_CPU = 2 };

/* Layer geometry and pool policy.  Read only during ft_moe_init_pool. */
typedef struct {
  int32_t num_layers;        /* L >= 1 */
  int32_t hidden;            /* H, multiple of 128 */
  int32_t inter;             /* I, multiple of 128 (expert intermediate size) */
  int32_t num_experts;       /* E per layer, 1..512 */
  int32_t top_k;             /* k, 1..min(E, 16) */
  int32_t has_shared_expert; /* 1: one always-resident shared expert per layer, weight 1 */
  const int32_t *layer_fmt;  /* host [L] FT_FMT_* */
  int64_t pool_slots;        /* > 0: number of expert slots C (top_k <= C <= 65536) */
  int64_t pool_bytes;        /* used if pool_slots == 0: C = floor(pool_bytes / largest expert size) */
  double hybrid_cpu_share;   /* 0: pure offload; (0,1]: fraction of each wave's misses computed on host */
  int32_t cpu_threads;       /* host threads for the hybrid worker (0 = 8) */
  int32_t device;            /* HIP device ordinal */
} ft_moe_config;

/*
 * Weights, in HOST memory owned by the caller and read only during init (the
 * library copies them; the caller may free them afterwards).
 * Canonical expert blob = [W_gate codes][W_up codes][W_down codes]
 * [gate scales][up scales][down scales][3 x fp32 tensor scales, NVFP4 only];
 * W_gate, W_up are [I][H], W_down is [H][I], row-major [out][in] with the
 * block scales running along `in`; FP4 codes two per byte, even element in
 * the low nibble; MXFP4 scales E8M0 per 32, NVFP4 scales E4M3 per 16, FP8
 * scales little-endian fp32 per 128.  Entries of `expert` that hold the same
 * pointer are stored once in pinned memory (they stay distinct cache keys).
 */
typedef struct {
  const void *const *expert; /* [L*E] blob of (layer l, expert e) at index l*E+e */
  const void *const *shared; /* [L] shared-expert blobs, or NULL */
  const float *router_w;     /* [L][E][H] fp32 router weights */
} ft_moe_weights;

/* Optional per-call trace, DEVICE memory owned by the caller, T*k entries
 * each, pair order = token-major then rank.  Any member may be NULL. */
typedef struct {
  int32_t *sel;  /* chosen expert of each pair (rank order: logit desc, index asc) */
  float *w;      /* routing weight of each pair */
  int32_t *slot; /* pool slot of the pair's expert, -1 for host-computed */
  uint8_t *flag; /* FT_PAIR_* */
  int32_t *row;  /* row of the pair in the expert-grouped order of its wave */
} ft_moe_trace;

typedef struct {
  uint64_t pair_hits, pair_misses;     /* per (token, rank) pair; hit rate = hits / (hits + misses) */
  uint64_t expert_hits, expert_misses; /* per distinct expert of a wave */
  uint64_t cpu_misses;                 /* experts computed on host cores */
  uint64_t evictions;                  /* resident experts displaced */
  uint64_t bytes_h2d;                  /* streamed expert bytes + host-computed result rows */
  uint64_t calls;                      /* forward calls */
  int64_t slots_used, slots_total;     /* cache fullness (whole pool) */
  double min_topk_gap;                 /* smallest logit gap between rank k and k+1 seen */
  /* milliseconds spent copying experts from host RAM (misses and prefill
   * staging): a device-driven miss copy is timed on the device's
   * constant-rate wall clock from its first workgroup's start to its last
   * workgroup's end; host-issued copies are bracketed by events on the copy
   * stream.  Copies that overlap other work count in full. */
  double copy_ms;
} ft_moe_stats;

/* Create a pool on cfg->device: validates the shapes, copies the expert
 * blobs into pinned host RAM (repacked for the GPU), allocates the slot arena,
 * the resident router weights and shared experts, and the device slot table.
 * Returns FT_OK, FT_WARN_STAGING_SMALL (pool usable for decode only), or an
 * error (then *out is NULL).  Env FT_MOE_FAULT (for tests): pinned_alloc
 * forces FT_E_OOM_PINNED here; work_alloc:<n> / mx_alloc:<n> make the pool's
 * n-th device allocation of per-call work buffers / of MX activation tiles
 * fail once (the call returns FT_E_OOM_DEVICE and leaves those buffers
 * unallocated; the next call allocates them again); corrupt:<n> damages the
 * n-th miss copy (256 bytes overwritten; host-driven path).
 * Debug environment, read here: FT_MOE_POISON fills every slot with 0xFF
 * bytes (NaN block scales) just before a copy into it, so a read racing the
 * copy shows up as NaN; FT_MOE_DEBUG_CHECKSUM checks, before each FFN, that
 * every slot it reads holds its key's weights (a checksum of the slot against
 * the host store's blob) and makes each call wait and return FT_E_HIP naming
 * the key and slot of a mismatch (no graph capture in this mode);
 * FT_MOE_LOG=<n> prints the counters on stderr every n forward calls. */
int ft_moe_init_pool(const ft_moe_config *cfg, const ft_moe_weights *w, ft_moe_pool **out);

/* One MoE layer call on `hip_stream` (a hipStream_t, NULL = default stream).
 * x_bf16: dev [T][H] bf16; router_bias: dev [E] fp32 added to the logits, or
 * NULL; out_bf16: dev [T][H] bf16 (may not alias x).  flags: FT_FWD_* |
 * FT_ACT_*.  A decode call whose pairs fit one wave (T*top_k <= pool slots)
 * with no hybrid share runs device-driven: router, resolve, miss copy (a
 * kernel reading the pinned store), FFN and combine are enqueued on the
 * stream with no host wait.  Other decode calls (hybrid share, several
 * waves, or env FT_MOE_DECODE_PATH=host) block the host once per wave to
 * read the miss list, issue the copies on the pool's copy streams and run
 * host-computed experts on host threads.  The call returns once the work is
 * enqueued.  On error no slot stays assigned to an expert whose copy failed.
 * Env FT_MOE_FAULT=copy:<n> fails the n-th miss copy of the pool (host-driven
 * path; for tests). */
int ft_moe_layer_forward(ft_moe_pool *p, int32_t layer, int32_t num_tokens, const void *x_bf16,
                         const float *router_bias, void *out_bf16, int32_t flags, void *hip_stream,
                         ft_moe_trace *trace);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * ft_moe_layer_forward for a device-driven decode call -- flags ==
 * FT_FWD_DECODE, no hybrid share, T * top_k <= pool slots, the device path
 * not switched off by FT_MOE_DECODE_PATH=host -- whose per-call work buffers
 * (logits, routing, pair and row records, h and p rows) are carved from one
 * static device array of 16 MiB per GPU instead of the pool's own buffers.
 * It calls no hipMalloc, hipFree or other allocating routine and creates no
 * events (stage timing is off for these calls); the pool, the caller's x,
 * out, router_bias and trace are used as in ft_moe_layer_forward, and the
 * slot table, counters and outputs are the same.  Limits: the call must fit
 * the array (about 170 KB per token at H 7168, I 2048, top-8 with a shared
 * expert: 64 tokens fit), else FT_E_INVALID with the bytes it needs; any
 * other kind of call is FT_E_INVALID.  The array's device address is looked
 * up once per GPU at pool creation (FT_E_HIP if that failed).
 * ft_moe_last_misses does not report these calls (it keeps the previous
 * call's lists).  Every call of this entry point on one GPU -- any pool, any
 * stream, any host thread -- uses the same array and leaves its contents
 * behind: calls that overlap in time on one GPU race and must be ordered by
 * the caller (one stream, or events). */
int ft_moe_layer_forward_noalloc(ft_moe_pool *p, int32_t layer, int32_t num_tokens, const void *x_bf16,
                                 const float *router_bias, void *out_bf16, int32_t flags, void *hip_stream,
                                 ft_moe_trace *trace);

/* Counters of one layer (or all layers for layer = -1); synchronises the
 * pool's device.  reset != 0 zeroes the counters afterwards. */
int ft_moe_pool_stats(ft_moe_pool *p, int32_t layer, ft_moe_stats *out, int32_t reset);

/* Streamed-miss and host-miss lists of the most recent forward call, in the
 * order the library resolved them (waves in order, each in first-appearance
 * order).  Host arrays of capacity `cap`; counts returned even if cap is
 * smaller. */
int ft_moe_last_misses(const ft_moe_pool *p, int32_t *stream_expert, int32_t *stream_slot,
                       int32_t *n_stream, int32_t *cpu_expert, int32_t *n_cpu, int32_t cap);

/* Copy of the device slot table (synchronises): slot_key[C] = layer*E+expert
 * or -1 if free, slot_last[C] = clock value of the last use, *clock.  Host
 * arrays of pool_slots entries; NULL members are skipped. */
int ft_moe_pool_table(ft_moe_pool *p, int32_t *slot_key, uint64_t *slot_last, uint64_t *clock,
                      int64_t *slots);

/* Change the number of pool slots at runtime, without reloading weights (the
 * pages: VRAM is re-allocated between the expert cache and other memory while
 * the engine runs -- dev.to "FreeToken uses bandwidth-adaptive CPU-GPU
 * co-execution on your desktop", section "Memory that moves while the engine
 * runs").  The new_slots most recently used residents survive (a shrink evicts
 * the least recently used); a survivor keeps its slot when the slot still
 * exists, the others, in ascending old slot, move to the lowest free slots
 * below new_slots (device-to-device copies).  Last uses and the clock are
 * unchanged; counters are not changed.  Synchronises the device.  A new slot
 * arena is allocated before the old one is freed (both exist for a moment);
 * if an allocation fails the pool is unchanged and FT_E_OOM_DEVICE is
 * returned.  Requires top_k <= new_slots <= 65536 (FT_E_INVALID) and no
 * prefill chunk in progress (FT_E_STATE).  Returns FT_WARN_STAGING_SMALL when
 * the new pool cannot hold two staged layers.  ft_moe_last_misses still
 * reports the call before the resize (its slot numbers may have moved). */
int ft_moe_resize_pool(ft_moe_pool *p, int64_t new_slots);

/* Grow the per-call work buffers for calls of up to max_tokens tokens now
 * (synchronises the device when it grows them; a call that needs no growth
 * allocates nothing; the buffers hold at least 64 tokens).  Needed before
 * capturing calls into a HIP graph.
 *
 * Graph capture (the pages list graph-compatible execution among the
 * runtime's mechanisms: dev.to "FreeToken uses bandwidth-adaptive CPU-GPU
 * co-execution on your desktop", section "What the project says it does").
 * ft_moe_layer_forward may be called on a stream that is capturing when the
 * call is a device-driven decode call (FT_FWD_DECODE, no hybrid share, T*top_k
 * <= pool slots, FT_MOE_DECODE_PATH not "host") that fits the buffers
 * already reserved; every other call returns FT_E_INVALID while capturing.  Captured
 * calls take no host decision: a replay resolves its experts against the slot
 * table as it stands when the replay runs, copies its own misses, and updates
 * table and counters like an eager call.  Stage timing is skipped while
 * capturing, and ft_moe_last_misses reports the most recent eager call. */
int ft_moe_reserve(ft_moe_pool *p, int32_t max_tokens);

/* Set the hybrid share used by later calls (0..1), for layers of every
 * weight format.  0 is the offload strategy (every miss streams); 1 is the cpu
 * strategy (every miss is computed on host cores and the pool never changes)
 * -- devpik "FreeToken: Run Frontier MoE Models on Your Own GPU, and the RAM
 * It Takes", section "Why a Huge MoE Model Fits on One Consumer GPU".  A call
 * on a layer uses the share of that layer's format (the split rule itself is
 * unchanged: m_cpu = floor(m * share + 1/2)).  Clears the in-situ
 * observations of ft_moe_rebalance. */
int ft_moe_set_hybrid_share(ft_moe_pool *p, double share);
/* The same for the layers of one format fmt (FT_FMT_*) only. */
int ft_moe_set_hybrid_share_format(ft_moe_pool *p, int32_t fmt, double share);
/* The share in use for layers of format fmt. */
int ft_moe_get_hybrid_share(const ft_moe_pool *p, int32_t fmt, double *share);

/* One-time strategy choice from measured rates (mindstudio "FreeToken
 * Explained: Run 290B+ MoE Models on One Gaming GPU", section "How does the
 * benchmark decide between hybrid and offload mode?"; the fused case: devpik,
 * section "Why a Huge MoE Model Fits on One Consumer GPU").  Arrays are
 * indexed by format FT_FMT_* (index 0 unused); rates are expert-weight bytes
 * per second, 0 for a format the model does not use. */
enum { FT_MODE_OFFLOAD = 0, FT_MODE_HYBRID = 1, FT_MODE_FUSED = 2 };
typedef struct {
  int32_t tokens;             /* rows per expert the rates were measured at */
  int32_t layers[4];          /* number of layers in each format */
  double expert_bytes[4];     /* canonical expert bytes of each format */
  double h2d_bytes_per_s[4];  /* pinned host -> device copies of experts */
  double gpu_bytes_per_s[4];  /* the device's grouped expert FFN at `tokens` rows per expert */
  double cpu_bytes_per_s[4];  /* the host expert path at `tokens` rows */
  int64_t pool_slots;         /* C */
  int64_t all_experts;        /* L * E */
  /* filled by the decision: */
  double t_stream;            /* s: one miss in every layer, copied and run on the device */
  double t_cpu;               /* s: the same misses on host cores */
  int32_t mode;               /* FT_MODE_* */
  double share;               /* the hybrid share the mode implies (0 unless hybrid) */
  double balanced_share;      /* t_stream / (t_stream + t_cpu) whatever the mode: the share at
                                 which streamed and host-computed misses finish together, for a
                                 caller that picks the hybrid strategy itself */
} ft_moe_mode_report;

/* The decision alone (host code, no device work): t_stream = sum over layers
 * of b/h2d + b/gpu, t_cpu = sum of b/cpu (b = the layer's expert bytes, rates
 * of the layer's format, layers in format order 1..3); FUSED when pool_slots
 * >= all_experts; else HYBRID when t_cpu < t_stream, with share =
 * t_stream / (t_stream + t_cpu), the split at which both paths finish a step's
 * misses together; else OFFLOAD.  The pages' cpu strategy (share 1) is never
 * chosen by this rule.  balanced_share is that split for every mode.  FT_E_INVALID if a used format has a rate <= 0 or
 * not finite. */
int ft_moe_decide_mode(ft_moe_mode_report *r);

/* Measure the rates on this machine, then decide (ft_moe_decide_mode).  For
 * each format the model uses, the first layer of that format supplies up to 16
 * experts: their blobs are copied from the pinned store into a temporary
 * device buffer (h2d), the grouped expert FFN runs on them with `tokens` rows
 * each (gpu), and the host expert path runs on all of them in one batched
 * call, as a step's host-computed misses do (cpu).  Takes
 * about a second; synchronises the device; allocates and frees the temporary
 * buffer; does not touch the slot table or the counters.  Keeps the device FFN
 * rates for ft_moe_rebalance.  apply != 0 sets the pool's hybrid share, for
 * every format, to the chosen share.  1 <= tokens <= 64. */
int ft_moe_measure_mode(ft_moe_pool *p, int32_t tokens, int32_t apply, ft_moe_mode_report *out);

/* Bandwidth-adaptive refinement of the hybrid split from the running
 * workload (dev.to "FreeToken uses bandwidth-adaptive CPU-GPU co-execution on
 * your desktop", section "What the project says it does").  Since the last
 * share change (or rebalance) every host-driven decode call has recorded, per
 * weight format, the expert bytes its host worker threads computed and their
 * wall time, and the expert bytes it streamed and their copy time (HIP events
 * around the copies).  For each format with both, the new share is the
 * balanced split of ft_moe_decide_mode with these in-situ costs per byte:
 * t_stream = copy seconds / copy bytes + 1 / (device FFN rate of the last
 * ft_moe_measure_mode, the term left out if none), t_cpu = host seconds /
 * host bytes, share = t_stream / (t_stream + t_cpu).  Formats without both
 * observations keep their share (changed[f] = 0).  Waits for the pool's
 * outstanding copies; apply != 0 sets the new shares; the observations are
 * cleared either way.  Arrays are indexed by FT_FMT_* (index 0 unused). */
typedef struct {
  double host_bytes[4];       /* expert bytes computed on host cores */
  double host_seconds[4];     /* their wall time (the host worker phase of each call) */
  double copy_bytes[4];       /* expert bytes streamed host -> device */
  double copy_seconds[4];     /* their copy time */
  double gpu_bytes_per_s[4];  /* device FFN rate from the last mode measurement, 0 if none */
  double share[4];            /* the refined share (the current one where changed[f] = 0) */
  int32_t changed[4];
} ft_moe_rebalance_report;
int ft_moe_rebalance(ft_moe_pool *p, int32_t apply, ft_moe_rebalance_report *out);

/* Time the host expert path on `tokens` rows of one expert of `layer`
 * (the one-time bandwidth measurement behind the hybrid share); returns
 * expert bytes processed per second in *bytes_per_s. */
int ft_moe_host_expert_rate(ft_moe_pool *p, int32_t layer, int32_t tokens, int32_t iters,
                            double *bytes_per_s);

/* Measured issue rate of the matrix-core instructions the prefill GEMM and
 * the router use, reported beside the data-sheet peaks.  kind 0:
 * v_mfma_scale_f32_32x32x64_f8f6f4 with FP4 operands; 1:
 * v_mfma_scale_f32_16x16x128_f8f6f4 with FP8 operands; 2:
 * v_mfma_f32_16x16x32_bf16; 3: v_mfma_f32_32x32x16_bf16; 4:
 * v_mfma_f64_16x16x4_f64 (the router's logits).  Runs 1024
 * workgroups of 4 waves, each wave issuing `iters` rounds of independent
 * MFMAs on register operands, once to warm up and once timed with HIP
 * events on `hip_stream` (a hipStream_t; null
 * = the null stream), and returns dense flops per second in *flops_per_s
 * (2 per multiply-add).  Allocates and frees a 1 MiB device buffer; blocks
 * until the timed run ends.  1 <= iters <= 2^20, else FT_E_INVALID. */
int ft_moe_mfma_rate(int32_t kind, int32_t iters, void *hip_stream, double *flops_per_s);

/* Per-stage timing with HIP events recorded on the stream each stage runs on
 * (the caller's stream for kernels, the pool's copy stream for miss copies),
 * for measurement.  `bytes` accumulates the algorithmic bytes of each stage:
 * FFN stages count the weights of the groups they run plus their activation
 * rows read and written; the copy stage counts the expert bytes streamed. */
enum { FT_STAGE_ROUTER = 0, FT_STAGE_TOPK, FT_STAGE_RESOLVE, FT_STAGE_FFN_GATEUP, FT_STAGE_FFN_DOWN,
       FT_STAGE_COMBINE, FT_STAGE_COPY,
       FT_STAGE_ACT_QUANT, /* MX activation modes: quantising x or h and laying the rows out as GEMM tiles */
       FT_STAGE_HOST_FFN,  /* hybrid split: the host-computed experts of a call, host wall time (overlaps the
                              GPU work); bytes = their expert bytes, flops = 6 x rows x H x I */
       FT_STAGE_COUNT };
typedef struct {
  double ms[FT_STAGE_COUNT];        /* summed event-measured durations */
  double bytes[FT_STAGE_COUNT];     /* summed algorithmic bytes */
  double flops[FT_STAGE_COUNT];     /* summed algorithmic flops (FFN stages: 2 per multiply-add) */
  uint64_t launches[FT_STAGE_COUNT];
} ft_moe_profile;

/* Name of the kernel (with its compile-time shape) behind the most recent
 * FT_STAGE_FFN_GATEUP or FT_STAGE_FFN_DOWN launch enqueued by this process,
 * for reports ("" before the first launch or for other stages).  The string
 * belongs to the library and changes with the next launch. */
const char *ft_moe_ffn_kernel_name(int32_t stage);

/* stage_mask: bit FT_STAGE_x set = record events around that stage in later
 * calls (0 = off, (1 << FT_STAGE_COUNT) - 1 = all). */
int ft_moe_set_profiling(ft_moe_pool *p, int32_t stage_mask);
/* Waits for recorded events, returns the sums; reset != 0 clears them. */
int ft_moe_profile_read(ft_moe_pool *p, ft_moe_profile *out, int32_t reset);

/* Diagnostics for tests: copies an internal device buffer of the pool into host
 * memory dst (bytes from its start), after waiting for all work on the device.
 * FT_DBG_H_CODES / FT_DBG_H_SCALES: the activation tiles of h that the latest
 * prefill call in an MX activation mode (FT_ACT_MXFP4 / FT_ACT_MXFP8) wrote
 * in its gate/up GEMM for its down GEMM -- per (128-row tile, 128-K step)
 * block: codes in 16-row sub-tiles of 1 KB (FP4) or 2 KB (FP8), a row's
 * 32-element block q at byte (16 q + row % 16) * 16 of its sub-tile (FP4: 32
 * E2M1 codes, element 2i in the low nibble of byte i; FP8: the two 16-byte
 * halves of the block at sub-tile bytes (q / 2) * 1024 + (16 (2 q % 4) + row
 * % 16) * 16 and the next lane's 16 bytes), and 512 bytes of E8M0 scales
 * (row * 4 + q); blocks of FP4 codes 8 KB apart, of FP8 codes 16 KB, of
 * scales 512 bytes.  FT_DBG_ROW_SLOT: int32 per row of that call, the row's
 * slot in the tiles (128 * tile + row in tile).  FT_E_INVALID when the buffer
 * does not exist yet or is smaller than bytes. */
enum { FT_DBG_H_CODES = 0, FT_DBG_H_SCALES = 1, FT_DBG_ROW_SLOT = 2 };
int ft_moe_debug_read(ft_moe_pool *p, int32_t what, void *dst, int64_t bytes);

void ft_moe_destroy_pool(ft_moe_pool *p);
const char *ft_moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* FTMOE_H */
