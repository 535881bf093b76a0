/*
 * ae.h -- C ABI of the MI355X (gfx950) action-expert denoise library.
 *
 * The library runs the flow-matching action-expert loop of a Pi0.5 /
 * MolmoBot-style vision-language-action model: given the VLM prefix K/V that
 * the caller has already computed once per query, it integrates an action
 * chunk from noise with N explicit Euler steps.  Each step runs the expert's
 * decoder layers (time-conditioned adaRMS norm, merged Q/K/V with RoPE,
 * attention of the action tokens over [visible prefix K/V | their own K/V],
 * gated residual, gelu-gated MLP, gated residual), then the final norm, the
 * action-out projection and x += dt * v.
 *
 * Sources (titles as on the pages):
 *  - MolmoBot PR "Inference optimization for MolmoBot VLA: torch.compile +
 *    CUDA graphs + action-expert KV cache", Part 2: the context K/V is
 *    projected once per query and reused by every flow step; only the action
 *    queries and the timestep change between steps.  Part 3: per-tensor
 *    dynamic fp8 e4m3 linears.
 *  - LoongForge blog "How to Speed Up VLA Training Step by Step: A 3x
 *    Acceleration Case Study on Pi0.5", sections 1-3: adaRMS with
 *    scale/shift/gate, gated residuals, gelu*up, rotate_half RoPE, the
 *    attention mask (actions see every valid prefix token and each other;
 *    padding and empty camera slots are invisible; pads do not advance
 *    positions), the single KV head broadcast to all query heads.
 *  - sglang PR 34599 summary, implementation items 1-4: merged Q/K/V and
 *    gate/up projections (shard order q, k, v), layout computed once per call,
 *    mutable prefix K/V and mask refreshed before an action-graph replay.
 *
 * Conventions
 *  - Every entry point returns an ae_status.  No exception crosses the ABI.
 *  - Every argument and shape check happens before any state change or HIP
 *    call: a call that fails with AE_ERR_INVALID_ARGUMENT,
 *    AE_ERR_SHAPE_MISMATCH, AE_ERR_NOT_READY or AE_ERR_UNSUPPORTED leaves the
 *    handle exactly as it was.  ae_last_error() gives the handle's message.
 *  - Device pointers are HIP device memory (e.g. from torch on ROCm).
 *    Streams are hipStream_t passed as void*; NULL means the default stream.
 *    All work is stream-ordered and asynchronous: no call synchronises the
 *    host except ae_create / ae_destroy.
 *  - One stream per handle at a time; the library does no locking.
 *  - Weight matrices are [in_features, out_features] row-major (y = x W + b).
 *  - Fields and arguments that name an enumerator are plain ints, so a value
 *    outside the enumeration is well defined and rejected by the checks.
 */
#ifndef AE_H
#define AE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ae_handle ae_handle;

typedef enum {
  AE_OK = 0,
  AE_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad value, unknown/missing weight */
  AE_ERR_SHAPE_MISMATCH = 2,   /* a shape disagrees with the config or earlier call */
  AE_ERR_NOT_READY = 3,        /* weights or prefix not set yet */
  AE_ERR_OUT_OF_MEMORY = 4,    /* device allocation failed (ae_create only) */
  AE_ERR_UNSUPPORTED = 5,      /* a config the kernels do not implement */
  AE_ERR_HIP = 6               /* a HIP runtime call failed (e.g. no GPU) */
} ae_status;

typedef enum { AE_F32 = 0, AE_BF16 = 1, AE_FP8_E4M3 = 2 } ae_dtype;

/* Decoder block of the expert.
 * AE_BLOCK_JOINT: one attention of the action tokens over [visible prefix |
 *   action tokens] with one softmax (Pi0.5 / LoongForge blog section 3).
 * AE_BLOCK_DIT: the DiT-style block of the MolmoBot action expert (MolmoBot
 *   PR Part 2: the block hands the cached context K/V to its second
 *   attention; its correctness table lists cross_attn and self_attn apart):
 *   attn1 of the action tokens over themselves (q, k, v, o), then attn2 of
 *   separate queries q2 over the visible prefix only (o2), each with its own
 *   softmax and its own adaRMS (scale, shift, gate), then the MLP; an empty
 *   prefix makes attn2 add nothing.  bf16 projections only. */
typedef enum { AE_BLOCK_JOINT = 0, AE_BLOCK_DIT = 1 } ae_block;

/* Which kernels run a denoise call (ae_config.exec_path).  The whole-call
 * kernel (one persistent launch for the whole call) takes a call that fits
 * it: batch * action_horizon <= 64, action_dim <= 32, bf16 or f32 projections,
 * AE_BLOCK_JOINT, and a device with cooperative launch; any other call runs
 * the per-phase kernels (a few launches per layer, replayed from a graph).
 * Both compute the same function (not bitwise the same values).
 * AE_PATH_AUTO takes the whole-call kernel for a call that fits it only when
 * the decoder layers' projection weights exceed the last-level cache (256 MiB
 * on MI355X): the whole-call kernel's time per layer is set by its
 * synchronisation, while the per-phase kernels gain from weights that stay
 * in that cache from one step to the next. */
typedef enum { AE_PATH_AUTO = 0, AE_PATH_WHOLE_CALL = 1, AE_PATH_PER_PHASE = 2 } ae_path;

/* Expert shape and numerics.  Fixed for the life of a handle. */
typedef struct {
  int n_layers;         /* decoder layers L */
  int width;            /* residual width D (multiple of 64) */
  int n_q_heads;        /* Hq */
  int n_kv_heads;       /* Hkv, divides Hq; query head h reads KV head h*Hkv/Hq */
  int head_dim;         /* dh, multiple of 32, at most 256 */
  int mlp_dim;          /* F (multiple of 64); gate and up are each [D, F] */
  int action_horizon;   /* T action tokens per request */
  int action_dim;       /* A action channels, at most 64 */
  int max_prefix_len;   /* largest prefix_len ae_set_prefix_kv accepts */
  int max_batch;        /* largest batch (requests) */
  int max_steps;        /* largest Euler step count ae_denoise accepts */
  int act_dtype;        /* an ae_dtype: AE_F32 or AE_BF16 (weights, prefix K/V, activations) */
  int proj_weight_dtype;/* an ae_dtype: act_dtype, or AE_FP8_E4M3 for the q/k/v,
                                 gate/up and down projections (bf16 only) */
  float rope_theta;     /* RoPE base (10000) */
  float rms_eps;        /* adaRMS epsilon (1e-6) */
  int use_graphs;       /* 1: replay denoise calls as captured hipGraphs; 0: launch directly */
  int graph_cache_size; /* captured graphs kept at most, in [0, 64]; 0 turns capture off */
  int graph_cache_evict;/* cache full and a new (batch, steps, bucket): 1 evicts the least
                           recently used graph (released once its last replay is done);
                           0 launches the new call directly, uncaptured */
  int context_width;    /* Dc of the context hidden states ae_prepare_prefix projects
                           (multiple of 64, <= 8192; bf16 only); 0: no context projection */
  int state_dim;        /* size of the robot state ae_prepare_prefix encodes as one more
                           context row (<= 64, needs context_width); 0: none */
  int block_type;       /* ae_block: AE_BLOCK_JOINT (0) or AE_BLOCK_DIT (1) */
  int fp8_rowwise;      /* with AE_FP8_E4M3 projections: 0 = a weight scale per logical tensor and
                           an activation scale per request (MolmoBot PR Part 3's per-tensor
                           dynamic recipe); 1 = a scale per weight output column and per
                           activation row (the row-wise recipe the PR names as unsupported on its
                           GPU) */
  int fp8_oproj;        /* 1: the attention output projection in fp8 as well (needs fp8_rowwise
                           and n_q_heads * head_dim a multiple of 128); 0: bf16 */
  int exec_path;        /* an ae_path: AE_PATH_AUTO (0), AE_PATH_WHOLE_CALL (1) or
                           AE_PATH_PER_PHASE (2) */
} ae_config;

/* One named logical weight, caller-owned device memory, dtype = act_dtype.
 * Names (all required; l = 0..L-1):
 *   time_mlp.1.w [D,D]  time_mlp.1.b [D]  time_mlp.2.w [D,D]  time_mlp.2.b [D]
 *   action_in.w [A,D]   action_in.b [D]   action_out.w [D,A]  action_out.b [A]
 *   final_mod.w [D,2D]  final_mod.b [2D]
 *   layers.l.q [D,Hq*dh]  layers.l.k [D,Hkv*dh]  layers.l.v [D,Hkv*dh]
 *   layers.l.o [Hq*dh,D]  layers.l.gate [D,F]  layers.l.up [D,F]  layers.l.down [F,D]
 *   layers.l.mod.w [D,6D] layers.l.mod.b [6D]  (chunks: scale_a, shift_a,
 *   gate_a, scale_m, shift_m, gate_m)
 * With block_type = AE_BLOCK_DIT instead: layers.l.mod.w [D,9D] and
 * layers.l.mod.b [9D] (chunks: scale, shift, gate of attn1, of attn2, of the
 * MLP), plus layers.l.q2 [D,Hq*dh] and layers.l.o2 [Hq*dh,D] (attn2's query
 * and output projections; attn2 reads the prefix K/V).
 * With context_width = Dc > 0 also: layers.l.ctx_k [Dc,Hkv*dh], layers.l.ctx_v
 * [Dc,Hkv*dh] (each layer's context K and V projections); with state_dim = S > 0
 * also: state_in.w [S,Dc], state_in.b [Dc] (the state's input layer). */
typedef struct {
  const char* name;
  const void* data;
  int ndim;
  long long shape[4];
  int dtype;  /* an ae_dtype, equal to act_dtype */
} ae_tensor_view;

typedef struct {
  long long denoise_calls;
  long long prefix_sets;
  long long graph_captures;
  long long graph_replays;
  long long eager_runs;      /* calls launched directly instead of replaying a graph */
  long long device_bytes;    /* bytes the handle holds on the device */
  long long device_errors;   /* whole-call launches whose waits timed out (their results are
                                invalid); counted on the device, read by ae_get_stats */
  long long persistent;      /* workgroups of the whole-call kernel (for calls that take it, see
                                ae_path); 0: the device cannot run it */
  long long persistent_calls;/* denoise calls that ran the whole-call kernel */
  long long graph_hits;      /* calls replayed from the graph cache */
  long long graph_misses;    /* calls whose signature was not cached (captured, or run directly) */
  long long graph_evictions; /* graphs evicted to make room */
  long long graphs_cached;   /* graphs in the cache now */
  long long prefix_bucket;   /* key span (prefix bucket) of the last ae_set_prefix_kv */
  long long graph_nodes;     /* nodes (kernel launches) of the graph the last ae_denoise call
                                replayed; 0 if it ran directly */
} ae_stats;

/* Validate the config, then allocate every device buffer the handle will
 * ever use (weights, prefix K/V at max size, activations, scratch).
 * Defined by: MolmoBot PR Part 1 (graph inputs are static buffers allocated
 * up front, never built lazily), so a replay reads fixed addresses.
 * Errors: INVALID_ARGUMENT / UNSUPPORTED (before any HIP call), HIP (no
 * device), OUT_OF_MEMORY.  On error *out is NULL.  The handle owns every
 * buffer until ae_destroy. */
ae_status ae_create(const ae_config* cfg, ae_handle** out);

/* Copy and pack the named weights: q|k|v merged into one projection in that
 * shard order and gate|up into another, each packed in the kernels' fragment
 * order; fp8 e4m3 codes with a static per-tensor scale when configured.
 * Defined by: sglang PR 34599 summary, implementation item 1 (merged Q/K/V
 * and gate/up projections, one GEMM each, with shard-aware loading of the
 * q/k/v pieces); MolmoBot PR Part 3 (per-tensor fp8 weights).
 * Arguments: n views of caller-owned device memory in act_dtype, names and
 * shapes as listed at ae_tensor_view.  All n views are validated (names,
 * ranks, shapes, dtypes) before anything is written: INVALID_ARGUMENT for a
 * missing, unknown, duplicate or null weight, SHAPE_MISMATCH for a wrong
 * shape.  Stream-ordered; the caller may free its tensors once the stream
 * passes the call.  Captured graphs stay valid (they read the packed
 * buffers by address); the time-path table is rebuilt on the next call. */
ae_status ae_load_weights(ae_handle* h, const ae_tensor_view* w, int n, void* stream);

/* Ingest one query's prefix K/V and mask into the static buffers.
 * Defined by: MolmoBot PR Part 2 (the context K/V is computed once per query
 * and reused by every flow step); sglang PR 34599 summary, implementation
 * item 4 (the mutable prefix K/V and mask are refreshed in place before an
 * action-graph replay); LoongForge blog section 1 (masked camera slots and
 * padding are invisible; pad tokens do not advance positions).
 * Arguments: K and V are device [L][batch][prefix_len][Hkv][dh] in
 * act_dtype, 16-byte aligned, K already rotated at the prefix's own
 * positions (the VLM's KV cache); valid_mask is device [batch][prefix_len] uint8 (0 = invisible:
 * padding or an empty camera slot, any pattern).  The library copies the
 * visible rows, in order, into its static buffers and computes, on the
 * device, each request's visible count n_b (the action tokens sit at
 * positions n_b .. n_b+T-1) and RoPE tables.  Invisible rows are never read
 * into arithmetic.  prefix_len may be 0 (K, V, mask may then be NULL).  The
 * prefix bucket is the smallest ae_set_prefix_buckets length >= prefix_len
 * (else max_prefix_len); rows past prefix_len count as masked padding.
 * Errors: SHAPE_MISMATCH for batch outside [1, max_batch] or prefix_len
 * outside [0, max_prefix_len], INVALID_ARGUMENT for a null or misaligned K or
 * V, or a null mask, with prefix_len > 0 (checked before any state change).
 * Stream-ordered; the caller may reuse its buffers once the stream passes
 * the call. */
ae_status ae_set_prefix_kv(ae_handle* h, int batch, int prefix_len, const void* K,
                           const void* V, const uint8_t* valid_mask, void* stream);

/* Prepare one query's prefix on the device from the context itself: each
 * layer's context K/V = hidden states times that layer's ctx_k / ctx_v, K
 * rotated at the row's count position (the number of visible rows before it),
 * written into the static buffers as ae_set_prefix_kv would write the result.
 * With a robot state, state_in turns it into one more context row, placed
 * after the visible context rows (its position is their count), projected by
 * every layer like them.
 * Defined by: MolmoBot PR Part 2 (prepare_cross_context / precompute_kv: the
 * context K/V and the state, projected once per query, reused by every flow
 * step); LoongForge blog section 1 (pads do not advance positions).
 * Arguments: hidden is device [L][batch][prefix_len][context_width] bf16 (the
 * VLM's per-layer hidden states of the context), valid_mask device
 * [batch][prefix_len] uint8 (0 = invisible: padding, an empty camera slot;
 * invisible rows are never stored, so NaN there is harmless), state device
 * [batch][state_dim] fp32 or NULL.  The prefix then holds n_b = visible rows
 * (+1 with a state); its bucket is chosen for prefix_len (+1).
 * Errors (before any state change): UNSUPPORTED without context_width (or a
 * state without state_dim), SHAPE_MISMATCH for batch outside [1, max_batch]
 * or prefix_len (+1 with a state) outside [0, max_prefix_len],
 * INVALID_ARGUMENT for a null hidden / mask with prefix_len > 0, NOT_READY
 * without weights.  Stream-ordered; the caller may reuse its buffers once the
 * stream passes the call. */
ae_status ae_prepare_prefix(ae_handle* h, int batch, int prefix_len, const void* hidden,
                            const uint8_t* valid_mask, const float* state, void* stream);

/* Configure prefix-length buckets: lengths[0..n) strictly increasing, each in
 * [1, max_prefix_len], n <= 32 (n = 0: one bucket, max_prefix_len).  Takes
 * effect at the next ae_set_prefix_kv.
 * Defined by: sglang PR 34599 summary, implementation items 4-5 (opt-in
 * prompt bucketing: right padding with the mask False to the smallest bucket
 * that holds the prompt, so one graph serves the whole bucket; bucket lengths
 * must be positive, strictly increasing and within the maximum length).
 * Here a bucket sizes the attention's key splits and keys the graph cache.
 * Errors: INVALID_ARGUMENT (the handle is left unchanged). */
ae_status ae_set_prefix_buckets(ae_handle* h, const int* lengths, int n);

/* Integrate: x_0 = noise, x_{k+1} = x_k + dt * v(x_k, t_k), t_k = (N-k)/N,
 * dt = -1/N, N = steps; writes x_N.
 * Defined by: MolmoBot PR Part 2 (generate_actions runs the expert's flow
 * steps over the cached context; only the action queries and the timestep
 * change between steps); LoongForge blog sections 2-3 and 5.3 (adaRMS with
 * scale/shift/gate, gated residuals, gelu*up, rotate_half RoPE, masked
 * attention over the visible prefix and the action tokens, time MLP, action
 * in/out projections and final norm); sglang PR 34599 summary, items 2-3
 * (layout and sinusoid computed once per call; calls replayed from a bounded
 * graph cache).
 * Arguments: noise and actions_out are device [batch][T][A] fp32 and may
 * alias; batch must equal the last ae_set_prefix_kv batch.  Errors (before
 * any state change): INVALID_ARGUMENT for null buffers or steps outside
 * [1, max_steps], NOT_READY without weights or prefix, SHAPE_MISMATCH for
 * another batch.  Asynchronous on `stream`. */
ae_status ae_denoise(ae_handle* h, const float* noise, int batch, int steps,
                     float* actions_out, void* stream);

/* ae_denoise for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments, checks and result as ae_denoise; the call allocates
 * nothing and creates nothing (no graph, no event): it launches the kernels
 * directly, and their scratch (split-K and attention partials, split
 * counters, barrier flags, packet generation base) lives in a static device
 * array of 24 MiB in the library, one copy per GPU, held until the process
 * ends.  Errors: as ae_denoise, plus UNSUPPORTED (before any state change)
 * when the call's scratch exceeds 24 MiB (e.g. a very large batch on the
 * per-phase path; ae_denoise has no such limit), HIP when the array has no
 * address on this device.  Calls on one GPU share the array and keep the last
 * call's contents: calls that overlap on one GPU (from any handle, on any
 * stream) race and must not be issued. */
ae_status ae_denoise_static(ae_handle* h, const float* noise, int batch, int steps,
                            float* actions_out, void* stream);

/* Counters, plus the device error count; reading it synchronises with the
 * device (the one call besides create/destroy that does).  INVALID_ARGUMENT
 * for null arguments. */
ae_status ae_get_stats(const ae_handle* h, ae_stats* out);
/* The handle's last error message ("" if none); "null handle" for NULL. */
const char* ae_last_error(const ae_handle* h);
/* A static description of a status code. */
const char* ae_status_string(int s);
/* Synchronise the device, release every graph and buffer, free the handle.
 * NULL is ignored. */
void ae_destroy(ae_handle* h);

#ifdef __cplusplus
}
#endif

#endif /* AE_H */
