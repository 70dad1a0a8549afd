/*
 * ds3.h -- C ABI of the constant-shape transformer decode step on MI355X (gfx950).
 *
 * The library exposes an executor shaped like the one on the poot documentation's "Execution" page (section
 * "Per backend", the executor contract: load the weights once, step per token, reset the carried state, report
 * statistics, unload): ds3_load_weights, ds3_step(tokens, pos) -> logits, ds3_reset_state, ds3_stats_get and
 * ds3_destroy. Every call is extern "C" over plain pointers and sizes; no C++ or PyTorch type crosses it.
 *
 * Memory ownership: the CALLER allocates every device buffer the engine uses (sizes from ds3_query_buffers) and
 * passes their addresses to ds3_create; the engine borrows them until ds3_destroy. The addresses must stay fixed,
 * because the first step records a HIP graph whose kernel arguments point at them ("Execution" page, sections
 * "A constant-shape decode graph" and "Slot buffers": grids and buffer addresses stay constant so one capture
 * serves every position up to the capacity). The engine owns only its pinned host staging, its HIP events and
 * its graph objects. The HIP stream is the caller's (borrowed), or the engine's own when NULL is passed.
 *
 * Errors ("Execution" page, section "Failure handling"): every call returns a ds3_status and never aborts the
 * process. Argument errors leave the engine unchanged and touch no device state. A failed in-kernel check marks
 * the engine NEEDS_RESET (ds3_step refuses until ds3_reset_state). A device error or a wait that outlasts the
 * timeout POISONS the engine: every later call except ds3_last_error/ds3_destroy returns DS3_E_POISONED without
 * a HIP call. ds3_last_error gives a message for the last failure.
 *
 * Threading: one engine is used by one host thread at a time.
 */
#ifndef DS3_H
#define DS3_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DS3_ABI_VERSION 5u

typedef struct ds3_engine ds3_engine;

typedef enum {
  DS3_OK = 0,
  DS3_E_INVALID = 1,       /* bad argument (null pointer, token/pos/map out of range, wrong shape); no effect */
  DS3_E_UNSUPPORTED = 2,   /* configuration outside what the kernels implement; the message names the field */
  DS3_E_UNBOUND = 3,       /* ds3_load_weights: a (role, layer) the step needs was not supplied */
  DS3_E_NOT_LOADED = 4,    /* ds3_step before a successful ds3_load_weights */
  DS3_E_NEEDS_RESET = 5,   /* an earlier step failed after replay; call ds3_reset_state */
  DS3_E_KERNEL_CHECK = 6,  /* an in-kernel check failed during this step; the engine now needs a reset */
  DS3_E_TIMEOUT = 7,       /* a device wait outlasted timeout_ms; the engine is now poisoned */
  DS3_E_DEVICE_LOST = 8,   /* a HIP call failed; the engine is now poisoned */
  DS3_E_POISONED = 9       /* the engine was poisoned earlier; the call did not touch the device */
} ds3_status;

enum { DS3_F32 = 0, DS3_BF16 = 1 };                  /* weight and KV storage types */
enum { DS3_KV_CONTIGUOUS = 0, DS3_KV_PAGED = 1 };    /* KV layouts */
enum { DS3_GRAPH = 0, DS3_EAGER = 1 };               /* replay one captured graph, or launch every kernel */
/* Kernel plan. PER_OP: one kernel per operation (embed, then per layer QKV, attention, split combine (absent when
 * the attention takes one split), o-proj, gate/up, down; then the LM head). FUSED: the whole step as one persistent kernel whose phases are those
 * operations, separated by grid barriers (one block per compute unit; one row, bf16 weights and K/V, contiguous
 * layout, the 1B and 8B model shapes, cap a multiple of 32 x 128 positions per 8 kv heads, a 256-CU device).
 * AUTO picks FUSED where it applies (the faster of the two on MI355X) and PER_OP elsewhere. Both compute the same
 * step; the graph records whichever runs. FUSED needs all of its 256 blocks resident at once: work running
 * concurrently on the device that keeps compute units busy makes its grid barriers wait, and a wait past the
 * barrier limit (2 s) ends the step with DS3_E_KERNEL_CHECK, never a hang. */
enum { DS3_PLAN_AUTO = 0, DS3_PLAN_PER_OP = 1, DS3_PLAN_FUSED = 2 };
/* Fused-plan tracing. OFF: the step kernel carries no trace code (the production build). BARRIERS: every step
 * records each block's grid-barrier arrival and release times; PHASES: also each block's sub-phase clocks. Both
 * run a separately compiled, traced variant of the step kernel, a little slower than the untraced one. */
enum { DS3_TRACE_OFF = 0, DS3_TRACE_BARRIERS = 1, DS3_TRACE_PHASES = 2 };

/*
 * Model shape and step shape. Llama-style pre-norm decoder without biases: per layer RMSNorm, Q/K/V projection
 * with rotary embedding on q and k, K/V write at the step's position, attention over the KV capacity with the
 * positions after the current one hidden, o-projection, RMSNorm, SwiGLU feed-forward; then the final RMSNorm
 * and the LM head ("Models, Registry and the Driver" page, section "Shared components": embed, one layer scope
 * per layer with x += mixer(norm(x)); x += ffn(norm(x)), final norm, head).
 *
 * rows: sequences per step (1..16). Up to 4 rows run the projections as vector GEMVs, more on the matrix cores
 * (bf16 weights, widths multiples of 128); 2..4 rows also go to the matrix cores when their activations (rows x
 * max(d_model, ffn_dim, q width) floats) do not fit a compute unit's 160 KB LDS, e.g. 3 or 4 rows of the 8B shape
 * ("Models, Registry and the Driver" page, section "The Model": a step shape of any number of sequences).
 * cap: KV capacity per row (positions 0..cap-1). kv_layout CONTIGUOUS keeps
 * K and V as [layer][row][kv_head][cap][head_dim]; PAGED keeps a pool [layer][page][kv_head][page_size][head_dim]
 * of pool_pages pages addressed through a per-row page table (see ds3_set_slot_map). timeout_ms = 0 selects the
 * default of 600000 ms ("Execution" page, section "Failure handling": every device wait is bounded).
 */
typedef struct {
  uint32_t abi_version;        /* DS3_ABI_VERSION */
  int32_t n_layers, d_model, n_q_heads, n_kv_heads, head_dim, ffn_dim, vocab;
  float rms_eps;
  double rope_theta;
  int32_t rows, cap, kv_layout, page_size, pool_pages;
  int32_t weight_dtype, kv_dtype, exec_mode;
  uint32_t timeout_ms;
  int32_t kernel_plan;         /* DS3_PLAN_*; FUSED where it does not apply -> DS3_E_UNSUPPORTED */
  int32_t trace;               /* DS3_TRACE_*: fused plan, what every step records for ds3_phase_trace */
  int32_t prefill_rows;        /* 0: no prefill step; 1..64: ds3_prefill takes this many tokens per launch */
} ds3_config;

/* Device buffers the caller allocates for ds3_create, in this id order. */
enum {
  DS3_BUF_WEIGHTS = 0,   /* packed weights: filled by ds3_load_weights */
  DS3_BUF_KV = 1,        /* K and V state of every layer (contiguous or pool) */
  DS3_BUF_WORK = 2,      /* slot buffers, activations, attention partials, rotary table, error word */
  DS3_BUF_LOGITS = 3,    /* float32 [rows][vocab]: the step's output */
  DS3_NUM_BUFFERS = 4
};

typedef struct {
  int32_t id;
  char name[32];
  uint64_t bytes;
  uint32_t align;   /* required alignment of the device address, in bytes */
} ds3_buffer_req;

/* Weight roles: a weight is bound by what it is, not by a checkpoint's tensor name ("Execution" page, section
 * "Per backend": load_weights binds each weight by its typed role; a weight nothing names stays unbound). */
typedef enum {
  DS3_W_EMBED = 0,       /* [vocab, d_model] */
  DS3_W_ATTN_NORM = 1,   /* [d_model] per layer */
  DS3_W_Q = 2,           /* [n_q_heads*head_dim, d_model] per layer */
  DS3_W_K = 3,           /* [n_kv_heads*head_dim, d_model] per layer */
  DS3_W_V = 4,           /* [n_kv_heads*head_dim, d_model] per layer */
  DS3_W_O = 5,           /* [d_model, n_q_heads*head_dim] per layer */
  DS3_W_FFN_NORM = 6,    /* [d_model] per layer */
  DS3_W_GATE = 7,        /* [ffn_dim, d_model] per layer */
  DS3_W_UP = 8,          /* [ffn_dim, d_model] per layer */
  DS3_W_DOWN = 9,        /* [d_model, ffn_dim] per layer */
  DS3_W_FINAL_NORM = 10, /* [d_model] */
  DS3_W_LM_HEAD = 11,    /* [vocab, d_model] */
  DS3_W_NUM_ROLES = 12
} ds3_role;

/* One weight tensor: row-major [rows, cols] ([out, in] for matrices; cols = length for norm gains) of dtype
 * DS3_F32 or DS3_BF16 (bf16 words), equal to cfg.weight_dtype. `data` may be a host or a device address. */
typedef struct {
  int32_t role;
  int32_t layer;     /* -1 for EMBED, FINAL_NORM and LM_HEAD */
  int32_t dtype;
  int64_t rows, cols;
  const void* data;
} ds3_weight_src;

typedef struct {
  uint64_t steps;            /* successful ds3_step calls */
  uint64_t replays;          /* graph launches */
  uint64_t captures;         /* graph captures (graph mode: 1 for the step, 2 more at the first ds3_prefill) */
  int32_t kernels_per_step;  /* kernel launches (eager) or kernel nodes (graph) per step */
  int32_t state;             /* 0 ready, 1 not loaded, 2 needs reset, 3 poisoned */
  double last_host_us;       /* host time of the last ds3_step, slot write to logits ready */
  double last_gpu_us;        /* device time of the last step's kernels (HIP events) */
  int32_t attn_splits;       /* split count of the attention sweep over [cap] */
  int32_t kernel_plan;       /* the plan in use: DS3_PLAN_PER_OP or DS3_PLAN_FUSED */
  double last_submit_us;     /* host time of the last ds3_step spent issuing work (slot copy, launch or replay,
                                readback copies), without the wait for the device */
  uint64_t prefill_tokens;   /* tokens taken by successful ds3_prefill calls */
  double last_prefill_gpu_us; /* device time of the last ds3_prefill (every chunk) */
} ds3_stats;

/* Per-kernel device timing of one step, from HIP events around each launch on the engine's stream. */
typedef struct {
  char name[40];
  int32_t launches;     /* launches of this kernel per step */
  double total_us;      /* summed over the launches of one step, averaged over the iterations */
  double bytes;         /* algorithmic bytes the launches move per step (weights, swept K/V, writes) */
} ds3_kernel_time;

/* Sizes of the device buffers for `cfg`. `out` has room for *n_inout entries; on return *n_inout is
 * DS3_NUM_BUFFERS. Validates the configuration (DS3_E_UNSUPPORTED names the failing field). Every size follows from
 * the configuration alone ("Models, Registry and the Driver" page, section "The Driver": capacity sizes the buffers
 * and is part of the step's shape, while tokens, positions and sampler parameters are bound inputs), so the caller can
 * allocate them once and the addresses never change ("Execution" page, section "Slot buffers"). */
ds3_status ds3_query_buffers(const ds3_config* cfg, ds3_buffer_req* out, int32_t* n_inout);

/* Create an engine over caller-allocated device buffers (`dev_ptrs[i]` for buffer id i, n = DS3_NUM_BUFFERS),
 * on HIP stream `hip_stream` (a hipStream_t; NULL = the engine creates its own). Uploads the rotary table and
 * zeroes the work and KV buffers. On success *out owns the engine; release it with ds3_destroy. */
ds3_status ds3_create(const ds3_config* cfg, void* const* dev_ptrs, int32_t n, void* hip_stream, ds3_engine** out);

/* Bind and pack all weights in one call. Every (role, layer) must be present exactly once with its shape and
 * dtype; a missing one -> DS3_E_UNBOUND naming it; a duplicate, unknown role or wrong shape/dtype ->
 * DS3_E_INVALID. Copies from `data` (host or device) and returns when the copies are done. */
ds3_status ds3_load_weights(ds3_engine* e, const ds3_weight_src* w, int32_t n);

/* Paged layout only: the per-row page table, int32 [rows][cap/page_size] of physical page ids in
 * [0, pool_pages). Rows must not share pages. Copied to its slot buffer; it stays until the next call. This is the
 * per-step SlotMap input of the "Execution" page, section "Slot buffers" (a device buffer at a stable address whose
 * contents the host rewrites), through which the sweep reads and from which the K/V write target is derived
 * (section "A constant-shape decode graph": the ScatterUpdate through the WriteMap for paged K/V). */
ds3_status ds3_set_slot_map(ds3_engine* e, const int32_t* slot_map);

/* One decode step for every row r: take token tokens[r] at absolute position pos[r] (0 <= pos < cap), write its
 * K/V at that position (contiguous: the position itself; paged: flat pool slot write_map[r], or, when write_map
 * is NULL, slot_map[r][pos/page_size]*page_size + pos%page_size), attend over positions 0..pos[r], and produce
 * logits float32 [rows][vocab] in the DS3_BUF_LOGITS buffer ("Execution" page, sections "A constant-shape decode
 * graph" and "Slot buffers"; "Models, Registry and the Driver" page, section "The Model": positions are absolute,
 * so positions need not be consecutive and a prefill is a sequence of steps). K/V of positions below pos[r] must
 * already be in the state (earlier steps or ds3_write_kv). The first step in graph mode captures the kernel
 * sequence into a HIP graph; every step replays it. If logits_host is not NULL the logits are also copied there.
 * flags (may be NULL) receives bit 0 = some logit is NaN or infinite (not an error by itself).
 * Paged layout: every step needs the page table (ds3_set_slot_map first, else DS3_E_INVALID), because the sweep
 * reads every position through it; an explicit write_map[r] must equal the page-table slot of pos[r] given above
 * (else DS3_E_INVALID: a K/V row written elsewhere would never be read at pos[r]). */
ds3_status ds3_step(ds3_engine* e, const int32_t* tokens, const int32_t* pos, const int32_t* write_map,
                    float* logits_host, uint32_t* flags);

/* Every step ends with the greedy pick on the device: for each row the index of its largest logit (the first
 * such index on ties; a NaN logit is never picked; all NaN -> 0) is written into the row's token slot and
 * pos + 1 into its position slot (paged: and the K/V write slot of pos + 1, from the page table), so the next
 * step can run without the host ("Execution" page, section "A constant-shape decode graph": the token a step
 * emits feeds the next step; "Slot buffers": a replay reads its inputs from device slots).
 *
 * ds3_step_greedy runs n_steps (1..DS3_MAX_CHAIN) such steps back to back with ONE host wait: the first from
 * tokens[r] at pos[r], each later one from the previous step's pick at the next position; pos[r] + n_steps must
 * not pass cap, and the paged layout needs the page table (ds3_set_slot_map) to cover those positions. ids
 * (host, int32 [n_steps][rows]) receives the picks, step by step; flags (host, uint32 [n_steps], may be NULL)
 * receives each step's non-finite bit (bit 0: some logit of that step is NaN or infinite). The logits of the last
 * step stay in the DS3_BUF_LOGITS buffer. Errors as for ds3_step; after an in-kernel check failure the whole run's
 * results are void (DS3_E_KERNEL_CHECK). */
#define DS3_MAX_CHAIN 1024
ds3_status ds3_step_greedy(ds3_engine* e, const int32_t* tokens, const int32_t* pos, int32_t n_steps,
                           int32_t* ids, uint32_t* flags);

/* Sampling suffix ("Models, Registry and the Driver" page, section "The Driver", item "The sampling suffix": every
 * sampling rule runs on the device, appended to the decode graph, with penalties and a logit bias read from a
 * per-sequence token history the device keeps and updates with every token it draws; the host reads back the
 * token id, a non-finite flag and, when asked, the top-n logprobs). The pages give no formulas; the readings:
 *   adjusted logits z_v = r(l_v) - presence * [c_v > 0] - frequency * c_v + bias_v, with c_v the row's history count
 *   of token v and r(x) = x / repetition_penalty if x > 0 else x * repetition_penalty when c_v > 0, r(x) = x
 *   otherwise (a NaN logit counts as -inf);
 *   temperature 0: greedy (first index of the largest z). Temperature T > 0: s = z / T, tokens ranked by (s
 *   descending, index ascending); top_k keeps the k best ranked (0: all); top_p keeps the shortest ranked prefix of
 *   those whose softmax(s) mass reaches top_p (1: all); min_p keeps the tokens whose probability is at least min_p
 *   times the top token's (0: all); the token is drawn by inverse CDF in index order over the kept weights, with
 *   u = the top 24 bits of output d of SplitMix64 seeded with `seed` (d = the row's draw count, reset to 0 by
 *   ds3_set_sampling) times 2^-24. Weights are exp(s - s_max) in 2^-40 fixed point, so the cuts are exact integer
 *   decisions on the device;
 *   logprobs: log-softmax of s (T = 1 for greedy) over every token: the drawn token's, then the top n by rank. */
#define DS3_MAX_LOGPROBS 8
typedef struct {
  float temperature;         /* >= 0; 0 = greedy */
  float top_p;               /* (0, 1]; 1 = off */
  float min_p;               /* [0, 1); 0 = off */
  float repetition_penalty;  /* > 0; 1 = off */
  float presence_penalty;    /* 0 = off */
  float frequency_penalty;   /* 0 = off */
  int32_t top_k;             /* >= 0; 0 = off */
  int32_t n_logprobs;        /* 0 .. DS3_MAX_LOGPROBS */
  uint64_t seed;
} ds3_sampling;

/* Row `row`'s sampling parameters for the following ds3_step_sample calls (default: greedy, no penalties); resets
 * the row's draw count. DS3_E_INVALID for a parameter out of range. */
ds3_status ds3_set_sampling(ds3_engine* e, int32_t row, const ds3_sampling* params);

/* Seed row `row`'s history: the counts of `tokens` (host int32 [n], e.g. the prompt) and the logit bias (host
 * float32 [vocab], NULL = none). The sampler adds each token it draws to the counts. */
ds3_status ds3_set_history(ds3_engine* e, int32_t row, const int32_t* tokens, int32_t n, const float* bias);

/* As ds3_step_greedy (n_steps chained steps, one host wait), with each row's token drawn by the sampling suffix.
 * logprobs (host float32 [n_steps][rows][1 + DS3_MAX_LOGPROBS], may be NULL): the drawn token's logprob, then the
 * top n_logprobs; logprob_ids (host int32 [n_steps][rows][DS3_MAX_LOGPROBS], may be NULL): their token ids. Slots
 * beyond a row's n_logprobs are unspecified. */
ds3_status ds3_step_sample(ds3_engine* e, const int32_t* tokens, const int32_t* pos, int32_t n_steps, int32_t* ids,
                           uint32_t* flags, float* logprobs, int32_t* logprob_ids);

/* Prefill (the step before decode): n tokens of one row at positions pos0 .. pos0 + n - 1, with their K/V written
 * into that row's state ("Models, Registry and the Driver" page, section "The Model": positions are absolute, and
 * a prefill is the same step taken from a given position, in chunks). The tokens go prefill_rows at a time through
 * one launch sequence (one graph replay): chunk k is a step of prefill_rows activation rows that all read and write the same K/V row, token
 * t of the chunk at position pos0 + k prefill_rows + t, so its attention sees the K/V of the chunk's earlier tokens
 * (written by the same step before the attention runs) and nothing after its own position -- the causal mask
 * inside the chunk is the position mask of the decode step. Chunks run their projections on the matrix cores
 * under the same rule as decode rows (see the rows field of ds3_config); a chunk of 17..64 rows takes four
 * 16-row activation tiles per weight tile, so its weights stream once for up to 64 tokens. The rows after the
 * last token of the last chunk repeat that token at its position. logits_host (float32
 * [vocab], may be NULL) receives the last token's logits, from which the first decode step's token is picked;
 * only the last chunk runs the final norm and the LM head (the other chunks' logits are never used, so their
 * launch sequence, a graph of its own, stops after the last layer). flags (may be NULL) bit 0: some logit of the
 * last chunk was NaN or infinite. n in 1..DS3_MAX_PREFILL; pos0 + n must
 * not pass cap; paged layout: the page table must be set. DS3_E_UNSUPPORTED when the engine was created with
 * prefill_rows = 0; other errors as ds3_step. */
#define DS3_MAX_PREFILL 8192
ds3_status ds3_prefill(ds3_engine* e, int32_t row, const int32_t* tokens, int32_t pos0, int32_t n,
                       float* logits_host, uint32_t* flags);

/* K/V sweep of the attention, from the next step on (a slot word: no recapture). FULL (the default) loads every
 * position of [cap], as the method does ("Execution" page, section "A constant-shape decode graph": the sweep
 * covers the whole preallocated capacity and the mask hides what lies after pos). VISIBLE skips loading (and
 * computing) the K/V chunks whose positions all lie after pos: the grid and every address stay the same, so the
 * captured graph still serves every position, and the outputs are bit-identical to FULL (a hidden position
 * contributes nothing either way). It goes beyond the pages and moves fewer bytes than the method's count.
 * DS3_E_INVALID for any other mode. */
enum { DS3_SWEEP_FULL = 0, DS3_SWEEP_VISIBLE = 1 };
ds3_status ds3_set_kv_sweep(ds3_engine* e, int32_t mode);

/* Zero every row's K/V state and the step's scratch state; clears NEEDS_RESET. Keeps weights and the graph. */
ds3_status ds3_reset_state(ds3_engine* e);

/* Write / read K and V of `n` logical positions pos0..pos0+n-1 of one row and layer. `k` and `v` are host arrays
 * [n_kv_heads][n][head_dim] in the KV dtype (float32 or bf16 words). Paged layout maps positions through the
 * row's page table. The K/V cache is the state the step program carries ("Models, Registry and the Driver" page,
 * section "The Model": the states of a program, the KV cache among them); writing it sets a sequence's state at a
 * position (e.g. a pre-filled context), and reading it lets a check compare every element of the carried state
 * with the oracle ("Execution" page, section "Verification", the stated-tolerance tier). */
ds3_status ds3_write_kv(ds3_engine* e, int32_t layer, int32_t row, int32_t pos0, int32_t n, const void* k,
                        const void* v);
ds3_status ds3_read_kv(ds3_engine* e, int32_t layer, int32_t row, int32_t pos0, int32_t n, void* k, void* v);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation): ds3_write_kv without any allocation. ds3_write_kv stages K and V through a device
 * buffer the library allocates on first use; this call stages them through a fixed device array of
 * DS3_NOALLOC_MAX_BYTES that the library holds on every GPU it runs on until the process ends, and transposes V on
 * the device. Same arguments, layout and result as ds3_write_kv (k, v: [n_kv_heads][n][head_dim] in the KV dtype,
 * host or device memory). 2 * n_kv_heads * n * head_dim * (2 or 4 bytes) must not exceed DS3_NOALLOC_MAX_BYTES
 * (else DS3_E_INVALID, nothing written). It calls no hipMalloc, hipFree or other allocating routine. Every call on
 * one GPU shares that GPU's array: calls that overlap on one GPU (several threads, or engines on different streams
 * at once) race and must be serialized by the caller; one call has finished with the array when it returns. */
#define DS3_NOALLOC_MAX_BYTES (8u << 20)
ds3_status ds3_write_kv_noalloc(ds3_engine* e, int32_t layer, int32_t row, int32_t pos0, int32_t n, const void* k,
                                const void* v);

ds3_status ds3_stats_get(const ds3_engine* e, ds3_stats* out);

/* Per kernel kind, the device time of one step's launches of that kind: they are captured as a graph of their
 * own (in step order, with the current slot contents) and replayed `iters` times between two HIP events on the
 * engine's stream. With the FUSED plan the one kernel is timed that way (kind "decode_step_fused"), and each
 * operation kind reports its phases' share of it: the time between the grid barriers that close them, read from
 * block 0's clock over `iters` further launches (launches = phases per step). Afterwards one whole step runs again with the same slots, so the K/V entries at the slot
 * positions and the work buffers hold what the last step left. `out` has room for *n_inout entries (at least the
 * number of kinds); on return *n_inout is the number of kinds. A HIP failure poisons the engine. */
ds3_status ds3_profile_kernels(ds3_engine* e, int32_t iters, ds3_kernel_time* out, int32_t* n_inout);

/* Fused plan only: the grid-barrier trace of the last step, uint64 [5 n_layers][256 blocks][2] = each block's
 * wall-clock time (100 MHz ticks) when it arrived at the barrier and when it was released; the barriers close the
 * QKV, attention, o-proj, gate/up and down phases of each layer in order. With room for five times as many words,
 * [5 n_layers][256][8] sub-phase clocks follow (zero unless the engine was created with trace =
 * DS3_TRACE_PHASES): GEMV phases -- start, first batch consumed, batches done, block done; attention -- start, inputs
 * in, sweep done, partial stored, all splits flagged, merge stored. *n_inout: room in `out` on entry, words
 * written on return. DS3_E_UNSUPPORTED with the per-operation plan or an engine created with trace = OFF. */
ds3_status ds3_phase_trace(ds3_engine* e, uint64_t* out, int32_t* n_inout);

/* Test hook for the failure path: DS3_INJECT_KERNEL_CHECK makes the next step's first kernel raise its check
 * bit, so that step returns DS3_E_KERNEL_CHECK and the engine needs a reset. DS3_INJECT_TIMEOUT_NEXT sets the
 * next step's wait limit to 0 ms so that it reports DS3_E_TIMEOUT (the kernels themselves run normally).
 * DS3_INJECT_BARRIER_TIMEOUT (fused plan) sets the next step's grid-barrier wait limit to one clock tick: the
 * blocks stop waiting for each other, the step's results are void, and it returns DS3_E_KERNEL_CHECK. */
enum { DS3_INJECT_KERNEL_CHECK = 1, DS3_INJECT_TIMEOUT_NEXT = 2, DS3_INJECT_BARRIER_TIMEOUT = 3 };
ds3_status ds3_debug_inject(ds3_engine* e, int32_t kind);

/* Measurement only, outside the step: enqueue one streaming read of `bytes` (a multiple of 16) of device memory
 * `buf` on HIP stream `hip_stream` (a hipStream_t; NULL = the null stream), with the access pattern the weight
 * streams use (16-byte non-temporal loads, 1 KB contiguous per wave instruction). `sink` is device memory of at
 * least 4096 bytes that the kernel may write (its contents carry no meaning). Returns after the launch (time it
 * with events on the stream). DS3_E_INVALID for a bad argument, DS3_E_DEVICE_LOST if the launch fails. */
ds3_status ds3_probe_read(const void* buf, uint64_t bytes, void* sink, void* hip_stream);

/* Message of the engine's last failure ("" if none); engine-owned, valid until the next call. With e == NULL,
 * the last failure of ds3_query_buffers/ds3_create on this thread. */
const char* ds3_last_error(const ds3_engine* e);

/* Release the engine (graph, events, staging). The caller's device buffers are not freed. */
void ds3_destroy(ds3_engine* e);

#ifdef __cplusplus
}
#endif

#endif /* DS3_H */
