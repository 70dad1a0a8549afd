// Host side of the decode-step library: configuration checks, buffer plan, weight packing, slot buffers,
// HIP-graph capture and replay, bounded waits and the engine's error state machine. See include/ds3.h.
#include "ds3.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "ds3_kernels.h"

using namespace ds3;

static_assert(kScratchBytes == DS3_NOALLOC_MAX_BYTES, "the scratch array is the size the header states");

namespace {

enum EngineState { ST_READY = 0, ST_NOT_LOADED = 1, ST_NEEDS_RESET = 2, ST_POISONED = 3 };
constexpr uint32_t kDefaultTimeoutMs = 600000;  // "Execution" page, section "Failure handling": 600 s default
constexpr size_t kAlign = 256;

thread_local std::string g_last_error;

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
size_t dtype_bytes(int dt) { return dt == DS3_BF16 ? 2 : 4; }

struct WorkPlan {
  size_t slots, status, x, q, attn, act, part, pre_slots, pre_logits, kvnew, sync, clocks, trace, pick_val, pick_idx,
      pick_done, ids, chain_flags, samp_rows, counts, bias, draws, zbuf, samp_part, lp, lp_ids, rope, slot_map, frag_hi, frag_lo,
      skpart, skss, total;
};

struct KernelKind {
  const char* name;
};
enum Kind { K_EMBED = 0, K_QKV, K_ATTN, K_OPROJ, K_GATEUP, K_DOWN, K_HEAD, K_SPLIT, K_COMBINE, K_FUSED, K_PICK, K_SAMPLE,
            K_QKVFIN, K_SWIGLU, K_NUM };
const char* kKindNames[K_NUM] = {"embed", "qkv_rope_kvwrite", "attention_splitk", "o_proj_residual",
                                 "gateup_swiglu", "down_proj_residual", "lm_head", "norm_prep_mfma",
                                 "attention_combine", "decode_step_fused", "greedy_pick", "sampler",
                                 "qkv_epilogue_mfma", "swiglu_split_mfma"};
constexpr int kMaxChain = DS3_MAX_CHAIN;   // steps of one ds3_step_greedy call
constexpr int kMaxPrefill = DS3_MAX_PREFILL;   // tokens of one ds3_prefill call
// fused plan: the operation kind of phase k of a layer (the grid barrier after it closes the phase)
const int kPhaseKind[kFusedPhases] = {K_QKV, K_ATTN, K_OPROJ, K_GATEUP, K_DOWN};

// RMSNorm sites of the MFMA path: a prep kernel adds the producing projection's partial products into x, writes
// the per-block sums of squares and the fragments of gain * x
enum Site { S_ATTN_NORM = 0, S_FFN_NORM, S_FINAL_NORM };

struct Launch {
  int kind;
  int layer;
  int site;
};

}  // namespace

struct ds3_engine {
  ds3_config cfg{};
  void* buf[DS3_NUM_BUFFERS]{};
  hipStream_t stream = nullptr;
  bool own_stream = false;
  int device = 0;

  // work buffer views
  int* slots = nullptr;
  StatusWords* status = nullptr;
  float *x = nullptr, *q = nullptr, *attn = nullptr, *act = nullptr, *part = nullptr, *rope = nullptr;
  int* slot_map = nullptr;
  float* logits = nullptr;
  uint16_t *frag_hi = nullptr, *frag_lo = nullptr;   // MFMA path: activation operands
  float *skpart = nullptr, *skss = nullptr;          // MFMA path: partial products, per-block sums of squares
  bool mfma = false;                                 // projections on the matrix cores (rows_on_mfma)
  bool fused = false;                                // the whole step as one persistent kernel
  float* kvnew = nullptr;                            // fused: this step's k and v [nkv][2][hd]
  unsigned* sync = nullptr;                          // fused: barrier and merge counters
  unsigned long long* clocks = nullptr;              // fused: block 0's clock per barrier
  unsigned long long* trace = nullptr;               // fused: every block's arrival and release per barrier
  bool profiling = false;                            // fused: profile_kernels' own launches record the clocks
  int32_t kv_sweep = DS3_SWEEP_FULL;                 // written into the sweep slot word every step
  float* pick_val = nullptr;                         // greedy pick: per-slice maxima [rows][kPickSplit]
  int* pick_idx = nullptr;
  unsigned* pick_done = nullptr;
  int32_t* ids = nullptr;                            // [kMaxChain][rows] picks of a chain of steps
  uint32_t* chain_flags = nullptr;                   // [kMaxChain] non-finite flag of each step
  SampleRow* samp_rows = nullptr;                    // sampling suffix: per-row parameters (uploaded per call)
  int32_t* counts = nullptr;                         // [rows][vocab] token history
  float* bias = nullptr;                             // [rows][vocab] logit bias
  uint32_t* draws = nullptr;                         // [rows] draws so far (the generator's counter)
  float* zbuf = nullptr;                             // [rows][vocab] adjusted logits (scratch)
  SampPart* samp_part = nullptr;                     // [rows][segments] the sampler's segment records (scratch)
  float* lp = nullptr;                               // [kMaxChain][rows][1 + kMaxLogprobs] logprobs
  int32_t* lp_ids = nullptr;                         // [kMaxChain][rows][kMaxLogprobs]
  std::vector<SampleRow> h_samp;                     // host copy of the per-row parameters
  std::vector<Launch> samp_sequence;                 // the step with the sampler as its pick
  hipGraph_t samp_graph = nullptr;
  hipGraphExec_t samp_exec = nullptr;
  bool samp_captured = false;
  SampleRow* h_samp_pinned = nullptr;                // pinned staging of h_samp
  float* h_lp = nullptr;                             // pinned: logprobs and their ids of the last call
  size_t sync_words = 0;
  size_t weight_lstride = 0;                         // bytes between consecutive layers' weights
  size_t work_bytes = 0;

  // weights
  struct LayerW {
    float* attn_norm;
    void* wqkv;
    void* wo;
    float* ffn_norm;
    void* wgu;
    void* wd;
  };
  std::vector<LayerW> L;
  void* embed = nullptr;
  float* final_norm = nullptr;
  void* lm_head = nullptr;

  KvView kv{};
  size_t kv_bytes = 0;
  int splits = 1, split_len = 1;
  int blocks[K_NUM]{};

  // host state
  int32_t* h_slots = nullptr;   // pinned: slot words followed by the two status words (zeroed every step)
  StatusWords* h_status = nullptr;
  int32_t* h_chain = nullptr;   // pinned: [kMaxChain][rows] picks, then [kMaxChain] flags, of the last call
  std::vector<int32_t> h_slot_map;
  bool slot_map_set = false;
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  bool captured = false;
  int graph_nodes = 0;
  hipEvent_t ev0 = nullptr, ev1 = nullptr, ev_done = nullptr;
  bool pending = false;   // work was enqueued that may still be running (after a timeout)
  int state = ST_NOT_LOADED;
  bool inject_check = false;
  bool inject_timeout = false;
  bool inject_barrier = false;
  ds3_stats stats{};
  std::string err;
  void* kv_staging = nullptr;
  size_t kv_staging_bytes = 0;
  void* scratch = nullptr;   // this device's allocation-free staging array (ds3_write_kv_noalloc)
  std::vector<Launch> sequence;

  // what enqueue_kernel launches for: the decode step (cfg.rows rows) or the prefill step (prefill_rows tokens
  // of one K/V row); both share the work buffers, weights and K/V
  struct RunCtx {
    int rows = 0;
    int* slots = nullptr;
    float* logits = nullptr;
    bool mfma = false;            // projections on the matrix cores (rows_on_mfma)
    const int* row_map = nullptr; // K/V row of each activation row (null: the row itself)
    int splits = 0, split_len = 0;  // attention split plan of a step of `rows` rows
  };
  RunCtx dec, pre, cur;
  std::vector<Launch> pre_sequence;
  hipGraph_t pre_graph = nullptr;
  hipGraphExec_t pre_exec = nullptr;
  // the prefill step without its final norm and LM head, for every chunk but the last (their logits are not used)
  size_t pre_body = 0;   // launches of pre_sequence before the final norm / head
  hipGraph_t pre_body_graph = nullptr;
  hipGraphExec_t pre_body_exec = nullptr;
  bool pre_captured = false;
  int32_t* h_pre = nullptr;   // pinned: the slot words of every chunk of one ds3_prefill call
};

namespace {

ds3_status fail(ds3_engine* e, ds3_status st, const std::string& msg) {
  if (e) e->err = msg;
  else g_last_error = msg;
  return st;
}

ds3_status poison(ds3_engine* e, ds3_status st, const std::string& msg) {
  e->state = ST_POISONED;
  return fail(e, st, msg);
}

#define HIP_OR_POISON(e, call)                                                                          \
  do {                                                                                                  \
    hipError_t _h = (call);                                                                             \
    if (_h != hipSuccess)                                                                               \
      return poison((e), DS3_E_DEVICE_LOST, std::string(#call) + ": " + hipGetErrorString(_h));         \
  } while (0)

void plan_splits(const ds3_config& c, int rows, int* splits, int* split_len);

// Why the fused step kernel cannot run this configuration ("" if it can, device aside).
std::string fused_refusal(const ds3_config& c) {
  if (c.rows != 1) return "rows must be 1";
  if (c.weight_dtype != DS3_BF16 || c.kv_dtype != DS3_BF16) return "weights and K/V must be bf16";
  if (c.kv_layout != DS3_KV_CONTIGUOUS) return "K/V must be contiguous";
  if (!fused_shape_supported(c.d_model, c.ffn_dim, c.head_dim, c.n_q_heads, c.n_kv_heads))
    return "no compiled instantiation for this model shape";
  const int S = kFusedBlocks / c.n_kv_heads;
  if (c.cap % (128 * S) != 0) return "cap must be a multiple of 128 positions per split";
  if (c.vocab < 16 * kFusedBlocks || c.vocab > 520 * kFusedBlocks) return "vocab out of the LM head's range";
  return "";
}

// Whether a step of R activation rows runs its projections on the matrix cores: above kMaxGemvRows rows, and for
// 2..4 rows too when the vector path's activations (R x the widest input, float32, in LDS) do not fit a CU's LDS.
bool rows_on_mfma(const ds3_config& c, int R) {
  if (R > kMaxGemvRows) return true;
  const int kres = std::max(c.ffn_dim, c.n_q_heads * c.head_dim);
  return gemv_lds_bytes(R, c.d_model, true) > 160 * 1024 || gemv_lds_bytes(R, kres, false) > 160 * 1024;
}

std::string check_config(const ds3_config* c) {
  if (!c) return "config is NULL";
  if (c->abi_version != DS3_ABI_VERSION) return "abi_version mismatch";
  if (c->n_layers < 1) return "n_layers must be >= 1";
  if (c->d_model < 8 || c->d_model % 8) return "d_model must be a positive multiple of 8";
  if (c->head_dim != 64 && c->head_dim != 128) return "head_dim must be 64 or 128";
  if (c->n_q_heads < 1 || c->n_kv_heads < 1 || c->n_q_heads % c->n_kv_heads) return "n_q_heads must be a multiple of n_kv_heads";
  {
    const int G = c->n_q_heads / c->n_kv_heads;
    if (G != 1 && G != 2 && G != 4 && G != 8) return "n_q_heads / n_kv_heads must be 1, 2, 4 or 8";
  }
  if (c->ffn_dim < 8 || c->ffn_dim % 8) return "ffn_dim must be a positive multiple of 8";
  if (c->vocab < 2 || c->vocab % 2) return "vocab must be even and >= 2";
  if (!(c->rms_eps >= 0.f)) return "rms_eps must be >= 0";
  if (!(c->rope_theta > 1.0)) return "rope_theta must be > 1";
  if (c->rows < 1 || c->rows > kMaxRows) return "rows must be in 1..16";
  if (c->cap < 1) return "cap must be >= 1";
  if (c->weight_dtype != DS3_F32 && c->weight_dtype != DS3_BF16) return "weight_dtype must be DS3_F32 or DS3_BF16";
  if (c->kv_dtype != DS3_F32 && c->kv_dtype != DS3_BF16) return "kv_dtype must be DS3_F32 or DS3_BF16";
  if (c->exec_mode != DS3_GRAPH && c->exec_mode != DS3_EAGER) return "exec_mode must be DS3_GRAPH or DS3_EAGER";
  if (c->kernel_plan != DS3_PLAN_AUTO && c->kernel_plan != DS3_PLAN_PER_OP && c->kernel_plan != DS3_PLAN_FUSED)
    return "kernel_plan must be DS3_PLAN_AUTO, DS3_PLAN_PER_OP or DS3_PLAN_FUSED";
  if (c->trace != DS3_TRACE_OFF && c->trace != DS3_TRACE_BARRIERS && c->trace != DS3_TRACE_PHASES)
    return "trace must be DS3_TRACE_OFF, DS3_TRACE_BARRIERS or DS3_TRACE_PHASES";
  if (c->kv_layout == DS3_KV_PAGED) {
    if (c->page_size < 1) return "page_size must be >= 1";
    if (c->cap % c->page_size) return "cap must be a multiple of page_size";
    if (c->pool_pages < 1) return "pool_pages must be >= 1";
    if ((int64_t)c->pool_pages * c->page_size > INT32_MAX) return "pool_pages * page_size must fit int32";
    if (c->page_size & (c->page_size - 1)) return "page_size must be a power of two";
  } else if (c->kv_layout != DS3_KV_CONTIGUOUS) {
    return "kv_layout must be DS3_KV_CONTIGUOUS or DS3_KV_PAGED";
  }
  if (c->kv_dtype == DS3_BF16) {
    // matrix-core attention: V is stored transposed and read in groups of 8 positions
    if (c->cap % 8) return "cap must be a multiple of 8 with bf16 K/V";
    if (c->kv_layout == DS3_KV_PAGED && c->page_size < 8) return "page_size must be >= 8 with bf16 K/V";
  }
  {
    const int64_t per_layer = c->kv_layout == DS3_KV_PAGED
                                  ? (int64_t)c->pool_pages * c->n_kv_heads * c->page_size * c->head_dim
                                  : (int64_t)c->rows * c->n_kv_heads * c->cap * c->head_dim;
    if (per_layer > INT32_MAX) return "cap / pool_pages: one layer's K must hold fewer than 2^31 elements";
  }
  for (const int R : {c->rows, c->prefill_rows}) {
    if (R < 1) continue;
    int splits = 0, split_len = 0;
    plan_splits(*c, R, &splits, &split_len);
    if (attn_lds_bytes(c->n_q_heads, c->n_kv_heads, c->head_dim, split_len, c->kv_dtype,
                       c->kv_layout == DS3_KV_PAGED ? c->page_size : 0) > 160 * 1024)
      return "cap / page_size: the attention page table of a split does not fit the 160 KB LDS";
  }
  if (c->kernel_plan == DS3_PLAN_FUSED) {
    const std::string why = fused_refusal(*c);
    if (!why.empty()) return "kernel_plan: the fused step kernel does not apply (" + why + ")";
  }
  if (c->prefill_rows < 0 || c->prefill_rows > kMaxPrefillRows) return "prefill_rows must be in 0..64";
  for (const int R : {c->rows, c->prefill_rows}) {
    if (R == 0) continue;
    const char* what = R == c->rows ? "rows" : "prefill_rows";
    if (!rows_on_mfma(*c, R)) continue;
    // matrix-core path: bf16 weights in whole 16-row tiles and 32-input steps
    const std::string why_gemv = R <= kMaxGemvRows ? " (the vector path's activations of rows x max(d_model, "
                                                     "ffn_dim, q width) floats exceed the 160 KB LDS)" : "";
    if (c->weight_dtype != DS3_BF16)
      return std::string(what) + ": the matrix-core path needs bf16 weights" + why_gemv;
    if (c->d_model % kSkChunk || c->ffn_dim % kSkChunk || (c->n_q_heads * c->head_dim) % kSkChunk)
      return std::string(what) + ": d_model, ffn_dim and n_q_heads x head_dim must be multiples of 128 on the "
             "matrix-core path" + why_gemv;
    if (c->head_dim % 32 || c->vocab % 32)
      return std::string(what) + ": head_dim and vocab must be multiples of 32 on the matrix-core path" + why_gemv;
    const int qkv = (c->n_q_heads + 2 * c->n_kv_heads) * c->head_dim, qw = c->n_q_heads * c->head_dim;
    if (!sk_plan(qkv, c->d_model, false).groups || !sk_plan(c->d_model, qw, false).groups ||
        !sk_plan(2 * c->ffn_dim, c->d_model, false).groups || !sk_plan(c->d_model, c->ffn_dim, false).groups ||
        !sk_plan(c->vocab, c->d_model, true).groups)
      return std::string(what) + ": vocab, d_model, 2 x ffn_dim and (n_q_heads + 2 n_kv_heads) x head_dim must be "
             "multiples of 128 on the matrix-core path" + why_gemv;
  }
  return "";
}

// Attention split plan of a step of `rows` rows (the decode rows, or a prefill chunk's tokens): about kAttnBlocks
// blocks over rows x kv heads x splits (measured best among 256..1024 on MI355X). A split is a whole number of LDS
// chunks, and there are no more splits than the in-kernel merge takes. The plan is a function of the configuration
// and the step alone, so a step always reduces in the same order.
constexpr int kAttnBlocks = 512;
void plan_splits(const ds3_config& c, int rows, int* splits, int* split_len) {
  const int chunk = attn_positions_per_pass(c.head_dim, c.kv_dtype);
  const int units = (c.cap + chunk - 1) / chunk;
  int s = std::max(1, kAttnBlocks / (rows * c.n_kv_heads));
  s = std::min(s, units);
  s = std::min(s, attn_max_splits(c.n_q_heads, c.n_kv_heads, c.head_dim));
  const int per = (units + s - 1) / s;
  *split_len = per * chunk;
  *splits = (c.cap + *split_len - 1) / *split_len;
}

WorkPlan plan_work(const ds3_config& c, int splits) {
  WorkPlan w{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = align_up(off + bytes, kAlign);
    return at;
  };
  const SlotLayout sl{c.rows};
  const int G = c.n_q_heads / c.n_kv_heads;
  const size_t RA = (size_t)std::max(c.rows, c.prefill_rows);   // activation rows of the larger step
  w.slots = take((size_t)sl.words() * 4);
  w.status = take(sizeof(StatusWords));
  w.x = take(RA * c.d_model * 4);
  w.q = take(RA * c.n_q_heads * c.head_dim * 4);
  w.attn = take(RA * c.n_q_heads * c.head_dim * 4);
  w.act = take(RA * c.ffn_dim * 4);
  size_t row_splits = RA * std::max(splits, kFusedBlocks / c.n_kv_heads);   // attention partials: rows x splits
  if (c.prefill_rows > 0) {
    int ps = 0, pl = 0;
    plan_splits(c, c.prefill_rows, &ps, &pl);
    row_splits = std::max(row_splits, (size_t)c.prefill_rows * ps);
  }
  w.part = take(row_splits * c.n_kv_heads * G * (c.head_dim + 4) * 4);
  w.pre_slots = take(c.prefill_rows ? (size_t)(SlotLayout{c.prefill_rows}.words() + c.prefill_rows) * 4 : 4);
  w.pre_logits = take(c.prefill_rows ? (size_t)c.prefill_rows * c.vocab * 4 : 4);
  w.kvnew = take((size_t)c.n_kv_heads * 2 * c.head_dim * 4);
  w.sync = take(fused_sync_words(c.n_layers, c.n_kv_heads) * 4);
  w.clocks = take(((size_t)kFusedPhases * c.n_layers + 2) * 8);
  w.trace = take((size_t)kFusedPhases * c.n_layers * kFusedBlocks * 10 * 8);   // barrier trace, then sub-phases
  w.pick_val = take((size_t)c.rows * kPickSplit * 4);
  w.pick_idx = take((size_t)c.rows * kPickSplit * 4);
  w.pick_done = take(4);
  w.ids = take((size_t)kMaxChain * c.rows * 4);
  w.chain_flags = take((size_t)kMaxChain * 4);
  w.samp_rows = take((size_t)c.rows * sizeof(SampleRow));
  w.counts = take((size_t)c.rows * c.vocab * 4);
  w.bias = take((size_t)c.rows * c.vocab * 4);
  w.draws = take((size_t)c.rows * 4);
  w.zbuf = take((size_t)c.rows * c.vocab * 4);
  w.samp_part = take((size_t)c.rows * samp_segments(c.vocab) * sizeof(SampPart));
  w.lp = take((size_t)kMaxChain * c.rows * (1 + kMaxLogprobs) * 4);
  w.lp_ids = take((size_t)kMaxChain * c.rows * kMaxLogprobs * 4);
  w.rope = take((size_t)c.cap * (c.head_dim / 2) * 2 * 4);
  w.slot_map = take(c.kv_layout == DS3_KV_PAGED ? (size_t)c.rows * (c.cap / c.page_size) * 4 : 4);
  const size_t kmax = (size_t)std::max(std::max(c.d_model, c.ffn_dim), c.n_q_heads * c.head_dim);
  const bool any_mfma = rows_on_mfma(c, c.rows) || (c.prefill_rows > 0 && rows_on_mfma(c, c.prefill_rows));
  const int nt_max = sk_tiles(std::max(c.rows, c.prefill_rows));   // activation tiles of the larger step
  const size_t frag = any_mfma ? kmax * kMfmaRows * nt_max * 2 : 16;
  w.frag_hi = take(frag);
  w.frag_lo = take(frag);
  size_t skp = 4;
  if (any_mfma) {
    const int qkv = (c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim, qw = c.n_q_heads * c.head_dim;
    for (const SkPlan& sp : {sk_plan(qkv, c.d_model, false), sk_plan(c.d_model, qw, false),
                             sk_plan(2 * c.ffn_dim, c.d_model, false), sk_plan(c.d_model, c.ffn_dim, false)})
      skp = std::max(skp, sk_partial_floats(sp, nt_max) * 4);
  }
  w.skpart = take(skp);
  w.skss = take((size_t)((c.d_model + kNormSpan - 1) / kNormSpan) * kSsRows * 4);
  w.total = off;
  return w;
}

size_t kv_state_bytes(const ds3_config& c) {
  const size_t per_layer = c.kv_layout == DS3_KV_PAGED
                               ? (size_t)c.pool_pages * c.n_kv_heads * c.page_size * c.head_dim
                               : (size_t)c.rows * c.n_kv_heads * c.cap * c.head_dim;
  return 2 * (size_t)c.n_layers * per_layer * dtype_bytes(c.kv_dtype);
}

struct WeightPlan {
  struct L {
    size_t attn_norm, wqkv, wo, ffn_norm, wgu, wd;
  };
  std::vector<L> layers;
  size_t embed, final_norm, lm_head, total;
};

WeightPlan plan_weights(const ds3_config& c) {
  WeightPlan p;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = align_up(off + bytes, kAlign);
    return at;
  };
  const size_t wb = dtype_bytes(c.weight_dtype);
  const size_t d = c.d_model, F = c.ffn_dim, qw = (size_t)c.n_q_heads * c.head_dim,
               kvw = (size_t)c.n_kv_heads * c.head_dim;
  for (int l = 0; l < c.n_layers; ++l) {
    WeightPlan::L L;
    L.attn_norm = take(d * 4);
    L.wqkv = take((qw + 2 * kvw) * d * wb);
    L.wo = take(d * qw * wb);
    L.ffn_norm = take(d * 4);
    L.wgu = take(2 * F * d * wb);
    L.wd = take(d * F * wb);
    p.layers.push_back(L);
  }
  p.embed = take((size_t)c.vocab * d * wb);
  p.final_norm = take(d * 4);
  p.lm_head = take((size_t)c.vocab * d * wb);
  p.total = off;
  return p;
}

// bytes a kind of kernel moves per step by the algorithm's count (streamed weights, swept and written K/V)
double kind_bytes(const ds3_config& c, int kind) {
  const double wb = (double)dtype_bytes(c.weight_dtype), kvb = (double)dtype_bytes(c.kv_dtype);
  const double d = c.d_model, F = c.ffn_dim, qw = (double)c.n_q_heads * c.head_dim,
               kvw = (double)c.n_kv_heads * c.head_dim, Lc = c.n_layers, R = c.rows;
  switch (kind) {
    case K_EMBED: return R * d * wb;
    case K_QKV: return Lc * ((qw + 2 * kvw) * d * wb + d * wb + R * 2 * kvw * kvb);
    case K_ATTN: return Lc * R * 2 * (double)c.cap * kvw * kvb;
    case K_OPROJ: return Lc * d * qw * wb;
    case K_GATEUP: return Lc * (2 * F * d * wb + d * wb);
    case K_DOWN: return Lc * d * F * wb;
    case K_HEAD: return (double)c.vocab * d * wb + d * wb;
    case K_PICK: return R * (double)c.vocab * 4;   // the logits, read once
    case K_SAMPLE: return R * (double)c.vocab * 12;   // logits, history and bias, read once
    case K_FUSED: {
      double t = 0;
      for (int k : {K_EMBED, K_QKV, K_ATTN, K_OPROJ, K_GATEUP, K_DOWN, K_HEAD}) t += kind_bytes(c, k);
      return t;
    }
  }
  return 0;
}

// GEMV launch: one resident round of waves (2 per SIMD at these kernels' register use: 8 per CU, 2048 on 256
// CUs, i.e. 2 blocks of 4 waves per CU); measured best among 256..4096 blocks.
int gemv_blocks(int n_pairs, int cus) { return std::max(1, std::min(2 * cus, (n_pairs + 3) / 4)); }

ds3_status wait_done(ds3_engine* e, hipEvent_t ev, uint32_t timeout_ms) {
  const auto t0 = std::chrono::steady_clock::now();
  int spins = 0;
  for (;;) {
    hipError_t q = hipEventQuery(ev);
    if (q == hipSuccess) {
      e->pending = false;
      return DS3_OK;
    }
    if (q != hipErrorNotReady) return poison(e, DS3_E_DEVICE_LOST, std::string("device wait: ") + hipGetErrorString(q));
    const double ms = std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
    if (ms >= (double)timeout_ms)
      return poison(e, DS3_E_TIMEOUT, "device wait exceeded " + std::to_string(timeout_ms) + " ms");
    if (++spins > 2000) std::this_thread::sleep_for(std::chrono::microseconds(50));
    else std::this_thread::yield();
  }
}

// One projection: the paired-row GEMV for up to 4 rows; beyond, the matrix-core GEMM on the activation fragments,
// which leaves partial products for the next kernel (the LM head writes the logits itself).
hipError_t run_projection(ds3_engine* e, const GemvParams& p, int mode, int kind) {
  const ds3_config& c = e->cfg;
  if (!e->cur.mfma) return launch_gemv(p, mode, c.weight_dtype, c.kv_dtype, e->blocks[kind], e->stream);
  const bool head = mode == GEMV_HEAD;
  SkGemmParams g{};
  g.w = reinterpret_cast<const uint16_t*>(p.w);
  g.hi = e->frag_hi;
  g.lo = e->frag_lo;
  g.K = p.K;
  g.plan = sk_plan(2 * p.n_pairs, p.K, head);
  g.part = e->skpart;
  g.out = p.out;
  g.rows = p.rows;
  g.nt = sk_tiles(p.rows);
  g.n_out = 2 * p.n_pairs;
  g.ss = e->skss;
  g.ss_blocks = (c.d_model + kNormSpan - 1) / kNormSpan;
  g.norm_dim = c.d_model;
  g.eps = c.rms_eps;
  g.status = e->status;
  return launch_sk_gemm(g, head, e->stream);
}

// the plans of the matrix-core projections whose partial products a consumer kernel sums
SkPlan plan_of(const ds3_config& c, int kind) {
  switch (kind) {
    case K_QKV: return sk_plan((c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim, c.d_model, false);
    case K_OPROJ: return sk_plan(c.d_model, c.n_q_heads * c.head_dim, false);
    case K_GATEUP: return sk_plan(2 * c.ffn_dim, c.d_model, false);
    default: return sk_plan(c.d_model, c.ffn_dim, false);   // K_DOWN
  }
}

hipError_t enqueue_kernel(ds3_engine* e, const Launch& l) {
  const ds3_config& c = e->cfg;
  const int R = e->cur.rows;
  KvView kv = e->kv;
  kv.row_map = e->cur.row_map;
  auto base = [&](GemvParams& p) {
    p.rows = R;
    p.eps = c.rms_eps;
    p.nq = c.n_q_heads;
    p.nkv = c.n_kv_heads;
    p.hd = c.head_dim;
    p.rope = e->rope;
    p.kv = kv;
    p.layer = l.layer;
    p.slots = e->cur.slots;
    p.status = e->status;
    p.ping_pong = true;
  };
  switch (l.kind) {
    case K_FUSED: {
      FusedParams p{};
      const char* wb = reinterpret_cast<const char*>(e->buf[DS3_BUF_WEIGHTS]);
      p.wbase = wb;
      p.lstride = e->weight_lstride;
      const auto& W0 = e->L[0];
      p.o_attn_norm = reinterpret_cast<const char*>(W0.attn_norm) - wb;
      p.o_wqkv = reinterpret_cast<const char*>(W0.wqkv) - wb;
      p.o_wo = reinterpret_cast<const char*>(W0.wo) - wb;
      p.o_ffn_norm = reinterpret_cast<const char*>(W0.ffn_norm) - wb;
      p.o_wgu = reinterpret_cast<const char*>(W0.wgu) - wb;
      p.o_wd = reinterpret_cast<const char*>(W0.wd) - wb;
      p.embed = reinterpret_cast<const uint16_t*>(e->embed);
      p.final_norm = e->final_norm;
      p.lm_head = reinterpret_cast<const uint16_t*>(e->lm_head);
      p.kv = e->kv;
      p.rope = e->rope;
      p.x = e->x;
      p.q = e->q;
      p.kvnew = e->kvnew;
      p.attn = e->attn;
      p.act = e->act;
      p.part = e->part;
      p.logits = e->logits;
      p.sync = e->sync;
      p.clocks = e->clocks;
      p.trace = e->trace;
      p.trace2 = c.trace >= DS3_TRACE_PHASES ? e->trace + (size_t)kFusedPhases * c.n_layers * kFusedBlocks * 2 : nullptr;
      p.slots = e->slots;
      p.status = e->status;
      p.ids = e->ids;
      p.chain_flags = e->chain_flags;
      p.max_chain = kMaxChain;
      p.n_layers = c.n_layers;
      p.vocab = c.vocab;
      p.cap = c.cap;
      p.split_len = c.cap / (kFusedBlocks / c.n_kv_heads);
      p.eps = c.rms_eps;
      p.scale = (float)(1.0 / std::sqrt((double)c.head_dim));
      // the traced variant only when a trace was asked for, or while profile_kernels reads the phase clocks
      const bool trace = c.trace != DS3_TRACE_OFF || e->profiling;
      return launch_fused(p, c.d_model, c.ffn_dim, c.head_dim, c.n_q_heads, c.n_kv_heads, trace, e->stream);
    }
    case K_SPLIT: {
      // x (+)= the o-proj (before the FFN norm) or down (before the next layer or the final norm) partials
      SkPrepParams pp{};
      pp.x = e->x;
      pp.part = (l.site == S_ATTN_NORM && l.layer == 0) ? nullptr : e->skpart;
      pp.plan = plan_of(c, l.site == S_FFN_NORM ? K_OPROJ : K_DOWN);
      pp.gain = l.site == S_ATTN_NORM ? e->L[l.layer].attn_norm
                                      : (l.site == S_FFN_NORM ? e->L[l.layer].ffn_norm : e->final_norm);
      pp.hi = e->frag_hi;
      pp.lo = e->frag_lo;
      pp.ss = e->skss;
      pp.D = c.d_model;
      pp.rows = R;
      pp.nt = sk_tiles(R);
      return launch_sk_prep(pp, e->stream);
    }
    case K_QKVFIN: {
      SkQkvParams qp{};
      qp.part = e->skpart;
      qp.plan = plan_of(c, K_QKV);
      qp.ss = e->skss;
      qp.ss_blocks = (c.d_model + kNormSpan - 1) / kNormSpan;
      qp.D = c.d_model;
      qp.eps = c.rms_eps;
      qp.q = e->q;
      qp.nq = c.n_q_heads;
      qp.nkv = c.n_kv_heads;
      qp.hd = c.head_dim;
      qp.rope = e->rope;
      qp.kv = kv;
      qp.layer = l.layer;
      qp.slots = e->cur.slots;
      qp.status = e->status;
      qp.rows = R;
      qp.nt = sk_tiles(R);
      return launch_sk_qkv(qp, c.kv_dtype, e->stream);
    }
    case K_SWIGLU: {
      SkActParams ap{};
      ap.part = e->skpart;
      ap.plan = plan_of(c, K_GATEUP);
      ap.ss = e->skss;
      ap.ss_blocks = (c.d_model + kNormSpan - 1) / kNormSpan;
      ap.D = c.d_model;
      ap.eps = c.rms_eps;
      ap.F = c.ffn_dim;
      ap.rows = R;
      ap.nt = sk_tiles(R);
      ap.hi = e->frag_hi;
      ap.lo = e->frag_lo;
      return launch_sk_swiglu(ap, e->stream);
    }
    case K_SAMPLE: {
      SampleParams p{};
      p.logits = e->logits;
      p.vocab = c.vocab;
      p.rows = R;
      p.slots = e->slots;
      p.page_table = c.kv_layout == DS3_KV_PAGED ? e->slot_map : nullptr;
      p.page_size = c.page_size;
      p.cap = c.cap;
      p.rowp = e->samp_rows;
      p.counts = e->counts;
      p.bias = e->bias;
      p.draws = e->draws;
      p.z = e->zbuf;
      p.part = e->samp_part;
      p.ids = e->ids;
      p.flags = e->chain_flags;
      p.lp = e->lp;
      p.lp_ids = e->lp_ids;
      p.max_chain = kMaxChain;
      p.status = e->status;
      p.done = e->pick_done;   // (the pick and the sampler never run in the same step; both leave it at zero)
      return launch_sample(p, e->stream);
    }
    case K_PICK: {
      PickParams p{};
      p.logits = e->logits;
      p.vocab = c.vocab;
      p.rows = R;
      p.slots = e->slots;
      p.page_table = c.kv_layout == DS3_KV_PAGED ? e->slot_map : nullptr;
      p.page_size = c.page_size;
      p.cap = c.cap;
      p.part_val = e->pick_val;
      p.part_idx = e->pick_idx;
      p.done = e->pick_done;
      p.ids = e->ids;
      p.flags = e->chain_flags;
      p.max_chain = kMaxChain;
      p.status = e->status;
      return launch_pick(p, e->stream);
    }
    case K_EMBED: {
      EmbedParams p{e->embed, e->x, c.d_model, c.vocab, R, e->cur.slots, e->status};
      return launch_embed(p, c.weight_dtype, e->stream);
    }
    case K_QKV: {
      GemvParams p{};
      base(p);
      const auto& W = e->L[l.layer];
      p.w = W.wqkv;
      p.in = e->x;
      p.gain = W.attn_norm;
      p.out = e->q;
      p.K = c.d_model;
      p.n_pairs = (c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim / 2;
      return run_projection(e, p, GEMV_QKV, K_QKV);
    }
    case K_ATTN:
    case K_COMBINE: {
      AttnParams p{};
      p.q = e->q;
      p.out = e->attn;
      p.part = e->part;
      p.kv = kv;
      p.layer = l.layer;
      p.nq = c.n_q_heads;
      p.nkv = c.n_kv_heads;
      p.hd = c.head_dim;
      p.splits = e->cur.splits;
      p.split_len = e->cur.split_len;
      p.scale = (float)(1.0 / std::sqrt((double)c.head_dim));
      p.slots = e->cur.slots;
      p.status = e->status;
      if (e->cur.mfma) {   // the combine also writes the o-projection's fragments
        p.frag_hi = e->frag_hi;
        p.frag_lo = e->frag_lo;
        p.nt = sk_tiles(R);
      }
      return l.kind == K_ATTN ? launch_attention(p, c.kv_dtype, R, e->stream)
                              : launch_attention_combine(p, R, e->stream);
    }
    case K_OPROJ: {
      GemvParams p{};
      base(p);
      p.w = e->L[l.layer].wo;
      p.in = e->attn;
      p.out = e->x;
      p.K = c.n_q_heads * c.head_dim;
      p.n_pairs = c.d_model / 2;
      return run_projection(e, p, GEMV_RESID, K_OPROJ);
    }
    case K_GATEUP: {
      GemvParams p{};
      base(p);
      const auto& W = e->L[l.layer];
      p.w = W.wgu;
      p.in = e->x;
      p.gain = W.ffn_norm;
      p.out = e->act;
      p.K = c.d_model;
      p.n_pairs = c.ffn_dim;
      p.up_offset = c.ffn_dim;
      return run_projection(e, p, GEMV_GATEUP, K_GATEUP);
    }
    case K_DOWN: {
      GemvParams p{};
      base(p);
      p.w = e->L[l.layer].wd;
      p.in = e->act;
      p.out = e->x;
      p.K = c.ffn_dim;
      p.n_pairs = c.d_model / 2;
      return run_projection(e, p, GEMV_RESID, K_DOWN);
    }
    case K_HEAD: {
      GemvParams p{};
      base(p);
      p.w = e->lm_head;
      p.in = e->x;
      p.gain = e->final_norm;
      p.out = e->cur.logits;
      p.K = c.d_model;
      p.n_pairs = c.vocab / 2;
      return run_projection(e, p, GEMV_HEAD, K_HEAD);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t enqueue_step(ds3_engine* e) {
  for (const Launch& l : e->sequence) {
    hipError_t h = enqueue_kernel(e, l);
    if (h != hipSuccess) return h;
  }
  return hipSuccess;
}

ds3_status ensure_captured(ds3_engine* e) {
  if (e->captured) return DS3_OK;
  HIP_OR_POISON(e, hipStreamBeginCapture(e->stream, hipStreamCaptureModeThreadLocal));
  hipError_t h = enqueue_step(e);
  hipGraph_t g = nullptr;
  hipError_t h2 = hipStreamEndCapture(e->stream, &g);
  if (h != hipSuccess || h2 != hipSuccess) {
    if (g) (void)hipGraphDestroy(g);
    return poison(e, DS3_E_DEVICE_LOST,
                  std::string("graph capture: ") + hipGetErrorString(h != hipSuccess ? h : h2));
  }
  e->graph = g;
  HIP_OR_POISON(e, hipGraphInstantiate(&e->exec, e->graph, nullptr, nullptr, 0));
  size_t n = 0;
  HIP_OR_POISON(e, hipGraphGetNodes(e->graph, nullptr, &n));
  e->graph_nodes = (int)n;
  e->captured = true;
  e->stats.captures++;
  return DS3_OK;
}

ds3_status refuse_if_unusable(ds3_engine* e) {
  if (!e) return fail(nullptr, DS3_E_INVALID, "engine is NULL");
  if (e->state == ST_POISONED) return fail(e, DS3_E_POISONED, "engine is poisoned: " + e->err);
  return DS3_OK;
}

}  // namespace

extern "C" {

ds3_status ds3_query_buffers(const ds3_config* cfg, ds3_buffer_req* out, int32_t* n_inout) {
  std::string why = check_config(cfg);
  if (!why.empty()) return fail(nullptr, cfg ? DS3_E_UNSUPPORTED : DS3_E_INVALID, why);
  if (!out || !n_inout || *n_inout < DS3_NUM_BUFFERS) return fail(nullptr, DS3_E_INVALID, "need room for 4 buffers");
  int splits, split_len;
  plan_splits(*cfg, cfg->rows, &splits, &split_len);
  const size_t sizes[DS3_NUM_BUFFERS] = {plan_weights(*cfg).total, kv_state_bytes(*cfg),
                                         plan_work(*cfg, splits).total,
                                         (size_t)cfg->rows * cfg->vocab * sizeof(float)};
  const char* names[DS3_NUM_BUFFERS] = {"weights", "kv", "work", "logits"};
  for (int i = 0; i < DS3_NUM_BUFFERS; ++i) {
    out[i].id = i;
    std::snprintf(out[i].name, sizeof(out[i].name), "%s", names[i]);
    out[i].bytes = sizes[i];
    out[i].align = kAlign;
  }
  *n_inout = DS3_NUM_BUFFERS;
  return DS3_OK;
}

ds3_status ds3_create(const ds3_config* cfg, void* const* dev_ptrs, int32_t n, void* hip_stream, ds3_engine** out) {
  std::string why = check_config(cfg);
  if (!why.empty()) return fail(nullptr, cfg ? DS3_E_UNSUPPORTED : DS3_E_INVALID, why);
  if (!dev_ptrs || n != DS3_NUM_BUFFERS || !out) return fail(nullptr, DS3_E_INVALID, "need 4 device buffers and out");
  for (int i = 0; i < DS3_NUM_BUFFERS; ++i)
    if (!dev_ptrs[i] || (reinterpret_cast<uintptr_t>(dev_ptrs[i]) % kAlign))
      return fail(nullptr, DS3_E_INVALID, "device buffer " + std::to_string(i) + " is NULL or not 256-byte aligned");
  *out = nullptr;
  ds3_engine* e = new ds3_engine();
  e->cfg = *cfg;
  if (e->cfg.timeout_ms == 0) e->cfg.timeout_ms = kDefaultTimeoutMs;
  const ds3_config& c = e->cfg;
  for (int i = 0; i < DS3_NUM_BUFFERS; ++i) e->buf[i] = dev_ptrs[i];
  auto bail = [&](ds3_status st, const std::string& msg) {
    g_last_error = msg;
    ds3_destroy(e);
    return st;
  };
  hipError_t h = hipGetDevice(&e->device);
  if (h != hipSuccess) return bail(DS3_E_DEVICE_LOST, std::string("hipGetDevice: ") + hipGetErrorString(h));
  if (hip_stream) {
    e->stream = reinterpret_cast<hipStream_t>(hip_stream);
  } else {
    h = hipStreamCreateWithFlags(&e->stream, hipStreamNonBlocking);
    if (h != hipSuccess) return bail(DS3_E_DEVICE_LOST, std::string("hipStreamCreate: ") + hipGetErrorString(h));
    e->own_stream = true;
  }
  // the allocation-free staging array of this device, looked up once per device while it is current
  h = scratch_device_ptr(e->device, &e->scratch);
  if (h != hipSuccess) return bail(DS3_E_DEVICE_LOST, std::string("scratch array: ") + hipGetErrorString(h));
  plan_splits(c, c.rows, &e->splits, &e->split_len);
  const WorkPlan wp = plan_work(c, e->splits);
  char* work = reinterpret_cast<char*>(e->buf[DS3_BUF_WORK]);
  e->slots = reinterpret_cast<int*>(work + wp.slots);
  e->status = reinterpret_cast<StatusWords*>(work + wp.status);
  e->x = reinterpret_cast<float*>(work + wp.x);
  e->q = reinterpret_cast<float*>(work + wp.q);
  e->attn = reinterpret_cast<float*>(work + wp.attn);
  e->act = reinterpret_cast<float*>(work + wp.act);
  e->part = reinterpret_cast<float*>(work + wp.part);
  e->rope = reinterpret_cast<float*>(work + wp.rope);
  e->slot_map = reinterpret_cast<int*>(work + wp.slot_map);
  e->kvnew = reinterpret_cast<float*>(work + wp.kvnew);
  e->sync = reinterpret_cast<unsigned*>(work + wp.sync);
  e->clocks = reinterpret_cast<unsigned long long*>(work + wp.clocks);
  e->trace = reinterpret_cast<unsigned long long*>(work + wp.trace);
  e->pick_val = reinterpret_cast<float*>(work + wp.pick_val);
  e->pick_idx = reinterpret_cast<int*>(work + wp.pick_idx);
  e->pick_done = reinterpret_cast<unsigned*>(work + wp.pick_done);
  e->ids = reinterpret_cast<int32_t*>(work + wp.ids);
  e->chain_flags = reinterpret_cast<uint32_t*>(work + wp.chain_flags);
  e->samp_rows = reinterpret_cast<SampleRow*>(work + wp.samp_rows);
  e->counts = reinterpret_cast<int32_t*>(work + wp.counts);
  e->bias = reinterpret_cast<float*>(work + wp.bias);
  e->draws = reinterpret_cast<uint32_t*>(work + wp.draws);
  e->zbuf = reinterpret_cast<float*>(work + wp.zbuf);
  e->samp_part = reinterpret_cast<SampPart*>(work + wp.samp_part);
  e->lp = reinterpret_cast<float*>(work + wp.lp);
  e->lp_ids = reinterpret_cast<int32_t*>(work + wp.lp_ids);
  e->sync_words = fused_sync_words(c.n_layers, c.n_kv_heads);
  e->frag_hi = reinterpret_cast<uint16_t*>(work + wp.frag_hi);
  e->frag_lo = reinterpret_cast<uint16_t*>(work + wp.frag_lo);
  e->skpart = reinterpret_cast<float*>(work + wp.skpart);
  e->skss = reinterpret_cast<float*>(work + wp.skss);
  e->mfma = rows_on_mfma(c, c.rows);
  e->work_bytes = wp.total;
  e->logits = reinterpret_cast<float*>(e->buf[DS3_BUF_LOGITS]);

  const WeightPlan wpl = plan_weights(c);
  char* wbase = reinterpret_cast<char*>(e->buf[DS3_BUF_WEIGHTS]);
  for (int l = 0; l < c.n_layers; ++l) {
    const auto& P = wpl.layers[l];
    e->L.push_back({reinterpret_cast<float*>(wbase + P.attn_norm), wbase + P.wqkv, wbase + P.wo,
                    reinterpret_cast<float*>(wbase + P.ffn_norm), wbase + P.wgu, wbase + P.wd});
  }
  e->weight_lstride = c.n_layers > 1 ? wpl.layers[1].attn_norm - wpl.layers[0].attn_norm : 0;
  e->embed = wbase + wpl.embed;
  e->final_norm = reinterpret_cast<float*>(wbase + wpl.final_norm);
  e->lm_head = wbase + wpl.lm_head;

  e->kv_bytes = kv_state_bytes(c);
  const size_t kvb = dtype_bytes(c.kv_dtype);
  e->kv.k = e->buf[DS3_BUF_KV];
  e->kv.v = reinterpret_cast<char*>(e->buf[DS3_BUF_KV]) + e->kv_bytes / 2;
  e->kv.layer_stride = (int64_t)(e->kv_bytes / 2 / kvb / c.n_layers);
  e->kv.paged = c.kv_layout == DS3_KV_PAGED;
  e->kv.v_t = c.kv_dtype == DS3_BF16;   // the matrix-core attention reads V position-contiguous
  e->kv.cap = c.cap;
  e->kv.page_size = e->kv.paged ? c.page_size : 1;
  e->kv.pool_pages = e->kv.paged ? c.pool_pages : 0;
  e->kv.slot_map = e->slot_map;

  // launch shapes
  int cus = 0;
  h = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, e->device);
  if (h != hipSuccess) return bail(DS3_E_DEVICE_LOST, std::string("hipDeviceGetAttribute: ") + hipGetErrorString(h));
  e->blocks[K_QKV] = gemv_blocks((c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim / 2, cus);
  e->blocks[K_OPROJ] = gemv_blocks(c.d_model / 2, cus);
  e->blocks[K_GATEUP] = gemv_blocks(c.ffn_dim, cus);
  e->blocks[K_DOWN] = gemv_blocks(c.d_model / 2, cus);
  e->blocks[K_HEAD] = gemv_blocks(c.vocab / 2, cus);

  // kernel plan: the fused step kernel needs its shape, one block per CU of a 256-CU device, and co-residency.
  // AUTO takes it wherever it applies (it is the faster plan at one row: no kernel boundaries, and the next
  // phase's weights stream while the grid synchronizes), else the per-operation kernels.
  if ((c.kernel_plan == DS3_PLAN_FUSED || c.kernel_plan == DS3_PLAN_AUTO) && fused_refusal(c).empty()) {
    int per_cu = 0;
    h = fused_blocks_per_cu(c.d_model, c.ffn_dim, c.head_dim, c.n_q_heads, c.n_kv_heads,
                            c.cap / (kFusedBlocks / c.n_kv_heads), &per_cu);
    if (h != hipSuccess) return bail(DS3_E_DEVICE_LOST, std::string("fused occupancy: ") + hipGetErrorString(h));
    e->fused = cus == kFusedBlocks && per_cu >= 1;
    if (!e->fused && c.kernel_plan == DS3_PLAN_FUSED)
      return bail(DS3_E_UNSUPPORTED, "kernel_plan: the fused step kernel needs " + std::to_string(kFusedBlocks) +
                                         " compute units with one block each (device has " + std::to_string(cus) +
                                         ", " + std::to_string(per_cu) + " block(s) per unit)");
  }
  // the per-operation sequence of R rows (above 4 rows: the matrix-core GEMMs and the kernels that consume their
  // partial products)
  // (a plan of one attention split needs no combine: the attention writes the merged output itself)
  auto per_op = [&](std::vector<Launch>& seq, bool mfma, bool combine, bool pick) {
    seq.push_back({K_EMBED, -1, 0});
    for (int l = 0; l < c.n_layers; ++l) {
      if (mfma) seq.push_back({K_SPLIT, l, S_ATTN_NORM});
      seq.push_back({K_QKV, l, 0});
      if (mfma) seq.push_back({K_QKVFIN, l, 0});
      seq.push_back({K_ATTN, l, 0});
      if (combine) seq.push_back({K_COMBINE, l, 0});
      seq.push_back({K_OPROJ, l, 0});
      if (mfma) seq.push_back({K_SPLIT, l, S_FFN_NORM});
      seq.push_back({K_GATEUP, l, 0});
      if (mfma) seq.push_back({K_SWIGLU, l, 0});
      seq.push_back({K_DOWN, l, 0});
    }
    if (mfma) seq.push_back({K_SPLIT, -1, S_FINAL_NORM});
    seq.push_back({K_HEAD, -1, 0});
    if (pick) seq.push_back({K_PICK, -1, 0});
  };
  if (e->fused) e->sequence.push_back({K_FUSED, -1, 0});   // (the fused kernel picks in its own last phase)
  else per_op(e->sequence, e->mfma, e->splits > 1, true);
  e->samp_sequence = e->sequence;   // the same step, the sampler as its pick
  if (e->fused) e->samp_sequence.push_back({K_SAMPLE, -1, 0});
  else e->samp_sequence.back() = {K_SAMPLE, -1, 0};
  e->h_samp.assign((size_t)c.rows, SampleRow{0.f, 1.f, 0.f, 1.f, 0.f, 0.f, 0, 0, 0u, 0u});
  h = hipHostMalloc(reinterpret_cast<void**>(&e->h_samp_pinned), (size_t)c.rows * sizeof(SampleRow), hipHostMallocDefault);
  if (h == hipSuccess)
    h = hipHostMalloc(reinterpret_cast<void**>(&e->h_lp), (size_t)kMaxChain * c.rows * (1 + 2 * kMaxLogprobs) * 4,
                      hipHostMallocDefault);
  if (h != hipSuccess) return bail(DS3_E_DEVICE_LOST, std::string("hipHostMalloc: ") + hipGetErrorString(h));
  e->dec.rows = c.rows;
  e->dec.splits = e->splits;
  e->dec.split_len = e->split_len;
  e->dec.slots = e->slots;
  e->dec.logits = e->logits;
  e->dec.mfma = e->mfma;
  e->cur = e->dec;
  if (c.prefill_rows > 0) {
    const int T = c.prefill_rows;
    e->pre.rows = T;
    plan_splits(c, T, &e->pre.splits, &e->pre.split_len);   // (the partials buffer holds either plan)
    e->pre.slots = reinterpret_cast<int*>(work + wp.pre_slots);
    e->pre.logits = reinterpret_cast<float*>(work + wp.pre_logits);
    e->pre.mfma = rows_on_mfma(c, T);
    e->pre.row_map = e->pre.slots + SlotLayout{T}.words();
    per_op(e->pre_sequence, e->pre.mfma, e->pre.splits > 1, false);
    e->pre_body = e->pre_sequence.size() - (e->pre.mfma ? 2 : 1);   // (the final norm prep, then the head)
    h = hipHostMalloc(reinterpret_cast<void**>(&e->h_pre),
                      (size_t)(kMaxPrefill / T + 1) * (SlotLayout{T}.words() + T) * 4, hipHostMallocDefault);
    if (h != hipSuccess) return bail(DS3_E_DEVICE_LOST, std::string("hipHostMalloc: ") + hipGetErrorString(h));
  }

  const SlotLayout sl{c.rows};
  h = hipHostMalloc(reinterpret_cast<void**>(&e->h_slots), (size_t)sl.words() * 4 + kAlign + sizeof(StatusWords),
                    hipHostMallocDefault);
  if (h != hipSuccess) return bail(DS3_E_DEVICE_LOST, std::string("hipHostMalloc: ") + hipGetErrorString(h));
  std::memset(e->h_slots, 0, (size_t)sl.words() * 4);
  e->h_status = reinterpret_cast<StatusWords*>(reinterpret_cast<char*>(e->h_slots) + align_up((size_t)sl.words() * 4, 16));
  h = hipHostMalloc(reinterpret_cast<void**>(&e->h_chain), (size_t)kMaxChain * (c.rows + 1) * 4, hipHostMallocDefault);
  if (h != hipSuccess) return bail(DS3_E_DEVICE_LOST, std::string("hipHostMalloc: ") + hipGetErrorString(h));
  for (hipEvent_t* ev : {&e->ev0, &e->ev1, &e->ev_done}) {
    h = hipEventCreate(ev);
    if (h != hipSuccess) return bail(DS3_E_DEVICE_LOST, std::string("hipEventCreate: ") + hipGetErrorString(h));
  }

  // rotary table: angle p * theta^(-2i/hd) in double, stored as float32 (cos, sin)
  {
    const int half = c.head_dim / 2;
    std::vector<float> tab((size_t)c.cap * half * 2);
    for (int p = 0; p < c.cap; ++p)
      for (int i = 0; i < half; ++i) {
        const double ang = (double)p * std::pow(c.rope_theta, -2.0 * i / c.head_dim);
        tab[((size_t)p * half + i) * 2] = (float)std::cos(ang);
        tab[((size_t)p * half + i) * 2 + 1] = (float)std::sin(ang);
      }
    h = hipMemcpyAsync(e->rope, tab.data(), tab.size() * 4, hipMemcpyHostToDevice, e->stream);
    if (h == hipSuccess) h = hipMemsetAsync(e->slots, 0, wp.rope, e->stream);  // slots .. partials
    if (h == hipSuccess) h = hipMemsetAsync(e->buf[DS3_BUF_KV], 0, e->kv_bytes, e->stream);
    if (h == hipSuccess) h = hipStreamSynchronize(e->stream);
    if (h != hipSuccess) return bail(DS3_E_DEVICE_LOST, std::string("create upload: ") + hipGetErrorString(h));
  }
  e->state = ST_NOT_LOADED;
  e->stats.attn_splits = e->fused ? kFusedBlocks / c.n_kv_heads : e->splits;
  e->stats.kernel_plan = e->fused ? DS3_PLAN_FUSED : DS3_PLAN_PER_OP;
  e->stats.state = e->state;
  *out = e;
  return DS3_OK;
}

ds3_status ds3_load_weights(ds3_engine* e, const ds3_weight_src* w, int32_t n) {
  if (ds3_status st = refuse_if_unusable(e)) return st;
  if (!w || n < 0) return fail(e, DS3_E_INVALID, "weights array is NULL");
  const ds3_config& c = e->cfg;
  const int64_t d = c.d_model, F = c.ffn_dim, qw = (int64_t)c.n_q_heads * c.head_dim,
                kvw = (int64_t)c.n_kv_heads * c.head_dim, V = c.vocab;
  auto expect = [&](int role, int64_t* rows, int64_t* cols) {
    switch (role) {
      case DS3_W_EMBED: case DS3_W_LM_HEAD: *rows = V; *cols = d; return;
      case DS3_W_ATTN_NORM: case DS3_W_FFN_NORM: case DS3_W_FINAL_NORM: *rows = 1; *cols = d; return;
      case DS3_W_Q: *rows = qw; *cols = d; return;
      case DS3_W_K: case DS3_W_V: *rows = kvw; *cols = d; return;
      case DS3_W_O: *rows = d; *cols = qw; return;
      case DS3_W_GATE: case DS3_W_UP: *rows = F; *cols = d; return;
      case DS3_W_DOWN: *rows = d; *cols = F; return;
    }
  };
  static const char* role_names[DS3_W_NUM_ROLES] = {"EMBED", "ATTN_NORM", "Q", "K", "V", "O", "FFN_NORM",
                                                    "GATE", "UP", "DOWN", "FINAL_NORM", "LM_HEAD"};
  auto is_global = [](int role) { return role == DS3_W_EMBED || role == DS3_W_FINAL_NORM || role == DS3_W_LM_HEAD; };
  // validate everything before touching the device
  std::vector<const ds3_weight_src*> slot((size_t)DS3_W_NUM_ROLES * (c.n_layers + 1), nullptr);
  for (int i = 0; i < n; ++i) {
    const ds3_weight_src& s = w[i];
    if (s.role < 0 || s.role >= DS3_W_NUM_ROLES) return fail(e, DS3_E_INVALID, "unknown role " + std::to_string(s.role));
    const bool glob = is_global(s.role);
    if (glob ? s.layer != -1 : (s.layer < 0 || s.layer >= c.n_layers))
      return fail(e, DS3_E_INVALID, std::string("bad layer for role ") + role_names[s.role]);
    int64_t er, ec;
    expect(s.role, &er, &ec);
    const bool is_norm = s.role == DS3_W_ATTN_NORM || s.role == DS3_W_FFN_NORM || s.role == DS3_W_FINAL_NORM;
    if (!(s.rows == er && s.cols == ec) && !(is_norm && s.rows * s.cols == ec))
      return fail(e, DS3_E_INVALID, std::string("wrong shape for ") + role_names[s.role]);
    if (s.dtype != c.weight_dtype) return fail(e, DS3_E_INVALID, std::string("wrong dtype for ") + role_names[s.role]);
    if (!s.data) return fail(e, DS3_E_INVALID, std::string("NULL data for ") + role_names[s.role]);
    const size_t k = (size_t)s.role * (c.n_layers + 1) + (glob ? c.n_layers : s.layer);
    if (slot[k]) return fail(e, DS3_E_INVALID, std::string("duplicate ") + role_names[s.role]);
    slot[k] = &s;
  }
  for (int role = 0; role < DS3_W_NUM_ROLES; ++role) {
    if (is_global(role)) {
      if (!slot[(size_t)role * (c.n_layers + 1) + c.n_layers])
        return fail(e, DS3_E_UNBOUND, std::string("unbound weight ") + role_names[role]);
    } else {
      for (int l = 0; l < c.n_layers; ++l)
        if (!slot[(size_t)role * (c.n_layers + 1) + l])
          return fail(e, DS3_E_UNBOUND, std::string("unbound weight ") + role_names[role] + " of layer " + std::to_string(l));
    }
  }
  const size_t wb = dtype_bytes(c.weight_dtype);
  auto src = [&](int role, int layer) { return slot[(size_t)role * (c.n_layers + 1) + (layer < 0 ? c.n_layers : layer)]; };
  auto copy = [&](void* dst, const ds3_weight_src* s, size_t bytes) -> hipError_t {
    return hipMemcpyAsync(dst, s->data, bytes, hipMemcpyDefault, e->stream);
  };
  // norm gains are kept as float32 on the device (exact widening of bf16 words)
  std::vector<std::vector<float>> gains;
  auto gain = [&](float* dst, const ds3_weight_src* s) -> hipError_t {
    std::vector<float> g((size_t)d);
    hipPointerAttribute_t attr{};
    const bool on_device = hipPointerGetAttributes(&attr, s->data) == hipSuccess && attr.type == hipMemoryTypeDevice;
    (void)!hipGetLastError();
    std::vector<uint8_t> host((size_t)d * wb);
    if (on_device) {
      hipError_t h = hipMemcpy(host.data(), s->data, host.size(), hipMemcpyDeviceToHost);
      if (h != hipSuccess) return h;
    } else {
      std::memcpy(host.data(), s->data, host.size());
    }
    for (int64_t i = 0; i < d; ++i) {
      if (c.weight_dtype == DS3_BF16) {
        uint16_t word;
        std::memcpy(&word, host.data() + i * 2, 2);
        uint32_t u = (uint32_t)word << 16;
        std::memcpy(&g[i], &u, 4);
      } else {
        std::memcpy(&g[i], host.data() + i * 4, 4);
      }
    }
    gains.push_back(std::move(g));
    return hipMemcpyAsync(dst, gains.back().data(), (size_t)d * 4, hipMemcpyHostToDevice, e->stream);
  };
  gains.reserve((size_t)2 * c.n_layers + 1);
  for (int l = 0; l < c.n_layers; ++l) {
    const auto& W = e->L[l];
    char* qkv = reinterpret_cast<char*>(W.wqkv);
    char* gu = reinterpret_cast<char*>(W.wgu);
    HIP_OR_POISON(e, gain(W.attn_norm, src(DS3_W_ATTN_NORM, l)));
    HIP_OR_POISON(e, copy(qkv, src(DS3_W_Q, l), (size_t)qw * d * wb));
    HIP_OR_POISON(e, copy(qkv + (size_t)qw * d * wb, src(DS3_W_K, l), (size_t)kvw * d * wb));
    HIP_OR_POISON(e, copy(qkv + (size_t)(qw + kvw) * d * wb, src(DS3_W_V, l), (size_t)kvw * d * wb));
    HIP_OR_POISON(e, copy(W.wo, src(DS3_W_O, l), (size_t)d * qw * wb));
    HIP_OR_POISON(e, gain(W.ffn_norm, src(DS3_W_FFN_NORM, l)));
    HIP_OR_POISON(e, copy(gu, src(DS3_W_GATE, l), (size_t)F * d * wb));
    HIP_OR_POISON(e, copy(gu + (size_t)F * d * wb, src(DS3_W_UP, l), (size_t)F * d * wb));
    HIP_OR_POISON(e, copy(W.wd, src(DS3_W_DOWN, l), (size_t)d * F * wb));
  }
  HIP_OR_POISON(e, copy(e->embed, src(DS3_W_EMBED, -1), (size_t)V * d * wb));
  HIP_OR_POISON(e, gain(e->final_norm, src(DS3_W_FINAL_NORM, -1)));
  HIP_OR_POISON(e, copy(e->lm_head, src(DS3_W_LM_HEAD, -1), (size_t)V * d * wb));
  HIP_OR_POISON(e, hipEventRecord(e->ev_done, e->stream));
  e->pending = true;
  if (ds3_status st = wait_done(e, e->ev_done, e->cfg.timeout_ms)) return st;
  if (e->state == ST_NOT_LOADED) e->state = ST_READY;
  e->stats.state = e->state;
  return DS3_OK;
}

ds3_status ds3_set_slot_map(ds3_engine* e, const int32_t* slot_map) {
  if (ds3_status st = refuse_if_unusable(e)) return st;
  const ds3_config& c = e->cfg;
  if (c.kv_layout != DS3_KV_PAGED) return fail(e, DS3_E_INVALID, "slot map needs the paged KV layout");
  if (!slot_map) return fail(e, DS3_E_INVALID, "slot map is NULL");
  const size_t n = (size_t)c.rows * (c.cap / c.page_size);
  std::vector<uint8_t> seen((size_t)c.pool_pages, 0);
  for (size_t i = 0; i < n; ++i) {
    const int32_t pg = slot_map[i];
    if (pg < 0 || pg >= c.pool_pages) return fail(e, DS3_E_INVALID, "page id out of range at " + std::to_string(i));
    if (seen[pg]) return fail(e, DS3_E_INVALID, "page " + std::to_string(pg) + " appears twice");
    seen[pg] = 1;
  }
  e->h_slot_map.assign(slot_map, slot_map + n);
  HIP_OR_POISON(e, hipMemcpyAsync(e->slot_map, e->h_slot_map.data(), n * 4, hipMemcpyHostToDevice, e->stream));
  HIP_OR_POISON(e, hipEventRecord(e->ev_done, e->stream));
  e->pending = true;
  if (ds3_status st = wait_done(e, e->ev_done, e->cfg.timeout_ms)) return st;
  e->slot_map_set = true;
  return DS3_OK;
}

// n_steps steps from the given slots: the first from the host's words, each later one from the slots the
// previous step's greedy pick advanced on the device (token = the pick, pos + 1). One host wait for all of them.
// Capture `seq` into a graph of its own (the sampling variant of the step).
static ds3_status capture_seq(ds3_engine* e, const std::vector<Launch>& seq, hipGraph_t* graph, hipGraphExec_t* exec,
                              bool* captured) {
  if (*captured) return DS3_OK;
  HIP_OR_POISON(e, hipStreamBeginCapture(e->stream, hipStreamCaptureModeThreadLocal));
  hipError_t h = hipSuccess;
  for (const Launch& l : seq)
    if (h == hipSuccess) h = enqueue_kernel(e, l);
  hipGraph_t g = nullptr;
  const hipError_t h2 = hipStreamEndCapture(e->stream, &g);
  if (h != hipSuccess || h2 != hipSuccess) {
    if (g) (void)hipGraphDestroy(g);
    return poison(e, DS3_E_DEVICE_LOST, std::string("graph capture: ") + hipGetErrorString(h != hipSuccess ? h : h2));
  }
  *graph = g;
  HIP_OR_POISON(e, hipGraphInstantiate(exec, g, nullptr, nullptr, 0));
  *captured = true;
  e->stats.captures++;
  return DS3_OK;
}

static ds3_status run_steps(ds3_engine* e, const int32_t* tokens, const int32_t* pos, const int32_t* write_map,
                            int32_t n_steps, float* logits_host, int32_t* ids_out, uint32_t* flags_out,
                            bool sample = false, float* lp_out = nullptr, int32_t* lp_ids_out = nullptr) {
  const auto t_start = std::chrono::steady_clock::now();
  if (ds3_status st = refuse_if_unusable(e)) return st;
  if (e->state == ST_NOT_LOADED) return fail(e, DS3_E_NOT_LOADED, "weights are not loaded");
  if (e->state == ST_NEEDS_RESET) return fail(e, DS3_E_NEEDS_RESET, "a previous step failed; reset_state first");
  const ds3_config& c = e->cfg;
  if (!tokens || !pos) return fail(e, DS3_E_INVALID, "tokens or pos is NULL");
  if (n_steps < 1 || n_steps > kMaxChain)
    return fail(e, DS3_E_INVALID, "n_steps must be in 1.." + std::to_string(kMaxChain));
  const SlotLayout sl{c.rows};
  const bool paged = c.kv_layout == DS3_KV_PAGED;
  // attention reads every position through the page table, so no paged step runs before one was set
  if (paged && !e->slot_map_set) return fail(e, DS3_E_INVALID, "paged step needs a slot map (ds3_set_slot_map)");
  for (int r = 0; r < c.rows; ++r) {
    if (tokens[r] < 0 || tokens[r] >= c.vocab) return fail(e, DS3_E_INVALID, "token out of range in row " + std::to_string(r));
    if (pos[r] < 0 || pos[r] >= c.cap) return fail(e, DS3_E_INVALID, "pos out of range in row " + std::to_string(r));
    if ((int64_t)pos[r] + n_steps > c.cap)
      return fail(e, DS3_E_INVALID, "pos + n_steps passes the capacity in row " + std::to_string(r));
    if (paged && write_map) {
      // the K/V write must land where the sweep reads position pos[r]: its page-table slot
      const int ppr = c.cap / c.page_size;
      const int64_t want =
          (int64_t)e->h_slot_map[(size_t)r * ppr + pos[r] / c.page_size] * c.page_size + pos[r] % c.page_size;
      if (write_map[r] != want)
        return fail(e, DS3_E_INVALID, "write_map of row " + std::to_string(r) + " is not the page-table slot of pos");
    }
  }
  // slot words, then the status words (cleared every call by the same copy)
  for (int r = 0; r < c.rows; ++r) {
    e->h_slots[sl.token() + r] = tokens[r];
    e->h_slots[sl.pos() + r] = pos[r];
    int32_t wm = 0;
    if (paged) {
      const int ppr = c.cap / c.page_size;
      wm = write_map ? write_map[r]
                     : e->h_slot_map[(size_t)r * ppr + pos[r] / c.page_size] * c.page_size + pos[r] % c.page_size;
    }
    e->h_slots[sl.write_map() + r] = wm;
  }
  e->h_slots[sl.inject()] = e->inject_check ? 1 : 0;
  e->h_slots[sl.spin()] = e->inject_barrier ? 1 : 0;   // fused kernel: 1 tick forces every barrier wait to time out
  e->h_slots[sl.chain()] = 0;
  e->h_slots[sl.sweep()] = e->kv_sweep;
  e->h_slots[sl.sample()] = sample ? 1 : 0;
  e->inject_check = false;
  e->inject_barrier = false;
  const uint32_t timeout = e->inject_timeout ? 0u : e->cfg.timeout_ms;
  e->inject_timeout = false;

  HIP_OR_POISON(e, hipMemcpyAsync(e->slots, e->h_slots, (size_t)sl.words() * 4, hipMemcpyHostToDevice, e->stream));
  e->h_status->err = 0;
  e->h_status->nonfinite = 0;
  HIP_OR_POISON(e, hipMemcpyAsync(e->status, e->h_status, sizeof(StatusWords), hipMemcpyHostToDevice, e->stream));
  if (sample) {
    std::memcpy(e->h_samp_pinned, e->h_samp.data(), (size_t)c.rows * sizeof(SampleRow));
    HIP_OR_POISON(e, hipMemcpyAsync(e->samp_rows, e->h_samp_pinned, (size_t)c.rows * sizeof(SampleRow),
                                    hipMemcpyHostToDevice, e->stream));
  }
  if (c.exec_mode == DS3_GRAPH) {
    if (sample) {
      if (ds3_status st = capture_seq(e, e->samp_sequence, &e->samp_graph, &e->samp_exec, &e->samp_captured)) return st;
    } else if (ds3_status st = ensure_captured(e)) {
      return st;
    }
    hipGraphExec_t x = sample ? e->samp_exec : e->exec;
    HIP_OR_POISON(e, hipEventRecord(e->ev0, e->stream));
    for (int i = 0; i < n_steps; ++i) HIP_OR_POISON(e, hipGraphLaunch(x, e->stream));
    HIP_OR_POISON(e, hipEventRecord(e->ev1, e->stream));
    e->stats.replays += n_steps;
  } else {
    HIP_OR_POISON(e, hipEventRecord(e->ev0, e->stream));
    for (int i = 0; i < n_steps; ++i)
      for (const Launch& l : sample ? e->samp_sequence : e->sequence) HIP_OR_POISON(e, enqueue_kernel(e, l));
    HIP_OR_POISON(e, hipEventRecord(e->ev1, e->stream));
  }
  HIP_OR_POISON(e, hipMemcpyAsync(e->h_status, e->status, sizeof(StatusWords), hipMemcpyDeviceToHost, e->stream));
  int32_t* h_ids = e->h_chain;
  uint32_t* h_flags = reinterpret_cast<uint32_t*>(e->h_chain + (size_t)kMaxChain * c.rows);
  if (ids_out)
    HIP_OR_POISON(e, hipMemcpyAsync(h_ids, e->ids, (size_t)n_steps * c.rows * 4, hipMemcpyDeviceToHost, e->stream));
  HIP_OR_POISON(e, hipMemcpyAsync(h_flags, e->chain_flags, (size_t)n_steps * 4, hipMemcpyDeviceToHost, e->stream));
  const size_t nlp = (size_t)n_steps * c.rows * (1 + kMaxLogprobs), nlpi = (size_t)n_steps * c.rows * kMaxLogprobs;
  if (sample && lp_out)
    HIP_OR_POISON(e, hipMemcpyAsync(e->h_lp, e->lp, nlp * 4, hipMemcpyDeviceToHost, e->stream));
  if (sample && lp_ids_out)
    HIP_OR_POISON(e, hipMemcpyAsync(e->h_lp + nlp, e->lp_ids, nlpi * 4, hipMemcpyDeviceToHost, e->stream));
  if (logits_host)
    HIP_OR_POISON(e, hipMemcpyAsync(logits_host, e->logits, (size_t)c.rows * c.vocab * 4, hipMemcpyDeviceToHost,
                                    e->stream));
  HIP_OR_POISON(e, hipEventRecord(e->ev_done, e->stream));
  e->pending = true;
  e->stats.last_submit_us =
      std::chrono::duration<double, std::micro>(std::chrono::steady_clock::now() - t_start).count();
  if (ds3_status st = wait_done(e, e->ev_done, timeout)) return st;
  float gpu_ms = 0.f;
  HIP_OR_POISON(e, hipEventElapsedTime(&gpu_ms, e->ev0, e->ev1));
  e->stats.last_gpu_us = gpu_ms * 1e3 / n_steps;
  e->stats.kernels_per_step = c.exec_mode == DS3_GRAPH ? e->graph_nodes : (int)e->sequence.size();
  const uint32_t errbits = e->h_status->err;
  if (ids_out) std::memcpy(ids_out, h_ids, (size_t)n_steps * c.rows * 4);
  if (flags_out) std::memcpy(flags_out, h_flags, (size_t)n_steps * 4);
  if (sample && lp_out) std::memcpy(lp_out, e->h_lp, nlp * 4);
  if (sample && lp_ids_out) std::memcpy(lp_ids_out, e->h_lp + nlp, nlpi * 4);
  e->stats.last_host_us =
      std::chrono::duration<double, std::micro>(std::chrono::steady_clock::now() - t_start).count();
  if (errbits) {
    e->state = ST_NEEDS_RESET;
    e->stats.state = e->state;
    return fail(e, DS3_E_KERNEL_CHECK, "in-kernel check failed, error bits 0x" + [&] {
      char b[16];
      std::snprintf(b, sizeof b, "%x", errbits);
      return std::string(b);
    }());
  }
  e->stats.steps += n_steps;
  return DS3_OK;
}

ds3_status ds3_step(ds3_engine* e, const int32_t* tokens, const int32_t* pos, const int32_t* write_map,
                    float* logits_host, uint32_t* flags) {
  return run_steps(e, tokens, pos, write_map, 1, logits_host, nullptr, flags);
}

ds3_status ds3_step_greedy(ds3_engine* e, const int32_t* tokens, const int32_t* pos, int32_t n_steps,
                           int32_t* ids, uint32_t* flags) {
  if (!ids) return fail(e, DS3_E_INVALID, "ids is NULL");
  return run_steps(e, tokens, pos, nullptr, n_steps, nullptr, ids, flags);
}

ds3_status ds3_prefill(ds3_engine* e, int32_t row, const int32_t* tokens, int32_t pos0, int32_t n,
                       float* logits_host, uint32_t* flags) {
  if (ds3_status st = refuse_if_unusable(e)) return st;
  if (e->state == ST_NOT_LOADED) return fail(e, DS3_E_NOT_LOADED, "weights are not loaded");
  if (e->state == ST_NEEDS_RESET) return fail(e, DS3_E_NEEDS_RESET, "a previous step failed; reset_state first");
  const ds3_config& c = e->cfg;
  const int T = c.prefill_rows;
  if (T < 1) return fail(e, DS3_E_UNSUPPORTED, "the engine was created with prefill_rows = 0");
  if (!tokens) return fail(e, DS3_E_INVALID, "tokens is NULL");
  if (row < 0 || row >= c.rows) return fail(e, DS3_E_INVALID, "row out of range");
  if (n < 1 || n > kMaxPrefill) return fail(e, DS3_E_INVALID, "n must be in 1.." + std::to_string(kMaxPrefill));
  if (pos0 < 0 || (int64_t)pos0 + n > c.cap) return fail(e, DS3_E_INVALID, "pos0 .. pos0 + n - 1 must lie in the capacity");
  const bool paged = c.kv_layout == DS3_KV_PAGED;
  if (paged && !e->slot_map_set) return fail(e, DS3_E_INVALID, "paged prefill needs a slot map");
  for (int i = 0; i < n; ++i)
    if (tokens[i] < 0 || tokens[i] >= c.vocab) return fail(e, DS3_E_INVALID, "token out of range at " + std::to_string(i));
  const SlotLayout sl{T};
  const int words = sl.words() + T;   // slot words, then the K/V row of each activation row
  const int chunks = (n + T - 1) / T;
  // chunk k holds tokens kT .. kT + T - 1 at positions pos0 + kT + t; the rows past the last token repeat the last
  // token at its position (they write the same K/V again and their logits are not used)
  for (int k = 0; k < chunks; ++k) {
    int32_t* w = e->h_pre + (size_t)k * words;
    for (int t = 0; t < T; ++t) {
      const int i = std::min(k * T + t, n - 1);
      const int p = pos0 + i;
      w[sl.token() + t] = tokens[i];
      w[sl.pos() + t] = p;
      int32_t wm = 0;
      if (paged) {
        const int ppr = c.cap / c.page_size;
        wm = e->h_slot_map[(size_t)row * ppr + p / c.page_size] * c.page_size + p % c.page_size;
      }
      w[sl.write_map() + t] = wm;
      w[sl.words() + t] = row;
    }
    w[sl.inject()] = 0;
    w[sl.spin()] = 0;
    w[sl.chain()] = 0;
    w[sl.sweep()] = e->kv_sweep;
  }
  const auto t_start = std::chrono::steady_clock::now();
  e->h_status->err = 0;
  e->h_status->nonfinite = 0;
  HIP_OR_POISON(e, hipMemcpyAsync(e->status, e->h_status, sizeof(StatusWords), hipMemcpyHostToDevice, e->stream));
  e->cur = e->pre;
  hipError_t h = hipSuccess;
  // two graphs: the whole prefill step (the last chunk) and the step without its final norm and head
  auto capture = [&](size_t n_launch, hipGraph_t* graph, hipGraphExec_t* exec) {
    hipError_t hc = hipStreamBeginCapture(e->stream, hipStreamCaptureModeThreadLocal);
    if (hc != hipSuccess) return hc;
    hipError_t h1 = hipSuccess;
    for (size_t i = 0; i < n_launch; ++i)
      if (h1 == hipSuccess) h1 = enqueue_kernel(e, e->pre_sequence[i]);
    hipGraph_t g = nullptr;
    hc = hipStreamEndCapture(e->stream, &g);
    if (hc == hipSuccess) hc = h1;
    if (hc != hipSuccess) {
      if (g) (void)hipGraphDestroy(g);
      return hc;
    }
    *graph = g;
    hc = hipGraphInstantiate(exec, g, nullptr, nullptr, 0);
    if (hc == hipSuccess) e->stats.captures++;
    return hc;
  };
  if (c.exec_mode == DS3_GRAPH && !e->pre_captured) {
    h = capture(e->pre_sequence.size(), &e->pre_graph, &e->pre_exec);
    if (h == hipSuccess) h = capture(e->pre_body, &e->pre_body_graph, &e->pre_body_exec);
    if (h == hipSuccess) e->pre_captured = true;
  }
  if (h == hipSuccess) h = hipEventRecord(e->ev0, e->stream);
  for (int k = 0; k < chunks && h == hipSuccess; ++k) {
    const bool last = k == chunks - 1;
    h = hipMemcpyAsync(e->pre.slots, e->h_pre + (size_t)k * words, (size_t)words * 4, hipMemcpyHostToDevice, e->stream);
    if (h != hipSuccess) break;
    if (c.exec_mode == DS3_GRAPH) {
      h = hipGraphLaunch(last ? e->pre_exec : e->pre_body_exec, e->stream);
    } else {
      const size_t n_launch = last ? e->pre_sequence.size() : e->pre_body;
      for (size_t i = 0; i < n_launch && h == hipSuccess; ++i) h = enqueue_kernel(e, e->pre_sequence[i]);
    }
  }
  e->cur = e->dec;
  HIP_OR_POISON(e, h);
  HIP_OR_POISON(e, hipEventRecord(e->ev1, e->stream));
  HIP_OR_POISON(e, hipMemcpyAsync(e->h_status, e->status, sizeof(StatusWords), hipMemcpyDeviceToHost, e->stream));
  if (logits_host)
    HIP_OR_POISON(e, hipMemcpyAsync(logits_host, e->pre.logits + (size_t)((n - 1) % T) * c.vocab, (size_t)c.vocab * 4,
                                    hipMemcpyDeviceToHost, e->stream));
  HIP_OR_POISON(e, hipEventRecord(e->ev_done, e->stream));
  e->pending = true;
  if (ds3_status st = wait_done(e, e->ev_done, e->cfg.timeout_ms)) return st;
  float gpu_ms = 0.f;
  HIP_OR_POISON(e, hipEventElapsedTime(&gpu_ms, e->ev0, e->ev1));
  e->stats.last_prefill_gpu_us = gpu_ms * 1e3;
  e->stats.last_host_us =
      std::chrono::duration<double, std::micro>(std::chrono::steady_clock::now() - t_start).count();
  if (flags) *flags = e->h_status->nonfinite ? 1u : 0u;
  if (e->h_status->err) {
    e->state = ST_NEEDS_RESET;
    e->stats.state = e->state;
    return fail(e, DS3_E_KERNEL_CHECK, "in-kernel check failed during the prefill");
  }
  e->stats.prefill_tokens += n;
  return DS3_OK;
}

ds3_status ds3_step_sample(ds3_engine* e, const int32_t* tokens, const int32_t* pos, int32_t n_steps, int32_t* ids,
                           uint32_t* flags, float* logprobs, int32_t* logprob_ids) {
  if (!ids) return fail(e, DS3_E_INVALID, "ids is NULL");
  return run_steps(e, tokens, pos, nullptr, n_steps, nullptr, ids, flags, true, logprobs, logprob_ids);
}

ds3_status ds3_set_sampling(ds3_engine* e, int32_t row, const ds3_sampling* s) {
  if (ds3_status st = refuse_if_unusable(e)) return st;
  if (!s) return fail(e, DS3_E_INVALID, "sampling parameters are NULL");
  if (row < 0 || row >= e->cfg.rows) return fail(e, DS3_E_INVALID, "row out of range");
  if (!(s->temperature >= 0.f) || !(s->top_p > 0.f && s->top_p <= 1.f) || !(s->min_p >= 0.f && s->min_p < 1.f) ||
      !(s->repetition_penalty > 0.f) || !std::isfinite(s->presence_penalty) || !std::isfinite(s->frequency_penalty) ||
      s->top_k < 0 || s->n_logprobs < 0 || s->n_logprobs > DS3_MAX_LOGPROBS)
    return fail(e, DS3_E_INVALID, "sampling parameter out of range");
  e->h_samp[(size_t)row] = SampleRow{s->temperature, s->top_p, s->min_p, s->repetition_penalty, s->presence_penalty,
                                     s->frequency_penalty, s->top_k, s->n_logprobs, (uint32_t)(s->seed & 0xffffffffu),
                                     (uint32_t)(s->seed >> 32)};
  // a new seed starts the row's generator over
  HIP_OR_POISON(e, launch_fill_u32(e->draws + row, 0u, 1, e->stream));
  HIP_OR_POISON(e, hipStreamSynchronize(e->stream));
  return DS3_OK;
}

ds3_status ds3_set_history(ds3_engine* e, int32_t row, const int32_t* tokens, int32_t n, const float* bias) {
  if (ds3_status st = refuse_if_unusable(e)) return st;
  const ds3_config& c = e->cfg;
  if (row < 0 || row >= c.rows) return fail(e, DS3_E_INVALID, "row out of range");
  if (n < 0 || (n > 0 && !tokens)) return fail(e, DS3_E_INVALID, "tokens is NULL");
  std::vector<int32_t> cnt((size_t)c.vocab, 0);
  for (int i = 0; i < n; ++i) {
    if (tokens[i] < 0 || tokens[i] >= c.vocab) return fail(e, DS3_E_INVALID, "token out of range at " + std::to_string(i));
    cnt[(size_t)tokens[i]] += 1;
  }
  std::vector<float> b((size_t)c.vocab, 0.f);
  if (bias)
    for (int v = 0; v < c.vocab; ++v) {
      if (!std::isfinite(bias[v])) return fail(e, DS3_E_INVALID, "bias must be finite");
      b[(size_t)v] = bias[v];
    }
  HIP_OR_POISON(e, hipMemcpyAsync(e->counts + (size_t)row * c.vocab, cnt.data(), (size_t)c.vocab * 4,
                                  hipMemcpyHostToDevice, e->stream));
  HIP_OR_POISON(e, hipMemcpyAsync(e->bias + (size_t)row * c.vocab, b.data(), (size_t)c.vocab * 4,
                                  hipMemcpyHostToDevice, e->stream));
  HIP_OR_POISON(e, hipStreamSynchronize(e->stream));
  return DS3_OK;
}

ds3_status ds3_set_kv_sweep(ds3_engine* e, int32_t mode) {
  if (ds3_status st = refuse_if_unusable(e)) return st;
  if (mode != DS3_SWEEP_FULL && mode != DS3_SWEEP_VISIBLE)
    return fail(e, DS3_E_INVALID, "mode must be DS3_SWEEP_FULL or DS3_SWEEP_VISIBLE");
  e->kv_sweep = mode;
  return DS3_OK;
}

ds3_status ds3_reset_state(ds3_engine* e) {
  if (ds3_status st = refuse_if_unusable(e)) return st;
  HIP_OR_POISON(e, hipMemsetAsync(e->buf[DS3_BUF_KV], 0, e->kv_bytes, e->stream));
  HIP_OR_POISON(e, launch_fill_u32(reinterpret_cast<uint32_t*>(e->status), 0u, 2, e->stream));
  HIP_OR_POISON(e, launch_fill_u32(e->sync, 0u, e->sync_words, e->stream));
  HIP_OR_POISON(e, launch_fill_u32(e->pick_done, 0u, 1, e->stream));
  HIP_OR_POISON(e, hipEventRecord(e->ev_done, e->stream));
  e->pending = true;
  if (ds3_status st = wait_done(e, e->ev_done, e->cfg.timeout_ms)) return st;
  if (e->state == ST_NEEDS_RESET) e->state = ST_READY;
  e->stats.state = e->state;
  return DS3_OK;
}

static ds3_status kv_transfer(ds3_engine* e, int32_t layer, int32_t row, int32_t pos0, int32_t n, void* k, void* v,
                              bool to_state) {
  if (ds3_status st = refuse_if_unusable(e)) return st;
  const ds3_config& c = e->cfg;
  if (!k || !v) return fail(e, DS3_E_INVALID, "k or v is NULL");
  if (layer < 0 || layer >= c.n_layers || row < 0 || row >= c.rows || pos0 < 0 || n < 0 || (int64_t)pos0 + n > c.cap)
    return fail(e, DS3_E_INVALID, "layer/row/position range out of bounds");
  if (c.kv_layout == DS3_KV_PAGED && !e->slot_map_set) return fail(e, DS3_E_INVALID, "paged KV needs a slot map");
  if (n == 0) return DS3_OK;
  const size_t kvb = dtype_bytes(c.kv_dtype);
  const size_t half = (size_t)c.n_kv_heads * n * c.head_dim * kvb;
  if (e->kv_staging_bytes < 2 * half) {
    if (e->kv_staging) HIP_OR_POISON(e, hipFree(e->kv_staging));
    e->kv_staging = nullptr;
    e->kv_staging_bytes = 0;
    HIP_OR_POISON(e, hipMalloc(&e->kv_staging, 2 * half));
    e->kv_staging_bytes = 2 * half;
  }
  char* stg = reinterpret_cast<char*>(e->kv_staging);
  // A transposed V state is staged as [nkv][hd][n] (the copy kernel then walks the state contiguously); the host
  // array is always [nkv][n][hd], so V is transposed on the host on the way in and on the way out.
  const bool vt = e->kv.v_t;
  const int nkv = c.n_kv_heads, hd = c.head_dim;
  auto transpose = [&](const char* src, char* dst, bool to_t) {
    // [nkv][n][hd] <-> [nkv][hd][n], in tiles of 64 positions so both sides stay cache-friendly
    auto run = [&](auto* d, const auto* s2) {
      for (int g = 0; g < nkv; ++g)
        for (int t0 = 0; t0 < n; t0 += 64)
          for (int x = 0; x < hd; ++x)
            for (int t = t0; t < std::min(n, t0 + 64); ++t) {
              const size_t a = ((size_t)g * n + t) * hd + x, b = ((size_t)g * hd + x) * n + t;
              if (to_t) d[b] = s2[a];
              else d[a] = s2[b];
            }
    };
    if (kvb == 2) run(reinterpret_cast<uint16_t*>(dst), reinterpret_cast<const uint16_t*>(src));
    else run(reinterpret_cast<uint32_t*>(dst), reinterpret_cast<const uint32_t*>(src));
  };
  std::vector<char> vtmp(vt ? half : 0);
  if (to_state) {
    if (vt) transpose(reinterpret_cast<const char*>(v), vtmp.data(), true);
    HIP_OR_POISON(e, hipMemcpyAsync(stg, k, half, hipMemcpyHostToDevice, e->stream));
    HIP_OR_POISON(e, hipMemcpyAsync(stg + half, vt ? vtmp.data() : v, half, hipMemcpyHostToDevice, e->stream));
    HIP_OR_POISON(e, launch_kv_copy(e->kv, c.kv_dtype, layer, row, pos0, n, nkv, hd, stg, 1, vt, e->status, e->stream));
  } else {
    HIP_OR_POISON(e, launch_kv_copy(e->kv, c.kv_dtype, layer, row, pos0, n, nkv, hd, stg, 0, vt, e->status, e->stream));
    HIP_OR_POISON(e, hipMemcpyAsync(k, stg, half, hipMemcpyDeviceToHost, e->stream));
    HIP_OR_POISON(e, hipMemcpyAsync(vt ? vtmp.data() : v, stg + half, half, hipMemcpyDeviceToHost, e->stream));
  }
  HIP_OR_POISON(e, hipEventRecord(e->ev_done, e->stream));
  e->pending = true;
  if (ds3_status st = wait_done(e, e->ev_done, e->cfg.timeout_ms)) return st;
  if (!to_state && vt) transpose(vtmp.data(), reinterpret_cast<char*>(v), false);
  return DS3_OK;
}

ds3_status ds3_write_kv(ds3_engine* e, int32_t layer, int32_t row, int32_t pos0, int32_t n, const void* k,
                        const void* v) {
  return kv_transfer(e, layer, row, pos0, n, const_cast<void*>(k), const_cast<void*>(v), true);
}

ds3_status ds3_read_kv(ds3_engine* e, int32_t layer, int32_t row, int32_t pos0, int32_t n, void* k, void* v) {
  return kv_transfer(e, layer, row, pos0, n, k, v, false);
}

// As ds3_write_kv, staged through the device's file-scope scratch array instead of a buffer the library allocates:
// the host arrays are copied into it as they are and the copy kernel transposes V on the device.
ds3_status ds3_write_kv_noalloc(ds3_engine* e, int32_t layer, int32_t row, int32_t pos0, int32_t n, const void* k,
                                const void* v) {
  if (ds3_status st = refuse_if_unusable(e)) return st;
  const ds3_config& c = e->cfg;
  if (!k || !v) return fail(e, DS3_E_INVALID, "k or v is NULL");
  if (layer < 0 || layer >= c.n_layers || row < 0 || row >= c.rows || pos0 < 0 || n < 0 || (int64_t)pos0 + n > c.cap)
    return fail(e, DS3_E_INVALID, "layer/row/position range out of bounds");
  if (c.kv_layout == DS3_KV_PAGED && !e->slot_map_set) return fail(e, DS3_E_INVALID, "paged KV needs a slot map");
  const size_t half = (size_t)c.n_kv_heads * n * c.head_dim * dtype_bytes(c.kv_dtype);
  if (2 * half > kScratchBytes)
    return fail(e, DS3_E_INVALID, "K and V of " + std::to_string(n) + " positions take " + std::to_string(2 * half) +
                                      " bytes, more than the " + std::to_string(kScratchBytes) + "-byte scratch array");
  if (n == 0) return DS3_OK;
  char* stg = reinterpret_cast<char*>(e->scratch);
  HIP_OR_POISON(e, hipMemcpyAsync(stg, k, half, hipMemcpyDefault, e->stream));
  HIP_OR_POISON(e, hipMemcpyAsync(stg + half, v, half, hipMemcpyDefault, e->stream));
  HIP_OR_POISON(e, launch_kv_copy(e->kv, c.kv_dtype, layer, row, pos0, n, c.n_kv_heads, c.head_dim, stg, 1, 0,
                                  e->status, e->stream));
  HIP_OR_POISON(e, hipEventRecord(e->ev_done, e->stream));
  e->pending = true;
  return wait_done(e, e->ev_done, e->cfg.timeout_ms);
}

ds3_status ds3_stats_get(const ds3_engine* e, ds3_stats* out) {
  if (!e || !out) return DS3_E_INVALID;
  *out = e->stats;
  out->state = e->state;
  out->attn_splits = e->fused ? kFusedBlocks / e->cfg.n_kv_heads : e->splits;
  out->kernel_plan = e->fused ? DS3_PLAN_FUSED : DS3_PLAN_PER_OP;
  if (out->kernels_per_step == 0) out->kernels_per_step = (int)e->sequence.size();
  return DS3_OK;
}

// Each kernel kind's launches of one step (in step order) are captured as a graph of their own and replayed
// `iters` times between two HIP events: the device time of that kind per step, measured as the step graph runs
// kernels (back to back, no host launch between them). A kind with fewer than 32 launches per step is captured
// repeated up to at least 32 kernels, and its time divided accordingly. One whole step then runs again with the same slots, which
// restores the K/V entries at the slot positions and the work buffers the replays overwrote.
ds3_status ds3_profile_kernels(ds3_engine* e, int32_t iters, ds3_kernel_time* out, int32_t* n_inout) {
  if (ds3_status st = refuse_if_unusable(e)) return st;
  if (e->state != ST_READY) return fail(e, DS3_E_NOT_LOADED, "engine is not ready");
  if (!out || !n_inout || *n_inout < K_NUM || iters < 1) return fail(e, DS3_E_INVALID, "need room for the kernel kinds");
  std::vector<double> tot(K_NUM, 0.0);
  std::vector<int> cnt(K_NUM, 0);
  for (const Launch& l : e->sequence) cnt[l.kind]++;
  e->h_status->err = 0;
  e->h_status->nonfinite = 0;
  HIP_OR_POISON(e, hipMemcpyAsync(e->status, e->h_status, sizeof(StatusWords), hipMemcpyHostToDevice, e->stream));
  for (int k = 0; k < K_NUM; ++k) {
    if (!cnt[k]) continue;
    // a kind with few launches per step (embed, LM head) is repeated so that the graph holds at least 32
    // kernels and the replay's own launch latency is spread thin
    const int reps = (32 + cnt[k] - 1) / cnt[k];
    HIP_OR_POISON(e, hipStreamBeginCapture(e->stream, hipStreamCaptureModeThreadLocal));
    hipError_t h = hipSuccess;
    for (int rep = 0; rep < reps; ++rep)
      for (const Launch& l : e->sequence)
        if (l.kind == k && h == hipSuccess) h = enqueue_kernel(e, l);
    hipGraph_t g = nullptr;
    hipError_t h2 = hipStreamEndCapture(e->stream, &g);
    if (h != hipSuccess || h2 != hipSuccess) {
      if (g) (void)hipGraphDestroy(g);
      return poison(e, DS3_E_DEVICE_LOST, std::string("profile capture: ") + hipGetErrorString(h != hipSuccess ? h : h2));
    }
    hipGraphExec_t x = nullptr;
    h = hipGraphInstantiate(&x, g, nullptr, nullptr, 0);
    if (h == hipSuccess) h = hipGraphLaunch(x, e->stream);   // warm-up replay
    if (h == hipSuccess) h = hipEventRecord(e->ev0, e->stream);
    for (int it = 0; it < iters && h == hipSuccess; ++it) h = hipGraphLaunch(x, e->stream);
    if (h == hipSuccess) h = hipEventRecord(e->ev1, e->stream);
    if (h == hipSuccess) h = hipEventRecord(e->ev_done, e->stream);
    ds3_status st = DS3_OK;
    if (h != hipSuccess) {
      st = poison(e, DS3_E_DEVICE_LOST, std::string("profile: ") + hipGetErrorString(h));
    } else {
      e->pending = true;
      st = wait_done(e, e->ev_done, e->cfg.timeout_ms);
    }
    float ms = 0.f;
    if (st == DS3_OK && hipEventElapsedTime(&ms, e->ev0, e->ev1) != hipSuccess)
      st = poison(e, DS3_E_DEVICE_LOST, "profile: event timing failed");
    if (x) (void)hipGraphExecDestroy(x);
    (void)hipGraphDestroy(g);
    if (st != DS3_OK) return st;
    tot[k] = ms * 1e3 / ((double)iters * reps);
  }
  // fused plan: each operation's share of the kernel, from block 0's clock at the start, after every barrier
  // and at the end (100 MHz), averaged over `iters` launches
  std::vector<double> phase_us(K_NUM, 0.0);
  std::vector<int> phases(K_NUM, 0);
  if (e->fused) {
    const int L = e->cfg.n_layers, nc = kFusedPhases * L + 2;
    std::vector<unsigned long long> clk((size_t)nc);
    for (int it = 0; it < iters; ++it) {
      HIP_OR_POISON(e, hipMemcpyAsync(e->slots, e->h_slots, (size_t)SlotLayout{e->cfg.rows}.words() * 4,
                                      hipMemcpyHostToDevice, e->stream));   // (each step's pick advanced them)
      e->profiling = true;
      const hipError_t hp = enqueue_step(e);
      e->profiling = false;
      HIP_OR_POISON(e, hp);
      HIP_OR_POISON(e, hipMemcpyAsync(clk.data(), e->clocks, (size_t)nc * 8, hipMemcpyDeviceToHost, e->stream));
      HIP_OR_POISON(e, hipEventRecord(e->ev_done, e->stream));
      e->pending = true;
      if (ds3_status st = wait_done(e, e->ev_done, e->cfg.timeout_ms)) return st;
      for (int b = 0; b < kFusedPhases * L; ++b)
        phase_us[kPhaseKind[b % kFusedPhases]] += (double)(clk[b + 1] - clk[b]) * 0.01 / iters;
      phase_us[K_HEAD] += (double)(clk[nc - 1] - clk[nc - 2]) * 0.01 / iters;
    }
    for (int k : kPhaseKind) phases[k] = L;
    phases[K_HEAD] = 1;
  }
  // the greedy pick's replays advanced the device slots: the closing step runs from the last call's words again
  HIP_OR_POISON(e, hipMemcpyAsync(e->slots, e->h_slots, (size_t)SlotLayout{e->cfg.rows}.words() * 4,
                                  hipMemcpyHostToDevice, e->stream));
  HIP_OR_POISON(e, enqueue_step(e));
  HIP_OR_POISON(e, hipEventRecord(e->ev_done, e->stream));
  e->pending = true;
  if (ds3_status st = wait_done(e, e->ev_done, e->cfg.timeout_ms)) return st;
  for (int k = 0; k < K_NUM; ++k) {
    std::snprintf(out[k].name, sizeof(out[k].name), "%s", kKindNames[k]);
    const bool phase = e->fused && k != K_FUSED && k != K_PICK;   // fused: a phase of the step kernel
    out[k].launches = phase ? phases[k] : cnt[k];
    out[k].total_us = phase ? phase_us[k] : tot[k];
    out[k].bytes = kind_bytes(e->cfg, k);
  }
  *n_inout = K_NUM;
  return DS3_OK;
}

ds3_status ds3_phase_trace(ds3_engine* e, uint64_t* out, int32_t* n_inout) {
  if (ds3_status st = refuse_if_unusable(e)) return st;
  if (!e->fused) return fail(e, DS3_E_UNSUPPORTED, "phase trace needs the fused plan");
  if (e->cfg.trace == DS3_TRACE_OFF)
    return fail(e, DS3_E_UNSUPPORTED, "phase trace needs an engine created with trace = DS3_TRACE_BARRIERS or above");
  const int64_t n2 = (int64_t)kFusedPhases * e->cfg.n_layers * kFusedBlocks * 2;
  if (!out || !n_inout || *n_inout < n2) return fail(e, DS3_E_INVALID, "need room for " + std::to_string(n2) + " words");
  const int64_t n = *n_inout >= 5 * n2 ? 5 * n2 : n2;   // with room: the sub-phase clocks follow
  HIP_OR_POISON(e, hipMemcpyAsync(out, e->trace, (size_t)n * 8, hipMemcpyDeviceToHost, e->stream));
  HIP_OR_POISON(e, hipEventRecord(e->ev_done, e->stream));
  e->pending = true;
  if (ds3_status st = wait_done(e, e->ev_done, e->cfg.timeout_ms)) return st;
  *n_inout = (int32_t)n;
  return DS3_OK;
}

ds3_status ds3_debug_inject(ds3_engine* e, int32_t kind) {
  if (ds3_status st = refuse_if_unusable(e)) return st;
  if (kind == DS3_INJECT_KERNEL_CHECK) e->inject_check = true;
  else if (kind == DS3_INJECT_TIMEOUT_NEXT) e->inject_timeout = true;
  else if (kind == DS3_INJECT_BARRIER_TIMEOUT) e->inject_barrier = true;
  else return fail(e, DS3_E_INVALID, "unknown injection");
  return DS3_OK;
}

ds3_status ds3_probe_read(const void* buf, uint64_t bytes, void* sink, void* hip_stream) {
  if (!buf || !sink || bytes < 16 || bytes % 16) return fail(nullptr, DS3_E_INVALID, "probe: buf, sink and bytes (a multiple of 16)");
  const hipError_t h = launch_stream_read(buf, (size_t)bytes, reinterpret_cast<uint32_t*>(sink),
                                          reinterpret_cast<hipStream_t>(hip_stream));
  if (h != hipSuccess) return fail(nullptr, DS3_E_DEVICE_LOST, std::string("probe: ") + hipGetErrorString(h));
  return DS3_OK;
}

const char* ds3_last_error(const ds3_engine* e) { return e ? e->err.c_str() : g_last_error.c_str(); }

void ds3_destroy(ds3_engine* e) {
  if (!e) return;
  // Work from an earlier step may still be running after a timeout: wait for it (bounded) before releasing
  // anything the kernels could touch.
  if (e->pending && e->ev_done) {
    const auto t0 = std::chrono::steady_clock::now();
    while (hipEventQuery(e->ev_done) == hipErrorNotReady &&
           std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count() <
               (double)(e->cfg.timeout_ms ? e->cfg.timeout_ms : kDefaultTimeoutMs))
      std::this_thread::sleep_for(std::chrono::microseconds(100));
  }
  if (e->exec) (void)hipGraphExecDestroy(e->exec);
  if (e->graph) (void)hipGraphDestroy(e->graph);
  if (e->samp_exec) (void)hipGraphExecDestroy(e->samp_exec);
  if (e->samp_graph) (void)hipGraphDestroy(e->samp_graph);
  if (e->h_samp_pinned) (void)hipHostFree(e->h_samp_pinned);
  if (e->h_lp) (void)hipHostFree(e->h_lp);
  if (e->pre_exec) (void)hipGraphExecDestroy(e->pre_exec);
  if (e->pre_graph) (void)hipGraphDestroy(e->pre_graph);
  if (e->pre_body_exec) (void)hipGraphExecDestroy(e->pre_body_exec);
  if (e->pre_body_graph) (void)hipGraphDestroy(e->pre_body_graph);
  if (e->h_pre) (void)hipHostFree(e->h_pre);
  for (hipEvent_t ev : {e->ev0, e->ev1, e->ev_done})
    if (ev) (void)hipEventDestroy(ev);
  if (e->h_slots) (void)hipHostFree(e->h_slots);
  if (e->h_chain) (void)hipHostFree(e->h_chain);
  if (e->kv_staging) (void)hipFree(e->kv_staging);
  if (e->own_stream && e->stream) (void)hipStreamDestroy(e->stream);
  delete e;
}

}  // extern "C"
