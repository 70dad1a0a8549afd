// Internal interface between the engine (host) and the decode-step kernels (device). Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ds3 {

// Bits of the device error word. A kernel that finds an out-of-range slot value sets its bit and substitutes a
// safe value, so every access stays in bounds and every wave exits normally.
enum : uint32_t {
  ERR_TOKEN = 1u,       // Slot::Token outside [0, vocab)
  ERR_POS = 2u,         // Slot::Pos outside [0, cap)
  ERR_WRITE_MAP = 4u,   // Slot::WriteMap outside the pool
  ERR_PAGE = 8u,        // a page id of the SlotMap outside [0, pool_pages)
  ERR_INJECTED = 16u,   // test hook
  ERR_BARRIER = 32u,    // fused step kernel: a grid barrier outlasted its spin limit (blocks not co-resident)
};

// Slot buffer layout (int32 words at fixed device addresses; the host rewrites them before every replay).
struct SlotLayout {
  int rows;
  __host__ __device__ int token() const { return 0; }
  __host__ __device__ int pos() const { return rows; }
  __host__ __device__ int write_map() const { return 2 * rows; }
  __host__ __device__ int inject() const { return 3 * rows; }
  __host__ __device__ int spin() const { return 3 * rows + 1; }   // fused kernel: barrier wait limit, 0 = default
  __host__ __device__ int chain() const { return 3 * rows + 2; }  // greedy pick: steps since the host wrote slots
  __host__ __device__ int sweep() const { return 3 * rows + 3; }  // 1: K/V chunks wholly after pos are not loaded
  __host__ __device__ int sample() const { return 3 * rows + 4; } // 1: the sampler kernel picks (fused: no pick)
  __host__ __device__ int words() const { return 3 * rows + 5; }
};

// Status words written by kernels and read back after every step.
struct StatusWords {
  uint32_t err;        // ERR_* bits
  uint32_t nonfinite;  // 1 if some logit is NaN or infinite
};

// Where the K/V state lives and how a (row, kv head, position) maps to an address.
struct KvView {
  void* k;               // layer 0 base of K (contiguous: [rows][nkv][cap][hd]; paged: [pages][nkv][ps][hd])
  void* v;               // layer 0 base of V: as K, or transposed when v_t (contiguous: [rows][nkv][hd][cap];
                         // paged: [pages][nkv][hd][ps]) -- the matrix-core attention reads V position-contiguous
  int64_t layer_stride;  // elements between consecutive layers
  int paged;             // 0 contiguous, 1 paged
  int v_t;               // 1: V stored transposed (bf16 KV)
  int cap;
  int page_size;
  int pool_pages;
  const int* slot_map;   // paged: [rows][cap/page_size]
  const int* row_map;    // null: activation row r uses K/V row r; else row_map[r] (a prefill: every token of the
                         // chunk is an activation row of the same K/V row)
};

enum GemvMode : int {
  GEMV_QKV = 0,      // RMSNorm(x) -> [q;k;v] rows, rotary epilogue, K/V write at Slot::Pos
  GEMV_GATEUP = 1,   // RMSNorm(x) -> gate/up rows, SwiGLU epilogue -> act
  GEMV_RESID = 2,    // act -> rows, residual add into x
  GEMV_HEAD = 3,     // RMSNorm(x) -> logits
};

struct GemvParams {
  const void* w;         // weight rows [n_rows_total][K] (bf16 words or float32)
  const float* in;       // activation input [rows][K] (fp32); RMSNorm input for the norm modes
  const float* gain;     // RMSNorm gain [K] (fp32), norm modes only
  float* out;            // QKV: q [rows][nq*hd]; GATEUP: act [rows][F]; RESID: x [rows][n_out]; HEAD: logits
  int K;                 // input width
  int n_pairs;           // output row pairs
  int rows;              // activation rows (1..kMaxGemvRows)
  float eps;
  // QKV only
  int nq, nkv, hd;
  const float* rope;     // [cap][hd/2][2] cos, sin
  KvView kv;
  int layer;
  // GATEUP: offset of the up rows after the gate rows (= F); HEAD/RESID: unused
  int up_offset;
  // shared
  const int* slots;      // slot buffer
  StatusWords* status;
  int ping_pong;         // rows longer than one group: two groups in flight per wave
};

struct AttnParams {
  const float* q;        // [rows][nq][hd]
  float* out;            // [rows][nq][hd]
  float* part;           // split partials: [rows][nkv][splits][G][hd + 2] (weighted value sums, max, weight sum)
  KvView kv;
  int layer;
  int nq, nkv, hd;
  int splits;
  int split_len;         // positions per split (multiple of the positions one block pass covers)
  float scale;           // 1/sqrt(hd)
  const int* slots;
  StatusWords* status;
  uint16_t* frag_hi;     // combine, matrix-core path: also the o-projection's activation fragments (else null)
  uint16_t* frag_lo;
  int nt;                // their activation tiles (sk_tiles(rows))
};

// Greedy pick after the LM head ("Execution" page, section "A constant-shape decode graph": the step's output
// token is chosen on the device, so a run of steps needs no host round trip). Each row's logits are split over
// kPickSplit blocks; every block writes the (value, index) of its slice's largest logit (first index on ties;
// NaN never wins); the last block to finish (device-scope counter) combines the slices of every row and writes
// the picks into the token slots, pos + 1 into the position slots (and the K/V write slot of pos + 1 from the
// page table, paged layout), the picks into ids[step % max_chain] and the step's non-finite flag into
// flags[step % max_chain] (then clears it for the next step), and advances the step counter.
constexpr int kPickSplit = 16;
struct PickParams {
  const float* logits;     // [rows][vocab]
  int vocab, rows;
  int32_t* slots;          // SlotLayout{rows}
  const int* page_table;   // paged: [rows][cap / page_size]; else null
  int page_size, cap;
  float* part_val;         // [rows][kPickSplit]
  int* part_idx;           // [rows][kPickSplit]
  unsigned* done;          // finished-block counter (back to 0 after every launch)
  int32_t* ids;            // [max_chain][rows]
  uint32_t* flags;         // [max_chain]
  int max_chain;
  StatusWords* status;
};

// Sampling suffix (the sampler kernel; one block per row). Per-row parameters: temperature 0 is greedy; top_k 0,
// top_p 1 and min_p 0 are off; penalties 1 / 0 / 0 are off.
constexpr int kMaxLogprobs = 8;
struct SampleRow {
  float temperature, top_p, min_p, rep, presence, frequency;
  int32_t top_k, n_logprobs;
  uint32_t seed_lo, seed_hi;
};
// The sampler's first kernel splits each row's vocabulary into segments of kSampSeg tokens, one block each, and
// leaves one record per (row, segment): the segment's best (value, index) of the adjusted logits, its log-sum-exp
// partial (max and sum of exp(s - max), s = z / T), its top kMaxLogprobs tokens by rank, and -- when the row's top-k
// is small enough for the candidate path -- its own top-k tokens in index order. The global top-k lies in the union
// of the segments' top-k sets, so the per-row kernel selects from at most kSampCand candidates instead of the
// vocabulary.
constexpr int kSampSeg = 2048;    // tokens per segment block
constexpr int kSampFastK = 128;   // largest top-k the candidate path takes
constexpr int kSampCand = 8192;   // most candidates of one row (segments x top-k)
struct SampPart {
  float best_v;
  int best_i;
  float m, l;                     // log-sum-exp partial: max of s and sum of exp(s - m) over the segment
  float top_v[kMaxLogprobs];      // top by rank (s descending, index ascending): s and token
  int top_i[kMaxLogprobs];
  int n_cand;
  int pad[3];
  int cand_v[kSampFastK];         // the segment's top-k tokens in index order, and their adjusted logits
  float cand_x[kSampFastK];
};
__host__ __device__ inline int samp_segments(int vocab) { return (vocab + kSampSeg - 1) / kSampSeg; }

struct SampleParams {
  const float* logits;      // [rows][vocab]
  int vocab, rows;
  int32_t* slots;           // SlotLayout{rows}
  const int* page_table;    // paged: [rows][cap / page_size]; else null
  int page_size, cap;
  const SampleRow* rowp;    // [rows]
  int32_t* counts;          // [rows][vocab] token history (the draws add to it)
  const float* bias;        // [rows][vocab] logit bias
  uint32_t* draws;          // [rows] temperature draws so far (the generator's counter)
  float* z;                 // [rows][vocab] scratch: adjusted logits
  SampPart* part;           // [rows][samp_segments(vocab)] scratch: the segment records
  int32_t* ids;             // [max_chain][rows]
  uint32_t* flags;          // [max_chain]
  float* lp;                // [max_chain][rows][1 + kMaxLogprobs]: the drawn token's logprob, then the top-n
  int32_t* lp_ids;          // [max_chain][rows][kMaxLogprobs]
  int max_chain;
  StatusWords* status;
  uint32_t* done;           // [1] the row blocks' ticket: the last one closes the step (zero between launches)
};

struct EmbedParams {
  const void* table;     // [vocab][d]
  float* x;              // [rows][d]
  int d, vocab, rows;
  const int* slots;
  StatusWords* status;
};

// MFMA path (5..16 rows of a decode step, 5..64 of a prefill step): activations are handed to the matrix cores as
// two bf16 parts, hi = bf16(a) and lo = bf16(a - hi), stored in the operand order of v_mfma_f32_16x16x32_bf16
// (step t of 32 inputs, tile c of 16 activation rows, lane l holds inputs 32t + 8(l/16) .. +8 of activation row
// 16c + l % 16), the "fragments" [K/32][nt][64][8] with nt = 1 (up to 16 rows) or 4 (up to 64). Rows past the
// step's rows are zero. The kernel that produces an activation writes its fragments.

constexpr int kMaxGemvRows = 4;
constexpr int kMaxRows = 16;          // rows of a decode step
constexpr int kMaxPrefillRows = 64;   // tokens of a prefill step
constexpr int kMfmaRows = 16;         // activation rows of one MFMA tile (rows are zero-padded to whole tiles)
constexpr int kSsRows = kMaxPrefillRows;   // row stride of the RMSNorm sums of squares
// activation tiles of a matrix-core step of `rows` rows
__host__ __device__ inline int sk_tiles(int rows) { return rows > kMfmaRows ? 4 : 1; }

// Matrix-core projection plan (stream-K). The weight matrix [N][K] is cut into groups of kSkRows rows (two 16-row
// tiles), four neighbouring groups form a quad, and the items (quad, chunk of kSkChunk inputs), numbered
// quad-major, are split into equal contiguous runs, one per block: block b streams items [first(b), first(b + 1))
// whatever N and K, its wave w taking group w of each quad (the four waves share the chunk's activations). A wave
// stores one partial product per group it touched: part[group][k][activation tile c][tile 0/1][lane 64][4] fp32,
// k = block - block_of(first item of the group's quad) (the MFMA output layout: lane l, element e is weight row
// 16 tile + 4 (l / 16) + e of the group and activation row 16 c + l % 16). The kernel that consumes the projection
// sums a group's k = 0, 1, ... in order, which is input order.
constexpr int kSkRows = 32;        // weight rows per group (two 16-row tiles)
constexpr int kSkQuad = 4;         // groups per quad = waves per block
constexpr int kSkChunk = 128;      // inputs per chunk
constexpr int kSkWaves = kSkQuad;  // waves per block (one block per CU: its LDS takes 120 KB)
constexpr int kSkMaxBlocks = 256;
constexpr int kActSpan = 256;      // SwiGLU consumer: outputs per block (one wave, 4 per lane)
constexpr int kNormSpan = 256;     // norm prep: inputs per block (one wave, 4 per lane), one sum of squares each
struct SkPlan {
  int groups;   // N / kSkRows
  int nck;      // K / kSkChunk
  int nb;       // blocks with work (every one has at least one item, or one quad with whole quads)
  int cmax;     // most blocks that contribute to one group
  __host__ __device__ int quads() const { return groups / kSkQuad; }
  __host__ __device__ unsigned total() const { return (unsigned)quads() * (unsigned)nck; }
  __host__ __device__ int first(int b) const { return (int)(total() * (unsigned)b / (unsigned)nb); }
  // the block whose run holds item i (total x nb < 2^32: sk_plan checks it)
  __host__ __device__ int block_of(int i) const { return (int)(((unsigned)(i + 1) * (unsigned)nb - 1) / total()); }
};
// whole_quads: each block takes whole quads (the LM head, whose epilogue writes the logits itself).
// Returns a plan with groups == 0 if the shape is outside what the kernels take.
SkPlan sk_plan(int n_rows, int K, bool whole_quads);
inline size_t sk_partial_floats(const SkPlan& p, int nt) { return (size_t)p.groups * p.cmax * nt * 512; }

struct SkGemmParams {
  const uint16_t* w;     // [N][K] bf16
  const uint16_t* hi;    // activation fragments [K/32][nt][64][8]
  const uint16_t* lo;
  int K;
  SkPlan plan;
  float* part;           // partial products (see SkPlan)
  // LM head (whole groups): logits[r][n] = scale_r * sum, scale_r from the final norm's sums of squares
  float* out;
  int rows, n_out;
  int nt;                // activation tiles (sk_tiles(rows))
  const float* ss;       // [ss_blocks][kSsRows] per-block sums of squares of x
  int ss_blocks, norm_dim;
  float eps;
  StatusWords* status;
};

// x (+)= the partial products of the projection that produced it (part null: x as it is); per block and row the
// sum of squares of x into ss; the fragments of gain * x. The RMSNorm's row scale is applied by the consumer.
struct SkPrepParams {
  float* x;              // [rows][D]
  const float* part;
  SkPlan plan;
  const float* gain;     // [D]
  uint16_t* hi;
  uint16_t* lo;
  float* ss;             // [ceil(D / kNormSpan)][kSsRows]
  int D, rows, nt;       // (nt: activation tiles of the partials and the fragments)
};

// QKV epilogue on the partial products: scale, rotary on q and k, q out, k and v stored at Slot::Pos / WriteMap.
struct SkQkvParams {
  const float* part;
  SkPlan plan;
  const float* ss;
  int ss_blocks, D;
  float eps;
  float* q;              // [rows][nq][hd]
  int nq, nkv, hd;
  const float* rope;     // [cap][hd/2][2]
  KvView kv;
  int layer;
  const int* slots;
  StatusWords* status;
  int rows, nt;
};

// SwiGLU on the partial products (gate rows 0..F-1, up rows F..2F-1): fragments of silu(gate) * up.
struct SkActParams {
  const float* part;
  SkPlan plan;
  const float* ss;
  int ss_blocks, D;
  float eps;
  int F, rows, nt;
  uint16_t* hi;
  uint16_t* lo;
};

// Fused step kernel (batch 1): the whole step as one persistent launch of kFusedBlocks blocks (one per CU),
// its phases separated by grid barriers. Weight offsets are relative to `wbase`; layer l's tensors sit at
// wbase + l * lstride + o_*.
constexpr int kFusedBlocks = 256;
constexpr int kFusedPhases = 5;   // per layer: qkv, attention, o-proj, gate/up, down (a grid barrier after each)

struct FusedParams {
  const char* wbase;
  size_t lstride;
  size_t o_attn_norm, o_wqkv, o_wo, o_ffn_norm, o_wgu, o_wd;
  const uint16_t* embed;       // [vocab][d] bf16
  const float* final_norm;     // [d]
  const uint16_t* lm_head;     // [vocab][d] bf16
  KvView kv;                   // contiguous bf16, V transposed
  const float* rope;           // [cap][hd/2][2]
  float* x;                    // [d] residual stream
  float* q;                    // [nq][hd]
  float* kvnew;                // [nkv][2][hd]: this step's k (rotated) and v, fp32
  float* attn;                 // [nq][hd] attention output
  float* act;                  // [ffn] SwiGLU output
  float* part;                 // [nkv][splits][G][hd + 2] split partials
  float* logits;               // [vocab]
  unsigned* sync;              // fused_sync_words: epoch, abort flag, arrival / release / split flags
  unsigned long long* clocks;  // [5 L + 2] block 0's clock at the start, after every barrier, at the end
  unsigned long long* trace;   // [5 L][kFusedBlocks][2] every block's arrival and release time per barrier
  unsigned long long* trace2;  // optional [5 L][kFusedBlocks][4] GEMV sub-phase clocks of wave 0 (null: off)
  int* slots;                  // read at the start; the greedy pick advances token and pos at the end
  StatusWords* status;
  int32_t* ids;                // greedy pick: [max_chain][1] picks and [max_chain] non-finite flags of a chain
  uint32_t* chain_flags;
  int max_chain;
  int n_layers, vocab, cap;
  int split_len;               // positions per split
  float eps, scale;            // RMSNorm eps, 1/sqrt(hd)
};
constexpr long long kFusedSpinTicks = 200000000LL;   // default grid-barrier wait limit: 2 s of the 100 MHz clock

// The fused kernel's sync region (32-bit words): [0] launch epoch, [1] abort flag, [kSyncArrive..+256) each
// block's barrier arrival flag, [kSyncSplit + 32 g + s] split s of kv head g has written its attention partial.
// No flag is ever reset: each holds the generation (epoch x (5 L + 1) + barrier + 1) it last signalled.
constexpr int kSyncArrive = 256, kSyncSplit = 1024;
inline size_t fused_sync_words(int n_layers, int nkv) { (void)n_layers; return (size_t)kSyncSplit + 32 * (size_t)nkv; }

// Host launchers (defined in ds3_kernels.hip). Each returns the launch error, if any.
hipError_t launch_sk_gemm(const SkGemmParams& p, bool head, hipStream_t s);
hipError_t launch_sk_prep(const SkPrepParams& p, hipStream_t s);
hipError_t launch_sk_qkv(const SkQkvParams& p, int kv_dtype, hipStream_t s);
hipError_t launch_sk_swiglu(const SkActParams& p, hipStream_t s);
hipError_t launch_embed(const EmbedParams& p, int weight_dtype, hipStream_t s);
hipError_t launch_gemv(const GemvParams& p, int mode, int weight_dtype, int kv_dtype, int blocks, hipStream_t s);
hipError_t launch_attention(const AttnParams& p, int kv_dtype, int rows, hipStream_t s);
hipError_t launch_attention_combine(const AttnParams& p, int rows, hipStream_t s);
// staging: K [nkv][n][hd], then V as [nkv][hd][n] when stage_vt, else [nkv][n][hd] (the state's own V order,
// transposed or not, is the KvView's)
hipError_t launch_kv_copy(const KvView& kv, int kv_dtype, int layer, int row, int pos0, int n, int nkv, int hd,
                          void* staging, int to_state, int stage_vt, StatusWords* status, hipStream_t s);
// Allocation-free staging: a file-scope device array of kScratchBytes per GPU (its address for `device`, looked
// up once per device)
constexpr size_t kScratchBytes = (size_t)8 << 20;
hipError_t scratch_device_ptr(int device, void** out);
hipError_t launch_fill_u32(uint32_t* p, uint32_t value, size_t n, hipStream_t s);
// Streaming-read probe (measurement): reads `bytes` (a multiple of 16) once; `sink` holds at least 1024 words.
hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t s);
hipError_t launch_pick(const PickParams& p, hipStream_t s);
hipError_t launch_sample(const SampleParams& p, hipStream_t s);
// Fused step kernel (ds3_fused.hip). fused_shape_supported: the model shape has a compiled instantiation.
bool fused_shape_supported(int d, int ffn, int hd, int nq, int nkv);
hipError_t launch_fused(const FusedParams& p, int d, int ffn, int hd, int nq, int nkv, bool trace, hipStream_t s);
// Blocks of the fused kernel one compute unit holds at once (its LDS and registers decide).
hipError_t fused_blocks_per_cu(int d, int ffn, int hd, int nq, int nkv, int split_len, int* out);

size_t gemv_lds_bytes(int rows, int K, bool norm);
int attn_positions_per_pass(int hd, int kv_dtype);
size_t attn_lds_bytes(int nq, int nkv, int hd, int split_len, int kv_dtype, int page_size /* 0: contiguous */);
int attn_max_splits(int nq, int nkv, int hd);   // splits the in-kernel merge can take

}  // namespace ds3
