// Host-side declarations shared by libfdllm's translation units (launchers and the handle).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <vector>

#include "../../include/libfdllm.h"

struct fdl_ctx {
  hipStream_t stream;
  int device;
  int num_cus;
  char* ws;              // workspace base (device)
  size_t ws_bytes;
  uint32_t* status;      // device status word
  uint32_t* tickets;     // split-merge tickets, kSyncStride apart per (b, head); left at zero
  uint32_t* barriers;    // split barriers of the fused kernel, kSyncStride apart per (b, head)
  int spin_limit;        // polls a fused-kernel split waits for its siblings (FDL_SPIN_LIMIT)
  char* sink_area;       // header area of the sink detection state
  char* scratch;         // general scratch after the fixed header
  size_t scratch_bytes;
  char last_error[256];
  bool capturing = false;   // between fdl_capture_begin and fdl_capture_end
  uint64_t* stamps = nullptr;   // fdl_set_phase_buffer
  uint32_t fused_serial = 0;    // fused launches issued (part of their score-exchange tag)
  bool safe_sync = false;       // FDL_SAFE_SYNC: no hand-over between workgroups through L2
  uint32_t debug_seen = 0;      // debug build: the status word as last reported
  int64_t stamp_words = 0;
  // optional event timing (fdl_profile_begin / fdl_profile_end)
  struct ProfRec {
    int kind;
    hipEvent_t a, b;
    int n = 1;   // launches (layers) the pair brackets
  };
  bool prof_on = false;
  uint32_t prof_mask = 0;
  int prof_every = 1;
  long long prof_seen[FDL_PROF_KINDS] = {};
  size_t prof_used = 0;
  std::vector<hipEvent_t> prof_pool;
  std::vector<ProfRec> prof_recs;
};

namespace fdl {

constexpr size_t kHeaderBytes = 1u << 20;        // status + tickets + barriers
constexpr int kMaxTickets = 65536;               // B * Hkv limit for split attention
constexpr size_t kTicketOffset = 4096;
// Heads split over several workgroups synchronise through per-head words in the header, each in a
// 256-byte line of its own so that the atomics of different heads do not queue on one L2 line.
// Only launches with at most kMaxSplitSegs (sequence, head) pairs split at all.
constexpr int kMaxSplitSegs = 256;
constexpr int kSyncStride = 64;                  // uint32 words between two heads' sync words
constexpr size_t kBarrierOffset = kTicketOffset + (size_t)kMaxSplitSegs * kSyncStride * sizeof(uint32_t);
// Sink detection keeps its candidate counts and bitmap here between calls when they fit: zero on
// entry, zeroed again after use (the counts by the scan, the bitmap by the compaction or, in the
// step driver, by a later fused launch or a fill).
constexpr size_t kSinkOffset = 256u << 10;
constexpr size_t kSinkAreaBytes = kHeaderBytes - kSinkOffset;
static_assert(kBarrierOffset + (size_t)kMaxSplitSegs * kSyncStride * sizeof(uint32_t) <= kSinkOffset,
              "header too small");

// Optional timing of one launcher call: a and b become the start and end of the launched work
// (for a single-kernel launch, the kernel's own dispatch timestamps).
struct KernelTimer {
  hipEvent_t a, b;
};

// Fused selection for the one-q-head-per-KV-head sparse attention: the attention kernel scores the
// blocks against the predicted queries and selects sinks + top-K itself.
constexpr int kFusedMaxUnits = 4096;   // blocks per head the fused path keeps in LDS
constexpr int kFusedMaxSel = 4096;     // selected blocks per head
constexpr int kFusedMaxSinks = 512;    // sink list entries (one per thread of the fused kernel)
constexpr int kFusedSinkWords = 1024;  // sink bitmap words the fused kernel reads (two per thread)
constexpr int kFusedTaggedUnits = 512; // blocks per head up to which the splits exchange tagged scores
struct FusedSelect {
  const uint64_t* pred_mask;   // [B]
  const float* ks;             // pooled keys [B][H][n_units][D]
  const int32_t* sink_pos;     // [B][max_sinks] or null
  const int32_t* n_sinks;      // [B]
  int max_sinks, top_k;
  float* scores;               // out: [B][H][n_units]
  int32_t* sel_idx;            // out: [B][H][max_sel], ascending
  int32_t* n_sel;              // out: [B][H]
  uint32_t* barriers;          // [B * H][2] split barrier state, left consistent by every launch
  int spin_limit;              // polls before a split stops waiting for its siblings
  float* xchg;                 // grouped-query heads: [B * Hkv * n_splits][n_units] score exchange
                               // of every (KV head, split) group but split 0's (which uses scores)
  // Sinks straight from the detection's bitmap [B][sink_words] (the layer that detected them): the
  // units of the first max_sinks set positions are forced instead of those of sink_pos, and the
  // workgroup of KV head 0, split 0, member 0 of each sequence writes the ascending list (-1 padded)
  // and its length to sink_pos_out / n_sinks_out, latching ST_SINK_OVERFLOW past max_sinks.
  const uint32_t* sink_bitmap;
  int32_t* sink_pos_out;
  int32_t* n_sinks_out;
  // a bitmap nothing reads any more (the detection's, one layer later): the same workgroups zero
  // their sequence's words for the next detection
  uint32_t* clear_bitmap;
  int sink_words;
  uint64_t* stamps;            // phase timestamps [grid][kStampsPerGroup] (FDL_PHASE_STAMPS builds)
  int64_t stamp_words;         // capacity of stamps
  uint32_t serial;             // launch counter of the handle (part of the exchange tag)
};

// Phase timestamps of the fused kernel, written only by a library built with FDL_PHASE_STAMPS:
// thread 0 of every workgroup stores the constant-rate clock (s_memrealtime, 100 MHz) at fixed
// points; slot kStampXcc holds the workgroup's HW_REG_XCC_ID word and its (split, head) ids.
constexpr int kStampsPerGroup = 16;
constexpr int kStampXcc = 15;

struct Geom {
  int B, Hq, Hkv, G, D, L, bt, T, dtype;
  int paged, page_tokens, page_log2, pps, n_pages;
  const int32_t* lens;   // device [B] per-sequence lengths (<= L after clamping), or NULL
};

// Cache write of rows [t0, t0 + n_tok) (K and V) with, when ks != NULL, the pooling of the units
// the write touches (units of 2^unit_log2 >= 16 tokens; longer than 64 tokens through the sub-sum
// scratch `sub`).
hipError_t launch_cache_write(hipStream_t s, const Geom& g, const void* k_new, const void* v_new, int t0, int n_tok,
                              void* k, void* v, const int32_t* page_table, int unit_log2, float* ks, uint32_t* status,
                              float* sub, size_t sub_bytes);

// The unmask update after a step (decoded may be NULL).
hipError_t launch_unmask(hipStream_t s, int batch, int T, const float* conf, uint8_t* masked, int n_unmask,
                         int32_t* decoded);

hipError_t launch_predict(hipStream_t s, int batch, int T, const float* prev_conf,
                          const uint8_t* masked, int top_k, int window, uint64_t* pred_mask,
                          int32_t* n_pred);

// sub / sub_bytes: scratch for the sub-unit sums of units longer than 64 tokens (two passes); with
// too little of it one pass runs.
hipError_t launch_pool_keys(hipStream_t s, const Geom& g, const void* k, const int32_t* page_table,
                            int unit_log2, float* ks, uint32_t* status, float* sub, size_t sub_bytes);

// Per-query (max) unit scores, bf16 queries, dec_len <= 32.
hipError_t launch_score_units_max(hipStream_t s, const Geom& g, const void* q, const uint64_t* pred_mask,
                                  const float* ks, int n_units, float* scores);
hipError_t launch_score_units(hipStream_t s, const Geom& g, const void* q, const uint64_t* pred_mask,
                              const float* ks, int n_units, int unit_log2, float* scores);
// Softmax-mass unit scores, bf16 queries, dec_len <= 32; scratch of mass_scratch_bytes.
size_t mass_scratch_bytes(const Geom& g, int n_units);
hipError_t launch_score_units_mass(hipStream_t s, const Geom& g, const void* q, const uint64_t* pred_mask,
                                   const float* ks, int n_units, int unit_log2, float* scores, char* scratch);

hipError_t launch_score_tokens(hipStream_t s, const Geom& g, const void* q, const uint64_t* pred_mask,
                               const void* k, const int32_t* page_table, int unit_log2,
                               const int32_t* cand_idx, int n_cand, float* scores,
                               uint32_t* status);

// Sink detection.  Needs scratch for per-split statistics, candidates and bitmaps.
size_t sink_scratch_bytes(const Geom& g, int* n_splits, int* cand_cap);
// The prediction inputs, when launch_sinks is the step's first reader of the prediction: it then
// computes the prediction into pred_mask / n_pred (inside the sink scan) instead of reading it.
struct PredictIn {
  const float* conf;       // previous step's confidences [B][T], or NULL (the whole block)
  const uint8_t* masked;   // [B][T]
  int top_k, window;
  uint64_t* pred_mask;     // [B], out
  int32_t* n_pred;         // [B], out
};
hipError_t launch_sinks(hipStream_t s, const Geom& g, const void* q, const uint64_t* pred_mask,
                        const void* k, const void* k_dec, float tau, int max_sinks,
                        int32_t* sink_pos, int32_t* n_sinks, char* scratch, int n_splits,
                        int cand_cap, uint32_t* status, int num_cus, uint32_t* tickets,
                        char* sink_area, uint64_t* stamps, int64_t stamp_words, const PredictIn* pin = nullptr,
                        bool keep_bitmap = false);
// The sink detection's per-sequence bitmap ([B][*words] uint32, one bit per cached token) when the
// detection keeps it in the handle's header (bf16 scan); NULL otherwise.  With keep_bitmap the
// detection ends with the bitmap set and no list: the fused kernel of the same layer then forces the
// units of the first max_sinks set positions, writes the list, and a later launch clears the words.
uint32_t* sink_bitmap_for(const Geom& g, char* sink_area, int* words);

// Level 2 in one kernel (tokens.hip): launch_score_tokens + launch_select with force_first, same
// outputs.  score_select_tokens_ok: the shapes it takes (bf16, dec_len <= 32, units of 256 to 4096
// tokens, pages of at least 16 tokens).
bool score_select_tokens_ok(const Geom& g, int unit_log2);
hipError_t launch_score_select_tokens(hipStream_t s, const Geom& g, const void* q, const uint64_t* pred_mask,
                                      const void* k, const int32_t* page_table, int unit_log2,
                                      const int32_t* cand_idx, int n_cand, int top_k, int max_sel,
                                      float* scores, int32_t* sel_idx, int32_t* n_sel, uint32_t* status);
// Both levels in one launch: level 1 (chunk scores over the chunk sums, top_k_chunks of them
// ascending) inside the level-2 kernel.  select_chunks_tokens_ok adds: at most 8 query heads per KV
// head and 64 chunks per sequence.
bool select_chunks_tokens_ok(const Geom& g, int unit_log2, int n_chunks);
hipError_t launch_select_chunks_tokens(hipStream_t s, const Geom& g, const void* q, const uint64_t* pred_mask,
                                       const float* chunk_sums, const void* k, const int32_t* page_table,
                                       int unit_log2, int top_k_chunks, int top_k, int max_sel, float* chunk_scores,
                                       int32_t* chunks, int32_t* n_chunks_sel, float* scores, int32_t* sel_idx,
                                       int32_t* n_sel, uint32_t* status, uint64_t* stamps = nullptr,
                                       int64_t stamp_words = 0);

hipError_t launch_select(hipStream_t s, const Geom& g, const float* scores, int n_units,
                         int unit_log2, const int32_t* sink_pos, const int32_t* n_sinks,
                         int max_sinks, const int32_t* cand_idx, int n_cand, int top_k,
                         int force_first, int max_sel, int32_t* sel_idx, int32_t* n_sel,
                         uint32_t* status, int shared = 0);

// Token-granular sink retention: selected units + the sink tokens outside them -> ascending token
// list.  expand_tokens_ok: max_sel <= 4096 and max_sinks <= 512.
bool expand_tokens_ok(int max_sel, int max_sinks);
hipError_t launch_expand_tokens(hipStream_t s, const Geom& g, const int32_t* sel_idx, const int32_t* n_sel,
                                int max_sel, int unit_log2, const int32_t* sink_pos, const int32_t* n_sinks,
                                int max_sinks, int32_t* tok_idx, int32_t* n_tok, int max_tok, uint32_t* status);

// Attention.  dense != 0 ignores sel_idx / n_sel.
size_t attn_scratch_bytes(const Geom& g, int n_splits);
hipError_t launch_attn(hipStream_t s, const Geom& g, const void* q, const void* k, const void* v,
                       const void* k_dec, const void* v_dec, const int32_t* page_table,
                       const int32_t* sel_idx, const int32_t* n_sel, int max_sel, int unit_log2,
                       int dense, void* out, char* scratch, int n_splits, uint32_t* tickets,
                       uint32_t* status, int n_hint, const KernelTimer* timer, bool safe = false);

// bf16, any number of query heads per KV head: the LDS-DMA streaming kernel.
int mha_choose_splits(const Geom& g, long long max_list_tokens, int num_cus);
// safe: no workgroup hands data to another through L2 inside the launch (the splits' partials are
// merged by a second launch); otherwise the last split of a head merges them in place.
hipError_t launch_attn_mha(hipStream_t s, const Geom& g, const void* q, const void* k, const void* v,
                           const void* k_dec, const void* v_dec, const int32_t* page_table,
                           const int32_t* sel_idx, const int32_t* n_sel, int max_sel, int unit_log2,
                           int dense, void* out, char* scratch, int n_splits, uint32_t* tickets,
                           uint32_t* status, int n_hint, const KernelTimer* timer,
                           const FusedSelect* fsel = nullptr, bool safe = false);

hipError_t launch_attn_combine(hipStream_t s, const float* part_o, const float2* part_ml, void* out,
                               int n_segs, int n_splits, int T, int D);

hipError_t launch_fill_u32(hipStream_t s, uint32_t* p, size_t n, uint32_t v);

// Streaming-bandwidth probe (probe.hip): mode 0 read into registers, 1 read by LDS DMA, 2 copy,
// 3 the attention kernels' tile pattern.
// Read modes write probe_out_words(n_blocks) checksum words to dst.
size_t probe_out_words(int n_blocks);
// Tiles mode: bytes of K (and of V) each workgroup streams; 0 when the buffer is too small.
size_t probe_tile_region(size_t bytes, int n_blocks);
hipError_t launch_probe(hipStream_t s, int mode, const void* src, size_t bytes, void* dst, int n_blocks);

}  // namespace fdl
