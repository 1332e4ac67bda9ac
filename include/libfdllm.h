/*
 * libfdllm -- one denoising step of confidence-guided, sink-aware block-sparse attention for a
 * diffusion LLM decoding over a long cached bidirectional KV context, on one AMD MI355X (gfx950).
 *
 * Sources (cited by page title and section):
 *   [FA]  "Focus-dLLM: Accelerating Long-Context Diffusion LLM Inference via Confidence-Guided
 *         Context Focusing", the authors' abstract.
 *   [FS]  the same paper, Elamur Research page, "Summary".
 *   [FK]  the same page, "Key points".
 *   [PA]  "Prefilling-dLLM: Predictive Prefilling for Long-Context Inference in Diffusion Language
 *         Models", abstract.
 * The pages give no formulas; the readings this library implements are stated at each call.
 *
 * Conventions shared by every call
 *   - Every tensor pointer is a DEVICE pointer owned by the caller.  fdl_geom lives on the host.
 *   - Layouts are row-major with head_dim innermost:
 *       q, out          [B][Hq][T][D]
 *       contiguous KV   [B][Hkv][L][D]
 *       paged KV pool   [n_pages][Hkv][page_tokens][D], page_table [B][pages_per_seq] int32
 *       k_dec, v_dec    [B][Hkv][T][D]      (the current decode block's own keys / values)
 *     q / k / v / out are bf16 (FDL_BF16, raw 16-bit patterns) or float32 (FDL_F32).
 *   - Every call is asynchronous on the handle's HIP stream and never synchronises the host,
 *     except fdl_get_status and fdl_profile_end.  No call allocates or frees device memory;
 *     fdl_create allocates the one workspace (fdl_capture_end leaves the graph's own resources to
 *     the HIP runtime).  Calls on one handle must come from one host thread at a time, and calls that
 *     share a handle are ordered by its stream (they reuse its workspace).
 *   - Argument errors return FDL_EINVAL (or FDL_EUNSUPPORTED for valid shapes outside the kernel
 *     set, FDL_ENOMEM when the workspace is too small) synchronously, before anything is launched;
 *     outputs are then untouched.  fdl_last_error() describes the last such error.
 *   - Conditions only the device can see (more sinks than max_sinks, more sink candidates than the
 *     workspace holds, an out-of-range page or unit index) are latched into a device status word
 *     and returned by fdl_get_status().
 *   - Workgroups of one head hand scores and partial results to each other through the L2 of the
 *     XCD they run on (workgroup i runs on XCD i mod 8 when the dispatcher assigns workgroups round
 *     robin, and the kernels give a head's workgroups ids of one residue).  That placement is
 *     checked at run time: a score hand-over whose writer ran elsewhere is redone locally
 *     (FDL_FLAG_PLACEMENT), a merge whose inputs are not all on one XCD is not done and reported
 *     (FDL_ESYNC).  With the environment variable FDL_SAFE_SYNC=1 set when a handle is created, no
 *     workgroup hands data to another inside a launch (every split scores every unit, split partials
 *     are merged by a second launch, sink detection runs one workgroup per head): the same results
 *     with no dependence on placement, at some speed.
 *   - A launch failure returns FDL_EHIP.
 */
#ifndef LIBFDLLM_H
#define LIBFDLLM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FDL_OK = 0,
  FDL_EINVAL = -1,
  FDL_ENOMEM = -2,
  FDL_EHIP = -3,
  FDL_EOVERFLOW = -4,
  FDL_EUNSUPPORTED = -5,
  FDL_EINDEX = -6,
  FDL_ESYNC = -7
} fdl_status;

typedef enum { FDL_F32 = 0, FDL_BF16 = 1 } fdl_dtype;

typedef struct fdl_ctx* fdl_handle;

/* Shape of one attention layer.  Limits checked by every call that takes it:
 *   batch >= 1; n_kv_heads >= 1; n_q_heads = G * n_kv_heads with 1 <= G <= 8;
 *   head_dim in {64, 128}; ctx_len >= 0; kv_block a power of two in [1, 4096];
 *   1 <= dec_len <= 64 (<= 32 for FDL_BF16 attention);
 *   paged: page_tokens a power of two in [1, 4096], pages_per_seq * page_tokens >= ctx_len,
 *   n_pages >= 1.
 * Ragged batches ([FK]: the contexts of a batch need not be equally long): ctx_lens, when not NULL,
 * is a DEVICE int32 array [batch] of per-sequence cached-token counts; sequence b then has
 * L_b = clamp(ctx_lens[b], 0, ctx_len) tokens, stored in the first L_b rows of its ctx_len-row
 * stride of the contiguous cache ([B][Hkv][ctx_len][D]).  Every per-sequence quantity follows L_b:
 * its units are the ceil(L_b / unit) units of its own tokens (the last one partial when L_b is not a
 * multiple of the unit, pooled over its valid tokens), the units past them have pooled keys +0,
 * score +0 and are never selected, sink detection and dense attention cover [0, L_b), and a unit
 * id at or past a sequence's units is out of range (FDL_EINDEX).  Taken by the pooling, scoring,
 * sink, selection (level 1), attention and step calls on contiguous caches; the other calls (paged
 * caches, level 2, the max / mass scorers, token expansion, cache write) return FDL_EUNSUPPORTED
 * with a non-NULL ctx_lens. */
typedef struct {
  int32_t batch;          /* B   sequences                                   */
  int32_t n_q_heads;      /* Hq  query heads                                 */
  int32_t n_kv_heads;     /* Hkv key/value heads (Hq / Hkv query heads each) */
  int32_t head_dim;       /* D                                               */
  int32_t ctx_len;        /* L   cached context tokens per sequence          */
  int32_t kv_block;       /* tokens per KV block (the selection unit)        */
  int32_t dec_len;        /* T   tokens of the current decode block          */
  int32_t dtype;          /* fdl_dtype of q, KV and out                      */
  int32_t paged;          /* 0: contiguous KV; 1: paged pool + page table    */
  int32_t page_tokens;    /* paged: tokens per page                          */
  int32_t pages_per_seq;  /* paged: page-table row length                    */
  int32_t n_pages;        /* paged: physical pages in the pool               */
  const int32_t* ctx_lens;  /* device [batch] per-sequence lengths, or NULL   */
} fdl_geom;

/* ---- handle ------------------------------------------------------------------------------ */

/* Create a handle bound to the current HIP device and to `hip_stream` (a hipStream_t; NULL = the
 * null stream).  Allocates a device workspace of `workspace_bytes` (0 = 64 MiB), zeroes its
 * counters and synchronises once.  Returns FDL_ENOMEM if the allocation fails. */
fdl_status fdl_create(fdl_handle* h, void* hip_stream, size_t workspace_bytes);
fdl_status fdl_destroy(fdl_handle h);
fdl_status fdl_set_stream(fdl_handle h, void* hip_stream);

/* Synchronise the handle's stream, return the first latched device condition (FDL_EOVERFLOW,
 * FDL_EINDEX) or FDL_OK, and clear it. */
fdl_status fdl_get_status(fdl_handle h);

/* Device condition bits, as latched by the kernels. */
#define FDL_FLAG_SINK_OVERFLOW 1u   /* more sinks than max_sinks: list truncated (FDL_EOVERFLOW)     */
#define FDL_FLAG_CAND_OVERFLOW 2u   /* more sink candidates than the workspace holds (FDL_EOVERFLOW) */
#define FDL_FLAG_BAD_INDEX 4u       /* unit or page id out of range: row skipped, not read or       */
                                    /* written, +0 in a key sum (FDL_EINDEX)                         */
#define FDL_FLAG_SEL_OVERFLOW 8u    /* more selected units than max_sel: list truncated (EOVERFLOW) */
#define FDL_FLAG_SPLIT_FALLBACK 16u /* informational: a split of fdl_focus_step's fused kernel did  */
                                    /* not wait for its siblings and scored every block itself;     */
                                    /* results are unaffected (FDL_OK)                               */
#define FDL_FLAG_PLACEMENT 32u      /* informational: a split of that kernel found a sibling on     */
                                    /* another XCD (no shared L2) and scored that sibling's blocks  */
                                    /* itself; results are unaffected (FDL_OK)                       */
#define FDL_FLAG_SPLIT_PLACEMENT 64u /* the workgroups of a head that merge partial results through */
                                    /* one XCD's L2 ran on different XCDs: that head's attention    */
                                    /* output (or sink list) was not written (FDL_ESYNC)            */

/* Like fdl_get_status, but also stores the raw condition bits (FDL_FLAG_*) in *bits (may be NULL)
 * before clearing them. */
fdl_status fdl_get_status_bits(fdl_handle h, uint32_t* bits);
const char* fdl_status_string(fdl_status s);
const char* fdl_last_error(fdl_handle h);

/* ---- cache side: pooled keys ---------------------------------------------------------------- */

/* Sum the keys of every `unit_tokens`-token unit (a KV block, or a prefix chunk) in float32, in the
 * pinned order: an adjacent-pair tree over the unit's tokens in logical order, zero-padded to a
 * power of two (tokens >= ctx_len count as +0).  Reading of [FS]/[FA] ("predicted queries select
 * the most relevant KV": units are represented by their key sums) and [PA] (chunks are cached once).
 *   k_cache     contiguous or paged keys (per g->paged); page_table used when paged, else ignored
 *   unit_tokens power of two in [1, 4096]
 *   ks          out: [B][Hkv][ceil(L / unit_tokens)][D] float32
 * A paged row whose page id lies outside [0, n_pages) counts +0 and latches FDL_EINDEX. */
fdl_status fdl_pool_keys(fdl_handle h, const fdl_geom* g, const void* k_cache,
                         const int32_t* page_table, int32_t unit_tokens, float* ks);

/* Cache side, written and pooled in one pass (no rereading of the written keys).  [FA] the context
 * cache is built once and reused, and the block scoring ranks units by their pooled keys; [PA] the
 * cache may be paged.  Reading: the write replaces the logical rows [t0, t0 + n_tok) of every
 * (sequence, KV head) with k_new / v_new [B][Hkv][n_tok][D] (g->dtype), bit for bit, in the
 * contiguous cache [B][Hkv][L][D] or, when g->paged, in the page pool through page_table; when ks
 * is not NULL, every unit of unit_tokens tokens that holds a written row gets the pooled key of the
 * updated cache (the same tree as fdl_pool_keys), and the other units of ks [B][Hkv][n_units][D] are
 * left as they are.  Requires 0 <= t0, n_tok >= 1, t0 + n_tok <= L and, with ks, unit_tokens a power
 * of two in [16, 4096]; units longer than 64 tokens use workspace scratch (B * Hkv * ceil(L / 64) * D
 * floats; FDL_ENOMEM if the workspace is smaller).  A row whose page id lies outside [0, n_pages)
 * has no place in the pool: it is not written (no page is touched for it), it counts +0 in the
 * pooled keys of its unit, and FDL_EINDEX is latched. */
fdl_status fdl_cache_write(fdl_handle h, const fdl_geom* g, const void* k_new, const void* v_new, int32_t t0,
                           int32_t n_tok, void* k_cache, void* v_cache, const int32_t* page_table,
                           int32_t unit_tokens, float* ks);

/* ---- step 1: past-confidence-guided query prediction ----------------------------------------- */

/* [FA], [FS], [FK]: the previous step's confidence predicts the next positions to be unmasked; the
 * top `top_k` still-masked positions (confidence descending, NaN lowest, ties to the lower position)
 * are widened to [i - window, i + window] clipped to [0, dec_len), and their union is the predicted
 * query set.  prev_conf == NULL (first step of a block) predicts every position; no masked position
 * predicts none.
 *   prev_conf [batch][dec_len] float32 or NULL;  masked [batch][dec_len] uint8 (non-zero = masked)
 *   pred_mask out [batch] uint64 (bit p = position p predicted);  n_pred out [batch] int32
 *   1 <= dec_len <= 64, top_k >= 0, window >= 0 */
fdl_status fdl_predict_queries(fdl_handle h, int32_t batch, int32_t dec_len, const float* prev_conf,
                               const uint8_t* masked, int32_t top_k, int32_t window,
                               uint64_t* pred_mask, int32_t* n_pred);

/* ---- step 2: score KV units against the predicted queries; detect sinks ---------------------- */

/* [FA], [FS]: the predicted queries estimate which KV matters.  Reading: per KV head g, the
 * predicted queries of its q-head group are summed in float32 (adjacent-pair tree over the dec_len
 * slots, non-predicted slots +0, then over the group's heads padded to a power of two); a unit's
 * score is the pinned float32 dot product of that sum with the unit's key sum (products rounded,
 * no fused multiply-add, adjacent-pair tree over D).
 *
 * Level 1 (cand_idx == NULL): scores [B][Hkv][n_units] from `ks` (fdl_pool_keys output with the
 *   same unit_tokens), n_units = ceil(L / unit_tokens).
 * Level 2 (cand_idx != NULL, [PA] token sparsity inside the chosen chunks): cand_idx
 *   [B][Hkv][n_cand] ascending unit ids (e.g. fdl_select_blocks level-1 output); every token of
 *   every candidate unit is scored against its own key from k_cache (paged through page_table if
 *   g->paged): scores [B][Hkv][n_cand][unit_tokens]; requires L % unit_tokens == 0.
 *
 * detect_sinks != 0 (level 1 only; the source layer): [FA], [FS], [FK] attention sinks.  Reading:
 *   for every q-head and predicted position p, softmax(q_p . k_t / sqrt(D)) over all L cached
 *   tokens and the block's dec_len own tokens (k_dec); a cached token whose mean weight over the
 *   predicted positions reaches sink_tau for at least one q-head is a sink.  The union over heads is
 *   written ascending to sink_pos [B][max_sinks] int32 with the count in n_sinks [B]; more than
 *   max_sinks sinks keeps the first max_sinks and latches FDL_EOVERFLOW.  Reads all of k_cache
 *   (contiguous only).  sink_tau > 0.  With detect_sinks == 0, k_cache / k_dec / sink_* may be
 *   NULL (level 1) and previously detected sinks are reused by fdl_select_blocks. */
fdl_status fdl_score_blocks(fdl_handle h, const fdl_geom* g, const void* q, const uint64_t* pred_mask,
                            const float* ks, int32_t unit_tokens, const int32_t* cand_idx,
                            int32_t n_cand, const void* k_cache, const void* k_dec,
                            const int32_t* page_table, float* scores, int32_t detect_sinks,
                            float sink_tau, int32_t max_sinks, int32_t* sink_pos, int32_t* n_sinks);

/* Per-query scoring, a reading the pages leave open next to the summed-query one of
 * fdl_score_blocks (level 1): a unit's score is the largest pinned float32 dot product of one
 * predicted query of the KV head's q-head group with the unit's key sum (same dot product tree as
 * fdl_score_blocks), so a unit that matters to any single predicted position ranks high; +0 when no
 * position is predicted, and a -0 result is written as +0.  scores [B][Hkv][n_units] from ks
 * (fdl_pool_keys output with the same unit_tokens).  bf16 queries with dec_len <= 32 only
 * (FDL_EUNSUPPORTED otherwise).  Its scores go to fdl_select_blocks like those of fdl_score_blocks. */
fdl_status fdl_score_blocks_max(fdl_handle h, const fdl_geom* g, const void* q, const uint64_t* pred_mask,
                                const float* ks, int32_t unit_tokens, float* scores);

/* Softmax-mass scoring, a third reading of how the predicted queries estimate attention
 * importance ([FA] Elamur "Summary"): every predicted query of the KV head's q-head group attends to
 * the units' mean keys (ks / valid tokens of the unit; a partial last unit counts its valid tokens)
 * with the scale 1/sqrt(head_dim), a softmax over the head's units; a unit's score is the
 * probability mass it receives summed over those queries (zeros when nothing is predicted, so each
 * head's scores sum to G * |predicted positions|).  float32 arithmetic with expf: scores agree with
 * a float64 evaluation to rounding, and units whose masses differ by less than that may rank
 * either way.  scores [B][Hkv][n_units] from ks (fdl_pool_keys output with the same unit_tokens).
 * bf16 queries with dec_len <= 32 only (FDL_EUNSUPPORTED otherwise); uses
 * B * Hkv * G * dec_len * (4 * n_units + 8) bytes of workspace (FDL_ENOMEM beyond it).  Its
 * scores go to fdl_select_blocks like those of fdl_score_blocks. */
fdl_status fdl_score_blocks_mass(fdl_handle h, const fdl_geom* g, const void* q, const uint64_t* pred_mask,
                                 const float* ks, int32_t unit_tokens, float* scores);

/* ---- step 3: keep sinks + top-K units; reuse sinks across layers ---------------------------- */

/* [FA], [FS]: sinks are always kept and their locations are reused in deeper layers; the rest of
 * the budget goes to the best-scoring units.  Ranking: score descending, -0 == +0, NaN lowest,
 * ties to the lower index.  Output ascending.
 *
 * Level 1 (cand_idx == NULL): scores [B][Hkv][n_units]; every unit holding a sink position
 *   (sink_pos[b][0 .. n_sinks[b]) / unit_tokens; sink_pos may be NULL for none) is forced in, plus
 *   the top `top_k` of the other units.  sel_idx [B][Hkv][max_sel] gets the unit ids, n_sel
 *   [B][Hkv] the count (= forced + min(top_k, n_units - forced)).  Passing the source layer's
 *   sink_pos / n_sinks unchanged is the cross-layer reuse.  max_sel must cover min(n_units,
 *   max_sinks + top_k); max_sinks bounds n_sinks.
 * Level 2 ([PA]; cand_idx != NULL): scores [B][Hkv][n_cand][unit_tokens] (fdl_score_blocks level 2);
 *   inside each candidate unit, token 0 (the chunk's leading BOS anchor) is forced when
 *   force_first != 0, plus the top `top_k` of its other tokens; sel_idx [B][Hkv][max_sel] gets the
 *   logical token ids (cand * unit_tokens + i), ascending; n_sel = n_cand * (force_first + top_k);
 *   requires top_k <= unit_tokens - force_first and max_sel >= that count. */
fdl_status fdl_select_blocks(fdl_handle h, const fdl_geom* g, const float* scores, int32_t n_units,
                             int32_t unit_tokens, const int32_t* sink_pos, const int32_t* n_sinks,
                             int32_t max_sinks, const int32_t* cand_idx, int32_t n_cand,
                             int32_t top_k, int32_t force_first, int32_t max_sel, int32_t* sel_idx,
                             int32_t* n_sel);

/* Level 1 with one selection per sequence, the other reading of [PA]'s "top-K most relevant chunks"
 * (per KV head above): unit i ranks by its scores summed over the sequence's KV heads (float32
 * adjacent-pair tree over the heads in head order, zero-padded), with the same forced units, ranking
 * and count as fdl_select_blocks level 1; every head's row of sel_idx / n_sel gets the same list.
 * n_kv_heads <= 32 (FDL_EUNSUPPORTED beyond); arguments and errors as fdl_select_blocks level 1. */
fdl_status fdl_select_blocks_shared(fdl_handle h, const fdl_geom* g, const float* scores, int32_t n_units,
                                    int32_t unit_tokens, const int32_t* sink_pos, const int32_t* n_sinks,
                                    int32_t max_sinks, int32_t top_k, int32_t max_sel, int32_t* sel_idx,
                                    int32_t* n_sel);

/* [PA] level 2 in one call: fdl_score_blocks at level 2 (token scores inside the n_cand candidate
 * units, written to scores [B][Hkv][n_cand][unit_tokens]) followed by fdl_select_blocks at level 2
 * with force_first = 1 (each unit's token 0 forced, plus the top `top_k` of its other tokens) --
 * the same scores, sel_idx [B][Hkv][max_sel] and n_sel [B][Hkv], bit for bit.  For bf16, dec_len <=
 * 32, units of 256 to 4096 tokens and pages of at least 16 tokens it runs as one kernel (scores and
 * selection without a round trip through memory); otherwise as the two calls.  Requirements are
 * those of the two calls: L % unit_tokens == 0, n_cand in [1, n_units], top_k <= unit_tokens - 1,
 * max_sel >= n_cand * (1 + top_k).  Out-of-range candidate units and page ids latch FDL_EINDEX (the
 * unit's selection is then -1s). */
fdl_status fdl_score_select_tokens(fdl_handle h, const fdl_geom* g, const void* q, const uint64_t* pred_mask,
                                   const void* k_cache, const int32_t* page_table, int32_t unit_tokens,
                                   const int32_t* cand_idx, int32_t n_cand, int32_t top_k, int32_t max_sel,
                                   float* scores, int32_t* sel_idx, int32_t* n_sel);

/* [PA] both levels of the chunked selection in one launch: the top-K chunks per (sequence, KV head),
 * then inside each the anchor plus the top `top_k` other tokens.  The same outputs, bit for bit, as
 *   fdl_score_blocks (level 1: chunk_sums [B][Hkv][n_chunks][D] float32 from fdl_pool_keys with
 *     unit_tokens = chunk_tokens, scores to chunk_scores [B][Hkv][n_chunks]),
 *   fdl_select_blocks (level 1, no sinks, top_k = max_sel = top_k_chunks: the chosen chunks
 *     ascending in chunks [B][Hkv][top_k_chunks], their count in n_chunks_sel [B][Hkv]),
 *   fdl_score_select_tokens (cand_idx = chunks, n_cand = top_k_chunks; token_scores
 *     [B][Hkv][top_k_chunks][chunk_tokens], sel_idx [B][Hkv][max_sel], n_sel [B][Hkv]),
 * with n_chunks = ctx_len / chunk_tokens.  Requirements: those of the three calls, plus bf16,
 * dec_len <= 32, chunks of 256 to 4096 tokens, pages of at least 16 tokens, at most 8 query heads
 * per KV head, n_chunks <= 64 and 1 <= top_k_chunks <= n_chunks (FDL_EUNSUPPORTED for a shape
 * outside them, FDL_EINVAL for bad arguments).  Out-of-range page ids latch FDL_EINDEX. */
fdl_status fdl_select_chunks_tokens(fdl_handle h, const fdl_geom* g, const void* q, const uint64_t* pred_mask,
                                    const float* chunk_sums, const void* k_cache, const int32_t* page_table,
                                    int32_t chunk_tokens, int32_t top_k_chunks, int32_t top_k, int32_t max_sel,
                                    float* chunk_scores, int32_t* chunks, int32_t* n_chunks_sel,
                                    float* token_scores, int32_t* sel_idx, int32_t* n_sel);

/* Token-granular sink retention, the other reading of how sinks are kept ([FA] Elamur "Summary":
 * sinks are always preserved; at which granularity is left open): select the units with
 * fdl_select_blocks level 1 WITHOUT sinks (so the top-K comes from all units), then this call
 * writes, per (sequence, KV head), the ascending list of the selected units' valid tokens merged
 * with the sink tokens sink_pos[b][0 .. n_sinks[b]) that lie outside those units (each token once;
 * positions outside [0, ctx_len) are dropped): tok_idx [B][Hkv][max_tok], n_tok [B][Hkv].  Feed the
 * list to fdl_sparse_attn with sel_unit_tokens = 1.  sel_idx [B][Hkv][max_sel] ascending unit ids
 * (out-of-range ids latch FDL_EINDEX and contribute nothing), n_sel [B][Hkv]; sink_pos / n_sinks
 * may both be NULL.  max_sel <= 4096 and max_sinks <= 512 (FDL_EUNSUPPORTED beyond); max_tok >=
 * max_sel * unit_tokens + max_sinks (FDL_EINVAL otherwise). */
fdl_status fdl_expand_tokens(fdl_handle h, const fdl_geom* g, const int32_t* sel_idx, const int32_t* n_sel,
                             int32_t max_sel, int32_t unit_tokens, const int32_t* sink_pos, const int32_t* n_sinks,
                             int32_t max_sinks, int32_t* tok_idx, int32_t* n_tok, int32_t max_tok);

/* ---- step 4: sparse bidirectional attention over the selected KV ---------------------------- */

/* [FA], [FS]: bidirectional attention of the current block's queries over only the selected KV;
 * [PA]: over chunk KV cached non-contiguously.  For every q-head h (KV head h / G) and every one of
 * the dec_len queries: out = softmax(q . k / sqrt(D)) v over the selected cached tokens plus the
 * block's own dec_len tokens (k_dec / v_dec), no mask.  The selected tokens are the units
 * sel_idx[b][g][0 .. n_sel[b][g]) of sel_unit_tokens tokens each (kv_block for blocks, 1 for token
 * lists); tokens >= ctx_len are skipped; paged KV is resolved through page_table.  bf16 runs on
 * MFMA with float32 accumulation and bf16 output; float32 runs in float32.
 * Unit ids outside [0, ceil(L / sel_unit_tokens)) and page ids outside [0, n_pages) are skipped
 * and latch FDL_EINDEX. */
fdl_status fdl_sparse_attn(fdl_handle h, const fdl_geom* g, const void* q, const void* k_cache,
                           const void* v_cache, const void* k_dec, const void* v_dec,
                           const int32_t* page_table, const int32_t* sel_idx, const int32_t* n_sel,
                           int32_t max_sel, int32_t sel_unit_tokens, void* out);

/* fdl_sparse_attn for callers that cannot allocate device memory -- code under HIP-graph capture,
 * tight serving loops, harnesses that forbid hipMalloc -- and so hold no handle: the same attention,
 * arguments and results (the same split count as fdl_sparse_attn with the default workspace, so the
 * outputs are bit for bit those of fdl_sparse_attn on a handle created with workspace_bytes = 0),
 * launched on `hip_stream` (a hipStream_t; NULL = the null stream) with no allocation of any kind.
 * The split partials, merge counters and a status word live in a static device array of 8 MiB that
 * each GPU the library runs on holds until the process ends; every call on a GPU shares that GPU's
 * array, so calls that overlap on one GPU (two streams, two threads) race and must be ordered by the
 * caller.  `status` (a device uint32, may be NULL) has FDL_FLAG_* bits OR-ed into it for the
 * device-side conditions (out-of-range unit or page ids, skipped); with NULL they are not reported.
 * Argument errors return FDL_EINVAL / FDL_EUNSUPPORTED as fdl_sparse_attn (no message: there is no
 * handle for fdl_last_error); FDL_ENOMEM when the split partials would exceed the static array. */
fdl_status fdl_sparse_attn_noalloc(void* hip_stream, const fdl_geom* g, const void* q, const void* k_cache,
                                   const void* v_cache, const void* k_dec, const void* v_dec,
                                   const int32_t* page_table, const int32_t* sel_idx, const int32_t* n_sel,
                                   int32_t max_sel, int32_t sel_unit_tokens, void* out, uint32_t* status);

/* Dense baseline and the shallow full-attention layers ([FS]): the same attention over all L cached
 * tokens plus the own block. */
fdl_status fdl_dense_attn(fdl_handle h, const fdl_geom* g, const void* q, const void* k_cache,
                          const void* v_cache, const void* k_dec, const void* v_dec,
                          const int32_t* page_table, void* out);


/* ---- a whole denoising step over a stack of layers ------------------------------------------ */

/* [FS]: shallow layers keep full attention; one source layer finds the sinks that deeper layers
 * reuse.  fdl_focus_step runs one denoising step over `n_layers` layers with a single host call:
 * fdl_predict_queries once, then per layer, by mode,
 *   FDL_LAYER_DENSE : fdl_dense_attn;
 *   FDL_LAYER_SOURCE: fdl_score_blocks with sink detection, fdl_select_blocks, fdl_sparse_attn;
 *   FDL_LAYER_REUSE : fdl_score_blocks, fdl_select_blocks with the current sink_pos / n_sinks
 *                     (those of the last source layer; on entry, whatever they hold), fdl_sparse_attn.
 * Scores, sinks and selections are identical to issuing those calls one by one, and outputs agree
 * with theirs to rounding: for bf16 contiguous caches of up to 4096 blocks the scoring, selection
 * and attention of a sparse layer run as one kernel, whose splits sum the tiles in another order.
 * When the first layer that is not dense is a source layer, the prediction is computed inside its
 * sink detection, and (bf16, sink bitmap in the handle's header) that layer's fused kernel turns the
 * detection's bitmap into sink_pos / n_sinks itself: two launches fewer, the same values.
 * Only launches are issued (no host synchronisation).  Each layer's KV is contiguous (g->paged == 0), its `ks` is the fdl_pool_keys
 * output with unit kv_block.  scores [B][Hkv][n_blk], sel_idx [B][Hkv][max_sel] and n_sel [B][Hkv]
 * are scratch reused layer to layer and hold the last sparse layer's values on return;
 * pred_mask / n_pred / sink_pos / n_sinks hold the step's.  max_sel must cover
 * min(n_blk, max_sinks + top_k_blocks). */
typedef enum { FDL_LAYER_DENSE = 0, FDL_LAYER_SOURCE = 1, FDL_LAYER_REUSE = 2 } fdl_layer_mode;

typedef struct {
  const void* q;        /* [B][Hq][T][D]   */
  const void* k_cache;  /* [B][Hkv][L][D]  */
  const void* v_cache;
  const void* k_dec;    /* [B][Hkv][T][D]  */
  const void* v_dec;
  const float* ks;      /* [B][Hkv][n_blk][D] pooled keys (ignored by dense layers) */
  void* out;            /* [B][Hq][T][D]   */
  int32_t mode;         /* fdl_layer_mode  */
} fdl_layer_io;

typedef struct {
  int32_t top_k_pos;     /* predictor: positions taken from the previous confidence */
  int32_t window;        /* predictor: +/- widening                                   */
  int32_t top_k_blocks;  /* non-sink blocks kept per KV head                          */
  int32_t max_sinks;     /* capacity of sink_pos                                       */
  int32_t max_sel;       /* capacity of sel_idx                                        */
  float sink_tau;        /* sink threshold (> 0)                                       */
} fdl_focus_params;

fdl_status fdl_focus_step(fdl_handle h, const fdl_geom* g, const fdl_focus_params* p,
                          const float* prev_conf, const uint8_t* masked, int32_t n_layers,
                          const fdl_layer_io* layers, uint64_t* pred_mask, int32_t* n_pred,
                          float* scores, int32_t* sink_pos, int32_t* n_sinks, int32_t* sel_idx,
                          int32_t* n_sel);

/* ---- the step after the path: the unmask update and the denoising loop ----------------------- */

/* [FA] Elamur "Summary": a block is decoded by denoising its masked positions step after step;
 * "Key points": the tokens a step decodes are the highest-confidence ones still masked, one position
 * per step at generation length = steps.  Reading: after a step, the n_unmask masked positions of
 * each sequence with the highest confidence conf[b] are decoded, ranked as fdl_predict_queries
 * ranks (ties to the lower position, NaN below every number, -0 == +0).
 *   conf    [batch][dec_len] float32, device, read only at masked positions.
 *   masked  [batch][dec_len] uint8, device, updated in place: decoded positions become 0.
 *   decoded [batch][n_unmask] int32, device, may be NULL: the decoded positions in rank order, -1
 *           past the number decoded (fewer masked positions than n_unmask: all of them).
 * 1 <= dec_len <= 64; 0 <= n_unmask <= 64.  FDL_EINVAL otherwise, before any launch. */
fdl_status fdl_unmask(fdl_handle h, int32_t batch, int32_t dec_len, const float* conf, uint8_t* masked,
                      int32_t n_unmask, int32_t* decoded);

/* n_steps denoising steps of one decode block with no host round trip: step s is fdl_focus_step
 * with prev_conf = (s == 0 ? prev_conf0 : conf + (s - 1) * B * T), the current masked flags and the
 * layer table layers + s * n_layers, followed by fdl_unmask(conf + s * B * T, masked, n_unmask,
 * decoded ? decoded + s * B * n_unmask : NULL).  conf [n_steps][B][T] holds the confidence each
 * step produces (supplied by the caller: the model's head is not part of this library);
 * prev_conf0 may be NULL (the first step of a block).  The other arguments are fdl_focus_step's and
 * hold the last step's values on return.  Every step's arguments are validated before anything is
 * launched.  Together with fdl_capture_begin / fdl_capture_end, a whole block (or a whole run of
 * blocks) becomes one graph launch. */
fdl_status fdl_decode_steps(fdl_handle h, const fdl_geom* g, const fdl_focus_params* p, int32_t n_steps,
                            const float* prev_conf0, const float* conf, uint8_t* masked, int32_t n_unmask,
                            int32_t* decoded, int32_t n_layers, const fdl_layer_io* layers,
                            uint64_t* pred_mask, int32_t* n_pred, float* scores, int32_t* sink_pos,
                            int32_t* n_sinks, int32_t* sel_idx, int32_t* n_sel);

/* HIP-graph capture of the launches issued on the handle's stream.  fdl_capture_begin starts
 * capturing that stream (not the null stream; not while profiling); every library call until
 * fdl_capture_end is recorded instead of run (argument errors are still reported at once, and a
 * call that failed records nothing).  fdl_capture_end ends the capture and instantiates the graph;
 * fdl_graph_launch replays it on the handle's stream, with the pointers and scalars of the captured
 * calls; fdl_graph_destroy releases it.  The library's launches record no memset node.  While
 * capturing, fdl_get_status, fdl_profile_* and switching the stream fail with FDL_EINVAL.  A graph
 * holds driver resources (allocated by the HIP runtime at fdl_capture_end) until it is destroyed;
 * replays that share a handle are ordered by its stream, like any other calls on it. */
typedef struct fdl_graph_s* fdl_graph;
fdl_status fdl_capture_begin(fdl_handle h);
fdl_status fdl_capture_end(fdl_handle h, fdl_graph* graph);
fdl_status fdl_graph_launch(fdl_handle h, fdl_graph graph);
fdl_status fdl_graph_destroy(fdl_graph graph);

/* ---- timing --------------------------------------------------------------------------------- */

/* Optional per-call timing with HIP events on the handle's stream, for the launches of the kinds
 * below (and whole layers inside fdl_focus_step) whose bit (1 << kind) is set in kind_mask.
 * Attention launches carry the events in the kernel dispatch itself (start and end of the kernel);
 * the other kinds are bracketed by event records.  Only every `every`-th launch of a kind is timed
 * (every >= 1), which keeps the cost of the events -- a few microseconds each -- out of a timed
 * run.  fdl_profile_begin creates a pool of 2 * max_records events and clears the records;
 * fdl_profile_end synchronises, writes the summed duration in microseconds and the number of timed
 * launches of every kind into total_us[FDL_PROF_KINDS] / counts[FDL_PROF_KINDS] and releases the
 * pool.  Records beyond max_records are dropped.  FDL_PROF_REUSE_RUN brackets each run of
 * consecutive reuse layers of fdl_focus_step with one pair of events and counts the layers of the
 * run, so total / count is the stream time per reuse layer (kernel plus the gap to the next). */
typedef enum {
  FDL_PROF_PREDICT = 0, FDL_PROF_POOL, FDL_PROF_SCORE, FDL_PROF_SINKS, FDL_PROF_SELECT,
  FDL_PROF_SPARSE_ATTN, FDL_PROF_DENSE_ATTN, FDL_PROF_LAYER_DENSE, FDL_PROF_LAYER_SOURCE,
  FDL_PROF_LAYER_REUSE, FDL_PROF_REUSE_RUN, FDL_PROF_KINDS
} fdl_prof_kind;

fdl_status fdl_profile_begin(fdl_handle h, int32_t max_records, uint32_t kind_mask, int32_t every);
fdl_status fdl_profile_end(fdl_handle h, double* total_us, int64_t* counts);

/* Diagnostic phase timeline of the fused score-select-attend kernel of fdl_focus_step.  Only a
 * library built with FDL_PHASE_STAMPS defined (python -m diffusion_long_context_amd.build
 * --phase-stamps) records anything; fdl_phase_stamps_built() tells which build is loaded.  With a
 * buffer set (stamps: device uint64 array of n_words; NULL and 0 to unset), every later fused launch
 * on the handle with at most n_words / 16 workgroups has thread 0 of workgroup w store the
 * 100 MHz constant clock at stamps[16 w + i] as it passes point i: 0 start, 1 predicted-query sum
 * done, 2 own block scores written, 3 the splits' score exchange done, 4 all scores read back,
 * 5 selection done, 6 first tile landed, 7 wave 0's tiles done, 8 all waves' tiles done, 9 merge
 * ticket taken, 10 merge done (the last split of a head only); stamps[16 w + 15] = the XCD-id register
 * (bits 0-31) | split << 32 | head << 40 | 1 << 63.  Each launch overwrites the previous one's stamps. */
fdl_status fdl_set_phase_buffer(fdl_handle h, uint64_t* stamps, int64_t n_words);
int32_t fdl_phase_stamps_built(void);

/* Measurement aid, not part of the method: stream `bytes` (a positive multiple of 1024) of the
 * device buffer `src` once, the way the HBM-bound kernels stream their inputs, so that their rate
 * can be set against what the memory system delivers to a plain coalesced stream as well as against
 * the vendor peak.  FDL_PROBE_READ: 16-byte non-temporal loads into registers, eight in flight per
 * thread; FDL_PROBE_READ_LDS: 1 KiB fetches straight into LDS (global_load_lds_dwordx4), eight in
 * flight per wave; both write one xor checksum word per wave to dst (n_blocks * 8 uint32,
 * dst_bytes at least that).  FDL_PROBE_COPY: the same read stream written to dst (dst_bytes >= bytes).
 * FDL_PROBE_TILES: the attention kernels' own pattern -- the first half of src stands for K, the
 * second for V, each workgroup streams a region of each of bytes / 2 / n_blocks (rounded down to
 * 8 KiB; EINVAL if that is 0) as 16 KiB K + V tiles into LDS, one tile in flight per wave; only
 * 16 KiB * (tiles actually read) count, and the checksum goes to dst as for the read modes.
 * n_blocks workgroups of 512 threads (0 = four per compute unit; one per compute unit for
 * FDL_PROBE_TILES).  Asynchronous on the handle's stream; time it with events around the call. */
typedef enum { FDL_PROBE_READ = 0, FDL_PROBE_READ_LDS = 1, FDL_PROBE_COPY = 2, FDL_PROBE_TILES = 3 } fdl_probe_mode;
fdl_status fdl_bandwidth_probe(fdl_handle h, int32_t mode, const void* src, size_t bytes, void* dst,
                               size_t dst_bytes, int32_t n_blocks);

#ifdef __cplusplus
}
#endif

#endif /* LIBFDLLM_H */
