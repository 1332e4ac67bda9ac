// libfdllm C ABI: argument validation, the handle and its workspace, and kernel launches.
// Every check happens on the host before anything is launched; device-side conditions are latched
// into the handle's status word.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <new>

#include "fdl_device.h"
#include "fdl_internal.h"

using fdl::Geom;

namespace {

fdl_status fail(fdl_handle h, fdl_status s, const char* fmt, ...) {
  if (h) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(h->last_error, sizeof(h->last_error), fmt, ap);
    va_end(ap);
  }
  return s;
}

fdl_status hip_status(fdl_handle h, hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(h, FDL_EHIP, "%s: %s", what, hipGetErrorString(e));
#ifdef FDL_DEBUG
  // Debug build: every launch is waited for at once, so that a failing kernel is reported by the
  // call that launched it, and a change of the status word is printed with the launch that made it.
  // (Not for streams that the caller captures into a graph: the wait would end the capture.)
  if (h && !h->capturing) {
    const hipError_t w = hipStreamSynchronize(h->stream);
    if (w != hipSuccess) return fail(h, FDL_EHIP, "%s (debug wait): %s", what, hipGetErrorString(w));
    uint32_t word = 0;
    if (hipMemcpy(&word, h->status, sizeof(word), hipMemcpyDeviceToHost) == hipSuccess && word != h->debug_seen) {
      fprintf(stderr, "libfdllm debug: after %s the status word is 0x%x\n", what, word);
      h->debug_seen = word;
    }
  }
#endif
  return FDL_OK;
}

bool is_pow2(long long x) { return x > 0 && (x & (x - 1)) == 0; }

int ilog2(long long x) {
  int l = 0;
  while ((1LL << l) < x) ++l;
  return l;
}

fdl_status check_geom(fdl_handle h, const fdl_geom* g, Geom& o) {
  if (!g) return fail(h, FDL_EINVAL, "geom is NULL");
  if (g->batch < 1) return fail(h, FDL_EINVAL, "batch must be >= 1");
  if (g->n_kv_heads < 1 || g->n_q_heads < g->n_kv_heads || g->n_q_heads % g->n_kv_heads)
    return fail(h, FDL_EINVAL, "n_q_heads must be a positive multiple of n_kv_heads");
  if (g->n_q_heads / g->n_kv_heads > 8)
    return fail(h, FDL_EUNSUPPORTED, "more than 8 query heads per KV head");
  if (g->head_dim != 64 && g->head_dim != 128)
    return fail(h, FDL_EUNSUPPORTED, "head_dim must be 64 or 128");
  if (g->ctx_len < 0) return fail(h, FDL_EINVAL, "ctx_len must be >= 0");
  if (g->ctx_len >= (1 << 24)) return fail(h, FDL_EUNSUPPORTED, "ctx_len must be < 2^24");
  if (!is_pow2(g->kv_block) || g->kv_block > 4096)
    return fail(h, FDL_EINVAL, "kv_block must be a power of two in [1, 4096]");
  if (g->dec_len < 1 || g->dec_len > 64) return fail(h, FDL_EINVAL, "dec_len must be in [1, 64]");
  if (g->dtype != FDL_F32 && g->dtype != FDL_BF16) return fail(h, FDL_EINVAL, "unknown dtype");
  if (g->ctx_lens && g->paged)
    return fail(h, FDL_EUNSUPPORTED, "per-sequence lengths (ctx_lens) take a contiguous cache");
  if (g->paged) {
    if (!is_pow2(g->page_tokens) || g->page_tokens > 4096)
      return fail(h, FDL_EINVAL, "page_tokens must be a power of two in [1, 4096]");
    if (g->pages_per_seq < 1 || (long long)g->pages_per_seq * g->page_tokens < g->ctx_len)
      return fail(h, FDL_EINVAL, "pages_per_seq * page_tokens must cover ctx_len");
    if (g->n_pages < 1) return fail(h, FDL_EINVAL, "n_pages must be >= 1");
  }
  o.B = g->batch;
  o.Hq = g->n_q_heads;
  o.Hkv = g->n_kv_heads;
  o.G = g->n_q_heads / g->n_kv_heads;
  o.D = g->head_dim;
  o.L = g->ctx_len;
  o.bt = g->kv_block;
  o.T = g->dec_len;
  o.dtype = g->dtype;
  o.paged = g->paged ? 1 : 0;
  o.page_tokens = g->paged ? g->page_tokens : 1;
  o.page_log2 = g->paged ? ilog2(g->page_tokens) : 0;
  o.pps = g->paged ? g->pages_per_seq : 0;
  o.n_pages = g->paged ? g->n_pages : 0;
  o.lens = g->ctx_lens;
  return FDL_OK;
}

// Records a pair of events around one launch (or one layer) when profiling is on.
// Times the launches in its scope when profiling is on for its kind.  Inner mode hands the events to
// the launcher instead (timer()), which ties them to the kernel's own dispatch timestamps.
struct ProfScope {
  fdl_handle h;
  int kind;
  bool inner;
  hipEvent_t a = nullptr, b = nullptr;
  fdl::KernelTimer kt{};
  ProfScope(fdl_handle hh, int k, bool inner_ = false) : h(hh), kind(k), inner(inner_) {
    if (h->prof_on && ((h->prof_mask >> k) & 1u) && (h->prof_seen[k]++ % h->prof_every) == 0 &&
        h->prof_used + 2 <= h->prof_pool.size()) {
      a = h->prof_pool[h->prof_used++];
      b = h->prof_pool[h->prof_used++];
      kt = {a, b};
      if (!inner) (void)hipEventRecord(a, h->stream);
    }
  }
  const fdl::KernelTimer* timer() const { return a ? &kt : nullptr; }
  ~ProfScope() {
    if (a) {
      if (!inner) (void)hipEventRecord(b, h->stream);
      h->prof_recs.push_back({kind, a, b});
    }
  }
};

// ---- validated launches shared by the single calls and fdl_focus_step ----------------------

fdl_status run_predict(fdl_handle h, int batch, int T, const float* prev_conf, const uint8_t* masked,
                       int top_k, int window, uint64_t* pred_mask, int32_t* n_pred) {
  ProfScope ps(h, FDL_PROF_PREDICT);
  return hip_status(h, fdl::launch_predict(h->stream, batch, T, prev_conf, masked, top_k, window,
                                           pred_mask, n_pred),
                    "predict launch");
}

fdl_status run_score_units(fdl_handle h, const Geom& g, const void* q, const uint64_t* pred_mask,
                           const float* ks, int n_units, int unit_log2, float* scores) {
  ProfScope ps(h, FDL_PROF_SCORE);
  return hip_status(h, fdl::launch_score_units(h->stream, g, q, pred_mask, ks, n_units, unit_log2, scores),
                    "score_units launch");
}

// The calls that do not take per-sequence lengths.
fdl_status no_lens(fdl_handle h, const Geom& g, const char* what) {
  if (g.lens) return fail(h, FDL_EUNSUPPORTED, "%s does not take per-sequence lengths (ctx_lens)", what);
  return FDL_OK;
}

fdl_status check_sinks(fdl_handle h, const Geom& g, const void* k_cache, const void* k_dec,
                       float tau, int max_sinks, const int32_t* sink_pos, const int32_t* n_sinks,
                       int* ns, int* cap) {
  if (!k_cache || !k_dec || !sink_pos || !n_sinks)
    return fail(h, FDL_EINVAL, "sink detection needs k_cache, k_dec, sink_pos and n_sinks");
  if (g.paged) return fail(h, FDL_EUNSUPPORTED, "sink detection reads a contiguous cache");
  if (!(tau > 0.f)) return fail(h, FDL_EINVAL, "sink_tau must be > 0");
  if (max_sinks < 1) return fail(h, FDL_EINVAL, "max_sinks must be >= 1");
  if (g.Hq > 255) return fail(h, FDL_EUNSUPPORTED, "sink detection supports up to 255 q-heads");
  if (g.dtype == FDL_BF16 && g.T > 32)
    return fail(h, FDL_EUNSUPPORTED, "bf16 sink detection needs dec_len <= 32");
  const size_t need = fdl::sink_scratch_bytes(g, ns, cap);
  if (need > h->scratch_bytes) return fail(h, FDL_ENOMEM, "workspace too small for sink detection");
  if (h->safe_sync) *ns = 1;   // one workgroup per head: nothing is merged across workgroups
  return FDL_OK;
}

// pin: the prediction inputs when this detection is the step's first reader of the prediction (it
// then computes pred_mask itself, see launch_sinks)
fdl_status run_sinks(fdl_handle h, const Geom& g, const void* q, const uint64_t* pred_mask,
                     const void* k_cache, const void* k_dec, float tau, int max_sinks,
                     int32_t* sink_pos, int32_t* n_sinks, int ns, int cap, const fdl::PredictIn* pin = nullptr,
                     bool keep_bitmap = false) {
  ProfScope ps(h, FDL_PROF_SINKS);
  return hip_status(h, fdl::launch_sinks(h->stream, g, q, pred_mask, k_cache, k_dec, tau, max_sinks,
                                         sink_pos, n_sinks, h->scratch, ns, cap, h->status,
                                         h->num_cus, h->tickets, h->sink_area,
                                         // the upper half of the phase buffer (the fused kernel uses the lower)
                                         h->stamps ? h->stamps + h->stamp_words / 2 : nullptr,
                                         h->stamp_words / 2, pin, keep_bitmap),
                    "sinks launch");
}

fdl_status run_select(fdl_handle h, const Geom& g, const float* scores, int n_units, int unit_log2,
                      const int32_t* sink_pos, const int32_t* n_sinks, int max_sinks,
                      const int32_t* cand_idx, int n_cand, int top_k, int force_first, int max_sel,
                      int32_t* sel_idx, int32_t* n_sel) {
  ProfScope ps(h, FDL_PROF_SELECT);
  return hip_status(h, fdl::launch_select(h->stream, g, scores, n_units, unit_log2, sink_pos, n_sinks,
                                          max_sinks, cand_idx, n_cand, top_k, force_first, max_sel,
                                          sel_idx, n_sel, h->status),
                    "select launch");
}

int attn_splits(fdl_handle h, const Geom& g, long long list_tokens) {
  if (g.dtype != FDL_BF16) return 1;
  int n_splits = fdl::mha_choose_splits(g, list_tokens, h->num_cus);
  while (n_splits > 1 && fdl::attn_scratch_bytes(g, n_splits) > h->scratch_bytes) n_splits /= 2;
  return n_splits;
}

fdl_status run_attn(fdl_handle h, const Geom& g, const void* q, const void* k_cache,
                    const void* v_cache, const void* k_dec, const void* v_dec,
                    const int32_t* page_table, const int32_t* sel_idx, const int32_t* n_sel,
                    int max_sel, int unit_log2, int dense, void* out, int n_hint = 0) {
  long long list_tokens = g.L;
  if (!dense) {
    list_tokens = (long long)max_sel << unit_log2;
    if (list_tokens > g.L) list_tokens = g.L;
  }
  const int n_splits = attn_splits(h, g, list_tokens);
  ProfScope ps(h, dense ? FDL_PROF_DENSE_ATTN : FDL_PROF_SPARSE_ATTN, /*inner=*/true);
  return hip_status(h, fdl::launch_attn(h->stream, g, q, k_cache, v_cache, k_dec, v_dec, page_table,
                                        sel_idx, n_sel, max_sel, unit_log2, dense, out, h->scratch,
                                        n_splits, h->tickets, h->status, n_hint, ps.timer(), h->safe_sync),
                    "attention launch");
}

// Score, select and attend in one kernel (bf16, contiguous cache): same outputs as
// run_score_units + run_select + run_attn.
bool fused_select_ok(const Geom& g, int n_blk, int max_sel, int max_sinks) {
  return g.dtype == FDL_BF16 && g.T <= 32 && !g.paged && g.L > 0 && n_blk <= fdl::kFusedMaxUnits &&
         max_sel <= fdl::kFusedMaxSel && max_sinks <= fdl::kFusedMaxSinks &&
         (g.G == 1 || (long long)g.B * g.Hkv <= fdl::kMaxSplitSegs);
}

// Grouped-query heads in the fused kernel: the (KV head, split) groups need a barrier word each
// and, past split 0, score-exchange rows after the attention partials in the scratch.
static size_t fused_xchg_offset(const Geom& g, int n_splits) {
  return (fdl::attn_scratch_bytes(g, n_splits) + 255) & ~(size_t)255;
}

// How a fused layer handles the sink detection's bitmap (see FusedSelect): read it in place of the
// list (the detecting layer, whose list it then writes), or clear it (a later layer).
struct SinkBitmapUse {
  const uint32_t* read = nullptr;
  uint32_t* clear = nullptr;
  int words = 0;
};

fdl_status run_select_attn(fdl_handle h, const Geom& g, const fdl_layer_io& io, const uint64_t* pred_mask,
                           const fdl_focus_params* fp, int bt_log2, int32_t* sink_pos,
                           int32_t* n_sinks, float* scores, int32_t* sel_idx, int32_t* n_sel,
                           const SinkBitmapUse& sbm = SinkBitmapUse{}) {
  long long list_tokens = (long long)fp->max_sel << bt_log2;
  if (list_tokens > g.L) list_tokens = g.L;
  int n_splits = attn_splits(h, g, list_tokens);
  const int n_blk = (g.L + g.bt - 1) / g.bt;
  float* xchg = nullptr;
  if (g.G == 1 && n_splits > 1 && n_blk <= fdl::kFusedTaggedUnits && !h->safe_sync) {
    // the splits' tagged score exchange: one 64-bit entry per (sequence, head, unit)
    if (fused_xchg_offset(g, n_splits) + (size_t)g.B * g.Hkv * n_blk * sizeof(uint64_t) <= h->scratch_bytes)
      xchg = reinterpret_cast<float*>(h->scratch + fused_xchg_offset(g, n_splits));
  } else if (g.G > 1) {
    while (n_splits > 1 && ((long long)g.B * g.Hkv * n_splits > fdl::kMaxSplitSegs ||
                            fused_xchg_offset(g, n_splits) + (size_t)g.B * g.Hkv * n_splits * n_blk * sizeof(float) >
                                h->scratch_bytes))
      --n_splits;
    if (fused_xchg_offset(g, n_splits) + (size_t)g.B * g.Hkv * n_splits * n_blk * sizeof(float) > h->scratch_bytes)
      return fail(h, FDL_ENOMEM, "workspace too small for the score exchange");
    xchg = reinterpret_cast<float*>(h->scratch + fused_xchg_offset(g, n_splits));
  }
  fdl::FusedSelect fs{};
  fs.pred_mask = pred_mask;
  fs.ks = io.ks;
  fs.sink_pos = sink_pos;
  fs.n_sinks = n_sinks;
  fs.max_sinks = fp->max_sinks;
  fs.top_k = fp->top_k_blocks;
  fs.scores = scores;
  fs.sel_idx = sel_idx;
  fs.n_sel = n_sel;
  fs.barriers = h->barriers;
  fs.spin_limit = h->spin_limit;
  fs.xchg = xchg;
  fs.sink_bitmap = sbm.read;
  fs.sink_pos_out = sink_pos;
  fs.n_sinks_out = n_sinks;
  fs.clear_bitmap = sbm.clear;
  fs.sink_words = sbm.words;
  fs.stamps = h->stamps;
  fs.stamp_words = h->stamp_words;
  fs.serial = h->fused_serial++;
  ProfScope ps(h, FDL_PROF_SPARSE_ATTN, /*inner=*/true);
  return hip_status(h, fdl::launch_attn_mha(h->stream, g, io.q, io.k_cache, io.v_cache, io.k_dec, io.v_dec,
                                            nullptr, sel_idx, n_sel, fp->max_sel, bt_log2, 0, io.out,
                                            h->scratch, n_splits, h->tickets, h->status, 0, ps.timer(), &fs,
                                            h->safe_sync),
                    "select-attention launch");
}

}  // namespace

extern "C" {

const char* fdl_status_string(fdl_status s) {
  switch (s) {
    case FDL_OK: return "ok";
    case FDL_EINVAL: return "invalid argument";
    case FDL_ENOMEM: return "out of memory (workspace too small or allocation failed)";
    case FDL_EHIP: return "HIP runtime error";
    case FDL_EOVERFLOW: return "device-side capacity overflow (sinks or sink candidates)";
    case FDL_EUNSUPPORTED: return "shape outside the supported kernel set";
    case FDL_EINDEX: return "out-of-range unit or page index (rows skipped)";
    case FDL_ESYNC: return "workgroups that merge through one L2 ran on different XCDs (outputs invalid)";
  }
  return "unknown status";
}

const char* fdl_last_error(fdl_handle h) { return h ? h->last_error : "no handle"; }

fdl_status fdl_create(fdl_handle* out, void* hip_stream, size_t workspace_bytes) {
  if (!out) return FDL_EINVAL;
  *out = nullptr;
  if (workspace_bytes == 0) workspace_bytes = (size_t)64 << 20;
  if (workspace_bytes < fdl::kHeaderBytes + ((size_t)1 << 20))
    workspace_bytes = fdl::kHeaderBytes + ((size_t)1 << 20);
  fdl_ctx* h = new (std::nothrow) fdl_ctx();
  if (!h) return FDL_ENOMEM;
  h->stream = static_cast<hipStream_t>(hip_stream);
  if (hipGetDevice(&h->device) != hipSuccess ||
      hipDeviceGetAttribute(&h->num_cus, hipDeviceAttributeMultiprocessorCount, h->device) !=
          hipSuccess) {
    delete h;
    return FDL_EHIP;
  }
  void* ws = nullptr;
  if (hipMalloc(&ws, workspace_bytes) != hipSuccess) {
    delete h;
    return FDL_ENOMEM;
  }
  if (hipMemset(ws, 0, fdl::kHeaderBytes) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
    (void)hipFree(ws);
    delete h;
    return FDL_EHIP;
  }
  h->ws = static_cast<char*>(ws);
  h->ws_bytes = workspace_bytes;
  h->status = reinterpret_cast<uint32_t*>(h->ws);
  h->tickets = reinterpret_cast<uint32_t*>(h->ws + fdl::kTicketOffset);
  h->barriers = reinterpret_cast<uint32_t*>(h->ws + fdl::kBarrierOffset);
  h->sink_area = h->ws + fdl::kSinkOffset;
  {
    const char* e = getenv("FDL_SPIN_LIMIT");
    h->spin_limit = e ? atoi(e) : 200000;
    const char* safe = getenv("FDL_SAFE_SYNC");
    h->safe_sync = safe != nullptr && safe[0] != '\0' && safe[0] != '0';
  }
  h->scratch = h->ws + fdl::kHeaderBytes;
  h->scratch_bytes = workspace_bytes - fdl::kHeaderBytes;
  h->last_error[0] = 0;
  *out = h;
  return FDL_OK;
}

fdl_status fdl_destroy(fdl_handle h) {
  if (!h) return FDL_EINVAL;
  if (h->capturing) {   // abandon an open capture
    hipGraph_t graph = nullptr;
    if (hipStreamEndCapture(h->stream, &graph) == hipSuccess && graph) (void)hipGraphDestroy(graph);
  }
  (void)hipStreamSynchronize(h->stream);
  (void)hipFree(h->ws);
  delete h;
  return FDL_OK;
}

fdl_status fdl_set_stream(fdl_handle h, void* hip_stream) {
  if (!h) return FDL_EINVAL;
  if (h->capturing && static_cast<hipStream_t>(hip_stream) != h->stream)
    return fail(h, FDL_EINVAL, "the handle's stream is being captured");
  h->stream = static_cast<hipStream_t>(hip_stream);
  return FDL_OK;
}

fdl_status fdl_get_status(fdl_handle h) { return fdl_get_status_bits(h, nullptr); }

fdl_status fdl_get_status_bits(fdl_handle h, uint32_t* bits) {
  static_assert(FDL_FLAG_SINK_OVERFLOW == fdl::ST_SINK_OVERFLOW && FDL_FLAG_CAND_OVERFLOW == fdl::ST_CAND_OVERFLOW &&
                    FDL_FLAG_BAD_INDEX == fdl::ST_BAD_INDEX && FDL_FLAG_SEL_OVERFLOW == fdl::ST_SEL_OVERFLOW &&
                    FDL_FLAG_SPLIT_FALLBACK == fdl::ST_SYNC_FALLBACK && FDL_FLAG_PLACEMENT == fdl::ST_PLACEMENT &&
                    FDL_FLAG_SPLIT_PLACEMENT == fdl::ST_SPLIT_PLACEMENT,
                "status bits");
  if (bits) *bits = 0;
  if (!h) return FDL_EINVAL;
  if (h->capturing) return fail(h, FDL_EINVAL, "the handle's stream is being captured");
  fdl_status st = hip_status(h, hipStreamSynchronize(h->stream), "hipStreamSynchronize");
  if (st != FDL_OK) return st;
  uint32_t word = 0;
  st = hip_status(h, hipMemcpy(&word, h->status, sizeof(word), hipMemcpyDeviceToHost), "hipMemcpy");
  if (st != FDL_OK) return st;
  if (word) {
    h->debug_seen = 0;
    st = hip_status(h, hipMemset(h->status, 0, sizeof(uint32_t)), "hipMemset");
    if (st != FDL_OK) return st;
    st = hip_status(h, hipDeviceSynchronize(), "hipDeviceSynchronize");
    if (st != FDL_OK) return st;
  }
  if (bits) *bits = word;
  if (word & fdl::ST_SPLIT_PLACEMENT) return FDL_ESYNC;
  if (word & (fdl::ST_SINK_OVERFLOW | fdl::ST_CAND_OVERFLOW | fdl::ST_SEL_OVERFLOW)) return FDL_EOVERFLOW;
  if (word & fdl::ST_BAD_INDEX) return FDL_EINDEX;
  return FDL_OK;
}

fdl_status fdl_pool_keys(fdl_handle h, const fdl_geom* gp, const void* k_cache,
                         const int32_t* page_table, int32_t unit_tokens, float* ks) {
  if (!h) return FDL_EINVAL;
  Geom g;
  fdl_status st = check_geom(h, gp, g);
  if (st != FDL_OK) return st;
  if (!k_cache || !ks) return fail(h, FDL_EINVAL, "k_cache and ks must be non-NULL");
  if (g.paged && !page_table) return fail(h, FDL_EINVAL, "paged layout needs a page_table");
  if (!is_pow2(unit_tokens) || unit_tokens > 4096)
    return fail(h, FDL_EINVAL, "unit_tokens must be a power of two in [1, 4096]");
  ProfScope ps(h, FDL_PROF_POOL);
  return hip_status(h, fdl::launch_pool_keys(h->stream, g, k_cache, page_table, ilog2(unit_tokens), ks,
                                             h->status, reinterpret_cast<float*>(h->scratch), h->scratch_bytes),
                    "pool_keys launch");
}

fdl_status fdl_cache_write(fdl_handle h, const fdl_geom* gp, const void* k_new, const void* v_new, int32_t t0,
                           int32_t n_tok, void* k_cache, void* v_cache, const int32_t* page_table,
                           int32_t unit_tokens, float* ks) {
  if (!h) return FDL_EINVAL;
  Geom g;
  fdl_status st = check_geom(h, gp, g);
  if (st != FDL_OK) return st;
  if (!k_new || !v_new || !k_cache || !v_cache)
    return fail(h, FDL_EINVAL, "k_new, v_new, k_cache and v_cache must be non-NULL");
  if ((st = no_lens(h, g, "fdl_cache_write")) != FDL_OK) return st;
  if (g.paged && !page_table) return fail(h, FDL_EINVAL, "paged layout needs a page_table");
  if (t0 < 0 || n_tok < 1 || (long long)t0 + n_tok > g.L)
    return fail(h, FDL_EINVAL, "the rows [t0, t0 + n_tok) must lie in [0, ctx_len) and be non-empty");
  int lg = 6;
  if (ks) {
    if (!is_pow2(unit_tokens) || unit_tokens < 16 || unit_tokens > 4096)
      return fail(h, FDL_EINVAL, "unit_tokens must be a power of two in [16, 4096]");
    lg = ilog2(unit_tokens);
    if (unit_tokens > 64 &&
        (size_t)g.B * g.Hkv * ((g.L + 63) / 64) * g.D * sizeof(float) > h->scratch_bytes)
      return fail(h, FDL_ENOMEM, "workspace too small for the sub-unit sums");
  }
  ProfScope ps(h, FDL_PROF_POOL);
  return hip_status(h, fdl::launch_cache_write(h->stream, g, k_new, v_new, t0, n_tok, k_cache, v_cache, page_table,
                                               lg, ks, h->status, reinterpret_cast<float*>(h->scratch),
                                               h->scratch_bytes),
                    "cache_write launch");
}

fdl_status fdl_predict_queries(fdl_handle h, int32_t batch, int32_t dec_len, const float* prev_conf,
                               const uint8_t* masked, int32_t top_k, int32_t window,
                               uint64_t* pred_mask, int32_t* n_pred) {
  if (!h) return FDL_EINVAL;
  if (batch < 1) return fail(h, FDL_EINVAL, "batch must be >= 1");
  if (dec_len < 1 || dec_len > 64) return fail(h, FDL_EINVAL, "dec_len must be in [1, 64]");
  if (top_k < 0) return fail(h, FDL_EINVAL, "top_k must be >= 0");
  if (window < 0) return fail(h, FDL_EINVAL, "window must be >= 0");
  if (!masked || !pred_mask || !n_pred)
    return fail(h, FDL_EINVAL, "masked, pred_mask and n_pred must be non-NULL");
  return run_predict(h, batch, dec_len, prev_conf, masked, top_k, window, pred_mask, n_pred);
}

fdl_status fdl_score_blocks(fdl_handle h, const fdl_geom* gp, const void* q, const uint64_t* pred_mask,
                            const float* ks, int32_t unit_tokens, const int32_t* cand_idx,
                            int32_t n_cand, const void* k_cache, const void* k_dec,
                            const int32_t* page_table, float* scores, int32_t detect_sinks,
                            float sink_tau, int32_t max_sinks, int32_t* sink_pos, int32_t* n_sinks) {
  if (!h) return FDL_EINVAL;
  Geom g;
  fdl_status st = check_geom(h, gp, g);
  if (st != FDL_OK) return st;
  if (!q || !pred_mask || !scores) return fail(h, FDL_EINVAL, "q, pred_mask and scores must be non-NULL");
  if (!is_pow2(unit_tokens) || unit_tokens > 4096)
    return fail(h, FDL_EINVAL, "unit_tokens must be a power of two in [1, 4096]");
  const int n_units = (g.L + unit_tokens - 1) / unit_tokens;
  if (cand_idx) {
    if (detect_sinks) return fail(h, FDL_EINVAL, "sink detection is a level-1 (cand_idx == NULL) option");
    if ((st = no_lens(h, g, "level-2 scoring")) != FDL_OK) return st;
    if (n_cand < 1 || n_cand > n_units) return fail(h, FDL_EINVAL, "n_cand must be in [1, n_units]");
    if (!k_cache) return fail(h, FDL_EINVAL, "level-2 scoring needs k_cache");
    if (g.paged && !page_table) return fail(h, FDL_EINVAL, "paged layout needs a page_table");
    if (g.L % unit_tokens) return fail(h, FDL_EINVAL, "level-2 scoring needs ctx_len %% unit_tokens == 0");
    ProfScope ps(h, FDL_PROF_SCORE);
    return hip_status(h, fdl::launch_score_tokens(h->stream, g, q, pred_mask, k_cache, page_table,
                                                  ilog2(unit_tokens), cand_idx, n_cand, scores,
                                                  h->status),
                      "score_tokens launch");
  }
  if (!ks) return fail(h, FDL_EINVAL, "level-1 scoring needs ks");
  int ns = 0, cap = 0;
  if (detect_sinks) {
    st = check_sinks(h, g, k_cache, k_dec, sink_tau, max_sinks, sink_pos, n_sinks, &ns, &cap);
    if (st != FDL_OK) return st;
  }
  st = run_score_units(h, g, q, pred_mask, ks, n_units, ilog2(unit_tokens), scores);
  if (st != FDL_OK || !detect_sinks) return st;
  return run_sinks(h, g, q, pred_mask, k_cache, k_dec, sink_tau, max_sinks, sink_pos, n_sinks, ns, cap);
}

fdl_status fdl_score_blocks_max(fdl_handle h, const fdl_geom* gp, const void* q, const uint64_t* pred_mask,
                                const float* ks, int32_t unit_tokens, float* scores) {
  if (!h) return FDL_EINVAL;
  Geom g;
  fdl_status st = check_geom(h, gp, g);
  if (st != FDL_OK) return st;
  if (!q || !pred_mask || !ks || !scores) return fail(h, FDL_EINVAL, "q, pred_mask, ks and scores must be non-NULL");
  if (!is_pow2(unit_tokens) || unit_tokens > 4096)
    return fail(h, FDL_EINVAL, "unit_tokens must be a power of two in [1, 4096]");
  if (g.dtype != FDL_BF16 || g.T > 32)
    return fail(h, FDL_EUNSUPPORTED, "per-query scoring runs bf16 queries with dec_len <= 32");
  if ((st = no_lens(h, g, "fdl_score_blocks_max")) != FDL_OK) return st;
  const int n_units = (g.L + unit_tokens - 1) / unit_tokens;
  ProfScope ps(h, FDL_PROF_SCORE);
  return hip_status(h, fdl::launch_score_units_max(h->stream, g, q, pred_mask, ks, n_units, scores),
                    "score_units_max launch");
}

fdl_status fdl_score_blocks_mass(fdl_handle h, const fdl_geom* gp, const void* q, const uint64_t* pred_mask,
                                 const float* ks, int32_t unit_tokens, float* scores) {
  if (!h) return FDL_EINVAL;
  Geom g;
  fdl_status st = check_geom(h, gp, g);
  if (st != FDL_OK) return st;
  if (!q || !pred_mask || !ks || !scores) return fail(h, FDL_EINVAL, "q, pred_mask, ks and scores must be non-NULL");
  if (!is_pow2(unit_tokens) || unit_tokens > 4096)
    return fail(h, FDL_EINVAL, "unit_tokens must be a power of two in [1, 4096]");
  if (g.dtype != FDL_BF16 || g.T > 32)
    return fail(h, FDL_EUNSUPPORTED, "softmax-mass scoring runs bf16 queries with dec_len <= 32");
  if ((st = no_lens(h, g, "fdl_score_blocks_mass")) != FDL_OK) return st;
  const int n_units = (g.L + unit_tokens - 1) / unit_tokens;
  if (fdl::mass_scratch_bytes(g, n_units) > h->scratch_bytes)
    return fail(h, FDL_ENOMEM, "workspace too small for softmax-mass scoring");
  ProfScope ps(h, FDL_PROF_SCORE);
  return hip_status(h, fdl::launch_score_units_mass(h->stream, g, q, pred_mask, ks, n_units, ilog2(unit_tokens),
                                                    scores, h->scratch),
                    "score_units_mass launch");
}

static fdl_status select_blocks_impl(fdl_handle h, const fdl_geom* gp, const float* scores, int32_t n_units,
                                     int32_t unit_tokens, const int32_t* sink_pos, const int32_t* n_sinks,
                                     int32_t max_sinks, const int32_t* cand_idx, int32_t n_cand,
                                     int32_t top_k, int32_t force_first, int32_t max_sel, int32_t* sel_idx,
                                     int32_t* n_sel, int shared) {
  if (!h) return FDL_EINVAL;
  Geom g;
  fdl_status st = check_geom(h, gp, g);
  if (st != FDL_OK) return st;
  if (shared && g.Hkv > 32) return fail(h, FDL_EUNSUPPORTED, "per-sequence selection takes at most 32 KV heads");
  if ((cand_idx || shared) && (st = no_lens(h, g, "level-2 and per-sequence selection")) != FDL_OK) return st;
  if (!scores || !sel_idx || !n_sel) return fail(h, FDL_EINVAL, "scores, sel_idx and n_sel must be non-NULL");
  if (!is_pow2(unit_tokens) || unit_tokens > 8192)
    return fail(h, FDL_EINVAL, "unit_tokens must be a power of two in [1, 8192]");
  if (n_units < 0 || n_units > 8192) return fail(h, FDL_EUNSUPPORTED, "n_units must be in [0, 8192]");
  if (top_k < 0) return fail(h, FDL_EINVAL, "top_k must be >= 0");
  if (max_sel < 1) return fail(h, FDL_EINVAL, "max_sel must be >= 1");
  if (cand_idx) {
    if (n_cand < 1 || n_cand > n_units) return fail(h, FDL_EINVAL, "n_cand must be in [1, n_units]");
    const int ff = force_first ? 1 : 0;
    if (top_k > unit_tokens - ff) return fail(h, FDL_EINVAL, "top_k exceeds the tokens of a unit");
    if ((long long)n_cand * (ff + top_k) > max_sel) return fail(h, FDL_EINVAL, "max_sel too small");
  } else {
    if ((sink_pos == nullptr) != (n_sinks == nullptr))
      return fail(h, FDL_EINVAL, "sink_pos and n_sinks go together");
    if (sink_pos && max_sinks < 1) return fail(h, FDL_EINVAL, "max_sinks must be >= 1");
    const long long forced_cap = sink_pos ? max_sinks : 0;
    long long need = forced_cap + top_k;
    if (need > n_units) need = n_units;
    if (need > max_sel) return fail(h, FDL_EINVAL, "max_sel must cover min(n_units, max_sinks + top_k)");
  }
  ProfScope ps(h, FDL_PROF_SELECT);
  return hip_status(h, fdl::launch_select(h->stream, g, scores, n_units, ilog2(unit_tokens), sink_pos, n_sinks,
                                          max_sinks, cand_idx, n_cand, top_k, force_first ? 1 : 0, max_sel,
                                          sel_idx, n_sel, h->status, shared),
                    "select launch");
}

fdl_status fdl_select_blocks(fdl_handle h, const fdl_geom* gp, const float* scores, int32_t n_units,
                             int32_t unit_tokens, const int32_t* sink_pos, const int32_t* n_sinks,
                             int32_t max_sinks, const int32_t* cand_idx, int32_t n_cand,
                             int32_t top_k, int32_t force_first, int32_t max_sel, int32_t* sel_idx,
                             int32_t* n_sel) {
  return select_blocks_impl(h, gp, scores, n_units, unit_tokens, sink_pos, n_sinks, max_sinks, cand_idx, n_cand,
                            top_k, force_first, max_sel, sel_idx, n_sel, 0);
}

fdl_status fdl_select_blocks_shared(fdl_handle h, const fdl_geom* gp, const float* scores, int32_t n_units,
                                    int32_t unit_tokens, const int32_t* sink_pos, const int32_t* n_sinks,
                                    int32_t max_sinks, int32_t top_k, int32_t max_sel, int32_t* sel_idx,
                                    int32_t* n_sel) {
  return select_blocks_impl(h, gp, scores, n_units, unit_tokens, sink_pos, n_sinks, max_sinks, nullptr, 0, top_k,
                            0, max_sel, sel_idx, n_sel, 1);
}

fdl_status fdl_expand_tokens(fdl_handle h, const fdl_geom* gp, const int32_t* sel_idx, const int32_t* n_sel,
                             int32_t max_sel, int32_t unit_tokens, const int32_t* sink_pos, const int32_t* n_sinks,
                             int32_t max_sinks, int32_t* tok_idx, int32_t* n_tok, int32_t max_tok) {
  if (!h) return FDL_EINVAL;
  Geom g;
  fdl_status st = check_geom(h, gp, g);
  if (st != FDL_OK) return st;
  if (!sel_idx || !n_sel || !tok_idx || !n_tok) return fail(h, FDL_EINVAL, "sel_idx, n_sel, tok_idx and n_tok must be non-NULL");
  if ((st = no_lens(h, g, "fdl_expand_tokens")) != FDL_OK) return st;
  if (!is_pow2(unit_tokens) || unit_tokens > 4096)
    return fail(h, FDL_EINVAL, "unit_tokens must be a power of two in [1, 4096]");
  if ((sink_pos == nullptr) != (n_sinks == nullptr)) return fail(h, FDL_EINVAL, "sink_pos and n_sinks go together");
  if (max_sel < 1 || (sink_pos && max_sinks < 1)) return fail(h, FDL_EINVAL, "max_sel and max_sinks must be >= 1");
  const int ms = sink_pos ? max_sinks : 0;
  if (!fdl::expand_tokens_ok(max_sel, ms)) return fail(h, FDL_EUNSUPPORTED, "max_sel <= 4096 and max_sinks <= 512");
  if ((long long)max_sel * unit_tokens + ms > max_tok)
    return fail(h, FDL_EINVAL, "max_tok must cover max_sel * unit_tokens + max_sinks");
  ProfScope ps(h, FDL_PROF_SELECT);
  return hip_status(h, fdl::launch_expand_tokens(h->stream, g, sel_idx, n_sel, max_sel, ilog2(unit_tokens), sink_pos,
                                                 n_sinks, ms, tok_idx, n_tok, max_tok, h->status),
                    "expand_tokens launch");
}

fdl_status fdl_score_select_tokens(fdl_handle h, const fdl_geom* gp, const void* q, const uint64_t* pred_mask,
                                   const void* k_cache, const int32_t* page_table, int32_t unit_tokens,
                                   const int32_t* cand_idx, int32_t n_cand, int32_t top_k, int32_t max_sel,
                                   float* scores, int32_t* sel_idx, int32_t* n_sel) {
  if (!h) return FDL_EINVAL;
  Geom g;
  fdl_status st = check_geom(h, gp, g);
  if (st != FDL_OK) return st;
  if (!q || !pred_mask || !k_cache || !cand_idx || !scores || !sel_idx || !n_sel)
    return fail(h, FDL_EINVAL, "q, pred_mask, k_cache, cand_idx, scores, sel_idx and n_sel must be non-NULL");
  if ((st = no_lens(h, g, "fdl_score_select_tokens")) != FDL_OK) return st;
  if (!is_pow2(unit_tokens) || unit_tokens > 4096)
    return fail(h, FDL_EINVAL, "unit_tokens must be a power of two in [1, 4096]");
  if (g.L % unit_tokens) return fail(h, FDL_EINVAL, "level-2 scoring needs ctx_len %% unit_tokens == 0");
  const int n_units = g.L / unit_tokens;
  if (n_cand < 1 || n_cand > n_units) return fail(h, FDL_EINVAL, "n_cand must be in [1, n_units]");
  if (g.paged && !page_table) return fail(h, FDL_EINVAL, "paged layout needs a page_table");
  if (top_k < 0 || top_k > unit_tokens - 1) return fail(h, FDL_EINVAL, "top_k must be in [0, unit_tokens - 1]");
  if (max_sel < 1 || (long long)n_cand * (1 + top_k) > max_sel) return fail(h, FDL_EINVAL, "max_sel too small");
  const int lg = ilog2(unit_tokens);
  if (fdl::score_select_tokens_ok(g, lg)) {
    ProfScope ps(h, FDL_PROF_SCORE);
    return hip_status(h, fdl::launch_score_select_tokens(h->stream, g, q, pred_mask, k_cache, page_table, lg,
                                                         cand_idx, n_cand, top_k, max_sel, scores, sel_idx,
                                                         n_sel, h->status),
                      "score_select_tokens launch");
  }
  {
    ProfScope ps(h, FDL_PROF_SCORE);
    st = hip_status(h, fdl::launch_score_tokens(h->stream, g, q, pred_mask, k_cache, page_table, lg, cand_idx,
                                                n_cand, scores, h->status),
                    "score_tokens launch");
    if (st != FDL_OK) return st;
  }
  return run_select(h, g, scores, n_units, lg, nullptr, nullptr, 0, cand_idx, n_cand, top_k, 1, max_sel, sel_idx,
                    n_sel);
}

fdl_status fdl_select_chunks_tokens(fdl_handle h, const fdl_geom* gp, const void* q, const uint64_t* pred_mask,
                                    const float* chunk_sums, const void* k_cache, const int32_t* page_table,
                                    int32_t chunk_tokens, int32_t top_k_chunks, int32_t top_k, int32_t max_sel,
                                    float* chunk_scores, int32_t* chunks, int32_t* n_chunks_sel,
                                    float* token_scores, int32_t* sel_idx, int32_t* n_sel) {
  if (!h) return FDL_EINVAL;
  Geom g;
  fdl_status st = check_geom(h, gp, g);
  if (st != FDL_OK) return st;
  if (!q || !pred_mask || !chunk_sums || !k_cache || !chunk_scores || !chunks || !n_chunks_sel || !token_scores ||
      !sel_idx || !n_sel)
    return fail(h, FDL_EINVAL, "every tensor argument but page_table must be non-NULL");
  if ((st = no_lens(h, g, "fdl_select_chunks_tokens")) != FDL_OK) return st;
  if (!is_pow2(chunk_tokens) || chunk_tokens > 4096)
    return fail(h, FDL_EINVAL, "chunk_tokens must be a power of two in [1, 4096]");
  if (g.L % chunk_tokens) return fail(h, FDL_EINVAL, "ctx_len %% chunk_tokens must be 0");
  const int n_chunks = g.L / chunk_tokens;
  if (top_k_chunks < 1 || top_k_chunks > n_chunks) return fail(h, FDL_EINVAL, "top_k_chunks must be in [1, n_chunks]");
  if (g.paged && !page_table) return fail(h, FDL_EINVAL, "paged layout needs a page_table");
  if (top_k < 0 || top_k > chunk_tokens - 1) return fail(h, FDL_EINVAL, "top_k must be in [0, chunk_tokens - 1]");
  if (max_sel < 1 || (long long)top_k_chunks * (1 + top_k) > max_sel) return fail(h, FDL_EINVAL, "max_sel too small");
  const int lg = ilog2(chunk_tokens);
  if (!fdl::select_chunks_tokens_ok(g, lg, n_chunks))
    return fail(h, FDL_EUNSUPPORTED, "one-launch chunk selection: bf16, dec_len <= 32, chunks of 256 to 4096 "
                                     "tokens, pages >= 16 tokens, G <= 8 and at most 64 chunks");
  ProfScope ps(h, FDL_PROF_SCORE);
  return hip_status(h, fdl::launch_select_chunks_tokens(h->stream, g, q, pred_mask, chunk_sums, k_cache, page_table,
                                                        lg, top_k_chunks, top_k, max_sel, chunk_scores, chunks,
                                                        n_chunks_sel, token_scores, sel_idx, n_sel, h->status,
                                                        h->stamps, h->stamp_words),
                    "select_chunks_tokens launch");
}

// ---- sparse attention for callers that cannot allocate ------------------------------------------
//
// The split partials, the merge tickets and a status word live in one file-scope device array instead
// of a handle's workspace.  Each GPU holds its own copy for the life of the process; host code
// reaches it only through the address hipGetSymbolAddress returns for the current device (the array's
// name on the host is a stand-in, not a device address).  Layout: status word at 0, tickets from
// kStaticTicketOffset (left at zero by every launch), partials from kStaticPartialOffset.
namespace {
constexpr size_t kStaticScratchBytes = (size_t)8 << 20;
constexpr size_t kStaticTicketOffset = 4096;
constexpr size_t kStaticPartialOffset =
    kStaticTicketOffset + (size_t)fdl::kMaxSplitSegs * fdl::kSyncStride * sizeof(uint32_t);
constexpr size_t kStaticPartialBytes = kStaticScratchBytes - kStaticPartialOffset;
constexpr int kStaticMaxDevices = 64;
// the default workspace of fdl_create: the split count the handle calls would choose
constexpr size_t kDefaultScratchBytes = ((size_t)64 << 20) - fdl::kHeaderBytes;

struct StaticDev {
  char* ptr = nullptr;   // device address of `scratch` on this device
  int num_cus = 0;
};
std::mutex g_static_mu;
StaticDev g_static[kStaticMaxDevices];
}  // namespace

static __device__ __align__(256) char scratch[kStaticScratchBytes];

// Set-up, once per device: the array's device address and the compute-unit count; the status word
// and the tickets are cleared by a fill kernel on the caller's stream (no memset node, so a first
// call under graph capture records a kernel).
static fdl_status static_scratch(hipStream_t stream, StaticDev* out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return FDL_EHIP;
  if (dev >= kStaticMaxDevices) return FDL_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_static_mu);
  StaticDev& d = g_static[dev];
  if (d.ptr == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return FDL_EHIP;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return FDL_EHIP;
    if (fdl::launch_fill_u32(stream, static_cast<uint32_t*>(p), kStaticPartialOffset / sizeof(uint32_t), 0u) !=
        hipSuccess)
      return FDL_EHIP;
    d.num_cus = cus;
    d.ptr = static_cast<char*>(p);
  }
  *out = d;
  return FDL_OK;
}

// Argument checks of the attention calls (h may be NULL: the codes are returned without a message).
static fdl_status check_attn(fdl_handle h, const fdl_geom* gp, Geom& g, const void* q, const void* k_cache,
                             const void* v_cache, const void* k_dec, const void* v_dec, const int32_t* page_table,
                             const int32_t* sel_idx, const int32_t* n_sel, int32_t max_sel, int32_t sel_unit_tokens,
                             int dense, const void* out, int* unit_log2) {
  fdl_status st = check_geom(h, gp, g);
  if (st != FDL_OK) return st;
  if (!q || !k_dec || !v_dec || !out) return fail(h, FDL_EINVAL, "q, k_dec, v_dec and out must be non-NULL");
  if (g.L > 0 && (!k_cache || !v_cache)) return fail(h, FDL_EINVAL, "k_cache and v_cache must be non-NULL");
  if (g.paged && !page_table) return fail(h, FDL_EINVAL, "paged layout needs a page_table");
  *unit_log2 = 0;
  if (!dense) {
    if (!sel_idx || !n_sel) return fail(h, FDL_EINVAL, "sel_idx and n_sel must be non-NULL");
    if (max_sel < 1) return fail(h, FDL_EINVAL, "max_sel must be >= 1");
    if (!is_pow2(sel_unit_tokens) || sel_unit_tokens > 4096)
      return fail(h, FDL_EINVAL, "sel_unit_tokens must be a power of two in [1, 4096]");
    *unit_log2 = ilog2(sel_unit_tokens);
    if ((long long)max_sel * sel_unit_tokens >= (1LL << 30))
      return fail(h, FDL_EUNSUPPORTED, "selection too large");
  }
  if (g.dtype == FDL_BF16 && g.T > 32) return fail(h, FDL_EUNSUPPORTED, "bf16 attention needs dec_len <= 32");
  return FDL_OK;
}

static fdl_status attn_common(fdl_handle h, const fdl_geom* gp, const void* q, const void* k_cache,
                              const void* v_cache, const void* k_dec, const void* v_dec,
                              const int32_t* page_table, const int32_t* sel_idx, const int32_t* n_sel,
                              int32_t max_sel, int32_t sel_unit_tokens, int dense, void* out) {
  if (!h) return FDL_EINVAL;
  Geom g;
  int unit_log2 = 0;
  const fdl_status st = check_attn(h, gp, g, q, k_cache, v_cache, k_dec, v_dec, page_table, sel_idx, n_sel, max_sel,
                                   sel_unit_tokens, dense, out, &unit_log2);
  if (st != FDL_OK) return st;
  return run_attn(h, g, q, k_cache, v_cache, k_dec, v_dec, page_table, sel_idx, n_sel, max_sel, unit_log2,
                  dense, out);
}

fdl_status fdl_sparse_attn_noalloc(void* hip_stream, const fdl_geom* gp, const void* q, const void* k_cache,
                                   const void* v_cache, const void* k_dec, const void* v_dec,
                                   const int32_t* page_table, const int32_t* sel_idx, const int32_t* n_sel,
                                   int32_t max_sel, int32_t sel_unit_tokens, void* out, uint32_t* status) {
  Geom g;
  int unit_log2 = 0;
  fdl_status st = check_attn(nullptr, gp, g, q, k_cache, v_cache, k_dec, v_dec, page_table, sel_idx, n_sel,
                             max_sel, sel_unit_tokens, 0, out, &unit_log2);
  if (st != FDL_OK) return st;
  const hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  StaticDev d;
  st = static_scratch(stream, &d);
  if (st != FDL_OK) return st;
  long long list_tokens = (long long)max_sel << unit_log2;
  if (list_tokens > g.L) list_tokens = g.L;
  int n_splits = 1;
  if (g.dtype == FDL_BF16) {   // the split count fdl_sparse_attn takes with the default workspace
    n_splits = fdl::mha_choose_splits(g, list_tokens, d.num_cus);
    while (n_splits > 1 && fdl::attn_scratch_bytes(g, n_splits) > kDefaultScratchBytes) n_splits /= 2;
  }
  if (fdl::attn_scratch_bytes(g, n_splits) > kStaticPartialBytes) return FDL_ENOMEM;
  uint32_t* stat = status ? status : reinterpret_cast<uint32_t*>(d.ptr);
  uint32_t* tickets = reinterpret_cast<uint32_t*>(d.ptr + kStaticTicketOffset);
  return hip_status(nullptr,
                    fdl::launch_attn(stream, g, q, k_cache, v_cache, k_dec, v_dec, page_table, sel_idx, n_sel,
                                     max_sel, unit_log2, 0, out, d.ptr + kStaticPartialOffset, n_splits, tickets,
                                     stat, 0, nullptr),
                    "attention launch");
}

fdl_status fdl_sparse_attn(fdl_handle h, const fdl_geom* g, const void* q, const void* k_cache,
                           const void* v_cache, const void* k_dec, const void* v_dec,
                           const int32_t* page_table, const int32_t* sel_idx, const int32_t* n_sel,
                           int32_t max_sel, int32_t sel_unit_tokens, void* out) {
  return attn_common(h, g, q, k_cache, v_cache, k_dec, v_dec, page_table, sel_idx, n_sel, max_sel,
                     sel_unit_tokens, 0, out);
}

fdl_status fdl_dense_attn(fdl_handle h, const fdl_geom* g, const void* q, const void* k_cache,
                          const void* v_cache, const void* k_dec, const void* v_dec,
                          const int32_t* page_table, void* out) {
  return attn_common(h, g, q, k_cache, v_cache, k_dec, v_dec, page_table, nullptr, nullptr, 0, 1, 1, out);
}

// One denoising step over the layer table; dry: validate only (nothing is launched).
static fdl_status focus_step_impl(fdl_handle h, const fdl_geom* gp, const fdl_focus_params* fp,
                                  const float* prev_conf, const uint8_t* masked, int32_t n_layers,
                                  const fdl_layer_io* layers, uint64_t* pred_mask, int32_t* n_pred,
                                  float* scores, int32_t* sink_pos, int32_t* n_sinks, int32_t* sel_idx,
                                  int32_t* n_sel, bool dry) {
  if (!h) return FDL_EINVAL;
  Geom g;
  fdl_status st = check_geom(h, gp, g);
  if (st != FDL_OK) return st;
  if (!fp || !masked || !pred_mask || !n_pred || n_layers < 0 || (n_layers > 0 && !layers))
    return fail(h, FDL_EINVAL, "params, masked, pred_mask, n_pred and layers must be non-NULL");
  if (g.paged) return fail(h, FDL_EUNSUPPORTED, "fdl_focus_step runs contiguous caches");
  if (g.dtype == FDL_BF16 && g.T > 32) return fail(h, FDL_EUNSUPPORTED, "bf16 attention needs dec_len <= 32");
  if (fp->top_k_pos < 0 || fp->window < 0 || fp->top_k_blocks < 0)
    return fail(h, FDL_EINVAL, "top_k_pos, window and top_k_blocks must be >= 0");
  const int n_blk = (g.L + g.bt - 1) / g.bt;
  const int bt_log2 = ilog2(g.bt);
  bool any_sparse = false;
  const fdl_layer_io* first_source = nullptr;
  for (int l = 0; l < n_layers; ++l) {
    const fdl_layer_io& io = layers[l];
    if (io.mode < FDL_LAYER_DENSE || io.mode > FDL_LAYER_REUSE) return fail(h, FDL_EINVAL, "layer %d: bad mode", l);
    if (!io.q || !io.k_dec || !io.v_dec || !io.out || (g.L > 0 && (!io.k_cache || !io.v_cache)))
      return fail(h, FDL_EINVAL, "layer %d: NULL tensor", l);
    if (io.mode != FDL_LAYER_DENSE) {
      any_sparse = true;
      if (!io.ks) return fail(h, FDL_EINVAL, "layer %d: sparse layer needs ks", l);
    }
    if (io.mode == FDL_LAYER_SOURCE && !first_source) first_source = &io;
  }
  int ns = 0, cap = 0;
  if (any_sparse) {
    if (!scores || !sel_idx || !n_sel || !sink_pos || !n_sinks)
      return fail(h, FDL_EINVAL, "sparse layers need scores, sink_pos, n_sinks, sel_idx and n_sel");
    if (n_blk > 8192) return fail(h, FDL_EUNSUPPORTED, "more than 8192 KV blocks");
    if (fp->max_sinks < 1) return fail(h, FDL_EINVAL, "max_sinks must be >= 1");
    long long need = (long long)fp->max_sinks + fp->top_k_blocks;
    if (need > n_blk) need = n_blk;
    if (fp->max_sel < 1 || need > fp->max_sel)
      return fail(h, FDL_EINVAL, "max_sel must cover min(n_blk, max_sinks + top_k_blocks)");
  }
  if (first_source) {
    st = check_sinks(h, g, first_source->k_cache, first_source->k_dec, fp->sink_tau, fp->max_sinks,
                     sink_pos, n_sinks, &ns, &cap);
    if (st != FDL_OK) return st;
  }
  if (dry) return FDL_OK;
  // The prediction is first read by the first layer that is not dense.  When that layer detects the
  // sinks, the sink scan computes the prediction itself (one launch fewer per step); otherwise it
  // runs first, on its own.
  int first_sparse = n_layers;
  for (int l = 0; l < n_layers; ++l)
    if (layers[l].mode != FDL_LAYER_DENSE) {
      first_sparse = l;
      break;
    }
  const bool pred_in_sinks = first_sparse < n_layers && layers[first_sparse].mode == FDL_LAYER_SOURCE;
  const fdl::PredictIn pin{prev_conf, masked, fp->top_k_pos, fp->window, pred_mask, n_pred};
  if (!pred_in_sinks) {
    st = run_predict(h, g.B, g.T, prev_conf, masked, fp->top_k_pos, fp->window, pred_mask, n_pred);
    if (st != FDL_OK) return st;
  }
  // runs of consecutive reuse layers, bracketed by one pair of events when FDL_PROF_REUSE_RUN is on
  hipEvent_t run_a = nullptr, run_b = nullptr;
  int run_n = 0;
  auto run_end = [&]() {
    if (run_a) {
      (void)hipEventRecord(run_b, h->stream);
      h->prof_recs.push_back({FDL_PROF_REUSE_RUN, run_a, run_b, run_n});
    }
    run_a = run_b = nullptr;
    run_n = 0;
  };
  // The sink detection's bitmap goes straight to the fused kernel of the detecting layer, which forces
  // the units of its first max_sinks positions and writes the list (no compaction launch), when it
  // sits in the handle's header and fits the kernel's read; the next fused layer clears it (or a
  // fill, before another detection or at the end of the step).
  int bm_words = 0;
  uint32_t* bm = fdl::sink_bitmap_for(g, h->sink_area, &bm_words);
  if (bm_words > fdl::kFusedSinkWords) bm = nullptr;
  bool bm_pending = false;   // bm holds the last detection's bits
  auto bm_fill = [&]() -> fdl_status {
    bm_pending = false;
    return hip_status(h, fdl::launch_fill_u32(h->stream, bm, (size_t)g.B * bm_words, 0u), "sink bitmap clear");
  };
  for (int l = 0; l < n_layers; ++l) {
    const fdl_layer_io& io = layers[l];
    if (io.mode == FDL_LAYER_REUSE) {
      if (run_n == 0 && h->prof_on && ((h->prof_mask >> FDL_PROF_REUSE_RUN) & 1u) &&
          (h->prof_seen[FDL_PROF_REUSE_RUN]++ % h->prof_every) == 0 && h->prof_used + 2 <= h->prof_pool.size()) {
        run_a = h->prof_pool[h->prof_used++];
        run_b = h->prof_pool[h->prof_used++];
        (void)hipEventRecord(run_a, h->stream);
      }
      ++run_n;
    } else if (run_n > 0) {
      run_end();
    }
    const int kind = io.mode == FDL_LAYER_DENSE ? FDL_PROF_LAYER_DENSE
                   : io.mode == FDL_LAYER_SOURCE ? FDL_PROF_LAYER_SOURCE : FDL_PROF_LAYER_REUSE;
    ProfScope layer_scope(h, kind);
    if (io.mode == FDL_LAYER_DENSE) {
      st = run_attn(h, g, io.q, io.k_cache, io.v_cache, io.k_dec, io.v_dec, nullptr, nullptr, nullptr, 0, 0,
                    1, io.out);
      if (st != FDL_OK) return st;
      continue;
    }
    const bool fused = fused_select_ok(g, n_blk, fp->max_sel, fp->max_sinks);
    const bool keep_bm = fused && bm != nullptr && io.mode == FDL_LAYER_SOURCE;
    if (io.mode == FDL_LAYER_SOURCE) {   // first: it may compute the prediction the scoring reads
      if (bm_pending) {   // a detection starts from a clear bitmap
        st = bm_fill();
        if (st != FDL_OK) return st;
      }
      st = run_sinks(h, g, io.q, pred_mask, io.k_cache, io.k_dec, fp->sink_tau, fp->max_sinks, sink_pos,
                     n_sinks, ns, cap, pred_in_sinks && l == first_sparse ? &pin : nullptr, keep_bm);
      if (st != FDL_OK) return st;
    }
    if (!fused) {
      st = run_score_units(h, g, io.q, pred_mask, io.ks, n_blk, bt_log2, scores);
      if (st != FDL_OK) return st;
    }
    if (fused) {
      SinkBitmapUse use;
      if (keep_bm) {
        use.read = bm;
        use.words = bm_words;
      } else if (bm_pending) {
        use.clear = bm;
        use.words = bm_words;
      }
      st = run_select_attn(h, g, io, pred_mask, fp, bt_log2, sink_pos, n_sinks, scores, sel_idx, n_sel, use);
      if (st != FDL_OK) return st;
      bm_pending = keep_bm;
      continue;
    }
    st = run_select(h, g, scores, n_blk, bt_log2, sink_pos, n_sinks, fp->max_sinks, nullptr, 0,
                    fp->top_k_blocks, 0, fp->max_sel, sel_idx, n_sel);
    if (st != FDL_OK) return st;
    st = run_attn(h, g, io.q, io.k_cache, io.v_cache, io.k_dec, io.v_dec, nullptr, sel_idx, n_sel,
                  fp->max_sel, bt_log2, 0, io.out, fp->top_k_blocks);
    if (st != FDL_OK) return st;
  }
  if (run_n > 0) run_end();
  if (bm_pending) return bm_fill();
  return FDL_OK;
}

fdl_status fdl_focus_step(fdl_handle h, const fdl_geom* gp, const fdl_focus_params* fp,
                          const float* prev_conf, const uint8_t* masked, int32_t n_layers,
                          const fdl_layer_io* layers, uint64_t* pred_mask, int32_t* n_pred,
                          float* scores, int32_t* sink_pos, int32_t* n_sinks, int32_t* sel_idx,
                          int32_t* n_sel) {
  return focus_step_impl(h, gp, fp, prev_conf, masked, n_layers, layers, pred_mask, n_pred, scores, sink_pos,
                         n_sinks, sel_idx, n_sel, false);
}

// ---- the decode loop: the unmask update, several steps in one call, graph capture -------------

static fdl_status check_unmask(fdl_handle h, int32_t batch, int32_t dec_len, const float* conf,
                               const uint8_t* masked, int32_t n_unmask) {
  if (batch < 1) return fail(h, FDL_EINVAL, "batch must be >= 1");
  if (dec_len < 1 || dec_len > 64) return fail(h, FDL_EINVAL, "dec_len must be in [1, 64]");
  if (n_unmask < 0 || n_unmask > 64) return fail(h, FDL_EINVAL, "n_unmask must be in [0, 64]");
  if (!conf || !masked) return fail(h, FDL_EINVAL, "conf and masked must be non-NULL");
  return FDL_OK;
}

fdl_status fdl_unmask(fdl_handle h, int32_t batch, int32_t dec_len, const float* conf, uint8_t* masked,
                      int32_t n_unmask, int32_t* decoded) {
  if (!h) return FDL_EINVAL;
  fdl_status st = check_unmask(h, batch, dec_len, conf, masked, n_unmask);
  if (st != FDL_OK) return st;
  return hip_status(h, fdl::launch_unmask(h->stream, batch, dec_len, conf, masked, n_unmask, decoded),
                    "unmask launch");
}

fdl_status fdl_decode_steps(fdl_handle h, const fdl_geom* gp, const fdl_focus_params* fp, int32_t n_steps,
                            const float* prev_conf0, const float* conf, uint8_t* masked, int32_t n_unmask,
                            int32_t* decoded, int32_t n_layers, const fdl_layer_io* layers,
                            uint64_t* pred_mask, int32_t* n_pred, float* scores, int32_t* sink_pos,
                            int32_t* n_sinks, int32_t* sel_idx, int32_t* n_sel) {
  if (!h) return FDL_EINVAL;
  if (n_steps < 0) return fail(h, FDL_EINVAL, "n_steps must be >= 0");
  if (n_steps == 0) return FDL_OK;
  if (!gp) return fail(h, FDL_EINVAL, "geometry must be non-NULL");
  if (n_layers > 0 && !layers) return fail(h, FDL_EINVAL, "layers must be non-NULL");
  fdl_status st = check_unmask(h, gp->batch, gp->dec_len, conf, masked, n_unmask);
  if (st != FDL_OK) return st;
  const int64_t bt = (int64_t)gp->batch * gp->dec_len;
  for (int s = 0; s < n_steps; ++s) {   // every step's table first: nothing runs unless all are valid
    st = focus_step_impl(h, gp, fp, s == 0 ? prev_conf0 : conf + (s - 1) * bt, masked, n_layers,
                         layers + (int64_t)s * n_layers, pred_mask, n_pred, scores, sink_pos, n_sinks, sel_idx,
                         n_sel, true);
    if (st != FDL_OK) return st;
  }
  for (int s = 0; s < n_steps; ++s) {
    st = focus_step_impl(h, gp, fp, s == 0 ? prev_conf0 : conf + (s - 1) * bt, masked, n_layers,
                         layers + (int64_t)s * n_layers, pred_mask, n_pred, scores, sink_pos, n_sinks, sel_idx,
                         n_sel, false);
    if (st != FDL_OK) return st;
    st = hip_status(h, fdl::launch_unmask(h->stream, gp->batch, gp->dec_len, conf + s * bt, masked, n_unmask,
                                          decoded ? decoded + (int64_t)s * gp->batch * n_unmask : nullptr),
                    "unmask launch");
    if (st != FDL_OK) return st;
  }
  return FDL_OK;
}

struct fdl_graph_s {
  hipGraph_t graph;
  hipGraphExec_t exec;
};

fdl_status fdl_capture_begin(fdl_handle h) {
  if (!h) return FDL_EINVAL;
  if (h->capturing) return fail(h, FDL_EINVAL, "already capturing");
  if (h->prof_on) return fail(h, FDL_EINVAL, "profiling is on: end it before capturing");
  if (h->stream == nullptr) return fail(h, FDL_EINVAL, "the null stream cannot be captured: set another stream");
  fdl_status st = hip_status(h, hipStreamBeginCapture(h->stream, hipStreamCaptureModeThreadLocal),
                             "hipStreamBeginCapture");
  if (st == FDL_OK) h->capturing = true;
  return st;
}

fdl_status fdl_capture_end(fdl_handle h, fdl_graph* out) {
  if (!h) return FDL_EINVAL;
  if (!out) return fail(h, FDL_EINVAL, "out must be non-NULL");
  *out = nullptr;
  if (!h->capturing) return fail(h, FDL_EINVAL, "not capturing");
  h->capturing = false;
  hipGraph_t graph = nullptr;
  fdl_status st = hip_status(h, hipStreamEndCapture(h->stream, &graph), "hipStreamEndCapture");
  if (st != FDL_OK) return st;
  hipGraphExec_t exec = nullptr;
  st = hip_status(h, hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0), "hipGraphInstantiate");
  if (st != FDL_OK) {
    (void)hipGraphDestroy(graph);
    return st;
  }
  fdl_graph g = new (std::nothrow) fdl_graph_s{graph, exec};
  if (!g) {
    (void)hipGraphExecDestroy(exec);
    (void)hipGraphDestroy(graph);
    return fail(h, FDL_ENOMEM, "out of host memory");
  }
  *out = g;
  return FDL_OK;
}

fdl_status fdl_graph_launch(fdl_handle h, fdl_graph g) {
  if (!h) return FDL_EINVAL;
  if (!g) return fail(h, FDL_EINVAL, "graph must be non-NULL");
  if (h->capturing) return fail(h, FDL_EINVAL, "the handle's stream is being captured");
  return hip_status(h, hipGraphLaunch(g->exec, h->stream), "hipGraphLaunch");
}

fdl_status fdl_graph_destroy(fdl_graph g) {
  if (!g) return FDL_OK;
  (void)hipGraphExecDestroy(g->exec);
  (void)hipGraphDestroy(g->graph);
  delete g;
  return FDL_OK;
}

fdl_status fdl_bandwidth_probe(fdl_handle h, int32_t mode, const void* src, size_t bytes, void* dst,
                               size_t dst_bytes, int32_t n_blocks) {
  if (!h) return FDL_EINVAL;
  if (mode < FDL_PROBE_READ || mode > FDL_PROBE_TILES) return fail(h, FDL_EINVAL, "unknown probe mode");
  if (!src || !dst) return fail(h, FDL_EINVAL, "src and dst must be non-NULL");
  if (bytes == 0 || bytes % 1024) return fail(h, FDL_EINVAL, "bytes must be a positive multiple of 1024");
  if (n_blocks < 0) return fail(h, FDL_EINVAL, "n_blocks must be >= 0");
  const int nb = n_blocks > 0 ? n_blocks : (mode == FDL_PROBE_TILES ? h->num_cus : 4 * h->num_cus);
  if (mode == FDL_PROBE_TILES && fdl::probe_tile_region(bytes, nb) == 0)
    return fail(h, FDL_EINVAL, "bytes too small for %d workgroups of 16 KiB tiles", nb);
  const size_t need = mode == FDL_PROBE_COPY ? bytes : fdl::probe_out_words(nb) * sizeof(uint32_t);
  if (dst_bytes < need) return fail(h, FDL_EINVAL, "dst holds %zu bytes, needs %zu", dst_bytes, need);
  return hip_status(h, fdl::launch_probe(h->stream, mode, src, bytes, dst, nb), "probe launch");
}

fdl_status fdl_set_phase_buffer(fdl_handle h, uint64_t* stamps, int64_t n_words) {
  if (!h) return FDL_EINVAL;
  if ((stamps == nullptr) != (n_words == 0) || n_words < 0)
    return fail(h, FDL_EINVAL, "stamps and n_words go together");
  h->stamps = stamps;
  h->stamp_words = n_words;
  return FDL_OK;
}

int32_t fdl_phase_stamps_built(void) {
#ifdef FDL_PHASE_STAMPS
  return 1;
#else
  return 0;
#endif
}

fdl_status fdl_profile_begin(fdl_handle h, int32_t max_records, uint32_t kind_mask, int32_t every) {
  if (!h || max_records < 1) return h ? fail(h, FDL_EINVAL, "max_records must be >= 1") : FDL_EINVAL;
  if (h->capturing) return fail(h, FDL_EINVAL, "the handle's stream is being captured");
  if (every < 1) return fail(h, FDL_EINVAL, "every must be >= 1");
  for (hipEvent_t e : h->prof_pool) (void)hipEventDestroy(e);
  h->prof_pool.clear();
  h->prof_recs.clear();
  h->prof_used = 0;
  h->prof_pool.reserve((size_t)2 * max_records);
  h->prof_recs.reserve((size_t)max_records);
  for (int i = 0; i < 2 * max_records; ++i) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) {
      for (hipEvent_t x : h->prof_pool) (void)hipEventDestroy(x);
      h->prof_pool.clear();
      return fail(h, FDL_EHIP, "hipEventCreate failed");
    }
    h->prof_pool.push_back(e);
  }
  h->prof_on = true;
  h->prof_mask = kind_mask;
  h->prof_every = every;
  for (int k = 0; k < FDL_PROF_KINDS; ++k) h->prof_seen[k] = 0;
  return FDL_OK;
}

fdl_status fdl_profile_end(fdl_handle h, double* total_us, int64_t* counts) {
  if (!h) return FDL_EINVAL;
  if (!total_us || !counts) return fail(h, FDL_EINVAL, "total_us and counts must be non-NULL");
  if (h->capturing) return fail(h, FDL_EINVAL, "the handle's stream is being captured");
  fdl_status st = hip_status(h, hipStreamSynchronize(h->stream), "hipStreamSynchronize");
  for (int k = 0; k < FDL_PROF_KINDS; ++k) {
    total_us[k] = 0.0;
    counts[k] = 0;
  }
  if (st == FDL_OK) {
    for (const auto& r : h->prof_recs) {
      float ms = 0.f;
      if (hipEventElapsedTime(&ms, r.a, r.b) == hipSuccess && r.kind >= 0 && r.kind < FDL_PROF_KINDS) {
        total_us[r.kind] += 1000.0 * ms;
        counts[r.kind] += r.n;
      }
    }
  }
  for (hipEvent_t e : h->prof_pool) (void)hipEventDestroy(e);
  h->prof_pool.clear();
  h->prof_recs.clear();
  h->prof_used = 0;
  h->prof_on = false;
  return st;
}

}  // extern "C"
