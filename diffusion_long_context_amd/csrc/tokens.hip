// Level 2 of the chunked, paged variant in one kernel: token scores inside each chosen chunk and the
// selection of the chunk's anchor plus its top-K other tokens.
//
// Prefilling-dLLM (abstract): after the top chunks are chosen, token-level sparsity inside each chunk
// keeps the most relevant tokens of non-contiguously cached KV; the chunk's leading token serves as
// an anchor and is always kept.  Same outputs, bit for bit, as score_tokens_kernel followed by
// select_kernel at level 2: the scores use the pinned query sum and row dot of fdl_score.h, the
// selection is select_core (fdl_select.h).
//
// With CHOOSE, level 1 runs in the same launch: every workgroup of a (sequence, KV head) scores its
// chunks against the same pinned query sum (the chunk sums' rows, as score_units_kernel does) and
// ranks them (key descending, ties to the lower chunk), exactly as fdl_select_blocks at level 1 with
// no sinks; slot c then takes the c-th chosen chunk in ascending order, and slot 0 writes the chunk
// scores and the chosen list.  Two launches and their round trips fewer than the three-call chain.
//
// One workgroup per (sequence, KV head, chosen chunk).  The chunk's page-table entries are read once
// into LDS, so every row address is known without a dependent load; the chunk's K rows then stream
// in batches of 256 rows, the next batch's loads in flight while the current one is scored (the last
// iteration re-requests its own rows, which L2 still holds, so no load sits under a branch).  Scores
// go to the scores output and, as order keys, to LDS, where the selection runs without another
// round trip through memory.
#include "fdl_device.h"
#include "fdl_internal.h"
#include "fdl_score.h"
#include "fdl_select.h"

namespace fdl {

constexpr int kTsThreads = 256;
constexpr int kTsMaxUnit = 4096;       // tokens per chunk (the level-2 bound of the API)
constexpr int kTsBatchRows = 256;      // rows per streaming batch
constexpr int kTsMinPage = 16;         // smallest page (tokens) this kernel takes
constexpr int kTsMaxPages = kTsThreads;   // page entries of one chunk: at most 4096 / 16 = 256

constexpr int kTsMaxChunks = 64;      // chunks per sequence when level 1 runs in the same launch

// Level 1 inside the level-2 launch (CHOOSE): chunk_sums [B][Hkv][n_chunks][D] float32, outputs
// chunk_scores [B][Hkv][n_chunks], the chosen chunks [B][Hkv][n_cand] ascending and their count.
struct ChunkChoice {
  const float* chunk_sums;
  float* chunk_scores;
  int32_t* chunks;
  int32_t* n_chunks_sel;
  int n_chunks;
  uint64_t* stamps;   // diagnostic build: per-workgroup phase timestamps, or NULL
};

// Diagnostic build (FDL_PHASE_STAMPS): thread 0 of each workgroup records s_memrealtime (100 MHz);
// nothing in the normal build.
#ifdef FDL_PHASE_STAMPS
#define TS_STAMP(cc, i)                                                                                \
  do {                                                                                                 \
    if (threadIdx.x == 0 && (cc).stamps != nullptr)                                                    \
      (cc).stamps[(((int64_t)blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x) * 16 + (i)] = \
          __builtin_amdgcn_s_memrealtime() | ((uint64_t)1 << 63);                                      \
  } while (0)
#else
#define TS_STAMP(cc, i) \
  do {                  \
  } while (0)
#endif

template <int D, bool PAGED, bool CHOOSE>
__global__ __launch_bounds__(kTsThreads, 2) void score_select_tokens_kernel(
    const uint16_t* __restrict__ q, const uint64_t* __restrict__ pred_mask, const uint16_t* __restrict__ k,
    KvRows<PAGED> rows, int Hq, int G, int T, int unit_log2, const int32_t* __restrict__ cand_idx, int n_cand,
    int top_k, int max_sel, float* __restrict__ scores, int32_t* __restrict__ sel_idx,
    int32_t* __restrict__ n_sel, uint32_t* __restrict__ status, const ChunkChoice cc) {
  constexpr int NT = kTsThreads;
  constexpr int LPR = D / 16;           // lanes per row, 16 dimensions each
  constexpr int RPW = 64 / LPR;         // rows per wave and pass
  constexpr int RPP = 4 * RPW;          // rows per pass
  constexpr int PB = kTsBatchRows / RPP;
  constexpr int STAGE = 8 * 32 * D;     // grouped query staging (bf16 elements)
  static_assert(STAGE * 2 >= kTsMaxUnit * 4, "the keys reuse the query staging");
  __shared__ __attribute__((aligned(16))) uint16_t big[STAGE];   // query stage, then the order keys
  __shared__ uint32_t forced[kTsMaxUnit / 32];
  __shared__ int hist[4 * 256];
  __shared__ int tmp[NT / 64];
  __shared__ float qs[D];
  __shared__ int32_t s_pages[kTsMaxPages];

  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane % LPR;
  const int n = 1 << unit_log2;
  const int n_units = rows.L >> unit_log2;   // ctx_len is a multiple of the unit
  const int64_t seg = (int64_t)b * rows.Hkv + g;
  TS_STAMP(cc, 0);
  __shared__ uint32_t s_ck[CHOOSE ? kTsMaxChunks : 1];   // level 1: the chunks' order keys
  __shared__ int s_u;

  // loads in the order they are needed: the group's query rows (with CHOOSE, then the chunk sums'
  // rows), the chunk's page entries, the first batch of K rows
  // one query head per KV head: its 32 rows alone (the grouped loader would fetch them once per
  // possible head); the same tree, so the same bits
  QsumGrouped<D, 32, NT, 8> qst;
  QsumG1<D, 32, NT> qs1;
  if (G == 1) qsum_g1_issue<D, 32, NT>(q + (seg * T) * D, T, qs1);   // uniform
  else qsum_grouped_issue<D, 32, NT, 8>(q + (int64_t)b * Hq * T * D, g * G, G, T, qst);
  constexpr int CP = CHOOSE ? kTsMaxChunks / RPP : 1;   // level-1 row passes
  float xc[CP][16];
  if constexpr (CHOOSE) {
#pragma unroll
    for (int ps = 0; ps < CP; ++ps) {
      int r = ps * RPP + wave * RPW + lane / LPR;
      r = r < cc.n_chunks ? r : cc.n_chunks - 1;
      load16<float>(cc.chunk_sums + (seg * cc.n_chunks + r) * D + 16 * j, xc[ps]);
    }
  }
  int u = 0;
  if constexpr (!CHOOSE) u = cand_idx[seg * n_cand + c];
  // with CHOOSE, the sequence's page entries (up to two per thread) are read now, so that the chosen
  // chunk's are at hand without a round trip after level 1
  constexpr int kPrePages = 2 * NT;
  const bool pre_pages = CHOOSE && PAGED && rows.pages_per_seq <= kPrePages;   // uniform
  int pp0 = 0, pp1 = 0;
  if (pre_pages) {
    const int32_t* ptb = rows.page_table + (int64_t)b * rows.pages_per_seq;
    pp0 = ptb[tid < rows.pages_per_seq ? tid : 0];
    pp1 = ptb[tid + NT < rows.pages_per_seq ? tid + NT : 0];
  }
  // the chunk's page entries (with CHOOSE and a page table too long to read early, once level 1
  // has chosen the chunk)
  auto page_loads = [&](int tok0_, int& pg0_, int& n_pg_, int& my_page_) {
    pg0_ = PAGED ? tok0_ >> rows.page_log2 : 0;
    n_pg_ = PAGED ? ((tok0_ + n - 1) >> rows.page_log2) - pg0_ + 1 : 0;
    my_page_ = 0;
    if (PAGED) {
      const int i = tid < n_pg_ ? tid : 0;
      my_page_ = rows.page_table[(int64_t)b * rows.pages_per_seq + pg0_ + i];
    }
  };
  bool uok = (unsigned)u < (unsigned)n_units;   // uniform
  int tok0 = uok ? u << unit_log2 : 0;
  int pg0 = 0, n_pg = 0, my_page = 0;
  if constexpr (!CHOOSE) page_loads(tok0, pg0, n_pg, my_page);
  // row offset of chunk row r (element units); invalid rows read row 0 of the pool and score -inf
  auto row_off = [&](int r, bool& ok) -> int64_t {
    const int t = tok0 + r;
    if constexpr (PAGED) {
      const int pp = s_pages[(t >> rows.page_log2) - pg0];
      ok = uok && (unsigned)pp < (unsigned)rows.n_pages;
      const int64_t pg = ok ? pp : 0;
      return (((pg * rows.Hkv + g) << rows.page_log2) | (int64_t)(t & ((1 << rows.page_log2) - 1))) * D;
    } else {
      ok = uok;
      return (seg * rows.L + t) * D;
    }
  };

  for (int i = tid; i < kTsMaxUnit / 32; i += NT) forced[i] = (i == 0) ? 1u : 0u;   // the anchor
  if (!CHOOSE && PAGED && tid < n_pg) s_pages[tid] = my_page;
  if (G == 1) qsum_g1_finish<D, 32, NT>(qs1, pred_mask[b], T, reinterpret_cast<float*>(big), qs);
  else qsum_grouped_finish<D, 32, NT, 8>(qst, pred_mask[b], G, T, big, qs);   // barriers inside
  __syncthreads();   // qs, the page entries and the forced bits; the stage is free again

  TS_STAMP(cc, 1);
  float qv[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) qv[i] = qs[16 * j + i];
  if constexpr (CHOOSE) {
    // level 1: the chunk scores (slot 0 writes them), then the rank of every chunk in one wave
#pragma unroll
    for (int ps = 0; ps < CP; ++ps) {
      const int r = ps * RPP + wave * RPW + lane / LPR;
      const float sc = row_dot<LPR>(xc[ps], qv);
      if (j == 0 && r < cc.n_chunks) {
        s_ck[r] = order_key(sc);
        if (c == 0) cc.chunk_scores[seg * cc.n_chunks + r] = sc;
      }
    }
    block_sync_lds();
    if (wave == 0) {
      const bool v = lane < cc.n_chunks;
      const uint32_t key = v ? s_ck[lane] : 0u;
      int rank = 0;
      for (int i = 0; i < cc.n_chunks; ++i) {   // uniform; ties go to the lower chunk
        const uint32_t ki = s_ck[i];
        rank += (ki > key || (ki == key && i < lane)) ? 1 : 0;
      }
      const bool chosen = v && rank < n_cand;
      const uint64_t cm = __ballot(chosen);
      if (chosen) {
        const int pos = __popcll(cm & ((1ull << lane) - 1ull));
        if (pos == c) s_u = lane;
        if (c == 0) cc.chunks[seg * n_cand + pos] = lane;
      }
      if (c == 0 && lane == 0) cc.n_chunks_sel[seg] = n_cand;
    }
    block_sync_lds();
    u = __builtin_amdgcn_readfirstlane(s_u);
    uok = (unsigned)u < (unsigned)n_units;
    tok0 = uok ? u << unit_log2 : 0;
    if (pre_pages) {
      pg0 = tok0 >> rows.page_log2;
      n_pg = ((tok0 + n - 1) >> rows.page_log2) - pg0 + 1;
      if (tid >= pg0 && tid < pg0 + n_pg) s_pages[tid - pg0] = pp0;
      if (tid + NT >= pg0 && tid + NT < pg0 + n_pg) s_pages[tid + NT - pg0] = pp1;
      my_page = 0;   // the range check of the entries reads them back from LDS below
    } else {
      page_loads(tok0, pg0, n_pg, my_page);
      if (PAGED && tid < n_pg) s_pages[tid] = my_page;
    }
    if (PAGED) block_sync_lds();   // the page entries, for every row
    if (pre_pages && tid < n_pg) my_page = s_pages[tid];
  }
  TS_STAMP(cc, 2);
  bool bad = !uok;
  uint32_t* keys = reinterpret_cast<uint32_t*>(big);
  float* sc_out = scores + (seg * n_cand + c) * (int64_t)n;
  const int nb = (n + kTsBatchRows - 1) / kTsBatchRows;

  uint4 ka[PB][2], kb[PB][2];
  bool oka[PB], okb[PB];
  auto issue = [&](int bt, uint4 (&dst)[PB][2], bool (&okd)[PB]) {
#pragma unroll
    for (int ps = 0; ps < PB; ++ps) {
      int r = bt * kTsBatchRows + ps * RPP + wave * RPW + lane / LPR;
      const bool in = r < n;
      r = in ? r : n - 1;
      bool ok;
      const int64_t off = row_off(r, ok);
      okd[ps] = ok && in;
      const uint4* src = reinterpret_cast<const uint4*>(k + off + 16 * j);
      dst[ps][0] = src[0];
      dst[ps][1] = src[1];
    }
  };
  auto consume = [&](int bt, const uint4 (&src)[PB][2], const bool (&okd)[PB]) {
#pragma unroll
    for (int ps = 0; ps < PB; ++ps) {
      const int r = bt * kTsBatchRows + ps * RPP + wave * RPW + lane / LPR;
      float x[16];
      const uint32_t w[8] = {src[ps][0].x, src[ps][0].y, src[ps][0].z, src[ps][0].w,
                             src[ps][1].x, src[ps][1].y, src[ps][1].z, src[ps][1].w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        x[2 * i] = bf16_bits_to_f32(w[i] & 0xFFFFu);
        x[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
      }
      const float s = okd[ps] ? row_dot<LPR>(x, qv) : -__builtin_inff();
      if (j == 0 && r < n) {
        sc_out[r] = s;
        keys[r] = order_key(s);
      }
    }
  };
  issue(0, ka, oka);
  bool first = true;
  for (int bt = 0; bt < nb; bt += 2) {
    issue(bt + 1 < nb ? bt + 1 : nb - 1, kb, okb);
    consume(bt, ka, oka);
    if (first) TS_STAMP(cc, 3);
    first = false;
    issue(bt + 2 < nb ? bt + 2 : nb - 1, ka, oka);
    if (bt + 1 < nb) consume(bt + 1, kb, okb);   // uniform; no load inside
  }
  if (PAGED) {
    // a page entry of the chunk that is out of range (its rows scored -inf above)
    const bool pbad = uok && tid < n_pg && (unsigned)my_page >= (unsigned)rows.n_pages;
    bad = bad || pbad;
  }
  latch_bad(status, bad);
  block_sync_lds();   // every key
  TS_STAMP(cc, 4);

  const int nf = 1;   // the anchor
  const int per_seg = nf + (top_k < n - nf ? top_k : n - nf);
  int32_t* out = sel_idx + seg * (int64_t)max_sel + (int64_t)c * per_seg;
  const SelScratch scr{hist, tmp};
  const SelResult r = select_core<NT, kTsMaxUnit / NT>(keys, forced, n, top_k, scr, [&](int pos, int i) {
    out[pos] = uok ? tok0 + i : -1;
  });
  if (tid == 0 && c == 0) n_sel[seg] = n_cand * (nf + r.kk);
  TS_STAMP(cc, 5);
}

template <int D, bool PAGED, bool CHOOSE>
static hipError_t launch_sst(hipStream_t s, const Geom& g, const uint16_t* q, const uint64_t* pm,
                             const uint16_t* k, const int32_t* page_table, int unit_log2,
                             const int32_t* cand_idx, int n_cand, int top_k, int max_sel, float* scores,
                             int32_t* sel_idx, int32_t* n_sel, uint32_t* status, const ChunkChoice& cc) {
  KvRows<PAGED> rows;
  rows.Hkv = g.Hkv;
  rows.L = g.L;
  rows.D = D;
  rows.page_log2 = g.page_log2;
  rows.pages_per_seq = g.pps;
  rows.n_pages = g.n_pages;
  rows.page_table = page_table;
  hipLaunchKernelGGL((score_select_tokens_kernel<D, PAGED, CHOOSE>), dim3(n_cand, g.Hkv, g.B), dim3(kTsThreads), 0,
                     s, q, pm, k, rows, g.Hq, g.G, g.T, unit_log2, cand_idx, n_cand, top_k, max_sel, scores,
                     sel_idx, n_sel, status, cc);
  return hipGetLastError();
}

template <bool CHOOSE>
static hipError_t dispatch_sst(hipStream_t s, const Geom& g, const void* q, const uint64_t* pred_mask, const void* k,
                               const int32_t* page_table, int unit_log2, const int32_t* cand_idx, int n_cand,
                               int top_k, int max_sel, float* scores, int32_t* sel_idx, int32_t* n_sel,
                               uint32_t* status, const ChunkChoice& cc) {
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint16_t* kk = static_cast<const uint16_t*>(k);
  if (g.D == 128)
    return g.paged ? launch_sst<128, true, CHOOSE>(s, g, qq, pred_mask, kk, page_table, unit_log2, cand_idx, n_cand,
                                                   top_k, max_sel, scores, sel_idx, n_sel, status, cc)
                   : launch_sst<128, false, CHOOSE>(s, g, qq, pred_mask, kk, page_table, unit_log2, cand_idx, n_cand,
                                                    top_k, max_sel, scores, sel_idx, n_sel, status, cc);
  return g.paged ? launch_sst<64, true, CHOOSE>(s, g, qq, pred_mask, kk, page_table, unit_log2, cand_idx, n_cand,
                                                top_k, max_sel, scores, sel_idx, n_sel, status, cc)
                 : launch_sst<64, false, CHOOSE>(s, g, qq, pred_mask, kk, page_table, unit_log2, cand_idx, n_cand,
                                                 top_k, max_sel, scores, sel_idx, n_sel, status, cc);
}

bool score_select_tokens_ok(const Geom& g, int unit_log2) {
  // chunks of 256 to 4096 tokens start on a page boundary when pages are no longer than a chunk,
  // so a chunk spans at most 4096 / 16 = 256 page entries
  return g.dtype == FDL_BF16 && g.T <= 32 && (g.D == 128 || g.D == 64) && unit_log2 <= 12 &&
         (1 << unit_log2) >= kTsBatchRows && (!g.paged || (1 << g.page_log2) >= kTsMinPage);
}

bool select_chunks_tokens_ok(const Geom& g, int unit_log2, int n_chunks) {
  return score_select_tokens_ok(g, unit_log2) && g.G <= 8 && n_chunks >= 1 && n_chunks <= kTsMaxChunks;
}

hipError_t launch_score_select_tokens(hipStream_t s, const Geom& g, const void* q, const uint64_t* pred_mask,
                                      const void* k, const int32_t* page_table, int unit_log2,
                                      const int32_t* cand_idx, int n_cand, int top_k, int max_sel,
                                      float* scores, int32_t* sel_idx, int32_t* n_sel, uint32_t* status) {
  if (!score_select_tokens_ok(g, unit_log2)) return hipErrorInvalidValue;
  return dispatch_sst<false>(s, g, q, pred_mask, k, page_table, unit_log2, cand_idx, n_cand, top_k, max_sel, scores,
                             sel_idx, n_sel, status, ChunkChoice{nullptr, nullptr, nullptr, nullptr, 0, nullptr});
}

hipError_t launch_select_chunks_tokens(hipStream_t s, const Geom& g, const void* q, const uint64_t* pred_mask,
                                       const float* chunk_sums, const void* k, const int32_t* page_table,
                                       int unit_log2, int top_k_chunks, int top_k, int max_sel, float* chunk_scores,
                                       int32_t* chunks, int32_t* n_chunks_sel, float* scores, int32_t* sel_idx,
                                       int32_t* n_sel, uint32_t* status, uint64_t* stamps, int64_t stamp_words) {
  const int n_chunks = g.L >> unit_log2;
  if (!select_chunks_tokens_ok(g, unit_log2, n_chunks) || top_k_chunks < 1 || top_k_chunks > n_chunks)
    return hipErrorInvalidValue;
  const bool st_ok = stamps != nullptr && stamp_words >= (int64_t)top_k_chunks * g.Hkv * g.B * 16;
  const ChunkChoice cc{chunk_sums, chunk_scores, chunks, n_chunks_sel, n_chunks, st_ok ? stamps : nullptr};
  return dispatch_sst<true>(s, g, q, pred_mask, k, page_table, unit_log2, nullptr, top_k_chunks, top_k, max_sel,
                            scores, sel_idx, n_sel, status, cc);
}

}  // namespace fdl
