// Level 2 of the chunked, paged variant in one kernel: token scores inside each chosen chunk and the
// selection of the chunk's anchor plus its top-K other tokens.
//
// Prefilling-dLLM (abstract): after the top chunks are chosen, token-level sparsity inside each chunk
// keeps the most relevant tokens of non-contiguously cached KV; the chunk's leading token serves as
// an anchor and is always kept.  Same outputs, bit for bit, as score_tokens_kernel followed by
// select_kernel at level 2: the scores use the pinned query sum and row dot of fdl_score.h, the
// selection is select_core (fdl_select.h).
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

template <int D, bool PAGED>
__global__ __launch_bounds__(kTsThreads, 2) void score_select_tokens_kernel(
    const uint16_t* __restrict__ q, const uint64_t* __restrict__ pred_mask, const uint16_t* __restrict__ k,
    KvRows<PAGED> rows, int Hq, int G, int T, int unit_log2, const int32_t* __restrict__ cand_idx, int n_cand,
    int top_k, int max_sel, float* __restrict__ scores, int32_t* __restrict__ sel_idx,
    int32_t* __restrict__ n_sel, uint32_t* __restrict__ status) {
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
  const int u = cand_idx[seg * n_cand + c];
  const bool uok = (unsigned)u < (unsigned)n_units;   // uniform
  const int tok0 = uok ? u << unit_log2 : 0;
  bool bad = !uok;

  // loads in the order they are needed: the group's query rows, the chunk's page entries, the
  // first batch of K rows
  QsumGrouped<D, 32, NT, 8> qst;
  qsum_grouped_issue<D, 32, NT, 8>(q + (int64_t)b * Hq * T * D, g * G, G, T, qst);
  const int pg0 = PAGED ? tok0 >> rows.page_log2 : 0;
  const int n_pg = PAGED ? ((tok0 + n - 1) >> rows.page_log2) - pg0 + 1 : 0;
  int my_page = 0;
  if (PAGED) {
    const int i = tid < n_pg ? tid : 0;
    my_page = rows.page_table[(int64_t)b * rows.pages_per_seq + pg0 + i];
  }
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
  if (PAGED && tid < n_pg) s_pages[tid] = my_page;
  qsum_grouped_finish<D, 32, NT, 8>(qst, pred_mask[b], G, T, big, qs);   // one barrier inside
  __syncthreads();   // qs, the page entries and the forced bits; the stage is free again

  float qv[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) qv[i] = qs[16 * j + i];
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
  for (int bt = 0; bt < nb; bt += 2) {
    issue(bt + 1 < nb ? bt + 1 : nb - 1, kb, okb);
    consume(bt, ka, oka);
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

  const int nf = 1;   // the anchor
  const int per_seg = nf + (top_k < n - nf ? top_k : n - nf);
  int32_t* out = sel_idx + seg * (int64_t)max_sel + (int64_t)c * per_seg;
  const SelScratch scr{hist, tmp};
  const SelResult r = select_core<NT, kTsMaxUnit / NT>(keys, forced, n, top_k, scr, [&](int pos, int i) {
    out[pos] = uok ? tok0 + i : -1;
  });
  if (tid == 0 && c == 0) n_sel[seg] = n_cand * (nf + r.kk);
}

template <int D, bool PAGED>
static hipError_t launch_sst(hipStream_t s, const Geom& g, const uint16_t* q, const uint64_t* pm,
                             const uint16_t* k, const int32_t* page_table, int unit_log2,
                             const int32_t* cand_idx, int n_cand, int top_k, int max_sel, float* scores,
                             int32_t* sel_idx, int32_t* n_sel, uint32_t* status) {
  KvRows<PAGED> rows;
  rows.Hkv = g.Hkv;
  rows.L = g.L;
  rows.D = D;
  rows.page_log2 = g.page_log2;
  rows.pages_per_seq = g.pps;
  rows.n_pages = g.n_pages;
  rows.page_table = page_table;
  hipLaunchKernelGGL((score_select_tokens_kernel<D, PAGED>), dim3(n_cand, g.Hkv, g.B), dim3(kTsThreads), 0, s, q,
                     pm, k, rows, g.Hq, g.G, g.T, unit_log2, cand_idx, n_cand, top_k, max_sel, scores, sel_idx,
                     n_sel, status);
  return hipGetLastError();
}

bool score_select_tokens_ok(const Geom& g, int unit_log2) {
  // chunks of 256 to 4096 tokens start on a page boundary when pages are no longer than a chunk,
  // so a chunk spans at most 4096 / 16 = 256 page entries
  return g.dtype == FDL_BF16 && g.T <= 32 && (g.D == 128 || g.D == 64) && unit_log2 <= 12 &&
         (1 << unit_log2) >= kTsBatchRows && (!g.paged || (1 << g.page_log2) >= kTsMinPage);
}

hipError_t launch_score_select_tokens(hipStream_t s, const Geom& g, const void* q, const uint64_t* pred_mask,
                                      const void* k, const int32_t* page_table, int unit_log2,
                                      const int32_t* cand_idx, int n_cand, int top_k, int max_sel,
                                      float* scores, int32_t* sel_idx, int32_t* n_sel, uint32_t* status) {
  if (!score_select_tokens_ok(g, unit_log2)) return hipErrorInvalidValue;
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint16_t* kk = static_cast<const uint16_t*>(k);
  if (g.D == 128)
    return g.paged ? launch_sst<128, true>(s, g, qq, pred_mask, kk, page_table, unit_log2, cand_idx, n_cand, top_k,
                                           max_sel, scores, sel_idx, n_sel, status)
                   : launch_sst<128, false>(s, g, qq, pred_mask, kk, page_table, unit_log2, cand_idx, n_cand, top_k,
                                            max_sel, scores, sel_idx, n_sel, status);
  return g.paged ? launch_sst<64, true>(s, g, qq, pred_mask, kk, page_table, unit_log2, cand_idx, n_cand, top_k,
                                        max_sel, scores, sel_idx, n_sel, status)
                 : launch_sst<64, false>(s, g, qq, pred_mask, kk, page_table, unit_log2, cand_idx, n_cand, top_k,
                                         max_sel, scores, sel_idx, n_sel, status);
}

}  // namespace fdl
