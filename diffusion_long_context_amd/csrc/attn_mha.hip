// Gathered block-sparse (or dense) bidirectional attention, bf16.
//
// Focus-dLLM (abstract; Elamur "Summary"): the block's queries attend bidirectionally over only the
// selected KV plus the block itself; Prefilling-dLLM (abstract): the same over chunk KV cached in
// non-contiguous pages.  The arithmetic is softmax(q k^T / sqrt(D)) v with an online softmax over
// 32-token tiles; the data movement is what this kernel is about.
//
// Layout of the work: one workgroup of 8 waves per (split, head, sequence); each wave streams its
// own 32-token tiles (tile 0 is the block's own tokens) through a private 16 KiB LDS slot:
//   1. the tile's K and V rows are fetched straight from HBM into LDS with global_load_lds_dwordx4
//      (no register staging): each instruction moves 1 KiB, 64 lanes x 16 bytes, and lane l's bytes
//      land at slot base + 16 l, so the lane -> global chunk map chooses the LDS layout; rows are
//      stored with their 16-byte chunks XOR-swizzled by the row index so that the MFMA operand reads
//      below are free of bank conflicts;
//   2. the wave copies the tile from LDS into registers in MFMA operand order (K as the A operand of
//      S^T = K Q^T; V read transposed as the A operand of O^T = V^T P^T);
//   3. it issues the next tile's fetch into the same slot, and only then computes on the registers,
//      so one tile per wave is always in flight while the MFMAs and the softmax run.
// An LDS read of the slot must follow a full vector-memory wait (the fetch only counts as done in
// vmcnt), which would also wait for a second buffer's fetch; hence the copy-to-registers step before
// the next fetch rather than double-buffering LDS.  The wait is written out at the top of the tile
// loop: the compiler's automatic one is not placed reliably across the back-edge.
// Softmax statistics stay in the lane that owns the query (S^T puts queries on lanes), so one
// cross-lane exchange per tile suffices.  At the end the 8 waves merge through LDS.  With several
// workgroups (splits) per head, all of them are placed on the same XCD, so their partial
// (max, sum, O) meet in that XCD's L2: each split stores its partial, waits for the stores to be
// acknowledged, takes a ticket, and the last one merges -- no device-wide cache writeback.
// Grouped-query heads (G query heads per KV head): one workgroup per (query head, split), the G
// workgroups of a (KV head, split) placed next to each other on one XCD so that the tiles they all
// read come from HBM once and from that XCD's L2 for the others; the splits of a KV head go to
// different XCDs (there are fewer KV heads than XCDs) and attn_combine_kernel merges them.
#include <hip/hip_ext.h>

#include <type_traits>

#include "fdl_device.h"
#include "fdl_internal.h"
#include "fdl_score.h"
#include "fdl_select.h"
#include "fdl_stream.h"

namespace fdl {

struct MhaParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* k_dec;
  const uint16_t* v_dec;
  const int32_t* sel_idx;
  const int32_t* n_sel;
  uint16_t* out;
  float* part_o;     // [B][H][S][32][D]
  float2* part_ml;   // [B][H][S][32]
  uint32_t* tickets;  // one per (b, h); left at zero by every launch
  uint32_t* status;
  const int32_t* page_table;
  int H, T, L, max_sel, unit_log2, n_units, n_splits, n_segs;
  int Hkv, G;     // KV heads and query heads per KV head (H = Hkv * G)
  int n_groups;   // G > 1: (sequence, KV head, split) triples
  int n_hint;   // expected selected units per head (0 = unknown)
  int page_log2, pages_per_seq, n_pages;
  int merge_here;   // 1: the last split of a head merges the partials; 0: attn_merge_kernel does
  const int32_t* lens;   // per-sequence lengths of a ragged batch, or NULL (every sequence has L)
  float scale_log2;
  // fused selection (SEL): every workgroup scores the blocks of its head against the predicted
  // queries and selects them itself; split 0 also writes the scores and the selection out
  FusedSelect fs;
};

// Phase timestamps (diagnostic builds only): thread 0 of the workgroup records the constant-rate
// clock at point i.
#ifdef FDL_PHASE_STAMPS
#define FDL_STAMP(p, i)                                                                                  \
  do {                                                                                                   \
    if (threadIdx.x == 0 && (p).fs.stamps != nullptr)                                                    \
      (p).fs.stamps[(int64_t)blockIdx.x * kStampsPerGroup + (i)] = __builtin_amdgcn_s_memrealtime();     \
  } while (0)
#else
#define FDL_STAMP(p, i) \
  do {                  \
  } while (0)
#endif

constexpr int kMhaWaves = 8;
constexpr int kMaxSplits = 32;   // workgroups per head (the final merge keeps their weights in LDS)
constexpr int kTileTok = 32;
constexpr float kRescaleSlack = 8.f;   // log2 headroom of the lazily rescaled softmax weights
constexpr int kPageTableLds = 2048;    // page entries per sequence kept in LDS (paged caches)

template <int D>
struct MhaShape {
  static constexpr int PROW = RowChunks<D>::PROW;                     // 16-byte chunks per row
  static constexpr int ROWS_PER_INSTR = RowChunks<D>::ROWS_PER_INSTR;   // rows one 1 KiB fetch covers
  static constexpr int INSTR = kTileTok / ROWS_PER_INSTR;   // fetches per tile for K (same for V)
  static constexpr int HALF = kTileTok * D;          // elements of K (or V) per tile
  static constexpr int SLOT = 2 * HALF;              // elements per wave slot
  static constexpr int KS = D / 16;
  static constexpr int DT = D / 32;
};

// Offset type: contiguous caches address rows relative to the head's base with 32 bits
// (L < 2^24, D <= 128); pages can sit anywhere in the pool and need 64 bits.
template <bool PAGED>
using RowOff = typename std::conditional<PAGED, int64_t, int32_t>::type;

// A tile fetch in two steps, so that the selection-index loads of tile i+1 can fly together with
// the data of tile i: mha_prepare issues the index loads of the lane's rows (clamped, so it needs
// neither the list length nor any earlier load), mha_issue resolves them to tokens, applies the
// list length, adds the page-table step when paged, and launches the LDS fetches.
template <int D>
struct TilePrep {
  int u[MhaShape<D>::INSTR];
};

template <int D, bool DENSE, bool SEL>
__device__ __forceinline__ void mha_prepare(const MhaParams& p, int e, const int32_t* __restrict__ sel_row,
                                            const uint16_t* sel_lds, int lane, TilePrep<D>& tp, bool contig) {
  using S = MhaShape<D>;
  if constexpr (!DENSE) {
    const int rsub = lane / S::PROW;
    if (e == 0) return;   // uniform: the own block needs no index
    if (contig) {   // uniform: the whole tile lies in one unit
      const int si = ((e - 1) * kTileTok) >> p.unit_log2;
      if constexpr (SEL) tp.u[0] = sel_lds[si < p.max_sel ? si : p.max_sel - 1];
      else tp.u[0] = sel_row[si < p.max_sel ? si : p.max_sel - 1];
#pragma unroll
      for (int j = 1; j < S::INSTR; ++j) tp.u[j] = tp.u[0];
      return;
    }
#pragma unroll
    for (int j = 0; j < S::INSTR; ++j) {
      const int i = (e - 1) * kTileTok + j * S::ROWS_PER_INSTR + rsub;
      const int si = i >> p.unit_log2;
      if constexpr (SEL) tp.u[j] = sel_lds[si < p.max_sel ? si : p.max_sel - 1];
      else tp.u[j] = sel_row[si < p.max_sel ? si : p.max_sel - 1];
    }
  }
}

// Barrier of the NS splits of one head.  They run on one XCD (see the kernel), so a relaxed
// atomic at L2 orders them and data they stored before arriving is in that L2.  `bar` is one 64-bit
// word: arrival count in the low half, generation in the high half.  The generation only moves once
// all NS splits of this launch have arrived, so thread 0 may read it (g0) any time before its own
// arrival -- the kernel does so at its start, off the critical path.  The last arrival takes the
// count back to 0 and bumps the generation with a single add.  A waiter gives up after spin_limit
// polls (returns false) instead of waiting on a sibling that is not resident; the caller then
// recomputes what it would have read.  All threads must call.
__device__ __forceinline__ uint32_t head_barrier_gen(const uint32_t* bar) {
  return __hip_atomic_load(&bar[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ bool head_barrier(uint32_t* bar, uint32_t g0, int NS, int spin_limit, int* s_flag) {
  __builtin_amdgcn_s_waitcnt(0);   // this thread's stores are acknowledged by L2
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t zero;
    asm volatile("v_mov_b32 %0, 0" : "=v"(zero) : "v"(g0));   // the arrival is issued after g0 is read
    uint64_t* word = reinterpret_cast<uint64_t*>(bar);
    const uint64_t old = __hip_atomic_fetch_add(word, 1ull + zero, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int ok = 1;
    if ((uint32_t)old == (uint32_t)(NS - 1)) {
      __hip_atomic_fetch_add(word, (1ull << 32) - (uint64_t)NS, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      int it = 0;
      while (__hip_atomic_load(&bar[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == g0) {
        if (++it > spin_limit) {
          ok = 0;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    *s_flag = ok;
  }
  __syncthreads();
  const bool ok = *s_flag != 0;
  asm volatile("buffer_inv sc0" ::: "memory");   // drop L1 lines: the siblings' stores are in L2
  return ok;
}

// Pinned float32 scores of pooled-key rows (the same tree as score_units_kernel).  A batch covers
// kRowBatch rows: lane l of wave w holds 16 floats of row base + ps*RPP + w*RPW + l/LPR.
constexpr int kScoreBatch = 4;   // passes whose loads fly together

// Passes [ps0, kScoreBatch) of the batch at base; ps0 = 1 after mha_load_first_pass.
template <int D>
__device__ __forceinline__ void mha_load_rows(const float* __restrict__ ksh, int base, int rb,
                                              float (&x)[kScoreBatch][16], int ps0 = 0) {
  constexpr int LPR = D / 16, RPW = 64 / LPR, RPP = kMhaWaves * RPW;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int ps = 0; ps < kScoreBatch; ++ps) {
    if (ps < ps0) continue;
    if (base + ps * RPP >= rb) break;   // uniform: no row of this pass is wanted
    int r = base + ps * RPP + wave * RPW + lane / LPR;
    r = r < rb ? r : rb - 1;
    load16<float>(ksh + (int64_t)r * D + 16 * (lane % LPR), x[ps]);
  }
}

// Pass 0 of the batch at base, loaded unconditionally (rows clamped to [0, rb - 1]): a fixed number
// of loads, so that a later wait for loads issued before these can leave them in flight.
template <int D>
__device__ __forceinline__ void mha_load_first_pass(const float* __restrict__ ksh, int base, int rb,
                                                    float (&x)[kScoreBatch][16]) {
  constexpr int LPR = D / 16, RPW = 64 / LPR;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int r = base + wave * RPW + lane / LPR;
  r = r < rb ? r : rb - 1;
  r = r > 0 ? r : 0;
  load16<float>(ksh + (int64_t)r * D + 16 * (lane % LPR), x[0]);
}

// keys[r] = order_key(score) and, when to_global, scores[r] as well, for the batch at base.
// xe (may be NULL): the split-exchange row of the head, where row r gets (score bits << 32) | tag.
template <int D>
__device__ __forceinline__ void mha_dot_rows(const float (&x)[kScoreBatch][16], int base, int rb, const float (&qv)[16],
                                             uint32_t* keys, float* __restrict__ scores, bool to_global,
                                             uint64_t* xe = nullptr, uint32_t tag = 0) {
  constexpr int LPR = D / 16, RPW = 64 / LPR, RPP = kMhaWaves * RPW;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int ps = 0; ps < kScoreBatch; ++ps) {
    if (base + ps * RPP >= rb) break;   // uniform
    const int r = base + ps * RPP + wave * RPW + lane / LPR;
    const float sc = row_dot<LPR>(x[ps], qv);
    if (lane % LPR == 0 && r < rb) {
      keys[r] = order_key(sc);
      if (to_global) scores[r] = sc;
      if (xe != nullptr)
        __hip_atomic_store(xe + r, ((uint64_t)__float_as_uint(sc) << 32) | tag, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Rows [ra, rb); pass 0 of the first batch may already be loaded (x, pre = true).
template <int D>
__device__ __forceinline__ void mha_score_rows(const float* __restrict__ ksh, int ra, int rb, const float (&qv)[16],
                                               uint32_t* keys, float* __restrict__ scores, bool to_global,
                                               float (&x)[kScoreBatch][16], bool pre, uint64_t* xe = nullptr,
                                               uint32_t tag = 0) {
  constexpr int RPP = kMhaWaves * (64 / (D / 16));
  if (rb <= ra) return;   // uniform
  for (int base = ra; base < rb; base += kScoreBatch * RPP) {
    mha_load_rows<D>(ksh, base, rb, x, (pre && base == ra) ? 1 : 0);
    mha_dot_rows<D>(x, base, rb, qv, keys, scores, to_global, xe, tag);
  }
}

// Fused selection, first phase of the SEL kernel, in two steps around the early tile fetches.
//
// mha_score_phase: the M members of a sharing group split the scoring -- the NS splits of a head
// (one query head per KV head), or the G query heads of one (KV head, split) (grouped-query heads,
// whose splits sit on different XCDs).  Member m scores rows [n m / M, n (m+1) / M) into sc_out,
// the members meet at head_barrier, and each then reads all n scores back as order keys (a member
// whose siblings do not arrive in time scores every row itself).  When the threshold selection applies (n <= NT, top_k <= 64), the forced units are
// already known here, so their list goes to the front of sel_lds (ascending) and its length is
// returned: those units' tiles can be fetched before the selection has run.
// mha_choose_phase: every split selects the forced units plus the top-K others into sel_lds
// (forced first, then the chosen, each ascending; the other selection paths write one ascending
// list) and split 0 writes the ascending selection and its count out.  Returns the list length.
// The scratch of both steps lives in the first tile slots, which hold no tile until then.
constexpr int kQbufOffsetF = 8192;   // floats: past qs, keys, forced bits and the selection scratch

template <int D>
struct SelLds {
  float* qs;          // [D]
  uint32_t* keys;     // [kFusedMaxUnits]
  uint32_t* forced;   // [kFusedMaxUnits / 32]
  int* hist;          // [4 * 256]
  int* tmp;           // [NT / 64]
  int* flag;          // [2]
  __device__ explicit SelLds(uint16_t* lds_raw) {
    constexpr int NT = kMhaWaves * 64;
    qs = reinterpret_cast<float*>(lds_raw);
    keys = reinterpret_cast<uint32_t*>(lds_raw) + D;
    forced = keys + kFusedMaxUnits;
    hist = reinterpret_cast<int*>(forced + kFusedMaxUnits / 32);
    tmp = hist + 4 * 256;
    flag = tmp + NT / 64;
    static_assert(D + kFusedMaxUnits + kFusedMaxUnits / 32 + 4 * 256 + NT / 64 + 2 <= kQbufOffsetF, "select scratch");
  }
};

// Scratch of the selection phase, in whole tile slots: waves from kFreeSlotWave on may fetch into
// their slots while it runs.
template <int D>
constexpr int kFreeSlotWave =
    (int)(((kQbufOffsetF + 32 * D) * sizeof(float) + 2 * MhaShape<D>::SLOT - 1) / (2 * MhaShape<D>::SLOT));

__device__ __forceinline__ bool threshold_select_ok(int n, int top_k) {
  return n <= kMhaWaves * 64 && top_k <= 64;
}

// The list of the forced units (ascending) at the front of sel_lds, written by one wave; the count
// goes to *nf_out.  n <= NT, so the NT / 32 <= 16 bit words fit one 16-lane row: lane w holds word w,
// a DPP scan along the row gives the number of forced units before it, and each lane writes its
// own units.
template <int NT>
__device__ __forceinline__ void mha_forced_list(const uint32_t* forced, int n, int max_sel, uint16_t* sel_lds,
                                                int* nf_out) {
  static_assert(NT / 32 <= 16, "bit words in one row");
  const int lane = threadIdx.x & 63;
  const int nw = (n + 31) / 32;
  uint32_t word = lane < nw ? forced[lane] : 0u;
  if (lane == nw - 1 && (n & 31) != 0) word &= (1u << (n & 31)) - 1u;
  const int c = __popc(word);
  const int incl = row_incl_scan(c);
  int pos = incl - c;
  for (uint32_t w = word; w != 0u; w &= w - 1u, ++pos)
    if (pos < max_sel) sel_lds[pos] = (uint16_t)(32 * lane + __builtin_ctz(w));
  const int nf = __builtin_amdgcn_readlane(incl, 15);
  if (lane == 0) *nf_out = nf;
}

// kvh: the KV head within sequence b; kvseg = b * Hkv + kvh; bar_i: the group's barrier word.
// nb: the units of sequence b (all of them unless the batch is ragged); rows are p.n_units apart.
template <int D, bool GQA, bool SAFE>
// seq_writer: the one workgroup of the sequence (KV head 0, split 0, member 0) that writes the sink
// list when the sinks come from the detection's bitmap.
__device__ int mha_score_phase(const MhaParams& p, int b, int kvh, int64_t kvseg, int64_t bar_i, float* sc_out,
                               int m, int M, uint16_t* lds_raw, uint16_t* sel_lds, int nb, bool seq_writer) {
  constexpr int NT = kMhaWaves * 64;
  constexpr int LPR = D / 16;
  static_assert((kQbufOffsetF + 32 * D) * sizeof(float) <= sizeof(uint16_t) * kMhaWaves * MhaShape<D>::SLOT,
                "query staging must fit in the tile slots");
  static_assert(kQbufOffsetF * sizeof(float) + 8 * 32 * D * sizeof(uint16_t) <=
                    sizeof(uint16_t) * kMhaWaves * MhaShape<D>::SLOT,
                "grouped query staging must fit in the tile slots");
  static_assert(kFusedMaxSinks <= NT, "one sink list entry per thread");
  const FusedSelect& f = p.fs;
  const SelLds<D> L(lds_raw);
  const int tid = threadIdx.x;
  const int j = (tid & 63) % LPR;
  const int n = nb;
  const float* ksh = f.ks + kvseg * (int64_t)p.n_units * D;
  uint32_t* bar = f.barriers + bar_i * kSyncStride;
  uint32_t g0 = 0;
  if (M > 1 && tid == 0) g0 = head_barrier_gen(bar);
  // Tagged exchange (one query head per KV head, up to NT units): instead of meeting at a barrier,
  // every split stores its rows' scores into the head's exchange row as 64-bit entries tagged with
  // this launch and the split's XCD, and every thread polls the entry of its own unit.  Entries of
  // an earlier launch carry another tag; entries written on another XCD (whose L2 this one does not
  // share) carry another XCD id and are not trusted: the split then scores every row itself.
  const bool tagged = !GQA && !SAFE && M > 1 && p.n_units <= NT && f.xchg != nullptr;
  __shared__ uint32_t s_tag;

  // Loads in the order they are needed, so that each wait leaves the later ones in flight (the
  // counter of outstanding loads drains in order): the queries, the sink list (thread t < max_sinks
  // holds entry t; the count trims it once the loads are back), then the pooled-key rows.
  // (grouped-query heads: the G heads' rows go to LDS by fetches that hold no registers)
  uint16_t* qstage = reinterpret_cast<uint16_t*>(reinterpret_cast<float*>(lds_raw) + kQbufOffsetF);
  QsumG1<D, 32, NT> qst;
  if constexpr (GQA) qsum_grouped_fetch<D, 32, NT, 8>(p.q + (int64_t)b * p.H * p.T * D, kvh * p.G, p.G, p.T, qstage);
  else qsum_g1_issue<D, 32, NT>(p.q + kvseg * (int64_t)p.T * D, p.T, qst);
  // (every load unconditional, from a valid address: a load under a branch would make the waits
  // below count conservatively)
  const uint64_t pred = f.pred_mask[b];
  // sinks from the detection's bitmap (thread t holds words 2t and 2t + 1), or from the list
  const bool from_bitmap = f.sink_bitmap != nullptr;   // uniform
  const bool have_sinks = !from_bitmap && f.sink_pos != nullptr;
  const bool sink_lane = have_sinks && tid < f.max_sinks;
  const int32_t* sp = have_sinks ? f.sink_pos + (int64_t)b * f.max_sinks + (tid < f.max_sinks ? tid : 0)
                                 : reinterpret_cast<const int32_t*>(f.pred_mask + b);
  const int sink_p = *sp;
  const int sink_n = have_sinks ? f.n_sinks[b] : 0;

  // safe mode: no member hands scores to another; each scores every unit itself
  const int ra = SAFE ? 0 : (int)((int64_t)n * m / M), rb = SAFE ? n : (int)((int64_t)n * (m + 1) / M);
  float x[kScoreBatch][16];
  const bool pre = rb > ra;
  __builtin_amdgcn_sched_barrier(0);
  mha_load_first_pass<D>(ksh, ra, rb, x);   // in flight during the query sum
  __builtin_amdgcn_sched_barrier(0);
  for (int i = tid; i < (n + 31) / 32; i += NT) L.forced[i] = 0u;
  // the query staging area sits above the keys' scratch in the (still unused) tile slots
  if constexpr (GQA) {
    __syncthreads();   // full vector-memory wait: every wave's query fetches have landed
    qsum_grouped_tree<D, 32, NT, 8>(pred, p.G, p.T, qstage, L.qs);
  } else {
    qsum_g1_finish<D, 32, NT>(qst, pred, p.T, reinterpret_cast<float*>(lds_raw) + kQbufOffsetF, L.qs);
  }
  if (tagged && tid == 0) {
    const uint32_t launch = ((g0 + 1u) ^ (f.serial << 12)) & 0x0FFFFFFFu;
    s_tag = (launch << 4) | (xcc_reg() & 0xFu);
    L.flag[0] = 0;
  }
  block_sync_lds();   // qs and the cleared bits
  FDL_STAMP(p, 1);
  if (sink_lane && tid < sink_n && sink_p >= 0) {
    const int u = sink_p >> p.unit_log2;
    if (u < n) atomicOr(&L.forced[u >> 5], 1u << (u & 31));
  }
  static_assert(2 * NT >= kFusedSinkWords, "two bitmap words per thread");
  if (from_bitmap) {   // uniform: the ascending set positions, the first max_sinks of them taken
    const int n_words = f.sink_words;
    const uint32_t* brow = f.sink_bitmap + (int64_t)b * n_words;
    const uint32_t bw0 = 2 * tid < n_words ? brow[2 * tid] : 0u;
    const uint32_t bw1 = 2 * tid + 1 < n_words ? brow[2 * tid + 1] : 0u;
    int total;
    int pos = block_excl_scan<NT>(__popc(bw0) + __popc(bw1), L.tmp, total);
    for (int k = 0; k < 2; ++k)
      for (uint32_t w = k ? bw1 : bw0; w != 0u && pos < f.max_sinks; w &= w - 1u, ++pos) {
        const int tok = 32 * (2 * tid + k) + __builtin_ctz(w);
        const int u = tok >> p.unit_log2;
        if (u < n) atomicOr(&L.forced[u >> 5], 1u << (u & 31));
        if (seq_writer) f.sink_pos_out[(int64_t)b * f.max_sinks + pos] = tok;
      }
    if (seq_writer) {
      for (int i = total + tid; i < f.max_sinks; i += NT) f.sink_pos_out[(int64_t)b * f.max_sinks + i] = -1;
      if (tid == 0) {
        f.n_sinks_out[b] = total < f.max_sinks ? total : f.max_sinks;
        if (total > f.max_sinks) latch(p.status, ST_SINK_OVERFLOW);
      }
    }
  }
  float qv[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) qv[i] = L.qs[16 * j + i];
  const uint32_t tag = tagged ? s_tag : 0u;
  uint64_t* xe = tagged ? reinterpret_cast<uint64_t*>(f.xchg) + kvseg * p.n_units : nullptr;
  mha_score_rows<D>(ksh, ra, rb, qv, L.keys, sc_out, !SAFE || m == 0, x, pre, xe, tag);
  FDL_STAMP(p, 2);
  const bool listing = threshold_select_ok(n, f.top_k);   // uniform
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  bool listed = false;
  bool redo = false;   // uniform: some of the others' scores did not come; this split scores them itself
  if (tagged) {
    // thread t < n fetches unit t's score: its own split's from LDS, the others' from the
    // exchange row (polled until this launch's entry is there)
    bool ok = f.spin_limit > 0;   // a zero spin limit never waits: every split scores every row
    uint32_t key = 0u;
    if (ok && tid < n && (tid < ra || tid >= rb)) {
      int it = 0;
      for (;;) {
        const uint64_t v = __hip_atomic_load(xe + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint32_t vt = (uint32_t)v;
        if (vt == tag) {
          key = order_key(__uint_as_float((uint32_t)(v >> 32)));
          break;
        }
        if ((vt >> 4) == (tag >> 4) || ++it > f.spin_limit) {   // written on another XCD, or too late
          if ((vt >> 4) == (tag >> 4)) latch(p.status, ST_PLACEMENT);
          ok = false;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    if (!ok) atomicOr(reinterpret_cast<uint32_t*>(L.flag), 1u);
    block_sync_lds();   // own keys, forced bits and the flag
    if (tid < n && (tid < ra || tid >= rb)) L.keys[tid] = key;
    if (listing && wave == 0) mha_forced_list<NT>(L.forced, n, p.max_sel, sel_lds, L.flag + 1);
    listed = true;
    FDL_STAMP(p, 3);
    redo = L.flag[0] != 0;
    if (redo) block_sync_lds();   // the forced list's flag word is read below; the keys are rewritten
  } else if (M > 1 && !SAFE) {
    const bool synced = head_barrier(bar, g0, M, f.spin_limit, L.flag);   // forced bits are complete
    FDL_STAMP(p, 3);
    // wave 0 lists the forced units while the others read the scores back
    if (listing && wave == 0) mha_forced_list<NT>(L.forced, n, p.max_sel, sel_lds, L.flag + 1);
    listed = true;
    if (synced) {
      for (int i = tid; i < n; i += NT)
        if (i < ra || i >= rb) L.keys[i] = order_key(sc_out[i]);
    }
    redo = !synced;
  }
  if (redo) {   // uniform
    mha_score_rows<D>(ksh, 0, ra, qv, L.keys, sc_out, false, x, false);
    mha_score_rows<D>(ksh, rb, n, qv, L.keys, sc_out, false, x, false);
    if (tid == 0) latch(p.status, ST_SYNC_FALLBACK);
  }
  block_sync_lds();   // keys and forced bits complete
  FDL_STAMP(p, 4);
  if (!listing) return 0;   // uniform
  if (!listed) {
    if (wave == 0) mha_forced_list<NT>(L.forced, n, p.max_sel, sel_lds, L.flag + 1);
    block_sync_lds();
  }
  const int nf = __builtin_amdgcn_readfirstlane(L.flag[1]);
  return nf < p.max_sel ? nf : p.max_sel;
}

// writer: the one workgroup of the KV head that writes the selection out.
template <int D>
__device__ int mha_choose_phase(const MhaParams& p, int64_t kvseg, bool writer, uint16_t* lds_raw, uint16_t* sel_lds,
                                int nb) {
  constexpr int NT = kMhaWaves * 64;
  const FusedSelect& f = p.fs;
  const SelLds<D> L(lds_raw);
  const int tid = threadIdx.x;
  const int n = nb;
  // a ragged batch: the units past the sequence's own score +0
  if (writer)
    for (int i = n + tid; i < p.n_units; i += NT) f.scores[kvseg * p.n_units + i] = 0.f;
  int32_t* gout = f.sel_idx + kvseg * p.max_sel;
  SelResult r;
  FDL_STAMP(p, 13);
  if (threshold_select_ok(n, f.top_k)) {
    auto emit = [&](int gpos, int lpos, int i) {
      if (lpos < p.max_sel) sel_lds[lpos] = (uint16_t)i;
      if (writer && gpos < p.max_sel) gout[gpos] = i;
    };
    r = select_top64<NT>(L.keys, L.forced, n, f.top_k, L.keys + kFusedMaxUnits - NT, L.hist, emit);
  } else {
    auto emit = [&](int pos, int i) {
      if (pos < p.max_sel) {
        sel_lds[pos] = (uint16_t)i;
        if (writer) gout[pos] = i;
      }
    };
    if (n <= NT) {
      r = select_small<NT>(L.keys, L.forced, n, f.top_k, reinterpret_cast<uint64_t*>(L.keys + kFusedMaxUnits - 2 * NT),
                           reinterpret_cast<uint32_t*>(L.hist), L.hist + 64, L.tmp, emit);
    } else {
      const SelScratch scr{L.hist, L.tmp};
      r = select_core<NT, kFusedMaxUnits / NT>(L.keys, L.forced, n, f.top_k, scr, emit);
    }
  }
  FDL_STAMP(p, 14);
  if (writer && tid == 0) f.n_sel[kvseg] = r.total < p.max_sel ? r.total : p.max_sel;
  if (tid == 0 && r.total > p.max_sel) latch(p.status, ST_SEL_OVERFLOW);
  block_sync_lds();   // sel_lds complete; the slots are free again
  return r.total < p.max_sel ? r.total : p.max_sel;
}

// Source of one 16-byte fetch.  Contiguous caches: a uniform base plus an unsigned 32-bit byte
// offset per lane, which the fetch takes in its scalar-base form.
__device__ __forceinline__ const void* row_src(const uint16_t* base, int32_t off) {
  return reinterpret_cast<const char*>(base) + (uint32_t)off * 2u;
}
__device__ __forceinline__ const void* row_src(const uint16_t* base, int64_t off) {
  return base + off;
}

// Per-lane byte offsets, within a run of 32 consecutive rows, of the 16-byte chunks the NI fetches
// of a tile move: fetch j, lane l covers row j * ROWS_PER_INSTR + l / PROW and stores the global
// chunk (l % PROW) ^ swz(row) at LDS chunk slot l % PROW.  They do not depend on the tile.
template <int D>
__device__ __forceinline__ void tile_chunk_offsets(int lane, uint32_t (&voff)[MhaShape<D>::INSTR]) {
  using S = MhaShape<D>;
  const int rsub = lane / S::PROW, sc = lane % S::PROW;
#pragma unroll
  for (int j = 0; j < S::INSTR; ++j) {
    const int r = j * S::ROWS_PER_INSTR + rsub;
    voff[j] = (uint32_t)((r * D + (sc ^ (swz(r) & (S::PROW - 1))) * 8) * 2);
  }
}

// Launch the LDS fetches of a prepared tile into the wave's slot; returns the 32-bit row mask.
// MAYBE_OWN = false: the caller knows e > 0 (a wave's later tiles), so the own-block branch goes.
// contig (uniform; contiguous caches with units of at least 32 tokens, or dense): a full tile is one
// run of 32 consecutive cache rows, fetched from a scalar base plus the fixed offsets voff.
// Lb, nb: the tokens and units of sequence b (the cache rows stay p.L apart).
template <int D, bool DENSE, bool PAGED, bool MAYBE_OWN = true, int POL = kStreamPolicy>
__device__ __forceinline__ uint32_t mha_issue(const MhaParams& p, const KvRows<PAGED>& rows, int b, int h,
                                              int e, int n_list, const TilePrep<D>& tp, uint16_t* slot,
                                              int lane, bool& bad, bool contig,
                                              const uint32_t (&voff)[MhaShape<D>::INSTR], int Lb, int nb,
                                              const int32_t* spt = nullptr) {
  using S = MhaShape<D>;
  constexpr int NI = S::INSTR;
  const int rsub = lane / S::PROW;
  const int sc = lane % S::PROW;
  const int64_t head = (int64_t)b * p.Hkv + h;   // h: the KV head within sequence b
  const bool dec = MAYBE_OWN && ((e == 0) || (Lb == 0));   // uniform
  if constexpr (!PAGED) {
    const int t0 = (e - 1) * kTileTok;   // list position of the tile's first row
    int tok0 = t0;
    bool uok = true;
    if (!dec && contig && !DENSE) {
      const int u = __builtin_amdgcn_readfirstlane(tp.u[0]);
      uok = (unsigned)u < (unsigned)nb;
      tok0 = (u << p.unit_log2) + (t0 & ((1 << p.unit_log2) - 1));
    }
    // a full tile of a valid unit that ends inside the cache (a cache whose last unit is partial
    // takes the general path for that unit's tiles)
    if (!dec && contig && t0 + kTileTok <= n_list && (!uok || tok0 + kTileTok <= Lb)) {   // uniform
      bad = bad || !uok;
      tok0 = uok ? tok0 : 0;   // an unusable unit reads the head's first rows and is masked out
      const char* kbase = reinterpret_cast<const char*>(p.k + (head * p.L + tok0) * D);
      const char* vbase = reinterpret_cast<const char*>(p.v + (head * p.L + tok0) * D);
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const void* src = kbase + voff[j];
        __builtin_amdgcn_global_load_lds(src, (lds_void_t*)(slot + j * 512), 16, 0, POL);
      }
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const void* src = vbase + voff[j];
        __builtin_amdgcn_global_load_lds(src, (lds_void_t*)(slot + S::HALF + j * 512), 16, 0, POL);
      }
      return uok ? 0xFFFFFFFFu : 0u;
    }
  }
  const uint16_t* kb;
  const uint16_t* vb;
  RowOff<PAGED> off[NI];
  bool ok[NI];
  if (dec) {
    kb = p.k_dec + head * p.T * D;
    vb = p.v_dec + head * p.T * D;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int r = j * S::ROWS_PER_INSTR + rsub;
      ok[j] = (e == 0) && r < p.T;
      off[j] = (RowOff<PAGED>)(((e == 0) && r < p.T ? r : 0) * D);
    }
  } else {
    int t[NI];
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int i = (e - 1) * kTileTok + j * S::ROWS_PER_INSTR + rsub;
      ok[j] = i < n_list;
      t[j] = ok[j] ? i : 0;
      if constexpr (!DENSE) {
        const int u = tp.u[j];
        const bool uok = (unsigned)u < (unsigned)nb;
        bad = bad || (ok[j] && !uok);
        ok[j] = ok[j] && uok;
        t[j] = uok ? (u << p.unit_log2) + (t[j] & ((1 << p.unit_log2) - 1)) : 0;
      }
      ok[j] = ok[j] && t[j] < Lb;
      t[j] = t[j] < Lb ? t[j] : 0;
    }
    if constexpr (PAGED) {
      kb = p.k;
      vb = p.v;
      bool pb[NI];
      if (spt != nullptr) {   // uniform: the sequence's page table sits in LDS
#pragma unroll
        for (int j = 0; j < NI; ++j) {
          const int pp = spt[t[j] >> p.page_log2];
          const bool good = (unsigned)pp < (unsigned)p.n_pages;
          pb[j] = !good;
          const int64_t pg = good ? pp : 0;
          off[j] = (((pg * p.Hkv + h) << p.page_log2) | (int64_t)(t[j] & ((1 << p.page_log2) - 1))) * D;
        }
      } else {
#pragma unroll
        for (int j = 0; j < NI; ++j) {
          pb[j] = false;
          off[j] = rows.off(b, h, t[j], pb[j]);
        }
      }
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        bad = bad || (ok[j] && pb[j]);
        ok[j] = ok[j] && !pb[j];
      }
    } else {
      kb = p.k + head * p.L * D;
      vb = p.v + head * p.L * D;
#pragma unroll
      for (int j = 0; j < NI; ++j) off[j] = (RowOff<PAGED>)(t[j] * D);
    }
  }
  uint32_t okm = 0;
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const int r = j * S::ROWS_PER_INSTR + rsub;
    off[j] += (sc ^ (swz(r) & (S::PROW - 1))) * 8;   // global chunk stored at LDS slot sc of row r
    const uint64_t bal = __ballot(ok[j]);
#pragma unroll
    for (int q = 0; q < S::ROWS_PER_INSTR; ++q)
      okm |= (uint32_t)((bal >> (q * S::PROW)) & 1ull) << (j * S::ROWS_PER_INSTR + q);
  }
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const void* src = row_src(kb, off[j]);
    __builtin_amdgcn_global_load_lds(src, (lds_void_t*)(slot + j * 512), 16, 0, POL);
  }
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const void* src = row_src(vb, off[j]);
    __builtin_amdgcn_global_load_lds(src, (lds_void_t*)(slot + S::HALF + j * 512), 16, 0, POL);
  }
  return okm;
}

// Merge of the NS partials (O, max, sum) of head seg into its bf16 output: thread (query qi, chunk
// pair dg).  Every split's (max, sum) and the partials of the first kMergeBatch splits are requested
// in one round trip (the statistics first, so that waiting for them leaves the partials in flight);
// the statistics are shared through LDS (s_ml2: [NS][32]).  Every thread derives its query's split
// weights itself: the common max, then per split exp2(m - M), the sum of l times the weight and the
// weighted partials, in split order.  Reads past NS are clamped to the last split and masked, so
// that they go out together.  Used by the last split of a head in the fused launch and by the safe
// mode's second launch alike, so both give the same bits.
template <int D>
__device__ __forceinline__ void merge_splits(const MhaParams& p, const float* po_base, const float2* pml_base,
                                             uint16_t* out, int T, int64_t seg, int NS, float2* s_ml2) {
  constexpr int NT = kMhaWaves * 64;
  constexpr int HC = D / 8;   // chunks per half row
  constexpr int kMergeBatch = 8;
  const int tid = threadIdx.x;
  const bool item = tid < 32 * HC;
  const int qi = item ? tid / HC : 0, dg = tid % HC;
  float2 ml[(kMaxSplits * 32 + NT - 1) / NT];
#pragma unroll
  for (int k = 0; k < (kMaxSplits * 32 + NT - 1) / NT; ++k) {
    const int i = tid + k * NT;
    if (i < NS * 32) ml[k] = pml_base[seg * NS * 32 + i];
  }
  __builtin_amdgcn_sched_barrier(0);   // keep the statistics loads ahead of the partials
  float4 a[kMergeBatch], c[kMergeBatch];
  auto load_batch = [&](int t0) {
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      const int t = t0 + j < NS ? t0 + j : NS - 1;
      const float* src = po_base + ((seg * NS + t) * 32 + qi) * D + 4 * dg;
      a[j] = *reinterpret_cast<const float4*>(src);
      c[j] = *reinterpret_cast<const float4*>(src + 4 * HC);
    }
  };
  load_batch(0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int k = 0; k < (kMaxSplits * 32 + NT - 1) / NT; ++k) {
    const int i = tid + k * NT;
    if (i < NS * 32) s_ml2[i] = ml[k];
  }
  block_sync_lds();   // the partial loads stay in flight
  FDL_STAMP(p, 11);
  float Mh = -__builtin_inff();
  for (int t0 = 0; t0 < NS; t0 += kMergeBatch) {
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      const int t = t0 + j < NS ? t0 + j : NS - 1;
      Mh = fmaxf(Mh, s_ml2[t * 32 + qi].x);
    }
  }
  float Ls = 0.f;
  float4 o1 = make_float4(0.f, 0.f, 0.f, 0.f), o2 = o1;
  for (int t0 = 0; t0 < NS; t0 += kMergeBatch) {
    if (t0 > 0) load_batch(t0);
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      const int t = t0 + j < NS ? t0 + j : NS - 1;
      const float2 v = s_ml2[t * 32 + qi];
      const float w = (t0 + j < NS && v.x != -__builtin_inff() && Mh != -__builtin_inff()) ? exp2_fast(v.x - Mh) : 0.f;
      Ls += v.y * w;
      o1.x += a[j].x * w; o1.y += a[j].y * w; o1.z += a[j].z * w; o1.w += a[j].w * w;
      o2.x += c[j].x * w; o2.y += c[j].y * w; o2.z += c[j].z * w; o2.w += c[j].w * w;
    }
  }
  FDL_STAMP(p, 12);
  if (item && qi < T) {
    const float inv = 1.f / Ls;
    uint16_t* dst = out + (seg * T + qi) * D + 4 * dg;
    *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(o1.x * inv, o1.y * inv), pack_bf16x2(o1.z * inv, o1.w * inv));
    *reinterpret_cast<uint2*>(dst + 4 * HC) =
        make_uint2(pack_bf16x2(o2.x * inv, o2.y * inv), pack_bf16x2(o2.z * inv, o2.w * inv));
  }
}

// SAFE (fused selection only): no workgroup hands data to another inside the launch -- every split
// scores every unit, and the partials are merged by attn_merge_kernel.
template <int D, bool DENSE, bool PAGED, bool SEL, bool GQA = false, bool SAFE = false>
__global__ __launch_bounds__(kMhaWaves * 64, 1) void attn_mha_kernel(const MhaParams p) {
  using S = MhaShape<D>;
  constexpr int NT = kMhaWaves * 64;
  constexpr int KS = S::KS, DT = S::DT, PROW = S::PROW;
  static_assert(!SEL || (!DENSE && !PAGED), "fused selection: contiguous sparse only");
  // grouped-query heads read every tile G times, through L2: their fetches keep the default
  // (cached) policy; one reader per tile streams with the non-temporal one
  constexpr int POL = GQA ? 0 : kStreamPolicy;
  __shared__ __attribute__((aligned(1024))) uint16_t lds[kMhaWaves * S::SLOT];
  __shared__ uint16_t sel_lds[SEL ? kFusedMaxSel : 1];

  // Workgroup i runs on XCD i % 8 (the dispatcher's round-robin order).  One query head per KV
  // head: all splits of a head are given workgroup ids with the same residue, so they share one L2
  // and the final merge can hand partials over through it.  G query heads per KV head: the G
  // workgroups of one (KV head, split) get consecutive ids of one residue, so they stream the same
  // tiles through one L2 at about the same time (one HBM read serves all G); the splits of a KV
  // head spread over the XCDs and their partials are merged by a second kernel.
  const int NS = p.n_splits;
  const int xcd = blockIdx.x & 7, xslot = blockIdx.x >> 3;
  int s, seg_i, kv_i;   // split, query head (b * H + h), KV head (b * Hkv + g)
  int gi = 0, member = 0;   // grouped-query heads: the (KV head, split) group and the head in it
  if constexpr (!GQA) {
    s = xslot % NS;
    seg_i = xcd + 8 * (xslot / NS);
    if (seg_i >= p.n_segs) return;
    kv_i = seg_i;
  } else {
    gi = xcd + 8 * (xslot / p.G);
    if (gi >= p.n_groups) return;
    kv_i = gi / NS;
    s = gi % NS;
    member = xslot % p.G;
    seg_i = (kv_i / p.Hkv) * p.H + (kv_i % p.Hkv) * p.G + member;
  }
  const int b = kv_i / p.Hkv, h = kv_i % p.Hkv;   // h: KV head within the sequence
  // the one workgroup of the sequence that writes its sink list (or clears the detection's bitmap)
  const bool seq_writer = h == 0 && s == 0 && member == 0;
  // A bitmap no one reads any more (the detection's, read by the layer before): zeroed for the next
  // detection by the sequence's writer at its way out, after its own work.
  auto clear_sinks = [&]() {
    if (SEL && p.fs.clear_bitmap != nullptr && seq_writer)
      for (int i = threadIdx.x; i < p.fs.sink_words; i += kMhaWaves * 64)
        p.fs.clear_bitmap[(int64_t)b * p.fs.sink_words + i] = 0u;
  };
  const int Lb = seq_len(p.lens, b, p.L);         // this sequence's tokens (ragged batches)
  const int nb = (Lb + (1 << p.unit_log2) - 1) >> p.unit_log2;
  FDL_STAMP(p, 0);
#ifdef FDL_PHASE_STAMPS
  if (threadIdx.x == 0 && p.fs.stamps != nullptr)
    p.fs.stamps[(int64_t)blockIdx.x * kStampsPerGroup + kStampXcc] =
        (uint64_t)xcc_reg() | ((uint64_t)s << 32) | ((uint64_t)seg_i << 40) | ((uint64_t)1 << 63);
#endif
  // the wave index is uniform: in a scalar register, the per-tile bookkeeping stays scalar
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ql = lane & 31, hh = lane >> 5;
  const int64_t seg = seg_i, kvseg = kv_i;
  KvRows<PAGED> rows;
  rows.Hkv = p.Hkv;
  rows.L = p.L;
  rows.D = D;
  rows.page_log2 = p.page_log2;
  rows.pages_per_seq = p.pages_per_seq;
  rows.n_pages = p.n_pages;
  rows.page_table = p.page_table;
  bool bad = false;
  // Paged caches: the sequence's page-table entries are copied to LDS once, so that a tile's row
  // addresses need no dependent global load.
  __shared__ int32_t s_pt[PAGED ? kPageTableLds : 1];
  const int32_t* spt = nullptr;
  if constexpr (PAGED) {
    if (p.pages_per_seq <= kPageTableLds) {   // uniform
      for (int i = tid; i < p.pages_per_seq; i += kMhaWaves * 64)
        s_pt[i] = p.page_table[(int64_t)b * p.pages_per_seq + i];
      __syncthreads();
      spt = s_pt;
    }
  }

  const int32_t* sel_row = DENSE ? nullptr : p.sel_idx + kvseg * p.max_sel;
  uint16_t* slot = lds + wave * S::SLOT;
  // Tile partition.  Dense: the list is the whole cache.  Sparse: when the caller knows the usual
  // selection size (n_hint units), the split ranges come from it, so the first tile's index loads
  // can go out together with the read of the actual count; the actual count then trims the ranges
  // and the last split takes any tiles beyond the hint.
  // contiguous tiles (see mha_issue) and the fixed chunk offsets of their fetches
  const bool contig = !PAGED && (DENSE || p.unit_log2 >= 5);
  uint32_t voff[S::INSTR];
  tile_chunk_offsets<D>(lane, voff);
  // A wave's tiles: e, then e + e_step while below e1 -- except in the fused kernel, where tiles
  // below e_pre (fetched early, one per wave) are followed by the wave's round-robin start e_rr.
  int e, e1, n_list;
  int e_step = kMhaWaves, e_pre = 0, e_rr = 0;
  int n_rounds = 0;   // dense: tile rounds that every wave of the workgroup completes
  TilePrep<D> tp;
  uint32_t vm_next = 0;
  bool issued = false;
  if constexpr (SEL) {
    // sharing group: the NS splits of the head, or the G heads of this (KV head, split); split 0's
    // group exchanges its scores through the scores output, the others through their own rows
    int nf;
    if constexpr (GQA) {
      float* xo = s == 0 ? p.fs.scores + kvseg * p.n_units : p.fs.xchg + (int64_t)gi * p.n_units;
      nf = mha_score_phase<D, true, SAFE>(p, b, h, kvseg, gi, xo, member, p.G, lds, sel_lds, nb, seq_writer);
    } else {
      nf = mha_score_phase<D, false, SAFE>(p, b, h, kvseg, seg, p.fs.scores + kvseg * p.n_units, s, NS, lds, sel_lds,
                                           nb, seq_writer);
    }
    // Known now: tile 0 (the block's own tokens) and the tiles of the nf forced units at the front
    // of the list.  Up to one of them per wave whose slot the selection scratch leaves free is
    // fetched while the selection runs.  The other tiles go round robin over all 8 NS waves of the
    // head, so that no wave streams more than its share after the selection; the waves that
    // fetched early come last in that order.
    constexpr int FW = kFreeSlotWave<D>;
    const int tpu = p.unit_log2 >= 5 ? 1 << (p.unit_log2 - 5) : 0;   // tiles per unit
    const int n_known = 1 + (Lb > 0 ? nf * tpu : 0);
    const int cap = (kMhaWaves - FW) * NS;
    e_pre = n_known < cap ? n_known : cap;
    const int rr = wave < FW ? wave : FW + (kMhaWaves - 1 - wave);
    e_rr = e_pre + rr * NS + s;
    e_step = kMhaWaves * NS;
    const int jp = (wave - FW) * NS + s;
    e = (wave >= FW && jp < e_pre) ? jp : e_rr;
    if (e < e_pre) {   // uniform per wave
      mha_prepare<D, false, true>(p, e, sel_row, sel_lds, lane, tp, contig);
      vm_next = mha_issue<D, false, false, true, POL>(p, rows, b, h, e, nf << p.unit_log2, tp, slot, lane, bad, contig, voff,
                                                      Lb, nb);
      issued = true;
    }
    const int ns = mha_choose_phase<D>(p, kvseg, s == 0 && member == 0, lds, sel_lds, nb);
    FDL_STAMP(p, 5);
    n_list = Lb == 0 ? 0 : ns << p.unit_log2;
    e1 = 1 + (n_list + kTileTok - 1) / kTileTok;
    if (!issued) mha_prepare<D, false, true>(p, e, sel_row, sel_lds, lane, tp, contig);
  } else {
    int n_part = DENSE ? Lb : (p.n_hint > 0 ? (p.n_hint < p.max_sel ? p.n_hint : p.max_sel) << p.unit_log2 : -1);
    if (!DENSE && n_part < 0) {
      const int ns_raw = p.n_sel[kvseg];   // no hint: the count comes first
      n_part = (ns_raw < 0 ? 0 : (ns_raw > p.max_sel ? p.max_sel : ns_raw)) << p.unit_log2;
    }
    if (Lb == 0) n_part = 0;
    const int n_tiles_part = 1 + (n_part + kTileTok - 1) / kTileTok;
    const int e0 = (int)((int64_t)n_tiles_part * s / NS);
    e1 = (int)((int64_t)n_tiles_part * (s + 1) / NS);
    n_rounds = DENSE ? (e1 - e0) / kMhaWaves : 0;   // wave w has ceil((e1 - e0 - w) / 8) >= this many
    e = e0 + wave;
    // unconditional: the last split may grow past the hinted range once the count is known
    mha_prepare<D, DENSE, false>(p, e, sel_row, sel_lds, lane, tp, contig);
    n_list = n_part;
    if (!DENSE && p.n_hint > 0) {
      int ns = p.n_sel[kvseg];
      ns = ns < 0 ? 0 : (ns > p.max_sel ? p.max_sel : ns);
      n_list = Lb == 0 ? 0 : ns << p.unit_log2;
      const int n_tiles = 1 + (n_list + kTileTok - 1) / kTileTok;
      if (s == NS - 1) e1 = n_tiles;
      e1 = e1 < n_tiles ? e1 : n_tiles;
    }
  }

  // Q fragments (B operand of S^T = K Q^T): lane (q, hh) holds q[q][hh*D/2 + 8ks .. +8]
  bf16x8 qf[KS];
  {
    const uint16_t* qrow = p.q + ((int64_t)seg * p.T + (ql < p.T ? ql : 0)) * D + hh * (D / 2);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 v = *reinterpret_cast<const uint4*>(qrow + ks * 8);
      if (ql >= p.T) v = make_uint4(0u, 0u, 0u, 0u);
      qf[ks] = as_bf16x8(v);
    }
  }

  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
  float m_run = -__builtin_inff(), l_run = 0.f;
  bool fresh = true;   // no tile accumulated yet (uniform)

  if (!issued && e < e1)
    vm_next = mha_issue<D, DENSE, PAGED, true, POL>(p, rows, b, h, e, n_list, tp, slot, lane, bad, contig, voff, Lb, nb,
                                                    spt);
  const int swz_k = swz(ql) & (PROW - 1);
#ifdef FDL_PHASE_STAMPS
  bool first_tile = true;
#endif
  for (int en; e < e1; e = en) {
    // This tile's LDS fetches must have landed before the slot is read.  Explicit, because the
    // compiler's own wait for LDS fetches is not placed reliably across the loop back-edge when
    // other vector loads are in flight.
    wait_vm0();
#ifdef FDL_PHASE_STAMPS
    if (first_tile) FDL_STAMP(p, 6);
    first_tile = false;
#endif
    const uint32_t vm = vm_next;
    en = (SEL && e < e_pre) ? e_rr : e + e_step;
    const bool more = en < e1;
    if (more) mha_prepare<D, DENSE, SEL>(p, en, sel_row, sel_lds, lane, tp, contig);
    // ---- K from LDS into A-operand registers, then S^T = K Q^T: register r holds token
    //      8*(r/4) + 4*hh + r%4 for query ql (K registers die here) ----
    f32x16 sacc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
    {
      uint4 ka[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int c = hh * (PROW / 2) + ks;
        ka[ks] = *reinterpret_cast<const uint4*>(slot + ql * D + ((c ^ swz_k) * 8));
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) sacc = mfma32(as_bf16x8(ka[ks]), qf[ks], sacc);
    }
    // ---- V from LDS, read transposed into the A operand of O^T = V^T P^T.  MFMA dt covers
    //      d = 64*(dt/2) + 2*i + (dt%2), i = 0..31, so one 32-bit read (columns 2i, 2i+1) feeds the
    //      operands of MFMAs 2p and 2p+1 at once ----
    uint4 va[2][DT];
#pragma unroll
    for (int kl = 0; kl < 2; ++kl) {
      const int r0 = 16 * kl + 4 * hh;
#pragma unroll
      for (int pp = 0; pp < DT / 2; ++pp) {
        const int d = 64 * pp + 2 * ql;
        const int cd = d >> 3, dd = d & 7;
        const uint16_t* vbase = slot + S::HALF;
        uint32_t w[8];
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          const int row = r0 + (x < 4 ? x : x + 4);
          w[x] = *reinterpret_cast<const uint32_t*>(vbase + row * D + ((cd ^ (swz(row) & (PROW - 1))) * 8) + dd);
        }
        // low halves of (w[2i], w[2i+1]) -> one word, high halves -> another (one byte permute each)
        constexpr uint32_t kLo = 0x05040100u, kHi = 0x07060302u;
        va[kl][2 * pp] = make_uint4(__builtin_amdgcn_perm(w[1], w[0], kLo), __builtin_amdgcn_perm(w[3], w[2], kLo),
                                    __builtin_amdgcn_perm(w[5], w[4], kLo), __builtin_amdgcn_perm(w[7], w[6], kLo));
        va[kl][2 * pp + 1] = make_uint4(__builtin_amdgcn_perm(w[1], w[0], kHi), __builtin_amdgcn_perm(w[3], w[2], kHi),
                                        __builtin_amdgcn_perm(w[5], w[4], kHi), __builtin_amdgcn_perm(w[7], w[6], kHi));
      }
    }
    wait_lgkm0();
    // ---- fetch the next tile into the same slot; it flies while this one is finished ----
    if (more)
      vm_next = mha_issue<D, DENSE, PAGED, false, POL>(p, rows, b, h, en, n_list, tp, slot, lane, bad, contig, voff, Lb,
                                                       nb, spt);
    float mx = -__builtin_inff();
    if (vm == 0xFFFFFFFFu) {   // uniform: every row of the tile is valid
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sacc[r] *= p.scale_log2;
        mx = fmaxf(mx, sacc[r]);
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 8 * (r >> 2) + 4 * hh + (r & 3);
        float x = sacc[r] * p.scale_log2;
        x = ((vm >> row) & 1u) ? x : -__builtin_inff();
        sacc[r] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = fmaxf(mx, lane_xor32f(mx));
    // Lazy rescaling: a query's running max m_run only moves when the tile's max exceeds it by more
    // than kRescaleSlack (log2 units); the weights exp2(s - m_run) then stay below 2^kRescaleSlack,
    // and most later tiles skip the rescaling of the accumulators.  The first tile always moves it
    // (m_run = -inf); its accumulators are still zero and need no rescaling.
    const bool grow = mx > m_run + kRescaleSlack;
    if (__ballot(grow) != 0) {   // uniform
      const float m_new = grow ? mx : m_run;
      const float alpha = exp2_fast(m_run - m_new);
      l_run *= alpha;
      m_run = m_new;
      if (!fresh) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
      }
    }
    fresh = false;
    if (m_run != -__builtin_inff()) {
      float rs = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pr = exp2_fast(sacc[r] - m_run);
        sacc[r] = pr;
        rs += pr;
      }
      rs += lane_xor32f(rs);
      l_run += rs;
      // ---- O^T += V^T P^T over 2 k-steps of 16 tokens ----
#pragma unroll
      for (int kl = 0; kl < 2; ++kl) {
        uint4 pb;
        pb.x = pack_bf16x2(sacc[8 * kl + 0], sacc[8 * kl + 1]);
        pb.y = pack_bf16x2(sacc[8 * kl + 2], sacc[8 * kl + 3]);
        pb.z = pack_bf16x2(sacc[8 * kl + 4], sacc[8 * kl + 5]);
        pb.w = pack_bf16x2(sacc[8 * kl + 6], sacc[8 * kl + 7]);
        const bf16x8 bfr = as_bf16x8(pb);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) oacc[dt] = mfma32(as_bf16x8(va[kl][dt]), bfr, oacc[dt]);
      }
    }
    // Dense: the waves of a workgroup meet after every round of tiles.  The memory system serves
    // them unevenly; left free, the last wave of a workgroup ends up to 14 us after the first and
    // the tail streams with few waves in flight.  Every wave passes exactly n_rounds barriers.
    if constexpr (DENSE) {
      if (n_rounds > 0) {
        --n_rounds;
        __builtin_amdgcn_s_barrier();
      }
    }
  }
  latch_bad(p.status, bad);
  FDL_STAMP(p, 7);

  // ---- merge the 8 waves.  Each wave stores its unnormalized O^T (relative to its own running
  //      max) and its (max, sum) as soon as its last tile is done, into its own slot (its fetches
  //      have all been consumed); after one barrier every thread combines its (query, chunk pair)
  //      over the waves with the weights exp2(m_w - M).
  //      Slot layout: query-major rows of D floats, 16-byte chunk c of row q stored at chunk
  //      c ^ (q & 15), so that both the writes (16 rows, one chunk) and the reads (one row, 16
  //      chunks) hit 16 different bank groups.  Lane (q, hh) holds, for each (dtp, rg), the eight
  //      consecutive d = 64 dtp + 16 rg + 8 hh + [0, 8) of query q (registers r = 4 rg + [0, 4) of
  //      MFMAs 2 dtp and 2 dtp + 1): chunks 16 dtp + 4 rg + 2 hh and the next. ----
  __shared__ float s_m[kMhaWaves][32], s_l[kMhaWaves][32];
  __shared__ uint32_t s_ticket, s_here;
  constexpr int CH = D / 4;   // 16-byte chunks per row
  constexpr int HC = D / 8;   // chunks per half row
  static_assert(32 * D * sizeof(float) == sizeof(uint16_t) * S::SLOT, "a wave's rows fill its slot");
  {
    float* mo = reinterpret_cast<float*>(slot);   // [32][D]
#pragma unroll
    for (int dtp = 0; dtp < DT / 2; ++dtp)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const f32x16& a = oacc[2 * dtp];
        const f32x16& c = oacc[2 * dtp + 1];
        const int c0 = 16 * dtp + 4 * rg + 2 * hh;
        float* row = mo + ql * D;
        *reinterpret_cast<float4*>(row + 4 * ((c0 ^ (ql & 15)) & (CH - 1))) =
            make_float4(a[4 * rg], c[4 * rg], a[4 * rg + 1], c[4 * rg + 1]);
        *reinterpret_cast<float4*>(row + 4 * (((c0 + 1) ^ (ql & 15)) & (CH - 1))) =
            make_float4(a[4 * rg + 2], c[4 * rg + 2], a[4 * rg + 3], c[4 * rg + 3]);
      }
    if (hh == 0) {
      s_m[wave][ql] = m_run;
      s_l[wave][ql] = l_run;
    }
  }
  __syncthreads();
  FDL_STAMP(p, 8);
  static_assert(32 * HC <= NT, "one (query, chunk pair) item per thread");
  const bool item = tid < 32 * HC;
  const int qi = item ? tid / HC : 0, dg = tid % HC;
  float* po_base = p.part_o;
  float2* pml_base = p.part_ml;
  uint16_t* const p_out = p.out;
  const int p_T = p.T;
  float Mq = -__builtin_inff(), Lq = 0.f;
  {
    float mw[kMhaWaves];
#pragma unroll
    for (int w = 0; w < kMhaWaves; ++w) {
      mw[w] = s_m[w][qi];
      Mq = fmaxf(Mq, mw[w]);
    }
    float4 o1 = make_float4(0.f, 0.f, 0.f, 0.f), o2 = o1;
#pragma unroll
    for (int w = 0; w < kMhaWaves; ++w) {
      const float ww = (mw[w] != -__builtin_inff()) ? exp2_fast(mw[w] - Mq) : 0.f;
      Lq += s_l[w][qi] * ww;
      const float* row = reinterpret_cast<const float*>(lds + w * S::SLOT) + qi * D;
      const float4 a = *reinterpret_cast<const float4*>(row + 4 * ((dg ^ (qi & 15)) & (CH - 1)));
      const float4 c = *reinterpret_cast<const float4*>(row + 4 * (((dg + HC) ^ (qi & 15)) & (CH - 1)));
      o1.x += a.x * ww; o1.y += a.y * ww; o1.z += a.z * ww; o1.w += a.w * ww;
      o2.x += c.x * ww; o2.y += c.y * ww; o2.z += c.z * ww; o2.w += c.w * ww;
    }
    if (NS == 1) {
      if (item && qi < p.T) {
        const float inv = 1.f / Lq;
        uint16_t* dst = p.out + (seg * p.T + qi) * D + 4 * dg;
        *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(o1.x * inv, o1.y * inv), pack_bf16x2(o1.z * inv, o1.w * inv));
        *reinterpret_cast<uint2*>(dst + 4 * HC) =
            make_uint2(pack_bf16x2(o2.x * inv, o2.y * inv), pack_bf16x2(o2.z * inv, o2.w * inv));
      }
    } else if (item) {
      float* dst = po_base + ((seg * NS + s) * 32 + qi) * D + 4 * dg;
      *reinterpret_cast<float4*>(dst) = o1;
      *reinterpret_cast<float4*>(dst + 4 * HC) = o2;
      if (dg == 0) pml_base[(seg * NS + s) * 32 + qi] = make_float2(Mq, Lq);
    }
  }
  // grouped-query heads: attn_combine_kernel merges the splits; the safe mode merges in a second
  // launch too (attn_merge_kernel, the same arithmetic)
  if (NS == 1 || GQA || SAFE || (!SEL && !p.merge_here)) {
    clear_sinks();
    return;
  }

  // ---- same-XCD hand-over: the last split of this head to finish merges all of them.  The
  //      partials sit in this XCD's L2: wait until our stores are acknowledged by it, take a
  //      ticket (which counts the takers per XCD), and the last taker drops its L1 copies before
  //      reading the partials back -- if every split ran on its XCD; otherwise the partials of
  //      the others are not in its L2, and the head's output is reported invalid. ----
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    bool here = true;
    s_ticket = take_ticket(p.tickets + seg * kSyncStride, NS, &here);
    s_here = here ? 1u : 0u;
  }
  __syncthreads();
  FDL_STAMP(p, 9);
  if (s_ticket != (uint32_t)(NS - 1)) {
    clear_sinks();
    return;
  }
  if (s_here == 0u) {   // uniform
    if (tid == 0) {
      latch(p.status, ST_SPLIT_PLACEMENT);
      reset_ticket(p.tickets + seg * kSyncStride);
    }
    clear_sinks();
    return;
  }
  asm volatile("buffer_inv sc0" ::: "memory");   // later loads miss L1 and read the partials from L2
  merge_splits<D>(p, po_base, pml_base, p_out, p_T, seg, NS, reinterpret_cast<float2*>(lds));
  if (tid == 0) {
    reset_ticket(p.tickets + seg * kSyncStride);
    // the tagged score exchange of this launch is over for every split: the next launch's tag
    if (SEL && p.fs.xchg != nullptr && p.n_units <= kMhaWaves * 64)
      __hip_atomic_fetch_add(&p.fs.barriers[seg * kSyncStride + 1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  FDL_STAMP(p, 10);
  clear_sinks();
}

// The safe mode's merge: one workgroup per (sequence, query head) merges its NS partials exactly as
// the last split does in the fused launch (merge_splits), after the kernel boundary has made them
// visible everywhere.
template <int D>
__global__ __launch_bounds__(kMhaWaves * 64) void attn_merge_kernel(const MhaParams p) {
  __shared__ float2 s_ml2[kMaxSplits * 32];
  merge_splits<D>(p, p.part_o, p.part_ml, p.out, p.T, (int64_t)blockIdx.x, p.n_splits, s_ml2);
}

// Merge the per-split partials (max, sum, O) of every head into the bf16 output (grouped-query
// heads, whose splits run on different XCDs).  Separate kernel: the kernel boundary makes the
// partials visible without a device-wide cache flush.
// grid (B*H, ceil(T / QW)), 4 waves: lane (query qb + lane / CH, 16-byte chunk lane % CH); wave w
// takes the splits w, w + 4, ...; the four waves' (max, sum, O) meet in LDS.
template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(const float* __restrict__ part_o,
                                                           const float2* __restrict__ part_ml,
                                                           uint16_t* __restrict__ out, int NS, int T) {
  constexpr int CH = D / 4;      // 16-byte chunks per row
  constexpr int QW = 64 / CH;    // queries per workgroup
  constexpr int NB = 4;          // splits in flight per lane
  __shared__ float s_m[4][64], s_l[4][64];
  __shared__ float4 s_o[4][64];
  const int64_t seg = blockIdx.x;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int q = blockIdx.y * QW + lane / CH, c = lane % CH;
  const int qc = q < 32 ? q : 31;   // partial rows exist for all 32 queries
  const float2* ml = part_ml + seg * NS * 32 + qc;
  const float* po = part_o + (seg * NS * 32 + qc) * D + 4 * c;
  float M = -__builtin_inff();
  float Ls = 0.f;
  float4 O = make_float4(0.f, 0.f, 0.f, 0.f);
  if (NS <= 4 * NB) {   // uniform: every split of this lane's in one round trip, statistics and partials
    float4 a[NB];
    float2 v[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int t = w + 4 * j < NS ? w + 4 * j : 0;   // reads past NS: split 0, never used
      a[j] = *reinterpret_cast<const float4*>(po + (int64_t)t * 32 * D);
      v[j] = ml[t * 32];
    }
#pragma unroll
    for (int j = 0; j < NB; ++j)
      if (w + 4 * j < NS) M = fmaxf(M, v[j].x);
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const float wt = (w + 4 * j < NS && v[j].x != -__builtin_inff()) ? exp2f(v[j].x - M) : 0.f;
      Ls += v[j].y * wt;
      O.x += a[j].x * wt; O.y += a[j].y * wt; O.z += a[j].z * wt; O.w += a[j].w * wt;
    }
  }
  if (NS > 4 * NB)   // uniform: the statistics first, then the partials in batches
    for (int t = w; t < NS; t += 4) M = fmaxf(M, ml[t * 32].x);
  for (int t0 = (NS <= 4 * NB ? NS : w); t0 < NS; t0 += 4 * NB) {
    float4 a[NB];
    float2 v[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int t = t0 + 4 * j < NS ? t0 + 4 * j : w;   // clamped reads go out together
      a[j] = *reinterpret_cast<const float4*>(po + (int64_t)t * 32 * D);
      v[j] = ml[t * 32];
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const float wt = (t0 + 4 * j < NS && v[j].x != -__builtin_inff()) ? exp2f(v[j].x - M) : 0.f;
      Ls += v[j].y * wt;
      O.x += a[j].x * wt; O.y += a[j].y * wt; O.z += a[j].z * wt; O.w += a[j].w * wt;
    }
  }
  s_m[w][lane] = M;
  s_l[w][lane] = Ls;
  s_o[w][lane] = O;
  __syncthreads();
  if (w != 0 || q >= T) return;
  float Mx = s_m[0][lane];
#pragma unroll
  for (int k = 1; k < 4; ++k) Mx = fmaxf(Mx, s_m[k][lane]);
  float L = 0.f;
  float4 R = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float mk = s_m[k][lane];
    const float wt = mk != -__builtin_inff() ? exp2f(mk - Mx) : 0.f;
    const float4 o = s_o[k][lane];
    L += s_l[k][lane] * wt;
    R.x += o.x * wt; R.y += o.y * wt; R.z += o.z * wt; R.w += o.w * wt;
  }
  const float inv = 1.f / L;
  *reinterpret_cast<uint2*>(out + (seg * T + q) * D + 4 * c) =
      make_uint2(pack_bf16x2(R.x * inv, R.y * inv), pack_bf16x2(R.z * inv, R.w * inv));
}

hipError_t launch_attn_combine(hipStream_t st, const float* part_o, const float2* part_ml, void* out,
                               int n_segs, int NS, int T, int D) {
  const int qw = 64 / (D / 4);
  dim3 grid(n_segs, (T + qw - 1) / qw);
  uint16_t* o = static_cast<uint16_t*>(out);
  if (D == 128) {
    hipLaunchKernelGGL((attn_combine_kernel<128>), grid, dim3(256), 0, st, part_o, part_ml, o, NS, T);
  } else {
    hipLaunchKernelGGL((attn_combine_kernel<64>), grid, dim3(256), 0, st, part_o, part_ml, o, NS, T);
  }
  return hipGetLastError();
}

int mha_choose_splits(const Geom& g, long long max_list_tokens, int num_cus) {
  const long long tiles = 1 + (max_list_tokens + kTileTok - 1) / kTileTok;
  const long long segs = (long long)g.B * g.Hkv;
  // At most one 8-wave workgroup per CU of every XCD (a second round on some CUs would double the
  // time): one q-head per KV head puts all splits of a head on one XCD, ceil(segs / 8) heads each;
  // grouped-query heads put G workgroups per (KV head, split) group on one XCD.
  const long long per_xcd = num_cus / 8 > 0 ? num_cus / 8 : 1;
  long long s;
  if (g.G == 1) {
    s = per_xcd / ((segs + 7) / 8);
  } else {
    const long long groups_per_xcd = per_xcd / g.G > 0 ? per_xcd / g.G : 1;
    s = 8 * groups_per_xcd / segs;
  }
  const long long per_wave_min = 1;
  if (s * kMhaWaves * per_wave_min > tiles) s = (tiles + kMhaWaves - 1) / kMhaWaves;
  if (s < 1) s = 1;
  if (s > kMaxSplits) s = kMaxSplits;
  if (g.G == 1 && segs > kMaxSplitSegs) s = 1;   // the in-kernel merge's tickets
  return (int)s;
}

// With a timer, the kernel is launched with hipExtLaunchKernelGGL so that the two events carry the
// dispatch's own start and end timestamps (no event packets around it).
template <typename Kern>
static void launch_one(Kern kern, dim3 grid, hipStream_t st, const MhaParams& p, const KernelTimer* timer) {
  const dim3 block(kMhaWaves * 64);
  if (timer) hipExtLaunchKernelGGL(kern, grid, block, 0, st, timer->a, timer->b, 0, p);
  else hipLaunchKernelGGL(kern, grid, block, 0, st, p);
}

template <int D>
static hipError_t launch_mha_d(hipStream_t st, const MhaParams& p, dim3 grid, bool dense, bool paged, bool sel,
                               const KernelTimer* timer) {
  const bool safe = !p.merge_here;
  if (sel && p.G > 1) {
    if (safe) launch_one(attn_mha_kernel<D, false, false, true, true, true>, grid, st, p, timer);
    else launch_one(attn_mha_kernel<D, false, false, true, true>, grid, st, p, timer);
  } else if (sel) {
    if (safe) launch_one(attn_mha_kernel<D, false, false, true, false, true>, grid, st, p, timer);
    else launch_one(attn_mha_kernel<D, false, false, true>, grid, st, p, timer);
  } else if (p.G > 1) {
    if (dense && paged) launch_one(attn_mha_kernel<D, true, true, false, true>, grid, st, p, timer);
    else if (dense) launch_one(attn_mha_kernel<D, true, false, false, true>, grid, st, p, timer);
    else if (paged) launch_one(attn_mha_kernel<D, false, true, false, true>, grid, st, p, timer);
    else launch_one(attn_mha_kernel<D, false, false, false, true>, grid, st, p, timer);
  } else if (dense) {
    if (paged) launch_one(attn_mha_kernel<D, true, true, false>, grid, st, p, timer);
    else launch_one(attn_mha_kernel<D, true, false, false>, grid, st, p, timer);
  } else {
    if (paged) launch_one(attn_mha_kernel<D, false, true, false>, grid, st, p, timer);
    else launch_one(attn_mha_kernel<D, false, false, false>, grid, st, p, timer);
  }
  return hipGetLastError();
}

hipError_t launch_attn_mha(hipStream_t st, const Geom& g, const void* q, const void* k, const void* v,
                           const void* k_dec, const void* v_dec, const int32_t* page_table,
                           const int32_t* sel_idx, const int32_t* n_sel, int max_sel, int unit_log2,
                           int dense, void* out, char* scratch, int n_splits, uint32_t* tickets,
                           uint32_t* status, int n_hint, const KernelTimer* timer, const FusedSelect* fsel,
                           bool safe) {
  MhaParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.k_dec = static_cast<const uint16_t*>(k_dec);
  p.v_dec = static_cast<const uint16_t*>(v_dec);
  p.sel_idx = sel_idx;
  p.n_sel = n_sel;
  p.out = static_cast<uint16_t*>(out);
  const size_t per = (size_t)g.B * g.Hq * n_splits * 32;
  p.part_o = reinterpret_cast<float*>(scratch);
  p.part_ml = reinterpret_cast<float2*>(scratch + per * g.D * sizeof(float));
  p.tickets = tickets;
  p.status = status;
  p.page_table = page_table;
  p.H = g.Hq;
  p.T = g.T;
  p.L = g.L;
  p.max_sel = max_sel;
  p.unit_log2 = unit_log2;
  p.n_units = (g.L + (1 << unit_log2) - 1) >> unit_log2;
  p.n_splits = n_splits;
  p.page_log2 = g.page_log2;
  p.pages_per_seq = g.pps;
  p.n_pages = g.n_pages;
  p.scale_log2 = 1.4426950408889634f / sqrtf((float)g.D);
  p.n_segs = g.B * g.Hq;
  p.Hkv = g.Hkv;
  p.G = g.G;
  p.n_groups = g.B * g.Hkv * n_splits;
  p.n_hint = dense ? 0 : n_hint;
  p.merge_here = safe ? 0 : 1;
  p.lens = g.lens;
  p.fs = fsel ? *fsel : FusedSelect{};
  // 8 XCDs: the splits of head seg run on XCD seg % 8; grouped-query heads: the G heads of KV
  // group i (a KV head and a split) run on XCD i % 8 (see the kernel)
  const dim3 grid(g.G == 1 ? 8 * ((p.n_segs + 7) / 8) * n_splits : 8 * ((p.n_groups + 7) / 8) * g.G);
  if (p.fs.stamps != nullptr && p.fs.stamp_words < (int64_t)grid.x * kStampsPerGroup) p.fs.stamps = nullptr;
  const bool sel = fsel != nullptr && !dense && !g.paged;
  if (sel && g.G > 1 && p.n_groups > kMaxSplitSegs) return hipErrorInvalidValue;   // barrier words
  const hipError_t err = g.D == 128 ? launch_mha_d<128>(st, p, grid, dense != 0, g.paged != 0, sel, timer)
                                    : launch_mha_d<64>(st, p, grid, dense != 0, g.paged != 0, sel, timer);
  if (err != hipSuccess || n_splits == 1) return err;
  if (g.G == 1) {
    if (!safe) return err;
    // safe mode: the partials are merged after the kernel boundary, with the fused merge's arithmetic
    const dim3 mgrid(g.B * g.Hq), mblock(kMhaWaves * 64);
    if (g.D == 128) hipLaunchKernelGGL(attn_merge_kernel<128>, mgrid, mblock, 0, st, p);
    else hipLaunchKernelGGL(attn_merge_kernel<64>, mgrid, mblock, 0, st, p);
    return hipGetLastError();
  }
  return launch_attn_combine(st, p.part_o, p.part_ml, out, g.B * g.Hq, n_splits, g.T, g.D);
}

}  // namespace fdl
