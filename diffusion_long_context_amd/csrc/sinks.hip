// Attention-sink detection at the source layer.
//
// Focus-dLLM (abstract; Elamur "Summary" and "Key points"): highly influential attention sinks must
// survive pruning, and since sink locations agree across layers they are found once and reused
// deeper.  The pages give no detection rule; the reading built here: for every q-head and
// predicted position p, take the softmax row of q_p . k_t / sqrt(D) over all cached tokens and the
// block's own tokens; a cached token whose mean weight over the predicted positions reaches tau for
// some head is a sink; the union over heads is the sequence's sink list (ascending).
//
// One pass over K (the only full-K read of a step): each wave streams 64-token tiles through bf16
// MFMA (S^T = K Q^T) and keeps a running log-sum-exp per query.  Because a running log-sum-exp never
// exceeds the final one, the mass a token gets under the running statistics is an upper bound of
// its true mass, so every token whose bound reaches tau (less a small rounding margin) is recorded
// as a candidate.  In the same kernel, the last workgroup of each head merges the partial
// statistics into the exact log-sum-exp, re-scores the head's few candidates in float32 and sets
// the survivors in a per-sequence bitmap.  A second kernel compacts the bitmap into the ascending
// sink list; in the step driver the fused kernel of the same layer, which runs next, reads the
// bitmap itself and writes the list.  When the scan is the step's first reader of the predicted
// query set, it also computes that set (wave 0 of every workgroup) and writes it out.
#include "fdl_device.h"
#include "fdl_internal.h"
#include "fdl_predict.h"
#include "fdl_stream.h"

namespace fdl {

// Diagnostic build (FDL_PHASE_STAMPS): thread 0 of each workgroup records s_memrealtime (100 MHz) at
// the points of the scan; nothing in the normal build.
#ifdef FDL_PHASE_STAMPS
#define SINK_STAMP(p, i)                                                                               \
  do {                                                                                                 \
    if (threadIdx.x == 0 && (p).stamps != nullptr)                                                     \
      (p).stamps[(int64_t)blockIdx.x * 16 + (i)] = __builtin_amdgcn_s_memrealtime();                   \
  } while (0)
#else
#define SINK_STAMP(p, i) \
  do {                   \
  } while (0)
#endif

__global__ void fill_u32_kernel(uint32_t* __restrict__ p, size_t n, uint32_t v) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}

hipError_t launch_fill_u32(hipStream_t s, uint32_t* p, size_t n, uint32_t v) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// One level of a transposing sum over lanes: values [0, 2H) -> [0, H).  A lane with bit J clear keeps
// its values [0, H) plus the partner's (lane ^ J) values [0, H); a lane with bit J set keeps its
// values [H, 2H) plus the partner's [H, 2H), stored at [0, H).
template <int H, int J>
__device__ __forceinline__ void reduce_half(float (&u)[16], int lane) {
  const bool up = (lane & J) != 0;
#pragma unroll
  for (int i = 0; i < H; ++i) {
    const float send = up ? u[i] : u[i + H];
    const float keep = up ? u[i + H] : u[i];
    u[i] = keep + __uint_as_float(lane_xor<J>(__float_as_uint(send)));
  }
}

constexpr float kCandSlack = 0.999f;
constexpr int kSinkLocalCand = 128;     // candidates a wave keeps in LDS before appending   // candidates use tau * (1 - 1e-3): absorbs float32 rounding
constexpr int kSinkWaves = 4;
constexpr int kSinkTile = 64;           // tokens per tile

struct SinkParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* k_dec;
  const uint64_t* pred_mask;
  // when pconf_given: the scan computes the prediction itself from these (the step's first reader
  // of it) and the workgroup of head 0, split 0 of each sequence writes it to pred_out / n_pred_out
  const float* pconf;
  const uint8_t* pmasked;
  uint64_t* pred_out;
  int32_t* n_pred_out;
  int pconf_given, ptop_k, pwindow;
  float2* stats;         // [B * Hq][n_splits * 4][32]  (running max in log2 units, running sum)
  uint32_t* cand_count;  // [B * Hq], zero on entry; the head's last split zeroes it again
  uint32_t* cand;        // [B * Hq][cand_cap]  token positions
  uint32_t* bitmap;      // [B][words], zero on entry; zeroed again by sink_compact_kernel or, in
                         // the step driver, by a later fused launch (or a fill)
  uint32_t* tickets;     // per (b, q-head), kSyncStride apart; left at zero
  uint32_t* status;
  const int32_t* lens;   // per-sequence cached lengths of a ragged batch, or NULL (all L)
  uint64_t* stamps;      // diagnostic build: per-workgroup phase timestamps, or NULL
  int Hq, Hkv, G, T, L, n_splits, n_segs, cand_cap, words;
  float scale_log2, tau;
};

// One pass over K per (sequence, q-head), split over n_splits workgroups of 4 waves that all run on
// one XCD (workgroup id mod 8).  Each wave streams 64-token tiles of K from HBM into its own 16 KiB
// LDS slot with LDS DMA (coalesced 1 KiB fetches), copies a tile into MFMA operand registers and
// fetches the next one into the slot while the current one is scored.  The last split of a head to
// finish (ticket) merges the partial statistics into the exact log-sum-exp per query, re-scores
// the head's candidates in float32 and sets the survivors in the sequence's bitmap.
// Placement: workgroup i runs on XCD i % 8; slot k = xcd + 8 (xslot / NS) and its NS splits share
// that XCD.  Slots go to q-heads KV-segment-major (k = kv + (B Hkv) j for the j-th head of KV
// segment kv), so the q-heads of one KV head sit on as few XCDs as there are slots per XCD for them
// and read the KV head's key tiles through one L2 (default cache policy for grouped-query heads;
// one reader per tile streams non-temporally).  With one q-head per KV head, k is the head.
template <int D, bool GQA>
__global__ __launch_bounds__(kSinkWaves * 64, 2) void sink_scan_kernel(const SinkParams p) {
  constexpr int POL = GQA ? 0 : kStreamPolicy;
  constexpr int KS = D / 16;
  constexpr int RB = kSinkTile / 32;   // 32-row MFMA blocks per tile
  using RC = RowChunks<D>;
  constexpr int PROW = RC::PROW, RPI = RC::ROWS_PER_INSTR, NI = kSinkTile / RPI;
  __shared__ __attribute__((aligned(1024))) uint16_t kslot[kSinkWaves * kSinkTile * D];
  __shared__ float2 s_part[8][32];
  __shared__ float2 s_run[kSinkWaves][32];   // each wave's latest running (max, sum) per query
  // Candidates found by each wave, kept in its quarter of an LDS list during the scan with the count
  // in a register (a global atomic's result, and an LDS atomic, would each be waited for behind the
  // tile fetch in flight), appended to the head's list after the scan.
  __shared__ uint32_t s_cand[kSinkWaves][kSinkLocalCand];
  __shared__ uint32_t s_ncand[kSinkWaves], s_cbase;
  __shared__ float s_lse[32];
  __shared__ uint32_t s_ticket, s_here;
  const int NS = p.n_splits;
  const int xcd = blockIdx.x & 7, xslot = blockIdx.x >> 3;
  const int s = xslot % NS;
  const int k_slot = xcd + 8 * (xslot / NS);
  if (k_slot >= p.n_segs) return;
  SINK_STAMP(p, 0);
#ifdef FDL_PHASE_STAMPS
  if (threadIdx.x == 0 && p.stamps != nullptr)
    p.stamps[(int64_t)blockIdx.x * 16 + 15] = (uint64_t)xcc_reg() | ((uint64_t)1 << 63);
#endif
  const int n_kv = p.n_segs / p.G;   // (sequence, KV head) segments
  const int kvs = k_slot % n_kv, jh = k_slot / n_kv;
  const int b = kvs / p.Hkv, g = kvs % p.Hkv, h = g * p.G + jh;
  const int seg = b * p.Hq + h;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ql = lane & 31, hh = lane >> 5;
  const int n_parts = NS * kSinkWaves;
  const int Lb = seq_len(p.lens, b, p.L);   // this sequence's cached tokens; its rows stay p.L apart
  float m_run = -__builtin_inff(), l_run = 0.f;
  if (tid < kSinkWaves * 32) s_run[tid >> 5][tid & 31] = make_float2(-__builtin_inff(), 0.f);
  const uint16_t* kdec = p.k_dec + ((int64_t)b * p.Hkv + g) * p.T * D;
  const uint16_t* kctx = p.k + ((int64_t)b * p.Hkv + g) * (int64_t)p.L * D;
  // The query rows and each wave's first tile are requested before anything waits: the
  // prediction below (and its barrier) overlaps their round trip.
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
  const int n_tiles = 1 + (Lb + kSinkTile - 1) / kSinkTile;
  const int e0 = (int)((int64_t)n_tiles * s / NS);
  const int e1 = (int)((int64_t)n_tiles * (s + 1) / NS);
  // tile e -> the wave's slot; rows are clamped so that every fetch is in bounds.  A full cache
  // tile is one run of kSinkTile rows: a scalar base plus per-lane chunk offsets fixed up front.
  uint16_t* slot = kslot + wave * kSinkTile * D;
  uint32_t voff[NI];
  {
    const int rsub = lane / PROW, sc = lane % PROW;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int r = j * RPI + rsub;
      voff[j] = (uint32_t)((r * D + (sc ^ (swz(r) & (PROW - 1))) * 8) * 2);
    }
  }
  auto issue = [&](int e) {
    const int rsub = lane / PROW, sc = lane % PROW;
    if (e > 0 && e * kSinkTile <= Lb) {   // uniform: a full tile of the cache
      const char* base = reinterpret_cast<const char*>(kctx + (int64_t)(e - 1) * kSinkTile * D);
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const void* src = base + voff[j];
        __builtin_amdgcn_global_load_lds(src, (lds_void_t*)(slot + j * 512), 16, 0, POL);
      }
      return;
    }
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int r = j * RPI + rsub;
      const int t = (e - 1) * kSinkTile + r;
      const uint16_t* row = (e == 0) ? kdec + (int64_t)(r < p.T ? r : p.T - 1) * D
                                     : kctx + (int64_t)(t < Lb ? t : Lb - 1) * D;
      const void* src = row + (sc ^ (swz(r) & (PROW - 1))) * 8;
      __builtin_amdgcn_global_load_lds(src, (lds_void_t*)(slot + j * 512), 16, 0, POL);
    }
  };
  int e = e0 + wave;
  if (e < e1) issue(e);
  __shared__ uint64_t s_pred;
  if (p.pconf_given) {   // uniform: wave 0 predicts the sequence's queries
    if (wave == 0) {
      const uint64_t pm = predict_mask(p.T, p.pconf ? p.pconf + (int64_t)b * p.T : nullptr,
                                       p.pmasked + (int64_t)b * p.T, p.ptop_k, p.pwindow, lane);
      if (lane == 0) {
        s_pred = pm;
        if (h == 0 && s == 0) {
          p.pred_out[b] = pm;
          p.n_pred_out[b] = __popcll(pm);
        }
      }
    }
  } else if (tid == 0) {
    s_pred = p.pred_mask[b];
  }
  __syncthreads();   // also: the queries and the first tiles have landed
  const uint64_t pred = s_pred;
  const int n_pred = __popcll(pred);
  uint32_t n_local = 0;   // this wave's candidates in s_cand[wave] (uniform)
  if (n_pred > 0) {   // uniform
    const bool qlive = ql < p.T && ((pred >> ql) & 1ull);
    const float inv_np = 1.f / (float)n_pred;
    const int swz_k = swz(ql) & (PROW - 1);
    // Upper-bound masses of a scored tile under the current running statistics, summed over the
    // predicted queries; tokens whose bound reaches tau become candidates.  A token's mean reaches
    // the threshold only if some single query's bound does, so a tile where none does is skipped
    // at once (the usual case: only sink tiles pass).  Register r of block rb holds token
    // 32 rb + 8 (r / 4) + 4 hh + r % 4 for query ql.
    const float log2_thr = __log2f(p.tau * kCandSlack);
    // The bound's log-sum-exp covers this wave's tokens and the ones the workgroup's other waves
    // have scored so far (their latest (max, sum), published in LDS as one 8-byte pair): a log-sum-
    // exp over any subset of the row stays below the row's own, so the bound stays an upper bound,
    // and with four waves' tokens it is tight enough that most tiles are not evaluated further.
    auto eval_tile = [&](const f32x16 (&sc)[RB], int et, int nv) {
      float mc = m_run, lc = l_run;
#pragma unroll
      for (int w = 0; w < kSinkWaves; ++w) {
        if (w == wave) continue;
        const float2 o = s_run[w][ql];
        if (o.y > 0.f) {
          const float mn = fmaxf(mc, o.x);
          lc = lc * exp2f(mc - mn) + o.y * exp2f(o.x - mn);
          mc = mn;
        }
      }
      const float lse = mc + __log2f(lc);
      bool hot = false;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int r = 0; r < 16; ++r) hot = hot || (qlive && sc[rb][r] - lse >= log2_thr);
      if (__ballot(hot) == 0ull) return;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        // sum over the 32 queries (lanes of a half) of the 16 token registers by a transposing
        // reduction: at the level of lane distance J the lane keeps half of its values and sends the
        // other half, so the count halves each level; lane ql of a half ends with the sum of token
        // register tr = 8 b0 + 4 b1 + 2 b2 + b3 (b_i = bit i of ql; lanes ql and ql ^ 16 agree)
        float u[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) u[r] = qlive ? exp2_fast(sc[rb][r] - lse) : 0.f;
        reduce_half<8, 1>(u, ql);
        reduce_half<4, 2>(u, ql);
        reduce_half<2, 4>(u, ql);
        reduce_half<1, 8>(u, ql);
        const float mine = u[0] + __uint_as_float(lane_xor<16>(__float_as_uint(u[0])));
        const int tr = 8 * (ql & 1) + 4 * ((ql >> 1) & 1) + 2 * ((ql >> 2) & 1) + ((ql >> 3) & 1);
        const int row = 32 * rb + 8 * (tr >> 2) + 4 * hh + (tr & 3);
        const bool is_cand = ql < 16 && row < nv && mine * inv_np >= p.tau * kCandSlack;
        const uint64_t cm = __ballot(is_cand);
        if (is_cand) {
          const uint32_t tok = (uint32_t)((et - 1) * kSinkTile + row);
          const uint32_t li = n_local + (uint32_t)__popcll(cm & ((1ull << lane) - 1ull));
          if (li < (uint32_t)kSinkLocalCand) {
            s_cand[wave][li] = tok;
          } else {   // the wave's list is full: straight to the head's list
            const uint32_t idx = atomicAdd(&p.cand_count[seg], 1u);
            if ((int)idx < p.cand_cap) p.cand[(int64_t)seg * p.cand_cap + idx] = tok;
            else latch(p.status, ST_CAND_OVERFLOW);
          }
        }
        n_local += (uint32_t)__popcll(cm);
      }
    };
    f32x16 sprev[RB];
    int prev_e = 0, prev_nvalid = 0;   // prev_e == 0: nothing pending (tile 0 is never evaluated)
    for (; e < e1; e += kSinkWaves) {
      wait_vm0();   // this tile's fetches have landed
      if (e == e0) SINK_STAMP(p, 1);
      // lane (token ql of block rb, half hh): dims hh*D/2 + 8 ks .. +8, as the MFMA A operand
      uint4 ka[RB][KS];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int c = hh * (PROW / 2) + ks;
          ka[rb][ks] = *reinterpret_cast<const uint4*>(slot + (32 * rb + ql) * D + ((c ^ swz_k) * 8));
        }
      wait_lgkm0();
      if (e + kSinkWaves < e1) issue(e + kSinkWaves);   // next tile flies while this one is scored
      const int nvalid = (e == 0) ? p.T : min(kSinkTile, Lb - (e - 1) * kSinkTile);
      f32x16 sacc[RB];
      float mx = -__builtin_inff();
      {
        // two independent accumulation chains per 32-row block (even and odd k-steps), so that
        // the MFMA latency of one chain is covered by the other
        f32x16 acc2[RB][2];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc2[rb][0][r] = acc2[rb][1][r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) acc2[rb][ks & 1] = mfma32(as_bf16x8(ka[rb][ks]), qf[ks], acc2[rb][ks & 1]);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[rb][r] = acc2[rb][0][r] + acc2[rb][1][r];
      }
      if (nvalid == kSinkTile) {   // uniform: every row of the tile is valid
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            sacc[rb][r] *= p.scale_log2;
            mx = fmaxf(mx, sacc[rb][r]);
          }
      } else {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = 32 * rb + 8 * (r >> 2) + 4 * hh + (r & 3);
            float x = sacc[rb][r] * p.scale_log2;
            if (row >= nvalid) x = -__builtin_inff();
            sacc[rb][r] = x;
            mx = fmaxf(mx, x);
          }
      }
      mx = fmaxf(mx, lane_xor32f(mx));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = exp2_fast(m_run - m_new);
      float rs = 0.f;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int r = 0; r < 16; ++r) rs += exp2_fast(sacc[rb][r] - m_new);
      rs += lane_xor32f(rs);
      l_run = l_run * alpha + rs;
      m_run = m_new;
      if (hh == 0) s_run[wave][ql] = make_float2(m_run, l_run);
      // candidates of the previous tile, bounded with the statistics that now include this one
      // (a one-tile delay, so that no bound rests on a single tile of tokens)
      if (prev_e > 0) eval_tile(sprev, prev_e, prev_nvalid);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) sprev[rb] = sacc[rb];
      prev_e = e;
      prev_nvalid = nvalid;
    }
    if (prev_e > 0) eval_tile(sprev, prev_e, prev_nvalid);   // the last tile, under the final stats
    SINK_STAMP(p, 2);
  }
  if (hh == 0) p.stats[((int64_t)seg * n_parts + s * kSinkWaves + wave) * 32 + ql] = make_float2(m_run, l_run);
  // append the workgroup's candidates to the head's list (one global atomic reserves the range)
  if (lane == 0) s_ncand[wave] = n_local < (uint32_t)kSinkLocalCand ? n_local : (uint32_t)kSinkLocalCand;
  __syncthreads();
  {
    uint32_t nw[kSinkWaves], nl = 0;
#pragma unroll
    for (int w = 0; w < kSinkWaves; ++w) {
      nw[w] = s_ncand[w];
      nl += nw[w];
    }
    if (nl > 0u) {   // uniform
      if (tid == 0) s_cbase = atomicAdd(&p.cand_count[seg], nl);
      __syncthreads();
      uint32_t base = s_cbase;
#pragma unroll
      for (int w = 0; w < kSinkWaves; ++w) {
        for (uint32_t i = tid; i < nw[w]; i += kSinkWaves * 64) {
          if (base + i < (uint32_t)p.cand_cap) p.cand[(int64_t)seg * p.cand_cap + base + i] = s_cand[w][i];
          else if (base + i == (uint32_t)p.cand_cap) latch(p.status, ST_CAND_OVERFLOW);
        }
        base += nw[w];
      }
    }
  }

  // ---- the last split of the head (same XCD, so the partials are in its L2) finishes it; the
  //      ticket counts the takers per XCD, and a head whose splits ran on different XCDs is
  //      reported instead (its partials are not all in one L2) ----
  if (NS > 1) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    SINK_STAMP(p, 3);
    if (tid == 0) {
      bool here = true;
      s_ticket = take_ticket(p.tickets + seg * kSyncStride, NS, &here);
      s_here = here ? 1u : 0u;
    }
    __syncthreads();
    SINK_STAMP(p, 4);
    if (s_ticket != (uint32_t)(NS - 1)) return;
    if (tid == 0) reset_ticket(p.tickets + seg * kSyncStride);
    if (s_here == 0u) {   // uniform
      if (tid == 0) {
        latch(p.status, ST_SPLIT_PLACEMENT);
        p.cand_count[seg] = 0u;
      }
      return;
    }
    // later loads miss L1 and read the other splits' statistics and candidates from L2 (no wait:
    // the invalidation is ordered before them)
    asm volatile("buffer_inv sc0" ::: "memory");
  } else {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  if (n_pred == 0) return;
  // What the re-scoring needs is requested before the log-sum-exp merge waits for its statistics:
  // the head's candidate count, each wave's first candidate and, once that is back, its key row
  // (lane (q, hh) the half hh of the row; the queries are still in the MFMA fragments qf).  Reads
  // past the count are clamped in bounds and never used.
  const int count_raw = (int)__hip_atomic_load(&p.cand_count[seg], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint32_t* cand_row = p.cand + (int64_t)seg * p.cand_cap;
  auto load_key_half = [&](uint32_t t, uint4 (&kr)[KS]) {
    const uint16_t* row = kctx + (int64_t)(t < (uint32_t)p.L ? t : 0u) * D + hh * (D / 2);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kr[ks] = *reinterpret_cast<const uint4*>(row + ks * 8);
  };
  const uint32_t t_first = cand_row[wave < p.cand_cap ? wave : p.cand_cap - 1];
  uint4 kr[KS];
  {
    // exact log-sum-exp per query: thread (q, j) merges parts j, j + 8, ...; then 8 -> 1
    const int q = tid & 31, j = tid >> 5;
    float M = -__builtin_inff(), S = 0.f;
    // the parts j, j + 8, ... are loaded kPartBatch at a time before any is used
    constexpr int kPartBatch = 8;
    float2 v[kPartBatch];
    auto load_parts = [&](int i0) {
#pragma unroll
      for (int u = 0; u < kPartBatch; ++u) {
        const int i = i0 + 8 * u;
        v[u] = p.stats[((int64_t)seg * n_parts + (i < n_parts ? i : j)) * 32 + q];
      }
    };
    load_parts(j);
    __builtin_amdgcn_sched_barrier(0);
    // the first candidate's key row goes out as soon as its index is back (the statistics stay in
    // flight: they were requested after it)
    load_key_half(t_first, kr);
    for (int i0 = j; i0 < n_parts; i0 += 8 * kPartBatch) {
      if (i0 != j) load_parts(i0);
#pragma unroll
      for (int u = 0; u < kPartBatch; ++u) {
        if (i0 + 8 * u >= n_parts) break;
        if (v[u].y > 0.f) {
          const float mn = fmaxf(M, v[u].x);
          S = S * exp2f(M - mn) + v[u].y * exp2f(v[u].x - mn);
          M = mn;
        }
      }
    }
    s_part[j][q] = make_float2(M, S);
    __syncthreads();
    if (tid < 32) {
      float M2 = -__builtin_inff(), S2 = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float2 v = s_part[i][tid];
        if (v.y > 0.f) {
          const float mn = fmaxf(M2, v.x);
          S2 = S2 * exp2f(M2 - mn) + v.y * exp2f(v.x - mn);
          M2 = mn;
        }
      }
      s_lse[tid] = M2 + __log2f(S2);
    }
    __syncthreads();
    SINK_STAMP(p, 5);
  }
  // re-score this head's candidates exactly (float32), one wave per candidate: lane (q, hh) takes
  // the dot product of query q with half hh of the key row (four interleaved partial sums), the two
  // halves meet across the row pair, and the 32 queries' probabilities are summed by lane swaps
  const int count = count_raw < p.cand_cap ? count_raw : p.cand_cap;
  const bool qlive = ql < p.T && ((pred >> ql) & 1ull);
  for (int c = wave; c < count; c += kSinkWaves) {
    const uint32_t t = c == wave ? t_first : cand_row[c];
    if (c != wave) load_key_half(t, kr);
    float acc4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint4 qa = __builtin_bit_cast(uint4, qf[ks]);
      const uint32_t qw[4] = {qa.x, qa.y, qa.z, qa.w};
      const uint32_t kw[4] = {kr[ks].x, kr[ks].y, kr[ks].z, kr[ks].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc4[i] += bf16_bits_to_f32(qw[i] & 0xFFFFu) * bf16_bits_to_f32(kw[i] & 0xFFFFu);
        acc4[i] += bf16_bits_to_f32(qw[i] >> 16) * bf16_bits_to_f32(kw[i] >> 16);
      }
    }
    float dot = (acc4[0] + acc4[1]) + (acc4[2] + acc4[3]);
    dot += lane_xor32f(dot);
    float e = (hh == 0 && qlive) ? exp2f(dot * p.scale_log2 - s_lse[ql]) : 0.f;
    e += __uint_as_float(lane_xor<1>(__float_as_uint(e)));
    e += __uint_as_float(lane_xor<2>(__float_as_uint(e)));
    e += __uint_as_float(lane_xor<4>(__float_as_uint(e)));
    e += __uint_as_float(lane_xor<8>(__float_as_uint(e)));
    e += __uint_as_float(lane_xor<16>(__float_as_uint(e)));
    if (lane == 0 && e / (float)n_pred >= p.tau && t < (uint32_t)Lb)
      atomicOr(&p.bitmap[(int64_t)b * p.words + (t >> 5)], 1u << (t & 31));
  }
  // this head's candidates are consumed (every thread read the count before the loop): its count
  // is left at zero for the next detection (the compaction, when it runs, zeroes it too)
  __syncthreads();
  if (tid == 0) p.cand_count[seg] = 0u;
#ifdef FDL_PHASE_STAMPS
  __syncthreads();
  SINK_STAMP(p, 6);
  if (threadIdx.x == 0 && p.stamps != nullptr) p.stamps[(int64_t)blockIdx.x * 16 + 7] = (uint64_t)count;
#endif
}

// float32 path (small workloads): thread = query row; two passes over the keys.
template <int D>
__global__ __launch_bounds__(64) void sink_f32_kernel(const float* __restrict__ q,
                                                      const float* __restrict__ k,
                                                      const float* __restrict__ k_dec,
                                                      const uint64_t* __restrict__ pred_mask,
                                                      uint32_t* __restrict__ bitmap, int Hq, int Hkv,
                                                      int G, int T, int L, int words, float tau,
                                                      const int32_t* __restrict__ lens) {
  __shared__ float kc[32][D + 1];
  __shared__ float ev[32][65];
  const int h = blockIdx.x, b = blockIdx.y, qi = threadIdx.x;
  const int g = h / G;
  const uint64_t pred = pred_mask[b];
  const int n_pred = __popcll(pred);
  if (n_pred == 0) return;
  const bool live = qi < T && ((pred >> qi) & 1ull);
  float qr[D];
  const float* qrow = q + (((int64_t)b * Hq + h) * T + (qi < T ? qi : 0)) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) qr[d] = qrow[d];
  const float scale = 1.0f / sqrtf((float)D);
  const float* kd = k_dec + ((int64_t)b * Hkv + g) * T * D;
  const float* kx = k + ((int64_t)b * Hkv + g) * (int64_t)L * D;
  const int Lb = seq_len(lens, b, L);   // a ragged batch: this sequence's tokens (rows stay L apart)
  const int total = T + Lb;
  // pass 1: log-sum-exp over own block + cached tokens
  float m = -__builtin_inff(), l = 0.f;
  for (int c0 = 0; c0 < total; c0 += 32) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < 32 * D; idx += 64) {
      const int r = idx / D, d = idx % D, i = c0 + r;
      kc[r][d] = (i < T) ? kd[(int64_t)i * D + d] : (i < total ? kx[(int64_t)(i - T) * D + d] : 0.f);
    }
    __syncthreads();
    for (int r = 0; r < 32 && c0 + r < total; ++r) {
      float acc = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) acc += qr[d] * kc[r][d];
      const float x = acc * scale;
      const float mn = fmaxf(m, x);
      l = l * __expf(m - mn) + __expf(x - mn);
      m = mn;
    }
  }
  const float lse = m + __logf(l);
  // pass 2: masses of cached tokens
  for (int c0 = 0; c0 < Lb; c0 += 32) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < 32 * D; idx += 64) {
      const int r = idx / D, d = idx % D, t = c0 + r;
      kc[r][d] = t < Lb ? kx[(int64_t)t * D + d] : 0.f;
    }
    __syncthreads();
    for (int r = 0; r < 32; ++r) {
      float acc = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) acc += qr[d] * kc[r][d];
      ev[r][qi] = live ? __expf(acc * scale - lse) : 0.f;
    }
    __syncthreads();
    if (qi < 32 && c0 + qi < Lb) {
      float a = 0.f;
      for (int j = 0; j < 64; ++j) a += ev[qi][j];
      if (a / (float)n_pred >= tau) {
        const int t = c0 + qi;
        atomicOr(&bitmap[(int64_t)b * words + (t >> 5)], 1u << (t & 31));
      }
    }
  }
}

// Bitmap -> ascending sink positions; one workgroup per sequence.
__global__ __launch_bounds__(256) void sink_compact_kernel(uint32_t* bitmap_rw, int words, int max_sinks,
                                                           int32_t* __restrict__ sink_pos,
                                                           int32_t* __restrict__ n_sinks,
                                                           uint32_t* __restrict__ cand_count, int n_heads,
                                                           uint32_t* __restrict__ status) {
  const uint32_t* bitmap = bitmap_rw;
  __shared__ int tmp[4];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int per = (words + 255) / 256;
  const int w0 = tid * per;
  int cnt = 0;
  for (int i = 0; i < per; ++i)
    if (w0 + i < words) cnt += __popc(bitmap[(int64_t)b * words + w0 + i]);
  int incl = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
  if (lane == 63) tmp[wave] = incl;
  __syncthreads();
  int off = 0, total = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    if (w < wave) off += tmp[w];
    total += tmp[w];
  }
  int pos = off + incl - cnt;
  for (int i = 0; i < per; ++i) {
    const int wi = w0 + i;
    if (wi >= words) break;
    uint32_t bits = bitmap[(int64_t)b * words + wi];
    while (bits) {
      const int bit = __ffs(bits) - 1;
      bits &= bits - 1;
      if (pos < max_sinks) sink_pos[(int64_t)b * max_sinks + pos] = wi * 32 + bit;
      ++pos;
    }
  }
  // pad the rest of the list with -1 so stale entries never look like sinks
  for (int i = total + tid; i < max_sinks; i += 256) sink_pos[(int64_t)b * max_sinks + i] = -1;
  // leave the bitmap and the candidate counts of this sequence at zero for the next detection
  for (int i = 0; i < per; ++i)
    if (w0 + i < words) bitmap_rw[(int64_t)b * words + w0 + i] = 0u;
  for (int i = tid; i < n_heads; i += 256) cand_count[(int64_t)b * n_heads + i] = 0u;
  if (tid == 0) {
    n_sinks[b] = total < max_sinks ? total : max_sinks;
    if (total > max_sinks) latch(status, ST_SINK_OVERFLOW);
  }
}

int sink_splits(const Geom& g) {
  const int n_tiles = 1 + (g.L + kSinkTile - 1) / kSinkTile;
  const long long segs = (long long)g.B * g.Hq;
  if (segs > kMaxSplitSegs) return 1;
  // about two 4-wave workgroups per CU (the kernel's occupancy) over all (sequence, q-head) pairs
  int s = (int)((2LL * 256 + segs - 1) / segs);
  // at least 4 tiles per wave, so that candidate bounds rest on enough tokens to be tight (with a
  // one-tile delay, the first bound of a wave covers 128 tokens)
  const int cap = n_tiles / (kSinkWaves * 4);
  if (s > cap) s = cap;
  return s < 1 ? 1 : s;
}

// Candidate counts and bitmap stay zero between detections: in the header's sink area when they
// fit there, else in scratch (cleared by a fill before every detection).
static bool sink_state_in_header(const Geom& g) {
  const size_t words = (size_t)(g.L + 31) / 32;
  return ((size_t)g.B * g.Hq + (size_t)g.B * words) * sizeof(uint32_t) <= kSinkAreaBytes;
}

uint32_t* sink_bitmap_for(const Geom& g, char* sink_area, int* words) {
  *words = (g.L + 31) / 32;
  if (g.dtype == FDL_F32 || g.L <= 0 || !sink_state_in_header(g)) return nullptr;
  return reinterpret_cast<uint32_t*>(sink_area) + (size_t)g.B * g.Hq;
}

size_t sink_scratch_bytes(const Geom& g, int* n_splits, int* cand_cap) {
  const int s = sink_splits(g);
  *n_splits = s;
  // candidates per (sequence, q-head): every token when the context is short (a wave then has few
  // tiles and loose bounds), else 1024 -- with 4+ tiles per wave a random token's bound is ~4 sigma
  // below tau, so only true sinks and a rare few others are candidates
  *cand_cap = g.L <= 4096 ? (g.L > 0 ? g.L : 1) : 1024;
  const int words = (g.L + 31) / 32;
  size_t bytes = 0;
  bytes += (size_t)g.B * g.Hq * s * kSinkWaves * 32 * sizeof(float2) + 256;   // stats
  bytes += (size_t)g.B * g.Hq * (*cand_cap) * sizeof(uint32_t) + 256;         // candidates
  if (!sink_state_in_header(g)) bytes += ((size_t)g.B * g.Hq + (size_t)g.B * words) * sizeof(uint32_t) + 256;
  return bytes + 1024;
}

hipError_t launch_sinks(hipStream_t st, const Geom& g, const void* q, const uint64_t* pred_mask,
                        const void* k, const void* k_dec, float tau, int max_sinks,
                        int32_t* sink_pos, int32_t* n_sinks, char* scratch, int n_splits,
                        int cand_cap, uint32_t* status, int num_cus, uint32_t* tickets,
                        char* sink_area, uint64_t* stamps, int64_t stamp_words, const PredictIn* pin,
                        bool keep_bitmap) {
  (void)num_cus;
  // the prediction, when it is asked for here: inside the scan when the scan runs, else first
  const bool scan_runs = g.dtype != FDL_F32 && g.L > 0;
  if (pin != nullptr && !scan_runs) {
    const hipError_t e = launch_predict(st, g.B, g.T, pin->conf, pin->masked, pin->top_k, pin->window,
                                        pin->pred_mask, pin->n_pred);
    if (e != hipSuccess) return e;
  }
  const int words = (g.L + 31) / 32;
  char* cur = scratch;
  auto take = [&](size_t bytes) {
    char* r = cur;
    cur += (bytes + 255) & ~(size_t)255;
    return r;
  };
  SinkParams p;
  p.stats = reinterpret_cast<float2*>(take((size_t)g.B * g.Hq * n_splits * kSinkWaves * 32 * sizeof(float2)));
  p.cand = reinterpret_cast<uint32_t*>(take((size_t)g.B * g.Hq * cand_cap * sizeof(uint32_t)));
  const bool in_header = sink_state_in_header(g);
  // counts then bitmap, contiguous
  p.cand_count = reinterpret_cast<uint32_t*>(
      in_header ? sink_area : take(((size_t)g.B * g.Hq + (size_t)g.B * words) * sizeof(uint32_t)));
  p.bitmap = p.cand_count + (size_t)g.B * g.Hq;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.k_dec = static_cast<const uint16_t*>(k_dec);
  p.pred_mask = pred_mask;
  p.pconf_given = pin != nullptr && scan_runs ? 1 : 0;
  p.pconf = pin ? pin->conf : nullptr;
  p.pmasked = pin ? pin->masked : nullptr;
  p.pred_out = pin ? pin->pred_mask : nullptr;
  p.n_pred_out = pin ? pin->n_pred : nullptr;
  p.ptop_k = pin ? pin->top_k : 0;
  p.pwindow = pin ? pin->window : 0;
  p.tickets = tickets;
  p.status = status;
  p.Hq = g.Hq;
  p.Hkv = g.Hkv;
  p.G = g.G;
  p.T = g.T;
  p.L = g.L;
  p.lens = g.lens;
  p.stamps = nullptr;
  p.n_splits = n_splits;
  p.n_segs = g.B * g.Hq;
  p.cand_cap = cand_cap;
  p.words = words;
  p.scale_log2 = 1.4426950408889634f / sqrtf((float)g.D);
  p.tau = tau;
  hipError_t err;
  if (!in_header) {
    err = launch_fill_u32(st, p.cand_count, (size_t)g.B * g.Hq + (size_t)g.B * words, 0u);
    if (err != hipSuccess) return err;
  }
  if (g.dtype == FDL_F32) {
    dim3 grid(g.Hq, g.B);
    const float* qq = static_cast<const float*>(q);
    const float* kk = static_cast<const float*>(k);
    const float* kd = static_cast<const float*>(k_dec);
    if (g.D == 128)
      hipLaunchKernelGGL((sink_f32_kernel<128>), grid, dim3(64), 0, st, qq, kk, kd, pred_mask,
                         p.bitmap, g.Hq, g.Hkv, g.G, g.T, g.L, words, tau, g.lens);
    else
      hipLaunchKernelGGL((sink_f32_kernel<64>), grid, dim3(64), 0, st, qq, kk, kd, pred_mask,
                         p.bitmap, g.Hq, g.Hkv, g.G, g.T, g.L, words, tau, g.lens);
  } else if (g.L > 0) {
    // the splits of slot k run on XCD k % 8 (see the kernel)
    dim3 grid(8 * ((p.n_segs + 7) / 8) * n_splits);
    if (stamps != nullptr && stamp_words >= (int64_t)grid.x * 16) p.stamps = stamps;
    if (g.D == 128) {
      if (g.G > 1) hipLaunchKernelGGL((sink_scan_kernel<128, true>), grid, dim3(kSinkWaves * 64), 0, st, p);
      else hipLaunchKernelGGL((sink_scan_kernel<128, false>), grid, dim3(kSinkWaves * 64), 0, st, p);
    } else {
      if (g.G > 1) hipLaunchKernelGGL((sink_scan_kernel<64, true>), grid, dim3(kSinkWaves * 64), 0, st, p);
      else hipLaunchKernelGGL((sink_scan_kernel<64, false>), grid, dim3(kSinkWaves * 64), 0, st, p);
    }
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  // keep_bitmap: the next launch reads the bitmap itself (sink_bitmap_for) and compacts it
  if (keep_bitmap && scan_runs && in_header) return hipSuccess;
  hipLaunchKernelGGL(sink_compact_kernel, dim3(g.B), dim3(256), 0, st, p.bitmap, words, max_sinks,
                     sink_pos, n_sinks, p.cand_count, g.Hq, status);
  return hipGetLastError();
}

}  // namespace fdl
