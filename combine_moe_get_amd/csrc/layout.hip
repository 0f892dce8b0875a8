// layout.hip -- routing layout: counts, offsets, is_token_in_rank, dst_row,
// src_info for a simulated expert-parallel world (one GPU, P ranks).
//
// Rows of expert e are ordered by (source rank, token, slot) (CANN
// "low_latency_dispatch", Deterministic Computation, read as a stable order);
// rank r owns experts [rL, rL + L) (DeepEP issue "#84 Questions on Profiling
// dispatch_t ...", the masking snippet).  Two launches:
//
//  1. count (one workgroup per source rank's chunk of BS tokens, or per
//     sub-chunk of at most 128 tokens where a larger chunk is split, see
//     layout_subchunks): the sub-chunk's ids are staged in LDS once; a
//     slot-parallel pass (one lane per slot) finds owners, specials and bad
//     ids; per-wave histograms in LDS are built with a "match" of the 64 slots
//     of a wave by expert id (ballots over the id bits, or for large chunks
//     per-wave LDS tables of lane masks), so a wave ranks 64 slots in order; a
//     scan over the waves turns them into sub-chunk-local stable ranks (kept in
//     dst_row), the sub-chunk's per-expert counts (a row of the workspace count
//     matrix; recv_counts[:, s] directly when the chunk is not split),
//     is_token_in_rank rows and per-sub-chunk rank / special counts.
//  2. scan + finalize (one workgroup per source rank): each reduces the
//     [P m][E] count matrix (m sub-chunks per chunk) with all loads in flight
//     at once, scans the expert totals into offsets and writes dst_row = first
//     row of (s, e) + the counts of the chunk's earlier sub-chunks + local rank
//     and src_info for its chunk (and recv_counts[:, s] when the chunk is
//     split); workgroup s also writes num_tokens_per_rank[s] and the totals of
//     special ids s, s + P, ... (their inputs loaded at the start), workgroup 0
//     the per-expert outputs.
//
// Small worlds (T * K <= 8192 slots) take one launch instead
// (layout_fused_kernel, below), optionally followed in the same kernel by the
// dispatch.
//
// All outputs are fully rewritten on every call; the only atomics are LDS
// integer adds, LDS ORs of lane masks (the match tables) and an OR into the
// sticky status word, none of which decides an order, so results are
// deterministic.
#include "dispatch_dev.hpp"

namespace moe {

int layout_waves(int E) { return E <= 1024 ? 16 : 8; }

// the single-launch layout re-reads every token's ids in each of the P workgroups; that pass is
// latency-bound, so it only pays while it is short (one launch saved).  With an int8 dispatch in
// the same kernel the bound is lower: per layer (layout + dispatch + combine, T=256..1024, H=7168,
// top-8, dynamic codes) the single kernel measured 18.4 against 19.0 us at 2048 slots, but 28.3
// against 27.4 at 4096 and 49.1 against 46.0-46.4 at 8192 (P = 4..32); with bf16 rows it stays
// ahead up to 8192 slots (29.8 against 32.2, 54.3 against 57.2 us at H=7168; 20.8 against 23.2,
// 34.4 against 37.8 at H=4096 with special experts).
static constexpr int64_t kFusedMaxSlots = 8192;  // measured: faster below ~10K slots, slower above
static constexpr int64_t kFusedInt8MaxSlots = 2048;  // the single kernel with an int8 dispatch
static constexpr size_t kMaxLds = 160 * 1024;  // gfx950 LDS per workgroup
static constexpr int kSpecPerBlock = 8;        // special-id totals one scan workgroup sums from its prefetch
static constexpr int kReadAheadWorkgroups = 128;  // per layout kernel, see launch_layout_dispatch

size_t layout_lds_bytes(int waves, int Epad, int Spad, int P, int NS, int BS, int mt) {
  return (size_t)waves * mt * 8 + (size_t)Spad * 4 + (size_t)waves * Epad * 2 + (size_t)Spad * 2 +
         (size_t)P * 4 + (size_t)NS * 4 + (size_t)BS;
}

__device__ __forceinline__ void zero_bytes(uint8_t *p, size_t n, int tid, int nthr) {
  const uintptr_t a = (uintptr_t)p;
  size_t head = (16 - (a & 15)) & 15;
  if (head > n) head = n;
  for (size_t i = tid; i < head; i += nthr) p[i] = 0;
  u32x4 *mid = (u32x4 *)(p + head);
  const size_t nmid = (n - head) >> 4;
  for (size_t i = tid; i < nmid; i += nthr) mid[i] = u32x4{0u, 0u, 0u, 0u};
  for (size_t i = head + (nmid << 4) + tid; i < n; i += nthr) p[i] = 0;
}

// Slot-parallel passes over tokens: the lanes of a wave take floor(64 / K) whole
// tokens, one slot each (lane = g * K + j: token g of the pass, slot j).
struct SlotLanes {
  int g, j, per;
  bool on;         // the lane holds a slot
  uint64_t group;  // the lanes of the same token
  __device__ SlotLanes(int K, uint32_t divK, int lane) {
    per = fast_div(64, divK);
    g = fast_div(lane, divK);
    j = lane - g * K;
    on = g < per;
    group = on ? (((1ull << K) - 1) << (g * K)) : 0ull;  // K <= 16
  }
};

// lanes whose key equals the calling lane's (keys < 2^nbits): a lane differs from the calling
// lane wherever the ballot of a key bit differs from the calling lane's own bit (all ones or
// all zeros), so the mismatches are ORed up per 32-bit half and complemented at the end.
// Every lane of the wave must call it.
__device__ __forceinline__ uint64_t match_key(int key, int nbits) {
  uint32_t mis_lo = 0u, mis_hi = 0u;
  for (int b = 0; b < nbits; ++b) {
    const uint32_t own = (uint32_t)(__builtin_amdgcn_sbfe(key, b, 1));  // all ones where the lane's bit is set
    const uint64_t bl = ballot(own != 0u);
    mis_lo |= (uint32_t)bl ^ own;
    mis_hi |= (uint32_t)(bl >> 32) ^ own;
  }
  return ~(((uint64_t)mis_hi << 32) | mis_lo);
}

// own >= 0 is the owner rank of the lane's slot: true for the first slot of its token
// with that owner (so each (token, rank) pair counts once).  Every lane must call it.
__device__ __forceinline__ bool first_of_owner(const SlotLanes &sl, int own, int nbits_p, int lane) {
  const uint64_t peers = match_key(own + 1, nbits_p) & sl.group;
  return own >= 0 && (peers & ((1ull << lane) - 1ull)) == 0ull;
}

// the DS instructions of one wave execute in issue order; this only keeps the compiler
// from moving LDS accesses across it (no s_barrier, no wait on other waves)
__device__ __forceinline__ void wave_lds_order() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// match_key through a per-wave table of 64-bit lane masks in LDS (tab[key], zero between
// calls; key < table size): each lane that takes part ORs its bit into its key's word,
// reads the word back, and clears it -- three LDS instructions in place of one ballot
// and its VALU work per key bit.  Lanes not taking part get 0.  Every lane must call it.
__device__ __forceinline__ uint64_t match_key_lds(uint64_t *tab, int key, bool on, int lane) {
  if (on) __hip_atomic_fetch_or(tab + key, 1ull << lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
  wave_lds_order();
  uint64_t peers = 0ull;
  if (on) peers = *(volatile uint64_t *)(tab + key);
  wave_lds_order();
  if (on) *(volatile uint64_t *)(tab + key) = 0ull;
  return peers;
}

// first_of_owner with the wave's LDS match table (at least P words)
__device__ __forceinline__ bool first_of_owner_lds(const SlotLanes &sl, int own, int lane, uint64_t *tab) {
  const uint64_t peers = match_key_lds(tab, own, own >= 0, lane) & sl.group;
  return own >= 0 && (peers & ((1ull << lane) - 1ull)) == 0ull;
}

// Exclusive scan over the W per-wave counters of each expert (cnt[w][e], u16), all loads
// issued before the first store; returns the expert's chunk total.
template <int W>
__device__ __forceinline__ int scan_wave_counts(uint16_t *cnt, int Epad, int e) {
  int c[W];
#pragma unroll
  for (int w = 0; w < W; ++w) c[w] = cnt[w * Epad + e];
  int run = 0;
#pragma unroll
  for (int w = 0; w < W; ++w) {
    cnt[w * Epad + e] = (uint16_t)run;
    run += c[w];
  }
  return run;
}

// BIG (sub-chunks of more than W * 64 slots, so every wave ranks several 64-slot groups):
// the id loads are all issued before the first LDS store, and slots are matched through LDS
// tables (a.mt words per wave) instead of ballots.  Measured on gfx950 (whole layout, chunks
// not yet split): 4096 slots per chunk 18.4 -> 16.3 us, 2048 slots 16.3 -> 15.7 us; at 1024
// slots the ballot version is as fast or faster.
//
// Workgroup v counts sub-chunk v = s m + q: tokens [q BSv, q BSv + nt) of source rank s's
// chunk (m = 1 and BSv = BS unless chunks of more than 128 tokens are split, so that more
// workgroups share the latency-bound passes); ranks are local to the sub-chunk and its
// counts go to row v of the workspace matrices, which the scan kernel combines.
template <int W, bool BIG, bool SUBS>
__global__ void __launch_bounds__(W * 64) layout_count_kernel(LayoutArgs a) {
  extern __shared__ __align__(16) unsigned char lds[];
  if ((int)blockIdx.x >= a.P * a.m) {  // a read-ahead workgroup (whole workgroup: no barrier skipped)
    read_ahead(a.pf, 0, a.pf_half, (int)blockIdx.x - a.P * a.m, a.pf_wgs);
    return;
  }
  const int vs = blockIdx.x;  // sub-chunk index s m + q
  const int s = SUBS ? vs / a.m : vs, q = vs - s * a.m;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int K = a.K, E = a.E, P = a.P, NS = a.NS;
  const int tq = q * a.BSv;                   // first token of the sub-chunk inside the chunk
  const int nt = min(a.BS, tq + a.BSv) - tq;  // its tokens (at least one)
  const int S = nt * K;
  const int t0 = s * a.BS + tq;
  const size_t slot0 = (size_t)t0 * K;

  const int mt = BIG ? a.mt : 0;
  uint64_t *mtab = (uint64_t *)lds + (size_t)wv * mt;  // [W][mt] match tables (BIG)
  int *ids = (int *)(lds + (size_t)W * mt * 8);        // [Svpad] the sub-chunk's expert ids
  uint16_t *cnt = (uint16_t *)(ids + a.Svpad);  // [W][Epad] per-wave running counts
  uint16_t *rk = cnt + W * a.Epad;              // [Svpad] rank of a slot inside its wave segment
  int *rank_tok = (int *)(rk + a.Svpad);        // [P]
  int *spec = rank_tok + P;                     // [NS]

  // one coalesced pass over the chunk's ids and mask; everything after reads LDS.  A slot of
  // an inactive token is stored as -1 (dropped), so no later pass looks at the mask.
  if constexpr (BIG) {  // every load issued before the first LDS store (S <= 512 * 16)
    constexpr int PER = 8192 / (W * 64);
    int v[PER];
    uint8_t on[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int i = tid + u * W * 64;
      v[u] = i < S ? a.topk_idx[slot0 + i] : 0;
      on[u] = (i < S && a.mask) ? a.mask[t0 + fast_div(i, a.divK)] : (uint8_t)1;
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int i = tid + u * W * 64;
      if (i < S) ids[i] = on[u] ? v[u] : -1;
    }
    for (int i = tid; i < W * mt; i += W * 64) ((uint64_t *)lds)[i] = 0ull;
  } else {
    for (int i = tid; i < S; i += W * 64) {
      const int v = a.topk_idx[slot0 + i];
      ids[i] = (!a.mask || a.mask[t0 + fast_div(i, a.divK)]) ? v : -1;
    }
  }
  for (int i = tid; i < W * a.Epad / 2; i += W * 64) ((uint32_t *)cnt)[i] = 0u;
  for (int i = tid; i < P; i += W * 64) rank_tok[i] = 0;
  for (int i = tid; i < NS; i += W * 64) spec[i] = 0;
  zero_bytes(a.itr + (size_t)t0 * P, (size_t)nt * P, tid, W * 64);
  __syncthreads();

  // ---- token phase (slot-parallel): owner ranks, specials, bad ids ---------
  bool bad = false;
  {
    const SlotLanes sl(K, a.divK, lane);
    const int nbp = 32 - __builtin_clz((unsigned)P);
    for (int tb = wv * sl.per; tb < nt; tb += W * sl.per) {  // uniform per wave
      const int tl = tb + sl.g;
      // the slot's class without nested branches: -1 (dropped), a bad id, a special id (one
      // predicated LDS add) or a routed id (its owner rank)
      const bool on = sl.on && tl < nt;
      const int id = on ? ids[on ? tl * K + sl.j : 0] : -1;
      const unsigned uid = (unsigned)id;
      bad = bad || (id != -1 && uid >= (unsigned)a.Etot);
      if (uid - (unsigned)E < (unsigned)NS) atomicAdd(&spec[id - E], 1);
      const int own = uid < (unsigned)E ? fast_div(id, a.divL) : -1;
      if (BIG ? first_of_owner_lds(sl, own, lane, mtab) : first_of_owner(sl, own, nbp, lane)) {
        a.itr[(size_t)(t0 + tl) * P + own] = 1;
        atomicAdd(&rank_tok[own], 1);
      }
    }
  }

  // ---- ranking phase: wave wv owns slots [beg, end) of the sub-chunk --------
  const int seg = (((S + W - 1) / W) + 63) & ~63;
  const int beg = wv * seg;
  const int end = min(S, beg + seg);
  uint16_t *mycnt = cnt + wv * a.Epad;
  for (int base = beg; base < end; base += 64) {  // uniform per wave
    const int i = base + lane;
    int key = E;  // sentinel: not a routed slot
    if (i < end) {
      const int id = ids[i];
      if (id >= 0 && id < E) key = id;
    }
    // lanes holding the same key
    const uint64_t peers = BIG ? match_key_lds(mtab, key, key < E, lane) : match_key(key, a.nbits);
    if (key < E) {
      const int r = (int)mycnt[key] + popc_below(peers);
      rk[i] = (uint16_t)r;
      if (((peers >> lane) >> 1) == 0ull) mycnt[key] = (uint16_t)(r + 1);  // last lane of the group
    }
  }
  __syncthreads();

  // ---- exclusive scan over the waves, per expert ----------------------------
  for (int e = tid; e < E; e += W * 64) {
    const int run = scan_wave_counts<W>(cnt, a.Epad, e);
    if constexpr (!SUBS) a.recv_counts[(size_t)e * P + s] = run;  // split chunks: the scan kernel sums
    a.ws_cnt_t[(size_t)vs * E + e] = run;
  }
  __syncthreads();

  // ---- sub-chunk-local stable rank of every slot (made global by the next kernel) ---
  for (int base = beg; base < end; base += 64) {
    const int i = base + lane;
    if (i < end) {
      const int id = ids[i];
      int r = -1;
      if (id >= 0 && id < E) r = (int)mycnt[id] + (int)rk[i];
      a.dst_row[slot0 + i] = r;
    }
  }
  for (int r = tid; r < P; r += W * 64) a.ws_rank_tok[(size_t)vs * P + r] = rank_tok[r];
  for (int z = tid; z < NS; z += W * 64) a.ws_special[(size_t)vs * NS + z] = spec[z];
  if (bad) atomicOr(a.status, (uint32_t)MOE_DEV_STATUS_BAD_EXPERT_ID);
}

// Sum of column `col` of a row-major [rows][ld] int matrix over rows r = r0, r0+step, ...,
// with the part over rows < lim returned separately.  Loads are issued in groups of 8 so the
// latency is paid once per group, not once per row.
__device__ __forceinline__ void column_sums(const int32_t *m, int ld, int col, int rows, int r0,
                                            int step, int lim, int &tot, int &below) {
  int r = r0;
  for (; r + 7 * step < rows; r += 8 * step) {
    int v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = m[(size_t)(r + u * step) * ld + col];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      tot += v[u];
      below += (r + u * step < lim) ? v[u] : 0;
    }
  }
  for (; r < rows; r += step) {
    const int v = m[(size_t)r * ld + col];
    tot += v;
    below += r < lim ? v : 0;
  }
}

// One workgroup of 1024 threads per source rank s.  Every workgroup reduces the [P m][E]
// count matrix (expert totals and the part sent by ranks below s), scans the totals into
// expert offsets, and turns its own chunk's sub-chunk ranks into rows (adding the counts
// of the chunk's earlier sub-chunks); workgroup 0 also writes the per-expert and per-rank
// outputs.  E <= 2048, m <= 4 and m E <= 4096.
// SPT: slots per thread loaded at the start (ceil(S / 1024) <= SPT, S <= 8192); with SPT = 1
// the slots past the first 1024 are loaded in the last loop.
template <int SPT, bool SUBS>
__global__ void __launch_bounds__(1024) layout_scan_finalize_kernel(LayoutArgs a) {
  __shared__ int red[2 * 2048];  // partial column sums; later the sub-chunk bases
  int *red_tot = red, *red_pre = red + 2048;
  int *subb = red;               // [m - 1][E]: first row of (sub-chunk q >= 1, e) past the chunk's
  __shared__ int totl[2048];
  __shared__ int basel[2048];
  __shared__ int liml[2048];
  __shared__ int offl[2049];
  __shared__ int wsum[16];
  __shared__ int acc_rt;             // distinct tokens on rank s, summed over the source chunks
  __shared__ int acc_sp[kSpecPerBlock];  // special ids s, s + P, ... summed over the source chunks
  if ((int)blockIdx.x >= a.P) {  // a read-ahead workgroup (whole workgroup: no barrier skipped)
    read_ahead(a.pf, a.pf_half, a.pf_bytes, (int)blockIdx.x - a.P, a.pf_wgs);
    return;
  }
  const int s = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int E = a.E, P = a.P, NS = a.NS, K = a.K;
  const int m = SUBS ? a.m : 1, Pv = P * m;  // sub-chunks per chunk; rows of the workspace matrices
  const int S = a.BS * K;
  const size_t slot0 = (size_t)s * S;
  // loads issued now so their latency overlaps the reduction below: the thread's first SPT
  // slots of the chunk (sub-chunk rank and id); the counts of this chunk's sub-chunks for
  // experts tid and tid + 1024; an element of column s of the per-sub-chunk rank-token
  // counts; an element of the per-sub-chunk special counts of the ids this workgroup
  // totals (s + k P, k < kSpecPerBlock, as element (i, k) = (e2 % Pv, e2 / Pv))
  int sub[2][4];  // m <= 4
  if constexpr (SUBS) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq)
        sub[h][qq] = (qq < m && tid + 1024 * h < E) ? a.ws_cnt_t[(size_t)(s * m + qq) * E + tid + 1024 * h] : 0;
  }
  int pre_v[SPT], pre_e[SPT];
#pragma unroll
  for (int u = 0; u < SPT; ++u) {
    const int i = tid + u * 1024;
    pre_v[u] = -1;
    pre_e[u] = 0;
    if (i < S) {
      pre_v[u] = a.dst_row[slot0 + i];
      pre_e[u] = a.topk_idx[slot0 + i];
    }
  }
  const int pre_rt = tid < Pv ? a.ws_rank_tok[(size_t)tid * P + s] : 0;
  const int nsp = s < NS ? min(kSpecPerBlock, (NS - s + P - 1) / P) : 0;  // special ids of this workgroup
  int pre_sp = 0;
  if (tid < Pv * nsp) pre_sp = a.ws_special[(size_t)(tid % Pv) * NS + s + (tid / Pv) * P];
  if (tid == 0) acc_rt = 0;
  if (tid < kSpecPerBlock) acc_sp[tid] = 0;

  // partial column sums: virtual thread (e, g) sums rows g, g+G, ... of the count matrix (the
  // 64 lanes of a wave read 64 neighbouring columns of one row: coalesced)
  const int G = E >= 1024 ? 1 : 1024 / E;  // row groups per expert column
  for (int v = tid; v < E * G; v += 1024) {
    const int g = fast_div(v, a.divE), e = v - g * E;
    int tot = 0, below = 0;
    column_sums(a.ws_cnt_t, E, e, Pv, g, G, s * m, tot, below);
    red_tot[v] = tot;
    red_pre[v] = below;
  }
  __syncthreads();

  // expert totals (tot) and the copies sent by the sub-chunks before this chunk (below): thread
  // t owns expert t (E <= 1024) or experts 2t and 2t + 1 (E > 1024, one row group); then the
  // exclusive scan of the totals, a wave scan now and the wave totals after the next barrier
  const bool pairs = E > 1024;
  const int eg = pairs ? 2 * tid : tid;
  int tot0 = 0, bel0 = 0, tot1 = 0, bel1 = 0;
  if (eg < E) {
    for (int g = 0; g < G; ++g) {
      tot0 += red_tot[g * E + eg];
      bel0 += red_pre[g * E + eg];
    }
  }
  if (pairs && eg + 1 < E) {
    tot1 = red_tot[eg + 1];
    bel1 = red_pre[eg + 1];
  }
  const int local = tot0 + tot1;
  const int incl = wave_inclusive_sum(local);
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  // distinct tokens on rank s: a DPP sum over the wave, then one LDS add per wave (an atomic
  // add of a per-lane value to one address compiles to a scalar loop over the active lanes:
  // ~1 us for 32 lanes on gfx950, on the critical path of workgroup wave 0)
  if (wv * 64 < Pv) {
    const int wsum_rt = wave_inclusive_sum(pre_rt);  // lane 63: the wave's total
    if (lane == 63 && wsum_rt) atomicAdd(&acc_rt, wsum_rt);
  }
  if (pre_sp) atomicAdd(&acc_sp[tid / Pv], pre_sp);
  // columns longer than the workgroup (Pv > 1024) and further special ids (rare)
  for (int i = tid + 1024; i < Pv; i += 1024) atomicAdd(&acc_rt, a.ws_rank_tok[(size_t)i * P + s]);
  for (int e2 = tid + 1024; e2 < Pv * nsp; e2 += 1024)
    atomicAdd(&acc_sp[e2 / Pv], a.ws_special[(size_t)(e2 % Pv) * NS + s + (e2 / Pv) * P]);
  // recv_counts column s, and the first row of each later sub-chunk relative to the chunk's
  // (subb aliases red, whose last reads were before the barrier above)
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int e = tid + 1024 * h;
    if (SUBS && e < E) {
      int run = sub[h][0];
#pragma unroll
      for (int qq = 1; qq < 4; ++qq) {
        if (qq < m) {
          subb[(qq - 1) * E + e] = run;
          run += sub[h][qq];
        }
      }
      a.recv_counts[(size_t)e * P + s] = run;
    }
  }
  // the exclusive prefix of the wave totals: every wave sums the totals of the waves before it
  const int wpre = readlane(wave_inclusive_sum(lane < wv ? wsum[lane] : 0), 63);
  if (eg < E) {
    const int excl = incl - local + wpre;
    totl[eg] = tot0;
    offl[eg] = excl;
    basel[eg] = bel0 + excl;
    liml[eg] = INT32_MAX;
    if (eg == E - 1) offl[E] = excl + tot0;  // N
    if (pairs && eg + 1 < E) {
      totl[eg + 1] = tot1;
      offl[eg + 1] = excl + tot0;
      basel[eg + 1] = bel1 + excl + tot0;
      liml[eg + 1] = INT32_MAX;
      if (eg + 1 == E - 1) offl[E] = excl + tot0 + tot1;
    }
  }
  __syncthreads();
  if (a.rank_stride > 0) {  // move the owner's rows into its window [r A, r A + A) (uniform branch)
    for (int e = tid; e < E; e += 1024) {
      const int r = fast_div(e, a.divL);
      const int64_t w0 = (int64_t)r * a.rank_stride;
      basel[e] = (int)(w0 + basel[e] - offl[r * a.L]);
      liml[e] = (int)(w0 + a.rank_stride);
    }
    __syncthreads();
  }

  // rows of this chunk's slots
  bool overflow = false;
  auto finalize_slot = [&](int i, int v, int e) {  // v: the slot's rank in its sub-chunk, or < 0
    if (v < 0) return;
    const int qq = SUBS ? fast_div(fast_div(i, a.divK), a.divBSv) : 0;
    const int row = basel[e] + (qq > 0 ? subb[(qq - 1) * E + e] : 0) + v;
    if (row >= liml[e]) {  // only a token repeating an expert id can overflow its window
      overflow = true;
      a.dst_row[slot0 + i] = -1;
      return;
    }
    a.dst_row[slot0 + i] = row;
    a.src_info[row] = (int)(slot0 + i);
  };
#pragma unroll
  for (int u = 0; u < SPT; ++u)
    if (tid + u * 1024 < S) finalize_slot(tid + u * 1024, pre_v[u], pre_e[u]);
  for (int i = tid + SPT * 1024; i < S; i += 1024) finalize_slot(i, a.dst_row[slot0 + i], a.topk_idx[slot0 + i]);
  if (overflow) atomicOr(a.status, (uint32_t)MOE_DEV_STATUS_RANK_OVERFLOW);

  // per-rank and special totals (accumulated after the first barrier; several barriers since)
  if (tid == 0) a.num_tokens_per_rank[s] = acc_rt;
  if (tid < nsp) a.special_counts[s + tid * P] = acc_sp[tid];
  // special ids beyond what P workgroups of kSpecPerBlock cover (NS > P kSpecPerBlock): summed here
  for (int z = s + kSpecPerBlock * P + tid * P; z < NS; z += 1024 * P) {
    int tot = 0, below = 0;
    column_sums(a.ws_special, NS, z, Pv, 0, 1, 0, tot, below);
    a.special_counts[z] = tot;
  }

  if (s != 0) return;
  for (int e = tid; e < E; e += 1024) {
    a.cnt[e] = totl[e];
    a.expert_offsets[e] = offl[e];
  }
  if (tid == 0) a.expert_offsets[E] = offl[E];
  for (int r = tid; r <= P; r += 1024) a.rank_offsets[r] = offl[r * a.L];
}


// ---- single-launch layout ---------------------------------------------------
// Workgroup (s, m) owns tokens [m tpw, m tpw + nt) of source rank s's chunk (a
// sub-chunk), with no communication between workgroups: each first histograms
// the ids of ALL tokens (slot-parallel, LDS integer atomics -- counts do not
// depend on order) into three bins: tokens before its sub-chunk (hist_lo), the
// rest of chunk s from the sub-chunk on (hist_mid) and the tokens after chunk s
// (hist_hi).  Expert totals are lo + mid + hi and the first row of the sub-chunk
// in expert e is offset[e] + hist_lo[e]; the sub-chunk's own slots are then ranked
// in order with the ballot match and written as final rows.  Workgroup (s, 0)
// also writes recv_counts[:, s] (its hist_mid is chunk s), workgroup (0, 0) the
// per-expert / per-rank outputs (it saw every token).  Used while the redundant
// pass stays small (T * K bounded); larger worlds take the two-launch path.
//
// With DM >= 0 the same kernel also dispatches (layout + dispatch in one launch,
// as the CANN dispatch op returns both): each workgroup quantizes / copies its own
// tokens with the rows it holds in LDS (dispatch_token_block; DM = quant mode, PE =
// per-expert scales).
// SUB: the chunk is split (M > 1 workgroups per chunk); otherwise two bins suffice (hist_hi
// then holds chunk s too) and recv_counts comes from the chunk's own ranking.
template <int W, int DM, bool PE, bool SUB>
__global__ void __launch_bounds__(W * 64) layout_fused_kernel(LayoutArgs a, DispatchArgs d, int tpw) {
  extern __shared__ __align__(16) unsigned char lds[];
  __shared__ int wsum[16];
  __shared__ float red[2][16];
  constexpr int NT = W * 64;
  const int s = blockIdx.x;
  const bool writer = blockIdx.y == 0;  // writes recv_counts[:, s]
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int T = a.T, K = a.K, E = a.E, P = a.P, BS = a.BS, NS = a.NS;
  const int Etot = E + NS;
  const int Ep2 = (Etot + 1) & ~1;
  const int tq = (int)blockIdx.y * tpw;          // first token of the sub-chunk inside the chunk
  const int nt = max(0, min(BS, tq + tpw) - tq);  // its tokens
  const int S = nt * K;
  const int Sp = tpw * K + ((tpw * K) & 1);
  const int cend = (s + 1) * BS;                 // end of chunk s
  const int u0 = s * BS + tq;                    // first token of the sub-chunk
  const size_t slot0 = (size_t)u0 * K;

  int *hist_lo = (int *)lds;                     // [Ep2] ids of tokens before the sub-chunk
  int *hist_mid = hist_lo + Ep2;                 // [Ep2] ids of the sub-chunk and the rest of chunk s
  int *hist_hi = hist_mid + Ep2;                 // [Ep2] ids of tokens after chunk s
  int *rtok = hist_hi + Ep2;                     // [P]  distinct tokens per rank (block 0)
  int *offl = rtok + P;                          // [E + 1]
  int *basel = offl + E + 1;                     // [E]
  int *liml = basel + E;                         // [E]
  int *ids = liml + E;                           // [Sp]
  uint16_t *cnt = (uint16_t *)(ids + Sp);        // [W][Epad]
  uint16_t *rk = cnt + W * a.Epad;               // [Sp]
  int *rows = (int *)(rk + Sp);                  // [Sp] final rows (DM >= 0 only)

  // loads issued before the first barrier, so their latency overlaps the set-up below:
  // this lane's slot of the first pass over all tokens, and the first token this
  // workgroup dispatches
  const SlotLanes sl(K, a.divK, lane);
  int pre_id = -1;
  bool pre_on = false;
  {
    const int t = wv * sl.per + sl.g;
    if (sl.on && t < T) {
      pre_id = a.topk_idx[(size_t)t * K + sl.j];
      pre_on = !a.mask || a.mask[t];
    }
  }
  TokenPrefetch pf;
  if constexpr (DM >= 0) {
    if (nt > 0) dispatch_prefetch<DM, PE>(d, u0, pf);
  }

  for (int i = tid; i < 3 * Ep2; i += NT) hist_lo[i] = 0;  // (hist_mid stays 0 without SUB)
  for (int i = tid; i < P; i += NT) rtok[i] = 0;
  for (int i = tid; i < W * a.Epad / 2; i += NT) ((uint32_t *)cnt)[i] = 0u;
  for (int i = tid; i < S; i += NT) {  // a slot of an inactive token is stored as -1 (dropped)
    const int v = a.topk_idx[slot0 + i];
    ids[i] = (!a.mask || a.mask[u0 + fast_div(i, a.divK)]) ? v : -1;
  }
  zero_bytes(a.itr + (size_t)u0 * P, (size_t)nt * P, tid, NT);
  __syncthreads();
  const bool first = writer && s == 0;  // the workgroup that writes the per-expert / per-rank outputs

  // ---- every token's ids (slot-parallel): totals, counts before the sub-chunk, chunk s's
  //      counts, distinct tokens per rank (first workgroup) --------------------------------
  bool bad = false;
  {
    const int nbp = 32 - __builtin_clz((unsigned)P);
    int it = 0;
    for (int tb = wv * sl.per; tb < T; tb += W * sl.per, ++it) {  // uniform per wave
      const int t = tb + sl.g;
      int id = pre_id;
      bool on = pre_on;
      if (it > 0) {
        id = -1;
        on = false;
        if (sl.on && t < T) {
          id = a.topk_idx[(size_t)t * K + sl.j];
          on = !a.mask || a.mask[t];
        }
      }
      // the slot's class without nested branches (see the count kernel)
      const unsigned uid = on ? (unsigned)id : 0xffffffffu;
      bad = bad || (on && id != -1 && uid >= (unsigned)Etot);
      if (uid < (unsigned)Etot) atomicAdd(&(t < u0 ? hist_lo : (SUB && t < cend) ? hist_mid : hist_hi)[id], 1);
      const int own = uid < (unsigned)E ? fast_div(id, a.divL) : -1;
      if (first) {  // uniform per workgroup
        if (first_of_owner(sl, own, nbp, lane)) atomicAdd(&rtok[own], 1);
      }
    }
  }

  // ---- this sub-chunk: is_token_in_rank rows --------------------------------------
  for (int i = tid; i < S; i += NT) {
    const int id = ids[i];
    if (id >= 0 && id < E) a.itr[(size_t)u0 * P + (size_t)fast_div(i, a.divK) * P + fast_div(id, a.divL)] = 1;
  }

  // ---- this sub-chunk: stable ranks inside each wave segment (ballot match) -------
  const int seg = (((S + W - 1) / W) + 63) & ~63;
  const int beg = wv * seg;
  const int end = min(S, beg + seg);
  uint16_t *mycnt = cnt + wv * a.Epad;
  for (int base = beg; base < end; base += 64) {
    const int i = base + lane;
    int key = E;
    if (i < end) {
      const int id = ids[i];
      if (id >= 0 && id < E) key = id;
    }
    const uint64_t peers = match_key(key, a.nbits);
    if (key < E) {
      const int r = (int)mycnt[key] + popc_below(peers);
      rk[i] = (uint16_t)r;
      if (((peers >> lane) >> 1) == 0ull) mycnt[key] = (uint16_t)(r + 1);
    }
  }
  __syncthreads();

  // ---- per expert: scan over the waves (sub-chunk-local bases); recv_counts column ---
  for (int e = tid; e < E; e += NT) {
    const int run = scan_wave_counts<W>(cnt, a.Epad, e);
    if (writer) a.recv_counts[(size_t)e * P + s] = SUB ? hist_mid[e] : run;
  }

  // ---- expert offsets: exclusive scan of the totals (thread t owns experts 4t ... 4t + 3) ---
  {
    constexpr int PER = 4;  // E <= 2048 with W >= 8: at most 4 experts per thread
    int v[PER], local = 0;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = tid * PER + u;
      v[u] = e < E ? hist_lo[e] + (SUB ? hist_mid[e] : 0) + hist_hi[e] : 0;
      local += v[u];
    }
    const int incl = wave_inclusive_sum(local);
    if (lane == 63) wsum[wv] = incl;
    __syncthreads();
    // the exclusive prefix of the wave totals: every wave sums the totals of the waves before it
    const int wpre = readlane(wave_inclusive_sum(lane < wv ? wsum[lane] : 0), 63);
    int run = incl - local + wpre;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = tid * PER + u;
      if (e < E) {
        offl[e] = run;
        basel[e] = run + hist_lo[e];
        liml[e] = INT32_MAX;
      }
      run += v[u];
      if (e == E - 1) offl[E] = run;
    }
  }
  __syncthreads();
  if (a.rank_stride > 0) {  // rank r's rows go to its window [r A, r A + A) (uniform branch)
    for (int e = tid; e < E; e += NT) {
      const int r = fast_div(e, a.divL);
      const int64_t w0 = (int64_t)r * a.rank_stride;
      basel[e] = (int)(w0 + basel[e] - offl[r * a.L]);
      liml[e] = (int)(w0 + a.rank_stride);
    }
    __syncthreads();
  }

  // ---- rows of this sub-chunk -----------------------------------------------------
  bool overflow = false;
  for (int base = beg; base < end; base += 64) {
    const int i = base + lane;
    if (i >= end) continue;
    const int id = ids[i];
    int row = -1;
    if (id >= 0 && id < E) {
      row = basel[id] + (int)mycnt[id] + (int)rk[i];
      if (row >= liml[id]) {  // only a token repeating an expert id can overflow its window
        overflow = true;
        row = -1;
      } else {
        a.src_info[row] = (int)(slot0 + i);
      }
    }
    a.dst_row[slot0 + i] = row;
    if constexpr (DM >= 0) rows[i] = row;
  }
  if (overflow) atomicOr(a.status, (uint32_t)MOE_DEV_STATUS_RANK_OVERFLOW);

  if (first) {
    if (bad) atomicOr(a.status, (uint32_t)MOE_DEV_STATUS_BAD_EXPERT_ID);
    for (int e = tid; e < E; e += NT) {
      a.cnt[e] = offl[e + 1] - offl[e];
      a.expert_offsets[e] = offl[e];
    }
    if (tid == 0) a.expert_offsets[E] = offl[E];
    for (int r = tid; r <= P; r += NT) a.rank_offsets[r] = offl[r * a.L];
    for (int r = tid; r < P; r += NT) a.num_tokens_per_rank[r] = rtok[r];
    for (int z = tid; z < NS; z += NT) a.special_counts[z] = hist_lo[E + z] + (SUB ? hist_mid[E + z] : 0) + hist_hi[E + z];
  }

  if constexpr (DM >= 0) {
    // ---- dispatch of this workgroup's tokens ----------------------------------------
    __syncthreads();  // rows[] complete
    int par = 0;
    for (int tl = 0; tl < nt; ++tl)
      dispatch_token_block<DM, PE>(d, u0 + tl, rows + tl * K, ids + tl * K, red, par, pf, tl == 0);
  }
}

// dynamic LDS of layout_fused_kernel for sub-chunks of tpw tokens
size_t layout_fused_lds_bytes(int waves, int E, int NS, int Epad, int K, int P, int tpw, bool rows) {
  const size_t ep2 = (size_t)((E + NS + 1) & ~1);
  const size_t sp = (size_t)tpw * K + (((size_t)tpw * K) & 1);
  return 3 * ep2 * 4 + (size_t)P * 4 + (size_t)(E + 1) * 4 + 2 * (size_t)E * 4 + sp * 4 +
         (size_t)waves * Epad * 2 + sp * 2 + (rows ? sp * 4 : 0) + (size_t)tpw;
}

// tokens per workgroup of the single-launch kernel: layout only, sub-chunks of at most 32
// tokens (more workgroups share the ranking); with the dispatch, about 256 workgroups over the
// world, at least one token each
static int fused_tpw(const LayoutArgs &a, bool dispatch) {
  int tpw = dispatch ? (a.T + 255) / 256 : (a.BS < 32 ? a.BS : 32);
  if (tpw > a.BS) tpw = a.BS;
  return tpw < 1 ? 1 : tpw;
}

// single launch while each workgroup's pass over every token stays small
// (rows: with the dispatch of quant_mode quant in the same kernel)
static bool use_fused(const LayoutArgs &a, bool rows, int quant = 0) {
  const size_t flds = layout_fused_lds_bytes(layout_waves(a.E), a.E, a.NS, a.Epad, a.K, a.P, fused_tpw(a, rows), rows);
  const int64_t max_slots = rows && quant != 0 ? kFusedInt8MaxSlots : kFusedMaxSlots;
  return (int64_t)a.T * a.K <= max_slots && flds <= kMaxLds;
}

int layout_launch_count(const LayoutArgs &a) { return use_fused(a, false) ? 1 : 2; }

int layout_dispatch_launch_count(const LayoutArgs &a, int quant_mode, int64_t x_bytes) {
  if (use_fused(a, true, quant_mode)) return 1;
  if (a.T == 0) return layout_launch_count(a);
  const bool ahead = !use_fused(a, false);  // the two layout kernels read the rows ahead
  return layout_launch_count(a) + dispatch_launch_count(quant_mode, 0, ahead, x_bytes);
}

template <int W, int DM, bool PE>
static hipError_t launch_fused(const LayoutArgs &a, const DispatchArgs &d, hipStream_t stream) {
  const int tpw = fused_tpw(a, DM >= 0);
  const size_t flds = layout_fused_lds_bytes(W, a.E, a.NS, a.Epad, a.K, a.P, tpw, DM >= 0);
  int M = (a.BS + tpw - 1) / tpw;  // sub-chunks per chunk
  if (M < 1) M = 1;
  // gfx950 has 160 KB of LDS per workgroup; more than 64 KB must be asked for
  if (flds > 65536) {
    const hipError_t e = hipFuncSetAttribute(M > 1 ? (const void *)&layout_fused_kernel<W, DM, PE, true>
                                                   : (const void *)&layout_fused_kernel<W, DM, PE, false>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)flds);
    if (e != hipSuccess) return e;
  }
  if (M > 1)
    hipLaunchKernelGGL((layout_fused_kernel<W, DM, PE, true>), dim3((unsigned)a.P, (unsigned)M), dim3(W * 64), flds,
                       stream, a, d, tpw);
  else
    hipLaunchKernelGGL((layout_fused_kernel<W, DM, PE, false>), dim3((unsigned)a.P, 1u), dim3(W * 64), flds, stream,
                       a, d, tpw);
  return hipGetLastError();
}

template <int W>
static hipError_t launch_fused_mode(const LayoutArgs &a, const DispatchArgs &d, int dm, bool pe, hipStream_t st) {
  switch (dm) {
    case -1: return launch_fused<W, -1, false>(a, d, st);
    case 0: return launch_fused<W, 0, false>(a, d, st);
    case 1: return pe ? launch_fused<W, 1, true>(a, d, st) : launch_fused<W, 1, false>(a, d, st);
    default: return pe ? launch_fused<W, 2, true>(a, d, st) : launch_fused<W, 2, false>(a, d, st);
  }
}

template <bool SUBS>
static hipError_t launch_count(const LayoutArgs &b, int W, bool big, dim3 grid, size_t lds, hipStream_t stream) {
  const void *fn = W == 16 ? (big ? (const void *)&layout_count_kernel<16, true, SUBS> : (const void *)&layout_count_kernel<16, false, SUBS>)
                           : (big ? (const void *)&layout_count_kernel<8, true, SUBS> : (const void *)&layout_count_kernel<8, false, SUBS>);
  if (lds > 65536) {  // gfx950 has 160 KB of LDS per workgroup; more than 64 KB must be asked for
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  if (W == 16 && big)
    hipLaunchKernelGGL((layout_count_kernel<16, true, SUBS>), grid, dim3(16 * 64), lds, stream, b);
  else if (W == 16)
    hipLaunchKernelGGL((layout_count_kernel<16, false, SUBS>), grid, dim3(16 * 64), lds, stream, b);
  else if (big)
    hipLaunchKernelGGL((layout_count_kernel<8, true, SUBS>), grid, dim3(8 * 64), lds, stream, b);
  else
    hipLaunchKernelGGL((layout_count_kernel<8, false, SUBS>), grid, dim3(8 * 64), lds, stream, b);
  return hipGetLastError();
}

hipError_t launch_layout(const LayoutArgs &a, hipStream_t stream) {
  const int W = layout_waves(a.E);
  if (use_fused(a, false)) {
    const DispatchArgs none{};
    return W == 16 ? launch_fused_mode<16>(a, none, -1, false, stream) : launch_fused_mode<8>(a, none, -1, false, stream);
  }
  const int S = a.BS * a.K;
  // LDS match tables for sub-chunks that give each wave several 64-slot groups, when they fit
  LayoutArgs b = a;
  const size_t base = layout_lds_bytes(W, a.Epad, a.Svpad, a.P, a.NS, a.BSv, 0);
  const int mw = a.E > a.P ? a.E : a.P;
  const bool big = a.BSv * a.K > W * 64 && base + (size_t)W * mw * 8 <= kMaxLds;
  b.mt = big ? mw : 0;
  const size_t lds = layout_lds_bytes(W, a.Epad, a.Svpad, a.P, a.NS, a.BSv, b.mt);
  const dim3 grid((unsigned)(a.P * a.m + a.pf_wgs));
  const bool subs = a.m > 1;
  hipError_t err = subs ? launch_count<true>(b, W, big, grid, lds, stream) : launch_count<false>(b, W, big, grid, lds, stream);
  if (err != hipSuccess) return err;
  // with more than 1024 slots per chunk every slot is loaded at the start
  const dim3 sgrid((unsigned)(a.P + a.pf_wgs));
  if (S > 1024 && subs)
    hipLaunchKernelGGL((layout_scan_finalize_kernel<8, true>), sgrid, dim3(1024), 0, stream, a);
  else if (S > 1024)
    hipLaunchKernelGGL((layout_scan_finalize_kernel<8, false>), sgrid, dim3(1024), 0, stream, a);
  else if (subs)
    hipLaunchKernelGGL((layout_scan_finalize_kernel<1, true>), sgrid, dim3(1024), 0, stream, a);
  else
    hipLaunchKernelGGL((layout_scan_finalize_kernel<1, false>), sgrid, dim3(1024), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_layout_dispatch(const LayoutArgs &a, const DispatchArgs &d, int quant_mode, bool per_expert,
                                  hipStream_t stream) {
  if (use_fused(a, true, quant_mode)) {
    return layout_waves(a.E) == 16 ? launch_fused_mode<16>(a, d, quant_mode, per_expert, stream)
                                   : launch_fused_mode<8>(a, d, quant_mode, per_expert, stream);
  }
  // the layout kernels are latency-bound on a few workgroups and leave HBM idle: extra workgroups
  // of theirs read the dispatch's token rows ahead into the Infinity Cache (results unchanged).
  // Measured per layer (layout + dispatch + combine, ten rotating input sets, one process, the same
  // builds alternated): T=4096, H=7168, top-8, int8 157.0 -> 152.0 us; T=16384 masked int8 570.4 ->
  // 560.3 us; bf16 rows (the copy's stores then non-temporal) about 1% (196.2 -> 194.6 us at T=4096,
  // 227.4 -> 224.9 us at T=8192, H=4096; 8 alternated repetitions).  128 extra workgroups per kernel
  // measured best of 64, 128 and 256 (64: slower than none).
  // (only the two-kernel layout carries the read-ahead workgroups; a world small enough for the
  // single-kernel layout, dispatched in a second kernel, reads its rows in the dispatch)
  LayoutArgs b = a;
  const bool ahead = d.x && a.T > 0 && !use_fused(a, false);
  if (ahead) {
    b.pf = d.x;
    b.pf_bytes = (int64_t)a.T * d.H * 2;
    b.pf_half = (b.pf_bytes / 32) * 16;
    b.pf_wgs = kReadAheadWorkgroups;
  }
  const hipError_t e = launch_layout(b, stream);
  if (e != hipSuccess) return e;
  return launch_dispatch(d, quant_mode, per_expert, stream, 0, ahead);
}

}  // namespace moe
