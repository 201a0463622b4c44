// The fp8-key scoring body (indexer + fused decode selection), shared by the
// scoring kernel and the fused decode step kernel.  Lightweight indexer:
// S_j = sum_h g_h * relu(q_h . K_j) for every pooled block j before the query's own
// block (reading notes "GLM-5.3-Flash: Hybrid Attention, IndexPool, and
// Vision-in-the-Loop", section 2 "Hybrid Attention: Linear State + Sparse
// Retrieval").
#pragma once
#include "append.hpp"
#include "select.hpp"

namespace ip {
namespace scorek {

constexpr int TILES = 4;                        // 32-key tiles per wave (default)
constexpr int SCORE_SPIN_LIMIT = 1 << 22;       // bound on the fallback's wait for score acknowledgements

// Waits until at most N of this wave's vector memory operations are outstanding
// (they complete in issue order).  vmcnt is bits 0..3 and 14..15 of the immediate;
// expcnt and lgkmcnt stay at their maxima (no wait).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
constexpr int HI = 32, DI = 128;

struct QStage {
  static constexpr int QROW = DI + 8;           // padded LDS row (272 bytes): conflict-free reads
  uint16_t qs[2][HI * QROW];                    // double-buffered query rows
  float gs[2][HI];
};

// the largest of the 16 values of this lane's 16-lane row (DPP within rows)
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp_f<0xB1>(-INFINITY, x));      // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp_f<0x4E>(-INFINITY, x));      // quad_perm [2,3,0,1]
  x = fmaxf(x, dpp_f<0x141>(-INFINITY, x));     // row_half_mirror
  x = fmaxf(x, dpp_f<0x140>(-INFINITY, x));     // row_mirror
  return x;
}

// The number of per-wave lists the fused selection ranks row r from (nel eligible
// blocks, need = k' - 1), or 0: the row is trivial (its own block alone, or every
// block), or too short or too long for lists (it selects from its scores).
template <int NWV, int TILES>
__device__ __forceinline__ int fused_list_count(int nel, int need, bool have_lists) {
  constexpr int NTW = NWV * 64, KEYS = NWV * TILES * 32;
  const bool trivial = need == 0 || need >= nel;
  const int n_lists = (nel + KEYS - 1) / KEYS * NWV;
  // rows long enough for about 2 winners per wave
  const bool ok = !trivial && have_lists && n_lists * sel::LIST <= sel::C_CAP && n_lists <= NTW &&
                  need <= TILES / 2 * n_lists;
  return ok ? n_lists : 0;
}

template <int NWV, bool FUSE>
constexpr size_t score_smem() {
  return FUSE && sizeof(sel::Shared<NWV * 64>) > sizeof(QStage) ? sizeof(sel::Shared<NWV * 64>) : sizeof(QStage);
}

// RPW query rows share one key chunk held in registers (prefill, where consecutive
// rows are tokens of one sequence); decode rows are separate sequences and use 1.
// A workgroup of NWV waves covers NWV * 128 keys.  All key loads of a wave are
// issued before the first MFMA: decode launches use 8 waves (1024 keys, 132 KB of
// pooled rows in flight per workgroup) so that one workgroup per compute unit
// covers the whole batch of the 128K-token decode workload at once.
// The body of the scoring kernel for the workgroup at grid position (bx, by) of a
// grid gx wide.  smem: score_smem<NWV, FUSE>() bytes of LDS, 16-byte aligned;
// last_here: one int of LDS.  sel_ready (fused selection only, or null): row r's
// word is set to 1 (device-coherent) once its selected ids are stored, for
// consumers in the same launch.
template <int RPW, int NWV, bool FUSE, int TILES = scorek::TILES>
__device__ __forceinline__ void score_fp8_body(const ScoreArgs& a, const int bx, const int by, const int gx,
                                               uint8_t* smem, int& last_here, uint32_t* sel_ready) {
  static_assert(!FUSE || RPW == 1, "the fused selection handles one row per workgroup");
  constexpr int NTW = NWV * 64;
  constexpr int KEYS = NWV * TILES * 32;
  static_assert(SCORE_TILE % KEYS == 0, "score rows pad to whole workgroup tiles");
  constexpr int QROW = QStage::QROW;
  QStage& st = *reinterpret_cast<QStage*>(smem);
  auto& qs = st.qs;
  auto& gs = st.gs;
  if (a.with_append && by >= a.n_rows) {
    // the fused decode append, one sequence per workgroup of the extra grid rows:
    // scoring reads pooled rows of blocks before the query's own block only, and
    // the append writes the new token's rows and the pooled row of the block it
    // completes (the query's own block)
    const int b = (by - a.n_rows) * gx + bx;
    if (b < a.append.batch) append_one<NTW>(a.append, b);
    return;
  }
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int kl = lane & 31, hh = lane >> 5;
  const int kc0 = bx * KEYS;
  const int rbeg = a.row0 + by * RPW;
  const int rend = min(rbeg + RPW, a.row0 + a.n_rows);

  // query rows (8 KB) and gates go through LDS; row r+1's are loaded while row r
  // is computed, and staged in the other buffer, so one barrier per row suffices
  // and the load latency of a row is hidden behind the previous one.  Thread t
  // (t < 256) holds elements 16t .. 16t+15 = head t/8, dims (t%8)*16 ..
  const bool qt = threadIdx.x < 256;
  u32x4_t qv0, qv1;
  float gv = 0.f;
  auto load_q = [&](int r) {
    const u32x4_t* qg = (const u32x4_t*)((const uint16_t*)a.q + (int64_t)r * HI * DI);
    if (qt) {
      qv0 = qg[2 * threadIdx.x];
      qv1 = qg[2 * threadIdx.x + 1];
    }
    if (threadIdx.x < HI) gv = a.gates[(int64_t)r * HI + threadIdx.x];
  };
  auto stage_q = [&](int buf) {
    const int h = threadIdx.x >> 3, d = (threadIdx.x & 7) * 16;
    if (qt) {
      *(u32x4_t*)(qs[buf] + h * QROW + d) = qv0;
      *(u32x4_t*)(qs[buf] + h * QROW + d + 8) = qv1;
    }
    if (threadIdx.x < HI) gs[buf][threadIdx.x] = gv;
  };
  // per-row sequence, position and pooled-row count, one row per lane, read once
  // (per-row loads inside the loop would each wait for every load in flight)
  int rb = 0, rp = 0, rn = 1;
  if (lane < rend - rbeg) {
    const int rr = rbeg + lane;
    rb = a.q_seq ? a.q_seq[rr] : rr;
    const int len = a.L.seq_lens[rb];
    rp = a.q_pos ? a.q_pos[rr] : len - 1;
    rn = (len + 3) >> 2;
  }
  load_q(rbeg);
  stage_q(0);
  if (rbeg + 1 < rend) load_q(rbeg + 1);

  // one row per workgroup: the fp8 codes stay as loaded and are widened tile by tile
  // as the MFMAs take them (half the registers); several rows: widened once
  constexpr bool LAZY = RPW == 1;
  u32x4_t kraw[LAZY ? TILES : 1][4];
  bf16x8_t kf[LAZY ? 1 : TILES][8];
  float ksig[TILES];
  float scv[TILES];                             // this lane's scores of the last row (all tiles)
  float gmv[TILES];                             // and their group maxima
  int cur_b = -1;

  for (int r = rbeg, i = 0; r < rend; ++r, ++i) {
    // row r's query is visible in buffer i&1, and every wave is done with buffer
    // (i+1)&1 (read in row r-1); LDS-only barrier: loads in flight are not waited for
    block_sync_lds();
    const int b = __builtin_amdgcn_readlane(rb, i);
    const int p = __builtin_amdgcn_readlane(rp, i);
    const int nel = p >> 2;                    // eligible blocks j < b_q
    const bool run = kc0 < nel;                // uniform over the workgroup
    if (run && b != cur_b) {
      cur_b = b;
      // pooled rows that exist; keys past them are clamped to the last one (their
      // scores are never written), so every load is unconditional and all of a
      // wave's loads are in flight together
      const int nrows = __builtin_amdgcn_readlane(rn, i);
      u32x4_t raw[LAZY ? 1 : TILES][4];
#pragma unroll
      for (int t = 0; t < TILES; ++t) {
        const int j = min(kc0 + (wv * TILES + t) * 32 + kl, nrows - 1);
        const int64_t row = a.L.pool_row(b, j);
        const u32x4_t* src = (const u32x4_t*)(a.keys + row * a.key_stride + hh * 64);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if constexpr (LAZY) kraw[t][c] = src[c];
          else raw[t][c] = src[c];
        }
        ksig[t] = a.key_scale[row];
      }
      if constexpr (!LAZY) {
#pragma unroll
        for (int t = 0; t < TILES; ++t)
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            kf[t][2 * c] = fp8x8_to_bf16x8_pk(raw[t][c][0], raw[t][c][1]);
            kf[t][2 * c + 1] = fp8x8_to_bf16x8_pk(raw[t][c][2], raw[t][c][3]);
          }
        // the scales land here too, so that no later use of them waits for the
        // query prefetch issued after this point
#pragma unroll
        for (int t = 0; t < TILES; ++t) asm volatile("" ::"v"(ksig[t]));
      }
    }
    const uint16_t* qb = qs[i & 1];
    const float* gb = gs[i & 1];
    // query fragment: head kl, dims hh*64 .. hh*64+63 (the same dims as the key half)
    bf16x8_t qf[8];
    // gates of the 16 heads this lane accumulates: rows (i/4)*8 + hh*4 + i%4
    float g[16];
    if (run) {
#pragma unroll
      for (int c = 0; c < 8; ++c) qf[c] = *(const bf16x8_t*)(qb + kl * QROW + hh * 64 + c * 8);
#pragma unroll
      for (int e = 0; e < 16; ++e) g[e] = gb[(e >> 2) * 8 + hh * 4 + (e & 3)];
    }
    // stage row r+1 and fetch row r+2.  Staging waits for row r+1's loads, issued
    // one row ago, and for whatever followed them (row r-1's score stores): both
    // have had a row's time to finish.
    if (r + 1 < rend) {
      stage_q((i + 1) & 1);
      if (r + 2 < rend) load_q(r + 2);
    }
    if (!run) continue;

    float* srow = a.scores + (int64_t)(r - a.row0) * a.ld;
    float* grow = a.gm + (int64_t)(r - a.row0) * a.gld;
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
      f32x16_t acc = {};
      if constexpr (LAZY) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[2 * c], fp8x8_to_bf16x8_pk(kraw[t][c][0], kraw[t][c][1]), acc,
                                                        0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[2 * c + 1], fp8x8_to_bf16x8_pk(kraw[t][c][2], kraw[t][c][3]),
                                                        acc, 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[c], kf[t][c], acc, 0, 0, 0);
      }
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) part = fmaf(g[e], fmaxf(acc[e], 0.f), part);
      part += __shfl_xor(part, 32);
      const int j = kc0 + (wv * TILES + t) * 32 + kl;
      const float sc = j < nel ? part * ksig[t] : -INFINITY;
      scv[t] = sc;
      // fused: stored after the wave's list (see below), so that building the list
      // does not wait for these stores
      if constexpr (FUSE) {
        // the maximum of each group of 16 consecutive blocks: lanes kl 0..15 and
        // 16..31 of the tile are 16-lane rows
        gmv[t] = row16_max(sc);
      } else {
        if (hh == 0 && j < nel) srow[j] = sc;
        if (a.gm) {                              // only the whole-row select reads them
          const float gmax = row16_max(sc);
          if (hh == 0 && j < nel && (kl & 15) == 0) grow[j >> 4] = gmax;
        }
      }
    }
  }
  if constexpr (FUSE) {
    // one row: select it once every workgroup that scored it has stored its part
    const int r = rbeg;
    const int p = __builtin_amdgcn_readlane(rp, 0);
    const int nel = p >> 2;
    const int need = min(a.top_k, nel + 1) - 1;
    int32_t* out = a.out + (int64_t)r * a.top_k;
    sel::Shared<NTW>& ss = *reinterpret_cast<sel::Shared<NTW>*>(smem);
    const bool trivial = need == 0 || need >= nel;   // nothing to rank: the own block alone, or every block
    const int n_run = (nel + KEYS - 1) / KEYS;
    const int n_lists = n_run * NWV;
    // rows long enough for about 2 winners per wave: every wave lists its best
    // (see sel::wave_list) and the last workgroup merges the lists
    const bool lists = fused_list_count<NWV, TILES>(nel, need, a.lists != nullptr && a.max_lists > 0) > 0;
    // the fused decode step: the attention workgroups of a list row merge its lists
    // themselves, those of a trivial row write its ids directly; the scoring
    // workgroups of those rows store their scores and lists and end
    const bool step = a.step != 0;
    // rows too long for per-wave lists (a 1M-token row has 2048 waves): the waves'
    // lists of a workgroup are reduced to one list of its 16 best (sel::wave_list
    // over their union), and the last workgroup merges one list per workgroup
    const bool wgl = FUSE && NWV == 8 && TILES == 4 && !step && !lists && !trivial && a.lists != nullptr && a.wg_lists >= n_run &&
                     n_run * sel::LIST <= sel::C_CAP && n_run <= NTW && need <= sel::LIST / 2 * n_run;
    const int lpr = lists ? a.max_lists : a.wg_lists;   // lists per row in the workspace
    uint64_t* lrow = (lists || wgl) ? a.lists + (int64_t)(r - a.row0) * lpr * sel::LIST : nullptr;
    uint2* mrow = (lists || wgl) ? a.lists_meta + (int64_t)(r - a.row0) * lpr : nullptr;
    // With lists and the scores in the workspace, a workgroup counts itself in once
    // its lists are acknowledged, without waiting for its score stores: the scores are
    // read only by the exact fallback, which first waits until every workgroup of the
    // row has counted its acknowledged scores into the counter of the row's current
    // parity (ack[0] = parity, ack[1 + parity] = the count; the row's selecting
    // workgroup clears the other counter and flips the parity for the next call,
    // after every workgroup of this call has read it).
    const bool defer = !step && lists && a.ack && a.scores_own;
    uint32_t* ack = defer ? a.ack + (int64_t)(r - a.row0) * 3 : nullptr;
    // the parity, read (device-coherently) before the lists are stored; it has landed
    // by the time the count moves, and is first used after that
    uint32_t par_v = 0;
    if (defer && kc0 < nel)
      par_v = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(sel::dev_rsrc(ack), 0u, 0, 16 /* sc1 */);
    if (kc0 < nel) {
      const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, hh = lane >> 5, kl = lane & 31;
      // the scores and group maxima (read by the exact fallback, and the caller's
      // score output)
      auto store_scores = [&]() {
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        float* srow = a.scores + (int64_t)(r - a.row0) * a.ld;
        float* grow = a.gm + (int64_t)(r - a.row0) * a.gld;
        if (defer || (step && a.scores_own)) {
          // every lane writes (the two halves hold the same score, a group's 16 lanes
          // the same maximum, and rows of the workspace are padded to whole tiles):
          // unconditional stores stay in flight together.  Deferred: exactly 2 TILES
          // stores per wave, after the lists, so that waiting for all but the last
          // 2 TILES of the wave's memory operations waits for its lists
#pragma unroll
          for (int t = 0; t < TILES; ++t) {
            const int j = kc0 + (wv * TILES + t) * 32 + kl;
            sel::st_agent(srow + j, scv[t]);
            sel::st_agent(grow + (j >> 4), gmv[t]);
          }
          if (defer) {
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            wait_vm<2 * TILES>();
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
          }
        } else {
#pragma unroll
          for (int t = 0; t < TILES; ++t) {
            const int j = kc0 + (wv * TILES + t) * 32 + kl;
            if (hh == 0 && j < nel) {
              sel::st_agent(srow + j, scv[t]);
              if ((kl & 15) == 0) sel::st_agent(grow + (j >> 4), gmv[t]);
            }
          }
        }
      };
      // the fused decode step: a wave stores its scores first and its list only once
      // they are acknowledged, so a row whose lists are all stored has all its scores
      // stored as well (the attention workgroups check every list before they merge,
      // and the exact fallback reads the scores after that).  Otherwise the scores go
      // after the list, so that building it does not wait for them.
      const bool scores_first = step && lists;
      if (scores_first) store_scores();
      if (lists) {
        constexpr int KPL = TILES / 2;           // keys per lane: half hh holds tiles KPL hh ..
        uint32_t k[KPL];
        int id[KPL];
#pragma unroll
        for (int i = 0; i < KPL; ++i) {
          const int t = KPL * hh + i;
          id[i] = kc0 + (wv * TILES + t) * 32 + kl;
          // scv read at indices known at compile time and blended by half (a
          // lane-dependent index would put the array in scratch or select chains)
          const uint32_t hm = 0u - (uint32_t)hh;
          const float sc = __uint_as_float((__float_as_uint(scv[i]) & ~hm) | (__float_as_uint(scv[KPL + i]) & hm));
          k[i] = id[i] < nel ? float_key(sc) : 0u;
        }
        const int slot = bx * NWV + wv;
        sel::wave_list<KPL>(k, id, lrow + (int64_t)slot * sel::LIST, mrow + slot, scores_first);
      }
      if constexpr (NWV == 8 && TILES == 4) if (wgl) {
        constexpr int KPL = TILES / 2;
        uint32_t k[KPL];
        int id[KPL];
#pragma unroll
        for (int i = 0; i < KPL; ++i) {
          const int t = KPL * hh + i;
          id[i] = kc0 + (wv * TILES + t) * 32 + kl;
          const uint32_t hm = 0u - (uint32_t)hh;
          const float sc = __uint_as_float((__float_as_uint(scv[i]) & ~hm) | (__float_as_uint(scv[KPL + i]) & hm));
          k[i] = id[i] < nel ? float_key(sc) : 0u;
        }
        // the wave's list into LDS (past the query stage, which other waves may
        // still read), then wave 0 lists the union of the NWV lists: entry u = 16w + p
        // (ascending ids) sits in segment u / 32 of wave_list's order, half u / 64
        static_assert(NWV * sel::LIST == 2 * 64 && KPL == 2, "the waves' lists fill two keys per lane");
        sel::wave_list<KPL, true>(k, id, ss.wl + wv * sel::LIST, ss.wm + wv);
        __syncthreads();
        if (wv == 0) {
          uint32_t uk[2];
          int ui[2];
          uint32_t lpm = 0u;
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const int u = 64 * (lane >> 5) + 32 * i + (lane & 31);
            const int w = u / sel::LIST, p = u % sel::LIST;
            const uint2 m = ss.wm[w];
            const uint64_t e = ss.wl[u];
            const bool on = p < (int)(m.x & 0xFFu);
            uk[i] = on ? (uint32_t)e : 0u;
            ui[i] = on ? (int)(e >> 32) : 0;
          }
#pragma unroll
          for (int w = 0; w < NWV; ++w) lpm = max(lpm, ss.wm[w].y);
          sel::wave_list<2>(uk, ui, lrow + (int64_t)bx * sel::LIST, mrow + bx, false, lpm);
        }
      }
      if (!scores_first) store_scores();
    }
    if (step && (trivial || lists)) return;
    // the row's ids are stored (device-coherent stores): publish them
    auto publish = [&]() {
      if (!sel_ready) return;
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (threadIdx.x == 0) sel::st_agent(sel_ready + (r - a.row0), 1u);
    };
    // this workgroup's scores are acknowledged: count them in (deferred mode)
    uint32_t par = 0;
    auto count_scores = [&]() {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      par = __builtin_amdgcn_readfirstlane(par_v);
      if (threadIdx.x == 0) atomicAdd(ack + 1 + par, 1u);
    };
    if (trivial) {
      if (bx == 0) {
        __syncthreads();
        sel::select_row<NTW>(nullptr, nullptr, nel, nel, a.top_k, out, ss);
        publish();
      }
      return;
    }
    if (kc0 >= nel) return;                      // this workgroup scored nothing
    // every list entry (and, unless deferred, every score and maximum) of this
    // workgroup is stored (acknowledged by memory) before it counts itself in: the
    // stores are device-coherent, so the workgroup that completes the count reads
    // them with device-coherent loads
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (!defer) __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __syncthreads();
    if (threadIdx.x == 0) last_here = atomicAdd(a.count + (r - a.row0), 1) == n_run - 1;
    __syncthreads();
    if (!last_here) {
      if (defer) count_scores();
      return;
    }
    if (threadIdx.x == 0) sel::st_agent(a.count + (r - a.row0), 0);   // clear for the next call
    if (!((lists || wgl) && sel::merge_lists<NTW>(lrow, mrow, wgl ? n_run : n_lists, need, nel, a.top_k, out, ss))) {
      if (defer) {
        // the fallback reads every score of the row: wait (bounded) until every
        // workgroup has counted its acknowledged scores in
        count_scores();
        if (threadIdx.x == 0)
          for (int n = 0; sel::ld_agent(ack + 1 + par) < (uint32_t)n_run && n < SCORE_SPIN_LIMIT; ++n)
            __builtin_amdgcn_s_sleep(1);
        __syncthreads();
      }
      __syncthreads();
      sel::select_row<NTW>(a.scores + (int64_t)(r - a.row0) * a.ld, a.gm + (int64_t)(r - a.row0) * a.gld, nel,
                           nel, a.top_k, out, ss);
    } else if (defer) {
      count_scores();
    }
    if (defer && threadIdx.x == 0) {
      // every workgroup of this call has read the parity (it counted itself in
      // before the row's count completed): clear the other counter, flip
      sel::st_agent(ack + 2 - par, 0u);
      sel::st_agent(ack, 1u - par);
    }
    publish();
  }
}

}  // namespace scorek
}  // namespace ip
