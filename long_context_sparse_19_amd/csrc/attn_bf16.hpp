// The bf16 latent attention bodies (64-head and 32-head units) and their helpers,
// shared by the kernels of attn.hip and the fused decode step with 32-head units
// (attn_step_h32.hip, a unit of its own so that each step kernel keeps the
// register allocation it has alone).
//
// Sparse attention over the tokens of the selected blocks.  G2C Brief "GLM-5.3-Flash:
// hybrid attention becomes the product", section "DSA keeps selected global access
// in eleven layers": the DSA layers keep a token-addressable MLA latent history
// (rank 512 per token) and attend over the selected subset of it.
//
// bf16 latent path (MQA, 64 heads over one 576-dim latent row, V = first 512 dims):
//   one workgroup (4 waves) per (query row, split of the selected blocks) covers all
//   64 heads, so every gathered latent row is read from memory once and feeds 64
//   heads.  The selected rows are staged 64 tokens (16 blocks of 4 contiguous rows)
//   at a time into LDS by LDS DMA, double buffered.  The kernel is bound by LDS
//   reads, so both products use v_mfma_f32_32x32x16_bf16, whose operand fragments
//   each feed 32 heads:
//   - S^T = K . q^T: wave w takes heads 32(w&1) .. +31 against tokens 32(w>>1) .. +31
//     (its 32 heads of q, 576 dims, stay in accumulation registers);
//   - online softmax in base 2 against a per-head reference maximum shared by the
//     two waves of a head block; it moves (and O and l with it) only when a tile
//     maximum passes it by more than 2^8, which after the first sub-tile is rare, so
//     the common path needs no exchange of maxima; P goes to LDS as bf16;
//   - O^T[dims, heads] += V^T . P^T: wave w takes dims 128w .. +127 for all 64 heads,
//     V read with the transposing LDS read (ds_read_b64_tr_b16).
//   Two barriers per sub-tile: P complete, and next sub-tile landed / buffer free.
//   With more than one split the partials (O, reference maximum, l) are merged by a
//   combine kernel.
// f32 path (small geometries): plain VALU, one workgroup per row.
#pragma once
#include "attn_common.hpp"
#include "score_fp8.hpp"
#include "stamps.hpp"

namespace ip {

namespace {

constexpr int NT = 256;                        // f32 path
constexpr int NTA = 256;                       // bf16 path: 4 waves
constexpr int NWA = NTA / 64;
constexpr int SUBT = 64;                       // tokens per sub-tile (16 blocks)
constexpr int SEGB = SUBT * 128;               // one 128-byte segment (64 dims) of all 64 rows
constexpr int KVBUF = NSEG * SEGB;             // 73728 bytes
constexpr int CHUNKS = LAT_DK * 2 / 16;        // 72 16-byte chunks per latent row
constexpr int KSTEPS = LAT_DK / 16;            // 36 MFMA k-steps over the 576 dims

typedef float f32x4v __attribute__((ext_vector_type(4)));

// The two latent sub-tile buffers are LDS objects of their own (filled by LDS DMA),
// apart from the rest of the shared data.  The compiler tags accesses with the LDS
// object they touch, so it can see that reading one buffer (or the other shared
// data) does not alias the DMA into the other buffer, and does not make those
// accesses wait for the outstanding sub-tile loads.  For that every access must
// name its buffer statically: the main loop is unrolled by two.
constexpr int PROW = SUBT * 2 + 16;            // P row of one head: 64 bf16 + pad = 144 bytes

struct __align__(16) AttnShared {
  uint32_t brow[MAX_BLOCKS_PER_SPLIT];
  float tmax[2][LAT_H];                        // tile maxima of the two token halves
  float lpart[2][LAT_H];                       // l of the two token halves (end)
  int need[4];                                 // a wave's tile maximum passed the reference
};

// Block table of the split: entry i = physical row of the first token of block
// sel[sb0 + i] with the number of its tokens at or before the query (0..4) in the
// top bits.  Entries that are -1, past the split or entirely after the query
// point at the query's own block (whose 4 rows exist) with 0 visible tokens, so
// every load stays inside the cache.  Thread t handles entries t and t + NTA: the
// selection ids are fetched first (fetch_blocks) and turned into entries together
// with the other ids of the prologue (block_entries).
struct BlockIds {
  int blk[MAX_BLOCKS_PER_SPLIT / NTA];
};

// selection id bi of the row: COH reads ids stored by another workgroup of the same
// launch (device-coherent load, sc1)
template <bool COH>
__device__ __forceinline__ int sel_id(const RowCtx& c, int bi) {
  if constexpr (COH) return (int)__builtin_amdgcn_raw_buffer_load_b32(sel::dev_rsrc(c.sel), (uint32_t)bi * 4u, 0, 16);
  return c.sel[bi];
}

template <bool COH>
__device__ __forceinline__ BlockIds fetch_blocks(const RowCtx& c, int sb0, int send) {
  BlockIds ids;
#pragma unroll
  for (int k = 0; k < MAX_BLOCKS_PER_SPLIT / NTA; ++k) {
    const int bi = sb0 + (int)threadIdx.x + k * NTA;
    ids.blk[k] = bi < send ? sel_id<COH>(c, bi) : -1;
  }
  return ids;
}


// Sub-tile layout in LDS: 9 segments of 8 KB, segment g holding bytes 128g ..
// 128g+127 (dims 64g .. 64g+63) of all 64 rows, row t at 128t, with the eight
// 16-byte chunks of each 128-byte piece stored in slots chunk ^ x(t),
// x(t) = 2(t % 4) + (t / 4) % 2.  Within 8 consecutive rows x takes all 8 values,
// so a K fragment read (the same chunk of 8 rows per LDS cycle) hits every bank
// once; within 4 consecutive rows x keeps the chunk pairs (2i, 2i+1) of the
// transposing V reads apart.
//
// Sub-tile n goes straight from global memory into that layout with
// global_load_lds_dwordx4 (lane l of one instruction fills bytes 16l .. 16l+15 of a
// 1 KB span): instruction (g, q) fills rows 8q .. 8q+7 of segment g, lane l taking
// slot l%8 of row 8q + l/8, i.e. chunk (l%8) ^ x of that row.  Each instruction
// touches 8 whole 128-byte lines.  Wave w issues the 18 instructions q = 2w, 2w+1
// and g = 0 .. 8, so each lane reads two rows per sub-tile.
constexpr int KV_LOADS = NSEG * 8 / NWA;       // 18 per wave


// byte offset in a sub-tile buffer of 16-byte chunk `ch` (0..71) of row `t`
__device__ __forceinline__ int kv_off(int t, int ch) {
  return (ch >> 3) * SEGB + t * 128 + 16 * ((ch & 7) ^ kv_swz(t));
}

// This lane's two source rows for sub-tile n; load k (0..17) is segment k/2 of
// row half k%2.
struct SubtileSrc {
  const uint8_t* row[2];
};

// The entries of this lane's two blocks, 4wv + (l >> 5) and that + 2, from one
// 16-byte read of entries 4wv .. 4wv+3.  (Two 4-byte reads get merged into one
// ds_read2 that the compiler can no longer tell apart from the LDS DMA in flight,
// and it then waits for all of it.)
__device__ __forceinline__ void subtile_entries(const AttnShared& sh, int n, uint32_t (&e)[2]) {
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const u32x4_t q = lds_ld((const u32x4_t*)&sh.brow[n * 16 + 4 * wv]);
  e[0] = (lane >> 5) ? q[1] : q[0];
  e[1] = (lane >> 5) ? q[3] : q[2];
}

// The query's own token row in the fused decode step: the cache row the same
// launch appends (row = its index) is read from the new token's input row (src)
// instead, so no workgroup reads a cache row while it is being written.  row =
// ~0u: no redirect.
struct NewRow {
  uint32_t row;
  const uint8_t* src;
};

template <bool STEP>
__device__ __forceinline__ const uint8_t* kv_row_src(const AttnArgs& a, const NewRow& nr, uint32_t grow, int swz) {
  if constexpr (STEP) return (grow == nr.row ? nr.src : a.k + (uint64_t)grow * a.k_stride) + swz;
  return a.k + (uint64_t)grow * a.k_stride + swz;
}

template <bool STEP>
__device__ __forceinline__ SubtileSrc subtile_src(const AttnArgs& a, const AttnShared& sh, int n, const NewRow& nr) {
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint32_t e[2];
  subtile_entries(sh, n, e);
  SubtileSrc src;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int t = 8 * (2 * wv + h) + (lane >> 3);
    const uint32_t grow = (e[h] & ROW_BITS) + (t & 3);
    src.row[h] = kv_row_src<STEP>(a, nr, grow, 16 * ((lane & 7) ^ kv_swz(t)));
  }
  return src;
}

__device__ __forceinline__ void load_column(const SubtileSrc& src, uint8_t* buf, int k) {
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = k >> 1, h = k & 1;
  __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(src.row[h] + 128 * g),
                                   (void __attribute__((address_space(3)))*)(buf + g * SEGB + (2 * wv + h) * 1024),
                                   16, 0, 0);
}


// The fused decode step's scoring role: 4 waves of 8 tiles (1024 keys per
// workgroup, as the standalone fused scoring's 8 waves of 4 tiles), the register
// budget of one wave per SIMD that the attention role needs anyway.
constexpr int STEP_NWV = 4, STEP_TILES = 8;
static_assert(sizeof(sel::Shared<NTA>) <= KVBUF, "the selection state fits a sub-tile buffer");
static_assert(MAX_BLOCKS_PER_SPLIT * 4 <= LAT_H * PROW, "a split's ids fit the P buffer");

// The fused decode step: the ids of positions [sb0, send) of row rl's selection
// into lid (LDS), and for the rows selected here into the row of sel_out.
//  - Trivial rows (the query's own block alone, or every block): the ids directly.
//  - List rows: the row's per-wave lists (whose loads sl started), merged as soon
//    as every list is stored (see sel::StepLists).  When the lists cannot decide the row, split 0 runs
//    the exact select over the row's scores once every scoring workgroup has counted
//    its scores in, and publishes the ids; the other splits wait for them.
//  - Other rows: the ids published by the row's last scoring workgroup.
// ss (the first sub-tile buffer) holds the selection state; it is free again on
// return.  Waits only on workgroups that started earlier, bounded as the others.
__device__ __forceinline__ void step_select(const AttnArgs& a, const RowCtx& c, int rl, int split, int sb0,
                                            int send, int32_t* lid, uint8_t* kv0, sel::StepLists<NTA, 8>& sl) {
  sel::Shared<NTA>& ss = *reinterpret_cast<sel::Shared<NTA>*>(kv0);
  const int nel = c.p >> 2;                      // eligible blocks j < b_q
  const int need = min(a.top_k, nel + 1) - 1;
  const int n = send - sb0;
  int32_t* row_out = a.sel_out + (int64_t)(a.row0 + rl) * a.top_k;
  bool local = true;
  if (need == 0 || need >= nel) {
    for (int i = threadIdx.x; i < n; i += NTA) {
      const int pos = sb0 + i;
      lid[i] = pos < need ? pos : (pos == need ? nel : -1);
    }
  } else {
    const int n_lists = scorek::fused_list_count<STEP_NWV, STEP_TILES>(nel, need, a.step_lists != nullptr);
    local = n_lists > 0 && sl.merge(n_lists, need, nel, a.top_k, sel::SliceOut{lid, sb0, send}, ss);
    if (!local && n_lists > 0 && split == 0) {
      // the merge saw every list of the row stored, and a scoring wave stores its list
      // only once its scores are acknowledged: every score of the row is in memory
      __syncthreads();
      sel::select_row<NTA>(a.step_scores + (int64_t)rl * a.step_ld, a.step_gm + (int64_t)rl * a.step_gld, nel, nel,
                           a.top_k, row_out, ss);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (threadIdx.x == 0) sel::st_agent(a.sel_ready + rl, 1u);
    }
  }
  if (!local) {
    if (threadIdx.x == 0)
      for (int k = 0; sel::ld_agent(a.sel_ready + rl) == 0u && k < STEP_SPIN_LIMIT; ++k) __builtin_amdgcn_s_sleep(1);
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += NTA) lid[i] = sel_id<true>(c, sb0 + i);
  }
  __syncthreads();                               // lid complete, ss free
  if (local)
    for (int i = threadIdx.x; i < n; i += NTA) __builtin_nontemporal_store(lid[i], row_out + sb0 + i);
}

// The body of the bf16 kernel for workgroup `bid` (4 waves, threads 0..255), over
// the LDS objects of the calling kernel.  STEP (the fused decode step): the query
// is fetched first, then the row's ids come from step_select (selected here, or
// published by another workgroup of the same launch), and the query's own token
// row comes from a.k_new.
template <bool STEP>
__device__ __forceinline__ void attn_bf16_body(const AttnArgs& a, const int bid, AttnShared& sh, uint8_t* pmat,
                                               uint8_t* kv0, uint8_t* kv1) {
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform (scalar)
  const int l32 = lane & 31, lh = lane >> 5;
  const int hb = wv & 1, th = wv >> 1;           // S^T tile: heads 32hb .., tokens 32th ..
  if (bid >= a.n_rows * a.n_split) return;
  // STEP: rows fastest, so that the splits of a row share a die (workgroups go to
  // the dies round robin) and split 0 of every row comes first
  const int split = STEP ? bid / a.n_rows : bid % a.n_split;
  const int rl = STEP ? bid % a.n_rows : bid / a.n_split;
  const int r = a.row0 + rl;
  const RowCtx c = row_ctx(a, r);
  const int sb0 = split * a.blocks_per_split;
  const int send = min(a.top_k, sb0 + a.blocks_per_split);
  const int nsub = (send - sb0 + 15) >> 4;
  const int hs = 32 * hb + l32;                  // head of this lane in the S^T layout
  // STEP: the first loads of the row's lists go out before anything else, while the
  // row's length is still on its way
  sel::StepLists<NTA, 8> sl;
  if constexpr (STEP)
    sl.start(a.step_lists + (int64_t)rl * a.step_max_lists * sel::LIST, a.step_meta + (int64_t)rl * a.step_max_lists,
             a.step_lists_n);

  // prologue: the selection ids (block-table entries and this lane's rows of
  // sub-tiles 0 and 1); the query row into kv1; sub-tile 0; q into registers; then
  // sub-tile 1 into kv1.  The query goes by LDS DMA in whole 128-byte lines (loads
  // of each lane's q fragments straight from memory measured 2.3 us slower per
  // decode step).
  BlockIds ids;
  // ids of this lane's source blocks for sub-tiles 0 and 1 (rows 8(2w + h) + l/8)
  int pid[2][2];
  // STEP: the split's ids in LDS (the P buffer, first written in step 0)
  int32_t* const lid = reinterpret_cast<int32_t*>(pmat);
  auto load_ids = [&]() {
    if constexpr (STEP) {
#pragma unroll
      for (int k = 0; k < MAX_BLOCKS_PER_SPLIT / NTA; ++k) {
        const int i = (int)threadIdx.x + k * NTA;
        ids.blk[k] = sb0 + i < send ? lid[i] : -1;
      }
    } else {
      ids = fetch_blocks<false>(c, sb0, send);
    }
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int bi = sb0 + 16 * n + ((8 * (2 * wv + h) + (lane >> 3)) >> 2);
        pid[n][h] = bi < send ? (STEP ? lid[bi - sb0] : sel_id<false>(c, bi)) : -1;
      }
  };
  if constexpr (!STEP) load_ids();
  {
    // the query row (64 heads x 576 dims = one sub-tile's bytes) goes to kv1 in the
    // sub-tile layout, head h as row h: whole 128-byte lines, and the fragment
    // reads below are the conflict-free K-fragment pattern
    SubtileSrc qsrc;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int t = 8 * (2 * wv + h) + (lane >> 3);
      qsrc.row[h] = (const uint8_t*)a.q + ((int64_t)r * LAT_H + t) * (LAT_DK * 2) + 16 * ((lane & 7) ^ kv_swz(t));
    }
#pragma unroll
    for (int k = 0; k < KV_LOADS; ++k) load_column(qsrc, kv1, k);
  }
  NewRow nr{~0u, nullptr};
  if constexpr (STEP) {
    nr = NewRow{(uint32_t)a.L.tok_row(c.b, c.p), a.k_new + (int64_t)c.b * a.k_new_stride};
    __builtin_amdgcn_sched_barrier(0);
    step_select(a, c, rl, split, sb0, send, lid, kv0, sl);
    IP_STAMP((int)blockIdx.x, ST_IDS);
    load_ids();
  }
  // every query DMA is issued before anything consumes the ids
  __builtin_amdgcn_sched_barrier(0);
  // entries: [0, 1] this thread's block-table entries, [2 + 2n + h] its source
  // rows of sub-tile n
  constexpr int NE = MAX_BLOCKS_PER_SPLIT / NTA;
  static_assert(NE == 2, "two block-table entries per thread");
  const int eb[6] = {ids.blk[0], ids.blk[1], pid[0][0], pid[0][1], pid[1][0], pid[1][1]};
  uint32_t ent[6];
  block_entries(a, c, eb, ent);
  const int nbt = ((send - sb0 + 15) >> 4) << 4;
  SubtileSrc src[2];
#pragma unroll
  for (int n = 0; n < 2; ++n)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int t = 8 * (2 * wv + h) + (lane >> 3);
      const uint32_t grow = (ent[2 + 2 * n + h] & ROW_BITS) + (t & 3);
      src[n].row[h] = kv_row_src<STEP>(a, nr, grow, 16 * ((lane & 7) ^ kv_swz(t)));
    }
#pragma unroll
  for (int k = 0; k < KV_LOADS; ++k) load_column(src[0], kv0, k);
#pragma unroll
  for (int k = 0; k < NE; ++k) {
    const int i = (int)threadIdx.x + k * NTA;
    if (i < nbt) lds_st(&sh.brow[i], ent[k]);
  }
  if (threadIdx.x < 4) lds_st(&sh.need[threadIdx.x], 0);
  wait_vm<KV_LOADS>();                           // this wave's part of q landed
  block_sync_lds();
  // q fragments: head hs, dims 16s + 8lh .. +8 for k-step s.  q only feeds MFMA B
  // operands, which may sit in accumulation registers: keep it there, leaving the
  // ordinary VGPRs to the O accumulators
  bf16x8_t qf[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) qf[s] = *(const bf16x8_t*)(kv1 + kv_off(hs, 2 * s + lh));
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) asm volatile("" : "+a"(qf[s]));
  block_sync_lds();                              // every wave has its q: kv1 is free
  // sub-tile 1, unconditionally (past the split the rows are the query's own
  // block), so that every path has the same loads in flight
#pragma unroll
  for (int k = 0; k < KV_LOADS; ++k) load_column(src[1], kv1, k);
  wait_vm<KV_LOADS>();                           // sub-tile 0 landed (this wave's part)
  block_sync_lds();
  if constexpr (STEP) IP_STAMP((int)blockIdx.x, ST_SUB0);
  const float cs = a.scale * LOG2E;

  // O^T tiles [32 dims, 32 heads]: o[i][db][k] = head 32i + l32, dim 128wv + 32db +
  // 8(k/4) + 4lh + k%4
  f32x16_t o[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int d = 0; d < 4; ++d) o[i][d] = f32x16_t{};
  // reference maxima: ms for head hs (S^T layout), mo[i] for head 32i + l32 (O layout)
  float ms = -INFINITY, mo[2] = {-INFINITY, -INFINITY};
  float l_half = 0.f;                            // l of head hs over this wave's token half

  // one sub-tile: compute on `buf`, while sub-tile n+1 streams into `nxt`
  auto step = [&](const int n, const uint8_t* buf, uint8_t* nxt) {
    // sub-tile n+1 is in flight since the previous step (or the prologue); `nxt`
    // was last read in step n-1, which every wave has left.  Sub-tile n+1 is
    // fetched one column per two k-steps of the S^T product below: each DMA
    // instruction takes long to issue, and between MFMAs that time is hidden.
    const bool fetch = n >= 1 && n + 1 < nsub;
    const SubtileSrc fsrc = subtile_src<STEP>(a, sh, fetch ? n + 1 : n, nr);
    // visible-token counts of this wave's 8 blocks, read before any fetch is in flight
    const u32x4_t bv0 = lds_ld((const u32x4_t*)&sh.brow[n * 16 + 8 * th]);
    const u32x4_t bv1 = lds_ld((const u32x4_t*)&sh.brow[n * 16 + 8 * th + 4]);
    // ---- S^T[token, head]: lane holds head hs, tokens 32th + 8q + 4lh + u (q, u < 4)
    //      Two accumulation chains (even and odd k-steps) keep back-to-back MFMAs
    //      independent; K fragments are read KPF k-steps ahead.
    f32x16_t sacc;
    {
      f32x16_t sa[2] = {f32x16_t{}, f32x16_t{}};
      const int t = 32 * th + l32;
      constexpr int KPF = 4;
      bf16x8_t kb[KPF];
#pragma unroll
      for (int p = 0; p < KPF; ++p) kb[p] = *(const bf16x8_t*)(buf + kv_off(t, 2 * p + lh));
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        sa[s & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb[s % KPF], qf[s], sa[s & 1], 0, 0, 0);
        if (s + KPF < KSTEPS) kb[s % KPF] = *(const bf16x8_t*)(buf + kv_off(t, 2 * (s + KPF) + lh));
        if ((s & 1) && fetch) load_column(fsrc, nxt, s >> 1);
      }
      sacc = sa[0] + sa[1];
    }
    // ---- masking, scale, this half's tile maximum of head hs
    float tm = -INFINITY;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t e = q < 2 ? (lh ? bv0[2 * q + 1] : bv0[2 * q]) : (lh ? bv1[2 * q - 3] : bv1[2 * q - 4]);
      const int vis = (int)(e >> VIS_SHIFT);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        sacc[4 * q + u] = u < vis ? sacc[4 * q + u] * cs : -INFINITY;
        tm = fmaxf(tm, sacc[4 * q + u]);
      }
    }
    tm = pair_max32(tm);
    if (lh == 0) lds_st(&sh.tmax[th][hs], tm);
    const bool need = __ballot(tm > ms + RESCALE_LOG2) != 0ull;
    if (need && lane == 0) lds_st(&sh.need[wv], 1);
    // P against the current reference (recomputed below in the rare case)
    auto write_p = [&](float m) {
      const float mu = m == -INFINITY ? 0.f : m;
      float ls = 0.f;
      uint8_t* pr = pmat + hs * PROW + (32 * th + 4 * lh) * 2;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float pv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) { pv[u] = exp2f(sacc[4 * q + u] - mu); ls += pv[u]; }
        lds_st((uint2*)(pr + 16 * q), make_uint2(pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3])));
      }
      return ls;
    };
    float ls = write_p(ms);
    block_sync_lds();
    // ---- rare: some head maximum passed its reference by more than 2^8.  Every
    //      wave moves the references to the new maxima, rescales what it holds,
    //      and P is rewritten.
    bool moved = false;
#pragma unroll
    for (int w = 0; w < 4; ++w) moved |= lds_ld(&sh.need[w]) != 0;
    if (moved) {
      const float msn = fmaxf(ms, fmaxf(lds_ld(&sh.tmax[0][hs]), lds_ld(&sh.tmax[1][hs])));
      l_half *= ms == -INFINITY ? 0.f : exp2f(ms - msn);
      ms = msn;
      ls = write_p(ms);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int h = 32 * i + l32;
        const float mon = fmaxf(mo[i], fmaxf(lds_ld(&sh.tmax[0][h]), lds_ld(&sh.tmax[1][h])));
        const float al = mo[i] == -INFINITY ? 0.f : exp2f(mo[i] - mon);
        mo[i] = mon;
#pragma unroll
        for (int d = 0; d < 4; ++d) o[i][d] *= al;
      }
      block_sync_lds();                          // new P complete; flags read by all
      if (threadIdx.x < 4) lds_st(&sh.need[threadIdx.x], 0);
    }
    l_half += pair_sum32(ls);
    // ---- O^T += V^T . P^T: dims 128wv + 32db, heads 32i, tokens 16ks .. +15
    {
      typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;
      // transposed V reads: in 16-lane group G, source lane s points at token
      // 16ks + 8(G>>1) + s/4 (+4 for the second read) and dims 16(G&1) + 4(s%4) of
      // the 32-dim block, so lane l receives dim l32 of tokens 16ks + 8lh + j
      const int g4 = lane >> 4, s16 = lane & 15;
      const int vt = 8 * (g4 >> 1) + (s16 >> 2);
      const int vd = 16 * (g4 & 1) + 4 * (s16 & 3);           // dim within the 32-dim block
      const int vch = vd >> 3, vin = (vd & 7) * 2;             // chunk of the block, byte in chunk
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        bf16x8_t pb[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) pb[i] = lds_ld((const bf16x8_t*)(pmat + (32 * i + l32) * PROW + (16 * ks + 8 * lh) * 2));
        // ks-step operands: 2 P reads and 8 V reads for 8 MFMAs
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const int ch = 4 * (4 * wv + db) + vch;             // chunk of the row: dims 128wv + 32db + vd
          const int t0 = 16 * ks + vt;
          const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(buf + kv_off(t0, ch) + vin));
          const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(buf + kv_off(t0 + 4, ch) + vin));
          const s16x4_t v8[2] = {lo, hi};
          const bf16x8_t va = __builtin_bit_cast(bf16x8_t, v8);
#pragma unroll
          for (int i = 0; i < 2; ++i) o[i][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[i], o[i][db], 0, 0, 0);
        }
      }
    }
    // ---- sub-tile n+1 has landed for every wave, and every wave is done with
    //      `buf` and with P, past this barrier.  The wait is unconditional: the
    //      compiler then knows no load is in flight when the next step starts
    //      (else it waits for sub-tile 1 at the top of step 0)
    wait_vm<0>();
    if (n + 1 < nsub) block_sync_lds();
  };
  for (int n = 0; n < nsub; n += 2) {
    step(n, kv0, kv1);
    if (n + 1 < nsub) step(n + 1, kv1, kv0);
  }
  if constexpr (STEP) IP_STAMP((int)blockIdx.x, ST_SUBS);

  // ---- epilogue: l of each head = sum of its two token halves
  if (lh == 0) lds_st(&sh.lpart[th][hs], l_half);
  block_sync_lds();                              // also: every wave is done with kv0 / kv1
  const bool final_out = a.n_split == 1;
  const int64_t pi = (int64_t)rl * a.n_split + split;
  // O in bf16 (normalised when final) goes through kv0 as rows of one head's 512
  // dims, OPITCH bytes apart (2-way bank conflicts at most on the writes), and
  // leaves in whole 1 KB rows; straight from the MFMA layout every store would
  // scatter 8-byte pieces over 64 rows
  constexpr int OPITCH = LAT_DV * 2 + 16;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int h = 32 * i + l32;
    const float sc = final_out ? 1.f / (lds_ld(&sh.lpart[0][h]) + lds_ld(&sh.lpart[1][h])) : 1.f;
    uint8_t* row = kv0 + h * OPITCH + (128 * wv + 4 * lh) * 2;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *(uint2*)(row + (32 * d + 8 * q) * 2) = make_uint2(pack_bf16x2(o[i][d][4 * q] * sc, o[i][d][4 * q + 1] * sc),
                                                           pack_bf16x2(o[i][d][4 * q + 2] * sc, o[i][d][4 * q + 3] * sc));
  }
  if (th == 0 && lh == 0) {
    const float lt = lds_ld(&sh.lpart[0][hs]) + lds_ld(&sh.lpart[1][hs]);
    if (final_out) {
      if (a.lse) a.lse[(int64_t)r * LAT_H + hs] = ((ms == -INFINITY ? 0.f : ms) + log2f(lt)) * LN2;
    } else {
      a.part_ml[(pi * LAT_H + hs) * 2] = ms == -INFINITY ? 0.f : ms;
      a.part_ml[(pi * LAT_H + hs) * 2 + 1] = lt;
    }
  }
  block_sync_lds();
  uint16_t* dst = final_out ? (uint16_t*)a.out + (int64_t)r * LAT_H * LAT_DV : a.part_o + pi * LAT_H * LAT_DV;
#pragma unroll
  // non-temporal stores: the rows stream out of the die's L2 as they are written
  // (a launch's end writes back what its workgroups left dirty there, and the
  // combine waits for that)
  for (int k = 0; k < LAT_H / NWA; ++k) {
    const int h = wv + NWA * k;
    __builtin_nontemporal_store(*(const u32x4_t*)(kv0 + h * OPITCH + lane * 16),
                                (u32x4_t*)(dst + h * LAT_DV + lane * 8));
  }
}


// ------------------------------------------------------------------ 32 heads per workgroup
// The bf16 attention in half-head units (the kernel above and the fused decode
// step, for launches of few (row, split) units): workgroup (row, split, head half
// hh) covers heads 32hh .. +31 of one (row, split), with the block table, gathers
// and hand-over of the body above.  Per 64-token sub-tile:
//  - S^T: wave w takes tokens 16w .. +15 against all 32 heads with
//    v_mfma_f32_16x16x32_bf16 (each K fragment feeds two 16-head tiles; a lane
//    ends with the 4 tokens of one block for one head of each tile);
//  - softmax as above, with the tile maxima of four token quarters;
//  - O^T[dims, heads] += V^T . P^T: wave w takes dims 128w .. +127 of the 32 heads.
// Each workgroup does half the MFMA work and writes half the partials of a 64-head
// workgroup, and a launch gets twice the workgroups; the two halves of a split
// gather the same rows (numbered rows fastest, they share a die and its L2).
constexpr int QS32 = LAT_DK / 32;              // 18 k-steps of 16x16x32 over the 576 dims
// The 32-head units pay where the (row, split) units are fewer than half the compute
// units: a 1M-token decode row (32 units) attends in 8.5 us against 10.0 us with
// 64-head units; at 128 units (a batch of 8 decode rows) the second gather of each
// split costs more than the halved MFMA work saves (0.4 us per decode step).
constexpr int H32_UNITS = 128;
__device__ __host__ __forceinline__ bool use_h32(const AttnArgs& a) { return a.n_rows * a.n_split < H32_UNITS; }

template <bool STEP>
__device__ __forceinline__ void attn_bf16_h32_body(const AttnArgs& a, const int bid, AttnShared& sh, uint8_t* pmat,
                                                   uint8_t* kv0, uint8_t* kv1) {
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform (scalar)
  const int l32 = lane & 31, lh = lane >> 5, l16 = lane & 15, lq = lane >> 4;
  if (bid >= 2 * a.n_rows * a.n_split) return;
  // rows fastest, then the head half, then the split: split 0 of every row first
  const int rl = bid % a.n_rows;
  const int hh = (bid / a.n_rows) & 1;
  const int split = bid / (2 * a.n_rows);
  const int H0 = 32 * hh;
  const int r = a.row0 + rl;
  const RowCtx c = row_ctx(a, r);
  const int sb0 = split * a.blocks_per_split;
  const int send = min(a.top_k, sb0 + a.blocks_per_split);
  const int nsub = (send - sb0 + 15) >> 4;
  sel::StepLists<NTA, 8> sl;
  if constexpr (STEP)
    sl.start(a.step_lists + (int64_t)rl * a.step_max_lists * sel::LIST, a.step_meta + (int64_t)rl * a.step_max_lists,
             a.step_lists_n);

  BlockIds ids;
  int pid[2][2];
  int32_t* const lid = reinterpret_cast<int32_t*>(pmat);
  auto load_ids = [&]() {
    if constexpr (STEP) {
#pragma unroll
      for (int k = 0; k < MAX_BLOCKS_PER_SPLIT / NTA; ++k) {
        const int i = (int)threadIdx.x + k * NTA;
        ids.blk[k] = sb0 + i < send ? lid[i] : -1;
      }
    } else {
      ids = fetch_blocks<false>(c, sb0, send);
    }
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int bi = sb0 + 16 * n + ((8 * (2 * wv + h) + (lane >> 3)) >> 2);
        pid[n][h] = bi < send ? (STEP ? lid[bi - sb0] : sel_id<false>(c, bi)) : -1;
      }
  };
  if constexpr (!STEP) load_ids();
  {
    // heads H0 .. H0 + 31 of the query row into kv1 in the sub-tile layout, head
    // H0 + t as row t: wave w fills rows 8w .. 8w + 7 of every segment
    const int t = 8 * wv + (lane >> 3);
    const uint8_t* qrow =
        (const uint8_t*)a.q + ((int64_t)r * LAT_H + H0 + t) * (LAT_DK * 2) + 16 * ((lane & 7) ^ kv_swz(t));
#pragma unroll
    for (int g = 0; g < NSEG; ++g)
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(qrow + 128 * g),
                                       (void __attribute__((address_space(3)))*)(kv1 + g * SEGB + wv * 1024), 16, 0,
                                       0);
  }
  NewRow nr{~0u, nullptr};
  if constexpr (STEP) {
    nr = NewRow{(uint32_t)a.L.tok_row(c.b, c.p), a.k_new + (int64_t)c.b * a.k_new_stride};
    __builtin_amdgcn_sched_barrier(0);
    step_select(a, c, rl, split, sb0, send, lid, kv0, sl);
    load_ids();
  }
  __builtin_amdgcn_sched_barrier(0);
  constexpr int NE = MAX_BLOCKS_PER_SPLIT / NTA;
  const int eb[6] = {ids.blk[0], ids.blk[1], pid[0][0], pid[0][1], pid[1][0], pid[1][1]};
  uint32_t ent[6];
  block_entries(a, c, eb, ent);
  const int nbt = ((send - sb0 + 15) >> 4) << 4;
  SubtileSrc src[2];
#pragma unroll
  for (int n = 0; n < 2; ++n)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int t = 8 * (2 * wv + h) + (lane >> 3);
      const uint32_t grow = (ent[2 + 2 * n + h] & ROW_BITS) + (t & 3);
      src[n].row[h] = kv_row_src<STEP>(a, nr, grow, 16 * ((lane & 7) ^ kv_swz(t)));
    }
#pragma unroll
  for (int k = 0; k < KV_LOADS; ++k) load_column(src[0], kv0, k);
#pragma unroll
  for (int k = 0; k < NE; ++k) {
    const int i = (int)threadIdx.x + k * NTA;
    if (i < nbt) lds_st(&sh.brow[i], ent[k]);
  }
  if (threadIdx.x < 4) lds_st(&sh.need[threadIdx.x], 0);
  wait_vm<KV_LOADS>();                           // this wave's part of q landed
  block_sync_lds();
  // q fragments (16x16x32 B operand): head H0 + 16g + l16, dims 32s + 8lq .. +7
  bf16x8_t qf[2][QS32];
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int s = 0; s < QS32; ++s) qf[g][s] = *(const bf16x8_t*)(kv1 + kv_off(16 * g + l16, 4 * s + lq));
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int s = 0; s < QS32; ++s) asm volatile("" : "+a"(qf[g][s]));
  block_sync_lds();                              // every wave has its q: kv1 is free
#pragma unroll
  for (int k = 0; k < KV_LOADS; ++k) load_column(src[1], kv1, k);
  wait_vm<KV_LOADS>();                           // sub-tile 0 landed (this wave's part)
  block_sync_lds();
  const float cs = a.scale * LOG2E;

  // O^T tile [32 dims, 32 heads]: o[db][k] = head H0 + l32, dim 128wv + 32db + 8(k/4)
  // + 4lh + k%4
  f32x16_t o[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) o[d] = f32x16_t{};
  // reference maxima: ms[g] for head H0 + 16g + l16 (S^T layout), mo for head H0 +
  // l32 (O layout); lp[g] this lane's part of l of head 16g + l16
  float ms[2] = {-INFINITY, -INFINITY}, mo = -INFINITY;
  float lp[2] = {0.f, 0.f};
  // tile maxima of the four token quarters: quarter w of local head h at
  // tmax[w >> 1][32 (w & 1) + h]
  auto tmax_at = [&](int w, int h) -> float& { return sh.tmax[w >> 1][32 * (w & 1) + h]; };

  auto step = [&](const int n, const uint8_t* buf, uint8_t* nxt) {
    const bool fetch = n >= 1 && n + 1 < nsub;
    const SubtileSrc fsrc = subtile_src<STEP>(a, sh, fetch ? n + 1 : n, nr);
    // visible tokens of this lane's block (4wv + lq of the sub-tile)
    const int vis = (int)(lds_ld(&sh.brow[16 * n + 4 * wv + lq]) >> VIS_SHIFT);
    // ---- S^T[token, head]: x[g][u] = token 16wv + 4lq + u, head H0 + 16g + l16
    f32x4_t x[2] = {f32x4_t{}, f32x4_t{}};
    {
      constexpr int KPF = 4;
      const int t = 16 * wv + l16;
      bf16x8_t kf[KPF];
#pragma unroll
      for (int p = 0; p < KPF; ++p) kf[p] = *(const bf16x8_t*)(buf + kv_off(t, 4 * p + lq));
#pragma unroll
      for (int s = 0; s < QS32; ++s) {
#pragma unroll
        for (int g = 0; g < 2; ++g) x[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[s % KPF], qf[g][s], x[g], 0, 0, 0);
        if (s + KPF < QS32) kf[s % KPF] = *(const bf16x8_t*)(buf + kv_off(t, 4 * (s + KPF) + lq));
        if (fetch) load_column(fsrc, nxt, s);
      }
    }
    // ---- masking, this quarter's tile maximum of each head (scaled after the
    //      maximum: cs > 0 and rounding is monotonic); P below takes cs S - m as one
    //      fmaf, and the products are __fmul_rn, so no contraction is left to the
    //      compiler
    float tm[2];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
#pragma unroll
      for (int u = 0; u < 4; ++u) x[g][u] = u < vis ? x[g][u] : -INFINITY;
      tm[g] = __fmul_rn(quad_max16(fmaxf(fmaxf(x[g][0], x[g][1]), fmaxf(x[g][2], x[g][3]))), cs);
      if (lq == 0) lds_st(&tmax_at(wv, 16 * g + l16), tm[g]);
    }
    const bool need = __ballot(tm[0] > ms[0] + RESCALE_LOG2 || tm[1] > ms[1] + RESCALE_LOG2) != 0ull;
    if (need && lane == 0) lds_st(&sh.need[wv], 1);
    // P against the current references (recomputed below in the rare case)
    float ls[2];
    auto write_p = [&]() {
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const float nmu = ms[g] == -INFINITY ? 0.f : -ms[g];
        float pv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) pv[u] = exp2f(fmaf(x[g][u], cs, nmu));
        ls[g] = (pv[0] + pv[1]) + (pv[2] + pv[3]);
        lds_st((uint2*)(pmat + (16 * g + l16) * PROW + (16 * wv + 4 * lq) * 2),
               make_uint2(pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3])));
      }
    };
    write_p();
    block_sync_lds();
    // ---- rare: some head maximum passed its reference by more than 2^8.  Every
    //      wave moves the references to the new maxima, rescales what it holds,
    //      and P is rewritten.
    bool moved = false;
#pragma unroll
    for (int w = 0; w < 4; ++w) moved |= lds_ld(&sh.need[w]) != 0;
    if (moved) {
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const int h = 16 * g + l16;
        const float msn = fmaxf(fmaxf(ms[g], fmaxf(lds_ld(&tmax_at(0, h)), lds_ld(&tmax_at(1, h)))),
                                fmaxf(lds_ld(&tmax_at(2, h)), lds_ld(&tmax_at(3, h))));
        lp[g] = __fmul_rn(lp[g], ms[g] == -INFINITY ? 0.f : exp2f(ms[g] - msn));
        ms[g] = msn;
      }
      write_p();
      {
        const float mon = fmaxf(fmaxf(mo, fmaxf(lds_ld(&tmax_at(0, l32)), lds_ld(&tmax_at(1, l32)))),
                                fmaxf(lds_ld(&tmax_at(2, l32)), lds_ld(&tmax_at(3, l32))));
        const float al = mo == -INFINITY ? 0.f : exp2f(mo - mon);
        mo = mon;
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
          for (int k = 0; k < 16; ++k) o[d][k] = __fmul_rn(o[d][k], al);
      }
      block_sync_lds();                          // new P complete; flags read by all
      if (threadIdx.x < 4) lds_st(&sh.need[threadIdx.x], 0);
    }
    lp[0] += ls[0];
    lp[1] += ls[1];
    // ---- O^T += V^T . P^T: dims 128wv + 32db, the 32 heads, tokens 16ks .. +15
    {
      typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;
      // transposed V reads as in attn_bf16_body: lane l receives dim l32 of tokens
      // 16ks + 8lh + j
      const int g4 = lane >> 4, s16 = lane & 15;
      const int vt = 8 * (g4 >> 1) + (s16 >> 2);
      const int vd = 16 * (g4 & 1) + 4 * (s16 & 3);
      const int vch = vd >> 3, vin = (vd & 7) * 2;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8_t pb = lds_ld((const bf16x8_t*)(pmat + l32 * PROW + (16 * ks + 8 * lh) * 2));
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const int ch = 4 * (4 * wv + db) + vch;
          const int t0 = 16 * ks + vt;
          const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(buf + kv_off(t0, ch) + vin));
          const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(buf + kv_off(t0 + 4, ch) + vin));
          const s16x4_t v8[2] = {lo, hi};
          const bf16x8_t va = __builtin_bit_cast(bf16x8_t, v8);
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, o[db], 0, 0, 0);
        }
      }
    }
    // sub-tile n+1 landed and every wave done with `buf` and P past this barrier
    wait_vm<0>();
    if (n + 1 < nsub) block_sync_lds();
  };
  for (int n = 0; n < nsub; n += 2) {
    step(n, kv0, kv1);
    if (n + 1 < nsub) step(n + 1, kv1, kv0);
  }

  // ---- epilogue: l of each head = sum over its 4 lanes and the 4 token quarters
  //      (lpart reused as [quarter][head] like tmax)
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const float lw = quad_sum16(lp[g]);
    if (lq == 0) lds_st(&sh.lpart[wv >> 1][32 * (wv & 1) + 16 * g + l16], lw);
  }
  block_sync_lds();                              // also: every wave is done with kv0 / kv1
  auto l_total = [&](int h) {
    return (lds_ld(&sh.lpart[0][h]) + lds_ld(&sh.lpart[0][32 + h])) +
           (lds_ld(&sh.lpart[1][h]) + lds_ld(&sh.lpart[1][32 + h]));
  };
  const bool final_out = a.n_split == 1;
  const int64_t pi = (int64_t)rl * a.n_split + split;
  constexpr int OPITCH = LAT_DV * 2 + 16;
  {
    const float sc = final_out ? 1.f / l_total(l32) : 1.f;
    uint8_t* row = kv0 + l32 * OPITCH + (128 * wv + 4 * lh) * 2;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *(uint2*)(row + (32 * d + 8 * q) * 2) =
            make_uint2(pack_bf16x2(__fmul_rn(o[d][4 * q], sc), __fmul_rn(o[d][4 * q + 1], sc)),
                       pack_bf16x2(__fmul_rn(o[d][4 * q + 2], sc), __fmul_rn(o[d][4 * q + 3], sc)));
  }
  if (wv == 0 && lq == 0) {
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int h = 16 * g + l16;
      const float lt = l_total(h);
      const float mm = ms[g] == -INFINITY ? 0.f : ms[g];
      if (final_out) {
        if (a.lse) a.lse[(int64_t)r * LAT_H + H0 + h] = (mm + log2f(lt)) * LN2;
      } else {
        a.part_ml[(pi * LAT_H + H0 + h) * 2] = mm;
        a.part_ml[(pi * LAT_H + H0 + h) * 2 + 1] = lt;
      }
    }
  }
  block_sync_lds();
  uint16_t* dst = final_out ? (uint16_t*)a.out + (int64_t)r * LAT_H * LAT_DV : a.part_o + pi * LAT_H * LAT_DV;
#pragma unroll
  // plain stores: a launch of few units leaves little to write back at its end,
  // and the combine then reads the partials from the last-level cache (streamed,
  // the 1M-token row's combine measured 7.3 against 5.3 us)
  for (int k = 0; k < 32 / NWA; ++k) {
    const int h = wv + NWA * k;
    *(u32x4_t*)(dst + (H0 + h) * LAT_DV + lane * 8) = *(const u32x4_t*)(kv0 + h * OPITCH + lane * 16);
  }
}

static_assert(scorek::score_smem<STEP_NWV, true>() <= KVBUF, "the scoring state fits a sub-tile buffer");

}  // namespace
}  // namespace ip
