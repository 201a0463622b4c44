// Sparse attention kernels and their launchers: the bf16 latent kernel (the bodies
// are in attn_bf16.hpp), the fused decode step with 64-head units, the fp8 latent
// tier, the split combine and the f32 path.  G2C Brief "GLM-5.3-Flash: hybrid
// attention becomes the product", section "DSA keeps selected global access in
// eleven layers".
#include "attn_bf16.hpp"

namespace ip {

namespace {

template <bool H32>
__global__ __launch_bounds__(NTA, 1) void attn_bf16_kernel(AttnArgs a) {
  __shared__ AttnShared sh;
  __shared__ __align__(16) uint8_t pmat[LAT_H * PROW];   // P[head][token] bf16
  __shared__ __align__(16) uint8_t kv0[KVBUF];
  __shared__ __align__(16) uint8_t kv1[KVBUF];
  if constexpr (H32)
    attn_bf16_h32_body<false>(a, blockIdx.x, sh, pmat, kv0, kv1);
  else
    attn_bf16_body<false>(a, blockIdx.x, sh, pmat, kv0, kv1);
}

// ------------------------------------------------------------------ fused decode step
// One launch for the decode step: workgroups [0, n_score) score (and list) the
// rows, [n_score, n_score + n_app) append the new tokens, and the rest run the
// attention of one (row, split) each, selecting the row's ids first (step_select).  Workgroups start in
// index order, so every attention workgroup waits only on workgroups that have
// started before it and never wait themselves: the wait ends.  The attention
// workgroups take their compute units as the scoring ones finish and fetch their
// query while the rows are being selected.  The scoring state lives in the first
// sub-tile buffer.

__global__ __launch_bounds__(NTA, 1) void decode_step_kernel(StepKArgs A) {
  __shared__ AttnShared sh;
  __shared__ __align__(16) uint8_t pmat[LAT_H * PROW];
  __shared__ __align__(16) uint8_t kv0[KVBUF];
  __shared__ __align__(16) uint8_t kv1[KVBUF];
  __shared__ int last_here;
  const int L = blockIdx.x;
  IP_STAMP(L, ST_START);
  if (L < A.n_score + A.n_app) {
    scorek::score_fp8_body<1, STEP_NWV, true, STEP_TILES>(A.s, L % A.gx, L / A.gx, A.gx, kv0, last_here,
                                                           A.at.sel_ready);
#ifdef IP_PHASE_STAMPS
    __builtin_amdgcn_s_waitcnt(0);               // its stores acknowledged
#endif
    IP_STAMP(L, ST_SCORED);
    return;
  }
  attn_bf16_body<true>(A.at, L - A.n_score - A.n_app, sh, pmat, kv0, kv1);
#ifdef IP_PHASE_STAMPS
  __builtin_amdgcn_s_waitcnt(0);                 // its partials acknowledged
#endif
  IP_STAMP(L, ST_END);
}

// ------------------------------------------------------------------ fp8 latent tier
// Latent rows stored as e4m3fn codes (576 bytes) with one fp32 scale per token;
// K_t = sigma_t dec(code_t), V_t its first 512 dims.  Same work split and softmax
// as the bf16 kernel; what changes:
//  - a sub-tile buffer holds 64 rows of codes in 5 segments of the same layout
//    (segment 4 = bytes 512 .. 575; its DMA reads those 64 bytes twice, so that
//    every slot is filled from inside the row) and the 64 scales of the sub-tile
//    arrive by one dword DMA issued by wave 0;
//  - K fragments: one 16-byte read gives the codes of two k-steps, widened to bf16
//    in registers (exact); q comes from global memory in the matching dim order
//    (k-step 2p: dims 32p + 16lh .. +7, k-step 2p+1: the next 8);
//  - S is multiplied by sigma_t per token (fp32), P carries sigma_t (P_t sigma_t in
//    bf16) while l sums the unscaled P;
//  - at the start of a step the 512 V dims of the sub-tile's codes are widened
//    into a bf16 copy in the bf16 layout, and O += V^T P^T runs as in the bf16
//    kernel.
constexpr int NSEG8 = 5;
constexpr int KVBUF8 = NSEG8 * SEGB;             // 40960 bytes
constexpr int KV_LOADS8 = NSEG8 * 8 / NWA;       // 10 per wave
constexpr int KPAIRS = LAT_DK / 32;              // 18 fragments of 16 codes (two k-steps)
constexpr int VCH8 = LAT_DV / 16;                // 32 16-byte chunks of V codes per row

struct SubtileSrc8 {
  const uint8_t* row[2];
  int cofs[2];                                   // byte of this lane's slot within a 128-byte piece
};

__device__ __forceinline__ SubtileSrc8 src8_from_rows(const AttnArgs& a, const uint32_t (&grow)[2]) {
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  SubtileSrc8 src;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int t = 8 * (2 * wv + h) + (lane >> 3);
    src.row[h] = a.k + (uint64_t)grow[h] * a.k_stride;
    src.cofs[h] = 16 * ((lane & 7) ^ kv_swz(t));
  }
  return src;
}

__device__ __forceinline__ SubtileSrc8 subtile_src8(const AttnArgs& a, const AttnShared& sh, int n) {
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint32_t e[2], grow[2];
  subtile_entries(sh, n, e);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int t = 8 * (2 * wv + h) + (lane >> 3);
    grow[h] = (e[h] & ROW_BITS) + (t & 3);
  }
  return src8_from_rows(a, grow);
}

// load k (0..9): segment k/2 of row half k%2
__device__ __forceinline__ void load_column8(const SubtileSrc8& src, uint8_t* buf, int k) {
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = k >> 1, h = k & 1;
  const int off = g < 4 ? 128 * g + src.cofs[h] : 512 + (src.cofs[h] & 48);
  __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(src.row[h] + off),
                                   (void __attribute__((address_space(3)))*)(buf + g * SEGB + (2 * wv + h) * 1024),
                                   16, 0, 0);
}

// the scales of the sub-tile's 64 tokens: lane l brings that of token l
__device__ __forceinline__ void load_scales(const float* src, float* sg) {
  __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)src,
                                   (void __attribute__((address_space(3)))*)sg, 4, 0, 0);
}

__device__ __forceinline__ const float* scale_src(const AttnArgs& a, const AttnShared& sh, int n) {
  const int lane = threadIdx.x & 63;
  return a.k_scale + (lds_ld(&sh.brow[n * 16 + (lane >> 2)]) & ROW_BITS) + (lane & 3);
}

__global__ __launch_bounds__(NTA, 1) void attn_fp8_kernel(AttnArgs a) {
  __shared__ AttnShared sh;
  __shared__ __align__(16) uint8_t pmat[LAT_H * PROW];   // P[head][token] bf16
  __shared__ __align__(16) uint8_t kv0[KVBUF8];
  __shared__ __align__(16) uint8_t kv1[KVBUF8];
  __shared__ __align__(16) uint8_t vb[LAT_DV / 64 * SEGB];   // bf16 V of the current sub-tile
  __shared__ __align__(16) float sg0[SUBT];
  __shared__ __align__(16) float sg1[SUBT];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, lh = lane >> 5;
  const int hb = wv & 1, th = wv >> 1;
  const int bid = blockIdx.x;
  if (bid >= a.n_rows * a.n_split) return;
  const int split = bid % a.n_split;
  const int rl = bid / a.n_split;
  const int r = a.row0 + rl;
  const RowCtx c = row_ctx(a, r);
  const int sb0 = split * a.blocks_per_split;
  const int send = min(a.top_k, sb0 + a.blocks_per_split);
  const int nsub = (send - sb0 + 15) >> 4;
  const int hs = 32 * hb + l32;

  // prologue: the ids (block table entries, this lane's rows of sub-tiles 0 and 1,
  // the tokens whose scales it brings); the query row by LDS DMA in whole 128-byte
  // lines, dims 0..511 into vb and 512..575 into pmat (both free until step 0),
  // head h as row h in the sub-tile layout; sub-tiles 0 and 1 with their scales;
  // then q into registers.
  const BlockIds ids = fetch_blocks<false>(c, sb0, send);
  int pid[2][2], sid[2];
#pragma unroll
  for (int n = 0; n < 2; ++n) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int bi = sb0 + 16 * n + ((8 * (2 * wv + h) + (lane >> 3)) >> 2);
      pid[n][h] = bi < send ? c.sel[bi] : -1;
    }
    const int bi = sb0 + 16 * n + (lane >> 2);
    sid[n] = bi < send ? c.sel[bi] : -1;
  }
  {
    SubtileSrc qsrc;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int t = 8 * (2 * wv + h) + (lane >> 3);
      qsrc.row[h] = (const uint8_t*)a.q + ((int64_t)r * LAT_H + t) * (LAT_DK * 2) + 16 * ((lane & 7) ^ kv_swz(t));
    }
#pragma unroll
    for (int k = 0; k < KV_LOADS; ++k) {
      const int g = k >> 1, h = k & 1;
      uint8_t* dst = (g < 8 ? vb + g * SEGB : pmat) + (2 * wv + h) * 1024;
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(qsrc.row[h] + 128 * g),
                                       (void __attribute__((address_space(3)))*)dst, 16, 0, 0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // entries: [0, 1] this thread's block-table entries, [2 + 2n + h] its source
  // rows of sub-tile n, [6 + n] the token whose scale it brings
  constexpr int NE = MAX_BLOCKS_PER_SPLIT / NTA;
  static_assert(NE == 2, "two block-table entries per thread");
  const int eb[8] = {ids.blk[0], ids.blk[1], pid[0][0], pid[0][1], pid[1][0], pid[1][1], sid[0], sid[1]};
  uint32_t ent[8];
  block_entries(a, c, eb, ent);
  const int nbt = ((send - sb0 + 15) >> 4) << 4;
  SubtileSrc8 src[2];
  const float* ssrc[2];
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    uint32_t grow[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int t = 8 * (2 * wv + h) + (lane >> 3);
      grow[h] = (ent[2 + 2 * n + h] & ROW_BITS) + (t & 3);
    }
    src[n] = src8_from_rows(a, grow);
    ssrc[n] = a.k_scale + (ent[6 + n] & ROW_BITS) + (lane & 3);
  }
  // sub-tiles 0 and 1 with their scales, unconditionally (past the split the
  // rows are the query's own block), so that every wave has the same loads in
  // flight on every path; all four waves bring the same scales
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    load_scales(ssrc[n], n ? sg1 : sg0);
#pragma unroll
    for (int k = 0; k < KV_LOADS8; ++k) load_column8(src[n], n ? kv1 : kv0, k);
  }
#pragma unroll
  for (int k = 0; k < NE; ++k) {
    const int i = (int)threadIdx.x + k * NTA;
    if (i < nbt) lds_st(&sh.brow[i], ent[k]);
  }
  if (threadIdx.x < 4) lds_st(&sh.need[threadIdx.x], 0);
  wait_vm<2 * (KV_LOADS8 + 1)>();                // the query landed
  block_sync_lds();
  // q fragments of head hs: qf[2p] = dims 32p + 16lh .. +7 (bf16 chunk 4p + 2lh of
  // the row), qf[2p+1] = the next 8
  bf16x8_t qf[2 * KPAIRS];
#pragma unroll
  for (int p = 0; p < KPAIRS; ++p)
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int ch = 4 * p + 2 * lh + e;
      qf[2 * p + e] = p < 16 ? lds_ld((const bf16x8_t*)(vb + kv_off(hs, ch)))
                             : lds_ld((const bf16x8_t*)(pmat + hs * 128 + 16 * ((ch & 7) ^ kv_swz(hs))));
    }
#pragma unroll
  for (int s = 0; s < 2 * KPAIRS; ++s) asm volatile("" : "+a"(qf[s]));
  wait_vm<KV_LOADS8 + 1>();                      // sub-tile 0 landed
  block_sync_lds();                              // and every wave has its q: vb, pmat free
  const float cs = a.scale * LOG2E;

  f32x16_t o[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int d = 0; d < 4; ++d) o[i][d] = f32x16_t{};
  float ms = -INFINITY, mo[2] = {-INFINITY, -INFINITY};
  float l_half = 0.f;

  auto step = [&](const int n, const uint8_t* buf, const float* sgb, uint8_t* nxt, float* sgn) {
    const bool fetch = n >= 1 && n + 1 < nsub;
    const SubtileSrc8 fsrc = subtile_src8(a, sh, fetch ? n + 1 : n);
    const float* fssrc = scale_src(a, sh, fetch ? n + 1 : n);
    const u32x4_t bv0 = lds_ld((const u32x4_t*)&sh.brow[n * 16 + 8 * th]);
    const u32x4_t bv1 = lds_ld((const u32x4_t*)&sh.brow[n * 16 + 8 * th + 4]);
    // ---- S^T[token, head] over the codes, as in the bf16 kernel with fragments of
    //      two k-steps.  In between: sub-tile n+1 is fetched, and the V codes of
    //      this sub-tile are widened into vb (bf16 layout; lane l takes token l,
    //      chunks wv + 4i of its 32 16-code chunks: read at pair 2i, written at 2i+1)
    f32x16_t sacc;
    {
      f32x16_t sa[2] = {f32x16_t{}, f32x16_t{}};
      const int t = 32 * th + l32;
      constexpr int KPF = 3;
      u32x4_t kr[KPF];
#pragma unroll
      for (int p = 0; p < KPF; ++p) kr[p] = *(const u32x4_t*)(buf + kv_off(t, 2 * p + lh));
      if (fetch) load_scales(fssrc, sgn);
      // the widening's LDS offsets: kv_off(l, wv + 4i) = dro[i & 1] + SEGB (i / 2) and
      // kv_off(l, 2(wv + 4i) + e) = dwo[e] + SEGB i.  In these address forms (and
      // with the stores through lds_st) the compiler can tell the widening and the
      // PV reads below from the DMA in flight; checked in the generated code, where
      // the only vmcnt waits in the loop are the end-of-step ones.
      const int dro[2] = {kv_off(lane, wv), kv_off(lane, wv + 4)};
      const int dwo[2] = {kv_off(lane, 2 * wv), kv_off(lane, 2 * wv + 1)};
      u32x4_t dq;
#pragma unroll
      for (int p = 0; p < KPAIRS; ++p) {
        const u32x4_t w = kr[p % KPF];
        if (p + KPF < KPAIRS) kr[p % KPF] = *(const u32x4_t*)(buf + kv_off(t, 2 * (p + KPF) + lh));
        sa[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fp8x8_to_bf16x8_pk(w[0], w[1]), qf[2 * p], sa[0], 0, 0, 0);
        sa[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fp8x8_to_bf16x8_pk(w[2], w[3]), qf[2 * p + 1], sa[1], 0, 0, 0);
#pragma unroll
        for (int k = 0; k < KV_LOADS8; ++k)
          if ((KPAIRS * k) / KV_LOADS8 == p && fetch) load_column8(fsrc, nxt, k);
        if (p < 2 * (VCH8 / NWA)) {
          const int i = p >> 1;
          if ((p & 1) == 0) {
            dq = *(const u32x4_t*)(buf + (dro[i & 1] + SEGB * (i >> 1)));
          } else {
            lds_st((bf16x8_t*)(vb + (dwo[0] + SEGB * i)), fp8x8_to_bf16x8_pk(dq[0], dq[1]));
            lds_st((bf16x8_t*)(vb + (dwo[1] + SEGB * i)), fp8x8_to_bf16x8_pk(dq[2], dq[3]));
          }
        }
      }
      sacc = sa[0] + sa[1];
    }
    // ---- per-token scales, masking, this half's tile maximum of head hs
    f32x4v sgv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) sgv[q] = *(const f32x4v*)(sgb + 32 * th + 8 * q + 4 * lh);
    float tm = -INFINITY;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t e = q < 2 ? (lh ? bv0[2 * q + 1] : bv0[2 * q]) : (lh ? bv1[2 * q - 3] : bv1[2 * q - 4]);
      const int vis = (int)(e >> VIS_SHIFT);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        sacc[4 * q + u] = u < vis ? sacc[4 * q + u] * (cs * sgv[q][u]) : -INFINITY;
        tm = fmaxf(tm, sacc[4 * q + u]);
      }
    }
    tm = pair_max32(tm);
    if (lh == 0) lds_st(&sh.tmax[th][hs], tm);
    const bool need = __ballot(tm > ms + RESCALE_LOG2) != 0ull;
    if (need && lane == 0) lds_st(&sh.need[wv], 1);
    auto write_p = [&](float m) {
      const float mu = m == -INFINITY ? 0.f : m;
      float ls = 0.f;
      uint8_t* pr = pmat + hs * PROW + (32 * th + 4 * lh) * 2;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float pv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) { pv[u] = exp2f(sacc[4 * q + u] - mu); ls += pv[u]; }
        lds_st((uint2*)(pr + 16 * q), make_uint2(pack_bf16x2(pv[0] * sgv[q][0], pv[1] * sgv[q][1]),
                                                 pack_bf16x2(pv[2] * sgv[q][2], pv[3] * sgv[q][3])));
      }
      return ls;
    };
    float ls = write_p(ms);
    block_sync_lds();
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
      block_sync_lds();
      if (threadIdx.x < 4) lds_st(&sh.need[threadIdx.x], 0);
    }
    l_half += pair_sum32(ls);
    // ---- O^T += V^T . P^T over the widened V, as in the bf16 kernel
    {
      typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;
      const int g4 = lane >> 4, s16 = lane & 15;
      const int vt = 8 * (g4 >> 1) + (s16 >> 2);
      const int vd = 16 * (g4 & 1) + 4 * (s16 & 3);
      const int vch = vd >> 3, vin = (vd & 7) * 2;
      // kv_off(16ks + vt (+4), 4(4wv + db) + vch) + vin = vofs[+4][db & 1] + 2048ks +
      // SEGB (db / 2): one lane offset per (token half, db parity), the rest constant.
      // Addresses formed as vb + one offset keep the LDS object visible to the
      // compiler, which then knows these reads do not touch the buffer in flight.
      int vofs[2][2];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int par = 0; par < 2; ++par) vofs[hf][par] = kv_off(vt + 4 * hf, 16 * wv + 4 * par + vch) + vin;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        bf16x8_t pb[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) pb[i] = lds_ld((const bf16x8_t*)(pmat + (32 * i + l32) * PROW + (16 * ks + 8 * lh) * 2));
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const int cofs = 2048 * ks + SEGB * (db >> 1);
          const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb + (vofs[0][db & 1] + cofs)));
          const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb + (vofs[1][db & 1] + cofs)));
          const s16x4_t v8[2] = {lo, hi};
          const bf16x8_t va = __builtin_bit_cast(bf16x8_t, v8);
#pragma unroll
          for (int i = 0; i < 2; ++i) o[i][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[i], o[i][db], 0, 0, 0);
        }
      }
    }
    // ---- sub-tile n+1 (codes and scales) has landed, and every wave is done with
    //      `buf`, vb and P, past this barrier (the wait unconditional, as above)
    wait_vm<0>();
    if (n + 1 < nsub) block_sync_lds();
  };
  for (int n = 0; n < nsub; n += 2) {
    step(n, kv0, sg0, kv1, sg1);
    if (n + 1 < nsub) step(n + 1, kv1, sg1, kv0, sg0);
  }

  // ---- epilogue as in the bf16 kernel; heads 0..31 go through kv0, 32..63 kv1
  //      (with one sub-tile, sub-tile 1's unused loads into kv1 land first)
  if (lh == 0) lds_st(&sh.lpart[th][hs], l_half);
  wait_vm<0>();
  block_sync_lds();
  const bool final_out = a.n_split == 1;
  const int64_t pi = (int64_t)rl * a.n_split + split;
  constexpr int OPITCH = LAT_DV * 2 + 16;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int h = 32 * i + l32;
    const float sc = final_out ? 1.f / (lds_ld(&sh.lpart[0][h]) + lds_ld(&sh.lpart[1][h])) : 1.f;
    uint8_t* row = (i == 0 ? kv0 : kv1) + l32 * OPITCH + (128 * wv + 4 * lh) * 2;
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
  for (int k = 0; k < LAT_H / NWA; ++k) {
    const int h = wv + NWA * k;
    const uint8_t* srow = (k < LAT_H / NWA / 2 ? kv0 + h * OPITCH : kv1 + (h - 32) * OPITCH) + lane * 16;
    *(u32x4_t*)(dst + h * LAT_DV + lane * 8) = *(const u32x4_t*)srow;
  }
}

// Merge split partials: per (row, head) O = sum_s 2^(m_s - m) O_s / sum_s 2^(m_s - m) l_s.
// Two heads per workgroup, 128 threads x 4 dims per head; the split weights are
// computed once per wave (lane s holds split s) and broadcast.
constexpr int MAX_SPLIT = 64;
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  // rows fastest (a row's workgroups share a die, as the fused step's attention)
  IP_STAMP(STAMP_STEP_ROWS + (int)blockIdx.x, ST_C_START);
  const int head = (int)(blockIdx.x / a.n_rows) * 2 + (threadIdx.x >> 7);
  const int rl = (int)(blockIdx.x % a.n_rows);
  const int r = a.row0 + rl;
  const int t = threadIdx.x & 127, lane = threadIdx.x & 63;
  const int S = a.n_split;
  const int64_t pi0 = (int64_t)rl * S;
  float ms = -INFINITY, ls = 0.f;
  if (lane < S) {
    const float2 ml = *(const float2*)&a.part_ml[((pi0 + lane) * LAT_H + head) * 2];
    ms = ml.x;
    ls = ml.y;
  }
  const uint16_t* base = a.part_o + (pi0 * LAT_H + head) * LAT_DV + t * 4;
  // up to CMB_REG splits: every partial load is issued at once, beside the weights'
  constexpr int CMB_REG = 16;
  uint2 v[CMB_REG];
  if (S <= CMB_REG) {
#pragma unroll
    for (int u = 0; u < CMB_REG; ++u)
      v[u] = u < S ? *(const uint2*)(base + (int64_t)u * LAT_H * LAT_DV) : make_uint2(0u, 0u);
  }
  float m = ms;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  const float wgt = (lane < S && ms != -INFINITY) ? exp2f(ms - m) : 0.f;
  float L = wgt * ls;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) L += __shfl_xor(L, o);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  auto add = [&](float wu, uint2 v) {
    acc.x = fmaf(wu, __uint_as_float(v.x << 16), acc.x);
    acc.y = fmaf(wu, __uint_as_float(v.x & 0xFFFF0000u), acc.y);
    acc.z = fmaf(wu, __uint_as_float(v.y << 16), acc.z);
    acc.w = fmaf(wu, __uint_as_float(v.y & 0xFFFF0000u), acc.w);
  };
  if (S <= CMB_REG) {
#pragma unroll
    for (int u = 0; u < CMB_REG; ++u)
      if (u < S) add(__shfl(wgt, u), v[u]);
  } else {
    int s = 0;
    for (; s + 4 <= S; s += 4) {
      uint2 w[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) w[u] = *(const uint2*)(base + (int64_t)(s + u) * LAT_H * LAT_DV);
#pragma unroll
      for (int u = 0; u < 4; ++u) add(__shfl(wgt, s + u), w[u]);
    }
    for (; s < S; ++s) add(__shfl(wgt, s), *(const uint2*)(base + (int64_t)s * LAT_H * LAT_DV));
  }
  // the fused step's words and lists of the row return to zero for the next launch
  // (every reader of them belongs to the step launch, which has ended); this
  // kernel's stores are non-temporal, so little is left to write back at its end
  if (a.sel_ready && blockIdx.x < (unsigned)a.n_rows && threadIdx.x == 0) {
    a.sel_ready[rl] = 0u;
  }
  if (a.step_lists) {
    const int g = (int)(blockIdx.x / a.n_rows) * 256 + threadIdx.x, G = LAT_H / 2 * 256;
    u32x4_t* l16 = (u32x4_t*)(a.step_lists + (int64_t)rl * a.step_max_lists * sel::LIST);
    for (int i = g; i < a.step_max_lists * sel::LIST / 2; i += G) __builtin_nontemporal_store(u32x4_t{0u, 0u, 0u, 0u}, l16 + i);
    uint2* m = a.step_meta + (int64_t)rl * a.step_max_lists;
    for (int i = g; i < a.step_max_lists; i += G) __builtin_nontemporal_store((uint64_t)0, (uint64_t*)(m + i));
  }
  const float inv = 1.f / L;
  uint16_t* out = (uint16_t*)a.out + ((int64_t)r * LAT_H + head) * LAT_DV + t * 4;
  __builtin_nontemporal_store((uint64_t)pack_bf16x2(acc.x * inv, acc.y * inv) |
                                  ((uint64_t)pack_bf16x2(acc.z * inv, acc.w * inv) << 32), (uint64_t*)out);
  if (a.lse && t == 0) a.lse[(int64_t)r * LAT_H + head] = (m + log2f(L)) * LN2;
#ifdef IP_PHASE_STAMPS
  __builtin_amdgcn_s_waitcnt(0);
#endif
  IP_STAMP(STAMP_STEP_ROWS + (int)blockIdx.x, ST_C_END);
}

// ------------------------------------------------------------------ f32 path
// Small geometries (n_heads <= 16, dk, dv <= 128, multiples of 4): one workgroup
// per query row, the selected tokens in tiles of 256.  Thread t scores token t of
// the tile for every head (its K row in registers, q broadcast from LDS).  Wave w
// owns heads w, w+4, w+8, w+12 for the online softmax and for O, where lane l
// accumulates dims l and l+64 from coalesced V row reads.  Masked tokens (t > p,
// or a -1 entry) point at the query's own row, so every load is unconditional and
// in bounds; their probability is exactly 0.
constexpr int F_MAXH = 16, F_MAXD = 128, F_TILE = 256, F_HPW = F_MAXH / 4;
__global__ __launch_bounds__(NT) void attn_f32_kernel(AttnArgs a) {
  __shared__ __align__(16) float qs[F_MAXH * F_MAXD];
  __shared__ float ps[F_MAXH][F_TILE];
  __shared__ int64_t rows[F_TILE];
  __shared__ __align__(16) float vs[F_TILE / 2][F_MAXD + 4];   // V rows of half a tile
  const int r = a.row0 + blockIdx.x;
  const RowCtx c = row_ctx(a, r);
  const int H = a.heads, dk = a.dk, dv = a.dv, dk4 = dk >> 2;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const float* q = (const float*)a.q + (int64_t)r * H * dk;
  const float qscale = a.scale * LOG2E;            // logits in base 2
  for (int i = threadIdx.x; i < H * dk; i += NT) qs[i] = q[i] * qscale;
  const int64_t own_row = a.L.tok_row(c.b, c.p);
  float m_run[F_HPW], l_run[F_HPW], acc[F_HPW][2];
#pragma unroll
  for (int i = 0; i < F_HPW; ++i) { m_run[i] = -INFINITY; l_run[i] = 0.f; acc[i][0] = acc[i][1] = 0.f; }
  const int d0 = min(lane, dv - 1), d1 = min(lane + 64, dv - 1);
  const int ntok = a.top_k * 4;
  for (int t0 = 0; t0 < ntok; t0 += F_TILE) {
    const int tt = t0 + threadIdx.x;
    int t = -1;
    if (tt < ntok) {
      const int blk = c.sel[tt >> 2];
      if (blk >= 0 && blk * 4 + (tt & 3) <= c.p) t = blk * 4 + (tt & 3);
    }
    const int64_t row = t >= 0 ? a.L.tok_row(c.b, t) : own_row;
    const float4* kr = (const float4*)(a.k + row * a.k_stride);
    float4 kv[F_MAXD / 4];
#pragma unroll
    for (int e = 0; e < F_MAXD / 4; ++e) kv[e] = kr[min(e, dk4 - 1)];
    __syncthreads();                               // q staged; last tile's reads done
    rows[threadIdx.x] = row;
    for (int h = 0; h < H; ++h) {
      const float4* qh = (const float4*)(qs + h * dk);
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < F_MAXD / 4; ++e) {
        if (e < dk4) {
          const float4 qv = qh[e];
          d = fmaf(qv.x, kv[e].x, d);
          d = fmaf(qv.y, kv[e].y, d);
          d = fmaf(qv.z, kv[e].z, d);
          d = fmaf(qv.w, kv[e].w, d);
        }
      }
      ps[h][threadIdx.x] = t >= 0 ? d : -INFINITY;
    }
    __syncthreads();
    // online softmax over the tile for this wave's heads
#pragma unroll
    for (int i = 0; i < F_HPW; ++i) {
      const int h = wv + 4 * i;
      if (h < H) {
        float sv[F_TILE / 64];
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < F_TILE / 64; ++j) { sv[j] = ps[h][lane + 64 * j]; mx = fmaxf(mx, sv[j]); }
        mx = wave_max(mx);
        const float mn = fmaxf(m_run[i], mx);
        const float mu = mn == -INFINITY ? 0.f : mn;
        const float al = exp2f(m_run[i] - mu);
        float sum = 0.f;
#pragma unroll
        for (int j = 0; j < F_TILE / 64; ++j) {
          const float pv = exp2f(sv[j] - mu);
          ps[h][lane + 64 * j] = pv;
          sum += pv;
        }
        l_run[i] = al * l_run[i] + wave_sum_f(sum);
        m_run[i] = mn;
        acc[i][0] *= al;
        acc[i][1] *= al;
      }
    }
    // O += P V over the tile.  V rows are staged through LDS half a tile at a time
    // (every row load of a half is in flight at once; rows F_MAXD + 4 floats apart)
    const int dv4 = dv >> 2;
    for (int hf = 0; hf < 2; ++hf) {
      __syncthreads();                             // P written / previous half read
      for (int i = threadIdx.x; i < (F_TILE / 2) * dv4; i += NT) {
        const int k = i / dv4, ch = i - k * dv4;
        *(float4*)&vs[k][4 * ch] = ((const float4*)(a.v + rows[hf * (F_TILE / 2) + k] * a.v_stride))[ch];
      }
      __syncthreads();
#pragma unroll 4
      for (int k = 0; k < F_TILE / 2; ++k) {
        const float v0 = vs[k][d0], v1 = vs[k][d1];
#pragma unroll
        for (int i = 0; i < F_HPW; ++i) {
          const int h = min(wv + 4 * i, H - 1);
          const float pk = ps[h][hf * (F_TILE / 2) + k];
          acc[i][0] = fmaf(pk, v0, acc[i][0]);
          acc[i][1] = fmaf(pk, v1, acc[i][1]);
        }
      }
    }
  }
  float* out = (float*)a.out + (int64_t)r * H * dv;
#pragma unroll
  for (int i = 0; i < F_HPW; ++i) {
    const int h = wv + 4 * i;
    if (h < H) {
      const float inv = 1.f / l_run[i];
      if (lane < dv) out[h * dv + lane] = acc[i][0] * inv;
      if (lane + 64 < dv) out[h * dv + lane + 64] = acc[i][1] * inv;
      if (a.lse && lane == 0) a.lse[(int64_t)r * H + h] = (m_run[i] + log2f(l_run[i])) * LN2;
    }
  }
}

}  // namespace

// the phase stamps of the last decode step (a library built with IP_PHASE_STAMPS)
bool phase_stamps(void* host, size_t bytes) {
#ifdef IP_PHASE_STAMPS
  if (bytes > sizeof(ip_phase_stamp_rows)) bytes = sizeof(ip_phase_stamp_rows);
  return hipMemcpyFromSymbol(host, HIP_SYMBOL(ip_phase_stamp_rows), bytes, 0, hipMemcpyDeviceToHost) == hipSuccess;
#else
  (void)host;
  (void)bytes;
  return false;
#endif
}

hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t s) {
  if (a.n_rows <= 0) return hipSuccess;
  // (row, split) units, or (row, split, head half) units of the 32-head body
  const dim3 grid((unsigned)((use_h32(a) ? 2 : 1) * (int64_t)a.n_rows * a.n_split));
  // long splits: the pipelined kernel
  if (a.blocks_per_split >= PIPE_MIN_BLOCKS) {
    const hipError_t e = launch_attn_bf16_pipe(a, s);
    if (e != hipSuccess) return e;
  } else {
    if (use_h32(a))
      launch(K_ATTN, attn_bf16_kernel<true>, grid, dim3(NTA), s, a);
    else
      launch(K_ATTN, attn_bf16_kernel<false>, grid, dim3(NTA), s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_split == 1) return e;
  launch(K_COMBINE, attn_combine_kernel, dim3(LAT_H / 2 * a.n_rows), dim3(256), s, a);
  return hipGetLastError();
}

bool decode_step_supported(const StepArgs& a) {
  return a.score.fuse && a.score.row0 == 0 && a.attn.row0 == 0 && a.attn.n_rows == a.score.n_rows &&
         a.attn.n_split > 1 && a.attn.blocks_per_split < PIPE_MIN_BLOCKS && a.attn.sel_ready && a.attn.k_new &&
         !a.attn.k_scale && a.score.max_blocks > 0 && a.score.step &&
         a.attn.step_lists == a.score.lists && a.attn.step_meta == a.score.lists_meta &&
         a.attn.step_max_lists == a.score.max_lists && a.attn.sel_out && a.attn.sel_out == a.score.out &&
         a.attn.n_split * a.attn.blocks_per_split >= a.attn.top_k;
}

hipError_t launch_decode_step(const StepArgs& a, hipStream_t s) {
  if (!decode_step_supported(a)) return hipErrorInvalidValue;
  constexpr int KEYS = STEP_NWV * STEP_TILES * 32;   // the scoring role's keys per workgroup
  StepKArgs k;
  k.s = a.score;
  k.at = a.attn;
  k.gx = (a.score.max_blocks + KEYS - 1) / KEYS;
  k.n_score = k.gx * a.score.n_rows;
  k.n_app = a.score.with_append ? a.score.append.batch : 0;   // one workgroup per sequence
  k.at.step_lists_n = STEP_NWV * k.gx;                         // lists of the longest row
  if (k.at.step_lists_n * sel::LIST > 8 * NTA || k.at.step_lists_n > a.attn.step_max_lists)
    return hipErrorInvalidValue;
  const int64_t grid = (int64_t)k.n_score + k.n_app + (use_h32(a.attn) ? 2 : 1) * (int64_t)a.attn.n_rows * a.attn.n_split;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipError_t e = hipSuccess;
  if (use_h32(a.attn)) {
    e = launch_decode_step_h32(k, (unsigned)grid, s);
  } else {
    launch(K_STEP, decode_step_kernel, dim3((unsigned)grid), dim3(NTA), s, k);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  launch(K_COMBINE, attn_combine_kernel, dim3(LAT_H / 2 * a.attn.n_rows), dim3(256), s, a.attn);
  return hipGetLastError();
}

hipError_t launch_attn_fp8(const AttnArgs& a, hipStream_t s) {
  if (a.n_rows <= 0) return hipSuccess;
  launch(K_ATTN, attn_fp8_kernel, dim3((unsigned)((int64_t)a.n_rows * a.n_split)), dim3(NTA), s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_split == 1) return e;
  launch(K_COMBINE, attn_combine_kernel, dim3(LAT_H / 2 * a.n_rows), dim3(256), s, a);
  return hipGetLastError();
}

hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t s) {
  if (a.n_rows <= 0) return hipSuccess;
  launch(K_ATTN, attn_f32_kernel, dim3(a.n_rows), dim3(NT), s, a);
  return hipGetLastError();
}

}  // namespace ip
