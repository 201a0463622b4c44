// Sparse attention over the tokens of the selected blocks, bf16 latent path, for
// long selections (a prefill row attends over 2048 tokens).  G2C Brief
// "GLM-5.3-Flash: hybrid attention becomes the product", section "DSA keeps
// selected global access in eleven layers"; same arithmetic and readings as the
// kernel in attn.hip.  There each of 4 waves runs a sub-tile's S^T product, its
// softmax and its PV product, and one wave per SIMD cannot issue the softmax's
// VALU work while its MFMAs run.  This form gives the two jobs to different waves,
// two per SIMD (8 waves), so that one wave's softmax issues while the other's
// MFMAs run:
//   - S-waves w < 4, (hb, th) = (w & 1, w >> 1), hold q of heads 32hb .. +31 in
//     registers and, for sub-tile n (32 tokens, 8 blocks), compute S^T = K . q^T
//     for tokens 16th .. +15 with v_mfma_f32_16x16x32_bf16 (every K fragment
//     feeds two 16-head tiles), the softmax (each lane: one head of each tile, the
//     4 tokens of one block) and P to LDS.
//   - O-waves w >= 4 hold O^T for dims 128(w-4) .. +127 of all 64 heads and, in
//     step n, add V^T . P^T of sub-tile n-1 (two 16-token k-steps of
//     v_mfma_f32_32x32x16_bf16, V by the transposing LDS read) and stream sub-tile
//     n+2 into LDS.
// One barrier per step.  Four sub-tile buffers: n (S^T), n-1 (PV), n+1 (landed or
// landing), n+2 (loading); P has two buffers (written in step n, read in n+1).
// Online softmax against a per-head agreed reference maximum m, which moves only
// when a tile maximum passes it by more than 2^8.  The two token halves of a head
// decide apart, without waiting for each other: each computes P against m, or
// (rare) against its own tile maximum, and publishes the reference it used; at the
// next step every wave takes the larger of the two as the new m (S-waves rescale
// their part of l, O-waves rescale O and the P of each half to it before the PV).
// The number of sub-tiles is rounded up to a multiple of 4 (the steps are unrolled
// by 4, so every buffer access names its buffer); the extra ones hold masked rows.
#include "attn_common.hpp"

namespace ip {

namespace {

constexpr int NTW = 512;                       // 8 waves
constexpr int SUBP = 32;                       // tokens per sub-tile (8 blocks)
constexpr int SEGP = SUBP * 128;               // one 128-byte segment (64 dims) of all 32 rows
constexpr int KVBP = NSEG * SEGP;              // 36864 bytes
constexpr int PROWP = SUBP * 2 + 16;           // P row of one head: 32 bf16 + pad = 80 bytes
constexpr int PBUF = LAT_H * PROWP;            // 5120 bytes
constexpr int QSTEPS = LAT_DK / 32;            // 18 k-steps of 16x16x32 over the 576 dims
constexpr int PL_LOADS = NSEG;                 // LDS DMA instructions per O-wave and sub-tile
constexpr int QHALF = LAT_DK;                  // bytes of half a query row (288 dims)

struct __align__(16) PipeShared {
  uint32_t brow[MAX_BLOCKS_PER_SPLIT];
  float rref[2][4 * 32];                       // [step parity][ref_at(head, half)]: references used for P
  int changed[2][4];                           // [step parity][S-wave]: a reference differs from the agreed one
  float lpart[2][LAT_H];                       // l of every head over each token half (end)
};

// slot of (head h, token half th) in a reference row: an O-wave lane reads those
// of its heads l and 32 + l (both halves) with one 16-byte read
__device__ __forceinline__ int ref_at(int h, int th) { return 4 * (h & 31) + 2 * (h >> 5) + th; }

// byte offset of 16-byte chunk `ch` (0..71) of row `t` in a 32-row buffer (the
// layout and swizzle of the 64-row buffers above, with 4 KB segments)
__device__ __forceinline__ int kvp_off(int t, int ch) {
  return (ch >> 3) * SEGP + t * 128 + 16 * ((ch & 7) ^ kv_swz(t));
}

// The sub-tiles arrive by loads to LDS.  A cache whose rows all lie within 4 GB of
// its base (OFF32) is read by buffer loads (buffer_load_dwordx4 ... lds) with 32-bit
// byte offsets; a paged cache, whose extent the host cannot bound, by
// global_load_lds from base + a 64-bit offset.  (The global form counts, for the
// compiler, as an access that may touch LDS through the flat path; while one is in
// flight it waits for all outstanding LDS reads wherever it needs one, so the K
// fragments read ahead are waited for together: slower on long contiguous splits,
// still far ahead of the one-sub-tile-in-flight kernel on gather-bound paged rows.)
// Lane l of O-wave p loads, of sub-tile m, row t = 8p + l/8 (block 2p + l/32),
// chunk slot l%8; instruction g fills rows 8p .. +7 of segment g, adding 128g
// through the scalar offset (or the address).  The two block-table entries come
// from one 8-byte LDS read.
// row_off: the byte offset from the cache base of this lane's 16 bytes of row t
// (entry e), 32-bit when OFF32.
template <bool OFF32>
struct PipeOff {
  using type = uint64_t;
};
template <>
struct PipeOff<true> {
  using type = uint32_t;
};
template <bool OFF32>
__device__ __forceinline__ typename PipeOff<OFF32>::type row_off(const AttnArgs& a, uint32_t e, int t) {
  const int lane = threadIdx.x & 63;
  using T = typename PipeOff<OFF32>::type;
  return (T)((e & ROW_BITS) + (t & 3)) * (T)a.k_stride + 16 * ((lane & 7) ^ kv_swz(t));
}
template <bool OFF32>
__device__ __forceinline__ typename PipeOff<OFF32>::type pipe_src(const AttnArgs& a, const uint32_t* brow, int m,
                                                                  int p) {
  const int lane = threadIdx.x & 63;
  const uint2 e2 = lds_ld((const uint2*)&brow[8 * m + 2 * p]);
  const uint32_t e = (lane >> 5) ? e2.y : e2.x;
  return row_off<OFF32>(a, e, 8 * p + (lane >> 3));
}

// a buffer resource over [base, base + 4 GB) (raw, no stride)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0xFFFFFFFF, 0x00020000);
}

__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff, uint8_t* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}

__device__ __forceinline__ void pipe_load(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint8_t* buf, int g, int p) {
  lds_dma16(rs, voff, 128 * g, buf + g * SEGP + p * 1024);
}
__device__ __forceinline__ void pipe_load(__amdgpu_buffer_rsrc_t, uint64_t off, const uint8_t* k, uint8_t* buf, int g,
                                          int p) {
  __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(k + off + 128 * g),
                                   (void __attribute__((address_space(3)))*)(buf + g * SEGP + p * 1024), 16, 0, 0);
}
template <bool OFF32>
__device__ __forceinline__ void pipe_load_t(__amdgpu_buffer_rsrc_t rs, typename PipeOff<OFF32>::type off,
                                            const uint8_t* k, uint8_t* buf, int g, int p) {
  if constexpr (OFF32)
    pipe_load(rs, off, buf, g, p);
  else
    pipe_load(rs, off, k, buf, g, p);
}

// 8-byte LDS store of (lo, hi) at base + off, as one integer store whose offset the
// compiler cannot relate to that of another store: two stores from one base are
// merged into one ds_write2, which loses the alias information that keeps it from
// waiting for the LDS DMA in flight
__device__ __forceinline__ void lds_st8(uint8_t* base, int off, uint32_t lo, uint32_t hi) {
  asm("" : "+v"(off));
  lds_st((uint64_t*)(base + off), (uint64_t)lo | ((uint64_t)hi << 32));
}

template <bool OFF32>
__global__ __launch_bounds__(NTW, 1) void attn_bf16_pipe_kernel(AttnArgs a) {
  __shared__ PipeShared sh;
  __shared__ __align__(16) uint8_t pb0[PBUF];    // P[head][token] bf16, even sub-tiles
  __shared__ __align__(16) uint8_t pb1[PBUF];    // odd sub-tiles
  __shared__ __align__(16) uint8_t kb0[KVBP];
  __shared__ __align__(16) uint8_t kb1[KVBP];
  __shared__ __align__(16) uint8_t kb2[KVBP];
  __shared__ __align__(16) uint8_t kb3[KVBP];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, lh = lane >> 5, l16 = lane & 15, lq = lane >> 4;
  const bool swave = wv < 4;
  const int pw = wv & 3;                         // S-wave: head group; O-wave: dim block and rows
  const int bid = blockIdx.x;
  if (bid >= a.n_rows * a.n_split) return;
  const int split = bid % a.n_split;
  const int rl = bid / a.n_split;
  const int r = a.row0 + rl;
  const RowCtx c = row_ctx(a, r);
  const int sb0 = split * a.blocks_per_split;
  const int send = min(a.top_k, sb0 + a.blocks_per_split);
  const int nsub = ((send - sb0 + 31) >> 5) << 2;       // 8-block sub-tiles, a multiple of 4 (<= 64)
  const int nbt = 8 * nsub;

  // ---- prologue: block table (one entry per thread); the query row into kb2 and
  //      kb3 (dims 0..287 and 288..575 of each head, by all waves); sub-tiles 0 and
  //      1 (O-waves)
  const int bi = sb0 + (int)threadIdx.x;
  const int p0 = sb0 + 2 * pw + lh;              // an O-wave lane's block of sub-tile 0 (+8: 1)
  const int eb[3] = {bi < send ? c.sel[bi] : -1, p0 < send ? c.sel[p0] : -1, p0 + 8 < send ? c.sel[p0 + 8] : -1};
  const __amdgpu_buffer_rsrc_t krs = raw_rsrc(a.k);
  {
    // instruction i of wave w fills bytes 1024j .. +1023 (j = 9(w%4) + i) of kb2
    // (S-waves) or kb3 (O-waves), lane l 16 of them
    const __amdgpu_buffer_rsrc_t qrs = raw_rsrc((const uint8_t*)a.q + (int64_t)r * LAT_H * (LAT_DK * 2));
#pragma unroll
    for (int i = 0; i < 9; ++i) {
      const int j = 9 * pw + i;
      const int b = 1024 * j + 16 * lane;
      const uint32_t qo = (b / QHALF) * (LAT_DK * 2) + b % QHALF;
      if (swave)
        lds_dma16(qrs, qo, 0, kb2 + 1024 * j);
      else
        lds_dma16(qrs, qo, QHALF, kb3 + 1024 * j);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  uint32_t ent[3];
  block_entries(a, c, eb, ent);
  if ((int)threadIdx.x < nbt) lds_st(&sh.brow[threadIdx.x], ent[0]);
  if (!swave) {
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int t = 8 * pw + (lane >> 3);
      const auto so = row_off<OFF32>(a, ent[1 + n], t);
#pragma unroll
      for (int g = 0; g < NSEG; ++g) pipe_load_t<OFF32>(krs, so, a.k, n ? kb1 : kb0, g, pw);
    }
  }
  wait_vm<0>();                                  // the query (and, O-waves, sub-tiles 0 and 1)
  block_sync_lds();
  const float cs = a.scale * LOG2E;
  const bool final_out = a.n_split == 1;
  const int64_t pi = (int64_t)rl * a.n_split + split;
  // O leaves in bf16 (normalised when final) through kb0 (heads 0..31) and kb1
  // (heads 32..63), rows OPITCH apart, then in whole 1 KB rows
  constexpr int OPITCH = LAT_DV * 2 + 16;
  static_assert(32 * OPITCH <= KVBP, "32 output rows fit one buffer");

  // The two roles run loops of their own (each holds only its own state across
  // them) with the same barriers: one per step, then two at the end.
  if (swave) {
    // ================================================================ S-waves
    // wave (hb, th) = (w & 1, w >> 1): heads 32hb .. +31 (two 16-head tiles g)
    // against tokens 16th .. +15.  q fragments (16x16x32 B operand): head 32hb +
    // 16g + l16, dims 32s + 8lq .. +7.  Per head of this lane (g = 0, 1): the agreed
    // reference m, this lane's part lp of l relative to it, and of the last step the
    // reference rr used for P and the sum ls.  (All 256 registers a wave has here are
    // ordinary VGPRs: nothing asks for accumulation registers.)
    const int hb = pw & 1, th = pw >> 1;
    bf16x8_t qf[2][QSTEPS];
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int s = 0; s < QSTEPS; ++s) {
        const int ofs = (32 * hb + 16 * g + l16) * QHALF + 64 * (s % (QSTEPS / 2)) + 16 * lq;
        qf[g][s] = *(const bf16x8_t*)((s < QSTEPS / 2 ? kb2 : kb3) + ofs);
      }
    float m[2] = {-INFINITY, -INFINITY}, lp[2] = {0.f, 0.f};
    float rr[2] = {-INFINITY, -INFINITY}, ls[2] = {0.f, 0.f};
    block_sync_lds();                            // q read: kb2 and kb3 are free

    // fold the last step into (m, lp): the new agreed reference of a head is the
    // larger of the two halves' references (equal to m unless one moved)
    auto fold = [&](int slot) __attribute__((always_inline)) {
      const u32x4_t ch = lds_ld((const u32x4_t*)sh.changed[slot]);
      if ((ch[hb] | ch[hb + 2]) != 0u) {
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const float2 r2 = lds_ld((const float2*)&sh.rref[slot][ref_at(32 * hb + 16 * g + l16, 0)]);
          const float R = fmaxf(r2.x, r2.y);
          lp[g] = (m[g] == -INFINITY ? 0.f : lp[g] * exp2f(m[g] - R)) + (rr[g] == -INFINITY ? 0.f : ls[g] * exp2f(rr[g] - R));
          m[g] = R;
        }
      } else {
        lp[0] += ls[0];
        lp[1] += ls[1];
      }
    };
    // S^T, softmax and P of sub-tile n from `buf` into `pout`
    auto sjob = [&](const int n, const uint8_t* buf, uint8_t* pout) __attribute__((always_inline)) {
      const int slot = n & 1;
      const int vis = (int)(lds_ld(&sh.brow[8 * n + 4 * th + lq]) >> VIS_SHIFT);
      // S^T[token, head]: x[g][u] = token 16th + 4lq + u, head 32hb + 16g + l16
      f32x4_t x[2] = {f32x4_t{}, f32x4_t{}};
      // the S^T MFMAs issue ahead of the O-wave's on this SIMD (the O-wave's PV
      // then runs while this wave's softmax issues VALU work)
      __builtin_amdgcn_s_setprio(3);
      {
        constexpr int KPF = 4;
        bf16x8_t kf[KPF];
#pragma unroll
        for (int p = 0; p < KPF; ++p) kf[p] = *(const bf16x8_t*)(buf + kvp_off(16 * th + l16, 4 * p + lq));
#pragma unroll
        for (int s = 0; s < QSTEPS; ++s) {
#pragma unroll
          for (int g = 0; g < 2; ++g) x[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[s % KPF], qf[g][s], x[g], 0, 0, 0);
          if (s + KPF < QSTEPS) kf[s % KPF] = *(const bf16x8_t*)(buf + kvp_off(16 * th + l16, 4 * (s + KPF) + lq));
        }
      }
      __builtin_amdgcn_s_setprio(0);
      // the last step's references, needed from here on (folded after the S^T MFMAs,
      // so that they start without waiting for the flags)
      if (n > 0) fold(slot ^ 1);
      // mask (-inf where a block's token is after the query), only in sub-tiles
      // that reach past the query or hold padding
      if (__ballot(vis < 4) != 0ull) {
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
          for (int u = 0; u < 4; ++u) x[g][u] = u < vis ? x[g][u] : -INFINITY;
      }
      // P = 2^(cs S - rr) against rr = the agreed reference m.  Rare: a P above 2^8
      // (a tile maximum passes m by more than 2^8) or a head without a reference
      // yet; then rr = the tile maximum of the unscaled S (cs > 0) over the 16 tokens
      // where it passes m by more than 2^8, else m, and P again.  Masked scores give 0.
      float pv[2][4];
      auto exps = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const float nmu = rr[g] == -INFINITY ? 0.f : -rr[g];
#pragma unroll
          for (int u = 0; u < 4; ++u) pv[g][u] = __builtin_amdgcn_exp2f(fmaf(x[g][u], cs, nmu));
        }
      };
      rr[0] = m[0];
      rr[1] = m[1];
      exps();
      const float pmax = fmaxf(fmaxf(fmaxf(pv[0][0], pv[0][1]), fmaxf(pv[0][2], pv[0][3])),
                               fmaxf(fmaxf(pv[1][0], pv[1][1]), fmaxf(pv[1][2], pv[1][3])));
      const bool rare = __ballot(pmax > 256.f || m[0] == -INFINITY || m[1] == -INFINITY) != 0ull;
      bool moved = false;
      if (rare) {
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const float tm = quad_max16(fmaxf(fmaxf(x[g][0], x[g][1]), fmaxf(x[g][2], x[g][3]))) * cs;
          rr[g] = tm > m[g] + RESCALE_LOG2 ? tm : m[g];
          moved |= rr[g] != m[g];
        }
        exps();
      }
#pragma unroll
      for (int g = 0; g < 2; ++g) lds_st(&sh.rref[slot][ref_at(32 * hb + 16 * g + l16, th)], rr[g]);  // the 4 lanes of a head agree
      lds_st(&sh.changed[slot][pw], (int)(__ballot(moved) != 0ull));
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        ls[g] = (pv[g][0] + pv[g][1]) + (pv[g][2] + pv[g][3]);
        lds_st8(pout, (32 * hb + 16 * g + l16) * PROWP + (16 * th + 4 * lq) * 2, pack_bf16x2(pv[g][0], pv[g][1]),
                pack_bf16x2(pv[g][2], pv[g][3]));
      }
    };
    for (int n = 0; n < nsub; n += 4) {
      sjob(n, kb0, pb0);
      block_sync_lds();
      sjob(n + 1, kb1, pb1);
      block_sync_lds();
      sjob(n + 2, kb2, pb0);
      block_sync_lds();
      sjob(n + 3, kb3, pb1);
      block_sync_lds();
    }
    block_sync_lds();                            // (the O-waves' last PV)
    fold((nsub - 1) & 1);
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const float lw = quad_sum16(lp[g]);
      if (lq == 0) lds_st(&sh.lpart[th][32 * hb + 16 * g + l16], lw);
    }
    block_sync_lds();                            // l of both halves in lpart
    if (th == 0 && lq == 0) {
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const int h = 32 * hb + 16 * g + l16;
        const float lt = lds_ld(&sh.lpart[0][h]) + lds_ld(&sh.lpart[1][h]);
        const float mm = m[g] == -INFINITY ? 0.f : m[g];
        if (final_out) {
          if (a.lse) a.lse[(int64_t)r * LAT_H + h] = (mm + log2f(lt)) * LN2;
        } else {
          a.part_ml[(pi * LAT_H + h) * 2] = mm;
          a.part_ml[(pi * LAT_H + h) * 2 + 1] = lt;
        }
      }
    }
    block_sync_lds();
  } else {
    // ================================================================ O-waves
    // O^T tiles o[i][db][k] = head 32i + l32, dim 128pw + 32db + 8(k/4) + 4lh + k%4;
    // mo[i] the reference maximum of head 32i + l32 that O is scaled to
    f32x16_t o[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int d = 0; d < 4; ++d) o[i][d] = f32x16_t{};
    float mo[2] = {-INFINITY, -INFINITY};
    block_sync_lds();                            // q read: kb2 and kb3 are free

    // O^T += V^T . P^T of sub-tile n from `buf` and `pin`, after moving O to the
    // references the S-waves used for it
    auto ojob = [&](const int n, const uint8_t* buf, const uint8_t* pin) __attribute__((always_inline)) {
      const int slot = n & 1;
      typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;
      const int g4 = lane >> 4, s16 = lane & 15;
      const int vt = 8 * (g4 >> 1) + (s16 >> 2);
      const int vd = 16 * (g4 & 1) + 4 * (s16 & 3);
      const int vch = vd >> 3, vin = (vd & 7) * 2;
      // operands of k-step ks: P fragments of the two head tiles, V^T of the four
      // 32-dim blocks (k-step 0's are read before the flags, so that their latency
      // overlaps the flag read)
      auto load_ks = [&](int ks, bf16x8_t (&pbv)[2], bf16x8_t (&va)[4]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 2; ++i) pbv[i] = lds_ld((const bf16x8_t*)(pin + (32 * i + l32) * PROWP + (16 * ks + 8 * lh) * 2));
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const int ch = 4 * (4 * pw + db) + vch;
          const int t0 = 16 * ks + vt;
          const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(buf + kvp_off(t0, ch) + vin));
          const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(buf + kvp_off(t0 + 4, ch) + vin));
          const s16x4_t v8[2] = {lo, hi};
          va[db] = __builtin_bit_cast(bf16x8_t, v8);
        }
      };
      bf16x8_t pb0[2], va0[4];
      load_ks(0, pb0, va0);
      // rare: move O to the new agreed references R (the larger of the two halves'),
      // and the P of each half from its reference to R (factor f[i][half])
      const u32x4_t ch = lds_ld((const u32x4_t*)sh.changed[slot]);
      const bool rescale = (ch[0] | ch[1] | ch[2] | ch[3]) != 0u;
      float f[2][2] = {{1.f, 1.f}, {1.f, 1.f}};
      if (rescale) {
        const float4 r4 = lds_ld((const float4*)&sh.rref[slot][ref_at(l32, 0)]);
        const float rh[2][2] = {{r4.x, r4.y}, {r4.z, r4.w}};
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const float R = fmaxf(rh[i][0], rh[i][1]);
          const float al = mo[i] == -INFINITY ? 0.f : exp2f(mo[i] - R);
          mo[i] = R;
#pragma unroll
          for (int d = 0; d < 4; ++d) o[i][d] *= al;
#pragma unroll
          for (int k = 0; k < 2; ++k) f[i][k] = rh[i][k] == -INFINITY ? 0.f : exp2f(rh[i][k] - R);
        }
      }
      auto mfma_ks = [&](int ks, bf16x8_t (&pbv)[2], const bf16x8_t (&va)[4]) __attribute__((always_inline)) {
        if (rescale) {
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e) pbv[i][e] = (__bf16)((float)pbv[i][e] * f[i][ks]);
        }
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int i = 0; i < 2; ++i) o[i][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[db], pbv[i], o[i][db], 0, 0, 0);
      };
      mfma_ks(0, pb0, va0);
      bf16x8_t pb1[2], va1[4];
      load_ks(1, pb1, va1);
      mfma_ks(1, pb1, va1);
    };
    // step n: stream sub-tile n+2 (clamped to the last) into `db`, add sub-tile
    // n-1 (`ob`, P from `pr`); past the barrier sub-tile n+1 has landed
    auto ostep = [&](const int n, const uint8_t* ob, const uint8_t* pr, uint8_t* db) __attribute__((always_inline)) {
      const auto so = pipe_src<OFF32>(a, sh.brow, min(n + 2, nsub - 1), pw);
#pragma unroll
      for (int g = 0; g < NSEG; ++g) pipe_load_t<OFF32>(krs, so, a.k, db, g, pw);
      if (n > 0) ojob(n - 1, ob, pr);
      wait_vm<PL_LOADS>();
      block_sync_lds();
    };
    for (int n = 0; n < nsub; n += 4) {
      ostep(n, kb3, pb1, kb2);
      ostep(n + 1, kb0, pb0, kb3);
      ostep(n + 2, kb1, pb1, kb0);
      ostep(n + 3, kb2, pb0, kb1);
    }
    ojob(nsub - 1, kb3, pb1);                    // nsub is a multiple of 4
    wait_vm<0>();                                // the clamped loads of the last steps
    block_sync_lds();
    block_sync_lds();                            // l of both halves is in lpart
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int h = 32 * i + l32;
      const float sc1 = final_out ? 1.f / (lds_ld(&sh.lpart[0][h]) + lds_ld(&sh.lpart[1][h])) : 1.f;
      uint8_t* row = (i ? kb1 : kb0) + l32 * OPITCH + (128 * pw + 4 * lh) * 2;
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *(uint2*)(row + (32 * d + 8 * q) * 2) = make_uint2(pack_bf16x2(o[i][d][4 * q] * sc1, o[i][d][4 * q + 1] * sc1),
                                                             pack_bf16x2(o[i][d][4 * q + 2] * sc1, o[i][d][4 * q + 3] * sc1));
    }
    block_sync_lds();
  }
  uint16_t* dst = final_out ? (uint16_t*)a.out + (int64_t)r * LAT_H * LAT_DV : a.part_o + pi * LAT_H * LAT_DV;
#pragma unroll
  for (int k = 0; k < LAT_H / 8; ++k) {
    const int h = wv + 8 * k;
    const uint8_t* srow = (k < LAT_H / 16 ? kb0 : kb1) + (h & 31) * OPITCH + lane * 16;
    *(u32x4_t*)(dst + h * LAT_DV + lane * 8) = *(const u32x4_t*)srow;
  }
}

}  // namespace

hipError_t launch_attn_bf16_pipe(const AttnArgs& a, hipStream_t s) {
  if (a.n_rows <= 0) return hipSuccess;
  const dim3 grid((unsigned)((int64_t)a.n_rows * a.n_split));
  if (a.k_off32)
    launch(K_ATTN, attn_bf16_pipe_kernel<true>, grid, dim3(NTW), s, a);
  else
    launch(K_ATTN, attn_bf16_pipe_kernel<false>, grid, dim3(NTW), s, a);
  return hipGetLastError();
}

}  // namespace ip
