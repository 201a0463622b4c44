// Sparse attention over the tokens of the selected blocks.  G2C Brief "GLM-5.3-Flash:
// hybrid attention becomes the product", section "DSA keeps selected global access
// in eleven layers": the DSA layers keep a token-addressable MLA latent history
// (rank 512 per token) and attend over the selected subset of it.
//
// bf16 latent path (MQA, 64 heads over one 576-dim latent row, V = first 512 dims):
//   one workgroup (4 waves) per (query row, split of the selected blocks) covers all
//   64 heads, so every gathered latent row is read from memory once and feeds 64
//   heads.  The selected rows are staged 64 tokens (16 blocks of 4 contiguous rows)
//   at a time into LDS, double buffered through registers.
//   - S^T = K . q^T on v_mfma_f32_32x32x16_bf16: wave w takes tokens 32*(w&1) .. +31
//     against heads 32*(w>>1) .. +31; its 32 heads of q (576 dims) stay in
//     registers for the whole row, K comes from LDS.
//   - Online softmax in base 2; the two waves that share a head block exchange their
//     per-head maxima and sums through LDS; P goes to LDS as bf16.
//   - O[64 heads, 128 dims of wave w] += P . V on the same MFMA, V read with the
//     transposing LDS read (ds_read_b64_tr_b16) from the rows K came from.
//   With more than one split the unnormalised partials (O, m, l) are merged by a
//   combine kernel.
// f32 path (small geometries): plain VALU, one workgroup per row.
#include "kernels.hpp"

namespace ip {

namespace {

constexpr int NT = 256;                        // f32 path
constexpr int NTA = 512;                       // bf16 path: 8 waves
constexpr int NWA = NTA / 64;
constexpr int SUBT = 64;                       // tokens per sub-tile (16 blocks)
constexpr int ROWB = LAT_DK * 2 + 16;          // padded LDS row: 1168 bytes
constexpr int KVBUF = SUBT * ROWB;             // 74752 bytes
constexpr int PROW = SUBT * 2 + 16;            // P row of one head: 64 bf16 + pad = 144 bytes
constexpr int CHUNKS = LAT_DK * 2 / 16;        // 72 16-byte chunks per latent row
constexpr int QSTEPS = LAT_DK / 32;            // 18 MFMA k-steps over the 576 dims
constexpr float LN2 = 0.69314718055994531f;
constexpr float LOG2E = 1.44269504088896341f;

constexpr int MAX_BLOCKS_PER_SPLIT = 512;      // host keeps splits within this
constexpr int VIS_SHIFT = 29;                  // block table: first row | visible tokens << 29
constexpr uint32_t ROW_BITS = (1u << VIS_SHIFT) - 1;

typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));

// The latent sub-tiles live in their own LDS object (filled by LDS DMA); keeping the
// other shared data in a separate object lets the compiler see that stores to it
// cannot alias the DMA, so it does not make them wait for outstanding loads.
struct __align__(16) AttnKV {
  uint8_t kv[2][KVBUF];
};
struct __align__(16) AttnShared {
  uint8_t p[LAT_H * PROW];
  uint32_t brow[MAX_BLOCKS_PER_SPLIT];
  float m_part[2][LAT_H];
  float l_part[2][LAT_H];
  float alpha[LAT_H];
  float lfin[LAT_H];
};

// LDS accesses that never touch the latent sub-tile buffers go through these.  The
// restrict-qualified pointer gives them alias-scope metadata, from which the
// compiler's wait insertion can tell that they do not alias the LDS DMA into those
// buffers; without it every LDS access would wait for all outstanding sub-tile loads.
template <class T>
__device__ __forceinline__ T lds_ld(const T* __restrict__ p) { return *p; }
template <class T>
__device__ __forceinline__ void lds_st(T* __restrict__ p, T v) { *p = v; }

struct RowCtx {
  int b, p;
  const int32_t* sel;
};

__device__ __forceinline__ RowCtx row_ctx(const AttnArgs& a, int r) {
  RowCtx c;
  c.b = a.q_seq ? a.q_seq[r] : r;
  c.p = a.q_pos ? a.q_pos[r] : a.L.seq_lens[c.b] - 1;
  c.sel = a.sel + (int64_t)r * a.top_k;
  return c;
}

// Combine over the four lanes l % 16 + 16q (q < 4).  v_permlane16_swap /
// v_permlane32_swap with the same register as both operands give every lane, in
// the two results, its own value and that of lane l ^ 16 (resp. l ^ 32).
__device__ __forceinline__ float quad_max16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float quad_sum16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Block table of the split: entry i = physical row of the first token of block
// sel[sb0 + i] with the number of its tokens at or before the query (0..4) in the
// top bits.  Entries that are -1, past the split or entirely after the query
// point at the query's own block (whose 4 rows exist) with 0 visible tokens, so
// every load stays inside the cache.
__device__ __forceinline__ void build_block_table(const AttnArgs& a, const RowCtx& c, int sb0, int send,
                                                  AttnShared& sh) {
  const int nb = ((send - sb0 + 15) >> 4) << 4;
  const uint32_t own = (uint32_t)a.L.tok_row(c.b, (int64_t)(c.p >> 2) * 4);
  for (int i = threadIdx.x; i < nb; i += NTA) {
    const int bi = sb0 + i;
    const int blk = bi < send ? c.sel[bi] : -1;
    uint32_t e = own;
    if (blk >= 0 && blk * 4 <= c.p) {
      const uint32_t row = (uint32_t)a.L.tok_row(c.b, (int64_t)blk * 4);
      e = row | ((uint32_t)min(4, c.p - blk * 4 + 1) << VIS_SHIFT);
    }
    sh.brow[i] = e;
  }
}

// Sub-tile n (64 tokens = 16 blocks) straight from global memory into LDS
// (global_load_lds_dwordx4: lane l of one instruction fills bytes 16l .. 16l+15 of
// a 1 KB LDS span).  The buffer holds 64 rows of 73 16-byte chunks (72 data + 1 pad);
// linear chunk c = 64k + lane of instruction k is chunk c % 73 of row c / 73, and a
// pad chunk loads chunk 0 of its row again.  73 instructions; wave w issues
// k = w, w+8, .. (10 for wave 0, 9 for the others).
constexpr int KV_INSTR = SUBT * (CHUNKS + 1) / 64;    // 73

__device__ __forceinline__ int subtile_loads(int wv) { return (KV_INSTR - wv + NWA - 1) / NWA; }

__device__ __forceinline__ void load_subtile(const AttnArgs& a, const AttnShared& sh, int n, uint8_t* buf) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < (KV_INSTR + NWA - 1) / NWA; ++i) {
    const int k = wv + NWA * i;
    if (k < KV_INSTR) {
      const int cl = 64 * k + lane;
      const int row = cl / (CHUNKS + 1);
      const int chunk = cl - (CHUNKS + 1) * row;
      const uint32_t grow = (lds_ld(&sh.brow[n * 16 + (row >> 2)]) & ROW_BITS) + (row & 3);
      const uint8_t* src = a.k + (uint64_t)grow * a.k_stride + (chunk < CHUNKS ? chunk : 0) * 16;
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)src,
                                       (void __attribute__((address_space(3)))*)(buf + 1024 * k), 16, 0, 0);
    }
  }
}

// Waits until at most `pending` (0, 9 or 10) of this wave's global loads are
// outstanding.  The vmcnt field of the s_waitcnt immediate is bits 0..3 and 14..15;
// expcnt (bits 4..6) and lgkmcnt (bits 8..11) stay at their maxima (no wait).
__device__ __forceinline__ void wait_loads(int pending) {
  constexpr int NOWAIT = (0x7 << 4) | (0xF << 8);
  if (pending >= 10) __builtin_amdgcn_s_waitcnt(10 | NOWAIT);
  else if (pending == 9) __builtin_amdgcn_s_waitcnt(9 | NOWAIT);
  else __builtin_amdgcn_s_waitcnt(NOWAIT);
}

__global__ __launch_bounds__(NTA, 1) void attn_bf16_kernel(AttnArgs a) {
  __shared__ AttnShared sh;
  __shared__ AttnKV kvs;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int l16 = lane & 15, q4 = lane >> 4;
  const int lr = lane & 31, lh = lane >> 5;
  const int tb = wv & 1, hg = wv >> 1;           // S^T tile: tokens 32tb .. +31, heads 16hg .. +15
  const int g = blockIdx.x;
  if (g >= a.n_rows * a.n_split) return;
  const int split = g % a.n_split;
  const int rl = g / a.n_split;
  const int r = a.row0 + rl;
  const RowCtx c = row_ctx(a, r);
  const int sb0 = split * a.blocks_per_split;
  const int send = min(a.top_k, sb0 + a.blocks_per_split);
  const int nsub = (send - sb0 + 15) >> 4;
  const int hq = 16 * hg + l16;                  // head of this lane in the S^T layout

  // q fragments of head hq: dims 32s + 8q4 .. +8 for k-step s
  bf16x8_t qf[QSTEPS];
  {
    const u32x4_t* qs = (const u32x4_t*)((const uint16_t*)a.q + ((int64_t)r * LAT_H + hq) * LAT_DK + 8 * q4);
#pragma unroll
    for (int s = 0; s < QSTEPS; ++s) qf[s] = __builtin_bit_cast(bf16x8_t, qs[4 * s]);
  }
  const float cs = a.scale * LOG2E;

  f32x16_t o[2][2];                              // [32-head block][32-dim block of this wave]
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) o[i][j] = f32x16_t{};
  float m_run = -INFINITY, l_run = 0.f;

  build_block_table(a, c, sb0, send, sh);
  // the q fragments (issued first) are in registers before the sub-tile loads
  // start, so the loop never waits on them behind the latent loads
  wait_loads(0);
  block_sync_lds();
  if (nsub > 0) load_subtile(a, sh, 0, kvs.kv[0]);
  if (nsub > 1) {
    load_subtile(a, sh, 1, kvs.kv[1]);
    wait_loads(subtile_loads(wv));               // sub-tile 0 landed (this wave's part)
  } else {
    wait_loads(0);
  }
  block_sync_lds();

  // transposed V reads: in 16-lane group G, source lane s points at token
  // 8*(G>>1) + s/4 (+4 for the second read) and dims 16*(G&1) + 4*(s%4) of the
  // 32-dim block, so lane l receives V[8*lh + j][32-dim block + lr], j = 0..3 (4..7)
  const int vtok = 8 * (q4 >> 1) + (l16 >> 2), vdim = 16 * (q4 & 1) + 4 * (l16 & 3);

  for (int n = 0; n < nsub; ++n) {
    const uint8_t* buf = kvs.kv[n & 1];
    // ---- S^T[token, head]: lane holds head hq and tokens 32tb + 16u + 4q4 + i
    //      (block 8tb + 4u + q4 of the sub-tile, offset i)
    f32x4v sacc[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      sacc[u] = f32x4v{0.f, 0.f, 0.f, 0.f};
      const uint8_t* kr = buf + (32 * tb + 16 * u + l16) * ROWB + q4 * 16;
#pragma unroll
      for (int s = 0; s < QSTEPS; ++s) {
        const bf16x8_t kf = *(const bf16x8_t*)(kr + s * 64);
        sacc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[s], sacc[u], 0, 0, 0);
      }
    }
    float mloc = -INFINITY;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int vis = (int)(lds_ld(&sh.brow[n * 16 + 8 * tb + 4 * u + q4]) >> VIS_SHIFT);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sacc[u][i] = i < vis ? sacc[u][i] * cs : -INFINITY;
        mloc = fmaxf(mloc, sacc[u][i]);
      }
    }
    mloc = quad_max16(mloc);                     // over the 4 lanes of head hq
    if (q4 == 0) lds_st(&sh.m_part[tb][hq], mloc);
    block_sync_lds();
    const float m_new = fmaxf(m_run, fmaxf(lds_ld(&sh.m_part[0][hq]), lds_ld(&sh.m_part[1][hq])));
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    m_run = m_new;
    float lsum = 0.f;
    {
      uint8_t* pr = sh.p + hq * PROW + (32 * tb + 4 * q4) * 2;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        float pv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) { pv[i] = exp2f(sacc[u][i] - m_use); lsum += pv[i]; }
        lds_st((uint2*)(pr + 32 * u), make_uint2((uint32_t)f32_to_bf16(pv[0]) | ((uint32_t)f32_to_bf16(pv[1]) << 16),
                                                 (uint32_t)f32_to_bf16(pv[2]) | ((uint32_t)f32_to_bf16(pv[3]) << 16)));
      }
    }
    lsum = quad_sum16(lsum);
    if (q4 == 0) {
      lds_st(&sh.l_part[tb][hq], lsum);
      if (tb == 0) lds_st(&sh.alpha[hq], alpha);
    }
    block_sync_lds();
    l_run = alpha * l_run + lds_ld(&sh.l_part[0][hq]) + lds_ld(&sh.l_part[1][hq]);

    // ---- O[head, dim] for dims 64wv .. +63: lane holds dim 64wv + 32j + lr and
    //      heads 32i + 8q + 4lh + u; rescale by the heads' alpha, then += P . V
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4v al = lds_ld((const f32x4v*)&sh.alpha[32 * i + 8 * q + 4 * lh]);
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int u = 0; u < 4; ++u) o[i][j][4 * q + u] *= al[u];
      }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8_t pa[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) pa[i] = lds_ld((const bf16x8_t*)(sh.p + (32 * i + lr) * PROW + (16 * ks + 8 * lh) * 2));
      const uint8_t* vr = buf + (16 * ks + vtok) * ROWB + (64 * wv + vdim) * 2;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;
        const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vr + j * 64));
        const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vr + 4 * ROWB + j * 64));
        const s16x4_t v8[2] = {lo, hi};
        const bf16x8_t vb = __builtin_bit_cast(bf16x8_t, v8);
#pragma unroll
        for (int i = 0; i < 2; ++i) o[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[i], vb, o[i][j], 0, 0, 0);
      }
    }
    // ---- every wave is done with buffer n&1 past this barrier: fetch sub-tile n+2
    //      into it, then make sure sub-tile n+1 (fetched an iteration ago) landed
    block_sync_lds();
    if (n + 1 < nsub) {
      if (n + 2 < nsub) {
        load_subtile(a, sh, n + 2, kvs.kv[n & 1]);
        wait_loads(subtile_loads(wv));
      } else {
        wait_loads(0);
      }
      block_sync_lds();
    }
  }

  // ---- epilogue: per-head l to the O layout
  if (tb == 0 && q4 == 0) lds_st(&sh.lfin[hq], l_run);
  if (a.n_split == 1) {
    if (tb == 0 && q4 == 0 && a.lse) a.lse[(int64_t)r * LAT_H + hq] = (m_run + log2f(l_run)) * LN2;
    block_sync_lds();
    uint16_t* out = (uint16_t*)a.out + (int64_t)r * LAT_H * LAT_DV + 64 * wv + lr;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4v lf = lds_ld((const f32x4v*)&sh.lfin[32 * i + 8 * q + 4 * lh]);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int h = 32 * i + 8 * q + 4 * lh + u;
          const float inv = 1.f / lf[u];
#pragma unroll
          for (int j = 0; j < 2; ++j) out[h * LAT_DV + 32 * j] = f32_to_bf16(o[i][j][4 * q + u] * inv);
        }
      }
  } else {
    const int64_t pi = (int64_t)rl * a.n_split + split;
    float* po = a.part_o + pi * LAT_H * LAT_DV + 64 * wv + lr;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int h = 32 * i + 8 * q + 4 * lh + u;
#pragma unroll
          for (int j = 0; j < 2; ++j) po[h * LAT_DV + 32 * j] = o[i][j][4 * q + u];
        }
    if (tb == 0 && q4 == 0) {
      a.part_ml[(pi * LAT_H + hq) * 2] = m_run;
      a.part_ml[(pi * LAT_H + hq) * 2 + 1] = l_run;
    }
  }
}

// Merge split partials: per (row, head) O = sum_s 2^(m_s - m) O_s / sum_s 2^(m_s - m) l_s.
// Two heads per workgroup, 128 threads x 4 dims per head; the split weights are
// computed once per wave (lane s holds split s) and broadcast.
constexpr int MAX_SPLIT = 64;
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  const int head = blockIdx.x * 2 + (threadIdx.x >> 7);
  const int rl = blockIdx.y;
  const int r = a.row0 + rl;
  const int t = threadIdx.x & 127, lane = threadIdx.x & 63;
  const int S = a.n_split;
  const int64_t pi0 = (int64_t)rl * S;
  float ms = -INFINITY, ls = 0.f;
  if (lane < S) {
    ms = a.part_ml[((pi0 + lane) * LAT_H + head) * 2];
    ls = a.part_ml[((pi0 + lane) * LAT_H + head) * 2 + 1];
  }
  float m = ms;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  const float wgt = (lane < S && ms != -INFINITY) ? exp2f(ms - m) : 0.f;
  float L = wgt * ls;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) L += __shfl_xor(L, o);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  const float* base = a.part_o + (pi0 * LAT_H + head) * LAT_DV + t * 4;
  int s = 0;
  for (; s + 4 <= S; s += 4) {
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = *(const float4*)(base + (int64_t)(s + u) * LAT_H * LAT_DV);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float wu = __shfl(wgt, s + u);
      acc.x = fmaf(wu, v[u].x, acc.x);
      acc.y = fmaf(wu, v[u].y, acc.y);
      acc.z = fmaf(wu, v[u].z, acc.z);
      acc.w = fmaf(wu, v[u].w, acc.w);
    }
  }
  for (; s < S; ++s) {
    const float4 v = *(const float4*)(base + (int64_t)s * LAT_H * LAT_DV);
    const float wu = __shfl(wgt, s);
    acc.x = fmaf(wu, v.x, acc.x);
    acc.y = fmaf(wu, v.y, acc.y);
    acc.z = fmaf(wu, v.z, acc.z);
    acc.w = fmaf(wu, v.w, acc.w);
  }
  const float inv = 1.f / L;
  uint16_t* out = (uint16_t*)a.out + ((int64_t)r * LAT_H + head) * LAT_DV + t * 4;
  const uint32_t lo = (uint32_t)f32_to_bf16(acc.x * inv) | ((uint32_t)f32_to_bf16(acc.y * inv) << 16);
  const uint32_t hi = (uint32_t)f32_to_bf16(acc.z * inv) | ((uint32_t)f32_to_bf16(acc.w * inv) << 16);
  *(uint2*)out = make_uint2(lo, hi);
  if (a.lse && t == 0) a.lse[(int64_t)r * LAT_H + head] = (m + log2f(L)) * LN2;
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
    __syncthreads();
    // O += P V over the tile
#pragma unroll 4
    for (int k = 0; k < F_TILE; ++k) {
      const float* vr = (const float*)(a.v + rows[k] * a.v_stride);
      const float v0 = vr[d0], v1 = vr[d1];
#pragma unroll
      for (int i = 0; i < F_HPW; ++i) {
        const int h = min(wv + 4 * i, H - 1);
        const float pk = ps[h][k];
        acc[i][0] = fmaf(pk, v0, acc[i][0]);
        acc[i][1] = fmaf(pk, v1, acc[i][1]);
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

hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t s) {
  if (a.n_rows <= 0) return hipSuccess;
  launch(K_ATTN, attn_bf16_kernel, dim3((unsigned)((int64_t)a.n_rows * a.n_split)), dim3(NTA), s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_split == 1) return e;
  launch(K_COMBINE, attn_combine_kernel, dim3(LAT_H / 2, a.n_rows), dim3(256), s, a);
  return hipGetLastError();
}

hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t s) {
  if (a.n_rows <= 0) return hipSuccess;
  launch(K_ATTN, attn_f32_kernel, dim3(a.n_rows), dim3(NT), s, a);
  return hipGetLastError();
}

}  // namespace ip
