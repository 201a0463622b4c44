// Sparse attention over the tokens of the selected blocks.  G2C Brief "GLM-5.3-Flash:
// hybrid attention becomes the product", section "DSA keeps selected global access
// in eleven layers": the DSA layers keep a token-addressable MLA latent history
// (rank 512 per token) and attend over the selected subset of it.
//
// bf16 latent path (MQA, 64 heads over one 576-dim latent row, V = first 512 dims):
//   one workgroup (4 waves) per (query row, split of the selected blocks, group of
//   16 heads).  The selected rows are gathered 64 tokens (16 blocks of 4 contiguous
//   rows) at a time into LDS, double buffered through registers.  Wave w computes
//   S^T = K . q^T for tokens 16w..16w+15 of the sub-tile on bf16 MFMA (16x16x32,
//   q kept in registers), so each lane holds one head and 4 tokens; the row
//   statistics are lane-local plus two exchanges.  The probabilities go to LDS as
//   bf16 and wave w then accumulates O[16 heads, dims 128w..128w+127] += P . V on
//   MFMA, with V read from the same LDS rows.  Online softmax in base 2.  With more
//   than one split the unnormalised partials (O, m, l) are merged by a combine
//   kernel.  The four head-group workgroups that read the same rows get block ids
//   congruent modulo 8, so they run on the same XCD and share its L2.
// f32 path (small geometries): plain VALU, one workgroup per row.
#include "kernels.hpp"

namespace ip {

namespace {

constexpr int NT = 256;
constexpr int SUBT = 64;                       // tokens per sub-tile (16 blocks)
constexpr int ROWB = LAT_DK * 2 + 16;          // padded LDS row: 1168 bytes
constexpr int KVBUF = SUBT * ROWB;             // 74752 bytes
constexpr int HPW = 16;                        // heads per workgroup
constexpr int HGRP = LAT_H / HPW;              // head groups per row
constexpr int PROW = SUBT * 2 + 16;            // P row: 64 bf16 + pad = 144 bytes
constexpr int CHUNKS = LAT_DK * 2 / 16;        // 72 16-byte chunks per latent row
constexpr int LOADS = SUBT * CHUNKS / NT;      // 18 chunks per thread per sub-tile
constexpr int QSTEPS = LAT_DK / 32;            // 18 MFMA k-steps over the 576 dims
constexpr float LN2 = 0.69314718055994531f;
constexpr float LOG2E = 1.44269504088896341f;

typedef float f32x4v __attribute__((ext_vector_type(4)));

constexpr int MAX_BLOCKS_PER_SPLIT = 512;     // host keeps splits within this
constexpr uint32_t MASKED = 0x80000000u;     // token-table flag: not visible (t > p or no block)

typedef short s16x4_t __attribute__((ext_vector_type(4)));

struct __align__(16) AttnShared {
  uint8_t kv[2][KVBUF];
  uint8_t p[HPW * PROW];
  uint32_t tok[MAX_BLOCKS_PER_SPLIT * 4];    // physical row of every selected token (| MASKED)
  float m_part[4][HPW];
  float l_part[4][HPW];
  float alpha[HPW];
  float lfin[HPW];
};

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

// Token table of the split: entry 4i+j is the physical row of token 4*sel[sb0+i]+j,
// flagged MASKED when that token is after the query (t > p) or the entry is -1 or
// past the split; masked entries point at the query's own row so that every load
// stays inside the cache.
__device__ __forceinline__ void build_token_table(const AttnArgs& a, const RowCtx& c, int sb0, int send,
                                                  AttnShared& sh) {
  const int nb = ((send - sb0 + 15) >> 4) << 4;
  const uint32_t prow = (uint32_t)a.L.tok_row(c.b, c.p);
  for (int i = threadIdx.x; i < nb; i += NT) {
    const int bi = sb0 + i;
    const int blk = bi < send ? c.sel[bi] : -1;
    uint4 e = make_uint4(prow | MASKED, prow | MASKED, prow | MASKED, prow | MASKED);
    if (blk >= 0 && blk * 4 <= c.p) {
      const uint32_t row = (uint32_t)a.L.tok_row(c.b, (int64_t)blk * 4);   // 4 consecutive rows
      const int vis = min(4, c.p - blk * 4 + 1);
      e.x = row;
      e.y = vis > 1 ? row + 1 : (prow | MASKED);
      e.z = vis > 2 ? row + 2 : (prow | MASKED);
      e.w = vis > 3 ? row + 3 : (prow | MASKED);
    }
    *(uint4*)&sh.tok[4 * i] = e;
  }
}

// Thread t stages token t/4 of the sub-tile, 16-byte chunks (t%4) + 4i (i < 18):
// one table lookup per thread and immediate-offset loads from one base address.
__device__ __forceinline__ void load_subtile(const AttnArgs& a, const AttnShared& sh, int n,
                                             u32x4_t (&st)[LOADS]) {
  const uint32_t row = sh.tok[n * SUBT + (threadIdx.x >> 2)] & ~MASKED;
  const u32x4_t* src = (const u32x4_t*)(a.k + (uint64_t)row * a.k_stride) + (threadIdx.x & 3);
#pragma unroll
  for (int i = 0; i < LOADS; ++i) st[i] = src[4 * i];
}

__device__ __forceinline__ void store_subtile(uint8_t* buf, const u32x4_t (&st)[LOADS]) {
  u32x4_t* dst = (u32x4_t*)(buf + (threadIdx.x >> 2) * ROWB) + (threadIdx.x & 3);
#pragma unroll
  for (int i = 0; i < LOADS; ++i) dst[4 * i] = st[i];
}

__global__ __launch_bounds__(NT, 1) void attn_bf16_kernel(AttnArgs a) {
  __shared__ AttnShared sh;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int l16 = lane & 15, q4 = lane >> 4;
  // block id -> (group g = row * n_split + split, head group hg); the HGRP
  // workgroups of one group share id % 8 (same XCD) and are dispatched together
  const int id = blockIdx.x;
  const int hg = (id >> 3) % HGRP;
  const int g = (id / (8 * HGRP)) * 8 + (id & 7);
  if (g >= a.n_rows * a.n_split) return;
  const int split = g % a.n_split;
  const int rl = g / a.n_split;
  const int r = a.row0 + rl;
  const int h0 = hg * HPW;
  const RowCtx c = row_ctx(a, r);
  const int sb0 = split * a.blocks_per_split;
  const int send = min(a.top_k, sb0 + a.blocks_per_split);
  const int nsub = (send - sb0 + 15) >> 4;

  // q^T fragments: head h0 + l16, dims s*32 + q4*8 .. +8
  bf16x8_t qf[QSTEPS];
  {
    const u32x4_t* qs = (const u32x4_t*)((const uint16_t*)a.q + ((int64_t)r * LAT_H + h0 + l16) * LAT_DK + q4 * 8);
#pragma unroll
    for (int s = 0; s < QSTEPS; ++s) qf[s] = __builtin_bit_cast(bf16x8_t, qs[4 * s]);
  }
  const float cs = a.scale * LOG2E;

  f32x4v o[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) o[n] = f32x4v{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  build_token_table(a, c, sb0, send, sh);
  block_sync_lds();
  u32x4_t st[LOADS];
  if (nsub > 0) {
    load_subtile(a, sh, 0, st);
    store_subtile(sh.kv[0], st);
    if (nsub > 1) load_subtile(a, sh, 1, st);
  }
  block_sync_lds();

  // transposed V reads: source lane (token t0 + l16/4, dims f + 4*(l16%4)) gives
  // output lane l16 the values V[t0 + j][f + l16], j = 0..3
  const int vtok = l16 >> 2, vdim = (l16 & 3) * 4;

  for (int n = 0; n < nsub; ++n) {
    const uint8_t* buf = sh.kv[n & 1];
    // ---- S^T[token, head] for tokens 16*wv .. 16*wv+15
    f32x4v sacc = {0.f, 0.f, 0.f, 0.f};
    {
      const uint8_t* kr = buf + (wv * 16 + l16) * ROWB + q4 * 16;
#pragma unroll
      for (int s = 0; s < QSTEPS; ++s) {
        const bf16x8_t kf = *(const bf16x8_t*)(kr + s * 64);
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[s], sacc, 0, 0, 0);
      }
    }
    // lane holds tokens 16*wv + 4*q4 + i of head h0 + l16
    float sv[4];
    float mloc = -INFINITY;
    {
      const uint4 tk = *(const uint4*)&sh.tok[n * SUBT + wv * 16 + q4 * 4];
      const uint32_t tv[4] = {tk.x, tk.y, tk.z, tk.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sv[i] = (tv[i] & MASKED) ? -INFINITY : sacc[i] * cs;
        mloc = fmaxf(mloc, sv[i]);
      }
    }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    if (q4 == 0) sh.m_part[wv][l16] = mloc;
    block_sync_lds();
    const float m_tile = fmaxf(fmaxf(sh.m_part[0][l16], sh.m_part[1][l16]), fmaxf(sh.m_part[2][l16], sh.m_part[3][l16]));
    const float m_new = fmaxf(m_run, m_tile);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    float pv[4], lsum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) { pv[i] = exp2f(sv[i] - m_use); lsum += pv[i]; }
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    {
      uint8_t* pr = sh.p + l16 * PROW + (wv * 16 + q4 * 4) * 2;
      *(uint2*)pr = make_uint2((uint32_t)f32_to_bf16(pv[0]) | ((uint32_t)f32_to_bf16(pv[1]) << 16),
                               (uint32_t)f32_to_bf16(pv[2]) | ((uint32_t)f32_to_bf16(pv[3]) << 16));
    }
    if (q4 == 0) {
      sh.l_part[wv][l16] = lsum;
      if (wv == 0) sh.alpha[l16] = alpha;
    }
    // every wave sees the same 16 maxima, so this test is uniform across the workgroup
    const bool rescale = __ballot(m_new != m_run) != 0ull;
    m_run = m_new;
    block_sync_lds();
    l_run = alpha * l_run + (sh.l_part[0][l16] + sh.l_part[1][l16]) + (sh.l_part[2][l16] + sh.l_part[3][l16]);

    // ---- O[16 heads, dims 128*wv .. +127] += P . V
    if (rescale) {
      float al[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) al[i] = sh.alpha[q4 * 4 + i];
#pragma unroll
      for (int nt = 0; nt < 8; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[nt][i] *= al[i];
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8_t pf = *(const bf16x8_t*)(sh.p + l16 * PROW + (ks * 32 + q4 * 8) * 2);
      const uint8_t* vr = buf + (ks * 32 + q4 * 8 + vtok) * ROWB + (wv * 128 + vdim) * 2;
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;
        const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vr + nt * 32));
        const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vr + 4 * ROWB + nt * 32));
        const s16x4_t v8[2] = {lo, hi};
        o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf, __builtin_bit_cast(bf16x8_t, v8), o[nt], 0, 0, 0);
      }
    }
    // ---- stage the next sub-tile, fetch the one after
    if (n + 1 < nsub) {
      store_subtile(sh.kv[(n + 1) & 1], st);
      if (n + 2 < nsub) load_subtile(a, sh, n + 2, st);
    }
    block_sync_lds();
  }

  // ---- epilogue: lane holds heads h0 + 4*q4 + i, dims 128*wv + 16*nt + l16
  if (a.n_split == 1) {
    if (wv == 0 && q4 == 0) {
      sh.lfin[l16] = l_run;
      if (a.lse) a.lse[(int64_t)r * LAT_H + h0 + l16] = (m_run + log2f(l_run)) * LN2;
    }
    __syncthreads();
    uint16_t* out = (uint16_t*)a.out + ((int64_t)r * LAT_H + h0) * LAT_DV;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hd = q4 * 4 + i;
      const float inv = 1.f / sh.lfin[hd];
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) out[hd * LAT_DV + wv * 128 + nt * 16 + l16] = f32_to_bf16(o[nt][i] * inv);
    }
  } else {
    const int64_t pi = (int64_t)rl * a.n_split + split;
    float* po = a.part_o + (pi * LAT_H + h0) * LAT_DV;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hd = q4 * 4 + i;
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) po[hd * LAT_DV + wv * 128 + nt * 16 + l16] = o[nt][i];
    }
    if (wv == 0 && q4 == 0) {
      a.part_ml[(pi * LAT_H + h0 + l16) * 2] = m_run;
      a.part_ml[(pi * LAT_H + h0 + l16) * 2 + 1] = l_run;
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
constexpr int F_MAXH = 16, F_MAXD = 128, F_TILE = 256;
__global__ __launch_bounds__(NT) void attn_f32_kernel(AttnArgs a) {
  __shared__ float qs[F_MAXH * F_MAXD];
  __shared__ float ps[F_MAXH][F_TILE];
  __shared__ int64_t rows[F_TILE];
  __shared__ float stat[3][F_MAXH];           // tile max, new max, alpha
  const int r = a.row0 + blockIdx.x;
  const RowCtx c = row_ctx(a, r);
  const int H = a.heads, dk = a.dk, dv = a.dv;
  const float* q = (const float*)a.q + (int64_t)r * H * dk;
  for (int i = threadIdx.x; i < H * dk; i += NT) qs[i] = q[i];
  const int nout = H * dv;                      // <= 2048 outputs, 8 per thread
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float m_run[F_MAXH], l_run[F_MAXH];
#pragma unroll
  for (int h = 0; h < F_MAXH; ++h) { m_run[h] = -INFINITY; l_run[h] = 0.f; }
  const int ntok = a.top_k * 4;
  __syncthreads();
  for (int t0 = 0; t0 < ntok; t0 += F_TILE) {
    const int tt = t0 + threadIdx.x;
    int t = -1;
    if (tt < ntok) {
      const int blk = c.sel[tt >> 2];
      if (blk >= 0 && blk * 4 + (tt & 3) <= c.p) t = blk * 4 + (tt & 3);
    }
    const int64_t row = t >= 0 ? a.L.tok_row(c.b, t) : -1;
    rows[threadIdx.x] = row;
    const float* kr = row >= 0 ? (const float*)(a.k + row * a.k_stride) : nullptr;
    for (int h = 0; h < H; ++h) {
      float s = -INFINITY;
      if (kr) {
        float d = 0.f;
        for (int e = 0; e < dk; ++e) d = fmaf(qs[h * dk + e], kr[e], d);
        s = d * a.scale;
      }
      ps[h][threadIdx.x] = s;
    }
    __syncthreads();
    // per-head tile max: 16 threads per head
    {
      const int h = threadIdx.x >> 4, sub = threadIdx.x & 15;
      float mx = -INFINITY;
      if (h < H)
        for (int i = sub; i < F_TILE; i += 16) mx = fmaxf(mx, ps[h][i]);
#pragma unroll
      for (int o = 8; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 16));
      if (h < H && sub == 0) stat[0][h] = mx;
    }
    __syncthreads();
    for (int h = 0; h < H; ++h) {
      const float mn = fmaxf(m_run[h], stat[0][h]);
      const float mu = mn == -INFINITY ? 0.f : mn;
      const float al = expf(m_run[h] - mu);
      const float pv = expf(ps[h][threadIdx.x] - mu);
      __syncthreads();
      ps[h][threadIdx.x] = pv;
      if (threadIdx.x == 0) { stat[1][h] = mu; stat[2][h] = al; }
      m_run[h] = mn;
      __syncthreads();
    }
    // l and O updates
    for (int h = 0; h < H; ++h) {
      float sum = 0.f;
      for (int i = 0; i < F_TILE; ++i) sum += ps[h][i];
      l_run[h] = stat[2][h] * l_run[h] + sum;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int oi = threadIdx.x + NT * k;
      if (oi < nout) {
        const int h = oi / dv, d = oi - h * dv;
        float x = acc[k] * stat[2][h];
        for (int i = 0; i < F_TILE; ++i) {
          const int64_t rw = rows[i];
          if (rw >= 0) x = fmaf(ps[h][i], ((const float*)(a.v + rw * a.v_stride))[d], x);
        }
        acc[k] = x;
      }
    }
    __syncthreads();
  }
  float* out = (float*)a.out + (int64_t)r * nout;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int oi = threadIdx.x + NT * k;
    if (oi < nout) out[oi] = acc[k] / l_run[oi / dv];
  }
  if (a.lse && threadIdx.x < H) {
    float mh = 0.f, lh = 0.f;
    for (int h = 0; h < H; ++h)
      if (h == (int)threadIdx.x) { mh = m_run[h]; lh = l_run[h]; }
    a.lse[(int64_t)r * H + threadIdx.x] = mh + logf(lh);
  }
}

}  // namespace

hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t s) {
  if (a.n_rows <= 0) return hipSuccess;
  const int64_t groups = (int64_t)a.n_rows * a.n_split;
  const unsigned grid = (unsigned)((groups + 7) / 8 * 8 * HGRP);
  launch(K_ATTN, attn_bf16_kernel, dim3(grid), dim3(NT), s, a);
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
