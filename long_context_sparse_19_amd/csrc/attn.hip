// Sparse attention over the tokens of the selected blocks.  G2C Brief "GLM-5.3-Flash:
// hybrid attention becomes the product", section "DSA keeps selected global access
// in eleven layers": the DSA layers keep a token-addressable MLA latent history
// (rank 512 per token) and attend over the selected subset of it.
//
// bf16 latent path (MQA, 64 heads over one 576-dim latent row, V = first 512 dims):
//   one workgroup (4 waves) per (query row, split of the selected blocks).  The
//   selected rows are gathered 64 tokens (16 blocks of 4 contiguous rows) at a time
//   into LDS, double buffered through registers.  Wave w = (hg, th) owns heads
//   32*hg..32*hg+31: it computes S^T = K . q^T for token half th of the sub-tile on
//   bf16 MFMA (32x32x16, q kept in registers), so each lane holds one head and 16
//   tokens and the softmax row statistics are lane-local plus one exchange.  The
//   probabilities go to LDS as bf16 and the same wave then accumulates
//   O[32 heads, 256 dims of half th] += P . V on MFMA, with V read from the same
//   LDS rows.  Online softmax in base 2.  With more than one split the unnormalised
//   partials (O, m, l) are merged by a combine kernel.
// f32 path (small geometries): plain VALU, one workgroup per row.
#include "kernels.hpp"

namespace ip {

namespace {

constexpr int NT = 256;
constexpr int SUBT = 64;                       // tokens per sub-tile (16 blocks)
constexpr int ROWB = LAT_DK * 2 + 16;          // padded LDS row: 1168 bytes
constexpr int KVBUF = SUBT * ROWB;             // 74752 bytes
constexpr int PROW = SUBT * 2 + 16;            // P row: 64 bf16 + pad = 144 bytes
constexpr int CHUNKS = LAT_DK * 2 / 16;        // 72 16-byte chunks per latent row
constexpr int LOADS = SUBT * CHUNKS / NT;      // 18 chunks per thread per sub-tile
constexpr float LN2 = 0.69314718055994531f;
constexpr float LOG2E = 1.44269504088896341f;

struct __align__(16) AttnShared {
  uint8_t kv[2][KVBUF];
  uint8_t p[LAT_H * PROW];
  float m_part[2][LAT_H];
  float l_part[2][LAT_H];
  float alpha[LAT_H];
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

// token of sub-tile slot tt (0..63) starting at selection entry sb; -1 if masked
__device__ __forceinline__ int slot_token(const RowCtx& c, int sb, int send, int tt) {
  const int bi = sb + (tt >> 2);
  if (bi >= send) return -1;
  const int blk = c.sel[bi];
  if (blk < 0) return -1;
  const int t = blk * 4 + (tt & 3);
  return t <= c.p ? t : -1;
}

__device__ __forceinline__ void load_subtile(const AttnArgs& a, const RowCtx& c, int sb, int send,
                                             u32x4_t (&st)[LOADS]) {
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int s = threadIdx.x + NT * i;
    const int tt = s / CHUNKS, ch = s - tt * CHUNKS;
    int t = slot_token(c, sb, send, tt);
    if (t < 0) t = c.p;                        // any valid row; masked later
    const int64_t row = a.L.tok_row(c.b, t);
    st[i] = *(const u32x4_t*)(a.k + row * a.k_stride + ch * 16);
  }
}

__device__ __forceinline__ void store_subtile(uint8_t* buf, const u32x4_t (&st)[LOADS]) {
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int s = threadIdx.x + NT * i;
    const int tt = s / CHUNKS, ch = s - tt * CHUNKS;
    *(u32x4_t*)(buf + tt * ROWB + ch * 16) = st[i];
  }
}

__global__ __launch_bounds__(NT, 1) void attn_bf16_kernel(AttnArgs a) {
  __shared__ AttnShared sh;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int kl = lane & 31, hh = lane >> 5;
  const int hg = wv >> 1, th = wv & 1;
  const int head = hg * 32 + kl;               // this lane's head in the QK layout
  const int split = blockIdx.x;
  const int r = a.row0 + blockIdx.y;
  const RowCtx c = row_ctx(a, r);
  const int sb0 = split * a.blocks_per_split;
  const int send = min(a.top_k, sb0 + a.blocks_per_split);
  const int nsub = (send - sb0 + 15) >> 4;

  // q^T fragments: head `head`, dims s*16 + hh*8 .. +8 for s = 0..35
  bf16x8_t qf[LAT_DK / 16];
  {
    const u32x4_t* qs = (const u32x4_t*)((const uint16_t*)a.q + ((int64_t)r * LAT_H + head) * LAT_DK + hh * 8);
#pragma unroll
    for (int s = 0; s < LAT_DK / 16; ++s) qf[s] = __builtin_bit_cast(bf16x8_t, qs[2 * s]);
  }
  const float cs = a.scale * LOG2E;

  f32x16_t o[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) o[n] = f32x16_t{};
  float m_run = -INFINITY, l_run = 0.f;

  u32x4_t st[LOADS];
  if (nsub > 0) {
    load_subtile(a, c, sb0, send, st);
    store_subtile(sh.kv[0], st);
    if (nsub > 1) load_subtile(a, c, sb0 + 16, send, st);
  }
  __syncthreads();

  for (int n = 0; n < nsub; ++n) {
    const uint8_t* buf = sh.kv[n & 1];
    const int sb = sb0 + n * 16;
    // ---- S^T[token, head] for the 32 tokens of half th
    f32x16_t sacc = {};
    {
      const uint8_t* kr = buf + (th * 32 + kl) * ROWB + hh * 16;
#pragma unroll
      for (int s = 0; s < LAT_DK / 16; ++s) {
        const bf16x8_t kf = *(const bf16x8_t*)(kr + s * 32);
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], sacc, 0, 0, 0);
      }
    }
    // lane holds tokens th*32 + (i/4)*8 + hh*4 + i%4 of head `head`
    float sv[16];
    float mloc = -INFINITY;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int tt0 = th * 32 + g * 8 + hh * 4;           // 4 tokens of one block
      const int bi = sb + (tt0 >> 2);
      const int blk = bi < send ? c.sel[bi] : -1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = blk >= 0 && blk * 4 + i <= c.p;
        const float v = ok ? sacc[g * 4 + i] * cs : -INFINITY;
        sv[g * 4 + i] = v;
        mloc = fmaxf(mloc, v);
      }
    }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    if (hh == 0) sh.m_part[th][head] = mloc;
    __syncthreads();
    const float m_new = fmaxf(m_run, fmaxf(sh.m_part[0][head], sh.m_part[1][head]));
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    float lsum = 0.f;
    uint32_t pk[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p0 = exp2f(sv[2 * i] - m_use);
      const float p1 = exp2f(sv[2 * i + 1] - m_use);
      lsum += p0 + p1;
      pk[i] = (uint32_t)f32_to_bf16(p0) | ((uint32_t)f32_to_bf16(p1) << 16);
    }
    lsum += __shfl_xor(lsum, 32);
    {
      // P row `head`, slots th*32 + hh*16 + i  (i = this lane's 16 values)
      uint8_t* pr = sh.p + head * PROW + (th * 32 + hh * 16) * 2;
      *(u32x4_t*)pr = u32x4_t{pk[0], pk[1], pk[2], pk[3]};
      *(u32x4_t*)(pr + 16) = u32x4_t{pk[4], pk[5], pk[6], pk[7]};
    }
    if (hh == 0) {
      sh.l_part[th][head] = lsum;
      if (th == 0) sh.alpha[head] = alpha;
    }
    m_run = m_new;
    __syncthreads();
    l_run = alpha * l_run + sh.l_part[0][head] + sh.l_part[1][head];

    // ---- O[32 heads of hg, 256 dims of half th] += P . V
    {
      float al[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) al[i] = sh.alpha[hg * 32 + (i >> 2) * 8 + hh * 4 + (i & 3)];
#pragma unroll
      for (int nt = 0; nt < 8; ++nt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[nt][i] *= al[i];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8_t pf = *(const bf16x8_t*)(sh.p + (hg * 32 + kl) * PROW + (ks * 16 + hh * 8) * 2);
        // slot ks*16 + hh*8 + e holds token tb + (e/4)*8 + e%4
        const int tb = (ks >> 1) * 32 + (ks & 1) * 4 + hh * 16;
        const uint8_t* vr = buf + th * 512 + kl * 2;
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
          uint16_t vv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e)
            vv[e] = *(const uint16_t*)(vr + (tb + (e >> 2) * 8 + (e & 3)) * ROWB + nt * 64);
          u32x4_t vp;
#pragma unroll
          for (int e = 0; e < 4; ++e) vp[e] = (uint32_t)vv[2 * e] | ((uint32_t)vv[2 * e + 1] << 16);
          o[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pf, __builtin_bit_cast(bf16x8_t, vp), o[nt], 0, 0, 0);
        }
      }
    }
    // ---- stage the next sub-tile, fetch the one after
    if (n + 1 < nsub) {
      store_subtile(sh.kv[(n + 1) & 1], st);
      if (n + 2 < nsub) load_subtile(a, c, sb + 32, send, st);
    }
    __syncthreads();
  }

  // ---- epilogue
  const int64_t ob = (int64_t)r - a.row0;
  if (a.n_split == 1) {
    if (hh == 0 && th == 0) sh.l_part[0][head] = l_run;
    if (a.lse && hh == 0 && th == 0) a.lse[(int64_t)r * LAT_H + head] = (m_run + log2f(l_run)) * LN2;
    __syncthreads();
    float inv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) inv[i] = 1.f / sh.l_part[0][hg * 32 + (i >> 2) * 8 + hh * 4 + (i & 3)];
    uint16_t* out = (uint16_t*)a.out + (int64_t)r * LAT_H * LAT_DV;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int hd = hg * 32 + (i >> 2) * 8 + hh * 4 + (i & 3);
        out[hd * LAT_DV + th * 256 + nt * 32 + kl] = f32_to_bf16(o[nt][i] * inv[i]);
      }
  } else {
    const int64_t pi = ob * a.n_split + split;
    float* po = a.part_o + pi * LAT_H * LAT_DV;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int hd = hg * 32 + (i >> 2) * 8 + hh * 4 + (i & 3);
        po[hd * LAT_DV + th * 256 + nt * 32 + kl] = o[nt][i];
      }
    if (hh == 0 && th == 0) {
      a.part_ml[(pi * LAT_H + head) * 2] = m_run;
      a.part_ml[(pi * LAT_H + head) * 2 + 1] = l_run;
    }
  }
}

// Merge split partials: per (row, head) O = sum_s 2^(m_s - m) O_s / sum_s 2^(m_s - m) l_s.
__global__ __launch_bounds__(128) void attn_combine_kernel(AttnArgs a) {
  const int head = blockIdx.x;
  const int rl = blockIdx.y;
  const int r = a.row0 + rl;
  float m = -INFINITY;
  for (int s = 0; s < a.n_split; ++s)
    m = fmaxf(m, a.part_ml[(((int64_t)rl * a.n_split + s) * LAT_H + head) * 2]);
  float L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < a.n_split; ++s) {
    const int64_t pi = (int64_t)rl * a.n_split + s;
    const float ms = a.part_ml[(pi * LAT_H + head) * 2];
    const float w = ms == -INFINITY ? 0.f : exp2f(ms - m);
    L += w * a.part_ml[(pi * LAT_H + head) * 2 + 1];
    const float4 v = *(const float4*)(a.part_o + (pi * LAT_H + head) * LAT_DV + threadIdx.x * 4);
    acc.x = fmaf(w, v.x, acc.x);
    acc.y = fmaf(w, v.y, acc.y);
    acc.z = fmaf(w, v.z, acc.z);
    acc.w = fmaf(w, v.w, acc.w);
  }
  const float inv = 1.f / L;
  uint16_t* out = (uint16_t*)a.out + ((int64_t)r * LAT_H + head) * LAT_DV + threadIdx.x * 4;
  const uint32_t lo = (uint32_t)f32_to_bf16(acc.x * inv) | ((uint32_t)f32_to_bf16(acc.y * inv) << 16);
  const uint32_t hi = (uint32_t)f32_to_bf16(acc.z * inv) | ((uint32_t)f32_to_bf16(acc.w * inv) << 16);
  *(uint2*)out = make_uint2(lo, hi);
  if (a.lse && threadIdx.x == 0) a.lse[(int64_t)r * LAT_H + head] = (m + log2f(L)) * LN2;
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
  hook_before(K_ATTN, s);
  hipLaunchKernelGGL(attn_bf16_kernel, dim3(a.n_split, a.n_rows), dim3(NT), 0, s, a);
  hook_after(K_ATTN, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_split == 1) return e;
  hook_before(K_COMBINE, s);
  hipLaunchKernelGGL(attn_combine_kernel, dim3(LAT_H, a.n_rows), dim3(128), 0, s, a);
  hook_after(K_COMBINE, s);
  return hipGetLastError();
}

hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t s) {
  if (a.n_rows <= 0) return hipSuccess;
  hook_before(K_ATTN, s);
  hipLaunchKernelGGL(attn_f32_kernel, dim3(a.n_rows), dim3(NT), 0, s, a);
  hook_after(K_ATTN, s);
  return hipGetLastError();
}

}  // namespace ip
