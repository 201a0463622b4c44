// KDA decode step: the linear-attention half of the hybrid layer.  G2C Brief
// "GLM-5.3-Flash: hybrid attention becomes the product", section "KDA carries fixed
// state through most layers" (a gated delta-rule recurrence over a fixed matrix
// state per head, a short convolution of width 4 and learned gates) and the release
// summary (64 heads of width 128: a 128 x 128 state per head).
//
// Per sequence b and head h, one step (readings in the design notes):
//   q, k, v = SiLU(causal depthwise conv4 of x_q, x_k, x_v)   (taps t-3 .. t)
//   q, k   /= sqrt(|.|^2 + 1e-6)                               (per head)
//   S'      = Diag(alpha) S          (alpha per key channel, in (0, 1])
//   S       = S' + beta k (v - S'^T k)^T
//   o       = S^T q / sqrt(128)
//
// Every column j of S is updated from column j alone (plus q, k, alpha, beta and
// v_j), so a head splits by columns: one workgroup of 256 threads per (head,
// 32-column slice, sequence), 4 per head.  Thread t holds columns 4(t % 8) .. +3 of
// the slice in rows t / 8 + 32p (p < 4) as 4 float4; a wave covers 8 rows x 128
// bytes, whole cache lines.  The state loads are issued first and land while the
// convolution runs (each workgroup convolves all 128 q and k channels for the
// norms and its own 32 v channels).  S'^T k and S^T q are column sums: over the 8
// row groups of a wave by lane exchanges, over the 4 waves through LDS.  The
// kernel is bound by HBM: 128 KB of state per head and step against ~4 flop per
// state element.  The conv state is read from one buffer and written to another
// (the caller alternates them), since the four workgroups of a head read the same
// taps.
#include "kernels.hpp"

namespace ip {

namespace {

constexpr int KT = 256;              // threads
constexpr int KD = KDA_D;            // 128 key / value channels per head
constexpr int KSL = 32;              // columns per workgroup
constexpr int KNS = KD / KSL;        // 4 slices per head
constexpr int KRG = KT / (KSL / 4);  // 32 row groups
constexpr int KROWS = KD / KRG;      // 4 rows per thread

struct KdaShared {
  float q[KD], k[KD], a[KD], v[KSL];
  float4 red[4][KSL / 4];            // per-wave column sums
  float nrm[2][2];                   // per-wave sums of q^2, k^2 (waves 0 and 1)
};

// x sigmoid(x), the reciprocal from the hardware (v_rcp_f32, 1 ulp)
__device__ __forceinline__ float silu(float x) { return x * __builtin_amdgcn_rcpf(1.f + __expf(-x)); }

// sum over the 8 row groups of a wave (lanes l, l ^ 8, l ^ 16, ... hold one column set)
__device__ __forceinline__ float4 wave_rows_sum(float4 v) {
#pragma unroll
  for (int m = 8; m < 64; m <<= 1) {
    v.x += __shfl_xor(v.x, m);
    v.y += __shfl_xor(v.y, m);
    v.z += __shfl_xor(v.z, m);
    v.w += __shfl_xor(v.w, m);
  }
  return v;
}

// column sums over all 32 row groups; every thread gets those of its own columns
__device__ __forceinline__ float4 column_sums(float4 part, KdaShared& sh) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  part = wave_rows_sum(part);
  if (lane < KSL / 4) sh.red[wv][lane] = part;
  __syncthreads();
  const int c = lane & (KSL / 4 - 1);
  float4 s = sh.red[0][c];
#pragma unroll
  for (int w = 1; w < 4; ++w) {
    const float4 r = sh.red[w][c];
    s = make_float4(s.x + r.x, s.y + r.y, s.z + r.z, s.w + r.w);
  }
  return s;
}

__global__ __launch_bounds__(KT) void kda_decode_kernel(KdaArgs a) {
  __shared__ KdaShared sh;
  const int h = blockIdx.x / KNS, sl = blockIdx.x % KNS, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int col4 = tid & (KSL / 4 - 1), rg = tid >> 3;
  const int64_t HD = (int64_t)a.heads * KD;
  float* S = a.state + ((int64_t)b * a.heads + h) * KD * KD + KSL * sl + 4 * col4;

  // ---- the state slice first: 4 float4 per thread in flight during the convolution
  float4 s[KROWS];
#pragma unroll
  for (int p = 0; p < KROWS; ++p) s[p] = *(const float4*)(S + (rg + KRG * p) * KD);

  // ---- short convolution + SiLU: thread t < 128 takes channel t of q and k,
  //      threads 128 .. 159 the slice's 32 v channels.  Taps come from conv_in; the
  //      shifted taps go to conv_out (q and k by the head's first slice only)
  {
    auto conv = [&](int which, const uint16_t* x, int64_t ch, bool store) {
      const float* ci = a.conv_in + ((int64_t)b * 3 + which) * 3 * HD + ch;
      const float x0 = ci[0], x1 = ci[HD], x2 = ci[2 * HD];
      const float xt = bf16_to_f32(x[(int64_t)b * HD + ch]);
      const float4 w = *(const float4*)(a.conv_w + ((int64_t)which * HD + ch) * 4);
      if (store) {
        float* co = a.conv_out + ((int64_t)b * 3 + which) * 3 * HD + ch;
        co[0] = x1;
        co[HD] = x2;
        co[2 * HD] = xt;
      }
      return silu(fmaf(w.x, x0, fmaf(w.y, x1, fmaf(w.z, x2, w.w * xt))));
    };
    if (tid < KD) {
      const int64_t ch = (int64_t)h * KD + tid;
      const float qc = conv(0, a.xq, ch, sl == 0), kc = conv(1, a.xk, ch, sl == 0);
      const float sq = wave_sum_f(qc * qc), sk = wave_sum_f(kc * kc);
      if (lane == 0) { sh.nrm[wv][0] = sq; sh.nrm[wv][1] = sk; }
      sh.q[tid] = qc;
      sh.k[tid] = kc;
      sh.a[tid] = a.alpha[((int64_t)b * a.heads + h) * KD + tid];
    } else if (tid < KD + KSL) {
      const int c = tid - KD;
      sh.v[c] = conv(2, a.xv, (int64_t)h * KD + KSL * sl + c, true);
    }
  }
  __syncthreads();
  const float rq = rsqrtf(sh.nrm[0][0] + sh.nrm[1][0] + 1e-6f);
  const float rk = rsqrtf(sh.nrm[0][1] + sh.nrm[1][1] + 1e-6f);
  const float beta = a.beta[(int64_t)b * a.heads + h];

  // ---- decay the key channels, then u = S'^T k over this thread's rows
  float4 u = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int p = 0; p < KROWS; ++p) {
    const int i = rg + KRG * p;
    const float al = sh.a[i], ki = sh.k[i] * rk;
    s[p] = make_float4(s[p].x * al, s[p].y * al, s[p].z * al, s[p].w * al);
    u = make_float4(fmaf(ki, s[p].x, u.x), fmaf(ki, s[p].y, u.y), fmaf(ki, s[p].z, u.z), fmaf(ki, s[p].w, u.w));
  }
  u = column_sums(u, sh);
  // ---- delta write, then o = S^T q over this thread's rows
  const float4 v4 = *(const float4*)&sh.v[4 * col4];
  const float4 d = make_float4(beta * (v4.x - u.x), beta * (v4.y - u.y), beta * (v4.z - u.z), beta * (v4.w - u.w));
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int p = 0; p < KROWS; ++p) {
    const int i = rg + KRG * p;
    const float ki = sh.k[i] * rk, qi = sh.q[i] * rq;
    s[p] = make_float4(fmaf(ki, d.x, s[p].x), fmaf(ki, d.y, s[p].y), fmaf(ki, d.z, s[p].z), fmaf(ki, d.w, s[p].w));
    o = make_float4(fmaf(qi, s[p].x, o.x), fmaf(qi, s[p].y, o.y), fmaf(qi, s[p].z, o.z), fmaf(qi, s[p].w, o.w));
    // streamed: the state leaves the die's L2 as it is written, not at the launch's end
    __builtin_nontemporal_store(f32x4_t{s[p].x, s[p].y, s[p].z, s[p].w}, (f32x4_t*)(S + i * KD));
  }
  __syncthreads();                   // every wave has read red[] (u) before it is rewritten
  o = column_sums(o, sh);
  if (tid < KSL / 4) {
    const float sc = rsqrtf((float)KD);
    *(float4*)(a.out + ((int64_t)b * a.heads + h) * KD + KSL * sl + 4 * col4) =
        make_float4(o.x * sc, o.y * sc, o.z * sc, o.w * sc);
  }
}

// ------------------------------------------------------------------ chunked form (prefill)
// The same recurrence over n_tokens consecutive tokens, 16 at a time.  Within a
// block of C = 16 tokens that starts from state S0, let G_i = sum_{m <= i} log
// alpha_m (per key channel, running over the block).  Unrolling the token steps
// gives exactly
//   u_i = beta_i (v_i - S0^T (k_i e^{G_i}) - sum_{j<i} A_ij u_j),
//         A_ij = sum_c k_i[c] k_j[c] e^{G_i[c] - G_j[c]}       (a lower-triangular solve)
//   o_i = (S0^T (q_i e^{G_i}) + sum_{j<=i} B_ij u_j) / sqrt(128),
//         B_ij = sum_c q_i[c] k_j[c] e^{G_i[c] - G_j[c]}
//   S   = Diag(e^{G_last}) S0 + sum_j (k_j e^{G_last - G_j}) u_j^T,
// where u_i is the delta-rule write of token i (S_i = Diag(alpha_i) S_{i-1} + k_i u_i^T).
// The products with S0, the outputs and the state update are dense contractions
// on fp32 MFMA (v_mfma_f32_16x16x4_f32).  A and B are (k e^G)(k e^-G)^T and
// (q e^G)(k e^-G)^T -- unless some e^-G of the block would leave fp32's range (a
// cumulative decay below 2^-115 inside 16 tokens), in which case they are summed
// term by term with e^{G_i - G_j} <= 1.  G is kept in base 2 (running sums of
// log2 alpha from v_log_f32, powers from v_exp_f32).  One workgroup per (head, 32-column slice,
// sequence), as in the decode step; the blocks of a sequence run in order inside it,
// the state slice staying in LDS.  Tokens past the end of the last block enter with
// zero input, alpha = 1 and beta = 0, which leaves the state and the taps unchanged.
constexpr int CC = 16;               // tokens per block
constexpr int CP = KD + 4;           // row of q~, k~, k^ (16-byte reads of 4 channels by 16 x 4 lanes)
constexpr int KBP = KD + 16;         // row of k-bar (read [token][channel] by 4 x 16 lanes)
constexpr int SP = KSL + 16;         // row of u
constexpr int STP = KD + 4;          // row of the transposed state slice: column c of S holds S[.][c]
constexpr float G_SAFE = -115.f;          // log2 of the decay: 2^115 stays inside fp32

typedef float f32x4_t __attribute__((ext_vector_type(4)));

struct __align__(16) KdaChunkShared {
  float hx[3][3][KD];                // conv taps x_{t-3 .. t-1}: q, k (128 channels), v (first 32)
  float yq[CC][KD], yk[CC][KD];      // raw inputs, then conv + SiLU
  float yv[CC][KSL];                 // raw v inputs
  float g[CC][KD];                   // log2 alpha, then its running sum (G in base 2)
  float qt[CC][CP], kt[CC][CP], kh[CC][CP];
  float kb[CC][KBP];
  float St[KSL][STP];                // the state slice, transposed: St[c][k] = S[k][c]
  float A[2][CC][CC], B[2][CC][CC];  // halves over channels 0..63, 64..127
  float U[CC][SP];                   // conv + SiLU of v, then v - S0^T k~, then u
  float gl[KD];                      // e^{G_last}
  float beta[CC], rq[CC], rk[CC];
  int unsafe;
};

// x[k] of a register array for a k known only at run time (compares, no indexing)
template <int N>
__device__ __forceinline__ float pick_tap(const float (&x)[N], int k) {
  float v = x[0];
#pragma unroll
  for (int i = 1; i < N; ++i) v = i == k ? x[i] : v;
  return v;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__global__ __launch_bounds__(KT) void kda_chunk_kernel(KdaChunkArgs a) {
  __shared__ KdaChunkShared sh;
  const int h = blockIdx.x / KNS, sl = blockIdx.x % KNS, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r16 = lane & 15, kq = lane >> 4;
  const int64_t HD = (int64_t)a.heads * KD;
  const int T = a.n_tokens;
  float* Sg = a.state + ((int64_t)b * a.heads + h) * KD * KD + KSL * sl;

  // ---- the state slice and the conv taps in
  for (int i = tid; i < KD * KSL / 4; i += KT) {
    const int row = i / (KSL / 4), c4 = i % (KSL / 4);
    const float4 v = *(const float4*)(Sg + (int64_t)row * KD + 4 * c4);
    sh.St[4 * c4][row] = v.x;
    sh.St[4 * c4 + 1][row] = v.y;
    sh.St[4 * c4 + 2][row] = v.z;
    sh.St[4 * c4 + 3][row] = v.w;
  }
  for (int i = tid; i < 3 * 3 * KD; i += KT) {
    const int w = i / (3 * KD), m = (i / KD) % 3, c = i % KD;
    if (w < 2 || c < KSL)
      sh.hx[w][m][c] = a.conv_in[((int64_t)b * 3 + w) * 3 * HD + m * HD + (int64_t)h * KD + (w < 2 ? c : KSL * sl + c)];
  }
  // conv weights: thread t takes channel t % 128 of q (t < 128) or k; threads < 32 also
  // the slice's v channel t
  const int cw = tid >> 7, cc = tid & (KD - 1);
  const float4 wqk = *(const float4*)(a.conv_w + ((int64_t)cw * HD + (int64_t)h * KD + cc) * 4);
  const float4 wv4c = *(const float4*)(a.conv_w + (2 * HD + (int64_t)h * KD + KSL * sl + (tid & (KSL - 1))) * 4);
  const float rs = rsqrtf((float)KD);

  // the inputs of a block, fetched into registers one block ahead: x (zero past the
  // chunk's end), alpha (1 past it), beta (0 past it)
  const int fi = tid >> 4, fc0 = 8 * (tid & 15);           // q, k: token, channels
  const int fiv = tid >> 2, fv0 = 8 * (tid & 3);           // v (threads < 64)
  u32x4_t pxq, pxk, pxv;
  float4 pal[2];
  float pbeta = 0.f;
  auto fetch = [&](int t0) {
    const int n = min(CC, T - t0);
    pxq = u32x4_t{0u, 0u, 0u, 0u};
    pxk = u32x4_t{0u, 0u, 0u, 0u};
    pxv = u32x4_t{0u, 0u, 0u, 0u};
    if (fi < n) {
      const int64_t off = ((int64_t)b * T + t0 + fi) * HD + (int64_t)h * KD + fc0;
      pxq = *(const u32x4_t*)(a.xq + off);
      pxk = *(const u32x4_t*)(a.xk + off);
    }
    if (tid < CC * KSL / 8 && fiv < n)
      pxv = *(const u32x4_t*)(a.xv + ((int64_t)b * T + t0 + fiv) * HD + (int64_t)h * KD + KSL * sl + fv0);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int idx = tid + KT * k, ia = idx >> 5, c4 = idx & 31;
      pal[k] = make_float4(1.f, 1.f, 1.f, 1.f);
      if (ia < n) pal[k] = *(const float4*)(a.alpha + (((int64_t)b * T + t0 + ia) * a.heads + h) * KD + 4 * c4);
    }
    if (tid < CC) pbeta = tid < n ? a.beta[((int64_t)b * T + t0 + tid) * a.heads + h] : 0.f;
  };
  // 16-byte LDS stores (8 channels of a token per thread, 4 log2 alpha per store)
  auto widen8 = [](const u32x4_t& x, float* dst) {
    *(float4*)dst = make_float4(bf16_lo(x[0]), bf16_hi(x[0]), bf16_lo(x[1]), bf16_hi(x[1]));
    *(float4*)(dst + 4) = make_float4(bf16_lo(x[2]), bf16_hi(x[2]), bf16_lo(x[3]), bf16_hi(x[3]));
  };
  auto stage = [&]() {
    widen8(pxq, &sh.yq[fi][fc0]);
    widen8(pxk, &sh.yk[fi][fc0]);
    if (tid < CC * KSL / 8) widen8(pxv, &sh.yv[fiv][fv0]);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int idx = tid + KT * k, ia = idx >> 5, c4 = idx & 31;
      *(float4*)&sh.g[ia][4 * c4] = make_float4(__builtin_amdgcn_logf(pal[k].x), __builtin_amdgcn_logf(pal[k].y),
                                                __builtin_amdgcn_logf(pal[k].z), __builtin_amdgcn_logf(pal[k].w));
    }
    if (tid < CC) sh.beta[tid] = pbeta;
    if (tid == 0) sh.unsafe = 0;
  };
  // block 0's inputs staged, block 1's in flight; a block's inputs are staged during
  // the previous block's substitution (by the threads it leaves idle) and just after it
  if (T > 0) {
    fetch(0);
    stage();
    if (CC < T) fetch(CC);
  }

  // LDS-only barriers inside the loop (block_sync_lds): the next block's loads stay
  // in flight across them
  for (int t0 = 0; t0 < T; t0 += CC) {
    const int n = min(CC, T - t0);
    const bool more = t0 + CC < T;               // a next block to stage
    auto stage_next = [&]() {
      stage();
      if (t0 + 2 * CC < T) fetch(t0 + 2 * CC);
    };
    block_sync_lds();                            // the block's inputs are staged
    // ---- short convolution + SiLU in place, taps sliding in registers (the taps after
    //      the block are the last 3 inputs up to token n-1); the running sum G
    {
      // every output of the block is independent of the others (the taps are inputs):
      // the 16 tokens of a channel are read, convolved and written unrolled
      float (*y)[KD] = cw ? sh.yk : sh.yq;
      {
        float x[CC + 3];
        x[0] = sh.hx[cw][0][cc];
        x[1] = sh.hx[cw][1][cc];
        x[2] = sh.hx[cw][2][cc];
#pragma unroll
        for (int i = 0; i < CC; ++i) x[i + 3] = y[i][cc];
#pragma unroll
        for (int i = 0; i < CC; ++i)
          y[i][cc] = silu(fmaf(wqk.x, x[i], fmaf(wqk.y, x[i + 1], fmaf(wqk.z, x[i + 2], wqk.w * x[i + 3]))));
        // the taps after the block: inputs n-3 .. n-1 (n = tokens of the block)
        sh.hx[cw][0][cc] = pick_tap(x, n);
        sh.hx[cw][1][cc] = pick_tap(x, n + 1);
        sh.hx[cw][2][cc] = pick_tap(x, n + 2);
      }
      // the slice's v channels: thread -> channel t % 32, tokens 2 (t / 32) and the next,
      // into U (yv keeps the raw inputs; their taps move on in the next phase)
      {
        const int c = tid & (KSL - 1), i0 = 2 * (tid >> 5);
        float x[5];
#pragma unroll
        for (int m = 0; m < 5; ++m) {
          const int j = i0 - 3 + m;                  // input token (negative: a tap)
          const float in = sh.yv[max(j, 0)][c], tap = sh.hx[2][min(j + 3, 2)][c];
          x[m] = j >= 0 ? in : tap;
        }
        const float4 w = wv4c;
#pragma unroll
        for (int m = 0; m < 2; ++m)
          sh.U[i0 + m][c] = silu(fmaf(w.x, x[m], fmaf(w.y, x[m + 1], fmaf(w.z, x[m + 2], w.w * x[m + 3]))));
      }
      if (tid < KD) {
        float gv[CC];
#pragma unroll
        for (int i = 0; i < CC; ++i) gv[i] = sh.g[i][tid];
#pragma unroll
        for (int i = 1; i < CC; ++i) gv[i] += gv[i - 1];
#pragma unroll
        for (int i = 0; i < CC; ++i) sh.g[i][tid] = gv[i];
      }
    }
    block_sync_lds();
    // ---- 1 / norms of q and k and the decayed operands: thread -> token t / 16,
    //      channels 8(t % 16) .. +7 (all reads issued together, 16-byte LDS accesses);
    //      the 16 lanes of a token sum its squares
    {
      const int i = tid >> 4, c0 = 8 * (tid & 15);
      float G[8], GL[8], q[8], k[8];
      auto ld8 = [](const float* p, float (&d)[8]) {
        const float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
        d[0] = a.x; d[1] = a.y; d[2] = a.z; d[3] = a.w; d[4] = b.x; d[5] = b.y; d[6] = b.z; d[7] = b.w;
      };
      ld8(&sh.g[i][c0], G);
      ld8(&sh.g[CC - 1][c0], GL);
      ld8(&sh.yq[i][c0], q);
      ld8(&sh.yk[i][c0], k);
      float sq = 0.f, sk = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        sq = fmaf(q[e], q[e], sq);
        sk = fmaf(k[e], k[e], sk);
      }
#pragma unroll
      for (int m = 1; m < 16; m <<= 1) {
        sq += __shfl_xor(sq, m);
        sk += __shfl_xor(sk, m);
      }
      const float nq = rsqrtf(sq + 1e-6f), nk = rsqrtf(sk + 1e-6f);
      if ((tid & 15) == 0) {
        sh.rq[i] = nq;                           // for the term-by-term coefficients
        sh.rk[i] = nk;
      }
      float qt[8], kt[8], kh[8], kb[8], eg[8];
      bool bad = false;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float qq = q[e] * nq, kk = k[e] * nk;
        eg[e] = __builtin_amdgcn_exp2f(G[e]);
        qt[e] = qq * eg[e];
        kt[e] = kk * eg[e];
        kh[e] = kk * __builtin_amdgcn_exp2f(-G[e]);
        kb[e] = kk * __builtin_amdgcn_exp2f(GL[e] - G[e]);
        bad |= GL[e] < G_SAFE;
      }
#pragma unroll
      for (int e = 0; e < 8; e += 4) {
        *(float4*)&sh.qt[i][c0 + e] = make_float4(qt[e], qt[e + 1], qt[e + 2], qt[e + 3]);
        *(float4*)&sh.kt[i][c0 + e] = make_float4(kt[e], kt[e + 1], kt[e + 2], kt[e + 3]);
        *(float4*)&sh.kh[i][c0 + e] = make_float4(kh[e], kh[e + 1], kh[e + 2], kh[e + 3]);
      }
      *(float4*)&sh.kb[i][c0] = make_float4(kb[0], kb[1], kb[2], kb[3]);
      *(float4*)&sh.kb[i][c0 + 4] = make_float4(kb[4], kb[5], kb[6], kb[7]);
      if (i == CC - 1) {
        *(float4*)&sh.gl[c0] = make_float4(eg[0], eg[1], eg[2], eg[3]);
        *(float4*)&sh.gl[c0 + 4] = make_float4(eg[4], eg[5], eg[6], eg[7]);
        if (bad) sh.unsafe = 1;
      }
      // the v taps after the block (every read of the old taps is done)
      if (tid < KSL) {
        float x[CC + 3];
        x[0] = sh.hx[2][0][tid];
        x[1] = sh.hx[2][1][tid];
        x[2] = sh.hx[2][2][tid];
#pragma unroll
        for (int j = 0; j < CC; ++j) x[j + 3] = sh.yv[j][tid];
        sh.hx[2][0][tid] = pick_tap(x, n);
        sh.hx[2][1][tid] = pick_tap(x, n + 1);
        sh.hx[2][2][tid] = pick_tap(x, n + 2);
      }
    }
    block_sync_lds();
    // ---- S0 products and the block coefficients on MFMA: waves 0 / 1 take k~ S0 for
    //      columns 16w .. +15 (then U = v - k~ S0), waves 2 / 3 keep q~ S0; then each
    //      wave one half (64 channels) of A (waves 0 / 1) or B (waves 2 / 3)
    f32x4_t r = {0.f, 0.f, 0.f, 0.f};
    {
      const int nt = wv & 1;
      const float (*lhs)[CP] = wv < 2 ? sh.kt : sh.qt;
      // the sum over channels runs in the order k = 32 kq + s (lane kq's channels
      // contiguous): one 16-byte read of each operand per four MFMAs
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < KD / 16; ++j) {
        const f32x4_t la = *(const f32x4_t*)&lhs[r16][32 * kq + 4 * j];
        const f32x4_t lb = *(const f32x4_t*)&sh.St[16 * nt + r16][32 * kq + 4 * j];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(la[e], lb[e], acc, 0, 0, 0);
      }
      if (wv < 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) sh.U[4 * kq + e][16 * nt + r16] -= acc[e];
      } else {
        r = acc;
      }
      const int k0 = 64 * nt;
      f32x4_t c2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < KD / 32; ++j) {
        const f32x4_t la = *(const f32x4_t*)&lhs[r16][k0 + 16 * kq + 4 * j];
        const f32x4_t lb = *(const f32x4_t*)&sh.kh[r16][k0 + 16 * kq + 4 * j];
#pragma unroll
        for (int e = 0; e < 4; ++e) c2 = __builtin_amdgcn_mfma_f32_16x16x4f32(la[e], lb[e], c2, 0, 0, 0);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 4 * kq + e;
        if (wv < 2) sh.A[nt][row][r16] = r16 < row ? c2[e] : 0.f;
        else sh.B[nt][row][r16] = r16 <= row ? c2[e] : 0.f;
      }
    }
    block_sync_lds();
    if (sh.unsafe) {
      // term by term: thread -> (i, j) = (t / 16, t % 16), e^{G_i - G_j} <= 1 for j <= i
      const int i = tid >> 4, j = tid & 15;
      if (j <= i) {
        const float nq = sh.rq[i], nki = sh.rk[i], nkj = sh.rk[j];
        float sa = 0.f, sb = 0.f;
        for (int c = 0; c < KD; ++c) {
          const float d = __builtin_amdgcn_exp2f(sh.g[i][c] - sh.g[j][c]);
          const float kj = sh.yk[j][c] * nkj;
          sa = fmaf(sh.yk[i][c] * nki * d, kj, sa);
          sb = fmaf(sh.yq[i][c] * nq * d, kj, sb);
        }
        if (j < i) {
          sh.A[0][i][j] = sa;
          sh.A[1][i][j] = 0.f;
        }
        sh.B[0][i][j] = sb;
        sh.B[1][i][j] = 0.f;
      }
      block_sync_lds();
    }
    // A as one matrix (its two channel halves summed, one entry per thread)
    sh.A[0][tid >> 4][tid & 15] += sh.A[1][tid >> 4][tid & 15];
    block_sync_lds();
    // ---- u by forward substitution: lanes 0 .. 31 of wave 0, one column each.  Each
    //      u_j goes into every later row's running sum at once (the same terms in the
    //      same order per row), so the dependent path is one fma and one multiply a row
    if (tid < KSL) {
      float p[CC], u[CC];
      float4 ar[CC][CC / 4];                    // A's rows, 16-byte reads (lower triangle used)
#pragma unroll
      for (int i = 0; i < CC; ++i) {
        p[i] = sh.U[i][tid];
#pragma unroll
        for (int q = 0; q < CC / 4; ++q)
          if (4 * q < i) ar[i][q] = *(const float4*)&sh.A[0][i][4 * q];
      }
      auto aij = [&](int i, int j) {
        const float4 v = ar[i][j >> 2];
        return (j & 3) == 0 ? v.x : ((j & 3) == 1 ? v.y : ((j & 3) == 2 ? v.z : v.w));
      };
#pragma unroll
      for (int j = 0; j < CC; ++j) {
        u[j] = sh.beta[j] * p[j];
#pragma unroll
        for (int i = j + 1; i < CC; ++i) p[i] = fmaf(-aij(i, j), u[j], p[i]);
      }
#pragma unroll
      for (int i = 0; i < CC; ++i) sh.U[i][tid] = u[i];
    } else if (more) {
      stage_next();                              // nothing below reads the staged buffers
    }
    block_sync_lds();
    if (tid < KSL && more) stage_next();
    // ---- outputs (waves 2 / 3): (q~ S0 + B u) / sqrt(128)
    if (wv >= 2) {
      const int nt = wv & 1;
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int s = 0; s < CC / 4; ++s)
          r = __builtin_amdgcn_mfma_f32_16x16x4f32(sh.B[hb][r16][4 * s + kq], sh.U[4 * s + kq][16 * nt + r16], r, 0, 0,
                                                   0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 4 * kq + e;
        if (row < n)
          a.out[(((int64_t)b * T + t0 + row) * a.heads + h) * KD + KSL * sl + 16 * nt + r16] = r[e] * rs;
      }
    }
    // ---- state update: S = Diag(e^{G_last}) S0 + k-bar^T u, tiles of 16 x 16, four per wave
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tile = 4 * wv + j, mt = tile >> 1, nt = tile & 1;
      // rows 16 mt + 4 kq .. +3 of column 16 nt + r16: one 16-byte piece of St
      f32x4_t* sp = (f32x4_t*)&sh.St[16 * nt + r16][16 * mt + 4 * kq];
      f32x4_t acc = *sp * *(const f32x4_t*)&sh.gl[16 * mt + 4 * kq];
#pragma unroll
      for (int s = 0; s < CC / 4; ++s)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(sh.kb[4 * s + kq][16 * mt + r16], sh.U[4 * s + kq][16 * nt + r16], acc,
                                                  0, 0, 0);
      *sp = acc;
    }
  }
  block_sync_lds();
  // ---- the state slice and the taps out (q and k taps by the head's first slice)
  for (int i = tid; i < KD * KSL / 4; i += KT) {
    const int row = i / (KSL / 4), c4 = i % (KSL / 4);
    *(float4*)(Sg + (int64_t)row * KD + 4 * c4) =
        make_float4(sh.St[4 * c4][row], sh.St[4 * c4 + 1][row], sh.St[4 * c4 + 2][row], sh.St[4 * c4 + 3][row]);
  }
  for (int i = tid; i < 3 * 3 * KD; i += KT) {
    const int w = i / (3 * KD), m = (i / KD) % 3, c = i % KD;
    if ((w < 2 && sl == 0) || (w == 2 && c < KSL))
      a.conv_out[((int64_t)b * 3 + w) * 3 * HD + m * HD + (int64_t)h * KD + (w < 2 ? c : KSL * sl + c)] = sh.hx[w][m][c];
  }
}

}  // namespace

hipError_t launch_kda_chunk(const KdaChunkArgs& a, hipStream_t s) {
  if (a.batch <= 0 || a.heads <= 0) return hipSuccess;
  launch(K_KDA, kda_chunk_kernel, dim3(a.heads * KNS, a.batch), dim3(KT), s, a);
  return hipGetLastError();
}

hipError_t launch_kda_decode(const KdaArgs& a, hipStream_t s) {
  if (a.batch <= 0 || a.heads <= 0) return hipSuccess;
  launch(K_KDA, kda_decode_kernel, dim3(a.heads * KNS, a.batch), dim3(KT), s, a);
  return hipGetLastError();
}

}  // namespace ip
