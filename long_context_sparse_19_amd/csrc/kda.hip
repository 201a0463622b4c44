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

__device__ __forceinline__ float silu(float x) { return x / (1.f + __expf(-x)); }

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
    *(float4*)(S + i * KD) = s[p];
  }
  __syncthreads();                   // every wave has read red[] (u) before it is rewritten
  o = column_sums(o, sh);
  if (tid < KSL / 4) {
    const float sc = rsqrtf((float)KD);
    *(float4*)(a.out + ((int64_t)b * a.heads + h) * KD + KSL * sl + 4 * col4) =
        make_float4(o.x * sc, o.y * sc, o.z * sc, o.w * sc);
  }
}

}  // namespace

hipError_t launch_kda_decode(const KdaArgs& a, hipStream_t s) {
  if (a.batch <= 0 || a.heads <= 0) return hipSuccess;
  launch(K_KDA, kda_decode_kernel, dim3(a.heads * KNS, a.batch), dim3(KT), s, a);
  return hipGetLastError();
}

}  // namespace ip
