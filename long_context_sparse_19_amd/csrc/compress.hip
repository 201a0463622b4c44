// IndexPool: weighted pooling of every 4 cached indexer keys into 1.
// Reading notes "GLM-5.3-Flash: Hybrid Attention, IndexPool, and Vision-in-the-Loop",
// section 2, sub-section "IndexPool" (learned weights instead of QSA's plain mean;
// the resident indexer state drops 4x); FP8 cache tier from section 4, "The serving
// stack".  Weights are the softmax of one logit per token within its block.
//
// A pure stream: each block reads 4 key rows (+4 scales, +4 logits) and writes one
// row (+1 scale).  Sixteen lanes cover one 128-byte fp8 row (8 codes per lane), so
// every wave touches whole, consecutive rows.
#include "kernels.hpp"

namespace ip {

namespace {

constexpr int NT = 256;

__device__ __forceinline__ void softmax4(const float* lg, float* w) {
  const float m = fmaxf(fmaxf(lg[0], lg[1]), fmaxf(lg[2], lg[3]));
  float e[4], s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) { e[i] = expf(lg[i] - m); s += e[i]; }
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = e[i] / s;
}

// D = 128 fp8 codes per row; 16 lanes per block, 16 blocks per workgroup.
__global__ __launch_bounds__(NT) void compress_fp8_kernel(CompressArgs a) {
  constexpr int LPB = 16;                      // lanes per block
  constexpr int BPW = NT / LPB;                // blocks per workgroup
  const int b = blockIdx.y;
  const int sub = threadIdx.x % LPB;
  const int seq_blocks = a.L.seq_lens[b] >> 2;
  const int begin = a.block_begin ? a.block_begin[b] : 0;
  const int end = min(begin + a.max_blocks, seq_blocks);
  const int j = begin + blockIdx.x * BPW + threadIdx.x / LPB;
  if (begin + (int)blockIdx.x * BPW >= end) return;   // whole workgroup idle
  const bool valid = j < end;

  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int64_t prow = 0;
  if (valid) {
    prow = a.L.pool_row(b, j);
    const int64_t t0 = prow * 4;               // token rows 4r .. 4r+3
    float lg[4], sc[4], w[4];
    uint2 c[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      c[i] = *(const uint2*)(a.keys + (t0 + i) * a.key_stride + sub * 8);
      lg[i] = a.logits[t0 + i];
      sc[i] = a.key_scale[t0 + i];
    }
    softmax4(lg, w);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float coef = w[i] * sc[i];
      float f[8];
      fp8x4_to_f32(c[i].x, f);
      fp8x4_to_f32(c[i].y, f + 4);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(coef, f[e], acc[e]);
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(acc[e]));
#pragma unroll
  for (int o = LPB / 2; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, LPB));
  if (!valid) return;

  const float sigma = amax / 448.0f;
  uint32_t lo = 0, hi = 0;
  if (amax > 0.f) {
    const float inv = 448.0f / amax;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float y0 = fminf(fmaxf(acc[e] * inv, -448.f), 448.f);
      const float y1 = fminf(fmaxf(acc[e + 4] * inv, -448.f), 448.f);
      lo |= f32_to_e4m3(y0) << (8 * e);
      hi |= f32_to_e4m3(y1) << (8 * e);
    }
  }
  *(uint2*)(a.out + prow * a.out_stride + sub * 8) = make_uint2(lo, hi);
  if (sub == 0) a.out_scale[prow] = sigma;
}

// float keys, dim <= 256 and a multiple of 4: one thread per (block, 4 elements).
__global__ __launch_bounds__(NT) void compress_f32_kernel(CompressArgs a) {
  const int b = blockIdx.y;
  const int q4 = a.dim >> 2;
  const int seq_blocks = a.L.seq_lens[b] >> 2;
  const int begin = a.block_begin ? a.block_begin[b] : 0;
  const int end = min(begin + a.max_blocks, seq_blocks);
  const int64_t idx = (int64_t)blockIdx.x * NT + threadIdx.x;
  const int64_t j = begin + idx / q4;
  const int e4 = (int)(idx % q4);
  if (j >= end) return;
  const int64_t prow = a.L.pool_row(b, j);
  const int64_t t0 = prow * 4;
  float lg[4], w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) lg[i] = a.logits[t0 + i];
  softmax4(lg, w);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 k = *(const float4*)(a.keys + (t0 + i) * a.key_stride + e4 * 16);
    acc.x = fmaf(w[i], k.x, acc.x);
    acc.y = fmaf(w[i], k.y, acc.y);
    acc.z = fmaf(w[i], k.z, acc.z);
    acc.w = fmaf(w[i], k.w, acc.w);
  }
  *(float4*)(a.out + prow * a.out_stride + e4 * 16) = acc;
}

// ---------------------------------------------------------------- decode append
// One workgroup per sequence writes its new token (position seq_lens[b] - 1) into
// the caches and, when that token completes a block, pools the block.  The new
// key's codes and scale stay in registers for the pooling, which follows the same
// arithmetic, in the same order, as compress_fp8_kernel / compress_f32_kernel.
constexpr int APPEND_MAX_DIM = 256;
__global__ __launch_bounds__(NT) void append_kernel(AppendArgs a) {
  __shared__ float red[NT / 64];
  const int b = blockIdx.x;
  const int len = a.L.seq_lens[b];
  if (len < 1) return;
  const int64_t t = len - 1;
  const int64_t row = a.L.tok_row(b, t);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  // latent (or K) and V rows: plain 16-byte copies (the fp8 latent tier below)
  if (!a.kv_scale)
    for (int i = tid; i < a.kv_row_bytes / 16; i += NT)
      *(uint4*)(a.kv + row * a.kv_stride + 16 * i) = *(const uint4*)(a.kv_new + (int64_t)b * a.kv_row_bytes + 16 * i);
  if (a.v)
    for (int i = tid; i < a.v_row_bytes / 16; i += NT)
      *(uint4*)(a.v + row * a.v_stride + 16 * i) = *(const uint4*)(a.v_new + (int64_t)b * a.v_row_bytes + 16 * i);
  auto block_max = [&](float v) {                // max over the workgroup (all threads call)
    v = wave_max(v);
    if (lane == 0) red[wv] = v;
    __syncthreads();
    float m = red[0];
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) m = fmaxf(m, red[w]);
    __syncthreads();
    return m;
  };
  // fp8 latent tier: the bf16 latent row quantised per token like the keys
  // (sigma = amax / 448); thread i takes values 4i .. 4i+3
  if (a.kv_scale) {
    const bool kon = 4 * tid < a.kv_dim;
    float kx[4] = {0.f, 0.f, 0.f, 0.f};
    if (kon) {
      const uint2 w = *(const uint2*)(a.kv_new + ((int64_t)b * a.kv_dim + 4 * tid) * 2);
      kx[0] = __uint_as_float(w.x << 16);
      kx[1] = __uint_as_float(w.x & 0xFFFF0000u);
      kx[2] = __uint_as_float(w.y << 16);
      kx[3] = __uint_as_float(w.y & 0xFFFF0000u);
    }
    const float kamax = block_max(fmaxf(fmaxf(fabsf(kx[0]), fabsf(kx[1])), fmaxf(fabsf(kx[2]), fabsf(kx[3]))));
    uint32_t packed = 0;
    if (kamax > 0.f) {
      const float inv = 448.0f / kamax;
#pragma unroll
      for (int i = 0; i < 4; ++i) packed |= f32_to_e4m3(fminf(fmaxf(kx[i] * inv, -448.f), 448.f)) << (8 * i);
    }
    if (kon) *(uint32_t*)(a.kv + row * a.kv_stride + 4 * tid) = packed;
    if (tid == 0) a.kv_scale[row] = kamax / 448.0f;
  }
  if (!a.keys) return;                           // a layer without indexer state (uniform)
  const bool on = tid < a.dim;
  float x = 0.f;
  if (on)
    x = a.key_bf16 ? bf16_to_f32(((const uint16_t*)a.key_new)[(int64_t)b * a.dim + tid])
                   : ((const float*)a.key_new)[(int64_t)b * a.dim + tid];
  const float lnew = a.logit_new[b];
  if (tid == 0) a.logits[row] = lnew;
  const bool fp8 = a.key_scale != nullptr;
  // the new token's key: fp8 with sigma = amax / 448, or the float key as is
  uint32_t code = 0;
  float sigma = 0.f;
  if (fp8) {
    const float amax = block_max(on ? fabsf(x) : 0.f);
    sigma = amax / 448.0f;
    if (amax > 0.f) code = f32_to_e4m3(fminf(fmaxf(x * (448.0f / amax), -448.f), 448.f));
    if (on) a.keys[row * a.key_stride + tid] = (uint8_t)code;
    if (tid == 0) a.key_scale[row] = sigma;
  } else if (on) {
    ((float*)(a.keys + row * a.key_stride))[tid] = x;
  }
  if ((len & 3) != 0) return;                    // uniform: no block completed
  // block t/4: tokens t-3 .. t (the block's rows are contiguous)
  const int64_t r0 = row - 3;
  const int64_t prow = a.L.pool_row(b, t >> 2);
  float lg[4], w[4];
#pragma unroll
  for (int i = 0; i < 3; ++i) lg[i] = a.logits[r0 + i];
  lg[3] = lnew;
  softmax4(lg, w);
  if (fp8) {
    float acc = 0.f;
    if (on) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float sc = i < 3 ? a.key_scale[r0 + i] : sigma;
        const uint32_t c = i < 3 ? a.keys[(r0 + i) * a.key_stride + tid] : code;
        float f[4];
        fp8x4_to_f32(c, f);
        acc = fmaf(w[i] * sc, f[0], acc);
      }
    }
    const float amax = block_max(on ? fabsf(acc) : 0.f);
    uint32_t pc = 0;
    if (amax > 0.f) pc = f32_to_e4m3(fminf(fmaxf(acc * (448.0f / amax), -448.f), 448.f));
    if (on) a.pooled[prow * a.pooled_stride + tid] = (uint8_t)pc;
    if (tid == 0) a.pooled_scale[prow] = amax / 448.0f;
  } else if (on) {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float k = i < 3 ? ((const float*)(a.keys + (r0 + i) * a.key_stride))[tid] : x;
      acc = fmaf(w[i], k, acc);
    }
    ((float*)(a.pooled + prow * a.pooled_stride))[tid] = acc;
  }
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, hipStream_t s) {
  if (a.batch <= 0) return hipSuccess;
  if (a.dim > APPEND_MAX_DIM || (a.kv_scale && (a.kv_dim % 4 || a.kv_dim > 4 * NT))) return hipErrorInvalidValue;
  launch(K_APPEND, append_kernel, dim3(a.batch), dim3(NT), s, a);
  return hipGetLastError();
}

hipError_t launch_compress_fp8(const CompressArgs& a, hipStream_t s) {
  if (a.max_blocks <= 0) return hipSuccess;
  dim3 grid((a.max_blocks + 15) / 16, a.batch);
  launch(K_COMPRESS, compress_fp8_kernel, grid, dim3(NT), s, a);
  return hipGetLastError();
}

hipError_t launch_compress_f32(const CompressArgs& a, hipStream_t s) {
  if (a.max_blocks <= 0) return hipSuccess;
  const int64_t threads = (int64_t)a.max_blocks * (a.dim / 4);
  dim3 grid((unsigned)((threads + NT - 1) / NT), a.batch);
  launch(K_COMPRESS, compress_f32_kernel, grid, dim3(NT), s, a);
  return hipGetLastError();
}

}  // namespace ip
