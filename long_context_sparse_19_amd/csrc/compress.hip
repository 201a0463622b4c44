// IndexPool: weighted pooling of every 4 cached indexer keys into 1.
// Reading notes "GLM-5.3-Flash: Hybrid Attention, IndexPool, and Vision-in-the-Loop",
// section 2, sub-section "IndexPool" (learned weights instead of QSA's plain mean;
// the resident indexer state drops 4x); FP8 cache tier from section 4, "The serving
// stack".  Weights are the softmax of one logit per token within its block.
//
// A pure stream: each block reads 4 key rows (+4 scales, +4 logits) and writes one
// row (+1 scale).  Sixteen lanes cover one 128-byte fp8 row (8 codes per lane), so
// every wave touches whole, consecutive rows.
#include "append.hpp"

namespace ip {

namespace {

constexpr int NT = 256;

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
// One workgroup per sequence (append_one, shared with the fused form in the
// scoring kernel).
__global__ __launch_bounds__(APPEND_NT) void append_kernel(AppendArgs a) { append_one(a, blockIdx.x); }

}  // namespace

hipError_t launch_append(const AppendArgs& a, hipStream_t s) {
  if (a.batch <= 0) return hipSuccess;
  if (a.dim > APPEND_MAX_DIM || (a.kv_scale && (a.kv_dim % 4 || a.kv_dim > 4 * APPEND_NT))) return hipErrorInvalidValue;
  launch(K_APPEND, append_kernel, dim3(a.batch), dim3(APPEND_NT), s, a);
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
