// Decode cache growth for one sequence, shared by the append kernel and by the
// scoring kernel's fused form (extra workgroups of the scoring launch: scoring never
// reads what the append writes, see index_score_topk's fused entry point).
#pragma once
#include "kernels.hpp"

namespace ip {

constexpr int APPEND_NT = 256;           // threads of the append kernel's workgroups
constexpr int APPEND_MAX_DIM = 256;

__device__ __forceinline__ void softmax4(const float* lg, float* w) {
  const float m = fmaxf(fmaxf(lg[0], lg[1]), fmaxf(lg[2], lg[3]));
  float e[4], s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) { e[i] = expf(lg[i] - m); s += e[i]; }
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = e[i] / s;
}

// One workgroup per sequence writes its new token (position seq_lens[b] - 1) into
// the caches and, when that token completes a block, pools the block.  The new
// key's codes and scale stay in registers for the pooling, which follows the same
// arithmetic, in the same order, as compress_fp8_kernel / compress_f32_kernel.
// NT: the workgroup's threads (at least 256: one key dim per thread, 4 latent
// values per thread), all of which call it.
template <int NT = APPEND_NT>
__device__ __forceinline__ void append_one(const AppendArgs& a, int b) {
  static_assert(NT >= 256 && NT % 64 == 0, "append workgroup size");
  __shared__ float red[NT / 64];
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

}  // namespace ip
