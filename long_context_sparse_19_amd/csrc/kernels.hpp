// Host-side launch interface of the gfx950 kernels (internal to libindexpool).
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>
#include <algorithm>
#include "common.hpp"

namespace ip {

enum KernelId { K_COMPRESS = 1, K_SCORE = 2, K_TOPK = 3, K_ATTN = 4, K_COMBINE = 5, K_APPEND = 6, K_KDA = 7, K_LAST = 7 };

// Takes (and disarms) the timing hook's events if one is armed for kernel `id`.
bool hook_take(int id, hipEvent_t* start, hipEvent_t* stop);

// Launches kernel `id`.  When the timing hook is armed for it, the launch goes
// through hipExtLaunchKernelGGL, which stores the dispatch's own start and end
// times in the two events (the same timestamps a kernel trace reports).
template <typename K, typename... Args>
void launch(int id, K kernel, dim3 grid, dim3 block, hipStream_t s, Args... args) {
  hipEvent_t e0, e1;
  if (hook_take(id, &e0, &e1))
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, e0, e1, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
}

// ------------------------------------------------------------ IndexPool
struct CompressArgs {
  Layout L;
  int batch;
  const int32_t* block_begin;  // [batch] or null
  int max_blocks;              // blocks per sequence covered by the grid
  const uint8_t* keys;         // token key rows
  int64_t key_stride;          // bytes
  const float* key_scale;      // [token rows] (fp8) or null
  const float* logits;         // [token rows]
  uint8_t* out;                // pooled rows
  int64_t out_stride;          // bytes
  float* out_scale;            // [pooled rows] (fp8) or null
  int dim;                     // elements per key row
};
hipError_t launch_compress_fp8(const CompressArgs& a, hipStream_t s);
hipError_t launch_compress_f32(const CompressArgs& a, hipStream_t s);

// ------------------------------------------------------------ decode cache append
struct AppendArgs {
  Layout L;
  int batch;
  const uint8_t* kv_new;       // [batch, kv_row_bytes]
  uint8_t* kv;                 // token rows
  int64_t kv_stride;
  int kv_row_bytes;            // a multiple of 16 (bytes copied when kv_scale is null)
  float* kv_scale;             // fp8 latent tier: [token rows] scales, kv_new is bf16
  int kv_dim;                  // fp8 latent tier: values per row (a multiple of 4, <= 1024)
  const uint8_t* v_new;        // [batch, v_row_bytes] or null
  uint8_t* v;
  int64_t v_stride;
  int v_row_bytes;
  const void* key_new;         // [batch, dim], bf16 or f32
  int key_bf16;
  uint8_t* keys;               // token key rows: fp8 codes (+ key_scale) or f32; null: the
                               // layer keeps no indexer state (only kv / v are written)
  int64_t key_stride;
  float* key_scale;            // [token rows] (fp8) or null
  int dim;
  const float* logit_new;      // [batch]
  float* logits;               // [token rows]
  uint8_t* pooled;             // pooled rows
  int64_t pooled_stride;
  float* pooled_scale;         // [pooled rows] (fp8) or null
};
hipError_t launch_append(const AppendArgs& a, hipStream_t s);

// ------------------------------------------------------------ indexer scoring
struct ScoreArgs {
  Layout L;
  int row0, n_rows;            // query rows [row0, row0 + n_rows)
  const int32_t* q_seq;        // [n_q] or null
  const int32_t* q_pos;        // [n_q] or null
  const void* q;               // [n_q, heads, dim]
  const float* gates;          // [n_q, heads]
  const uint8_t* keys;         // pooled rows
  int64_t key_stride;
  const float* key_scale;      // [pooled rows] (fp8) or null
  float* scores;               // [n_rows, ld], row r - row0
  int64_t ld;
  int heads, dim;
  int max_blocks;              // key range covered by the grid
  int32_t* topk_count;         // [n_rows] or null: zeroed here for the top-k that follows
  int with_append;             // decode: extra grid rows of workgroups run `append`,
  AppendArgs append;           // one sequence each (see append.hpp)
};
hipError_t launch_score_fp8_bf16(const ScoreArgs& a, hipStream_t s);
hipError_t launch_score_f32(const ScoreArgs& a, hipStream_t s);

// ------------------------------------------------------------ top-k selection
struct TopkArgs {
  Layout L;
  int row0, n_rows;
  const int32_t* q_seq;
  const int32_t* q_pos;
  const float* scores;         // [n_rows, ld]
  int64_t ld;
  int top_k;
  int32_t* out;                // [n_q, top_k], row r
  uint32_t* cand_key;          // [n_rows, n_chunks, top_k - 1]
  int32_t* cand_idx;           // same
  int n_chunks;                // chunks per row covered by the grid
  int chunk;                   // scores per chunk (topk_chunk_size)
  int32_t* count;              // [n_rows] chunks done per row, zero on entry (n_chunks > 1)
};
constexpr int TOPK_MAX_CHUNK = 16384;   // scores per chunk workgroup (512 threads x 32)
constexpr int TOPK_MERGE_CAP = 16384;   // candidate slots per row in the in-kernel merge (512 x 32)
int topk_chunk_size(int max_blocks);
hipError_t launch_topk(const TopkArgs& a, hipStream_t s);

// ------------------------------------------------------------ sparse attention
struct AttnArgs {
  Layout L;
  int row0, n_rows;
  const int32_t* q_seq;
  const int32_t* q_pos;
  const void* q;               // [n_q, H, dk]
  const uint8_t* k;            // K rows (bf16 or fp8 latent, or f32)
  int64_t k_stride;
  const float* k_scale;        // per-token scales of an fp8 latent cache, else null
  const uint8_t* v;            // V rows (f32 path)
  int64_t v_stride;
  const int32_t* sel;          // [n_q, top_k]
  int top_k;
  float scale;
  void* out;                   // [n_q, H, dv]
  float* lse;                  // [n_q, H] or null
  uint16_t* part_o;            // [n_rows, n_split, H, dv] bf16, unnormalised (split > 1)
  float* part_ml;              // [n_rows, n_split, H, 2]
  int n_split, blocks_per_split;
  int heads, dk, dv;
  int k_off32;                 // every K row lies within 4 GB of k (32-bit byte offsets)
};
// bf16 latent MQA: 64 heads, dk 576, dv 512
constexpr int LAT_H = 64, LAT_DK = 576, LAT_DV = 512;
hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t s);
// the pipelined bf16 kernel alone (no combine); launch_attn_bf16 picks it for splits
// of at least PIPE_MIN_BLOCKS blocks when every K row lies within 4 GB of k
constexpr int PIPE_MIN_BLOCKS = 128;
hipError_t launch_attn_bf16_pipe(const AttnArgs& a, hipStream_t s);
hipError_t launch_attn_fp8(const AttnArgs& a, hipStream_t s);

// KDA decode step (the linear-attention half): 128 key and value channels per head
constexpr int KDA_D = 128;
struct KdaArgs {
  int batch, heads;
  const uint16_t* xq;          // [batch, heads * 128] bf16, before the convolution
  const uint16_t* xk;
  const uint16_t* xv;
  const float* alpha;          // [batch, heads, 128] per-key-channel decay
  const float* beta;           // [batch, heads] write strength
  const float* conv_w;         // [3 (q, k, v), heads * 128, 4] taps t-3 .. t
  const float* conv_in;        // [batch, 3, 3 (t-3 .. t-1), heads * 128] taps before the step
  float* conv_out;             // the same layout, taps after the step (a different buffer)
  float* state;                // [batch, heads, 128, 128] rows = key channels, updated
  float* out;                  // [batch, heads, 128]
};
hipError_t launch_kda_decode(const KdaArgs& a, hipStream_t s);
hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t s);

}  // namespace ip
