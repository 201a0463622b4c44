// Host-side launch interface of the gfx950 kernels (internal to libindexpool).
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>
#include <algorithm>
#include "common.hpp"

namespace ip {

enum KernelId { K_COMPRESS = 1, K_SCORE = 2, K_TOPK = 3 /* select */, K_ATTN = 4, K_COMBINE = 5, K_APPEND = 6, K_KDA = 7,
                K_STEP = 8, K_LAST = 8 };

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

// ------------------------------------------------------------ indexer scoring + selection
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
  int64_t ld;                  // a multiple of 512
  float* gm;                   // [n_rows, gld] maxima of groups of 16 consecutive scores (non-fused: or null)
  int64_t gld;                 // ld / 16
  int heads, dim;
  int max_blocks;              // key range covered by the grid
  int fuse;                    // select in the same launch (one row per workgroup)
  int top_k;                   // fused selection: ids out
  int32_t* out;                // [n_q, top_k], row r
  int32_t* count;              // [n_rows] per-row counters, zero on entry and on exit
  uint32_t* ack;               // with lists: [n_rows][3] per row (parity, two counters), zero-filled once
  int scores_own;              // scores is the workspace (rows may be written past b_q)
  uint64_t* lists;             // fused: [n_rows, max_lists, 16] per-wave candidate lists, or null
  uint2* lists_meta;           // [n_rows, max_lists] (count, threshold) of each list
  int max_lists;               // waves per row covered by the grid
  int wg_lists;                // rows too long for per-wave lists (max_lists 0): one list per
                               // workgroup in lists / lists_meta, this many per row, or 0
  int with_append;             // decode: extra grid rows of workgroups run `append`,
  AppendArgs append;           // one sequence each (see append.hpp)
  // the fused decode step only (else 0): the attention workgroups select the rows
  // that use lists (and the trivial rows) themselves.  A wave of a list row stores its
  // scores, then (once they are acknowledged) its list; the lists are zero on entry
  // (cleared by the combine)
  int step;
};
hipError_t launch_score_fp8_bf16(const ScoreArgs& a, hipStream_t s);
hipError_t launch_score_f32(const ScoreArgs& a, hipStream_t s);
// whether launch_score_fp8_bf16 selects in the same launch for these arguments
// (then a.fuse must be set; otherwise launch_select follows)
bool score_fuses_select(const ScoreArgs& a);
constexpr int SCORE_TILE = 1024;    // score rows pad to whole tiles of the scoring workgroups

// ------------------------------------------------------------ top-k selection
// One workgroup per row chunk holds up to 48 x 512 scores in registers (topk.hip):
// the faster select for rows of at most TOPK_SINGLE_MAX eligible blocks whose score
// rows are padded to a whole chunk (prefill rows of a 73728-token chunk).  Only the
// single-chunk form is launched (n_chunks == 1, cand_* and count unused).
struct TopkArgs {
  Layout L;
  int row0, n_rows;
  const int32_t* q_seq;
  const int32_t* q_pos;
  const float* scores;         // [n_rows, ld]
  int64_t ld;
  int top_k;
  int32_t* out;                // [n_q, top_k], row r
  uint32_t* cand_key;          // unused (multi-chunk rows)
  int32_t* cand_idx;
  int n_chunks;                // 1
  int chunk;                   // scores per chunk (topk_chunk_size)
  int32_t* count;
};
constexpr int TOPK_MAX_CHUNK = 16384;   // scores per chunk workgroup (512 threads x 32)
constexpr int TOPK_MERGE_CAP = 16384;
constexpr int TOPK_SINGLE_MAX = 512 * 48;
int topk_chunk_size(int max_blocks);
hipError_t launch_topk(const TopkArgs& a, hipStream_t s);

struct SelectArgs {
  Layout L;
  int row0, n_rows;
  const int32_t* q_seq;
  const int32_t* q_pos;
  const float* scores;         // [n_rows, ld]
  int64_t ld;
  const float* gm;             // [n_rows, gld]
  int64_t gld;
  int top_k;
  int32_t* out;                // [n_q, top_k], row r
};
hipError_t launch_select(const SelectArgs& a, hipStream_t s);

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
  // fused decode step only (else null): sel_ready[r - row0] is set to 1 by the
  // workgroup that stores row r's ids in the same launch (cleared by the combine),
  // and the query's own token row is read from k_new + b * k_new_stride
  uint32_t* sel_ready;
  const uint8_t* k_new;
  int64_t k_new_stride;
  // the fused decode step's selection of the list rows (see ScoreArgs::step),
  // done by the attention workgroups: the row's lists, its scores and group maxima
  // (for the exact fallback), and the row's ids written to sel_out (= sel)
  uint64_t* step_lists;
  uint2* step_meta;
  int step_max_lists;          // lists per row in step_lists / step_meta
  int step_lists_n;            // lists of the longest row (<= step_max_lists, * 16 <= 8 * 256)
  const float* step_scores;
  int64_t step_ld;
  const float* step_gm;
  int64_t step_gld;
  int32_t* sel_out;
};
// bf16 latent MQA: 64 heads, dk 576, dv 512
constexpr int LAT_H = 64, LAT_DK = 576, LAT_DV = 512;
hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t s);
// the pipelined bf16 kernel alone (no combine); launch_attn_bf16 picks it for splits
// of at least PIPE_MIN_BLOCKS blocks (32-bit offsets when k_off32, else 64-bit)
constexpr int PIPE_MIN_BLOCKS = 128;
hipError_t launch_attn_bf16_pipe(const AttnArgs& a, hipStream_t s);
hipError_t launch_attn_fp8(const AttnArgs& a, hipStream_t s);

// The fused decode step: one launch whose first workgroups score, select (and
// append) every row as launch_score_fp8_bf16 does with fuse set, and whose last
// workgroups run the bf16 attention of each (row, split) once the row's ids are
// published; then the combine.  score: one pass over all rows, fuse and
// with_append set; attn: n_split > 1, blocks_per_split < PIPE_MIN_BLOCKS,
// sel_ready and k_new set.  A waiting workgroup gives up after STEP_SPIN_LIMIT
// polls (only possible if earlier workgroups of the launch never run).
constexpr int STEP_SPIN_LIMIT = 1 << 22;
struct StepArgs {
  ScoreArgs score;
  AttnArgs attn;
};
bool decode_step_supported(const StepArgs& a);
hipError_t launch_decode_step(const StepArgs& a, hipStream_t s);
// The step kernel's arguments: the scoring and attention arguments, the scoring
// grid's width (workgroups per row), and the numbers of scoring and append
// workgroups before the attention ones.
struct StepKArgs {
  ScoreArgs s;
  AttnArgs at;
  int gx, n_score, n_app;
};
// the step kernel with 32-head attention units, over `grid` workgroups
hipError_t launch_decode_step_h32(const StepKArgs& k, unsigned grid, hipStream_t s);
// Copies the phase stamps of the last decode step (ip_phase_stamps); false unless
// the library was built with IP_PHASE_STAMPS.
bool phase_stamps(void* host, size_t bytes);

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
// KDA over a chunk of n_tokens consecutive tokens per sequence (prefill): the same
// recurrence as n_tokens decode steps.  x* [batch, n_tokens, heads * 128] bf16,
// alpha [batch, n_tokens, heads, 128], beta [batch, n_tokens, heads], out
// [batch, n_tokens, heads, 128]; conv and state as in KdaArgs.
struct KdaChunkArgs {
  int batch, heads, n_tokens;
  const uint16_t* xq;
  const uint16_t* xk;
  const uint16_t* xv;
  const float* alpha;
  const float* beta;
  const float* conv_w;
  const float* conv_in;
  float* conv_out;
  float* state;
  float* out;
};
hipError_t launch_kda_chunk(const KdaChunkArgs& a, hipStream_t s);
hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t s);

}  // namespace ip
