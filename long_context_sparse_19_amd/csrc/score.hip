// Lightweight indexer: S_j = sum_h g_h * relu(q_h . K_j) for every pooled block j
// before the query's own block.  Reading notes "GLM-5.3-Flash: Hybrid Attention,
// IndexPool, and Vision-in-the-Loop", section 2 "Hybrid Attention: Linear State +
// Sparse Retrieval" (sparse attention as the global retriever through a lightweight
// indexer; DeepSeek-V3.2's DSA indexer as its lineage).
//
// fp8 keys x bf16 queries: the heads x keys product is a dense contraction
// (32 heads x 128 dims x keys), so it runs on bf16 MFMA (v_mfma_f32_32x32x16_bf16)
// with the 32 heads as M and 32 keys per tile as N.  The fp8 codes are widened to
// bf16 exactly, so every product is exact in the fp32 accumulator.  The per-block
// scale sigma_j > 0 is applied after the ReLU (relu(sigma x) = sigma relu(x)).
// The output layout puts one key per lane and 16 heads per lane, so the gated
// head-sum is 16 local FMAs plus one cross-half exchange.
//
// Every scoring kernel also writes the largest score of each group of 16
// consecutive blocks (the group maxima the selection starts from).  Decode-shaped
// launches (one query row per workgroup) select in the same launch: each
// workgroup counts itself in on a per-row counter once its scores are stored, and
// the one that completes the count selects the row (select.hpp) and clears the
// counter for the next call.
#include "score_fp8.hpp"

namespace ip {

namespace {

using scorek::row16_max;
constexpr int NT = 256;                         // f32 kernel; prefill fp8 workgroups
constexpr int TILES = scorek::TILES;

template <int RPW, int NWV, bool FUSE>
__global__ __launch_bounds__(NWV * 64) void score_fp8_bf16_kernel(ScoreArgs a) {
  // the query stage, and (fused) the selection's state once scoring is done
  __shared__ __align__(16) uint8_t smem[scorek::score_smem<NWV, FUSE>()];
  __shared__ int last_here;
  // fused (decode rows): the scoring workgroups take their (key chunk, row) rows
  // fastest in dispatch order, so the first chunks of every row go before the later
  // chunks of the long rows, and the append workgroups come last.  Consecutive
  // workgroups go to the dies in turn, so every die keeps an even share of the
  // scoring (a one-row grid is unchanged).
  if constexpr (FUSE) {
    const int gx = (int)gridDim.x, nr = a.n_rows;
    const int L = (int)(blockIdx.y * gridDim.x + blockIdx.x);
    const int A = L - nr * gx;                   // >= 0: an append workgroup
    const int bx = A < 0 ? L / nr : A % gx;
    const int by = A < 0 ? L % nr : nr + A / gx;
    scorek::score_fp8_body<RPW, NWV, FUSE>(a, bx, by, gx, smem, last_here, nullptr);
  } else
    scorek::score_fp8_body<RPW, NWV, FUSE>(a, blockIdx.x, blockIdx.y, gridDim.x, smem, last_here, nullptr);
}

// float keys and queries (small geometries): one thread per key, queries in LDS.
constexpr int F32_MAX_Q = 64 * 256;
__global__ __launch_bounds__(NT) void score_f32_kernel(ScoreArgs a) {
  __shared__ float qs[F32_MAX_Q / 4];          // heads * dim <= 4096 floats
  __shared__ float gs[64];
  const int r = a.row0 + blockIdx.y;
  const int b = a.q_seq ? a.q_seq[r] : r;
  const int p = a.q_pos ? a.q_pos[r] : a.L.seq_lens[b] - 1;
  const int nel = p >> 2;
  const int j = blockIdx.x * NT + threadIdx.x;
  if ((int)(blockIdx.x * NT) >= nel) return;
  const int HD = a.heads * a.dim;
  const float* q = (const float*)a.q + (int64_t)r * HD;
  for (int i = threadIdx.x; i < HD; i += NT) qs[i] = q[i];
  for (int i = threadIdx.x; i < a.heads; i += NT) gs[i] = a.gates[(int64_t)r * a.heads + i];
  __syncthreads();
  float s = -INFINITY;
  if (j < nel) {
    const float* k = (const float*)(a.keys + a.L.pool_row(b, j) * a.key_stride);
    s = 0.f;
    for (int h = 0; h < a.heads; ++h) {
      float d = 0.f;
      for (int e = 0; e < a.dim; ++e) d = fmaf(qs[h * a.dim + e], k[e], d);
      s = fmaf(gs[h], fmaxf(d, 0.f), s);
    }
    a.scores[(int64_t)(r - a.row0) * a.ld + j] = s;
  }
  // groups of 16 consecutive blocks are 16-lane rows of the wave
  const float gmax = row16_max(s);
  if (a.gm && (threadIdx.x & 15) == 0 && j < nel) a.gm[(int64_t)(r - a.row0) * a.gld + (j >> 4)] = gmax;
}

}  // namespace

hipError_t launch_score_fp8_bf16(const ScoreArgs& a, hipStream_t s) {
  if (a.n_rows <= 0 || a.max_blocks <= 0) return hipSuccess;
  if (!score_fuses_select(a)) {
    // prefill: consecutive rows are query tokens of one sequence and share its keys
    constexpr int R = 32, W = 4, KEYS = W * TILES * 32;
    const unsigned gx = (a.max_blocks + KEYS - 1) / KEYS;
    launch(K_SCORE, score_fp8_bf16_kernel<R, W, false>, dim3(gx, (a.n_rows + R - 1) / R), dim3(W * 64), s, a);
  } else {
    constexpr int W = 8, KEYS = W * TILES * 32;
    const unsigned gx = (a.max_blocks + KEYS - 1) / KEYS;
    const unsigned app_rows = a.with_append ? (a.append.batch + gx - 1) / gx : 0;
    if (!a.fuse) return hipErrorInvalidValue;
    launch(K_SCORE, score_fp8_bf16_kernel<1, W, true>, dim3(gx, a.n_rows + app_rows), dim3(W * 64), s, a);
  }
  return hipGetLastError();
}

bool score_fuses_select(const ScoreArgs& a) { return !(a.q_seq && a.n_rows >= 64 && !a.with_append); }

hipError_t launch_score_f32(const ScoreArgs& a, hipStream_t s) {
  if (a.n_rows <= 0 || a.max_blocks <= 0) return hipSuccess;
  dim3 grid((a.max_blocks + NT - 1) / NT, a.n_rows);
  launch(K_SCORE, score_f32_kernel, grid, dim3(NT), s, a);
  return hipGetLastError();
}

}  // namespace ip
