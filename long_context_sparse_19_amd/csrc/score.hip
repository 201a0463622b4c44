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
#include "append.hpp"

namespace ip {

namespace {

constexpr int NT = 256;
static_assert(NT == APPEND_NT, "the fused append runs in scoring workgroups");
constexpr int TILES = 4;                        // 32-key tiles per wave
constexpr int KEYS_PER_WG = 4 * TILES * 32;     // 512
constexpr int HI = 32, DI = 128;

// RPW query rows share one key chunk held in registers (prefill, where consecutive
// rows are tokens of one sequence); decode rows are separate sequences and use 1.
// All key loads of a wave are issued before the first MFMA, so each compute unit
// keeps ~128 KB of the pooled cache in flight.
template <int RPW>
__global__ __launch_bounds__(NT) void score_fp8_bf16_kernel(ScoreArgs a) {
  constexpr int QROW = DI + 8;                  // padded LDS row (272 bytes): conflict-free reads
  __shared__ __align__(16) uint16_t qs[2][HI * QROW];   // double-buffered query rows
  __shared__ float gs[2][HI];
  if (a.with_append && (int)blockIdx.y >= a.n_rows) {
    // the fused decode append, one sequence per workgroup of the extra grid rows:
    // scoring reads pooled rows of blocks before the query's own block only, and
    // the append writes the new token's rows and the pooled row of the block it
    // completes (the query's own block)
    const int b = ((int)blockIdx.y - a.n_rows) * (int)gridDim.x + (int)blockIdx.x;
    if (b < a.append.batch) append_one(a.append, b);
    return;
  }
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int kl = lane & 31, hh = lane >> 5;
  const int kc0 = blockIdx.x * KEYS_PER_WG;
  const int rbeg = a.row0 + blockIdx.y * RPW;
  const int rend = min(rbeg + RPW, a.row0 + a.n_rows);
  if (a.topk_count && blockIdx.x == 0 && (int)threadIdx.x < rend - rbeg)
    a.topk_count[rbeg + threadIdx.x - a.row0] = 0;

  // query rows (8 KB) and gates go through LDS; row r+1's are loaded while row r
  // is computed, and staged in the other buffer, so one barrier per row suffices
  // and the load latency of a row is hidden behind the previous one.  Thread t
  // holds elements 16t .. 16t+15 = head t/8, dims (t%8)*16 ..
  u32x4_t qv0, qv1;
  float gv = 0.f;
  auto load_q = [&](int r) {
    const u32x4_t* qg = (const u32x4_t*)((const uint16_t*)a.q + (int64_t)r * HI * DI);
    qv0 = qg[2 * threadIdx.x];
    qv1 = qg[2 * threadIdx.x + 1];
    if (threadIdx.x < HI) gv = a.gates[(int64_t)r * HI + threadIdx.x];
  };
  auto stage_q = [&](int buf) {
    const int h = threadIdx.x >> 3, d = (threadIdx.x & 7) * 16;
    *(u32x4_t*)(qs[buf] + h * QROW + d) = qv0;
    *(u32x4_t*)(qs[buf] + h * QROW + d + 8) = qv1;
    if (threadIdx.x < HI) gs[buf][threadIdx.x] = gv;
  };
  // per-row sequence, position and pooled-row count, one row per lane, read once
  // (per-row loads inside the loop would each wait for every load in flight)
  int rb = 0, rp = 0, rn = 1;
  if (lane < rend - rbeg) {
    const int rr = rbeg + lane;
    rb = a.q_seq ? a.q_seq[rr] : rr;
    const int len = a.L.seq_lens[rb];
    rp = a.q_pos ? a.q_pos[rr] : len - 1;
    rn = (len + 3) >> 2;
  }
  load_q(rbeg);
  stage_q(0);
  if (rbeg + 1 < rend) load_q(rbeg + 1);

  bf16x8_t kf[TILES][8];
  float ksig[TILES];
  int cur_b = -1;

  for (int r = rbeg, i = 0; r < rend; ++r, ++i) {
    // row r's query is visible in buffer i&1, and every wave is done with buffer
    // (i+1)&1 (read in row r-1); LDS-only barrier: loads in flight are not waited for
    block_sync_lds();
    const int b = __builtin_amdgcn_readlane(rb, i);
    const int p = __builtin_amdgcn_readlane(rp, i);
    const int nel = p >> 2;                    // eligible blocks j < b_q
    const bool run = kc0 < nel;                // uniform over the workgroup
    if (run && b != cur_b) {
      cur_b = b;
      // pooled rows that exist; keys past them are clamped to the last one (their
      // scores are never written), so every load is unconditional and all of a
      // wave's loads are in flight together
      const int nrows = __builtin_amdgcn_readlane(rn, i);
      u32x4_t raw[TILES][4];
#pragma unroll
      for (int t = 0; t < TILES; ++t) {
        const int j = min(kc0 + (wv * TILES + t) * 32 + kl, nrows - 1);
        const int64_t row = a.L.pool_row(b, j);
        const u32x4_t* src = (const u32x4_t*)(a.keys + row * a.key_stride + hh * 64);
#pragma unroll
        for (int c = 0; c < 4; ++c) raw[t][c] = src[c];
        ksig[t] = a.key_scale[row];
      }
#pragma unroll
      for (int t = 0; t < TILES; ++t)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          kf[t][2 * c] = fp8x8_to_bf16x8(raw[t][c][0], raw[t][c][1]);
          kf[t][2 * c + 1] = fp8x8_to_bf16x8(raw[t][c][2], raw[t][c][3]);
        }
      // the scales land here too, so that no later use of them waits for the
      // query prefetch issued after this point
#pragma unroll
      for (int t = 0; t < TILES; ++t) asm volatile("" ::"v"(ksig[t]));
    }
    const uint16_t* qb = qs[i & 1];
    const float* gb = gs[i & 1];
    // query fragment: head kl, dims hh*64 .. hh*64+63 (the same dims as the key half)
    bf16x8_t qf[8];
    // gates of the 16 heads this lane accumulates: rows (i/4)*8 + hh*4 + i%4
    float g[16];
    if (run) {
#pragma unroll
      for (int c = 0; c < 8; ++c) qf[c] = *(const bf16x8_t*)(qb + kl * QROW + hh * 64 + c * 8);
#pragma unroll
      for (int e = 0; e < 16; ++e) g[e] = gb[(e >> 2) * 8 + hh * 4 + (e & 3)];
    }
    // stage row r+1 and fetch row r+2.  Staging waits for row r+1's loads, issued
    // one row ago, and for whatever followed them (row r-1's score stores): both
    // have had a row's time to finish.
    if (r + 1 < rend) {
      stage_q((i + 1) & 1);
      if (r + 2 < rend) load_q(r + 2);
    }
    if (!run) continue;

#pragma unroll
    for (int t = 0; t < TILES; ++t) {
      f32x16_t acc = {};
#pragma unroll
      for (int c = 0; c < 8; ++c) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[c], kf[t][c], acc, 0, 0, 0);
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) part = fmaf(g[e], fmaxf(acc[e], 0.f), part);
      part += __shfl_xor(part, 32);
      const int j = kc0 + (wv * TILES + t) * 32 + kl;
      if (hh == 0 && j < nel) a.scores[(int64_t)(r - a.row0) * a.ld + j] = part * ksig[t];
    }
  }
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
  if (a.topk_count && blockIdx.x == 0 && threadIdx.x == 0) a.topk_count[blockIdx.y] = 0;
  if ((int)(blockIdx.x * NT) >= nel) return;
  const int HD = a.heads * a.dim;
  const float* q = (const float*)a.q + (int64_t)r * HD;
  for (int i = threadIdx.x; i < HD; i += NT) qs[i] = q[i];
  for (int i = threadIdx.x; i < a.heads; i += NT) gs[i] = a.gates[(int64_t)r * a.heads + i];
  __syncthreads();
  if (j >= nel) return;
  const float* k = (const float*)(a.keys + a.L.pool_row(b, j) * a.key_stride);
  float s = 0.f;
  for (int h = 0; h < a.heads; ++h) {
    float d = 0.f;
    for (int e = 0; e < a.dim; ++e) d = fmaf(qs[h * a.dim + e], k[e], d);
    s = fmaf(gs[h], fmaxf(d, 0.f), s);
  }
  a.scores[(int64_t)(r - a.row0) * a.ld + j] = s;
}

}  // namespace

hipError_t launch_score_fp8_bf16(const ScoreArgs& a, hipStream_t s) {
  if (a.n_rows <= 0 || a.max_blocks <= 0) return hipSuccess;
  const unsigned gx = (a.max_blocks + KEYS_PER_WG - 1) / KEYS_PER_WG;
  if (a.q_seq && a.n_rows >= 64 && !a.with_append) {
    // prefill: consecutive rows are query tokens of one sequence and share its keys
    constexpr int R = 32;
    launch(K_SCORE, score_fp8_bf16_kernel<R>, dim3(gx, (a.n_rows + R - 1) / R), dim3(NT), s, a);
  } else {
    const unsigned app_rows = a.with_append ? (a.append.batch + gx - 1) / gx : 0;
    launch(K_SCORE, score_fp8_bf16_kernel<1>, dim3(gx, a.n_rows + app_rows), dim3(NT), s, a);
  }
  return hipGetLastError();
}

hipError_t launch_score_f32(const ScoreArgs& a, hipStream_t s) {
  if (a.n_rows <= 0 || a.max_blocks <= 0) return hipSuccess;
  dim3 grid((a.max_blocks + NT - 1) / NT, a.n_rows);
  launch(K_SCORE, score_f32_kernel, grid, dim3(NT), s, a);
  return hipGetLastError();
}

}  // namespace ip
