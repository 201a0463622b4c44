// Learned sparse selection: keep the query's own block plus the k'-1 best-scoring
// earlier blocks (k' = min(top_k, b_q + 1)), ties to the lower block id, ids out in
// ascending order.  G2C Brief "GLM-5.3-Flash: hybrid attention becomes the product",
// section "DSA keeps selected global access in eleven layers" (top 2048 tokens =
// 512 pooled blocks).
//
// Exact radix select on order-preserving 32-bit keys, MSB first, 8 bits per pass,
// with the keys held in registers (each thread owns a contiguous index range, so
// "lower index first" is a prefix sum over threads):
//   stage 1: one workgroup per (row, 8192-score chunk) selects the chunk's best
//            min(k'-1, chunk) ids; a row with a single chunk writes its final
//            answer directly;
//   stage 2: one workgroup per multi-chunk row selects among the concatenated
//            chunk winners (which are already in ascending index order).
#include "kernels.hpp"

namespace ip {

namespace {

struct SelectShared {
  int hist[256];
  int scan[32];
  int digit, above;
};

// Finds T and r such that the kk largest keys (ties broken toward lower index)
// are exactly: all keys > T, plus the first r keys == T in index order.
// Key 0 marks an empty slot and is never counted.  Requires 1 <= kk <= number of
// non-empty keys, and NT >= 256 (the first four waves scan the 256 bins).
template <int NT, int E>
__device__ void radix_select(const uint32_t (&key)[E], int kk, SelectShared& sh,
                             uint32_t* T_out, int* r_out) {
  uint32_t prefix = 0, pmask = 0;
  int remaining = kk;
#pragma unroll 1
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < 256; i += NT) sh.hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint32_t k = key[e];
      if (k != 0u && (k & pmask) == prefix) atomicAdd(&sh.hist[(k >> shift) & 0xFFu], 1);
    }
    __syncthreads();
    // thread t < 256 holds bin 255 - t; the inclusive scan over t counts the
    // matching keys whose digit is >= 255 - t
    int h = 0, x = 0;
    if (threadIdx.x < 256) {
      const int lane = threadIdx.x & 63;
      h = sh.hist[255 - threadIdx.x];
      x = h;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
      }
      if (lane == 63) sh.scan[threadIdx.x >> 6] = x;
    }
    __syncthreads();
    if (threadIdx.x < 256) {
      const int wv = threadIdx.x >> 6;
      int base = 0;
      for (int i = 0; i < wv; ++i) base += sh.scan[i];
      const int incl = base + x;
      if (incl >= remaining && incl - h < remaining) {   // exactly one bin
        sh.digit = 255 - (int)threadIdx.x;
        sh.above = incl - h;
      }
    }
    __syncthreads();
    remaining -= sh.above;
    prefix |= (uint32_t)sh.digit << shift;
    pmask |= 0xFFu << shift;
  }
  *T_out = prefix;
  *r_out = remaining;
}

// Output position of every selected key (or -1): keys > T, then the first r keys
// equal to T in index order; positions follow index order.  Thread t owns the
// contiguous index range [t*E, (t+1)*E).
template <int NT, int E>
__device__ void compact_positions(const uint32_t (&key)[E], uint32_t T, int r, int* tmp,
                                  int (&pos)[E]) {
  int nt = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) nt += (key[e] != 0u && key[e] == T);
  int total;
  int tb = block_exclusive_scan<NT>(nt, tmp, &total);
  bool sel[E];
  int cnt = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    bool s = false;
    if (key[e] != 0u) {
      if (key[e] > T) s = true;
      else if (key[e] == T) { s = tb < r; ++tb; }
    }
    sel[e] = s;
    cnt += s;
  }
  int ob = block_exclusive_scan<NT>(cnt, tmp, &total);
#pragma unroll
  for (int e = 0; e < E; ++e) pos[e] = sel[e] ? ob++ : -1;
}

struct RowInfo {
  int bq, nel, need, nchunks;
};

__device__ __forceinline__ RowInfo row_info(const TopkArgs& a, int r) {
  const int b = a.q_seq ? a.q_seq[r] : r;
  const int p = a.q_pos ? a.q_pos[r] : a.L.seq_lens[b] - 1;
  RowInfo ri;
  ri.bq = p >> 2;
  ri.nel = ri.bq;
  ri.need = min(a.top_k, ri.bq + 1) - 1;
  ri.nchunks = max(1, (ri.nel + TOPK_CHUNK - 1) / TOPK_CHUNK);
  return ri;
}

// own block after the kept ids, then -1 padding
__device__ __forceinline__ void write_tail(const TopkArgs& a, int r, const RowInfo& ri, int nt) {
  int32_t* out = a.out + (int64_t)r * a.top_k;
  for (int i = ri.need + threadIdx.x; i < a.top_k; i += nt) out[i] = (i == ri.need) ? ri.bq : -1;
}

template <int NT, int E>
__global__ __launch_bounds__(NT) void topk_stage1_kernel(TopkArgs a) {
  static_assert(NT * E == TOPK_CHUNK, "chunk size");
  __shared__ SelectShared sh;
  __shared__ int tmp[NT / 64 + 1];
  const int rl = blockIdx.y, r = a.row0 + rl, c = blockIdx.x;
  const RowInfo ri = row_info(a, r);
  if (c >= ri.nchunks) return;
  const int c0 = c * TOPK_CHUNK;
  const int clen = max(0, min(TOPK_CHUNK, ri.nel - c0));
  const int kk = min(ri.need, clen);

  uint32_t key[E];
  const float* src = a.scores + (int64_t)rl * a.ld + c0 + threadIdx.x * E;
  const int i0 = threadIdx.x * E;
  if (i0 + E <= clen) {
#pragma unroll
    for (int e = 0; e < E; e += 4) {
      const float4 v = *(const float4*)(src + e);
      key[e] = float_key(v.x); key[e + 1] = float_key(v.y);
      key[e + 2] = float_key(v.z); key[e + 3] = float_key(v.w);
    }
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) key[e] = (i0 + e < clen) ? float_key(src[e]) : 0u;
  }

  uint32_t T = 0;
  int rr = 0;
  if (kk > 0 && kk < clen) radix_select<NT, E>(key, kk, sh, &T, &rr);
  int pos[E];
  if (kk > 0) {
    compact_positions<NT, E>(key, T, rr, tmp, pos);
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) pos[e] = -1;
  }

  if (ri.nchunks == 1) {
    int32_t* out = a.out + (int64_t)r * a.top_k;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (pos[e] >= 0) out[pos[e]] = c0 + i0 + e;
    write_tail(a, r, ri, NT);
  } else {
    const int64_t base = ((int64_t)rl * a.n_chunks + c) * (a.top_k - 1);
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (pos[e] >= 0) {
        a.cand_key[base + pos[e]] = key[e];
        a.cand_idx[base + pos[e]] = c0 + i0 + e;
      }
  }
}

template <int NT, int E>
__global__ __launch_bounds__(NT) void topk_stage2_kernel(TopkArgs a) {
  static_assert(NT * E == TOPK_MERGE_CAP, "merge capacity");
  __shared__ SelectShared sh;
  __shared__ int tmp[NT / 64 + 1];
  const int rl = blockIdx.x, r = a.row0 + rl;
  const RowInfo ri = row_info(a, r);
  if (ri.nchunks <= 1) return;
  const int km1 = a.top_k - 1;
  const int64_t base = (int64_t)rl * a.n_chunks * km1;
  const int nslots = ri.nchunks * km1;

  uint32_t key[E];
  const int s0 = threadIdx.x * E;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int s = s0 + e;
    uint32_t k = 0u;
    if (s < nslots) {
      const int c = s / km1, i = s - c * km1;
      const int kk_c = min(ri.need, min(TOPK_CHUNK, ri.nel - c * TOPK_CHUNK));
      if (i < kk_c) k = a.cand_key[base + s];
    }
    key[e] = k;
  }
  uint32_t T;
  int rr;
  radix_select<NT, E>(key, ri.need, sh, &T, &rr);
  int pos[E];
  compact_positions<NT, E>(key, T, rr, tmp, pos);
  int32_t* out = a.out + (int64_t)r * a.top_k;
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (pos[e] >= 0) out[pos[e]] = a.cand_idx[base + s0 + e];
  write_tail(a, r, ri, NT);
}

}  // namespace

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
  if (a.n_rows <= 0) return hipSuccess;
  constexpr int NT1 = 512, E1 = TOPK_CHUNK / NT1;
  constexpr int NT2 = 1024, E2 = TOPK_MERGE_CAP / NT2;
  hook_before(K_TOPK, s);
  hipLaunchKernelGGL((topk_stage1_kernel<NT1, E1>), dim3(a.n_chunks, a.n_rows), dim3(NT1), 0, s, a);
  hook_after(K_TOPK, s);
  if (a.n_chunks > 1)
    hipLaunchKernelGGL((topk_stage2_kernel<NT2, E2>), dim3(a.n_rows), dim3(NT2), 0, s, a);
  return hipGetLastError();
}

}  // namespace ip
