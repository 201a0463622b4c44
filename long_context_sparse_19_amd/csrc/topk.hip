// Learned sparse selection: keep the query's own block plus the k'-1 best-scoring
// earlier blocks (k' = min(top_k, b_q + 1)), ties to the lower block id, ids out in
// ascending order.  G2C Brief "GLM-5.3-Flash: hybrid attention becomes the product",
// section "DSA keeps selected global access in eleven layers" (top 2048 tokens =
// 512 pooled blocks).
//
// Exact radix select on order-preserving 32-bit keys held in registers, by one
// 1024-thread workgroup per row (chunk):
//   * wave w owns the contiguous index range [w*64*E, (w+1)*64*E); lane l holds
//     indices w*64*E + i*64 + l (i < E), so every load is a coalesced 256-byte row
//     and index order inside a wave is (i, lane);
//   * one histogram pass over 2048 linear buckets of the row's score range, then
//     three passes over 11/11/10-bit digits of the keys in the boundary bucket
//     (LDS atomics) find the threshold key T and how many keys equal to T to keep;
//   * ordered compaction with wave ballots: ties are ranked and survivors placed by
//     ballot popcounts, with one 16-entry scan across waves per phase.
// Rows longer than one chunk (1024*32 scores) are split: every chunk keeps its own
// best min(k'-1, chunk) ids and a second launch selects among the concatenated
// winners, which are already in ascending index order.
#include "kernels.hpp"

namespace ip {

namespace {

constexpr int NT = 1024;
constexpr int NW = NT / 64;
constexpr int NBINS = 2048;

struct SelShared {
  int hist[NBINS];
  int wsum[NW];
  int woff[NW + 1];
  uint32_t wmin[NW], wmax[NW];
  int digit, above;
};

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & 63;
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// exclusive scan of one value per wave (16 waves) through LDS; returns this
// wave's offset, *total the sum
__device__ __forceinline__ int wave_offsets(int v, SelShared& sh, int* total) {
  const int wv = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) sh.wsum[wv] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    int s = 0;
    for (int i = 0; i < NW; ++i) { sh.woff[i] = s; s += sh.wsum[i]; }
    sh.woff[NW] = s;
  }
  __syncthreads();
  *total = sh.woff[NW];
  return sh.woff[wv];
}

__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Histogram scan: thread t holds bins 2047-2t and 2046-2t (descending); finds the
// bin d with count(bins > d) < remaining <= count(bins >= d), stores it in
// sh.digit / sh.above and clears the histogram for the next pass.
__device__ __forceinline__ void find_bin(SelShared& sh, int remaining) {
  const int b0 = NBINS - 1 - 2 * (int)threadIdx.x;
  const int h0 = sh.hist[b0], h1 = sh.hist[b0 - 1];
  sh.hist[b0] = 0;
  sh.hist[b0 - 1] = 0;
  const int lane = threadIdx.x & 63;
  int x = h0 + h1;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  int tot;
  const int base = wave_offsets(__shfl(x, 63, 64), sh, &tot);
  const int incl = base + x;                 // keys in bins >= b0 - 1
  const int before = incl - h0 - h1;         // keys in bins > b0
  if (before < remaining && before + h0 >= remaining) {
    sh.digit = b0;
    sh.above = before;
  } else if (before + h0 < remaining && incl >= remaining) {
    sh.digit = b0 - 1;
    sh.above = before + h0;
  }
  __syncthreads();
}

// Threshold T and the number r of keys equal to T to keep, so that the kk largest
// keys (ties to the lower index) are: every key > T, then the first r keys == T.
// Key 0 marks an empty slot.  1 <= kk <= number of non-empty keys.
//
// Pass 0 buckets the scores linearly between the row's min and max (2048 buckets;
// a monotone map, so every key in a higher bucket is larger), which spreads a
// narrow score distribution over many bins and keeps LDS atomics uncontended.
// Passes 1-3 resolve the exact 32-bit threshold among the keys of the boundary
// bucket only.
template <int E>
__device__ void radix_threshold(const uint32_t (&key)[E], int kk, SelShared& sh, uint32_t* T_out,
                                int* r_out) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (key[e] != 0u) { kmin = min(kmin, key[e]); kmax = max(kmax, key[e]); }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o));
  }
  if (lane == 0) { sh.wmin[wv] = kmin; sh.wmax[wv] = kmax; }
  for (int i = threadIdx.x; i < NBINS; i += NT) sh.hist[i] = 0;
  __syncthreads();
  kmin = sh.wmin[0];
  kmax = sh.wmax[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) { kmin = min(kmin, sh.wmin[i]); kmax = max(kmax, sh.wmax[i]); }
  const float fmin = key_float(kmin);
  const float range = key_float(kmax) - fmin;
  const float inv = (range > 0.f && range < INFINITY) ? (float)(NBINS - 1) / range : 0.f;
  auto bucket = [&](uint32_t k) -> int {
    const float b = (key_float(k) - fmin) * inv;
    return b >= (float)(NBINS - 1) ? NBINS - 1 : (int)b;
  };

  int remaining = kk;
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (key[e] != 0u) atomicAdd(&sh.hist[bucket(key[e])], 1);
  __syncthreads();
  find_bin(sh, remaining);
  const int B = sh.digit;
  remaining -= sh.above;
  uint32_t inb = 0;                           // keys in the boundary bucket
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (key[e] != 0u && bucket(key[e]) == B) inb |= 1u << e;

  constexpr int SHIFT[3] = {21, 10, 0};
  constexpr int BITS[3] = {11, 11, 10};
  uint32_t prefix = 0, pmask = 0;
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = SHIFT[pass];
    const uint32_t dmask = (1u << BITS[pass]) - 1u;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint32_t k = key[e];
      if (((inb >> e) & 1u) && (k & pmask) == prefix) atomicAdd(&sh.hist[(k >> shift) & dmask], 1);
    }
    __syncthreads();
    find_bin(sh, remaining);
    remaining -= sh.above;
    prefix |= (uint32_t)sh.digit << shift;
    pmask |= dmask << shift;
  }
  *T_out = prefix;
  *r_out = remaining;
}

// Output positions (or -1) in index order: keys > T, then the first r keys == T.
template <int E>
__device__ void ordered_positions(const uint32_t (&key)[E], uint32_t T, int r, SelShared& sh, int (&pos)[E]) {
  const uint64_t lt = lanemask_lt();
  // tie ranks
  int wt = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) wt += __popcll(__ballot(key[e] != 0u && key[e] == T));
  int tot;
  int tie = wave_offsets(wt, sh, &tot);
  bool sel[E];
  int wc = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool eq = key[e] != 0u && key[e] == T;
    const uint64_t be = __ballot(eq);
    const int rank = tie + __popcll(be & lt);
    tie += __popcll(be);
    sel[e] = (key[e] != 0u && key[e] > T) || (eq && rank < r);
    wc += __popcll(__ballot(sel[e]));
  }
  int off = wave_offsets(wc, sh, &tot);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint64_t bs = __ballot(sel[e]);
    pos[e] = sel[e] ? off + __popcll(bs & lt) : -1;
    off += __popcll(bs);
  }
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
  ri.nchunks = max(1, (ri.nel + a.chunk - 1) / a.chunk);
  return ri;
}

// own block after the kept ids, then -1 padding
__device__ __forceinline__ void write_tail(const TopkArgs& a, int r, const RowInfo& ri) {
  int32_t* out = a.out + (int64_t)r * a.top_k;
  for (int i = ri.need + threadIdx.x; i < a.top_k; i += NT) out[i] = (i == ri.need) ? ri.bq : -1;
}

template <int E>
__global__ __launch_bounds__(NT) void topk_chunk_kernel(TopkArgs a) {
  __shared__ SelShared sh;
  const int rl = blockIdx.y, r = a.row0 + rl, c = blockIdx.x;
  const RowInfo ri = row_info(a, r);
  if (c >= ri.nchunks) return;
  const int c0 = c * a.chunk;
  const int clen = max(0, min(a.chunk, ri.nel - c0));
  const int kk = min(ri.need, clen);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int wbase = wv * 64 * E;

  // loads are unconditional (index clamped into the chunk) so that all E of them
  // are in flight together; out-of-range slots become empty keys afterwards
  uint32_t key[E];
  const float* src = a.scores + (int64_t)rl * a.ld + c0;
  if (clen > 0) {
    float v[E];
#pragma unroll
    for (int e = 0; e < E; ++e) v[e] = src[min(wbase + e * 64 + lane, clen - 1)];
#pragma unroll
    for (int e = 0; e < E; ++e) key[e] = (wbase + e * 64 + lane < clen) ? float_key(v[e]) : 0u;
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) key[e] = 0u;
  }
  uint32_t T = 0;
  int rr = 0;
  if (kk > 0 && kk < clen) radix_threshold<E>(key, kk, sh, &T, &rr);
  int pos[E];
  if (kk > 0) {
    ordered_positions<E>(key, T, rr, sh, pos);
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) pos[e] = -1;
  }

  if (ri.nchunks == 1) {
    int32_t* out = a.out + (int64_t)r * a.top_k;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (pos[e] >= 0) out[pos[e]] = c0 + wbase + e * 64 + lane;
    write_tail(a, r, ri);
  } else {
    const int km1 = a.top_k - 1;
    const int64_t base = ((int64_t)rl * a.n_chunks + c) * km1;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (pos[e] >= 0) {
        a.cand_key[base + pos[e]] = key[e];
        a.cand_idx[base + pos[e]] = c0 + wbase + e * 64 + lane;
      }
    for (int i = kk + threadIdx.x; i < km1; i += NT) a.cand_key[base + i] = 0u;   // unused slots
  }
}

template <int E>
__global__ __launch_bounds__(NT) void topk_merge_kernel(TopkArgs a) {
  __shared__ SelShared sh;
  const int rl = blockIdx.x, r = a.row0 + rl;
  const RowInfo ri = row_info(a, r);
  if (ri.nchunks <= 1) return;
  const int km1 = a.top_k - 1;
  const int64_t base = (int64_t)rl * a.n_chunks * km1;
  const int nslots = ri.nchunks * km1;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int wbase = wv * 64 * E;
  uint32_t key[E];
  {
    uint32_t v[E];
#pragma unroll
    for (int e = 0; e < E; ++e) v[e] = a.cand_key[base + min(wbase + e * 64 + lane, nslots - 1)];
#pragma unroll
    for (int e = 0; e < E; ++e) key[e] = (wbase + e * 64 + lane < nslots) ? v[e] : 0u;
  }
  uint32_t T;
  int rr;
  radix_threshold<E>(key, ri.need, sh, &T, &rr);
  int pos[E];
  ordered_positions<E>(key, T, rr, sh, pos);
  int32_t* out = a.out + (int64_t)r * a.top_k;
  int32_t idx[E];
#pragma unroll
  for (int e = 0; e < E; ++e) idx[e] = a.cand_idx[base + min(wbase + e * 64 + lane, nslots - 1)];
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (pos[e] >= 0) out[pos[e]] = idx[e];
  write_tail(a, r, ri);
}

template <int E>
void launch_chunks(const TopkArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((topk_chunk_kernel<E>), dim3(a.n_chunks, a.n_rows), dim3(NT), 0, s, a);
}

template <int E>
void launch_merge(const TopkArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((topk_merge_kernel<E>), dim3(a.n_rows), dim3(NT), 0, s, a);
}

int per_thread(int n) {
  const int e = (n + NT - 1) / NT;
  return e <= 1 ? 1 : e <= 2 ? 2 : e <= 4 ? 4 : e <= 8 ? 8 : e <= 16 ? 16 : 32;
}

}  // namespace

int topk_chunk_size(int max_blocks) {
  return NT * per_thread(std::min(max_blocks, TOPK_MAX_CHUNK));
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
  if (a.n_rows <= 0) return hipSuccess;
  hook_before(K_TOPK, s);
  switch (a.chunk / NT) {
    case 1: launch_chunks<1>(a, s); break;
    case 2: launch_chunks<2>(a, s); break;
    case 4: launch_chunks<4>(a, s); break;
    case 8: launch_chunks<8>(a, s); break;
    case 16: launch_chunks<16>(a, s); break;
    default: launch_chunks<32>(a, s); break;
  }
  hook_after(K_TOPK, s);
  if (a.n_chunks > 1) {
    switch (per_thread(a.n_chunks * (a.top_k - 1))) {
      case 1: launch_merge<1>(a, s); break;
      case 2: launch_merge<2>(a, s); break;
      case 4: launch_merge<4>(a, s); break;
      case 8: launch_merge<8>(a, s); break;
      case 16: launch_merge<16>(a, s); break;
      default: launch_merge<32>(a, s); break;
    }
  }
  return hipGetLastError();
}

}  // namespace ip
