// Learned sparse selection: keep the query's own block plus the k'-1 best-scoring
// earlier blocks (k' = min(top_k, b_q + 1)), ties to the lower block id, ids out in
// ascending order.  G2C Brief "GLM-5.3-Flash: hybrid attention becomes the product",
// section "DSA keeps selected global access in eleven layers" (top 2048 tokens =
// 512 pooled blocks).
//
// One 512-thread workgroup selects the kk best of a chunk of up to 16384 scores
// held in registers.  Thread t owns the contiguous slots [t*E, t*E+E), so "lower
// slot first" is a per-thread count plus one workgroup prefix sum.
//   1. Threshold: with m the kk-th largest maximum of 8-score groups, at least kk
//      scores are >= m, so the answer lies in {v >= m}.  A 2048-bucket histogram
//      of the group maxima (linear between their min and max) gives T <= m.
//   2. If fewer than kk scores are > T, T itself is the kk-th largest value: keep
//      every v > T and the first kk - #(v > T) ties in slot order.
//   3. Else if at most 4096 scores are >= T, compact them in slot order into LDS
//      and run an exact radix select (2048 linear buckets, then 11/11/10-bit
//      digits of the order-preserving keys) on those few.
//   4. Else raise T with a histogram of the scores >= T and repeat (T strictly
//      increases, so this ends; typical rows never get here).
// Rows longer than one chunk are split: every chunk keeps its own best
// min(k'-1, chunk) and a merge launch selects among the concatenated winners,
// which are already in ascending index order.
#include "kernels.hpp"

namespace ip {

namespace {

constexpr int NT = 512;
constexpr int NW = NT / 64;
constexpr int NBINS = 2048;
constexpr int BPT = NBINS / NT;          // histogram bins scanned per thread
constexpr int CAND_CAP = 4096;           // candidates compacted into LDS
constexpr int EC = CAND_CAP / NT;        // candidates per thread in the exact select

struct SelShared {
  int hist[NBINS];
  int wsum[NW], wsum2[NW];
  int woff[NW + 1];
  float fa[NW], fb[NW];
  int digit, above;
  uint32_t ckey[CAND_CAP + 1];           // last entry: sink for non-candidates
  int32_t cid[CAND_CAP + 1];
};

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & 63;
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// exclusive scan of one value per wave through LDS: returns this wave's offset
// and *total the sum over the workgroup
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

// workgroup sums of two per-wave counts
__device__ __forceinline__ void wave_sum2(int x, int y, SelShared& sh, int* sx, int* sy) {
  const int wv = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { sh.wsum[wv] = x; sh.wsum2[wv] = y; }
  __syncthreads();
  int a = 0, b = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) { a += sh.wsum[i]; b += sh.wsum2[i]; }
  *sx = a;
  *sy = b;
  __syncthreads();
}

// workgroup min of lo and max of hi
__device__ __forceinline__ void minmax(float lo, float hi, SelShared& sh, float* mn, float* mx) {
  const int wv = threadIdx.x >> 6;
  lo = wave_min(lo);
  hi = wave_max(hi);
  if ((threadIdx.x & 63) == 0) { sh.fa[wv] = lo; sh.fb[wv] = hi; }
  __syncthreads();
  lo = sh.fa[0];
  hi = sh.fb[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) { lo = fminf(lo, sh.fa[i]); hi = fmaxf(hi, sh.fb[i]); }
  *mn = lo;
  *mx = hi;
  __syncthreads();
}

__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Histogram scan: thread t holds the BPT bins below 2048 - BPT*t (descending);
// finds the bin d with count(bins > d) < remaining <= count(bins >= d) into
// sh.digit / sh.above, and clears the histogram for the next pass.
__device__ __forceinline__ void find_bin(SelShared& sh, int remaining) {
  const int top = NBINS - 1 - BPT * (int)threadIdx.x;
  int h[BPT];
  int sum = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) {
    h[i] = sh.hist[top - i];
    sh.hist[top - i] = 0;
    sum += h[i];
  }
  const int x = wave_incl_scan(sum);
  int tot;
  const int base = wave_offsets(lane63(x), sh, &tot);
  int before = base + x - sum;               // values in bins > top
#pragma unroll
  for (int i = 0; i < BPT; ++i) {
    if (before < remaining && before + h[i] >= remaining) {
      sh.digit = top - i;
      sh.above = before;
    }
    before += h[i];
  }
  __syncthreads();
}

// monotone map of a float range onto the 2048 histogram bins
struct Buckets {
  float lo, inv;
  __device__ __forceinline__ int operator()(float f) const {
    const float b = (f - lo) * inv;
    return b >= (float)(NBINS - 1) ? NBINS - 1 : (b > 0.f ? (int)b : 0);
  }
};

__device__ __forceinline__ Buckets make_buckets(float lo, float hi) {
  const float range = hi - lo;
  Buckets bk;
  bk.lo = lo;
  bk.inv = (range > 0.f && range < INFINITY) ? (float)(NBINS - 1) / range : 0.f;
  return bk;
}

// exclusive prefix sum of one int per thread over the workgroup
__device__ __forceinline__ int block_scan(int x, SelShared& sh, int* total) {
  const int incl = wave_incl_scan(x);
  const int base = wave_offsets(lane63(incl), sh, total);
  return base + incl - x;
}

// Exact select over the compacted candidates (sh.ckey / sh.cid [0..M)), 1 <= kk <= M:
// emit(rank, id, key) for the kk best, ties to the lower candidate position.
template <class Emit>
__device__ void select_candidates(int M, int kk, SelShared& sh, Emit emit) {
  const int cb = threadIdx.x * EC;
  uint32_t key[EC];
#pragma unroll
  for (int e = 0; e < EC; ++e) key[e] = cb + e < M ? sh.ckey[cb + e] : 0u;
  uint32_t prefix = 0;
  int remaining = kk;
  if (kk < M) {
    // pass 0: linear buckets over the candidates' value range
    float lo = INFINITY, hi = -INFINITY;
#pragma unroll
    for (int e = 0; e < EC; ++e)
      if (key[e]) { lo = fminf(lo, key_float(key[e])); hi = fmaxf(hi, key_float(key[e])); }
    minmax(lo, hi, sh, &lo, &hi);
    const Buckets bk = make_buckets(lo, hi);
#pragma unroll
    for (int e = 0; e < EC; ++e)
      if (key[e]) atomicAdd(&sh.hist[bk(key_float(key[e]))], 1);
    __syncthreads();
    find_bin(sh, remaining);
    const int B = sh.digit;
    remaining -= sh.above;
    uint32_t inb = 0;
#pragma unroll
    for (int e = 0; e < EC; ++e)
      if (key[e] && bk(key_float(key[e])) == B) inb |= 1u << e;
    // passes 1-3: exact digits of the keys in the boundary bucket
    uint32_t pmask = 0;
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
      const uint32_t dmask = pass == 2 ? 0x3FFu : 0x7FFu;
#pragma unroll
      for (int e = 0; e < EC; ++e)
        if (((inb >> e) & 1u) && (key[e] & pmask) == prefix) atomicAdd(&sh.hist[(key[e] >> shift) & dmask], 1);
      __syncthreads();
      find_bin(sh, remaining);
      remaining -= sh.above;
      prefix |= (uint32_t)sh.digit << shift;
      pmask |= dmask << shift;
    }
  }
  // ordered output: keys > prefix, then the first `remaining` keys == prefix
  int nt = 0;
#pragma unroll
  for (int e = 0; e < EC; ++e) nt += (key[e] != 0u && key[e] == prefix);
  int tot;
  int tie = block_scan(nt, sh, &tot);
  uint32_t smask = 0;
  int ns = 0;
#pragma unroll
  for (int e = 0; e < EC; ++e) {
    const bool eq = key[e] != 0u && key[e] == prefix;
    const bool sl = (key[e] != 0u && key[e] > prefix) || (eq && tie < remaining);
    tie += eq;
    smask |= (uint32_t)sl << e;
    ns += sl;
  }
  int off = block_scan(ns, sh, &tot);
#pragma unroll
  for (int e = 0; e < EC; ++e)
    if ((smask >> e) & 1u) emit(off++, sh.cid[cb + e], key[e]);
}

// The kk best of v (NaN = empty), ties to the lower slot, 1 <= kk <= #values;
// emit(rank, id, key) once per kept value (id[] carried along, key = float_key(v)),
// ranks in slot order.  Nothing is loaded from memory at emit time: a load inside
// the per-element branches would serialise one round trip per element.
template <int E, class Emit>
__device__ void select_top(const float (&v)[E], const int32_t (&id)[E], int kk, SelShared& sh, Emit emit) {
  constexpr int GS = E >= 8 ? 8 : E;          // scores per group maximum
  constexpr int NG = E / GS;
  // every histogram pass below starts from zeroed bins (find_bin re-zeroes them)
  for (int i = threadIdx.x; i < NBINS; i += NT) sh.hist[i] = 0;
  __syncthreads();

  // 1. T <= the kk-th largest group maximum (or -inf if there are fewer groups)
  float gm[NG];
  int ngv = 0;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    float m = v[g * GS];
#pragma unroll
    for (int i = 1; i < GS; ++i) m = fmaxf(m, v[g * GS + i]);    // NaN-ignoring
    gm[g] = m;
    ngv += !__builtin_isnan(m);
  }
  int nval, unused;
  wave_sum2(wave_sum(ngv), 0, sh, &nval, &unused);
  float T = -INFINITY;
  if (kk <= nval) {
    float lo = INFINITY, hi = -INFINITY;
#pragma unroll
    for (int g = 0; g < NG; ++g)
      if (!__builtin_isnan(gm[g])) { lo = fminf(lo, gm[g]); hi = fmaxf(hi, gm[g]); }
    minmax(lo, hi, sh, &lo, &hi);
    const Buckets bk = make_buckets(lo, hi);
#pragma unroll
    for (int g = 0; g < NG; ++g)
      if (!__builtin_isnan(gm[g])) atomicAdd(&sh.hist[bk(gm[g])], 1);
    __syncthreads();
    find_bin(sh, kk);
    const int B = sh.digit;
    float m = INFINITY;
#pragma unroll
    for (int g = 0; g < NG; ++g)
      if (!__builtin_isnan(gm[g]) && bk(gm[g]) >= B) m = fminf(m, gm[g]);
    minmax(m, m, sh, &T, &hi);
  }

#pragma unroll 1
  for (;;) {
    int g = 0, q = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      g += v[e] > T;
      q += v[e] >= T;
    }
    int G, Q;
    const int qoff = block_scan(q, sh, &Q);
    wave_sum2(wave_sum(g), 0, sh, &G, &unused);
    if (G < kk) {
      // 2. T is the kk-th largest value: every v > T, then the first kk - G ties
      int nt = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) nt += v[e] == T;
      int tot;
      int tie = block_scan(nt, sh, &tot);
      uint64_t smask = 0;
      int ns = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const bool eq = v[e] == T;
        const bool sl = v[e] > T || (eq && tie < kk - G);
        tie += eq;
        smask |= (uint64_t)sl << e;
        ns += sl;
      }
      int off = block_scan(ns, sh, &tot);
#pragma unroll
      for (int e = 0; e < E; ++e)
        if ((smask >> e) & 1ull) emit(off++, id[e], float_key(v[e]));
      return;
    }
    if (Q <= CAND_CAP) {
      // 3. compact {v >= T} in slot order (non-candidates write the sink entry),
      //    then the exact select on the candidates
      int off = qoff;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const bool c = v[e] >= T;
        const int at = c ? off : CAND_CAP;
        sh.ckey[at] = float_key(v[e]);
        sh.cid[at] = id[e];
        off += c;
      }
      __syncthreads();
      select_candidates(Q, kk, sh, emit);
      return;
    }
    // 4. raise T: histogram of {v >= T} over [T, max]; the new T stays <= the
    //    kk-th largest value and strictly increases
    float hi = -INFINITY;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (v[e] >= T) hi = fmaxf(hi, v[e]);
    float lo;
    minmax(INFINITY, hi, sh, &lo, &hi);
    const Buckets bk = make_buckets(T, hi);
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (v[e] >= T) atomicAdd(&sh.hist[bk(v[e])], 1);
    __syncthreads();
    find_bin(sh, kk);
    const int B = sh.digit;
    float m = INFINITY, above = INFINITY;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (v[e] >= T && bk(v[e]) >= B) m = fminf(m, v[e]);
      if (v[e] > T) above = fminf(above, v[e]);
    }
    float Tn, An;
    minmax(m, -above, sh, &Tn, &An);
    // more than kk values exceed T here, so the smallest of them is also safe
    T = Tn > T ? Tn : -An;
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
  const bool final_out = ri.nchunks == 1;
  int32_t* out = a.out + (int64_t)r * a.top_k;
  const int km1 = a.top_k - 1;
  const int64_t cbase = ((int64_t)rl * a.n_chunks + c) * km1;
  const float* src = a.scores + (int64_t)rl * a.ld + c0;

  if (kk > 0) {
    // thread t reads scores [t*E, t*E+E) of the chunk with 16-byte loads (score
    // rows are padded to whole chunks, so they stay inside the row); slots past
    // the eligible blocks become NaN (empty)
    float v[E];
    const int s0 = threadIdx.x * E;
    if constexpr (E >= 4) {
#pragma unroll
      for (int e = 0; e < E; e += 4) {
        const float4 x = *(const float4*)(src + s0 + e);
        v[e] = x.x; v[e + 1] = x.y; v[e + 2] = x.z; v[e + 3] = x.w;
      }
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) v[e] = src[s0 + e];
    }
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (s0 + e >= clen) v[e] = __builtin_nanf("");
    int32_t id[E];
#pragma unroll
    for (int e = 0; e < E; ++e) id[e] = c0 + s0 + e;
    // ranks are < kk by construction; the guard keeps a logic error from ever
    // writing outside this row's output
    if (final_out) {
      select_top<E>(v, id, kk, sh, [&](int pos, int32_t i, uint32_t) {
        if (pos < kk) out[pos] = i;
      });
    } else {
      select_top<E>(v, id, kk, sh, [&](int pos, int32_t i, uint32_t key) {
        if (pos < kk) {
          a.cand_key[cbase + pos] = key;
          a.cand_idx[cbase + pos] = i;
        }
      });
    }
  }
  if (final_out) {
    write_tail(a, r, ri);
  } else {
    for (int i = kk + threadIdx.x; i < km1; i += NT) a.cand_key[cbase + i] = 0u;   // unused slots
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
  const int s0 = threadIdx.x * E;
  float v[E];
  int32_t id[E];
  {
    uint32_t k[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int64_t at = base + min(s0 + e, nslots - 1);
      k[e] = a.cand_key[at];
      id[e] = a.cand_idx[at];
    }
#pragma unroll
    for (int e = 0; e < E; ++e) v[e] = (s0 + e < nslots && k[e] != 0u) ? key_float(k[e]) : __builtin_nanf("");
  }
  int32_t* out = a.out + (int64_t)r * a.top_k;
  if (ri.need > 0)
    select_top<E>(v, id, ri.need, sh, [&](int pos, int32_t i, uint32_t) {
      if (pos < ri.need) out[pos] = i;
    });
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
