// Learned sparse selection: keep the query's own block plus the k'-1 best-scoring
// earlier blocks (k' = min(top_k, b_q + 1)), ties to the lower block id, ids out in
// ascending order.  G2C Brief "GLM-5.3-Flash: hybrid attention becomes the product",
// section "DSA keeps selected global access in eleven layers" (top 2048 tokens =
// 512 pooled blocks).
//
// One 512-thread workgroup selects the kk best of a chunk of up to 16384 scores
// held in registers.  Thread t owns the contiguous slots [t*E, t*E+E), so "lower
// slot first" is a per-thread count plus one workgroup prefix sum.  Cross-lane
// steps use DPP; a cross-wave step is one LDS exchange and one barrier (the
// exchange slots alternate between two sets, so no second barrier is needed
// before they are rewritten).  A typical row costs about a dozen barriers.
//   1. Threshold: with m the kk-th largest maximum of 8-score groups, at least kk
//      scores are >= m, so the answer lies in {v >= m}.  A 2048-bucket histogram
//      of the group maxima (linear between their min and max) gives T <= m.
//   2. If fewer than kk scores are > T, T itself is the kk-th largest value: keep
//      every v > T and the first kk - #(v > T) ties in slot order.
//   3. Else if at most 4096 scores are >= T, compact them in slot order into LDS
//      and bucket them linearly over [T, max].  Candidates above the boundary
//      bucket are kept; the few in the boundary bucket are ranked by direct
//      comparison (value, then position).  A boundary bucket holding more than 64
//      candidates is resolved by radix passes over the 11/11/10-bit digits of the
//      order-preserving keys instead.
//   4. Else raise T with a histogram of the scores >= T and repeat (T strictly
//      increases, so this ends; typical rows never get here).
// Used for rows of one chunk (prefill rows); longer rows and the decode rows are
// selected by select.hpp (in the decode scoring launch, or select_kernel).
#include "kernels.hpp"

namespace ip {

namespace {

constexpr int NT = 512;
constexpr int NW = NT / 64;
constexpr int NBINS = 2048;
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));
constexpr int CAND_CAP = 8192;           // candidates compacted into LDS (>= top_k - 1)
constexpr int EC = CAND_CAP / NT;        // candidates per thread in the exact select (at most)
constexpr int BND_CAP = 64;              // boundary candidates ranked directly

struct SelShared {
  __attribute__((aligned(16))) int hist[NBINS + 64];   // + one spare bin per lane (never read)
  int xi[2][NW], xj[2][NW];              // per-wave exchange slots, two sets
  float xf[2][NW], xg[2][NW], xh[2][NW];
  int digit, above;
  __attribute__((aligned(16))) uint32_t ckey[CAND_CAP + 64];   // candidates, then the kept
  __attribute__((aligned(16))) int32_t cid[CAND_CAP + 64];      // pairs; + one spare entry per lane
  __attribute__((aligned(16))) uint32_t bkey[BND_CAP + 4];   // boundary candidates
  int bkeep[BND_CAP];                    // boundary candidate i is kept
};

__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Workgroup exchanges: each holds exactly one barrier.  Two consecutive calls
// must use different sets p (a call's slots may still be read by slower waves
// until the next barrier has passed).

// sum of an int; min of a, max of b, min of c
__device__ __forceinline__ void x_stats(int n, float a, float b, float c, SelShared& sh, int p, int* sn,
                                        float* ma, float* mb, float* mc) {
  const int wv = threadIdx.x >> 6;
  n = wave_sum(n);
  a = wave_min(a);
  b = wave_max(b);
  c = wave_min(c);
  if ((threadIdx.x & 63) == 0) { sh.xi[p][wv] = n; sh.xf[p][wv] = a; sh.xg[p][wv] = b; sh.xh[p][wv] = c; }
  __syncthreads();
  int s = 0;
  float x = INFINITY, y = -INFINITY, z = INFINITY;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    s += sh.xi[p][i];
    x = fminf(x, sh.xf[p][i]);
    y = fmaxf(y, sh.xg[p][i]);
    z = fminf(z, sh.xh[p][i]);
  }
  *sn = s;
  *ma = x;
  *mb = y;
  *mc = z;
}

// min of a and of b
__device__ __forceinline__ void x_min2(float a, float b, SelShared& sh, int p, float* ma, float* mb) {
  const int wv = threadIdx.x >> 6;
  a = wave_min(a);
  b = wave_min(b);
  if ((threadIdx.x & 63) == 0) { sh.xf[p][wv] = a; sh.xh[p][wv] = b; }
  __syncthreads();
  float x = INFINITY, y = INFINITY;
#pragma unroll
  for (int i = 0; i < NW; ++i) { x = fminf(x, sh.xf[p][i]); y = fminf(y, sh.xh[p][i]); }
  *ma = x;
  *mb = y;
}

// exclusive prefix of x over the threads, its total, and the sum of y
__device__ __forceinline__ int x_scan(int x, int y, SelShared& sh, int p, int* total, int* ysum) {
  const int wv = threadIdx.x >> 6;
  const int incl = wave_incl_scan(x);
  y = wave_sum(y);
  if ((threadIdx.x & 63) == 0) { sh.xi[p][wv] = lane63(incl); sh.xj[p][wv] = y; }
  __syncthreads();
  int before = 0, tot = 0, ys = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int c = sh.xi[p][i];
    before += i < wv ? c : 0;
    tot += c;
    ys += sh.xj[p][i];
  }
  *total = tot;
  *ysum = ys;
  return before + incl - x;
}

// Histogram scan by the first wave, in two levels: lane i sums the 32 bins below
// NBINS - 32 i (descending) and a wave scan finds the lane c whose range holds
// the bin d with count(bins > d) < remaining <= count(bins >= d); then lane t
// takes bin (c's top) - t and a second wave scan finds d.  Writes sh.digit /
// sh.above and clears the histogram for the next pass.  Enters after the barrier
// that completed the histogram; one barrier.  Needs 1 <= remaining <= total.
__device__ __forceinline__ void find_bin(SelShared& sh, int remaining) {
  if (threadIdx.x < 64) {
    constexpr int BW = NBINS / 64;
    const int lane = threadIdx.x;
    const int lo = NBINS - BW * (lane + 1);    // this lane's bins [lo, lo + BW)
    int sum = 0;
#pragma unroll
    for (int i = 0; i < BW; i += 4) {
      const i32x4_t x = *(const i32x4_t*)&sh.hist[lo + i];
      sum += x[0] + x[1] + x[2] + x[3];
    }
    const int incl = wave_incl_scan(sum);
    const int before = incl - sum;             // values in bins >= lo + BW
    const uint64_t m = __ballot(before < remaining && incl >= remaining);
    const int c = m ? __ffsll((unsigned long long)m) - 1 : 0;
    const int ctop = NBINS - 1 - BW * c;       // lane c's highest bin
    const int h = lane < BW ? sh.hist[ctop - lane] : 0;
    const int incl2 = wave_incl_scan(h);
    const int before2 = __shfl(before, c) + incl2 - h;
    const uint64_t m2 = __ballot(lane < BW && before2 < remaining && before2 + h >= remaining);
    if (m2 && lane == __ffsll((unsigned long long)m2) - 1) {
      sh.digit = ctop - lane;
      sh.above = before2;
    }
    // in issue order after the reads above (one wave's LDS accesses stay ordered)
#pragma unroll
    for (int i = 0; i < BW; i += 4) *(i32x4_t*)&sh.hist[lo + i] = i32x4_t{0, 0, 0, 0};
  }
  __syncthreads();
}

// monotone map of a float range onto the histogram bins
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

// Exact select over the compacted candidates (sh.ckey / sh.cid [0..M), key 0 =
// empty slot), all in [lo, hi], 1 <= kk <= #non-empty: the kk best, ties to the
// lower candidate position, are left in sh.ckey / sh.cid [0..kk) in candidate
// order once the caller's next barrier has passed.  Enters right after a barrier;
// its first exchange uses set 0.
template <int EC>
__device__ __forceinline__ void select_candidates_ec(int M, int kk, float lo, float hi, SelShared& sh) {
  const int cb = threadIdx.x * EC;
  const int lane = threadIdx.x & 63;
  uint32_t key[EC];
  int32_t cid[EC];
  // 16-byte LDS reads (a lane's slots are contiguous; the arrays end past
  // NT * EC), then the slots past M are emptied
#pragma unroll
  for (int e = 0; e < EC; e += 4) {
    const u32x4_t k4 = *(const u32x4_t*)&sh.ckey[cb + e];
    const u32x4_t i4 = *(const u32x4_t*)&sh.cid[cb + e];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      key[e + i] = cb + e + i < M ? k4[i] : 0u;
      cid[e + i] = (int32_t)i4[i];
    }
  }
  uint32_t sel = 0;                       // bit e: candidate e is kept
  if (kk >= M) {
#pragma unroll
    for (int e = 0; e < EC; ++e) sel |= (uint32_t)(key[e] != 0u) << e;
  } else {
    const Buckets bk = make_buckets(lo, hi);
    int bin[EC];
#pragma unroll
    for (int e = 0; e < EC; ++e) {
      bin[e] = key[e] ? bk(key_float(key[e])) : -1;
      atomicAdd(&sh.hist[key[e] ? bin[e] : NBINS + lane], 1);   // empty slots: this lane's spare bin
    }
    __syncthreads();
    find_bin(sh, kk);
    const int B = sh.digit;
    const int remaining = kk - sh.above;  // boundary candidates still to keep
    int nb = 0;
#pragma unroll
    for (int e = 0; e < EC; ++e) {
      sel |= (uint32_t)(bin[e] > B) << e;
      nb += bin[e] == B;
    }
    int NB, unused;
    int bpos = x_scan(nb, 0, sh, 1, &NB, &unused);
    if (NB <= BND_CAP) {
      // one wave ranks the boundary candidates (lane i holds the i-th in candidate
      // order): a higher key, or an equal key at a lower position, ranks before
      // it.  Entries NB .. 63 are zero keys, which never rank before one.
#pragma unroll
      for (int e = 0; e < EC; ++e)
        if (bin[e] == B) sh.bkey[bpos++] = key[e];
      if ((int)threadIdx.x >= NB && threadIdx.x < 64) sh.bkey[threadIdx.x] = 0u;
      __syncthreads();
      if (threadIdx.x < 64) {
        const uint32_t ki = sh.bkey[lane];
        int rank = 0;
#pragma unroll 1
        for (int j = 0; j < NB; j += 4) {
          const u32x4_t k4 = *(const u32x4_t*)&sh.bkey[j];
#pragma unroll
          for (int i = 0; i < 4; ++i) rank += k4[i] > ki || (k4[i] == ki && j + i < lane);
        }
        sh.bkeep[lane] = rank < remaining;
      }
      __syncthreads();
      bpos -= nb;
#pragma unroll
      for (int e = 0; e < EC; ++e) {
        if (bin[e] == B) {
          sel |= (uint32_t)sh.bkeep[bpos] << e;
          ++bpos;
        }
      }
    } else {
      // a crowded boundary bucket: exact digits of its keys
      uint32_t prefix = 0, pmask = 0;
      int rem = remaining;
#pragma unroll 1
      for (int pass = 0; pass < 3; ++pass) {
        const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
        const uint32_t dmask = pass == 2 ? 0x3FFu : 0x7FFu;
#pragma unroll
        for (int e = 0; e < EC; ++e)
          if (bin[e] == B && (key[e] & pmask) == prefix) atomicAdd(&sh.hist[(key[e] >> shift) & dmask], 1);
        __syncthreads();
        find_bin(sh, rem);
        rem -= sh.above;
        prefix |= (uint32_t)sh.digit << shift;
        pmask |= dmask << shift;
      }
      // keys > prefix, then the first rem keys == prefix in candidate order
      int nt = 0;
#pragma unroll
      for (int e = 0; e < EC; ++e) nt += bin[e] == B && key[e] == prefix;
      int tot;
      int tie = x_scan(nt, 0, sh, 1, &tot, &unused);
#pragma unroll
      for (int e = 0; e < EC; ++e) {
        if (bin[e] == B) {
          const bool eq = key[e] == prefix;
          sel |= (uint32_t)(key[e] > prefix || (eq && tie < rem)) << e;
          tie += eq;
        }
      }
    }
  }
  int ns = 0;
#pragma unroll
  for (int e = 0; e < EC; ++e) ns += (sel >> e) & 1u;
  int tot, unused;
  int off = x_scan(ns, 0, sh, 0, &tot, &unused);
  // every candidate was read before the barrier above, so the store is free;
  // dropped ones go to this lane's spare entry (no branch, no shared address)
#pragma unroll
  for (int e = 0; e < EC; ++e) {
    const bool k = (sel >> e) & 1u;
    const int at = k ? off : CAND_CAP + lane;
    sh.ckey[at] = key[e];
    sh.cid[at] = cid[e];
    off += k;
  }
}

// the exact select with 8 candidate slots per thread while they suffice (MAXM:
// a bound on M known at compile time)
template <int MAXM>
__device__ __forceinline__ void select_candidates(int M, int kk, float lo, float hi, SelShared& sh) {
  if (MAXM <= NT * 8 || M <= NT * 8) select_candidates_ec<8>(M, kk, lo, hi, sh);
  else select_candidates_ec<EC>(M, kk, lo, hi, sh);
}

// The kk best of v (NaN = empty), ties to the lower slot, 1 <= kk <= #values:
// their (order-preserving key, id) pairs are left in sh.ckey / sh.cid [0..kk) in
// slot order once the caller's next barrier has passed.
template <int E, class IdOf>
__device__ __forceinline__ void select_top(const float (&v)[E], IdOf id, int kk, SelShared& sh) {
  constexpr int GS = E >= 8 ? 8 : E;          // scores per group maximum
  constexpr int NG = E / GS;
  const int lane = threadIdx.x & 63;
  // zeroed before the first exchange's barrier; find_bin re-zeroes what it reads
  for (int i = threadIdx.x; i < NBINS; i += NT) sh.hist[i] = 0;

  // 1. T <= the kk-th largest group maximum (or the smallest value if there are
  //    fewer than kk groups)
  float gm[NG];
  int ngv = 0;
  float glo = INFINITY, vhi = -INFINITY, vlo = INFINITY;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    float m = v[g * GS], mn = v[g * GS];
#pragma unroll
    for (int i = 1; i < GS; ++i) {
      m = fmaxf(m, v[g * GS + i]);               // NaN-ignoring
      mn = fminf(mn, v[g * GS + i]);
    }
    gm[g] = m;
    if (!__builtin_isnan(m)) {
      ++ngv;
      glo = fminf(glo, m);
      vhi = fmaxf(vhi, m);
      vlo = fminf(vlo, mn);
    }
  }
  int nval;
  x_stats(ngv, glo, vhi, vlo, sh, 0, &nval, &glo, &vhi, &vlo);
  float T = vlo;
  int par = 1;
  if (kk <= nval) {
    const Buckets bk = make_buckets(glo, vhi);
#pragma unroll
    for (int g = 0; g < NG; ++g)
      atomicAdd(&sh.hist[__builtin_isnan(gm[g]) ? NBINS + lane : bk(gm[g])], 1);
    __syncthreads();
    find_bin(sh, kk);
    const int B = sh.digit;
    float m = INFINITY;
#pragma unroll
    for (int g = 0; g < NG; ++g)
      if (!__builtin_isnan(gm[g]) && bk(gm[g]) >= B) m = fminf(m, gm[g]);
    float unusedf;
    x_min2(m, INFINITY, sh, 0, &T, &unusedf);
  }

  // T is always one of the values, so every candidate lies in [T, vhi]
#pragma unroll 1
  for (;;) {
    int g = 0, q = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      g += v[e] > T;
      q += v[e] >= T;
    }
    int Q, G;
    const int qoff = x_scan(q, g, sh, par, &Q, &G);
    par ^= 1;
    if (G < kk) {
      // 2. T is the kk-th largest value: every v > T, then the first kk - G ties
      int nt = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) nt += v[e] == T;
      int tot, unused;
      int tie = x_scan(nt, 0, sh, par, &tot, &unused);
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
      int off = x_scan(ns, 0, sh, par ^ 1, &tot, &unused);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const bool k = (smask >> e) & 1ull;
        const int at = k ? off : CAND_CAP + lane;
        sh.ckey[at] = float_key(v[e]);
        sh.cid[at] = id(e);
        off += k;
      }
      return;
    }
    if (Q <= CAND_CAP) {
      // 3. compact {v >= T} in slot order (the others write this lane's spare
      //    entry: no branch, no shared address), then the exact select on them
      int off = qoff;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const bool c = v[e] >= T;
        const int at = c ? off : CAND_CAP + lane;
        sh.ckey[at] = float_key(v[e]);
        sh.cid[at] = id(e);
        off += c;
      }
      __syncthreads();
      select_candidates<E * NT>(Q, kk, T, vhi, sh);
      return;
    }
    // 4. raise T: histogram of {v >= T} over [T, vhi]; the new T stays <= the
    //    kk-th largest value and strictly increases
    const Buckets bk = make_buckets(T, vhi);
#pragma unroll
    for (int e = 0; e < E; ++e) atomicAdd(&sh.hist[v[e] >= T ? bk(v[e]) : NBINS + lane], 1);
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
    x_min2(m, above, sh, par ^ 1, &Tn, &An);
    // more than kk values exceed T here, so the smallest of them is also safe
    T = Tn > T ? Tn : An;
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

// The row's output from the staged pairs (sh.cid [0..kept), kept = need):
// the kept ids, the own block, then -1 padding; coalesced.
__device__ __forceinline__ void write_row(const TopkArgs& a, int r, const RowInfo& ri, const SelShared& sh) {
  int32_t* out = a.out + (int64_t)r * a.top_k;
  for (int i = threadIdx.x; i < a.top_k; i += NT)
    out[i] = i < ri.need ? sh.cid[i] : (i == ri.need ? ri.bq : -1);
}

// E scores per thread, one chunk per row.
template <int E>
__global__ __launch_bounds__(NT) void topk_chunk_kernel(TopkArgs a) {
  __shared__ SelShared sh;
  const int rl = blockIdx.y, r = a.row0 + rl, c = blockIdx.x;
  const RowInfo ri = row_info(a, r);
  if (c >= ri.nchunks) return;
  const int c0 = c * a.chunk;
  const int clen = max(0, min(a.chunk, ri.nel - c0));
  const int kk = min(ri.need, clen);
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
    const int id0 = c0 + s0;
    select_top<E>(v, [=](int e) { return id0 + e; }, kk, sh);
  }
  __syncthreads();
  write_row(a, r, ri, sh);      // kk == need here
}

template <int E>
void launch_chunks(const TopkArgs& a, hipStream_t s) {
  launch(K_TOPK, topk_chunk_kernel<E>, dim3(a.n_chunks, a.n_rows), dim3(NT), s, a);
}

int per_thread(int n) {
  int e = 1;
  while (e < 32 && e * NT < n) e *= 2;
  return e;
}

}  // namespace

// Scores per chunk workgroup for rows of up to max_blocks eligible blocks: one
// chunk of 512 x E (E a power of two up to 32, else 36, 40 or 48); 0 when a row
// does not fit one chunk.
int topk_chunk_size(int max_blocks) {
  if (max_blocks <= TOPK_MAX_CHUNK) return NT * per_thread(max_blocks);
  for (int e : {36, 40, 48})
    if (max_blocks <= NT * e) return NT * e;
  return 0;
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
  if (a.n_rows <= 0) return hipSuccess;
  if (a.n_chunks != 1 || a.chunk <= 0 || a.chunk > a.ld) return hipErrorInvalidValue;   // one whole chunk per padded row
  switch (a.chunk / NT) {
    case 48: launch_chunks<48>(a, s); break;
    case 40: launch_chunks<40>(a, s); break;
    case 36: launch_chunks<36>(a, s); break;
    case 1: launch_chunks<1>(a, s); break;
    case 2: launch_chunks<2>(a, s); break;
    case 4: launch_chunks<4>(a, s); break;
    case 8: launch_chunks<8>(a, s); break;
    case 16: launch_chunks<16>(a, s); break;
    default: launch_chunks<32>(a, s); break;
  }
  return hipGetLastError();
}

}  // namespace ip
