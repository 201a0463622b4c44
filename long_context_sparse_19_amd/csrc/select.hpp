// Learned sparse selection of one query row: keep the query's own block plus the
// k'-1 best-scoring earlier blocks (k' = min(top_k, b_q + 1)), ties to the lower
// block id, ids out in ascending order.  G2C Brief "GLM-5.3-Flash: hybrid
// attention becomes the product", section "DSA keeps selected global access in
// eleven layers" (top 2048 tokens = 512 pooled blocks).
//
// Scores are compared through their order-preserving uint32 keys.  Every
// threshold below is found by narrowing a key interval: the keys of the interval
// are bucketed linearly over it (2048 buckets), the bucket that holds the wanted
// rank becomes the next interval, until it holds few keys, is kept whole, or is a
// single key.  That works for any score distribution, heavy tails included.  The
// scoring kernels also write, for every group of 16 consecutive blocks, the
// largest score of the group.  One workgroup selects the need = k'-1 best of the
// row's n eligible scores:
//   1. a key bound G from the group maxima: the lower end of a narrow interval
//      holding the need-th largest maximum.  At least need maxima -- so at least
//      need scores -- have keys >= G, so every winner has a key >= G, and so has
//      the maximum of its group;
//   2. the scores with keys >= G: a superset of the winners, typically a few
//      percent larger than need, compacted in ascending id order into LDS.  Rows
//      of up to 32 scores per thread are read whole in one pass (their group
//      maxima are taken in registers); longer rows read the stored maxima first
//      and then only the groups whose maximum reaches G;
//   3. the exact select among those candidates, narrowing to the need-th largest
//      key; equal keys at the boundary go to the lower id.
// Rows with fewer than 2 need groups take the bound from the scores themselves.
// When the candidates do not fit in LDS (scores that are largely equal), a radix
// select over the keys of the whole row runs instead.
//
// Scores and group maxima written by other workgroups of the same kernel are read
// with device-coherent loads (they bypass this die's L2, which may not have seen
// them); data written by an earlier kernel reads the same way.  The selected ids
// are stored device-coherently too, so that a consumer in the same launch (the
// fused decode step's attention) can read them once the row is published.
#pragma once
#include "kernels.hpp"

namespace ip {
namespace sel {

typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int GROUP = 16;          // scores per group maximum
constexpr int NBINS = 2048;        // buckets of a key interval (and one 11-bit digit)
constexpr int CG_CAP = 2048;       // candidate groups held in LDS
constexpr int C_CAP = 4096;        // candidate scores held in LDS (> top_k - 1)
constexpr int RE = 16;             // scores per thread per tile of the row-wide radix path
constexpr int REFINE = 32;         // a bound's interval holding more keys is narrowed further
constexpr int VB = 16;             // values of the bound's source per thread per tile

template <int NT>
struct Shared {
  static constexpr int NW = NT / 64;
  int hist[NBINS + 64];            // + one spare bin per lane for empty slots (never read)
  int xi[2][NW], xj[2][NW];        // per-wave exchange slots, two sets
  int digit, above, count;         // find_bin's result
  int wn[2][NW];                   // per-wave counts, two sets
  int fb[NW];                      // find_bin's per-wave bin sums
  int cg[CG_CAP];                  // candidate groups, ascending
  uint32_t ckey[C_CAP + 64];       // candidates (order-preserving key, id), ascending id;
  int32_t cid[C_CAP + 64];         // + one spare entry per lane
  uint64_t wl[NW * 16];            // the waves' lists of a workgroup list (see wave_list)
  uint2 wm[NW];
};

// digit l of a key: bits 31..21, 20..10, 9..0
__device__ __forceinline__ int dshift(int l) { return l == 0 ? 21 : (l == 1 ? 10 : 0); }
__device__ __forceinline__ uint32_t dmask(int l) { return l == 2 ? 0x3FFu : 0x7FFu; }
__device__ __forceinline__ int digit_of(uint32_t k, int l) { return (int)((k >> dshift(l)) & dmask(l)); }

// ---------------------------------------------------------------- device-coherent access
template <typename T>
__device__ __forceinline__ void st_agent(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T ld_agent(const T* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Device-coherent 16-byte reads of data other workgroups of the kernel stored with
// st_agent: plain buffer loads with the device-scope cache policy (sc1), which the
// compiler keeps in flight together (an atomic load waits for each one in turn).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t dev_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0xFFFFFFFF, 0x00020000);
}
__device__ __forceinline__ u32x4_t ld16_dev(__amdgpu_buffer_rsrc_t rs, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(rs, byte_off, 0, 16 /* sc1 */);
}

// ---------------------------------------------------------------- workgroup exchanges
// Each holds exactly one barrier.  Two consecutive calls must use different slot
// sets p (a call's slots may still be read by slower waves until the next barrier).

// exclusive prefix of x over the threads (thread order), its total, and the sum of y
template <int NT>
__device__ __forceinline__ int x_scan(int x, int y, Shared<NT>& sh, int p, int* total, int* ysum) {
  const int wv = threadIdx.x >> 6;
  const int incl = wave_incl_scan(x);
  y = wave_sum(y);
  if ((threadIdx.x & 63) == 0) { sh.xi[p][wv] = lane63(incl); sh.xj[p][wv] = y; }
  __syncthreads();
  int before = 0, tot = 0, ys = 0;
#pragma unroll
  for (int i = 0; i < Shared<NT>::NW; ++i) {
    const int c = sh.xi[p][i];
    before += i < wv ? c : 0;
    tot += c;
    ys += sh.xj[p][i];
  }
  *total = tot;
  *ysum = ys;
  return before + incl - x;
}

// min and max of unsigned keys over the threads (DPP within waves, one exchange)
__device__ __forceinline__ uint32_t wave_umin(uint32_t x) {
  x = min(x, (uint32_t)dpp_i<0xB1>((int)0xFFFFFFFF, (int)x));
  x = min(x, (uint32_t)dpp_i<0x4E>((int)0xFFFFFFFF, (int)x));
  x = min(x, (uint32_t)dpp_i<0x141>((int)0xFFFFFFFF, (int)x));
  x = min(x, (uint32_t)dpp_i<0x140>((int)0xFFFFFFFF, (int)x));
  x = min(x, (uint32_t)dpp_i<0x142, 0xA>((int)0xFFFFFFFF, (int)x));
  x = min(x, (uint32_t)dpp_i<0x143, 0xC>((int)0xFFFFFFFF, (int)x));
  return (uint32_t)lane63((int)x);
}
__device__ __forceinline__ uint32_t wave_umax(uint32_t x) {
  x = max(x, (uint32_t)dpp_i<0xB1>(0, (int)x));
  x = max(x, (uint32_t)dpp_i<0x4E>(0, (int)x));
  x = max(x, (uint32_t)dpp_i<0x141>(0, (int)x));
  x = max(x, (uint32_t)dpp_i<0x140>(0, (int)x));
  x = max(x, (uint32_t)dpp_i<0x142, 0xA>(0, (int)x));
  x = max(x, (uint32_t)dpp_i<0x143, 0xC>(0, (int)x));
  return (uint32_t)lane63((int)x);
}
template <int NT>
__device__ __forceinline__ void x_uminmax(uint32_t& mn, uint32_t& mx, Shared<NT>& sh, int p) {
  const int wv = threadIdx.x >> 6;
  mn = wave_umin(mn);
  mx = wave_umax(mx);
  if ((threadIdx.x & 63) == 0) { sh.xi[p][wv] = (int)mn; sh.xj[p][wv] = (int)mx; }
  __syncthreads();
  uint32_t a = 0xFFFFFFFFu, b = 0u;
#pragma unroll
  for (int i = 0; i < Shared<NT>::NW; ++i) { a = min(a, (uint32_t)sh.xi[p][i]); b = max(b, (uint32_t)sh.xj[p][i]); }
  mn = a;
  mx = b;
}

// wave_excl of a flag (x in {0, 1}): one ballot instead of a scan
__device__ __forceinline__ int wave_excl_bit(bool x, int& total) {
  const uint64_t m = __ballot(x);
  total = __popcll(m);
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// exclusive prefix of x over the lanes, and the wave total
__device__ __forceinline__ int wave_excl(int x, int& total) {
  const int incl = wave_incl_scan(x);
  total = lane63(incl);
  return incl - x;
}

// Histogram scan over bins [0, NB) by the whole workgroup: thread t owns the
// C = NB / NT bins below NB - C t (descending order over the threads), reads them
// with 16-byte LDS reads (adjacent threads, adjacent addresses: no bank
// conflicts), and one workgroup scan of the per-thread sums finds the thread whose
// bins hold the bin d with count(bins > d) < remaining <= count(bins >= d); it
// resolves d among its own bins.  Leaves sh.digit = d, sh.above = count(bins > d)
// and sh.count = count(bin d), and clears the bins for the next use.  Enters after
// the barrier that completed the histogram; two barriers.  Needs 1 <= remaining
// <= total.
template <int NB, int NT>
__device__ __forceinline__ void find_bin(Shared<NT>& sh, int remaining) {
  constexpr int C = NB / NT;
  static_assert(C >= 4 && C % 4 == 0, "bins per thread");
  const int t = threadIdx.x, wv = t >> 6;
  const int lo = NB - C * (t + 1);
  int v[C];
#pragma unroll
  for (int q = 0; q < C; q += 4) {
    const i32x4_t x = *(const i32x4_t*)&sh.hist[lo + q];
    v[q] = x[0]; v[q + 1] = x[1]; v[q + 2] = x[2]; v[q + 3] = x[3];
  }
  int sum = 0;
#pragma unroll
  for (int q = 0; q < C; ++q) sum += v[q];
  int wt;
  const int excl = wave_excl(sum, wt);
  if ((t & 63) == 0) sh.fb[wv] = wt;
  // every read above is done before the bins are cleared (in issue order for this
  // wave; the other waves read only their own bins)
#pragma unroll
  for (int q = 0; q < C; q += 4) *(i32x4_t*)&sh.hist[lo + q] = i32x4_t{0, 0, 0, 0};
  __syncthreads();
  int before = excl;
#pragma unroll
  for (int i = 0; i < Shared<NT>::NW; ++i) before += i < wv ? sh.fb[i] : 0;
  if (before < remaining && before + sum >= remaining) {
    int acc = before;
#pragma unroll
    for (int q = C - 1; q >= 0; --q) {
      if (acc < remaining && acc + v[q] >= remaining) {
        sh.digit = lo + q;
        sh.above = acc;
        sh.count = v[q];
      }
      acc += v[q];
    }
  }
  __syncthreads();
}

// Histogram update of one value per lane (an LDS atomic costs the same per wave
// instruction whether its lanes' buckets are spread or shared).
__device__ __forceinline__ void hist_add(int* hist, int bin, bool valid) {
  if (valid) atomicAdd(&hist[bin], 1);
}

// Narrows to the key interval [base, base + width) holding the need-th largest of
// the keys the threads hold (key 0 = none; need <= their number): the interval of
// all keys, then repeatedly the one of its 2048 linear buckets that holds the
// rank, until that bucket holds at most `stop` keys (stop = 0: never), is kept
// whole, or is a single key (width 1).  On return every key >= base + width
// ranks above the need-th, and `rem` (1 .. count) keys of the interval complete
// the need; whole: rem equals the interval's count.  Enters after a barrier.
template <int NT, int E>
__device__ __forceinline__ void narrow(const uint32_t (&key)[E], int need, int stop, Shared<NT>& sh,
                                       uint32_t& base, uint64_t& width, int& rem, bool& whole, uint32_t kmin = 0,
                                       uint32_t kmax = 0) {
  // the keys' range, unless the caller knows it (kmax != 0)
  uint32_t mn = kmin, mx = kmax;
  if (!kmax) {
    mn = 0xFFFFFFFFu;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (key[e]) { mn = min(mn, key[e]); mx = max(mx, key[e]); }
    x_uminmax(mn, mx, sh, 0);
  }
  base = mn;
  width = (uint64_t)(mx - mn) + 1;
  const uint32_t span = mx - mn;
  int shift = (span >> 11) ? 32 - __clz((int)(span >> 11)) : 0;   // span >> shift < 2048
  rem = need;
  whole = false;
#pragma unroll 1
  for (;;) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const bool in = key[e] && key[e] >= base && (uint64_t)(key[e] - base) < width;
      hist_add(sh.hist, in ? (int)((key[e] - base) >> shift) : 0, in);
    }
    __syncthreads();
    find_bin<NBINS>(sh, rem);
    rem -= sh.above;
    const int cnt = sh.count;
    base += (uint32_t)sh.digit << shift;
    width = (uint64_t)1 << shift;
    whole = cnt == rem;
    if (whole || shift == 0 || cnt <= stop) break;
    shift = shift > 11 ? shift - 11 : 0;
  }
}

// ---------------------------------------------------------------- ordered compaction
// A workgroup's waves each hold `n` consecutive entries of an ascending list and
// keep some of them: the kept entries are written to dst [0, ...) in list order.
// Wave w's entries come first in the list when w is lower; within a wave lane l's
// entries of round q come before lane l+1's, and round q's before round q+1's.
// Counting and writing are two steps around one exchange of the wave totals.

// wave totals -> this wave's offset in the workgroup and the workgroup total (one
// barrier; set p alternates between consecutive calls)
template <int NT>
__device__ __forceinline__ int wave_base(int wave_total, Shared<NT>& sh, int p, int& all) {
  const int wv = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) sh.wn[p][wv] = wave_total;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < Shared<NT>::NW; ++i) {
    const int c = sh.wn[p][i];
    before += i < wv ? c : 0;
    tot += c;
  }
  all = tot;
  return before;
}

// Where a selection puts the row's ids (positions 0 .. top_k - 1): the kept ids in
// ascending id order, then the query's own block at position need, then -1.
// RowOut: every position, device-coherent stores to the row of `out`.  SliceOut:
// positions [lo, hi) only, into LDS (lds[pos - lo]), for a workgroup that consumes
// one slice of the row itself.
struct RowOut {
  int32_t* out;
  __device__ __forceinline__ void put(int pos, int32_t id) const { st_agent(out + pos, id); }
  template <int NT>
  __device__ __forceinline__ void tail(int need, int bq, int top_k) const {
    for (int i = need + threadIdx.x; i < top_k; i += NT) st_agent(out + i, i == need ? bq : -1);
  }
};
struct SliceOut {
  int32_t* lds;
  int lo, hi;                                    // hi <= top_k
  __device__ __forceinline__ void put(int pos, int32_t id) const {
    if (pos >= lo && pos < hi) lds[pos - lo] = id;
  }
  template <int NT>
  __device__ __forceinline__ void tail(int need, int bq, int top_k) const {
    for (int i = max(need, lo) + threadIdx.x; i < hi; i += NT) lds[i - lo] = i == need ? bq : -1;
  }
};

// Keeps the need best (ties to the lower id) of a flat candidate list held in
// registers: wave w holds entries [w per, (w+1) per), lane l of round i entry
// w per + 64 i + l (key 0 = an empty slot; more than need entries in all), and
// puts their ids at positions [0, need) of `out` in list (ascending id) order.  Writes nothing
// and returns false when `limit` exceeds the lower end of the interval found for
// the need-th key (the caller's lists may then miss a winner); `limit` 0 never
// does.  kmax != 0: [kmin, kmax] is the keys' range.  Enters after a barrier.
template <int NT, int E, class O>
__device__ __forceinline__ bool keep_best_regs(const uint32_t (&key)[E], const int32_t (&cid)[E], int need,
                                               const O& out, Shared<NT>& sh, uint32_t limit, uint32_t kmin,
                                               uint32_t kmax) {
  uint32_t base;
  uint64_t width;
  int rem;
  bool whole;
  narrow<NT, E>(key, need, 0, sh, base, width, rem, whole, kmin, kmax);
  if (limit > base) return false;                 // uniform
  const uint64_t top = (uint64_t)base + width;    // keys >= top are kept
  // ties at the boundary (width 1, not kept whole) go to the lowest ids: their
  // rank in list order
  int tie_w = 0;
  int pos[E];
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const bool in = key[i] && key[i] >= base && (uint64_t)key[i] < top;
    int t;
    pos[i] = tie_w + wave_excl_bit(in, t);
    tie_w += t;
  }
  int all;
  const int tie0 = whole ? 0 : wave_base(tie_w, sh, 1, all);
  bool k[E];
  int kept_w = 0;
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const bool in = key[i] && key[i] >= base && (uint64_t)key[i] < top;
    k[i] = (uint64_t)key[i] >= top || (in && (whole || tie0 + pos[i] < rem));
    int t;
    pos[i] = kept_w + wave_excl_bit(k[i], t);     // now: this entry's place among the wave's kept
    kept_w += t;
  }
  const int off = wave_base(kept_w, sh, 0, all);
#pragma unroll
  for (int i = 0; i < E; ++i)
    if (k[i]) out.put(off + pos[i], cid[i]);
  return true;
}

// keep_best_regs over the flat candidate list sh.ckey / sh.cid [0, M), M <= C_CAP.
template <int NT>
__device__ __noinline__ bool keep_best(int M, int need, int32_t* out, Shared<NT>& sh, uint32_t limit = 0) {
  constexpr int NW = Shared<NT>::NW, E = C_CAP / NT;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int per = (M + NW - 1) / NW;
  const int lo = wv * per, hi = min(M, lo + per);
  uint32_t key[E];
  int32_t cid[E];
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const int at = lo + 64 * i + lane;
    key[i] = at < hi ? sh.ckey[at] : 0u;          // key 0: no entry (no score maps to it)
    cid[i] = at < hi ? sh.cid[at] : 0;
  }
  return keep_best_regs<NT, E>(key, cid, need, RowOut{out}, sh, limit, 0u, 0u);
}

// Radix select over the order-preserving keys of the whole row (any score
// distribution): the need-th largest key digit by digit, then the kept ids (keys
// above it, then ties in id order) are written straight to `out`.
template <int NT>
__device__ __noinline__ void radix_row(const float* S, int nel, int need, int bq, int top_k, int32_t* out,
                                       Shared<NT>& sh) {
  const int t0 = threadIdx.x * RE;
  const __amdgpu_buffer_rsrc_t rs = dev_rsrc(S);
  auto load_keys = [&](int base, uint32_t (&key)[RE]) {
    const int j0 = base + t0;
    u32x4_t v[RE / 4];
    // rows are padded past nel to whole tiles of 1024: a started chunk stays inside
#pragma unroll
    for (int q = 0; q < RE / 4; ++q) v[q] = j0 < nel ? ld16_dev(rs, (uint32_t)(j0 + 4 * q) * 4u) : u32x4_t{};
#pragma unroll
    for (int e = 0; e < RE; ++e) key[e] = j0 + e < nel ? float_key(__uint_as_float(v[e >> 2][e & 3])) : 0u;
  };
  for (int i = threadIdx.x; i < NBINS; i += NT) sh.hist[i] = 0;
  __syncthreads();
  uint32_t prefix = 0, pmask = 0;
  int rem = need;
#pragma unroll 1
  for (int l = 0; l < 3; ++l) {
#pragma unroll 1
    for (int base = 0; base < nel; base += NT * RE) {
      uint32_t key[RE];
      load_keys(base, key);
#pragma unroll
      for (int e = 0; e < RE; ++e) {
        const bool in = key[e] && (key[e] & pmask) == prefix;
        hist_add(sh.hist, in ? digit_of(key[e], l) : 0, in);
      }
    }
    __syncthreads();
    find_bin<NBINS>(sh, rem);
    rem -= sh.above;
    prefix |= (uint32_t)sh.digit << dshift(l);
    pmask |= dmask(l) << dshift(l);
  }
  // prefix is the need-th largest key; keep every key above it and the first rem
  // equal to it, in id order
  int done = 0, ties = 0, par = 0;
#pragma unroll 1
  for (int base = 0; base < nel; base += NT * RE) {
    uint32_t key[RE];
    load_keys(base, key);
    int nt = 0;
#pragma unroll
    for (int e = 0; e < RE; ++e) nt += key[e] == prefix;
    int tt, unused;
    int tie = ties + x_scan(nt, 0, sh, par, &tt, &unused);
    uint32_t km = 0;
    int nk = 0;
#pragma unroll
    for (int e = 0; e < RE; ++e) {
      const bool eq = key[e] == prefix;
      const bool k = key[e] > prefix || (eq && tie < rem);
      tie += eq;
      km |= (uint32_t)k << e;
      nk += k;
    }
    int kt;
    int off = done + x_scan(nk, 0, sh, par ^ 1, &kt, &unused);
#pragma unroll
    for (int e = 0; e < RE; ++e)
      if ((km >> e) & 1u) st_agent(out + off++, (int32_t)(base + t0 + e));
    done += kt;
    ties += tt;
  }
  for (int i = need + threadIdx.x; i < top_k; i += NT) st_agent(out + i, i == need ? bq : -1);
}

// One tile of the bound's source V: wave w holds V [t0 + w 64 VB, + 64 VB), lane l
// of round q the 4 values at t0 + w 64 VB + 256 q + 4 l (coalesced 16-byte loads).
template <int NT>
struct VTile {
  uint32_t k[VB];                                // keys, 0 = none
  __device__ __forceinline__ int first(int t0, int q) const {
    return t0 + (threadIdx.x >> 6) * 64 * VB + 256 * q + 4 * (threadIdx.x & 63);
  }
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rv, int nv, int t0) {
#pragma unroll
    for (int q = 0; q < VB / 4; ++q) {
      const int g = first(t0, q);
      // V is padded past nv (maxima to whole tiles of 64, scores of 1024): a
      // started group of 4 stays inside the row
      const u32x4_t v = g < nv ? ld16_dev(rv, (uint32_t)g * 4u) : u32x4_t{};
#pragma unroll
      for (int e = 0; e < 4; ++e) k[4 * q + e] = g + e < nv ? float_key(__uint_as_float(v[e])) : 0u;
    }
  }
};

// Appends the tile's entries with keys >= G, in order, to dst [n0, cap) (ids for
// dst_id: the entry's index; keys for dst_key when given); returns the new count
// (entries past cap are counted, not stored).  One barrier.
template <int NT>
__device__ __forceinline__ int append_ge(const VTile<NT>& vt, int t0, uint32_t G, int n0, int cap, int32_t* dst_id,
                                         uint32_t* dst_key, Shared<NT>& sh, int p) {
  int pos[VB / 4], wt = 0;
#pragma unroll
  for (int q = 0; q < VB / 4; ++q) {
    int c = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) c += vt.k[4 * q + e] >= G && vt.k[4 * q + e];
    int t;
    pos[q] = wt + wave_excl(c, t);
    wt += t;
  }
  int all;
  const int base = n0 + wave_base(wt, sh, p, all);
#pragma unroll
  for (int q = 0; q < VB / 4; ++q) {
    int at = base + pos[q];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (vt.k[4 * q + e] >= G && vt.k[4 * q + e]) {
        if (at < cap) {
          dst_id[at] = vt.first(t0, q) + e;
          if (dst_key) dst_key[at] = vt.k[4 * q + e];
        }
        ++at;
      }
  }
  return n0 + all;
}

// The selection of one row (called by every thread of the workgroup, after a
// barrier that frees `sh`).  S: the row's scores [0, nel), GM: its group maxima
// [0, ceil(nel / 16)), both padded (scores to whole tiles of 1024, maxima to
// whole tiles of 64); out: [top_k].
template <int NT>
__device__ __noinline__ void select_row(const float* S, const float* GM, int nel, int bq, int top_k, int32_t* out,
                                        Shared<NT>& sh) {
  constexpr int NW = Shared<NT>::NW;
  const int need = min(top_k, bq + 1) - 1;
  if (need == 0 || need >= nel) {
    // the own block alone, or every eligible block (need == nel)
    for (int i = threadIdx.x; i < top_k; i += NT) st_agent(out + i, i < need ? i : (i == need ? bq : -1));
    return;
  }
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int ng = (nel + GROUP - 1) / GROUP;
  const bool direct = ng < 2 * need;             // bound from the scores themselves
  const float* V = direct ? S : GM;              // the values the bound comes from
  const int nv = direct ? nel : ng;
  const __amdgpu_buffer_rsrc_t rv = dev_rsrc(V);
  constexpr int TILE = NT * VB;
  for (int i = threadIdx.x; i < NBINS; i += NT) sh.hist[i] = 0;   // visible after the next barrier

  // 1. the bound G: a one-tile V is narrowed directly; a longer one by the digits
  //    of its keys (one pass over V per digit)
  VTile<NT> vt;
  uint32_t G = 0;
  if (nv <= TILE) {
    vt.load(rv, nv, 0);
    uint32_t base;
    uint64_t width;
    int rem;
    bool whole;
    narrow<NT, VB>(vt.k, need, REFINE, sh, base, width, rem, whole);
    G = base;
  } else {
    uint32_t gmask = 0;
    int rem = need;
#pragma unroll 1
    for (int l = 0; l < 3; ++l) {
#pragma unroll 1
      for (int t0 = 0; t0 < nv; t0 += TILE) {
        vt.load(rv, nv, t0);
#pragma unroll
        for (int e = 0; e < VB; ++e) {
          const bool in = vt.k[e] && (vt.k[e] & gmask) == G;
          hist_add(sh.hist, in ? digit_of(vt.k[e], l) : 0, in);
        }
      }
      __syncthreads();
      find_bin<NBINS>(sh, rem);
      rem -= sh.above;
      G |= (uint32_t)sh.digit << dshift(l);
      gmask |= dmask(l) << dshift(l);
      if (sh.count <= REFINE) break;
    }
  }

  // 2. the entries of V with keys >= G, in order: the candidates (direct), or the
  //    candidate groups
  int nc = 0, par = 0;
#pragma unroll 1
  for (int t0 = 0; t0 < nv; t0 += TILE) {
    if (nv > TILE) vt.load(rv, nv, t0);
    nc = direct ? append_ge<NT>(vt, t0, G, nc, C_CAP, sh.cid, sh.ckey, sh, par)
                : append_ge<NT>(vt, t0, G, nc, CG_CAP, sh.cg, nullptr, sh, par);
    par ^= 1;
  }
  __syncthreads();                                // the list complete
  if (nc > (direct ? C_CAP : CG_CAP)) {
    radix_row<NT>(S, nel, need, bq, top_k, out, sh);
    return;
  }
  int M = nc;
  if (!direct) {
    // 3. the scores with keys >= G of the candidate groups, in order: wave w takes
    //    groups [w pg, (w+1) pg), lane l of round q group w pg + 64 q + l
    constexpr int GR = CG_CAP / NT;               // rounds per wave at most
    const int pg = (nc + NW - 1) / NW;
    const int g0 = wv * pg, g1 = min(nc, g0 + pg);
    const __amdgpu_buffer_rsrc_t rs = dev_rsrc(S);
    uint32_t keep[GR];                            // 16 keep bits per round
    int gid[GR], pos[GR], wt = 0;
    u32x4_t v[GR][GROUP / 4];
#pragma unroll
    for (int q = 0; q < GR; ++q) {
      const int i = g0 + 64 * q + lane;
      gid[q] = i < g1 ? sh.cg[i] : -1;
#pragma unroll
      for (int c = 0; c < GROUP / 4; ++c)
        v[q][c] = gid[q] >= 0 ? ld16_dev(rs, (uint32_t)(gid[q] * GROUP + 4 * c) * 4u) : u32x4_t{};
    }
#pragma unroll
    for (int q = 0; q < GR; ++q) {
      keep[q] = 0;
#pragma unroll
      for (int e = 0; e < GROUP; ++e) {
        const uint32_t kk = float_key(__uint_as_float(v[q][e >> 2][e & 3]));
        keep[q] |= (uint32_t)(gid[q] >= 0 && gid[q] * GROUP + e < nel && kk >= G) << e;
      }
      int t;
      pos[q] = wt + wave_excl(__popc(keep[q]), t);
      wt += t;
    }
    const int base = wave_base(wt, sh, par, M);
#pragma unroll
    for (int q = 0; q < GR; ++q) {
      int at = base + pos[q];
#pragma unroll
      for (int e = 0; e < GROUP; ++e)
        if ((keep[q] >> e) & 1u) {
          if (at < C_CAP) {
            sh.ckey[at] = float_key(__uint_as_float(v[q][e >> 2][e & 3]));
            sh.cid[at] = gid[q] * GROUP + e;
          }
          ++at;
        }
    }
    __syncthreads();                              // the candidates complete
    if (M > C_CAP) {
      radix_row<NT>(S, nel, need, bq, top_k, out, sh);
      return;
    }
  }

  // 4. the exact select among them (M >= need: the entries of V with keys >= G
  //    are candidates, or maxima of candidate groups, themselves)
  if (M > need) {
    keep_best<NT>(M, need, out, sh);
  } else {
    for (int i = threadIdx.x; i < need; i += NT) st_agent(out + i, sh.cid[i]);
  }
  for (int i = need + threadIdx.x; i < top_k; i += NT) st_agent(out + i, i == need ? bq : -1);
}

// ---------------------------------------------------------------- per-wave lists
// A scoring wave of 64 KPL consecutive blocks writes the blocks whose keys reach its
// own threshold L (its 16th largest key, found bit by bit with ballots): at most
// LIST entries (key | id << 32) in ascending id, with (count, L') where L' = L, or
// L + 1 when ties at L did not all fit (the list then holds every key > L).  The
// union of the lists of a row holds every score whose key is >= the largest L',
// so it holds the row's winners whenever the need-th largest key of the union is
// at least every L' -- which the merge checks.
constexpr int LIST = 16;
constexpr uint32_t LIST_WRITTEN = 0x100;   // set in every stored count word (a zeroed word: not yet stored)
constexpr int LIST_POLL_LIMIT = 1 << 16;   // bound on the rounds of a merge that polls its lists

// number of lanes whose key k[i] passes `pred`, over the KPL keys of each lane
template <int KPL, class P>
__device__ __forceinline__ int wave_count(const uint32_t (&k)[KPL], P pred) {
  int c = 0;
#pragma unroll
  for (int i = 0; i < KPL; ++i) c += __popcll(__ballot(pred(k[i])));
  return c;
}

// wave_count for three thresholds at once: every ballot is taken before the first
// population count, so the compares issue back to back instead of each waiting for
// the scalar count of the one before
template <int KPL>
__device__ __forceinline__ void wave_count3(const uint32_t (&k)[KPL], uint32_t t1, uint32_t t2, uint32_t t3, int& c1,
                                            int& c2, int& c3) {
  uint64_t m1[KPL], m2[KPL], m3[KPL];
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    m1[i] = __ballot(k[i] >= t1);
    m2[i] = __ballot(k[i] >= t2);
    m3[i] = __ballot(k[i] >= t3);
  }
  c1 = c2 = c3 = 0;
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    c1 += __popcll(m1[i]);
    c2 += __popcll(m2[i]);
    c3 += __popcll(m3[i]);
  }
}

// The wave's list from its KPL keys per lane (key 0 = none).  Ids ascend over the
// segments (half, i): lanes 0..31 hold the lower half, k[i] before k[i + 1].
// The entries go to `dst` [0, count) in that order, (count, L') to `meta`, with
// L' raised to lp_floor when that is larger (a list of lists: every key above the
// lower lists' L' is in them).  after_prior: the list's stores wait until every
// earlier memory operation of the wave is acknowledged (a reader that sees the list
// stored sees those too).  LDS_DST: dst and meta are in LDS (plain stores).
template <int KPL, bool LDS_DST = false>
__device__ __forceinline__ void wave_list(const uint32_t (&k)[KPL], const int (&id)[KPL], uint64_t* dst, uint2* meta,
                                          bool after_prior = false, uint32_t lp_floor = 0u) {
  static_assert(LIST == 16, "one lower bound per group of 4 lanes");
  const int lane = threadIdx.x & 63;
  const int valid = wave_count<KPL>(k, [](uint32_t x) { return x != 0u; });
  uint32_t T = 0;
  if (valid > LIST) {
    // the largest T with count(keys >= T) >= LIST.  T is at most the wave's largest
    // key and at least lb: the smallest key (every valid key counts, and there are
    // more than LIST), and the smallest of the 16 four-lane groups' largest keys
    // (each group holds one key >= it).  So T shares the bits of the two above
    // their highest differing bit; the bits below are found two at a time (three
    // trial counts per step, independent of each other).  Stop once the count is
    // exactly LIST (the set is then the wave's LIST best).
    uint32_t mx = 0u, mn = 0xFFFFFFFFu;
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
      mx = max(mx, k[i]);
      mn = min(mn, k[i] ? k[i] : 0xFFFFFFFFu);
    }
    mx = max(mx, (uint32_t)dpp_i<0xB1>(0, (int)mx));       // the group of 4 lanes
    mx = max(mx, (uint32_t)dpp_i<0x4E>(0, (int)mx));
    const uint32_t kmx = wave_umax(mx);
    const uint32_t lb = max(wave_umin(mn), wave_umin(mx));
    const uint32_t diff = kmx ^ lb;
    int b = diff ? 31 - __clz((int)diff) : -1;    // highest differing bit
    T = diff ? kmx & ~((2u << b) - 1u) : kmx;      // the shared prefix (b == 31: none)
    if (b == 31) T = 0;
#pragma unroll 1
    for (; b >= 1; b -= 2) {
      const uint32_t t1 = T | (1u << (b - 1)), t2 = T | (2u << (b - 1)), t3 = T | (3u << (b - 1));
      int c1, c2, c3;
      wave_count3<KPL>(k, t1, t2, t3, c1, c2, c3);
      const int c = c3 >= LIST ? c3 : (c2 >= LIST ? c2 : c1);
      T = c3 >= LIST ? t3 : (c2 >= LIST ? t2 : (c1 >= LIST ? t1 : T));
      if (c == LIST) { b = -1; break; }
    }
    if (b == 0) {
      const uint32_t t1 = T | 1u;
      if (wave_count<KPL>(k, [=](uint32_t x) { return x >= t1; }) >= LIST) T = t1;
    }
  }
  // keys >= T: all kept when they fit (T = 0: every valid key), else the keys > T
  // and the ties at T up to LIST in id order; segment by segment in list order
  constexpr int NS = 2 * KPL;
  auto mbcnt = [](uint64_t m) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
  };
  uint64_t mk[NS];
  bool kp[NS];
  uint32_t Lp = T;                               // L' = T, or T + 1 when some ties at T were left out
  int ge_c[KPL];
  {
    uint64_t mg[KPL];
#pragma unroll
    for (int i = 0; i < KPL; ++i) mg[i] = __ballot(k[i] && k[i] >= T);
#pragma unroll
    for (int i = 0; i < KPL; ++i) ge_c[i] = __popcll(mg[i]);
  }
  int ge = 0;
#pragma unroll
  for (int i = 0; i < KPL; ++i) ge += ge_c[i];
  if (ge <= LIST) {
    // the ballots of all segments are independent
#pragma unroll
    for (int sgm = 0; sgm < NS; ++sgm) {
      const uint32_t kk = k[sgm % KPL];
      kp[sgm] = (lane >> 5) == sgm / KPL && kk && kk >= T;
      mk[sgm] = __ballot(kp[sgm]);
    }
  } else {
    const int gt = wave_count<KPL>(k, [=](uint32_t x) { return x > T && x; });
    const int room = LIST - gt;
    // the tie ballots of all segments first (independent of each other), then the
    // running counts
    uint64_t mt[NS];
#pragma unroll
    for (int sgm = 0; sgm < NS; ++sgm) {
      const bool mine = (lane >> 5) == sgm / KPL;
      const uint32_t kk = k[sgm % KPL];
      mt[sgm] = __ballot(mine && kk && kk == T && T);
    }
    int ties = 0;
#pragma unroll
    for (int sgm = 0; sgm < NS; ++sgm) {
      const bool mine = (lane >> 5) == sgm / KPL;
      const uint32_t kk = k[sgm % KPL];
      const int trank = ties + mbcnt(mt[sgm]);
      kp[sgm] = mine && kk && (kk > T || (kk == T && (T == 0 || trank < room)));
      mk[sgm] = __ballot(kp[sgm]);
      ties += __popcll(mt[sgm]);
    }
    if (T && ties > room) Lp = T + 1;
  }
  if (after_prior) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  }
  Lp = max(Lp, lp_floor);
  int n = 0;
#pragma unroll
  for (int sgm = 0; sgm < NS; ++sgm) {
    const int pos = n + mbcnt(mk[sgm]);
    if (kp[sgm] && pos < LIST) {
      const uint64_t e = (uint64_t)k[sgm % KPL] | ((uint64_t)(uint32_t)id[sgm % KPL] << 32);
      if constexpr (LDS_DST)
        dst[pos] = e;
      else
        st_agent(dst + pos, e);
    }
    n += __popcll(mk[sgm]);
  }
  const uint64_t mw = (uint64_t)((uint32_t)min(n, LIST) | LIST_WRITTEN) | ((uint64_t)Lp << 32);
  if (lane == 0) {
    if constexpr (LDS_DST)
      *(uint64_t*)meta = mw;
    else
      st_agent((uint64_t*)meta, mw);
  }
}

// A merge's candidates in the registers of keep_best_regs' layout, from loaded list
// words: slot at = lo + 64 i + lane holds entry ev[i] of list at / LIST, whose count
// word is mv[i]; the wave's slots end at m (slots at >= m hold no entry).  ok (checked by the fused decode step,
// whose lists are being stored while it loads them, and were zero before its
// launch): every list below m is stored (its count word carries LIST_WRITTEN) and so
// is every counted entry (nonzero: an entry is one 8-byte store and no key is 0).
template <int E>
__device__ __forceinline__ void list_cands(const u32x2_t (&ev)[E], const u32x2_t (&mv)[E], int lo, int m,
                                           uint32_t (&key)[E], int32_t (&cid)[E], uint32_t& cnt, uint32_t& kmn,
                                           uint32_t& kmx, uint32_t& lmax, bool& ok) {
  const int lane = threadIdx.x & 63;
  ok = true;
  cnt = 0;
  kmn = 0xFFFFFFFFu;
  kmx = 0u;
  lmax = 0u;
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const int at = lo + 64 * i + lane;
    const bool in = at < m;
    const bool on = in && (at % LIST) < (int)(mv[i][0] & 0xFFu);
    key[i] = on ? ev[i][0] : 0u;
    cid[i] = (int32_t)ev[i][1];
    cnt += on;
    if (on) { kmn = min(kmn, key[i]); kmx = max(kmx, key[i]); }
    if (in) {
      lmax = max(lmax, mv[i][1]);
      ok = ok && (mv[i][0] & LIST_WRITTEN) && (!on || ev[i][0] != 0u);
    }
  }
}

// The merge once the candidates are in registers: one exchange (entries, the
// largest L', the keys' range), then the exact select of the need best.  False
// (nothing written) when a list's L' exceeds the need-th largest key of the union,
// or the union holds too few entries.  Enters after a barrier that frees `sh`
// (whose contents are arbitrary), and uses no slot of set 0 of sh.xi / sh.xj before
// its first barrier.
template <int NT, int E, class O>
__device__ __forceinline__ bool merge_cands(const uint32_t (&key)[E], const int32_t (&cid)[E], uint32_t cnt,
                                            uint32_t kmn, uint32_t kmx, uint32_t lmax, int need, int bq, int top_k,
                                            const O& out, Shared<NT>& sh) {
  constexpr int NW = Shared<NT>::NW;
  const int t = threadIdx.x, wv = t >> 6, lane = t & 63;
  for (int i = t; i < NBINS; i += NT) sh.hist[i] = 0;   // visible after the next barrier
  const int tot = wave_sum((int)cnt);
  lmax = wave_umax(lmax);
  const uint32_t mn = wave_umin(kmn), mx = wave_umax(kmx);
  if (lane == 0) {
    sh.xi[1][wv] = tot;
    sh.xj[1][wv] = (int)lmax;
    sh.wn[0][wv] = (int)mn;
    sh.wn[1][wv] = (int)mx;
  }
  __syncthreads();
  int total = 0;
  uint32_t limit = 0, kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    total += sh.xi[1][i];
    limit = max(limit, (uint32_t)sh.xj[1][i]);
    kmin = min(kmin, (uint32_t)sh.wn[0][i]);
    kmax = max(kmax, (uint32_t)sh.wn[1][i]);
  }
  if (total <= need) return false;
  if (!keep_best_regs<NT, E>(key, cid, need, out, sh, limit, kmin, kmax)) return false;
  out.template tail<NT>(need, bq, top_k);
  return true;
}

// The last workgroup of a row merges its n_lists wave lists (n_lists * LIST <=
// E NT <= C_CAP, n_lists <= NT): the entries go straight from memory into
// registers (device-coherent loads), then merge_cands.  Called after a barrier that
// frees `sh`.
template <int NT, int E, class O>
__device__ __noinline__ bool merge_lists_e(const uint64_t* lists, const uint2* meta, int n_lists, int need, int bq,
                                           int top_k, const O& out, Shared<NT>& sh) {
  constexpr int NW = Shared<NT>::NW;
  static_assert(E * NT <= C_CAP, "candidates fit the exchange buffers");
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int M = n_lists * LIST;
  const int per = (M + NW - 1) / NW;
  const int lo = wv * per, hi = min(M, lo + per);
  const __amdgpu_buffer_rsrc_t rl = dev_rsrc(lists), rm = dev_rsrc(meta);
  u32x2_t ev[E], mv[E];
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const int at = lo + 64 * i + lane;
    ev[i] = at < hi ? __builtin_amdgcn_raw_buffer_load_b64(rl, (uint32_t)at * 8u, 0, 16 /* sc1 */) : u32x2_t{};
    mv[i] = at < hi ? __builtin_amdgcn_raw_buffer_load_b64(rm, (uint32_t)(at / LIST) * 8u, 0, 16) : u32x2_t{};
  }
  uint32_t key[E];
  int32_t cid[E];
  uint32_t cnt, kmn, kmx, lmax;
  bool ok;
  list_cands<E>(ev, mv, lo, hi, key, cid, cnt, kmn, kmx, lmax, ok);
  return merge_cands<NT, E>(key, cid, cnt, kmn, kmx, lmax, need, bq, top_k, out, sh);
}

// merge_lists_e with as few entries per thread as the lists need (8 for up to 8 NT
// entries: the 4-wave step's 128 lists of a 128K-token row); the row's ids to
// out[0, top_k)
template <int NT>
__device__ __forceinline__ bool merge_lists(const uint64_t* lists, const uint2* meta, int n_lists, int need, int bq,
                                            int top_k, int32_t* out, Shared<NT>& sh) {
  constexpr int EMAX = C_CAP / NT, ESMALL = EMAX > 8 ? 8 : EMAX;
  if (EMAX > ESMALL && n_lists * LIST <= ESMALL * NT)
    return merge_lists_e<NT, ESMALL>(lists, meta, n_lists, need, bq, top_k, RowOut{out}, sh);
  return merge_lists_e<NT, EMAX>(lists, meta, n_lists, need, bq, top_k, RowOut{out}, sh);
}

// The fused decode step's merge of one row's lists, by a workgroup that consumes
// the ids itself, while other workgroups of the launch are still storing the lists
// (which were zero before the launch).  start() issues the loads of every slot of
// the m_lists lists the row may have (m_lists * LIST <= E NT) before the row's
// length is known; merge() takes the row's n_lists <= m_lists lists, loads again
// (bounded by LIST_POLL_LIMIT rounds, false when it runs out) until all of them
// are stored, and merges them (merge_cands).
template <int NT, int E>
struct StepLists {
  static constexpr int NW = NT / 64;
  __amdgpu_buffer_rsrc_t rl, rm;
  int lo, hi;
  u32x2_t ev[E], mv[E];
  __device__ __forceinline__ void load() {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const int at = lo + 64 * i + lane;
      ev[i] = at < hi ? __builtin_amdgcn_raw_buffer_load_b64(rl, (uint32_t)at * 8u, 0, 16 /* sc1 */) : u32x2_t{};
      mv[i] = at < hi ? __builtin_amdgcn_raw_buffer_load_b64(rm, (uint32_t)(at / LIST) * 8u, 0, 16) : u32x2_t{};
    }
  }
  __device__ __forceinline__ void start(const uint64_t* lists, const uint2* meta, int m_lists) {
    const int wv = threadIdx.x >> 6;
    const int m = m_lists * LIST;
    const int per = (m + NW - 1) / NW;
    rl = dev_rsrc(lists);
    rm = dev_rsrc(meta);
    lo = wv * per;
    hi = min(m, lo + per);
    load();
  }
  template <class O>
  __device__ __forceinline__ bool merge(int n_lists, int need, int bq, int top_k, const O& out, Shared<NT>& sh) {
    static_assert(E * NT <= C_CAP, "candidates fit the exchange buffers");
    const int wv = threadIdx.x >> 6;
    const int M = n_lists * LIST;
    uint32_t key[E];
    int32_t cid[E];
    uint32_t cnt, kmn, kmx, lmax;
#pragma unroll 1
    for (int round = 0;; ++round) {
      bool ok;
      list_cands<E>(ev, mv, lo, min(M, hi), key, cid, cnt, kmn, kmx, lmax, ok);
      // every slot of the workgroup stored?  (slots alternate between rounds;
      // merge_cands uses the other sets before its first barrier)
      int* slot = (round & 1) ? sh.xj[0] : sh.xi[0];
      const bool wave_ok = __ballot(!ok) == 0ull;   // every lane's (outside the lane-0 branch)
      if ((threadIdx.x & 63) == 0) slot[wv] = wave_ok;
      __syncthreads();
      bool all = true;
#pragma unroll
      for (int w = 0; w < NW; ++w) all = all && slot[w];
      if (all) break;
      if (round >= LIST_POLL_LIMIT) return false;
      __builtin_amdgcn_s_sleep(1);
      load();
    }
    return merge_cands<NT, E>(key, cid, cnt, kmn, kmx, lmax, need, bq, top_k, out, sh);
  }
};

}  // namespace sel
}  // namespace ip
