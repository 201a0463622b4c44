// Helpers shared by the sparse attention kernels (attn.hip, attn_pipe.hip): the
// block table of a selection, LDS access wrappers, cross-lane reductions, waits.
#pragma once
#include "kernels.hpp"

namespace ip {
namespace {

constexpr int NSEG = LAT_DK * 2 / 128;         // 9 segments per latent row
constexpr float LN2 = 0.69314718055994531f;
constexpr float LOG2E = 1.44269504088896341f;
constexpr float RESCALE_LOG2 = 8.f;            // reference maximum moves when passed by more

constexpr int MAX_BLOCKS_PER_SPLIT = 512;      // host keeps splits within this
constexpr int VIS_SHIFT = 29;                  // block table: first row | visible tokens << 29
constexpr uint32_t ROW_BITS = (1u << VIS_SHIFT) - 1;

typedef short s16x4_t __attribute__((ext_vector_type(4)));

// LDS accesses that never touch the latent sub-tile buffers go through these.  The
// restrict-qualified pointer gives them alias-scope metadata, from which the
// compiler's wait insertion can tell that they do not alias the LDS DMA into those
// buffers; without it every LDS access would wait for all outstanding sub-tile loads.
template <class T>
__device__ __forceinline__ T lds_ld(const T* __restrict__ p) { return *p; }
template <class T>
__device__ __forceinline__ void lds_st(T* __restrict__ p, T v) { *p = v; }

struct RowCtx {
  int b, p;
  const int32_t* sel;
};

__device__ __forceinline__ RowCtx row_ctx(const AttnArgs& a, int r) {
  RowCtx c;
  c.b = a.q_seq ? a.q_seq[r] : r;
  c.p = a.q_pos ? a.q_pos[r] : a.L.seq_lens[c.b] - 1;
  c.sel = a.sel + (int64_t)r * a.top_k;
  return c;
}

// Lanes l and l ^ 32 combined (v_permlane32_swap with the same register as both
// operands gives every lane its own value and that of lane l ^ 32).
__device__ __forceinline__ float pair_max32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Combine over the four lanes l % 16 + 16q (q < 4).  v_permlane16_swap /
// v_permlane32_swap with the same register as both operands give every lane, in
// the two results, its own value and that of lane l ^ 16 (resp. l ^ 32).
__device__ __forceinline__ float quad_max16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float quad_sum16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint32_t block_entry(const AttnArgs& a, const RowCtx& c, int blk) {
  const bool vis = blk >= 0 && blk * 4 <= c.p;
  const int t0 = vis ? blk * 4 : (c.p >> 2) * 4;
  return (uint32_t)a.L.tok_row(c.b, t0) | (vis ? (uint32_t)min(4, c.p - t0 + 1) << VIS_SHIFT : 0u);
}

// block_entry of N blocks at once: one branch on the layout around all N, so that
// their page-table reads are in flight together (one wait instead of N)
template <int N>
__device__ __forceinline__ void block_entries(const AttnArgs& a, const RowCtx& c, const int (&blk)[N],
                                              uint32_t (&out)[N]) {
  uint32_t t0[N], vis[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const bool v = blk[i] >= 0 && blk[i] * 4 <= c.p;
    t0[i] = (uint32_t)(v ? blk[i] * 4 : (c.p >> 2) * 4);
    vis[i] = v ? (uint32_t)min(4, c.p - (int)t0[i] + 1) << VIS_SHIFT : 0u;
  }
  if (a.L.page_table) {
    const uint32_t pt = (uint32_t)a.L.page_tokens;
    const int32_t* pr = a.L.page_table + (int64_t)c.b * a.L.max_pages;
    int32_t pg[N];
#pragma unroll
    for (int i = 0; i < N; ++i) pg[i] = pr[t0[i] / pt];
#pragma unroll
    for (int i = 0; i < N; ++i) out[i] = ((uint32_t)pg[i] * pt + t0[i] % pt) | vis[i];
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) out[i] = (uint32_t)((int64_t)c.b * a.L.seq_stride + t0[i]) | vis[i];
  }
}

// 16-byte chunk swizzle of a latent row in LDS: within 8 consecutive rows x(t)
// takes all 8 values (conflict-free K fragment reads); within 4 rows it keeps the
// chunk pairs of the transposing V reads apart
__device__ __forceinline__ int kv_swz(int t) { return ((t & 3) << 1) | ((t >> 2) & 1); }

// Waits until at most N of this wave's global loads (LDS DMA included) are
// outstanding.  The vmcnt field of the s_waitcnt immediate is bits 0..3 (low) and
// 14..15 (high); expcnt (bits 4..6) and lgkmcnt (bits 8..11) stay at their maxima
// (no wait).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

}  // namespace
}  // namespace ip
