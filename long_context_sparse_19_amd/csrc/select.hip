// Learned sparse selection as a kernel of its own, one workgroup per query row
// (prefill chunks and float scores; decode-shaped launches select inside the
// scoring launch instead).  The selection itself is in select.hpp.  G2C Brief
// "GLM-5.3-Flash: hybrid attention becomes the product", section "DSA keeps
// selected global access in eleven layers" (top 2048 tokens = 512 pooled blocks).
#include "select.hpp"

namespace ip {

namespace {

constexpr int NT = 512;              // rows of up to 32768 scores are read whole

__global__ __launch_bounds__(NT) void select_kernel(SelectArgs a) {
  __shared__ sel::Shared<NT> sh;
  const int rl = blockIdx.x;
  const int r = a.row0 + rl;
  const int b = a.q_seq ? a.q_seq[r] : r;
  const int p = a.q_pos ? a.q_pos[r] : a.L.seq_lens[b] - 1;
  const int bq = p >> 2;
  sel::select_row<NT>(a.scores + (int64_t)rl * a.ld, a.gm + (int64_t)rl * a.gld, bq, bq, a.top_k,
                      a.out + (int64_t)r * a.top_k, sh);
}

}  // namespace

hipError_t launch_select(const SelectArgs& a, hipStream_t s) {
  if (a.n_rows <= 0) return hipSuccess;
  launch(K_TOPK, select_kernel, dim3(a.n_rows), dim3(NT), s, a);
  return hipGetLastError();
}

}  // namespace ip
