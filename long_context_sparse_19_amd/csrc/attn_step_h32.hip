// The fused decode step with the 32-head attention units (launches of few (row,
// split) units; launch_decode_step picks it).  A unit of its own: beside the
// 64-head step kernel it changed that kernel's register allocation (the two share
// the selection's out-of-line slow paths), which cost 0.7 us per decode step.
#include "attn_bf16.hpp"

namespace ip {

namespace {

__global__ __launch_bounds__(NTA, 1) void decode_step_h32_kernel(StepKArgs A) {
  __shared__ AttnShared sh;
  __shared__ __align__(16) uint8_t pmat[LAT_H * PROW];
  __shared__ __align__(16) uint8_t kv0[KVBUF];
  __shared__ __align__(16) uint8_t kv1[KVBUF];
  __shared__ int last_here;
  const int L = blockIdx.x;
  if (L < A.n_score + A.n_app) {
    scorek::score_fp8_body<1, STEP_NWV, true, STEP_TILES>(A.s, L % A.gx, L / A.gx, A.gx, kv0, last_here,
                                                           A.at.sel_ready);
    return;
  }
  attn_bf16_h32_body<true>(A.at, L - A.n_score - A.n_app, sh, pmat, kv0, kv1);
}

}  // namespace

hipError_t launch_decode_step_h32(const StepKArgs& k, unsigned grid, hipStream_t s) {
  launch(K_STEP, decode_step_h32_kernel, dim3(grid), dim3(NTA), s, k);
  return hipGetLastError();
}

}  // namespace ip
