// Phase stamps of the fused decode step, for timelines of its latency chain.  Only a
// library built with IP_PHASE_STAMPS (`python -m long_context_sparse_19_amd.build
// --stamps`, a library of its own) records them: thread 0 of a workgroup writes
// s_memrealtime (a 100 MHz clock shared by every compute unit) into a slot of its
// row of a static device array, which ip_phase_stamps() copies to the host.  In the
// normal build every stamp compiles to nothing.
#pragma once
#include <hip/hip_runtime.h>

namespace ip {
constexpr int STAMP_SLOTS = 8;
constexpr int STAMP_STEP_ROWS = 4096;          // rows [0, 4096): the step's workgroups
constexpr int STAMP_ROWS = STAMP_STEP_ROWS + 1024;   // then the combine's
// the step's slots
enum : int { ST_START = 0, ST_SCORED = 1, ST_IDS = 2, ST_SUB0 = 3, ST_SUBS = 4, ST_END = 5 };
// the combine's
enum : int { ST_C_START = 0, ST_C_END = 1 };
}  // namespace ip

#ifdef IP_PHASE_STAMPS
// one copy per source that includes this header; attn.hip reads its own, which the
// 64-head step kernel and the combine write
static __device__ unsigned long long ip_phase_stamp_rows[ip::STAMP_ROWS * ip::STAMP_SLOTS];
#define IP_STAMP(row, slot)                                                                            \
  do {                                                                                                 \
    if (threadIdx.x == 0 && (row) < ip::STAMP_ROWS)                                                    \
      ip_phase_stamp_rows[(row) * ip::STAMP_SLOTS + (slot)] = __builtin_amdgcn_s_memrealtime();         \
  } while (0)
#else
#define IP_STAMP(row, slot) \
  do {                      \
  } while (0)
#endif
