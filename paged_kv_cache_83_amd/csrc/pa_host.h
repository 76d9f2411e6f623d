// Host pieces shared by the translation units of libpa: pool geometry checks,
// tile sizes, launch status and per-launch timing.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/pa.h"

namespace pa_detail {

inline bool geom_ok(const pa_geom* g) {
  return g && g->num_layers > 0 && g->num_kv_heads > 0 && g->head_dim > 0 && g->block_size > 0 &&
         g->num_blocks > 0 && (g->dtype == PA_F32 || g->dtype == PA_BF16 || g->dtype == PA_FP8);
}
inline int64_t esize(const pa_geom* g) {
  return g->dtype == PA_F32 ? 4 : g->dtype == PA_BF16 ? 2 : 1;
}
// Bytes of one (layer, block, head) tile of K or V: B*d elements, and for FP8
// pools the B scale bytes that follow them.
inline int64_t tile_bytes(const pa_geom* g) {
  return (int64_t)g->block_size * g->head_dim * esize(g) + (g->dtype == PA_FP8 ? g->block_size : 0);
}

inline pa_status launch_status() { return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP; }

// Times one launch when timing is on (pa_prof_enable) and `allowed` (the
// allocation-free entry point creates no events). The start event is recorded
// on the stream when the scope opens. A scope made with `bind` holds exactly
// one kernel, launched with PA_TIMED_LAUNCH, which hands the stop event to the
// launch itself (hipExtLaunchKernelGGL): it takes the kernel's own end, so the
// span leaves out the latency of a second event command after the kernel.
// Other scopes record the stop event on the stream after their launches.
// (Handing the launch the start event as well costs about 15 us of host time
// per launch, which stalls short kernels.)
struct ProfScope {
  const char* name;
  hipStream_t st;
  hipEvent_t a = nullptr, b = nullptr;
  bool on;
  bool bind;
  bool bound = false;
  ProfScope(const char* n, hipStream_t s, bool allowed = true, bool bind_kernel = false);
  ~ProfScope();
  // True once, for the scope's one kernel, when its stop event goes to the launch.
  bool take_events() {
    if (!on || !bind || bound) return false;
    bound = true;
    return true;
  }
};

// Launch inside a ProfScope made with `bind`: with the scope's stop event when
// timing is on, a plain launch otherwise.
#define PA_TIMED_LAUNCH(PS, KERNEL, GRID, BLOCK, LDS, ST, ...)                                 \
  do {                                                                                        \
    if ((PS).take_events())                                                                   \
      hipExtLaunchKernelGGL(KERNEL, GRID, BLOCK, LDS, ST, nullptr, (PS).b, 0, __VA_ARGS__);   \
    else                                                                                      \
      hipLaunchKernelGGL(KERNEL, GRID, BLOCK, LDS, ST, __VA_ARGS__);                          \
  } while (0)

}  // namespace pa_detail
