// Asynchronous migration of KV blocks between the HBM pool and a pinned host
// frame pool, overlapped with compute.
//
// "KV Cache Management", section "Asynchronous paged swapping": frames for the
// outgoing blocks come from a pre-allocated page-locked host pool as one
// contiguous run; the copy is queued on a dedicated copy stream so that it
// overlaps compute; when it completes, a host callback retags the entries as
// host-resident and returns the vacated blocks to the free queue. The same
// section (and "Speculative prefetch and pipelined chunked reload") gives the
// return path: fresh blocks are reserved, the copy back is queued in chunks,
// and the entries point at the new blocks once it has completed.
//
// A block is not contiguous in the pool (each layer's K and V live in their own
// region), so each chunk of blocks is first packed into a device staging buffer
// by a gather kernel (one work-group per 32 KiB run), then moved by one DMA
// copy into the run of host frames; the way back is one DMA copy per run of
// consecutive frames, then a scatter kernel. Everything of one swapper is
// ordered on its own stream, so one staging buffer serves every chunk.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cstdint>
#include <mutex>
#include <new>
#include <thread>
#include <vector>

#include "../../include/pa.h"
#include "pa_device.h"
#include "pa_move.h"

using namespace pa_detail;

struct pa_swapper {
  pa_geom g{};
  pa_bm* bm = nullptr;
  void* k_pool = nullptr;
  void* v_pool = nullptr;
  int32_t num_frames = 0;
  int32_t chunk_blocks = 0;
  int64_t frame_bytes = 0;  // one block: 2 * L runs
  int64_t run_bytes = 0;    // one (layer, K-or-V) run of a block
  char* host = nullptr;     // pinned, num_frames * frame_bytes
  char* staging = nullptr;  // device, chunk_blocks * frame_bytes
  hipStream_t stream = nullptr;
  hipEvent_t after = nullptr;  // marks the caller's stream before a migration
  hipEvent_t done = nullptr;   // marks the copy stream for pa_swapper_fence
  std::mutex issue_mu;         // one issuing thread at a time
  std::atomic<int32_t> pending{0};
  std::atomic<int32_t> error{PA_OK};
  std::atomic<int64_t> bytes_out{0};
  std::atomic<int64_t> bytes_in{0};
};

namespace {

// The completion step of one migration, run by the HIP runtime on its
// host-function thread once everything queued before it on the copy stream has
// finished. It makes no HIP calls.
struct Job {
  pa_swapper* s;
  int32_t seq;
  bool out;
  std::vector<int32_t> logical;
};

void finish_job(void* p) {
  Job* j = static_cast<Job*>(p);
  pa_swapper* s = j->s;
  const int32_t n = (int32_t)j->logical.size();
  pa_status st = j->out ? pa_bm_swap_out_finish(s->bm, j->seq, j->logical.data(), n)
                        : pa_bm_swap_in_finish(s->bm, j->seq, j->logical.data(), n);
  if (st != PA_OK) {
    int32_t ok = PA_OK;
    s->error.compare_exchange_strong(ok, (int32_t)st);
  }
  (j->out ? s->bytes_out : s->bytes_in).fetch_add((int64_t)n * s->frame_bytes);
  delete j;
  s->pending.fetch_sub(1);
}

// Gather (MODE 1) or scatter (MODE 2) of blocks ids[0..m) against staging frames
// 0..m-1, in launches of at most kArgIds ids carried in the kernel arguments.
template <int MODE>
bool move_chunk(pa_swapper* s, const int32_t* ids, int32_t m) {
  ProfScope ps(MODE == 1 ? "swap_gather" : "swap_scatter", s->stream);
  for (int32_t a = 0; a < m; a += kArgIds) {
    const int32_t c = std::min(kArgIds, m - a);
    ArgIds arg;
    for (int32_t k = 0; k < kArgIds; ++k) arg.v[k] = k < c ? ids[a + k] : -1;
    const dim3 grid((unsigned)((int64_t)c * s->g.num_layers * 2)), block(256);
    char* stg = s->staging + (int64_t)a * s->frame_bytes;
    if (s->run_bytes % 16 == 0)
      hipLaunchKernelGGL((block_move_kernel<MODE, u32x4, ArgIds, NoIds>), grid, block, 0,
                         s->stream, (char*)s->k_pool, (char*)s->v_pool, stg, arg, NoIds{},
                         s->g.num_layers, s->g.num_blocks, s->run_bytes);
    else if (s->run_bytes % 4 == 0)
      hipLaunchKernelGGL((block_move_kernel<MODE, uint32_t, ArgIds, NoIds>), grid, block, 0,
                         s->stream, (char*)s->k_pool, (char*)s->v_pool, stg, arg, NoIds{},
                         s->g.num_layers, s->g.num_blocks, s->run_bytes);
    else
      hipLaunchKernelGGL((block_move_kernel<MODE, uint16_t, ArgIds, NoIds>), grid, block, 0,
                         s->stream, (char*)s->k_pool, (char*)s->v_pool, stg, arg, NoIds{},
                         s->g.num_layers, s->g.num_blocks, s->run_bytes);
    if (hipGetLastError() != hipSuccess) return false;
  }
  return true;
}

bool order_after(pa_swapper* s, void* after_stream) {
  if (!after_stream) return true;
  return hipEventRecord(s->after, (hipStream_t)after_stream) == hipSuccess &&
         hipStreamWaitEvent(s->stream, s->after, 0) == hipSuccess;
}

// Queue the completion step; on failure the migration stays in flight and the
// swapper reports PA_ERR_HIP from then on.
pa_status queue_finish(pa_swapper* s, Job* job, bool issued_ok) {
  if (issued_ok) {
    s->pending.fetch_add(1);
    if (hipLaunchHostFunc(s->stream, finish_job, job) == hipSuccess) return PA_OK;
    s->pending.fetch_sub(1);
  }
  delete job;
  s->error.store(PA_ERR_HIP);
  return PA_ERR_HIP;
}

void release(pa_swapper* s) {
  if (s->stream) (void)hipStreamSynchronize(s->stream);
  if (s->host) (void)hipHostFree(s->host);
  if (s->staging) (void)hipFree(s->staging);
  if (s->after) (void)hipEventDestroy(s->after);
  if (s->done) (void)hipEventDestroy(s->done);
  if (s->stream) (void)hipStreamDestroy(s->stream);
  delete s;
}

}  // namespace

extern "C" {

pa_status pa_swapper_create(const pa_geom* g, pa_bm* bm, void* k_pool, void* v_pool,
                            int32_t num_frames, int32_t chunk_blocks, pa_swapper** out) {
  if (!out) return PA_ERR_INVALID_ARG;
  *out = nullptr;
  if (!geom_ok(g) || !bm || !k_pool || !v_pool || num_frames <= 0 || chunk_blocks < 0)
    return PA_ERR_INVALID_ARG;
  const int64_t run = (int64_t)g->num_kv_heads * g->block_size * g->head_dim * esize(g);
  const int64_t frame = 2 * (int64_t)g->num_layers * run;
  if (chunk_blocks == 0)  // about 256 MiB of staging, at least one block
    chunk_blocks = (int32_t)std::max<int64_t>(1, std::min<int64_t>(4096, (256ll << 20) / frame));
  pa_swapper* s = new (std::nothrow) pa_swapper();
  if (!s) return PA_ERR_INVALID_ARG;
  s->g = *g;
  s->bm = bm;
  s->k_pool = k_pool;
  s->v_pool = v_pool;
  s->num_frames = num_frames;
  s->chunk_blocks = chunk_blocks;
  s->frame_bytes = frame;
  s->run_bytes = run;
  bool ok = hipStreamCreateWithFlags(&s->stream, hipStreamNonBlocking) == hipSuccess &&
            hipEventCreateWithFlags(&s->after, hipEventDisableTiming) == hipSuccess &&
            hipEventCreateWithFlags(&s->done, hipEventDisableTiming) == hipSuccess &&
            hipMalloc((void**)&s->staging, (size_t)chunk_blocks * frame) == hipSuccess &&
            hipHostMalloc((void**)&s->host, (size_t)num_frames * frame, hipHostMallocDefault) ==
                hipSuccess;
  if (!ok) {
    release(s);
    return PA_ERR_HIP;
  }
  pa_status st = pa_bm_attach_host_pool(bm, num_frames);
  if (st != PA_OK) {
    release(s);
    return st;
  }
  *out = s;
  return PA_OK;
}

pa_status pa_swapper_sync(pa_swapper* s) {
  if (!s) return PA_ERR_INVALID_ARG;
  if (hipStreamSynchronize(s->stream) != hipSuccess) return PA_ERR_HIP;
  // The stream has drained; its host functions may still be finishing.
  const auto t0 = std::chrono::steady_clock::now();
  while (s->pending.load() > 0) {
    if (std::chrono::steady_clock::now() - t0 > std::chrono::seconds(30)) return PA_ERR_HIP;
    std::this_thread::sleep_for(std::chrono::microseconds(20));
  }
  return (pa_status)s->error.load();
}

pa_status pa_swapper_destroy(pa_swapper* s) {
  if (!s) return PA_ERR_INVALID_ARG;
  pa_status st = pa_swapper_sync(s);
  release(s);
  return st;
}

pa_status pa_swap_out_async(pa_swapper* s, int32_t seq, const int32_t* logical, int32_t n,
                            void* after_stream) {
  if (!s || n <= 0 || !logical) return PA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(s->issue_mu);
  if (s->error.load() != PA_OK) return (pa_status)s->error.load();
  std::vector<int32_t> phys(n);
  int32_t first = -1;
  pa_status st = pa_bm_swap_out_begin(s->bm, seq, logical, n, phys.data(), &first);
  if (st != PA_OK) return st;
  Job* job = new (std::nothrow) Job{s, seq, true, std::vector<int32_t>(logical, logical + n)};
  bool ok = job && order_after(s, after_stream);
  for (int32_t c0 = 0; ok && c0 < n; c0 += s->chunk_blocks) {
    const int32_t m = std::min(s->chunk_blocks, n - c0);
    ok = move_chunk<1>(s, phys.data() + c0, m) &&
         hipMemcpyAsync(s->host + (int64_t)(first + c0) * s->frame_bytes, s->staging,
                        (size_t)m * s->frame_bytes, hipMemcpyDeviceToHost, s->stream) == hipSuccess;
  }
  if (!job) {
    s->error.store(PA_ERR_HIP);
    return PA_ERR_HIP;
  }
  return queue_finish(s, job, ok);
}

pa_status pa_swap_in_async(pa_swapper* s, int32_t seq, const int32_t* logical, int32_t n,
                           void* after_stream) {
  if (!s || n <= 0 || !logical) return PA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(s->issue_mu);
  if (s->error.load() != PA_OK) return (pa_status)s->error.load();
  std::vector<int32_t> phys(n), frames(n);
  pa_status st = pa_bm_swap_in_begin(s->bm, seq, logical, n, phys.data(), frames.data());
  if (st != PA_OK) return st;
  Job* job = new (std::nothrow) Job{s, seq, false, std::vector<int32_t>(logical, logical + n)};
  bool ok = job && order_after(s, after_stream);
  for (int32_t c0 = 0; ok && c0 < n; c0 += s->chunk_blocks) {
    const int32_t m = std::min(s->chunk_blocks, n - c0);
    for (int32_t k = 0; ok && k < m;) {  // one copy per run of consecutive frames
      int32_t e = k + 1;
      while (e < m && frames[c0 + e] == frames[c0 + e - 1] + 1) ++e;
      ok = hipMemcpyAsync(s->staging + (int64_t)k * s->frame_bytes,
                          s->host + (int64_t)frames[c0 + k] * s->frame_bytes,
                          (size_t)(e - k) * s->frame_bytes, hipMemcpyHostToDevice,
                          s->stream) == hipSuccess;
      k = e;
    }
    ok = ok && move_chunk<2>(s, phys.data() + c0, m);
  }
  if (!job) {
    s->error.store(PA_ERR_HIP);
    return PA_ERR_HIP;
  }
  return queue_finish(s, job, ok);
}

pa_status pa_swapper_fence(pa_swapper* s, void* stream) {
  if (!s) return PA_ERR_INVALID_ARG;
  return hipEventRecord(s->done, s->stream) == hipSuccess &&
                 hipStreamWaitEvent((hipStream_t)stream, s->done, 0) == hipSuccess
             ? PA_OK
             : PA_ERR_HIP;
}

int32_t pa_swapper_pending(const pa_swapper* s) { return s ? s->pending.load() : -1; }

pa_status pa_swapper_info(const pa_swapper* s, void** host_frames, void** stream,
                          int64_t* frame_bytes, int32_t* chunk_blocks, int64_t* bytes_out,
                          int64_t* bytes_in) {
  if (!s) return PA_ERR_INVALID_ARG;
  if (host_frames) *host_frames = s->host;
  if (stream) *stream = s->stream;
  if (frame_bytes) *frame_bytes = s->frame_bytes;
  if (chunk_blocks) *chunk_blocks = s->chunk_blocks;
  if (bytes_out) *bytes_out = s->bytes_out.load();
  if (bytes_in) *bytes_in = s->bytes_in.load();
  return PA_OK;
}

}  // extern "C"
