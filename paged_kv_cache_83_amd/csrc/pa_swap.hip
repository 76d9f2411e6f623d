// Asynchronous migration of KV blocks between the HBM pool and a pinned host
// frame pool, overlapped with compute.
//
// "KV Cache Management", section "Asynchronous paged swapping": frames for the
// outgoing blocks come from a pre-allocated page-locked host pool as one
// contiguous run; the copy is queued on a dedicated copy stream so that it
// overlaps compute; when it completes, a host callback retags the entries as
// host-resident and returns the vacated blocks to the free queue. The same
// section gives the return path (its paragraphs on speculative prefetch and on
// the pipelined chunked reload): fresh blocks are reserved, the copy back is
// queued in chunks, and the entries point at the new blocks once it has
// completed.
//
// A block is not contiguous in the pool (each layer's K and V live in their own
// region), so each chunk of blocks is packed into a device staging buffer by a
// gather kernel and moved by one DMA copy into the run of host frames; the way
// back is one DMA copy per run of consecutive frames, then a scatter kernel.
// Two staging buffers alternate between a kernel stream and a DMA stream, so
// the gather of chunk k+1 runs while chunk k crosses the host link. The gather
// and scatter use only a few work-groups: they have to keep ahead of the link
// (tens of GB/s), not run at HBM speed, and the rest of the GPU stays with the
// decode that the migration is meant to hide behind.

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
#include "pa_host.h"
#include "pa_move.h"

using namespace pa_detail;

// Work-groups of one gather / scatter launch. Too few and the launch waits for
// CU slots behind decode, stalling the link; 512 keeps the link at full rate
// while decode is running.
constexpr int32_t kDefaultMoveWgs = 512;

struct pa_swapper {
  pa_geom g{};
  pa_bm* bm = nullptr;
  void* k_pool = nullptr;
  void* v_pool = nullptr;
  int32_t num_frames = 0;
  int32_t chunk_blocks = 0;
  int32_t move_wgs = 0;
  bool direct = false;      // strided DMA straight from / to the pool, no staging
  int64_t frame_bytes = 0;  // one block: 2 * L runs
  int64_t run_bytes = 0;    // one (layer, K-or-V) run of a block
  char* host = nullptr;     // caller's pinned buffer, num_frames * frame_bytes
  char* host_dev = nullptr; // the same buffer as the device addresses it
  char* staging[2] = {nullptr, nullptr};  // halves of the caller's device staging buffer
  hipStream_t kstream = nullptr;          // gather / scatter kernels
  hipStream_t dstream = nullptr;          // DMA copies over the host link
  hipEvent_t full[2] = {nullptr, nullptr};   // staging[b] written by its producer
  hipEvent_t empty[2] = {nullptr, nullptr};  // staging[b] drained by its consumer
  hipEvent_t after = nullptr;   // marks the caller's stream before a migration
  hipEvent_t done[2] = {nullptr, nullptr};   // marks both streams for pa_swapper_fence
  int next_buf = 0;             // staging buffers alternate across chunks and migrations
  std::mutex issue_mu;          // one issuing thread at a time
  std::atomic<int32_t> pending{0};
  std::atomic<int32_t> error{PA_OK};
  std::atomic<int64_t> bytes_out{0};
  std::atomic<int64_t> bytes_in{0};
};

namespace {

// The completion step of one migration, run by the HIP runtime on its
// host-function thread once the migration's last copy or kernel has finished
// (every earlier chunk precedes it through stream order and the hand-over
// events). It makes no HIP calls.
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

// Gather (MODE 1) or scatter (MODE 2) of blocks ids[0..m) against staging
// frames 0..m-1 of `stg` on the kernel stream, in launches of at most kArgIds
// ids carried in the kernel arguments.
template <int MODE>
bool move_chunk(pa_swapper* s, char* stg, const int32_t* ids, int32_t m) {
  ProfScope ps(MODE == 1 ? "swap_gather" : "swap_scatter", s->kstream);
  for (int32_t a = 0; a < m; a += kArgIds) {
    const int32_t c = std::min(kArgIds, m - a);
    ArgIds arg;
    for (int32_t k = 0; k < kArgIds; ++k) arg.v[k] = k < c ? ids[a + k] : -1;
    const int64_t runs = (int64_t)c * s->g.num_layers * 2;
    const dim3 grid((unsigned)std::min<int64_t>(runs, s->move_wgs)), block(256);
    char* dst = stg + (int64_t)a * s->frame_bytes;
    if (s->run_bytes % 16 == 0)
      hipLaunchKernelGGL((block_move_kernel<MODE, u32x4, ArgIds, NoIds>), grid, block, 0,
                         s->kstream, (char*)s->k_pool, (char*)s->v_pool, dst, arg, NoIds{},
                         s->g.num_layers, s->g.num_blocks, s->run_bytes, runs);
    else if (s->run_bytes % 4 == 0)
      hipLaunchKernelGGL((block_move_kernel<MODE, uint32_t, ArgIds, NoIds>), grid, block, 0,
                         s->kstream, (char*)s->k_pool, (char*)s->v_pool, dst, arg, NoIds{},
                         s->g.num_layers, s->g.num_blocks, s->run_bytes, runs);
    else if (s->run_bytes % 2 == 0)
      hipLaunchKernelGGL((block_move_kernel<MODE, uint16_t, ArgIds, NoIds>), grid, block, 0,
                         s->kstream, (char*)s->k_pool, (char*)s->v_pool, dst, arg, NoIds{},
                         s->g.num_layers, s->g.num_blocks, s->run_bytes, runs);
    else
      hipLaunchKernelGGL((block_move_kernel<MODE, uint8_t, ArgIds, NoIds>), grid, block, 0,
                         s->kstream, (char*)s->k_pool, (char*)s->v_pool, dst, arg, NoIds{},
                         s->g.num_layers, s->g.num_blocks, s->run_bytes, runs);
    if (hipGetLastError() != hipSuccess) return false;
  }
  return true;
}

// Next staging buffer: `producer` waits until its previous consumer is done.
int take_buffer(pa_swapper* s, hipStream_t producer, bool* ok) {
  const int b = s->next_buf;
  s->next_buf ^= 1;
  *ok = *ok && hipStreamWaitEvent(producer, s->empty[b], 0) == hipSuccess;
  return b;
}

// One contiguous copy over the host link on the DMA stream. Both sides are
// given as device addresses (the pinned buffer's device view) with the copy kind
// that asks for the DMA engines rather than compute units, so that the copy
// takes no CU slots from the decode running beside it. The ROCm 7.2 runtime
// honours it; the HIP runtime bundled with PyTorch 2.10 (ROCm 7.0) still serves
// device-to-host copies with a blit kernel in a torch process (measured).
bool link_copy(pa_swapper* s, void* dst, const void* src, size_t bytes) {
  return hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDeviceNoCU, s->dstream) == hipSuccess;
}

// Hand buffer b from the producer stream to the consumer stream.
bool hand_over(pa_swapper* s, int b, hipStream_t producer, hipStream_t consumer) {
  return hipEventRecord(s->full[b], producer) == hipSuccess &&
         hipStreamWaitEvent(consumer, s->full[b], 0) == hipSuccess;
}

// The stream that touches the pool (kernel stream, or the DMA stream in direct
// mode) follows the caller's stream.
bool order_after(pa_swapper* s, void* after_stream) {
  if (!after_stream) return true;
  return hipEventRecord(s->after, (hipStream_t)after_stream) == hipSuccess &&
         hipStreamWaitEvent(s->direct ? s->dstream : s->kstream, s->after, 0) == hipSuccess;
}

// Direct mode: block `phys` <-> frame `frame` as two strided copies (K, V), each
// L rows of one run: pool pitch N * run, frame pitch 2 * run (the staging layout).
bool direct_copy(pa_swapper* s, int32_t phys, int32_t frame, bool to_host) {
  const size_t run = (size_t)s->run_bytes, pitch = (size_t)s->g.num_blocks * run;
  char* f = s->host + (int64_t)frame * s->frame_bytes;
  char* pools[2] = {(char*)s->k_pool, (char*)s->v_pool};
  for (int kv = 0; kv < 2; ++kv) {
    char* p = pools[kv] + (size_t)phys * run;
    char* h = f + kv * run;
    hipError_t e = to_host ? hipMemcpy2DAsync(h, 2 * run, p, pitch, run, s->g.num_layers,
                                              hipMemcpyDeviceToHost, s->dstream)
                           : hipMemcpy2DAsync(p, pitch, h, 2 * run, run, s->g.num_layers,
                                              hipMemcpyHostToDevice, s->dstream);
    if (e != hipSuccess) return false;
  }
  return true;
}

// Queue the completion step behind the migration's last operation, on `last`;
// on failure the migration stays in flight and the swapper reports PA_ERR_HIP
// from then on.
pa_status queue_finish(pa_swapper* s, hipStream_t last, Job* job, bool issued_ok) {
  if (issued_ok) {
    s->pending.fetch_add(1);
    if (hipLaunchHostFunc(last, finish_job, job) == hipSuccess) return PA_OK;
    s->pending.fetch_sub(1);
  }
  delete job;
  s->error.store(PA_ERR_HIP);
  return PA_ERR_HIP;
}

// Frees what the swapper itself created (streams, events, the object); the
// frame and staging buffers belong to the caller.
void release(pa_swapper* s) {
  if (s->kstream) (void)hipStreamSynchronize(s->kstream);
  if (s->dstream) (void)hipStreamSynchronize(s->dstream);
  for (int b = 0; b < 2; ++b) {
    if (s->full[b]) (void)hipEventDestroy(s->full[b]);
    if (s->empty[b]) (void)hipEventDestroy(s->empty[b]);
    if (s->done[b]) (void)hipEventDestroy(s->done[b]);
  }
  if (s->after) (void)hipEventDestroy(s->after);
  if (s->kstream) (void)hipStreamDestroy(s->kstream);
  if (s->dstream) (void)hipStreamDestroy(s->dstream);
  delete s;
}

struct SwapSizes {
  int64_t run, frame;
  int32_t chunk_blocks, move_wgs;
  bool direct;
  size_t host_bytes, staging_bytes;
};

pa_status swap_sizes(const pa_geom* g, int32_t num_frames, const pa_swap_opts* opts, SwapSizes* z) {
  int32_t chunk_blocks = opts ? opts->chunk_blocks : 0;
  const int32_t move_wgs = opts && opts->move_wgs ? opts->move_wgs : kDefaultMoveWgs;
  if (!geom_ok(g) || num_frames <= 0 || chunk_blocks < 0 || move_wgs < 0) return PA_ERR_INVALID_ARG;
  z->run = (int64_t)g->num_kv_heads * tile_bytes(g);
  z->frame = 2 * (int64_t)g->num_layers * z->run;
  if (chunk_blocks == 0)  // about 64 MiB per staging half, at least one block
    chunk_blocks = (int32_t)std::max<int64_t>(1, std::min<int64_t>(4096, (64ll << 20) / z->frame));
  z->chunk_blocks = chunk_blocks;
  z->move_wgs = move_wgs;
  z->direct = opts && opts->direct;
  z->host_bytes = (size_t)num_frames * (size_t)z->frame;
  z->staging_bytes = z->direct ? 0 : 2 * (size_t)chunk_blocks * (size_t)z->frame;
  return PA_OK;
}

}  // namespace

extern "C" {

pa_status pa_swapper_buffer_bytes(const pa_geom* g, int32_t num_frames, const pa_swap_opts* opts,
                                  size_t* host_bytes, size_t* staging_bytes) {
  SwapSizes z;
  const pa_status st = swap_sizes(g, num_frames, opts, &z);
  if (st != PA_OK) return st;
  if (host_bytes) *host_bytes = z.host_bytes;
  if (staging_bytes) *staging_bytes = z.staging_bytes;
  return PA_OK;
}

pa_status pa_swapper_create(const pa_geom* g, pa_bm* bm, void* k_pool, void* v_pool,
                            int32_t num_frames, const pa_swap_opts* opts, void* host_frames,
                            size_t host_bytes, void* staging, size_t staging_bytes,
                            pa_swapper** out) {
  if (!out) return PA_ERR_INVALID_ARG;
  *out = nullptr;
  SwapSizes z;
  pa_status st = swap_sizes(g, num_frames, opts, &z);
  if (st != PA_OK) return st;
  if (!bm || !k_pool || !v_pool || !host_frames || (!z.direct && !staging))
    return PA_ERR_INVALID_ARG;
  if (host_bytes < z.host_bytes || staging_bytes < z.staging_bytes) return PA_ERR_WORKSPACE;
  // The frames must be page-locked host memory that the device can address.
  char* host_dev = nullptr;
  if (hipHostGetDevicePointer((void**)&host_dev, host_frames, 0) != hipSuccess || !host_dev) {
    (void)hipGetLastError();
    return PA_ERR_INVALID_ARG;
  }
  pa_swapper* s = new (std::nothrow) pa_swapper();
  if (!s) return PA_ERR_INVALID_ARG;
  s->g = *g;
  s->bm = bm;
  s->k_pool = k_pool;
  s->v_pool = v_pool;
  s->num_frames = num_frames;
  s->chunk_blocks = z.chunk_blocks;
  s->move_wgs = z.move_wgs;
  s->direct = z.direct;
  s->frame_bytes = z.frame;
  s->run_bytes = z.run;
  s->host = (char*)host_frames;
  s->host_dev = host_dev;
  if (!z.direct) {
    s->staging[0] = (char*)staging;
    s->staging[1] = (char*)staging + (size_t)z.chunk_blocks * (size_t)z.frame;
  }
  bool ok = hipStreamCreateWithFlags(&s->kstream, hipStreamNonBlocking) == hipSuccess &&
            hipStreamCreateWithFlags(&s->dstream, hipStreamNonBlocking) == hipSuccess &&
            hipEventCreateWithFlags(&s->after, hipEventDisableTiming) == hipSuccess;
  for (int b = 0; ok && b < 2; ++b)
    ok = hipEventCreateWithFlags(&s->full[b], hipEventDisableTiming) == hipSuccess &&
         hipEventCreateWithFlags(&s->empty[b], hipEventDisableTiming) == hipSuccess &&
         hipEventCreateWithFlags(&s->done[b], hipEventDisableTiming) == hipSuccess &&
         hipEventRecord(s->empty[b], s->kstream) == hipSuccess;   // both start drained
  if (!ok) {
    release(s);
    return PA_ERR_HIP;
  }
  st = pa_bm_attach_host_pool(bm, num_frames);
  if (st != PA_OK) {
    release(s);
    return st;
  }
  *out = s;
  return PA_OK;
}

pa_status pa_swapper_sync(pa_swapper* s) {
  if (!s) return PA_ERR_INVALID_ARG;
  if (hipStreamSynchronize(s->kstream) != hipSuccess ||
      hipStreamSynchronize(s->dstream) != hipSuccess)
    return PA_ERR_HIP;
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
  const pa_status st = pa_swapper_sync(s);
  // A completion step still to run would touch the swapper: keep it.
  if (s->pending.load() > 0) return PA_ERR_HIP;
  // Frames still held by host-resident or in-flight entries keep the pool
  // attached and the swapper alive: their bytes are in the caller's buffer and
  // only this swapper can bring them back.
  if (pa_bm_host_frames_free(s->bm) >= 0) {   // (unless the caller detached it already)
    const pa_status dt = pa_bm_detach_host_pool(s->bm);
    if (dt != PA_OK) return dt;
  }
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
  if (!job) {
    s->error.store(PA_ERR_HIP);   // the reservation stands; nothing was queued
    return PA_ERR_HIP;
  }
  bool ok = order_after(s, after_stream);
  if (s->direct) {
    for (int32_t k = 0; ok && k < n; ++k) ok = direct_copy(s, phys[k], first + k, true);
    return queue_finish(s, s->dstream, job, ok);
  }
  for (int32_t c0 = 0; ok && c0 < n; c0 += s->chunk_blocks) {
    const int32_t m = std::min(s->chunk_blocks, n - c0);
    const int b = take_buffer(s, s->kstream, &ok);
    ok = ok && move_chunk<1>(s, s->staging[b], phys.data() + c0, m) &&
         hand_over(s, b, s->kstream, s->dstream) &&
         link_copy(s, s->host_dev + (int64_t)(first + c0) * s->frame_bytes, s->staging[b],
                   (size_t)m * s->frame_bytes) &&
         hipEventRecord(s->empty[b], s->dstream) == hipSuccess;
  }
  return queue_finish(s, s->dstream, job, ok);
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
  if (!job) {
    s->error.store(PA_ERR_HIP);   // the reservation stands; nothing was queued
    return PA_ERR_HIP;
  }
  bool ok = order_after(s, after_stream);
  if (s->direct) {
    for (int32_t k = 0; ok && k < n; ++k) ok = direct_copy(s, phys[k], frames[k], false);
    return queue_finish(s, s->dstream, job, ok);
  }
  for (int32_t c0 = 0; ok && c0 < n; c0 += s->chunk_blocks) {
    const int32_t m = std::min(s->chunk_blocks, n - c0);
    const int b = take_buffer(s, s->dstream, &ok);
    for (int32_t k = 0; ok && k < m;) {  // one copy per run of consecutive frames
      int32_t e = k + 1;
      while (e < m && frames[c0 + e] == frames[c0 + e - 1] + 1) ++e;
      ok = link_copy(s, s->staging[b] + (int64_t)k * s->frame_bytes,
                     s->host_dev + (int64_t)frames[c0 + k] * s->frame_bytes,
                     (size_t)(e - k) * s->frame_bytes);
      k = e;
    }
    ok = ok && hand_over(s, b, s->dstream, s->kstream) &&
         move_chunk<2>(s, s->staging[b], phys.data() + c0, m) &&
         hipEventRecord(s->empty[b], s->kstream) == hipSuccess;
  }
  return queue_finish(s, s->kstream, job, ok);
}

pa_status pa_swapper_fence(pa_swapper* s, void* stream) {
  if (!s) return PA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(s->issue_mu);
  hipStream_t own[2] = {s->kstream, s->dstream};
  for (int b = 0; b < 2; ++b)
    if (hipEventRecord(s->done[b], own[b]) != hipSuccess ||
        hipStreamWaitEvent((hipStream_t)stream, s->done[b], 0) != hipSuccess)
      return PA_ERR_HIP;
  return PA_OK;
}

int32_t pa_swapper_pending(const pa_swapper* s) { return s ? s->pending.load() : -1; }

pa_status pa_swapper_info(const pa_swapper* s, void** host_frames, void** kernel_stream,
                          void** dma_stream, int64_t* frame_bytes, int32_t* chunk_blocks,
                          int64_t* bytes_out, int64_t* bytes_in) {
  if (!s) return PA_ERR_INVALID_ARG;
  if (host_frames) *host_frames = s->host;
  if (kernel_stream) *kernel_stream = s->kstream;
  if (dma_stream) *dma_stream = s->dstream;
  if (frame_bytes) *frame_bytes = s->frame_bytes;
  if (chunk_blocks) *chunk_blocks = s->chunk_blocks;
  if (bytes_out) *bytes_out = s->bytes_out.load();
  if (bytes_in) *bytes_in = s->bytes_in.load();
  return PA_OK;
}

}  // extern "C"
