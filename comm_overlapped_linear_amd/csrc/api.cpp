// C ABI of libtpgemm: validation, the stage scheduler and the graph cache.
//
// The scheduler follows "Distributed GEMM" (Hassani et al., SHI Labs,
// Dec 2024): the peers' shards are moved by asynchronous copies while the
// matrix cores run the local stage, and the stage kernels need no
// communication code of their own (Introduction; Approach, observations 2 and
// 4; Background, Figure 4: local shard first, then rotate). On one MI355X the
// peers' shards are buffers in the same HBM: a run's deliveries are one
// launch of the library's copy kernel (the all-gather and weight-gradient
// default), the runtime's shader copy, or the SDMA copy engines (the
// reduce-scatter default), and one event after a run's deliveries gates
// exactly the stage run that reads them. Stage launches fan out over up to four streams
// forked from and joined back into the caller's stream. Calls are issued
// eagerly; with TPG_FORCE_GRAPH one call is recorded once into a hipGraph and
// replayed on request (launch gaps between stages are overhead, Approach
// observation 4; on MI355X eager issue measured faster, see tpgemm.h).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <deque>
#include <limits>
#include <chrono>
#include <thread>
#include <cstdio>
#include <cstring>
#include <functional>
#include <mutex>
#include <sstream>
#include <string>
#include <unordered_map>
#include <vector>

#include "gemm.h"
#include "tpgemm.h"

namespace {

thread_local std::string g_err;

tpg_status fail(tpg_status st, const std::string& msg) {
  g_err = msg;
  return st;
}

#define HIP_TRY(expr)                                                                     \
  do {                                                                                    \
    hipError_t e_ = (expr);                                                               \
    if (e_ != hipSuccess)                                                                 \
      return fail(TPG_ERR_HIP, std::string(#expr) + " failed: " + hipGetErrorString(e_)); \
  } while (0)

constexpr int kStreams = 4;       // compute streams per call (index 0 = root)
constexpr int kMaxP = 64;
constexpr size_t kMaxGraphs = 512;
constexpr uint32_t kKnownFlags = TPG_UNSTAGED | TPG_NO_COPY | TPG_NO_GRAPH | TPG_COPY_SDMA |
                                 TPG_SERIAL_STAGES | TPG_PROFILE | TPG_FORCE_GRAPH |
                                 TPG_DEBUG_HOLD_DELIVERIES | TPG_COPY_SHADER | TPG_COPY_KERNEL |
                                 TPG_DEBUG_NO_GATE | TPG_IN_KERNEL_GATES | TPG_DEBUG_GATE_TIMEOUT;
constexpr uint32_t kCopyFlags = TPG_COPY_SDMA | TPG_COPY_SHADER | TPG_COPY_KERNEL;
// Internal (never accepted from a caller): a latency-bound staged all-gather
// the library runs as one launch carrying its deliveries (enqueue_ag_gated).
constexpr uint32_t kAutoCarried = 1u << 31;
// In-kernel gate counters after the all-gather's receive slots: one 32-bit
// counter per (delivered slice, K-chunk)
constexpr int kMaxGateChunks = 8;
constexpr size_t kGateCounterBytes = size_t(tpg::kMaxGateSlices) * kMaxGateChunks * 4;
// Staged calls below this many flops run on one stream: their GEMMs take
// well under the few microseconds each cross-stream event costs (the P = 2
// bf16 workload: 20 us on one stream, 40-45 us on two).
constexpr double kLatencyBoundFlop = 1e9;
// The staged all-gather runs as one launch carrying its deliveries (its
// tiles and copy workgroups all on the chip at once) up to this many flops.
// Measured on MI355X against the default multi-stream schedule, bf16, µs:
// 1024^3 in 2 slices 17.0 vs 33-35, 4096 x 512 x 1024 in 8: 28.5 vs 38-39,
// 1024 x 2048 x 4096 in 4: 53.5 vs 72, 1024 x 1024 x 8192 in 8: 95.5 vs 116;
// but 2048 x 1024 x 8192 in 2 (34 GFLOP): 99 vs 65, whose remote tiles read
// their one 16 MiB delivered slice device-coherently, past L2, eight times.
constexpr double kCarriedMaxFlop = 2e10;

struct ProfRec {
  hipEvent_t a, b;
  double flop;
};

// A recorded call: the executable graph and an event recorded after its
// latest replay (a retired graph is destroyed once that event has completed).
struct GraphEntry {
  hipGraphExec_t exec = nullptr;
  hipEvent_t done = nullptr;
};

// Numbers handed out for one static word array of a device: number n is
// word n mod size, stamped with n / size + 1.
//
// The dependency words: every word a call stamps is written on one of the
// library's internal streams, or awaited there (the fork, a run's wait for
// its deliveries), so once each internal stream has passed a point, every
// dependency of the calls issued before it has been both written and read.
// The numbers are therefore handed out in blocks: when a call ends with at
// least kSyncBlock numbers taken since the last block closed, the block is
// closed with an event on each internal stream; before number n is handed
// out, the block holding n - size must have completed (its events fired), so
// calls in flight never share a word, whatever streams they run on. That
// wait blocks the host only when the device lags so far behind that calls
// in flight hold all but a block of the array. No call stamps more than a
// block's worth.
//
// The gate words (one per latency-bound call carrying its deliveries, on the
// caller's stream only) are counters that only grow: each copy workgroup of
// a call adds 1, and the host, which enqueued every add, knows the total a
// call's tiles wait for. They are simply many: two calls share a word only
// 2^20 such calls apart, so that two calls sharing one are never in flight
// at once (their adds would mix).
struct WordRing {
  struct Block {
    uint64_t first;                 // the block's first number
    hipEvent_t done[kStreams];      // fired once all of its calls' dependencies have been written and read
  };
  uint64_t next = 0;
  uint64_t open = 0;                // first number of the block not yet closed
  std::deque<Block> closed;
};

// The gate words (calls that took a gate counter) and the
// dependency words (cross-stream dependencies issued as stream memory
// operations) of one device, with completed events kept for reuse.
struct WordSeq {
  WordRing gate, sync;
  std::vector<hipEvent_t> spare;
  bool events_made = false;
  std::vector<uint64_t> gate_total;   // each gate word's count: all the adds enqueued to it so far
};

constexpr uint64_t kSyncBlock = tpg::kSyncWords / 8;
// Closed blocks held at once: at most the array's blocks, plus the one that
// a wrapping number is about to free. Their events are created with the
// device's first context, so later calls create none.
constexpr int kSyncBlockEvents = int(tpg::kSyncWords / kSyncBlock + 1) * (kStreams - 1);

struct Ctx {
  int device = -1;
  hipStream_t comp[kStreams] = {};   // comp[0] unused: the root stream takes its place
  hipStream_t capture = nullptr;
  hipEvent_t ev_fork = nullptr;
  hipEvent_t ev_copy[kMaxP] = {};
  hipEvent_t ev_join[kStreams] = {};
  std::unordered_map<std::string, GraphEntry> graphs;
  std::vector<GraphEntry> retired;
  std::vector<ProfRec> prof;
  std::vector<hipEvent_t> prof_pool;
  WordSeq* seq = nullptr;            // this device's gate and dependency word numbers
  uint64_t sync_first = 0;           // the dependency word number next when the current call began
  bool capturing = false;            // the call being enqueued is being recorded into a graph (ours or the caller's)
};

std::mutex g_mu;
std::unordered_map<int, Ctx*> g_ctx;
// Never cleared: tpg_release_caches drops the contexts but the static words
// keep their last values for the life of the process, so a number (and the
// value it stamps) must never be handed out twice.
std::unordered_map<int, WordSeq> g_seq;

void destroy_ctx(Ctx* c);

tpg_status make_ctx_into(Ctx* c) {
  for (int i = 1; i < kStreams; ++i) HIP_TRY(hipStreamCreateWithFlags(&c->comp[i], hipStreamNonBlocking));
  HIP_TRY(hipStreamCreateWithFlags(&c->capture, hipStreamNonBlocking));
  HIP_TRY(hipEventCreateWithFlags(&c->ev_fork, hipEventDisableTiming));
  for (int i = 0; i < kMaxP; ++i) HIP_TRY(hipEventCreateWithFlags(&c->ev_copy[i], hipEventDisableTiming));
  for (int i = 0; i < kStreams; ++i) HIP_TRY(hipEventCreateWithFlags(&c->ev_join[i], hipEventDisableTiming));
  return TPG_OK;
}

// A context whose creation fails part way is released again (nothing leaks).
tpg_status make_ctx(int dev, Ctx** out) {
  Ctx* c = new Ctx();
  c->device = dev;
  c->seq = &g_seq[dev];            // element references survive rehashing
  tpg_status st = TPG_OK;
  if (!c->seq->events_made) {
    while (c->seq->spare.size() < size_t(kSyncBlockEvents) && st == TPG_OK) {
      hipEvent_t e = nullptr;
      const hipError_t err = hipEventCreateWithFlags(&e, hipEventDisableTiming);
      if (err != hipSuccess)
        st = fail(TPG_ERR_HIP, std::string("hipEventCreateWithFlags failed: ") + hipGetErrorString(err));
      else
        c->seq->spare.push_back(e);
    }
    if (st == TPG_OK) c->seq->events_made = true;
  }
  if (c->seq->gate_total.empty()) c->seq->gate_total.assign(tpg::kGateWords, 0);
  if (st == TPG_OK) st = make_ctx_into(c);
  if (st != TPG_OK) {
    destroy_ctx(c);
    return st;
  }
  *out = c;
  return TPG_OK;
}

tpg_status get_ctx(Ctx** out) {
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  auto it = g_ctx.find(dev);
  if (it != g_ctx.end()) {
    *out = it->second;
    return TPG_OK;
  }
  Ctx* c = nullptr;
  tpg_status st = make_ctx(dev, &c);
  if (st != TPG_OK) return st;
  g_ctx[dev] = c;
  *out = c;
  return TPG_OK;
}

void destroy_graph(const GraphEntry& g) {
  if (g.exec) (void)hipGraphExecDestroy(g.exec);
  if (g.done) (void)hipEventDestroy(g.done);
}

void destroy_ctx(Ctx* c) {
  for (auto& kv : c->graphs) destroy_graph(kv.second);
  for (auto& g : c->retired) destroy_graph(g);
  for (auto& r : c->prof) {
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  for (auto e : c->prof_pool) (void)hipEventDestroy(e);
  for (int i = 1; i < kStreams; ++i)
    if (c->comp[i]) (void)hipStreamDestroy(c->comp[i]);
  if (c->capture) (void)hipStreamDestroy(c->capture);
  if (c->ev_fork) (void)hipEventDestroy(c->ev_fork);
  for (int i = 0; i < kMaxP; ++i)
    if (c->ev_copy[i]) (void)hipEventDestroy(c->ev_copy[i]);
  for (int i = 0; i < kStreams; ++i)
    if (c->ev_join[i]) (void)hipEventDestroy(c->ev_join[i]);
  delete c;
}

// ---------------------------------------------------------------- helpers
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
  const void* p;
  size_t bytes;
};

bool overlaps(const Range& x, const Range& y) {
  if (!x.p || !y.p || x.bytes == 0 || y.bytes == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(x.p), a1 = a0 + x.bytes;
  const uintptr_t b0 = reinterpret_cast<uintptr_t>(y.p), b1 = b0 + y.bytes;
  return a0 < b1 && b0 < a1;
}

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int elem_bytes(int32_t dt) { return dt == TPG_E4M3 ? 1 : 2; }

bool fits_int(int64_t v) { return v >= 0 && v < (int64_t(1) << 31); }

// gemm_on layout of the weight gradient: A and B both contraction-major.
constexpr int kLayoutAT = 2;

struct Launch {
  hipStream_t root;
  bool profile;
};

// TPG_PROFILE: events around one launch on its own stream. `work` is the
// launch's algorithmic flop count (GEMMs) or the negative of its algorithmic
// HBM bytes (row kernels), as tpg_profile_read reports it.
tpg_status prof_begin(Ctx& cx, const Launch& L, hipStream_t s, double work, ProfRec& rec) {
  rec = ProfRec{nullptr, nullptr, work};
  if (!L.profile) return TPG_OK;
  for (hipEvent_t* e : {&rec.a, &rec.b}) {
    if (!cx.prof_pool.empty()) {
      *e = cx.prof_pool.back();
      cx.prof_pool.pop_back();
    } else {
      HIP_TRY(hipEventCreate(e));
    }
  }
  HIP_TRY(hipEventRecord(rec.a, s));
  return TPG_OK;
}

tpg_status prof_end(Ctx& cx, const Launch& L, hipStream_t s, const ProfRec& rec) {
  if (!L.profile) return TPG_OK;
  HIP_TRY(hipEventRecord(rec.b, s));
  cx.prof.push_back(rec);
  return TPG_OK;
}

tpg_status gemm_on(Ctx& cx, const Launch& L, hipStream_t s, const tpg::GemmParams& p, int dtype,
                   int layout, int epi) {
  ProfRec rec;
  if (tpg_status st = prof_begin(cx, L, s, 2.0 * p.M * double(p.N) * p.K * p.batch, rec); st != TPG_OK) return st;
  hipError_t e = layout == kLayoutAT      ? tpg::launch_gemm_at(p, s)
                 : p.cp_blocks > 0         ? tpg::launch_gemm_carrying_copy(p, dtype, layout, epi, s)
                                           : tpg::launch_gemm(p, dtype, layout, epi, s);
  if (e != hipSuccess) return fail(TPG_ERR_HIP, std::string("gemm launch failed: ") + hipGetErrorString(e));
  return prof_end(cx, L, s, rec);
}

// Next gate word number (a counter of the static array).
uint64_t take_gate_number(WordSeq& ws) { return ws.gate.next++; }

// Next dependency word number, for a call that took its first at call_first
// (or takes this one first).
tpg_status take_sync_number(WordSeq& ws, uint64_t call_first, uint64_t* out) {
  WordRing& r = ws.sync;
  const uint64_t n = r.next;
  if (n - call_first >= kSyncBlock)
    return fail(TPG_ERR_UNSUPPORTED, "a call with more cross-stream dependencies than the library tracks at once");
  if (n >= tpg::kSyncWords) {
    while (!r.closed.empty() && r.closed.front().first <= n - tpg::kSyncWords) {
      for (int i = 1; i < kStreams; ++i) {
        HIP_TRY(hipEventSynchronize(r.closed.front().done[i]));
        ws.spare.push_back(r.closed.front().done[i]);
      }
      r.closed.pop_front();
    }
  }
  *out = r.next++;
  return TPG_OK;
}

// After an eager call: close the dependency words' open block once it holds
// kSyncBlock numbers. A call that failed part way may have marked
// dependencies its streams never awaited: the host waits for the streams
// instead, after which every number handed out so far is free.
tpg_status close_sync_block(Ctx& cx, hipStream_t stream, bool failed) {
  WordSeq& ws = *cx.seq;
  WordRing& r = ws.sync;
  if (failed) {
    if (r.next == cx.sync_first) return TPG_OK;          // this call stamped nothing
    for (int i = 1; i < kStreams; ++i) (void)hipStreamSynchronize(cx.comp[i]);
    (void)hipStreamSynchronize(stream);
    for (auto& b : r.closed)
      for (int i = 1; i < kStreams; ++i) ws.spare.push_back(b.done[i]);
    r.closed.clear();
    r.open = r.next;
    return TPG_OK;
  }
  if (r.next - r.open < kSyncBlock) return TPG_OK;
  WordRing::Block b{r.open, {}};
  for (int i = 1; i < kStreams; ++i) {
    if (!ws.spare.empty()) {
      b.done[i] = ws.spare.back();
      ws.spare.pop_back();
    } else {
      HIP_TRY(hipEventCreateWithFlags(&b.done[i], hipEventDisableTiming));
    }
    HIP_TRY(hipEventRecord(b.done[i], cx.comp[i]));
  }
  r.closed.push_back(b);
  r.open = r.next;
  return TPG_OK;
}

// A cross-stream dependency: marked on the producing stream after its work
// so far, awaited on the consuming one. An eager call marks it with a
// stream memory operation: a 64-bit word of a static device array, taken
// round-robin and stamped with a value that grows on every reuse of the word,
// which the consumer waits to reach (measured on MI355X: a fork and join of
// two tiny kernels took 16 us per round with these, 30 us with events). A
// call being recorded into a graph uses the event instead, and so does a
// mark whose producing stream runs critical-path work right after it: the
// write holds that work back by about 2 us (measured on the staged e4m3
// all-gather, M x N x K = 8192 x 1024 x 8192 over 8 slices, whose deliveries
// follow the fork on the root: with every dependency written 94.1 us, with
// the fork an event and the rest written 91.3, with events only 93.2).
struct Dep {
  hipEvent_t ev = nullptr;
  unsigned long long* word = nullptr;
  uint64_t value = 0;
};

tpg_status dep_mark(Ctx& cx, hipEvent_t ev, hipStream_t from, Dep* d, bool as_event = false) {
  if (as_event || cx.capturing) {
    HIP_TRY(hipEventRecord(ev, from));
    *d = Dep{ev, nullptr, 0};
    return TPG_OK;
  }
  unsigned long long* words = nullptr;
  HIP_TRY(tpg::sync_words(&words));
  uint64_t seq = 0;
  if (tpg_status st = take_sync_number(*cx.seq, cx.sync_first, &seq); st != TPG_OK) return st;
  *d = Dep{nullptr, words + seq % tpg::kSyncWords, seq / tpg::kSyncWords + 1};
  HIP_TRY(hipStreamWriteValue64(from, d->word, d->value, 0));
  return TPG_OK;
}

tpg_status dep_await(hipStream_t to, const Dep& d) {
  if (d.word) {
    HIP_TRY(hipStreamWaitValue64(to, d.word, d.value, hipStreamWaitValueGte, ~0ull));
  } else {
    HIP_TRY(hipStreamWaitEvent(to, d.ev, 0));
  }
  return TPG_OK;
}

// `to` waits for the work issued on `from` so far.
tpg_status dep_now(Ctx& cx, hipEvent_t ev, hipStream_t from, hipStream_t to) {
  Dep d;
  if (tpg_status st = dep_mark(cx, ev, from, &d); st != TPG_OK) return st;
  return dep_await(to, d);
}

// Fork n-1 internal compute streams from the root; comp[0] is the root.
// root_critical: the root's next work is on the critical path (an event mark).
tpg_status fork_streams(Ctx& cx, hipStream_t root, int n, hipStream_t* streams, bool root_critical = false) {
  streams[0] = root;
  Dep d;
  if (n > 1) {
    if (tpg_status st = dep_mark(cx, cx.ev_fork, root, &d, root_critical); st != TPG_OK) return st;
  }
  for (int i = 1; i < n; ++i) {
    streams[i] = cx.comp[i];
    if (tpg_status st = dep_await(streams[i], d); st != TPG_OK) return st;
  }
  return TPG_OK;
}

tpg_status join_streams(Ctx& cx, hipStream_t root, int n, const hipStream_t* streams) {
  for (int i = 1; i < n; ++i)
    if (tpg_status st = dep_now(cx, cx.ev_join[i], streams[i], root); st != TPG_OK) return st;
  return TPG_OK;
}

// TPG_DEBUG_HOLD_DELIVERIES: the deliveries queue behind a host callback
// that sleeps, so every gated stage run is issued long before its slices
// exist (an ordering test forced from the host; the results must not change).
constexpr int kHoldMs = 20;
void hold_cb(void*) { std::this_thread::sleep_for(std::chrono::milliseconds(kHoldMs)); }

tpg_status hold_deliveries(uint32_t flags, hipStream_t s) {
  if (flags & TPG_DEBUG_HOLD_DELIVERIES) HIP_TRY(hipLaunchHostFunc(s, hold_cb, nullptr));
  return TPG_OK;
}

// Delivery copy: the entry point's default unless a flag overrides it
// (the defaults and their measurements are stated in tpgemm.h).
enum class Copy { Kernel, Shader, Sdma };

Copy copy_of(uint32_t flags, Copy dflt) {
  if (flags & TPG_COPY_SDMA) return Copy::Sdma;
  if (flags & TPG_COPY_SHADER) return Copy::Shader;
  if (flags & TPG_COPY_KERNEL) return Copy::Kernel;
  return dflt;
}

bool copy_flags_ok(uint32_t flags) {
  const uint32_t c = flags & kCopyFlags;
  return (c & (c - 1)) == 0;                       // at most one copy kind
}

// n slices of `bytes` from src[0..n) to dst + i * dst_stride on stream s:
// one launch of the library's delivery kernel, or runtime copies (slices
// back to back in memory and in the slots move as one copy). Arguments the
// kernel does not take (unaligned sizes) go to the runtime's shader copy.
tpg_status deliver_slices(Copy k, const void* const* src, int n, size_t bytes, char* dst, size_t dst_stride,
                          hipStream_t s) {
  if (n <= 0 || bytes == 0) return TPG_OK;
  if (k == Copy::Kernel && tpg::deliver_ok(src, n, bytes, dst, dst_stride)) {
    HIP_TRY(tpg::launch_deliver(src, n, bytes, dst, dst_stride, s));
    return TPG_OK;
  }
  const hipMemcpyKind mk = k == Copy::Sdma ? hipMemcpyDeviceToDeviceNoCU : hipMemcpyDeviceToDevice;
  for (int i = 0; i < n;) {
    int run = 1;
    while (dst_stride == bytes && i + run < n &&
           static_cast<const char*>(src[i + run]) == static_cast<const char*>(src[i]) + run * bytes)
      ++run;
    HIP_TRY(hipMemcpyAsync(dst + i * dst_stride, src[i], run * bytes, mk, s));
    i += run;
  }
  return TPG_OK;
}

// Records `enqueue` into a graph once per key and replays it on `user`, or
// runs it eagerly.
// Issue policy (stated and measured in tpgemm.h): eager unless
// TPG_FORCE_GRAPH asks for a recorded graph.
bool stream_capturing(hipStream_t stream);

tpg_status run_call(Ctx& cx, uint32_t flags, const std::string& key, hipStream_t user,
                    const std::function<tpg_status(const Launch&)>& enqueue) {
  const bool eager = !(flags & TPG_FORCE_GRAPH) ||
                     (flags & (TPG_NO_GRAPH | TPG_PROFILE | TPG_DEBUG_HOLD_DELIVERIES | TPG_DEBUG_NO_GATE)) != 0;
  if (eager) {
    // a caller recording its stream into a graph records this call too: its
    // dependencies must then be events, which join the internal streams to
    // the capture and replay correctly
    cx.capturing = stream_capturing(user);
    cx.sync_first = cx.seq->sync.next;
    const tpg_status st = enqueue(Launch{user, (flags & TPG_PROFILE) != 0});
    const bool recorded = cx.capturing;
    cx.capturing = false;
    if (recorded) {
      if (st == TPG_OK && cx.seq->sync.next != cx.sync_first)
        return fail(TPG_ERR_UNSUPPORTED, "internal: a static word was stamped in a recorded call");
      return st;
    }
    const tpg_status cs = close_sync_block(cx, user, st != TPG_OK);
    return st != TPG_OK ? st : cs;
  }
  auto it = cx.graphs.find(key);
  if (it == cx.graphs.end()) {
    // retired graphs whose last replay has completed are destroyed; the
    // others wait for a later call (no call blocks the host on the GPU)
    for (size_t i = 0; i < cx.retired.size();) {
      if (hipEventQuery(cx.retired[i].done) == hipSuccess) {
        destroy_graph(cx.retired[i]);
        cx.retired[i] = cx.retired.back();
        cx.retired.pop_back();
      } else {
        ++i;
      }
    }
    if (cx.graphs.size() >= kMaxGraphs) {
      for (auto& kv : cx.graphs) cx.retired.push_back(kv.second);
      cx.graphs.clear();
    }
    HIP_TRY(hipStreamBeginCapture(cx.capture, hipStreamCaptureModeThreadLocal));
    cx.capturing = true;                      // dependencies as events (recordable)
    const uint64_t g0 = cx.seq->gate.next, s0 = cx.seq->sync.next;
    tpg_status st = enqueue(Launch{cx.capture, false});
    cx.capturing = false;
    if (st == TPG_OK && (cx.seq->gate.next != g0 || cx.seq->sync.next != s0))   // a replay would repeat them
      st = fail(TPG_ERR_UNSUPPORTED, "internal: a static word was stamped in a recorded call");
    hipGraph_t g = nullptr;
    hipError_t e = hipStreamEndCapture(cx.capture, &g);
    if (st != TPG_OK) {
      if (g) (void)hipGraphDestroy(g);
      return st;
    }
    if (e != hipSuccess) return fail(TPG_ERR_HIP, std::string("graph capture failed: ") + hipGetErrorString(e));
    GraphEntry ge;
    e = hipGraphInstantiate(&ge.exec, g, nullptr, nullptr, 0);
    (void)hipGraphDestroy(g);
    if (e != hipSuccess) return fail(TPG_ERR_HIP, std::string("graph instantiate failed: ") + hipGetErrorString(e));
    e = hipEventCreateWithFlags(&ge.done, hipEventDisableTiming);
    if (e != hipSuccess) {
      destroy_graph(ge);
      return fail(TPG_ERR_HIP, std::string("hipEventCreateWithFlags failed: ") + hipGetErrorString(e));
    }
    it = cx.graphs.emplace(key, ge).first;
  }
  HIP_TRY(hipGraphLaunch(it->second.exec, user));
  HIP_TRY(hipEventRecord(it->second.done, user));
  return TPG_OK;
}

template <typename T>
void put(std::ostringstream& os, const T& v) {
  os << v << '|';
}

// TPG_DEBUG_NO_GATE applies to staged calls of the entry points that
// implement it (`supported`).
tpg_status validate_no_gate(uint32_t flags, bool supported) {
  if (!(flags & TPG_DEBUG_NO_GATE)) return TPG_OK;
  if (!supported) return fail(TPG_ERR_UNSUPPORTED, "TPG_DEBUG_NO_GATE: not implemented by this call");
  if (flags & (TPG_UNSTAGED | TPG_SERIAL_STAGES))
    return fail(TPG_ERR_INVALID, "TPG_DEBUG_NO_GATE needs a staged call on several streams");
  return TPG_OK;
}

// TPG_IN_KERNEL_GATES applies to the staged rotating-A all-gather only.
tpg_status validate_in_kernel_gates(uint32_t flags, bool supported) {
  if ((flags & TPG_DEBUG_GATE_TIMEOUT) && !(flags & TPG_IN_KERNEL_GATES))
    return fail(TPG_ERR_INVALID, "TPG_DEBUG_GATE_TIMEOUT needs TPG_IN_KERNEL_GATES");
  if (!(flags & TPG_IN_KERNEL_GATES)) return TPG_OK;
  if (!supported) return fail(TPG_ERR_UNSUPPORTED, "TPG_IN_KERNEL_GATES: not implemented by this call");
  if (flags & (TPG_UNSTAGED | TPG_SERIAL_STAGES))
    return fail(TPG_ERR_UNSUPPORTED, "TPG_IN_KERNEL_GATES needs a staged call on several streams");
  if (flags & (TPG_COPY_SDMA | TPG_COPY_SHADER))
    return fail(TPG_ERR_UNSUPPORTED, "TPG_IN_KERNEL_GATES delivers with the library's copy kernel");
  return TPG_OK;
}

// In-kernel gates depend on the copy running while the GEMM waits (and the
// carried form on a count known when it is issued): a call being captured into a graph
// cannot take them.
// Whether `stream` is being captured (a failed query counts as captured, and
// its error is cleared so that no later launch check reports it).
bool stream_capturing(hipStream_t stream) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cs) != hipSuccess) {
    (void)hipGetLastError();
    return true;
  }
  return cs != hipStreamCaptureStatusNone;
}

tpg_status gates_not_captured(uint32_t flags, hipStream_t stream) {
  if ((flags & TPG_IN_KERNEL_GATES) && stream_capturing(stream))
    return fail(TPG_ERR_UNSUPPORTED, "TPG_IN_KERNEL_GATES: the call cannot be captured into a graph");
  return TPG_OK;
}

// ---------------------------------------------------------------- all-gather
// Default stage runs of the all-gather: one gate for all P-1 remote stages.
// On one GPU the deliveries (the copy kernel: ~23-26 us for 7 x 8 MiB) are
// short next to the remote GEMM work, the local stage covers them, and one
// full-chip launch over the delivered slices makes the fewest partial tile
// waves. More runs were measured slower for every workload here: the e4m3
// workload took 90 / 103 / 122 / 162 us with 1 / 2 / 3 / 7 runs (earlier
// runs start sooner but slow the remaining deliveries, and each run's launch
// is smaller).
int auto_groups(int remote) { return remote > 0 ? 1 : 0; }

tpg_status validate_ag(const tpg_ag_args* a, size_t need) {
  if (!a) return fail(TPG_ERR_INVALID, "args is NULL");
  if (a->P < 1 || a->P > kMaxP) return fail(TPG_ERR_INVALID, "P must be in [1, 64]");
  if (a->rank < 0 || a->rank >= a->P) return fail(TPG_ERR_INVALID, "rank must be in [0, P)");
  if (a->M < 0 || a->N < 0 || a->K < 0) return fail(TPG_ERR_INVALID, "negative dimension");
  if (a->schedule != TPG_ROTATE_A && a->schedule != TPG_ROTATE_B) return fail(TPG_ERR_INVALID, "bad schedule");
  const bool rotb = a->schedule == TPG_ROTATE_B;
  if (!rotb && a->M % a->P) return fail(TPG_ERR_INVALID, "M must be a multiple of P");
  if (rotb && a->N % a->P) return fail(TPG_ERR_INVALID, "TPG_ROTATE_B: N must be a multiple of P");
  if (rotb && (a->N / a->P) % 8) return fail(TPG_ERR_UNSUPPORTED, "TPG_ROTATE_B: N/P must be a multiple of 8");
  if (rotb && a->epilogue != TPG_EPI_ALPHA_BETA)
    return fail(TPG_ERR_UNSUPPORTED, "TPG_ROTATE_B needs the alpha/beta epilogue");
  if (a->flags & ~kKnownFlags) return fail(TPG_ERR_INVALID, "unknown flag bits");
  if (!copy_flags_ok(a->flags))
    return fail(TPG_ERR_INVALID, "TPG_COPY_SDMA, TPG_COPY_SHADER and TPG_COPY_KERNEL are exclusive");
  if (tpg_status ng = validate_no_gate(a->flags, !rotb); ng != TPG_OK) return ng;
  if (tpg_status ig = validate_in_kernel_gates(a->flags, !rotb); ig != TPG_OK) return ig;
  if (a->ab_dtype != TPG_BF16 && a->ab_dtype != TPG_E4M3) return fail(TPG_ERR_INVALID, "bad ab_dtype");
  if (a->b_layout != TPG_B_NK && a->b_layout != TPG_B_KN) return fail(TPG_ERR_INVALID, "bad b_layout");
  if (a->epilogue != TPG_EPI_ALPHA_BETA && a->epilogue != TPG_EPI_SWIGLU)
    return fail(TPG_ERR_INVALID, "bad epilogue");
  const bool sw = a->epilogue == TPG_EPI_SWIGLU;
  if (sw && (a->N % 2)) return fail(TPG_ERR_INVALID, "SWIGLU needs an even N");
  if (!fits_int(a->M) || !fits_int(a->N) || !fits_int(a->K))
    return fail(TPG_ERR_UNSUPPORTED, "dimensions must be below 2^31");
  if (a->ab_dtype == TPG_E4M3 && a->b_layout == TPG_B_KN)
    return fail(TPG_ERR_UNSUPPORTED, "e4m3 operands need the NK layout of B");
  if (a->K % (a->ab_dtype == TPG_E4M3 ? 16 : 8))
    return fail(TPG_ERR_UNSUPPORTED, "K must be a multiple of 8 (bf16) or 16 (e4m3)");
  const int64_t nout = sw ? a->N / 2 : a->N;
  if (a->b_layout == TPG_B_KN && (nout % 8 || a->N % 8))
    return fail(TPG_ERR_UNSUPPORTED, "KN layout needs N (and N/2 with SWIGLU) multiple of 8");
  if (a->beta != 0.0f && !a->c) return fail(TPG_ERR_INVALID, "beta != 0 needs C");
  const int eb = elem_bytes(a->ab_dtype);
  std::vector<Range> inputs;
  if (!rotb) {
    const int64_t m = a->M / a->P;
    const size_t slice_b = size_t(m) * a->K * eb;
    if (!a->a_slices && a->M > 0) return fail(TPG_ERR_INVALID, "a_slices is NULL");
    for (int s = 0; a->M > 0 && s < a->P; ++s) {
      if (!a->a_slices[s] && slice_b) return fail(TPG_ERR_INVALID, "NULL A slice");
      if (!aligned16(a->a_slices[s])) return fail(TPG_ERR_UNSUPPORTED, "A slice not 16-byte aligned");
      inputs.push_back({a->a_slices[s], slice_b});
    }
    const size_t b_b = size_t(a->N) * a->K * eb;
    if (!a->b && b_b) return fail(TPG_ERR_INVALID, "B is NULL");
    if (!aligned16(a->b)) return fail(TPG_ERR_UNSUPPORTED, "B not 16-byte aligned");
    inputs.push_back({a->b, b_b});
  } else {
    const size_t a_b = size_t(a->M) * a->K * eb;
    const size_t bslice_b = size_t(a->N / a->P) * a->K * eb;
    if (!a->a_slices || (!a->a_slices[0] && a_b)) return fail(TPG_ERR_INVALID, "A (a_slices[0]) is NULL");
    if (!aligned16(a->a_slices[0])) return fail(TPG_ERR_UNSUPPORTED, "A not 16-byte aligned");
    inputs.push_back({a->a_slices[0], a_b});
    if (!a->b_slices && a->N > 0) return fail(TPG_ERR_INVALID, "b_slices is NULL");
    for (int s = 0; a->N > 0 && s < a->P; ++s) {
      if (!a->b_slices[s] && bslice_b) return fail(TPG_ERR_INVALID, "NULL B slice");
      if (!aligned16(a->b_slices[s])) return fail(TPG_ERR_UNSUPPORTED, "B slice not 16-byte aligned");
      inputs.push_back({a->b_slices[s], bslice_b});
    }
  }
  const size_t d_b = size_t(a->M) * nout * 2;
  if (a->beta != 0.0f) {
    if (!aligned16(a->c)) return fail(TPG_ERR_UNSUPPORTED, "C not 16-byte aligned");
    inputs.push_back({a->c, d_b});
  }
  if (!a->d && d_b) return fail(TPG_ERR_INVALID, "D is NULL");
  if (!aligned16(a->d)) return fail(TPG_ERR_UNSUPPORTED, "D not 16-byte aligned");
  if (need && (!a->workspace || a->workspace_bytes < need))
    return fail(TPG_ERR_WORKSPACE, "workspace smaller than tpgemm_stage_ag_workspace_size()");
  const Range dr{a->d, d_b}, wr{a->workspace, need};
  for (const auto& r : inputs) {
    if (overlaps(dr, r)) return fail(TPG_ERR_INVALID, "D overlaps an input");
    if (overlaps(wr, r)) return fail(TPG_ERR_INVALID, "workspace overlaps an input");
  }
  if (overlaps(dr, wr)) return fail(TPG_ERR_INVALID, "workspace overlaps D");
  if (need && !aligned16(a->workspace)) return fail(TPG_ERR_UNSUPPORTED, "workspace not 16-byte aligned");
  if ((a->flags & TPG_UNSTAGED) && (a->flags & TPG_NO_COPY) && a->M > 0 && a->N > 0) {
    if (rotb && a->b_layout == TPG_B_KN)
      return fail(TPG_ERR_UNSUPPORTED, "UNSTAGED|NO_COPY with TPG_ROTATE_B needs the NK layout");
    const void* const* sl = rotb ? a->b_slices : a->a_slices;
    const size_t slice_b = rotb ? size_t(a->N / a->P) * a->K * eb : size_t(a->M / a->P) * a->K * eb;
    for (int s = 1; s < a->P; ++s)
      if (static_cast<const char*>(sl[s]) != static_cast<const char*>(sl[0]) + s * slice_b)
        return fail(TPG_ERR_UNSUPPORTED, "UNSTAGED|NO_COPY needs the slices to be contiguous");
  }
  if (a->flags & TPG_IN_KERNEL_GATES) {
    if (a->P > tpg::kMaxGateSlices) return fail(TPG_ERR_UNSUPPORTED, "TPG_IN_KERNEL_GATES needs P <= 8");
    if ((a->M / a->P) % 128) return fail(TPG_ERR_UNSUPPORTED, "TPG_IN_KERNEL_GATES needs M/P a multiple of 128");
    if ((a->K * eb) % 128) return fail(TPG_ERR_UNSUPPORTED, "TPG_IN_KERNEL_GATES needs K * element bytes a multiple of 128");
    if ((a->flags & TPG_NO_COPY) && a->M > 0) {
      const size_t slice_b = size_t(a->M / a->P) * a->K * eb;
      for (int s = 1; s < a->P; ++s)
        if (static_cast<const char*>(a->a_slices[s]) != static_cast<const char*>(a->a_slices[0]) + s * slice_b)
          return fail(TPG_ERR_UNSUPPORTED, "TPG_IN_KERNEL_GATES|NO_COPY needs the slices to be contiguous");
    }
  }
  return TPG_OK;
}

// Bytes of one delivered slice: an A row slice, or with TPG_ROTATE_B a B slice.
size_t ag_slice_bytes(const tpg_ag_args* a) {
  const size_t rows = a->schedule == TPG_ROTATE_B ? size_t(a->N) / a->P : size_t(a->M) / a->P;
  return rows * a->K * elem_bytes(a->ab_dtype);
}

size_t ag_ws(const tpg_ag_args* a) {
  if (!a || a->P < 1 || a->M < 0 || a->N < 0 || a->K < 0 || (a->flags & TPG_NO_COPY)) return 0;
  const size_t slice = ag_slice_bytes(a);
  if (a->flags & TPG_UNSTAGED) return slice * a->P;
  if (a->flags & TPG_IN_KERNEL_GATES) return round_up(slice * (a->P - 1), 256) + kGateCounterBytes;
  return slice * (a->P - 1);
}

tpg::GemmParams base_params() {
  tpg::GemmParams p;
  std::memset(&p, 0, sizeof(p));
  p.add_row0 = 0;
  p.add_row1 = 0;
  p.add_col0 = 0;
  p.add_col1 = std::numeric_limits<int>::max();   // addends (when any) span every column
  p.batch = 1;
  return p;
}

// All-gather with rotating B (TPG_ROTATE_B): the column dual of enqueue_ag.
// A is local; stage t multiplies slice s = (rank + t) mod P of B and writes
// columns [s*n, (s+1)*n) of D. Receive slots: (N, K) layout, slot j holds the
// (n, K) rows of one slice, back to back; (K, N) layout, one (K, W*n)
// matrix whose column block j holds one slice (W = P-1 staged, P unstaged),
// filled with 2-D copies. Stream roles, runs, gates and CU budgets are those
// of the rotating-A form.
tpg_status enqueue_ag_rotb(Ctx& cx, const tpg_ag_args& a, const Launch& L) {
  const int P = a.P, r = a.rank;
  const int eb = elem_bytes(a.ab_dtype);
  const bool kn = a.b_layout == TPG_B_KN;
  const int64_t n = a.N / P;
  const size_t slice_b = size_t(n) * a.K * eb;
  const bool copies = !(a.flags & TPG_NO_COPY) && slice_b > 0 && (P > 1 || (a.flags & TPG_UNSTAGED));
  const Copy ck = copy_of(a.flags, Copy::Kernel);
  const hipMemcpyKind kind2d = ck == Copy::Sdma ? hipMemcpyDeviceToDeviceNoCU : hipMemcpyDeviceToDevice;
  char* ws = static_cast<char*>(a.workspace);
  uint16_t* D = static_cast<uint16_t*>(a.d);
  const uint16_t* C = static_cast<const uint16_t*>(a.c);

  tpg::GemmParams p = base_params();
  p.a = a.a_slices[0];
  p.lda = a.K;
  p.ldc = a.N;
  p.ldd = a.N;
  p.M = static_cast<int>(a.M);
  p.K = static_cast<int>(a.K);
  p.alpha = a.alpha;
  p.beta = a.beta;
  p.vec_ok = (a.N % 8) == 0;
  const int dtype = a.ab_dtype == TPG_E4M3 ? tpg::kE4m3 : tpg::kBf16;
  const int layout = kn ? tpg::kKN : tpg::kNK;

  // slices src[0..cnt) into receive slots j .. j+cnt of a W-slot receive area:
  // (N, K) slots back to back; (K, N) column blocks by 2-D runtime copies
  auto deliver = [&](int j, const void* const* src, int cnt, int W) -> tpg_status {
    if (!kn) return deliver_slices(ck, src, cnt, slice_b, ws + j * slice_b, slice_b, L.root);
    for (int i = 0; i < cnt; ++i)
      HIP_TRY(hipMemcpy2DAsync(ws + size_t(j + i) * n * eb, size_t(W) * n * eb, src[i], size_t(n) * eb,
                               size_t(n) * eb, a.K, kind2d, L.root));
    return TPG_OK;
  };
  // columns [s*n, (s+run)*n) of D from B at Bp (row stride ldb elements)
  auto launch_cols = [&](hipStream_t cs, const void* Bp, int64_t ldb, int s, int run, int cus, int wrap_col = 0) {
    tpg::GemmParams q = p;
    q.b = Bp;
    q.ldb = ldb;
    q.N = static_cast<int>(run * n);
    q.d = D + s * n;
    q.c = C ? C + s * n : nullptr;
    q.cu_budget = cus;
    // the persistent grid too (e4m3 8192 x 1024 x 8192 in 8 slices of 128
    // columns, ranks 1 and 4: 96-97 / 94-95 us against 100 / 97-98 uncapped;
    // ranks 0 and 7 alike within noise)
    q.grid_cap = cus;
    if (wrap_col > 0) {    // slices past P-1: D's and C's columns P * n earlier
      q.wrap_col = wrap_col;
      q.wrap_back_col = static_cast<int>(P * n);
    }
    return gemm_on(cx, L, cs, q, dtype, layout, tpg::kEpiAlphaBeta);
  };

  if (a.flags & TPG_UNSTAGED) {
    // single stage: gather every slice (rank order) into B, then one GEMM
    const void* Bp = a.b_slices[0];
    int64_t ldb = a.K;                  // NO_COPY: contiguous (N, K) slices (validated)
    if (copies) {
      tpg_status hs = hold_deliveries(a.flags, L.root);
      if (hs != TPG_OK) return hs;
      hs = deliver(0, a.b_slices, P, P);
      if (hs != TPG_OK) return hs;
      Bp = ws;
      ldb = kn ? a.N : a.K;
    }
    return launch_cols(L.root, Bp, ldb, 0, P, 0);
  }

  const int remote = P - 1;
  const int G = remote == 0 ? 0 : (a.groups > 0 ? std::min(a.groups, remote) : auto_groups(remote));
  auto t0 = [&](int g) { return 1 + (g * remote) / G; };
  auto adjacent = [&](int s, int run) {   // NK slices s .. s+run back to back in memory
    if (kn) return run == 1;
    for (int i = 1; i < run; ++i)
      if (static_cast<const char*>(a.b_slices[s + i]) != static_cast<const char*>(a.b_slices[s]) + i * slice_b)
        return false;
    return true;
  };
  // A run whose slices pass slice P-1 writes two stretches of D's columns:
  // with delivered slices of a multiple of 256 columns (no tile straddles the
  // wrap; the slots hold the run's slices in arrival order) one launch whose
  // tiles past the wrap write P * n columns earlier; else one launch per
  // stretch, one after the other (side by side on two streams they took
  // longer: e4m3 8192 x 1024 x 8192 in 8 slices of 128 columns, rank 1, 106
  // against 99 us; rank 0 86).
  tpg::GemmParams probe = p;
  probe.N = static_cast<int>(remote * n);     // the widest run
  probe.ldb = kn ? int64_t(remote) * n : a.K;
  const bool wrap_one = copies && n % 256 == 0 && tpg::wrap_in_one_launch(probe, dtype, layout);
  auto passes_last = [&](int g) { return (r + t0(g)) % P + (t0(g + 1) - t0(g)) > P; };
  const int ns = (a.flags & TPG_SERIAL_STAGES) ? 1 : std::min(G + 1, kStreams);
  hipStream_t st[kStreams];
  tpg_status stat = fork_streams(cx, L.root, ns, st, copies);   // the deliveries follow on the root
  if (stat != TPG_OK) return stat;
  const int stack = (G + 1 + ns - 1) / ns;
  auto budget = [&](int stages) {
    if (ns == 1) return 0;
    return static_cast<int>(std::min<int64_t>(tpg::device_cus(),
                                              std::max<int64_t>(8, int64_t(tpg::device_cus()) * stages * stack / P)));
  };
  auto side = [&](int i) { return ns > 1 ? st[1 + i % (ns - 1)] : L.root; };
  stat = launch_cols(side(0), a.b_slices[r], kn ? n : a.K, r, 1, budget(1));   // the local slice
  if (stat != TPG_OK) return stat;
  if (copies) {
    stat = hold_deliveries(a.flags, L.root);
    if (stat != TPG_OK) return stat;
  }
  for (int g = 0; g < G; ++g) {
    if (copies) {
      const void* src[kMaxP];
      for (int t = t0(g); t < t0(g + 1); ++t) src[t - t0(g)] = a.b_slices[(r + t) % P];
      stat = deliver(t0(g) - 1, src, t0(g + 1) - t0(g), remote);
      if (stat != TPG_OK) return stat;
    }
    const bool last = g == G - 1;
    hipStream_t cs = last ? L.root : side(g + 1);
    if (!last && copies && ns > 1) {
      if (tpg_status ds = dep_now(cx, cx.ev_copy[g], L.root, cs); ds != TPG_OK) return ds;
    }
    if (wrap_one && passes_last(g)) {
      const int t = t0(g), s = (r + t) % P, run = t0(g + 1) - t;
      const void* Bp = kn ? static_cast<const void*>(ws + size_t(t - 1) * n * eb)
                          : static_cast<const void*>(ws + (t - 1) * slice_b);
      stat = launch_cols(cs, Bp, kn ? int64_t(remote) * n : a.K, s, run, budget(run), static_cast<int>((P - s) * n));
      if (stat != TPG_OK) return stat;
      continue;
    }
    for (int t = t0(g); t < t0(g + 1);) {
      const int s = (r + t) % P;
      int run = std::min(t0(g + 1) - t, P - s);
      if (!copies)
        while (run > 1 && !adjacent(s, run)) --run;      // in place: one launch per adjacent stretch
      const void* Bp;
      int64_t ldb;
      if (copies) {
        Bp = kn ? static_cast<const void*>(ws + size_t(t - 1) * n * eb) : static_cast<const void*>(ws + (t - 1) * slice_b);
        ldb = kn ? int64_t(remote) * n : a.K;
      } else {
        Bp = a.b_slices[s];
        ldb = kn ? n : a.K;
      }
      stat = launch_cols(cs, Bp, ldb, s, run, budget(t0(g + 1) - t0(g)));
      if (stat != TPG_OK) return stat;
      t += run;
    }
  }
  return join_streams(cx, L.root, ns, st);
}

// Column-segmented output of the all-gather (several projections sharing
// the gathered input): output columns [col[i], col[i+1]) go to d[i], row
// stride ld[i].
struct OutSegs {
  int n = 0;
  int col[tpg::kMaxSeg] = {};
  uint16_t* d[tpg::kMaxSeg] = {};
  int64_t ld[tpg::kMaxSeg] = {};
};

// Points q's output at global output row `row0`: d, or every segment.
void set_out_rows(tpg::GemmParams& q, const tpg_ag_args& a, const OutSegs* segs, int64_t row0, int64_t nout) {
  if (!segs) {
    q.d = static_cast<uint16_t*>(a.d) + row0 * nout;
    return;
  }
  q.n_seg = segs->n;
  for (int i = 0; i < segs->n; ++i) {
    q.seg_col[i] = segs->col[i];
    q.seg_d[i] = segs->d[i] + row0 * segs->ld[i];
    q.seg_ld[i] = segs->ld[i];
  }
  q.d = q.seg_d[0];
}

// Copy workgroups carried by a gated launch: about 2048 vectors each, at most
// 64, a multiple of 8 (copy first, the tiles keep their XCD placement).
int carried_copy_blocks(size_t slice_b, int P) {
  const int64_t vecs = int64_t(slice_b / 16) * (P - 1);
  const int64_t n = std::min<int64_t>(64, std::max<int64_t>(1, (vecs + 2047) / 2048));
  return static_cast<int>((n + 7) / 8 * 8);
}

// A gated call that carries its deliveries in the GEMM launch: under
// kCarriedMaxFlop, every tile and copy workgroup on the chip at once, and no
// test flag that needs the deliveries on a stream of their own.
bool carried_gates_fit(const tpg_ag_args& a, int dtype, int epi) {
  const int P = a.P;
  if (P < 2 || P - 1 > tpg::kMaxCopySlices || 2.0 * a.M * double(a.N) * a.K >= kCarriedMaxFlop) return false;
  if (a.flags & (TPG_DEBUG_HOLD_DELIVERIES | TPG_DEBUG_NO_GATE | TPG_NO_COPY)) return false;
  const size_t slice_b = size_t(a.M / P) * a.K * elem_bytes(a.ab_dtype);
  const int cp = carried_copy_blocks(slice_b, P);
  return tpg::gated_tiles(static_cast<int>(a.M), static_cast<int>(a.N), dtype, epi, cp) + cp <=
         tpg::device_cus();
}

// Whether a staged call with library-chosen grouping can run as one gated
// launch carrying its deliveries (the staged all-gather's
// prepended per-stage wait inside one persistent launch): the shape rules of
// TPG_IN_KERNEL_GATES, the library's copy kernel, eager issue, and a caller
// stream that is not being captured (a replay would wait for a count its
// counter has already passed).
bool auto_carried(const tpg_ag_args& a, hipStream_t stream) {
  if (a.schedule != TPG_ROTATE_A || a.groups != 0 || a.P < 2 || a.P > tpg::kMaxGateSlices) return false;
  if (a.flags & (TPG_UNSTAGED | TPG_SERIAL_STAGES | TPG_FORCE_GRAPH | TPG_COPY_SDMA | TPG_COPY_SHADER |
                 TPG_IN_KERNEL_GATES | TPG_DEBUG_HOLD_DELIVERIES | TPG_DEBUG_NO_GATE | TPG_NO_COPY))
    return false;
  const int eb = elem_bytes(a.ab_dtype);
  if ((a.M / a.P) % 128 || (a.K * eb) % 128) return false;
  if (stream_capturing(stream)) return false;
  const int dtype = a.ab_dtype == TPG_E4M3 ? tpg::kE4m3 : tpg::kBf16;
  const int epi = a.epilogue == TPG_EPI_SWIGLU ? tpg::kEpiSwiglu : tpg::kEpiAlphaBeta;
  return carried_gates_fit(a, dtype, epi);
}

// TPG_IN_KERNEL_GATES: the staged all-gather as one launch. The stages are
// those of the rotating-A form (the local slice needs no delivery; slice
// (rank + t) mod P arrives in slot t-1), but instead of one GEMM launch per
// run behind a stream event, one launch covers all M rows and each tile of a
// delivered slice waits inside the kernel, before the DMA of each K-chunk,
// for that chunk's counter. The copy kernel runs beside it on a side stream,
// K-chunk-major, storing write-through and bumping the counter of each
// chunk it completes; the counters are zeroed on the root first.
// A call under kCarriedMaxFlop whose tiles and copy workgroups fit on the
// chip at once instead carries the deliveries in the
// GEMM launch itself, as extra workgroups that each bump one counter when
// done, and its delivered slices' tiles wait for all of them before their
// first DMA: one stream and one launch, the counter a word
// of a static array (no zeroing launch). (Not with
// TPG_DEBUG_HOLD_DELIVERIES or TPG_DEBUG_NO_GATE, whose tests need the
// deliveries on a stream of their own.)
// (TPG_NO_COPY: one launch over the slices in place, no gates.)
tpg_status enqueue_ag_gated(Ctx& cx, const tpg_ag_args& a, const Launch& L, const OutSegs* segs,
                            tpg::GemmParams p, int dtype, int layout, int epi, int64_t nout) {
  const int P = a.P, r = a.rank;
  const int eb = elem_bytes(a.ab_dtype);
  const int64_t m = a.M / P;
  const int64_t row_b = a.K * eb;
  const size_t slice_b = size_t(m) * row_b;
  const bool copies = !(a.flags & TPG_NO_COPY) && slice_b > 0 && P > 1;
  char* ws = static_cast<char*>(a.workspace);
  const int nk = static_cast<int>(row_b / 128);                   // 128-byte K-steps
  const int ksteps = (nk + kMaxGateChunks - 1) / kMaxGateChunks;  // K-steps per chunk
  const int nch = (nk + ksteps - 1) / ksteps;
  const int wgs = tpg::chunk_deliver_wgs_per_slice(static_cast<int>(m));
  unsigned* gate = copies ? reinterpret_cast<unsigned*>(ws + round_up(slice_b * (P - 1), 256)) : nullptr;

  p.a = a.a_slices[r];
  p.M = static_cast<int>(a.M);
  p.c = static_cast<const uint16_t*>(a.c);
  set_out_rows(p, a, segs, 0, nout);
  p.a_slice_rows = static_cast<int>(m);
  // delivered slices in their slots after the local one; in place (no
  // copies) the slices are back to back from a_slices[0]
  p.a_local = copies ? static_cast<const uint8_t*>(a.a_slices[r]) : nullptr;
  p.a_slots = copies ? reinterpret_cast<const uint8_t*>(ws) : static_cast<const uint8_t*>(a.a_slices[0]);
  p.gate_local = copies ? r : -1;
  p.gate = gate;
  p.gate_nch = nch;
  p.gate_ksteps = ksteps;
  p.gate_off = (a.flags & TPG_DEBUG_NO_GATE) ? 1 : 0;
  p.gate_need = static_cast<unsigned>(wgs);
  // TPG_DEBUG_GATE_TIMEOUT: one arrival more than will come, 20 us deadline
  const unsigned extra = (a.flags & TPG_DEBUG_GATE_TIMEOUT) ? 1u : 0u;
  if (extra) p.gate_deadline = 2000u;
  p.gate_need += extra;
  if (!copies) return gemm_on(cx, L, L.root, p, dtype, layout, epi);

  if (carried_gates_fit(a, dtype, epi)) {
    // the copy rides in the GEMM launch, its workgroups first; one
    // counter (a slot of the static array that only grows: no zeroing launch)
    unsigned long long* words = nullptr;
    HIP_TRY(tpg::gate_words(&words));
    const size_t w = static_cast<size_t>(take_gate_number(*cx.seq) % tpg::kGateWords);
    std::vector<uint64_t>& total = cx.seq->gate_total;
    p.gate = nullptr;
    p.gate64 = words + w;
    p.cp_blocks = carried_copy_blocks(slice_b, P);
    p.cp_n = P - 1;
    for (int t = 1; t < P; ++t) p.cp_src[t - 1] = static_cast<const uint8_t*>(a.a_slices[(r + t) % P]);
    p.cp_dst = reinterpret_cast<uint8_t*>(ws);
    p.cp_dst_stride = static_cast<int64_t>(slice_b);
    p.cp_nvec = static_cast<int64_t>(slice_b / 16);
    p.gate_nch = 0;          // one word for every delivered slice
    p.gate_ksteps = nk;      // waited for once, before a tile's first DMA
    p.gate_want64 = total[w] + static_cast<uint64_t>(p.cp_blocks) + extra;
    const tpg_status gs = gemm_on(cx, L, L.root, p, dtype, layout, epi);
    if (gs == TPG_OK) total[w] += static_cast<uint64_t>(p.cp_blocks);   // the copy workgroups' adds
    return gs;
  }
  if (a.flags & kAutoCarried) return fail(TPG_ERR_INVALID, "internal: carried gates chosen but not possible");
  HIP_TRY(tpg::launch_fill_zero16(gate, kGateCounterBytes, L.root));
  hipStream_t st[kStreams];
  tpg_status stat = fork_streams(cx, L.root, 2, st);   // the side stream starts after the zeroing
  if (stat != TPG_OK) return stat;
  // the copy is issued first: were the two launches ever run one after the
  // other, it must be the copy that goes first
  stat = hold_deliveries(a.flags, st[1]);
  if (stat != TPG_OK) return stat;
  tpg::ChunkDeliverParams d;
  std::memset(&d, 0, sizeof(d));
  for (int t = 1; t < P; ++t) d.src[t - 1] = static_cast<const uint8_t*>(a.a_slices[(r + t) % P]);
  d.dst = reinterpret_cast<uint8_t*>(ws);
  d.gate = gate;
  d.rows = static_cast<int>(m);
  d.row_bytes = row_b;
  d.chunk_bytes = int64_t(ksteps) * 128;
  d.n = P - 1;
  d.nch = nch;
  d.wg_per_slice = wgs;
  HIP_TRY(tpg::launch_chunk_deliver(d, st[1]));
  stat = gemm_on(cx, L, L.root, p, dtype, layout, epi);
  if (stat != TPG_OK) return stat;
  return join_streams(cx, L.root, 2, st);
}

tpg_status enqueue_ag(Ctx& cx, const tpg_ag_args& a, const Launch& L, const OutSegs* segs = nullptr) {
  if (a.schedule == TPG_ROTATE_B) return enqueue_ag_rotb(cx, a, L);
  const int P = a.P, r = a.rank;
  const int eb = elem_bytes(a.ab_dtype);
  const int64_t m = a.M / P;
  const bool sw = a.epilogue == TPG_EPI_SWIGLU;
  const int64_t nout = sw ? a.N / 2 : a.N;
  const size_t slice_b = size_t(m) * a.K * eb;
  const bool copies = !(a.flags & TPG_NO_COPY) && slice_b > 0 && (P > 1 || (a.flags & TPG_UNSTAGED));
  const Copy ck = copy_of(a.flags, Copy::Kernel);
  char* ws = static_cast<char*>(a.workspace);

  tpg::GemmParams p = base_params();
  p.b = a.b;
  p.ldb = a.b_layout == TPG_B_NK ? a.K : a.N;
  p.lda = a.K;
  p.ldc = nout;
  p.ldd = nout;
  p.N = static_cast<int>(a.N);
  p.K = static_cast<int>(a.K);
  p.alpha = a.alpha;
  p.beta = a.beta;
  p.vec_ok = (nout % 8) == 0;
  const int dtype = a.ab_dtype == TPG_E4M3 ? tpg::kE4m3 : tpg::kBf16;
  const int layout = a.b_layout == TPG_B_KN ? tpg::kKN : tpg::kNK;
  const int epi = sw ? tpg::kEpiSwiglu : tpg::kEpiAlphaBeta;

  if (a.flags & (TPG_IN_KERNEL_GATES | kAutoCarried))
    return enqueue_ag_gated(cx, a, L, segs, p, dtype, layout, epi, nout);

  if (a.flags & TPG_UNSTAGED) {
    // single stage: gather every slice (rank order), then one GEMM over all M rows
    const void* A = a.M > 0 ? a.a_slices[0] : nullptr;
    if (copies) {
      tpg_status hs = hold_deliveries(a.flags, L.root);
      if (hs != TPG_OK) return hs;
      hs = deliver_slices(ck, a.a_slices, P, slice_b, ws, slice_b, L.root);
      if (hs != TPG_OK) return hs;
      A = ws;
    }
    p.a = A;
    p.c = static_cast<const uint16_t*>(a.c);
    set_out_rows(p, a, segs, 0, nout);
    p.M = static_cast<int>(a.M);
    return gemm_on(cx, L, L.root, p, dtype, layout, epi);
  }

  // staged: stage t multiplies slice s = (rank + t) mod P, local first. The
  // P-1 remote stages are cut into G runs; run g waits for one event and is
  // one GEMM launch per stretch of D rows that does not wrap past slice P-1.
  const int remote = P - 1;
  const int G = remote == 0 ? 0 : (a.groups > 0 ? std::min(a.groups, remote) : auto_groups(remote));
  auto t0 = [&](int g) { return 1 + (g * remote) / G; };
  auto adjacent = [&](int s, int run) {   // a_slices[s .. s+run) back to back in memory
    for (int i = 1; i < run; ++i)
      if (static_cast<const char*>(a.a_slices[s + i]) != static_cast<const char*>(a.a_slices[s]) + i * slice_b)
        return false;
    return true;
  };
  const bool no_gate = (a.flags & TPG_DEBUG_NO_GATE) != 0;
  // A run whose slices pass slice P-1 writes two stretches of output rows.
  // With slices of a multiple of 256 rows (no tile straddles the wrap) it is
  // one launch whose tiles past the wrap write P * m rows earlier, reading A
  // from the slots in arrival order or, in place, from the slices back to
  // back from a_slices[0]. Otherwise it is one launch per stretch, the
  // second on a stream of its own beside the first (on one stream, one
  // after the other, the two took twice as long: 1024 x 2048 x 16384 bf16
  // in 4 slices at rank 1, 207 against 109 us unstaged).
  auto passes_last = [&](int g) { return (r + t0(g)) % P + (t0(g + 1) - t0(g)) > P; };
  tpg::GemmParams probe = p;
  probe.M = static_cast<int>(m);
  const bool wrap_one = m % 256 == 0 && tpg::wrap_in_one_launch(probe, dtype, layout) && (copies || adjacent(0, P));
  bool wraps = false;
  for (int g = 0; g < G && !no_gate; ++g) wraps = wraps || (!wrap_one && passes_last(g));
  const int ns = (a.flags & TPG_SERIAL_STAGES) ? 1 : std::min(G + 1 + (wraps ? 1 : 0), kStreams);
  const bool split_side = wraps && ns > 2;
  hipStream_t st[kStreams];
  tpg_status stat = fork_streams(cx, L.root, ns, st, copies);   // the deliveries follow on the root
  if (stat != TPG_OK) return stat;
  // Stage runs on parallel streams share the chip: each launch sizes its
  // tiles for the CUs its run's rows would get (runs that must share a
  // stream get proportionally more), so the launches in flight together form
  // about one wave of tiles rather than each sizing its tiles for the chip.
  const int stack = (G + 1 + ns - 1) / ns;                // runs per stream
  auto budget = [&](int stages) {
    if (ns == 1) return 0;
    return static_cast<int>(std::min<int64_t>(tpg::device_cus(),
                                              std::max<int64_t>(8, int64_t(tpg::device_cus()) * stages * stack / P)));
  };
  auto launch_rows = [&](hipStream_t cs, const void* A, int s, int run, int cus, const tpg::GemmParams* job,
                         int wrap_row = 0) {
    tpg::GemmParams q = p;
    q.a = A;
    q.M = static_cast<int>(run * m);
    q.c = a.c ? static_cast<const uint16_t*>(a.c) + s * m * nout : nullptr;
    set_out_rows(q, a, segs, s * m, nout);
    q.cu_budget = cus;
    if (wrap_row > 0) {
      q.wrap_row = wrap_row;
      q.wrap_back = static_cast<int>(P * m);
      q.wrap_a = copies ? 0 : 1;
    }
    if (job) {
      q.cp_blocks = job->cp_blocks;
      q.cp_n = job->cp_n;
      for (int i = 0; i < job->cp_n; ++i) q.cp_src[i] = job->cp_src[i];
      q.cp_dst = job->cp_dst;
      q.cp_dst_stride = job->cp_dst_stride;
      q.cp_nvec = job->cp_nvec;
    }
    return gemm_on(cx, L, cs, q, dtype, layout, epi);
  };
  // On one stream (a latency-bound call) the local stage's launch carries
  // the deliveries as extra workgroups: the local stage then runs beside
  // them, as the staged schedule intends, with one launch fewer. The remote
  // run follows in stream order. (Only with the library's copy kernel, a
  // single remote run of at most kMaxCopySlices slices, and a latency-bound
  // call: a larger call on one stream, TPG_SERIAL_STAGES asked for, runs its
  // deliveries and stages strictly one after another.)
  tpg::GemmParams job = base_params();
  bool carry = false;
  if (copies && ns == 1 && G == 1 && ck == Copy::Kernel && remote <= tpg::kMaxCopySlices &&
      2.0 * a.M * double(a.N) * a.K < kLatencyBoundFlop) {
    const void* src[kMaxP];
    for (int t = 1; t < P; ++t) src[t - 1] = a.a_slices[(r + t) % P];
    const int64_t vecs = int64_t(slice_b / 16) * remote;
    const int cp_blocks = static_cast<int>(std::min<int64_t>(64, std::max<int64_t>(1, (vecs + 2047) / 2048)));
    // the copy workgroups must find CUs of their own beside the local stage's
    // tiles (the persistent grid holds one workgroup per CU): otherwise they
    // would queue behind the tile loop and the deliveries run separately
    const int local_tiles = tpg::gemm_tiles(static_cast<int>(m), static_cast<int>(a.N), dtype, epi, 1, 0);
    if (tpg::deliver_ok(src, remote, slice_b, ws, slice_b) && local_tiles + cp_blocks <= tpg::device_cus()) {
      carry = true;
      job.cp_n = remote;
      for (int i = 0; i < remote; ++i) job.cp_src[i] = static_cast<const uint8_t*>(src[i]);
      job.cp_dst = reinterpret_cast<uint8_t*>(ws);
      job.cp_dst_stride = static_cast<int64_t>(slice_b);
      job.cp_nvec = static_cast<int64_t>(slice_b / 16);
      job.cp_blocks = cp_blocks;
    }
  }
  // Stream roles. The deliveries run back to back on the root and the last
  // run follows them there in stream order, so the call's critical path (last
  // delivery, then the last run) waits on no other queue. The local stage,
  // which needs no delivery, and the earlier runs go to the other streams,
  // each earlier run gated by one event recorded on the root after its
  // slices. (With the local stage on the root and the deliveries on a side
  // stream, the first delivery started ~17 us late and the call took ~127 us.)
  auto side = [&](int i) { return ns > 1 ? st[1 + i % (ns - 1)] : L.root; };
  // Issue order: every delivery first (they are the critical path; issued
  // after the local stage's launch, the first started ~10 us late), then
  // the local stage, then the runs.
  Dep copied[kMaxP];                     // run g's slices delivered (runs before the last)
  if (copies) {
    stat = hold_deliveries(a.flags, L.root);
    if (stat != TPG_OK) return stat;
    for (int g = 0; g < G && !carry; ++g) {
      const void* src[kMaxP];
      for (int t = t0(g); t < t0(g + 1); ++t) src[t - t0(g)] = a.a_slices[(r + t) % P];
      stat = deliver_slices(ck, src, t0(g + 1) - t0(g), slice_b, ws + (t0(g) - 1) * slice_b, slice_b, L.root);
      if (stat != TPG_OK) return stat;
      if (g < G - 1 && ns > 1 && !no_gate) {
        stat = dep_mark(cx, cx.ev_copy[g], L.root, &copied[g]);
        if (stat != TPG_OK) return stat;
      }
    }
  }
  Dep delivered;                          // every delivery done (the last run's second part waits for it)
  if (copies && split_side) {
    stat = dep_mark(cx, cx.ev_copy[G], L.root, &delivered, true);   // the last run follows on the root
    if (stat != TPG_OK) return stat;
  }
  stat = launch_rows(side(0), a.a_slices[r], r, 1, budget(1), carry ? &job : nullptr);   // stage 0: the local slice
  if (stat != TPG_OK) return stat;
  for (int g = 0; g < G; ++g) {
    const bool last = g == G - 1;
    // TPG_DEBUG_NO_GATE: every run on a side stream, with no wait for its slices
    hipStream_t cs = (last && !no_gate) ? L.root : side(g + 1);
    if (!last && copies && ns > 1 && !no_gate) {
      stat = dep_await(cs, copied[g]);
      if (stat != TPG_OK) return stat;
    }
    if (wrap_one && passes_last(g)) {
      const int s = (r + t0(g)) % P, run = t0(g + 1) - t0(g);
      const void* A = copies ? static_cast<const void*>(ws + (t0(g) - 1) * slice_b) : a.a_slices[s];
      stat = launch_rows(cs, A, s, run, budget(run), nullptr, static_cast<int>((P - s) * m));
      if (stat != TPG_OK) return stat;
      continue;
    }
    const bool run_wraps = split_side && passes_last(g);
    for (int t = t0(g); t < t0(g + 1);) {
      const int s = (r + t) % P;
      int run = std::min(t0(g + 1) - t, P - s);
      if (!copies)
        while (run > 1 && !adjacent(s, run)) --run;      // in place: one launch per adjacent stretch
      const void* A = copies ? static_cast<const void*>(ws + (t - 1) * slice_b) : a.a_slices[s];
      hipStream_t ps = cs;
      if (run_wraps && s < (r + t0(g)) % P) {            // past slice P-1: beside the first part
        ps = st[ns - 1];
        if (copies) {
          stat = dep_await(ps, last ? delivered : copied[g]);
          if (stat != TPG_OK) return stat;
        }
      }
      // the two parts of a wrapping run side by side: each sized for its own stages
      stat = launch_rows(ps, A, s, run, budget(run_wraps ? run : t0(g + 1) - t0(g)), nullptr);
      if (stat != TPG_OK) return stat;
      t += run;
    }
  }
  return join_streams(cx, L.root, ns, st);
}

std::string ag_key(const tpg_ag_args& a) {
  std::ostringstream os;
  os << "ag|";
  put(os, a.M); put(os, a.N); put(os, a.K); put(os, a.P); put(os, a.rank); put(os, a.ab_dtype);
  put(os, a.b_layout); put(os, a.epilogue); put(os, a.b); put(os, a.c); put(os, a.d);
  put(os, a.alpha); put(os, a.beta); put(os, a.workspace); put(os, a.flags); put(os, a.groups);
  put(os, a.schedule);
  const int na = a.schedule == TPG_ROTATE_B ? 1 : a.P;
  for (int s = 0; s < na && a.a_slices; ++s) put(os, a.a_slices[s]);
  for (int s = 0; a.schedule == TPG_ROTATE_B && s < a.P && a.b_slices; ++s) put(os, a.b_slices[s]);
  return os.str();
}

// ---------------------------------------------------------------- several projections
// The projections of one gathered input run as one all-gather GEMM over the
// weights side by side (N = sum n[i]); the epilogue stores each column block
// to its own output. Weights already back to back in memory are read in
// place; otherwise they are copied side by side into the workspace (after
// the all-gather's receive slots) on the root stream first.
int64_t agm_ntot(const tpg_agm_args* a) {
  int64_t t = 0;
  for (int i = 0; i < a->n_out && i < TPG_MAX_PROJ; ++i) t += a->n[i];
  return t;
}

bool agm_weights_adjacent(const tpg_agm_args* a) {
  const int eb = elem_bytes(a->ab_dtype);
  const char* at = static_cast<const char*>(a->b[0]);
  for (int i = 0; i < a->n_out; ++i) {
    if (a->n[i] == 0) continue;
    if (static_cast<const char*>(a->b[i]) != at) return false;
    at += size_t(a->n[i]) * a->K * eb;
  }
  return true;
}

// The equivalent single-B all-gather call (B and D filled in by the caller).
tpg_ag_args agm_as_ag(const tpg_agm_args* a) {
  tpg_ag_args g;
  std::memset(&g, 0, sizeof(g));
  g.M = a->M;
  g.N = agm_ntot(a);
  g.K = a->K;
  g.P = a->P;
  g.rank = a->rank;
  g.ab_dtype = a->ab_dtype;
  g.b_layout = TPG_B_NK;
  g.epilogue = TPG_EPI_ALPHA_BETA;
  g.a_slices = a->a_slices;
  g.alpha = a->alpha;
  g.beta = 0.0f;
  g.flags = a->flags;
  g.groups = a->groups;
  g.schedule = TPG_ROTATE_A;
  return g;
}

size_t agm_ws(const tpg_agm_args* a) {
  if (!a || a->n_out < 1 || a->n_out > TPG_MAX_PROJ || a->P < 1 || a->M < 0 || a->K < 0) return 0;
  for (int i = 0; i < a->n_out; ++i)
    if (a->n[i] < 0) return 0;
  const tpg_ag_args g = agm_as_ag(a);
  size_t need = round_up(ag_ws(&g), 256);
  if (!agm_weights_adjacent(a)) need += round_up(size_t(g.N) * a->K * elem_bytes(a->ab_dtype), 256);
  return need;
}

tpg_status validate_agm(const tpg_agm_args* a, size_t need) {
  if (!a) return fail(TPG_ERR_INVALID, "args is NULL");
  if (a->n_out < 1 || a->n_out > TPG_MAX_PROJ) return fail(TPG_ERR_INVALID, "n_out must be in [1, 4]");
  int64_t ntot = 0;
  for (int i = 0; i < a->n_out; ++i) {
    if (a->n[i] < 0 || a->n[i] % 8) return fail(TPG_ERR_INVALID, "every n[i] must be a non-negative multiple of 8");
    ntot += a->n[i];
  }
  if (!fits_int(ntot)) return fail(TPG_ERR_UNSUPPORTED, "sum of n[i] must be below 2^31");
  // the shared checks (P, rank, M, K, dtype, slices, flags) on an equivalent
  // call with one 8-column projection (the weights and outputs are checked
  // below, each with its own size)
  tpg_ag_args g = agm_as_ag(a);
  g.N = 0;
  for (int i = 0; i < a->n_out; ++i)
    if (a->n[i] > 0) {
      g.N = 8;
      g.b = a->b[i];
      g.d = a->d[i];
      break;
    }
  tpg_status st = validate_ag(&g, 0);
  if (st != TPG_OK) return st;
  const int eb = elem_bytes(a->ab_dtype);
  std::vector<Range> ins, outs;
  for (int s = 0; a->M > 0 && s < a->P; ++s) ins.push_back({a->a_slices[s], size_t(a->M / a->P) * a->K * eb});
  for (int i = 0; i < a->n_out; ++i) {
    if (a->n[i] == 0) continue;
    if ((!a->b[i] && a->K) || (!a->d[i] && a->M)) return fail(TPG_ERR_INVALID, "NULL weight or output");
    if (!aligned16(a->b[i]) || !aligned16(a->d[i])) return fail(TPG_ERR_UNSUPPORTED, "weights and outputs must be 16-byte aligned");
    ins.push_back({a->b[i], size_t(a->n[i]) * a->K * eb});
    outs.push_back({a->d[i], size_t(a->M) * a->n[i] * 2});
  }
  if (need && (!a->workspace || a->workspace_bytes < need))
    return fail(TPG_ERR_WORKSPACE, "workspace smaller than tpgemm_stage_ag_multi_workspace_size()");
  const Range wr{a->workspace, need};
  if (need && !aligned16(a->workspace)) return fail(TPG_ERR_UNSUPPORTED, "workspace not 16-byte aligned");
  for (size_t i = 0; i < outs.size(); ++i) {
    for (const auto& r : ins)
      if (overlaps(outs[i], r)) return fail(TPG_ERR_INVALID, "an output overlaps an input");
    for (size_t j = i + 1; j < outs.size(); ++j)
      if (overlaps(outs[i], outs[j])) return fail(TPG_ERR_INVALID, "outputs overlap each other");
    if (overlaps(outs[i], wr)) return fail(TPG_ERR_INVALID, "workspace overlaps an output");
  }
  for (const auto& r : ins)
    if (overlaps(wr, r)) return fail(TPG_ERR_INVALID, "workspace overlaps an input");
  return TPG_OK;
}

tpg_status enqueue_agm(Ctx& cx, const tpg_agm_args& a, const Launch& L) {
  tpg_ag_args g = agm_as_ag(&a);
  const int eb = elem_bytes(a.ab_dtype);
  char* ws = static_cast<char*>(a.workspace);
  g.workspace = ws;
  g.workspace_bytes = a.workspace_bytes;
  OutSegs segs;
  int col = 0;
  for (int i = 0; i < a.n_out; ++i) {
    if (a.n[i] == 0) continue;
    segs.col[segs.n] = col;
    segs.d[segs.n] = static_cast<uint16_t*>(a.d[i]);
    segs.ld[segs.n] = a.n[i];
    ++segs.n;
    col += static_cast<int>(a.n[i]);
  }
  g.d = segs.d[0];
  if (agm_weights_adjacent(&a)) {
    for (int i = 0; i < a.n_out; ++i)
      if (a.n[i] > 0) {
        g.b = a.b[i];
        break;
      }
  } else {
    // weights side by side after the receive slots, on the root before any stage
    char* wb = ws + round_up(ag_ws(&g), 256);
    size_t off = 0;
    for (int i = 0; i < a.n_out; ++i) {
      if (a.n[i] == 0) continue;
      const size_t bytes = size_t(a.n[i]) * a.K * eb;
      tpg_status st = deliver_slices(Copy::Kernel, &a.b[i], 1, bytes, wb + off, bytes, L.root);
      if (st != TPG_OK) return st;
      off += bytes;
    }
    g.b = wb;
  }
  return enqueue_ag(cx, g, L, &segs);
}

std::string agm_key(const tpg_agm_args& a) {
  std::ostringstream os;
  os << "agm|";
  put(os, a.M); put(os, a.K); put(os, a.P); put(os, a.rank); put(os, a.ab_dtype); put(os, a.n_out);
  for (int i = 0; i < a.n_out; ++i) {
    put(os, a.b[i]); put(os, a.n[i]); put(os, a.d[i]);
  }
  put(os, a.alpha); put(os, a.flags); put(os, a.groups); put(os, a.workspace);
  for (int s = 0; a.a_slices && s < a.P; ++s) put(os, a.a_slices[s]);
  return os.str();
}

// ---------------------------------------------------------------- reduce-scatter
// One incoming partial: an (m, N) row block, or with TPG_TILE_B an (M, n)
// column block, bf16.
size_t rs_part_bytes(const tpg_rs_args* a) {
  return a->schedule == TPG_TILE_B ? size_t(a->M) * (a->N / a->P) * 2 : size_t(a->M / a->P) * a->N * 2;
}

size_t rs_slot(const tpg_rs_args* a) { return round_up(rs_part_bytes(a), 256); }

size_t rs_ws(const tpg_rs_args* a) {
  if (!a || a->P < 1 || a->M < 0 || a->N < 0 || !a->incoming || (a->flags & TPG_NO_COPY)) return 0;
  return rs_slot(a) * (a->P - 1);
}

tpg_status validate_rs(const tpg_rs_args* a, size_t need) {
  if (!a) return fail(TPG_ERR_INVALID, "args is NULL");
  if (a->P < 1 || a->P > kMaxP) return fail(TPG_ERR_INVALID, "P must be in [1, 64]");
  if (a->rank < 0 || a->rank >= a->P) return fail(TPG_ERR_INVALID, "rank must be in [0, P)");
  if (a->M < 0 || a->N < 0 || a->K < 0) return fail(TPG_ERR_INVALID, "negative dimension");
  if (a->schedule != TPG_TILE_A && a->schedule != TPG_TILE_B) return fail(TPG_ERR_INVALID, "bad schedule");
  const bool tileb = a->schedule == TPG_TILE_B;
  if (!tileb && a->M % a->P) return fail(TPG_ERR_INVALID, "M must be a multiple of P");
  if (tileb && a->N % a->P) return fail(TPG_ERR_INVALID, "TPG_TILE_B: N must be a multiple of P");
  if (tileb && (a->N / a->P) % 8) return fail(TPG_ERR_UNSUPPORTED, "TPG_TILE_B: N/P must be a multiple of 8");
  if (a->flags & ~kKnownFlags) return fail(TPG_ERR_INVALID, "unknown flag bits");
  if (tpg_status ng = validate_no_gate(a->flags, true); ng != TPG_OK) return ng;
  if (tpg_status ig = validate_in_kernel_gates(a->flags, false); ig != TPG_OK) return ig;
  if (!copy_flags_ok(a->flags))
    return fail(TPG_ERR_INVALID, "TPG_COPY_SDMA, TPG_COPY_SHADER and TPG_COPY_KERNEL are exclusive");
  if (a->ab_dtype != TPG_BF16 && a->ab_dtype != TPG_E4M3) return fail(TPG_ERR_INVALID, "bad ab_dtype");
  if (a->b_layout != TPG_B_NK && a->b_layout != TPG_B_KN) return fail(TPG_ERR_INVALID, "bad b_layout");
  if (!fits_int(a->M) || !fits_int(a->N) || !fits_int(a->K))
    return fail(TPG_ERR_UNSUPPORTED, "dimensions must be below 2^31");
  if (a->ab_dtype == TPG_E4M3 && a->b_layout == TPG_B_KN)
    return fail(TPG_ERR_UNSUPPORTED, "e4m3 operands need the NK layout of B");
  if (a->K % (a->ab_dtype == TPG_E4M3 ? 16 : 8))
    return fail(TPG_ERR_UNSUPPORTED, "K must be a multiple of 8 (bf16) or 16 (e4m3)");
  if (a->b_layout == TPG_B_KN && a->N % 8) return fail(TPG_ERR_UNSUPPORTED, "KN layout needs N % 8 == 0");
  const int eb = elem_bytes(a->ab_dtype);
  std::vector<Range> inputs;
  const size_t a_b = size_t(a->M) * a->K * eb, b_b = size_t(a->N) * a->K * eb;
  if (!a->a && a_b) return fail(TPG_ERR_INVALID, "A is NULL");
  if (!a->b && b_b) return fail(TPG_ERR_INVALID, "B is NULL");
  if (!aligned16(a->a) || !aligned16(a->b)) return fail(TPG_ERR_UNSUPPORTED, "A/B not 16-byte aligned");
  inputs.push_back({a->a, a_b});
  inputs.push_back({a->b, b_b});
  int n_in = 0;
  const size_t part_b = rs_part_bytes(a);
  if (a->incoming) {
    for (int j = 0; j < a->P; ++j) {
      if (j == a->rank || !a->incoming[j]) continue;
      if (!aligned16(a->incoming[j])) return fail(TPG_ERR_UNSUPPORTED, "incoming partial not 16-byte aligned");
      inputs.push_back({a->incoming[j], part_b});
      ++n_in;
    }
  }
  if ((a->flags & TPG_NO_COPY) && n_in > tpg::kMaxAddList)
    return fail(TPG_ERR_UNSUPPORTED, "NO_COPY reads at most 16 incoming partials in place");
  const size_t d_b = size_t(a->M) * a->N * 2;
  if (!a->d && d_b) return fail(TPG_ERR_INVALID, "D is NULL");
  if (!aligned16(a->d)) return fail(TPG_ERR_UNSUPPORTED, "D not 16-byte aligned");
  if (need && (!a->workspace || a->workspace_bytes < need))
    return fail(TPG_ERR_WORKSPACE, "workspace smaller than tpgemm_stage_rs_workspace_size()");
  const Range dr{a->d, d_b}, wr{a->workspace, need};
  for (const auto& r : inputs) {
    if (overlaps(dr, r)) return fail(TPG_ERR_INVALID, "D overlaps an input");
    if (overlaps(wr, r)) return fail(TPG_ERR_INVALID, "workspace overlaps an input");
  }
  if (overlaps(dr, wr)) return fail(TPG_ERR_INVALID, "workspace overlaps D");
  if (need && !aligned16(a->workspace)) return fail(TPG_ERR_UNSUPPORTED, "workspace not 16-byte aligned");
  return TPG_OK;
}

tpg_status enqueue_rs(Ctx& cx, const tpg_rs_args& a, const Launch& L) {
  const int P = a.P, r = a.rank;
  const int eb = elem_bytes(a.ab_dtype);
  const bool tileb = a.schedule == TPG_TILE_B;
  const int64_t m = a.M / P;          // TPG_TILE_A: rows per block
  const int64_t n = a.N / P;          // TPG_TILE_B: columns per block
  const size_t part_b = rs_part_bytes(&a);
  const size_t slot = rs_slot(&a);
  char* ws = static_cast<char*>(a.workspace);
  const Copy ck = copy_of(a.flags, Copy::Kernel);

  // peers whose partial for block `rank` arrives, in ring order rank+1, rank+2, ...
  std::vector<int> peers;
  if (a.incoming)
    for (int t = 1; t < P; ++t) {
      const int j = (r + t) % P;
      if (a.incoming[j]) peers.push_back(j);
    }
  const bool copies = !(a.flags & TPG_NO_COPY) && !peers.empty() && part_b > 0;

  tpg::GemmParams p = base_params();
  p.b = a.b;
  p.ldb = a.b_layout == TPG_B_NK ? a.K : a.N;
  p.lda = a.K;
  p.ldd = a.N;
  p.ld_add = tileb ? n : a.N;
  p.N = static_cast<int>(a.N);
  p.K = static_cast<int>(a.K);
  p.alpha = a.alpha;
  p.beta = 0.0f;
  p.vec_ok = (a.N % 8) == 0;
  const int dtype = a.ab_dtype == TPG_E4M3 ? tpg::kE4m3 : tpg::kBf16;
  const int layout = a.b_layout == TPG_B_KN ? tpg::kKN : tpg::kNK;

  auto set_adds = [&](tpg::GemmParams& q) {
    if (copies) {
      q.add_base = reinterpret_cast<const uint16_t*>(ws);
      q.add_stride = static_cast<int64_t>(slot / 2);
      q.n_add_strided = static_cast<int>(peers.size());
    } else {
      for (size_t i = 0; i < peers.size(); ++i)
        q.add_list[i] = static_cast<const uint16_t*>(a.incoming[peers[i]]);
      q.n_add_list = static_cast<int>(peers.size());
    }
  };

  // Deliveries go back to back on the root (the caller's stream or the
  // capture stream); whatever reads them follows there in stream order.
  auto deliver = [&]() -> tpg_status {
    if (!copies) return TPG_OK;
    tpg_status hs = hold_deliveries(a.flags, L.root);
    if (hs != TPG_OK) return hs;
    const void* src[kMaxP];
    for (size_t i = 0; i < peers.size(); ++i) src[i] = a.incoming[peers[i]];
    return deliver_slices(ck, src, static_cast<int>(peers.size()), part_b, ws, slot, L.root);
  };

  if (a.flags & TPG_UNSTAGED) {
    // one GEMM over all blocks once every partial has arrived; the adds apply
    // to the rows of the own block only
    tpg_status ds = deliver();
    if (ds != TPG_OK) return ds;
    p.a = a.a;
    p.d = static_cast<uint16_t*>(a.d);
    p.M = static_cast<int>(a.M);
    if (!tileb) {
      p.add_row0 = static_cast<int>(r * m);
      p.add_row1 = static_cast<int>((r + 1) * m);
    } else {
      p.add_row0 = 0;
      p.add_row1 = static_cast<int>(a.M);
      p.add_col0 = static_cast<int>(r * n);
      p.add_col1 = static_cast<int>((r + 1) * n);
    }
    set_adds(p);
    return gemm_on(cx, L, L.root, p, dtype, layout, tpg::kEpiAlphaBeta);
  }

  // stages 0..P-2 emit the blocks (rank+1+t) mod P, cut into G runs (one
  // launch per run and non-wrapping stretch); the own block is the last stage
  const int emit = P - 1;
  // emitted blocks wait for nothing: by default one launch per non-wrapping
  // stretch, so each launch fills the chip with the largest tiles
  const int G = emit == 0 ? 0 : (a.groups > 0 ? std::min(a.groups, emit) : 1);
  auto t0 = [&](int g) { return (g * emit) / G; };
  const int ns = (a.flags & TPG_SERIAL_STAGES) ? 1 : std::min(G + 1, kStreams);
  hipStream_t st[kStreams];
  tpg_status stat = fork_streams(cx, L.root, ns, st);
  if (stat != TPG_OK) return stat;
  auto side = [&](int i) { return ns > 1 ? st[1 + i % (ns - 1)] : L.root; };
  // The own block waits for every delivery while the emitted blocks run;
  // it sizes its tiles for the CUs the emitted launches leave idle in their
  // last round of tiles, so that it fills that round instead of adding one.
  int64_t emitted_tiles = 0;
  auto launch_blocks = [&](hipStream_t cs, int blk, int run, bool own, int wrap_row = 0) {
    tpg::GemmParams q = p;
    if (!tileb) {     // row blocks: rows of A and D
      q.M = static_cast<int>(run * m);
      q.a = static_cast<const char*>(a.a) + size_t(blk) * m * a.K * eb;
      q.d = static_cast<uint16_t*>(a.d) + blk * m * a.N;
      if (wrap_row > 0) {    // blocks past P-1: A's and D's rows P * m earlier
        q.wrap_row = wrap_row;
        q.wrap_back = static_cast<int>(P * m);
        q.wrap_a = 1;
      }
    } else {          // column blocks: rows of B (NK) or its columns (KN), columns of D
      q.M = static_cast<int>(a.M);
      q.a = a.a;
      q.N = static_cast<int>(run * n);
      q.b = static_cast<const char*>(a.b) + size_t(blk) * n * (a.b_layout == TPG_B_NK ? a.K : 1) * eb;
      q.d = static_cast<uint16_t*>(a.d) + blk * n;
    }
    if (own) {
      q.add_row0 = 0;
      q.add_row1 = q.M;
      set_adds(q);
      const int cus = tpg::device_cus();
      const int rem = static_cast<int>(emitted_tiles % cus);
      if (ns > 1 && rem > 0) q.cu_budget = cus - rem;
    } else {
      emitted_tiles += tpg::gemm_tiles(q.M, q.N, dtype, tpg::kEpiAlphaBeta, 1, 0);
    }
    return gemm_on(cx, L, cs, q, dtype, layout, tpg::kEpiAlphaBeta);
  };
  // A run of row blocks that passes block P-1 is one launch whose tiles
  // past the wrap go P * m rows back (blocks of a multiple of 256 rows: no
  // tile straddles the wrap), else one launch per stretch.
  tpg::GemmParams probe = p;
  probe.M = static_cast<int>(m);
  const bool wrap_one = !tileb && m % 256 == 0 && tpg::wrap_in_one_launch(probe, dtype, layout);
  // Stream roles as in the all-gather: the emitted runs on the other streams
  // start at once; the root takes the deliveries and then the own block,
  // which reads them, in stream order.
  for (int g = 0; g < G; ++g) {
    hipStream_t cs = side(g);
    const int first = (r + 1 + t0(g)) % P, span = t0(g + 1) - t0(g);
    if (wrap_one && first + span > P) {
      stat = launch_blocks(cs, first, span, false, static_cast<int>((P - first) * m));
      if (stat != TPG_OK) return stat;
      continue;
    }
    for (int t = t0(g); t < t0(g + 1);) {
      const int blk = (r + 1 + t) % P;
      const int run = std::min(t0(g + 1) - t, P - blk);
      stat = launch_blocks(cs, blk, run, false);
      if (stat != TPG_OK) return stat;
      t += run;
    }
  }
  stat = deliver();
  if (stat != TPG_OK) return stat;
  // TPG_DEBUG_NO_GATE: the own block on a side stream, not after the deliveries
  stat = launch_blocks((a.flags & TPG_DEBUG_NO_GATE) ? side(G) : L.root, r, 1, true);
  if (stat != TPG_OK) return stat;
  return join_streams(cx, L.root, ns, st);
}

std::string rs_key(const tpg_rs_args& a) {
  std::ostringstream os;
  os << "rs|";
  put(os, a.M); put(os, a.N); put(os, a.K); put(os, a.P); put(os, a.rank); put(os, a.ab_dtype);
  put(os, a.b_layout); put(os, a.a); put(os, a.b); put(os, a.d); put(os, a.alpha);
  put(os, a.workspace); put(os, a.flags); put(os, a.groups); put(os, a.schedule);
  for (int j = 0; a.incoming && j < a.P; ++j) put(os, a.incoming[j]);
  return os.str();
}

// ---------------------------------------------------------------- weight gradient
// d (N, K) = alpha * sum_i G[i, n] X[i, k] over M token rows, one operand
// arriving as P row slices. On the kernel: D rows = n, D columns = k, the
// contraction runs over token rows; A = G read contraction-major (row stride
// N), B = X in the (K, N) layout (row stride K).
int64_t wg_width(const tpg_wg_args* a) { return a->gathered == TPG_GATHER_X ? a->K : a->N; }

size_t wg_slice_bytes(const tpg_wg_args* a) { return size_t(a->M / a->P) * wg_width(a) * 2; }

// Library choice (groups == 0): one gathered launch. Measured on MI355X at
// the weight gradients of the e4m3 all-gather shape (1024 x 8192 over 8192
// token rows, X gathered) and of the SwiGLU block (w13: 4096 x 3584, G
// gathered; w2: 1792 x 4096, X gathered), in us, staged with one run / two
// runs / unstaged: 233 / 233 / 212, 278 / 301 / 252, 181 / 196 / 162. Every
// stage here spans the whole output, so a split contraction pays a second
// prologue and epilogue and an fp32 round trip of the output, and the local
// stage (1/8 of the work) takes longer than its share while the deliveries
// compete with it for the chip.
bool wg_unstaged(const tpg_wg_args* a) { return (a->flags & TPG_UNSTAGED) || a->groups == 0; }

// Receive slots: (P-1) slices in ring order staged, P in rank order unstaged.
size_t wg_recv(const tpg_wg_args* a) {
  if (a->flags & TPG_NO_COPY) return 0;
  return round_up(wg_slice_bytes(a) * (wg_unstaged(a) ? a->P : a->P - 1), 256);
}

// The fp32 partial exists when the call makes more than one launch: staged
// with P > 1.
bool wg_chain(const tpg_wg_args* a) { return !wg_unstaged(a) && a->P > 1; }

size_t wg_ws(const tpg_wg_args* a) {
  if (!a || a->P < 1 || a->P > kMaxP || a->M <= 0 || a->N <= 0 || a->K <= 0 || a->M % a->P) return 0;
  return wg_recv(a) + (wg_chain(a) ? size_t(a->N) * a->K * 4 : 0);
}

tpg_status validate_wg(const tpg_wg_args* a, size_t need) {
  if (!a) return fail(TPG_ERR_INVALID, "args is NULL");
  if (a->P < 1 || a->P > kMaxP) return fail(TPG_ERR_INVALID, "P must be in [1, 64]");
  if (a->rank < 0 || a->rank >= a->P) return fail(TPG_ERR_INVALID, "rank must be in [0, P)");
  if (a->M < 0 || a->N < 0 || a->K < 0) return fail(TPG_ERR_INVALID, "negative dimension");
  if (a->M % a->P) return fail(TPG_ERR_INVALID, "M must be a multiple of P");
  if (a->gathered != TPG_GATHER_X && a->gathered != TPG_GATHER_G) return fail(TPG_ERR_INVALID, "bad gathered");
  if (a->flags & ~kKnownFlags) return fail(TPG_ERR_INVALID, "unknown flag bits");
  if (tpg_status ng = validate_no_gate(a->flags, false); ng != TPG_OK) return ng;
  if (tpg_status ig = validate_in_kernel_gates(a->flags, false); ig != TPG_OK) return ig;
  if (!copy_flags_ok(a->flags))
    return fail(TPG_ERR_INVALID, "TPG_COPY_SDMA, TPG_COPY_SHADER and TPG_COPY_KERNEL are exclusive");
  if (!fits_int(a->M) || !fits_int(a->N) || !fits_int(a->K))
    return fail(TPG_ERR_UNSUPPORTED, "dimensions must be below 2^31");
  const int64_t m = a->M / a->P;
  if (m % 64) return fail(TPG_ERR_UNSUPPORTED, "M/P must be a multiple of 64");
  if (a->N % 8 || a->K % 8) return fail(TPG_ERR_UNSUPPORTED, "N and K must be multiples of 8");
  // the kernel's 31-bit offsets: 64 contraction rows of either operand plus one tile row
  if (int64_t(64) * a->N * 2 + a->N * 2 >= (int64_t(1) << 31) || int64_t(64) * a->K * 2 + a->K * 2 >= (int64_t(1) << 31))
    return fail(TPG_ERR_UNSUPPORTED, "N or K too large for the kernel's 31-bit offsets");
  if (!a->d && a->N && a->K) return fail(TPG_ERR_INVALID, "D is NULL");
  if (!aligned16(a->d)) return fail(TPG_ERR_UNSUPPORTED, "D not 16-byte aligned");
  const size_t d_b = size_t(a->N) * a->K * 2;
  std::vector<Range> inputs;
  if (a->M > 0 && a->N > 0 && a->K > 0) {
    const size_t local_b = size_t(a->M) * (a->gathered == TPG_GATHER_X ? a->N : a->K) * 2;
    if (!a->local) return fail(TPG_ERR_INVALID, "local is NULL");
    if (!aligned16(a->local)) return fail(TPG_ERR_UNSUPPORTED, "local not 16-byte aligned");
    inputs.push_back({a->local, local_b});
    if (!a->slices) return fail(TPG_ERR_INVALID, "slices is NULL");
    const size_t slice_b = wg_slice_bytes(a);
    for (int s = 0; s < a->P; ++s) {
      if (!a->slices[s]) return fail(TPG_ERR_INVALID, "NULL slice");
      if (!aligned16(a->slices[s])) return fail(TPG_ERR_UNSUPPORTED, "slice not 16-byte aligned");
      inputs.push_back({a->slices[s], slice_b});
    }
  }
  if (need && (!a->workspace || a->workspace_bytes < need))
    return fail(TPG_ERR_WORKSPACE, "workspace smaller than tpgemm_stage_wgrad_workspace_size()");
  const Range dr{a->d, d_b}, wr{a->workspace, need};
  for (const auto& r : inputs) {
    if (overlaps(dr, r)) return fail(TPG_ERR_INVALID, "D overlaps an input");
    if (overlaps(wr, r)) return fail(TPG_ERR_INVALID, "workspace overlaps an input");
  }
  if (overlaps(dr, wr)) return fail(TPG_ERR_INVALID, "workspace overlaps D");
  if (need && !aligned16(a->workspace)) return fail(TPG_ERR_UNSUPPORTED, "workspace not 16-byte aligned");
  if (wg_unstaged(a) && (a->flags & TPG_NO_COPY) && a->M > 0) {
    const size_t slice_b = wg_slice_bytes(a);
    for (int s = 1; s < a->P; ++s)
      if (static_cast<const char*>(a->slices[s]) != static_cast<const char*>(a->slices[0]) + s * slice_b)
        return fail(TPG_ERR_UNSUPPORTED, "UNSTAGED|NO_COPY needs the slices to be contiguous");
  }
  return TPG_OK;
}

// Launch chain. The local stage comes first, then the P-1 remote stages in
// `groups` runs; every launch but the last writes the fp32 partial, every
// launch but the first adds it (in place: each element is read and written
// by the same thread). Stream roles as in the all-gather: the deliveries run
// back to back on the root and the last run follows them there, after one
// wait for the chain's previous link, so the critical path (last delivery,
// then the last run) waits on no other queue; the local stage and earlier
// runs go to one side stream, each run gated by one event after its slices.
// With TPG_NO_COPY the slices are read in place, one launch per stretch that
// is contiguous in memory and does not wrap past slice P-1.
tpg_status enqueue_wg(Ctx& cx, const tpg_wg_args& a, const Launch& L) {
  const int P = a.P, r = a.rank;
  const int64_t m = a.M / P;
  const bool gx = a.gathered == TPG_GATHER_X;
  const int64_t lw = gx ? a.N : a.K;              // row width of the local operand
  const size_t slice_b = wg_slice_bytes(&a);
  const bool copies = !(a.flags & TPG_NO_COPY);
  const Copy ck = copy_of(a.flags, Copy::Kernel);
  char* ws = static_cast<char*>(a.workspace);
  float* part = wg_chain(&a) ? reinterpret_cast<float*>(ws + wg_recv(&a)) : nullptr;
  const char* loc = static_cast<const char*>(a.local);

  tpg::GemmParams p = base_params();
  p.M = static_cast<int>(a.N);
  p.N = static_cast<int>(a.K);
  p.lda = a.N;
  p.ldb = a.K;
  p.ldd = a.K;
  p.ld_acc = a.K;
  p.d = static_cast<uint16_t*>(a.d);
  p.alpha = a.alpha;
  p.beta = 0.0f;
  p.vec_ok = 1;                                   // K % 8 == 0 (validated)
  p.kwrap_rows = a.M;
  // One launch: contraction over `rows` token rows, the gathered operand's
  // rows contiguous at g, the local operand's from token row l0 on (wrapping
  // past M back to row 0).
  auto launch = [&](hipStream_t s, const void* g, int64_t l0, int64_t rows, bool first, bool last) {
    tpg::GemmParams q = p;
    q.K = static_cast<int>(rows);
    const void* lp = loc + l0 * lw * 2;
    const int wrap = l0 + rows > a.M ? static_cast<int>(a.M - l0) : 0;
    if (gx) {
      q.a = lp;
      q.b = g;
      q.a_kwrap = wrap;
    } else {
      q.a = g;
      q.b = lp;
      q.b_kwrap = wrap;
    }
    q.acc_in = first ? nullptr : part;
    q.acc_out = last ? nullptr : part;
    return gemm_on(cx, L, s, q, TPG_BF16, kLayoutAT, TPG_EPI_ALPHA_BETA);
  };
  // deliveries of stages [t_begin, t_end) into their ring-order slots on the
  // root, adjacent slices merged into one copy
  auto adjacent = [&](int s, int run) {
    for (int i = 1; i < run; ++i)
      if (static_cast<const char*>(a.slices[s + i]) != static_cast<const char*>(a.slices[s]) + i * slice_b)
        return false;
    return true;
  };

  if (wg_unstaged(&a)) {
    const void* g = a.slices[0];
    if (copies) {
      tpg_status hs = hold_deliveries(a.flags, L.root);
      if (hs != TPG_OK) return hs;
      hs = deliver_slices(ck, a.slices, P, slice_b, ws, slice_b, L.root);   // rank order
      if (hs != TPG_OK) return hs;
      g = ws;
    }
    return launch(L.root, g, 0, a.M, true, true);
  }
  if (P == 1) return launch(L.root, a.slices[0], 0, m, true, true);

  const int remote = P - 1;
  const int G = std::min(a.groups, remote);       // >= 1 here
  auto t0 = [&](int g) { return 1 + (g * remote) / G; };
  const int ns = (a.flags & TPG_SERIAL_STAGES) ? 1 : 2;
  hipStream_t st[kStreams];
  tpg_status stat = fork_streams(cx, L.root, ns, st);
  if (stat != TPG_OK) return stat;
  hipStream_t cs = st[ns - 1];                    // the chain's side stream
  stat = launch(cs, a.slices[r], r * m, m, true, false);   // the local stage: no delivery needed
  if (stat != TPG_OK) return stat;
  if (copies) {
    stat = hold_deliveries(a.flags, L.root);
    if (stat != TPG_OK) return stat;
  }
  for (int g = 0; g < G; ++g) {
    const bool last_run = g == G - 1;
    if (copies) {
      const void* src[kMaxP];
      for (int t = t0(g); t < t0(g + 1); ++t) src[t - t0(g)] = a.slices[(r + t) % P];
      stat = deliver_slices(ck, src, t0(g + 1) - t0(g), slice_b, ws + (t0(g) - 1) * slice_b, slice_b, L.root);
      if (stat != TPG_OK) return stat;
      hipStream_t rs = cs;
      if (ns > 1 && !last_run) {
        stat = dep_now(cx, cx.ev_copy[g], L.root, cs);
        if (stat != TPG_OK) return stat;
      } else if (ns > 1) {                        // the last run: on the root, after the chain's last link
        stat = dep_now(cx, cx.ev_copy[G], cs, L.root);
        if (stat != TPG_OK) return stat;
        rs = L.root;
      }
      const int s0 = (r + t0(g)) % P;
      stat = launch(rs, ws + (t0(g) - 1) * slice_b, s0 * m, (t0(g + 1) - t0(g)) * m, false, last_run);
      if (stat != TPG_OK) return stat;
    } else {
      for (int t = t0(g); t < t0(g + 1);) {
        const int s = (r + t) % P;
        int run = std::min(t0(g + 1) - t, P - s);
        while (run > 1 && !adjacent(s, run)) --run;
        const bool last = last_run && t + run == t0(g + 1);
        stat = launch(cs, a.slices[s], s * m, run * m, false, last);
        if (stat != TPG_OK) return stat;
        t += run;
      }
    }
  }
  return join_streams(cx, L.root, ns, st);
}

std::string wg_key(const tpg_wg_args& a) {
  std::ostringstream os;
  os << "wg|";
  put(os, a.M); put(os, a.N); put(os, a.K); put(os, a.P); put(os, a.rank); put(os, a.gathered);
  put(os, a.groups); put(os, a.local); put(os, a.d); put(os, a.alpha); put(os, a.flags); put(os, a.workspace);
  for (int s = 0; a.slices && s < a.P; ++s) put(os, a.slices[s]);
  return os.str();
}

// ---------------------------------------------------------------- FFN
// Two phases. (1) Per slot, pipelined over two compute streams, each with
// its own z buffer: GEMM1 writes z, the LayerNorm / SiLU pass turns it into
// the slot's h. The row pass of one slot (HBM-bound) overlaps GEMM1 of the
// next (MFMA-bound), and the two slots' z (126 MB each at the workload size)
// stay in the 256 MB Infinity Cache between GEMM1 and the row pass. (One
// batched GEMM1 over all slots was measured slower: its 1 GB z round-trips
// through HBM.) (2) GEMM2 of every slot as one batched launch over the h of
// all slots: per slot it is only PB x D output (80 tiles of 256 x 256 at the
// workload size), so slot by slot it filled a third of the chip.
// TPG_SERIAL_STAGES uses one stream and one z buffer.
int ffn_bufs(uint32_t flags) { return (flags & TPG_SERIAL_STAGES) ? 1 : 2; }

// Workspace: ffn_bufs z buffers [PB][2H], then h of every slot [L][PB][H], bf16.
size_t ffn_zbuf(const tpg_ffn_args* a) { return round_up(size_t(a->PB) * 2 * a->H * 2, 256); }

size_t ffn_ws(const tpg_ffn_args* a) {
  if (!a || a->PB < 0 || a->H < 0 || a->L < 0) return 0;
  return size_t(ffn_bufs(a->flags)) * ffn_zbuf(a) + round_up(size_t(a->L) * a->PB * a->H * 2, 256);
}

tpg_status validate_ffn(const tpg_ffn_args* a, size_t need) {
  if (!a) return fail(TPG_ERR_INVALID, "args is NULL");
  if (a->PB < 0 || a->L < 0 || a->D < 0 || a->H < 0) return fail(TPG_ERR_INVALID, "negative dimension");
  if (a->flags & ~kKnownFlags) return fail(TPG_ERR_INVALID, "unknown flag bits");
  if (tpg_status ng = validate_no_gate(a->flags, false); ng != TPG_OK) return ng;
  if (tpg_status ig = validate_in_kernel_gates(a->flags, false); ig != TPG_OK) return ig;
  if (!fits_int(a->PB) || !fits_int(a->L * a->D) || !fits_int(2 * a->H))
    return fail(TPG_ERR_UNSUPPORTED, "dimensions too large");
  if (a->D % 8 || a->H % 8) return fail(TPG_ERR_UNSUPPORTED, "D and H must be multiples of 8");
  if (a->H > 8 * 256 * 8) return fail(TPG_ERR_UNSUPPORTED, "H above 16384");
  if (!(a->eps >= 0.0f)) return fail(TPG_ERR_INVALID, "eps must be >= 0");
  const size_t PB = a->PB, L = a->L, D = a->D, H = a->H;
  const Range in[] = {{a->x, PB * L * D * 2}, {a->w1, L * D * 2 * H * 2}, {a->b1, L * 2 * H * 2},
                      {a->wout, L * H * D * 2}, {a->bout, L * D * 2}, {a->gx, H * 2},
                      {a->bx, H * 2}, {a->gg, H * 2}, {a->bg, H * 2}};
  const bool work = PB * L * D > 0;
  for (const auto& r : in) {
    if (work && r.bytes && !r.p) return fail(TPG_ERR_INVALID, "NULL FFN tensor");
    if (!aligned16(r.p)) return fail(TPG_ERR_UNSUPPORTED, "FFN tensor not 16-byte aligned");
  }
  const Range yr{a->y, PB * L * D * 2}, wr{a->workspace, need};
  if (work && !a->y) return fail(TPG_ERR_INVALID, "y is NULL");
  if (!aligned16(a->y)) return fail(TPG_ERR_UNSUPPORTED, "y not 16-byte aligned");
  if (work && need && (!a->workspace || a->workspace_bytes < need))
    return fail(TPG_ERR_WORKSPACE, "workspace smaller than ffn_slot_forward_workspace_size()");
  for (const auto& r : in) {
    if (overlaps(yr, r)) return fail(TPG_ERR_INVALID, "y overlaps an input");
    if (overlaps(wr, r)) return fail(TPG_ERR_INVALID, "workspace overlaps an input");
  }
  if (overlaps(yr, wr)) return fail(TPG_ERR_INVALID, "workspace overlaps y");
  if (work && need && (!a->workspace || a->workspace_bytes < need))
    return fail(TPG_ERR_WORKSPACE, "workspace smaller than ffn_slot_forward_workspace_size()");
  if (!aligned16(a->workspace)) return fail(TPG_ERR_UNSUPPORTED, "workspace not 16-byte aligned");
  return TPG_OK;
}

tpg_status enqueue_ffn(Ctx& cx, const tpg_ffn_args& a, const Launch& L) {
  const int64_t PB = a.PB, Ls = a.L, D = a.D, H = a.H;
  if (PB == 0 || Ls == 0 || D == 0) return TPG_OK;
  const int nb = ffn_bufs(a.flags);
  hipStream_t st[kStreams];
  tpg_status stat = fork_streams(cx, L.root, nb, st);
  if (stat != TPG_OK) return stat;
  const size_t zbuf_b = ffn_zbuf(&a);
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  const uint16_t* w1 = static_cast<const uint16_t*>(a.w1);
  const uint16_t* b1 = static_cast<const uint16_t*>(a.b1);
  const uint16_t* wo = static_cast<const uint16_t*>(a.wout);
  const uint16_t* bo = static_cast<const uint16_t*>(a.bout);
  uint16_t* y = static_cast<uint16_t*>(a.y);
  uint16_t* h_all = reinterpret_cast<uint16_t*>(static_cast<char*>(a.workspace) + nb * zbuf_b);
  // phase 1: z and h of every slot
  for (int64_t l = 0; l < Ls && H > 0; ++l) {
    hipStream_t cs = st[l % nb];
    uint16_t* z = reinterpret_cast<uint16_t*>(static_cast<char*>(a.workspace) + (l % nb) * zbuf_b);
    uint16_t* h = h_all + l * PB * H;
    tpg::GemmParams g1 = base_params();
    g1.a = x + l * D;  g1.lda = Ls * D;
    g1.b = w1 + l * D * 2 * H;  g1.ldb = 2 * H;
    g1.bias = b1 + l * 2 * H;
    g1.d = z;  g1.ldd = 2 * H;
    g1.M = static_cast<int>(PB);  g1.N = static_cast<int>(2 * H);  g1.K = static_cast<int>(D);
    g1.alpha = 1.0f;  g1.vec_ok = 1;  g1.keep_out = 1;   // z: read next by the LayerNorm pass
    stat = gemm_on(cx, L, cs, g1, tpg::kBf16, tpg::kKN, tpg::kEpiAlphaBeta);
    if (stat != TPG_OK) return stat;
    // algorithmic bytes: z (2H) in and h (H) out per row, bf16
    ProfRec rec;
    stat = prof_begin(cx, L, cs, -6.0 * double(PB) * H, rec);
    if (stat != TPG_OK) return stat;
    hipError_t e = tpg::launch_ln_silu(z, 2 * H, h, H, static_cast<int>(PB), static_cast<int>(H),
                                       static_cast<const uint16_t*>(a.gx), static_cast<const uint16_t*>(a.bx),
                                       static_cast<const uint16_t*>(a.gg), static_cast<const uint16_t*>(a.bg),
                                       a.eps, cs);
    if (e != hipSuccess) return fail(TPG_ERR_HIP, std::string("ln_silu launch failed: ") + hipGetErrorString(e));
    stat = prof_end(cx, L, cs, rec);
    if (stat != TPG_OK) return stat;
  }
  stat = join_streams(cx, L.root, nb, st);
  if (stat != TPG_OK) return stat;
  // phase 2: y[:, l, :] = h_l wout[l] + bout[l] for every slot, one batched
  // launch (blockIdx.y = slot)
  tpg::GemmParams g2 = base_params();
  g2.a = h_all;  g2.lda = H;  g2.a_bstride = PB * H;
  g2.b = wo;  g2.ldb = D;  g2.b_bstride = H * D;
  g2.bias = bo;  g2.bias_bstride = D;
  g2.d = y;  g2.ldd = Ls * D;  g2.d_bstride = D;
  g2.M = static_cast<int>(PB);  g2.N = static_cast<int>(D);  g2.K = static_cast<int>(H);
  g2.alpha = 1.0f;  g2.vec_ok = 1;
  g2.batch = static_cast<int>(Ls);      // H == 0: an empty contraction, y is the bias
  return gemm_on(cx, L, L.root, g2, tpg::kBf16, tpg::kKN, tpg::kEpiAlphaBeta);
}

std::string ffn_key(const tpg_ffn_args& a) {
  std::ostringstream os;
  os << "ffn|";
  put(os, a.PB); put(os, a.L); put(os, a.D); put(os, a.H); put(os, a.x); put(os, a.w1); put(os, a.b1);
  put(os, a.wout); put(os, a.bout); put(os, a.gx); put(os, a.bx); put(os, a.gg); put(os, a.bg);
  put(os, a.eps); put(os, a.y); put(os, a.workspace); put(os, a.flags);
  return os.str();
}

// ---------------------------------------------------------------- FFN backward
// Per slot: recompute z and h, then dh, the row backward (dz and the column
// partials), the bias reductions and the three weight / input gradient
// GEMMs, over two streams so that independent steps share the chip:
//   s0: z = GEMM1, h = ln_silu -> [h ready] -> wait dh -> rows -> [dz ready]
//       -> dw1, db1
//   s1: dh -> [dh ready] -> wait h -> dwout, dbout -> wait dz -> dx
// (dh beside GEMM1, dwout beside the row backward, dx beside dw1). h is
// double-buffered; z, dh and dz are reused in stream order (each next
// writer follows the last reader through the events above). Workspace
// layout (bytes): z [PB][2H] bf16, h [2][PB][H], dh [PB][H], dz [PB][2H],
// then fp32 partials: gamma/beta [nblk][4H], b1 [nblk][2H], bout [nblk][D].
constexpr int kBwdBlocks = 256;

struct FfnbLayout {
  size_t z, h, dh, dz, pgb, pb1, pbo, total;
};

FfnbLayout ffnb_layout(const tpg_ffnb_args* a) {
  FfnbLayout o{};
  const size_t PB = a->PB, D = a->D, H = a->H;
  size_t at = 0;
  auto take = [&](size_t bytes) {
    const size_t p = at;
    at += round_up(bytes, 256);
    return p;
  };
  o.z = take(PB * 2 * H * 2);
  o.h = take(2 * PB * H * 2);                  // two buffers: slot l uses l % 2
  o.dh = take(PB * H * 2);
  o.dz = take(PB * 2 * H * 2);
  o.pgb = take(size_t(kBwdBlocks) * 4 * H * 4);
  o.pb1 = take(size_t(kBwdBlocks) * 2 * H * 4);
  o.pbo = take(size_t(kBwdBlocks) * D * 4);
  o.total = at;
  return o;
}

size_t ffnb_ws(const tpg_ffnb_args* a) {
  if (!a || a->PB <= 0 || a->L <= 0 || a->D <= 0 || a->H <= 0) return 0;
  return ffnb_layout(a).total;
}

tpg_status validate_ffnb(const tpg_ffnb_args* a, size_t need) {
  if (!a) return fail(TPG_ERR_INVALID, "args is NULL");
  if (a->PB < 0 || a->L < 0 || a->D < 0 || a->H < 0) return fail(TPG_ERR_INVALID, "negative dimension");
  if (a->flags & ~(TPG_PROFILE | TPG_NO_GRAPH | TPG_FORCE_GRAPH | TPG_SERIAL_STAGES))
    return fail(TPG_ERR_INVALID, "unsupported flag bits");
  if (!fits_int(a->PB) || !fits_int(a->L * a->D) || !fits_int(2 * a->H))
    return fail(TPG_ERR_UNSUPPORTED, "dimensions too large");
  if (a->D % 8 || a->H % 8) return fail(TPG_ERR_UNSUPPORTED, "D and H must be multiples of 8");
  if (a->H > 8192) return fail(TPG_ERR_UNSUPPORTED, "H above 8192");
  if (a->PB % 64) return fail(TPG_ERR_UNSUPPORTED, "PB must be a multiple of 64");
  if (!(a->eps >= 0.0f)) return fail(TPG_ERR_INVALID, "eps must be >= 0");
  const size_t PB = a->PB, L = a->L, D = a->D, H = a->H;
  const bool work = PB * L * D * H > 0;
  const Range in[] = {{a->x, PB * L * D * 2}, {a->w1, L * D * 2 * H * 2}, {a->b1, L * 2 * H * 2},
                      {a->wout, L * H * D * 2}, {a->gx, H * 2}, {a->bx, H * 2}, {a->gg, H * 2},
                      {a->bg, H * 2}, {a->dy, PB * L * D * 2}};
  const Range out[] = {{a->dx, PB * L * D * 2}, {a->dw1, L * D * 2 * H * 2}, {a->db1, L * 2 * H * 2},
                       {a->dwout, L * H * D * 2}, {a->dbout, L * D * 2}, {a->dgx, H * 2},
                       {a->dbx, H * 2}, {a->dgg, H * 2}, {a->dbg, H * 2}};
  for (const auto& r : in) {
    if (work && !r.p) return fail(TPG_ERR_INVALID, "NULL FFN input");
    if (!aligned16(r.p)) return fail(TPG_ERR_UNSUPPORTED, "FFN input not 16-byte aligned");
  }
  for (const auto& r : out) {
    if (work && !r.p) return fail(TPG_ERR_INVALID, "NULL gradient output");
    if (!aligned16(r.p)) return fail(TPG_ERR_UNSUPPORTED, "gradient output not 16-byte aligned");
  }
  if (work && need && (!a->workspace || a->workspace_bytes < need))
    return fail(TPG_ERR_WORKSPACE, "workspace smaller than ffn_slot_backward_workspace_size()");
  if (!aligned16(a->workspace)) return fail(TPG_ERR_UNSUPPORTED, "workspace not 16-byte aligned");
  const Range wr{a->workspace, need};
  const int nout = sizeof(out) / sizeof(out[0]);
  for (int i = 0; i < nout; ++i) {
    for (const auto& r : in)
      if (overlaps(out[i], r)) return fail(TPG_ERR_INVALID, "a gradient output overlaps an input");
    for (int j = i + 1; j < nout; ++j)
      if (overlaps(out[i], out[j])) return fail(TPG_ERR_INVALID, "gradient outputs overlap each other");
    if (overlaps(out[i], wr)) return fail(TPG_ERR_INVALID, "workspace overlaps a gradient output");
  }
  for (const auto& r : in)
    if (overlaps(wr, r)) return fail(TPG_ERR_INVALID, "workspace overlaps an input");
  return TPG_OK;
}

tpg_status enqueue_ffnb(Ctx& cx, const tpg_ffnb_args& a, const Launch& L) {
  const int64_t PB = a.PB, Ls = a.L, D = a.D, H = a.H;
  const FfnbLayout o = ffnb_layout(&a);
  char* ws = static_cast<char*>(a.workspace);
  uint16_t* z = reinterpret_cast<uint16_t*>(ws + o.z);
  uint16_t* dh = reinterpret_cast<uint16_t*>(ws + o.dh);
  uint16_t* dz = reinterpret_cast<uint16_t*>(ws + o.dz);
  float* pgb = reinterpret_cast<float*>(ws + o.pgb);
  float* pb1 = reinterpret_cast<float*>(ws + o.pb1);
  float* pbo = reinterpret_cast<float*>(ws + o.pbo);
  auto bf = [](const void* p) { return static_cast<const uint16_t*>(p); };
  auto bfm = [](void* p) { return static_cast<uint16_t*>(p); };
  auto hip = [&](hipError_t e, const char* what) -> tpg_status {
    if (e != hipSuccess) return fail(TPG_ERR_HIP, std::string(what) + " launch failed: " + hipGetErrorString(e));
    return TPG_OK;
  };
  const int ns = (a.flags & TPG_SERIAL_STAGES) ? 1 : 2;
  hipStream_t st[kStreams];
  tpg_status fs = fork_streams(cx, L.root, ns, st);
  if (fs != TPG_OK) return fs;
  const hipStream_t s0 = st[0], s1 = st[ns - 1];
  // slot l's events: ev_copy[3 (l mod 21) + {0: h ready, 1: dh ready, 2: dz ready}]
  auto ev = [&](int64_t l, int k) { return 3 * (l % 21) + k; };
  Dep deps[63];
  auto record = [&](hipStream_t from, int e) -> tpg_status {
    if (ns > 1) return dep_mark(cx, cx.ev_copy[e], from, &deps[e]);
    return TPG_OK;
  };
  auto wait = [&](hipStream_t to, int e) -> tpg_status {
    if (ns > 1) return dep_await(to, deps[e]);
    return TPG_OK;
  };
#define TPG_STEP(expr)                 \
  do {                                 \
    tpg_status st_ = (expr);           \
    if (st_ != TPG_OK) return st_;     \
  } while (0)
  for (int64_t l = 0; l < Ls; ++l) {
    uint16_t* h = reinterpret_cast<uint16_t*>(ws + o.h) + (l % 2) * PB * H;
    // s1: dh = dY_l wout[l]^T   (wout[l] is (H, D): the (N, K) layout)
    tpg::GemmParams g2 = base_params();
    g2.a = bf(a.dy) + l * D;  g2.lda = Ls * D;
    g2.b = bf(a.wout) + l * H * D;  g2.ldb = D;
    g2.d = dh;  g2.ldd = H;
    g2.M = int(PB);  g2.N = int(H);  g2.K = int(D);
    g2.alpha = 1.0f;  g2.vec_ok = 1;  g2.keep_out = 1;   // dh: read next by the row backward
    TPG_STEP(gemm_on(cx, L, s1, g2, tpg::kBf16, tpg::kNK, tpg::kEpiAlphaBeta));
    TPG_STEP(record(s1, ev(l, 1)));
    // s0: z = X_l w1[l] + b1[l]; h = LN_x(u) silu(LN_gate(g))   (recomputed)
    tpg::GemmParams g1 = base_params();
    g1.a = bf(a.x) + l * D;  g1.lda = Ls * D;
    g1.b = bf(a.w1) + l * D * 2 * H;  g1.ldb = 2 * H;
    g1.bias = bf(a.b1) + l * 2 * H;
    g1.d = z;  g1.ldd = 2 * H;
    g1.M = int(PB);  g1.N = int(2 * H);  g1.K = int(D);
    g1.alpha = 1.0f;  g1.vec_ok = 1;  g1.keep_out = 1;   // z: read next by the LayerNorm pass
    TPG_STEP(gemm_on(cx, L, s0, g1, tpg::kBf16, tpg::kKN, tpg::kEpiAlphaBeta));
    TPG_STEP(hip(tpg::launch_ln_silu(z, 2 * H, h, H, int(PB), int(H), bf(a.gx), bf(a.bx), bf(a.gg), bf(a.bg),
                                     a.eps, s0),
                 "ln_silu"));
    TPG_STEP(record(s0, ev(l, 0)));
    // s0: dz and the column partials (needs dh), then dw1[l] = X_l^T dz and db1[l]
    TPG_STEP(wait(s0, ev(l, 1)));
    TPG_STEP(hip(tpg::launch_ffn_bwd_rows(z, 2 * H, dh, H, dz, 2 * H, int(PB), int(H), bf(a.gx), bf(a.bx),
                                          bf(a.gg), bf(a.bg), a.eps, pgb, l > 0 ? 1 : 0, pb1, kBwdBlocks, s0),
                 "ffn_bwd_rows"));
    TPG_STEP(record(s0, ev(l, 2)));
    tpg::GemmParams g4 = base_params();
    g4.a = bf(a.x) + l * D;  g4.lda = Ls * D;
    g4.b = dz;  g4.ldb = 2 * H;
    g4.d = bfm(a.dw1) + l * D * 2 * H;  g4.ldd = 2 * H;
    g4.M = int(D);  g4.N = int(2 * H);  g4.K = int(PB);
    g4.alpha = 1.0f;  g4.vec_ok = 1;
    TPG_STEP(gemm_on(cx, L, s0, g4, TPG_BF16, kLayoutAT, TPG_EPI_ALPHA_BETA));
    TPG_STEP(hip(tpg::launch_colsum_f32(pb1, kBwdBlocks, 2 * H, int(2 * H), bfm(a.db1) + l * 2 * H, s0), "colsum"));
    // s1: dwout[l] = h^T dY_l and dbout[l] (need h), then dx[:, l, :] = dz w1[l]^T (needs dz)
    TPG_STEP(wait(s1, ev(l, 0)));
    tpg::GemmParams g3 = base_params();
    g3.a = h;  g3.lda = H;
    g3.b = bf(a.dy) + l * D;  g3.ldb = Ls * D;
    g3.d = bfm(a.dwout) + l * H * D;  g3.ldd = D;
    g3.M = int(H);  g3.N = int(D);  g3.K = int(PB);
    g3.alpha = 1.0f;  g3.vec_ok = 1;
    TPG_STEP(gemm_on(cx, L, s1, g3, TPG_BF16, kLayoutAT, TPG_EPI_ALPHA_BETA));
    TPG_STEP(hip(tpg::launch_colsum_bf16(bf(a.dy) + l * D, int(PB), int(D), Ls * D, pbo, kBwdBlocks, s1), "colsum"));
    TPG_STEP(hip(tpg::launch_colsum_f32(pbo, kBwdBlocks, D, int(D), bfm(a.dbout) + l * D, s1), "colsum"));
    TPG_STEP(wait(s1, ev(l, 2)));
    tpg::GemmParams g5 = base_params();
    g5.a = dz;  g5.lda = 2 * H;
    g5.b = bf(a.w1) + l * D * 2 * H;  g5.ldb = 2 * H;
    g5.d = bfm(a.dx) + l * D;  g5.ldd = Ls * D;
    g5.M = int(PB);  g5.N = int(D);  g5.K = int(2 * H);
    g5.alpha = 1.0f;  g5.vec_ok = 1;
    TPG_STEP(gemm_on(cx, L, s1, g5, tpg::kBf16, tpg::kNK, tpg::kEpiAlphaBeta));
  }
  // the LayerNorm parameter gradients: sums over every slot's row blocks
  TPG_STEP(hip(tpg::launch_colsum_f32(pgb, kBwdBlocks, 4 * H, int(H), bfm(a.dgx), s0), "colsum"));
  TPG_STEP(hip(tpg::launch_colsum_f32(pgb + H, kBwdBlocks, 4 * H, int(H), bfm(a.dbx), s0), "colsum"));
  TPG_STEP(hip(tpg::launch_colsum_f32(pgb + 2 * H, kBwdBlocks, 4 * H, int(H), bfm(a.dgg), s0), "colsum"));
  TPG_STEP(hip(tpg::launch_colsum_f32(pgb + 3 * H, kBwdBlocks, 4 * H, int(H), bfm(a.dbg), s0), "colsum"));
#undef TPG_STEP
  return join_streams(cx, L.root, ns, st);
}

std::string ffnb_key(const tpg_ffnb_args& a) {
  std::ostringstream os;
  os << "ffnb|";
  put(os, a.PB); put(os, a.L); put(os, a.D); put(os, a.H); put(os, a.x); put(os, a.w1); put(os, a.b1);
  put(os, a.wout); put(os, a.gx); put(os, a.bx); put(os, a.gg); put(os, a.bg); put(os, a.eps); put(os, a.dy);
  put(os, a.dx); put(os, a.dw1); put(os, a.db1); put(os, a.dwout); put(os, a.dbout); put(os, a.dgx);
  put(os, a.dbx); put(os, a.dgg); put(os, a.dbg); put(os, a.workspace); put(os, a.flags);
  return os.str();
}

// ---------------------------------------------------------------- permutes
tpg_status permute_common(bool dispatch, const void* const* src, void* dst, int32_t P, int32_t rank,
                          int64_t B, int64_t T, int64_t D, int32_t eb, void* stream) {
  if (P < 1 || P > kMaxP) return fail(TPG_ERR_INVALID, "P must be in [1, 64]");
  if (rank < 0 || rank >= P) return fail(TPG_ERR_INVALID, "rank must be in [0, P)");
  if (B < 0 || T < 0 || D < 0) return fail(TPG_ERR_INVALID, "negative dimension");
  if (T % P) return fail(TPG_ERR_INVALID, "T must be a multiple of P");
  if (eb != 1 && eb != 2 && eb != 4 && eb != 8) return fail(TPG_ERR_INVALID, "elem_bytes must be 1, 2, 4 or 8");
  const int64_t L = T / P;
  const size_t total = size_t(B) * T * D * eb;     // bytes of one source (= of dst)
  if (total == 0) return TPG_OK;
  if (!src || !dst) return fail(TPG_ERR_INVALID, "NULL src or dst");
  tpg::PermuteParams p;
  std::memset(&p, 0, sizeof(p));
  const Range dr{dst, total};
  for (int s = 0; s < P; ++s) {
    if (!src[s]) return fail(TPG_ERR_INVALID, "NULL source");
    if (overlaps(dr, Range{src[s], total})) return fail(TPG_ERR_INVALID, "dst overlaps a source");
    p.src[s] = static_cast<const uint8_t*>(src[s]);
  }
  p.dst = static_cast<uint8_t*>(dst);
  p.B = B;
  p.run_bytes = L * D * eb;
  if (dispatch) {   // dst[s*B + b, l] = src_s[b, rank*L + l]
    p.src_base = rank * L * D * eb;
    p.src_bstride = T * D * eb;
    p.dst_sstride = B * L * D * eb;
    p.dst_bstride = L * D * eb;
  } else {          // dst[b, s*L + l] = src_s[rank*B + b, l]
    p.src_base = rank * B * L * D * eb;
    p.src_bstride = L * D * eb;
    p.dst_sstride = L * D * eb;
    p.dst_bstride = T * D * eb;
  }
  hipError_t e = tpg::launch_permute(p, P, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(TPG_ERR_HIP, std::string("permute launch failed: ") + hipGetErrorString(e));
  return TPG_OK;
}

template <typename F>
tpg_status guarded(F&& f) {
  try {
    g_err.clear();
    return f();
  } catch (const std::exception& ex) {
    return fail(TPG_ERR_HIP, std::string("host exception: ") + ex.what());
  } catch (...) {
    return fail(TPG_ERR_HIP, "unknown host exception");
  }
}

}  // namespace

extern "C" {

size_t tpgemm_stage_ag_workspace_size(const tpg_ag_args* args) { return ag_ws(args); }

tpg_status tpgemm_stage_ag(const tpg_ag_args* args, void* stream) {
  return guarded([&]() -> tpg_status {
    std::lock_guard<std::mutex> lk(g_mu);
    tpg_status st = validate_ag(args, ag_ws(args));
    if (st != TPG_OK) return st;
    if (args->M == 0 || args->N == 0) return TPG_OK;       // empty output: nothing to enqueue
    Ctx* cx = nullptr;
    st = get_ctx(&cx);
    if (st != TPG_OK) return st;
    tpg_ag_args a = *args;
    hipStream_t us = static_cast<hipStream_t>(stream);
    if (tpg_status gs = gates_not_captured(a.flags, us); gs != TPG_OK) return gs;
    if (auto_carried(a, us))
      a.flags |= kAutoCarried | TPG_NO_GRAPH;
    else if (!(a.flags & (TPG_UNSTAGED | TPG_DEBUG_NO_GATE | TPG_IN_KERNEL_GATES)) && a.groups == 0 &&
             2.0 * a.M * double(a.N) * a.K < kLatencyBoundFlop)
      a.flags |= TPG_SERIAL_STAGES;
    if (a.flags & TPG_IN_KERNEL_GATES) a.flags |= TPG_NO_GRAPH;   // the two launches must run concurrently
    return run_call(*cx, a.flags, ag_key(a), static_cast<hipStream_t>(stream),
                    [&](const Launch& L) { return enqueue_ag(*cx, a, L); });
  });
}

tpg_status tpgemm_stage_ag_noalloc(const tpg_ag_args* args, void* stream) {
  return guarded([&]() -> tpg_status {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!args) return fail(TPG_ERR_INVALID, "args is NULL");
    if (args->flags & (TPG_FORCE_GRAPH | TPG_PROFILE))
      return fail(TPG_ERR_UNSUPPORTED, "tpgemm_stage_ag_noalloc issues eagerly: no TPG_FORCE_GRAPH or TPG_PROFILE");
    tpg_ag_args a = *args;
    a.workspace = nullptr;                   // the receive slots are the static scratch
    a.workspace_bytes = 0;
    const size_t need = ag_ws(&a);
    if (need > tpg::kStaticScratchBytes)
      return fail(TPG_ERR_WORKSPACE, "receive slots need " + std::to_string(need) +
                                         " bytes, above the static scratch of " +
                                         std::to_string(tpg::kStaticScratchBytes) + " bytes");
    tpg_status st = validate_ag(&a, 0);      // everything but the workspace (the scratch overlaps nothing)
    if (st != TPG_OK) return st;
    if (a.M == 0 || a.N == 0) return TPG_OK;
    Ctx* cx = nullptr;
    st = get_ctx(&cx);
    if (st != TPG_OK) return st;
    HIP_TRY(tpg::static_scratch(&a.workspace));
    a.workspace_bytes = tpg::kStaticScratchBytes;
    hipStream_t us = static_cast<hipStream_t>(stream);
    if (tpg_status gs = gates_not_captured(a.flags, us); gs != TPG_OK) return gs;
    if (auto_carried(a, us))
      a.flags |= kAutoCarried;
    else if (!(a.flags & (TPG_UNSTAGED | TPG_DEBUG_NO_GATE | TPG_IN_KERNEL_GATES)) && a.groups == 0 &&
             2.0 * a.M * double(a.N) * a.K < kLatencyBoundFlop)
      a.flags |= TPG_SERIAL_STAGES;
    return run_call(*cx, a.flags | TPG_NO_GRAPH, std::string(), static_cast<hipStream_t>(stream),
                    [&](const Launch& L) { return enqueue_ag(*cx, a, L); });
  });
}

size_t tpgemm_stage_ag_multi_workspace_size(const tpg_agm_args* args) { return agm_ws(args); }

tpg_status tpgemm_stage_ag_multi(const tpg_agm_args* args, void* stream) {
  return guarded([&]() -> tpg_status {
    std::lock_guard<std::mutex> lk(g_mu);
    tpg_status st = validate_agm(args, agm_ws(args));
    if (st != TPG_OK) return st;
    if (args->M == 0 || agm_ntot(args) == 0) return TPG_OK;   // empty outputs: nothing to enqueue
    Ctx* cx = nullptr;
    st = get_ctx(&cx);
    if (st != TPG_OK) return st;
    tpg_agm_args a = *args;
    if (!(a.flags & (TPG_UNSTAGED | TPG_DEBUG_NO_GATE)) && a.groups == 0 && 2.0 * a.M * double(agm_ntot(&a)) * a.K < kLatencyBoundFlop)
      a.flags |= TPG_SERIAL_STAGES;
    return run_call(*cx, a.flags, agm_key(a), static_cast<hipStream_t>(stream),
                    [&](const Launch& L) { return enqueue_agm(*cx, a, L); });
  });
}

size_t tpgemm_stage_rs_workspace_size(const tpg_rs_args* args) { return rs_ws(args); }

tpg_status tpgemm_stage_rs(const tpg_rs_args* args, void* stream) {
  return guarded([&]() -> tpg_status {
    std::lock_guard<std::mutex> lk(g_mu);
    tpg_status st = validate_rs(args, rs_ws(args));
    if (st != TPG_OK) return st;
    if (args->M == 0 || args->N == 0) return TPG_OK;       // empty output: nothing to enqueue
    Ctx* cx = nullptr;
    st = get_ctx(&cx);
    if (st != TPG_OK) return st;
    tpg_rs_args a = *args;
    if (!(a.flags & (TPG_UNSTAGED | TPG_DEBUG_NO_GATE)) && a.groups == 0 && 2.0 * a.M * double(a.N) * a.K < kLatencyBoundFlop)
      a.flags |= TPG_SERIAL_STAGES;
    return run_call(*cx, a.flags, rs_key(a), static_cast<hipStream_t>(stream),
                    [&](const Launch& L) { return enqueue_rs(*cx, a, L); });
  });
}

size_t tpgemm_stage_wgrad_workspace_size(const tpg_wg_args* args) { return wg_ws(args); }

tpg_status tpgemm_stage_wgrad(const tpg_wg_args* args, void* stream) {
  return guarded([&]() -> tpg_status {
    std::lock_guard<std::mutex> lk(g_mu);
    tpg_status st = validate_wg(args, wg_ws(args));
    if (st != TPG_OK) return st;
    if (args->N == 0 || args->K == 0) return TPG_OK;       // empty output: nothing to enqueue
    if (args->M == 0) {                                    // an empty sum
      HIP_TRY(tpg::launch_fill_zero16(args->d, size_t(args->N) * args->K * 2, static_cast<hipStream_t>(stream)));
      return TPG_OK;
    }
    Ctx* cx = nullptr;
    st = get_ctx(&cx);
    if (st != TPG_OK) return st;
    const tpg_wg_args& a = *args;
    return run_call(*cx, a.flags, wg_key(a), static_cast<hipStream_t>(stream),
                    [&](const Launch& L) { return enqueue_wg(*cx, a, L); });
  });
}

size_t ffn_slot_backward_workspace_size(const tpg_ffnb_args* args) { return ffnb_ws(args); }

tpg_status ffn_slot_backward(const tpg_ffnb_args* args, void* stream) {
  return guarded([&]() -> tpg_status {
    std::lock_guard<std::mutex> lk(g_mu);
    tpg_status st = validate_ffnb(args, ffnb_ws(args));
    if (st != TPG_OK) return st;
    if (args->PB == 0 || args->L == 0 || args->D == 0 || args->H == 0) {
      // empty sums: every parameter gradient that has elements is zero
      const hipStream_t hs = static_cast<hipStream_t>(stream);
      const size_t L = args->L, D = args->D, H = args->H;
      const std::pair<void*, size_t> zero[] = {{args->dw1, L * D * 2 * H * 2}, {args->db1, L * 2 * H * 2},
                                               {args->dwout, L * H * D * 2}, {args->dbout, L * D * 2},
                                               {args->dgx, H * 2}, {args->dbx, H * 2}, {args->dgg, H * 2},
                                               {args->dbg, H * 2}};
      for (const auto& zb : zero)
        if (zb.first && zb.second) HIP_TRY(tpg::launch_fill_zero16(zb.first, zb.second, hs));
      return TPG_OK;
    }
    Ctx* cx = nullptr;
    st = get_ctx(&cx);
    if (st != TPG_OK) return st;
    return run_call(*cx, args->flags, ffnb_key(*args), static_cast<hipStream_t>(stream),
                    [&](const Launch& L) { return enqueue_ffnb(*cx, *args, L); });
  });
}

size_t ffn_slot_forward_workspace_size(const tpg_ffn_args* args) { return ffn_ws(args); }

tpg_status ffn_slot_forward(const tpg_ffn_args* args, void* stream) {
  return guarded([&]() -> tpg_status {
    std::lock_guard<std::mutex> lk(g_mu);
    tpg_status st = validate_ffn(args, ffn_ws(args));
    if (st != TPG_OK) return st;
    if (args->PB == 0 || args->L == 0 || args->D == 0) return TPG_OK;
    Ctx* cx = nullptr;
    st = get_ctx(&cx);
    if (st != TPG_OK) return st;
    const tpg_ffn_args a = *args;
    return run_call(*cx, a.flags, ffn_key(a), static_cast<hipStream_t>(stream),
                    [&](const Launch& L) { return enqueue_ffn(*cx, a, L); });
  });
}

tpg_status dispatch_permute(const void* const* src, void* dst, int32_t P, int32_t rank, int64_t B,
                            int64_t T, int64_t D, int32_t elem_bytes, void* stream) {
  return guarded([&]() { return permute_common(true, src, dst, P, rank, B, T, D, elem_bytes, stream); });
}

tpg_status combine_permute(const void* const* src, void* dst, int32_t P, int32_t rank, int64_t B,
                           int64_t T, int64_t D, int32_t elem_bytes, void* stream) {
  return guarded([&]() { return permute_common(false, src, dst, P, rank, B, T, D, elem_bytes, stream); });
}

tpg_status tpg_deliver(const void* const* src, int32_t n, size_t bytes, void* dst, size_t dst_stride,
                       uint32_t flags, void* stream) {
  return guarded([&]() -> tpg_status {
    if (n < 0 || n > kMaxP) return fail(TPG_ERR_INVALID, "n must be in [0, 64]");
    if (flags & ~kCopyFlags) return fail(TPG_ERR_INVALID, "only copy-kind flags apply");
    if (!copy_flags_ok(flags)) return fail(TPG_ERR_INVALID, "copy-kind flags are exclusive");
    if (n == 0 || bytes == 0) return TPG_OK;
    if (!src || !dst) return fail(TPG_ERR_INVALID, "NULL src or dst");
    if (dst_stride < bytes) return fail(TPG_ERR_INVALID, "dst_stride < bytes");
    const Range dr{dst, dst_stride * (n - 1) + bytes};
    for (int i = 0; i < n; ++i) {
      if (!src[i]) return fail(TPG_ERR_INVALID, "NULL source slice");
      if (overlaps(dr, Range{src[i], bytes})) return fail(TPG_ERR_INVALID, "dst overlaps a source");
    }
    return deliver_slices(copy_of(flags, Copy::Kernel), src, n, bytes, static_cast<char*>(dst), dst_stride,
                          static_cast<hipStream_t>(stream));
  });
}

tpg_status tpg_device_info(int32_t* cus, int32_t* clock_khz, int32_t* wall_clock_khz) {
  return guarded([&]() -> tpg_status {
    int dev = 0, v = 0;
    HIP_TRY(hipGetDevice(&dev));
    if (cus) *cus = tpg::device_cus();
    if (clock_khz) {
      HIP_TRY(hipDeviceGetAttribute(&v, hipDeviceAttributeClockRate, dev));
      *clock_khz = v;
    }
    if (wall_clock_khz) {
      HIP_TRY(hipDeviceGetAttribute(&v, hipDeviceAttributeWallClockRate, dev));
      *wall_clock_khz = v;
    }
    return TPG_OK;
  });
}

tpg_status tpg_mfma_probe(int32_t dtype, int32_t iters, int32_t blocks, uint64_t* sink, size_t sink_bytes,
                          double* flop, void* stream) {
  return guarded([&]() -> tpg_status {
    if (dtype != TPG_BF16 && dtype != TPG_E4M3) return fail(TPG_ERR_UNSUPPORTED, "mfma probe: dtype must be bf16 or e4m3");
    if (iters < 1 || iters > (1 << 24)) return fail(TPG_ERR_INVALID, "mfma probe: iters must be in [1, 2^24]");
    if (blocks < 1 || blocks > 65536) return fail(TPG_ERR_INVALID, "mfma probe: blocks must be in [1, 65536]");
    const size_t need = size_t(blocks) * (tpg::kProbeThreads / 64) * 2 * sizeof(uint64_t);
    if (!sink || sink_bytes < need) return fail(TPG_ERR_WORKSPACE, "mfma probe: sink needs " + std::to_string(need) + " bytes");
    if (reinterpret_cast<uintptr_t>(sink) % 8) return fail(TPG_ERR_UNSUPPORTED, "mfma probe: sink must be 8-byte aligned");
    if (flop) *flop = tpg::probe_flop_per_iter(dtype) * double(blocks) * iters;
    HIP_TRY(tpg::launch_mfma_probe(dtype, iters, blocks, reinterpret_cast<unsigned long long*>(sink),
                                   static_cast<hipStream_t>(stream)));
    return TPG_OK;
  });
}

const char* tpg_last_error(void) { return g_err.c_str(); }

void tpg_release_caches(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_ctx.empty()) return;
  (void)hipDeviceSynchronize();
  for (auto& kv : g_ctx) destroy_ctx(kv.second);
  g_ctx.clear();
}

int32_t tpg_profile_read(float* ms, double* flop, int32_t cap) {
  std::lock_guard<std::mutex> lk(g_mu);
  int32_t n = 0;
  for (auto& kv : g_ctx) {
    Ctx& c = *kv.second;
    for (auto& r : c.prof) {
      if (n < cap && hipEventSynchronize(r.b) == hipSuccess) {
        float t = 0.0f;
        if (hipEventElapsedTime(&t, r.a, r.b) == hipSuccess) {
          if (ms) ms[n] = t;
          if (flop) flop[n] = r.flop;
          ++n;
        }
      }
      c.prof_pool.push_back(r.a);
      c.prof_pool.push_back(r.b);
    }
    c.prof.clear();
  }
  return n;
}

}  // extern "C"
