// Replay buffer of the distillation ("Flux2TTRTrainer", section "How the
// distillation works": samples keep full keys and values but subsampled
// queries, offloaded to CPU memory within a budget, 768 MB by default).
//
// A FIFO of samples in one ring of pinned host memory. The budget counts the
// samples' footprints (each stored array rounded up to 256 bytes); the ring
// holds budget + max_sample bytes. With that slack a contiguous placement at
// the ring's tail (or, after a wrap, at its start) always exists once the
// oldest samples have been evicted down to the budget:
//   not wrapped, live [h, t): if the tail gap is too small, t > ring - s >= budget
//     while t - h <= budget - s, so h > s and the sample fits at 0;
//   wrapped, live [h, e) + [0, t): e > ring - max_sample >= budget (the wrap
//     happened because the gap after e was too small), so the free span
//     h - t = e - used > budget - (budget - s) = s.
// Hence the samples held are exactly the longest run of recent pushes that
// fits the budget, and placement never evicts beyond the budget rule.
//
// Device->host copies run on the object's own side stream: a gather kernel
// packs the query and teacher rows into a device staging area (reading the
// indices from the ring through its device mapping), then DMA copies move
// the rows, K and V into the ring. Host->device copies (fetch) are DMA
// on the caller's stream.
// Per sample, one event marks its push complete and one its last fetch; ring
// space is reused only after both have completed.
#include <hip/hip_runtime.h>

#include <cstring>
#include <deque>
#include <mutex>
#include <vector>

#include "../../include/ttr.h"
#include "launch.hpp"
#include "validate.hpp"

using namespace ttr;

namespace {

constexpr size_t kAlign = 256;

size_t round_up(size_t n) { return (n + kAlign - 1) / kAlign * kAlign; }

struct Parts {  // byte sizes (unrounded) of one sample's arrays
  size_t kv, q, t, idx;
  size_t foot() const { return 2 * round_up(kv) + round_up(q) + round_up(t) + round_up(idx); }
};

Parts parts_of(const ttr_dims& d, int32_t Nq, bool teacher) {
  const size_t io = dtype_bytes(d.dtype), slices = (size_t)d.B * d.H;
  Parts p;
  p.kv = slices * d.N * d.D * io;
  p.q = slices * Nq * d.D * io;
  p.t = teacher ? slices * Nq * d.D * sizeof(float) : 0;
  p.idx = (size_t)Nq * sizeof(int32_t);
  return p;
}

// Sample dims with F taken as D (the identity feature map's rule).
ttr_status check_sample_dims(ttr_dims d, int32_t Nq) {
  d.F = d.D;
  d.fmap = TTR_FMAP_ELU1;
  const ttr_status st = check_dims(d, false);
  if (st != TTR_OK) return st;
  if (Nq < 1 || Nq > d.N) return TTR_ERR_SHAPE;
  return TTR_OK;
}

struct Sample {
  int64_t id;
  size_t off, foot;
  ttr_dims d;
  int32_t Nq;
  bool teacher;
  Parts parts;
  hipEvent_t done;       // recorded on the side stream after the push's copies
  hipEvent_t read;       // recorded on a fetch stream after its copies
  bool read_recorded;
  size_t off_k() const { return off; }
  size_t off_v() const { return off + round_up(parts.kv); }
  size_t off_q() const { return off + 2 * round_up(parts.kv); }
  size_t off_t() const { return off_q() + round_up(parts.q); }
  size_t off_i() const { return off_t() + round_up(parts.t); }
};

}  // namespace

struct ttr_replay {
  std::mutex mu;
  int device = 0;
  size_t budget = 0, max_sample = 0, ring = 0;
  uint8_t* host = nullptr;     // pinned ring
  uint8_t* mapped = nullptr;   // the ring's device address
  uint8_t* staging = nullptr;  // device, max_sample bytes: a push's gathered rows
  hipStream_t side = nullptr;
  hipEvent_t inputs_ready = nullptr;  // caller stream -> side stream
  hipEvent_t last_push = nullptr;     // side stream, after the latest push
  std::vector<hipEvent_t> events;     // pool of per-sample events not in use
  bool any_push = false;
  std::deque<Sample> live;
  size_t used = 0;
  int64_t next_id = 0, evicted = 0;
};

namespace {

ttr_status check_device(const ttr_replay* rb) {
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess || cur != rb->device) return TTR_ERR_DEVICE;
  return TTR_OK;
}

hipError_t take_event(ttr_replay* rb, hipEvent_t* ev) {
  if (!rb->events.empty()) {
    *ev = rb->events.back();
    rb->events.pop_back();
    return hipSuccess;
  }
  return hipEventCreateWithFlags(ev, hipEventDisableTiming);
}

// Wait until no copy touches the sample's ring bytes, then return its events to the pool.
hipError_t retire(ttr_replay* rb, Sample& s) {
  hipError_t e = hipEventSynchronize(s.done);
  if (e == hipSuccess && s.read_recorded) e = hipEventSynchronize(s.read);
  rb->events.push_back(s.done);
  rb->events.push_back(s.read);
  return e;
}

// Offset for a new sample of `foot` bytes (the caller evicted down to the budget).
bool place(const ttr_replay* rb, size_t foot, size_t* off) {
  if (rb->live.empty()) {
    *off = 0;
    return foot <= rb->ring;
  }
  const size_t h = rb->live.front().off, t = rb->live.back().off + rb->live.back().foot;
  if (rb->live.back().off >= h) {  // not wrapped: free [t, ring) and [0, h)
    if (rb->ring - t >= foot) {
      *off = t;
      return true;
    }
    *off = 0;
    return h >= foot;
  }
  *off = t;  // wrapped: free [t, h)
  return h - t >= foot;
}

Sample* find(ttr_replay* rb, int64_t id) {
  if (rb->live.empty()) return nullptr;
  const int64_t first = rb->live.front().id;
  if (id < first || id >= first + (int64_t)rb->live.size()) return nullptr;
  return &rb->live[(size_t)(id - first)];  // ids held are consecutive
}

}  // namespace

extern "C" {

size_t ttr_replay_sample_bytes(ttr_dims d, int32_t Nq, int32_t with_teacher) {
  if (check_sample_dims(d, Nq) != TTR_OK) return 0;
  return parts_of(d, Nq, with_teacher != 0).foot();
}

ttr_status ttr_replay_create(size_t budget_bytes, size_t max_sample_bytes, ttr_replay** out) {
  if (out == nullptr) return TTR_ERR_NULL;
  *out = nullptr;
  if (budget_bytes < kAlign || max_sample_bytes < kAlign || max_sample_bytes > budget_bytes) return TTR_ERR_SHAPE;
  ttr_replay* rb = new ttr_replay();
  rb->budget = budget_bytes;
  rb->max_sample = round_up(max_sample_bytes);
  rb->ring = round_up(budget_bytes) + rb->max_sample;
  hipError_t e = hipGetDevice(&rb->device);
  void* host = nullptr;
  if (e == hipSuccess) e = hipHostMalloc(&host, rb->ring, hipHostMallocDefault);
  rb->host = static_cast<uint8_t*>(host);
  void* mapped = nullptr;
  if (e == hipSuccess) e = hipHostGetDevicePointer(&mapped, host, 0);
  rb->mapped = static_cast<uint8_t*>(mapped);
  void* staging = nullptr;
  if (e == hipSuccess) e = hipMalloc(&staging, rb->max_sample);
  rb->staging = static_cast<uint8_t*>(staging);
  if (e == hipSuccess) e = hipStreamCreateWithFlags(&rb->side, hipStreamNonBlocking);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&rb->inputs_ready, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&rb->last_push, hipEventDisableTiming);
  if (e != hipSuccess) {
    ttr_replay_destroy(rb);
    return report_hip(e);
  }
  *out = rb;
  return TTR_OK;
}

void ttr_replay_destroy(ttr_replay* rb) {
  if (rb == nullptr) return;
  if (rb->side != nullptr) (void)hipStreamSynchronize(rb->side);
  for (Sample& s : rb->live) (void)retire(rb, s);
  rb->live.clear();
  for (hipEvent_t ev : rb->events) (void)hipEventDestroy(ev);
  if (rb->inputs_ready != nullptr) (void)hipEventDestroy(rb->inputs_ready);
  if (rb->last_push != nullptr) (void)hipEventDestroy(rb->last_push);
  if (rb->side != nullptr) (void)hipStreamDestroy(rb->side);
  if (rb->host != nullptr) (void)hipHostFree(rb->host);
  if (rb->staging != nullptr) (void)hipFree(rb->staging);
  delete rb;
}

ttr_status ttr_replay_push(ttr_replay* rb, ttr_dims d, int32_t Nq, const void* Q, const void* K, const void* V,
                           const float* teacher, const int32_t* q_index, void* stream, int64_t* id_out) {
  if (rb == nullptr || q_index == nullptr || id_out == nullptr) return TTR_ERR_NULL;
  const ttr_status ds = check_sample_dims(d, Nq);
  if (ds != TTR_OK) return ds;
  for (const void* p : {Q, K, V}) {
    const ttr_status st = check_ptr(p);
    if (st != TTR_OK) return st;
  }
  const ttr_status ts = check_opt_ptr(teacher);
  if (ts != TTR_OK) return ts;
  if (q_index[0] < 0 || q_index[Nq - 1] >= d.N) return TTR_ERR_SHAPE;
  for (int32_t i = 1; i < Nq; ++i)
    if (q_index[i] <= q_index[i - 1]) return TTR_ERR_SHAPE;
  d.F = d.D;
  const Parts parts = parts_of(d, Nq, teacher != nullptr);
  const size_t foot = parts.foot();

  std::lock_guard<std::mutex> lock(rb->mu);
  const ttr_status dev = check_device(rb);
  if (dev != TTR_OK) return dev;
  if (foot > rb->budget || foot > rb->max_sample) return TTR_ERR_BUDGET;
  while (!rb->live.empty() && rb->used + foot > rb->budget) {
    Sample& old = rb->live.front();
    const hipError_t e = retire(rb, old);
    rb->used -= old.foot;
    rb->live.pop_front();
    ++rb->evicted;
    if (e != hipSuccess) return report_hip(e);
  }
  Sample s{};
  if (!place(rb, foot, &s.off)) return TTR_ERR_BUDGET;  // unreachable for foot <= max_sample (see above)
  s.id = rb->next_id;
  s.foot = foot;
  s.d = d;
  s.Nq = Nq;
  s.teacher = teacher != nullptr;
  s.parts = parts;
  std::memcpy(rb->host + s.off_i(), q_index, parts.idx);

  hipStream_t caller = static_cast<hipStream_t>(stream);
  hipError_t e = take_event(rb, &s.done);
  if (e == hipSuccess) e = take_event(rb, &s.read);
  if (e == hipSuccess) e = hipEventRecord(rb->inputs_ready, caller);
  if (e == hipSuccess) e = hipStreamWaitEvent(rb->side, rb->inputs_ready, 0);
  StageTimer timer = take_stage_timer(rb->side);  // optional events around the copies
  // staging (device): [Q rows | T rows], laid out like the sample's rows in the ring; the
  // kernel reads the indices from the ring through its device mapping (a few KB)
  uint8_t* st_q = rb->staging;
  uint8_t* st_t = st_q + round_up(parts.q);
  const size_t rows_bytes = teacher != nullptr ? round_up(parts.q) + parts.t : parts.q;
  if (e == hipSuccess)
    e = launch_replay_gather(Q, st_q, d.D * (int)dtype_bytes(d.dtype), teacher, st_t, d.D * (int)sizeof(float),
                             reinterpret_cast<const int32_t*>(rb->mapped + s.off_i()), d.B * d.H, d.N, Nq,
                             rb->side);
  timer.mark();
  if (e == hipSuccess) e = hipMemcpyAsync(rb->host + s.off_q(), st_q, rows_bytes, hipMemcpyDeviceToHost, rb->side);
  timer.mark();
  if (e == hipSuccess) e = hipMemcpyAsync(rb->host + s.off_k(), K, parts.kv, hipMemcpyDeviceToHost, rb->side);
  timer.mark();
  if (e == hipSuccess) e = hipMemcpyAsync(rb->host + s.off_v(), V, parts.kv, hipMemcpyDeviceToHost, rb->side);
  timer.finish();
  if (e == hipSuccess) e = hipEventRecord(s.done, rb->side);
  if (e == hipSuccess) e = hipEventRecord(rb->last_push, rb->side);
  if (e != hipSuccess) {
    // the sample is not kept; copies already enqueued finish before its bytes are reused
    (void)hipStreamSynchronize(rb->side);
    if (s.done != nullptr) rb->events.push_back(s.done);
    if (s.read != nullptr) rb->events.push_back(s.read);
    return report_hip(e);
  }
  rb->any_push = true;
  rb->used += foot;
  rb->live.push_back(s);
  *id_out = rb->next_id++;
  return TTR_OK;
}

ttr_status ttr_replay_wait_pushed(ttr_replay* rb, void* stream) {
  if (rb == nullptr) return TTR_ERR_NULL;
  std::lock_guard<std::mutex> lock(rb->mu);
  const ttr_status dev = check_device(rb);
  if (dev != TTR_OK) return dev;
  if (!rb->any_push) return TTR_OK;
  const hipError_t e = hipStreamWaitEvent(static_cast<hipStream_t>(stream), rb->last_push, 0);
  return e == hipSuccess ? TTR_OK : report_hip(e);
}

ttr_status ttr_replay_synchronize(ttr_replay* rb) {
  if (rb == nullptr) return TTR_ERR_NULL;
  std::lock_guard<std::mutex> lock(rb->mu);
  const ttr_status dev = check_device(rb);
  if (dev != TTR_OK) return dev;
  const hipError_t e = hipStreamSynchronize(rb->side);
  return e == hipSuccess ? TTR_OK : report_hip(e);
}

ttr_status ttr_replay_fetch(ttr_replay* rb, int64_t id, void* Qs, void* K, void* V, float* teacher_rows,
                            int32_t* q_index, void* stream) {
  if (rb == nullptr) return TTR_ERR_NULL;
  for (const void* p : {Qs, K, V}) {
    const ttr_status st = check_ptr(p);
    if (st != TTR_OK) return st;
  }
  const ttr_status ts = check_opt_ptr(teacher_rows);
  if (ts != TTR_OK) return ts;
  std::lock_guard<std::mutex> lock(rb->mu);
  const ttr_status dev = check_device(rb);
  if (dev != TTR_OK) return dev;
  Sample* s = find(rb, id);
  if (s == nullptr) return TTR_ERR_NOT_FOUND;
  if (teacher_rows != nullptr && !s->teacher) return TTR_ERR_SHAPE;
  const Range outs[] = {{Qs, s->parts.q}, {K, s->parts.kv}, {V, s->parts.kv},
                        {teacher_rows, teacher_rows ? s->parts.t : 0}};
  const ttr_status al = check_no_alias(outs, 4, nullptr, 0);
  if (al != TTR_OK) return al;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = hipStreamWaitEvent(st, s->done, 0);
  if (e == hipSuccess) e = hipMemcpyAsync(K, rb->host + s->off_k(), s->parts.kv, hipMemcpyHostToDevice, st);
  if (e == hipSuccess) e = hipMemcpyAsync(V, rb->host + s->off_v(), s->parts.kv, hipMemcpyHostToDevice, st);
  if (e == hipSuccess) e = hipMemcpyAsync(Qs, rb->host + s->off_q(), s->parts.q, hipMemcpyHostToDevice, st);
  if (e == hipSuccess && teacher_rows != nullptr)
    e = hipMemcpyAsync(teacher_rows, rb->host + s->off_t(), s->parts.t, hipMemcpyHostToDevice, st);
  // The sample keeps one read event. A fetch on another stream than the last
  // one's would otherwise replace it: the stream first waits for the earlier
  // record (after its own copies are enqueued, so they are not delayed), and
  // the new record then stands for every fetch so far.
  if (e == hipSuccess && s->read_recorded) e = hipStreamWaitEvent(st, s->read, 0);
  // recorded even after a failed copy so that reuse of the ring space waits for what was enqueued
  const hipError_t er = hipEventRecord(s->read, st);
  if (er == hipSuccess) s->read_recorded = true;
  if (e == hipSuccess) e = er;
  if (e != hipSuccess) return report_hip(e);
  if (q_index != nullptr) std::memcpy(q_index, rb->host + s->off_i(), s->parts.idx);
  return TTR_OK;
}

ttr_status ttr_replay_info(ttr_replay* rb, int64_t id, ttr_dims* d, int32_t* Nq, int32_t* has_teacher) {
  if (rb == nullptr) return TTR_ERR_NULL;
  std::lock_guard<std::mutex> lock(rb->mu);
  const Sample* s = find(rb, id);
  if (s == nullptr) return TTR_ERR_NOT_FOUND;
  if (d != nullptr) *d = s->d;
  if (Nq != nullptr) *Nq = s->Nq;
  if (has_teacher != nullptr) *has_teacher = s->teacher ? 1 : 0;
  return TTR_OK;
}

ttr_status ttr_replay_get_stats(ttr_replay* rb, ttr_replay_stats* out) {
  if (rb == nullptr || out == nullptr) return TTR_ERR_NULL;
  std::lock_guard<std::mutex> lock(rb->mu);
  out->count = (int32_t)rb->live.size();
  out->first_id = rb->live.empty() ? -1 : rb->live.front().id;
  out->pushed = rb->next_id;
  out->evicted = rb->evicted;
  out->bytes_used = rb->used;
  out->budget_bytes = rb->budget;
  out->max_sample_bytes = rb->max_sample;
  out->ring_bytes = rb->ring;
  return TTR_OK;
}

}  // extern "C"
