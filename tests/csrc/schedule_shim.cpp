// Test shim: exposes the library's host state machine (schedule.hpp) through a
// tiny C interface so CPU tests can drive it without a GPU.
#include <cstdint>
#include <vector>

#include "schedule.hpp"

using bkv::Schedule;

extern "C" {

void* sched_new(int convkv, int layers, int frames, int tpf, int window, int statics, int k, int bank,
                int kernel, int memory_frames) {
  Schedule::Shape s{convkv != 0, layers, frames, tpf, window, statics, k, bank, kernel, memory_frames};
  return new Schedule(s);
}
void* sched_new_ref(int layers, int frames, int tpf, int window, int statics, int k, int bank, int ref_frames,
                    int relative) {
  Schedule::Shape s{false, layers, frames, tpf, window, statics, k, bank, 1, 0, ref_frames, relative != 0};
  return new Schedule(s);
}
// pose-aware bank decided on the device: `spare` extra slots
void* sched_new_pose(int layers, int frames, int tpf, int window, int statics, int k, int bank, int spare) {
  Schedule::Shape s{false, layers, frames, tpf, window, statics, k, bank, 1, 0, 0, false, spare};
  return new Schedule(s);
}
int sched_resolve(void* p, int64_t id) { return static_cast<Schedule*>(p)->resolve_displaced(id) ? 1 : 0; }
int sched_bank_count(void* p) { return static_cast<Schedule*>(p)->bank_count(); }
int sched_free_slots(void* p) { return static_cast<Schedule*>(p)->free_slots(); }
int sched_deferred_code() { return Schedule::kDisplaceDeferred; }
// commit with the bank position the leaving block displaces (-1: FIFO)
int sched_commit_displace(void* p, int displace) {
  std::vector<bkv::ConvTap> taps;
  return static_cast<Schedule*>(p)->commit(&taps, displace) ? 1 : 0;
}
int64_t sched_pending(void* p) { return static_cast<Schedule*>(p)->pending_eviction().first; }
int sched_bank_full(void* p) { return static_cast<Schedule*>(p)->bank_full() ? 1 : 0; }
void sched_free(void* p) { delete static_cast<Schedule*>(p); }
int sched_n_slots(void* p) { return static_cast<Schedule*>(p)->n_slots(); }
int sched_open(void* p) { return static_cast<Schedule*>(p)->open() ? 1 : 0; }
int sched_mark(void* p, int layer) { return static_cast<Schedule*>(p)->mark_attended(layer) ? 1 : 0; }
int sched_cur_slot(void* p) { return static_cast<Schedule*>(p)->cur_slot(); }
int64_t sched_last_evicted(void* p) { return static_cast<Schedule*>(p)->last_evicted(); }
int sched_memory_count(void* p) { return static_cast<Schedule*>(p)->memory_count(); }
int sched_n_dynamic(void* p) { return static_cast<Schedule*>(p)->n_dynamic(); }

int sched_commit(void* p, int* tap_slot, int* tap_frame, int cap, int* ntaps) {
  std::vector<bkv::ConvTap> taps;
  if (!static_cast<Schedule*>(p)->commit(&taps)) return 0;
  *ntaps = (int)taps.size();
  for (int i = 0; i < (int)taps.size() && i < cap; ++i) {
    tap_slot[i] = taps[i].slot;
    tap_frame[i] = taps[i].frame;
  }
  return 1;
}

// rows of 7 int64: kind, id, tokens, t0, slot, dyn, ctx_off
int sched_segments(void* p, int64_t* out, int cap) {
  const auto& s = static_cast<Schedule*>(p)->segments();
  for (int i = 0; i < (int)s.size() && i < cap; ++i) {
    int64_t* r = out + 7 * i;
    r[0] = s[i].kind; r[1] = s[i].id; r[2] = s[i].tokens; r[3] = s[i].t0;
    r[4] = s[i].slot; r[5] = s[i].dyn; r[6] = s[i].ctx_off;
  }
  return (int)s.size();
}

int sched_bank(void* p, int64_t* ids, int* slots, int cap) {
  const auto& b = static_cast<Schedule*>(p)->bank();
  for (int i = 0; i < (int)b.size() && i < cap; ++i) {
    ids[i] = b[i].first;
    slots[i] = b[i].second;
  }
  return (int)b.size();
}
}
