// Host bookkeeping of the bounded cache: slots, static sink, rolling window,
// FIFO bank (PR-Sink) or staged evicted blocks + memory (ConvKV), the call
// order and the context of the open block.  Pure C++ (no HIP): the library
// drives it, and the CPU tests build it alone.
//
// PR-Sink (LiveAnimate page, section 方法, PR-Sink bullets): static sink =
// block 0, kept for good; rolling window = last `window` blocks; retrievable
// history = a FIFO bank of the last `bank` blocks that left the window (the
// page keeps a fixed number of blocks).  ConvKV (SoulX-LiveAct page, section
// 技术内核, ConvKV Memory bullet): window of exact KV; evicted frames feed a
// stride=kernel temporal conv whose output (memory_frames frames) is rebuilt
// at each commit from the newest kernel*memory_frames evicted frames.
//
// Reference frames (PR-Sink, ref_frames = R > 0): a permanent first segment
// (outside the slots) at temporal positions 0..R-1; generated blocks then sit
// at t0 = R + id * frames.
//
// Context-relative PR-Sink (relative = true): the context's blocks sit at
// consecutive frames in stream-id order (static, retrieved, window, current)
// after the reference; each segment gets a row range of the context-K buffer
// (ctx_off), as for ConvKV.  A retrieved block's id is known on the device
// only, so its segment carries the first position of the retrieved run and
// the device adds its rank among the selected ids.
//
// Slots: every block in the cache occupies one slot (K and V of every layer).
// A block keeps its slot until it leaves the cache, so a commit moves ids
// between lists and never copies tensor data.
//
// Pose-aware bank replacement decided on the device: a commit into a full
// bank may leave the displaced member unknown to the host for a while
// (kDisplaceDeferred).  The leaving block joins the host's bank list at once
// and the list carries one unresolved member ("ghost") until
// resolve_displaced(id) names it and frees its slot; spare slots (Shape.spare)
// let blocks open meanwhile.
#pragma once
#include <algorithm>
#include <cstdint>
#include <deque>
#include <utility>
#include <vector>

namespace bkv {

enum SegKind { SEG_STATIC = 0, SEG_DYNAMIC = 1, SEG_WINDOW = 2, SEG_CURRENT = 3, SEG_MEMORY = 4,
               SEG_REFERENCE = 5 };

struct SegPlan {
  int kind;
  int64_t id;       // block id; memory: frame index; dynamic, reference: -1
  int tokens;
  int64_t t0;       // temporal RoPE position of the segment's first frame
                    // (relative PR-Sink, dynamic: first position of the retrieved run)
  int slot;         // slot id, -1 for memory, dynamic and reference segments
  int dyn;          // dynamic: rank index into the device selection, else -1
  int ctx_off;      // ConvKV, relative PR-Sink: row offset in the context-K buffer, else 0
  int x_off;        // the same, FP8 keys: first 64-token tile exponent of the segment
};

struct ConvTap { int slot; int frame; };   // one source frame of the conv memory

class Schedule {
 public:
  struct Shape {
    bool convkv;
    int layers, frames, tokens_per_frame;   // T = frames * tokens_per_frame
    int window, statics, k, bank;
    int kernel, memory_frames;
    int ref_frames;                         // PR-Sink reference frames (0 = none)
    bool relative;                          // PR-Sink context-relative positions
    int spare = 0;                          // extra slots (deferred bank displacements)
  };
  static constexpr int kDisplaceDeferred = -2;

  explicit Schedule(const Shape& s) : s_(s) {
    T_ = s.frames * s.tokens_per_frame;
    if (s.convkv) {
      int need = s.kernel * s.memory_frames;
      staged_max_ = (need + s.frames - 1) / s.frames;
      n_slots_ = s.window + 1 + staged_max_;
    } else {
      staged_max_ = 0;
      n_slots_ = s.statics + s.window + 1 + s.bank + s.spare;
    }
    reset();
  }

  int n_slots() const { return n_slots_; }
  int staged_max() const { return staged_max_; }
  int tokens() const { return T_; }
  // Largest context the handle can see: sizes the ConvKV context-K buffer.
  int max_context_tokens() const {
    if (s_.convkv) return s_.memory_frames * s_.tokens_per_frame + (s_.window + 1) * T_;
    return ref_tokens() + (s_.statics + s_.k + s_.window + 1) * T_;
  }
  int max_segments() const {
    return s_.convkv ? s_.memory_frames + s_.window + 1
                     : (s_.ref_frames > 0) + s_.statics + s_.k + s_.window + 1;
  }
  int ref_tokens() const { return s_.convkv ? 0 : s_.ref_frames * s_.tokens_per_frame; }
  // Temporal position of block b's first frame (PR-Sink).
  int64_t block_t0(int64_t b) const { return (s_.convkv ? 0 : s_.ref_frames) + b * s_.frames; }
  // Rows of the context-K buffer (ConvKV, relative PR-Sink): the context less the reference.
  int ctx_tokens() const { return max_context_tokens() - ref_tokens(); }
  // Temporal positions a context-relative context uses: 0 .. max_context_frames()-1.
  int max_context_frames() const {
    if (s_.convkv) return s_.memory_frames + (s_.window + 1) * s_.frames;
    return s_.ref_frames + (s_.statics + s_.k + s_.window + 1) * s_.frames;
  }
  bool ctx_mode() const { return s_.convkv || s_.relative; }
  // 64-token tiles of the largest context-K buffer (FP8 keys: one exponent each per head)
  int ctx_xtiles() const {
    const int tb = (T_ + 63) / 64;
    if (s_.convkv) return s_.memory_frames * ((s_.tokens_per_frame + 63) / 64) + (s_.window + 1) * tb;
    return (s_.statics + s_.k + s_.window + 1) * tb;
  }

  void reset() {
    next_ = 0;
    open_ = false;
    cur_slot_ = -1;
    static_.clear();
    window_.clear();
    bank_.clear();
    staged_.clear();
    free_.clear();
    for (int i = n_slots_ - 1; i >= 0; --i) free_.push_back(i);   // pop_back hands out 0, 1, ...
    evicted_frames_ = 0;
    last_evicted_ = -1;
    ghosts_ = 0;
    attended_.assign(s_.layers, false);
    segs_.clear();
  }

  bool is_open() const { return open_; }
  int64_t block() const { return next_; }
  int cur_slot() const { return cur_slot_; }
  int64_t last_evicted() const { return last_evicted_; }
  const std::vector<SegPlan>& segments() const { return segs_; }
  const std::deque<std::pair<int64_t, int>>& bank() const { return bank_; }
  // members of the bank (the host's list less its unresolved displaced members)
  int bank_count() const { return (int)bank_.size() - ghosts_; }
  int unresolved() const { return ghosts_; }
  int free_slots() const { return (int)free_.size(); }
  int n_dynamic() const {
    return s_.convkv ? 0 : std::min(s_.k, bank_count());
  }
  int memory_count() const {
    if (!s_.convkv) return 0;
    int64_t m = evicted_frames_ / s_.kernel;
    return (int)std::min<int64_t>(s_.memory_frames, m);
  }
  int64_t context_tokens() const {
    int64_t n = 0;
    for (auto& g : segs_) n += g.tokens;
    return n;
  }
  bool attended(int layer) const { return attended_[layer]; }

  // Open the next block: take a free slot, lay out its context.  false if open.
  bool open() {
    if (open_ || free_.empty()) return false;
    cur_slot_ = free_.back();
    free_.pop_back();
    open_ = true;
    attended_.assign(s_.layers, false);
    build_segments();
    return true;
  }

  bool mark_attended(int layer) {
    if (!open_ || layer < 0 || layer >= s_.layers) return false;
    attended_[layer] = true;
    return true;
  }

  // The block that would leave the window at the next commit, with its slot
  // ({-1, -1} if none), and whether the bank is full.
  std::pair<int64_t, int> pending_eviction() const {
    if (!open_ || s_.convkv || (int)static_.size() < s_.statics) return {-1, -1};
    if ((int)window_.size() + 1 <= s_.window) return {-1, -1};
    return window_.front();
  }
  bool bank_full() const { return s_.bank > 0 && bank_count() == s_.bank; }

  // A deferred displacement resolved: the displaced member `id` leaves the
  // host's list and its slot is free.  false if `id` is not a member or no
  // displacement is unresolved.
  bool resolve_displaced(int64_t id) {
    if (ghosts_ == 0) return false;
    for (size_t i = 0; i < bank_.size(); ++i) {
      if (bank_[i].first == id) {
        free_.push_back(bank_[i].second);
        bank_.erase(bank_.begin() + (long)i);
        --ghosts_;
        return true;
      }
    }
    return false;
  }

  bool all_attended() const {
    for (bool a : attended_)
      if (!a) return false;
    return true;
  }

  // Close the open block.  On success fills `taps` (ConvKV: the frames the
  // memory is rebuilt from, tap order, n_mem*kernel entries; empty = none).
  // PR-Sink: `displace` >= 0 names the bank position the leaving block
  // replaces when the bank is full (pose-aware replacement); -1 = FIFO;
  // kDisplaceDeferred: it replaces a member the host learns of later.
  bool commit(std::vector<ConvTap>* taps, int displace = -1) {
    if (!open_ || !all_attended()) return false;
    taps->clear();
    const int64_t m = next_;
    last_evicted_ = -1;
    if (!s_.convkv) {
      if ((int)static_.size() < s_.statics) {
        static_.push_back({m, cur_slot_});
      } else {
        window_.push_back({m, cur_slot_});
        if ((int)window_.size() > s_.window) {
          auto e = window_.front();
          window_.pop_front();
          last_evicted_ = e.first;
          if (s_.bank > 0) {
            const bool full = bank_count() == s_.bank;
            if (displace >= 0 && displace < (int)bank_.size() && full) {
              free_.push_back(bank_[displace].second);
              bank_.erase(bank_.begin() + displace);
            } else if (displace == kDisplaceDeferred && full) {
              ++ghosts_;
            }
            bank_.push_back(e);
            if (bank_count() > s_.bank) {
              free_.push_back(bank_.front().second);
              bank_.pop_front();
            }
          } else {
            free_.push_back(e.second);
          }
        }
      }
    } else {
      window_.push_back({m, cur_slot_});
      if ((int)window_.size() > s_.window) {
        auto e = window_.front();
        window_.pop_front();
        last_evicted_ = e.first;
        staged_.push_back(e);
        evicted_frames_ += s_.frames;
        if ((int)staged_.size() > staged_max_) {
          free_.push_back(staged_.front().second);
          staged_.pop_front();
        }
        int n_mem = memory_count();
        if (n_mem > 0) {
          // newest n_mem*kernel evicted frames, oldest first
          int64_t first = evicted_frames_ - (int64_t)n_mem * s_.kernel;
          for (int64_t f = first; f < evicted_frames_; ++f) {
            int64_t b = f / s_.frames;
            int slot = -1;
            for (auto& st : staged_)
              if (st.first == b) slot = st.second;
            taps->push_back({slot, (int)(f % s_.frames)});
          }
        }
      }
    }
    open_ = false;
    cur_slot_ = -1;
    segs_.clear();
    ++next_;
    return true;
  }

 private:
  void build_segments() {
    segs_.clear();
    const int64_t m = next_;
    const int F = s_.frames;
    if (!s_.convkv && s_.relative) {
      if (s_.ref_frames > 0) segs_.push_back({SEG_REFERENCE, -1, ref_tokens(), 0, -1, -1, 0});
      int64_t t = s_.ref_frames;
      int off = 0, xo = 0;
      const int tb = (T_ + 63) / 64;
      for (auto& st : static_) {
        segs_.push_back({SEG_STATIC, st.first, T_, t, st.second, -1, off, xo});
        t += F;
        off += T_;
        xo += tb;
      }
      const int nd = n_dynamic();
      for (int j = 0; j < nd; ++j) {
        segs_.push_back({SEG_DYNAMIC, -1, T_, t, -1, j, off, xo});
        off += T_;
        xo += tb;
      }
      t += (int64_t)nd * F;
      for (auto& w : window_) {
        segs_.push_back({SEG_WINDOW, w.first, T_, t, w.second, -1, off, xo});
        t += F;
        off += T_;
        xo += tb;
      }
      segs_.push_back({SEG_CURRENT, m, T_, t, cur_slot_, -1, off, xo});
    } else if (!s_.convkv) {
      if (s_.ref_frames > 0) segs_.push_back({SEG_REFERENCE, -1, ref_tokens(), 0, -1, -1, 0});
      for (auto& st : static_) segs_.push_back({SEG_STATIC, st.first, T_, block_t0(st.first), st.second, -1, 0});
      for (int j = 0; j < n_dynamic(); ++j) segs_.push_back({SEG_DYNAMIC, -1, T_, -1, -1, j, 0});
      for (auto& w : window_) segs_.push_back({SEG_WINDOW, w.first, T_, block_t0(w.first), w.second, -1, 0});
      segs_.push_back({SEG_CURRENT, m, T_, block_t0(m), cur_slot_, -1, 0});
    } else {
      const int n_mem = memory_count();
      const int Tf = s_.tokens_per_frame;
      const int tf = (Tf + 63) / 64, tb = (T_ + 63) / 64;
      int off = 0, xo = 0;
      for (int j = 0; j < n_mem; ++j) {
        segs_.push_back({SEG_MEMORY, j, Tf, j, -1, -1, off, xo});
        off += Tf;
        xo += tf;
      }
      int64_t t = n_mem;
      for (auto& w : window_) {
        segs_.push_back({SEG_WINDOW, w.first, T_, t, w.second, -1, off, xo});
        off += T_;
        xo += tb;
        t += F;
      }
      segs_.push_back({SEG_CURRENT, m, T_, t, cur_slot_, -1, off, xo});
    }
  }

  Shape s_;
  int T_ = 0, n_slots_ = 0, staged_max_ = 0;
  int64_t next_ = 0;
  bool open_ = false;
  int cur_slot_ = -1;
  std::deque<std::pair<int64_t, int>> static_, window_, bank_, staged_;
  std::vector<int> free_;
  int ghosts_ = 0;
  int64_t evicted_frames_ = 0;
  int64_t last_evicted_ = -1;
  std::vector<bool> attended_;
  std::vector<SegPlan> segs_;
};

}  // namespace bkv
