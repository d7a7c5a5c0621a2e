// Host-side bookkeeping of the device factor cache: which span factor blocks
// sit in the cache's HBM arena, where, and which one leaves when a new block
// needs room.  Plain C++ (no HIP), so it runs and is tested without a GPU.
//
// The pages keep the factor tier in CPU memory and load a span's factors on
// expansion; they name the CPU-GPU link as the cost of that design (German
// explainer, "Technisches Resümee" > "Bedeutung und Ansprüche", limitation
// paragraph; "Methodik" part 2 for the tiering).  The cache keeps recently
// expanded spans' blocks on the GPU across decode steps and layers.
//
// Policy (slab classes with per-class LRU):
//   - The arena is cut into 2 MiB pages.  A block goes to the smallest slot
//     class that holds it; class sizes grow by about 1.25x from 1 KiB, in
//     multiples of 256 bytes, up to the largest block a span can have.
//   - A class takes a whole page when it has no free slot and unassigned pages
//     remain; pages never change class (until clear()).
//   - Otherwise the class's least recently used block is evicted, unless it
//     was already used in the current batch (one decode call): a batch's
//     blocks stay put until the batch has been read, and a block that finds
//     every slot of its class pinned that way is a bypass (read from host
//     memory directly).
//   - A hit is a block with the same key, pool offset and size; a key whose
//     offset or size changed is dropped and refilled.
#pragma once
#include <stdint.h>

#include <algorithm>
#include <unordered_map>
#include <vector>

namespace sekv {

class FactorCacheBook {
 public:
  static constexpr int64_t kPageBytes = int64_t(2) << 20;
  static constexpr int64_t kMinSlot = 1024;
  // largest block: r = L = 128, d = 128, separate bases, float32 elements
  // (128*128 + 2*128*128 + 128*128 elements), plus a 4*128-float sigma|gate entry
  static constexpr int64_t kMaxBlock = int64_t(65536) * 4 + 2048;
  enum : int32_t { kHit = 0, kFill = 1, kBypass = 2 };

  struct Stats {
    int64_t lookups = 0, hits = 0, fills = 0, bypasses = 0, evictions = 0;
    int64_t bytes_hit = 0, bytes_filled = 0, bytes_bypassed = 0;
  };

  explicit FactorCacheBook(int64_t arena_bytes) : n_pages_(std::max<int64_t>(0, arena_bytes / kPageBytes)) {
    for (int64_t s = kMinSlot;; ) {
      cls_.push_back(Cls{s});
      if (s >= kMaxBlock) break;
      const int64_t nx = std::max(s + 256, (s * 5 + 3) / 4);
      s = (nx + 255) / 256 * 256;
    }
  }

  int64_t pages() const { return n_pages_; }
  int64_t pages_used() const { return next_page_; }
  int64_t arena_bytes() const { return n_pages_ * kPageBytes; }
  int classes() const { return (int)cls_.size(); }
  int64_t class_bytes(int c) const { return cls_[c].slot; }
  int64_t resident_blocks() const { return (int64_t)map_.size(); }
  int64_t resident_bytes() const { return resident_bytes_; }
  const Stats& stats() const { return st_; }
  void reset_stats() { st_ = Stats{}; }

  // Smallest class whose slots hold `bytes`, or -1.
  int class_of(int64_t bytes) const {
    if (bytes <= 0 || bytes > cls_.back().slot) return -1;
    const auto it = std::lower_bound(cls_.begin(), cls_.end(), bytes,
                                     [](const Cls& c, int64_t b) { return c.slot < b; });
    return (int)(it - cls_.begin());
  }

  // Start a batch: blocks looked up from now on are pinned until the next begin().
  void begin() { ++epoch_; }

  // Look up one block.  Writes the slot's arena byte offset for kHit / kFill
  // (the caller copies the block there for kFill), -1 for kBypass.
  int32_t lookup(uint64_t key, int64_t bytes, int64_t tag, int64_t* offset) {
    ++st_.lookups;
    const auto it = map_.find(key);
    if (it != map_.end()) {
      Entry& e = ent_[it->second];
      if (e.tag == tag && e.bytes == bytes) {
        unlink(it->second);
        push_front(it->second);
        e.epoch = epoch_;
        ++st_.hits;
        st_.bytes_hit += bytes;
        *offset = e.off;
        return kHit;
      }
      drop(it->second);
    }
    const int c = class_of(bytes);
    int64_t slot = -1;
    if (c < 0 || !take_slot(c, &slot)) {
      ++st_.bypasses;
      st_.bytes_bypassed += bytes;
      *offset = -1;
      return kBypass;
    }
    int32_t id;
    if (!free_ent_.empty()) {
      id = free_ent_.back();
      free_ent_.pop_back();
    } else {
      id = (int32_t)ent_.size();
      ent_.emplace_back();
    }
    Entry& e = ent_[id];
    e.key = key;
    e.tag = tag;
    e.bytes = bytes;
    e.off = slot;
    e.epoch = epoch_;
    e.cls = c;
    push_front(id);
    map_.emplace(key, id);
    resident_bytes_ += bytes;
    ++st_.fills;
    st_.bytes_filled += bytes;
    *offset = slot;
    return kFill;
  }

  // Drop every block whose key's top 16 bits equal `layer` (all when layer < 0).
  void invalidate(int32_t layer) {
    std::vector<int32_t> ids;
    for (const auto& kv : map_)
      if (layer < 0 || (int32_t)(kv.first >> 48) == layer) ids.push_back(kv.second);
    std::sort(ids.begin(), ids.end());
    for (int32_t id : ids) drop(id);
  }

  // Forget everything, including which class owns which page.
  void clear() {
    map_.clear();
    ent_.clear();
    free_ent_.clear();
    for (Cls& c : cls_) c = Cls{c.slot};
    next_page_ = 0;
    resident_bytes_ = 0;
  }

  static uint64_t key(int32_t layer, int32_t group, int32_t span) {
    return ((uint64_t)(uint16_t)layer << 48) | ((uint64_t)(uint16_t)group << 32) | (uint32_t)span;
  }

 private:
  struct Entry {
    uint64_t key = 0;
    int64_t tag = 0, bytes = 0, off = 0, epoch = 0;
    int32_t cls = 0, prev = -1, next = -1;
  };
  struct Cls {
    int64_t slot;
    int32_t head = -1, tail = -1;     // most / least recently used
    std::vector<int64_t> free;        // free slot offsets, lowest last
  };

  bool take_slot(int c, int64_t* slot) {
    Cls& k = cls_[c];
    if (k.free.empty() && next_page_ < n_pages_) {
      const int64_t base = next_page_++ * kPageBytes, n = kPageBytes / k.slot;
      for (int64_t i = n - 1; i >= 0; --i) k.free.push_back(base + i * k.slot);
    }
    if (!k.free.empty()) {
      *slot = k.free.back();
      k.free.pop_back();
      return true;
    }
    if (k.tail >= 0 && ent_[k.tail].epoch != epoch_) {
      const int32_t id = k.tail;
      *slot = ent_[id].off;
      unlink(id);
      map_.erase(ent_[id].key);
      resident_bytes_ -= ent_[id].bytes;
      free_ent_.push_back(id);
      ++st_.evictions;
      return true;
    }
    return false;
  }
  void drop(int32_t id) {
    Entry& e = ent_[id];
    unlink(id);
    cls_[e.cls].free.push_back(e.off);
    map_.erase(e.key);
    resident_bytes_ -= e.bytes;
    free_ent_.push_back(id);
  }
  void unlink(int32_t id) {
    Entry& e = ent_[id];
    Cls& k = cls_[e.cls];
    if (e.prev >= 0) ent_[e.prev].next = e.next; else k.head = e.next;
    if (e.next >= 0) ent_[e.next].prev = e.prev; else k.tail = e.prev;
    e.prev = e.next = -1;
  }
  void push_front(int32_t id) {
    Entry& e = ent_[id];
    Cls& k = cls_[e.cls];
    e.prev = -1;
    e.next = k.head;
    if (k.head >= 0) ent_[k.head].prev = id; else k.tail = id;
    k.head = id;
  }

  int64_t n_pages_ = 0, next_page_ = 0, epoch_ = 0, resident_bytes_ = 0;
  std::vector<Cls> cls_;
  std::vector<Entry> ent_;
  std::vector<int32_t> free_ent_;
  std::unordered_map<uint64_t, int32_t> map_;
  Stats st_;
};

}  // namespace sekv
