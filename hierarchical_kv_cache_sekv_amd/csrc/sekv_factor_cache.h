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
// Policy (partitions of slab classes with per-class LRU):
//   - The arena is cut into 2 MiB pages, split evenly among the partitions;
//     the blocks of KV group g (b * Hkv + kv) belong to partition g mod
//     partitions, and each partition runs the rules below on its own pages.
//   - A block goes to the smallest slot
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
#include <stddef.h>
#include <stdint.h>

#include <algorithm>
#include <cstddef>
#include <vector>

namespace sekv {

// Key -> entry index, open addressing with linear probing over a power-of-two
// table kept at most half full; deletion shifts later members of the probe
// run back (no tombstones).  Keys are mixed with the 64-bit finalizer of
// MurmurHash3 before probing.
class KeyIndex {
 public:
  KeyIndex() { t_.assign(1024, Slot{}); }
  // Room for n keys without growing (the table stays at most half full).
  void reserve(size_t n) {
    size_t cap = t_.size();
    while (cap < 2 * n) cap *= 2;
    if (cap == t_.size()) return;
    std::vector<Slot> old(cap, Slot{});
    old.swap(t_);
    for (const Slot& s : old)
      if (s.val >= 0) put(s.key, s.val);
  }
  int32_t find(uint64_t k) const {
    for (uint64_t i = home(k);; i = (i + 1) & mask()) {
      if (t_[i].val < 0) return -1;
      if (t_[i].key == k) return t_[i].val;
    }
  }
  void insert(uint64_t k, int32_t v) {   // k absent
    if (2 * (n_ + 1) > t_.size()) grow();
    put(k, v);
    ++n_;
  }
  void erase(uint64_t k) {               // k present
    uint64_t i = home(k);
    while (t_[i].key != k || t_[i].val < 0) i = (i + 1) & mask();
    for (uint64_t j = i;;) {
      j = (j + 1) & mask();
      if (t_[j].val < 0) break;
      const uint64_t h = home(t_[j].key);
      // move j back to i unless its home lies cyclically in (i, j]
      const bool stays = i <= j ? (h > i && h <= j) : (h > i || h <= j);
      if (!stays) {
        t_[i] = t_[j];
        i = j;
      }
    }
    t_[i] = Slot{};
    --n_;
  }
  void clear() {
    t_.assign(1024, Slot{});
    n_ = 0;
  }
  size_t size() const { return n_; }
  template <class F> void for_each(F&& f) const {
    for (const Slot& s : t_)
      if (s.val >= 0) f(s.key, s.val);
  }

 private:
  struct Slot {
    uint64_t key = 0;
    int32_t val = -1;
  };
  uint64_t mask() const { return t_.size() - 1; }
  uint64_t home(uint64_t k) const {
    k ^= k >> 33;
    k *= 0xff51afd7ed558ccdull;
    k ^= k >> 33;
    k *= 0xc4ceb9fe1a85ec53ull;
    k ^= k >> 33;
    return k & mask();
  }
  void put(uint64_t k, int32_t v) {
    uint64_t i = home(k);
    while (t_[i].val >= 0) i = (i + 1) & mask();
    t_[i] = Slot{k, v};
  }
  void grow() {
    std::vector<Slot> old(t_.size() * 2, Slot{});
    old.swap(t_);
    for (const Slot& s : old)
      if (s.val >= 0) put(s.key, s.val);
  }
  std::vector<Slot> t_;
  size_t n_ = 0;
};

// One partition of the cache: its own pages (a fixed range of the arena),
// slot classes, LRU order and key index.
class CachePart {
 public:
  static constexpr int64_t kPageBytes = int64_t(2) << 20;
  static constexpr int64_t kMinSlot = 1024;
  // largest block: r = L = 128, d = 128, separate bases, float32 elements
  // (128*128 + 2*128*128 + 128*128 elements), plus a 4*128-float sigma|gate entry
  static constexpr int64_t kMaxBlock = int64_t(65536) * 4 + 2048;
  static constexpr int64_t kExpectBlock = 4096;
  enum : int32_t { kHit = 0, kFill = 1, kBypass = 2 };

  struct Stats {
    int64_t lookups = 0, hits = 0, fills = 0, bypasses = 0, evictions = 0;
    int64_t bytes_hit = 0, bytes_filled = 0, bytes_bypassed = 0;
  };

  CachePart(int64_t first_page, int64_t n_pages) : page0_(first_page), n_pages_(n_pages) {
    for (int64_t s = kMinSlot;; ) {
      cls_.push_back(Cls{s});
      if (s >= kMaxBlock) break;
      const int64_t nx = std::max(s + 256, (s * 5 + 3) / 4);
      s = (nx + 255) / 256 * 256;
    }
    // index and entries sized for blocks of 4 KiB and more (the smallest
    // factor block of a d = 128 span is about 2.3 KiB), so that a filling
    // cache does not rebuild its index in the middle of a call
    const size_t expect = (size_t)(n_pages * (kPageBytes / kExpectBlock));
    map_.reserve(expect);
    ent_.reserve(expect);
  }

  int64_t pages() const { return n_pages_; }
  int64_t pages_used() const { return next_page_; }
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
    const int32_t found = map_.find(key);
    if (found >= 0) {
      Entry& e = ent_[found];
      if (e.tag == tag && e.bytes() == bytes) {
        e.epoch = epoch_;
        used(e.cls(), found);
        ++st_.hits;
        st_.bytes_hit += bytes;
        *offset = e.offset();
        return kHit;
      }
      drop(found);
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
    e.epoch = epoch_;
    e.off256 = (uint32_t)(slot >> 8);
    e.meta = (uint32_t)bytes | ((uint32_t)c << 24);
    used(c, id);
    ++cls_[c].live;
    map_.insert(key, id);
    resident_bytes_ += bytes;
    ++st_.fills;
    st_.bytes_filled += bytes;
    *offset = slot;
    return kFill;
  }

  // Drop every block whose key's top 16 bits equal `layer` (all when layer < 0).
  void invalidate(int32_t layer) {
    std::vector<int32_t> ids;
    map_.for_each([&](uint64_t k, int32_t id) {
      if (layer < 0 || (int32_t)(k >> 48) == layer) ids.push_back(id);
    });
    std::sort(ids.begin(), ids.end());
    for (int32_t id : ids) drop(id);
  }

  // Forget everything, including which class owns which page.
  void clear() {
    map_.clear();
    map_.reserve((size_t)(n_pages_ * (kPageBytes / kExpectBlock)));
    ent_.clear();
    free_ent_.clear();
    for (Cls& c : cls_) c = Cls{c.slot};
    next_page_ = 0;
    resident_bytes_ = 0;
  }

 private:
  // One resident block (32 bytes).  meta: size in bytes (low 24 bits) and slot
  // class (high 8); meta 0 marks a free entry.  Slots are 256-byte aligned.
  struct Entry {
    uint64_t key = 0;
    int64_t tag = 0, epoch = 0;
    uint32_t off256 = 0, meta = 0;
    int64_t bytes() const { return meta & 0xffffff; }
    int cls() const { return (int)(meta >> 24); }
    int64_t offset() const { return (int64_t)off256 << 8; }
  };
  // A use of entry `id` in batch `ep` (low 32 bits).  Each class keeps its
  // uses in order; a use is current while the entry is live, still in this
  // class and last used in that batch, so the first current use in the queue
  // is the class's least recently used block (a call looks each key up once).
  struct Use {
    int32_t id;
    uint32_t ep;
  };
  struct Cls {
    int64_t slot;
    std::vector<int64_t> free;   // free slot offsets, lowest last
    std::vector<Use> q;          // uses, oldest first from qh
    size_t qh = 0;
    int64_t live = 0;            // resident blocks of this class
  };

  bool current(int c, const Use& u) const {
    const Entry& e = ent_[u.id];
    return e.meta != 0 && e.cls() == c && (uint32_t)e.epoch == u.ep;
  }
  void used(int c, int32_t id) {
    Cls& k = cls_[c];
    k.q.push_back(Use{id, (uint32_t)epoch_});
    if (k.q.size() - k.qh > 4 * (size_t)k.live + 4096) {
      // more stale uses than live blocks: keep the current ones, in order
      size_t w = 0;
      for (size_t r = k.qh; r < k.q.size(); ++r)
        if (current(c, k.q[r])) k.q[w++] = k.q[r];
      k.q.resize(w);
      k.qh = 0;
    } else if (k.qh > 4096 && 2 * k.qh > k.q.size()) {
      k.q.erase(k.q.begin(), k.q.begin() + (std::ptrdiff_t)k.qh);
      k.qh = 0;
    }
  }
  bool take_slot(int c, int64_t* slot) {
    Cls& k = cls_[c];
    if (k.free.empty() && next_page_ < n_pages_) {
      const int64_t base = (page0_ + next_page_++) * kPageBytes, n = kPageBytes / k.slot;
      for (int64_t i = n - 1; i >= 0; --i) k.free.push_back(base + i * k.slot);
    }
    if (!k.free.empty()) {
      *slot = k.free.back();
      k.free.pop_back();
      return true;
    }
    while (k.qh < k.q.size() && !current(c, k.q[k.qh])) ++k.qh;
    if (k.qh == k.q.size()) return false;
    const int32_t id = k.q[k.qh].id;
    if (ent_[id].epoch == epoch_) return false;   // the least recent is in this batch: all are
    ++k.qh;
    *slot = ent_[id].offset();
    release(id);
    ++st_.evictions;
    return true;
  }
  // Remove a live entry; its slot goes to the caller (release) or back to
  // its class's free list (drop).
  void release(int32_t id) {
    Entry& e = ent_[id];
    map_.erase(e.key);
    resident_bytes_ -= e.bytes();
    --cls_[e.cls()].live;
    e.meta = 0;
    free_ent_.push_back(id);
  }
  void drop(int32_t id) {
    cls_[ent_[id].cls()].free.push_back(ent_[id].offset());
    release(id);
  }

  int64_t page0_ = 0, n_pages_ = 0, next_page_ = 0, epoch_ = 0, resident_bytes_ = 0;
  std::vector<Cls> cls_;
  std::vector<Entry> ent_;
  std::vector<int32_t> free_ent_;
  KeyIndex map_;
  Stats st_;
};

// The whole cache: `parts` partitions with an even share of the pages each
// (pages [p n / parts, (p + 1) n / parts) of n); the block of KV group g
// lives in partition g mod parts.  Partitions share nothing: each one's index
// and entries stay small, and they could be looked up on different threads.
class FactorCacheBook {
 public:
  static constexpr int64_t kPageBytes = CachePart::kPageBytes;
  enum : int32_t { kHit = CachePart::kHit, kFill = CachePart::kFill, kBypass = CachePart::kBypass };
  using Stats = CachePart::Stats;

  FactorCacheBook(int64_t arena_bytes, int parts) : n_pages_(std::max<int64_t>(0, arena_bytes / kPageBytes)) {
    for (int p = 0; p < parts; ++p)
      part_.emplace_back(n_pages_ * p / parts, n_pages_ * (p + 1) / parts - n_pages_ * p / parts);
  }

  int parts() const { return (int)part_.size(); }
  CachePart& part(int p) { return part_[p]; }
  int part_of_group(int g) const { return g % (int)part_.size(); }
  int64_t pages() const { return n_pages_; }
  int64_t arena_bytes() const { return n_pages_ * kPageBytes; }
  int64_t pages_used() const { return sum([](const CachePart& p) { return p.pages_used(); }); }
  int64_t resident_blocks() const { return sum([](const CachePart& p) { return p.resident_blocks(); }); }
  int64_t resident_bytes() const { return sum([](const CachePart& p) { return p.resident_bytes(); }); }
  Stats stats() const {
    Stats t;
    for (const CachePart& p : part_) {
      const Stats& s = p.stats();
      t.lookups += s.lookups; t.hits += s.hits; t.fills += s.fills; t.bypasses += s.bypasses;
      t.evictions += s.evictions; t.bytes_hit += s.bytes_hit; t.bytes_filled += s.bytes_filled;
      t.bytes_bypassed += s.bytes_bypassed;
    }
    return t;
  }
  void reset_stats() { for (CachePart& p : part_) p.reset_stats(); }
  void begin() { for (CachePart& p : part_) p.begin(); }
  void invalidate(int32_t layer) { for (CachePart& p : part_) p.invalidate(layer); }
  void clear() { for (CachePart& p : part_) p.clear(); }

  static uint64_t key(int32_t layer, int32_t group, int32_t span) {
    return ((uint64_t)(uint16_t)layer << 48) | ((uint64_t)(uint16_t)group << 32) | (uint32_t)span;
  }

 private:
  template <class F> int64_t sum(F f) const {
    int64_t t = 0;
    for (const CachePart& p : part_) t += f(p);
    return t;
  }
  int64_t n_pages_;
  std::vector<CachePart> part_;
};

}  // namespace sekv
