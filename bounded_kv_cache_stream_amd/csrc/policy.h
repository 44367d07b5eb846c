// Host-side cache policy of one layer: keyframe rule, page allocation,
// sliding-window eviction, application of compaction results, and the merge
// of ragged pages.
//
// Pages: GCTStream explainer ("KV Cache Lifecycle Management": skip-append of
// non-keyframes; "Sliding Window Eviction": the oldest blocks go once the
// cache is over the window; "Special Token Persistence": special tokens
// survive the eviction of their frame); LingBot-Map 20 FPS explainer
// ("Sliding-Window Eviction Strategy": the window counts frames, the first
// scale frames are kept).  Readings: the window counts persisted non-scale
// frames; frame t is a keyframe iff t < S or (t - S) % k == 0; page ids come
// from a per-layer pool, lowest free id first; a frame's page is allocated
// before the eviction of the same frame; freed ids are free at once.  Special
// tokens are a frame's first slots; at each eviction (oldest victim first)
// they go to the end of the last special page, a new one being taken (lowest
// free id, the victim still holding its own) when they do not fit; special
// pages sit after the scale frames and count as no frame of the window.
#pragma once

#include <stdint.h>

#include <map>
#include <set>
#include <vector>

namespace kvs {

struct PageEntry {
  int32_t page;   // layer-local page id
  int32_t len;    // valid tokens in the page (the largest head length when heads differ)
  int64_t frame;  // frame index (of the first frame a merged page holds)
  std::vector<int32_t> hlen;  // per-head lengths once heads keep different tokens; empty: every head holds len
  bool special = false;       // holds the special tokens of evicted frames (frame = the first of them)
};

inline int32_t head_len(const PageEntry& e, int h) { return e.hlen.empty() ? e.len : e.hlen[(size_t)h]; }

// One page merge: the `count` tokens of page `src` go to slots
// dst_off .. dst_off + count - 1 of page `dst`.
struct MergeMove {
  int32_t src, dst, dst_off, count;
};

// One per-head page merge: rows 0 .. count[h]-1 of head h of page src go to
// slots dst_off[h] .. of head h of page dst.
struct HeadMergeMove {
  int32_t src, dst;
  std::vector<int32_t> dst_off, count;
};

class LayerPolicy {
 public:
  void init(int32_t pages, int32_t scale_frames, int32_t window, int32_t keyframe_interval, int32_t page_tokens,
            int32_t special_tokens) {
    pages_ = pages;
    S_ = scale_frames;
    W_ = window;
    k_ = keyframe_interval;
    T_ = page_tokens;
    SP_ = special_tokens;
    reset();
  }

  void reset() {
    ++gen;
    table.clear();
    free_ids.clear();
    for (int32_t i = 0; i < pages_; ++i) free_ids.insert(i);
    transient_pending = false;
    transient_frame = -1;
    last_frame = -1;
    evictions = 0;
    compactions = 0;
    last_keep = 0;
    merges = 0;
    prunes = 0;
  }

  bool is_keyframe(int64_t t) const { return t < S_ || (t - S_) % k_ == 0; }

  // Page that frame t would go to: a fresh page id, or -1 for the transient
  // page.  Returns 0 on success, else an error code (1 order, 2 no page).
  int plan_append(int64_t t, bool force_transient, int32_t* page) const {
    if (t <= last_frame || transient_pending) return 1;
    if (force_transient || !is_keyframe(t)) {
      *page = -1;
      return 0;
    }
    if (free_ids.empty()) return 2;
    *page = *free_ids.begin();
    return 0;
  }

  void commit_append(int64_t t, int32_t page) {
    last_frame = t;
    if (page < 0) {
      transient_pending = true;
      transient_frame = t;
      return;
    }
    free_ids.erase(page);
    table.push_back(PageEntry{page, T_, t, {}, false});
    ++gen;
  }

  bool is_window_frame(const PageEntry& e) const { return e.frame >= S_ && !e.special; }

  // Window eviction.  With special tokens on, each victim's first SP_ rows go
  // to the last special page (the copies are returned for the device); a
  // special page that cannot be had leaves everything unchanged and returns
  // -1.  Otherwise returns the number of frames evicted.
  int32_t evict(std::vector<MergeMove>* copies) {
    if (W_ <= 0) return 0;
    if (SP_ == 0) {  // no special tokens: whole pages go, nothing can fail, edit in place
      int32_t n = 0;
      for (;;) {
        int32_t nonscale = 0;
        for (const auto& e : table)
          if (is_window_frame(e)) ++nonscale;
        if (nonscale <= W_) break;
        size_t idx = 0;
        while (!is_window_frame(table[idx])) ++idx;
        free_ids.insert(table[idx].page);
        table.erase(table.begin() + (long)idx);
        ++n;
      }
      evictions += n;
      if (n) ++gen;
      if (copies) copies->clear();
      return n;
    }
    std::vector<PageEntry> tab = table;
    std::set<int32_t> free_set = free_ids;
    std::vector<MergeMove> mv;
    int32_t n = 0;
    for (;;) {
      int32_t nonscale = 0;
      for (const auto& e : tab)
        if (is_window_frame(e)) ++nonscale;
      if (nonscale <= W_) break;
      size_t idx = 0;
      while (!is_window_frame(tab[idx])) ++idx;
      const PageEntry victim = tab[idx];
      if (SP_ > 0) {
        // the special block follows the scale frames
        size_t end = 0;
        while (end < tab.size() && !is_window_frame(tab[end])) ++end;
        size_t last = end;
        for (size_t i = 0; i < end; ++i)
          if (tab[i].special) last = i;
        if (last == end || tab[last].len + SP_ > T_) {
          if (free_set.empty()) return -1;
          const int32_t id = *free_set.begin();
          free_set.erase(free_set.begin());
          tab.insert(tab.begin() + (long)end, PageEntry{id, 0, victim.frame, {}, true});
          last = end;
          ++idx;
        }
        mv.push_back(MergeMove{victim.page, tab[last].page, tab[last].len, SP_});
        tab[last].len += SP_;
      }
      free_set.insert(victim.page);
      tab.erase(tab.begin() + (long)idx);
      ++n;
    }
    table.swap(tab);
    free_ids.swap(free_set);
    evictions += n;
    if (n) ++gen;
    if (copies) *copies = mv;
    return n;
  }

  int32_t special_pages() const {
    int32_t n = 0;
    for (const auto& e : table) n += e.special;
    return n;
  }

  int64_t special_tokens() const {
    int64_t n = 0;
    for (const auto& e : table)
      if (e.special) n += e.len;
    return n;
  }

  // Index of the first table entry that is neither a scale frame nor a
  // special page (those lead the table).
  size_t first_candidate() const {
    size_t i = 0;
    while (i < table.size() && !is_window_frame(table[i])) ++i;
    return i;
  }

  // New lengths for entries first_candidate().. (same count); empty pages
  // leave the table and their ids are freed.
  void apply_compaction(const std::vector<int32_t>& new_lens, int64_t kept) {
    size_t f = first_candidate();
    std::vector<PageEntry> out(table.begin(), table.begin() + (long)f);
    for (size_t i = f; i < table.size(); ++i) {
      PageEntry e = table[i];
      e.len = new_lens[i - f];
      e.hlen.clear();
      if (e.len == 0)
        free_ids.insert(e.page);
      else
        out.push_back(e);
    }
    table.swap(out);
    ++compactions;
    last_keep = kept;
    ++gen;
  }

  // Page merge (defragmentation of the ragged pages compaction leaves): walk
  // the table in order from the first non-scale entry; a page whose length
  // fits after the page before it (sum <= page_tokens) is appended to it.
  // Returns the moves; the table is unchanged until commit_merges.
  std::vector<MergeMove> plan_merges() const {
    std::vector<MergeMove> mv;
    size_t f = first_candidate();
    if (f >= table.size()) return mv;
    int32_t cur = table[f].page, cur_len = table[f].len;
    for (size_t i = f + 1; i < table.size(); ++i) {
      if (cur_len + table[i].len <= T_) {
        mv.push_back(MergeMove{table[i].page, cur, cur_len, table[i].len});
        cur_len += table[i].len;
      } else {
        cur = table[i].page;
        cur_len = table[i].len;
      }
    }
    return mv;
  }

  void commit_merges(const std::vector<MergeMove>& mv) {
    std::set<int32_t> gone;
    std::map<int32_t, int32_t> grow;
    for (const auto& m : mv) {
      gone.insert(m.src);
      grow[m.dst] += m.count;
    }
    std::vector<PageEntry> out;
    for (const auto& e0 : table) {
      if (gone.count(e0.page)) {
        free_ids.insert(e0.page);
        continue;
      }
      PageEntry e = e0;
      auto it = grow.find(e.page);
      if (it != grow.end()) e.len += it->second;
      out.push_back(e);
    }
    table.swap(out);
    merges += (int64_t)mv.size();
    if (!mv.empty()) ++gen;
  }

  // Page merge once heads hold different rows: walk the table from the first
  // candidate; a page whose rows fit after the page before it in every head
  // (per-head sums <= page_tokens) is appended to it head by head, so each
  // head keeps its row order.  Returns the moves; the table is unchanged until
  // commit_head_merges.
  std::vector<HeadMergeMove> plan_head_merges(int heads) const {
    std::vector<HeadMergeMove> mv;
    size_t f = first_candidate();
    if (f >= table.size()) return mv;
    int32_t cur = table[f].page;
    std::vector<int32_t> cur_len((size_t)heads);
    for (int h = 0; h < heads; ++h) cur_len[(size_t)h] = head_len(table[f], h);
    for (size_t i = f + 1; i < table.size(); ++i) {
      bool fits = true;
      for (int h = 0; h < heads && fits; ++h) fits = cur_len[(size_t)h] + head_len(table[i], h) <= T_;
      if (fits) {
        HeadMergeMove m{table[i].page, cur, cur_len, std::vector<int32_t>((size_t)heads)};
        for (int h = 0; h < heads; ++h) {
          m.count[(size_t)h] = head_len(table[i], h);
          cur_len[(size_t)h] += m.count[(size_t)h];
        }
        mv.push_back(std::move(m));
      } else {
        cur = table[i].page;
        for (int h = 0; h < heads; ++h) cur_len[(size_t)h] = head_len(table[i], h);
      }
    }
    return mv;
  }

  void commit_head_merges(const std::vector<HeadMergeMove>& mv, int heads) {
    if (mv.empty()) return;
    std::set<int32_t> gone;
    std::map<int32_t, std::vector<int32_t>> grow;
    for (const auto& m : mv) {
      gone.insert(m.src);
      auto& g = grow[m.dst];
      if (g.empty()) g.assign((size_t)heads, 0);
      for (int h = 0; h < heads; ++h) g[(size_t)h] += m.count[(size_t)h];
    }
    size_t w = 0;
    for (size_t i = 0; i < table.size(); ++i) {
      if (gone.count(table[i].page)) {
        free_ids.insert(table[i].page);
        continue;
      }
      PageEntry& e = table[i];
      auto it = grow.find(e.page);
      if (it != grow.end()) {
        if (e.hlen.empty()) e.hlen.assign((size_t)heads, e.len);
        int32_t mx = 0;
        for (int h = 0; h < heads; ++h) {
          e.hlen[(size_t)h] += it->second[(size_t)h];
          mx = e.hlen[(size_t)h] > mx ? e.hlen[(size_t)h] : mx;
        }
        e.len = mx;
      }
      if (w != i) table[w] = std::move(e);
      ++w;
    }
    table.erase(table.begin() + (long)w, table.end());
    merges += (int64_t)mv.size();
    ++gen;
  }

  // Per-head new lengths for entries first_candidate().. ([entry][head]); a
  // page whose heads are all empty leaves the table and its id is freed.
  // Every remaining candidate page keeps its per-head lengths: its heads now
  // hold different tokens even where their counts agree.
  void apply_head_compaction(const int32_t* new_lens, int heads) {
    // in place: entries keep their per-head length vectors (no reallocation)
    const size_t f = first_candidate();
    size_t w = f;
    for (size_t i = f; i < table.size(); ++i) {
      const int32_t* nl = &new_lens[(i - f) * (size_t)heads];
      int32_t mx = 0;
      for (int h = 0; h < heads; ++h) mx = nl[h] > mx ? nl[h] : mx;
      if (mx == 0) {
        free_ids.insert(table[i].page);
        continue;
      }
      PageEntry& e = table[i];
      e.len = mx;
      e.hlen.assign(nl, nl + heads);
      if (w != i) table[w] = std::move(e);
      ++w;
    }
    table.erase(table.begin() + (long)w, table.end());
    ++prunes;
    ++gen;
  }

  // True when every page holds the same tokens in every head.
  bool same_tokens() const {
    for (const auto& e : table)
      if (!e.hlen.empty()) return false;
    return true;
  }

  // True when every page holds as many rows in every head.
  bool same_lengths() const {
    for (const auto& e : table)
      for (int32_t n : e.hlen)
        if (n != e.len) return false;
    return true;
  }

  int64_t tokens() const {
    int64_t n = 0;
    for (const auto& e : table) n += e.len;
    return n;
  }

  int32_t pages() const { return pages_; }
  int32_t page_tokens() const { return T_; }

  std::vector<PageEntry> table;
  std::set<int32_t> free_ids;
  bool transient_pending = false;
  int64_t transient_frame = -1;
  int64_t last_frame = -1;
  int64_t evictions = 0;
  int64_t compactions = 0;
  int64_t last_keep = 0;
  int64_t merges = 0;
  int64_t prunes = 0;
  int64_t gen = 0;  // changes whenever the table does (never reset, so a stale copy never matches)

 private:
  int32_t pages_ = 0, S_ = 0, W_ = 0, k_ = 1, T_ = 0, SP_ = 0;
};

}  // namespace kvs
