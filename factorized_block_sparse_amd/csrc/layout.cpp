// Host-side layout builder: head patterns -> per-pattern index maps, visible
// key intervals, and the CSR / CSC lists of active (query-tile, key-tile)
// pairs, packed into one position-independent blob.
//
// The visibility sets are those of "Sparse Transformers 深度解读报告",
// section 2.2 (strided: local band and stride; fixed: same block and summary
// columns), all causal (section 2.1).  Tile-level skipping follows report
// section 3.5 and the block-sparse execution of the blog post on sliding
// windows and block sparsity, section 05 (only tile pairs that contain a
// visible pair are computed; a fine mask applies inside partial tiles).
//
// Each pattern is mapped to a "layout space" in which every query row reads a
// prefix [0, pre) and a single interval [lo, hi] of key positions:
//   local, same-block: identity order, interval [max(0,i-l), i] or [l*floor(i/l), i];
//   stride: residue-class order (the grid-column view of the comparison
//           article "稀疏与局部注意力", section 2), interval = the row's own
//           class up to itself;
//   summary: keys packed as the summary cells in order, so a row reads a
//           prefix of them; rows that read nothing (before the first summary
//           cell) read a key slot holding their own token;
//   merged fixed (report section 3.1, Eq. 7: one head reads both fixed sets):
//           the summary cells packed first, so a row's cells up to itself are
//           a prefix; the other tokens follow in order, so the rest of its
//           block up to itself is an interval;
//   local + global tokens (blog post sections 03, 04): identity order, the
//           global tokens before the window as the prefix;
//   merged strided (report section 3.1, Eq. 7, on the strided pattern): no
//           single order makes both its sets intervals, so the head runs as
//           two parts with disjoint key sets -- its local band (a local
//           pattern) and the stride members at distance >= 2l (residue-class
//           order, the row's class up to two positions before itself) --
//           whose results are combined per token by the kernels.
// The prefix is empty for the first four kinds.  This is what makes tiles
// dense for the stride and summary heads instead of holding one useful key
// per row.

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <map>
#include <new>
#include <tuple>
#include <vector>

#include "sparse_attn.h"

namespace {

constexpr int64_t kMaxN = int64_t(1) << 26;
constexpr int kMaxHeads = 4096;

struct Pattern {
  sa_head_pattern p{};
  int32_t s = 0;
  int64_t pairs = 0;
  std::vector<int32_t> qmap, kmap, lo, hi, pre, count;  // pre: empty = no prefixes
  std::vector<int32_t> row_ptr, col, col_ptr, row;
  std::vector<uint8_t> fflag, bflag;
};

bool valid_tile(int32_t t) { return t == 32 || t == 64 || t == 128; }

// Canonical form of a head pattern so that equal patterns share one record.
bool has_summary(int32_t kind) { return kind == SA_SUMMARY || kind == SA_FIXED_MERGED; }

sa_head_pattern canonical(const sa_head_pattern& h) {
  sa_head_pattern c = h;
  if (has_summary(h.kind)) {
    c.sub = h.sub % (h.l / h.c);
  } else if (h.kind == SA_LOCAL_GLOBAL) {
    c.sub = 0;
  } else {
    c.c = 0;
    c.sub = 0;
  }
  return c;
}

int check_head(const sa_head_pattern& h) {
  if (h.kind < SA_LOCAL || h.kind > SA_STRIDED_MERGED) return SA_EINVAL;
  if (h.l < 1) return SA_EINVAL;
  if (has_summary(h.kind)) {
    if (h.c < 1 || h.c > h.l || h.sub < 0) return SA_EINVAL;
  }
  if (h.kind == SA_LOCAL_GLOBAL && h.c < 0) return SA_EINVAL;
  return SA_OK;
}

// Index maps and intervals in layout space (see the header for the maps).
int build_maps(Pattern& P, int64_t n64, int32_t n_pad, bool self_if_empty) {
  const int32_t n = int32_t(n64);
  const int32_t l = P.p.l;
  P.qmap.assign(n_pad, -1);
  P.kmap.assign(n_pad, -1);
  P.lo.assign(n_pad, 1);
  P.hi.assign(n_pad, 0);
  P.count.assign(n, 0);
  switch (P.p.kind) {
    case SA_LOCAL:
      for (int32_t i = 0; i < n; ++i) {
        P.qmap[i] = P.kmap[i] = i;
        P.lo[i] = i > l ? i - l : 0;
        P.hi[i] = i;
      }
      break;
    case SA_SAMEBLOCK:
      for (int32_t i = 0; i < n; ++i) {
        P.qmap[i] = P.kmap[i] = i;
        P.lo[i] = (i / l) * l;
        P.hi[i] = i;
      }
      break;
    case SA_STRIDE:
    case SA_STRIDE_FAR: {
      // Residue r holds ceil((n - r) / l) tokens; classes are laid out in order.
      // The far variant stops two positions short (distance >= 2l); its rows
      // t < 2 read nothing.
      const int32_t skip = P.p.kind == SA_STRIDE_FAR ? 2 : 0;
      const int32_t classes = int32_t(std::min<int64_t>(l, n));
      std::vector<int32_t> off(classes + 1, 0);
      for (int32_t r = 0; r < classes; ++r) off[r + 1] = off[r] + (n - r + l - 1) / l;
      for (int32_t i = 0; i < n; ++i) {
        const int32_t r = i % l, t = i / l;
        const int32_t p = off[r] + t;
        P.qmap[p] = P.kmap[p] = i;
        if (t >= skip) {
          P.lo[p] = off[r];
          P.hi[p] = p - skip;
        }
      }
      break;
    }
    case SA_SUMMARY: {
      const int32_t c = P.p.c;
      const int32_t s = l - (P.p.sub + 1) * c;
      P.s = s;
      std::vector<uint8_t> used(n, 0);
      int32_t e = 0;
      for (int64_t base = 0; base < n; base += l) {
        for (int32_t u = 0; u < c; ++u) {
          const int64_t j = base + s + u;
          if (j < n) {
            P.kmap[e++] = int32_t(j);
            used[j] = 1;
          }
        }
      }
      for (int32_t i = 0; i < n; ++i) {
        P.qmap[i] = i;
        const int32_t rr = i % l - s + 1;
        const int32_t cnt = (i / l) * c + std::min(std::max(rr, 0), c);
        if (cnt > 0) {
          P.lo[i] = 0;
          P.hi[i] = cnt - 1;
        } else {
          if (!self_if_empty) return SA_EINVAL;  // empty row: no softmax
          P.kmap[e] = i;
          used[i] = 1;
          P.lo[i] = P.hi[i] = e;
          ++e;
        }
      }
      for (int32_t j = 0; j < n; ++j)
        if (!used[j]) P.kmap[e++] = j;
      if (e != n) return SA_EINVAL;
      break;
    }
    case SA_FIXED_MERGED: {
      const int32_t c = P.p.c;
      const int32_t s = l - (P.p.sub + 1) * c;
      P.s = s;
      P.pre.assign(n_pad, 0);
      auto is_cell = [&](int32_t j) { return j % l >= s && j % l < s + c; };
      std::vector<int32_t> pos(n, -1);  // key position of each non-summary token
      int32_t e = 0;
      for (int32_t j = 0; j < n; ++j)
        if (is_cell(j)) P.kmap[e++] = j;
      for (int32_t j = 0; j < n; ++j)
        if (!is_cell(j)) {
          pos[j] = e;
          P.kmap[e++] = j;
        }
      for (int32_t i = 0; i < n; ++i) {
        const int32_t b = i / l, r = i % l;
        P.qmap[i] = i;
        P.pre[i] = b * c + std::min(std::max(r - s + 1, 0), c);  // cells j <= i
        // The block's other tokens up to i: from its first non-cell token to
        // the last non-cell token <= i (consecutive key positions).
        const int32_t first = s > 0 ? b * l : b * l + c;
        const int32_t last = is_cell(i) ? b * l + s - 1 : i;
        if (first <= last) {
          P.lo[i] = pos[first];
          P.hi[i] = pos[last];
        }
      }
      break;
    }
    case SA_LOCAL_GLOBAL: {
      const int32_t glob = P.p.c;
      P.pre.assign(n_pad, 0);
      for (int32_t i = 0; i < n; ++i) {
        P.qmap[i] = P.kmap[i] = i;
        P.lo[i] = i > l ? i - l : 0;
        P.hi[i] = i;
        P.pre[i] = std::min(glob, P.lo[i]);  // global tokens before the window
      }
      break;
    }
    default:
      return SA_EINVAL;
  }
  bool any_pre = false;
  for (int32_t v : P.pre) any_pre |= v > 0;
  if (!any_pre) P.pre.clear();
  P.pairs = 0;
  for (int32_t p = 0; p < n; ++p) {
    const int32_t cnt = std::max(P.hi[p] - P.lo[p] + 1, 0) + (P.pre.empty() ? 0 : P.pre[p]);
    P.count[P.qmap[p]] = cnt;
    P.pairs += cnt;
  }
  return SA_OK;
}

// An upper bound on the active tiles of a pattern, from each query tile's
// widest key interval and longest prefix (no tile is touched outside them).
int64_t tile_bound(const Pattern& P, int32_t n, int32_t n_pad, int32_t bq, int32_t bk) {
  const int32_t nqt = n_pad / bq, nkt = n_pad / bk;
  int64_t bound = 0;
  for (int32_t qt = 0; qt < nqt; ++qt) {
    int32_t lo = INT32_MAX, hi = -1, pre = 0;
    for (int32_t r = qt * bq; r < std::min(qt * bq + bq, n); ++r) {
      if (P.lo[r] <= P.hi[r]) {
        lo = std::min(lo, P.lo[r]);
        hi = std::max(hi, P.hi[r]);
      }
      if (!P.pre.empty()) pre = std::max(pre, P.pre[r]);
    }
    int64_t t = (hi >= lo ? int64_t(hi / bk - lo / bk + 1) : 0) + (pre + bk - 1) / bk;
    bound += std::min<int64_t>(t, nkt);
  }
  return bound;
}

// CSR / CSC arrays are indexed with int32: layouts whose active tiles could
// exceed that range are refused (SA_EUNSUPPORTED) before they are built.
int build_tiles(Pattern& P, int32_t n, int32_t n_pad, int32_t bq, int32_t bk) {
  if (tile_bound(P, n, n_pad, bq, bk) > int64_t(INT32_MAX)) return SA_EUNSUPPORTED;
  const int32_t nqt = n_pad / bq, nkt = n_pad / bk;
  P.row_ptr.assign(nqt + 1, 0);
  P.col.clear();
  P.fflag.clear();
  std::vector<uint8_t> mark(nkt, 0);
  std::vector<int32_t> touched;
  for (int32_t qt = 0; qt < nqt; ++qt) {
    const int32_t r0 = qt * bq, r1 = std::min(r0 + bq, n);
    int32_t max_lo = INT32_MIN, min_hi = INT32_MAX;
    touched.clear();
    auto touch = [&](int32_t kt) {
      if (!mark[kt]) {
        mark[kt] = 1;
        touched.push_back(kt);
      }
    };
    for (int32_t r = r0; r < r1; ++r) {
      const int32_t lo = P.lo[r], hi = P.hi[r];
      max_lo = std::max(max_lo, lo);
      min_hi = std::min(min_hi, hi);
      if (lo <= hi)
        for (int32_t kt = lo / bk; kt <= hi / bk; ++kt) touch(kt);
      if (!P.pre.empty() && P.pre[r] > 0)
        for (int32_t kt = 0; kt <= (P.pre[r] - 1) / bk; ++kt) touch(kt);
    }
    std::sort(touched.begin(), touched.end());
    const bool rows_all_valid = (r0 + bq <= n);
    // Every key of [a, b] visible to row r: inside the prefix, or inside the
    // interval (extended to 0 when the prefix reaches it).
    auto covered = [&](int32_t r, int32_t a, int32_t b) {
      const int32_t pre = P.pre[r], lo = P.lo[r], hi = P.hi[r];
      if (b < pre) return true;
      if (lo > hi) return false;
      return a >= (pre >= lo ? 0 : lo) && b <= hi;
    };
    for (int32_t kt : touched) {
      bool full = rows_all_valid;
      if (full && P.pre.empty()) {
        full = kt * bk >= max_lo && (kt + 1) * bk - 1 <= min_hi;
      } else {
        for (int32_t r = r0; full && r < r1; ++r) full = covered(r, kt * bk, (kt + 1) * bk - 1);
      }
      P.col.push_back(kt);
      P.fflag.push_back(full ? SA_TILE_FULL : SA_TILE_PARTIAL);
      mark[kt] = 0;
    }
    P.row_ptr[qt + 1] = int32_t(P.col.size());
  }
  // CSC by counting sort; rows come out ascending because CSR rows are visited in order.
  const int32_t nnz = int32_t(P.col.size());
  P.col_ptr.assign(nkt + 1, 0);
  for (int32_t e = 0; e < nnz; ++e) P.col_ptr[P.col[e] + 1]++;
  for (int32_t kt = 0; kt < nkt; ++kt) P.col_ptr[kt + 1] += P.col_ptr[kt];
  P.row.assign(nnz, 0);
  P.bflag.assign(nnz, 0);
  std::vector<int32_t> fill(P.col_ptr.begin(), P.col_ptr.end() - 1);
  for (int32_t qt = 0; qt < nqt; ++qt) {
    for (int32_t e = P.row_ptr[qt]; e < P.row_ptr[qt + 1]; ++e) {
      const int32_t dst = fill[P.col[e]]++;
      P.row[dst] = qt;
      P.bflag[dst] = P.fflag[e];
    }
  }
  return SA_OK;
}

int64_t align64(int64_t x) { return (x + 63) & ~int64_t(63); }

struct Writer {
  uint8_t* base;  // NULL while sizing
  int64_t pos = 0;
  template <class T>
  int64_t put(const T* data, size_t count) {
    pos = align64(pos);
    const int64_t at = pos;
    if (base && count) std::memcpy(base + at, data, count * sizeof(T));
    pos += int64_t(count * sizeof(T));
    return at;
  }
  template <class T>
  int64_t put(const std::vector<T>& v) {
    return put(v.data(), v.size());
  }
};

struct SchedItem {
  int32_t head, tile, work;
  int32_t e0 = 0, e1 = 0, slot = -1;
  int32_t pattern = 0, slot0 = -1, nchunks = 1;  // head's pattern; split tile: its slots
  int32_t first = -1;  // first list entry packed as (tile << 1) | FULL; -1 if none
};

// Per-XCD lists over the sorted schedule `sorted` (work in sorted order):
// the items are taken in natural order (head, tile, e0), cut into SA_XCDS
// contiguous runs of about equal work, each run sorted heaviest first, and
// every list padded with -1 to the longest.  Returns the list length.
int32_t xcd_lists(const std::vector<SchedItem>& sorted, std::vector<int32_t>& out) {
  const int32_t n = int32_t(sorted.size());
  std::vector<int32_t> order(n);
  for (int32_t i = 0; i < n; ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
    const SchedItem &x = sorted[a], &y = sorted[b];
    if (x.head != y.head) return x.head < y.head;
    if (x.tile != y.tile) return x.tile < y.tile;
    return x.e0 < y.e0;
  });
  int64_t total = 0;
  for (const auto& it : sorted) total += it.work;
  std::vector<std::vector<int32_t>> lists(SA_XCDS);
  int64_t run = 0;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t idx = order[i];
    // XCD of the item's work midpoint
    const int64_t mid2 = 2 * run + sorted[idx].work;
    int32_t x = total > 0 ? int32_t(mid2 * SA_XCDS / (2 * total)) : 0;
    x = std::min<int32_t>(std::max<int32_t>(x, 0), SA_XCDS - 1);
    lists[x].push_back(idx);
    run += sorted[idx].work;
  }
  int32_t len = 0;
  for (auto& l : lists) {
    // indices into `sorted` ascend with decreasing work: sorting them keeps heaviest first
    std::sort(l.begin(), l.end());
    len = std::max<int32_t>(len, int32_t(l.size()));
  }
  out.assign(size_t(SA_XCDS) * len, -1);
  for (int32_t x = 0; x < SA_XCDS; ++x)
    for (size_t j = 0; j < lists[x].size(); ++j) out[size_t(x) * len + j] = lists[x][j];
  return len;
}

// Heaviest first; ties keep (head, tile) order.  SA_SCHED_FIELDS ints per
// entry: (head, tile, e0, e1, slot, pattern, slot0, nchunks, first).
std::vector<int32_t> sorted_schedule(std::vector<SchedItem>& items) {
  std::stable_sort(items.begin(), items.end(),
                   [](const SchedItem& a, const SchedItem& b) { return a.work > b.work; });
  std::vector<int32_t> out;
  out.reserve(items.size() * SA_SCHED_FIELDS);
  for (const auto& it : items)
    out.insert(out.end(),
               {it.head, it.tile, it.e0, it.e1, it.slot, it.pattern, it.slot0, it.nchunks, it.first});
  return out;
}

int build(const sa_layout_desc* desc, uint8_t* blob, size_t* blob_bytes) {
  if (!desc || !blob_bytes) return SA_EINVAL;
  if (desc->n < 1 || desc->n > kMaxN) return SA_EINVAL;
  if (desc->num_heads < 1 || desc->num_heads > kMaxHeads || !desc->heads) return SA_EINVAL;
  if (!valid_tile(desc->block_q) || !valid_tile(desc->block_k)) return SA_EUNSUPPORTED;
  if (desc->flags & ~(SA_SELF_IF_EMPTY | SA_NO_SEGMENT_PASS)) return SA_EINVAL;
  if (desc->split_keys < 0 || desc->split_rows < 0) return SA_EINVAL;
  const bool self_if_empty = (desc->flags & SA_SELF_IF_EMPTY) != 0;
  const int32_t n = int32_t(desc->n);
  const int32_t bq = desc->block_q, bk = desc->block_k;
  const int32_t t = std::max(bq, bk);
  const int32_t n_pad = int32_t(((desc->n + t - 1) / t) * t);
  const int32_t nqt = n_pad / bq, nkt = n_pad / bk;

  std::vector<Pattern> pats;
  std::map<std::tuple<int32_t, int32_t, int32_t, int32_t>, int32_t> index;
  std::vector<int32_t> head_pat(desc->num_heads), head_part(desc->num_heads, -1);
  std::vector<int32_t> head_merged(desc->num_heads, -1);
  int32_t num_merged = 0;
  // Index of pattern c, built on first use (negative: an error status).
  auto pattern_index = [&](const sa_head_pattern& c) -> int32_t {
    const auto key = std::make_tuple(c.kind, c.l, c.c, c.sub);
    auto it = index.find(key);
    if (it == index.end()) {
      Pattern P;
      P.p = c;
      const int rc2 = build_maps(P, n, n_pad, self_if_empty);
      if (rc2 != SA_OK) return rc2;
      const int rc3 = build_tiles(P, n, n_pad, bq, bk);
      if (rc3 != SA_OK) return rc3;
      it = index.emplace(key, int32_t(pats.size())).first;
      pats.push_back(std::move(P));
    }
    return it->second;
  };
  for (int32_t h = 0; h < desc->num_heads; ++h) {
    const int rc = check_head(desc->heads[h]);
    if (rc != SA_OK) return rc;
    const sa_head_pattern c = canonical(desc->heads[h]);
    if (c.kind == SA_STRIDED_MERGED) {
      const int32_t a = pattern_index(sa_head_pattern{SA_LOCAL, c.l, 0, 0});
      const int32_t f = pattern_index(sa_head_pattern{SA_STRIDE_FAR, c.l, 0, 0});
      if (a < 0) return a;
      if (f < 0) return f;
      head_pat[h] = a;
      head_part[h] = f;
      head_merged[h] = num_merged++;
    } else {
      const int32_t a = pattern_index(c);
      if (a < 0) return a;
      head_pat[h] = a;
    }
  }
  if (pats.size() > 0xffff || num_merged > 0x3ffe) return SA_EUNSUPPORTED;

  const int32_t split_rows = desc->split_rows > 0 ? desc->split_rows : SA_SPLIT_ROWS;
  const int32_t split_keys = desc->split_keys > 0 ? desc->split_keys : SA_SPLIT_KEYS;
  const int32_t cap = std::max<int32_t>(1, split_rows / bq);   // q-tiles per dK/dV chunk
  const int32_t qcap = std::max<int32_t>(1, split_keys / bk);  // k-tiles per forward / dQ chunk
  // Heads whose backward runs in the segment pass: stride heads (each
  // residue class is a run of layout positions that reads only itself) with
  // classes of at most SA_SEGMENT_ROWS rows and no split tile.
  std::vector<uint8_t> seg_head(desc->num_heads, 0);
  int32_t seg_rows_max = 0;
  for (int32_t h = 0; h < desc->num_heads && !(desc->flags & SA_NO_SEGMENT_PASS); ++h) {
    const Pattern& P = pats[head_pat[h]];
    if (head_part[h] >= 0 || P.p.kind != SA_STRIDE) continue;
    const int32_t rows = (n + P.p.l - 1) / P.p.l;  // the longest class
    if (rows > SA_SEGMENT_ROWS) continue;
    bool split = false;
    for (int32_t qt = 0; qt < nqt && !split; ++qt) split = P.row_ptr[qt + 1] - P.row_ptr[qt] > qcap;
    for (int32_t kt = 0; kt < nkt && !split; ++kt) split = P.col_ptr[kt + 1] - P.col_ptr[kt] > cap;
    if (split) continue;
    seg_head[h] = 1;
    seg_rows_max = std::max(seg_rows_max, rows);
  }

  std::vector<SchedItem> fwd_items, bwd_items, seg_items;
  std::vector<int32_t> red_sched;   // (head, k-tile, first slot, chunks)
  std::vector<int32_t> comb_sched;  // (head, q-tile, first slot, chunks)
  int32_t num_slots = 0, num_qslots = 0;
  int64_t pairs_all = 0, tiles_all = 0;
  for (int32_t h = 0; h < desc->num_heads; ++h) {
    const Pattern& P = pats[head_pat[h]];
    pairs_all += P.pairs;
    tiles_all += int64_t(P.col.size());
    if (head_part[h] >= 0) {
      pairs_all += pats[head_part[h]].pairs;
      tiles_all += int64_t(pats[head_part[h]].col.size());
    }
    for (int32_t qt = 0; qt < nqt; ++qt) {
      const int32_t r0 = P.row_ptr[qt], r1 = P.row_ptr[qt + 1], len = r1 - r0;
      if (len == 0) continue;
      if (len <= qcap) {
        SchedItem it{h, qt, len};
        it.e0 = r0;
        it.e1 = r1;
        fwd_items.push_back(it);
        continue;
      }
      const int32_t chunks = (len + qcap - 1) / qcap;
      comb_sched.insert(comb_sched.end(), {h, qt, num_qslots, chunks});
      for (int32_t c = 0; c < chunks; ++c) {
        SchedItem it{h, qt, 0};
        it.e0 = r0 + int32_t(int64_t(len) * c / chunks);
        it.e1 = r0 + int32_t(int64_t(len) * (c + 1) / chunks);
        it.work = it.e1 - it.e0;
        it.slot = num_qslots + c;
        it.slot0 = num_qslots;
        it.nchunks = chunks;
        fwd_items.push_back(it);
      }
      num_qslots += chunks;
    }
    if (seg_head[h]) {
      // One item per residue class r: tokens r + l t, t < rows, at layout
      // positions [off, off + rows) (the maps' class order); work ~ its
      // visible pairs.
      const int32_t classes = std::min(P.p.l, n);
      for (int32_t r = 0, off = 0; r < classes; ++r) {
        const int32_t rows = (n - r + P.p.l - 1) / P.p.l;
        SchedItem it{h, off, int32_t(int64_t(rows) * (rows + 1) / 2)};
        it.e0 = r;
        it.e1 = rows;
        it.slot = P.p.l;
        seg_items.push_back(it);
        off += rows;
      }
      continue;  // no dK/dV items
    }
    for (int32_t kt = 0; kt < nkt; ++kt) {
      if (kt * bk >= n) continue;  // all padding keys
      const int32_t c0 = P.col_ptr[kt], c1 = P.col_ptr[kt + 1], len = c1 - c0;
      if (len <= cap) {
        SchedItem it{h, kt, len + 1};
        it.e0 = c0;
        it.e1 = c1;
        bwd_items.push_back(it);
        continue;
      }
      // Split into `chunks` nearly equal runs of CSC entries, one partial slot each.
      const int32_t chunks = (len + cap - 1) / cap;
      red_sched.insert(red_sched.end(), {h, kt, num_slots, chunks});
      for (int32_t c = 0; c < chunks; ++c) {
        SchedItem it{h, kt, 0};
        it.e0 = c0 + int32_t(int64_t(len) * c / chunks);
        it.e1 = c0 + int32_t(int64_t(len) * (c + 1) / chunks);
        it.work = it.e1 - it.e0 + 1;
        it.slot = num_slots + c;
        it.slot0 = num_slots;
        it.nchunks = chunks;
        bwd_items.push_back(it);
      }
      num_slots += chunks;
    }
  }
  // Pattern field: pattern index, (two-part head index + 1) << 16, and
  // kPartInit on the first chunk of each of a two-part head's tiles.
  constexpr int32_t kPartInit = int32_t(1) << 30;
  auto pattern_field = [&](int32_t h, int32_t pat, bool first) {
    int32_t f = pat;
    if (head_merged[h] >= 0) f |= ((head_merged[h] + 1) << 16) | (first ? kPartInit : 0);
    return f;
  };
  for (auto& it : fwd_items) it.pattern = pattern_field(it.head, head_pat[it.head], it.slot == it.slot0);
  for (auto& it : bwd_items) it.pattern = pattern_field(it.head, head_pat[it.head], it.slot == it.slot0);
  for (auto& it : seg_items) it.pattern = head_pat[it.head];
  // Second parts: every tile holding a token, none split.
  std::vector<SchedItem> fwdp_items, bwdp_items;
  for (int32_t h = 0; h < desc->num_heads; ++h) {
    if (head_part[h] < 0) continue;
    const Pattern& P = pats[head_part[h]];
    const int32_t f = pattern_field(h, head_part[h], false);
    for (int32_t qt = 0; qt < nqt && qt * bq < n; ++qt) {
      SchedItem it{h, qt, P.row_ptr[qt + 1] - P.row_ptr[qt] + 1};
      it.e0 = P.row_ptr[qt];
      it.e1 = P.row_ptr[qt + 1];
      it.pattern = f;
      fwdp_items.push_back(it);
    }
    for (int32_t kt = 0; kt < nkt && kt * bk < n; ++kt) {
      SchedItem it{h, kt, P.col_ptr[kt + 1] - P.col_ptr[kt] + 1};
      it.e0 = P.col_ptr[kt];
      it.e1 = P.col_ptr[kt + 1];
      it.pattern = f;
      bwdp_items.push_back(it);
    }
  }
  // The first entry of each item's list, so a workgroup can start its first
  // tile's loads without reading the list.
  auto set_first = [&](std::vector<SchedItem>& items, bool csc) {
    for (auto& it : items) {
      if (it.e0 >= it.e1) continue;
      const Pattern& P = pats[it.pattern & 0xffff];
      const int32_t tile = csc ? P.row[it.e0] : P.col[it.e0];
      const uint8_t flag = csc ? P.bflag[it.e0] : P.fflag[it.e0];
      it.first = (tile << 1) | (flag == SA_TILE_FULL ? 1 : 0);
    }
  };
  set_first(fwd_items, false);
  set_first(fwdp_items, false);
  set_first(bwd_items, true);
  set_first(bwdp_items, true);
  // The dQ pass: the forward's query-tile entries of the heads without segments.
  std::vector<SchedItem> dq_items;
  for (const auto& it : fwd_items)
    if (!seg_head[it.head]) dq_items.push_back(it);
  const std::vector<int32_t> dq_sched = sorted_schedule(dq_items);
  const std::vector<int32_t> seg_sched = sorted_schedule(seg_items);
  const std::vector<int32_t> fwd_sched = sorted_schedule(fwd_items);
  const std::vector<int32_t> bwd_sched = sorted_schedule(bwd_items);
  const std::vector<int32_t> fwdp_sched = sorted_schedule(fwdp_items);
  const std::vector<int32_t> bwdp_sched = sorted_schedule(bwdp_items);
  std::vector<int32_t> fwd_xl, bwd_xl, fwdp_xl, bwdp_xl;
  const int32_t fwd_xl_len = xcd_lists(fwd_items, fwd_xl);
  const int32_t bwd_xl_len = xcd_lists(bwd_items, bwd_xl);
  const int32_t fwdp_xl_len = fwdp_items.empty() ? 0 : xcd_lists(fwdp_items, fwdp_xl);
  const int32_t bwdp_xl_len = bwdp_items.empty() ? 0 : xcd_lists(bwdp_items, bwdp_xl);
  std::vector<int32_t> dq_xl, seg_xl;
  const int32_t dq_xl_len = xcd_lists(dq_items, dq_xl);
  const int32_t seg_xl_len = seg_items.empty() ? 0 : xcd_lists(seg_items, seg_xl);
  // The entries in list order (padding: all -1).
  auto list_items = [](const std::vector<int32_t>& xl, const std::vector<int32_t>& sched) {
    std::vector<int32_t> out;
    out.reserve(xl.size() * SA_SCHED_FIELDS);
    for (const int32_t idx : xl)
      for (int f = 0; f < SA_SCHED_FIELDS; ++f)
        out.push_back(idx < 0 ? -1 : sched[size_t(idx) * SA_SCHED_FIELDS + f]);
    return out;
  };
  const std::vector<int32_t> fwd_xitem = list_items(fwd_xl, fwd_sched);
  const std::vector<int32_t> bwd_xitem = list_items(bwd_xl, bwd_sched);
  const std::vector<int32_t> fwdp_xitem = list_items(fwdp_xl, fwdp_sched);
  const std::vector<int32_t> bwdp_xitem = list_items(bwdp_xl, bwdp_sched);
  const std::vector<int32_t> dq_xitem = list_items(dq_xl, dq_sched);
  const std::vector<int32_t> seg_xitem = list_items(seg_xl, seg_sched);

  // Two passes: size, then write.
  for (int pass = 0; pass < 2; ++pass) {
    uint8_t* base = pass == 0 ? nullptr : blob;
    Writer w{base};
    sa_blob_header hdr{};
    const int64_t hdr_at = w.put(&hdr, 1);
    std::vector<sa_pattern_rec> recs(pats.size());
    const int64_t rec_at = w.put(recs.data(), recs.size());
    hdr.head_pattern_off = w.put(head_pat);
    hdr.fwd_sched_off = w.put(fwd_sched);
    hdr.bwd_sched_off = w.put(bwd_sched);
    hdr.red_sched_off = w.put(red_sched);
    hdr.fwd_xl_off = w.put(fwd_xl);
    hdr.comb_sched_off = w.put(comb_sched);
    hdr.bwd_xl_off = w.put(bwd_xl);
    hdr.fwd_xitem_off = w.put(fwd_xitem);
    hdr.bwd_xitem_off = w.put(bwd_xitem);
    hdr.head_part_off = w.put(head_part);
    hdr.head_merged_off = w.put(head_merged);
    hdr.fwdp_sched_off = w.put(fwdp_sched);
    hdr.bwdp_sched_off = w.put(bwdp_sched);
    hdr.fwdp_xitem_off = w.put(fwdp_xitem);
    hdr.bwdp_xitem_off = w.put(bwdp_xitem);
    hdr.dq_xitem_off = w.put(dq_xitem);
    hdr.seg_xitem_off = w.put(seg_xitem);
    for (size_t i = 0; i < pats.size(); ++i) {
      const Pattern& P = pats[i];
      sa_pattern_rec& r = recs[i];
      r.kind = P.p.kind;
      r.l = P.p.l;
      r.c = P.p.c;
      r.sub = P.p.sub;
      r.s = P.s;
      r.nnz = int32_t(P.col.size());
      r.pairs = P.pairs;
      r.qmap_off = w.put(P.qmap);
      r.kmap_off = w.put(P.kmap);
      r.lo_off = w.put(P.lo);
      r.hi_off = w.put(P.hi);
      r.pre_off = P.pre.empty() ? 0 : w.put(P.pre);
      r.count_off = w.put(P.count);
      r.row_ptr_off = w.put(P.row_ptr);
      r.col_off = w.put(P.col);
      r.fflag_off = w.put(P.fflag);
      r.col_ptr_off = w.put(P.col_ptr);
      r.row_off = w.put(P.row);
      r.bflag_off = w.put(P.bflag);
    }
    const int64_t total = align64(w.pos);
    if (pass == 0) {
      if (!blob) {
        *blob_bytes = size_t(total);
        return SA_OK;
      }
      if (*blob_bytes < size_t(total)) {
        *blob_bytes = size_t(total);
        return SA_ESIZE;
      }
      std::memset(blob, 0, size_t(total));
      continue;
    }
    hdr.magic = SA_BLOB_MAGIC;
    hdr.version = SA_BLOB_VERSION;
    hdr.n = desc->n;
    hdr.block_q = bq;
    hdr.block_k = bk;
    hdr.num_heads = desc->num_heads;
    hdr.num_patterns = int32_t(pats.size());
    hdr.n_pad = n_pad;
    hdr.nqt = nqt;
    hdr.nkt = nkt;
    hdr.flags = desc->flags;
    hdr.total_bytes = total;
    hdr.pattern_off = rec_at;
    hdr.fwd_sched_len = int32_t(fwd_items.size());
    hdr.bwd_sched_len = int32_t(bwd_items.size());
    hdr.red_sched_len = int32_t(red_sched.size() / 4);
    hdr.num_slots = num_slots;
    hdr.fwd_xl_len = fwd_xl_len;
    hdr.comb_sched_len = int32_t(comb_sched.size() / 4);
    hdr.num_qslots = num_qslots;
    hdr.split_keys = split_keys;
    hdr.split_rows = split_rows;
    hdr.bwd_xl_len = bwd_xl_len;
    hdr.pairs_all_heads = pairs_all;
    hdr.tiles_all_heads = tiles_all;
    hdr.num_merged = num_merged;
    hdr.fwdp_sched_len = int32_t(fwdp_items.size());
    hdr.bwdp_sched_len = int32_t(bwdp_items.size());
    hdr.fwdp_xl_len = fwdp_xl_len;
    hdr.bwdp_xl_len = bwdp_xl_len;
    hdr.dq_xl_len = dq_xl_len;
    hdr.seg_xl_len = seg_xl_len;
    hdr.seg_len = int32_t(seg_items.size());
    hdr.seg_tiles = (seg_rows_max + 31) / 32;
    std::memcpy(blob + hdr_at, &hdr, sizeof(hdr));
    std::memcpy(blob + rec_at, recs.data(), recs.size() * sizeof(sa_pattern_rec));
    *blob_bytes = size_t(total);
  }
  return SA_OK;
}

bool in_blob(int64_t off, int64_t bytes, int64_t total) {
  return off >= 0 && bytes >= 0 && off <= total && bytes <= total - off && (off % 4) == 0;
}

}  // namespace

extern "C" int sparse_attn_layout(const sa_layout_desc* desc, void* blob, size_t* blob_bytes) {
  try {
    return build(desc, static_cast<uint8_t*>(blob), blob_bytes);
  } catch (const std::bad_alloc&) {
    return SA_ENOMEM;  // host memory for the build ran out: never throw across the ABI
  } catch (...) {
    return SA_EINVAL;
  }
}

extern "C" int sparse_attn_layout_check(const void* blob_host, size_t blob_bytes) {
  if (!blob_host || blob_bytes < sizeof(sa_blob_header)) return SA_EINVAL;
  const uint8_t* b = static_cast<const uint8_t*>(blob_host);
  sa_blob_header h;
  std::memcpy(&h, b, sizeof(h));
  if (h.magic != SA_BLOB_MAGIC || h.version != SA_BLOB_VERSION) return SA_EINVAL;
  const int64_t total = h.total_bytes;
  if (total < int64_t(sizeof(h)) || size_t(total) > blob_bytes) return SA_ESIZE;
  if (h.n < 1 || h.n > kMaxN || !valid_tile(h.block_q) || !valid_tile(h.block_k)) return SA_EINVAL;
  // At most two patterns per head (the parts of a merged strided head).
  if (h.num_heads < 1 || h.num_heads > kMaxHeads || h.num_patterns < 1 ||
      h.num_patterns > 2 * h.num_heads)
    return SA_EINVAL;
  const int64_t t = std::max(h.block_q, h.block_k);
  if (h.n_pad != ((h.n + t - 1) / t) * t || h.nqt * h.block_q != h.n_pad ||
      h.nkt * h.block_k != h.n_pad)
    return SA_EINVAL;
  if (!in_blob(h.head_pattern_off, 4 * int64_t(h.num_heads), total) ||
      !in_blob(h.pattern_off, int64_t(sizeof(sa_pattern_rec)) * h.num_patterns, total) ||
      !in_blob(h.fwd_sched_off, 4 * SA_SCHED_FIELDS * int64_t(h.fwd_sched_len), total) ||
      !in_blob(h.comb_sched_off, 16 * int64_t(h.comb_sched_len), total) || h.num_qslots < 0 ||
      !in_blob(h.bwd_sched_off, 4 * SA_SCHED_FIELDS * int64_t(h.bwd_sched_len), total) ||
      !in_blob(h.red_sched_off, 16 * int64_t(h.red_sched_len), total) || h.num_slots < 0 ||
      !in_blob(h.fwd_xl_off, 4 * int64_t(SA_XCDS) * h.fwd_xl_len, total) ||
      !in_blob(h.bwd_xl_off, 4 * int64_t(SA_XCDS) * h.bwd_xl_len, total) ||
      !in_blob(h.fwd_xitem_off, 4 * SA_SCHED_FIELDS * int64_t(SA_XCDS) * h.fwd_xl_len, total) ||
      !in_blob(h.bwd_xitem_off, 4 * SA_SCHED_FIELDS * int64_t(SA_XCDS) * h.bwd_xl_len, total) ||
      !in_blob(h.head_part_off, 4 * int64_t(h.num_heads), total) ||
      !in_blob(h.head_merged_off, 4 * int64_t(h.num_heads), total) || h.num_merged < 0 ||
      h.num_merged > h.num_heads || h.fwdp_sched_len < 0 || h.bwdp_sched_len < 0 ||
      h.fwdp_xl_len < 0 || h.bwdp_xl_len < 0 ||
      !in_blob(h.fwdp_sched_off, 4 * SA_SCHED_FIELDS * int64_t(h.fwdp_sched_len), total) ||
      !in_blob(h.bwdp_sched_off, 4 * SA_SCHED_FIELDS * int64_t(h.bwdp_sched_len), total) ||
      !in_blob(h.fwdp_xitem_off, 4 * SA_SCHED_FIELDS * int64_t(SA_XCDS) * h.fwdp_xl_len, total) ||
      !in_blob(h.bwdp_xitem_off, 4 * SA_SCHED_FIELDS * int64_t(SA_XCDS) * h.bwdp_xl_len, total) ||
      h.dq_xl_len < 0 || h.seg_xl_len < 0 || h.seg_len < 0 || h.seg_tiles < 0 ||
      h.seg_tiles > (SA_SEGMENT_ROWS + 31) / 32 || (h.seg_tiles == 0) != (h.seg_len == 0) ||
      !in_blob(h.dq_xitem_off, 4 * SA_SCHED_FIELDS * int64_t(SA_XCDS) * h.dq_xl_len, total) ||
      !in_blob(h.seg_xitem_off, 4 * SA_SCHED_FIELDS * int64_t(SA_XCDS) * h.seg_xl_len, total))
    return SA_EINVAL;
  for (int32_t i = 0; i < h.num_patterns; ++i) {
    sa_pattern_rec r;
    std::memcpy(&r, b + h.pattern_off + i * sizeof(sa_pattern_rec), sizeof(r));
    const int64_t np = 4 * int64_t(h.n_pad);
    if (!in_blob(r.qmap_off, np, total) || !in_blob(r.kmap_off, np, total) ||
        !in_blob(r.lo_off, np, total) || !in_blob(r.hi_off, np, total) ||
        (r.pre_off != 0 && !in_blob(r.pre_off, np, total)) ||
        !in_blob(r.count_off, 4 * h.n, total) ||
        !in_blob(r.row_ptr_off, 4 * int64_t(h.nqt + 1), total) ||
        !in_blob(r.col_off, 4 * int64_t(r.nnz), total) ||
        !in_blob(r.col_ptr_off, 4 * int64_t(h.nkt + 1), total) ||
        !in_blob(r.row_off, 4 * int64_t(r.nnz), total) || r.fflag_off < 0 ||
        r.fflag_off + r.nnz > total || r.bflag_off < 0 || r.bflag_off + r.nnz > total)
      return SA_EINVAL;
  }
  for (int32_t hh = 0; hh < h.num_heads; ++hh) {
    int32_t p, q, m;
    std::memcpy(&p, b + h.head_pattern_off + 4 * hh, 4);
    std::memcpy(&q, b + h.head_part_off + 4 * hh, 4);
    std::memcpy(&m, b + h.head_merged_off + 4 * hh, 4);
    if (p < 0 || p >= h.num_patterns || q < -1 || q >= h.num_patterns) return SA_EINVAL;
    if ((q < 0) != (m < 0) || m >= h.num_merged) return SA_EINVAL;
  }
  return SA_OK;
}

extern "C" const char* sparse_attn_strerror(int status) {
  switch (status) {
    case SA_OK: return "success";
    case SA_EINVAL: return "invalid argument";
    case SA_EUNSUPPORTED: return "unsupported configuration";
    case SA_ESIZE: return "buffer too small";
    case SA_EHIP: return "HIP runtime error";
    case SA_ENOMEM: return "out of host memory";
    default: return "unknown status";
  }
}
