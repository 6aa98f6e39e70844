// Host planner: the sequence-aware schedule of one attention call.
//
// One-device form of the schedule the HSAP summary page
// (gptget.net/papers/2606.30460, method section) generates ahead of the run
// for incomplete tensors and irregular attention: from the document
// boundaries and the segment tables of a call it lists only the
// (Q tile, KV tile) pairs holding an allowed (query, key) pair, classifies
// each pair's mask, and lays the list out as work queues for the kernels.
//
// Masks are decided on global positions (AutoSP page,
// gist.science/zh/paper/2604.27089, section 2.A, index recomputation), so a
// zigzag or ring shard plans exactly like the unsharded sequence restricted
// to its rows.
//
// Class rules for a Q tile at positions [a, b] and a KV tile at [c, e], with
// ds(p) the first position of p's document:
//   EMPTY    <=> c > b  or  e < ds(a)      the union of the rows' windows
//                                          [ds(p), p] is [ds(a), b]
//   FULL     <=> e <= a and c >= ds(b)     every window covers [c, e]
//   DIAGONAL <=> not FULL and c >= ds(b)   lower bounds never bind: key <= query
//   PARTIAL  otherwise                     a document start cuts the tile
#include <algorithm>
#include <cstring>
#include <functional>
#include <new>
#include <numeric>
#include <queue>
#include <utility>

#include "sap_internal.h"

namespace sap {
namespace {

bool valid_block(int32_t b) { return b == 16 || b == 32 || b == 64 || b == 128 || b == 256; }

// Validates a segment table and returns its segments in local-row order.
bool check_segments(const sap_segment *segs, int32_t n, int64_t total, const char *name,
                    std::vector<sap_segment> *sorted, int32_t *rows, std::string *err) {
  sorted->assign(segs, segs + n);
  for (int32_t i = 0; i < n; ++i) {
    const sap_segment &s = (*sorted)[i];
    if (s.global_start < 0 || s.global_end < s.global_start || s.global_end > total ||
        s.local_start < 0) {
      *err = std::string(name) + ": segment " + std::to_string(i) + " out of range";
      return false;
    }
    if (int64_t(s.local_start) + (s.global_end - s.global_start) > INT32_MAX) {
      *err = std::string(name) + ": local rows overflow int32";
      return false;
    }
  }
  std::vector<sap_segment> by_global = *sorted;
  auto empty = [](const sap_segment &s) { return s.global_end == s.global_start; };
  sorted->erase(std::remove_if(sorted->begin(), sorted->end(), empty), sorted->end());
  by_global.erase(std::remove_if(by_global.begin(), by_global.end(), empty), by_global.end());
  std::stable_sort(sorted->begin(), sorted->end(),
                   [](const sap_segment &x, const sap_segment &y) { return x.local_start < y.local_start; });
  std::stable_sort(by_global.begin(), by_global.end(),
                   [](const sap_segment &x, const sap_segment &y) { return x.global_start < y.global_start; });
  int64_t end_rows = 0;
  for (size_t i = 0; i < sorted->size(); ++i) {
    const sap_segment &s = (*sorted)[i];
    int64_t len = s.global_end - s.global_start;
    if (i > 0) {
      const sap_segment &p = (*sorted)[i - 1];
      if (int64_t(p.local_start) + (p.global_end - p.global_start) > s.local_start) {
        *err = std::string(name) + ": local row ranges overlap";
        return false;
      }
    }
    end_rows = std::max<int64_t>(end_rows, s.local_start + len);
  }
  for (size_t i = 1; i < by_global.size(); ++i) {
    if (by_global[i - 1].global_end > by_global[i].global_start) {
      *err = std::string(name) + ": global ranges overlap";
      return false;
    }
  }
  *rows = int32_t(end_rows);
  return true;
}

void tiles_of(const std::vector<sap_segment> &segs, int32_t b, std::vector<TileDesc> *out,
              std::vector<int32_t> *first_tile_of_seg) {
  out->clear();
  first_tile_of_seg->clear();
  for (const sap_segment &s : segs) {
    first_tile_of_seg->push_back(int32_t(out->size()));
    int32_t len = s.global_end - s.global_start;
    for (int32_t off = 0; off < len; off += b)
      out->push_back(TileDesc{s.local_start + off, std::min(b, len - off), s.global_start + off});
  }
}

// Allowed pairs of a non-FULL tile: row p sees keys [max(ds(p), c), min(p, e)].
int64_t count_pairs(const std::vector<int32_t> &cu, int32_t a, int32_t b, int32_t c, int32_t e) {
  int64_t n = 0;
  size_t di = size_t(std::upper_bound(cu.begin(), cu.end(), a) - cu.begin()) - 1;
  for (int32_t p = a; p <= b; ++p) {
    while (di + 1 < cu.size() && cu[di + 1] <= p) ++di;
    int32_t lo = std::max(cu[di], c), hi = std::min(p, e);
    if (hi >= lo) n += hi - lo + 1;
  }
  return n;
}

// Heaviest work first (longest-processing-time order), ties by tile id.
template <class Count>
std::vector<int32_t> lpt_order(size_t n, Count count) {
  std::vector<int32_t> idx(n);
  std::iota(idx.begin(), idx.end(), 0);
  std::stable_sort(idx.begin(), idx.end(), [&](int32_t x, int32_t y) { return count(x) > count(y); });
  return idx;
}

}  // namespace

sap_status build_plan(const int32_t *cu_in, int32_t n_docs, const sap_segment *q_segs,
                      int32_t n_q, const sap_segment *kv_segs, int32_t n_kv, int32_t bm,
                      int32_t bn, Plan *plan, std::string *err) {
  if (!cu_in || n_docs < 1) { *err = "cu_seqlens: need at least one document"; return SAP_ERR_INVALID_ARG; }
  if (n_q < 0 || n_kv < 0 || (n_q > 0 && !q_segs) || (n_kv > 0 && !kv_segs)) {
    *err = "segment table pointer/count invalid";
    return SAP_ERR_INVALID_ARG;
  }
  if (!valid_block(bm) || !valid_block(bn)) { *err = "block_m/block_n must be 16, 32, 64, 128 or 256"; return SAP_ERR_INVALID_ARG; }
  if (cu_in[0] != 0) { *err = "cu_seqlens[0] must be 0"; return SAP_ERR_INVALID_ARG; }
  for (int32_t i = 0; i < n_docs; ++i)
    if (cu_in[i + 1] < cu_in[i]) { *err = "cu_seqlens must be non-decreasing"; return SAP_ERR_INVALID_ARG; }
  const int64_t total = cu_in[n_docs];

  Plan &P = *plan;
  P.bm = bm;
  P.bn = bn;
  // documents: drop empty ones (they hold no position) so ds() is one search
  P.cu.clear();
  P.cu.push_back(0);
  for (int32_t i = 1; i <= n_docs; ++i)
    if (cu_in[i] != P.cu.back()) P.cu.push_back(cu_in[i]);
  const std::vector<int32_t> &cu = P.cu;
  auto ds = [&](int32_t p) { return *(std::upper_bound(cu.begin(), cu.end(), p) - 1); };

  std::vector<sap_segment> qs, ks;
  if (!check_segments(q_segs, n_q, total, "q_segs", &qs, &P.tq, err)) return SAP_ERR_INVALID_ARG;
  if (!check_segments(kv_segs, n_kv, total, "kv_segs", &ks, &P.tkv, err)) return SAP_ERR_INVALID_ARG;

  std::vector<int32_t> q_first, kv_first;
  tiles_of(qs, bm, &P.q_tiles, &q_first);
  tiles_of(ks, bn, &P.kv_tiles, &kv_first);

  // document start of every local Q row (kernels mask PARTIAL tiles with it)
  P.ds_q.assign(size_t(P.tq), -1);
  for (const TileDesc &t : P.q_tiles)
    for (int32_t r = 0; r < t.n; ++r) P.ds_q[size_t(t.local_start + r)] = ds(t.global_start + r);

  P.q_tile.clear(); P.kv_tile.clear(); P.cls.clear();
  P.useful = 0;
  P.n_class[0] = P.n_class[1] = P.n_class[2] = 0;
  std::vector<int64_t> q_ptr(P.q_tiles.size() + 1, 0);
  for (size_t qi = 0; qi < P.q_tiles.size(); ++qi) {
    const TileDesc &qt = P.q_tiles[qi];
    const int32_t a = qt.global_start, b = qt.global_start + qt.n - 1;
    const int32_t ds_a = ds(a), ds_b = ds(b);
    // per KV segment, the tiles meeting [ds_a, b] are one contiguous run
    for (size_t si = 0; si < ks.size(); ++si) {
      const sap_segment &s = ks[si];
      const int32_t lo = std::max(ds_a, s.global_start), hi = std::min(b, s.global_end - 1);
      if (lo > hi) continue;
      const int32_t t0 = (lo - s.global_start) / bn, t1 = (hi - s.global_start) / bn;
      for (int32_t t = t0; t <= t1; ++t) {
        const int32_t ki = kv_first[si] + t;
        const TileDesc &kt = P.kv_tiles[size_t(ki)];
        const int32_t c = kt.global_start, e = kt.global_start + kt.n - 1;
        uint8_t cl;
        if (e <= a && c >= ds_b) cl = SAP_TILE_FULL;
        else if (c >= ds_b) cl = SAP_TILE_DIAGONAL;
        else cl = SAP_TILE_PARTIAL;
        P.q_tile.push_back(int32_t(qi));
        P.kv_tile.push_back(ki);
        P.cls.push_back(cl);
        P.n_class[cl]++;
        P.useful += cl == SAP_TILE_FULL ? int64_t(qt.n) * kt.n : count_pairs(cu, a, b, c, e);
      }
    }
    q_ptr[qi + 1] = int64_t(P.q_tile.size());
  }
  const int64_t n_tiles = int64_t(P.q_tile.size());
  if (n_tiles > INT32_MAX) { *err = "too many tiles for one plan"; return SAP_ERR_INVALID_ARG; }

  // touched Q tiles
  P.touched.clear();
  P.touched_rows.clear();
  for (size_t qi = 0; qi < P.q_tiles.size(); ++qi)
    if (q_ptr[qi + 1] > q_ptr[qi]) {
      P.touched.push_back(int32_t(qi));
      P.touched_rows.push_back(P.q_tiles[qi].local_start);
      P.touched_rows.push_back(P.q_tiles[qi].n);
    }

  // forward work: touched Q tiles, heaviest first; partner list per item
  P.q_work.clear(); P.q_range.clear(); P.q_partners.clear();
  P.q_partners.reserve(size_t(n_tiles));
  std::vector<int32_t> order = lpt_order(P.touched.size(), [&](int32_t i) {
    int32_t qi = P.touched[size_t(i)];
    return q_ptr[size_t(qi) + 1] - q_ptr[size_t(qi)];
  });
  for (int32_t oi : order) {
    const int32_t qi = P.touched[size_t(oi)];
    const TileDesc &qt = P.q_tiles[size_t(qi)];
    P.q_work.push_back(WorkItem{qt.local_start, qt.n, qt.global_start, qi});
    P.q_range.push_back(WorkRange{int32_t(P.q_partners.size()), int32_t(q_ptr[size_t(qi) + 1] - q_ptr[size_t(qi)])});
    for (int64_t t = q_ptr[size_t(qi)]; t < q_ptr[size_t(qi) + 1]; ++t) {
      const TileDesc &kt = P.kv_tiles[size_t(P.kv_tile[size_t(t)])];
      P.q_partners.push_back(PartnerEntry{kt.local_start, kt.global_start, kt.n, P.cls[size_t(t)]});
    }
  }

  // backward work: transposed list (per KV tile, its Q tiles ascending)
  std::vector<int64_t> kv_cnt(P.kv_tiles.size() + 1, 0);
  for (int64_t t = 0; t < n_tiles; ++t) kv_cnt[size_t(P.kv_tile[size_t(t)]) + 1]++;
  std::vector<int64_t> kv_ptr(kv_cnt);
  for (size_t i = 1; i < kv_ptr.size(); ++i) kv_ptr[i] += kv_ptr[i - 1];
  std::vector<int32_t> tr_q(static_cast<size_t>(n_tiles));
  std::vector<uint8_t> tr_c(static_cast<size_t>(n_tiles));
  {
    std::vector<int64_t> fill(kv_ptr.begin(), kv_ptr.end() - 1);
    for (int64_t t = 0; t < n_tiles; ++t) {  // q_tile ascending already
      int64_t pos = fill[size_t(P.kv_tile[size_t(t)])]++;
      tr_q[size_t(pos)] = P.q_tile[size_t(t)];
      tr_c[size_t(pos)] = P.cls[size_t(t)];
    }
  }
  P.kv_work.clear(); P.kv_range.clear(); P.kv_partners.clear(); P.kv_slot.clear();
  P.kv_partners.reserve(size_t(n_tiles));
  std::vector<int32_t> kv_touched;
  for (size_t ki = 0; ki < P.kv_tiles.size(); ++ki)
    if (kv_ptr[ki + 1] > kv_ptr[ki]) kv_touched.push_back(int32_t(ki));
  P.n_touched_kv = int32_t(kv_touched.size());
  order = lpt_order(kv_touched.size(), [&](int32_t i) {
    int32_t ki = kv_touched[size_t(i)];
    return kv_ptr[size_t(ki) + 1] - kv_ptr[size_t(ki)];
  });
  // Chunks: a KV tile's partner list (ascending Q tile) is cut where the Q
  // tile index crosses a multiple of `per`, so the chunks of different KV
  // tiles in one bin stream the same Q / dO rows; a piece shorter than per / 2
  // joins the next one (the last joins the one before). `per` keeps about
  // kTargetChunks bins over the plan (times the KV heads = workgroups of the
  // dK / dV pass) and at least kMinChunk partners in each.
  constexpr int64_t kTargetChunks = 128, kMinChunk = 8;
  const int64_t per = std::max<int64_t>(kMinChunk, (n_tiles + kTargetChunks - 1) / kTargetChunks);
  std::vector<WorkItem> cw;
  std::vector<WorkRange> cr;
  std::vector<int32_t> cs, cbin;
  P.kv_reduce.clear();
  P.n_kv_slots = 0;
  std::vector<std::pair<int64_t, int64_t>> runs;
  for (int32_t oi : order) {
    const int32_t ki = kv_touched[size_t(oi)];
    const TileDesc &kt = P.kv_tiles[size_t(ki)];
    const WorkItem item{kt.local_start, kt.n, kt.global_start, ki};
    const int64_t begin = int64_t(P.kv_partners.size());
    const int64_t t0 = kv_ptr[size_t(ki)], cnt = kv_ptr[size_t(ki) + 1] - t0;
    // partners listed from the last Q tile down: the chunks of one bin all
    // start at its last Q tile (they differ only in where the diagonal ends
    // them), so workgroups of a bin read each Q / dO tile at about the same
    // time
    for (int64_t t = t0 + cnt - 1; t >= t0; --t) {
      const TileDesc &qt = P.q_tiles[size_t(tr_q[size_t(t)])];
      P.kv_partners.push_back(PartnerEntry{qt.local_start, qt.global_start, qt.n, tr_c[size_t(t)]});
    }
    auto bin = [&](int64_t i) { return int64_t(tr_q[size_t(t0 + i)]) / per; };
    runs.clear();
    for (int64_t i = 1, rb = 0; i <= cnt; ++i) {
      if (i < cnt && bin(i) == bin(i - 1)) continue;
      if (!runs.empty() && runs.back().second - runs.back().first < per / 2) runs.back().second = i;
      else runs.emplace_back(rb, i);
      rb = i;
    }
    if (runs.size() > 1 && runs.back().second - runs.back().first < per / 2) {
      runs[runs.size() - 2].second = runs.back().second;
      runs.pop_back();
    }
    if (runs.size() == 1) {
      cw.push_back(item);
      cr.push_back(WorkRange{int32_t(begin), int32_t(cnt)});
      cs.push_back(-1);
      cbin.push_back(int32_t(bin(cnt - 1)));
      continue;
    }
    P.kv_reduce.push_back(ReduceItem{kt.local_start, kt.n, P.n_kv_slots, int32_t(runs.size())});
    for (const auto &r : runs) {
      cw.push_back(item);
      // run [first, second) of the ascending list, in the descending one
      cr.push_back(WorkRange{int32_t(begin + cnt - r.second), int32_t(r.second - r.first)});
      cs.push_back(P.n_kv_slots++);
      cbin.push_back(int32_t(bin(r.second - 1)));
    }
  }
  // Chunks of at least per / 2 partners first, by bin (workgroups that run
  // side by side on an XCD then stream the same Q / dO rows), the lighter
  // ones after them, heaviest first.
  std::vector<int32_t> corder(cw.size());
  std::iota(corder.begin(), corder.end(), 0);
  auto light = [&](int32_t i) { return int64_t(cr[size_t(i)].count) < per / 2; };
  std::stable_sort(corder.begin(), corder.end(), [&](int32_t x, int32_t y) {
    const bool lx = light(x), ly = light(y);
    if (lx != ly) return ly;
    if (lx) return cr[size_t(x)].count > cr[size_t(y)].count;
    return cbin[size_t(x)] < cbin[size_t(y)];
  });
  for (int32_t i : corder) {
    P.kv_work.push_back(cw[size_t(i)]);
    P.kv_range.push_back(cr[size_t(i)]);
    P.kv_slot.push_back(cs[size_t(i)]);
  }
  if (bm == 64 && bn == 128) {
    // the dQ pass's work over 128-row Q tiles (same segments, same KV tiles)
    Plan P2;
    const sap_status s2 = build_plan(cu_in, n_docs, q_segs, n_q, kv_segs, n_kv, 128, 128, &P2, err);
    if (s2 != SAP_OK) return s2;
    P.q2_work = std::move(P2.q_work);
    P.q2_range = std::move(P2.q_range);
    P.q2_partners = std::move(P2.q_partners);
  }
  return SAP_OK;
}

// Document-aware assignment of query chunks to ranks.
//
// The SP blog page (bmjup.com/post/14448.html, future trends and challenges)
// notes that uneven sequence lengths leave GPUs idle; the HSAP summary page
// (gptget.net/papers/2606.30460, technical contributions) balances devices by
// scheduling. Every rank keeps the same number of chunks (the same token
// count); chunks go heaviest first (ties: lower index) to the least-loaded
// rank that still has room (ties: lower rank). A chunk's work is its allowed
// pairs, summed per document run in closed form: the rows [x, y) of a
// document starting at d see x-d+1 .. y-d keys, T(y-d) - T(x-d) in total with
// T(n) = n (n + 1) / 2.
sap_status balance_chunks(const int32_t *cu, int32_t n_docs, int32_t n_ranks, int32_t chunk,
                          std::vector<int32_t> *owner, std::vector<int64_t> *load, std::string *err) {
  if (!cu || n_docs < 1) { *err = "cu_seqlens: need at least one document"; return SAP_ERR_INVALID_ARG; }
  if (cu[0] != 0) { *err = "cu_seqlens[0] must be 0"; return SAP_ERR_INVALID_ARG; }
  for (int32_t i = 0; i < n_docs; ++i)
    if (cu[i + 1] < cu[i]) { *err = "cu_seqlens must be non-decreasing"; return SAP_ERR_INVALID_ARG; }
  if (n_ranks < 1 || chunk < 1) { *err = "need n_ranks >= 1 and chunk_rows >= 1"; return SAP_ERR_INVALID_ARG; }
  const int64_t total = cu[n_docs];
  if (total == 0 || total % (int64_t(chunk) * n_ranks) != 0) {
    *err = "total length must be a positive multiple of chunk_rows * n_ranks";
    return SAP_ERR_INVALID_ARG;
  }
  const int64_t n_chunks = total / chunk;
  const int64_t cap = n_chunks / n_ranks;
  auto tri = [](int64_t n) { return n * (n + 1) / 2; };
  std::vector<int64_t> work(size_t(n_chunks), 0);
  int32_t di = 0;
  for (int64_t c = 0; c < n_chunks; ++c) {
    const int64_t x0 = c * chunk, y0 = x0 + chunk;
    while (cu[di + 1] <= x0) ++di;  // document holding x0 (empty ones skipped)
    for (int32_t dj = di; dj < n_docs && cu[dj] < y0; ++dj) {
      const int64_t x = std::max<int64_t>(x0, cu[dj]), y = std::min<int64_t>(y0, cu[dj + 1]);
      if (y > x) work[size_t(c)] += tri(y - cu[dj]) - tri(x - cu[dj]);
    }
  }
  std::vector<int32_t> order(static_cast<size_t>(n_chunks));
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(),
                   [&](int32_t a, int32_t b) { return work[size_t(a)] > work[size_t(b)]; });
  // ranks with room, least loaded first (ties: lower rank)
  typedef std::pair<int64_t, int32_t> Entry;
  std::priority_queue<Entry, std::vector<Entry>, std::greater<Entry>> open;
  for (int32_t r = 0; r < n_ranks; ++r) open.push(Entry(0, r));
  std::vector<int64_t> count(size_t(n_ranks), 0);
  owner->assign(size_t(n_chunks), -1);
  load->assign(size_t(n_ranks), 0);
  for (int32_t c : order) {
    const Entry e = open.top();
    open.pop();
    const int32_t r = e.second;
    (*owner)[size_t(c)] = r;
    (*load)[size_t(r)] = e.first + work[size_t(c)];
    if (++count[size_t(r)] < cap) open.push(Entry((*load)[size_t(r)], r));
  }
  return SAP_OK;
}

}  // namespace sap
