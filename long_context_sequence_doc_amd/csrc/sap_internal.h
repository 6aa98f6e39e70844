// Internal data structures of libsap: the host plan and the device tables the
// kernels read. Not part of the ABI.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "../../include/sap.h"

namespace sap {

// A run of consecutive rows inside one segment: local rows
// [local_start, local_start + n) hold global positions [global_start, +n).
struct TileDesc {
  int32_t local_start;
  int32_t n;
  int32_t global_start;
};

// One unit of kernel work: a touched tile and its list of partner tiles.
// Forward: a Q tile and the KV tiles it meets. Backward: a KV tile and the Q
// tiles that meet it. 16 bytes, read with one scalar load.
struct WorkItem {
  int32_t local_start;
  int32_t n;
  int32_t global_start;
  int32_t tile;       // tile index (Q tile for forward, KV tile for backward)
};

struct WorkRange {
  int32_t begin;      // first entry in the partner list
  int32_t count;      // number of partners
};

// One partner tile of a work item with the class of the pair.
struct PartnerEntry {
  int32_t local_start;
  int32_t global_start;
  int32_t n;
  int32_t cls;        // SAP_TILE_FULL / DIAGONAL / PARTIAL
};

// A split backward work item whose chunks left partial dK / dV sums in
// workspace slots [slot_begin, slot_begin + slot_count) of the KV tile at
// local rows [local_start, local_start + n).
struct ReduceItem {
  int32_t local_start;
  int32_t n;
  int32_t slot_begin;
  int32_t slot_count;
};

// Device copies of the tables (one allocation, see DeviceTables offsets).
struct DeviceTables {
  void *base = nullptr;
  size_t bytes = 0;
  const WorkItem *q_work = nullptr;      // touched Q tiles, heaviest first
  const WorkRange *q_range = nullptr;
  const PartnerEntry *q_partners = nullptr;
  const WorkItem *kv_work = nullptr;     // chunks of touched KV tiles, heaviest first
  const WorkRange *kv_range = nullptr;
  const PartnerEntry *kv_partners = nullptr;
  const int32_t *kv_slot = nullptr;      // workspace slot of each chunk, -1 = unsplit
  const ReduceItem *kv_reduce = nullptr; // split KV tiles
  const int32_t *ds_q = nullptr;         // [tq] document start of each local Q row
  const int32_t *touched_rows = nullptr; // [n_touched] (local_start, n) pairs, ascending
  const WorkItem *q2_work = nullptr;     // 128-row Q tiles (dQ pass), heaviest first
  const WorkRange *q2_range = nullptr;
  const PartnerEntry *q2_partners = nullptr;
  int device = -1;
};

struct Plan {
  int32_t bm = 0, bn = 0;
  int32_t tq = 0, tkv = 0;
  std::vector<int32_t> cu;
  std::vector<TileDesc> q_tiles, kv_tiles;
  // canonical tile list
  std::vector<int32_t> q_tile, kv_tile;
  std::vector<uint8_t> cls;
  int64_t useful = 0;
  int64_t n_class[3] = {0, 0, 0};
  // forward work (Q-major) and backward work (KV-major). A KV tile with many
  // partner Q tiles is split into chunks (kv_work / kv_range entries of the
  // same tile over consecutive partner runs) so the dK / dV pass has enough
  // workgroups; each chunk of a split tile owns a workspace slot (kv_slot,
  // -1 for unsplit tiles) that kv_reduce lists per tile.
  std::vector<WorkItem> q_work, kv_work;
  std::vector<WorkRange> q_range, kv_range;
  std::vector<PartnerEntry> q_partners, kv_partners;
  std::vector<int32_t> kv_slot;
  std::vector<ReduceItem> kv_reduce;
  int32_t n_kv_slots = 0;
  std::vector<int32_t> ds_q;
  // A 64 x 128 plan (the backward's) also lists its work over 128-row Q
  // tiles against the same 128-key KV tiles: the dQ pass of workgroups with
  // one or two query heads streams each K / V part for twice the rows.
  std::vector<WorkItem> q2_work;
  std::vector<WorkRange> q2_range;
  std::vector<PartnerEntry> q2_partners;
  std::vector<int32_t> touched;       // touched Q tile ids, ascending
  std::vector<int32_t> touched_rows;  // (local_start, n) of touched Q tiles, ascending
  int32_t n_touched_kv = 0;
  DeviceTables dev;
};

// Builds a host plan; returns SAP_OK or an error with *err filled.
sap_status build_plan(const int32_t *cu, int32_t n_docs, const sap_segment *q_segs,
                      int32_t n_q, const sap_segment *kv_segs, int32_t n_kv, int32_t bm,
                      int32_t bn, Plan *out, std::string *err);

// Owner rank of every chunk_rows-position chunk and the work per rank
// (sap_balance); returns SAP_OK or an error with *err filled.
sap_status balance_chunks(const int32_t *cu, int32_t n_docs, int32_t n_ranks, int32_t chunk,
                          std::vector<int32_t> *owner, std::vector<int64_t> *load, std::string *err);

}  // namespace sap
