// Kernel launchers (internal). Each returns hipSuccess or the launch error.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "sap_internal.h"

namespace sap {

struct FwdLaunch {
  const void *q, *k, *v;
  int64_t q_row_stride, kv_row_stride;
  int32_t hq, hkv, d;
  float scale;
  float *o, *lse;
  int32_t tq;
  const WorkItem *work;
  const WorkRange *range;
  const PartnerEntry *partners;
  const int32_t *ds_q;
  int32_t n_work;
  int32_t block_m;    // Q tile rows of the plan: 128 or 256
  bool merge;         // o / lse are a running result to merge into
};

hipError_t launch_attn_fwd(const FwdLaunch &a, hipStream_t stream);
// nullptr if the launch's grid fits the hardware's dispatch limits, else why not
const char *attn_fwd_limits(const FwdLaunch &a);

struct MergeLaunch {
  float *o_acc, *lse_acc;
  const float *o_part, *lse_part;
  int32_t tq, hq, d;
  const int32_t *touched_rows;  // device (local_start, n) pairs; nullptr = all rows
  int32_t n_touched;
  int32_t max_rows;             // rows of the largest touched tile
};

hipError_t launch_lse_merge(const MergeLaunch &a, hipStream_t stream);
const char *lse_merge_limits(const MergeLaunch &a);

struct BwdLaunch {
  const void *q, *k, *v, *dout;
  const float *o, *lse;
  int64_t q_row_stride, kv_row_stride;
  int32_t hq, hkv, d;
  float scale;
  float *dq, *dk, *dv;
  float *delta;                 // row terms [hq][tq]
  int32_t tq;
  const int32_t *touched_rows;  // Q tiles of the plan: (local_start, n) pairs
  int32_t n_touched_q;
  int32_t max_q_rows;
  const WorkItem *work;         // KV-major work (dK, dV)
  const WorkRange *range;
  const PartnerEntry *partners;
  int32_t n_work;
  const WorkItem *q_work;       // Q-major work (dQ) over the plan's 64-row Q tiles
  const WorkRange *q_range;
  const PartnerEntry *q_partners;
  int32_t n_q_work;
  const WorkItem *q2_work;      // the same over 128-row Q tiles
  const WorkRange *q2_range;
  const PartnerEntry *q2_partners;
  int32_t n_q2_work;
  const int32_t *ds_q;
  const int32_t *kv_slot;       // per KV-major chunk: workspace slot, -1 = owns its dK / dV rows
  const ReduceItem *kv_reduce;  // split KV tiles: slots to add up
  int32_t n_reduce;
  int32_t n_slots;
  float *partial;               // [2][n_slots][hkv][128][d] fp32 (dK then dV), or nullptr if n_slots == 0
};

// D_r = dO_r . O_r for the rows of the given tiles
hipError_t launch_bwd_rowterm(const BwdLaunch &a, hipStream_t stream);
const char *bwd_rowterm_limits(const BwdLaunch &a);
// dk / dv given a.delta: the KV-major kernel, then the ordered reduce of split tiles
hipError_t launch_attn_bwd_dkdv(const BwdLaunch &a, hipStream_t stream);
// dq given a.delta: the Q-major kernel
hipError_t launch_attn_bwd_dq(const BwdLaunch &a, hipStream_t stream);
const char *attn_bwd_limits(const BwdLaunch &a);

// Bytes of the allocation-free backward's device scratch (one per GPU).
constexpr size_t kNoAllocScratchBytes = size_t(SAP_BWD_NOALLOC_MAX_BYTES);
// Device address of that scratch on the current device (looked up once per
// device with hipGetSymbolAddress, then cached). Allocates nothing.
hipError_t noalloc_scratch(void **ptr);

}  // namespace sap
