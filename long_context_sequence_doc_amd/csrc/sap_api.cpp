// C ABI of libsap: argument checks, plan lifetime and kernel dispatch.
// Every check runs on the host before anything is launched; no C++
// exception crosses the ABI.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <new>
#include <string>

#include "kernels.h"
#include "sap_internal.h"

struct sap_plan_s {
  sap::Plan p;
};

namespace {

thread_local std::string g_last_error;

sap_status fail(sap_status s, const std::string &msg) {
  g_last_error = msg;
  return s;
}

sap_status ok() {
  g_last_error.clear();
  return SAP_OK;
}

sap_status hip_fail(hipError_t e, const char *what) {
  return fail(SAP_ERR_HIP, std::string(what) + ": " + hipGetErrorName(e) + " (" + hipGetErrorString(e) + ")");
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }

template <class T>
size_t bytes_of(const std::vector<T> &v) { return v.size() * sizeof(T); }

sap_status check_heads(int32_t hq, int32_t hkv, int32_t d) {
  if (hq <= 0 || hkv <= 0 || hq % hkv != 0) return fail(SAP_ERR_INVALID_ARG, "need hq > 0, hkv > 0, hq % hkv == 0");
  if (d != 64 && d != 128) return fail(SAP_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  return SAP_OK;
}

// A plan with work must be uploaded to the current device before a launch.
sap_status check_uploaded(sap_plan_t plan) {
  if (!plan->p.dev.base) return fail(SAP_ERR_STATE, "plan has not been uploaded (call sap_plan_upload)");
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != plan->p.dev.device)
    return fail(SAP_ERR_STATE, "plan was uploaded to another device");
  return SAP_OK;
}

}  // namespace

extern "C" {

int32_t sap_version(void) { return 300; }

const char *sap_last_error(void) { return g_last_error.c_str(); }

sap_status sap_plan(const int32_t *cu_seqlens, int32_t n_docs, const sap_segment *q_segs,
                    int32_t n_q_segs, const sap_segment *kv_segs, int32_t n_kv_segs,
                    int32_t block_m, int32_t block_n, sap_plan_t *out) {
  if (!out) return fail(SAP_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  sap_plan_s *h = new (std::nothrow) sap_plan_s();
  if (!h) return fail(SAP_ERR_NO_MEMORY, "plan allocation failed");
  std::string err;
  sap_status s;
  try {
    s = sap::build_plan(cu_seqlens, n_docs, q_segs, n_q_segs, kv_segs, n_kv_segs, block_m, block_n, &h->p, &err);
  } catch (const std::bad_alloc &) {
    s = SAP_ERR_NO_MEMORY;
    err = "host memory exhausted while planning";
  } catch (...) {
    s = SAP_ERR_INVALID_ARG;
    err = "planner failed";
  }
  if (s != SAP_OK) {
    delete h;
    return fail(s, err);
  }
  *out = h;
  return ok();
}

sap_status sap_balance(const int32_t *cu_seqlens, int32_t n_docs, int32_t n_ranks, int32_t chunk_rows,
                       int32_t *owner, int64_t cap_owner, int64_t *rank_work) {
  if (!owner) return fail(SAP_ERR_INVALID_ARG, "owner is NULL");
  std::vector<int32_t> own;
  std::vector<int64_t> load;
  std::string err;
  sap_status s;
  try {
    s = sap::balance_chunks(cu_seqlens, n_docs, n_ranks, chunk_rows, &own, &load, &err);
  } catch (const std::bad_alloc &) {
    s = SAP_ERR_NO_MEMORY;
    err = "host memory exhausted while balancing";
  }
  if (s != SAP_OK) return fail(s, err);
  if (cap_owner < int64_t(own.size())) return fail(SAP_ERR_INVALID_ARG, "owner capacity smaller than the chunk count");
  std::copy(own.begin(), own.end(), owner);
  if (rank_work) std::copy(load.begin(), load.end(), rank_work);
  return ok();
}

sap_status sap_plan_upload(sap_plan_t plan, void *hip_stream) {
  if (!plan) return fail(SAP_ERR_INVALID_ARG, "plan is NULL");
  sap::Plan &P = plan->p;
  if (P.dev.base) return ok();
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  // one allocation; each table 256-byte aligned
  constexpr int NT = 13;
  size_t off[NT], total = 0;
  const void *src[NT] = {P.q_work.data(), P.q_range.data(), P.q_partners.data(), P.kv_work.data(),
                         P.kv_range.data(), P.kv_partners.data(), P.ds_q.data(), P.touched_rows.data(),
                         P.kv_slot.data(), P.kv_reduce.data(), P.q2_work.data(), P.q2_range.data(),
                         P.q2_partners.data()};
  size_t len[NT] = {bytes_of(P.q_work), bytes_of(P.q_range), bytes_of(P.q_partners), bytes_of(P.kv_work),
                    bytes_of(P.kv_range), bytes_of(P.kv_partners), bytes_of(P.ds_q), bytes_of(P.touched_rows),
                    bytes_of(P.kv_slot), bytes_of(P.kv_reduce), bytes_of(P.q2_work), bytes_of(P.q2_range),
                    bytes_of(P.q2_partners)};
  for (int i = 0; i < NT; ++i) {
    off[i] = total;
    total += align_up(std::max<size_t>(len[i], 1));
  }
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  void *base = nullptr;
  e = hipMalloc(&base, total);
  if (e == hipErrorOutOfMemory) return fail(SAP_ERR_NO_MEMORY, "hipMalloc of plan tables failed");
  if (e != hipSuccess) return hip_fail(e, "hipMalloc");
  for (int i = 0; i < NT; ++i) {
    if (!len[i]) continue;
    e = hipMemcpyAsync(static_cast<char *>(base) + off[i], src[i], len[i], hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) {
      (void)hipFree(base);
      return hip_fail(e, "hipMemcpyAsync of plan tables");
    }
  }
  e = hipStreamSynchronize(stream);
  if (e != hipSuccess) {
    (void)hipFree(base);
    return hip_fail(e, "hipStreamSynchronize after plan upload");
  }
  char *b = static_cast<char *>(base);
  P.dev.base = base;
  P.dev.bytes = total;
  P.dev.q_work = reinterpret_cast<const sap::WorkItem *>(b + off[0]);
  P.dev.q_range = reinterpret_cast<const sap::WorkRange *>(b + off[1]);
  P.dev.q_partners = reinterpret_cast<const sap::PartnerEntry *>(b + off[2]);
  P.dev.kv_work = reinterpret_cast<const sap::WorkItem *>(b + off[3]);
  P.dev.kv_range = reinterpret_cast<const sap::WorkRange *>(b + off[4]);
  P.dev.kv_partners = reinterpret_cast<const sap::PartnerEntry *>(b + off[5]);
  P.dev.ds_q = reinterpret_cast<const int32_t *>(b + off[6]);
  P.dev.touched_rows = reinterpret_cast<const int32_t *>(b + off[7]);
  P.dev.kv_slot = reinterpret_cast<const int32_t *>(b + off[8]);
  P.dev.kv_reduce = reinterpret_cast<const sap::ReduceItem *>(b + off[9]);
  P.dev.q2_work = reinterpret_cast<const sap::WorkItem *>(b + off[10]);
  P.dev.q2_range = reinterpret_cast<const sap::WorkRange *>(b + off[11]);
  P.dev.q2_partners = reinterpret_cast<const sap::PartnerEntry *>(b + off[12]);
  P.dev.device = dev;
  return ok();
}

sap_status sap_plan_info(sap_plan_t plan, sap_plan_stats *out) {
  if (!plan || !out) return fail(SAP_ERR_INVALID_ARG, "plan or out is NULL");
  const sap::Plan &P = plan->p;
  std::memset(out, 0, sizeof(*out));
  out->n_tiles = int64_t(P.q_tile.size());
  out->n_full = P.n_class[SAP_TILE_FULL];
  out->n_diagonal = P.n_class[SAP_TILE_DIAGONAL];
  out->n_partial = P.n_class[SAP_TILE_PARTIAL];
  out->useful_pairs_per_head = P.useful;
  out->n_q_tiles = int32_t(P.q_tiles.size());
  out->n_kv_tiles = int32_t(P.kv_tiles.size());
  out->n_touched_q_tiles = int32_t(P.touched.size());
  out->n_touched_kv_tiles = P.n_touched_kv;
  out->tq = P.tq;
  out->tkv = P.tkv;
  out->block_m = P.bm;
  out->block_n = P.bn;
  out->uploaded = P.dev.base ? 1 : 0;
  return ok();
}

sap_status sap_plan_tiles(sap_plan_t plan, int32_t *q_tile, int32_t *kv_tile, uint8_t *cls, int64_t cap) {
  if (!plan) return fail(SAP_ERR_INVALID_ARG, "plan is NULL");
  const sap::Plan &P = plan->p;
  const int64_t n = int64_t(P.q_tile.size());
  if (cap < n) return fail(SAP_ERR_INVALID_ARG, "capacity smaller than n_tiles");
  if (n == 0) return ok();
  if (q_tile) std::memcpy(q_tile, P.q_tile.data(), size_t(n) * 4);
  if (kv_tile) std::memcpy(kv_tile, P.kv_tile.data(), size_t(n) * 4);
  if (cls) std::memcpy(cls, P.cls.data(), size_t(n));
  return ok();
}

sap_status sap_plan_q_tiles(sap_plan_t plan, int32_t *touched, int32_t cap_touched, int32_t *desc,
                            int32_t cap_desc) {
  if (!plan) return fail(SAP_ERR_INVALID_ARG, "plan is NULL");
  const sap::Plan &P = plan->p;
  if (touched) {
    if (cap_touched < int32_t(P.touched.size())) return fail(SAP_ERR_INVALID_ARG, "touched capacity too small");
    std::copy(P.touched.begin(), P.touched.end(), touched);
  }
  if (desc) {
    if (cap_desc < 3 * int32_t(P.q_tiles.size())) return fail(SAP_ERR_INVALID_ARG, "desc capacity too small");
    for (size_t i = 0; i < P.q_tiles.size(); ++i) {
      desc[3 * i] = P.q_tiles[i].local_start;
      desc[3 * i + 1] = P.q_tiles[i].n;
      desc[3 * i + 2] = P.q_tiles[i].global_start;
    }
  }
  return ok();
}

void sap_plan_free(sap_plan_t plan) {
  if (!plan) return;
  if (plan->p.dev.base) (void)hipFree(plan->p.dev.base);
  delete plan;
}

namespace {

sap_status fwd_impl(sap_plan_t plan, const void *q, const void *k, const void *v, int64_t q_row_stride,
                    int64_t kv_row_stride, int32_t hq, int32_t hkv, int32_t d, float scale, float *o, float *lse,
                    bool merge, void *hip_stream) {
  if (!plan) return fail(SAP_ERR_INVALID_ARG, "plan is NULL");
  sap_status s = check_heads(hq, hkv, d);
  if (s != SAP_OK) return s;
  const sap::Plan &P = plan->p;
  if ((P.bm != 128 && P.bm != 256) || P.bn != 64)
    return fail(SAP_ERR_UNSUPPORTED, "forward needs a 128 x 64 or 256 x 64 plan");
  if (!(scale > 0.f) || !(scale < 1e30f)) return fail(SAP_ERR_INVALID_ARG, "scale must be positive and finite");
  if (P.q_work.empty()) return ok();
  if (!q || !k || !v || !o || !lse) return fail(SAP_ERR_INVALID_ARG, "NULL tensor pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return fail(SAP_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  if (q_row_stride < int64_t(hq) * d || q_row_stride % 8) return fail(SAP_ERR_INVALID_ARG, "q_row_stride must be >= hq*d and a multiple of 8");
  if (kv_row_stride < int64_t(hkv) * d || kv_row_stride % 8) return fail(SAP_ERR_INVALID_ARG, "kv_row_stride must be >= hkv*d and a multiple of 8");
  sap::FwdLaunch a{};
  a.q = q; a.k = k; a.v = v;
  a.q_row_stride = q_row_stride; a.kv_row_stride = kv_row_stride;
  a.hq = hq; a.hkv = hkv; a.d = d; a.scale = scale;
  a.o = o; a.lse = lse; a.tq = P.tq;
  a.n_work = int32_t(P.q_work.size());
  a.block_m = P.bm;
  a.merge = merge;
  if (const char *why = sap::attn_fwd_limits(a)) return fail(SAP_ERR_UNSUPPORTED, why);
  if ((s = check_uploaded(plan)) != SAP_OK) return s;
  a.work = P.dev.q_work; a.range = P.dev.q_range; a.partners = P.dev.q_partners; a.ds_q = P.dev.ds_q;
  hipError_t e = sap::launch_attn_fwd(a, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return hip_fail(e, "attn_fwd launch");
  return ok();
}

}  // namespace

sap_status sap_attn_fwd(sap_plan_t plan, const void *q, const void *k, const void *v,
                        int64_t q_row_stride, int64_t kv_row_stride, int32_t hq, int32_t hkv,
                        int32_t d, float scale, float *o, float *lse, void *hip_stream) {
  return fwd_impl(plan, q, k, v, q_row_stride, kv_row_stride, hq, hkv, d, scale, o, lse, false, hip_stream);
}

sap_status sap_attn_fwd_merge(sap_plan_t plan, const void *q, const void *k, const void *v,
                              int64_t q_row_stride, int64_t kv_row_stride, int32_t hq, int32_t hkv,
                              int32_t d, float scale, float *o_acc, float *lse_acc, void *hip_stream) {
  return fwd_impl(plan, q, k, v, q_row_stride, kv_row_stride, hq, hkv, d, scale, o_acc, lse_acc, true, hip_stream);
}

sap_status sap_lse_merge(sap_plan_t plan, float *o_acc, float *lse_acc, const float *o_part,
                         const float *lse_part, int32_t tq, int32_t hq, int32_t d, void *hip_stream) {
  if (hq <= 0 || d < 4 || d > 256 || (d & (d - 1))) return fail(SAP_ERR_INVALID_ARG, "need hq > 0 and d a power of two in [4, 256]");
  if (tq < 0) return fail(SAP_ERR_INVALID_ARG, "tq < 0");
  sap::MergeLaunch a{};
  if (plan) {
    if (tq != plan->p.tq) return fail(SAP_ERR_INVALID_ARG, "tq differs from the plan's local Q rows");
    if (plan->p.touched.empty()) return ok();
    sap_status s = check_uploaded(plan);
    if (s != SAP_OK) return s;
    a.touched_rows = plan->p.dev.touched_rows;
    a.n_touched = int32_t(plan->p.touched.size());
    a.max_rows = plan->p.bm;
  } else {
    a.touched_rows = nullptr;
    a.n_touched = tq > 0 ? 1 : 0;
    a.max_rows = tq;
  }
  if (a.n_touched == 0) return ok();
  if (!o_acc || !lse_acc || !o_part || !lse_part) return fail(SAP_ERR_INVALID_ARG, "NULL tensor pointer");
  if (!aligned16(o_acc) || !aligned16(o_part)) return fail(SAP_ERR_INVALID_ARG, "O pointers must be 16-byte aligned");
  a.o_acc = o_acc; a.lse_acc = lse_acc; a.o_part = o_part; a.lse_part = lse_part;
  a.tq = tq; a.hq = hq; a.d = d;
  if (const char *why = sap::lse_merge_limits(a)) return fail(SAP_ERR_UNSUPPORTED, why);
  hipError_t e = sap::launch_lse_merge(a, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return hip_fail(e, "lse_merge launch");
  return ok();
}

namespace {

// fp32 partial dK and dV of every workspace slot: [2][slots][hkv][block_n][d]
size_t partial_bytes(const sap::Plan &P, int32_t hkv, int32_t d) {
  if (P.n_kv_slots == 0) return 0;
  return align_up(2 * size_t(P.n_kv_slots) * size_t(hkv) * size_t(P.bn) * size_t(d) * sizeof(float));
}

}  // namespace

size_t sap_attn_bwd_workspace(sap_plan_t plan, int32_t hq, int32_t hkv, int32_t d) {
  if (!plan || hq < 0 || hkv <= 0 || d <= 0) return 0;
  const size_t delta = hq > 0 ? align_up(size_t(hq) * size_t(std::max(plan->p.tq, 1)) * sizeof(float)) : 0;
  return delta + partial_bytes(plan->p, hkv, d);
}

namespace {

sap_status check_bwd_common(sap_plan_t plan, int32_t hq, int32_t hkv, int32_t d) {
  if (!plan) return fail(SAP_ERR_INVALID_ARG, "plan is NULL");
  sap_status s = check_heads(hq, hkv, d);
  if (s != SAP_OK) return s;
  if (plan->p.bm != 64 || plan->p.bn != 128) return fail(SAP_ERR_UNSUPPORTED, "backward needs a 64 x 128 plan");
  return SAP_OK;
}

void fill_bwd(const sap::Plan &P, sap::BwdLaunch *a) {
  a->tq = P.tq;
  a->touched_rows = P.dev.touched_rows;
  a->n_touched_q = int32_t(P.touched.size());
  a->max_q_rows = P.bm;
  a->work = P.dev.kv_work;
  a->range = P.dev.kv_range;
  a->partners = P.dev.kv_partners;
  a->n_work = int32_t(P.kv_work.size());
  a->kv_slot = P.dev.kv_slot;
  a->kv_reduce = P.dev.kv_reduce;
  a->n_reduce = int32_t(P.kv_reduce.size());
  a->n_slots = P.n_kv_slots;
  a->q_work = P.dev.q_work;
  a->q_range = P.dev.q_range;
  a->q_partners = P.dev.q_partners;
  a->n_q_work = int32_t(P.q_work.size());
  a->q2_work = P.dev.q2_work;
  a->q2_range = P.dev.q2_range;
  a->q2_partners = P.dev.q2_partners;
  a->n_q2_work = int32_t(P.q2_work.size());
  a->ds_q = P.dev.ds_q;
}

// Checks of the row-term pass; fills *a. Launches nothing.
sap_status rowterm_check(sap_plan_t plan, const float *o, const void *dout, int64_t q_row_stride, int32_t hq,
                         int32_t d, float *delta, sap::BwdLaunch *a) {
  const sap::Plan &P = plan->p;
  if (!o || !dout || !delta) return fail(SAP_ERR_INVALID_ARG, "NULL pointer");
  if (!aligned16(o) || !aligned16(dout) || !aligned16(delta)) return fail(SAP_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  if (q_row_stride < int64_t(hq) * d || q_row_stride % 8) return fail(SAP_ERR_INVALID_ARG, "q_row_stride must be >= hq*d and a multiple of 8");
  *a = sap::BwdLaunch{};
  a->o = o; a->dout = dout; a->q_row_stride = q_row_stride; a->hq = hq; a->d = d; a->delta = delta;
  fill_bwd(P, a);
  if (const char *why = sap::bwd_rowterm_limits(*a)) return fail(SAP_ERR_UNSUPPORTED, why);
  const sap_status s = check_uploaded(plan);
  if (s != SAP_OK) return s;
  fill_bwd(P, a);          // the device tables' addresses, now that they exist
  return SAP_OK;
}

// Which passes of the backward a call runs.
enum BwdPasses { kDkDv = 1, kDq = 2, kBoth = 3 };

// Checks of the dK/dV and / or dQ passes; fills *a. Launches nothing.
sap_status accumulate_check(sap_plan_t plan, const void *q, const void *k, const void *v, const float *lse_final,
                            const float *delta, const void *dout, int64_t q_row_stride, int64_t kv_row_stride,
                            int32_t hq, int32_t hkv, int32_t d, float scale, float *dq, float *dk, float *dv,
                            float *partial, size_t partial_avail, int passes, sap::BwdLaunch *a) {
  const sap::Plan &P = plan->p;
  if (!(scale > 0.f) || !(scale < 1e30f)) return fail(SAP_ERR_INVALID_ARG, "scale must be positive and finite");
  if (passes & kDkDv) {
    const size_t need = partial_bytes(P, hkv, d);
    if (need > 0 && (!partial || partial_avail < need))
      return fail(SAP_ERR_INVALID_ARG, "workspace too small (see sap_attn_bwd_workspace)");
    if (partial && !aligned16(partial)) return fail(SAP_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    if (!dk || !dv || !aligned16(dk) || !aligned16(dv)) return fail(SAP_ERR_INVALID_ARG, "dk / dv must be 16-byte aligned device pointers");
  }
  if ((passes & kDq) && (!dq || !aligned16(dq))) return fail(SAP_ERR_INVALID_ARG, "dq must be a 16-byte aligned device pointer");
  if (!q || !k || !v || !lse_final || !delta || !dout) return fail(SAP_ERR_INVALID_ARG, "NULL pointer");
  const void *ptrs[] = {q, k, v, lse_final, delta, dout};
  for (const void *p : ptrs)
    if (!aligned16(p)) return fail(SAP_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  if (q_row_stride < int64_t(hq) * d || q_row_stride % 8) return fail(SAP_ERR_INVALID_ARG, "q_row_stride must be >= hq*d and a multiple of 8");
  if (kv_row_stride < int64_t(hkv) * d || kv_row_stride % 8) return fail(SAP_ERR_INVALID_ARG, "kv_row_stride must be >= hkv*d and a multiple of 8");
  *a = sap::BwdLaunch{};
  a->q = q; a->k = k; a->v = v; a->dout = dout; a->lse = lse_final; a->delta = const_cast<float *>(delta);
  a->q_row_stride = q_row_stride; a->kv_row_stride = kv_row_stride;
  a->hq = hq; a->hkv = hkv; a->d = d; a->scale = scale;
  a->dq = dq; a->dk = dk; a->dv = dv;
  a->partial = partial;
  fill_bwd(P, a);
  if (const char *why = sap::attn_bwd_limits(*a)) return fail(SAP_ERR_UNSUPPORTED, why);
  const sap_status s = check_uploaded(plan);
  if (s != SAP_OK) return s;
  fill_bwd(P, a);          // the device tables' addresses, now that they exist
  return SAP_OK;
}

sap_status accumulate_launch(const sap::BwdLaunch &a, int passes, hipStream_t stream) {
  if (passes & kDkDv) {
    const hipError_t e = sap::launch_attn_bwd_dkdv(a, stream);
    if (e != hipSuccess) return hip_fail(e, "attn_bwd dK/dV launch");
  }
  if (passes & kDq) {
    const hipError_t e = sap::launch_attn_bwd_dq(a, stream);
    if (e != hipSuccess) return hip_fail(e, "attn_bwd dQ launch");
  }
  return SAP_OK;
}

sap_status accumulate_entry(sap_plan_t plan, const void *q, const void *k, const void *v, const float *lse_final,
                            const float *delta, const void *dout, int64_t q_row_stride, int64_t kv_row_stride,
                            int32_t hq, int32_t hkv, int32_t d, float scale, float *dq, float *dk, float *dv,
                            void *workspace, size_t workspace_bytes, int passes, void *hip_stream) {
  sap_status s = check_bwd_common(plan, hq, hkv, d);
  if (s != SAP_OK) return s;
  if (plan->p.kv_work.empty()) {
    if (!(scale > 0.f) || !(scale < 1e30f)) return fail(SAP_ERR_INVALID_ARG, "scale must be positive and finite");
    return ok();
  }
  sap::BwdLaunch a;
  if ((s = accumulate_check(plan, q, k, v, lse_final, delta, dout, q_row_stride, kv_row_stride, hq, hkv, d, scale,
                            dq, dk, dv, static_cast<float *>(workspace), workspace ? workspace_bytes : 0, passes,
                            &a)) != SAP_OK)
    return s;
  if ((s = accumulate_launch(a, passes, static_cast<hipStream_t>(hip_stream))) != SAP_OK) return s;
  return ok();
}

}  // namespace

sap_status sap_attn_bwd_rowterm(sap_plan_t plan, const float *o, const void *dout, int64_t q_row_stride,
                                int32_t hq, int32_t d, float *delta, void *hip_stream) {
  sap_status s = check_bwd_common(plan, hq, 1, d);
  if (s != SAP_OK) return s;
  if (plan->p.touched.empty()) return ok();
  sap::BwdLaunch a;
  if ((s = rowterm_check(plan, o, dout, q_row_stride, hq, d, delta, &a)) != SAP_OK) return s;
  const hipError_t e = sap::launch_bwd_rowterm(a, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return hip_fail(e, "bwd row-term launch");
  return ok();
}

sap_status sap_attn_bwd_accumulate(sap_plan_t plan, const void *q, const void *k, const void *v,
                                   const float *lse_final, const float *delta, const void *dout,
                                   int64_t q_row_stride, int64_t kv_row_stride, int32_t hq, int32_t hkv,
                                   int32_t d, float scale, float *dq, float *dk, float *dv, void *workspace,
                                   size_t workspace_bytes, void *hip_stream) {
  return accumulate_entry(plan, q, k, v, lse_final, delta, dout, q_row_stride, kv_row_stride, hq, hkv, d, scale, dq,
                          dk, dv, workspace, workspace_bytes, kBoth, hip_stream);
}

sap_status sap_attn_bwd_dkdv(sap_plan_t plan, const void *q, const void *k, const void *v, const float *lse_final,
                             const float *delta, const void *dout, int64_t q_row_stride, int64_t kv_row_stride,
                             int32_t hq, int32_t hkv, int32_t d, float scale, float *dk, float *dv, void *workspace,
                             size_t workspace_bytes, void *hip_stream) {
  return accumulate_entry(plan, q, k, v, lse_final, delta, dout, q_row_stride, kv_row_stride, hq, hkv, d, scale,
                          nullptr, dk, dv, workspace, workspace_bytes, kDkDv, hip_stream);
}

sap_status sap_attn_bwd_dq(sap_plan_t plan, const void *q, const void *k, const void *v, const float *lse_final,
                           const float *delta, const void *dout, int64_t q_row_stride, int64_t kv_row_stride,
                           int32_t hq, int32_t hkv, int32_t d, float scale, float *dq, void *hip_stream) {
  return accumulate_entry(plan, q, k, v, lse_final, delta, dout, q_row_stride, kv_row_stride, hq, hkv, d, scale, dq,
                          nullptr, nullptr, nullptr, 0, kDq, hip_stream);
}

}  // extern "C"

namespace {

sap_status bwd_impl(sap_plan_t plan, const void *q, const void *k, const void *v, const float *o,
                        const float *lse_final, const void *dout, int64_t q_row_stride,
                        int64_t kv_row_stride, int32_t hq, int32_t hkv, int32_t d, float scale,
                        float *dq, float *dk, float *dv, void *workspace, size_t workspace_bytes,
                        void *hip_stream) {
  sap_status s = check_bwd_common(plan, hq, hkv, d);
  if (s != SAP_OK) return s;
  if (!(scale > 0.f) || !(scale < 1e30f)) return fail(SAP_ERR_INVALID_ARG, "scale must be positive and finite");
  if (plan->p.kv_work.empty()) return ok();
  if (!workspace) return fail(SAP_ERR_INVALID_ARG, "workspace is NULL");
  if (workspace_bytes < sap_attn_bwd_workspace(plan, hq, hkv, d)) return fail(SAP_ERR_INVALID_ARG, "workspace too small");
  if (!aligned16(workspace)) return fail(SAP_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  float *delta = static_cast<float *>(workspace);
  const size_t delta_bytes = sap_attn_bwd_workspace(plan, hq, hkv, d) - sap_attn_bwd_workspace(plan, 0, hkv, d);
  float *partial = reinterpret_cast<float *>(static_cast<char *>(workspace) + delta_bytes);
  // every check of both passes before anything is launched
  sap::BwdLaunch ra, ba;
  if ((s = rowterm_check(plan, o, dout, q_row_stride, hq, d, delta, &ra)) != SAP_OK) return s;
  if ((s = accumulate_check(plan, q, k, v, lse_final, delta, dout, q_row_stride, kv_row_stride, hq, hkv, d, scale,
                            dq, dk, dv, partial, workspace_bytes - delta_bytes, kBoth, &ba)) != SAP_OK)
    return s;
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  const hipError_t e = sap::launch_bwd_rowterm(ra, stream);
  if (e != hipSuccess) return hip_fail(e, "bwd row-term launch");
  if ((s = accumulate_launch(ba, kBoth, stream)) != SAP_OK) return s;
  return ok();
}

}  // namespace

extern "C" {

sap_status sap_attn_bwd(sap_plan_t plan, const void *q, const void *k, const void *v, const float *o,
                        const float *lse_final, const void *dout, int64_t q_row_stride,
                        int64_t kv_row_stride, int32_t hq, int32_t hkv, int32_t d, float scale,
                        float *dq, float *dk, float *dv, void *workspace, size_t workspace_bytes,
                        void *hip_stream) {
  return bwd_impl(plan, q, k, v, o, lse_final, dout, q_row_stride, kv_row_stride, hq, hkv, d, scale, dq, dk, dv,
                  workspace, workspace_bytes, hip_stream);
}

sap_status sap_attn_bwd_noalloc(sap_plan_t plan, const void *q, const void *k, const void *v, const float *o,
                                const float *lse_final, const void *dout, int64_t q_row_stride,
                                int64_t kv_row_stride, int32_t hq, int32_t hkv, int32_t d, float scale,
                                float *dq, float *dk, float *dv, void *hip_stream) {
  sap_status s = check_bwd_common(plan, hq, hkv, d);
  if (s != SAP_OK) return s;
  const size_t need = sap_attn_bwd_workspace(plan, hq, hkv, d);
  if (need > sap::kNoAllocScratchBytes)
    return fail(SAP_ERR_UNSUPPORTED, "sap_attn_bwd_noalloc: the plan needs " + std::to_string(need) +
                                         " bytes of scratch, more than its fixed " +
                                         std::to_string(sap::kNoAllocScratchBytes) +
                                         " (use sap_attn_bwd with a workspace)");
  if (plan->p.kv_work.empty()) {
    if (!(scale > 0.f) || !(scale < 1e30f)) return fail(SAP_ERR_INVALID_ARG, "scale must be positive and finite");
    return ok();
  }
  // host checks first: nothing touches a device for a call that is refused
  if ((s = check_uploaded(plan)) != SAP_OK) return s;
  void *ws = nullptr;
  const hipError_t e = sap::noalloc_scratch(&ws);
  if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress of the backward scratch");
  return bwd_impl(plan, q, k, v, o, lse_final, dout, q_row_stride, kv_row_stride, hq, hkv, d, scale, dq, dk, dv, ws,
                  sap::kNoAllocScratchBytes, hip_stream);
}

}  // extern "C"
