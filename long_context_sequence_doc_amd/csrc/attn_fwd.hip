// Forward kernel: document-masked causal attention over a plan's tile list,
// for gfx950 (CDNA4) bf16 matrix cores.
//
// Computes, for every touched Q tile and query head, the attention of its
// rows against the KV rows of the call (HSAP summary page,
// gptget.net/papers/2606.30460, original abstract: exact causal attention on
// packed sequences, no cross-document attention), returning O and the
// natural-log log-sum-exp so partial results over disjoint KV sets merge
// exactly.
//
// Layout of the work (one workgroup = one Q tile of the plan x NH query heads
// of one KV head: 128-row tiles with NH = 2 when the GQA group size is even,
// else 1; 256-row tiles with NH = 1):
//   * one wave per 32 query rows of the tile and head; all the workgroup's
//     waves (8, or 4 for 128-row tiles of an odd group) share every staged
//     K / V tile.
//   * Per 64-key KV tile: S^T = K Q^T with v_mfma_f32_32x32x16_bf16. In the
//     32x32 accumulator a lane holds one column (= one query) and 16 rows (=
//     keys), so a query's scores sit in one lane pair (lane, lane ^ 32): row
//     max/sum are in-register plus one v_permlane32_swap across the halves.
//   * P^T (bf16) is already in the B-operand layout of O^T += V^T P^T, so P
//     never goes through LDS. Its registers carry the keys of every 16-key
//     step in the order (0-3, 8-11 | 4-7, 12-15) (lane halves), so the V^T
//     A operand is two ds_read_b64_tr_b16 transposing reads of 4 keys each
//     from row-major V.
//   * K and V tiles go from global memory straight into LDS
//     (global_load_lds_dwordx4 through copy_to_lds: no registers, no VALU)
//     into a double buffer; copies issued in an iteration are waited for at
//     the barrier that ends it. Each load instruction fills 1 KB of LDS, 16 bytes per lane in lane
//     order, so the layout is chosen through the global address each lane
//     loads: rows are unpadded and the 16-byte chunks of a row are
//     XOR-swizzled by the row index, which keeps the matrix-operand reads
//     free of bank conflicts.
//   * Eight-wave workgroups run a software pipeline with K one tile ahead
//     of V: while the vector ALUs turn tile j's scores into P_j, the matrix
//     cores already compute tile j+1's scores (the two waves a SIMD holds
//     are barrier-locked in the same phase, so without this the matrix
//     cores idle through the softmax); in that loop one wave of each pair
//     sharing a SIMD issues the tile copies, twice as many, while its
//     partner starts on the tile. Four-wave workgroups (several per CU)
//     keep the plain double buffer.
//   * Online softmax in fp32 with exp2 and the scale folded into one FMA.
//     The running max is only moved (and O, l rescaled) when it grows by
//     more than 2^8, which keeps the result exact (O / l normalises) while
//     skipping most rescales.
//   * Class FULL tiles skip masking; DIAGONAL masks key > query; PARTIAL also
//     masks keys before the query's document start; ragged tiles mask
//     columns past the tile end (their K/V rows repeat the tile's last row).
//   * Workgroup ids are mapped so that the query heads sharing one KV head
//     and consecutive work items of one KV head land on the same XCD (ids
//     are dealt round-robin over the 8 XCDs), to share K/V in that XCD's L2.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "kernels.h"
#include "lds_copy.h"

namespace sap {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int BN = 64;
constexpr int NXCD = 8;
constexpr float LOG2E = 1.4426950408889634f;
// running max moves only when the new max exceeds it by more than this many
// powers of two (p = 2^(s*c - m*c) then stays <= 2^8)
constexpr float RESCALE_LOG2 = 8.0f;

struct FwdParams {
  const unsigned short *q, *k, *v;
  int64_t q_row_stride, kv_row_stride;
  float *o, *lse;
  const WorkItem *work;
  const WorkRange *range;
  const PartnerEntry *partners;
  const int32_t *ds_q;
  int32_t hq, hkv, group, tq;
  int32_t n_groups;   // work items x KV heads
  float scale, c;     // c = scale * log2(e)
};

// LDS geometry of one stage: K tile then V tile, each BN rows x D bf16,
// row-major, unpadded; 16-byte chunk j of row r is stored at chunk position
// j ^ ksw(r) (K) or j ^ vsw(r) (V).
template <int D, int NT>
struct Stage {
  static constexpr int CPR = D / 8;                    // 16-byte chunks per row
  static constexpr int ROW = 2 * D;                    // bytes per row
  static constexpr int TILE = BN * ROW;                // bytes of the K (or V) tile
  static constexpr int BYTES = 2 * TILE;
  static constexpr int LOADS = BN * CPR / NT;          // 16-byte loads per thread per tile
  static_assert(LOADS * NT == BN * CPR, "the tile must split evenly over the threads");
  // K is read as 16-byte row chunks by 32 consecutive rows: chunk ^ (row % CPR)
  // spreads any run of CPR consecutive rows over distinct chunk positions.
  static __device__ int ksw(int row) { return row % CPR; }
  // V is read by ds_read_b64_tr_b16: each half-wave takes 8 bytes from each
  // of 4 consecutive rows at 4 adjacent chunks. With 256-byte rows (one bank
  // line) XOR by 4 * (row % 4) puts the 16 (row, chunk) pairs on distinct
  // banks; with 128-byte rows two rows share a line and 2 * (row % 4) does.
  static __device__ int vsw(int row) { return CPR >= 16 ? 4 * (row % 4) : 2 * (row % 4); }
};

// Per-thread element offsets (from the tile's first row of the KV head) of
// the global chunks this thread copies into LDS. Chunk position P of a tile
// (16 bytes each, in LDS order) is written by load i = P / NT of wave
// (P / 64) % (NT / 64), lane P % 64, for a workgroup of NT threads. Rows past
// a short tile's end repeat its last row (finite values; their scores are
// masked to -inf, their P is 0).
template <int D, int NT>
struct LoadOffsets {
  int k[Stage<D, NT>::LOADS];
  int v[Stage<D, NT>::LOADS];
};

template <int D, int NT>
__device__ inline LoadOffsets<D, NT> load_offsets(int stride, int wave, int lane, int rows) {
  using G = Stage<D, NT>;
  LoadOffsets<D, NT> o;
#pragma unroll
  for (int i = 0; i < G::LOADS; ++i) {
    const int P = (i * (NT / 64) + wave) * 64 + lane;
    const int row = P / G::CPR, pos = P % G::CPR;
    const int src = min(row, rows - 1) * stride;
    o.k[i] = src + 8 * (pos ^ G::ksw(row));
    o.v[i] = src + 8 * (pos ^ G::vsw(row));
  }
  return o;
}

// Issues the direct global -> LDS copies of one KV tile's K rows (V = false)
// or V rows (V = true) into the stage at byte offset stage of lds.
template <int D, int NT, bool V>
__device__ inline void issue_half(const FwdParams &p, const PartnerEntry &pe, int g, const unsigned char *lds,
                                  int stage, int wave, int lane, const LoadOffsets<D, NT> &full) {
  using G = Stage<D, NT>;
  const int64_t base = int64_t(pe.local_start) * p.kv_row_stride + int64_t(g) * D;
  const unsigned short *src = (V ? p.v : p.k) + base;
  const LoadOffsets<D, NT> o = pe.n == BN ? full : load_offsets<D, NT>(int(p.kv_row_stride), wave, lane, pe.n);
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
  for (int i = 0; i < G::LOADS; ++i)
    copy_to_lds(src + (V ? o.v[i] : o.k[i]), lds, stage + (V ? G::TILE : 0) + (i * (NT / 64) + wave_s) * 1024);
}

// The same copies issued by four waves of an eight-wave workgroup (c = 0..3
// numbers them): chunk position P = (i * 4 + c) * 64 + lane, offsets
// computed here (nothing held in registers across the loop).
template <int D, int NT, bool V>
__device__ inline void issue_half_by4(const FwdParams &p, const PartnerEntry &pe, int g, const unsigned char *lds,
                                      int stage, int c, int lane) {
  using G = Stage<D, NT>;
  constexpr int L4 = BN * G::CPR / 256;
  const int64_t base = int64_t(pe.local_start) * p.kv_row_stride + int64_t(g) * D;
  const unsigned short *src = (V ? p.v : p.k) + base;
  const int stride = int(p.kv_row_stride);
#pragma unroll
  for (int i = 0; i < L4; ++i) {
    const int P = (i * 4 + c) * 64 + lane;
    const int row = P / G::CPR, pos = P % G::CPR;
    const int off = min(row, pe.n - 1) * stride + 8 * (pos ^ (V ? G::vsw(row) : G::ksw(row)));
    copy_to_lds(src + off, lds, stage + (V ? G::TILE : 0) + (i * 4 + c) * 1024);
  }
}

__device__ inline bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

// max / sum of a lane's value and that of lane ^ 32, the same in both lanes.
// v_permlane32_swap exchanges the upper 32 lanes of its first operand with
// the lower 32 lanes of its second; with the value passed as both, each
// lane finds its partner's value in one result and its own in the other.
__device__ inline float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float xor32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// two fp32 -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32
__device__ inline unsigned pack_bf16(float lo, float hi) {
  const bf16x2 v = __builtin_convertvector(f32x2{lo, hi}, bf16x2);
  return __builtin_bit_cast(unsigned, v);
}

// MERGE: o / lse hold a running result that this call's partial is merged
// into (the ring step's merge folded into the epilogue), instead of being
// overwritten.
// TM: rows of the plan's Q tiles (128 or 256), one 32-row slice per wave;
// NH: query heads per workgroup (2 only with TM = 128).
template <int D, bool MERGE, int TM, int NH>
__global__ __launch_bounds__(2 * TM * NH) __attribute__((amdgpu_waves_per_eu(2))) void attn_fwd_kernel(FwdParams p) {
  constexpr int WPH = TM / 32;                    // waves per query head
  constexpr int NT = 64 * WPH * NH;
  static_assert(NH == 1 || TM == 128, "two heads per workgroup only with 128-row tiles");
  using ST = Stage<D, NT>;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[2 * ST::BYTES];

  // workgroup -> (work item, query head), XCD-aware
  const int b = blockIdx.x;
  const int xcd = b % NXCD, slot = b / NXCD;
  const int pairs = p.group / NH;
  const int G = (slot / pairs) * NXCD + xcd;
  if (G >= p.n_groups) return;
  const int w = G / p.hkv, g = G % p.hkv;
  const int h = g * p.group + (slot % pairs) * NH + (int(threadIdx.x) >> 6) / WPH;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const WorkItem wi = p.work[w];
  const WorkRange rg = p.range[w];

  const int my_row = (wave % WPH) * 32 + l32;     // row within the Q tile
  const bool row_ok = my_row < wi.n;
  const int qg = wi.global_start + my_row;        // global position of this lane's query
  const int dsq = row_ok ? p.ds_q[wi.local_start + my_row] : 0;

  // this lane's Q fragment: B operand of S^T = K Q^T (8 consecutive d per k-step)
  bf16x8 qf[D / 16];
  {
    const unsigned short *qp = p.q + int64_t(wi.local_start + my_row) * p.q_row_stride + int64_t(h) * D + 8 * hf;
#pragma unroll
    for (int t = 0; t < D / 16; ++t)
      qf[t] = row_ok ? as_bf16x8(*reinterpret_cast<const u32x4 *>(qp + 16 * t)) : as_bf16x8(u32x4{0u, 0u, 0u, 0u});
  }

  f32x16 oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};
  float m_used = -INFINITY;   // reference max (raw score units), same in both lane halves
  float l_part = 0.f;         // this lane's share of the softmax denominator
  const float c = p.c;

  const LoadOffsets<D, NT> full_offs = load_offsets<D, NT>(int(p.kv_row_stride), wave, lane, BN);

  // LDS byte offsets (within a stage) of this lane's operand reads.
  // K (A operand of S^T): row l32 (+32 for the second key block), chunk
  // 2t + hf of k-step t; (2t + hf) ^ sw = 2t ^ (hf ^ sw), so the offset of
  // step t is k_off ^ (32 t).
  const int k_off = l32 * ST::ROW + 16 * (hf ^ ST::ksw(l32));
  // V^T (A operand of O^T += V^T P^T): within each 16-lane group q (lanes
  // 16q..16q+15), lane s addresses row 4 * (q / 2) + s / 4 (plus the key
  // step's base) and columns 16 * (q % 2) + 4 * (s % 4) .. +3 of the D/32
  // block db; the transposing read hands lane s the 4 keys of column
  // 16 * (q % 2) + s, which is A-operand row l % 32.
  int v_off[D / 32];
  {
    const int q = lane >> 4, s16 = lane & 15;
    const int vrow = 4 * (q >> 1) + (s16 >> 2);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int col = db * 32 + 16 * (q & 1) + 4 * (s16 & 3);
      v_off[db] = ST::TILE + vrow * ST::ROW + 16 * ((col >> 3) ^ ST::vsw(vrow)) + 2 * (col & 7);
    }
  }
  // S^T of 64 keys x this wave's 32 queries from the K tile of a stage: two
  // independent accumulator chains (key blocks)
  auto scores = [&](f32x16 (&s)[2], const unsigned char *stage) {
    s[0] = f32x16{};
    s[1] = f32x16{};
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      const unsigned char *kp = stage + (k_off ^ (32 * t));
      const bf16x8 a0 = as_bf16x8(*reinterpret_cast<const u32x4 *>(kp));
      const bf16x8 a1 = as_bf16x8(*reinterpret_cast<const u32x4 *>(kp + 32 * ST::ROW));
      s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[t], s[0], 0, 0, 0);
      s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[t], s[1], 0, 0, 0);
    }
  };

  // Everything after S^T for one tile: mask by class, online softmax, O^T +=
  // V^T P^T from the V tile of a stage. `overlap` runs between the max
  // update and the exponentials; its matrix work (the next tile's scores)
  // does not depend on them, so the two interleave.
  auto tile_math = [&](f32x16 (&s)[2], const PartnerEntry &cur, const unsigned char *stage, auto &&overlap) {
    if (cur.cls != SAP_TILE_FULL || cur.n < BN) {
      // allowed keys of this lane's query, as tile-local key indices [lo, hi];
      // element i of key block kb holds key kbase + kb*32 + 8*(i/4) + (i%4)
      const int kbase = 4 * hf;
      int hi = cur.n - 1;
      if (cur.cls != SAP_TILE_FULL) hi = min(hi, qg - cur.global_start);
      const int lo = cur.cls == SAP_TILE_PARTIAL ? dsq - cur.global_start : 0;
      const int hi_r = hi - kbase, lo_r = lo - kbase;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kc = kb * 32 + 8 * (i >> 2) + (i & 3);
          s[kb][i] = (kc <= hi_r && kc >= lo_r) ? s[kb][i] : -INFINITY;
        }
    }

    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    mx = xor32_max(mx);
    const bool need = mx > m_used && (m_used == -INFINITY || (mx - m_used) * c > RESCALE_LOG2);
    if (__any(need)) {
      const float m_new = need ? mx : m_used;
      const float alpha = need ? __builtin_amdgcn_exp2f((m_used - m_new) * c) : 1.f;
      m_used = m_new;
      l_part *= alpha;
#pragma unroll
      for (int i = 0; i < D / 32; ++i) oacc[i] *= alpha;
    }
    const float mc = m_used == -INFINITY ? 0.f : m_used * c;

    overlap();

    // P = 2^(s c - m c); B operands of O^T += V^T P^T
    bf16x8 pb[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        float e[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          e[q] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][8 * u + q], c, -mc));
          l_part += e[q];
        }
        u32x4 pk;
        pk.x = pack_bf16(e[0], e[1]);
        pk.y = pack_bf16(e[2], e[3]);
        pk.z = pack_bf16(e[4], e[5]);
        pk.w = pack_bf16(e[6], e[7]);
        pb[kb][u] = as_bf16x8(pk);
      }

    // O^T += V^T P^T: the D/32 output blocks are independent chains
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          // keys kb*32 + 16u + 4hf + (0..3 | 8..11): rows +0 and +8 of the lane's 4-row group
          const unsigned char *vp = stage + v_off[db] + (kb * 32 + 16 * u) * ST::ROW;
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(vp));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(vp + 8 * ST::ROW));
          const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kb][u], oacc[db], 0, 0, 0);
        }
    // keeps the denominator's additions in this tile (otherwise they sink
    // past the barrier and hold the tile's P values in registers)
    asm volatile("" : "+v"(l_part));
  };

  // Partner entries are wave-uniform: each is read by a vector load one
  // iteration before its first use and moved to scalar registers after the
  // barrier that ends that iteration (whose wait covers the load), so no
  // wait for it lands inside an iteration.
  const PartnerEntry *pes = p.partners + rg.begin;
  const int cnt = __builtin_amdgcn_readfirstlane(rg.count);
  auto uniform = [](const PartnerEntry &e) {
    return PartnerEntry{__builtin_amdgcn_readfirstlane(e.local_start), __builtin_amdgcn_readfirstlane(e.global_start),
                        __builtin_amdgcn_readfirstlane(e.n), __builtin_amdgcn_readfirstlane(e.cls)};
  };
  auto raw = [&](int i) { return pes[i < cnt ? i : 0]; };
  PartnerEntry e0 = uniform(raw(0));
  PartnerEntry e1 = uniform(raw(1));

  if constexpr (NT >= 512) {
    // Eight waves: software pipeline over the partner tiles, K one tile
    // ahead of V. When iteration j starts, S_j is in registers and K_{j+1}
    // and V_j are in LDS (stages (j+1) % 2 and j % 2). The iteration issues
    // the copies of K_{j+2} (into K_j's slot) and V_{j+1} (into V_{j-1}'s
    // slot), turns S_j into P_j on the vector ALUs while the matrix cores
    // compute S_{j+1}, adds V_j P_j into O, and ends at a barrier that makes
    // its copies visible and frees the slots it read.
    // waves 1, 3, 4, 6: one of each pair (w, w + 4), the two waves a SIMD
    // holds (the choice also takes one of each pair (2i, 2i + 1))
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const bool copier = ((wave_u >> 2) ^ wave_u) & 1;
    const int copier_id = wave_u >> 1;
    PartnerEntry e2 = uniform(raw(2));
    issue_half<D, NT, false>(p, e0, g, lds, 0, wave, lane, full_offs);
    issue_half<D, NT, true>(p, e0, g, lds, 0, wave, lane, full_offs);
    if (cnt > 1) issue_half<D, NT, false>(p, e1, g, lds, ST::BYTES, wave, lane, full_offs);
    wait_copies();
    __syncthreads();
    f32x16 sA[2], sB[2];
    scores(sA, lds);
    __syncthreads();   // every wave has read K_0 before K_2 replaces it

    auto body = [&](f32x16 (&s)[2], f32x16 (&s_next)[2], int j, auto has_next) {
      constexpr bool HN = decltype(has_next)::value;
      const int off_j = (j & 1) * ST::BYTES, off_n = ((j + 1) & 1) * ST::BYTES;
      const unsigned char *stage_j = lds + off_j, *stage_n = lds + off_n;
      // one wave of each pair that shares a SIMD issues the copies (twice as
      // many); its partner starts on the tile meanwhile
      if (copier) {
        if (j + 2 < cnt) issue_half_by4<D, NT, false>(p, e2, g, lds, off_j, copier_id, lane);
        if (HN) issue_half_by4<D, NT, true>(p, e1, g, lds, off_n, copier_id, lane);
      }
      const PartnerEntry raw3 = raw(j + 3);
      tile_math(s, e0, stage_j, [&] {
        if (HN) scores(s_next, stage_n);
      });
      // the copies have landed and every wave is done with this iteration's slots
      wait_copies();
      __syncthreads();
      // nothing moves above the barrier: the entry load's wait stays behind it
      __builtin_amdgcn_sched_barrier(0);
      e0 = e1;
      e1 = e2;
      e2 = uniform(raw3);
    };

    using yes = std::integral_constant<bool, true>;
    using no = std::integral_constant<bool, false>;
    int j = 0;
    for (; j + 2 < cnt; j += 2) {
      body(sA, sB, j, yes{});
      body(sB, sA, j + 1, yes{});
    }
    if (cnt - j == 2) {
      body(sA, sB, j, yes{});
      body(sB, sA, j + 1, no{});
    } else {
      body(sA, sB, j, no{});
    }
  } else {
    // Four waves (more workgroups per CU, which overlap one another's
    // phases): plain double buffer; the next tile's K and V are copied
    // while this tile is computed.
    issue_half<D, NT, false>(p, e0, g, lds, 0, wave, lane, full_offs);
    issue_half<D, NT, true>(p, e0, g, lds, 0, wave, lane, full_offs);
    wait_copies();
    __syncthreads();
    for (int j = 0; j < cnt; ++j) {
      const unsigned char *stage_j = lds + (j & 1) * ST::BYTES;
      const int off_n = ((j + 1) & 1) * ST::BYTES;
      if (j + 1 < cnt) {
        issue_half<D, NT, false>(p, e1, g, lds, off_n, wave, lane, full_offs);
        issue_half<D, NT, true>(p, e1, g, lds, off_n, wave, lane, full_offs);
      }
      const PartnerEntry raw2 = raw(j + 2);
      f32x16 s[2];
      scores(s, stage_j);
      tile_math(s, e0, stage_j, [] {});
      wait_copies();
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
      e0 = e1;
      e1 = uniform(raw2);
    }
  }

  // epilogue: O = O / l, LSE = m * scale + ln l
  const float l = xor32_sum(l_part);
  if (!row_ok) return;
  const int row = wi.local_start + my_row;
  const bool empty = !(l > 0.f);
  float *op = p.o + (int64_t(row) * p.hq + h) * D + 4 * hf;
  float *lp = p.lse + int64_t(h) * p.tq + row;
  if (MERGE) {
    // merge into the running (O, LSE) of the row:
    //   L = ln(e^La + e^Lb), O = e^(La - L) O_a + e^(Lb - L) O_b
    // a row with no key in this call keeps its running result
    if (empty) return;
    const float lb = m_used * p.scale + __logf(l);
    const float la = *lp;                        // both lanes read before lane hf == 0 writes
    const float mx = fmaxf(la, lb), mn = fminf(la, lb);
    const float L = mx + log1pf(__expf(mn - mx));
    const float wb = __expf(lb - L) / l;
    if (la == -INFINITY) {
      // the running side holds no keys: its O is not read (a select, so
      // whatever it holds cannot leak into the result)
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int ig = 0; ig < 4; ++ig) {
          f32x4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = wb * oacc[db][4 * ig + e];
          *reinterpret_cast<f32x4 *>(op + db * 32 + 8 * ig) = v4;
        }
    } else {
      const float wa = __expf(la - L);
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int ig = 0; ig < 4; ++ig) {
          const f32x4 a = *reinterpret_cast<const f32x4 *>(op + db * 32 + 8 * ig);
          f32x4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = wa * a[e] + wb * oacc[db][4 * ig + e];
          *reinterpret_cast<f32x4 *>(op + db * 32 + 8 * ig) = v4;
        }
    }
    if (hf == 0) *lp = L;
    return;
  }
  const float inv = empty ? 0.f : 1.f / l;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int ig = 0; ig < 4; ++ig) {
      f32x4 v4;
      v4.x = oacc[db][4 * ig + 0] * inv;
      v4.y = oacc[db][4 * ig + 1] * inv;
      v4.z = oacc[db][4 * ig + 2] * inv;
      v4.w = oacc[db][4 * ig + 3] * inv;
      *reinterpret_cast<f32x4 *>(op + db * 32 + 8 * ig) = v4;
    }
  if (hf == 0) *lp = empty ? -INFINITY : m_used * p.scale + __logf(l);
}

}  // namespace

namespace {

// workgroups and threads per workgroup of a forward launch
void fwd_grid(const FwdLaunch &a, int64_t *blocks, int *threads) {
  const int group = a.hq / a.hkv;
  const int nh = a.block_m == 128 && group % 2 == 0 ? 2 : 1;   // query heads per workgroup
  const int64_t slots = (int64_t(a.n_work) * a.hkv + NXCD - 1) / NXCD;
  *blocks = slots * NXCD * (group / nh);
  *threads = 2 * a.block_m * nh;
}

}  // namespace

const char *attn_fwd_limits(const FwdLaunch &a) {
  if (a.block_m != 128 && a.block_m != 256) return "forward Q tiles must have 128 or 256 rows";
  int64_t blocks;
  int threads;
  fwd_grid(a, &blocks, &threads);
  // a dispatch counts its work-items in 32 bits
  if (blocks * threads > int64_t(UINT32_MAX)) return "forward grid too large (Q tiles x KV heads x head groups)";
  // K / V row offsets inside a 64-row tile are 32-bit
  if (a.kv_row_stride > INT32_MAX / BN) return "kv_row_stride too large for 32-bit tile offsets";
  return nullptr;
}

hipError_t launch_attn_fwd(const FwdLaunch &a, hipStream_t stream) {
  if (attn_fwd_limits(a)) return hipErrorInvalidValue;
  FwdParams p;
  p.q = static_cast<const unsigned short *>(a.q);
  p.k = static_cast<const unsigned short *>(a.k);
  p.v = static_cast<const unsigned short *>(a.v);
  p.q_row_stride = a.q_row_stride;
  p.kv_row_stride = a.kv_row_stride;
  p.o = a.o;
  p.lse = a.lse;
  p.work = a.work;
  p.range = a.range;
  p.partners = a.partners;
  p.ds_q = a.ds_q;
  p.hq = a.hq;
  p.hkv = a.hkv;
  p.group = a.hq / a.hkv;
  p.tq = a.tq;
  p.n_groups = a.n_work * a.hkv;
  p.scale = a.scale;
  p.c = a.scale * LOG2E;
  // 128-row tiles: two query heads per workgroup when the GQA group is even;
  // 256-row tiles: one head, its 8 waves over the tile's rows. Either way
  // 8 waves share each staged K / V tile (4 for 128-row tiles, odd groups).
  const int tm = a.block_m;
  const int nh = tm == 128 && p.group % 2 == 0 ? 2 : 1;   // query heads per workgroup
  int64_t blocks;
  int threads;
  fwd_grid(a, &blocks, &threads);
  const dim3 grid{static_cast<unsigned>(blocks)}, block{static_cast<unsigned>(threads)};
#define SAP_FWD_LAUNCH(DD, MM, TT, HH) \
  hipLaunchKernelGGL((attn_fwd_kernel<DD, MM, TT, HH>), grid, block, 0, stream, p)
#define SAP_FWD_SHAPES(DD, MM)                                   \
  do {                                                           \
    if (tm == 256) SAP_FWD_LAUNCH(DD, MM, 256, 1);               \
    else if (nh == 2) SAP_FWD_LAUNCH(DD, MM, 128, 2);            \
    else SAP_FWD_LAUNCH(DD, MM, 128, 1);                         \
  } while (0)
  if (a.d == 128) {
    if (a.merge) SAP_FWD_SHAPES(128, true); else SAP_FWD_SHAPES(128, false);
  } else {
    if (a.merge) SAP_FWD_SHAPES(64, true); else SAP_FWD_SHAPES(64, false);
  }
#undef SAP_FWD_SHAPES
#undef SAP_FWD_LAUNCH
  return hipGetLastError();
}

}  // namespace sap
