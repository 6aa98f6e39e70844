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
// Layout of the work (one workgroup = one Q tile x one query head):
//   * 4 waves, each owns 32 query rows of the 128-row tile.
//   * Per 64-key KV tile: S^T = K Q^T with v_mfma_f32_32x32x16_bf16. In the
//     32x32 accumulator a lane holds one column (= one query) and 16 rows (=
//     keys), so a query's scores sit in one lane pair (lane, lane ^ 32): row
//     max/sum are in-register plus a single cross-half exchange.
//   * P^T (bf16) is already in the B-operand layout of O^T += V^T P^T, so P
//     never goes through LDS. V^T is the A operand: V is stored transposed
//     in LDS with the 4-key groups of every 16 keys ordered
//     (0-3, 8-11, 4-7, 12-15), which is the key order P^T's registers carry;
//     each operand is then a single 16-byte LDS read.
//   * K and V^T tiles are double-buffered in LDS: the next tile's global
//     loads are issued before the current tile's math, stored after it.
//   * Online softmax in fp32 with exp2 and the scale folded into one FMA.
//     The running max is only moved (and O, l rescaled) when it grows by
//     more than 2^8, which keeps the result exact (O / l normalises) while
//     skipping most rescales.
//   * Class FULL tiles skip masking; DIAGONAL masks key > query; PARTIAL also
//     masks keys before the query's document start; ragged tiles mask
//     columns past the tile end (their K/V rows are zero-filled).
//   * Workgroup ids are mapped so that the query heads sharing one KV head
//     and consecutive work items of one KV head land on the same XCD (ids
//     are dealt round-robin over the 8 XCDs), to share K/V in that XCD's L2.
#include <hip/hip_runtime.h>

#include <cmath>

#include "kernels.h"

namespace sap {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;

constexpr int BM = 128;
constexpr int BN = 64;
constexpr int NTHREADS = 256;
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

__device__ inline int perm16(int key) {
  // position of a key inside its 16-key group in the V^T LDS layout
  return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
}

template <int D>
struct Smem {
  static constexpr int KS = D + 8;        // K row stride (bf16 elements), padded
  static constexpr int VS = BN + 8;       // V^T row stride
  static constexpr int KBUF = BN * KS;
  static constexpr int VBUF = D * VS;
  static constexpr int BUF = KBUF + VBUF; // one stage
};

template <int D>
struct TileRegs {
  // K: D/32 chunks of 8 elements per thread; V: D/32 keys x 8 d per thread
  static constexpr int KL = D / 32;
  static constexpr int VL = D / 32;
  u32x4 kr[KL];
  u32x4 vr[VL];
};

// Per-thread element offsets of the KV tile loads, relative to the tile's
// first row of the KV head; loop-invariant for full 64-row tiles.
template <int D>
struct LoadOffsets {
  int k[D / 32];
  int v[D / 32];
};

template <int D>
__device__ inline LoadOffsets<D> load_offsets(int stride, int tid, int rows) {
  constexpr int CPR = D / 8;                 // 16-byte chunks per K row
  constexpr int RPI = NTHREADS / CPR;        // rows covered per pass
  constexpr int KPT = D / 32;                // consecutive keys per thread (V)
  constexpr int NKG = BN / KPT;              // key groups
  LoadOffsets<D> o;
  const int last = rows - 1;
#pragma unroll
  for (int i = 0; i < D / 32; ++i) o.k[i] = min(tid / CPR + RPI * i, last) * stride + 8 * (tid % CPR);
#pragma unroll
  for (int i = 0; i < KPT; ++i) o.v[i] = min((tid % NKG) * KPT + i, last) * stride + 8 * (tid / NKG);
  return o;
}

// Global -> register loads of one KV tile. Rows past a short tile's end are
// clamped to its last row (finite values; their scores are masked to -inf and
// their P is 0), so the loads need no per-row branches.
template <int D>
__device__ inline void load_tile(TileRegs<D> &r, const FwdParams &p, const PartnerEntry &pe, int g,
                                 int tid, const LoadOffsets<D> &full) {
  const int64_t base = int64_t(pe.local_start) * p.kv_row_stride + int64_t(g) * D;
  const unsigned short *kb = p.k + base;
  const unsigned short *vb = p.v + base;
  if (pe.n == BN) {
#pragma unroll
    for (int i = 0; i < D / 32; ++i) r.kr[i] = *reinterpret_cast<const u32x4 *>(kb + full.k[i]);
#pragma unroll
    for (int i = 0; i < D / 32; ++i) r.vr[i] = *reinterpret_cast<const u32x4 *>(vb + full.v[i]);
  } else {
    const LoadOffsets<D> o = load_offsets<D>(int(p.kv_row_stride), tid, pe.n);
#pragma unroll
    for (int i = 0; i < D / 32; ++i) r.kr[i] = *reinterpret_cast<const u32x4 *>(kb + o.k[i]);
#pragma unroll
    for (int i = 0; i < D / 32; ++i) r.vr[i] = *reinterpret_cast<const u32x4 *>(vb + o.v[i]);
  }
}

template <int D>
__device__ inline void store_tile(const TileRegs<D> &r, unsigned short *buf, int tid) {
  using S = Smem<D>;
  constexpr int CPR = D / 8;
  constexpr int RPI = NTHREADS / CPR;
  const int c = tid % CPR;
#pragma unroll
  for (int i = 0; i < TileRegs<D>::KL; ++i) {
    const int row = tid / CPR + RPI * i;
    *reinterpret_cast<u32x4 *>(buf + row * S::KS + 8 * c) = r.kr[i];
  }
  constexpr int KPT = D / 32;
  constexpr int NKG = BN / KPT;
  const int kg = tid % NKG, dc = tid / NKG;
  unsigned short *vt = buf + S::KBUF;
  const int key0 = kg * KPT;
  const int col = (key0 & ~15) | perm16(key0 & 15);
  // transpose: for each of the 8 d values gather the KPT keys' elements
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int w = j >> 1;
    const unsigned sel = (j & 1) ? 0x07060302u : 0x05040100u;
    unsigned short *dst = vt + (8 * dc + j) * S::VS + col;
    if constexpr (KPT == 4) {
      u32x2 pk;
      pk.x = __builtin_amdgcn_perm(r.vr[1][w], r.vr[0][w], sel);
      pk.y = __builtin_amdgcn_perm(r.vr[3][w], r.vr[2][w], sel);
      *reinterpret_cast<u32x2 *>(dst) = pk;
    } else {
      *reinterpret_cast<unsigned *>(dst) = __builtin_amdgcn_perm(r.vr[1][w], r.vr[0][w], sel);
    }
  }
}

__device__ inline bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// two fp32 -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32
__device__ inline unsigned pack_bf16(float lo, float hi) {
  const bf16x2 v = __builtin_convertvector(f32x2{lo, hi}, bf16x2);
  return __builtin_bit_cast(unsigned, v);
}

template <int D>
__global__ __launch_bounds__(NTHREADS) void attn_fwd_kernel(FwdParams p) {
  using S = Smem<D>;
  __shared__ __attribute__((aligned(16))) unsigned short lds[2 * S::BUF];

  // workgroup -> (work item, query head), XCD-aware
  const int b = blockIdx.x;
  const int xcd = b % NXCD, slot = b / NXCD;
  const int G = (slot / p.group) * NXCD + xcd;
  if (G >= p.n_groups) return;
  const int w = G / p.hkv, g = G % p.hkv;
  const int h = g * p.group + slot % p.group;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const WorkItem wi = p.work[w];
  const WorkRange rg = p.range[w];

  const int my_row = wave * 32 + l32;             // row within the Q tile
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

  TileRegs<D> regs;
  const LoadOffsets<D> full_offs = load_offsets<D>(int(p.kv_row_stride), tid, BN);
  const PartnerEntry *pes = p.partners + rg.begin;
  PartnerEntry pe = pes[0];
  load_tile<D>(regs, p, pe, g, tid, full_offs);
  store_tile<D>(regs, lds, tid);
  __syncthreads();

  for (int it = 0; it < rg.count; ++it) {
    const unsigned short *kbuf = lds + (it & 1) * S::BUF;
    const unsigned short *vbuf = kbuf + S::KBUF;
    const PartnerEntry cur = pe;
    const bool more = it + 1 < rg.count;
    if (more) {
      pe = pes[it + 1];
      load_tile<D>(regs, p, pe, g, tid, full_offs);
    }

    // S^T for 64 keys x this wave's 32 queries: two independent accumulator
    // chains (key blocks) interleaved so each LDS read is issued ahead of use
    f32x16 s[2] = {f32x16{}, f32x16{}};
    {
      const unsigned short *kp = kbuf + l32 * S::KS + 8 * hf;
#pragma unroll
      for (int t = 0; t < D / 16; ++t) {
        const bf16x8 a0 = as_bf16x8(*reinterpret_cast<const u32x4 *>(kp + 16 * t));
        const bf16x8 a1 = as_bf16x8(*reinterpret_cast<const u32x4 *>(kp + 32 * S::KS + 16 * t));
        s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[t], s[0], 0, 0, 0);
        s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[t], s[1], 0, 0, 0);
      }
    }

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
    mx = fmaxf(mx, __shfl_xor(mx, 32));
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

    // P = 2^(s c - m c); B operands of O^T += V^T P^T
    bf16x8 pb[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        float e[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          e[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][8 * u + j], c, -mc));
          l_part += e[j];
        }
        u32x4 pk;
        pk.x = pack_bf16(e[0], e[1]);
        pk.y = pack_bf16(e[2], e[3]);
        pk.z = pack_bf16(e[4], e[5]);
        pk.w = pack_bf16(e[6], e[7]);
        pb[kb][u] = as_bf16x8(pk);
      }

    // O^T += V^T P^T: the D/32 output blocks are independent chains, so the
    // inner loop over them keeps several MFMAs and LDS reads in flight
    {
      const unsigned short *vp = vbuf + l32 * S::VS + 8 * hf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4 *>(vp + db * 32 * S::VS + kb * 32 + 16 * u));
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kb][u], oacc[db], 0, 0, 0);
          }
    }

    if (more) store_tile<D>(regs, lds + ((it + 1) & 1) * S::BUF, tid);
    __syncthreads();
  }

  // epilogue: O = O / l, LSE = m * scale + ln l
  const float l = l_part + __shfl_xor(l_part, 32);
  if (!row_ok) return;
  const int row = wi.local_start + my_row;
  const bool empty = !(l > 0.f);
  const float inv = empty ? 0.f : 1.f / l;
  float *op = p.o + (int64_t(row) * p.hq + h) * D + 4 * hf;
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
  if (hf == 0) p.lse[int64_t(h) * p.tq + row] = empty ? -INFINITY : m_used * p.scale + __logf(l);
}

}  // namespace

hipError_t launch_attn_fwd(const FwdLaunch &a, hipStream_t stream) {
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
  const int64_t slots = (int64_t(p.n_groups) + NXCD - 1) / NXCD;
  const int64_t blocks = slots * NXCD * p.group;
  // 32-bit row offsets inside a 64-row tile
  if (blocks > INT32_MAX || a.kv_row_stride > INT32_MAX / BN) return hipErrorInvalidValue;
  const dim3 grid{static_cast<unsigned>(blocks)}, block{NTHREADS};
  if (a.d == 128)
    hipLaunchKernelGGL(attn_fwd_kernel<128>, grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL(attn_fwd_kernel<64>, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace sap
