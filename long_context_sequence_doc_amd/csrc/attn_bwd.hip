// Backward kernels (recompute form) for document-masked causal attention on
// gfx950 bf16 matrix cores.
//
// The forward keeps only O and the log-sum-exp; the backward recomputes the
// probabilities from them -- the attention-level echo of the AutoSP page's
// section 2.B (gist.science/zh/paper/2604.27089: keep attention's saved
// state, recompute instead of storing the big intermediates). With the
// final, all-KV LSE and O of each query row:
//     P = exp(scale q.k - LSE)                  on allowed pairs (else 0)
//     D_r = dO_r . O_r                          (bwd_rowterm_kernel)
//     dV += P^T dO,   dS = P o (dO V^T - D),   dK += scale dS^T Q,   dQ += scale dS K
// so per-step calls of a ring sum to the full gradient.
//
// Two kernels share the work so that no output needs atomics (device-scope
// atomics from the 8 XCDs cannot stay in their L2s and go out to memory):
//
// attn_bwd_kv_kernel -- dK, dV. One workgroup = one chunk of a 128-key KV
//   tile's partner Q tiles x one KV head; 8 waves = 4 key groups (32 keys)
//   x 2 row blocks (32 rows of each 64-row Q tile). The K / V tile sits in
//   LDS for the whole workgroup and the Q / dO rows of each (Q tile, query
//   head) iteration arrive by direct global -> LDS copies into a double
//   buffer. S = Q K^T and dP = dO V^T (K / V rows as B operands) leave the
//   32x32 accumulators with keys across lanes and queries across registers
//   -- exactly the B-operand layout of dV^T += dO^T P and dK^T += Q^T dS,
//   whose A operands dO^T, Q^T come from transposing LDS reads. The two row
//   blocks' dK / dV partial sums are added through LDS at the end and
//   written once. Two waves per SIMD (each holds only its keys' dK^T / dV^T
//   accumulators). KV tiles with many partners are split into several
//   chunks by the planner (so the pass has enough workgroups), cut on a
//   fixed grid of Q tiles and walked from the last Q tile down, so the
//   workgroups an XCD runs side by side stream the same Q / dO rows through
//   its L2; split tiles' chunks store partial sums in workspace slots and
//   bwd_kv_reduce_kernel adds the slots up in order, so the result stays
//   deterministic. Each iteration issues the next stage's copies after its
//   S / dP products, so the waves' wait for the memory pipeline to take them
//   runs beside the matrix work.
//
// attn_bwd_dq_kernel -- dQ. One workgroup = one Q tile x one, two or four
//   query heads of a KV head: with four heads the plan's 64-row Q tiles, with
//   one or two its 128-row list (the same rows, paired; consecutive 64-row
//   tiles nearly always meet the same 128-key KV tiles), so each staged K / V
//   part serves at least 256 query rows x heads. One wave per 32 query rows
//   and head; the waves walk the KV tiles that meet the Q tile, in parts of
//   128 keys (eight waves), 64 (four) or 32 (two) copied straight into a
//   double-buffered LDS stage shared by the heads. As in the forward,
//   S^T = K Q^T and dP^T = V dO^T put one query per lane pair, P^T and dS^T
//   come out in the B-operand layout of dQ^T += K^T dS^T, whose K^T operand
//   comes from transposing LDS reads. Each workgroup owns its dQ rows: the
//   result is added once at the end with plain loads and stores.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>
#include <cmath>
#include <mutex>
#include <type_traits>

#include "kernels.h"
#include "lds_copy.h"

// Device scratch of the allocation-free backward (sap_attn_bwd_noalloc): the
// row terms and split-tile partial sums that sap_attn_bwd keeps in the
// caller's workspace. One copy per GPU, held until the process ends. Host
// code never passes this name to a kernel (on the host it is only a stand-in
// for the symbol): its device address comes from hipGetSymbolAddress, once
// per device (noalloc_scratch below).
static __device__ __align__(256) unsigned char scratch[sap::kNoAllocScratchBytes];

namespace sap {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int BMB = 64;     // query rows per Q tile
constexpr int BNB = 128;    // keys per KV tile
constexpr int NT = 256;     // threads of the KV kernel
constexpr int NXCD = 8;
constexpr float LOG2E = 1.4426950408889634f;

__device__ inline bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

// f(integral_constant<int, i>) for i = 0 .. N-1, unrolled at compile time
// (the index can then feed immediate instruction operands)
template <int N, int I = 0, class F>
__device__ inline void static_for(F &&f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

__device__ inline unsigned pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// ---------------------------------------------------------------------------
// D_r = sum_d dO[r,h,d] * O[r,h,d] for the rows of the plan's Q tiles.
// d / 8 threads per (row, head), each one 16-byte load of dO (8 bf16) and
// two of O (8 fp32), then a butterfly over the group.
__global__ __launch_bounds__(NT) void bwd_rowterm_kernel(const unsigned short *dout, int64_t q_row_stride,
                                                         const float *o, float *delta, const int32_t *tiles,
                                                         int32_t hq, int32_t d, int32_t tq) {
  const int r0 = tiles[2 * blockIdx.x], n = tiles[2 * blockIdx.x + 1];
  const int tpp = d / 8;                           // threads per (row, head): a power of two <= 64
  const int pair = blockIdx.y * (NT / tpp) + threadIdx.x / tpp;   // (row, head) index inside the tile
  const int sub = threadIdx.x % tpp;
  if (pair >= n * hq) return;                      // whole groups leave together
  const int row = r0 + pair / hq, h = pair % hq;
  const u32x4 dv = *reinterpret_cast<const u32x4 *>(dout + int64_t(row) * q_row_stride + int64_t(h) * d + 8 * sub);
  const float *op = o + (int64_t(row) * hq + h) * d + 8 * sub;
  const f32x4 o0 = *reinterpret_cast<const f32x4 *>(op), o1 = *reinterpret_cast<const f32x4 *>(op + 4);
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = __builtin_bit_cast(float, dv[i] << 16), hi = __builtin_bit_cast(float, dv[i] & 0xffff0000u);
    acc += lo * (i < 2 ? o0[2 * i] : o1[2 * i - 4]) + hi * (i < 2 ? o0[2 * i + 1] : o1[2 * i - 3]);
  }
  for (int m = tpp / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, tpp);
  if (sub == 0) delta[int64_t(h) * tq + row] = acc;
}

// ---------------------------------------------------------------------------
struct BwdParams {
  const unsigned short *q, *k, *v, *dout;
  const float *lse, *delta;
  int64_t q_row_stride, kv_row_stride;
  float *dq, *dk, *dv;
  const WorkItem *work;
  const WorkRange *range;
  const PartnerEntry *partners;
  const int32_t *ds_q;
  const int32_t *slot;     // KV-major chunks: workspace slot (-1: add into dk / dv directly)
  float *partial;          // [2][n_slots][hkv][BNB][D]: unscaled dK^T, then dV^T partial sums
  int32_t n_slots;
  int32_t hq, hkv, group, tq, n_work;
  float scale, c;   // c = scale * log2(e)
};

// LDS tile of BMB rows x D bf16, row-major and unpadded, filled by direct
// global -> LDS copies (16 bytes per lane, lane order). Chunk j (16 bytes)
// of row r sits at chunk position j ^ sw(r). With 16 chunks a row (one
// 256-byte bank line), sw(r) = 4 (r % 4) + (r / 4) % 4 is a bijection on any
// 16 consecutive rows, so the row-operand reads (ds_read_b128: 16 rows, one
// chunk each per cycle) hit 16 distinct bank groups, and any 4 rows r0..r0+3
// (r0 % 4 == 0) put 4 adjacent chunks on 16 distinct positions (transposing
// reads, ds_read_b64_tr_b16: 4 rows x 4 chunks per half-wave). Rows 8 apart
// differ in chunk bit 1 only (TR8: the byte offset of the +8-row read).
// With 8 chunks a row, sw(r) = 2 (r % 4) + (r / 4) % 2.
template <int D>
struct RowTile {
  static constexpr int CPR = D / 8;                  // 16-byte chunks per row
  static constexpr int ROW = 2 * D;                  // bytes per row
  static constexpr int BYTES = BMB * ROW;
  static constexpr int TR8 = 32;                     // sw(r + 8) = sw(r) ^ 2 (r % 16 < 8, 16 chunks)
  static __device__ int sw(int r) {
    return CPR >= 16 ? 4 * (r & 3) + ((r >> 2) & 3) : 2 * (r & 3) + ((r >> 2) & 1);
  }
};

template <int D>
struct KvStage {
  static constexpr int Q = 0;                        // Q rows of the (Q tile, head)
  static constexpr int DO = RowTile<D>::BYTES;       // dO rows
  static constexpr int LSE2 = 2 * RowTile<D>::BYTES; // float[BMB]: LSE * log2(e) (+inf: row sees no key)
  static constexpr int DELTA = LSE2 + 4 * BMB;       // float[BMB]
  static constexpr int DS = DELTA + 4 * BMB;         // int[BMB]: document start (INT_MIN unless PARTIAL)
  static constexpr int BYTES = DS + 4 * BMB;
};

constexpr int NTK = 512;    // threads of the KV kernel: 8 waves = 4 key groups x 2 row blocks

template <int D>
__global__ __launch_bounds__(NTK) void attn_bwd_kv_kernel(BwdParams p) {
  using RT = RowTile<D>;
  using KS = KvStage<D>;
  constexpr int NW = NTK / 64;
  constexpr int KVT = BNB * RT::ROW;                 // bytes of the K (or V) tile
  constexpr int STAGE = (KS::BYTES + 1023) & ~1023;
  constexpr int ST0 = 2 * KVT;                       // first Q / dO stage
  constexpr int BYTES = ST0 + 2 * STAGE;
  static_assert(BYTES >= 2 * (BNB * D * 4), "the dK / dV exchange reuses the buffers");
  __shared__ __attribute__((aligned(1024))) unsigned char lds[BYTES];

  const int w = blockIdx.x / p.hkv, g = blockIdx.x % p.hkv;
  if (w >= p.n_work) return;
  const WorkItem kt = p.work[w];
  const WorkRange rg = p.range[w];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);   // the same, in a scalar register
  const int k4 = wave & 3, qb = wave >> 2;           // key group (32 keys) and Q row block (32 rows)

  // this wave's keys: local key index k4*32 + l32 within the tile
  const int my_key = k4 * 32 + l32;
  const bool key_ok = my_key < kt.n;
  const int kg = kt.global_start + my_key;
  const int64_t kv_base = int64_t(kt.local_start) * p.kv_row_stride + int64_t(g) * D;

  f32x16 dka[D / 32], dva[D / 32];     // dK^T / dV^T blocks over this wave's rows: lane = key, registers = d
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    dka[i] = f32x16{};
    dva[i] = f32x16{};
  }
  const float c = p.c;

  // The K / V tile (BNB rows) is copied once into LDS; the Q / dO rows of
  // each iteration into a double-buffered stage. Copy geometry of a tile:
  // chunk position P = (i * NW + wave) * 64 + lane holds row P / CPR, chunk
  // (P % CPR) ^ sw(row).
  {
    constexpr int KL = BNB * RT::CPR / NTK;
#pragma unroll
    for (int i = 0; i < KL; ++i) {
      const int P = (i * NW + wave) * 64 + lane;
      const int row = P / RT::CPR;
      const int64_t off = kv_base + int64_t(min(row, kt.n - 1)) * p.kv_row_stride + 8 * ((P % RT::CPR) ^ RT::sw(row));
      const int dst = (i * NW + wave_s) * 1024;
      copy_to_lds(p.k + off, lds, dst);
      copy_to_lds(p.v + off, lds, KVT + dst);
    }
  }
  constexpr int LOADS = BMB * RT::CPR / NTK;
  static_assert(LOADS >= 1 && LOADS * NTK == BMB * RT::CPR, "Q / dO copies must split evenly");
  int src_row[LOADS], src_col[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int P = (i * NW + wave) * 64 + lane;
    src_row[i] = P / RT::CPR;
    src_col[i] = 8 * ((P % RT::CPR) ^ RT::sw(P / RT::CPR));
  }
  // Row-operand reads: A of S = Q K^T, dP = dO V^T (row qb*32 + l32, chunk
  // 2t + hf) and B = K / V rows of this wave's keys (row k4*32 + l32); the
  // swizzle depends on the low 4 row bits only, so both are r_off-based and
  // the offset of k-step t is off ^ (32 t).
  const int r_off = l32 * RT::ROW + 16 * (hf ^ RT::sw(l32));
  const int a_off = qb * 32 * RT::ROW + r_off;
  const int b_off = k4 * 32 * RT::ROW + r_off;
  // Transposing reads (A of dV^T += dO^T P, dK^T += Q^T dS): within each
  // 16-lane group q, lane s addresses row 4 (q / 2) + s / 4 (+ the step's
  // base, a multiple of 8) and columns 16 (q % 2) + 4 (s % 4) .. +3 of the
  // 32-column block db; it receives the 4 rows of column 16 (q % 2) + s.
  // The +8-row read of a pair flips chunk bit 1 of the swizzle (byte offset
  // XOR TR8, rows of 16 chunks only).
  int t_off[D / 32];
  {
    const int q4 = lane >> 4, s16 = lane & 15;
    const int row = 4 * (q4 >> 1) + (s16 >> 2);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int col = db * 32 + 16 * (q4 & 1) + 4 * (s16 & 3);
      t_off[db] = row * RT::ROW + 16 * ((col >> 3) ^ RT::sw(row)) + 2 * (col & 7);
    }
  }
  // per-lane transposing-read offsets of this wave's row block: rows
  // qb*32 + (0..7) and, for the second read of a pair, + 8
  int t_lo[D / 32], t_hi[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    t_lo[db] = t_off[db] + qb * 32 * RT::ROW;
    t_hi[db] = (RT::CPR >= 16 ? (t_off[db] ^ RT::TR8) : t_off[db]) + (qb * 32 + 8) * RT::ROW;
  }

  // The (Q tile, query head) iterations run in order it * group + hi.
  // Partner entries come through the scalar cache (the index is uniform), so
  // no vector load has to wait behind the in-flight row copies.
  const int n_iter = rg.count * p.group;
  typedef __attribute__((address_space(4))) const PartnerEntry const_entry;
  const const_entry *cpart = (const const_entry *)p.partners;
  const int pbase = __builtin_amdgcn_readfirstlane(rg.begin);
  auto entry = [&](int itr) {
    const const_entry &e = cpart[__builtin_amdgcn_readfirstlane(pbase + itr / p.group)];
    return PartnerEntry{e.local_start, e.global_start, e.n, e.cls};
  };
  auto issue_rows = [&](int itr, int stage) {   // stage: byte offset in lds
    const PartnerEntry t = entry(itr);
    const int hh = g * p.group + itr % p.group;
    const int64_t base = int64_t(t.local_start) * p.q_row_stride + int64_t(hh) * D;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int64_t off = base + int64_t(min(src_row[i], t.n - 1)) * p.q_row_stride + src_col[i];
      copy_to_lds(p.q + off, lds, stage + KS::Q + (i * NW + wave_s) * 1024);
      copy_to_lds(p.dout + off, lds, stage + KS::DO + (i * NW + wave_s) * 1024);
    }
  };
  // per-row terms of one iteration (threads 0..BMB-1, one row each): loaded
  // raw at the start of the previous iteration and turned into the stage's
  // form only when stored at its end, so nothing waits for them (or for the
  // row copies issued before them) in between
  float rt_l = 0.f, rt_d = 0.f;
  int rt_s = 0;
  PartnerEntry rt_t{};
  auto load_terms = [&](int itr) {
    rt_t = entry(itr);
    const int hh = g * p.group + itr % p.group;
    const int row = min(tid, rt_t.n - 1);
    const int64_t li = int64_t(hh) * p.tq + rt_t.local_start + row;
    rt_l = p.lse[li];
    rt_d = p.delta[li];
    // document start bounds keys only in PARTIAL tiles
    rt_s = rt_t.cls == SAP_TILE_PARTIAL ? p.ds_q[rt_t.local_start + row] : INT_MIN;
  };
  auto store_terms = [&](unsigned char *stage) {
    // rows past the tile end or with no key at all get P = 0
    reinterpret_cast<float *>(stage + KS::LSE2)[tid] = (tid < rt_t.n && rt_l != -INFINITY) ? rt_l * LOG2E : INFINITY;
    reinterpret_cast<float *>(stage + KS::DELTA)[tid] = rt_d;
    reinterpret_cast<int *>(stage + KS::DS)[tid] = rt_s;
  };

  issue_rows(0, ST0);
  if (tid < BMB) {
    load_terms(0);
    store_terms(lds + ST0);
  }
  wait_copies();
  __syncthreads();

  for (int itr = 0; itr < n_iter; ++itr) {
    const PartnerEntry qt = entry(itr);
    unsigned char *cur = lds + ST0 + (itr & 1) * STAGE;
    unsigned char *nxt = lds + ST0 + ((itr + 1) & 1) * STAGE;
    const bool more = itr + 1 < n_iter;

    // ---- S = Q K^T, dP = dO V^T (this wave's 32 rows x 32 keys)
    f32x16 sacc = f32x16{}, pacc = f32x16{};
    {
      auto rd = [&](const unsigned char *base, int off) { return as_bf16x8(*reinterpret_cast<const u32x4 *>(base + off)); };
      bf16x8 aq = rd(cur + KS::Q, a_off), ad = rd(cur + KS::DO, a_off), bk = rd(lds, b_off), bv = rd(lds + KVT, b_off);
#pragma unroll
      for (int t = 0; t < D / 16; ++t) {
        bf16x8 naq = aq, nad = ad, nbk = bk, nbv = bv;
        if (t + 1 < D / 16) {
          naq = rd(cur + KS::Q, a_off ^ (32 * (t + 1)));
          nad = rd(cur + KS::DO, a_off ^ (32 * (t + 1)));
          nbk = rd(lds, b_off ^ (32 * (t + 1)));
          nbv = rd(lds + KVT, b_off ^ (32 * (t + 1)));
        }
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, bk, sacc, 0, 0, 0);
        pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ad, bv, pacc, 0, 0, 0);
        aq = naq; ad = nad; bk = nbk; bv = nbv;
      }
    }

    // the next stage's copies and row terms, issued while the matrix cores
    // work through S and dP (all waves issue them at the same point, and the
    // memory pipeline takes them in turn)
    if (more) {
      issue_rows(itr + 1, ST0 + ((itr + 1) & 1) * STAGE);
      if (tid < BMB) load_terms(itr + 1);
    }

    // ---- P and dS; accumulator element i is query row
    //      qb*32 + 8*(i/4) + 4*hf + (i%4), key my_key. The per-row terms of a
    //      lane's 16 rows come as four 4-row vector reads.
    const bool masked = qt.cls != SAP_TILE_FULL || qt.n < BMB || kt.n < BNB;
    // a row r sees this lane's key iff r >= rmin (causality; invalid keys see
    // no row) and kg >= ds[r] (document start; INT_MIN unless PARTIAL)
    const int rmin = key_ok ? kg - qt.global_start : (1 << 30);
    const float *s_lse2 = reinterpret_cast<const float *>(cur + KS::LSE2);
    const float *s_delta = reinterpret_cast<const float *>(cur + KS::DELTA);
    const int *s_ds = reinterpret_cast<const int *>(cur + KS::DS);
    bf16x8 pb[2], sb[2];
    auto p_and_ds = [&](auto mask_tag) {
      constexpr bool MASK = decltype(mask_tag)::value;
      f32x4 l4[4], d4[4];
      int ds4[4][4];
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int r0 = qb * 32 + 8 * g4 + 4 * hf;
        l4[g4] = *reinterpret_cast<const f32x4 *>(s_lse2 + r0);
        d4[g4] = *reinterpret_cast<const f32x4 *>(s_delta + r0);
        if (MASK) {
          const u32x4 dsv = *reinterpret_cast<const u32x4 *>(s_ds + r0);
#pragma unroll
          for (int e = 0; e < 4; ++e) ds4[g4][e] = int(dsv[e]);
        }
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        float pv[8], sv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int i = 8 * u + j;
          const int g4 = i >> 2, e = i & 3;
          float x = __builtin_fmaf(sacc[i], c, -l4[g4][e]);
          if (MASK) {          // masked pairs: exp2(-inf) = 0 (a select, not a branch)
            const int r = qb * 32 + 8 * g4 + 4 * hf + e;
            x = ((r >= rmin) & (kg >= ds4[g4][e])) ? x : -INFINITY;
          }
          const float pr = __builtin_amdgcn_exp2f(x);
          pv[j] = pr;
          sv[j] = pr * (pacc[i] - d4[g4][e]);
        }
        u32x4 pk, sk;
        pk.x = pack_bf16(pv[0], pv[1]);
        pk.y = pack_bf16(pv[2], pv[3]);
        pk.z = pack_bf16(pv[4], pv[5]);
        pk.w = pack_bf16(pv[6], pv[7]);
        sk.x = pack_bf16(sv[0], sv[1]);
        sk.y = pack_bf16(sv[2], sv[3]);
        sk.z = pack_bf16(sv[4], sv[5]);
        sk.w = pack_bf16(sv[6], sv[7]);
        pb[u] = as_bf16x8(pk);
        sb[u] = as_bf16x8(sk);
      }
    };
    if (masked)
      p_and_ds(std::true_type{});
    else
      p_and_ds(std::false_type{});

    // ---- dV^T += dO^T P, dK^T += Q^T dS (k = 16 query rows per step; the
    //      rows of step u are qb*32 + 16u + 4hf + (0..3 | 8..11))
    {
      // one offset per 32-column block and read of a pair; the tile (dO or
      // Q) and the 16-row step are constants the reads take as immediates
      auto rd = [&](int t, int imm) { return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(cur + t + imm)); };
      auto join = [](const i16x4 &lo, const i16x4 &hi) {
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      static_for<2 * (D / 32)>([&](auto kc) {
        constexpr int k = decltype(kc)::value;
        constexpr int u = k / (D / 32), db = k % (D / 32);
        constexpr int odo = KS::DO + 16 * u * RT::ROW, oq = KS::Q + 16 * u * RT::ROW;
        dva[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(join(rd(t_lo[db], odo), rd(t_hi[db], odo)), pb[u], dva[db], 0, 0, 0);
        dka[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(join(rd(t_lo[db], oq), rd(t_hi[db], oq)), sb[u], dka[db], 0, 0, 0);
      });
      // schedule: the reads of step k + 1 go out before the products of step k
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      static_for<2 * (D / 32)>([&](auto kc) {
        __builtin_amdgcn_sched_group_barrier(0x100, decltype(kc)::value + 1 < 2 * (D / 32) ? 4 : 0, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      });
    }

    // the next iteration's row terms (loaded above, latency hidden by the math)
    if (more && tid < BMB) store_terms(nxt);
    // copies for the next iteration have landed and every wave is done with this stage
    wait_copies();
    __syncthreads();
  }

  // ---- the two row blocks' partial sums meet in LDS: row block 1 stores its
  //      registers lane-minor ([k4][register quad][lane] float4s), row block 0
  //      adds them
  f32x4 *xk = reinterpret_cast<f32x4 *>(lds);
  f32x4 *xv = xk + 4 * (D / 8) * 64;
  if (qb == 1) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int ig = 0; ig < 4; ++ig) {
        const int idx = (k4 * (D / 8) + db * 4 + ig) * 64 + lane;
        f32x4 a, b;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[e] = dka[db][4 * ig + e];
          b[e] = dva[db][4 * ig + e];
        }
        xk[idx] = a;
        xv[idx] = b;
      }
  }
  __syncthreads();
  if (qb == 1) return;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int ig = 0; ig < 4; ++ig) {
      const int idx = (k4 * (D / 8) + db * 4 + ig) * 64 + lane;
      const f32x4 a = xk[idx], b = xv[idx];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dka[db][4 * ig + e] += a[e];
        dva[db][4 * ig + e] += b[e];
      }
    }

  if (!key_ok) return;
  const int slot = p.slot[w];
  if (slot >= 0) {
    // ---- one chunk of a split KV tile: its partial sums go to the slot
    const int64_t rows = int64_t(p.n_slots) * p.hkv * BNB;
    float *pk = p.partial + ((int64_t(slot) * p.hkv + g) * BNB + my_key) * D + 4 * hf;
    float *pv = pk + rows * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int ig = 0; ig < 4; ++ig) {
        const int off = db * 32 + 8 * ig;
        f32x4 a, b;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[e] = dka[db][4 * ig + e];
          b[e] = dva[db][4 * ig + e];
        }
        *reinterpret_cast<f32x4 *>(pk + off) = a;
        *reinterpret_cast<f32x4 *>(pv + off) = b;
      }
    return;
  }
  // ---- dK += scale dK^T, dV += dV^T for this wave's keys
  float *dkp = p.dk + (int64_t(kt.local_start + my_key) * p.hkv + g) * D + 4 * hf;
  float *dvp = p.dv + (int64_t(kt.local_start + my_key) * p.hkv + g) * D + 4 * hf;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int ig = 0; ig < 4; ++ig) {
      const int off = db * 32 + 8 * ig;
      f32x4 a = *reinterpret_cast<f32x4 *>(dkp + off);
      f32x4 b = *reinterpret_cast<f32x4 *>(dvp + off);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a[e] += p.scale * dka[db][4 * ig + e];
        b[e] += dva[db][4 * ig + e];
      }
      *reinterpret_cast<f32x4 *>(dkp + off) = a;
      *reinterpret_cast<f32x4 *>(dvp + off) = b;
    }
}

// ---------------------------------------------------------------------------
// dK += scale * sum of a split KV tile's partial dK^T slots, dV += sum of its
// dV^T slots, the slots added in order (deterministic). One workgroup per
// (split tile, KV head, group of RK keys); each thread handles 4 consecutive
// d of one key.
constexpr int RK = 16;
__global__ __launch_bounds__(NT) void bwd_kv_reduce_kernel(const ReduceItem *items, const float *partial,
                                                           int32_t n_slots, int32_t hkv, int32_t d, float scale,
                                                           float *dk, float *dv) {
  const ReduceItem it = items[blockIdx.x / hkv];
  const int g = blockIdx.x % hkv;
  const int k0 = blockIdx.y * RK;
  if (k0 >= it.n) return;
  const int64_t slot_stride = int64_t(hkv) * BNB * d;            // floats per slot
  const float *pk = partial + (int64_t(it.slot_begin) * hkv + g) * BNB * d;
  const float *pv = pk + int64_t(n_slots) * slot_stride;
  const int quads = min(RK, it.n - k0) * (d / 4);
  for (int idx = threadIdx.x; idx < quads; idx += NT) {
    const int key = k0 + idx / (d / 4), e4 = 4 * (idx % (d / 4));
    f32x4 sk = *reinterpret_cast<const f32x4 *>(pk + key * d + e4);
    f32x4 sv = *reinterpret_cast<const f32x4 *>(pv + key * d + e4);
    for (int c = 1; c < it.slot_count; ++c) {
      sk += *reinterpret_cast<const f32x4 *>(pk + c * slot_stride + key * d + e4);
      sv += *reinterpret_cast<const f32x4 *>(pv + c * slot_stride + key * d + e4);
    }
    const int64_t o = (int64_t(it.local_start + key) * hkv + g) * d + e4;
    f32x4 a = *reinterpret_cast<f32x4 *>(dk + o);
    f32x4 b = *reinterpret_cast<f32x4 *>(dv + o);
    a += scale * sk;
    b += sv;
    *reinterpret_cast<f32x4 *>(dk + o) = a;
    *reinterpret_cast<f32x4 *>(dv + o) = b;
  }
}

// ---------------------------------------------------------------------------
constexpr int HK = 64;      // keys per half of a KV tile in the dQ kernel

// dQ kernel: one workgroup = one 64-row Q tile x NH query heads of one KV
// head (NH = 4 when the GQA group size is a multiple of 4, else 2 when it is
// even, so 8 or 4 waves share each staged K / V part-tile). Wave w owns head hq0 + w / 2, rows 32 (w % 2) ..
// +31. Per part of a partner KV tile (64 keys with two or four heads; 32 with one,
// so four 2-wave workgroups fit a CU), staged by direct copies into a
// double-buffered LDS stage (K rows, V rows; swizzled as RowTile):
//   S^T = K Q^T, dP^T = V dO^T            (A: K / V rows, B: Q / dO in registers)
//   dS^T = P^T o (dP^T - D)               (one query per lane pair: LSE, D scalars)
//   dQ^T += K^T dS^T                      (A: K^T by transposing reads of K rows)
// TQ: rows of the Q tiles (64: the plan's own; 128: its 128-row list), one
// wave per 32 rows and head.
template <int D, int NH, int TQ>
__global__ __launch_bounds__(2 * TQ * NH) void attn_bwd_dq_kernel(BwdParams p) {
  using RT = RowTile<D>;
  constexpr int WPH = TQ / 32;                       // waves per head
  constexpr int NWV = WPH * NH;                      // waves
  constexpr int NTD = 64 * NWV;                      // threads
  // keys per stage: a whole 128-key KV tile with eight waves per workgroup
  // (one workgroup per CU, 128 KB of LDS; half the barriers per key); 64
  // (half a tile) with four waves (two workgroups per CU); 32 with two (four)
  constexpr int HKQ = NWV >= 8 ? 2 * HK : NWV >= 4 ? HK : HK / 2;
  constexpr int KBQ = HKQ / 32;                      // 32-key blocks per stage
  constexpr int KOFF = 0, VOFF = HKQ * RT::ROW;      // K, V part-tiles (RowTile rows)
  constexpr int STAGE = 2 * HKQ * RT::ROW;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[2 * STAGE];

  // workgroup -> (Q tile, head pair); the head pairs of one KV head and
  // consecutive Q tiles of one KV head go to the same XCD (ids are dealt
  // round-robin over the XCDs), to share K / V in its L2
  const int pairs = p.group / NH;
  const int b = blockIdx.x;
  const int xcd = b % NXCD, slot = b / NXCD;
  const int G = (slot / pairs) * NXCD + xcd;
  if (G >= p.n_work * p.hkv) return;
  const int w = G / p.hkv, g = G % p.hkv;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);   // the same, in a scalar register
  const int h = g * p.group + (slot % pairs) * NH + wave / WPH;
  const WorkItem qt = p.work[w];
  const WorkRange rg = p.range[w];

  const int my_row = (wave % WPH) * 32 + l32;     // query row within the Q tile
  const bool row_ok = my_row < qt.n;
  const int qrow = qt.local_start + min(my_row, qt.n - 1);
  const int qg = qt.global_start + my_row;
  const int dsq = p.ds_q[qrow];
  const float lse = p.lse[int64_t(h) * p.tq + qrow];
  // rows past the tile end or with no key at all get P = 0
  const float lse2 = (row_ok && lse != -INFINITY) ? lse * LOG2E : INFINITY;
  const float dlt = p.delta[int64_t(h) * p.tq + qrow];

  // this lane's Q and dO fragments: B operands of S^T = K Q^T and dP^T = V dO^T
  bf16x8 qf[D / 16], of[D / 16];
  {
    const int64_t off = int64_t(qrow) * p.q_row_stride + int64_t(h) * D + 8 * hf;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      qf[t] = as_bf16x8(*reinterpret_cast<const u32x4 *>(p.q + off + 16 * t));
      of[t] = as_bf16x8(*reinterpret_cast<const u32x4 *>(p.dout + off + 16 * t));
    }
  }
  f32x16 qacc[D / 32];                            // dQ^T blocks: lane = query, registers = d
#pragma unroll
  for (int i = 0; i < D / 32; ++i) qacc[i] = f32x16{};
  const float c = p.c;

  // copy geometry of a half-tile (see RowTile): chunk position
  // P = (i * NWV + wave) * 64 + lane holds row P / CPR, chunk (P % CPR) ^ sw(row)
  constexpr int LOADS = HKQ * RT::CPR / NTD;
  static_assert(LOADS * NTD == HKQ * RT::CPR, "copies must split evenly");
  int src_row[LOADS], src_col[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int P = (i * NWV + wave) * 64 + lane;
    src_row[i] = P / RT::CPR;
    src_col[i] = 8 * ((P % RT::CPR) ^ RT::sw(P / RT::CPR));
  }
  const int r_off = l32 * RT::ROW + 16 * (hf ^ RT::sw(l32));
  int t_off[D / 32];
  {
    const int q4 = lane >> 4, s16 = lane & 15;
    const int row = 4 * (q4 >> 1) + (s16 >> 2);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int col = db * 32 + 16 * (q4 & 1) + 4 * (s16 & 3);
      t_off[db] = row * RT::ROW + 16 * ((col >> 3) ^ RT::sw(row)) + 2 * (col & 7);
    }
  }
  auto issue_half = [&](const PartnerEntry &kt, int half, int stage) {   // stage: byte offset in lds
    const int kn = min(HKQ, kt.n - half * HKQ);
    const int64_t base = int64_t(kt.local_start + half * HKQ) * p.kv_row_stride + int64_t(g) * D;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int64_t off = base + int64_t(min(src_row[i], kn - 1)) * p.kv_row_stride + src_col[i];
      const int dst = (i * NWV + wave_s) * 1024;
      copy_to_lds(p.k + off, lds, stage + KOFF + dst);
      copy_to_lds(p.v + off, lds, stage + VOFF + dst);
    }
  };

  // partner entries through the scalar cache (uniform index): no vector
  // load waits behind the in-flight copies
  typedef __attribute__((address_space(4))) const PartnerEntry const_entry;
  const const_entry *cpart = (const const_entry *)p.partners;
  const int pbase = __builtin_amdgcn_readfirstlane(rg.begin);
  auto entry = [&](int i) {
    const const_entry &e = cpart[__builtin_amdgcn_readfirstlane(pbase + i)];
    return PartnerEntry{e.local_start, e.global_start, e.n, e.cls};
  };

  // iterations: the 64-key halves of the partner tiles, in order
  int it = 0, half = 0, stage_i = 0;
  if (rg.count > 0) issue_half(entry(0), 0, 0);
  wait_copies();
  __syncthreads();
  while (it < rg.count) {
    const PartnerEntry kt = entry(it);
    unsigned char *cur = lds + stage_i * STAGE;
    // the next half: this tile's second one, or the next tile's first
    int nit = it, nhalf = half + 1;
    if (nhalf * HKQ >= kt.n) {
      nit = it + 1;
      nhalf = 0;
    }
    const int k0 = half * HKQ;                    // first key of this part within the tile
    const int kn = min(HKQ, kt.n - k0);           // keys in this part

    // The stage's keys go in 32-key blocks, each through S^T / dP^T, dS^T and
    // its dQ^T steps before the next, so only one block's score
    // accumulators are live (room for the unmasked path of FULL tiles).
    const bool masked = kt.cls != SAP_TILE_FULL || kn < HKQ || qt.n < TQ;
    int lo = -(1 << 30), hi = kn - 1;             // allowed stage-local key range of this query
    if (masked) {
      if (kt.cls != SAP_TILE_FULL) hi = min(hi, qg - (kt.global_start + k0));
      if (kt.cls == SAP_TILE_PARTIAL) lo = dsq - (kt.global_start + k0);
    }
    const int hi_r = hi - 4 * hf, lo_r = lo - 4 * hf;
    // transposing reads of K^T: one offset per 32-column block and read of
    // a pair, the 16-key step a constant the reads take as an immediate
    int k_lo[D / 32], k_hi[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      k_lo[db] = KOFF + t_off[db];
      k_hi[db] = KOFF + (RT::CPR >= 16 ? (t_off[db] ^ RT::TR8) : t_off[db]) + 8 * RT::ROW;
    }
    auto rd = [&](int t, int imm) { return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(cur + t + imm)); };
    static_for<KBQ>([&](auto kbc) {
      constexpr int kb = decltype(kbc)::value;
      // ---- S^T = K Q^T, dP^T = V dO^T (32 keys x this wave's 32 queries)
      f32x16 sacc = f32x16{}, pacc = f32x16{};
#pragma unroll
      for (int t = 0; t < D / 16; ++t) {
        const int off = kb * 32 * RT::ROW + (r_off ^ (32 * t));
        const bf16x8 ak = as_bf16x8(*reinterpret_cast<const u32x4 *>(cur + KOFF + off));
        const bf16x8 av = as_bf16x8(*reinterpret_cast<const u32x4 *>(cur + VOFF + off));
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, qf[t], sacc, 0, 0, 0);
        pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, of[t], pacc, 0, 0, 0);
      }
      // the next half's copies, issued while the matrix cores work through
      // the first block's S^T and dP^T (all waves issue them at the same
      // point, and the memory pipeline takes them in turn)
      if constexpr (kb == 0)
        if (nit < rg.count) issue_half(entry(nit), nhalf, (stage_i ^ 1) * STAGE);
      // ---- dS^T = P^T o (dP^T - D); element i is key k0 + kb*32 + 8*(i/4) + 4*hf + (i%4)
      bf16x8 sb[2];
      auto ds_t = [&](auto mask_tag) {
        constexpr bool MASK = decltype(mask_tag)::value;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          float sv[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int i = 8 * u + j;
            float x = __builtin_fmaf(sacc[i], c, -lse2);
            if (MASK) {
              const int kc = kb * 32 + 8 * (i >> 2) + (i & 3);
              x = (kc <= hi_r && kc >= lo_r) ? x : -INFINITY;    // masked pairs: exp2(-inf) = 0
            }
            const float pr = __builtin_amdgcn_exp2f(x);
            sv[j] = pr * (pacc[i] - dlt);
          }
          u32x4 sk;
          sk.x = pack_bf16(sv[0], sv[1]);
          sk.y = pack_bf16(sv[2], sv[3]);
          sk.z = pack_bf16(sv[4], sv[5]);
          sk.w = pack_bf16(sv[6], sv[7]);
          sb[u] = as_bf16x8(sk);
        }
      };
      // FULL, complete tiles skip the per-pair mask (uniform over the workgroup)
      if (masked)
        ds_t(std::true_type{});
      else
        ds_t(std::false_type{});
      // ---- dQ^T += K^T dS^T (k = 16 keys per step: kb*32 + 16u + 4hf + (0..3 | 8..11))
      static_for<2>([&](auto uc) {
        constexpr int off = 16 * (2 * kb + decltype(uc)::value) * RT::ROW;   // kb * 32 + 16 u rows
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const i16x4 lo = rd(k_lo[db], off), hi = rd(k_hi[db], off);
          const bf16x8 ak = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          qacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, sb[decltype(uc)::value], qacc[db], 0, 0, 0);
        }
      });
    });

    // the next half's copies have landed and every wave is done with this stage
    wait_copies();
    __syncthreads();
    stage_i ^= 1;
    it = nit;
    half = nhalf;
  }

  // ---- dQ += scale dQ^T for this lane's query row
  if (!row_ok) return;
  float *dqp = p.dq + (int64_t(qrow) * p.hq + h) * D + 4 * hf;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int ig = 0; ig < 4; ++ig) {
      const int off = db * 32 + 8 * ig;
      f32x4 a = *reinterpret_cast<f32x4 *>(dqp + off);
#pragma unroll
      for (int e = 0; e < 4; ++e) a[e] += p.scale * qacc[db][4 * ig + e];
      *reinterpret_cast<f32x4 *>(dqp + off) = a;
    }
}

}  // namespace

namespace {

// (row, head) pairs of the row-term kernel per workgroup, and its grid
int rowterm_per_block(int d) { return NT / (d / 8); }

BwdParams bwd_params(const BwdLaunch &a) {
  BwdParams p;
  p.q = static_cast<const unsigned short *>(a.q);
  p.k = static_cast<const unsigned short *>(a.k);
  p.v = static_cast<const unsigned short *>(a.v);
  p.dout = static_cast<const unsigned short *>(a.dout);
  p.lse = a.lse;
  p.delta = a.delta;
  p.q_row_stride = a.q_row_stride;
  p.kv_row_stride = a.kv_row_stride;
  p.dq = a.dq;
  p.dk = a.dk;
  p.dv = a.dv;
  p.ds_q = a.ds_q;
  p.slot = a.kv_slot;
  p.partial = a.partial;
  p.n_slots = a.n_slots;
  p.hq = a.hq;
  p.hkv = a.hkv;
  p.group = a.hq / a.hkv;
  p.tq = a.tq;
  p.scale = a.scale;
  p.c = a.scale * LOG2E;
  return p;
}

// query heads per dQ workgroup and its workgroup count
int dq_heads(int group) { return group % 4 == 0 ? 4 : group % 2 == 0 ? 2 : 1; }
// rows of its Q tiles: with four heads the plan's 64-row tiles; with one or
// two its 128-row list (four waves per head, so each staged K / V part
// serves twice the rows)
int dq_rows(int group) { return dq_heads(group) == 4 ? 64 : 128; }
int32_t dq_items(const BwdLaunch &a) { return dq_rows(a.hq / a.hkv) == 64 ? a.n_q_work : a.n_q2_work; }
int64_t dq_blocks(const BwdLaunch &a) {
  const int group = a.hq / a.hkv;
  const int64_t slots = (int64_t(dq_items(a)) * a.hkv + NXCD - 1) / NXCD;
  return slots * NXCD * (group / dq_heads(group));
}

}  // namespace

const char *bwd_rowterm_limits(const BwdLaunch &a) {
  if (a.d % 8 || a.d / 8 > 64) return "row terms need d a multiple of 8, at most 512";
  // a dispatch counts its work-items in 32 bits; the second grid dimension is at most 65535
  if (int64_t(a.n_touched_q) * NT > int64_t(UINT32_MAX)) return "row-term grid too large (touched Q tiles)";
  const int64_t by = (int64_t(a.max_q_rows) * a.hq + rowterm_per_block(a.d) - 1) / rowterm_per_block(a.d);
  if (by > 65535) return "row-term grid too large (Q tile rows x query heads)";
  return nullptr;
}

const char *attn_bwd_limits(const BwdLaunch &a) {
  const int64_t cap = int64_t(UINT32_MAX);
  if (int64_t(a.n_work) * a.hkv * NTK > cap) return "dK/dV grid too large (KV-tile chunks x KV heads)";
  if (int64_t(a.n_reduce) * a.hkv * NT > cap) return "split-tile reduce grid too large";
  if (dq_blocks(a) * 2 * dq_rows(a.hq / a.hkv) * dq_heads(a.hq / a.hkv) > cap)
    return "dQ grid too large (Q tiles x query heads)";
  return nullptr;
}

hipError_t noalloc_scratch(void **ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void *addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    // with this device current: its own copy of the array, at its own address
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_bwd_rowterm(const BwdLaunch &a, hipStream_t stream) {
  if (bwd_rowterm_limits(a)) return hipErrorInvalidValue;
  const int pairs = a.max_q_rows * a.hq, per_block = rowterm_per_block(a.d);
  const dim3 grid{static_cast<unsigned>(a.n_touched_q), static_cast<unsigned>((pairs + per_block - 1) / per_block)};
  hipLaunchKernelGGL(bwd_rowterm_kernel, grid, dim3(NT), 0, stream,
                     static_cast<const unsigned short *>(a.dout), a.q_row_stride, a.o, a.delta, a.touched_rows,
                     a.hq, a.d, a.tq);
  return hipGetLastError();
}

hipError_t launch_attn_bwd_dkdv(const BwdLaunch &a, hipStream_t stream) {
  if (a.n_work <= 0) return hipSuccess;
  if (attn_bwd_limits(a)) return hipErrorInvalidValue;
  BwdParams p = bwd_params(a);
  p.work = a.work;
  p.range = a.range;
  p.partners = a.partners;
  p.n_work = a.n_work;
  const dim3 grid{static_cast<unsigned>(a.n_work * a.hkv)};
  if (a.d == 128)
    hipLaunchKernelGGL(attn_bwd_kv_kernel<128>, grid, dim3(NTK), 0, stream, p);
  else
    hipLaunchKernelGGL(attn_bwd_kv_kernel<64>, grid, dim3(NTK), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.n_reduce > 0) {
    hipLaunchKernelGGL(bwd_kv_reduce_kernel, dim3(static_cast<unsigned>(a.n_reduce * a.hkv), BNB / RK), dim3(NT), 0,
                       stream, a.kv_reduce, a.partial, a.n_slots, a.hkv, a.d, a.scale, a.dk, a.dv);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_attn_bwd_dq(const BwdLaunch &a, hipStream_t stream) {
  if (dq_items(a) <= 0) return hipSuccess;
  if (attn_bwd_limits(a)) return hipErrorInvalidValue;
  BwdParams p = bwd_params(a);
  const int nh = dq_heads(p.group), tq = dq_rows(p.group);
  p.work = tq == 64 ? a.q_work : a.q2_work;
  p.range = tq == 64 ? a.q_range : a.q2_range;
  p.partners = tq == 64 ? a.q_partners : a.q2_partners;
  p.n_work = dq_items(a);
  const dim3 grid{static_cast<unsigned>(dq_blocks(a))}, block{static_cast<unsigned>(2 * tq * nh)};
  if (a.d == 128) {
    if (nh == 4)
      hipLaunchKernelGGL((attn_bwd_dq_kernel<128, 4, 64>), grid, block, 0, stream, p);
    else if (nh == 2)
      hipLaunchKernelGGL((attn_bwd_dq_kernel<128, 2, 128>), grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL((attn_bwd_dq_kernel<128, 1, 128>), grid, block, 0, stream, p);
  } else {
    if (nh == 4)
      hipLaunchKernelGGL((attn_bwd_dq_kernel<64, 4, 64>), grid, block, 0, stream, p);
    else if (nh == 2)
      hipLaunchKernelGGL((attn_bwd_dq_kernel<64, 2, 128>), grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL((attn_bwd_dq_kernel<64, 1, 128>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace sap
