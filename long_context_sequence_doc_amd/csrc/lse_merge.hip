// Merge kernel: exact combination of a partial attention result into the
// running one, for the rows a ring step touched.
//
// Sequence parallelism is computation-equivalent to one-device attention
// (SP blog page, bmjup.com/post/14448.html, FAQ Q1) and the ring hands every
// rank the full-sequence result (same page, core principles). With partial
// results over disjoint KV sets given as (O, LSE):
//     L = ln(e^La + e^Lb),  O = e^(La - L) O_a + e^(Lb - L) O_b
// A side whose LSE is -inf holds no keys and contributes nothing.
//
// HBM-bound elementwise work: (12 D + 12) bytes per (row, head). A touched Q
// tile's rows are one contiguous [rows][Hq][D] block of O, so the blocks of
// grid row x stream float4s of touched tile x; the (row, head) LSE pair is
// read by the D/4 threads of its row segment, which all sit in one wave (D is
// a power of two <= 256), and written back by the first of them after every
// lane of the wave has read it.
#include <hip/hip_runtime.h>

#include <cmath>

#include "kernels.h"

namespace sap {
namespace {

typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int NTHREADS = 256;
constexpr int PER_THREAD = 4;

struct MergeParams {
  float *o_acc, *lse_acc;
  const float *o_part, *lse_part;
  const int32_t *touched_rows;
  int32_t tq, hq, d, d4;
  int32_t single_rows;   // rows when merging everything (touched_rows == nullptr)
};

__global__ __launch_bounds__(NTHREADS) void lse_merge_kernel(MergeParams p) {
  int r0, n;
  if (p.touched_rows) {
    r0 = p.touched_rows[2 * blockIdx.x];
    n = p.touched_rows[2 * blockIdx.x + 1];
  } else {
    r0 = 0;
    n = p.single_rows;
  }
  const int64_t per_row4 = int64_t(p.hq) * p.d4;
  const int64_t total4 = int64_t(n) * per_row4;
  const int64_t base4 = int64_t(r0) * per_row4;
  f32x4 *oa = reinterpret_cast<f32x4 *>(p.o_acc) + base4;
  const f32x4 *ob = reinterpret_cast<const f32x4 *>(p.o_part) + base4;
  const int64_t stride = int64_t(gridDim.y) * NTHREADS;
  for (int64_t e = int64_t(blockIdx.y) * NTHREADS + threadIdx.x; e < total4; e += stride) {
    const int64_t rh = e / p.d4;                 // (row, head) index inside the block
    const int row = r0 + int(rh / p.hq);
    const int head = int(rh % p.hq);
    const int64_t li = int64_t(head) * p.tq + row;
    const float la = p.lse_acc[li], lb = p.lse_part[li];
    const float mx = fmaxf(la, lb), mn = fminf(la, lb);
    float L, wa, wb;
    if (mx == -INFINITY) {
      L = -INFINITY;
      wa = 0.f;
      wb = 0.f;
    } else {
      L = mx + log1pf(__expf(mn - mx));          // mn = -inf gives exactly mx
      wa = la == -INFINITY ? 0.f : __expf(la - L);
      wb = lb == -INFINITY ? 0.f : __expf(lb - L);
    }
    const f32x4 a = oa[e], b = ob[e];
    oa[e] = wa * a + wb * b;
    if (e % p.d4 == 0) p.lse_acc[li] = L;
  }
}

}  // namespace

hipError_t launch_lse_merge(const MergeLaunch &a, hipStream_t stream) {
  MergeParams p;
  p.o_acc = a.o_acc;
  p.lse_acc = a.lse_acc;
  p.o_part = a.o_part;
  p.lse_part = a.lse_part;
  p.touched_rows = a.touched_rows;
  p.tq = a.tq;
  p.hq = a.hq;
  p.d = a.d;
  p.d4 = a.d / 4;
  p.single_rows = a.touched_rows ? 0 : a.tq;
  const int64_t total4 = int64_t(a.max_rows) * a.hq * p.d4;
  int64_t by = (total4 + int64_t(NTHREADS) * PER_THREAD - 1) / (int64_t(NTHREADS) * PER_THREAD);
  if (by < 1) by = 1;
  if (by > 65535) by = 65535;
  const dim3 grid{static_cast<unsigned>(a.n_touched), static_cast<unsigned>(by)}, block{NTHREADS};
  hipLaunchKernelGGL(lse_merge_kernel, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace sap
