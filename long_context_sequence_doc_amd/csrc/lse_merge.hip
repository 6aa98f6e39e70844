// Merge kernel: exact combination of a partial attention result into the
// running one, for the rows a ring step touched.
//
// Sequence parallelism is computation-equivalent to one-device attention
// (SP blog page, bmjup.com/post/14448.html, FAQ Q1) and the ring hands every
// rank the full-sequence result (same page, core principles). With partial
// results over disjoint KV sets given as (O, LSE):
//     L = ln(e^La + e^Lb),  O = e^(La - L) O_a + e^(Lb - L) O_b
// A side whose LSE is -inf holds no keys and contributes nothing (its O is
// not read into the result at all); both -inf leaves O = 0, LSE = -inf.
//
// HBM-bound elementwise work: (12 D + 12) bytes per (row, head). A touched Q
// tile's rows are one contiguous [rows][Hq][D] block of O; D/4 consecutive
// threads take one (row, head), one float4 each, so a block pass streams
// NTHREADS * 16 bytes of each operand. The (row, head) LSE pair is read by
// those D/4 threads, which sit in one wave (D/4 divides 64), and written
// back by the first of them after every lane of the wave has read it.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "kernels.h"

namespace sap {
namespace {

typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int NTHREADS = 256;

struct MergeParams {
  float *o_acc, *lse_acc;
  const float *o_part, *lse_part;
  const int32_t *touched_rows;
  int32_t tq, hq;
  int32_t single_rows;   // rows when merging everything (touched_rows == nullptr)
};

template <int D>
__global__ __launch_bounds__(NTHREADS) void lse_merge_kernel(MergeParams p) {
  constexpr int D4 = D / 4;                      // float4s per (row, head)
  constexpr int RH = NTHREADS / D4;              // (row, head) pairs per block pass
  static_assert(64 % D4 == 0, "a (row, head) must sit inside one wave");
  int r0, n;
  if (p.touched_rows) {
    r0 = p.touched_rows[2 * blockIdx.x];
    n = p.touched_rows[2 * blockIdx.x + 1];
  } else {
    r0 = 0;
    n = p.single_rows;
  }
  const int nrh = n * p.hq;                      // (row, head) pairs of this tile (< 2^31, checked on the host)
  const int c = int(threadIdx.x) % D4;
  f32x4 *oa = reinterpret_cast<f32x4 *>(p.o_acc) + int64_t(r0) * p.hq * D4;
  const f32x4 *ob = reinterpret_cast<const f32x4 *>(p.o_part) + int64_t(r0) * p.hq * D4;
  for (int rh = int(blockIdx.y) * RH + int(threadIdx.x) / D4; rh < nrh; rh += int(gridDim.y) * RH) {
    const int rr = rh / p.hq;
    const int row = r0 + rr, head = rh - rr * p.hq;
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
    const int64_t e = int64_t(rh) * D4 + c;
    const f32x4 a = oa[e], b = ob[e];
    // a side with LSE = -inf holds no keys: it is dropped by a select, not
    // multiplied by 0, so whatever its O holds (even NaN) cannot leak in
    f32x4 m;
    if (la == -INFINITY)
      m = lb == -INFINITY ? f32x4{0.f, 0.f, 0.f, 0.f} : wb * b;
    else
      m = lb == -INFINITY ? wa * a : wa * a + wb * b;
    oa[e] = m;
    if (c == 0) p.lse_acc[li] = L;
  }
}

}  // namespace

const char *lse_merge_limits(const MergeLaunch &a) {
  if (int64_t(a.max_rows) * a.hq > INT32_MAX / 2) return "merge tile too large (rows x heads)";
  if (int64_t(a.n_touched) * NTHREADS > int64_t(UINT32_MAX)) return "merge grid too large (touched Q tiles)";
  return nullptr;
}

hipError_t launch_lse_merge(const MergeLaunch &a, hipStream_t stream) {
  if (lse_merge_limits(a)) return hipErrorInvalidValue;
  MergeParams p;
  p.o_acc = a.o_acc;
  p.lse_acc = a.lse_acc;
  p.o_part = a.o_part;
  p.lse_part = a.lse_part;
  p.touched_rows = a.touched_rows;
  p.tq = a.tq;
  p.hq = a.hq;
  p.single_rows = a.touched_rows ? 0 : a.tq;
  const int64_t pairs = int64_t(a.max_rows) * a.hq;
  const int rh = a.d >= 4 && a.d <= 256 ? NTHREADS / (a.d / 4) : 1;
  int64_t by = (pairs + rh - 1) / rh;
  if (by < 1) by = 1;
  if (by > 65535) by = 65535;
  const dim3 grid{static_cast<unsigned>(a.n_touched), static_cast<unsigned>(by)}, block{NTHREADS};
  switch (a.d) {   // the head dims the entry point accepts: powers of two in [4, 256]
    case 4: hipLaunchKernelGGL(lse_merge_kernel<4>, grid, block, 0, stream, p); break;
    case 8: hipLaunchKernelGGL(lse_merge_kernel<8>, grid, block, 0, stream, p); break;
    case 16: hipLaunchKernelGGL(lse_merge_kernel<16>, grid, block, 0, stream, p); break;
    case 32: hipLaunchKernelGGL(lse_merge_kernel<32>, grid, block, 0, stream, p); break;
    case 64: hipLaunchKernelGGL(lse_merge_kernel<64>, grid, block, 0, stream, p); break;
    case 128: hipLaunchKernelGGL(lse_merge_kernel<128>, grid, block, 0, stream, p); break;
    case 256: hipLaunchKernelGGL(lse_merge_kernel<256>, grid, block, 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace sap
