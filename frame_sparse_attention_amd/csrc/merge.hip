// Exact merge of two partial attentions through their log-sum-exp
// (ISPA §2 item 1 and §3 item 2: decomposable attention, local and history
// branches combined afterwards with online-softmax algebra).
//
// HBM-bound: reads two [rows][D] float32 partials and their LSE, writes one.
// Each group of 32 lanes owns one row; lanes stride over D so every load and
// store of a wave covers contiguous 128-byte segments.
#include "fsa_internal.h"

namespace {

constexpr int kLanesPerRow = 32;
constexpr int kThreads = 256;

__global__ void __launch_bounds__(kThreads) merge_lse_kernel(
    const float *o1, const float *lse1, const float *o2, const float *lse2, long long rows,
    int D, float *o, float *lse) {
  const int lane = threadIdx.x % kLanesPerRow;
  const long long rows_per_block = kThreads / kLanesPerRow;
  for (long long row = blockIdx.x * rows_per_block + threadIdx.x / kLanesPerRow; row < rows;
       row += (long long)gridDim.x * rows_per_block) {
    const float a = lse1[row], b = lse2[row];
    float wa, wb, L;
    if (a == -INFINITY && b == -INFINITY) {
      wa = wb = 0.f;
      L = -INFINITY;
    } else if (b == -INFINITY) {
      wa = 1.f;
      wb = 0.f;
      L = a;
    } else if (a == -INFINITY) {
      wa = 0.f;
      wb = 1.f;
      L = b;
    } else {
      const float m = fmaxf(a, b);
      L = m + logf(expf(a - m) + expf(b - m));
      wa = expf(a - L);
      wb = expf(b - L);
    }
    const long long base = row * D;
    for (int d = lane; d < D; d += kLanesPerRow) {
      // a zero weight must not touch the other operand (it may hold anything)
      float x = wa != 0.f ? wa * o1[base + d] : 0.f;
      float y = wb != 0.f ? wb * o2[base + d] : 0.f;
      o[base + d] = x + y;
    }
    // Every lane of this row has read lse1/lse2 above (the 32 lanes of a row
    // sit in one wavefront and execute in lockstep), so an aliased write is safe.
    if (lane == 0) lse[row] = L;
  }
}

}  // namespace

extern "C" fsa_status fsa_merge_lse(const float *o1, const float *lse1, const float *o2,
                                    const float *lse2, int64_t rows, int32_t D, float *o,
                                    float *lse, void *stream) {
  fsa::clear_error();
  FSA_REQUIRE(rows >= 0, FSA_E_ARG, "rows=%lld must be >= 0", (long long)rows);
  FSA_REQUIRE(D >= 1, FSA_E_ARG, "D=%d must be >= 1", D);
  if (rows == 0) return FSA_OK;
  FSA_REQUIRE(o1 && lse1 && o2 && lse2 && o && lse, FSA_E_ARG, "null pointer argument");
  const long long rows_per_block = kThreads / kLanesPerRow;
  long long blocks = (rows + rows_per_block - 1) / rows_per_block;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(merge_lse_kernel, dim3((unsigned)blocks), dim3(kThreads), 0,
                     fsa::as_stream(stream), o1, lse1, o2, lse2, (long long)rows, D, o, lse);
  return fsa::check_launch("merge_lse");
}
