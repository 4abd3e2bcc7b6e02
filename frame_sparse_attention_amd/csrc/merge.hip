// Exact merge of two partial attentions through their log-sum-exp
// (ISPA §2 item 1 and §3 item 2: decomposable attention, local and history
// branches combined afterwards with online-softmax algebra).
//
// HBM-bound: reads two [rows][D] float32 partials and their LSE, writes one
// (and the same for S partials of a split frame list).
// Each group of 32 lanes owns one row; lanes stride over D so every load and
// store of a wave covers contiguous 128-byte segments.
#include "fsa_internal.h"

namespace {

constexpr int kLanesPerRow = 32;
constexpr int kThreads = 256;

__global__ void __launch_bounds__(kThreads) merge_lse_kernel(
    const float *o1, const float *lse1, const float *o2, const float *lse2, long long rows,
    int D, bool vec4, float *o, float *lse) {
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
    if (vec4) {
      // 16-byte accesses: lane t covers channels 4t .. 4t+3 of each 128-channel span
      for (int d = 4 * lane; d < D; d += 4 * kLanesPerRow) {
        const float4 a = wa != 0.f ? *reinterpret_cast<const float4 *>(o1 + base + d)
                                   : make_float4(0.f, 0.f, 0.f, 0.f);
        const float4 c = wb != 0.f ? *reinterpret_cast<const float4 *>(o2 + base + d)
                                   : make_float4(0.f, 0.f, 0.f, 0.f);
        float4 r;
        r.x = (wa != 0.f ? wa * a.x : 0.f) + (wb != 0.f ? wb * c.x : 0.f);
        r.y = (wa != 0.f ? wa * a.y : 0.f) + (wb != 0.f ? wb * c.y : 0.f);
        r.z = (wa != 0.f ? wa * a.z : 0.f) + (wb != 0.f ? wb * c.z : 0.f);
        r.w = (wa != 0.f ? wa * a.w : 0.f) + (wb != 0.f ? wb * c.w : 0.f);
        *reinterpret_cast<float4 *>(o + base + d) = r;
      }
    } else {
      for (int d = lane; d < D; d += kLanesPerRow) {
        // a zero weight must not touch the other operand (it may hold anything)
        float x = wa != 0.f ? wa * o1[base + d] : 0.f;
        float y = wb != 0.f ? wb * o2[base + d] : 0.f;
        o[base + d] = x + y;
      }
    }
    // Every lane of this row has read lse1/lse2 above (the 32 lanes of a row
    // sit in one wavefront and execute in lockstep), so an aliased write is safe.
    if (lane == 0) lse[row] = L;
  }
}

// Merge of S partials of one attention (the parts of a split frame list):
// L = M + ln sum_s exp(LSE_s - M), O = sum_s exp(LSE_s - L) O_s, in ascending
// s; parts with LSE_s = -inf have weight 0 and are not read.  Partial s of
// row r is o_parts[(s * rows + r) * D ...], lse_parts[s * rows + r].
constexpr int kMaxSplits = 16;

__global__ void __launch_bounds__(kThreads) merge_splits_kernel(
    const float *__restrict__ o_parts, const float *__restrict__ lse_parts, int S, long long rows,
    int D, float *__restrict__ o, float *__restrict__ lse) {
  const int lane = threadIdx.x % kLanesPerRow;
  const long long rows_per_block = kThreads / kLanesPerRow;
  for (long long row = blockIdx.x * rows_per_block + threadIdx.x / kLanesPerRow; row < rows;
       row += (long long)gridDim.x * rows_per_block) {
    float ls[kMaxSplits];
    float m = -INFINITY;
    for (int sp = 0; sp < S; ++sp) {
      ls[sp] = lse_parts[sp * rows + row];
      m = fmaxf(m, ls[sp]);
    }
    const long long base = row * D;
    if (m == -INFINITY) {
      for (int d = lane; d < D; d += kLanesPerRow) o[base + d] = 0.f;
      if (lane == 0) lse[row] = -INFINITY;
      continue;
    }
    float sum = 0.f;
    for (int sp = 0; sp < S; ++sp) sum += ls[sp] == -INFINITY ? 0.f : expf(ls[sp] - m);
    const float L = m + logf(sum);
    for (int sp = 0; sp < S; ++sp) ls[sp] = ls[sp] == -INFINITY ? 0.f : expf(ls[sp] - L);
    for (int d = lane; d < D; d += kLanesPerRow) {
      float acc = 0.f;
      for (int sp = 0; sp < S; ++sp)
        if (ls[sp] != 0.f) acc += ls[sp] * o_parts[(sp * rows + row) * D + d];
      o[base + d] = acc;
    }
    if (lane == 0) lse[row] = L;
  }
}

}  // namespace

namespace fsa {
fsa_status launch_merge_splits(const float *o_parts, const float *lse_parts, int S,
                               long long rows, int D, float *o, float *lse, hipStream_t stream) {
  FSA_REQUIRE(S >= 1 && S <= kMaxSplits, FSA_E_ARG, "splits=%d outside [1, %d]", S, kMaxSplits);
  if (rows == 0) return FSA_OK;
  const long long rows_per_block = kThreads / kLanesPerRow;
  long long blocks = (rows + rows_per_block - 1) / rows_per_block;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(merge_splits_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                     o_parts, lse_parts, S, rows, D, o, lse);
  return check_launch("merge of split partials");
}
}  // namespace fsa

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
  const bool vec4 = D % 4 == 0 && ((reinterpret_cast<uintptr_t>(o1) | reinterpret_cast<uintptr_t>(o2) |
                                    reinterpret_cast<uintptr_t>(o)) & 15u) == 0;
  hipLaunchKernelGGL(merge_lse_kernel, dim3((unsigned)blocks), dim3(kThreads), 0,
                     fsa::as_stream(stream), o1, lse1, o2, lse2, (long long)rows, D, vec4, o, lse);
  return fsa::check_launch("merge_lse");
}
