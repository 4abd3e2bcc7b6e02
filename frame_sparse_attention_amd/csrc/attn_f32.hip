// Frame-sparse attention for float32 inputs, computed in float32 end to end
// (LVSA §2 core mechanism: each query frame attends only to the frames of
// A(t); ISPA §2 item 1: the log-sum-exp of every row is returned).
//
// This is the exact-precision path for small float32 problems, not the
// throughput path: one wavefront per block, D/64 lanes per query row (each
// lane owns 64 channels of q and of the output accumulator), 32-key K/V tiles
// staged through LDS and read as broadcasts, online softmax per tile.
#include "attn_common.h"

namespace fsa {
namespace {

constexpr int kTileKeys = 32;

template <int D>
__global__ void __launch_bounds__(64) attn_f32_kernel(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ v,
    const int32_t *__restrict__ idx, const int32_t *__restrict__ cnt, int cap, int H, int Nq,
    int Nk, int P, int Tq, int qtiles, float scale, float *__restrict__ o,
    float *__restrict__ lse) {
  constexpr int kSplit = D / 64;        // lanes per query row
  constexpr int kRows = 64 / kSplit;    // query rows per block
  __shared__ float s_k[kTileKeys][D];
  __shared__ float s_v[kTileKeys][D];
  __shared__ int s_lo[FSA_MAX_CAP], s_hi[FSA_MAX_CAP];
  __shared__ int s_nruns;

  const int lane = threadIdx.x;
  int tile = blockIdx.x;
  const int qt = tile % qtiles;
  tile /= qtiles;
  const int tq = tile % Tq;
  tile /= Tq;
  const int h = tile % H;
  const int b = tile / H;
  const long long head = (long long)b * H + h;
  const long long list = head * Tq + tq;
  const int Tk = Nk / P;

  const int nruns = build_runs(idx + list * cap, cnt[list], cap, Tk, RunList{s_lo, s_hi}, &s_nruns);

  const int r = lane / kSplit, part = lane % kSplit;
  const int prow = qt * kRows + r;           // row inside the frame
  const bool row_ok = prow < P;
  const long long row = (long long)tq * P + (row_ok ? prow : P - 1);
  const float *qp = q + (head * Nq + row) * D + part * 64;
  float qr[64], acc[64];
  for (int d = 0; d < 64; ++d) {
    qr[d] = qp[d] * scale;
    acc[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const float *kh = k + head * Nk * D;
  const float *vh = v + head * Nk * D;

  for (int rr = 0; rr < nruns; ++rr) {
    const long long n_end = (long long)(s_hi[rr] + 1) * P;
    for (long long n0 = (long long)s_lo[rr] * P; n0 < n_end; n0 += kTileKeys) {
      const int nk = (int)(n_end - n0 < kTileKeys ? n_end - n0 : kTileKeys);
      __syncthreads();
      for (int e = lane; e < kTileKeys * D; e += 64) {
        const int j = e / D, d = e % D;
        const long long n = n0 + (j < nk ? j : nk - 1);
        s_k[j][d] = kh[n * D + d];
        s_v[j][d] = vh[n * D + d];
      }
      __syncthreads();
      float s[kTileKeys];
      float mt = -INFINITY;
      for (int j = 0; j < kTileKeys; ++j) {
        float dot = 0.f;
        for (int d = 0; d < 64; ++d) dot = fmaf(qr[d], s_k[j][part * 64 + d], dot);
        for (int off = 1; off < kSplit; off <<= 1) dot += __shfl_xor(dot, off);
        s[j] = j < nk ? dot : -INFINITY;
        mt = fmaxf(mt, s[j]);
      }
      const float mn = fmaxf(m, mt);
      const float alpha = expf(m - mn);  // m = -inf on the first tile gives 0
      float psum = 0.f;
      for (int d = 0; d < 64; ++d) acc[d] *= alpha;
      for (int j = 0; j < kTileKeys; ++j) {
        const float p = expf(s[j] - mn);
        psum += p;
        for (int d = 0; d < 64; ++d) acc[d] = fmaf(p, s_v[j][part * 64 + d], acc[d]);
      }
      l = l * alpha + psum;
      m = mn;
    }
  }
  if (!row_ok) return;
  float *op = o + (head * Nq + row) * D + part * 64;
  if (l > 0.f) {
    const float inv = 1.f / l;
    for (int d = 0; d < 64; ++d) op[d] = acc[d] * inv;
    if (part == 0) lse[head * Nq + row] = m + logf(l);
  } else {
    for (int d = 0; d < 64; ++d) op[d] = 0.f;
    if (part == 0) lse[head * Nq + row] = -INFINITY;
  }
}

}  // namespace

fsa_status launch_attn_f32(const float *q, const float *k, const float *v, const int32_t *idx,
                           const int32_t *cnt, int cap, int B, int H, int Nq, int Nk, int D,
                           int P, float scale, float *o, float *lse, hipStream_t stream) {
  const int Tq = Nq / P;
  const int rows = 64 / (D / 64);
  const int qtiles = (P + rows - 1) / rows;
  const long long blocks = (long long)B * H * Tq * qtiles;
  FSA_REQUIRE(blocks < (1LL << 31), FSA_E_SHAPE, "too many query tiles (%lld)", blocks);
  if (D == 64)
    hipLaunchKernelGGL(attn_f32_kernel<64>, dim3((unsigned)blocks), dim3(64), 0, stream, q, k, v,
                       idx, cnt, cap, H, Nq, Nk, P, Tq, qtiles, scale, o, lse);
  else
    hipLaunchKernelGGL(attn_f32_kernel<128>, dim3((unsigned)blocks), dim3(64), 0, stream, q, k,
                       v, idx, cnt, cap, H, Nq, Nk, P, Tq, qtiles, scale, o, lse);
  return check_launch("sparse_frame_attn (f32)");
}

}  // namespace fsa
