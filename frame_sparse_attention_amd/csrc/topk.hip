// Frame mean-pooling and top-k frame selection for memory heads
// (Light Forcing §2.2: query and key tokens are compressed to frame
// granularity by mean pooling and each query block picks its most relevant
// history frames; Head Forcing methodology §2: memory heads).
//
// Pooling is kept as float64 sums (a mean differs by a positive factor, so
// the ranking is unchanged and no division enters the bits).  Every sum runs
// in one fixed sequential order and products are rounded before they are
// added (fp contraction is off in this file), so the selected frames are
// bit-reproducible.  Three small launches:
//   pool_queries  one thread per (b, h, group, d): sum over the group's tokens
//   pool_keys     one thread per (b, h, frame, d): sum over the frame's tokens
//   score_select  one wavefront per (b, h, group): scores, then k rounds of a
//                 wavefront argmax on (score desc, frame asc), then sorting.
// The pooling launches read every token once (HBM-bound); the last is tiny.
#pragma clang fp contract(off)

#include "fsa_internal.h"

namespace {

constexpr int kMaxCand = 4096;
constexpr int kMaxTopk = 64;

__device__ inline double load_as_double(const float *p, long long i) { return (double)p[i]; }
// bfloat16 storage: the raw 16 bits
struct Bf16 {
  uint16_t bits;
};
__device__ inline double load_as_double(const Bf16 *p, long long i) {
  // bfloat16 -> float32 is exact (the bits move to the high half); float -> double is exact
  return (double)__uint_as_float((uint32_t)p[i].bits << 16);
}

template <typename T>
__global__ void pool_queries_kernel(const T *__restrict__ q, int H, int Nq, int D, int h_begin,
                                    int Hs, int group_tokens, double *__restrict__ qsum) {
  // blockIdx.x = (b * Hs + hs) * G + g ; threadIdx.x + blockIdx.y*blockDim.x = d
  const int d = blockIdx.y * blockDim.x + threadIdx.x;
  if (d >= D) return;
  const int G = Nq / group_tokens;
  const int g = blockIdx.x % G;
  const int hs = (blockIdx.x / G) % Hs;
  const int b = blockIdx.x / (G * Hs);
  const long long head = (long long)b * H + h_begin + hs;
  const long long row0 = head * Nq + (long long)g * group_tokens;
  double acc = 0.0;
  for (int i = 0; i < group_tokens; ++i) acc = acc + load_as_double(q, (row0 + i) * D + d);
  qsum[(long long)blockIdx.x * D + d] = acc;
}

template <typename T>
__global__ void pool_keys_kernel(const T *__restrict__ k, int H, int Nk, int D, int P,
                                 int h_begin, int Hs, int cand_begin, int F,
                                 double *__restrict__ ksum) {
  // blockIdx.x = (b * Hs + hs) * F + fi
  const int d = blockIdx.y * blockDim.x + threadIdx.x;
  if (d >= D) return;
  const int fi = blockIdx.x % F;
  const int hs = (blockIdx.x / F) % Hs;
  const int b = blockIdx.x / (F * Hs);
  const long long head = (long long)b * H + h_begin + hs;
  const long long row0 = head * Nk + (long long)(cand_begin + fi) * P;
  double acc = 0.0;
  for (int p = 0; p < P; ++p) acc = acc + load_as_double(k, (row0 + p) * D + d);
  ksum[(long long)blockIdx.x * D + d] = acc;
}

// (score, frame) order: higher score first, then lower frame.
__device__ inline bool better(double s1, int f1, double s2, int f2) {
  return s1 > s2 || (s1 == s2 && f1 < f2);
}

__global__ void __launch_bounds__(64) score_select_kernel(
    const double *__restrict__ qsum, const double *__restrict__ ksum, int H, int D, int h_begin,
    int Hs, int G, int cand_begin, int F, int topk, int32_t *__restrict__ out_frames,
    double *__restrict__ out_scores) {
  __shared__ double s_score[kMaxCand];
  __shared__ unsigned char s_taken[kMaxCand];
  const int lane = threadIdx.x;
  const int g = blockIdx.x % G;
  const int hs = (blockIdx.x / G) % Hs;
  const int b = blockIdx.x / (G * Hs);
  const double *qs = qsum + (long long)blockIdx.x * D;
  const double *ks = ksum + (long long)(b * Hs + hs) * F * D;
  const long long out_head = (long long)b * H + h_begin + hs;
  for (int fi = lane; fi < F; fi += 64) {
    double acc = 0.0;
    for (int d = 0; d < D; ++d) {
      const double prod = qs[d] * ks[(long long)fi * D + d];
      acc = acc + prod;
    }
    s_score[fi] = acc;
    s_taken[fi] = 0;
    if (out_scores) out_scores[(out_head * G + g) * F + fi] = acc;
  }
  __syncthreads();
  int mine = -1;  // frame selected in round == lane
  for (int round = 0; round < topk; ++round) {
    double bs = 0.0;
    int bf = -1;
    for (int fi = lane; fi < F; fi += 64) {
      if (s_taken[fi]) continue;
      const double s = s_score[fi];
      if (bf < 0 || better(s, fi, bs, bf)) {
        bs = s;
        bf = fi;
      }
    }
    for (int off = 32; off >= 1; off >>= 1) {
      const double os = __shfl_xor(bs, off);
      const int of = __shfl_xor(bf, off);
      if (of >= 0 && (bf < 0 || better(os, of, bs, bf))) {
        bs = os;
        bf = of;
      }
    }
    if (lane == round) mine = bf;
    if (lane == 0) s_taken[bf] = 1;
    __syncthreads();
  }
  // ascending order: the rank of each selected frame among the selected ones
  int rank = 0;
  for (int j = 0; j < topk; ++j) {
    const int other = __shfl(mine, j);
    if (other < mine) ++rank;
  }
  if (lane < topk) out_frames[(out_head * G + g) * topk + rank] = cand_begin + mine;
}

fsa_status check_args(int32_t B, int32_t H, int32_t Nq, int32_t D, int32_t P, int32_t q_group,
                      int32_t cand_begin, int32_t cand_end) {
  FSA_REQUIRE(B >= 0 && H >= 0 && Nq >= 0, FSA_E_ARG, "negative size");
  FSA_REQUIRE(D >= 1 && D <= 1024, FSA_E_SHAPE, "D=%d outside [1, 1024]", D);
  FSA_REQUIRE(P >= 1, FSA_E_SHAPE, "P=%d must be >= 1", P);
  FSA_REQUIRE(q_group >= 1, FSA_E_ARG, "q_group=%d must be >= 1", q_group);
  FSA_REQUIRE(Nq % ((long long)q_group * P) == 0, FSA_E_SHAPE,
              "Nq=%d is not a multiple of q_group*P=%lld", Nq, (long long)q_group * P);
  FSA_REQUIRE(cand_begin >= 0 && cand_end > cand_begin, FSA_E_ARG,
              "candidate range [%d, %d) is empty or negative", cand_begin, cand_end);
  FSA_REQUIRE(cand_end - cand_begin <= kMaxCand, FSA_E_ARG, "more than %d candidate frames",
              kMaxCand);
  return FSA_OK;
}

size_t workspace_bytes_for(int32_t B, int32_t H, int32_t Nq, int32_t D, int32_t P,
                           int32_t q_group, int32_t F) {
  const long long G = Nq / ((long long)q_group * P);
  return (size_t)B * H * (G + F) * D * sizeof(double);
}

}  // namespace

extern "C" fsa_status fsa_select_topk_workspace_size(int32_t B, int32_t H, int32_t Nq, int32_t D,
                                                     int32_t P, int32_t q_group,
                                                     int32_t cand_begin, int32_t cand_end,
                                                     size_t *bytes) {
  fsa::clear_error();
  FSA_REQUIRE(bytes != nullptr, FSA_E_ARG, "bytes is NULL");
  fsa_status st = check_args(B, H, Nq, D, P, q_group, cand_begin, cand_end);
  if (st != FSA_OK) return st;
  *bytes = workspace_bytes_for(B, H, Nq, D, P, q_group, cand_end - cand_begin);
  return FSA_OK;
}

extern "C" fsa_status fsa_select_topk_frames(const void *q, const void *k, int32_t dt, int32_t B,
                                             int32_t H, int32_t Nq, int32_t Nk, int32_t D,
                                             int32_t P, int32_t h_begin, int32_t h_end,
                                             int32_t q_group, int32_t cand_begin,
                                             int32_t cand_end, int32_t topk_k,
                                             int32_t *out_frames, double *out_scores,
                                             void *workspace, size_t workspace_bytes,
                                             void *stream) {
  fsa::clear_error();
  fsa_status st = check_args(B, H, Nq, D, P, q_group, cand_begin, cand_end);
  if (st != FSA_OK) return st;
  FSA_REQUIRE(dt == FSA_F32 || dt == FSA_BF16, FSA_E_DTYPE, "unknown dtype %d", dt);
  FSA_REQUIRE(Nk >= 0 && Nk % P == 0, FSA_E_SHAPE, "Nk=%d is not a multiple of P=%d", Nk, P);
  const int Tk = Nk / P;
  FSA_REQUIRE(cand_end <= Tk, FSA_E_ARG, "candidate frames [%d, %d) exceed Tk=%d", cand_begin,
              cand_end, Tk);
  FSA_REQUIRE(0 <= h_begin && h_begin <= h_end && h_end <= H, FSA_E_ARG,
              "head range [%d, %d) outside [0, %d]", h_begin, h_end, H);
  const int F = cand_end - cand_begin;
  FSA_REQUIRE(topk_k >= 1 && topk_k <= kMaxTopk, FSA_E_ARG, "topk=%d outside [1, %d]", topk_k,
              kMaxTopk);
  FSA_REQUIRE(topk_k <= F, FSA_E_ARG, "topk=%d exceeds the %d candidate frames", topk_k, F);
  const int Hs = h_end - h_begin;
  const int G = Nq / (q_group * P);
  if (B == 0 || Hs == 0 || G == 0) return FSA_OK;
  FSA_REQUIRE(q && k && out_frames && workspace, FSA_E_ARG, "null pointer argument");
  const size_t need = (size_t)B * Hs * (G + F) * D * sizeof(double);
  FSA_REQUIRE(workspace_bytes >= need, FSA_E_CAPACITY, "workspace of %zu bytes < %zu needed",
              workspace_bytes, need);
  double *qsum = static_cast<double *>(workspace);
  double *ksum = qsum + (size_t)B * Hs * G * D;
  hipStream_t s = fsa::as_stream(stream);
  const int tpb = D < 128 ? ((D + 63) / 64) * 64 : 128;
  const dim3 blk(tpb);
  const unsigned dy = (unsigned)((D + tpb - 1) / tpb);
  const int group_tokens = q_group * P;
  if (dt == FSA_BF16) {
    auto qq = static_cast<const Bf16 *>(q);
    auto kk = static_cast<const Bf16 *>(k);
    hipLaunchKernelGGL(pool_queries_kernel<Bf16>, dim3(B * Hs * G, dy), blk, 0, s, qq,
                       H, Nq, D, h_begin, Hs, group_tokens, qsum);
    hipLaunchKernelGGL(pool_keys_kernel<Bf16>, dim3(B * Hs * F, dy), blk, 0, s, kk, H,
                       Nk, D, P, h_begin, Hs, cand_begin, F, ksum);
  } else {
    auto qq = static_cast<const float *>(q);
    auto kk = static_cast<const float *>(k);
    hipLaunchKernelGGL(pool_queries_kernel<float>, dim3(B * Hs * G, dy), blk, 0, s, qq, H, Nq, D,
                       h_begin, Hs, group_tokens, qsum);
    hipLaunchKernelGGL(pool_keys_kernel<float>, dim3(B * Hs * F, dy), blk, 0, s, kk, H, Nk, D, P,
                       h_begin, Hs, cand_begin, F, ksum);
  }
  hipLaunchKernelGGL(score_select_kernel, dim3(B * Hs * G), dim3(64), 0, s, qsum, ksum, H, D,
                     h_begin, Hs, G, cand_begin, F, topk_k, out_frames, out_scores);
  return fsa::check_launch("select_topk_frames");
}
