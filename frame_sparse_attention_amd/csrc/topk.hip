// Frame mean-pooling and top-k frame selection for memory heads
// (Light Forcing §2.2: query and key tokens are compressed to frame
// granularity by mean pooling and each query block picks its most relevant
// history frames; Head Forcing methodology §2: memory heads).
//
// Pooling is kept as float64 sums (a mean differs by a positive factor, so
// the ranking is unchanged and no division enters the bits).  Every sum runs
// in one fixed sequential order and products are rounded before they are
// added (fp contraction is off in this file), so the selected frames are
// bit-reproducible.  Queries, like keys, are pooled per frame first; the
// pooled query of a group is the ordered sum of its frame sums.  Two launches:
//   pool          one block per (b, h, query frame) and per (b, h, key frame):
//                 rows staged through LDS, one sequential float64 chain per
//                 channel; every token is read once
//   score_select  one wavefront per (b, h, group): scores, then the k best on
//                 (score desc, frame asc) by rank (k rounds of a wavefront
//                 argmax beyond 1024 candidates), written in ascending order.
#pragma clang fp contract(off)

#include <mutex>

#include "pooling.h"

namespace {

constexpr int kMaxCand = 4096;
constexpr int kMaxTopk = 64;

// (score, frame) order: higher score first, then lower frame.
__device__ inline bool better(double s1, int f1, double s2, int f2) {
  return s1 > s2 || (s1 == s2 && f1 < f2);
}

__global__ void __launch_bounds__(64) score_select_kernel(
    const double *__restrict__ qframe, const double *__restrict__ ksum, int H, int D,
    int h_begin, int Hs, int G, int q_group, int cand_begin, int F, int topk,
    int32_t *__restrict__ out_frames, double *__restrict__ out_scores) {
  __shared__ double s_score[kMaxCand];
  __shared__ unsigned char s_taken[kMaxCand];
  __shared__ double qs[kMaxPoolD];
  const int lane = threadIdx.x;
  const int g = blockIdx.x % G;
  const int hs = (blockIdx.x / G) % Hs;
  const int b = blockIdx.x / (G * Hs);
  // pooled query of the group: its frame sums added one at a time in frame order
  const double *qf = qframe + ((long long)(b * Hs + hs) * G * q_group + (long long)g * q_group) * D;
  for (int d = lane; d < D; d += 64) {
    double a = 0.0;
    for (int f = 0; f < q_group; ++f) a = a + qf[(long long)f * D + d];
    qs[d] = a;
  }
  __syncthreads();
  const double *ks = ksum + (long long)(b * Hs + hs) * F * D;
  const long long out_head = (long long)b * H + h_begin + hs;
  for (int fi = lane; fi < F; fi += 64) {
    const double acc = ordered_dot(qs, ks + (long long)fi * D, D);
    // a NaN score (from non-finite inputs) ranks as -inf, so (score, frame)
    // stays a strict total order and exactly topk frames are kept
    s_score[fi] = acc != acc ? -INFINITY : acc;
    s_taken[fi] = 0;
    if (out_scores) out_scores[(out_head * G + g) * F + fi] = acc;
  }
  __syncthreads();
  int32_t *out = out_frames + (out_head * G + g) * topk;
  if (F <= 1024) {
    // the topk best by rank: a candidate is kept when fewer than topk others
    // come first in the strict (score desc, frame asc) order
    for (int fi = lane; fi < F; fi += 64) {
      const double si = s_score[fi];
      int ahead = 0;
      for (int j = 0; j < F; ++j) ahead += better(s_score[j], j, si, fi) ? 1 : 0;
      s_taken[fi] = ahead < topk ? 1 : 0;
    }
    __syncthreads();
    // ascending frames: position = kept candidates before this one
    int count = 0;
    for (int base = 0; base < F; base += 64) {
      const int fi = base + lane;
      const bool keep = fi < F && s_taken[fi];
      const unsigned long long mask = __ballot(keep);
      const int pos = count + __popcll(mask & ((1ull << lane) - 1ull));
      if (keep && pos < topk) out[pos] = cand_begin + fi;
      count += __popcll(mask);
    }
    return;
  }
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
  if (lane < topk) out[rank] = cand_begin + mine;
}

fsa_status check_args(int32_t B, int32_t H, int32_t Nq, int32_t D, int32_t P, int32_t q_group,
                      int32_t cand_begin, int32_t cand_end) {
  FSA_REQUIRE(B >= 0 && H >= 0 && Nq >= 0, FSA_E_ARG, "negative size");
  FSA_REQUIRE(D >= 1 && D <= kMaxPoolD, FSA_E_SHAPE, "D=%d outside [1, %d]", D, kMaxPoolD);
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

size_t workspace_bytes_for(int32_t B, int32_t H, int32_t Nq, int32_t D, int32_t P, int32_t F) {
  const long long Tq = Nq / P;
  return (size_t)B * H * (Tq + F) * D * sizeof(double);
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
  *bytes = workspace_bytes_for(B, H, Nq, D, P, cand_end - cand_begin);
  return FSA_OK;
}

namespace {

// Checks everything but the workspace; returns the workspace bytes the call
// needs in *need (0 when there is nothing to compute).
fsa_status check_select(int32_t dt, int32_t B, int32_t H, int32_t Nq, int32_t Nk, int32_t D,
                        int32_t P, int32_t h_begin, int32_t h_end, int32_t q_group,
                        int32_t cand_begin, int32_t cand_end, int32_t topk_k, const void *q,
                        const void *k, const int32_t *out_frames, size_t *need) {
  *need = 0;
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
  FSA_REQUIRE(q && k && out_frames, FSA_E_ARG, "null pointer argument");
  *need = (size_t)B * Hs * ((size_t)G * q_group + F) * D * sizeof(double);
  return FSA_OK;
}

// Pooling and selection with the pooled sums in `workspace` (>= the bytes
// check_select reported; every byte the kernels read there they wrote first).
fsa_status launch_select(int32_t dt, const void *q, const void *k, int32_t B, int32_t H,
                         int32_t Nq, int32_t Nk, int32_t D, int32_t P, int32_t h_begin,
                         int32_t h_end, int32_t q_group, int32_t cand_begin, int32_t cand_end,
                         int32_t topk_k, int32_t *out_frames, double *out_scores,
                         void *workspace, hipStream_t s) {
  const int F = cand_end - cand_begin;
  const int Hs = h_end - h_begin;
  const int G = Nq / (q_group * P);
  const int Tq = G * q_group;
  double *qframe = static_cast<double *>(workspace);
  double *ksum = qframe + (size_t)B * Hs * Tq * D;
  const long long blocks = (long long)B * Hs * (Tq + F);
  FSA_REQUIRE(blocks < (1LL << 31), FSA_E_SHAPE, "too many pooling segments (%lld)", blocks);
  launch_pool(dt, q, k, H, Nq, Nk, D, P, h_begin, Hs, Tq, cand_begin, F, blocks, qframe, ksum, s);
  hipLaunchKernelGGL(score_select_kernel, dim3(B * Hs * G), dim3(64), 0, s, qframe, ksum, H, D,
                     h_begin, Hs, G, q_group, cand_begin, F, topk_k, out_frames, out_scores);
  return fsa::check_launch("select_topk_frames");
}

// Scratch of the allocation-free entry point: one array per GPU, created with
// the library's code object and held until the process ends.  Host code uses
// the device address from hipGetSymbolAddress, resolved once per device with
// that device current; the array's own name is only a host-side stand-in.
static __device__ __align__(256) unsigned char scratch[FSA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch[kMaxDevices];

fsa_status scratch_of_current_device(void **ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  FSA_REQUIRE(e == hipSuccess, FSA_E_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  FSA_REQUIRE(dev >= 0 && dev < kMaxDevices, FSA_E_HIP, "device %d beyond the %d supported", dev,
              kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    FSA_REQUIRE(e == hipSuccess && p != nullptr, FSA_E_HIP,
                "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return FSA_OK;
}

}  // namespace

extern "C" fsa_status fsa_select_topk_frames(const void *q, const void *k, int32_t dt, int32_t B,
                                             int32_t H, int32_t Nq, int32_t Nk, int32_t D,
                                             int32_t P, int32_t h_begin, int32_t h_end,
                                             int32_t q_group, int32_t cand_begin,
                                             int32_t cand_end, int32_t topk_k,
                                             int32_t *out_frames, double *out_scores,
                                             void *workspace, size_t workspace_bytes,
                                             void *stream) {
  fsa::clear_error();
  size_t need = 0;
  fsa_status st = check_select(dt, B, H, Nq, Nk, D, P, h_begin, h_end, q_group, cand_begin,
                               cand_end, topk_k, q, k, out_frames, &need);
  if (st != FSA_OK || need == 0) return st;
  FSA_REQUIRE(workspace != nullptr, FSA_E_ARG, "null pointer argument");
  FSA_REQUIRE(workspace_bytes >= need, FSA_E_CAPACITY, "workspace of %zu bytes < %zu needed",
              workspace_bytes, need);
  return launch_select(dt, q, k, B, H, Nq, Nk, D, P, h_begin, h_end, q_group, cand_begin,
                       cand_end, topk_k, out_frames, out_scores, workspace,
                       fsa::as_stream(stream));
}

extern "C" fsa_status fsa_select_topk_frames_noalloc(
    const void *q, const void *k, int32_t dt, int32_t B, int32_t H, int32_t Nq, int32_t Nk,
    int32_t D, int32_t P, int32_t h_begin, int32_t h_end, int32_t q_group, int32_t cand_begin,
    int32_t cand_end, int32_t topk_k, int32_t *out_frames, double *out_scores, void *stream) {
  fsa::clear_error();
  size_t need = 0;
  fsa_status st = check_select(dt, B, H, Nq, Nk, D, P, h_begin, h_end, q_group, cand_begin,
                               cand_end, topk_k, q, k, out_frames, &need);
  if (st != FSA_OK || need == 0) return st;
  FSA_REQUIRE(need <= FSA_NOALLOC_SCRATCH_BYTES, FSA_E_CAPACITY,
              "the pooled sums need %zu bytes, more than the %zu bytes of device scratch this "
              "entry point has; use fsa_select_topk_frames with a workspace",
              need, (size_t)FSA_NOALLOC_SCRATCH_BYTES);
  void *ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st != FSA_OK) return st;
  return launch_select(dt, q, k, B, H, Nq, Nk, D, P, h_begin, h_end, q_group, cand_begin,
                       cand_end, topk_k, out_frames, out_scores, ws, fsa::as_stream(stream));
}
