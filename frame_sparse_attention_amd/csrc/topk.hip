// Frame mean-pooling and top-k frame selection for memory heads
// (Light Forcing §2.2: query and key tokens are compressed to frame
// granularity by mean pooling and each query block picks its most relevant
// history frames; Head Forcing methodology §2: memory heads).
//
// Pooling is kept as float64 sums (a mean differs by a positive factor, so
// the ranking is unchanged and no division enters the bits).  Each pooled sum
// -- a query group's, a key frame's -- is the exact sum of its tokens rounded
// once to float64, so it has no summation order (pooling.h).  The score of a
// frame is the ascending-d dot product of the two sums with every product
// rounded before it is added (fp contraction is off in this file), so the
// selected frames are bit-reproducible.  Three launches:
//   pool          one block per piece (<= 128 rows) of every query group and
//                 every candidate key frame: float64 partial sums; every token
//                 is read once
//   finalize      one block per group / frame: the exact sums
//   score_select  one wavefront per (b, h, group): scores (one lane per frame,
//                 its row read 64 values ahead of the ordered adds), then the
//                 k best on (score desc, frame asc) by rank (k rounds of a
//                 wavefront argmax beyond 1024 candidates), written in
//                 ascending order.
#pragma clang fp contract(off)

#include <mutex>

#include "pooling.h"

namespace {

constexpr int kMaxCand = 4096;
constexpr int kMaxTopk = 64;

__global__ void __launch_bounds__(64) score_select_kernel(
    const double *__restrict__ qsum, const double *__restrict__ ksum, int H, int D,
    int h_begin, int Hs, int G, int cand_begin, int F, int topk,
    int32_t *__restrict__ out_frames, double *__restrict__ out_scores) {
  __shared__ double s_score[kMaxCand];
  __shared__ unsigned char s_taken[kMaxCand];
  __shared__ double qs[kMaxPoolD];
  const int lane = threadIdx.x;
  const int g = blockIdx.x % G;
  const int hs = (blockIdx.x / G) % Hs;
  const int b = blockIdx.x / (G * Hs);
  const double *qg = qsum + ((long long)(b * Hs + hs) * G + g) * D;
  for (int d = lane; d < D; d += 64) qs[d] = qg[d];
  __syncthreads();
  const double *ks = ksum + (long long)(b * Hs + hs) * F * D;
  const long long out_head = (long long)b * H + h_begin + hs;
  for (int fi = lane; fi < F; fi += 64) {
    const double acc = ordered_dot(qs, ks + (long long)fi * D, D);
    s_score[fi] = nan_last(acc);
    if (out_scores) out_scores[(out_head * G + g) * F + fi] = acc;
  }
  __syncthreads();
  take_best(s_score, s_taken, F, topk);
  int32_t *out = out_frames + (out_head * G + g) * topk;
  compact_taken(s_taken, F, topk, [&](int pos, int fi) { out[pos] = cand_begin + fi; });
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

// Workspace layout for Hs selected heads: the pooled sums of the G query
// groups and F candidate frames of each head, then the pieces' partial sums
// and magnitude keys of both families.  With ws == nullptr only the size is
// computed; otherwise the families' pointers are set.
struct TopkLayout {
  SegFamily qf, kf;
  double *qsum, *ksum;
  size_t bytes;
};
TopkLayout topk_layout(const void *q, const void *k, int B, int H, int Nq, int Nk, int D, int P,
                       int h_begin, int Hs, int q_group, int cand_begin, int F, void *ws) {
  TopkLayout L{};
  const int G = Nq / (q_group * P);
  L.qf = make_family(q, Nq, 0, q_group * P, G, H, h_begin, Hs);
  L.kf = make_family(k, Nk, (long long)cand_begin * P, P, F, H, h_begin, Hs);
  unsigned char *p = static_cast<unsigned char *>(ws);
  const size_t qbytes = align256((size_t)B * Hs * G * D * sizeof(double));
  const size_t kbytes = align256((size_t)B * Hs * F * D * sizeof(double));
  L.bytes = qbytes + kbytes + family_part_bytes(L.qf, B, D) + family_part_bytes(L.kf, B, D);
  if (ws != nullptr) {
    L.qsum = reinterpret_cast<double *>(p);
    p += qbytes;
    L.ksum = reinterpret_cast<double *>(p);
    p += kbytes;
    place_family(L.qf, B, D, &p);
    place_family(L.kf, B, D, &p);
  }
  return L;
}

size_t workspace_bytes_for(int32_t B, int32_t H, int32_t Nq, int32_t D, int32_t P,
                           int32_t q_group, int32_t F) {
  return topk_layout(nullptr, nullptr, B, H, Nq, 0, D, P, 0, H, q_group, 0, F, nullptr).bytes;
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
  *need = topk_layout(q, k, B, H, Nq, Nk, D, P, h_begin, Hs, q_group, cand_begin, F, nullptr)
              .bytes;
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
  TopkLayout L = topk_layout(q, k, B, H, Nq, Nk, D, P, h_begin, Hs, q_group, cand_begin, F,
                             workspace);
  const long long pieces = (long long)(family_pieces(L.qf, B) + family_pieces(L.kf, B));
  FSA_REQUIRE(pieces < (1LL << 31), FSA_E_SHAPE, "too many pooling pieces (%lld)", pieces);
  launch_pool(dt, pool_vec(dt, D, q, k), L.qf, L.kf, B, D, s);
  launch_finalize(dt, FinalFamily{L.qf, 1, L.qsum}, FinalFamily{L.kf, 1, L.ksum}, no_final(), B,
                  D, s);
  hipLaunchKernelGGL(score_select_kernel, dim3(B * Hs * G), dim3(64), 0, s, L.qsum, L.ksum, H,
                     D,
                     h_begin, Hs, G, cand_begin, F, topk_k, out_frames, out_scores);
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
