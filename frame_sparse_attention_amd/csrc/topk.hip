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
//   score_select  one wavefront per (b, h, group): scores, then k rounds of a
//                 wavefront argmax on (score desc, frame asc), then sorting.
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

// Pooling of one segment of rows (a query group, or one key frame) of one
// head, for 128 channels per block: chunks of kRowsPerChunk rows are staged
// through LDS with 16-byte loads (two chunks in flight), then thread d adds
// its column one row at a time in ascending row order.  The float64 adds of a
// channel form one sequential chain, exactly as the definition orders them;
// the memory traffic around that chain is bulk and overlapped.
constexpr int kPoolThreads = 128;
constexpr int kRowsPerChunk = 32;
constexpr int kMaxPoolD = 256;  // LDS: 2 chunks x 32 rows x 256 x 4 B = 64 KB at most

template <typename T>
__device__ inline double elem_as_double(const T *row_tile, int r, int d, int D);
template <>
__device__ inline double elem_as_double<float>(const float *t, int r, int d, int D) {
  return (double)t[r * D + d];
}
template <>
__device__ inline double elem_as_double<Bf16>(const Bf16 *t, int r, int d, int D) {
  return (double)__uint_as_float((uint32_t)t[r * D + d].bits << 16);
}

// Adds rows [0, rows) of the LDS chunk `t` into this thread's channel sums.
template <typename T>
__device__ inline void add_chunk(const T *t, int rows, int D, double *acc) {
  const int tid = threadIdx.x;
  for (int i = 0; i * kPoolThreads + tid < D; ++i) {
    const int d = i * kPoolThreads + tid;
    double a = acc[i];
    if (rows == kRowsPerChunk) {
      // read the whole column chunk first (independent LDS loads), then add in order
      double x[kRowsPerChunk];
#pragma unroll
      for (int r = 0; r < kRowsPerChunk; ++r) x[r] = elem_as_double<T>(t, r, d, D);
#pragma unroll
      for (int r = 0; r < kRowsPerChunk; ++r) a = a + x[r];
    } else {
      for (int r = 0; r < rows; ++r) a = a + elem_as_double<T>(t, r, d, D);
    }
    acc[i] = a;
  }
}

// s_waitcnt immediates: vmcnt(n) with expcnt and lgkmcnt at their maxima
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Sums rows [row0, row0 + nrows) of `src` (row stride D) into out[0..D).
// Chunks of kRowsPerChunk rows stream from HBM into an LDS ring of kRing
// slots with global_load_lds (no registers in flight), kRing - 1 chunks ahead
// of the chunk being added; rows past the segment repeat its last row (in
// bounds, never added).  Needs a chunk of whole 1 KB wavefront transfers.
constexpr int kRing = 8;
template <typename T>
__device__ void pool_segment_dma(const T *__restrict__ src, long long row0, int nrows, int D,
                                 unsigned char *lds, double *__restrict__ out) {
  const int tid = threadIdx.x, lane = tid % 64;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int row_bytes = D * (int)sizeof(T);
  const int chunk_bytes = kRowsPerChunk * row_bytes;
  const int per_wave = chunk_bytes / 1024 / (kPoolThreads / 64);  // DMA instructions per wave
  const int nchunks = (nrows + kRowsPerChunk - 1) / kRowsPerChunk;
  const char *base = reinterpret_cast<const char *>(src) + row0 * row_bytes;
  auto issue = [&](int c) {
    unsigned char *slot = lds + (c % kRing) * chunk_bytes;
    for (int i = 0; i < per_wave; ++i) {
      const int unit = (i * (kPoolThreads / 64) + wave) * 64 + lane;  // 16-byte unit in chunk
      int r = c * kRowsPerChunk + unit * 16 / row_bytes;
      r = r < nrows ? r : nrows - 1;
      const char *g = base + (long long)r * row_bytes + (unit * 16) % row_bytes;
      __builtin_amdgcn_global_load_lds(
          (const void *)g,
          (__attribute__((address_space(3))) void *)(slot + (i * (kPoolThreads / 64) + wave) * 1024),
          16, 0, 0);
    }
  };
  double acc[kMaxPoolD / kPoolThreads];
  for (int i = 0; i < kMaxPoolD / kPoolThreads; ++i) acc[i] = 0.0;
  for (int c = 0; c < kRing - 1 && c < nchunks; ++c) issue(c);
  for (int c = 0; c < nchunks; ++c) {
    if (c + kRing - 1 < nchunks) {
      issue(c + kRing - 1);
      // chunk c landed once at most kRing - 1 later chunks are outstanding
      if (per_wave == 1) wait_vmcnt<kRing - 1>();
      else if (per_wave == 2) wait_vmcnt<2 * (kRing - 1)>();
      else if (per_wave == 4) wait_vmcnt<4 * (kRing - 1)>();
      else wait_vmcnt<0>();
    } else {
      wait_vmcnt<0>();
    }
    __syncthreads();
    const int rows = min(kRowsPerChunk, nrows - c * kRowsPerChunk);
    add_chunk<T>(reinterpret_cast<const T *>(lds + (c % kRing) * chunk_bytes), rows, D, acc);
    __syncthreads();  // slot c % kRing is refilled by the next issue
  }
  for (int i = 0; i * kPoolThreads + tid < D; ++i) out[i * kPoolThreads + tid] = acc[i];
}

// Fallback for shapes the DMA path cannot take: chunks go through registers.
template <typename T>
__device__ void pool_segment(const T *__restrict__ src, long long row0, int nrows, int D,
                             T *tile /* LDS [kRowsPerChunk * D] */, double *__restrict__ out) {
  const int tid = threadIdx.x;
  const int nchunks = (nrows + kRowsPerChunk - 1) / kRowsPerChunk;
  double acc[kMaxPoolD / kPoolThreads];
  for (int i = 0; i < kMaxPoolD / kPoolThreads; ++i) acc[i] = 0.0;
  for (int c = 0; c < nchunks; ++c) {
    const int rows = min(kRowsPerChunk, nrows - c * kRowsPerChunk);
    const T *g = src + (row0 + (long long)c * kRowsPerChunk) * D;
    for (int u = tid; u < rows * D; u += kPoolThreads) tile[u] = g[u];
    __syncthreads();
    add_chunk<T>(tile, rows, D, acc);
    __syncthreads();
  }
  for (int i = 0; i * kPoolThreads + tid < D; ++i) out[i * kPoolThreads + tid] = acc[i];
}

// One launch pools every query frame and every candidate key frame of the
// selected heads (one block each).
template <typename T>
__global__ void __launch_bounds__(kPoolThreads) pool_kernel(
    const T *__restrict__ q, const T *__restrict__ k, int H, int Nq, int Nk, int D, int P,
    int h_begin, int Hs, int Tq, int cand_begin, int F, bool use_dma,
    double *__restrict__ qframe, double *__restrict__ ksum) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  T *tile = reinterpret_cast<T *>(smem);
  const long long bid = blockIdx.x;
  const int chunk_bytes = kRowsPerChunk * D * (int)sizeof(T);
  const int per_wave = chunk_bytes / 1024 / (kPoolThreads / 64);
  const bool dma = use_dma && chunk_bytes % 2048 == 0 &&
                   (per_wave == 1 || per_wave == 2 || per_wave == 4);
  // block layout: b-major, then [Tq query frames | F key frames] per selected head
  const int per_b = Hs * (Tq + F);
  const int b = (int)(bid / per_b);
  const int rem = (int)(bid % per_b);
  if (rem < Hs * Tq) {
    const int hs = rem / Tq, t = rem % Tq;
    const long long head = (long long)b * H + h_begin + hs;
    double *dst = qframe + ((long long)(b * Hs + hs) * Tq + t) * D;
    if (dma)
      pool_segment_dma<T>(q, head * Nq + (long long)t * P, P, D, smem, dst);
    else
      pool_segment<T>(q, head * Nq + (long long)t * P, P, D, tile, dst);
  } else {
    const int r2 = rem - Hs * Tq;
    const int hs = r2 / F, fi = r2 % F;
    const long long head = (long long)b * H + h_begin + hs;
    double *dst = ksum + ((long long)(b * Hs + hs) * F + fi) * D;
    if (dma)
      pool_segment_dma<T>(k, head * Nk + (long long)(cand_begin + fi) * P, P, D, smem, dst);
    else
      pool_segment<T>(k, head * Nk + (long long)(cand_begin + fi) * P, P, D, tile, dst);
  }
}

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
  const int Tq = G * q_group;
  const size_t need = (size_t)B * Hs * (Tq + F) * D * sizeof(double);
  FSA_REQUIRE(workspace_bytes >= need, FSA_E_CAPACITY, "workspace of %zu bytes < %zu needed",
              workspace_bytes, need);
  double *qframe = static_cast<double *>(workspace);
  double *ksum = qframe + (size_t)B * Hs * Tq * D;
  hipStream_t s = fsa::as_stream(stream);
  const long long blocks = (long long)B * Hs * (Tq + F);
  FSA_REQUIRE(blocks < (1LL << 31), FSA_E_SHAPE, "too many pooling segments (%lld)", blocks);
  const bool aligned = ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k)) & 15u) == 0;
  if (dt == FSA_BF16) {
    const size_t chunk = (size_t)kRowsPerChunk * D * sizeof(Bf16);
    const size_t lds = aligned && chunk * kRing <= 65536 ? chunk * kRing : chunk;
    hipLaunchKernelGGL(pool_kernel<Bf16>, dim3((unsigned)blocks), dim3(kPoolThreads), lds, s,
                       static_cast<const Bf16 *>(q), static_cast<const Bf16 *>(k), H, Nq, Nk, D,
                       P, h_begin, Hs, Tq, cand_begin, F, lds > chunk, qframe, ksum);
  } else {
    const size_t chunk = (size_t)kRowsPerChunk * D * sizeof(float);
    const size_t lds = aligned && chunk * kRing <= 65536 ? chunk * kRing : chunk;
    hipLaunchKernelGGL(pool_kernel<float>, dim3((unsigned)blocks), dim3(kPoolThreads), lds, s,
                       static_cast<const float *>(q), static_cast<const float *>(k), H, Nq, Nk,
                       D, P, h_begin, Hs, Tq, cand_begin, F, lds > chunk, qframe, ksum);
  }
  hipLaunchKernelGGL(score_select_kernel, dim3(B * Hs * G), dim3(64), 0, s, qframe, ksum, H, D,
                     h_begin, Hs, G, q_group, cand_begin, F, topk_k, out_frames, out_scores);
  return fsa::check_launch("select_topk_frames");
}
