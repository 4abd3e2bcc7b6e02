// Two-level (frame, then block) selection of hierarchical sparse attention
// (Light Forcing §2.2: query and key tokens are compressed to block and frame
// granularity by mean pooling; per query block a few history frames are
// retrieved with the frame-level keys, then the critical blocks inside them
// with the block-level keys; attention runs over the chosen blocks).
//
// Units: a block is `block` consecutive tokens inside a frame, nb = P / block
// blocks per frame, global block index = frame * nb + block-in-frame.  The
// output lists are in block units, so the attention kernels run on them with
// "frames" of `block` tokens.
//
// Arithmetic (fixed, so the lists are bit-reproducible): float64 sums; a block
// sum adds its tokens in ascending order, a frame sum adds its block sums in
// ascending order; a score adds rounded products in ascending channel order;
// ranking is (score descending, index ascending).  Three launches:
//   pool         block sums of every query block and of every key block of the
//                candidate frames (the shared pooling kernel)
//   frame_sums   frame sums from the block sums
//   select       one wavefront per (b, h, query block): frame scores, the kf
//                best by rank, block scores over the chosen frames, the kb best
//                by rank, then the ascending list with the recent frames.
#pragma clang fp contract(off)

#include "pooling.h"

namespace {

constexpr int kMaxHsaCand = 4096;  // candidate frames, and candidate blocks per query block

__global__ void __launch_bounds__(kPoolThreads) hsa_frame_sums_kernel(
    const double *__restrict__ kblk, int D, int nb, int Fc, long long n_frames,
    double *__restrict__ kframe) {
  // one block per (b, hs, frame); frame sum = ordered sum of its nb block sums
  const long long fid = blockIdx.x;
  if (fid >= n_frames) return;
  const double *src = kblk + fid * nb * D;
  for (int d = threadIdx.x; d < D; d += kPoolThreads) {
    double a = 0.0;
    for (int i = 0; i < nb; ++i) a = a + src[(long long)i * D + d];
    kframe[fid * D + d] = a;
  }
  (void)Fc;
}

// A NaN score (from non-finite inputs) ranks as -inf, so (score, index) stays
// a strict total order and exactly k candidates are kept.
__device__ inline double nan_last(double s) { return s != s ? -INFINITY : s; }

// (score, index) order: higher score first, then lower index.
__device__ inline bool hsa_better(double s1, int i1, double s2, int i2) {
  return s1 > s2 || (s1 == s2 && i1 < i2);
}

// Marks in s_taken the k best of s_score[0..n) in the (score descending,
// index ascending) order, a strict total order: up to 1024 candidates, each
// lane counts for its candidates how many others come first and keeps those
// with fewer than k (one pass of n comparisons per candidate); beyond that, k
// rounds of a wavefront argmax.  Both give the same set.  Needs k <= n and
// s_taken[0..n) cleared.
__device__ void take_best(const double *s_score, unsigned char *s_taken, int n, int k) {
  const int lane = threadIdx.x;
  if (n <= 1024) {
    for (int i = lane; i < n; i += 64) {
      const double si = s_score[i];
      int ahead = 0;
      for (int j = 0; j < n; ++j) ahead += hsa_better(s_score[j], j, si, i) ? 1 : 0;
      s_taken[i] = ahead < k ? 1 : 0;
    }
    __syncthreads();
    return;
  }
  for (int round = 0; round < k; ++round) {
    double bs = 0.0;
    int bi = -1;
    for (int i = lane; i < n; i += 64) {
      if (s_taken[i]) continue;
      const double s = s_score[i];
      if (bi < 0 || hsa_better(s, i, bs, bi)) {
        bs = s;
        bi = i;
      }
    }
    for (int off = 32; off >= 1; off >>= 1) {
      const double os = __shfl_xor(bs, off);
      const int oi = __shfl_xor(bi, off);
      if (oi >= 0 && (bi < 0 || hsa_better(os, oi, bs, bi))) {
        bs = os;
        bi = oi;
      }
    }
    if (lane == 0) s_taken[bi] = 1;
    __syncthreads();
  }
}

// Writes the indices i < n with s_taken[i] set, ascending, through emit(pos, i);
// returns how many there were.
template <typename Emit>
__device__ int compact_taken(const unsigned char *s_taken, int n, Emit emit) {
  const int lane = threadIdx.x;
  int count = 0;
  for (int base = 0; base < n; base += 64) {
    const int i = base + lane;
    const bool flag = i < n && s_taken[i];
    const unsigned long long mask = __ballot(flag);
    const int before = __popcll(mask & ((1ull << lane) - 1ull));
    if (flag) emit(count + before, i);
    count += __popcll(mask);
  }
  return count;
}

__global__ void __launch_bounds__(64) hsa_select_kernel(
    const double *__restrict__ qblk, const double *__restrict__ kblk,
    const double *__restrict__ kframe, int H, int D, int h_begin, int Hs, int Gq, int nb,
    int Fc, int offset, int chunk, int n_recent, int kf, int kb, int cap,
    int32_t *__restrict__ idx, int32_t *__restrict__ cnt) {
  __shared__ double s_score[kMaxHsaCand];
  __shared__ unsigned char s_taken[kMaxHsaCand];
  __shared__ int s_frames[kMaxHsaCand];
  __shared__ double qs[kMaxPoolD];
  const int lane = threadIdx.x;
  const int j = blockIdx.x % Gq;
  const int hs = (blockIdx.x / Gq) % Hs;
  const int b = blockIdx.x / (Gq * Hs);
  const int tq = j / nb;  // query frame of this query block
  const int e = offset + (tq / chunk + 1) * chunk - 1;
  const int first_recent = e - n_recent + 1;  // candidates: frames 0 .. first_recent-1
  const long long bh = (long long)b * Hs + hs;

  for (int d = lane; d < D; d += 64) qs[d] = qblk[(bh * Gq + j) * D + d];
  __syncthreads();

  // level 1: frames
  const double *kf_base = kframe + bh * Fc * D;
  for (int f = lane; f < first_recent; f += 64) {
    s_score[f] = nan_last(ordered_dot(qs, kf_base + (long long)f * D, D));
    s_taken[f] = 0;
  }
  __syncthreads();
  take_best(s_score, s_taken, first_recent, kf);
  compact_taken(s_taken, first_recent, [&](int pos, int f) {
    if (pos < kf) s_frames[pos] = f;
  });
  __syncthreads();

  // level 2: blocks of the chosen frames; candidate c is block
  // s_frames[c / nb] * nb + c % nb, so candidate order is block order
  const int nbc = kf * nb;
  const double *kb_base = kblk + bh * (long long)Fc * nb * D;
  for (int c = lane; c < nbc; c += 64) {
    const long long blk = (long long)s_frames[c / nb] * nb + c % nb;
    s_score[c] = nan_last(ordered_dot(qs, kb_base + blk * D, D));
    s_taken[c] = 0;
  }
  __syncthreads();
  take_best(s_score, s_taken, nbc, kb);

  const long long row = ((long long)b * H + h_begin + hs) * Gq + j;
  int32_t *out = idx + row * cap;
  compact_taken(s_taken, nbc, [&](int pos, int c) {
    if (pos < kb) out[pos] = s_frames[c / nb] * nb + c % nb;
  });
  const int n_rec = n_recent * nb;
  for (int r = lane; r < n_rec; r += 64) out[kb + r] = first_recent * nb + r;
  for (int p = kb + n_rec + lane; p < cap; p += 64) out[p] = -1;
  if (lane == 0) cnt[row] = kb + n_rec;
}

struct HsaShape {
  int Tq, Tk, nb, Gq, Fc, e_min, e_max;
};

fsa_status check_hsa(int32_t B, int32_t H, int32_t Nq, int32_t Nk, int32_t D, int32_t P,
                     int32_t block, int32_t q_kv_offset, int32_t chunk, int32_t h_begin,
                     int32_t h_end, int32_t n_recent, HsaShape *sh) {
  FSA_REQUIRE(B >= 0 && H >= 0 && Nq >= 0 && Nk >= 0, FSA_E_ARG, "negative size");
  FSA_REQUIRE(D >= 1 && D <= kMaxPoolD, FSA_E_SHAPE, "D=%d outside [1, %d]", D, kMaxPoolD);
  FSA_REQUIRE(P >= 1 && block >= 1 && P % block == 0, FSA_E_SHAPE,
              "P=%d is not a positive multiple of block=%d", P, block);
  FSA_REQUIRE(Nq % P == 0 && Nk % P == 0, FSA_E_SHAPE, "Nq=%d or Nk=%d is not a multiple of P=%d",
              Nq, Nk, P);
  FSA_REQUIRE(chunk >= 1, FSA_E_ARG, "chunk=%d must be >= 1", chunk);
  FSA_REQUIRE(q_kv_offset >= 0, FSA_E_ARG, "q_kv_offset=%d must be >= 0", q_kv_offset);
  FSA_REQUIRE(n_recent >= 0, FSA_E_ARG, "n_recent=%d must be >= 0", n_recent);
  FSA_REQUIRE(0 <= h_begin && h_begin <= h_end && h_end <= H, FSA_E_ARG,
              "head range [%d, %d) outside [0, %d]", h_begin, h_end, H);
  sh->Tq = Nq / P;
  sh->Tk = Nk / P;
  sh->nb = P / block;
  sh->Gq = Nq / block;
  sh->e_min = q_kv_offset + chunk - 1;
  sh->e_max = sh->Tq > 0 ? q_kv_offset + ((sh->Tq - 1) / chunk + 1) * chunk - 1 : sh->e_min;
  sh->Fc = sh->e_max - n_recent + 1;
  if (sh->Tq > 0) {
    FSA_REQUIRE(sh->e_max < sh->Tk, FSA_E_ARG,
                "the last chunk ends at KV frame %d, beyond the %d cached frames", sh->e_max,
                sh->Tk);
    FSA_REQUIRE(sh->e_min - n_recent + 1 >= 0, FSA_E_ARG,
                "n_recent=%d reaches before KV frame 0", n_recent);
    FSA_REQUIRE(sh->Fc <= kMaxHsaCand, FSA_E_ARG, "more than %d candidate frames", kMaxHsaCand);
  }
  return FSA_OK;
}

size_t hsa_workspace(int32_t B, int32_t Hs, const HsaShape &sh, int32_t D) {
  const size_t per_head = (size_t)sh.Gq + (size_t)sh.Fc * sh.nb + (size_t)sh.Fc;
  return (size_t)B * Hs * per_head * D * sizeof(double);
}

}  // namespace

extern "C" fsa_status fsa_select_hsa_workspace_size(int32_t B, int32_t H, int32_t Nq, int32_t Nk,
                                                    int32_t D, int32_t P, int32_t block,
                                                    int32_t q_kv_offset, int32_t chunk,
                                                    int32_t h_begin, int32_t h_end,
                                                    int32_t n_recent, size_t *bytes) {
  fsa::clear_error();
  FSA_REQUIRE(bytes != nullptr, FSA_E_ARG, "bytes is NULL");
  HsaShape sh;
  fsa_status st = check_hsa(B, H, Nq, Nk, D, P, block, q_kv_offset, chunk, h_begin, h_end,
                            n_recent, &sh);
  if (st != FSA_OK) return st;
  *bytes = sh.Tq > 0 ? hsa_workspace(B, h_end - h_begin, sh, D) : 0;
  return FSA_OK;
}

extern "C" fsa_status fsa_select_hsa_blocks(
    const void *q, const void *k, int32_t dt, int32_t B, int32_t H, int32_t Nq, int32_t Nk,
    int32_t D, int32_t P, int32_t block, int32_t q_kv_offset, int32_t chunk, int32_t h_begin,
    int32_t h_end, int32_t n_recent, int32_t topk_frames, int32_t topk_blocks, int32_t cap,
    int32_t *idx, int32_t *cnt, void *workspace, size_t workspace_bytes, void *stream) {
  fsa::clear_error();
  HsaShape sh;
  fsa_status st = check_hsa(B, H, Nq, Nk, D, P, block, q_kv_offset, chunk, h_begin, h_end,
                            n_recent, &sh);
  if (st != FSA_OK) return st;
  FSA_REQUIRE(dt == FSA_F32 || dt == FSA_BF16, FSA_E_DTYPE, "unknown dtype %d", dt);
  const int Hs = h_end - h_begin;
  if (B == 0 || Hs == 0 || sh.Tq == 0) return FSA_OK;
  const int n_cand_min = sh.e_min - n_recent + 1;
  FSA_REQUIRE(topk_frames >= 1 && topk_frames <= n_cand_min, FSA_E_ARG,
              "topk_frames=%d outside [1, %d] (candidate frames of the first chunk)", topk_frames,
              n_cand_min);
  FSA_REQUIRE((long long)topk_frames * sh.nb <= kMaxHsaCand, FSA_E_ARG,
              "topk_frames x blocks per frame = %lld exceeds %d", (long long)topk_frames * sh.nb,
              kMaxHsaCand);
  FSA_REQUIRE(topk_blocks >= 0 && topk_blocks <= topk_frames * sh.nb, FSA_E_ARG,
              "topk_blocks=%d outside [0, %d]", topk_blocks, topk_frames * sh.nb);
  const long long need_cap = (long long)topk_blocks + (long long)n_recent * sh.nb;
  FSA_REQUIRE(cap >= need_cap && cap >= 1 && cap <= FSA_MAX_CAP, FSA_E_CAPACITY,
              "cap=%d must hold %lld blocks and lie in [1, %d]", cap, need_cap, FSA_MAX_CAP);
  FSA_REQUIRE(q && k && idx && cnt && workspace, FSA_E_ARG, "null pointer argument");
  const size_t need = hsa_workspace(B, Hs, sh, D);
  FSA_REQUIRE(workspace_bytes >= need, FSA_E_CAPACITY, "workspace of %zu bytes < %zu needed",
              workspace_bytes, need);
  double *qblk = static_cast<double *>(workspace);
  double *kblk = qblk + (size_t)B * Hs * sh.Gq * D;
  double *kframe = kblk + (size_t)B * Hs * sh.Fc * sh.nb * D;
  hipStream_t s = fsa::as_stream(stream);
  const int Fb = sh.Fc * sh.nb;  // key blocks pooled per head
  const long long pool_blocks = (long long)B * Hs * (sh.Gq + Fb);
  FSA_REQUIRE(pool_blocks < (1LL << 31), FSA_E_SHAPE, "too many pooling segments (%lld)",
              pool_blocks);
  launch_pool(dt, q, k, H, Nq, Nk, D, block, h_begin, Hs, sh.Gq, 0, Fb, pool_blocks, qblk, kblk,
              s);
  const long long n_frames = (long long)B * Hs * sh.Fc;
  if (n_frames > 0)
    hipLaunchKernelGGL(hsa_frame_sums_kernel, dim3((unsigned)n_frames), dim3(kPoolThreads), 0, s,
                       kblk, D, sh.nb, sh.Fc, n_frames, kframe);
  hipLaunchKernelGGL(hsa_select_kernel, dim3((unsigned)(B * Hs * sh.Gq)), dim3(64), 0, s, qblk,
                     kblk, kframe, H, D, h_begin, Hs, sh.Gq, sh.nb, sh.Fc, q_kv_offset, chunk,
                     n_recent, topk_frames, topk_blocks, cap, idx, cnt);
  return fsa::check_launch("select_hsa_blocks");
}
