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
// Arithmetic (fixed, so the lists are bit-reproducible): a block sum and a
// frame sum are each the exact sum of their tokens rounded once to float64
// (pooling.h); a score adds rounded products in ascending channel order;
// ranking is (score descending, index ascending).  Three launches:
//   pool       float64 partial sums of the pieces of every query block and
//              every key block of the candidate frames
//   finalize   exact query-block, key-block and key-frame sums (a frame's
//              sum from the pieces of its blocks)
//   select     one block per (b, h, query block), one thread per candidate
//              up to 256: frame scores, the kf
//              best by rank, block scores over the chosen frames, the kb best
//              by rank, then the ascending list with the recent frames.
#pragma clang fp contract(off)

#include "pooling.h"

namespace {

constexpr int kMaxHsaCand = 4096;  // candidate frames, and candidate blocks per query block

__global__ void __launch_bounds__(256) hsa_select_kernel(
    const double *__restrict__ qblk, const double *__restrict__ kblk,
    const double *__restrict__ kframe, int H, int D, int h_begin, int Hs, int Gq, int nb,
    int Fc, int offset, int chunk, int n_recent, int kf, int kb, int cap,
    int32_t *__restrict__ idx, int32_t *__restrict__ cnt) {
  __shared__ double s_score[kMaxHsaCand];
  __shared__ unsigned char s_taken[kMaxHsaCand];
  __shared__ int s_frames[kMaxHsaCand];
  __shared__ double qs[kMaxPoolD];
  const int lane = threadIdx.x, nt = blockDim.x;
  const int j = blockIdx.x % Gq;
  const int hs = (blockIdx.x / Gq) % Hs;
  const int b = blockIdx.x / (Gq * Hs);
  const int tq = j / nb;  // query frame of this query block
  const int e = offset + (tq / chunk + 1) * chunk - 1;
  const int first_recent = e - n_recent + 1;  // candidates: frames 0 .. first_recent-1
  const long long bh = (long long)b * Hs + hs;

  for (int d = lane; d < D; d += nt) qs[d] = qblk[(bh * Gq + j) * D + d];
  __syncthreads();

  // level 1: frames
  const double *kf_base = kframe + bh * Fc * D;
  for (int f = lane; f < first_recent; f += nt)
    s_score[f] = nan_last(ordered_dot(qs, kf_base + (long long)f * D, D));
  __syncthreads();
  take_best(s_score, s_taken, first_recent, kf);
  compact_taken(s_taken, first_recent, kf, [&](int pos, int f) { s_frames[pos] = f; });
  __syncthreads();

  // level 2: blocks of the chosen frames; candidate c is block
  // s_frames[c / nb] * nb + c % nb, so candidate order is block order
  const int nbc = kf * nb;
  const double *kb_base = kblk + bh * (long long)Fc * nb * D;
  for (int c = lane; c < nbc; c += nt) {
    const long long blk = (long long)s_frames[c / nb] * nb + c % nb;
    s_score[c] = nan_last(ordered_dot(qs, kb_base + blk * D, D));
  }
  __syncthreads();
  take_best(s_score, s_taken, nbc, kb);

  const long long row = ((long long)b * H + h_begin + hs) * Gq + j;
  int32_t *out = idx + row * cap;
  compact_taken(s_taken, nbc, kb,
                [&](int pos, int c) { out[pos] = s_frames[c / nb] * nb + c % nb; });
  const int n_rec = n_recent * nb;
  for (int r = lane; r < n_rec; r += nt) out[kb + r] = first_recent * nb + r;
  for (int p = kb + n_rec + lane; p < cap; p += nt) out[p] = -1;
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

// Workspace layout for Hs selected heads: query-block, key-block and
// key-frame sums, then the pieces of the query-block and key-block families.
// With ws == nullptr only the size is computed.
struct HsaLayout {
  SegFamily qf, kf;
  double *qblk, *kblk, *kframe;
  size_t bytes;
};
HsaLayout hsa_layout(const void *q, const void *k, int B, int H, int Nq, int Nk, int D,
                     int block, int h_begin, int Hs, const HsaShape &sh, void *ws) {
  HsaLayout L{};
  L.qf = make_family(q, Nq, 0, block, sh.Gq, H, h_begin, Hs);
  L.kf = make_family(k, Nk, 0, block, sh.Fc * sh.nb, H, h_begin, Hs);
  const size_t qb = align256((size_t)B * Hs * sh.Gq * D * sizeof(double));
  const size_t kb = align256((size_t)B * Hs * sh.Fc * sh.nb * D * sizeof(double));
  const size_t kfb = align256((size_t)B * Hs * sh.Fc * D * sizeof(double));
  L.bytes = qb + kb + kfb + family_part_bytes(L.qf, B, D) + family_part_bytes(L.kf, B, D);
  if (ws != nullptr) {
    unsigned char *p = static_cast<unsigned char *>(ws);
    L.qblk = reinterpret_cast<double *>(p);
    p += qb;
    L.kblk = reinterpret_cast<double *>(p);
    p += kb;
    L.kframe = reinterpret_cast<double *>(p);
    p += kfb;
    place_family(L.qf, B, D, &p);
    place_family(L.kf, B, D, &p);
  }
  return L;
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
  *bytes = sh.Tq > 0 ? hsa_layout(nullptr, nullptr, B, H, Nq, Nk, D, block, h_begin,
                                  h_end - h_begin, sh, nullptr).bytes
                     : 0;
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
  HsaLayout L = hsa_layout(q, k, B, H, Nq, Nk, D, block, h_begin, Hs, sh, nullptr);
  FSA_REQUIRE(workspace_bytes >= L.bytes, FSA_E_CAPACITY, "workspace of %zu bytes < %zu needed",
              workspace_bytes, L.bytes);
  L = hsa_layout(q, k, B, H, Nq, Nk, D, block, h_begin, Hs, sh, workspace);
  hipStream_t s = fsa::as_stream(stream);
  const long long pieces = (long long)(family_pieces(L.qf, B) + family_pieces(L.kf, B));
  FSA_REQUIRE(pieces < (1LL << 31), FSA_E_SHAPE, "too many pooling pieces (%lld)", pieces);
  // one-piece blocks are summed exactly by the pooling kernel itself; frames
  // (nb blocks each, or blocks of several pieces) go through finalize
  SegFamily qf = L.qf, kf = L.kf;
  if (qf.pieces == 1) qf.direct = L.qblk;
  if (kf.pieces == 1) kf.direct = L.kblk;
  launch_pool(dt, pool_vec(dt, D, q, k), qf, kf, B, D, s);
  launch_finalize(dt, qf.pieces == 1 ? no_final() : FinalFamily{L.qf, 1, L.qblk},
                  kf.pieces == 1 ? no_final() : FinalFamily{L.kf, 1, L.kblk},
                  FinalFamily{L.kf, sh.nb, L.kframe}, B, D, s);
  // one thread per candidate of the larger level, in whole wavefronts, up to 256
  const int most = sh.Fc > topk_frames * sh.nb ? sh.Fc : topk_frames * sh.nb;
  const int threads = most > 192 ? 256 : (most + 63) / 64 * 64;
  hipLaunchKernelGGL(hsa_select_kernel, dim3((unsigned)(B * Hs * sh.Gq)), dim3(threads), 0, s,
                     L.qblk, L.kblk, L.kframe, H, D, h_begin, Hs, sh.Gq, sh.nb, sh.Fc,
                     q_kv_offset, chunk, n_recent, topk_frames, topk_blocks, cap, idx, cnt);
  return fsa::check_launch("select_hsa_blocks");
}
