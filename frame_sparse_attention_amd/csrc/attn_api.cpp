// C entry points of the sparse frame attention: argument validation and
// dispatch to the float32 or the bfloat16 (matrix-core) kernels.
#include <cmath>

#include "fsa_internal.h"

namespace fsa {
fsa_status launch_attn_f32(const float *q, const float *k, const float *v, const int32_t *idx,
                           const int32_t *cnt, int cap, int B, int H, int Nq, int Nk, int D,
                           int P, float scale, float *o, float *lse, hipStream_t stream);
fsa_status launch_prepare_values_bf16(const void *v, int B, int H, int Nk, int D, void *prepared,
                                      hipStream_t stream);
fsa_status launch_attn_bf16_prepared(const void *q, const void *k, const void *prepared,
                                     const int32_t *idx, const int32_t *cnt, int cap,
                                     const int32_t *idx_b, const int32_t *cnt_b, int cap_b,
                                     int B, int H, int Nq, int Nk, int D, int P, float scale,
                                     float *o_first, float *lse_first, float *o, float *lse,
                                     int splits, hipStream_t stream);
size_t attn_bf16_workspace(long long heads, int Nk, int D);
fsa_status launch_merge_splits(const float *o_parts, const float *lse_parts, int S,
                               long long rows, int D, float *o, float *lse, hipStream_t stream);
}  // namespace fsa

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

fsa_status check_common(int32_t dt, int32_t B, int32_t H, int32_t Nk, int32_t D) {
  FSA_REQUIRE(dt == FSA_F32 || dt == FSA_BF16, FSA_E_DTYPE, "unknown dtype %d", dt);
  FSA_REQUIRE(D == 64 || D == 128, FSA_E_DTYPE, "head_dim D=%d is not 64 or 128", D);
  FSA_REQUIRE(B >= 0 && H >= 0 && Nk >= 0, FSA_E_ARG, "negative size (B=%d H=%d Nk=%d)", B, H,
              Nk);
  return FSA_OK;
}

}  // namespace

extern "C" fsa_status fsa_sparse_frame_attn_workspace_size(int32_t dt, int32_t B, int32_t H,
                                                           int32_t Nk, int32_t D,
                                                           size_t *bytes) {
  fsa::clear_error();
  FSA_REQUIRE(bytes != nullptr, FSA_E_ARG, "bytes is NULL");
  fsa_status st = check_common(dt, B, H, Nk, D);
  if (st != FSA_OK) return st;
  *bytes = dt == FSA_BF16 ? fsa::attn_bf16_workspace((long long)B * H, Nk, D) : 0;
  return FSA_OK;
}

// Checks shared by the attention entry points; returns FSA_OK with *skip set
// when there is nothing to compute.
fsa_status check_attn(const void *q, const void *k, int32_t dt, int32_t B, int32_t H, int32_t Nq,
                      int32_t Nk, int32_t D, int32_t P, const int32_t *idx, const int32_t *cnt,
                      int32_t cap, float scale, const float *o, const float *lse, bool *skip) {
  fsa_status st = check_common(dt, B, H, Nk, D);
  if (st != FSA_OK) return st;
  FSA_REQUIRE(Nq >= 0, FSA_E_ARG, "Nq=%d must be >= 0", Nq);
  FSA_REQUIRE(P >= 1, FSA_E_SHAPE, "P=%d must be >= 1", P);
  FSA_REQUIRE(Nq % P == 0, FSA_E_SHAPE, "Nq=%d is not a multiple of P=%d", Nq, P);
  FSA_REQUIRE(Nk % P == 0, FSA_E_SHAPE, "Nk=%d is not a multiple of P=%d", Nk, P);
  FSA_REQUIRE(cap >= 1 && cap <= FSA_MAX_CAP, FSA_E_CAPACITY, "cap=%d outside [1, %d]", cap,
              FSA_MAX_CAP);
  FSA_REQUIRE(std::isfinite(scale), FSA_E_ARG, "scale is not finite");
  *skip = (long long)B * H * Nq == 0;
  if (*skip) return FSA_OK;
  FSA_REQUIRE(q && o && lse && idx && cnt, FSA_E_ARG, "null pointer argument");
  FSA_REQUIRE(Nk == 0 || k, FSA_E_ARG, "k or v is NULL");
  return FSA_OK;
}

extern "C" fsa_status fsa_prepare_values(const void *v, int32_t dt, int32_t B, int32_t H,
                                         int32_t Nk, int32_t D, void *prepared,
                                         size_t prepared_bytes, void *stream) {
  fsa::clear_error();
  fsa_status st = check_common(dt, B, H, Nk, D);
  if (st != FSA_OK) return st;
  FSA_REQUIRE(dt == FSA_BF16, FSA_E_DTYPE, "prepared values exist for bf16 only");
  const size_t need = fsa::attn_bf16_workspace((long long)B * H, Nk, D);
  if (need == 0) return FSA_OK;
  FSA_REQUIRE(v && prepared, FSA_E_ARG, "null pointer argument");
  FSA_REQUIRE(aligned16(v) && aligned16(prepared), FSA_E_ARG,
              "v and the prepared buffer must be 16-byte aligned");
  FSA_REQUIRE(prepared_bytes >= need, FSA_E_CAPACITY, "prepared buffer of %zu bytes < %zu needed",
              prepared_bytes, need);
  return fsa::launch_prepare_values_bf16(v, B, H, Nk, D, prepared, fsa::as_stream(stream));
}

extern "C" fsa_status fsa_sparse_frame_attn_prepared(
    const void *q, const void *k, const void *prepared, int32_t dt, int32_t B, int32_t H,
    int32_t Nq, int32_t Nk, int32_t D, int32_t P, const int32_t *idx, const int32_t *cnt,
    int32_t cap, float scale, float *o, float *lse, size_t prepared_bytes, void *stream) {
  fsa::clear_error();
  bool skip = false;
  fsa_status st = check_attn(q, k, dt, B, H, Nq, Nk, D, P, idx, cnt, cap, scale, o, lse, &skip);
  if (st != FSA_OK || skip) return st;
  FSA_REQUIRE(dt == FSA_BF16, FSA_E_DTYPE, "prepared values exist for bf16 only");
  const size_t need = fsa::attn_bf16_workspace((long long)B * H, Nk, D);
  FSA_REQUIRE(need == 0 || prepared, FSA_E_ARG, "k or v is NULL");
  FSA_REQUIRE(prepared_bytes >= need, FSA_E_CAPACITY, "prepared buffer of %zu bytes < %zu needed",
              prepared_bytes, need);
  FSA_REQUIRE(aligned16(q) && aligned16(k) && aligned16(prepared) && aligned16(o), FSA_E_ARG,
              "q, k, o and the prepared buffer must be 16-byte aligned");
  if (scale <= 0.f) scale = 1.f / std::sqrt((float)D);
  return fsa::launch_attn_bf16_prepared(q, k, prepared, idx, cnt, cap, nullptr, nullptr, 0, B, H,
                                        Nq, Nk, D, P, scale, nullptr, nullptr, o, lse, 1,
                                        fsa::as_stream(stream));
}

extern "C" fsa_status fsa_sparse_frame_attn_dual_prepared(
    const void *q, const void *k, const void *prepared, int32_t dt, int32_t B, int32_t H,
    int32_t Nq, int32_t Nk, int32_t D, int32_t P, const int32_t *idx_a, const int32_t *cnt_a,
    int32_t cap_a, const int32_t *idx_b, const int32_t *cnt_b, int32_t cap_b, float scale,
    float *o_a, float *lse_a, float *o_ab, float *lse_ab, size_t prepared_bytes, void *stream) {
  fsa::clear_error();
  bool skip = false;
  fsa_status st =
      check_attn(q, k, dt, B, H, Nq, Nk, D, P, idx_a, cnt_a, cap_a, scale, o_ab, lse_ab, &skip);
  if (st != FSA_OK || skip) return st;
  FSA_REQUIRE(dt == FSA_BF16, FSA_E_DTYPE, "prepared values exist for bf16 only");
  FSA_REQUIRE(idx_b && cnt_b && o_a && lse_a, FSA_E_ARG, "null pointer argument");
  FSA_REQUIRE(cap_b >= 1 && cap_a + cap_b <= FSA_MAX_CAP, FSA_E_CAPACITY,
              "cap_a + cap_b = %d outside [2, %d]", cap_a + cap_b, FSA_MAX_CAP);
  const size_t need = fsa::attn_bf16_workspace((long long)B * H, Nk, D);
  FSA_REQUIRE(need == 0 || prepared, FSA_E_ARG, "k or v is NULL");
  FSA_REQUIRE(prepared_bytes >= need, FSA_E_CAPACITY, "prepared buffer of %zu bytes < %zu needed",
              prepared_bytes, need);
  FSA_REQUIRE(aligned16(q) && aligned16(k) && aligned16(prepared) && aligned16(o_a) &&
                  aligned16(o_ab),
              FSA_E_ARG, "q, k, the outputs and the prepared buffer must be 16-byte aligned");
  if (scale <= 0.f) scale = 1.f / std::sqrt((float)D);
  return fsa::launch_attn_bf16_prepared(q, k, prepared, idx_a, cnt_a, cap_a, idx_b, cnt_b, cap_b,
                                        B, H, Nq, Nk, D, P, scale, o_a, lse_a, o_ab, lse_ab, 1,
                                        fsa::as_stream(stream));
}

extern "C" fsa_status fsa_sparse_frame_attn(const void *q, const void *k, const void *v,
                                            int32_t dt, int32_t B, int32_t H, int32_t Nq,
                                            int32_t Nk, int32_t D, int32_t P, const int32_t *idx,
                                            const int32_t *cnt, int32_t cap, float scale,
                                            float *o, float *lse, void *workspace,
                                            size_t workspace_bytes, void *stream) {
  fsa::clear_error();
  bool skip = false;
  fsa_status st = check_attn(q, k, dt, B, H, Nq, Nk, D, P, idx, cnt, cap, scale, o, lse, &skip);
  if (st != FSA_OK || skip) return st;
  FSA_REQUIRE(Nk == 0 || v, FSA_E_ARG, "k or v is NULL");
  if (scale <= 0.f) scale = 1.f / std::sqrt((float)D);
  hipStream_t s = fsa::as_stream(stream);
  if (dt == FSA_F32)
    return fsa::launch_attn_f32(static_cast<const float *>(q), static_cast<const float *>(k),
                                static_cast<const float *>(v), idx, cnt, cap, B, H, Nq, Nk, D,
                                P, scale, o, lse, s);
  const size_t need = fsa::attn_bf16_workspace((long long)B * H, Nk, D);
  FSA_REQUIRE(need == 0 || workspace != nullptr, FSA_E_ARG, "workspace is NULL");
  FSA_REQUIRE(workspace_bytes >= need, FSA_E_CAPACITY, "workspace of %zu bytes < %zu needed",
              workspace_bytes, need);
  FSA_REQUIRE(aligned16(q) && aligned16(k) && aligned16(v) && aligned16(o) &&
                  aligned16(workspace),
              FSA_E_ARG, "q, k, v, o and the workspace must be 16-byte aligned (bf16 path)");
  if (need > 0) {
    st = fsa::launch_prepare_values_bf16(v, B, H, Nk, D, workspace, s);
    if (st != FSA_OK) return st;
  }
  return fsa::launch_attn_bf16_prepared(q, k, workspace, idx, cnt, cap, nullptr, nullptr, 0, B, H,
                                        Nq, Nk, D, P, scale, nullptr, nullptr, o, lse, 1, s);
}

namespace {
constexpr int kMaxSplits = 16;
constexpr long long kCUs = 256;                // compute units of an MI355X
constexpr long long kBlockSlots = kCUs * 2;     // resident attention blocks: two per CU

// Splits for a grid of `blocks` attention blocks.  Measured on the AR-chunk
// shapes (468 blocks): one part is fastest for its short lists and two parts
// gain 4 % on 49-frame lists, so parts are added only when the grid has fewer
// blocks than compute units, enough to give every unit about two.
int default_splits(long long blocks) {
  if (blocks <= 0 || blocks >= kCUs) return 1;
  long long s = (kBlockSlots + blocks - 1) / blocks;
  return (int)(s > 8 ? 8 : s);
}
}  // namespace

extern "C" fsa_status fsa_attn_split_plan(int32_t B, int32_t H, int32_t Nq, int32_t D, int32_t P,
                                          int32_t splits_req, int32_t *splits,
                                          size_t *workspace_bytes) {
  fsa::clear_error();
  FSA_REQUIRE(splits && workspace_bytes, FSA_E_ARG, "null pointer argument");
  FSA_REQUIRE(B >= 0 && H >= 0 && Nq >= 0, FSA_E_ARG, "negative size");
  FSA_REQUIRE(D == 64 || D == 128, FSA_E_DTYPE, "head_dim D=%d is not 64 or 128", D);
  FSA_REQUIRE(P >= 1 && Nq % P == 0, FSA_E_SHAPE, "Nq=%d is not a multiple of P=%d", Nq, P);
  FSA_REQUIRE(splits_req <= kMaxSplits, FSA_E_ARG, "splits=%d above %d", splits_req, kMaxSplits);
  const long long qtiles = (P + 127) / 128;
  const int S = splits_req >= 1 ? splits_req
                                : default_splits((long long)B * H * (Nq / P) * qtiles);
  *splits = S;
  *workspace_bytes = S > 1 ? (size_t)S * B * H * Nq * (size_t)(D + 1) * sizeof(float) : 0;
  return FSA_OK;
}

extern "C" fsa_status fsa_sparse_frame_attn_prepared_split(
    const void *q, const void *k, const void *prepared, int32_t dt, int32_t B, int32_t H,
    int32_t Nq, int32_t Nk, int32_t D, int32_t P, const int32_t *idx, const int32_t *cnt,
    int32_t cap, float scale, int32_t splits, float *o, float *lse, size_t prepared_bytes,
    void *workspace, size_t workspace_bytes, void *stream) {
  fsa::clear_error();
  bool skip = false;
  fsa_status st = check_attn(q, k, dt, B, H, Nq, Nk, D, P, idx, cnt, cap, scale, o, lse, &skip);
  if (st != FSA_OK) return st;
  FSA_REQUIRE(splits >= 1 && splits <= kMaxSplits, FSA_E_ARG, "splits=%d outside [1, %d]",
              splits, kMaxSplits);
  if (skip) return FSA_OK;
  FSA_REQUIRE(dt == FSA_BF16, FSA_E_DTYPE, "prepared values exist for bf16 only");
  const size_t need = fsa::attn_bf16_workspace((long long)B * H, Nk, D);
  FSA_REQUIRE(need == 0 || prepared, FSA_E_ARG, "k or v is NULL");
  FSA_REQUIRE(prepared_bytes >= need, FSA_E_CAPACITY, "prepared buffer of %zu bytes < %zu needed",
              prepared_bytes, need);
  const long long rows = (long long)B * H * Nq;
  const size_t parts = splits > 1 ? (size_t)splits * rows * (size_t)(D + 1) * sizeof(float) : 0;
  FSA_REQUIRE(parts == 0 || workspace, FSA_E_ARG, "workspace is NULL");
  FSA_REQUIRE(workspace_bytes >= parts, FSA_E_CAPACITY, "workspace of %zu bytes < %zu needed",
              workspace_bytes, parts);
  FSA_REQUIRE(aligned16(q) && aligned16(k) && aligned16(prepared) && aligned16(o) &&
                  aligned16(workspace),
              FSA_E_ARG, "q, k, o, the workspace and the prepared buffer must be 16-byte aligned");
  if (scale <= 0.f) scale = 1.f / std::sqrt((float)D);
  hipStream_t s = fsa::as_stream(stream);
  if (splits == 1)
    return fsa::launch_attn_bf16_prepared(q, k, prepared, idx, cnt, cap, nullptr, nullptr, 0, B,
                                          H, Nq, Nk, D, P, scale, nullptr, nullptr, o, lse, 1, s);
  float *o_parts = static_cast<float *>(workspace);
  float *lse_parts = o_parts + (size_t)splits * rows * D;
  st = fsa::launch_attn_bf16_prepared(q, k, prepared, idx, cnt, cap, nullptr, nullptr, 0, B, H,
                                      Nq, Nk, D, P, scale, nullptr, nullptr, o_parts, lse_parts,
                                      splits, s);
  if (st != FSA_OK) return st;
  return fsa::launch_merge_splits(o_parts, lse_parts, splits, rows, D, o, lse, s);
}
