// Host side of frame-set construction: capacity, argument checks, the host
// builder and the validator (LVSA §2 core mechanism; Head Forcing methodology
// §2; ISPA §2 item 1).  Plain C++: the per-frame routine is the one the device
// kernel runs (frame_sets_core.h).
#include <algorithm>

#include "fsa_internal.h"
#include "frame_sets_core.h"

using fsa_sets::pos_mod;

namespace fsa {

fsa_status policy_capacity(const fsa_head_policy &p, int Tq, int Tk, int offset, int chunk,
                           int *need) {
  (void)Tq;
  (void)chunk;
  (void)offset;
  switch (p.kind) {
    case FSA_POL_FULL:
      *need = Tk;
      break;
    case FSA_POL_LVSA: {
      if (p.t_per < 1) return fsa::fail(FSA_E_ARG, "t_per=%d must be >= 1", p.t_per);
      int r = pos_mod(p.step, p.t_per);
      int n_anchor = r < Tk ? (Tk - 1 - r) / p.t_per + 1 : 0;
      int c = std::min(p.budget, Tk);
      int w = n_anchor + std::min(p.window, Tk);
      *need = std::min(Tk, std::max(c, w));
      break;
    }
    case FSA_POL_SINK_WINDOW:
      *need = std::min(Tk, std::min(p.n_sink, Tk) + std::min(p.window, Tk));
      break;
    case FSA_POL_MEMORY:
      *need = std::min(Tk, p.topk + p.n_recent);
      break;
    case FSA_POL_RANGE: {
      int lo = std::max(0, p.lo), hi = std::min(p.hi, Tk - 1);
      *need = hi >= lo ? hi - lo + 1 : 0;
      break;
    }
    default:
      return fsa::fail(FSA_E_ARG, "unknown policy kind %d", p.kind);
  }
  return FSA_OK;
}

fsa_status check_policies(int32_t B, int32_t H, int32_t Tq, int32_t Tk, int32_t offset,
                          int32_t chunk, const fsa_head_policy *pol, int32_t topk_k,
                          bool have_selected, int32_t cap, bool check_cap) {
  FSA_REQUIRE(B >= 0 && H >= 0 && Tq >= 0 && Tk >= 0, FSA_E_ARG,
              "negative size (B=%d H=%d Tq=%d Tk=%d)", B, H, Tq, Tk);
  FSA_REQUIRE(H <= FSA_MAX_HEADS, FSA_E_ARG, "H=%d exceeds FSA_MAX_HEADS=%d", H,
              FSA_MAX_HEADS);
  FSA_REQUIRE(H == 0 || pol != nullptr, FSA_E_ARG, "policies is NULL");
  FSA_REQUIRE(chunk >= 1, FSA_E_ARG, "chunk=%d must be >= 1", chunk);
  FSA_REQUIRE(Tq % chunk == 0, FSA_E_ARG, "Tq=%d is not a multiple of chunk=%d", Tq, chunk);
  FSA_REQUIRE(offset >= 0, FSA_E_ARG, "offset=%d must be >= 0", offset);
  FSA_REQUIRE(cap >= 1 && cap <= FSA_MAX_CAP, FSA_E_CAPACITY, "cap=%d outside [1, %d]", cap,
              FSA_MAX_CAP);
  for (int h = 0; h < H; ++h) {
    const fsa_head_policy &p = pol[h];
    switch (p.kind) {
      case FSA_POL_FULL:
      case FSA_POL_RANGE:
        break;
      case FSA_POL_LVSA:
        FSA_REQUIRE(p.t_per >= 1, FSA_E_ARG, "head %d: t_per=%d must be >= 1", h, p.t_per);
        FSA_REQUIRE(p.window >= 0 && p.budget >= 0, FSA_E_ARG,
                    "head %d: window=%d and budget=%d must be >= 0", h, p.window, p.budget);
        FSA_REQUIRE(offset + Tq <= Tk, FSA_E_ARG,
                    "head %d: query frames offset+Tq=%d exceed Tk=%d", h, offset + Tq, Tk);
        break;
      case FSA_POL_SINK_WINDOW:
        FSA_REQUIRE(p.window >= 0 && p.n_sink >= 0, FSA_E_ARG,
                    "head %d: window=%d and n_sink=%d must be >= 0", h, p.window, p.n_sink);
        FSA_REQUIRE(offset + Tq <= Tk, FSA_E_ARG,
                    "head %d: query chunk end offset+Tq=%d exceeds Tk=%d", h, offset + Tq, Tk);
        break;
      case FSA_POL_MEMORY:
        FSA_REQUIRE(p.n_recent >= 0 && p.topk >= 0, FSA_E_ARG,
                    "head %d: n_recent=%d and topk=%d must be >= 0", h, p.n_recent, p.topk);
        FSA_REQUIRE(have_selected, FSA_E_ARG, "head %d is MEMORY but selected is NULL", h);
        FSA_REQUIRE(p.topk <= topk_k, FSA_E_ARG,
                    "head %d: topk=%d exceeds the %d selected frames per group", h, p.topk,
                    topk_k);
        FSA_REQUIRE(offset + Tq <= Tk, FSA_E_ARG,
                    "head %d: query chunk end offset+Tq=%d exceeds Tk=%d", h, offset + Tq, Tk);
        break;
      default:
        return fsa::fail(FSA_E_ARG, "head %d: unknown policy kind %d", h, p.kind);
    }
    if (check_cap) {
      int need = 0;
      fsa_status st = policy_capacity(p, Tq, Tk, offset, chunk, &need);
      if (st != FSA_OK) return st;
      FSA_REQUIRE(need <= cap, FSA_E_CAPACITY, "head %d needs cap >= %d, got %d", h, need, cap);
    }
  }
  return FSA_OK;
}

}  // namespace fsa

extern "C" fsa_status fsa_frame_set_capacity(int32_t H, const fsa_head_policy *policies,
                                             int32_t Tq, int32_t Tk, int32_t offset,
                                             int32_t chunk, int32_t *cap_out) {
  fsa::clear_error();
  FSA_REQUIRE(cap_out != nullptr, FSA_E_ARG, "cap_out is NULL");
  FSA_REQUIRE(H >= 0 && H <= FSA_MAX_HEADS, FSA_E_ARG, "H=%d outside [0, %d]", H, FSA_MAX_HEADS);
  FSA_REQUIRE(H == 0 || policies != nullptr, FSA_E_ARG, "policies is NULL");
  FSA_REQUIRE(Tk >= 0, FSA_E_ARG, "Tk=%d must be >= 0", Tk);
  int cap = 1;
  for (int h = 0; h < H; ++h) {
    int need = 0;
    fsa_status st = fsa::policy_capacity(policies[h], Tq, Tk, offset, chunk, &need);
    if (st != FSA_OK) return st;
    cap = std::max(cap, need);
  }
  *cap_out = cap;
  return FSA_OK;
}

extern "C" fsa_status fsa_build_frame_sets_host(int32_t B, int32_t H, int32_t Tq, int32_t Tk,
                                                int32_t offset, int32_t chunk,
                                                const fsa_head_policy *policies,
                                                const int32_t *selected, int32_t topk_k,
                                                int32_t cap, int32_t *idx, int32_t *cnt) {
  fsa::clear_error();
  fsa_status st = fsa::check_policies(B, H, Tq, Tk, offset, chunk, policies, topk_k,
                                 selected != nullptr, cap, true);
  if (st != FSA_OK) return st;
  const long long total = (long long)B * H * Tq;
  if (total == 0) return FSA_OK;
  FSA_REQUIRE(idx != nullptr && cnt != nullptr, FSA_E_ARG, "idx or cnt is NULL");
  const int groups = Tq / chunk;
  for (long long i = 0; i < total; ++i) {
    const int tq = (int)(i % Tq);
    const int h = (int)((i / Tq) % H);
    const int b = (int)(i / ((long long)Tq * H));
    const fsa_head_policy &pol = policies[h];
    const int32_t *sel = nullptr;
    if (pol.kind == FSA_POL_MEMORY)
      sel = selected + (((long long)b * H + h) * groups + tq / chunk) * topk_k;
    cnt[i] = fsa_sets::build_one(pol, Tk, offset, chunk, tq, sel, cap, idx + i * cap);
  }
  return FSA_OK;
}

extern "C" fsa_status fsa_validate_frame_sets(int32_t B, int32_t H, int32_t Tq, int32_t Tk,
                                              int32_t cap, const int32_t *idx,
                                              const int32_t *cnt) {
  fsa::clear_error();
  FSA_REQUIRE(B >= 0 && H >= 0 && Tq >= 0 && Tk >= 0 && cap >= 1, FSA_E_ARG,
              "bad sizes (B=%d H=%d Tq=%d Tk=%d cap=%d)", B, H, Tq, Tk, cap);
  const long long total = (long long)B * H * Tq;
  if (total == 0) return FSA_OK;
  FSA_REQUIRE(idx != nullptr && cnt != nullptr, FSA_E_ARG, "idx or cnt is NULL");
  for (long long i = 0; i < total; ++i) {
    const int tq = (int)(i % Tq), h = (int)((i / Tq) % H), b = (int)(i / ((long long)Tq * H));
    const int n = cnt[i];
    FSA_REQUIRE(n >= 0 && n <= cap, FSA_E_LIST, "(b=%d,h=%d,t=%d): cnt=%d outside [0, %d]", b, h,
                tq, n, cap);
    for (int j = 0; j < n; ++j) {
      const int f = idx[i * cap + j];
      FSA_REQUIRE(f >= 0 && f < Tk, FSA_E_LIST, "(b=%d,h=%d,t=%d): entry %d = %d outside [0, %d)",
                  b, h, tq, j, f, Tk);
      FSA_REQUIRE(j == 0 || f > idx[i * cap + j - 1], FSA_E_LIST,
                  "(b=%d,h=%d,t=%d): entry %d = %d not above the previous entry", b, h, tq, j, f);
    }
  }
  return FSA_OK;
}
