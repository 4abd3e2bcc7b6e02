// Frame-set construction on the device: one wavefront per (b, h, query
// frame) applies the membership test of frame_sets_core.h (LVSA §2 core
// mechanism; Head Forcing methodology §2; ISPA §2 item 1) to 64 frames at a
// time, one per lane, and writes the kept frames in ascending order through
// a ballot prefix count; the host routine runs the same test frame by frame.
// The host entry points and the argument checks are in frame_sets_host.cpp.
#include "fsa_internal.h"
#include "frame_sets_core.h"

namespace {

struct PolicyArray {
  fsa_head_policy p[FSA_MAX_HEADS];
};

constexpr int kListsPerBlock = 4;  // one wavefront per list

__global__ void __launch_bounds__(64 * kListsPerBlock) build_frame_sets_kernel(
    int B, int H, int Tq, int Tk, int offset, int chunk, PolicyArray pols,
    const int32_t *__restrict__ selected, int topk_k, int cap, int32_t *__restrict__ idx,
    int32_t *__restrict__ cnt) {
  const int lane = threadIdx.x % 64;
  const long long i = (long long)blockIdx.x * kListsPerBlock + threadIdx.x / 64;
  const long long total = (long long)B * H * Tq;
  if (i >= total) return;
  const int tq = (int)(i % Tq);
  const int h = (int)((i / Tq) % H);
  const int b = (int)(i / ((long long)Tq * H));
  const fsa_head_policy &pol = pols.p[h];
  const int groups = Tq / chunk;
  const int32_t *sel = nullptr;
  if (pol.kind == FSA_POL_MEMORY)
    sel = selected + (((long long)b * H + h) * groups + tq / chunk) * topk_k;
  const fsa_sets::FrameTest ft = fsa_sets::frame_test(pol, Tk, offset, chunk, tq, sel);
  int32_t *out = idx + i * cap;
  const unsigned long long below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  int count = 0;
  for (int base = 0; base < Tk && count < cap; base += 64) {
    const int f = base + lane;
    const bool keep = f < Tk && fsa_sets::keep_frame(ft, f);
    const unsigned long long mask = __ballot(keep);
    const int pos = count + __popcll(mask & below);
    if (keep && pos < cap) out[pos] = f;
    count += __popcll(mask);
  }
  const int n = count < cap ? count : cap;
  for (int p = n + lane; p < cap; p += 64) out[p] = -1;
  if (lane == 0) cnt[i] = n;
}

}  // namespace

extern "C" fsa_status fsa_build_frame_sets(int32_t B, int32_t H, int32_t Tq, int32_t Tk,
                                           int32_t offset, int32_t chunk,
                                           const fsa_head_policy *policies,
                                           const int32_t *selected, int32_t topk_k, int32_t cap,
                                           int32_t *idx, int32_t *cnt, void *stream) {
  fsa::clear_error();
  fsa_status st = fsa::check_policies(B, H, Tq, Tk, offset, chunk, policies, topk_k,
                                 selected != nullptr, cap, true);
  if (st != FSA_OK) return st;
  const long long total = (long long)B * H * Tq;
  if (total == 0) return FSA_OK;
  FSA_REQUIRE(idx != nullptr && cnt != nullptr, FSA_E_ARG, "idx or cnt is NULL");
  PolicyArray arr{};
  for (int h = 0; h < H; ++h) arr.p[h] = policies[h];
  const long long blocks = (total + kListsPerBlock - 1) / kListsPerBlock;
  FSA_REQUIRE(blocks < (1LL << 31), FSA_E_ARG, "too many query frames (%lld)", total);
  hipLaunchKernelGGL(build_frame_sets_kernel, dim3((unsigned)blocks), dim3(64 * kListsPerBlock), 0,
                     fsa::as_stream(stream), B, H, Tq, Tk, offset, chunk, arr, selected,
                     topk_k, cap, idx, cnt);
  return fsa::check_launch("build_frame_sets");
}

