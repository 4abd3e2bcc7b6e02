// Frame-set construction on the device: one thread per (b, h, query frame)
// runs the routine of frame_sets_core.h (LVSA §2 core mechanism; Head Forcing
// methodology §2; ISPA §2 item 1).  The host entry points and the argument
// checks are in frame_sets_host.cpp.
#include "fsa_internal.h"
#include "frame_sets_core.h"

namespace {

struct PolicyArray {
  fsa_head_policy p[FSA_MAX_HEADS];
};

__global__ void build_frame_sets_kernel(int B, int H, int Tq, int Tk, int offset, int chunk,
                                        PolicyArray pols, const int32_t *__restrict__ selected,
                                        int topk_k, int cap, int32_t *__restrict__ idx,
                                        int32_t *__restrict__ cnt) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
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
  cnt[i] = fsa_sets::build_one(pol, Tk, offset, chunk, tq, sel, cap, idx + i * cap);
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
  const int threads = 64;
  const long long blocks = (total + threads - 1) / threads;
  FSA_REQUIRE(blocks < (1LL << 31), FSA_E_ARG, "too many query frames (%lld)", total);
  hipLaunchKernelGGL(build_frame_sets_kernel, dim3((unsigned)blocks), dim3(threads), 0,
                     fsa::as_stream(stream), B, H, Tq, Tk, offset, chunk, arr, selected,
                     topk_k, cap, idx, cnt);
  return fsa::check_launch("build_frame_sets");
}

