// Device helpers shared by the attention kernels: turning a frame list into
// runs of consecutive frames, and the XCD-aware tile order.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "fsa_internal.h"

namespace fsa {

// Runs of consecutive frames of one list, in LDS: run r covers frames
// run_lo[r] .. run_hi[r].  Consecutive frames are contiguous in memory
// (token n = f*P + p), so one run is one contiguous key range and the tile
// loop walks it without per-frame tails (LVSA §2: the attended set is a union
// of an interval and the anchors, so a list of 21-33 frames is 5-15 runs).
struct RunList {
  int *lo;
  int *hi;
};

// Builds the runs of list[0..n) (n clamped to [0, cap]) with wavefront 0 of
// the block; entries outside [0, Tk) are skipped.  Returns the run count to
// every thread (after a block barrier).  `s_count` is one LDS int.
__device__ inline int build_runs(const int32_t *__restrict__ list, int n, int cap, int Tk,
                                 RunList runs, int *s_count) {
  n = n < 0 ? 0 : (n > cap ? cap : n);
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    int carry = 0;
    for (int base = 0; base < n; base += 64) {
      const int i = base + lane;
      const int f = i < n ? list[i] : -1;
      const int fp = (i < n && i > 0) ? list[i - 1] : -1;
      const int fn = (i + 1 < n) ? list[i + 1] : -1;
      const bool valid = i < n && f >= 0 && f < Tk;
      const bool pvalid = fp >= 0 && fp < Tk;
      const bool nvalid = fn >= 0 && fn < Tk;
      const bool starts = valid && !(pvalid && fp == f - 1);
      const bool ends = valid && !(nvalid && fn == f + 1);
      const uint64_t smask = __ballot(starts);
      const int before = carry + __popcll(smask & lt);
      if (starts) runs.lo[before] = f;
      // the run an entry belongs to is the one opened by the latest start at or before it
      if (ends) runs.hi[before + (starts ? 1 : 0) - 1] = f;
      carry += __popcll(smask);
    }
    if (lane == 0) *s_count = carry;
  }
  __syncthreads();
  return *s_count;
}

// Maps the hardware block id to a logical tile id so that consecutive
// logical tiles run on the same XCD.  Blocks are dealt to the 8 XCDs of an
// MI355X round-robin (block b on XCD b % 8); each XCD gets one contiguous
// range of logical tiles, so the query tiles of one (head, frame) -- which
// read the same K/V frames -- share that XCD's L2.
__device__ inline int xcd_logical_tile(int bid, int nblk) {
  constexpr int kXcd = 8;
  const int per = nblk / kXcd, rem = nblk % kXcd;
  const int xcd = bid % kXcd, local = bid / kXcd;
  return xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
}

// Head order for small grids.  The contiguous per-XCD tile ranges hold whole
// heads in turn, so when heads differ in cost (per-head policies: local,
// anchor and memory heads) the XCDs finish at different times.  Heads are
// ranked by cost, heaviest first (ties by index), and dealt from both ends of
// that ranking -- heaviest, lightest, second heaviest, ... -- so each XCD range
// pairs heavy heads with light ones.  Equal costs keep the plain order.  The
// cost of a head is the number of frames its query frames list (list B
// included).  Every block computes the same permutation; `s_tmp` is 128 LDS
// ints; returns the head placed at position `slot`.
__device__ inline int balanced_head(int slot, int G, int Tq, const int32_t *cnt_a, int cap_a,
                                    const int32_t *cnt_b, int cap_b, int *s_tmp) {
  const int l = threadIdx.x;
  if (l < 64) {
    int c = 0;
    if (l < G) {
      for (int t = 0; t < Tq; ++t) {
        int n = cnt_a[(long long)l * Tq + t];
        c += n < 0 ? 0 : (n > cap_a ? cap_a : n);
        if (cnt_b != nullptr) {
          n = cnt_b[(long long)l * Tq + t];
          c += n < 0 ? 0 : (n > cap_b ? cap_b : n);
        }
      }
    }
    s_tmp[l] = c;
  }
  __syncthreads();
  if (l < G) {
    const int c = s_tmp[l], c0 = s_tmp[0];
    int rank = 0;
    bool equal = true;
    for (int j = 0; j < G; ++j) {
      const int cj = s_tmp[j];
      rank += (cj > c || (cj == c && j < l)) ? 1 : 0;
      equal = equal && cj == c0;
    }
    const int pos = equal ? l : (rank < (G + 1) / 2 ? 2 * rank : 2 * (G - 1 - rank) + 1);
    s_tmp[64 + pos] = l;
  }
  __syncthreads();
  return s_tmp[64 + slot];
}

// Block order for grids of 257 to 512 blocks, which are resident all at once
// at two blocks per CU.  On an MI355X the blocks of one XCD (local index
// k = bid / 8) land so that k and k + 32 share a CU and k < 32 without such
// a partner runs alone (measured with the hardware's CU ids).  A CU then runs
// until its longer block ends, and that block speeds up once its partner is
// done.  The blocks are ranked by the cost of their list, heaviest first; the
// 32 heaviest of the first 256 go to XCD 0, the next 32 to XCD 1, and so on,
// the heaviest of each XCD's share to its unpartnered slots.  The remaining
// blocks, the lightest, fill the partner slots, lightest paired with
// heaviest, the lightest share on XCD 0.  Each XCD holds two contiguous
// ranges of the ranking, so the query tiles of one list mostly share an L2.
// L lists of qtiles blocks each make the N = L * qtiles blocks of the grid
// (257 <= N <= 512); `s_tmp` holds 2 * L LDS ints and `s_flag` one.  Returns
// false (and leaves the outputs) when every list costs the same, where the
// contiguous order is better.
__device__ inline bool paired_list_tile(int bid, int qtiles, int L, const int32_t *cnt_a,
                                        int cap_a, const int32_t *cnt_b, int cap_b, int *s_tmp,
                                        int *s_flag, int *list_out, int *qt_out) {
  constexpr int kXcd = 8, kSlots = 32;  // CUs per XCD
  const int nt = blockDim.x;
  if (threadIdx.x == 0) *s_flag = 0;
  for (int l = threadIdx.x; l < L; l += nt) {
    int n = cnt_a[l];
    int c = n < 0 ? 0 : (n > cap_a ? cap_a : n);
    if (cnt_b != nullptr) {
      n = cnt_b[l];
      c += n < 0 ? 0 : (n > cap_b ? cap_b : n);
    }
    s_tmp[l] = c;
  }
  __syncthreads();
  for (int l = threadIdx.x; l < L; l += nt) {
    const int c = s_tmp[l];
    int rank = 0;
    bool equal = true;
    for (int j = 0; j < L; ++j) {
      const int cj = s_tmp[j];
      rank += (cj > c || (cj == c && j < l)) ? 1 : 0;
      equal = equal && cj == c;
    }
    s_tmp[L + rank] = l;
    if (!equal) *s_flag = 1;
  }
  __syncthreads();
  if (*s_flag == 0) return false;
  const int N = L * qtiles;
  const int xcd = bid % kXcd, k = bid / kXcd;
  const int per = N / kXcd, rem = N % kXcd;
  const int s_x = per + (xcd < rem ? 1 : 0) - kSlots;        // partnered slots of this XCD
  const int p_x = xcd * (per - kSlots) + (xcd < rem ? xcd : rem);  // of the XCDs before it
  int i;  // position of this block in the ranking
  if (k < kSlots)
    i = kSlots * xcd + (k >= s_x ? k - s_x : kSlots - s_x + k);
  else
    i = N - p_x - s_x + (s_x - 1 - (k - kSlots));
  *list_out = s_tmp[L + i / qtiles];
  *qt_out = i % qtiles;
  return true;
}

}  // namespace fsa
