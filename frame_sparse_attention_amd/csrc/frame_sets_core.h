// Frame-set construction shared by the device kernel and the host entry
// points: the set A(t) of one query frame under one head's policy.
//
// Policies follow LVSA §2 core mechanism (rotating global anchors united with
// a local window that is widened until |A(t)| reaches the budget C), Head
// Forcing methodology §2 (local, anchor and memory heads) and ISPA §2 item 1
// (local stream = current chunk + sink frame).  Integer arithmetic only; the
// functions compile for the host as well (FSA_HD may be defined empty).
#pragma once

#include <cstdint>

#include "../../include/fsa.h"

#ifndef FSA_HD
#define FSA_HD __host__ __device__
#endif

namespace fsa_sets {

FSA_HD inline int pos_mod(int a, int m) {
  int r = a % m;
  return r < 0 ? r + m : r;
}

// LVSA window for query frame t: returns the inclusive interval [lo, hi]
// (hi < lo when empty) of the nearest frames, grown from min(W, T) frames
// until anchors ∪ window holds min(C, T) frames.  Frames join the window in
// the order of (|f - t|, f): t, t-1, t+1, t-2, ... with the earlier frame
// first on ties; at an end of the video the other side keeps growing.
FSA_HD inline void lvsa_window(int T, int C, int W, int t_per, int r, int t,
                                            int *lo_out, int *hi_out) {
  int n_anchor = r < T ? (T - 1 - r) / t_per + 1 : 0;
  int target = C < T ? C : T;
  int base = W < T ? W : T;
  int lo = t, hi = t - 1;  // empty
  int size = 0, uni = n_anchor;
  while (size < T && (size < base || uni < target)) {
    int f;
    if (size == 0) {
      f = t;
      lo = hi = t;
    } else {
      int left = lo - 1, right = hi + 1;
      bool take_left = left >= 0 && (right >= T || (t - left) <= (right - t));
      if (take_left) {
        f = left;
        lo = left;
      } else {
        f = right;
        hi = right;
      }
    }
    ++size;
    if (pos_mod(f, t_per) != r) ++uni;
  }
  *lo_out = lo;
  *hi_out = hi;
}

// Membership test of the frame set of one query frame under one policy: the
// set A(t) is the ascending list of frames f in [0, Tk) for which keep(f)
// holds.  Built once per (policy, query frame); `sel` holds the group's
// selected frames (MEMORY heads read the first pol.topk of them).
struct FrameTest {
  int kind;
  int lo, hi;       // LVSA window, SINK_WINDOW window, MEMORY recent frames, RANGE bounds
  int r, t_per;     // LVSA rotating anchors: f mod t_per == r
  int n_sink;       // SINK_WINDOW sink frames 0 .. n_sink-1
  const int32_t *sel;
  int topk;
};

FSA_HD inline FrameTest frame_test(const fsa_head_policy &pol, int Tk, int offset, int chunk,
                                   int tq, const int32_t *sel) {
  FrameTest ft{};
  ft.kind = pol.kind;
  const int e = offset + (tq / chunk + 1) * chunk - 1;  // last KV frame of tq's chunk
  switch (pol.kind) {
    case FSA_POL_LVSA:
      ft.t_per = pol.t_per;
      ft.r = pos_mod(pol.step, pol.t_per);
      lvsa_window(Tk, pol.budget, pol.window, pol.t_per, ft.r, offset + tq, &ft.lo, &ft.hi);
      break;
    case FSA_POL_SINK_WINDOW:
      ft.n_sink = pol.n_sink;
      ft.lo = e - pol.window + 1;
      ft.hi = e;
      break;
    case FSA_POL_MEMORY:
      ft.lo = e - pol.n_recent + 1;
      ft.hi = e;
      ft.sel = sel;
      ft.topk = pol.topk;
      break;
    case FSA_POL_RANGE:
      ft.lo = pol.lo;
      ft.hi = pol.hi;
      break;
    default:
      break;
  }
  return ft;
}

FSA_HD inline bool keep_frame(const FrameTest &ft, int f) {
  switch (ft.kind) {
    case FSA_POL_FULL:
      return true;
    case FSA_POL_LVSA:
      return (f >= ft.lo && f <= ft.hi) || pos_mod(f, ft.t_per) == ft.r;
    case FSA_POL_SINK_WINDOW:
      return f < ft.n_sink || (f >= ft.lo && f <= ft.hi);
    case FSA_POL_MEMORY: {
      bool keep = f >= ft.lo && f <= ft.hi;
      for (int j = 0; j < ft.topk && !keep; ++j) keep = ft.sel[j] == f;
      return keep;
    }
    case FSA_POL_RANGE:
      return f >= ft.lo && f <= ft.hi;
    default:
      return false;
  }
}

// Frame set of query frame tq under one policy, serially: writes at most
// `cap` entries to out (ascending), pads the rest of the row with -1 and
// returns the number of frames written.
FSA_HD inline int build_one(const fsa_head_policy &pol, int Tk, int offset, int chunk, int tq,
                            const int32_t *sel, int cap, int32_t *out) {
  const FrameTest ft = frame_test(pol, Tk, offset, chunk, tq, sel);
  int n = 0;
  for (int f = 0; f < Tk && n < cap; ++f)
    if (keep_frame(ft, f)) out[n++] = f;
  for (int j = n; j < cap; ++j) out[j] = -1;
  return n;
}

}  // namespace fsa_sets

namespace fsa {
// Host checks shared by the device and host entry points (frame_sets_host.cpp).
fsa_status policy_capacity(const fsa_head_policy &p, int Tq, int Tk, int offset, int chunk,
                           int *need);
fsa_status check_policies(int32_t B, int32_t H, int32_t Tq, int32_t Tk, int32_t offset,
                          int32_t chunk, const fsa_head_policy *pol, int32_t topk_k,
                          bool have_selected, int32_t cap, bool check_cap);
}  // namespace fsa
