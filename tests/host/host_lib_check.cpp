// Host driver for the library's host code (frame-set capacity, construction
// and validation; the chunk-aware growth schedule; the error text), built by
// tests/test_host_lib_sanitized.py with g++ and the address and
// undefined-behaviour sanitizers, linked with the library's own sources
// csrc/frame_sets_host.cpp, csrc/cag.cpp and csrc/errors.cpp.
//
// Commands on stdin (whitespace separated), one result line per command:
//   C H Tq Tk offset chunk  <H x 10 policy ints>
//       -> "status cap"
//   B B H Tq Tk offset chunk topk_k cap  <H x 10 policy ints>  [selected]
//       (selected: B*H*(Tq/chunk)*topk_k ints when topk_k > 0)
//       -> "status cnt... idx..." (cnt and idx only when status is 0)
//   V B H Tq Tk cap  <B*H*Tq*cap idx>  <B*H*Tq cnt>
//       -> "status"
//   S n s_target s_base s_max  <n cost>  <n candidates>   (doubles as hex bits)
//       -> "status beta sparsity... budgets..." (doubles as hex bits)
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "fsa.h"

static bool read_policies(int H, std::vector<fsa_head_policy> *pol) {
  pol->assign((size_t)(H > 0 ? H : 0), fsa_head_policy{});
  for (int h = 0; h < H; ++h) {
    int32_t *f = &(*pol)[(size_t)h].kind;  // ten consecutive int32 fields
    for (int i = 0; i < 10; ++i)
      if (std::scanf("%d", &f[i]) != 1) return false;
  }
  return true;
}

static double read_hex_double() {
  unsigned long long b = 0;
  std::scanf("%llx", &b);
  double d;
  std::memcpy(&d, &b, sizeof d);
  return d;
}

static unsigned long long bits(double d) {
  unsigned long long b;
  std::memcpy(&b, &d, sizeof b);
  return b;
}

int main() {
  char cmd[4];
  while (std::scanf("%3s", cmd) == 1) {
    if (cmd[0] == 'C') {
      int H, Tq, Tk, off, chunk;
      std::scanf("%d %d %d %d %d", &H, &Tq, &Tk, &off, &chunk);
      std::vector<fsa_head_policy> pol;
      read_policies(H, &pol);
      int32_t cap = -1;
      const int st = fsa_frame_set_capacity(H, pol.data(), Tq, Tk, off, chunk, &cap);
      std::printf("%d %d\n", st, cap);
    } else if (cmd[0] == 'B') {
      int B, H, Tq, Tk, off, chunk, topk, cap;
      std::scanf("%d %d %d %d %d %d %d %d", &B, &H, &Tq, &Tk, &off, &chunk, &topk, &cap);
      std::vector<fsa_head_policy> pol;
      read_policies(H, &pol);
      std::vector<int32_t> sel;
      if (topk > 0 && chunk > 0) {
        sel.resize((size_t)B * H * (Tq / chunk) * topk);
        for (auto &v : sel) std::scanf("%d", &v);
      }
      const size_t n = (size_t)B * H * Tq;
      std::vector<int32_t> idx(n * (size_t)(cap > 0 ? cap : 1)), cnt(n);
      const int st = fsa_build_frame_sets_host(B, H, Tq, Tk, off, chunk, pol.data(),
                                               sel.empty() ? nullptr : sel.data(), topk, cap,
                                               idx.data(), cnt.data());
      std::printf("%d", st);
      if (st == 0) {
        for (size_t i = 0; i < n; ++i) std::printf(" %d", cnt[i]);
        for (size_t i = 0; i < n * (size_t)cap; ++i) std::printf(" %d", idx[i]);
      }
      std::printf("\n");
    } else if (cmd[0] == 'V') {
      int B, H, Tq, Tk, cap;
      std::scanf("%d %d %d %d %d", &B, &H, &Tq, &Tk, &cap);
      const size_t n = (size_t)B * H * Tq;
      std::vector<int32_t> idx(n * (size_t)cap), cnt(n);
      for (auto &v : idx) std::scanf("%d", &v);
      for (auto &v : cnt) std::scanf("%d", &v);
      std::printf("%d\n", fsa_validate_frame_sets(B, H, Tq, Tk, cap, idx.data(), cnt.data()));
    } else if (cmd[0] == 'S') {
      int n;
      std::scanf("%d", &n);
      const double st_ = read_hex_double(), sb = read_hex_double(), sm = read_hex_double();
      std::vector<double> cost((size_t)n), sp((size_t)n);
      std::vector<int32_t> cand((size_t)n), bud((size_t)n);
      for (auto &c : cost) c = read_hex_double();
      for (auto &c : cand) std::scanf("%d", &c);
      double beta = 0.0;
      const int st = fsa_cag_schedule(n, cost.data(), st_, sb, sm, cand.data(), sp.data(),
                                      bud.data(), &beta);
      std::printf("%d", st);
      if (st == 0) {
        std::printf(" %llx", bits(beta));
        for (double v : sp) std::printf(" %llx", bits(v));
        for (int32_t v : bud) std::printf(" %d", v);
      } else {
        std::printf(" %s", fsa_last_error()[0] ? "error-text" : "no-text");
      }
      std::printf("\n");
    }
  }
  return 0;
}
