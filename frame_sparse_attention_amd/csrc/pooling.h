// Float64 pooling of token segments (a query group or block, a key frame or
// block) shared by the frame-level top-k and the two-level block selection
// (Light Forcing §2.2: query and key tokens are compressed by mean pooling).
//
// A pooled sum is the exact sum of the segment's tokens in each channel,
// rounded once to float64 (nearest, ties to even): it has no order of
// summation, so the work can be cut any way.  Two launches:
//
//   pool_pieces_kernel  HBM-bound.  Each segment is cut into balanced pieces
//       of at most 128 rows; one 256-thread block per piece streams its rows
//       with 16-byte loads (8 per thread in flight), adds them in float64 and
//       records the smallest and largest magnitude it saw.  Output per piece:
//       D float64 partial sums and two magnitude keys.
//   finalize_kernel  one block per segment.  When the segment's magnitudes
//       span few enough binades (fsa_exact::exact_by_range), every float64
//       partial sum above was exact, in any order, so the pieces' sums add up
//       to the exact sum.  Otherwise the segment's rows are read again and
//       summed exactly (fsa_exact::ExactSum), then rounded once.  On bfloat16
//       data the first case holds unless one segment mixes magnitudes about
//       2^34 apart; float32 data takes the second case more often.
//
// A family of segments is a regular layout: for each selected head, `nseg`
// segments of `seg_rows` rows starting at row `row0` of that head, each cut
// into `pieces` pieces of `piece_rows` rows (the last one shorter).  Piece
// results are stored segment-major, so the pieces of `group` consecutive
// segments (e.g. the blocks of one frame) are consecutive as well.
#pragma once
#pragma clang fp contract(off)

#include "exact_sum.h"
#include "fsa_internal.h"

namespace {

// bfloat16 storage: the raw 16 bits
struct Bf16 {
  uint16_t bits;
};

constexpr int kPoolThreads = 256;
constexpr int kPoolUnroll = 8;     // row steps issued together: loads in flight per thread
constexpr int kPieceRows = 128;    // rows per piece at most (independent of dtype and alignment)
constexpr int kMaxPoolD = 256;

struct SegFamily {
  const void *src;        // [B][H][head_rows][D] tensor
  long long head_rows;    // rows of one head in src (Nq or Nk)
  long long row0;         // first row of segment 0 inside a head
  int seg_rows;           // rows per segment
  int nseg;               // segments per selected head
  int H;                  // heads per batch entry in src
  int h_begin;            // first selected head
  int nheads;             // selected heads (b-major: B * nheads segments lists)
  int pieces;             // pieces per segment
  int piece_rows;         // rows per piece (the last piece of a segment may be shorter)
  double *part;           // [segments * pieces][D] float64 partial sums
  uint32_t *keys;         // [segments * pieces][2] magnitude keys (min - 1, max)
  double *direct;         // one-piece segments: [segments][D] exact sums written by the
                          // pooling block itself (nullptr: left to finalize_kernel)
  long long count() const { return (long long)nheads * nseg; }  // per batch entry
};

// First row (in src) of segment `seg` of family f (batch entry b, head slot
// hs, segment s).  Segment and piece counts stay below 2^31 (the launches
// check), so the index arithmetic is 32-bit; only the row offset is 64-bit.
__device__ inline long long seg_first_row(const SegFamily &f, int seg) {
  const int per_b = f.nheads * f.nseg;
  const int b = seg / per_b;
  const int r = seg - b * per_b;
  const int hs = r / f.nseg;
  const int s = r - hs * f.nseg;
  const long long head = (long long)b * f.H + f.h_begin + hs;
  return head * f.head_rows + f.row0 + (long long)s * f.seg_rows;
}

// 16-byte unit loads of VEC elements (VEC = 16 / sizeof(T)), or single
// elements (VEC = 1) when rows are not 16-byte multiples or not aligned.
template <typename T, int VEC>
struct Unit {
  uint32_t w[VEC * sizeof(T) / 4 > 0 ? VEC * sizeof(T) / 4 : 1];
};

template <typename T, int VEC>
__device__ inline Unit<T, VEC> load_unit(const T *p) {
  Unit<T, VEC> u;
  if constexpr (VEC * sizeof(T) == 16) {
    const uint4 v = *reinterpret_cast<const uint4 *>(p);
    u.w[0] = v.x, u.w[1] = v.y, u.w[2] = v.z, u.w[3] = v.w;
  } else if constexpr (sizeof(T) == 4) {
    u.w[0] = __float_as_uint(*reinterpret_cast<const float *>(p));
  } else {
    u.w[0] = (uint32_t)reinterpret_cast<const Bf16 *>(p)->bits;  // VEC = 1, bf16
  }
  return u;
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Adds one unit into acc[0..VEC) and its magnitudes into the keys.  bf16 pairs
// update 16-bit keys two at a time; float32 updates 32-bit keys.
template <typename T, int VEC>
__device__ inline void add_unit(const Unit<T, VEC> &u, double *acc, u16x2 &k16min,
                                u16x2 &k16max, uint32_t &k32min, uint32_t &k32max) {
  if constexpr (sizeof(T) == 2 && VEC > 1) {
#pragma unroll
    for (int e = 0; e < VEC / 2; ++e) {
      const uint32_t w = u.w[e];
      acc[2 * e] = acc[2 * e] + (double)__uint_as_float(w << 16);
      acc[2 * e + 1] = acc[2 * e + 1] + (double)__uint_as_float(w & 0xFFFF0000u);
      const u16x2 a = __builtin_bit_cast(u16x2, w & 0x7FFF7FFFu);
      const u16x2 one = {1, 1};
      k16min = __builtin_elementwise_min(k16min, a - one);  // zeros wrap to 0xFFFF
      k16max = __builtin_elementwise_max(k16max, a);
    }
  } else {
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const uint32_t bits = sizeof(T) == 2 ? u.w[0] << 16 : u.w[e];
      acc[e] = acc[e] + (double)__uint_as_float(bits);
      const uint32_t a = bits & 0x7FFFFFFFu;
      k32min = min(k32min, a - 1u);  // zero wraps to 0xFFFFFFFF
      k32max = max(k32max, a);
    }
  }
}

template <typename T>
__device__ inline uint32_t elem_bits(const T *p);
template <>
__device__ inline uint32_t elem_bits<float>(const float *p) {
  return __float_as_uint(*p);
}
template <>
__device__ inline uint32_t elem_bits<Bf16>(const Bf16 *p) {
  return (uint32_t)p->bits << 16;
}

// One block per piece of family a (pieces [0, na)) or b (the rest).
template <typename T, int VEC>
__global__ void __launch_bounds__(kPoolThreads) pool_pieces_kernel(SegFamily fa, SegFamily fb,
                                                                   long long na, int D) {
  // per-row-group partials; when the units of a row divide a wavefront, the
  // row groups of one wavefront are first added with shuffles and only one
  // partial per wavefront reaches LDS
  __shared__ double s_red[kPoolThreads * VEC];
  __shared__ uint32_t s_kmin, s_kmax;
  int pid = (int)blockIdx.x;
  const bool in_a = pid < na;
  const SegFamily f = in_a ? fa : fb;
  if (!in_a) pid -= (int)na;
  const int seg = pid / f.pieces;
  const int piece = pid - seg * f.pieces;
  const int first = piece * f.piece_rows;
  const int nrows = min(f.piece_rows, f.seg_rows - first);
  const T *src =
      static_cast<const T *>(f.src) + (seg_first_row(f, seg) + first) * (long long)D;

  const int U = D / VEC;                      // units per row
  const int RS = kPoolThreads / U;            // rows per step
  const int t = threadIdx.x;
  const int u = t % U, rg = t / U;
  if (t == 0) {
    s_kmin = fsa_exact::kKeyMinInit;
    s_kmax = fsa_exact::kKeyMaxInit;
  }
  double acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.0;
  u16x2 k16min = {0xFFFF, 0xFFFF}, k16max = {0, 0};
  uint32_t k32min = fsa_exact::kKeyMinInit, k32max = fsa_exact::kKeyMaxInit;
  if (rg < RS) {
    for (int r0 = rg; r0 < nrows; r0 += kPoolUnroll * RS) {
      Unit<T, VEC> x[kPoolUnroll];
#pragma unroll
      for (int i = 0; i < kPoolUnroll; ++i) {
        const int r = r0 + i * RS;
        if (r < nrows) {
          x[i] = load_unit<T, VEC>(src + (long long)r * D + u * VEC);
        } else {
#pragma unroll
          for (int j = 0; j < (int)(sizeof(x[i].w) / 4); ++j) x[i].w[j] = 0u;  // adds +0
        }
      }
#pragma unroll
      for (int i = 0; i < kPoolUnroll; ++i)
        add_unit<T, VEC>(x[i], acc, k16min, k16max, k32min, k32max);
    }
  }
  if constexpr (sizeof(T) == 2 && VEC > 1) {
    const unsigned short m = min(k16min.x, k16min.y);
    k32min = m == 0xFFFF ? fsa_exact::kKeyMinInit : ((((uint32_t)m + 1u) << 16) - 1u);
    k32max = (uint32_t)max(k16max.x, k16max.y) << 16;
  }
  // block reduction: the partials of a channel are added in float64; every
  // such sum is exact whenever the segment passes exact_by_range
  for (int off = 32; off >= 1; off >>= 1) {
    k32min = min(k32min, (uint32_t)__shfl_xor((int)k32min, off));
    k32max = max(k32max, (uint32_t)__shfl_xor((int)k32max, off));
  }
  __syncthreads();
  if (t % 64 == 0) {
    atomicMin(&s_kmin, k32min);
    atomicMax(&s_kmax, k32max);
  }
  const bool by_wave = U <= 64 && 64 % U == 0;   // U a power of two up to 64
  int groups = RS;                                 // partials per channel in LDS
  if (by_wave) {
    // lanes l, l ^ U, l ^ 2U, ... of a wavefront hold the same unit
    for (int off = U; off < 64; off <<= 1) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[e] = acc[e] + __shfl_xor(acc[e], off);
    }
    groups = kPoolThreads / 64;
    if ((t % 64) < U) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) s_red[(t / 64) * D + u * VEC + e] = acc[e];
    }
  } else if (rg < RS) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) s_red[rg * D + u * VEC + e] = acc[e];
  }
  __syncthreads();
  double *out = f.part + (long long)pid * D;
  // a segment of one piece is finished here: its exact sum, directly
  const bool direct = f.direct != nullptr && f.pieces == 1;
  const int mbits = sizeof(T) == 2 ? fsa_exact::kBf16Bits : fsa_exact::kF32Bits;
  const bool cheap = fsa_exact::exact_by_range(s_kmin, s_kmax, f.seg_rows, mbits);
  for (int d = t; d < D; d += kPoolThreads) {
    double s = 0.0;
    for (int g = 0; g < groups; ++g) s = s + s_red[g * D + d];
    out[d] = s;
    if (direct) {
      if (!cheap) {
        fsa_exact::ExactSum acc;
        acc.clear();
        for (int r = 0; r < nrows; ++r) acc.add(elem_bits<T>(src + (long long)r * D + d));
        s = acc.rounded();
      }
      f.direct[(long long)seg * D + d] = s + 0.0;
    }
  }
  if (t == 0) {
    f.keys[2LL * pid] = s_kmin;
    f.keys[2LL * pid + 1] = s_kmax;
  }
}

// Final sums of a family of segments.  `group` consecutive segments of the
// pooled family form one output segment (a frame made of its blocks); the
// output segment has group * seg_rows rows.
struct FinalFamily {
  SegFamily pooled;   // the family whose pieces hold the partial sums
  int group;          // pooled segments per output segment
  double *out;        // [output segments][D]
  long long count() const { return pooled.count() / group; }  // per batch entry
};

constexpr int kFinalThreads = 256;
constexpr int kFinalBatch = 16;  // partials each thread requests together

template <typename T>
__global__ void __launch_bounds__(kFinalThreads) finalize_kernel(FinalFamily fa, FinalFamily fb,
                                                                 FinalFamily fc, long long na,
                                                                 long long nb, int D) {
  __shared__ double s_part[kFinalThreads];
  __shared__ uint32_t s_kmin, s_kmax;
  long long sid = blockIdx.x;
  const int which = sid < na ? 0 : (sid < na + nb ? 1 : 2);
  sid -= which == 0 ? 0 : (which == 1 ? na : na + nb);
  const FinalFamily ff = which == 0 ? fa : (which == 1 ? fb : fc);
  const SegFamily &f = ff.pooled;
  const int np = ff.group * f.pieces;             // pieces of this output segment
  const long long p0 = sid * np;
  const long long nrows = (long long)ff.group * f.seg_rows;
  const int t = threadIdx.x;
  if (t == 0) {
    s_kmin = fsa_exact::kKeyMinInit;
    s_kmax = fsa_exact::kKeyMaxInit;
  }
  __syncthreads();
  uint32_t kmin = fsa_exact::kKeyMinInit, kmax = fsa_exact::kKeyMaxInit;
  for (int p = t; p < np; p += kFinalThreads) {
    kmin = min(kmin, f.keys[2 * (p0 + p)]);
    kmax = max(kmax, f.keys[2 * (p0 + p) + 1]);
  }
  for (int off = 32; off >= 1; off >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, off));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, off));
  }
  if (t % 64 == 0) {
    atomicMin(&s_kmin, kmin);
    atomicMax(&s_kmax, kmax);
  }
  __syncthreads();
  const int mbits = sizeof(T) == 2 ? fsa_exact::kBf16Bits : fsa_exact::kF32Bits;
  double *out = ff.out + sid * (long long)D;
  if (fsa_exact::exact_by_range(s_kmin, s_kmax, nrows, mbits)) {
    // Every addition is exact here, in any order: the pieces of a channel
    // are shared out over `parts` threads, each requesting its partials
    // together, and the threads' sums are added at the end.
    const int parts = D <= kFinalThreads ? kFinalThreads / D : 1;
    for (int d0 = 0; d0 < D; d0 += kFinalThreads) {
      const int d = d0 + t % D, part = t / D;
      double s = 0.0;
      if (part < parts && d < D) {
        const double *pp = f.part + p0 * D + d;
        for (int pb = part; pb < np; pb += parts * kFinalBatch) {
          double x[kFinalBatch];
#pragma unroll
          for (int i = 0; i < kFinalBatch; ++i) {
            const int p = pb + i * parts;
            x[i] = p < np ? pp[(long long)p * D] : 0.0;
          }
#pragma unroll
          for (int i = 0; i < kFinalBatch; ++i) s = s + x[i];
        }
      }
      if (parts > 1) {
        s_part[t] = s;
        __syncthreads();
        if (t < D) {
          s = 0.0;
          for (int q = 0; q < parts; ++q) s = s + s_part[q * D + t];
        }
        __syncthreads();
      }
      if (t < D && d0 + t < D) out[d0 + t] = s + 0.0;
      if (parts > 1) break;  // D <= kFinalThreads: one pass covered every channel
    }
    return;
  }
  // the first pooled segment of this output segment: its rows and the next
  // group - 1 segments' rows are consecutive in memory
  const T *src =
      static_cast<const T *>(f.src) + seg_first_row(f, (int)(sid * ff.group)) * (long long)D;
  for (int d = t; d < D; d += kFinalThreads) {
    fsa_exact::ExactSum acc;
    acc.clear();
    for (long long r = 0; r < nrows; ++r) acc.add(elem_bits<T>(src + r * D + d));
    out[d] = acc.rounded();
  }
}

// Pieces per segment and rows per piece (balanced) for `rows`-row segments.
inline void piece_plan(int rows, int *pieces, int *piece_rows) {
  *pieces = (rows + kPieceRows - 1) / kPieceRows;
  *piece_rows = (rows + *pieces - 1) / *pieces;
}

// Unit width for rows of D elements of the given dtype: 16 bytes when rows
// are 16-byte multiples and both tensors are 16-byte aligned, else 1 element.
inline int pool_vec(int32_t dt, int D, const void *a, const void *b) {
  const int esz = dt == FSA_BF16 ? 2 : 4;
  const bool aligned =
      ((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b)) & 15u) == 0;
  return (aligned && (D * esz) % 16 == 0) ? 16 / esz : 1;
}

// Fills in the piece layout of a family for `rows`-row segments.
inline SegFamily make_family(const void *src, long long head_rows, long long row0, int seg_rows,
                             int nseg, int H, int h_begin, int nheads) {
  SegFamily f{};
  f.src = src;
  f.head_rows = head_rows;
  f.row0 = row0;
  f.seg_rows = seg_rows;
  f.nseg = nseg;
  f.H = H;
  f.h_begin = h_begin;
  f.nheads = nheads;
  piece_plan(seg_rows, &f.pieces, &f.piece_rows);
  return f;
}

// A family with no segments (an unused launch slot).
inline SegFamily no_family() {
  SegFamily f{};
  f.nseg = 1;
  f.pieces = 1;
  f.piece_rows = 1;
  f.seg_rows = 1;
  return f;
}
inline FinalFamily no_final() { return FinalFamily{no_family(), 1, nullptr}; }

inline size_t align256(size_t n) { return (n + 255) / 256 * 256; }

// Workspace of the partial sums and keys of a family over B batch entries.
inline size_t family_pieces(const SegFamily &f, int B) {
  return (size_t)B * f.nheads * f.nseg * f.pieces;
}
inline size_t family_part_bytes(const SegFamily &f, int B, int D) {
  const size_t n = family_pieces(f, B);
  return align256(n * (size_t)D * sizeof(double)) + align256(n * 2 * sizeof(uint32_t));
}
// Carves the family's partials and keys out of `ws` (advanced past them).
inline void place_family(SegFamily &f, int B, int D, unsigned char **ws) {
  const size_t n = family_pieces(f, B);
  f.part = reinterpret_cast<double *>(*ws);
  *ws += align256(n * (size_t)D * sizeof(double));
  f.keys = reinterpret_cast<uint32_t *>(*ws);
  *ws += align256(n * 2 * sizeof(uint32_t));
}

// Pools families a and b (pieces), then finalizes up to three output families.
template <typename T, int VEC>
void launch_pool_t(const SegFamily &a, const SegFamily &b, int B, int D, hipStream_t s) {
  const long long na = (long long)family_pieces(a, B), nbp = (long long)family_pieces(b, B);
  if (na + nbp > 0)
    hipLaunchKernelGGL((pool_pieces_kernel<T, VEC>), dim3((unsigned)(na + nbp)),
                       dim3(kPoolThreads), 0, s, a, b, na, D);
}

inline void launch_pool(int32_t dt, int vec, const SegFamily &a, const SegFamily &b, int B, int D,
                        hipStream_t s) {
  if (dt == FSA_BF16) {
    if (vec == 8)
      launch_pool_t<Bf16, 8>(a, b, B, D, s);
    else
      launch_pool_t<Bf16, 1>(a, b, B, D, s);
  } else {
    if (vec == 4)
      launch_pool_t<float, 4>(a, b, B, D, s);
    else
      launch_pool_t<float, 1>(a, b, B, D, s);
  }
}

inline void launch_finalize(int32_t dt, const FinalFamily &a, const FinalFamily &b,
                            const FinalFamily &c, int B, int D, hipStream_t s) {
  const long long na = B * a.count(), nb = B * b.count(), nc = B * c.count();
  if (na + nb + nc == 0) return;
  const dim3 grid((unsigned)(na + nb + nc)), block(kFinalThreads);
  if (dt == FSA_BF16)
    hipLaunchKernelGGL(finalize_kernel<Bf16>, grid, block, 0, s, a, b, c, na, nb, D);
  else
    hipLaunchKernelGGL(finalize_kernel<float>, grid, block, 0, s, a, b, c, na, nb, D);
}

// sum_d qs[d] * row[d] in ascending d, each product rounded to float64 before
// it is added (contraction is off in every file that includes this header).
// The row (global memory) is read 64 values at a time into registers ahead of
// the ordered adds, so the loads overlap instead of each add waiting for its
// own load.
__device__ inline double ordered_dot(const double *qs, const double *__restrict__ row, int D) {
  double acc = 0.0;
  int d0 = 0;
  if ((reinterpret_cast<uintptr_t>(row) & 15u) == 0) {
    for (; d0 + 64 <= D; d0 += 64) {
      double2 x[32];
#pragma unroll
      for (int t = 0; t < 32; ++t) x[t] = reinterpret_cast<const double2 *>(row + d0)[t];
#pragma unroll
      for (int t = 0; t < 32; ++t) {
        const double p0 = qs[d0 + 2 * t] * x[t].x;
        acc = acc + p0;
        const double p1 = qs[d0 + 2 * t + 1] * x[t].y;
        acc = acc + p1;
      }
    }
  }
  for (; d0 < D; ++d0) {
    const double p = qs[d0] * row[d0];
    acc = acc + p;
  }
  return acc;
}

// (score, index) order: higher score first, then lower index.  A NaN score
// (from non-finite inputs) ranks as -inf, so the order stays a strict total
// order and exactly k candidates are kept.
__device__ inline double nan_last(double s) { return s != s ? -INFINITY : s; }
__device__ inline bool score_before(double s1, int i1, double s2, int i2) {
  return s1 > s2 || (s1 == s2 && i1 < i2);
}

// Marks in s_taken the k best of s_score[0..n) in (score desc, index asc)
// order; every thread of the block calls it (it holds block barriers), scores
// NaN-free, k <= n.  Up to 1024 candidates each thread counts, for its
// candidates, how many others come first, and keeps those with fewer than k;
// beyond that, k rounds of an argmax by the first wavefront.  Both give the
// same set.
__device__ inline void take_best(const double *s_score, unsigned char *s_taken, int n, int k) {
  const int t = threadIdx.x, nt = blockDim.x;
  if (n <= 1024) {
    for (int i = t; i < n; i += nt) {
      const double si = s_score[i];
      int ahead = 0;
      for (int j = 0; j < n; ++j) ahead += score_before(s_score[j], j, si, i) ? 1 : 0;
      s_taken[i] = ahead < k ? 1 : 0;
    }
    __syncthreads();
    return;
  }
  for (int i = t; i < n; i += nt) s_taken[i] = 0;
  __syncthreads();
  for (int round = 0; round < k; ++round) {
    if (t < 64) {
      double bs = 0.0;
      int bi = -1;
      for (int i = t; i < n; i += 64) {
        if (s_taken[i]) continue;
        const double s = s_score[i];
        if (bi < 0 || score_before(s, i, bs, bi)) {
          bs = s;
          bi = i;
        }
      }
      for (int off = 32; off >= 1; off >>= 1) {
        const double os = __shfl_xor(bs, off);
        const int oi = __shfl_xor(bi, off);
        if (oi >= 0 && (bi < 0 || score_before(os, oi, bs, bi))) {
          bs = os;
          bi = oi;
        }
      }
      if (t == 0) s_taken[bi] = 1;
    }
    __syncthreads();
  }
}

// Calls emit(pos, i) for the indices i < n with s_taken[i] set, pos counting
// them in ascending i, for pos < limit; the first wavefront does it (threads
// beyond it return at once).
template <typename Emit>
__device__ inline void compact_taken(const unsigned char *s_taken, int n, int limit, Emit emit) {
  const int lane = threadIdx.x;
  if (lane >= 64) return;
  int count = 0;
  for (int base = 0; base < n; base += 64) {
    const int i = base + lane;
    const bool flag = i < n && s_taken[i];
    const unsigned long long mask = __ballot(flag);
    const int pos = count + __popcll(mask & ((1ull << lane) - 1ull));
    if (flag && pos < limit) emit(pos, i);
    count += __popcll(mask);
  }
}

}  // namespace
