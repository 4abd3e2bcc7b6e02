// Float64 pooling of token segments (a query frame or block, a key frame or
// block) shared by the frame-level top-k and the two-level block selection.
// Every channel sum is one sequential chain in ascending token order, and
// floating-point contraction is off, so the sums are reproducible bit for bit.
#pragma once
#pragma clang fp contract(off)

#include "fsa_internal.h"

namespace {

// bfloat16 storage: the raw 16 bits
struct Bf16 {
  uint16_t bits;
};

// Pooling of one segment of rows (a query group, or one key frame) of one
// head, for 128 channels per block: chunks of kRowsPerChunk rows are staged
// through LDS with 16-byte loads (two chunks in flight), then thread d adds
// its column one row at a time in ascending row order.  The float64 adds of a
// channel form one sequential chain, exactly as the definition orders them;
// the memory traffic around that chain is bulk and overlapped.
constexpr int kPoolThreads = 128;
constexpr int kRowsPerChunk = 32;
constexpr int kMaxPoolD = 256;  // LDS: 2 chunks x 32 rows x 256 x 4 B = 64 KB at most

template <typename T>
__device__ inline double elem_as_double(const T *row_tile, int r, int d, int D);
template <>
__device__ inline double elem_as_double<float>(const float *t, int r, int d, int D) {
  return (double)t[r * D + d];
}
template <>
__device__ inline double elem_as_double<Bf16>(const Bf16 *t, int r, int d, int D) {
  return (double)__uint_as_float((uint32_t)t[r * D + d].bits << 16);
}

// Adds rows [0, rows) of the LDS chunk `t` into this thread's channel sums.
template <typename T>
__device__ inline void add_chunk(const T *t, int rows, int D, double *acc) {
  const int tid = threadIdx.x;
  for (int i = 0; i * kPoolThreads + tid < D; ++i) {
    const int d = i * kPoolThreads + tid;
    double a = acc[i];
    if (rows == kRowsPerChunk) {
      // read the whole column chunk first (independent LDS loads), then add in order
      double x[kRowsPerChunk];
#pragma unroll
      for (int r = 0; r < kRowsPerChunk; ++r) x[r] = elem_as_double<T>(t, r, d, D);
#pragma unroll
      for (int r = 0; r < kRowsPerChunk; ++r) a = a + x[r];
    } else {
      for (int r = 0; r < rows; ++r) a = a + elem_as_double<T>(t, r, d, D);
    }
    acc[i] = a;
  }
}

// s_waitcnt immediates: vmcnt(n) with expcnt and lgkmcnt at their maxima
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Sums rows [row0, row0 + nrows) of `src` (row stride D) into out[0..D).
// Chunks of kRowsPerChunk rows stream from HBM into an LDS ring of kRing
// slots with global_load_lds (no registers in flight), kRing - 1 chunks ahead
// of the chunk being added; rows past the segment repeat its last row (in
// bounds, never added).  Needs a chunk of whole 1 KB wavefront transfers.
constexpr int kRing = 8;
template <typename T>
__device__ void pool_segment_dma(const T *__restrict__ src, long long row0, int nrows, int D,
                                 unsigned char *lds, double *__restrict__ out) {
  const int tid = threadIdx.x, lane = tid % 64;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int row_bytes = D * (int)sizeof(T);
  const int chunk_bytes = kRowsPerChunk * row_bytes;
  const int per_wave = chunk_bytes / 1024 / (kPoolThreads / 64);  // DMA instructions per wave
  const int nchunks = (nrows + kRowsPerChunk - 1) / kRowsPerChunk;
  const char *base = reinterpret_cast<const char *>(src) + row0 * row_bytes;
  auto issue = [&](int c) {
    unsigned char *slot = lds + (c % kRing) * chunk_bytes;
    for (int i = 0; i < per_wave; ++i) {
      const int unit = (i * (kPoolThreads / 64) + wave) * 64 + lane;  // 16-byte unit in chunk
      int r = c * kRowsPerChunk + unit * 16 / row_bytes;
      r = r < nrows ? r : nrows - 1;
      const char *g = base + (long long)r * row_bytes + (unit * 16) % row_bytes;
      __builtin_amdgcn_global_load_lds(
          (const void *)g,
          (__attribute__((address_space(3))) void *)(slot + (i * (kPoolThreads / 64) + wave) * 1024),
          16, 0, 0);
    }
  };
  double acc[kMaxPoolD / kPoolThreads];
  for (int i = 0; i < kMaxPoolD / kPoolThreads; ++i) acc[i] = 0.0;
  for (int c = 0; c < kRing - 1 && c < nchunks; ++c) issue(c);
  for (int c = 0; c < nchunks; ++c) {
    if (c + kRing - 1 < nchunks) {
      issue(c + kRing - 1);
      // chunk c landed once at most kRing - 1 later chunks are outstanding
      if (per_wave == 1) wait_vmcnt<kRing - 1>();
      else if (per_wave == 2) wait_vmcnt<2 * (kRing - 1)>();
      else if (per_wave == 4) wait_vmcnt<4 * (kRing - 1)>();
      else wait_vmcnt<0>();
    } else {
      wait_vmcnt<0>();
    }
    __syncthreads();
    const int rows = min(kRowsPerChunk, nrows - c * kRowsPerChunk);
    add_chunk<T>(reinterpret_cast<const T *>(lds + (c % kRing) * chunk_bytes), rows, D, acc);
    __syncthreads();  // slot c % kRing is refilled by the next issue
  }
  for (int i = 0; i * kPoolThreads + tid < D; ++i) out[i * kPoolThreads + tid] = acc[i];
}

// Fallback for shapes the DMA path cannot take: chunks go through registers.
template <typename T>
__device__ void pool_segment(const T *__restrict__ src, long long row0, int nrows, int D,
                             T *tile /* LDS [kRowsPerChunk * D] */, double *__restrict__ out) {
  const int tid = threadIdx.x;
  const int nchunks = (nrows + kRowsPerChunk - 1) / kRowsPerChunk;
  double acc[kMaxPoolD / kPoolThreads];
  for (int i = 0; i < kMaxPoolD / kPoolThreads; ++i) acc[i] = 0.0;
  for (int c = 0; c < nchunks; ++c) {
    const int rows = min(kRowsPerChunk, nrows - c * kRowsPerChunk);
    const T *g = src + (row0 + (long long)c * kRowsPerChunk) * D;
    for (int u = tid; u < rows * D; u += kPoolThreads) tile[u] = g[u];
    __syncthreads();
    add_chunk<T>(tile, rows, D, acc);
    __syncthreads();
  }
  for (int i = 0; i * kPoolThreads + tid < D; ++i) out[i * kPoolThreads + tid] = acc[i];
}

// One launch pools every query frame and every candidate key frame of the
// selected heads (one block each).
template <typename T>
__global__ void __launch_bounds__(kPoolThreads) pool_kernel(
    const T *__restrict__ q, const T *__restrict__ k, int H, int Nq, int Nk, int D, int P,
    int h_begin, int Hs, int Tq, int cand_begin, int F, bool use_dma,
    double *__restrict__ qframe, double *__restrict__ ksum) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  T *tile = reinterpret_cast<T *>(smem);
  const long long bid = blockIdx.x;
  const int chunk_bytes = kRowsPerChunk * D * (int)sizeof(T);
  const int per_wave = chunk_bytes / 1024 / (kPoolThreads / 64);
  const bool dma = use_dma && chunk_bytes % 2048 == 0 &&
                   (per_wave == 1 || per_wave == 2 || per_wave == 4);
  // block layout: b-major, then [Tq query frames | F key frames] per selected head
  const int per_b = Hs * (Tq + F);
  const int b = (int)(bid / per_b);
  const int rem = (int)(bid % per_b);
  if (rem < Hs * Tq) {
    const int hs = rem / Tq, t = rem % Tq;
    const long long head = (long long)b * H + h_begin + hs;
    double *dst = qframe + ((long long)(b * Hs + hs) * Tq + t) * D;
    if (dma)
      pool_segment_dma<T>(q, head * Nq + (long long)t * P, P, D, smem, dst);
    else
      pool_segment<T>(q, head * Nq + (long long)t * P, P, D, tile, dst);
  } else {
    const int r2 = rem - Hs * Tq;
    const int hs = r2 / F, fi = r2 % F;
    const long long head = (long long)b * H + h_begin + hs;
    double *dst = ksum + ((long long)(b * Hs + hs) * F + fi) * D;
    if (dma)
      pool_segment_dma<T>(k, head * Nk + (long long)(cand_begin + fi) * P, P, D, smem, dst);
    else
      pool_segment<T>(k, head * Nk + (long long)(cand_begin + fi) * P, P, D, tile, dst);
  }
}

// One wavefront per segment, for rows of a power-of-two size between 16 and
// 1024 bytes and D <= 128 even: lane t adds channels 2t and 2t+1 (two
// independent float64 chains, each in ascending row order).  Rows stream
// through an LDS ring of kWaveRing (2 or 4) chunks of 16 KB with global_load_lds,
// kWaveRing - 1 chunks ahead; a single wavefront needs no barrier, since its
// own vmcnt wait makes a chunk visible and the reads of a slot finish before
// the adds that use them, i.e. before the slot is refilled.
constexpr int kWaveChunk = 16384;  // bytes per ring slot: 16 DMA instructions of 1 KB

template <typename T>
__device__ inline void pair_as_double(const unsigned char *p, double &x0, double &x1);
template <>
__device__ inline void pair_as_double<float>(const unsigned char *p, double &x0, double &x1) {
  const float2 v = *reinterpret_cast<const float2 *>(p);
  x0 = (double)v.x;
  x1 = (double)v.y;
}
template <>
__device__ inline void pair_as_double<Bf16>(const unsigned char *p, double &x0, double &x1) {
  const uint32_t w = *reinterpret_cast<const uint32_t *>(p);
  x0 = (double)__uint_as_float(w << 16);
  x1 = (double)__uint_as_float(w & 0xFFFF0000u);
}

template <typename T, int kWaveRing, int CSPLIT>
__device__ void pool_segment_wave(const T *__restrict__ src, long long row0, int nrows, int D,
                                  int cgroup, double *__restrict__ out) {
  __shared__ __attribute__((aligned(16))) unsigned char ring[kWaveRing][kWaveChunk];
  const int lane = threadIdx.x;
  // this wavefront's channels: [cgroup * D / CSPLIT, (cgroup + 1) * D / CSPLIT)
  const int Dw = D / CSPLIT;
  const int row_stride = D * (int)sizeof(T);       // bytes between rows in memory
  const int row_bytes = Dw * (int)sizeof(T);       // bytes of a row this wavefront stages
  const int col0 = cgroup * row_bytes;
  const int rows_per_chunk = kWaveChunk / row_bytes;
  const int nchunks = (nrows + rows_per_chunk - 1) / rows_per_chunk;
  const char *base = reinterpret_cast<const char *>(src) + row0 * row_stride;
  auto issue = [&](int c) {
#pragma unroll
    for (int i = 0; i < kWaveChunk / 1024; ++i) {
      const int unit = i * 64 + lane;  // 16-byte unit of the chunk
      int r = c * rows_per_chunk + unit * 16 / row_bytes;
      r = r < nrows ? r : nrows - 1;  // past the segment: repeat its last row (never added)
      const char *g = base + (long long)r * row_stride + col0 + (unit * 16) % row_bytes;
      __builtin_amdgcn_global_load_lds(
          (const void *)g, (__attribute__((address_space(3))) void *)&ring[c % kWaveRing][i * 1024],
          16, 0, 0);
    }
  };
  // CSPLIT == 1: lane t adds channels 2t, 2t+1; CSPLIT == 2: lane t adds channel t
  constexpr int kCh = CSPLIT == 1 ? 2 : 1;
  const int ch = kCh * lane;
  const bool active = ch < Dw;
  double a0 = 0.0, a1 = 0.0;
  for (int c = 0; c < kWaveRing - 1 && c < nchunks; ++c) issue(c);
  for (int c = 0; c < nchunks; ++c) {
    if (c + kWaveRing - 1 < nchunks) {
      issue(c + kWaveRing - 1);
      wait_vmcnt<(kWaveChunk / 1024) * (kWaveRing - 1)>();  // chunk c has landed
    } else {
      wait_vmcnt<0>();
    }
    const int rows = min(rows_per_chunk, nrows - c * rows_per_chunk);
    const unsigned char *t = ring[c % kWaveRing];
    if (active) {
      if (kCh == 2) {
        for (int r = 0; r < rows; ++r) {
          double x0, x1;
          pair_as_double<T>(t + r * row_bytes + ch * (int)sizeof(T), x0, x1);
          a0 = a0 + x0;
          a1 = a1 + x1;
        }
      } else {
        for (int r = 0; r < rows; ++r)
          a0 = a0 + elem_as_double<T>(reinterpret_cast<const T *>(t + r * row_bytes), 0, ch, 0);
      }
    }
  }
  if (active) {
    out[cgroup * Dw + ch] = a0;
    if (kCh == 2) out[cgroup * Dw + ch + 1] = a1;
  }
}

template <typename T, int kWaveRing, int CSPLIT>
__global__ void __launch_bounds__(64) pool_wave_kernel(
    const T *__restrict__ q, const T *__restrict__ k, int H, int Nq, int Nk, int D, int P,
    int h_begin, int Hs, int Tq, int cand_begin, int F, double *__restrict__ qframe,
    double *__restrict__ ksum) {
  const long long bid = blockIdx.x / CSPLIT;
  const int cgroup = (int)(blockIdx.x % CSPLIT);
  // layout: b-major, then [Tq query segments | F key segments] per selected head
  const int per_b = Hs * (Tq + F);
  const int b = (int)(bid / per_b);
  const int rem = (int)(bid % per_b);
  if (rem < Hs * Tq) {
    const int hs = rem / Tq, t = rem % Tq;
    const long long head = (long long)b * H + h_begin + hs;
    pool_segment_wave<T, kWaveRing, CSPLIT>(q, head * Nq + (long long)t * P, P, D, cgroup,
                         qframe + ((long long)(b * Hs + hs) * Tq + t) * D);
  } else {
    const int r2 = rem - Hs * Tq;
    const int hs = r2 / F, fi = r2 % F;
    const long long head = (long long)b * H + h_begin + hs;
    pool_segment_wave<T, kWaveRing, CSPLIT>(k, head * Nk + (long long)(cand_begin + fi) * P, P, D,
                                            cgroup,
                         ksum + ((long long)(b * Hs + hs) * F + fi) * D);
  }
}

// sum_d qs[d] * row[d] in ascending d, each product rounded before it is
// added.  The row (global memory) is read 16 values at a time into registers
// ahead of the ordered adds, so the loads overlap instead of each add waiting
// for its own load.
__device__ inline double ordered_dot(const double *qs, const double *__restrict__ row, int D) {
  double acc = 0.0;
  int d0 = 0;
  if ((reinterpret_cast<uintptr_t>(row) & 15u) == 0) {
    for (; d0 + 16 <= D; d0 += 16) {
      double2 x[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) x[t] = reinterpret_cast<const double2 *>(row + d0)[t];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
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

// Pools every query segment [t*P, (t+1)*P) of Nq and every key segment
// cand_begin + fi, fi < F, of the heads [h_begin, h_begin + Hs): one wavefront
// per segment where the rows allow it, else pool_kernel.
inline void launch_pool(int32_t dt, const void *q, const void *k, int H, int Nq, int Nk, int D,
                        int P, int h_begin, int Hs, int Tq, int cand_begin, int F, long long blocks,
                        double *qframe, double *ksum, hipStream_t s) {
  const bool aligned =
      ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k)) & 15u) == 0;
  const int row_bytes = D * (dt == FSA_BF16 ? 2 : 4);
  const bool pow2_row = row_bytes >= 16 && row_bytes <= 1024 && (row_bytes & (row_bytes - 1)) == 0;
  if (aligned && pow2_row && D % 2 == 0 && D <= 128) {
    // segments of at most two chunks fit a two-slot ring: smaller LDS, more
    // wavefronts per CU; longer segments stream through four slots, and when
    // a half row is still 128 bytes or more their channels are split over two
    // wavefronts (one ordered chain per lane, half the instructions each)
    const bool short_seg = P <= 2 * (kWaveChunk / row_bytes);
    const bool split = !short_seg && row_bytes >= 256;
    const dim3 grid((unsigned)(blocks * (split ? 2 : 1))), block(64);
    if (dt == FSA_BF16) {
      auto qq = static_cast<const Bf16 *>(q);
      auto kk = static_cast<const Bf16 *>(k);
      if (short_seg)
        hipLaunchKernelGGL((pool_wave_kernel<Bf16, 2, 1>), grid, block, 0, s, qq, kk, H, Nq, Nk,
                           D, P, h_begin, Hs, Tq, cand_begin, F, qframe, ksum);
      else if (split)
        hipLaunchKernelGGL((pool_wave_kernel<Bf16, 4, 2>), grid, block, 0, s, qq, kk, H, Nq, Nk,
                           D, P, h_begin, Hs, Tq, cand_begin, F, qframe, ksum);
      else
        hipLaunchKernelGGL((pool_wave_kernel<Bf16, 4, 1>), grid, block, 0, s, qq, kk, H, Nq, Nk,
                           D, P, h_begin, Hs, Tq, cand_begin, F, qframe, ksum);
    } else {
      auto qq = static_cast<const float *>(q);
      auto kk = static_cast<const float *>(k);
      if (short_seg)
        hipLaunchKernelGGL((pool_wave_kernel<float, 2, 1>), grid, block, 0, s, qq, kk, H, Nq, Nk,
                           D, P, h_begin, Hs, Tq, cand_begin, F, qframe, ksum);
      else if (split)
        hipLaunchKernelGGL((pool_wave_kernel<float, 4, 2>), grid, block, 0, s, qq, kk, H, Nq, Nk,
                           D, P, h_begin, Hs, Tq, cand_begin, F, qframe, ksum);
      else
        hipLaunchKernelGGL((pool_wave_kernel<float, 4, 1>), grid, block, 0, s, qq, kk, H, Nq, Nk,
                           D, P, h_begin, Hs, Tq, cand_begin, F, qframe, ksum);
    }
    return;
  }
  if (dt == FSA_BF16) {
    const size_t chunk = (size_t)kRowsPerChunk * D * sizeof(Bf16);
    const size_t lds = aligned && chunk * kRing <= 65536 ? chunk * kRing : chunk;
    hipLaunchKernelGGL(pool_kernel<Bf16>, dim3((unsigned)blocks), dim3(kPoolThreads), lds, s,
                       static_cast<const Bf16 *>(q), static_cast<const Bf16 *>(k), H, Nq, Nk, D,
                       P, h_begin, Hs, Tq, cand_begin, F, lds > chunk, qframe, ksum);
  } else {
    const size_t chunk = (size_t)kRowsPerChunk * D * sizeof(float);
    const size_t lds = aligned && chunk * kRing <= 65536 ? chunk * kRing : chunk;
    hipLaunchKernelGGL(pool_kernel<float>, dim3((unsigned)blocks), dim3(kPoolThreads), lds, s,
                       static_cast<const float *>(q), static_cast<const float *>(k), H, Nq, Nk,
                       D, P, h_begin, Hs, Tq, cand_begin, F, lds > chunk, qframe, ksum);
  }
}

}  // namespace
