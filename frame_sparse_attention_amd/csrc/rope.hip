// Per-head frame-level rotary re-encoding of an assembled KV cache
// (Head Forcing §3: keys are cached with the spatial rotary encoding only;
// when a head's cache is assembled its frame-level positions are encoded
// again, per head, so query-key relative positions stay in the trained range).
//
// For one sorted frame set A per (b, h): key frame f = A[r] turns by position
// r, query frame tq (KV frame offset + tq) by the number of frames of A before
// it.  Pair i = channels (2i, 2i+1), i < rot/2, turns by pos * base^(-2i/rot);
// channels from rot on are copied.  The rotation runs in float64 with
// contraction off and is rounded once to the storage type (nearest, ties to
// even), so the results are reproducible bit for bit.
//
// One block per (b, h, slot, 64-row piece of the frame): slots [0, cap) are
// the listed key frames, slots [cap, cap + Tq) the query frames.  The host
// passes cos and sin of each pair's frequency theta_i = base^(-2i/rot); the
// block raises (cos theta_i, sin theta_i) to its integer position by complex
// squaring in float64 (about log2(pos) products instead of a transcendental
// call).  A row is D/8 units of 8 channels (16 bytes of bf16, 32 of float32);
// the ceil(rot/8) units holding rotated pairs and the units copied as they
// are form two index spaces of their own, so every lane of a wavefront takes
// the same path: first the copies (they need no table, so they stream while
// it is built), then the rotations.  With 64-row pieces a thread has all of
// its units in flight at once for D = 128 (measured: 64-row pieces 21.9 us on
// the AR chunk, 128-row 22.5, 256-row 26.4, 32-row 22.2).  HBM-bound: every
// element of a listed frame is read and written once.
#pragma clang fp contract(off)

#include <cmath>

#include "fsa_internal.h"

namespace {

constexpr int kRopeThreads = 256;
constexpr int kMaxRotPairs = 128;  // rot <= 256
constexpr int kRopeRows = 64;      // token rows of one frame per block
constexpr int kRopeUnroll = 2;     // rotated 8-channel units in flight per thread
constexpr int kCopyUnroll = 4;     // copied 8-channel units in flight per thread

// cos and sin of every pair's frequency, computed on the host
struct RopeFreqs {
  double c[kMaxRotPairs];
  double s[kMaxRotPairs];
};

// the nearest bfloat16 (ties to even) of a double, as raw bits.  Results in
// the normal bfloat16 range are rounded on the bit pattern: the 45 low
// fraction bits go, half-way cases to the even neighbour; a carry out of the
// fraction moves into the exponent as it should.  Zeros, subnormal and
// overflowing results, infinities and NaN take the scaled arithmetic path.
__device__ inline uint16_t bf16_bits_nearest(double x) {
  const unsigned long long b = (unsigned long long)__double_as_longlong(x);
  const int ex = (int)((b >> 52) & 0x7FF) - 1023;  // unbiased exponent
  if (ex >= -126 && ex <= 126) {
    const unsigned long long mag = b & 0x7FFFFFFFFFFFFFFFull;
    const unsigned long long lsb = (mag >> 45) & 1ull;
    const unsigned long long r = (mag + 0x0FFFFFFFFFFFull + lsb) >> 45;  // 11+7 bits left
    // rebias the exponent from 1023 to 127: subtract (1023 - 127) << 7
    const unsigned int bits = (unsigned int)(r - (896ull << 7));
    return (uint16_t)(((b >> 48) & 0x8000u) | bits);
  }
  double r = x;
  if (x != 0.0 && isfinite(x)) {
    int e;
    (void)frexp(x, &e);            // x = m * 2^e, 0.5 <= |m| < 1
    e = e < -125 ? -125 : e;       // below the normal range the spacing is 2^-133
    const double q = rint(ldexp(x, 8 - e));  // 8 significant bits, ties to even
    r = ldexp(q, e - 8);
    if (fabs(r) > 3.3895313892515355e38) r = copysign((double)INFINITY, x);
  }
  return (uint16_t)(__float_as_uint((float)r) >> 16);  // r is a bfloat16 value: exact
}

// 8 consecutive channels as loaded: 16 bytes of bf16 or 32 of float32
template <typename T>
struct Chunk8 {
  uint4 w[sizeof(T) == 2 ? 1 : 2];
};
template <typename T>
__device__ inline Chunk8<T> load_chunk(const T *p) {
  Chunk8<T> c;
#pragma unroll
  for (int i = 0; i < (int)(sizeof(c.w) / 16); ++i) c.w[i] = reinterpret_cast<const uint4 *>(p)[i];
  return c;
}
template <typename T>
__device__ inline void store_chunk(T *p, const Chunk8<T> &c) {
#pragma unroll
  for (int i = 0; i < (int)(sizeof(c.w) / 16); ++i) reinterpret_cast<uint4 *>(p)[i] = c.w[i];
}
__device__ inline void widen8(const Chunk8<uint16_t> &c, double *x) {
  const uint32_t w[4] = {c.w[0].x, c.w[0].y, c.w[0].z, c.w[0].w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = (double)__uint_as_float(w[i] << 16);
    x[2 * i + 1] = (double)__uint_as_float(w[i] & 0xFFFF0000u);
  }
}
__device__ inline void widen8(const Chunk8<float> &c, double *x) {
  const uint32_t w[8] = {c.w[0].x, c.w[0].y, c.w[0].z, c.w[0].w,
                         c.w[1].x, c.w[1].y, c.w[1].z, c.w[1].w};
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = (double)__uint_as_float(w[i]);
}
__device__ inline bool bf16_normal(double x) {
  const int ex = (int)(((unsigned long long)__double_as_longlong(x) >> 52) & 0x7FF) - 1023;
  return ex >= -126 && ex <= 126;
}
__device__ inline uint32_t bf16_fast(double x) {
  const unsigned long long b = (unsigned long long)__double_as_longlong(x);
  const unsigned long long mag = b & 0x7FFFFFFFFFFFFFFFull;
  const unsigned long long lsb = (mag >> 45) & 1ull;
  const unsigned long long r = (mag + 0x0FFFFFFFFFFFull + lsb) >> 45;
  return (uint32_t)(((b >> 48) & 0x8000u) | (unsigned int)(r - (896ull << 7)));
}
__device__ inline void store8(uint16_t *p, const double *y) {
  uint32_t h[8];
  bool all = true;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    h[i] = bf16_fast(y[i]);
    all = all && bf16_normal(y[i]);
  }
  if (!all) {
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = bf16_bits_nearest(y[i]);
  }
  *reinterpret_cast<uint4 *>(p) =
      make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
}

__device__ inline void store8(float *p, const double *y) {
  *reinterpret_cast<float4 *>(p) = make_float4((float)y[0], (float)y[1], (float)y[2], (float)y[3]);
  *reinterpret_cast<float4 *>(p + 4) =
      make_float4((float)y[4], (float)y[5], (float)y[6], (float)y[7]);
}


// (cos p x, sin p x) from (cos x, sin x) for an integer p >= 0, by binary
// powers of the unit complex number; each product is rounded (contraction is
// off), and the result is within a few units in the last place of float64.
__device__ inline void cis_power(double c1, double s1, int p, double *c, double *s) {
  double rc = 1.0, rs = 0.0, bc = c1, bs = s1;
  while (p > 0) {
    if (p & 1) {
      const double a = rc * bc, b = rs * bs, e = rc * bs, f = rs * bc;
      rc = a - b;
      rs = e + f;
    }
    const double a = bc * bc, b = bs * bs, e = bc * bs;
    bc = a - b;
    bs = e + e;
    p >>= 1;
  }
  *c = rc;
  *s = rs;
}

template <typename T>
__global__ void __launch_bounds__(kRopeThreads) rope_reencode_kernel(
    const T *q, const T *k, T *qo, T *ko,
    const int32_t *__restrict__ idx, const int32_t *__restrict__ cnt, int cap, int Nq, int Nk,
    int D, int P, int Tk, int offset, int rot, RopeFreqs freqs, int slots, int row_blocks) {
  __shared__ double s_cos[kMaxRotPairs], s_sin[kMaxRotPairs];
  __shared__ int s_pos;
  const int tid = threadIdx.x;
  const int rb = blockIdx.x % row_blocks;
  const int slot = (blockIdx.x / row_blocks) % slots;
  const long long bh = blockIdx.x / ((long long)row_blocks * slots);
  const int32_t *lst = idx + bh * cap;
  // the list count and this slot's entry are requested together
  int n = cnt[bh];
  const int f = slot < cap ? lst[slot] : 0;
  n = n < 0 ? 0 : (n > cap ? cap : n);
  const T *src;
  T *dst;
  if (slot < cap) {  // listed key frame: its rank is its slot
    if (slot >= n || f < 0 || f >= Tk) return;
    src = k + (bh * Nk + (long long)f * P) * D;
    dst = ko + (bh * Nk + (long long)f * P) * D;
  } else {  // query frame tq = slot - cap
    src = q + (bh * Nq + (long long)(slot - cap) * P) * D;
    dst = qo + (bh * Nq + (long long)(slot - cap) * P) * D;
  }
  if (tid < 64) {
    if (slot < cap) {
      if (tid == 0) s_pos = slot;
    } else {  // rank of KV frame offset + tq among the listed frames, 64 entries at a time
      const int target = offset + (slot - cap);
      int before = 0;
      for (int i0 = 0; i0 < n; i0 += 64) {
        const int i = i0 + tid;
        before += __popcll(__ballot(i < n && lst[i] < target));
      }
      if (tid == 0) s_pos = before;
    }
  }
  const int per_row = D / 8;
  const int rot_units = (rot + 7) / 8;  // units 0 .. rot_units-1 of a row hold rotated pairs
  const int copy_units = per_row - rot_units;
  const int row0 = rb * kRopeRows;
  const int rows = P - row0 < kRopeRows ? P - row0 : kRopeRows;
  const T *sb = src + (long long)row0 * D;
  T *db = dst + (long long)row0 * D;
  // the first rotated units are requested before anything else
  const int nrot = rows * rot_units;
  Chunk8<T> xr[kRopeUnroll];
#pragma unroll
  for (int i = 0; i < kRopeUnroll; ++i) {
    const int u = tid + i * kRopeThreads;
    if (u < nrot) xr[i] = load_chunk(sb + (u / rot_units) * D + (u % rot_units) * 8);
  }
  // units without a rotated pair: the bytes move as they are
  const int ncopy = rows * copy_units;
  for (int u0 = tid; u0 < ncopy; u0 += kCopyUnroll * kRopeThreads) {
    Chunk8<T> x[kCopyUnroll];
#pragma unroll
    for (int i = 0; i < kCopyUnroll; ++i) {
      const int u = u0 + i * kRopeThreads;
      if (u < ncopy) x[i] = load_chunk(sb + (u / copy_units) * D + (rot_units + u % copy_units) * 8);
    }
#pragma unroll
    for (int i = 0; i < kCopyUnroll; ++i) {
      const int u = u0 + i * kRopeThreads;
      if (u < ncopy) store_chunk(db + (u / copy_units) * D + (rot_units + u % copy_units) * 8, x[i]);
    }
  }
  __syncthreads();
  for (int i = tid; i < rot / 2; i += kRopeThreads) {
    double c, sn;
    cis_power(freqs.c[i], freqs.s[i], s_pos, &c, &sn);
    s_cos[i] = c;
    s_sin[i] = sn;
  }
  __syncthreads();
  // units with rotated pairs
  for (int u0 = tid; u0 < nrot; u0 += kRopeUnroll * kRopeThreads) {
    Chunk8<T> x[kRopeUnroll];
#pragma unroll
    for (int i = 0; i < kRopeUnroll; ++i) {
      const int u = u0 + i * kRopeThreads;
      if (u0 == tid)
        x[i] = xr[i];
      else if (u < nrot)
        x[i] = load_chunk(sb + (u / rot_units) * D + (u % rot_units) * 8);
    }
#pragma unroll
    for (int i = 0; i < kRopeUnroll; ++i) {
      const int u = u0 + i * kRopeThreads;
      if (u >= nrot) continue;
      const int c0 = (u % rot_units) * 8;
      double v[8], y[8];
      widen8(x[i], v);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int pr = c0 / 2 + j;
        if (2 * pr < rot) {
          const double c = s_cos[pr], s = s_sin[pr];
          const double a0 = v[2 * j] * c, a1 = v[2 * j + 1] * s;
          const double b0 = v[2 * j] * s, b1 = v[2 * j + 1] * c;
          y[2 * j] = a0 - a1;
          y[2 * j + 1] = b0 + b1;
        } else {
          y[2 * j] = v[2 * j];
          y[2 * j + 1] = v[2 * j + 1];
        }
      }
      store8(db + (u / rot_units) * D + c0, y);
    }
  }
}

}  // namespace

extern "C" fsa_status fsa_rope_reencode(const void *q, const void *k, int32_t dt, int32_t B,
                                        int32_t H, int32_t Nq, int32_t Nk, int32_t D, int32_t P,
                                        const int32_t *idx, const int32_t *cnt, int32_t cap,
                                        int32_t q_kv_offset, int32_t rot, double base,
                                        void *q_out, void *k_out, void *stream) {
  fsa::clear_error();
  FSA_REQUIRE(B >= 0 && H >= 0 && Nq >= 0 && Nk >= 0, FSA_E_ARG, "negative size");
  FSA_REQUIRE(dt == FSA_F32 || dt == FSA_BF16, FSA_E_DTYPE, "unknown dtype %d", dt);
  FSA_REQUIRE(D >= 8 && D <= 2 * kMaxRotPairs && D % 8 == 0, FSA_E_SHAPE,
              "D=%d must be a multiple of 8 in [8, %d]", D, 2 * kMaxRotPairs);
  FSA_REQUIRE(P >= 1, FSA_E_SHAPE, "P=%d must be >= 1", P);
  FSA_REQUIRE(Nq % P == 0 && Nk % P == 0, FSA_E_SHAPE, "Nq=%d or Nk=%d is not a multiple of P=%d",
              Nq, Nk, P);
  FSA_REQUIRE(rot >= 0 && rot <= D && rot % 2 == 0, FSA_E_ARG, "rot=%d must be even in [0, D=%d]",
              rot, D);
  FSA_REQUIRE(base > 0.0 && base < 1e300, FSA_E_ARG, "base must be positive and finite");
  FSA_REQUIRE(cap >= 1 && cap <= FSA_MAX_CAP, FSA_E_CAPACITY, "cap=%d outside [1, %d]", cap,
              FSA_MAX_CAP);
  FSA_REQUIRE(q_kv_offset >= 0, FSA_E_ARG, "q_kv_offset=%d must be >= 0", q_kv_offset);
  const int Tq = Nq / P, Tk = Nk / P;
  const long long slots = (long long)cap + Tq;
  const int row_blocks = (P + kRopeRows - 1) / kRopeRows;
  const long long blocks = (long long)B * H * slots * row_blocks;
  if (blocks == 0) return FSA_OK;
  FSA_REQUIRE(q && k && idx && cnt && q_out && k_out, FSA_E_ARG, "null pointer argument");
  const uintptr_t align = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
                          reinterpret_cast<uintptr_t>(q_out) | reinterpret_cast<uintptr_t>(k_out);
  FSA_REQUIRE((align & 15u) == 0, FSA_E_ARG, "q, k, q_out and k_out must be 16-byte aligned");
  FSA_REQUIRE(blocks < (1LL << 31) && slots < (1LL << 30), FSA_E_SHAPE,
              "too many frames (%lld blocks)", blocks);
  // theta_i = base^(-2i/rot) and its cos / sin, in float64 on the host
  RopeFreqs freqs{};
  for (int i = 0; i < rot / 2; ++i) {
    const double th = std::pow(base, (-2.0 * i) / rot);
    freqs.c[i] = std::cos(th);
    freqs.s[i] = std::sin(th);
  }
  hipStream_t s = fsa::as_stream(stream);
  if (dt == FSA_BF16)
    hipLaunchKernelGGL(rope_reencode_kernel<uint16_t>, dim3((unsigned)blocks), dim3(kRopeThreads),
                       0, s, static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
                       static_cast<uint16_t *>(q_out), static_cast<uint16_t *>(k_out), idx, cnt,
                       cap, Nq, Nk, D, P, Tk, q_kv_offset, rot, freqs, (int)slots, row_blocks);
  else
    hipLaunchKernelGGL(rope_reencode_kernel<float>, dim3((unsigned)blocks), dim3(kRopeThreads), 0,
                       s, static_cast<const float *>(q), static_cast<const float *>(k),
                       static_cast<float *>(q_out), static_cast<float *>(k_out), idx, cnt, cap,
                       Nq, Nk, D, P, Tk, q_kv_offset, rot, freqs, (int)slots, row_blocks);
  return fsa::check_launch("rope_reencode");
}
