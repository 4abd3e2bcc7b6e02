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
// One block per (b, h, slot, 128-row piece of the frame): slots [0, cap) are
// the listed key frames, slots [cap, cap + Tq) the query frames.  The block
// computes the frame's cos/sin table in LDS, then streams its rows, 8
// channels (16 bytes of bf16, 32 of float32) per thread and step; 8-channel
// units with no rotated pair are copied as they are.  HBM-bound: every
// element of a listed frame is read and written once.
#pragma clang fp contract(off)

#include "fsa_internal.h"

namespace {

constexpr int kRopeThreads = 256;
constexpr int kMaxRotPairs = 128;  // rot <= 256
constexpr int kRopeRows = 128;     // token rows of one frame per block

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

__device__ inline void load8(const uint16_t *p, double *x) {
  const uint4 raw = *reinterpret_cast<const uint4 *>(p);
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = (double)__uint_as_float(w[i] << 16);
    x[2 * i + 1] = (double)__uint_as_float(w[i] & 0xFFFF0000u);
  }
}
__device__ inline void store8(uint16_t *p, const double *y) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = (uint32_t)bf16_bits_nearest(y[2 * i]) | ((uint32_t)bf16_bits_nearest(y[2 * i + 1]) << 16);
  *reinterpret_cast<uint4 *>(p) = make_uint4(w[0], w[1], w[2], w[3]);
}
__device__ inline void load8(const float *p, double *x) {
  const float4 a = *reinterpret_cast<const float4 *>(p);
  const float4 b = *reinterpret_cast<const float4 *>(p + 4);
  x[0] = a.x, x[1] = a.y, x[2] = a.z, x[3] = a.w;
  x[4] = b.x, x[5] = b.y, x[6] = b.z, x[7] = b.w;
}
__device__ inline void store8(float *p, const double *y) {
  *reinterpret_cast<float4 *>(p) = make_float4((float)y[0], (float)y[1], (float)y[2], (float)y[3]);
  *reinterpret_cast<float4 *>(p + 4) =
      make_float4((float)y[4], (float)y[5], (float)y[6], (float)y[7]);
}

__device__ inline void copy8(const uint16_t *p, uint16_t *q) {
  *reinterpret_cast<uint4 *>(q) = *reinterpret_cast<const uint4 *>(p);
}
__device__ inline void copy8(const float *p, float *q) {
  const float4 a = *reinterpret_cast<const float4 *>(p);
  const float4 b = *reinterpret_cast<const float4 *>(p + 4);
  *reinterpret_cast<float4 *>(q) = a;
  *reinterpret_cast<float4 *>(q + 4) = b;
}

template <typename T>
__global__ void __launch_bounds__(kRopeThreads) rope_reencode_kernel(
    const T *q, const T *k, T *qo, T *ko,
    const int32_t *__restrict__ idx, const int32_t *__restrict__ cnt, int cap, int Nq, int Nk,
    int D, int P, int Tk, int offset, int rot, double base, int slots, int row_blocks) {
  __shared__ double s_cos[kMaxRotPairs], s_sin[kMaxRotPairs];
  __shared__ int s_pos;
  const int tid = threadIdx.x;
  const int rb = blockIdx.x % row_blocks;
  const int slot = (blockIdx.x / row_blocks) % slots;
  const long long bh = blockIdx.x / ((long long)row_blocks * slots);
  const int32_t *lst = idx + bh * cap;
  int n = cnt[bh];
  n = n < 0 ? 0 : (n > cap ? cap : n);
  const T *src;
  T *dst;
  if (slot < cap) {  // listed key frame: its rank is its slot
    if (slot >= n) return;
    const int f = lst[slot];
    if (f < 0 || f >= Tk) return;
    if (tid == 0) s_pos = slot;
    src = k + (bh * Nk + (long long)f * P) * D;
    dst = ko + (bh * Nk + (long long)f * P) * D;
  } else {  // query frame tq: rank of KV frame offset + tq among the listed frames
    const int tq = slot - cap;
    if (tid == 0) {
      int before = 0;
      for (int i = 0; i < n; ++i) before += lst[i] < offset + tq ? 1 : 0;
      s_pos = before;
    }
    src = q + (bh * Nq + (long long)tq * P) * D;
    dst = qo + (bh * Nq + (long long)tq * P) * D;
  }
  __syncthreads();
  const double pos = (double)s_pos;
  for (int i = tid; i < rot / 2; i += kRopeThreads) {
    const double ang = pos * pow(base, (-2.0 * i) / rot);
    s_cos[i] = cos(ang);
    s_sin[i] = sin(ang);
  }
  __syncthreads();
  const int per_row = D / 8;
  const int row0 = rb * kRopeRows;
  const int rows = P - row0 < kRopeRows ? P - row0 : kRopeRows;
  const int units = rows * per_row;
  const int rot_units = (rot + 7) / 8;  // 8-channel units holding rotated pairs
  for (int u = tid; u < units; u += kRopeThreads) {
    const int row = row0 + u / per_row, c0 = (u % per_row) * 8;
    const long long off = (long long)row * D + c0;
    if (u % per_row >= rot_units) {  // no rotated channel: the 16 or 32 bytes move as they are
      copy8(src + off, dst + off);
      continue;
    }
    double x[8], y[8];
    load8(src + off, x);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int pr = c0 / 2 + j;
      if (2 * pr < rot) {
        const double c = s_cos[pr], s = s_sin[pr];
        const double a0 = x[2 * j] * c, a1 = x[2 * j + 1] * s;
        const double b0 = x[2 * j] * s, b1 = x[2 * j + 1] * c;
        y[2 * j] = a0 - a1;
        y[2 * j + 1] = b0 + b1;
      } else {
        y[2 * j] = x[2 * j];
        y[2 * j + 1] = x[2 * j + 1];
      }
    }
    store8(dst + off, y);
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
  hipStream_t s = fsa::as_stream(stream);
  if (dt == FSA_BF16)
    hipLaunchKernelGGL(rope_reencode_kernel<uint16_t>, dim3((unsigned)blocks), dim3(kRopeThreads),
                       0, s, static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
                       static_cast<uint16_t *>(q_out), static_cast<uint16_t *>(k_out), idx, cnt,
                       cap, Nq, Nk, D, P, Tk, q_kv_offset, rot, base, (int)slots, row_blocks);
  else
    hipLaunchKernelGGL(rope_reencode_kernel<float>, dim3((unsigned)blocks), dim3(kRopeThreads), 0,
                       s, static_cast<const float *>(q), static_cast<const float *>(k),
                       static_cast<float *>(q_out), static_cast<float *>(k_out), idx, cnt, cap,
                       Nq, Nk, D, P, Tk, q_kv_offset, rot, base, (int)slots, row_blocks);
  return fsa::check_launch("rope_reencode");
}
