// Frame-sparse attention for bfloat16 inputs on CDNA4 matrix cores.
//
// What is computed (LVSA §2 core mechanism and complexity paragraph; Light
// Forcing §2.2 execution over the selected frames; ISPA §2 item 1 LSE state):
// for each query row of frame t, softmax attention over the keys of the frames
// in A(t) only, returning O (float32) and the natural-log LSE.  The frames of
// A(t) are first merged into runs of consecutive frames (one contiguous key
// range each), and the kernel streams 64-key tiles of those runs.
//
// Layout and mapping (one block = 4 wavefronts = 128 query rows of one
// (b, h, frame); each wavefront owns 32 rows):
//   S^T = K Q^T   v_mfma_f32_32x32x16_bf16; A = K tile rows from LDS, B = the
//                 wavefront's Q rows held in VGPRs.  The output puts one query
//                 row per lane (lane l and l^32 share row l%32), so the row max
//                 and row sum are in-register reductions plus one cross-half
//                 exchange.
//   softmax       online, float32, base 2 with scale*log2(e) folded in; the
//                 row sum is accumulated from the float32 probabilities.
//   O^T += V^T P^T  v_mfma_f32_32x32x16_f16; B = the probabilities rounded to
//                 float16 straight from the S^T registers, A = V^T from LDS.
// K rows are stored in LDS in a permuted slot order (slot = key with bits 2
// and 3 swapped) so that the probabilities a lane holds after S^T are 8
// consecutive keys, which lets V^T be read as plain 16-byte rows.
// V is converted once per call to a float16, key-chunked transposed layout
// [B*H][ceil(Nk/8)][D][8] in the caller's workspace, so one 64-key V tile is a
// single contiguous 16 KB block.  (float16 probabilities keep max|dO| well
// inside 1e-2 on data with x8 outlier channels; bfloat16 ones do not.)
#include "attn_common.h"

namespace fsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kRowsPerWave = 32;
constexpr int kRows = 128;
constexpr int kTileKeys = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// s_waitcnt immediate: vmcnt(0), expcnt and lgkmcnt left at their maxima
constexpr int kWaitVm0 = 0x0F70;

__device__ inline float bf16_bits_to_float(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Value of x in the lane 32 apart (the other half of the wavefront).
__device__ inline float other_half(float x) { return __shfl_xor(x, 32); }

// ---------------------------------------------------------------------------
// V prepass: Vt[head][kc][d][e] = float16(V[head][8*kc + e][d]), zero past Nk.
// One thread per (head, kc, d); each reads 8 rows (coalesced across d) and
// writes 16 contiguous bytes.
__global__ void __launch_bounds__(256) v_to_f16_chunked_kernel(
    const uint16_t *__restrict__ v, _Float16 *__restrict__ vt, long long total, int Nk, int NkC,
    int D) {
  const long long u = (long long)blockIdx.x * 256 + threadIdx.x;
  if (u >= total) return;
  const int d = (int)(u % D);
  const long long hk = u / D;
  const int kc = (int)(hk % NkC);
  const long long hd = hk / NkC;
  const uint16_t *src = v + (hd * Nk) * D + d;
  f16x8 out;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int n = kc * 8 + e;
    out[e] = (_Float16)(n < Nk ? bf16_bits_to_float(src[(long long)n * D]) : 0.f);
  }
  *reinterpret_cast<f16x8 *>(vt + u * 8) = out;
}

// Slot of a key inside a 64-key K tile: bits 2 and 3 swapped (an involution).
__device__ inline int key_slot(int kk) {
  return (kk & ~12) | ((kk >> 1) & 4) | ((kk << 1) & 8);
}

struct Tile {
  int r;             // run index
  long long start;   // first key of the run
  long long end;     // one past the last key of the run
  long long n0;      // first key of the tile (multiple of 8, <= start on a run's first tile)
};

template <int D>
__global__ void __launch_bounds__(kThreads) attn_bf16_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const _Float16 *__restrict__ vt, const int32_t *__restrict__ idx,
    const int32_t *__restrict__ cnt, int cap, int H, int Nq, int Nk, int NkC, int P, int Tq,
    int qtiles, float scale_log2, float *__restrict__ o, float *__restrict__ lse) {
  constexpr int NCH = D / 8;                 // 16-byte chunks per K row
  constexpr int KBYTES = kTileKeys * D * 2;  // one K tile
  constexpr int VBYTES = (kTileKeys / 8) * D * 16;
  constexpr int KLD = KBYTES / 16 / kThreads;  // 16-byte K loads per thread per tile
  constexpr int VLD = VBYTES / 16 / kThreads;
  constexpr int SWZ = (NCH < 16 ? NCH : 16) - 1;
  __shared__ __attribute__((aligned(16))) unsigned char s_k[2][KBYTES];
  __shared__ __attribute__((aligned(16))) unsigned char s_v[2][VBYTES];
  __shared__ int s_lo[FSA_MAX_CAP], s_hi[FSA_MAX_CAP];
  __shared__ int s_nruns;

  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64, j = lane % 32, g = lane / 32;

  int tile = xcd_logical_tile(blockIdx.x, gridDim.x);
  const int qt = tile % qtiles;
  tile /= qtiles;
  const int tq = tile % Tq;
  tile /= Tq;
  const int h = tile % H;
  const int b = tile / H;
  const long long head = (long long)b * H + h;
  const long long list = head * Tq + tq;
  const int Tk = Nk / P;
  const int nruns = build_runs(idx + list * cap, cnt[list], cap, Tk, RunList{s_lo, s_hi}, &s_nruns);

  const int prow0 = qt * kRows + wave * kRowsPerWave;  // first row of this wave in the frame
  const bool wave_active = prow0 < P;
  const int my_prow = prow0 + j;
  const bool row_ok = my_prow < P;
  const long long qrow = (long long)tq * P + (my_prow < P ? my_prow : P - 1);

  // Q rows of this wave as the B operand: lane (j + 32g) holds row j, d = 16ks + 8g .. +7
  bf16x8 qf[D / 16];
  {
    const uint16_t *qp = q + (head * Nq + qrow) * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qf[ks] = *reinterpret_cast<const bf16x8 *>(qp + 16 * ks);
  }

  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};
  float m = -INFINITY;  // running row max, in scaled base-2 units
  float l = 0.f;        // running row sum (this lane's half of the keys)

  const uint16_t *kh = k + head * (long long)Nk * D;
  const _Float16 *vh = vt + head * (long long)NkC * D * 8;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);

  // Tile loads go straight from HBM into LDS (global_load_lds_dwordx4): each
  // wavefront instruction fills 64 consecutive 16-byte LDS units, one per
  // lane, and the lane picks the global chunk that belongs at its unit.
  // K: unit u -> slot u / NCH, stored chunk u % NCH, which holds logical chunk
  // (u % NCH) ^ (slot & SWZ) of key key_slot(slot).  V^T: unit u is the u-th
  // 16-byte chunk of the tile, contiguous in the workspace.
  int koff[KLD];
#pragma unroll
  for (int it = 0; it < KLD; ++it) {
    const int u = (it * 4 + wave_u) * 64 + lane;
    const int slot = u / NCH, pc = u % NCH;
    const int kk = key_slot(slot), c = pc ^ (slot & SWZ);
    koff[it] = kk * D + c * 8;
  }
  auto issue_tile = [&](long long n0, int b) {
    const bool k_tail = n0 + kTileKeys > Nk;
#pragma unroll
    for (int it = 0; it < KLD; ++it) {
      const uint16_t *src = kh + n0 * D + koff[it];
      if (k_tail) {
        long long key = n0 + koff[it] / D;
        key = key < Nk ? key : Nk - 1;
        src = kh + key * D + koff[it] % D;
      }
      __builtin_amdgcn_global_load_lds(
          (const void *)src,
          (__attribute__((address_space(3))) void *)&s_k[b][(it * 4 + wave_u) * 1024], 16, 0, 0);
    }
    const bool v_tail = n0 / 8 + kTileKeys / 8 > NkC;
#pragma unroll
    for (int it = 0; it < VLD; ++it) {
      const int u = (it * 4 + wave_u) * 64 + lane;
      long long chunk = n0 / 8 + u / D;
      if (v_tail) chunk = chunk < NkC ? chunk : NkC - 1;
      const _Float16 *src = vh + (chunk * D + u % D) * 8;
      __builtin_amdgcn_global_load_lds(
          (const void *)src,
          (__attribute__((address_space(3))) void *)&s_v[b][(it * 4 + wave_u) * 1024], 16, 0, 0);
    }
  };
  auto first_tile = [&](int r) {
    Tile t;
    t.r = r;
    if (r < nruns) {
      t.start = (long long)s_lo[r] * P;
      t.end = (long long)(s_hi[r] + 1) * P;
      t.n0 = t.start & ~7LL;
    } else {
      t.start = t.end = t.n0 = 0;
    }
    return t;
  };

  Tile cur = first_tile(0);
  if (nruns > 0) issue_tile(cur.n0, 0);
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();
  int buf = 0;
  while (cur.r < nruns) {
    Tile nxt = cur;
    nxt.n0 += kTileKeys;
    if (nxt.n0 >= nxt.end) nxt = first_tile(cur.r + 1);
    const bool has_next = nxt.r < nruns;
    if (has_next) issue_tile(nxt.n0, buf ^ 1);

    if (wave_active) {
      const unsigned char *kb_base = s_k[buf];
      const unsigned char *vb_base = s_v[buf];
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x16{};
        const int slot = kb * 32 + j;
        const unsigned char *krow = kb_base + slot * D * 2;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          const int c = 2 * ks + g;
          const bf16x8 a = *reinterpret_cast<const bf16x8 *>(krow + ((c ^ (slot & SWZ)) * 16));
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[kb], 0, 0, 0);
        }
      }
      // keys of this tile outside the run: [lo_rel, hi_rel) are valid
      const int lo_rel = (int)(cur.start > cur.n0 ? cur.start - cur.n0 : 0);
      const long long span = cur.end - cur.n0;
      const int hi_rel = span < kTileKeys ? (int)span : kTileKeys;
      if (lo_rel > 0 || hi_rel < kTileKeys) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = 32 * kb + (i & 7) + 8 * g + 16 * (i >> 3);
            if (key < lo_rel || key >= hi_rel) s[kb][i] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
      mx = fmaxf(mx, other_half(mx));
      const float m_new = fmaxf(m, mx * scale_log2);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m - m_use);
      f16x8 pf[4];
      float psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][i], scale_log2, -m_use));
          psum += p;
          pf[2 * kb + (i >> 3)][i & 7] = (_Float16)p;
        }
      l = l * alpha + psum;
      m = m_new;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) acc[db] *= alpha;
#pragma unroll
      for (int ms = 0; ms < 4; ++ms) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const f16x8 a =
              *reinterpret_cast<const f16x8 *>(vb_base + ((2 * ms + g) * D + db * 32 + j) * 16);
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pf[ms], acc[db], 0, 0, 0);
        }
      }
    }

    __builtin_amdgcn_s_waitcnt(kWaitVm0);  // this wave's tile loads have landed in LDS
    __syncthreads();
    buf ^= 1;
    cur = nxt;
  }

  if (!wave_active) return;
  const float l_tot = l + other_half(l);
  if (!row_ok) return;
  const long long orow = head * Nq + (long long)tq * P + my_prow;
  float inv, lse_v;
  if (l_tot > 0.f) {
    inv = 1.f / l_tot;
    lse_v = (m + __log2f(l_tot)) * kLn2;
  } else {
    inv = 0.f;
    lse_v = -INFINITY;
  }
  float *op = o + orow * D;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      float4 val;
      val.x = acc[db][4 * q4 + 0] * inv;
      val.y = acc[db][4 * q4 + 1] * inv;
      val.z = acc[db][4 * q4 + 2] * inv;
      val.w = acc[db][4 * q4 + 3] * inv;
      *reinterpret_cast<float4 *>(op + db * 32 + 8 * q4 + 4 * g) = val;
    }
  if (g == 0) lse[orow] = lse_v;
}

}  // namespace

size_t attn_bf16_workspace(long long heads, int Nk, int D) {
  const long long NkC = (Nk + 7) / 8;
  return (size_t)heads * NkC * D * 8 * sizeof(_Float16);
}

fsa_status launch_prepare_values_bf16(const void *v, int B, int H, int Nk, int D, void *prepared,
                                      hipStream_t stream) {
  const long long heads = (long long)B * H;
  const int NkC = (Nk + 7) / 8;
  if (NkC == 0 || heads == 0) return FSA_OK;
  const long long total = heads * NkC * D;
  const long long blocks = (total + 255) / 256;
  FSA_REQUIRE(blocks < (1LL << 31), FSA_E_SHAPE, "V too large (%lld blocks)", blocks);
  hipLaunchKernelGGL(v_to_f16_chunked_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<const uint16_t *>(v), static_cast<_Float16 *>(prepared), total,
                     Nk, NkC, D);
  return check_launch("prepare_values");
}

fsa_status launch_attn_bf16_prepared(const void *q, const void *k, const void *prepared,
                                     const int32_t *idx, const int32_t *cnt, int cap, int B,
                                     int H, int Nq, int Nk, int D, int P, float scale, float *o,
                                     float *lse, hipStream_t stream) {
  const long long heads = (long long)B * H;
  const int NkC = (Nk + 7) / 8;
  const int Tq = Nq / P;
  const int qtiles = (P + kRows - 1) / kRows;
  const long long blocks = heads * Tq * qtiles;
  FSA_REQUIRE(blocks < (1LL << 31), FSA_E_SHAPE, "too many query tiles (%lld)", blocks);
  const float scale_log2 = scale * kLog2e;
  auto qq = static_cast<const uint16_t *>(q);
  auto kk = static_cast<const uint16_t *>(k);
  auto vt = static_cast<const _Float16 *>(prepared);
  if (D == 64)
    hipLaunchKernelGGL(attn_bf16_kernel<64>, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                       qq, kk, vt, idx, cnt, cap, H, Nq, Nk, NkC, P, Tq, qtiles, scale_log2, o,
                       lse);
  else
    hipLaunchKernelGGL(attn_bf16_kernel<128>, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                       qq, kk, vt, idx, cnt, cap, H, Nq, Nk, NkC, P, Tq, qtiles, scale_log2, o,
                       lse);
  return check_launch("sparse_frame_attn (bf16)");
}

}  // namespace fsa
