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

// ---------------------------------------------------------------------------
// V prepass: Vt[head][kc][d][e] = float16(V[head][8*kc + e][d]), zero past Nk.
// One block per (head, 64 keys): 16-byte coalesced loads of the [64][D] bf16
// tile, conversion to float16 into LDS, then 16-byte coalesced stores of the
// [8 chunks][D][8] image (HBM-bound: 2 bytes read + 2 written per element).
//
// Values beyond the float16 range saturate to +-65504 instead of becoming
// infinite: a 64-key tile also holds keys outside a row's frame set (before
// an unaligned run start, after a run end), whose probabilities are exactly
// 0, and 0 * inf would turn that row's output into NaN.  NaN stays NaN.
__device__ inline _Float16 f16_saturate(float x) {
  const float c = fminf(fmaxf(x, -65504.f), 65504.f);
  return (_Float16)(x != x ? x : c);
}
template <int D>
__global__ void __launch_bounds__(256) v_to_f16_chunked_kernel(const uint16_t *__restrict__ v,
                                                               _Float16 *__restrict__ vt,
                                                               int Nk, int NkC) {
  constexpr int kKeys = 64, NCH = D / 8;
  __shared__ _Float16 tile[kKeys][D + 2];  // +2: rows start on different banks
  const long long head = blockIdx.y;
  const int key0 = blockIdx.x * kKeys;
  const uint16_t *src = v + (head * Nk + key0) * D;
  for (int u = threadIdx.x; u < kKeys * NCH; u += 256) {
    const int kk = u / NCH, c = u % NCH;
    uint4 raw = make_uint4(0, 0, 0, 0);
    if (key0 + kk < Nk) raw = *reinterpret_cast<const uint4 *>(src + kk * D + c * 8);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      tile[kk][c * 8 + 2 * e] = f16_saturate(__uint_as_float(w[e] << 16));
      tile[kk][c * 8 + 2 * e + 1] = f16_saturate(__uint_as_float(w[e] & 0xffff0000u));
    }
  }
  __syncthreads();
  const int c0 = key0 / 8;
  for (int u = threadIdx.x; u < (kKeys / 8) * D; u += 256) {
    const int kc = u / D, d = u % D;
    if (c0 + kc >= NkC) break;
    f16x8 out;
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = tile[kc * 8 + e][d];
    *reinterpret_cast<f16x8 *>(vt + ((head * NkC + c0 + kc) * D + d) * 8) = out;
  }
}

// Slot of a key inside a 64-key K tile: bits 2 and 3 swapped (an involution).
__device__ inline int key_slot(int kk) {
  return (kk & ~12) | ((kk >> 1) & 4) | ((kk << 1) & 8);
}

// The reference max of a row moves exactly to the running max: the largest
// probability of a row is then exactly 1.0, which float16 holds without error
// (a stale reference would put it anywhere in [1, 2^k) and give it the full
// float16 rounding error, which on peaked rows with large values approaches
// the output tolerance).  Tiles where no row of the wavefront found a new max
// skip the rescale altogether; that is bitwise identical to multiplying by 1.
// Cross-half exchange: {x, x of lane l^32} via v_permlane32_swap.
struct HalfPair {
  float a, b;
};
__device__ inline HalfPair with_other_half(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}

// A frame-list argument (idx [B][H][Tq][cap], cnt [B][H][Tq]) and an output pair.
struct ListArg {
  const int32_t *idx;
  const int32_t *cnt;
  int cap;
};
struct OutArg {
  float *o;
  float *lse;
};

// DUAL = false: attention over the frames of list `la`, written to `all`.
// DUAL = true: one pass over the runs of `la` followed by the runs of `lb`
// with a single running softmax state; after the last tile of `la` the state
// is written to `first` (attention over A alone), at the end to `all`
// (attention over A and B together, exact when the two lists are disjoint).
template <int D, bool DUAL>
__global__ void __launch_bounds__(kThreads, 2) attn_bf16_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const _Float16 *__restrict__ vt, ListArg la, ListArg lb, int H, int Nq, int Nk, int NkC,
    int P, int Tq, int qtiles, float scale_log2, OutArg first, OutArg all, int splits,
    long long o_split_stride, long long lse_split_stride) {
  constexpr int NCH = D / 8;                 // 16-byte chunks per K row
  constexpr int KBYTES = kTileKeys * D * 2;  // one K tile
  constexpr int VBYTES = (kTileKeys / 8) * D * 16;
  constexpr int KLD = KBYTES / 16 / kThreads;  // 16-byte K loads per thread per tile
  constexpr int VLD = VBYTES / 16 / kThreads;
  constexpr int SWZ = (NCH < 16 ? NCH : 16) - 1;
  __shared__ __attribute__((aligned(16))) unsigned char s_k[2][KBYTES];
  __shared__ __attribute__((aligned(16))) unsigned char s_v[2][VBYTES];
  __shared__ int s_lo[FSA_MAX_CAP], s_hi[FSA_MAX_CAP];
  __shared__ int s_nruns[2];
  __shared__ int s_unequal;
  __shared__ int s_order[128];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lane = tid % 64, j = lane % 32, g = lane / 32;

  int tile, qt, sp, tq;
  int lst;
  // (D = 128: two blocks per CU; the D = 64 kernel fits three, other pairs)
  if (D == 128 && splits == 1 && gridDim.x > 256 && gridDim.x <= 512 &&
      paired_list_tile(blockIdx.x, qtiles, (int)(gridDim.x / (unsigned)qtiles), la.cnt, la.cap,
                       DUAL ? lb.cnt : nullptr, lb.cap, reinterpret_cast<int *>(&s_k[0][0]),
                       &s_unequal, &lst, &qt)) {
    // all blocks resident at once and lists of unequal cost: heavy blocks on CUs
    // of their own or next to light ones
    sp = 0;
    tq = lst % Tq;
    tile = lst / Tq;
  } else {
    tile = xcd_logical_tile(blockIdx.x, gridDim.x);
    qt = tile % qtiles;
    tile /= qtiles;
    sp = tile % splits;  // part of the list this block attends (DUAL: always 0 of 1)
    tile /= splits;
    tq = tile % Tq;
    tile /= Tq;
    // tile is now the head slot b * H + h; small grids visit heads in a
    // cost-balanced order (at most 64 heads, at most 1024 blocks)
    const int G = (int)(gridDim.x / ((unsigned)qtiles * splits * Tq));
    if (gridDim.x <= 1024 && G <= 64)
      tile = balanced_head(tile, G, Tq, la.cnt, la.cap, DUAL ? lb.cnt : nullptr, lb.cap, s_order);
  }
  const int h = tile % H;
  const int b = tile / H;
  const long long head = (long long)b * H + h;
  const long long list = head * Tq + tq;
  const int Tk = Nk / P;
  // runs of list A (split: its entries [e0, e1)), then (DUAL) the runs of list B after them
  int cnt_a = la.cnt[list];
  cnt_a = cnt_a < 0 ? 0 : (cnt_a > la.cap ? la.cap : cnt_a);
  const int e0 = (int)((long long)cnt_a * sp / splits);
  const int e1 = (int)((long long)cnt_a * (sp + 1) / splits);
  const int nruns_a = build_runs(la.idx + list * la.cap + e0, e1 - e0, la.cap - e0, Tk,
                                 RunList{s_lo, s_hi}, &s_nruns[0]);
  // a split writes its partial (O, LSE) to its own slice of the output
  all.o += sp * o_split_stride;
  all.lse += sp * lse_split_stride;
  int nruns = nruns_a;
  if (DUAL)
    nruns += build_runs(lb.idx + list * lb.cap, lb.cnt[list], lb.cap, Tk,
                        RunList{s_lo + nruns_a, s_hi + nruns_a}, &s_nruns[1]);

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
  float m = -INFINITY;  // running row max, scaled base-2 units
  float l = 0.f;        // running row sum (this lane's half of the keys)

  const char *kh = reinterpret_cast<const char *>(k + head * (long long)Nk * D);
  const char *vh = reinterpret_cast<const char *>(vt + head * (long long)NkC * D * 8);

  // Tile loads go straight from HBM into LDS (global_load_lds_dwordx4): each
  // wavefront instruction fills 64 consecutive 16-byte LDS units, one per
  // lane, and the lane picks the global chunk that belongs at its unit.
  // K: unit u -> slot u / NCH, stored chunk u % NCH, which holds logical chunk
  // (u % NCH) ^ (slot & SWZ) of key key_slot(slot).  V^T: unit u is the u-th
  // 16-byte chunk of the tile, contiguous in the workspace.  The per-lane byte
  // offsets are fixed; only the tile's (wave-uniform) base address changes.
  unsigned koff[KLD];
  int kkey[KLD];
#pragma unroll
  for (int it = 0; it < KLD; ++it) {
    const int u = (it * 4 + wave) * 64 + lane;
    const int slot = u / NCH, pc = u % NCH;
    kkey[it] = key_slot(slot);
    koff[it] = (unsigned)(kkey[it] * D + (pc ^ (slot & SWZ)) * 8) * 2u;
  }
  auto issue_k = [&](int n0, int bsel) {
    const char *base = kh + (long long)n0 * D * 2;
    if (n0 + kTileKeys <= Nk) {
#pragma unroll
      for (int it = 0; it < KLD; ++it)
        __builtin_amdgcn_global_load_lds(
            (const void *)(base + koff[it]),
            (__attribute__((address_space(3))) void *)&s_k[bsel][(it * 4 + wave) * 1024], 16, 0,
            0);
    } else {
      // last tile of the keys: rows past Nk repeat row Nk-1 (their scores are masked)
#pragma unroll
      for (int it = 0; it < KLD; ++it) {
        const int over = n0 + kkey[it] - (Nk - 1);
        const unsigned off = over > 0 ? koff[it] - (unsigned)(over * D * 2) : koff[it];
        __builtin_amdgcn_global_load_lds(
            (const void *)(base + off),
            (__attribute__((address_space(3))) void *)&s_k[bsel][(it * 4 + wave) * 1024], 16, 0,
            0);
      }
    }
  };
  auto issue_v = [&](int n0, int bsel) {
    const int c0 = n0 / 8;
    const char *base = vh + (long long)c0 * D * 16;
    const bool whole = c0 + kTileKeys / 8 <= NkC;
#pragma unroll
    for (int it = 0; it < VLD; ++it) {
      const int u = (it * 4 + wave) * 64 + lane;
      unsigned off = (unsigned)u * 16u;
      if (!whole) {
        const int over = c0 + u / D - (NkC - 1);
        if (over > 0) off -= (unsigned)(over * D * 16);
      }
      __builtin_amdgcn_global_load_lds(
          (const void *)(base + off),
          (__attribute__((address_space(3))) void *)&s_v[bsel][(it * 4 + wave) * 1024], 16, 0, 0);
    }
  };
  // S^T of one tile: 2 blocks of 32 keys x 32 query rows
  auto qk = [&](int bsel, f32x16 *sacc) {
    const unsigned char *kb_base = s_k[bsel];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb] = f32x16{};
      const int slot = kb * 32 + j;
      const unsigned char *krow = kb_base + slot * D * 2;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const int c = 2 * ks + g;
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(krow + ((c ^ (slot & SWZ)) * 16));
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], sacc[kb], 0, 0, 0);
      }
    }
  };

  // Tile cursor.  The loop is software-pipelined: iteration i holds S of tile
  // i (computed one iteration earlier) and issues the Q.K^T MFMAs of tile i+1
  // next to the softmax of tile i, then the P.V MFMAs of tile i.  K and V
  // each have two LDS slots, staggered: during iteration i, K of tile i+1 and
  // V of tile i are read while K of tile i+2 and V of tile i+1 stream in.
  struct Cur {
    int r, start, end, n0;
  };
  auto advance = [&](Cur c) {
    c.n0 += kTileKeys;
    if (c.n0 >= c.end) {
      ++c.r;
      if (c.r < nruns) {
        c.start = s_lo[c.r] * P;
        c.end = (s_hi[c.r] + 1) * P;
        c.n0 = c.start & ~7;
      }
    }
    return c;
  };
  Cur cur{0, 0, 0, 0};
  if (nruns > 0) {
    cur.start = s_lo[0] * P;
    cur.end = (s_hi[0] + 1) * P;
    cur.n0 = cur.start & ~7;
  }
  Cur nxt = advance(cur);
  int ks_slot = 0;  // K slot holding the tile whose S is computed next
  if (nruns > 0) {
    issue_k(cur.n0, 0);
    issue_v(cur.n0, 0);
    if (nxt.r < nruns) issue_k(nxt.n0, 1);
  }
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();

  const int g8 = 8 * g;
  f32x16 sc[2];
  if (wave_active && nruns > 0) qk(0, sc);
  // every wave has read K slot 0 before iteration 0 streams tile 2 into it
  __syncthreads();
  // O = acc / l and LSE = (m + log2 l) ln 2 of this wave's rows, written to `out`
  auto store_out = [&](OutArg out) {
    const HalfPair lp = with_other_half(l);
    const float l_tot = lp.a + lp.b;
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
    float *op = out.o + orow * D;
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
    if (g == 0) out.lse[orow] = lse_v;
  };
  int vs = 0;  // V slot of the current tile
  // One tile: scur holds S of tile i, snext receives S of tile i+1.  The loop
  // below unrolls by two and swaps the roles of the two register sets, so S
  // never has to be copied from one to the other.
  auto step = [&](f32x16 (&scur)[2], f32x16 (&snext)[2]) {
    const Cur nn = advance(nxt);  // tile i+2
    const bool has_next = nxt.r < nruns;
    if (nn.r < nruns) issue_k(nn.n0, vs);        // K slot of tile i is free now
    if (has_next) issue_v(nxt.n0, vs ^ 1);       // V slot of tile i-1 is free now
    __builtin_amdgcn_s_setprio(0);  // raised since the P.V MFMAs of the last tile

    if (wave_active) {
      // keys of this tile outside the run: only [lo_rel, hi_rel) are valid
      const int lo_rel = cur.start > cur.n0 ? cur.start - cur.n0 : 0;
      const int hi_rel = cur.end - cur.n0 < kTileKeys ? cur.end - cur.n0 : kTileKeys;
      if (lo_rel > 0 || hi_rel < kTileKeys) {
        const int lo_l = lo_rel - g8, hi_l = hi_rel - g8;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = 32 * kb + (i & 7) + 16 * (i >> 3);  // minus this lane's 8g
            if (key < lo_l || key >= hi_l) scur[kb][i] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, scur[kb][i]);
      {
        const HalfPair pr = with_other_half(mx);
        mx = fmaxf(pr.a, pr.b) * scale_log2;
      }
      // rescale only when some row of the wavefront found a new max
      if (__builtin_amdgcn_ballot_w64(mx > m) != 0) {
        const float m_new = fmaxf(m, mx);
        const float alpha = __builtin_amdgcn_exp2f(m - m_new);  // 0 on the first tile
        l *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) acc[db] *= alpha;
        m = m_new;
      }
      // Q.K^T of the next tile (on a stale slot after the last tile: unused)
      qk(ks_slot ^ 1, snext);
      f16x8 pf[4];
      float psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = __builtin_amdgcn_exp2f(fmaf(scur[kb][i], scale_log2, -m));
          psum += p;
          pf[2 * kb + (i >> 3)][i & 7] = (_Float16)p;
        }
      l += psum;
      const unsigned char *vb_base = s_v[vs];
      // Wave priority: the two wavefronts of a SIMD interleave a VALU-heavy
      // softmax and MFMA streams.  Issuing first from the wavefront that is in
      // its P.V MFMAs, its tile-end wait and its next DMA issue keeps the
      // matrix core fed while the other one runs its softmax (measured +3.5 %
      // on the 42-frame LVSA step; raising Q.K^T as well loses 5 %).
      __builtin_amdgcn_s_setprio(1);
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
    ks_slot ^= 1;
    vs ^= 1;
    cur = nxt;
    nxt = nn;
  };
  f32x16 sd[2];
  // DUAL: once the cursor has left the runs of list A, the state holds exactly
  // the tiles of A (the next tile's S is computed but not yet accumulated)
  bool a_done = !DUAL;
  auto after_tile = [&]() {
    if (DUAL && !a_done && cur.r >= nruns_a) {
      if (wave_active) store_out(first);
      a_done = true;
    }
  };
  after_tile();
  while (cur.r < nruns) {
    step(sc, sd);
    after_tile();
    if (cur.r >= nruns) break;
    step(sd, sc);
    after_tile();
  }
  if (wave_active) store_out(all);
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
  FSA_REQUIRE(heads < 65536, FSA_E_SHAPE, "B*H=%lld exceeds 65535", heads);
  const dim3 grid((unsigned)((Nk + 63) / 64), (unsigned)heads);
  auto vv = static_cast<const uint16_t *>(v);
  auto out = static_cast<_Float16 *>(prepared);
  if (D == 64)
    hipLaunchKernelGGL(v_to_f16_chunked_kernel<64>, grid, dim3(256), 0, stream, vv, out, Nk, NkC);
  else
    hipLaunchKernelGGL(v_to_f16_chunked_kernel<128>, grid, dim3(256), 0, stream, vv, out, Nk, NkC);
  return check_launch("prepare_values");
}

fsa_status launch_attn_bf16_prepared(const void *q, const void *k, const void *prepared,
                                     const int32_t *idx, const int32_t *cnt, int cap,
                                     const int32_t *idx_b, const int32_t *cnt_b, int cap_b,
                                     int B, int H, int Nq, int Nk, int D, int P, float scale,
                                     float *o_first, float *lse_first, float *o, float *lse,
                                     int splits, hipStream_t stream) {
  const long long heads = (long long)B * H;
  const int NkC = (Nk + 7) / 8;
  const int Tq = Nq / P;
  const int qtiles = (P + kRows - 1) / kRows;
  const long long blocks = heads * Tq * qtiles * splits;
  const long long o_stride = heads * Nq * D, lse_stride = heads * Nq;
  FSA_REQUIRE(blocks < (1LL << 31), FSA_E_SHAPE, "too many query tiles (%lld)", blocks);
  const float scale_log2 = scale * kLog2e;
  auto qq = static_cast<const uint16_t *>(q);
  auto kk = static_cast<const uint16_t *>(k);
  auto vt = static_cast<const _Float16 *>(prepared);
  const ListArg la{idx, cnt, cap}, lb{idx_b, cnt_b, cap_b};
  const OutArg first{o_first, lse_first}, all{o, lse};
  const bool dual = idx_b != nullptr;
  const dim3 grid((unsigned)blocks), block(kThreads);
  if (D == 64) {
    if (dual)
      hipLaunchKernelGGL((attn_bf16_kernel<64, true>), grid, block, 0, stream, qq, kk, vt, la, lb,
                         H, Nq, Nk, NkC, P, Tq, qtiles, scale_log2, first, all, splits, o_stride,
                         lse_stride);
    else
      hipLaunchKernelGGL((attn_bf16_kernel<64, false>), grid, block, 0, stream, qq, kk, vt, la,
                         lb, H, Nq, Nk, NkC, P, Tq, qtiles, scale_log2, first, all, splits, o_stride,
                         lse_stride);
  } else {
    if (dual)
      hipLaunchKernelGGL((attn_bf16_kernel<128, true>), grid, block, 0, stream, qq, kk, vt, la,
                         lb, H, Nq, Nk, NkC, P, Tq, qtiles, scale_log2, first, all, splits, o_stride,
                         lse_stride);
    else
      hipLaunchKernelGGL((attn_bf16_kernel<128, false>), grid, block, 0, stream, qq, kk, vt, la,
                         lb, H, Nq, Nk, NkC, P, Tq, qtiles, scale_log2, first, all, splits, o_stride,
                         lse_stride);
  }
  return check_launch(dual ? "sparse_frame_attn_dual (bf16)" : "sparse_frame_attn (bf16)");
}

}  // namespace fsa
