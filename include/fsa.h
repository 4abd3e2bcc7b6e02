/*
 * fsa.h -- C ABI of libfsa: frame-block-sparse softmax attention for video
 * diffusion transformers on AMD Instinct MI355X (gfx950).
 *
 * Each query frame t of each head attends only to a set A(t) of key/value
 * frames.  The library builds those sets, picks frames by pooled scores,
 * computes the attention with its log-sum-exp (LSE), and merges partial
 * results over disjoint frame sets.
 *
 * Common conventions
 * ------------------
 *  - Every function returns fsa_status; FSA_OK is 0.  On any other status,
 *    fsa_last_error() returns a message for the calling thread.
 *  - Tensors are dense, contiguous, row-major.  q is [B][H][Nq][D]; k and v
 *    are [B][H][Nk][D].  Token n of frame f is n = f*P + p (frame-major, P
 *    tokens per frame), so Nq = Tq*P and Nk = Tk*P.
 *  - Frame sets are idx [B][H][Tq][cap] int32 plus cnt [B][H][Tq] int32:
 *    A(t) = idx[b][h][t][0 .. cnt-1], sorted ascending, no duplicates, every
 *    entry in [0, Tk).  Entries past cnt are -1 when the library writes them
 *    and ignored when it reads them.
 *  - The caller owns every buffer.  The library never allocates or frees
 *    device or host memory; scratch space comes in through explicit workspace
 *    arguments.  It keeps no state beyond the thread-local error text, except
 *    for the one allocation-free entry point below
 *    (fsa_select_topk_frames_noalloc), whose scratch is a static device array
 *    per GPU.
 *  - "device" functions only validate their host arguments, enqueue kernels
 *    on `stream` (a hipStream_t; NULL = the default stream) and return; the
 *    results are ready when the stream reaches that point.  Launch failures
 *    return FSA_E_HIP.  "host" functions are synchronous and touch host
 *    memory only; they need no GPU.
 *  - Device kernels never read or write outside the buffers described here,
 *    even for malformed frame lists: list entries outside [0, Tk) are
 *    skipped and cnt is clamped to [0, cap].  Unsorted or duplicated lists
 *    give unspecified (but memory-safe) results; fsa_validate_frame_sets
 *    checks a host copy.
 *
 * Sources.  The operations follow these pages (gist.science technical
 * summaries):
 *  [LVSA]   LVSA, training-free sparse attention for long video diffusion:
 *           §2 core mechanism (A(t) = G ∪ W(t), rotating anchors, widened
 *           window, budget C) and its complexity paragraph.
 *  [LF]     Light Forcing: §2.1 chunk-aware growth of the sparsity ratio;
 *           §2.2 hierarchical sparse attention (mean-pooled
 *           queries/keys, frame selection per query block, block selection
 *           inside the chosen frames, attention over the selected pairs
 *           only).
 *  [ISPA]   ISPA, instance-specific parametric absorption: §2 item 1
 *           dual-stream warmup and decomposable attention merged through LSE;
 *           §3 item 2.
 *  [HF]     Head Forcing: methodology §2, per-head KV sets (local, anchor,
 *           memory with fast memory of recent frames); §3 per-head RoPE
 *           re-encoding of the assembled cache.
 *  [ARL2]   ARL2: §2.1 item 1, bidirectional softmax inside each frame
 *           (the special case A(t) = {t}).
 */
#ifndef FSA_H_
#define FSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FSA_ABI_VERSION 1

/* Largest number of heads one policy array may describe. */
#define FSA_MAX_HEADS 64
/* Largest frame-set capacity (entries per list) the kernels accept. */
#define FSA_MAX_CAP 1024

typedef enum fsa_status {
  FSA_OK = 0,
  FSA_E_ARG = 1,      /* null pointer, negative size, bad scalar argument      */
  FSA_E_SHAPE = 2,    /* sizes inconsistent (N not a multiple of P, D, ...)    */
  FSA_E_DTYPE = 3,    /* unsupported dtype / head_dim combination              */
  FSA_E_CAPACITY = 4, /* cap or workspace too small for what is asked          */
  FSA_E_LIST = 5,     /* a frame list is unsorted, duplicated or out of range  */
  FSA_E_HIP = 6       /* the HIP runtime reported an error                     */
} fsa_status;

typedef enum fsa_dtype {
  FSA_F32 = 0,  /* float32 inputs; computed in float32 end to end             */
  FSA_BF16 = 1  /* bfloat16 inputs; MFMA with float32 accumulation            */
} fsa_dtype;

/* Frame-set policy of one head (fields a policy does not use are ignored). */
typedef enum fsa_policy_kind {
  FSA_POL_FULL = 0,        /* every KV frame: dense attention                   */
  FSA_POL_LVSA = 1,        /* [LVSA] anchors G_s ∪ window widened to budget     */
  FSA_POL_SINK_WINDOW = 2, /* [HF] local / anchor heads, [ISPA] local stream    */
  FSA_POL_MEMORY = 3,      /* [HF] memory heads: selected frames ∪ recent       */
  FSA_POL_RANGE = 4        /* frames lo..hi (e.g. [ISPA] history branch)        */
} fsa_policy_kind;

typedef struct fsa_head_policy {
  int32_t kind;      /* fsa_policy_kind                                          */
  int32_t n_sink;    /* SINK_WINDOW: frames 0..n_sink-1 are always kept          */
  int32_t window;    /* LVSA: base window W; SINK_WINDOW: frames ending at e     */
  int32_t budget;    /* LVSA: target |A(t)| = C                                  */
  int32_t t_per;     /* LVSA: anchor period T_per (>= 1)                         */
  int32_t step;      /* LVSA: denoising step s (anchors f with f%T_per == s%T_per)*/
  int32_t topk;      /* MEMORY: selected frames per query group                  */
  int32_t n_recent;  /* MEMORY: recent frames e-n_recent+1..e (fast memory)      */
  int32_t lo, hi;    /* RANGE: inclusive frame range                             */
} fsa_head_policy;

/* ABI version the library was built with (FSA_ABI_VERSION). */
int32_t fsa_abi_version(void);

/* Message for the last non-OK status returned on this thread ("" if none).
 * The pointer stays valid until the next library call on this thread. */
const char *fsa_last_error(void);

/* ------------------------------------------------------------------------
 * Frame sets  [LVSA §2 core mechanism; HF methodology §2; ISPA §2 item 1]
 *
 * Query frame tq sits at KV frame offset+tq.  In chunked (autoregressive)
 * mode `chunk` consecutive query frames form one chunk; the chunk's last KV
 * frame is e = offset + (tq/chunk + 1)*chunk - 1, and all its frames share one
 * set.  Per policy:
 *   FULL         A = {0 .. Tk-1}.
 *   LVSA         with T = Tk, t = offset+tq, r = step mod t_per:
 *                G = {f : f mod t_per == r}; frames ordered by (|f-t|, f);
 *                take the first k = min(window, T) of them and keep adding the
 *                next one while |G ∪ first-k| < min(budget, T); A = G ∪ first-k.
 *                (The window never shrinks below W and anchors are never
 *                dropped, so A may exceed the budget when G ∪ W already does.)
 *   SINK_WINDOW  A = {0..n_sink-1} ∪ {max(0, e-window+1) .. e}.
 *   MEMORY       A = (topk selected frames of tq's group) ∪ {e-n_recent+1..e}.
 *   RANGE        A = {max(0,lo) .. min(hi, Tk-1)}.
 * ---------------------------------------------------------------------- */

/* host.  Smallest cap that holds every set the policies can produce
 * (an upper bound for LVSA/MEMORY, exact for the others). */
fsa_status fsa_frame_set_capacity(int32_t H, const fsa_head_policy *policies /* host [H] */,
                                  int32_t Tq, int32_t Tk, int32_t offset, int32_t chunk,
                                  int32_t *cap_out /* host, 1 */);

/* device.  Build idx/cnt for every (b, h, tq).
 *   policies   host [H] (copied into the launch; H <= FSA_MAX_HEADS)
 *   selected   device [B][H][Tq/chunk][topk_k] int32, the frames picked for
 *              each query group (read for MEMORY heads only; may be NULL if no
 *              head is MEMORY); entries outside [0,Tk) are skipped
 *   idx        device [B][H][Tq][cap] int32 out (padded with -1)
 *   cnt        device [B][H][Tq] int32 out
 * Errors: FSA_E_ARG (bad sizes, Tq % chunk != 0, unknown kind, t_per < 1,
 * budget/window < 0, MEMORY head without `selected`), FSA_E_CAPACITY (cap
 * below fsa_frame_set_capacity or above FSA_MAX_CAP), FSA_E_HIP. */
fsa_status fsa_build_frame_sets(int32_t B, int32_t H, int32_t Tq, int32_t Tk, int32_t offset,
                                int32_t chunk, const fsa_head_policy *policies,
                                const int32_t *selected, int32_t topk_k, int32_t cap,
                                int32_t *idx, int32_t *cnt, void *stream);

/* host.  The same construction on host buffers (selected, idx, cnt are host
 * pointers).  Provided for callers that build lists on the CPU; the device
 * path above does not use it. */
fsa_status fsa_build_frame_sets_host(int32_t B, int32_t H, int32_t Tq, int32_t Tk,
                                     int32_t offset, int32_t chunk,
                                     const fsa_head_policy *policies, const int32_t *selected,
                                     int32_t topk_k, int32_t cap, int32_t *idx, int32_t *cnt);

/* host.  FSA_OK iff every list of a host copy of idx/cnt is sorted, unique,
 * within [0, Tk) and 0 <= cnt <= cap; else FSA_E_LIST naming the first bad
 * (b, h, t). */
fsa_status fsa_validate_frame_sets(int32_t B, int32_t H, int32_t Tq, int32_t Tk, int32_t cap,
                                   const int32_t *idx, const int32_t *cnt);

/* ------------------------------------------------------------------------
 * Frame selection  [LF §2.2 token compression + frame selection; HF §2
 * memory heads]
 *
 * For each batch b, head h in [h_begin, h_end) and query group g (query
 * frames g*q_group .. g*q_group+q_group-1):
 *   qf[t,d]   = sum of q over query frame t's P tokens, float64, added one
 *               token at a time in ascending order (frame-level compression);
 *   qsum[d]   = sum of qf over the group's frames, added in frame order;
 *   ksum[f,d] = sum of k over frame f's P tokens, float64, ascending p;
 *   score[f]  = sum over d of (qsum[d]*ksum[f,d]), each product rounded to
 *               float64 then added in ascending d (no fused multiply-add);
 * for candidate frames f in [cand_begin, cand_end).  Frames are ranked by
 * (score descending, f ascending) and the first topk_k are written in
 * ascending order.  Sums stand in for means (same ranking, no division).
 * Every operation has a fixed order, so the result is bit-reproducible.
 *   q, k        device, dtype dt, [B][H][Nq][D] and [B][H][Nk][D]
 *   out_frames  device [B][H][Nq/(q_group*P)][topk_k] int32 (heads outside
 *               [h_begin,h_end) untouched)
 *   out_scores  device [B][H][G][cand_end-cand_begin] float64, or NULL
 *   workspace   device, >= fsa_select_topk_workspace_size() bytes
 * Errors: FSA_E_ARG (topk_k < 1 or > 64, topk_k > number of candidates,
 * candidates outside [0, Tk) or more than 4096 of them, q_group does not
 * divide Tq, bad head range), FSA_E_SHAPE (D outside [1, 256], ...),
 * FSA_E_DTYPE, FSA_E_CAPACITY (workspace), FSA_E_HIP.
 * Non-finite inputs give unspecified frames (a precondition); a NaN score
 * ranks below every number, so each row still receives exactly topk_k
 * distinct candidate frames and nothing outside out_frames is written. */
fsa_status fsa_select_topk_workspace_size(int32_t B, int32_t H, int32_t Nq, int32_t D,
                                          int32_t P, int32_t q_group, int32_t cand_begin,
                                          int32_t cand_end, size_t *bytes);
fsa_status fsa_select_topk_frames(const void *q, const void *k, int32_t dt, int32_t B,
                                  int32_t H, int32_t Nq, int32_t Nk, int32_t D, int32_t P,
                                  int32_t h_begin, int32_t h_end, int32_t q_group,
                                  int32_t cand_begin, int32_t cand_end, int32_t topk_k,
                                  int32_t *out_frames, double *out_scores, void *workspace,
                                  size_t workspace_bytes, void *stream);

/* device.  fsa_select_topk_frames without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).  The pooled sums live in a
 * static device array of FSA_NOALLOC_SCRATCH_BYTES bytes that the library
 * holds on each GPU it runs on until the process ends; the call itself
 * allocates and frees nothing.  The array of the current device is used, so
 * call it with the device of `stream` current.  Every call on a GPU shares
 * that GPU's array: calls that overlap on one GPU (concurrent streams, or
 * threads) race and give undefined frames; calls ordered on one stream are
 * safe.  The kernels write every scratch byte they read, so nothing needs to
 * start at zero.  Arguments, results and errors as fsa_select_topk_frames,
 * plus FSA_E_CAPACITY when the pooled sums, B * (h_end - h_begin) *
 * (Nq/P + cand_end - cand_begin) * D * 8 bytes, exceed the array (checked
 * before anything is launched), and FSA_E_HIP when the array's device
 * address cannot be resolved. */
#define FSA_NOALLOC_SCRATCH_BYTES (16u << 20)
fsa_status fsa_select_topk_frames_noalloc(const void *q, const void *k, int32_t dt, int32_t B,
                                          int32_t H, int32_t Nq, int32_t Nk, int32_t D,
                                          int32_t P, int32_t h_begin, int32_t h_end,
                                          int32_t q_group, int32_t cand_begin,
                                          int32_t cand_end, int32_t topk_k,
                                          int32_t *out_frames, double *out_scores,
                                          void *stream);

/* ------------------------------------------------------------------------
 * Chunk-aware growth of the sparsity ratio  [LF §2.1: first chunk dense,
 * later chunks sparser, s_i = s_base - alpha_i * beta with alpha_i following
 * the noise level as 1/sqrt, beta matching the total FLOPs to a target]
 *
 * host, synchronous.  For chunks i = 0..n_chunks-1 with dense attention cost
 * cost[i] > 0:
 *   s_0 = 0;  s_i = clip(s_base - beta / sqrt(i + 1), 0, s_max)  (i >= 1)
 *   beta: the upper end of a fixed float64 bisection (at most 200 halvings)
 *         of a bracket clipping every s_i at s_max at one end and at 0 at the
 *         other, with sum_i (1 - s_i) cost[i] >= (1 - s_target) sum_i cost[i]
 *         (sums in ascending i, no fused multiply-add)
 *   budgets[i] = floor((1 - s_i) * candidates[i] + 1/2) clipped to
 *         [1, candidates[i]]: frames (or blocks) kept by chunk i
 *   sparsity    host double [n_chunks] out
 *   candidates  host int32 [n_chunks], needed only with budgets
 *   budgets     host int32 [n_chunks] out, or NULL
 *   beta_out    host double out, or NULL
 * Errors: FSA_E_ARG (n_chunks < 1; null pointer; s_target or s_max outside
 * [0, 1), s_base outside [0, 1]; a cost not positive and finite; a
 * candidate count < 1; a target that no beta reaches). */
fsa_status fsa_cag_schedule(int32_t n_chunks, const double *cost, double s_target, double s_base,
                            double s_max, const int32_t *candidates, double *sparsity,
                            int32_t *budgets, double *beta_out);

/* ------------------------------------------------------------------------
 * Two-level (frame, then block) selection  [LF §2.2 hierarchical sparse
 * attention: token compression to block and frame granularity, frame
 * selection per query block with frame-level keys, block selection inside the
 * chosen frames with block-level keys; Head Forcing methodology §2 for the
 * recent frames kept whole]
 *
 * device.  Writes block-unit lists for heads [h_begin, h_end): a block is
 * `block` consecutive tokens of a frame (P % block == 0, nb = P / block), and
 * block index g = frame * nb + block-in-frame.  For query block j (tokens
 * [j*block, (j+1)*block), query frame tq = j / nb, whose chunk ends at KV
 * frame e = q_kv_offset + (tq / chunk + 1) * chunk - 1):
 *   qs      = sum of the block's query tokens (float64, ascending tokens)
 *   kblk[g] = sum of key block g's tokens (float64, ascending tokens)
 *   kfr[f]  = sum of frame f's nb block sums (float64, ascending blocks)
 *   level 1: the topk_frames best frames f in [0, e - n_recent] by
 *            qs . kfr[f] (rounded products added in ascending channel order),
 *            ties to the lower frame
 *   level 2: the topk_blocks best blocks of those frames by qs . kblk[g],
 *            ties to the lower block
 *   idx row = the chosen blocks ascending, then every block of the frames
 *            e - n_recent + 1 .. e ascending; cnt = topk_blocks + n_recent*nb;
 *            the rest of the row is -1.
 * Rows of heads outside [h_begin, h_end) are not touched, so other heads'
 * block-unit lists can come from fsa_build_frame_sets with every frame size
 * and count multiplied by nb.  Attend with P = block.
 *   q, k        device [B][H][Nq][D] / [B][H][Nk][D], float32 or bfloat16
 *   idx, cnt    device int32 [B][H][Nq/block][cap] / [B][H][Nq/block] out
 *   workspace   device, >= fsa_select_hsa_workspace_size() bytes
 * Errors: FSA_E_ARG (bad head range; the last chunk ends past the cache;
 * recent frames before frame 0; topk_frames outside [1, candidates of the
 * first chunk]; topk_frames * nb > 4096; topk_blocks outside
 * [0, topk_frames * nb]; more than 4096 candidate frames), FSA_E_SHAPE (D
 * outside [1, 256]; P not a multiple of block; Nq or Nk not a multiple of P),
 * FSA_E_DTYPE, FSA_E_CAPACITY (cap below topk_blocks + n_recent*nb or above
 * FSA_MAX_CAP; workspace), FSA_E_HIP.  Non-finite inputs give unspecified
 * blocks (a precondition); a NaN score ranks below every number, so each row
 * still holds exactly topk_blocks chosen blocks and nothing past its cap is
 * written. */
fsa_status fsa_select_hsa_workspace_size(int32_t B, int32_t H, int32_t Nq, int32_t Nk, int32_t D,
                                         int32_t P, int32_t block, int32_t q_kv_offset,
                                         int32_t chunk, int32_t h_begin, int32_t h_end,
                                         int32_t n_recent, size_t *bytes);
fsa_status fsa_select_hsa_blocks(const void *q, const void *k, int32_t dt, int32_t B, int32_t H,
                                 int32_t Nq, int32_t Nk, int32_t D, int32_t P, int32_t block,
                                 int32_t q_kv_offset, int32_t chunk, int32_t h_begin,
                                 int32_t h_end, int32_t n_recent, int32_t topk_frames,
                                 int32_t topk_blocks, int32_t cap, int32_t *idx, int32_t *cnt,
                                 void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Per-head frame-level RoPE re-encoding  [HF §3: keys cached with the spatial
 * rotary encoding only; frame-level positions encoded again per head when
 * its cache is assembled, keeping query-key relative positions in range]
 *
 * device.  For each (b, h) with its sorted, duplicate-free frame set
 * A = idx[b][h][0..cnt[b][h]) (frames outside [0, Tk) are skipped):
 *   key rows of frame A[r]            turn by position r
 *   query rows of query frame tq      turn by #{f in A : f < q_kv_offset + tq}
 * Turning by position p: channel pair (2i, 2i+1), i < rot/2, becomes
 *   (x0 c - x1 s, x0 s + x1 c),  c, s = cos, sin(p * base^(-2i/rot)),
 * in float64 without fused multiply-add, rounded once to the storage type
 * (nearest, ties to even); channels >= rot are copied unchanged.
 *   q, k          device [B][H][Nq][D] / [B][H][Nk][D] (dt: FSA_F32/FSA_BF16)
 *   idx, cnt      device int32 [B][H][cap] / [B][H]: one frame set per head
 *                 (e.g. the set shared by a chunk's query frames)
 *   q_out         device [B][H][Nq][D]: every row written (may alias q)
 *   k_out         device [B][H][Nk][D]: only rows of listed frames written
 *                 (may alias k); attend to k_out with the same set
 * Requires 16-byte aligned q, k, q_out, k_out.
 * Errors: FSA_E_ARG (rot odd or outside [0, D]; base not positive and
 * finite; negative offset; null or misaligned pointer), FSA_E_SHAPE (D not a
 * multiple of 8 in [8, 256]; Nq or Nk not a multiple of P), FSA_E_DTYPE,
 * FSA_E_CAPACITY (cap outside [1, FSA_MAX_CAP]), FSA_E_HIP. */
fsa_status fsa_rope_reencode(const void *q, const void *k, int32_t dt, int32_t B, int32_t H,
                             int32_t Nq, int32_t Nk, int32_t D, int32_t P, const int32_t *idx,
                             const int32_t *cnt, int32_t cap, int32_t q_kv_offset, int32_t rot,
                             double base, void *q_out, void *k_out, void *stream);

/* ------------------------------------------------------------------------
 * Sparse frame attention  [LVSA §2 core mechanism and complexity; LF §2.2
 * execution over the selected frames; ISPA §2 item 1 (LSE output)]
 *
 * For every (b, h) and query token i of frame t = i / P:
 *   S_ij  = scale * q_i . k_j   for keys j with j/P in A(t)
 *   LSE_i = ln sum_j exp(S_ij)  (natural log)
 *   O_i   = sum_j exp(S_ij - LSE_i) v_j
 * An empty A(t) gives O_i = 0 and LSE_i = -inf.
 *   scale      <= 0 selects 1/sqrt(D)
 *   o          device [B][H][Nq][D] float32 out
 *   lse        device [B][H][Nq] float32 out
 *   workspace  device, >= fsa_sparse_frame_attn_workspace_size() bytes
 *              (bf16: a float16, key-chunked transposed copy of v)
 * Precision: dt = FSA_F32 computes in float32 throughout.  dt = FSA_BF16
 * forms Q.K^T with bf16 MFMA (float32 accumulation), keeps the softmax and
 * its row sums in float32, and forms P.V with float16 MFMA on float16
 * probabilities and float16 values (float32 accumulation); O and LSE are
 * float32.
 * Value range (bf16 path): values are used as float16, so attended values
 * must satisfy |v| <= 65504 (a precondition); larger finite values and
 * infinities are saturated to +-65504 when the float16 copy is made, so a
 * large value in a frame a row does not attend never reaches that row's
 * output.  NaN values stay NaN and may spread to rows whose 64-key tiles
 * hold them.
 * Supported: D in {64, 128}; P >= 1; Nq % P == 0; Nk % P == 0.  The bf16
 * path reads and writes 16 bytes at a time: q, k, v, o and the workspace must
 * be 16-byte aligned (FSA_E_ARG otherwise).
 * Errors: FSA_E_ARG, FSA_E_SHAPE, FSA_E_DTYPE, FSA_E_CAPACITY, FSA_E_HIP. */
fsa_status fsa_sparse_frame_attn_workspace_size(int32_t dt, int32_t B, int32_t H, int32_t Nk,
                                                int32_t D, size_t *bytes);
fsa_status fsa_sparse_frame_attn(const void *q, const void *k, const void *v, int32_t dt,
                                 int32_t B, int32_t H, int32_t Nq, int32_t Nk, int32_t D,
                                 int32_t P, const int32_t *idx, const int32_t *cnt, int32_t cap,
                                 float scale, float *o, float *lse, void *workspace,
                                 size_t workspace_bytes, void *stream);

/* device.  The two halves of fsa_sparse_frame_attn, for callers that reuse
 * the same values across calls (an autoregressive KV cache attended by every
 * denoising step and by several branches):
 *   fsa_prepare_values           bf16 only: writes the float16, key-chunked
 *                                transposed copy of v into `prepared`
 *                                (>= fsa_sparse_frame_attn_workspace_size
 *                                bytes, layout [B*H][ceil(Nk/8)][D][8]; keys
 *                                past Nk are zero; values beyond +-65504
 *                                saturate, as above).
 *   fsa_sparse_frame_attn_prepared  the attention itself, reading that copy
 *                                instead of v.
 * fsa_sparse_frame_attn(v, workspace) equals prepare(v -> workspace)
 * followed by prepared(workspace).  Errors as above; FSA_E_DTYPE for
 * dt != FSA_BF16. */
fsa_status fsa_prepare_values(const void *v, int32_t dt, int32_t B, int32_t H, int32_t Nk,
                              int32_t D, void *prepared, size_t prepared_bytes, void *stream);
fsa_status fsa_sparse_frame_attn_prepared(const void *q, const void *k, const void *prepared,
                                          int32_t dt, int32_t B, int32_t H, int32_t Nq,
                                          int32_t Nk, int32_t D, int32_t P, const int32_t *idx,
                                          const int32_t *cnt, int32_t cap, float scale,
                                          float *o, float *lse, size_t prepared_bytes,
                                          void *stream);

/* device.  fsa_sparse_frame_attn_prepared with every frame list cut into
 * `splits` parts of consecutive entries (part s holds entries
 * [s*cnt/splits, (s+1)*cnt/splits)); each part is attended by its own blocks
 * and the partial (O, LSE) are merged exactly through their log-sum-exp
 * (the merge of fsa_merge_lse, over all parts in ascending order).  For grids
 * with few query tiles (short autoregressive chunks) this spreads a long list
 * over more compute units.  splits = 1 is fsa_sparse_frame_attn_prepared.
 *   fsa_attn_split_plan: the split count (splits_req >= 1 is taken as given;
 *                        <= 0 picks one from the grid size: 1 when the grid
 *                        holds >= 256 blocks of 128 query rows, else enough
 *                        parts for about 512 blocks, at most 8) and the
 *                        workspace it needs, splits * B*H*Nq * (D + 1) floats
 *                        (0 for one part)
 *   workspace          device, >= that many bytes, 16-byte aligned (partials)
 * Errors: as fsa_sparse_frame_attn_prepared; FSA_E_ARG (splits outside
 * [1, 16]; workspace NULL), FSA_E_CAPACITY (workspace too small). */
fsa_status fsa_attn_split_plan(int32_t B, int32_t H, int32_t Nq, int32_t D, int32_t P,
                               int32_t splits_req, int32_t *splits, size_t *workspace_bytes);
fsa_status fsa_sparse_frame_attn_prepared_split(const void *q, const void *k, const void *prepared,
                                                int32_t dt, int32_t B, int32_t H, int32_t Nq,
                                                int32_t Nk, int32_t D, int32_t P,
                                                const int32_t *idx, const int32_t *cnt,
                                                int32_t cap, float scale, int32_t splits,
                                                float *o, float *lse, size_t prepared_bytes,
                                                void *workspace, size_t workspace_bytes,
                                                void *stream);

/* device.  Single-pass decomposable attention [ISPA §2 item 1: the local
 * stream (current frames + sink) and the full-history stream are both
 * collected in one forward pass with negligible extra FLOPs, through the LSE
 * state].  For every query row of frame t, with A = A_a(t) and B = A_b(t)
 * (two frame lists, disjoint for an exact union):
 *   (o_a,  lse_a)  = attention over the frames of A            (local branch)
 *   (o_ab, lse_ab) = attention over the frames of A and B      (full branch)
 * The kernel walks the runs of A, writes its running state to (o_a, lse_a),
 * and continues over the runs of B from that same state, so the union costs
 * one pass over the keys; overlapping lists count shared frames twice.
 * bf16 only, values from fsa_prepare_values; cap_a + cap_b <= FSA_MAX_CAP.
 * Shapes, precision, alignment and errors as fsa_sparse_frame_attn_prepared. */
fsa_status fsa_sparse_frame_attn_dual_prepared(
    const void *q, const void *k, const void *prepared, int32_t dt, int32_t B, int32_t H,
    int32_t Nq, int32_t Nk, int32_t D, int32_t P, const int32_t *idx_a, const int32_t *cnt_a,
    int32_t cap_a, const int32_t *idx_b, const int32_t *cnt_b, int32_t cap_b, float scale,
    float *o_a, float *lse_a, float *o_ab, float *lse_ab, size_t prepared_bytes, void *stream);

/* ------------------------------------------------------------------------
 * LSE merge  [ISPA §2 item 1, §3 item 2]
 *
 * For each of `rows` rows, with partials (o1, lse1) and (o2, lse2) over
 * disjoint key sets:
 *   M = max(lse1, lse2);  L = M + ln(exp(lse1-M) + exp(lse2-M));
 *   O = exp(lse1-L)*o1 + exp(lse2-L)*o2.
 * A partial with LSE = -inf contributes nothing; both -inf gives O = 0,
 * L = -inf.  Exact only for disjoint key sets (the caller's duty).
 *   o1, o2, o   device [rows][D] float32;  lse1, lse2, lse  device [rows]
 *   o may alias o1 or o2 and lse may alias lse1 or lse2 (in-place merge).
 * Errors: FSA_E_ARG (null pointer, rows < 0, D < 1), FSA_E_HIP. */
fsa_status fsa_merge_lse(const float *o1, const float *lse1, const float *o2,
                         const float *lse2, int64_t rows, int32_t D, float *o, float *lse,
                         void *stream);

#ifdef __cplusplus
}
#endif

#endif /* FSA_H_ */
