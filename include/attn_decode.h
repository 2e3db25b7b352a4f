/*
 * attn_decode.h - C ABI of the MI355X (gfx950) paged-KV decode-attention
 * library libattn_decode.so.
 *
 * What it computes.  For every query row r = (b, t, h) of a decode step with
 * q_len = T query tokens per sequence, the scaled dot-product softmax
 * attention over the keys of sequence b that the row sees:
 *
 *     s_i = scale * <q'_r, k_i>,   p = softmax(s),   o_r = sum_i p_i v_i,
 *     lse_r = ln sum_i exp(s_i)            (natural log, scale included)
 *
 * Key i of a sequence of length L sits at position i; query t sits at
 * position L - T + t; with causal masking (T > 1, speculative verification,
 * "Hardware-Efficient Attention for Fast Decoding", "If this is right") row
 * t sees keys i <= L - T + t, otherwise all L keys.  Query head h uses group
 * j = floor(h / g), g = h_q / groups (grouped-query attention as summarised
 * on "The Gist Talk" podcast page).  The three variants differ in what the
 * cache holds per token and how k, v and q' are formed
 * ("Hardware-Efficient Attention for Fast Decoding", "What carries the
 * argument", "Core claim", Figure 2 caption):
 *
 *   GQA    : k = K[j], v = V[j], q' = q                       (separate K, V)
 *   GTA    : k = [S[j][0 : d-d_r] || RoPE(R, i)], v = S[j],
 *            q' = [q[0 : d-d_r] || RoPE(q[d-d_r : d], L-T+t)] (tied state S,
 *            one RoPE head R broadcast to every group)
 *   latent : k = [C[j] || R], v = C[j], q' = q                (MLA: 1 latent
 *            head; GLA: h_c heads; q is the weight-absorbed query whose last
 *            d_r entries are already rotated; output is d_c wide)
 *
 * RoPE pairs element k with element k + d_r/2 and rotates the pair by the
 * angle pos * theta^(-2k/d_r).
 *
 * Method.  Split-KV decoding: a host-side plan cuts every sequence into
 * chunks (work items); one kernel computes, per item, the online-softmax
 * attention over its chunk; a second kernel merges the chunks of a sequence
 * through their softmax denominators (the decomposition noted for Hydragen
 * on the "Efficient Inference" tag page).
 *
 * Memory and ownership.  Every pointer passed to a decode call is DEVICE
 * memory owned by the caller (except where marked host).  The library never
 * allocates, frees or synchronises; all GPU work is enqueued on the given
 * stream and ATTN_OK means "enqueued".  Arguments are validated on the host
 * before anything is enqueued; a negative status means nothing was launched.
 * The library keeps no state and is reentrant.
 */
#ifndef ATTN_DECODE_H
#define ATTN_DECODE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = -1, /* null pointer, bad size, inconsistent shapes     */
  ATTN_ERR_UNSUPPORTED = -2, /* valid but not compiled in (head dims, dtype...)  */
  ATTN_ERR_WORKSPACE = -3,   /* workspace / plan buffer too small               */
  ATTN_ERR_HIP = -4          /* a HIP launch reported an error                  */
} attn_status_t;

typedef enum { ATTN_FP32 = 0, ATTN_BF16 = 1 } attn_dtype_t;

typedef enum { ATTN_KIND_GQA = 0, ATTN_KIND_GTA = 1, ATTN_KIND_LATENT = 2 } attn_kind_t;

/* Bits of the `flags` argument of the decode calls. */
enum {
  ATTN_CAUSAL = 1,      /* q_len > 1: row t sees keys i <= L - q_len + t           */
  ATTN_DEFER_MERGE = 2  /* leave split partials in the workspace (plan->counters
                           is not used); the caller runs attn_decode_merge (same
                           stream) to finish the output                           */
};

/*
 * Paged KV cache descriptor ("Hardware-Efficient Attention for Fast
 * Decoding", "If this is right": paged KV with a per-sequence page table).
 *
 * Logical token i of sequence b lives in physical page
 * page_table[b * max_pages_per_seq + i / page_size], slot i % page_size.
 * Element (page, slot, head, e) of pool0/pool1 is at
 *     page * page_stride + slot * token_stride + head * head_stride + e
 * and of rope_pool at the rope_* strides (strides in ELEMENTS).  The default
 * layout is [num_pages][page_size][heads][width] row-major.
 *
 *   pool0     GQA: K pool | GTA: tied-state pool | latent: latent pool
 *   pool1     GQA: V pool | otherwise NULL
 *   rope_pool GTA: un-rotated single-head RoPE key | latent: rotated RoPE key
 *             | GQA: NULL
 *   page_table int32 [batch][max_pages_per_seq]; entries for pages a
 *             sequence uses are in [0, num_pages); the rest may be -1 and are
 *             never read.
 *   seqlens   int32 [batch], 0 <= seqlens[b] <= max_pages_per_seq*page_size.
 *             Read only by attn_kv_append: the decode calls take every
 *             sequence's length from the plan (attn_decode_plan's
 *             seqlens_host), so a plan must be made from the lengths the
 *             cache holds when the decode runs.
 *
 * Requirements: page_size is a power of two; pool base pointers and every
 * row start are 16-byte aligned (strides * element size multiple of 16).
 * Slots past a sequence's length and pages no sequence uses are never read,
 * so they may hold anything (NaN included).
 */
typedef struct {
  const void* pool0;
  const void* pool1;
  const void* rope_pool;
  const int32_t* page_table;
  const int32_t* seqlens;
  int32_t batch;
  int32_t max_pages_per_seq;
  int32_t page_size;
  int32_t num_pages;
  int64_t page_stride, token_stride, head_stride;
  int64_t rope_page_stride, rope_token_stride, rope_head_stride;
  attn_dtype_t dtype;
} attn_paged_kv_t;

/*
 * Split plan: which (sequence, group, token chunk) each workgroup handles.
 * Filled on the host by attn_decode_plan.  The kernels read it either from
 * device copies of the two host arrays (the caller copies them and stores
 * the device pointers in `items` and `seqinfo`) or, when `inline_ok` is set
 * and both pointers are left NULL, from the launch arguments, packed by the
 * call from the host arrays (see "Launch-argument plans" below: no copy is
 * needed).  Either way the host arrays must still hold what
 * attn_decode_plan wrote when a decode or merge call is made: every call
 * checks them on the host (each length at most max_pages_per_seq *
 * page_size, at least q_len for causal calls; chunks, splits, partial slots
 * and items consistent) and returns INVALID_ARG, launching nothing, if they
 * are not.  Device copies must equal the host arrays.
 *
 *   items   [n_items][4]  int32: b, group j, split index s, first token t0
 *           (the chunk is [t0, min(t0 + chunk, L_b)))
 *   seqinfo [batch][4]    int32: n_splits_b, partial slot base, L_b, chunk
 *
 * counters: with a non-NULL device array of attn_decode_counter_count()
 * uint32 the streaming kernels merge split rows themselves (the last split
 * workgroup of each (sequence, group, block of 32 query rows) to finish
 * merges them, counted with atomic counters that wrap back to zero), so no
 * merge launch follows.  The array must hold zeros before its first use;
 * every complete call leaves it zero, so one array serves every later call
 * and plan it is large enough for, as long as calls sharing it do not
 * overlap.  NULL (what attn_decode_plan stores): the merge is a second
 * launch on the stream.
 */
typedef struct {
  int32_t n_items;
  int32_t batch;
  int32_t n_groups;
  int32_t q_len;
  int32_t max_splits;      /* largest n_splits_b                                 */
  int32_t n_partial_slots; /* sum of n_splits_b over sequences with n_splits_b>1 */
  const int32_t* items;    /* DEVICE copy of items_host                          */
  const int32_t* seqinfo;  /* DEVICE copy of seqinfo_host                        */
  uint32_t* counters;      /* DEVICE merge arrival counters or NULL (see below)  */
  const int32_t* items_host;   /* the host arrays attn_decode_plan filled        */
  const int32_t* seqinfo_host;
  int32_t inline_ok;       /* 1: the plan fits the kernels' launch arguments     */
  uint32_t* queue;         /* DEVICE work-queue counter or NULL (see below)      */
} attn_plan_t;

/*
 * queue: with a non-NULL device uint32 (zero before its first use) the GQA
 * streaming kernel launches only as many workgroups as the GPU keeps
 * resident; each takes one item of the plan's order first and then draws
 * the next unstarted item from this counter as it finishes, so work moves
 * to whichever XCD frees up first.  Every complete call leaves the counter
 * zero, so one counter serves every later call; calls sharing it must not
 * overlap.  NULL (what attn_decode_plan stores): a fixed item per workgroup.
 * Other kernels ignore it.
 */

/*
 * Launch-argument plans.  A plan needs 3 * batch + n_items / n_groups int32
 * in compact form (three per sequence, one per chunk; half an int32 per
 * chunk when batch <= 2048 and every n_splits_b <= 32); when that is at
 * most ATTN_PLAN_INLINE_MAX (and batch and n_splits_b stay below 65536 and
 * every chunk below 2^22 tokens), attn_decode_plan sets inline_ok.  A decode or merge call whose
 * plan then has items == NULL and seqinfo == NULL packs the plan from
 * items_host / seqinfo_host (which must still hold what attn_decode_plan
 * wrote) into the kernels' launch arguments, so no upload is needed.  With
 * items and seqinfo NULL and inline_ok 0 the calls return INVALID_ARG.
 */
#define ATTN_PLAN_INLINE_MAX 800

/*
 * Shape of a decode call, as the planner needs it.
 *   kind      GQA, GTA or latent (MLA / GLA)
 *   groups    KV heads h_kv (GQA/GTA) or latent heads h_c (latent)
 *   head_dim  d (GQA/GTA) or d_c (latent); d_rope: 0 for GQA
 *   flags     ATTN_CAUSAL if the call is causal (q_len > 1)
 */
typedef struct {
  attn_kind_t kind;
  attn_dtype_t dtype;
  int32_t batch, q_len, h_q, groups, head_dim, d_rope, page_size, flags;
} attn_shape_t;

/* Upper bound on the work items attn_decode_plan can emit (host-only). */
int attn_decode_plan_max_items(int batch, int n_groups, int max_seqlen);

/*
 * Build a split plan on the host (integer work only, no GPU calls).
 *   shape         the decode call's shape (see attn_shape_t)
 *   seqlens_host  host int32 [batch]
 *   cu_count      compute units of the target GPU (256 on MI355X)
 *   chunk_tokens  0: automatic split (balances the longest chunk, given how
 *                 many workgroups the chosen kernel keeps per CU, against
 *                 the partial-result traffic that more splits cost);
 *                 > 0: force chunks of this many tokens (multiple of 64)
 *   items_host    host int32 [max_items][4], seqinfo_host host int32 [batch][4]
 * Errors: INVALID_ARG for null pointers, non-positive sizes, negative
 * lengths, causal lengths below q_len, chunk_tokens not a multiple of 64;
 * WORKSPACE if max_items is too small.  On success plan->items and
 * plan->seqinfo are NULL: the caller sets them to device copies of the host
 * arrays, or, when plan->inline_ok is 1, may leave them NULL so that the
 * calls pass the plan in the kernels' launch arguments.  The host arrays
 * must outlive every call made with the plan.
 */
int attn_decode_plan(const attn_shape_t* shape, const int32_t* seqlens_host, int cu_count,
                     int chunk_tokens, int32_t* items_host, int32_t* seqinfo_host,
                     int max_items, attn_plan_t* plan);

/*
 * Bytes of device workspace a decode call needs: fp32 O_part
 * [slots][q_len][h_q][d_v] and fp32 LSE_part [slots][q_len][h_q] for split
 * partials (slots = plan->n_partial_slots), then per-workgroup flags of the
 * latent kernel's fix-up pass.  Contents need no initialisation.
 */
size_t attn_decode_workspace_size(const attn_plan_t* plan, int h_q, int d_v);

/*
 * Number of uint32 merge counters (plan->counters) a call with this plan
 * and h_q uses: batch * groups * ceil(rows / 32), rows = (h_q / groups) *
 * q_len.  Returns 0 for an invalid plan.
 */
size_t attn_decode_counter_count(const attn_plan_t* plan, int h_q);

/*
 * GQA decode (GTA/MQA/MHA-compatible layout with separate K and V pools).
 *   q    [batch][q_len][h_q][d]       dtype of kv->dtype, contiguous
 *   out  [batch][q_len][h_q][d]       same dtype, contiguous
 *   lse  [batch][q_len][h_q] fp32, or NULL
 *   flags ATTN_CAUSAL and/or ATTN_DEFER_MERGE
 *   plan, workspace  from attn_decode_plan / attn_decode_workspace_size;
 *        the workspace is always required (its size is at least 256 bytes)
 *        and must be 256-byte aligned
 * Supported: d in {64, 128}; h_q % h_kv == 0; q_len in [1, 16].
 */
int attn_decode_gqa(const attn_paged_kv_t* kv, const void* q, void* out, float* lse,
                    int q_len, int h_q, int h_kv, int d, float softmax_scale, int flags,
                    const attn_plan_t* plan, void* workspace, size_t workspace_bytes,
                    hipStream_t stream);

/*
 * Allocation-free GQA decode, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  The same call and results as attn_decode_gqa (the
 * same kernels, bit for bit), without the workspace argument: the split
 * partials live in a device array of ATTN_STATIC_SCRATCH_BYTES inside the
 * library, one per GPU the library runs on, held until the process ends
 * (its device address is looked up once per device, on the first call made
 * with that device current).  No call allocates or frees memory, and
 * nothing in the array needs to start at zero.
 * Every call on one GPU shares that array and it keeps the last call's
 * contents: calls that overlap in time on one GPU (several streams or host
 * threads) race on it, so the caller must serialise them.
 * Errors: as attn_decode_gqa; ATTN_ERR_WORKSPACE when the plan needs more
 * than ATTN_STATIC_SCRATCH_BYTES (attn_decode_workspace_size(plan, h_q, d)
 * > ATTN_STATIC_SCRATCH_BYTES); INVALID_ARG with ATTN_DEFER_MERGE (the
 * partials would be out of the caller's reach); ATTN_ERR_HIP when the
 * array's device address cannot be obtained.
 */
#define ATTN_STATIC_SCRATCH_BYTES (16u << 20)
int attn_decode_gqa_static(const attn_paged_kv_t* kv, const void* q, void* out, float* lse,
                           int q_len, int h_q, int h_kv, int d, float softmax_scale, int flags,
                           const attn_plan_t* plan, hipStream_t stream);

/*
 * GTA decode: tied state pool0 [.., h_kv, d], single-head RoPE key
 * rope_pool [.., n_rope_heads = 1, d_rope].  With rope_theta > 0 the key's
 * RoPE slice and the query's last d_rope entries are rotated in the kernel;
 * with rope_theta <= 0 both are taken as already rotated.
 *   q [batch][q_len][h_q][d], out [batch][q_len][h_q][d], lse as for GQA.
 * Supported: bf16, d = 128, d_rope = 64, n_rope_heads = 1.
 */
int attn_decode_gta(const attn_paged_kv_t* kv, const void* q, void* out, float* lse,
                    int q_len, int h_q, int h_kv, int d, int d_rope, int n_rope_heads,
                    float rope_theta, float softmax_scale, int flags,
                    const attn_plan_t* plan, void* workspace, size_t workspace_bytes,
                    hipStream_t stream);

/*
 * Latent decode (MLA: h_c = 1, GLA: h_c > 1) in the weight-absorbed space.
 *   q   [batch][q_len][h_q][d_c + d_rope] (RoPE part already rotated)
 *   out [batch][q_len][h_q][d_c]
 * Supported: bf16, (d_c, d_rope) in {(512, 64), (256, 64)}, h_q % h_c == 0.
 */
int attn_decode_latent(const attn_paged_kv_t* kv, const void* q, void* out, float* lse,
                       int q_len, int h_q, int h_c, int d_c, int d_rope,
                       float softmax_scale, int flags, const attn_plan_t* plan,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Log-sum-exp merge of split partials (the second half of a decode call made
 * with ATTN_DEFER_MERGE; Hydragen's softmax-denominator decomposition on the
 * "Efficient Inference" tag page).  For every sequence with n_splits > 1 and
 * every row: M = max_s lse_s, w_s = exp(lse_s - M),
 * out = sum_s w_s O_s / sum_s w_s, lse = M + ln sum_s w_s.  Rows of
 * sequences with one split were already written by the decode call.
 *   workspace  the decode call's workspace (partials), device
 *   out        [batch][q_len][h_q][d_v] in `dtype`; lse [batch][q_len][h_q]
 *              fp32 or NULL
 * Supported: d_v in {64, 128, 256, 512}.
 */
int attn_decode_merge(const attn_plan_t* plan, int h_q, int d_v, attn_dtype_t dtype,
                      const void* workspace, size_t workspace_bytes, void* out, float* lse,
                      hipStream_t stream);

/*
 * Paged KV append: write the rows of a step's new tokens into the cache
 * before the decode call that reads them.  Sequence b's q_len new tokens
 * take positions L_b - q_len .. L_b - 1 (kv->seqlens already counts them, as
 * in the decode calls) and land in page page_table[b][pos / page_size],
 * slot pos % page_size, through the descriptor's strides; the caller has
 * already assigned those pages.  Positions below 0 are skipped.
 *   new0      [batch][q_len][heads][width] rows for pool0 (GQA keys, GTA tied
 *             state, latent rows), device, kv->dtype
 *   new1      same shape for pool1 (GQA values) or NULL (pool1 untouched)
 *   new_rope  [batch][q_len][d_rope] RoPE key rows for rope_pool, or NULL;
 *             with rope_theta > 0 each is rotated at its position
 *             (rotate-half pairs (k, k + d_rope/2), angle pos *
 *             theta^(-2k/d_rope), computed in fp32) before it is stored:
 *             latent caches hold rotated keys ("Hardware-Efficient Attention
 *             for Fast Decoding", review page, Core claim), GTA caches raw
 *             ones (pass rope_theta <= 0; the decode rotates them).
 * A row whose position falls past the sequence's page-table row
 * (pos / page_size >= max_pages_per_seq) or whose page-table entry is not in
 * [0, num_pages) is skipped: nothing is written for it.
 * Copies are exact; rotated keys are rounded to kv->dtype.  Row starts and
 * row widths must be multiples of 16 bytes, d_rope even and at most 64.
 * Returns ATTN_OK once enqueued on `stream`, INVALID_ARG (nothing enqueued)
 * for inconsistent arguments.
 */
int attn_kv_append(const attn_paged_kv_t* kv, int q_len, int heads, int width, const void* new0,
                   const void* new1, int d_rope, const void* new_rope, float rope_theta,
                   hipStream_t stream);

/*
 * Projections around attn_decode_latent (MLA / GLA weight absorption).  The
 * latent kernel attends in the latent space ("Hardware-Efficient Attention
 * for Fast Decoding", review page: Core claim, What carries the argument);
 * the per-head key and value up-projections act on the query and on the
 * latent output instead of on the cache.  For every token m (the step's
 * batch * q_len query rows) and query head h, in fp32 from bf16 inputs:
 *
 * attn_latent_absorb_query:
 *   q_out[m][h][n]       = sum_k q_nope[m][h][k] * w_uk[h][n][k],  n < d_c
 *   q_out[m][h][d_c + j] = q_rope[m][h][j]  (copied),              j < d_rope
 *   q_nope  [n_tok][h_q][d_nope] bf16, device
 *   q_rope  [n_tok][h_q][d_rope] bf16, device, already rotated; NULL iff
 *           d_rope == 0
 *   w_uk    [h_q][d_c][d_nope] bf16, device: head h's key up-projection
 *           stored transposed (row n holds the weights of latent dim n)
 *   q_out   [n_tok][h_q][d_c + d_rope] bf16, device: the latent kernel's q
 * so that q_out[m][h][0:d_c] . c = q_nope[m][h] . (w_uk[h]^T c) for a latent
 * row c.
 *
 * attn_latent_project_output:
 *   out[m][h][n] = sum_c o_lat[m][h][c] * w_uv[h][n][c],  n < d_v
 *   o_lat  [n_tok][h_q][d_c] bf16, device: the latent kernel's output
 *   w_uv   [h_q][d_v][d_c] bf16, device: head h's value up-projection
 *   out    [n_tok][h_q][d_v] bf16, device
 *
 * Results are rounded to bf16 once.  Requirements: d_nope and (for the
 * output projection) d_c multiples of 32; d_c (absorb) and d_v multiples
 * of 64; d_rope a multiple of 8; every pointer 16-byte aligned; n_tok = 0
 * enqueues nothing and accepts NULL buffers.  The caller owns every buffer;
 * outputs must not alias inputs.  Returns ATTN_OK once enqueued on `stream`,
 * INVALID_ARG (nothing enqueued) for inconsistent arguments.
 */
int attn_latent_absorb_query(const void* q_nope, const void* q_rope, const void* w_uk,
                             void* q_out, int n_tok, int h_q, int d_nope, int d_c, int d_rope,
                             hipStream_t stream);
int attn_latent_project_output(const void* o_lat, const void* w_uv, void* out, int n_tok,
                               int h_q, int d_c, int d_v, hipStream_t stream);

/*
 * Host-side consistency check of a descriptor whose page_table and seqlens
 * point to HOST copies: every page a sequence uses is in [0, num_pages) and
 * every length fits the page table.  Returns ATTN_OK or INVALID_ARG.
 */
int attn_paged_kv_check(const attn_paged_kv_t* host_copy);

/*
 * Measurement probes (not part of the decode path): the ceilings the decode
 * kernels are compared with on the GPU they run on.  Decode is bound by
 * reading the KV cache from HBM ("Hardware-Efficient Attention for Fast
 * Decoding", review page, Core claim) or, at high arithmetic intensity, by
 * the matrix cores (its Figure 3 caption, the roofline).
 *
 * attn_probe_stream_read: read `bytes` of device memory at `buf` once,
 *   split into 64 KB blocks over a few workgroups per CU, with the
 *   nontemporal hint; mode 0 loads into registers, mode 1 loads straight
 *   into LDS (global_load_lds_dwordx4, the decode kernels' path).  The
 *   bytes read are exactly `bytes`: time the launch with events on
 *   `stream` to get the streaming-read rate.  `sink` is a device uint32
 *   the kernel may write (to keep the loads); nothing else is written.
 *   Requirements: `bytes` a positive multiple of 65536, `buf` 1024-byte
 *   aligned; INVALID_ARG otherwise.
 * attn_probe_mfma: every wave of two 4-wave workgroups per CU runs `iters`
 *   rounds of 8 independent v_mfma_f32_16x16x32_bf16 products on register
 *   operands; *flops_out (host) receives the launch's FLOPs (2 per
 *   multiply-add) so that FLOPs / duration is the matrix cores' bf16 rate.
 *   `sink` is a device float the kernel may write.
 * Both return ATTN_OK once enqueued on `stream`.
 */
int attn_probe_stream_read(const void* buf, size_t bytes, int mode, uint32_t* sink,
                           hipStream_t stream);
int attn_probe_mfma(int iters, float* sink, double* flops_out, hipStream_t stream);

/* Static description of a status code. */
const char* attn_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* ATTN_DECODE_H */
