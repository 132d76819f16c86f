/*
 * mla_decode.h -- C ABI of the MI355X (gfx950) weight-absorbed MLA decode library.
 *
 * Operation (web page "MLA deep compression", operatorworld.com, sections
 * "Absorption: an equivalent rewrite at inference" and "Decoupled RoPE"; and
 * "Attention-head anatomy: one cache, four wirings", romaanj.github.io, section 5):
 * every query head i of a new token scores the shared per-token cache row
 * [c_j (d_c values) | k^R_j (d_r values)] with its absorbed query q~_i = W^QK_i h
 * (q_nope) and its rotated RoPE query q^R_i (q_pe):
 *
 *     s_ij = softmax_scale * (q~_i . c_j + q^R_i . k^R_j)
 *     a_i  = softmax_j(s_ij)          over the visible tokens j
 *     u_i  = sum_j a_ij c_j           (latent space, d_c values)
 *     o_i  = W^UV_i u_i               (d_v values)
 *     lse_i = ln sum_j exp(s_ij)
 *
 * With s_q new tokens per sequence (multi-token decode, GQLA abstract on
 * chatpaper.ai: s_q = 1 and s_q = 2), query position q of sequence b sits at
 * index L_b - s_q + q and sees tokens 0 .. L_b - s_q + q (causal within the new
 * tokens, each new token sees itself; L_b counts the new tokens).
 *
 * Conventions shared by every entry point
 *  - Every pointer argument is a DEVICE pointer owned by the caller, except the
 *    params pointer (host).  The library never allocates, frees or synchronizes:
 *    work is enqueued on `stream` (a hipStream_t; NULL = the null stream).
 *  - All validation happens on the host before any launch; a failed check returns
 *    an error status and enqueues nothing.  Data that lives on the device
 *    (seq_lens, block_table, positions) cannot be checked synchronously: see the
 *    per-argument notes for what the kernels do with out-of-range values.
 *  - Status codes, never exceptions or aborts, cross the ABI.
 *  - Arrays are dense row-major with the shapes given; "elements" are of the
 *    array's own dtype.
 *  - The library keeps two kinds of state: cached device attributes (per device,
 *    read once) and one per-thread measurement setting, the events that
 *    mla_set_attention_events() asks the partial-attention launches of the calling
 *    thread to record (none unless a caller sets them).  Nothing else persists
 *    between calls; calls on different streams may overlap if their outputs and
 *    workspaces are disjoint.
 *  - Sizes of the pool are given, not bounds on the lengths: the params carry
 *    num_pages (pool pages, to reject page ids) and max_pages_per_seq (row stride of
 *    the block table); there is no max_seq_len field, since every kernel reads the
 *    lengths from seq_lens on the device and clamps them to max_pages_per_seq * P.
 *  - num_splits counts shares of the whole batch's tokens (the split rule below),
 *    not splits per sequence: one call launches num_splits workgroups per group of
 *    query rows, however the lengths are spread over the batch.
 */
#ifndef MLA_DECODE_H_
#define MLA_DECODE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_ABI_VERSION 1
#define MLA_SPLIT_UNIT 64 /* tokens per scheduling unit of the split rule */

typedef enum {
  MLA_DTYPE_F32 = 0,
  MLA_DTYPE_BF16 = 1,
  MLA_DTYPE_FP8_E4M3 = 2 /* OCP FP8 E4M3 "fn": bias 7, max 448, NaN = 0x7F/0xFF, no inf */
} mla_dtype_t;

typedef enum {
  MLA_OK = 0,
  MLA_ERR_NULL = 1,        /* a required pointer is NULL */
  MLA_ERR_SHAPE = 2,       /* a size, stride or shape combination is unsupported */
  MLA_ERR_DTYPE = 3,       /* an unsupported dtype combination */
  MLA_ERR_WORKSPACE = 4,   /* workspace missing or smaller than mla_decode_workspace_size() */
  MLA_ERR_HIP = 5,         /* the HIP runtime reported an error at launch */
  MLA_ERR_UNSUPPORTED = 6, /* no kernel for this device */
  MLA_ERR_TOO_LARGE = 7    /* mla_decode_fwd_noalloc: the call needs more than its static workspace */
} mla_status_t;

/*
 * Shapes and options of one decode call.
 *
 * Supported combinations (q_dtype, kv_dtype, w_dtype, out_dtype):
 *   (F32,  F32,       F32,  F32)   any d_c <= 1024, d_r <= 256, d_v <= 1024, n_h <= 1024
 *   (BF16, BF16,      BF16, BF16)  d_c = 512, d_r = 64, d_v = 128, n_h = 16, 32 or a multiple of 64
 *   (BF16, FP8_E4M3,  BF16, BF16)  d_c = 512, d_r = 64, d_v = 128, n_h a multiple of 16 and
 *                                  s_q * n_h <= 128 or a multiple of 128
 * batch >= 1, 1 <= s_q <= 16, page_size a positive multiple of 64.
 */
typedef struct {
  int32_t batch;             /* B: sequences in the call */
  int32_t s_q;               /* new query tokens per sequence */
  int32_t n_h;               /* query heads */
  int32_t d_c;               /* latent width (512 in DeepSeek-V2/V3) */
  int32_t d_r;               /* decoupled-RoPE key/query width (64) */
  int32_t d_v;               /* per-head output width (128) */
  int32_t page_size;         /* P: tokens per cache page; a contiguous cache is one page per sequence */
  int32_t num_pages;         /* pages in the pool; page ids outside [0, num_pages) are never read */
  int32_t max_pages_per_seq; /* row stride of block_table */
  int32_t num_splits;        /* G >= 1: shares of the batch's tokens (see the split rule); 0 = auto */
  int64_t c_kv_stride;       /* elements between consecutive pool slots of c_kv (>= d_c) */
  int64_t k_pe_stride;       /* elements between consecutive pool slots of k_pe (>= d_r) */
  float softmax_scale;       /* applied to the sum of both dot products, e.g. 1/sqrt(d_h + d_r) */
  mla_dtype_t q_dtype, kv_dtype, w_dtype, out_dtype;
} mla_decode_params_t;

/*
 * Split rule (how one call is divided into partial attentions).
 * Sequence b is cut into n_b = ceil(L_b / 64) units; the units of all sequences, in
 * batch order, form one list of U = sum_b n_b units, cut into G = num_splits shares
 * of ceil(U / G) consecutive units.  Share w meets sequence b in at most one piece
 * (tokens [t0, t1), t0 a multiple of 64); that piece's partial is stored in slot
 * w + b.  Each sequence therefore owns the consecutive slots [first_b, first_b +
 * count_b) with count_b = number of shares its units fall in.
 *
 * Workspace layout (all offsets from the workspace base, each 256-byte aligned):
 *   split_table  int32 [B][2]                     (first slot, count) per sequence; (0, 0) if L_b = 0
 *   partial_lse  float [num_slots][s_q][n_h]      ln-sum-exp of the piece's scores; -inf if empty
 *   partial_u    E     [num_slots][s_q][n_h][d_c] u of the piece, normalized by its own softmax sum
 * with num_slots = G + B and E = float for the fp32 dtype combination, bf16 (round to
 * nearest even) for the bf16 and E4M3-cache combinations, whose output is bf16 anyway.
 * Rows of a piece that see no token have lse = -inf and u = 0.
 */

/* Effective number of splits G for these params on the current device
 * (num_splits when positive, else a choice that fills the GPU).  Returns <= 0 on
 * invalid params or when no device is present. */
int32_t mla_decode_num_splits(const mla_decode_params_t* params);

/* Bytes of workspace mla_decode_fwd needs (0 on invalid params). */
size_t mla_decode_workspace_size(const mla_decode_params_t* params);

/*
 * One decode step of absorbed MLA over a paged latent cache.
 *
 *  q_nope      [B, s_q, n_h, d_c]  q_dtype  absorbed content queries q~_i
 *  q_pe        [B, s_q, n_h, d_r]  q_dtype  RoPE queries, already rotated
 *  c_kv        pool of latents; slot s at c_kv + s * c_kv_stride (kv_dtype, d_c values)
 *  k_pe        pool of RoPE keys; slot s at k_pe + s * k_pe_stride (kv_dtype, d_r values,
 *              already rotated).  A packed cache row [c | k^R] is c_kv = row base,
 *              k_pe = row base + d_c, both strides d_c + d_r.
 *  kv_scale    [num_pages * page_size] float, per-slot dequantization scale when
 *              kv_dtype = FP8_E4M3 (value = code * scale); must be NULL otherwise
 *  block_table [B, max_pages_per_seq] int32: token t of sequence b lives in slot
 *              block_table[b][t / P] * P + t % P.  Entries past the sequence's last
 *              page are not read; a page id outside [0, num_pages) makes its
 *              tokens invisible (never read).
 *  seq_lens    [B] int32: L_b, tokens in the cache of sequence b including the s_q
 *              new ones; values are clamped to [0, max_pages_per_seq * P].
 *  w_uv        [n_h, d_v, d_c] w_dtype: per-head up-projection W^UV_i
 *  out         [B, s_q, n_h, d_v] out_dtype, or NULL to stop after the partials
 *  lse         [B, s_q, n_h] float (natural log), or NULL
 *  workspace   device buffer of workspace_bytes >= mla_decode_workspace_size()
 *
 * A row with no visible token yields o = 0 and lse = -inf.  Results depend only on
 * the logical token order, not on the page placement.
 */
mla_status_t mla_decode_fwd(const mla_decode_params_t* params, const void* q_nope, const void* q_pe,
                            const void* c_kv, const void* k_pe, const float* kv_scale,
                            const int32_t* block_table, const int32_t* seq_lens, const void* w_uv,
                            void* out, float* lse, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Merge split partials and up-project: for every (b, q, head),
 *   lse = ln sum_s exp(lse_s)  over the sequence's slots (skipping -inf),
 *   u   = sum_s exp(lse_s - lse) u_s,   o = W^UV_i u.
 * Reads split_table, partial_lse and partial_u from `workspace` (layout above),
 * e.g. as left by mla_decode_fwd with out == NULL, or written by the caller.
 * w_uv may be NULL: then out receives the merged latents u as float32
 * [B, s_q, n_h, d_c] instead of o (the input of mla_output_projection with folded
 * weights).
 * Slot ranges are clipped to [0, G + B); a sequence whose slots are all empty
 * yields o = 0 and lse = -inf.
 */
mla_status_t mla_decode_splitkv_combine(const mla_decode_params_t* params, const void* workspace,
                                        size_t workspace_bytes, const void* w_uv, void* out, float* lse,
                                        void* stream);

/*
 * Append new cache rows (the write that precedes attention; page "MLA deep
 * compression", low-rank projection and decoupled-RoPE sections: only c_t and
 * k^R_t are cached).
 *
 *  c_new     [B, s_new, d_c] in_dtype,  k_pe_new [B, s_new, d_r] in_dtype
 *  positions [B, s_new] int32 absolute token indices (distinct within a sequence)
 *  c_kv, k_pe, kv_scale, block_table: the pool as in mla_decode_fwd (written in place)
 *
 * kv_dtype == in_dtype (F32 or BF16): the rows are copied bit for bit.
 * kv_dtype == FP8_E4M3 (in_dtype F32 or BF16): each token's d_c + d_r values are
 * quantized together: amax = max |x| (float32); amax = 0 gives scale = 1 and
 * inv = 1, else inv = fp32(448 / amax) and scale = fp32(amax / 448);
 * code = E4M3(fp32(x * inv)) rounded to nearest even, saturated to +-448;
 * kv_scale[slot] = scale.
 * A position whose page index is >= max_pages_per_seq, or whose page id is
 * outside [0, num_pages), is skipped.  Uses params->batch, d_c, d_r, page_size,
 * num_pages, max_pages_per_seq, strides and kv_dtype.
 */
mla_status_t mla_paged_cache_append(const mla_decode_params_t* params, const void* c_new,
                                    const void* k_pe_new, int32_t s_new, mla_dtype_t in_dtype,
                                    const int32_t* positions, const int32_t* block_table, void* c_kv,
                                    void* k_pe, float* kv_scale, void* stream);

/*
 * Append, then decode: the same effect as mla_paged_cache_append(params, c_new, k_pe_new,
 * s_new, in_dtype, positions, block_table, c_kv, k_pe, kv_scale) followed by
 * mla_decode_fwd(params, q_nope, ..., stream) on the same stream (arguments and
 * validation as there; nothing is launched unless both would be accepted).
 * When the cache and the new rows are bf16, n_h is a multiple of 128 and s_new <= 2,
 * both happen in the one partial-attention launch: tiles that hold a new position take
 * that row from c_new / k_pe_new, and the pool rows are written at the end of the
 * launch.  The outputs and the pool afterwards are the same bits as with the two calls.
 * Otherwise the two calls are made.
 */
mla_status_t mla_decode_fwd_append(const mla_decode_params_t* params, const void* c_new, const void* k_pe_new,
                                   int32_t s_new, mla_dtype_t in_dtype, const int32_t* positions,
                                   const void* q_nope, const void* q_pe, void* c_kv, void* k_pe, float* kv_scale,
                                   const int32_t* block_table, const int32_t* seq_lens, const void* w_uv,
                                   void* out, float* lse, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Measurement hook (for callers that time the attention kernel, such as a benchmark):
 * the partial-attention kernel of every later mla_decode_fwd call made by the calling
 * thread records `start` when it begins executing and `stop` when it ends (hipEvent_t
 * handles created by the caller, which keeps ownership).  Unlike events recorded on
 * the stream around the call, these exclude the dispatch gap before the kernel.
 * NULL, NULL restores plain launches.  The setting is per thread; it does not touch
 * the append or combine kernels.  Always returns MLA_OK.
 */
mla_status_t mla_set_attention_events(void* start, void* stop);

/*
 * ----------------------------------------------------------------------------------
 * Projections adjacent to the decode step (page "MLA deep compression": low-rank
 * projection, absorption and decoupled-RoPE sections; "Attention-head anatomy",
 * section 5: W^UK folds into the query path, W^UV into W^O).  Operands are dense
 * row-major; every product contracts over the last (contiguous) index of both operands.
 * bf16 operands (params->q_dtype / w_dtype == BF16) run on MFMAs with float32
 * accumulation and need the contraction width a multiple of 32, the other product
 * widths multiples of 16 and 16-byte aligned operand pointers, and each activation
 * operand (h, q^C, o or u) below 2 GiB (a weight of 2 GiB or more runs as several launches
 * over its rows); float32 operands accept any size.  RoPE rotates interleaved pairs (x[2m], x[2m+1]) at position p by the angle
 * p * rope_base^(-2m/d_r), taken in float64.  Each call needs a workspace of the size
 * its *_workspace_size function returns (0 means invalid params); a workspace too small
 * gives MLA_ERR_WORKSPACE.  None of them reads seq_lens.
 * ----------------------------------------------------------------------------------
 */

/*
 * Cache write: the new tokens' cache rows from their hidden states, written into the
 * paged pool (the step that precedes attention):
 *     c_t = W^DKV h_t,   k^R_t = RoPE(W^KR h_t, positions[t]),   pool row = [c_t | k^R_t]
 *  h          [B, s_new, d_model]  q_dtype (BF16 or F32)
 *  w_dkv      [d_c, d_model]       q_dtype
 *  w_kr       [d_r, d_model]       q_dtype
 *  positions  [B, s_new] int32: absolute token index, the RoPE position and the slot
 *             (same slot rule and skips as mla_paged_cache_append)
 *  c_kv, k_pe, kv_scale, block_table: the pool, as in mla_paged_cache_append.
 * The row is computed in float32 and stored per params->kv_dtype: BF16 (round to
 * nearest even; needs q_dtype BF16), F32 (needs q_dtype F32), or FP8_E4M3 with the
 * per-token scale of mla_paged_cache_append's quantizer applied to the float32 row.
 * Uses params batch, d_c, d_r (both even, d_c + d_r <= 1280), page_size, num_pages,
 * max_pages_per_seq, strides, q_dtype and kv_dtype.
 */
size_t mla_cache_write_workspace_size(const mla_decode_params_t* params, int32_t d_model, int32_t s_new);
mla_status_t mla_cache_write(const mla_decode_params_t* params, int32_t d_model, int32_t s_new, const void* h,
                             const void* w_dkv, const void* w_kr, const int32_t* positions, float rope_base,
                             const int32_t* block_table, void* c_kv, void* k_pe, float* kv_scale, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * Query prologue: the decode call's queries from the new tokens' hidden states,
 *     q_nope[.., i, :] = (W^UK_i)^T (W^Q_i h_t)      (= W^QK_i h_t of the score-side
 *                                                     equation, formed in two products)
 *     q_pe[.., i, :]   = RoPE(W^QR_i h_t, positions[t])
 *  h        [B, s_q, d_model]      q_dtype (BF16 or F32)
 *  w_q      [n_h * d_h, d_model]   rows i*d_h .. are W^Q_i
 *  w_uk_t   [n_h, d_c, d_h]        head i's (W^UK_i)^T (the up-projection transposed)
 *  w_qr     [n_h * d_r, d_model]   rows i*d_r .. are W^QR_i
 *  positions [B, s_q] int32
 *  q_nope   [B, s_q, n_h, d_c], q_pe [B, s_q, n_h, d_r]   q_dtype (the inputs of
 *           mla_decode_fwd)
 * W^Q_i h is kept in float32 and enters the second product as a bf16 high part plus
 * remainder.  Uses params batch, s_q, n_h, d_c, d_r and q_dtype.
 */
size_t mla_query_prologue_workspace_size(const mla_decode_params_t* params, int32_t d_model, int32_t d_h);
mla_status_t mla_query_prologue(const mla_decode_params_t* params, int32_t d_model, int32_t d_h, const void* h,
                                const void* w_q, const void* w_uk_t, const void* w_qr, const int32_t* positions,
                                float rope_base, void* q_nope, void* q_pe, void* workspace, size_t workspace_bytes,
                                void* stream);

/*
 * Output projection y = W x of the B * s_q rows of x:
 *   unfolded  x = the decode output o [B, s_q, n_h, d_v] (width = n_h * d_v), W = W^O
 *             [d_model, n_h * d_v] (column block i is W^O_i): y = sum_i W^O_i W^UV_i u_i;
 *   folded    x = the merged latents u [B, s_q, n_h, d_c] (float32, from
 *             mla_decode_splitkv_combine with w_uv = NULL; width = n_h * d_c), W = W^OV
 *             from mla_fold_output_weights: the same y.
 *  x_dtype    BF16 or F32 (F32 enters bf16 products as high part plus remainder)
 *  w          [d_model, width]  params->w_dtype
 *  y          [B, s_q, d_model] params->out_dtype
 */
size_t mla_output_projection_workspace_size(const mla_decode_params_t* params, int32_t d_model, int32_t width,
                                            mla_dtype_t x_dtype);
mla_status_t mla_output_projection(const mla_decode_params_t* params, int32_t d_model, int32_t width,
                                   mla_dtype_t x_dtype, const void* x, const void* w, void* y, void* workspace,
                                   size_t workspace_bytes, void* stream);

/*
 * Offline fold of W^UV into W^O: w_ov [d_model, n_h * d_c] with column block i =
 * W^O_i W^UV_i ([d_model, d_v] x [d_v, d_c]), in params->w_dtype (bf16: float32
 * accumulation, one rounding).  w_o [d_model, n_h * d_v], w_uv [n_h, d_v, d_c].  The
 * folded weights hold d_c / d_v times the bytes of W^O (4x at the V3 shape), so at decode
 * the unfolded projection reads less; the fold is the page's offline form.
 */
size_t mla_fold_output_weights_workspace_size(const mla_decode_params_t* params);
mla_status_t mla_fold_output_weights(const mla_decode_params_t* params, int32_t d_model, const void* w_o,
                                     const void* w_uv, void* w_ov, void* workspace, size_t workspace_bytes,
                                     void* stream);

/*
 * GQLA's per-group path (GQLA abstract, chatpaper.ai: the same weights expose an
 * MQA-absorb path identical to MLA's and a GQA path with a per-group expanded cache).
 * The n_h heads form n_g equal groups (heads g*n_h/n_g ..) that share W^UK_g and W^UV_g,
 * so the absorbed path is mla_decode_fwd with q_nope_i = (W^UK_g)^T q^C_i and
 * W^UV_i = W^UV_g, and the GQA path below reads instead a cache expanded per group.
 *
 * mla_gqla_expand_cache: for every pool slot s and group g,
 *     k_exp[s][g][:] = W^UK_g c_s  (d_h values),  v_exp[s][g][:] = W^UV_g c_s  (d_v values),
 * bf16 with float32 accumulation; w_uk_g [n_g, d_h, d_c], w_uv_g [n_g, d_v, d_c], c_kv the
 * latent pool (slot s at c_kv + s * c_kv_stride), k_exp [num_pages * P, n_g, d_h],
 * v_exp [num_pages * P, n_g, d_v].  The RoPE keys stay in the latent pool.
 *
 * mla_gqla_decode: per head i of group g and query position q (visibility as in
 * mla_decode_fwd),
 *     s_ij = softmax_scale (q_c_i . k_exp[j][g] + q_pe_i . k^R_j),
 *     out_i = sum_j softmax_j(s_i) v_exp[j][g],   lse_i = ln sum_j exp(s_ij),
 * with q_c [B, s_q, n_h, d_h], q_pe [B, s_q, n_h, d_r], k_pe the pool's RoPE keys, the
 * block table and seq_lens of mla_decode_fwd, out [B, s_q, n_h, d_v] bf16 and lse
 * [B, s_q, n_h] float (or NULL).  All dtypes bf16; n_h a multiple of n_g with
 * (n_h / n_g) * s_q <= 32; (d_h + d_r, d_v) one of (192, 128), (64, 64), (32, 32).
 * The workspace (mla_gqla_decode_workspace_size bytes) holds the split partials.
 */
mla_status_t mla_gqla_expand_cache(const mla_decode_params_t* params, int32_t n_g, int32_t d_h, const void* w_uk_g,
                                   const void* w_uv_g, const void* c_kv, void* k_exp, void* v_exp, void* stream);
size_t mla_gqla_decode_workspace_size(const mla_decode_params_t* params, int32_t n_g, int32_t d_h);
mla_status_t mla_gqla_decode(const mla_decode_params_t* params, int32_t n_g, int32_t d_h, const void* q_c,
                             const void* q_pe, const void* k_exp, const void* v_exp, const void* k_pe,
                             const int32_t* block_table, const int32_t* seq_lens, void* out, float* lse,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * mla_decode_fwd without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, results and validation as mla_decode_fwd, except:
 *  - the workspace is a static device array inside the library, one per device, of
 *    mla_decode_noalloc_capacity() bytes (64 MiB), set up on the first call on each
 *    device and kept until the process ends; the call allocates and frees nothing;
 *  - a call whose workspace (mla_decode_workspace_size) would exceed that size returns
 *    MLA_ERR_TOO_LARGE and enqueues nothing;
 *  - out must not be NULL (the partials stay in the library's array);
 *  - every call on one device shares that device's array, which keeps the last call's
 *    contents: calls that overlap on one device (e.g. on two streams) race and must be
 *    ordered by the caller.  No part of the array needs to start at zero.
 */
mla_status_t mla_decode_fwd_noalloc(const mla_decode_params_t* params, const void* q_nope, const void* q_pe,
                                    const void* c_kv, const void* k_pe, const float* kv_scale,
                                    const int32_t* block_table, const int32_t* seq_lens, const void* w_uv,
                                    void* out, float* lse, void* stream);

/* Bytes of the static workspace of mla_decode_fwd_noalloc (per device). */
size_t mla_decode_noalloc_capacity(void);

/* Static description of a status code. */
const char* mla_status_string(mla_status_t status);

/* MLA_ABI_VERSION of the built library. */
int32_t mla_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H_ */
