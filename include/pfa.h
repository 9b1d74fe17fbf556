/*
 * pfa.h -- C ABI of libpfa, the MI355X (gfx950) prefill attention core:
 * per-(token, head) RMSNorm of Q and K, NeoX rotary embedding, and causal
 * grouped-query softmax attention over token-major f32 activations.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  Layout.  Token-major and contiguous: element (token t, head h, dim c) of a
 *    tensor with `heads` heads sits at (t * heads + h) * head_dim + c.  Q and the
 *    attention output are [T, n_head * head_dim]; K and V are
 *    [T, n_head_kv * head_dim].  This is the layout the dense Qwen3 prefill of
 *    memra-engine 0.130.0 (src/forward.rs, `Model::forward`, activation-layout
 *    note and SDPA block) keeps between its projections and its attention.
 *  Pointers.  Tensor pointers are DEVICE pointers owned by the caller, 16-byte
 *    aligned (a misaligned f32 tensor is rejected with PFA_ERR_INVALID_ARG before
 *    anything is enqueued).  The library allocates no device memory and keeps no state beyond
 *    its loaded code objects; the attention calls take a caller-owned device
 *    workspace (see pfa_workspace_bytes).
 *  Sequences.  `seq_offsets` is a HOST array of n_seqs + 1 int32 values
 *    (cumulative lengths: seq_offsets[0] = 0, non-decreasing, seq_offsets[n_seqs]
 *    = T).  NULL means one sequence [0, T) (n_seqs is then ignored).  Token t of
 *    sequence s has rotary position t - seq_offsets[s]; attention never crosses
 *    a sequence boundary.  At most PFA_MAX_SEQS sequences; empty sequences are
 *    allowed and skipped.
 *  Streams.  `stream` is a hipStream_t (NULL: the null stream).  Every call only
 *    enqueues kernels on it and returns; nothing synchronises.  A device fault
 *    therefore surfaces at the caller's next synchronisation.
 *  Errors.  Each call returns a pfa_status and never aborts or throws.  All
 *    arguments are checked on the host before anything is enqueued, so a
 *    non-OK return means no kernel ran; pfa_last_error() then describes the
 *    problem (thread-local, valid until the next call on the same thread).
 *    T == 0 is a successful no-op.
 *  Limits.  head_dim in {64, 128}; n_head a multiple of n_head_kv, at most
 *    PFA_MAX_HEADS; rope_dim even, 2 <= rope_dim <= head_dim;
 *    T * max(n_head, n_head_kv) * head_dim < 2^31.
 */
#ifndef PFA_H
#define PFA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PFA_MAX_SEQS 128
#define PFA_MAX_HEADS 1024

typedef enum {
    PFA_OK = 0,
    PFA_ERR_INVALID_ARG = -1, /* a pointer, size or flag is invalid */
    PFA_ERR_UNSUPPORTED = -2, /* valid but outside what the kernels implement */
    PFA_ERR_HIP = -3          /* the HIP runtime refused a launch */
} pfa_status;

/* Input type of the two matrix products inside attention.  Accumulation,
 * softmax and the output are f32 in every case (the inputs and output stay f32
 * tensors; the 16-bit modes convert K and V once into the workspace).
 *  PFA_PREC_F32    f32 products.
 *  PFA_PREC_BF16   the (scaled) Q, K, V and the softmax weights are rounded to
 *                  bf16 (round to nearest even) before each product.
 *  PFA_PREC_BF16X3 as PFA_PREC_BF16 for P.V; the scores use Q and K each split
 *                  into a bf16 high part plus a bf16 low part (three products),
 *                  which keeps the score error from growing with large key norms.
 *  PFA_PREC_F16    as PFA_PREC_BF16 with IEEE binary16 in place of bf16 (round to
 *                  nearest even; 11 significant bits against 8, so about 8 times
 *                  less rounding, at the same matrix-core rate).  Its range is
 *                  narrower: a scaled Q, K or V value beyond 65504 in magnitude
 *                  becomes infinite and the rows it reaches come out NaN (the
 *                  softmax weights stay <= 256 and cannot overflow).
 * Every attention entry point takes every mode (qk_prep_chunk_attn_tiled all but
 * PFA_PREC_F32). */
typedef enum {
    PFA_PREC_F32 = 0,
    PFA_PREC_BF16 = 1,
    PFA_PREC_BF16X3 = 2,
    PFA_PREC_F16 = 3
} pfa_precision;

/* Device workspace in bytes that gqa_prefill_attn (fused = 0) or qk_prep_attn
 * (fused = 1) uses for these arguments (the same seq_offsets, n_seqs, T, heads,
 * head_dim and precision as the call).  It holds, in this order:
 *  - 16-bit modes: K and V converted once to bf16 (f16 for PFA_PREC_F16) in 64-key
 *    tiles per sequence (K twice, high and low parts, for PFA_PREC_BF16X3),
 *      n_head_kv * sum_s ceil(len_s / 64) * 64 * head_dim * 2 * (2 or 3) bytes,
 *    then, for qk_prep_attn, a rotary table of max_s(len_s) * (head_dim / 2) * 8
 *    bytes;
 *  - PFA_PREC_F32, qk_prep_attn: the normalised, rotated K, T * n_head_kv *
 *    head_dim * 4 bytes (not used when the call is given k_rot_out);
 *  - any precision, short inputs only, at the next multiple of 256 bytes: when
 *    the (query block, head) work items cannot fill the GPU (the current device's
 *    compute units, 256 on MI355X and when no device is visible; query with the
 *    same device current as the call) and, for PFA_PREC_BF16 and PFA_PREC_F16 (and
 *    the 8-bit calls), some sequence spans at least 2048 key rows, each item's key range is
 *    split over several workgroups whose partial results (32 x head_dim f32 plus
 *    two f32 per row, per wavefront) are merged (the chunk length is chosen from each
 *    item's causally visible key tiles; a call with causal = 0 needs no more than this
 *    size, which assumes a causal call): when no item has more than 4 key
 *    chunks, by the last of its workgroups to finish (then, at the next multiple
 *    of 256 bytes, one 8-byte arrival counter per item, head group and K/V head;
 *    tagged per call, so they need no clearing, and left 0), else by one more
 *    kernel; 0 bytes otherwise.  Calls that share a workspace must not overlap.
 * For PFA_PREC_F32 the partial results are optional: without room for them the
 * call runs without the key split.  Returns 0 when nothing is needed or the
 * arguments are ones the attention calls would reject (pfa_last_error() then
 * says why). */
size_t pfa_workspace_bytes(const int32_t* seq_offsets, int n_seqs, int T, int n_head,
                           int n_head_kv, int head_dim, int precision, int fused);

/*
 * qknorm_rope -- QK-norm followed by NeoX rotary embedding, for Q and K at once.
 *
 * Passages: memra-engine 0.130.0 src/forward.rs, `Model::forward`, QK-norm block
 * (RMSNorm over head_dim rows, one row per (token, head), each row multiplied by
 * the learned q_norm / k_norm vector of length head_dim) and RoPE block (NeoX
 * rotation of Q and K given head_dim, the rotated-dimension count and the
 * frequency base); needle-core v3/model.rs, `rope_at` / `rope` (frequency of
 * pair i = base^(-2i / dims), angle = position x frequency).
 *
 * For every row x of length head_dim (T * n_head rows of Q, T * n_head_kv of K):
 *   y_c = x_c * w_c / sqrt(mean_c(x_c^2) + rms_eps)        (w = q_norm_w or k_norm_w)
 * then, for j < rope_dim / 2, with p the token's position and
 * theta = p * rope_freq_base^(-2j / rope_dim):
 *   (y_j, y_{j+rope_dim/2}) <- (y_j cos theta - y_{j+rope_dim/2} sin theta,
 *                               y_j sin theta + y_{j+rope_dim/2} cos theta)
 * and dimensions rope_dim..head_dim-1 are left as normalised.  The angle is
 * reduced in f64 before its cosine and sine are taken, so long positions keep
 * f32 accuracy.
 *
 *  q_in  [T, n_head*head_dim]     f32, device, read
 *  k_in  [T, n_head_kv*head_dim]  f32, device, read
 *  q_out, k_out  same shapes, f32, device, written; q_out may equal q_in and
 *        k_out may equal k_in (in place); any other overlap is an error.
 *  q_norm_w, k_norm_w  [head_dim] f32, device, read
 *  rms_eps >= 0, rope_freq_base > 0.
 */
int qknorm_rope(const float* q_in, const float* k_in, float* q_out, float* k_out,
                const float* q_norm_w, const float* k_norm_w,
                const int32_t* seq_offsets, int n_seqs,
                int T, int n_head, int n_head_kv, int head_dim, int rope_dim,
                float rope_freq_base, float rms_eps, void* stream);

/*
 * gqa_prefill_attn -- causal grouped-query scaled-dot-product attention.
 *
 * Passages: memra-engine 0.130.0 src/forward.rs, `Model::forward`, SDPA block
 * (query heads n_head over n_head_kv K/V heads, T_q = T_kv = T, causal, scale
 * 1/sqrt(head_dim) from the start of the function); memra-engine 0.101.0
 * src/spec.rs, `full_attn_verify` per-row fallback (row r attends its own key
 * and every earlier one).
 *
 * With g = n_head / n_head_kv, query head h reads K/V head kv = h / g.  For a
 * query token i of sequence s = [a, b), the visible keys are a <= j <= i when
 * `causal` is non-zero, else a <= j < b, and
 *   out[i, h, :] = sum_j softmax_j(scale * q[i,h,:] . k[j,kv,:]) v[j,kv,:].
 *
 *  q    [T, n_head*head_dim]     f32, device, read (already normalised/rotated)
 *  k, v [T, n_head_kv*head_dim]  f32, device, read
 *  out  [T, n_head*head_dim]     f32, device, written; must not overlap q, k, v.
 *  scale  finite; precision  a pfa_precision value.
 *  workspace, workspace_bytes  device memory owned by the caller, 256-byte
 *        aligned, at least pfa_workspace_bytes(seq_offsets, n_seqs, T, n_head,
 *        n_head_kv, head_dim, precision, 0) bytes, not overlapping the tensors; its
 *        contents are overwritten (calls in flight at the same time need separate
 *        workspaces).  Required for the 16-bit modes; optional for PFA_PREC_F32: with
 *        NULL (or too small a workspace) short inputs run without the key split, which
 *        is correct but slower -- about twice as slow at T = 512 with 16 query heads
 *        over 8 K/V heads (the items then cannot fill the GPU).  pfa_attn_plan reports
 *        which plan a given workspace size gets.
 */
int gqa_prefill_attn(const float* q, const float* k, const float* v, float* out,
                     const int32_t* seq_offsets, int n_seqs,
                     int T, int n_head, int n_head_kv, int head_dim,
                     float scale, int causal, int precision,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * gqa_prefill_attn_noalloc -- gqa_prefill_attn for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  The arguments are gqa_prefill_attn's without the workspace; the call uses a
 * device array of pfa_noalloc_scratch_bytes() (64 MiB) that the library itself holds on
 * each GPU it runs on, until the process ends, and calls no allocator.  The results are
 * gqa_prefill_attn's, bit for bit (the same kernels and plan).
 *  A call whose workspace would exceed the array (pfa_workspace_bytes(..., 0) larger than
 *  pfa_noalloc_scratch_bytes(): e.g. the bf16 modes beyond 16384 key rows at 8 K/V heads of
 *  128) fails with PFA_ERR_UNSUPPORTED before anything is enqueued.
 *  Every call on one GPU shares that GPU's array, which keeps what the last call left
 *  (staged tiles, partial results, the key split's arrival counters); nothing needs
 *  clearing between calls (the counters are tagged per call and left 0).  Calls that
 *  overlap in time on one GPU (on different streams, or from different threads) race and
 *  must not be issued.
 */
int gqa_prefill_attn_noalloc(const float* q, const float* k, const float* v, float* out,
                             const int32_t* seq_offsets, int n_seqs, int T, int n_head,
                             int n_head_kv, int head_dim, float scale, int causal, int precision,
                             void* stream);

/* Size in bytes of the per-GPU device array gqa_prefill_attn_noalloc uses. */
size_t pfa_noalloc_scratch_bytes(void);

/*
 * qk_prep_attn -- the whole attention core in one call: qknorm_rope applied to
 * the raw Q and K, then gqa_prefill_attn.  The normalised, rotated Q never goes
 * to memory (each attention workgroup builds its Q rows on chip); K is prepared
 * once per call, into the workspace (bf16: straight into the bf16 tiles; f32:
 * into k_rot_out when given, else the workspace).
 *
 * Passages: as for qknorm_rope and gqa_prefill_attn; needle-core v3/model.rs,
 * cache fill after the prefill (the keys a cache keeps are the normalised,
 * rotated ones) for the optional k_rot_out.
 *
 *  q [T, n_head*head_dim], k, v [T, n_head_kv*head_dim]  raw f32, device, read
 *  out  [T, n_head*head_dim] f32, device, written; must not overlap the inputs.
 *  k_rot_out  NULL, or [T, n_head_kv*head_dim] f32, device: also receives the
 *        normalised, rotated K (what a KV cache would store); must not overlap
 *        the inputs or out.
 *  workspace, workspace_bytes  as for gqa_prefill_attn, at least
 *        pfa_workspace_bytes(..., precision, 1) bytes; for PFA_PREC_F32 it may be
 *        NULL only when k_rot_out is given (short inputs then run without the key
 *        split).
 */
int qk_prep_attn(const float* q, const float* k, const float* v, float* out,
                 const float* q_norm_w, const float* k_norm_w,
                 const int32_t* seq_offsets, int n_seqs,
                 int T, int n_head, int n_head_kv, int head_dim, int rope_dim,
                 float rope_freq_base, float rms_eps, float scale, int causal, int precision,
                 float* k_rot_out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * gqa_chunk_attn -- attention of a block of new query rows over a K/V cache that
 * already holds each sequence's earlier rows (chunked prefill, or verifying a
 * block of drafted tokens).
 *
 * Passages: memra-engine 0.101.0 src/spec.rs, `full_attn_verify` (the block's
 * rows are appended to the cache after base_len rows; row r then attends cache
 * rows 0 .. base_len + r, the per-row fallback spelling out base_len + r + 1
 * keys); needle-core v3/model.rs, cache fill after the prefill (the cache keeps
 * the normalised, rotated keys and the values).
 *
 *  q        [T_q, n_head*head_dim]   f32, device, read: the new rows, already
 *           normalised and rotated at their positions.
 *  k_cache, v_cache  [T_kv, n_head_kv*head_dim]  f32, device, read: sequence s
 *           owns cache rows kv_offsets[s] .. kv_offsets[s+1]-1, of which the
 *           last (q_offsets[s+1] - q_offsets[s]) are its new rows (already in
 *           place) and the ones before them, base_s, its earlier rows.
 *  out      [T_q, n_head*head_dim]   f32, device, written; must not overlap the
 *           other tensors.
 *  gate     NULL, or f32, device, read: a gated output, out = O * sigmoid(gate)
 *           (needle-core v3/model.rs: every output element times the sigmoid of its
 *           gate element; memra-engine 0.101.0 src/spec.rs: the gate split off the
 *           Q projection, or one value per head in its step35 layers), the gate
 *           [T_q, n_head*head_dim] (gate_per_head = 0) or [T_q, n_head] (1), not
 *           overlapping out.
 *  q_offsets, kv_offsets  host arrays of n_seqs+1 cumulative offsets, as
 *           seq_offsets above, both NULL (one sequence) or both given; every
 *           sequence needs at least as many cache rows as new rows.
 *  Row r of sequence s (position base_s + r) sees, when causal, cache rows
 *  0 .. base_s + r of its sequence; otherwise all of them.  base_s = 0 for every
 *  sequence is gqa_prefill_attn.
 *  window  0, or (causal only) a sliding window: row r sees only the last `window`
 *        of those keys, its own included -- cache rows base_s + r - window + 1 ..
 *        base_s + r (memra-engine 0.101.0 src/spec.rs, the step35 MTP layers'
 *        sliding-window view; needle-core v3/model.rs, per-layer attention span).
 *        Negative, or positive without causal: PFA_ERR_INVALID_ARG.
 *  scale, precision, workspace as for gqa_prefill_attn, the workspace sized by
 *  pfa_chunk_workspace_bytes(..., 0).
 */
int gqa_chunk_attn(const float* q, const float* k_cache, const float* v_cache, float* out,
                   const float* gate, int gate_per_head,
                   const int32_t* q_offsets, const int32_t* kv_offsets, int n_seqs,
                   int T_q, int T_kv, int n_head, int n_head_kv, int head_dim,
                   float scale, int causal, int window, int precision,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * qk_prep_chunk_attn -- the whole verify step of a block of new rows in one
 * call: QK-norm + NeoX RoPE of the raw new Q and K at their positions (base_s +
 * r), the rotated K rows and the V rows written into the caller's cache, then
 * gqa_chunk_attn over the cache.
 *
 * Passages: as for gqa_chunk_attn and qknorm_rope.
 *
 *  q [T_q, n_head*head_dim], k, v [T_q, n_head_kv*head_dim]  raw f32, device,
 *        read: the new rows.
 *  k_cache, v_cache  [T_kv, n_head_kv*head_dim] f32, device, read and written:
 *        rows kv_offsets[s] .. kv_offsets[s+1]-1 - len_s hold sequence s's
 *        earlier rows (rotated K, V) and are read; its last len_s rows receive
 *        the new rows' rotated K and V.  They must not overlap each other or the
 *        other tensors.
 *  out  [T_q, n_head*head_dim] f32, device, written.
 *  gate, gate_per_head, window  as for gqa_chunk_attn.
 *  workspace  as for gqa_prefill_attn, sized by pfa_chunk_workspace_bytes(...,
 *        1); PFA_PREC_F32 needs none unless the key split is wanted.
 */
int qk_prep_chunk_attn(const float* q, const float* k, const float* v, float* out,
                       const float* gate, int gate_per_head,
                       const float* q_norm_w, const float* k_norm_w,
                       float* k_cache, float* v_cache,
                       const int32_t* q_offsets, const int32_t* kv_offsets, int n_seqs,
                       int T_q, int T_kv, int n_head, int n_head_kv, int head_dim, int rope_dim,
                       float rope_freq_base, float rms_eps, float scale, int causal, int window,
                       int precision, void* workspace, size_t workspace_bytes, void* stream);

/* Device workspace in bytes that gqa_chunk_attn (fused = 0), qk_prep_chunk_attn
 * (fused = 1) or qk_prep_chunk_attn_tiled (fused = 2) uses for these arguments: as
 * pfa_workspace_bytes, with the bf16 tiles covering each sequence's cache rows (sum_s
 * ceil(kv_len_s / 64) tiles) and the rotary table max_s(kv_len_s) rows; the f32 modes,
 * and the tiled entry (its tiles and table are in kv_tiles), need room only for the
 * key split.  Returns 0 when nothing is needed or the arguments are ones the calls
 * would reject (pfa_last_error() then says why). */
size_t pfa_chunk_workspace_bytes(const int32_t* q_offsets, const int32_t* kv_offsets, int n_seqs,
                                 int T_q, int T_kv, int n_head, int n_head_kv, int head_dim,
                                 int precision, int fused);

/*
 * qk_prep_chunk_attn_tiled -- qk_prep_chunk_attn in the 16-bit modes, keeping the cache's
 * 16-bit K/V tiles across calls.  qk_prep_chunk_attn converts every cache row to the bf16
 * tiles the attention kernel reads, on every call; a caller that appends blocks of rows
 * to the same cache call after call (memra-engine 0.101.0 src/spec.rs,
 * `full_attn_verify`: a block of rows verified against, and appended to, a persistent
 * cache) keeps them in kv_tiles instead, and each call converts only the tiles its new
 * rows fall in.  The result, and what the call writes to k_cache / v_cache, are
 * qk_prep_chunk_attn's, bit for bit, given tiles that hold the cache's earlier rows.
 *
 * Passages: as for qk_prep_chunk_attn.
 *
 *  Arguments as for qk_prep_chunk_attn, precision PFA_PREC_BF16, PFA_PREC_BF16X3 or
 *  PFA_PREC_F16 (PFA_PREC_F32: PFA_ERR_INVALID_ARG), workspace sized by pfa_chunk_workspace_bytes(...,
 *  2) (the key split's partial results only; often 0), and:
 *  kv_tiles  device, read and written, 256-byte aligned, pfa_kv_tiles_bytes(n_slots,
 *        max_rows, n_head_kv, head_dim, precision) bytes, n_slots being this call's
 *        sequence count (1 when the offsets are NULL); owned by the caller, not
 *        overlapping the other tensors or the workspace.  Slot s holds the 16-bit tiles of
 *        sequence s's cache rows 0 .. max_rows-1 (64 rows a tile), then a rotary table of
 *        (cos, sin) pairs by position.  The call stages from k_cache / v_cache -- after
 *        writing its new rows there -- the tiles holding cache rows floor(base_s / 64) *
 *        64 .. kv_len_s - 1 of each sequence with new rows, and their table rows; it
 *        reads the tiles of rows below that from kv_tiles as earlier calls left them.
 *        So every call on one kv_tiles must pass the same sequence count, max_rows,
 *        n_head_kv, head_dim, precision, rope_dim and rope_freq_base, and sequence s's
 *        rows below base_s must have been written by earlier calls on it (a first call
 *        with base_s = 0 writes all of them).  Rows of a sequence beyond its current
 *        kv_len_s in a tile are zeros.
 *  max_rows  >= 1: the most cache rows any sequence may reach (kv_len_s > max_rows:
 *        PFA_ERR_INVALID_ARG).
 */
int qk_prep_chunk_attn_tiled(const float* q, const float* k, const float* v, float* out,
                             const float* gate, int gate_per_head,
                             const float* q_norm_w, const float* k_norm_w,
                             float* k_cache, float* v_cache, void* kv_tiles, int max_rows,
                             const int32_t* q_offsets, const int32_t* kv_offsets, int n_seqs,
                             int T_q, int T_kv, int n_head, int n_head_kv, int head_dim,
                             int rope_dim, float rope_freq_base, float rms_eps, float scale,
                             int causal, int window, int precision, void* workspace,
                             size_t workspace_bytes, void* stream);

/* Bytes of the kv_tiles of qk_prep_chunk_attn_tiled: n_slots slots (1 .. PFA_MAX_SEQS) of
 * ceil(max_rows / 64) tiles per K/V head (K: 64 x head_dim 16-bit values, twice for
 * PFA_PREC_BF16X3; V: 64 x head_dim) and a rotary table of ceil(max_rows / 64) * 64
 * rows of head_dim / 2 (cos, sin) f32 pairs.  0 (and pfa_last_error()) for arguments the
 * call would reject. */
size_t pfa_kv_tiles_bytes(int n_slots, int max_rows, int n_head_kv, int head_dim, int precision);

/*
 * 8-bit quantised sessions
 * ------------------------
 * Passages: needle-core v3/model.rs, `quant_rows` (a quantised session
 * quantises every (token, head) row of the query, the keys and the values with
 * 8 bits right after RoPE, before attention and before the cache write),
 * `quantize_rows` and its int8 K/V store (integer rows plus one scale per row,
 * the form decode reads; the store's reader takes the scales out of the dot
 * products).  The page prints neither quantiser's body.  This library's reading of
 * the rule (symmetric, 8 bits, one scale per row), in IEEE single precision: a row's
 * scale is its largest magnitude / 127; a value's code is the nearest integer to
 * value / scale, ties to even, within -127..127; a row of zeros has scale 0 and codes
 * 0.  The divisor 127 and the tie direction are choices of that reading, not
 * statements of the page.  A value of the store is code * scale.
 *
 * An 8-bit store of `heads` heads over `rows` rows is a pair of device arrays:
 * codes int8 [rows, heads*head_dim] (16-byte aligned) and scales f32
 * [rows, heads], row-major like the f32 tensors.
 */

/*
 * pfa_quantize_rows -- quantise n_rows rows of row_len floats (one row per
 * (token, head) when row_len is the head size).
 *  x       [n_rows, row_len] f32, device, read.
 *  codes   [n_rows, row_len] int8, device, written.
 *  scales  [n_rows] f32, device, written.
 *  x_fq    NULL, or [n_rows, row_len] f32, device, written: the fake-quantised
 *          values code * scale; may be x itself (in place, as `quant_rows`
 *          does), otherwise must not overlap x.  codes, scales and x_fq must not
 *          overlap each other or x.
 *  1 <= row_len <= 65536, n_rows * row_len <= 2^40; n_rows == 0 is a no-op.
 */
int pfa_quantize_rows(const float* x, int64_t n_rows, int row_len, int8_t* codes,
                      float* scales, float* x_fq, void* stream);

/*
 * gqa_attn_q8 -- gqa_chunk_attn through 8-bit stores: the scores are the
 * integer dot products of the Q and K codes (exact) times the two row scales
 * and `scale`; the weights multiply the dequantised V rows.  Plain prefill is
 * q_offsets = kv_offsets (or both NULL with T_q = T_kv).
 *  q, q_scale  8-bit store of the query rows, [T_q, n_head*head_dim] codes and
 *        [T_q, n_head] scales, device, read.
 *  k_cache, k_scale, v_cache, v_scale  8-bit stores of the keys and values,
 *        [T_kv, n_head_kv*head_dim] codes and [T_kv, n_head_kv] scales, device,
 *        read; sequence s owns rows kv_offsets[s] .. kv_offsets[s+1]-1, its new
 *        rows last, as for gqa_chunk_attn.
 *  out   [T_q, n_head*head_dim] f32, device, written; must not overlap the rest.
 *  gate, gate_per_head, q_offsets, kv_offsets, n_seqs, causal, window  as for
 *        gqa_chunk_attn.
 *  scale  finite and > 0 (the row scales are applied inside the exponent).
 *  The scores are exact integer dot products (int8 matrix cores for head_dim 128;
 *  for 64, codes in bf16 on bf16 matrix cores, where every partial sum is an
 *  integer below 2^24); V is dequantised and rounded to bf16, and the weights are
 *  rounded to bf16, as in PFA_PREC_BF16.
 *  workspace  device, 256-byte aligned, pfa_q8_workspace_bytes(..., 0) bytes.
 */
int gqa_attn_q8(const int8_t* q, const float* q_scale, const int8_t* k_cache,
                const float* k_scale, const int8_t* v_cache, const float* v_scale, float* out,
                const float* gate, int gate_per_head, const int32_t* q_offsets,
                const int32_t* kv_offsets, int n_seqs, int T_q, int T_kv, int n_head,
                int n_head_kv, int head_dim, float scale, int causal, int window,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * qk_prep_attn_q8 -- a quantised session's attention step in one call: QK-norm +
 * NeoX RoPE of the raw new Q and K at their positions (as qk_prep_chunk_attn),
 * then Q, K and V quantised per (token, head); the K and V codes and scales go
 * into the last rows of each sequence's range of the caller's 8-bit store, the
 * Q codes into the workspace, and gqa_attn_q8 runs over the store.
 *  q [T_q, n_head*head_dim], k, v [T_q, n_head_kv*head_dim]  raw f32, device, read.
 *  k_cache, k_scale, v_cache, v_scale  the 8-bit K/V store over T_kv rows, device,
 *        read and written as k_cache / v_cache of qk_prep_chunk_attn; none may
 *        overlap another tensor.
 *  out, gate, gate_per_head, offsets, window  as for gqa_chunk_attn; scale as for
 *        gqa_attn_q8.
 *  workspace  device, 256-byte aligned, pfa_q8_workspace_bytes(..., 1) bytes.
 */
int qk_prep_attn_q8(const float* q, const float* k, const float* v, float* out,
                    const float* gate, int gate_per_head,
                    const float* q_norm_w, const float* k_norm_w,
                    int8_t* k_cache, float* k_scale, int8_t* v_cache, float* v_scale,
                    const int32_t* q_offsets, const int32_t* kv_offsets, int n_seqs,
                    int T_q, int T_kv, int n_head, int n_head_kv, int head_dim, int rope_dim,
                    float rope_freq_base, float rms_eps, float scale, int causal, int window,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Device workspace in bytes of gqa_attn_q8 (fused = 0) or qk_prep_attn_q8
 * (fused = 1): K/V tiles over each sequence's store rows (sum_s ceil(kv_len_s /
 * 64) tiles per K/V head, each 64 * head_dim bytes of K codes for head_dim 128 or
 * 64 * head_dim * 2 of bf16 K for 64, plus 64 * head_dim * 2 of bf16 V), 256 bytes
 * of key scales per tile and head, (fused) the Q codes and scales, and the key
 * split's partial results.  0 when T_q == 0 or the arguments would be
 * rejected (pfa_last_error() then says why). */
size_t pfa_q8_workspace_bytes(const int32_t* q_offsets, const int32_t* kv_offsets, int n_seqs,
                              int T_q, int T_kv, int n_head, int n_head_kv, int head_dim,
                              int fused);

/*
 * Plan report
 * -----------
 * What an attention call would enqueue for given arguments, decided by the same host
 * code the entry point runs; nothing is enqueued and no device is needed (the key split
 * is planned for the current device's compute units, 256 when none is visible).  For
 * tools and tests: profilers name the kernels, and the work schedule can be checked.
 *
 * `entry` picks the entry point.  The arguments are the call's: for the prefill entries
 * q_offsets is seq_offsets and kv_offsets / T_kv are ignored; rope_dim matters for the
 * entries that prepare Q and K; window for the chunk and 8-bit entries; precision is
 * ignored by the 8-bit ones.  has_k_rot_out: qk_prep_attn is given a k_rot_out.
 * workspace_bytes: the workspace the call will be given (0: none; SIZE_MAX: enough).
 * It matters only for PFA_PREC_F32, which drops the key split when the workspace has no
 * room for the partial results.
 */
typedef enum {
    PFA_ENTRY_PREFILL = 0,    /* gqa_prefill_attn */
    PFA_ENTRY_PREP = 1,       /* qk_prep_attn */
    PFA_ENTRY_CHUNK = 2,      /* gqa_chunk_attn */
    PFA_ENTRY_CHUNK_PREP = 3, /* qk_prep_chunk_attn */
    PFA_ENTRY_Q8 = 4,         /* gqa_attn_q8 */
    PFA_ENTRY_Q8_PREP = 5,    /* qk_prep_attn_q8 */
    PFA_ENTRY_CHUNK_TILED = 6 /* qk_prep_chunk_attn_tiled */
} pfa_entry;

typedef struct {
    int items;               /* (sequence, query super-block) work items, longest first */
    int rows_per_item;       /* query rows of a super-block */
    int waves_per_workgroup; /* wavefronts of an attention workgroup */
    int tile_keys;           /* keys per K/V tile */
    int key_chunk_tiles;     /* key split: tiles per key chunk (0: not split) */
    int max_key_chunks;      /* key chunks of the longest item (1: not split) */
    int paired;              /* f32: attention workgroup j takes items j and items-1-j */
    int merge_in_place;      /* key split merged by each item's last workgroup (no extra
                                kernel); 0: by attn_combine_kernel, or not split */
    int64_t workgroups;      /* grid of the attention kernel */
    size_t workspace_bytes;  /* device workspace the call uses */
    char kernels[320];       /* kernels enqueued, in launch order, joined by " + " */
} pfa_plan;

/* Fills *plan.  Returns PFA_OK, or the status the entry point would return for these
 * arguments (pfa_last_error() says why).  T_q == 0: a zeroed plan. */
int pfa_attn_plan(int entry, const int32_t* q_offsets, const int32_t* kv_offsets, int n_seqs,
                  int T_q, int T_kv, int n_head, int n_head_kv, int head_dim, int rope_dim,
                  int causal, int window, int precision, int has_k_rot_out,
                  size_t workspace_bytes, pfa_plan* plan);

/* The work unit of every attention workgroup, decoded on the host by the kernels' own
 * code.  One record of PFA_UNIT_FIELDS int32 per (workgroup, item it takes): workgroup
 * index, pass (1 for the second item of a paired workgroup, else 0), item (its index in
 * the longest-first order), sequence, super-block of the sequence, key chunk, K/V head,
 * head chunk of the group, first key tile, end key tile (tiles of tile_keys keys counted
 * from the sequence's first key row; first >= end: the workgroup exits at once).
 * Writes at most max_records records (host array `records`) and returns how many there
 * are, or a negative pfa_status. */
#define PFA_UNIT_FIELDS 10
int64_t pfa_attn_units(int entry, const int32_t* q_offsets, const int32_t* kv_offsets,
                       int n_seqs, int T_q, int T_kv, int n_head, int n_head_kv, int head_dim,
                       int rope_dim, int causal, int window, int precision, int has_k_rot_out,
                       size_t workspace_bytes, int32_t* records, int64_t max_records);

/* Message for the last non-OK return on the calling thread ("" if none). */
const char* pfa_last_error(void);

/* Library version string. */
const char* pfa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PFA_H */
