/*
 * spd.h -- C ABI of the prompt-deduplicated split-attention library (libspd.so)
 * for AMD Instinct MI355X (gfx950).
 *
 * The operations follow "How Prompt Deduplication Works":
 *   spd_group            -- Core Algorithm, "Finding Prompt Groups"
 *   spd_pack             -- Core Algorithm, "Creating Deduplicated Batch";
 *                           "Working with Packed/Unpacked Sequences"
 *   spd_pack_rows        -- the same packing applied to per-token rows
 *   spd_split_attn_fwd   -- Phase 2, "Split Attention Optimization"
 *   spd_split_attn_bwd   -- "Correctness & Gradients" (gradients flow through
 *                           the deduplicated computation)
 *   spd_reconstruct      -- Core Algorithm, "Reconstructing Original Batch";
 *                           Phase 3, "Transparent Reconstruction"
 *   spd_reconstruct_bwd, spd_pack_rows_bwd
 *                        -- "Correctness & Gradients": gradients flow back
 *                           through the reconstruction and the deduplication
 *   spd_group_singletons, spd_repack_rows, spd_repack_rows_bwd
 *                        -- Phase 2, "Standard QKV Optimization": Q, K, V of
 *                           the deduplicated batch reconstructed to the full
 *                           batch for standard causal attention
 *   spd_mask_to_varlen, spd_varlen_params
 *                        -- "Flash Attention Integration": variable-length
 *                           (cu_seqlens) parameters
 *
 * Conventions shared by every call
 * --------------------------------
 * - Pointers named as device pointers must be device memory of the current
 *   HIP device, 16-byte aligned, contiguous, row-major.  The library never
 *   allocates, frees or keeps a pointer after the call returns: the caller
 *   owns every buffer, including workspaces sized by the *_workspace_bytes
 *   queries.
 * - Every call is asynchronous on the given stream (a hipStream_t passed as
 *   void*; NULL = the null stream) and keeps no state between calls (apart
 *   from the opt-in, per-thread kernel timing at the end of this header and
 *   the fixed scratch array of spd_split_attn_fwd_noalloc), so calls on
 *   different streams may run concurrently on disjoint buffers.
 * - Arguments are validated on the host before anything is launched; a
 *   non-zero spd_status is returned and nothing runs.  SPD_ERR_HIP means a
 *   launch failed (hipGetLastError after the launch); spd_last_hip_error()
 *   gives the HIP code.
 * - Index arrays are int32 (packed rows, batch rows and (b*S+t) indices all
 *   stay below 2^31); byte offsets inside kernels are 64-bit.
 * - A buffer with zero rows -- every [T, ...] buffer when T = 0, e.g. a batch
 *   whose every token unpad removed -- may be NULL; the other arguments are
 *   checked as usual, and calls that write [B, S, ...] outputs (reconstruct,
 *   the backward of pack_rows) still write them (all zeros).
 *
 * Notation: B samples, S padded sequence length, P = S - response_length
 * prompt columns, G groups, T packed tokens, Hq / Hkv query / key-value heads,
 * d head dimension.
 */
#ifndef SPD_H
#define SPD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum spd_status {
  SPD_OK = 0,
  SPD_ERR_INVALID_ARG = -1, /* null pointer, negative or inconsistent size */
  SPD_ERR_UNSUPPORTED = -2, /* a shape or dtype this build does not handle */
  SPD_ERR_ALIGNMENT = -3,   /* pointer or row size not a multiple of 16 bytes */
  SPD_ERR_WORKSPACE = -4,   /* workspace null or smaller than the query says */
  SPD_ERR_HIP = -5          /* a HIP launch failed */
} spd_status;

typedef enum spd_dtype { SPD_F32 = 0, SPD_BF16 = 1 } spd_dtype;

/*
 * The deduplication plan: device arrays owned by the caller, filled by
 * spd_group (group arrays) and spd_pack (segment arrays).  Capacities depend
 * only on B and S, so everything can be allocated before the number of groups
 * G or packed tokens T is known.  counts[0] = G and counts[1] = T are written
 * on the device; the caller reads them back when it needs host copies.
 *
 * Segments: group g's prompt occupies packed rows
 * [prompt_off[g], prompt_off[g] + prompt_len[g]); its members' responses
 * follow in ascending sample order, sample b at [resp_off[b], resp_off[b] +
 * resp_len[b]).  seg_start[j] is the first row of the segment containing j.
 */
typedef struct spd_plan {
  int64_t B;            /* host: samples */
  int64_t S;            /* host: padded sequence length */
  int64_t P;            /* host: prompt columns, S - response_length */
  int32_t *group_of;    /* [B]     group of each sample */
  int32_t *grp_off;     /* [B + 1] CSR offsets of groups (first G + 1 used) */
  int32_t *grp_idx;     /* [B]     members, grouped, ascending within a group */
  int32_t *rep;         /* [B]     first member of each group (first G used) */
  int32_t *prompt_off;  /* [B]     packed start of each group's prompt */
  int32_t *prompt_len;  /* [B]     packed prompt tokens of each group */
  int32_t *resp_off;    /* [B]     packed start of each sample's response */
  int32_t *resp_len;    /* [B]     packed response tokens of each sample */
  int32_t *src;         /* [B * S] capacity; packed row j -> b * S + t (first T used) */
  int32_t *dst;         /* [B * S] (b, t) -> packed row, or -1 if no packed token maps */
  int32_t *seg_start;   /* [B * S] capacity; first packed row of j's segment */
  int32_t *counts;      /* [8]     counts[0] = G, counts[1] = T, counts[2] = batch cells mapped to
                                     no packed row (unpad mode), counts[3] = packed rows whose
                                     attention-mask entry is 0 (padded mode with a mask),
                                     counts[4] = L0, prompt columns of a shared prefix (0: none),
                                     counts[5] = packed rows of that prefix, [6..7] reserved */
  int32_t padded_with_mask; /* host: written by spd_pack -- 1 when it packed in padded mode
                                     (use_unpad = 0) with an attention mask, so pads may sit among
                                     the packed rows; 0 otherwise.  The attention calls reject a
                                     plan with this flag set (see spd_split_attn_fwd).  A caller
                                     that has read counts[3] == 0 (no pad was kept) may clear it. */
} spd_plan;

/* ---------------------------------------------------------------- grouping */

/* Workspace bytes spd_group needs for a batch of B rows of S tokens. */
size_t spd_group_workspace_bytes(int64_t B, int64_t S);

/*
 * Group samples by identical prompt ("Finding Prompt Groups").
 *   input_ids        device int64 [B, S].
 *   response_length  the response columns; the prompt is the first
 *                    P = S - response_length columns of every row
 *                    (0 <= response_length <= S; plan->P must equal P).
 *   plan             writes group_of, grp_off, grp_idx, rep, counts[0] = G.
 *                    Groups are numbered in order of first occurrence and list
 *                    their members ascending; two rows group together exactly
 *                    when all P prompt ids are equal (a hash narrows the
 *                    candidates, a full comparison decides).
 *   unique_prompts   optional (NULL to skip) device int64 with capacity
 *                    [B, P]; row g < G receives group g's prompt ids.
 * Constraints: 1 <= B <= 65536, B * S < 2^31.
 */
spd_status spd_group(const int64_t *input_ids, int64_t B, int64_t S, int64_t response_length,
                     const spd_plan *plan, int64_t *unique_prompts,
                     void *workspace, size_t workspace_bytes, void *stream);

/* ----------------------------------------------------------------- packing */

/*
 * Workspace bytes spd_pack needs (device memory, caller-owned, any contents):
 * 2 B int32 for the segment-offset scan plus 3 int32 per 1024 columns of every
 * row for the unpadded pack's per-chunk kept counts, each part rounded up to
 * 256 bytes.  0 when B < 1 or S < 1.
 */
size_t spd_pack_workspace_bytes(int64_t B, int64_t S);

/*
 * Build the packed sequence ("Creating Deduplicated Batch"), after spd_group
 * on the same plan.  Order: [prompt of group 0][responses of its members,
 * ascending][prompt of group 1]...  The prompt copy packed for a group, and
 * its positions and mask, are its first member's.
 *   input_ids, position_ids  device int64 [B, S]; positions are gathered,
 *                            not renumbered.
 *   attention_mask           device [B, S] of mask_elem_bytes-byte integers
 *                            (1, 4 or 8), non-zero = valid; may be NULL when
 *                            use_unpad == 0 (padded mode keeps every token).
 *   use_unpad                1: drop tokens whose mask is 0 ("Unpacked
 *                            Format"); 0: keep every token.
 *   dedup_ids, dedup_pos     device int64 with capacity B * S; the first T
 *                            entries receive the packed ids and positions.
 * Writes prompt_off, prompt_len, resp_off, resp_len, src, dst, seg_start,
 * counts[1] = T, counts[2] (cells left out by unpad) and counts[3] (packed
 * rows whose mask entry is 0: padded mode with a mask keeps such pads in the
 * packed sequence, where they are no sample's tokens).  On the host it sets
 * plan->padded_with_mask (1 for use_unpad == 0 with a mask, else 0).
 * Attention over such a batch (Working with Packed/Unpacked Sequences: pads
 * take no part) runs on the same batch packed with use_unpad = 1 -- a second
 * plan with the same group arrays -- with the rows moved between the two
 * layouts by spd_repack_rows (pads come back as zeros).
 */
spd_status spd_pack(const int64_t *input_ids, const int64_t *position_ids,
                    const void *attention_mask, int32_t mask_elem_bytes, int32_t use_unpad,
                    spd_plan *plan, int64_t *dedup_ids, int64_t *dedup_pos,
                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * Pack per-token rows with the plan: packed[j, :] = rows[src[j], :].
 *   rows       device [B, S, row_bytes] (any element type; copied as bytes).
 *   packed     device [T, row_bytes].
 *   T          the packed length (counts[1] of the plan).
 * row_bytes must be a positive multiple of 16.
 */
spd_status spd_pack_rows(const spd_plan *plan, int64_t T, const void *rows, int64_t row_bytes,
                         void *packed, void *stream);

/*
 * Reconstruct the batch ("Reconstructing Original Batch"):
 * out[b, t, :] = packed[dst[b * S + t], :], or zeros where dst is -1.  Each
 * packed prompt row is read once and written to every member of its group.
 *   packed     device [T, row_bytes].
 *   out        device [B, S, row_bytes].
 * row_bytes must be a positive multiple of 16.
 */
spd_status spd_reconstruct(const spd_plan *plan, int64_t T, const void *packed, int64_t row_bytes,
                           void *out, void *stream);

/*
 * Backward of spd_reconstruct ("Correctness & Gradients": the gradient flows
 * back through the reconstruction).  reconstruct is linear, so its adjoint:
 *   dpacked[j, :] = sum over every (b, t) with dst[b * S + t] == j of dout[b, t, :].
 * A packed prompt row thus receives the sum over all members of its group
 * (column t of each), added in ascending member order in fp32 and rounded
 * once (round-to-nearest-even for bf16); a response row receives its own
 * (b, t)'s gradient.  Rows of dout that map nowhere (unpad pads) are ignored.
 *   dout       device [B, S, row_bytes], elements of type dtype.
 *   dtype      SPD_F32 or SPD_BF16 (else SPD_ERR_UNSUPPORTED).
 *   dpacked    device [T, row_bytes], same dtype; every row is written.
 * row_bytes must be a positive multiple of 16.
 */
spd_status spd_reconstruct_bwd(const spd_plan *plan, int64_t T, const void *dout, int64_t row_bytes,
                               int32_t dtype, void *dpacked, void *stream);

/*
 * Backward of spd_pack_rows (the adjoint of packed[j] = rows[src[j]]):
 *   drows[src[j], :] = dpacked[j, :] for every packed row j, and zeros in every
 * other (b, t) -- the prompt columns of group members other than the one the
 * prompt was taken from, and rows that map nowhere (unpad pads).  Bytes are
 * copied, so any element type works.
 *   dpacked    device [T, row_bytes].
 *   drows      device [B, S, row_bytes]; every row is written.
 * row_bytes must be a positive multiple of 16.
 */
spd_status spd_pack_rows_bwd(const spd_plan *plan, int64_t T, const void *dpacked, int64_t row_bytes,
                             void *drows, void *stream);

/*
 * Shared prompt prefix ("Key Limitations & Future Work": prefix caching for
 * partially overlapping prompts).  After spd_group: counts[4] = L0, the number
 * of leading prompt columns on which the first members of all groups agree
 * (0 with fewer than two groups).  spd_pack then packs those columns once,
 * from the first sample, ahead of every group -- [prefix][prompt 1][responses
 * of 1][prompt 2]... with prompt g now its columns L0..P-1 -- and every call
 * that takes the plan (attention, reconstruct, row moves) treats the prefix
 * rows as part of every sample's sequence.  Without this call spd_group
 * leaves counts[4] = 0 (no prefix level).
 */
spd_status spd_share_prefix(const int64_t *input_ids, int64_t B, int64_t S, int64_t response_length,
                            const spd_plan *plan, void *stream);

/*
 * The plan of the non-deduplicated batch: every sample is its own group
 * (group_of[b] = rep[b] = b, counts[0] = B), no hashing.  spd_pack with this
 * plan lays the batch out sample by sample -- each sample's prompt, then its
 * response -- which is the full batch in variable-length form, and the split
 * attention calls on it compute standard per-sample causal attention (the
 * "Standard QKV Optimization" of Phase 2).  Same argument rules as spd_group.
 */
spd_status spd_group_singletons(int64_t B, int64_t S, int64_t response_length, const spd_plan *plan,
                                void *stream);

/*
 * Moves rows between the packed layouts of two plans of the same batch (same
 * B, S, P and attention mask):
 *   out[j, :] = in[from.dst[to.src[j]], :]     (zeros if that cell has no row in "from")
 * e.g. deduplicated Q -> the full batch (to = singleton plan), or the full
 * batch's attention output -> the deduplicated layout (to = deduplicated plan;
 * a prompt row takes the copy of the member it was packed from).
 *   in         device [T_from, row_bytes] (any element type; copied as bytes).
 *   out        device [T_to, row_bytes].
 * row_bytes must be a positive multiple of 16.
 */
spd_status spd_repack_rows(const spd_plan *to, int64_t T_to, const spd_plan *from, int64_t T_from,
                           const void *in, int64_t row_bytes, void *out, void *stream);

/*
 * Backward of spd_repack_rows (its transpose):
 *   din[i, :] = sum over rows j of "to" with from.dst[to.src[j]] == i of dout[j, :],
 * summed in ascending member order in fp32 and rounded once.  From the
 * deduplicated layout to the full batch, a prompt row collects every member's
 * copy; from the full batch to the deduplicated layout, only the copy of the
 * member the prompt row was packed from receives the gradient (others 0).
 *   dout       device [T_to, row_bytes], elements of type dtype (SPD_F32 or SPD_BF16).
 *   din        device [T_from, row_bytes], same dtype; every row is written.
 */
spd_status spd_repack_rows_bwd(const spd_plan *to, int64_t T_to, const spd_plan *from, int64_t T_from,
                               const void *dout, int64_t row_bytes, int32_t dtype, void *din, void *stream);

/* ------------------------------------------------- variable-length parameters */

/* Workspace bytes of spd_mask_to_varlen for total_q query rows. */
size_t spd_mask_varlen_workspace_bytes(int64_t total_q);

/*
 * "Flash Attention Integration": a block-diagonal [total_q, total_kv] attention
 * mask (row = query, column = key, non-zero = visible) -> cu_seqlens.  Block i
 * owns query rows [cu_seqlens_q[i], cu_seqlens_q[i+1]) and keys
 * [cu_seqlens_k[i], cu_seqlens_k[i+1]).  A row's block is named by its first
 * visible key; a row that sees no key belongs to the block of the next row
 * that sees one (trailing ones to the last block); the last key boundary is
 * one past the last visible key.
 *   mask             device [total_q, total_kv], elements of mask_elem_bytes
 *                    (1, 2, 4 or 8) bytes; row-major, contiguous.
 *   cu_seqlens_q/k   device int32 [total_q + 1]; entries 0..num_seqs written.
 *   stats            device int32 [4]: num_seqs, max_seqlen_q, max_seqlen_k,
 *                    and the number of rows whose visible keys leave their
 *                    block's range (0 for a block-diagonal mask; the caller
 *                    decides whether that is an error).
 * total_q < 2^31 and total_kv * mask_elem_bytes < 2^31, else
 * SPD_ERR_UNSUPPORTED.
 */
spd_status spd_mask_to_varlen(const void *mask, int32_t mask_elem_bytes, int64_t total_q, int64_t total_kv,
                              int32_t *cu_seqlens_q, int32_t *cu_seqlens_k, int32_t *stats, void *workspace,
                              size_t workspace_bytes, void *stream);

/*
 * The variable-length parameters of the two attention calls of Phase 2
 * ("Split Attention Optimization") for a packed batch:
 *   cu_seqlens_prompt  device int32 [B + 1]; entries 0..G: prompt-to-prompt,
 *                      over the unique prompts (queries and keys alike).
 *   cu_seqlens_q       device int32 [B + 1]: response-to-full queries, each
 *                      sample's response rows.
 *   cu_seqlens_k       device int32 [B + 1]: response-to-full keys, each
 *                      sample's prompt followed by its response (the full
 *                      batch laid out sample by sample).
 *   max_seqlens        device int32 [3]: longest prompt, response, prompt +
 *                      response.
 */
spd_status spd_varlen_params(const spd_plan *plan, int32_t *cu_seqlens_prompt, int32_t *cu_seqlens_q,
                             int32_t *cu_seqlens_k, int32_t *max_seqlens, void *stream);

/* ---------------------------------------------------------- split attention */

typedef struct spd_attn_desc {
  int32_t num_q_heads;   /* Hq */
  int32_t num_kv_heads;  /* Hkv; Hq % Hkv == 0, query head h reads kv head h / (Hq / Hkv) */
  int32_t head_dim;      /* d: 64 or 128 */
  int32_t dtype;         /* spd_dtype of q, k, v, o, dout, dq, dk, dv */
  float softmax_scale;   /* usually 1 / sqrt(d); must be > 0 */
} spd_attn_desc;

/*
 * Workspace bytes spd_split_attn_bwd needs for T packed rows of a B-sample
 * plan (also enough for the forward).  For bf16 it includes the partial-sum
 * slots for split key tiles: min(64, 1024 / Hkv) slots of 256 keys x Hkv x d
 * fp32, for dk and for dv (128 MiB at Hkv 8, d 128; at most 256 MiB).
 * Returns 0 for an invalid descriptor, B < 1 or T < 0.
 */
size_t spd_attn_workspace_bytes(const spd_attn_desc *desc, int64_t B, int64_t T);

/*
 * Workspace bytes spd_split_attn_fwd needs: the query-tile list and the
 * planner's scratch only, about 100 bytes per 128 packed rows plus 8 bytes
 * per sample.  Returns 0 for an invalid descriptor, B < 1 or T < 0.
 */
size_t spd_attn_fwd_workspace_bytes(const spd_attn_desc *desc, int64_t B, int64_t T);

/*
 * Split attention forward ("Split Attention Optimization").  In the packed
 * batch, a prompt row i of group g attends causally to its prompt's rows
 * 0..i; a response row i of sample b attends to all of its group's prompt
 * rows and to its own response rows 0..i, never to another group or a
 * sibling response.  This equals causal attention over each sample's own
 * [prompt][response] sequence.
 *   q        device [T, Hq, d];  k, v  device [T, Hkv, d]  (dtype of desc)
 *   o        device [T, Hq, d]   softmax(scale q k^T) v, same dtype
 *   lse      device float [Hq, T]  natural-log softmax denominator per row,
 *            kept for the backward
 *   T        the packed length written by spd_pack (rows >= T are never read)
 *   workspace at least spd_attn_fwd_workspace_bytes(desc, plan->B, T) bytes
 * bf16 runs on matrix cores with fp32 accumulation and one rounding of o;
 * fp32 is a plain-arithmetic path for small problems.
 * Limits: T * Hkv * d * (element bytes) < 2^32 (the key/value tensors stay
 * within 4 GiB: 2,097,151 rows at Hkv 8, d 128, bf16) and Hq * T * d < 2^40,
 * else SPD_ERR_UNSUPPORTED.  A plan with padded_with_mask set is rejected
 * with SPD_ERR_UNSUPPORTED: its pads would otherwise be attended as tokens.
 */
spd_status spd_split_attn_fwd(const spd_attn_desc *desc, const spd_plan *plan, int64_t T,
                              const void *q, const void *k, const void *v, void *o, float *lse,
                              void *workspace, size_t workspace_bytes, void *stream);

/*
 * spd_split_attn_fwd without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  It allocates nothing (no hipMalloc, no
 * allocating library routine); its scratch -- the query-tile list -- lives in
 * a fixed device array of 4 MiB (4,194,304 bytes) inside the library, one
 * per device, held until the process ends.  The
 * caller still passes every input and output.  Same arguments, rules and
 * results (bitwise) as spd_split_attn_fwd; sizes whose forward workspace
 * (spd_attn_fwd_workspace_bytes) exceeds the array return SPD_ERR_WORKSPACE
 * (e.g. about 4.2 million packed rows in bf16 at 8 query heads per kv head,
 * 2.8 million in fp32; fewer with many samples, about 200 bytes per sample).  The first call on a device looks
 * up the array's address there (SPD_ERR_HIP if that fails).  Every call on one
 * device shares the array: calls that overlap on one device (different
 * streams, or threads without ordering) race and must be serialised by the
 * caller; calls in order on one stream are safe.
 */
spd_status spd_split_attn_fwd_noalloc(const spd_attn_desc *desc, const spd_plan *plan, int64_t T,
                                      const void *q, const void *k, const void *v, void *o, float *lse,
                                      void *stream);

/*
 * Split attention backward ("Correctness & Gradients").  Given o and lse from
 * the forward and dout = dL/do, writes dq [T, Hq, d], dk, dv [T, Hkv, d].
 * A prompt key's dk / dv sum over the prompt's own causal queries and every
 * response row of its group; query heads sharing a kv head add into it.
 * Accumulation is fp32 and each output is rounded once.  Sums run in a fixed
 * order (a key read by very many rows is split over several blocks whose fp32
 * partial sums are added in chunk order), so results are bitwise reproducible
 * run to run.  The workspace (spd_attn_workspace_bytes) holds per-row
 * statistics, the tile lists and, for bf16, the partial-sum slots.  Same
 * limits and padded_with_mask rule as the forward.
 */
spd_status spd_split_attn_bwd(const spd_attn_desc *desc, const spd_plan *plan, int64_t T,
                              const void *q, const void *k, const void *v, const void *o,
                              const float *lse, const void *dout, void *dq, void *dk, void *dv,
                              void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------ kernel timing */

/*
 * Opt-in timing of the library's main kernels with HIP events recorded on the
 * stream each kernel is launched on (for benchmarks; per host thread).
 * Between spd_profile_begin() and spd_profile_end() every entry point records
 * an event pair around each of its main kernels, at most 1024 launches per
 * kernel.  spd_profile_end() waits for those events, writes per kernel id the
 * number of timed launches and their summed milliseconds into arrays of
 * SPD_K_COUNT entries, and stops recording.  When no profile is active the
 * entry points record nothing.
 */
enum {
  SPD_K_FWD = 0,          /* split-attention forward kernel */
  SPD_K_BWD_PRE = 1,      /* backward: rowsum(dO * O) */
  SPD_K_BWD_DQ = 2,       /* backward: dq kernel */
  SPD_K_BWD_DKDV = 3,     /* backward: dk / dv kernel */
  SPD_K_RECONSTRUCT = 4,  /* reconstruct gather (and the zero fill) */
  SPD_K_PACK_ROWS = 5,    /* row packing gather */
  SPD_K_RECONSTRUCT_BWD = 6,  /* backward of reconstruct: segment sum */
  SPD_K_PACK_ROWS_BWD = 7,    /* backward of pack_rows: scatter (and the zero fill) */
  SPD_K_MASK_VARLEN = 8,      /* spd_mask_to_varlen: all four launches */
  SPD_K_COUNT = 9
};
spd_status spd_profile_begin(void);
spd_status spd_profile_end(int64_t *launches, double *total_ms);

/* ------------------------------------------------------------------- misc */

const char *spd_status_string(spd_status status);
int spd_last_hip_error(void);   /* HIP error code behind the last SPD_ERR_HIP on this thread */
int spd_version(void);          /* major * 10000 + minor * 100 + patch */

#ifdef __cplusplus
}
#endif

#endif /* SPD_H */
