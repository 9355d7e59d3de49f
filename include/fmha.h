/*
 * fmha.h -- C ABI of libfmha.so, fused multi-head attention for AMD MI355X
 * (gfx950, CDNA4).
 *
 * What every entry point computes.  For batch b, query head h and query row
 * i (0 <= i < T), with kv = h / (n_h / n_kv_h) and pos_i = s_k - T + i (the
 * T queries are the last T positions of the sequence):
 *
 *   key j is visible iff j < s_k and (causal == 0 or j <= pos_i)
 *                        and (window == 0 or j > pos_i - window)
 *   s_j   = scale * <Q[b,i,h,:], K[b,j,kv,:]>
 *   O     = sum_j softmax(s)_j * V[b,j,kv,:]   over visible j
 *   lse   = ln sum_j exp(s_j)                  over visible j (natural log)
 *
 * Sources (nvfp4-megamoe-kernel pages, directory dsv4/):
 *   - "CURRENT_ISSUE.md: UMMA FMHA -- Full Pipeline + Production",
 *     section "What's working": the fused QK -> softmax -> PV pipeline;
 *     section "Key lessons": the product Q.K is taken unscaled and the
 *     1/sqrt(HD) factor is applied in the softmax (here `scale`, which the
 *     caller sets, normally to 1/sqrt(hd));
 *     section "Next steps", item 4: KV lengths over many tiles combined by
 *     the D5 merge O = sum_i exp(lse_i) O_i / sum_i exp(lse_i).
 *   - commit log at e4ee9fdc: one workgroup grid over (head, batch), MQA
 *     expressed as a K/V head stride of 0, a pure C API loaded through
 *     ctypes, one launch with no device synchronisation, the multi-tile
 *     kernel's running max / running sum (online softmax) over KV tiles.
 *   - commit log at 593bc25a: the sliding-window mask (D3) and the causal
 *     mask (D4) of the reference kernel.
 * A row with no visible key yields O = 0 and lse = -inf.
 *
 * Conventions shared by all entry points
 *   - Element types: q, k, v and o are bfloat16 bit patterns (uint16_t in
 *     memory); lse, o_part and lse_part are float32.  Accumulation and the
 *     softmax are float32; o is rounded to bf16 to nearest-even.
 *   - Layout: every tensor is addressed through an fmha_strides triple in
 *     ELEMENTS: element (b, token, head, d) lives at
 *     base + b*batch + token*token_stride + head*head + d.  The head dimension
 *     is contiguous (stride 1).  The natural layouts are
 *     q, o [batch][T][n_h][hd] and k, v [batch][s_k][n_kv_h][hd].
 *     A K/V head stride of 0 with n_kv_h == n_h is MQA and gives the same
 *     result as n_kv_h == 1.
 *   - Ownership: all pointers are DEVICE memory owned by the caller.  The
 *     library never allocates, frees or retains memory and keeps no mutable
 *     global state; calls are thread-safe.
 *   - Asynchrony: every call enqueues its kernels on `stream` (a
 *     hipStream_t; NULL is the default stream) and returns without
 *     synchronising.  Outputs are valid once the stream reaches that point.
 *   - Errors: the return value is an fmha_status.  Arguments are validated
 *     on the host before any HIP call; on a validation error nothing is
 *     launched and no output is touched.  FMHA_ERR_LAUNCH reports a HIP
 *     launch failure (hipGetLastError after the launch).  Nothing is
 *     printed and no exception crosses the ABI.
 *   - Alignment: every pointer must be 16-byte aligned and every batch,
 *     token and head stride a multiple of 8 elements (0 is allowed for a
 *     K/V head stride): the kernels move 16-byte vectors.
 *   - Supported sizes: hd in {64, 128, 256, 512}; 1 <= T <= 2^20;
 *     1 <= s_k <= 2^30; n_h a multiple of n_kv_h with (n_h / n_kv_h) * T
 *     <= 2^30; K and V token strides below 2^32 elements (key rows are
 *     addressed with 32-bit products; FMHA_ERR_UNSUPPORTED otherwise).
 *     With K and V head strides both 0 all n_h query heads share one KV
 *     head, and the row limit reads n_h * T <= 2^30.  A launch must fit one
 *     dispatch packet: fewer than 2^32 work-items in its grid (for example
 *     the merge runs 256 per output row, so batch * n_h * T < 2^24);
 *     FMHA_ERR_UNSUPPORTED otherwise.  With causal or window set, T must not
 *     exceed s_k.  Decode
 *     (T = 1), short prefill and long prefill (T up to s_k, the prefill the
 *     "Next steps" of CURRENT_ISSUE.md call for) share the entry points.
 */
#ifndef FMHA_H
#define FMHA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Strides of a 4-D [batch][token][head][hd] tensor, in elements. */
typedef struct {
    int64_t batch;
    int64_t token;
    int64_t head;
} fmha_strides;

typedef enum {
    FMHA_OK = 0,
    FMHA_ERR_INVALID_ARG = 1, /* null pointer, size <= 0, n_h % n_kv_h != 0, bad mask
                                 arguments, T > s_k with a mask, split_len <= 0 */
    FMHA_ERR_UNSUPPORTED = 2, /* hd not in {64,128,256,512}, or a size over its limit */
    FMHA_ERR_ALIGNMENT = 3,   /* pointer not 16-byte aligned or stride not a multiple of 8 */
    FMHA_ERR_LAUNCH = 4,      /* the HIP launch failed */
    FMHA_ERR_WORKSPACE = 5    /* workspace missing or smaller than the call needs */
} fmha_status;

/*
 * fmha_forward -- fused attention in one launch.
 *
 * Computes O and (optionally) lse as defined above, over all s_k keys, with
 * the online softmax (running max and running sum, rescaling the partial
 * output as each 32-key slice arrives) of the multi-tile kernel in the
 * e4ee9fdc commit log.
 *
 *   q      [batch][T][n_h][hd]      bf16, strides q_st
 *   k, v   [batch][s_k][n_kv_h][hd] bf16, strides k_st, v_st (head 0 = MQA)
 *   o      [batch][T][n_h][hd]      bf16, strides o_st (written)
 *   lse    [batch][n_h][T]          fp32, dense (written); may be NULL
 *   scale  multiplies the unscaled dot product (normally 1/sqrt(hd))
 *   window 0 = none; else only keys j > pos_i - window stay visible
 *   causal 0 or 1
 *   stream hipStream_t or NULL
 */
int fmha_forward(const void *q, const void *k, const void *v, void *o, float *lse,
                 int batch, int n_h, int n_kv_h, int T, int s_k, int hd,
                 fmha_strides q_st, fmha_strides k_st, fmha_strides v_st, fmha_strides o_st,
                 float scale, int window, int causal, void *stream);

/*
 * fmha_forward_ws -- fmha_forward with a caller-provided workspace, for grids
 * of few units.  A call with fewer 16-row tiles (rows = query positions x
 * query heads per KV head) than the GPU has compute units, whose tiles each
 * see many keys, is split over the keys into partitions of at most 128 keys
 * -- the multi-CTA split ("D2 multi-CTA" in the 593bc25a log) -- written as
 * fp32 partial outputs into the workspace, and combined by the D5 merge
 * ("Next steps", item 4 of CURRENT_ISSUE.md) in a second launch on the same
 * stream.  Other calls run exactly as fmha_forward and leave the workspace
 * untouched.  The result is the attention defined above either way.
 *
 *   workspace        device memory, 16-byte aligned, owned by the caller; its
 *                    contents on entry do not matter, and on return it holds
 *                    the partials (valid once the stream reaches that point)
 *   workspace_bytes  its size; fmha_forward_ws_size gives the bytes a call of
 *                    given sizes needs (0 when it runs fused, where workspace
 *                    may be NULL)
 * The other arguments are as for fmha_forward.  Errors: as fmha_forward;
 * FMHA_ERR_WORKSPACE when the call splits and the workspace is NULL or
 * smaller than needed; FMHA_ERR_ALIGNMENT for a misaligned workspace.  Two
 * calls in flight at once must not share a workspace.
 */
int fmha_forward_ws(const void *q, const void *k, const void *v, void *o, float *lse,
                    int batch, int n_h, int n_kv_h, int T, int s_k, int hd,
                    fmha_strides q_st, fmha_strides k_st, fmha_strides v_st, fmha_strides o_st,
                    float scale, int window, int causal,
                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * fmha_forward_noalloc -- fmha_forward_ws for callers that cannot allocate
 * (code under HIP graph capture, serving loops, harnesses that forbid
 * hipMalloc): the same computation and kernels, with the split path's
 * partials in 32 MiB of static device scratch that the library holds on each
 * GPU it runs on until the process ends, instead of a caller workspace.  The
 * call allocates nothing.  A call whose split needs more than 32 MiB (as
 * fmha_forward_ws_size reports) is rejected before any HIP call.  The scratch
 * of a GPU is shared by every call on it: calls that overlap on one GPU
 * (different streams, or threads) race and must not be issued; the first
 * call on a GPU looks the scratch address up once (hipGetSymbolAddress).
 * Errors: as fmha_forward_ws; FMHA_ERR_WORKSPACE when the split needs more
 * than the 32 MiB; FMHA_ERR_LAUNCH if the scratch address cannot be found.
 */
int fmha_forward_noalloc(const void *q, const void *k, const void *v, void *o, float *lse,
                         int batch, int n_h, int n_kv_h, int T, int s_k, int hd,
                         fmha_strides q_st, fmha_strides k_st, fmha_strides v_st, fmha_strides o_st,
                         float scale, int window, int causal, void *stream);

/* Bytes of workspace fmha_forward_ws needs for a call of these sizes (0 when
 * it runs fused): host-only, launches nothing.  k_st / v_st matter through
 * their head strides (both 0 = MQA).  Errors: as fmha_forward for sizes and
 * mask arguments; FMHA_ERR_INVALID_ARG for a null `bytes`. */
int fmha_forward_ws_size(int batch, int n_h, int n_kv_h, int T, int s_k, int hd,
                         fmha_strides k_st, fmha_strides v_st, int window, int causal, size_t *bytes);

/*
 * fmha_decode_splitkv -- attention per KV partition (split-KV, "D2
 * multi-CTA" in the 593bc25a log; partitions merged by the D5 formula of
 * "Next steps", item 4).
 *
 * Partition p covers keys [p*split_len, min((p+1)*split_len, s_k)),
 * p = 0 .. n_split-1 with n_split = ceil(s_k / split_len).  For each
 * (b, h, i, p) it writes the attention restricted to that range, NORMALISED
 * within the partition, and its lse; a partition with no visible key gets
 * O_p = 0 and lse_p = -inf.  Any T within the size limits is accepted
 * (decode is T = 1).
 *
 *   o_part   [batch][n_h][T][n_split][hd] fp32, dense (written)
 *   lse_part [batch][n_h][T][n_split]     fp32, dense (written)
 * The other arguments are as for fmha_forward.  Feed both outputs to
 * fmha_lse_merge on the same stream.
 */
int fmha_decode_splitkv(const void *q, const void *k, const void *v,
                        float *o_part, float *lse_part,
                        int batch, int n_h, int n_kv_h, int T, int s_k, int hd,
                        fmha_strides q_st, fmha_strides k_st, fmha_strides v_st,
                        float scale, int window, int causal, int split_len, void *stream);

/*
 * fmha_forward_varlen -- fmha_forward over a ragged batch in a padded cache:
 * batch row b holds seqlens_k[b] keys (positions 0 .. seqlens_k[b] - 1 of
 * k and v, which are allocated for s_k_max keys), and its T queries sit at
 * positions seqlens_k[b] - T + i.  Everything else is as fmha_forward with
 * s_k = seqlens_k[b] for that row; a query at a negative position under a
 * causal mask, or a row of length 0, sees no key (O = 0, lse = -inf).
 * Lengths are read on the device and clamped to [0, s_k_max].
 * The per-row length generalises the single-segment decode of the commit
 * log at e4ee9fdc, whose fast path took one uniform length per call.
 *
 *   seqlens_k  [batch] int32, DEVICE memory, 4-byte aligned (read)
 * Errors: as fmha_forward with s_k = s_k_max (T <= s_k_max when masked);
 * FMHA_ERR_INVALID_ARG for a null seqlens_k, FMHA_ERR_ALIGNMENT for a
 * misaligned one.
 */
int fmha_forward_varlen(const void *q, const void *k, const void *v, const int *seqlens_k,
                        void *o, float *lse,
                        int batch, int n_h, int n_kv_h, int T, int s_k_max, int hd,
                        fmha_strides q_st, fmha_strides k_st, fmha_strides v_st, fmha_strides o_st,
                        float scale, int window, int causal, void *stream);

/*
 * fmha_decode_splitkv_segment -- fmha_decode_splitkv for one key segment of
 * several (for example a few global "sink" keys in one cache and a sliding
 * window in another), writing its partitions into slots
 * [part_offset, part_offset + ceil(s_k / split_len)) of partial buffers that
 * hold n_split_total slots per row.  One fmha_lse_merge over all
 * n_split_total slots then yields attention over the union of the segments:
 * the D5 merge ("Next steps", item 4 of CURRENT_ISSUE.md) applies to any
 * set of disjoint key sets, and the commit log at e4ee9fdc names
 * multi-segment calls as the case its fast path left to a slower one.
 * Masks and query positions are taken within the segment (positions
 * s - T + i for a segment of s keys).  seqlens_k (nullable, device int32
 * [batch]) gives per-row segment lengths as in fmha_forward_varlen; slots
 * whose keys lie past a row's length are written empty (O_p = 0,
 * lse_p = -inf).  Slots outside this call's range are not touched.
 *
 *   o_part   [batch][n_h][T][n_split_total][hd] fp32 (slots written)
 *   lse_part [batch][n_h][T][n_split_total]     fp32 (slots written)
 * Errors: as fmha_decode_splitkv; FMHA_ERR_INVALID_ARG for part_offset < 0
 * or part_offset + ceil(s_k / split_len) > n_split_total;
 * FMHA_ERR_ALIGNMENT for a misaligned seqlens_k.
 */
int fmha_decode_splitkv_segment(const void *q, const void *k, const void *v, const int *seqlens_k,
                                float *o_part, float *lse_part,
                                int batch, int n_h, int n_kv_h, int T, int s_k, int hd,
                                fmha_strides q_st, fmha_strides k_st, fmha_strides v_st,
                                float scale, int window, int causal, int split_len,
                                int part_offset, int n_split_total, void *stream);

/*
 * fmha_lse_merge -- the D5 merge ("Next steps", item 4 of CURRENT_ISSUE.md):
 *   O   = sum_p exp(lse_p) O_p / sum_p exp(lse_p)
 *   lse = ln sum_p exp(lse_p)
 * evaluated with max_p lse_p factored out.  Partitions with lse_p = -inf
 * carry no weight; a row whose partitions are all -inf gets O = 0 and
 * lse = -inf.
 *
 *   o_part   [batch][n_h][T][n_split][hd] fp32, dense (read)
 *   lse_part [batch][n_h][T][n_split]     fp32, dense (read)
 *   o        [batch][T][n_h][hd]          bf16, strides o_st (written)
 *   lse      [batch][n_h][T]              fp32, dense (written); may be NULL
 * Errors: FMHA_ERR_INVALID_ARG for null inputs/o or sizes <= 0,
 * FMHA_ERR_UNSUPPORTED for hd outside {64,128,256,512}, FMHA_ERR_ALIGNMENT
 * as above.
 */
int fmha_lse_merge(const float *o_part, const float *lse_part, void *o, float *lse,
                   int batch, int n_h, int T, int hd, int n_split,
                   fmha_strides o_st, void *stream);

/*
 * Output in an OCP microscaling (MX) format instead of bf16: the output
 * quantisation step the pages attach to the attention epilogue (the FP4 pack
 * slot of the one-way epilogue on CURRENT_ISSUE.md; the NVFP4 quantiser and
 * its round-to-nearest-even thresholds in the commit log at 593bc25a), in
 * the MX formats of this hardware.  Each block of 32 consecutive head-dim
 * columns of an output row shares one E8M0 scale 2^X with
 * X = floor(log2 max|o|) - emax (emax = 8 for E4M3, 2 for E2M1), clamped to
 * [-127, 127] (-127 for an all-zero block); every element o / 2^X is rounded
 * to nearest, ties to even, saturating at 448 (E4M3) or 6 (E2M1).
 *   FMHA_MX_FP8_E4M3: one byte per element, sign | exponent (bias 7) |
 *                     3 mantissa bits (exponent field 0: subnormals)
 *   FMHA_MX_FP4_E2M1: sign | exponent (bias 1) | 1 mantissa bit, two per
 *                     byte, the lower column in the low nibble
 * Layouts (dense, caller-owned device memory):
 *   o_codes  [batch][T][n_h][hd]      (E4M3) or [batch][T][n_h][hd / 2] (E2M1),
 *            16-byte aligned
 *   o_scales [batch][T][n_h][hd / 32] E8M0 codes (X + 127)
 */
enum { FMHA_MX_FP8_E4M3 = 1, FMHA_MX_FP4_E2M1 = 2 };

/* fmha_forward with MX output; lse as in fmha_forward.  Errors: as
 * fmha_forward; FMHA_ERR_INVALID_ARG for a null o_codes / o_scales or an
 * unknown format. */
int fmha_forward_mx(const void *q, const void *k, const void *v, void *o_codes, void *o_scales, float *lse,
                    int batch, int n_h, int n_kv_h, int T, int s_k, int hd,
                    fmha_strides q_st, fmha_strides k_st, fmha_strides v_st,
                    float scale, int window, int causal, int format, void *stream);

/* fmha_lse_merge with MX output.  Errors: as fmha_lse_merge;
 * FMHA_ERR_INVALID_ARG for a null o_codes / o_scales or an unknown format. */
int fmha_lse_merge_mx(const float *o_part, const float *lse_part, void *o_codes, void *o_scales, float *lse,
                      int batch, int n_h, int T, int hd, int n_split, int format, void *stream);

/*
 * How fmha_forward (split_len = 0) or fmha_decode_splitkv (split_len > 0)
 * would run a call of these sizes: a host-only query that launches nothing
 * and needs no device, for diagnostics and tests that must reach every
 * kernel variant.  The work decomposition (one unit per batch, KV head,
 * row block and key partition) refines the per-(head, batch) grid of the
 * commit log at e4ee9fdc for this hardware.
 *
 *   waves_per_group  4 or 8: wavefronts per workgroup; 8 for few-unit
 *                    grids (fewer than two 16-row units per compute unit),
 *                    the one-pass / pass kernels and the hd-512 row kernel
 *   tiles_per_group  16-row tiles per workgroup (1 or 2; 4 or 8 row-parallel)
 *   one_slice        1 when every workgroup's key range fits one pass
 *   streaming        1 when no two workgroups read the same K/V rows
 *   row_parallel     1 when each wave owns whole rows (at hd 512 half of
 *                    each row's head dim) and the waves share K/V chunks
 *                    staged in LDS (many rows per KV head)
 *   workgroups       grid size
 *   threads_per_group  work-items per workgroup (64 * waves_per_group)
 *   kernel           NUL-terminated name of the kernel template instance the
 *                    call launches, e.g. "stream_kernel<128, true, true, 4, 1>"
 * k_st / v_st matter through their head strides (both 0 = MQA) and their
 * token strides: the row-parallel kernel stages K/V by buffer loads with
 * 32-bit offsets from a load's (hd 512: a 32-key chunk's) first key row, so
 * it is chosen only when (1024 / (2 hd) - 1) * token stride * 2 + 2 hd
 * (hd 512: 31 * token stride * 2 + 1024) < 2^31 bytes; the one-pass and
 * pass kernels address a wave's rows (up to 64) the same way, and are chosen
 * only when 63 * token stride * 2 + 256 < 2^31.
 * Errors: as fmha_forward for sizes and mask arguments (including
 * FMHA_ERR_UNSUPPORTED for a grid of 2^32 work-items or more);
 * FMHA_ERR_INVALID_ARG for a null plan or split_len < 0.
 */
typedef struct {
    int waves_per_group;
    int tiles_per_group;
    int one_slice;
    int streaming;
    int row_parallel;
    int64_t workgroups;
    int threads_per_group;
    char kernel[96];
} fmha_plan;

int fmha_attention_plan(int batch, int n_h, int n_kv_h, int T, int s_k, int hd,
                        fmha_strides k_st, fmha_strides v_st, int window, int causal,
                        int split_len, fmha_plan *plan);

/* Static, human-readable text for a status code (never NULL). */
const char *fmha_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FMHA_H */
