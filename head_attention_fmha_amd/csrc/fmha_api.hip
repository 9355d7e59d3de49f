// fmha_api.hip -- the C ABI of libfmha.so (declared in include/fmha.h):
// argument validation, shape-class dispatch and kernel launches.
//
// Validation runs entirely on the host before any HIP call, so invalid
// calls return a status without touching the device (and work on a machine
// with no GPU).  Every launch goes to the caller's stream; nothing here
// synchronises, allocates or keeps state.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <mutex>

#include "fmha.h"
#include "attn_kernel.hpp"
#include "rows_kernel.hpp"
#include "stream_kernel.hpp"
#include "rows_split_kernel.hpp"
#include "pass_kernel.hpp"
#include "cols_kernel.hpp"
#include "merge_kernel.hpp"

namespace {

using fmha::FwdParams;
using fmha::MergeParams;

bool aligned16(const void *ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

bool stride_ok(int64_t s) { return s >= 0 && (s % 8) == 0; }

bool strides_ok(const fmha_strides &st) {
    return stride_ok(st.batch) && stride_ok(st.token) && stride_ok(st.head);
}

// K/V rows are addressed with 32 x 32-bit products: token strides below 2^32.
bool kv_token_strides_ok(const fmha_strides &k_st, const fmha_strides &v_st) {
    return k_st.token < (1ll << 32) && v_st.token < (1ll << 32);
}

bool hd_supported(int hd) { return hd == 64 || hd == 128 || hd == 256 || hd == 512; }

// Size limits: keep every row, key and partition index inside int.
constexpr int kMaxT = 1 << 20;
constexpr int kMaxKeys = 1 << 30;
constexpr int64_t kMaxRows = int64_t(1) << 30;  // stacked rows (group * T) per KV head

// K and V both with head stride 0 hold one KV head for every query head: the
// call runs as MQA (n_kv_h = 1), streaming K/V once per batch row.
int effective_kv_heads(int n_kv_h, const fmha_strides &k_st, const fmha_strides &v_st) {
    return (k_st.head == 0 && v_st.head == 0) ? 1 : n_kv_h;
}

// Sizes and mask arguments of an attention call.  The row limit applies to
// the stacked rows per KV head the kernels will see: with K/V head strides of
// 0 all n_h query heads share one KV head.
int validate_dims(int batch, int n_h, int n_kv_h, int T, int s_k, int hd, int window, int causal,
                  const fmha_strides &k_st, const fmha_strides &v_st) {
    if (batch <= 0 || n_h <= 0 || n_kv_h <= 0 || T <= 0 || s_k <= 0 || hd <= 0) return FMHA_ERR_INVALID_ARG;
    if (n_h % n_kv_h != 0) return FMHA_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return FMHA_ERR_INVALID_ARG;
    if (window < 0) return FMHA_ERR_INVALID_ARG;
    if ((causal || window > 0) && T > s_k) return FMHA_ERR_INVALID_ARG;
    const int kv_eff = effective_kv_heads(n_kv_h, k_st, v_st);
    if (!hd_supported(hd) || T > kMaxT || s_k > kMaxKeys || (int64_t)(n_h / kv_eff) * T > kMaxRows)
        return FMHA_ERR_UNSUPPORTED;
    return FMHA_OK;
}

// A dispatch packet counts work-items in 32 bits: a grid of `workgroups`
// workgroups of `threads` work-items each must stay below 2^32.
bool grid_fits(int64_t workgroups, int threads) {
    return workgroups > 0 && workgroups * threads <= int64_t(0xffffffff);
}

// Shared validation of fmha_forward / fmha_decode_splitkv.
int validate_attention(const void *q, const void *k, const void *v, const void *out0, const void *out1,
                       bool out1_required, int batch, int n_h, int n_kv_h, int T, int s_k, int hd,
                       const fmha_strides &q_st, const fmha_strides &k_st, const fmha_strides &v_st,
                       const fmha_strides *o_st, int window, int causal) {
    if (!q || !k || !v || !out0 || (out1_required && !out1)) return FMHA_ERR_INVALID_ARG;
    const int rc = validate_dims(batch, n_h, n_kv_h, T, s_k, hd, window, causal, k_st, v_st);
    if (rc != FMHA_OK) return rc;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out0) || (out1 && !aligned16(out1)))
        return FMHA_ERR_ALIGNMENT;
    if (!strides_ok(q_st) || !strides_ok(k_st) || !strides_ok(v_st) || (o_st && !strides_ok(*o_st)))
        return FMHA_ERR_ALIGNMENT;
    if (!kv_token_strides_ok(k_st, v_st)) return FMHA_ERR_UNSUPPORTED;
    return FMHA_OK;
}

FwdParams make_params(const void *q, const void *k, const void *v, int batch, int n_h, int n_kv_h, int T,
                      int s_k, const fmha_strides &q_st, const fmha_strides &k_st, const fmha_strides &v_st,
                      float scale, int window, int causal) {
    n_kv_h = effective_kv_heads(n_kv_h, k_st, v_st);
    FwdParams p{};
    p.q = static_cast<const uint16_t *>(q);
    p.k = static_cast<const uint16_t *>(k);
    p.v = static_cast<const uint16_t *>(v);
    p.q_sb = q_st.batch; p.q_st = q_st.token; p.q_sh = q_st.head;
    p.k_sb = k_st.batch; p.k_st = k_st.token; p.k_sh = k_st.head;
    p.v_sb = v_st.batch; p.v_st = v_st.token; p.v_sh = v_st.head;
    p.batch = batch; p.n_h = n_h; p.n_kv_h = n_kv_h; p.T = T; p.s_k = s_k;
    p.group = n_h / n_kv_h;
    p.rows = p.group * T;
    p.window = window;
    p.causal = causal;
    p.scale_log2 = scale * fmha::kLog2e;
    return p;
}

// compute units of an MI355X (8 XCDs x 32)
constexpr int kComputeUnits = 256;

// Head-dim parts per workgroup: one up to hd 128, two at 256, four at 512
// (64 or 128 columns per wave).
int head_parts(int hd) { return hd <= 128 ? 1 : hd / 128; }

// Positions a 16-row tile can span: rows are numbered t * group + head and
// tiles start at multiples of 16.
int tile_positions(int group) {
    if (16 % group == 0) return 16 / group;
    if (group % 16 == 0) return 1;
    return 15 / group + 2;
}

// Row-parallel kernel: keys per LDS chunk for one tile per wave (two tiles
// per wave take 32: two chunks of scores are live in its pipeline).  At hd
// 512 one wave's full-width Q and output tiles fill a SIMD's registers (one
// wave per SIMD), and the chunk pipeline still beats the per-wave kernel.
constexpr int rows_chunk_keys(int hd) { return hd <= 128 ? 64 : 32; }

// The row-parallel kernel stages K/V by buffer loads of 1 KiB, each from a
// scalar base at its first key row with 32-bit lane offsets: the rows of one
// load (1024 / (2 hd) of them) must lie within 2^31 bytes.
bool rows_loads_fit(const FwdParams &p, int hd) {
    const int64_t st = p.k_st > p.v_st ? p.k_st : p.v_st;
    // (hd 512: the head-split kernel addresses a whole 32-key chunk from its
    // first row)
    const int64_t rows = hd == 512 ? 31 : 1024 / (2 * hd) - 1;
    return rows * st * 2 + 2 * hd < (int64_t(1) << 31);
}

// The stream kernel stores split partials by buffer stores with 32-bit byte
// offsets from the first partial row of the KV head: its rows (at least the
// 16 of one tile) lie within rows * n_split_total rows of hd fp32 values.
bool stream_offsets_fit(const FwdParams &p, int hd) {
    const int64_t slots = p.n_split_total > 0 ? p.n_split_total : p.n_split;
    const int64_t rows = p.rows > 16 ? p.rows : 16;
    return rows * slots * hd * 4 < (int64_t(1) << 31);
}

// The stream and pass kernels load K/V by buffer loads from each wave's first key
// row with 32-bit lane offsets: a wave's rows (at most 64) must lie within
// 2^31 bytes.
bool stream_loads_fit(const FwdParams &p) {
    const int64_t st = p.k_st > p.v_st ? p.k_st : p.v_st;
    return 63 * st * 2 + 2 * 128 < (int64_t(1) << 31);
}

// Kernel variants the dispatcher launches (one template family each).
enum Variant : int {
    kRowsTwoTiles,  // rows_kernel<HD, 2, 32>: 128 rows per workgroup (hd <= 128)
    kRowsOneTile,   // rows_kernel<HD, 1, rows_chunk_keys(HD)>: 64 rows per workgroup
    kRowsSplit,     // rows_split_kernel<512>: 64 rows per workgroup, each tile's head dim over two waves
    kAttnEight,     // attn_kernel, eight waves, several slices (hd >= 256)
    kStream,        // stream_kernel<128, STREAM = true, 4, 1>: one pass, non-temporal whole-line K/V loads
    kStreamShared,  // stream_kernel<128, STREAM = false, 4, 1>: one pass, row blocks sharing K/V through L2
    kStreamWide,    // stream_kernel<HD <= 128, true, 8, 1>: one pass of up to 256 keys, eight waves
    kStreamWideShared,
    kStreamWide2,   // stream_kernel<HD <= 128, true, 8, 2>: one pass of up to 512 keys, eight waves
    kStreamWide2Shared,
    kPass,          // pass_kernel<HD>: one pass over <= 128 keys, every load up front (hd >= 256)
    kPassLoop,      // pass_loop_kernel<HD>: 128-key passes, few-unit grids (hd >= 256)
    kCols,          // cols_kernel<512, LOOP = false>: one pass over <= 128 keys, keys by wave for the scores, columns for PV
    kColsLoop,      // cols_kernel<512, LOOP = true>: 128-key passes, few-unit grids
    kAttnOneStream, // attn_kernel, one slice, streamed
    kAttnOne,       // attn_kernel, one slice, K/V shared with other row blocks
    kAttnTwoTiles,  // attn_kernel, several slices, two tiles per workgroup
    kAttnOneTile,   // attn_kernel, several slices, one tile per workgroup
};

// The kernel variant and grid for one call.  A workgroup serves MT 16-row
// tiles of one (batch, KV head, partition); its NW waves split head-dim
// columns (NH parts) and keys (NK = NW / NH groups of 32-key slices).
fmha_plan plan_attention(const FwdParams &p, int hd, bool split, int *variant_out = nullptr) {
    fmha_plan pl{};
    // the widest key range any 16-row tile can see
    int span = p.split_len < p.s_k ? p.split_len : p.s_k;
    // causal + window: a tile's rows span at most tile_positions() positions,
    // so at most window + positions - 1 keys are visible to any of them
    const int ppt = tile_positions(p.group);
    if (p.causal && p.window > 0 && (int64_t)p.window + ppt - 1 < span) span = p.window + ppt - 1;
    // too few 16-row units to give every compute unit two workgroups, at head
    // dims whose four waves hold only one or two key groups, and keys enough
    // for several slices per wave even with eight: eight waves per workgroup,
    // so each walks half as many slices in sequence (at hd <= 128 four key
    // groups already share the keys, and eight only add merge work)
    const int64_t units1 = (int64_t)((p.rows + 15) / 16) * p.n_split * p.n_kv_h * p.batch;
    const bool few_units = units1 < 2 * kComputeUnits;
    pl.waves_per_group = (hd >= 256 && few_units && span > 32 * (8 / head_parts(hd))) ? 8 : 4;
    const int nk = pl.waves_per_group / head_parts(hd);
    // one chunk of 32*NK keys covers every range: the one-slice variant
    pl.one_slice = span <= 32 * nk ? 1 : 0;
    // several slices per workgroup: two tiles per workgroup share every K/V
    // load, worth it while that still leaves two workgroups per compute unit
    // (the multi-slice kernel's occupancy); below that, parallelism wins
    pl.tiles_per_group = 1;
    if (!pl.one_slice && pl.waves_per_group == 4 && p.rows > 16) {
        const int64_t blocks2 = (int64_t)((p.rows + 31) / 32) * p.n_split * p.n_kv_h * p.batch;
        if (blocks2 >= 2 * kComputeUnits) pl.tiles_per_group = 2;
    }
    // many rows per KV head and several passes over the keys: the row-parallel
    // kernel, whose four waves share every K/V chunk through LDS.  One 16-row
    // tile per wave while that is needed to give every compute unit a
    // workgroup (short prefill); two -- every K operand read from LDS then
    // feeds two MFMAs -- once the grid has two workgroups per compute unit
    // even so (long prefill).  At hd <= 128 also when one slice covers every
    // tile's keys: a 64-row workgroup then reads each K/V byte once where four
    // one-slice workgroups each read it (causal MHA prefill T 128 over 128
    // keys: hd 64 8.2 -> 6.5 us, hd 128 11.1 -> 9.4 us; over 64 keys, no
    // mask, hd 64: 6.2 -> 5.6 us) -- but not under a window, where the 64
    // rows of a workgroup see many more keys than the 16 of a tile (window 32
    // over 512 keys: 8.3 -> 9.8 us), nor over 32 keys or fewer, half a chunk
    // (hd 128: 7.1 -> 7.6 us)
    const bool rows_one_slice = hd <= 128 && p.window == 0 && span > 32;
    if ((!pl.one_slice || rows_one_slice) && p.rows >= 64 && rows_loads_fit(p, hd)) {
        const int64_t per_kv = (int64_t)p.n_split * p.n_kv_h * p.batch;
        const int64_t groups1 = (int64_t)((p.rows + 63) / 64) * per_kv;
        const int64_t groups2 = (int64_t)((p.rows + 127) / 128) * per_kv;
        if (groups1 >= kComputeUnits) {
            pl.row_parallel = 1;
            // hd 512: every tile's head dimension over two waves (eight per
            // workgroup, two per SIMD)
            pl.waves_per_group = hd == 512 ? 8 : 4;
            // (two tiles of 256 or 512 columns would spill: one tile per wave)
            pl.tiles_per_group = (hd <= 128 && groups2 >= 2 * kComputeUnits) ? 8 : 4;
        }
    }
    // hd 256 / 512, not the row-parallel kernel's many-row work: the pass
    // kernel (eight waves, 128-key passes) when every tile's keys fit one pass
    // or the grid holds at most one tile per compute unit (each workgroup then
    // takes in its whole range: whole-row loads, one pass's loads in flight
    // behind the other's math)
    const bool pass = !pl.row_parallel && hd >= 256 && (span <= 128 || units1 <= kComputeUnits) &&
                      stream_loads_fit(p);
    // hd 64 / 128, up to 512 keys per tile and at most one tile per compute unit:
    // each workgroup must take in its whole key range, and whole-row loads
    // (the stream kernel, eight waves of 32 or 64 keys) reach it at about
    // three times the rate of loads in the MFMA operand shape (MQA decode hd
    // 64 over 512 keys: 6.4 -> 5.7 us against the per-wave kernel; one-slice
    // work at hd 64 measured the same on either and stays on the per-wave
    // kernel)
    const bool wide = !pl.row_parallel && hd <= 128 && !pl.one_slice && span <= 512 && units1 <= kComputeUnits &&
                      stream_loads_fit(p) && (!split || stream_offsets_fit(p, hd));
    if (pass || wide) {
        pl.waves_per_group = 8;
        pl.tiles_per_group = 1;
        pl.one_slice = (wide || span <= 128) ? 1 : 0;  // (the pass kernel may take several passes)
    }
    const int rows_per_group = 16 * pl.tiles_per_group;
    const int row_blocks = (p.rows + rows_per_group - 1) / rows_per_group;
    // one slice and one row block per KV head: nothing another workgroup reads
    pl.streaming = (pl.one_slice && row_blocks == 1) ? 1 : 0;
    pl.workgroups = (int64_t)row_blocks * p.n_split * p.n_kv_h * p.batch;
    pl.threads_per_group = 64 * pl.waves_per_group;

    // the variant, and the kernel template instance it launches
    int var;
    const int nh = head_parts(hd);
    const char *sp = split ? "true" : "false";
    if (pl.row_parallel && hd == 512) {
        var = kRowsSplit;
        snprintf(pl.kernel, sizeof pl.kernel, "rows_split_kernel<%d, %s>", hd, sp);
    } else if (pl.row_parallel) {
        var = (hd <= 128 && pl.tiles_per_group == 8) ? kRowsTwoTiles : kRowsOneTile;
        snprintf(pl.kernel, sizeof pl.kernel, "rows_kernel<%d, %d, %d, %s>", hd, var == kRowsTwoTiles ? 2 : 1,
                 var == kRowsTwoTiles ? 32 : rows_chunk_keys(hd), sp);
    } else if (pass) {
        // hd 512: the column-split kernel over one pass, and over several when
        // row blocks share each KV head's K/V through L2 (MQA decode hd 512
        // over 256 / 384 / 512 keys: 16.0 / 20.6 / 25.1 -> 14.6 / 19.3 / 24.2
        // us); a lone row block per KV head streams K/V that no other
        // workgroup reads, where the pass loop's 256-byte row parts went
        // faster (causal MHA prefill T 1 / T 4 over 512 keys: 30.2 / 30.3
        // against 31.1 / 31.4 us)
        // At hd 256 only one-pass calls whose row blocks share K/V (MQA
        // decode over 128 keys 6.64 -> 6.11 us); over several passes, or with
        // one row block per KV head, the one-pass and pass-loop kernels
        // stayed faster (MQA decode over 384 / 512 keys 11.3 / 14.5 against
        // 12.1 / 16.5 us, causal MHA prefill T 1 over 128 keys 7.9 against
        // 8.3 us).  A split call takes the same kernel as the fused one.
        const bool shared_kv = (p.rows + 15) / 16 > 1;
        const bool cols = hd == 512 ? (span <= 128 || shared_kv) : (span <= 128 && shared_kv);
        if (cols) {
            var = span > 128 ? kColsLoop : kCols;
            snprintf(pl.kernel, sizeof pl.kernel, "cols_kernel<%d, %s, %s>", hd, sp, var == kColsLoop ? "true" : "false");
        } else {
            var = span > 128 ? kPassLoop : kPass;
            snprintf(pl.kernel, sizeof pl.kernel, "%s<%d, %s>", var == kPass ? "pass_kernel" : "pass_loop_kernel", hd, sp);
        }
    } else if (wide) {
        const int ks = span <= 256 ? 1 : 2;
        var = ks == 1 ? (pl.streaming ? kStreamWide : kStreamWideShared)
                      : (pl.streaming ? kStreamWide2 : kStreamWide2Shared);
        snprintf(pl.kernel, sizeof pl.kernel, "stream_kernel<%d, %s, %s, 8, %d>", hd, sp,
                 pl.streaming ? "true" : "false", ks);
    } else if (pl.one_slice && hd == 128 && stream_loads_fit(p) && (!split || stream_offsets_fit(p, hd))) {
        var = pl.streaming ? kStream : kStreamShared;
        snprintf(pl.kernel, sizeof pl.kernel, "stream_kernel<%d, %s, %s, 4, 1>", hd, sp,
                 pl.streaming ? "true" : "false");
    } else {
        const int nw = pl.waves_per_group;
        const bool one = pl.one_slice, stream = pl.one_slice && pl.streaming;
        var = nw == 8 ? kAttnEight
              : stream ? kAttnOneStream
              : one ? kAttnOne
              : pl.tiles_per_group == 2 ? kAttnTwoTiles : kAttnOneTile;
        snprintf(pl.kernel, sizeof pl.kernel, "attn_kernel<%d, %d, %d, %d, %d, %s, %s, %s>", hd, nw, nw / nh, nh,
                 pl.tiles_per_group, sp, one ? "true" : "false", stream ? "true" : "false");
    }
    if (variant_out) *variant_out = var;
    return pl;
}

template <int HD, int NW, int MT, bool SPLIT, bool ONE, bool STREAM>
void launch_kernel(const FwdParams &p, hipStream_t stream) {
    constexpr int NH = HD <= 128 ? 1 : HD / 128;
    constexpr int NK = NW / NH;
    hipLaunchKernelGGL((fmha::attn_kernel<HD, NW, NK, NH, MT, SPLIT, ONE, STREAM>), dim3(p.n_units), dim3(64 * NW),
                       0, stream, p);
}

template <int HD, bool SPLIT>
void launch_hd(const FwdParams &p, int var, hipStream_t s) {
    switch (var) {
        case kRowsTwoTiles:
            if constexpr (HD <= 128)
                hipLaunchKernelGGL((fmha::rows_kernel<HD, 2, 32, SPLIT>), dim3(p.n_units), dim3(256), 0, s, p);
            break;
        case kRowsOneTile:
            if constexpr (HD < 512)
                hipLaunchKernelGGL((fmha::rows_kernel<HD, 1, rows_chunk_keys(HD), SPLIT>), dim3(p.n_units), dim3(256),
                                   0, s, p);
            break;
        case kRowsSplit:
            if constexpr (HD == 512)
                hipLaunchKernelGGL((fmha::rows_split_kernel<HD, SPLIT>), dim3(p.n_units), dim3(512), 0, s, p);
            break;
        case kAttnEight:
            // chosen only for several slices per wave (never one-slice), hd >= 256
            if constexpr (HD >= 256) launch_kernel<HD, 8, 1, SPLIT, false, false>(p, s);
            break;
        case kStream:
            if constexpr (HD == 128)
                hipLaunchKernelGGL((fmha::stream_kernel<HD, SPLIT, true, 4, 1>), dim3(p.n_units), dim3(256), 0, s, p);
            break;
        case kStreamShared:
            if constexpr (HD == 128)
                hipLaunchKernelGGL((fmha::stream_kernel<HD, SPLIT, false, 4, 1>), dim3(p.n_units), dim3(256), 0, s, p);
            break;
        case kStreamWide:
            if constexpr (HD <= 128)
                hipLaunchKernelGGL((fmha::stream_kernel<HD, SPLIT, true, 8, 1>), dim3(p.n_units), dim3(512), 0, s, p);
            break;
        case kStreamWideShared:
            if constexpr (HD <= 128)
                hipLaunchKernelGGL((fmha::stream_kernel<HD, SPLIT, false, 8, 1>), dim3(p.n_units), dim3(512), 0, s, p);
            break;
        case kStreamWide2:
            if constexpr (HD <= 128)
                hipLaunchKernelGGL((fmha::stream_kernel<HD, SPLIT, true, 8, 2>), dim3(p.n_units), dim3(512), 0, s, p);
            break;
        case kStreamWide2Shared:
            if constexpr (HD <= 128)
                hipLaunchKernelGGL((fmha::stream_kernel<HD, SPLIT, false, 8, 2>), dim3(p.n_units), dim3(512), 0, s, p);
            break;
        case kPass:
            if constexpr (HD == 256)
                hipLaunchKernelGGL((fmha::pass_kernel<HD, SPLIT>), dim3(p.n_units), dim3(64 * fmha::PassShape<HD>::NW),
                                   0, s, p);
            break;
        case kCols:
            if constexpr (HD >= 256)
                hipLaunchKernelGGL((fmha::cols_kernel<HD, SPLIT, false>), dim3(p.n_units),
                                   dim3(64 * fmha::ColsShape<HD>::NW), 0, s, p);
            break;
        case kColsLoop:
            if constexpr (HD == 512)
                hipLaunchKernelGGL((fmha::cols_kernel<HD, SPLIT, true>), dim3(p.n_units),
                                   dim3(64 * fmha::ColsShape<HD>::NW), 0, s, p);
            break;
        case kPassLoop:
            if constexpr (HD >= 256)
                hipLaunchKernelGGL((fmha::pass_loop_kernel<HD, SPLIT>), dim3(p.n_units),
                                   dim3(64 * fmha::PassShape<HD>::NW), 0, s, p);
            break;
        // one-slice work at hd >= 256 runs the one-pass kernel
        case kAttnOneStream:
            if constexpr (HD <= 128) launch_kernel<HD, 4, 1, SPLIT, true, true>(p, s);
            break;
        case kAttnOne:
            if constexpr (HD <= 128) launch_kernel<HD, 4, 1, SPLIT, true, false>(p, s);
            break;
        case kAttnTwoTiles: launch_kernel<HD, 4, 2, SPLIT, false, false>(p, s); break;
        default: launch_kernel<HD, 4, 1, SPLIT, false, false>(p, s); break;
    }
}

template <bool SPLIT>
int launch_attention(FwdParams p, int hd, void *stream) {
    int var = 0;
    const fmha_plan pl = plan_attention(p, hd, SPLIT, &var);
    if (!grid_fits(pl.workgroups, pl.threads_per_group)) return FMHA_ERR_UNSUPPORTED;
    p.n_row_blocks = (p.rows + 16 * pl.tiles_per_group - 1) / (16 * pl.tiles_per_group);
    p.n_units = (int)pl.workgroups;
    // only row blocks share data across workgroups; streaming units run best
    // in plain order (neighbouring blocks read neighbouring memory)
    p.xcd_remap = (p.n_row_blocks > 1 && p.n_units % 8 == 0) ? 1 : 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (hd) {
        case 64: launch_hd<64, SPLIT>(p, var, s); break;
        case 128: launch_hd<128, SPLIT>(p, var, s); break;
        case 256: launch_hd<256, SPLIT>(p, var, s); break;
        default: launch_hd<512, SPLIT>(p, var, s); break;
    }
    return hipGetLastError() == hipSuccess ? FMHA_OK : FMHA_ERR_LAUNCH;
}

int launch_merge(MergeParams p, int batch, int n_h, int T, int hd, int n_split, void *stream) {
    const int64_t rows = (int64_t)batch * n_h * T;
    p.n_h = n_h;
    p.T = T;
    p.n_split = n_split;
    int rpw;
    switch (hd) {
        case 64: rpw = fmha::MergeShape<64>::RPW; break;
        case 128: rpw = fmha::MergeShape<128>::RPW; break;
        case 256: rpw = fmha::MergeShape<256>::RPW; break;
        default: rpw = fmha::MergeShape<512>::RPW; break;
    }
    const int64_t blocks = (rows + rpw - 1) / rpw;
    if (rows > 0x7fffffff || !grid_fits(blocks, 256)) return FMHA_ERR_UNSUPPORTED;
    p.rows = (int)rows;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const dim3 grid((unsigned)blocks), block(256);
    switch (hd) {
        case 64: hipLaunchKernelGGL(fmha::merge_kernel<64>, grid, block, 0, s, p); break;
        case 128: hipLaunchKernelGGL(fmha::merge_kernel<128>, grid, block, 0, s, p); break;
        case 256: hipLaunchKernelGGL(fmha::merge_kernel<256>, grid, block, 0, s, p); break;
        default: hipLaunchKernelGGL(fmha::merge_kernel<512>, grid, block, 0, s, p); break;
    }
    return hipGetLastError() == hipSuccess ? FMHA_OK : FMHA_ERR_LAUNCH;
}

// ---- few-unit calls split over the keys (fmha_forward_ws) --------------------
//
// A call with fewer 16-row tiles than compute units leaves most of the chip
// idle, each workgroup walking its tile's keys alone (the MQA decode of 128
// query heads over one KV head has 8 tiles per batch row).  With a workspace
// the keys are split into partitions -- the split-KV decode of the pages'
// "D2 multi-CTA" -- so the grid covers the chip, and the D5 merge ("Next
// steps", item 4 of CURRENT_ISSUE.md) combines them in a second launch.

// fused work per tile (keys x hd) from which the split pays for the second
// launch and the partial traffic
constexpr int64_t kSplitMinWork = 96 * 1024;

struct SplitChoice {
    int split_len = 0;  // 0: run fused
    int n_split = 1;
};

SplitChoice choose_split(const FwdParams &p, int hd) {
    SplitChoice c;
    const int64_t tiles = (int64_t)((p.rows + 15) / 16) * p.n_kv_h * p.batch;
    if (tiles >= kComputeUnits) return c;
    int64_t span = p.s_k;
    const int ppt = tile_positions(p.group);
    if (p.causal && p.window > 0 && (int64_t)p.window + ppt - 1 < span) span = p.window + ppt - 1;
    if (span * hd < kSplitMinWork) return c;
    // partitions of at most 128 keys (one pass of the one-slice kernels), as
    // many as it takes to give every compute unit a workgroup
    const int64_t want = (kComputeUnits + tiles - 1) / tiles;
    int64_t len = (p.s_k + want - 1) / want;
    len = ((len + 31) / 32) * 32;
    if (len > 128) len = 128;
    if (len >= p.s_k) return c;
    c.split_len = (int)len;
    c.n_split = (int)((p.s_k + len - 1) / len);
    return c;
}

// workspace layout: o_part [rows][n_split][hd] fp32, then lse_part [rows][n_split]
// fp32 at the next 256-byte boundary
int64_t split_workspace_bytes(int64_t rows, int n_split, int hd) {
    const int64_t o_bytes = (rows * n_split * hd * 4 + 255) / 256 * 256;
    return o_bytes + rows * n_split * 4;
}

// fmha_forward through a workspace: split + merge when choose_split says so,
// the fused call otherwise.  `ws` is device memory of at least the bytes
// split_workspace_bytes gives (checked by the callers).
int forward_split_or_fused(FwdParams p, int hd, const SplitChoice &c, void *ws, const fmha_strides &o_st,
                           void *stream) {
    if (c.split_len == 0) {
        p.split_len = p.s_k;
        p.n_split = 1;
        p.n_split_total = 1;
        return launch_attention<false>(p, hd, stream);
    }
    const int64_t rows = (int64_t)p.batch * p.n_h * p.T;
    float *o_part = static_cast<float *>(ws);
    float *lse_part = reinterpret_cast<float *>(static_cast<unsigned char *>(ws) +
                                                (rows * c.n_split * hd * 4 + 255) / 256 * 256);
    uint16_t *o = p.o;
    float *lse = p.lse;
    p.o = nullptr;
    p.lse = nullptr;
    p.o_part = o_part;
    p.lse_part = lse_part;
    p.split_len = c.split_len;
    p.n_split = c.n_split;
    p.part_offset = 0;
    p.n_split_total = c.n_split;
    int rc = launch_attention<true>(p, hd, stream);
    if (rc != FMHA_OK) return rc;
    MergeParams m{};
    m.o_part = o_part;
    m.lse_part = lse_part;
    m.o = o;
    m.lse = lse;
    m.o_sb = o_st.batch; m.o_st = o_st.token; m.o_sh = o_st.head;
    m.out_format = fmha::kOutBf16;
    return launch_merge(m, p.batch, p.n_h, p.T, hd, c.n_split, stream);
}

// ---- the static scratch of fmha_forward_noalloc -------------------------------
//
// For callers that cannot allocate (code under graph capture, serving loops
// that forbid it): the split path's partials go to this array instead of a
// workspace.  Every GPU the library runs on holds its own copy until the
// process ends.  In host code `scratch` names a host-side stand-in, not the
// device address: kernels and copies get the address hipGetSymbolAddress
// returns, fetched once per device and kept in scratch_ptr_of.
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void *scratch_ptr_of[kMaxDevices] = {};

// The scratch address on the current device (looked up on its first use).
int scratch_address(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return FMHA_ERR_LAUNCH;
    if (dev < 0 || dev >= kMaxDevices) return FMHA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(scratch_mutex);
    if (!scratch_ptr_of[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return FMHA_ERR_LAUNCH;
        scratch_ptr_of[dev] = ptr;
    }
    *out = scratch_ptr_of[dev];
    return FMHA_OK;
}

}  // namespace

extern "C" {

int fmha_forward(const void *q, const void *k, const void *v, void *o, float *lse, int batch, int n_h,
                 int n_kv_h, int T, int s_k, int hd, fmha_strides q_st, fmha_strides k_st, fmha_strides v_st,
                 fmha_strides o_st, float scale, int window, int causal, void *stream) {
    int rc = validate_attention(q, k, v, o, lse, false, batch, n_h, n_kv_h, T, s_k, hd, q_st, k_st, v_st, &o_st,
                                window, causal);
    if (rc != FMHA_OK) return rc;
    FwdParams p = make_params(q, k, v, batch, n_h, n_kv_h, T, s_k, q_st, k_st, v_st, scale, window, causal);
    p.o = static_cast<uint16_t *>(o);
    p.lse = lse;
    p.o_sb = o_st.batch; p.o_st = o_st.token; p.o_sh = o_st.head;
    p.split_len = s_k;
    p.n_split = 1;
    p.n_split_total = 1;
    return launch_attention<false>(p, hd, stream);
}

int fmha_forward_ws_size(int batch, int n_h, int n_kv_h, int T, int s_k, int hd, fmha_strides k_st,
                         fmha_strides v_st, int window, int causal, size_t *bytes) {
    if (!bytes) return FMHA_ERR_INVALID_ARG;
    const int rc = validate_dims(batch, n_h, n_kv_h, T, s_k, hd, window, causal, k_st, v_st);
    if (rc != FMHA_OK) return rc;
    const fmha_strides none{0, 0, 0};
    const FwdParams p = make_params(nullptr, nullptr, nullptr, batch, n_h, n_kv_h, T, s_k, none, k_st, v_st, 1.f,
                                    window, causal);
    const SplitChoice c = choose_split(p, hd);
    *bytes = c.split_len ? (size_t)split_workspace_bytes((int64_t)batch * n_h * T, c.n_split, hd) : 0;
    return FMHA_OK;
}

int fmha_forward_ws(const void *q, const void *k, const void *v, void *o, float *lse, int batch, int n_h,
                    int n_kv_h, int T, int s_k, int hd, fmha_strides q_st, fmha_strides k_st, fmha_strides v_st,
                    fmha_strides o_st, float scale, int window, int causal, void *workspace, size_t workspace_bytes,
                    void *stream) {
    int rc = validate_attention(q, k, v, o, lse, false, batch, n_h, n_kv_h, T, s_k, hd, q_st, k_st, v_st, &o_st,
                                window, causal);
    if (rc != FMHA_OK) return rc;
    FwdParams p = make_params(q, k, v, batch, n_h, n_kv_h, T, s_k, q_st, k_st, v_st, scale, window, causal);
    p.o = static_cast<uint16_t *>(o);
    p.lse = lse;
    p.o_sb = o_st.batch; p.o_st = o_st.token; p.o_sh = o_st.head;
    const SplitChoice c = choose_split(p, hd);
    if (c.split_len) {
        const int64_t need = split_workspace_bytes((int64_t)batch * n_h * T, c.n_split, hd);
        if (!workspace || (int64_t)workspace_bytes < need) return FMHA_ERR_WORKSPACE;
        if (!aligned16(workspace)) return FMHA_ERR_ALIGNMENT;
    }
    return forward_split_or_fused(p, hd, c, workspace, o_st, stream);
}

int fmha_forward_noalloc(const void *q, const void *k, const void *v, void *o, float *lse, int batch, int n_h,
                         int n_kv_h, int T, int s_k, int hd, fmha_strides q_st, fmha_strides k_st, fmha_strides v_st,
                         fmha_strides o_st, float scale, int window, int causal, void *stream) {
    int rc = validate_attention(q, k, v, o, lse, false, batch, n_h, n_kv_h, T, s_k, hd, q_st, k_st, v_st, &o_st,
                                window, causal);
    if (rc != FMHA_OK) return rc;
    FwdParams p = make_params(q, k, v, batch, n_h, n_kv_h, T, s_k, q_st, k_st, v_st, scale, window, causal);
    p.o = static_cast<uint16_t *>(o);
    p.lse = lse;
    p.o_sb = o_st.batch; p.o_st = o_st.token; p.o_sh = o_st.head;
    const SplitChoice c = choose_split(p, hd);
    void *ws = nullptr;
    if (c.split_len) {
        // every partial slot the merge reads is written by the split launch
        // first, so nothing in the scratch needs clearing between calls
        if (split_workspace_bytes((int64_t)batch * n_h * T, c.n_split, hd) > (int64_t)kScratchBytes)
            return FMHA_ERR_WORKSPACE;
        rc = scratch_address(&ws);
        if (rc != FMHA_OK) return rc;
    }
    return forward_split_or_fused(p, hd, c, ws, o_st, stream);
}

int fmha_forward_varlen(const void *q, const void *k, const void *v, const int *seqlens_k, void *o, float *lse,
                        int batch, int n_h, int n_kv_h, int T, int s_k_max, int hd, fmha_strides q_st,
                        fmha_strides k_st, fmha_strides v_st, fmha_strides o_st, float scale, int window, int causal,
                        void *stream) {
    if (!seqlens_k) return FMHA_ERR_INVALID_ARG;
    int rc = validate_attention(q, k, v, o, lse, false, batch, n_h, n_kv_h, T, s_k_max, hd, q_st, k_st, v_st,
                                &o_st, window, causal);
    if (rc != FMHA_OK) return rc;
    if ((reinterpret_cast<uintptr_t>(seqlens_k) & 3u) != 0) return FMHA_ERR_ALIGNMENT;
    FwdParams p = make_params(q, k, v, batch, n_h, n_kv_h, T, s_k_max, q_st, k_st, v_st, scale, window, causal);
    p.seqlens = seqlens_k;
    p.o = static_cast<uint16_t *>(o);
    p.lse = lse;
    p.o_sb = o_st.batch; p.o_st = o_st.token; p.o_sh = o_st.head;
    p.split_len = s_k_max;
    p.n_split = 1;
    p.n_split_total = 1;
    return launch_attention<false>(p, hd, stream);
}

int fmha_forward_mx(const void *q, const void *k, const void *v, void *o_codes, void *o_scales, float *lse,
                    int batch, int n_h, int n_kv_h, int T, int s_k, int hd, fmha_strides q_st, fmha_strides k_st,
                    fmha_strides v_st, float scale, int window, int causal, int format, void *stream) {
    if (!o_scales) return FMHA_ERR_INVALID_ARG;
    if (format != FMHA_MX_FP8_E4M3 && format != FMHA_MX_FP4_E2M1) return FMHA_ERR_INVALID_ARG;
    int rc = validate_attention(q, k, v, o_codes, lse, false, batch, n_h, n_kv_h, T, s_k, hd, q_st, k_st, v_st,
                                nullptr, window, causal);
    if (rc != FMHA_OK) return rc;
    FwdParams p = make_params(q, k, v, batch, n_h, n_kv_h, T, s_k, q_st, k_st, v_st, scale, window, causal);
    p.lse = lse;
    p.out_format = format;
    p.o_codes = static_cast<uint8_t *>(o_codes);
    p.o_scales = static_cast<uint8_t *>(o_scales);
    p.split_len = s_k;
    p.n_split = 1;
    p.n_split_total = 1;
    return launch_attention<false>(p, hd, stream);
}

int fmha_decode_splitkv_segment(const void *q, const void *k, const void *v, const int *seqlens_k, float *o_part,
                                float *lse_part, int batch, int n_h, int n_kv_h, int T, int s_k, int hd,
                                fmha_strides q_st, fmha_strides k_st, fmha_strides v_st, float scale, int window,
                                int causal, int split_len, int part_offset, int n_split_total, void *stream) {
    if (split_len <= 0 || part_offset < 0) return FMHA_ERR_INVALID_ARG;
    int rc = validate_attention(q, k, v, o_part, lse_part, true, batch, n_h, n_kv_h, T, s_k, hd, q_st, k_st, v_st,
                                nullptr, window, causal);
    if (rc != FMHA_OK) return rc;
    const int64_t n_split = ((int64_t)s_k + split_len - 1) / split_len;
    if ((int64_t)part_offset + n_split > n_split_total) return FMHA_ERR_INVALID_ARG;
    if (seqlens_k && (reinterpret_cast<uintptr_t>(seqlens_k) & 3u) != 0) return FMHA_ERR_ALIGNMENT;
    FwdParams p = make_params(q, k, v, batch, n_h, n_kv_h, T, s_k, q_st, k_st, v_st, scale, window, causal);
    p.seqlens = seqlens_k;
    p.o_part = o_part;
    p.lse_part = lse_part;
    p.split_len = split_len;
    p.n_split = (int)n_split;
    p.part_offset = part_offset;
    p.n_split_total = n_split_total;
    return launch_attention<true>(p, hd, stream);
}

int fmha_decode_splitkv(const void *q, const void *k, const void *v, float *o_part, float *lse_part, int batch,
                        int n_h, int n_kv_h, int T, int s_k, int hd, fmha_strides q_st, fmha_strides k_st,
                        fmha_strides v_st, float scale, int window, int causal, int split_len, void *stream) {
    if (split_len <= 0) return FMHA_ERR_INVALID_ARG;
    const int64_t n_split = ((int64_t)s_k + split_len - 1) / split_len;
    return fmha_decode_splitkv_segment(q, k, v, nullptr, o_part, lse_part, batch, n_h, n_kv_h, T, s_k, hd, q_st,
                                       k_st, v_st, scale, window, causal, split_len, 0,
                                       n_split > 0x7fffffff ? 0x7fffffff : (int)n_split, stream);
}

int fmha_lse_merge(const float *o_part, const float *lse_part, void *o, float *lse, int batch, int n_h, int T,
                   int hd, int n_split, fmha_strides o_st, void *stream) {
    if (!o_part || !lse_part || !o) return FMHA_ERR_INVALID_ARG;
    if (batch <= 0 || n_h <= 0 || T <= 0 || hd <= 0 || n_split <= 0) return FMHA_ERR_INVALID_ARG;
    if (!hd_supported(hd)) return FMHA_ERR_UNSUPPORTED;
    if (!aligned16(o_part) || !aligned16(lse_part) || !aligned16(o) || (lse && !aligned16(lse)))
        return FMHA_ERR_ALIGNMENT;
    if (!strides_ok(o_st)) return FMHA_ERR_ALIGNMENT;
    MergeParams p{};
    p.o_part = o_part;
    p.lse_part = lse_part;
    p.o = static_cast<uint16_t *>(o);
    p.lse = lse;
    p.o_sb = o_st.batch; p.o_st = o_st.token; p.o_sh = o_st.head;
    p.out_format = fmha::kOutBf16;
    return launch_merge(p, batch, n_h, T, hd, n_split, stream);
}

int fmha_lse_merge_mx(const float *o_part, const float *lse_part, void *o_codes, void *o_scales, float *lse,
                      int batch, int n_h, int T, int hd, int n_split, int format, void *stream) {
    if (!o_part || !lse_part || !o_codes || !o_scales) return FMHA_ERR_INVALID_ARG;
    if (format != FMHA_MX_FP8_E4M3 && format != FMHA_MX_FP4_E2M1) return FMHA_ERR_INVALID_ARG;
    if (batch <= 0 || n_h <= 0 || T <= 0 || hd <= 0 || n_split <= 0) return FMHA_ERR_INVALID_ARG;
    if (!hd_supported(hd)) return FMHA_ERR_UNSUPPORTED;
    if (!aligned16(o_part) || !aligned16(lse_part) || !aligned16(o_codes) || (lse && !aligned16(lse)))
        return FMHA_ERR_ALIGNMENT;
    MergeParams p{};
    p.o_part = o_part;
    p.lse_part = lse_part;
    p.lse = lse;
    p.out_format = format;
    p.o_codes = static_cast<uint8_t *>(o_codes);
    p.o_scales = static_cast<uint8_t *>(o_scales);
    return launch_merge(p, batch, n_h, T, hd, n_split, stream);
}

int fmha_attention_plan(int batch, int n_h, int n_kv_h, int T, int s_k, int hd, fmha_strides k_st,
                        fmha_strides v_st, int window, int causal, int split_len, fmha_plan *plan) {
    if (!plan || split_len < 0) return FMHA_ERR_INVALID_ARG;
    const int rc = validate_dims(batch, n_h, n_kv_h, T, s_k, hd, window, causal, k_st, v_st);
    if (rc != FMHA_OK) return rc;
    const fmha_strides none{0, 0, 0};
    FwdParams p = make_params(nullptr, nullptr, nullptr, batch, n_h, n_kv_h, T, s_k, none, k_st, v_st, 1.f,
                              window, causal);
    p.split_len = split_len == 0 ? s_k : split_len;
    p.n_split = (int)(((int64_t)s_k + p.split_len - 1) / p.split_len);
    *plan = plan_attention(p, hd, split_len > 0);
    // the same limit the launch applies
    if (!grid_fits(plan->workgroups, plan->threads_per_group)) return FMHA_ERR_UNSUPPORTED;
    return FMHA_OK;
}

const char *fmha_status_string(int status) {
    switch (status) {
        case FMHA_OK: return "FMHA_OK: success";
        case FMHA_ERR_INVALID_ARG: return "FMHA_ERR_INVALID_ARG: null pointer, non-positive size, n_h not a "
                                          "multiple of n_kv_h, bad mask arguments or split_len";
        case FMHA_ERR_UNSUPPORTED: return "FMHA_ERR_UNSUPPORTED: head dim must be 64, 128, 256 or 512, T at most 2^20, "
                                          "s_k at most 2^30 and (n_h / n_kv_h) * T at most 2^30";
        case FMHA_ERR_ALIGNMENT: return "FMHA_ERR_ALIGNMENT: pointers must be 16-byte aligned and strides multiples of 8 elements";
        case FMHA_ERR_LAUNCH: return "FMHA_ERR_LAUNCH: the HIP kernel launch failed";
        case FMHA_ERR_WORKSPACE: return "FMHA_ERR_WORKSPACE: the call needs a workspace of more bytes than were "
                                        "given (fmha_forward_ws_size tells how many; fmha_forward_noalloc has "
                                        "32 MiB of static scratch)";
        default: return "unknown fmha status";
    }
}

}  // extern "C"
