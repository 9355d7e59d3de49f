// merge_kernel.hpp -- the D5 merge of per-partition attention results.
//
// For each output row (b, h, t) with partials (O_p, lse_p), p < n_split:
//   M = max_p lse_p,  w_p = exp(lse_p - M)  (0 for lse_p = -inf)
//   O = sum_p w_p O_p / sum_p w_p,   lse = M + ln sum_p w_p
// which is O = sum_p exp(lse_p) O_p / sum_p exp(lse_p) with exp(M) factored
// out ("Next steps", item 4, of the CURRENT_ISSUE.md page).
//
// Bandwidth-bound streaming.  A row is served by PG groups of HD/4 lanes; a lane
// owns four adjacent columns, and group g takes partitions g, g+PG, ...,
// reading each with one 16-byte load, UNROLL partitions in flight.  The PG
// partial sums are combined through LDS in a fixed order (deterministic).
#pragma once

#include "device_common.hpp"
#include "mx_quant.hpp"

namespace fmha {

struct MergeParams {
    const float *o_part;    // [rows][n_split][hd]
    const float *lse_part;  // [rows][n_split]
    uint16_t *o;            // bf16, strided [b][t][h][hd]
    float *lse;             // [b][n_h][T], may be null
    int64_t o_sb, o_st, o_sh;
    int n_h, T, rows, n_split;
    int out_format;         // OutFormat: bf16 o, or MX codes + scales
    uint8_t *o_codes;       // MX: dense [b][T][n_h][hd] (E4M3) or [..][hd / 2] (E2M1)
    uint8_t *o_scales;      // MX: dense [b][T][n_h][hd / 32]
};

// One row per workgroup: 256 / (HD/4) partition groups (16, 8, 4, 2 for hd
// 64..512), so a 64-partition row is read in a single round of loads.
template <int HD>
struct MergeShape {
    static constexpr int TPR = HD / 4;     // lanes per row group
    static constexpr int PG = 256 / TPR;   // partition groups per row
    static constexpr int RPW = 1;          // rows per workgroup
};

template <int HD>
__global__ __launch_bounds__(256) void merge_kernel(const MergeParams p) {
    constexpr int TPR = MergeShape<HD>::TPR;
    constexpr int PG = MergeShape<HD>::PG;
    constexpr int RPW = MergeShape<HD>::RPW;
    constexpr int UNROLL = 8;
    __shared__ f32x4 red_acc[RPW][PG][TPR];
    __shared__ float red_den[RPW][PG];

    const int slot = threadIdx.x / TPR;  // (row in block, partition group)
    const int rib = slot / PG;
    const int g = slot % PG;
    const int lane_c = threadIdx.x % TPR;
    const int col = lane_c * 4;
    const int row = blockIdx.x * RPW + rib;
    const bool live = row < p.rows;

    // running maximum over this group's partitions (base-2 domain): a larger
    // lse rescales what has been summed so far, so the partial outputs are
    // loaded from the start without a separate pass over the lse values
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float den = 0.f, M = -INFINITY;
    if (live) {
        const float *lp = p.lse_part + (int64_t)row * p.n_split;
        const float *op = p.o_part + (int64_t)row * p.n_split * HD + col;
        for (int i0 = g; i0 < p.n_split; i0 += UNROLL * PG) {
            f32x4 ov[UNROLL];
            float lv[UNROLL];
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                const int i = i0 + u * PG;
                const bool in = i < p.n_split;
                lv[u] = in ? lp[i] * kLog2e : -INFINITY;
                // each partial is read once, in whole cache lines: non-temporal
                ov[u] = in ? __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(op + (int64_t)i * HD))
                           : f32x4{0.f, 0.f, 0.f, 0.f};
            }
            float mb = M;
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) mb = fmaxf(mb, lv[u]);
            if (mb == -INFINITY) continue;  // nothing visible yet
            if (mb > M) {
                const float r = fast_exp2(M - mb);  // 0 when M = -inf
                den *= r;
                acc = acc * r;
                M = mb;
            }
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                if (lv[u] != -INFINITY) {  // an empty partition carries no weight, whatever O_p holds
                    const float w = fast_exp2(lv[u] - M);
                    den += w;
                    acc += w * ov[u];
                }
            }
        }
    }
    if constexpr (PG > 1) {
        __shared__ float red_max[RPW][PG];
        red_acc[rib][g][lane_c] = acc;
        if (lane_c == 0) {
            red_den[rib][g] = den;
            red_max[rib][g] = M;
        }
        __syncthreads();
        if (g != 0) return;
        float Mall = M;
#pragma unroll
        for (int gg = 1; gg < PG; ++gg) Mall = fmaxf(Mall, red_max[rib][gg]);
        if (Mall != -INFINITY) {
            acc = {0.f, 0.f, 0.f, 0.f};
            den = 0.f;
#pragma unroll
            for (int gg = 0; gg < PG; ++gg) {
                const float mg = red_max[rib][gg];
                if (mg == -INFINITY) continue;
                const float r = fast_exp2(mg - Mall);
                acc += r * red_acc[rib][gg][lane_c];
                den += r * red_den[rib][gg];
            }
        }
        M = Mall;
    }
    if (!live) return;

    const int t = row % p.T;
    const int bh = row / p.T;
    const int h = bh % p.n_h;
    const int b = bh / p.n_h;
    const float inv = den > 0.f ? 1.f / den : 0.f;
    if (p.out_format != kOutBf16) {
        // a 32-column block is held by 8 adjacent lanes (TPR is a multiple of 8)
        const int64_t orow = ((int64_t)b * p.T + t) * p.n_h + h;
        const float v[4] = {acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
        mx_store_block_8lanes(v, p.out_format, p.o_codes + orow * (p.out_format == kOutMxFp8E4M3 ? HD : HD / 2),
                              p.o_scales + orow * (HD / 32), col & ~31, lane_c & 7);
    } else {
        uint2 packed;
        packed.x = (uint32_t)bf16_bits(acc[0] * inv) | ((uint32_t)bf16_bits(acc[1] * inv) << 16);
        packed.y = (uint32_t)bf16_bits(acc[2] * inv) | ((uint32_t)bf16_bits(acc[3] * inv) << 16);
        *reinterpret_cast<uint2 *>(p.o + (int64_t)b * p.o_sb + (int64_t)t * p.o_st + (int64_t)h * p.o_sh + col) =
            packed;
    }
    if (col == 0 && p.lse != nullptr) p.lse[row] = den > 0.f ? (M + __log2f(den)) * kLn2 : -INFINITY;
}

}  // namespace fmha
