// merge_kernel.hpp -- the D5 merge of per-partition attention results.
//
// For each output row (b, h, t) with partials (O_p, lse_p), p < n_split:
//   M = max_p lse_p,  w_p = exp(lse_p - M)  (0 for lse_p = -inf)
//   O = sum_p w_p O_p / sum_p w_p,   lse = M + ln sum_p w_p
// which is O = sum_p exp(lse_p) O_p / sum_p exp(lse_p) with exp(M) factored
// out ("Next steps", item 4, of the CURRENT_ISSUE.md page).
//
// HBM-bound streaming.  A row is served by PG groups of HD/4 lanes; a lane
// owns four adjacent columns, and group g takes partitions g, g+PG, ...,
// reading each with one 16-byte load, UNROLL partitions in flight.  The PG
// partial sums are combined through LDS in a fixed order (deterministic).
#pragma once

#include "device_common.hpp"

namespace fmha {

struct MergeParams {
    const float *o_part;    // [rows][n_split][hd]
    const float *lse_part;  // [rows][n_split]
    uint16_t *o;            // bf16, strided [b][t][h][hd]
    float *lse;             // [b][n_h][T], may be null
    int64_t o_sb, o_st, o_sh;
    int n_h, T, rows, n_split;
};

template <int HD>
struct MergeShape {
    static constexpr int TPR = HD / 4;                         // lanes per row group
    static constexpr int PG = (256 / TPR) >= 4 ? 4 : 256 / TPR;  // partition groups per row
    static constexpr int RPW = 256 / (TPR * PG);                // rows per workgroup
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

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float den = 0.f, M = -INFINITY;
    if (live) {
        const float *lp = p.lse_part + (int64_t)row * p.n_split;
        const float *op = p.o_part + (int64_t)row * p.n_split * HD + col;
        for (int i = 0; i < p.n_split; ++i) M = fmaxf(M, lp[i]);
        if (M != -INFINITY) {
            int i = g;
            for (; i + (UNROLL - 1) * PG < p.n_split; i += UNROLL * PG) {
                f32x4 ov[UNROLL];
                float lv[UNROLL];
#pragma unroll
                for (int u = 0; u < UNROLL; ++u) {
                    lv[u] = lp[i + u * PG];
                    ov[u] = *reinterpret_cast<const f32x4 *>(op + (int64_t)(i + u * PG) * HD);
                }
#pragma unroll
                for (int u = 0; u < UNROLL; ++u) {
                    if (lv[u] != -INFINITY) {  // an empty partition carries no weight, whatever O_p holds
                        const float w = fast_exp2((lv[u] - M) * kLog2e);
                        den += w;
                        acc += w * ov[u];
                    }
                }
            }
            for (; i < p.n_split; i += PG) {
                const float li = lp[i];
                if (li != -INFINITY) {
                    const float w = fast_exp2((li - M) * kLog2e);
                    den += w;
                    acc += w * *reinterpret_cast<const f32x4 *>(op + (int64_t)i * HD);
                }
            }
        }
    }
    if constexpr (PG > 1) {
        red_acc[rib][g][lane_c] = acc;
        if (lane_c == 0) red_den[rib][g] = den;
        __syncthreads();
        if (g != 0) return;
        acc = red_acc[rib][0][lane_c];
        den = red_den[rib][0];
#pragma unroll
        for (int gg = 1; gg < PG; ++gg) {
            acc += red_acc[rib][gg][lane_c];
            den += red_den[rib][gg];
        }
    }
    if (!live) return;

    const int t = row % p.T;
    const int bh = row / p.T;
    const int h = bh % p.n_h;
    const int b = bh / p.n_h;
    const float inv = den > 0.f ? 1.f / den : 0.f;
    uint2 packed;
    packed.x = (uint32_t)bf16_bits(acc[0] * inv) | ((uint32_t)bf16_bits(acc[1] * inv) << 16);
    packed.y = (uint32_t)bf16_bits(acc[2] * inv) | ((uint32_t)bf16_bits(acc[3] * inv) << 16);
    *reinterpret_cast<uint2 *>(p.o + (int64_t)b * p.o_sb + (int64_t)t * p.o_st + (int64_t)h * p.o_sh + col) = packed;
    if (col == 0 && p.lse != nullptr) p.lse[row] = den > 0.f ? M + __logf(den) : -INFINITY;
}

}  // namespace fmha
