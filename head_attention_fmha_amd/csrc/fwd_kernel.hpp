// fwd_kernel.hpp -- fused attention kernel for gfx950.
//
// One workgroup computes a block of "rows" of one (batch, kv_head) pair
// over one key range.  A row is one (query position t, query head h) that
// reads this KV head: rows are numbered r = t * group + (h - kv*group), so
// GQA/MQA query heads that share K/V are stacked into the same MFMA tile
// and the rows of one tile sit at the same or adjacent positions (tight
// causal / window key ranges).
//
// Work split inside the workgroup: NWR x NWK waves.  Waves along NWR own
// different 16-row tiles; waves along NWK own different 32-key slices of
// each key chunk (key-parallel decode) and are merged at the end.  The
// chunk of CK = 32*NWK keys is staged in LDS once for all waves.
//
// The products are computed transposed, with keys in the MFMA M dimension:
//   S^T (keys x rows) = K (keys x hd) . Q^T (hd x rows)
//   O^T (hd x rows)  += V^T (hd x keys) . P^T (keys x rows)
// so every softmax statistic of row lr lives in lane lr (+16, +32, +48):
// the running max / sum / rescale factor are per-lane scalars, and the
// probabilities leave the first MFMA already in the register layout the
// second MFMA takes as its B operand.
//
// Online softmax (running max m, running sum l, rescale of the partial
// output by exp(m_old - m_new) when a new slice raises the max) follows the
// multi-tile kernel described in the e4ee9fdc commit log of the pages; the
// division by l happens exactly once, in the epilogue (the same log records
// the bug of normalising twice).  Scores are kept in the base-2 domain:
// x = (q.k) * scale * log2(e), so exp() is one v_exp_f32.
#pragma once

#include "device_common.hpp"

namespace fmha {

struct FwdParams {
    const uint16_t *q, *k, *v;
    uint16_t *o;      // forward mode: bf16 output (strided)
    float *lse;       // forward mode: [b][n_h][T], may be null
    float *o_part;    // split mode: [b][n_h][T][n_split][hd]
    float *lse_part;  // split mode: [b][n_h][T][n_split]
    int64_t q_sb, q_st, q_sh;
    int64_t k_sb, k_st, k_sh;
    int64_t v_sb, v_st, v_sh;
    int64_t o_sb, o_st, o_sh;
    int batch, n_h, n_kv_h, T, s_k;
    int group;        // n_h / n_kv_h
    int rows;         // group * T rows per (batch, kv_head)
    int window, causal;
    int split_len, n_split;
    int n_row_blocks;
    int n_units;      // gridDim.x
    int xcd_remap;    // 1: n_units % 8 == 0, give each XCD a contiguous unit range
    float scale_log2; // scale * log2(e)
};

template <int HD, int NWR, int NWK, bool SPLIT>
__global__ __launch_bounds__(64 * NWR * NWK) void fwd_kernel(const FwdParams p) {
    constexpr int NT = 64 * NWR * NWK;
    constexpr int CK = 32 * NWK;       // keys per LDS chunk
    constexpr int LDS_ROW = HD + 8;    // padded row (bf16 elements): 16 B skew per key row
    constexpr int KSTEPS = HD / 32;    // MFMA steps over the head dimension
    constexpr int NB = HD / 16;        // 16-wide head-dim blocks of O^T
    constexpr int PIECES = CK * HD / 8;  // 16-byte pieces per staged tensor

    constexpr int STAGE_ELEMS = 2 * CK * LDS_ROW;                      // K + V chunk (bf16)
    constexpr int MERGE_ELEMS = NWK > 1 ? NWR * NWK * (NB * 4 + 3) * 64 * 2 : 0;  // fp32 slots
    __shared__ __attribute__((aligned(16))) uint16_t smem[STAGE_ELEMS > MERGE_ELEMS ? STAGE_ELEMS : MERGE_ELEMS];
    uint16_t *sK = smem;
    uint16_t *sV = smem + CK * LDS_ROW;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wr = wave / NWK;
    const int wk = wave % NWK;
    const int lr = lane & 15;
    const int lg = lane >> 4;

    // ---- work unit ------------------------------------------------------
    int bid = blockIdx.x;
    if (p.xcd_remap) {
        const int per = p.n_units >> 3;
        bid = (bid & 7) * per + (bid >> 3);
    }
    const int rb = bid % p.n_row_blocks;
    bid /= p.n_row_blocks;
    const int part = bid % p.n_split;
    bid /= p.n_split;
    const int kvh = bid % p.n_kv_h;
    const int b = bid / p.n_kv_h;

    const int row0_wg = rb * 16 * NWR;
    const int row_last_wg = min(row0_wg + 16 * NWR, p.rows) - 1;
    const int pos_lo_wg = p.s_k - p.T + row0_wg / p.group;
    const int pos_hi_wg = p.s_k - p.T + row_last_wg / p.group;

    // key range of this workgroup: partition, then the union of the rows' masks
    int klo = part * p.split_len;
    int khi = min(klo + p.split_len, p.s_k);
    if (p.causal) khi = min(khi, pos_hi_wg + 1);
    if (p.window > 0) klo = max(klo, pos_lo_wg - p.window + 1);

    // ---- this lane's row --------------------------------------------------
    const int row = row0_wg + wr * 16 + lr;
    const bool row_ok = row < p.rows;
    const int t = row_ok ? row / p.group : 0;
    const int h = kvh * p.group + (row_ok ? row % p.group : 0);
    const int pos = p.s_k - p.T + t;
    int r_hi = p.causal ? min(khi, pos + 1) : khi;
    const int r_lo = p.window > 0 ? max(klo, pos - p.window + 1) : klo;
    if (!row_ok) r_hi = r_lo;  // no visible key: the row stays at -inf

    // Q^T as the B operand: lane holds Q[row lr][32*s + 8*lg + 0..7]
    bf16x8 qf[KSTEPS];
    {
        const uint16_t *qp = p.q + (int64_t)b * p.q_sb + (int64_t)t * p.q_st + (int64_t)h * p.q_sh + 8 * lg;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
            if (row_ok)
                qf[s] = *reinterpret_cast<const bf16x8 *>(qp + 32 * s);
            else
                qf[s] = bf16x8{};
        }
    }

    f32x4 acc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY;  // running max (base-2 domain), same in the 4 lanes of a row
    float l = 0.f;        // this lane's share of the running sum of exp (fp32): gives lse
    float lq = 0.f;       // the same sum over the bf16-rounded weights: normalises O

    const uint16_t *kbase = p.k + (int64_t)b * p.k_sb + (int64_t)kvh * p.k_sh;
    const uint16_t *vbase = p.v + (int64_t)b * p.v_sb + (int64_t)kvh * p.v_sh;

    for (int c = klo; c < khi; c += CK) {
        // ---- stage CK keys of K and V in LDS (zeros past khi) -------------
#pragma unroll
        for (int it = 0; it < (PIECES + NT - 1) / NT; ++it) {
            const int idx = threadIdx.x + it * NT;
            if (PIECES % NT == 0 || idx < PIECES) {
                const int key = idx / (HD / 8);
                const int col = (idx % (HD / 8)) * 8;
                const int gk = c + key;
                uint4 kx = {0u, 0u, 0u, 0u}, vx = {0u, 0u, 0u, 0u};
                if (gk < khi) {
                    kx = *reinterpret_cast<const uint4 *>(kbase + (int64_t)gk * p.k_st + col);
                    vx = *reinterpret_cast<const uint4 *>(vbase + (int64_t)gk * p.v_st + col);
                }
                *reinterpret_cast<uint4 *>(sK + key * LDS_ROW + col) = kx;
                *reinterpret_cast<uint4 *>(sV + key * LDS_ROW + col) = vx;
            }
        }
        __syncthreads();

        const int ks = 32 * wk;  // this wave's 32-key slice within the chunk
        const int k0 = c + ks;
        if (k0 < khi) {
            // ---- S^T = K . Q^T for two 16-key blocks ------------------------
            f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KSTEPS; ++s) {
                const bf16x8 a0 = *reinterpret_cast<const bf16x8 *>(sK + (ks + lr) * LDS_ROW + 32 * s + 8 * lg);
                const bf16x8 a1 = *reinterpret_cast<const bf16x8 *>(sK + (ks + 16 + lr) * LDS_ROW + 32 * s + 8 * lg);
                s0 = mfma_16x16x32(a0, qf[s], s0);
                s1 = mfma_16x16x32(a1, qf[s], s1);
            }
            // lane holds S^T[key k0 + 4*lg + j][row lr] (s0) and key k0 + 16 + 4*lg + j (s1)
            float x[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int ka = k0 + 4 * lg + j;
                const int kb = ka + 16;
                x[j] = (ka >= r_lo && ka < r_hi) ? s0[j] * p.scale_log2 : -INFINITY;
                x[4 + j] = (kb >= r_lo && kb < r_hi) ? s1[j] * p.scale_log2 : -INFINITY;
            }
            float mx = x[0];
#pragma unroll
            for (int j = 1; j < 8; ++j) mx = fmaxf(mx, x[j]);
            mx = fmaxf(mx, xor_shuffle(mx, 16));
            mx = fmaxf(mx, xor_shuffle(mx, 32));
            const float m_new = fmaxf(m, mx);
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            const float alpha = fast_exp2(m - m_use);
            bf16x8 pt;
            float psum = 0.f, qsum = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                // O is normalised by the sum of the same bf16 weights the PV
                // product consumes (an exact convex combination of V rows);
                // lse uses the unrounded sum
                const float pj = fast_exp2(x[j] - m_use);
                const __bf16 pb = to_bf16(pj);
                pt[j] = pb;
                psum += pj;
                qsum += (float)pb;
            }
            l = l * alpha + psum;
            lq = lq * alpha + qsum;
            m = m_new;
            // ---- O^T = alpha * O^T + V^T . P^T ------------------------------
            // the reduction index of item j of lane group lg is key
            // ks + 4*lg + j (j < 4) or ks + 16 + 4*lg + (j - 4) (j >= 4),
            // matching where those probabilities sit in pt
            const uint16_t *v0 = sV + (ks + 4 * lg) * LDS_ROW + lr;
            const uint16_t *v1 = v0 + 16 * LDS_ROW;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                bf16x8 vt;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    vt[j] = __builtin_bit_cast(__bf16, v0[j * LDS_ROW + 16 * nb]);
                    vt[4 + j] = __builtin_bit_cast(__bf16, v1[j * LDS_ROW + 16 * nb]);
                }
                acc[nb] = acc[nb] * alpha;
                acc[nb] = mfma_16x16x32(vt, pt, acc[nb]);
            }
        }
        __syncthreads();
    }

    // full row sums over the four lanes of the row
    l += xor_shuffle(l, 16);
    l += xor_shuffle(l, 32);
    lq += xor_shuffle(lq, 16);
    lq += xor_shuffle(lq, 32);

    // ---- merge the NWK key-slices of each row tile (fixed order) ------------
    if constexpr (NWK > 1) {
        constexpr int SLOTS = NB * 4 + 3;
        float *red = reinterpret_cast<float *>(smem);
        static_assert(NWR * NWK * SLOTS * 64 * 4 <= (int)sizeof(smem), "merge buffer exceeds LDS");
        float *mine = red + wave * SLOTS * 64 + lane;
        mine[0] = m;
        mine[64] = l;
        mine[128] = lq;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int j = 0; j < 4; ++j) mine[(3 + nb * 4 + j) * 64] = acc[nb][j];
        __syncthreads();
        if (wk != 0) return;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NWK; ++w) M = fmaxf(M, red[(wr * NWK + w) * SLOTS * 64 + lane]);
        const float M_use = (M == -INFINITY) ? 0.f : M;
        float L = 0.f, LQ = 0.f;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < NWK; ++w) {
            const float *src = red + (wr * NWK + w) * SLOTS * 64 + lane;
            const float wgt = fast_exp2(src[0] - M_use);
            L += wgt * src[64];
            LQ += wgt * src[128];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[nb][j] += wgt * src[(3 + nb * 4 + j) * 64];
        }
        m = M;
        l = L;
        lq = LQ;
    }

    if (!row_ok) return;

    // ---- epilogue: divide once by lq; lse = (m + log2 l) * ln 2 -------------
    const float inv = lq > 0.f ? 1.f / lq : 0.f;
    const float lse_val = l > 0.f ? (m + __log2f(l)) * kLn2 : -INFINITY;
    if constexpr (SPLIT) {
        const int64_t r = (((int64_t)b * p.n_h + h) * p.T + t) * p.n_split + part;
        float *op = p.o_part + r * HD + 4 * lg;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const f32x4 val = acc[nb] * inv;
            *reinterpret_cast<f32x4 *>(op + 16 * nb) = val;
        }
        if (lg == 0) p.lse_part[r] = lse_val;
    } else {
        uint16_t *op = p.o + (int64_t)b * p.o_sb + (int64_t)t * p.o_st + (int64_t)h * p.o_sh + 4 * lg;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            uint2 packed;
            packed.x = (uint32_t)bf16_bits(acc[nb][0] * inv) | ((uint32_t)bf16_bits(acc[nb][1] * inv) << 16);
            packed.y = (uint32_t)bf16_bits(acc[nb][2] * inv) | ((uint32_t)bf16_bits(acc[nb][3] * inv) << 16);
            *reinterpret_cast<uint2 *>(op + 16 * nb) = packed;
        }
        if (lg == 0 && p.lse != nullptr) p.lse[((int64_t)b * p.n_h + h) * p.T + t] = lse_val;
    }
}

}  // namespace fmha
