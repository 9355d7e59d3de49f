// rows_kernel.hpp -- row-parallel attention for prefill-shaped work (many
// query rows per KV head) on gfx950.
//
// One workgroup (4 waves) serves 64*RT consecutive stacked rows of one
// (batch, KV head, partition): wave w owns 16-row tiles w*RT .. w*RT + RT - 1
// of the block, over the FULL head dimension and EVERY key of the range.
// K/V are streamed through LDS in chunks of KC keys shared by all four
// waves, so each K/V byte leaves L2 once per 64*RT rows (the per-wave kernel of attn_kernel.hpp fetches it
// once per 16*MT rows).  This is the tiled prefill loop of the pages' fused
// kernel -- Q tile resident, K/V tiles staged on chip, online softmax state
// in registers -- laid out for CDNA4:
//   * a chunk travels HBM -> LDS by global_load_lds_dwordx4 (no registers),
//     double-buffered: chunk n+1 is in flight while chunk n is computed;
//   * LDS key row r holds its 16-byte column chunk c at slot
//     (c + 2*(r mod 8)) mod CHUNKS, for both K and V;
//   * S^T = K . Q^T with the K A-operand read from LDS (16 bytes per lane),
//     O^T += V^T . P^T with V^T from the transposing LDS read
//     ds_read_b64_tr_b16, P^T straight from the QK result registers -- the
//     same transposed-product scheme as attn_kernel.hpp (keys in the MFMA M
//     dimension, all softmax state of row lr in lanes lr + 16*lg).
// A wave skips the chunks that none of its rows sees (the causal upper
// triangle).
#pragma once

#include "device_common.hpp"
#include "mx_quant.hpp"
#include "params.hpp"

namespace fmha {

template <int HD, int RT, int KC>
struct RowsShape {
    static constexpr int KSTEPS = HD / 32;         // QK MFMA steps
    static constexpr int NB = HD / 16;             // 16-column blocks of O^T
    static constexpr int CHUNKS = HD / 8;          // 16-byte chunks per key row
    static constexpr int ROW_BYTES = HD * 2;
    static constexpr int KB = KC / 16;             // 16-key blocks per chunk
    static constexpr int KS = KC / 32;             // 32-key PV slices per chunk
    static constexpr int PART_BYTES = KC * ROW_BYTES;  // K (or V) part of a stage
    static constexpr int STAGE_BYTES = 2 * PART_BYTES;
    static constexpr int LOADS = PART_BYTES / (256 * 16);  // 16-byte loads per lane per part
    static constexpr int ROWS = 64 * RT;           // rows per workgroup
    static_assert(KC % 32 == 0 && PART_BYTES % (256 * 16) == 0, "whole wave-wide loads");
    static_assert(2 * STAGE_BYTES <= 160 * 1024, "two stages fit the LDS");
};

template <int HD, int RT, int KC, bool SPLIT>
__global__ __launch_bounds__(256, (2 * RowsShape<HD, RT, KC>::STAGE_BYTES <= 64 * 1024 ? 2 : 1)) void rows_kernel(
    const FwdParams p) {
    using S = RowsShape<HD, RT, KC>;
    constexpr int KSTEPS = S::KSTEPS, NB = S::NB, CHUNKS = S::CHUNKS, ROW_BYTES = S::ROW_BYTES;
    constexpr int KB = S::KB, KS = S::KS, PART_BYTES = S::PART_BYTES, STAGE_BYTES = S::STAGE_BYTES;
    constexpr int LOADS = S::LOADS;
    // two stages as two LDS objects, used alternately by a loop unrolled by
    // two: the compiler can then tell the prefetch into one stage from the
    // reads of the other and need not wait for the prefetch before them
    __shared__ __attribute__((aligned(16))) unsigned char stage0[STAGE_BYTES];
    __shared__ __attribute__((aligned(16))) unsigned char stage1[STAGE_BYTES];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lr = lane & 15;
    const int lg = lane >> 4;

    // ---- work unit (row blocks fastest, last block first; regrouped per XCD
    // when they share K/V) -- the same order as attn_kernel.hpp
    int bid = blockIdx.x;
    if (p.xcd_remap) {
        const int per = p.n_units >> 3;
        bid = (bid & 7) * per + (bid >> 3);
    }
    const int rb = p.n_row_blocks - 1 - bid % p.n_row_blocks;
    bid /= p.n_row_blocks;
    const int part = bid % p.n_split;
    bid /= p.n_split;
    const int kvh = bid % p.n_kv_h;
    const int b = bid / p.n_kv_h;
    // keys of this batch row: s_k, or the row's own length in a ragged batch
    // (clamped to the cache capacity s_k)
    const int s_k = p.seqlens ? min(max(p.seqlens[b], 0), p.s_k) : p.s_k;

    const int row0 = rb * S::ROWS;
    const int row_last = min(row0 + S::ROWS, p.rows) - 1;
    // key range: the partition, cut to the union of the block rows' masks
    int klo = part * p.split_len;
    int khi = min(klo + p.split_len, s_k);
    if (p.causal) khi = min(khi, s_k - p.T + row_last / p.group + 1);
    if (p.window > 0) klo = max(klo, s_k - p.T + row0 / p.group - p.window + 1);

    // ---- this wave's tiles: rows, masks, and the key range of each tile ----
    bool row_ok[RT];
    int t_of[RT], h_of[RT], r_lo[RT], r_hi[RT], tile_lo[RT], tile_hi[RT], full_lo[RT], full_hi[RT];
#pragma unroll
    for (int mt = 0; mt < RT; ++mt) {
        const int first = row0 + 16 * (wave * RT + mt);
        const int last = min(first + 15, row_last);
        const int row = first + lr;
        row_ok[mt] = row <= row_last;
        t_of[mt] = row_ok[mt] ? row / p.group : 0;
        h_of[mt] = kvh * p.group + (row_ok[mt] ? row % p.group : 0);
        const int pos = s_k - p.T + t_of[mt];
        r_hi[mt] = p.causal ? min(khi, pos + 1) : khi;
        r_lo[mt] = p.window > 0 ? max(klo, pos - p.window + 1) : klo;
        if (!row_ok[mt]) r_hi[mt] = r_lo[mt];
        // wave-uniform bounds of the keys any row of the tile can see
        if (first > row_last) {
            tile_lo[mt] = khi;
            tile_hi[mt] = klo;  // empty tile
            full_lo[mt] = khi;
            full_hi[mt] = klo;
        } else {
            const int pos_first = s_k - p.T + first / p.group;
            const int pos_last = s_k - p.T + last / p.group;
            tile_hi[mt] = p.causal ? min(khi, pos_last + 1) : khi;
            tile_lo[mt] = p.window > 0 ? max(klo, pos_first - p.window + 1) : klo;
            // keys visible to EVERY row of the tile: chunks inside need no mask
            // (rows past the end of the block hold Q = 0 and are never stored)
            full_hi[mt] = p.causal ? min(khi, pos_first + 1) : khi;
            full_lo[mt] = p.window > 0 ? max(klo, pos_last - p.window + 1) : klo;
        }
    }

    // Scores enter the softmax as s * c with c = |scale| log2 e >= 0: a
    // negative scale flips the sign of Q instead (exact in bf16), so the
    // running maximum can be kept on raw scores and the scaling folded into
    // the exponent's fma.
    const float c_scale = fabsf(p.scale_log2);
    const unsigned q_flip = p.scale_log2 < 0.f ? 0x80008000u : 0u;
    bf16x8 qf[RT][KSTEPS];  // Q^T B operand: Q[row lr][32*s + 8*lg + 0..7]
#pragma unroll
    for (int mt = 0; mt < RT; ++mt) {
        const uint16_t *qp =
            p.q + (int64_t)b * p.q_sb + (int64_t)t_of[mt] * p.q_st + (int64_t)h_of[mt] * p.q_sh + 8 * lg;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
            u32x4 raw = row_ok[mt] ? *reinterpret_cast<const u32x4 *>(qp + 32 * s) : u32x4{0u, 0u, 0u, 0u};
            raw ^= q_flip;
            qf[mt][s] = __builtin_bit_cast(bf16x8, raw);
        }
    }

    f32x4 acc[RT][NB];
    f32x4 accq[RT];  // every element: the running sum of row lr's bf16 weights (-> O)
    float m[RT], l[RT];
#pragma unroll
    for (int mt = 0; mt < RT; ++mt) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[mt][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
        accq[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        m[mt] = -INFINITY;  // running max (base 2), equal in the 4 lanes of a row
        l[mt] = 0.f;        // this lane's share of the fp32 sum of weights (-> lse)
    }
    // A operand of ones: one MFMA per 32-key slice sums the bf16 weights the PV
    // product consumes, already complete in every lane of the row
    bf16x8 ones;
#pragma unroll
    for (int j = 0; j < 8; ++j) ones[j] = (__bf16)1.0f;

    const uint16_t *kbase = p.k + (int64_t)b * p.k_sb + (int64_t)kvh * p.k_sh;
    const uint16_t *vbase = p.v + (int64_t)b * p.v_sb + (int64_t)kvh * p.v_sh;
    auto rot_of = [](int r) __attribute__((always_inline)) { return (2 * (r & 7)) % CHUNKS; };

    // ---- one chunk HBM -> LDS stage: wave w fills bytes [w*LOADS*1 KiB, ...)
    // of each part; the lane writing LDS byte x of a part fetches the global
    // chunk that belongs at x under the rotation.  The lane's row and chunk
    // are fixed, so its byte offset from the chunk's first key is computed
    // once; a chunk then costs one scalar base per tensor.  The last chunk
    // of a range clamps keys past khi to key khi-1 instead.
    int ld_row[LOADS], ld_col[LOADS];
    unsigned ld_koff[LOADS], ld_voff[LOADS];
    const bool offsets32 = (int64_t)(KC - 1) * (p.k_st > p.v_st ? p.k_st : p.v_st) * 2 + ROW_BYTES < (1ll << 31);
#pragma unroll
    for (int it = 0; it < LOADS; ++it) {
        const int x = ((wave * LOADS + it) * 64 + lane) * 16;  // LDS byte of this lane
        ld_row[it] = x / ROW_BYTES;
        ld_col[it] = ((x % ROW_BYTES) / 16 - rot_of(ld_row[it]) + CHUNKS) % CHUNKS;
        ld_koff[it] = (unsigned)(((int64_t)ld_row[it] * p.k_st + ld_col[it] * 8) * 2);
        ld_voff[it] = (unsigned)(((int64_t)ld_row[it] * p.v_st + ld_col[it] * 8) * 2);
    }
    auto issue_chunk = [&](int k0, unsigned char *stage) __attribute__((always_inline)) {
        unsigned char *sK = stage;
        unsigned char *sV = stage + PART_BYTES;
        if (offsets32 && k0 + KC <= khi) {  // wave-uniform
            const char *kc = reinterpret_cast<const char *>(kbase + (int64_t)k0 * p.k_st);
            const char *vc = reinterpret_cast<const char *>(vbase + (int64_t)k0 * p.v_st);
#pragma unroll
            for (int it = 0; it < LOADS; ++it) {
                load_lds_16(kc + ld_koff[it], sK + (wave * LOADS + it) * 1024);
                load_lds_16(vc + ld_voff[it], sV + (wave * LOADS + it) * 1024);
            }
        } else {
#pragma unroll
            for (int it = 0; it < LOADS; ++it) {
                const int key = min(k0 + ld_row[it], khi - 1);
                load_lds_16(kbase + key_offset(key, p.k_st) + ld_col[it] * 8, sK + (wave * LOADS + it) * 1024);
                load_lds_16(vbase + key_offset(key, p.v_st) + ld_col[it] * 8, sV + (wave * LOADS + it) * 1024);
            }
        }
    };

    // V^T transposing-read coordinates (see attn_kernel.hpp): lane s of block
    // lg addresses key 4*lg + s/4 (+16) of a 32-key slice, columns 4*(s%4)..+3
    const int tr_row0 = 4 * lg + (lr >> 2);
    const int tr_col = 4 * (lr & 3);

    // ---- the products of one staged chunk for every tile of this wave.  Each
    // K operand and each V^T operand read from LDS feeds the MFMAs of all the
    // wave's tiles.  Once any tile sees the chunk, every tile's products are
    // issued, free of branches (which would split the MFMA/LDS schedule into
    // small blocks); a tile that sees none of its keys gets weights 0.
    auto compute_chunk = [&](int k0, const unsigned char *sK) __attribute__((always_inline)) {
        const unsigned char *sV = sK + PART_BYTES;
        bool live[RT];  // wave-uniform: does any row of the tile see a key of the chunk?
        bool any_live = false;
#pragma unroll
        for (int mt = 0; mt < RT; ++mt) {
            live[mt] = k0 < tile_hi[mt] && k0 + KC > tile_lo[mt];
            any_live = any_live || live[mt];
        }
        if (!any_live) return;
        // ---- S^T for the chunk: KB blocks of 16 keys
        f32x4 sc[RT][KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const int r = 16 * kb + lr;
            const unsigned char *krow = sK + r * ROW_BYTES;
#pragma unroll
            for (int mt = 0; mt < RT; ++mt) sc[mt][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KSTEPS; ++s) {
                const int slot = (4 * s + lg + rot_of(r)) % CHUNKS;
                const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(krow + slot * 16);
#pragma unroll
                for (int mt = 0; mt < RT; ++mt) sc[mt][kb] = mfma_16x16x32(kf, qf[mt][s], sc[mt][kb]);
            }
        }
        // ---- online softmax over the chunk's keys, per tile.  The maximum is
        // taken on raw scores (masked keys excluded only in chunks that cut
        // through some row's range); the reference point m moves -- rescaling
        // the accumulators -- only when some row of the wave exceeds it by
        // more than 2^8, so weights stay below 256 and most chunks rescale
        // nothing
        bf16x8 pt[RT][KS];
#pragma unroll
        for (int mt = 0; mt < RT; ++mt) {
            if (!live[mt]) {  // weights 0: the tile's products below add nothing
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) pt[mt][ks] = bf16x8{};
                continue;
            }
            const bool full = k0 >= full_lo[mt] && k0 + KC <= full_hi[mt];  // wave-uniform
            bool vis[KB][4];
            float mr = -INFINITY;
            if (full) {
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int j = 0; j < 4; ++j) mr = fmaxf(mr, sc[mt][kb][j]);
            } else {
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int key = k0 + 16 * kb + 4 * lg + j;
                        vis[kb][j] = key >= r_lo[mt] && key < r_hi[mt];
                        mr = fmaxf(mr, vis[kb][j] ? sc[mt][kb][j] : -INFINITY);
                    }
            }
            mr = row4_max(mr);
            const float mx = mr * c_scale;  // NaN (ignored by fmaxf) for a fully masked row when c = 0
            if (__any(mx > m[mt] + kRescaleLog2)) {
                const float m_new = fmaxf(m[mt], mx);
                const float alpha = fast_exp2(m[mt] - ((m_new == -INFINITY) ? 0.f : m_new));
                l[mt] *= alpha;
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) acc[mt][nb] = acc[mt][nb] * alpha;
                accq[mt] = accq[mt] * alpha;
                m[mt] = m_new;
            }
            const float neg_m = (m[mt] == -INFINITY) ? 0.f : -m[mt];
            float psum = 0.f;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float xj = fmaf(sc[mt][kb][j], c_scale, neg_m);
                    if (!full) xj = vis[kb][j] ? xj : -INFINITY;
                    const float pj = fast_exp2(xj);
                    pt[mt][kb >> 1][(kb & 1) * 4 + j] = to_bf16(pj);
                    psum += pj;
                }
            l[mt] += psum;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) accq[mt] = mfma_16x16x32(ones, pt[mt][ks], accq[mt]);
        }
        // ---- O^T += V^T . P^T
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                bf16x4 q2[2];
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const int r = 32 * ks + 16 * half + tr_row0;
                    const int c = 16 * nb + tr_col;
                    const int off = r * ROW_BYTES + (((c >> 3) + rot_of(r)) % CHUNKS) * 16 + (c & 7) * 2;
                    q2[half] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                        (__attribute__((address_space(3))) bf16x4 *)(sV + off));
                }
                const bf16x8 vt = __builtin_shufflevector(q2[0], q2[1], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
                for (int mt = 0; mt < RT; ++mt) acc[mt][nb] = mfma_16x16x32(vt, pt[mt][ks], acc[mt][nb]);
            }
        }
    };

    // chunk n+1 is fetched into the other stage while chunk n is computed
    auto step = [&](int n, int nchunks, unsigned char *cur, unsigned char *next) __attribute__((always_inline)) {
        const int k0 = klo + n * KC;
        if (n + 1 < nchunks) {
            issue_chunk(k0 + KC, next);
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * LOADS));  // this wave's part of chunk n has landed
        } else {
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        }
        lds_barrier();  // ... and every wave's part
        compute_chunk(k0, cur);
        lds_barrier();  // every wave is done with this stage before it is refilled
    };

    // Two chunks per iteration.  Chunk n+2 (fetched during chunk n+1) is
    // waited for before the back-edge, after chunk n+1's products: no
    // LDS-direct load crosses the back-edge, which the compiler's wait
    // placement would otherwise answer with a wait for all loads before the
    // first LDS read of the iteration -- the prefetch included.
    const int nchunks = khi > klo ? (khi - klo + KC - 1) / KC : 0;
    if (nchunks > 0) issue_chunk(klo, stage0);
    for (int n = 0; n < nchunks; n += 2) {
        step(n, nchunks, stage0, stage1);
        if (n + 1 < nchunks) {
            step(n + 1, nchunks, stage1, stage0);
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        }
    }

    // ---- epilogue: full row sums, one division, lse = (m + log2 l) ln 2 ------
#pragma unroll
    for (int mt = 0; mt < RT; ++mt) {
        l[mt] = row4_sum(l[mt]);
        if (!row_ok[mt]) continue;
        const int t = t_of[mt], h = h_of[mt];
        const float lq = accq[mt][0];
        const float inv = lq > 0.f ? 1.f / lq : 0.f;
        const float lse_val = l[mt] > 0.f ? (m[mt] + __log2f(l[mt])) * kLn2 : -INFINITY;
        if constexpr (SPLIT) {
            const int64_t r = (((int64_t)b * p.n_h + h) * p.T + t) * p.n_split_total + p.part_offset + part;
            float *op = p.o_part + r * HD + 4 * lg;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                __builtin_nontemporal_store(acc[mt][nb] * inv, reinterpret_cast<f32x4 *>(op + 16 * nb));
            if (lg == 0) p.lse_part[r] = lse_val;
        } else if (p.out_format != kOutBf16) {
            // MX codes: 32-column blocks = pairs of 16-column blocks over the row's 4 lanes
            const int64_t orow = ((int64_t)b * p.T + t) * p.n_h + h;
            uint8_t *crow = p.o_codes + orow * (p.out_format == kOutMxFp8E4M3 ? HD : HD / 2);
            uint8_t *srow = p.o_scales + orow * (HD / 32);
#pragma unroll
            for (int nb = 0; nb < NB; nb += 2) {
                float v[8];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    v[j] = acc[mt][nb][j] * inv;
                    v[4 + j] = acc[mt][nb + 1][j] * inv;
                }
                mx_store_block_4lanes(v, p.out_format, crow, srow, 16 * nb, lg);
            }
            if (lg == 0 && p.lse != nullptr) p.lse[((int64_t)b * p.n_h + h) * p.T + t] = lse_val;
        } else {
            uint16_t *op = p.o + (int64_t)b * p.o_sb + (int64_t)t * p.o_st + (int64_t)h * p.o_sh + 4 * lg;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                uint2 packed;
                packed.x = (uint32_t)bf16_bits(acc[mt][nb][0] * inv) |
                           ((uint32_t)bf16_bits(acc[mt][nb][1] * inv) << 16);
                packed.y = (uint32_t)bf16_bits(acc[mt][nb][2] * inv) |
                           ((uint32_t)bf16_bits(acc[mt][nb][3] * inv) << 16);
                *reinterpret_cast<uint2 *>(op + 16 * nb) = packed;
            }
            if (lg == 0 && p.lse != nullptr) p.lse[((int64_t)b * p.n_h + h) * p.T + t] = lse_val;
        }
    }
}

}  // namespace fmha
