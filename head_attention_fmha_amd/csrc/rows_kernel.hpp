// rows_kernel.hpp -- row-parallel attention for prefill-shaped work (many
// query rows per KV head) on gfx950, hd 64 to 256 (hd 512:
// rows_split_kernel.hpp).
//
// One workgroup (4 waves) serves 64*RT consecutive stacked rows of one
// (batch, KV head, partition): wave w owns 16-row tiles w*RT .. w*RT + RT - 1
// of the block, over the FULL head dimension and EVERY key of the range.
// K/V are streamed through LDS in chunks of KC keys shared by all four
// waves, so each K/V byte leaves L2 once per 64*RT rows (the per-wave
// kernel of attn_kernel.hpp fetches it once per 16*MT rows).  This is the tiled prefill loop of the pages' fused
// kernel -- Q tile resident, K/V tiles staged on chip, online softmax state
// in registers -- laid out for CDNA4:
//   * a chunk travels HBM -> LDS by buffer_load_dwordx4 ... lds (no
//     registers; the buffer form, unlike global_load_lds, leaves the
//     compiler's waits for LDS reads exact) into one of two K and two V
//     slots; K runs one chunk ahead of V, so the QK product of chunk n+1 is
//     issued together with the softmax of chunk n (independent MFMA and
//     vector work in one basic block, which the hardware overlaps) and
//     chunk n's PV product;
//   * LDS key row r holds its 16-byte column chunk c at slot
//     (c + 2*(r mod 8)) mod CHUNKS, for both K and V;
//   * S^T = K . Q^T with the K A-operand read from LDS (16 bytes per lane),
//     O^T += V^T . P^T with V^T from the transposing LDS read
//     ds_read_b64_tr_b16, P^T straight from the QK result registers -- the
//     same transposed-product scheme as attn_kernel.hpp (keys in the MFMA M
//     dimension, all softmax state of row lr in lanes lr + 16*lg).
// A wave computes every chunk of the workgroup's range; keys its rows do not
// see (the causal diagonal, at most one chunk per wave) get weight 0.
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
    static constexpr int PART_BYTES = KC * ROW_BYTES;  // K (or V) bytes of one chunk
    static constexpr int LOADS = PART_BYTES / (256 * 16);  // 16-byte loads per lane per slot
    static constexpr int ROWS = 64 * RT;           // rows per workgroup
    static constexpr int SLOT_BYTES = PART_BYTES;  // one K or V chunk in LDS
    static_assert(KC % 32 == 0 && PART_BYTES % (256 * 16) == 0, "whole wave-wide loads");
    // four slots: 32 or 64 KiB (two workgroups per CU)
    static_assert(4 * SLOT_BYTES <= 80 * 1024, "four slots leave room for two workgroups per CU");
};

template <int HD, int RT, int KC, bool SPLIT>
__global__ __launch_bounds__(256, 2) void rows_kernel(const FwdParams p) {
    using S = RowsShape<HD, RT, KC>;
    constexpr int KSTEPS = S::KSTEPS, NB = S::NB, CHUNKS = S::CHUNKS, ROW_BYTES = S::ROW_BYTES;
    constexpr int KB = S::KB, KS = S::KS, SLOT_BYTES = S::SLOT_BYTES;
    constexpr int LOADS = S::LOADS;
    // two K and two V slots as four LDS objects, used in turn by a loop
    // unrolled by two: the compiler can then tell each prefetch from the
    // reads of the other slot and need not wait for the prefetch before them
    __shared__ __attribute__((aligned(16))) unsigned char sK0[SLOT_BYTES];
    __shared__ __attribute__((aligned(16))) unsigned char sK1[SLOT_BYTES];
    __shared__ __attribute__((aligned(16))) unsigned char sV0[SLOT_BYTES];
    __shared__ __attribute__((aligned(16))) unsigned char sV1[SLOT_BYTES];

    fetch_launch_params(p);
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
    int t_of[RT], h_of[RT], r_lo[RT], r_hi[RT], full_lo[RT], full_hi[RT];
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
        // wave-uniform bounds of the keys visible to EVERY row of the tile:
        // chunks inside need no mask (an empty tile has none)
        if (first > row_last) {
            full_lo[mt] = khi;
            full_hi[mt] = klo;
        } else {
            const int pos_first = s_k - p.T + first / p.group;
            const int pos_last = s_k - p.T + last / p.group;
            // (rows past the end of the block hold Q = 0 and are never stored)
            full_hi[mt] = p.causal ? min(khi, pos_first + 1) : khi;
            full_lo[mt] = p.window > 0 ? max(klo, pos_last - p.window + 1) : klo;
        }
    }

    // Scores enter the softmax as s * c with c = |scale| log2 e > 0: a
    // negative scale flips the sign of Q instead (exact in bf16), so the
    // running maximum can be kept on raw scores and the scaling folded into
    // the exponent's fma.  A zero scale is taken as the smallest normal
    // float, so that a masked score (-inf) still scales to -inf: scaled
    // scores then stay below 2^-26 in magnitude for |s| < 2^100 and every
    // weight rounds to exactly 1, as with the scale 0 itself.
    const float c_scale = fmaxf(fabsf(p.scale_log2), FLT_MIN);
    const unsigned q_flip = p.scale_log2 < 0.f ? 0x80008000u : 0u;
    // Q^T B operand: Q[row lr][32*s + 8*lg + 0..7], loaded unconditionally (a
    // row past the end reads row 0 of the group, valid memory) and zeroed and
    // sign-flipped only once the first chunks' loads are issued: a load under
    // a lane condition, or one used right away, was waited for on the spot,
    // a full memory round trip before the first K/V load went out
    u32x4 qraw[RT][KSTEPS];
#pragma unroll
    for (int mt = 0; mt < RT; ++mt) {
        const uint16_t *qp =
            p.q + (int64_t)b * p.q_sb + (int64_t)t_of[mt] * p.q_st + (int64_t)h_of[mt] * p.q_sh + 8 * lg;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) qraw[mt][s] = *reinterpret_cast<const u32x4 *>(qp + 32 * s);
    }
    bf16x8 qf[RT][KSTEPS];
    auto finish_q = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int mt = 0; mt < RT; ++mt)
#pragma unroll
            for (int s = 0; s < KSTEPS; ++s)
                qf[mt][s] = __builtin_bit_cast(bf16x8, (qraw[mt][s] & (row_ok[mt] ? 0xffffffffu : 0u)) ^ q_flip);
    };

    f32x4 acc[RT][NB];
    f32x4 accq[RT];  // every element: the running sum of row lr's bf16 weights (-> O)
    float m[RT], neg_m[RT], l[RT];
#pragma unroll
    for (int mt = 0; mt < RT; ++mt) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[mt][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
        accq[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        m[mt] = -INFINITY;  // running max (base 2), equal in the 4 lanes of a row
        neg_m[mt] = 0.f;    // -m, or 0 while m = -inf (every weight is then 0)
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

    // ---- one chunk HBM -> an LDS slot: wave w issues loads w*LOADS ..
    // w*LOADS + LOADS-1, each 1 KiB of consecutive LDS bytes covering key rows
    // r0 .. r0 + 1024/ROW_BYTES - 1 of the chunk; the lane writing LDS byte x
    // fetches the global chunk that belongs at x under the rotation (a shifted
    // row: load i is row i, lane j its chunk j).  A load is a buffer load from
    // a scalar base at its first key row; the lane's byte offset from there
    // is fixed and computed once (the host picks this kernel only when it
    // stays below 2^31).  The last chunk of a range clamps keys past khi to
    // key khi-1 instead.
    int ld_r0[LOADS], ld_row[LOADS], ld_col[LOADS], ld_dst[LOADS];
    unsigned ld_koff[LOADS], ld_voff[LOADS];
#pragma unroll
    for (int it = 0; it < LOADS; ++it) {
        const int i = wave * LOADS + it;  // wave-uniform
        ld_r0[it] = i * 1024 / ROW_BYTES;
        const int x = (i * 64 + lane) * 16;  // LDS byte of this lane
        ld_row[it] = x / ROW_BYTES;
        ld_col[it] = ((x % ROW_BYTES) / 16 - rot_of(ld_row[it]) + CHUNKS) % CHUNKS;
        ld_dst[it] = i * 1024;
        ld_koff[it] = (unsigned)(((int64_t)(ld_row[it] - ld_r0[it]) * p.k_st + ld_col[it] * 8) * 2);
        ld_voff[it] = (unsigned)(((int64_t)(ld_row[it] - ld_r0[it]) * p.v_st + ld_col[it] * 8) * 2);
    }
    auto issue = [&](const uint16_t *base, int64_t st, const unsigned (&off)[LOADS], int k0, unsigned char *slot)
                     __attribute__((always_inline)) {
        if (k0 + KC <= khi) {  // wave-uniform
#pragma unroll
            for (int it = 0; it < LOADS; ++it)
                load_lds_buf(base + key_offset(min(k0 + ld_r0[it], khi - 1), st), off[it], slot + ld_dst[it]);
        } else {
#pragma unroll
            for (int it = 0; it < LOADS; ++it) {
                const int first = min(k0 + ld_r0[it], khi - 1);
                const int key = min(k0 + ld_row[it], khi - 1);
                const unsigned o = (unsigned)(((int64_t)(key - first) * st + ld_col[it] * 8) * 2);
                load_lds_buf(base + key_offset(first, st), o, slot + ld_dst[it]);
            }
        }
    };

    // V^T transposing-read coordinates (see attn_kernel.hpp): lane s of block
    // lg addresses key 4*lg + s/4 (+16) of a 32-key slice, columns 4*(s%4)..+3
    const int tr_row0 = 4 * lg + (lr >> 2);
    const int tr_col = 4 * (lr & 3);
    // one 32-key PV slice per chunk and at least four head-dim steps: the
    // step runs in the explicit order below (operands read ahead of their
    // MFMAs); rotated rows then need one address per head-dim step (K) and
    // per column block (V^T) -- a row's rotation depends on its index mod 8,
    // which 16-key block offsets keep
    constexpr bool ORDERED = KS == 1 && KSTEPS >= 4 && NB >= 4;
    constexpr int NKA = ORDERED ? KSTEPS : 1, NVA = ORDERED ? NB : 1;
    int k_at[NKA], v_at[NVA];
#pragma unroll
    for (int st = 0; st < NKA; ++st) k_at[st] = lr * ROW_BYTES + ((4 * st + lg + rot_of(lr)) % CHUNKS) * 16;
#pragma unroll
    for (int nb = 0; nb < NVA; ++nb) {
        const int c = 16 * nb + tr_col;
        v_at[nb] = tr_row0 * ROW_BYTES + (((c >> 3) + rot_of(tr_row0)) % CHUNKS) * 16 + (c & 7) * 2;
    }

    // ---- S^T of one staged chunk for every tile of this wave: KB blocks of 16
    // keys; each K operand read from LDS feeds the MFMAs of all the tiles.
    // With fewer than four (tile, key-block) accumulators (one tile per wave
    // at 32-key chunks, hd 256), each is split into NP partial sums over
    // alternate head-dim steps, added at the end in a fixed order.
    constexpr int NP = RT * KB >= 4 ? 1 : 4 / (RT * KB);
    auto qk = [&](const unsigned char *sK, f32x4 (&sc)[RT][KB]) __attribute__((always_inline)) {
        f32x4 part[NP][RT][KB];
#pragma unroll
        for (int q = 0; q < NP; ++q)
#pragma unroll
            for (int mt = 0; mt < RT; ++mt)
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) part[q][mt][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
        // head-dim steps outermost: the accumulators are independent chains,
        // and consecutive MFMAs go to different ones (a chain's next MFMA
        // waits for the previous one's result)
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
            bf16x8 kf[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const int r = 16 * kb + lr;
                const int slot = (4 * s + lg + rot_of(r)) % CHUNKS;
                kf[kb] = *reinterpret_cast<const bf16x8 *>(sK + r * ROW_BYTES + slot * 16);
            }
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int mt = 0; mt < RT; ++mt)
                    part[s % NP][mt][kb] = mfma_16x16x32(kf[kb], qf[mt][s], part[s % NP][mt][kb]);
        }
#pragma unroll
        for (int mt = 0; mt < RT; ++mt)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                sc[mt][kb] = part[0][mt][kb];
#pragma unroll
                for (int q = 1; q < NP; ++q) sc[mt][kb] = sc[mt][kb] + part[q][mt][kb];
            }
    };

    // ---- online softmax, first half: mask, maximum, rescale.  A chunk that
    // cuts through some row's visible range sets the scores of masked keys
    // to -inf (weight 0); chunks inside every tile's fully visible range skip
    // that.  The maximum is taken on raw scores; the reference point m moves
    // -- rescaling the accumulators -- only when some row of the wave
    // exceeds it by more than 2^8, so weights stay below 256 and most chunks
    // rescale nothing.
    auto prep = [&](int k0, f32x4 (&sc)[RT][KB]) __attribute__((always_inline)) {
        bool all_full = true;  // wave-uniform
#pragma unroll
        for (int mt = 0; mt < RT; ++mt) all_full = all_full && k0 >= full_lo[mt] && k0 + KC <= full_hi[mt];
        if (!all_full) {
#pragma unroll
            for (int mt = 0; mt < RT; ++mt)
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int key = k0 + 16 * kb + 4 * lg + j;
                        if (key < r_lo[mt] || key >= r_hi[mt]) sc[mt][kb][j] = -INFINITY;
                    }
        }
#pragma unroll
        for (int mt = 0; mt < RT; ++mt) {
            float mr = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int j = 0; j < 4; ++j) mr = fmaxf(mr, sc[mt][kb][j]);
            // a row's maximum exceeds the reference point by more than 2^8 iff
            // one of its four lanes' maxima does: the row maximum itself (a
            // reduction across the four lanes) is needed only when it moves
            if (__any(mr * c_scale > m[mt] + kRescaleLog2)) {
                const float m_new = fmaxf(m[mt], row4_max(mr) * c_scale);
                const float alpha = fast_exp2(m[mt] - ((m_new == -INFINITY) ? 0.f : m_new));
                l[mt] *= alpha;
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) acc[mt][nb] = acc[mt][nb] * alpha;
                accq[mt] = accq[mt] * alpha;
                m[mt] = m_new;
                neg_m[mt] = (m_new == -INFINITY) ? 0.f : -m_new;
            }
        }
    };

    // ---- second half: weights 2^(s c - m) (2^-inf = 0), their bf16 forms for
    // the PV product, the fp32 sum for lse and the bf16 sum (one MFMA against
    // the ones operand per 32 keys) for the normalisation
    auto weights = [&](const f32x4 (&sc)[RT][KB], bf16x8 (&pt)[RT][KS]) __attribute__((always_inline)) {
#pragma unroll
        for (int mt = 0; mt < RT; ++mt) {
            float psum = 0.f;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float pj = fast_exp2(fmaf(sc[mt][kb][j], c_scale, neg_m[mt]));
                    pt[mt][kb >> 1][(kb & 1) * 4 + j] = to_bf16(pj);
                    psum += pj;
                }
            l[mt] += psum;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) accq[mt] = mfma_16x16x32(ones, pt[mt][ks], accq[mt]);
        }
    };

    // ---- O^T += V^T . P^T; each V^T operand read from LDS feeds every tile
    auto pv = [&](const unsigned char *sV, const bf16x8 (&pt)[RT][KS]) __attribute__((always_inline)) {
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

    // ---- one 32-key PV slice per chunk (hd 128 and 256 at 32-key chunks):
    // the straight-line part of a step in an explicit order; the scheduling
    // barriers keep the compiler from regrouping (it would issue every LDS
    // read just before its use and wait for it there, and put every
    // exponential ahead of the first MFMA).
    //  * hd 128 (four head-dim steps, two tiles per wave on the long
    //    prefill): every K operand of chunk n+1 is read up front; chunk n's
    //    weights are computed one (or a few) per QK MFMA of chunk n+1, so
    //    the quarter-rate exponentials issue beside the MFMA pipe instead of
    //    ahead of it; chunk n's V^T operands are read during the QK product
    //    and its PV product follows (measured: long causal GQA prefill
    //    1.5-2% faster than weights-then-MFMAs).
    //  * hd 256: chunk n's weights, then chunk n+1's QK product interleaved
    //    with chunk n's PV product.  The QK product has only RT KB
    //    accumulators (2), each a chain over the head-dim steps, and a
    //    16x16x32 MFMA that depends on the one just issued waits for it: each
    //    QK step is therefore followed by the PV MFMAs of NB / KSTEPS column
    //    blocks, so the MFMA pipe always has independent work.  Each K
    //    operand is read D head-dim steps and each V^T operand DV steps
    //    before its MFMAs (all of them up front would not fit the registers).
    auto fused = [&](const unsigned char *sK, f32x4 (&sn)[RT][KB], const f32x4 (&sc)[RT][KB],
                     const unsigned char *sV) __attribute__((always_inline)) {
        static_assert(!ORDERED || (KS == 1 && KSTEPS >= 4 && NB % KSTEPS == 0), "one PV slice per chunk");
        constexpr int D = 4, R = D + 1;     // K read-ahead (head-dim steps), ring size
        constexpr int BPS = NB / KSTEPS;    // PV column blocks per QK step
        constexpr int DV = 2, RV = DV + 1;  // V^T read-ahead (steps), ring size
        auto read_k = [&](int st, bf16x8 (&kf)[KB]) __attribute__((always_inline)) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
                kf[kb] = *reinterpret_cast<const bf16x8 *>(sK + k_at[st] + 16 * kb * ROW_BYTES);
        };
        auto read_v = [&](int nb) __attribute__((always_inline)) {
            bf16x4 q2[2];
#pragma unroll
            for (int half = 0; half < 2; ++half)
                q2[half] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                    (__attribute__((address_space(3))) bf16x4 *)(sV + v_at[nb] + 16 * half * ROW_BYTES));
            return __builtin_shufflevector(q2[0], q2[1], 0, 1, 2, 3, 4, 5, 6, 7);
        };
        if constexpr (KSTEPS == 4) {
            constexpr int NQ = KSTEPS * KB * RT;  // QK MFMAs of the step
            constexpr int NE = RT * KB * 4;       // weights of the step, per lane
            static_assert(NE % KSTEPS == 0, "weight sums spread evenly over the PV groups");
            bf16x8 kf[KSTEPS][KB];
            bf16x8 vt[NB];
#pragma unroll
            for (int st = 0; st < KSTEPS; ++st) read_k(st, kf[st]);
            // raised wave priority over the step's MFMA work: of the two waves
            // on a SIMD (two workgroups per CU), the one with MFMAs to issue
            // is picked first (long causal GQA prefill 2-3% faster)
            __builtin_amdgcn_s_setprio(1);
            float pf[RT][KB * 4];  // chunk n's weights (fp32)
            bf16x8 pt[RT];         // and their bf16 forms, the PV B operand
            float psum[RT];
#pragma unroll
            for (int mt = 0; mt < RT; ++mt) {
                psum[mt] = 0.f;
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) sn[mt][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
            // QK MFMA qi of chunk n+1, then weights qi NE/NQ .. (qi+1) NE/NQ - 1
            // of chunk n (weight e: tile e / 4KB, block (e / 4) % KB, element e % 4)
#pragma unroll
            for (int st = 0; st < KSTEPS; ++st) {
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int mt = 0; mt < RT; ++mt) {
                        const int qi = (st * KB + kb) * RT + mt;
                        __builtin_amdgcn_sched_barrier(0);
                        sn[mt][kb] = mfma_16x16x32(kf[st][kb], qf[mt][st], sn[mt][kb]);
#pragma unroll
                        for (int e = qi * NE / NQ; e < (qi + 1) * NE / NQ; ++e) {
                            const int et = e / (KB * 4), ek = (e / 4) % KB, ej = e % 4;
                            pf[et][ek * 4 + ej] = fast_exp2(fmaf(sc[et][ek][ej], c_scale, neg_m[et]));
                            pt[et][ek * 4 + ej] = to_bf16(pf[et][ek * 4 + ej]);
                        }
                    }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int u = 0; u < BPS; ++u) vt[st * BPS + u] = read_v(st * BPS + u);
            }
            // chunk n's PV product (and the bf16 weight sum), the fp32 weight
            // sums in between, in the same order as a plain loop over e
#pragma unroll
            for (int st = 0; st < KSTEPS; ++st) {
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int u = 0; u < BPS; ++u)
#pragma unroll
                    for (int mt = 0; mt < RT; ++mt)
                        acc[mt][st * BPS + u] = mfma_16x16x32(vt[st * BPS + u], pt[mt], acc[mt][st * BPS + u]);
                if (st == 0) {
#pragma unroll
                    for (int mt = 0; mt < RT; ++mt) accq[mt] = mfma_16x16x32(ones, pt[mt], accq[mt]);
                }
#pragma unroll
                for (int e = st * NE / KSTEPS; e < (st + 1) * NE / KSTEPS; ++e)
                    psum[e / (KB * 4)] += pf[e / (KB * 4)][e % (KB * 4)];
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int mt = 0; mt < RT; ++mt) l[mt] += psum[mt];
            __builtin_amdgcn_s_setprio(0);
        } else {
            bf16x8 kf[R][KB];
            bf16x8 vt[RV][BPS];
#pragma unroll
            for (int st = 0; st < D; ++st) read_k(st, kf[st]);
#pragma unroll
            for (int sv = 0; sv < DV; ++sv)
#pragma unroll
                for (int u = 0; u < BPS; ++u) vt[sv][u] = read_v(sv * BPS + u);
            __builtin_amdgcn_s_setprio(1);  // as above
            // chunk n's weights 2^(s c - m), their bf16 forms and sums
            bf16x8 pt[RT];
#pragma unroll
            for (int mt = 0; mt < RT; ++mt) {
                float psum = 0.f;
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float pj = fast_exp2(fmaf(sc[mt][kb][j], c_scale, neg_m[mt]));
                        pt[mt][kb * 4 + j] = to_bf16(pj);
                        psum += pj;
                    }
                l[mt] += psum;
            }
#pragma unroll
            for (int mt = 0; mt < RT; ++mt)
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) sn[mt][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < KSTEPS; ++st) {
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int mt = 0; mt < RT; ++mt) sn[mt][kb] = mfma_16x16x32(kf[st % R][kb], qf[mt][st], sn[mt][kb]);
#pragma unroll
                for (int u = 0; u < BPS; ++u)
#pragma unroll
                    for (int mt = 0; mt < RT; ++mt)
                        acc[mt][st * BPS + u] = mfma_16x16x32(vt[st % RV][u], pt[mt], acc[mt][st * BPS + u]);
                if (st == 0) {
#pragma unroll
                    for (int mt = 0; mt < RT; ++mt) accq[mt] = mfma_16x16x32(ones, pt[mt], accq[mt]);
                }
                if (st + D < KSTEPS) read_k(st + D, kf[(st + D) % R]);
                if (st + DV < KSTEPS) {
#pragma unroll
                    for (int u = 0; u < BPS; ++u) vt[(st + DV) % RV][u] = read_v((st + DV) * BPS + u);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_setprio(0);
        }
    };

    // ---- the pipeline.  Step n starts with chunk n+1's K and chunk n's V on
    // chip and chunk n's scores in registers; it requests chunk n+2's K and
    // chunk n+1's V into the slots step n-1 finished with, then computes
    // chunk n+1's scores alongside chunk n's weights and PV product.  One
    // barrier per step: every wave's loads of the previous step have landed
    // and every wave is done reading the slots about to be refilled.  After
    // the last chunk the QK product reads a stale K slot; those scores are
    // never used.  (Loads issued two steps ahead, from a ring of three slots
    // per operand at hd 128, measured 1-2% slower on the long prefill.)
    const int nchunks = khi > klo ? (khi - klo + KC - 1) / KC : 0;  // wave-uniform
    f32x4 sc[RT][KB];
    if (nchunks > 0) {
        // chunk 0's scores need only Q and chunk 0's K (the oldest loads):
        // chunk 0's V and chunk 1's K stay in flight during that product
        issue(kbase, p.k_st, ld_koff, klo, sK0);
        issue(vbase, p.v_st, ld_voff, klo, sV0);
        if (nchunks > 1) issue(kbase, p.k_st, ld_koff, klo + KC, sK1);
        __builtin_amdgcn_sched_barrier(0);  // every prologue load issued before Q is used
        if (nchunks > 1) {
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * LOADS));
        } else {
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(LOADS));
        }
        lds_barrier();
        finish_q();
        qk(sK0, sc);
    }
    auto step = [&](int n, const unsigned char *sKnext, const unsigned char *sVcur, unsigned char *sKfill,
                    unsigned char *sVfill) __attribute__((always_inline)) {
        const int k0 = klo + n * KC;
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        lds_barrier();
        if (n + 2 < nchunks) issue(kbase, p.k_st, ld_koff, k0 + 2 * KC, sKfill);
        if (n + 1 < nchunks) issue(vbase, p.v_st, ld_voff, k0 + KC, sVfill);
        prep(k0, sc);
        f32x4 sn[RT][KB];
        if constexpr (ORDERED) {
            fused(sKnext, sn, sc, sVcur);
        } else {
            qk(sKnext, sn);
            bf16x8 pt[RT][KS];
            weights(sc, pt);
            pv(sVcur, pt);
        }
#pragma unroll
        for (int mt = 0; mt < RT; ++mt)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) sc[mt][kb] = sn[mt][kb];
    };
    // two steps per iteration (the slots alternate); no LDS-direct load
    // crosses the back-edge, which the compiler's wait placement would answer
    // with a wait for all loads before the iteration's first LDS read
    for (int n = 0; n < nchunks; n += 2) {
        step(n, sK1, sV0, sK0, sV1);
        if (n + 1 < nchunks) step(n + 1, sK0, sV1, sK1, sV0);
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
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
