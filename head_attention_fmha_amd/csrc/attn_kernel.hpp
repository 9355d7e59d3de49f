// attn_kernel.hpp -- the fused attention kernel for gfx950.
//
// One workgroup (NW = 4 or 8 waves) computes MT adjacent 16-row tiles of one
// (batch, kv head) over one key range.  A row is one (query position t, query head h)
// that reads this KV head, numbered r = t * group + (h - kv*group): the
// GQA/MQA query heads sharing K/V are stacked into the same MFMA tile, and
// the rows of a tile have the same or adjacent positions (tight mask ranges).
//
// The NW waves form NK key groups x NH head-dimension parts (HDP = HD/NH
// columns each, 64 or 128); every wave covers all MT tiles:
//   * key group g takes keys [c + 32g, c + 32g + 32) of every chunk of
//     32*NK keys and keeps its own online-softmax state; the NK groups are
//     merged once at the end, in a fixed order;
//   * head part j loads only columns [j*HDP, (j+1)*HDP) of K and V, so every
//     byte of K/V is fetched once per workgroup, and each loaded K operand
//     and each gathered V operand feeds the MFMAs of all MT tiles.  The NH
//     partial QK scores of a slice are summed through LDS in a fixed order,
//     so the NH waves of a key group hold bit-identical scores and
//     probabilities.
//
// Both products are taken transposed, keys in the MFMA M dimension
// (v_mfma_f32_16x16x32_bf16; lane l = lr + 16*lg):
//   S^T (keys x rows) = K . Q^T      lane holds S^T[4*lg + j][lr]
//   O^T (hd x rows)  += V^T . P^T    lane holds O^T[4*lg + j][lr]
// so all softmax state of row lr lives in lanes lr, lr+16, lr+32, lr+48:
// the running max and sum reduce over those four lanes in two lane-swap
// steps (v_permlane16_swap, v_permlane32_swap), the rescale factor is a
// per-lane scalar, and the probabilities leave the QK result registers in
// exactly the B-operand layout of the PV product (the 32-key reduction
// index is permuted identically in both PV operands).
//
// Data movement per 32-key slice and wave:
//   * K: HBM -> QK A-operand registers (lane lr + 16*lg loads 16 bytes of
//     key lr at column offset 32*s + 8*lg) -- no LDS round trip;
//   * V: HBM -> a wave-private LDS slice, a run of lanes covering one whole
//     key-row part (coalesced): directly with global_load_lds_dwordx4 when
//     a workgroup has one slice, through registers when slices are
//     pipelined (the compiler does not count LDS-direct loads, so it would
//     wait for all of them).  The 16-byte chunks of LDS key row k are
//     rotated by 2*(k mod 8) positions, so one transposing read of 16 keys
//     spreads over the banks;
//   * the PV operand V^T comes from ds_read_b64_tr_b16, gfx950's
//     transposing LDS read (see pv below).
//
// Softmax: online (running max m, running sum l, rescale of the partial
// output by exp(m_old - m_new) when a slice raises the max), as in the
// multi-tile kernel of the e4ee9fdc commit log of the pages, with one
// division by the sum in the epilogue.  Scores are kept in base 2
// (x = q.k * scale * log2 e), so exp is one v_exp_f32.  The output is
// normalised by the sum of the same bf16-rounded weights the PV product
// consumes (an exact convex combination of V rows); lse uses the fp32 sum.
#pragma once

#include "device_common.hpp"
#include "mx_quant.hpp"
#include "params.hpp"

namespace fmha {

template <int HD, int NW, int NK, int NH, int MT>
struct AttnShape {
    static_assert(NK * NH == NW && (NW == 4 || NW == 8), "four or eight waves per workgroup");
    static constexpr int HDP = HD / NH;               // head-dim columns per wave
    static constexpr int KSTEPS = HDP / 32;           // QK MFMA steps
    static constexpr int NB = HDP / 16;               // 16-column blocks of O^T
    static constexpr int CHUNKS = HDP / 8;            // 16-byte chunks per key-row part
    static constexpr int ROW_BYTES = HDP * 2;         // LDS key-row part
    static constexpr int KEYS_PER_LOAD = 64 / CHUNKS;  // keys per wave-wide 16-byte load
    static constexpr int VLOADS = 32 / KEYS_PER_LOAD;
    static constexpr int SLOTS = NB * 4 + 3;          // merge record per lane and tile: m, l, lq, O^T
    static constexpr int M_BYTES = (NK - 1) * NH * MT * SLOTS * 64 * 4;
    static constexpr int S_FLOATS = MT * NW * 8 * 64;  // one buffer of partial scores
    static constexpr int S_BUF = NH > 1 ? S_FLOATS * 4 : 0;
    static_assert(HDP == 64 || HDP == 128, "head-dim part of 64 or 128 columns");
};

// ONE: every workgroup's key range fits one chunk of 32*NK keys (split-KV
// decode with 128-key partitions, short caches).  The chunk loop collapses to
// one pass, no state is carried in from an earlier slice, and the output
// accumulator is born from the first PV product -- so nothing but Q is live
// while the loads are in flight, which buys a fifth wave per SIMD.
// MT: 16-row tiles per workgroup.  Two when a workgroup streams several
// slices for more than 16 rows: each K/V byte brought on chip then serves
// twice the rows.
// STREAM (one-slice work with a single row block per KV head): no other
// workgroup reads this workgroup's V, so it is fetched with the non-temporal
// hint.  Split partials are always stored with it: the merge reads them in a
// later launch.
// NW = 8: for grids too small to fill the chip twice, twice the key groups
// per workgroup halve the slices each wave walks through in sequence.
constexpr int attn_min_waves(int nw, int nh, bool one) { return one ? (nw == 4 && nh == 1 ? 5 : 4) : 2; }

template <int HD, int NW, int NK, int NH, int MT, bool SPLIT, bool ONE, bool STREAM>
__global__ __launch_bounds__(64 * NW, attn_min_waves(NW, NH, ONE)) void attn_kernel(const FwdParams p) {
    using S = AttnShape<HD, NW, NK, NH, MT>;
    static_assert(MT == 1 || !ONE, "one-slice work uses single tiles");
    static_assert(ONE || !STREAM, "only one-slice work streams");
    constexpr int HDP = S::HDP, KSTEPS = S::KSTEPS, NB = S::NB, CHUNKS = S::CHUNKS;
    constexpr int ROW_BYTES = S::ROW_BYTES, KEYS_PER_LOAD = S::KEYS_PER_LOAD, VLOADS = S::VLOADS;
    constexpr int SLOTS = S::SLOTS;
    // one V slice per wave (the final key-group merge reuses that space);
    // partial-score buffers alternate by slice parity (one suffices for ONE)
    constexpr int V_BYTES = NW * 32 * ROW_BYTES;
    constexpr int VM_BYTES = V_BYTES > S::M_BYTES ? V_BYTES : S::M_BYTES;
    __shared__ __attribute__((aligned(16))) unsigned char smem[VM_BYTES + (ONE ? 1 : 2) * S::S_BUF];

    fetch_launch_params(p);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int kg = wave / NH;  // key group
    const int hp = wave % NH;  // head-dim part
    const int lr = lane & 15;
    const int lg = lane >> 4;

    // ---- work unit: row blocks fastest (they share K/V through L2), then
    // partitions (consecutive key ranges of one KV head; their partial outputs
    // are adjacent in memory), then KV heads and batches.  With several row
    // blocks the units are regrouped so that one XCD (one L2) runs consecutive
    // ones: blocks are dealt to the 8 XCDs round-robin.  Row blocks run last
    // first: under a causal mask the last rows see the most keys, and starting
    // the longest units first keeps them out of the tail of the launch -------
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

    const int row0 = rb * 16 * MT;
    const int row_last = min(row0 + 16 * MT, p.rows) - 1;
    const int pos_lo = s_k - p.T + row0 / p.group;
    const int pos_hi = s_k - p.T + row_last / p.group;
    // key range: the partition, cut to the union of the block rows' masks
    int klo = part * p.split_len;
    int khi = min(klo + p.split_len, s_k);
    if (p.causal) khi = min(khi, pos_hi + 1);
    if (p.window > 0) klo = max(klo, pos_lo - p.window + 1);

    // ---- this lane's row in each tile ---------------------------------------------
    bool row_ok[MT];
    int t_of[MT], h_of[MT], r_lo[MT], r_hi[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int row = row0 + 16 * mt + lr;
        row_ok[mt] = row < p.rows;
        t_of[mt] = row_ok[mt] ? row / p.group : 0;
        h_of[mt] = kvh * p.group + (row_ok[mt] ? row % p.group : 0);
        const int pos = s_k - p.T + t_of[mt];
        r_hi[mt] = p.causal ? min(khi, pos + 1) : khi;
        r_lo[mt] = p.window > 0 ? max(klo, pos - p.window + 1) : klo;
        if (!row_ok[mt]) r_hi[mt] = r_lo[mt];  // no visible key: the row stays at -inf
    }
    // keys visible to EVERY valid row of tile mt (wave-uniform): slices inside
    // need no mask (rows past the end hold Q = 0 and are never stored)
    int full_lo[MT], full_hi[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int first = row0 + 16 * mt;
        const int last = min(first + 15, row_last);
        if (first > row_last) {
            full_lo[mt] = khi;
            full_hi[mt] = klo;
        } else {
            full_hi[mt] = p.causal ? min(khi, s_k - p.T + first / p.group + 1) : khi;
            full_lo[mt] = p.window > 0 ? max(klo, s_k - p.T + last / p.group - p.window + 1) : klo;
        }
    }

    // LAZY (two-tile workgroups, where the softmax's vector work matters more
    // than one slice's latency): the running maximum is kept on raw scores,
    // c = |scale| log2 e is folded into the exponent's fma (a negative scale
    // flips the sign of Q instead, exact in bf16), the reference maximum
    // moves only when exceeded by more than 2^8, and the bf16 weight sums
    // come from an MFMA.  Single-tile workgroups are latency-bound and keep
    // the eager form, which has the shorter dependency chain per slice.
    constexpr bool LAZY = !ONE && MT == 2;
    const float c_scale = fabsf(p.scale_log2);
    const unsigned q_flip = (LAZY && p.scale_log2 < 0.f) ? 0x80008000u : 0u;
    const int col0 = hp * HDP;  // first head-dim column of this wave
    // Q^T B operand: Q[row lr][col0 + 32*s + 8*lg + 0..7], loaded
    // unconditionally: a row past the end reads row 0 of the group (valid
    // memory; its lanes' scores, softmax state and output stay in its own
    // MFMA column and are never stored).  A load under a lane condition, or
    // one used right away, was waited for on the spot, a full memory round
    // trip before the first K/V load went out: only the lazy form's sign
    // flip touches Q, once the first slice's loads are issued (finish_q)
    u32x4 qraw[MT][KSTEPS];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const uint16_t *qp = p.q + (int64_t)b * p.q_sb + (int64_t)t_of[mt] * p.q_st + (int64_t)h_of[mt] * p.q_sh +
                             col0 + 8 * lg;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) qraw[mt][s] = *reinterpret_cast<const u32x4 *>(qp + 32 * s);
    }
    bf16x8 qf[MT][KSTEPS];
    auto finish_q = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int s = 0; s < KSTEPS; ++s)
                qf[mt][s] = __builtin_bit_cast(bf16x8, LAZY ? qraw[mt][s] ^ q_flip : qraw[mt][s]);
    };

    f32x4 acc[MT][NB];
    f32x4 accq[MT];  // LAZY: the bf16 weight sum of row lr, in every element (-> O)
    float m[MT], l[MT], lq[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[mt][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
        accq[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        m[mt] = -INFINITY;  // running max (base 2), equal in the 4 lanes of a row
        l[mt] = 0.f;        // this lane's share of the fp32 sum of weights (-> lse)
        lq[mt] = 0.f;       // eager form: the same over the bf16-rounded weights (-> O)
    }
    // A operand of ones: one MFMA per slice sums the bf16 weights the PV
    // product consumes, already complete in every lane of the row
    bf16x8 ones;
#pragma unroll
    for (int j = 0; j < 8; ++j) ones[j] = (__bf16)1.0f;

    const uint16_t *kbase = p.k + (int64_t)b * p.k_sb + (int64_t)kvh * p.k_sh + col0;
    const uint16_t *vbase = p.v + (int64_t)b * p.v_sb + (int64_t)kvh * p.v_sh + col0;
    unsigned char *sVw = smem + wave * 32 * ROW_BYTES;  // this wave's V slice
    float *sS = reinterpret_cast<float *>(smem + VM_BYTES);
    const int v_row_in_load = lane / CHUNKS;
    const int v_slot = lane % CHUNKS;

    // ---- K part of a slice: HBM -> QK A-operand registers (keys past khi read
    // key khi-1; their scores are masked) ---------------------------------------
    auto load_k = [&](int k0, bf16x8 (&kf)[2][KSTEPS]) __attribute__((always_inline)) {
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            const int key = min(k0 + 16 * blk + lr, khi - 1);
            const uint16_t *kp = kbase + key_offset(key, p.k_st) + 8 * lg;
#pragma unroll
            for (int s = 0; s < KSTEPS; ++s) kf[blk][s] = *reinterpret_cast<const bf16x8 *>(kp + 32 * s);
        }
    };
    // LDS row r of the slice holds its 16-byte chunk c in slot (c + rot(r)) % CHUNKS:
    // the 16 keys of one transposed read then cover the LDS banks evenly
    auto rot_of = [](int r) __attribute__((always_inline)) { return (2 * (r & 7)) % CHUNKS; };

    // ---- QK of every tile and (NH > 1) the fixed-order sum of the head-part
    // scores ------------------------------------------------------------------------
    auto scores = [&](bool active, int iter, const bf16x8 (&kf)[2][KSTEPS], f32x4 (&s0)[MT], f32x4 (&s1)[MT])
                      __attribute__((always_inline)) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            s0[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
            s1[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        // multi-slice work always holds loaded K (keys clamp into the range),
        // so its products need no branch; an inactive key group's scores are
        // never used
        if (!ONE || active) {
#pragma unroll
            for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    s0[mt] = mfma_16x16x32(kf[0][s], qf[mt][s], s0[mt]);
                    s1[mt] = mfma_16x16x32(kf[1][s], qf[mt][s], s1[mt]);
                }
        }
        if constexpr (NH > 1) {
            float *buf = sS + (ONE ? 0 : (iter & 1) * S::S_FLOATS);
            if (active) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        buf[((mt * NW + wave) * 8 + j) * 64 + lane] = s0[mt][j];
                        buf[((mt * NW + wave) * 8 + 4 + j) * 64 + lane] = s1[mt][j];
                    }
            }
            // LDS-only barrier: a full __syncthreads() would also wait for the
            // next slice's loads already in flight
            lds_barrier();
            if (active) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        float a = 0.f, c2 = 0.f;
#pragma unroll
                        for (int q = 0; q < NH; ++q) {
                            a += buf[((mt * NW + kg * NH + q) * 8 + j) * 64 + lane];
                            c2 += buf[((mt * NW + kg * NH + q) * 8 + 4 + j) * 64 + lane];
                        }
                        s0[mt][j] = a;
                        s1[mt][j] = c2;
                    }
            }
        }
    };

    // ---- mask + online softmax of tile mt: returns the rescale factor, fills P^T
    auto softmax = [&](int mt, int k0, const f32x4 &s0, const f32x4 &s1, bf16x8 &pt) __attribute__((always_inline))
        -> float {
        float x[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int ka = k0 + 4 * lg + j;
            const int kb = ka + 16;
            x[j] = (ka >= r_lo[mt] && ka < r_hi[mt]) ? s0[j] * p.scale_log2 : -INFINITY;
            x[4 + j] = (kb >= r_lo[mt] && kb < r_hi[mt]) ? s1[j] * p.scale_log2 : -INFINITY;
        }
        float mx = x[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) mx = fmaxf(mx, x[j]);
        mx = row4_max(mx);
        const float m_new = ONE ? mx : fmaxf(m[mt], mx);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = ONE ? 0.f : fast_exp2(m[mt] - m_use);
        float psum = 0.f, qsum = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float pj = fast_exp2(x[j] - m_use);
            const __bf16 pb = to_bf16(pj);
            pt[j] = pb;
            psum += pj;
            qsum += (float)pb;
        }
        l[mt] = ONE ? psum : l[mt] * alpha + psum;
        lq[mt] = ONE ? qsum : lq[mt] * alpha + qsum;
        m[mt] = m_new;
        return alpha;
    };

    // ---- LAZY: online softmax of tile mt over a slice.  The
    // maximum is taken on raw scores (masked keys excluded only in slices that
    // cut through some row's range); the reference point m moves -- rescaling
    // the accumulators -- only when some row of the wave exceeds it by more
    // than 2^8, so weights stay below 256 and most slices rescale nothing.
    auto softmax_lazy = [&](int mt, int k0, const f32x4 &s0, const f32x4 &s1, bf16x8 &pt) __attribute__((always_inline)) {
        const bool full = k0 >= full_lo[mt] && k0 + 32 <= full_hi[mt];  // wave-uniform
        float sv[8];
        bool vis[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            sv[j] = s0[j];
            sv[4 + j] = s1[j];
        }
        float mr = -INFINITY;
        if (full) {
#pragma unroll
            for (int j = 0; j < 8; ++j) mr = fmaxf(mr, sv[j]);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int key = k0 + 4 * lg + (j & 3) + (j >> 2) * 16;
                vis[j] = key >= r_lo[mt] && key < r_hi[mt];
                mr = fmaxf(mr, vis[j] ? sv[j] : -INFINITY);
            }
        }
        // a row's maximum exceeds the reference point by more than 2^8 iff one
        // of its four lanes' maxima does: the row maximum itself (a reduction
        // across the four lanes) is needed only when the reference moves
        if (__any(mr * c_scale > m[mt] + kRescaleLog2)) {
            const float mx = row4_max(mr) * c_scale;  // NaN (ignored by fmaxf) for a fully masked row when c = 0
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
        for (int j = 0; j < 8; ++j) {
            float xj = fmaf(sv[j], c_scale, neg_m);
            if (!full) xj = vis[j] ? xj : -INFINITY;
            const float pj = fast_exp2(xj);
            pt[j] = to_bf16(pj);
            psum += pj;
        }
        l[mt] += psum;
        accq[mt] = mfma_16x16x32(ones, pt, accq[mt]);
    };

    // ---- O^T = alpha O^T + V^T . P^T for every tile, from the wave's LDS slice.
    // Item j of lane (lr, lg) is key 4*lg + j (j < 4) or 16 + 4*lg + (j - 4),
    // column 16*nb + lr.  Each half comes from one transposing read
    // (ds_read_b64_tr_b16: within a 16-lane block, lane i item j receives
    // element i%4 of the 8 bytes addressed by lane 4j + i/4), so lane s of
    // block lg addresses key 4*lg + s/4 (+16), columns 16*nb + 4*(s%4) .. +3.
    int tr_row[2], tr_col[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        tr_row[half] = 16 * half + 4 * lg + (lr >> 2);
        tr_col[half] = 4 * (lr & 3);
    }
    auto pv = [&](const float (&alpha)[MT], const bf16x8 (&pt)[MT]) __attribute__((always_inline)) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            bf16x4 q[2];
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int r = tr_row[half];
                const int c = 16 * nb + tr_col[half];
                const int off = r * ROW_BYTES + (((c >> 3) + rot_of(r)) % CHUNKS) * 16 + (c & 7) * 2;
                q[half] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4 *)(sVw + off));
            }
            // whole-vector concatenation (element-wise inserts are mis-lowered)
            const bf16x8 vt = __builtin_shufflevector(q[0], q[1], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                if constexpr (ONE) {
                    acc[mt][nb] = mfma_16x16x32(vt, pt[mt], f32x4{0.f, 0.f, 0.f, 0.f});
                } else if constexpr (LAZY) {  // rescaled (if at all) in softmax_lazy
                    acc[mt][nb] = mfma_16x16x32(vt, pt[mt], acc[mt][nb]);
                } else {
                    acc[mt][nb] = acc[mt][nb] * alpha[mt];
                    acc[mt][nb] = mfma_16x16x32(vt, pt[mt], acc[mt][nb]);
                }
            }
        }
    };

    const int chunk_keys = 32 * NK;
    const int nslices = khi > klo ? (khi - klo + chunk_keys - 1) / chunk_keys : 0;  // uniform
    if constexpr (ONE) {
        // one slice: V goes HBM -> LDS directly (global_load_lds, no registers in flight)
        if (nslices > 0) {
            const int k0 = klo + 32 * kg;
            const bool active = k0 < khi;
            bf16x8 kf[2][KSTEPS];
            if (active) {
#pragma unroll
                for (int it = 0; it < VLOADS; ++it) {
                    const int r = it * KEYS_PER_LOAD + v_row_in_load;
                    const int chunk = (v_slot - rot_of(r) + CHUNKS) % CHUNKS;
                    const int key = min(k0 + r, khi - 1);
                    load_lds_16<STREAM>(vbase + key_offset(key, p.v_st) + chunk * 8, sVw + it * 64 * 16);
                }
                load_k(k0, kf);
                __builtin_amdgcn_sched_barrier(0);  // every load issued before the first wait
            }
            finish_q();
            f32x4 s0[MT], s1[MT];
            scores(active, 0, kf, s0, s1);
            if (active) {
                bf16x8 pt[MT];
                float alpha[MT];
                alpha[0] = softmax(0, k0, s0[0], s1[0], pt[0]);
                __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // V has landed in LDS
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                pv(alpha, pt);
            }
        }
    } else {
        // pipelined: K and V are loaded into registers ahead of their slice's
        // math; V reaches LDS (rotated) just before its PV product.  Plain
        // register loads keep the compiler's wait counting exact, so the waits
        // for one slice leave later slices' loads in flight.
        auto load_v = [&](int k0, u32x4 (&vr)[VLOADS]) __attribute__((always_inline)) {
#pragma unroll
            for (int it = 0; it < VLOADS; ++it) {
                const int key = min(k0 + it * KEYS_PER_LOAD + v_row_in_load, khi - 1);
                vr[it] = *reinterpret_cast<const u32x4 *>(vbase + key_offset(key, p.v_st) + v_slot * 8);
            }
        };
        // after_qk / after_v: run once this slice's K registers / V registers
        // are consumed (the caller refills them there)
        auto step = [&](int n, const bf16x8 (&kf)[2][KSTEPS], const u32x4 (&vr)[VLOADS], auto after_qk,
                        auto after_v) __attribute__((always_inline)) {
            const int k0 = klo + n * chunk_keys + 32 * kg;
            const bool active = k0 < khi;
            f32x4 s0[MT], s1[MT];
            scores(active, n, kf, s0, s1);
            after_qk();
            if (!active) {
                after_v();
                return;
            }
            bf16x8 pt[MT];
            float alpha[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                if constexpr (LAZY) {
                    softmax_lazy(mt, k0, s0[mt], s1[mt], pt[mt]);
                    alpha[mt] = 1.f;
                } else {
                    alpha[mt] = softmax(mt, k0, s0[mt], s1[mt], pt[mt]);
                }
            }
            // the previous slice's V^T reads are done before its LDS slice is reused
            __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
#pragma unroll
            for (int it = 0; it < VLOADS; ++it) {
                const int r = it * KEYS_PER_LOAD + v_row_in_load;
                const int slot = (v_slot + rot_of(r)) % CHUNKS;
                *reinterpret_cast<u32x4 *>(sVw + r * ROW_BYTES + slot * 16) = vr[it];
            }
            after_v();
            __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
            pv(alpha, pt);
        };
        auto nothing = [] {};
        if constexpr (MT == 1 && NW == 4) {
            // two slices per iteration, both loaded up front: the second
            // slice's loads are in flight while the first is computed.  The
            // loads are unconditional (key indices clamp to khi-1, so a slice
            // past the range reads valid memory and is then skipped) and no
            // load target crosses the loop back-edge: both keep the compiler's
            // wait counts exact, so it waits for the first slice only.
            for (int n = 0; n < nslices; n += 2) {
                bf16x8 kfA[2][KSTEPS], kfB[2][KSTEPS];
                u32x4 vrA[VLOADS], vrB[VLOADS];
                load_k(klo + n * chunk_keys + 32 * kg, kfA);
                load_v(klo + n * chunk_keys + 32 * kg, vrA);
                load_k(klo + (n + 1) * chunk_keys + 32 * kg, kfB);
                load_v(klo + (n + 1) * chunk_keys + 32 * kg, vrB);
                __builtin_amdgcn_sched_barrier(0);  // keep all 2 x (K + V) loads ahead of the math
                if (n == 0) finish_q();
                step(n, kfA, vrA, nothing, nothing);
                if (n + 1 < nslices) step(n + 1, kfB, vrB, nothing, nothing);
            }
        } else {
            // two tiles already double the math per loaded slice; one slice per
            // iteration keeps the registers within two waves per SIMD.  The
            // next slice's K is requested as soon as this slice's QK has
            // consumed the K registers, so its latency overlaps this slice's
            // softmax and PV product; V is requested at the top of its own
            // slice and waited for only before its copy to LDS, after the
            // softmax.  A load past the range clamps its keys to khi - 1
            // (valid memory; the last prefetch is never used)
            bf16x8 kf[2][KSTEPS];
            if (nslices > 0) load_k(klo + 32 * kg, kf);  // khi > klo >= 0: clamped keys are valid
            __builtin_amdgcn_sched_barrier(0);
            finish_q();
            for (int n = 0; n < nslices; ++n) {
                const int k_cur = klo + n * chunk_keys + 32 * kg;
                u32x4 vr[VLOADS];
                load_v(k_cur, vr);
                step(
                    n, kf, vr, [&]() __attribute__((always_inline)) { load_k(k_cur + chunk_keys, kf); }, nothing);
            }
        }
    }

    // full row sums over the four lanes of a row
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        l[mt] = row4_sum(l[mt]);
        if constexpr (LAZY) {
            lq[mt] = accq[mt][0];
        } else {
            lq[mt] = row4_sum(lq[mt]);
        }
    }

    // ---- merge the NK key groups of each head part and tile (fixed order) ----------
    if constexpr (NK > 1) {
        __syncthreads();  // all V slices and score buffers are consumed
        float *red = reinterpret_cast<float *>(smem);
        auto slot_of = [&](int g, int mt) __attribute__((always_inline)) {
            return red + ((((g - 1) * NH + hp) * MT + mt) * SLOTS) * 64 + lane;
        };
        if (kg != 0) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                float *mine = slot_of(kg, mt);
                mine[0] = m[mt];
                mine[64] = l[mt];
                mine[128] = lq[mt];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int j = 0; j < 4; ++j) mine[(3 + nb * 4 + j) * 64] = acc[mt][nb][j];
            }
        }
        __syncthreads();
        if (kg != 0) return;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            float M = m[mt];
#pragma unroll
            for (int g = 1; g < NK; ++g) M = fmaxf(M, slot_of(g, mt)[0]);
            const float M_use = (M == -INFINITY) ? 0.f : M;
            const float w0 = fast_exp2(m[mt] - M_use);
            l[mt] *= w0;
            lq[mt] *= w0;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) acc[mt][nb] = acc[mt][nb] * w0;
#pragma unroll
            for (int g = 1; g < NK; ++g) {
                const float *src = slot_of(g, mt);
                const float wgt = fast_exp2(src[0] - M_use);
                l[mt] += wgt * src[64];
                lq[mt] += wgt * src[128];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[mt][nb][j] += wgt * src[(3 + nb * 4 + j) * 64];
            }
            m[mt] = M;
        }
    }

    // ---- epilogue: one division; lse = (m + log2 l) ln 2 -------------------------
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        if (!row_ok[mt]) continue;
        const int t = t_of[mt], h = h_of[mt];
        const float inv = lq[mt] > 0.f ? 1.f / lq[mt] : 0.f;
        const float lse_val = l[mt] > 0.f ? (m[mt] + __log2f(l[mt])) * kLn2 : -INFINITY;
        if constexpr (SPLIT) {
            const int64_t r = (((int64_t)b * p.n_h + h) * p.T + t) * p.n_split_total + p.part_offset + part;
            float *op = p.o_part + r * HD + col0 + 4 * lg;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                __builtin_nontemporal_store(acc[mt][nb] * inv, reinterpret_cast<f32x4 *>(op + 16 * nb));
            if (hp == 0 && lg == 0) p.lse_part[r] = lse_val;
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
                mx_store_block_4lanes(v, p.out_format, crow, srow, col0 + 16 * nb, lg);
            }
            if (hp == 0 && lg == 0 && p.lse != nullptr) p.lse[((int64_t)b * p.n_h + h) * p.T + t] = lse_val;
        } else {
            uint16_t *op = p.o + (int64_t)b * p.o_sb + (int64_t)t * p.o_st + (int64_t)h * p.o_sh + col0 + 4 * lg;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                uint2 packed;
                packed.x = (uint32_t)bf16_bits(acc[mt][nb][0] * inv) |
                           ((uint32_t)bf16_bits(acc[mt][nb][1] * inv) << 16);
                packed.y = (uint32_t)bf16_bits(acc[mt][nb][2] * inv) |
                           ((uint32_t)bf16_bits(acc[mt][nb][3] * inv) << 16);
                *reinterpret_cast<uint2 *>(op + 16 * nb) = packed;
            }
            if (hp == 0 && lg == 0 && p.lse != nullptr) p.lse[((int64_t)b * p.n_h + h) * p.T + t] = lse_val;
        }
    }
}

}  // namespace fmha
