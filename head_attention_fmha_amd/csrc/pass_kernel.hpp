// pass_kernel.hpp -- attention at hd 256 and 512 on gfx950 for few-unit
// grids: a workgroup computes one 16-row tile (one KV head, one key range)
// in one pass over at most 128 keys with every load it needs in flight
// together (pass_kernel, launched at hd 256; one pass at hd 512 runs the
// column-split kernel of cols_kernel.hpp, as do one-pass calls at hd 256
// whose row blocks share K/V), or in several such passes
// (pass_loop_kernel, below, where cols_kernel is not chosen).
//
// Grids of this kind are few-unit and latency-bound: the MQA decode of 128
// query heads over one KV head (64 tiles; as split-KV, 128-key partitions),
// the sliding-window prefill (a tile of 16 heads at one position sees its
// 128-key window).  Walking the keys in 32- or 64-key slices costs one
// dependent round trip to L2 per slice plus a barrier; here the only
// dependent chain is: loads -> QK -> one exchange of head-part scores ->
// softmax -> PV -> one merge of key groups -> stores, with V still
// streaming in during the first three.
//
// Eight waves = NK key groups x NH head parts (NH = HD / 128 columns of 128;
// NK = 8 / NH, KPW = 128 / NK keys per wave: 64 at hd 512, 32 at hd 256).
// Every load moves whole 256-byte key-row parts, four rows per wave-wide
// load: read from L2 in the MFMA operand shape (16 rows x 64 bytes per
// load) the same bytes arrive at about a quarter of the rate (measured
// 37 against 130 GB/s per CU).  Wave (kg, hp) loads:
//   * Q: its 128 columns of the tile's 16 rows (QK B operand, registers);
//   * K: its keys x its columns into its LDS slice (LDS-direct loads); the
//     QK A operand is then read from LDS, 16 bytes per lane, in the key
//     order below; LDS key row r holds its 16-byte chunk c in slot
//     (c + rot(r)) mod 16 so the 16 rows of one read use every bank;
//   * V: its keys x its columns into registers, lane m + 16g taking columns
//     8m .. 8m+7 of keys 8g .. 8g+7 of each 32-key step, then transposed in
//     the lane into the PV A operands of eight MFMAs, MFMA j covering
//     columns 8m + j.
// Products (v_mfma_f32_16x16x32_bf16, keys in M; lane l = lr + 16 lg):
//   S^T = K . Q^T   32-key step ks, block b: M row lr <-> key 32ks + 8(lr/4) + 4b + lr%4
//   O^T += V^T . P^T  MFMA j: M row m <-> column 128hp + 8m + j
// so lane (lr, lg) holds the scores of keys 32ks + 8lg .. +7, in order --
// the PV B operand as it stands -- and ends with row lr's columns
// 128hp + 32lg .. +31.  The NH head parts' partial scores are summed
// through LDS in a fixed order (the NH waves of a key group then hold
// bit-identical scores); each key group keeps its own (max, sum, output),
// and the NK groups are combined once, in a fixed order, through LDS, each
// wave combining and storing 128 / NK columns of the 16 rows.
//
// Softmax: the multi-tile kernel's running max / running sum (the e4ee9fdc
// commit log of the pages), one step per key group and one combination of
// the groups; scores in base 2 (x = q.k * scale * log2 e);
// O divided once by the sum of the bf16 weights the PV product consumes,
// lse from the fp32 sum (as in attn_kernel.hpp).
#pragma once

#include "device_common.hpp"
#include "mx_quant.hpp"
#include "params.hpp"

namespace fmha {

template <int HD>
struct PassShape {
    static_assert(HD == 256 || HD == 512, "the one-pass kernel serves hd 256 and 512");
    static constexpr int NH = HD / 128;       // head parts of 128 columns
    static constexpr int NW = 8;              // waves (16 at hd 512, 32 keys each, measured slower)
    static constexpr int NK = NW / NH;        // key groups
    static constexpr int KPW = 128 / NK;      // keys per wave
    static constexpr int KS = KPW / 32;       // 32-key steps per wave
    static constexpr int CPW = 128 / NK;      // columns each wave combines and stores
    static constexpr int LPR = CPW / 4;       // lanes per row in the store (4 columns each)
    static constexpr int RPI = 64 / LPR;      // rows per store instruction
    static constexpr int K_BYTES = NW * KPW * 256;             // every wave's K slice (128 keys x HD)
    static constexpr int S_BYTES = NW * KS * 2 * 4 * 64 * 4;   // partial scores of every wave
    // after the QK products (the K slices are free): every wave's 16 x 128
    // fp32 output tile, and the row maxima / sums exchanged between waves
    static constexpr int O_BYTES = NW * 16 * 512;
    static constexpr int SMALL_BYTES = NW * 16 * 4 * 4;          // per wave and row: m, l, lq
    // (written with the tiles, once every wave is done with K and the scores)
    static constexpr int SMALL_OFF = O_BYTES;
    static constexpr int SMEM = K_BYTES + S_BYTES;  // 160 KiB at hd 512, 80 KiB at hd 256
    static_assert(O_BYTES + SMALL_BYTES <= SMEM && SMEM <= 160 * 1024, "LDS budget");
};

// The NK key groups of a pass or pass-loop workgroup combined and stored.
// Each wave parks its 16 x 128 fp32 tile in LDS (16-byte chunk c of row r at
// chunk c ^ r: one wave-wide write or read then touches every bank once)
// with its rows' (m, l, lq) -- at hd 512 in its own K slice (16 KiB, read by
// no other wave, so no barrier is needed before the writes), at hd 256 (8 KiB
// slices) from the start of LDS once every wave is done with the K slices
// and the scores; then wave (kg, hp) combines the groups' tiles, in
// a fixed order, over columns 128 hp + CPW kg .. + CPW -- a store instruction
// writes RPI rows x 4 CPW contiguous bytes.  out_row / lse_idx: the output
// rows of this lane (lane / LPR + RPI ps), computed by the caller.
template <int HD, bool SPLIT>
__device__ __forceinline__ void pass_combine_store(const FwdParams &p, unsigned char *smem, int wave, int lane, int klo,
                                                   int khi, float m, float l, float lq, const f32x4 (&acc)[8],
                                                   const int64_t (&out_row)[16 / PassShape<HD>::RPI],
                                                   const int64_t (&lse_idx)[16 / PassShape<HD>::RPI]) {
    using S = PassShape<HD>;
    constexpr int NH = S::NH, NK = S::NK, KPW = S::KPW;
    constexpr int CPW = S::CPW, LPR = S::LPR, RPI = S::RPI;
    constexpr int PASSES = 16 / RPI;
    const int kg = wave / NH, hp = wave % NH;
    const int lr = lane & 15, lg = lane >> 4;
    const int col0 = 128 * hp;
    constexpr bool OWN = KPW * 256 >= 16 * 512 + 16 * 16;  // tile and records fit the wave's K slice
    auto tile = [&](int w) __attribute__((always_inline)) { return smem + w * (OWN ? KPW * 256 : 16 * 512); };
    // per wave and row: m, l, lq
    auto rec_of = [&](int w) __attribute__((always_inline)) {
        return OWN ? reinterpret_cast<float *>(smem + w * KPW * 256 + 16 * 512)
                   : reinterpret_cast<float *>(smem + S::SMALL_OFF) + w * 16 * 4;
    };
    // key group g holds keys [klo + KPW g, ...): it has data iff that is below khi
    const int n_groups = min(NK, (khi - klo + KPW - 1) / KPW);  // wave-uniform
    if constexpr (!OWN) lds_barrier();  // every wave is done with the K slices and the scores
    if (kg < n_groups) {
        unsigned char *mine = tile(wave);
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int chunk = (8 * lg + 2 * t + h) ^ lr;
                *reinterpret_cast<f32x4 *>(mine + lr * 512 + chunk * 16) =
                    f32x4{acc[4 * h][t], acc[4 * h + 1][t], acc[4 * h + 2][t], acc[4 * h + 3][t]};
            }
        if (lg == 0) *reinterpret_cast<f32x4 *>(rec_of(wave) + lr * 4) = f32x4{m, l, lq, 0.f};
    }
    lds_barrier();
    const int q = lane % LPR;
    const int cw = CPW * kg + 4 * q;  // column within the head part
    const int c = col0 + cw;
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
        const int rr = lane / LPR + RPI * ps;
        f32x4 part_o[NK], rec[NK];
#pragma unroll
        for (int g = 0; g < NK; ++g) {
            if (g < n_groups) {
                const int w = g * NH + hp;
                part_o[g] = *reinterpret_cast<const f32x4 *>(tile(w) + rr * 512 + (((cw >> 2) ^ rr) * 16));
                rec[g] = *reinterpret_cast<const f32x4 *>(rec_of(w) + rr * 4);
            } else {
                part_o[g] = f32x4{0.f, 0.f, 0.f, 0.f};
                rec[g] = f32x4{-INFINITY, 0.f, 0.f, 0.f};
            }
        }
        float M = -INFINITY;
#pragma unroll
        for (int g = 0; g < NK; ++g) M = fmaxf(M, rec[g][0]);
        const float M_use = (M == -INFINITY) ? 0.f : M;
        float L = 0.f, LQ = 0.f;
        f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int g = 0; g < NK; ++g) {
            const float wgt = fast_exp2(rec[g][0] - M_use);  // 0 for a group with no visible key
            L += wgt * rec[g][1];
            LQ += wgt * rec[g][2];
            o += wgt * part_o[g];
        }
        if (out_row[ps] < 0) continue;
        const float inv = LQ > 0.f ? 1.f / LQ : 0.f;
        const float lse_val = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
        o = o * inv;
        const bool lse_lane = hp == 0 && kg == 0 && q == 0;
        if constexpr (SPLIT) {
            __builtin_nontemporal_store(o, reinterpret_cast<f32x4 *>(p.o_part + out_row[ps] * HD + c));
            if (lse_lane) p.lse_part[out_row[ps]] = lse_val;
        } else {
            if (p.out_format != kOutBf16) {
                // 32-column MX blocks over 8 adjacent lanes of the row
                const int64_t orow = out_row[ps];
                const float v4[4] = {o[0], o[1], o[2], o[3]};
                mx_store_block_8lanes(v4, p.out_format, p.o_codes + orow * (p.out_format == kOutMxFp8E4M3 ? HD : HD / 2),
                                      p.o_scales + orow * (HD / 32), c & ~31, q & 7);
            } else {
                uint2 packed;
                packed.x = (uint32_t)bf16_bits(o[0]) | ((uint32_t)bf16_bits(o[1]) << 16);
                packed.y = (uint32_t)bf16_bits(o[2]) | ((uint32_t)bf16_bits(o[3]) << 16);
                *reinterpret_cast<uint2 *>(p.o + out_row[ps] + c) = packed;
            }
            if (lse_lane && p.lse != nullptr) p.lse[lse_idx[ps]] = lse_val;
        }
    }
}

template <int HD, bool SPLIT>
__global__ __launch_bounds__(512, 2) void pass_kernel(const FwdParams p) {
    using S = PassShape<HD>;
    constexpr int NH = S::NH, KPW = S::KPW, KS = S::KS;
    constexpr int LPR = S::LPR, RPI = S::RPI;
    __shared__ __attribute__((aligned(16))) unsigned char smem[S::SMEM];

    fetch_launch_params(p);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int kg = wave / NH;  // key group
    const int hp = wave % NH;  // head part
    const int lr = lane & 15;
    const int lg = lane >> 4;

    // ---- work unit: row blocks fastest (regrouped per XCD when they share
    // K/V, last block first), then partitions, KV heads, batch rows --------
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
    const int s_k = p.seqlens ? min(max(p.seqlens[b], 0), p.s_k) : p.s_k;

    const int row0 = rb * 16;
    const int row_last = min(row0 + 16, p.rows) - 1;
    const int pos_lo = s_k - p.T + row0 / p.group;
    const int pos_hi = s_k - p.T + row_last / p.group;
    int klo = part * p.split_len;
    int khi = min(klo + p.split_len, s_k);
    if (p.causal) khi = min(khi, pos_hi + 1);
    if (p.window > 0) klo = max(klo, pos_lo - p.window + 1);

    // this lane's row and its visible keys
    const int row = row0 + lr;
    const bool row_ok = row < p.rows;
    const int t_row = row_ok ? row / p.group : 0;
    const int h_row = kvh * p.group + (row_ok ? row % p.group : 0);
    int r_lo, r_hi;
    {
        const int pos = s_k - p.T + t_row;
        r_hi = p.causal ? min(khi, pos + 1) : khi;
        r_lo = p.window > 0 ? max(klo, pos - p.window + 1) : klo;
        if (!row_ok) r_hi = r_lo;
    }

    const int k0 = klo + KPW * kg;  // this wave's first key
    const bool active = k0 < khi;    // wave-uniform
    const int col0 = 128 * hp;      // this wave's first column

    // ---- the pass's loads: Q and K issued at once, V per 32-key step once
    // that step's QK is issued (the last step's after the softmax at hd 512),
    // so that the QK products, the head-part exchange and the softmax run
    // while V streams in -- a wave issues in order, and with every load ahead
    // of them those waited for the whole pass's ingest (sliding-window
    // prefill 10.2 -> 10.0 us, MQA decode hd 512 over 128 keys 9.6 -> 9.0
    // us).  Keys past the range read key khi - 1 (finite data, weight 0);
    // rows past the end read row 0 of the group and are zeroed ------------
    // chunk c of LDS key row r sits in slot (c + rot(r)) mod 16: the 16 rows
    // one QK operand read touches (keys 8(i/4) + 4b + i%4 of a 32-key step)
    // fall in 16 different slots
    auto rot_of = [](int r) __attribute__((always_inline)) { return (r + 4 * (r >> 4)) & 15; };
    unsigned char *sKw = smem + wave * KPW * 256;
    u32x4 qraw[4];
    u32x4 vr[KS][8];
    if (active) {
        const uint16_t *qp = p.q + (int64_t)b * p.q_sb + (int64_t)t_row * p.q_st + (int64_t)h_row * p.q_sh + col0 + 8 * lg;
#pragma unroll
        for (int s = 0; s < 4; ++s) qraw[s] = *reinterpret_cast<const u32x4 *>(qp + 32 * s);
        __builtin_amdgcn_sched_barrier(0);
        // K: KPW / 4 wave-wide loads of four whole 256-byte row parts into the
        // wave's LDS slice (lane L lands at byte 16 L of the load's 1 KiB)
        const uint16_t *kbase = p.k + (int64_t)b * p.k_sb + (int64_t)kvh * p.k_sh + col0;
#pragma unroll
        for (int it = 0; it < KPW / 4; ++it) {
            const int r = 4 * it + lg;
            const int chunk = (lr - rot_of(r)) & 15;
            const int key = min(k0 + r, khi - 1);
            load_lds_16<false>(kbase + key_offset(key, p.k_st) + 8 * chunk, sKw + it * 1024);
        }
        __builtin_amdgcn_sched_barrier(0);  // Q, then K: the waits below count on that order
    }
    const uint16_t *vbase = p.v + (int64_t)b * p.v_sb + (int64_t)kvh * p.v_sh + col0 + 8 * lr;
    auto issue_v = [&](int ks) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int key = min(k0 + 32 * ks + 8 * lg + i, khi - 1);
            vr[ks][i] = *reinterpret_cast<const u32x4 *>(vbase + key_offset(key, p.v_st));
        }
    };

    // ---- QK over this wave's columns, then the fixed-order sum over the NH
    // head parts of the key group ------------------------------------------
    f32x4 sc[KS][2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) sc[ks][0] = sc[ks][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (active) {
        const unsigned qmask = row_ok ? 0xffffffffu : 0u;
        bf16x8 qf[4];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            // Q and this step's K have landed; the later steps' K and the
            // earlier steps' V (8 loads per step) may still fly
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(8 * (KS - 1)));
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            __builtin_amdgcn_sched_barrier(0);  // nothing that reads a load result moves above the wait
            if (ks == 0) {
#pragma unroll
                for (int s = 0; s < 4; ++s) qf[s] = __builtin_bit_cast(bf16x8, qraw[s] & qmask);
            }
            bf16x8 kf[4][2];
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int blk = 0; blk < 2; ++blk) {
                    const int r = 32 * ks + 8 * (lr >> 2) + 4 * blk + (lr & 3);
                    kf[s][blk] =
                        *reinterpret_cast<const bf16x8 *>(sKw + r * 256 + 16 * ((4 * s + lg + rot_of(r)) & 15));
                }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int blk = 0; blk < 2; ++blk) sc[ks][blk] = mfma_16x16x32(kf[s][blk], qf[s], sc[ks][blk]);
            __builtin_amdgcn_sched_barrier(0);
            if (KS == 1 || ks + 1 < KS) issue_v(ks);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    float *sS = reinterpret_cast<float *>(smem + S::K_BYTES);
    // one 16-byte record per lane and 16-key block: [wave][ks][blk][lane]
    auto s_slot = [&](int w, int ks, int blk) __attribute__((always_inline)) {
        return reinterpret_cast<f32x4 *>(sS) + ((w * KS + ks) * 2 + blk) * 64 + lane;
    };
    if (active) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) *s_slot(wave, ks, blk) = sc[ks][blk];
    }
    // LDS-only barrier: V may still be in flight (a full __syncthreads()
    // would wait for it here)
    lds_barrier();
    if (active) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
                f32x4 a = *s_slot(kg * NH, ks, blk);
#pragma unroll
                for (int q = 1; q < NH; ++q) a += *s_slot(kg * NH + q, ks, blk);
                sc[ks][blk] = a;
            }
    }

    // output rows of this lane in the combine step, fixed before any barrier:
    // lane (rr, q) = (lane / LPR, lane % LPR) takes 4 columns of rows rr,
    // rr + RPI, ... (the integer divisions by the group size are done here)
    constexpr int PASSES = 16 / RPI;
    int64_t out_row[PASSES];  // o_part row (split) or element offset of the row (fused); -1: past the end
    int64_t lse_idx[PASSES];
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
        const int rw = row0 + lane / LPR + RPI * ps;
        const int t_o = rw / p.group, h_o = kvh * p.group + rw % p.group;
        lse_idx[ps] = ((int64_t)b * p.n_h + h_o) * p.T + t_o;
        if (rw >= p.rows) out_row[ps] = -1;
        else if (SPLIT) out_row[ps] = (((int64_t)b * p.n_h + h_o) * p.T + t_o) * p.n_split_total + p.part_offset + part;
        else if (p.out_format != kOutBf16) out_row[ps] = ((int64_t)b * p.T + t_o) * p.n_h + h_o;
        else out_row[ps] = (int64_t)b * p.o_sb + (int64_t)t_o * p.o_st + (int64_t)h_o * p.o_sh;
    }

    // ---- softmax of the key group (its own reference maximum) and
    // O^T += V^T . P^T over the wave's keys ------------------------------------
    float m = -INFINITY, l = 0.f, lq = 0.f;
    f32x4 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (active) {
        float x[KS][8];
        float mx = -INFINITY;
        // keys visible to every row of the tile (the first row's upper bound,
        // the last row's lower one): the wave's keys need no mask
        const int pos_f = s_k - p.T + row0 / p.group;
        const int full_hi = p.causal ? min(khi, pos_f + 1) : khi;
        const int full_lo = p.window > 0 ? max(klo, pos_hi - p.window + 1) : klo;
        if (k0 >= full_lo && k0 + KPW <= full_hi) {  // wave-uniform
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    x[ks][j] = (j < 4 ? sc[ks][0][j] : sc[ks][1][j - 4]) * p.scale_log2;
                    mx = fmaxf(mx, x[ks][j]);
                }
        } else {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int key = k0 + 32 * ks + 8 * lg + j;
                    const float s = j < 4 ? sc[ks][0][j] : sc[ks][1][j - 4];
                    x[ks][j] = (key >= r_lo && key < r_hi) ? s * p.scale_log2 : -INFINITY;
                    mx = fmaxf(mx, x[ks][j]);
                }
        }
        m = row4_max(mx);
        const float m_use = (m == -INFINITY) ? 0.f : m;
        bf16x8 pt[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float pj = fast_exp2(x[ks][j] - m_use);
                const __bf16 pb = to_bf16(pj);
                pt[ks][j] = pb;
                l += pj;
                lq += (float)pb;
            }
        if (KS > 1) issue_v(KS - 1);
        // V^T operands: element i of MFMA j's operand is V[key 8lg + i][8lr + j]
        // (dword u pairs keys 2u, 2u+1 -- halves of dword j/2 of registers 2u, 2u+1)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (KS > 1) {  // step 0's V before the last step's, issued last
                if (ks == 0) __builtin_amdgcn_s_waitcnt(waitcnt_vm(8));
                else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const unsigned sel = (j & 1) ? 0x07060302u : 0x05040100u;
                u32x4 a;
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    a[u] = __builtin_amdgcn_perm(vr[ks][2 * u + 1][j >> 1], vr[ks][2 * u][j >> 1], sel);
                acc[j] = mfma_16x16x32(__builtin_bit_cast(bf16x8, a), pt[ks], acc[j]);
            }
            if (KS > 1) __builtin_amdgcn_sched_barrier(0);
        }
        l = row4_sum(l);
        lq = row4_sum(lq);
    }

    pass_combine_store<HD, SPLIT>(p, smem, wave, lane, klo, khi, m, l, lq, acc, out_row, lse_idx);
}

// The same tile over any number of 128-key passes (few-unit grids whose
// tiles see more than 128 keys: MQA decode and short prefill over longer
// caches).  Pass P: wave (kg, hp) takes keys klo + 128 P + KPW kg .. + KPW - 1;
// its K slice is requested by pass P-1 as soon as every wave is done reading
// the slices, its V registers at the end of pass P-1, so the QK product
// waits for K only.  The head-part scores meet through LDS between two
// barriers (the first also frees the K slices for the next pass's loads);
// each key group keeps a running (max, sum, output) -- the multi-tile
// kernel's online softmax of the e4ee9fdc commit log of the pages -- and the
// groups merge once at the end, as in pass_kernel.  Measured against the
// per-wave kernel it replaced: MQA decode hd 256 over 512 keys 16.3 ->
// 14.7 us, hd 512 27.1 -> 25.8 us.  (Run for a single pass it was 3-7%
// slower than pass_kernel, which keeps that case.)
template <int HD, bool SPLIT>
__global__ __launch_bounds__(512, 2) void pass_loop_kernel(const FwdParams p) {
    using S = PassShape<HD>;
    constexpr int NH = S::NH, KPW = S::KPW, KS = S::KS;
    constexpr int LPR = S::LPR, RPI = S::RPI;
    __shared__ __attribute__((aligned(16))) unsigned char smem[S::SMEM];

    fetch_launch_params(p);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int kg = wave / NH;  // key group
    const int hp = wave % NH;  // head part
    const int lr = lane & 15;
    const int lg = lane >> 4;

    // ---- work unit: row blocks fastest (regrouped per XCD when they share
    // K/V, last block first), then partitions, KV heads, batch rows --------
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
    const int s_k = p.seqlens ? min(max(p.seqlens[b], 0), p.s_k) : p.s_k;

    const int row0 = rb * 16;
    const int row_last = min(row0 + 16, p.rows) - 1;
    const int pos_lo = s_k - p.T + row0 / p.group;
    const int pos_hi = s_k - p.T + row_last / p.group;
    int klo = part * p.split_len;
    int khi = min(klo + p.split_len, s_k);
    if (p.causal) khi = min(khi, pos_hi + 1);
    if (p.window > 0) klo = max(klo, pos_lo - p.window + 1);

    // this lane's row and its visible keys
    const int row = row0 + lr;
    const bool row_ok = row < p.rows;
    const int t_row = row_ok ? row / p.group : 0;
    const int h_row = kvh * p.group + (row_ok ? row % p.group : 0);
    int r_lo, r_hi;
    {
        const int pos = s_k - p.T + t_row;
        r_hi = p.causal ? min(khi, pos + 1) : khi;
        r_lo = p.window > 0 ? max(klo, pos - p.window + 1) : klo;
        if (!row_ok) r_hi = r_lo;
    }

    const int col0 = 128 * hp;  // this wave's first column

    // ---- loads.  chunk c of LDS key row r sits in slot (c + rot(r)) mod 16:
    // the 16 rows one QK operand read touches (keys 8(i/4) + 4b + i%4 of a
    // 32-key step) fall in 16 different slots.  K and V are buffer loads
    // from the wave's first key row of the pass (32-bit lane offsets, the
    // host keeps a wave's rows within 2^31 bytes); keys past the range read
    // key khi - 1 (finite data, weight 0)
    auto rot_of = [](int r) __attribute__((always_inline)) { return (r + 4 * (r >> 4)) & 15; };
    unsigned char *sKw = smem + wave * KPW * 256;
    const uint16_t *kbase = p.k + (int64_t)b * p.k_sb + (int64_t)kvh * p.k_sh + col0;
    const uint16_t *vbase = p.v + (int64_t)b * p.v_sb + (int64_t)kvh * p.v_sh + col0;
    const unsigned kstride = (unsigned)p.k_st * 2u, vstride = (unsigned)p.v_st * 2u;
    auto issue_k = [&](int k0) __attribute__((always_inline)) {
        const uint16_t *kw = kbase + key_offset(k0, p.k_st);
        const int last = khi - 1 - k0;
#pragma unroll
        for (int it = 0; it < KPW / 4; ++it) {
            const int r = 4 * it + lg;
            load_lds_buf(kw, (unsigned)min(r, last) * kstride + 16u * ((lr - rot_of(r)) & 15), sKw + it * 1024);
        }
    };
    u32x4 vr[KS][8];  // V[key k0 + 32ks + 8lg + i][col0 + 8lr .. +7]
    auto issue_v = [&](int k0) __attribute__((always_inline)) {
        const uint16_t *vw = vbase + key_offset(k0, p.v_st);
        const int last = khi - 1 - k0;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int i = 0; i < 8; ++i)
                vr[ks][i] = load16_buf<false>(vw, (unsigned)min(32 * ks + 8 * lg + i, last) * vstride + 16u * lr);
    };
    float *sS = reinterpret_cast<float *>(smem + S::K_BYTES);
    // one 16-byte record per lane and 16-key block: [wave][ks][blk][lane]
    auto s_slot = [&](int w, int ks, int blk) __attribute__((always_inline)) {
        return reinterpret_cast<f32x4 *>(sS) + ((w * KS + ks) * 2 + blk) * 64 + lane;
    };

    // ---- passes of 128 keys.  Pass P: wave (kg, hp) takes keys
    // klo + 128 P + KPW kg .. + KPW - 1 and columns col0 .. col0 + 127.  Its
    // K slice was requested by pass P-1 (right after every wave was done
    // reading the slices) and its V registers at the end of pass P-1: the
    // QK product waits for K only.  The head-part scores meet through LDS
    // between two barriers (the first also frees the K slices for the next
    // pass's loads, the second publishes the scores); each key group keeps
    // a running (max, sum, output) -- the multi-tile kernel's online softmax
    // of the e4ee9fdc commit log of the pages -- over its passes.
    const int npass = khi > klo ? (khi - klo + 127) / 128 : 0;  // workgroup-uniform
    float m = -INFINITY, l = 0.f, lq = 0.f;
    f32x4 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    u32x4 qraw[4];
    {
        const uint16_t *qp = p.q + (int64_t)b * p.q_sb + (int64_t)t_row * p.q_st + (int64_t)h_row * p.q_sh + col0 + 8 * lg;
#pragma unroll
        for (int s = 0; s < 4; ++s) qraw[s] = *reinterpret_cast<const u32x4 *>(qp + 32 * s);
    }
    if (npass > 0 && klo + KPW * kg < khi) {
        __builtin_amdgcn_sched_barrier(0);
        issue_k(klo + KPW * kg);
        __builtin_amdgcn_sched_barrier(0);  // Q, then K, then V: the waits below count on that order
        issue_v(klo + KPW * kg);
        __builtin_amdgcn_sched_barrier(0);
    }
    bf16x8 qf[4];
    for (int P = 0; P < npass; ++P) {
        const int k0 = klo + 128 * P + KPW * kg;  // this wave's first key of the pass
        const bool active = k0 < khi;             // wave-uniform
        // ---- QK over this wave's columns
        f32x4 sc[KS][2];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) sc[ks][0] = sc[ks][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (active) {
            // the pass's K has landed (its V, requested after it, may still fly)
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(8 * KS));
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            if (P == 0) {
                const unsigned qmask = row_ok ? 0xffffffffu : 0u;
#pragma unroll
                for (int s = 0; s < 4; ++s) qf[s] = __builtin_bit_cast(bf16x8, qraw[s] & qmask);
            }
            // the K operand reads of RS head-dim steps issued before their
            // MFMAs (a read waited for right before its MFMA costs a full LDS
            // round trip each; at hd 512 all four steps at once would not fit
            // the registers beside the pass's V)
            constexpr int RS = HD == 512 ? 2 : 4;
#pragma unroll
            for (int s2 = 0; s2 < 4; s2 += RS) {
                bf16x8 kf[RS][KS][2];
#pragma unroll
                for (int s = 0; s < RS; ++s)
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                        for (int blk = 0; blk < 2; ++blk) {
                            const int r = 32 * ks + 8 * (lr >> 2) + 4 * blk + (lr & 3);
                            kf[s][ks][blk] = *reinterpret_cast<const bf16x8 *>(
                                sKw + r * 256 + 16 * ((4 * (s2 + s) + lg + rot_of(r)) & 15));
                        }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int s = 0; s < RS; ++s)
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                        for (int blk = 0; blk < 2; ++blk)
                            sc[ks][blk] = mfma_16x16x32(kf[s][ks][blk], qf[s2 + s], sc[ks][blk]);
            }
        }
        // every wave is done reading the K slices (and the previous pass's
        // scores): request the next pass's K, publish this pass's partial
        // scores (a single pass needs neither, nor this barrier)
        if (P > 0 || P + 1 < npass) lds_barrier();
        const bool next_active = P + 1 < npass && k0 + 128 < khi;  // wave-uniform
        if (next_active) issue_k(k0 + 128);
        if (active) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int blk = 0; blk < 2; ++blk) *s_slot(wave, ks, blk) = sc[ks][blk];
        }
        lds_barrier();
        if (!active) continue;  // (a wave inactive in a pass is inactive in every later pass)
        // ---- the fixed-order sum over the NH head parts of the key group
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
                f32x4 a = *s_slot(kg * NH, ks, blk);
#pragma unroll
                for (int q = 1; q < NH; ++q) a += *s_slot(kg * NH + q, ks, blk);
                sc[ks][blk] = a;
            }
        // ---- online softmax of the key group and O^T += V^T . P^T
        float x[KS][8];
        float mx = -INFINITY;
        // keys visible to every row of the tile (the first row's upper
        // bound, the last row's lower one): the wave's keys need no mask
        const int full_hi = p.causal ? min(khi, pos_lo + 1) : khi;
        const int full_lo = p.window > 0 ? max(klo, pos_hi - p.window + 1) : klo;
        if (k0 >= full_lo && k0 + 32 * KS <= full_hi) {  // wave-uniform
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    x[ks][j] = (j < 4 ? sc[ks][0][j] : sc[ks][1][j - 4]) * p.scale_log2;
                    mx = fmaxf(mx, x[ks][j]);
                }
        } else {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int key = k0 + 32 * ks + 8 * lg + j;
                    const float s = j < 4 ? sc[ks][0][j] : sc[ks][1][j - 4];
                    x[ks][j] = (key >= r_lo && key < r_hi) ? s * p.scale_log2 : -INFINITY;
                    mx = fmaxf(mx, x[ks][j]);
                }
        }
        const float m_new = fmaxf(m, row4_max(mx));
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        if (P > 0) {  // (exp2(-inf) = 0 for a group with no visible key so far)
            const float alpha = fast_exp2(m - m_use);
            l *= alpha;
            lq *= alpha;
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[j] = acc[j] * alpha;
        }
        m = m_new;
        bf16x8 pt[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float pj = fast_exp2(x[ks][j] - m_use);
                const __bf16 pb = to_bf16(pj);
                pt[ks][j] = pb;
                l += pj;
                lq += (float)pb;
            }
        // V^T operands: element i of MFMA j's operand is V[key 8lg + i][8lr + j]
        // (dword u pairs keys 2u, 2u+1 -- halves of dword j/2 of registers 2u, 2u+1)
        if (next_active) __builtin_amdgcn_s_waitcnt(waitcnt_vm(KPW / 4));  // (the next K may fly)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const unsigned sel = (j & 1) ? 0x07060302u : 0x05040100u;
                u32x4 a;
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    a[u] = __builtin_amdgcn_perm(vr[ks][2 * u + 1][j >> 1], vr[ks][2 * u][j >> 1], sel);
                acc[j] = mfma_16x16x32(__builtin_bit_cast(bf16x8, a), pt[ks], acc[j]);
            }
        // the V registers are free: request the next pass's V
        if (next_active) {
            __builtin_amdgcn_sched_barrier(0);
            issue_v(k0 + 128);
        }
    }
    l = row4_sum(l);
    lq = row4_sum(lq);

    // output rows of this lane in the combine step, fixed before its
    // barriers: lane (rr, q) = (lane / LPR, lane % LPR) takes 4 columns of
    // rows rr, rr + RPI, ... (the integer divisions by the group size)
    constexpr int PASSES = 16 / RPI;
    int64_t out_row[PASSES];  // o_part row (split) or element offset of the row (fused); -1: past the end
    int64_t lse_idx[PASSES];
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
        const int rw = row0 + lane / LPR + RPI * ps;
        const int t_o = rw / p.group, h_o = kvh * p.group + rw % p.group;
        lse_idx[ps] = ((int64_t)b * p.n_h + h_o) * p.T + t_o;
        if (rw >= p.rows) out_row[ps] = -1;
        else if (SPLIT) out_row[ps] = (((int64_t)b * p.n_h + h_o) * p.T + t_o) * p.n_split_total + p.part_offset + part;
        else if (p.out_format != kOutBf16) out_row[ps] = ((int64_t)b * p.T + t_o) * p.n_h + h_o;
        else out_row[ps] = (int64_t)b * p.o_sb + (int64_t)t_o * p.o_st + (int64_t)h_o * p.o_sh;
    }

    pass_combine_store<HD, SPLIT>(p, smem, wave, lane, klo, khi, m, l, lq, acc, out_row, lse_idx);
}

}  // namespace fmha
