// rows_split_kernel.hpp -- row-parallel attention at hd 512 with every
// 16-row tile's head dimension split over two waves.
//
// The row-parallel kernel (rows_kernel.hpp) gives each wave a whole tile:
// at hd 512 its Q and O tiles alone take 192 registers, so it runs one wave
// per SIMD, and counters showed the MFMA pipe busy 13% of the time -- the
// single wave stalls on LDS reads, on its own dependent MFMAs and at every
// barrier with nothing else to issue.  Here a workgroup of eight waves
// serves the same 64 rows: wave w takes tile w / 2 and head-dim half w % 2
// (256 columns of Q, of the QK product and of O), so a wave needs half the
// registers and two waves share each SIMD.
//
// Per 32-key chunk a wave computes its half's partial scores S^T_h = K_h .
// Q_h^T (8 head-dim steps, keys in the MFMA M dimension as in
// attn_kernel.hpp) and the two halves meet through LDS: each wave writes its
// partial tile, and after the next step's barrier -- the barrier the chunk
// pipeline has anyway -- reads its partner's and adds the two in a fixed
// order (half 0 + half 1), so both waves of a tile hold bit-identical scores
// and take identical softmax decisions.  Each then multiplies its 256 V^T
// columns by the weights.  Everything else -- chunk pipeline through two K
// and two V LDS slots filled by LDS-direct buffer loads, the lazy online
// softmax (the reference maximum moves only when exceeded by more than 2^8),
// the QK product of chunk n+1 interleaved with the PV product of chunk n,
// the division by the bf16 weight sum and lse from the fp32 sum -- follows
// rows_kernel.hpp.  LDS key row r holds its 16-byte chunk c at slot
// (c + 2 (r mod 8)) mod 64.
#pragma once

#include "device_common.hpp"
#include "mx_quant.hpp"
#include "params.hpp"

namespace fmha {

template <int HD, bool SPLIT>
__global__ __launch_bounds__(512, 2) void rows_split_kernel(const FwdParams p) {
    static_assert(HD == 512, "the head-split row kernel serves hd 512");
    constexpr int HW = HD / 2;              // head-dim columns per wave
    constexpr int KSTEPS = HW / 32;         // QK MFMA steps per wave (8)
    constexpr int NB = HW / 16;             // 16-column blocks of the wave's O^T (16)
    constexpr int BPS = NB / KSTEPS;        // PV blocks issued per QK step (2)
    constexpr int CHUNKS = HD / 8;          // 16-byte chunks per key row (64)
    constexpr int ROW_BYTES = HD * 2;       // one key row = one wave-wide 1 KiB load
    constexpr int KC = 32, KB = 2;          // keys per chunk, 16-key blocks per chunk
    constexpr int SLOT_BYTES = KC * ROW_BYTES;
    constexpr int LOADS = KC / 8;           // rows (= loads) per wave per slot
    constexpr int ROWS = 64;                // rows per workgroup (4 tiles)
    // two K and two V chunk slots, and the exchange of partial scores: two
    // parities x 8 waves x 2 blocks x 64 lanes x 16 bytes (160 KiB in all)
    __shared__ __attribute__((aligned(16))) unsigned char sK0[SLOT_BYTES];
    __shared__ __attribute__((aligned(16))) unsigned char sK1[SLOT_BYTES];
    __shared__ __attribute__((aligned(16))) unsigned char sV0[SLOT_BYTES];
    __shared__ __attribute__((aligned(16))) unsigned char sV1[SLOT_BYTES];
    __shared__ __attribute__((aligned(16))) f32x4 xch[2][8][KB][64];

    fetch_launch_params(p);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ti = wave >> 1;  // tile of the workgroup
    const int hp = wave & 1;   // head-dim half
    const int lr = lane & 15;
    const int lg = lane >> 4;

    // ---- work unit (row blocks fastest, last block first; regrouped per XCD
    // when they share K/V) -- the order of rows_kernel.hpp
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

    const int row0 = rb * ROWS;
    const int row_last = min(row0 + ROWS, p.rows) - 1;
    int klo = part * p.split_len;
    int khi = min(klo + p.split_len, s_k);
    if (p.causal) khi = min(khi, s_k - p.T + row_last / p.group + 1);
    if (p.window > 0) klo = max(klo, s_k - p.T + row0 / p.group - p.window + 1);

    // ---- this wave's tile: its rows, masks and fully visible key range ----
    const int first = row0 + 16 * ti;
    const int last = min(first + 15, row_last);
    const int row = first + lr;
    const bool row_ok = row <= row_last;
    const int t_row = row_ok ? row / p.group : 0;
    const int h_row = kvh * p.group + (row_ok ? row % p.group : 0);
    int r_lo, r_hi, full_lo, full_hi;
    {
        const int pos = s_k - p.T + t_row;
        r_hi = p.causal ? min(khi, pos + 1) : khi;
        r_lo = p.window > 0 ? max(klo, pos - p.window + 1) : klo;
        if (!row_ok) r_hi = r_lo;
        if (first > row_last) {
            full_lo = khi;
            full_hi = klo;
        } else {
            const int pos_first = s_k - p.T + first / p.group;
            const int pos_last = s_k - p.T + last / p.group;
            full_hi = p.causal ? min(khi, pos_first + 1) : khi;
            full_lo = p.window > 0 ? max(klo, pos_last - p.window + 1) : klo;
        }
    }

    // scores enter the softmax as s * c with c = |scale| log2 e > 0 (a
    // negative scale flips the sign of Q; a zero scale is taken as the
    // smallest normal float), as in rows_kernel.hpp
    const float c_scale = fmaxf(fabsf(p.scale_log2), FLT_MIN);
    const unsigned q_flip = p.scale_log2 < 0.f ? 0x80008000u : 0u;
    // Q^T B operand of the wave's half: Q[row lr][256 hp + 32 s + 8 lg + 0..7];
    // loaded unconditionally (rows past the end read row 0 of the group) and
    // masked once the first chunks' loads are issued
    u32x4 qraw[KSTEPS];
    {
        const uint16_t *qp =
            p.q + (int64_t)b * p.q_sb + (int64_t)t_row * p.q_st + (int64_t)h_row * p.q_sh + HW * hp + 8 * lg;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) qraw[s] = *reinterpret_cast<const u32x4 *>(qp + 32 * s);
    }
    bf16x8 qf[KSTEPS];

    f32x4 acc[NB];
    f32x4 accq = {0.f, 0.f, 0.f, 0.f};  // the bf16 weight sum of row lr, in every element (-> O)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, neg_m = 0.f, l = 0.f;
    bf16x8 ones;
#pragma unroll
    for (int j = 0; j < 8; ++j) ones[j] = (__bf16)1.0f;

    const uint16_t *kbase = p.k + (int64_t)b * p.k_sb + (int64_t)kvh * p.k_sh;
    const uint16_t *vbase = p.v + (int64_t)b * p.v_sb + (int64_t)kvh * p.v_sh;
    auto rot_of = [](int r) __attribute__((always_inline)) { return (2 * (r & 7)) % CHUNKS; };

    // ---- one chunk HBM -> an LDS slot: wave w loads key rows LOADS w ..
    // LOADS w + LOADS - 1, one whole row per load, lane L fetching the 16-byte
    // chunk that belongs at slot L under the row's rotation; a row past khi
    // rereads row khi - 1 (finite data, weight 0)
    // A chunk inside the range is addressed from its first key row with fixed
    // lane offsets (row times token stride plus the chunk; the host keeps a
    // chunk's rows within 2^31 bytes), one scalar multiply per chunk; the last
    // chunk of a range clamps row by row.
    unsigned ld_off[LOADS], ld_koff[LOADS], ld_voff[LOADS];
#pragma unroll
    for (int it = 0; it < LOADS; ++it) {
        const int r = LOADS * wave + it;
        ld_off[it] = 16u * ((lane - rot_of(r)) & (CHUNKS - 1));
        ld_koff[it] = (unsigned)(r * p.k_st * 2) + ld_off[it];
        ld_voff[it] = (unsigned)(r * p.v_st * 2) + ld_off[it];
    }
    auto issue = [&](const uint16_t *base, int64_t st, const unsigned (&full_off)[LOADS], int k0,
                     unsigned char *slot) __attribute__((always_inline)) {
        if (k0 + KC <= khi) {  // workgroup-uniform
            const uint16_t *cb = base + key_offset(k0, st);
#pragma unroll
            for (int it = 0; it < LOADS; ++it)
                load_lds_buf(cb, full_off[it], slot + (LOADS * wave + it) * ROW_BYTES);
        } else {
#pragma unroll
            for (int it = 0; it < LOADS; ++it) {
                const int r = LOADS * wave + it;
                load_lds_buf(base + key_offset(min(k0 + r, khi - 1), st), ld_off[it], slot + r * ROW_BYTES);
            }
        }
    };

    // per-lane LDS byte offsets of the operand reads: K chunk 32 hp + 4 s + lg
    // of key row 16 kb + lr (+ 16 kb ROW_BYTES); V^T columns 256 hp + 16 nb +
    // tr_col of key row 16 half + tr_row0 (+ 16 half ROW_BYTES) -- a row's
    // rotation depends on its index mod 8, which the 16-row offsets keep
    const int tr_row0 = 4 * lg + (lr >> 2);
    const int tr_col = 4 * (lr & 3);
    int k_at[KSTEPS], v_at[NB];
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) k_at[s] = lr * ROW_BYTES + ((32 * hp + 4 * s + lg + rot_of(lr)) % CHUNKS) * 16;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int c = HW * hp + 16 * nb + tr_col;
        v_at[nb] = tr_row0 * ROW_BYTES + (((c >> 3) + rot_of(tr_row0)) % CHUNKS) * 16 + (c & 7) * 2;
    }
    auto read_k = [&](const unsigned char *sK, int s, bf16x8 (&kf)[KB]) __attribute__((always_inline)) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
            kf[kb] = *reinterpret_cast<const bf16x8 *>(sK + k_at[s] + 16 * kb * ROW_BYTES);
    };
    auto read_v = [&](const unsigned char *sV, int nb) __attribute__((always_inline)) {
        bf16x4 q2[2];
#pragma unroll
        for (int half = 0; half < 2; ++half)
            q2[half] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (__attribute__((address_space(3))) bf16x4 *)(sV + v_at[nb] + 16 * half * ROW_BYTES));
        return __builtin_shufflevector(q2[0], q2[1], 0, 1, 2, 3, 4, 5, 6, 7);
    };

    // ---- the wave's partial scores of a chunk, published for the partner
    auto publish = [&](int par, const f32x4 (&part_s)[KB]) __attribute__((always_inline)) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) xch[par][wave][kb][lane] = part_s[kb];
    };
    // ... and the full scores, half 0 + half 1 in that order in both waves
    auto combine = [&](int par, const f32x4 (&own)[KB], f32x4 (&sc)[KB]) __attribute__((always_inline)) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const f32x4 other = xch[par][wave ^ 1][kb][lane];
            sc[kb] = hp == 0 ? own[kb] + other : other + own[kb];
        }
    };

    // ---- online softmax, first half (as rows_kernel.hpp): mask the chunks
    // that cut through a row's range, raw-score maximum, lazy rescale
    auto prep = [&](int k0, f32x4 (&sc)[KB]) __attribute__((always_inline)) {
        if (!(k0 >= full_lo && k0 + KC <= full_hi)) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int key = k0 + 16 * kb + 4 * lg + j;
                    if (key < r_lo || key >= r_hi) sc[kb][j] = -INFINITY;
                }
        }
        float mr = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int j = 0; j < 4; ++j) mr = fmaxf(mr, sc[kb][j]);
        if (__any(mr * c_scale > m + kRescaleLog2)) {
            const float m_new = fmaxf(m, row4_max(mr) * c_scale);
            const float alpha = fast_exp2(m - ((m_new == -INFINITY) ? 0.f : m_new));
            l *= alpha;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) acc[nb] = acc[nb] * alpha;
            accq = accq * alpha;
            m = m_new;
            neg_m = (m_new == -INFINITY) ? 0.f : -m_new;
        }
    };

    // ---- one step's straight-line part: chunk n's weights, then chunk n+1's
    // partial QK product interleaved with chunk n's PV product (BPS column
    // blocks after each QK step), operands read ahead of their MFMAs
    auto fused = [&](const unsigned char *sK, f32x4 (&sn)[KB], const f32x4 (&sc)[KB], const unsigned char *sV)
                     __attribute__((always_inline)) {
        constexpr int D = 4, R = D + 1;     // K read-ahead (steps), ring size
        constexpr int DV = 2, RV = DV + 1;  // V^T read-ahead (steps), ring size
        bf16x8 kf[R][KB];
        bf16x8 vt[RV][BPS];
#pragma unroll
        for (int s = 0; s < D; ++s) read_k(sK, s, kf[s]);
#pragma unroll
        for (int sv = 0; sv < DV; ++sv)
#pragma unroll
            for (int u = 0; u < BPS; ++u) vt[sv][u] = read_v(sV, sv * BPS + u);
        // raised wave priority over the step's MFMA work (as rows_kernel.hpp)
        __builtin_amdgcn_s_setprio(1);
        bf16x8 pt;
        float psum = 0.f;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float pj = fast_exp2(fmaf(sc[kb][j], c_scale, neg_m));
                pt[kb * 4 + j] = to_bf16(pj);
                psum += pj;
            }
        l += psum;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) sn[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) sn[kb] = mfma_16x16x32(kf[s % R][kb], qf[s], sn[kb]);
#pragma unroll
            for (int u = 0; u < BPS; ++u) acc[s * BPS + u] = mfma_16x16x32(vt[s % RV][u], pt, acc[s * BPS + u]);
            if (s == 0) accq = mfma_16x16x32(ones, pt, accq);
            if (s + D < KSTEPS) read_k(sK, s + D, kf[(s + D) % R]);
            if (s + DV < KSTEPS) {
#pragma unroll
                for (int u = 0; u < BPS; ++u) vt[(s + DV) % RV][u] = read_v(sV, (s + DV) * BPS + u);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
    };

    // ---- the pipeline (rows_kernel.hpp): step n starts with chunk n+1's K
    // and chunk n's V on chip and the wave's partial scores of chunk n in
    // registers; after the barrier it completes chunk n's scores with the
    // partner's half, requests chunk n+2's K and chunk n+1's V into the slots
    // step n-1 finished with, and runs the fused part, publishing its partial
    // scores of chunk n+1 (parity (n+1) % 2: the partner read the other
    // parity before this step's barrier)
    const int nchunks = khi > klo ? (khi - klo + KC - 1) / KC : 0;  // workgroup-uniform
    f32x4 own[KB];
    if (nchunks > 0) {
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
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) qf[s] = __builtin_bit_cast(bf16x8, (qraw[s] & (row_ok ? 0xffffffffu : 0u)) ^ q_flip);
        f32x4 part_s[KB] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
            bf16x8 kf[KB];
            read_k(sK0, s, kf);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) part_s[kb] = mfma_16x16x32(kf[kb], qf[s], part_s[kb]);
        }
        publish(0, part_s);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) own[kb] = part_s[kb];
    }
    auto step = [&](int n, const unsigned char *sKnext, const unsigned char *sVcur, unsigned char *sKfill,
                    unsigned char *sVfill) __attribute__((always_inline)) {
        const int k0 = klo + n * KC;
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        lds_barrier();
        if (n + 2 < nchunks) issue(kbase, p.k_st, ld_koff, k0 + 2 * KC, sKfill);
        if (n + 1 < nchunks) issue(vbase, p.v_st, ld_voff, k0 + KC, sVfill);
        f32x4 sc[KB];
        combine(n & 1, own, sc);
        prep(k0, sc);
        f32x4 sn[KB];
        fused(sKnext, sn, sc, sVcur);
        publish((n + 1) & 1, sn);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) own[kb] = sn[kb];
    };
    // two steps per iteration (the slots alternate); no LDS-direct load
    // crosses the back-edge
    for (int n = 0; n < nchunks; n += 2) {
        step(n, sK1, sV0, sK0, sV1);
        if (n + 1 < nchunks) step(n + 1, sK0, sV1, sK1, sV0);
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    }

    // ---- epilogue: full row sum, one division, lse = (m + log2 l) ln 2; the
    // wave stores its 256 columns (half 0 also the lse)
    l = row4_sum(l);
    if (!row_ok) return;
    const float lq = accq[0];
    const float inv = lq > 0.f ? 1.f / lq : 0.f;
    const float lse_val = l > 0.f ? (m + __log2f(l)) * kLn2 : -INFINITY;
    const int col0 = HW * hp + 4 * lg;
    if constexpr (SPLIT) {
        const int64_t r = (((int64_t)b * p.n_h + h_row) * p.T + t_row) * p.n_split_total + p.part_offset + part;
        float *op = p.o_part + r * HD + col0;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            __builtin_nontemporal_store(acc[nb] * inv, reinterpret_cast<f32x4 *>(op + 16 * nb));
        if (hp == 0 && lg == 0) p.lse_part[r] = lse_val;
    } else if (p.out_format != kOutBf16) {
        // MX codes: 32-column blocks = pairs of 16-column blocks over the row's 4 lanes
        const int64_t orow = ((int64_t)b * p.T + t_row) * p.n_h + h_row;
        uint8_t *crow = p.o_codes + orow * (p.out_format == kOutMxFp8E4M3 ? HD : HD / 2);
        uint8_t *srow = p.o_scales + orow * (HD / 32);
#pragma unroll
        for (int nb = 0; nb < NB; nb += 2) {
            float v[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[j] = acc[nb][j] * inv;
                v[4 + j] = acc[nb + 1][j] * inv;
            }
            mx_store_block_4lanes(v, p.out_format, crow, srow, HW * hp + 16 * nb, lg);
        }
        if (hp == 0 && lg == 0 && p.lse != nullptr) p.lse[((int64_t)b * p.n_h + h_row) * p.T + t_row] = lse_val;
    } else {
        uint16_t *op = p.o + (int64_t)b * p.o_sb + (int64_t)t_row * p.o_st + (int64_t)h_row * p.o_sh + col0;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            uint2 packed;
            packed.x = (uint32_t)bf16_bits(acc[nb][0] * inv) | ((uint32_t)bf16_bits(acc[nb][1] * inv) << 16);
            packed.y = (uint32_t)bf16_bits(acc[nb][2] * inv) | ((uint32_t)bf16_bits(acc[nb][3] * inv) << 16);
            *reinterpret_cast<uint2 *>(op + 16 * nb) = packed;
        }
        if (hp == 0 && lg == 0 && p.lse != nullptr) p.lse[((int64_t)b * p.n_h + h_row) * p.T + t_row] = lse_val;
    }
}

}  // namespace fmha
