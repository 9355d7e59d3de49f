// cols_kernel.hpp -- one 16-row tile at hd 512 (and 256) for few-unit grids, over at
// most 128 keys in one pass (the sliding-window MQA prefill, the MQA decode
// over 128 keys, the 128-key partitions of a split call) or, with LOOP, over
// several 128-key passes (the MQA decode over longer caches), with the work
// of a pass divided between the eight waves by keys for the scores and by
// output columns for the product with V, so that no wave's partial result
// has to be summed with another's:
//
//   * scores: wave w takes keys klo + 16w .. +15 over the whole head
//     dimension (16 MFMA steps of 32 columns, four independent chains summed
//     in a fixed order); Q is staged once in LDS for all eight waves, each
//     wave's K rows in its own LDS slice;
//   * softmax: the waves exchange their rows' maxima (one barrier), all take
//     the tile-wide maximum M, and each writes its keys' bf16 weights
//     exp2(x - M) and its rows' partial sums (a second barrier);
//   * O = P V: wave w computes output columns 64w .. 64w+63 over all the
//     tile's keys, reading the weights from LDS and its V columns from
//     registers, and stores them.
//
// Against the one-pass kernel (key groups x head parts of 128 columns) this
// trades its head-part score exchange and its combine of the key groups'
// 16 x 128 fp32 output tiles for two small exchanges (maxima, then 4 KiB of
// weights and the sums), and the last loads to land (V) feed straight into
// the last product and the stores.
//
// Products (v_mfma_f32_16x16x32_bf16, lane l = lr + 16 lg):
//   S^T = K . Q^T   head-dim step s: M row lr <-> key klo + 16w + lr,
//                   N column lr <-> tile row lr; lane (lr, lg) ends with the
//                   scores of row lr for keys 16w + 4lg .. +3
//   O^T += V^T . P^T  32-key step ks, MFMA j (0..3): M row m <-> column
//                   64w + 4m + j; lane (lr, lg) ends with row lr's columns
//                   64w + 16lg .. +15 (element 4t + j in acc[j][t])
// V: lane (lr, lg) loads 8 bytes (4 columns, 64w + 4lr ..) of keys
// 32ks + 8lg .. +7, sixteen lanes covering one 128-byte line of a key row;
// MFMA j's A operand is column 4lr + j of those eight keys, two keys per
// dword (v_perm).
//
// LDS rows of 1 KiB (Q and K) keep 16-byte chunk c of row r in slot
// (c + r) mod 64, so the sixteen rows one operand read touches fall in
// sixteen different slots; the weight rows are padded to 272 bytes for the
// same reason.
//
// Softmax as in the pages' single-tile form (one maximum, one pass of
// exponentials; scores in base 2, x = q.k * scale * log2 e); O divided once by
// the sum of the bf16 weights the PV product consumes, lse from the fp32 sum
// (as in the other kernels).
#pragma once

#include "device_common.hpp"
#include "mx_quant.hpp"
#include "params.hpp"

namespace fmha {

template <int HD>
struct ColsShape {
    static_assert(HD == 256 || HD == 512, "the column-split kernel serves hd 256 and 512");
    static constexpr int NW = 8;                  // waves
    static constexpr int KPW = 16;                // keys per wave (scores)
    static constexpr int CPW = 64;                // output columns per wave
    static constexpr int NPV = HD / CPW;          // waves with output columns (8, or 4 at hd 256)
    static constexpr int ROW = HD * 2;            // bytes per Q / K row (1 KiB at hd 512)
    static constexpr int CH = ROW / 16;           // 16-byte chunks per row
    static constexpr int RPI = 1024 / ROW;        // rows per wave-wide 16-byte load
    static constexpr int LPR = 64 / RPI;          // lanes per row in such a load
    static constexpr int KI = KPW / RPI;          // K load instructions per wave and pass
    static constexpr int HS = HD / 32;            // head-dim steps of the QK product
    static constexpr int P_STRIDE = 128 * 2 + 16; // bytes per weight row (padded)
    static constexpr int Q_OFF = 0;
    static constexpr int K_OFF = Q_OFF + 16 * ROW;
    static constexpr int QK_BYTES = K_OFF + NW * KPW * ROW;  // 144 KiB, filled by LDS-direct loads
    // the exchanges, a separate LDS object: the compiler can then tell their
    // writes from the LDS-direct loads and need not wait for every load in
    // flight (V) before them
    static constexpr int P_OFF = 0;
    static constexpr int MX_OFF = P_OFF + 16 * P_STRIDE;  // row maxima [wave][row]
    static constexpr int SUM_OFF = MX_OFF + NW * 16 * 4;  // (l, lq) [wave][row]
    static constexpr int X_BYTES = SUM_OFF + NW * 16 * 8;
    static_assert(QK_BYTES + X_BYTES <= 160 * 1024, "LDS budget");
};

// MX-coded output of one lane's 16 columns (col0 + 16 lg ..) of row (t, h):
// 32-column blocks over the lane pair lg, lg ^ 1 of the row.
template <int HD>
__device__ __forceinline__ void mx_store_fused(const FwdParams &p, int b, int t, int h, const float (&v)[16], int col0,
                                               int lg) {
    const int64_t orow = ((int64_t)b * p.T + t) * p.n_h + h;
    mx_store_block_2lanes(v, p.out_format, p.o_codes + orow * (p.out_format == kOutMxFp8E4M3 ? HD : HD / 2),
                          p.o_scales + orow * (HD / 32), col0 + 32 * (lg >> 1), lg & 1);
}

template <int HD, bool SPLIT, bool LOOP>
__global__ __launch_bounds__(512, 2) void cols_kernel(const FwdParams p) {
    using S = ColsShape<HD>;
    constexpr int ROW = S::ROW, CH = S::CH, HS = S::HS, KPW = S::KPW, P_STRIDE = S::P_STRIDE;
    constexpr int RPI = S::RPI, LPR = S::LPR, KI = S::KI, NPV = S::NPV;
    __shared__ __attribute__((aligned(16))) unsigned char smem[S::QK_BYTES];
    __shared__ __attribute__((aligned(16))) unsigned char xmem[S::X_BYTES];

    fetch_launch_params(p);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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
    const bool any = khi > klo;  // workgroup-uniform; at most 128 keys without LOOP (host plan)

    // this lane's row (N column of both products) and its visible keys
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
    const int k0 = klo + KPW * wave;  // this wave's first key (scores)
    const bool active = k0 < khi;     // wave-uniform
    const int col0 = S::CPW * wave;   // this wave's first output column
    const bool pv = NPV == S::NW || wave < NPV;  // the wave has output columns (wave-uniform)

    // output addresses of this lane's row
    const int64_t lse_idx = ((int64_t)b * p.n_h + h_row) * p.T + t_row;
    int64_t out_row;
    if (SPLIT) out_row = lse_idx * p.n_split_total + p.part_offset + part;
    else out_row = (int64_t)b * p.o_sb + (int64_t)t_row * p.o_st + (int64_t)h_row * p.o_sh;
    unsigned char *sQ = smem + S::Q_OFF;
    unsigned char *sK = smem + S::K_OFF + wave * KPW * ROW;
    unsigned char *sP = xmem + S::P_OFF;
    float *sMx = reinterpret_cast<float *>(xmem + S::MX_OFF);
    float *sSum = reinterpret_cast<float *>(xmem + S::SUM_OFF);

    // no visible key (an empty partition, or rows before the first key): O =
    // 0, lse = -inf.  Workgroup-uniform, so every load below is issued
    // unconditionally (K: by the waves that hold keys) and the waits count
    // them exactly
    if (!any) {
        if (!row_ok || !pv) return;
        const int c = col0 + 16 * lg;
        if constexpr (SPLIT) {
#pragma unroll
            for (int t = 0; t < 4; ++t)
                *reinterpret_cast<f32x4 *>(p.o_part + out_row * HD + c + 4 * t) = f32x4{0.f, 0.f, 0.f, 0.f};
            if (wave == 0 && lg == 0) p.lse_part[out_row] = -INFINITY;
        } else {
            if (p.out_format != kOutBf16) {
                const float zero[16] = {};
                mx_store_fused<HD>(p, b, t_row, h_row, zero, col0, lg);
            } else {
#pragma unroll
                for (int t = 0; t < 4; ++t) *reinterpret_cast<uint2 *>(p.o + out_row + c + 4 * t) = uint2{0u, 0u};
            }
            if (wave == 0 && lg == 0 && p.lse != nullptr) p.lse[lse_idx] = -INFINITY;
        }
        return;
    }

    // ---- loads, in this order: Q rows 2w, 2w+1 of the tile (LDS, shared by
    // every wave; rows past the end read row 0 of the group: their results
    // are never stored), the wave's 16 K rows (its LDS slice; keys past the
    // range read key khi - 1, finite data, weight 0), V steps 0 and 1
    // (registers); V steps 2 and 3 follow the QK product.  A wave issues in
    // order at the compute unit's ingest rate, so loads placed ahead of the
    // QK product delay it -- and loads placed after it leave the ingest idle
    // while it runs.  Each load moves whole rows (Q, K: one 1 KiB row per
    // wave-wide load; V: four 128-byte lines).
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int rr = 2 * wave + i;  // wave-uniform
        const int r = row0 + rr;
        const bool ok = r < p.rows;
        const int t = ok ? r / p.group : 0;
        const int h = kvh * p.group + (ok ? r % p.group : 0);
        const uint16_t *qrow = p.q + (int64_t)b * p.q_sb + (int64_t)t * p.q_st + (int64_t)h * p.q_sh;
        if constexpr (RPI == 1) {
            load_lds_buf(qrow, 16u * (unsigned)((lane - rr) & (CH - 1)), sQ + rr * ROW);
        } else {
            // two rows per load would need one base for both: one row per
            // load, its half of the lanes (lane L lands at byte 16 L of rows
            // 2w, 2w+1)
            if ((lane >> 5) == i) load_lds_buf(qrow, 16u * (unsigned)((lane - rr) & (CH - 1)), sQ + 2 * wave * ROW);
        }
    }
    const unsigned kstride = (unsigned)p.k_st * 2u, vstride = (unsigned)p.v_st * 2u;
    const uint16_t *khead = p.k + (int64_t)b * p.k_sb + (int64_t)kvh * p.k_sh;
    // the wave's 16 K rows from key k (keys past the range read key khi - 1)
    auto issue_k = [&](int k) __attribute__((always_inline)) {
        const uint16_t *kw = khead + key_offset(k, p.k_st);
        const int last = khi - 1 - k;
#pragma unroll
        for (int it = 0; it < KI; ++it) {
            const int r = RPI * it + lane / LPR;
            load_lds_buf(kw, (unsigned)min(r, last) * kstride + 16u * (unsigned)((lane % LPR - r) & (CH - 1)),
                         sK + it * 1024);
        }
    };
    if (active) issue_k(k0);
    u32x2 vr[4][8];  // V[key kp + 32ks + 8lg + i][col0 + 4lr .. +3] of the pass from key kp
    const uint16_t *vhead = p.v + (int64_t)b * p.v_sb + (int64_t)kvh * p.v_sh + col0;
    auto issue_v = [&](int kp, int ks) __attribute__((always_inline)) {
        // the step's first key row (key khi - 1 for a step past the range),
        // wave-uniform: the buffer base
        const int first = min(kp + 32 * ks, khi - 1);
        const uint16_t *vw = vhead + key_offset(first, p.v_st);
        const int last = khi - 1 - first;  // >= 0
#pragma unroll
        for (int i = 0; i < 8; ++i)
            vr[ks][i] = load8_buf<false>(vw, (unsigned)min(8 * lg + i, last) * vstride + 8u * (unsigned)lr);
    };
    // Q and K have landed (V steps 0 and 1 may still fly), then every wave's
    // Q rows are in LDS
    if (pv) {
        __builtin_amdgcn_sched_barrier(0);
        issue_v(klo, 0);
        issue_v(klo, 1);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(16));
    } else {
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    }
    lds_barrier();

    // keys visible to every row of the tile (the first row's upper bound, the
    // last row's lower one): a wave whose keys lie inside needs no mask
    const int pos_f = s_k - p.T + row0 / p.group;
    const int full_hi = p.causal ? min(khi, pos_f + 1) : khi;
    const int full_lo = p.window > 0 ? max(klo, pos_hi - p.window + 1) : klo;

    // ---- passes of 128 keys (one without LOOP).  Pass P from key kp: the
    // scores of wave w's keys kp + 16w .. +15, the tile-wide row maximum
    // (running over the passes: the accumulators and sums are rescaled when
    // it grows -- the multi-tile online softmax of the e4ee9fdc commit log
    // of the pages), the weights, and O += P V over the pass's keys.  The
    // next pass's K is requested into the wave's own slice once its QK
    // product has read it, the next pass's V registers once its PV product
    // has consumed them.
    const int npass = LOOP ? (khi - klo + 127) / 128 : 1;  // workgroup-uniform, >= 1
    float M = -INFINITY, L = 0.f, LQ = 0.f;
    f32x4 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int P = 0; P < npass; ++P) {
        const int kp = klo + 128 * P;
        const int kw0 = kp + KPW * wave;  // this wave's first key of the pass
        const bool act = kw0 < khi;       // wave-uniform
        // ---- S^T = K . Q^T over the whole head dimension
        float x[4];
        float mx = -INFINITY;
        if (act) {
            f32x4 sacc[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) sacc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s4 = 0; s4 < HS; s4 += 4) {
                bf16x8 kf[4], qf[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int slot = (4 * (s4 + u) + lg + lr) & (CH - 1);
                    kf[u] = *reinterpret_cast<const bf16x8 *>(sK + lr * ROW + 16 * slot);
                    qf[u] = *reinterpret_cast<const bf16x8 *>(sQ + lr * ROW + 16 * slot);
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) sacc[u] = mfma_16x16x32(kf[u], qf[u], sacc[u]);
            }
            const f32x4 sc = ((sacc[0] + sacc[1]) + sacc[2]) + sacc[3];
            if (kw0 >= full_lo && kw0 + KPW <= full_hi) {  // wave-uniform
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    x[t] = sc[t] * p.scale_log2;
                    mx = fmaxf(mx, x[t]);
                }
            } else {
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int key = kw0 + 4 * lg + t;
                    x[t] = (key >= r_lo && key < r_hi) ? sc[t] * p.scale_log2 : -INFINITY;
                    mx = fmaxf(mx, x[t]);
                }
            }
            mx = row4_max(mx);
        }
        // the next pass's K into the wave's slice, once the QK reads are done
        bool next_k = false;
        if constexpr (LOOP) {
            next_k = P + 1 < npass && kw0 + 128 < khi;  // wave-uniform
            if (next_k) {
                __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
                __builtin_amdgcn_sched_barrier(0);
                issue_k(kw0 + 128);
            }
        }
        if (pv) {
            __builtin_amdgcn_sched_barrier(0);
            issue_v(kp, 2);
            issue_v(kp, 3);
            __builtin_amdgcn_sched_barrier(0);
        }

        // ---- the tile-wide row maximum, the weights and their sums
        if (lg == 0) sMx[wave * 16 + lr] = mx;
        lds_barrier();
        float m_new = M;
#pragma unroll
        for (int w = 0; w < S::NW; ++w) m_new = fmaxf(m_new, sMx[w * 16 + lr]);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        if constexpr (LOOP) {
            if (P > 0) {  // (exp2(-inf) = 0 while no key was visible)
                const float alpha = fast_exp2(M - m_use);
                L *= alpha;
                LQ *= alpha;
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[j] = acc[j] * alpha;
            }
        }
        M = m_new;
        {
            float l = 0.f, lq = 0.f;
            unsigned pw[2] = {0u, 0u};
            if (act) {
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const float pj = fast_exp2(x[t] - m_use);
                    const uint16_t pb = bf16_bits(pj);
                    l += pj;
                    lq += __uint_as_float((unsigned)pb << 16);
                    pw[t >> 1] |= (unsigned)pb << (16 * (t & 1));
                }
                l = row4_sum(l);
                lq = row4_sum(lq);
            }
            *reinterpret_cast<uint2 *>(sP + lr * P_STRIDE + 2 * (KPW * wave + 4 * lg)) = uint2{pw[0], pw[1]};
            if (lg == 0) *reinterpret_cast<float2 *>(sSum + 2 * (wave * 16 + lr)) = float2{l, lq};
        }
        lds_barrier();
#pragma unroll
        for (int w = 0; w < S::NW; ++w) {
            const float2 s2 = *reinterpret_cast<const float2 *>(sSum + 2 * (w * 16 + lr));
            L += s2.x;
            LQ += s2.y;
        }

        // ---- O^T += V^T . P^T over the pass's keys, this wave's 64 columns
        const int nks = pv ? min(4, (khi - kp + 31) / 32) : 0;  // 32-key steps holding keys (uniform)
#pragma unroll
        for (int ks = 0; ks < 4 && pv; ++ks) {
            // step ks's V has landed (the later steps', 8 loads each, and the
            // next pass's K, KI, requested between steps 1 and 2, may fly)
            if (ks == 0) {
                if (next_k) __builtin_amdgcn_s_waitcnt(waitcnt_vm(24 + KI));
                else __builtin_amdgcn_s_waitcnt(waitcnt_vm(24));
            } else if (ks == 1) {
                if (next_k) __builtin_amdgcn_s_waitcnt(waitcnt_vm(16 + KI));
                else __builtin_amdgcn_s_waitcnt(waitcnt_vm(16));
            } else if (ks == 2) {
                __builtin_amdgcn_s_waitcnt(waitcnt_vm(8));
            } else {
                __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
            }
            __builtin_amdgcn_sched_barrier(0);
            if (ks < nks) {
                const bf16x8 pt = *reinterpret_cast<const bf16x8 *>(sP + lr * P_STRIDE + 64 * ks + 16 * lg);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const unsigned sel = (j & 1) ? 0x07060302u : 0x05040100u;
                    u32x4 a;
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        a[u] = __builtin_amdgcn_perm(vr[ks][2 * u + 1][j >> 1], vr[ks][2 * u][j >> 1], sel);
                    acc[j] = mfma_16x16x32(__builtin_bit_cast(bf16x8, a), pt, acc[j]);
                }
            }
        }
        // the V registers are free: the next pass's steps 0 and 1 (its K has
        // landed: the wait before step 3 covered it; a wave with no output
        // columns waits for its K here)
        if constexpr (LOOP) {
            if (!pv) __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
            if (P + 1 < npass && pv) {
                __builtin_amdgcn_sched_barrier(0);
                issue_v(kp + 128, 0);
                issue_v(kp + 128, 1);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }

    // ---- stores: row lr, columns col0 + 16lg + 4t + j = acc[j][t] / LQ.  fp32
    // partials and bf16 rows pass through the wave's own K slice (free since
    // its QK product, read by no other wave) so that every store instruction
    // writes whole 128-byte lines: stored straight from the MFMA layout, a
    // lane's 16-byte pieces lie 64 bytes apart (the split partials, written
    // non-temporally, then took 1.4x as long as the one-pass kernel's) -----
    const float inv = LQ > 0.f ? 1.f / LQ : 0.f;
    const float lse_val = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
    if (!pv) return;
    const int n_ok = row_last - row0 + 1;  // rows of the tile that exist (workgroup-uniform)
    auto wave_sync = []() __attribute__((always_inline)) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };
    if constexpr (SPLIT) {
        // [16 rows][64 columns] fp32, 16-byte chunk q of row r at chunk q ^ r
#pragma unroll
        for (int t = 0; t < 4; ++t)
            *reinterpret_cast<f32x4 *>(sK + lr * 256 + 16 * ((4 * lg + t) ^ lr)) =
                f32x4{acc[0][t] * inv, acc[1][t] * inv, acc[2][t] * inv, acc[3][t] * inv};
        wave_sync();
        const int cc = lane & 15;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rr = 4 * i + (lane >> 4);
            const f32x4 o = *reinterpret_cast<const f32x4 *>(sK + rr * 256 + 16 * (cc ^ rr));
            if (rr < n_ok) {
                const int rw = row0 + rr;
                const int t_o = rw / p.group, h_o = kvh * p.group + rw % p.group;
                const int64_t orow = (((int64_t)b * p.n_h + h_o) * p.T + t_o) * p.n_split_total + p.part_offset + part;
                __builtin_nontemporal_store(o, reinterpret_cast<f32x4 *>(p.o_part + orow * HD + col0 + 4 * cc));
            }
        }
        if (wave == 0 && lg == 0 && row_ok) p.lse_part[out_row] = lse_val;
    } else if (p.out_format != kOutBf16) {
        if (!row_ok) return;
        float v16[16];
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) v16[4 * t + j] = acc[j][t] * inv;
        mx_store_fused<HD>(p, b, t_row, h_row, v16, col0, lg);
        if (wave == 0 && lg == 0 && p.lse != nullptr) p.lse[lse_idx] = lse_val;
    } else {
        // [16 rows][64 columns] bf16 (128-byte rows), chunk q of row r at q ^ (r & 7)
        auto pk = [&](int j, int t) __attribute__((always_inline)) {
            return (uint32_t)bf16_bits(acc[j][t] * inv) | ((uint32_t)bf16_bits(acc[j + 1][t] * inv) << 16);
        };
#pragma unroll
        for (int h = 0; h < 2; ++h)
            *reinterpret_cast<u32x4 *>(sK + lr * 128 + 16 * ((2 * lg + h) ^ (lr & 7))) =
                u32x4{pk(0, 2 * h), pk(2, 2 * h), pk(0, 2 * h + 1), pk(2, 2 * h + 1)};
        wave_sync();
        const int cc = lane & 7;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int rr = 8 * i + (lane >> 3);
            const u32x4 o = *reinterpret_cast<const u32x4 *>(sK + rr * 128 + 16 * (cc ^ (rr & 7)));
            if (rr < n_ok) {
                const int rw = row0 + rr;
                const int t_o = rw / p.group, h_o = kvh * p.group + rw % p.group;
                *reinterpret_cast<u32x4 *>(p.o + (int64_t)b * p.o_sb + (int64_t)t_o * p.o_st + (int64_t)h_o * p.o_sh +
                                           col0 + 8 * cc) = o;
            }
        }
        if (wave == 0 && lg == 0 && row_ok && p.lse != nullptr) p.lse[lse_idx] = lse_val;
    }
}

}  // namespace fmha
