// attn_kernel.hpp -- the fused attention kernel for gfx950.
//
// One workgroup (4 waves) computes one 16-row tile of one (batch, kv head)
// over one key range.  A row is one (query position t, query head h) that
// reads this KV head, numbered r = t * group + (h - kv*group): the GQA/MQA
// query heads sharing K/V are stacked into the same MFMA tile, and the rows
// of a tile have the same or adjacent positions (tight mask ranges).
//
// The four waves form NK key groups x NH head-dimension parts (HDP = HD/NH
// columns each, 64 or 128):
//   * key group g takes keys [c + 32g, c + 32g + 32) of every chunk of
//     32*NK keys and keeps its own online-softmax state; the NK groups are
//     merged once at the end, in a fixed order;
//   * head part j loads only columns [j*HDP, (j+1)*HDP) of K and V, so every
//     byte of K/V is fetched once per workgroup and the output accumulator
//     is 16 rows x HDP columns per wave for every hd (<= 32 registers).
//     The NH partial QK scores of a slice are summed through LDS in a fixed
//     order, so the NH waves of a key group hold bit-identical scores and
//     probabilities.
//
// Both products are taken transposed, keys in the MFMA M dimension
// (v_mfma_f32_16x16x32_bf16; lane l = lr + 16*lg):
//   S^T (keys x rows) = K . Q^T      lane holds S^T[4*lg + j][lr]
//   O^T (hd x rows)  += V^T . P^T    lane holds O^T[4*lg + j][lr]
// so all softmax state of row lr lives in lanes lr, lr+16, lr+32, lr+48:
// the running max needs two butterfly steps, the rescale factor is a
// per-lane scalar, and the probabilities leave the QK result registers in
// exactly the B-operand layout of the PV product (the 32-key reduction
// index is permuted identically in both PV operands).
//
// Data movement per 32-key slice and wave:
//   * K: HBM -> QK A-operand registers (lane lr + 16*lg loads 16 bytes of
//     key lr at column offset 32*s + 8*lg) -- no LDS round trip;
//   * V: HBM -> a wave-private LDS slice with global_load_lds_dwordx4 (no
//     registers held in flight); a run of lanes covers one whole key-row
//     part, so loads stay coalesced.  The 16-byte chunks of LDS key row k
//     are rotated by 2*((k/4) % 4) positions: the PV operand gathers V[k][d]
//     for keys 4*lg + j across the four lane groups, and the rotation puts
//     the four groups on disjoint LDS banks.
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
#include "params.hpp"

namespace fmha {

template <int HD, int NK, int NH>
struct AttnShape {
    static_assert(NK * NH == 4, "four waves per workgroup");
    static constexpr int HDP = HD / NH;               // head-dim columns per wave
    static constexpr int KSTEPS = HDP / 32;           // QK MFMA steps
    static constexpr int NB = HDP / 16;               // 16-column blocks of O^T
    static constexpr int CHUNKS = HDP / 8;            // 16-byte chunks per key-row part
    static constexpr int ROW_BYTES = HDP * 2;         // LDS key-row part
    static constexpr int KEYS_PER_LOAD = 64 / CHUNKS;  // keys per wave-wide 16-byte load
    static constexpr int VLOADS = 32 / KEYS_PER_LOAD;
    static constexpr int SLOTS = NB * 4 + 3;          // merge record per lane: m, l, lq, O^T
    static constexpr int M_BYTES = (NK - 1) * NH * SLOTS * 64 * 4;
    static constexpr int S_BUF = NH > 1 ? 4 * 8 * 64 * 4 : 0;  // one buffer of partial scores
    static_assert(HDP == 64 || HDP == 128, "head-dim part of 64 or 128 columns");
};

// ONE: every workgroup's key range fits one chunk of 32*NK keys (split-KV
// decode with 128-key partitions, short caches).  The chunk loop collapses to
// one pass, no state is carried in from an earlier slice, and the output
// accumulator is born from the first PV product -- so nothing but Q is live
// while the loads are in flight, which buys a fifth wave per SIMD.
template <int HD, int NK, int NH, bool SPLIT, bool ONE>
__global__ __launch_bounds__(256, (ONE ? (NH == 1 ? 5 : 4) : 2)) void attn_kernel(const FwdParams p) {
    using S = AttnShape<HD, NK, NH>;
    constexpr int HDP = S::HDP, KSTEPS = S::KSTEPS, NB = S::NB, CHUNKS = S::CHUNKS;
    constexpr int ROW_BYTES = S::ROW_BYTES, KEYS_PER_LOAD = S::KEYS_PER_LOAD, VLOADS = S::VLOADS;
    constexpr int SLOTS = S::SLOTS;
    // one V slice per wave (the final key-group merge reuses that space);
    // partial-score buffers alternate by slice parity (one suffices for ONE)
    constexpr int V_BYTES = 4 * 32 * ROW_BYTES;
    constexpr int VM_BYTES = V_BYTES > S::M_BYTES ? V_BYTES : S::M_BYTES;
    __shared__ __attribute__((aligned(16))) unsigned char smem[VM_BYTES + (ONE ? 1 : 2) * S::S_BUF];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int kg = wave / NH;  // key group
    const int hp = wave % NH;  // head-dim part
    const int lr = lane & 15;
    const int lg = lane >> 4;

    // ---- work unit: row tiles fastest (they share K/V through L2), then
    // partitions (consecutive key ranges of one KV head; their partial outputs
    // are adjacent in memory), then KV heads and batches.  With several row
    // tiles the units are regrouped so that one XCD (one L2) runs consecutive
    // ones: blocks are dealt to the 8 XCDs round-robin ------------------------
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

    const int row0 = rb * 16;
    const int row_last = min(row0 + 16, p.rows) - 1;
    const int pos_lo = p.s_k - p.T + row0 / p.group;
    const int pos_hi = p.s_k - p.T + row_last / p.group;
    // key range: the partition, cut to the union of the tile rows' masks
    int klo = part * p.split_len;
    int khi = min(klo + p.split_len, p.s_k);
    if (p.causal) khi = min(khi, pos_hi + 1);
    if (p.window > 0) klo = max(klo, pos_lo - p.window + 1);

    const int row = row0 + lr;
    const bool row_ok = row < p.rows;
    const int t = row_ok ? row / p.group : 0;
    const int h = kvh * p.group + (row_ok ? row % p.group : 0);
    const int pos = p.s_k - p.T + t;
    int r_hi = p.causal ? min(khi, pos + 1) : khi;
    const int r_lo = p.window > 0 ? max(klo, pos - p.window + 1) : klo;
    if (!row_ok) r_hi = r_lo;  // no visible key: the row stays at -inf

    const int col0 = hp * HDP;  // first head-dim column of this wave
    bf16x8 qf[KSTEPS];          // Q^T B operand: Q[row lr][col0 + 32*s + 8*lg + 0..7]
    {
        const uint16_t *qp = p.q + (int64_t)b * p.q_sb + (int64_t)t * p.q_st + (int64_t)h * p.q_sh + col0 + 8 * lg;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s)
            qf[s] = row_ok ? *reinterpret_cast<const bf16x8 *>(qp + 32 * s) : bf16x8{};
    }

    f32x4 acc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY;  // running max (base 2), equal in the 4 lanes of a row
    float l = 0.f;        // this lane's share of the fp32 sum of weights (-> lse)
    float lq = 0.f;       // the same over the bf16-rounded weights (-> O)

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
            const uint16_t *kp = kbase + (int64_t)key * p.k_st + 8 * lg;
#pragma unroll
            for (int s = 0; s < KSTEPS; ++s) kf[blk][s] = *reinterpret_cast<const bf16x8 *>(kp + 32 * s);
        }
    };
    // LDS row r of the slice holds its 16-byte chunk c in slot (c + rot(r)) % CHUNKS:
    // the 16 keys of one transposed read then cover the LDS banks evenly
    auto rot_of = [](int r) __attribute__((always_inline)) { return (2 * (r & 7)) % CHUNKS; };

    // ---- QK and (NH > 1) the fixed-order sum of the head-part scores -----------
    auto scores = [&](int k0, bool active, int iter, const bf16x8 (&kf)[2][KSTEPS], f32x4 &s0, f32x4 &s1) __attribute__((always_inline)) {
        s0 = f32x4{0.f, 0.f, 0.f, 0.f};
        s1 = f32x4{0.f, 0.f, 0.f, 0.f};
        if (active) {
#pragma unroll
            for (int s = 0; s < KSTEPS; ++s) {
                s0 = mfma_16x16x32(kf[0][s], qf[s], s0);
                s1 = mfma_16x16x32(kf[1][s], qf[s], s1);
            }
        }
        if constexpr (NH > 1) {
            float *buf = sS + (ONE ? 0 : (iter & 1) * (4 * 8 * 64));
            if (active) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    buf[(wave * 8 + j) * 64 + lane] = s0[j];
                    buf[(wave * 8 + 4 + j) * 64 + lane] = s1[j];
                }
            }
            __syncthreads();
            if (active) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float a = 0.f, c2 = 0.f;
#pragma unroll
                    for (int q = 0; q < NH; ++q) {
                        a += buf[((kg * NH + q) * 8 + j) * 64 + lane];
                        c2 += buf[((kg * NH + q) * 8 + 4 + j) * 64 + lane];
                    }
                    s0[j] = a;
                    s1[j] = c2;
                }
            }
        }
    };

    // ---- mask + online softmax: returns the rescale factor, fills P^T ----------
    auto softmax = [&](int k0, const f32x4 &s0, const f32x4 &s1, bf16x8 &pt) __attribute__((always_inline)) -> float {
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
        const float m_new = ONE ? mx : fmaxf(m, mx);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = ONE ? 0.f : fast_exp2(m - m_use);
        float psum = 0.f, qsum = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float pj = fast_exp2(x[j] - m_use);
            const __bf16 pb = to_bf16(pj);
            pt[j] = pb;
            psum += pj;
            qsum += (float)pb;
        }
        l = ONE ? psum : l * alpha + psum;
        lq = ONE ? qsum : lq * alpha + qsum;
        m = m_new;
        return alpha;
    };

    // ---- O^T = alpha O^T + V^T . P^T from the wave's LDS slice.  Item j of
    // lane (lr, lg) is key 4*lg + j (j < 4) or 16 + 4*lg + (j - 4), column
    // 16*nb + lr.  Each half comes from one transposing read
    // (ds_read_b64_tr_b16: within a 16-lane block, lane i item j receives
    // element i%4 of the 8 bytes addressed by lane 4j + i/4), so lane s of
    // block lg addresses key 4*lg + s/4 (+16), columns 16*nb + 4*(s%4) .. +3.
    int tr_row[2], tr_col[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        tr_row[half] = 16 * half + 4 * lg + (lr >> 2);
        tr_col[half] = 4 * (lr & 3);
    }
    auto pv = [&](float alpha, const bf16x8 &pt) __attribute__((always_inline)) {
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
            if constexpr (ONE) {
                acc[nb] = mfma_16x16x32(vt, pt, f32x4{0.f, 0.f, 0.f, 0.f});
            } else {
                acc[nb] = acc[nb] * alpha;
                acc[nb] = mfma_16x16x32(vt, pt, acc[nb]);
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
                    load_lds_16(vbase + (int64_t)key * p.v_st + chunk * 8, sVw + it * 64 * 16);
                }
                load_k(k0, kf);
                __builtin_amdgcn_sched_barrier(0);  // every load issued before the first wait
            }
            f32x4 s0, s1;
            scores(k0, active, 0, kf, s0, s1);
            if (active) {
                bf16x8 pt;
                const float alpha = softmax(k0, s0, s1, pt);
                __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // V has landed in LDS
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                pv(alpha, pt);
            }
        }
    } else {
        // pipelined: K and V of slice n+1 are loaded into registers while slice
        // n is computed; V reaches LDS (rotated) just before its PV product.
        // Plain register loads keep the compiler's wait counting exact, so the
        // waits for slice n leave slice n+1's loads in flight.
        auto load_v = [&](int k0, u32x4 (&vr)[VLOADS]) __attribute__((always_inline)) {
#pragma unroll
            for (int it = 0; it < VLOADS; ++it) {
                const int key = min(k0 + it * KEYS_PER_LOAD + v_row_in_load, khi - 1);
                vr[it] = *reinterpret_cast<const u32x4 *>(vbase + (int64_t)key * p.v_st + v_slot * 8);
            }
        };
        auto step = [&](int n, const bf16x8 (&kf)[2][KSTEPS], const u32x4 (&vr)[VLOADS]) __attribute__((always_inline)) {
            const int k0 = klo + n * chunk_keys + 32 * kg;
            const bool active = k0 < khi;
            f32x4 s0, s1;
            scores(k0, active, n, kf, s0, s1);
            if (!active) return;
            bf16x8 pt;
            const float alpha = softmax(k0, s0, s1, pt);
            // the previous slice's V^T reads are done before its LDS slice is reused
            __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
#pragma unroll
            for (int it = 0; it < VLOADS; ++it) {
                const int r = it * KEYS_PER_LOAD + v_row_in_load;
                const int slot = (v_slot + rot_of(r)) % CHUNKS;
                *reinterpret_cast<u32x4 *>(sVw + r * ROW_BYTES + slot * 16) = vr[it];
            }
            __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
            pv(alpha, pt);
        };
        // two slices per iteration, both loaded up front: the second slice's
        // loads are in flight while the first is computed.  The loads are
        // unconditional (key indices clamp to khi-1, so a slice past the range
        // reads valid memory and is then skipped) and no load target crosses
        // the loop back-edge: both keep the compiler's wait counts exact, so it
        // waits for the first slice only.
        for (int n = 0; n < nslices; n += 2) {
            bf16x8 kfA[2][KSTEPS], kfB[2][KSTEPS];
            u32x4 vrA[VLOADS], vrB[VLOADS];
            load_k(klo + n * chunk_keys + 32 * kg, kfA);
            load_v(klo + n * chunk_keys + 32 * kg, vrA);
            load_k(klo + (n + 1) * chunk_keys + 32 * kg, kfB);
            load_v(klo + (n + 1) * chunk_keys + 32 * kg, vrB);
            __builtin_amdgcn_sched_barrier(0);  // keep all 2 x (K + V) loads ahead of the math
            step(n, kfA, vrA);
            if (n + 1 < nslices) step(n + 1, kfB, vrB);
        }
    }

    // full row sums over the four lanes of a row
    l += xor_shuffle(l, 16);
    l += xor_shuffle(l, 32);
    lq += xor_shuffle(lq, 16);
    lq += xor_shuffle(lq, 32);

    // ---- merge the NK key groups of each head part (fixed order) -----------------
    if constexpr (NK > 1) {
        __syncthreads();  // all V slices and score buffers are consumed
        float *red = reinterpret_cast<float *>(smem);
        if (kg != 0) {
            float *mine = red + ((kg - 1) * NH + hp) * SLOTS * 64 + lane;
            mine[0] = m;
            mine[64] = l;
            mine[128] = lq;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int j = 0; j < 4; ++j) mine[(3 + nb * 4 + j) * 64] = acc[nb][j];
        }
        __syncthreads();
        if (kg != 0) return;
        float M = m;
#pragma unroll
        for (int g = 1; g < NK; ++g) M = fmaxf(M, red[((g - 1) * NH + hp) * SLOTS * 64 + lane]);
        const float M_use = (M == -INFINITY) ? 0.f : M;
        const float w0 = fast_exp2(m - M_use);
        l *= w0;
        lq *= w0;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[nb] = acc[nb] * w0;
#pragma unroll
        for (int g = 1; g < NK; ++g) {
            const float *src = red + ((g - 1) * NH + hp) * SLOTS * 64 + lane;
            const float wgt = fast_exp2(src[0] - M_use);
            l += wgt * src[64];
            lq += wgt * src[128];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[nb][j] += wgt * src[(3 + nb * 4 + j) * 64];
        }
        m = M;
    }
    if (!row_ok) return;

    // ---- epilogue: one division; lse = (m + log2 l) ln 2 -------------------------
    const float inv = lq > 0.f ? 1.f / lq : 0.f;
    const float lse_val = l > 0.f ? (m + __log2f(l)) * kLn2 : -INFINITY;
    if constexpr (SPLIT) {
        const int64_t r = (((int64_t)b * p.n_h + h) * p.T + t) * p.n_split + part;
        float *op = p.o_part + r * HD + col0 + 4 * lg;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) *reinterpret_cast<f32x4 *>(op + 16 * nb) = acc[nb] * inv;
        if (hp == 0 && lg == 0) p.lse_part[r] = lse_val;
    } else {
        uint16_t *op = p.o + (int64_t)b * p.o_sb + (int64_t)t * p.o_st + (int64_t)h * p.o_sh + col0 + 4 * lg;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            uint2 packed;
            packed.x = (uint32_t)bf16_bits(acc[nb][0] * inv) | ((uint32_t)bf16_bits(acc[nb][1] * inv) << 16);
            packed.y = (uint32_t)bf16_bits(acc[nb][2] * inv) | ((uint32_t)bf16_bits(acc[nb][3] * inv) << 16);
            *reinterpret_cast<uint2 *>(op + 16 * nb) = packed;
        }
        if (hp == 0 && lg == 0 && p.lse != nullptr) p.lse[((int64_t)b * p.n_h + h) * p.T + t] = lse_val;
    }
}

}  // namespace fmha
