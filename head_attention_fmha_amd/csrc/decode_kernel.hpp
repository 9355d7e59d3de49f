// decode_kernel.hpp -- attention for tiles of at most 16 rows (decode and
// short GQA/MQA groups), gfx950.
//
// Same mathematics and register layouts as fwd_kernel.hpp (keys in the MFMA
// M dimension, per-lane softmax state, probabilities passed from the QK
// result registers straight into the PV MFMA), organised for bandwidth:
//
//   * the four waves of a workgroup own disjoint 32-key slices of every
//     128-key chunk and never share staged data, so there is no workgroup
//     barrier until the final merge of the four slices;
//   * K goes from HBM straight into the A-operand registers of the QK MFMA
//     (lane lr + 16*lg loads 16 bytes of key lr at head-dim offset
//     32*s + 8*lg): no LDS round trip;
//   * V goes from HBM straight into a wave-private LDS slice with
//     global_load_lds_dwordx4 (no registers held while the load is in
//     flight); each run of lanes covers one whole key row, so the loads stay
//     fully coalesced;
//   * the 16-byte chunks of LDS key row k are rotated by 2*((k/4) % 4)
//     positions.  The PV operand gathers V[k][d] for keys 4*lg + j across the
//     four lane groups lg and 16 consecutive d: the rotation puts the four
//     groups on disjoint LDS banks;
//   * registers stay near 128 per lane, so four waves per SIMD (four
//     workgroups per CU) keep ~256 KiB of K/V in flight per CU.
#pragma once

#include "device_common.hpp"
#include "fwd_kernel.hpp"

namespace fmha {

template <int HD, bool SPLIT>
__global__ __launch_bounds__(256, 4) void decode_kernel(const FwdParams p) {
    constexpr int NW = 4;
    constexpr int KSTEPS = HD / 32;
    constexpr int NB = HD / 16;
    constexpr int CHUNKS = HD / 8;             // 16-byte chunks per key row
    constexpr int ROW_BYTES = HD * 2;          // LDS key row, unpadded
    constexpr int KEYS_PER_LOAD = 64 / CHUNKS;  // keys covered by one wave-wide 16-byte load
    constexpr int VLOADS = 32 / KEYS_PER_LOAD;
    constexpr int SLOTS = NB * 4 + 3;          // merge record per lane: m, l, lq, O^T
    constexpr int V_BYTES = NW * 32 * ROW_BYTES;
    constexpr int M_BYTES = (NW - 1) * SLOTS * 64 * 4;
    static_assert(HD == 64 || HD == 128, "decode_kernel covers hd 64 and 128");
    __shared__ __attribute__((aligned(16))) unsigned char smem[V_BYTES > M_BYTES ? V_BYTES : M_BYTES];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lr = lane & 15;
    const int lg = lane >> 4;

    int bid = blockIdx.x;
    if (p.xcd_remap) {
        const int per = p.n_units >> 3;
        bid = (bid & 7) * per + (bid >> 3);
    }
    // KV heads fastest: the units that read the same rows of a [token][kv_head][hd]
    // cache (same batch, same partition) run together
    const int kvh = bid % p.n_kv_h;
    bid /= p.n_kv_h;
    const int part = bid % p.n_split;
    const int b = bid / p.n_split;

    // all rows of this (b, kv head) form one tile: rows <= 16
    const int pos_lo = p.s_k - p.T;
    const int pos_hi = p.s_k - 1;
    int klo = part * p.split_len;
    int khi = min(klo + p.split_len, p.s_k);
    if (p.causal) khi = min(khi, pos_hi + 1);
    if (p.window > 0) klo = max(klo, pos_lo - p.window + 1);

    const int row = lr;
    const bool row_ok = row < p.rows;
    const int t = row_ok ? row / p.group : 0;
    const int h = kvh * p.group + (row_ok ? row % p.group : 0);
    const int pos = p.s_k - p.T + t;
    int r_hi = p.causal ? min(khi, pos + 1) : khi;
    const int r_lo = p.window > 0 ? max(klo, pos - p.window + 1) : klo;
    if (!row_ok) r_hi = r_lo;

    bf16x8 qf[KSTEPS];
    {
        const uint16_t *qp = p.q + (int64_t)b * p.q_sb + (int64_t)t * p.q_st + (int64_t)h * p.q_sh + 8 * lg;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s)
            qf[s] = row_ok ? *reinterpret_cast<const bf16x8 *>(qp + 32 * s) : bf16x8{};
    }

    f32x4 acc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, l = 0.f, lq = 0.f;

    const uint16_t *kbase = p.k + (int64_t)b * p.k_sb + (int64_t)kvh * p.k_sh;
    const uint16_t *vbase = p.v + (int64_t)b * p.v_sb + (int64_t)kvh * p.v_sh;
    unsigned char *sV = smem + wave * 32 * ROW_BYTES;

    // V loads: in load `it` lane L fills LDS row it*KEYS_PER_LOAD + L/CHUNKS,
    // slot L%CHUNKS, with the chunk that the row's rotation puts there
    const int v_row_in_load = lane / CHUNKS;
    const int v_slot = lane % CHUNKS;

    for (int c = klo; c < khi; c += 32 * NW) {
        const int k0 = c + 32 * wave;
        if (k0 >= khi) continue;  // wave-uniform
        // the previous slice's LDS reads must be complete before new V lands
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        // ---- V: HBM -> LDS, keys past khi replaced by key khi-1 (weight 0) ------
#pragma unroll
        for (int it = 0; it < VLOADS; ++it) {
            const int r = it * KEYS_PER_LOAD + v_row_in_load;
            const int rot = (2 * ((r >> 2) & 3)) % CHUNKS;
            const int chunk = (v_slot - rot + CHUNKS) % CHUNKS;
            const int key = min(k0 + r, khi - 1);
            load_lds_16(vbase + (int64_t)key * p.v_st + chunk * 8, sV + it * 64 * 16);
        }
        // ---- K: HBM -> QK A-operand registers ------------------------------------
        bf16x8 kf[2][KSTEPS];
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            // keys past khi read key khi-1 instead; their scores are masked
            const int key = min(k0 + 16 * blk + lr, khi - 1);
            const uint16_t *kp = kbase + (int64_t)key * p.k_st + 8 * lg;
#pragma unroll
            for (int s = 0; s < KSTEPS; ++s) kf[blk][s] = *reinterpret_cast<const bf16x8 *>(kp + 32 * s);
        }
        // keep every load of the slice ahead of the first wait
        __builtin_amdgcn_sched_barrier(0);
        // ---- S^T = K . Q^T ------------------------------------------------------
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
            s0 = mfma_16x16x32(kf[0][s], qf[s], s0);
            s1 = mfma_16x16x32(kf[1][s], qf[s], s1);
        }
        // ---- mask, online softmax ------------------------------------------------
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
            const float pj = fast_exp2(x[j] - m_use);
            const __bf16 pb = to_bf16(pj);
            pt[j] = pb;
            psum += pj;
            qsum += (float)pb;
        }
        l = l * alpha + psum;
        lq = lq * alpha + qsum;
        m = m_new;
        // ---- V has landed in LDS ---------------------------------------------------
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // ---- O^T = alpha O^T + V^T . P^T: item j of lane (lr, lg) is key
        // 4*lg + j (j < 4) or 16 + 4*lg + (j - 4); both rows rotate by 2*lg ----------
        const int rot = (2 * lg) % CHUNKS;
        const unsigned char *r0 = sV + (4 * lg) * ROW_BYTES;
        const unsigned char *r1 = r0 + 16 * ROW_BYTES;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int d = 16 * nb + lr;
            const int off = (((d >> 3) + rot) % CHUNKS) * 16 + (d & 7) * 2;
            bf16x8 vt;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                vt[j] = *reinterpret_cast<const __bf16 *>(r0 + j * ROW_BYTES + off);
                vt[4 + j] = *reinterpret_cast<const __bf16 *>(r1 + j * ROW_BYTES + off);
            }
            acc[nb] = acc[nb] * alpha;
            acc[nb] = mfma_16x16x32(vt, pt, acc[nb]);
        }
    }

    l += xor_shuffle(l, 16);
    l += xor_shuffle(l, 32);
    lq += xor_shuffle(lq, 16);
    lq += xor_shuffle(lq, 32);

    // ---- merge the four key slices in a fixed order (wave 0 finishes) -------------
    __syncthreads();  // every wave is done with its V slice
    float *red = reinterpret_cast<float *>(smem);
    if (wave != 0) {
        float *mine = red + (wave - 1) * SLOTS * 64 + lane;
        mine[0] = m;
        mine[64] = l;
        mine[128] = lq;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int j = 0; j < 4; ++j) mine[(3 + nb * 4 + j) * 64] = acc[nb][j];
    }
    __syncthreads();
    if (wave != 0) return;
    float M = m;
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, red[(w - 1) * SLOTS * 64 + lane]);
    const float M_use = (M == -INFINITY) ? 0.f : M;
    {
        const float w0 = fast_exp2(m - M_use);
        l *= w0;
        lq *= w0;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[nb] = acc[nb] * w0;
    }
#pragma unroll
    for (int w = 1; w < NW; ++w) {
        const float *src = red + (w - 1) * SLOTS * 64 + lane;
        const float wgt = fast_exp2(src[0] - M_use);
        l += wgt * src[64];
        lq += wgt * src[128];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[nb][j] += wgt * src[(3 + nb * 4 + j) * 64];
    }
    m = M;
    if (!row_ok) return;

    const float inv = lq > 0.f ? 1.f / lq : 0.f;
    const float lse_val = l > 0.f ? (m + __log2f(l)) * kLn2 : -INFINITY;
    if constexpr (SPLIT) {
        const int64_t r = (((int64_t)b * p.n_h + h) * p.T + t) * p.n_split + part;
        float *op = p.o_part + r * HD + 4 * lg;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) *reinterpret_cast<f32x4 *>(op + 16 * nb) = acc[nb] * inv;
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
