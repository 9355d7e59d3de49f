// stream_kernel.hpp -- one-pass attention at hd 128 on gfx950: every
// workgroup's keys fit one 128-key pass (the split-KV decode with 128-key
// partitions; caches of at most 128 keys).
//
// Such work is bound by HBM bandwidth alone, and this GPU streams reads at
// its best only with the non-temporal hint on loads that fetch whole cache
// lines.  A wave-wide 16-byte load in the MFMA operand layout covers 16 key
// rows x 64 bytes, half lines; so neither operand is loaded in that layout:
//   * K (QK A operand, one key row per lane): HBM -> LDS by non-temporal
//     LDS-direct loads, each covering four whole 256-byte key rows; the
//     operand is then read from LDS (16 bytes per lane);
//   * V (PV A operand, the transpose of the stored rows): HBM -> registers by
//     non-temporal loads, each covering four whole key rows (lane m + 16g
//     takes columns 8m .. 8m+7 of keys 8g .. 8g+7, one key per load), then
//     transposed inside the lane: eight 8-column x 8-key blocks become the
//     operands of eight MFMAs, MFMA j covering head-dim columns 8m + j
//     (m = 0..15).  Each output column is still one contiguous dot product
//     over the keys, just on a different MFMA row than in attn_kernel.
//
// Products as in attn_kernel.hpp (v_mfma_f32_16x16x32_bf16, keys in the M
// dimension, lane l = lr + 16*lg):
//   S^T (keys x rows) = K . Q^T   QK block b, M row lr <-> key 8(lr/4) + 4b + lr%4
//   O^T (hd x rows)  += V^T . P^T  MFMA j, M row m <-> column 8m + j
// The key order of the QK blocks puts keys 8lg .. 8lg+7 (in order) in the
// result registers of lane (lr, lg) -- the PV B operand for row lr as it
// stands, and the key order of the V registers.  The PV result leaves lane
// (lr, lg) holding row lr's columns 32lg .. 32lg+31.
//
// Softmax: each of the four waves takes 32 consecutive keys of the pass and
// computes its own (max, sum, output) in one step -- the multi-tile kernel's
// running max / running sum of the e4ee9fdc commit log of the pages with one
// slice per wave -- and the four are combined once, in a fixed order,
// through LDS, each wave combining and storing one quarter of the columns
// (whole 128-byte lines of fp32 partials per store instruction, with the
// device-scope cache policy).  Scores are base 2 (x = q.k * scale * log2 e); O is
// normalised by the sum of the bf16-rounded weights the PV product consumes
// and lse uses the fp32 sum, as in attn_kernel.hpp.
#pragma once

#include "device_common.hpp"
#include "mx_quant.hpp"
#include "params.hpp"

namespace fmha {

// STREAM: one row block per KV head -- nobody else reads this workgroup's
// K/V, which is then loaded with the non-temporal hint.  Otherwise the row
// blocks of a KV head share its K/V through L2 (plain loads, units
// regrouped per XCD).
template <int HD, bool SPLIT, bool STREAM>
__global__ __launch_bounds__(256, 4) void stream_kernel(const FwdParams p) {
    static_assert(HD == 128, "the stream kernel serves hd 128: one 16-lane run covers a key row");
    constexpr int KSTEPS = HD / 32;     // QK MFMA steps over the head dim
    constexpr int CHUNKS = HD / 8;      // 16-byte chunks per key row
    constexpr int ROW_BYTES = HD * 2;
    constexpr int WAVE_KEYS = 32;
    constexpr int K_BYTES = 4 * WAVE_KEYS * ROW_BYTES;  // four waves' K slices (32 KiB)
    constexpr int SLOTS = 3 + 32;                       // merge record per lane: m, l, lq, 32 outputs
    constexpr int M_BYTES = 4 * SLOTS * 64 * 4;          // four waves' records (35 KiB)
    // the K slices, then (after every wave's QK) the merge records
    __shared__ __attribute__((aligned(16))) unsigned char smem[M_BYTES > K_BYTES ? M_BYTES : K_BYTES];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lr = lane & 15;
    const int lg = lane >> 4;

    // ---- work unit: row blocks fastest (regrouped per XCD, last block first;
    // streaming work has one), then partitions, KV heads, batch rows --
    // neighbouring workgroups read neighbouring cache rows and write
    // neighbouring partials --------------------------------------------------
    int bid = blockIdx.x;
    if (!STREAM && p.xcd_remap) {
        const int per = p.n_units >> 3;
        bid = (bid & 7) * per + (bid >> 3);
    }
    const int rb = STREAM ? 0 : p.n_row_blocks - 1 - bid % p.n_row_blocks;
    if (!STREAM) bid /= p.n_row_blocks;
    const int part = bid % p.n_split;
    bid /= p.n_split;
    const int kvh = bid % p.n_kv_h;
    const int b = bid / p.n_kv_h;
    const int s_k = p.seqlens ? min(max(p.seqlens[b], 0), p.s_k) : p.s_k;

    const int row0 = 16 * rb;
    const int row_last = min(row0 + 16, p.rows) - 1;
    const int pos_lo = s_k - p.T + row0 / p.group;
    const int pos_hi = s_k - p.T + row_last / p.group;
    int klo = part * p.split_len;
    int khi = min(klo + p.split_len, s_k);
    if (p.causal) khi = min(khi, pos_hi + 1);
    if (p.window > 0) klo = max(klo, pos_lo - p.window + 1);

    const int row = row0 + lr;
    const bool row_ok = row < p.rows;
    const int t_row = row_ok ? row / p.group : 0;
    const int h_row = kvh * p.group + (row_ok ? row % p.group : 0);
    int r_lo, r_hi;  // visible keys of row lr
    {
        const int pos = s_k - p.T + t_row;
        r_hi = p.causal ? min(khi, pos + 1) : khi;
        r_lo = p.window > 0 ? max(klo, pos - p.window + 1) : klo;
        if (!row_ok) r_hi = r_lo;
    }

    const int k0 = klo + WAVE_KEYS * wave;  // this wave's first key
    const bool active = k0 < khi;            // wave-uniform

    // rotation of LDS key row r: chunk c lives in slot (c + rot(r)) % 16, so
    // the 16 rows one QK read touches (keys 8(i/4) + 4b + i%4) use 16
    // different slots -- all the banks
    auto rot_of = [](int r) __attribute__((always_inline)) { return (r + 4 * (r >> 4)) & (CHUNKS - 1); };
    unsigned char *sKw = smem + wave * WAVE_KEYS * ROW_BYTES;

    u32x4 qraw[KSTEPS];  // Q^T B operand: Q[row lr][32s + 8lg .. +7]
    u32x4 vr[8];        // V[key k0 + 8lg + i][8lr .. 8lr + 7]
    if (active) {
        const uint16_t *qp = p.q + (int64_t)b * p.q_sb + (int64_t)t_row * p.q_st + (int64_t)h_row * p.q_sh + 8 * lg;
        // rows past the end read row 0 of the group (valid memory); they are
        // zeroed once loaded
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) qraw[s] = *reinterpret_cast<const u32x4 *>(qp + 32 * s);
        __builtin_amdgcn_sched_barrier(0);
        // K: eight wave-wide loads of four whole key rows each, into the
        // wave's LDS slice (lane L lands at byte 16 L of the load's 1 KiB);
        // keys past the range read key khi - 1 (finite data, weight 0)
        const uint16_t *kbase = p.k + (int64_t)b * p.k_sb + (int64_t)kvh * p.k_sh;
#pragma unroll
        for (int it = 0; it < WAVE_KEYS / 4; ++it) {
            const int r = 4 * it + (lane >> 4);
            const int chunk = (lr - rot_of(r)) & (CHUNKS - 1);
            const int key = min(k0 + r, khi - 1);
            load_lds_16<STREAM>(kbase + key_offset(key, p.k_st) + 8 * chunk, sKw + it * 1024);
        }
        __builtin_amdgcn_sched_barrier(0);  // Q, then K, then V: the waits below count on that order
        // V: eight wave-wide register loads of four whole key rows each
        const uint16_t *vbase = p.v + (int64_t)b * p.v_sb + (int64_t)kvh * p.v_sh + 8 * lr;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int key = min(k0 + 8 * lg + i, khi - 1);
            const u32x4 *vp = reinterpret_cast<const u32x4 *>(vbase + key_offset(key, p.v_st));
            vr[i] = STREAM ? __builtin_nontemporal_load(vp) : *vp;
        }
        __builtin_amdgcn_sched_barrier(0);  // every load issued before the first wait
    }

    float m = -INFINITY, l = 0.f, lq = 0.f;
    f32x4 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (active) {
        // Q and K have landed (V's eight loads, issued last, may still fly)
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(8));
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const unsigned qmask = row_ok ? 0xffffffffu : 0u;
        bf16x8 qf[KSTEPS];
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) qf[s] = __builtin_bit_cast(bf16x8, qraw[s] & qmask);
        f32x4 sc[2];
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            const int r = 8 * (lr >> 2) + 4 * blk + (lr & 3);
            const unsigned char *rowp = sKw + r * ROW_BYTES;
            const int rot = rot_of(r);
            sc[blk] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KSTEPS; ++s) {
                const int slot = (4 * s + lg + rot) & (CHUNKS - 1);
                const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(rowp + 16 * slot);
                sc[blk] = mfma_16x16x32(kf, qf[s], sc[blk]);
            }
        }
        // scores of keys k0 + 8lg + j, j = 0..7: block 0 holds j < 4, block 1 the rest
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int key = k0 + 8 * lg + j;
            const float s = j < 4 ? sc[0][j] : sc[1][j - 4];
            x[j] = (key >= r_lo && key < r_hi) ? s * p.scale_log2 : -INFINITY;
        }
        float mx = x[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) mx = fmaxf(mx, x[j]);
        m = row4_max(mx);
        const float m_use = (m == -INFINITY) ? 0.f : m;
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
        l = psum;
        lq = qsum;
        // V^T operands: element i of MFMA j's operand is V[key 8lg + i][8lr + j];
        // dword u pairs keys 2u, 2u+1 -- the low (j even) or high (j odd)
        // halves of dword j/2 of registers 2u and 2u+1 (v_perm_b32)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const unsigned sel = (j & 1) ? 0x07060302u : 0x05040100u;
            u32x4 a;
#pragma unroll
            for (int u = 0; u < 4; ++u) a[u] = __builtin_amdgcn_perm(vr[2 * u + 1][j >> 1], vr[2 * u][j >> 1], sel);
            acc[j] = mfma_16x16x32(__builtin_bit_cast(bf16x8, a), pt, f32x4{0.f, 0.f, 0.f, 0.f});
        }
    }

    l = row4_sum(l);
    lq = row4_sum(lq);

    // ---- combine the four waves' (m, l, lq, O) and store, by column quarters:
    // every wave publishes its record, then wave w merges columns 32w .. 32w+31
    // of every row in a fixed order (g = 0..3).  Lane (rr, q) = (lane / 8,
    // lane % 8) takes rows rr and rr + 8, columns 32w + 4q .. +3, so each store
    // instruction covers 8 rows x 128 contiguous bytes (fp32 partials: whole
    // cache lines; a lane-local 32-column layout stored directly would leave
    // 16-byte pieces, which measured 23% slower on the split decode)
    __syncthreads();  // every wave is done reading its K slice
    float *red = reinterpret_cast<float *>(smem);
    {
        float *mine = red + wave * SLOTS * 64 + lane;
        mine[0] = m;
        mine[64] = l;
        mine[128] = lq;
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int t = 0; t < 4; ++t) mine[(3 + 4 * j + t) * 64] = acc[j][t];
    }
    __syncthreads();
    const int q = lane & 7;
    const int c = 32 * wave + 4 * q;     // this lane's first column
    const int src_lg = c >> 5;           // source lane group: columns 32 lg .. 32 lg + 31
    const int j0 = c & 7, t0 = (c & 31) >> 3;  // columns c + e sit at acc[j0 + e][t0]
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const int rr = (lane >> 3) + 8 * half;
        const int src = rr + 16 * src_lg;
        float M = -INFINITY;
#pragma unroll
        for (int g = 0; g < 4; ++g) M = fmaxf(M, red[g * SLOTS * 64 + src]);
        const float M_use = (M == -INFINITY) ? 0.f : M;
        float L = 0.f, LQ = 0.f;
        f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const float *rec = red + g * SLOTS * 64 + src;
            const float wgt = fast_exp2(rec[0] - M_use);  // 0 for a wave with no visible key
            L += wgt * rec[64];
            LQ += wgt * rec[128];
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] += wgt * rec[(3 + 4 * (j0 + e) + t0) * 64];
        }
        const int rw = row0 + rr;
        if (rw >= p.rows) continue;
        const int t_o = rw / p.group, h_o = kvh * p.group + rw % p.group;
        const float inv = LQ > 0.f ? 1.f / LQ : 0.f;
        const float lse_val = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
        o = o * inv;
        if constexpr (SPLIT) {
            // rows of this KV head: r0 + ((rw % group) T + rw / group) n_split_total;
            // byte offsets from the first fit 32 bits (the host checks it)
            const int64_t r0 = ((int64_t)b * p.n_h + kvh * p.group) * p.T * p.n_split_total + p.part_offset + part;
            const int64_t dr = ((int64_t)(rw % p.group) * p.T + rw / p.group) * p.n_split_total;
            store16_device_scope(p.o_part + r0 * HD, (unsigned)((dr * HD + c) * 4), o);
            if (wave == 0 && q == 0) p.lse_part[r0 + dr] = lse_val;
        } else {
            if (p.out_format != kOutBf16) {
                // the wave's 32 columns are one MX block, over the 8 lanes of the row
                const int64_t orow = ((int64_t)b * p.T + t_o) * p.n_h + h_o;
                const float v4[4] = {o[0], o[1], o[2], o[3]};
                mx_store_block_8lanes(v4, p.out_format, p.o_codes + orow * (p.out_format == kOutMxFp8E4M3 ? HD : HD / 2),
                                      p.o_scales + orow * (HD / 32), 32 * wave, q);
            } else {
                uint2 packed;
                packed.x = (uint32_t)bf16_bits(o[0]) | ((uint32_t)bf16_bits(o[1]) << 16);
                packed.y = (uint32_t)bf16_bits(o[2]) | ((uint32_t)bf16_bits(o[3]) << 16);
                *reinterpret_cast<uint2 *>(p.o + (int64_t)b * p.o_sb + (int64_t)t_o * p.o_st + (int64_t)h_o * p.o_sh +
                                           c) = packed;
            }
            if (wave == 0 && q == 0 && p.lse != nullptr) p.lse[((int64_t)b * p.n_h + h_o) * p.T + t_o] = lse_val;
        }
    }
}

}  // namespace fmha
