// stream_kernel.hpp -- one-pass attention at hd 128 (and 64) on gfx950:
// every workgroup's keys fit one pass of NW waves x 32 KS keys (four waves x
// 32: the split-KV decode with 128-key partitions, caches of at most 128
// keys; eight waves x 32 or 64: ranges of up to 256 or 512 keys on grids of
// at most one workgroup per compute unit, such as the MQA decode of 128 query
// heads over one KV head, where a workgroup must take in its whole range --
// the only use at hd 64).
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
//     At hd 64 a lane loads 8 bytes (columns 4m .. 4m+3, still sixteen lanes
//     to a row) and four MFMAs cover columns 4m + j; K rows are 128 bytes,
//     eight to a load.
//
// Products as in attn_kernel.hpp (v_mfma_f32_16x16x32_bf16, keys in the M
// dimension, lane l = lr + 16*lg):
//   S^T (keys x rows) = K . Q^T   QK block b, M row lr <-> key 8(lr/4) + 4b + lr%4
//   O^T (hd x rows)  += V^T . P^T  MFMA j, M row m <-> column (hd/16) m + j
// The key order of the QK blocks puts keys 8lg .. 8lg+7 (in order) in the
// result registers of lane (lr, lg) -- the PV B operand for row lr as it
// stands, and the key order of the V registers.  The PV result leaves lane
// (lr, lg) holding row lr's columns (hd/4) lg .. (hd/4) lg + hd/4 - 1.
//
// Softmax: each wave takes 32 KS consecutive keys of the pass and computes
// its own (max, sum, output) in one step -- the multi-tile kernel's running
// max / running sum of the e4ee9fdc commit log of the pages with one slice
// per wave -- and the NW waves are combined once, in a fixed order, through
// LDS, each wave combining and storing one quarter of the columns of eight
// or sixteen rows at hd 128, four whole rows at hd 64 (whole 128-byte lines
// of fp32 partials per store instruction, with the device-scope cache
// policy).  Scores are base 2 (x = q.k * scale * log2 e); O is
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
// NW waves of 32 KS keys each; four waves per SIMD for up to 32 keys per
// wave (V takes 32 registers), two for 64.
template <int HD, bool SPLIT, bool STREAM, int NW, int KS>
__global__ __launch_bounds__(64 * NW, KS == 1 ? 4 : 2) void stream_kernel(const FwdParams p) {
    static_assert(HD == 64 || HD == 128, "the stream kernel serves hd 64 and 128: one 16-lane run covers a key row");
    static_assert((NW == 4 && KS == 1) || (NW == 8 && (KS == 1 || KS == 2)), "4 x 32, 8 x 32 or 8 x 64 keys");
    constexpr bool H64 = HD == 64;
    constexpr int KSTEPS = HD / 32;     // QK MFMA steps over the head dim
    constexpr int CHUNKS = HD / 8;      // 16-byte chunks per key row
    constexpr int ROW_BYTES = HD * 2;
    constexpr int RPL = 1024 / ROW_BYTES;                // key rows per wave-wide K load
    constexpr int NB = HD / 16;                          // PV MFMAs per 32 keys (16 output columns each)
    constexpr int WAVE_KEYS = 32 * KS;
    constexpr int K_BYTES = NW * WAVE_KEYS * ROW_BYTES;  // every wave's K slice (16 to 128 KiB)
    constexpr int REC = HD / 4 + 4;                      // merge record per lane: HD/4 outputs, m, l, lq, pad
    constexpr int M_BYTES = NW * 64 * REC * 4;           // every wave's records (20 to 72 KiB)
    // the K slices, then (after every wave's QK) the merge records
    __shared__ __attribute__((aligned(16))) unsigned char smem[M_BYTES > K_BYTES ? M_BYTES : K_BYTES];

    fetch_launch_params(p);
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

    // rotation of LDS key row r: chunk c lives in slot (c + rot(r)) % CHUNKS,
    // so the 16 rows one QK read touches (keys 32ks + 8(i/4) + 4b + i%4) use
    // 16 different 16-byte bank groups -- all the banks (hd 64: two 128-byte
    // rows per group of banks, the rotation found by exhaustive search)
    auto rot_of = [](int r) __attribute__((always_inline)) {
        return H64 ? ((r >> 1) ^ (r >> 3)) & (CHUNKS - 1) : (r + 4 * (r >> 4)) & (CHUNKS - 1);
    };
    unsigned char *sKw = smem + wave * WAVE_KEYS * ROW_BYTES;

    u32x4 qraw[KSTEPS];  // Q^T B operand: Q[row lr][32s + 8lg .. +7]
    // V[key k0 + 32ks + 8lg + i][NB lr .. NB lr + NB - 1]: 16 bytes per lane
    // at hd 128, 8 at hd 64 -- sixteen lanes cover a key row either way
    using VRow = typename std::conditional<H64, u32x2, u32x4>::type;
    VRow vr[KS][8];
    // Eight-wave workgroups (one per compute unit: few-unit grids, where a
    // CU's ingest bounds the pass) request V step by step: Q and K first,
    // each 32-key step's QK product as soon as its K has landed, that step's
    // V after it -- the last step's after the softmax -- so the QK and the
    // softmax overlap the V ingest (a wave issues in order, and load issue
    // runs at the CU's ingest rate: with every load ahead of them they waited
    // for the whole pass).  MQA decode hd 128 over 256 / 384 / 512 keys 5.98 /
    // 6.72 / 7.13 -> 5.75 / 6.46 / 6.97 us; hd 64 over 512 keys 5.62 -> 5.54
    // us.  Four-wave workgroups (the split decode, several per CU, bound by
    // HBM) keep every load in flight at once.
    constexpr bool LATE = NW == 8;
    constexpr int KL = 32 / RPL;    // K loads per 32-key step
    auto issue_v = [&](int ks) __attribute__((always_inline)) {
        const int last = khi - 1 - k0;
        const uint16_t *vw = p.v + (int64_t)b * p.v_sb + (int64_t)kvh * p.v_sh + key_offset(k0, p.v_st);
        const unsigned vstride = (unsigned)p.v_st * 2u;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const unsigned off = (unsigned)min(32 * ks + 8 * lg + i, last) * vstride + 2u * NB * lr;
            if constexpr (H64) vr[ks][i] = load8_buf<STREAM>(vw, off);
            else vr[ks][i] = load16_buf<STREAM>(vw, off);
        }
    };
    if (active) {
        const uint16_t *qp = p.q + (int64_t)b * p.q_sb + (int64_t)t_row * p.q_st + (int64_t)h_row * p.q_sh + 8 * lg;
        // rows past the end read row 0 of the group (valid memory); they are
        // zeroed once loaded
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) qraw[s] = *reinterpret_cast<const u32x4 *>(qp + 32 * s);
        __builtin_amdgcn_sched_barrier(0);
        // K and V by buffer loads from the wave's first key row: a lane's
        // byte offset is its row (clamped to the last key of the range:
        // rows past it reread that key -- finite data, weight 0) times the
        // token stride, one 32-bit multiply-add per load (the host keeps a
        // wave's rows within 2^31 bytes)
        const int last = khi - 1 - k0;  // >= 0: the wave is active
        const uint16_t *kw = p.k + (int64_t)b * p.k_sb + (int64_t)kvh * p.k_sh + key_offset(k0, p.k_st);
        const uint16_t *vw = p.v + (int64_t)b * p.v_sb + (int64_t)kvh * p.v_sh + key_offset(k0, p.v_st);
        const unsigned kstride = (unsigned)p.k_st * 2u, vstride = (unsigned)p.v_st * 2u;
        // K: wave-wide loads of RPL whole key rows each (4 at hd 128, 8 at
        // hd 64), into the wave's LDS slice (lane L lands at byte 16 L of the
        // load's 1 KiB)
#pragma unroll
        for (int it = 0; it < WAVE_KEYS / RPL; ++it) {
            const int r = RPL * it + lane / CHUNKS;
            const int chunk = (lane % CHUNKS - rot_of(r)) & (CHUNKS - 1);
            load_lds_buf<STREAM>(kw, (unsigned)min(r, last) * kstride + 16u * chunk, sKw + it * 1024);
        }
        __builtin_amdgcn_sched_barrier(0);  // Q, then K, then V: the waits below count on that order
        if constexpr (!LATE) {
            // V: 8 KS wave-wide register loads of four whole key rows each
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const unsigned off = (unsigned)min(32 * ks + 8 * lg + i, last) * vstride + 2u * NB * lr;
                    if constexpr (H64) vr[ks][i] = load8_buf<STREAM>(vw, off);
                    else vr[ks][i] = load16_buf<STREAM>(vw, off);
                }
            __builtin_amdgcn_sched_barrier(0);  // every load issued before the first wait
        }
    }

    float m = -INFINITY, l = 0.f, lq = 0.f;
    f32x4 acc[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (active) {
      const unsigned qmask = row_ok ? 0xffffffffu : 0u;
      bf16x8 qf[KSTEPS];
      f32x4 sc[KS][2];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) sc[ks][0] = sc[ks][1] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (LATE) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            // Q and this step's K have landed (the next step's K, or this
            // wave's first V loads, may still fly)
            if (ks == 0) __builtin_amdgcn_s_waitcnt(waitcnt_vm((KS - 1) * KL));
            else __builtin_amdgcn_s_waitcnt(waitcnt_vm(8));
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            __builtin_amdgcn_sched_barrier(0);
            if (ks == 0) {
#pragma unroll
                for (int s = 0; s < KSTEPS; ++s) qf[s] = __builtin_bit_cast(bf16x8, qraw[s] & qmask);
            }
            bf16x8 kf[KSTEPS][2];
#pragma unroll
            for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
                for (int blk = 0; blk < 2; ++blk) {
                    const int r = 32 * ks + 8 * (lr >> 2) + 4 * blk + (lr & 3);
                    const int slot = (4 * s + lg + rot_of(r)) & (CHUNKS - 1);
                    kf[s][blk] = *reinterpret_cast<const bf16x8 *>(sKw + r * ROW_BYTES + 16 * slot);
                }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
                for (int blk = 0; blk < 2; ++blk) sc[ks][blk] = mfma_16x16x32(kf[s][blk], qf[s], sc[ks][blk]);
            __builtin_amdgcn_sched_barrier(0);
            if (KS == 1 || ks + 1 < KS) issue_v(ks);
            __builtin_amdgcn_sched_barrier(0);
        }
      } else {
        // Q and K have landed (V's 8 KS loads, issued last, may still fly)
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(8 * KS));
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) qf[s] = __builtin_bit_cast(bf16x8, qraw[s] & qmask);
        // every K operand read is issued before the first MFMA (a read waited
        // for right before its MFMA costs a full LDS round trip each); the
        // MFMAs then alternate between the 2 KS independent accumulators
        bf16x8 kf[KSTEPS][KS][2];
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int blk = 0; blk < 2; ++blk) {
                    const int r = 32 * ks + 8 * (lr >> 2) + 4 * blk + (lr & 3);
                    const int slot = (4 * s + lg + rot_of(r)) & (CHUNKS - 1);
                    kf[s][ks][blk] = *reinterpret_cast<const bf16x8 *>(sKw + r * ROW_BYTES + 16 * slot);
                }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int blk = 0; blk < 2; ++blk) sc[ks][blk] = mfma_16x16x32(kf[s][ks][blk], qf[s], sc[ks][blk]);
      }
        // scores of keys k0 + 32ks + 8lg + j, j = 0..7: block 0 holds j < 4,
        // block 1 the rest
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
        m = row4_max(mx);
        const float m_use = (m == -INFINITY) ? 0.f : m;
        bf16x8 pt[KS];
        float psum = 0.f, qsum = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float pj = fast_exp2(x[ks][j] - m_use);
                const __bf16 pb = to_bf16(pj);
                pt[ks][j] = pb;
                psum += pj;
                qsum += (float)pb;
            }
        l = psum;
        lq = qsum;
        if constexpr (LATE) {
            if (KS > 1) issue_v(KS - 1);
        }
        // V^T operands: element i of MFMA j's operand is V[key 32ks + 8lg + i][NB lr + j];
        // dword u pairs keys 2u, 2u+1 -- the low (j even) or high (j odd)
        // halves of dword j/2 of registers 2u and 2u+1 (v_perm_b32)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (LATE && KS > 1) {  // step 0's V ahead of the last step's, issued last
                if (ks == 0) __builtin_amdgcn_s_waitcnt(waitcnt_vm(8));
                else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const unsigned sel = (j & 1) ? 0x07060302u : 0x05040100u;
                u32x4 a;
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    a[u] = __builtin_amdgcn_perm(vr[ks][2 * u + 1][j >> 1], vr[ks][2 * u][j >> 1], sel);
                acc[j] = mfma_16x16x32(__builtin_bit_cast(bf16x8, a), pt[ks],
                                       ks == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[j]);
            }
            if (LATE && KS > 1) __builtin_amdgcn_sched_barrier(0);
        }
    }

    l = row4_sum(l);
    lq = row4_sum(lq);

    // ---- combine the NW waves' (m, l, lq, O) and store, by column quarters:
    // every wave publishes its record, then wave w merges columns 32cb ..
    // 32cb + 31 (cb = w % 4) of its rows in a fixed order (g = 0 .. NW-1).
    // Lane (rr, q) = (lane / 8, lane % 8) takes columns 32cb + 4q .. +3 of
    // rows rr and rr + 8 (four waves) or of row rr + 8 (w / 4) (eight), so
    // each store instruction covers 8 rows x 128 contiguous bytes (fp32
    // partials: whole cache lines; a lane-local 32-column layout stored
    // directly would leave 16-byte pieces, which measured 23% slower on the
    // split decode).  Records are lane-major -- lane (lr, lg)'s 32 columns
    // 32lg .. 32lg + 31 of row lr in order, then (m, l, lq) -- so a combine
    // read of four columns or of (m, l, lq) is one 16-byte read, and the 8
    // lanes of a row read 128 contiguous bytes (a slot-major layout put all
    // of a record in one bank: 8-way conflicts)
    // At hd 64 a row's 64 columns are 256 bytes of fp32 partials: wave w < 4
    // merges rows 4w .. 4w + 3, all columns, lane (rr, q) = (lane / 16, lane %
    // 16) taking columns 4q .. 4q + 3 of row 4w + rr (the other four waves of
    // an eight-wave workgroup have no part in it).
    const int q = H64 ? lane & 15 : lane & 7;
    const int cb = wave & 3;                      // column quarter (hd 128)
    const int c = H64 ? 4 * q : 32 * cb + 4 * q;  // this lane's first column
    constexpr int HALVES = (NW == 4 && !H64) ? 2 : 1;
    const bool merges = !H64 || wave < 4;         // wave-uniform
    // output addressing of this lane's rows, fixed before the barriers
    int rows_rr[HALVES];
    int64_t o_off[HALVES], l_off[HALVES];
#pragma unroll
    for (int hh = 0; hh < HALVES; ++hh) {
        const int half = NW == 4 ? hh : (wave >> 2);
        const int rr = H64 ? 4 * cb + (lane >> 4) : (lane >> 3) + 8 * half;
        rows_rr[hh] = rr;
        const int rw = row0 + rr;
        const int rwc = rw < p.rows ? rw : row0;
        const int t_o = rwc / p.group, g_o = rwc % p.group, h_o = kvh * p.group + g_o;
        if constexpr (SPLIT) {
            // partial rows of this KV head: r0 + (g_o T + t_o) n_split_total
            o_off[hh] = ((int64_t)g_o * p.T + t_o) * p.n_split_total;
            l_off[hh] = o_off[hh];
        } else {
            o_off[hh] = p.out_format != kOutBf16 ? ((int64_t)b * p.T + t_o) * p.n_h + h_o
                                                 : (int64_t)b * p.o_sb + (int64_t)t_o * p.o_st + (int64_t)h_o * p.o_sh;
            l_off[hh] = ((int64_t)b * p.n_h + h_o) * p.T + t_o;
        }
    }
    __syncthreads();  // every wave is done reading its K slice
    float *red = reinterpret_cast<float *>(smem);
    {
        float *mine = red + (wave * 64 + lane) * REC;
        // lane (lr, lg) holds columns NB (4 lg + t) + j of row lr (MFMA j,
        // element t): HD/4 consecutive columns, stored in order
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int h = 0; h < NB / 4; ++h)
                *reinterpret_cast<f32x4 *>(mine + NB * t + 4 * h) =
                    f32x4{acc[4 * h][t], acc[4 * h + 1][t], acc[4 * h + 2][t], acc[4 * h + 3][t]};
        *reinterpret_cast<f32x4 *>(mine + HD / 4) = f32x4{m, l, lq, 0.f};
    }
    __syncthreads();
    if (!merges) return;
#pragma unroll
    for (int hh = 0; hh < HALVES; ++hh) {
        const int rr = rows_rr[hh];
        // the record of lane (rr, column group) of wave g: + g * 64 * REC
        const float *src = red + (rr + 16 * (H64 ? q >> 2 : cb)) * REC;
        const int val_off = H64 ? 4 * (q & 3) : 4 * q;
        f32x4 rec[NW], val[NW];
#pragma unroll
        for (int g = 0; g < NW; ++g) {
            rec[g] = *reinterpret_cast<const f32x4 *>(src + g * 64 * REC + HD / 4);
            val[g] = *reinterpret_cast<const f32x4 *>(src + g * 64 * REC + val_off);
        }
        float M = -INFINITY;
#pragma unroll
        for (int g = 0; g < NW; ++g) M = fmaxf(M, rec[g][0]);
        const float M_use = (M == -INFINITY) ? 0.f : M;
        float L = 0.f, LQ = 0.f;
        f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int g = 0; g < NW; ++g) {
            const float wgt = fast_exp2(rec[g][0] - M_use);  // 0 for a wave with no visible key
            L += wgt * rec[g][1];
            LQ += wgt * rec[g][2];
            o += wgt * val[g];
        }
        if (row0 + rr >= p.rows) continue;
        const float inv = LQ > 0.f ? 1.f / LQ : 0.f;
        const float lse_val = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
        o = o * inv;
        const bool lse_lane = q == 0 && (H64 || cb == 0);
        if constexpr (SPLIT) {
            // byte offsets from the KV head's first partial row fit 32 bits
            // (the host checks it)
            const int64_t r0 = ((int64_t)b * p.n_h + kvh * p.group) * p.T * p.n_split_total + p.part_offset + part;
            store16_device_scope(p.o_part + r0 * HD, (unsigned)((o_off[hh] * HD + c) * 4), o);
            if (lse_lane) p.lse_part[r0 + l_off[hh]] = lse_val;
        } else {
            if (p.out_format != kOutBf16) {
                // 32-column MX blocks over 8 adjacent lanes of the row (hd
                // 128: the wave's 32 columns; hd 64: two blocks per row)
                const int64_t orow = o_off[hh];
                const float v4[4] = {o[0], o[1], o[2], o[3]};
                mx_store_block_8lanes(v4, p.out_format, p.o_codes + orow * (p.out_format == kOutMxFp8E4M3 ? HD : HD / 2),
                                      p.o_scales + orow * (HD / 32), H64 ? 32 * (q >> 3) : 32 * cb, q & 7);
            } else {
                uint2 packed;
                packed.x = (uint32_t)bf16_bits(o[0]) | ((uint32_t)bf16_bits(o[1]) << 16);
                packed.y = (uint32_t)bf16_bits(o[2]) | ((uint32_t)bf16_bits(o[3]) << 16);
                *reinterpret_cast<uint2 *>(p.o + o_off[hh] + c) = packed;
            }
            if (lse_lane && p.lse != nullptr) p.lse[l_off[hh]] = lse_val;
        }
    }
}

}  // namespace fmha
