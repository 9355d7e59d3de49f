// params.hpp -- launch parameters of the attention kernels.
#pragma once

#include <stdint.h>

namespace fmha {

struct FwdParams {
    const uint16_t *q, *k, *v;
    uint16_t *o;      // forward mode: bf16 output (strided)
    float *lse;       // forward mode: [b][n_h][T], may be null
    float *o_part;    // split mode: [b][n_h][T][n_split][hd]
    float *lse_part;  // split mode: [b][n_h][T][n_split]
    int64_t q_sb, q_st, q_sh;
    int64_t k_sb, k_st, k_sh;
    int64_t v_sb, v_st, v_sh;
    int64_t o_sb, o_st, o_sh;
    int batch, n_h, n_kv_h, T, s_k;
    int group;        // n_h / n_kv_h
    int rows;         // group * T rows per (batch, kv_head)
    int window, causal;
    int split_len, n_split;
    const int *seqlens;  // device [batch] keys per batch row (ragged batch), or null: s_k for all
    int part_offset;     // split mode: first partition slot this call writes
    int n_split_total;   // split mode: partition slots per row in o_part / lse_part
    int n_row_blocks;
    int n_units;      // gridDim.x
    int xcd_remap;    // 1: n_units % 8 == 0, give each XCD a contiguous unit range
    float scale_log2; // scale * log2(e)
    int out_format;   // forward mode: OutFormat (bf16 o, or MX codes + scales)
    uint8_t *o_codes;  // MX: [b][T][n_h][hd] E4M3 or [..][hd / 2] E2M1 pairs, dense
    uint8_t *o_scales; // MX: [b][T][n_h][hd / 32] E8M0, dense
};

}  // namespace fmha
