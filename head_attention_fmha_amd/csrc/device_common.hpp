// device_common.hpp -- small gfx950 building blocks shared by the fmha kernels.
//
// MFMA register layouts used throughout (v_mfma_f32_16x16x32_bf16, wave64):
//   lane l = lr + 16*lg   (lr = l % 16, lg = l / 16)
//   A (16 x 32):  lane l holds A[lr][8*lg + 0..7]        (8 bf16, one row)
//   B (32 x 16):  lane l holds B[8*lg + 0..7][lr]        (8 bf16, one column)
//   D (16 x 16):  lane l holds D[4*lg + 0..3][lr]        (4 fp32)
// A and B index their reduction dimension through the same (lg, item)
// pairs, so any permutation of that dimension applied to both operands
// leaves the product unchanged; the kernels use this to feed softmax
// probabilities straight from one MFMA's result registers into the next.
#pragma once

#include <hip/hip_runtime.h>
#include <float.h>
#include <stdint.h>

namespace fmha {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef unsigned u32x4 __attribute__((__vector_size__(4 * sizeof(unsigned))));
typedef unsigned u32x2 __attribute__((__vector_size__(2 * sizeof(unsigned))));
typedef __bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));

constexpr float kLog2e = 1.4426950408889634f;
// Lazy online softmax: the running maximum moves only when a score exceeds
// it by more than this (base-2 units), so weights stay below 2^8, far inside
// bf16 and fp32 range.
constexpr float kRescaleLog2 = 8.f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x4 mfma_16x16x32(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 2^x on the transcendental unit (v_exp_f32); 2^-inf = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Butterfly over lanes l ^ mask (wave64; every lane participates).
__device__ __forceinline__ float xor_shuffle(float x, int mask) {
    const int lane = __lane_id();
    return __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, __float_as_int(x)));
}

// Max / sum over the four lanes lr + 16*lg (lg = 0..3) that hold one row of
// an MFMA result, on the VALU.  v_permlane16_swap exchanges the odd 16-lane
// rows of one register with the even rows of another, v_permlane32_swap the
// upper 32 lanes of one with the lower 32 of another; handed the same value
// twice, each leaves lane l holding its own value and that of lane l ^ 16
// (resp. l ^ 32) in its two results.  Both operations are commutative, so
// the four lanes end with identical bits.
__device__ __forceinline__ float row4_max(float x) {
    const unsigned u = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const unsigned v = __float_as_uint(y);
    const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float row4_sum(float x) {
    const unsigned u = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const unsigned v = __float_as_uint(y);
    const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Element offset of key row `key` (>= 0) for a K/V token stride below 2^32
// (the host rejects larger ones): a single 32 x 32 -> 64-bit multiply.
__device__ __forceinline__ int64_t key_offset(int key, int64_t stride) {
    return (int64_t)((uint64_t)(uint32_t)key * (uint64_t)(uint32_t)stride);
}

// Every launch parameter a forward kernel's prologue reads, requested in one
// batch of scalar loads.  Left to itself the compiler fetches each field
// where it is first used, and the prologue then waits for several dependent
// rounds of kernel-argument loads before the first K/V load can be issued
// (0.2-0.4 us of a few-microsecond launch, measured on the MQA decode).
template <class Params>
__device__ __forceinline__ void fetch_launch_params(const Params &p) {
    asm volatile("" ::"s"(p.q), "s"(p.k), "s"(p.v), "s"(p.q_sb), "s"(p.q_st), "s"(p.q_sh), "s"(p.k_sb),
                 "s"(p.k_st), "s"(p.k_sh), "s"(p.v_sb), "s"(p.v_st), "s"(p.v_sh), "s"(p.n_split), "s"(p.n_kv_h),
                 "s"(p.n_row_blocks), "s"(p.xcd_remap), "s"(p.n_units), "s"(p.s_k), "s"(p.T), "s"(p.rows),
                 "s"(p.group), "s"(p.causal), "s"(p.window), "s"(p.split_len), "s"(p.seqlens));
}

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// 6:4, lgkmcnt 11:8; a field at its maximum does not wait).
constexpr int waitcnt_vm(int n) { return (n & 15) | (((n >> 4) & 3) << 14) | (7 << 4) | (15 << 8); }
constexpr int kWaitLgkm0 = 15 | (3 << 14) | (7 << 4);

// 16 bytes per lane straight from global memory into LDS
// (global_load_lds_dwordx4): lane L's data lands at lds_base + 16*L.  The
// LDS write completes asynchronously and is tracked by vmcnt, not by the
// compiler: wait with s_waitcnt vmcnt before reading the destination.
// NT: non-temporal hint (the nt cache-policy bit) for data that no other
// workgroup will read again, so it does not displace data that will be.
template <bool NT = false>
__device__ __forceinline__ void load_lds_16(const void *gptr, void *lds_base) {
    __builtin_amdgcn_global_load_lds(gptr, (__attribute__((address_space(3))) void *)lds_base, 16, 0, NT ? 2 : 0);
}

// 16 bytes per lane into LDS by a buffer load (buffer_load_dwordx4 ... lds):
// lane L copies the 16 bytes at base + voffset(L) to lds_base + 16L, with
// base wave-uniform (a buffer resource in scalar registers) and voffset the
// lane's byte offset from it (below 2^31).  Like load_lds_16 it completes
// asynchronously and is tracked by vmcnt.  Unlike the global form, which the
// compiler counts as a possible LDS access of a flat instruction -- after
// which it can only wait for all LDS reads at once (lgkmcnt(0)) -- the
// buffer form leaves the compiler's waits for LDS reads exact, so reads
// issued ahead of their use stay in flight.  Raw buffer, 32-bit data format,
// range check off (records = 2^32 - 1).
template <bool NT = false>
__device__ __forceinline__ void load_lds_buf(const void *base, unsigned voffset, void *lds_base) {
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, -1, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void *)lds_base, 16,
                                             voffset, 0, 0, NT ? 2 : 0);
}

// 16 bytes per lane into registers by a buffer load: base wave-uniform,
// voffset the lane's byte offset from it (below 2^31); NT as above.  Lanes
// then address rows by one 32-bit multiply-add instead of 64-bit pointer
// arithmetic per load.
template <bool NT = false>
__device__ __forceinline__ u32x4 load16_buf(const void *base, unsigned voffset) {
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, -1, 0x00020000);
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, voffset, 0, NT ? 2 : 0));
}

// 8 bytes per lane into registers by a buffer load, as load16_buf.
template <bool NT = false>
__device__ __forceinline__ u32x2 load8_buf(const void *base, unsigned voffset) {
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, -1, 0x00020000);
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rsrc, voffset, 0, NT ? 2 : 0));
}

// 16 bytes per lane stored by a buffer store with the device-scope cache
// policy (sc1): base wave-uniform (a buffer resource in scalar registers),
// voffset the lane's byte offset from it (below 2^31).  For the split
// decode's fp32 partials -- written once, read by the merge launch that
// follows -- this policy measured faster than plain or non-temporal stores
// (the GQA decode workload: split 178 -> 173 us, split + merge 194 -> 186 us).
__device__ __forceinline__ void store16_device_scope(void *base, unsigned voffset, const f32x4 &v) {
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(base, (short)0, -1, 0x00020000);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rsrc, voffset, 0, 16);
}

// Workgroup barrier for LDS staged by global_load_lds.  The caller has
// already waited (vmcnt) for its own LDS-direct loads that others will read;
// this waits for the wave's LDS reads and writes, then meets the other
// waves.  A memory fence here would also wait for every global load in
// flight -- the next chunk's prefetch -- as __syncthreads() does, because
// LDS-direct loads count as LDS writes.  The signal fences keep the compiler
// from moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ __bf16 to_bf16(float x) { return (__bf16)x; }

__device__ __forceinline__ uint16_t bf16_bits(float x) {
    __bf16 b = (__bf16)x;
    return __builtin_bit_cast(uint16_t, b);
}

}  // namespace fmha
