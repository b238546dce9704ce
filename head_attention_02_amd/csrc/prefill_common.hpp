// prefill_common.hpp -- device helpers shared by the matrix-core prefill kernels
// (prefill_bf16.hip, head dim 128; prefill_bf16_narrow.hip, head dims 32 and 64).
#pragma once

#include "mi_attn_device.hpp"
#include "mi_attn_kernels.hpp"
#include "tile_plan.hpp"

namespace mi_attn {

constexpr int kXcds = 8;   // accelerator complex dies (one L2 each) on MI355X

typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ float max3(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

// Row max / sum over both halves of the wave (lanes l and l^32 hold the same query row
// in the S^T = K Q^T accumulator layout of the 32x32 MFMA).
__device__ __forceinline__ float halves_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// One 16-byte-per-lane copy from global memory straight into LDS: lane l reads
// sbase + voff and its 16 bytes land at LDS address m0 + 16 * l (sbase and m0 are
// wave-uniform).  Written as inline assembly so that the compiler does not track it as
// an outstanding LDS write -- it would otherwise wait for every copy in flight
// (vmcnt(0)), including the next tile's, before each LDS read -- and the kernel's own
// vmcnt wait and barrier order the copies against the reads.  The instruction has no
// register result, so nothing of it is left in flight in a register.
__device__ __forceinline__ void lds_dma16(const void* sbase, uint32_t voff, uint32_t m0) {
    asm volatile("global_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(sbase), "{m0}"(m0));
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}

// s_waitcnt vmcnt(0): every global load (tile copies included) of this wave has landed.
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// s_waitcnt vmcnt(N): at most the N vector memory operations this wave issued last are
// still in flight (they complete in issue order, stores included); expcnt and lgkmcnt are
// not waited for.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | 0x0F70);
}

// Marks a rarely taken, wave-uniform branch as having a side effect so that the compiler
// keeps it a branch instead of computing its body on every tile and selecting.
__device__ __forceinline__ void keep_branch() { asm volatile("" ::); }

// Per query row block of 32 rows [r0, r0+32) of one (item, head): this lane's key
// interval, and the keys every / some row of the block sees.  Rows that see no key (a
// position at or past the valid keys, or no query row at all) are written as zeros
// whatever their scores, so `inter` holds the keys every OTHER row of the block sees: a
// tile inside it needs no mask for any row whose output is kept.
struct RowBlockKeys {
    plan::Keys lane;    // this lane's row (empty for a padded row or one past the end)
    plan::Keys inter;   // keys every row of the block that sees a key sees (all keys if none does)
    plan::Keys uni;     // keys some row of the block sees (superset; empty if no row is a query)
};

__device__ __forceinline__ RowBlockKeys row_block_keys(const PrefillArgs& a, int r0, int rows, int my_row,
                                                       int q_len, int valid) {
    RowBlockKeys k;
    const bool causal = a.causal != 0;
    k.lane = plan::row_keys(a.pos_offset + my_row, valid, causal, a.window);
    if (my_row >= q_len) k.lane.hi = -1;
    const int r1 = min(r0 + rows - 1, q_len - 1);
    const int bp_lo = a.pos_offset + r0, bp_hi = a.pos_offset + r1;
    const int bs_hi = min(bp_hi, valid - 1);   // position of the block's last row that sees a key
    k.inter = (r0 < q_len && bs_hi >= bp_lo) ? plan::span_inter(bp_lo, bs_hi, valid, causal, a.window)
                                             : plan::Keys{0, 0x7fffffff};
    k.uni = plan::span_union(bp_lo, bp_hi, valid, causal, a.window);
    if (r0 >= q_len) k.uni.hi = -1;   // no row of the block is a query
    return k;
}

}  // namespace mi_attn
