// sa_device.h -- device-side helpers shared by the gfx950 kernels of libsparse_attn.
//
// Vector types for MFMA operands, bf16 bit conversions, the direct global->LDS
// copy (one 16-byte chunk per lane) and the explicit wait/barrier primitives the
// gather pipeline relies on; one host-side size check.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));

#define SA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two f32 -> packed pair of bf16 (low half = a), round to nearest even: one
// gfx950 v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// Rotation of one adjacent pair (a, b) of bf16 values, packed with a in the low
// half, as the complex number a + i b times c + i sn (times c - i sn when
// inverse) in f32 -- each real product rounded, then the sum (no fused
// multiply-add) -- rounded back to bf16.
//   forward: (a c - b sn, a sn + b c)     inverse: (a c + b sn, b c - a sn)
__device__ __forceinline__ uint32_t rope_pair(uint32_t pk, float c, float sn, bool inverse) {
#pragma clang fp contract(off)
    const float a = __uint_as_float(pk << 16), b = __uint_as_float(pk & 0xffff0000u);
    const float ac = a * c, bs = b * sn, as = a * sn, bc = b * c;
    const float re = inverse ? ac + bs : ac - bs;
    const float im = inverse ? bc - as : as + bc;
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{re, im}, bf16x2_t));
}

__device__ __forceinline__ uint32_t lds_addr(const SA_LDS void *p) {
    return (uint32_t)(uintptr_t)p;
}

// Direct global -> LDS copy of one 16-byte chunk per lane (gfx950
// global_load_lds_dwordx4).  The wave's 64 chunks land contiguously at the
// wave-uniform LDS byte address `lds_base` (lane i at lds_base + 16 i).  Issued
// through inline asm so that the compiler adds no waits of its own; completion
// is tracked by the caller with wait_vmcnt_barrier().
//
// The copy takes its LDS address from M0.  On gfx950 an LDS DMA that follows
// an SALU write of M0 with no wait state in between can read the previous M0
// (the compiler puts an s_nop 0 there for its own global_load_lds), which
// would land the row in the previous copy's slot; the asm keeps that wait
// state itself, since the compiler cannot see into it.
__device__ __forceinline__ void dma_16B(const void *src, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "s"(lds_base)
                 : "memory", "m0");
}

// The same copy with the non-temporal hint, for data read once (a query's head
// rows, its index list): it is kept from displacing the latent rows that many
// workgroups of an XCD share in its L2.
__device__ __forceinline__ void dma_16B_nt(const void *src, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
                 :
                 : "v"(src), "s"(lds_base)
                 : "memory", "m0");
}

// Direct global -> LDS copy of one 4-byte value per lane (gfx950
// global_load_lds_dword): lane i's value lands at lds_base + 4 i (inactive lanes
// write nothing), with the non-temporal hint (index lists are read once).
// Completion is tracked by the caller's vmcnt waits; the M0 wait state as in
// dma_16B.
__device__ __forceinline__ void dma_4B(const void *src, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off nt"
                 :
                 : "v"(src), "s"(lds_base)
                 : "memory", "m0");
}

// Partial waits.  s_waitcnt vmcnt(N) returns once at most N of this wave's
// vector-memory operations are outstanding.  A wave's loads, these copies
// included, complete in the order it issued them, so while a copy is
// outstanding every load issued after it is too: if the wave issued at least N
// loads or copies after the ones it needs, vmcnt(N) returns only when those
// are done.  Stores do not count toward N: one may complete ahead of earlier
// loads, but while the needed copy is outstanding the N loads behind it keep
// the count above N; extra loads in between (the compiler's own) only make the
// wait longer.  Every partial wait in the kernels names the copies issued
// behind the ones it waits for; each is one instruction of the whole wave,
// issued with at least one lane active (an instruction with none may be
// skipped by an exec branch and then does not count).  The compiler's waits for
// its own loads count only its own operations, so a copy issued after one of
// its loads only lengthens them.
//
// Wait until at most N vector-memory operations of this wave are outstanding,
// then barrier the workgroup (all LDS writes of completed copies visible).
template <int N>
__device__ __forceinline__ void wait_vmcnt_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" : : "n"(N) : "memory");
}

// Wait for all of this wave's memory operations (copies into LDS and LDS
// writes), then barrier the workgroup.
__device__ __forceinline__ void wait_all_barrier() {
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" : : : "memory");
}

// Wait for this wave's LDS operations, then barrier the workgroup.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
}

// 16-byte store of a result read by no later workgroup, with the
// non-temporal hint (streamed out without displacing shared rows in L2)
__device__ __forceinline__ void store_16B_nt(void *dst, u32x4_t v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t *>(dst));
}

__device__ __forceinline__ float shfl_xor_f32(float v, int mask) {
    return __shfl_xor(v, mask, 64);
}

// Host-side size check: a * b <= limit for non-negative a, b, without forming a
// product that could overflow (entry points reject sizes past it before any launch).
inline bool mul_le(int64_t a, int64_t b, int64_t limit) { return a == 0 || b <= limit / a; }

}  // namespace sa
