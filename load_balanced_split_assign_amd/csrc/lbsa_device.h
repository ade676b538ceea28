// Device helpers shared by the attention kernels of liblbsa.so (decode split /
// static / combine and prefill): vector types, LDS address arithmetic,
// asynchronous global->LDS loads, explicit wait counts, and the asm LDS reads
// whose completion the caller controls.
#pragma once

#include "lbsa_internal.h"

namespace lbsa {
namespace dev {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) float lds_float;

constexpr int kWaves = kSplitThreads / 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

__device__ inline float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ inline uint4 lds_load16(const lds_char* p) {
    return __builtin_bit_cast(uint4, *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(p));
}
__device__ inline void lds_store16(lds_char* p, uint4 v) {
    *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(p) = __builtin_bit_cast(u32x4, v);
}
__device__ inline uint32_t lds_addr(const lds_char* p) { return (uint32_t)(size_t)p; }

// 16-byte chunk swizzle of a bf16 V row (16 chunks) inside its 16-row slice,
// for the transposed reads of V^T (ds_read_b64_tr_b16).  One pass of such a
// read covers 8 rows (4 g + r / 4 for g = 0, 1, or g = 2, 3), each row's
// lanes reading one aligned 32-byte chunk pair; this swizzle puts the 8 rows'
// pairs on 8 different 32-byte bank groups, so the pass has no bank conflict
// (chunk ^ row would pair rows 2k and 2k + 1 on the same banks).
__device__ inline int swz_v(int row) { return ((row << 1) & 14) | ((row >> 3) & 1); }

// Two floats -> two bf16 (round to nearest even) in one dword through one
// packed convert (v_cvt_pk_bf16_f32), low half first.
typedef float f32x2_v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
__device__ inline uint32_t bf16x2_pack(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_v){lo, hi}, bf16x2_v));
}

__device__ inline uint32_t bf16x2_bits(float lo, float hi) {
    __bf16 a = (__bf16)lo, b = (__bf16)hi;          // round to nearest even
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// 4 e4m3fn codes (one dword) -> 4 bf16 (two dwords); exact, since every e4m3
// value has at most 4 significant bits.  Two packed converts (bytes 0-1 and
// 2-3 to fp32 pairs) and two byte permutes keeping the upper halves.  The
// converts are written as asm: through the builtin, this toolchain
// miscompiled the use of the pair's second element (it read element 0 twice).
__device__ inline uint2 fp8x4_to_bf16x4(uint32_t w) {
    uint64_t lo, hi;
    __asm__("v_cvt_pk_f32_fp8_e32 %0, %2\n\t"
            "v_cvt_pk_f32_fp8_sdwa %1, %2 src0_sel:WORD_1"
            : "=&v"(lo), "=&v"(hi)
            : "v"(w));
    uint2 r;
    r.x = __builtin_amdgcn_perm((uint32_t)(lo >> 32), (uint32_t)lo, 0x07060302u);   // {e0.hi16, e1.hi16}
    r.y = __builtin_amdgcn_perm((uint32_t)(hi >> 32), (uint32_t)hi, 0x07060302u);
    return r;
}

// 8 e4m3 codes (two dwords) -> 8 bf16 (16 bytes).
__device__ inline uint4 fp8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
    uint2 a = fp8x4_to_bf16x4(w0), b = fp8x4_to_bf16x4(w1);
    return make_uint4(a.x, a.y, b.x, b.y);
}

__device__ inline bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

// Uniform (scalar-cache) view of read-only metadata: page table, task map,
// lengths.  Loads through it with a wave-uniform address become s_load.
template <typename T>
__device__ inline const __attribute__((address_space(4))) T* uniform_ptr(const void* p) {
    return (const __attribute__((address_space(4))) T*)(p);
}

// s_waitcnt vmcnt(N) with the LDS and export counters left unconstrained,
// fenced for the compiler so no LDS access moves above it.
template <int N>
__device__ inline void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit field");
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
    __asm__ volatile("" ::: "memory");
}

// Workgroup barrier for LDS exchange only.  __syncthreads() also fences
// global memory, which would wait for every asynchronous load in flight; the
// merge only needs this wave's LDS writes done (lgkmcnt(0)) before s_barrier.
__device__ inline void lds_barrier() {
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));   // lgkmcnt(0), vmcnt(63)
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
}

// Asynchronous global -> LDS loads: lane i's 16 (or 4) bytes land at
// lds + 16 i (or 4 i).  Non-template wrappers keep the target builtin out of
// dependent (template) contexts.
__device__ inline void dma16(const void* g, lds_char* l) {
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)l, 16, 0, 0);
}
__device__ inline void dma4(const void* g, lds_char* l) {
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)l, 4, 0, 0);
}
// The same with the non-temporal hint (cache policy NT): for data read once,
// such as a decode step's K/V pages.  A global->LDS stream of 512 MiB reads at
// about 6.9 TB/s with it against 6.0 TB/s without, on MI355X.
__device__ inline void dma16_nt(const void* g, lds_char* l) {
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)l, 16, 0, 2);
}
__device__ inline void dma4_nt(const void* g, lds_char* l) {
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)l, 4, 0, 2);
}

// LDS accesses to the ring are written as small asm blocks that complete
// before returning (s_waitcnt lgkmcnt(0)).  The compiler does not see them as
// LDS accesses, so it adds no wait of its own for the asynchronous loads in
// flight (its alias reasoning about those loads is conservative and falls
// back to waiting for all of them); their ordering after the loads is the
// caller's explicit vmcnt wait, and the memory clobbers keep program order.
//
// The 8 transposed V reads of one tile (one per 16-wide d block).
__device__ inline void vt_read8(s16x4 (&va)[8], const uint32_t (&addr)[8]) {
    typedef short s16x4_v __attribute__((ext_vector_type(4)));
    s16x4_v o0, o1, o2, o3, o4, o5, o6, o7;
    __asm__ volatile(
        "ds_read_b64_tr_b16 %0, %8\n\t"
        "ds_read_b64_tr_b16 %1, %9\n\t"
        "ds_read_b64_tr_b16 %2, %10\n\t"
        "ds_read_b64_tr_b16 %3, %11\n\t"
        "ds_read_b64_tr_b16 %4, %12\n\t"
        "ds_read_b64_tr_b16 %5, %13\n\t"
        "ds_read_b64_tr_b16 %6, %14\n\t"
        "ds_read_b64_tr_b16 %7, %15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(o0), "=&v"(o1), "=&v"(o2), "=&v"(o3), "=&v"(o4), "=&v"(o5), "=&v"(o6), "=&v"(o7)
        : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3]), "v"(addr[4]), "v"(addr[5]), "v"(addr[6]),
          "v"(addr[7])
        : "memory");
    va[0] = __builtin_bit_cast(s16x4, o0);
    va[1] = __builtin_bit_cast(s16x4, o1);
    va[2] = __builtin_bit_cast(s16x4, o2);
    va[3] = __builtin_bit_cast(s16x4, o3);
    va[4] = __builtin_bit_cast(s16x4, o4);
    va[5] = __builtin_bit_cast(s16x4, o5);
    va[6] = __builtin_bit_cast(s16x4, o6);
    va[7] = __builtin_bit_cast(s16x4, o7);
}

// Two 16-byte LDS reads completed before returning.
__device__ inline void lds_read2x16(uint4& x, uint4& y, uint32_t ax, uint32_t ay) {
    u32x4 ox, oy;
    __asm__ volatile(
        "ds_read_b128 %0, %2\n\t"
        "ds_read_b128 %1, %3\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(ox), "=&v"(oy)
        : "v"(ax), "v"(ay)
        : "memory");
    x = __builtin_bit_cast(uint4, ox);
    y = __builtin_bit_cast(uint4, oy);
}

// Four 16-byte LDS reads completed before returning.
__device__ inline void lds_read4x16(uint4 (&o)[4], const uint32_t (&addr)[4]) {
    u32x4 o0, o1, o2, o3;
    __asm__ volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %5\n\t"
        "ds_read_b128 %2, %6\n\t"
        "ds_read_b128 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(o0), "=&v"(o1), "=&v"(o2), "=&v"(o3)
        : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3])
        : "memory");
    o[0] = __builtin_bit_cast(uint4, o0);
    o[1] = __builtin_bit_cast(uint4, o1);
    o[2] = __builtin_bit_cast(uint4, o2);
    o[3] = __builtin_bit_cast(uint4, o3);
}

// One 4-byte LDS read completed before returning.
__device__ inline float lds_read_f32(uint32_t addr) {
    float o;
    __asm__ volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(o) : "v"(addr) : "memory");
    return o;
}

// Four 16-byte LDS writes (the fp8 V copy), ordered by program order with the
// asm reads around them.
__device__ inline void lds_write4x16(const uint32_t (&addr)[4], const uint4 (&v)[4]) {
    __asm__ volatile(
        "ds_write_b128 %0, %4\n\t"
        "ds_write_b128 %1, %5\n\t"
        "ds_write_b128 %2, %6\n\t"
        "ds_write_b128 %3, %7"
        :
        : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3]), "v"(__builtin_bit_cast(u32x4, v[0])),
          "v"(__builtin_bit_cast(u32x4, v[1])), "v"(__builtin_bit_cast(u32x4, v[2])),
          "v"(__builtin_bit_cast(u32x4, v[3]))
        : "memory");
}

// bf16 tile: the 4 K-operand reads and the 8 transposed V reads in one block.
__device__ inline void lds_read_tile_bf16(uint4 (&k)[4], s16x4 (&va)[8], const uint32_t (&ka)[4],
                                          const uint32_t (&va_addr)[8]) {
    typedef short s16x4_v __attribute__((ext_vector_type(4)));
    u32x4 k0, k1, k2, k3;
    s16x4_v o0, o1, o2, o3, o4, o5, o6, o7;
    __asm__ volatile(
        "ds_read_b128 %0, %12\n\t"
        "ds_read_b128 %1, %13\n\t"
        "ds_read_b128 %2, %14\n\t"
        "ds_read_b128 %3, %15\n\t"
        "ds_read_b64_tr_b16 %4, %16\n\t"
        "ds_read_b64_tr_b16 %5, %17\n\t"
        "ds_read_b64_tr_b16 %6, %18\n\t"
        "ds_read_b64_tr_b16 %7, %19\n\t"
        "ds_read_b64_tr_b16 %8, %20\n\t"
        "ds_read_b64_tr_b16 %9, %21\n\t"
        "ds_read_b64_tr_b16 %10, %22\n\t"
        "ds_read_b64_tr_b16 %11, %23\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(k0), "=&v"(k1), "=&v"(k2), "=&v"(k3), "=&v"(o0), "=&v"(o1), "=&v"(o2), "=&v"(o3), "=&v"(o4),
          "=&v"(o5), "=&v"(o6), "=&v"(o7)
        : "v"(ka[0]), "v"(ka[1]), "v"(ka[2]), "v"(ka[3]), "v"(va_addr[0]), "v"(va_addr[1]), "v"(va_addr[2]),
          "v"(va_addr[3]), "v"(va_addr[4]), "v"(va_addr[5]), "v"(va_addr[6]), "v"(va_addr[7])
        : "memory");
    k[0] = __builtin_bit_cast(uint4, k0);
    k[1] = __builtin_bit_cast(uint4, k1);
    k[2] = __builtin_bit_cast(uint4, k2);
    k[3] = __builtin_bit_cast(uint4, k3);
    va[0] = __builtin_bit_cast(s16x4, o0);
    va[1] = __builtin_bit_cast(s16x4, o1);
    va[2] = __builtin_bit_cast(s16x4, o2);
    va[3] = __builtin_bit_cast(s16x4, o3);
    va[4] = __builtin_bit_cast(s16x4, o4);
    va[5] = __builtin_bit_cast(s16x4, o5);
    va[6] = __builtin_bit_cast(s16x4, o6);
    va[7] = __builtin_bit_cast(s16x4, o7);
}

// The same reads at a compile-time byte offset OFF from every address (the
// DS offset field), so that a caller's lane addresses stay fixed across ring
// stages and sub-tiles.
template <int OFF>
__device__ inline void lds_read_tile_bf16_at(uint4 (&k)[4], s16x4 (&va)[8], const uint32_t (&ka)[4],
                                             const uint32_t (&va_addr)[8]) {
    static_assert(OFF >= 0 && OFF < 65536, "DS offset field");
    typedef short s16x4_v __attribute__((ext_vector_type(4)));
    u32x4 k0, k1, k2, k3;
    s16x4_v o0, o1, o2, o3, o4, o5, o6, o7;
    __asm__ volatile(
        "ds_read_b128 %0, %12 offset:%24\n\t"
        "ds_read_b128 %1, %13 offset:%24\n\t"
        "ds_read_b128 %2, %14 offset:%24\n\t"
        "ds_read_b128 %3, %15 offset:%24\n\t"
        "ds_read_b64_tr_b16 %4, %16 offset:%24\n\t"
        "ds_read_b64_tr_b16 %5, %17 offset:%24\n\t"
        "ds_read_b64_tr_b16 %6, %18 offset:%24\n\t"
        "ds_read_b64_tr_b16 %7, %19 offset:%24\n\t"
        "ds_read_b64_tr_b16 %8, %20 offset:%24\n\t"
        "ds_read_b64_tr_b16 %9, %21 offset:%24\n\t"
        "ds_read_b64_tr_b16 %10, %22 offset:%24\n\t"
        "ds_read_b64_tr_b16 %11, %23 offset:%24\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(k0), "=&v"(k1), "=&v"(k2), "=&v"(k3), "=&v"(o0), "=&v"(o1), "=&v"(o2), "=&v"(o3), "=&v"(o4),
          "=&v"(o5), "=&v"(o6), "=&v"(o7)
        : "v"(ka[0]), "v"(ka[1]), "v"(ka[2]), "v"(ka[3]), "v"(va_addr[0]), "v"(va_addr[1]), "v"(va_addr[2]),
          "v"(va_addr[3]), "v"(va_addr[4]), "v"(va_addr[5]), "v"(va_addr[6]), "v"(va_addr[7]), "i"(OFF)
        : "memory");
    k[0] = __builtin_bit_cast(uint4, k0);
    k[1] = __builtin_bit_cast(uint4, k1);
    k[2] = __builtin_bit_cast(uint4, k2);
    k[3] = __builtin_bit_cast(uint4, k3);
    va[0] = __builtin_bit_cast(s16x4, o0);
    va[1] = __builtin_bit_cast(s16x4, o1);
    va[2] = __builtin_bit_cast(s16x4, o2);
    va[3] = __builtin_bit_cast(s16x4, o3);
    va[4] = __builtin_bit_cast(s16x4, o4);
    va[5] = __builtin_bit_cast(s16x4, o5);
    va[6] = __builtin_bit_cast(s16x4, o6);
    va[7] = __builtin_bit_cast(s16x4, o7);
}

// fp8 tile: the two K chunks and the k/v scales (ds_read_b128), and the four
// transposed byte reads of V^T (ds_read_b64_tr_b8), in one block.
__device__ inline void lds_read_tile_fp8_tr(uint4 (&o)[4], uint2 (&v)[4], const uint32_t (&addr)[4],
                                            const uint32_t (&vaddr)[4]) {
    u32x4 o0, o1, o2, o3;
    u32x2 v0, v1, v2, v3;
    __asm__ volatile(
        "ds_read_b128 %0, %8\n\t"
        "ds_read_b128 %1, %9\n\t"
        "ds_read_b128 %2, %10\n\t"
        "ds_read_b128 %3, %11\n\t"
        "ds_read_b64_tr_b8 %4, %12\n\t"
        "ds_read_b64_tr_b8 %5, %13\n\t"
        "ds_read_b64_tr_b8 %6, %14\n\t"
        "ds_read_b64_tr_b8 %7, %15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(o0), "=&v"(o1), "=&v"(o2), "=&v"(o3), "=&v"(v0), "=&v"(v1), "=&v"(v2), "=&v"(v3)
        : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3]), "v"(vaddr[0]), "v"(vaddr[1]), "v"(vaddr[2]),
          "v"(vaddr[3])
        : "memory");
    o[0] = __builtin_bit_cast(uint4, o0);
    o[1] = __builtin_bit_cast(uint4, o1);
    o[2] = __builtin_bit_cast(uint4, o2);
    o[3] = __builtin_bit_cast(uint4, o3);
    v[0] = __builtin_bit_cast(uint2, v0);
    v[1] = __builtin_bit_cast(uint2, v1);
    v[2] = __builtin_bit_cast(uint2, v2);
    v[3] = __builtin_bit_cast(uint2, v3);
}

// fp8 tile: the two K chunks, the two V chunks and the k/v scales in one block.
__device__ inline void lds_read_tile_fp8(uint4 (&o)[6], const uint32_t (&addr)[6]) {
    u32x4 o0, o1, o2, o3, o4, o5;
    __asm__ volatile(
        "ds_read_b128 %0, %6\n\t"
        "ds_read_b128 %1, %7\n\t"
        "ds_read_b128 %2, %8\n\t"
        "ds_read_b128 %3, %9\n\t"
        "ds_read_b128 %4, %10\n\t"
        "ds_read_b128 %5, %11\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(o0), "=&v"(o1), "=&v"(o2), "=&v"(o3), "=&v"(o4), "=&v"(o5)
        : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3]), "v"(addr[4]), "v"(addr[5])
        : "memory");
    o[0] = __builtin_bit_cast(uint4, o0);
    o[1] = __builtin_bit_cast(uint4, o1);
    o[2] = __builtin_bit_cast(uint4, o2);
    o[3] = __builtin_bit_cast(uint4, o3);
    o[4] = __builtin_bit_cast(uint4, o4);
    o[5] = __builtin_bit_cast(uint4, o5);
}

}  // namespace dev
}  // namespace lbsa
