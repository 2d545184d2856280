// Inline-assembly building blocks of the hand-scheduled kernels (gfx950).
//
// These kernels issue LDS and global loads from assembly at fixed points of a
// static schedule and wait for each with an explicit s_waitcnt count derived
// from the issue order (LDS reads complete in order), instead of the
// conservative waits the compiler would insert.  MFMAs are issued from
// assembly as well, so that accumulators stay where the kernel puts them
// (VGPRs for products the VALU reads, AGPRs for long-lived sums).
#pragma once

#include <type_traits>

#include "common.hpp"

namespace attn {

// Compile-time loop: f(std::integral_constant<int, i>) for i = I .. N-1, so
// that indices are constants (immediate offsets, if constexpr).
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

// Products whose results the VALU reads (S, dP) are issued as VGPR-form
// MFMAs: with the long-lived accumulators (dK / dV, O) in the AGPR file,
// leaving the choice to the compiler puts every MFMA result in AGPRs and
// overflows them.  Hazards this implies (the compiler inserts them for its
// own MFMAs): a VALU read of an MFMA result needs 12 wait states after the
// MFMA (mfma_v_settle2 gives 16), dependent accumulation and LDS loads into
// the operand registers need none.
__device__ __forceinline__ void mfma_v(f32x16& c, const bf16x8& a, const bf16x8& b) {
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}

__device__ __forceinline__ void mfma_v0(f32x16& c, const bf16x8& a, const bf16x8& b) {
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=v"(c) : "v"(a), "v"(b));
}

// c = a b + cin (cin another register tuple, not overwritten)
__device__ __forceinline__ void mfma_vc(f32x16& c, const bf16x8& a, const bf16x8& b, const f32x16& cin) {
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %3" : "=&v"(c) : "v"(a), "v"(b), "v"(cin));
}

__device__ __forceinline__ void mfma_v_settle2(f32x16& a, f32x16& b) {
    asm volatile("s_nop 15" : "+v"(a), "+v"(b));
}

// Accumulation into the AGPR file (dV / dK, O); no VALU reads these
// registers until an s_nop settle after the last one.
__device__ __forceinline__ void mfma_a(f32x16& c, const bf16x8& a, const bf16x8& b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}

// Transposing LDS reads issued from inline assembly.  The compiler treats its
// own ds_read_b64_tr_b16 as possibly reading what an in-flight buffer -> LDS
// copy writes and waits for all of them (vmcnt(0)) first, which would expose
// the next tile's copy latency in every iteration; these reads only touch the
// tile being computed on, which the copies never write.  The compiler does not track
// their completion, so tr_wait must follow before the results are used: with
// `pending` = the number of LDS reads issued after them, lgkmcnt(pending)
// guarantees they are done (LDS operations complete in order).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)p);
}

__device__ __forceinline__ void tr_read4(u32x2& a, u32x2& b, u32x2& c, u32x2& d, uint32_t pa,
                                         uint32_t pb, uint32_t pc, uint32_t pd) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %4\n\t"
        "ds_read_b64_tr_b16 %1, %5\n\t"
        "ds_read_b64_tr_b16 %2, %6\n\t"
        "ds_read_b64_tr_b16 %3, %7"
        : "=&v"(a), "=&v"(b), "=&v"(c), "=&v"(d)
        : "v"(pa), "v"(pb), "v"(pc), "v"(pd));
}

__device__ __forceinline__ void tr_read2(u32x2& a, u32x2& b, uint32_t pa, uint32_t pb) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %2\n\t"
        "ds_read_b64_tr_b16 %1, %3"
        : "=&v"(a), "=&v"(b)
        : "v"(pa), "v"(pb));
}

template <int OFF>
__device__ __forceinline__ void tr_read2o(u32x2& a, u32x2& b, uint32_t pa, uint32_t pb) {
    static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
    asm volatile(
        "ds_read_b64_tr_b16 %0, %2 offset:%4\n\t"
        "ds_read_b64_tr_b16 %1, %3 offset:%4"
        : "=&v"(a), "=&v"(b)
        : "v"(pa), "v"(pb), "n"(OFF));
}

template <int PENDING>
__device__ __forceinline__ void tr_wait2(u32x2& a, u32x2& b) {
    static_assert(PENDING >= 0 && PENDING <= 15, "pending count");
    asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(a), "+v"(b) : "n"(PENDING));
}

// 16-byte LDS read at a + OFF, issued where it stands; lgkm_wait must follow
// before the result is used.
template <int OFF, typename T>
__device__ __forceinline__ void lds_ld(T& d, uint32_t a) {
    static_assert(sizeof(T) == 16 && OFF >= 0 && OFF < 65536, "b128 read");
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=&v"(d) : "v"(a), "n"(OFF));
}

// The same reads into AGPRs (matrix-core operands that no VALU instruction
// touches can live in the AGPR file; MFMA reads A and B from either file).
template <int OFF, typename T>
__device__ __forceinline__ void lds_ld_a(T& d, uint32_t a) {
    static_assert(sizeof(T) == 16 && OFF >= 0 && OFF < 65536, "b128 read");
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=&a"(d) : "v"(a), "n"(OFF));
}

template <int OFF>
__device__ __forceinline__ void tr_read2o_a(u32x2& a, u32x2& b, uint32_t pa, uint32_t pb) {
    static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
    asm volatile(
        "ds_read_b64_tr_b16 %0, %2 offset:%4\n\t"
        "ds_read_b64_tr_b16 %1, %3 offset:%4"
        : "=&a"(a), "=&a"(b)
        : "v"(pa), "v"(pb), "n"(OFF));
}

// a ^ C, computed where it stands (C = 0: a itself)
template <int C>
__device__ __forceinline__ uint32_t vxor(uint32_t a) {
    if constexpr (C == 0) {
        return a;
    } else {
        uint32_t r;
        asm volatile("v_xor_b32 %0, %1, %2" : "=v"(r) : "n"(C), "v"(a));
        return r;
    }
}

// s_waitcnt lgkmcnt(N) (N above 15 waits for 15, which is stricter), tied to
// the registers whose loads it completes
template <int N, typename A>
__device__ __forceinline__ void lgkm_wait(A& a) {
    static_assert(N >= 0, "wait count");
    asm volatile("s_waitcnt lgkmcnt(%[n])" : "+v"(a) : [n] "n"(N > 15 ? 15 : N));
}
template <int N, typename A, typename B>
__device__ __forceinline__ void lgkm_wait(A& a, B& b) {
    static_assert(N >= 0, "wait count");
    asm volatile("s_waitcnt lgkmcnt(%[n])" : "+v"(a), "+v"(b) : [n] "n"(N > 15 ? 15 : N));
}
template <int N, typename A, typename B, typename C>
__device__ __forceinline__ void lgkm_wait(A& a, B& b, C& c) {
    static_assert(N >= 0, "wait count");
    asm volatile("s_waitcnt lgkmcnt(%[n])" : "+v"(a), "+v"(b), "+v"(c) : [n] "n"(N > 15 ? 15 : N));
}

// lgkm_wait for reads into AGPRs
template <int N, typename A>
__device__ __forceinline__ void lgkm_wait_a(A& a) {
    static_assert(N >= 0, "wait count");
    asm volatile("s_waitcnt lgkmcnt(%[n])" : "+a"(a) : [n] "n"(N > 15 ? 15 : N));
}
template <int N, typename A, typename B>
__device__ __forceinline__ void lgkm_wait_a(A& a, B& b) {
    static_assert(N >= 0, "wait count");
    asm volatile("s_waitcnt lgkmcnt(%[n])" : "+a"(a), "+a"(b) : [n] "n"(N > 15 ? 15 : N));
}

// 16-byte global load at base + voff + OFF (OFF < 4096), issued where it
// stands; vm_wait must follow before the result is used.
template <int OFF>
__device__ __forceinline__ void gload16(bf16x8& d, const void* base, uint32_t voff) {
    static_assert(OFF >= 0 && OFF < 4096, "global offset field");
    asm volatile("global_load_dwordx4 %0, %1, %2 offset:%3" : "=&v"(d) : "v"(voff), "s"(base), "n"(OFF));
}

// gload16 that misses the CU's L1 (data other CUs wrote during the kernel)
template <int OFF>
__device__ __forceinline__ void gload16_l2(bf16x8& d, const void* base, uint32_t voff) {
    static_assert(OFF >= 0 && OFF < 4096, "global offset field");
    asm volatile("global_load_dwordx4 %0, %1, %2 offset:%3 sc0" : "=&v"(d) : "v"(voff), "s"(base), "n"(OFF));
}

// s_waitcnt vmcnt(N), tied to the eight registers whose loads it completes
template <int N>
__device__ __forceinline__ void vm_wait(bf16x8* r) {
    static_assert(N >= 0 && N < 64, "vmcnt");
    asm volatile("s_waitcnt vmcnt(%[n])"
                 : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]), "+v"(r[4]), "+v"(r[5]), "+v"(r[6]), "+v"(r[7])
                 : [n] "n"(N)
                 : "memory");
}

template <int PENDING>
__device__ __forceinline__ void tr_wait(u32x2& a, u32x2& b, u32x2& c, u32x2& d) {
    static_assert(PENDING == 0 || PENDING == 4, "pending count");
    if (PENDING == 0)
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
    else
        asm volatile("s_waitcnt lgkmcnt(4)" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
}

__device__ __forceinline__ bf16x8 cat_u(u32x2 lo, u32x2 hi) {
    return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
}

}  // namespace attn
