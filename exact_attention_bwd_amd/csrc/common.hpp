// Device-side building blocks shared by the attention kernels (gfx950 / CDNA4).
//
// Matrix-core conventions used throughout (v_mfma_f32_32x32x16_bf16, wave64):
//   A operand, 32 (M) x 16 (K): lane l holds A[m = l % 32][k = 8 * (l / 32) + e], e = 0..7
//   B operand, 16 (K) x 32 (N): lane l holds B[k = 8 * (l / 32) + e][n = l % 32]
//   C/D,       32 x 32 fp32:    lane l holds C[m = 8 * (r / 4) + 4 * (l / 32) + r % 4][n = l % 32],
//                               r = 0..15
// A and B share the same (lane group, element) -> k assignment, so any
// consistent relabelling of k on both operands gives the same product.  The
// kernels use that freedom to feed an accumulator tile back in as an A operand
// without a trip through LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.f;
    return z;
}

// Round-to-nearest-even fp32 -> bf16 of eight values (v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16x8 to_bf16x8(f32x8 x) {
    return __builtin_convertvector(x, bf16x8);
}

// Eight consecutive accumulator entries (r = base .. base + 7) of a C tile,
// rounded to bf16: the A or B operand for one 16-deep k step.
__device__ __forceinline__ bf16x8 pack_c8(const f32x16& c, int base) {
    f32x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = c[base + e];
    return to_bf16x8(v);
}

__device__ __forceinline__ bf16x8 lds_read16(const __bf16* p) {
    return *reinterpret_cast<const bf16x8*>(p);
}

__device__ __forceinline__ bf16x4 lds_read8(const __bf16* p) {
    return *reinterpret_cast<const bf16x4*>(p);
}

__device__ __forceinline__ bf16x8 cat44(bf16x4 lo, bf16x4 hi) {
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Global 16-byte load through the vector memory path.
__device__ __forceinline__ u32x4 gload16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

// Select the 16-bit element `c` (0..7) of a 16-byte row chunk.
__device__ __forceinline__ uint32_t half_of(const u32x4& v, int c) {
    uint32_t w = v[c >> 1];
    return (c & 1) ? (w >> 16) : (w & 0xffffu);
}

// Transposed 4x8 -> 8x4: rows r0..r3 hold 8 bf16 each; returns for column c the
// four values (r0[c], r1[c], r2[c], r3[c]) packed as two dwords.
__device__ __forceinline__ u32x2 column4(const u32x4& r0, const u32x4& r1,
                                         const u32x4& r2, const u32x4& r3, int c) {
    // v_perm_b32 selector: bytes of (src0:src1); pick the low or high half of
    // the dword that holds column c from each of two rows.
    const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
    u32x2 out;
    out[0] = __builtin_amdgcn_perm(r1[c >> 1], r0[c >> 1], sel);
    out[1] = __builtin_amdgcn_perm(r3[c >> 1], r2[c >> 1], sel);
    return out;
}

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane i receives element i % 4 of the 8 bytes addressed by lanes i / 4,
// 4 + i / 4, 8 + i / 4 and 12 + i / 4.  If lane t of the group addresses row
// r0 + t / 4, columns c0 + 4 (t % 4) .. + 3 of a row-major tile, lane i gets
// column c0 + i of rows r0 .. r0 + 3.
__device__ __forceinline__ bf16x4 lds_read_tr(const __bf16* p) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(p));
    return __builtin_bit_cast(bf16x4, v);
}

// Direct global -> LDS copy: lane l of the wave writes its `bytes` (4 or 16)
// at lds_base + l * bytes; lds_base is the same for the whole wave.
__device__ __forceinline__ void dma16(const void* src, void* lds_base) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}

__device__ __forceinline__ void dma4(const void* src, void* lds_base) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_base, 4, 0, 0);
}

// Raw buffer resource over `bytes` bytes from `base`: loads past the end read
// as zero, stores past the end are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// Buffer -> LDS copy: lane l of the wave writes its BYTES at lds_base + l * BYTES.
__device__ __forceinline__ void bdma16(__amdgpu_buffer_rsrc_t r, int voff, void* lds_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 16,
                                             voff, 0, 0, 0);
}

// The same copy marked non-temporal, for data read exactly once (a stored dS
// tile): it streams through the caches instead of displacing shared tiles.
__device__ __forceinline__ void bdma16_nt(__amdgpu_buffer_rsrc_t r, int voff, void* lds_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 16,
                                             voff, 0, 0, 2);
}

__device__ __forceinline__ void bdma4(__amdgpu_buffer_rsrc_t r, int voff, void* lds_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 4,
                                             voff, 0, 0, 0);
}

// Index of this lane's wave in the workgroup, as a wave-uniform (scalar) value:
// values derived from it (LDS bases, buffer descriptors) stay in SGPRs.
__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

__device__ __forceinline__ float wave_max_pair32(float x) {
    // combine lane l with lane l ^ 32
    return fmaxf(x, __shfl_xor(x, 32));
}

// Map a hardware workgroup index to a logical one so that consecutive logical
// indices run on the same XCD (workgroups are dealt round-robin over the 8
// XCDs).  Bijective on [0, total).
__device__ __forceinline__ int xcd_remap(int hw, int total) {
    constexpr int kXcd = 8;
    const int q = total / kXcd, r = total % kXcd;
    const int x = hw % kXcd, local = hw / kXcd;
    return x * q + (x < r ? x : r) + local;
}

// Grouped-query attention: flattened query head bh = b * H + h reads the
// key / value head b * (H / G) + h / G (G query heads per K / V head; G = 1 is
// ordinary multi-head attention).
__device__ __forceinline__ int kv_head(int bh, int H, int G) {
    return (bh / H) * (H / G) + (bh % H) / G;
}

}  // namespace attn
