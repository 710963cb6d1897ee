// common.h -- device-side helpers shared by the librehyat HIP kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rehyat {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) uint16_t lds_u16;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Unpack 8 bf16 held in a 16-byte vector into fp32.
__device__ __forceinline__ void unpack8(const u32x4 w, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(w[i] << 16);
        f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}

// Round two fp32 to bf16 (nearest-even) and pack them, low element first.
__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
    bf16x2 p = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, p);
}

__device__ __forceinline__ float round_bf16(float a) {
    return (float)(__bf16)a;
}

// Two-term bf16 split of a pair, returned as {hi, lo}: hi = the pair rounded to
// bf16 (nearest-even, low element first), lo = the bf16 rounding of a - hi_a and
// b - hi_b, so that hi + lo carries about 16 significant bits.  One conversion
// yields both hi halves, which widen back to fp32 exactly by shifting and masking
// (the empty asm keeps the compiler from converting the low element again for
// the shift).
__device__ __forceinline__ u32x2 split2_bf16(float a, float b) {
    uint32_t hi = pack2_bf16(a, b);
    asm("" : "+v"(hi));
    const float ha = __uint_as_float(hi << 16), hb = __uint_as_float(hi & 0xffff0000u);
    return u32x2{hi, pack2_bf16(a - ha, b - hb)};
}

// elu(x) + 1 with alpha = 1.
__device__ __forceinline__ float elu1(float x) {
    return x > 0.0f ? x + 1.0f : __expf(x);
}

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// LDS transposed read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// source lane s points at 4 consecutive 16-bit elements; lane i receives
// element (i % 4) of the source lanes 4e + i/4, e = 0..3.  Pointing source
// lane s at (row e = s/4, column c0 + 4*(s%4)) of a row-major array therefore
// hands lane i the column c0 + i of rows 0..3.
__device__ __forceinline__ bf16x4 lds_read_tr(const lds_u16* base, int elem_offset) {
    s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + elem_offset));
    return __builtin_bit_cast(bf16x4, r);
}

// Row pitch (in 16-bit elements) for a row-major LDS tile of `cols` columns
// that is read with lds_read_tr: each read covers 8 rows x 64 bytes, so rows
// should start 16 banks apart (pitch = 64 or 192 bytes mod 256) to spread them
// over all 64 banks.
constexpr int tr_pitch(int cols) {
    int pad = 0;
    while (((cols + pad) * 2) % 256 != 64 && ((cols + pad) * 2) % 256 != 192) pad += 8;
    return cols + pad;
}

__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ bf16x8 lds_read_b128(const lds_u16* base, int elem_offset) {
    return *(const __attribute__((address_space(3))) bf16x8*)(base + elem_offset);
}

__device__ __forceinline__ void lds_write_b128(lds_u16* base, int elem_offset, u32x4 v) {
    *(__attribute__((address_space(3))) u32x4*)(base + elem_offset) = v;
}

__device__ __forceinline__ u32x4 ldg_b128(const uint16_t* p) {
    return *(const u32x4*)p;
}

// Combine the values of lanes l and l ^ 32 (the two halves of a wave).
// v_permlane32_swap exchanges the upper half of its first operand with the
// lower half of its second; with both operands x, the two results hold, in
// every lane l, x[l % 32] and x[32 + l % 32] (no LDS traffic, unlike a
// shuffle through ds_bpermute).
__device__ __forceinline__ float xhalf_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Map a linear block index so that consecutive logical work items land on the
// same XCD (the dispatcher deals workgroups round-robin over the 8 XCDs).
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
    constexpr int kXcd = 8;
    const int per = nblocks / kXcd;     // full rounds
    const int tail = nblocks % kXcd;
    const int xcd = bid % kXcd;
    const int idx = bid / kXcd;
    // XCDs < tail own per+1 items, the others own per
    const int start = xcd < tail ? xcd * (per + 1) : tail * (per + 1) + (xcd - tail) * per;
    return start + idx;
}

}  // namespace rehyat
