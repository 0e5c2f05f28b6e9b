// Device helpers shared by the decode and multi-token decode kernels: vector
// types, buffer loads with a range check, base-2 exponent, 16-lane DPP
// reductions, bf16/f16 packing and dot products, and the int8 / e4m3 code
// conversions onto f16.  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));   // store operand type

// Cache-policy immediate of buffer accesses for system-scope coherence
// (sc0 sc1): stores write through to memory, loads bypass the caches.
constexpr int kSysCoherent = 17;
// s_waitcnt immediates (gfx9 layout: vmcnt bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8; a field at its maximum does not wait).
constexpr int kWaitVm0 = 0x0F70;     // vmcnt(0)
constexpr int kWaitVm16 = 0x4F70;    // vmcnt(16)
constexpr int kWaitLgkm0 = 0xC07F;   // lgkmcnt(0)
// Cache-policy immediate for data read once (nt, streaming).
constexpr int kStreaming = 2;

// Raw buffer loads, bit-cast to plain structs at once: reading lanes of the
// builtins' vector results through a local vector variable was seen to
// compile to a single-dword load whose value fills every lane.
template <int AUX = 0>
__device__ __forceinline__ void buf_st16(uint4 v, __amdgpu_buffer_rsrc_t r, int off) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, off, 0, AUX);
}
template <int AUX = 0>
__device__ __forceinline__ void buf_st4(uint32_t v, __amdgpu_buffer_rsrc_t r, int off) {
    __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, AUX);
}
// AUX is the cache-policy immediate.
template <int AUX = 0>
__device__ __forceinline__ uint4 buf_ld16(__amdgpu_buffer_rsrc_t r, int off, int soff) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, AUX));
}
template <int AUX = 0>
__device__ __forceinline__ uint2 buf_ld8(__amdgpu_buffer_rsrc_t r, int off, int soff) {
    return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, soff, AUX));
}
template <int AUX = 0>
__device__ __forceinline__ float buf_ldf(__amdgpu_buffer_rsrc_t r, int off, int soff) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, soff, AUX));
}
// 16 bytes per lane straight into LDS: lane l's bytes land at lds + 16 l
// (lds is uniform); bytes past the resource's range arrive as zeros.
// Completion is counted by vmcnt like any other load.
template <int AUX = 0>
__device__ __forceinline__ void buf_ld16_lds(__amdgpu_buffer_rsrc_t r, void *lds, int off,
                                             int soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16,
                                             off, soff, 0, AUX);
}

// Word 3 of a gfx9 buffer resource for raw (untyped, unswizzled) access:
// data format field = 32-bit, so dword loads of any width are range checked
// against the descriptor's byte size.
constexpr int kBufferWord3 = 0x00020000;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();
constexpr float kPosInf = __builtin_inff();

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// DPP lane permutations inside a 16-lane row.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
// Butterfly over the 16 lanes of a row: xor 1, xor 2, half-row mirror, row mirror.
__device__ __forceinline__ float row_max16(float x) {
    x = fmaxf(x, dpp<0xB1>(x));
    x = fmaxf(x, dpp<0x4E>(x));
    x = fmaxf(x, dpp<0x141>(x));
    x = fmaxf(x, dpp<0x140>(x));
    return x;
}
__device__ __forceinline__ float row_sum16(float x) {
    x = x + dpp<0xB1>(x);
    x = x + dpp<0x4E>(x);
    x = x + dpp<0x141>(x);
    x = x + dpp<0x140>(x);
    return x;
}

// Lane l combined with lane l ^ 16 (xor16) or l ^ 32 (xor32), by the gfx950
// cross-lane swaps (vector ALU, no LDS round trip as a shuffle takes).  A
// value swapped with a copy of itself: v_permlane16_swap exchanges the odd
// 16-lane rows of the first operand with the even rows of the second,
// leaving rows (0, 0, 2, 2) and (1, 1, 3, 3); v_permlane32_swap exchanges
// the upper 32 lanes of the first with the lower 32 of the second, leaving
// (lo, lo) and (hi, hi).  Every lane then combines the same two values as
// with a shuffle (the operands of a commutative operation in the other
// order for half of the lanes: same result).  Whole wave active.
__device__ __forceinline__ float add_xor16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float add_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Whether the requests of a batch have about the same number of pages: the
// longest at most 6/5 of the mean.  A split walk gives a workgroup the pages
// of several splits of one request, so it pays only for such a batch; in a
// ragged one the longest requests' walks trail the rest.  Li is request
// `lane`'s length (ignored where lane >= batch); lanes load the requests past
// the first 64.  Lengths are cut to [0, max_len]; page counts are summed as
// floats (exact while the batch holds under 2^24 pages).  Whole wave active;
// the result is the same in every lane.
__device__ __forceinline__ bool pages_balanced(const int32_t *__restrict__ seq_lens, int batch,
                                               int Li, int64_t max_len, int page, int lane) {
    float tot = 0.f, mx = 0.f;
    auto add = [&](int len) {
        const int64_t l = min((int64_t)max(len, 0), max_len);
        const float pg = (float)((l + page - 1) / page);
        tot += pg;
        mx = fmaxf(mx, pg);
    };
    if (lane < batch) add(Li);
    for (int i = lane + 64; i < batch; i += 64) add(seq_lens[i]);
    tot = add_xor32(add_xor16(row_sum16(tot)));
    mx = max_xor32(max_xor16(row_max16(mx)));
    return __builtin_amdgcn_readfirstlane(5.f * mx * (float)batch <= 6.f * tot) != 0;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2_t v;
    v[0] = (__bf16)lo;   // round to nearest even
    v[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, v);
}
// The low bf16 terms of (lo, hi) given their high terms `hi_terms` (a
// pack_bf16x2 of the same pair): x - bf16(x) is exact in fp32 and rounds to
// the next 8 significant bits.
__device__ __forceinline__ uint32_t bf16x2_residual(float lo, float hi, uint32_t hi_terms) {
    return pack_bf16x2(lo - __uint_as_float(hi_terms << 16),
                       hi - __uint_as_float(hi_terms & 0xffff0000u));
}
__device__ __forceinline__ uint16_t to_bf16_bits(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    f16x2_t v;
    v[0] = (_Float16)lo;   // round to nearest even
    v[1] = (_Float16)hi;
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b),
                                  c, false);
}
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
// Eight int8 key codes -> eight exact f16 values.  The sign bits are flipped
// (code + 128, in 1..255), each code becomes the low mantissa byte under the
// f16 exponent of 1024 -- one byte permute with a 0x64 constant per pair --
// reading 1152 + code, and one packed subtract of 1152 leaves the code.
__device__ __forceinline__ f16x8_t i8x8_to_f16(uint2 w) {
    const uint32_t x = w.x ^ 0x80808080u, y = w.y ^ 0x80808080u;
    constexpr uint32_t kExp = 0x64646464u;
    const uint32_t d0 = __builtin_amdgcn_perm(kExp, x, 0x04010400u);
    const uint32_t d1 = __builtin_amdgcn_perm(kExp, x, 0x04030402u);
    const uint32_t d2 = __builtin_amdgcn_perm(kExp, y, 0x04010400u);
    const uint32_t d3 = __builtin_amdgcn_perm(kExp, y, 0x04030402u);
    const f16x2_t bias = {(_Float16)1152.f, (_Float16)1152.f};
    const f16x2_t h0 = __builtin_bit_cast(f16x2_t, d0) - bias;
    const f16x2_t h1 = __builtin_bit_cast(f16x2_t, d1) - bias;
    const f16x2_t h2 = __builtin_bit_cast(f16x2_t, d2) - bias;
    const f16x2_t h3 = __builtin_bit_cast(f16x2_t, d3) - bias;
    return f16x8_t{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
}

// Eight e4m3 key codes (dims in byte order) -> their exact f16 values; the
// converter takes bytes 0-1 (word_sel false) or 2-3 of a word, low byte to
// the low half.
// Eight int8 value codes -> eight exact f16 values 1152 + code (the bias is
// removed once per split through the sum of the probabilities).
__device__ __forceinline__ f16x8_t i8x8_to_f16_biased(uint2 w) {
    const uint32_t x = w.x ^ 0x80808080u, y = w.y ^ 0x80808080u;
    constexpr uint32_t kExp = 0x64646464u;
    return __builtin_bit_cast(f16x8_t, make_uint4(__builtin_amdgcn_perm(kExp, x, 0x04010400u),
                                                  __builtin_amdgcn_perm(kExp, x, 0x04030402u),
                                                  __builtin_amdgcn_perm(kExp, y, 0x04010400u),
                                                  __builtin_amdgcn_perm(kExp, y, 0x04030402u)));
}
__device__ __forceinline__ f16x8_t e4m3x8_to_f16(uint2 w) {
    const f16x2_t h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.x, 1.f, false);
    const f16x2_t h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.x, 1.f, true);
    const f16x2_t h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.y, 1.f, false);
    const f16x2_t h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.y, 1.f, true);
    return f16x8_t{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
}

// e4m3 value codes -> f16 pairs for the token pair (a, b): bytes k and k+1
// of wa and wb (k = 0 or 2) give the pairs (a_k, b_k) and (a_k+1, b_k+1),
// each value / 256 (exact: the converter keeps f16 subnormals).
constexpr float kF8ValueScale = 256.f;
template <int K>
__device__ __forceinline__ void e4m3_pairs_f16(uint32_t wb, uint32_t wa, uint32_t &p0,
                                               uint32_t &p1) {
    constexpr uint32_t sel = (uint32_t)K | ((uint32_t)(4 + K) << 8) | ((uint32_t)(K + 1) << 16) |
                             ((uint32_t)(5 + K) << 24);
    const uint32_t w = __builtin_amdgcn_perm(wb, wa, sel);   // a_k, b_k, a_k+1, b_k+1
    p0 = __builtin_bit_cast(uint32_t,
                            __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.f / kF8ValueScale, false));
    p1 = __builtin_bit_cast(uint32_t,
                            __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.f / kF8ValueScale, true));
}

// int8 value codes -> exact f16, biased: byte k of wa (token a) and of wb
// (token b) become the f16 pair (1152 + a_k, 1152 + b_k).  With its sign bit
// flipped a code is x + 128 in [1, 255]; placed as the low mantissa byte under
// the f16 exponent of 1024 it reads 1024 + x + 128.
constexpr float kI8Bias = 1152.f;
constexpr uint32_t kF16One2 = 0x3C003C00u;   // f16 pair (1, 1)
template <int K>
__device__ __forceinline__ uint32_t i8_pair_f16(uint32_t wb, uint32_t wa) {
    constexpr uint32_t sel = (uint32_t)K | (0x0Cu << 8) | ((uint32_t)(4 + K) << 16) | (0x0Cu << 24);
    return __builtin_amdgcn_perm(wb, wa, sel) ^ 0x64806480u;
}

// Maximum over the 64 lanes of a wave, returned as a wave-uniform value: the
// row butterfly (xor 1, xor 2, half-row mirror, row mirror), then row 0 into
// row 1 and row 2 into row 3 (broadcast of each row's lane 15), then rows 0-1
// into rows 2-3 (lane 31), so lane 63 holds the maximum of all four rows.
// One v_max_f32 with a DPP source per step; written out because the compiler
// splits each step into a DPP move, a NaN-quieting max and the max.  The
// inputs are never NaN.  s_nop 1 gives each DPP read the two wait states it
// needs after the VALU write of its source.
__device__ __forceinline__ float wave_max(float x) {
    float y;
    __asm__("s_nop 1\n\t"
            "v_max_f32_dpp %0, %1, %1 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
            "s_nop 1\n\t"
            "v_max_f32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
            "s_nop 1\n\t"
            "v_max_f32_dpp %0, %0, %0 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
            "s_nop 1\n\t"
            "v_max_f32_dpp %0, %0, %0 row_mirror row_mask:0xf bank_mask:0xf\n\t"
            "s_nop 1\n\t"
            "v_max_f32_dpp %0, %0, %0 row_bcast:15 row_mask:0xa bank_mask:0xf\n\t"
            "s_nop 1\n\t"
            "v_max_f32_dpp %0, %0, %0 row_bcast:31 row_mask:0xc bank_mask:0xf"
            : "=&v"(y)
            : "v"(x));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(y), 63));
}

// Transposed LDS reads (gfx950; lane mappings measured with an in-bounds
// probe).  In each group of 16 lanes 16G .. 16G + 15, every lane supplies the
// address of one 8-byte chunk, and
//  * ds_read_b64_tr_b16: lane 16G + i receives as 16-bit element e (0..3)
//    element i mod 4 of the chunk addressed by lane 16G + 4e + i/4;
//  * ds_read_b64_tr_b8: lane 16G + i receives as byte e (0..7) byte i mod 8
//    of the chunk addressed by lane 16G + 2e + i/8.
// With chunks that are rows of a token-major tile, a lane thus gathers one
// column (a head, a dimension) over 4 or 8 tokens: a matrix-core operand
// whose contraction runs over tokens.
__device__ __forceinline__ uint64_t lds_tr16_b64(const uint16_t *p) {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
    const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16 *)(const_cast<uint16_t *>(p)));
    return __builtin_bit_cast(uint64_t, v);
}
__device__ __forceinline__ uint2 lds_tr8_b64(const uint8_t *p) {
    typedef int v2i32 __attribute__((ext_vector_type(2)));
    typedef __attribute__((address_space(3))) v2i32 lds_v2i32;
    const v2i32 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i32 *)(const_cast<uint8_t *>(p)));
    return make_uint2((uint32_t)v.x, (uint32_t)v.y);
}
__device__ __forceinline__ bf16x8_t join_bf16x8(uint64_t lo, uint64_t hi) {
    return __builtin_bit_cast(bf16x8_t, make_uint4((uint32_t)lo, (uint32_t)(lo >> 32),
                                                   (uint32_t)hi, (uint32_t)(hi >> 32)));
}
__device__ __forceinline__ f16x8_t join_f16x8(uint64_t lo, uint64_t hi) {
    return __builtin_bit_cast(f16x8_t, make_uint4((uint32_t)lo, (uint32_t)(lo >> 32),
                                                  (uint32_t)hi, (uint32_t)(hi >> 32)));
}

// v_g of four per-lane values, g = 0..3 (two levels of selects on the bits of
// g, which compile to conditional moves rather than branches).
__device__ __forceinline__ float pick4(float v0, float v1, float v2, float v3, int g) {
    const float lo = (g & 1) ? v1 : v0;
    const float hi = (g & 1) ? v3 : v2;
    return (g & 2) ? hi : lo;
}

// Value of v in lane src (a cross-lane permute, no memory access).
__device__ __forceinline__ float lane_value(float v, int src) {
    return __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(v)));
}

}  // namespace spa
