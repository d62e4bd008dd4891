// Device-side building blocks shared by the BitDelta kernels (gfx950 only).
//
// The reconstruction implements the effective weight of "BitDelta : servir
// 14 modèles Zen depuis un seul cluster GPU" (hanzo-blog, 2026-02-28),
// section "Serving architecture": W_eff = W_base + α·sign(Δ), formed as an
// fp32 sum of the bf16 base weight and ±α and rounded once to bf16, rebuilt
// in registers from the packed sign bits ("Infrastructure details": 8 signs
// per byte; here least significant bit first, bit 1 = +1).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bd_internal.h"

namespace bd {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr uint32_t kSignBits = 0x80008000u;

// Keeps a value in a VGPR and hides its provenance from the optimiser (the
// compiler would otherwise fold the per-pair shifts below into 32-bit
// multiplies, which issue at quarter rate).
template <typename T>
__device__ __forceinline__ T opaque(T v) {
    asm("" : "+v"(v));
    return v;
}

// Two fp32 values -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2_t f = {lo, hi};
    bf16x2_t h = __builtin_convertvector(f, bf16x2_t);
    return __builtin_bit_cast(uint32_t, h);
}

// Store one output of the single-variant linear: fp32, or rounded to bf16
// (nearest even, NaN kept) by v_cvt_pk_bf16_f32.
__device__ __forceinline__ void store_y(const YOut& y, int64_t i, float v) {
    if (y.bf16)
        static_cast<uint16_t*>(y.p)[i] = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xffffu);
    else
        static_cast<float*>(y.p)[i] = v;
}

// Rebuild 8 consecutive effective weights.
//   w      8 bf16 base weights, elements k..k+7 (dword p = elements 2p, 2p+1)
//   sbyte  their sign byte (bit b = sign of element k+b, 1 = +1)
//   alpha  the fp32 scale of this row
// Result: 8 bf16 W_eff values in the same packing.
//
// With s = ±1 the sign of an element, round-to-nearest-even is symmetric
// under negation, so RNE_bf16(RNE_f32(w + s·α)) == s·RNE_bf16(RNE_f32(s·w + α)):
// the sign is applied by flipping the bf16 sign bits of the packed pair
// before the fp32 add and again after the conversion, which costs two
// bitwise ops per pair instead of a select per element.  The value is exact;
// only an exact-zero sum with s = -1 comes out as -0 instead of +0, which no
// product can tell apart.  Per pair: 1 shift, 2 bitop3, 2 unpacks, 2 fp32
// adds, 1 v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint4 recon8(uint4 w, uint32_t sbyte, float alpha) {
    // bit b of the byte copied to bits b and b+15, so one left shift by
    // 15-2p puts bit 2p at 15 and bit 2p+1 at 31.
    uint32_t spread = opaque(sbyte | (sbyte << 15));
    uint32_t ws[4] = {w.x, w.y, w.z, w.w};
    uint32_t out[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        uint32_t flip = ~(spread << (15 - 2 * p)) & kSignBits;  // set where the sign is -1
        uint32_t sw = ws[p] ^ flip;
        float lo = __uint_as_float(sw << 16) + alpha;
        float hi = __uint_as_float(sw & 0xffff0000u) + alpha;
        out[p] = pack_bf16x2(lo, hi) ^ flip;
    }
    return make_uint4(out[0], out[1], out[2], out[3]);
}

// Rebuild for several sign sets over the same base weights (one base, many
// variants).  The base's 8 bf16 values are widened to fp32 once (exact), and
// each sign set then forms ±α per element by writing its sign bit into the
// sign of -α, so W_eff = bf16_RNE(w + (±α)) is exactly the definition (no
// symmetry argument, so an exact-zero sum is +0 as in fp32).  The sign bits
// are lined up with one 64-bit shift per pair: the 64-bit value
// {lo: word, hi: word >> 1} shifted left by 31 - 2p - 8g puts bit 8g + 2p of
// the word at bit 31 of the low half and bit 8g + 2p + 1 at bit 31 of the
// high half (g = which byte of the word the 8 weights use).  Per pair:
// 1 shift, 2 bitop3, 2 fp32 adds (double rate), 1 v_cvt_pk_bf16_f32.
struct Widened8 {
    float lo[4], hi[4];
};
__device__ __forceinline__ Widened8 widen8(uint4 w) {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
    Widened8 b;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        b.lo[p] = __uint_as_float(ws[p] << 16);
        b.hi[p] = __uint_as_float(ws[p] & 0xffff0000u);
    }
    return b;
}
// Per-lane shift counts for recon8_word: shifts[p] = 31 - 2p - 8·byte.
struct SignShifts {
    uint32_t s[4];
};
__device__ __forceinline__ SignShifts sign_shifts(int byte) {
    SignShifts r;
#pragma unroll
    for (int p = 0; p < 4; ++p) r.s[p] = (uint32_t)(31 - 2 * p - 8 * byte);
    return r;
}
__device__ __forceinline__ uint64_t shl64(uint64_t v, uint32_t s) {
    uint64_t r;
    asm("v_lshlrev_b64 %0, %1, %2" : "=v"(r) : "v"(s), "v"(v));
    return r;
}
// The 64-bit spread {lo: word, hi: word >> 1} of a sign word.  The low half
// is a fresh copy, so the word's own register (often a load destination
// reused across loop iterations) is never tied into a register pair.
__device__ __forceinline__ uint64_t sign_spread(uint32_t word) {
    uint32_t lo;
    asm("v_mov_b32 %0, %1" : "=v"(lo) : "v"(word));
    return ((uint64_t)(word >> 1) << 32) | lo;
}
//   b       the widened base weights k..k+7
//   spread  sign_spread(word) of 32 sign bits; this lane's 8 are bits
//           8·byte .. 8·byte+7 of the word
//   sh      sign_shifts(byte)
//   nalpha  bit pattern of -α for this row
__device__ __forceinline__ uint4 recon8_word(const Widened8& b, uint64_t spread, const SignShifts& sh,
                                             uint32_t nalpha) {
    uint32_t out[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const uint64_t t = shl64(spread, sh.s[p]);
        const float al = __uint_as_float(nalpha ^ ((uint32_t)t & 0x80000000u));
        const float ah = __uint_as_float(nalpha ^ ((uint32_t)(t >> 32) & 0x80000000u));
        out[p] = pack_bf16x2(b.lo[p] + al, b.hi[p] + ah);
    }
    return make_uint4(out[0], out[1], out[2], out[3]);
}

// Dot product of 8 bf16 pairs' worth (4 packed dwords) with fp32 result:
// a short chain of v_dot2c_f32_bf16 started from zero, so its rounding stays
// local; callers add the partial into their running sum with an fp32 add.
__device__ __forceinline__ float dot8_bf16(uint4 a, uint4 b) {
    float s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.x),
                                              __builtin_bit_cast(bf16x2_t, b.x), 0.0f, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.y),
                                        __builtin_bit_cast(bf16x2_t, b.y), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.z),
                                        __builtin_bit_cast(bf16x2_t, b.z), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.w),
                                        __builtin_bit_cast(bf16x2_t, b.w), s, false);
    return s;
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// Streaming loads: the base weights and sign bytes are read exactly once.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4n_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream16(const uint4* p) {
    u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float4 load_stream16(const float4* p) {
    f32x4n_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4n_t*>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t load_stream_u8(const uint8_t* p) {
    return (uint32_t)__builtin_nontemporal_load(p);
}

// Raw buffer access: a 128-bit resource (base, byte size) in SGPRs, a per-lane
// 32-bit offset and a uniform offset.  Reads at or past the size return zero.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;  // raw, untyped 32-bit buffer
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRsrcWord3);
}
__device__ __forceinline__ uint4 buf_load16(rsrc_t r, uint32_t voff, uint32_t soff) {
    u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 buf_load8(rsrc_t r, uint32_t voff, uint32_t soff) {
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
    return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint32_t buf_load_u8(rsrc_t r, uint32_t voff, uint32_t soff) {
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, voff, soff, 0);
}

// Butterfly sum over the 64 lanes of a wave; every lane gets the same total.
// Fixed pairing order, so the result is run-to-run reproducible.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

}  // namespace bd
