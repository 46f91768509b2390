// dev_common.hpp -- device helpers shared by the gfx950 kernels of libqgemm.
//
// Operand encodings (INT4 GEMM article, www.cf-1.com/news/6060138, §2.1):
// packed int4 holds element 2i in the low nibble of byte i and element 2i+1
// in the high nibble, 4-bit two's complement.
//
// CDNA4 has no int4 matrix instruction, so int4 operands are widened to int8
// in registers before the int8 MFMA.  The widening places each nibble in the
// TOP half of its byte:
//     lo = (p << 4) & 0xF0F0F0F0   -> bytes 16*v[2i]
//     hi =  p       & 0xF0F0F0F0   -> bytes 16*v[2i+1]
// A byte whose top nibble is the code and bottom nibble is 0 reads, as a
// signed int8, exactly 16 times the nibble's signed value.  Products of two
// widened operands are therefore 256*a*b and products with an int8 operand
// 16*a*b; the epilogue shifts the exact int32 sum right by 8 or 4, which is
// exact because the sum is a multiple of 256 or 16 and stays inside int32
// for the K bounds the API enforces.
//
// The widening splits even and odd elements into separate dwords, so the
// matrix instruction sees K in a permuted order.  A sum over K does not
// depend on the order as long as both operands use the same one: an int4 x
// int4 product widens both sides identically, and an int8 operand facing an
// int4 one is permuted the same way with v_perm_b32 (even_odd_split).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));

// 8 packed bytes (16 int4 values, dwords p.x = values 0..7, p.y = 8..15)
// -> 16 int8 bytes in the order [0,2,4,6 | 1,3,5,7 | 8,10,12,14 | 9,11,13,15],
// each value scaled by 16.
__device__ __forceinline__ v4i widen_int4_x16(v2u p)
{
    v4i r;
    r[0] = (int)((p.x << 4) & 0xF0F0F0F0u);
    r[1] = (int)(p.x & 0xF0F0F0F0u);
    r[2] = (int)((p.y << 4) & 0xF0F0F0F0u);
    r[3] = (int)(p.y & 0xF0F0F0F0u);
    return r;
}

// 16 int8 bytes in natural order -> the same permutation widen_int4_x16
// produces: [0,2,4,6 | 1,3,5,7 | 8,10,12,14 | 9,11,13,15].
// v_perm_b32 picks bytes of the 64-bit {src0, src1} (src1 = bytes 0..3).
// MSB: the int4 operand is packed high nibble first (INT4 GEMM article §3.2's
// other order), so widen_int4_x16's low-nibble dwords hold the odd elements;
// the int8 side then takes [1,3,5,7 | 0,2,4,6 | ...] instead, which costs
// nothing.
template <bool MSB = false>
__device__ __forceinline__ v4i even_odd_split(v4i q)
{
    constexpr unsigned kFirst = MSB ? 0x07050301u : 0x06040200u;
    constexpr unsigned kSecond = MSB ? 0x06040200u : 0x07050301u;
    v4i r;
    r[0] = (int)__builtin_amdgcn_perm((unsigned)q[1], (unsigned)q[0], kFirst);
    r[1] = (int)__builtin_amdgcn_perm((unsigned)q[1], (unsigned)q[0], kSecond);
    r[2] = (int)__builtin_amdgcn_perm((unsigned)q[3], (unsigned)q[2], kFirst);
    r[3] = (int)__builtin_amdgcn_perm((unsigned)q[3], (unsigned)q[2], kSecond);
    return r;
}

// Q31 requantize of one accumulator (MCU conv front-end article,
// news.rkmt.cn/news/16638, §2.3): x = acc + bias, t = x * mult (64-bit),
// t += 2^(shift-1), t >>= shift (arithmetic), then the output zero point zo
// (that article's §3.3; 0 for symmetric outputs) and saturation to
// [lo, hi]: the int8 range, or tighter bounds for a fused activation (ReLU is
// lo = zo; Voyager quantization article, www.dpshk.com/news/2695434, §3.1).
// `rnd` is 2^(shift-1), computed once per channel by the caller.  acc + bias
// is formed modulo 2^32: the asymmetric forms pass accumulators whose
// compensation terms may wrap, and the true x fits in int32.  y + zo is
// saturated as y clamped to [lo - zo, hi - zo], plus zo.
// The 64-bit quotient is saturated from its two halves: when the high word is
// not the sign extension of the low word, |y| >= 2^31 and the result is the
// bound on y's side whatever zo is.
__device__ __forceinline__ int wrap_add(int a, int b)
{
    return (int)((unsigned)a + (unsigned)b);
}

__device__ __forceinline__ int wrap_sub(int a, int b)
{
    return (int)((unsigned)a - (unsigned)b);
}

__device__ __forceinline__ int requant_one(int acc, int bias, int mult, int shift, long long rnd,
                                           int zo = 0, int lo = -128, int hi = 127)
{
    const int x = wrap_add(acc, bias);
    const long long y = ((long long)x * (long long)mult + rnd) >> shift;
    const int ylo = (int)y, yhi = (int)(y >> 32);
    const int c = min(max(ylo, lo - zo), hi - zo) + zo;
    return yhi == (ylo >> 31) ? c : (yhi < 0 ? lo : hi);
}

// The same when shift >= 31: |x * mult| < 2^62 then keeps y inside int32, so
// the low word of the 64-bit shift is y itself.
__device__ __forceinline__ int requant_one_s31(int acc, int bias, int mult, int shift,
                                               long long rnd, int zo = 0, int lo = -128,
                                               int hi = 127)
{
    const int x = wrap_add(acc, bias);
    const int y = (int)(((long long)x * (long long)mult + rnd) >> shift);
    return min(max(y, lo - zo), hi - zo) + zo;
}

// The same when shift >= 33: with x * mult = H * 2^32 + L (0 <= L < 2^32,
// H the high word of the signed product), t / 2^shift =
// (H + 2^(shift-33) + L / 2^32) / 2^(shift-32), and the fraction L / 2^32
// never changes the floor, so y = (H + 2^(shift-33)) >> (shift-32) exactly.
// |H| <= 2^30, so the sum stays inside int32.
__device__ __forceinline__ int requant_one_s33(int acc, int bias, int mult, int shift, int zo = 0,
                                               int lo = -128, int hi = 127)
{
    const int x = wrap_add(acc, bias);
    const int h = __mulhi(x, mult);
    const int y = (h + (1 << ((shift - 33) & 31))) >> ((shift - 32) & 31);
    return min(max(y, lo - zo), hi - zo) + zo;
}

// binary16 bits of a binary32 value, rounded to nearest even.  The empty asm
// pins u as a binary32 register value: without it the compiler folds the
// product that produced u into v_fma_mixlo_f16, which rounds once (to
// binary16) where the definition rounds twice (to binary32, then binary16).
__device__ __forceinline__ unsigned short f32_to_f16_bits(float u)
{
    asm volatile("" : "+v"(u));
    return __builtin_bit_cast(unsigned short, (_Float16)u);
}

// One 16-byte direct-to-LDS load per lane through a raw buffer resource:
// lane L reads base + voff + soff (voff per lane, soff uniform) and writes
// LDS at lds + 16 L.  Reads at or past `nbytes` return zeros.  The resource
// is a scalar value the compiler builds once; a per-lane 32-bit offset costs
// one VGPR and no address arithmetic, where a flat 64-bit address costs a
// VGPR pair and a 64-bit add per load.
__device__ __forceinline__ void buffer_load_lds16(const void *base, uint32_t nbytes,
                                                  uint32_t voff, uint32_t soff, void *lds)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)nbytes,
                                          0x00020000),
        (__attribute__((address_space(3))) void *)lds, 16, voff, soff, 0, 0);
}

__device__ __forceinline__ unsigned pack4_i8(int a, int b, int c, int d)
{
    return (unsigned)(a & 0xFF) | ((unsigned)(b & 0xFF) << 8) | ((unsigned)(c & 0xFF) << 16) |
           ((unsigned)(d & 0xFF) << 24);
}

// Workgroups are dispatched round-robin over the 8 XCDs of an MI355X, each
// with its own L2.  Renumber them so that consecutive tile ids land on the
// same XCD: XCD x runs ids [x * per, (x + 1) * per) (the first nwg % 8 XCDs
// take one more).  Neighbouring tiles then share A/B panels in one L2.
__device__ __forceinline__ int xcd_remap(int bid, int nwg)
{
    constexpr int NXCD = 8;
    int xcd = bid % NXCD;
    int slot = bid / NXCD;
    int per = nwg / NXCD;
    int rem = nwg % NXCD;
    return xcd < rem ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
}

}  // namespace qg
