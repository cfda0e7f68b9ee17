// ssd_lds.h -- LDS layouts and accessors shared by the bf16 MFMA kernels of
// the scan (ssd_scan_tr.hip) and of its gradients (ssd_bwd.hip): swizzled
// [row][column] tiles that serve both plain and transposing
// (ds_read_b64_tr_b16) reads, accesses at 32-bit LDS addresses, and the
// operand fragments built from them.  Internal to libssd.so.
#pragma once

#include "ssd_device.h"

#define SSD_LDS __attribute__((address_space(3)))
#define SSD_GLOBAL __attribute__((address_space(1)))

namespace ssd {

// Word 3 of a raw (unswizzled, untyped) buffer resource on gfx9-family GPUs.
constexpr int kRawBufferWord3 = 0x00020000;
// s_waitcnt immediate: vmcnt(0), expcnt and lgkmcnt left at their maximum.
constexpr int kWaitVmcnt0 = 0x0F70;
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 16, "vmcnt immediate");
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0 | N);
}

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- LDS layout

// Tiles read by transposing reads: 32-byte unit u of row r is stored at unit
// u ^ tr_swz(r).  Sixteen lanes of one such read cover four consecutive rows
// (32 bytes each), 32 lanes eight rows; the swizzle puts them on distinct
// banks for either phase width.
template <int ROW>
__device__ __forceinline__ int tr_swz(int r) {
    if constexpr (ROW == 128) return (r & 3) ^ ((r >> 2) & 1);
    else return r & 7;
}
template <int ROW>
__device__ __forceinline__ int tr_off(int r, int byte_col) {
    return r * ROW + (((byte_col >> 5) ^ tr_swz<ROW>(r)) << 5) + (byte_col & 31);
}

// LDS accesses at 32-bit LDS byte addresses.  Lane-dependent addresses are
// computed once per workgroup and kept opaque to the optimizer (lds_keep), so
// that every access in the chunk loop is one instruction with an immediate
// offset instead of re-deriving its address.  Each access is formed inside
// the __shared__ object it touches (lds_at): the compiler then still knows
// that it does not alias copies in flight into the other buffers, and inserts
// no wait for them.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return static_cast<uint32_t>(reinterpret_cast<size_t>((const SSD_LDS char*)p));
}
__device__ __forceinline__ uint32_t lds_keep(uint32_t a) {
    asm volatile("" : "+v"(a));
    return a;
}
// A wave-uniform value made opaque at its point of use: what is derived from
// it there (copy destinations, guards) is recomputed by a scalar instruction
// or two instead of being held in scalar registers across the chunk loop.
__device__ __forceinline__ int s_opaque(int v) {
    asm volatile("" : "+s"(v));
    return v;
}
// Pointer into the LDS object `obj` at absolute LDS address a (inside obj).
__device__ __forceinline__ const SSD_LDS char* lds_at(const void* obj, uint32_t a) {
    return (const SSD_LDS char*)obj + (a - lds_addr(obj));
}
__device__ __forceinline__ uint2 ds_tr16(const void* obj, uint32_t a) {
    const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SSD_LDS i16x4_t*)lds_at(obj, a));
    return __builtin_bit_cast(uint2, v);
}
// Loads and stores of 4-, 8- and 16-byte values (as plain vectors of words).
template <int BYTES> struct LdsWords;
template <> struct LdsWords<4> { typedef uint32_t type; };
template <> struct LdsWords<8> { typedef unsigned int type __attribute__((ext_vector_type(2))); };
template <> struct LdsWords<16> { typedef unsigned int type __attribute__((ext_vector_type(4))); };
template <typename T>
__device__ __forceinline__ T lds_ld(const void* obj, uint32_t a) {
    typedef typename LdsWords<sizeof(T)>::type W;
    const W w = *(const SSD_LDS W*)lds_at(obj, a);
    return __builtin_bit_cast(T, w);
}
template <typename T>
__device__ __forceinline__ void lds_st(void* obj, uint32_t a, const T& v) {
    typedef typename LdsWords<sizeof(T)>::type W;
    *(SSD_LDS W*)lds_at(obj, a) = __builtin_bit_cast(W, v);
}

// Lane byte offset of the transposing read of column block mb at k step 0.
// A ds_read_b64_tr_b16 returns to lane i of a 16-lane group element k of the
// 4-element read of lane i/4 + 4k in that group, position i % 4; so lane jj
// of group g reads row 4g + jj/4, columns 16mb + 4(jj % 4) .. +3, and lane i
// receives column 16mb + i of rows 4g .. 4g + 3.
template <int ROW>
__device__ __forceinline__ int tr_lane_off(int mb, int lane) {
    const int g = lane >> 4, jj = lane & 15;
    return tr_off<ROW>(4 * g + (jj >> 2), 32 * mb + 8 * (jj & 3));
}

// Operand fragment of k step s from a [token][column] tile.  The swizzle of
// rows r, r + 16 and r + 32s is the same, so steps are plain row offsets.
template <int ROW>
__device__ __forceinline__ Frag<uint16_t> tr_frag(const void* tile, uint32_t lane_base, int s) {
    const uint2 lo = ds_tr16(tile, lane_base + 32 * s * ROW);
    const uint2 hi = ds_tr16(tile, lane_base + (32 * s + 16) * ROW);
    Frag<uint16_t> f;
    f.v = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
    return f;
}

__device__ __forceinline__ float bf_lo(uint32_t d) { return __uint_as_float(d << 16); }
__device__ __forceinline__ float bf_hi(uint32_t d) { return __uint_as_float(d & 0xFFFF0000u); }

// Fragment elements (token order above) scaled by per-token weights.
__device__ __forceinline__ Frag<uint16_t> scale_frag(const Frag<uint16_t>& f, const float4& w0,
                                                     const float4& w1) {
    const uint4 u = __builtin_bit_cast(uint4, f.v);
    const float v[8] = {bf_lo(u.x) * w0.x, bf_hi(u.x) * w0.y, bf_lo(u.y) * w0.z,
                        bf_hi(u.y) * w0.w, bf_lo(u.z) * w1.x, bf_hi(u.z) * w1.y,
                        bf_lo(u.w) * w1.z, bf_hi(u.w) * w1.w};
    return frag_from_f32<uint16_t>(v);
}

__device__ __forceinline__ Frag<uint16_t> frag_of(const uint4& u) {
    Frag<uint16_t> f;
    f.v = __builtin_bit_cast(bf16x8_t, u);
    return f;
}

}  // namespace ssd
