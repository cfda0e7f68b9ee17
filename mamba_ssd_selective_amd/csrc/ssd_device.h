// ssd_device.h -- device functions shared by every SSD kernel (gfx950, wave64).
//
// The chunked prefill path and the single-token decode path use the same
// per-token arithmetic from here (RL-Kernel RFC "Nemotron-3-Nano-30B-A3B",
// section 7: train/prefill and decode of the Mamba-2 mixer must share device
// functions): the dt transform of section 3 Figure 2 box [F2]
// (softplus(dt + dt_bias), dt_limit), the decay exp(dt * A), the bf16 <-> fp32
// conversions and the head -> B/C group map.
//
// MFMA conventions (one 16x16 output tile per wave, K = 32 per step):
//   lane l, r16 = l & 15, q = l >> 4
//   A operand: row r16, eight k values k(q, e) = 8q + e, e = 0..7
//   B operand: column r16, the same eight k values
//   accumulator: rows 4q + i (i = 0..3), column r16
// Any bijection between (q, e) and the 32 logical k indices is allowed as
// long as A and B use the same one; the kernels use two of them (contiguous
// runs of 8, or two runs of 4) to feed accumulators back in as operands.
// bf16 uses one v_mfma_f32_16x16x32_bf16; fp32 uses eight v_mfma_f32_16x16x4_f32
// (sub-step e takes element e of every lane, so the k mapping is the same).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace ssd {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ----------------------------------------------------------------- scalars

__device__ __forceinline__ float bf16_to_f32(uint16_t u) {
    return __uint_as_float(static_cast<uint32_t>(u) << 16);
}

// Round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// log(1 + e^v) without overflow.
__device__ __forceinline__ float softplus_f32(float v) {
    return fmaxf(v, 0.0f) + log1pf(expf(-fabsf(v)));
}

// dt_t = clamp(softplus(dt_raw + dt_bias), dt_min, dt_max)   (box [F2])
__device__ __forceinline__ float dt_transform(float raw, float bias, int softplus,
                                              float dt_min, float dt_max) {
    float v = raw + bias;
    if (softplus) v = softplus_f32(v);
    return fminf(fmaxf(v, dt_min), dt_max);
}

// exp of a non-positive log-decay (a difference of running sums, or dt * A).
__device__ __forceinline__ float decay_exp(float log_decay) { return __expf(log_decay); }

__device__ __forceinline__ int group_of_head(int h, int heads_per_group) {
    return h / heads_per_group;
}

// ------------------------------------------------------------ io element types

template <typename T> struct Io;

template <> struct Io<float> {
    static constexpr int kVec = 4;  // elements per 16 bytes
    __device__ static __forceinline__ float to_f32(float v) { return v; }
    __device__ static __forceinline__ float from_f32(float v) { return v; }
};

template <> struct Io<uint16_t> {
    static constexpr int kVec = 8;
    __device__ static __forceinline__ float to_f32(uint16_t v) { return bf16_to_f32(v); }
    __device__ static __forceinline__ uint16_t from_f32(float v) { return f32_to_bf16(v); }
};

// 16-byte vector of io elements.
template <typename T> struct Vec16 { T v[16 / sizeof(T)]; };

template <typename T>
__device__ __forceinline__ Vec16<T> load16(const T* p) {
    uint4 u = *reinterpret_cast<const uint4*>(p);
    return __builtin_bit_cast(Vec16<T>, u);
}
template <typename T>
__device__ __forceinline__ void store16(T* p, const Vec16<T>& v) {
    *reinterpret_cast<uint4*>(p) = __builtin_bit_cast(uint4, v);
}
template <typename T>
__device__ __forceinline__ Vec16<T> zero16() {
    return __builtin_bit_cast(Vec16<T>, make_uint4(0, 0, 0, 0));
}

// Four consecutive io elements (8 bytes bf16, 16 bytes fp32).
template <typename T> struct Vec4 { T v[4]; };

template <typename T>
__device__ __forceinline__ Vec4<T> load4(const T* p) {
    if constexpr (sizeof(T) == 2) {
        return __builtin_bit_cast(Vec4<T>, *reinterpret_cast<const uint2*>(p));
    } else {
        return __builtin_bit_cast(Vec4<T>, *reinterpret_cast<const uint4*>(p));
    }
}
template <typename T>
__device__ __forceinline__ void store4(T* p, const Vec4<T>& v) {
    if constexpr (sizeof(T) == 2) {
        *reinterpret_cast<uint2*>(p) = __builtin_bit_cast(uint2, v);
    } else {
        *reinterpret_cast<uint4*>(p) = __builtin_bit_cast(uint4, v);
    }
}

// --------------------------------------------------------- raw 16-byte vectors
// Global tiles are moved as raw uint4 (16 bytes) so that a load never has to
// complete before the code that issued it moves on; elements are unpacked only
// where they are used.

__device__ __forceinline__ uint4 ld_raw16(const void* p) {
    return *reinterpret_cast<const uint4*>(p);
}
// the same 16 bytes from a 4-byte aligned address
__device__ __forceinline__ uint4 ld_words16(const void* p) {
    const uint32_t* w = static_cast<const uint32_t*>(p);
    return make_uint4(w[0], w[1], w[2], w[3]);
}
__device__ __forceinline__ uint4 raw_keep(bool keep, const uint4& v) {
    return make_uint4(keep ? v.x : 0u, keep ? v.y : 0u, keep ? v.z : 0u, keep ? v.w : 0u);
}
template <int I>
__device__ __forceinline__ uint32_t u4_at(const uint4& v) {
    static_assert(I >= 0 && I < 4, "dword index");
    if constexpr (I == 0) return v.x;
    else if constexpr (I == 1) return v.y;
    else if constexpr (I == 2) return v.z;
    else return v.w;
}

// Element E of a raw 16-byte vector of io elements, as fp32.
template <typename T, int E>
__device__ __forceinline__ float raw_elem_f32(const uint4& v) {
    if constexpr (sizeof(T) == 2) {
        const uint32_t d = u4_at<E / 2>(v);
        return __uint_as_float((E % 2 == 0) ? (d << 16) : (d & 0xFFFF0000u));
    } else {
        return __uint_as_float(u4_at<E>(v));
    }
}

// Element E (< 4) of four packed bf16 values.
template <typename T, int E>
__device__ __forceinline__ float raw_elem_f32(const uint2& v) {
    static_assert(sizeof(T) == 2, "uint2 holds four 16-bit elements");
    const uint32_t d = E < 2 ? v.x : v.y;
    return __uint_as_float((E % 2 == 0) ? (d << 16) : (d & 0xFFFF0000u));
}

// Two fp32 values -> packed bf16 pair (RNE), low half first.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    bf16x2_t v;
    v[0] = static_cast<__bf16>(lo);
    v[1] = static_cast<__bf16>(hi);
    return __builtin_bit_cast(uint32_t, v);
}

// Store four fp32 values as four consecutive io elements (8 or 16 bytes).
template <typename T>
__device__ __forceinline__ void store4_f32(T* p, float a, float b, float c, float d) {
    if constexpr (sizeof(T) == 2) {
        *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
    } else {
        *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
    }
}

// Column E of a 4-row x (16 bytes) block: the four elements rows[0..3][E],
// stored as four consecutive io elements.
template <typename T, int E>
__device__ __forceinline__ void store_col4(T* p, const uint4 (&rows)[4]) {
    if constexpr (sizeof(T) == 2) {
        // v_perm_b32 byte selectors: low halves {0,1 | 4,5}, high halves {2,3 | 6,7}
        constexpr uint32_t sel = (E % 2 == 0) ? 0x05040100u : 0x07060302u;
        const uint32_t lo = __builtin_amdgcn_perm(u4_at<E / 2>(rows[1]), u4_at<E / 2>(rows[0]), sel);
        const uint32_t hi = __builtin_amdgcn_perm(u4_at<E / 2>(rows[3]), u4_at<E / 2>(rows[2]), sel);
        *reinterpret_cast<uint2*>(p) = make_uint2(lo, hi);
    } else {
        *reinterpret_cast<uint4*>(p) =
            make_uint4(u4_at<E>(rows[0]), u4_at<E>(rows[1]), u4_at<E>(rows[2]), u4_at<E>(rows[3]));
    }
}

// ------------------------------------------------------------------ fragments

template <typename T> struct Frag;

template <> struct Frag<uint16_t> {
    bf16x8_t v;
};
template <> struct Frag<float> {
    float v[8];
};

// A fragment's worth of raw bytes (16 for bf16, 32 for fp32), loaded without
// waiting; turned into a Frag where it is used.
template <typename T> struct RawFrag {
    uint4 r[sizeof(T) == 2 ? 1 : 2];
};
template <typename T>
__device__ __forceinline__ RawFrag<T> raw_frag_load8(const T* p) {
    RawFrag<T> f;
    f.r[0] = ld_raw16(p);
    if constexpr (sizeof(T) == 4) f.r[1] = ld_raw16(p + 4);
    return f;
}
template <typename T>
__device__ __forceinline__ Frag<T> frag_from_raw(const RawFrag<T>& f, bool keep) {
    Frag<T> out;
    if constexpr (sizeof(T) == 2) {
        out.v = __builtin_bit_cast(bf16x8_t, raw_keep(keep, f.r[0]));
    } else {
        const uint4 a = raw_keep(keep, f.r[0]), b = raw_keep(keep, f.r[1]);
        out.v[0] = __uint_as_float(a.x); out.v[1] = __uint_as_float(a.y);
        out.v[2] = __uint_as_float(a.z); out.v[3] = __uint_as_float(a.w);
        out.v[4] = __uint_as_float(b.x); out.v[5] = __uint_as_float(b.y);
        out.v[6] = __uint_as_float(b.z); out.v[7] = __uint_as_float(b.w);
    }
    return out;
}

// Eight consecutive elements (k = 8q + e) from LDS or global memory.
template <typename T>
__device__ __forceinline__ Frag<T> frag_load8(const T* p) {
    Frag<T> f;
    if constexpr (sizeof(T) == 2) {
        f.v = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(p));
    } else {
        float4 a = *reinterpret_cast<const float4*>(p);
        float4 b = *reinterpret_cast<const float4*>(p + 4);
        f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
        f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
    }
    return f;
}

template <typename T>
__device__ __forceinline__ Frag<T> frag_zero() {
    Frag<T> f;
    if constexpr (sizeof(T) == 2) {
        f.v = __builtin_bit_cast(bf16x8_t, make_uint4(0, 0, 0, 0));
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) f.v[e] = 0.0f;
    }
    return f;
}

// Two runs of four (elements 0..3 from p0, 4..7 from p1).
template <typename T>
__device__ __forceinline__ Frag<T> frag_load4x2(const T* p0, const T* p1) {
    Frag<T> f;
    if constexpr (sizeof(T) == 2) {
        uint2 a = *reinterpret_cast<const uint2*>(p0);
        uint2 b = *reinterpret_cast<const uint2*>(p1);
        f.v = __builtin_bit_cast(bf16x8_t, make_uint4(a.x, a.y, b.x, b.y));
    } else {
        float4 a = *reinterpret_cast<const float4*>(p0);
        float4 b = *reinterpret_cast<const float4*>(p1);
        f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
        f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
    }
    return f;
}

// Eight fp32 values rounded to the operand type (one rounding, RNE).
template <typename T>
__device__ __forceinline__ Frag<T> frag_from_f32(const float (&x)[8]) {
    Frag<T> f;
    if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int e = 0; e < 8; ++e) f.v[e] = static_cast<__bf16>(x[e]);
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) f.v[e] = x[e];
    }
    return f;
}

__device__ __forceinline__ void mma(f32x4_t& acc, const Frag<uint16_t>& a,
                                    const Frag<uint16_t>& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}

__device__ __forceinline__ void mma(f32x4_t& acc, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], acc, 0, 0, 0);
}

__device__ __forceinline__ f32x4_t acc_zero() { return f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}; }

// ----------------------------------------------------------- wave primitives

// Cross-lane sums on VALU moves: DPP within a 16-lane row, the permlane swaps
// across rows, in place of LDS permutes (ds_bpermute, one trip through the LDS
// unit per step).  Each step adds to every lane the value of a partner; where
// that partner is not the xor butterfly's, the two hold the same value at that
// step, so the sums are the butterfly's, bit for bit.
template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), kCtrl, 0xF, 0xF, false));
}
// v + v of lane ^ 16 (rows 0/1 and 2/3 trade places), then the same with ^ 32
__device__ __forceinline__ float add_lane_xor16(float v) {
    const uint32_t u = __float_as_uint(v);
    const auto s = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}
__device__ __forceinline__ float add_lane_xor32(float v) {
    const uint32_t u = __float_as_uint(v);
    const auto s = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}
// Sum over each 16-lane row, the butterfly over offsets 1, 2, 4, 8.
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_f32<0xB1>(v);   // quad_perm [1,0,3,2]: lane ^ 1
    v += dpp_f32<0x4E>(v);   // quad_perm [2,3,0,1]: lane ^ 2
    v += dpp_f32<0x141>(v);  // row_half_mirror: a lane of the other quad of the half row
    v += dpp_f32<0x140>(v);  // row_mirror: a lane of the other half of the row
    return v;
}
// Sum over the wave, the butterfly over offsets 1, 2, ..., 32.
__device__ __forceinline__ float wave_sum(float v) {
    return add_lane_xor32(add_lane_xor16(row16_sum(v)));
}
// Sum over aligned groups of kG lanes (a power of two, 2..64), the butterfly
// from the widest offset down: kG / 2, ..., 2, 1.
template <int kG>
__device__ __forceinline__ float group_sum_wide_first(float v) {
    static_assert(kG >= 2 && kG <= 64 && (kG & (kG - 1)) == 0, "group size");
    if constexpr (kG >= 64) v = add_lane_xor32(v);
    if constexpr (kG >= 32) v = add_lane_xor16(v);
    if constexpr (kG >= 16) {
        v += dpp_f32<0x128>(v);  // row_ror:8: lane ^ 8
        v += dpp_f32<0x124>(v);  // row_ror:4: a lane equal to lane ^ 4 after the step above
    } else if constexpr (kG == 8) {
        v += __shfl_xor(v, 4, kWave);  // the first step: no DPP move gives lane ^ 4
    }
    if constexpr (kG >= 4) v += dpp_f32<0x4E>(v);  // lane ^ 2
    v += dpp_f32<0xB1>(v);                          // lane ^ 1
    return v;
}

// Inclusive segmented scan over the 64 lanes: a set `head` flag starts a new
// segment at that lane.  Fixed tree order (deterministic).
__device__ __forceinline__ float wave_segmented_scan(float v, int head) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        float pv = __shfl_up(v, d, kWave);
        int ph = __shfl_up(head, d, kWave);
        if (lane >= d && !head) {
            v = pv + v;
            head = ph;
        }
    }
    return v;
}

}  // namespace ssd
