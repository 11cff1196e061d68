// os_device.hpp -- device building blocks for the gfx950 (CDNA4, wave64)
// softmax kernels: the normaliser state and its merge, cross-lane reductions
// on DPP and the gfx950 permlane swaps, 128-bit loads and stores, and bf16
// packing.
//
// The state (m, d) and the merge follow "OnlineSoftmax: Online normalizer
// calculation for softmax" (paper summary), sections 3.1 and 3.3.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace onorm {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.44269504088896340736f;
// Start value of every running maximum: -FLT_MAX rather than -inf, so that
// differences of two maxima are never inf - inf (a NaN).  On every state a
// kernel can build, (kFloor, 0) behaves exactly as the identity (-inf, 0):
// max(m, kFloor) = m for any m >= kFloor, and its d = 0 adds nothing.  A
// -inf input still contributes e^{-inf - m} = 0.
constexpr float kFloor = -3.40282346638528859812e+38f;

// e^t as 2^(t * log2 e) on the hardware base-2 exponential (v_exp_f32).
// Callers form t = x - m first, so the rounding of the product stays
// relative to the small difference, not to |x|.
__device__ __forceinline__ float exp_e(float t) { return __builtin_amdgcn_exp2f(t * kLog2e); }

__device__ __forceinline__ float rcp(float v) { return __builtin_amdgcn_rcpf(v); }

constexpr float kLn2 = 0.693147180559945309417f;
// m + ln(d) as one fused multiply-add on the hardware base-2 logarithm
// (v_log_f32): ln d = log2(d) * ln 2.  Callers pass d >= 1 (a normal number).
__device__ __forceinline__ float add_log_e(float m, float d) { return fmaf(__builtin_amdgcn_logf(d), kLn2, m); }

// ---------------------------------------------------------------------------
// The normaliser state and the merge (+).
// ---------------------------------------------------------------------------
struct State {
    float m;  // running maximum
    float d;  // sum of e^{x - m} over the elements folded so far
};

// (m1,d1) (+) (m2,d2) = (max, d_big + d_small * e^{m_small - m_big}).
// This is the paper summary's two-exponential form with the factor
// e^{m_big - max} = 1 dropped, so one exponential per merge.  It is exactly
// symmetric in its operands (same bits either way round), which keeps every
// lane of a butterfly reduction bit-identical.
__device__ __forceinline__ State oplus(State a, State b) {
    const float hi = fmaxf(a.m, b.m);
    const float s = exp_e(-fabsf(a.m - b.m));
    const float d = (a.m >= b.m) ? fmaf(b.d, s, a.d) : fmaf(a.d, s, b.d);
    return {hi, d};
}

// ---------------------------------------------------------------------------
// Cross-lane data movement.
// ---------------------------------------------------------------------------
enum : int {
    kDppXor1 = 0xB1,        // quad_perm [1,0,3,2]
    kDppXor2 = 0x4E,        // quad_perm [2,3,0,1]
    kDppHalfMirror = 0x141, // row_half_mirror: lane i <-> 7-i within 8
    kDppMirror = 0x140,     // row_mirror: lane i <-> 15-i within 16
    kDppWaveShr1 = 0x138,   // wave_shr:1, lane i reads lane i-1
    kDppRev4 = 0x1B,        // quad_perm [3,2,1,0]: lane i <-> 3-i within 4
    kDppRowShl4 = 0x104,    // row_shl:4, lane i reads lane i+4 within its row of 16
    kDppRowShr4 = 0x114,    // row_shr:4, lane i reads lane i-4 within its row of 16
    kDppRowRor8 = 0x128,    // row_ror:8, lane i reads lane i^8 within its row of 16
};

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(
        __builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, 0xF, 0xF, false));
}

template <int CTRL>
__device__ __forceinline__ int dpp(int v) {
    return __builtin_amdgcn_update_dpp(v, v, CTRL, 0xF, 0xF, false);
}

// The value held by lane (lane ^ MASK), for the masks the sorting networks
// use: DPP where the partner sits in the same row of 16, ds_bpermute (the LDS
// crossbar, no memory access) otherwise.
template <int MASK>
__device__ __forceinline__ int lane_xor(int v, int lane) {
    if constexpr (MASK == 0) return v;
    else if constexpr (MASK == 1) return dpp<kDppXor1>(v);
    else if constexpr (MASK == 2) return dpp<kDppXor2>(v);
    else if constexpr (MASK == 3) return dpp<kDppRev4>(v);
    else if constexpr (MASK == 4) {
        const int up = dpp<kDppRowShl4>(v);
        const int down = dpp<kDppRowShr4>(v);
        return (lane & 4) ? down : up;
    } else if constexpr (MASK == 7) return dpp<kDppHalfMirror>(v);
    else if constexpr (MASK == 8) return dpp<kDppRowRor8>(v);
    else if constexpr (MASK == 15) return dpp<kDppMirror>(v);
    else return __builtin_amdgcn_ds_bpermute((lane ^ MASK) << 2, v);
}

template <int MASK>
__device__ __forceinline__ float lane_xor(float v, int lane) {
    return __int_as_float(lane_xor<MASK>(__float_as_int(v), lane));
}

// v_permlane16_swap: returns {own row's copy, partner row's copy} so that
// every lane of row pair (0,1) or (2,3) sees the values of both rows at its
// position within the row.
__device__ __forceinline__ f32x2 swap_rows16(float v) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return f32x2{__uint_as_float(r[0]), __uint_as_float(r[1])};
}

// v_permlane32_swap: the same between the two 32-lane halves.
__device__ __forceinline__ f32x2 swap_rows32(float v) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return f32x2{__uint_as_float(r[0]), __uint_as_float(r[1])};
}

// Maximum / sum over an aligned group of G lanes (1..64), same bits in every lane.
template <int G>
__device__ __forceinline__ float group_max(float v) {
    if constexpr (G >= 2) v = fmaxf(v, dpp<kDppXor1>(v));
    if constexpr (G >= 4) v = fmaxf(v, dpp<kDppXor2>(v));
    if constexpr (G >= 8) v = fmaxf(v, dpp<kDppHalfMirror>(v));
    if constexpr (G >= 16) v = fmaxf(v, dpp<kDppMirror>(v));
    if constexpr (G >= 32) {
        const f32x2 t = swap_rows16(v);
        v = fmaxf(t[0], t[1]);
    }
    if constexpr (G >= 64) {
        const f32x2 t = swap_rows32(v);
        v = fmaxf(t[0], t[1]);
    }
    return v;
}

template <int G>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (G >= 2) v = v + dpp<kDppXor1>(v);
    if constexpr (G >= 4) v = v + dpp<kDppXor2>(v);
    if constexpr (G >= 8) v = v + dpp<kDppHalfMirror>(v);
    if constexpr (G >= 16) v = v + dpp<kDppMirror>(v);
    if constexpr (G >= 32) {
        const f32x2 t = swap_rows16(v);
        v = t[0] + t[1];
    }
    if constexpr (G >= 64) {
        const f32x2 t = swap_rows32(v);
        v = t[0] + t[1];
    }
    return v;
}

// (+) over the G lane states of a group, applied to all G operands at once:
// m = max_l m_l, d = sum_l d_l e^{m_l - m}.  By associativity and
// commutativity this equals any bracketing of the binary operator; it costs
// one exponential per lane plus a max and a sum reduction, instead of one
// exponential and a select per butterfly step.
template <int G>
__device__ __forceinline__ State group_merge(State s) {
    const float m = group_max<G>(s.m);
    return State{m, group_sum<G>(s.d * exp_e(s.m - m))};
}

// Plain maximum / sum over the whole wave (for the three-pass baseline and
// the top-K threshold); every lane ends with the same bits.
__device__ __forceinline__ float wave_max(float v) { return group_max<64>(v); }
__device__ __forceinline__ float wave_sum(float v) { return group_sum<64>(v); }

__device__ __forceinline__ float readlane(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}
__device__ __forceinline__ int readlane(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }

// ---------------------------------------------------------------------------
// Buffer access.  Every kernel reads and writes through a buffer resource
// that covers exactly the bytes it may touch (one row, or one copy tile).
// The hardware range check turns out-of-range loads into 0 and drops
// out-of-range stores, so tails need no branches; loads therefore issue
// back to back instead of each waiting behind a bounds-check branch.
// Offsets are 32-bit bytes; every resource spans at most 2^30 bytes (rows
// are at most 2^28 elements), so offset 2^31 is always outside.
// ---------------------------------------------------------------------------
constexpr int kBufferWord3 = 0x00020000;  // gfx9-family raw buffer: 32-bit data format
constexpr int kNonTemporal = 2;           // cache-policy bit: streaming (nt)

struct Buf {
    __amdgpu_buffer_rsrc_t r;
    __device__ __forceinline__ Buf(const void* base, uint32_t bytes)
        : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                              kBufferWord3)) {}
    // STREAM = true: data touched once (non-temporal).  A pass whose data is
    // read again later uses plain loads so the re-read can hit in cache.
    template <bool STREAM>
    __device__ __forceinline__ u32x4 load16(uint32_t off) const {
        return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, STREAM ? kNonTemporal : 0);
    }
    __device__ __forceinline__ uint32_t load4(uint32_t off) const {
        return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
    }
    __device__ __forceinline__ uint16_t load2(uint32_t off) const {
        return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
    }
    __device__ __forceinline__ void store16(uint32_t off, u32x4 v) const {
        __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kNonTemporal);
    }
    __device__ __forceinline__ void store4(uint32_t off, uint32_t v) const {
        __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, 0);
    }
    __device__ __forceinline__ void store2(uint32_t off, uint16_t v) const {
        __builtin_amdgcn_raw_buffer_store_b16(v, r, off, 0, 0);
    }
};

// ---------------------------------------------------------------------------
// Element access.  A 16-byte vector holds 4 fp32 or 8 bf16 values.
// ---------------------------------------------------------------------------
template <bool BF16>
struct Elt;

template <>
struct Elt<false> {
    static constexpr int kVec = 4;
    static constexpr int kSize = 4;
    __device__ static __forceinline__ void unpack(u32x4 r, float* v) {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(r[i]);
    }
    __device__ static __forceinline__ u32x4 pack(const float* v) {
        return u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                     __float_as_uint(v[3])};
    }
    // byte offsets; an offset outside the resource reads 0 / is dropped
    __device__ static __forceinline__ float load1(const Buf& b, uint32_t off) {
        return __uint_as_float(b.load4(off));
    }
    __device__ static __forceinline__ void store1(const Buf& b, uint32_t off, float v) {
        b.store4(off, __float_as_uint(v));
    }
};

// bf16 -> fp32 is exact (the bf16 bits are the top half of the fp32 word);
// fp32 -> bf16 rounds to nearest-even in hardware (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2 f = {lo, hi};
    const bf16x2 b = __builtin_convertvector(f, bf16x2);
    return __builtin_bit_cast(uint32_t, b);
}

template <>
struct Elt<true> {
    static constexpr int kVec = 8;
    static constexpr int kSize = 2;
    __device__ static __forceinline__ void unpack(u32x4 r, float* v) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(r[i] << 16);
            v[2 * i + 1] = __uint_as_float(r[i] & 0xFFFF0000u);
        }
    }
    __device__ static __forceinline__ u32x4 pack(const float* v) {
        return u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                     pack_bf16x2(v[6], v[7])};
    }
    __device__ static __forceinline__ float load1(const Buf& b, uint32_t off) {
        return __uint_as_float(static_cast<uint32_t>(b.load2(off)) << 16);
    }
    __device__ static __forceinline__ void store1(const Buf& b, uint32_t off, float v) {
        b.store2(off, static_cast<uint16_t>(pack_bf16x2(v, 0.0f) & 0xFFFFu));
    }
};

}  // namespace onorm
