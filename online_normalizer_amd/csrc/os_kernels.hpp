// os_kernels.hpp -- gfx950 kernels for row-wise softmax with the online
// normalizer ("OnlineSoftmax: Online normalizer calculation for softmax",
// paper summary, sections 3.1-3.3 and 4): the register-resident and streaming
// forwards (optionally writing (m, d) or the logsumexp), the split-row
// forward, the fused softmax + top-K; the three-pass safe-softmax baseline
// (same page, section 2); and two plain copies used as bandwidth references.
//
// Row layout: row-major, stride == cols.  Every kernel moves rows in 16-byte
// vector slots with 128-bit buffer accesses.  A row's slots are the 16-byte
// blocks of memory from a grid origin: the 128-byte line holding its first
// element where a workgroup works on one row at a time (each wavefront then
// moves whole cache lines; a wavefront access that straddles lines costs
// 5-20% on MI355X), else the 16-byte block holding it.  A row whose first
// element lies `ph` elements past its origin has slot vi = elements
// [vi*VEC - ph, vi*VEC - ph + VEC); slots wholly before the row are not
// fetched, and entries outside the row are masked by their index.  ALIGNED
// kernels serve rows whose starts are all 16-byte aligned (an aligned base,
// row bytes a multiple of 16), so every slot is wholly inside or outside the
// row.  Rows are read and written through buffer resources that cover only
// the rows, or the row slice, a workgroup works on, widened to the grid: every
// 16-byte block, or 128-byte line, such a resource covers holds an element of
// the row range, so no access leaves the array's pages (memory is mapped in
// pages, which lines never straddle).  Masked entries read as -inf (e^{-inf}
// adds 0 to any state); stores outside the resource are dropped by the
// hardware, and stores never touch an element outside the row.
#pragma once

#include <climits>

#include "os_device.hpp"

namespace onorm {

constexpr int kTopKMax = 32;
constexpr int kTopKMaxSplits = 16;

// An offset no buffer resource here reaches: accesses there are dropped.
constexpr uint32_t kOutside = 0x80000000u;

// Grid origins: the 16-byte block or the 128-byte line holding a row's first
// element (the value is the mask of the address bits below the origin).
constexpr uint32_t kGrid16 = 15u;
constexpr uint32_t kGrid128 = 127u;

// Where a row sits in its buffer resource: its first element lies `ph`
// elements past the grid origin at byte `blk`.  Slot vi is the block at
// blk + 16 vi; element e of the row is at byte blk + (e + ph) * element size.
struct RowAt {
    uint32_t blk;
    int ph;
};

// A buffer resource's base and size over n elements from element e0 of the
// array at p, widened down to the grid origin (`gmask`) and up to a whole
// 16-byte block; `lead` is the byte offset of element e0 in it.
struct Span {
    const char* base;
    uint32_t bytes;
    uint32_t lead;
};

template <bool BF16>
__device__ __forceinline__ Span span_of(const void* p, int64_t e0, int64_t n, uint32_t gmask) {
    constexpr int SZ = Elt<BF16>::kSize;
    const char* a = static_cast<const char*>(p) + e0 * SZ;
    const uint32_t bytes = static_cast<uint32_t>(n * SZ);
    const uint32_t lead = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(a) & gmask);
    return Span{a - lead, (lead + bytes + 15u) & ~15u, lead};
}

// The row whose first element is at byte `start` of a resource.
template <bool BF16>
__device__ __forceinline__ RowAt row_at(uint32_t start, uint32_t gmask) {
    return RowAt{start & ~gmask, static_cast<int>((start & gmask) / Elt<BF16>::kSize)};
}

// A run of rows that a multi-row workgroup reads through one resource.  On
// the 16-byte grid an ALIGNED row starts its first block exactly, which the
// compiler is told (ph = 0), so no per-slot row-start test survives.
template <bool BF16, bool ALIGNED, bool MULTI>
__device__ __forceinline__ Span rows_span(const void* p, int64_t e0, int64_t n, uint32_t gmask) {
    if constexpr (ALIGNED && MULTI)
        return Span{static_cast<const char*>(p) + e0 * Elt<BF16>::kSize, static_cast<uint32_t>(n * Elt<BF16>::kSize),
                    0u};
    return span_of<BF16>(p, e0, n, MULTI ? kGrid16 : gmask);
}

template <bool BF16, bool ALIGNED, bool MULTI>
__device__ __forceinline__ RowAt rows_row(uint32_t start, uint32_t gmask) {
    if constexpr (ALIGNED && MULTI) return RowAt{start, 0};
    return row_at<BF16>(start, MULTI ? kGrid16 : gmask);
}

// Slots from a row's grid origin to its last element.
template <bool BF16>
__device__ __forceinline__ int slot_count(int cols, int ph) {
    constexpr int VEC = Elt<BF16>::kVec;
    return (cols + ph + VEC - 1) / VEC;
}

// True when in and out rows lie at the same offset within their 16-byte
// blocks (then a slot of the input is a whole block of the output too).
__device__ __forceinline__ bool same_phase(const void* a, const void* b) {
    return ((reinterpret_cast<uintptr_t>(a) ^ reinterpret_cast<uintptr_t>(b)) & 15u) == 0;
}

// Slots that begin before a row's first element lie within the 128 bytes
// before it, so their indices are below 8; every caller steps by at least 8
// slots (on the 16-byte grid only slot 0 can begin before the row), so only a
// lane's first step can meet one and the test is made there alone.
constexpr int kHeadSlots = 8;

// Load VPL slots first, first + stride, ... of row r into x: issue the raw
// 128-bit loads of all of them, fence the scheduler, then unpack.  Without
// the fence the scheduler may sink each load next to its unpack code, and
// every load then waits for the previous one to return.  Slots at or past
// `lim`, slots wholly before the row, and rows that are not live are not
// fetched (their loads go outside the resource); their entries, and
// (unaligned rows) entries outside the row's elements, become -inf.
template <bool BF16, int VPL, bool ALIGNED, bool STREAM, bool SKIP = false>
__device__ __forceinline__ void load_slots(const Buf& b, RowAt r, int first, int stride, int lim, int cols,
                                           bool live, float (&x)[VPL][Elt<BF16>::kVec]) {
    using E = Elt<BF16>;
    constexpr int VEC = E::kVec;
    u32x4 raw[VPL];
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
        const int slot = first + v * stride;
        const bool fetch = live & (slot < lim) & ((v > 0) | (slot * VEC - r.ph > -VEC));
        raw[v] = b.load16<STREAM>(fetch ? r.blk + static_cast<uint32_t>(slot) * 16u : kOutside);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
        // SKIP: first < stride, so a step v >= 1 with v stride >= lim holds
        // no slot of the row in any lane; its entries are left unset (the
        // caller reads none of them)
        if (SKIP && v > 0 && v * stride >= lim) continue;
        E::unpack(raw[v], x[v]);
        const int slot = first + v * stride;
        const int e0 = slot * VEC - r.ph;  // row index of the slot's first entry
        const bool ok = live & (slot < lim) & ((v > 0) | (e0 > -VEC));
        if constexpr (ALIGNED) {
            // e0 is a multiple of VEC: the slot is wholly inside the row or out
#pragma unroll
            for (int k = 0; k < VEC; ++k) x[v][k] = ok ? x[v][k] : -INFINITY;
        } else {
            // only a row's first and last slots are partial: mask entry by
            // entry in a branch the other lanes skip
            if (!(ok & ((v > 0) | (e0 >= 0)) & (e0 + VEC <= cols))) {
#pragma unroll
                for (int k = 0; k < VEC; ++k)
                    x[v][k] =
                        (ok & (static_cast<uint32_t>(e0 + k) < static_cast<uint32_t>(cols))) ? x[v][k] : -INFINITY;
            }
        }
    }
}

// Store slot vi of an input row with phase `ph` (values v[VEC]) to output row
// ro.  Only the row's own elements are written: a slot wholly inside the row
// goes out as one 128-bit store when the output has the input's phase
// (`same`), entries at the row's ends, and every entry when the phases differ,
// element by element.  Slots at or past `lim`, slots wholly before the row
// (possible only where `first_step`, a lane's first step) and rows that are
// not live store nothing.
template <bool BF16, bool ALIGNED>
__device__ __forceinline__ void store_slot(const Buf& b, RowAt ro, int ph, bool same, int vi, int lim, int cols,
                                           bool live, const float* v, bool first_step) {
    using E = Elt<BF16>;
    constexpr int VEC = E::kVec;
    const int e0 = vi * VEC - ph;  // row index of the slot's first entry
    const bool ok = live & (vi < lim) & (!first_step | (e0 > -VEC));
    // with equal 16-byte offsets, element e0 starts a 16-byte block of the
    // output: byte ro.blk + (e0 + ro.ph) * size, a fixed distance from 16 vi
    const uint32_t blk_out =
        ro.blk + static_cast<uint32_t>(ro.ph - ph) * E::kSize + static_cast<uint32_t>(vi) * 16u;
    if constexpr (ALIGNED) {
        b.store16(ok ? blk_out : kOutside, E::pack(v));
    } else {
        if (same) {
            const bool whole = ok & (!first_step | (e0 >= 0)) & (e0 + VEC <= cols);
            b.store16(whole ? blk_out : kOutside, E::pack(v));
            if (ok & !whole) {
#pragma unroll
                for (int k = 0; k < VEC; ++k) {
                    const int e = e0 + k;
                    E::store1(b,
                              static_cast<uint32_t>(e) < static_cast<uint32_t>(cols)
                                  ? ro.blk + static_cast<uint32_t>(e + ro.ph) * E::kSize
                                  : kOutside,
                              v[k]);
                }
            }
        } else {
#pragma unroll
            for (int k = 0; k < VEC; ++k) {
                const int e = e0 + k;
                E::store1(b,
                          (ok & (static_cast<uint32_t>(e) < static_cast<uint32_t>(cols)))
                              ? ro.blk + static_cast<uint32_t>(e + ro.ph) * E::kSize
                              : kOutside,
                          v[k]);
            }
        }
    }
}

// Per-row statistics a forward launch may write besides y; each pointer may
// be null.  m and d: the row's state ((-inf, 0) for an empty or all -inf
// row; m = -inf and d = NaN when the only entries above -inf are NaN).  lse:
// the logsumexp L = m + ln d, -inf for an empty or all -inf row, NaN when d is.
struct RowStats {
    float* m;
    float* d;
    float* lse;
};

__device__ __forceinline__ bool any_stats(const RowStats& o) { return (o.m != nullptr) | (o.lse != nullptr); }

__device__ __forceinline__ void put_stats(const RowStats& o, int64_t row, State s) {
    // d >= 1 exactly whenever an entry above -inf was folded (the maximum
    // contributes e^0), so a start-value maximum with d below 1 (0, or NaN
    // from a NaN entry) means the row had no such entry
    const bool no_entry = (s.m == kFloor) & !(s.d >= 1.0f);
    if (o.m != nullptr) {
        o.m[row] = no_entry ? -INFINITY : s.m;
        o.d[row] = s.d;
    }
    if (o.lse != nullptr) o.lse[row] = s.d == 0.0f ? -INFINITY : add_log_e(s.m, s.d);
}

// ---------------------------------------------------------------------------
// Register-resident forward: the row is read from HBM once.
//
// LPR lanes share a row and each holds VPL vectors of it in VGPRs.  LPR <= 64:
// 256-thread workgroups carry 256/LPR rows and the merge stays inside the
// wavefront.  LPR = 64*W: one row per W-wave workgroup; the W wave states meet
// once in LDS (one barrier per row; the LDS slots alternate between rows so
// the next row's writes never race this row's reads).
//
// Pass 1 per lane (the tile form of the recurrence, with the lane's slice as
// one tile): m_l = max of the slice, e_k = e^{x_k - m_l}, d_l = sum e_k; the
// e_k stay in registers.  The lane states merge with (+).  Pass 2 writes
// y_k = e_k * (e^{m_l - m} / d): one exponential per element in all.
// Writes y when out != nullptr, and the statistics that `st` asks for.
// ---------------------------------------------------------------------------
// Shapes of at most 4 vectors per lane fit in 64 VGPRs, so 8 waves per SIMD
// are requested: two 1024-lane (four 512-lane) workgroups then stay resident
// on a CU, which the register count would otherwise decide by a few
// registers.  Unaligned bf16 rows of 4 vectors on 256 or more lanes, or read
// through LDS (STAGE 2), would spill to fit, and are left to the compiler.
template <bool BF16, int LPR, int VPL, bool ALIGNED, int STAGE>
constexpr int resident_min_waves() {
    return (VPL <= 4 && !(BF16 && !ALIGNED && VPL == 4 && (LPR >= 256 || STAGE == 2))) ? 8 : 1;
}

//
// STAGE (multi-row workgroups on rows that are not 16-byte aligned): the
// workgroup's rows are one contiguous run of the output, so pass 2 assembles
// that run in LDS, with each lane placing only its own row's elements, and the
// workgroup then writes it as whole 16-byte blocks.  Only the run's first and
// last blocks, shared with the neighbouring workgroups, go out element by
// element, instead of every row's two partial slots.  STAGE = 2 also reads the
// input run into LDS as whole blocks first; a lane's slots then start at its
// row's first element (slot vi holds entries vi * VEC ..), so such rows need
// only cols / VEC slots, as aligned rows do, and no row pays a partial slot at
// its front.
//
// MINW > 0 replaces the waves-per-SIMD request (the same code on a tighter
// register budget, so the same results bit for bit).
template <bool BF16, int LPR, int VPL, bool ALIGNED, int STAGE, int MINW = 0>
__global__ void __launch_bounds__(LPR <= 64 ? 256 : LPR,
                                  (MINW > 0 ? MINW : resident_min_waves<BF16, LPR, VPL, ALIGNED, STAGE>()))
    k_resident(const void* in, void* out, RowStats st, int64_t rows, int cols, uint32_t gmask) {
    using E = Elt<BF16>;
    constexpr int VEC = E::kVec;
    constexpr int BLOCK = LPR <= 64 ? 256 : LPR;
    constexpr int RPB = BLOCK / LPR;
    constexpr int W = LPR > 64 ? LPR / 64 : 1;
    constexpr int GROUP = LPR < 64 ? LPR : 64;
    static_assert(STAGE == 0 || (LPR <= 64 && !ALIGNED), "staging is for multi-row unaligned rows");
    // One-row shapes of 128 and 256 lanes skip the vector steps that no lane
    // of the row reaches: the plan gives them rows of half their capacity and
    // up (bf16 rows of 2047 columns on 128 x 4 measured 104.9 -> 92.4 us,
    // 4500 columns on 128 x 8 100.4 -> 96.6 us; bitwise the same results).
    // 512- and 1024-lane shapes are planned with at most one step to spare,
    // and the added branches measured 1-3% slower there.
    constexpr bool kSkip = LPR > 64 && LPR <= 256;
    __shared__ State lds[2][W];
    // the run's bytes: each row spans at most LPR * VPL blocks, and the run
    // starts inside its first block
    __shared__ u32x4 img[STAGE ? RPB * LPR * VPL + 2 : 1];
    char* const ib = reinterpret_cast<char*>(img);

    const int tid = threadIdx.x;
    const int j = tid % LPR;
    const int g = tid / LPR;
    const uint32_t row_bytes = static_cast<uint32_t>(cols) * E::kSize;
    const bool same = same_phase(in, out);
    int par = 0;

    for (int64_t rb = blockIdx.x; rb * RPB < rows; rb += gridDim.x) {
        // One buffer resource per workgroup, over its (up to RPB) rows: the
        // descriptor is uniform, and rows past the end fall outside it.
        const int64_t row0 = rb * RPB;
        const int64_t nrows = (rows - row0) < RPB ? (rows - row0) : RPB;
        const int64_t row = row0 + g;
        const bool live = g < nrows;
        const Span si = rows_span<BF16, ALIGNED, (LPR <= 64)>(in, row0 * cols, nrows * cols, gmask);
        const Buf bin(si.base, si.bytes);
        const RowAt ri = rows_row<BF16, ALIGNED, (LPR <= 64)>(si.lead + static_cast<uint32_t>(g) * row_bytes, gmask);
        const int ns = slot_count<BF16>(cols, ri.ph);

        float x[VPL][VEC];
        if constexpr (STAGE == 2) {
            // the run, as whole blocks, into LDS; then this lane's entries
            const int nbi = static_cast<int>(si.bytes / 16u);
            u32x4 t[VPL + 1];
#pragma unroll
            for (int q = 0; q <= VPL; ++q) {
                const int i = tid + q * BLOCK;
                t[q] = bin.load16<true>(i < nbi ? static_cast<uint32_t>(i) * 16u : kOutside);
            }
#pragma unroll
            for (int q = 0; q <= VPL; ++q)
                if (tid + q * BLOCK < nbi) img[tid + q * BLOCK] = t[q];
            __syncthreads();
            const uint32_t r0 = si.lead + static_cast<uint32_t>(g) * row_bytes;
#pragma unroll
            for (int v = 0; v < VPL; ++v)
#pragma unroll
                for (int k = 0; k < VEC; ++k) {
                    const int e = (v * LPR + j) * VEC + k;
                    const uint32_t at = r0 + static_cast<uint32_t>(e) * E::kSize;
                    float val = -INFINITY;
                    if (live & (e < cols)) {
                        if constexpr (BF16)
                            val = __uint_as_float(static_cast<uint32_t>(*reinterpret_cast<const uint16_t*>(ib + at)) << 16);
                        else
                            val = *reinterpret_cast<const float*>(ib + at);
                    }
                    x[v][k] = val;
                }
            // every lane has its entries: the image may be overwritten
            __syncthreads();
        } else {
            load_slots<BF16, VPL, ALIGNED, true, kSkip>(bin, ri, j, LPR, ns, cols, live, x);
        }

        // One-row workgroups: a vector step that no lane of the row reaches
        // (v LPR >= ns, the same for the whole workgroup) holds only -inf and
        // is skipped; it would add -inf to the maximum and +0 to the sum.
        auto reached = [&](int v) { return !kSkip || v == 0 || v * LPR < ns; };
        float ml = kFloor;
#pragma unroll
        for (int v = 0; v < VPL; ++v)
            if (reached(v)) {
#pragma unroll
                for (int k = 0; k < VEC; ++k) ml = fmaxf(ml, x[v][k]);
            }
        float dl = 0.0f;
#pragma unroll
        for (int v = 0; v < VPL; ++v)
            if (reached(v)) {
#pragma unroll
                for (int k = 0; k < VEC; ++k) {
                    x[v][k] = exp_e(x[v][k] - ml);
                    dl += x[v][k];
                }
            }

        State s = group_merge<GROUP>(State{ml, dl});
        if constexpr (W > 1) {
            if ((tid & (kWave - 1)) == 0) lds[par][tid / kWave] = s;
            __syncthreads();
            s = lds[par][0];
#pragma unroll
            for (int w = 1; w < W; ++w) s = oplus(s, lds[par][w]);
            par ^= 1;
        }

        if (any_stats(st) && live && j == 0) put_stats(st, row, s);
        if (out != nullptr) {
            const float scale = exp_e(ml - s.m) * rcp(s.d);
            const Span so = rows_span<BF16, ALIGNED, (LPR <= 64)>(out, row0 * cols, nrows * cols, gmask);
            const Buf bout(so.base, so.bytes);
            const RowAt ro = rows_row<BF16, ALIGNED, (LPR <= 64)>(so.lead + static_cast<uint32_t>(g) * row_bytes, gmask);
            if constexpr (STAGE == 2) {
                // the output run's image
                const uint32_t r0 = so.lead + static_cast<uint32_t>(g) * row_bytes;
#pragma unroll
                for (int v = 0; v < VPL; ++v)
#pragma unroll
                    for (int k = 0; k < VEC; ++k) {
                        const int e = (v * LPR + j) * VEC + k;
                        const uint32_t at = r0 + static_cast<uint32_t>(e) * E::kSize;
                        const float val = x[v][k] * scale;
                        if (live & (e < cols)) {
                            if constexpr (BF16)
                                *reinterpret_cast<uint16_t*>(ib + at) = static_cast<uint16_t>(pack_bf16x2(val, 0.0f) & 0xFFFFu);
                            else
                                *reinterpret_cast<float*>(ib + at) = val;
                        }
                    }
            }
            if constexpr (STAGE == 1) {
                // place this lane's entries at their byte offsets in the run
#pragma unroll
                for (int v = 0; v < VPL; ++v) {
#pragma unroll
                    for (int k = 0; k < VEC; ++k) x[v][k] *= scale;
                    const int vi = v * LPR + j;
                    const int e0 = vi * VEC - ri.ph;
                    const bool ok = live & (vi < ns) & ((v > 0) | (e0 > -VEC));
                    const bool whole = ok & (e0 >= 0) & (e0 + VEC <= cols) & same;
                    if (whole) img[(ro.blk + static_cast<uint32_t>(ro.ph - ri.ph) * E::kSize) / 16u + vi] = E::pack(x[v]);
                    if (ok & !whole) {
#pragma unroll
                        for (int k = 0; k < VEC; ++k) {
                            const int e = e0 + k;
                            if (static_cast<uint32_t>(e) < static_cast<uint32_t>(cols)) {
                                const uint32_t at = ro.blk + static_cast<uint32_t>(e + ro.ph) * E::kSize;
                                if constexpr (BF16)
                                    *reinterpret_cast<uint16_t*>(ib + at) =
                                        static_cast<uint16_t>(pack_bf16x2(x[v][k], 0.0f) & 0xFFFFu);
                                else
                                    *reinterpret_cast<float*>(ib + at) = x[v][k];
                            }
                        }
                    }
                }
            }
            if constexpr (STAGE != 0) {
                __syncthreads();
                // the run: bytes [so.lead, so.lead + n) of so.bytes / 16 blocks;
                // blocks holding bytes of other workgroups' rows go out entry by entry
                const uint32_t n = static_cast<uint32_t>(nrows) * row_bytes;
                const int nblk = static_cast<int>(so.bytes / 16u);
                for (int i = tid; i < nblk; i += BLOCK) {
                    const uint32_t b0 = static_cast<uint32_t>(i) * 16u;
                    const bool edge = (b0 < so.lead) | (b0 + 16u > so.lead + n);
                    if (!edge) {
                        bout.store16(b0, img[i]);
                    } else {
#pragma unroll
                        for (int k = 0; k < VEC; ++k) {
                            const uint32_t at = b0 + static_cast<uint32_t>(k) * E::kSize;
                            const bool mine = (at >= so.lead) & (at < so.lead + n);
                            if constexpr (BF16)
                                bout.store2(mine ? at : kOutside, *reinterpret_cast<const uint16_t*>(ib + at));
                            else
                                bout.store4(mine ? at : kOutside, *reinterpret_cast<const uint32_t*>(ib + at));
                        }
                    }
                }
                __syncthreads();
            } else {
#pragma unroll
                for (int v = 0; v < VPL; ++v)
                    if (reached(v)) {
#pragma unroll
                        for (int k = 0; k < VEC; ++k) x[v][k] *= scale;
                        store_slot<BF16, ALIGNED>(bout, ro, ri.ph, same, v * LPR + j, ns, cols, live, x[v], v == 0);
                    }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Streaming two-pass forward for rows too long for registers: one W-wave
// workgroup per row.  Pass 1 folds U vectors per lane at a time:
// m' = max(m, max(tile)), d = d e^{m - m'} + sum e^{x - m'} (the tile form of
// the recurrence); the lane states merge with (+) across the wave and then
// through LDS.  Pass 2 re-reads the row (plain loads in pass 1 leave it in
// L2 / Infinity Cache where it fits) and writes y = e^{x - m} / d.
// ---------------------------------------------------------------------------
template <bool BF16, int W, int U, bool ALIGNED>
__global__ void __launch_bounds__(W * 64)
    k_stream(const void* in, void* out, RowStats st, int64_t rows, int cols, uint32_t gmask) {
    using E = Elt<BF16>;
    constexpr int VEC = E::kVec;
    constexpr int BLOCK = W * 64;
    __shared__ State lds[2][W];

    const int tid = threadIdx.x;
    const bool same = same_phase(in, out);
    int par = 0;

    for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
        const Span si = span_of<BF16>(in, row * cols, cols, gmask);
        const Buf bin(si.base, si.bytes);
        const RowAt ri = row_at<BF16>(si.lead, gmask);
        const int nvec = slot_count<BF16>(cols, ri.ph);
        float ml = kFloor, dl = 0.0f;
        for (int base = 0; base < nvec; base += BLOCK * U) {
            float x[U][VEC];
            load_slots<BF16, U, ALIGNED, false>(bin, ri, base + tid, BLOCK, nvec, cols, true, x);
            float mc = kFloor;
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int k = 0; k < VEC; ++k) mc = fmaxf(mc, x[u][k]);
            const float mn = fmaxf(ml, mc);
            float acc = dl * exp_e(ml - mn);
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int k = 0; k < VEC; ++k) acc += exp_e(x[u][k] - mn);
            dl = acc;
            ml = mn;
        }
        State s = group_merge<64>(State{ml, dl});
        if constexpr (W > 1) {
            if ((tid & (kWave - 1)) == 0) lds[par][tid / kWave] = s;
            __syncthreads();
            s = lds[par][0];
#pragma unroll
            for (int w = 1; w < W; ++w) s = oplus(s, lds[par][w]);
            par ^= 1;
        }
        if (any_stats(st) && tid == 0) put_stats(st, row, s);
        if (out != nullptr) {
            const float inv_d = rcp(s.d);
            const Span so = span_of<BF16>(out, row * cols, cols, gmask);
            const Buf bout(so.base, so.bytes);
            const RowAt ro = row_at<BF16>(so.lead, gmask);
            for (int base = 0; base < nvec; base += BLOCK * U) {
                float x[U][VEC];
                load_slots<BF16, U, ALIGNED, true>(bin, ri, base + tid, BLOCK, nvec, cols, true, x);
#pragma unroll
                for (int u = 0; u < U; ++u) {
#pragma unroll
                    for (int k = 0; k < VEC; ++k) x[u][k] = exp_e(x[u][k] - s.m) * inv_d;
                    store_slot<BF16, ALIGNED>(bout, ro, ri.ph, same, base + u * BLOCK + tid, nvec, cols, true, x[u], u == 0);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Hybrid forward for rows longer than the register-resident kernels hold: one
// 1024-lane workgroup per row keeps the row's first 1024 * VPL vectors in
// registers (read once, as in k_resident) and streams the rest twice (as in
// k_stream).  Pass 1: e_k = e^{x_k - m_r} over the resident slots (m_r the
// lane's resident maximum), then the streamed tiles fold into the same lane
// state by the tile form of the recurrence; lanes and waves merge with (+).
// Pass 2 writes the resident slots as e_k * (e^{m_r - m} / d).  The first
// STASH streamed tiles are also kept in LDS during pass 1 (up to 128 KiB: the
// workgroup has the CU to itself), so pass 2 re-reads only the streamed tiles
// past them.  HBM traffic per row: in + out + the streamed part beyond
// the LDS copy again.
// ---------------------------------------------------------------------------
template <bool BF16>
__device__ __forceinline__ u32x4 pack_exact(const float* v) {
    if constexpr (BF16) {  // values widened from bf16: their top halves
        u32x4 r;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            r[i] = __builtin_amdgcn_perm(__float_as_uint(v[2 * i + 1]), __float_as_uint(v[2 * i]), 0x07060302u);
        return r;
    } else {
        return Elt<false>::pack(v);
    }
}

template <bool BF16, int VPL, int U, bool ALIGNED, int STASH>
__global__ void __launch_bounds__(1024)
    k_hybrid(const void* in, void* out, RowStats st, int64_t rows, int cols, uint32_t gmask) {
    using E = Elt<BF16>;
    constexpr int VEC = E::kVec;
    constexpr int W = 16;
    constexpr int BLOCK = W * 64;
    constexpr int RES = BLOCK * VPL;  // resident vector slots per row
    constexpr int TILE = BLOCK * U;   // streamed slots per step
    static_assert(STASH * TILE * 16 <= 128 * 1024, "LDS copy of at most 128 KiB");
    __shared__ State lds[2][W];
    // streamed tile t < STASH, slot u * BLOCK + lane at
    // stash[t * TILE + u * BLOCK + lane]: each lane reads back only what it
    // wrote, so pass 2 needs no barrier for it
    __shared__ u32x4 stash[STASH > 0 ? STASH * TILE : 1];

    const int tid = threadIdx.x;
    const bool same = same_phase(in, out);
    int par = 0;

    for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
        const Span si = span_of<BF16>(in, row * cols, cols, gmask);
        const Buf bin(si.base, si.bytes);
        const RowAt ri = row_at<BF16>(si.lead, gmask);
        const int nvec = slot_count<BF16>(cols, ri.ph);
        float xr[VPL][VEC];
        load_slots<BF16, VPL, ALIGNED, true>(bin, ri, tid, BLOCK, nvec, cols, true, xr);
        float mr = kFloor;
#pragma unroll
        for (int v = 0; v < VPL; ++v)
#pragma unroll
            for (int k = 0; k < VEC; ++k) mr = fmaxf(mr, xr[v][k]);
        float dl = 0.0f;
#pragma unroll
        for (int v = 0; v < VPL; ++v)
#pragma unroll
            for (int k = 0; k < VEC; ++k) {
                xr[v][k] = exp_e(xr[v][k] - mr);
                dl += xr[v][k];
            }
        float ml = mr;
        auto fold = [&](const float (&x)[U][VEC]) {
            float mc = kFloor;
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int k = 0; k < VEC; ++k) mc = fmaxf(mc, x[u][k]);
            const float mn = fmaxf(ml, mc);
            float acc = dl * exp_e(ml - mn);
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int k = 0; k < VEC; ++k) acc += exp_e(x[u][k] - mn);
            dl = acc;
            ml = mn;
        };
        int base = RES;
        if (out != nullptr) {  // the tiles kept in LDS
            for (int t = 0; (t < STASH) & (base < nvec); ++t, base += TILE) {
                float x[U][VEC];
                load_slots<BF16, U, ALIGNED, false>(bin, ri, base + tid, BLOCK, nvec, cols, true, x);
#pragma unroll
                for (int u = 0; u < U; ++u) stash[t * TILE + u * BLOCK + tid] = pack_exact<BF16>(x[u]);
                fold(x);
            }
        }
        for (; base < nvec; base += TILE) {
            float x[U][VEC];
            load_slots<BF16, U, ALIGNED, false>(bin, ri, base + tid, BLOCK, nvec, cols, true, x);
            fold(x);
        }
        State s = group_merge<64>(State{ml, dl});
        if ((tid & (kWave - 1)) == 0) lds[par][tid / kWave] = s;
        __syncthreads();
        s = lds[par][0];
#pragma unroll
        for (int w = 1; w < W; ++w) s = oplus(s, lds[par][w]);
        par ^= 1;
        if (any_stats(st) && tid == 0) put_stats(st, row, s);
        if (out != nullptr) {
            const float inv_d = rcp(s.d);
            const float scale = exp_e(mr - s.m) * inv_d;
            const Span so = span_of<BF16>(out, row * cols, cols, gmask);
            const Buf bout(so.base, so.bytes);
            const RowAt ro = row_at<BF16>(so.lead, gmask);
#pragma unroll
            for (int v = 0; v < VPL; ++v) {
#pragma unroll
                for (int k = 0; k < VEC; ++k) xr[v][k] *= scale;
                store_slot<BF16, ALIGNED>(bout, ro, ri.ph, same, v * BLOCK + tid, nvec, cols, true, xr[v], v == 0);
            }
            auto put = [&](float (&x)[U][VEC], int b) {
#pragma unroll
                for (int u = 0; u < U; ++u) {
#pragma unroll
                    for (int k = 0; k < VEC; ++k) x[u][k] = exp_e(x[u][k] - s.m) * inv_d;
                    store_slot<BF16, ALIGNED>(bout, ro, ri.ph, same, b + u * BLOCK + tid, nvec, cols, true, x[u], u == 0);
                }
            };
            int b = RES;
            for (int t = 0; (t < STASH) & (b < nvec); ++t, b += TILE) {
                float x[U][VEC];
#pragma unroll
                for (int u = 0; u < U; ++u) E::unpack(stash[t * TILE + u * BLOCK + tid], x[u]);
                put(x, b);
            }
            for (; b < nvec; b += TILE) {
                float x[U][VEC];
                load_slots<BF16, U, ALIGNED, true>(bin, ri, b + tid, BLOCK, nvec, cols, true, x);
                put(x, b);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Baseline: safe softmax in three streaming passes over global memory
// (maximum; sum of e^{x - m}; normalise and store), same geometry and loads
// as k_stream so that the two differ only in the passes.
// naive != 0: the unshifted softmax of the paper summary's section 2 instead,
// pass 1 skipped and m = 0 (two passes: sum of e^x, then e^x / d); e^x
// overflows past x = 88.7 and the row then turns to NaN, as the page warns.
// ---------------------------------------------------------------------------
template <bool BF16, int W, int U, bool ALIGNED>
__global__ void __launch_bounds__(W * 64)
    k_safe3(const void* in, void* out, int64_t rows, int cols, uint32_t gmask, int naive) {
    using E = Elt<BF16>;
    constexpr int VEC = E::kVec;
    constexpr int BLOCK = W * 64;
    __shared__ float lds_m[2][W];
    __shared__ float lds_d[2][W];

    const int tid = threadIdx.x;
    const bool same = same_phase(in, out);
    int par = 0;

    for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
        const Span si = span_of<BF16>(in, row * cols, cols, gmask);
        const Buf bin(si.base, si.bytes);
        const RowAt ri = row_at<BF16>(si.lead, gmask);
        const int nvec = slot_count<BF16>(cols, ri.ph);
        // pass 1: maximum (uniform skip for the naive form)
        float m = 0.0f;
        if (!naive) {
            m = kFloor;
            for (int base = 0; base < nvec; base += BLOCK * U) {
                float x[U][VEC];
                load_slots<BF16, U, ALIGNED, false>(bin, ri, base + tid, BLOCK, nvec, cols, true, x);
#pragma unroll
                for (int u = 0; u < U; ++u)
#pragma unroll
                    for (int k = 0; k < VEC; ++k) m = fmaxf(m, x[u][k]);
            }
            m = wave_max(m);
            if constexpr (W > 1) {
                if ((tid & (kWave - 1)) == 0) lds_m[par][tid / kWave] = m;
                __syncthreads();
                m = lds_m[par][0];
#pragma unroll
                for (int w = 1; w < W; ++w) m = fmaxf(m, lds_m[par][w]);
            }
        }
        // pass 2: sum of e^{x - m}
        float d = 0.0f;
        for (int base = 0; base < nvec; base += BLOCK * U) {
            float x[U][VEC];
            load_slots<BF16, U, ALIGNED, false>(bin, ri, base + tid, BLOCK, nvec, cols, true, x);
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int k = 0; k < VEC; ++k) d += exp_e(x[u][k] - m);
        }
        d = wave_sum(d);
        if constexpr (W > 1) {
            if ((tid & (kWave - 1)) == 0) lds_d[par][tid / kWave] = d;
            __syncthreads();
            d = lds_d[par][0];
#pragma unroll
            for (int w = 1; w < W; ++w) d += lds_d[par][w];
            par ^= 1;
        }
        // pass 3: normalise and store
        const float inv_d = rcp(d);
        const Span so = span_of<BF16>(out, row * cols, cols, gmask);
        const Buf bout(so.base, so.bytes);
        const RowAt ro = row_at<BF16>(so.lead, gmask);
        for (int base = 0; base < nvec; base += BLOCK * U) {
            float x[U][VEC];
            load_slots<BF16, U, ALIGNED, true>(bin, ri, base + tid, BLOCK, nvec, cols, true, x);
#pragma unroll
            for (int u = 0; u < U; ++u) {
#pragma unroll
                for (int k = 0; k < VEC; ++k) x[u][k] = exp_e(x[u][k] - m) * inv_d;
                store_slot<BF16, ALIGNED>(bout, ro, ri.ph, same, base + u * BLOCK + tid, nvec, cols, true, x[u], u == 0);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Baseline with the register-resident geometry: safe softmax in three passes
// over global memory (maximum; sum of e^{x - m}; normalise and store), LPR
// lanes per row and VPL vectors per lane exactly as k_resident, but every
// pass reloads the row's slots instead of keeping them in registers.  Pass 1
// and 2 use plain loads, so re-reads of short rows can hit in cache, which is
// the regime the pages' benchmark describes for short vectors.  Shapes of at
// most 8 vectors per lane; longer rows take the streaming baseline.
// naive != 0: the unshifted two-pass softmax, as in k_safe3.
// ---------------------------------------------------------------------------
template <bool BF16, int LPR, int VPL, bool ALIGNED>
__global__ void __launch_bounds__(LPR <= 64 ? 256 : LPR)
    k_safe3_rows(const void* in, void* out, int64_t rows, int cols, uint32_t gmask, int naive) {
    using E = Elt<BF16>;
    constexpr int VEC = E::kVec;
    constexpr int BLOCK = LPR <= 64 ? 256 : LPR;
    constexpr int RPB = BLOCK / LPR;
    constexpr int W = LPR > 64 ? LPR / 64 : 1;
    constexpr int GROUP = LPR < 64 ? LPR : 64;
    __shared__ float lds_m[2][W];
    __shared__ float lds_d[2][W];

    const int tid = threadIdx.x;
    const int j = tid % LPR;
    const int g = tid / LPR;
    const uint32_t row_bytes = static_cast<uint32_t>(cols) * E::kSize;
    const bool same = same_phase(in, out);
    int par = 0;

    for (int64_t rb = blockIdx.x; rb * RPB < rows; rb += gridDim.x) {
        const int64_t row0 = rb * RPB;
        const int64_t nrows = (rows - row0) < RPB ? (rows - row0) : RPB;
        const bool live = g < nrows;
        const Span si = rows_span<BF16, ALIGNED, (LPR <= 64)>(in, row0 * cols, nrows * cols, gmask);
        const Buf bin(si.base, si.bytes);
        const RowAt ri = rows_row<BF16, ALIGNED, (LPR <= 64)>(si.lead + static_cast<uint32_t>(g) * row_bytes, gmask);
        const int nvec = slot_count<BF16>(cols, ri.ph);
        static_assert(VPL <= 8, "the baseline streams rows past 8 vectors per lane");
        float x[VPL][VEC];

        // pass 1: maximum (uniform skip for the naive form)
        float m = 0.0f;
        if (!naive) {
            m = kFloor;
            load_slots<BF16, VPL, ALIGNED, false>(bin, ri, j, LPR, nvec, cols, live, x);
#pragma unroll
            for (int v = 0; v < VPL; ++v)
#pragma unroll
                for (int k = 0; k < VEC; ++k) m = fmaxf(m, x[v][k]);
            m = group_max<GROUP>(m);
            if constexpr (W > 1) {
                if ((tid & (kWave - 1)) == 0) lds_m[par][tid / kWave] = m;
                __syncthreads();
                m = lds_m[par][0];
#pragma unroll
                for (int w = 1; w < W; ++w) m = fmaxf(m, lds_m[par][w]);
            }
        }
        // pass 2: sum of e^{x - m}
        float d = 0.0f;
        load_slots<BF16, VPL, ALIGNED, false>(bin, ri, j, LPR, nvec, cols, live, x);
#pragma unroll
        for (int v = 0; v < VPL; ++v)
#pragma unroll
            for (int k = 0; k < VEC; ++k) d += exp_e(x[v][k] - m);
        d = group_sum<GROUP>(d);
        if constexpr (W > 1) {
            if ((tid & (kWave - 1)) == 0) lds_d[par][tid / kWave] = d;
            __syncthreads();
            d = lds_d[par][0];
#pragma unroll
            for (int w = 1; w < W; ++w) d += lds_d[par][w];
            par ^= 1;
        }
        // pass 3: normalise and store
        const float inv_d = rcp(d);
        const Span so = rows_span<BF16, ALIGNED, (LPR <= 64)>(out, row0 * cols, nrows * cols, gmask);
        const Buf bout(so.base, so.bytes);
        const RowAt ro = rows_row<BF16, ALIGNED, (LPR <= 64)>(so.lead + static_cast<uint32_t>(g) * row_bytes, gmask);
        load_slots<BF16, VPL, ALIGNED, true>(bin, ri, j, LPR, nvec, cols, live, x);
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
#pragma unroll
            for (int k = 0; k < VEC; ++k) x[v][k] = exp_e(x[v][k] - m) * inv_d;
            store_slot<BF16, ALIGNED>(bout, ro, ri.ph, same, v * LPR + j, nvec, cols, live, x[v], v == 0);
        }
    }
}

// ---------------------------------------------------------------------------
// Split-row forward for batches with too few rows to fill the chip: S
// workgroups per row, each over a contiguous slice of the row's vector slots,
// in two launches (the launch boundary orders the phases):
//   k_split_fold   workgroup (row, s) folds its slice into (m, d) (the tile form
//                  of the recurrence, merged with (+) across lanes and waves)
//                  and writes it to ws[row * S + s];
//   k_split_norm   workgroup (row, s) merges the row's S states with (+) in a
//                  fixed order (so every slice of a row uses the same bits),
//                  re-reads its slice and writes y = e^{x - m} / d.
// Each slice's buffer resource ends with the slice, so loads past its end
// touch no memory and stores past it are dropped.
// ---------------------------------------------------------------------------
struct Slice {
    int v0, v1;      // vector slots [v0, v1) of the row
    uint32_t bytes;  // resource bytes from the row's first block to the end of the slice
};

// Slice `seg` of S over a row of `ns` slots whose widened span has
// `span_bytes` bytes; slices start on multiples of `quant` slots.
__device__ __forceinline__ Slice slice_of(int seg, int S, int ns, uint32_t span_bytes, int quant) {
    const int seg_vec = ((ns + S - 1) / S + quant - 1) / quant * quant;
    const int v0 = seg * seg_vec < ns ? seg * seg_vec : ns;
    const int v1 = v0 + seg_vec < ns ? v0 + seg_vec : ns;
    const uint32_t end = static_cast<uint32_t>(v1) * 16u;
    return Slice{v0, v1, end < span_bytes ? end : span_bytes};
}

template <bool BF16, int W, int U, bool ALIGNED>
__global__ void __launch_bounds__(W * 64)
    k_split_fold(const void* in, State* ws, int64_t rows, int cols, int S) {
    using E = Elt<BF16>;
    constexpr int VEC = E::kVec;
    constexpr int BLOCK = W * 64;
    __shared__ State lds[2][W];
    const int tid = threadIdx.x;
    const int64_t units = rows * S;
    int par = 0;
    for (int64_t unit = blockIdx.x; unit < units; unit += gridDim.x) {
        const int64_t row = unit / S;
        const Span si = span_of<BF16>(in, row * cols, cols, kGrid128);
        const RowAt ri = row_at<BF16>(si.lead, kGrid128);
        const Slice sl =
            slice_of(static_cast<int>(unit - row * S), S, slot_count<BF16>(cols, ri.ph), si.bytes, 8);
        const Buf bin(si.base, sl.bytes);
        float ml = kFloor, dl = 0.0f;
        for (int base = sl.v0; base < sl.v1; base += BLOCK * U) {
            float x[U][VEC];
            load_slots<BF16, U, ALIGNED, false>(bin, ri, base + tid, BLOCK, sl.v1, cols, true, x);
            float mc = kFloor;
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int k = 0; k < VEC; ++k) mc = fmaxf(mc, x[u][k]);
            const float mn = fmaxf(ml, mc);
            float acc = dl * exp_e(ml - mn);
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int k = 0; k < VEC; ++k) acc += exp_e(x[u][k] - mn);
            dl = acc;
            ml = mn;
        }
        State st = group_merge<64>(State{ml, dl});
        if constexpr (W > 1) {
            if ((tid & (kWave - 1)) == 0) lds[par][tid / kWave] = st;
            __syncthreads();
            st = lds[par][0];
#pragma unroll
            for (int w = 1; w < W; ++w) st = oplus(st, lds[par][w]);
            par ^= 1;
        }
        if (tid == 0) ws[unit] = st;
    }
}

template <bool BF16, int W, int U, bool ALIGNED>
__global__ void __launch_bounds__(W * 64)
    k_split_norm(const void* in, void* out, const State* ws, int64_t rows, int cols, int S) {
    using E = Elt<BF16>;
    constexpr int VEC = E::kVec;
    constexpr int BLOCK = W * 64;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int64_t units = rows * S;
    const bool same = same_phase(in, out);
    for (int64_t unit = blockIdx.x; unit < units; unit += gridDim.x) {
        const int64_t row = unit / S;
        const Span si = span_of<BF16>(in, row * cols, cols, kGrid128);
        const RowAt ri = row_at<BF16>(si.lead, kGrid128);
        const Slice sl =
            slice_of(static_cast<int>(unit - row * S), S, slot_count<BF16>(cols, ri.ph), si.bytes, 8);
        // the row's S slice states: lane l folds states l, l + 64, ... in
        // order, then the wave merges the 64 lane states (same bits in every
        // lane, and in every workgroup of the row)
        State t{kFloor, 0.0f};
        for (int q = lane; q < S; q += kWave) t = oplus(t, ws[row * S + q]);
        t = group_merge<64>(t);
        const float m = t.m;
        const float inv_d = rcp(t.d);
        const Buf bin(si.base, sl.bytes);
        const Span so = span_of<BF16>(out, row * cols, cols, kGrid128);
        const Buf bout(so.base, so.bytes);
        const RowAt ro = row_at<BF16>(so.lead, kGrid128);
        for (int base = sl.v0; base < sl.v1; base += BLOCK * U) {
            float x[U][VEC];
            load_slots<BF16, U, ALIGNED, true>(bin, ri, base + tid, BLOCK, sl.v1, cols, true, x);
#pragma unroll
            for (int u = 0; u < U; ++u) {
#pragma unroll
                for (int k = 0; k < VEC; ++k) x[u][k] = exp_e(x[u][k] - m) * inv_d;
                store_slot<BF16, ALIGNED>(bout, ro, ri.ph, same, base + u * BLOCK + tid, sl.v1, cols, true, x[u], u == 0);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Fused softmax + top-K (paper summary, section 4), one read of the input.
//
// One W-wave workgroup per row (per row slice with SPLIT), fp32 or bf16
// logits.  Every lane folds (m, d) over its slots as in k_stream.
// Candidates: each wave keeps ONE sorted list of the best K
// (value, index) pairs it has seen, spread over lanes 0..K-1 (lane k holds
// rank k) under the total order (value desc, index asc).  Most elements are
// rejected by a compare with a wave-uniform threshold T, a lower bound on the
// row's K-th largest value:
//   - first tile: the workgroup's tile is cut into 64 disjoint parts of W
//     lanes; the K-th largest of the 64 part maxima is a tile element with
//     at least K elements at or above it (two barriers, before any insert);
//   - a quarter of the way through a segment of >= 4 tiles: the same bound
//     over everything seen so far (each part is then W lanes' slots of every
//     tile so far, and its maximum the lanes' running maxima);
//   - then: the K-th entry of the wave's own list, and the largest K-th entry
//     published by any wave of the workgroup (an LDS atomic max).
// Survivors (x >= T, so ties at T are kept; while T is still -inf, entries
// in the row that rank ahead of the wave's K-th entry) are inserted one at a
// time:
// position p = number of entries ahead of the new pair, entries from p on
// shift down one lane (DPP wave_shr:1).  Every true top-K element survives
// every filter and stays in its wave's list, so the final merge of the W
// sorted lists (a bitonic merge in one wave, lowest index on ties) is exact.
// Output: probs = e^{u - m} / d over the whole row, and indices.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int ordered_bits(float f) {
    const int i = __float_as_int(f);
    return i >= 0 ? i : (i ^ 0x7FFFFFFF);
}
__device__ __forceinline__ float from_ordered_bits(int i) {
    return __int_as_float(i >= 0 ? i : (i ^ 0x7FFFFFFF));
}

// (a_v, a_i) ranks ahead of (b_v, b_i)
// (bitwise, so it compiles to compares and mask logic, not branches)
__device__ __forceinline__ bool ahead_of(float av, int ai, float bv, int bi) {
    return (av > bv) | ((av == bv) & (ai < bi));
}

// Insert the wave-uniform pair (v, i) into the lane-distributed sorted list.
__device__ __forceinline__ void list_insert(float& L, int& I, float v, int i, int K, int lane,
                                            uint64_t kmask) {
    const int p = __popcll(__ballot(ahead_of(L, I, v, i)) & kmask);
    if (p < K) {
        const float Ls = dpp<kDppWaveShr1>(L);
        const int Is = dpp<kDppWaveShr1>(I);
        const bool shift = lane > p, put = lane == p;
        L = shift ? Ls : (put ? v : L);
        I = shift ? Is : (put ? i : I);
    }
}

// A lower bound on the K-th largest element of a W-wave workgroup's tile,
// from each lane's tile maximum mx: the tile is cut into 64 disjoint parts of
// W lanes (64 / W parts per wave), each part's maximum is one of its elements,
// so the K-th largest of the 64 part maxima (K <= 64) has at least K distinct
// tile elements at or above it.  Ranks are taken under (value desc, part asc),
// a permutation, so exactly one part has rank K - 1; wave w counts, for every
// part, how many of its own 64 / W parts rank ahead, and the counts are summed
// in s_rank (zeroed by the caller before a barrier that precedes this call).
// A NaN maximum (a part of NaNs only) counts as -inf: NaN is never a
// candidate.  Contains two workgroup barriers: every wave must call it.
template <int W>
__device__ __forceinline__ float tile_bound(float mx, int K, int w, int lane, float* s_sub, int* s_rank) {
    constexpr int J = 64 / W;
    float g = (mx == mx) ? mx : -INFINITY;
    if constexpr (W >= 2) g = fmaxf(g, dpp<kDppXor1>(g));
    if constexpr (W >= 4) g = fmaxf(g, dpp<kDppXor2>(g));
    if constexpr (W >= 8) g = fmaxf(g, dpp<kDppHalfMirror>(g));
    if constexpr (W >= 16) g = fmaxf(g, dpp<kDppMirror>(g));
    if ((lane & (W - 1)) == 0) s_sub[w * J + lane / W] = g;
    __syncthreads();
    const float a = s_sub[lane];
    int r = 0;
#pragma unroll
    for (int jj = 0; jj < J; ++jj) {
        const int j = w * J + jj;
        const float b = s_sub[j];
        r += static_cast<int>((b > a) | ((b == a) & (j < lane)));
    }
    if (r != 0) __hip_atomic_fetch_add(&s_rank[lane], r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    __syncthreads();
    const int rank = __hip_atomic_load(&s_rank[lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    const uint64_t sel = __ballot(rank == K - 1);
    return sel != 0 ? readlane(a, __builtin_ctzll(sel)) : -INFINITY;  // sel has one bit (ranks are a permutation)
}

// One (value, index) entry of a segment's partial top-K list.
struct TopkEntry {
    float v;
    int i;
};

// Top-K of up to NL sorted lists, by a truncating bitonic merge inside one
// wave.  Each list (value desc, index asc; K <= KP entries, KP a power of two
// <= 32, read through get(list, pos, v, i)) is padded to KP entries with the
// sentinel (-inf, INT_MAX), which ranks after every real entry, and lists are
// packed 64 / KP to a register (register r, lane l: list (64 r + l) / KP,
// position (64 r + l) % KP).
//   - Two registers A and B merge lane by lane: A keeps the better of A[l] and
//     B[l ^ (KP - 1)], B reversed within each KP-block.  Each block then holds
//     the KP best of its two lists as a bitonic sequence.
//   - Within a register, blocks merge in pairs at distance 1, 2, 4, ... blocks:
//     lane l and lane l ^ (2^t KP - 1) both keep the better, so both blocks of
//     a pair hold the KP best (one reversed), and the next level's mirror meets
//     the right partner.
//   - After every merge, half-cleaners at lane distances KP/2, ..., 1 (the
//     lower lane keeps the better) sort every block.
// Lane k < K ends with the k-th best entry of all lists.
template <int S>
__device__ __forceinline__ void keep_better(float& v, int& i, int lane) {  // both lanes keep the better
    const float ov = lane_xor<S>(v, lane);
    const int oi = lane_xor<S>(i, lane);
    const bool t = ahead_of(ov, oi, v, i);
    v = t ? ov : v;
    i = t ? oi : i;
}

template <int S>
__device__ __forceinline__ void half_clean(float& v, int& i, int lane) {  // lower lane keeps the better
    const float ov = lane_xor<S>(v, lane);
    const int oi = lane_xor<S>(i, lane);
    const bool t = ahead_of(ov, oi, v, i) != ((lane & S) != 0);
    v = t ? ov : v;
    i = t ? oi : i;
}

template <int KP>
__device__ __forceinline__ void sort_blocks(float& v, int& i, int lane) {
    if constexpr (KP >= 32) half_clean<16>(v, i, lane);
    if constexpr (KP >= 16) half_clean<8>(v, i, lane);
    if constexpr (KP >= 8) half_clean<4>(v, i, lane);
    if constexpr (KP >= 4) half_clean<2>(v, i, lane);
    if constexpr (KP >= 2) half_clean<1>(v, i, lane);
}

template <int KP, int B, int SPAN>
__device__ __forceinline__ void merge_blocks(float& v, int& i, int lane) {
    if constexpr (B <= 64 && B / 2 < SPAN) {
        keep_better<B - 1>(v, i, lane);
        sort_blocks<KP>(v, i, lane);
        merge_blocks<KP, 2 * B, SPAN>(v, i, lane);
    }
}

template <int KP, int NL, typename Get>
__device__ __forceinline__ void bitonic_topk(int n, int K, int lane, Get get, float& out_v, int& out_i) {
    constexpr int NREG = NL * KP > 64 ? NL * KP / 64 : 1;
    static_assert((NL & (NL - 1)) == 0 && NL * KP <= 64 * 8, "NL a power of two");
    float v[NREG];
    int ix[NREG];
#pragma unroll
    for (int r = 0; r < NREG; ++r) {
        const int e = r * 64 + lane;
        const int list = e / KP, pos = e % KP;
        v[r] = -INFINITY;
        ix[r] = 0x7FFFFFFF;
        if ((list < n) & (pos < K)) get(list, pos, v[r], ix[r]);
    }
#pragma unroll
    for (int half = NREG / 2; half >= 1; half /= 2) {
#pragma unroll
        for (int r = 0; r < half; ++r) {
            const float bv = lane_xor<KP - 1>(v[r + half], lane);
            const int bi = lane_xor<KP - 1>(ix[r + half], lane);
            const bool t = ahead_of(bv, bi, v[r], ix[r]);
            v[r] = t ? bv : v[r];
            ix[r] = t ? bi : ix[r];
            sort_blocks<KP>(v[r], ix[r], lane);
        }
    }
    // lists still spread over blocks of register 0: NL * KP lanes, at most 64
    merge_blocks<KP, 2 * KP, (NL * KP < 64 ? NL * KP : 64)>(v[0], ix[0], lane);
    out_v = v[0];
    out_i = ix[0];
}

template <int NL, typename Get>
__device__ __forceinline__ void topk_of_lists(int n, int K, int lane, Get get, float& out_v, int& out_i) {
    if (K <= 1) bitonic_topk<1, NL>(n, K, lane, get, out_v, out_i);
    else if (K <= 2) bitonic_topk<2, NL>(n, K, lane, get, out_v, out_i);
    else if (K <= 4) bitonic_topk<4, NL>(n, K, lane, get, out_v, out_i);
    else if (K <= 8) bitonic_topk<8, NL>(n, K, lane, get, out_v, out_i);
    else if (K <= 16) bitonic_topk<16, NL>(n, K, lane, get, out_v, out_i);
    else bitonic_topk<32, NL>(n, K, lane, get, out_v, out_i);
}

// SPLIT = false: one workgroup per row, results written directly.
// SPLIT = true: S workgroups per row, each over a contiguous slice of the
// row's vector slots, each writing its state (m, d) and its sorted K-list to
// the workspace; k_topk_merge (the next launch on the stream, so every
// partial is visible) combines them.
// select != 0 (SPLIT = false only): top-K selection alone, the TopK stage of
// the paper summary's unfused pipelines (section 4, the access table): no
// (m, d) fold, no exponential, and the K entries themselves are written in
// place of probabilities.
template <bool BF16, int W, int U, bool ALIGNED, bool SPLIT>
__global__ void __launch_bounds__(W * 64)
    k_topk(const void* in, float* probs, int* idx, int64_t rows, int cols, int K, int S, State* ws_state,
           TopkEntry* ws_list, int select) {
    using E = Elt<BF16>;
    static_assert(W == 1 || W == 2 || W == 4 || W == 8 || W == 16,
                  "the final merge packs W lists of up to 32 entries into at most 8 registers");
    constexpr int BLOCK = W * 64;
    constexpr int VEC = E::kVec;
    constexpr int STEP = BLOCK * U;
    __shared__ float s_val[W][kTopKMax];
    __shared__ int s_idx[W][kTopKMax];
    __shared__ State s_md[W];
    __shared__ float s_sub[64];
    __shared__ int s_rank[2][64];  // one per bound: the first tile's, the refresh
    __shared__ int s_thr;

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = tid / kWave;
    const uint64_t kmask = (K >= 64) ? ~0ull : ((1ull << K) - 1ull);
    const int64_t units = SPLIT ? rows * S : rows;

    for (int64_t unit = blockIdx.x; unit < units; unit += gridDim.x) {
        const int64_t row = SPLIT ? unit / S : unit;
        const int seg = SPLIT ? static_cast<int>(unit - row * S) : 0;
        const Span si = span_of<BF16>(in, row * cols, cols, kGrid16);
        const int ph = row_at<BF16>(si.lead, kGrid16).ph;  // the row's first block is at byte 0
        // The resource ends with the segment, so loads issued ahead past its
        // end (into the next segment or past the row) touch no memory.
        const Slice sl = slice_of(seg, SPLIT ? S : 1, slot_count<BF16>(cols, ph), si.bytes, 1);
        const int v0 = sl.v0, v1 = sl.v1;
        const Buf bin(si.base, sl.bytes);
        // the first tile's loads go out before the barrier below, which
        // waits for every wave of the workgroup to start
        u32x4 raw[U];
#pragma unroll
        for (int u = 0; u < U; ++u) raw[u] = bin.load16<true>(static_cast<uint32_t>(v0 + u * BLOCK + tid) * 16u);
        if (tid == 0) s_thr = ordered_bits(-INFINITY);
        if (tid < 128) s_rank[tid / 64][tid % 64] = 0;
        __syncthreads();

        float ml = kFloor, dl = 0.0f;
        float L = -INFINITY;
        int I = 0x7FFFFFFF;
        float T = -INFINITY;
        const int ntiles = (v1 - v0 + STEP - 1) / STEP;
        const int refresh = ntiles >= 4 ? ntiles / 4 : -1;  // tile index of the refreshed bound
        int t = 0;

        // One tile: unpack the raw loads (entries outside the segment or the
        // row become -inf), issue the next tile's loads into the same
        // registers, fold (m, d), then look for candidates.
        auto tile = [&](u32x4 (&raw)[U], const int base) {
            float x[U][VEC];
#pragma unroll
            for (int u = 0; u < U; ++u) E::unpack(raw[u], x[u]);
            // Only a segment's last tile can hold slots past its end (read as
            // 0 by the range check), and, for an unaligned row, its first and
            // last tiles entries outside the row; the tests are uniform.
            if constexpr (ALIGNED) {
                if (base + STEP > v1) {
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const bool ok = base + u * BLOCK + tid < v1;
#pragma unroll
                        for (int k = 0; k < VEC; ++k) x[u][k] = ok ? x[u][k] : -INFINITY;
                    }
                }
            } else {
                if (base == v0 || base + STEP >= v1) {
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const int slot = base + u * BLOCK + tid;
                        const int e0 = slot * VEC - ph;
#pragma unroll
                        for (int k = 0; k < VEC; ++k)
                            x[u][k] = ((slot < v1) & (static_cast<uint32_t>(e0 + k) < static_cast<uint32_t>(cols)))
                                          ? x[u][k]
                                          : -INFINITY;
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
                raw[u] = bin.load16<true>(static_cast<uint32_t>(base + STEP + u * BLOCK + tid) * 16u);
            __builtin_amdgcn_sched_barrier(0);

            float mx = -INFINITY;
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int k = 0; k < VEC; ++k) mx = fmaxf(mx, x[u][k]);
            // (m, d) fold over the tile (the running maximum alone when
            // selecting: the refreshed bound reads it)
            const float mn = fmaxf(ml, mx);
            if (!select) {
                float acc = dl * exp_e(ml - mn);
#pragma unroll
                for (int u = 0; u < U; ++u)
#pragma unroll
                    for (int k = 0; k < VEC; ++k) acc += exp_e(x[u][k] - mn);
                dl = acc;
            }
            ml = mn;
            // candidates
            // every wave of the workgroup runs every tile of the segment (v0,
            // v1 and the tile count are uniform), so all reach the barriers
            // inside tile_bound
            if (t == 0) {
                T = tile_bound<W>(mx, K, w, lane, s_sub, s_rank[0]);
            } else if (t == refresh) {
                // a lane that has seen no element yet holds kFloor: not an element
                T = fmaxf(T, tile_bound<W>(ml > kFloor ? ml : -INFINITY, K, w, lane, s_sub, s_rank[1]));
            }
            ++t;
            T = fmaxf(T, from_ordered_bits(__hip_atomic_load(&s_thr, __ATOMIC_RELAXED,
                                                             __HIP_MEMORY_SCOPE_WORKGROUP)));
            if (__ballot(mx >= T) != 0) {
                if (T > -INFINITY) {
                    // entries outside the segment or the row read -inf, and
                    // cannot reach T
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const int wave_slot0 = base + u * BLOCK + w * kWave;
#pragma unroll
                        for (int k = 0; k < VEC; ++k) {
                            uint64_t mask = __ballot(x[u][k] >= T);
                            while (mask != 0) {
                                const int l = __builtin_ctzll(mask);
                                mask &= mask - 1;
                                list_insert(L, I, readlane(x[u][k], l), (wave_slot0 + l) * VEC + k - ph, K, lane,
                                            kmask);
                            }
                        }
                    }
                } else {
                    // T = -inf (a row or slice shorter than the workgroup's
                    // first tile, or with few entries above -inf): every
                    // entry would pass, so take only in-row entries that rank
                    // ahead of the wave's K-th entry, re-read every round
                    // (once the list holds K entries of -inf, later -inf
                    // entries of higher index are skipped).  A NaN entry
                    // ranks as -inf here, so a row with fewer than K numbers
                    // still yields K distinct in-row columns.  (A finite T
                    // has at least K numbers at or above it, so NaN entries
                    // are never needed once T is finite.)
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const int wave_slot0 = base + u * BLOCK + w * kWave;
                        const int my_slot = wave_slot0 + lane;
#pragma unroll
                        for (int k = 0; k < VEC; ++k) {
                            const int i_me = my_slot * VEC + k - ph;  // column index
                            const bool in_row =
                                (my_slot < v1) & (static_cast<uint32_t>(i_me) < static_cast<uint32_t>(cols));
                            const float xv = (x[u][k] == x[u][k]) ? x[u][k] : -INFINITY;
                            uint64_t mask =
                                __ballot(in_row & ahead_of(xv, i_me, readlane(L, K - 1), readlane(I, K - 1)));
                            while (mask != 0) {
                                const int l = __builtin_ctzll(mask);
                                mask &= mask - 1;
                                list_insert(L, I, readlane(xv, l), (wave_slot0 + l) * VEC + k - ph, K, lane, kmask);
                            }
                        }
                    }
                }
                const float kth = readlane(L, K - 1);
                if (kth > T) {
                    T = kth;
                    if (lane == 0)
                        __hip_atomic_fetch_max(&s_thr, ordered_bits(kth), __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_WORKGROUP);
                }
            }
        };

        // Software pipeline over the segment's tiles: the loads of the next
        // tile are in flight while one is folded.  Loads past the end of the
        // segment touch no memory (buffer range check).
        for (int base = v0; base < v1; base += STEP) tile(raw, base);

        const State st = group_merge<64>(State{ml, dl});
        if (lane < K) {
            s_val[w][lane] = L;
            s_idx[w][lane] = I;
        }
        if (lane == 0) s_md[w] = st;
        __syncthreads();

        if (w == 0) {
            State t = s_md[0];
#pragma unroll
            for (int ww = 1; ww < W; ++ww) t = oplus(t, s_md[ww]);
            float out_v;
            int out_i;
            topk_of_lists<W>(
                W, K, lane, [&](int l, int p, float& v, int& i) { v = s_val[l][p]; i = s_idx[l][p]; }, out_v,
                out_i);
            if constexpr (!SPLIT) {
                if (lane < K) {
                    probs[row * K + lane] = select ? out_v : exp_e(out_v - t.m) * rcp(t.d);
                    idx[row * K + lane] = out_i;
                }
            } else {
                if (lane < K) ws_list[unit * K + lane] = TopkEntry{out_v, out_i};
                if (lane == 0) ws_state[unit] = t;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Fused softmax + top-K for short rows (paper summary, section 4), the shape
// of a mixture-of-experts router: many rows of up to 2048 entries.  LPR <= 64
// lanes share a row and hold it in registers (VPL 16-byte slots each, at most
// 64 entries per lane), several rows per wavefront, no barriers; the row is
// read once.
//   - State: the row maximum M and d = sum e^{x - M} by reductions over the
//     row's lanes.
//   - Selection keys: each entry becomes an integer that orders as the value
//     does (-0.0 and +0.0 equal); entries outside the row, and entries
//     already output, take the lowest key.  Ties between keys go to the lower
//     column, the order of the oracle.  NaN entries get keys too (above +inf
//     or below -inf by sign), so a row holding NaN still yields K distinct
//     in-row indices, in no specified order, with NaN probabilities.
//   - K rounds: each lane offers its best remaining entry; a butterfly over
//     the row's lanes finds the row's best, written by the row's first lane
//     (probability e^{u - M} / d over the whole row, and the index).  The
//     lane that held it retires it and finds its next best.  With more than
//     8 entries per lane they sit in groups of at most 8 (4 groups up to 32
//     entries, 8 groups of 8 for 64) with a best per group, and the keys also
//     live in LDS (each lane only touches its own words, so no barrier):
//     retiring an entry is one store and refreshing its group reads that
//     group's keys instead of rescanning all of them.  FEWK (K = 1:
//     nothing is ever retired) keeps the keys in registers and needs no LDS,
//     which leaves room for more workgroups per CU.
// ---------------------------------------------------------------------------
constexpr int kKeyRetired = INT_MIN;  // outside the row, or already output

__device__ __forceinline__ int order_key(float x) {
    const int b = __float_as_int(x + 0.0f);  // -0.0 + 0.0 = +0.0
    const int k = b ^ ((b >> 31) & 0x7FFFFFFF);
    return k > kKeyRetired ? k : kKeyRetired + 1;  // the all-ones NaN pattern
}

__device__ __forceinline__ float key_value(int k) { return __int_as_float(k ^ ((k >> 31) & 0x7FFFFFFF)); }

// Integer maximum over an aligned group of G lanes, same value in every lane.
template <int G>
__device__ __forceinline__ int group_max_i32(int v) {
    if constexpr (G >= 2) v = max(v, dpp<kDppXor1>(v));
    if constexpr (G >= 4) v = max(v, dpp<kDppXor2>(v));
    if constexpr (G >= 8) v = max(v, dpp<kDppHalfMirror>(v));
    if constexpr (G >= 16) v = max(v, dpp<kDppMirror>(v));
    if constexpr (G >= 32) {
        const f32x2 t = swap_rows16(__int_as_float(v));
        v = max(__float_as_int(t[0]), __float_as_int(t[1]));
    }
    if constexpr (G >= 64) {
        const f32x2 t = swap_rows32(__int_as_float(v));
        v = max(__float_as_int(t[0]), __float_as_int(t[1]));
    }
    return v;
}

// Integer minimum over an aligned group of G lanes, same value in every lane.
template <int G>
__device__ __forceinline__ int group_min_i32(int v) {
    if constexpr (G >= 2) v = min(v, dpp<kDppXor1>(v));
    if constexpr (G >= 4) v = min(v, dpp<kDppXor2>(v));
    if constexpr (G >= 8) v = min(v, dpp<kDppHalfMirror>(v));
    if constexpr (G >= 16) v = min(v, dpp<kDppMirror>(v));
    if constexpr (G >= 32) {
        const f32x2 t = swap_rows16(__int_as_float(v));
        v = min(__float_as_int(t[0]), __float_as_int(t[1]));
    }
    if constexpr (G >= 64) {
        const f32x2 t = swap_rows32(__int_as_float(v));
        v = min(__float_as_int(t[0]), __float_as_int(t[1]));
    }
    return v;
}

// Every lane of each aligned group of LPR lanes ends with the group's best
// (key, column): the largest key, then the lowest column among the lanes
// offering it.  Two integer reductions (a maximum, then a minimum), each step
// one DPP operand and one max or min.
template <int LPR>
__device__ __forceinline__ void group_best_key(int& k, int& c) {
    const int m = group_max_i32<LPR>(k);
    c = group_min_i32<LPR>(k == m ? c : INT_MAX);
    k = m;
}

template <bool BF16, int LPR, int VPL, bool ALIGNED, bool FEWK>
__global__ void __launch_bounds__(256)
    k_topk_rows(const void* in, float* probs, int* idx, int64_t rows, int cols, int K) {
    using E = Elt<BF16>;
    constexpr int VEC = E::kVec;
    constexpr int RPB = 256 / LPR;
    constexpr int N = VPL * VEC;                // entries per lane
    constexpr bool kLds = (N > 8) & !FEWK;      // keys in LDS, in groups
    constexpr int NG = kLds ? (N > 32 ? 8 : 4) : 1;  // groups per lane
    constexpr int G = N / NG;                   // entries per group
    constexpr int NQ = kLds ? N / 4 : 1;        // 4-key LDS words per lane
    static_assert(LPR >= 4 && LPR <= 64 && N <= 64, "one row within a wavefront, at most 64 entries per lane");
    static_assert(N <= 32 || !FEWK, "64 entries per lane only with the keys in LDS");
    static_assert(!kLds || G % 4 == 0, "groups of whole 4-key words");
    // lane t's keys 4q..4q+3 at s_keys[q][t]: each lane reads and writes only
    // its own words, with consecutive lanes on consecutive 16 bytes
    __shared__ int4 s_keys[NQ][kLds ? 256 : 1];

    const int tid = threadIdx.x;
    const int j = tid % LPR;
    const int g = tid / LPR;
    const uint32_t row_bytes = static_cast<uint32_t>(cols) * E::kSize;
    constexpr int LGV = VEC == 8 ? 3 : 2;

    for (int64_t rb = blockIdx.x; rb * RPB < rows; rb += gridDim.x) {
        const int64_t row0 = rb * RPB;
        const int64_t nrows = (rows - row0) < RPB ? (rows - row0) : RPB;
        const int64_t row = row0 + g;
        const bool live = g < nrows;
        const Span si = rows_span<BF16, ALIGNED, true>(in, row0 * cols, nrows * cols, kGrid16);
        const Buf bin(si.base, si.bytes);
        const RowAt ri = rows_row<BF16, ALIGNED, true>(si.lead + static_cast<uint32_t>(g) * row_bytes, kGrid16);
        const int ns = slot_count<BF16>(cols, ri.ph);

        float x[VPL][VEC];
        load_slots<BF16, VPL, ALIGNED, true>(bin, ri, j, LPR, ns, cols, live, x);

        // the row's state: M and d = sum e^{x - M} (entries outside the row
        // read -inf and add 0)
        float ml = kFloor;
#pragma unroll
        for (int v = 0; v < VPL; ++v)
#pragma unroll
            for (int k = 0; k < VEC; ++k) ml = fmaxf(ml, x[v][k]);
        const float M = group_max<LPR>(ml);
        float dl = 0.0f;
#pragma unroll
        for (int v = 0; v < VPL; ++v)
#pragma unroll
            for (int k = 0; k < VEC; ++k) dl += exp_e(x[v][k] - M);
        const float inv_d = rcp(group_sum<LPR>(dl));

        if constexpr (FEWK) {
            // K = 1 (the only K this form is launched for): the row's best is
            // its maximum M, so the answer is the lowest in-row column holding
            // M, with no keys at all (-0.0 == +0.0 as the key order has it).
            // A row of only -inf (or NaN) has no entry equal to M, which starts
            // at -FLT_MAX; it takes column 0, where the key order puts a row
            // of only -inf too.  On rows without NaN this is the key order's
            // answer; a row holding NaN takes its lowest column equal to the
            // largest number (the key order would rank a NaN first), which is
            // still an in-row column with a NaN probability.
            // Entries are visited from the last, so the lowest column stays.
            int cl = INT_MAX;
#pragma unroll
            for (int v = VPL - 1; v >= 0; --v) {
                const int e0 = (v * LPR + j) * VEC - ri.ph;
#pragma unroll
                for (int k = VEC - 1; k >= 0; --k) {
                    const bool in_row = live & ((v * LPR + j) < ns) &
                                        (ALIGNED | (static_cast<uint32_t>(e0 + k) < static_cast<uint32_t>(cols)));
                    cl = (in_row & (x[v][k] == M)) ? e0 + k : cl;
                }
            }
            const int wc = group_min_i32<LPR>(cl);
            if (live & (j == 0)) {
                const bool hit = wc != INT_MAX;
                probs[row * K] = exp_e((hit ? M : -INFINITY) - M) * inv_d;
                idx[row * K] = hit ? wc : 0;
            }
            continue;
        }

        // keys; entry e = v * VEC + k of this lane is column
        // ((e >> LGV) * LPR + j) * VEC + (e & (VEC - 1)) - ph.  Rows whose
        // length is a whole number of slots hold only in-row entries in
        // their slots.
        int key[N];
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
            const int e0 = (v * LPR + j) * VEC - ri.ph;
#pragma unroll
            for (int k = 0; k < VEC; ++k) {
                const bool in_row = live & ((v * LPR + j) < ns) &
                                    (ALIGNED | (static_cast<uint32_t>(e0 + k) < static_cast<uint32_t>(cols)));
                key[v * VEC + k] = in_row ? order_key(x[v][k]) : kKeyRetired;
            }
        }
        auto column = [&](int e) { return ((e >> LGV) * LPR + j) * VEC + (e & (VEC - 1)) - ri.ph; };

        // best of each group (entries scanned in column order with a strict
        // compare, so the lower column wins ties)
        int gk[NG], ge[NG];
        auto scan_group = [&](int q, const int* t) {
            int nk = t[0], ne = 0;
#pragma unroll
            for (int u = 1; u < G; ++u) {
                const bool b = t[u] > nk;
                nk = b ? t[u] : nk;
                ne = b ? u : ne;
            }
            gk[q] = nk;
            ge[q] = q * G + ne;
        };
#pragma unroll
        for (int q = 0; q < NG; ++q) scan_group(q, key + q * G);
        int bk, be;
        auto best_of_groups = [&]() {
            bk = gk[0];
            be = ge[0];
#pragma unroll
            for (int q = 1; q < NG; ++q) {
                const bool b = gk[q] > bk;
                bk = b ? gk[q] : bk;
                be = b ? ge[q] : be;
            }
        };
        best_of_groups();
        if constexpr (kLds) {
            if (K > 1) {
#pragma unroll
                for (int q = 0; q < NQ; ++q)
                    s_keys[q][tid] = int4{key[4 * q], key[4 * q + 1], key[4 * q + 2], key[4 * q + 3]};
            }
        }

        for (int r = 0; r < K; ++r) {
            const int bc = bk == kKeyRetired ? INT_MAX : column(be);
            int wk = bk, wc = bc;
            group_best_key<LPR>(wk, wc);
            if (live & (j == 0)) {
                probs[row * K + r] = exp_e(key_value(wk) - M) * inv_d;
                idx[row * K + r] = wc;
            }
            if ((r + 1 < K) & (bc == wc) & (wc != INT_MAX)) {
                // this lane held the row's best: retire it, then refresh the
                // best of its group
                if constexpr (kLds) {
                    const int q = be / G;
                    // the store comes first: one lane's LDS accesses complete
                    // in order, so the group read below sees it
                    reinterpret_cast<int*>(&s_keys[be >> 2][tid])[be & 3] = kKeyRetired;
                    int t[G];
#pragma unroll
                    for (int w = 0; w < G / 4; ++w) {
                        const int4 kk = s_keys[q * (G / 4) + w][tid];
                        t[4 * w] = kk.x;
                        t[4 * w + 1] = kk.y;
                        t[4 * w + 2] = kk.z;
                        t[4 * w + 3] = kk.w;
                    }
                    int nk = t[0], ne = 0;
#pragma unroll
                    for (int u = 1; u < G; ++u) {
                        const bool b = t[u] > nk;
                        nk = b ? t[u] : nk;
                        ne = b ? u : ne;
                    }
#pragma unroll
                    for (int p = 0; p < NG; ++p) {
                        gk[p] = p == q ? nk : gk[p];
                        ge[p] = p == q ? q * G + ne : ge[p];
                    }
                } else {
#pragma unroll
                    for (int u = 0; u < N; ++u) key[u] = u == be ? kKeyRetired : key[u];
                    scan_group(0, key);
                }
                best_of_groups();
            }
        }
    }
}

// bf16 rows: a bf16 value's order key fits in 16 bits, so an entry packs its
// key and its column into one int, (key << 16) | (0xFFFF - column).  The
// integer order is then the selection order (larger value first, then lower
// column), every compare of the selection is one integer max, and the column
// comes back with the winner.  Columns stay below 2048 here.
constexpr int kPackedRetired = INT_MIN;  // outside the row, or already output

__device__ __forceinline__ int packed_entry(float x, int col) {
    // the 32-bit key of a widened bf16 value carries the 16-bit key in its top
    // half; the all-ones NaN pattern would land on the retired value's key
    const int k16 = max(order_key(x) >> 16, -32767);
    return static_cast<int>((static_cast<uint32_t>(k16) << 16) | static_cast<uint32_t>(0xFFFF - col));
}

__device__ __forceinline__ float packed_value(int p) {
    const int k16 = p >> 16;
    return __int_as_float(static_cast<int>(static_cast<uint32_t>(k16 ^ ((k16 >> 31) & 0x7FFF)) << 16));
}

__device__ __forceinline__ int packed_column(int p) { return 0xFFFF - (p & 0xFFFF); }

// k_topk_rows for bf16 rows on packed entries: the same state, rounds, groups
// and LDS layout, with the lane's best a plain maximum and the lane holding
// the row's winner the one whose best equals it (columns are unique).
template <int LPR, int VPL, bool ALIGNED, bool FEWK>
__global__ void __launch_bounds__(256)
    k_topk_rows_bf16(const void* in, float* probs, int* idx, int64_t rows, int cols, int K) {
    using E = Elt<true>;
    constexpr int VEC = E::kVec;
    constexpr int RPB = 256 / LPR;
    constexpr int N = VPL * VEC;                     // entries per lane
    constexpr bool kLds = (N > 8) & !FEWK;           // entries in LDS, in groups
    constexpr int NG = kLds ? (N > 32 ? 8 : 4) : 1;  // groups per lane
    constexpr int G = N / NG;                        // entries per group
    constexpr int NQ = kLds ? N / 4 : 1;             // 4-entry LDS words per lane
    constexpr int LGL = LPR == 4 ? 2 : LPR == 8 ? 3 : LPR == 16 ? 4 : LPR == 32 ? 5 : 6;
    static_assert(LPR >= 4 && LPR <= 64 && N <= 64, "one row within a wavefront, at most 64 entries per lane");
    static_assert(N <= 32 || !FEWK, "64 entries per lane only with the entries in LDS");
    static_assert(!kLds || G % 4 == 0, "groups of whole 4-entry words");
    __shared__ int4 s_keys[NQ][kLds ? 256 : 1];

    const int tid = threadIdx.x;
    const int j = tid % LPR;
    const int g = tid / LPR;
    const uint32_t row_bytes = static_cast<uint32_t>(cols) * E::kSize;

    for (int64_t rb = blockIdx.x; rb * RPB < rows; rb += gridDim.x) {
        const int64_t row0 = rb * RPB;
        const int64_t nrows = (rows - row0) < RPB ? (rows - row0) : RPB;
        const int64_t row = row0 + g;
        const bool live = g < nrows;
        const Span si = rows_span<true, ALIGNED, true>(in, row0 * cols, nrows * cols, kGrid16);
        const Buf bin(si.base, si.bytes);
        const RowAt ri = rows_row<true, ALIGNED, true>(si.lead + static_cast<uint32_t>(g) * row_bytes, kGrid16);
        const int ns = slot_count<true>(cols, ri.ph);

        float x[VPL][VEC];
        load_slots<true, VPL, ALIGNED, true>(bin, ri, j, LPR, ns, cols, live, x);

        float ml = kFloor;
#pragma unroll
        for (int v = 0; v < VPL; ++v)
#pragma unroll
            for (int k = 0; k < VEC; ++k) ml = fmaxf(ml, x[v][k]);
        const float M = group_max<LPR>(ml);
        float dl = 0.0f;
#pragma unroll
        for (int v = 0; v < VPL; ++v)
#pragma unroll
            for (int k = 0; k < VEC; ++k) dl += exp_e(x[v][k] - M);
        const float inv_d = rcp(group_sum<LPR>(dl));

        // entry e = v * VEC + k of this lane is column (v * LPR + j) * VEC + k - ph
        int key[N];
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
            const int e0 = (v * LPR + j) * VEC - ri.ph;
#pragma unroll
            for (int k = 0; k < VEC; ++k) {
                const bool in_row = live & ((v * LPR + j) < ns) &
                                    (ALIGNED | (static_cast<uint32_t>(e0 + k) < static_cast<uint32_t>(cols)));
                key[v * VEC + k] = in_row ? packed_entry(x[v][k], e0 + k) : kPackedRetired;
            }
        }
        int gk[NG];
#pragma unroll
        for (int q = 0; q < NG; ++q) {
            int b = key[q * G];
#pragma unroll
            for (int u = 1; u < G; ++u) b = max(b, key[q * G + u]);
            gk[q] = b;
        }
        auto best_of_groups = [&]() {
            int b = gk[0];
#pragma unroll
            for (int q = 1; q < NG; ++q) b = max(b, gk[q]);
            return b;
        };
        int bk = best_of_groups();
        if constexpr (kLds) {
            if (K > 1) {
#pragma unroll
                for (int q = 0; q < NQ; ++q)
                    s_keys[q][tid] = int4{key[4 * q], key[4 * q + 1], key[4 * q + 2], key[4 * q + 3]};
            }
        }

        for (int r = 0; r < K; ++r) {
            const int w = group_max_i32<LPR>(bk);
            if (live & (j == 0)) {
                probs[row * K + r] = exp_e(packed_value(w) - M) * inv_d;
                idx[row * K + r] = packed_column(w);
            }
            if ((r + 1 < K) & (bk == w) & (w != kPackedRetired)) {
                // this lane held the row's winner: retire it and refresh its group
                const int c = packed_column(w) + ri.ph;  // (v * LPR + j) * VEC + k
                const int e = ((c / VEC) >> LGL) * VEC + (c & (VEC - 1));
                if constexpr (kLds) {
                    const int q = e / G;
                    // the store comes first: one lane's LDS accesses complete
                    // in order, so the group read below sees it
                    reinterpret_cast<int*>(&s_keys[e >> 2][tid])[e & 3] = kPackedRetired;
                    int nk = kPackedRetired;
#pragma unroll
                    for (int u = 0; u < G / 4; ++u) {
                        const int4 kk = s_keys[q * (G / 4) + u][tid];
                        nk = max(max(nk, kk.x), max(kk.y, max(kk.z, kk.w)));
                    }
#pragma unroll
                    for (int p = 0; p < NG; ++p) gk[p] = p == q ? nk : gk[p];
                } else {
                    int b = kPackedRetired;
#pragma unroll
                    for (int u = 0; u < N; ++u) {
                        key[u] = u == e ? kPackedRetired : key[u];
                        b = max(b, key[u]);
                    }
                    gk[0] = b;
                }
                bk = best_of_groups();
            }
        }
    }
}

// Second launch of the split top-K: one wavefront per row folds the S slice
// states with (+) in slice order and merges the S sorted lists (bitonic, as
// above), then writes the K probabilities and indices.
__global__ void __launch_bounds__(256)
    k_topk_merge(float* probs, int* idx, int64_t rows, int K, int S, const State* ws_state,
                 const TopkEntry* ws_list) {
    const int lane = threadIdx.x & (kWave - 1);
    // one row per wavefront; rows past the grid stride (no barrier here, so
    // wavefronts may leave independently)
    for (int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / kWave; row < rows;
         row += static_cast<int64_t>(gridDim.x) * 4) {
        const int64_t u0 = row * S;
        State r = ws_state[u0];
        for (int q = 1; q < S; ++q) r = oplus(r, ws_state[u0 + q]);
        float out_v;
        int out_i;
        topk_of_lists<kTopKMaxSplits>(
            S, K, lane,
            [&](int l, int p, float& v, int& i) {
                const TopkEntry e = ws_list[(u0 + l) * K + p];
                v = e.v;
                i = e.i;
            },
            out_v, out_i);
        if (lane < K) {
            probs[row * K + lane] = exp_e(out_v - r.m) * rcp(r.d);
            idx[row * K + lane] = out_i;
        }
    }
}

// ---------------------------------------------------------------------------
// Plain 128-bit copy (bandwidth reference and counter calibration): each
// thread moves one 16-byte vector, 256-thread workgroups, one 4 KiB tile each
// (striding over further tiles past the grid cap).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) k_copy(const char* src, char* dst, int64_t bytes) {
    const uint32_t off = threadIdx.x * 16u;
    for (int64_t t0 = static_cast<int64_t>(blockIdx.x) * 4096; t0 < bytes; t0 += static_cast<int64_t>(gridDim.x) * 4096) {
        const int64_t left = bytes - t0;
        const uint32_t tile = static_cast<uint32_t>(left < 4096 ? left : 4096);
        const Buf bs(src + t0, tile), bd(dst + t0, tile);
        bd.store16(off, bs.load16<true>(off));
    }
}

// ---------------------------------------------------------------------------
// Plain 128-bit read (the read-only bandwidth reference, for kernels that only
// read, such as the fused top-K): each thread reads one 16-byte vector per
// 4 KiB tile, 256-thread workgroups striding over the tiles; each wave writes
// one float (its sum) to sink[workgroup * 4 + wave], so no load is dropped.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) k_read(const char* src, int64_t bytes, float* sink) {
    const uint32_t off = threadIdx.x * 16u;
    float acc = 0.0f;
    for (int64_t t0 = static_cast<int64_t>(blockIdx.x) * 4096; t0 < bytes; t0 += static_cast<int64_t>(gridDim.x) * 4096) {
        const int64_t left = bytes - t0;
        const Buf bs(src + t0, static_cast<uint32_t>(left < 4096 ? left : 4096));
        float x[4];
        Elt<false>::unpack(bs.load16<true>(off), x);
        acc += (x[0] + x[1]) + (x[2] + x[3]);
    }
    acc = wave_sum(acc);
    if ((threadIdx.x & (kWave - 1)) == 0) sink[static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / kWave] = acc;
}

// ---------------------------------------------------------------------------
// Copy with the register-resident forward's access pattern on rows of up to
// 128 KiB: one 1024-lane workgroup per row, 8 vectors per lane (slot
// v * 1024 + lane), every load issued before any store.  It is the bandwidth
// ceiling of that pattern, the one k_resident<*, 1024, 8> runs at.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(1024) k_copy_rows(const char* src, char* dst, int64_t rows, uint32_t row_bytes) {
    constexpr int VPL = 8;
    const uint32_t tid = threadIdx.x;
    for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
        const Buf bs(src + row * row_bytes, row_bytes), bd(dst + row * row_bytes, row_bytes);
        u32x4 v[VPL];
#pragma unroll
        for (int i = 0; i < VPL; ++i) v[i] = bs.load16<true>((i * 1024u + tid) * 16u);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < VPL; ++i) bd.store16((i * 1024u + tid) * 16u, v[i]);
    }
}

// ---------------------------------------------------------------------------
// Rate of the hardware base-2 exponential (v_exp_f32), the second ceiling of
// the per-element work beside HBM (every element of a fold costs one).  Each
// lane runs `iters` rounds over CHAINS values; a round is one v_exp_f32 and
// one fused multiply-add per value, v <- 2^v * 0.5 - 0.5, which keeps v in
// [-0.15, 0.21).  CHAINS = 1: one dependent chain per lane (latency bound);
// CHAINS = 8: eight independent chains (throughput).  One float per lane is
// written so that no round can be dropped.
// ---------------------------------------------------------------------------
template <int CHAINS>
__global__ void __launch_bounds__(256) k_exp_rate(float* out, int iters) {
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    float v[CHAINS];
#pragma unroll
    for (int c = 0; c < CHAINS; ++c) v[c] = static_cast<float>(gid & 255) * (1.0f / 1024.0f) + c * (1.0f / 64.0f) - 0.25f;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int c = 0; c < CHAINS; ++c) v[c] = fmaf(__builtin_amdgcn_exp2f(v[c]), 0.5f, -0.5f);
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < CHAINS; ++c) s += v[c];
    out[gid] = s;
}

}  // namespace onorm
