// os_attention.hpp -- attention forward on the online normalizer for gfx950:
// O = softmax(scale * Q K^T) V per head, with the running (m, l, o~) state of
// "OnlineSoftmax: Online normalizer calculation for softmax" (paper summary),
// section 7.2.3, in the delayed-rescaling form of "6.2 FlashAttention V2 chi
// tiết", sections 3.2 and 6.1: per tile of keys the state is rescaled by
// e^{m_old - m_new} and the tile's e^{s - m_new} V is added; O = o~ / l once,
// at the end.  The two products run on the bf16 MFMA units; the softmax state
// and the rescaling in fp32 registers.
//
// Layout: bf16 Q [heads, nq, 128], K and V [heads, nk, 128], O like Q; the
// per-row logsumexp L = m + ln l in fp32 [heads, nq].
//
// One workgroup = 4 waves = 128 query rows of one head (the outer loop over
// query blocks of "6.2 FlashAttention V2 chi tiết", section 2.2); each wave
// owns 32 query rows (its section 4.2: no exchange between waves), walks the
// key tiles of 64 keys in order, and keeps its rows' (m, l) and o~ in
// registers.  The workgroup loads each tile of K and V straight from global
// memory into LDS (buffer loads that write LDS, no register round trip),
// both row-major, double-buffered: tile t + 1's loads are in flight while
// tile t is used.
//
// The products are computed transposed, S^T = K Q^T and O^T = V^T P^T, with
// v_mfma_f32_32x32x16_bf16 (A: lane l holds row l % 32 and 8 consecutive k
// from 8 (l / 32); B: lane l holds column l % 32 and the same k; C: lane l
// holds column l % 32, rows 4 (l / 32) + 8 i + j in register 4 i + j; checked
// on the hardware).  A lane's column is then one query row, so the row
// statistics need one exchange between the two lane halves, and the
// accumulator registers of S^T are already the B operand of the second
// product: registers 8p .. 8p+7 of a 32-key block hold keys
// 16p + 4 (l / 32) + {0,1,2,3, 8,9,10,11}.  The matching A operand, V^T for
// those keys, comes from row-major V through gfx950's transposing LDS read
// (ds_read_b64_tr_b16), two reads of 4 keys each.
//
// The running maximum moves only when a tile's maximum exceeds it by more
// than 8 in log2 units: the weights e^{s - m} then stay below 2^8, and a wave
// whose rows all keep their maximum skips the rescaling of o~ and l.  In exact
// arithmetic the result does not depend on which m is used, since O = o~ / l
// and L = m + ln l are invariant under a common shift of the logits (the
// max-subtraction argument of "CUDA算子优化(3)：Softmax"); a larger m only
// keeps the exponentials from overflowing.
#pragma once

#include "os_device.hpp"

namespace onorm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kAttnD = 128;                // head dimension
constexpr int kAttnBc = 64;                // keys per tile
// 4 waves = 128 query rows per workgroup, two workgroups per CU (64 KB of
// LDS each) at 2 waves per SIMD.  Measured on the 256-head 2048 x 128
// workload against one 8-wave workgroup per CU with three LDS stages: 547 ->
// 547 us, causal 374 -> 345 us (the causal diagonal wastes less in 128-row
// blocks); 16 waves would cap a lane at 128 VGPRs and spill.
constexpr int kAttnWaves = 4;              // waves per workgroup
constexpr int kAttnBr = 32 * kAttnWaves;   // query rows per workgroup

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 r) { return __builtin_bit_cast(bf16x8, r); }

// One 16-byte buffer load per lane straight into LDS: lane l's 16 bytes land
// at lds + 16 l (lds: the wave's base, the same for every lane).  The whole
// byte offset goes in the per-lane offset, which the buffer's range check
// covers (the scalar offset is left 0: on this family it is not range-checked),
// so a load past the buffer's end reads nothing.
__device__ __forceinline__ void load_lds16(const Buf& b, uint16_t* lds, uint32_t off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(b.r, (__attribute__((address_space(3))) void*)lds, 16, off, 0, 0, 0);
}

// Meet the workgroup's other waves once this wave's loads into LDS, all but
// the newest `pending` of them, have landed.  No release fence: a fence here
// would also wait for the newest loads.  The empty asm keeps the compiler from
// moving LDS accesses across the barrier.
template <int PENDING>
__device__ __forceinline__ void lds_loads_barrier() {
    static_assert(PENDING >= 0 && PENDING < 16, "vmcnt field");
    __builtin_amdgcn_s_waitcnt(0x0F70 | PENDING);  // vmcnt(PENDING); expcnt, lgkmcnt unconstrained
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Four bf16 of one column of a 4 x 16 block, transposed across a 16-lane
// group: lane 4e + q names row e, elements 4q .. 4q + 3 of the block; lane j
// receives element j of rows 0 .. 3.
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* p) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(__attribute__((address_space(3))) void*)p);
    return __builtin_bit_cast(u32x2, r);
}

template <bool CAUSAL>
__global__ void __attribute__((amdgpu_flat_work_group_size(kAttnWaves * 64, kAttnWaves * 64), amdgpu_waves_per_eu(2)))
    k_attn_fwd(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
               uint16_t* __restrict__ o, float* __restrict__ lse, int64_t heads, int nq, int nk, float scale) {
    constexpr int NT = kAttnWaves * 64;             // threads
    constexpr int CH = kAttnBc * kAttnD / 8 / NT;   // 16-byte chunks of K (and of V) per thread per tile
    constexpr int TILE = kAttnBc * kAttnD;          // elements of one K or V tile
    // Two stages of K and V (16 KB each), as separate arrays so that the
    // compiler tells them apart when it waits for the loads into one of them.
    // K rows keep their 16 chunks of 16 bytes at positions chunk ^ (row % 16),
    // V rows at chunk ^ 4 (row % 4): both reads below then spread a
    // wavefront's quarter over all LDS banks.
    __shared__ __attribute__((aligned(16))) uint16_t sK0[TILE];
    __shared__ __attribute__((aligned(16))) uint16_t sK1[TILE];
    __shared__ __attribute__((aligned(16))) uint16_t sV0[TILE];
    __shared__ __attribute__((aligned(16))) uint16_t sV1[TILE];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = tid / kWave;
    const int col = lane & 31;  // this lane's query row within the wave, and its MFMA row / column
    const int h = lane >> 5;    // lane half
    const float c = scale * kLog2e;
    const int nqb = (nq + kAttnBr - 1) / kAttnBr;
    const int64_t units = heads * nqb;
    static_assert(CH * NT * 8 == TILE, "staging shape");

    // this thread's staging chunks: position tid + NT r of a tile, row
    // (tid + NT r) / 16; the global chunk it loads is the one that position holds
    uint32_t koff[CH], voff[CH];  // byte offsets within a tile
#pragma unroll
    for (int r = 0; r < CH; ++r) {
        const int idx = tid + NT * r;
        const int row = idx >> 4;
        koff[r] = static_cast<uint32_t>(row * kAttnD + (((idx & 15) ^ (row & 15)) * 8)) * 2u;
        voff[r] = static_cast<uint32_t>(row * kAttnD + (((idx & 15) ^ ((row & 3) << 2)) * 8)) * 2u;
    }
    // the transposed V reads: this lane's row e and dims 4q .. 4q + 3 of its
    // group's 4 x 16 block
    const int tr_e = (lane >> 2) & 3, tr_q = lane & 3, tr_g = lane >> 4;

    for (int64_t unit = blockIdx.x; unit < units; unit += gridDim.x) {
        // Workgroups go to the 8 XCDs in turn (unit % 8), and each XCD has its
        // own L2.  When the heads split evenly, all query blocks of a head run
        // on one XCD, so its K and V tiles are fetched into one L2, and every
        // XCD gets the same mix of long and short (causal) query blocks.
        int64_t head = unit / nqb;
        int qbi = static_cast<int>(unit - head * nqb);
        if (heads % 8 == 0) {
            const int64_t slot = unit >> 3;
            head = (slot / nqb) * 8 + (unit & 7);
            qbi = static_cast<int>(slot % nqb);
        }
        // causal: the longest query blocks (most key tiles) first
        const int qb = CAUSAL ? nqb - 1 - qbi : qbi;
        const int q0 = qb * kAttnBr;
        const int qrow = q0 + w * 32 + col;  // this lane's query row
        const Buf bq(q + head * nq * kAttnD, static_cast<uint32_t>(nq) * kAttnD * 2u);
        const Buf bk(k + head * nk * kAttnD, static_cast<uint32_t>(nk) * kAttnD * 2u);
        const Buf bv(v + head * nk * kAttnD, static_cast<uint32_t>(nk) * kAttnD * 2u);
        const int kv_end = CAUSAL ? (q0 + kAttnBr < nk ? q0 + kAttnBr : nk) : nk;
        const int ntiles = (kv_end + kAttnBc - 1) / kAttnBc;

        // Q^T as the B operand of S^T = K Q^T: 8 k-steps of 16 dims, 8 dims per lane
        bf16x8 qb8[kAttnD / 16];
#pragma unroll
        for (int ks = 0; ks < kAttnD / 16; ++ks)
            qb8[ks] = as_bf16x8(bq.load16<true>((static_cast<uint32_t>(qrow) * kAttnD + ks * 16 + h * 8) * 2u));

        // tile t's K and V into one stage: CH loads of each per thread, one
        // wavefront's load filling 1 KB of the stage.  Keys past nk read
        // nothing (the buffer range check); causal tiles past the diagonal
        // are real keys, unused.
        auto load_tile = [&](int t, uint16_t* sk, uint16_t* sv) {
            const uint32_t tile_off = static_cast<uint32_t>(t) * (kAttnBc * kAttnD * 2);
#pragma unroll
            for (int r = 0; r < CH; ++r) load_lds16(bk, sk + (w * 64 + NT * r) * 8, tile_off + koff[r]);
#pragma unroll
            for (int r = 0; r < CH; ++r) load_lds16(bv, sv + (w * 64 + NT * r) * 8, tile_off + voff[r]);
        };

        f32x16 oacc[kAttnD / 32];
#pragma unroll
        for (int db = 0; db < kAttnD / 32; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[db][i] = 0.0f;
        float m = -INFINITY;  // running maximum of this row's raw logits q.k
        float l = 0.0f;       // this lane's share of sum e^{(s - m) scale} (its half of the keys)

        load_tile(0, sK0, sV0);
        // Q and tile 0 here, for every wave
        lds_loads_barrier<0>();
        // One tile: issue tile t + 1's loads into stage (t + 1) % 2 (last read
        // by tile t - 1, which every wave left at the barrier ending it), the
        // products on stage t % 2, then wait for tile t + 1's loads and meet
        // the other waves.
        auto tile = [&](const int t, const uint16_t* sk, const uint16_t* sv, uint16_t* nk_, uint16_t* nv_) {
            load_tile(t + 1, nk_, nv_);

            // causal: a tile whose first key lies past this wave's last row adds nothing to it
            const bool wave_live = !CAUSAL || (t * kAttnBc <= q0 + w * 32 + 31);
            if (wave_live) {
            // S^T = K Q^T for the tile's two 32-key blocks
            f32x16 s[2];
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
                for (int i = 0; i < 16; ++i) s[mb][i] = 0.0f;
#pragma unroll
                for (int ks = 0; ks < kAttnD / 16; ++ks) {
                    const int row = mb * 32 + col;
                    const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(
                        &sk[row * kAttnD + (((2 * ks + h) ^ (col & 15)) * 8)]));
                    s[mb] = mfma32(a, qb8[ks], s[mb]);
                }
            }
            // mask keys past the end, and (causal) keys after the query row
            const int key0 = t * kAttnBc;
            const bool edge = (key0 + kAttnBc > nk) | (CAUSAL & (key0 + kAttnBc - 1 > q0 + w * 32));
            if (edge) {
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const int key = key0 + mb * 32 + 4 * h + 8 * i + j;
                            const bool hide = (key >= nk) | (CAUSAL & (key > qrow));
                            s[mb][4 * i + j] = hide ? -INFINITY : s[mb][4 * i + j];
                        }
            }
            // the row's new maximum: this lane's 32 keys, then the other half's
            float mt = -INFINITY;
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s[mb][i]);
            {
                const f32x2 x = swap_rows32(mt);
                mt = fmaxf(x[0], x[1]);
            }
            // keep the running maximum unless the tile's exceeds it by more than
            // 8 in log2 units (weights then stay below 2^8); skip the rescaling
            // of o~ when no row of the wave moves its maximum
            const bool grow = (mt - m) * c > 8.0f;  // true on the first tile (m = -inf)
            float alpha = 1.0f;
            if (__builtin_amdgcn_ballot_w64(grow) != 0) {
                const float m_new = grow ? mt : m;
                alpha = __builtin_amdgcn_exp2f((m - m_new) * c);  // 0 on the first tile, 1 where kept
                m = m_new;
#pragma unroll
                for (int db = 0; db < kAttnD / 32; ++db)
#pragma unroll
                    for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
            }
            const float mc = m * c;
            // P = e^{(s - m) scale} as the B operand of O^T = V^T P^T, and this
            // lane's row sum, one k-step of 16 keys at a time, each followed
            // by its products: O^T += V^T P^T over the 4 dim blocks.  The A
            // operand of step kk = 2 mb + p holds, for this lane's dim, keys
            // 32 mb + 16 p + 4 h + {0..3} and the same + 8 (the order of P^T's
            // registers): two transposed reads of 4 keys each.  Each dim
            // block still adds its k-steps in order 0..3.
            float rs = 0.0f;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int mb = kk >> 1, p = kk & 1;
                float e[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    e[u] = __builtin_amdgcn_exp2f(fmaf(s[mb][8 * p + u], c, -mc));
                    rs += e[u];
                }
                const bf16x8 pbk = __builtin_bit_cast(
                    bf16x8, u32x4{pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3]), pack_bf16x2(e[4], e[5]),
                                  pack_bf16x2(e[6], e[7])});
                const int row = 16 * kk + 4 * h + tr_e;  // 32 mb + 16 p = 16 kk
#pragma unroll
                for (int db = 0; db < kAttnD / 32; ++db) {
                    const int dd = db * 32 + 16 * (tr_g & 1) + 4 * tr_q;  // first of this lane's 4 dims
                    const int pos = ((dd >> 3) ^ (tr_e << 2)) * 8 + (dd & 7);
                    const u32x2 lo = lds_read_tr16(&sv[row * kAttnD + pos]);
                    const u32x2 hi = lds_read_tr16(&sv[(row + 8) * kAttnD + pos]);
                    const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
                    oacc[db] = mfma32(a, pbk, oacc[db]);
                }
            }
            l = fmaf(l, alpha, rs);
            }  // wave_live
            if (t + 1 < ntiles) {
                // tile t + 1's loads
                lds_loads_barrier<0>();
            }
        };
        for (int t = 0; t < ntiles; t += 2) {
            tile(t, sK0, sV0, sK1, sV1);
            if (t + 1 < ntiles) tile(t + 1, sK1, sV1, sK0, sV0);
        }
        // the row's sum over both halves; O = o~ / l
        {
            const f32x2 x = swap_rows32(l);
            l = x[0] + x[1];
        }
        const float inv_l = rcp(l);
        const Buf bo(o + head * nq * kAttnD, static_cast<uint32_t>(nq) * kAttnD * 2u);
#pragma unroll
        for (int db = 0; db < kAttnD / 32; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int d0 = db * 32 + 4 * h + 8 * i;
                const uint32_t lo = pack_bf16x2(oacc[db][4 * i] * inv_l, oacc[db][4 * i + 1] * inv_l);
                const uint32_t hi = pack_bf16x2(oacc[db][4 * i + 2] * inv_l, oacc[db][4 * i + 3] * inv_l);
                __builtin_amdgcn_raw_buffer_store_b64(u32x2{lo, hi}, bo.r,
                                                      (static_cast<uint32_t>(qrow) * kAttnD + d0) * 2u, 0, 0);
            }
        if ((lse != nullptr) & (h == 0) & (qrow < nq))
            lse[head * nq + qrow] = fmaf(m, scale, __builtin_amdgcn_logf(l) * kLn2);
        // the loads issued past the last tile land before the next unit reuses the stages
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }
}

}  // namespace onorm
