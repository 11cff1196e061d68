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
// One workgroup = 8 waves = 256 query rows of one head (the outer loop over
// query blocks of "6.2 FlashAttention V2 chi tiết", section 2.2); each wave
// owns 32 query rows (its section 4.2: no exchange between waves), walks the
// key tiles of 64 keys in order, and keeps its rows' (m, l) and o~ in
// registers.  The workgroup stages each tile of K (row-major) and V
// (transposed) in LDS, double-buffered: the next tile's loads are in flight
// while the current one is used.
//
// The products are computed transposed, S^T = K Q^T and O^T = V^T P^T, with
// v_mfma_f32_32x32x16_bf16 (A: lane l holds row l % 32 and 8 consecutive k
// from 8 (l / 32); B: lane l holds column l % 32 and the same k; C: lane l
// holds column l % 32, rows 4 (l / 32) + 8 i + j in register 4 i + j; checked
// on the hardware).  A lane's column is then one query row, so the row
// statistics need one exchange between the two lane halves, and the
// accumulator registers of S^T are already the B operand of the second
// product: registers 8p .. 8p+7 of a 32-key block hold keys
// 16p + 4 (l / 32) + {0,1,2,3, 8,9,10,11}, and V^T is stored in LDS with the
// keys of each 16-key group in that order, so the matching A operand is one
// 16-byte read.
#pragma once

#include "os_device.hpp"

namespace onorm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kAttnD = 128;                // head dimension
constexpr int kAttnBc = 64;                // keys per tile
// 8 waves = 256 query rows per workgroup, one workgroup per CU at 2 waves per
// SIMD: each staged K/V tile feeds twice the products of a 4-wave workgroup
// (measured 870 -> 719 us on the 256-head 2048 x 128 workload; 16 waves
// would cap a lane at 128 VGPRs and spill)
constexpr int kAttnWaves = 8;              // waves per workgroup
constexpr int kAttnBr = 32 * kAttnWaves;   // query rows per workgroup
constexpr int kAttnKStride = kAttnD + 8;   // LDS row stride of a K tile (elements; +16 B against bank conflicts)
constexpr int kAttnVStride = kAttnBc + 8;  // LDS row stride of a V^T tile

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 r) { return __builtin_bit_cast(bf16x8, r); }

// Position of key kk (0..63) of a tile in its V^T row: within each group of
// 16 keys, the groups of 4 go in the order 0, 2, 1, 3 (keys 0-3, 8-11, 4-7,
// 12-15), so lane half h finds its 8 keys at positions 8h .. 8h + 7.
__device__ __forceinline__ int vt_pos(int kk) {
    const int g = (kk >> 2) & 3;
    return (kk & ~15) | (((g & 1) << 3) | ((g & 2) << 1)) | (kk & 3);
}

template <bool CAUSAL>
__global__ void __attribute__((amdgpu_flat_work_group_size(kAttnWaves * 64, kAttnWaves * 64), amdgpu_waves_per_eu(2)))
    k_attn_fwd(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
               uint16_t* __restrict__ o, float* __restrict__ lse, int64_t heads, int nq, int nk, float scale) {
    constexpr int NT = kAttnWaves * 64;        // threads
    constexpr int KV = kAttnBc * kAttnD / 8 / NT;  // K vectors per thread per tile
    constexpr int VK = kAttnBc * kAttnD / 8 / NT;  // V keys per thread per tile (one 8-dim chunk each)
    __shared__ __attribute__((aligned(16))) uint16_t sK[2][kAttnBc * kAttnKStride];
    __shared__ __attribute__((aligned(16))) uint16_t sV[2][kAttnD * kAttnVStride];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = tid / kWave;
    const int col = lane & 31;  // this lane's query row within the wave, and its MFMA row / column
    const int h = lane >> 5;    // lane half
    const float c = scale * kLog2e;
    const int nqb = (nq + kAttnBr - 1) / kAttnBr;
    const int64_t units = heads * nqb;

    static_assert(KV * NT * 8 == kAttnBc * kAttnD && (VK == 1 || VK == 2 || VK == 4), "staging shape");
    for (int64_t unit = blockIdx.x; unit < units; unit += gridDim.x) {
        // Workgroups go to the 8 XCDs in turn (unit % 8), and each XCD has its
        // own L2.  When the heads split evenly, all query blocks of a head run
        // on one XCD, so its K and V tiles are fetched into one L2, and every
        // XCD gets the same mix of long and short (causal) query blocks.
        // Measured on the 256-head 2048 x 128 workload: 963 -> 855 us, and
        // causal 865 -> 592 us (with heads in plain order one XCD drew the
        // longest causal blocks of every head).
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

        // tile staging: thread tid moves K vectors tid + NT r, and V keys
        // VK (tid % (64 / VK)) .. + VK - 1, dims 8 (tid / (64 / VK)), through one of two
        // register sets: tile j's loads go to set j % 2 two tiles before its
        // LDS store, so their latency hides behind two tiles of products
        struct Stage {
            u32x4 k[KV], v[VK];
        };
        Stage st0, st1;
        // Consecutive lanes take consecutive keys of one dim chunk, so a V^T
        // store instruction fills one LDS row across the banks (with the
        // chunk in the low lane bits, the 16 chunks' rows, 1152 bytes apart,
        // fell on the same banks)
        constexpr int VGROUPS = kAttnBc / VK;  // key groups per tile
        const int vkey0 = (tid % VGROUPS) * VK, vchunk = tid / VGROUPS;
        auto load_tile = [&](int t, Stage& sg) {
            const int key0 = t * kAttnBc;
#pragma unroll
            for (int r = 0; r < KV; ++r) {
                const int idx = tid + NT * r;
                sg.k[r] = bk.load16<true>((static_cast<uint32_t>(key0 + (idx >> 4)) * kAttnD + (idx & 15) * 8) * 2u);
            }
#pragma unroll
            for (int r = 0; r < VK; ++r)
                sg.v[r] = bv.load16<true>((static_cast<uint32_t>(key0 + vkey0 + r) * kAttnD + vchunk * 8) * 2u);
        };
        auto store_tile = [&](const Stage& sg, int buf) {
#pragma unroll
            for (int r = 0; r < KV; ++r) {
                const int idx = tid + NT * r;
                *reinterpret_cast<u32x4*>(&sK[buf][(idx >> 4) * kAttnKStride + (idx & 15) * 8]) = sg.k[r];
            }
            // transpose VK keys x 8 dims: dim dd of the keys becomes VK consecutive V^T entries
            const int pos = vt_pos(vkey0);
#pragma unroll
            for (int dd = 0; dd < 8; ++dd) {
                const int word = dd >> 1, hi = dd & 1;
                uint32_t e[VK];
#pragma unroll
                for (int r = 0; r < VK; ++r) e[r] = hi ? (sg.v[r][word] >> 16) : (sg.v[r][word] & 0xFFFFu);
                if constexpr (VK == 4)
                    *reinterpret_cast<u32x2*>(&sV[buf][(vchunk * 8 + dd) * kAttnVStride + pos]) =
                        u32x2{e[0] | (e[1] << 16), e[2] | (e[3] << 16)};
                else if constexpr (VK == 2)
                    *reinterpret_cast<uint32_t*>(&sV[buf][(vchunk * 8 + dd) * kAttnVStride + pos]) = e[0] | (e[1] << 16);
                else
                    sV[buf][(vchunk * 8 + dd) * kAttnVStride + pos] = static_cast<uint16_t>(e[0]);
            }
        };

        f32x16 oacc[kAttnD / 32];
#pragma unroll
        for (int db = 0; db < kAttnD / 32; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[db][i] = 0.0f;
        float m = -INFINITY;  // running maximum of this row's raw logits q.k
        float l = 0.0f;       // this lane's share of sum e^{(s - m) scale} (its half of the keys)

        load_tile(0, st0);
        store_tile(st0, 0);
        __syncthreads();
        // Q must be in registers before the loop: otherwise the compiler's
        // wait for Q's loads inside the first product also waits for the
        // next tiles' loads, every tile (measured 1018 -> 963 us)
        __builtin_amdgcn_s_waitcnt(0);
        load_tile(1, st1);
        // One tile: issue tile t + 2's loads into `cur` (free: it held tile t,
        // stored before this tile began), the products on LDS buffer t % 2,
        // then tile t + 1 from `nxt` into the other buffer.  The loads are
        // issued even past the last tile (keys past nk read nothing: the
        // buffer range check; causal tiles past the diagonal are real keys,
        // unused): a conditional load would make the compiler wait for it
        // together with `nxt`'s loads before the store.
        auto tile = [&](const int t, Stage& cur, const Stage& nxt) {
            const int buf = t & 1;
            load_tile(t + 2, cur);

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
                    const bf16x8 a = as_bf16x8(
                        *reinterpret_cast<const u32x4*>(&sK[buf][(mb * 32 + col) * kAttnKStride + ks * 16 + h * 8]));
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
            const float m_new = fmaxf(m, mt);  // finite from the first tile on (key 0 is visible to every row)
            const float alpha = __builtin_amdgcn_exp2f((m - m_new) * c);  // 0 on the first tile
            const float mc = m_new * c;
            m = m_new;
            // P = e^{(s - m) scale} as the B operand of O^T = V^T P^T, and this lane's row sum
            float rs = 0.0f;
            bf16x8 pb[4];
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    float e[8];
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        e[u] = __builtin_amdgcn_exp2f(fmaf(s[mb][8 * p + u], c, -mc));
                        rs += e[u];
                    }
                    pb[mb * 2 + p] = __builtin_bit_cast(
                        bf16x8, u32x4{pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3]), pack_bf16x2(e[4], e[5]),
                                      pack_bf16x2(e[6], e[7])});
                }
            l = fmaf(l, alpha, rs);
#pragma unroll
            for (int db = 0; db < kAttnD / 32; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
            // O^T += V^T P^T: 4 dim blocks x 4 k-steps of 16 keys
#pragma unroll
            for (int db = 0; db < kAttnD / 32; ++db)
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(
                        &sV[buf][(db * 32 + col) * kAttnVStride + (kk >> 1) * 32 + (kk & 1) * 16 + h * 8]));
                    oacc[db] = mfma32(a, pb[kk], oacc[db]);
                }
            }  // wave_live
            if (t + 1 < ntiles) {
                store_tile(nxt, buf ^ 1);
                __syncthreads();
            }
        };
        for (int t = 0; t < ntiles; t += 2) {
            tile(t, st0, st1);
            if (t + 1 < ntiles) tile(t + 1, st1, st0);
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
        __syncthreads();  // the next unit's first tile overwrites buffer 0
    }
}

}  // namespace onorm
