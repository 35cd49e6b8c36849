// MFMA GEMM for the projector's Linear layers on gfx950.
//
// Every Linear of the projector ("Qwen3.8-27B-KVA" model card, "What the
// hell?": the input Linear, the blocks' Q/K/V/O and SwiGLU matrices, and the
// per-layer heads) is C = A * W^T with A the activations [tokens][in] and W
// the weight [out][in], both contiguous along `in`.  That is exactly the
// operand layout of the 32x32x16 MFMA: each lane feeds 8 consecutive
// K-values of one row of A and 8 consecutive K-values of one row of W.
//
// One kernel, gemm_t32, with fused epilogues (fp32 split-K partial, fp16
// Q|K plus transposed V, SwiGLU, bias + per-head scatter).  Activations are
// 16-bit in the tiled32_index layout; weights are 16-bit in the same layout
// (fp16 trunk, bf16 heads) or q8_0 (int8 codes + fp16 scales, tiled the same
// way, so a slab's weight bytes are half those of fp16).  Workgroup ids are
// remapped so that the tiles of one weight strip (all M-tiles of an N-tile)
// run back to back on the same XCD and share its L2: the hardware deals
// workgroups to the 8 XCDs round-robin.  Accumulation is fp32, over K in
// plain sequential order.
#include "kva_internal.h"
#include "kva_kv.h"

#include <type_traits>

namespace kva {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));


template <bool BF16>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    if constexpr (BF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint16_t to_f16_bits(float v) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(v));
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) void* gbl_ptr_t;

// Output element (lane, r) of a 32x32 MFMA tile sits at
//   row = 8*(r/4) + 4*(lane/32) + r%4,  col = lane%32.
//
// Fused epilogue of a BM x BN tile held as 32x32 MFMA accumulators by a
// WGM x WGN grid of waves (acc[i][j]: the wave's i-th 32-row, j-th 32-column
// block).  `smem` (SMEM_BYTES, free when called) is used by the head
// epilogue to turn whole-head tiles into full-row stores.
// Stores of rows past a call's M land here (one word per lane; never read).
__device__ float g_discard[64];

// A workgroup barrier for LDS hand-offs only: this wave's LDS accesses have
// completed (lgkmcnt(0)) when it arrives, and there is no memory fence, so
// the global stores already issued (the epilogue's output rows) keep
// draining across it.  __syncthreads' release fence would wait for them
// first, although no wave reads another wave's global writes here.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x3 << 14));   // lgkmcnt(0); vmcnt, expcnt untouched
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    __asm__ volatile("" ::: "memory");
}

template <int BM, int BN, int WGM, int WGN, int EPI, int MI, int NI, int SMEM_BYTES>
__device__ __forceinline__ void epilogue(const GemmArgs& g, f32x16 (&acc)[MI][NI], int tm, int tn, int split,
                                         uint16_t* smem) {
    constexpr int NW = WGM * WGN;
    constexpr int WM = BM / WGM, WN = BN / WGN;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WGN, wn = wave % WGN;
    const int row_base = tm * BM + wm * WM + 4 * (lane >> 5);
    const int col_base = tn * BN + wn * WN + (lane & 31);
    const EpiArgs& e = g.epi;

    if constexpr (EPI == EPI_PARTIAL || EPI == EPI_INPUT) {
        float* out = e.out_f32 + (int64_t)split * g.split_stride;
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            const int col = col_base + j * 32;
            if (col >= e.n_real) continue;
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = row_base + i * 32 + 8 * (r >> 2) + (r & 3);
                    if (row < g.M) out[(int64_t)row * e.ld_f32 + col] = acc[i][j][r];
                }
        }
    } else if constexpr (EPI == EPI_QKV) {
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            const int col = col_base + j * 32;
            if (col >= e.n_real) continue;
            if (col < e.n_split) {
                const float qs = col < e.n_split / 2 ? kAttnQScale : 1.0f;   // Q | K
#pragma unroll
                for (int i = 0; i < MI; ++i)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int row = row_base + i * 32 + 8 * (r >> 2) + (r & 3);
                        if (row < g.M) e.out16[(int64_t)row * e.ld16 + col] = to_f16_bits(acc[i][j][r] * qs);
                    }
            } else {
                // V^T: the lane's 4 consecutive rows are 4 consecutive tokens
                uint16_t* vt = e.vt + (int64_t)(col - e.n_split) * e.ld_vt;
#pragma unroll
                for (int i = 0; i < MI; ++i)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int row = row_base + i * 32 + 8 * q;
                        if (row < g.M) {
                            u32x2 pk;
                            pk[0] = (uint32_t)to_f16_bits(acc[i][j][4 * q + 0]) |
                                    ((uint32_t)to_f16_bits(acc[i][j][4 * q + 1]) << 16);
                            pk[1] = (uint32_t)to_f16_bits(acc[i][j][4 * q + 2]) |
                                    ((uint32_t)to_f16_bits(acc[i][j][4 * q + 3]) << 16);
                            *(u32x2*)(vt + row) = pk;
                        }
                    }
            }
        }
    } else if constexpr (EPI == EPI_SWIGLU) {
        static_assert(NI % 2 == 0, "gate/up pairs need an even number of 32-column tiles");
#pragma unroll
        for (int j = 0; j < NI; j += 2) {
            const int f = (tn * BN + wn * WN + j * 32) / 2 + (lane & 31);
            if (2 * f >= e.n_real) continue;
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = row_base + i * 32 + 8 * (r >> 2) + (r & 3);
                    if (row < g.M)
                        e.out16[tiled32_index(row, f, e.ld16)] = to_f16_bits(silu(acc[i][j][r]) * acc[i][j + 1][r]);
                }
        }
    } else if constexpr (EPI == EPI_HEADS) {
        static_assert(kHeadTileN % BN == 0, "a GEMM tile lies inside one packed 256-column tile");
        const int t256 = tn * BN / kHeadTileN;          // packed tile holding this GEMM tile
        const int th = e.tile_head[t256];
        // A whole-head tile goes out through LDS when it feeds the fused KV
        // epilogue (k_norm needs a token's 256 columns in one wave), and for
        // plain outputs of a 256-row tile whose destination rows are 16-byte
        // aligned: CR rows x 256 fp32 at a time are transposed there and
        // leave as full 1 KB rows, one row per wave and 4 columns per lane
        // (a quarter of the store instructions of the direct path).
        if constexpr (BN == kHeadTileN && WGN == 4) {
            const int slot = (th >= 0 && e.kv_n > 0) ? e.kv_slot[th] : -1;
            const bool plain = BM == 256 && WGM == 2 && th >= 0 && (e.heads.ld[th] % 4) == 0 &&
                               ((uintptr_t)e.heads.ptr[th] % 16) == 0;
            if (slot >= 0 || plain) {
                constexpr int CR0 = (SMEM_BYTES / (BN * 4)) / 32 * 32;
                constexpr int CR = CR0 < WM ? CR0 : WM;       // rows staged at a time
                static_assert(CR >= 32 && WM % CR == 0 && CR % NW == 0, "epilogue staging");
                float* lds = reinterpret_cast<float*>(smem);   // [CR][256], rows rotated by 32 every 4 rows
                const float* bias = e.bias ? e.bias + tn * BN : nullptr;
                const int part = e.tile_col0[t256] / kKvHeadDim;   // KV tile: 0..3 k, 4..7 v of that KV head
                const bool is_k = part < kKvHeads;
                const int kvh = is_k ? part : part - kKvHeads;
                const KvPool* pool = slot >= 0 ? &e.kv_pool[slot] : nullptr;
                float* dst0 = slot >= 0 ? nullptr : e.heads.ptr[th] + e.tile_col0[t256];
                const int64_t ld = slot >= 0 ? 0 : e.heads.ld[th];
                constexpr int NC = WM / CR;                     // staging steps per wave row
                KvLane kl{};
                if (slot >= 0 && is_k) kl = kv_lane_setup(lane, pool->k_gain, e.kv_rope);
                const int c4 = lane * 4;
                const float4 b = bias ? *(const float4*)(bias + c4) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
                for (int half = 0; half < WGM; ++half) {
#pragma unroll
                    for (int c = 0; c < NC; ++c) {
                        if (wm == half) {
#pragma unroll
                            for (int j = 0; j < NI; ++j)
#pragma unroll
                                for (int ii = 0; ii < CR / 32; ++ii)
#pragma unroll
                                    for (int r = 0; r < 16; ++r) {
                                        const int lr = ii * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                                        const int lc = wn * WN + j * 32 + (lane & 31);
                                        lds[lr * BN + ((lc + 32 * ((lr >> 2) & 1)) & (BN - 1))] =
                                            acc[c * (CR / 32) + ii][j][r];
                                    }
                        }
                        lds_barrier();
                        // CR rows x 64 chunks of 4 columns; one wave takes one full row
                        const int row0 = tm * BM + half * WM + c * CR;
                        if (slot < 0) {
                            // all of the wave's rows read first, then stored: each store
                            // keeps its own source registers, so no store waits for the
                            // previous one to have read its data (one register set
                            // reused across the rows made every store wait for the one
                            // before it to complete: 9.6 -> 7.8 us per 256x256 tile)
                            float4 rv[CR / NW];
#pragma unroll
                            for (int q = 0; q < CR / NW; ++q) {
                                const int lr = q * NW + wave;
                                rv[q] = *(const float4*)(lds + lr * BN + ((c4 + 32 * ((lr >> 2) & 1)) & (BN - 1)));
                            }
                            if (bias) {
#pragma unroll
                                for (int q = 0; q < CR / NW; ++q) {
                                    rv[q].x += b.x; rv[q].y += b.y; rv[q].z += b.z; rv[q].w += b.w;
                                }
                            }
#pragma unroll
                            for (int q = 0; q < CR / NW; ++q) {
                                const int lr = q * NW + wave;
                                if (row0 + lr < g.M) *(float4*)(dst0 + (int64_t)(row0 + lr) * ld + c4) = rv[q];
                            }
                        } else {
                            // the physical pages of this wave's rows, one per lane,
                            // fetched together before the row loop
                            int my_pg = -1;
                            if (lane < CR / NW && row0 + lane * NW + wave < g.M)
                                my_pg = kv_page(*pool, e.kv_pos0 + row0 + lane * NW + wave);
                            // not unrolled: the KV row code is large, and unrolled
                            // copies of it would crowd the instruction cache
#pragma unroll 1
                            for (int q = 0; q < CR / NW; ++q) {
                                const int lr = q * NW + wave;
                                const int row = row0 + lr;
                                if (row >= g.M) break;             // uniform over the wave; rows ascend
                                float4 v = *(const float4*)(lds + lr * BN + ((c4 + 32 * ((lr >> 2) & 1)) & (BN - 1)));
                                if (bias) { v.x += b.x; v.y += b.y; v.z += b.z; v.w += b.w; }
                                const int64_t p = e.kv_pos0 + row;
                                const int pg = __shfl(my_pg, q);
                                if (is_k) v = kv_k_norm_rope(v, lane, p, kl, e.kv_rope.n_rot, e.kv_rope.eps);
                                if (pg >= 0) kv_store_row(*pool, is_k, kv_row_index(*pool, pg, p, kvh), lane, v);
                            }
                        }
                        lds_barrier();
                    }
                }
                return;
            }
        }
        // a KV head's tiles leave only through the staged path above (the
        // launch keeps them 256 columns wide); never store them as fp32
        if (th >= 0 && e.kv_n > 0 && e.kv_slot[th] >= 0) return;
        // The bias is added in place, so every store reads its own accumulator
        // register (a sum in one reused temporary made each store wait for
        // the previous one to complete).
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            const int col = col_base + j * 32;
            const float b = e.bias ? e.bias[col] : 0.0f;
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] += b;
        }
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            const int col = col_base + j * 32;
            float* dst;
            int64_t ld;
            if (th >= 0) {
                dst = e.heads.ptr[th] + e.tile_col0[t256] + (col - t256 * kHeadTileN);
                ld = e.heads.ld[th];
            } else {
                const int c = col - e.tail_start;
                const int h = e.tail_head[c];
                if (h < 0) continue;
                dst = e.heads.ptr[h] + e.tail_col[c];
                ld = e.heads.ld[h];
            }
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    // rows past M go to a discard word instead of a branch per
                    // store (a store under its own branch gets its sum formed
                    // there, in one reused register, and waits for the last)
                    const int row = row_base + i * 32 + 8 * (r >> 2) + (r & 3);
                    float* p = row < g.M ? dst + (int64_t)row * ld : &g_discard[lane];
                    *p = acc[i][j][r];
                }
        }
    }
}

// The input GEMM's operand arithmetic (EPI_INPUT), the same for every tile
// shape so that a row's bits never depend on the tile a call takes:
//  - four activations x (one 16-byte chunk of a row, K-values 4c..4c+3) and
//    their norm gains -> fp16(x * gain), two per dword (whole-vector casts: a
//    bit cast of one vector element compiled to element 0 for every index);
//  - the chunk's sum of squares, x0^2 + x1^2 + x2^2 + x3^2 in this order.
// A row's sum of squares over a K range is then, per chunk position c of the
// 32-wide slabs, S_c = the slabs' chunk sums added in slab order, and the
// total ((S0 + S1) + (S2 + S3)) + ((S4 + S5) + (S6 + S7)).
__device__ __forceinline__ u32x2 input_f16x4(f32x4 x, f32x4 gv) {
    u32x2 o;
    o[0] = (uint32_t)to_f16_bits(x[0] * gv[0]) | ((uint32_t)to_f16_bits(x[1] * gv[1]) << 16);
    o[1] = (uint32_t)to_f16_bits(x[2] * gv[2]) | ((uint32_t)to_f16_bits(x[3] * gv[3]) << 16);
    return o;
}
__device__ __forceinline__ float input_chunk_sq(f32x4 x) {
    return __builtin_fmaf(x[3], x[3], __builtin_fmaf(x[2], x[2], __builtin_fmaf(x[1], x[1], x[0] * x[0])));
}

// K is walked in 32-wide slabs through a ring of S LDS stages.
//  - A slab's A rows and B rows are each one contiguous block in global
//    memory (the tiled layouts), copied straight into LDS with
//    global_load_lds (1 KB per wave instruction; the q8_0 scales a few
//    dozen bytes per wave).
//    S - 1 slabs are in flight while one is consumed, which covers the L2
//    latency at full MFMA rate.
//  - The MFMA fragments are double-buffered in registers: the LDS reads of
//    the next 16-wide K step are issued before the MFMAs of the current one,
//    including across the slab barrier, so LDS latency hides behind MFMAs.
//    q8_0: a lane's weight fragment (8 codes of one row and that row's block
//    scale) is read raw and turned into fp16 after the current MFMAs are
//    issued: d*q is one correctly rounded fp16 multiply, which is exactly the
//    fp32 product d*q (11 x 8 significant bits) rounded once to fp16.
//  - The K order of the accumulation is the plain one (slab by slab, step by
//    step) for every tile shape, so the tile choice never changes the bits.
//  - Each slab ends with one barrier: it publishes the next slab (every wave
//    has waited for its own DMA of it) and frees the stage the next DMA
//    refills.
//  - Split-K (EPI_PARTIAL only): the slabs are cut into `splits` consecutive
//    ranges, one per workgroup, each writing its own partial buffer.
// Tiles: 256x256 with 2 x 4 waves of 128 x 64, or 128x128 (small enough in
// LDS for two or three workgroups per CU) with 2 x 2 waves of 64 x 64, or for
// q8_0 (except SwiGLU, whose gate/up pairs need two 32-column blocks a wave)
// 1 x 4 waves of 128 x 32, so that each weight fragment is converted by one
// wave only.
template <int BM, int BN, int OPD, int EPI>
struct T32Shape {
    static constexpr bool Q8 = OPD == OPD_Q8;
    static constexpr bool Q4 = OPD == OPD_Q4;
    static constexpr bool QW = Q8 || Q4;                            // block-quantised weights
    static constexpr int KB = 32;
    static constexpr int A_BYTES = BM * KB * 2;
    static constexpr int B_ROW = Q8 ? KB : Q4 ? KB / 2 : KB * 2;    // weight bytes of a row per slab
    static constexpr int B_BYTES = BN * B_ROW;
    static constexpr int S_BYTES = QW ? BN * 2 : 0;                 // fp16 block scales
    static constexpr int STAGE = A_BYTES + B_BYTES + S_BYTES;
    // the head epilogue stages whole 256-column tiles through LDS (128 KB at
    // a time for a 256-row tile)
    static constexpr bool LDS_EPI = EPI == EPI_HEADS && BN == kHeadTileN;
    // 64-row tiles (calls of at most 64 rows) stream every weight once from
    // few workgroups: a deeper ring keeps more slabs in flight
    static constexpr int S = (LDS_EPI && BM == 256) ? (128 * 1024 + STAGE - 1) / STAGE : (BM == 64 && EPI != EPI_HEADS) ? 8 : 4;
    static constexpr int BYTES = S * STAGE;
};

// Quantised weight fragment: codes (8 consecutive K-values of one row; q4_0
// uses the first dword) and the row's fp16 block scale -> 8 fp16 weights.
template <bool Q4>
__device__ __forceinline__ u32x4 q_fragment(u32x2 codes, uint16_t d_bits) {
    uint32_t o[4];
    if constexpr (Q4) q4_0_f16x8(codes[0], d_bits, o);
    else q8_0_f16x8(codes[0], codes[1], d_bits, o);
    u32x4 out;
#pragma unroll
    for (int h = 0; h < 4; ++h) out[h] = o[h];
    return out;
}

template <int BM, int BN, int WGM, int WGN, int OPD, int EPI>
__device__ __forceinline__ void t32_tile(const GemmArgs& g, int tm, int tn, int split, uint8_t* smem) {
    using Sh = T32Shape<BM, BN, OPD, EPI>;
    constexpr bool BF16 = OPD == OPD_BF16;
    constexpr bool Q4 = Sh::Q4;
    constexpr bool QW = Sh::QW;          // block-quantised weights (q8_0 or q4_0)
    constexpr int NW = WGM * WGN, KB = Sh::KB, S = Sh::S;
    constexpr int WM = BM / WGM, WN = BN / WGN, MI = WM / 32, NI = WN / 32;
    // DMA instructions per wave and slab: 16 bytes per lane, or 4 for a
    // weight slab too small to give every wave a whole kilobyte (q4_0)
    constexpr int BSZ = Sh::B_BYTES >= 1024 * NW ? 16 : 4;
    constexpr int AI = Sh::A_BYTES / (1024 * NW), BI = Sh::B_BYTES / (64 * BSZ * NW);
    // q8_0 scales: every wave copies an equal share of them (SL lanes x 4
    // bytes), so that every wave issues the same number of DMA instructions
    constexpr int SL = Sh::S_BYTES / (4 * NW);
    constexpr int L = AI + BI + (QW ? 1 : 0);
    static_assert(AI >= 1 && BI >= 1 && AI * 1024 * NW == Sh::A_BYTES && BI * 64 * BSZ * NW == Sh::B_BYTES,
                  "tile too small for the wave grid");
    static_assert(!QW || (SL >= 1 && SL <= 64 && SL * 4 * NW == Sh::S_BYTES), "scale DMA split");
    static_assert((S - 2) * L < 64, "vmcnt range");
    static_assert(!Sh::LDS_EPI || BM != 256 || Sh::BYTES >= 128 * 1024, "the head epilogue stages 128 KB through LDS");
    static_assert(kWeightTileRows % BM == 0 && kWeightTileRows % BN == 0, "tiles inside 256-row groups");
    const int SP = g.splits;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WGN, wn = wave % WGN;
    const int nk_all = g.K / KB;
    const int kb = split * nk_all / SP;                // this split's slabs: [kb, kb + nk)
    const int nk = (split + 1) * nk_all / SP - kb;
    // slab kt of the rows [r0, r0 + BM) of 256-row group t starts at element
    // (t * nk_all + kt) * 256 * KB + r0 * KB (q8_0 codes: bytes, scales: (..) * 256 + r0)
    const int64_t a_slab0 = ((int64_t)(tm * BM / kWeightTileRows) * nk_all + kb);
    const int64_t b_slab0 = ((int64_t)(tn * BN / kWeightTileRows) * nk_all + kb);
    const uint8_t* Ab = reinterpret_cast<const uint8_t*>(g.A) +
                        (a_slab0 * kWeightTileRows + (tm * BM) % kWeightTileRows) * KB * 2;
    const uint8_t* Bb = (QW ? reinterpret_cast<const uint8_t*>(g.Bq) : reinterpret_cast<const uint8_t*>(g.B)) +
                        (b_slab0 * kWeightTileRows + (tn * BN) % kWeightTileRows) * Sh::B_ROW;
    const uint8_t* Sb = QW ? reinterpret_cast<const uint8_t*>(g.Bs) +
                                 (b_slab0 * kWeightTileRows + (tn * BN) % kWeightTileRows) * 2
                           : nullptr;
    constexpr int64_t A_SLAB = (int64_t)kWeightTileRows * KB * 2;              // bytes between slabs
    constexpr int64_t B_SLAB = (int64_t)kWeightTileRows * Sh::B_ROW;
    constexpr int64_t S_SLAB = (int64_t)kWeightTileRows * 2;
    auto issue = [&](int kt, int st) {
        uint8_t* sa = smem + st * Sh::STAGE;
        uint8_t* sb = sa + Sh::A_BYTES;
#pragma unroll
        for (int i = 0; i < AI; ++i)
            __builtin_amdgcn_global_load_lds((gbl_ptr_t)(Ab + kt * A_SLAB + (i * NW + wave) * 1024 + lane * 16),
                                             (lds_ptr_t)(sa + (i * NW + wave) * 1024), 16, 0, 0);
#pragma unroll
        for (int i = 0; i < BI; ++i) {
            const uint8_t* src = Bb + kt * B_SLAB + (i * NW + wave) * 64 * BSZ + lane * BSZ;
            uint8_t* dst = sb + (i * NW + wave) * 64 * BSZ;
            if constexpr (BSZ == 16) __builtin_amdgcn_global_load_lds((gbl_ptr_t)src, (lds_ptr_t)dst, 16, 0, 0);
            else __builtin_amdgcn_global_load_lds((gbl_ptr_t)src, (lds_ptr_t)dst, 4, 0, 0);
        }
        if constexpr (QW) {
            if (lane < SL)
                __builtin_amdgcn_global_load_lds((gbl_ptr_t)(Sb + kt * S_SLAB + wave * SL * 4 + lane * 4),
                                                 (lds_ptr_t)(sb + Sh::B_BYTES + wave * SL * 4), 4, 0, 0);
        }
    };
    // vmcnt(n) with lgkmcnt / expcnt left alone; lgkmcnt(0) alone.  (The
    // builtin, unlike inline asm, is seen by the compiler's own wait
    // insertion, which then knows which LDS reads have landed.)
    auto vm_wait = [](auto n) {
        constexpr int N = decltype(n)::value;
        __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
    };
    auto lds_wait = []() { __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x3 << 14)); };
    f32x16 acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    const int frow = lane & 31, fk = lane >> 5;
    const int sw = tiled32_swizzle(frow);                // fragment rows differ by multiples of 32
    const int swq = Q4 ? (frow >> 3) & 3 : (frow >> 2) & 3;   // q4_0 / q8_0 code chunk swizzle
    int aoff[MI], boff[NI];
#pragma unroll
    for (int i = 0; i < MI; ++i) aoff[i] = (wm * WM + i * 32 + frow) * KB * 2;
#pragma unroll
    for (int j = 0; j < NI; ++j) boff[j] = Sh::A_BYTES + (wn * WN + j * 32 + frow) * Sh::B_ROW;
    // fragments: fa/fb ready for the MFMA; for q8_0, qc/qs hold the raw codes and scales
    u32x4 fa0[MI], fb0[NI], fa1[MI], fb1[NI];
    u32x2 qc0[NI], qc1[NI];
    uint16_t qs0[NI], qs1[NI];
    auto rd = [&](int st, int ks, u32x4* fa, u32x4* fb, u32x2* qc, uint16_t* qs) {
        const uint8_t* base = smem + st * Sh::STAGE;
        const int c = ((ks * 2 + fk) ^ sw) << 4;
#pragma unroll
        for (int i = 0; i < MI; ++i) fa[i] = *(const u32x4*)(base + aoff[i] + c);
        if constexpr (QW) {
            const int cq = ((ks * 2 + fk) ^ swq) << (Q4 ? 2 : 3);
#pragma unroll
            for (int j = 0; j < NI; ++j) {
                if constexpr (Q4) qc[j] = u32x2{*(const uint32_t*)(base + boff[j] + cq), 0u};
                else qc[j] = *(const u32x2*)(base + boff[j] + cq);
                qs[j] = *(const uint16_t*)(base + Sh::A_BYTES + Sh::B_BYTES + (wn * WN + j * 32 + frow) * 2);
            }
        } else {
#pragma unroll
            for (int j = 0; j < NI; ++j) fb[j] = *(const u32x4*)(base + boff[j] + c);
        }
    };
    auto cvt = [&](u32x4* fb, const u32x2* qc, const uint16_t* qs) {
        if constexpr (QW) {
#pragma unroll
            for (int j = 0; j < NI; ++j) fb[j] = q_fragment<Q4>(qc[j], qs[j]);
        }
    };
    auto mm = [&](const u32x4* fa, const u32x4* fb) {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NI; ++j) acc[i][j] = mfma32<BF16>(fa[i], fb[j], acc[i][j]);
    };

#pragma unroll
    for (int p = 0; p < S - 1; ++p)
        if (p < nk) issue(p, p);
    if (nk >= S - 1) vm_wait(std::integral_constant<int, (S - 2) * L>{});
    else vm_wait(std::integral_constant<int, 0>{});
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
    rd(0, 0, fa0, fb0, qc0, qs0);
    cvt(fb0, qc0, qs0);
    lds_wait();
    // Instruction order of one K step: the LDS reads of the next step first,
    // then the current MFMAs (q8_0: with the conversion of the next
    // fragments between their two halves; it waits for the reads, and the
    // first MFMAs cover that latency).
    auto order = [&]() {
        if constexpr (QW) {
            __builtin_amdgcn_sched_group_barrier(0x100, MI + 2 * NI, 0);   // LDS reads
            __builtin_amdgcn_sched_group_barrier(0x008, MI * NI / 2, 0);   // MFMAs
            __builtin_amdgcn_sched_group_barrier(0x002, 64, 0);            // VALU: conversion
            __builtin_amdgcn_sched_group_barrier(0x008, MI * NI / 2, 0);   // MFMAs
        } else {
            // one LDS read after each of the first MFMAs
#pragma unroll
            for (int q = 0; q < MI + NI; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, MI * NI - (MI + NI), 0);
        }
    };
    // q8_0 / q4_0 trunk GEMMs: the wave in its MFMA + conversion phase gets
    // issue priority over the other wave of its SIMD (measured: 3-6% faster;
    // the 16-bit path is faster without it, and so is the q8_0 head GEMM, by
    // 1.5%)
    auto prio = [](auto p) {
        if constexpr (QW && EPI != EPI_HEADS) {
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_setprio(decltype(p)::value);
        }
    };
    // one slab; MORE: a later slab is still to be issued (the drain of the
    // last S - 1 slabs runs as its own loop so that neither loop branches)
    auto slab = [&](int kt, auto more_c) {
        constexpr bool MORE = decltype(more_c)::value;
        // the stage of slab kt-1 was released by the previous barrier
        if constexpr (MORE) issue(kt + S - 1, (kt + S - 1) % S);
        rd(kt % S, 1, fa1, fb1, qc1, qs1);
        prio(std::integral_constant<int, 1>{});
        mm(fa0, fb0);
        cvt(fb1, qc1, qs1);
        order();
        prio(std::integral_constant<int, 0>{});
        __builtin_amdgcn_sched_barrier(0);      // the waits below stay after this step's MFMAs
        if constexpr (MORE) vm_wait(std::integral_constant<int, (S - 2) * L>{});   // slab kt+1 has landed
        else vm_wait(std::integral_constant<int, 0>{});
        lds_wait();                                                      // slab kt fully read
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        __asm__ volatile("" ::: "memory");
        // after the last slab this reads a stale stage (in bounds); the values are not used
        rd((kt + 1) % S, 0, fa0, fb0, qc0, qs0);
        prio(std::integral_constant<int, 1>{});
        mm(fa1, fb1);
        cvt(fb0, qc0, qs0);
        order();
        prio(std::integral_constant<int, 0>{});
        __builtin_amdgcn_sched_barrier(0);
        lds_wait();     // the next step's fragments: long landed, and now known to be
    };
    int kt = 0;
    for (; kt + S - 1 < nk; ++kt) slab(kt, std::true_type{});
    for (; kt < nk; ++kt) slab(kt, std::false_type{});
    if constexpr (Sh::LDS_EPI) __syncthreads();    // the head epilogue reuses LDS
    epilogue<BM, BN, WGM, WGN, EPI, MI, NI, Sh::BYTES>(g, acc, tm, tn, split, reinterpret_cast<uint16_t*>(smem));
}

// The input GEMM (EPI_INPUT: the input RMSNorm folded into the input
// Linear), on the tiles whose accumulators leave room for its registers
// (not 256x256: the host maps that choice to 128x256 or 128x128).  The fp32
// activation rows and the weight slabs come through registers, three slabs
// ahead, and are written to LDS by this kernel: the activations already as
// the fp16 operand fp16(x * gain) in the tiled32 slab layout, so that the
// MFMA fragment reads are those of t32_tile (fp32 rows in LDS would double
// them).  Per thread
// and slab: AQ 16-byte chunks of activation rows (8 threads to a row), one
// chunk of gains, BQ 16-byte pieces of the weight slab and, for code planes,
// one piece of its block scales (copies of their contiguous tiled blocks;
// threads past the last piece load it again and do not write it).  Two LDS
// stages, one barrier per slab; the MFMA order over K, the fragment layout
// and the dequantisation are those of t32_tile, and the row sums of squares
// follow input_chunk_sq's order (thread chunk c = t % 8 holds S_c).
template <int BM, int BN, int OPD>
struct InputShape {
    static constexpr bool QW = OPD == OPD_Q8 || OPD == OPD_Q4;
    static constexpr int KB = 32;
    static constexpr int B_ROW = OPD == OPD_Q8 ? KB : OPD == OPD_Q4 ? KB / 2 : KB * 2;
    static constexpr int A_BYTES = BM * KB * 2, B_BYTES = BN * B_ROW, S_BYTES = QW ? BN * 2 : 0;
    static constexpr int STAGE = A_BYTES + B_BYTES + S_BYTES;
    static constexpr int BYTES = 2 * STAGE;
};

template <int BM, int BN, int WGM, int WGN, int OPD>
__device__ __forceinline__ void t32_tile_input(const GemmArgs& g, int tm, int tn, int split, uint8_t* smem) {
    using Sh = InputShape<BM, BN, OPD>;
    constexpr bool QW = Sh::QW, Q4 = OPD == OPD_Q4;
    constexpr int NW = WGM * WGN, NT = 64 * NW, KB = Sh::KB;
    constexpr int WM = BM / WGM, WN = BN / WGN, MI = WM / 32, NI = WN / 32;
    constexpr int AQ = BM * KB / 4 / NT;          // activation chunks per thread and slab
    constexpr int NBP = Sh::B_BYTES / 16;         // weight pieces per slab
    constexpr int BQ = (NBP + NT - 1) / NT;       // weight pieces per thread and slab
    constexpr int NSP = Sh::S_BYTES / 16;         // scale pieces per slab (code planes)
    constexpr int SQ = QW ? 1 : 0;
    constexpr int RPQ = NT / 8;                   // rows covered by one chunk index q
    static_assert(AQ >= 1 && AQ * 4 * NT == BM * KB && NBP * 16 == Sh::B_BYTES && NSP <= NT, "input tile");
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WGN, wn = wave % WGN;
    const int nk_all = g.K / KB;
    const int kb = split * nk_all / g.splits;
    const int nk = (split + 1) * nk_all / g.splits - kb;
    const int c4 = tid & 7;                       // this thread's 4-value chunk of a slab row
    // activation sources (rows past M read row M - 1: in bounds, never stored)
    const float* X = reinterpret_cast<const float*>(g.A);
    const float* xs[AQ];
#pragma unroll
    for (int q = 0; q < AQ; ++q) {
        const int row = min(tm * BM + q * RPQ + (tid >> 3), g.M - 1);
        xs[q] = X + (int64_t)row * g.lda + (int64_t)kb * KB + c4 * 4;
    }
    const float* gs = g.epi.a_gain + (int64_t)kb * KB + c4 * 4;
    const int64_t b_slab0 = (int64_t)(tn * BN / kWeightTileRows) * nk_all + kb;
    const int64_t b_row0 = b_slab0 * kWeightTileRows + (tn * BN) % kWeightTileRows;
    const uint8_t* Bb = (QW ? reinterpret_cast<const uint8_t*>(g.Bq) : reinterpret_cast<const uint8_t*>(g.B)) +
                        b_row0 * Sh::B_ROW;
    const uint8_t* Sb = QW ? reinterpret_cast<const uint8_t*>(g.Bs) + b_row0 * 2 : nullptr;
    constexpr int64_t B_SLAB = (int64_t)kWeightTileRows * Sh::B_ROW;
    constexpr int64_t S_SLAB = (int64_t)kWeightTileRows * 2;
    int bp[BQ];                                    // this thread's weight pieces (clamped)
#pragma unroll
    for (int q = 0; q < BQ; ++q) bp[q] = min(q * NT + tid, NBP - 1) * 16;
    const int sp = QW ? min(tid, NSP - 1) * 16 : 0;
    // LDS byte offset of this thread's fp16 chunk of row r (tiled32 slab
    // layout: 64-byte rows, 16-byte chunk cc at cc ^ swizzle(r), 8 bytes = half)
    int a_dst[AQ];
#pragma unroll
    for (int q = 0; q < AQ; ++q) {
        const int r = q * RPQ + (tid >> 3);
        a_dst[q] = r * 64 + (((c4 >> 1) ^ tiled32_swizzle(r)) << 4) + (c4 & 1) * 8;
    }
    struct Regs {
        f32x4 a[AQ];
        f32x4 gn;
        u32x4 b[BQ];
        u32x4 sc[SQ > 0 ? SQ : 1];
    };
    Regs R0, R1, R2;
    auto load = [&](Regs& R, int kt) {
#pragma unroll
        for (int q = 0; q < AQ; ++q) R.a[q] = *(const f32x4*)(xs[q] + kt * KB);
        R.gn = *(const f32x4*)(gs + kt * KB);
#pragma unroll
        for (int q = 0; q < BQ; ++q) R.b[q] = *(const u32x4*)(Bb + kt * B_SLAB + bp[q]);
        if constexpr (QW) R.sc[0] = *(const u32x4*)(Sb + kt * S_SLAB + sp);
    };
    float S[AQ];                                   // running chunk sums of squares
#pragma unroll
    for (int q = 0; q < AQ; ++q) S[q] = 0.0f;
    // (valid false: a repeated last slab, written but not counted)
    auto commit = [&](Regs& R, int st, bool valid) {
        uint8_t* sa = smem + st * Sh::STAGE;
#pragma unroll
        for (int q = 0; q < AQ; ++q) {
            *(u32x2*)(sa + a_dst[q]) = input_f16x4(R.a[q], R.gn);
            S[q] += valid ? input_chunk_sq(R.a[q]) : 0.0f;
        }
#pragma unroll
        for (int q = 0; q < BQ; ++q)
            if (BQ * NT == NBP || q * NT + tid < NBP) *(u32x4*)(sa + Sh::A_BYTES + (q * NT + tid) * 16) = R.b[q];
        if constexpr (QW)
            if (tid < NSP) *(u32x4*)(sa + Sh::A_BYTES + Sh::B_BYTES + tid * 16) = R.sc[0];
    };
    f32x16 acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    const int frow = lane & 31, fk = lane >> 5;
    const int sw = tiled32_swizzle(frow);
    const int swq = Q4 ? (frow >> 3) & 3 : (frow >> 2) & 3;   // q4_0 / q8_0 code chunk swizzle
    int aoff[MI], boff[NI];
#pragma unroll
    for (int i = 0; i < MI; ++i) aoff[i] = (wm * WM + i * 32 + frow) * KB * 2;
#pragma unroll
    for (int j = 0; j < NI; ++j) boff[j] = Sh::A_BYTES + (wn * WN + j * 32 + frow) * Sh::B_ROW;
    u32x4 fa0[MI], fb0[NI], fa1[MI], fb1[NI];
    u32x2 qc0[NI], qc1[NI];
    uint16_t qs0[NI], qs1[NI];
    // code planes: the raw codes and scale of a weight fragment, turned into
    // fp16 weights by cvt after the current step's MFMAs are issued
    auto rd = [&](int st, int ks, u32x4* fa, u32x4* fb, u32x2* qc, uint16_t* qs) {
        const uint8_t* base = smem + st * Sh::STAGE;
        const int c = ((ks * 2 + fk) ^ sw) << 4;
#pragma unroll
        for (int i = 0; i < MI; ++i) fa[i] = *(const u32x4*)(base + aoff[i] + c);
        if constexpr (QW) {
            const int cq = ((ks * 2 + fk) ^ swq) << (Q4 ? 2 : 3);
#pragma unroll
            for (int j = 0; j < NI; ++j) {
                if constexpr (Q4) qc[j] = u32x2{*(const uint32_t*)(base + boff[j] + cq), 0u};
                else qc[j] = *(const u32x2*)(base + boff[j] + cq);
                qs[j] = *(const uint16_t*)(base + Sh::A_BYTES + Sh::B_BYTES + (wn * WN + j * 32 + frow) * 2);
            }
        } else {
#pragma unroll
            for (int j = 0; j < NI; ++j) fb[j] = *(const u32x4*)(base + boff[j] + c);
        }
    };
    auto cvt = [&](u32x4* fb, const u32x2* qc, const uint16_t* qs) {
        if constexpr (QW) {
#pragma unroll
            for (int j = 0; j < NI; ++j) fb[j] = q_fragment<Q4>(qc[j], qs[j]);
        }
    };
    auto mm = [&](const u32x4* fa, const u32x4* fb) {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NI; ++j) acc[i][j] = mfma32<false>(fa[i], fb[j], acc[i][j]);
    };
    // (the scheduling barriers keep the next commit's conversion, which waits
    // for the other register set, from being hoisted above the barrier)
    auto barrier = []() {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x3 << 14));   // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        __asm__ volatile("" ::: "memory");
    };
    // Every load is issued unconditionally (slab indexes clamped to the last
    // slab), so that the compiler's wait before a commit counts exactly the
    // other register set's loads as still in flight; a branch around the
    // loads made it wait for all of them.
    const int last = nk - 1;
    load(R0, 0);
    load(R1, min(1, last));
    load(R2, min(2, last));
    commit(R0, 0, true);
    load(R0, min(3, last));
    barrier();
    rd(0, 0, fa0, fb0, qc0, qs0);
    cvt(fb0, qc0, qs0);
    // slab kt from stage kt & 1; Rn holds slab kt + 1 (committed to the other
    // stage, whose last reader passed the previous barrier), then reloaded
    // with slab kt + 4: three slabs of loads in flight
    auto step = [&](int kt, Regs& Rn) {
        const int st = kt & 1;
        rd(st, 1, fa1, fb1, qc1, qs1);
        mm(fa0, fb0);
        cvt(fb1, qc1, qs1);
        commit(Rn, st ^ 1, kt + 1 < nk);
        load(Rn, min(kt + 4, last));
        barrier();
        rd(st ^ 1, 0, fa0, fb0, qc0, qs0);         // after the last slab: a stale stage, not used
        mm(fa1, fb1);
        cvt(fb0, qc0, qs0);
    };
    int kt = 0;
    for (; kt + 3 <= nk; kt += 3) {
        step(kt, R1);
        step(kt + 1, R2);
        step(kt + 2, R0);
    }
    if (kt < nk) step(kt, R1);
    if (kt + 1 < nk) step(kt + 1, R2);
    // S[q] of the 8 threads of a row are its chunk sums S_0..S_7 (thread
    // chunk c4): ((S0 + S1) + (S2 + S3)) + ((S4 + S5) + (S6 + S7))
    if (tn == 0) {
#pragma unroll
        for (int q = 0; q < AQ; ++q) {
            float v = S[q];
            v += __shfl_xor(v, 1);
            v += __shfl_xor(v, 2);
            v += __shfl_xor(v, 4);
            const int row = tm * BM + q * RPQ + (tid >> 3);
            if (c4 == 0 && row < g.M) g.epi.ss[split * g.epi.ss_stride + row] = v;
        }
    }
    epilogue<BM, BN, WGM, WGN, EPI_INPUT, MI, NI, 0>(g, acc, tm, tn, split, nullptr);
}

// Workgroup ids are dealt to the 8 XCDs round-robin; this remaps them so that
// consecutive tile indices run on one XCD (count: the grid, a multiple of 8).
__device__ __forceinline__ int xcd_remap(int bid, int count) { return (bid % 8) * (count / 8) + bid / 8; }

// EPI_INPUT runs t32_tile_input
template <int BM, int BN, int OPD, int EPI>
constexpr int kT32Smem = EPI == EPI_INPUT ? InputShape<BM, BN, OPD>::BYTES : T32Shape<BM, BN, OPD, EPI>::BYTES;

template <int BM, int BN, int WGM, int WGN, int OPD, int EPI>
__global__ void __launch_bounds__(64 * WGM * WGN) gemm_t32(GemmArgs g) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[kT32Smem<BM, BN, OPD, EPI>];
    const int mt = (g.M + BM - 1) / BM;
    const int nt = g.N / BN;
    const int total = mt * nt * g.splits;
    const int v = xcd_remap(blockIdx.x, gridDim.x);
    if (v >= total) return;
    // M-tiles fastest, then splits, then N-tiles: the tiles sharing a weight
    // strip run back to back on one XCD.  EPI_INPUT (fp32 activations, twice
    // the bytes of the weights' rows): M-tiles, then N-tiles, then splits, so
    // that an XCD's tiles read the activation rows of one K range only
    // (about 80 instead of 195 MB of L2 fills at 1024 tokens)
    if constexpr (EPI == EPI_INPUT)
        t32_tile_input<BM, BN, WGM, WGN, OPD>(g, v % mt, (v / mt) % nt, v / (mt * nt), smem);
    else
        t32_tile<BM, BN, WGM, WGN, OPD, EPI>(g, v % mt, v / (mt * g.splits), (v / mt) % g.splits, smem);
}

// The head GEMM in one launch of two parts: the first n_big 256-column
// N-tiles as 256x256 tiles (a whole number of rounds over the CUs), the
// remaining columns as 128 x SBN tiles (a quarter or half of the work), so
// that no round of 256x256 tiles is left partly empty.  Both tile shapes accumulate K
// in the same order: the split point never changes the bits.  SBN: 256 (a
// half tile: q8_0's 128-column weight slab is too small for 8 waves' DMA,
// and for bf16 it measured 0.5% faster than 128), 128 for q4_0.
template <int OPD>
constexpr int kTailBN = OPD == OPD_Q4 ? 128 : 256;

template <int OPD>
__global__ void __launch_bounds__(512) gemm_t32_heads(GemmArgs g, int n_big, int grid_big) {
    constexpr int SBN = kTailBN<OPD>;
    using ShB = T32Shape<256, 256, OPD, EPI_HEADS>;
    using ShS = T32Shape<128, SBN, OPD, EPI_HEADS>;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[ShB::BYTES > ShS::BYTES ? ShB::BYTES : ShS::BYTES];
    // The small tiles go first: the CUs that start with one finish it after
    // about half a 256x256 tile and from then on run their 256x256 tiles out
    // of phase with the others, so that the tiles' epilogues (each
    // writes 256 KB) are not all due at once (measured: 1.7% faster on r2,
    // 3% on r3, than with the small tiles last).
    const int grid_small = (int)gridDim.x - grid_big;
    if ((int)blockIdx.x >= grid_small) {
        const int mt = (g.M + 255) / 256;
        const int v = xcd_remap(blockIdx.x - grid_small, grid_big);
        if (v >= mt * n_big) return;
        t32_tile<256, 256, 2, 4, OPD, EPI_HEADS>(g, v % mt, v / mt, 0, smem);
    } else {
        const int mt = (g.M + 127) / 128;
        const int tn0 = n_big * (256 / SBN);            // first SBN-column tile
        const int v = xcd_remap(blockIdx.x, grid_small);
        if (v >= mt * (g.N / SBN - tn0)) return;
        t32_tile<128, SBN, 2, 4, OPD, EPI_HEADS>(g, v % mt, tn0 + v / mt, 0, smem);
    }
}

// Skinny GEMM: calls of at most 32 rows in contexts created for at most 32
// tokens per call.  Such a call reads every weight once and does little
// MFMA work per weight, so the tiled GEMM's LDS ring (a barrier per 32-wide
// slab, every wave waiting on the slowest DMA) is the wrong shape for it.
// Here the operands stream from global memory straight into the MFMA
// fragments of each wave (P slabs in flight per wave in registers, no LDS,
// no barrier in the K loop); the NWK waves of a workgroup share one block
// of 32 * NB output columns and each takes one contiguous range of the K
// slabs of the workgroup's split (blockIdx.y of g.splits, EPI_PARTIAL
// only); at the end the waves' partial sums are added through LDS in a
// fixed tree order (wave w + NWK/2 into w, halving) and wave 0 runs the
// fused epilogue of the tiled GEMM on the 32 * MI rows.  The K order is
// therefore not the tiled GEMM's; a context uses one kernel for all its
// calls (chosen from max_tokens), so a row's bits never depend on the call.
template <int MI, int NB, int NWK, int P, int OPD, int EPI>
__global__ void __launch_bounds__(64 * NWK) gemm_skinny(GemmArgs g) {
    constexpr bool QW = OPD == OPD_Q8 || OPD == OPD_Q4;
    constexpr bool Q4 = OPD == OPD_Q4;
    constexpr bool BF16 = OPD == OPD_BF16;
    constexpr int NACC = MI * NB * 16;                    // accumulator floats per lane
    __shared__ float red[NWK / 2][NACC][64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int tn = blockIdx.x, split = blockIdx.y;
    const int64_t nk_all = g.K / 32;
    const int64_t sb0 = split * nk_all / g.splits, nks = (split + 1) * nk_all / g.splits - sb0;
    const int kb0 = (int)(sb0 + wave * nks / NWK), kb1 = (int)(sb0 + (wave + 1) * nks / NWK);
    const int frow = lane & 31, fk = lane >> 5;
    f32x16 acc[MI][NB];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    // per-lane element offsets of slab 0 (A rows 32 i + frow of the first
    // 256-row group; weight rows n = tn * 32 NB + 32 j + frow), chunk 2 ks + fk
    int64_t aoff[MI][2], boff[NB][2], soff[NB];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) aoff[i][ks] = tiled32_index(32 * i + frow, (2 * ks + fk) * 8, g.K);
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        const int64_t n = (int64_t)tn * 32 * NB + 32 * j + frow;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int64_t k = (2 * ks + fk) * 8;
            boff[j][ks] = Q4 ? q4_code_chunk(n, k, g.K) : OPD == OPD_Q8 ? q8_code_chunk(n, k, g.K)
                                                                       : tiled32_index(n, k, g.K);
        }
        soff[j] = q8_scale_index(n, 0, g.K);
    }
    constexpr int64_t A_SLAB = (int64_t)kWeightTileRows * 32;                     // elements
    constexpr int64_t B_SLAB = (int64_t)kWeightTileRows * (QW ? (Q4 ? 16 : 32) : 32);  // bytes (q) / elements
    struct Buf {
        u32x4 a[MI][2];
        u32x4 b[NB][2];
        u32x2 qc[NB][2];
        uint16_t qs[NB];
    };
    Buf buf[P];
    auto load = [&](Buf& f, int kt) {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) f.a[i][ks] = *(const u32x4*)(g.A + aoff[i][ks] + kt * A_SLAB);
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            if constexpr (QW) {
                const uint8_t* q = reinterpret_cast<const uint8_t*>(g.Bq) + kt * B_SLAB;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    if constexpr (Q4) f.qc[j][ks] = u32x2{*(const uint32_t*)(q + boff[j][ks]), 0u};
                    else f.qc[j][ks] = *(const u32x2*)(q + boff[j][ks]);
                }
                f.qs[j] = g.Bs[soff[j] + (int64_t)kt * kWeightTileRows];
            } else {
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) f.b[j][ks] = *(const u32x4*)(g.B + boff[j][ks] + kt * B_SLAB);
            }
        }
    };
    auto compute = [&](Buf& f) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const u32x4 b = QW ? q_fragment<Q4>(f.qc[j][ks], f.qs[j]) : f.b[j][ks];
#pragma unroll
                for (int i = 0; i < MI; ++i) acc[i][j] = mfma32<BF16>(f.a[i][ks], b, acc[i][j]);
            }
        }
    };
#pragma unroll
    for (int p = 0; p < P; ++p)
        if (kb0 + p < kb1) load(buf[p], kb0 + p);
    for (int kt = kb0; kt < kb1; kt += P) {
#pragma unroll
        for (int p = 0; p < P; ++p) {
            if (kt + p < kb1) {                           // uniform over the wave
                compute(buf[p]);
                if (kt + p + P < kb1) load(buf[p], kt + p + P);
            }
        }
    }
    // tree sum of the waves' partials: (w + h) into w for h = NWK/2, NWK/4, .., 1
#pragma unroll
    for (int h = NWK / 2; h >= 1; h /= 2) {
        if (wave >= h && wave < 2 * h) {
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NB; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) red[wave - h][(i * NB + j) * 16 + r][lane] = acc[i][j][r];
        }
        __syncthreads();
        if (wave < h) {
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NB; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[i][j][r] += red[wave][(i * NB + j) * 16 + r][lane];
        }
        __syncthreads();
    }
    if (wave == 0) epilogue<32 * MI, 32 * NB, 1, 1, EPI, MI, NB, 0>(g, acc, 0, tn, split, nullptr);
}

// P: slabs in flight per wave (register buffers)
template <int MI, int NB, int NWK, int P, int OPD, int EPI>
hipError_t launch_skinny(const GemmArgs& a, hipStream_t s) {
    if (a.N % (32 * NB)) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_skinny<MI, NB, NWK, P, OPD, EPI>), dim3(a.N / (32 * NB), a.splits), dim3(64 * NWK), 0, s,
                       a);
    return hipGetLastError();
}

template <int OPD>
hipError_t launch_skinny_epi(EpiKind epi, const GemmArgs& a, hipStream_t s) {
    // wave counts and depths measured best on r2 / r3 q8_0 16-token calls
    if (epi == EPI_PARTIAL) return launch_skinny<1, 1, 8, 3, OPD, EPI_PARTIAL>(a, s);
    if (a.splits != 1) return hipErrorInvalidValue;
    if (epi == EPI_QKV) return launch_skinny<1, 1, 8, 3, OPD, EPI_QKV>(a, s);
    if (epi == EPI_SWIGLU) return launch_skinny<1, 2, 4, 6, OPD, EPI_SWIGLU>(a, s);
    return hipErrorNotSupported;
}

template <int BM, int BN, int WGM, int WGN, int OPD, int EPI>
hipError_t launch_t32(const GemmArgs& a, hipStream_t s) {
    if (a.N % BN) return hipErrorInvalidValue;
    if (a.splits < 1 || a.splits > a.K / 32 || (a.splits > 1 && EPI != EPI_PARTIAL && EPI != EPI_INPUT))
        return hipErrorInvalidValue;
    if (EPI == EPI_INPUT && (!a.epi.a_gain || !a.epi.ss || a.lda % 4 || ((uintptr_t)a.A % 16) ||
                             ((uintptr_t)a.epi.a_gain % 16) || a.epi.ss_stride < a.M))
        return hipErrorInvalidValue;
    if ((OPD == OPD_Q8 || OPD == OPD_Q4) ? (!a.Bq || !a.Bs) : !a.B) return hipErrorInvalidValue;
    const int total = ((a.M + BM - 1) / BM) * (a.N / BN) * a.splits;
    const int grid = (total + 7) / 8 * 8;
    hipLaunchKernelGGL((gemm_t32<BM, BN, WGM, WGN, OPD, EPI>), dim3(grid), dim3(64 * WGM * WGN), 0, s, a);
    return hipGetLastError();
}

}  // namespace

// The instantiated (operand, tile, epilogue) combinations.

hipError_t launch_gemm_heads(GemmOperand opd, const GemmArgs& a, int n_cu, int min_big, hipStream_t s) {
    if (a.M <= 0) return hipSuccess;
    if (a.K % 32 != 0 || a.K <= 0 || a.N % 256 || a.splits != 1) return hipErrorInvalidValue;
    if ((opd == OPD_Q8 || opd == OPD_Q4) ? (!a.Bq || !a.Bs) : !a.B) return hipErrorInvalidValue;
    if (a.epi.kv_n > 0 && min_big * 256 > a.N) return hipErrorInvalidValue;
    if (opd != OPD_BF16 && opd != OPD_F16 && opd != OPD_Q8 && opd != OPD_Q4) return hipErrorNotSupported;
    // Few rows: one M-tile of 64 or 128 rows, so that every weight strip is
    // read once by a workgroup whose MFMA work matches the real rows (with
    // 256-row tiles a short call would run a 256-row product on padding).
    if (a.M <= 64) {
        if (opd == OPD_BF16) return launch_t32<64, 256, 1, 4, OPD_BF16, EPI_HEADS>(a, s);
        if (opd == OPD_F16) return launch_t32<64, 256, 1, 4, OPD_F16, EPI_HEADS>(a, s);
        if (opd == OPD_Q4) return launch_t32<64, 256, 1, 4, OPD_Q4, EPI_HEADS>(a, s);
        return launch_t32<64, 256, 1, 4, OPD_Q8, EPI_HEADS>(a, s);
    }
    if (a.M <= 128) {
        if (opd == OPD_BF16) return launch_t32<128, 256, 2, 4, OPD_BF16, EPI_HEADS>(a, s);
        if (opd == OPD_F16) return launch_t32<128, 256, 2, 4, OPD_F16, EPI_HEADS>(a, s);
        if (opd == OPD_Q4) return launch_t32<128, 256, 2, 4, OPD_Q4, EPI_HEADS>(a, s);
        return launch_t32<128, 256, 2, 4, OPD_Q8, EPI_HEADS>(a, s);
    }
    const int mt = (a.M + 255) / 256, nt = a.N / 256, total = mt * nt;
    // whole rounds of 256x256 tiles; the rest of the columns in 128-row tiles
    // (128 x kTailBN) when that shortens the last round
    int n_big = nt;
    if (n_cu > 0 && total > n_cu && total % n_cu != 0) n_big = (total / n_cu) * n_cu / mt;
    if (n_big < min_big) n_big = min_big < nt ? min_big : nt;
    const int grid_big = (mt * n_big + 7) / 8 * 8;
    const int sbn = opd == OPD_Q8 ? kTailBN<OPD_Q8> : opd == OPD_Q4 ? kTailBN<OPD_Q4> : kTailBN<OPD_BF16>;
    static_assert(kTailBN<OPD_F16> == kTailBN<OPD_BF16>, "16-bit tail tiles");
    const int n_small = ((a.M + 127) / 128) * ((a.N - 256 * n_big) / sbn);
    const int grid = grid_big + (n_small + 7) / 8 * 8;
    if (opd == OPD_BF16)
        hipLaunchKernelGGL(gemm_t32_heads<OPD_BF16>, dim3(grid), dim3(512), 0, s, a, n_big, grid_big);
    else if (opd == OPD_F16)
        hipLaunchKernelGGL(gemm_t32_heads<OPD_F16>, dim3(grid), dim3(512), 0, s, a, n_big, grid_big);
    else if (opd == OPD_Q8)
        hipLaunchKernelGGL(gemm_t32_heads<OPD_Q8>, dim3(grid), dim3(512), 0, s, a, n_big, grid_big);
    else if (opd == OPD_Q4)
        hipLaunchKernelGGL(gemm_t32_heads<OPD_Q4>, dim3(grid), dim3(512), 0, s, a, n_big, grid_big);
    else
        return hipErrorNotSupported;
    return hipGetLastError();
}

hipError_t launch_gemm_skinny(GemmOperand opd, EpiKind epi, const GemmArgs& a, hipStream_t s) {
    if (a.M <= 0) return hipSuccess;
    if (a.M > 32 || a.K % 32 != 0 || a.K <= 0 || a.splits < 1 || a.splits > a.K / 32) return hipErrorInvalidValue;
    if ((opd == OPD_Q8 || opd == OPD_Q4) ? (!a.Bq || !a.Bs) : !a.B) return hipErrorInvalidValue;
    if (opd == OPD_F16) return launch_skinny_epi<OPD_F16>(epi, a, s);
    if (opd == OPD_Q8) return launch_skinny_epi<OPD_Q8>(epi, a, s);
    if (opd == OPD_Q4) return launch_skinny_epi<OPD_Q4>(epi, a, s);
    return hipErrorNotSupported;
}

#define KVA_T32_CASE(OPD_, TILE_, EPI_, BM_, BN_, WGM_, WGN_) \
    if (opd == OPD_ && tile == TILE_ && epi == EPI_) return launch_t32<BM_, BN_, WGM_, WGN_, OPD_, EPI_>(a, s);

hipError_t launch_gemm_t32(GemmOperand opd, GemmTile tile, EpiKind epi, const GemmArgs& a, hipStream_t s) {
    if (a.M <= 0) return hipSuccess;
    if (a.K % 32 != 0 || a.K <= 0) return hipErrorInvalidValue;
    KVA_T32_CASE(OPD_F16, TILE_256x256, EPI_PARTIAL, 256, 256, 2, 4)
    KVA_T32_CASE(OPD_F16, TILE_256x256, EPI_QKV, 256, 256, 2, 4)
    KVA_T32_CASE(OPD_F16, TILE_256x256, EPI_SWIGLU, 256, 256, 2, 4)
    KVA_T32_CASE(OPD_F16, TILE_256x128, EPI_PARTIAL, 256, 128, 4, 2)
    KVA_T32_CASE(OPD_F16, TILE_256x128, EPI_INPUT, 256, 128, 4, 2)
    KVA_T32_CASE(OPD_F16, TILE_128x256, EPI_INPUT, 128, 256, 2, 4)
    KVA_T32_CASE(OPD_F16, TILE_256x128, EPI_QKV, 256, 128, 4, 2)
    KVA_T32_CASE(OPD_F16, TILE_256x128, EPI_SWIGLU, 256, 128, 4, 2)
    KVA_T32_CASE(OPD_F16, TILE_128x128, EPI_PARTIAL, 128, 128, 2, 2)
    KVA_T32_CASE(OPD_F16, TILE_128x128, EPI_INPUT, 128, 128, 2, 2)
    KVA_T32_CASE(OPD_F16, TILE_128x128, EPI_QKV, 128, 128, 2, 2)
    KVA_T32_CASE(OPD_F16, TILE_128x128, EPI_SWIGLU, 128, 128, 2, 2)
    KVA_T32_CASE(OPD_Q8, TILE_256x256, EPI_PARTIAL, 256, 256, 2, 4)
    KVA_T32_CASE(OPD_Q8, TILE_256x256, EPI_QKV, 256, 256, 2, 4)
    KVA_T32_CASE(OPD_Q8, TILE_256x256, EPI_SWIGLU, 256, 256, 2, 4)
    KVA_T32_CASE(OPD_Q8, TILE_128x128, EPI_PARTIAL, 128, 128, 1, 4)
    KVA_T32_CASE(OPD_Q8, TILE_128x128, EPI_INPUT, 128, 128, 1, 4)
    KVA_T32_CASE(OPD_Q8, TILE_128x128, EPI_QKV, 128, 128, 1, 4)
    KVA_T32_CASE(OPD_Q8, TILE_128x128, EPI_SWIGLU, 128, 128, 2, 2)
    KVA_T32_CASE(OPD_Q4, TILE_256x256, EPI_PARTIAL, 256, 256, 2, 4)
    KVA_T32_CASE(OPD_Q4, TILE_256x256, EPI_QKV, 256, 256, 2, 4)
    KVA_T32_CASE(OPD_Q4, TILE_256x256, EPI_SWIGLU, 256, 256, 2, 4)
    KVA_T32_CASE(OPD_Q4, TILE_128x128, EPI_PARTIAL, 128, 128, 1, 4)
    KVA_T32_CASE(OPD_Q4, TILE_128x128, EPI_INPUT, 128, 128, 1, 4)
    KVA_T32_CASE(OPD_Q4, TILE_128x128, EPI_QKV, 128, 128, 1, 4)
    KVA_T32_CASE(OPD_Q4, TILE_128x128, EPI_SWIGLU, 128, 128, 2, 2)
    KVA_T32_CASE(OPD_F16, TILE_64xN, EPI_PARTIAL, 64, 64, 1, 2)
    KVA_T32_CASE(OPD_F16, TILE_64xN, EPI_INPUT, 64, 64, 1, 2)
    KVA_T32_CASE(OPD_F16, TILE_64xN, EPI_QKV, 64, 64, 1, 2)
    KVA_T32_CASE(OPD_F16, TILE_64xN, EPI_SWIGLU, 64, 128, 1, 2)
    KVA_T32_CASE(OPD_Q8, TILE_64xN, EPI_PARTIAL, 64, 64, 1, 2)
    KVA_T32_CASE(OPD_Q8, TILE_64xN, EPI_INPUT, 64, 64, 1, 2)
    KVA_T32_CASE(OPD_Q8, TILE_64xN, EPI_QKV, 64, 64, 1, 2)
    KVA_T32_CASE(OPD_Q8, TILE_64xN, EPI_SWIGLU, 64, 128, 1, 2)
    KVA_T32_CASE(OPD_Q4, TILE_64xN, EPI_PARTIAL, 64, 64, 1, 2)
    KVA_T32_CASE(OPD_Q4, TILE_64xN, EPI_INPUT, 64, 64, 1, 2)
    KVA_T32_CASE(OPD_Q4, TILE_64xN, EPI_QKV, 64, 64, 1, 2)
    KVA_T32_CASE(OPD_Q4, TILE_64xN, EPI_SWIGLU, 64, 128, 1, 2)
    return hipErrorNotSupported;
}
#undef KVA_T32_CASE

}  // namespace kva
