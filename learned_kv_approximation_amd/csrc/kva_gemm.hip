// MFMA GEMM for the projector's Linear layers on gfx950.
//
// Every Linear of the projector ("Qwen3.8-27B-KVA" model card, "What the
// hell?": the input Linear, the blocks' Q/K/V/O and SwiGLU matrices, and the
// per-layer heads) is C = A * W^T with A the activations [tokens][in] and W
// the weight [out][in], both contiguous along `in`.  That is exactly the
// operand layout of the 32x32x16 MFMA: each lane feeds 8 consecutive
// K-values of one row of A and 8 consecutive K-values of one row of W.
//
// Two kernels share the fused epilogues (fp32 split-K partial, fp16
// Q|K plus transposed V, SwiGLU, bias + per-head scatter):
//  - gemm_t32: 16-bit weights (fp16 trunk, bf16 heads).  Both operands are
//    stored in the tiled32_index layout; four LDS stages of 32-wide slabs.
//  - gemm_q8: q8_0 weights.  The activation (fp16, row-major) is copied into
//    LDS directly; the weight half of each 64-wide slab goes through
//    registers, where d*q is formed exactly and rounded once to fp16.
// In both, workgroup ids are remapped so that the tiles of one weight strip
// (all M-tiles of an N-tile) run back to back on the same XCD and share its
// L2: the hardware deals workgroups to the 8 XCDs round-robin.  Accumulation
// is fp32, over K in plain sequential order.
#include "kva_internal.h"

#include <type_traits>

namespace kva {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int BK = 64;          // gemm_q8: K per slab (fp16 elements): 128-byte LDS rows

// gemm_q8's LDS swizzle: the 16-byte chunk c of row r sits at chunk c ^ swz(r),
// so the 16 rows one ds_read_b128 phase touches land on distinct banks.
__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

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
// block).  `smem` (at least 128 KB, free when called) is used by the head
// epilogue to turn whole-head tiles into full-row stores.
template <int BM, int BN, int WGM, int WGN, int EPI, int MI, int NI>
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

    if constexpr (EPI == EPI_PARTIAL) {
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
#pragma unroll
                for (int i = 0; i < MI; ++i)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int row = row_base + i * 32 + 8 * (r >> 2) + (r & 3);
                        if (row < g.M) e.out16[(int64_t)row * e.ld16 + col] = to_f16_bits(acc[i][j][r]);
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
                    if (row < g.M) {
                        const int64_t at = e.out16_t32 ? tiled32_index(row, f, e.ld16) : (int64_t)row * e.ld16 + f;
                        e.out16[at] = to_f16_bits(silu(acc[i][j][r]) * acc[i][j + 1][r]);
                    }
                }
        }
    } else if constexpr (EPI == EPI_HEADS) {
        static_assert(BN == kHeadTileN, "head packing assumes one head per column tile");
        const int th = e.tile_head[tn];
        // A whole-head tile whose destination rows are 16-byte aligned goes out
        // through LDS: each half of the tile (128 x 256 fp32 = the 128 KB of
        // LDS) is transposed there and written as full 1 KB rows with 16-byte
        // stores (a quarter of the store instructions of the direct path).
        if constexpr (BM == 256 && WGM == 2 && WGN == 4) {
            if (th >= 0 && (e.heads.ld[th] % 4) == 0 && ((uintptr_t)e.heads.ptr[th] % 16) == 0) {
                float* lds = reinterpret_cast<float*>(smem);       // [128][256], rows rotated by 32 every 4 rows
                float* dst0 = e.heads.ptr[th] + e.tile_col0[tn];
                const int64_t ld = e.heads.ld[th];
                const float* bias = e.bias ? e.bias + tn * BN : nullptr;
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    if (wm == half) {
#pragma unroll
                        for (int j = 0; j < NI; ++j)
#pragma unroll
                            for (int i = 0; i < MI; ++i)
#pragma unroll
                                for (int r = 0; r < 16; ++r) {
                                    const int lr = i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                                    const int lc = wn * WN + j * 32 + (lane & 31);
                                    lds[lr * BN + ((lc + 32 * ((lr >> 2) & 1)) & (BN - 1))] = acc[i][j][r];
                                }
                    }
                    __syncthreads();
                    // 128 rows x 64 chunks of 4 columns; one wave stores one full row
#pragma unroll
                    for (int q = 0; q < (128 * 64) / (64 * NW); ++q) {
                        const int id = q * 64 * NW + tid;
                        const int lr = id >> 6, c4 = (id & 63) * 4;
                        const int row = tm * BM + half * 128 + lr;
                        float4 v = *(const float4*)(lds + lr * BN + ((c4 + 32 * ((lr >> 2) & 1)) & (BN - 1)));
                        if (bias) {
                            const float4 b = *(const float4*)(bias + c4);
                            v.x += b.x; v.y += b.y; v.z += b.z; v.w += b.w;
                        }
                        if (row < g.M) *(float4*)(dst0 + (int64_t)row * ld + c4) = v;
                    }
                    __syncthreads();
                }
                return;
            }
        }
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            const int col = col_base + j * 32;
            float* dst;
            int64_t ld;
            if (th >= 0) {
                dst = e.heads.ptr[th] + e.tile_col0[tn] + (col - tn * BN);
                ld = e.heads.ld[th];
            } else {
                const int c = col - e.tail_start;
                const int h = e.tail_head[c];
                if (h < 0) continue;
                dst = e.heads.ptr[h] + e.tail_col[c];
                ld = e.heads.ld[h];
            }
            const float b = e.bias ? e.bias[col] : 0.0f;
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = row_base + i * 32 + 8 * (r >> 2) + (r & 3);
                    if (row < g.M) dst[(int64_t)row * ld] = acc[i][j][r] + b;
                }
        }
    }
}

// q8_0 weights.  A BM x BN tile is computed by WGM x WGN waves, each owning
// a (BM/WGM) x (BN/WGN) sub-tile.  The activation half of each 64-wide slab
// is copied from global memory straight into LDS (global_load_lds, 16 bytes
// per lane; one wave instruction fills 8 consecutive 128-byte rows): lane L
// lands at row L/8, physical chunk L%8, so it fetches the logical chunk
// (L%8) ^ swz(row) of that row.  Two LDS buffers, one barrier a slab.
template <int BM, int BN, int WGM, int WGN, int EPI>
__global__ void __launch_bounds__(64 * WGM * WGN) gemm_q8(GemmArgs g) {
    constexpr int NW = WGM * WGN;
    constexpr int WM = BM / WGM, WN = BN / WGN;
    constexpr int MI = WM / 32, NI = WN / 32;
    constexpr int AI = BM / (8 * NW);   // wave DMA instructions per slab
    static_assert(AI >= 1 && MI >= 1 && NI >= 1, "tile too small for the wave grid");
    static_assert(64 * NW == 2 * BN, "q8_0 weights: two threads per weight row");
    constexpr int STAGE = (BM + BN) * BK;
    __shared__ __attribute__((aligned(1024))) uint16_t smem[2 * STAGE];

    const int mt = (g.M + BM - 1) / BM;
    const int nt = g.N / BN;
    const int S = g.splits;
    const int total = mt * nt * S;
    const int per_xcd = gridDim.x / 8;
    const int v = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    if (v >= total) return;
    // M-tiles fastest, then splits, then N-tiles: the tiles sharing a weight
    // strip run back to back on one XCD
    const int tm = v % mt;
    const int split = (v / mt) % S;
    const int tn = v / (mt * S);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WGN, wn = wave % WGN;

    // rows >= M of A are padding rows of the activation scratch: loaded, never stored
    const uint16_t* Ab = g.A + (int64_t)tm * BM * g.lda;
    const int nk_all = g.K / BK;
    int offa[AI];
    {
        const int rr = lane >> 3, pc = lane & 7;
#pragma unroll
        for (int i = 0; i < AI; ++i) {
            const int row = (i * NW + wave) * 8 + rr;
            offa[i] = row * (int)g.lda + ((pc ^ swz(row)) << 3);
        }
    }
    auto issue = [&](int kt, int buf) {
        uint16_t* sa = smem + buf * STAGE;
#pragma unroll
        for (int i = 0; i < AI; ++i)
            __builtin_amdgcn_global_load_lds((gbl_ptr_t)(Ab + offa[i] + kt * BK),
                                             (lds_ptr_t)(sa + (i * NW + wave) * 8 * BK), 16, 0, 0);
    };

    // q8_0 weights: thread t owns one 32-code block of weight row t/2 per slab
    // (half t%2 of the slab's 64 K-values): codes and scale go through
    // registers, d*q is rounded once to fp16 and written to LDS.
    const int qrow = tid >> 1, qhalf = tid & 1;
    const int kblocks = g.K / 32;
    const int8_t* Bq = g.Bq + ((int64_t)tn * BN + qrow) * g.ldb + qhalf * 32;
    const uint16_t* Bs = g.Bs + ((int64_t)tn * BN + qrow) * kblocks + qhalf;
    u32x4 qr0, qr1;
    uint16_t qd = 0;
    auto qload = [&](int kt) {
        qr0 = *(const u32x4*)(Bq + kt * BK);
        qr1 = *(const u32x4*)(Bq + kt * BK + 16);
        qd = Bs[kt * 2];
    };
    auto qstore = [&](int buf) {
        uint16_t* sb = smem + buf * STAGE + BM * BK + qrow * BK;
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
            const u32x4& src = c4 < 2 ? qr0 : qr1;
            const uint32_t w0 = src[(c4 & 1) * 2], w1 = src[(c4 & 1) * 2 + 1];
            u32x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t w = e < 2 ? w0 : w1;
                const int q0 = (int)(int8_t)(w >> (16 * (e & 1)));
                const int q1 = (int)(int8_t)(w >> (16 * (e & 1) + 8));
                o[e] = (uint32_t)to_f16_bits(q8_0_value(qd, q0)) |
                       ((uint32_t)to_f16_bits(q8_0_value(qd, q1)) << 16);
            }
            const int c = qhalf * 4 + c4;
            *(u32x4*)(sb + ((c ^ swz(qrow)) << 3)) = o;
        }
    };

    f32x16 acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int kb = split * nk_all / S;                 // this split's slabs: [kb, kb + nk)
    const int nk = (split + 1) * nk_all / S - kb;
    const int frow = lane & 31, fk = lane >> 5;
    qload(kb);
    issue(kb, 0);
    qstore(0);
    // global_load_lds completes through vmcnt: wait for it explicitly, then
    // the barrier publishes the slab to every wave
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        // the other buffer was last read before the previous barrier: refill it
        if (kt + 1 < nk) {
            qload(kb + kt + 1);
            issue(kb + kt + 1, buf ^ 1);
        }
        const uint16_t* sa = smem + buf * STAGE;
        const uint16_t* sb = sa + BM * BK;
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int c = ks * 2 + fk;
            u32x4 af[MI], bfr[NI];
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                const int r = wm * WM + i * 32 + frow;
                af[i] = *(const u32x4*)(sa + r * BK + ((c ^ swz(r)) << 3));
            }
#pragma unroll
            for (int j = 0; j < NI; ++j) {
                const int r = wn * WN + j * 32 + frow;
                bfr[j] = *(const u32x4*)(sb + r * BK + ((c ^ swz(r)) << 3));
            }
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NI; ++j) acc[i][j] = mfma32<false>(af[i], bfr[j], acc[i][j]);
        }
        if (kt + 1 < nk) qstore(buf ^ 1);
        __builtin_amdgcn_s_waitcnt(0);   // the next slab has landed
        __syncthreads();                 // ... for all waves, and all are done with this one
    }

    epilogue<BM, BN, WGM, WGN, EPI, MI, NI>(g, acc, tm, tn, split, smem);
}

template <int BM, int BN, int WGM, int WGN, int EPI>
hipError_t launch_q8(const GemmArgs& a, hipStream_t s) {
    if (a.N % BN) return hipErrorInvalidValue;
    if (a.splits < 1 || a.splits > a.K / BK || (a.splits > 1 && EPI != EPI_PARTIAL)) return hipErrorInvalidValue;
    const int mt = (a.M + BM - 1) / BM;
    const int nt = a.N / BN;
    const int total = mt * nt * a.splits;
    const int grid = (total + 7) / 8 * 8;
    hipLaunchKernelGGL((gemm_q8<BM, BN, WGM, WGN, EPI>), dim3(grid), dim3(64 * WGM * WGN), 0, s, a);
    return hipGetLastError();
}


// Four-stage variant for operands that are both stored in the tiled32_index
// layout (the head GEMM, and the trunk GEMMs when their weights are 16-bit).
// BM x BN tiles (256x256 with 2 x 4 waves of 128 x 64, or 128x128 with 2 x 2
// waves of 64 x 64, whose 64 KB of LDS lets two workgroups share a CU).
//  - K is walked in 32-wide slabs; the A and the B half of a slab are each one
//    contiguous block in global memory, copied straight into LDS (1 KB per
//    wave instruction).  Four LDS stages: three slabs are in flight while one
//    is consumed, which covers the L2 latency at full MFMA rate.
//  - The MFMA fragments are double-buffered in registers: the LDS reads of
//    the next 16-wide K step are issued before the MFMAs of the current one,
//    including across the slab barrier, so LDS latency hides behind MFMAs.
//    The K order of the accumulation is the plain one (slab by slab, step by
//    step) for every tile shape, so the tile choice never changes the bits.
//  - Each slab ends with one barrier: it publishes the next slab (every wave
//    has waited for its own DMA of it) and frees the stage the DMA of the
//    slab after next refills.
//  - Split-K (EPI_PARTIAL only): the slabs are cut into `splits` consecutive
//    ranges, one per workgroup, each writing its own partial buffer.
template <int BM, int BN, int WGM, int WGN, int OPD, int EPI>
__global__ void __launch_bounds__(64 * WGM * WGN) gemm_t32(GemmArgs g) {
    constexpr bool BF16 = OPD == OPD_BF16;
    constexpr int NW = WGM * WGN, KB = 32, S = 4;
    constexpr int WM = BM / WGM, WN = BN / WGN, MI = WM / 32, NI = WN / 32;
    constexpr int AI = BM / (16 * NW), BI = BN / (16 * NW);   // DMA instructions per wave per slab
    constexpr int L = AI + BI;
    constexpr int STAGE = (BM + BN) * KB;
    static_assert(AI >= 1 && BI >= 1, "tile too small for the wave grid");
    static_assert(EPI != EPI_HEADS || S * STAGE * 2 >= 128 * 1024, "the head epilogue stages 128 KB through LDS");
    static_assert((S - 2) * L < 16, "vmcnt immediate");
    static_assert(kWeightTileRows % BM == 0 && kWeightTileRows % BN == 0, "tiles inside 256-row groups");
    __shared__ __attribute__((aligned(1024))) uint16_t smem[S * STAGE];

    const int mt = (g.M + BM - 1) / BM;
    const int nt = g.N / BN;
    const int SP = g.splits;
    const int total = mt * nt * SP;
    const int per_xcd = gridDim.x / 8;
    const int v = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    if (v >= total) return;
    // M-tiles fastest, then splits, then N-tiles: the tiles sharing a weight
    // strip run back to back on one XCD
    const int tm = v % mt;
    const int split = (v / mt) % SP;
    const int tn = v / (mt * SP);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WGN, wn = wave % WGN;
    const int nk_all = g.K / KB;
    const int kb = split * nk_all / SP;                // this split's slabs: [kb, kb + nk)
    const int nk = (split + 1) * nk_all / SP - kb;
    // slab kt of the rows [r0, r0 + BM) of a 256-row group t starts at
    // ((t * nk_all + kt) * 256 + r0) * KB
    const uint16_t* Ab = g.A + (((int64_t)(tm * BM / kWeightTileRows) * nk_all + kb) * kWeightTileRows +
                                (tm * BM) % kWeightTileRows) * KB;
    const uint16_t* Bb = g.B + (((int64_t)(tn * BN / kWeightTileRows) * nk_all + kb) * kWeightTileRows +
                                (tn * BN) % kWeightTileRows) * KB;
    auto issue = [&](int kt, int st) {
        uint16_t* sa = smem + st * STAGE;
        uint16_t* sb = sa + BM * KB;
        const int64_t o = (int64_t)kt * kWeightTileRows * KB;
#pragma unroll
        for (int i = 0; i < AI; ++i)
            __builtin_amdgcn_global_load_lds((gbl_ptr_t)(Ab + o + (i * NW + wave) * 16 * KB + lane * 8),
                                             (lds_ptr_t)(sa + (i * NW + wave) * 16 * KB), 16, 0, 0);
#pragma unroll
        for (int i = 0; i < BI; ++i)
            __builtin_amdgcn_global_load_lds((gbl_ptr_t)(Bb + o + (i * NW + wave) * 16 * KB + lane * 8),
                                             (lds_ptr_t)(sb + (i * NW + wave) * 16 * KB), 16, 0, 0);
    };
    f32x16 acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    const int frow = lane & 31, fk = lane >> 5;
    const int sw = ((frow >> 1) ^ (frow >> 3)) & 3;     // fragment rows differ by multiples of 32
    int aoff[MI], boff[NI];
#pragma unroll
    for (int i = 0; i < MI; ++i) aoff[i] = (wm * WM + i * 32 + frow) * KB;
#pragma unroll
    for (int j = 0; j < NI; ++j) boff[j] = BM * KB + (wn * WN + j * 32 + frow) * KB;
    u32x4 fa0[MI], fb0[NI], fa1[MI], fb1[NI];
    auto rd = [&](int st, int ks, u32x4* fa, u32x4* fb) {
        const uint16_t* base = smem + st * STAGE;
        const int c = ((ks * 2 + fk) ^ sw) << 3;
#pragma unroll
        for (int i = 0; i < MI; ++i) fa[i] = *(const u32x4*)(base + aoff[i] + c);
#pragma unroll
        for (int j = 0; j < NI; ++j) fb[j] = *(const u32x4*)(base + boff[j] + c);
    };
    auto mm = [&](const u32x4* fa, const u32x4* fb) {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NI; ++j) acc[i][j] = mfma32<BF16>(fa[i], fb[j], acc[i][j]);
    };
    // vmcnt(n) with lgkmcnt / expcnt left alone
    auto vm_wait = [](auto n) {
        constexpr int N = decltype(n)::value;
        __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
    };

#pragma unroll
    for (int p = 0; p < S - 1; ++p)
        if (p < nk) issue(p, p);
    if (nk >= S - 1) vm_wait(std::integral_constant<int, (S - 2) * L>{});
    else vm_wait(std::integral_constant<int, 0>{});
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
    rd(0, 0, fa0, fb0);
    for (int kt = 0; kt < nk; ++kt) {
        const bool more = kt + S - 1 < nk;
        // the stage of slab kt-1 was released by the previous barrier
        if (more) issue(kt + S - 1, (kt + S - 1) % S);
        rd(kt % S, 1, fa1, fb1);
        mm(fa0, fb0);
        if (more) vm_wait(std::integral_constant<int, (S - 2) * L>{});   // slab kt+1 has landed
        else vm_wait(std::integral_constant<int, 0>{});
        __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");           // slab kt fully read
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        __asm__ volatile("" ::: "memory");
        // after the last slab this reads a stale stage (in bounds); the values are not used
        rd((kt + 1) % S, 0, fa0, fb0);
        mm(fa1, fb1);
        __builtin_amdgcn_sched_barrier(0);
    }
    __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if constexpr (EPI == EPI_HEADS) __syncthreads();    // the head epilogue reuses LDS
    epilogue<BM, BN, WGM, WGN, EPI, MI, NI>(g, acc, tm, tn, split, smem);
}

template <int BM, int BN, int WGM, int WGN, int OPD, int EPI>
hipError_t launch_t32(const GemmArgs& a, hipStream_t s) {
    if (a.N % BN) return hipErrorInvalidValue;
    if (a.splits < 1 || a.splits > a.K / 32 || (a.splits > 1 && EPI != EPI_PARTIAL)) return hipErrorInvalidValue;
    const int total = ((a.M + BM - 1) / BM) * (a.N / BN) * a.splits;
    const int grid = (total + 7) / 8 * 8;
    hipLaunchKernelGGL((gemm_t32<BM, BN, WGM, WGN, OPD, EPI>), dim3(grid), dim3(64 * WGM * WGN), 0, s, a);
    return hipGetLastError();
}

}  // namespace

// The instantiated (tile, epilogue) combinations of each kernel.
#define KVA_Q8_CASE(TILE_, EPI_, BM_, BN_, WGM_, WGN_) \
    if (tile == TILE_ && epi == EPI_) return launch_q8<BM_, BN_, WGM_, WGN_, EPI_>(a, s);

hipError_t launch_gemm_q8(GemmTile tile, EpiKind epi, const GemmArgs& a, hipStream_t s) {
    if (a.M <= 0) return hipSuccess;
    if (a.K % BK != 0 || a.K <= 0) return hipErrorInvalidValue;
    if (!a.Bq || !a.Bs) return hipErrorInvalidValue;
    KVA_Q8_CASE(TILE_256x256, EPI_HEADS, 256, 256, 2, 4)
    KVA_Q8_CASE(TILE_256x256, EPI_PARTIAL, 256, 256, 2, 4)
    KVA_Q8_CASE(TILE_256x256, EPI_SWIGLU, 256, 256, 2, 4)
    KVA_Q8_CASE(TILE_256x256, EPI_QKV, 256, 256, 2, 4)
    KVA_Q8_CASE(TILE_128x128, EPI_PARTIAL, 128, 128, 2, 2)
    KVA_Q8_CASE(TILE_128x128, EPI_QKV, 128, 128, 2, 2)
    KVA_Q8_CASE(TILE_128x128, EPI_SWIGLU, 128, 128, 2, 2)
    return hipErrorNotSupported;
}
#undef KVA_Q8_CASE

#define KVA_T32_CASE(OPD_, TILE_, EPI_, BM_, BN_, WGM_, WGN_) \
    if (opd == OPD_ && tile == TILE_ && epi == EPI_) return launch_t32<BM_, BN_, WGM_, WGN_, OPD_, EPI_>(a, s);

hipError_t launch_gemm_t32(GemmOperand opd, GemmTile tile, EpiKind epi, const GemmArgs& a, hipStream_t s) {
    if (a.M <= 0) return hipSuccess;
    if (a.K % 32 != 0 || a.K <= 0) return hipErrorInvalidValue;
    KVA_T32_CASE(OPD_BF16, TILE_256x256, EPI_HEADS, 256, 256, 2, 4)
    KVA_T32_CASE(OPD_F16, TILE_256x256, EPI_PARTIAL, 256, 256, 2, 4)
    KVA_T32_CASE(OPD_F16, TILE_256x256, EPI_QKV, 256, 256, 2, 4)
    KVA_T32_CASE(OPD_F16, TILE_256x256, EPI_SWIGLU, 256, 256, 2, 4)
    KVA_T32_CASE(OPD_F16, TILE_128x128, EPI_PARTIAL, 128, 128, 2, 2)
    KVA_T32_CASE(OPD_F16, TILE_128x128, EPI_QKV, 128, 128, 2, 2)
    KVA_T32_CASE(OPD_F16, TILE_128x128, EPI_SWIGLU, 128, 128, 2, 2)
    return hipErrorNotSupported;
}
#undef KVA_T32_CASE

}  // namespace kva
