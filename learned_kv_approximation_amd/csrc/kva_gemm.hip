// MFMA GEMM for the projector's Linear layers on gfx950.
//
// Every Linear of the projector ("Qwen3.8-27B-KVA" model card, "What the
// hell?": the input Linear, the blocks' Q/K/V/O and SwiGLU matrices, and the
// per-layer heads) is C = A * W^T with A the activations [tokens][in] and W
// the weight [out][in], both contiguous along `in`.  That is exactly the
// operand layout of the 32x32x16 MFMA: each lane feeds 8 consecutive
// K-values of one row of A and 8 consecutive K-values of one row of W.
//
// Structure (one workgroup = 4 waves in a 2x2 grid, one BM x BN tile):
//  - K is walked in slabs of 64.  Each thread fetches 16-byte chunks of the
//    next slab from global memory into registers while the waves run MFMAs
//    on the current slab from LDS (double-buffered LDS, one barrier a slab).
//  - LDS rows are 128 bytes; the 16-byte chunk c of row r is stored at chunk
//    c ^ swz(r), so the 16 rows one ds_read_b128 phase touches land on
//    distinct banks.
//  - Workgroup ids are remapped so that the tiles of one weight strip (all
//    M-tiles of an N-tile) run back to back on the same XCD and share its L2:
//    the hardware deals workgroups to the 8 XCDs round-robin.
//  - fp32 accumulation; the epilogue is fused (fp32 store / residual add,
//    fp16 Q|K plus transposed V, SwiGLU, bias + per-head scatter).
#include "kva_internal.h"

namespace kva {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int BK = 64;          // K per slab (16-bit elements): 128-byte LDS rows
constexpr int kThreads = 256;

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

// Output element (lane, r) of a 32x32 MFMA tile sits at
//   row = 8*(r/4) + 4*(lane/32) + r%4,  col = lane%32.
template <int BM, int BN, bool BF16, int EPI>
__global__ void __launch_bounds__(kThreads) gemm_nt(GemmArgs g) {
    constexpr int WM = BM / 2, WN = BN / 2;
    constexpr int MI = WM / 32, NI = WN / 32;
    constexpr int AP = BM / 32, BP = BN / 32;   // 16-byte chunks per thread per slab
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (BM + BN) * BK];

    const int mt = (g.M + BM - 1) / BM;
    const int nt = g.N / BN;
    const int total = mt * nt;
    const int per_xcd = gridDim.x / 8;
    const int v = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    if (v >= total) return;
    const int tm = v % mt, tn = v / mt;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int lrow = tid >> 3, lch = tid & 7;

    const uint16_t* pa = g.A + (int64_t)(tm * BM + lrow) * g.lda + lch * 8;
    const uint16_t* pb = g.B + (int64_t)(tn * BN + lrow) * g.ldb + lch * 8;
    const int64_t stepa = 32 * g.lda, stepb = 32 * g.ldb;

    u32x4 ra[AP], rb[BP];
    auto gload = [&](int kt) {
#pragma unroll
        for (int p = 0; p < AP; ++p) ra[p] = *(const u32x4*)(pa + p * stepa + kt * BK);
#pragma unroll
        for (int p = 0; p < BP; ++p) rb[p] = *(const u32x4*)(pb + p * stepb + kt * BK);
    };
    auto sstore = [&](int buf) {
        uint16_t* sa = smem + buf * BM * BK;
        uint16_t* sb = smem + 2 * BM * BK + buf * BN * BK;
#pragma unroll
        for (int p = 0; p < AP; ++p) {
            const int r = p * 32 + lrow;
            *(u32x4*)(sa + r * BK + ((lch ^ swz(r)) << 3)) = ra[p];
        }
#pragma unroll
        for (int p = 0; p < BP; ++p) {
            const int r = p * 32 + lrow;
            *(u32x4*)(sb + r * BK + ((lch ^ swz(r)) << 3)) = rb[p];
        }
    };

    f32x16 acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int nk = g.K / BK;
    gload(0);
    sstore(0);
    __syncthreads();
    const int frow = lane & 31, fk = lane >> 5;
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) gload(kt + 1);
        const uint16_t* sa = smem + buf * BM * BK;
        const uint16_t* sb = smem + 2 * BM * BK + buf * BN * BK;
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
                for (int j = 0; j < NI; ++j) acc[i][j] = mfma32<BF16>(af[i], bfr[j], acc[i][j]);
        }
        if (kt + 1 < nk) sstore(buf ^ 1);
        __syncthreads();
    }

    // ------------------------------------------------------------ epilogue
    const int row_base = tm * BM + wm * WM + 4 * (lane >> 5);
    const int col_base = tn * BN + wn * WN + (lane & 31);
    const EpiArgs& e = g.epi;

    if constexpr (EPI == EPI_STORE_F32 || EPI == EPI_ADD_F32) {
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            const int col = col_base + j * 32;
            if (col >= e.n_real) continue;
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = row_base + i * 32 + 8 * (r >> 2) + (r & 3);
                    if (row < g.M) {
                        float* p = e.out_f32 + (int64_t)row * e.ld_f32 + col;
                        if constexpr (EPI == EPI_ADD_F32) *p += acc[i][j][r];
                        else *p = acc[i][j][r];
                    }
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
                    if (row < g.M)
                        e.out16[(int64_t)row * e.ld16 + f] =
                            to_f16_bits(silu(acc[i][j][r]) * acc[i][j + 1][r]);
                }
        }
    } else if constexpr (EPI == EPI_HEADS) {
        static_assert(BN == kHeadTileN, "head packing assumes one head per column tile");
        const int th = e.tile_head[tn];
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

template <int BM, int BN, bool BF16, int EPI>
hipError_t launch_one(const GemmArgs& a, hipStream_t s) {
    const int mt = (a.M + BM - 1) / BM;
    const int nt = a.N / BN;
    const int total = mt * nt;
    const int grid = (total + 7) / 8 * 8;
    hipLaunchKernelGGL((gemm_nt<BM, BN, BF16, EPI>), dim3(grid), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(GemmOperand opd, GemmTile tile, EpiKind epi, const GemmArgs& a,
                       hipStream_t s) {
    if (a.M <= 0) return hipSuccess;
    if (a.K % BK != 0) return hipErrorInvalidValue;
    if (opd == OPD_BF16 && tile == TILE_256x256 && epi == EPI_HEADS) {
        if (a.N % 256) return hipErrorInvalidValue;
        return launch_one<256, 256, true, EPI_HEADS>(a, s);
    }
    if (opd == OPD_F16 && tile == TILE_128x128) {
        if (a.N % 128) return hipErrorInvalidValue;
        switch (epi) {
            case EPI_STORE_F32: return launch_one<128, 128, false, EPI_STORE_F32>(a, s);
            case EPI_ADD_F32: return launch_one<128, 128, false, EPI_ADD_F32>(a, s);
            case EPI_QKV: return launch_one<128, 128, false, EPI_QKV>(a, s);
            case EPI_SWIGLU: return launch_one<128, 128, false, EPI_SWIGLU>(a, s);
            default: break;
        }
    }
    return hipErrorNotSupported;
}

}  // namespace kva
