// Row-wise kernels: RMSNorm (fused with the 16-bit cast that feeds the next
// MFMA GEMM), the attention-layer KV-cache write (k_norm + partial RoPE +
// paged bf16 store) and the q8_0 dequantisation test hook.
#include "kva_internal.h"
#include "kva_kv.h"

namespace kva {
namespace {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

__device__ __forceinline__ uint16_t to_bits(float v, bool bf16) {
    return bf16 ? __builtin_bit_cast(uint16_t, static_cast<__bf16>(v))
                : __builtin_bit_cast(uint16_t, static_cast<_Float16>(v));
}

// RMSNorm ("Qwen3.8-27B-KVA" model card, "What the hell?": the projector's
// input norm, the two pre-norms of each block and the final norm):
// y = x / sqrt(mean(x^2) + eps) * g.  One workgroup per row; fixed
// reduction order, so a row's result never depends on other rows.
// The output goes out in the tiled32_index layout of the next GEMM's A
// operand (4 consecutive columns stay within one 8-value chunk).
template <bool BF16>
__global__ void __launch_bounds__(256) rmsnorm_cast(const float* __restrict__ x, int64_t ldx,
                                                    const float* __restrict__ gain, int32_t cols,
                                                    float eps, uint16_t* __restrict__ out) {
    __shared__ float part[4];
    const int row = blockIdx.x, tid = threadIdx.x;
    const float* xr = x + (int64_t)row * ldx;
    float ss = 0.0f;
    for (int c = tid * 4; c < cols; c += 1024) {
        const float4 v = *(const float4*)(xr + c);
        ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
    ss = wave_sum(ss);
    if ((tid & 63) == 0) part[tid >> 6] = ss;
    __syncthreads();
    const float tot = (part[0] + part[1]) + (part[2] + part[3]);
    const float r = 1.0f / sqrtf(tot / (float)cols + eps);
    for (int c = tid * 4; c < cols; c += 1024) {
        const float4 v = *(const float4*)(xr + c);
        const float4 gg = *(const float4*)(gain + c);
        ushort4 o;
        o.x = to_bits(v.x * r * gg.x, BF16);
        o.y = to_bits(v.y * r * gg.y, BF16);
        o.z = to_bits(v.z * r * gg.z, BF16);
        o.w = to_bits(v.w * r * gg.w, BF16);
        *(ushort4*)(out + tiled32_index(row, c, cols)) = o;
    }
}

// Plain cast of fp32 rows to the 16-bit tiled32_index layout of a GEMM's A
// operand (no norm), one workgroup per row: the single-map projector's input.
template <bool BF16>
__global__ void __launch_bounds__(256) cast_tiled(const float* __restrict__ x, int64_t ldx, int32_t cols,
                                                  uint16_t* __restrict__ out) {
    const int row = blockIdx.x;
    const float* xr = x + (int64_t)row * ldx;
    for (int c = threadIdx.x * 4; c < cols; c += 1024) {
        const float4 v = *(const float4*)(xr + c);
        ushort4 o;
        o.x = to_bits(v.x, BF16);
        o.y = to_bits(v.y, BF16);
        o.z = to_bits(v.z, BF16);
        o.w = to_bits(v.w, BF16);
        *(ushort4*)(out + tiled32_index(row, c, cols)) = o;
    }
}

// 1/RMS of an input row from the per-split sums of squares an EPI_INPUT
// GEMM wrote (added in split order).
__device__ __forceinline__ float input_rinv(const float* ss, int64_t ss_stride, int splits, int row, int cols,
                                            float eps) {
    float tot = 0.0f;
    for (int sp = 0; sp < splits; ++sp) tot += ss[sp * ss_stride + row];
    return 1.0f / sqrtf(tot / (float)cols + eps);
}

// Split-K fold + RMSNorm: the residual update that follows a split GEMM,
// fused with the norm that reads the updated residual.  The partials are
// added in a fixed order, so the result is deterministic and independent of
// how many rows the call has.  The normalised output goes out in the
// tiled32_index layout (4 consecutive columns stay within one 8-value chunk).
template <bool BF16>
__global__ void __launch_bounds__(256) fold_rmsnorm(float* __restrict__ h, int64_t ldh, int add,
                                                    const float* __restrict__ partials, int32_t splits,
                                                    int64_t pstride, int64_t ldp,
                                                    const float* __restrict__ gain, int32_t cols, float eps,
                                                    uint16_t* __restrict__ out, const float* __restrict__ in_ss,
                                                    int64_t ss_stride, int32_t ss_cols) {
    __shared__ float part[4];
    const int row = blockIdx.x, tid = threadIdx.x;
    float* hr = h + (int64_t)row * ldh;
    const float* pr = partials + (int64_t)row * ldp;
    const float rin = in_ss ? input_rinv(in_ss, ss_stride, splits, row, ss_cols, eps) : 1.0f;
    float ss = 0.0f;
    for (int c = tid * 4; c < cols; c += 1024) {
        float4 v = add ? *(const float4*)(hr + c) : make_float4(0.f, 0.f, 0.f, 0.f);
        for (int sp = 0; sp < splits; ++sp) {
            const float4 p = *(const float4*)(pr + sp * pstride + c);
            v.x += p.x; v.y += p.y; v.z += p.z; v.w += p.w;
        }
        if (in_ss) { v.x *= rin; v.y *= rin; v.z *= rin; v.w *= rin; }
        *(float4*)(hr + c) = v;
        ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
    ss = wave_sum(ss);
    if ((tid & 63) == 0) part[tid >> 6] = ss;
    __syncthreads();
    const float tot = (part[0] + part[1]) + (part[2] + part[3]);
    const float r = 1.0f / sqrtf(tot / (float)cols + eps);
    for (int c = tid * 4; c < cols; c += 1024) {
        const float4 v = *(const float4*)(hr + c);     // written above by this thread
        const float4 gg = *(const float4*)(gain + c);
        ushort4 o;
        o.x = to_bits(v.x * r * gg.x, BF16);
        o.y = to_bits(v.y * r * gg.y, BF16);
        o.z = to_bits(v.z * r * gg.z, BF16);
        o.w = to_bits(v.w * r * gg.w, BF16);
        *(ushort4*)(out + tiled32_index(row, c, cols)) = o;
    }
}

// The same with the row held in registers: V float4 per thread, thread t
// owning columns 4 (t + i * blockDim.x) .. +3 for i < V (consecutive threads
// read consecutive 16 bytes), and every load of the row (residual and
// partials) issued before the first one is used.  Rows of up to 4096
// columns in at most 512 threads (at 1024 tokens the whole grid is then
// resident at once).
constexpr int kMaxFoldSplits = 8;
template <bool BF16, int V>
__global__ void __launch_bounds__(1024) fold_rmsnorm_row(float* __restrict__ h, int64_t ldh, int add,
                                                         const float* __restrict__ partials, int32_t splits,
                                                         int64_t pstride, int64_t ldp,
                                                         const float* __restrict__ gain, int32_t cols, float eps,
                                                         uint16_t* __restrict__ out, const float* __restrict__ in_ss,
                                                         int64_t ss_stride, int32_t ss_cols) {
    __shared__ float part[16];
    const int row = blockIdx.x, tid = threadIdx.x, nt = blockDim.x;
    float* hr = h + (int64_t)row * ldh;
    const float* pr = partials + (int64_t)row * ldp;
    const float rin = in_ss ? input_rinv(in_ss, ss_stride, splits, row, ss_cols, eps) : 1.0f;
    float4 v[V], p[kMaxFoldSplits][V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
        const int c = (tid + i * nt) * 4;
        const bool live = c < cols;
        v[i] = (live && add) ? *(const float4*)(hr + c) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int sp = 0; sp < kMaxFoldSplits; ++sp)
            if (live && sp < splits) p[sp][i] = *(const float4*)(pr + sp * pstride + c);
    }
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < V; ++i) {
        const int c = (tid + i * nt) * 4;
        if (c < cols) {
#pragma unroll
            for (int sp = 0; sp < kMaxFoldSplits; ++sp)
                if (sp < splits) {
                    v[i].x += p[sp][i].x; v[i].y += p[sp][i].y; v[i].z += p[sp][i].z; v[i].w += p[sp][i].w;
                }
            if (in_ss) { v[i].x *= rin; v[i].y *= rin; v[i].z *= rin; v[i].w *= rin; }
            *(float4*)(hr + c) = v[i];
        }
        ss += v[i].x * v[i].x + v[i].y * v[i].y + v[i].z * v[i].z + v[i].w * v[i].w;
    }
    ss = wave_sum(ss);
    if ((tid & 63) == 0) part[tid >> 6] = ss;
    __syncthreads();
    float tot = 0.0f;
    for (int w = 0; w < (nt >> 6); ++w) tot += part[w];
    const float r = 1.0f / sqrtf(tot / (float)cols + eps);
#pragma unroll
    for (int i = 0; i < V; ++i) {
        const int c = (tid + i * nt) * 4;
        if (c < cols) {
            const float4 gg = *(const float4*)(gain + c);
            ushort4 o;
            o.x = to_bits(v[i].x * r * gg.x, BF16);
            o.y = to_bits(v[i].y * r * gg.y, BF16);
            o.z = to_bits(v[i].z * r * gg.z, BF16);
            o.w = to_bits(v[i].w * r * gg.w, BF16);
            *(ushort4*)(out + tiled32_index(row, c, cols)) = o;
        }
    }
}

// rmsnorm_cast with the row held in registers (same thread-to-column map as
// fold_rmsnorm_row): x is read once.
template <bool BF16, int V>
__global__ void __launch_bounds__(1024) rmsnorm_cast_row(const float* __restrict__ x, int64_t ldx,
                                                         const float* __restrict__ gain, int32_t cols,
                                                         float eps, uint16_t* __restrict__ out) {
    __shared__ float part[16];
    const int row = blockIdx.x, tid = threadIdx.x, nt = blockDim.x;
    const float* xr = x + (int64_t)row * ldx;
    float4 v[V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
        const int c = (tid + i * nt) * 4;
        v[i] = c < cols ? *(const float4*)(xr + c) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < V; ++i) ss += v[i].x * v[i].x + v[i].y * v[i].y + v[i].z * v[i].z + v[i].w * v[i].w;
    ss = wave_sum(ss);
    if ((tid & 63) == 0) part[tid >> 6] = ss;
    __syncthreads();
    float tot = 0.0f;
    for (int w = 0; w < (nt >> 6); ++w) tot += part[w];
    const float r = 1.0f / sqrtf(tot / (float)cols + eps);
#pragma unroll
    for (int i = 0; i < V; ++i) {
        const int c = (tid + i * nt) * 4;
        if (c < cols) {
            const float4 gg = *(const float4*)(gain + c);
            ushort4 o;
            o.x = to_bits(v[i].x * r * gg.x, BF16);
            o.y = to_bits(v[i].y * r * gg.y, BF16);
            o.z = to_bits(v[i].z * r * gg.z, BF16);
            o.w = to_bits(v[i].w * r * gg.w, BF16);
            *(ushort4*)(out + tiled32_index(row, c, cols)) = o;
        }
    }
}

// Threads of a register-resident row kernel with V float4 per thread.
inline unsigned row_threads(int32_t cols, int V) { return (unsigned)((cols / 4 / V + 63) / 64 * 64); }

// Inverse of the tiled32_index layout, one row per workgroup (test hook).
__global__ void __launch_bounds__(256) untile32_kernel(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst,
                                                       int32_t cols) {
    const int row = blockIdx.x;
    for (int c = threadIdx.x * 4; c < cols; c += 1024)
        *(ushort4*)(dst + (int64_t)row * cols + c) = *(const ushort4*)(src + tiled32_index(row, c, cols));
}

// KV-cache write for one full-attention layer (the routines and their
// sources are in kva_kv.h): bf16 rows, or Hadamard-rotated q8_0 rows.  One
// wave per token and HPW of its KV heads: lane l holds dims 4l..4l+3 of each
// head's k and v; the token's page and rotary angles are formed once per
// wave.  The q8_0 rows take two heads a wave (their per-row arithmetic is
// long; measured 11% faster than one with the scale rule of kva_kv.h), the
// bf16 rows one (memory-bound; 7% faster than two).
template <int HPW, bool Q8>
__global__ void __launch_bounds__(256) kv_write_kernel(KvWriteArgs a) {
    constexpr int WPT = kKvHeads / HPW;                // waves per token
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform: scalar page lookup
    const int t = blockIdx.x * (4 / WPT) + w / WPT;
    const int h0 = (w % WPT) * HPW;
    if (t >= a.n_tokens) return;
    const int64_t p = a.pos0 + t;
    const int pg = kv_page(a.pool, p);
    if (pg < 0) return;
    const float* kr = a.kv + (int64_t)t * a.ld_kv + lane * 4;
    float4 k[HPW], v[HPW];
#pragma unroll
    for (int h = 0; h < HPW; ++h) {
        k[h] = *(const float4*)(kr + (h0 + h) * kKvHeadDim);
        v[h] = *(const float4*)(kr + (kKvHeads + h0 + h) * kKvHeadDim);
    }
    const KvLane L = kv_lane_setup(lane, a.pool.k_gain, a.rope);
    const KvAngles A = kv_rope_angles(lane, p, L, a.rope.n_rot);
    const int64_t row0 = kv_row_index(a.pool, pg, p, h0);
#pragma unroll
    for (int h = 0; h < HPW; ++h)
        kv_store_row_as<Q8>(a.pool, true, row0 + h, lane,
                            kv_k_norm_rope(k[h], lane, A, L, a.rope.n_rot, a.rope.eps));
#pragma unroll
    for (int h = 0; h < HPW; ++h) kv_store_row_as<Q8>(a.pool, false, row0 + h, lane, v[h]);
}

// The q8_0 scale rule of kva_kv.h against correctly rounded division over
// all 2^32 binary32 patterns x (test hook): counts[0] += patterns where
// q8_scale_d(x) != x / 127 (x = -0 excluded: a block maximum is never -0),
// counts[1] += patterns with q8_scale_fast_ok(x) where q8_scale_inv_fast(x)
// != 1 / x, counts[2] += patterns where q8_scale_inv(x) (the guarded form,
// as its wave takes it) != (x != 0 ? 1 / x : 0).  NaN equals any NaN.
__device__ __forceinline__ bool same_f32(float a, float b) {
    if (a != a || b != b) return a != a && b != b;
    return __builtin_bit_cast(uint32_t, a) == __builtin_bit_cast(uint32_t, b);
}

__global__ void __launch_bounds__(256) check_q8_scale_kernel(unsigned long long* __restrict__ counts) {
    unsigned long long bad[3] = {0, 0, 0};
    for (uint32_t hi = 0; hi < 256; ++hi) {
        const uint32_t u = (hi << 24) | (blockIdx.x << 8) | threadIdx.x;
        const float x = __builtin_bit_cast(float, u);
        const bool b0 = u != 0x80000000u && !same_f32(q8_scale_d(x), x / 127.0f);
        const float inv = 1.0f / x;
        const bool b1 = q8_scale_fast_ok(x) && !same_f32(q8_scale_inv_fast(x), inv);
        const bool b2 = !same_f32(q8_scale_inv(x), x != 0.0f ? inv : 0.0f);
        bad[0] += (unsigned long long)__popcll(__builtin_amdgcn_ballot_w64(b0));
        bad[1] += (unsigned long long)__popcll(__builtin_amdgcn_ballot_w64(b1));
        bad[2] += (unsigned long long)__popcll(__builtin_amdgcn_ballot_w64(b2));
    }
    if ((threadIdx.x & 63) == 0)
        for (int i = 0; i < 3; ++i)
            if (bad[i]) atomicAdd(&counts[i], bad[i]);
}

__global__ void dequant_q8_0_kernel(const uint8_t* __restrict__ blocks, int64_t n_blocks,
                                    float* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // one value per thread
    if (i >= n_blocks * 32) return;
    const int64_t b = i >> 5;
    const uint8_t* blk = blocks + b * 34;
    const uint16_t d = (uint16_t)blk[0] | ((uint16_t)blk[1] << 8);
    out[i] = q8_0_value(d, (int)(int8_t)blk[2 + (i & 31)]);
}

// The fp16 weights of q8_0 blocks as the GEMM forms them (q8_0_f16x8), one
// thread per 8 values (test hook).
__global__ void dequant_q8_0_f16_kernel(const uint8_t* __restrict__ blocks, int64_t n_blocks,
                                        uint16_t* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // group of 8 values
    if (i >= n_blocks * 4) return;
    const uint8_t* blk = blocks + (i >> 2) * 34;
    const int8_t* c = reinterpret_cast<const int8_t*>(blk + 2 + (i & 3) * 8);
    const uint16_t d = (uint16_t)blk[0] | ((uint16_t)blk[1] << 8);
    int8_t q[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) q[e] = c[e];
    uint32_t c0, c1;
    q8_chunk_pack(q, &c0, &c1);
    uint32_t o[4];
    q8_0_f16x8(c0, c1, d, o);   // shared with the q8_0 GEMM
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        out[i * 8 + 2 * h] = (uint16_t)(o[h] & 0xFFFF);
        out[i * 8 + 2 * h + 1] = (uint16_t)(o[h] >> 16);
    }
}

// The fp16 weights of q4_0 blocks as the GEMM forms them (q4_0_f16x8), one
// thread per 8 values: the 8 codes of K-values 8c..8c+7 are gathered from
// the block's ggml order into the GEMM's chunk order first (test hook).
__global__ void dequant_q4_0_f16_kernel(const uint8_t* __restrict__ blocks, int64_t n_blocks,
                                        uint16_t* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // group of 8 values
    if (i >= n_blocks * 4) return;
    const uint8_t* blk = blocks + (i >> 2) * 18;
    const int c = (int)(i & 3);
    const uint16_t d = (uint16_t)blk[0] | ((uint16_t)blk[1] << 8);
    uint8_t nn[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int k = 8 * c + e;                                 // input of the block
        nn[e] = k < 16 ? (blk[2 + k] & 0xF) : (blk[2 + k - 16] >> 4);
    }
    uint32_t o[4];
    q4_0_f16x8(q4_chunk_pack(nn), d, o);    // shared with the q4_0 GEMM
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        out[i * 8 + 2 * h] = (uint16_t)(o[h] & 0xFFFF);
        out[i * 8 + 2 * h + 1] = (uint16_t)(o[h] >> 16);
    }
}

// Pure MFMA loop: each wave runs n_iter rounds of 8 independent bf16
// 32x32x16 MFMAs on register operands (no memory traffic), then folds its
// accumulators into sink so nothing is dead.  Measures the MFMA rate the
// device sustains at its current clock.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
__global__ void __launch_bounds__(256) mfma_loop_kernel(int32_t n_iter, float* __restrict__ sink) {
    const int lane = threadIdx.x & 63;
    bf16x8_t a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)(1.0f + 0.001f * (float)((lane + e) & 7));
        b[e] = (__bf16)(0.5f - 0.001f * (float)((lane * 3 + e) & 7));
    }
    f32x16_t acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
    for (int it = 0; it < n_iter; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
    }
    float t = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) t += acc[j][r];
    sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = t;
}

}  // namespace

hipError_t launch_mfma_loop(int32_t n_iter, int32_t n_workgroups, float* sink, hipStream_t s) {
    if (n_iter <= 0 || n_workgroups <= 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(mfma_loop_kernel, dim3(n_workgroups), dim3(256), 0, s, n_iter, sink);
    return hipGetLastError();
}

hipError_t launch_rmsnorm_cast(const float* x, int64_t ldx, const float* g, int32_t rows,
                               int32_t cols, float eps, uint16_t* out, bool bf16, hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    if (cols % 32) return hipErrorInvalidValue;
    if (cols <= 2048) {
        const dim3 t(row_threads(cols, 2));
        if (bf16) hipLaunchKernelGGL((rmsnorm_cast_row<true, 2>), dim3(rows), t, 0, s, x, ldx, g, cols, eps, out);
        else hipLaunchKernelGGL((rmsnorm_cast_row<false, 2>), dim3(rows), t, 0, s, x, ldx, g, cols, eps, out);
    } else if (cols <= 8192) {
        const dim3 t(row_threads(cols, 4));
        if (bf16) hipLaunchKernelGGL((rmsnorm_cast_row<true, 4>), dim3(rows), t, 0, s, x, ldx, g, cols, eps, out);
        else hipLaunchKernelGGL((rmsnorm_cast_row<false, 4>), dim3(rows), t, 0, s, x, ldx, g, cols, eps, out);
    } else if (bf16) {
        hipLaunchKernelGGL(rmsnorm_cast<true>, dim3(rows), dim3(256), 0, s, x, ldx, g, cols, eps, out);
    } else {
        hipLaunchKernelGGL(rmsnorm_cast<false>, dim3(rows), dim3(256), 0, s, x, ldx, g, cols, eps, out);
    }
    return hipGetLastError();
}

hipError_t launch_cast_tiled(const float* x, int64_t ldx, int32_t rows, int32_t cols, uint16_t* out, bool bf16,
                             hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    if (cols % 32) return hipErrorInvalidValue;
    if (bf16)
        hipLaunchKernelGGL(cast_tiled<true>, dim3(rows), dim3(256), 0, s, x, ldx, cols, out);
    else
        hipLaunchKernelGGL(cast_tiled<false>, dim3(rows), dim3(256), 0, s, x, ldx, cols, out);
    return hipGetLastError();
}

hipError_t launch_fold_rmsnorm(float* h, int64_t ldh, bool add, const float* partials, int32_t splits,
                               int64_t pstride, int64_t ldp, const float* g, int32_t rows, int32_t cols,
                               float eps, uint16_t* out, bool bf16, hipStream_t s, const float* ss,
                               int64_t ss_stride, int32_t ss_cols) {
    if (rows <= 0) return hipSuccess;
    if (cols % 32 || splits < 1) return hipErrorInvalidValue;
    if (ss && (add || ss_cols <= 0 || ss_stride < rows)) return hipErrorInvalidValue;
    if (cols <= 4096 && splits <= kMaxFoldSplits) {
        const bool two = cols > 1024;
        const dim3 t(row_threads(cols, two ? 2 : 1));
        if (bf16 && two)
            hipLaunchKernelGGL((fold_rmsnorm_row<true, 2>), dim3(rows), t, 0, s, h, ldh, (int)add, partials,
                               splits, pstride, ldp, g, cols, eps, out, ss, ss_stride, ss_cols);
        else if (two)
            hipLaunchKernelGGL((fold_rmsnorm_row<false, 2>), dim3(rows), t, 0, s, h, ldh, (int)add, partials,
                               splits, pstride, ldp, g, cols, eps, out, ss, ss_stride, ss_cols);
        else if (bf16)
            hipLaunchKernelGGL((fold_rmsnorm_row<true, 1>), dim3(rows), t, 0, s, h, ldh, (int)add, partials,
                               splits, pstride, ldp, g, cols, eps, out, ss, ss_stride, ss_cols);
        else
            hipLaunchKernelGGL((fold_rmsnorm_row<false, 1>), dim3(rows), t, 0, s, h, ldh, (int)add, partials,
                               splits, pstride, ldp, g, cols, eps, out, ss, ss_stride, ss_cols);
    } else if (bf16)
        hipLaunchKernelGGL(fold_rmsnorm<true>, dim3(rows), dim3(256), 0, s, h, ldh, (int)add, partials, splits,
                           pstride, ldp, g, cols, eps, out, ss, ss_stride, ss_cols);
    else
        hipLaunchKernelGGL(fold_rmsnorm<false>, dim3(rows), dim3(256), 0, s, h, ldh, (int)add, partials, splits,
                           pstride, ldp, g, cols, eps, out, ss, ss_stride, ss_cols);
    return hipGetLastError();
}

hipError_t launch_untile32(const uint16_t* src, uint16_t* dst, int32_t rows, int32_t cols, hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    if (cols % 32) return hipErrorInvalidValue;
    hipLaunchKernelGGL(untile32_kernel, dim3(rows), dim3(256), 0, s, src, dst, cols);
    return hipGetLastError();
}

hipError_t launch_kv_write(const KvWriteArgs& a, hipStream_t s) {
    if (a.n_tokens <= 0) return hipSuccess;
    if (a.rope.n_rot % 8 || a.rope.n_rot > 64 || a.rope.n_rot <= 0) return hipErrorInvalidValue;
    if (a.pool.q8)
        hipLaunchKernelGGL((kv_write_kernel<2, true>), dim3((a.n_tokens + 1) / 2), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((kv_write_kernel<1, false>), dim3(a.n_tokens), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_check_q8_scale(unsigned long long* counts, hipStream_t s) {
    hipLaunchKernelGGL(check_q8_scale_kernel, dim3(65536), dim3(256), 0, s, counts);
    return hipGetLastError();
}

hipError_t launch_dequant_q4_0_f16(const void* blocks, int64_t n_blocks, uint16_t* out, hipStream_t s) {
    if (n_blocks <= 0) return hipSuccess;
    const int64_t n = n_blocks * 4;
    hipLaunchKernelGGL(dequant_q4_0_f16_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       (const uint8_t*)blocks, n_blocks, out);
    return hipGetLastError();
}

hipError_t launch_dequant_q8_0_f16(const void* blocks, int64_t n_blocks, uint16_t* out, hipStream_t s) {
    if (n_blocks <= 0) return hipSuccess;
    const int64_t n = n_blocks * 4;
    hipLaunchKernelGGL(dequant_q8_0_f16_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       (const uint8_t*)blocks, n_blocks, out);
    return hipGetLastError();
}

hipError_t launch_dequant_q8_0(const void* blocks, int64_t n_blocks, float* out, hipStream_t s) {
    if (n_blocks <= 0) return hipSuccess;
    const int64_t n = n_blocks * 32;
    hipLaunchKernelGGL(dequant_q8_0_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       (const uint8_t*)blocks, n_blocks, out);
    return hipGetLastError();
}

}  // namespace kva
