// Device routines of the attention-layer KV-cache write ("Qwen3.8-27B-KVA"
// card, "What the hell?": after projection the engine applies k_norm and RoPE
// and writes the KV cache; geometry from the "Qwen3.8-27B-MLA" card, "What
// this is": 4 KV heads of 256 dims with 64 rotary dims each).
//
// One full wave handles one token's 256 values of one KV head: lane l holds
// dims 4l..4l+3.  The stand-alone write kernel and the head GEMM's fused
// epilogue both call these routines with that mapping, so the two paths give
// the same bits for the same fp32 inputs.
#pragma once
#include "kva_internal.h"

namespace kva {

// Butterfly sum over the 64 lanes (fixed order; every lane gets the total).
__device__ __forceinline__ float kv_wave_sum(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

// k_norm then RoPE on one KV head of one token at absolute position p.
//   k_norm: k / sqrt(mean(k^2) + eps) * gain (per KV head, 256 dims);
//   RoPE: the pair (j, j + n_rot/2), j < n_rot/2, is turned by p * inv_freq[j].
// The rotary pair of lane l < n_rot/8 lives in lane l + n_rot/8.  The angle is
// formed and reduced modulo 2 pi in double (p reaches 65535 and more: an fp32
// product would be off by several 1e-3 rad), then fp32 sincos.
// Must be called by all 64 lanes of a wave together.
__device__ __forceinline__ float4 kv_k_norm_rope(float4 k, int lane, int64_t p, const float* __restrict__ gain,
                                                 const KvRope& rope) {
    const float ss = kv_wave_sum(k.x * k.x + k.y * k.y + k.z * k.z + k.w * k.w);
    const float r = 1.0f / sqrtf(ss / (float)kKvHeadDim + rope.eps);
    const float4 gg = *(const float4*)(gain + lane * 4);
    k.x *= r * gg.x; k.y *= r * gg.y; k.z *= r * gg.z; k.w *= r * gg.w;

    const int half_lanes = rope.n_rot / 8;     // lanes holding the first half of the rotary dims
    const float4 other = make_float4(__shfl_xor(k.x, half_lanes), __shfl_xor(k.y, half_lanes),
                                     __shfl_xor(k.z, half_lanes), __shfl_xor(k.w, half_lanes));
    if (lane < 2 * half_lanes) {
        const bool first = lane < half_lanes;
        const int j0 = (first ? lane : lane - half_lanes) * 4;
        float kk[4] = {k.x, k.y, k.z, k.w};
        const float oo[4] = {other.x, other.y, other.z, other.w};
        const double two_pi = 6.283185307179586476925286766559;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            double th = (double)p * rope.inv_freq[j0 + e];
            th -= two_pi * floor(th / two_pi);
            float sn, cs;
            sincosf((float)th, &sn, &cs);
            // first half: x' = x cos - y sin ; second half: y' = x sin + y cos
            kk[e] = first ? (kk[e] * cs - oo[e] * sn) : (oo[e] * sn + kk[e] * cs);
        }
        k = make_float4(kk[0], kk[1], kk[2], kk[3]);
    }
    return k;
}

// Element offset of dims 4*lane.. of KV head kvh for position p in a pool
// [n_pages][page_size][kKvHeads][kKvHeadDim], or -1 when the page-table entry
// is outside [0, n_pages) (nothing is written for that token).
__device__ __forceinline__ int64_t kv_slot_offset(const KvPool& c, int64_t p, int kvh, int lane) {
    const int pg = c.page_table[p / c.page_size];
    if (pg < 0 || pg >= c.n_pages) return -1;
    const int slot = (int)(p % c.page_size);
    return (((int64_t)pg * c.page_size + slot) * kKvHeads + kvh) * kKvHeadDim + lane * 4;
}

// Round to bf16 (nearest even) and store 4 values.
__device__ __forceinline__ void kv_store_bf16(uint16_t* dst, float4 v) {
    ushort4 o;
    o.x = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v.x));
    o.y = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v.y));
    o.z = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v.z));
    o.w = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v.w));
    *(ushort4*)dst = o;
}

}  // namespace kva
