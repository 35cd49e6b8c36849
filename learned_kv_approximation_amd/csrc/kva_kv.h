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

#include <type_traits>

namespace kva {

// The value of lane (lane ^ M), M a power of two below 64, by the cheapest
// route: DPP moves inside a row of 16 lanes (xor 1 and 2: quad permutes; xor
// 4: half-row mirror then quad reverse, i -> 7 - (i ^ 3) = i ^ 4; xor 8: row
// rotate by 8), a swizzle inside 32 lanes (xor 16), a permute across the
// halves (xor 32).  Same pairing as __shfl_xor, so the same results.
template <int M>
__device__ __forceinline__ int lane_xor_bits(int x) {
    if constexpr (M == 1) return __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true);       // quad_perm 1,0,3,2
    else if constexpr (M == 2) return __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true);  // quad_perm 2,3,0,1
    else if constexpr (M == 4) {
        const int h = __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, true);                  // row_half_mirror
        return __builtin_amdgcn_mov_dpp(h, 0x1B, 0xF, 0xF, true);                          // quad_perm 3,2,1,0
    } else if constexpr (M == 8) return __builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, true); // row_ror 8
    else if constexpr (M == 16) return __builtin_amdgcn_ds_swizzle(x, (16 << 10) | 0x1F);  // bitmask: xor 16
    else {
        static_assert(M == 32, "lane_xor: mask");
        return __shfl_xor(x, 32);
    }
}

template <int M>
__device__ __forceinline__ float lane_xor(float v) {
    return __builtin_bit_cast(float, lane_xor_bits<M>(__builtin_bit_cast(int, v)));
}

// Butterfly sum over the 64 lanes (fixed order; every lane gets the total).
__device__ __forceinline__ float kv_wave_sum(float v) {
#pragma clang fp contract(off)
    v += lane_xor<32>(v);
    v += lane_xor<16>(v);
    v += lane_xor<8>(v);
    v += lane_xor<4>(v);
    v += lane_xor<2>(v);
    v += lane_xor<1>(v);
    return v;
}

// Per-lane constants of the k path, loaded once and reused for every token:
// the lane's 4 k_norm gains and, for lane j < n_rot/2, the frequency of
// rotary pair j.
struct KvLane {
    float4 gain;
    double inv_freq;
};

__device__ __forceinline__ KvLane kv_lane_setup(int lane, const float* __restrict__ gain, const KvRope& rope) {
    KvLane L;
    L.gain = *(const float4*)(gain + lane * 4);
    L.inv_freq = lane < rope.n_rot / 2 ? rope.inv_freq[lane] : 0.0;
    return L;
}

// sin and cos of an angle th >= 0 given in double (th below 2^40 or so):
// the quadrant q = nearest integer of th / (pi/2) and the remainder
// r = th - q*pi/2 (|r| <= pi/4) are formed in double, then the Taylor
// polynomials of sin and cos at 0 (through r^9 and r^10; the first omitted
// terms are below 2e-9 on |r| <= pi/4) are evaluated in fp32 and permuted and
// negated by q mod 4.  Branch-free, a few dozen instructions; absolute error
// about 1e-7 (an fp32 sincosf would also carry a large-argument path that a
// compiler may evaluate on every call).
__device__ __forceinline__ void kv_sincos(double th, float* sn, float* cs) {
#pragma clang fp contract(off)
    const double half_pi = 1.5707963267948966192313216916398;
    const double q = rint(th * (1.0 / half_pi));
    const float r = (float)(th - q * half_pi);
    const float r2 = r * r;
    const float s = r + r * r2 * (-1.0f / 6 + r2 * (1.0f / 120 + r2 * (-1.0f / 5040 + r2 * (1.0f / 362880))));
    const float c = 1.0f + r2 * (-0.5f + r2 * (1.0f / 24 + r2 * (-1.0f / 720 + r2 * (1.0f / 40320 +
                                                                            r2 * (-1.0f / 3628800)))));
    const int qi = (int)((int64_t)q & 3);
    const float sv = (qi & 1) ? c : s;          // sin(r + q pi/2): s, c, -s, -c
    const float cv = (qi & 1) ? s : c;          // cos(r + q pi/2): c, -s, -c, s
    *sn = (qi & 2) ? -sv : sv;
    *cs = ((qi + 1) & 2) ? -cv : cv;
}

// Sine and cosine of the rotary angles of lane l's 4 dims at absolute
// position p: lane j < n_rot/2 turns the angle of pair j (kv_sincos, formed in
// double: p reaches 65535 and more, where an fp32 product would be off by
// several 1e-3 rad) and the lanes holding the pair's two values fetch it
// from there.  The same for every KV head of the token.  Must be called by
// all 64 lanes of a wave together.
struct KvAngles {
    float sn[4], cs[4];
};

__device__ __forceinline__ KvAngles kv_rope_angles(int lane, int64_t p, const KvLane& L, int n_rot) {
    float sj, cj;
    kv_sincos((double)(int32_t)p * L.inv_freq, &sj, &cj);     // positions are below 2^31 (checked on the host)
    const int half_lanes = n_rot / 8;          // lanes holding the first half of the rotary dims
    const int j0 = (lane < half_lanes ? lane : lane - half_lanes) * 4;
    KvAngles A;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        A.sn[e] = __shfl(sj, j0 + e);
        A.cs[e] = __shfl(cj, j0 + e);
    }
    return A;
}

// k_norm then RoPE on one KV head of one token, with the token's angles.
//   k_norm: k / sqrt(mean(k^2) + eps) * gain (per KV head, 256 dims);
//   RoPE: the pair (j, j + n_rot/2), j < n_rot/2, is turned by p * inv_freq[j].
// The rotary pair of lane l < n_rot/8 lives in lane l + n_rot/8.
// Must be called by all 64 lanes of a wave together.
__device__ __forceinline__ float4 kv_k_norm_rope(float4 k, int lane, const KvAngles& A, const KvLane& L,
                                                 int n_rot, float eps) {
    // No multiply-add contraction: whether the compiler fuses a product into
    // an add may depend on the code around an inlined copy, and every caller
    // must round exactly alike.
#pragma clang fp contract(off)
    const float ss = kv_wave_sum(k.x * k.x + k.y * k.y + k.z * k.z + k.w * k.w);
    const float r = __builtin_amdgcn_rsqf(ss / (float)kKvHeadDim + eps);   // hardware reciprocal square root (~1 ulp)
    k.x *= r * L.gain.x; k.y *= r * L.gain.y; k.z *= r * L.gain.z; k.w *= r * L.gain.w;

    const int half_lanes = n_rot / 8;
    float4 other;
    if (half_lanes == 8)        // 64 rotary dims: the partner is 8 lanes away inside a row of 16
        other = make_float4(lane_xor<8>(k.x), lane_xor<8>(k.y), lane_xor<8>(k.z), lane_xor<8>(k.w));
    else
        other = make_float4(__shfl_xor(k.x, half_lanes), __shfl_xor(k.y, half_lanes),
                            __shfl_xor(k.z, half_lanes), __shfl_xor(k.w, half_lanes));
    if (lane < 2 * half_lanes) {
        const bool first = lane < half_lanes;
        float kk[4] = {k.x, k.y, k.z, k.w};
        const float oo[4] = {other.x, other.y, other.z, other.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
            // first half: x' = x cos - y sin ; second half: y' = x sin + y cos
            kk[e] = first ? (kk[e] * A.cs[e] - oo[e] * A.sn[e]) : (oo[e] * A.sn[e] + kk[e] * A.cs[e]);
        k = make_float4(kk[0], kk[1], kk[2], kk[3]);
    }
    return k;
}

// The same at absolute position p (angles formed here).
__device__ __forceinline__ float4 kv_k_norm_rope(float4 k, int lane, int64_t p, const KvLane& L,
                                                 int n_rot, float eps) {
    return kv_k_norm_rope(k, lane, kv_rope_angles(lane, p, L, n_rot), L, n_rot, eps);
}

// Physical page of position p (positions are below 2^31, checked on the
// host), or -1 when the page-table entry is outside [0, n_pages): nothing is
// written for that token.
__device__ __forceinline__ int kv_page(const KvPool& c, int64_t p) {
    const int pg = c.page_table[(uint32_t)p / (uint32_t)c.page_size];
    return (pg < 0 || pg >= c.n_pages) ? -1 : pg;
}

// Row index (token slot and KV head) of position p on page pg in a pool
// [n_pages][page_size][kKvHeads][row].
__device__ __forceinline__ int64_t kv_row_index(const KvPool& c, int pg, int64_t p, int kvh) {
    const int slot = (int)((uint32_t)p % (uint32_t)c.page_size);
    return ((int64_t)pg * c.page_size + slot) * kKvHeads + kvh;
}

// Orthonormal Walsh-Hadamard transform of Sylvester order over the wave's
// 256 values (lane l holds dims 4l..4l+3): y = H x / 16 with
// H[i][j] = (-1)^popcount(i & j).  One butterfly stage per bit of the dim
// index, (a, b) -> (a + b, a - b) on the pair that differs in that bit:
// bits 0 and 1 inside the lane, bits 2..7 across lanes (lane bit 0..5).  The
// quantised KV cache stores K and V rotated this way ([KVA] "Other notes":
// the approximated K/V are rotated by the same Hadamard transform as the
// exactly computed ones).  Must be called by all 64 lanes of a wave together.
//
// A cross-lane stage is one fused multiply-add per value, b <- b + c * o with
// o the partner lane's value and c = -1 on the lane whose stage bit is set,
// 1 on the other: that lane then holds b - o, the exact negation of the
// butterfly's o - b (o * c is exact, so the sum is rounded once, and
// rounding to nearest is symmetric).  Its partner differs from it only in
// bits of later stages, so both carry the same sign and every later stage
// stays a plain sum or difference; the sign of the result is
// (-1)^popcount(lane), folded into the 1/16 scale.  The stages inside a row
// of 16 lanes take the partner's value by DPP as the multiply-add's first
// operand (one instruction per value; a DPP read needs two wait states after
// the write of its source, which the s_nop gives for the first read and the
// interleaving of the four values for the others).
__device__ __forceinline__ float4 kv_hadamard256(float4 x, int lane) {
#pragma clang fp contract(off)
    const float a0 = x.x + x.y, a1 = x.x - x.y, a2 = x.z + x.w, a3 = x.z - x.w;
    float b0 = a0 + a2, b1 = a1 + a3, b2 = a0 - a2, b3 = a1 - a3;
    const float c1 = (lane & 1) ? -1.0f : 1.0f, c2 = (lane & 2) ? -1.0f : 1.0f;
    const float c4 = (lane & 4) ? -1.0f : 1.0f, c8 = (lane & 8) ? -1.0f : 1.0f;
    float t0, t1, t2, t3;
    asm("s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %0, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %1, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %2, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %3, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %0, %9 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %1, %9 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %2, %9 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %3, %9 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
        // xor 4: half-row mirror, then the quad reversal as the DPP operand
        "v_mov_b32_dpp %4, %0 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
        "v_mov_b32_dpp %5, %1 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
        "v_mov_b32_dpp %6, %2 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
        "v_mov_b32_dpp %7, %3 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %10 quad_perm:[3,2,1,0] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %5, %10 quad_perm:[3,2,1,0] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %10 quad_perm:[3,2,1,0] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %7, %10 quad_perm:[3,2,1,0] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %0, %11 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %1, %11 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %2, %11 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %3, %11 row_ror:8 row_mask:0xf bank_mask:0xf"
        : "+v"(b0), "+v"(b1), "+v"(b2), "+v"(b3), "=&v"(t0), "=&v"(t1), "=&v"(t2), "=&v"(t3)
        : "v"(c1), "v"(c2), "v"(c4), "v"(c8));
    const float c16 = (lane & 16) ? -1.0f : 1.0f, c32 = (lane & 32) ? -1.0f : 1.0f;
    b0 = __builtin_fmaf(lane_xor<16>(b0), c16, b0);
    b1 = __builtin_fmaf(lane_xor<16>(b1), c16, b1);
    b2 = __builtin_fmaf(lane_xor<16>(b2), c16, b2);
    b3 = __builtin_fmaf(lane_xor<16>(b3), c16, b3);
    b0 = __builtin_fmaf(lane_xor<32>(b0), c32, b0);
    b1 = __builtin_fmaf(lane_xor<32>(b1), c32, b1);
    b2 = __builtin_fmaf(lane_xor<32>(b2), c32, b2);
    b3 = __builtin_fmaf(lane_xor<32>(b3), c32, b3);
    const float sc = (__builtin_popcount(lane) & 1) ? -0.0625f : 0.0625f;
    return make_float4(b0 * sc, b1 * sc, b2 * sc, b3 * sc);
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

// The q8_0 block rule's scale and its reciprocal from the block maximum
// amax >= 0: d = amax / 127 and id = 1 / d (0 when d = 0), both the correctly
// rounded binary32 results.  Without the division instruction sequence:
//  - d: q0 = amax * RN(1/127), then one correction with the exact residual
//    amax - 127 q0 (an fma), q0 + residual * RN(1/127) rounded once
//    (Markstein's correction step); an infinite q0 passes through;
//  - id, for 2^-126 <= d < 2^126 (d and 1/d normal): the hardware
//    reciprocal y0, then one Newton step y0 + y0 (1 - d y0) with fma
//    (Markstein's reciprocal iteration).
// Both agree with correctly rounded division on every binary32 input they
// are used for (d: every amax except -0; id: every d in that range);
// kva_debug_check_q8_scale runs that comparison over all 2^32 patterns on
// the device.  A wave in which some lane's d is outside the range (zero,
// subnormal, infinite, NaN, or 2^126 and above, which d = amax / 127 never
// reaches) takes the division instead, all lanes together.
__device__ __forceinline__ float q8_scale_d(float amax) {
#pragma clang fp contract(off)
    const float q0 = amax * (1.0f / 127.0f);
    const float d = __builtin_fmaf(__builtin_fmaf(-q0, 127.0f, amax), 1.0f / 127.0f, q0);
    return __builtin_isinf(q0) ? q0 : d;
}

__device__ __forceinline__ bool q8_scale_fast_ok(float d) { return d >= 0x1p-126f && d < 0x1p126f; }

__device__ __forceinline__ float q8_scale_inv_fast(float d) {
    const float y0 = __builtin_amdgcn_rcpf(d);
    return __builtin_fmaf(__builtin_fmaf(-d, y0, 1.0f), y0, y0);
}

// Must be called by all 64 lanes of a wave together.
__device__ __forceinline__ float q8_scale_inv(float d) {
    if (__builtin_amdgcn_ballot_w64(!q8_scale_fast_ok(d)) != 0) return d != 0.0f ? 1.0f / d : 0.0f;
    return q8_scale_inv_fast(d);
}

// q8_0 (ggml's block: fp16 scale d, 32 int8 codes, value d * q) of the
// wave's 256 values into one row of 8 blocks of 34 bytes.  Block b holds dims
// 32b..32b+31, i.e. lanes 8b..8b+7.  The quantisation is decided in fp32 by
// ggml's q8_0 block rule: d = amax / 127, its reciprocal 1/d (both correctly
// rounded divisions; 0 when d = 0), q = round-half-away(y * (1/d)), clamped
// to [-127, 127]; d is stored rounded to fp16 (nearest even).  Must be called
// by all 64 lanes of a wave together.
__device__ __forceinline__ void kv_store_q8_0(uint8_t* row, float4 y, int lane) {
#pragma clang fp contract(off)
    // block maximum of |y|: non-negative binary32 values order as their bit
    // patterns, so the exchanges compare integers
    const float am0 = fmaxf(fmaxf(fabsf(y.x), fabsf(y.y)), fmaxf(fabsf(y.z), fabsf(y.w)));
    uint32_t ab = __builtin_bit_cast(uint32_t, am0);
    ab = max(ab, (uint32_t)lane_xor_bits<1>((int)ab));
    ab = max(ab, (uint32_t)lane_xor_bits<2>((int)ab));
    ab = max(ab, (uint32_t)lane_xor_bits<4>((int)ab));
    const float d = q8_scale_d(__builtin_bit_cast(float, ab));
    const float id = q8_scale_inv(d);
    const float yy[4] = {y.x, y.y, y.z, y.w};
    // round half away from zero as trunc(t + copysign(h, t)), h the largest
    // binary32 below 1/2: for |t| < 2^23 the sum rounds up to the next integer
    // exactly when t's fraction is at least 1/2 (checked over every such
    // binary32 value); the float-to-int conversion truncates
    const float h = __builtin_bit_cast(float, 0x3EFFFFFFu);
    uint32_t packed = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float t = yy[e] * id;
        // clamped before the conversion (a NaN becomes -127, never an
        // out-of-range conversion); the same as clamping the integer
        const int q = (int)fminf(fmaxf(t + copysignf(h, t), -127.0f), 127.0f);
        packed |= (uint32_t)(uint8_t)(int8_t)q << (8 * e);
    }
    uint8_t* blk = row + (lane >> 3) * 34;
    uint16_t* codes = reinterpret_cast<uint16_t*>(blk + 2 + (lane & 7) * 4);   // 2-byte aligned
    codes[0] = (uint16_t)(packed & 0xFFFF);
    codes[1] = (uint16_t)(packed >> 16);
    if ((lane & 7) == 0)
        *reinterpret_cast<uint16_t*>(blk) = __builtin_bit_cast(uint16_t, static_cast<_Float16>(d));
}

// Stores one KV head's 256 values of one token (k after k_norm and RoPE, or
// v) at row `row` of the pool: bf16, or Hadamard-rotated q8_0.
// Q8: the pool's format known at compile time.
template <bool Q8>
__device__ __forceinline__ void kv_store_row_as(const KvPool& c, bool is_k, int64_t row, int lane, float4 x) {
    void* pool = is_k ? c.k_pool : c.v_pool;
    if constexpr (Q8)
        kv_store_q8_0(static_cast<uint8_t*>(pool) + row * kKvQ8RowBytes, kv_hadamard256(x, lane), lane);
    else
        kv_store_bf16(static_cast<uint16_t*>(pool) + row * kKvHeadDim + lane * 4, x);
}

__device__ __forceinline__ void kv_store_row(const KvPool& c, bool is_k, int64_t row, int lane, float4 x) {
    if (c.q8) kv_store_row_as<true>(c, is_k, row, lane, x);
    else kv_store_row_as<false>(c, is_k, row, lane, x);
}

}  // namespace kva
