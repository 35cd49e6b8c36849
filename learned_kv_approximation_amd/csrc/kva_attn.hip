// Block-causal multi-head attention for the projector's transformer blocks.
//
// Attention in the projector is causal and confined to the ubatch (attention
// block) a token arrived in ("Qwen3.8-27B-KVA" model card, "What the hell?"
// and the r2/r3 table: heads of 128, causal within 1024-token blocks).  For
// query i of head h in block [s, e):  o_i = sum_{s<=j<=i} softmax_j(q_i.k_j/sqrt(128)) v_j.
//
// One workgroup = 64 queries of one head, its key range split between
// groups of 2 waves (32 queries per wave); each group stages K and V of 64
// keys at a time in LDS (copied by global_load_lds into a ring of two
// stages, the next tile in flight while the current one is used) and the
// groups' partial softmax states are merged at the end.
// Per key tile a wave computes S^T = K Q^T with 32x32x16 MFMAs, so each lane
// holds the scores of ONE query (column lane%32) for 32 keys: the online
// softmax (running max m, running sum l, fp32) is per lane plus one exchange
// with lane^32.  O^T += V^T P^T then takes P straight from registers: V is
// produced transposed (vt[c][t]) by the QKV GEMM, and the key rows of the K
// tile are stored in LDS in the order that makes each lane's 8 P values 8
// consecutive keys, so one 16-byte LDS read fetches the matching V^T chunk.
// Keys after the query, and keys at or past n_tokens, get probability 0
// (their scores are replaced by -inf before the max; V past n_tokens is
// zeroed so 0 * V stays 0).
#include "kva_internal.h"

namespace kva {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) void* gbl_ptr_t;

constexpr int HD = 128;     // head dim
constexpr int QT = 64;      // queries per workgroup
// Keys per tile and key-range groups per workgroup.  Also measured at 1024
// tokens: 32-key tiles with 4 groups (8 waves, 2 per SIMD) 3% slower, with 2
// groups 8% slower.
constexpr int kKeyTile = 64;
constexpr int kKeySplit = 2;
constexpr float kLazyShift = 8.0f;   // log2 units a score may exceed the softmax reference point by

__device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// LDS row rho of the K tile holds key perm(rho) of the tile: bits 2 and 3 of
// the index are swapped (an involution).
__device__ __forceinline__ int perm(int rho) {
    return (rho & ~12) | ((rho & 4) << 1) | ((rho & 8) >> 1);
}

// Chunk swizzle of the V^T tile ([d][KT], KT / 8 chunks of 16 bytes per
// row): the 16 rows one half-wave reads at one chunk index land in 16
// different 16-byte bank groups.
template <int KT>
__device__ __forceinline__ int vswz(int d) {
    if constexpr (KT == 64) return (d & 7) ^ ((d >> 3) & 1);
    else return (d >> 2) & 3;
}

__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)b) << 16);
}

// One workgroup = 64 queries of one head, KS groups of 2 waves.  Group g
// takes the key tiles t = g, g + KS, g + 2 KS, ... of the query tile's range,
// so the longest chain of tiles a wave walks is ceil(tiles / KS).  Within a
// group, wave w % 2 owns queries 32 (w % 2) .. +31.  Each group stages its
// own K and V^T tiles in LDS (two stages, copied one tile ahead).  At
// the end the groups' running (max, sum, O) are merged through LDS:
//   m = max_g m_g,  l = sum_g l_g 2^(m_g - m),  O = sum_g O_g 2^(m_g - m) / l.
// O goes out in the tiled32_index layout of the next GEMM's A operand (each
// 8-byte store is 4 consecutive columns inside one 8-value chunk).
template <int KS, int KT>
__global__ void __launch_bounds__(128 * KS) attn_fwd(const uint16_t* __restrict__ qk, int64_t ld_qk,
                                                     int32_t k_off, const uint16_t* __restrict__ vt,
                                                     int64_t ld_vt, uint16_t* __restrict__ o,
                                                     int64_t ld_o, int32_t n, int32_t n_heads,
                                                     int32_t attn_block) {
    constexpr int TILE = KT * HD;                       // elements of one K (or V^T) tile
    constexpr int STAGE = 2 * TILE;                     // K | V^T
    constexpr int NST = KT / 32;                        // 32-key S^T blocks per tile
    constexpr int NM = KT / 16;                         // 16-key PV steps per tile
    constexpr int NI = KT * 16 / 128;                   // DMA instructions per wave per operand
    static_assert(KT == 32 || KT == 64, "key tile");
    static_assert((KS - 1) * 2 * 64 * 66 * 4 <= KS * 2 * STAGE * 2, "merge records fit the tile stages");
    __shared__ __attribute__((aligned(1024))) uint16_t smem[KS * 2 * STAGE];   // per group: two stages

    // Work items in descending order of key range over ALL heads and blocks:
    // the r-th round of n_heads * n_blocks items holds local q-tile tpb-1-r.
    const int tpb = attn_block / QT;                  // q-tiles per attention block
    const int nblk = (n + attn_block - 1) / attn_block;
    const int per_round = n_heads * nblk;
    const int L = blockIdx.x;
    const int lt = tpb - 1 - L / per_round;
    const int h = (L % per_round) % n_heads;
    const int qt = ((L % per_round) / n_heads) * tpb + lt;
    const int q0 = qt * QT;
    if (q0 >= n) return;                              // past the ragged last block
    const int bs = (q0 / attn_block) * attn_block;    // start of this block
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 1, gw = wave & 1;         // key-range group, wave within the group
    const int g = lane >> 5;
    const int myq = q0 + gw * 32 + (lane & 31);
    const int kv_end = min(q0 + QT, n);
    const int ntiles = (kv_end - bs + KT - 1) / KT;
    const int iters = (ntiles + KS - 1) / KS;          // same for every wave (barriers)
    uint16_t* sG = smem + grp * 2 * STAGE;

    // Q fragments (B operand of S^T = K Q^T): 8 consecutive dims per lane per 16-dim step
    u32x4 qf[HD / 16];
    {
        const uint16_t* qr = qk + (int64_t)min(myq, n - 1) * ld_qk + h * HD + g * 8;
#pragma unroll
        for (int ks = 0; ks < HD / 16; ++ks) qf[ks] = *(const u32x4*)(qr + ks * 16);
    }

    // DMA of the group's tile at key kv0 into stage st: K as [rho][128] and
    // V^T as [d][64], both chunk-swizzled, 1024 16-byte units each; LDS unit u
    // comes from lane u % 64 of instruction u / 128 of wave (u / 64) % 2.  K
    // rows past n_tokens repeat row n-1 (their scores are masked); V^T
    // columns past n_tokens are read from the allocated padding and zeroed
    // in registers after the LDS read.  Addresses: a block-relative base
    // (uniform) plus 32-bit element offsets (the host checks they fit).
    const uint16_t* kbase = qk + (int64_t)bs * ld_qk + k_off + h * HD;
    const uint16_t* vbase = vt + (int64_t)(h * HD) * ld_vt + bs;
    const int nrel = n - bs;                          // keys of this block present
    int koff[NI], voff[NI];                           // tile-independent parts
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int u = (2 * i + gw) * 64 + lane;
        const int rho = u >> 4, d = u / (KT / 8);
        koff[i] = perm(rho) * (int)ld_qk + (((u & 15) ^ (rho & 15)) << 3);
        voff[i] = d * (int)ld_vt + (((u % (KT / 8)) ^ vswz<KT>(d)) << 3);
    }
    auto issue = [&](int t, int st) {
        uint16_t* sK = sG + st * STAGE;
        uint16_t* sV = sK + TILE;
        const int k0 = t * KT;                        // first key of the tile, block-relative
        if (k0 + KT <= nrel) {
#pragma unroll
            for (int i = 0; i < NI; ++i)
                __builtin_amdgcn_global_load_lds((gbl_ptr_t)(kbase + k0 * (int)ld_qk + koff[i]),
                                                 (lds_ptr_t)(sK + (2 * i + gw) * 512), 16, 0, 0);
        } else {
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int u = (2 * i + gw) * 64 + lane;
                const int rho = u >> 4;
                const int kv = min(k0 + perm(rho), nrel - 1);
                __builtin_amdgcn_global_load_lds(
                    (gbl_ptr_t)(kbase + kv * (int)ld_qk + (((u & 15) ^ (rho & 15)) << 3)),
                    (lds_ptr_t)(sK + (2 * i + gw) * 512), 16, 0, 0);
            }
        }
#pragma unroll
        for (int i = 0; i < NI; ++i)
            __builtin_amdgcn_global_load_lds((gbl_ptr_t)(vbase + k0 + voff[i]),
                                             (lds_ptr_t)(sV + (2 * i + gw) * 512), 16, 0, 0);
    };

    float m_i = -INFINITY, l_i = 0.0f;
    f32x16 oacc[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.0f;

    // Two stages per group: tile t + KS is copied while tile t is used.  One
    // barrier per tile publishes tile t (every wave has waited for its own
    // DMA of it) and frees the stage the next copy overwrites.
    if (grp < ntiles) issue(grp, 0);
    for (int it = 0; it < iters; ++it) {
        const int t = grp + it * KS;                   // this group's tile, if t < ntiles
        const int st = it & 1;
        __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));   // vmcnt(0): own DMA of tile t landed
        __syncthreads();
        if (t + KS < ntiles) issue(t + KS, st ^ 1);
        if (t >= ntiles) continue;
        const int kv0 = bs + t * KT;
        const uint16_t* sK = sG + st * STAGE;
        const uint16_t* sV = sK + TILE;

        u32x4 kf[NST][HD / 16];
#pragma unroll
        for (int ks = 0; ks < HD / 16; ++ks)
#pragma unroll
            for (int st2 = 0; st2 < NST; ++st2) {
                const int rho = st2 * 32 + (lane & 31);
                const int c = ks * 2 + g;
                kf[st2][ks] = *(const u32x4*)(&sK[rho * HD + ((c ^ (rho & 15)) << 3)]);
            }

        // S^T[rho][q] for rho in [0, KT): KT / 32 MFMA tiles of 32 keys
        f32x16 s[NST];
#pragma unroll
        for (int st = 0; st < NST; ++st)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[st][r] = 0.0f;
#pragma unroll
        for (int ks = 0; ks < HD / 16; ++ks)
#pragma unroll
            for (int st2 = 0; st2 < NST; ++st2) s[st2] = mfma(kf[st2][ks], qf[ks], s[st2]);

        // V^T fragments (A operand of O^T += V^T P^T), read while the S MFMAs run
        u32x4 vf[4][NM];
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
            const int d = dt * 32 + (lane & 31);
            const int sw = vswz<KT>(d);
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                const int c = 2 * m + g;
                vf[dt][m] = *(const u32x4*)(&sV[d * KT + ((c ^ sw) << 3)]);
            }
        }
        if (kv0 + KT > n) {                            // zero V of keys past the end (0 * V must stay 0)
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                const int t0 = kv0 + 16 * m + 8 * g;   // keys of vf[.][m]: t0 .. t0 + 7
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t keep = (t0 + 2 * e >= n ? 0u : 0x0000FFFFu) | (t0 + 2 * e + 1 >= n ? 0u : 0xFFFF0000u);
#pragma unroll
                    for (int dt = 0; dt < 4; ++dt) vf[dt][m][e] &= keep;
                }
            }
        }

        // mask, running max.  Element (st, r) is LDS row
        // rho = 32 st + 8 (r/4) + 4 g + r%4, i.e. key kv0 + perm(rho).  Only
        // the diagonal tile and a tile reaching past n_tokens need the mask;
        // the test is uniform across the wave.
        float mx = m_i;
        const int wq0 = q0 + (wave & 1) * 32;          // lowest query of this wave
        if (kv0 + KT - 1 > wq0 || kv0 + KT > n) {
#pragma unroll
            for (int st = 0; st < NST; ++st)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int rho = st * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
                    const int kv = kv0 + perm(rho);
                    float v = s[st][r];                 // Q came scaled by log2(e) / sqrt(128)
                    if (kv > myq || kv >= n) v = -INFINITY;
                    s[st][r] = v;
                    mx = fmaxf(mx, v);
                }
        } else {
#pragma unroll
            for (int st = 0; st < NST; ++st)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[st][r]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        // A query's reference point m_i of l and O moves only when one of
        // its scores is more than kLazyShift above it (softmax is invariant
        // to the shift, so this changes only roundings): the rescale of O
        // then runs about once per wave instead of once per tile, and
        // P = 2^(s - m_i) <= 2^kLazyShift stays far inside fp16.  The
        // decision is per query; the wave runs the multiply when any of its
        // queries moves, with the factor 1 (exact) for the others, so a
        // query's result depends on its own scores alone and a block's
        // first tokens come out bit for bit the same whatever follows them.
        // The first unmasked tile sets m_i (it starts at -inf).  Exponents
        // below are then <= kLazyShift (and -inf for masked keys): the
        // hardware exp2 is exact enough, and flushing underflow to 0 is what
        // softmax wants.
        const bool move = mx > m_i + kLazyShift;
        if (__builtin_amdgcn_ballot_w64(move) != 0) {
            const float alpha = move ? __builtin_amdgcn_exp2f(m_i - mx) : 1.0f;
            m_i = move ? mx : m_i;
            l_i *= alpha;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
        }

        // A query that has seen only masked keys so far (a 32-key tile can lie
        // wholly after the first half of the q-tile) keeps m_i = -inf; its P
        // must be 0, not 2^(-inf + inf).
        const float mref = m_i == -INFINITY ? 0.0f : m_i;

        // P^T fragments: MFMA m covers keys [16m, 16m+16) of the tile; lane holds
        // keys 16m + 8g + 0..7 = registers 8(m%2)..8(m%2)+7 of s[m/2]
        u32x4 pf[NM];
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            float p[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                p[e] = __builtin_amdgcn_exp2f(s[m >> 1][8 * (m & 1) + e] - mref);
                l_i += p[e];
            }
            pf[m][0] = pack_f16(p[0], p[1]);
            pf[m][1] = pack_f16(p[2], p[3]);
            pf[m][2] = pack_f16(p[4], p[5]);
            pf[m][3] = pack_f16(p[6], p[7]);
        }

        // O^T[d][q] += V^T[d][kv] P^T[kv][q]
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int m = 0; m < NM; ++m) oacc[dt] = mfma(vf[dt][m], pf[m], oacc[dt]);
    }

    // ---- merge the KS groups (group 0 writes the output)
    l_i += __shfl_xor(l_i, 32);                       // both halves of the keys of this query
    if constexpr (KS > 1) {
        float* xo = reinterpret_cast<float*>(smem);    // [KS-1][2 waves][64 + 64 + 64*64] floats
        constexpr int REC = 64 * 66;
        __syncthreads();                               // all LDS tile reads are done
        if (grp > 0) {
            float* rec = xo + ((grp - 1) * 2 + (wave & 1)) * REC;
            rec[lane] = m_i;
            rec[64 + lane] = l_i;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) rec[128 + (dt * 16 + r) * 64 + lane] = oacc[dt][r];
        }
        __syncthreads();
        if (grp > 0) return;
        float mt = m_i;
#pragma unroll
        for (int gg = 1; gg < KS; ++gg) mt = fmaxf(mt, xo[((gg - 1) * 2 + (wave & 1)) * REC + lane]);
        const float a0 = __builtin_amdgcn_exp2f(m_i - mt);
        l_i *= a0;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[dt][r] *= a0;
#pragma unroll
        for (int gg = 1; gg < KS; ++gg) {
            const float* rec = xo + ((gg - 1) * 2 + (wave & 1)) * REC;
            const float ag = __builtin_amdgcn_exp2f(rec[lane] - mt);   // 0 for a group that saw no key
            l_i += rec[64 + lane] * ag;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[dt][r] += rec[128 + (dt * 16 + r) * 64 + lane] * ag;
        }
    }

    const float inv = 1.0f / l_i;
    if (myq < n) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                // rows d = 32 dt + 8 q + 4 g + 0..3 of O^T, all for this lane's query
                u32x2 pk;
                pk[0] = pack_f16(oacc[dt][4 * q + 0] * inv, oacc[dt][4 * q + 1] * inv);
                pk[1] = pack_f16(oacc[dt][4 * q + 2] * inv, oacc[dt][4 * q + 3] * inv);
                *(u32x2*)(o + tiled32_index(myq, h * HD + dt * 32 + 8 * q + 4 * g, ld_o)) = pk;
            }
    }
}

}  // namespace

hipError_t launch_attention(const uint16_t* qk, int64_t ld_qk, int32_t k_off, const uint16_t* vt,
                            int64_t ld_vt, uint16_t* o, int64_t ld_o, int32_t n, int32_t n_heads,
                            int32_t attn_block, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    if (attn_block % QT || ld_o % 32) return hipErrorInvalidValue;
    // The kernel's per-lane element offsets are 32-bit: up to
    // (HD - 1) ld_vt + attn_block + KT into V^T from the block's first
    // column, up to (attn_block + KT) ld_qk into Q|K from the block's first
    // row (max_tokens <= 2^24 keeps the first within range).
    if ((int64_t)(HD - 1) * ld_vt + attn_block + kKeyTile > INT32_MAX ||
        (int64_t)(attn_block + kKeyTile) * ld_qk > INT32_MAX)
        return hipErrorInvalidValue;
    const int nblk = (n + attn_block - 1) / attn_block;
    const dim3 grid(n_heads * nblk * (attn_block / QT));
    hipLaunchKernelGGL((attn_fwd<kKeySplit, kKeyTile>), grid, dim3(128 * kKeySplit), 0, s, qk, ld_qk, k_off, vt, ld_vt, o,
                       ld_o, n, n_heads, attn_block);
    return hipGetLastError();
}

}  // namespace kva
