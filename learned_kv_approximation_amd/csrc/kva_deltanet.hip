// Gated-DeltaNet state update for the DeltaNet layers the projector feeds
// ("Qwen3.8-27B-KVA" card, "What the hell?": after projection the engine runs
// conv + silu, l2-norm and the DeltaNet scan over the approximated tokens).
// The formulas are the gated delta rule's (see include/kva.h):
//   causal depthwise conv (width 4) + SiLU on the raw q|k|v rows,
//   k <- k / sqrt(|k|^2 + 1e-6) per key head,
//   alpha = exp(-exp(A_log) * softplus(a + dt_bias)), beta = sigmoid(b),
//   S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T.
//
// One workgroup (8 waves) per (layer, key head) updates the value heads that
// read that key head (up to 3), walking the tokens in chunks of C = 32 with
// the 128 x 128 fp32 states in MFMA accumulators.  Within a chunk
// (chunk-start state S0, gamma_t = alpha_1 ... alpha_t from the chunk start)
// the recurrence unrolls to
//   S_C = gamma_C S0 + sum_t (gamma_C / gamma_t) w_t k_t^T,
//   (I + A) W = diag(beta) V - diag(beta gamma) K S0^T,
//   A[t][i] = beta_t (gamma_t / gamma_i) (k_t . k_i) for i < t, else 0.
// K K^T (shared by the heads), K S0^T and the state update W^T K are
// 32x32x16 fp16 MFMAs with fp32 accumulation (unit keys, the chunk-start
// state and W are rounded to fp16 as operands; the states stay fp32); the
// unit lower-triangular solve for W runs in fp32, one value column per thread.
#include "kva_internal.h"

namespace kva {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kC = 32;                 // tokens per chunk
constexpr int kD = kDnHeadDim;         // key and value head width
constexpr int kG = 3;                  // value heads per key head a workgroup can take
constexpr int kRowT = kC + 8;          // fp16 row of 32 values, padded (80 B)
constexpr int kRowH = kD + 8;          // fp16 row of 128 values, padded (272 B)
constexpr int kThreads = 512;
constexpr int kTilesPerWave = 2 * kG;  // 16 state tiles per head over 8 waves

// (K S0^T)^T and then W^T are kept [m][v][t] with 32 t per row (64 B) and
// no padding; the four 16-byte chunks of row v are rotated by (v >> 2) & 3
// so that a wave's 16-byte fragment reads (32 rows, two chunks per row) fall
// on distinct banks (the rotation of the GEMM operand layout).
__device__ __forceinline__ int wt_index(int v, int t) {
    return v * kC + ((((t >> 3) ^ ((v >> 2) & 3)) << 3) | (t & 7));
}

struct DnSmem {
    _Float16 s0h[kG][kD][kRowH];       // chunk-start states [m][v][k] (padded rows)
    _Float16 kht[kD][kRowT];           // unit keys transposed [k][t]
    _Float16 kh[kC][kRowH];            // unit keys [t][k]
    float aft[kG][kC][kC + 4];         // A transposed [m][i][t] (rows padded: a lane per i writes a column)
    float gcum[kG][kC];                // G_t = log gamma_t
    float beta[kG][kC];
    float gam[kG][kC];                 // gamma_t
    float sc[kG][kC];                  // gamma_C / gamma_t
    float rn[kC];                      // 1 / |k_t|
    union {
        float kr[kC][kD];                          // raw keys [t][k]
        _Float16 ks0[kG][kD * kC];                 // (K S0^T)^T, then W^T scaled, wt_index layout
    } r1;
};

__device__ __forceinline__ f32x16 mma(f16x8 a, f16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Row of element q of a 32x32 MFMA accumulator held by lane l (its column is l % 32).
__device__ __forceinline__ int acc_row(int q, int lane) { return 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3); }

// SiLU with the hardware exponential and reciprocal (a few ulp; the values
// feed fp16 MFMA operands and an fp32 solve whose own error is larger).
__device__ __forceinline__ float silu_f(float x) { return __fdividef(x, 1.0f + __expf(-x)); }
__device__ __forceinline__ float softplus_f(float x) { return fmaxf(x, 0.0f) + log1pf(expf(-fabsf(x))); }
__device__ __forceinline__ float sigmoid_f(float x) {
    const float e = expf(-fabsf(x));
    return x >= 0.0f ? 1.0f / (1.0f + e) : e / (1.0f + e);
}

__global__ void __launch_bounds__(kThreads) deltanet_scan(DnArgs g) {
    __shared__ __attribute__((aligned(16))) DnSmem sm;
    const int L = blockIdx.x / g.n_k, kh = blockIdx.x % g.n_k;
    const DnLayer& ly = g.layer[L];
    const int G = g.n_v / g.n_k;                      // value heads of this key head (<= kG)
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int qkv = (2 * g.n_k + g.n_v) * kD;
    // threads [0, 128 G): value channel dv of head m; [384, 512): key channel
    const bool is_k = tid >= kG * kD;
    const bool is_v = tid < G * kD;
    const int m = tid / kD, j = tid & (kD - 1);
    const int hv = kh * G + m;                        // global value head of a value thread
    const int ch = is_k ? g.n_k * kD + kh * kD + j : 2 * g.n_k * kD + hv * kD + j;
    const bool active = is_k || is_v;
    const int T = g.n_tokens;

    float4 cw = make_float4(0.f, 0.f, 0.f, 0.f);
    float xm3 = 0.f, xm2 = 0.f, xm1 = 0.f;
    if (active) {
        cw = *(const float4*)(ly.conv_w + (int64_t)ch * 4);
        xm3 = ly.conv_state[ch]; xm2 = ly.conv_state[qkv + ch]; xm1 = ly.conv_state[2 * qkv + ch];
    }
    // gate lanes: wave m < G, lane r = token
    const int gm = wave;
    const bool gate_wave = gm < G;
    const float decay_rate = gate_wave ? expf(ly.a_log[kh * G + gm]) : 0.f;
    const float dtb = gate_wave ? ly.dt_bias[kh * G + gm] : 0.f;

    // states: tile tau = wave + 8 i (i < 2G): head tau / 16, rows 32 ((tau % 16) / 4), keys 32 (tau % 4)
    f32x16 S[kTilesPerWave];
#pragma unroll
    for (int i = 0; i < kTilesPerWave; ++i) {
        const int tau = wave + 8 * i, hm = tau >> 4, rt = (tau & 15) >> 2, ct = tau & 3;
        if (tau < 16 * G) {
            const float* Sg = ly.state + (int64_t)(kh * G + hm) * kD * kD;
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int v = 32 * rt + acc_row(q, lane), k = 32 * ct + (lane & 31);
                S[i][q] = Sg[v * kD + k];
                sm.s0h[hm][v][k] = (_Float16)S[i][q];
            }
        }
    }

    __syncthreads();
    // X holds a chunk's raw rows, then (after conv + SiLU) its values, then the
    // right-hand side and solution; once the solution is stored, the next
    // chunk's raw rows are loaded into it, so the loads overlap the state
    // update.  Rows past the end re-read the last row (values unused).
    float X[kC];
    float a_in = 0.f, b_in = 0.f;
    auto fetch = [&](int c0) {
        if (active) {
#pragma unroll
            for (int r = 0; r < kC; ++r) {
                const int t = c0 + r < T ? c0 + r : T - 1;
                X[r] = ly.x[(int64_t)t * ly.ld + ch];
            }
        }
        if (gate_wave && lane < kC) {
            const int t = c0 + lane < T ? c0 + lane : T - 1;
            const float* row = ly.x + (int64_t)t * ly.ld;
            a_in = row[qkv + kh * G + gm];
            b_in = row[qkv + g.n_v + kh * G + gm];
        }
    };
    fetch(0);
    for (int t0 = 0; t0 < T; t0 += kC) {
        const int nv = T - t0 < kC ? T - t0 : kC;
        // ---- conv + SiLU of this thread's channel (zero past the end)
#pragma unroll
        for (int r = 0; r < kC; ++r) {
            const float xr = X[r];
            const float c = cw.x * xm3 + cw.y * xm2 + cw.z * xm1 + cw.w * xr;
            X[r] = r < nv ? silu_f(c) : 0.0f;
            xm3 = xm2; xm2 = xm1; xm1 = xr;
        }
        if (is_k) {
#pragma unroll
            for (int r = 0; r < kC; ++r) sm.r1.kr[r][j] = X[r];
        }
        // ---- gates and their running log-decay
        if (gate_wave) {
            float gl = 0.0f, be = 0.0f;
            if (lane < nv) {
                gl = -decay_rate * softplus_f(a_in + dtb);
                be = sigmoid_f(b_in);
            }
            float Gs = gl;
#pragma unroll
            for (int o = 1; o < kC; o <<= 1) {
                const float y = __shfl_up(Gs, o);
                if ((lane & 31) >= o) Gs += y;
            }
            const float GC = __shfl(Gs, kC - 1);
            if (lane < kC) {
                sm.gcum[gm][lane] = Gs;
                sm.beta[gm][lane] = be;
                sm.gam[gm][lane] = expf(Gs);
                sm.sc[gm][lane] = expf(GC - Gs);
            }
        }
        __syncthreads();
        // ---- key norms: 8 threads per token
        if (tid < 8 * kC) {
            const int r = tid >> 3, part = tid & 7;
            float ss = 0.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                // element 8 ((i + r) % 16) + part: the 64 lanes of a wave
                // (8 tokens x 8 parts) fall on 64 different banks
                const float v = sm.r1.kr[r][((i + r) & 15) * 8 + part];
                ss += v * v;
            }
            ss += __shfl_xor(ss, 1);
            ss += __shfl_xor(ss, 2);
            ss += __shfl_xor(ss, 4);
            if (part == 0) sm.rn[r] = 1.0f / sqrtf(ss + 1e-6f);
        }
        __syncthreads();
        if (is_k) {
#pragma unroll
            for (int r8 = 0; r8 < kC; r8 += 8) {
                f16x8 h8;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    h8[e] = (_Float16)(X[r8 + e] * sm.rn[r8 + e]);
                    sm.kh[r8 + e][j] = h8[e];
                }
                *(f16x8*)&sm.kht[j][r8] = h8;           // this channel's row, 16 bytes at a time
            }
        }
        __syncthreads();
        // ---- MFMA phase: A_m from K K^T (wave 5 + m, which have one K S0^T tile
        //      each below); (K S0_m^T)^T tiles (every wave)
        if (wave >= 5 && wave - 5 < G) {
            const int hm = wave - 5;
            f32x16 acc = {};
#pragma unroll
            for (int ks = 0; ks < kD / 16; ++ks) {
                const f16x8 a = *(const f16x8*)&sm.kh[lane & 31][ks * 16 + (lane >> 5) * 8];
                acc = mma(a, a, acc);
            }
            const int i = lane & 31;
            const float gi = sm.gcum[hm][i];
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int t = acc_row(q, lane);
                sm.aft[hm][i][t] = i < t ? sm.beta[hm][t] * __expf(sm.gcum[hm][t] - gi) * acc[q] : 0.0f;
            }
        }
        // tile u = wave + 8 i (u < 4 G): head u / 4, values 32 (u % 4); K = keys
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int u = wave + 8 * i;
            if (u < 4 * G) {
                const int hm = u >> 2, vt = u & 3;
                f32x16 acc = {};
#pragma unroll
                for (int ks = 0; ks < kD / 16; ++ks) {
                    const int k0 = ks * 16 + (lane >> 5) * 8;
                    const f16x8 a = *(const f16x8*)&sm.kh[lane & 31][k0];
                    const f16x8 b = *(const f16x8*)&sm.s0h[hm][32 * vt + (lane & 31)][k0];
                    acc = mma(a, b, acc);
                }
#pragma unroll
                for (int q = 0; q < 16; ++q)
                    sm.r1.ks0[hm][wt_index(32 * vt + (lane & 31), acc_row(q, lane))] = (_Float16)acc[q];
            }
        }
        __syncthreads();
        // ---- W_m = (I + A_m)^-1 (diag(beta) V - diag(beta gamma) K S0^T), one value
        //      column per thread, in place, column by column
        if (is_v) {
            _Float16* rowp = sm.r1.ks0[m];
#pragma unroll
            for (int r8 = 0; r8 < kC; r8 += 8) {
                const f16x8 ks8 = *(const f16x8*)&rowp[wt_index(j, r8)];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int r = r8 + e;
                    X[r] = sm.beta[m][r] * (X[r] - sm.gam[m][r] * (float)ks8[e]);
                }
            }
#pragma unroll
            for (int i = 0; i < kC - 1; ++i) {
#pragma unroll
                for (int r4 = (i + 1) & ~3; r4 < kC; r4 += 4) {
                    const float4 a4 = *(const float4*)&sm.aft[m][i][r4];
                    if (r4 + 0 > i) X[r4 + 0] -= a4.x * X[i];
                    if (r4 + 1 > i) X[r4 + 1] -= a4.y * X[i];
                    if (r4 + 2 > i) X[r4 + 2] -= a4.z * X[i];
                    if (r4 + 3 > i) X[r4 + 3] -= a4.w * X[i];
                }
                if (i & 1) __builtin_amdgcn_sched_barrier(0);
            }
            // W^T scaled by gamma_C / gamma_t, over this thread's own row of ks0
#pragma unroll
            for (int r8 = 0; r8 < kC; r8 += 8) {
                f16x8 w8;
#pragma unroll
                for (int e = 0; e < 8; ++e) w8[e] = (_Float16)(X[r8 + e] * sm.sc[m][r8 + e]);
                *(f16x8*)&rowp[wt_index(j, r8)] = w8;
            }
        }
        if (t0 + kC < T) fetch(t0 + kC);
        __syncthreads();
        // ---- S_m = gamma_C S0_m + sum_t (gamma_C / gamma_t) w_t k_t^T
#pragma unroll
        for (int i = 0; i < kTilesPerWave; ++i) {
            const int tau = wave + 8 * i, hm = tau >> 4, rt = (tau & 15) >> 2, ct = tau & 3;
            if (tau < 16 * G) {
                const float gC = sm.gam[hm][kC - 1];
#pragma unroll
                for (int q = 0; q < 16; ++q) S[i][q] *= gC;
#pragma unroll
                for (int s = 0; s < kC / 16; ++s) {
                    const int t8 = s * 16 + (lane >> 5) * 8;
                    const f16x8 a = *(const f16x8*)&sm.r1.ks0[hm][wt_index(32 * rt + (lane & 31), t8)];
                    const f16x8 b = *(const f16x8*)&sm.kht[32 * ct + (lane & 31)][t8];
                    S[i] = mma(a, b, S[i]);
                }
            }
        }
        // the fp16 copy of the new state for the next chunk's K S0^T (no
        // barrier before it: this phase reads no s0h; the one after it keeps
        // the next chunk's writes off ks0, kht and the gates until every
        // wave is done here)
#pragma unroll
        for (int i = 0; i < kTilesPerWave; ++i) {
            const int tau = wave + 8 * i, hm = tau >> 4, rt = (tau & 15) >> 2, ct = tau & 3;
            if (tau < 16 * G) {
#pragma unroll
                for (int q = 0; q < 16; ++q)
                    sm.s0h[hm][32 * rt + acc_row(q, lane)][32 * ct + (lane & 31)] = (_Float16)S[i][q];
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < kTilesPerWave; ++i) {
        const int tau = wave + 8 * i, hm = tau >> 4, rt = (tau & 15) >> 2, ct = tau & 3;
        if (tau < 16 * G) {
            float* Sg = ly.state + (int64_t)(kh * G + hm) * kD * kD;
#pragma unroll
            for (int q = 0; q < 16; ++q) Sg[(32 * rt + acc_row(q, lane)) * kD + 32 * ct + (lane & 31)] = S[i][q];
        }
    }
}

// New conv state: the last (width - 1) rows of [old state ; the call's raw
// q|k|v rows], one thread per channel (reads before writes, so in place).
__global__ void __launch_bounds__(256) deltanet_conv_state(DnArgs g) {
    const int L = blockIdx.y;
    const DnLayer& ly = g.layer[L];
    const int qkv = (2 * g.n_k + g.n_v) * kD;
    const int c = blockIdx.x * 256 + threadIdx.x;
    if (c >= qkv) return;
    const int T = g.n_tokens;
    float nw[kDnConv - 1];
#pragma unroll
    for (int r = 0; r < kDnConv - 1; ++r) {
        const int idx = T + r;                  // index into [old state ; rows]
        nw[r] = idx < kDnConv - 1 ? ly.conv_state[(int64_t)idx * qkv + c]
                                  : ly.x[(int64_t)(idx - (kDnConv - 1)) * ly.ld + c];
    }
#pragma unroll
    for (int r = 0; r < kDnConv - 1; ++r) ly.conv_state[(int64_t)r * qkv + c] = nw[r];
}

}  // namespace

hipError_t launch_deltanet_update(const DnArgs& a, hipStream_t s) {
    if (a.n_tokens <= 0 || a.n_layers <= 0) return hipSuccess;
    if (a.n_layers > kMaxDnLayers || a.n_k <= 0 || a.n_v % a.n_k || a.n_v / a.n_k > kG)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(deltanet_scan, dim3(a.n_layers * a.n_k), dim3(kThreads), 0, s, a);
    const int qkv = (2 * a.n_k + a.n_v) * kD;
    hipLaunchKernelGGL(deltanet_conv_state, dim3((qkv + 255) / 256, a.n_layers), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace kva
