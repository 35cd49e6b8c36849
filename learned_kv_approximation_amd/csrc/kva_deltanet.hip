// Gated-DeltaNet state update for the DeltaNet layers the projector feeds
// ("Qwen3.8-27B-KVA" card, "What the hell?": after projection the engine runs
// conv + silu, l2-norm and the DeltaNet scan over the approximated tokens).
// The formulas are the gated delta rule's (see include/kva.h):
//   causal depthwise conv (width 4) + SiLU on the raw q|k|v rows,
//   k <- k / sqrt(|k|^2 + 1e-6) per key head,
//   alpha = exp(-exp(A_log) * softplus(a + dt_bias)), beta = sigmoid(b),
//   S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T.
//
// One workgroup per (layer, value head) walks the tokens in chunks of C = 32
// and keeps the 128 x 128 fp32 state in MFMA accumulators.  Within a chunk
// (chunk-start state S0, gamma_t = alpha_1 ... alpha_t from the chunk start)
// the recurrence unrolls to
//   S_C = gamma_C S0 + sum_t (gamma_C / gamma_t) w_t k_t^T,
//   (I + A) W = diag(beta) V - diag(beta gamma) K S0^T,
//   A[t][i] = beta_t (gamma_t / gamma_i) (k_t . k_i) for i < t, else 0,
// so W = U - Wk S0^T with [U | Wk] = (I + A)^-1 [diag(beta) V | diag(beta gamma) K].
// The unit lower-triangular solve runs in fp32 by forward substitution, one
// column of [U | Wk] per thread; K K^T, Wk S0^T and W^T K are 32x32x16 fp16
// MFMAs with fp32 accumulation (keys are unit vectors; S0, Wk and W are
// rounded to fp16 as MFMA operands only, the state itself stays fp32).
#include "kva_internal.h"

namespace kva {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kC = 32;                 // tokens per chunk
constexpr int kD = kDnHeadDim;         // key and value head width
constexpr int kRowH = kD + 8;          // fp16 row of 128 values, padded (272 B)
constexpr int kRowT = kC + 8;          // fp16 row of 32 values, padded (80 B)

struct DnSmem {
    _Float16 s0h[kD][kRowH];           // chunk-start state S0 [v][k], fp16 operand
    _Float16 kht[kD][kRowT];           // unit keys transposed [k][t]
    float af[kC][kC];                  // A [t][i]
    float gcum[kC];                    // G_t = log gamma_t
    float beta[kC];
    float rn[kC];                      // 1 / |k_t|
    union {
        struct { float kr[kC][kD]; _Float16 kh[kC][kRowH]; } a;    // raw keys, unit keys [t][k]
        struct { float uf[kC][kD]; _Float16 wkh[kC][kRowH]; } b;   // U [t][v], -Wk [t][k]
        _Float16 wt[kD][kRowT];                                    // W^T scaled [v][t]
    } r1;
};

__device__ __forceinline__ f32x16 mma(f16x8 a, f16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Row of element q of a 32x32 MFMA accumulator held by lane l (its column is l % 32).
__device__ __forceinline__ int acc_row(int q, int lane) { return 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3); }

__device__ __forceinline__ float silu_f(float x) { return x / (1.0f + expf(-x)); }
__device__ __forceinline__ float softplus_f(float x) { return fmaxf(x, 0.0f) + log1pf(expf(-fabsf(x))); }
__device__ __forceinline__ float sigmoid_f(float x) {
    const float e = expf(-fabsf(x));
    return x >= 0.0f ? 1.0f / (1.0f + e) : e / (1.0f + e);
}

__global__ void __launch_bounds__(256) deltanet_scan(DnArgs g) {
    __shared__ __attribute__((aligned(16))) DnSmem sm;
    const int L = blockIdx.x / g.n_v, h = blockIdx.x % g.n_v;
    const DnLayer& ly = g.layer[L];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kh = h / (g.n_v / g.n_k);
    const int qkv = (2 * g.n_k + g.n_v) * kD;
    const bool is_v = tid < kD;                       // waves 0-1: value channels, 2-3: key channels
    const int j = tid & (kD - 1);
    const int ch = is_v ? 2 * g.n_k * kD + h * kD + j : g.n_k * kD + kh * kD + j;
    const int T = g.n_tokens;

    const float4 cw = *(const float4*)(ly.conv_w + (int64_t)ch * 4);
    float xm3 = ly.conv_state[ch], xm2 = ly.conv_state[qkv + ch], xm1 = ly.conv_state[2 * qkv + ch];
    const float decay_rate = expf(ly.a_log[h]);
    const float dtb = ly.dt_bias[h];

    // state: wave w holds rows v in [32w, 32w + 32), one accumulator per 32 keys
    float* Sg = ly.state + (int64_t)h * kD * kD;
    f32x16 S[4];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt)
#pragma unroll
        for (int q = 0; q < 16; ++q)
            S[jt][q] = Sg[(32 * wave + acc_row(q, lane)) * kD + 32 * jt + (lane & 31)];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt)
#pragma unroll
        for (int q = 0; q < 16; ++q)
            sm.s0h[32 * wave + acc_row(q, lane)][32 * jt + (lane & 31)] = (_Float16)S[jt][q];

    for (int t0 = 0; t0 < T; t0 += kC) {
        const int nv = T - t0 < kC ? T - t0 : kC;
        // ---- conv + SiLU of this thread's channel over the chunk (zero past the end)
        float xin[kC], val[kC];
#pragma unroll
        for (int r = 0; r < kC; ++r) xin[r] = r < nv ? ly.x[(int64_t)(t0 + r) * ly.ld + ch] : 0.0f;
#pragma unroll
        for (int r = 0; r < kC; ++r) {
            const float c = cw.x * xm3 + cw.y * xm2 + cw.z * xm1 + cw.w * xin[r];
            val[r] = r < nv ? silu_f(c) : 0.0f;
            xm3 = xm2; xm2 = xm1; xm1 = xin[r];
        }
        if (!is_v) {
#pragma unroll
            for (int r = 0; r < kC; ++r) sm.r1.a.kr[r][j] = val[r];
        }
        // ---- gates and their running log-decay (wave 0, lane r = token)
        if (wave == 0) {
            float gl = 0.0f, be = 0.0f;
            if (lane < nv) {
                const float* row = ly.x + (int64_t)(t0 + lane) * ly.ld;
                gl = -decay_rate * softplus_f(row[qkv + h] + dtb);
                be = sigmoid_f(row[qkv + g.n_v + h]);
            }
            float G = gl;
#pragma unroll
            for (int o = 1; o < kC; o <<= 1) {
                const float y = __shfl_up(G, o);
                if ((lane & 31) >= o) G += y;
            }
            if (lane < kC) {
                sm.gcum[lane] = G;
                sm.beta[lane] = be;
            }
        }
        __syncthreads();
        // ---- key norms: 8 threads per token
        {
            const int r = tid >> 3, part = tid & 7;
            float ss = 0.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float v = sm.r1.a.kr[r][part * 16 + i];
                ss += v * v;
            }
            ss += __shfl_xor(ss, 1);
            ss += __shfl_xor(ss, 2);
            ss += __shfl_xor(ss, 4);
            if (part == 0) sm.rn[r] = 1.0f / sqrtf(ss + 1e-6f);
        }
        __syncthreads();
        if (!is_v) {
#pragma unroll
            for (int r = 0; r < kC; ++r) {
                val[r] *= sm.rn[r];
                const _Float16 hv = (_Float16)val[r];
                sm.r1.a.kh[r][j] = hv;
                sm.kht[j][r] = hv;
            }
        }
        __syncthreads();
        // ---- A = strictly lower (beta_t gamma_t / gamma_i k_t . k_i)   (wave 0)
        if (wave == 0) {
            f32x16 acc = {};
#pragma unroll
            for (int ks = 0; ks < kD / 16; ++ks) {
                const f16x8 a = *(const f16x8*)&sm.r1.a.kh[lane & 31][ks * 16 + (lane >> 5) * 8];
                acc = mma(a, a, acc);
            }
            const int i = lane & 31;
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int t = acc_row(q, lane);
                sm.af[t][i] = i < t ? sm.beta[t] * expf(sm.gcum[t] - sm.gcum[i]) * acc[q] : 0.0f;
            }
        }
        __syncthreads();
        // ---- [U | Wk] = (I + A)^-1 [diag(beta) V | diag(beta gamma) K], one column per thread
        float X[kC];
#pragma unroll
        for (int r = 0; r < kC; ++r) {
            float s = sm.beta[r] * val[r];
            if (!is_v) s *= expf(sm.gcum[r]);
#pragma unroll
            for (int i4 = 0; i4 < r; i4 += 4) {
                const float4 a4 = *(const float4*)&sm.af[r][i4];
                s -= a4.x * X[i4];
                if (i4 + 1 < r) s -= a4.y * X[i4 + 1];
                if (i4 + 2 < r) s -= a4.z * X[i4 + 2];
                if (i4 + 3 < r) s -= a4.w * X[i4 + 3];
            }
            X[r] = s;
        }
        if (is_v) {
#pragma unroll
            for (int r = 0; r < kC; ++r) sm.r1.b.uf[r][j] = X[r];
        } else {
#pragma unroll
            for (int r = 0; r < kC; ++r) sm.r1.b.wkh[r][j] = (_Float16)(-X[r]);
        }
        __syncthreads();
        // ---- W = U - Wk S0^T: wave w takes values [32w, 32w + 32)
        f32x16 W;
#pragma unroll
        for (int q = 0; q < 16; ++q) W[q] = sm.r1.b.uf[acc_row(q, lane)][32 * wave + (lane & 31)];
#pragma unroll
        for (int ks = 0; ks < kD / 16; ++ks) {
            const f16x8 a = *(const f16x8*)&sm.r1.b.wkh[lane & 31][ks * 16 + (lane >> 5) * 8];
            const f16x8 b = *(const f16x8*)&sm.s0h[32 * wave + (lane & 31)][ks * 16 + (lane >> 5) * 8];
            W = mma(a, b, W);
        }
        __syncthreads();
        const float GC = sm.gcum[kC - 1];
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int t = acc_row(q, lane);
            sm.r1.wt[32 * wave + (lane & 31)][t] = (_Float16)(W[q] * expf(GC - sm.gcum[t]));
        }
        __syncthreads();
        // ---- S = gamma_C S0 + sum_t (gamma_C / gamma_t) w_t k_t^T
        const float gC = expf(GC);
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
#pragma unroll
            for (int q = 0; q < 16; ++q) S[jt][q] *= gC;
#pragma unroll
            for (int s = 0; s < kC / 16; ++s) {
                const f16x8 a = *(const f16x8*)&sm.r1.wt[32 * wave + (lane & 31)][s * 16 + (lane >> 5) * 8];
                const f16x8 b = *(const f16x8*)&sm.kht[32 * jt + (lane & 31)][s * 16 + (lane >> 5) * 8];
                S[jt] = mma(a, b, S[jt]);
            }
        }
#pragma unroll
        for (int jt = 0; jt < 4; ++jt)
#pragma unroll
            for (int q = 0; q < 16; ++q)
                sm.s0h[32 * wave + acc_row(q, lane)][32 * jt + (lane & 31)] = (_Float16)S[jt][q];
        __syncthreads();
    }
#pragma unroll
    for (int jt = 0; jt < 4; ++jt)
#pragma unroll
        for (int q = 0; q < 16; ++q)
            Sg[(32 * wave + acc_row(q, lane)) * kD + 32 * jt + (lane & 31)] = S[jt][q];
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
    if (a.n_layers > kMaxDnLayers || a.n_k <= 0 || a.n_v % a.n_k) return hipErrorInvalidValue;
    hipLaunchKernelGGL(deltanet_scan, dim3(a.n_layers * a.n_v), dim3(256), 0, s, a);
    const int qkv = (2 * a.n_k + a.n_v) * kD;
    hipLaunchKernelGGL(deltanet_conv_state, dim3((qkv + 255) / 256, a.n_layers), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace kva
