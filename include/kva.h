/*
 * kva.h -- C ABI of the KVA projector library for AMD Instinct MI355X (gfx950).
 *
 * The KVA projector ("Qwen3.8-27B-KVA: late-layer KV approximation", model
 * card, section "What the hell?") maps the layer-31 residual of every prompt
 * token (5120 wide) to the token-mixer inputs of the 32 late layers of the
 * base model:
 *
 *   RMSNorm -> Linear(5120 -> d) -> 3 x [causal transformer block]
 *           -> RMSNorm -> one Linear head per late layer
 *
 * where each block is pre-norm multi-head causal attention (heads of 128)
 * followed by a SwiGLU FFN, and attention never crosses the 1024-token ubatch
 * (here: "attention block") the tokens were given in.  Per the card's table
 * of predicted inputs, a gated-DeltaNet layer receives in_proj_qkv | in_proj_a
 * | in_proj_b (10240 + 48 + 48 values per token) and a full-attention layer
 * receives k_proj | v_proj before k_norm and RoPE (1024 + 1024).  The r3
 * variant adds drafter heads (kva.res.34, kva.res.48, kva.res.62, kva.final,
 * r2/r3 table) that read the same final-normed trunk state.
 *
 * Conventions for every entry point:
 *  - Sizes are element counts; matrices are row-major; a Linear weight is
 *    stored [out][in] (row o holds the weights of output o).
 *  - "device" pointers are HIP device memory on the context's device,
 *    "host" pointers are ordinary CPU memory.
 *  - `stream` is a hipStream_t (NULL = the legacy default stream).  Compute
 *    entry points validate their arguments on the host, enqueue work on
 *    `stream` and return without synchronising.  Buffers passed to them must
 *    stay valid until the stream has passed the call.
 *  - Every call returns a kva_status; nothing aborts or throws across the
 *    ABI.  kva_last_error() gives a human-readable detail for the calling
 *    thread's most recent failure.  Device faults surface asynchronously at
 *    the caller's next synchronisation of the stream.  A HIP error left
 *    pending on the thread by earlier work outside this library is cleared
 *    (not reported) when a compute entry point starts.
 *  - A context is used by one stream at a time (calls on one context must be
 *    serialised by the caller).
 */
#ifndef KVA_H
#define KVA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KVA_OK = 0,
    KVA_ERR_ARG = 1,          /* NULL pointer or invalid enum value          */
    KVA_ERR_SHAPE = 2,        /* unsupported or inconsistent dimensions      */
    KVA_ERR_DTYPE = 3,        /* unsupported storage type                    */
    KVA_ERR_OOM = 4,          /* device or host allocation failed            */
    KVA_ERR_RANGE = 5,        /* a weight does not fit the compute type      */
    KVA_ERR_UNSUPPORTED = 6,  /* valid request the library does not implement */
    KVA_ERR_HIP = 7           /* a HIP runtime call or kernel launch failed  */
} kva_status;

typedef enum {
    KVA_DTYPE_F32 = 0,   /* IEEE binary32                                        */
    KVA_DTYPE_BF16 = 1,  /* bfloat16 bit patterns (uint16)                       */
    KVA_DTYPE_Q8_0 = 2,  /* blocks of 32 inputs: fp16 scale d, then 32 int8 q;   */
                         /* weight = d * q; 34 bytes per block, blocks run along */
                         /* the `in` axis of each row                            */
    KVA_DTYPE_Q4_0 = 3   /* blocks of 32 inputs: fp16 scale d, then 16 bytes of  */
                         /* 4-bit codes n (byte j: input j in the low nibble,   */
                         /* input j+16 in the high one); weight = d * (n - 8);   */
                         /* 18 bytes per block, blocks along `in`                */
} kva_dtype;

typedef enum {
    KVA_HEAD_DELTANET = 0,  /* gated-DeltaNet layer: qkv | a | b               */
    KVA_HEAD_ATTN = 1,      /* full-attention layer: k | v (pre k_norm/RoPE)  */
    KVA_HEAD_DRAFT = 2      /* drafter residual kva.res.N or kva.final        */
} kva_head_kind;

/* One output head (one late layer, or one drafter). */
typedef struct {
    int32_t kind;     /* kva_head_kind (informational; all heads are Linear+bias) */
    int32_t layer;    /* base-model layer the head feeds (informational)          */
    int32_t out_dim;  /* outputs per token, e.g. 10336, 2048 or 5120              */
} kva_head_desc;

/* Projector shape.  Field meanings follow the card's r2/r3 table:
 * r2 = {5120, 2560, 3, 20, 128, 7040}, r3 = {5120, 3072, 3, 24, 128, 8448}. */
typedef struct {
    int32_t n_in;          /* residual width, 5120 for the base model            */
    int32_t d_model;       /* trunk width d                                      */
    int32_t n_blocks;      /* transformer blocks (3)                             */
    int32_t n_heads;       /* attention heads per block; n_heads*head_dim==d     */
    int32_t head_dim;      /* must be 128                                        */
    int32_t d_ffn;         /* SwiGLU hidden width                                */
    int32_t attn_block;    /* tokens per causal attention block (1024)           */
    int32_t max_tokens;    /* largest n_tokens a call may pass                   */
    float eps;             /* RMSNorm epsilon (inside the square root), 1e-6     */
    int32_t weight_dtype;  /* kva_dtype of every Linear weight                   */
    int32_t has_head_bias; /* 1: each head has an fp32 bias of out_dim values    */
    int32_t n_out_heads;   /* number of entries in out_heads (1..64)             */
    const kva_head_desc* out_heads; /* host array, copied by kva_create          */
} kva_config;

/* Weights of one transformer block (host pointers, weight_dtype storage). */
typedef struct {
    const float* attn_norm;  /* [d] fp32 gain                                   */
    const void* wq;          /* [d][d]   (n_heads*head_dim rows)                */
    const void* wk;          /* [d][d]                                           */
    const void* wv;          /* [d][d]                                           */
    const void* wo;          /* [d][d]                                           */
    const float* ffn_norm;   /* [d] fp32 gain                                   */
    const void* w_gate;      /* [d_ffn][d]                                       */
    const void* w_up;        /* [d_ffn][d]                                       */
    const void* w_down;      /* [d][d_ffn]                                       */
} kva_block_weights;

/* All projector weights, as HOST pointers.  kva_create copies (and repacks)
 * them into memory the context owns; the caller may free them afterwards. */
typedef struct {
    const float* in_norm;              /* [n_in] fp32 gain                      */
    const void* in_proj;               /* [d][n_in]                             */
    const kva_block_weights* blocks;   /* n_blocks entries                      */
    const float* out_norm;             /* [d] fp32 gain                         */
    const void* const* head_w;         /* n_out_heads pointers, [out_dim][d]    */
    const float* const* head_b;        /* n_out_heads pointers to [out_dim]     */
                                       /* fp32, or NULL when !has_head_bias     */
} kva_weights;

typedef struct kva_ctx kva_ctx;

typedef struct {
    uint64_t calls;         /* successful kva_project_ubatch calls              */
    uint64_t tokens;        /* tokens projected by them                         */
    uint64_t blocks;        /* attention blocks processed                       */
    uint64_t weight_bytes;  /* device bytes held for weights                    */
    uint64_t scratch_bytes; /* device bytes held for activations                */
} kva_stats;

/* Checks a config on the host only (no device is touched): dimensions
 * positive and consistent, head_dim == 128, n_heads*head_dim == d_model,
 * n_in, d_model and d_ffn multiples of 64, attn_block a positive multiple of
 * 64, 1 <= n_out_heads <= 64, every out_dim positive, weight_dtype known.
 * Returns KVA_OK, KVA_ERR_ARG, KVA_ERR_SHAPE or KVA_ERR_DTYPE. */
kva_status kva_validate_config(const kva_config* cfg);

/* Creates a projector on HIP device `device`: validates `cfg`, allocates the
 * weight arena and scratch for cfg->max_tokens tokens, converts and uploads
 * the weights.  fp32/bf16 weights: trunk weights are converted to fp16 for
 * the MFMA path (KVA_ERR_RANGE if a weight is outside fp16's finite range),
 * head weights are kept as bf16 (fp32 ones rounded to nearest even).  q8_0
 * weights are split losslessly into an int8 code plane and an fp16 scale
 * plane; the GEMMs form each weight as d*q rounded once to fp16 on the fly
 * (see kva_debug_dequant_q8_0_f16) and run fp16 MFMA throughout: the weight
 * the product uses is fp16(d*q), within 2^-12 relative of d*q (2^-25
 * absolute where d*q is below fp16's normal range), not d*q itself.  q4_0
 * weights likewise: a 4-bit code plane and an fp16 scale plane, weights
 * d*(n-8) rounded once to fp16 (kva_debug_dequant_q4_0_f16).  For
 * cfg->max_tokens > 256 q8_0 / q4_0 weights are instead expanded at create
 * into those same fp16 values, stored like fp16 weights (about twice the
 * q8_0 bytes): at such call sizes the GEMMs are bound by MFMA issue, not by
 * weight bytes, and the in-register conversion costs more than the extra
 * reads.  Outputs are bit-identical to a code-plane context that splits K
 * the same way.  KVA_ERR_RANGE
 * if a q8_0 / q4_0 block's scale is not finite or d*code rounds past fp16's
 * largest finite value (|d| * max|code| >= 65520).  The call is
 * synchronous.  On success *out owns all device memory it allocated; on
 * failure *out is NULL and nothing is leaked. */
kva_status kva_create(const kva_config* cfg, const kva_weights* w, int device, kva_ctx** out);

/* The hot path: projects n_tokens residual rows.
 *   x        device, [n_tokens][n_in] fp32 (layer-31 residuals), 16-byte aligned
 *   head_out host array of n_out_heads DEVICE pointers; head i receives
 *            [n_tokens][out_dim_i] fp32, row-major, columns in the head's
 *            segment order (qkv|a|b, k|v, or the drafter's 5120).
 * Tokens [0, n_tokens) are split into consecutive attention blocks of
 * attn_block tokens starting at token 0; the last block may be shorter.
 * Attention is causal within a block and never crosses blocks, so a block's
 * outputs are bitwise identical whether it is passed alone or inside a longer
 * call on the same context.  (The K order of the trunk GEMMs is fixed per
 * context from d_model and max_tokens: the d-wide GEMMs' K split (2 or 3
 * ways, 8 for max_tokens <= 128), and for max_tokens <= 32 every trunk GEMM
 * on a kernel that splits K over the waves of a workgroup.  Contexts created
 * with a different max_tokens may therefore differ in the last bits, within
 * the tolerance.)
 * 1 <= n_tokens <= max_tokens (else KVA_ERR_SHAPE).  Output buffers
 * must not alias x or each other.  Asynchronous on `stream`. */
kva_status kva_project_ubatch(kva_ctx* ctx, const float* x, int32_t n_tokens,
                              float* const* head_out, void* stream);

/* Synchronises the context's device, frees everything it owns.  NULL-safe. */
kva_status kva_destroy(kva_ctx* ctx);

/* Storage of a paged KV cache. */
typedef enum {
    KVA_KV_BF16 = 0,           /* rows of head_dim bf16 values                   */
    KVA_KV_Q8_0_HADAMARD = 1   /* rows of head_dim/32 q8_0 blocks (34 bytes:     */
                               /* fp16 scale d, 32 int8 codes q, value d*q) of   */
                               /* the Hadamard-rotated values, see below         */
} kva_kv_type;

/* The single-map projector of the R9V forum post ("R9V Update: Created and
 * adopted KVA projections ...", first implementation): one dense linear map
 * per later layer from the residual at a chosen start layer straight to that
 * layer's input, y_l = W_l x + b_l, with no trunk (the post fits each map by
 * ridge regression; here the maps are given).  The start layer only decides
 * how many maps there are (the later layers).  A context made here holds the
 * maps packed like kva_create's heads and runs them as one grouped GEMM:
 *   n_in         residual width (a multiple of 32), also every map's width
 *   n_maps       maps, 1..64 (e.g. 51 for start layer 12 of 64 layers)
 *   weight_dtype KVA_DTYPE_F32 or _BF16 (rounded to bf16; the input x is
 *                rounded to bf16 too), or _Q8_0 / _Q4_0 (weights d*q rounded
 *                once to fp16, x to fp16)
 *   w            host array of n_maps host pointers, [n_in (out)][n_in (in)]
 *   b            host array of n_maps host pointers to fp32 [n_in], or NULL
 *   max_tokens   largest n_tokens a call may pass
 * Errors as kva_create (KVA_ERR_SHAPE / _DTYPE / _ARG / _OOM / _HIP).  Such a
 * context works with kva_map_project, kva_profile_*, kva_get_stats and
 * kva_destroy; kva_project_ubatch on it returns KVA_ERR_UNSUPPORTED. */
kva_status kva_map_create(int32_t n_in, int32_t n_maps, int32_t weight_dtype, const void* const* w,
                          const float* const* b, int32_t max_tokens, int device, kva_ctx** out);

/* y_l = W_l x + b_l for the n_tokens rows of x (device fp32 [n_tokens][n_in],
 * 16-byte aligned; KVA_ERR_ARG otherwise);
 * out: host array of n_maps device pointers, map l writes fp32
 * [n_tokens][n_in].  fp32 accumulation over n_in in a fixed order, so a row's
 * results do not depend on the other rows of the call.  1 <= n_tokens <=
 * max_tokens.  Asynchronous on `stream`. */
kva_status kva_map_project(kva_ctx* ctx, const float* x, int32_t n_tokens, float* const* out, void* stream);

/* kva_map_project for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same kernels and the same results, bit for bit, but the residual's
 * tiled 16-bit copy (round_up(n_tokens, 256) * n_in * 2 bytes) goes to a
 * static device array of 16 MiB that the library holds on each device until
 * the process ends, instead of the context's scratch.  The call allocates
 * nothing (no hipMalloc, no events; kva_profile_* records nothing for it).
 * Every call on one device shares that array: calls that overlap on one GPU
 * (other streams, other threads, other contexts) race and must be ordered by
 * the caller.  KVA_ERR_SHAPE if the copy would exceed 16 MiB (n_in = 5120:
 * at most 1536 tokens) or n_tokens is outside [1, max_tokens]; otherwise
 * errors as kva_map_project.  Asynchronous on `stream`. */
kva_status kva_map_project_noalloc(kva_ctx* ctx, const float* x, int32_t n_tokens, float* const* out,
                                   void* stream);

/* Paged KV cache of one full-attention layer of the base model
 * ("Qwen3.8-27B-MLA" card, "What this is": 4 KV heads of 256 dims, 64 of
 * which are rotary).  Pools are device arrays laid out
 * [n_pages][page_size][n_kv_heads][row], a row being one KV head of one token
 * in the kv_type's format (bf16: 512 bytes; q8_0: 272 bytes, 2-byte aligned
 * pools); page_table is a device int32 array mapping logical page
 * (position / page_size) to a physical page.
 *
 * KVA_KV_Q8_0_HADAMARD ("Qwen3.8-27B-KVA" card, "Other notes": q8_0 K/V
 * caches are supported, and the approximated K/V are rotated by the same
 * Hadamard transform as the exactly computed ones): each row is first rotated by the
 * orthonormal Walsh-Hadamard transform of Sylvester order, y = H x / 16 with
 * H[i][j] = (-1)^popcount(i & j) over the 256 dims (an orthogonal involution:
 * a consumer rotates queries alike, or rotates y back), then stored as 8 q8_0
 * blocks of 32 consecutive dims, decided in fp32 by ggml's q8_0 block rule:
 * d = amax / 127, its reciprocal 1/d formed once (0 when d = 0),
 * q = round-half-away(y * (1/d)), clamped to [-127, 127], d stored rounded
 * to fp16 (nearest even).  The rotation itself is computed in fp32 (exact
 * for integer-valued rows of moderate size). */
typedef struct {
    void* k_pool;
    void* v_pool;
    const int32_t* page_table;
    int32_t page_size;     /* 256                                        */
    int32_t n_pages;       /* physical pages in each pool                */
    int32_t n_logical;     /* entries in page_table                      */
    int32_t n_kv_heads;    /* 4                                          */
    int32_t head_dim;      /* 256                                        */
    int32_t n_rot;         /* rotary dims at the start of each KV head   */
    double rope_base;      /* 1e7                                        */
    float eps;             /* k_norm epsilon, 1e-6                       */
    int32_t kv_type;       /* kva_kv_type (KVA_ERR_DTYPE if unknown)     */
} kva_paged_kv;

/* The attention-layer state update that follows the projection ("What the
 * hell?": k_norm + RoPE + KV-cache writes for the attention layers).  For
 * token t at absolute position p = pos0 + t:
 *   k = kv[t][0 : n_kv_heads*head_dim] viewed [n_kv_heads][head_dim];
 *   each KV head: RMSNorm (eps inside the root) times k_gain[head_dim];
 *   RoPE on dims [0, n_rot): pair (j, j + n_rot/2) turned by
 *     p * rope_base^(-2j/n_rot) (the angle is reduced in double precision);
 *   v = kv[t][n_kv_heads*head_dim : 2*n_kv_heads*head_dim] unchanged;
 *   both stored in the cache's kv_type (bf16 rounded to nearest even, or
 *   Hadamard-rotated q8_0) at pool[page_table[p / page_size]][p % page_size].
 *   kv      device fp32, row t at kv + t*ld_kv (ld_kv >= 2*n_kv_heads*head_dim)
 *   k_gain  device fp32 [head_dim]
 * A token whose page-table entry lies outside [0, n_pages) is skipped
 * (nothing is written for it).  KVA_ERR_SHAPE when pos0 + n_tokens exceeds
 * n_logical * page_size or that product reaches 2^31.  Asynchronous. */
kva_status kva_attn_kv_write(const float* kv, int64_t ld_kv, int32_t n_tokens, int64_t pos0,
                             const float* k_gain, const kva_paged_kv* cache, void* stream);

/* One full-attention head's destination for kva_project_ubatch_kv. */
typedef struct {
    const float* k_gain;    /* device fp32 [head_dim], that layer's k_norm gain */
    kva_paged_kv cache;     /* that layer's pools and page table                */
} kva_attn_dest;

/* kva_project_ubatch with the attention-layer state update fused into the
 * head GEMM ("Qwen3.8-27B-KVA" card, "What the hell?": k_norm + RoPE + KV
 * cache writes follow the projection).  Every head of kind KVA_HEAD_ATTN
 * whose out_dim is 2 * 4 * 256 (k | v of 4 KV heads of 256 dims) is not
 * written as fp32: its k and v go through exactly the arithmetic of
 * kva_attn_kv_write, token t at position pos0 + t, into attn[a] (a = rank
 * of that head among such heads, in head order).  The pools then hold the
 * same bits as kva_project_ubatch followed by one kva_attn_kv_write per
 * such head (kv = that head's output, ld_kv = 2048), without the fp32 k|v
 * round trip through memory.
 *   head_out  as for kva_project_ubatch; entries of the fused heads are
 *             ignored and may be NULL
 *   attn      host array of n_attn destinations (device pools, gains and
 *             page tables); n_attn must equal the number of such heads
 *             (KVA_ERR_SHAPE), at most 16; every cache must satisfy the
 *             checks of kva_attn_kv_write and all must share n_rot,
 *             rope_base and eps (KVA_ERR_UNSUPPORTED)
 * Pools must not alias x, each other or the outputs.  Asynchronous. */
kva_status kva_project_ubatch_kv(kva_ctx* ctx, const float* x, int32_t n_tokens,
                                 float* const* head_out, int64_t pos0,
                                 const kva_attn_dest* attn, int32_t n_attn, void* stream);

/* One gated-DeltaNet layer for kva_deltanet_update. */
typedef struct {
    const float* mixer_in;  /* device [n_tokens][ld_in]: the projector's output for
                               this layer, q|k|v (raw, before conv) then a then b */
    int64_t ld_in;          /* >= (2*n_k_heads + n_v_heads)*head_dim + 2*n_v_heads  */
    const float* conv_w;    /* device [qkv channels][4], 16-byte aligned             */
    const float* a_log;     /* device [n_v_heads]                                    */
    const float* dt_bias;   /* device [n_v_heads]                                    */
    float* conv_state;      /* device [3][qkv channels], in/out: raw rows of the 3
                               tokens before the call, oldest first (zeros at the
                               start of a sequence)                                  */
    float* state;           /* device [n_v_heads][head_dim][head_dim] fp32, in/out:
                               S[h][i][j] maps key dim j to value dim i             */
} kva_deltanet_layer;

/* The DeltaNet layers' state update after a projection ("Qwen3.8-27B-KVA"
 * card, "What the hell?": conv + silu, l2-norm and the DeltaNet scan over the
 * approximated tokens).  The card names the steps, not their formulas; this
 * is the gated delta rule (Qwen3-Next-style gated DeltaNet layer):
 *   qkv channels: q (n_k_heads*head_dim) | k (same) | v (n_v_heads*head_dim);
 *   c = causal depthwise conv of width 4 over tokens (conv_w[ch][3] multiplies
 *       the current token, [0] the token 3 back; rows before the call come
 *       from conv_state), then SiLU;
 *   k_h = c_k,h / sqrt(|c_k,h|^2 + 1e-6) per key head; v_h = c_v,h;
 *   per value head h and token: alpha = exp(-exp(a_log[h]) *
 *       softplus(a[h] + dt_bias[h])), beta = sigmoid(b[h]);
 *   value head h reads key head h / (n_v_heads / n_k_heads), and
 *   S_h <- alpha S_h (I - beta k k^T) + beta v k^T over the tokens in order.
 * On return (on the stream) state holds S after the last token and
 * conv_state the last 3 raw qkv rows of [old conv_state ; mixer_in rows].
 * q's conv is not formed (the layer's output is not produced here).  An
 * engine that runs the ubatch's last token exactly passes n_tokens - 1
 * rows.  All layers share n_tokens and the head counts; any number of layers
 * (launched 32 at a time).  head_dim must be 128 and n_v_heads / n_k_heads
 * at most 3 (KVA_ERR_UNSUPPORTED);
 * KVA_ERR_SHAPE for inconsistent counts or a short ld_in; KVA_ERR_ARG for
 * NULL or misaligned pointers.  Buffers of different layers must not alias.
 * The scan runs in fp32 with the MFMA operands (unit keys, the chunk-start
 * state and the chunk's corrections) rounded to fp16; the state stays fp32.
 * Asynchronous on `stream`. */
kva_status kva_deltanet_update(const kva_deltanet_layer* layers, int32_t n_layers, int32_t n_tokens,
                               int32_t n_k_heads, int32_t n_v_heads, int32_t head_dim, void* stream);

/* Test hook: dequantises n_blocks q8_0 blocks (device, 34 bytes each: fp16
 * scale d, then 32 int8 codes q; format from [KVA] "Projector quantization and
 * flash-attn") to fp32 (device, 32*n_blocks values): out = float(d) * q,
 * exact, fp16 subnormal scales honoured.  This is the format's value; the
 * GEMMs do not run this routine (their operand is kva_debug_dequant_q8_0_f16).  Asynchronous on `stream`;
 * KVA_ERR_ARG for NULL pointers, KVA_ERR_SHAPE for n_blocks < 0. */
kva_status kva_debug_dequant_q8_0(const void* blocks, int64_t n_blocks, float* out, void* stream);

/* Test hook: the weights the q8_0 GEMMs actually feed to the fp16 MFMA, made
 * by the GEMMs' own device routine: for n_blocks q8_0 blocks (device, 34
 * bytes each) writes 32*n_blocks fp16 bit patterns (device), each the exact
 * product d * q rounded once to nearest-even binary16 (overflow to +-inf).
 * Asynchronous on `stream`; errors as kva_debug_dequant_q8_0. */
kva_status kva_debug_dequant_q8_0_f16(const void* blocks, int64_t n_blocks, uint16_t* out, void* stream);

/* Test hook: the same for q4_0 blocks (device, 18 bytes each; see
 * KVA_DTYPE_Q4_0): 32*n_blocks fp16 bit patterns, each d * (n - 8) rounded
 * once to nearest-even binary16, made by the q4_0 GEMMs' own device routine.
 * Asynchronous on `stream`; errors as kva_debug_dequant_q8_0. */
kva_status kva_debug_dequant_q4_0_f16(const void* blocks, int64_t n_blocks, uint16_t* out, void* stream);

/* Test hook: the q8_0 block rule's scale and reciprocal as the KV-cache
 * write forms them (d = amax / 127 and 1 / d by a multiply-add correction and
 * a reciprocal Newton step instead of division; [KVA] "Other notes" for the
 * Hadamard-rotated q8_0 cache, ggml's q8_0 rule for the block) against
 * correctly rounded division, over all 2^32 binary32 patterns on the device.
 * Adds to counts (device, 3 x uint64, the caller zeroes them): [0] patterns
 * whose scale differs (-0 excluded), [1] patterns in [2^-126, 2^126) whose
 * fast reciprocal differs, [2] patterns whose guarded reciprocal (0 for 0)
 * differs; NaN matches any NaN.  Asynchronous on `stream` (a few ms);
 * KVA_ERR_ARG for NULL counts. */
kva_status kva_debug_check_q8_scale(unsigned long long* counts, void* stream);

/* Measurement hook: a pure-MFMA loop with no memory traffic.  Launches
 * n_workgroups workgroups of 4 waves; each wave issues n_iter x 8 independent
 * bf16 v_mfma_f32_32x32x16 (32768 FLOP each), i.e.
 * n_workgroups * 4 * n_iter * 8 * 32768 FLOP in all, and writes one float
 * per thread to sink (device, 256 * n_workgroups floats) so the work is not
 * dead.  Timing it gives the MFMA rate the device sustains at its current
 * clock.  Asynchronous on `stream`; KVA_ERR_ARG for a NULL sink,
 * KVA_ERR_SHAPE for non-positive counts. */
kva_status kva_debug_mfma_loop(int32_t n_iter, int32_t n_workgroups, float* sink, void* stream);

/* Test hook: copies the final-normed trunk state z of the most recent
 * kva_project_ubatch call ([n_tokens][d_model] 16-bit patterns, the head
 * GEMM's A operand: bf16, or fp16 for q8_0 / q4_0 weights) to device buffer `dst`.
 * Asynchronous on `stream`. */
kva_status kva_debug_copy_z(kva_ctx* ctx, uint16_t* dst, int32_t n_tokens, void* stream);

/* Test hook: fills every byte of the context's activation scratch (the
 * buffers kva_create sizes for max_tokens: normed input, residual stream,
 * split-K partials, Q|K, V^T, attention output, SwiGLU output, z) with 0xFF,
 * a NaN in fp32, fp16 and bf16 alike.  A following projection must give the
 * same bits as on clean scratch: no kernel may read a scratch value that
 * the same call did not write first, except where it discards the result.
 * Asynchronous on `stream`; KVA_ERR_ARG for a NULL ctx. */
kva_status kva_debug_poison_scratch(kva_ctx* ctx, void* stream);

/* Test hook (host only, no device): the packed column order of the head
 * GEMM for `cfg`.  Head outputs are packed into 256-column tiles: first the
 * 8 tiles of every full-attention head with out_dim 2048 (the heads
 * kva_project_ubatch_kv fuses), then the out_dim / 256 full tiles of every
 * other head, each group in head order, then one tail segment gathering
 * every head's last out_dim % 256 columns (padded to a multiple of 256).  For packed column c, col_head[c] is the head (-1 for
 * padding) and col_index[c] the column inside that head.  *n_cols receives the
 * packed width; nothing is written past `capacity` entries (KVA_ERR_SHAPE if
 * capacity is too small). */
kva_status kva_debug_head_plan(const kva_config* cfg, int32_t* n_cols, int32_t* col_head,
                               int32_t* col_index, int64_t capacity);

/* Test hook (host only, no device): packs one weight [rows][K] (src, host,
 * in src_dtype storage: fp32, bf16, or q8_0 / q4_0 blocks along K) the way
 * kva_create lays it out in device memory, rows padded with zero rows to a
 * multiple of 256.  target 0: fp16 values, 1: bf16 values (both in 32-wide K
 * slabs of 256 rows, 16-byte chunk c of row r at c ^ ((r >> 2) & 3)); 2: q8_0
 * code plane (out) and fp16 scale plane (scales); 3: q4_0 likewise.  Target
 * 0 also takes q8_0 / q4_0 blocks: each weight is expanded to fp16(d*code),
 * the layout of a context with max_tokens > 256.  out
 * receives the values or codes (out_bytes capacity), scales the scales
 * (n_scales capacity; quantised targets only).  Errors as kva_create's
 * packing (KVA_ERR_DTYPE, _RANGE), KVA_ERR_SHAPE for short buffers. */
kva_status kva_debug_pack_weight(const void* src, int32_t src_dtype, int32_t rows, int32_t K, int32_t target,
                                 void* out, int64_t out_bytes, uint16_t* scales, int64_t n_scales);

/* Test hook (host only): the conversion kva_create applies to trunk weights,
 * src_dtype (KVA_DTYPE_F32 or KVA_DTYPE_BF16) -> fp16 bit patterns, rounding
 * to nearest even.  KVA_ERR_RANGE if a finite value rounds past fp16's
 * largest finite value (dst is still fully written, with infinities). */
kva_status kva_debug_host_to_f16(const void* src, int32_t src_dtype, int64_t n, uint16_t* dst);

/* Stages of one projection, for kva_profile_*. */
typedef enum {
    KVA_STAGE_NORM = 0,        /* RMSNorm + cast kernels (2 per block, final; the
                                  input norm too in contexts of <= 32 tokens per call) */
    KVA_STAGE_GEMM_IN = 1,     /* input RMSNorm + Linear n_in -> d in one GEMM (the
                                  row's 1/RMS applied by the first block's norm)      */
    KVA_STAGE_GEMM_QKV = 2,    /* Q|K|V projection                                    */
    KVA_STAGE_ATTN = 3,        /* block-causal attention                               */
    KVA_STAGE_GEMM_O = 4,      /* output projection + residual                         */
    KVA_STAGE_GEMM_GATEUP = 5, /* gate/up + SwiGLU                                     */
    KVA_STAGE_GEMM_DOWN = 6,   /* down projection + residual                           */
    KVA_STAGE_GEMM_HEADS = 7,  /* all heads + bias + per-head scatter                  */
    KVA_N_STAGES = 8
} kva_stage;

typedef struct {
    int32_t launches;   /* kernel launches timed since the last read            */
    double total_ms;    /* their summed device time (HIP event pairs)           */
} kva_stage_time;

/* Benchmark support: while bit s of stage_mask is set, kva_project_ubatch
 * records a HIP event pair on its stream around every launch of stage s.
 * 0 disables recording.  Recording adds no synchronisation. */
kva_status kva_profile_enable(kva_ctx* ctx, uint32_t stage_mask);

/* Waits for the recorded events, writes per-stage totals to out[KVA_N_STAGES]
 * and clears them. */
kva_status kva_profile_read(kva_ctx* ctx, kva_stage_time* out);

kva_status kva_get_stats(const kva_ctx* ctx, kva_stats* out);
const char* kva_status_str(kva_status s);
const char* kva_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* KVA_H */
